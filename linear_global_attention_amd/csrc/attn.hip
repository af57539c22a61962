// Tile-sparse and dense softmax attention for gfx950 (bf16 MFMA).
//
// Zebra3D pages, "Linear-centered stages plus tile-sparse stages": kept key
// tiles keep full softmax interactions, omitted tiles are seen through their
// mean-K/V landmark, special-token keys are always visible, special query
// rows are dense and every patch query keeps its own key. "Global attention
// dominates runtime as views grow": dense attention over all tokens is the
// baseline this stage replaces.
//
// One wave owns one query group: a patch query tile (<= 64 rows) or 64
// special-token rows. It walks 32-key blocks in ascending order -- the
// tokens of its kept tiles, then all landmarks (kept ones masked), then the
// special keys -- with a flash-style online softmax in the exp2 domain.
//   S^T = K Q^T : v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 channels read as
//                 16-byte rows of the packed keys, B = Q held in registers.
//   O^T += V^T P^T: A = 16 channels x 32 keys read from the d-major value
//                 blocks, B = the bf16 probabilities straight from the S^T
//                 accumulators (lane l of group g holds keys 4g..4g+3 of both
//                 16-key halves, which is the k-slot order A uses too).
// Landmark keys are fp32 means; they enter as a bf16 high and low part so
// their logits carry ~16 mantissa bits. The self key enters last, only if
// the query tile's own tile was not kept.
#include "common.hpp"

namespace zebra {

constexpr float QK_LOG2 = 1.4426950408889634f * 0.125f;  // log2(e) / sqrt(64)
constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float M_INIT = -1.0e30f;

struct WaveState {
  bf16x8 q[4][2];   // [query block][channel half]
  f32x4 o[4][4];    // [d block][query block]: O^T
  float m[4];       // running max (log2 domain) of query qb*16 + lane%16
  float l[4];       // lane-partial row sum
};

template <bool LO>
__device__ __forceinline__ void attend_block(WaveState& st, int nqb, const u16* __restrict__ kb,
                                             const u16* __restrict__ kb_lo,
                                             const u16* __restrict__ vb, int nvalid,
                                             unsigned keymask, const float* __restrict__ bias) {
  const int lane = threadIdx.x & 63, g = lane >> 4, tl = lane & 15;
  bf16x8 kf[2][2], kl[2][2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      const int off = (h2 * 16 + tl) * D + ds * 32 + 8 * g;
      kf[h2][ds] = *(const bf16x8*)(kb + off);
      if (LO) kl[h2][ds] = *(const bf16x8*)(kb_lo + off);
    }
  // per-key additive term (log2 domain) and validity for keys h2*16+4g+r
  float add[2][4];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = h2 * 16 + 4 * g + r;
      const bool ok = key < nvalid && ((keymask >> key) & 1u);
      add[h2][r] = ok ? (bias ? bias[key] * LOG2E_F : 0.f) : -INFINITY;
    }
  bf16x8 vf[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const u16* vr = vb + (db * 16 + tl) * KBLK;
    const uint2 lo4 = *(const uint2*)(vr + 4 * g);
    const uint2 hi4 = *(const uint2*)(vr + 16 + 4 * g);
    uint4 w = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
    vf[db] = __builtin_bit_cast(bf16x8, w);
  }
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    if (qb >= nqb) break;
    f32x4 s[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h2][ds], st.q[qb][ds], a, 0, 0, 0);
        if (LO) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl[h2][ds], st.q[qb][ds], a, 0, 0, 0);
      }
      s[h2] = a;
    }
    float x[2][4];
    float bm = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[h2][r] = s[h2][r] * QK_LOG2 + add[h2][r];
        bm = fmaxf(bm, x[h2][r]);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = fmaxf(st.m[qb], bm);
    const float alpha = __builtin_amdgcn_exp2f(st.m[qb] - mn);
    st.m[qb] = mn;
    bf16x8 p;
    float ps = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u16 pb = f2bf(__builtin_amdgcn_exp2f(x[h2][r] - mn));
        ps += bf2f(pb);
        p[h2 * 4 + r] = __builtin_bit_cast(__bf16, pb);
      }
    st.l[qb] = st.l[qb] * alpha + ps;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      st.o[db][qb] *= alpha;
      st.o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], p, st.o[db][qb], 0, 0, 0);
    }
  }
}

// grid (T + ceil(nspec/64), H), block 64.
__global__ void __launch_bounds__(64) attn_kernel(Geom g, AttnArgs A) {
  const int h = blockIdx.y;
  const int grp = blockIdx.x;
  const int lane = threadIdx.x & 63, lg = lane >> 4, tl = lane & 15;
  const bool patch = grp < g.T;
  int f = 0, tl_id = 0, nrows;
  if (patch) {
    f = grp / g.tpf;
    tl_id = grp - f * g.tpf;
    nrows = g.th[tl_id] * g.tw[tl_id];
  } else {
    nrows = min(64, g.nspec - (grp - g.T) * 64);
  }
  const int nqb = (nrows + 15) / 16;
  const long long rs = (long long)g.H * D;

  // token of query row j of this group
  auto row_token = [&](int j) -> long long {
    if (patch) {
      const int a = tl_id / g.tc, b = tl_id - a * g.tc;
      const int tw = g.tw[tl_id];
      const int r = TILE * a + j / tw, c = TILE * b + j % tw;
      return (long long)f * g.tok_pf + g.S + (long long)r * g.C + c;
    }
    const int i = (grp - g.T) * 64 + j;
    return (long long)(i / g.S) * g.tok_pf + (i % g.S);
  };

  WaveState st;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int j = qb * 16 + tl;
    const bool ok = j < nrows;
    const long long tok = ok ? row_token(j) : 0;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (ok) w = *(const uint4*)(A.Q + tok * rs + h * D + ds * 32 + 8 * lg);
      st.q[qb][ds] = __builtin_bit_cast(bf16x8, w);
    }
    st.m[qb] = M_INIT;
    st.l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const u16* Kh = A.Kt + (long long)h * g.slots * D;
  const u16* Vh = A.Vt + (long long)h * g.slots * D;
  const bool sparse_rows = A.sparse && patch;
  const unsigned* mrow = sparse_rows ? A.selmask + ((long long)h * g.T + grp) * A.nwords : nullptr;

  // (1) token keys of the kept tiles (all tiles when dense)
  auto do_tile = [&](int u) {
    const int fu = u / g.tpf, tu = u - fu * g.tpf;
    const int n = g.th[tu] * g.tw[tu];
    const long long base = (long long)fu * g.slots_pf + g.slot_off[tu];
    for (int b0 = 0; b0 < n; b0 += KBLK) {
      attend_block<false>(st, nqb, Kh + (base + b0) * D, nullptr,
                          Vh + ((base + b0) / KBLK) * D * KBLK, n - b0, 0xFFFFFFFFu, nullptr);
    }
  };
  bool own_kept = true;
  if (sparse_rows) {
    for (int w = 0; w < A.nwords; ++w) {
      unsigned bits = mrow[w];
      while (bits) {
        const int u = w * 32 + __builtin_ctz(bits);
        bits &= bits - 1u;
        do_tile(u);
      }
    }
    own_kept = (mrow[grp >> 5] >> (grp & 31)) & 1u;
  } else {
    for (int u = 0; u < g.T; ++u) do_tile(u);
  }

  // (2) landmarks of the omitted tiles: logit q.kbar/8 + ln n
  if (sparse_rows) {
    const u16* lmk = A.LM + (long long)h * 3 * g.T_pad * D;
    const u16* lml = lmk + (long long)g.T_pad * D;
    const u16* lmv = lml + (long long)g.T_pad * D;
    for (int lb = 0; lb < g.T_pad / KBLK; ++lb) {
      const unsigned kept = lb < A.nwords ? mrow[lb] : 0xFFFFFFFFu;
      if (kept == 0xFFFFFFFFu) continue;
      attend_block<true>(st, nqb, lmk + (long long)lb * KBLK * D, lml + (long long)lb * KBLK * D,
                         lmv + (long long)lb * D * KBLK, g.T - lb * KBLK, ~kept,
                         A.logn + lb * KBLK);
    }
  }

  // (3) special keys of every frame
  {
    const u16* Ksh = A.Ks + (long long)h * g.spec_pad * D;
    const u16* Vsh = A.Vs + (long long)h * g.spec_pad * D;
    for (int b0 = 0; b0 < g.nspec; b0 += KBLK)
      attend_block<false>(st, nqb, Ksh + (long long)b0 * D, nullptr, Vsh + (long long)b0 * D,
                          g.nspec - b0, 0xFFFFFFFFu, nullptr);
  }

  // (4) the self key, when the own tile was not kept
  if (sparse_rows && !own_kept) {
    const long long base = (long long)f * g.slots_pf + g.slot_off[tl_id];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      if (qb >= nqb) break;
      const int j = qb * 16 + tl;  // row j's key sits in slot j of its own tile
      float dot = 0.f;
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        const uint4 kw = *(const uint4*)(Kh + (base + j) * D + ds * 32 + 8 * lg);
        const bf16x8 kv = __builtin_bit_cast(bf16x8, kw);
#pragma unroll
        for (int m = 0; m < 8; ++m) dot += (float)st.q[qb][ds][m] * (float)kv[m];
      }
      dot += __shfl_xor(dot, 16, 64);
      dot += __shfl_xor(dot, 32, 64);
      const float x = (j < nrows) ? dot * QK_LOG2 : M_INIT;
      const float mn = fmaxf(st.m[qb], x);
      const float alpha = __builtin_amdgcn_exp2f(st.m[qb] - mn);
      const float p = __builtin_amdgcn_exp2f(x - mn);
      st.m[qb] = mn;
      st.l[qb] = st.l[qb] * alpha + (lg == 0 ? p : 0.f);
      const long long vblk = (base + j) / KBLK;
      const int vk = (int)((base + j) % KBLK);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = db * 16 + 4 * lg + r;
          const float v = (j < nrows) ? bf2f(Vh[(vblk * D + d) * KBLK + vk]) : 0.f;
          st.o[db][qb][r] = st.o[db][qb][r] * alpha + p * v;
        }
    }
  }

  // finalize: O = O^T / l, row = query qb*16 + tl, channels db*16 + 4*lg + r
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    if (qb >= nqb) break;
    float lt = st.l[qb];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = 1.0f / lt;
    const int j = qb * 16 + tl;
    if (j < nrows) {
      const long long tok = row_token(j);
      u16* orow = A.O + tok * rs + h * D;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint2 w;
        w.x = (unsigned)f2bf(st.o[db][qb][0] * inv) | ((unsigned)f2bf(st.o[db][qb][1] * inv) << 16);
        w.y = (unsigned)f2bf(st.o[db][qb][2] * inv) | ((unsigned)f2bf(st.o[db][qb][3] * inv) << 16);
        *(uint2*)(orow + db * 16 + 4 * lg) = w;
      }
    }
  }
}

hipError_t launch_attn(const Geom& g, const AttnArgs& a, hipStream_t s) {
  const int groups = g.T + (g.nspec + 63) / 64;
  hipLaunchKernelGGL(attn_kernel, dim3(groups, g.H), dim3(64), 0, s, g, a);
  return hipGetLastError();
}

}  // namespace zebra
