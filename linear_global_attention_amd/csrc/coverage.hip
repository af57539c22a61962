// Attention-mass coverage diagnostic of a tile-sparse stage for gfx950.
//
// Zebra3D pages, "Sensitive stages also concentrate their attention": the
// stages are profiled by how concentrated their attention mass is, and the
// sparse stages are those where the selected tiles cover most of it;
// "Linear-centered stages plus tile-sparse stages" for the kept tiles and
// the mean-K/V landmarks that stand in for the omitted ones.
//
// For every head and patch query tile t, over the tile's rows i:
//   coverage  = mean_i  (dense softmax mass of row i on the tokens of the
//               key tiles t kept) / (its whole dense mass, all N keys)
//   lm_error  = mean_i  1 - L_i / E_i, E_i the exact mass of the omitted
//               tiles' tokens, L_i the mass their landmarks give them
//               (n_u exp(q_i . kbar_u / 8)); 0 when nothing is omitted.
//
// Work decomposition: a workgroup of four waves takes four query tiles,
// one per wave, each wave holding its tile's up to 64 rows as four 16-row
// MFMA slots. The head's packed keys stream through an LDS ring of four
// 32-key blocks shared by the four waves (async global->LDS copies two
// blocks ahead, one barrier per block); every wave uses every block, so
// the work is balanced. Two passes over the stream: the exact row maximum
// over all token keys, then the three mass sums (kept tiles, omitted tiles,
// special keys) and the landmark sum, with p = exp2((s - max) log2(e) / 8).
// A landmark's logit is at most the largest token logit of its tile plus
// ln n_u <= ln 64, so the token maximum keeps every term finite. Only
// QK^T is computed (v_mfma_f32_16x16x32_bf16); no values are read.
#include "attn_common.hpp"

namespace zebra {

constexpr int CV_WAVES = 4;
constexpr int CV_RING = 4;        // 32-key blocks in the LDS ring
constexpr int CV_BLOCK = 4096;    // bytes of one staged block (32 keys x 128 B)

// Token of row j of tile (f, tl).
__device__ inline long long cv_token(const Geom& g, int f, int tl, int j) {
  const int a = tl / g.tc, b = tl - a * g.tc;
  const int tw = tile_w(g, tl);
  return (long long)f * g.tok_pf + g.S + (long long)(TILE * a + j / tw) * g.C + TILE * b + j % tw;
}

// One 32-key block of the stream: its source (32 rows of 128 B), how many
// keys are real, its kind (0 token tile, 1 special keys, 2 landmarks) and,
// for a token block, its tile; for a landmark block, its block index.
struct CvBlock {
  const char* src;
  int nvalid, kind, tile;
};

// Walks the key stream: the tiles' blocks in tile order, then the special
// blocks, then (second pass) the landmark blocks. Every wave walks it
// itself, in scalar registers.
struct CvStream {
  const Geom& g;
  const char* kt;  // this head's packed keys
  const char* ks;  // this head's packed special keys
  const char* lm;  // this head's landmark key blocks
  bool landmarks;
  int u, blk;      // current tile and block within it (tile phase)
  int sb, lb;      // special / landmark block
  __device__ CvStream(const Geom& g_, const char* kt_, const char* ks_, const char* lm_, bool lmk)
      : g(g_), kt(kt_), ks(ks_), lm(lm_), landmarks(lmk), u(0), blk(0), sb(0), lb(0) {}
  // Next block; false at the end.
  __device__ bool next(CvBlock& b) {
    if (u < g.T) {
      const int f = frame_of_tile(g, u), tl = u - f * g.tpf;
      const int n = tile_n(g, tl);
      const long long slot = (long long)f * g.slots_pf + tile_off(g, tl) + blk * KBLK;
      b.src = kt + slot * (D * 2);
      b.nvalid = min(KBLK, n - blk * KBLK);
      b.kind = 0;
      b.tile = u;
      if (++blk * KBLK >= n) {
        blk = 0;
        ++u;
      }
      return true;
    }
    if (sb < g.spec_pad / KBLK) {
      b.src = ks + (long long)sb * KBLK * D * 2;
      b.nvalid = min(KBLK, g.nspec - sb * KBLK);
      b.kind = 1;
      b.tile = -1;
      ++sb;
      return true;
    }
    if (landmarks && lb < g.T_pad / KBLK) {
      b.src = lm + (long long)lb * LM_KEY_BLOCK;
      b.nvalid = min(KBLK, g.T - lb * KBLK);
      b.kind = 2;
      b.tile = lb;
      ++lb;
      return true;
    }
    return false;
  }
};

// This wave's 1 KB share (key rows 8w..8w+7) of a block's async copy into
// LDS, swizzled as load_kfrag reads it: 16-byte column c of key row k at
// column c ^ (k % 8).
__device__ __forceinline__ void cv_stage(char* dst, const char* src, int wave, int lane) {
  const int P = wave * 1024 + lane * 16;
  const int key = P >> 7, col = (P >> 4) & 7;
  __builtin_amdgcn_global_load_lds((const void*)(src + key * 128 + ((col ^ (key & 7)) << 4)),
                                   (lds_void*)(dst + P), 16, 0, 0);
}

__global__ void __launch_bounds__(CV_WAVES * 64) coverage_kernel(Geom g, const u16* __restrict__ Q,
                                                                 const u16* __restrict__ Kt,
                                                                 const u16* __restrict__ Ks,
                                                                 const u16* __restrict__ LM,
                                                                 const unsigned* __restrict__ selmask, int nwords,
                                                                 float* __restrict__ cov, float* __restrict__ err) {
  __shared__ __attribute__((aligned(1024))) char ring[CV_RING][CV_BLOCK];
  const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
  const int lg = lane >> 4, tl16 = lane & 15;
  const int h = blockIdx.y;
  const int t = blockIdx.x * CV_WAVES + wave;
  const bool tvalid = t < g.T;
  const int f = tvalid ? frame_of_tile(g, t) : 0, tl = tvalid ? t - f * g.tpf : 0;
  const int nrows = tvalid ? tile_n(g, tl) : 0;

  // query fragments of the four slots (rows s*16 + lane%16), zero past the tile
  bf16x8 q[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int j = s * 16 + tl16;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (j < nrows)
        w = *(const uint4*)(Q + cv_token(g, f, tl, j) * g.in_tok + (long long)h * g.in_head + ds * 32 + 8 * lg);
      q[s][ds] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  const char* kt = (const char*)(Kt + (long long)h * g.slots * D);
  const char* ks = (const char*)(Ks + (long long)h * g.spec_pad * D);
  const char* lmh = (const char*)LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE;
  const cmask_ptr mrow = (cmask_ptr)(selmask + ((long long)h * g.T + (tvalid ? t : 0)) * nwords);

  float mx[4], acc[4][4];  // running max (lane part); kept, omitted, special, landmark sums
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    mx[s] = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[s][c] = 0.f;
  }
  float m2[4];  // log2-scaled row maximum (second pass)

  for (int pass = 0; pass < 2; ++pass) {
    CvStream st(g, kt, ks, lmh, pass == 1);
    // blocks i, i + 1, i + 2 of the stream (named, not an indexed array, so
    // that they stay in registers)
    CvBlock b_cur, b_n1, b_n2;
    int nq = 0;
    // prime the ring two blocks ahead
    if (st.next(b_cur)) {
      cv_stage(ring[0], b_cur.src, wave, lane);
      nq = 1;
      if (st.next(b_n1)) {
        cv_stage(ring[1], b_n1.src, wave, lane);
        nq = 2;
      }
    }
    for (int i = 0; i < nq; ++i) {
      // issue block i + 2 (its slot held block i - 2, finished before the
      // previous barrier), then wait for block i and meet
      if (nq == i + 2 && st.next(b_n2)) {
        cv_stage(ring[(i + 2) % CV_RING], b_n2.src, wave, lane);
        ++nq;
      }
      if (nq > i + 2)
        __builtin_amdgcn_s_waitcnt(0x0F70 | 2);  // vmcnt(2): blocks i+1, i+2 may still fly
      else if (nq > i + 1)
        __builtin_amdgcn_s_waitcnt(0x0F70 | 1);
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);
      ring_barrier();
      const CvBlock b = b_cur;
      b_cur = b_n1;
      b_n1 = b_n2;
      const char* kb = ring[i % CV_RING];
      bf16x8 kf[2][2];
      load_kfrag(kb, 0, lane, kf);
      // initial S^T values: -inf past the block's real keys; for a landmark
      // block, log2(n_u)/C for the omitted tiles and -inf for the kept ones
      f32x4 b0, b1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        b0[r] = 4 * lg + r < b.nvalid ? 0.f : -INFINITY;
        b1[r] = 16 + 4 * lg + r < b.nvalid ? 0.f : -INFINITY;
      }
      int cls = 2;  // special
      if (b.kind == 0) cls = ((mrow[b.tile >> 5] >> (b.tile & 31)) & 1u) ? 0 : 1;
      if (b.kind == 2) {
        // log2 n_u of the block's tiles: row 32 of the landmark key block,
        // read from memory (the ring holds rows 0..31)
        float l2n[8];
        load_row8(b.src + LM_LOG2N_ROW * 128, lane, l2n);
        const unsigned kept = mrow[b.tile];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (4 * lg + r < b.nvalid)
            b0[r] = ((kept >> (4 * lg + r)) & 1u) ? -INFINITY : l2n[r] * (1.0f / QK_LOG2);
          if (16 + 4 * lg + r < b.nvalid)
            b1[r] = ((kept >> (16 + 4 * lg + r)) & 1u) ? -INFINITY : l2n[4 + r] * (1.0f / QK_LOG2);
        }
        cls = 3;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s * 16 >= nrows) continue;  // uniform: the slot has no rows
        f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][0], q[s][0], b0, 0, 0, 0);
        f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][0], q[s][0], b1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][1], q[s][1], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][1], q[s][1], a1, 0, 0, 0);
        if (pass == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) mx[s] = __builtin_fmaxf(mx[s], __builtin_fmaxf(a0[r], a1[r]));
        } else {
          float sum = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sum += __builtin_amdgcn_exp2f(fmaf(a0[r], QK_LOG2, -m2[s])) +
                   __builtin_amdgcn_exp2f(fmaf(a1[r], QK_LOG2, -m2[s]));
          acc[s][cls] += sum;
        }
      }
    }
    ring_barrier();  // the ring is reused by the next pass
    if (pass == 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) m2[s] = xmax32(xmax16(mx[s])) * QK_LOG2;  // row max over the lane groups
    }
  }

  // per row: the four lane groups' sums, then the coverage and landmark
  // error of the rows, averaged over the tile
  float csum = 0.f, esum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float kp = xsum32(xsum16(acc[s][0])), op = xsum32(xsum16(acc[s][1]));
    const float sp = xsum32(xsum16(acc[s][2])), lp = xsum32(xsum16(acc[s][3]));
    const bool row = lg == 0 && s * 16 + tl16 < nrows;  // each row once
    if (row) {
      csum += kp / (kp + op + sp);
      esum += op > 0.f ? 1.0f - lp / op : 0.f;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    csum += __shfl_xor(csum, o, 64);
    esum += __shfl_xor(esum, o, 64);
  }
  if (tvalid && lane == 0) {
    cov[(long long)h * g.T + t] = csum / nrows;
    err[(long long)h * g.T + t] = esum / nrows;
  }
}

hipError_t launch_coverage(const Geom& g, const u16* Q, const u16* Kt, const u16* Ks, const u16* LM,
                           const unsigned* selmask, float* cov, float* err, hipStream_t s) {
  const int nwords = (g.T + 31) / 32;
  hipLaunchKernelGGL(coverage_kernel, dim3((g.T + CV_WAVES - 1) / CV_WAVES, g.H), dim3(CV_WAVES * 64), 0, s, g, Q,
                     Kt, Ks, LM, selmask, nwords, cov, err);
  return hipGetLastError();
}

}  // namespace zebra
