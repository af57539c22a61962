// Tile-sparse and dense softmax attention for gfx950 (bf16 MFMA, LDS-shared
// key/value tiles, fixed per-row softmax offsets).
//
// Zebra3D pages, "Linear-centered stages plus tile-sparse stages": kept key
// tiles keep full softmax interactions, omitted tiles are seen through their
// mean-K/V landmark, special-token keys are always visible, special query
// rows are dense and every patch query keeps its own key. "Global attention
// dominates runtime as views grow": dense attention over all tokens is the
// baseline this stage replaces.
//
// Work decomposition. A workgroup of 4 waves owns G query groups of one head
// (a query group is a patch query tile of <= 64 rows, or 64 special rows).
// Row block j (16 rows) of group s belongs to wave (s + j) % 4, so every wave
// holds at most one 16-row slot of every group and all four waves do the
// same work for every key block. The workgroup streams staged items through
// a ring of NBUF LDS buffers (async global->LDS loads, exact vmcnt waits,
// one barrier per item):
//   1. bound pass: every landmark block and every special-key block, S only;
//   2. the landmark blocks again (tile-sparse only; a group masks the tiles
//      it kept), the UNION of the tiles the groups kept in ascending order
//      (all tiles when dense) and the special blocks, with P.V;
// then each group's self key.
//
// Softmax offsets. Instead of a running max (a per-block max, cross-lane
// reductions and O rescaling), each row i uses one offset M_i that is >=
// every logit it can see, found in the bound pass: for a tile u and every
// key j of u, q.k_j <= q.kbar_u + |q| r_u (r_u: the tile's key radius);
// a landmark's logit is q.kbar_u/8 + ln n_u; special logits are exact. With
// p = exp2(x - M_i) <= 1 nothing overflows. The row's own key is always
// visible, so M_i minus the own logit bounds how far below 1 the largest p
// can be; rows where that gap exceeds SAFE_GAP (log2 units) are flagged and
// recomputed by an exact online-softmax kernel (attn_exact.hip).
//
// Per 32-key block and 16-row slot: S^T = K Q^T (4 v_mfma_f32_16x16x32_bf16,
// A = keys from LDS, B = Q in registers), p = exp2(S*log2(e)/8 - M),
// O^T += V^T P^T (4 MFMAs; lane group g holds keys 4g..4g+3 of both 16-key
// halves of S^T, the k-slot order of the value fragment, whose 32-key
// blocks are stored [64 channels][32] with keys permuted by value_pos).
// LDS layouts are XOR-swizzled at 16-byte granularity (keys: column ^ key%8,
// values: column ^ (channel/2)%4) so fragment reads are bank-conflict free;
// the swizzle is applied through the per-lane source address of the async
// loads, which write LDS linearly.

#include "attn_common.hpp"

namespace zebra {

template <int G>
struct WaveState {
  bf16x8 q[G][2];  // B operand of each slot: query (lane%16), channels ds*32+8g..+7
  f32x4 o[G][4];   // O^T of each slot: channel db*16+4g+r, query lane%16
  float l[G];      // lane-partial row sums
  float negm[G];   // -M (log2 units); during the bound pass: the running bound
  float qnc[G];    // |q| * log2(e)/8
};

template <int G>
__device__ __forceinline__ void qk(const WaveState<G>& st, int s, const bf16x8 kf[2][2], f32x4& s0, f32x4& s1) {
  s0 = f32x4{0.f, 0.f, 0.f, 0.f};
  s1 = s0;
  s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][0], st.q[s][0], s0, 0, 0, 0);
  s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][0], st.q[s][0], s1, 0, 0, 0);
  s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][1], st.q[s][1], s0, 0, 0, 0);
  s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][1], st.q[s][1], s1, 0, 0, 0);
}

// p (8 lane values, in S^T order) -> row sums and O^T += V^T P^T.
template <int G>
__device__ __forceinline__ void accumulate(WaveState<G>& st, int s, const float p[8], const bf16x8 vf[4]) {
  st.l[s] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  uint4 w;
  w.x = pack_bf16(p[0], p[1]);
  w.y = pack_bf16(p[2], p[3]);
  w.z = pack_bf16(p[4], p[5]);
  w.w = pack_bf16(p[6], p[7]);
  const bf16x8 P = __builtin_bit_cast(bf16x8, w);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    st.o[s][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], P, st.o[s][db], 0, 0, 0);
}

// Main pass over one staged 32-key block for every user slot:
// p = exp2(s*C - M), times n_u for a landmark (its logit carries + ln n_u);
// keys past nvalid, and landmarks of tiles the slot's group kept, drop out.
template <int G>
__device__ __forceinline__ void main_block(WaveState<G>& st, unsigned users, const char* kb, int key0,
                                           const char* vb, int nvalid, cmask_ptr mrow0, int nwords,
                                           int lb, int lane) {
  bf16x8 kf[2][2], vf[4];
  load_kfrag(kb, key0, lane, kf);
  load_vfrag(vb, lane, vf);
  const int lg = lane >> 4;
  const bool is_lm = lb >= 0;
  float nmul[8];  // n_u = 2^log2(n_u) of the lane's 8 landmarks
  if (is_lm) {
    load_row8(kb + LM_LOG2N_ROW * 128, lane, nmul);
#pragma unroll
    for (int i = 0; i < 8; ++i) nmul[i] = __builtin_amdgcn_exp2f(nmul[i]);
  }
  const unsigned valid = lane_valid_mask(nvalid, lane);
#pragma unroll
  for (int s = 0; s < G; ++s) {
    if (!((users >> s) & 1u)) continue;
    unsigned keep = valid;
    if (is_lm) {
      const unsigned kept = mrow0[(long long)s * nwords + lb];
      keep &= ~(((kept >> (4 * lg)) & 0xFu) | (((kept >> (16 + 4 * lg)) & 0xFu) << 4));
    }
    f32x4 s0, s1;
    qk(st, s, kf, s0, s1);
    const float nm = st.negm[s];
    float p[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], QK_LOG2, nm));
      p[4 + r] = __builtin_amdgcn_exp2f(fmaf(s1[r], QK_LOG2, nm));
    }
    if (is_lm) {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] *= nmul[i];
    }
    if (keep != 0xFFu) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (!((keep >> i) & 1u)) p[i] = 0.f;
    }
    accumulate(st, s, p, vf);
  }
}

// Bound pass over one staged 32-key block: raises each row's running bound
// by max over keys of s*C + max(log2 n_u, |q| r_u C) for a landmark block
// (an upper bound of the logits of the tile's tokens and of its landmark),
// or by the exact logits s*C of a special block's valid keys.
template <int G>
__device__ __forceinline__ void bound_block(WaveState<G>& st, unsigned slots, const char* kb, bool is_lm,
                                            int nvalid, int lane) {
  bf16x8 kf[2][2];
  load_kfrag(kb, 0, lane, kf);
  float l2n[8], rad[8];
  if (is_lm) {
    load_row8(kb + LM_LOG2N_ROW * 128, lane, l2n);
    load_row8(kb + LM_RADIUS_ROW * 128, lane, rad);
  } else {
    const unsigned valid = lane_valid_mask(nvalid, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      l2n[i] = ((valid >> i) & 1u) ? 0.f : -INFINITY;
      rad[i] = 0.f;
    }
  }
#pragma unroll
  for (int s = 0; s < G; ++s) {
    if (!((slots >> s) & 1u)) continue;
    f32x4 s0, s1;
    qk(st, s, kf, s0, s1);
    float b = st.negm[s];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      b = __builtin_fmaxf(b, fmaf(s0[r], QK_LOG2, __builtin_fmaxf(l2n[r], st.qnc[s] * rad[r])));
      b = __builtin_fmaxf(b, fmaf(s1[r], QK_LOG2, __builtin_fmaxf(l2n[4 + r], st.qnc[s] * rad[4 + r])));
    }
    st.negm[s] = b;
  }
}

template <int G>
__device__ __forceinline__ void attend_item(const Geom& g, const AttnArgs& A, int work, int items_per_head,
                                            int patch_items, char* lds, int* qcode, unsigned* qusers,
                                            int* unsafe) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = lane >> 4, tl = lane & 15;
  const int h = work / items_per_head;
  const int item = work - h * items_per_head;
  const QueryGroups qg(g, item, patch_items, G, wave);
  const bool sparse = A.sparse && qg.patch;
  const long long rs = (long long)g.H * D;
  const u16* Kt16 = A.Kt + (long long)h * g.slots * D;
  const u16* Vt16 = A.Vt + (long long)h * g.slots * D;
  const u16* Ks16 = A.Ks + (long long)h * g.spec_pad * D;
  const u16* Vs16 = A.Vs + (long long)h * g.spec_pad * D;

  unsigned slots = 0u, valid_groups = 0u;
#pragma unroll
  for (int s = 0; s < G; ++s) {
    const int n = qg.rows(s);
    if (qg.row_block(s) * 16 < n) slots |= 1u << s;
    if (n > 0) valid_groups |= 1u << s;
  }

  WaveState<G> st;
  float own[G];  // own-key logit (log2 units): a visible key of every row
#pragma unroll
  for (int s = 0; s < G; ++s) {
    const int j = qg.row_block(s) * 16 + tl;
    const bool ok = ((slots >> s) & 1u) && j < qg.rows(s);
    float qq = 0.f, qko = 0.f;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 w = make_uint4(0, 0, 0, 0), kw = make_uint4(0, 0, 0, 0);
      if (ok) {
        w = *(const uint4*)(A.Q + qg.token(s, j) * rs + h * D + ds * 32 + 8 * lg);
        kw = *(const uint4*)((qg.patch ? Kt16 : Ks16) + qg.own_slot(s, j) * D + ds * 32 + 8 * lg);
      }
      st.q[s][ds] = __builtin_bit_cast(bf16x8, w);
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kw);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float a = (float)st.q[s][ds][m];
        qq = fmaf(a, a, qq);
        qko = fmaf(a, (float)kv[m], qko);
      }
    }
    qq = xsum32(xsum16(qq));
    qko = xsum32(xsum16(qko));
    st.qnc[s] = sqrtf(qq) * QK_LOG2 * 1.0001f;
    own[s] = qko * QK_LOG2;
    st.negm[s] = own[s];  // running bound during the bound pass
    st.l[s] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[s][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const char* lmh = (const char*)A.LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE;
  // kept-tile bitmap row of group s: mrow0 + s * nwords (patch groups are
  // consecutive query tiles)
  const cmask_ptr mrow0 =
      (cmask_ptr)(sparse ? A.selmask + ((long long)h * g.T + qg.gid0) * A.nwords : A.selmask);
  auto mask_word = [&](int s, int word) -> unsigned { return mrow0[(long long)s * A.nwords + word]; };

  // Item codes. Bound pass (flag BOUND): T + lb landmark block lb < nlb_all,
  // T + nlb_all + b special block b. Main pass: u < T token tile u,
  // T + lb landmark block (tile-sparse only), T + nlb + b special block b.
  const int nlb_all = g.T_pad / KBLK;
  const int nlb = sparse ? nlb_all : 0;
  const int nsb = g.spec_pad / KBLK;
  constexpr int BOUND = 1 << 30;
  int phase = 0, w = -1, cnt = 0;
  unsigned bits = 0u;
  auto next = [&](int& code, unsigned& users) -> bool {
    if (phase == 0) {  // bound pass
      if (cnt < nlb_all + nsb) {
        code = BOUND | (g.T + cnt++);
        users = valid_groups;
        return true;
      }
      phase = 1;
      cnt = 0;
    }
    if (phase == 1) {  // landmark blocks not kept entirely by every group
      while (cnt < nlb) {
        const int lb = cnt++;
        unsigned us = 0u;
#pragma unroll
        for (int s = 0; s < G; ++s)
          if (((valid_groups >> s) & 1u) && mask_word(s, lb) != 0xFFFFFFFFu) us |= 1u << s;
        if (us) {
          code = g.T + lb;
          users = us;
          return true;
        }
      }
      phase = 2;
    }
    if (phase == 2) {  // union of the kept tiles (every tile when dense)
      while (bits == 0u) {
        if (++w >= A.nwords) {
          phase = 3;
          cnt = 0;
          break;
        }
        if (sparse) {
          unsigned un = 0u;
#pragma unroll
          for (int s = 0; s < G; ++s)
            if ((valid_groups >> s) & 1u) un |= mask_word(s, w);
          bits = un;
        } else {
          const int rem = g.T - w * 32;
          bits = rem >= 32 ? 0xFFFFFFFFu : ((1u << rem) - 1u);
        }
      }
      if (phase == 2) {
        const int b = __builtin_ctz(bits);
        bits &= bits - 1u;
        code = w * 32 + b;
        if (sparse) {
          unsigned us = 0u;
#pragma unroll
          for (int s = 0; s < G; ++s)
            if ((valid_groups >> s) & 1u) us |= ((mask_word(s, w) >> b) & 1u) << s;
          users = us;
        } else {
          users = valid_groups;
        }
        return true;
      }
    }
    if (cnt < nsb) {  // special blocks
      code = g.T + nlb + cnt++;
      users = valid_groups;
      return true;
    }
    return false;
  };
  auto issue = [&](int code_in, int buf) {
    const int cin = uni(code_in);
    const int code = cin & ~BOUND;
    char* d = lds + buf * LDS_BUF;
    const char *ksrc, *vsrc;
    int kbytes, vbytes;
    int lb = -1, sb = -1;
    if (cin & BOUND) {
      if (code < g.T + nlb_all) lb = code - g.T;
      else sb = code - g.T - nlb_all;
    } else if (code >= g.T) {
      if (code < g.T + nlb) lb = code - g.T;
      else sb = code - g.T - nlb;
    }
    if (lb >= 0) {
      ksrc = lmh + (long long)lb * LM_KEY_BLOCK;
      vsrc = lmh + (long long)nlb_all * LM_KEY_BLOCK + (long long)lb * (KBLK * D * 2);
      kbytes = LM_KEY_BLOCK;
      vbytes = KBLK * D * 2;
    } else if (sb >= 0) {
      ksrc = (const char*)Ks16 + (long long)sb * KBLK * D * 2;
      vsrc = (const char*)Vs16 + (long long)sb * KBLK * D * 2;
      kbytes = vbytes = KBLK * D * 2;
    } else {
      const int fu = code / g.tpf, tu = code - fu * g.tpf;
      const long long base = (long long)fu * g.slots_pf + tile_off(g, tu);
      kbytes = vbytes = pad32(tile_n(g, tu)) * D * 2;
      ksrc = (const char*)Kt16 + base * D * 2;
      vsrc = (const char*)Vt16 + base * D * 2;
    }
    stage_keys(d, ksrc, kbytes, wave, lane);
    stage_vals(d + LDS_V, vsrc, vbytes, wave, lane);
  };
  bool bound_done = false;
  auto finish_bound = [&]() {
    // M = max over the row's lanes; flag rows whose bound is too far above
    // their own logit (underflow risk) for the exact kernel
    bool bad = false;
#pragma unroll
    for (int s = 0; s < G; ++s) {
      const float m = xmax32(xmax16(st.negm[s]));
      const bool okrow = ((slots >> s) & 1u) && qg.row_block(s) * 16 + tl < qg.rows(s);
      if (okrow && m - own[s] > SAFE_GAP) bad = true;
      st.negm[s] = -m;
    }
    if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) atomicOr(unsafe + work, 1);
  };

  int issued = 0;
  bool done = false;
  for (int j = 0; j < NBUF - 1; ++j) {
    int c;
    unsigned u;
    if (!next(c, u)) {
      done = true;
      break;
    }
    if (threadIdx.x == 0) {
      qcode[j] = c;
      qusers[j] = u;
    }
    issue(c, j);
    ++issued;
  }
  for (int i = 0; i < issued; ++i) {
    wait_loads(min(NBUF - 2, issued - i - 1));
    ring_barrier();
    if (!done) {
      int c;
      unsigned u;
      if (next(c, u)) {
        const int jn = issued % NBUF;
        if (threadIdx.x == 0) {
          qcode[jn] = c;
          qusers[jn] = u;
        }
        issue(c, jn);
        ++issued;
      } else {
        done = true;
      }
    }
    const int buf = i % NBUF;
    const int cin = uni(qcode[buf]);
    const int code = cin & ~BOUND;
    const unsigned us = (unsigned)uni((int)qusers[buf]) & slots;
    const char* kb = lds + buf * LDS_BUF;
    if (cin & BOUND) {
      if (us) {
        const bool is_lm = code < g.T + nlb_all;
        bound_block<G>(st, us, kb, is_lm, is_lm ? 32 : min(32, g.nspec - (code - g.T - nlb_all) * KBLK),
                       lane);
      }
      continue;
    }
    if (!bound_done) {
      finish_bound();
      bound_done = true;
    }
    if (!us) continue;
    int nkeys, lb = -1;
    if (code < g.T) {
      nkeys = tile_n(g, code % g.tpf);
    } else if (code < g.T + nlb) {
      nkeys = 32;
      lb = code - g.T;
    } else {
      nkeys = min(32, g.nspec - (code - g.T - nlb) * KBLK);
    }
#pragma nounroll
    for (int k0 = 0; k0 < nkeys; k0 += KBLK)
      main_block<G>(st, us, kb, k0, kb + LDS_V + k0 * 128, nkeys - k0, mrow0, A.nwords, lb, lane);
  }
  if (!bound_done) finish_bound();
  ring_barrier();

  // self key of patch rows whose own tile was not kept
  if (sparse) {
#pragma unroll
    for (int s = 0; s < G; ++s) {
      if (!((slots >> s) & 1u)) continue;
      const int t = qg.gid0 + s;
      if ((mask_word(s, t >> 5) >> (t & 31)) & 1u) continue;
      const int j = qg.row_block(s) * 16 + tl;
      const bool okrow = j < qg.rows(s);
      const float p = okrow ? __builtin_amdgcn_exp2f(own[s] + st.negm[s]) : 0.f;
      st.l[s] += (lg == 0 ? p : 0.f);
      const long long slot = qg.own_slot(s, j);
      const long long vblk = slot / KBLK;
      const int pos = value_pos((int)(slot % KBLK));
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = db * 16 + 4 * lg + r;
          const float v = okrow ? bf2f(Vt16[(vblk * D + d) * KBLK + pos]) : 0.f;
          st.o[s][db][r] = fmaf(p, v, st.o[s][db][r]);
        }
    }
  }

  // finalize: O = O^T / l; row = query (rb*16 + lane%16), channels db*16+4g+r
#pragma unroll
  for (int s = 0; s < G; ++s) {
    if (!((slots >> s) & 1u)) continue;
    const float inv = 1.0f / xsum32(xsum16(st.l[s]));
    const int j = qg.row_block(s) * 16 + tl;
    if (j < qg.rows(s)) {
      u16* orow = A.O + qg.token(s, j) * rs + h * D;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint2 wv;
        wv.x = pack_bf16(st.o[s][db][0] * inv, st.o[s][db][1] * inv);
        wv.y = pack_bf16(st.o[s][db][2] * inv, st.o[s][db][3] * inv);
        *(uint2*)(orow + db * 16 + 4 * lg) = wv;
      }
    }
  }
}

// One work item (head, G query groups) per workgroup; items first..first+n-1
// of the head-major numbering (blockIdx.x -> head h, item within head).
template <int G>
__global__ void __launch_bounds__(ATT_THREADS, 2) attn_kernel(Geom g, AttnArgs A, int items_per_head,
                                                              int patch_items, int first, int count,
                                                              int* unsafe) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * LDS_BUF];
  __shared__ int qcode[NBUF];
  __shared__ unsigned qusers[NBUF];
  const int h = blockIdx.x / count, i = blockIdx.x - h * count;
  attend_item<G>(g, A, h * items_per_head + first + i, items_per_head, patch_items, lds, qcode, qusers,
                 unsafe);
}

// Patch items (one workgroup per item, head-major), then the special-row
// items (dense over every key, one workgroup each).
hipError_t launch_attn_fast(const Geom& g, const AttnArgs& a, int* unsafe, hipStream_t s) {
  const ItemCounts ic(g, ATTN_GROUPS);
  hipLaunchKernelGGL(attn_kernel<ATTN_GROUPS>, dim3(ic.patch_items * g.H), dim3(ATT_THREADS), 0, s, g, a,
                     ic.per_head, ic.patch_items, 0, ic.patch_items, unsafe);
  const int spec_items = ic.per_head - ic.patch_items;
  if (spec_items > 0)
    hipLaunchKernelGGL(attn_kernel<ATTN_GROUPS>, dim3(spec_items * g.H), dim3(ATT_THREADS), 0, s, g, a,
                       ic.per_head, ic.patch_items, ic.patch_items, spec_items, unsafe);
  return hipGetLastError();
}

}  // namespace zebra
