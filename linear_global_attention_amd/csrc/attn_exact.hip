// Exact-offset fallback of the attention kernel (gfx950).
//
// Same staging and visible key set as attn.hip, but with an online softmax:
// a running row max (raised only when a block exceeds it by more than TAU,
// then O and l are rescaled). Its work items hold ATTN_GROUPS query groups;
// it recomputes only the items with a group that attn_bound_kernel flagged
// (a row whose logit bound was too loose to use as a fixed offset); every
// other workgroup exits at once.
#include "attn_common.hpp"

namespace zebra {

constexpr float TAU = 8.0f;  // lazy-max headroom, log2 units
constexpr float M_INIT = -1.0e30f;

template <int G>
struct ExactState {
  bf16x8 q[G][2];
  f32x4 o[G][4];
  float m[G];  // running (lazy) max, log2 units
  float l[G];  // lane-partial row sums
};

// One 32-key block of slot s: x = logits in log2 units (masked keys -inf).
template <int G>
__device__ __forceinline__ void exact_softmax_pv(ExactState<G>& st, int s, float x[8], const bf16x8 vf[4]) {
  float bm = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) bm = __builtin_fmaxf(bm, x[i]);
  bm = xmax32(xmax16(bm));
  if (bm > st.m[s] + TAU) {  // row-uniform (reduced over the row's 4 lanes)
    const float alpha = __builtin_amdgcn_exp2f(st.m[s] - bm);
    st.m[s] = bm;
    st.l[s] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[s][db] *= alpha;
  }
  const float m = st.m[s];
  float p[8], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = __builtin_amdgcn_exp2f(x[i] - m);
    ps += p[i];
  }
  st.l[s] += ps;
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

// One staged 32-key block for every user slot. Landmark blocks (lb >= 0)
// add log2 n_u and mask the tiles a slot's group kept.
template <int G>
__device__ __forceinline__ void exact_block(ExactState<G>& st, unsigned users, const char* kb, int key0,
                                            const char* vb, int nvalid, cmask_ptr mrow0, int nwords,
                                            int lb, int lane) {
  bf16x8 kf[2][2], vf[4];
  load_kfrag(kb, key0, lane, kf);
  load_vfrag(vb, lane, vf);
  const int lg = lane >> 4;
  float bias[8];
  if (lb >= 0) {
    load_row8(kb + LM_LOG2N_ROW * 128, lane, bias);
  } else {
    const unsigned valid = lane_valid_mask(nvalid, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) bias[i] = ((valid >> i) & 1u) ? 0.f : -INFINITY;
  }
#pragma unroll
  for (int s = 0; s < G; ++s) {
    if (!((users >> s) & 1u)) continue;
    const unsigned kept = lb >= 0 ? mrow0[(long long)s * nwords + lb] : 0u;
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][0], st.q[s][0], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][0], st.q[s][0], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][1], st.q[s][1], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][1], st.q[s][1], s1, 0, 0, 0);
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool k0 = (kept >> (4 * lg + r)) & 1u, k1 = (kept >> (16 + 4 * lg + r)) & 1u;
      x[r] = k0 ? -INFINITY : fmaf(s0[r], QK_LOG2, bias[r]);
      x[4 + r] = k1 ? -INFINITY : fmaf(s1[r], QK_LOG2, bias[4 + r]);
    }
    exact_softmax_pv(st, s, x, vf);
  }
}

template <int G>
__global__ void __launch_bounds__(ATT_THREADS, 1) attn_exact_kernel(Geom g, AttnArgs A, int items_per_head,
                                                                    int patch_items, const int* flags) {
  const int work = blockIdx.x;
  {  // any flagged group in this item? (uniform over the workgroup)
    const int h = work / items_per_head, item = work - h * items_per_head;
    const FastItems fi(g);
    const bool patch = item < patch_items;
    const int gid0 = (patch ? 0 : g.T) + (patch ? item : item - patch_items) * G;
    const int gend = patch ? g.T : fi.groups_per_head;
    int any = 0;
    for (int s = 0; s < G && gid0 + s < gend; ++s) any |= flags[(long long)h * fi.groups_per_head + gid0 + s];
    if (!any) return;
  }
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * LDS_BUF];
  __shared__ int qcode[NBUF];
  __shared__ unsigned qusers[NBUF];
  const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
  const int lg = lane >> 4, tl = lane & 15;
  const int h = work / items_per_head;
  const int item = work - h * items_per_head;
  const QueryGroups qg(g, item, patch_items, G, wave);
  const bool sparse = A.sparse && qg.patch;
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
  ExactState<G> st;
#pragma unroll
  for (int s = 0; s < G; ++s) {
    const int j = qg.row_block(s) * 16 + tl;
    const bool ok = ((slots >> s) & 1u) && j < qg.rows(s);
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (ok) w = *(const uint4*)(A.Q + qg.token(s, j) * g.in_tok + h * g.in_head + ds * 32 + 8 * lg);
      st.q[s][ds] = __builtin_bit_cast(bf16x8, w);
    }
    st.m[s] = M_INIT;
    st.l[s] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[s][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const char* lmh = (const char*)A.LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE;
  const cmask_ptr mrow0 =
      (cmask_ptr)(sparse ? A.selmask + ((long long)h * g.T + qg.gid0) * A.nwords : A.selmask);
  auto mask_word = [&](int s, int word) -> unsigned { return mrow0[(long long)s * A.nwords + word]; };

  // items: T + lb landmark block (tile-sparse), u < T tile u of the union
  // (every tile when dense), T + nlb + b special block b
  const int nlb_all = g.T_pad / KBLK;
  const int nlb = sparse ? nlb_all : 0;
  const int nsb = g.spec_pad / KBLK;
  int phase = 1, w = -1, cnt = 0;
  unsigned bits = 0u;
  auto next = [&](int& code, unsigned& users) -> bool {
    if (phase == 1) {
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
    if (phase == 2) {
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
        unsigned us = valid_groups;
        if (sparse) {
          us = 0u;
#pragma unroll
          for (int s = 0; s < G; ++s)
            if ((valid_groups >> s) & 1u) us |= ((mask_word(s, w) >> b) & 1u) << s;
        }
        users = us;
        return true;
      }
    }
    if (cnt < nsb) {
      code = g.T + nlb + cnt++;
      users = valid_groups;
      return true;
    }
    return false;
  };
  auto issue = [&](int code_in, int buf) {
    const int code = uni(code_in);
    char* d = lds + buf * LDS_BUF;
    const char *ksrc, *vsrc;
    int kbytes, vbytes;
    if (code < g.T) {
      const int fu = code / g.tpf, tu = code - fu * g.tpf;
      const long long base = (long long)fu * g.slots_pf + tile_off(g, tu);
      kbytes = vbytes = pad32(tile_n(g, tu)) * D * 2;
      ksrc = (const char*)Kt16 + base * D * 2;
      vsrc = (const char*)Vt16 + base * D * 2;
    } else if (code < g.T + nlb) {
      const long long lb = code - g.T;
      ksrc = lmh + lb * LM_KEY_BLOCK;
      vsrc = lmh + (long long)nlb_all * LM_KEY_BLOCK + lb * (KBLK * D * 2);
      kbytes = LM_KEY_BLOCK;
      vbytes = KBLK * D * 2;
    } else {
      const long long b = code - g.T - nlb;
      ksrc = (const char*)Ks16 + b * KBLK * D * 2;
      vsrc = (const char*)Vs16 + b * KBLK * D * 2;
      kbytes = vbytes = KBLK * D * 2;
    }
    stage_keys(d, ksrc, kbytes, wave, lane);
    stage_vals(d + LDS_V, vsrc, vbytes, wave, lane);
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
    const int code = uni(qcode[buf]);
    const unsigned us = (unsigned)uni((int)qusers[buf]) & slots;
    if (!us) continue;
    const char* kb = lds + buf * LDS_BUF;
    int nkeys, lb = -1;
    if (code < g.T) {
      nkeys = tile_n(g, code % g.tpf);
    } else if (code < g.T + nlb) {
      nkeys = 32;
      lb = code - g.T;
    } else {
      nkeys = min(32, g.nspec - (code - g.T - nlb) * KBLK);
    }
    for (int k0 = 0; k0 < nkeys; k0 += KBLK)
      exact_block<G>(st, us, kb, k0, kb + LDS_V + k0 * 128, nkeys - k0, mrow0, A.nwords, lb, lane);
  }
  ring_barrier();

  if (sparse) {  // self key of patch rows whose own tile was not kept
#pragma unroll
    for (int s = 0; s < G; ++s) {
      if (!((slots >> s) & 1u)) continue;
      const int t = qg.gid0 + s;
      if ((mask_word(s, t >> 5) >> (t & 31)) & 1u) continue;
      const int j = qg.row_block(s) * 16 + tl;
      const bool okrow = j < qg.rows(s);
      const long long slot = qg.own_slot(s, j);
      float dot = 0.f;
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        const uint4 kw = *(const uint4*)(Kt16 + slot * D + ds * 32 + 8 * lg);
        const bf16x8 kv = __builtin_bit_cast(bf16x8, kw);
#pragma unroll
        for (int m = 0; m < 8; ++m) dot = fmaf((float)st.q[s][ds][m], (float)kv[m], dot);
      }
      dot = xsum32(xsum16(dot));
      const float x = okrow ? dot * QK_LOG2 : M_INIT;
      const float mn = __builtin_fmaxf(st.m[s], x);
      const float alpha = __builtin_amdgcn_exp2f(st.m[s] - mn);
      const float p = __builtin_amdgcn_exp2f(x - mn);
      st.m[s] = mn;
      st.l[s] = st.l[s] * alpha + (lg == 0 ? p : 0.f);
      const long long vblk = slot / KBLK;
      const int pos = value_pos((int)(slot % KBLK));
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = db * 16 + 4 * lg + r;
          const float v = okrow ? bf2f(Vt16[(vblk * D + d) * KBLK + pos]) : 0.f;
          st.o[s][db][r] = st.o[s][db][r] * alpha + p * v;
        }
    }
  }

#pragma unroll
  for (int s = 0; s < G; ++s) {
    if (!((slots >> s) & 1u)) continue;
    const float inv = 1.0f / xsum32(xsum16(st.l[s]));
    const int j = qg.row_block(s) * 16 + tl;
    if (j < qg.rows(s)) {
      u16* orow = A.O + qg.token(s, j) * g.out_tok + h * g.out_head;
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

// Recomputes the work items that hold a flagged group (one int per group,
// head-major, as written by attn_bound_kernel).
hipError_t launch_attn_exact(const Geom& g, const AttnArgs& a, const int* flags, hipStream_t s) {
  const ItemCounts ic(g, ATTN_GROUPS);
  hipLaunchKernelGGL(attn_exact_kernel<ATTN_GROUPS>, dim3(ic.total), dim3(ATT_THREADS), 0, s, g, a,
                     ic.per_head, ic.patch_items, flags);
  return hipGetLastError();
}

}  // namespace zebra
