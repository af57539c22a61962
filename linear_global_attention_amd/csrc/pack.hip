// Tile-major K/V packing and mean-K/V landmarks for gfx950.
//
// Zebra3D pages, "Speedup scales with the number of input views": the
// sparse-stage kernels pack the key/value sequence into tile-major order.
// "Linear-centered stages plus tile-sparse stages": omitted tiles are
// summarised as mean key/value landmarks.
//
// Both kernels are pure HBM streams: one workgroup per (tile or 32 special
// tokens, head). Keys keep their row-major [slot][64] layout so the attention
// kernel reads 16-byte key fragments; values are transposed per 32-slot block
// to [64][32] so the attention kernel reads 8-byte runs of consecutive keys.
#include "common.hpp"

namespace zebra {

__device__ inline long long tile_token(const Geom& g, int f, int tl, int s) {
  const int a = tl / g.tc, b = tl - a * g.tc;
  const int tw = g.tw[tl];
  const int r = TILE * a + s / tw, c = TILE * b + s % tw;
  return (long long)f * g.tok_pf + g.S + (long long)r * g.C + c;
}

// grid (T + spec_pad/32, H), block 256.
__global__ void __launch_bounds__(256) pack_kernel(Geom g, const u16* __restrict__ K,
                                                   const u16* __restrict__ V, u16* __restrict__ Kt,
                                                   u16* __restrict__ Vt, u16* __restrict__ Ks,
                                                   u16* __restrict__ Vs) {
  __shared__ u16 vstage[KBLK][D + 8];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int slot_in = tid >> 3;  // 0..31
  const int chunk = tid & 7;     // 8 channels each
  const long long rowstride = (long long)g.H * D;

  long long base_slot;  // first packed slot of this group
  int nslots, nreal, f = 0, tl = 0;
  bool special = blockIdx.x >= (unsigned)g.T;
  u16 *Kdst, *Vdst;
  if (!special) {
    const int u = blockIdx.x;
    f = u / g.tpf;
    tl = u - f * g.tpf;
    nreal = g.th[tl] * g.tw[tl];
    nslots = pad32(nreal);
    base_slot = (long long)f * g.slots_pf + g.slot_off[tl];
    Kdst = Kt + (long long)h * g.slots * D;
    Vdst = Vt + (long long)h * g.slots * D;
  } else {
    const int sb = blockIdx.x - g.T;
    base_slot = (long long)sb * KBLK;
    nslots = KBLK;
    nreal = min(KBLK, g.nspec - sb * KBLK);
    Kdst = Ks + (long long)h * g.spec_pad * D;
    Vdst = Vs + (long long)h * g.spec_pad * D;
  }
  for (int blk = 0; blk < nslots / KBLK; ++blk) {
    const int s = blk * KBLK + slot_in;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (s < nreal) {
      long long tok;
      if (!special) {
        tok = tile_token(g, f, tl, s);
      } else {
        const int i = (int)base_slot + s;  // special index = frame*S + s
        tok = (long long)(i / g.S) * g.tok_pf + (i % g.S);
      }
      kv = *(const uint4*)(K + tok * rowstride + (long long)h * D + chunk * 8);
      vv = *(const uint4*)(V + tok * rowstride + (long long)h * D + chunk * 8);
    }
    *(uint4*)(Kdst + (base_slot + s) * D + chunk * 8) = kv;
    const u16* pv = (const u16*)&vv;
#pragma unroll
    for (int i = 0; i < 8; ++i) vstage[slot_in][chunk * 8 + i] = pv[i];
    __syncthreads();
    // transpose: thread -> (d = tid>>2, 8 keys starting at (tid&3)*8)
    {
      const int d = tid >> 2, k0 = (tid & 3) * 8;
      u16 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = vstage[k0 + i][d];
      const long long vblk = (base_slot / KBLK) + blk;
      *(uint4*)(Vdst + (vblk * D + d) * KBLK + k0) = *(const uint4*)w;
    }
    __syncthreads();
  }
}

// grid (T_pad, H), block 64 (thread = channel).
__global__ void __launch_bounds__(64) landmark_kernel(Geom g, const u16* __restrict__ Kt,
                                                      const u16* __restrict__ Vt,
                                                      double* __restrict__ kbar,
                                                      float* __restrict__ vbar,
                                                      float* __restrict__ logn,
                                                      u16* __restrict__ LM) {
  const int u = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  u16* lmk_hi = LM + (long long)h * 3 * g.T_pad * D;
  u16* lmk_lo = lmk_hi + (long long)g.T_pad * D;
  u16* lmv = lmk_lo + (long long)g.T_pad * D;
  const long long vpos = ((long long)(u / KBLK) * D + d) * KBLK + (u % KBLK);
  if (u >= g.T) {  // padding landmarks: zero key and value
    lmk_hi[(long long)u * D + d] = 0;
    lmk_lo[(long long)u * D + d] = 0;
    lmv[vpos] = 0;
    return;
  }
  const int f = u / g.tpf, tl = u - f * g.tpf;
  const int n = g.th[tl] * g.tw[tl];
  const long long base = (long long)f * g.slots_pf + g.slot_off[tl];
  const u16* kp = Kt + ((long long)h * g.slots + base) * D + d;
  const u16* vp = Vt + (long long)h * g.slots * D;
  double sk = 0.0, sv = 0.0;  // exact: sums of <= 64 bf16 values
  for (int s = 0; s < n; ++s) {
    sk += (double)bf2f(kp[(long long)s * D]);
    const long long vb = base / KBLK + s / KBLK;
    sv += (double)bf2f(vp[(vb * D + d) * KBLK + (s % KBLK)]);
  }
  const double mk = sk / n;
  const float mv = (float)(sv / n);
  kbar[((long long)h * g.T + u) * D + d] = mk;
  vbar[((long long)h * g.T + u) * D + d] = mv;
  const float hi = (float)mk;
  const u16 hb = f2bf(hi);
  const u16 lb = f2bf((float)(mk - (double)bf2f(hb)));
  lmk_hi[(long long)u * D + d] = hb;
  lmk_lo[(long long)u * D + d] = lb;
  lmv[vpos] = f2bf(mv);
  if (h == 0 && d == 0) logn[u] = logf((float)n);
}

hipError_t launch_pack(const Geom& g, const u16* K, const u16* V, u16* Kt, u16* Vt, u16* Ks,
                       u16* Vs, hipStream_t s) {
  hipLaunchKernelGGL(pack_kernel, dim3(g.T + g.spec_pad / KBLK, g.H), dim3(256), 0, s, g, K, V,
                     Kt, Vt, Ks, Vs);
  return hipGetLastError();
}

hipError_t launch_landmarks(const Geom& g, const u16* Kt, const u16* Vt, double* kbar,
                            float* vbar, float* logn, u16* LM, hipStream_t s) {
  hipLaunchKernelGGL(landmark_kernel, dim3(g.T_pad, g.H), dim3(64), 0, s, g, Kt, Vt, kbar, vbar,
                     logn, LM);
  return hipGetLastError();
}

}  // namespace zebra
