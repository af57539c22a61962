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
// to [64][32] with the keys of a block permuted (value_pos) so the attention
// kernel reads each lane's 8 keys of a channel as one 16-byte run.
#include "common.hpp"

namespace zebra {

__device__ inline long long tile_token(const Geom& g, int f, int tl, int s) {
  const int a = tl / g.tc, b = tl - a * g.tc;
  const int tw = tile_w(g, tl);
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
    nreal = tile_n(g, tl);
    nslots = pad32(nreal);
    base_slot = (long long)f * g.slots_pf + tile_off(g, tl);
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
      for (int i = 0; i < 8; ++i) w[i] = vstage[value_key(k0 + i)][d];
      const long long vblk = (base_slot / KBLK) + blk;
      *(uint4*)(Vdst + (vblk * D + d) * KBLK + k0) = *(const uint4*)w;
    }
    __syncthreads();
  }
}

// grid (T_pad, H), block 64 (thread = channel). Also writes, per tile, a
// key radius r_u >= max_j |k_j - kbar_u| (per-channel max deviations, their
// Euclidean norm, inflated to also cover the bf16 rounding of kbar), which
// the attention kernel uses to bound the logits of the tile's keys.
__global__ void __launch_bounds__(64) landmark_kernel(Geom g, const u16* __restrict__ Kt,
                                                      const u16* __restrict__ Vt,
                                                      double* __restrict__ kbar,
                                                      float* __restrict__ vbar,
                                                      float* __restrict__ logn,
                                                      char* __restrict__ LM) {
  const int u = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int lb = u / KBLK, r = u % KBLK;
  char* lmh = LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE;
  char* kblk = lmh + (long long)lb * LM_KEY_BLOCK;
  u16* krow = (u16*)(kblk + r * D * 2);
  float* log2n_row = (float*)(kblk + LM_LOG2N_ROW * D * 2);
  float* rad_row = (float*)(kblk + LM_RADIUS_ROW * D * 2);
  u16* vblk = (u16*)(lmh + (long long)(g.T_pad / KBLK) * LM_KEY_BLOCK + (long long)lb * KBLK * D * 2);
  // rows 32..63 beyond the two table rows are zero
  if (r < KBLK && KBLK + r != LM_LOG2N_ROW && KBLK + r != LM_RADIUS_ROW)
    ((u16*)(kblk + (KBLK + r) * D * 2))[d] = 0;
  if (u >= g.T) {  // padding landmarks: zero key and value, log2 n = -inf
    krow[d] = 0;
    vblk[d * KBLK + value_pos(r)] = 0;
    if (d == 0) {
      log2n_row[r] = -INFINITY;
      rad_row[r] = 0.f;
    }
    return;
  }
  const int f = u / g.tpf, tl = u - f * g.tpf;
  const int n = tile_n(g, tl);
  const long long base = (long long)f * g.slots_pf + tile_off(g, tl);
  const u16* kp = Kt + ((long long)h * g.slots + base) * D + d;
  const u16* vp = Vt + (long long)h * g.slots * D;
  double sk = 0.0, sv = 0.0;  // exact: sums of <= 64 bf16 values
  for (int s = 0; s < n; ++s) {
    sk += (double)bf2f(kp[(long long)s * D]);
    const long long vb = base / KBLK + s / KBLK;
    sv += (double)bf2f(vp[(vb * D + d) * KBLK + value_pos(s % KBLK)]);
  }
  const double mk = sk / n;
  const float mv = (float)(sv / n);
  kbar[((long long)h * g.T + u) * D + d] = mk;
  vbar[((long long)h * g.T + u) * D + d] = mv;
  const u16 kb16 = f2bf((float)mk);
  krow[d] = kb16;
  vblk[d * KBLK + value_pos(r)] = f2bf(mv);
  // radius about the bf16-rounded mean the attention kernel uses
  const double kq = (double)bf2f(kb16);
  double dev = 0.0;
  for (int s = 0; s < n; ++s) dev = fmax(dev, fabs((double)bf2f(kp[(long long)s * D]) - kq));
  __shared__ double red[64];
  red[d] = dev * dev;
  __syncthreads();
  for (int o = 32; o > 0; o >>= 1) {
    if (d < o) red[d] += red[d + o];
    __syncthreads();
  }
  if (d == 0) {
    log2n_row[r] = log2f((float)n);
    rad_row[r] = (float)(sqrt(red[0]) * 1.0001 + 1e-6);
  }
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
                     logn, (char*)LM);
  return hipGetLastError();
}

}  // namespace zebra
