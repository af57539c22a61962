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

// Landmark buffers written by the packing pass.
struct LandmarkOut {
  double* kbar;
  float* vbar;
  float* logn;
  char* LM;
};

__device__ inline char* lm_key_block(const Geom& g, char* LM, int h, int u) {
  return LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE + (long long)(u / KBLK) * LM_KEY_BLOCK;
}

__device__ inline u16* lm_value_block(const Geom& g, char* LM, int h, int u) {
  char* lmh = LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE;
  return (u16*)(lmh + (long long)(g.T_pad / KBLK) * LM_KEY_BLOCK + (long long)(u / KBLK) * KBLK * D * 2);
}

// Rows 32..63 of a key block other than the log2 n row are zero; the tile
// at position r of the block writes row 32 + r.
__device__ inline void lm_zero_row(char* kblk, int r, int d) {
  if (KBLK + r != LM_LOG2N_ROW) ((u16*)(kblk + (KBLK + r) * D * 2))[d] = 0;
}

// grid (T + spec_pad/32 [+ T_pad - T when LMK], H), block 256. With LMK the
// same pass also writes every tile's landmark (as landmark_kernel does from
// the packed buffers) and the padding landmarks past T.
template <bool LMK>
__global__ void __launch_bounds__(256) pack_kernel(Geom g, const u16* __restrict__ K,
                                                   const u16* __restrict__ V, u16* __restrict__ Kt,
                                                   u16* __restrict__ Vt, u16* __restrict__ Ks,
                                                   u16* __restrict__ Vs, LandmarkOut lo) {
  __shared__ u16 vstage[KBLK][D + 8];
  __shared__ u16 kstage[LMK ? KBLK : 1][D + 8];  // the block's keys, for the landmark sums
  __shared__ double red[LMK ? 2 : 1][4][D];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int slot_in = tid >> 3;  // 0..31
  const int chunk = tid & 7;     // 8 channels each
  const int lane = tid & 63, wave = tid >> 6;
  const int spec_blocks = g.spec_pad / KBLK;

  if (LMK && blockIdx.x >= (unsigned)(g.T + spec_blocks)) {  // padding landmark
    const int u = g.T + (blockIdx.x - g.T - spec_blocks), r = u % KBLK;
    if (tid < D) {
      char* kblk = lm_key_block(g, lo.LM, h, u);
      lm_zero_row(kblk, r, tid);
      ((u16*)(kblk + r * D * 2))[tid] = 0;
      lm_value_block(g, lo.LM, h, u)[tid * KBLK + value_pos(r)] = 0;
      if (tid == 0) ((float*)(kblk + LM_LOG2N_ROW * D * 2))[r] = -INFINITY;
    }
    return;
  }

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
  // landmark sums: lane = channel, wave w adds slots 8w..8w+7 of each block.
  // Sums of at most 64 bf16 values are exact in fp64, in any order.
  double sk = 0.0, sv = 0.0;
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
      const long long row = tok * g.in_tok + (long long)h * g.in_head;
      kv = *(const uint4*)(K + row + chunk * 8);
      vv = *(const uint4*)(V + row + chunk * 8);
    }
    *(uint4*)(Kdst + (base_slot + s) * D + chunk * 8) = kv;
    const u16* pv = (const u16*)&vv;
#pragma unroll
    for (int i = 0; i < 8; ++i) vstage[slot_in][chunk * 8 + i] = pv[i];
    if (LMK && !special) {
      const u16* pk = (const u16*)&kv;
#pragma unroll
      for (int i = 0; i < 8; ++i) kstage[slot_in][chunk * 8 + i] = pk[i];
    }
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
    if (LMK && !special) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sk += (double)bf2f(kstage[8 * wave + j][lane]);
        sv += (double)bf2f(vstage[8 * wave + j][lane]);
      }
    }
    __syncthreads();
  }
  if (!LMK || special) return;  // uniform

  const int u = blockIdx.x, r = u % KBLK;
  red[0][wave][lane] = sk;
  red[1][wave][lane] = sv;
  __syncthreads();
  char* kblk = lm_key_block(g, lo.LM, h, u);
  if (tid < D) {
    const int d = tid;
    const double tk = (red[0][0][d] + red[0][1][d]) + (red[0][2][d] + red[0][3][d]);
    const double tv = (red[1][0][d] + red[1][1][d]) + (red[1][2][d] + red[1][3][d]);
    const double mk = tk / nreal;
    const float mv = (float)(tv / nreal);
    lo.kbar[((long long)h * g.T + u) * D + d] = mk;
    lo.vbar[((long long)h * g.T + u) * D + d] = mv;
    const u16 kb16 = f2bf((float)mk);
    ((u16*)(kblk + r * D * 2))[d] = kb16;
    lm_value_block(g, lo.LM, h, u)[d * KBLK + value_pos(r)] = f2bf(mv);
    lm_zero_row(kblk, r, d);
    if (d == 0) {
      ((float*)(kblk + LM_LOG2N_ROW * D * 2))[r] = log2f((float)nreal);
      if (h == 0) lo.logn[u] = logf((float)nreal);
    }
  }
}

// grid (T_pad, H), block 64 (thread = channel).
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
  u16* vblk = (u16*)(lmh + (long long)(g.T_pad / KBLK) * LM_KEY_BLOCK + (long long)lb * KBLK * D * 2);
  lm_zero_row(kblk, r, d);
  if (u >= g.T) {  // padding landmarks: zero key and value, log2 n = -inf
    krow[d] = 0;
    vblk[d * KBLK + value_pos(r)] = 0;
    if (d == 0) log2n_row[r] = -INFINITY;
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
  if (d == 0) log2n_row[r] = log2f((float)n);
  if (h == 0 && d == 0) logn[u] = logf((float)n);
}

hipError_t launch_pack(const Geom& g, const u16* K, const u16* V, u16* Kt, u16* Vt, u16* Ks,
                       u16* Vs, double* kbar, float* vbar, float* logn, u16* LM, hipStream_t s) {
  const LandmarkOut lo{kbar, vbar, logn, (char*)LM};
  const int blocks = g.T + g.spec_pad / KBLK;
  if (kbar)
    hipLaunchKernelGGL(pack_kernel<true>, dim3(blocks + (g.T_pad - g.T), g.H), dim3(256), 0, s, g, K,
                       V, Kt, Vt, Ks, Vs, lo);
  else
    hipLaunchKernelGGL(pack_kernel<false>, dim3(blocks, g.H), dim3(256), 0, s, g, K, V, Kt, Vt, Ks,
                       Vs, lo);
  return hipGetLastError();
}

hipError_t launch_landmarks(const Geom& g, const u16* Kt, const u16* Vt, double* kbar,
                            float* vbar, float* logn, u16* LM, hipStream_t s) {
  hipLaunchKernelGGL(landmark_kernel, dim3(g.T_pad, g.H), dim3(64), 0, s, g, Kt, Vt, kbar, vbar,
                     logn, (char*)LM);
  return hipGetLastError();
}

}  // namespace zebra
