// The attention steps either side of a global stage, for gfx950.
//
// Zebra3D pages, "Global attention dominates runtime as views grow": the
// backbones alternate frame-wise attention with global attention.
// "Linear-centered stages plus tile-sparse stages": conversion keeps the
// normalisation layers and positional encoding, so the queries and keys of
// a sparse stage pass through per-head RMSNorm and 2D rotary first.
//
//   qk_prologue_kernel  x -> RoPE2D(RMSNorm(x)) for the rows of Q and K,
//                       bf16 out (one thread per (token, head) row; HBM-bound)
//   frame_attn_kernel   softmax attention of every token over the tokens
//                       of its own frame (bf16 MFMA, online softmax)
#include "attn_common.hpp"

namespace zebra {

// ---------------------------------------------------------------- prologue
constexpr int PRO_THREADS = 256;

// Position of token n: (patch row, patch column); special tokens (0, 0).
__device__ inline void pro_pos(const Geom& g, long long n, int& pr, int& pc) {
  const long long f = n / g.tok_pf;
  const int loc = (int)(n - f * g.tok_pf);
  if (loc < g.S) {
    pr = pc = 0;
    return;
  }
  const int p = loc - g.S;
  pr = p / g.C;
  pc = p - pr * g.C;
}

// One (token, head) row per thread: RMSNorm over the 64 channels (fp32,
// eps, gain), then the pair (j, j+16) of each 32-channel half turned by
// p * base^(-j/16), p the patch row (first half) or column (second half),
// read from an LDS table of {cos, sin}. Rows are read whole before they are
// written, so out may alias in.
__global__ void __launch_bounds__(PRO_THREADS) qk_prologue_kernel(Geom g, const u16* __restrict__ X,
                                                                  const float* __restrict__ gain, float eps,
                                                                  float base, u16* __restrict__ Y) {
  extern __shared__ float2 ptab[];  // [max(R, C)][16]
  const int npos = g.R > g.C ? g.R : g.C;
  for (int i = threadIdx.x; i < npos * 16; i += blockDim.x) {
    const int p = i >> 4, j = i & 15;
    const double ang = (double)p * pow((double)base, -(double)j / 16.0);
    double s, c;
    sincos(ang, &s, &c);
    ptab[i] = make_float2((float)c, (float)s);
  }
  __syncthreads();
  const long long row = (long long)blockIdx.x * PRO_THREADS + threadIdx.x;
  if (row >= g.N * g.H) return;
  const long long n = row / g.H;
  const int h = (int)(row - n * g.H);
  const long long off = n * g.in_tok + (long long)h * g.in_head;
  float x[D];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 w = *(const uint4*)(X + off + c * 8);
    const u16* e = (const u16*)&w;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[c * 8 + i] = bf2f(e[i]);
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) ss = fmaf(x[c], x[c], ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
  for (int c = 0; c < D; ++c) x[c] *= r * (gain ? gain[h * D + c] : 1.0f);
  int pr, pc;
  pro_pos(g, n, pr, pc);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const float2* t = ptab + (half == 0 ? pr : pc) * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float a = x[half * 32 + j], b = x[half * 32 + 16 + j];
      const float2 cs = t[j];
      x[half * 32 + j] = a * cs.x - b * cs.y;
      x[half * 32 + 16 + j] = b * cs.x + a * cs.y;
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint4 w;
    u16* e = (u16*)&w;
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = f2bf(x[c * 8 + i]);
    *(uint4*)(Y + off + c * 8) = w;
  }
}

hipError_t launch_qk_prologue(const Geom& g, const u16* X, const float* gain, float eps, float base, u16* Y,
                              hipStream_t s) {
  const long long rows = g.N * g.H;
  const size_t tab = (size_t)(g.R > g.C ? g.R : g.C) * 16 * sizeof(float2);
  hipLaunchKernelGGL(qk_prologue_kernel, dim3((unsigned)((rows + PRO_THREADS - 1) / PRO_THREADS)),
                     dim3(PRO_THREADS), tab, s, g, X, gain, eps, base, Y);
  return hipGetLastError();
}

// ---------------------------------------------------------------- frame attention
constexpr int FR_WAVES = 4;
constexpr int FR_ROWS = FR_WAVES * 64;  // query rows per workgroup

// One online-softmax step of a 16-row slot over a 32-key block: S^T = K Q^T
// (bias: -inf on masked keys), running row max m (log2 units), O and the
// lane's part of the row sum rescaled when m grows, then O^T += V^T P^T.
__device__ __forceinline__ void frame_step(const bf16x8 kf[2][2], const bf16x8 vf[4], const bf16x8 q[2],
                                           const f32x4& b0, const f32x4& b1, float& m, float& l, f32x4 o[4]) {
  f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][0], q[0], b0, 0, 0, 0);
  f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][0], q[0], b1, 0, 0, 0);
  a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][1], q[1], a0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][1], q[1], a1, 0, 0, 0);
  float bm = __builtin_fmaxf(__builtin_fmaxf(a0[0], a0[1]), __builtin_fmaxf(a0[2], a0[3]));
  bm = __builtin_fmaxf(bm, __builtin_fmaxf(__builtin_fmaxf(a1[0], a1[1]), __builtin_fmaxf(a1[2], a1[3])));
  bm = xmax32(xmax16(bm)) * QK_LOG2;  // the block's row maximum, every lane group of the row
  const float mn = __builtin_fmaxf(m, bm);
  const float sc = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first block (m = -inf)
  m = mn;
  l *= sc;
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] *= sc;
  float p[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = __builtin_amdgcn_exp2f(fmaf(a0[r], QK_LOG2, -mn));
    p[4 + r] = __builtin_amdgcn_exp2f(fmaf(a1[r], QK_LOG2, -mn));
  }
  l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  const bf16x8 P = __builtin_bit_cast(
      bf16x8, make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])));
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], P, o[db], 0, 0, 0);
}

// grid (ceil(tok_pf / FR_ROWS), F, H), block FR_WAVES waves. Each wave holds
// 64 query rows of one frame and head (four 16-row slots) and walks the
// frame's keys: its tiles' packed 32-slot blocks (fragments read straight
// from Kt, and from Vt, already in the P.V operand order), then its special
// keys, gathered from K and V.
__global__ void __launch_bounds__(FR_WAVES * 64) frame_attn_kernel(Geom g, const u16* __restrict__ Q,
                                                                   const u16* __restrict__ K,
                                                                   const u16* __restrict__ V,
                                                                   const u16* __restrict__ Kt,
                                                                   const u16* __restrict__ Vt, u16* __restrict__ O) {
  const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
  const int lg = lane >> 4, tl = lane & 15;
  const int f = blockIdx.y, h = blockIdx.z;
  const int r0 = blockIdx.x * FR_ROWS + wave * 64;  // first query row (within the frame)
  const long long tok0 = (long long)f * g.tok_pf;
  bf16x8 q[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r = r0 + s * 16 + tl;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (r < g.tok_pf) w = *(const uint4*)(Q + (tok0 + r) * g.in_tok + (long long)h * g.in_head + ds * 32 + 8 * lg);
      q[s][ds] = __builtin_bit_cast(bf16x8, w);
    }
  }
  float m[4], l[4];
  f32x4 o[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    m[s] = -INFINITY;
    l[s] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[s][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u16* Kh = Kt + (long long)h * g.slots * D;
  const u16* Vh = Vt + (long long)h * g.slots * D;
  const bool live = r0 < g.tok_pf;  // uniform: the wave has rows
  // the frame's tiles
  for (int t = 0; t < g.tpf && live; ++t) {
    const int n = tile_n(g, t);
    const long long slot0 = (long long)f * g.slots_pf + tile_off(g, t);
    for (int kb = 0; kb * KBLK < n; ++kb) {
      const long long s0 = slot0 + kb * KBLK;
      bf16x8 kf[2][2], vf[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int ds = 0; ds < 2; ++ds)
          kf[h2][ds] = *(const bf16x8*)(Kh + (s0 + h2 * 16 + tl) * D + (ds * 4 + lg) * 8);
#pragma unroll
      for (int db = 0; db < 4; ++db) vf[db] = *(const bf16x8*)(Vh + (s0 / KBLK * D + db * 16 + tl) * KBLK + lg * 8);
      const int nv = min(KBLK, n - kb * KBLK);
      f32x4 b0, b1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        b0[r] = 4 * lg + r < nv ? 0.f : -INFINITY;
        b1[r] = 16 + 4 * lg + r < nv ? 0.f : -INFINITY;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) frame_step(kf, vf, q[s], b0, b1, m[s], l[s], o[s]);
    }
  }
  // the frame's special keys (at most 32 per block), gathered from K and V:
  // key slot k of the block holds special kb*32 + k; the value fragment of
  // lane group lg takes keys value_key(8 lg + i)
  for (int kb = 0; kb * KBLK < g.S && live; ++kb) {
    const int nv = min(KBLK, g.S - kb * KBLK);
    bf16x8 kf[2][2], vf[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int key = kb * KBLK + h2 * 16 + tl;
      const long long row = (tok0 + (key < g.S ? key : 0)) * g.in_tok + (long long)h * g.in_head;
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) kf[h2][ds] = *(const bf16x8*)(K + row + (ds * 4 + lg) * 8);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      u16 e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = kb * KBLK + value_key(8 * lg + i);
        e[i] = key < g.S ? V[(tok0 + key) * g.in_tok + (long long)h * g.in_head + db * 16 + tl] : (u16)0;
      }
      vf[db] = __builtin_bit_cast(bf16x8, make_uint4(e[0] | (unsigned)e[1] << 16, e[2] | (unsigned)e[3] << 16,
                                                      e[4] | (unsigned)e[5] << 16, e[6] | (unsigned)e[7] << 16));
    }
    f32x4 b0, b1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      b0[r] = 4 * lg + r < nv ? 0.f : -INFINITY;
      b1[r] = 16 + 4 * lg + r < nv ? 0.f : -INFINITY;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) frame_step(kf, vf, q[s], b0, b1, m[s], l[s], o[s]);
  }
  // O = O^T / l, rows r0 + s*16 + lane%16, channels db*16 + 4 lg + r
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float inv = 1.0f / xsum32(xsum16(l[s]));
    const int r = r0 + s * 16 + tl;
    if (r < g.tok_pf) {
      u16* orow = O + (tok0 + r) * g.out_tok + (long long)h * g.out_head;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        uint2 wv;
        wv.x = pack_bf16(o[s][db][0] * inv, o[s][db][1] * inv);
        wv.y = pack_bf16(o[s][db][2] * inv, o[s][db][3] * inv);
        *(uint2*)(orow + db * 16 + 4 * lg) = wv;
      }
    }
  }
}

hipError_t launch_frame_attn(const Geom& g, const u16* Q, const u16* K, const u16* V, const u16* Kt, const u16* Vt,
                             u16* O, hipStream_t s) {
  hipLaunchKernelGGL(frame_attn_kernel, dim3((g.tok_pf + FR_ROWS - 1) / FR_ROWS, g.F, g.H), dim3(FR_WAVES * 64), 0,
                     s, g, Q, K, V, Kt, Vt, O);
  return hipGetLastError();
}

}  // namespace zebra
