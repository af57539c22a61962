// Device helpers shared by the linear-attention kernels (forward and
// backward): the per-head RMSNorm, 2D rotary and channel-softmax feature map
// in the lane layout below, bf16 packing and cross-lane pair reductions.
//
// Lane layout of the feature map: lane l holds token l%16 of a 16-token
// pass and, with g = l/16, the 16 channels ch(g,i) = (i/4)*16 + 4g + i%4.
// Each rotary pair (j, j+16) therefore sits in one lane; channel sums need
// two cross-lane steps.
#pragma once

#include "common.hpp"

namespace zebra {

constexpr int LIN_THREADS = 256;
constexpr int LIN_WAVES = LIN_THREADS / 64;
constexpr int LIN_RESIDENT = 512;  // workgroups resident at once: 256 CUs x 2
constexpr float LOG2E = 1.4426950408889634f;
constexpr int LIN_STATE = D * D + D;  // floats of one partial state: S [64][64] then z [64]

struct LinParams {
  float eps;
  float base;
};

__device__ inline int lane_channel(int g, int i) { return (i >> 2) * 16 + 4 * g + (i & 3); }

// Rotary table in dynamic LDS, max(R, C) * 16 entries (rope_table_bytes).
extern __shared__ float2 rope_tab[];
inline size_t rope_table_bytes(const Geom& g) { return (size_t)(g.R > g.C ? g.R : g.C) * 16 * sizeof(float2); }

// cos/sin of p * base^(-j/16) for p < npos, j < 16, in LDS: tab[p][j] = {c, s}
__device__ inline void build_rope_table(float2* tab, int npos, float base) {
  for (int i = threadIdx.x; i < npos * 16; i += blockDim.x) {
    const int p = i >> 4, j = i & 15;
    const double ang = (double)p * pow((double)base, -(double)j / 16.0);
    double s, c;
    sincos(ang, &s, &c);
    tab[i] = make_float2((float)c, (float)s);
  }
}

// Reciprocals for token -> (frame, patch row, patch column) without integer
// division: quotients from a rounded reciprocal, then one exact correction.
struct PosDiv {
  double inv_tpf;  // 1 / tokens per frame
  float inv_c;     // 1 / patch columns
  __device__ explicit PosDiv(const Geom& g) : inv_tpf(1.0 / (double)g.tok_pf), inv_c(1.0f / (float)g.C) {}
};

// Position of token tok within its frame, 0 <= loc < tokens per frame.
__device__ inline int token_loc(const Geom& g, const PosDiv& dv, long long tok) {
  const long long f = (long long)((double)tok * dv.inv_tpf);
  long long loc = tok - f * g.tok_pf;
  if (loc < 0) loc += g.tok_pf;
  else if (loc >= g.tok_pf) loc -= g.tok_pf;
  return (int)loc;
}

// Rotary position (patch row, patch column) of the token at frame position
// loc; specials (0, 0).
__device__ inline void loc_pos(const Geom& g, const PosDiv& dv, int loc, int& pr, int& pc) {
  const int p = max(loc - g.S, 0);  // p < 2^14: exact in fp32
  int r = (int)((float)p * dv.inv_c);
  int c = p - r * g.C;
  if (c < 0) {
    --r;
    c += g.C;
  } else if (c >= g.C) {
    ++r;
    c -= g.C;
  }
  const bool special = loc < g.S;
  pr = special ? 0 : r;
  pc = special ? 0 : c;
}

// Rotary position of token tok.
__device__ inline void token_pos(const Geom& g, const PosDiv& dv, long long tok, int& pr, int& pc) {
  loc_pos(g, dv, token_loc(g, dv, tok), pr, pc);
}

// Frame position of the token 64 further on (a wave's next 16-token group).
__device__ inline int loc_step64(const Geom& g, int loc) {
  loc += 64;
  while (loc >= g.tok_pf) loc -= g.tok_pf;
  return loc;
}

// Sum / max of v over lane pairs (l, l ^ 16) or (l, l ^ 32) on the VALU
// (v_permlane16/32_swap give each lane the pair in the same order, so both
// lanes get the same bits), instead of a cross-lane LDS permute.
__device__ inline float lin_pair16(float v, bool mx) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return mx ? fmaxf(a, b) : a + b;
}
__device__ inline float lin_pair32(float v, bool mx) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return mx ? fmaxf(a, b) : a + b;
}

// Feature map of one token's 16 lane channels (x holds them, fp32, in
// lane order). On return x holds phi(x) for those channels, or, with
// NORMALIZE false, phi(x) times a positive per-token constant (enough where
// phi only enters a ratio). `gained`: multiply by the RMSNorm gains. cr[i]
// and cc[i] are the rotary {cos, sin} of channel pair 4g + i at the token's
// patch row and column.
template <bool NORMALIZE>
__device__ inline void featurize16_rot(float x[16], bool gained, const float gain[16], const float2 cr[4],
                                       const float2 cc[4], float eps) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ss += x[i] * x[i];
  ss = lin_pair32(lin_pair16(ss, false), false);
  const float r = __builtin_amdgcn_rsqf(ss * (1.0f / 64.0f) + eps);
  if (gained) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] *= gain[i];
  }
  // rotary: pairs (i, i+4) for i in 0..3 (row) and 8..11 (column)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x[i], b = x[i + 4];
    x[i] = a * cr[i].x - b * cr[i].y;
    x[i + 4] = b * cr[i].x + a * cr[i].y;
    const float a2 = x[i + 8], b2 = x[i + 12];
    x[i + 8] = a2 * cc[i].x - b2 * cc[i].y;
    x[i + 12] = b2 * cc[i].x + a2 * cc[i].y;
  }
  float m = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fmaxf(m, x[i]);
  m = lin_pair32(lin_pair16(m, true), true);
  const float sc = r * LOG2E, off = -m * sc;
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(fmaf(x[i], sc, off));
  if (NORMALIZE) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i];
    s = lin_pair32(lin_pair16(s, false), false);
    const float inv = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] *= inv;
  }
}

// The same with the rotary values read from the table tab[p][j] = {cos, sin}.
template <bool NORMALIZE>
__device__ inline void featurize16(float x[16], bool gained, const float gain[16], const float2* tab, int pr,
                                   int pc, int g, float eps) {
  float2 cr[4], cc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cr[i] = tab[pr * 16 + 4 * g + i];
    cc[i] = tab[pc * 16 + 4 * g + i];
  }
  featurize16_rot<NORMALIZE>(x, gained, gain, cr, cc, eps);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 (hardware round to nearest even), a in the low half
__device__ inline unsigned pack_bf16x2(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));
}

// The lane's 16 channels of one bf16 row, raw (4 x 8 bytes); zeros past the end.
__device__ inline void fetch16(const u16* row, int g, bool ok, uint2 w[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = ok ? *(const uint2*)(row + q * 16 + 4 * g) : make_uint2(0u, 0u);
}

__device__ inline void unpack16(const uint2 w[4], float x[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[q * 4 + 0] = __uint_as_float(w[q].x << 16);
    x[q * 4 + 1] = __uint_as_float(w[q].x & 0xFFFF0000u);
    x[q * 4 + 2] = __uint_as_float(w[q].y << 16);
    x[q * 4 + 3] = __uint_as_float(w[q].y & 0xFFFF0000u);
  }
}

// Fixed-order fp64 sums of the per-workgroup partial states of each head
// are taken in LIN_SUM_PARTS contiguous quarters (see linear_sum_kernel).
constexpr int LIN_SUM_PARTS = 4;

}  // namespace zebra
