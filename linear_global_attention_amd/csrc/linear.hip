// Linear global attention for gfx950: fused RMSNorm, 2D rotary and
// channel-softmax feature map, a per-head KV state on MFMA, and the centred
// affine output correction folded into that state.
//
// Zebra3D pages, "Speedup scales with the number of input views": the linear
// stages fuse Q/K normalisation, positional rotation and a channel-softmax
// feature map. "A closed-form fit avoids retraining from scratch": a centred
// affine correction y = mu + W (o - mu) + b is applied to the output.
//
// Four kernels:
//   linear_state  stream K and V once through per-wave LDS rings: phi(k)
//                 for 16 tokens per group, written back in place, then
//                 S += phi(K)^T V (bf16 MFMA on transposing LDS reads, fp32
//                 accumulators) and z += phi(k); one partial per workgroup
//                 (its waves added in a fixed order).
//   linear_sum    fixed-order fp64 sum of the partials, one element per
//                 thread over all of a head's partials;
//   linear_fold   S' = S W^T split into bf16 high/low parts and
//                 b' = mu - W mu + b, because W o = phi(q)^T S W^T / den.
//   linear_apply  stream Q once: phi(q), y^T = S'^T phi(q)^T on MFMA,
//                 divide by phi(q).z, add b', store bf16.
//
// Lane layout of the feature map: lane l holds token l%16 of a 16-token
// pass and, with g = l/16, the 16 channels ch(g,i) = (i/4)*16 + 4g + i%4.
// Each rotary pair (j, j+16) therefore sits in one lane; channel sums need
// two cross-lane steps. For the apply MFMA the reduction index a runs over
// these channels in lane order, so S'^T is stored column-permuted to match.
#include "linear_common.hpp"

namespace zebra {

typedef void __attribute__((address_space(3))) lin_lds_void;
constexpr int AP_NB = 6;  // LDS ring slots per wave in linear_apply

// Wait until at most n (even, <= 24) of this wave's vector memory
// operations are pending.
#define LIN_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
__device__ inline void lin_wait_vm(int n) {
  switch (n) {
    case 0: LIN_VMCNT(0); break;
    case 2: LIN_VMCNT(2); break;
    case 4: LIN_VMCNT(4); break;
    case 6: LIN_VMCNT(6); break;
    case 8: LIN_VMCNT(8); break;
    case 10: LIN_VMCNT(10); break;
    case 12: LIN_VMCNT(12); break;
    case 14: LIN_VMCNT(14); break;
    case 16: LIN_VMCNT(16); break;
    case 18: LIN_VMCNT(18); break;
    case 20: LIN_VMCNT(20); break;
    case 22: LIN_VMCNT(22); break;
    case 24: LIN_VMCNT(24); break;
    default: LIN_VMCNT(0); break;
  }
}
static_assert(6 * (AP_NB - 2) <= 24, "lin_wait_vm covers the pending counts of linear_apply");

// grid (nchunks, H), block 256. Partial p = chunk holds
// S [64][64] (row a = phi channel, column c = value channel) then z [64].
//
// Each wave streams its 16-token groups of K and V (group m: tokens
// first + 64 m .. +15, first = t_begin + 16 w) through a private LDS ring of
// ST_NB slots, ST_NB - 1 groups ahead, by async 16-byte copies; no workgroup
// barrier in the loop. A slot holds the group's K rows then its V rows,
// token-major, a 128-byte row as eight 16-byte chunks, chunk c of row r at
// slot c ^ ls_swz(r) (both access patterns below then spread over the
// banks). The K rows are read in the feature-map lane layout (one token per
// 4 lanes), turned into phi(k) (bf16) and written back in place; transposing
// LDS reads then give the MFMA operands, 4 consecutive tokens of one channel
// per lane. Every two groups, S += phi^T V and z += phi^T 1 take 20 bf16
// MFMAs (16x16x32, k = the two groups' 32 tokens; the all-ones operand gives
// z from the same bf16 phi as S). The ring is read and written by inline asm
// that waits on LDS only: as plain accesses the compiler would first wait
// for every copy in flight into the ring. The workgroup adds its waves'
// states in wave order.
constexpr int ST_NB = 4;       // LDS ring slots per wave
constexpr int ST_SLOT = 4096;  // bytes per slot: 16 K rows, then 16 V rows
__device__ inline int ls_swz(int r) { return (r ^ (r >> 2)) & 7; }
typedef short st_v4s __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(LIN_THREADS) linear_state_kernel(
    Geom g, LinParams P, const u16* __restrict__ K, const u16* __restrict__ V,
    const float* __restrict__ gk, float* __restrict__ partials, int nchunks, int tpw) {
  float2* tab = rope_tab;
  __shared__ __attribute__((aligned(1024))) char sring[LIN_WAVES][ST_NB][ST_SLOT];
  static_assert(sizeof(sring) >= LIN_STATE * sizeof(float), "the partial fits the rings");
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, tl = lane & 15;
  build_rope_table(tab, max(g.R, g.C), P.base);
  const PosDiv dv(g);
  float gain[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) gain[i] = gk ? gk[h * D + lane_channel(grp, i)] : 1.0f;
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 zacc[4];  // z[16 ab + 4 grp + r] in zacc[ab][r] (every column alike)
#pragma unroll
  for (int a = 0; a < 4; ++a) zacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint2 ones2 = make_uint2(0x3F803F80u, 0x3F803F80u);
  __syncthreads();  // the rotary table

  const long long t_begin = (long long)chunk * tpw;
  const long long t_end = min((long long)g.N, t_begin + tpw);
  const long long first = t_begin + 16 * __builtin_amdgcn_readfirstlane(wave);
  const int n = first < t_end ? (int)((t_end - first + 16 * LIN_WAVES - 1) / (16 * LIN_WAVES)) : 0;
  char* ring = &sring[wave][0][0];
  // group m into slot m % ST_NB: copy j of each of K and V fills row
  // 8j + lane/8, slot lane % 8 (chunk (lane % 8) ^ ls_swz(row)). Rows past
  // t_end repeat the last token (their phi is zeroed). Every lane issues all
  // four copies, so the wave's memory counter advances by 4 per group.
  // byte offset of this lane's piece of copy j within a group whose first
  // token is at offset zero; a whole group then only adds a uniform base
  long long loff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + (lane >> 3);
    loff[j] = ((long long)r * g.in_tok + (long long)h * g.in_head) * 2 + (((lane & 7) ^ ls_swz(r)) << 4);
  }
  auto stage = [&](int m) {
    const long long r0 = first + 64LL * m;
    char* dst = ring + (m % ST_NB) * ST_SLOT;
    if (r0 + 15 < t_end) {
      const long long base = r0 * g.in_tok * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_global_load_lds((const void*)((const char*)K + base + loff[j]), (lin_lds_void*)(dst + j * 1024),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)((const char*)V + base + loff[j]),
                                         (lin_lds_void*)(dst + 2048 + j * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 8 * j + (lane >> 3);
        const long long tok = min(r0 + r, t_end - 1);
        const long long off = (tok * g.in_tok + h * g.in_head) * 2 + (((lane & 7) ^ ls_swz(r)) << 4);
        __builtin_amdgcn_global_load_lds((const void*)((const char*)K + off), (lin_lds_void*)(dst + j * 1024), 16, 0,
                                         0);
        __builtin_amdgcn_global_load_lds((const void*)((const char*)V + off), (lin_lds_void*)(dst + 2048 + j * 1024),
                                         16, 0, 0);
      }
    }
  };
  for (int m = 0; m < ST_NB - 1 && m < n; ++m) stage(m);
  int loc = token_loc(g, dv, first + tl);  // frame position of this lane's token of the current group
  auto group = [&](int m, uint2 (&A)[4], uint2 (&B)[4]) {
    // group m has landed once at most the newer groups' copies are pending
    lin_wait_vm(4 * min(ST_NB - 2, n - 1 - m));
    asm volatile("" ::: "memory");
    const unsigned sb = (unsigned)(size_t)(ring + (m % ST_NB) * ST_SLOT);
    // this lane's K row pieces: token tl, channels 16q + 4 grp .. +3 =
    // chunk 2q + grp/2, half grp % 2
    unsigned ka[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ka[q] = sb + tl * 128 + (((2 * q + (grp >> 1)) ^ ls_swz(tl)) << 4) + (grp & 1) * 8;
    uint2 w4[4];
    asm volatile(
        "ds_read_b64 %0, %4\n\t"
        "ds_read_b64 %1, %5\n\t"
        "ds_read_b64 %2, %6\n\t"
        "ds_read_b64 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w4[0]), "=&v"(w4[1]), "=&v"(w4[2]), "=&v"(w4[3])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3])
        : "memory");
    const long long tok = first + 64LL * m + tl;
    float x[16];
    unpack16(w4, x);
    // rotary position of the token (rows past t_end: (0, 0), their phi is
    // zeroed); loc then steps to this lane's token of the next group
    int pr = 0, pc = 0;
    loc_pos(g, dv, loc, pr, pc);
    if (tok >= t_end) pr = pc = 0;
    loc = loc_step64(g, loc);
    // the rotary values of pairs 4 grp .. +3 at (pr, pc), by asm for the
    // same reason as the ring (the table is an extern LDS array)
    float2 cr[4], cc[4];
    {
      const unsigned tr0 = (unsigned)(size_t)(tab + pr * 16 + 4 * grp), tc0 = (unsigned)(size_t)(tab + pc * 16 + 4 * grp);
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %4 offset:16\n\t"
          "ds_read_b128 %2, %5\n\t"
          "ds_read_b128 %3, %5 offset:16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(*(float4*)&cr[0]), "=&v"(*(float4*)&cr[2]), "=&v"(*(float4*)&cc[0]), "=&v"(*(float4*)&cc[2])
          : "v"(tr0), "v"(tc0)
          : "memory");
    }
    featurize16_rot<true>(x, gk != nullptr, gain, cr, cc, P.eps);
    if (tok >= t_end) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.f;
    }
    uint2 pw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pw[q].x = pack_bf16x2(x[4 * q], x[4 * q + 1]);  // round to nearest even
      pw[q].y = pack_bf16x2(x[4 * q + 2], x[4 * q + 3]);
    }
    // phi in place of the K rows, then the MFMA operands: lane i of each 16
    // names row 4 grp + i/4, columns 16 b + 4 (i % 4) .. +3 of the phi (A)
    // or V (B) rows, and receives column 16 b + i of rows 4 grp .. +3
    unsigned ta[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = 4 * grp + (tl >> 2), col = 16 * b + 4 * (tl & 3);
      ta[b] = sb + row * 128 + (((col >> 3) ^ ls_swz(row)) << 4) + (col & 4) * 2;
    }
    asm volatile(
        "ds_write_b64 %8, %12\n\t"
        "ds_write_b64 %9, %13\n\t"
        "ds_write_b64 %10, %14\n\t"
        "ds_write_b64 %11, %15\n\t"
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %17\n\t"
        "ds_read_b64_tr_b16 %2, %18\n\t"
        "ds_read_b64_tr_b16 %3, %19\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:2048\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:2048\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:2048\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(A[0]), "=&v"(A[1]), "=&v"(A[2]), "=&v"(A[3]), "=&v"(B[0]), "=&v"(B[1]), "=&v"(B[2]), "=&v"(B[3])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(pw[0]), "v"(pw[1]), "v"(pw[2]), "v"(pw[3]),
          "v"(ta[0]), "v"(ta[1]), "v"(ta[2]), "v"(ta[3])
        : "memory");
    if (m + ST_NB - 1 < n) stage(m + ST_NB - 1);
  };
  const uint4 ones4 = make_uint4(ones2.x, ones2.y, ones2.x, ones2.y);
  for (int m = 0; m < n; m += 2) {
    uint2 A0[4], B0[4], A1[4], B1[4];
    group(m, A0, B0);
    if (m + 1 < n) {
      group(m + 1, A1, B1);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) A1[i] = B1[i] = make_uint2(0u, 0u);
    }
    // S[16 ab + 4 grp + r][16 cb + tl] += sum over the two groups' 32 tokens
    // (k = 8 grp + j: token 4 grp + j of group m for j < 4, of group m + 1 else)
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(A0[ab].x, A0[ab].y, A1[ab].x, A1[ab].y));
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[ab][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8, make_uint4(B0[cb].x, B0[cb].y, B1[cb].x, B1[cb].y)), acc[ab][cb], 0, 0, 0);
      zacc[ab] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, ones4), zacc[ab], 0, 0, 0);
    }
  }
  // the workgroup's partial: the 4 waves' states added in wave order in LDS
  // (over the rings, once every wave has left its loop), then written once
  float* red = (float*)&sring[0][0][0];
  __syncthreads();
  for (int w = 0; w < LIN_WAVES; ++w) {
    if (wave == w) {
      // MFMA 16x16 output: lane holds column tl, rows 4*grp + 0..3
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* e = &red[(ab * 16 + 4 * grp + r) * D + cb * 16 + tl];
            *e = w == 0 ? acc[ab][cb][r] : *e + acc[ab][cb][r];
          }
      if (tl == 0) {
#pragma unroll
        for (int ab = 0; ab < 4; ++ab)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* e = &red[D * D + ab * 16 + 4 * grp + r];
            *e = w == 0 ? zacc[ab][r] : *e + zacc[ab][r];
          }
      }
    }
    __syncthreads();
  }
  float* out = partials + ((long long)h * nchunks + chunk) * LIN_STATE;
  for (int e = threadIdx.x; e < LIN_STATE; e += LIN_THREADS) out[e] = red[e];
}

// grid (ceil(LIN_STATE / 256), H, LIN_SUM_PARTS), block 256: fixed-order
// fp64 sums of the per-workgroup partial states of a head, one element per
// thread, each z-slice over its own contiguous quarter of the partials (the
// fold adds the quarters in order). Four chains of loads per element instead
// of one long one.
__global__ void __launch_bounds__(256) linear_sum_kernel(const float* __restrict__ partials, int nparts,
                                                         double* __restrict__ state) {
  const int h = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x, part = blockIdx.z;
  if (e >= LIN_STATE) return;
  const int p0 = (int)((long long)nparts * part / LIN_SUM_PARTS);
  const int p1 = (int)((long long)nparts * (part + 1) / LIN_SUM_PARTS);
  const float* base = partials + (long long)h * nparts * LIN_STATE + e;
  double s = 0.0;
  for (int p = p0; p < p1; ++p) s += (double)base[(long long)p * LIN_STATE];
  state[((long long)h * LIN_SUM_PARTS + part) * LIN_STATE + e] = s;
}

// grid (H), block 256. Folds the affine correction into the state: writes
// per head Sp_hi, Sp_lo bf16 [64][64] holding (S W^T)^T with columns in
// lane-channel order, z fp32 [64] and b' = mu - W mu + b fp32 [64].
__global__ void __launch_bounds__(256) linear_fold_kernel(const double* __restrict__ state,
                                                          const float* __restrict__ W, const float* __restrict__ b,
                                                          const float* __restrict__ mu, u16* __restrict__ sp,
                                                          float* __restrict__ zb) {
  __shared__ double S[D][D + 1];
  __shared__ double zs[D];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* st = state + (long long)h * LIN_SUM_PARTS * LIN_STATE;
  for (int e = tid; e < LIN_STATE; e += 256) {
    double v = 0.0;
#pragma unroll
    for (int q = 0; q < LIN_SUM_PARTS; ++q) v += st[(long long)q * LIN_STATE + e];
    if (e < D * D)
      S[e / D][e % D] = v;
    else
      zs[e - D * D] = v;
  }
  __syncthreads();
  const float* Wh = W ? W + (long long)h * D * D : nullptr;
  u16* hi = sp + (long long)h * 2 * D * D;
  u16* lo = hi + D * D;
  // Sp^T[e][p] = sum_c S[ch(p)][c] W[e][c], p = ks*32 + 8g + m -> channel
  for (int idx = tid; idx < D * D; idx += 256) {
    const int e = idx / D, p = idx % D;
    const int ks = p >> 5, gg = (p & 31) >> 3, m = p & 7;
    const int a = lane_channel(gg, ks * 8 + m);
    double v;
    if (Wh) {
      v = 0.0;
      for (int c = 0; c < D; ++c) v += S[a][c] * (double)Wh[e * D + c];
    } else {
      v = S[a][e];
    }
    const u16 hb = f2bf((float)v);
    hi[idx] = hb;
    lo[idx] = f2bf((float)(v - (double)bf2f(hb)));
  }
  float* zo = zb + (long long)h * 2 * D;
  if (tid < D) {
    zo[tid] = (float)zs[tid];
    // b' = mu - W mu + b
    double wm = 0.0, m_e = mu ? (double)mu[h * D + tid] : 0.0;
    if (mu) {
      for (int c = 0; c < D; ++c)
        wm += (Wh ? (double)Wh[tid * D + c] : (c == tid ? 1.0 : 0.0)) * (double)mu[h * D + c];
    }
    zo[D + tid] = (float)(m_e - wm + (b ? (double)b[h * D + tid] : 0.0));
  }
}

// grid (nchunks, H), block 256. Each wave streams its 16-token groups of Q
// through a private LDS ring of AP_NB slots (async global->LDS loads, no
// workgroup barrier), AP_NB - 1 groups ahead.
__global__ void __launch_bounds__(LIN_THREADS, 2) linear_apply_kernel(
    Geom g, LinParams P, const u16* __restrict__ Q, const float* __restrict__ gq,
    const u16* __restrict__ sp, const float* __restrict__ zb, u16* __restrict__ out, int tpw) {
  __shared__ float2 tab[MAX_GRID * 16];
  __shared__ __attribute__((aligned(1024))) char qring[LIN_WAVES][AP_NB][2048];
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, tl = lane & 15;
  build_rope_table(tab, max(g.R, g.C), P.base);
  const PosDiv dv(g);
  float gain[16], zl[16], bp[16];
  const float* zo = zb + (long long)h * 2 * D;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ch = lane_channel(grp, i);
    gain[i] = gq ? gq[h * D + ch] : 1.0f;
    zl[i] = zo[ch];
  }
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int r = 0; r < 4; ++r) bp[eb * 4 + r] = zo[D + eb * 16 + 4 * grp + r];
  // A operands: Sp^T rows e = eb*16 + tl, k slots ks*32 + 8*grp + 0..7
  bf16x8 Ahi[4][2], Alo[4][2];
  const u16* hi = sp + (long long)h * 2 * D * D;
  const u16* lo = hi + D * D;
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int off = (eb * 16 + tl) * D + ks * 32 + 8 * grp;
      Ahi[eb][ks] = *(const bf16x8*)(hi + off);
      Alo[eb][ks] = *(const bf16x8*)(lo + off);
    }
  __syncthreads();
  const long long t_begin = (long long)chunk * tpw;
  const long long t_end = min((long long)g.N, t_begin + tpw);
    // This wave's 16-token groups: m = 0..n-1, first token t_begin + 16 (wave + 4m).
  const long long first = t_begin + 16 * __builtin_amdgcn_readfirstlane(wave);
  const int n = first < t_end ? (int)((t_end - first + 16 * LIN_WAVES - 1) / (16 * LIN_WAVES)) : 0;
  char* ring = &qring[wave][0][0];
  // Stage group m's 16 Q rows (2 KB) into ring slot m % AP_NB: two async
  // 1 KB loads, lane l -> row 8j + l/8, 16-byte column (l%8) ^ (row%8)
  // (swizzled so the row-per-lane reads below are spread over the banks).
  // Rows past t_end repeat the last token, whose output they then rewrite
  // with the same value: every lane issues every load and store, so the
  // wave's memory counter advances by exactly 2 per group staged and 2 per
  // group stored.
  // byte offsets of this lane's copy pieces and output pieces within a
  // group whose first token is at offset zero (rows 8j + l/8, 16-byte
  // column l%8, swizzled for the loads)
  long long qoff[2], ooff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + (lane >> 3);
    qoff[j] = ((long long)r * g.in_tok + (long long)h * g.in_head) * 2 + (((lane & 7) ^ (r & 7)) << 4);
    ooff[j] = ((long long)r * g.out_tok + (long long)h * g.out_head) * 2 + (lane & 7) * 16;
  }
  auto stage = [&](int m) {
    const long long r0 = first + 64LL * m;
    char* dst = ring + (m % AP_NB) * 2048;
    if (r0 + 15 < t_end) {
      const char* base = (const char*)Q + r0 * g.in_tok * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(base + qoff[j]), (lin_lds_void*)(dst + j * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 8 * j + (lane >> 3);
        const long long tok = min(r0 + r, t_end - 1);
        const int c = (lane & 7) ^ (r & 7);
        const char* src = (const char*)(Q + tok * g.in_tok + h * g.in_head) + c * 16;
        __builtin_amdgcn_global_load_lds((const void*)src, (lin_lds_void*)(dst + j * 1024), 16, 0, 0);
      }
    }
  };
  int loc = token_loc(g, dv, first + tl);  // frame position of this lane's token of group m
  for (int m = 0; m < AP_NB - 1 && m < n; ++m) stage(m);
  for (int m = 0; m < n; ++m) {
    // group m has landed once at most `later` newer memory operations of
    // this wave are pending: the newer stages (2 each) and stores (2 each)
    const int later = 2 * min(AP_NB - 2, n - 1 - m) + 2 * min(m, AP_NB - 2);
    lin_wait_vm(later);
    asm volatile("" ::: "memory");
    const char* src = ring + (m % AP_NB) * 2048 + tl * 128;
    uint2 qr[4];
    {
      // one asm block that also waits for its reads: as plain loads the
      // compiler would first wait for every copy in flight into the ring
      unsigned qa[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = (2 * q + (grp >> 1)) ^ (tl & 7);
        qa[q] = (unsigned)(size_t)(src + cc * 16 + (grp & 1) * 8);
      }
      asm volatile(
          "ds_read_b64 %0, %4\n\t"
          "ds_read_b64 %1, %5\n\t"
          "ds_read_b64 %2, %6\n\t"
          "ds_read_b64 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(qr[0]), "=&v"(qr[1]), "=&v"(qr[2]), "=&v"(qr[3])
          : "v"(qa[0]), "v"(qa[1]), "v"(qa[2]), "v"(qa[3])
          : "memory");
    }
    const long long r0 = first + 64LL * m;
    const bool whole = r0 + 15 < t_end;  // no row of the group past t_end
    float x[16];
    unpack16(qr, x);
    int pr = 0, pc = 0;
    // rows past t_end repeat the last token, so they take its position
    if (whole) loc_pos(g, dv, loc, pr, pc);
    else token_pos(g, dv, min(r0 + tl, t_end - 1), pr, pc);
    loc = loc_step64(g, loc);
    // phi(q) enters o = phi(q)^T S' / phi(q)^T z only as a ratio
    featurize16<false>(x, gq != nullptr, gain, tab, pr, pc, grp, P.eps);
    unsigned pw[8];
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      pw[i >> 1] = pack_bf16x2(x[i], x[i + 1]);
      den = fmaf(__uint_as_float(pw[i >> 1] << 16), zl[i], den);
      den = fmaf(__uint_as_float(pw[i >> 1] & 0xFFFF0000u), zl[i + 1], den);
    }
    bf16x8 Bk[2];
    Bk[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    Bk[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
    den = lin_pair32(lin_pair16(den, false), false);
    const float inv = __builtin_amdgcn_rcpf(den);
    f32x4 y[4];
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi[eb][ks], Bk[ks], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo[eb][ks], Bk[ks], a, 0, 0, 0);
      }
      y[eb] = a;
    }
    // Output token tl of the group (MFMA column), channels eb*16 + 4*grp + r.
    // The 16 x 128-byte output tile goes through this group's ring slot
    // (its queries are already in registers), swizzled as the input, so
    // that each row is stored whole: 8 lanes x 16 bytes per row.
    // Written and read back in one asm block that waits on LDS only: as
    // plain stores the compiler would first wait for every copy in flight
    // into the ring.
    char* slot = ring + (m % AP_NB) * 2048;
    uint2 w[4];
    unsigned wa[4];
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) {
      w[eb].x = pack_bf16x2(fmaf(y[eb][0], inv, bp[eb * 4 + 0]), fmaf(y[eb][1], inv, bp[eb * 4 + 1]));
      w[eb].y = pack_bf16x2(fmaf(y[eb][2], inv, bp[eb * 4 + 2]), fmaf(y[eb][3], inv, bp[eb * 4 + 3]));
      const int c = 2 * eb + (grp >> 1);
      wa[eb] = (unsigned)(size_t)(slot + tl * 128 + ((c ^ (tl & 7)) << 4) + (grp & 1) * 8);
    }
    // row r = 8j + lane/8 of the tile, 16-byte column lane % 8, for j = 0, 1
    const int rr = lane >> 3, rc = lane & 7;
    const unsigned ra0 = (unsigned)(size_t)(slot + rr * 128 + ((rc ^ (rr & 7)) << 4));
    const unsigned ra1 = (unsigned)(size_t)(slot + (rr + 8) * 128 + ((rc ^ ((rr + 8) & 7)) << 4));
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    u4 t0, t1;
    asm volatile(
        "ds_write_b64 %2, %6\n\t"
        "ds_write_b64 %3, %7\n\t"
        "ds_write_b64 %4, %8\n\t"
        "ds_write_b64 %5, %9\n\t"
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b128 %1, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t0), "=&v"(t1)
        : "v"(wa[0]), "v"(wa[1]), "v"(wa[2]), "v"(wa[3]), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(ra0),
          "v"(ra1)
        : "memory");
    if (whole) {
      char* ob = (char*)out + r0 * g.out_tok * 2;
      *(uint4*)(ob + ooff[0]) = make_uint4(t0[0], t0[1], t0[2], t0[3]);
      *(uint4*)(ob + ooff[1]) = make_uint4(t1[0], t1[1], t1[2], t1[3]);
    } else {
      const long long otok0 = min(r0 + rr, t_end - 1), otok1 = min(r0 + rr + 8, t_end - 1);
      *(uint4*)(out + otok0 * g.out_tok + h * g.out_head + rc * 8) = make_uint4(t0[0], t0[1], t0[2], t0[3]);
      *(uint4*)(out + otok1 * g.out_tok + h * g.out_head + rc * 8) = make_uint4(t1[0], t1[1], t1[2], t1[3]);
    }
    if (m + AP_NB - 1 < n) stage(m + AP_NB - 1);
  }
}

// Statistics of the closed-form centred affine fit (Zebra3D pages, "A
// closed-form fit avoids retraining from scratch": teacher outputs t and
// linear outputs o accumulated over tokens and heads for a regularised
// least-squares solve in fp64). grid (nchunks, H), block 256; partial p =
// chunk of head h holds, in fp32: sum o [64], sum t [64], sum o o^T [64][64],
// sum o t^T [64][64] over its tokens. The same per-wave rings as
// linear_state (a slot holds 16 rows of o, then 16 rows of t), the same
// transposing reads and the same 16x16x32 MFMAs over pairs of groups; the
// sums come from MFMAs against an all-ones operand, and of the symmetric
// o o^T only the blocks on and above the diagonal are accumulated.
constexpr int AF_PART = 2 * D + 2 * D * D;  // floats of one partial
// index of block (ab, cb), ab <= cb < 4, in the upper triangle, row by row
#define AF_TRI(ab, cb) ((ab) * 4 - (ab) * ((ab) - 1) / 2 + (cb) - (ab))

__global__ void __launch_bounds__(LIN_THREADS, 2) affine_stats_kernel(Geom g, const u16* __restrict__ O,
                                                                   const u16* __restrict__ Tt,
                                                                   float* __restrict__ partials, int nchunks,
                                                                   int tpw) {
  __shared__ __attribute__((aligned(1024))) char sring[LIN_WAVES][ST_NB][ST_SLOT];
  static_assert(sizeof(sring) >= AF_PART * sizeof(float), "the partial fits the rings");
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, tl = lane & 15;
  // o o^T is symmetric: only its blocks ab <= cb are accumulated, in
  // aoo[AF_TRI(ab, cb)]
  f32x4 aoo[10], aot[4][4], so[4], st[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    so[a] = st[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) aot[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < 10; ++i) aoo[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const long long t_begin = (long long)chunk * tpw;
  const long long t_end = min((long long)g.N, t_begin + tpw);
  const long long first = t_begin + 16 * __builtin_amdgcn_readfirstlane(wave);
  const int n = first < t_end ? (int)((t_end - first + 16 * LIN_WAVES - 1) / (16 * LIN_WAVES)) : 0;
  char* ring = &sring[wave][0][0];
  // group m into slot m % ST_NB (as in linear_state): rows past t_end
  // repeat the last token (every lane issues all four copies, so the wave's
  // memory counter advances by 4 per group); those rows are zeroed in LDS
  // before they are read.
  // byte offsets of this lane's pieces of copy j (o: the output's strides,
  // teacher: q's strides) within a group whose first token is at offset 0
  long long ooff[2], toff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + (lane >> 3);
    const long long sw = ((lane & 7) ^ ls_swz(r)) << 4;
    ooff[j] = ((long long)r * g.out_tok + (long long)h * g.out_head) * 2 + sw;
    toff[j] = ((long long)r * g.in_tok + (long long)h * g.in_head) * 2 + sw;
  }
  auto stage = [&](int m) {
    const long long r0 = first + 64LL * m;
    char* dst = ring + (m % ST_NB) * ST_SLOT;
    if (r0 + 15 < t_end) {
      const char* ob = (const char*)O + r0 * g.out_tok * 2;
      const char* tb = (const char*)Tt + r0 * g.in_tok * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_global_load_lds((const void*)(ob + ooff[j]), (lin_lds_void*)(dst + j * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(tb + toff[j]), (lin_lds_void*)(dst + 2048 + j * 1024), 16, 0,
                                         0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 8 * j + (lane >> 3);
        const long long tok = min(r0 + r, t_end - 1);
        const long long sw = ((lane & 7) ^ ls_swz(r)) << 4;
        const long long offo = (tok * g.out_tok + h * g.out_head) * 2 + sw;
        const long long offt = (tok * g.in_tok + h * g.in_head) * 2 + sw;
        __builtin_amdgcn_global_load_lds((const void*)((const char*)O + offo), (lin_lds_void*)(dst + j * 1024), 16, 0,
                                         0);
        __builtin_amdgcn_global_load_lds((const void*)((const char*)Tt + offt), (lin_lds_void*)(dst + 2048 + j * 1024),
                                         16, 0, 0);
      }
    }
  };
  for (int m = 0; m < ST_NB - 1 && m < n; ++m) stage(m);
  auto group = [&](int m, uint2 (&A)[4], uint2 (&B)[4]) {
    lin_wait_vm(4 * min(ST_NB - 2, n - 1 - m));
    asm volatile("" ::: "memory");
    const unsigned sb = (unsigned)(size_t)(ring + (m % ST_NB) * ST_SLOT);
    // rows of this group past t_end hold a repeated token: zero them (o and
    // t) before the reads; lane (row tl, 16-byte chunk grp * 2 + half) pairs
    const long long valid = t_end - (first + 64LL * m);
    unsigned ta[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = 4 * grp + (tl >> 2), col = 16 * b + 4 * (tl & 3);
      ta[b] = sb + row * 128 + (((col >> 3) ^ ls_swz(row)) << 4) + (col & 4) * 2;
    }
    if (valid >= 16) {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %9\n\t"
          "ds_read_b64_tr_b16 %2, %10\n\t"
          "ds_read_b64_tr_b16 %3, %11\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
          "ds_read_b64_tr_b16 %5, %9 offset:2048\n\t"
          "ds_read_b64_tr_b16 %6, %10 offset:2048\n\t"
          "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(A[0]), "=&v"(A[1]), "=&v"(A[2]), "=&v"(A[3]), "=&v"(B[0]), "=&v"(B[1]), "=&v"(B[2]), "=&v"(B[3])
          : "v"(ta[0]), "v"(ta[1]), "v"(ta[2]), "v"(ta[3])
          : "memory");
    } else {
      // the last, part-filled group: zero the rows past t_end first (lane
      // l clears the 16-byte chunk l % 8 of row l / 8 + 8j of o and of t)
      unsigned za[4];
      uint2 zero = make_uint2(0u, 0u);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 8 * j + (lane >> 3);
        za[2 * j] = sb + r * 128 + ((lane & 7) << 4);
        za[2 * j + 1] = r >= valid ? 1u : 0u;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (za[2 * j + 1])
          asm volatile(
              "ds_write_b64 %0, %1\n\t"
              "ds_write_b64 %0, %1 offset:8\n\t"
              "ds_write_b64 %0, %1 offset:2048\n\t"
              "ds_write_b64 %0, %1 offset:2056\n\t"
              "s_waitcnt lgkmcnt(0)"
              :
              : "v"(za[2 * j]), "v"(zero)
              : "memory");
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %9\n\t"
          "ds_read_b64_tr_b16 %2, %10\n\t"
          "ds_read_b64_tr_b16 %3, %11\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
          "ds_read_b64_tr_b16 %5, %9 offset:2048\n\t"
          "ds_read_b64_tr_b16 %6, %10 offset:2048\n\t"
          "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(A[0]), "=&v"(A[1]), "=&v"(A[2]), "=&v"(A[3]), "=&v"(B[0]), "=&v"(B[1]), "=&v"(B[2]), "=&v"(B[3])
          : "v"(ta[0]), "v"(ta[1]), "v"(ta[2]), "v"(ta[3])
          : "memory");
    }
    if (m + ST_NB - 1 < n) stage(m + ST_NB - 1);
  };
  for (int m = 0; m < n; m += 2) {
    uint2 A0[4], B0[4], A1[4], B1[4];
    group(m, A0, B0);
    if (m + 1 < n) {
      group(m + 1, A1, B1);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) A1[i] = B1[i] = make_uint2(0u, 0u);
    }
    // oa[b]: o of channels 16 b + i, tb[b]: t of channels 16 b + i, for the
    // 8 tokens k = 8 grp + j (token 4 grp + j of group m for j < 4, of group
    // m + 1 else)
    bf16x8 oa[4], tb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      oa[b] = __builtin_bit_cast(bf16x8, make_uint4(A0[b].x, A0[b].y, A1[b].x, A1[b].y));
      tb[b] = __builtin_bit_cast(bf16x8, make_uint4(B0[b].x, B0[b].y, B1[b].x, B1[b].y));
    }
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      so[ab] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[ab], ones, so[ab], 0, 0, 0);
      st[ab] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tb[ab], ones, st[ab], 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if (cb >= ab) aoo[AF_TRI(ab, cb)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[ab], oa[cb], aoo[AF_TRI(ab, cb)], 0, 0, 0);
        aot[ab][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[ab], tb[cb], aot[ab][cb], 0, 0, 0);
      }
    }
  }
  // the workgroup's partial: the 4 waves added in wave order in LDS (over
  // the rings, once every wave has left its loop), then written once.
  // MFMA 16x16 output: lane holds column tl, rows 4*grp + 0..3; the sums
  // are in every column (all-ones operand), taken from column 0.
  float* red = (float*)&sring[0][0][0];
  __syncthreads();
  for (int w = 0; w < LIN_WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int a = ab * 16 + 4 * grp + r;
          if (tl == 0) {
            red[a] = w == 0 ? so[ab][r] : red[a] + so[ab][r];
            red[D + a] = w == 0 ? st[ab][r] : red[D + a] + st[ab][r];
          }
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            float* e2 = &red[2 * D + D * D + a * D + cb * 16 + tl];
            *e2 = w == 0 ? aot[ab][cb][r] : *e2 + aot[ab][cb][r];
            if (cb >= ab) {
              // element (a, c) of o o^T and, off the diagonal blocks, (c, a)
              const float v = aoo[AF_TRI(ab, cb)][r];
              const int c = cb * 16 + tl;
              float* e1 = &red[2 * D + a * D + c];
              *e1 = w == 0 ? v : *e1 + v;
              if (cb > ab) {
                float* e1t = &red[2 * D + c * D + a];
                *e1t = w == 0 ? v : *e1t + v;
              }
            }
          }
        }
    }
    __syncthreads();
  }
  float* out = partials + ((long long)h * nchunks + chunk) * AF_PART;
  for (int e = threadIdx.x; e < AF_PART; e += LIN_THREADS) out[e] = red[e];
}

// The partials are added in a fixed order in two levels: level 1, grid
// (ceil(AF_PART / 256), AF_GROUPS), sums partials j, j + AF_GROUPS, ... into
// group j (fp64); level 2, grid (ceil(AF_PART / 256)), adds the groups in
// order into stats[1 + e], and n into stats[0].
constexpr int AF_GROUPS = 64;

__global__ void __launch_bounds__(256) affine_sum1_kernel(const float* __restrict__ partials, int nparts,
                                                          double* __restrict__ groups) {
  const int e = blockIdx.x * 256 + threadIdx.x, j = blockIdx.y;
  if (e >= AF_PART) return;
  double s = 0.0;
  for (int p = j; p < nparts; p += AF_GROUPS) s += (double)partials[(long long)p * AF_PART + e];
  groups[(long long)j * AF_PART + e] = s;
}

__global__ void __launch_bounds__(256) affine_sum2_kernel(const double* __restrict__ groups, double n,
                                                          double* __restrict__ stats) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e == 0) stats[0] += n;
  if (e >= AF_PART) return;
  double s = 0.0;
  for (int j = 0; j < AF_GROUPS; ++j) s += groups[(long long)j * AF_PART + e];
  stats[1 + e] += s;
}

// Tokens per workgroup (a multiple of 128), chosen so that the H x chunks
// workgroups fill whole waves of LIN_RESIDENT: about 8,192 tokens, rounded
// so that no last, part-filled wave of workgroups runs alone.
int linear_tokens_per_wg(const Geom& g) {
  const long long base = 8192;
  const long long wgs = (long long)g.H * ((g.N + base - 1) / base);
  const long long waves = (wgs + LIN_RESIDENT - 1) / LIN_RESIDENT;
  const long long nch = (waves * LIN_RESIDENT + g.H - 1) / g.H;
  const long long tpw = ((g.N + nch - 1) / nch + 127) / 128 * 128;
  return (int)tpw;
}

int linear_chunks(const Geom& g) {
  const long long tpw = linear_tokens_per_wg(g);
  return (int)((g.N + tpw - 1) / tpw);
}

size_t linear_workspace_bytes(const Geom& g) {
  const size_t parts = (size_t)g.H * linear_chunks(g) * LIN_STATE * sizeof(float);
  const size_t state = (size_t)g.H * LIN_SUM_PARTS * LIN_STATE * sizeof(double);
  const size_t red = (size_t)g.H * (2 * D * D * sizeof(u16) + 2 * D * sizeof(float));
  return parts + state + red;
}

void launch_linear_sum(const Geom& g, const float* parts, int nch, double* quarters, hipStream_t s) {
  hipLaunchKernelGGL(linear_sum_kernel, dim3((LIN_STATE + 255) / 256, g.H, LIN_SUM_PARTS), dim3(256), 0, s, parts,
                     nch, quarters);
}

// S = phi(K)^T V and z = sum phi(k) of every head: per-workgroup partials
// [H][linear_chunks][LIN_STATE] fp32, then their fixed-order fp64 sums in
// quarters [H][LIN_SUM_PARTS][LIN_STATE].
void launch_linear_kv_state(const Geom& g, LinParams P, const u16* K, const u16* V, const float* gk, float* parts,
                            double* quarters, hipStream_t s) {
  const int nch = linear_chunks(g), tpw = linear_tokens_per_wg(g);
  hipLaunchKernelGGL(linear_state_kernel, dim3(nch, g.H), dim3(LIN_THREADS), rope_table_bytes(g), s, g, P, K, V, gk,
                     parts, nch, tpw);
  launch_linear_sum(g, parts, nch, quarters, s);
}

// Workspace: partials, the summed quarters fp64 [H][LIN_SUM_PARTS][LIN_STATE], then Sp
// [H][2][64][64] bf16, then zb [H][2][64] fp32.
hipError_t launch_linear(const Geom& g, float eps, float base, const u16* Q, const u16* K,
                         const u16* V, const float* W, const float* b, const float* mu,
                         const float* gq, const float* gk, u16* out, void* ws, hipStream_t s) {
  const int nch = linear_chunks(g), tpw = linear_tokens_per_wg(g);
  float* parts = (float*)ws;
  double* state = (double*)(parts + (size_t)g.H * nch * LIN_STATE);
  u16* sp = (u16*)(state + (size_t)g.H * LIN_SUM_PARTS * LIN_STATE);
  float* zb = (float*)(sp + (size_t)g.H * 2 * D * D);
  LinParams P{eps, base};
  launch_linear_kv_state(g, P, K, V, gk, parts, state, s);
  hipLaunchKernelGGL(linear_fold_kernel, dim3(g.H), dim3(256), 0, s, (const double*)state, W, b, mu, sp, zb);
  hipLaunchKernelGGL(linear_apply_kernel, dim3(nch, g.H), dim3(LIN_THREADS), 0, s, g, P, Q, gq, sp,
                     zb, out, tpw);
  return hipGetLastError();
}

size_t affine_workspace_bytes(const Geom& g) {
  return (size_t)g.H * linear_chunks(g) * AF_PART * sizeof(float) + (size_t)AF_GROUPS * AF_PART * sizeof(double);
}

// Workspace: the partials [H][nchunks][AF_PART] fp32, then the group sums
// [AF_GROUPS][AF_PART] fp64.
hipError_t launch_affine_stats(const Geom& g, const u16* O, const u16* Tt, double* stats, void* ws,
                               hipStream_t s) {
  const int nch = linear_chunks(g), tpw = linear_tokens_per_wg(g);
  float* parts = (float*)ws;
  double* groups = (double*)(parts + (size_t)g.H * nch * AF_PART);
  hipLaunchKernelGGL(affine_stats_kernel, dim3(nch, g.H), dim3(LIN_THREADS), 0, s, g, O, Tt, parts, nch, tpw);
  hipLaunchKernelGGL(affine_sum1_kernel, dim3((AF_PART + 255) / 256, AF_GROUPS), dim3(256), 0, s,
                     (const float*)parts, g.H * nch, groups);
  hipLaunchKernelGGL(affine_sum2_kernel, dim3((AF_PART + 255) / 256), dim3(256), 0, s, (const double*)groups,
                     (double)g.N * g.H, stats);
  return hipGetLastError();
}

}  // namespace zebra
