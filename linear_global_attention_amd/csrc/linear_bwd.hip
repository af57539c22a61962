// Backward of the linear global attention stage for gfx950: the gradients
// of the stage inputs q, k and v from the gradient dy of its output.
//
// Zebra3D pages, "A closed-form fit avoids retraining from scratch": after
// the training-free conversion an optional training stage (task
// supervision plus output and relational distillation) fine-tunes the
// converted model, which needs gradients through the linear stages. The
// affine correction (W, b, mu), the RMSNorm gains, eps and the rotary base
// are constants here; b and mu drop out.
//
// Per head, with u = phi(q) (the normalised feature map of a query row),
// z = sum phi(k), S = phi(K)^T V, den = u . z and Sp = S W^T (the state
// with the correction folded in, as in the forward):
//   yhat = Sp^T u / den                      (= W o)
//   s    = dy . yhat
//   du   = (Sp dy - z s) / den               (gradient of phi(q))
//   E    = sum_i (u_i / den_i) dy_i^T ,  dS = E W
//   dz   = - sum_i (u_i / den_i) s_i
//   dphi(k_j) = dS v_j + dz ,  dv_j = dS^T phi(k_j).
// Every output o_i is close to the mean value m, so Sp dy and z s are large
// and nearly equal, and so are dS v_j and dz. With the centred state
// St = (S - z m^T) W^T in place of Sp (m = sum_a S[a][.] / sum_a z[a]) the
// m terms cancel exactly: du = (St dy - z st) / den with st = dy . St^T u /
// den, and the sum dzt = - sum_i (u_i / den_i) st_i equals dz + dS m, so
// dphi(k_j) = dS (v_j - m) + dzt. Both kernels work with those small
// differences directly.
// and the feature map, rotary and RMSNorm are taken back row by row:
//   softmax   dt = u * (du - u . du)
//   rotary    the pair turns back by minus its angle
//   RMSNorm   dx = r (g dt') - x r^3 sum((g dt') x) / 64, r = (mean x^2 + eps)^-1/2
//
// Kernels, in stream order:
//   linear_bwd_state + linear_sum: fp64 S and z (phi(k) split in two bf16
//     parts for the product, unlike the forward's single rounding).
//   linear_bwd_ops (Y = St): m, and A-operand fragments of St^T and St.
//   linear_bwd_query: stream q and dy, write dq; per-workgroup partials of
//     E and dzt (E on MFMA from transposing LDS reads, k = token).
//   linear_sum: fixed-order fp64 sums of those partials.
//   linear_bwd_ops (Y = E W): A-operand fragments of dS^T and dS.
//   linear_bwd_key: stream k and v, write dk and dv.
// Every product with a state matrix runs on MFMA with that matrix split
// into bf16 high and low parts (and phi split the same way where it is the
// other operand), so that it carries about 16 significant bits.
#include "linear_common.hpp"

namespace zebra {

int linear_tokens_per_wg(const Geom& g);
int linear_chunks(const Geom& g);
void launch_linear_sum(const Geom& g, const float* parts, int nch, double* quarters, hipStream_t s);

// One head's operand set: four 64 x 64 bf16 A operands (first hi, first
// lo, second hi, second lo), each as 8 fragments of 64 lanes x 8 values.
constexpr int LB_MAT = D * D;
constexpr int LB_OPS = 4 * LB_MAT;

typedef short lb_v4s __attribute__((ext_vector_type(4)));

// Channel of k-slot p of an A operand (p = 32 ks + 8 g + m): the channel
// that lane group g holds at lane index 8 ks + m, so that a lane's B
// operand is its own 16 feature-map channels in lane order.
__device__ inline int slot_channel(int p) { return lane_channel((p & 31) >> 3, (p >> 5) * 8 + (p & 7)); }

__device__ inline void split_bf16(float v, u16& hi, u16& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

// grid (H), block 256. X, x: the fp64 quarters [H][LIN_SUM_PARTS][LIN_STATE]
// of a 64 x 64 matrix then a 64-vector per head; W [H][64][64] fp32
// (nullptr: the identity).
//   query side (center = 1; X = S, x = z): m = sum_a S[a][.] / sum_a z[a]
//     (the mean value), X <- S - z m^T, Y = X W^T; writes mean[h] = m.
//   key side (center = 0; X = E, x = dz~): Y = X W.
// Writes per head ops[h] = the A operands of v_mfma_f32_16x16x32_bf16
//   first  M[m][p] = Y[ch(p)][m]       second  M[m][p] = Y[m][ch(p)]
// (bf16 high part, then low part, each) in fragment order: fragment
// f = 2 (m / 16) + p / 32, lane l = m % 16 + 16 ((p % 32) / 8), element
// (f * 64 + l) * 8 + p % 8; and vec[h] = x (fp32).
__global__ void __launch_bounds__(256) linear_bwd_ops_kernel(const double* __restrict__ quarters,
                                                             const float* __restrict__ W, int center,
                                                             u16* __restrict__ ops, float* __restrict__ vec,
                                                             float* __restrict__ mean) {
  __shared__ double X[D][D + 1];
  __shared__ double Y[D][D + 1];
  __shared__ double xv[D], mv[D];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double* st = quarters + (long long)h * LIN_SUM_PARTS * LIN_STATE;
  for (int e = tid; e < LIN_STATE; e += 256) {
    double v = 0.0;
#pragma unroll
    for (int q = 0; q < LIN_SUM_PARTS; ++q) v += st[(long long)q * LIN_STATE + e];
    if (e < D * D) {
      X[e / D][e % D] = v;
    } else {
      xv[e - D * D] = v;
      vec[h * D + e - D * D] = (float)v;
    }
  }
  __syncthreads();
  if (center) {
    // the mean value m, then S - z m^T (the m terms cancel exactly in the
    // query gradient; see linear_bwd_query)
    if (tid < D) {
      double cs = 0.0, zs = 0.0;
      for (int a = 0; a < D; ++a) {
        cs += X[a][tid];
        zs += xv[a];
      }
      mv[tid] = cs / zs;
      mean[h * D + tid] = (float)(cs / zs);
    }
    __syncthreads();
    for (int idx = tid; idx < D * D; idx += 256) X[idx / D][idx % D] -= xv[idx / D] * mv[idx % D];
    __syncthreads();
  }
  const float* Wh = W ? W + (long long)h * D * D : nullptr;
  for (int idx = tid; idx < D * D; idx += 256) {
    const int i = idx / D, j = idx % D;
    double v = 0.0;
    if (!Wh) {
      v = X[i][j];
    } else if (center) {
      for (int c = 0; c < D; ++c) v += X[i][c] * (double)Wh[j * D + c];
    } else {
      for (int c = 0; c < D; ++c) v += X[i][c] * (double)Wh[c * D + j];
    }
    Y[i][j] = v;
  }
  __syncthreads();
  u16* o = ops + (long long)h * LB_OPS;
  for (int idx = tid; idx < LB_MAT; idx += 256) {
    const int f = idx >> 9, l = (idx >> 3) & 63, e8 = idx & 7;
    const int m = (f >> 1) * 16 + (l & 15), p = (f & 1) * 32 + 8 * (l >> 4) + e8;
    const int c = slot_channel(p);
    u16 hi, lo;
    split_bf16((float)Y[c][m], hi, lo);
    o[idx] = hi;
    o[LB_MAT + idx] = lo;
    split_bf16((float)Y[m][c], hi, lo);
    o[2 * LB_MAT + idx] = hi;
    o[3 * LB_MAT + idx] = lo;
  }
}

// Rotary table of the backward kernels: tab[p * RT_STRIDE + j] = {cos, sin}
// of p * base^(-j/16). Rows of 18 entries (144 bytes) rather than 16, so
// that the 16 tokens of a group, at 16 different patch columns, read their
// 16-byte pieces from different banks.
constexpr int RT_STRIDE = 18;
__device__ inline void build_rope_table_bwd(float2* tab, int npos, float base) {
  for (int i = threadIdx.x; i < npos * 16; i += blockDim.x) {
    const int p = i >> 4, j = i & 15;
    const double ang = (double)p * pow((double)base, -(double)j / 16.0);
    double sn, cs;
    sincos(ang, &sn, &cs);
    tab[p * RT_STRIDE + j] = make_float2((float)cs, (float)sn);
  }
}

// The shared front of both row kernels: one 16-token group of a head.
// Lane (tl, grp) holds token tl of the group and the 16 feature-map
// channels ch(grp, i). x: the raw row (fp32), u: phi(x) (normalised),
// r: 1 / sqrt(mean(x^2) + eps), cr/cc the rotary {cos, sin} of the lane's
// pairs at the token's patch row and column.
struct RowFwd {
  float x[16], u[16], r;
  float2 cr[4], cc[4];
};

__device__ inline void row_forward(RowFwd& R, const float2* tab, bool gained, const float gain[16], int pr, int pc,
                                   int grp, float eps) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    R.cr[i] = tab[pr * RT_STRIDE + 4 * grp + i];
    R.cc[i] = tab[pc * RT_STRIDE + 4 * grp + i];
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ss += R.x[i] * R.x[i];
  ss = lin_pair32(lin_pair16(ss, false), false);
  R.r = __builtin_amdgcn_rsqf(ss * (1.0f / 64.0f) + eps);
#pragma unroll
  for (int i = 0; i < 16; ++i) R.u[i] = R.x[i];
  featurize16_rot<true>(R.u, gained, gain, R.cr, R.cc, eps);
}

// dphi -> dx: softmax, rotary, gain and RMSNorm backward of one row (dp is
// overwritten with dx).
__device__ inline void row_backward(const RowFwd& R, float dp[16], bool gained, const float gain[16]) {
  float c = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) c += R.u[i] * dp[i];
  c = lin_pair32(lin_pair16(c, false), false);
#pragma unroll
  for (int i = 0; i < 16; ++i) dp[i] = R.u[i] * (dp[i] - c);
  // the forward turned (a, b) into (a c - b s, b c + a s): back by -angle
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = dp[i], b = dp[i + 4];
    dp[i] = a * R.cr[i].x + b * R.cr[i].y;
    dp[i + 4] = b * R.cr[i].x - a * R.cr[i].y;
    const float a2 = dp[i + 8], b2 = dp[i + 12];
    dp[i + 8] = a2 * R.cc[i].x + b2 * R.cc[i].y;
    dp[i + 12] = b2 * R.cc[i].x - a2 * R.cc[i].y;
  }
  if (gained) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] *= gain[i];
  }
  float sx = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sx += dp[i] * R.x[i];
  sx = lin_pair32(lin_pair16(sx, false), false);
  const float k3 = R.r * R.r * R.r * sx * (1.0f / 64.0f);
#pragma unroll
  for (int i = 0; i < 16; ++i) dp[i] = R.r * dp[i] - R.x[i] * k3;
}

// The lane's 16 channels ch(grp, i) of a 64-float LDS vector (i = 4q + j
// at 16q + 4grp + j: four 16-byte reads).
__device__ inline void lds16(const float* v, int grp, float out[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 t = *(const float4*)(v + q * 16 + 4 * grp);
    out[4 * q] = t.x;
    out[4 * q + 1] = t.y;
    out[4 * q + 2] = t.z;
    out[4 * q + 3] = t.w;
  }
}

// 16 fp32 lane values -> bf16 high and low parts as two 8-value B operands.
__device__ inline void split_operand(const float v[16], bf16x8 hi[2], bf16x8 lo[2]) {
  unsigned h[8], l[8];
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    h[i >> 1] = pack_bf16x2(v[i], v[i + 1]);
    l[i >> 1] = pack_bf16x2(v[i] - __uint_as_float(h[i >> 1] << 16), v[i + 1] - __uint_as_float(h[i >> 1] & 0xFFFF0000u));
  }
  hi[0] = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  hi[1] = __builtin_bit_cast(bf16x8, make_uint4(h[4], h[5], h[6], h[7]));
  lo[0] = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
  lo[1] = __builtin_bit_cast(bf16x8, make_uint4(l[4], l[5], l[6], l[7]));
}

// C[m][token] = sum_p M[m][p] B[p][token] over the 64 slots, M from an LDS
// operand set (fragment order), for the four 16-row blocks; with `three`,
// hi.b + lo.b + hi.b_lo, else hi.b + lo.b.
__device__ inline void mat_times(const bf16x8* Mhi, const bf16x8* Mlo, const bf16x8 b[2], const bf16x8* blo,
                                 int lane, f32x4 out[4]) {
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) {
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int f = eb * 2 + ks;
      const bf16x8 mh = Mhi[f * 64 + lane];
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh, b[ks], a, 0, 0, 0);
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Mlo[f * 64 + lane], b[ks], a, 0, 0, 0);
      if (blo) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh, blo[ks], a, 0, 0, 0);
    }
    out[eb] = a;
  }
}

// Swizzle of the 16-byte chunks of row r in a wave's 16-row staging tile.
__device__ inline int lb_swz(int r) { return (r ^ (r >> 2)) & 7; }

// A group's 16 bf16 rows, loaded as whole 16-byte chunks (lane l: chunk
// l % 8 of row l / 8 in c0, of row 8 + l / 8 in c1), into the feature-map
// lane layout through the wave's 2 KB LDS tile xs: w[q] = channels
// 16 q + 4 grp .. +3 of token tl, the pieces unpack16 takes.
__device__ __forceinline__ void lb_relayout(u16* xs, uint4 c0, uint4 c1, int lane, uint2 w[4]) {
  const int grp = lane >> 4, tl = lane & 15;
  __builtin_amdgcn_wave_barrier();  // the tile's previous reads come first
  const int r0 = lane >> 3, r1 = 8 + (lane >> 3);
  *(uint4*)(xs + r0 * D + (((lane & 7) ^ lb_swz(r0)) << 3)) = c0;
  *(uint4*)(xs + r1 * D + (((lane & 7) ^ lb_swz(r1)) << 3)) = c1;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q)  // channels 16 q + 4 grp .. +3: chunk 2 q + grp / 2, half grp % 2
    w[q] = *(const uint2*)(xs + tl * D + (((2 * q + (grp >> 1)) ^ lb_swz(tl)) << 3) + (grp & 1) * 4);
}

// A group's 16 output rows, given in the feature-map lane layout (lane
// (tl, grp): token tl, channels ch(grp, i) in v), stored as bf16 through the
// wave's 2 KB LDS tile xs so that 8 lanes write each 128-byte row whole:
// lane l stores chunk l % 8 of rows l / 8 and 8 + l / 8 (rows of tokens at
// or past t_end, i.e. r >= valid, are not stored).
__device__ __forceinline__ void lb_store_rows(u16* xs, const float v[16], int lane, u16* out0, long long tok_stride,
                                     int valid) {
  const int grp = lane >> 4, tl = lane & 15;
  __builtin_amdgcn_wave_barrier();  // the tile's previous reads come first
#pragma unroll
  for (int q = 0; q < 4; ++q)  // channels 16 q + 4 grp .. +3: chunk 2 q + grp / 2, half grp % 2
    *(uint2*)(xs + tl * D + (((2 * q + (grp >> 1)) ^ lb_swz(tl)) << 3) + (grp & 1) * 4) =
        make_uint2(pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3]));
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + (lane >> 3);
    const uint4 c = *(const uint4*)(xs + r * D + (((lane & 7) ^ lb_swz(r)) << 3));
    if (r < valid) *(uint4*)(out0 + r * tok_stride + (lane & 7) * 8) = c;
  }
}

// The lane's 16 channels of a bf16 row (ch(grp, i), i = 4q + j at
// 16q + 4grp + j) as 4 x 8 bytes.
__device__ inline void store16(u16* row, int grp, const float v[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(uint2*)(row + q * 16 + 4 * grp) =
        make_uint2(pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3]));
}

// Element offset in a 16 x 64 bf16 scratch tile of the 4 channels
// col .. col + 3 (col % 4 == 0) of token row r: the 8-byte chunk col / 4 is
// XORed with 4 (r % 4) + (r / 4) % 4, so that the 16 lanes writing one
// chunk column of 16 rows, and the 16 lanes of a transposing read (4 rows x
// 4 chunks), all reach different banks.
__device__ inline int xs_off(int r, int col) { return r * D + ((((col >> 2) ^ (4 * (r & 3) + ((r >> 2) & 3)))) << 2); }

// X += a b^T over the 16 tokens of a group (k = token): a fp32 (split into
// bf16 high and low parts), b raw bf16, both in the lane layout. Both go
// through the wave's LDS scratch xs (3 tiles of 16 token rows x 64
// channels, swizzled by xs_off) and come back through transposing reads:
// lane i of each 16 names row 4 grp + i / 4, columns 16 b + 4 (i % 4) .. +3,
// and receives column 16 b + i of rows 4 grp .. +3. X[ab][cb] holds rows
// (a channels) 16 ab + 4 grp + r and column (b channel) 16 cb + tl.
__device__ inline void accum_outer(u16* xs, const float a[16], const uint2 b[4], int grp, int tl, f32x4 X[4][4]) {
  bf16x8 th[2], tlo[2];
  split_operand(a, th, tlo);
  const uint4 h0 = __builtin_bit_cast(uint4, th[0]), h1 = __builtin_bit_cast(uint4, th[1]);
  const uint4 l0 = __builtin_bit_cast(uint4, tlo[0]), l1 = __builtin_bit_cast(uint4, tlo[1]);
  const uint2 hq[4] = {make_uint2(h0.x, h0.y), make_uint2(h0.z, h0.w), make_uint2(h1.x, h1.y), make_uint2(h1.z, h1.w)};
  const uint2 lq[4] = {make_uint2(l0.x, l0.y), make_uint2(l0.z, l0.w), make_uint2(l1.x, l1.y), make_uint2(l1.z, l1.w)};
  asm volatile("" ::: "memory");  // the previous group's reads come first
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int off = xs_off(tl, q * 16 + 4 * grp);
    *(uint2*)(xs + off) = hq[q];
    *(uint2*)(xs + 16 * D + off) = lq[q];
    *(uint2*)(xs + 32 * D + off) = b[q];
  }
  asm volatile("" ::: "memory");
  lb_v4s Ah[4], Al[4], B[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int off = xs_off(4 * grp + (tl >> 2), 16 * c + 4 * (tl & 3));
    typedef __attribute__((address_space(3))) lb_v4s lds_v4s;
    Ah[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(xs + off));
    Al[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(xs + 16 * D + off));
    B[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(xs + 32 * D + off));
  }
#pragma unroll
  for (int ab = 0; ab < 4; ++ab)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      X[ab][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Ah[ab], B[cb], X[ab][cb], 0, 0, 0);
      X[ab][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Al[ab], B[cb], X[ab][cb], 0, 0, 0);
    }
}

// The workgroup's partial [X [64][64], x [64]] (LIN_STATE floats): x summed
// over the 16 token lanes of each channel group, the waves added in wave
// order in LDS at red (LIN_STATE floats that no wave reads any more: the
// caller's loop is over), then written to out. Every thread calls it.
__device__ inline void write_partial(const f32x4 X[4][4], float x[16], float* red, int wave, int grp, int tl,
                                     float* __restrict__ out) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = x[i];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    x[i] = v;
  }
  __syncthreads();
  for (int w = 0; w < LIN_WAVES; ++w) {
    if (wave == w) {
      // MFMA 16x16 output: lane holds column tl, rows 4 grp + 0..3
#pragma unroll
      for (int ab = 0; ab < 4; ++ab)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* e = &red[(ab * 16 + 4 * grp + r) * D + cb * 16 + tl];
            *e = w == 0 ? X[ab][cb][r] : *e + X[ab][cb][r];
          }
      if (tl == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float* e = &red[D * D + lane_channel(grp, i)];
          *e = w == 0 ? x[i] : *e + x[i];
        }
      }
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < LIN_STATE; e += LIN_THREADS) out[e] = red[e];
}

// grid (nchunks, H), block 256: S = phi(K)^T V and z = sum phi(k) of the
// workgroup's tokens, as the forward's linear_state but with phi(k) split
// into bf16 high and low parts for the product and z summed from the fp32
// phi(k): the backward works with S - z m^T, a remainder far smaller than S,
// which the forward's single bf16 rounding of phi(k) would swamp. Writes the
// partial [S [64][64], z [64]].
__global__ void __launch_bounds__(LIN_THREADS, 2) linear_bwd_state_kernel(
    Geom g, LinParams P, const u16* __restrict__ K, const u16* __restrict__ V, const float* __restrict__ gk,
    float* __restrict__ partials, int nchunks, int tpw) {
  __shared__ __attribute__((aligned(16))) float2 tab[MAX_GRID * RT_STRIDE];
  __shared__ __attribute__((aligned(16))) u16 sxp[LIN_WAVES][3][16 * D];
  __shared__ __attribute__((aligned(16))) float sgain[D];
  static_assert(sizeof(sxp) >= LIN_STATE * sizeof(float), "the partial fits the scratch");
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, tl = lane & 15;
  build_rope_table_bwd(tab, max(g.R, g.C), P.base);
  if (threadIdx.x < D) sgain[threadIdx.x] = gk ? gk[h * D + threadIdx.x] : 1.0f;
  const PosDiv dv(g);
  float zacc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) zacc[i] = 0.f;
  f32x4 S[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) S[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  u16* xs = &sxp[wave][0][0];
  const long long t_begin = (long long)chunk * tpw;
  const long long t_end = min((long long)g.N, t_begin + tpw);
  const long long first = t_begin + 16 * wave;
  const int n = first < t_end ? (int)((t_end - first + 16 * LIN_WAVES - 1) / (16 * LIN_WAVES)) : 0;
  // the rows of the next group are loaded while this group is processed
  // as whole 16-byte chunks (rows l / 8 and 8 + l / 8, chunk l % 8), put
  // into the lane layout through the first scratch tile
  uint4 nk0, nk1, nv0, nv1;
  auto fetch = [&](int m) __attribute__((always_inline)) {
    const long long t0 = min(first + 64LL * m + (lane >> 3), t_end - 1);
    const long long t1 = min(first + 64LL * m + 8 + (lane >> 3), t_end - 1);
    const long long c = (long long)h * g.in_head + (lane & 7) * 8;
    nk0 = *(const uint4*)(K + t0 * g.in_tok + c);
    nv0 = *(const uint4*)(V + t0 * g.in_tok + c);
    nk1 = *(const uint4*)(K + t1 * g.in_tok + c);
    nv1 = *(const uint4*)(V + t1 * g.in_tok + c);
  };
  if (n > 0) fetch(0);
  int loc = token_loc(g, dv, first + tl);  // frame position of this lane's token of group m
  for (int m = 0; m < n; ++m) {
    const long long tok = first + 64LL * m + tl;
    const bool valid = tok < t_end;
    uint2 wk[4], wv[4];
    lb_relayout(xs, nk0, nk1, lane, wk);
    lb_relayout(xs, nv0, nv1, lane, wv);
    if (m + 1 < n) fetch(m + 1);
    RowFwd R;
    unpack16(wk, R.x);
    int pr = 0, pc = 0;
    loc_pos(g, dv, loc, pr, pc);  // rows past t_end: masked, any position serves
    loc = loc_step64(g, loc);
    float gain[16];
    lds16(sgain, grp, gain);
    row_forward(R, tab, gk != nullptr, gain, pr, pc, grp, P.eps);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      R.u[i] = valid ? R.u[i] : 0.f;
      zacc[i] += R.u[i];
    }
    accum_outer(xs, R.u, wv, grp, tl, S);
  }
  write_partial(S, zacc, (float*)&sxp[0][0][0], wave, grp, tl,
                partials + ((long long)h * nchunks + chunk) * LIN_STATE);
}

// grid (nchunks, H), block 256: the query rows of workgroup `chunk` (tokens
// [chunk tpw, +tpw)), each wave its 16-token groups first + 64 m. ops[h]:
// first = St^T, second = St (linear_bwd_ops, centred); zv [H][64] = z.
// Writes dq (q's strides) and the workgroup's partial [E [64][64], dzt [64]]
// (its waves added in wave order).
__global__ void __launch_bounds__(LIN_THREADS, 2) linear_bwd_query_kernel(
    Geom g, LinParams P, const u16* __restrict__ Q, const u16* __restrict__ dY, const float* __restrict__ gq,
    const u16* __restrict__ ops, const float* __restrict__ zv, u16* __restrict__ dQ, float* __restrict__ partials,
    int nchunks, int tpw) {
  __shared__ __attribute__((aligned(16))) float2 tab[MAX_GRID * RT_STRIDE];
  __shared__ __attribute__((aligned(16))) u16 sops[LB_OPS];
  // per wave: u/den high part, low part and dy of the group, token-major
  __shared__ __attribute__((aligned(16))) u16 sxp[LIN_WAVES][3][16 * D];
  static_assert(sizeof(sops) >= LIN_STATE * sizeof(float), "the partial fits the operand buffer");
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, tl = lane & 15;
  build_rope_table_bwd(tab, max(g.R, g.C), P.base);
  {
    const uint4* src = (const uint4*)(ops + (long long)h * LB_OPS);
    for (int i = threadIdx.x; i < LB_OPS / 8; i += LIN_THREADS) ((uint4*)sops)[i] = src[i];
  }
  __shared__ __attribute__((aligned(16))) float sgain[D], svec[D];
  if (threadIdx.x < D) {
    sgain[threadIdx.x] = gq ? gq[h * D + threadIdx.x] : 1.0f;
    svec[threadIdx.x] = zv[h * D + threadIdx.x];
  }
  const PosDiv dv(g);
  float zacc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) zacc[i] = 0.f;
  f32x4 E[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) E[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const bf16x8* F = (const bf16x8*)sops;
  u16* xs = &sxp[wave][0][0];
  const long long t_begin = (long long)chunk * tpw;
  const long long t_end = min((long long)g.N, t_begin + tpw);
  const long long first = t_begin + 16 * wave;
  const int n = first < t_end ? (int)((t_end - first + 16 * LIN_WAVES - 1) / (16 * LIN_WAVES)) : 0;
  // the rows of the next group are loaded while this group is processed
  auto fetch = [&](int m, uint2 (&a)[4], uint2 (&b)[4]) {
    const long long tk = min(first + 64LL * m + tl, t_end - 1);
    fetch16(Q + tk * g.in_tok + (long long)h * g.in_head, grp, true, a);
    fetch16(dY + tk * g.out_tok + (long long)h * g.out_head, grp, true, b);
  };
  uint2 nq[4], nd[4];
  if (n > 0) fetch(0, nq, nd);
  int loc = token_loc(g, dv, first + tl);  // frame position of this lane's token of group m
  for (int m = 0; m < n; ++m) {
    const long long tok = first + 64LL * m + tl;
    const bool valid = tok < t_end;
    uint2 wq[4], wd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wq[i] = nq[i];
      wd[i] = nd[i];
    }
    if (m + 1 < n) fetch(m + 1, nq, nd);
    RowFwd R;
    unpack16(wq, R.x);
    int pr = 0, pc = 0;
    loc_pos(g, dv, loc, pr, pc);  // rows past t_end: masked, any position serves
    loc = loc_step64(g, loc);
    float gain[16], zl[16];
    lds16(sgain, grp, gain);
    row_forward(R, tab, gq != nullptr, gain, pr, pc, grp, P.eps);
    lds16(svec, grp, zl);
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) den = fmaf(R.u[i], zl[i], den);
    den = lin_pair32(lin_pair16(den, false), false);
    const float inv = 1.0f / den;
    bf16x8 uh[2], ul[2];
    split_operand(R.u, uh, ul);
    // yhat - W m = St^T u / den in the lane layout; st = dy . (yhat - W m)
    f32x4 acc[4];
    mat_times(F, F + 8 * 64, uh, ul, lane, acc);
    float dy[16];
    unpack16(wd, dy);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = fmaf(dy[i], acc[i >> 2][i & 3], s);
    s = lin_pair32(lin_pair16(s, false), false) * inv;
    // St dy (dy is exact in bf16)
    const bf16x8 bd[2] = {__builtin_bit_cast(bf16x8, make_uint4(wd[0].x, wd[0].y, wd[1].x, wd[1].y)),
                          __builtin_bit_cast(bf16x8, make_uint4(wd[2].x, wd[2].y, wd[3].x, wd[3].y))};
    mat_times(F + 16 * 64, F + 24 * 64, bd, nullptr, lane, acc);
    float dp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = (acc[i >> 2][i & 3] - zl[i] * s) * inv;
    // E += (u/den) dy^T and dzt -= (u/den) st over the group's valid tokens
    float ut[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ut[i] = valid ? R.u[i] * inv : 0.f;
      zacc[i] = fmaf(-ut[i], s, zacc[i]);
    }
    lds16(sgain, grp, gain);
    row_backward(R, dp, gq != nullptr, gain);
    if (valid) store16(dQ + tok * g.in_tok + (long long)h * g.in_head, grp, dp);
    accum_outer(xs, ut, wd, grp, tl, E);
  }
  write_partial(E, zacc, (float*)sops, wave, grp, tl,
                partials + ((long long)h * nchunks + chunk) * LIN_STATE);
}
// grid (nchunks, H), block 256: the key rows, as linear_bwd_query. ops[h]:
// first = dS^T, second = dS (linear_bwd_ops with Y = E W); dzv [H][64] =
// dzt, mean [H][64] = m. Writes dk and dv (q's strides).
__global__ void __launch_bounds__(LIN_THREADS, 3) linear_bwd_key_kernel(
    Geom g, LinParams P, const u16* __restrict__ K, const u16* __restrict__ V, const float* __restrict__ gk,
    const u16* __restrict__ ops, const float* __restrict__ dzv, const float* __restrict__ mean,
    u16* __restrict__ dK, u16* __restrict__ dV, int tpw) {
  float2* tab = rope_tab;  // max(R, C) * RT_STRIDE entries (dynamic LDS)
  __shared__ __attribute__((aligned(16))) u16 sops[LB_OPS];
  __shared__ __attribute__((aligned(16))) u16 sxo[LIN_WAVES][16 * D];  // per wave: a group's output rows
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, tl = lane & 15;
  build_rope_table_bwd(tab, max(g.R, g.C), P.base);
  {
    const uint4* src = (const uint4*)(ops + (long long)h * LB_OPS);
    for (int i = threadIdx.x; i < LB_OPS / 8; i += LIN_THREADS) ((uint4*)sops)[i] = src[i];
  }
  __shared__ __attribute__((aligned(16))) float sgain[D], svec[D], smean[D];
  if (threadIdx.x < D) {
    sgain[threadIdx.x] = gk ? gk[h * D + threadIdx.x] : 1.0f;
    svec[threadIdx.x] = dzv[h * D + threadIdx.x];
    smean[threadIdx.x] = mean[h * D + threadIdx.x];
  }
  const PosDiv dv(g);
  __syncthreads();
  const bf16x8* F = (const bf16x8*)sops;
  const long long t_begin = (long long)chunk * tpw;
  const long long t_end = min((long long)g.N, t_begin + tpw);
  const long long first = t_begin + 16 * wave;
  const int n = first < t_end ? (int)((t_end - first + 16 * LIN_WAVES - 1) / (16 * LIN_WAVES)) : 0;
  // the rows of the next group are loaded while this group is processed
  uint4 nk0, nk1, nv0, nv1;
  auto fetch = [&](int m) __attribute__((always_inline)) {
    const long long t0 = min(first + 64LL * m + (lane >> 3), t_end - 1);
    const long long t1 = min(first + 64LL * m + 8 + (lane >> 3), t_end - 1);
    const long long c = (long long)h * g.in_head + (lane & 7) * 8;
    nk0 = *(const uint4*)(K + t0 * g.in_tok + c);
    nv0 = *(const uint4*)(V + t0 * g.in_tok + c);
    nk1 = *(const uint4*)(K + t1 * g.in_tok + c);
    nv1 = *(const uint4*)(V + t1 * g.in_tok + c);
  };
  if (n > 0) fetch(0);
  u16* xo = &sxo[__builtin_amdgcn_readfirstlane(wave)][0];
  int loc = token_loc(g, dv, first + tl);  // frame position of this lane's token of group m
  for (int m = 0; m < n; ++m) {
    // the operand fragments are read from LDS where they are used, not
    // hoisted out of the loop into 128 registers
    asm volatile("" ::: "memory");
    uint2 wk[4], wv[4];
    lb_relayout(xo, nk0, nk1, lane, wk);
    lb_relayout(xo, nv0, nv1, lane, wv);
    if (m + 1 < n) fetch(m + 1);
    RowFwd R;
    unpack16(wk, R.x);
    int pr = 0, pc = 0;
    loc_pos(g, dv, loc, pr, pc);  // rows past t_end: masked, any position serves
    loc = loc_step64(g, loc);
    float gain[16];
    lds16(sgain, grp, gain);
    row_forward(R, tab, gk != nullptr, gain, pr, pc, grp, P.eps);
    bf16x8 uh[2], ul[2];
    split_operand(R.u, uh, ul);
    f32x4 acc[4];
    float o[16];
    // dv = dS^T phi(k)
    mat_times(F, F + 8 * 64, uh, ul, lane, acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = acc[i >> 2][i & 3];
    const int nvalid = (int)min(16LL, t_end - (first + 64LL * m));  // rows of the group before t_end
    const long long orow0 = (first + 64LL * m) * g.in_tok + (long long)h * g.in_head;
    lb_store_rows(xo, o, lane, dV + orow0, g.in_tok, nvalid);
    // dphi(k) = dS (v - m) + dzt
    unpack16(wv, o);
    {
      float mv[16];
      lds16(smean, grp, mv);
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] -= mv[i];
    }
    split_operand(o, uh, ul);
    mat_times(F + 16 * 64, F + 24 * 64, uh, ul, lane, acc);
    lds16(svec, grp, o);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] += acc[i >> 2][i & 3];
    lds16(sgain, grp, gain);
    row_backward(R, o, gk != nullptr, gain);
    lb_store_rows(xo, o, lane, dK + orow0, g.in_tok, nvalid);
  }
}

size_t linear_bwd_workspace_bytes(const Geom& g) {
  const size_t parts = (size_t)g.H * linear_chunks(g) * LIN_STATE * sizeof(float);
  const size_t quarters = (size_t)g.H * LIN_SUM_PARTS * LIN_STATE * sizeof(double);
  const size_t ops = (size_t)2 * g.H * LB_OPS * sizeof(u16);
  const size_t vecs = (size_t)3 * g.H * D * sizeof(float);
  return parts + quarters + ops + vecs;
}

// Workspace: partials [H][nchunks][LIN_STATE] fp32, fp64 quarters
// [H][LIN_SUM_PARTS][LIN_STATE] (first of S and z, then of E and dz), the
// query and key operand sets [2][H][LB_OPS] bf16, then z, dzt and m [3][H][64].
hipError_t launch_linear_bwd(const Geom& g, float eps, float base, const u16* Q, const u16* K, const u16* V,
                             const float* W, const float* gq, const float* gk, const u16* dY, u16* dQ, u16* dK,
                             u16* dV, void* ws, hipStream_t s) {
  const int nch = linear_chunks(g), tpw = linear_tokens_per_wg(g);
  float* parts = (float*)ws;
  double* quarters = (double*)(parts + (size_t)g.H * nch * LIN_STATE);
  u16* opsq = (u16*)(quarters + (size_t)g.H * LIN_SUM_PARTS * LIN_STATE);
  u16* opsk = opsq + (size_t)g.H * LB_OPS;
  float* zq = (float*)(opsk + (size_t)g.H * LB_OPS);
  float* dzk = zq + (size_t)g.H * D;
  float* mean = dzk + (size_t)g.H * D;
  const LinParams P{eps, base};
  hipLaunchKernelGGL(linear_bwd_state_kernel, dim3(nch, g.H), dim3(LIN_THREADS), 0, s, g, P, K, V, gk, parts, nch,
                     tpw);
  launch_linear_sum(g, parts, nch, quarters, s);
  hipLaunchKernelGGL(linear_bwd_ops_kernel, dim3(g.H), dim3(256), 0, s, (const double*)quarters, W, 1, opsq, zq, mean);
  hipLaunchKernelGGL(linear_bwd_query_kernel, dim3(nch, g.H), dim3(LIN_THREADS), 0, s, g, P, Q, dY, gq,
                     (const u16*)opsq, (const float*)zq, dQ, parts, nch, tpw);
  launch_linear_sum(g, parts, nch, quarters, s);
  hipLaunchKernelGGL(linear_bwd_ops_kernel, dim3(g.H), dim3(256), 0, s, (const double*)quarters, W, 0, opsk, dzk, nullptr);
  hipLaunchKernelGGL(linear_bwd_key_kernel, dim3(nch, g.H), dim3(LIN_THREADS),
                     (size_t)max(g.R, g.C) * RT_STRIDE * sizeof(float2), s, g, P, K, V, gk,
                     (const u16*)opsk, (const float*)dzk, (const float*)mean, dK, dV, tpw);
  return hipGetLastError();
}

}  // namespace zebra
