// Backward of the tile-sparse attention stage for gfx950: dq, dk and dv
// from dout, for the stage zebra_sparse_attn computes.
//
// Zebra3D pages, "A closed-form fit avoids retraining from scratch": an
// optional training stage after conversion fine-tunes the converted model,
// which needs gradients through its tile-sparse stages. "Linear-centered
// stages plus tile-sparse stages" defines the forward: a patch row of query
// tile t attends to every token of the tiles t kept, to the mean-key/value
// landmark of every omitted tile (logit q.kbar_u/8 + ln n_u), to every
// special token, and to its own key when t itself is not kept; special rows
// attend to every token. The selection passes no gradient (the kept tiles
// are those of the forward); a landmark hands 1/n_u of its gradient to each
// token of its tile.
//
// With l_ij the logits, P = softmax, dP_ij = dout_i . v_j and
// D_i = sum_j P_ij dP_ij, the logit gradients are dS_ij = P_ij (dP_ij - D_i)
// and dq_i = sum_j dS_ij k_j / 8, dk_j = sum_i dS_ij q_i / 8,
// dv_j = sum_i P_ij dout_i.
//
// Kernels, in stream order (per head; rows and keys addressed through the
// strides of q, k, v and dout):
//   sbwd_lmparts      the landmarks' bf16 high and low parts, once, in the
//                     layout the query-major passes stage them in.
//   sbwd_rows<STATS>  query-major: every row's log2-sum-exp2 of its logits
//                     (log2 units) and D, in one pass over its visible keys
//                     (each lane keeps running partials over its own keys,
//                     merged at the end: P stays exact fp32).
//   sbwd_rows<DQ>     query-major again: dS in fp32, dq += K dS on MFMA
//                     (K^T fragments from transposing LDS reads), plus the
//                     self key; writes dq.
//   sbwd_transpose    the kept-tile bitmap transposed: for every key tile,
//                     the query tiles that keep it (32 x 32 bit blocks by
//                     ballot).
//   sbwd_keys<GLOBAL> key-major over special keys and landmarks, 64 per
//                     workgroup, against every query row (landmarks masked
//                     where the row's tile keeps them), in row chunks:
//                     partial dk, dv per chunk.
//   sbwd_reduce       fixed-order sums of those partials: dk, dv of the
//                     special tokens; the landmark gradients.
//   sbwd_keys<TILE>   key-major over the tokens of each key tile, against
//                     the query tiles that keep it and every special row,
//                     plus the self key and 1/n of the tile's landmark
//                     gradient; writes dk, dv.
// Per 32-key (query-major) or 32-row (key-major) block and wave: 4 MFMAs for
// the logits, 4 for dP, 4 or 8 for the gradient products
// (v_mfma_f32_16x16x32_bf16; P and dS enter as bf16). Landmarks enter at
// full precision (the fp64 mean keys and fp32 mean values, each as bf16
// high and low parts: two MFMAs where a token key takes one).
#include "common.hpp"

namespace zebra {

constexpr int SB_THREADS = 256;                      // 4 waves, 16 rows or keys each
constexpr float SB_C = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
constexpr int SB_CHUNKS = 8;                         // row chunks of the global-key pass

// Rounds of the query-major passes. Each pass runs as one launch per round
// of SB_OCC workgroups per compute unit, the workgroups resident at once,
// so that they start together; special-row units (which walk every key
// tile in the same order and so stay in step) come first, then the patch
// units head by head. A patch unit walks its kept tiles in ascending
// order, and the units of a round drift apart as they go, until an XCD's
// L2 no longer holds a tile when the next unit reads it: every key tile
// then crosses the fabric once per unit. So patch units meet at a
// checkpoint every SB_CK_TILES key tiles. Counters are per XCD group
// (workgroups are dealt to the XCDs in turn, so the L2 a workgroup shares
// is that of blockIdx.x % 8); a workgroup goes on once SB_CK_PCT percent of
// its group's patch units have arrived, or after SB_CK_SPIN polls, so no
// wait is unbounded. A unit whose kept tiles skip a segment still arrives
// at the checkpoints in between, and at the remaining ones when its token
// walk ends, so every checkpoint is reached by every patch unit of the
// round.
constexpr int SB_OCC = 4;          // workgroups of the query-major passes per compute unit
constexpr int SB_XG = 8;           // XCD groups
constexpr int SB_CK_TILES = 2048;  // key tiles per checkpoint segment
constexpr int SB_CK_PCT = 85;
constexpr int SB_CK_SPIN = 1000;
constexpr int SB_ROUND_MIN = 256;  // smallest round the workspace provides counters for

struct SbRound {
  int u0;      // first flattened unit of the round
  int pfirst;  // flattened index of the first patch unit (H x special units per head)
  int nck;     // checkpoints per walk (segments - 1)
  int* ck;     // this round's counters [nck][SB_XG], zero at launch
};

typedef void __attribute__((address_space(3))) sb_lds_void;
typedef short sb_v4s __attribute__((ext_vector_type(4)));
typedef void __attribute__((address_space(3))) sb_lds_void;

// ---------------------------------------------------------------- rows and units

// A query unit: patch tile t (< T), or special-row unit T + s (64 special
// rows each). Rows of a unit and the token of its row j.
__device__ inline int unit_rows(const Geom& g, int unit) {
  if (unit < g.T) return tile_n(g, unit - frame_of_tile(g, unit) * g.tpf);
  return min(64, g.nspec - (unit - g.T) * 64);
}

__device__ inline long long unit_token(const Geom& g, int unit, int j) {
  if (unit < g.T) {
    const int f = frame_of_tile(g, unit), tl = unit - f * g.tpf;
    const int a = tl / g.tc, b = tl - a * g.tc;
    const int tw = tile_w(g, tl);
    const int jr = j / tw;
    const int r = TILE * a + jr, c = TILE * b + (j - jr * tw);
    return (long long)f * g.tok_pf + g.S + (long long)r * g.C + c;
  }
  const int i = (unit - g.T) * 64 + j;
  const int f = i / g.S;
  return (long long)f * g.tok_pf + (i - f * g.S);
}

__device__ inline long long special_token(const Geom& g, int i) {
  const int f = i / g.S;
  return (long long)f * g.tok_pf + (i - f * g.S);
}

__device__ inline int num_units(const Geom& g) { return g.T + (g.nspec + 63) / 64; }

// ---------------------------------------------------------------- LDS tiles
// A tile of 32 rows x 64 bf16 channels (4 KB), the 16-byte chunk c of row
// r stored at chunk c ^ (r % 8): the 16 lanes of an A-operand read (16 rows,
// one chunk column) and of a transposing read (4 rows x 4 pieces) spread
// over the banks.
__device__ inline int sb_off(int r, int ch) { return r * D + ((((ch >> 3) ^ (r & 7))) << 3) + (ch & 7); }

// A operand rows 16 h + lane%16, channels 32 ks + 8 (lane/16) .. +7
__device__ inline bf16x8 row_frag(const u16* t, int h, int ks, int lane) {
  const int r = 16 * h + (lane & 15);
  return *(const bf16x8*)(t + sb_off(r, 32 * ks + 8 * (lane >> 4)));
}

// A operand of the transposed tile: rows = channels 16 cb + lane%16, k-slots
// 8 g + j = tile rows 4 g + j (j < 4) and 16 + 4 g + j - 4 (j >= 4), g = lane/16.
__device__ inline bf16x8 col_frag(const u16* t, int cb, int lane) {
  typedef __attribute__((address_space(3))) sb_v4s lds_v4s;
  const int i = lane & 15, g = lane >> 4;
  const int ch = 16 * cb + 4 * (i & 3);
  const sb_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + sb_off(4 * g + (i >> 2), ch)));
  const sb_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + sb_off(16 + 4 * g + (i >> 2), ch)));
  typedef short sb_v8s __attribute__((ext_vector_type(8)));
  const sb_v8s v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ inline unsigned sb_pack(float a, float b) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, b2));
}

// 8 lane values (the lane's two 4-row halves) as a bf16 B operand
__device__ inline bf16x8 pack8(const float v[8]) {
  return __builtin_bit_cast(bf16x8, make_uint4(sb_pack(v[0], v[1]), sb_pack(v[2], v[3]), sb_pack(v[4], v[5]),
                                               sb_pack(v[6], v[7])));
}

// Sum / max over the 4 lanes l, l^16, l^32, l^48 that hold one row's or
// key's pieces.
__device__ inline float sb_sum4(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sb_max4(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 16 bytes (8 channels) at element offset `off` of a bf16 tensor; zeros
// when !ok
__device__ inline uint4 ld16(const u16* base, long long off, bool ok) {
  return ok ? *(const uint4*)(base + off) : make_uint4(0u, 0u, 0u, 0u);
}

struct SbArgs {
  const u16* Q;
  const u16* K;
  const u16* V;
  const u16* dO;
  const u16* LM;          // landmark key blocks (row 32: fp32 log2 n)
  const double* kbar;     // [H][T][64] exact landmark keys
  const float* vbar;      // [H][T][64] landmark values
  const int* sel;         // [H][T][keep] kept tiles, ascending
  const unsigned* selmask;   // [H][T][nw] bit u of word u/32: t keeps u
  unsigned* selT;            // [H][T][nw] bit t of word t/32: t keeps u
  float* lse;             // [H][N] log2-sum-exp2 of the row's logits (log2 units)
  float* dsum;            // [H][N] D
  float* part;            // [SB_CHUNKS][H][nspec_pad + T_pad][2][64] partial dk, dv of global keys
  float* lgrad;           // [H][T][2][64] landmark dk, dv
  u16* lmp;               // [H][ceil(T/64)][4][64][64] landmark bf16 parts (sbwd_lmparts_kernel)
  u16* dQ;
  u16* dK;
  u16* dV;
  int keep, nw;
  long long o_tok, o_head;  // dout strides
  unsigned tc_magic;        // floor(2^32 / tc) + 1 (tc >= 2): tile row of a frame's tile by multiply-high
};

__device__ inline const char* lm_kblock(const Geom& g, const u16* LM, int h, int b) {
  return (const char*)LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE + (long long)b * LM_KEY_BLOCK;
}

// Token of the first key of tile u (row-major within the tile), and u's
// tile within its frame; no divisions (multiply-high by the frame's and
// the tile row's reciprocals).
// tc_magic = floor(2^32 / tc) + 1 (tc >= 2): v / tc = umulhi(v, tc_magic)
// for v * tc < 2^32.
__device__ inline long long tile_first_token(const Geom& g, unsigned tc_magic, int u, int& tl) {
  const int f = frame_of_tile(g, u);
  tl = u - f * g.tpf;
  const int a = g.tc == 1 ? tl : (int)__umulhi((unsigned)tl, tc_magic), b = tl - a * g.tc;
  return (long long)f * g.tok_pf + g.S + (long long)TILE * a * g.C + TILE * b;
}

// Token offset, from the tile's first token, of its row-major key j in a
// tile w tokens wide (meaningful for j below the tile's key count; callers
// discard the value otherwise, and unsigned arithmetic keeps it defined).
__device__ inline unsigned in_tile(const Geom& g, int j, int w) {
  return (unsigned)(j / w) * (unsigned)g.C + (unsigned)(j % w);
}

// ---------------------------------------------------------------- query-major passes

enum { SB_STATS = 0, SB_DQ = 1 };

// 8 fp32 values as bf16 high parts and low parts (the rounding remainders)
__device__ inline void split8(const float v[8], uint4& hi, uint4& lo) {
  unsigned h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = sb_pack(v[2 * i], v[2 * i + 1]);
    l[i] = sb_pack(v[2 * i] - __uint_as_float(h[i] << 16), v[2 * i + 1] - __uint_as_float(h[i] & 0xFFFF0000u));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Channels c8 .. c8 + 7 of landmark u: the exact mean key (fp64) and value
// (fp32), each as bf16 high and low parts.
__device__ inline void landmark_parts(const Geom& g, const SbArgs& A, int h, int u, int c8, uint4& khi, uint4& klo,
                                      uint4& vhi, uint4& vlo) {
  const double* kr = A.kbar + ((long long)h * g.T + u) * D + c8;
  const float4* vr = (const float4*)(A.vbar + ((long long)h * g.T + u) * D + c8);
  float kv[8], vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) kv[i] = (float)kr[i];
  const float4 a = vr[0], b = vr[1];
  vv[0] = a.x;
  vv[1] = a.y;
  vv[2] = a.z;
  vv[3] = a.w;
  vv[4] = b.x;
  vv[5] = b.y;
  vv[6] = b.z;
  vv[7] = b.w;
  split8(kv, khi, klo);
  split8(vv, vhi, vlo);
}

// grid (ceil(T / 64), H), block 256: the bf16 high and low parts of the
// exact mean keys and values of landmarks 64 b .. 64 b + 63 (zero rows past
// the last tile), laid out as the query-major passes hold a landmark block
// in LDS: [K high, V high, K low, V low], each 64 rows at sb_off. Those
// passes then copy a block into LDS as it is, with no conversion.
__global__ void __launch_bounds__(256) sbwd_lmparts_kernel(Geom g, SbArgs A, int nlb) {
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, u = 64 * b + r;
  u16* dst = A.lmp + ((long long)h * nlb + b) * 4 * 64 * D;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c8 = 16 * (tid & 3) + 8 * i;
    uint4 khi = make_uint4(0u, 0u, 0u, 0u), klo = khi, vhi = khi, vlo = khi;
    if (u < g.T) landmark_parts(g, A, h, u, c8, khi, klo, vhi, vlo);
    const int off = sb_off(r, c8);
    *(uint4*)(dst + off) = khi;
    *(uint4*)(dst + 64 * D + off) = vhi;
    *(uint4*)(dst + 2 * 64 * D + off) = klo;
    *(uint4*)(dst + 3 * 64 * D + off) = vlo;
  }
}

// grid (units, H), block 256: one query unit (up to 64 rows, 16 per wave).
template <int MODE>
__global__ void __launch_bounds__(SB_THREADS, SB_OCC) sbwd_rows_kernel(Geom g, SbArgs A, SbRound R) {
  __shared__ __attribute__((aligned(16))) u16 sK[64 * D], sV[64 * D], sK2[64 * D], sV2[64 * D];
  __shared__ __attribute__((aligned(16))) float sB[64], sB2[64];
  const int nsu = (g.nspec + 63) / 64;
  const int uid = R.u0 + blockIdx.x;
  int unit, h;
  if (uid < R.pfirst) {
    h = uid / nsu;
    unit = g.T + (uid - h * nsu);
  } else {
    h = (uid - R.pfirst) / g.T;
    unit = (uid - R.pfirst) - h * g.T;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = lane >> 4, tl = lane & 15;
  const bool patch = unit < g.T;
  const int nrows = unit_rows(g, unit);
  const int j = 16 * wave + tl;  // this lane's row of the unit
  const bool valid = j < nrows;
  const long long tok = valid ? unit_token(g, unit, j) : 0;
  const long long qrow = tok * g.in_tok + (long long)h * g.in_head;
  const long long orow = tok * A.o_tok + (long long)h * A.o_head;
  bf16x8 qb[2], ob[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    qb[ks] = __builtin_bit_cast(bf16x8, ld16(A.Q, qrow + 32 * ks + 8 * lg, valid));
    ob[ks] = __builtin_bit_cast(bf16x8, ld16(A.dO, orow + 32 * ks + 8 * lg, valid));
  }
  // The row's own key: its logit xs and dP (from the lane's 16 channels,
  // summed over the row's 4 lanes). A patch row always sees its own token
  // (in its kept tile or as the self key) and a special row sees every
  // token, so xs is at most the row's largest logit.
  float xs, dps;
  {
    const u16* kr = A.K + qrow;
    const u16* vr = A.V + qrow;
    float sq = 0.f, sd = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 kw = ld16(kr, 32 * ks + 8 * lg, valid), vw = ld16(vr, 32 * ks + 8 * lg, valid);
      const uint4 qw = __builtin_bit_cast(uint4, qb[ks]), ow = __builtin_bit_cast(uint4, ob[ks]);
      const unsigned qa[4] = {qw.x, qw.y, qw.z, qw.w}, ka[4] = {kw.x, kw.y, kw.z, kw.w};
      const unsigned oa[4] = {ow.x, ow.y, ow.z, ow.w}, va[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sq = fmaf(__uint_as_float(qa[e] << 16), __uint_as_float(ka[e] << 16), sq);
        sq = fmaf(__uint_as_float(qa[e] & 0xFFFF0000u), __uint_as_float(ka[e] & 0xFFFF0000u), sq);
        sd = fmaf(__uint_as_float(oa[e] << 16), __uint_as_float(va[e] << 16), sd);
        sd = fmaf(__uint_as_float(oa[e] & 0xFFFF0000u), __uint_as_float(va[e] & 0xFFFF0000u), sd);
      }
    }
    xs = sb_sum4(sq) * SB_C;
    dps = sb_sum4(sd);
  }
  // STATS: per-lane partials over the lane's keys, relative to a running
  // offset m (log2 units) that starts at the own logit and only moves up.
  // DQ: the row's statistics, which enter as the initial values of the
  // logit and dP accumulators (-lse / C and -D), so that a logit leaves the
  // MFMAs with the row's log-sum-exp taken off and dP with D taken off.
  // Rows past the unit's end have zero q, dout and statistics, so their dS
  // is exactly zero and reaches only their own (unwritten) dq column.
  float m = valid ? xs : 64.f, l = 0.f, dsm = 0.f;  // (past the end: no logit reaches m)
  float lse2 = 0.f, Drow = 0.f;
  if (MODE == SB_DQ && valid) {
    lse2 = A.lse[(long long)h * g.N + tok];
    Drow = A.dsum[(long long)h * g.N + tok];
  }
  const float soff_dq = -lse2 * (1.0f / SB_C), doff_dq = -Drow;
  f32x4 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 32 staged keys (rows 32 sub .. of the LDS tiles) against the wave's rows
  auto block = [&](int kind, int sub, const u16* bK, const u16* bV, const float* bB) {
    const u16* tK = bK + sub * 32 * D;
    const u16* tV = bV + sub * 32 * D;
    const u16* tK2 = sK2 + sub * 32 * D;
    const u16* tV2 = sV2 + sub * 32 * D;
    const float* tB = bB + 32 * sub;
    const float so = MODE == SB_STATS ? -m * (1.0f / SB_C) : soff_dq;
    const float dpo = MODE == SB_STATS ? 0.f : doff_dq;
    f32x4 s[2], dp[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      s[hh] = f32x4{so, so, so, so};
      dp[hh] = f32x4{dpo, dpo, dpo, dpo};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        s[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_frag(tK, hh, ks, lane), qb[ks], s[hh], 0, 0, 0);
        dp[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_frag(tV, hh, ks, lane), ob[ks], dp[hh], 0, 0, 0);
        if (kind == 2) {
          s[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_frag(tK2, hh, ks, lane), qb[ks], s[hh], 0, 0, 0);
          dp[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_frag(tV2, hh, ks, lane), ob[ks], dp[hh], 0, 0, 0);
        }
      }
    }
    // lane (row tl, group lg) holds keys 4 lg + r and 16 + 4 lg + r
    const float4 b0 = *(const float4*)(tB + 4 * lg), b1 = *(const float4*)(tB + 16 + 4 * lg);
    const float bias[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    float x[8], d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = fmaf(s[i >> 2][i & 3], SB_C, bias[i]);
      d[i] = dp[i >> 2][i & 3];
    }
    if (MODE == SB_STATS) {
      // x = logit - m. The offset moves only when some lane of the wave
      // sees a logit above its own m (a wave-uniform branch, taken on a
      // few percent of the blocks); the other lanes shift by zero.
      float bm = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) bm = fmaxf(bm, x[i]);
      if (__builtin_amdgcn_ballot_w64(bm > 0.f)) {
        const float sh = fmaxf(bm, 0.f), sc = __builtin_amdgcn_exp2f(-sh);
        m += sh;
        l *= sc;
        dsm *= sc;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] -= sh;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[i]);
        l += p;
        dsm = fmaf(p, d[i], dsm);
      }
    } else {
      // x = logit - lse, d = dP - D
      float ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ds[i] = __builtin_amdgcn_exp2f(x[i]) * d[i];
      const bf16x8 dsb = pack8(ds);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(col_frag(tK, cb, lane), dsb, acc[cb], 0, 0, 0);
        if (kind == 2)
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(col_frag(tK2, cb, lane), dsb, acc[cb], 0, 0, 0);
      }
    }
  };

  // The unit's key blocks in order, 64 keys each: its kept tiles (all tiles
  // for special rows), the special keys, then (patch rows) the landmarks.
  const int* kept = A.sel + ((long long)h * g.T + unit) * A.keep;
  const unsigned* mrow = A.selmask + ((long long)h * g.T + (patch ? unit : 0)) * A.nw;
  const int ntb = patch ? A.keep : g.T, nsb = (g.nspec + 63) / 64, nlb = patch ? (g.T + 63) / 64 : 0;
  const int nblk = ntb + nsb;
  auto desc = [&](int i, int& kind, int& blk) {
    if (i < ntb) {
      kind = 0;
      blk = patch ? kept[i] : i;
    } else {
      kind = 1;
      blk = i - ntb;
    }
  };
  // Token and special blocks go into LDS by async 16-byte copies, one block
  // ahead, alternating between two buffers: (sK, sV, sB) and (sK2, sV2,
  // sB2), the landmark low-part tiles, which are free until the landmark
  // blocks. The loop is unrolled over the two buffers so that every LDS
  // access names its array and the compiler sees that the fragment reads
  // miss the copies in flight. One barrier per block.
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  // checkpoints (patch units): the counters of this workgroup's XCD group,
  // the release target (SB_CK_PCT percent of the group's patch units in the
  // round: flattened units >= pfirst, so blocks >= bp), and the segment the
  // walk is in
  const int xg = blockIdx.x % SB_XG;
  int* ckg = R.ck + xg;
  int ck_target = 0;
  if (patch && R.nck > 0) {
    const int bp = max(0, R.pfirst - R.u0);
    auto cnt = [&](int m) { return m > xg ? (m - xg + SB_XG - 1) / SB_XG : 0; };
    ck_target = ((cnt((int)gridDim.x) - cnt(bp)) * SB_CK_PCT + 99) / 100;
  }
  int cseg = 0;
  // arrive at checkpoints cseg .. c1 - 1 (one arrival per workgroup), then,
  // if asked, poll until the group's target has arrived at c1 - 1
  auto cross = [&](int c1, bool wait) __attribute__((always_inline)) {
    if (threadIdx.x == 0)
      for (int c = cseg; c < c1; ++c) __hip_atomic_fetch_add(ckg + c * SB_XG, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wait) {
      int* ctr = ckg + (c1 - 1) * SB_XG;
#pragma nounroll
      for (int it = 0; it < SB_CK_SPIN; ++it) {
        const int v = __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (v >= ck_target) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    cseg = c1;
  };
  // Element offsets, from a token tile's first key row, of this lane's
  // 16-byte source chunk in each of its two copy rows (16 w + 8 j + lane / 8,
  // chunk (lane % 8) ^ (row % 8), so that LDS holds the sb_off layout), for
  // a tile of full width (TILE) and one of the last tile column's width
  // (computed once: every tile has one of the two widths), and for a row
  // past the tile's last key, which reads the first key (its bias is -inf,
  // so it adds exact zeros). The host keeps TILE tile rows of tokens below
  // 2^31 elements, so the offsets fit 32 bits.
  const int wlast = g.C - TILE * (g.tc - 1);
  unsigned cf[2], cl[2], c0[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * wu + 8 * j + (lane >> 3);
    const unsigned ch = 8u * (unsigned)((lane & 7) ^ (r & 7));
    cf[j] = in_tile(g, r, TILE) * (unsigned)g.in_tok + ch;
    cl[j] = in_tile(g, r, wlast) * (unsigned)g.in_tok + ch;
    c0[j] = ch;
  }
  // (kind, key count) of block i come back to the caller, which hands them
  // to compute: a second read of the kept-tile list there would be a memory
  // load issued after the next block's copies, and waiting for it would
  // wait for them too
  auto issue = [&](int i, u16* bK, u16* bV, float* bB, int& kind, int& nk) __attribute__((always_inline)) {
    int blk;
    desc(i, kind, blk);
    if (patch && R.nck > 0 && kind == 0) {
      const int sg = min(blk / SB_CK_TILES, R.nck);
      if (sg > cseg) cross(sg, true);
    }
    // wave w copies rows 16 w + 8 j + lane / 8 (above); rows past a special
    // block's last key repeat it (bias -inf)
    if (kind == 0) {
      // token tile: a uniform base row, per-lane 32-bit offsets
      int tl;
      const long long tok0 = tile_first_token(g, A.tc_magic, blk, tl);
      nk = tile_n(g, tl);
      const bool full = tile_w(g, tl) == TILE;
      const long long base = tok0 * g.in_tok + (long long)h * g.in_head;
      const u16* kb = A.K + base;
      const u16* vb = A.V + base;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r0 = 16 * wu + 8 * j;
        const unsigned off = r0 + (lane >> 3) >= nk ? c0[j] : full ? cf[j] : cl[j];
        __builtin_amdgcn_global_load_lds((const void*)(kb + off), (sb_lds_void*)(bK + r0 * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vb + off), (sb_lds_void*)(bV + r0 * D), 16, 0, 0);
      }
    } else {
      nk = min(64, g.nspec - 64 * blk);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r0 = 16 * wu + 8 * j, r = r0 + (lane >> 3);
        const long long src = special_token(g, 64 * blk + min(r, nk - 1)) * g.in_tok + (long long)h * g.in_head +
                              8 * ((lane & 7) ^ (r & 7));
        __builtin_amdgcn_global_load_lds((const void*)(A.K + src), (sb_lds_void*)(bK + r0 * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(A.V + src), (sb_lds_void*)(bV + r0 * D), 16, 0, 0);
      }
    }
    if (threadIdx.x < 64) bB[threadIdx.x] = (int)threadIdx.x < nk ? 0.f : -INFINITY;
  };
  auto compute = [&](int kind, int nk, const u16* bK, const u16* bV, const float* bB) __attribute__((always_inline)) {
    block(kind, 0, bK, bV, bB);
    if (nk > 32) block(kind, 1, bK, bV, bB);
  };
  int k0 = 0, n0 = 0, k1 = 0, n1 = 0;  // (kind, key count) of the block in each buffer
  if (nblk > 0) issue(0, sK, sV, sB, k0, n0);
  for (int i = 0; i < nblk; i += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of block i have landed
    __syncthreads();  // ... in every wave, and block i - 1 is read
    if (i + 1 < nblk) issue(i + 1, sK2, sV2, sB2, k1, n1);
    compute(k0, n0, sK, sV, sB);
    if (i + 1 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (i + 2 < nblk) issue(i + 2, sK, sV, sB, k0, n0);
    compute(k1, n1, sK2, sV2, sB2);
  }
  if (patch && cseg < R.nck) cross(R.nck, false);
  // landmark blocks (patch rows): their precomputed bf16 parts copied into
  // the LDS tiles as they are (async 16-byte copies, wave w one part), and
  // the row's biases (log2 n_u; -inf past the last tile or where the row's
  // tile keeps it)
  {
    u16* dpart = wu == 0 ? sK : wu == 1 ? sV : wu == 2 ? sK2 : sV2;
    for (int b = 0; b < nlb; ++b) {
      __syncthreads();  // the previous block's reads are done
      const u16* src = A.lmp + (((long long)h * nlb + b) * 4 + wu) * 64 * D + 8 * lane;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(src + 512 * i), (sb_lds_void*)(dpart + 512 * i), 16, 0, 0);
      if (threadIdx.x < 64) {
        const int t = threadIdx.x, b32 = 2 * b + (t >> 5), key = t & 31;
        float bias = -INFINITY;
        if (64 * b + t < g.T && !(((b32 < A.nw ? mrow[b32] : ~0u) >> key) & 1u))
          bias = ((const float*)(lm_kblock(g, A.LM, h, b32) + LM_LOG2N_ROW * 128))[key];
        sB[t] = bias;
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
      __syncthreads();
      block(2, 0, sK, sV, sB);
      if (64 * b + 32 < g.T) block(2, 1, sK, sV, sB);
    }
  }
  // the self key: a patch row whose own tile is not kept attends to its
  // own key (logit xs, dP dps from above)
  bool self = false;
  if (patch) self = ((mrow[unit >> 5] >> (unit & 31)) & 1u) == 0;
  if (MODE == SB_STATS) {
    if (self && lg == 0) {  // one of the row's 4 lanes counts the self key
      const float mx = fmaxf(m, xs), sc = __builtin_amdgcn_exp2f(m - mx), p = __builtin_amdgcn_exp2f(xs - mx);
      l = l * sc + p;
      dsm = dsm * sc + p * dps;
      m = mx;
    }
    const float M = sb_max4(m);
    const float sc = __builtin_amdgcn_exp2f(m - M);
    const float L = sb_sum4(l * sc), Dn = sb_sum4(dsm * sc);
    if (valid && lg == 0) {
      A.lse[(long long)h * g.N + tok] = M + __log2f(L);
      A.dsum[(long long)h * g.N + tok] = Dn / L;
    }
  } else {
    // dq of row j (lane tl): channels 16 cb + 4 lg + r, times 1/8, plus the
    // self key's dS k / 8
    const float dss = self ? __builtin_amdgcn_exp2f(xs - lse2) * (dps - Drow) : 0.f;
    if (valid) {
      u16* out = A.dQ + qrow;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int ch = 16 * cb + 4 * lg;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[cb][r];
        if (self) {
          const uint2 kw = *(const uint2*)(A.K + qrow + ch);
          v[0] = fmaf(dss, __uint_as_float(kw.x << 16), v[0]);
          v[1] = fmaf(dss, __uint_as_float(kw.x & 0xFFFF0000u), v[1]);
          v[2] = fmaf(dss, __uint_as_float(kw.y << 16), v[2]);
          v[3] = fmaf(dss, __uint_as_float(kw.y & 0xFFFF0000u), v[3]);
        }
        *(uint2*)(out + ch) = make_uint2(sb_pack(v[0] * 0.125f, v[1] * 0.125f), sb_pack(v[2] * 0.125f, v[3] * 0.125f));
      }
    }
  }
}

// ---------------------------------------------------------------- transposed selection

// grid (ceil(nw / 2), nw, H), block 64: two 32 x 32 bit blocks per wave.
// Lane i of half b' reads word [t = 32 a + i][wb] of the kept bitmap; the
// ballot of bit j over the half is word [u = 32 wb + j][a] of the transposed
// bitmap.
__global__ void __launch_bounds__(64) sbwd_transpose_kernel(Geom g, const unsigned* __restrict__ selmask,
                                                            unsigned* __restrict__ selT, int nw) {
  const int lane = threadIdx.x, half = lane >> 5, i = lane & 31;
  const int wb = 2 * blockIdx.x + half, a = blockIdx.y, h = blockIdx.z;
  const int t = 32 * a + i;
  unsigned w = 0u;
  if (wb < nw && t < g.T) w = selmask[((long long)h * g.T + t) * nw + wb];
  unsigned mine = 0u;
#pragma unroll 4
  for (int j = 0; j < 32; ++j) {
    const unsigned long long b = __ballot((w >> j) & 1u);
    const unsigned col = half ? (unsigned)(b >> 32) : (unsigned)b;
    if (i == j) mine = col;
  }
  const int u = 32 * wb + i;
  if (wb < nw && u < g.T) selT[((long long)h * g.T + u) * nw + a] = mine;
}

// ---------------------------------------------------------------- key-major passes

enum { SB_TILE = 0, SB_SPEC = 1, SB_LMK = 2 };

// grid:
//   TILE (T, H):                 keys = the tokens of tile blockIdx.x
//   SPEC (ceil(nspec/64), H, SB_CHUNKS), LMK (ceil(T/64), H, SB_CHUNKS):
//                                keys = 64 special keys or landmarks, rows =
//                                chunk blockIdx.z of the query units
// Wave w owns keys 16 w .. 16 w + 15 (lane tl: key 16 w + tl).
template <int MODE>
__global__ void __launch_bounds__(SB_THREADS, 3) sbwd_keys_kernel(Geom g, SbArgs A) {
  __shared__ __attribute__((aligned(16))) u16 sQ[32 * D], sO[32 * D];
  __shared__ __attribute__((aligned(16))) float sL[32], sD[32];
  __shared__ unsigned sT[MODE == SB_TILE ? 1024 : 1];  // TILE: this key tile's transposed-bitmap row (T <= 32,768)
  const int kb = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = lane >> 4, tl = lane & 15;
  const int key = 16 * wave + tl;
  // this lane's key: its K and V rows as B operands, and its logit bias
  bool kvalid;
  long long ktok = 0;
  int lmk = 0;
  float kbias = 0.f;
  bf16x8 kfrag[2], vfrag[2], kfrag2[2], vfrag2[2];  // *2: low parts (landmarks only)
  if (MODE == SB_TILE) {
    kvalid = key < unit_rows(g, kb);
    if (kvalid) ktok = unit_token(g, kb, key);
  } else if (MODE == SB_SPEC) {
    const int i = 64 * kb + key;
    kvalid = i < g.nspec;
    if (kvalid) ktok = special_token(g, i);
  } else {
    lmk = 64 * kb + key;
    kvalid = lmk < g.T;
  }
  if (MODE == SB_LMK) {
    const char* blk = lm_kblock(g, A.LM, h, lmk >> 5);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 kw = make_uint4(0u, 0u, 0u, 0u), vw = kw, kl = kw, vl = kw;
      if (kvalid) landmark_parts(g, A, h, lmk, 32 * ks + 8 * lg, kw, kl, vw, vl);
      kfrag[ks] = __builtin_bit_cast(bf16x8, kw);
      vfrag[ks] = __builtin_bit_cast(bf16x8, vw);
      kfrag2[ks] = __builtin_bit_cast(bf16x8, kl);
      vfrag2[ks] = __builtin_bit_cast(bf16x8, vl);
    }
    kbias = kvalid ? ((const float*)(blk + LM_LOG2N_ROW * 128))[lmk & 31] : -INFINITY;
  } else {
    const long long row = ktok * g.in_tok + (long long)h * g.in_head;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kfrag[ks] = __builtin_bit_cast(bf16x8, ld16(A.K, row + 32 * ks + 8 * lg, kvalid));
      vfrag[ks] = __builtin_bit_cast(bf16x8, ld16(A.V, row + 32 * ks + 8 * lg, kvalid));
    }
    kbias = kvalid ? 0.f : -INFINITY;
  }
  f32x4 dk[4], dv[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) dk[cb] = dv[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One thread's share of rows 32 hb .. +31 of query unit t (row tid / 8,
  // channels 8 (tid % 8) .. +7), loaded one step ahead of its use, and the
  // lane's landmark mask word of the unit.
  struct RowFetch {
    uint4 q, o;
    float lse, d;
    unsigned mw;
  };
  // Token offsets, from a patch tile's first token, of this thread's rows
  // 32 hb + tid / 8 (hb = 0, 1) in a tile of full width (TILE) and in one
  // of the last tile column's width, computed once: a patch unit's rows
  // are then a uniform base plus a per-thread offset, with no division.
  const int wlast = g.C - TILE * (g.tc - 1);
  const unsigned tf0 = in_tile(g, threadIdx.x >> 3, TILE), tf1 = in_tile(g, 32 + (threadIdx.x >> 3), TILE);
  const unsigned tw0 = in_tile(g, threadIdx.x >> 3, wlast), tw1 = in_tile(g, 32 + (threadIdx.x >> 3), wlast);
  auto fetch_rows = [&](int t, int hb, RowFetch& f) {
    const int tid = threadIdx.x, r = tid >> 3, c = tid & 7;
    const int jr = 32 * hb + r;
    bool ok;
    long long tk0;    // uniform: the unit's first token (patch) or 0 (special rows)
    unsigned toff;    // this thread's row: token tk0 + toff
    if (t < g.T) {
      int tl;
      tk0 = tile_first_token(g, A.tc_magic, t, tl);
      ok = jr < tile_n(g, tl);
      const bool full = tile_w(g, tl) == TILE;
      toff = !ok ? 0u : full ? (hb ? tf1 : tf0) : (hb ? tw1 : tw0);
    } else {
      ok = jr < unit_rows(g, t);
      tk0 = 0;
      toff = ok ? (unsigned)unit_token(g, t, jr) : 0u;
    }
    // q and dout rows: uniform bases, 32-bit per-thread element offsets
    // (the host keeps 8 patch rows below 2^31 elements; special rows take
    // the 64-bit path through a zero base)
    const u16* qb = A.Q + tk0 * g.in_tok + (long long)h * g.in_head;
    const u16* ob = A.dO + tk0 * A.o_tok + (long long)h * A.o_head;
    if (t < g.T) {
      f.q = ld16(qb, (long long)(toff * (unsigned)g.in_tok + 8u * c), ok);
      f.o = ld16(ob, (long long)(toff * (unsigned)A.o_tok + 8u * c), ok);
    } else {
      f.q = ld16(qb, (long long)toff * g.in_tok + 8 * c, ok);
      f.o = ld16(ob, (long long)toff * A.o_tok + 8 * c, ok);
    }
    f.lse = INFINITY;
    f.d = 0.f;
    if (ok && c == 0) {
      const long long i = (long long)h * g.N + tk0 + toff;
      f.lse = A.lse[i];
      f.d = A.dsum[i];
    }
    f.mw = 0u;
    if (MODE == SB_LMK && kvalid) f.mw = A.selmask[((long long)h * g.T + t) * A.nw + (lmk >> 5)];
  };
  auto commit_rows = [&](const RowFetch& f) {
    const int tid = threadIdx.x, r = tid >> 3, c = tid & 7;
    *(uint4*)(sQ + sb_off(r, 8 * c)) = f.q;
    *(uint4*)(sO + sb_off(r, 8 * c)) = f.o;
    if (c == 0) {
      sL[r] = -f.lse * (1.0f / SB_C);
      sD[r] = -f.d;
    }
  };
  // the staged rows against the workgroup's keys; `bias` is this lane's key
  // bias for the unit (-inf: not visible)
  auto rows = [&](float bias) {
    const u16* tQ = sQ;
    const u16* tO = sO;
    const float* tL = sL;
    const float* tD = sD;
    // lane (key tl, group lg) holds rows 4 lg + r and 16 + 4 lg + r; the
    // rows' -lse / C and -D are the initial values of the logit and dP
    // accumulators (rows past the unit's end: -inf and 0, so P = dS = 0)
    f32x4 s[2], dp[2];
    s[0] = *(const f32x4*)(tL + 4 * lg);
    s[1] = *(const f32x4*)(tL + 16 + 4 * lg);
    dp[0] = *(const f32x4*)(tD + 4 * lg);
    dp[1] = *(const f32x4*)(tD + 16 + 4 * lg);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 qa = row_frag(tQ, hh, ks, lane), oa = row_frag(tO, hh, ks, lane);
        s[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kfrag[ks], s[hh], 0, 0, 0);
        dp[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vfrag[ks], dp[hh], 0, 0, 0);
        if (MODE == SB_LMK) {
          s[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kfrag2[ks], s[hh], 0, 0, 0);
          dp[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vfrag2[ks], dp[hh], 0, 0, 0);
        }
      }
    }
    float p[8], ds[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(s[i >> 2][i & 3], SB_C, bias));
      ds[i] = p[i] * dp[i >> 2][i & 3];
    }
    const bf16x8 pb = pack8(p), dsb = pack8(ds);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      dv[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(col_frag(tO, cb, lane), pb, dv[cb], 0, 0, 0);
      dk[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(col_frag(tQ, cb, lane), dsb, dk[cb], 0, 0, 0);
    }
  };
  // The (unit, half) steps in order. TILE: the query tiles that keep this
  // tile (set bits of its transposed-bitmap row), then every special-row
  // unit; SPEC / LMK: the units of this chunk (no special rows for LMK).
  const int nunits = num_units(g);
  const unsigned* trow = A.selT + ((long long)h * g.T + (MODE == SB_TILE ? kb : 0)) * A.nw;
  int w = 0, tcur = -1;
  unsigned bits = 0u;
  int t0 = 0, t1 = 0;
  if (MODE == SB_TILE) {
    // the bitmap row goes to LDS once: words read in the walk are then LDS
    // reads, which do not wait for the next step's row loads in flight
    for (int i = threadIdx.x; i < A.nw; i += SB_THREADS) sT[i] = trow[i];
    __syncthreads();
    bits = A.nw > 0 ? (unsigned)__builtin_amdgcn_readfirstlane((int)sT[0]) : 0u;
  } else {
    const int lastu = MODE == SB_LMK ? g.T : nunits;  // special rows see no landmark
    const int c = blockIdx.z;
    t0 = (int)((long long)lastu * c / SB_CHUNKS);
    t1 = (int)((long long)lastu * (c + 1) / SB_CHUNKS);
  }
  // the unit after tcur, or -1
  auto next_unit = [&]() -> int {
    if (MODE != SB_TILE) {
      if (tcur < 0) return t0 < t1 ? t0 : -1;
      return tcur + 1 < t1 ? tcur + 1 : -1;
    }
    if (tcur >= g.T) return tcur + 1 < nunits ? tcur + 1 : -1;  // the special-row units
    while (bits == 0u && w + 1 < A.nw) bits = (unsigned)__builtin_amdgcn_readfirstlane((int)sT[++w]);
    if (bits) {
      const int t = 32 * w + __builtin_ctz(bits);
      bits &= bits - 1u;
      return t;
    }
    return g.T < nunits ? g.T : -1;
  };
  // the step after (t, hb), in place (t = -1: none)
  auto advance = [&](int& t, int& hb) {
    if (t < 0) return;
    if (hb == 0 && unit_rows(g, t) > 32) {
      hb = 1;
    } else {
      tcur = t;
      t = next_unit();
      hb = 0;
    }
  };
  // Rows are fetched two steps ahead, into two register sets used in turn:
  // a step commits its set to LDS, then the same set takes the rows two
  // steps on, so no set in flight is ever copied.
  int ta = next_unit(), ha = 0;  // the current step (rows in the set of its turn)
  int tb = ta, hb2 = ha;         // the next one (rows in the other set)
  advance(tb, hb2);
  RowFetch f0, f1;
  if (ta >= 0) fetch_rows(ta, ha, f0);
  if (tb >= 0) fetch_rows(tb, hb2, f1);
  auto step = [&](RowFetch& f) __attribute__((always_inline)) {
    float bias = kbias;
    if (MODE == SB_LMK && ((f.mw >> (lmk & 31)) & 1u)) bias = -INFINITY;
    int tc = tb, hc = hb2;
    advance(tc, hc);
    __syncthreads();  // the previous rows' reads are done
    commit_rows(f);
    if (tc >= 0) fetch_rows(tc, hc, f);
    __syncthreads();
    rows(bias);
    ta = tb;
    ha = hb2;
    tb = tc;
    hb2 = hc;
  };
  while (ta >= 0) {
    step(f0);
    if (ta < 0) break;
    step(f1);
  }

  // lane (key tl, group lg) holds channels 16 cb + 4 lg + r of dk (x 1/8 to
  // come) and dv
  if (MODE == SB_TILE) {
    if (!kvalid) return;
    float vk[16], vv[16];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vk[4 * cb + r] = dk[cb][r];
        vv[4 * cb + r] = dv[cb][r];
      }
    const long long row = ktok * g.in_tok + (long long)h * g.in_head;
    // the self key: a row of this tile whose tile is not kept attends to its
    // own key (row `key` of unit kb is token ktok)
    const bool self = ((A.selmask[((long long)h * g.T + kb) * A.nw + (kb >> 5)] >> (kb & 31)) & 1u) == 0;
    if (self) {
      const long long orow = ktok * A.o_tok + (long long)h * A.o_head;
      float qv[16], ov[16], kv[16], vw[16];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int ch = 16 * cb + 4 * lg;
        const uint2 a = *(const uint2*)(A.Q + row + ch), b = *(const uint2*)(A.dO + orow + ch);
        const uint2 c = *(const uint2*)(A.K + row + ch), d = *(const uint2*)(A.V + row + ch);
        const unsigned aa[2] = {a.x, a.y}, bb[2] = {b.x, b.y}, cc[2] = {c.x, c.y}, dd[2] = {d.x, d.y};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          qv[4 * cb + 2 * e] = __uint_as_float(aa[e] << 16);
          qv[4 * cb + 2 * e + 1] = __uint_as_float(aa[e] & 0xFFFF0000u);
          ov[4 * cb + 2 * e] = __uint_as_float(bb[e] << 16);
          ov[4 * cb + 2 * e + 1] = __uint_as_float(bb[e] & 0xFFFF0000u);
          kv[4 * cb + 2 * e] = __uint_as_float(cc[e] << 16);
          kv[4 * cb + 2 * e + 1] = __uint_as_float(cc[e] & 0xFFFF0000u);
          vw[4 * cb + 2 * e] = __uint_as_float(dd[e] << 16);
          vw[4 * cb + 2 * e + 1] = __uint_as_float(dd[e] & 0xFFFF0000u);
        }
      }
      float sq = 0.f, sd = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sq = fmaf(qv[i], kv[i], sq);
        sd = fmaf(ov[i], vw[i], sd);
      }
      sq = sb_sum4(sq);
      sd = sb_sum4(sd);
      const float ps = __builtin_amdgcn_exp2f(sq * SB_C - A.lse[(long long)h * g.N + ktok]);
      const float dss = ps * (sd - A.dsum[(long long)h * g.N + ktok]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        vk[i] = fmaf(dss, qv[i], vk[i]);
        vv[i] = fmaf(ps, ov[i], vv[i]);
      }
    }
    // 1/n of the tile's landmark gradient (already scaled like dk: the
    // landmark pass stores sum dS q, without the 1/8)
    const float invn = 1.0f / (float)unit_rows(g, kb);
    const float* lgk = A.lgrad + ((long long)h * g.T + kb) * 2 * D;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int ch = 16 * cb + 4 * lg;
      const float4 a = *(const float4*)(lgk + ch), b = *(const float4*)(lgk + D + ch);
      vk[4 * cb] = fmaf(a.x, invn, vk[4 * cb]);
      vk[4 * cb + 1] = fmaf(a.y, invn, vk[4 * cb + 1]);
      vk[4 * cb + 2] = fmaf(a.z, invn, vk[4 * cb + 2]);
      vk[4 * cb + 3] = fmaf(a.w, invn, vk[4 * cb + 3]);
      vv[4 * cb] = fmaf(b.x, invn, vv[4 * cb]);
      vv[4 * cb + 1] = fmaf(b.y, invn, vv[4 * cb + 1]);
      vv[4 * cb + 2] = fmaf(b.z, invn, vv[4 * cb + 2]);
      vv[4 * cb + 3] = fmaf(b.w, invn, vv[4 * cb + 3]);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int ch = 16 * cb + 4 * lg;
      *(uint2*)(A.dK + row + ch) = make_uint2(sb_pack(vk[4 * cb] * 0.125f, vk[4 * cb + 1] * 0.125f),
                                             sb_pack(vk[4 * cb + 2] * 0.125f, vk[4 * cb + 3] * 0.125f));
      *(uint2*)(A.dV + row + ch) =
          make_uint2(sb_pack(vv[4 * cb], vv[4 * cb + 1]), sb_pack(vv[4 * cb + 2], vv[4 * cb + 3]));
    }
  } else {
    // partial sums of this chunk: global key index (specials first, then
    // landmarks), [2][64] each
    const int gk = MODE == SB_SPEC ? 64 * kb + key : g.spec_pad + lmk;
    const int nglob = g.spec_pad + g.T_pad;
    float* pp = A.part + (((long long)blockIdx.z * g.H + h) * nglob + gk) * 2 * D;
    if (kvalid) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int ch = 16 * cb + 4 * lg;
        *(float4*)(pp + ch) = make_float4(dk[cb][0], dk[cb][1], dk[cb][2], dk[cb][3]);
        *(float4*)(pp + D + ch) = make_float4(dv[cb][0], dv[cb][1], dv[cb][2], dv[cb][3]);
      }
    }
  }
}

// grid (ceil((nspec + T) / 2), H), block 128: the partials of one global key
// per 64 threads (one channel each), summed over the chunks in order. A
// special key's sums are its dk (x 1/8) and dv; a landmark's go to lgrad.
__global__ void __launch_bounds__(128) sbwd_reduce_kernel(Geom g, SbArgs A) {
  const int h = blockIdx.y, ch = threadIdx.x & 63;
  const int i = 2 * blockIdx.x + (threadIdx.x >> 6);
  if (i >= g.nspec + g.T) return;
  const int gk = i < g.nspec ? i : g.spec_pad + (i - g.nspec);
  const int nglob = g.spec_pad + g.T_pad;
  float sk = 0.f, sv = 0.f;
  for (int c = 0; c < SB_CHUNKS; ++c) {
    const float* pp = A.part + (((long long)c * g.H + h) * nglob + gk) * 2 * D;
    sk += pp[ch];
    sv += pp[D + ch];
  }
  if (i < g.nspec) {
    const long long row = special_token(g, i) * g.in_tok + (long long)h * g.in_head;
    A.dK[row + ch] = f2bf(sk * 0.125f);
    A.dV[row + ch] = f2bf(sv);
  } else {
    float* lgk = A.lgrad + ((long long)h * g.T + (i - g.nspec)) * 2 * D;
    lgk[ch] = sk;
    lgk[D + ch] = sv;
  }
}

// ---------------------------------------------------------------- host side

// grid ceil(n / 256), block 256: zero n ints (checkpoint counters)
__global__ void __launch_bounds__(256) sbwd_zero_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Checkpoint counters of the query-major passes: [2 passes][rounds][nck][SB_XG],
// for rounds of at least SB_ROUND_MIN units.
struct SbCounters {
  int nck, rounds;
  size_t ints;
  explicit SbCounters(const Geom& g) {
    const int nseg = (g.T + SB_CK_TILES - 1) / SB_CK_TILES;
    nck = nseg > 1 ? nseg - 1 : 0;
    const long long units = (long long)g.H * (g.T + (g.nspec + 63) / 64);
    rounds = (int)((units + SB_ROUND_MIN - 1) / SB_ROUND_MIN);
    ints = (size_t)2 * rounds * (nck > 0 ? nck : 1) * SB_XG;
  }
};

size_t sparse_bwd_workspace_bytes(const Geom& g) {
  const size_t ck = SbCounters(g).ints * sizeof(int);
  const size_t nw = (size_t)(g.T + 31) / 32;
  const size_t stats = (size_t)2 * g.H * g.N * sizeof(float);
  const size_t selT = (size_t)g.H * g.T * nw * sizeof(unsigned);
  const size_t part = (size_t)SB_CHUNKS * g.H * (g.spec_pad + g.T_pad) * 2 * D * sizeof(float);
  const size_t lgrad = (size_t)g.H * g.T * 2 * D * sizeof(float);
  const size_t lmp = (size_t)g.H * ((g.T + 63) / 64) * 4 * 64 * D * sizeof(u16);
  return stats + selT + part + lgrad + lmp + ck + 256 * 6;
}

// Workspace: lse [H][N], dsum [H][N] fp32; selT [H][T][nw]; the global-key
// partials [SB_CHUNKS][H][spec_pad + T_pad][2][64] fp32; lgrad [H][T][2][64];
// the landmark parts [H][ceil(T / 64)][4][64][64] bf16; the checkpoint
// counters of the query-major passes.
hipError_t launch_sparse_bwd(const Geom& g, int keep, const u16* Q, const u16* K, const u16* V, const u16* dO,
                             long long o_tok, long long o_head, const u16* LM, const double* kbar,
                             const float* vbar, const int* sel,
                             const unsigned* selmask, u16* dQ, u16* dK, u16* dV, void* ws, hipStream_t s) {
  const int nw = (g.T + 31) / 32;
  auto align = [](char* p) { return (char*)(((uintptr_t)p + 255) & ~(uintptr_t)255); };
  char* p = align((char*)ws);
  SbArgs A;
  A.Q = Q;
  A.K = K;
  A.V = V;
  A.dO = dO;
  A.LM = LM;
  A.kbar = kbar;
  A.vbar = vbar;
  A.sel = sel;
  A.selmask = selmask;
  A.lse = (float*)p;
  A.dsum = A.lse + (size_t)g.H * g.N;
  p = align((char*)(A.dsum + (size_t)g.H * g.N));
  A.selT = (unsigned*)p;
  p = align((char*)(A.selT + (size_t)g.H * g.T * nw));
  A.part = (float*)p;
  p = align((char*)(A.part + (size_t)SB_CHUNKS * g.H * (g.spec_pad + g.T_pad) * 2 * D));
  A.lgrad = (float*)p;
  p = align((char*)(A.lgrad + (size_t)g.H * g.T * 2 * D));
  A.lmp = (u16*)p;
  p = align((char*)(A.lmp + (size_t)g.H * ((g.T + 63) / 64) * 4 * 64 * D));
  const SbCounters ckc(g);
  int* ck = (int*)p;
  A.dQ = dQ;
  A.dK = dK;
  A.dV = dV;
  A.keep = keep;
  A.nw = nw;
  A.o_tok = o_tok;
  A.o_head = o_head;
  A.tc_magic = g.tc >= 2 ? (unsigned)((1ULL << 32) / (unsigned)g.tc + 1) : 0u;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int rsz = max(SB_OCC * cus, SB_ROUND_MIN);
  const int total = g.H * (g.T + (g.nspec + 63) / 64);
  const int ckr = (ckc.nck > 0 ? ckc.nck : 1) * SB_XG;  // counters per round
  hipLaunchKernelGGL(sbwd_zero_kernel, dim3((unsigned)((ckc.ints + 255) / 256)), dim3(256), 0, s, ck, (int)ckc.ints);
  hipLaunchKernelGGL(sbwd_lmparts_kernel, dim3((g.T + 63) / 64, g.H), dim3(256), 0, s, g, A, (g.T + 63) / 64);
  for (int pass = 0; pass < 2; ++pass)
    for (int u0 = 0, r = 0; u0 < total; u0 += rsz, ++r) {
      const SbRound R{u0, g.H * ((g.nspec + 63) / 64), ckc.nck, ck + ((size_t)pass * ckc.rounds + r) * ckr};
      const int n = min(rsz, total - u0);
      if (pass == 0)
        hipLaunchKernelGGL(sbwd_rows_kernel<SB_STATS>, dim3(n), dim3(SB_THREADS), 0, s, g, A, R);
      else
        hipLaunchKernelGGL(sbwd_rows_kernel<SB_DQ>, dim3(n), dim3(SB_THREADS), 0, s, g, A, R);
    }
  hipLaunchKernelGGL(sbwd_transpose_kernel, dim3((nw + 1) / 2, nw, g.H), dim3(64), 0, s, g, selmask, A.selT, nw);
  if (g.nspec > 0)
    hipLaunchKernelGGL(sbwd_keys_kernel<SB_SPEC>, dim3((g.nspec + 63) / 64, g.H, SB_CHUNKS), dim3(SB_THREADS), 0, s,
                       g, A);
  hipLaunchKernelGGL(sbwd_keys_kernel<SB_LMK>, dim3((g.T + 63) / 64, g.H, SB_CHUNKS), dim3(SB_THREADS), 0, s, g, A);
  hipLaunchKernelGGL(sbwd_reduce_kernel, dim3((g.nspec + g.T + 1) / 2, g.H), dim3(128), 0, s, g, A);
  hipLaunchKernelGGL(sbwd_keys_kernel<SB_TILE>, dim3(g.T, g.H), dim3(SB_THREADS), 0, s, g, A);
  return hipGetLastError();
}

}  // namespace zebra
