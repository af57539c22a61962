// Tile selector for gfx950: fp64 tile scores and an exact fp64 top-k.
//
// Zebra3D pages, "Linear-centered stages plus tile-sparse stages": for each
// query tile the selector keeps a key-tile fraction 1 - y. A tile's score is
// the mean query of the query tile dotted with the key tile's mean key,
// divided by sqrt(64), over all key tiles of all frames. Ties go to the lower
// tile index. The kept/not-kept decision is taken on float64 scores on both
// sides of the parity check.
//
// Three kernels: qbar (mean patch query per tile, exact fp64 sums),
// scores (a 64x64-blocked fp64 product qbar . kbar^T on the fp64 matrix
// cores, each score stored rounded to fp32 as an order-preserving 32-bit
// key) and topk (one 1024-thread workgroup per query tile: the key of the
// k-th tile found by histogram range narrowing; rounding never reverses an
// order, so only tiles whose key equals that key can rank differently in
// fp64, and when they straddle the cut their fp64 scores are recomputed and
// ranked; then an ascending compaction from one scan of per-wave counts
// that also writes the bitmap).
#include "common.hpp"

namespace zebra {

__device__ inline long long tile_token_s(const Geom& g, int f, int tl, int s) {
  const int a = tl / g.tc, b = tl - a * g.tc;
  const int tw = tile_w(g, tl);
  const int r = TILE * a + s / tw, c = TILE * b + s % tw;
  return (long long)f * g.tok_pf + g.S + (long long)r * g.C + c;
}

// grid (ceil(T / 4), H), block 256: qbar[h][t][d] = mean over tile t's
// patch queries, wave w for tile 4 blockIdx.x + w, lane d for channel d.
// A tile holds at most 64 bf16 values (8-bit significands) per channel:
// whenever they span less than 2^38 in magnitude (any ordinary data) every
// partial sum and the total are exact in fp64, so the four independent
// partial sums, which give the loads room to overlap, equal a serial sum.
__global__ void __launch_bounds__(256) qbar_kernel(Geom g, const u16* __restrict__ Q,
                                                   double* __restrict__ qbar) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), h = blockIdx.y, d = threadIdx.x & 63;
  if (t >= g.T) return;
  const int f = t / g.tpf, tl = t - f * g.tpf;
  const int n = tile_n(g, tl);
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = 0; i < n; i += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + j < n) s[j] += (double)bf2f(Q[tile_token_s(g, f, tl, i + j) * g.in_tok + (long long)h * g.in_head + d]);
  }
  qbar[((long long)h * g.T + t) * D + d] = ((s[0] + s[1]) + (s[2] + s[3])) / n;
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Order key of a score rounded to fp32 (round to nearest even, which never
// reverses an order), -0 taken as +0: unsigned order is score order.
__device__ inline unsigned f32_key(float x) {
  if (x == 0.0f) x = 0.0f;
  const unsigned b = __float_as_uint(x);
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

__device__ inline float key_f32(unsigned k) {
  return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}

// Scores of query tiles [t0, t0+nq) of head h against every key tile:
// out[tq][u] = key((sum_d qbar[t0+tq][d] * kbar[u][d]) * 0.125), the products
// on the fp64 matrix cores, rounded to fp32 order keys on the way out.
//
// grid (key-tile ranges, ceil(nq/128)), block 512: a workgroup keeps a
// block of 128 query rows in LDS and walks its range of 64-wide key tiles;
// wave w computes the 32 x 32 part (rows 32 (w >> 1), columns 32 (w & 1)) of
// each as 2 x 2 16x16x4 MFMA tiles over the 16 steps of 4 channels (two
// waves per SIMD, so one's stores and waits run under the other's matrix
// work). Key tiles
// stream into two LDS buffers by async 16-byte global-to-LDS copies, one
// tile ahead of the one being multiplied, so the copies run under the
// matrix work. A key tile row is 32 16-byte chunks, chunk c stored at slot
// c ^ (row % 16): the 16 rows that a step reads then fall on different
// banks (in the query block a row stride of 68 doubles does that). A tile's
// keys are stored while the next tile is multiplied, so the full wait at
// the start of a tile finds only copies and stores issued a tile earlier.
// Rows past the end repeat the last row (their scores are not stored).
constexpr int SC_LD = D + 4;        // query block row stride (doubles)
constexpr int SC_KT = 64 * D;       // one key tile (doubles)
constexpr int SC_QB = 128;          // query rows per workgroup
constexpr int SC_WAVES = SC_QB / 16;  // each 32 x 32 of the 128 x 64 block
constexpr int SC_TARGET_WGS = 256;  // one workgroup per CU
typedef void __attribute__((address_space(3))) sc_lds_void;

__global__ void __launch_bounds__(SC_WAVES * 64) scores_kernel(Geom g, int h, int t0, int nq, int tiles_per_wg,
                                                     const double* __restrict__ qbar,
                                                     const double* __restrict__ kbar,
                                                     unsigned* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) double qs[SC_QB * SC_LD];
  __shared__ __attribute__((aligned(1024))) double kt0[SC_KT];
  __shared__ __attribute__((aligned(1024))) double kt1[SC_KT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = blockIdx.y * SC_QB;
  const int nut = (g.T + 63) / 64;
  const int ut0 = blockIdx.x * tiles_per_wg, ut1 = min(nut, ut0 + tiles_per_wg);
  const double* qb = qbar + ((long long)h * g.T + t0) * D;
  const double* kb = kbar + (long long)h * g.T * D;
  // key tile ut into dst: wave w's copy j fills slots (8j + w) * 64 + lane,
  // that is row r = 2 (8j + w) + lane / 32, slot lane % 32
  auto stage = [&](int ut, double* dst) {
#pragma unroll
    for (int j = 0; j < 32 / SC_WAVES; ++j) {
      const int r = 2 * (SC_WAVES * j + wave) + (lane >> 5), slot = lane & 31;
      const double* src = kb + (long long)min(ut * 64 + r, g.T - 1) * D + 2 * (slot ^ (r & 15));
      __builtin_amdgcn_global_load_lds((const void*)src, (sc_lds_void*)(dst + (SC_WAVES * j + wave) * 128), 16, 0,
                                       0);
    }
  };
  if (ut0 < ut1) stage(ut0, kt0);
  {
    // the query block: thread row tid / 4, doubles 16 (tid % 4) .. +15
    const int r = tid >> 2, c0 = (tid & 3) * 16;
    const uint4* qsrc = (const uint4*)(qb + (long long)min(q0 + r, nq - 1) * D + c0);
    uint4 qv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[c] = qsrc[c];
#pragma unroll
    for (int c = 0; c < 8; ++c) *(uint4*)(qs + r * SC_LD + c0 + 2 * c) = qv[c];
  }
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  const int m = lane & 15, kq = lane >> 4;
  // keys of the previous tile, stored while the next one is multiplied:
  // pend[(i * 4 + r) * 2 + j] is query row wr + 16 i + 4 r + kq, key column
  // wc + 16 j + m (the f64 MFMA's output element r of lane l is row 4 r + l / 16)
  unsigned pend[16];
  int pend_ut = -1;
  auto flush = [&]() {
    if (pend_ut < 0) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int q = q0 + wr + 16 * i + 4 * r + kq;
          const int u = pend_ut * 64 + wc + 16 * j + m;
          if (q < nq && u < g.T) out[(long long)q * g.T + u] = pend[(i * 4 + r) * 2 + j];
        }
  };
  auto tile = [&](int ut, const double* cur, double* ahead) {
    // this tile's copies (issued a tile ago) and the stores of two tiles ago
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();  // ... in every wave; the previous tile's buffer is free
    if (ut + 1 < ut1) stage(ut + 1, ahead);
    flush();
    f64x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    // all 16 steps unrolled: with a loop the accumulators would be copied
    // out of and back into the matrix registers, draining the pipe, each trip
#pragma unroll
    for (int s4 = 0; s4 < D / 4; ++s4) {
      const int k = 4 * s4 + kq;
      const int slot = ((k >> 1) ^ m) * 2 + (k & 1);  // key rows wc + 16 i + m: row % 16 = m
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = qs[(wr + 16 * i + m) * SC_LD + k];
        b[i] = cur[(wc + 16 * i + m) * D + slot];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 2; ++j) pend[(i * 4 + r) * 2 + j] = f32_key((float)(acc[i][j][r] * 0.125));
    pend_ut = ut;
  };
  // the loop over the two buffers, unrolled so that every LDS read names
  // its buffer (and the compiler need not wait for copies into the other)
  for (int ut = ut0; ut < ut1; ut += 2) {
    tile(ut, kt0, kt1);
    if (ut + 1 < ut1) tile(ut + 1, kt1, kt0);
  }
  flush();
}

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_NW = TOPK_THREADS / 64;
constexpr int SELECT_CHUNK = 4096;     // query tiles scored per launch
constexpr int TOPK_MAX_ROUNDS = 32;    // T <= 32768
constexpr int TOPK_BINS = 4096;        // histogram bins per refinement level
constexpr int TOPK_CAND = 256;         // most keys in a bin that ends the narrowing
constexpr int TOPK_RANK_CHUNK = 2048;  // tie-group scores ranked per LDS pass (in the histogram)

// Exclusive prefix, in place, of the per-(round, wave) counts tab[0, nvalid)
// (round-major, so in tile order), by the first wave; entries past nvalid
// count as zero.
template <int N>
__device__ inline void table_scan(unsigned* tab, int nvalid) {
  constexpr int PER = (N + 63) / 64;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    unsigned v[PER], sum = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane * PER + j;
      v[j] = e < nvalid ? tab[e] : 0u;
      sum += v[j];
    }
    unsigned incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    unsigned run = incl - sum;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane * PER + j;
      if (e < N) tab[e] = run;
      run += v[j];
    }
  }
}

// A copy of x the compiler cannot see through: values derived from the keys
// are recomputed in each pass instead of being kept live in registers.
__device__ inline unsigned opaque(unsigned x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Workgroup min and max of (lo, hi) through per-wave slots w[0..2*NW); every
// thread gets the result. Barrier on entry and exit.
template <typename V>
__device__ inline void block_minmax(V& lo, V& hi, V* w) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const V ol = __shfl_xor(lo, off, 64), oh = __shfl_xor(hi, off, 64);
    lo = ol < lo ? ol : lo;
    hi = oh > hi ? oh : hi;
  }
  const int wave = threadIdx.x >> 6, j = threadIdx.x & (TOPK_NW - 1);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    w[wave] = lo;
    w[TOPK_NW + wave] = hi;
  }
  __syncthreads();
  // lane j of each group of 16 takes wave j's pair; the group reduces it
  lo = w[j];
  hi = w[TOPK_NW + j];
#pragma unroll
  for (int off = TOPK_NW / 2; off >= 1; off >>= 1) {
    const V ol = __shfl_xor(lo, off, 64), oh = __shfl_xor(hi, off, 64);
    lo = ol < lo ? ol : lo;
    hi = oh > hi ? oh : hi;
  }
  __syncthreads();
}

// The fp64 score of one key tile, recomputed as a single fixed-order chain
// of fused multiply-adds over channels 0..63 (the query row in LDS): equal
// rows give equal scores.
__device__ inline double exact_score(const double* qs, const double* __restrict__ krow) {
  double s = 0.0;
#pragma unroll 4
  for (int c = 0; c < D; c += 2) {
    const double2 b = *(const double2*)(krow + c);
    s = fma(qs[c], b.x, s);
    s = fma(qs[c + 1], b.y, s);
  }
  return s * 0.125;
}

// Per-row record of the top-k kernel for the resolve kernel: flag (1 when
// the tiles holding K* straddle the cut), K*, how many of them to keep, and
// how many there are.
constexpr int TOPK_INFO = 4;

// Keys of tiles u = i * 1024 + tid into kv[i]; bit i of vmask says u < T.
// The loads are unconditional (the tail repeats the last key).
template <int P>
__device__ inline unsigned topk_load(const unsigned* __restrict__ row, int T, unsigned (&kv)[P]) {
  unsigned vmask = 0u;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int u = i * TOPK_THREADS + (int)threadIdx.x;
    const bool ok = u < T;
    kv[i] = row[ok ? u : T - 1];
    vmask |= (ok ? 1u : 0u) << i;
  }
  return vmask;
}

// Tile u = i * 1024 + tid exists: whole rounds below PMIN - 1; else bit i of
// vmask, read through opaque() so that per-round tests are not kept live.
#define TOPK_VALID(i) ((i) < PMIN - 1 || ((opaque(vmask) >> (i)) & 1u))
// Round i is past the last one (uniform).
#define TOPK_SKIP(i) ((i) >= PMIN && (i) >= rounds)

// The kept tiles of one row, in ascending order, and its bitmap: lane i of
// each wave holds round i's kept count, then, after a scan, its output
// offset. Returns this thread's greatest unkept key (0 if none).
template <int PMIN, int P, typename Take>
__device__ inline unsigned topk_emit(const unsigned (&kv)[P], unsigned vmask, int rounds, int k, int nwords,
                                     unsigned* tab, int* __restrict__ selrow, unsigned* __restrict__ maskrow,
                                     Take take) {
  constexpr int NW = TOPK_NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long below_lanes = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  unsigned cntv = 0u;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    if (TOPK_SKIP(i)) continue;
    const unsigned c = (unsigned)__popcll(__ballot(take(i, opaque(kv[i]))));
    cntv = lane == i ? c : cntv;
  }
  if (lane < rounds) tab[lane * NW + wave] = cntv;
  __syncthreads();
  table_scan<P * NW>(tab, rounds * NW);
  __syncthreads();
  const unsigned basev = lane < rounds ? tab[lane * NW + wave] : 0u;
  unsigned maskv = 0u, below_key = 0u;
  const int utid = (int)opaque((unsigned)tid);  // tile indices recomputed, not held
#pragma unroll
  for (int i = 0; i < P; ++i) {
    if (TOPK_SKIP(i)) continue;
    const int u = i * TOPK_THREADS + utid;
    const unsigned x = opaque(kv[i]);
    const bool tk = take(i, x);
    const unsigned long long bt = __ballot(tk);
    // lanes 2i and 2i+1 hold this round's two bitmap words
    maskv = lane == 2 * i ? (unsigned)bt : lane == 2 * i + 1 ? (unsigned)(bt >> 32) : maskv;
    const unsigned pos = (unsigned)__builtin_amdgcn_readlane((int)basev, i) + (unsigned)__popcll(bt & below_lanes);
    if (tk && pos < (unsigned)k) selrow[pos] = u;
    below_key = TOPK_VALID(i) && !tk && x > below_key ? x : below_key;
  }
  const int word = (lane >> 1) * (TOPK_THREADS / 32) + wave * 2 + (lane & 1);
  if (lane < 2 * rounds && word < nwords) maskrow[word] = maskv;
  return below_key;
}

// grid (nq), block 1024: top-k of query tile t0+blockIdx.x of head h, from
// its row of fp32 order keys. Thread tid holds the keys of tiles
// u = i * 1024 + tid (round i); the rounds number PMIN..P, so rounds below
// PMIN - 1 are whole.
//
// The kept set is the k tiles ranked first by (fp64 score descending, tile
// index ascending). Rounding to fp32 preserves order, so every tile whose
// key exceeds the key K* of the k-th ranked tile is kept and every tile
// below it is not; only the tiles whose key equals K* can rank differently
// in fp64. K* is found by narrowing a key interval with 4096-bin
// histograms (bins uniform in score on the first level, in key bits after
// that) until the bin holding the k-th key has at most 256 keys, which are
// compared pairwise in LDS, or a single key value. When the tiles with key
// K* are all kept (the usual case) this kernel writes the row; when they
// straddle the cut it records K* for topk_resolve_kernel instead.
template <int PMIN, int P>
__global__ void __launch_bounds__(TOPK_THREADS) __attribute__((amdgpu_waves_per_eu(8, 8)))
topk_kernel(Geom g, int h, int t0, int k, const unsigned* __restrict__ keys, unsigned* __restrict__ info,
            int* __restrict__ sel, unsigned* __restrict__ selmask, double* __restrict__ gap) {
  static_assert(P <= 32 && 2 * P <= 64, "a lane per round and a mask bit per round");
  constexpr int NW = TOPK_NW, BPT = TOPK_BINS / TOPK_THREADS;
  __shared__ __attribute__((aligned(16))) unsigned hist[TOPK_BINS];
  __shared__ unsigned tab[P * NW];
  __shared__ unsigned cand[TOPK_CAND];
  __shared__ unsigned wsum[NW];
  __shared__ unsigned wred_u[2 * NW];
  __shared__ unsigned sh_bin, sh_want, sh_cnt, sh_nc, sh_kstar, sh_gt, sh_ge, sh_below;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = t0 + blockIdx.x;
  const int T = g.T;
  const int nwords = (T + 31) / 32;
  const int rounds = (T + TOPK_THREADS - 1) / TOPK_THREADS;
  const unsigned* row = keys + (long long)blockIdx.x * T;
  int* selrow = sel + ((long long)h * T + t) * k;
  unsigned* maskrow = selmask + ((long long)h * T + t) * nwords;
  const unsigned long long below_lanes = lane == 0 ? 0ull : (~0ull >> (64 - lane));

  unsigned kv[P];
  const unsigned vmask = topk_load(row, T, kv);

  if (k == 0 || k == T) {  // nothing to rank
    if (tid == 0) info[blockIdx.x * TOPK_INFO] = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int u = i * TOPK_THREADS + tid;
      if (TOPK_VALID(i) && k == T) selrow[u] = u;
    }
    for (int w = tid; w < nwords; w += TOPK_THREADS) {
      unsigned m = 0u;
      if (k == T) m = (w == nwords - 1 && (T & 31)) ? ((1u << (T & 31)) - 1u) : 0xFFFFFFFFu;
      maskrow[w] = m;
    }
    if (gap && tid == 0) gap[(long long)h * T + t] = __longlong_as_double(0x7FF0000000000000ll);
    return;
  }

  unsigned lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    if (TOPK_SKIP(i)) continue;  // uniform
    const bool v = TOPK_VALID(i);
    lo = v && kv[i] < lo ? kv[i] : lo;
    hi = v && kv[i] > hi ? kv[i] : hi;
  }
  block_minmax(lo, hi, wred_u);

  unsigned want = (unsigned)k, cnt = (unsigned)T;
  bool gathered = false;
  // One narrowing step over the keys in [lo, hi] under the monotone bin map
  // `digit`: the histogram, the bin holding the want-th key from the top,
  // and then either that bin's keys gathered (at most TOPK_CAND) or its key
  // range as the new [lo, hi].
  auto narrow = [&](auto digit) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) hist[j * TOPK_THREADS + tid] = 0u;
    if (tid == 0) sh_nc = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (TOPK_SKIP(i)) continue;
      const unsigned x = opaque(kv[i]);
      if (TOPK_VALID(i) & (x >= lo) & (x <= hi)) atomicAdd(&hist[digit(x)], 1u);
    }
    __syncthreads();
    // thread tid owns bins 4095-4tid .. 4092-4tid (descending order)
    unsigned c[BPT], sum = 0u;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = hist[TOPK_BINS - 1 - BPT * tid - j];
      sum += c[j];
    }
    unsigned incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned above = incl - sum;
    for (int w = 0; w < wave; ++w) above += wsum[w];
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (above < want && want <= above + c[j]) {
        sh_bin = TOPK_BINS - 1 - BPT * tid - j;
        sh_want = want - above;
        sh_cnt = c[j];
      }
      above += c[j];
    }
    __syncthreads();
    const unsigned bin = sh_bin;
    want = sh_want;
    cnt = sh_cnt;
    if (cnt <= (unsigned)TOPK_CAND) {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        if (TOPK_SKIP(i)) continue;
        const unsigned x = opaque(kv[i]);
        const bool inb = TOPK_VALID(i) & (x >= lo) & (x <= hi) & (digit(x) == bin);
        const unsigned long long bi = __ballot(inb);
        if (bi) {
          unsigned base = 0u;
          if (lane == 0) base = atomicAdd(&sh_nc, (unsigned)__popcll(bi));
          base = (unsigned)__shfl(base, 0, 64);
          if (inb) cand[base + (unsigned)__popcll(bi & below_lanes)] = x;
        }
      }
      gathered = true;
      __syncthreads();
    } else {
      unsigned blo = 0xFFFFFFFFu, bhi = 0u;
#pragma unroll
      for (int i = 0; i < P; ++i) {
        if (TOPK_SKIP(i)) continue;
        const unsigned x = opaque(kv[i]);
        const bool inb = TOPK_VALID(i) & (x >= lo) & (x <= hi) & (digit(x) == bin);
        blo = inb && x < blo ? x : blo;
        bhi = inb && x > bhi ? x : bhi;
      }
      block_minmax(blo, bhi, wred_u);
      lo = blo;
      hi = bhi;
    }
  };
  if (lo != hi && cnt > (unsigned)TOPK_CAND) {
    // first step: bins uniform in score over [lo, hi], when that span and
    // its inverse are finite fp32 numbers
    const float flo = key_f32(lo), fspan = key_f32(hi) - flo, inv = (float)TOPK_BINS / fspan;
    if (fspan > 0.0f && fspan <= 3.0e38f && inv <= 3.0e38f)
      narrow([&](unsigned x) -> unsigned {
        const float y = (key_f32(x) - flo) * inv;
        return y < (float)(TOPK_BINS - 1) ? (unsigned)y : (unsigned)(TOPK_BINS - 1);
      });
  }
  // then bins uniform in key bits, 12 bits per step
  while (!gathered && lo != hi && cnt > (unsigned)TOPK_CAND) {
    const unsigned klo = lo;
    const int top = 32 - __clz((int)(hi - lo));
    const int sh = top > 12 ? top - 12 : 0;
    narrow([&](unsigned x) -> unsigned { return (x - klo) >> sh; });
  }
  if (!gathered && lo != hi) {  // few keys from the start: all are candidates
    if (tid == 0) sh_nc = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (TOPK_SKIP(i)) continue;
      const bool inb = TOPK_VALID(i);
      const unsigned long long bi = __ballot(inb);
      if (bi) {
        unsigned base = 0u;
        if (lane == 0) base = atomicAdd(&sh_nc, (unsigned)__popcll(bi));
        base = (unsigned)__shfl(base, 0, 64);
        if (inb) cand[base + (unsigned)__popcll(bi & below_lanes)] = kv[i];
      }
    }
    gathered = true;
    __syncthreads();
  }

  // K*, and how many keys of the final interval lie above it (gt) and at or
  // above it (ge): gt < want <= ge
  unsigned kstar, gt, ge;
  if (gathered) {
    if (tid < (int)cnt) {
      const unsigned kc = cand[tid];
      unsigned a = 0u, b = 0u;
      for (int j = 0; j < (int)cnt; ++j) {
        const unsigned kj = cand[j];
        a += kj > kc ? 1u : 0u;
        b += kj >= kc ? 1u : 0u;
      }
      if (a < want && want <= b) {  // every thread holding K* writes the same
        sh_kstar = kc;
        sh_gt = a;
        sh_ge = b;
      }
    }
    if (tid == 0) sh_below = 0u;
    __syncthreads();
    kstar = sh_kstar;
    gt = sh_gt;
    ge = sh_ge;
    // the greatest candidate key below K*, if any (read after a barrier)
    if (tid < (int)cnt && cand[tid] < kstar) atomicMax(&sh_below, cand[tid]);
  } else {  // one key value left
    kstar = lo;
    gt = 0u;
    ge = cnt;
  }
  if (ge > want) {  // the tiles with key K* straddle the cut
    if (tid == 0) {
      info[blockIdx.x * TOPK_INFO] = 1u;
      info[blockIdx.x * TOPK_INFO + 1] = kstar;
      info[blockIdx.x * TOPK_INFO + 2] = want - gt;
      info[blockIdx.x * TOPK_INFO + 3] = ge - gt;
    }
    return;
  }
  if (tid == 0) info[blockIdx.x * TOPK_INFO] = 0u;

  // every key at or above K* is kept
  unsigned below = topk_emit<PMIN, P>(kv, vmask, rounds, k, nwords, tab, selrow, maskrow,
                                      [&](int i, unsigned x) -> bool { return TOPK_VALID(i) & (x >= kstar); });
  if (gap) {
    // Relative gap between the k-th and (k+1)-th ranked scores from their
    // fp32-rounded values, K* and the greatest unkept key (different keys:
    // within 1.2e-7 of the fp64 gap)
    if (gathered && ge < cnt) {
      below = sh_below;
    } else {  // no candidate below K*: over all keys
      unsigned dummy = 0u;
      block_minmax(dummy, below, wred_u);
    }
    if (tid == 0) {
      const double st = (double)key_f32(kstar), sb = (double)key_f32(below);
      const double den = fmax(fmax(fabs(st), fabs(sb)), 1e-300);
      gap[(long long)h * T + t] = fabs(st - sb) / den;
    }
  }
}

// grid (nq), block 1024: the rows that topk_kernel left, those where the
// ng tiles with key K* straddle the cut. Of those tiles the gwant first by
// (fp64 score descending, tile index ascending) are kept: their fp64 scores
// are recomputed, and ranked by tile index alone when all are equal, else
// pairwise in LDS chunks (a running count per tile in this row's rank
// area). Other rows return at once.
template <int PMIN, int P>
__global__ void __launch_bounds__(TOPK_THREADS) topk_resolve_kernel(
    Geom g, int h, int t0, int k, const unsigned* __restrict__ keys, const unsigned* __restrict__ info,
    unsigned* __restrict__ ranks, const double* __restrict__ qbar, const double* __restrict__ kbar,
    int* __restrict__ sel, unsigned* __restrict__ selmask, double* __restrict__ gap) {
  constexpr int NW = TOPK_NW;
  if (info[blockIdx.x * TOPK_INFO] == 0u) return;
  const unsigned kstar = info[blockIdx.x * TOPK_INFO + 1], gwant = info[blockIdx.x * TOPK_INFO + 2];
  const unsigned ng = info[blockIdx.x * TOPK_INFO + 3];
  __shared__ __attribute__((aligned(16))) double chunk[TOPK_RANK_CHUNK];
  __shared__ unsigned tab[P * NW];
  __shared__ unsigned gbits[P * TOPK_THREADS / 32];
  __shared__ double wred_d[2 * NW];
  __shared__ double sh_st, sh_sb;
  __shared__ double qs[D];  // the query tile's mean query
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = t0 + blockIdx.x;
  const int T = g.T;
  const int nwords = (T + 31) / 32;
  const int rounds = (T + TOPK_THREADS - 1) / TOPK_THREADS;
  const unsigned* row = keys + (long long)blockIdx.x * T;
  unsigned* rank_row = ranks + (long long)blockIdx.x * T;
  int* selrow = sel + ((long long)h * T + t) * k;
  unsigned* maskrow = selmask + ((long long)h * T + t) * nwords;
  const double* kb = kbar + (long long)h * T * D;
  const unsigned long long below_lanes = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  if (tid < D) qs[tid] = qbar[((long long)h * T + t) * D + tid];

  unsigned kv[P];
  const unsigned vmask = topk_load(row, T, kv);
  // gm: this thread's rounds holding K*; pos: a member's rank by tile index
  unsigned gm = 0u;
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (!TOPK_SKIP(i) && TOPK_VALID(i) && kv[i] == kstar) gm |= 1u << i;
  for (int w = tid; w < P * TOPK_THREADS / 32; w += TOPK_THREADS) gbits[w] = 0u;
  for (int i = 0; i < rounds; ++i) {
    const unsigned long long be = __ballot((gm >> i) & 1u);
    if (lane == 0) tab[i * NW + wave] = (unsigned)__popcll(be);
  }
  __syncthreads();
  table_scan<P * NW>(tab, rounds * NW);
  __syncthreads();
  double smin = __longlong_as_double(0x7FF0000000000000ll), smax = -smin;
  for (unsigned b = gm; b; b &= b - 1u) {
    const int u = (__ffs((int)b) - 1) * TOPK_THREADS + tid;
    const double s = exact_score(qs, kb + (long long)u * D);
    smin = s < smin ? s : smin;
    smax = s > smax ? s : smax;
  }
  block_minmax(smin, smax, wred_d);
  const bool all_equal = smin == smax;  // then the rank is the index rank
  for (unsigned c0 = 0; c0 < (all_equal ? 0u : ng); c0 += TOPK_RANK_CHUNK) {
    // the scores of group positions [c0, c0 + cn) into LDS; then every
    // member adds the chunk's members ranked before it to its running count
    const unsigned cn = min((unsigned)TOPK_RANK_CHUNK, ng - c0);
    __syncthreads();
    for (int i = 0; i < rounds; ++i) {
      const bool eq = (gm >> i) & 1u;
      const unsigned long long be = __ballot(eq);
      const unsigned pos = tab[i * NW + wave] + (unsigned)__popcll(be & below_lanes);
      if (eq && pos >= c0 && pos < c0 + cn)
        chunk[pos - c0] = exact_score(qs, kb + (long long)(i * TOPK_THREADS + tid) * D);
    }
    __syncthreads();
    for (int i = 0; i < rounds; ++i) {
      const bool eq = (gm >> i) & 1u;
      const unsigned long long be = __ballot(eq);
      const unsigned pos = tab[i * NW + wave] + (unsigned)__popcll(be & below_lanes);
      if (eq) {
        const int u = i * TOPK_THREADS + tid;
        const double s = exact_score(qs, kb + (long long)u * D);
        unsigned r = 0u;
        for (unsigned j = 0; j < cn; ++j) {
          const double sj = chunk[j];
          r += (sj > s || (sj == s && c0 + j < pos)) ? 1u : 0u;
        }
        rank_row[u] = c0 == 0 ? r : rank_row[u] + r;
      }
    }
  }
  for (int i = 0; i < rounds; ++i) {
    const bool eq = (gm >> i) & 1u;
    const unsigned long long be = __ballot(eq);
    const unsigned pos = tab[i * NW + wave] + (unsigned)__popcll(be & below_lanes);
    const int u = i * TOPK_THREADS + tid;
    const unsigned r = all_equal ? pos : (eq ? rank_row[u] : 0u);
    if (eq && r < gwant) atomicOr(&gbits[u >> 5], 1u << (u & 31));
    // the k-th and (k+1)-th ranked scores are the group's gwant-th and
    // (gwant+1)-th (ng > gwant)
    if (gap && eq && (r == gwant - 1u || r == gwant)) {
      const double sc = all_equal ? smin : exact_score(qs, kb + (long long)u * D);
      if (r == gwant - 1u) sh_st = sc;
      else sh_sb = sc;
    }
  }
  __syncthreads();
  topk_emit<PMIN, P>(kv, vmask, rounds, k, nwords, tab, selrow, maskrow, [&](int i, unsigned x) -> bool {
    const int u = i * TOPK_THREADS + tid;
    return TOPK_VALID(i) & ((x > kstar) | ((x == kstar) & (((gbits[u >> 5] >> (u & 31)) & 1u) != 0u)));
  });
  if (gap && tid == 0) {
    const double st = sh_st, sb = sh_sb;
    const double den = fmax(fmax(fabs(st), fabs(sb)), 1e-300);
    gap[(long long)h * T + t] = fabs(st - sb) / den;
  }
}
#undef TOPK_VALID
#undef TOPK_SKIP

size_t select_chunk(const Geom& g) { return (size_t)(g.T < SELECT_CHUNK ? g.T : SELECT_CHUNK); }

size_t select_workspace_bytes(const Geom& g) {
  return (size_t)g.H * g.T * D * sizeof(double) + 2 * select_chunk(g) * (size_t)g.T * sizeof(unsigned) +
         select_chunk(g) * TOPK_INFO * sizeof(unsigned);
}

// Workspace: qbar [H][T][64] fp64, the score keys [chunk][T] u32, the rank
// area [chunk][T] u32 (touched only for tie groups that straddle the cut),
// then the per-row records [chunk][4] u32.
hipError_t launch_select(const Geom& g, int k, const u16* Q, const double* kbar, int* sel,
                         unsigned* selmask, double* gap, void* ws, hipStream_t s) {
  double* qbar = (double*)ws;
  const int chunk = (int)select_chunk(g);
  unsigned* keys = (unsigned*)(qbar + (size_t)g.H * g.T * D);
  unsigned* ranks = keys + (size_t)chunk * g.T;
  unsigned* info = ranks + (size_t)chunk * g.T;
  const int rounds = (g.T + TOPK_THREADS - 1) / TOPK_THREADS;
  auto topk = rounds <= 4    ? topk_kernel<1, 4>
              : rounds <= 16 ? topk_kernel<5, 16>
              : rounds <= 25 ? topk_kernel<17, 25>
                             : topk_kernel<26, TOPK_MAX_ROUNDS>;
  auto resolve = rounds <= 4    ? topk_resolve_kernel<1, 4>
                 : rounds <= 16 ? topk_resolve_kernel<5, 16>
                 : rounds <= 25 ? topk_resolve_kernel<17, 25>
                                : topk_resolve_kernel<26, TOPK_MAX_ROUNDS>;
  hipLaunchKernelGGL(qbar_kernel, dim3((g.T + 3) / 4, g.H), dim3(256), 0, s, g, Q, qbar);
  for (int h = 0; h < g.H; ++h) {
    for (int t0 = 0; t0 < g.T; t0 += chunk) {
      const int nq = g.T - t0 < chunk ? g.T - t0 : chunk;
      if (k > 0 && k < g.T) {
        // about one workgroup per CU, each over an equal range of key tiles
        const int nut = (g.T + 63) / 64, nqb = (nq + SC_QB - 1) / SC_QB;
        const int per = (nut * nqb + SC_TARGET_WGS - 1) / SC_TARGET_WGS;
        hipLaunchKernelGGL(scores_kernel, dim3((nut + per - 1) / per, nqb), dim3(SC_WAVES * 64), 0, s, g, h, t0, nq,
                           per, qbar, kbar, keys);
      }
      hipLaunchKernelGGL(topk, dim3(nq), dim3(TOPK_THREADS), 0, s, g, h, t0, k, keys, info, sel, selmask,
                         gap);
      if (k > 0 && k < g.T)
        hipLaunchKernelGGL(resolve, dim3(nq), dim3(TOPK_THREADS), 0, s, g, h, t0, k, keys, info, ranks,
                           qbar, kbar, sel, selmask, gap);
    }
  }
  return hipGetLastError();
}

}  // namespace zebra
