// Tile selector for gfx950: fp64 tile scores and exact top-k.
//
// Zebra3D pages, "Linear-centered stages plus tile-sparse stages": for each
// query tile the selector keeps a key-tile fraction 1 - y. A tile's score is
// the mean query of the query tile dotted with the key tile's mean key,
// divided by sqrt(64), over all key tiles of all frames. Ties go to the lower
// tile index. Scores are float64 on both sides of the parity check so that
// the integer decision (kept or not) is taken in the same precision.
//
// Three kernels: qbar (mean patch query per tile, exact fp64 sums),
// scores (a 64x64-blocked fp64 product qbar . kbar^T into a workspace
// chunk) and topk (one 1024-thread workgroup per query tile: the k-th key
// found by histogram range narrowing over order-preserving 64-bit keys, then
// an ascending compaction from one scan of per-wave counts that also writes
// the bitmap).
#include "common.hpp"

namespace zebra {

__device__ inline long long tile_token_s(const Geom& g, int f, int tl, int s) {
  const int a = tl / g.tc, b = tl - a * g.tc;
  const int tw = tile_w(g, tl);
  const int r = TILE * a + s / tw, c = TILE * b + s % tw;
  return (long long)f * g.tok_pf + g.S + (long long)r * g.C + c;
}

// grid (T, H), block 64: qbar[h][t][d] = mean over tile t's patch queries.
__global__ void __launch_bounds__(64) qbar_kernel(Geom g, const u16* __restrict__ Q,
                                                  double* __restrict__ qbar) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int f = t / g.tpf, tl = t - f * g.tpf;
  const int n = tile_n(g, tl);
  double s = 0.0;
  for (int i = 0; i < n; ++i) {
    const long long tok = tile_token_s(g, f, tl, i);
    s += (double)bf2f(Q[(tok * g.H + h) * D + d]);
  }
  qbar[((long long)h * g.T + t) * D + d] = s / n;
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Scores of query tiles [t0, t0+nq) of head h against every key tile:
// out[tq][u] = (sum_d qbar[t0+tq][d] * kbar[u][d]) * 0.125, on the fp64
// matrix cores. grid (ceil(T/64), ceil(nq/64)), block 256: a 64 x 64 tile,
// wave w its 32 x 32 quarter (rows 32 (w >> 1), columns 32 (w & 1)) as 2 x 2
// 16x16x4 MFMA tiles over the 16 steps of 4 channels. Both operands sit in
// LDS row-major with a row stride of 68 doubles, so that a step's 64 lane
// reads (16 rows x 4 channels) cover the 64 banks twice.
constexpr int SC_LD = D + 4;
__global__ void __launch_bounds__(256) scores_kernel(Geom g, int h, int t0, int nq,
                                                     const double* __restrict__ qbar,
                                                     const double* __restrict__ kbar,
                                                     double* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) double qs[64 * SC_LD];
  __shared__ __attribute__((aligned(16))) double ks[64 * SC_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u0 = blockIdx.x * 64, q0 = blockIdx.y * 64;
  const double* qb = qbar + ((long long)h * g.T + t0) * D;
  const double* kb = kbar + (long long)h * g.T * D;
  {
    // thread: row tid / 4, doubles 16 (tid % 4) .. +15 of both tiles; all
    // sixteen 16-byte loads are issued before the first LDS write. Rows past
    // the end repeat the last row (their outputs are not stored).
    const int r = tid >> 2, c0 = (tid & 3) * 16;
    const uint4* qsrc = (const uint4*)(qb + (long long)min(q0 + r, nq - 1) * D + c0);
    const uint4* ksrc = (const uint4*)(kb + (long long)min(u0 + r, g.T - 1) * D + c0);
    uint4 qv[8], kv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      qv[c] = qsrc[c];
      kv[c] = ksrc[c];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      *(uint4*)(qs + r * SC_LD + c0 + 2 * c) = qv[c];
      *(uint4*)(ks + r * SC_LD + c0 + 2 * c) = kv[c];
    }
  }
  __syncthreads();
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  const int m = lane & 15, kq = lane >> 4;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int s4 = 0; s4 < D / 4; ++s4) {
    const int k = 4 * s4 + kq;
    double a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = qs[(wr + 16 * i + m) * SC_LD + k];
      b[i] = ks[(wc + 16 * i + m) * SC_LD + k];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  // acc[i][j][r]: query row wr + 16 i + 4 r + kq, key column wc + 16 j + m
  // (the f64 MFMA's output element r of lane l is row 4 r + l / 16)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = q0 + wr + 16 * i + 4 * r + kq;
      if (q >= nq) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int u = u0 + wc + 16 * j + m;
        if (u < g.T) out[(long long)q * g.T + u] = acc[i][j][r] * 0.125;
      }
    }
}

constexpr int TOPK_THREADS = 1024;
constexpr int SELECT_CHUNK = 4096;  // query tiles scored per launch
constexpr int TOPK_PER_THREAD = 32;  // T <= 32768

__device__ inline unsigned long long score_key(double s) {
  if (s == 0.0) s = 0.0;  // -0 and +0 compare equal
  const unsigned long long b = (unsigned long long)__double_as_longlong(s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ inline double key_score(unsigned long long k) {
  const unsigned long long b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}

constexpr int TOPK_BINS = 4096;  // histogram bins per refinement level
constexpr int TOPK_CAND = 256;   // candidates ranked pairwise in LDS

// Exclusive prefix, in place, of the per-(round, wave) counts tab[0, nvalid)
// (round-major, so in tile order), by the first wave; entries past nvalid
// (rounds past the last tile) count as zero.
__device__ inline void table_scan(unsigned* tab, int nvalid) {
  constexpr int N = TOPK_PER_THREAD * (TOPK_THREADS / 64), PER = N / 64;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    unsigned v[PER], sum = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      v[j] = lane * PER + j < nvalid ? tab[lane * PER + j] : 0u;
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
      tab[lane * PER + j] = run;
      run += v[j];
    }
  }
}

// A copy of x the compiler cannot see through: bin maps are recomputed in
// each pass instead of being kept live across passes in registers.
__device__ inline double opaque(double x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Workgroup min and max (by comparisons: the scores hold no NaN, and fmin
// would make canonicalised copies of them) of the scores (lo, hi) through per-wave slots w[0..31];
// every thread gets the result. Barrier on entry and exit.
__device__ inline void block_minmax(double& lo, double& hi, double* w) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ol = __shfl_xor(lo, off, 64), oh = __shfl_xor(hi, off, 64);
    lo = ol < lo ? ol : lo;
    hi = oh > hi ? oh : hi;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    w[wave] = lo;
    w[16 + wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TOPK_THREADS / 64; ++j) {
    lo = w[j] < lo ? w[j] : lo;
    hi = w[16 + j] > hi ? w[16 + j] : hi;
  }
  __syncthreads();
}

// grid (nq), block 1024: top-k of query tile t0+blockIdx.x of head h.
// Thread tid holds the scores of tiles u = i * 1024 + tid (round i).
//
// The kept set is every (score, u) ranked at or above the k-th in the order
// (score descending, tile index ascending). That k-th pair is found by
// narrowing a score interval: a 4096-bin histogram of the interval (bins
// uniform in score on the first level, in the order-preserving key bits
// after that), and the bin holding the k-th score becomes the next
// interval, until the bin holds at most 256 scores, which are ranked
// pairwise in LDS, or one score value, whose tie is cut by tile index. Every
// bin map is monotone, so bins are score intervals and a key in a higher bin
// is strictly greater. Keys above the chosen bin are counted per (round,
// wave) as each level is scanned; with the ranked candidates this gives
// every kept key's output position, and one last pass writes the list and
// the bitmap.
__global__ void __launch_bounds__(TOPK_THREADS) topk_kernel(Geom g, int h, int t0, int k,
                                                            const double* __restrict__ scores,
                                                            int* __restrict__ sel,
                                                            unsigned* __restrict__ selmask,
                                                            double* __restrict__ gap) {
  constexpr int NW = TOPK_THREADS / 64, BPT = TOPK_BINS / TOPK_THREADS;
  __shared__ unsigned hist[TOPK_BINS];
  __shared__ unsigned wsum[NW];
  __shared__ unsigned take_tab[TOPK_PER_THREAD * NW];  // kept keys per (round, wave)
  __shared__ unsigned eq_tab[TOPK_PER_THREAD * NW];
  __shared__ double cand_s[TOPK_CAND];
  __shared__ int cand_u[TOPK_CAND];
  __shared__ double wred[2 * NW];
  __shared__ unsigned sh_bin, sh_want, sh_cnt, sh_nc;
  __shared__ double sh_st;
  __shared__ int sh_ut;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = t0 + blockIdx.x;
  const int T = g.T;
  const int nwords = (T + 31) / 32;
  const int rounds = (T + TOPK_THREADS - 1) / TOPK_THREADS;
  const int last = rounds - 1;
  const bool tail_ok = tid < T - last * TOPK_THREADS;  // valid in the last round
  const double* row = scores + (long long)blockIdx.x * T;
  int* selrow = sel + ((long long)h * T + t) * k;
  unsigned* maskrow = selmask + ((long long)h * T + t) * nwords;
  const unsigned long long below_lanes = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#define TOPK_VALID(i) ((i) < last || tail_ok)

  double sc[TOPK_PER_THREAD];
#pragma unroll
  for (int i = 0; i < TOPK_PER_THREAD; ++i) {
    const int u = i * TOPK_THREADS + tid;
    sc[i] = (u < T) ? row[u] : 0.0;
  }

  if (k == 0 || k == T) {  // nothing to rank
#pragma unroll
    for (int i = 0; i < TOPK_PER_THREAD; ++i) {
      const int u = i * TOPK_THREADS + tid;
      if (u < T && k == T) selrow[u] = u;
    }
    for (int w = tid; w < nwords; w += TOPK_THREADS) {
      unsigned m = 0u;
      if (k == T) m = (w == nwords - 1 && (T & 31)) ? ((1u << (T & 31)) - 1u) : 0xFFFFFFFFu;
      maskrow[w] = m;
    }
    if (gap && tid == 0) gap[(long long)h * T + t] = __longlong_as_double(0x7FF0000000000000ll);
    return;
  }

  if (tid < TOPK_PER_THREAD * NW) take_tab[tid] = 0u;
  double lo = __longlong_as_double(0x7FF0000000000000ll), hi = -lo;
#pragma unroll
  for (int i = 0; i < TOPK_PER_THREAD; ++i) {
    if (i >= rounds) continue;  // uniform
    if (TOPK_VALID(i)) {
      lo = sc[i] < lo ? sc[i] : lo;
      hi = sc[i] > hi ? sc[i] : hi;
    }
  }
  block_minmax(lo, hi, wred);

  unsigned want = (unsigned)k, cnt = (unsigned)T;
  bool gathered = false;
  // One narrowing step over the scores in [lo, hi] (all scores when `all`)
  // under the monotone bin map `digit`: histogram, the bin holding the
  // want-th score, per-(round, wave) counts of the scores above that bin,
  // and then either the bin's scores gathered as candidates (at most
  // TOPK_CAND) or the bin's interval as the new [lo, hi].
  auto narrow = [&](auto digit, bool all) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) hist[j * TOPK_THREADS + tid] = 0u;
    if (tid == 0) sh_nc = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TOPK_PER_THREAD; ++i) {
      if (i >= rounds) continue;
      if (TOPK_VALID(i) && (all || (sc[i] >= lo && sc[i] <= hi))) atomicAdd(&hist[digit(opaque(sc[i]))], 1u);
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
    const bool gather = cnt <= (unsigned)TOPK_CAND;
    double blo = __longlong_as_double(0x7FF0000000000000ll), bhi = -blo;
#pragma unroll
    for (int i = 0; i < TOPK_PER_THREAD; ++i) {
      if (i >= rounds) continue;
      const int u = i * TOPK_THREADS + tid;
      const bool inr = TOPK_VALID(i) && (all || (sc[i] >= lo && sc[i] <= hi));
      const unsigned d = inr ? digit(opaque(sc[i])) : 0u;
      const unsigned long long ba = __ballot(inr && d > bin);
      if (lane == 0) take_tab[i * NW + wave] += (unsigned)__popcll(ba);
      const bool inb = inr && d == bin;
      if (gather) {
        const unsigned long long bi = __ballot(inb);
        if (bi) {
          unsigned base = 0u;
          if (lane == 0) base = atomicAdd(&sh_nc, (unsigned)__popcll(bi));
          base = (unsigned)__shfl(base, 0, 64);
          if (inb) {
            const unsigned slot = base + (unsigned)__popcll(bi & below_lanes);
            cand_s[slot] = sc[i];
            cand_u[slot] = u;
          }
        }
      } else if (inb) {
        blo = sc[i] < blo ? sc[i] : blo;
        bhi = sc[i] > bhi ? sc[i] : bhi;
      }
    }
    if (gather) {
      gathered = true;
      __syncthreads();
    } else {
      block_minmax(blo, bhi, wred);
      lo = blo;
      hi = bhi;
    }
  };
  if (lo != hi && cnt > (unsigned)TOPK_CAND) {
    // first step: bins uniform in score, when the span is a normal number
    const double fspan = hi - lo;
    const double inv = (double)TOPK_BINS / fspan;
    if (fspan > 1e-300 && fspan < 1e300 && inv < 1e300) {
      const double flo = lo;
      narrow(
          [&](double x) -> unsigned {
            const double y = (x - flo) * inv;
            return y < (double)(TOPK_BINS - 1) ? (unsigned)y : (unsigned)(TOPK_BINS - 1);
          },
          true);
    }
  }
  // then bins uniform in key bits, 12 bits per step
  while (!gathered && lo != hi && cnt > (unsigned)TOPK_CAND) {
    const unsigned long long klo = score_key(lo), span = score_key(hi) - klo;
    const int top = 64 - __clzll((long long)span);
    const int sh = top > 12 ? top - 12 : 0;
    narrow([&](double x) -> unsigned { return (unsigned)((score_key(x) - klo) >> sh); }, false);
  }

  // the k-th pair (st, ut) and the kept keys of the final bin
  if (gathered || (lo != hi && cnt <= (unsigned)TOPK_CAND)) {
    if (!gathered) {  // few scores from the start: all are candidates
      if (tid == 0) sh_nc = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TOPK_PER_THREAD; ++i) {
        if (i >= rounds) continue;
        const bool inb = TOPK_VALID(i);
        const unsigned long long bi = __ballot(inb);
        if (bi) {
          unsigned base = 0u;
          if (lane == 0) base = atomicAdd(&sh_nc, (unsigned)__popcll(bi));
          base = (unsigned)__shfl(base, 0, 64);
          if (inb) {
            const unsigned slot = base + (unsigned)__popcll(bi & below_lanes);
            cand_s[slot] = sc[i];
            cand_u[slot] = i * TOPK_THREADS + tid;
          }
        }
      }
      __syncthreads();
    }
    if (tid < (int)cnt) {
      const double sc_c = cand_s[tid];
      const int uc = cand_u[tid];
      unsigned rank = 0u;
      for (int j = 0; j < (int)cnt; ++j) {
        const double sj = cand_s[j];
        rank += (sj > sc_c || (sj == sc_c && cand_u[j] < uc)) ? 1u : 0u;
      }
      if (rank == want - 1u) {
        sh_st = sc_c;
        sh_ut = uc;
      }
      if (rank < want) atomicAdd(&take_tab[(uc / TOPK_THREADS) * NW + (uc % TOPK_THREADS) / 64], 1u);
    }
  } else {
    // one score value (lo == hi) in the final interval: keep the want
    // smallest tile indices holding it
#pragma unroll
    for (int i = 0; i < TOPK_PER_THREAD; ++i) {
      if (i >= rounds) continue;
      const unsigned long long be = __ballot(TOPK_VALID(i) && sc[i] == lo);
      if (lane == 0) eq_tab[i * NW + wave] = (unsigned)__popcll(be);
    }
    __syncthreads();
    table_scan(eq_tab, rounds * NW);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TOPK_PER_THREAD; ++i) {
      if (i >= rounds) continue;
      const bool eq = TOPK_VALID(i) && sc[i] == lo;
      const unsigned long long be = __ballot(eq);
      const unsigned r = eq_tab[i * NW + wave] + (unsigned)__popcll(be & below_lanes);
      const unsigned long long bk = __ballot(eq && r < want);
      if (lane == 0) take_tab[i * NW + wave] += (unsigned)__popcll(bk);
      if (eq && r == want - 1u) {
        sh_st = lo;
        sh_ut = i * TOPK_THREADS + tid;
      }
    }
  }
  __syncthreads();
  table_scan(take_tab, rounds * NW);
  __syncthreads();
  const double st = sh_st;
  const int ut = sh_ut;

  // kept tiles in ascending order, and the bitmap
  double below_max = -__longlong_as_double(0x7FF0000000000000ll);
#pragma unroll
  for (int i = 0; i < TOPK_PER_THREAD; ++i) {
    if (i >= rounds) continue;
    const int u = i * TOPK_THREADS + tid;
    const bool v = TOPK_VALID(i);
    const bool take = v && (sc[i] > st || (sc[i] == st && u <= ut));
    const unsigned long long bt = __ballot(take);
    const int word = (i * TOPK_THREADS + wave * 64) / 32;
    if (lane == 0 && word < nwords) maskrow[word] = (unsigned)bt;
    if (lane == 0 && word + 1 < nwords) maskrow[word + 1] = (unsigned)(bt >> 32);
    const unsigned pos = take_tab[i * NW + wave] + (unsigned)__popcll(bt & below_lanes);
    if (take && pos < (unsigned)k) selrow[pos] = u;
    if (v && !take && sc[i] > below_max) below_max = sc[i];
  }
#undef TOPK_VALID
  if (gap) {
    double dummy = 0.0;
    block_minmax(dummy, below_max, wred);
    if (tid == 0) {
      // k-th ranked score and (k+1)-th (greatest not kept; equal to the
      // k-th when a tie straddles the cut)
      const double den = fmax(fmax(fabs(st), fabs(below_max)), 1e-300);
      gap[(long long)h * T + t] = fabs(st - below_max) / den;
    }
  }
}

size_t select_chunk(const Geom& g) { return (size_t)(g.T < SELECT_CHUNK ? g.T : SELECT_CHUNK); }

size_t select_workspace_bytes(const Geom& g) {
  return (size_t)g.H * g.T * D * sizeof(double) + select_chunk(g) * (size_t)g.T * sizeof(double);
}

// Workspace: qbar [H][T][64] fp64, then scores [chunk][T] fp64.
hipError_t launch_select(const Geom& g, int k, const u16* Q, const double* kbar, int* sel,
                         unsigned* selmask, double* gap, void* ws, hipStream_t s) {
  double* qbar = (double*)ws;
  double* scores = qbar + (size_t)g.H * g.T * D;
  hipLaunchKernelGGL(qbar_kernel, dim3(g.T, g.H), dim3(64), 0, s, g, Q, qbar);
  const int chunk = (int)select_chunk(g);
  for (int h = 0; h < g.H; ++h) {
    for (int t0 = 0; t0 < g.T; t0 += chunk) {
      const int nq = g.T - t0 < chunk ? g.T - t0 : chunk;
      if (k > 0 && k < g.T)
        hipLaunchKernelGGL(scores_kernel, dim3((g.T + 63) / 64, (nq + 63) / 64), dim3(256), 0, s,
                           g, h, t0, nq, qbar, kbar, scores);
      hipLaunchKernelGGL(topk_kernel, dim3(nq), dim3(TOPK_THREADS), 0, s, g, h, t0, k, scores,
                         sel, selmask, gap);
    }
  }
  return hipGetLastError();
}

}  // namespace zebra
