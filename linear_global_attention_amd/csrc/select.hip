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
// chunk) and topk (one 1024-thread workgroup per query tile: MSB-first
// radix select over order-preserving 64-bit keys, then an ascending
// compaction by workgroup prefix sums that also writes the bitmap).
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

// Scores of query tiles [t0, t0+nq) of head h against every key tile:
// out[tq][u] = (sum_d qbar[t0+tq][d] * kbar[u][d]) * 0.125.
// grid (ceil(T/64), ceil(nq/64)), block 256 (16x16 threads, 4x4 each).
__global__ void __launch_bounds__(256) scores_kernel(Geom g, int h, int t0, int nq,
                                                     const double* __restrict__ qbar,
                                                     const double* __restrict__ kbar,
                                                     double* __restrict__ out) {
  __shared__ double qs[D][64 + 1];
  __shared__ double ks[D][64 + 1];
  const int tid = threadIdx.x;
  const int u0 = blockIdx.x * 64, q0 = blockIdx.y * 64;
  const double* qb = qbar + ((long long)h * g.T + t0) * D;
  const double* kb = kbar + (long long)h * g.T * D;
  for (int i = tid; i < 64 * D; i += 256) {
    const int r = i / D, d = i % D;
    qs[d][r] = (q0 + r < nq) ? qb[(long long)(q0 + r) * D + d] : 0.0;
    ks[d][r] = (u0 + r < g.T) ? kb[(long long)(u0 + r) * D + d] : 0.0;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;
  double acc[4][4] = {};
  for (int d = 0; d < D; ++d) {
    double a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = qs[d][ty * 4 + i];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = ks[d][tx * 4 + j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = q0 + ty * 4 + i;
    if (q >= nq) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = u0 + tx * 4 + j;
      if (u < g.T) out[(long long)q * g.T + u] = acc[i][j] * 0.125;
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

// Exclusive prefix over the workgroup (tid order) of two flags at once.
// Returns prefix in .x/.y and writes the totals.
__device__ inline int2 wg_prefix2(bool a, bool b, int* lds /*[2*16]*/, int& tot_a, int& tot_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long ba = __ballot(a), bb = __ballot(b);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int pa = __popcll(ba & below), pb = __popcll(bb & below);
  __syncthreads();
  if (lane == 0) {
    lds[wave] = __popcll(ba);
    lds[16 + wave] = __popcll(bb);
  }
  __syncthreads();
  int ta = 0, tb = 0;
  for (int w = 0; w < TOPK_THREADS / 64; ++w) {
    const int ca = lds[w], cb = lds[16 + w];
    if (w < wave) {
      pa += ca;
      pb += cb;
    }
    ta += ca;
    tb += cb;
  }
  tot_a = ta;
  tot_b = tb;
  return make_int2(pa, pb);
}

// grid (nq), block 1024: top-k of query tile t0+blockIdx.x of head h.
__global__ void __launch_bounds__(TOPK_THREADS) topk_kernel(Geom g, int h, int t0, int k,
                                                            const double* __restrict__ scores,
                                                            int* __restrict__ sel,
                                                            unsigned* __restrict__ selmask,
                                                            double* __restrict__ gap) {
  __shared__ unsigned hist[256];
  __shared__ unsigned long long sh_prefix;
  __shared__ unsigned sh_want;
  __shared__ int lds[32];
  __shared__ unsigned long long sh_below;
  const int tid = threadIdx.x;
  const int t = t0 + blockIdx.x;
  const int T = g.T;
  const int nwords = (T + 31) / 32;
  const double* row = scores + (long long)blockIdx.x * T;
  int* selrow = sel + ((long long)h * T + t) * k;
  unsigned* maskrow = selmask + ((long long)h * T + t) * nwords;

  unsigned long long key[TOPK_PER_THREAD];
#pragma unroll
  for (int i = 0; i < TOPK_PER_THREAD; ++i) {
    const int u = i * TOPK_THREADS + tid;
    key[i] = (u < T) ? score_key(row[u]) : 0ull;
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

  // MSB-first radix select of the k-th largest key.
  unsigned long long prefix = 0ull, pmask = 0ull;
  unsigned want = (unsigned)k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += TOPK_THREADS) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TOPK_PER_THREAD; ++i) {
      const int u = i * TOPK_THREADS + tid;
      if (u < T && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending order)
      unsigned c[4], s = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * tid - j];
        s += c[j];
      }
      // exclusive prefix of s over lanes (lane order = descending bins)
      unsigned incl = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned o = __shfl_up(incl, off, 64);
        if (tid >= off) incl += o;
      }
      unsigned above = incl - s;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < want && want <= above + c[j]) {
          sh_prefix = prefix | ((unsigned long long)(255 - 4 * tid - j) << shift);
          sh_want = want - above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    want = sh_want;
    pmask |= 255ull << shift;
    __syncthreads();
  }
  const unsigned long long kth = prefix;  // key of the k-th ranked tile

  // Ascending compaction: keys above kth, then the first `want` ties.
  if (tid == 0) sh_below = 0ull;
  int sel_base = 0, tie_base = 0;
  unsigned long long below_max = 0ull;
  for (int i = 0; i < TOPK_PER_THREAD; ++i) {
    if (i * TOPK_THREADS >= T) break;  // uniform across the workgroup
    const int u = i * TOPK_THREADS + tid;
    const bool valid = u < T;
    const bool gt = valid && key[i] > kth;
    const bool eq = valid && key[i] == kth;
    if (valid && key[i] < kth && key[i] > below_max) below_max = key[i];
    int teq, dummy;
    const int2 pe = wg_prefix2(eq, false, lds, teq, dummy);
    const bool take = gt || (eq && (tie_base + pe.x) < (int)want);
    int ttake;
    const int2 pt = wg_prefix2(take, false, lds, ttake, dummy);
    if (take && sel_base + pt.x < k) selrow[sel_base + pt.x] = u;
    const unsigned long long bal = __ballot(take);
    const int lane = tid & 63;
    const int word = (i * TOPK_THREADS + (tid - lane)) / 32;
    if (lane == 0 && word < nwords) maskrow[word] = (unsigned)bal;
    if (lane == 0 && word + 1 < nwords) maskrow[word + 1] = (unsigned)(bal >> 32);
    sel_base += ttake;
    tie_base += teq;
  }
  if (gap) {
    atomicMax(&sh_below, below_max);
    __syncthreads();
    if (tid == 0) {
      const double sk = key_score(kth);
      double sk1;
      if (tie_base > (int)want) sk1 = sk;  // another tile ties the k-th
      else sk1 = key_score(sh_below);
      const double den = fmax(fmax(fabs(sk), fabs(sk1)), 1e-300);
      gap[(long long)h * T + t] = fabs(sk - sk1) / den;
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
