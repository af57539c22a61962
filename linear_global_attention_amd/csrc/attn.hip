// Tile-sparse and dense softmax attention for gfx950 (bf16 MFMA, LDS-shared
// key/value tiles, fixed per-row softmax offsets).
//
// Zebra3D pages, "Linear-centered stages plus tile-sparse stages": kept key
// tiles keep full softmax interactions, omitted tiles are seen through their
// mean-K/V landmark, special-token keys are always visible, special query
// rows are dense and every patch query keeps its own key. "Global attention
// dominates runtime as views grow": dense attention over all tokens is the
// baseline this stage replaces.
//
// Work decomposition. A workgroup of 4 waves owns FG = 5 query groups of one
// head (a group is a patch query tile of <= 64 rows, or 64 special rows);
// two workgroups share a CU. Row block j (16 rows) of group s belongs to wave
// (s + j) % 4, so every wave holds one 16-row slot of (almost) every group:
// all four waves have the same active slots for every staged key tile and
// none waits for another at the tile barrier, while the two workgroups of
// a CU, each with its own barrier, fill each other's MFMA and VALU gaps.
// Tiles are streamed through a ring of FNBUF = 4 LDS buffers in batches of
// two (async global->LDS loads; one wait and one barrier per batch, while
// the next batch loads). The tiles a
// workgroup stages are the union of its groups' kept tiles, and the more
// groups share a staged tile the fewer bytes each kept (row, key) pair costs.
//
// Softmax offsets. Instead of a running max, each row i uses one offset M_i
// that is >= every logit it can see, found by attn_bound_kernel from |q_i|
// and the head's largest key norm (Cauchy-Schwarz, plus ln n_u <= ln 64 for
// a landmark). With p = exp2(x - M_i) <= 1 nothing overflows, and the partial sums
// of different key segments simply add. The row's own key is always visible,
// so M_i minus the own logit bounds how far below 1 the largest p can be;
// groups with a row where that gap exceeds SAFE_GAP (log2 units) are flagged
// and recomputed by an exact online-softmax kernel (attn_exact.hip).
//
// Rounds. The main kernel runs once per round of work units, a round being
// the workgroups that are resident at once: they all start together on the
// same head and walk its key tiles in ascending order, so each XCD's L2
// fetches a tile once for all of its workgroups that use it (reads past the
// L2 run at about the HBM rate, reads that hit it at about four times that).
// A special item sees every key; it is split into key segments whose
// partial O and l are summed by attn_special_combine_kernel.
//
// Per 32-key block and 16-row slot: S^T = K (C Q)^T - M (4
// v_mfma_f32_16x16x32_bf16, A = keys from LDS, B = the queries scaled by
// C = log2(e)/8 and rounded to bf16 once per unit, the accumulators starting
// at -M), p = exp2(S^T) with no further arithmetic, O^T += V^T P^T (4
// MFMAs; lane group g holds keys 4g..4g+3 of both 16-key halves of S^T, the
// k-slot order of the value fragment, whose 32-key blocks are stored [64
// channels][32] with keys permuted by value_pos). Row sums use the
// bf16-rounded p that P.V sees, through one more MFMA whose A operand is 1
// for real keys and 0 for the zero padding of a tile's last block. The bf16
// rounding of C q changes a logit by at most 2^-8 of |C q_c k_c| per channel
// term (measured: 8.3e-4 against 7.6e-4 max-abs at 1,024 views), and saves
// the per-score multiply-add that used to sit between the MFMAs.
// LDS layouts are XOR-swizzled at 16-byte granularity (keys: column ^ key%8,
// values: column ^ (channel/2)%4) so fragment reads are bank-conflict free;
// the swizzle is applied through the per-lane source address of the async
// loads, which write LDS linearly.
#include "attn_common.hpp"

namespace zebra {

// wait until at most n of this wave's vector memory operations are pending
#define ZEBRA_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))


// Per-lane source offsets of a wave's 1 KB shares (chunks c = wave,
// wave + FWAVES, ...) of a staged 8 KB key or value half (swizzled as in
// stage_keys / stage_vals), for an 8 KB source and for a 4 KB source (read
// twice). Computed once per wave.
constexpr int FCHUNKS = 8 / FWAVES;  // 1 KB shares per wave per 8 KB half
struct StageOffsets {
  unsigned k8[FCHUNKS], k4[FCHUNKS], v8[FCHUNKS], v4[FCHUNKS];
  __device__ StageOffsets(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < FCHUNKS; ++i) {
      const int c = wave + i * FWAVES;
      const int P8 = c * 1024 + lane * 16, P4 = (c * 1024) % 4096 + lane * 16;
      k8[i] = koff(P8);
      k4[i] = koff(P4);
      v8[i] = voff(P8);
      v4[i] = voff(P4);
    }
  }
  static __device__ unsigned koff(int P) {
    const int key = P >> 7, col = (P >> 4) & 7;
    return (unsigned)(key * 128 + ((col ^ (key & 7)) << 4));
  }
  static __device__ unsigned voff(int P) {
    const int d = (P >> 6) & 63, col = (P >> 4) & 3;
    return (unsigned)((P & ~63) + ((col ^ ((d >> 1) & 3)) << 4));
  }
};

// One wave's shares of the async copy of an 8 KB half of a staged item;
// `off` holds the wave's per-chunk offsets for the source's size.
// The wave's LDS offset passes through an empty asm statement, so that the
// compiler computes each destination as offset + constant at the copy
// instead of holding every (buffer, chunk) destination in its own scalar
// register across the loop.
__device__ __forceinline__ void stage_share(char* dst, int wave, const char* src, const unsigned (&off)[FCHUNKS]) {
  int wofs = wave * 1024;
  asm volatile("" : "+s"(wofs));
#pragma unroll
  for (int i = 0; i < FCHUNKS; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(src + off[i]), (lds_void*)(dst + wofs + i * FWAVES * 1024),
                                     16, 0, 0);
}


template <int G>
struct MainState {
  bf16x8 q[G][2];  // B operand of each slot: query (lane%16), channels ds*32+8g..+7
  f32x4 o[G][4];   // O^T of each slot: channel db*16+4g+r, query lane%16
  f32x4 l[G];      // row sums of bf16(P) by MFMA: every element = sum of query lane%16
  f32x4 negm[G];   // -M (log2 units) in every element: the initial S^T of a token block
  bf16x8 lmask;    // A operand of the row-sum MFMA: 1 for the block's real keys, 0 for padding
};

constexpr unsigned BF16_ONE2 = 0x3F803F80u;  // two bf16 ones

// All-ones row-sum operand, opaque to the compiler so that it stays in
// registers rather than being rebuilt around every MFMA that reads it.
__device__ __forceinline__ bf16x8 ones_operand() {
  uint4 w = make_uint4(BF16_ONE2, BF16_ONE2, BF16_ONE2, BF16_ONE2);
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
  return __builtin_bit_cast(bf16x8, w);
}

// Row-sum operand of a block whose first n < 32 keys are real: k-slot j of
// lane group g is key 4g + j (j < 4) or 16 + 4g + j - 4, the order of the
// probabilities in pv().
__device__ __forceinline__ bf16x8 key_mask_operand(int n, int lane) {
  const int t0 = n - 4 * (lane >> 4), t1 = t0 - 16;
  auto pair = [](bool a, bool b) { return (a ? 0x3F80u : 0u) | (b ? 0x3F800000u : 0u); };
  return __builtin_bit_cast(bf16x8, make_uint4(pair(0 < t0, 1 < t0), pair(2 < t0, 3 < t0), pair(0 < t1, 1 < t1),
                                               pair(2 < t1, 3 < t1)));
}

// Slot s of this wave: its queries as MFMA B fragments (zero for rows past
// the group's end).
template <int G>
__device__ __forceinline__ void load_queries(const Geom& g, const AttnArgs& A, const QueryGroups& qg, int h,
                                             unsigned slots, int lane, bf16x8 q[G][2]) {
  const int lg = lane >> 4, tl = lane & 15;
#pragma unroll
  for (int s = 0; s < G; ++s) {
    const int j = qg.row_block(s) * 16 + tl;
    const bool ok = ((slots >> s) & 1u) && j < qg.rows(s);
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (ok) w = *(const uint4*)(A.Q + qg.token(s, j) * g.in_tok + h * g.in_head + ds * 32 + 8 * lg);
      q[s][ds] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// p = exp2(s) for the lane's 8 keys of a 32-key block (s already in log2
// units with the row's offset applied)
__device__ __forceinline__ void probs(const f32x4& s0, const f32x4& s1, float p[8]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = __builtin_amdgcn_exp2f(s0[r]);
    p[4 + r] = __builtin_amdgcn_exp2f(s1[r]);
  }
}

// The queries of a slot scaled by C = log2(e)/8 and rounded to bf16, so that
// S^T = K (C Q)^T - M comes out of the MFMAs in log2 units with the row's
// offset already applied (the offset is the accumulators' initial value).
__device__ __forceinline__ void scale_queries(bf16x8 q[2]) {
#pragma unroll
  for (int ds = 0; ds < 2; ++ds) {
    uint4 w;
    unsigned* wp = (unsigned*)&w;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      wp[m] = pack_bf16((float)q[ds][2 * m] * QK_LOG2, (float)q[ds][2 * m + 1] * QK_LOG2);
    q[ds] = __builtin_bit_cast(bf16x8, w);
  }
}

// Whether slot s is set in the wave-uniform mask m, as a scalar test: the
// value passes through readfirstlane so that the compiler branches on it
// directly (s_bitcmp + s_cbranch) instead of building exec-mask flow blocks
// around each slot (measured faster in the token-block loop; not in the
// landmark and bound loops).
__device__ __forceinline__ bool slot_on(unsigned m, int s) {
  return __builtin_amdgcn_readfirstlane((int)((m >> s) & 1u)) != 0;
}

// O^T += V^T bf16(P)^T, and the row sums of bf16(P) as one more MFMA whose
// A operand is 1 for real keys and 0 for padding (cheaper than eight adds
// per lane).
__device__ __forceinline__ void pv(const float p[8], const bf16x8 vf[4], const bf16x8& lmask, f32x4 o[4],
                                   f32x4& l) {
  const unsigned w0 = pack_bf16(p[0], p[1]), w1 = pack_bf16(p[2], p[3]);
  const unsigned w2 = pack_bf16(p[4], p[5]), w3 = pack_bf16(p[6], p[7]);
  const bf16x8 P = __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], P, o[db], 0, 0, 0);
  l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lmask, P, l, 0, 0, 0);
}

// One staged 32-key block of token or special keys (rows key0.. of the
// LDS item, the first n real) for every user slot. Padding keys are zero in
// K and V (the packed layouts pad every tile and the special keys with
// zeros), so their p = exp2(-M) is finite and adds nothing to O^T; the
// row-sum operand leaves them out of l. S^T therefore starts from zero.
template <int SW>
__device__ __forceinline__ void attend_block(MainState<SW>& st, unsigned us, const char* kb, int key0, int n,
                                             int lane) {
  bf16x8 kf[2][2], vf[4];
  load_kfrag(kb, key0, lane, kf);
  load_vfrag(kb + LDS_V + key0 * 128, lane, vf);
  const bool part = n < KBLK;
  if (part) st.lmask = key_mask_operand(n, lane);
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    if (!slot_on(us, s)) continue;
    f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][0], st.q[s][0], st.negm[s], 0, 0, 0);
    f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][0], st.q[s][0], st.negm[s], 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][1], st.q[s][1], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][1], st.q[s][1], a1, 0, 0, 0);
    float p[8];
    probs(a0, a1, p);
    pv(p, vf, st.lmask, st.o[s], st.l[s]);
  }
  if (part) st.lmask = ones_operand();
}

// The landmark block lb (landmarks of tiles 32lb..32lb+31) for every user
// slot: logit q.kbar/8 + ln n_u, value vbar_u. In log2 units the landmark
// term log2(n_u) - M (-inf past the last tile, and -inf for the tiles the
// slot's group kept) is the initial value of the S^T accumulators.
template <int SW>
__device__ __forceinline__ void attend_landmarks(MainState<SW>& st, unsigned us, const char* kb, int lb,
                                                 cmask_ptr mrow0, long long mstep, int lane) {
  bf16x8 kf[2][2], vf[4];
  load_kfrag(kb, 0, lane, kf);
  load_vfrag(kb + LDS_V, lane, vf);
  const int lg = lane >> 4;
  float l2n[8];
  load_row8(kb + LM_LOG2N_ROW * 128, lane, l2n);
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    if (!((us >> s) & 1u)) continue;
    const unsigned kept = mrow0[s * mstep + lb];
    f32x4 c0, c1;
    const float nm = st.negm[s][0];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c0[r] = (kept >> (4 * lg + r)) & 1u ? -INFINITY : l2n[r] + nm;
      c1[r] = (kept >> (16 + 4 * lg + r)) & 1u ? -INFINITY : l2n[4 + r] + nm;
    }
    f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][0], st.q[s][0], c0, 0, 0, 0);
    f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][0], st.q[s][0], c1, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][1], st.q[s][1], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][1], st.q[s][1], a1, 0, 0, 0);
    float p[8];
    probs(a0, a1, p);
    pv(p, vf, st.lmask, st.o[s], st.l[s]);
  }
}

// Work item -> (head, query groups): per head the special items first (they
// walk every key tile), then the patch items.
struct FastItem {
  int h, item;  // item in QueryGroups numbering
  __device__ FastItem(const Geom& g, int block) {
    const FastItems fi(g);
    h = block / fi.per_head;
    const int b = block - h * fi.per_head;
    item = b < fi.spec_items ? fi.patch_items + b : b - fi.spec_items;
  }
};

// Index of this lane's record of slot s in the per-lane workspace arrays;
// record >> 8 is the group's index (head-major) in the flag array.
__device__ __forceinline__ long long lane_record(const Geom& g, const QueryGroups& qg, int h, int s, int lane) {
  const FastItems fi(g);
  const int gid = (qg.patch ? 0 : g.T) + qg.tile(s);
  return (((long long)h * fi.groups_per_head + gid) * 4 + qg.row_block(s)) * 64 + lane;
}

// One staged item, as a plan entry: x = kind << 28 | index (kind 0: token
// tile, index = its first 32-slot block within the head; kind 1: landmark
// block; kind 2: special-key block), y = users | key count << 8 (users: the
// item's groups that see it).
struct Item {
  unsigned x, y;
  __device__ int kind() const { return (int)(x >> 28); }
  __device__ int index() const { return (int)(x & 0x0FFFFFFFu); }
  __device__ unsigned users() const { return y & 0xFFu; }
  __device__ int nkeys() const { return (int)(y >> 8); }
};
constexpr int KIND_TILE = 0, KIND_LANDMARK = 1, KIND_SPECIAL = 2, KIND_CHECKPOINT = 3, KIND_NOP = 4;
// Patch units meet every CK_WORDS words of key tiles (a checkpoint entry in
// their plans), so that the workgroups of a round, which drift apart as
// they walk the keys at slightly different speeds, stay close enough for an
// XCD's L2 to still hold a tile when most of them read it. A wave goes on
// once three quarters of the round's waves have arrived (CK_RELEASE_PCT):
// the fast ones wait and none runs more than a segment ahead, while the
// slowest quarter never waits. The wait is bounded: after CK_SPIN_MAX polls
// a wave goes on regardless. (64 words and 75% measured best at 1,024
// views, 4% ahead of 128 words and 50%.)
constexpr int CK_WORDS = 64;
// Plan entries a wave copies to LDS at a time (one 16-byte async load per lane).
constexpr int PLAN_CHUNK = 128;
constexpr int CK_SPIN_MAX = 1000;
constexpr int CK_RELEASE_PCT = 85;
static_assert(FG <= 8, "plan entries hold 8 user bits");

// Streams items through an LDS ring of two halves, ringA and ringB (two
// items each, separate arrays), in batches of two: `next(items)` yields the
// next batch (up to two items), `issue(item, buf)` starts an item's async
// loads, and once a batch has landed in every wave `consume(item, buf)` runs
// for each of its items while the next batch loads into the other half. One
// wait and one barrier per batch. The loop is unrolled over the two halves
// so that every LDS read names the half it reads: the compiler then knows
// that it cannot alias the copies in flight into the other half and adds no
// wait for them. A batch's plan entries are taken before its copies are
// issued, and `refill()` then starts any plan copy that next() asked for.
// Every wave walks the same sequence itself and keeps the batches in scalar
// registers.
template <typename Next, typename Issue, typename Consume, typename Refill>
__device__ __forceinline__ void stream_items(char* ringA, char* ringB, Next next, Issue issue, Consume consume,
                                             Refill refill) {
  static_assert(FNBUF == 4, "two halves of two items");
  bool more = true;
  auto fetch = [&](Item (&it)[2]) -> int {
    const int n = more ? next(it) : 0;
    more = n == 2;
    return n;
  };
  Item a[2], b[2];
  int na = fetch(a), nb = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (j < na) issue(a[j], ringA + j * LDS_BUF);
  refill();
  while (na > 0) {
    ZEBRA_VMCNT(0);  // batch a (ringA) has landed
    ring_barrier();  // ... in every wave; ringB is free
    nb = fetch(b);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < nb) issue(b[j], ringB + j * LDS_BUF);
    refill();
    consume(a[0], ringA);
    if (na > 1) consume(a[1], ringA + LDS_BUF);
    if (nb == 0) break;
    ZEBRA_VMCNT(0);  // batch b (ringB) has landed
    ring_barrier();  // ... in every wave; ringA is free
    na = fetch(a);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < na) issue(a[j], ringA + j * LDS_BUF);
    refill();
    consume(b[0], ringB);
    if (nb > 1) consume(b[1], ringB + LDS_BUF);
  }
  ring_barrier();
}

// Per head, the largest squared key norm over every packed patch key and
// special key (zero padding included), as the bits of a non-negative float
// in kmax2[h] (cleared beforehand). grid (KN_BLOCKS, H), block 256: four
// lanes per key row (16 channels each), rows strided over the grid, one
// atomic per workgroup.
constexpr int KN_BLOCKS = 256;
__global__ void __launch_bounds__(256) key_norm_max_kernel(Geom g, AttnArgs A, unsigned* kmax2) {
  __shared__ float wmax[4];
  const int h = blockIdx.y;
  const int part = threadIdx.x & 3;
  const long long nrows = g.slots + g.spec_pad;
  float best = 0.f;
  for (long long r = (long long)blockIdx.x * 64 + (threadIdx.x >> 2); r < nrows; r += (long long)KN_BLOCKS * 64) {
    const u16* row = r < g.slots ? A.Kt + ((long long)h * g.slots + r) * D
                                 : A.Ks + ((long long)h * g.spec_pad + (r - g.slots)) * D;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 w = *(const uint4*)(row + part * 16 + c * 8);
      const bf16x8 v = __builtin_bit_cast(bf16x8, w);
#pragma unroll
      for (int m = 0; m < 8; ++m) ss = fmaf((float)v[m], (float)v[m], ss);
    }
    ss += __shfl_xor(ss, 1, 64);  // the row's four lanes (all active together)
    ss += __shfl_xor(ss, 2, 64);
    best = fmaxf(best, ss);
  }
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) best = fmaxf(best, __shfl_xor(best, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(&kmax2[h], __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

// Offsets. Every logit a row sees is at most |q| K_max / 8 (Cauchy-Schwarz,
// K_max the head's largest key norm, which also bounds a landmark's mean key
// up to its bf16 rounding), and a landmark adds at most log2(64) = 6 (log2
// units) for ln n_u. So M_i = C |q_i| K_max * 1.01 + 6 bounds every logit of
// row i (C = log2(e) / 8); -M goes to the row's lane records. A group with a
// row whose own logit lies more than SAFE_GAP below M is flagged, and the
// exact kernel recomputes it afterwards.
template <int G, int SW>
__global__ void __launch_bounds__(FWAVES * 64) attn_bound_kernel(Geom g, AttnArgs A, float* ws_negm, int* flags,
                                                                 const unsigned* kmax2) {
  const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
  const int lg = lane >> 4, tl = lane & 15;
  const int simd = wave & 3, s0 = (wave >> 2) * SW;
  const FastItem it(g, blockIdx.x);
  const int h = it.h;
  const FastItems fi(g);
  const QueryGroups qg(g, it.item, fi.patch_items, G, simd, s0, true);  // this wave's SW slots
  const u16* Kt16 = A.Kt + (long long)h * g.slots * D;
  const u16* Ks16 = A.Ks + (long long)h * g.spec_pad * D;
  const float kmax = sqrtf(__uint_as_float(kmax2[h])) * 1.01f;

  unsigned slots = 0u;
#pragma unroll
  for (int s = 0; s < SW; ++s)
    if (qg.row_block(s) * 16 < qg.rows(s)) slots |= 1u << s;
  bf16x8 q[SW][2];
  load_queries<SW>(g, A, qg, h, slots, lane, q);
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    if (!((slots >> s) & 1u)) continue;
    const int j = qg.row_block(s) * 16 + tl;
    const bool ok = j < qg.rows(s);
    float qq = 0.f, qko = 0.f;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds) {
      uint4 kw = make_uint4(0, 0, 0, 0);
      if (ok) kw = *(const uint4*)((qg.patch ? Kt16 : Ks16) + qg.own_slot(s, j) * D + ds * 32 + 8 * lg);
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kw);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float a = (float)q[s][ds][m];
        qq = fmaf(a, a, qq);
        qko = fmaf(a, (float)kv[m], qko);
      }
    }
    qq = xsum32(xsum16(qq));
    qko = xsum32(xsum16(qko));
    const float m = sqrtf(qq) * QK_LOG2 * 1.0001f * kmax + 6.0f;
    const bool bad = __builtin_amdgcn_ballot_w64(ok && m - qko * QK_LOG2 > SAFE_GAP) != 0;
    const long long rec = lane_record(g, qg, h, s, lane);
    ws_negm[rec] = -m;
    if (bad && lane == 0) flags[rec >> 8] = 1;
  }
}

// The plan of the units [unit0, unit0 + nunits) (one wave per unit, one
// word of 32 tiles per lane): first, for tile-sparse patch items, the
// landmark block of every word of which some group omitted a tile; then for
// each key word in order the word's tiles that some group kept, ascending
// (every tile for dense items and special segments), each with the bit set
// of groups that see it; then, for patch items and the last segment of a
// special item, the special-key blocks. Patch units also get a
// checkpoint entry after every CK_WORDS-th word but the last. The landmark
// section is padded to an even length with a no-op entry, so that the main
// kernel takes both entries of a batch with one LDS read. Writes count[2i]
// entries of at most `stride` to plan + i * stride for unit unit0 + i and
// the landmark section's length to count[2i + 1], and zeroes the round's
// checkpoint counters.
template <int G>
__global__ void __launch_bounds__(256) attn_plan_kernel(Geom g, AttnArgs A, int segs, int unit0, int nunits,
                                                        uint2* plan, int* count, int stride, int* ckpt,
                                                        int nckpt) {
  __shared__ int tiles[MAX_TPF];
  for (int i = threadIdx.x; i < g.tpf; i += blockDim.x) tiles[i] = g.tile[i];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nckpt; i += blockDim.x) ckpt[i] = 0;  // this round's checkpoint counters
  __syncthreads();
  const FastItems fi(g);
  const int lane = threadIdx.x & 63;
  const int local = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (local >= nunits) return;  // uniform per wave
  const Unit un(g, segs, unit0 + local);
  const QueryGroups qgi(g, un.item, fi.patch_items, G, 0, 0, true);
  const long long mstep = (long long)qgi.stride * A.nwords;  // mask words between the item's groups
  const bool sparse = A.sparse && qgi.patch;
  int w0, w1;
  seg_words(A.nwords, segs, un.seg, w0, w1);
  unsigned valid = 0u;
#pragma unroll
  for (int s = 0; s < G; ++s)
    if (qgi.rows(s) > 0) valid |= 1u << s;
  const unsigned* mrow = sparse ? A.selmask + ((long long)un.h * g.T + qgi.gid0) * A.nwords : A.selmask;
  uint2* out = plan + (long long)local * stride;
  int base = 0;
  if (sparse) {  // the landmark blocks first
    for (int wb = w0; wb < w1; wb += 64) {
      const int w = wb + lane;
      unsigned lm = 0u;
#pragma unroll
      for (int s = 0; s < G; ++s)
        if (w < w1 && ((valid >> s) & 1u) && mrow[s * mstep + w] != 0xFFFFFFFFu) lm |= 1u << s;
      const unsigned long long bal = __ballot(lm != 0u);
      if (lm)
        out[base + __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u))] =
            make_uint2((unsigned)(KIND_LANDMARK << 28) | (unsigned)w, lm | (unsigned)(KBLK << 8));
      base += __builtin_popcountll(bal);
    }
    if (base & 1) {  // pad the landmark section to whole batches of two
      if (lane == 0) out[base] = make_uint2((unsigned)(KIND_NOP << 28), 0u);
      ++base;
    }
  }
  const int nlm = base;
  for (int wb = w0; wb < w1; wb += 64) {
    const int w = wb + lane;
    const bool on = w < w1;
    unsigned m[G], un_bits = 0u;
#pragma unroll
    for (int s = 0; s < G; ++s) {
      unsigned v = 0u;
      if (on && ((valid >> s) & 1u)) {
        if (sparse) {
          v = mrow[s * mstep + w];
        } else {
          const int rem = g.T - w * 32;
          v = rem >= 32 ? 0xFFFFFFFFu : ((1u << rem) - 1u);
        }
      }
      m[s] = v;
      un_bits |= v;
    }
    const bool ck = qgi.patch && on && (w + 1) % CK_WORDS == 0 && w + 1 < w1;
    const int cnt = __builtin_popcount(un_bits) + (ck ? 1 : 0);
    int incl = cnt;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    int o = base + incl - cnt;
    for (unsigned bits = un_bits; bits; bits &= bits - 1u) {
      const int b = __builtin_ctz(bits), u = w * 32 + b;
      unsigned users = 0u;
#pragma unroll
      for (int s = 0; s < G; ++s) users |= ((m[s] >> b) & 1u) << s;
      const int fu = frame_of_tile(g, u), te = tiles[u - fu * g.tpf];
      const int slot = fu * g.slots_pf + (te & 0xFFFFF);
      const int nk = ((te >> 20) & 15) * ((te >> 24) & 15);
      out[o++] = make_uint2((unsigned)(KIND_TILE << 28) | (unsigned)(slot / KBLK), users | (unsigned)(nk << 8));
    }
    if (ck) out[o++] = make_uint2((unsigned)(KIND_CHECKPOINT << 28) | (unsigned)((w + 1) / CK_WORDS - 1), 0u);
    base += __shfl(incl, 63, 64);
  }
  if (un.seg < 0 || un.seg == segs - 1) {
    const int nsb = g.spec_pad / KBLK;
    for (int b = lane; b < nsb; b += 64)
      out[base + b] = make_uint2((unsigned)(KIND_SPECIAL << 28) | (unsigned)b,
                                 valid | (unsigned)(min(KBLK, g.nspec - b * KBLK) << 8));
    base += nsb;
  }
  if (lane == 0) {
    count[2 * local] = base;
    count[2 * local + 1] = nlm;
  }
}

// Index of this lane's partial record of slot s of a special segment unit:
// (head, special item, segment, group of the item, row block, lane).
__device__ __forceinline__ long long spec_record(const Geom& g, int h, int item, int seg, const QueryGroups& qg,
                                                 int s, int lane) {
  const FastItems fi(g);
  const int si = item - fi.patch_items;
  return ((((long long)(h * fi.spec_items + si) * SPEC_SEGS_MAX + seg) * FG + (qg.s0 + s)) * 4 +
          qg.row_block(s)) * 64 + lane;
}

// O = O^T / l for slot s and bf16 store of its rows (row = query
// row_block*16 + lane%16, channels db*16 + 4g + r). Every lane takes part in
// the row-sum reduction.
__device__ __forceinline__ void store_slot(const Geom& g, const AttnArgs& A, const QueryGroups& qg, int h, int s,
                                           const f32x4 o[4], float l, int lane) {
  const int lg = lane >> 4, tl = lane & 15;
  const float inv = 1.0f / xsum32(xsum16(l));
  const int j = qg.row_block(s) * 16 + tl;
  if (j < qg.rows(s)) {
    u16* orow = A.O + qg.token(s, j) * g.out_tok + h * g.out_head;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      uint2 wv;
      wv.x = pack_bf16(o[db][0] * inv, o[db][1] * inv);
      wv.y = pack_bf16(o[db][2] * inv, o[db][3] * inv);
      *(uint2*)(orow + db * 16 + 4 * lg) = wv;
    }
  }
}

// Checkpoint c of a round: this wave arrives, then polls (vector atomic
// loads, bounded) until `target` waves of the round's patch units have
// arrived.
__device__ __forceinline__ void checkpoint_wait(int* ctr, int target) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma nounroll
  for (int i = 0; i < CK_SPIN_MAX; ++i) {
    const int v = uni(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (v >= target) break;
    __builtin_amdgcn_s_sleep(2);
  }
}

// One work unit: a patch item over every key word (tile-sparse: landmark
// block of each word minus the tiles each group kept, and the union of the
// kept tiles; dense: every tile), then the special keys, the self key and
// the bf16 output; or one key segment of a special item, whose partial O
// and l go to the workspace for attn_special_combine_kernel.
template <int G, int SW>
__global__ void __launch_bounds__(FWAVES * 64, FOCC) attn_main_kernel(Geom g, AttnArgs A, int segs, int unit0,
                                                                   const uint2* plan, const int* plan_count,
                                                                   int plan_stride, const float* ws_negm,
                                                                   float* sp_l, f32x4* sp_o, int* ckpt,
                                                                   int ck_target) {
  __shared__ __attribute__((aligned(1024))) char ringA[2 * LDS_BUF];
  __shared__ __attribute__((aligned(1024))) char ringB[2 * LDS_BUF];
  __shared__ __attribute__((aligned(16))) uint2 plan_lds[FWAVES * 2 * PLAN_CHUNK];
  const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
  const int simd = wave & 3, s0 = (wave >> 2) * SW;
  const Unit un(g, segs, unit0 + blockIdx.x);
  const int h = un.h;
  const FastItems fi(g);
  const QueryGroups qg(g, un.item, fi.patch_items, G, simd, s0, true);   // this wave's SW slots
  const bool sparse = A.sparse && qg.patch;
  const u16* Kt16 = A.Kt + (long long)h * g.slots * D;
  const u16* Vt16 = A.Vt + (long long)h * g.slots * D;
  const u16* Ks16 = A.Ks + (long long)h * g.spec_pad * D;
  const u16* Vs16 = A.Vs + (long long)h * g.spec_pad * D;

  unsigned slots = 0u;  // this wave's non-empty slots
#pragma unroll
  for (int s = 0; s < SW; ++s)
    if (qg.row_block(s) * 16 < qg.rows(s)) slots |= 1u << s;

  MainState<SW> st;
  st.lmask = ones_operand();
  load_queries<SW>(g, A, qg, h, slots, lane, st.q);
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    float nm = 0.f;
    st.l[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[s][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    if ((slots >> s) & 1u) nm = ws_negm[lane_record(g, qg, h, s, lane)];
    st.negm[s] = f32x4{nm, nm, nm, nm};
  }
  ZEBRA_VMCNT(0);
#pragma unroll
  for (int s = 0; s < SW; ++s) scale_queries(st.q[s]);

  const char* lmh = (const char*)A.LM + (long long)h * g.T_pad * LM_BYTES_PER_TILE;
  // kept-tile bitmap row of this wave's slot s: mrow0 + s * mstep (the
  // item's groups are stride tiles apart)
  const cmask_ptr mrow0 =
      (cmask_ptr)(sparse ? A.selmask + ((long long)h * g.T + qg.gid0) * A.nwords : A.selmask);
  const long long mstep = (long long)qg.stride * A.nwords;
  const int nlb = g.T_pad / KBLK;

  // This unit's plan: `count` entries, in chunks of PLAN_CHUNK that each
  // wave copies into its own LDS buffer with one async load, a chunk ahead
  // (every batch of the ring starts with a full vmcnt wait, so a chunk has
  // landed long before it is read); entries are read back as uniform LDS
  // loads at the start of a batch, before its copies are issued.
  const uint2* pl = plan + (long long)blockIdx.x * plan_stride;
  const int count = uni(plan_count[2 * blockIdx.x]), nlm = uni(plan_count[2 * blockIdx.x + 1]);
  uint2* pbuf = plan_lds + wave * 2 * PLAN_CHUNK;
  auto load_chunk = [&](int c) {
    if (c * PLAN_CHUNK < count)
      __builtin_amdgcn_global_load_lds((const void*)(pl + c * PLAN_CHUNK + 2 * lane),
                                       (lds_void*)(pbuf + (c & 1) * PLAN_CHUNK), 16, 0, 0);
  };
  load_chunk(0);
  load_chunk(1);
  ZEBRA_VMCNT(0);
  // The plan is taken two entries at a time (one 16-byte LDS read; e stays
  // even, so a pair never straddles two chunks): first the landmark section
  // [0, nlm), then the rest up to `count`. Checkpoint entries are waited for
  // here; they and no-op entries stage and compute nothing.
  unsigned e = 0u, end = (unsigned)nlm;
  int want = -1;
  auto next2 = [&](Item (&it)[2]) -> int {
    if (e >= end) return 0;
    const uint4 v = *(const uint4*)(pbuf + (e & (2 * PLAN_CHUNK - 1)));
    it[0].x = (unsigned)uni((int)v.x);
    it[0].y = (unsigned)uni((int)v.y);
    it[1].x = (unsigned)uni((int)v.z);
    it[1].y = (unsigned)uni((int)v.w);
    if ((e & (PLAN_CHUNK - 1)) == 0 && e > 0) want = (int)(e / PLAN_CHUNK) + 1;  // into the chunk just finished
    const int n = end - e >= 2u ? 2 : 1;
    e += 2u;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < n && it[j].kind() == KIND_CHECKPOINT) checkpoint_wait(ckpt + it[j].index(), ck_target);
    return n;
  };
  const StageOffsets so(wave, lane);
  auto issue = [&](const Item& it, char* d) {
    const int kind = it.kind();
    if (kind >= KIND_CHECKPOINT) return;
    const bool vbig = kind == KIND_TILE && it.nkeys() > KBLK;
    const bool kbig = vbig || kind == KIND_LANDMARK;
    const long long idx = it.index();
    const char* ks;
    const char* vs;
    if (kind == KIND_TILE) {
      ks = (const char*)Kt16 + idx * (KBLK * D * 2);
      vs = (const char*)Vt16 + idx * (KBLK * D * 2);
    } else if (kind == KIND_LANDMARK) {
      ks = lmh + idx * LM_KEY_BLOCK;
      vs = lmh + (long long)nlb * LM_KEY_BLOCK + idx * (KBLK * D * 2);
    } else {
      ks = (const char*)Ks16 + idx * (KBLK * D * 2);
      vs = (const char*)Vs16 + idx * (KBLK * D * 2);
    }
    unsigned ko[FCHUNKS], vo[FCHUNKS];
#pragma unroll
    for (int i = 0; i < FCHUNKS; ++i) {
      ko[i] = kbig ? so.k8[i] : so.k4[i];
      vo[i] = vbig ? so.v8[i] : so.v4[i];
    }
    stage_share(d, wave, ks, ko);
    stage_share(d + LDS_V, wave, vs, vo);
  };
  auto consume_lm = [&](const Item& it, const char* kb) {
    if (it.kind() != KIND_LANDMARK) return;
    const unsigned us = (((unsigned)uni((int)it.y) & 0xFFu) >> s0) & slots;
    if (us) attend_landmarks<SW>(st, us, kb, it.index(), mrow0, mstep, lane);
  };
  auto consume = [&](const Item& it, const char* kb) {
    // the entry again as a scalar (the compiler may have parked it in a
    // vector register), so that the slot tests below are scalar bit tests
    const unsigned y = (unsigned)uni((int)it.y);
    const unsigned us = ((y & 0xFFu) >> s0) & slots;
    if (!us) return;
    const int nk = (int)(y >> 8);
    attend_block<SW>(st, us, kb, 0, nk, lane);
    if (nk > KBLK) attend_block<SW>(st, us, kb, KBLK, nk - KBLK, lane);
  };
  auto refill = [&] {
    if (want >= 0) {
      load_chunk(want);
      want = -1;
    }
  };
  stream_items(ringA, ringB, next2, issue, consume_lm, refill);
  end = (unsigned)count;
  stream_items(ringA, ringB, next2, issue, consume, refill);
  // Per-lane indices are recomputed after the walk rather than kept live
  // across it from the set-up (register pressure).
  int lane_a = lane;
  asm volatile("" : "+v"(lane_a));
  const int lg_a = lane_a >> 4, tl_a = lane_a & 15;
  // lane-partial row sums: the MFMA row sum counted once, in lanes 0..15
  float lpart[SW];
#pragma unroll
  for (int s = 0; s < SW; ++s) lpart[s] = lg_a == 0 ? st.l[s][0] : 0.f;

  if (un.seg >= 0) {
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      if (!((slots >> s) & 1u)) continue;
      const long long rec = spec_record(g, h, un.item, un.seg, qg, s, lane_a);
      sp_l[rec] = lpart[s];
#pragma unroll
      for (int db = 0; db < 4; ++db) sp_o[rec * 4 + db] = st.o[s][db];
    }
    return;
  }

  // self key of patch rows whose own tile was not kept
  if (sparse) {
#pragma unroll
    for (int s = 0; s < SW; ++s) {
      if (!((slots >> s) & 1u)) continue;
      const int t = qg.tile(s);
      if ((mrow0[s * mstep + (t >> 5)] >> (t & 31)) & 1u) continue;
      const int j = qg.row_block(s) * 16 + tl_a;
      const bool okrow = j < qg.rows(s);
      const long long slot = qg.own_slot(s, j);
      float dot = 0.f;
#pragma unroll
      for (int ds = 0; ds < 2; ++ds) {
        uint4 kw = make_uint4(0, 0, 0, 0);
        if (okrow) kw = *(const uint4*)(Kt16 + slot * D + ds * 32 + 8 * lg_a);
        const bf16x8 kv = __builtin_bit_cast(bf16x8, kw);
#pragma unroll
        for (int m = 0; m < 8; ++m) dot = fmaf((float)st.q[s][ds][m], (float)kv[m], dot);
      }
      dot = xsum32(xsum16(dot));  // C q . k (the queries are scaled)
      const float p = okrow ? __builtin_amdgcn_exp2f(dot + st.negm[s][0]) : 0.f;
      lpart[s] += (lg_a == 0 ? p : 0.f);
      const long long vblk = slot / KBLK;
      const int pos = value_pos((int)(slot % KBLK));
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = db * 16 + 4 * lg_a + r;
          const float v = okrow ? bf2f(Vt16[(vblk * D + d) * KBLK + pos]) : 0.f;
          st.o[s][db][r] = fmaf(p, v, st.o[s][db][r]);
        }
    }
  }

#pragma unroll
  for (int s = 0; s < SW; ++s)
    if ((slots >> s) & 1u) store_slot(g, A, qg, h, s, st.o[s], lpart[s], lane_a);
}

// Sums the key-segment partials of every special item (one workgroup per
// head and special item, the slot layout of the main kernel) and writes
// the special rows.
template <int G, int SW>
__global__ void __launch_bounds__(FWAVES * 64) attn_special_combine_kernel(Geom g, AttnArgs A, int segs,
                                                                          const float* sp_l, const f32x4* sp_o) {
  const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
  const int simd = wave & 3, s0 = (wave >> 2) * SW;
  const FastItems fi(g);
  const int h = blockIdx.x / fi.spec_items, si = blockIdx.x - h * fi.spec_items;
  const QueryGroups qg(g, fi.patch_items + si, fi.patch_items, G, simd, s0, true);
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    if (qg.row_block(s) * 16 >= qg.rows(s)) continue;  // uniform
    f32x4 o[4] = {};
    float l = 0.f;
    for (int seg = 0; seg < segs; ++seg) {
      const long long rec = spec_record(g, h, fi.patch_items + si, seg, qg, s, lane);
      l += sp_l[rec];
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] += sp_o[rec * 4 + db];
    }
    store_slot(g, A, qg, h, s, o, l, lane);
  }
}

// Zeroes the per-group flags before the bound kernel (a kernel, not a
// memset, so that the sequence can be captured in a graph).
__global__ void clear_flags_kernel(int* flags, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) flags[i] = 0;
}

// Key segments per special item: about T / k, so that a special segment
// (every tile of 1/segs of the keys for all of its groups) costs about as
// much as a tile-sparse patch item (k of the T tiles).
static int spec_segs(const Geom& g, const AttnArgs& a) {
  if (!a.sparse) return 1;
  const int nwords = (g.T + 31) / 32;
  const int k = a.keep > 0 ? a.keep : 1;
  int s = (int)((2LL * g.T + k) / (2LL * k));  // round(T / k)
  if (s > SPEC_SEGS_MAX) s = SPEC_SEGS_MAX;
  if (s > nwords) s = nwords;
  return s < 1 ? 1 : s;
}

// Units per round: one launch of the main kernel holds exactly the
// workgroups that are resident at once (FOCC per CU), so they all start
// together on the same head and walk its key tiles in the same order, and
// each XCD's L2 serves one fetch of a tile to all of its workgroups that
// use it. The kernel boundary keeps the rounds in step.
constexpr int ROUND_MAX = 512;

// Workspace of the attention entry points: flags (one int per group), -M
// per lane record, the plans of one round, and the special-segment
// partials.
struct AttnWorkspace {
  long long groups, records, sp_records;
  int plan_stride;  // plan entries per unit: words x 33 + checkpoints + special blocks
  int nckpt;        // checkpoint counters of a round
  size_t flags_off, kmax_off, negm_off, count_off, ckpt_off, plan_off, spl_off, spo_off, bytes;
  explicit AttnWorkspace(const Geom& g) {
    const FastItems fi(g);
    groups = (long long)g.H * fi.groups_per_head;
    records = groups * 4 * 64;
    sp_records = (long long)g.H * fi.spec_items * SPEC_SEGS_MAX * FG * 4 * 64;
    const int nwords = (g.T + 31) / 32;
    nckpt = nwords / CK_WORDS + 1;
    plan_stride = nwords * 33 + nckpt + g.spec_pad / KBLK;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    flags_off = 0;
    kmax_off = (size_t)groups * sizeof(int);  // H words right after the flags (cleared with them)
    negm_off = up(kmax_off + (size_t)g.H * sizeof(unsigned));
    count_off = up(negm_off + (size_t)records * sizeof(float));
    ckpt_off = up(count_off + (size_t)ROUND_MAX * 2 * sizeof(int));
    plan_off = up(ckpt_off + (size_t)nckpt * sizeof(int));
    // the last unit's final plan chunk may be read past its stride
    spl_off = up(plan_off + ((size_t)ROUND_MAX * plan_stride + PLAN_CHUNK) * sizeof(uint2));
    spo_off = up(spl_off + (size_t)sp_records * sizeof(float));
    bytes = spo_off + (size_t)sp_records * 4 * sizeof(f32x4);
  }
};

size_t attn_workspace_bytes(const Geom& g) { return AttnWorkspace(g).bytes; }

hipError_t launch_attn_exact(const Geom& g, const AttnArgs& a, const int* flags, hipStream_t s);

// Offsets, the rounds of units (plan, then main kernel), the special
// combine, then the exact kernel for flagged groups.
hipError_t launch_attn(const Geom& g, const AttnArgs& a, void* workspace, hipStream_t s) {
  const AttnWorkspace ws(g);
  char* base = (char*)workspace;
  int* flags = (int*)(base + ws.flags_off);
  unsigned* kmax2 = (unsigned*)(base + ws.kmax_off);
  float* negm = (float*)(base + ws.negm_off);
  int* count = (int*)(base + ws.count_off);
  int* ckpt = (int*)(base + ws.ckpt_off);
  uint2* plan = (uint2*)(base + ws.plan_off);
  float* spl = (float*)(base + ws.spl_off);
  f32x4* spo = (f32x4*)(base + ws.spo_off);
  const FastItems fi(g);
  const int segs = spec_segs(g, a);
  const Units units(g, segs);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int round = FOCC * cus;
  if (round > ROUND_MAX) round = ROUND_MAX;
  if (round < 1) round = 1;
  hipLaunchKernelGGL(clear_flags_kernel, dim3((unsigned)((ws.groups + g.H + 255) / 256)), dim3(256), 0, s, flags,
                     ws.groups + g.H);
  hipLaunchKernelGGL(key_norm_max_kernel, dim3(KN_BLOCKS, g.H), dim3(256), 0, s, g, a, kmax2);
  hipLaunchKernelGGL((attn_bound_kernel<FG, FSLOTS>), dim3(fi.total), dim3(FWAVES * 64), 0, s, g, a, negm, flags,
                     (const unsigned*)kmax2);
  for (int u0 = 0; u0 < units.total; u0 += round) {
    const int n = units.total - u0 < round ? units.total - u0 : round;
    int patch_units = 0;  // units of the round that are patch items (they meet at the checkpoints)
    for (int u = u0; u < u0 + n;) {
      const int b = u % units.per_head, sp = fi.spec_items * segs;
      const int end = u - b + units.per_head < u0 + n ? u - b + units.per_head : u0 + n;
      const int first_patch = u - b + sp;
      if (end > first_patch) patch_units += end - (u > first_patch ? u : first_patch);
      u = end;
    }
    hipLaunchKernelGGL(attn_plan_kernel<FG>, dim3((n + 3) / 4), dim3(256), 0, s, g, a, segs, u0, n, plan, count,
                       ws.plan_stride, ckpt, ws.nckpt);
    hipLaunchKernelGGL((attn_main_kernel<FG, FSLOTS>), dim3(n), dim3(FWAVES * 64), 0, s, g, a, segs, u0,
                       (const uint2*)plan, (const int*)count, ws.plan_stride, (const float*)negm, spl, spo, ckpt,
                       (patch_units * FWAVES * CK_RELEASE_PCT + 99) / 100);
  }
  if (fi.spec_items > 0)
    hipLaunchKernelGGL((attn_special_combine_kernel<FG, FSLOTS>), dim3(g.H * fi.spec_items), dim3(FWAVES * 64), 0,
                       s, g, a, segs, (const float*)spl, (const f32x4*)spo);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_exact(g, a, flags, s);
}

}  // namespace zebra
