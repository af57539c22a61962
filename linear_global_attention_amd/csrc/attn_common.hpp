// Shared pieces of the two attention kernels (attn.hip: fixed per-row
// softmax offsets; attn_exact.hip: online softmax for the rows the first
// one flags): LDS staging, fragment loads, work-item geometry.
#pragma once

#include "common.hpp"

namespace zebra {

constexpr int NWAVES = 4;
constexpr int ATT_THREADS = 64 * NWAVES;
constexpr int ATTN_GROUPS = 5;      // query groups per workgroup (fits 2 workgroups per CU)
constexpr float QK_LOG2 = 1.4426950408889634f * 0.125f;  // log2(e) / sqrt(64)
constexpr float SAFE_GAP = 100.0f;  // largest allowed bound - own-logit gap (log2 units)
constexpr int LDS_BUF = 16384;      // one staged item: keys [0, 8K), values [8K, 16K)
constexpr int LDS_V = 8192;
constexpr int NBUF = 4;             // LDS ring of the exact kernel
// Fast kernels: FOCC workgroups of FWAVES waves per CU; each workgroup owns
// FG query groups, each wave FSLOTS 16-row slots of them.
constexpr int FG = 5;
constexpr int FWAVES = 4;
constexpr int FOCC = 2;
constexpr int FSLOTS = FG * 4 / FWAVES;
constexpr int FNBUF = 4;            // LDS ring per workgroup (16 KB items)
static_assert(FG * 4 % FWAVES == 0 && (FWAVES == 4 || FWAVES == 8), "fast kernel layout");
constexpr int LOADS_PER_ITEM = 4;   // async 1 KB loads per wave per item

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef void __attribute__((address_space(3))) lds_void;
// Bitmap words are read through the constant address space so the uniform
// loads are scalar (lgkmcnt): a vector load would share vmcnt with the
// in-flight async tile loads and its wait would drain the prefetch ring.
typedef const unsigned __attribute__((address_space(4)))* cmask_ptr;

__device__ __forceinline__ float xsum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xmax16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A wave-uniform value in a scalar register (table reads indexed by it then
// become scalar loads).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Async copy of 8 KB of key rows (128 B each) into LDS at `dst`, swizzled:
// 16-byte column c' of key row k holds column c' ^ (k%8). A source of
// `bytes` < 8 KB is repeated (only its first `bytes` are read back). NW
// waves share the copy (1 KB per wave per load).
template <int NW = NWAVES>
__device__ __forceinline__ void stage_keys(char* dst, const char* src, int bytes, int wave, int lane) {
#pragma unroll
  for (int c = wave; c < 8; c += NW) {
    const int P = (c * 1024) % bytes + lane * 16;
    const int key = P >> 7, col = (P >> 4) & 7;
    const char* s = src + key * 128 + ((col ^ (key & 7)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)s, (lds_void*)(dst + c * 1024), 16, 0, 0);
  }
}

// Async copy of 8 KB of value blocks ([64][32] bf16, 4 KB each) into LDS,
// swizzled: 16-byte column c' of channel row d holds column c' ^ ((d/2)%4).
template <int NW = NWAVES>
__device__ __forceinline__ void stage_vals(char* dst, const char* src, int bytes, int wave, int lane) {
#pragma unroll
  for (int c = wave; c < 8; c += NW) {
    const int P = (c * 1024) % bytes + lane * 16;
    const int d = (P >> 6) & 63, col = (P >> 4) & 3;
    const char* s = src + (P & ~63) + ((col ^ ((d >> 1) & 3)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)s, (lds_void*)(dst + c * 1024), 16, 0, 0);
  }
}

// Workgroup barrier of the staging ring: this wave's LDS writes done
// (lgkmcnt(0)), compiler-only memory fences, s_barrier. Unlike
// __syncthreads() it leaves vmcnt alone, so later items' loads stay in flight.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most `later` staged items' loads are still in flight.
__device__ __forceinline__ void wait_loads(int later) {
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;  // vmcnt(0)
    case 1: __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS_PER_ITEM); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LOADS_PER_ITEM)); break;
  }
}

// Key fragments of one 32-key block (rows key0..key0+31 of the staged keys).
__device__ __forceinline__ void load_kfrag(const char* kb, int key0, int lane, bf16x8 kf[2][2]) {
  const int g = lane >> 4, tl = lane & 15;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int key = key0 + h2 * 16 + tl;
#pragma unroll
    for (int ds = 0; ds < 2; ++ds)
      kf[h2][ds] = *(const bf16x8*)(kb + key * 128 + (((ds * 4 + g) ^ (key & 7)) << 4));
  }
}

// Value fragments of one staged value block ([64][32], rows of 64 B).
__device__ __forceinline__ void load_vfrag(const char* vb, int lane, bf16x8 vf[4]) {
  const int g = lane >> 4, tl = lane & 15;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 16 + tl;
    vf[db] = *(const bf16x8*)(vb + d * 64 + ((g ^ ((d >> 1) & 3)) << 4));
  }
}

// Lane's 8 values of a 32-float table row staged unswizzled (a row whose
// index is a multiple of 8): keys 4g..4g+3 and 16+4g..16+4g+3.
__device__ __forceinline__ void load_row8(const char* row, int lane, float v[8]) {
  const int g = lane >> 4;
  const float4 a = *(const float4*)(row + 16 * g);
  const float4 b = *(const float4*)(row + 64 + 16 * g);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Bit i set when the lane's value i (keys 4g+i, then 16+4g+i-4) is < nvalid.
__device__ __forceinline__ unsigned lane_valid_mask(int nvalid, int lane) {
  if (nvalid >= 32) return 0xFFu;
  const int g = lane >> 4;
  unsigned m = 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m |= (4 * g + r < nvalid ? 1u : 0u) << r;
    m |= (16 + 4 * g + r < nvalid ? 1u : 0u) << (4 + r);
  }
  return m;
}

// The query groups of one work item (G groups), seen from one wave that
// holds slots i = 0.. for groups s = s0 + i; slot i is group tile(i) =
// gid0 + i * stride. Patch item: G query tiles, either consecutive ones
// (stride 1) or, with by_position, the tiles at one tile position in G
// frames of the same parity, two apart (stride = two frames' tiles: the
// same image region seen from nearby views keeps similar key tiles, so the
// item's groups share more of the tiles it stages; on the tile-centroid
// inputs a query tile's kept set overlaps most with the one two frames
// away, whose neighbouring frames it shares). Items per tile position: two
// per 2G frames (even and odd frames), the last pair possibly short. Special
// item: groups of 64 special rows. Row block j (16 rows) of group s belongs to the wave with `wave` ==
// (s + j) % 4 (the SIMD index when two waves share a SIMD).
struct QueryGroups {
  const Geom& g;
  bool patch;
  int gid0;
  int stride;
  int wave;
  int s0;
  __device__ QueryGroups(const Geom& g_, int item, int patch_items, int G, int wave_, int s0_ = 0,
                         bool by_position = false)
      : g(g_), patch(item < patch_items), wave(wave_), s0(s0_) {
    if (!patch) {
      gid0 = (item - patch_items) * G + s0_;
      stride = 1;
    } else if (by_position) {
      const int nfb = 2 * ((g.F + 2 * G - 1) / (2 * G));  // items per tile position
      const int u = item / nfb, b = item - u * nfb;
      gid0 = ((b >> 1) * 2 * G + (b & 1) + 2 * s0_) * g.tpf + u;
      stride = 2 * g.tpf;
    } else {
      gid0 = item * G + s0_;
      stride = 1;
    }
  }
  __device__ int tile(int s) const { return gid0 + s * stride; }
  __device__ int rows(int s) const {
    const int id = tile(s);
    if (patch) return id < g.T ? tile_n(g, id % g.tpf) : 0;
    return max(0, min(64, g.nspec - id * 64));
  }
  __device__ int row_block(int s) const { return (wave - s0 - s) & 3; }
  // token index of row j of group s
  __device__ long long token(int s, int j) const {
    const int id = tile(s);
    if (patch) {
      const int f = id / g.tpf, tl = id - f * g.tpf;
      const int a = tl / g.tc, b = tl - a * g.tc;
      const int tw = tile_w(g, tl);
      const int r = TILE * a + j / tw, c = TILE * b + j % tw;
      return (long long)f * g.tok_pf + g.S + (long long)r * g.C + c;
    }
    const int i = id * 64 + j;
    return (long long)(i / g.S) * g.tok_pf + (i % g.S);
  }
  // packed slot of the row's own key (in Kt/Vt for patch rows, Ks/Vs else)
  __device__ long long own_slot(int s, int j) const {
    const int id = tile(s);
    if (patch) {
      const int f = id / g.tpf, tl = id - f * g.tpf;
      return (long long)f * g.slots_pf + tile_off(g, tl) + j;
    }
    return (long long)id * 64 + j;
  }
};

// Work items of one attention launch: per head, ceil(T/G) patch items then
// ceil(ceil(nspec/64)/G) special items.
struct ItemCounts {
  int patch_items, per_head, total;
  __host__ ItemCounts(const Geom& g, int G) {
    patch_items = (g.T + G - 1) / G;
    const int spec_groups = (g.nspec + 63) / 64;
    per_head = patch_items + (spec_groups + G - 1) / G;
    total = per_head * g.H;
  }
};

// Work items of the fast kernels (FG groups each), per head: the special
// items first, then the patch items (grouped by tile position: FG
// consecutive frames at one tile position). Groups of a head: T patch query
// tiles, then ceil(nspec/64) special groups.
struct FastItems {
  int spec_items, patch_items, per_head, total, groups_per_head;
  __host__ __device__ explicit FastItems(const Geom& g) {
    patch_items = g.tpf * 2 * ((g.F + 2 * FG - 1) / (2 * FG));
    const int sg = (g.nspec + 63) / 64;
    spec_items = (sg + FG - 1) / FG;
    per_head = spec_items + patch_items;
    total = per_head * g.H;
    groups_per_head = g.T + sg;
  }
};

// Work units of the main attention kernel, per head: every special item
// split into `segs` key segments (units item * segs + seg, so the segments
// of one item run side by side), then the patch items. A special group sees
// every key, so splitting its keys keeps a special unit about as long as a
// patch unit; the segments' partial sums are added afterwards.
constexpr int SPEC_SEGS_MAX = 8;
struct Units {
  int segs, per_head, total;
  __host__ __device__ Units(const Geom& g, int segs_) : segs(segs_) {
    const FastItems fi(g);
    per_head = fi.spec_items * segs + fi.patch_items;
    total = per_head * g.H;
  }
};

struct Unit {
  int h, item, seg;  // item in QueryGroups numbering; seg = -1 for a patch item
  __device__ Unit(const Geom& g, int segs, int u) {
    const FastItems fi(g);
    const int per_head = fi.spec_items * segs + fi.patch_items;
    h = u / per_head;
    const int b = u - h * per_head;
    if (b < fi.spec_items * segs) {
      const int si = b / segs;
      seg = b - si * segs;
      item = fi.patch_items + si;
    } else {
      seg = -1;
      item = b - fi.spec_items * segs;
    }
  }
};

// Key words [w0, w1) of segment `seg` (seg < 0: every word).
__host__ __device__ inline void seg_words(int nwords, int segs, int seg, int& w0, int& w1) {
  if (seg < 0) {
    w0 = 0;
    w1 = nwords;
  } else {
    w0 = (int)((long long)nwords * seg / segs);
    w1 = (int)((long long)nwords * (seg + 1) / segs);
  }
}

}  // namespace zebra
