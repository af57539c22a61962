// Shared definitions of libzebra's host code and gfx950 kernels: the tile
// geometry of a multi-view sequence, the packed buffer layouts, bf16 helpers
// and MFMA vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zebra {

constexpr int D = 64;          // head dim (fixed)
constexpr int TILE = 8;        // 8x8 patches per complete tile
constexpr int MAX_GRID = 128;  // R, C <= 128
constexpr int MAX_TPF = (MAX_GRID / TILE) * (MAX_GRID / TILE);  // tiles per frame
constexpr int KBLK = 32;       // key-slot granularity of the packed layouts
constexpr int LM_KEY_BLOCK = 8192;                      // bytes per landmark key block
constexpr int LM_LOG2N_ROW = 32;                        // row of log2(n_u) in a key block
constexpr int LM_BYTES_PER_TILE = (LM_KEY_BLOCK + KBLK * D * 2) / KBLK;  // 384

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

// Geometry of one (F, S, R, C, H) layout, passed to kernels by value.
//   token of patch (f, r, c) = f*tok_pf + S + r*C + c
//   special s of frame f     = f*tok_pf + s
//   tile u = f*tpf + a*tc + b, patch rows [8a, 8a+th), cols [8b, 8b+tw)
// Packed key/value slots: tile (f, tl) starts at slot f*slots_pf +
// tile_off(tl) and owns pad32(n) slots (n = th*tw real tokens, rest zero).
struct Geom {
  int F, S, R, C, H;
  int tr, tc, tpf;     // tile rows/cols per frame, tiles per frame
  int T;               // tiles
  int tok_pf;          // tokens per frame, S + R*C
  long long N;         // tokens
  int slots_pf;        // packed slots per frame
  long long slots;     // F*slots_pf
  int nspec;           // F*S special tokens
  int spec_pad;        // nspec rounded up to KBLK
  int T_pad;           // T rounded up to KBLK
  unsigned tpf_magic;  // floor(2^32 / tpf) + 1 (tpf >= 2): u / tpf = umulhi(u, magic) for u*tpf < 2^32
  // element strides: (token n, head h) row of q/k/v at n*in_tok + h*in_head,
  // of the output at n*out_tok + h*out_head
  long long in_tok, in_head, out_tok, out_head;
  // per tile of a frame: bits 0..19 first packed slot (within the frame),
  // bits 20..23 patch rows th, bits 24..27 patch columns tw. One 32-bit word
  // per tile so that uniform lookups are scalar loads.
  int tile[MAX_TPF];
};

// Frame of tile u (u / tpf without a division; exact because T * tpf < 2^32).
__device__ inline int frame_of_tile(const Geom& g, int u) {
  return g.tpf == 1 ? u : (int)__umulhi((unsigned)u, g.tpf_magic);
}

__host__ __device__ inline int tile_off(const Geom& g, int tl) { return g.tile[tl] & 0xFFFFF; }
__host__ __device__ inline int tile_h(const Geom& g, int tl) { return (g.tile[tl] >> 20) & 15; }
__host__ __device__ inline int tile_w(const Geom& g, int tl) { return (g.tile[tl] >> 24) & 15; }
__host__ __device__ inline int tile_n(const Geom& g, int tl) { return tile_h(g, tl) * tile_w(g, tl); }

// Buffer layouts (element counts are per head unless stated):
//   Kt  bf16 [H][slots][64]                    key of slot s, row-major
//   Vt  bf16 [H][slots/32][64][32]             value, d-major per 32 slots,
//                                              key k of a block at position
//                                              value_pos(k) (see below)
//   Ks  bf16 [H][spec_pad][64]
//   Vs  bf16 [H][spec_pad/32][64][32]
//   LM  per head: T_pad/32 landmark key blocks of LM_KEY_BLOCK bytes (rows
//       0..31: kbar of the block's tiles, bf16 [32][64]; row 32: 32 fp32
//       log2(n_u), -inf past the last tile; other rows zero), then T_pad/32
//       value blocks [64][32] bf16 of vbar (keys permuted by value_pos)

// Arguments of the attention kernel (tile-sparse or dense).
struct AttnArgs {
  const u16* Q;
  u16* O;
  const u16* Kt;
  const u16* Vt;
  const u16* Ks;
  const u16* Vs;
  const u16* LM;
  const float* logn;
  const unsigned* selmask;  // nullptr: every tile kept (dense)
  int nwords;               // ceil(T/32)
  int sparse;               // 1: landmarks + self key for patch groups
  int keep;                 // kept tiles per query tile (T when dense)
};

// Position of key k (0..31) inside a 32-key value block: the 8 keys
// {4g..4g+3, 16+4g..16+4g+3} of lane group g are contiguous, matching the
// k-slot order of the probabilities fed to the P.V MFMA.
__host__ __device__ inline int value_pos(int k) { return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3); }
// Inverse of value_pos.
__host__ __device__ inline int value_key(int p) { return ((p & 7) >> 2) * 16 + (p >> 3) * 4 + (p & 3); }

__host__ __device__ inline int pad32(int n) { return (n + KBLK - 1) / KBLK * KBLK; }

__device__ inline float bf2f(u16 b) { return __uint_as_float(((unsigned)b) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite here)
__device__ inline u16 f2bf(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

}  // namespace zebra
