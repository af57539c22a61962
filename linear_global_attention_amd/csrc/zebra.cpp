// libzebra host side: argument validation, tile geometry, buffer sizing and
// kernel launches behind the C ABI declared in include/zebra.h.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/zebra.h"
#include "common.hpp"

namespace zebra {
hipError_t launch_pack(const Geom&, const u16*, const u16*, u16*, u16*, u16*, u16*, double*, float*, float*,
                       u16*, hipStream_t);
hipError_t launch_landmarks(const Geom&, const u16*, const u16*, double*, float*, float*, u16*,
                            hipStream_t);
size_t select_workspace_bytes(const Geom&);
hipError_t launch_select(const Geom&, int, const u16*, const double*, int*, unsigned*, double*,
                         void*, hipStream_t);
hipError_t launch_attn(const Geom&, const AttnArgs&, void*, hipStream_t);
size_t attn_workspace_bytes(const Geom&);
size_t linear_workspace_bytes(const Geom&);
size_t linear_bwd_workspace_bytes(const Geom&);
size_t sparse_bwd_workspace_bytes(const Geom&);
hipError_t launch_sparse_bwd(const Geom&, int, const u16*, const u16*, const u16*, const u16*, long long, long long,
                             const u16*, const double*, const float*, const int*, const unsigned*, u16*, u16*, u16*,
                             void*, hipStream_t);
hipError_t launch_linear_bwd(const Geom&, float, float, const u16*, const u16*, const u16*, const float*,
                             const float*, const float*, const u16*, u16*, u16*, u16*, void*, hipStream_t);
hipError_t launch_linear(const Geom&, float, float, const u16*, const u16*, const u16*,
                         const float*, const float*, const float*, const float*, const float*,
                         u16*, void*, hipStream_t);
size_t affine_workspace_bytes(const Geom&);
hipError_t launch_affine_stats(const Geom&, const u16*, const u16*, double*, void*, hipStream_t);
hipError_t launch_qk_prologue(const Geom&, const u16*, const float*, float, float, u16*, hipStream_t);
hipError_t launch_frame_attn(const Geom&, const u16*, const u16*, const u16*, const u16*, const u16*, u16*,
                             hipStream_t);
hipError_t launch_coverage(const Geom&, const u16*, const u16*, const u16*, const u16*, const unsigned*, float*,
                           float*, hipStream_t);
}  // namespace zebra

using namespace zebra;

namespace {

thread_local std::string g_err;

zebra_status fail(zebra_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// Fills g from L; returns ZEBRA_OK or an error (message set).
zebra_status make_geom(const zebra_layout* L, Geom& g) {
  if (!L) return fail(ZEBRA_ERR_INVALID_ARG, "layout is NULL");
  if (L->head_dim != D) return fail(ZEBRA_ERR_UNSUPPORTED, "head_dim must be 64");
  if (L->frames < 1 || L->heads < 1 || L->specials < 0 || L->rows < 1 || L->cols < 1)
    return fail(ZEBRA_ERR_INVALID_ARG, "frames, heads, rows, cols must be >= 1, specials >= 0");
  if (L->rows > MAX_GRID || L->cols > MAX_GRID)
    return fail(ZEBRA_ERR_UNSUPPORTED, "patch grid larger than 128 x 128");
  if (L->heads > 65535) return fail(ZEBRA_ERR_UNSUPPORTED, "more than 65535 heads");
  memset(&g, 0, sizeof(g));
  g.F = L->frames;
  g.S = L->specials;
  g.R = L->rows;
  g.C = L->cols;
  g.H = L->heads;
  g.tr = (g.R + TILE - 1) / TILE;
  g.tc = (g.C + TILE - 1) / TILE;
  g.tpf = g.tr * g.tc;
  const long long T = (long long)g.F * g.tpf;
  g.tok_pf = g.S + g.R * g.C;
  g.N = (long long)g.F * g.tok_pf;
  if (T > (1LL << 30) || g.N > (1LL << 40) || T * g.tpf >= (1LL << 32))
    return fail(ZEBRA_ERR_UNSUPPORTED, "sequence too long");
  g.T = (int)T;
  g.tpf_magic = g.tpf >= 2 ? (unsigned)((1ULL << 32) / (unsigned)g.tpf + 1) : 0u;
  int off = 0;
  for (int a = 0; a < g.tr; ++a)
    for (int b = 0; b < g.tc; ++b) {
      const int tl = a * g.tc + b;
      const int th = (g.R - TILE * a) < TILE ? (g.R - TILE * a) : TILE;
      const int tw = (g.C - TILE * b) < TILE ? (g.C - TILE * b) : TILE;
      g.tile[tl] = off | (th << 20) | (tw << 24);
      off += pad32(th * tw);
    }
  g.slots_pf = off;
  g.slots = (long long)g.F * g.slots_pf;
  const long long nspec = (long long)g.F * g.S;
  if (nspec > (1LL << 30)) return fail(ZEBRA_ERR_UNSUPPORTED, "too many special tokens");
  g.nspec = (int)nspec;
  g.spec_pad = pad32(g.nspec);
  g.T_pad = pad32(g.T);
  const long long rowdef = (long long)g.H * D;
  const long long st[4] = {L->tok_stride, L->head_stride, L->out_tok_stride, L->out_head_stride};
  for (int i = 0; i < 4; ++i)
    if (st[i] != 0 && (st[i] < D || st[i] % 8 != 0 || st[i] > (1LL << 40)))
      return fail(ZEBRA_ERR_INVALID_ARG, "strides must be 0 or multiples of 8 elements, at least 64");
  g.in_tok = L->tok_stride ? L->tok_stride : rowdef;
  g.in_head = L->head_stride ? L->head_stride : D;
  g.out_tok = L->out_tok_stride ? L->out_tok_stride : rowdef;
  g.out_head = L->out_head_stride ? L->out_head_stride : D;
  return ZEBRA_OK;
}

// 16-byte alignment of a caller's tensor pointer (the kernels move rows in
// 16-byte pieces).
bool misaligned(const void* p) { return p && ((uintptr_t)p & 15u) != 0; }

int64_t keep_count(const Geom& g, double y) {
  if (!(y >= 0.0 && y <= 1.0)) return -1;
  double k = nearbyint((1.0 - y) * (double)g.T);  // round half to even (default mode)
  if (k < 0) k = 0;
  if (k > g.T) k = g.T;
  return (int64_t)k;
}

size_t buf_bytes(const Geom& g, int64_t k, int which) {
  const size_t H = (size_t)g.H, T = (size_t)g.T;
  switch (which) {
    case ZEBRA_BUF_KT:
    case ZEBRA_BUF_VT: return H * (size_t)g.slots * D * sizeof(u16);
    case ZEBRA_BUF_KS:
    case ZEBRA_BUF_VS: return H * (size_t)(g.spec_pad ? g.spec_pad : KBLK) * D * sizeof(u16);
    case ZEBRA_BUF_KBAR: return H * T * D * sizeof(double);
    case ZEBRA_BUF_VBAR: return H * T * D * sizeof(float);
    case ZEBRA_BUF_LOGN: return T * sizeof(float);
    case ZEBRA_BUF_LM: return H * (size_t)g.T_pad * LM_BYTES_PER_TILE;
    case ZEBRA_BUF_SEL: return H * T * (size_t)(k > 0 ? k : 1) * sizeof(int32_t);
    case ZEBRA_BUF_SELMASK: return H * T * ((T + 31) / 32) * sizeof(uint32_t);
    case ZEBRA_BUF_GAP: return H * T * sizeof(double);
    case ZEBRA_BUF_WORKSPACE: {
      size_t m = select_workspace_bytes(g);
      const size_t b = linear_workspace_bytes(g), c = attn_workspace_bytes(g), f = affine_workspace_bytes(g);
      const size_t lb = linear_bwd_workspace_bytes(g);
      if (lb > m) m = lb;
      if (b > m) m = b;
      if (c > m) m = c;
      if (f > m) m = f;
      return m;
    }
    case ZEBRA_BUF_BWD_WORKSPACE: {
      const size_t w = buf_bytes(g, k, ZEBRA_BUF_WORKSPACE), sb = sparse_bwd_workspace_bytes(g);
      return sb > w ? sb : w;
    }
    default: return 0;
  }
}

zebra_status check_common(const zebra_args* a, Geom& g) {
  if (!a) return fail(ZEBRA_ERR_INVALID_ARG, "args is NULL");
  const zebra_status s = make_geom(&a->L, g);
  if (s != ZEBRA_OK) return s;
  if (misaligned(a->q) || misaligned(a->k) || misaligned(a->v) || misaligned(a->out))
    return fail(ZEBRA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  return ZEBRA_OK;
}

#define NEED(ptr, name) \
  if (!(ptr)) return fail(ZEBRA_ERR_INVALID_ARG, std::string(name) + " is NULL")

zebra_status validate(const zebra_args* a, int op, Geom& g, int64_t& k) {
  zebra_status s = check_common(a, g);
  if (s != ZEBRA_OK) return s;
  k = keep_count(g, a->y);
  switch (op) {
    case ZEBRA_OP_PACK:
      NEED(a->k, "k");
      NEED(a->v, "v");
      NEED(a->kt, "kt");
      NEED(a->vt, "vt");
      NEED(a->ks, "ks");
      NEED(a->vs, "vs");
      if (a->kbar || a->vbar || a->logn || a->lm) {  // landmarks in the same pass
        NEED(a->kbar, "kbar");
        NEED(a->vbar, "vbar");
        NEED(a->logn, "logn");
        NEED(a->lm, "lm");
      }
      break;
    case ZEBRA_OP_LANDMARKS:
      NEED(a->kt, "kt");
      NEED(a->vt, "vt");
      NEED(a->kbar, "kbar");
      NEED(a->vbar, "vbar");
      NEED(a->logn, "logn");
      NEED(a->lm, "lm");
      break;
    case ZEBRA_OP_SELECT:
      if (k < 0) return fail(ZEBRA_ERR_INVALID_ARG, "y must lie in [0, 1]");
      if (g.T > 32768) return fail(ZEBRA_ERR_UNSUPPORTED, "selection supports at most 32768 tiles");
      NEED(a->q, "q");
      NEED(a->kbar, "kbar");
      NEED(a->sel, "sel");
      NEED(a->selmask, "selmask");
      NEED(a->workspace, "workspace");
      if (a->workspace_bytes < select_workspace_bytes(g))
        return fail(ZEBRA_ERR_WORKSPACE, "workspace too small for zebra_select_tiles");
      break;
    case ZEBRA_OP_SPARSE:
      if (k < 0) return fail(ZEBRA_ERR_INVALID_ARG, "y must lie in [0, 1]");
      NEED(a->q, "q");
      NEED(a->out, "out");
      NEED(a->kt, "kt");
      NEED(a->vt, "vt");
      NEED(a->ks, "ks");
      NEED(a->vs, "vs");
      NEED(a->lm, "lm");
      NEED(a->logn, "logn");
      NEED(a->selmask, "selmask");
      NEED(a->workspace, "workspace");
      if (a->workspace_bytes < attn_workspace_bytes(g))
        return fail(ZEBRA_ERR_WORKSPACE, "workspace too small for zebra_sparse_attn");
      break;
    case ZEBRA_OP_LINEAR:
      NEED(a->q, "q");
      NEED(a->k, "k");
      NEED(a->v, "v");
      NEED(a->out, "out");
      NEED(a->workspace, "workspace");
      if (a->workspace_bytes < linear_workspace_bytes(g))
        return fail(ZEBRA_ERR_WORKSPACE, "workspace too small for zebra_linear_attn");
      if (a->mu && !a->W) {
        /* allowed: W = I makes mu cancel */
      }
      break;
    case ZEBRA_OP_DENSE:
      NEED(a->q, "q");
      NEED(a->k, "k");
      NEED(a->v, "v");
      NEED(a->out, "out");
      NEED(a->kt, "kt");
      NEED(a->vt, "vt");
      NEED(a->ks, "ks");
      NEED(a->vs, "vs");
      NEED(a->kbar, "kbar");
      NEED(a->vbar, "vbar");
      NEED(a->logn, "logn");
      NEED(a->lm, "lm");
      NEED(a->workspace, "workspace");
      if (a->workspace_bytes < attn_workspace_bytes(g))
        return fail(ZEBRA_ERR_WORKSPACE, "workspace too small for zebra_dense_attn");
      break;
    case ZEBRA_OP_AFFINE_STATS:
      NEED(a->out, "out (the linear outputs)");
      NEED(a->workspace, "workspace");
      if (a->workspace_bytes < affine_workspace_bytes(g))
        return fail(ZEBRA_ERR_WORKSPACE, "workspace too small for zebra_affine_stats");
      break;
    case ZEBRA_OP_PROLOGUE:
      NEED(a->q, "q");
      NEED(a->k, "k");
      break;
    case ZEBRA_OP_FRAME:
      if (g.F > 65535) return fail(ZEBRA_ERR_UNSUPPORTED, "frame-wise attention supports at most 65535 frames");
      NEED(a->q, "q");
      NEED(a->k, "k");
      NEED(a->v, "v");
      NEED(a->out, "out");
      NEED(a->kt, "kt");
      NEED(a->vt, "vt");
      NEED(a->ks, "ks");
      NEED(a->vs, "vs");
      break;
    case ZEBRA_OP_LINEAR_BWD:
      NEED(a->q, "q");
      NEED(a->k, "k");
      NEED(a->v, "v");
      NEED(a->workspace, "workspace");
      if (a->workspace_bytes < linear_bwd_workspace_bytes(g))
        return fail(ZEBRA_ERR_WORKSPACE, "workspace too small for zebra_linear_attn_bwd");
      break;
    case ZEBRA_OP_SPARSE_BWD:
      if (k < 0) return fail(ZEBRA_ERR_INVALID_ARG, "y must lie in [0, 1]");
      if (g.T > 32768) return fail(ZEBRA_ERR_UNSUPPORTED, "the sparse backward supports at most 32768 tiles");
      if (g.N >= (1LL << 31)) return fail(ZEBRA_ERR_UNSUPPORTED, "the sparse backward supports fewer than 2^31 tokens");
      // its kernels address a key tile's rows by 32-bit element offsets
      // from the tile's first row
      if ((long long)TILE * g.C * std::max(g.in_tok, g.out_tok) >= (1LL << 31))
        return fail(ZEBRA_ERR_UNSUPPORTED,
                    "the sparse backward needs 8 patch rows of q, k, v and dout to span fewer than 2^31 elements");
      NEED(a->q, "q");
      NEED(a->k, "k");
      NEED(a->v, "v");
      NEED(a->lm, "lm");
      NEED(a->kbar, "kbar");
      NEED(a->vbar, "vbar");
      NEED(a->sel, "sel");
      NEED(a->selmask, "selmask");
      NEED(a->workspace, "workspace");
      if (a->workspace_bytes < sparse_bwd_workspace_bytes(g))
        return fail(ZEBRA_ERR_WORKSPACE, "workspace too small for zebra_sparse_attn_bwd (ZEBRA_BUF_BWD_WORKSPACE)");
      break;
    case ZEBRA_OP_COVERAGE:
      if (k < 0) return fail(ZEBRA_ERR_INVALID_ARG, "y must lie in [0, 1]");
      NEED(a->q, "q");
      NEED(a->kt, "kt");
      NEED(a->ks, "ks");
      NEED(a->lm, "lm");
      NEED(a->selmask, "selmask");
      break;
    default:
      return fail(ZEBRA_ERR_INVALID_ARG, "unknown operation");
  }
  g_err.clear();
  return ZEBRA_OK;
}

zebra_status hip_result(hipError_t e, const char* what);

// Device scratch of zebra_linear_attn_noalloc: the linear stage's partial KV
// states, their fp64 sum and the folded state, in place of a workspace. One
// copy per device, held until the process ends. Host code never passes
// `scratch` itself to a kernel (on the host it names a stand-in, not device
// memory): it takes the device address that hipGetSymbolAddress returns, once
// per device, with that device current.
static __device__ __align__(256) char scratch[ZEBRA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's scratch address (looked up on its first use).
zebra_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_result(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(ZEBRA_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_result(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(ZEBRA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ZEBRA_OK;
}

zebra_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    char buf[256];
    snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
    return fail(ZEBRA_ERR_HIP, buf);
  }
  return ZEBRA_OK;
}

}  // namespace

extern "C" {

zebra_status zebra_validate(const zebra_args* a, int op) {
  Geom g;
  int64_t k;
  return validate(a, op, g, k);
}

size_t zebra_buffer_bytes(const zebra_layout* L, double y, int which) {
  Geom g;
  if (make_geom(L, g) != ZEBRA_OK) return 0;
  const int64_t k = keep_count(g, y);
  if (k < 0 && which == ZEBRA_BUF_SEL) return 0;
  return buf_bytes(g, k, which);
}

int64_t zebra_keep_count(const zebra_layout* L, double y) {
  Geom g;
  if (make_geom(L, g) != ZEBRA_OK) return -1;
  return keep_count(g, y);
}

int64_t zebra_num_tiles(const zebra_layout* L) {
  Geom g;
  if (make_geom(L, g) != ZEBRA_OK) return -1;
  return g.T;
}

const char* zebra_last_error(void) { return g_err.c_str(); }

const char* zebra_version(void) { return "zebra-mi355x 0.1 (gfx950)"; }

zebra_status zebra_pack_tiles(const zebra_args* a, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_PACK, g, k);
  if (s != ZEBRA_OK) return s;
  return hip_result(launch_pack(g, (const u16*)a->k, (const u16*)a->v, (u16*)a->kt, (u16*)a->vt,
                                (u16*)a->ks, (u16*)a->vs, a->kbar, a->vbar, a->logn, (u16*)a->lm,
                                (hipStream_t)stream),
                    "zebra_pack_tiles");
}

zebra_status zebra_landmarks(const zebra_args* a, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_LANDMARKS, g, k);
  if (s != ZEBRA_OK) return s;
  return hip_result(launch_landmarks(g, (const u16*)a->kt, (const u16*)a->vt, a->kbar, a->vbar,
                                     a->logn, (u16*)a->lm, (hipStream_t)stream),
                    "zebra_landmarks");
}

zebra_status zebra_select_tiles(const zebra_args* a, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_SELECT, g, k);
  if (s != ZEBRA_OK) return s;
  return hip_result(launch_select(g, (int)k, (const u16*)a->q, a->kbar, (int*)a->sel,
                                  (unsigned*)a->selmask, a->gap, a->workspace,
                                  (hipStream_t)stream),
                    "zebra_select_tiles");
}

zebra_status zebra_sparse_attn(const zebra_args* a, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_SPARSE, g, k);
  if (s != ZEBRA_OK) return s;
  AttnArgs A{(const u16*)a->q, (u16*)a->out, (const u16*)a->kt, (const u16*)a->vt,
             (const u16*)a->ks, (const u16*)a->vs, (const u16*)a->lm, a->logn,
             (const unsigned*)a->selmask, (g.T + 31) / 32, 1, (int)k};
  return hip_result(launch_attn(g, A, a->workspace, (hipStream_t)stream), "zebra_sparse_attn");
}

zebra_status zebra_dense_attn(const zebra_args* a, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_DENSE, g, k);
  if (s != ZEBRA_OK) return s;
  s = hip_result(launch_pack(g, (const u16*)a->k, (const u16*)a->v, (u16*)a->kt, (u16*)a->vt,
                             (u16*)a->ks, (u16*)a->vs, a->kbar, a->vbar, a->logn, (u16*)a->lm,
                             (hipStream_t)stream),
                 "zebra_dense_attn (pack and landmarks)");
  if (s != ZEBRA_OK) return s;
  AttnArgs A{(const u16*)a->q, (u16*)a->out, (const u16*)a->kt, (const u16*)a->vt,
             (const u16*)a->ks, (const u16*)a->vs, (const u16*)a->lm, a->logn, (const unsigned*)nullptr,
             (g.T + 31) / 32, 0, g.T};
  return hip_result(launch_attn(g, A, a->workspace, (hipStream_t)stream), "zebra_dense_attn");
}

zebra_status zebra_linear_attn(const zebra_args* a, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_LINEAR, g, k);
  if (s != ZEBRA_OK) return s;
  const float eps = a->rms_eps > 0.f ? a->rms_eps : 1e-6f;
  const float base = a->rope_base > 0.f ? a->rope_base : 100.0f;
  return hip_result(launch_linear(g, eps, base, (const u16*)a->q, (const u16*)a->k,
                                  (const u16*)a->v, a->W, a->b, a->mu, a->gq, a->gk,
                                  (u16*)a->out, a->workspace, (hipStream_t)stream),
                    "zebra_linear_attn");
}

zebra_status zebra_linear_attn_bwd(const zebra_args* a, const void* dout, void* dq, void* dk, void* dv,
                                   zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_LINEAR_BWD, g, k);
  if (s != ZEBRA_OK) return s;
  if (!dout || !dq || !dk || !dv) return fail(ZEBRA_ERR_INVALID_ARG, "dout, dq, dk and dv must be non-NULL");
  if (misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv))
    return fail(ZEBRA_ERR_INVALID_ARG, "dout, dq, dk and dv must be 16-byte aligned");
  const float eps = a->rms_eps > 0.f ? a->rms_eps : 1e-6f;
  const float base = a->rope_base > 0.f ? a->rope_base : 100.0f;
  return hip_result(launch_linear_bwd(g, eps, base, (const u16*)a->q, (const u16*)a->k, (const u16*)a->v, a->W,
                                      a->gq, a->gk, (const u16*)dout, (u16*)dq, (u16*)dk, (u16*)dv, a->workspace,
                                      (hipStream_t)stream),
                    "zebra_linear_attn_bwd");
}

zebra_status zebra_sparse_attn_bwd(const zebra_args* a, const void* dout, void* dq, void* dk, void* dv,
                                   zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_SPARSE_BWD, g, k);
  if (s != ZEBRA_OK) return s;
  if (!dout || !dq || !dk || !dv) return fail(ZEBRA_ERR_INVALID_ARG, "dout, dq, dk and dv must be non-NULL");
  if (misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv))
    return fail(ZEBRA_ERR_INVALID_ARG, "dout, dq, dk and dv must be 16-byte aligned");
  return hip_result(launch_sparse_bwd(g, (int)k, (const u16*)a->q, (const u16*)a->k, (const u16*)a->v,
                                      (const u16*)dout, g.out_tok, g.out_head, (const u16*)a->lm, a->kbar, a->vbar,
                                      (const int*)a->sel, (const unsigned*)a->selmask, (u16*)dq, (u16*)dk, (u16*)dv,
                                      a->workspace, (hipStream_t)stream),
                    "zebra_sparse_attn_bwd");
}

zebra_status zebra_linear_attn_noalloc(const zebra_args* a, zebra_stream stream) {
  Geom g;
  zebra_status s = check_common(a, g);
  if (s != ZEBRA_OK) return s;
  NEED(a->q, "q");
  NEED(a->k, "k");
  NEED(a->v, "v");
  NEED(a->out, "out");
  const size_t need = linear_workspace_bytes(g);
  if (need > (size_t)ZEBRA_NOALLOC_SCRATCH_BYTES) {
    char buf[160];
    snprintf(buf, sizeof buf, "zebra_linear_attn_noalloc: layout needs %zu scratch bytes, the maximum is %zu",
             need, (size_t)ZEBRA_NOALLOC_SCRATCH_BYTES);
    return fail(ZEBRA_ERR_WORKSPACE, buf);
  }
  void* ws = nullptr;
  s = device_scratch(&ws);
  if (s != ZEBRA_OK) return s;
  g_err.clear();
  const float eps = a->rms_eps > 0.f ? a->rms_eps : 1e-6f;
  const float base = a->rope_base > 0.f ? a->rope_base : 100.0f;
  return hip_result(launch_linear(g, eps, base, (const u16*)a->q, (const u16*)a->k,
                                  (const u16*)a->v, a->W, a->b, a->mu, a->gq, a->gk,
                                  (u16*)a->out, ws, (hipStream_t)stream),
                    "zebra_linear_attn_noalloc");
}

zebra_status zebra_qk_prologue(const zebra_args* a, void* q_out, void* k_out, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_PROLOGUE, g, k);
  if (s != ZEBRA_OK) return s;
  if (!q_out || !k_out) return fail(ZEBRA_ERR_INVALID_ARG, "q_out and k_out must be non-NULL");
  if (misaligned(q_out) || misaligned(k_out)) return fail(ZEBRA_ERR_INVALID_ARG, "q_out and k_out must be 16-byte aligned");
  const float eps = a->rms_eps > 0.f ? a->rms_eps : 1e-6f;
  const float base = a->rope_base > 0.f ? a->rope_base : 100.0f;
  s = hip_result(launch_qk_prologue(g, (const u16*)a->q, a->gq, eps, base, (u16*)q_out, (hipStream_t)stream),
                 "zebra_qk_prologue (q)");
  if (s != ZEBRA_OK) return s;
  return hip_result(launch_qk_prologue(g, (const u16*)a->k, a->gk, eps, base, (u16*)k_out, (hipStream_t)stream),
                    "zebra_qk_prologue (k)");
}

zebra_status zebra_frame_attn(const zebra_args* a, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_FRAME, g, k);
  if (s != ZEBRA_OK) return s;
  s = hip_result(launch_pack(g, (const u16*)a->k, (const u16*)a->v, (u16*)a->kt, (u16*)a->vt, (u16*)a->ks,
                             (u16*)a->vs, nullptr, nullptr, nullptr, nullptr, (hipStream_t)stream),
                 "zebra_frame_attn (pack)");
  if (s != ZEBRA_OK) return s;
  return hip_result(launch_frame_attn(g, (const u16*)a->q, (const u16*)a->k, (const u16*)a->v, (const u16*)a->kt,
                                      (const u16*)a->vt, (u16*)a->out, (hipStream_t)stream),
                    "zebra_frame_attn");
}

zebra_status zebra_coverage(const zebra_args* a, float* coverage, float* lm_error, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_COVERAGE, g, k);
  if (s != ZEBRA_OK) return s;
  if (!coverage || !lm_error) return fail(ZEBRA_ERR_INVALID_ARG, "coverage and lm_error must be non-NULL");
  return hip_result(launch_coverage(g, (const u16*)a->q, (const u16*)a->kt, (const u16*)a->ks, (const u16*)a->lm,
                                    (const unsigned*)a->selmask, coverage, lm_error, (hipStream_t)stream),
                    "zebra_coverage");
}

zebra_status zebra_affine_stats(const zebra_args* a, const void* teacher, double* stats, zebra_stream stream) {
  Geom g;
  int64_t k;
  zebra_status s = validate(a, ZEBRA_OP_AFFINE_STATS, g, k);
  if (s != ZEBRA_OK) return s;
  if (!teacher) return fail(ZEBRA_ERR_INVALID_ARG, "teacher is NULL");
  if (misaligned(teacher)) return fail(ZEBRA_ERR_INVALID_ARG, "teacher must be 16-byte aligned");
  if (!stats) return fail(ZEBRA_ERR_INVALID_ARG, "stats is NULL");
  return hip_result(launch_affine_stats(g, (const u16*)a->out, (const u16*)teacher, stats, a->workspace,
                                        (hipStream_t)stream),
                    "zebra_affine_stats");
}

zebra_status zebra_affine_solve(const double* stats, double lambda_rel, float* W, float* b, float* mu) {
  if (!stats || !W || !b || !mu) return fail(ZEBRA_ERR_INVALID_ARG, "stats, W, b and mu must be non-NULL");
  if (!(lambda_rel >= 0.0) || !isfinite(lambda_rel)) return fail(ZEBRA_ERR_INVALID_ARG, "lambda_rel must be >= 0");
  const int d = D;
  const double n = stats[0];
  if (!(n >= 1.0)) return fail(ZEBRA_ERR_INVALID_ARG, "no samples accumulated");
  const double* so = stats + 1;
  const double* st = so + d;
  const double* oo = st + d;
  const double* ot = oo + d * d;
  double m[D], tb[D];
  for (int i = 0; i < d; ++i) {
    m[i] = so[i] / n;
    tb[i] = st[i] / n;
  }
  // centred Gram G = sum (o - m)(o - m)^T and cross term Cx = sum (o - m)(t - tb)^T
  static thread_local double G[D * D], Cx[D * D];
  double tr = 0.0;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      G[i * d + j] = oo[i * d + j] - n * m[i] * m[j];
      Cx[i * d + j] = ot[i * d + j] - n * m[i] * tb[j];
    }
  for (int i = 0; i < d; ++i) tr += G[i * d + i];
  const double lam = lambda_rel * tr / d;
  for (int i = 0; i < d; ++i) G[i * d + i] += lam;
  // Cholesky G = L L^T (lower, in place)
  for (int j = 0; j < d; ++j) {
    double s = G[j * d + j];
    for (int p = 0; p < j; ++p) s -= G[j * d + p] * G[j * d + p];
    if (!(s > 0.0)) return fail(ZEBRA_ERR_INVALID_ARG, "Gram matrix (plus ridge) is not positive definite");
    const double l = sqrt(s);
    G[j * d + j] = l;
    for (int i = j + 1; i < d; ++i) {
      double t = G[i * d + j];
      for (int p = 0; p < j; ++p) t -= G[i * d + p] * G[j * d + p];
      G[i * d + j] = t / l;
    }
  }
  // X = G^-1 Cx, column by column; W[c][a] = X[a][c]
  for (int c = 0; c < d; ++c) {
    double x[D];
    for (int i = 0; i < d; ++i) {
      double t = Cx[i * d + c];
      for (int p = 0; p < i; ++p) t -= G[i * d + p] * x[p];
      x[i] = t / G[i * d + i];
    }
    for (int i = d - 1; i >= 0; --i) {
      double t = x[i];
      for (int p = i + 1; p < d; ++p) t -= G[p * d + i] * x[p];
      x[i] = t / G[i * d + i];
    }
    for (int a = 0; a < d; ++a) W[c * d + a] = (float)x[a];
  }
  for (int i = 0; i < d; ++i) {
    b[i] = (float)(tb[i] - m[i]);
    mu[i] = (float)m[i];
  }
  g_err.clear();
  return ZEBRA_OK;
}

}  // extern "C"
