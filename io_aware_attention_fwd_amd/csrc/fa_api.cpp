// C ABI of libfa.so: argument validation, folding of the scale, dispatch.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and needs no GPU.  The operation, layouts and error codes are
// documented in include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa_launch.h"
#include "fa_variants.h"

namespace {

constexpr float kLog2e = 1.44269504088896341f;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int elem_bytes(fa::Dtype dt) { return dt == fa::Dtype::FP8 ? 1 : 2; }

// Shape of one call: dense [B,H,N,d] (cu == nullptr) or packed [total,H,d]
// sequences delimited by cu (N = the longest sequence).
struct Layout {
  const int* cu;
  int B, H, N, total, d;
};

// Dropout settings of one call: t = 256 keeps every score (no dropout).
struct Dropout {
  uint32_t t;
  uint64_t seed;
  uint32_t offset;
};
constexpr Dropout kNoDropout{256u, 0u, 0u};

int forward(const void* q, const void* k, const void* v, void* o, float* lse, const Layout& L, float scale, int causal,
            fa::Dtype dt, float q_descale, float k_descale, float v_descale, const Dropout& drop, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  const bool packed = L.cu != nullptr;
  if (L.B < 1 || L.H < 1 || L.N < 1 || (packed && L.total < 0)) return FA_ERR_SHAPE;
  const int d = L.d;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return FA_ERR_SCALE;
  const int eb = elem_bytes(dt);
  const int ob = 2;  // O is binary16 / bfloat16 (bfloat16 for fp8 inputs)
  const int vi = fa::selected_variant(dt, d, causal != 0, L.N, drop.t < 256, packed);
  const int br = fa::kVariants[vi].qw * fa::kVariants[vi].nw;  // query rows per workgroup
  // The rows of one (sequence, head), plus the padding rows of its last tile,
  // must be addressable with 32-bit byte offsets (the kernels use buffer loads).
  const int64_t in_row = packed ? (int64_t)L.H * d * eb : (int64_t)d * eb;
  if ((int64_t)(L.N + br) * in_row >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  const int64_t n_qtiles = ((int64_t)L.N + br - 1) / br;
  // dense causal grids: one workgroup per pair of query tiles (the kernel's two jobs)
  const int64_t total_wg = (causal && !packed ? (n_qtiles + 1) / 2 : n_qtiles) * L.B * L.H;
  if (total_wg >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      (packed && !aligned(L.cu, 4)))
    return FA_ERR_ALIGN;
  const int64_t rows = packed ? (int64_t)L.total : (int64_t)L.B * L.N;  // rows per head
  const size_t in_bytes = (size_t)rows * L.H * d * eb;
  const size_t o_bytes = (size_t)rows * L.H * d * ob;
  const size_t lse_bytes = (size_t)rows * L.H * sizeof(float);
  for (const void* in : {q, k, v}) {
    if (overlap(o, o_bytes, in, in_bytes) || overlap(lse, lse_bytes, in, in_bytes)) return FA_ERR_ALIAS;
  }
  if (overlap(o, o_bytes, lse, lse_bytes)) return FA_ERR_ALIAS;

  // Fold the scale (and fp8 Q/K descales) into the exp2 multiplier; its sign
  // goes into Q's sign bits and a zero scale zeroes Q, both exact.
  const double eff = (double)scale * (double)q_descale * (double)k_descale;
  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu = L.cu;
  p.B = L.B;
  p.H = L.H;
  p.N = L.N;
  p.total = packed ? L.total : 0;
  p.n_qtiles = (int)n_qtiles;
  p.total_wg = (int)total_wg;
  if (packed) {
    p.in_batch = 0;
    p.in_head = (long long)d * eb;
    p.in_row = (int)in_row;
    p.out_batch = 0;
    p.out_head = (long long)d * ob;
    p.out_row = L.H * d * ob;
    p.lse_batch = 0;
    p.lse_head = L.total;
  } else {
    p.in_row = d * eb;
    p.in_head = (long long)L.N * p.in_row;
    p.in_batch = (long long)L.H * p.in_head;
    p.out_row = d * ob;
    p.out_head = (long long)L.N * p.out_row;
    p.out_batch = (long long)L.H * p.out_head;
    p.lse_head = L.N;
    p.lse_batch = (long long)L.H * L.N;
  }
  const uint32_t sign_bits = dt == fa::Dtype::FP8 ? 0x80808080u : 0x80008000u;
  p.q_xor = eff < 0 ? sign_bits : 0u;
  p.q_and = eff == 0 ? 0u : 0xFFFFFFFFu;
  const double c = eff == 0 ? 1.0 : fabs(eff) * (double)kLog2e;
  if (!(c <= (double)FLT_MAX)) return FA_ERR_SCALE;  // checked in double: a float conversion out of range is undefined
  p.c = (float)c;
  p.o_mul = v_descale * (float)(256.0 / drop.t);
  p.drop_t = drop.t;
  p.seed_lo = (uint32_t)drop.seed;
  p.seed_hi = (uint32_t)(drop.seed >> 32);
  p.drop_offset = drop.offset;
  p.variant = vi;

  if (packed && L.total == 0) return FA_OK;  // no rows: nothing to compute
  if (fa::launch_fwd(dt, d, causal != 0, p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

// delta == nullptr with `static_delta`: D goes to the library's static device
// workspace (fa_bwd_noalloc), looked up after every argument check.
int backward(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, float* delta, bool static_delta, int B, int H, int N, int d, float scale, int causal,
             int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || (!delta && !static_delta)) return FA_ERR_NULL_PTR;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const int64_t row = (int64_t)d * 2;
  if ((int64_t)(N + fa::kBwdRows) * row >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  const int64_t n_blocks = ((int64_t)N + fa::kBwdRows - 1) / fa::kBwdRows;
  const int64_t total_wg = n_blocks * B * H;
  if (total_wg >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (static_delta && (int64_t)B * H * N > fa::kBwdScratchRows) return FA_ERR_SCRATCH;
  for (const void* ptr : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned(ptr, 16)) return FA_ERR_ALIGN;
  if (!aligned(lse, 4) || (!static_delta && !aligned(delta, 4))) return FA_ERR_ALIGN;
  const size_t t_bytes = (size_t)B * H * N * d * 2;
  const size_t r_bytes = (size_t)B * H * N * sizeof(float);
  const void* ins[] = {q, k, v, o, lse, dout};
  const size_t in_sz[] = {t_bytes, t_bytes, t_bytes, t_bytes, r_bytes, t_bytes};
  void* outs[] = {dq, dk, dv, delta};
  const size_t out_sz[] = {t_bytes, t_bytes, t_bytes, r_bytes};
  const int n_outs = static_delta ? 3 : 4;  // the static workspace overlaps nothing the caller owns
  for (int i = 0; i < n_outs; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], out_sz[i], ins[j], in_sz[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < n_outs; ++j)
      if (overlap(outs[i], out_sz[i], outs[j], out_sz[j])) return FA_ERR_ALIAS;
  }
  const double c = (double)scale * (double)kLog2e;
  if (!(fabs(c) <= (double)FLT_MAX)) return FA_ERR_SCALE;  // checked in double, before the float conversion
  if (static_delta && fa::bwd_scratch(static_cast<hipStream_t>(stream), &delta) != hipSuccess) return FA_ERR_HIP;
  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = delta;
  p.B = B;
  p.H = H;
  p.N = N;
  p.n_blocks = (int)n_blocks;
  p.total_wg = (int)total_wg;
  p.c = (float)c;
  p.scale = scale;
  if (fa::launch_bwd(static_cast<fa::Dtype>(dtype), d, causal != 0, p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

int qkv_proj(const void* x, const void* w, const void* bias, void* q, void* k, void* v, int B, int N, int D, int H,
             int d, int dtype, void* stream) {
  if (!x || !w || !q || !k || !v) return FA_ERR_NULL_PTR;
  if (B < 1 || N < 1 || H < 1 || D < 64 || D % 64 != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  const int64_t M = (int64_t)B * N, ncol = (int64_t)3 * H * d;
  // X and W are addressed with 32-bit byte offsets, and the grid must fit an int
  // (a tile's rows included: its loads use 32-bit offsets too)
  const fa::ProjTiling tl = fa::proj_tiling(M, ncol);
  const int64_t tile_rows = tl.tokens > tl.features ? tl.tokens : tl.features;
  if (M * D * 2 >= ((int64_t)1 << 31) || ncol * D * 2 >= ((int64_t)1 << 31) || tile_rows * D * 2 >= ((int64_t)1 << 31))
    return FA_ERR_SHAPE;
  const int64_t n_ftiles = (ncol + tl.features - 1) / tl.features;
  const int64_t total_wg = n_ftiles * ((M + tl.tokens - 1) / tl.tokens);
  if (total_wg >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      (bias && !aligned(bias, 8)))
    return FA_ERR_ALIGN;
  const size_t x_sz = (size_t)M * D * 2, w_sz = (size_t)ncol * D * 2, b_sz = bias ? (size_t)ncol * 2 : 0;
  const size_t o_sz = (size_t)M * H * d * 2;
  const void* ins[3] = {x, w, bias};
  const size_t in_sz[3] = {x_sz, w_sz, b_sz};
  void* outs[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (in_sz[j] && overlap(outs[i], o_sz, ins[j], in_sz[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], o_sz, outs[j], o_sz)) return FA_ERR_ALIAS;
  }
  fa::ProjParams p;
  p.x = x;
  p.w = w;
  p.bias = bias;
  p.q = q;
  p.k = k;
  p.v = v;
  p.M = (int)M;
  p.N = N;
  p.D = D;
  p.H = H;
  p.d = d;
  p.Ncol = (int)ncol;
  p.tiling = tl.index;
  p.n_ftiles = (int)n_ftiles;
  p.total_wg = (int)total_wg;
  if (fa::launch_qkv_proj(static_cast<fa::Dtype>(dtype), p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

bool known_dtype(int dtype) { return dtype == FA_DTYPE_F16 || dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_FP8_E4M3; }

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, float scale,
           int causal, int dtype, void* stream) {
  if (!known_dtype(dtype)) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
    return FA_ERR_DTYPE;
  }
  return forward(q, k, v, o, lse, Layout{nullptr, B, H, N, 0, d}, scale, causal, static_cast<fa::Dtype>(dtype), 1.0f,
                 1.0f, 1.0f, kNoDropout, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, float q_descale, float k_descale, float v_descale, void* stream) {
  return forward(q, k, v, o, lse, Layout{nullptr, B, H, N, 0, d}, scale, causal, fa::Dtype::FP8, q_descale, k_descale,
                 v_descale, kNoDropout, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens, int B,
                  int H, int total, int max_seqlen, int d, float scale, int causal, int dtype, void* stream) {
  if (!cu_seqlens) return FA_ERR_NULL_PTR;
  if (!known_dtype(dtype)) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
    return FA_ERR_DTYPE;
  }
  return forward(q, k, v, o, lse, Layout{cu_seqlens, B, H, max_seqlen, total, d}, scale, causal,
                 static_cast<fa::Dtype>(dtype), 1.0f, 1.0f, 1.0f, kNoDropout, stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, int dtype, float p_drop, unsigned long long seed, unsigned int offset,
                   void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  // t = floor(256 (1 - p) + 1/2), exact in binary64 for a binary32 p in [0, 1)
  if (!(p_drop >= 0.0f && p_drop < 1.0f)) return FA_ERR_DROPOUT;
  const double t = floor(256.0 * (1.0 - (double)p_drop) + 0.5);
  if (t < 1.0) return FA_ERR_DROPOUT;
  return forward(q, k, v, o, lse, Layout{nullptr, B, H, N, 0, d}, scale, causal, static_cast<fa::Dtype>(dtype), 1.0f,
                 1.0f, 1.0f, Dropout{(uint32_t)t, (uint64_t)seed, (uint32_t)offset}, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream) {
  return backward(q, k, v, o, lse, dout, dq, dk, dv, delta, false, B, H, N, d, scale, causal, dtype, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                   void* stream) {
  return backward(q, k, v, o, lse, dout, dq, dk, dv, nullptr, true, B, H, N, d, scale, causal, dtype, stream);
}

int fa_qkv_proj(const void* x, const void* w, const void* bias, void* q, void* k, void* v, int B, int N, int D, int H,
                int d, int dtype, void* stream) {
  return qkv_proj(x, w, bias, q, k, v, B, N, D, H, d, dtype, stream);
}

int fa_fwd_tile(int N, int d, int causal, int dtype, int mode, int* tile) {
  if (!tile) return FA_ERR_NULL_PTR;
  if (!known_dtype(dtype)) return FA_ERR_DTYPE;
  if (mode != FA_TILE_DENSE && mode != FA_TILE_VARLEN && mode != FA_TILE_DROPOUT) return FA_ERR_SHAPE;
  if (mode == FA_TILE_DROPOUT && dtype == FA_DTYPE_FP8_E4M3) return FA_ERR_DTYPE;
  if (N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  const fa::Variant& v = fa::kVariants[fa::selected_variant(static_cast<fa::Dtype>(dtype), d, causal != 0, N,
                                                            mode == FA_TILE_DROPOUT, mode == FA_TILE_VARLEN)];
  tile[0] = v.qw;
  tile[1] = v.nw;
  tile[2] = v.bc;
  tile[3] = v.sched;
  tile[4] = v.wpe;
  return FA_OK;
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL_PTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "invalid shape: B, H and N (or max_seqlen) must be >= 1, total >= 0, and one slice must stay below 2 GiB";
    case FA_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case FA_ERR_DTYPE: return "unknown dtype (or fp8 given to the backward pass)";
    case FA_ERR_SCALE: return "scale or descale is not finite";
    case FA_ERR_ALIGN: return "misaligned pointer: q, k, v, o need 16 bytes, lse and cu_seqlens 4 bytes";
    case FA_ERR_ALIAS: return "an output overlaps an input or the other output";
    case FA_ERR_HIP: return "the kernel launch reported a HIP error";
    case FA_ERR_DROPOUT: return "dropout rate outside [0, 1), NaN, or so close to 1 that no score is kept";
    case FA_ERR_SCRATCH: return "B * H * N exceeds the static workspace of fa_bwd_noalloc (2^22 rows)";
    default: return "unknown error code";
  }
}

int fa_version(void) { return FA_VERSION; }

}  // extern "C"
