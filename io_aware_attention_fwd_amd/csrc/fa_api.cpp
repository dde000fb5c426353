// C ABI of libfa.so: argument validation, folding of the scale, dispatch.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and needs no GPU.  The operation, layouts and error codes are
// documented in include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_launch.h"

namespace {

constexpr float kLog2e = 1.44269504088896341f;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int elem_bytes(fa::Dtype dt) { return dt == fa::Dtype::FP8 ? 1 : 2; }

int forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
            float scale, int causal, fa::Dtype dt, float q_descale, float k_descale, float v_descale,
            void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return FA_ERR_SCALE;
  const int eb = elem_bytes(dt);
  const int br = fa::rows_per_workgroup(dt, d, causal != 0, N);
  // One (batch, head) slice, plus the padding rows of its last tile, must be
  // addressable with 32-bit byte offsets (the kernels use buffer loads).
  const int64_t slice_bytes = (int64_t)(N + br) * d * eb;
  if (slice_bytes >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  const int64_t n_qtiles = ((int64_t)N + br - 1) / br;
  const int64_t total_wg = n_qtiles * B * H;
  if (total_wg >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  const size_t in_bytes = (size_t)B * H * N * d * eb;
  const size_t o_bytes = (size_t)B * H * N * d * (dt == fa::Dtype::FP8 ? 2 : eb);
  const size_t lse_bytes = (size_t)B * H * N * sizeof(float);
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
  p.B = B;
  p.H = H;
  p.N = N;
  p.n_qtiles = (int)n_qtiles;
  p.total_wg = (int)total_wg;
  const uint32_t sign_bits = dt == fa::Dtype::FP8 ? 0x80808080u : 0x80008000u;
  p.q_xor = eff < 0 ? sign_bits : 0u;
  p.q_and = eff == 0 ? 0u : 0xFFFFFFFFu;
  p.c = eff == 0 ? 1.0f : (float)(fabs(eff) * (double)kLog2e);
  if (!isfinite(p.c)) return FA_ERR_SCALE;
  p.o_mul = v_descale;

  if (fa::launch_fwd(dt, d, causal != 0, p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, float scale,
           int causal, int dtype, void* stream) {
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
    return FA_ERR_DTYPE;
  }
  return forward(q, k, v, o, lse, B, H, N, d, scale, causal, static_cast<fa::Dtype>(dtype), 1.0f, 1.0f, 1.0f,
                 stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, float q_descale, float k_descale, float v_descale, void* stream) {
  return forward(q, k, v, o, lse, B, H, N, d, scale, causal, fa::Dtype::FP8, q_descale, k_descale, v_descale,
                 stream);
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL_PTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: B, H and N must be >= 1 and one slice must stay below 2 GiB";
    case FA_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_SCALE: return "scale or descale is not finite";
    case FA_ERR_ALIGN: return "misaligned pointer: q, k, v, o need 16 bytes, lse 4 bytes";
    case FA_ERR_ALIAS: return "an output overlaps an input or the other output";
    case FA_ERR_HIP: return "the kernel launch reported a HIP error";
    default: return "unknown error code";
  }
}

int fa_version(void) { return FA_VERSION; }

}  // extern "C"
