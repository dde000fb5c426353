/*
 * fa.h -- C ABI of libfa.so, the gfx950 (MI355X) FlashAttention forward pass,
 * with its packed-batch, dropout and backward forms and the fused QKV
 * projection that feeds it.  The operation below is fa_fwd's; each other
 * entry point states how it differs.
 *
 * Operation.  For each batch b and head h, with Q, K, V the [N, d] slices at
 * (b, h) and X^ the exact value an input element stands for:
 *
 *   S   = scale * Q^ K^T                      (scores; never stored)
 *   S_ij = -inf for j > i when causal != 0    (lower triangle, diagonal kept)
 *   P   = softmax of each row of S
 *   O   = P V^                                (written to o)
 *   lse_i = ln(sum_j exp(S_ij))               (written to lse)
 *
 * The order scale -> mask -> softmax -> weighted sum is the fused attention
 * sequence of page "FlashAttention与TensorRT 10集成", section "算子融合的极致
 * 优化", item 2; computing it in on-chip tiles so that the N x N matrix never
 * reaches device memory is the block decomposition of that page's section
 * "FlashAttention的技术革命" and the "0 MB (重计算)" attention row of the
 * Flash Attention 2 memory table on page "Optimization Flash Attention 基准测试".
 * The causal flag is the one in the tuning dict of page "从RTX 3090到H100：
 * FlashAttention在NVIDIA各代GPU架构上的性能全景分析", section 3.2.  The online
 * softmax and the lse output are not on the pages: lse is the natural-log
 * logsumexp of each score row (scale included), what a backward pass needs to
 * recompute P.
 *
 * Layout.  q, k, v, o are dense row-major [B, H, N, d] arrays, d innermost
 * (element (b,h,n,c) at offset ((b*H + h)*N + n)*d + c).  lse is a dense
 * float32 [B, H, N] array.  All pointers are device pointers.
 *
 * Ownership.  The caller allocates and owns every buffer.  The library
 * allocates no device or host memory, keeps no mutable global state and may be
 * called from several host threads at once.  Work is enqueued on `stream` (a
 * hipStream_t; NULL is the null stream) and the call returns without waiting.
 *
 * Errors.  Every entry point returns FA_OK (0) or a negative FA_ERR_* code
 * and never throws.  All argument checks run before any HIP call, so a
 * rejected call enqueues nothing.  A fault inside the kernel surfaces as a HIP
 * error at the caller's next synchronisation of `stream`.
 */
#ifndef FA_H_
#define FA_H_

#ifdef __cplusplus
extern "C" {
#endif

#define FA_VERSION 400 /* major * 10000 + minor * 100 + patch: 0.4.0 */

/* Storage format of q, k, v. */
typedef enum {
  FA_DTYPE_F16 = 0,      /* IEEE binary16; o is binary16 */
  FA_DTYPE_BF16 = 1,     /* bfloat16; o is bfloat16 */
  FA_DTYPE_FP8_E4M3 = 2  /* OCP FP8 E4M3 codes (max 448, no inf); o is bfloat16 */
} fa_dtype;

/* Return codes. */
enum {
  FA_OK = 0,
  FA_ERR_NULL_PTR = -1, /* a required pointer (q, k, v, o, lse, cu_seqlens, dout, dq, dk, dv, delta) is NULL */
  FA_ERR_SHAPE = -2,    /* B, H or N (max_seqlen) < 1, total < 0, a slice of 2 GiB or more, too many tiles,
                           or (fa_qkv_proj) D not a positive multiple of 64 */
  FA_ERR_HEADDIM = -3,  /* d is not 64 or 128 */
  FA_ERR_DTYPE = -4,    /* dtype is not an fa_dtype value (or is FP8_E4M3 for fa_bwd) */
  FA_ERR_SCALE = -5,    /* scale or a descale is NaN or infinite */
  FA_ERR_ALIGN = -6,    /* a tensor not 16-byte aligned, lse / cu_seqlens / delta not 4-byte, bias not 8-byte */
  FA_ERR_ALIAS = -7,    /* an output (o, lse; dq, dk, dv, delta; q, k, v of fa_qkv_proj) overlaps an input or another output */
  FA_ERR_HIP = -8,      /* the kernel launch reported a HIP error */
  FA_ERR_DROPOUT = -9,  /* fa_fwd_dropout: p_drop NaN, outside [0, 1), or keeping no score (t = 0) */
  FA_ERR_SCRATCH = -10  /* fa_bwd_noalloc: B * H * N above its static workspace (2^22 rows) */
};

/*
 * fa_fwd -- attention forward over [B, H, N, d] tensors of one dtype.
 *
 *   q, k, v  inputs, `dtype` elements, read only.
 *   o        output [B, H, N, d]: binary16 for F16, bfloat16 for BF16 and
 *            FP8_E4M3; rounded to nearest even from float32.
 *   lse      output [B, H, N] float32, natural-log logsumexp of each score row.
 *   B, H, N  batch, heads, sequence length (queries and keys alike), each >= 1.
 *            Any N is accepted: a tail shorter than a tile is masked, not padded.
 *   d        head dimension, 64 or 128.
 *   scale    multiplies Q K^T; any finite value (0 gives a uniform average).
 *            Scores are scaled in float32, except for binary16 at d = 64 with
 *            |scale| * log2(e) in [1/16, 1]: there Q is multiplied by that
 *            factor and rounded to binary16 in the kernel (2^-11 relative per
 *            element) before the product.
 *   causal   nonzero: query i sees keys 0..i only.
 *   dtype    an fa_dtype value.  FA_DTYPE_FP8_E4M3 here means descales of 1.
 *   stream   hipStream_t to enqueue on, or NULL.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream);

/*
 * fa_fwd_fp8 -- fa_fwd for OCP FP8 E4M3 inputs with one float32 descale per
 * tensor: the value of an element is code * descale (FP8 attention is the
 * "Flash Attn 3 (FP8)" column of the H100 80GB table on page "Optimization
 * Flash Attention 基准测试"; per-tensor scaling is this library's reading).
 * S = scale * q_descale * k_descale * (Qcode Kcode^T) is formed by the fp8
 * matrix cores with float32 accumulation; O = softmax(S) * (Vcode * v_descale)
 * is formed in bfloat16 (V codes widen exactly to bfloat16, probabilities are
 * rounded to bfloat16) with float32 accumulation and written as bfloat16.
 * Descales must be finite.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               float q_descale, float k_descale, float v_descale, void* stream);

/*
 * fa_fwd_varlen -- the same operation for B sequences of different lengths,
 * packed back to back without padding.  (The pages meet unaligned sequence
 * lengths by padding them -- page "从RTX 3090到H100：FlashAttention在NVIDIA各代
 * GPU架构上的性能全景分析", section 3.2, common pitfalls item 2 -- and list
 * better dynamic-shape support as a direction -- page "FlashAttention与
 * TensorRT 10集成", section "推理优化的未来方向" item 1; packing instead of
 * padding is this library's reading.)  Each sequence b is an independent
 * attention problem over its own rows; causal masking is within a sequence.
 *
 *   q, k, v     packed inputs [total, H, d], `dtype` elements: row t of head h
 *               at element offset (t*H + h)*d.
 *   o           output [total, H, d], binary16 for F16, bfloat16 otherwise.
 *   lse         output [H, total] float32 (row t of head h at h*total + t).
 *   cu_seqlens  device int32 array of B+1 offsets: sequence b owns rows
 *               cu_seqlens[b] .. cu_seqlens[b+1]-1.  Expected non-decreasing
 *               from 0 to total.  It is read on the device, not checked on
 *               the host: a pair that is negative, decreasing, past total or
 *               longer than max_seqlen makes that sequence empty (its rows are
 *               not written); no access leaves the buffers.
 *   B           number of sequences, >= 1 (empty sequences are allowed).
 *   H, d        heads, head dimension (64 or 128).
 *   total       rows of the packed tensors, >= 0 (0 enqueues nothing).
 *   max_seqlen  an upper bound of every sequence length, >= 1; sizes the grid.
 *   scale, causal, dtype, stream  as for fa_fwd (FP8_E4M3 with descales 1).
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens, int B, int H, int total, int max_seqlen,
                  int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_dropout -- fa_fwd with dropout on the probabilities.  The tuning
 * dict of page "从RTX 3090到H100：FlashAttention在NVIDIA各代GPU架构上的性能全景
 * 分析", section 3.2, carries a dropout rate and notes that a non-zero rate
 * needs special handling; the pages define nothing further, so:
 *   O_i = sum_j (P_ij * M_ij * 256 / t) V_j,   lse as for fa_fwd (no dropout),
 * with t = floor(256 * (1 - p_drop) + 1/2) and M_ij = 1 iff the generator
 * byte u_ij of the score is below t (keep probability t / 256 exactly, so the
 * expected output is fa_fwd's).  u_ij comes from Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011)
 * with key (seed mod 2^32, seed div 2^32): writing the key column as
 * j = 32g + 8q + 4s + u (s in {0, 1}; q, u in 0..3), the counter is
 * (2g + s, i, b*H + h, offset) and u_ij is bits 8u..8u+7 of output word q.
 * The same (seed, offset) gives the same mask on every call.
 *
 *   q, k, v, o, lse, B, H, N, d, scale, causal, stream  as for fa_fwd.
 *   dtype   F16 or BF16 (FP8_E4M3 returns FA_ERR_DTYPE).
 *   p_drop  drop rate in [0, 1) with t >= 1 (p_drop <= 1 - 1/512); 0 gives
 *           fa_fwd's result bit for bit.  Otherwise FA_ERR_DROPOUT.
 *   seed    the 64-bit Philox key.
 *   offset  counter word 3: calls that must draw independent masks with one
 *           seed use different offsets.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   float p_drop, unsigned long long seed, unsigned int offset, void* stream);

/*
 * fa_bwd -- gradients of fa_fwd: given the output gradient dO, write dQ, dK
 * and dV.  The probabilities are recomputed from q, k and the saved lse rather
 * than stored, which is what the "0 MB (重计算)" attention row of the Flash
 * Attention 2 memory table on page "Optimization Flash Attention 基准测试"
 * relies on; the formulas are the derivative of the forward definition:
 *   P = softmax(scale * Q K^T + mask),  dV = P^T dO,  dP = dO V^T,
 *   dS = P * (dP - rowsum(dO * O)),  dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 *   q, k, v, o  the forward inputs and output, [B, H, N, d], F16 or BF16.
 *   lse         the forward lse, [B, H, N] float32.
 *   dout        dO, [B, H, N, d], same dtype.
 *   dq, dk, dv  outputs, [B, H, N, d], same dtype (rounded from float32).
 *   delta       workspace [B, H, N] float32, overwritten with rowsum(dO * O).
 *   B, H, N, d, scale, causal, stream  as for fa_fwd; dtype F16 or BF16
 *               (FP8_E4M3 returns FA_ERR_DTYPE).
 * Outputs and the workspace must not overlap any input or each other.  Two
 * kernels are enqueued on `stream` in order.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd without the workspace argument, for callers that
 * cannot allocate device memory or hand the library a workspace: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation.  The same kernels run; D = rowsum(dO * O) goes to a static
 * device array of the library instead of `delta`.
 *
 *   Arguments as for fa_bwd, without delta.
 *   Limit: B * H * N <= 2^22 (4 Mi rows, a 16 MiB array per GPU, reserved
 *          from the library's load until the process ends); larger problems
 *          return FA_ERR_SCRATCH before any HIP call.
 * The array's device address on the GPU that `stream` belongs to (the
 * current device for the null stream) is looked up on the first call for
 * that GPU; the call allocates nothing, then or later.  Every row of D a
 * call reads was written earlier in the same call, so nothing carries over
 * from the previous call.  All calls on one GPU share that GPU's array:
 * calls that may run at the same time on one GPU (different streams, or
 * several host threads) race on it and must be serialised by the caller.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_qkv_proj -- the fused input projection ahead of attention: page
 * "FlashAttention与TensorRT 10集成", section "算子融合的极致优化", item 1,
 * merges the projection with the transpose and rearrangement into one
 * kernel.  For the layer input X and one packed weight W of the three
 * projections (stored [out, in], as a linear layer's):
 *   Y = X W^T + bias,   out_s[b, h, n, c] = Y[b, n, s*H*d + h*d + c]
 * with s = 0, 1, 2 writing q, k, v.  The outputs are exactly fa_fwd's inputs.
 *
 *   x        [B, N, D] token-major, F16 or BF16.
 *   w        [3*H*d, D], same dtype.
 *   bias     [3*H*d], same dtype, or NULL for none.
 *   q, k, v  outputs, each [B, H, N, d], same dtype (rounded from float32).
 *   B, N, H  >= 1; D a multiple of 64 (>= 64); d = 64 or 128.
 * x, w, q, k, v need 16-byte alignment, bias 8; outputs may not overlap the
 * inputs or each other.  X and W must each stay below 2 GiB.
 */
int fa_qkv_proj(const void* x, const void* w, const void* bias, void* q, void* k, void* v,
                int B, int N, int D, int H, int d, int dtype, void* stream);

/*
 * fa_fwd_tile -- which compiled kernel shape a forward call with these
 * arguments runs (a query about this library, not an operation of the
 * pages).  The shape is chosen from N, d, the mask and the dtype, and the
 * FA_TILE environment variable (QWxNWxBCxSCHEDxWPE) may select another
 * compiled shape; this reports the outcome, so a caller can tell whether an
 * FA_TILE request was honoured or fell back to the default.
 *
 *   N       sequence length (fa_fwd_varlen: max_seqlen), >= 1.
 *   d       64 or 128.   causal, dtype  as for fa_fwd.
 *   mode    FA_TILE_DENSE (fa_fwd, fa_fwd_fp8), FA_TILE_VARLEN (fa_fwd_varlen)
 *           or FA_TILE_DROPOUT (fa_fwd_dropout; FA_TILE is ignored there).
 *   tile    out, 5 ints: query rows per wave, waves per workgroup, keys per
 *           tile, schedule (0 = every wave runs each tile's products and
 *           softmax in turn, 1 = two wave groups alternate them), and the
 *           waves per SIMD the kernel's registers are budgeted for.
 * Returns FA_OK, FA_ERR_NULL_PTR, FA_ERR_SHAPE (N < 1 or an unknown mode),
 * FA_ERR_HEADDIM or FA_ERR_DTYPE (unknown, or fp8 with FA_TILE_DROPOUT).
 * Makes no HIP call.
 */
enum { FA_TILE_DENSE = 0, FA_TILE_VARLEN = 1, FA_TILE_DROPOUT = 2 };
int fa_fwd_tile(int N, int d, int causal, int dtype, int mode, int* tile);

/* Static description of a return code; never NULL. */
const char* fa_strerror(int code);

/* FA_VERSION of the built library. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
