// Internal interface between the C-ABI layer (fa_api.cpp) and the kernels
// (fa_fwd.hip).  Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a kernel instance needs, already validated and folded on the host.
// One slice is the rows of one (sequence, head); byte strides locate it:
//   dense [B,H,N,d]:      batch = H*N*row, head = N*row, row = d*elem
//   packed [total,H,d]:   batch = 0, head = d*elem, row = H*d*elem, and the
//                         sequence's first row cu[b] is added
// lse is indexed the same way in elements (dense [B,H,N], packed [H,total]).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* cu;  // packed layout: B+1 sequence offsets (device memory); nullptr for dense
  int B, H, N;    // N: rows per sequence (dense) or the longest sequence (packed)
  int total;      // packed layout: rows of the packed tensors
  int n_qtiles;   // ceil(N / rows per workgroup)
  int total_wg;   // workgroups: n_qtiles * B * H, or ceil(n_qtiles / 2) * B * H for dense causal grids
  long long in_batch, in_head;    // byte strides of Q, K, V
  int in_row;
  long long out_batch, out_head;  // byte strides of O
  int out_row;
  long long lse_batch, lse_head;  // element strides of lse
  float c;        // |effective scale| * log2(e); 1 when the effective scale is 0
  uint32_t q_xor; // xor applied to every packed Q word: flips signs when the scale is negative
  uint32_t q_and; // and applied to every packed Q word: 0 when the scale is 0
  float o_mul;    // final multiplier of O (the V descale for fp8, times 256/t with dropout)
  // Dropout: a score is kept iff its generator byte is below drop_t (1..256;
  // 256 keeps every score and selects the kernels without dropout).  Philox
  // key (seed_lo, seed_hi); counter word 3 is drop_offset.
  uint32_t drop_t;
  uint32_t seed_lo, seed_hi, drop_offset;
  int variant;    // index into kVariants (fa_variants.h) of the tile shape to run
};

// Backward pass over dense [B,H,N,d] tensors (16-bit types).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [B,H,N] workspace: rowsum(dO * O), written by the dQ kernel, read by the dK/dV kernel
  int B, H, N;
  int n_blocks;  // ceil(N / rows per workgroup), the same for both kernels
  int total_wg;  // n_blocks * B * H
  float c;       // scale * log2(e), signed (may be 0)
  float scale;   // multiplies dQ and dK at the end
};

// Fused QKV projection: Y = X W^T + bias written as Q, K, V in [B, H, N, d].
struct ProjParams {
  const void* x;     // [M, D] tokens, M = B * N
  const void* w;     // [Ncol, D] weight, Ncol = 3 * H * d
  const void* bias;  // [Ncol] or nullptr
  void* q;
  void* k;
  void* v;
  int M, N, D, H, d, Ncol;
  int tiling;    // which compiled tile (from proj_tiling)
  int n_ftiles;  // ceil(Ncol / tile features)
  int total_wg;  // n_ftiles * ceil(M / tile tokens)
};

// The QKV projection's tile for an M x Ncol product: an index and its size.
struct ProjTiling {
  int index, features, tokens;
};
ProjTiling proj_tiling(int64_t M, int64_t ncol);

enum class Dtype { F16 = 0, BF16 = 1, FP8 = 2 };

// Enqueue one forward pass; returns hipSuccess or the launch error.
hipError_t launch_fwd(Dtype dt, int d, bool causal, const FwdParams& p, hipStream_t stream);
// The same for one dtype (the instances of each live in their own object).
hipError_t launch_fwd_f16(int d, bool causal, const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_bf16(int d, bool causal, const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_fp8(int d, bool causal, const FwdParams& p, hipStream_t stream);

// Enqueue the fused QKV projection (16-bit types; D a multiple of 64).
hipError_t launch_qkv_proj(Dtype dt, const ProjParams& p, hipStream_t stream);

// Rows (queries for dQ, keys for dK/dV) one backward workgroup owns.
constexpr int kBwdRows = 128;

// Enqueue the backward pass (dQ kernel, then dK/dV kernel, on one stream).
hipError_t launch_bwd(Dtype dt, int d, bool causal, const BwdParams& p, hipStream_t stream);

// Rows of D the allocation-free backward entry point holds in its static
// device workspace (B * H * N at most): 2^22 float32 rows, 16 MiB per GPU.
constexpr int64_t kBwdScratchRows = int64_t(1) << 22;

// Device address of that workspace on the GPU `stream` belongs to (the
// current device for the null stream), looked up once per device.
hipError_t bwd_scratch(hipStream_t stream, float** out);

}  // namespace fa
