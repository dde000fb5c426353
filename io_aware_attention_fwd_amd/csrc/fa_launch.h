// Internal interface between the C-ABI layer (fa_api.cpp) and the kernels
// (fa_fwd.hip).  Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a kernel instance needs, already validated and folded on the host.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N;
  int n_qtiles;   // ceil(N / rows per workgroup)
  int total_wg;   // n_qtiles * B * H
  float c;        // |effective scale| * log2(e); 1 when the effective scale is 0
  uint32_t q_xor; // xor applied to every packed Q word: flips signs when the scale is negative
  uint32_t q_and; // and applied to every packed Q word: 0 when the scale is 0
  float o_mul;    // final multiplier of O (the V descale for fp8, else 1)
};

enum class Dtype { F16 = 0, BF16 = 1, FP8 = 2 };

// Rows of Q one workgroup owns for the instance chosen for this call (sizes the grid).
int rows_per_workgroup(Dtype dt, int d, bool causal, int N);

// Enqueue one forward pass; returns hipSuccess or the launch error.
hipError_t launch_fwd(Dtype dt, int d, bool causal, const FwdParams& p, hipStream_t stream);

}  // namespace fa
