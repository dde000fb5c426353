// Fused QKV projection for gfx950 (MI355X, CDNA4): the input projection,
// transpose and rearrangement that page "FlashAttention与TensorRT 10集成",
// section "算子融合的极致优化", item 1, merges into one kernel ahead of the
// attention kernel.
//
//   Y = X W^T + bias,   X [B*N, D] token-major, W [3 H d, D] ([out, in]),
//   out_s[b, h, n, c] = Y[b*N + n, s H d + h d + c]   (s = 0, 1, 2: Q, K, V)
//
// so the three attention inputs come out in the dense [B, H, N, d] layout,
// without a separate transpose pass.
//
// The kernel computes Y^T, a 3Hd x BN product, on 32x32x16 matrix
// instructions: A = a 32-row block of W, B^T = a 32-row block of X.  Both
// operands are rows read along k, so both tiles use the padded-row LDS layout
// and the direct HBM -> LDS loads of the attention kernels.  In the
// accumulator, lane (half, j) holds token j of the block and features
// 8*(r/4) + 4*half + r%4: four consecutive features, i.e. four consecutive
// columns c of one head, which the epilogue writes as one 8-byte store into
// the [B, H, N, d] output.
//
// Workgroup: 4 waves as 2 (features) x 2 (tokens), 64 x 64 outputs per wave,
// a 128 x 128 tile per workgroup; k advances 64 at a time through two LDS
// stages.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kPT = 128;               // features (and tokens) per workgroup tile
constexpr int kPK = 64;                // k per stage
constexpr int kPRow = kPK * 2;         // bytes of one tile row per stage
constexpr int kPRS = kPRow + 16;       // padded LDS row (one pad granule)
constexpr int kPGR = kPRow / 16 + 1;   // LDS granules per padded row
constexpr int kPGran = kPT * kPGR;     // granules per tile
constexpr int kPBlk = (kPGran + 63) / 64;  // direct-load instructions per tile
constexpr int kPStage = kPT * kPRS;    // bytes per tile per stage

}  // namespace

template <bool BF16>
__global__ __launch_bounds__(256, 2) void fa_qkv_proj_kernel(ProjParams p) {
  __shared__ __attribute__((aligned(16))) char lw0[kPStage];
  __shared__ __attribute__((aligned(16))) char lw1[kPStage];
  __shared__ __attribute__((aligned(16))) char lx0[kPStage];
  __shared__ __attribute__((aligned(16))) char lx1[kPStage];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, l32 = lane & 31;
  const int tile = xcd_remap(blockIdx.x, p.total_wg);
  const int ft = tile % p.n_ftiles, tt = tile / p.n_ftiles;  // consecutive tiles share the token block
  const int f0 = ft * kPT, t0 = tt * kPT;
  const int wf = (wave & 1) * 64, wt = (wave >> 1) * 64;    // the wave's 64 x 64 corner

  const u32 rowb = (u32)p.D * 2;
  const auto rw = make_rsrc((const char*)p.w + (size_t)f0 * rowb, (u32)(min(kPT, p.Ncol - f0)) * rowb);
  const auto rx = make_rsrc((const char*)p.x + (size_t)t0 * rowb, (u32)(min(kPT, p.M - t0)) * rowb);

  // Lane L of direct-load instruction blk fills granule 64*blk + L of the
  // padded tile: row g / kPGR, chunk g % kPGR (chunk kPGR-1 is the pad).
  auto issue = [&](int kk, char* dw, char* dx) __attribute__((always_inline)) {
    const int kbyte = kk * kPRow;
#pragma unroll
    for (int j = 0; j < (kPBlk + 3) / 4; ++j) {
      const int blk = wave + 4 * j;
      const int g = blk * 64 + lane;
      const int r = g / kPGR, c = g - r * kPGR;
      if (blk < kPBlk && g < kPGran && c < kPGR - 1) {
        load_lds16(rw, dw + blk * 1024, r * (int)rowb + kbyte + c * 16);
        load_lds16(rx, dx + blk * 1024, r * (int)rowb + kbyte + c * 16);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int abase = (wf + l32) * kPRS + 16 * half;  // W row of feature block 0 of the wave
  const int bbase = (wt + l32) * kPRS + 16 * half;  // X row of token block 0 of the wave

  auto step = [&](const char* tw, const char* tx) __attribute__((always_inline)) {
    u32x4 a[2][kPK / 16], b[2][kPK / 16];
#pragma unroll
    for (int s = 0; s < kPK / 16; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i][s] = lds_read_b128(tw, abase + 32 * i * kPRS + 32 * s);
        b[i][s] = lds_read_b128(tx, bbase + 32 * i * kPRS + 32 * s);
      }
#pragma unroll
    for (int s = 0; s < kPK / 16; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16(a[i][s], b[j][s], acc[i][j], BF16);
  };

  const int nk = p.D / kPK;
  issue(0, lw0, lx0);
  for (int kk = 0; kk < nk; kk += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kk + 1 < nk) issue(kk + 1, lw1, lx1);
    step(lw0, lx0);
    if (kk + 1 < nk) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kk + 2 < nk) issue(kk + 2, lw0, lx0);
      step(lw1, lx1);
    }
  }

  // ---- epilogue: bias, round, and store four consecutive columns per group
  const int HD = p.H * p.d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + wf + 32 * i + 8 * g + 4 * half;  // first of four features
      if (f >= p.Ncol) continue;
      const int s = f / HD, rem = f - s * HD, h = rem / p.d, c = rem - h * p.d;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias) {
        const u32x2 bw = *reinterpret_cast<const u32x2*>((const char*)p.bias + (size_t)f * 2);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32 word = bw[e];
          if (BF16) {
            bv[2 * e] = __builtin_bit_cast(float, word << 16);
            bv[2 * e + 1] = __builtin_bit_cast(float, word & 0xFFFF0000u);
          } else {
            const fp16x2 hv = __builtin_bit_cast(fp16x2, word);
            bv[2 * e] = (float)hv[0];
            bv[2 * e + 1] = (float)hv[1];
          }
        }
      }
      char* outs = (char*)(s == 0 ? p.q : s == 1 ? p.k : p.v);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = t0 + wt + 32 * j + l32;  // token
        if (m >= p.M) continue;
        const int b = m / p.N, n = m - b * p.N;
        u32x2 w;
        w[0] = pack_p<BF16>(acc[i][j][4 * g + 0] + bv[0], acc[i][j][4 * g + 1] + bv[1]);
        w[1] = pack_p<BF16>(acc[i][j][4 * g + 2] + bv[2], acc[i][j][4 * g + 3] + bv[3]);
        *reinterpret_cast<u32x2*>(outs + ((((size_t)b * p.H + h) * p.N + n) * p.d + c) * 2) = w;
      }
    }
  }
}

hipError_t launch_qkv_proj(Dtype dt, const ProjParams& p, hipStream_t stream) {
  if (dt == Dtype::F16)
    hipLaunchKernelGGL((fa_qkv_proj_kernel<false>), dim3(p.total_wg), dim3(256), 0, stream, p);
  else if (dt == Dtype::BF16)
    hipLaunchKernelGGL((fa_qkv_proj_kernel<true>), dim3(p.total_wg), dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
