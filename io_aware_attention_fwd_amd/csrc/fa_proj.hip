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
// Workgroup: NWF x NWT waves (features x tokens), each owning 64 features x
// WT tokens; k advances 64 at a time through two LDS stages.  Two shapes
// are compiled: 4 waves of 64 x 64 (a 128 x 128 tile, two workgroups per
// CU) and 8 waves of 64 x 128 (a 256 x 256 tile, one workgroup per CU).  The
// larger tile halves the bytes each FLOP pulls from L2 into LDS, which is
// what bounds large products; it is used when the grid still has at least
// four workgroups per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kPK = 64;                // k per stage
constexpr int kPRow = kPK * 2;         // bytes of one tile row per stage
constexpr int kPRS = kPRow + 16;       // padded LDS row (one pad granule)
constexpr int kPGR = kPRow / 16 + 1;   // LDS granules per padded row

template <int NWF, int NWT, int WT>
struct ProjTile {
  static constexpr int kNW = NWF * NWT;             // waves per workgroup
  static constexpr int kTB = WT / 32;               // 32-token blocks per wave
  static constexpr int kTF = NWF * 64;              // features per tile
  static constexpr int kTT = NWT * WT;              // tokens per tile
  static constexpr int kBlkW = (kTF * kPGR + 63) / 64;  // direct-load instructions per stage
  static constexpr int kBlkX = (kTT * kPGR + 63) / 64;
  static constexpr int kStW = kBlkW * 1024;         // whole blocks: a partial last block
  static constexpr int kStX = kBlkX * 1024;         // writes into the stage's own tail
};
using TileSmall = ProjTile<2, 2, 64>;   // 128 x 128, 4 waves
using TileLarge = ProjTile<4, 2, 128>;  // 256 x 256, 8 waves

}  // namespace

template <bool BF16, int NWF, int NWT, int WT>
__global__ __launch_bounds__(NWF * NWT * 64, 8 / (NWF * NWT)) void fa_qkv_proj_kernel(ProjParams p) {
  using T = ProjTile<NWF, NWT, WT>;
  __shared__ __attribute__((aligned(16))) char lw0[T::kStW];
  __shared__ __attribute__((aligned(16))) char lw1[T::kStW];
  __shared__ __attribute__((aligned(16))) char lx0[T::kStX];
  __shared__ __attribute__((aligned(16))) char lx1[T::kStX];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, l32 = lane & 31;
  const int tile = xcd_remap(blockIdx.x, p.total_wg);
  const int ft = tile % p.n_ftiles, tt = tile / p.n_ftiles;  // consecutive tiles share the token block
  const int f0 = ft * T::kTF, t0 = tt * T::kTT;
  const int wf = (wave % NWF) * 64, wt = (wave / NWF) * WT;  // the wave's corner

  const u32 rowb = (u32)p.D * 2;
  const auto rw = make_rsrc((const char*)p.w + (size_t)f0 * rowb, (u32)(min(T::kTF, p.Ncol - f0)) * rowb);
  const auto rx = make_rsrc((const char*)p.x + (size_t)t0 * rowb, (u32)(min(T::kTT, p.M - t0)) * rowb);

  // Lane L of direct-load instruction blk fills granule 64*blk + L of the
  // padded tile: row g / kPGR, chunk g % kPGR.  The pad chunk (and lanes of
  // a partial last block) load an in-bounds duplicate rather than being
  // masked off; rows past the matrix read as zero (range-checked).
  auto load_blk = [&](__amdgpu_buffer_rsrc_t rs, char* dst, int blk, int kbyte) __attribute__((always_inline)) {
    const int g = blk * 64 + lane;
    const int r = g / kPGR, c = min(g - r * kPGR, kPGR - 2);
    load_lds16(rs, dst + blk * 1024, r * (int)rowb + kbyte + c * 16);
  };
  auto issue = [&](int kk, char* dw, char* dx) __attribute__((always_inline)) {
    const int kbyte = kk * kPRow;
#pragma unroll
    for (int j = 0; j < (T::kBlkW + T::kNW - 1) / T::kNW; ++j)
      if (wave + T::kNW * j < T::kBlkW) load_blk(rw, dw, wave + T::kNW * j, kbyte);
#pragma unroll
    for (int j = 0; j < (T::kBlkX + T::kNW - 1) / T::kNW; ++j)
      if (wave + T::kNW * j < T::kBlkX) load_blk(rx, dx, wave + T::kNW * j, kbyte);
  };

  f32x16 acc[2][T::kTB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < T::kTB; ++j) acc[i][j] = f32x16{};
  const int abase = (wf + l32) * kPRS + 16 * half;  // W row of feature block 0 of the wave
  const int bbase = (wt + l32) * kPRS + 16 * half;  // X row of token block 0 of the wave

  // One matrix k-step reads 2 W and kTB X operands for 2 x kTB instructions.
  auto step = [&](const char* tw, const char* tx) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kPK / 16; ++s) {
      u32x4 a[2], b[T::kTB];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = lds_read_b128(tw, abase + 32 * i * kPRS + 32 * s);
#pragma unroll
      for (int j = 0; j < T::kTB; ++j) b[j] = lds_read_b128(tx, bbase + 32 * j * kPRS + 32 * s);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < T::kTB; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j], BF16);
    }
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
      for (int j = 0; j < T::kTB; ++j) {
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

namespace {

template <class T>
int64_t grid_of(int64_t M, int64_t ncol) {
  return ((ncol + T::kTF - 1) / T::kTF) * ((M + T::kTT - 1) / T::kTT);
}

template <bool BF16, class T, int NWF, int NWT, int WT>
void launch_tile(const ProjParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fa_qkv_proj_kernel<BF16, NWF, NWT, WT>), dim3(p.total_wg), dim3(T::kNW * 64), 0, stream, p);
}

}  // namespace

ProjTiling proj_tiling(int64_t M, int64_t ncol) {
  // 256 CUs: the large tile once its grid has at least four workgroups per CU
  if (grid_of<TileLarge>(M, ncol) >= 4 * 256) return {1, TileLarge::kTF, TileLarge::kTT};
  return {0, TileSmall::kTF, TileSmall::kTT};
}

hipError_t launch_qkv_proj(Dtype dt, const ProjParams& p, hipStream_t stream) {
  if (dt != Dtype::F16 && dt != Dtype::BF16) return hipErrorInvalidValue;
  const bool bf = dt == Dtype::BF16;
  if (p.tiling == 1) {
    if (bf)
      launch_tile<true, TileLarge, 4, 2, 128>(p, stream);
    else
      launch_tile<false, TileLarge, 4, 2, 128>(p, stream);
  } else {
    if (bf)
      launch_tile<true, TileSmall, 2, 2, 64>(p, stream);
    else
      launch_tile<false, TileSmall, 2, 2, 64>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace fa
