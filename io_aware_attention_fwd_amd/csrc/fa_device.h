// Device-side building blocks shared by the attention kernels (forward and
// backward): vector types, matrix-core wrappers, half-wave exchanges, buffer
// resources, LDS reads and the LDS tile layouts.  Everything here is inline
// and internal to each translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Debug build (compiled with FA_SYNC_CHECK): full memory waits and a
// workgroup barrier at extra points that every wave of a workgroup reaches.
// The kernels' results must not change, bit for bit; a difference against
// the normal build exposes a missing wait or barrier (there is no LDS race
// checker on this platform).
#ifdef FA_SYNC_CHECK
#define FA_SYNC_POINT()                                            \
  do {                                                             \
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");    \
    __syncthreads();                                               \
  } while (0)
#else
#define FA_SYNC_POINT() \
  do {                  \
  } while (0)
#endif

namespace fa {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleThreshold = 8.0f;  // log2 of the largest probability allowed before rescaling
constexpr float kSpeculativeSumLimit = 32768.0f;  // largest per-lane tile sum accepted without the tile's maxima
constexpr u32 kRsrcWord3 = 0x00020000u;    // raw buffer, 32-bit data format, range-checked

// ---------------------------------------------------------------- dtype traits
struct TrF16 {
  static constexpr bool kFp8 = false;
  static constexpr int kEK = 2;  // bytes per Q/K element
  static constexpr int kEV = 2;  // bytes per V element
  static constexpr bool kPvBf16 = false;
};
struct TrBF16 {
  static constexpr bool kFp8 = false;
  static constexpr int kEK = 2;
  static constexpr int kEV = 2;
  static constexpr bool kPvBf16 = true;
};
struct TrFP8 {
  static constexpr bool kFp8 = true;
  static constexpr int kEK = 1;
  static constexpr int kEV = 1;
  static constexpr bool kPvBf16 = true;  // P V in bfloat16 with V widened exactly
};

__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c, bool bf16) {
  if (bf16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // operand format code 0 = E4M3 for both; zero scale operands leave them unscaled
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two floats -> one packed 16-bit pair, round to nearest even (one
// v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 on gfx950).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <bool BF16>
__device__ __forceinline__ u32 pack_p(float lo, float hi) {
  const f32x2 x = {lo, hi};
  if (BF16) return __builtin_bit_cast(u32, __builtin_convertvector(x, bf16x2));
  return __builtin_bit_cast(u32, __builtin_convertvector(x, f16x2));
}

// Combine lane l with lane l ^ 32 (the other half-wave) without touching LDS
// (an LDS permute would be ordered behind the operand reads in flight).
// v_permlane32_swap exchanges the upper half-wave of its first operand with
// the lower half-wave of its second; applied to two copies of x it leaves the
// lower half-wave's values in every lane of one and the upper half-wave's in
// every lane of the other, so a symmetric combination of the two gives each
// lane the pairwise result.  It is written as inline assembly because the
// compiler's model of the builtin folds that symmetric combination into a
// single operand.
__device__ __forceinline__ void swap_halves(u32& a, u32& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds over a 128-bit counter with a
// 64-bit key.  A round multiplies counter words 0 and 2 by the two Philox
// constants, swaps the high halves (xored with the other counter words and
// the key) into words 0 and 2 and the low halves into 3 and 1; the key grows
// by the two Weyl constants between rounds.  Each 32 x 32 -> 64-bit product is
// one v_mad_u64_u32.
__device__ __forceinline__ u32x4 philox4x32_10(u32 c0, u32 c1, u32 c2, u32 c3, u32 k0, u32 k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const u32 n0 = (u32)(p1 >> 32) ^ c1 ^ k0;
    const u32 n2 = (u32)(p0 >> 32) ^ c3 ^ k1;
    c1 = (u32)p1;
    c3 = (u32)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// This lane's index in the wave, recomputed from the exec-independent lane
// counter rather than kept in a register (used after long loops, where a
// register holding it would be live all the way through).
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ float halves_max(float x) {
  u32 a = __builtin_bit_cast(u32, x), b = a;
  swap_halves(a, b);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float halves_sum(float x) {
  u32 a = __builtin_bit_cast(u32, x), b = a;
  swap_halves(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// acc + p0 + p1 for the row sum.  PACKED sums the binary16-rounded pair with
// one v_dot2c_f32_f16 (rounding moves the sum by at most 2^-11 relative, well
// inside the lse bar, and matches the values that enter P V): half the
// instructions, but each waits for the pair's conversion, which lengthens a
// lone wave's dependency chains.  Otherwise the float32 values are summed
// (always for bfloat16, whose 2^-8 rounding would be too coarse for lse).
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
template <bool PACKED>
__device__ __forceinline__ float sum_pair(u32 packed, float p0, float p1, float acc) {
  if (!PACKED) return acc + (p0 + p1);
  const fp16x2 one = {(__fp16)1.0f, (__fp16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, packed), one, acc, false);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, u32 bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// 16 bytes per lane from a buffer straight into LDS: lane L of the wave writes
// lds_block + 16 * L; an out-of-range offset writes zeros.  (Kept in a device
// function: in a lambda the host pass would see the builtin too.)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, char* lds_block, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_block, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read_b128(const char* smem, u32 off) {
  return *reinterpret_cast<const u32x4*>(smem + off);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* smem, u32 off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off)));
}

__device__ __forceinline__ u32x2 lds_read_tr8(const char* smem, u32 off) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(smem + off)));
}

// Workgroup id -> logical tile id such that consecutive logical ids run on the
// same XCD (hardware hands workgroups to the 8 XCDs round-robin).  Consecutive
// logical ids are query tiles of one (batch, head), so that slice's K and V
// are fetched once into that XCD's L2 and reused by its other query tiles.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int kXcd = 8;
  const int xcd = wg % kXcd, pos = wg / kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  return xcd < rem ? xcd * (per + 1) + pos : rem * (per + 1) + (xcd - rem) * per + pos;
}

// LDS tile layouts.  The LDS has 64 four-byte banks (256 bytes per cycle): a
// 128-bit read is served 16 lanes per cycle and a 64-bit (transposing) read
// 32 lanes per cycle.  Rows are padded rather than swizzled, so that every
// operand read of a tile is one per-lane base address plus a compile-time
// offset (no address arithmetic, and no address registers, per read):
//   * K rows (read 16 consecutive rows x one 16-byte chunk at a time) are
//     followed by one 16-byte pad granule, which staggers consecutive rows
//     by 4 banks (row bytes + 16 is 4 mod 64 words for every row size here).
//   * V rows are read by the transposing reads as 4 consecutive rows x 64
//     contiguous bytes (16-bit values) or rows {r..r+3, r+8..r+11} x 32
//     contiguous bytes (8-bit values); pads after every 1, 2 or 8 rows give
//     each of those rows its own bank range.  The byte offset of row r is
//     RB*r + PA*(r >> SA) + PB*(r >> SB); groups of 2^SG rows repeat the same
//     pattern, and every read's 16-row block offset is a multiple of a group.
template <int RB, bool FP8>
struct VLayout {
  static_assert(RB == 64 || RB == 128 || RB == 256, "row size");
  static constexpr int PA = FP8 ? 32 : 64;
  static constexpr int SA = FP8 ? (RB == 64 ? 3 : 1) : (RB == 256 ? 0 : 1);
  static constexpr int PB = FP8 && RB == 128 ? 64 : 0;
  static constexpr int SB = 3;
  static constexpr int SG = PB ? SB : SA;               // log2 rows per group
  static constexpr int kGroupRows = 1 << SG;
  __host__ __device__ static constexpr int row(int r) { return RB * r + PA * (r >> SA) + (PB ? PB * (r >> SB) : 0); }
  static constexpr int kGroupBytes = row(kGroupRows);   // bytes from one group to the next
  static_assert(kGroupBytes % 16 == 0 && 16 % kGroupRows == 0, "groups of whole granules within 16 rows");
};

// Software pipeline over a fixed sequence of N matrix instructions whose A
// operands come from LDS: the operand of instruction i + DEPTH is read right
// after instruction i issues, so every read has DEPTH instructions' time to
// land.  Instructions [0, NPV) take two operand reads each, the rest one.
// The sched_group_barrier sequence pins that order through scheduling (left
// alone, the scheduler sinks each read next to its use).
template <int I, int N, int NPV, int DEPTH, int MPO, int QKR>
__device__ __forceinline__ void pipeline_order() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, MPO, 0);  // the step's matrix instructions
    if constexpr (I + DEPTH < N) __builtin_amdgcn_sched_group_barrier(0x100, I + DEPTH < NPV ? 2 : QKR, 0);  // its reads
    pipeline_order<I + 1, N, NPV, DEPTH, MPO, QKR>();
  }
}

// MPO: matrix instructions per step (one per query block that shares the
// operand).  QKR: LDS reads per step from NPV on (1, or 2 where a step also
// reads a query operand from LDS).  Read returns the step's operands, of one
// type for every step.
template <int N, int NPV, int DEPTH, int MPO, int QKR = 1, class Read, class Mma>
__device__ __forceinline__ void op_pipeline(Read read, Mma mma) {
  using Op = decltype(read(0));
  Op buf[DEPTH];
  constexpr int P = DEPTH < N ? DEPTH : N;
#pragma unroll
  for (int i = 0; i < P; ++i) buf[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    mma(i, buf[i % DEPTH]);
    if (i + DEPTH < N) buf[i % DEPTH] = read(i + DEPTH);
  }
  constexpr int kPro = (P < NPV ? P : NPV) * 2 + (P > NPV ? P - NPV : 0) * QKR;
  __builtin_amdgcn_sched_group_barrier(0x100, kPro, 0);  // the first DEPTH operands' reads
  pipeline_order<0, N, NPV, DEPTH, MPO, QKR>();
}

}  // namespace
}  // namespace fa
