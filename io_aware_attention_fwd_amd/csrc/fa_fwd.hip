// FlashAttention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup owns BR = NW * QW consecutive query rows of one (batch, head)
// slice and streams that slice's keys and values through LDS in tiles of BC
// rows, so the N x N score matrix only ever exists one BC-wide tile at a time,
// in registers (the block decomposition into on-chip tiles of page
// "FlashAttention与TensorRT 10集成", section "FlashAttention的技术革命"; the
// fused scale -> mask -> softmax -> weighted-sum sequence of its section
// "算子融合的极致优化").  Each row keeps a reference maximum and a running sum
// so that partial results are rescaled when a later tile raises the maximum
// (online softmax; not on the pages, the standard exact formulation).
//
// Decomposition (every product is a 32 x 32 matrix-core block):
//   * NW waves per workgroup, QW = 32 * QB query rows per wave.
//   * Scores are computed transposed, S^T = K Q^T: A = 32 keys read from LDS,
//     B = 32 of the wave's queries, held in registers for the whole kernel.
//     In the accumulator layout each lane then owns one query per 32-row
//     block (lane % 32) and 16 of the block's keys, so row max and row sum
//     are lane-local plus one exchange between the two half-waves.  With
//     QB = 2 every K operand read from LDS feeds two instructions.
//   * O^T = V^T P^T: B = the probabilities taken straight from the score
//     accumulators (converted to 16 bits in place, no data movement), A = V^T
//     read from the row-major V tile with the transposing LDS reads of gfx950
//     (ds_read_b64_tr_b16, or ds_read_b64_tr_b8 for fp8 values, which are then
//     widened exactly to bfloat16).
//   * K and V tiles go HBM -> LDS with buffer loads that write LDS directly
//     (no registers, out-of-range rows read as zero), double buffered: tile
//     t+1 is in flight while tile t is computed; one barrier per tile.
//   * LDS rows are padded so that operand reads are free of bank conflicts
//     and need no per-read address arithmetic.
//   * Rescaling is lazy and exact: the first tile sets each row's reference
//     maximum; later tiles are exponentiated against the current reference
//     without taking their own maxima, and only a lane whose partial sum over
//     the tile leaves [0, 2^15] (so a probability might leave the 16-bit
//     range of the P operand) sends its wave back to take the tile's maxima,
//     raise the references (by more than 2^8 in the exp2 domain, or not at
//     all), rescale O and l, and exponentiate again.  The row maxima are the
//     one softmax step whose vector work this removes from most tiles.
//   * Causal: tiles right of a wave's last row are skipped; tiles that cross
//     the diagonal (and the ragged last tile) are masked element-wise.
//   * exp is v_exp_f32 (exp2) with scale * log2(e) folded into one fma; for
//     binary16 at d = 64, where the vector work bounds the kernel, Q is
//     multiplied by scale * log2(e) as it is loaded and each score
//     accumulator starts at minus its row's reference, so the matrix
//     instructions deliver the exponent directly.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_variants.h"

namespace fa {
namespace {

template <class Tr, int D, int QW, int NW, int BC>
struct Shape {
  static constexpr int kQB = QW / 32;         // 32-query blocks per wave
  static constexpr int kKB = BC / 32;         // 32-key blocks per tile
  static constexpr int kDB = D / 32;          // 32-wide blocks of the head dimension
  static constexpr int kBR = NW * QW;         // query rows per workgroup
  static constexpr int kRK = D * Tr::kEK;     // bytes per K row
  static constexpr int kRV = D * Tr::kEV;     // bytes per V row
  static constexpr int kCK = kRK / 16;        // 16-byte chunks per K row
  static constexpr int kCV = kRV / 16;
  static constexpr int kRSK = kRK + 16;       // LDS bytes per K row (one pad granule)
  static constexpr int kGK = kCK + 1;         // LDS granules per K row
  static constexpr int kGranK = BC * kGK;     // LDS granules per K stage
  static constexpr int kSK = BC * kRSK;       // bytes per K stage
  using VL = VLayout<kRV, Tr::kFp8>;
  static constexpr int kGV = VL::kGroupBytes / 16;         // LDS granules per group of V rows
  static constexpr int kGranV = BC / VL::kGroupRows * kGV;  // LDS granules per V stage
  static constexpr int kSV = kGranV * 16;                   // bytes per V stage
  static constexpr int kBlkK = (kGranK + 63) / 64;  // direct-load instructions (64 granules each) per K stage
  static constexpr int kBlkV = (kGranV + 63) / 64;
  // Stage allocations are whole direct-load blocks, so the lanes of a partial
  // last block write into the stage's own tail.
  static constexpr int kAllocK = kBlkK * 1024;
  static constexpr int kAllocV = kBlkV * 1024;
  static constexpr int kJK = (kBlkK + NW - 1) / NW;  // direct loads per wave per K stage (at most)
  static constexpr int kJV = (kBlkV + NW - 1) / NW;
  static constexpr int kQSteps = Tr::kFp8 ? D / 64 : D / 16;  // QK instructions per 32x32 block
  static constexpr int kKReads = kKB * kQSteps * (Tr::kFp8 ? 2 : 1);  // 128-bit LDS reads of K per tile
  static constexpr int kQKMfma = kKB * kQSteps * kQB;                 // Q K^T instructions per tile
  static_assert(BC % 32 == 0, "whole 32-key blocks");
};

// Binary16 inputs whose Q the kernel multiplies by c = scale * log2(e) and
// rounds to binary16 as it loads it (relative error 2^-11 per element).  The
// host takes these instances only for d = 64 and c in [2^-4, 1], where the
// product can neither overflow binary16 nor fall far into its subnormals.
struct TrF16Scaled : TrF16 {};
template <class Tr>
constexpr bool kScaledQ = std::is_same<Tr, TrF16Scaled>::value;
typedef unsigned long long u64;
typedef u64 u64x8 __attribute__((ext_vector_type(8)));  // a score block as eight 64-bit pairs

}  // namespace

// Binary16 at d = 64 with Q pre-multiplied by p.c (defined in the object
// built with FA_FWD_PART 3; taken without dropout when p.c lies in [2^-4, 1]).
hipError_t launch_fwd_f16_scaled(bool causal, const FwdParams& p, hipStream_t stream);

// The kernel template has external linkage so that every instantiation's
// host-side launch stub is emitted.
// SCHED: 0 = plain (every wave runs Q K^T, softmax, P V of a tile in turn),
//        1 = ping-pong between wave groups.
// DROP: dropout on the probabilities (kept iff the score's Philox byte is
// below p.drop_t; the 256/t rescale is part of p.o_mul).
template <class Tr, int D, bool CAUSAL, int QW, int NW, int BC, int SCHED, int WPE, bool DROP>
__global__ __launch_bounds__(NW * 64, WPE) void fa_fwd_kernel(FwdParams p) {
  constexpr bool PP = SCHED == 1;
  // Q pre-multiplied by c, and each score accumulator started at minus its
  // row's reference: the matrix instructions then deliver S*c - m and the
  // softmax needs no fma per score (d = 64, where vector work bounds the
  // kernel; at d = 128 the extra register block measured slower).
  constexpr bool kPS = kScaledQ<Tr> && D == 64 && !DROP;
  // Row sums of binary16 probabilities from the packed pairs only where
  // several independent waves of a SIMD run their softmax at once (plain
  // schedule): measured faster there, slower in the lone softmax wave of the
  // ping-pong schedule, and slower with the causal mask unless Q is
  // pre-scaled (there they also keep the four-wave kernel within its
  // registers).
  constexpr bool kPackedSum = !Tr::kPvBf16 && !PP && (!CAUSAL || kPS);
  static_assert(!PP || NW == 8 || NW == 16, "the ping-pong schedule splits the waves into two groups that each hold NW/8 waves of every SIMD");
  using S = Shape<Tr, D, QW, NW, BC>;
  constexpr bool kBf = Tr::kPvBf16;
  // Two LDS stages.  Separate arrays let the compiler tell the
  // direct-to-LDS loads of one stage from the reads of the other (with one
  // array and computed offsets it waits for every load before any read).
  __shared__ __attribute__((aligned(16))) char lds_k0[S::kAllocK];
  __shared__ __attribute__((aligned(16))) char lds_k1[S::kAllocK];
  __shared__ __attribute__((aligned(16))) char lds_v0[S::kAllocV];
  __shared__ __attribute__((aligned(16))) char lds_v1[S::kAllocV];

  // With 64-row waves at d = 128 and 16-bit values the second 32-row query
  // block's Q operands live in LDS (one padded row per query, laid out like a
  // K tile), so that the O accumulators and scores fit the register budget of
  // two waves per SIMD; each wave reads only its own rows.
  constexpr bool kQ1Lds = !Tr::kFp8 && QW == 64 && D == 128;
  __shared__ __attribute__((aligned(16))) char lds_q1[kQ1Lds ? NW * 32 * S::kRSK : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int q1base = (wave * 32 + l32) * S::kRSK + 16 * half;  // this lane's row of lds_q1, k-group `half`

  // Dense causal grids give each workgroup two query tiles of one slice,
  // n-1-i and i (the longest with the shortest), so that every workgroup has
  // the same work.  The long tile walks its keys up from key 0 and the short
  // one walks them down to key 0: a slice's workgroups start and end
  // together, and in both phases they read the same K/V tile at about the
  // same time, so a slice whose K and V exceed an XCD's L2 is still fetched
  // from HBM about once.  Packed batches of mixed lengths keep one query tile
  // per workgroup, longest first (measured faster there).
  const bool paired = CAUSAL && !p.cu;
  const int tile = xcd_remap(blockIdx.x, p.total_wg);
  const int per_slice = paired ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
  const int bh = tile / per_slice;
  const int pair = tile - bh * per_slice;
  const int b = bh / p.H, h = bh - b * p.H;
  // Rows of this (sequence, head) slice.  Packed sequences read their bounds
  // from cu; an inconsistent pair (negative, decreasing or past the end)
  // makes the sequence empty, so no access can leave the tensors.
  int N = p.N, row0 = 0;
  if (p.cu) {
    const int s0 = p.cu[b], s1 = p.cu[b + 1];
    const bool ok = 0 <= s0 && s0 <= s1 && s1 <= p.total && s1 - s0 <= p.N;
    N = ok ? s1 - s0 : 0;
    row0 = ok ? s0 : 0;
  }
  const int rowb = p.in_row;  // bytes from one row of the slice to the next
  const size_t in_base = (size_t)b * p.in_batch + (size_t)h * p.in_head + (size_t)row0 * rowb;
  const u32 slice_bytes = (u32)N * (u32)rowb;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + in_base, slice_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + in_base, slice_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)p.v + in_base, slice_bytes);

  const int nq = p.n_qtiles;
  const int n_jobs = paired && 2 * pair + 1 < nq ? 2 : 1;
  for (int job = 0; job < n_jobs; ++job) {
    const int qt = !CAUSAL ? pair : job == 0 ? nq - 1 - pair : pair;  // longest first
    const bool down = paired && job == 1;  // keys from the diagonal down to key 0
    if (job > 0) __syncthreads();  // the first tile's LDS stages and Q rows are free again
    const int q0 = qt * S::kBR;
    if (q0 >= N) continue;  // the whole workgroup: this query tile is past the sequence
    const int qw0 = q0 + wave * QW;  // first query row of this wave

    // ---- Q operands, kept in registers.  Lane (half, l32) of query block qb
    // holds row qw0 + 32*qb + l32; k-group `half` of each instruction step.
    u32x4 q16[S::kQB][Tr::kFp8 ? 1 : S::kQSteps];
    i32x8 q8[S::kQB][Tr::kFp8 ? S::kQSteps : 1];
    // Byte offset of the lane's first Q row, opaque to the compiler: it would
    // otherwise keep the other query block's offset live through the job.
    int qrow = (qw0 + l32) * rowb;
    asm volatile("" : "+v"(qrow));
#pragma unroll
    for (int qb = 0; qb < S::kQB; ++qb) {
      const int rowoff = qrow + 32 * qb * rowb;
      if constexpr (Tr::kFp8) {
#pragma unroll
        for (int s = 0; s < S::kQSteps; ++s) {
          const int off = rowoff + 64 * s + 32 * half;
          const u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
          const u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            q8[qb][s][e] = (int)((x0[e] ^ p.q_xor) & p.q_and);
            q8[qb][s][4 + e] = (int)((x1[e] ^ p.q_xor) & p.q_and);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < S::kQSteps; ++s) {
          u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, rowoff + (16 * s + 8 * half) * 2, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (x[e] ^ p.q_xor) & p.q_and;
          if constexpr (kPS) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // copied out first: this compiler's __builtin_bit_cast of a
              // vector-element expression reads element 0
              const u32 w = x[e];
              const f32x2 f = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
              x[e] = pack_p<false>(f[0] * p.c, f[1] * p.c);
            }
          }
          if (kQ1Lds && qb == 1)
            *reinterpret_cast<u32x4*>(lds_q1 + q1base + 32 * s) = x;
          else
            q16[qb][s] = x;
        }
      }
    }

    FA_SYNC_POINT();  // (debug build) Q in registers and LDS before anything else

    // B operand of query block qb, instruction step s (16-bit values)
    auto qop = [&](int qb, int s) __attribute__((always_inline)) {
      return kQ1Lds && qb == 1 ? lds_read_b128(lds_q1, q1base + 32 * s) : q16[qb][s];
    };

    const int n_all = (N + BC - 1) / BC;
    const int n_kv = CAUSAL ? min(n_all, (q0 + S::kBR - 1) / BC + 1) : n_all;
    // key tile of step i (steps are counted in the order the tiles are visited)
    auto ktile = [&](int i) __attribute__((always_inline)) { return down ? n_kv - 1 - i : i; };

    // ---- direct HBM -> LDS tile loads.  Lane L of direct-load instruction
    // `blk` writes LDS granule 64*blk + L of the stage and fetches the chunk of
    // the tile that the layout places there.  Lanes whose granule is padding
    // (or past the tile, in a partial last block) fetch a harmless in-bounds
    // duplicate instead of being masked off, so a load is one instruction with
    // no exec-mask branches.  The per-lane source offsets within a tile are
    // computed once and the tile's offset is added per load; it stays in the
    // per-lane offset (not the scalar one) because only that part is checked
    // against the slice's range, which zero-fills the rows past N of the last
    // tile.  The block index (uniform within the wave) is a scalar.
    int koff[S::kJK], voff[S::kJV], kblk[S::kJK], vblk[S::kJV];
#pragma unroll
    for (int j = 0; j < S::kJK; ++j) {
      kblk[j] = __builtin_amdgcn_readfirstlane(wave + j * NW);
      const int g = (wave + j * NW) * 64 + lane;
      const int r = g / S::kGK;
      const int c = min(g - r * S::kGK, S::kCK - 1);  // the pad granule repeats the row's last chunk
      koff[j] = r * rowb + c * 16;
    }
#pragma unroll
    for (int j = 0; j < S::kJV; ++j) {
      vblk[j] = __builtin_amdgcn_readfirstlane(wave + j * NW);
      const int g = (wave + j * NW) * 64 + lane;
      const int grp = g / S::kGV;
      const int off = (g - grp * S::kGV) * 16;  // byte offset inside the group of rows
      int r = grp * S::VL::kGroupRows, c = 0;    // pad granules repeat the group's first chunk
#pragma unroll
      for (int i = 0; i < S::VL::kGroupRows; ++i)
        if (off >= S::VL::row(i) && off < S::VL::row(i) + S::kRV) {
          r = grp * S::VL::kGroupRows + i;
          c = (off - S::VL::row(i)) / 16;
        }
      voff[j] = r * rowb + c * 16;
    }
    auto issue_k = [&](int kt, char* dk) __attribute__((always_inline)) {
      const int toff = ktile(kt) * BC * rowb;
#pragma unroll
      for (int j = 0; j < S::kJK; ++j)
        if (kblk[j] < S::kBlkK) load_lds16(rk, dk + kblk[j] * 1024, koff[j] + toff);
    };
    auto issue_v = [&](int kt, char* dv) __attribute__((always_inline)) {
      const int toff = ktile(kt) * BC * rowb;
#pragma unroll
      for (int j = 0; j < S::kJV; ++j)
        if (vblk[j] < S::kBlkV) load_lds16(rv, dv + vblk[j] * 1024, voff[j] + toff);
    };

    f32x16 oacc[S::kDB][S::kQB];
#pragma unroll
    for (int db = 0; db < S::kDB; ++db)
#pragma unroll
      for (int qb = 0; qb < S::kQB; ++qb) oacc[db][qb] = f32x16{};
    float mref[S::kQB], lsum[S::kQB];  // reference max (exp2 domain) and this half-wave's running sum
#pragma unroll
    for (int qb = 0; qb < S::kQB; ++qb) {
      mref[qb] = -INFINITY;
      lsum[qb] = 0.f;
    }
    const float c = p.c;
    // The reference a row's scores are taken against (0 before the first),
    // and the accumulator start of a score block: minus that reference when Q
    // is pre-scaled, else 0.
    auto ref_off = [&](int qb) __attribute__((always_inline)) { return mref[qb] == -INFINITY ? 0.f : mref[qb]; };
    // The accumulator start blocks of this tile's score blocks, built once
    // per Q K^T product (prep_qk) from eight 64-bit moves of a (-ref, -ref)
    // pair (the compiler would spend fifteen 32-bit ones; volatile, so that
    // they are not merged into one move and copies).
    f32x16 qinit[kPS ? S::kQB : 1];
    auto prep_qk = [&]() __attribute__((always_inline)) {
      if constexpr (kPS) {
#pragma unroll
        for (int qb = 0; qb < S::kQB; ++qb) {
          const u32 nb = __float_as_uint(-ref_off(qb));
          const u64 pr = ((u64)nb << 32) | nb;
          u64x8 r;
#pragma unroll
          for (int i = 0; i < 8; ++i) asm volatile("v_mov_b64 %0, %1" : "=v"(r[i]) : "v"(pr));
          qinit[qb] = __builtin_bit_cast(f32x16, r);
        }
      }
    };
    auto qk_init = [&](int qb) __attribute__((always_inline)) {
      if constexpr (kPS)
        return qinit[qb];
      else
        return f32x16{};
    };

    // Scores of the tile between its matrix phase and its softmax phase, and
    // probabilities between the softmax phase and the next matrix phase.
    f32x16 sacc[S::kKB][S::kQB];
    u32x4 pb[S::kKB][S::kQB][2];

    // Operand registers.  All LDS reads of a product are issued before its
    // first matrix instruction so that their latencies overlap.
    u32x4 kop16[S::kKB][Tr::kFp8 ? 1 : S::kQSteps];
    i32x8 kop8[S::kKB][Tr::kFp8 ? S::kQSteps : 1];
    u32x4 vop16[S::kDB][S::kKB][2];
    u32x2 vop8[S::kDB][S::kKB][Tr::kFp8 ? 2 : 1];

    // ---- K operands: lane (half, l32) of block kb reads key row 32*kb + l32,
    // k-group `half` of each instruction step (two 16-byte chunks for 8-bit
    // values, one otherwise).
    const int kbase = l32 * S::kRSK + half * (Tr::kFp8 ? 32 : 16);
    auto k_read16 = [&](const char* lk, int kb, int s) __attribute__((always_inline)) {
      return lds_read_b128(lk, kbase + 32 * kb * S::kRSK + 32 * s);
    };
    auto k_read8 = [&](const char* lk, int kb, int s) __attribute__((always_inline)) {
      const u32x4 a0 = lds_read_b128(lk, kbase + 32 * kb * S::kRSK + 64 * s);
      const u32x4 a1 = lds_read_b128(lk, kbase + 32 * kb * S::kRSK + 64 * s + 16);
      return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    };
    auto load_k = [&](const char* lk) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
        for (int s = 0; s < S::kQSteps; ++s) {
          if constexpr (Tr::kFp8)
            kop8[kb][s] = k_read8(lk, kb, s);
          else
            kop16[kb][s] = k_read16(lk, kb, s);
        }
    };

    // ---- S^T = K Q^T into `dst`
    auto mma_qk_into = [&](f32x16 (&dst)[S::kKB][S::kQB]) __attribute__((always_inline)) {
      prep_qk();
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb) {
#pragma unroll
        for (int qb = 0; qb < S::kQB; ++qb) dst[kb][qb] = qk_init(qb);
#pragma unroll
        for (int s = 0; s < S::kQSteps; ++s)
#pragma unroll
          for (int qb = 0; qb < S::kQB; ++qb) {
            if constexpr (Tr::kFp8)
              dst[kb][qb] = mfma_fp8(kop8[kb][s], q8[qb][s], dst[kb][qb]);
            else
              dst[kb][qb] = mfma16(kop16[kb][s], qop(qb, s), dst[kb][qb], kBf);
          }
      }
    };
    auto mma_qk = [&]() __attribute__((always_inline)) { mma_qk_into(sacc); };

    using SArr = f32x16[S::kKB][S::kQB];

    // ---- mask keys past N and (causal) keys after the query
    auto mask_tile = [&](int kt, SArr& sc) __attribute__((always_inline)) {
      const int k0 = ktile(kt) * BC;
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < S::kQB; ++qb) {
          const int qi = qw0 + 32 * qb + l32;
          const int lim = CAUSAL ? min(qi, N - 1) : N - 1;  // last visible key
          // element r of block kb holds key k0 + 32*kb + 8*(r/4) + 4*half + r%4; comparing the
          // compile-time part of that offset with one per-lane bound needs no per-element address
#pragma unroll
          for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              if (key > lim) sc[kb][qb][r] = -INFINITY;
            }
        }
      }
    };

    // ---- online softmax with lazy rescaling: row maxima, then (rarely) a new
    // reference maximum with O and l rescaled.  Reductions use independent
    // partial results so that no long dependency chain forms.  mq: the
    // references the scores were formed against (pre-scaled Q).
    auto max_rescale = [&](SArr& sc, const float (&mq)[S::kQB]) __attribute__((always_inline)) {
      float mx[S::kQB];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < S::kQB; ++qb) {
        // IEEE maximum (v_maximum3_f32): no NaN quieting of the inputs needed
        float part[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            part[r / 2 & 1] = __builtin_elementwise_maximum(
                part[r / 2 & 1], __builtin_elementwise_maximum(sc[kb][qb][r], sc[kb][qb][r + 1]));
        const float m = __builtin_elementwise_maximum(part[0], part[1]);
        mx[qb] = kPS ? halves_max(m) + mq[qb] : halves_max(m) * c;
        grow |= mx[qb] > mref[qb] + kRescaleThreshold;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // some row of the wave needs a new reference
#pragma unroll
        for (int qb = 0; qb < S::kQB; ++qb) {
          const float mnew = fmaxf(mref[qb], mx[qb]);
          const float alpha = mnew == -INFINITY ? 1.f : exp2f(mref[qb] - mnew);
          mref[qb] = mnew;
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < S::kDB; ++db) oacc[db][qb] *= alpha;
        }
      }
    };

    // ---- probabilities P = exp2(S*c - m) as 16-bit pairs, row sums (spec:
    // the scores were formed against the current references).  With
    // dropout, one Philox call per lane and 32-key block gives the 16 bytes of
    // the lane's 16 scores: element r of the accumulator (key 8*(r/4) +
    // 4*half + r%4 of the block) takes byte r, i.e. bits 8*(r%4).. of word r/4.
    // The counter is (2 * block + half, query row, slice, offset).  Dropped
    // probabilities are zeroed in the P operand only: the row sum (and so the
    // normaliser and lse) is that of the whole row.
    auto exp_tile = [&](int kt, SArr& sc, float (&tsum)[S::kQB], const float (&mq)[S::kQB], bool spec)
                        __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < S::kQB; ++qb) {
        const float mb = ref_off(qb);
        const float sh = mq[qb] - mb;  // pre-scaled Q: from the scores' reference to the current one
        // independent partial sums per row: two where Q is pre-scaled (fewer
        // instructions to start and join them; measured +1.5 to +2 %), four
        // elsewhere (shorter dependency chains for a lone softmax wave)
        constexpr int kChains = kPS ? 2 : 4;
        float rs[kChains];
#pragma unroll
        for (int kb = 0; kb < S::kKB; ++kb) {
          u32x4 rnd{};
          if constexpr (DROP)
            rnd = philox4x32_10(2u * (u32)(ktile(kt) * S::kKB + kb) + (u32)half, (u32)(qw0 + 32 * qb + l32), (u32)bh,
                                p.drop_offset, p.seed_lo, p.seed_hi);
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float s0 = sc[kb][qb][8 * t + 2 * e], s1 = sc[kb][qb][8 * t + 2 * e + 1];
              const float p0 = __builtin_amdgcn_exp2f(kPS ? (spec ? s0 : s0 + sh) : __builtin_fmaf(s0, c, -mb));
              const float p1 = __builtin_amdgcn_exp2f(kPS ? (spec ? s1 : s1 + sh) : __builtin_fmaf(s1, c, -mb));
              const u32 w = pack_p<kBf>(p0, p1);
              if constexpr (DROP) {
                // elements 8t+2e and 8t+2e+1: word 2t + e/2, bytes 2*(e%2) and 2*(e%2)+1
                const u32 word = rnd[2 * t + (e >> 1)] >> (16 * (e & 1));
                const u32 keep = ((word & 0xFFu) < p.drop_t ? 0x0000FFFFu : 0u) |
                                 (((word >> 8) & 0xFFu) < p.drop_t ? 0xFFFF0000u : 0u);
                pb[kb][qb][t][e] = w & keep;
              } else {
                pb[kb][qb][t][e] = w;
              }
              rs[e % kChains] =
                  sum_pair<kPackedSum>(w, p0, p1, kb == 0 && t == 0 && e < kChains ? 0.f : rs[e % kChains]);
            }
        }
        tsum[qb] = kChains == 2 ? rs[0] + rs[1] : (rs[0] + rs[1]) + (rs[2 % kChains] + rs[3 % kChains]);
      }
    };

    // Tiles after the first are exponentiated against the current reference
    // maximum without taking their own row maxima first.  The reference never
    // exceeds the row's running maximum, so nothing underflows that the plain
    // recurrence would keep; the danger is the other way, and a lane whose
    // partial sum over the tile stays within kSpeculativeSumLimit has every
    // probability within it, inside the 16-bit range of the P operand.  If any
    // lane of the wave exceeds it (or produced inf / NaN), the wave takes the
    // tile's maxima, raises its references, rescales, and exponentiates again.
    // A wave speculates only once every one of its rows has seen a visible key
    // in an earlier tile, so that the reference is finite and from data: from
    // the second tile on when walking up from key 0 (which every row sees), and
    // when walking down once the tiles already visited reach the wave's first
    // row (the diagonal tiles visited first may hold no visible key for some of
    // its rows).  Dropout tiles always take the maxima first.
    auto softmax = [&](int kt) __attribute__((always_inline)) {
      mask_tile(kt, sacc);
      float tsum[S::kQB], mq[S::kQB];
#pragma unroll
      for (int qb = 0; qb < S::kQB; ++qb) mq[qb] = ref_off(qb);
      if constexpr (!DROP) {
        if (down ? (ktile(kt) + 1) * BC <= qw0 : kt > 0) {
          exp_tile(kt, sacc, tsum, mq, true);
          bool redo = false;
#pragma unroll
          for (int qb = 0; qb < S::kQB; ++qb) redo |= !(tsum[qb] <= kSpeculativeSumLimit);
          if (__builtin_amdgcn_ballot_w64(redo) == 0) {
#pragma unroll
            for (int qb = 0; qb < S::kQB; ++qb) lsum[qb] += tsum[qb];
            return;
          }
        }
      }
      max_rescale(sacc, mq);
      exp_tile(kt, sacc, tsum, mq, false);
#pragma unroll
      for (int qb = 0; qb < S::kQB; ++qb) lsum[qb] += tsum[qb];
    };

    // ---- V^T operands.  Element e of lane (half, col) of the V^T operand is
    // V[32*kb + 16*t + 8*(e/4) + 4*half + e%4][col], matching the key held in
    // element e of the P operand (accumulator row 8*t + e of the S^T block).
    // 16-bit values: lane (g, u) = (lane / 16, lane % 16) reads 4 values of
    // columns 32*db + 16*(g%2) + 4*(u%4) from rows r0 = 32*kb + 16*t + 4*half +
    // u/4 and r0 + 8.  8-bit values: 8 keys of byte column 32*db + 16*(g%2) +
    // 8*(u%2) from the rows listed above, e = u/2.  Rows 32*kb + 16*t start a
    // group of the layout, so their offsets are compile-time constants.
    const int vbase = [&] {
      const int g = lane >> 4, u = lane & 15;
      if constexpr (Tr::kFp8) {
        const int ep = u >> 1;
        return S::VL::row(8 * (ep >> 2) + 4 * half + (ep & 3)) + 16 * (g & 1) + 8 * (u & 1);
      } else {
        return S::VL::row(4 * half + (u >> 2)) + 2 * (16 * (g & 1) + 4 * (u & 3));
      }
    }();
    auto v_read16 = [&](const char* lv, int db, int kb, int t) __attribute__((always_inline)) {
      const int o = vbase + S::VL::row(32 * kb + 16 * t) + 64 * db;
      const u32x2 lo = lds_read_tr16(lv, o);
      const u32x2 hi = lds_read_tr16(lv, o + S::VL::row(8));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    auto v_read8 = [&](const char* lv, int db, int kb, int t) __attribute__((always_inline)) {
      return lds_read_tr8(lv, vbase + S::VL::row(32 * kb + 16 * t) + 32 * db);
    };
    auto load_v = [&](const char* lv) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < S::kDB; ++db)
#pragma unroll
        for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if constexpr (Tr::kFp8)
              vop8[db][kb][t] = v_read8(lv, db, kb, t);
            else
              vop16[db][kb][t] = v_read16(lv, db, kb, t);
          }
    };

    // ---- O^T += V^T P^T (fp8 values are widened exactly to bfloat16 here)
    auto mma_pv = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < S::kDB; ++db)
#pragma unroll
        for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            u32x4 a;
            if constexpr (Tr::kFp8) {
              const u32x2 x = vop8[db][kb][t];
              const bf16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[0], 1.0f, false);
              const bf16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[0], 1.0f, true);
              const bf16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[1], 1.0f, false);
              const bf16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[1], 1.0f, true);
              a = u32x4{__builtin_bit_cast(u32, w0), __builtin_bit_cast(u32, w1), __builtin_bit_cast(u32, w2),
                        __builtin_bit_cast(u32, w3)};
            } else {
              a = vop16[db][kb][t];
            }
#pragma unroll
            for (int qb = 0; qb < S::kQB; ++qb) oacc[db][qb] = mfma16(a, pb[kb][qb][t], oacc[db][qb], kBf);
          }
    };

    // Interleaved forms: each operand is read right before its instruction,
    // which keeps fewer operand registers live (used where registers are short).
    auto qk_interleaved = [&](const char* lk) __attribute__((always_inline)) {
      prep_qk();
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb) {
#pragma unroll
        for (int qb = 0; qb < S::kQB; ++qb) sacc[kb][qb] = qk_init(qb);
#pragma unroll
        for (int s = 0; s < S::kQSteps; ++s) {
          if constexpr (Tr::kFp8) {
            const i32x8 a = k_read8(lk, kb, s);
#pragma unroll
            for (int qb = 0; qb < S::kQB; ++qb) sacc[kb][qb] = mfma_fp8(a, q8[qb][s], sacc[kb][qb]);
          } else {
            const u32x4 a = k_read16(lk, kb, s);
#pragma unroll
            for (int qb = 0; qb < S::kQB; ++qb) sacc[kb][qb] = mfma16(a, qop(qb, s), sacc[kb][qb], kBf);
          }
        }
      }
    };
    auto pv_interleaved = [&](const char* lv) __attribute__((always_inline)) {
      load_v(lv);
      mma_pv();
    };

    // A wave works on tile kt only if some of its rows exist and can see a key
    // of it.  (The row test also keeps the branch per-wave in the compiler's
    // eyes; with a workgroup-uniform branch it hoists work across the matrix
    // phase's alternatives and runs out of registers at d = 128.)
    auto active = [&](int kt) __attribute__((always_inline)) {
      return kt >= 0 && kt < n_kv && qw0 < N && !(CAUSAL && ktile(kt) * BC > qw0 + QW - 1);
    };

    // ---- main loop: ping-pong between two groups of waves on each SIMD.
    // Waves are dealt to the four SIMDs round-robin, so the first and second
    // halves of the workgroup (group 0 and group 1) each hold NW/8 waves of
    // every SIMD: one each with 8 waves, two each with 16 (whose softmax then
    // runs on two waves of a SIMD at once, at the higher two-wave issue rate).
    // Time is cut into phases separated by workgroup barriers; in every phase
    // one group runs matrix-core work (P V of the previous tile, Q K^T of the
    // current one) while the other runs the softmax of the tile it has scores
    // for, so each SIMD overlaps MFMAs of one group with VALU work of the other.
    //   phase 2t   : group 0 MFMA(t)            group 1 softmax(t-1)
    //   phase 2t+1 : group 0 softmax(t)         group 1 MFMA(t)
    // K(t) lives in stage t%2 for phases 2t..2t+1; V(t) in stage t%2 for phases
    // 2t+2..2t+3.  Both are issued at phase 2t (K one tile ahead) and waited for
    // at the end of phase 2t+1.
    const int group = wave / (NW / 2);
    // Matrix phase: P V of the previous tile, then Q K^T of this one.  For
    // 16-bit types both run as one pipelined stream of instructions (P V in
    // (kb, t, db) order, db fastest, so consecutive instructions feed
    // different accumulators; Q K^T in (step, kb) order).  The wave raises its
    // issue priority for the phase: the other wave of its SIMD is running the
    // vector-heavy softmax, and the matrix stream should not wait behind it.
    constexpr int kNPV = S::kDB * S::kKB * 2;
    constexpr int kNQK = S::kKB * S::kQSteps;
    // operand reads in flight (fewer where registers are short: four waves per
    // SIMD, or 64-row waves at d = 128)
    constexpr int kDepth = WPE >= 4 || (QW == 64 && D == 128) ? 2 : 4;
    // A step's LDS operands: the A operand, and for Q K^T steps with kQ1Lds the
    // second query block's B operand (left unused, and so never read, otherwise).
    struct Ops {
      u32x4 a, q1;
    };
    constexpr int kQKReads = kQ1Lds ? 2 : 1;
    auto pv_op = [&](int i, Ops o) __attribute__((always_inline)) {
      const int db = i % S::kDB, t = (i / S::kDB) % 2, kb = i / (2 * S::kDB);
#pragma unroll
      for (int qb = 0; qb < S::kQB; ++qb) oacc[db][qb] = mfma16(o.a, pb[kb][qb][t], oacc[db][qb], kBf);
    };
    auto qk_op = [&](int i, Ops o) __attribute__((always_inline)) {
      if (i == 0) prep_qk();  // the start blocks live from the first Q K^T instruction on
      const int kb = i % S::kKB, st = i / S::kKB;
#pragma unroll
      for (int qb = 0; qb < S::kQB; ++qb)
        sacc[kb][qb] = mfma16(o.a, kQ1Lds && qb == 1 ? o.q1 : q16[qb][st], st == 0 ? qk_init(qb) : sacc[kb][qb], kBf);
    };
    auto pv_rd = [&](const char* lv, int i) __attribute__((always_inline)) {
      return Ops{v_read16(lv, i % S::kDB, i / (2 * S::kDB), (i / S::kDB) % 2), u32x4{}};
    };
    auto qk_rd = [&](const char* lk, int i) __attribute__((always_inline)) {
      const int st = i / S::kKB;
      return Ops{k_read16(lk, i % S::kKB, st), kQ1Lds ? lds_read_b128(lds_q1, q1base + 32 * st) : u32x4{}};
    };
    auto mfma_phase = [&](int kt, const char* lk, const char* lv_prev) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);
      const bool a_pv = active(kt - 1), a_qk = active(kt);
      if constexpr (Tr::kFp8) {
        if (a_pv) pv_interleaved(lv_prev);
        if (a_qk) qk_interleaved(lk);
      } else if (a_pv && a_qk) {
        op_pipeline<kNPV + kNQK, kNPV, kDepth, S::kQB, kQKReads>(
            [&](int i) __attribute__((always_inline)) { return i < kNPV ? pv_rd(lv_prev, i) : qk_rd(lk, i - kNPV); },
            [&](int i, Ops o) __attribute__((always_inline)) {
              if (i < kNPV)
                pv_op(i, o);
              else
                qk_op(i - kNPV, o);
            });
      } else if (a_pv) {
        op_pipeline<kNPV, kNPV, kDepth, S::kQB>([&](int i) __attribute__((always_inline)) { return pv_rd(lv_prev, i); },
                                        [&](int i, Ops o) __attribute__((always_inline)) { pv_op(i, o); });
      } else if (a_qk) {
        op_pipeline<kNQK, 0, kDepth, S::kQB, kQKReads>([&](int i) __attribute__((always_inline)) { return qk_rd(lk, i); },
                                     [&](int i, Ops o) __attribute__((always_inline)) { qk_op(i, o); });
      }
      __builtin_amdgcn_s_setprio(0);
    };
    auto tile_step = [&](int kt, const char* lk, const char* lv_prev, char* k_next, char* v_cur) __attribute__((always_inline)) {
      if (kt + 1 < n_kv) issue_k(kt + 1, k_next);
      if (kt < n_kv) issue_v(kt, v_cur);
      FA_SYNC_POINT();
      if (group == 0) {
        mfma_phase(kt, lk, lv_prev);
      } else if (active(kt - 1)) {
        softmax(kt - 1);
      }
      __syncthreads();
      if (group == 0) {
        if (active(kt)) softmax(kt);
      } else {
        mfma_phase(kt, lk, lv_prev);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };

    if constexpr (SCHED == 1) {
      issue_k(0, lds_k0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      for (int kt = 0; kt <= n_kv; kt += 2) {
        tile_step(kt, lds_k0, lds_v1, lds_k1, lds_v0);
        if (kt + 1 <= n_kv) tile_step(kt + 1, lds_k1, lds_v0, lds_k0, lds_v1);
      }
    } else {
      // Plain schedule: every wave runs Q K^T, softmax and P V of a tile in
      // turn; with several workgroups per CU the waves of different
      // workgroups interleave matrix-core and vector work on each SIMD.
      auto plain_step = [&](int kt, const char* kc, const char* vc, char* kn, char* vn) __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile kt landed for every wave; the other stage is no longer read
        if (kt + 1 < n_kv) {
          issue_k(kt + 1, kn);
          issue_v(kt + 1, vn);
        }
        FA_SYNC_POINT();
        if (active(kt)) {
          if constexpr (WPE >= 4) {
            // Four waves per SIMD leave 128 registers: few operand registers
            // may be live, so Q K^T keeps two K operand reads in flight
            // (16-bit values) and P V reads its operands as it goes.
            if constexpr (!Tr::kFp8 && !kQ1Lds)
              op_pipeline<kNQK, 0, 2, S::kQB>([&](int i) __attribute__((always_inline)) { return qk_rd(kc, i); },
                                              [&](int i, Ops o) __attribute__((always_inline)) { qk_op(i, o); });
            else
              qk_interleaved(kc);
            softmax(kt);
            pv_interleaved(vc);
          } else {
            load_k(kc);
            mma_qk();
            // All K operand reads go out before the first Q K^T instruction.
            __builtin_amdgcn_sched_group_barrier(0x100, S::kKReads, 0);  // DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, S::kQKMfma, 0);  // matrix instructions
            __builtin_amdgcn_sched_barrier(0);
            load_v(vc);  // in flight during the softmax
            softmax(kt);
            mma_pv();
          }
        }
        FA_SYNC_POINT();
      };
      issue_k(0, lds_k0);
      issue_v(0, lds_v0);
      for (int kt = 0; kt < n_kv; kt += 2) {
        plain_step(kt, lds_k0, lds_v0, lds_k1, lds_v1);
        if (kt + 1 < n_kv) plain_step(kt + 1, lds_k1, lds_v1, lds_k0, lds_v0);
      }
    }

    FA_SYNC_POINT();
    // ---- epilogue: combine the half-wave sums, normalise, store.  The lane's
    // position is recomputed here: registers holding it through the loop made
    // the four-wave causal kernels spill.
    const int e_lane = lane_id(), e_half = e_lane >> 5, e_l32 = e_lane & 31;
#pragma unroll
    for (int qb = 0; qb < S::kQB; ++qb) {
      const int qi = qw0 + 32 * qb + e_l32;
      const float l_tot = halves_sum(lsum[qb]);
      const float inv = l_tot > 0.f ? p.o_mul / l_tot : 0.f;
      if (qi < N) {
        if (e_half == 0)
          p.lse[(size_t)b * p.lse_batch + (size_t)h * p.lse_head + row0 + qi] =
              l_tot > 0.f ? (mref[qb] + __log2f(l_tot)) * kLn2 : -INFINITY;
        char* orow = (char*)p.o + (size_t)b * p.out_batch + (size_t)h * p.out_head + (size_t)(row0 + qi) * p.out_row;
#pragma unroll
        for (int db = 0; db < S::kDB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const int col = 32 * db + 8 * a4 + 4 * e_half;
            u32x2 w;
            w[0] = pack_p<kBf>(oacc[db][qb][4 * a4 + 0] * inv, oacc[db][qb][4 * a4 + 1] * inv);
            w[1] = pack_p<kBf>(oacc[db][qb][4 * a4 + 2] * inv, oacc[db][qb][4 * a4 + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + col * 2) = w;
          }
      }
    }
  }
}

namespace {

// ---------------------------------------------------------------- instances
template <class Tr, int D, bool CAUSAL, int QW, int NW, int BC, int SCHED, int WPE, bool DROP>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<Tr, D, CAUSAL, QW, NW, BC, SCHED, WPE, DROP>), dim3(p.total_wg), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <class Tr, int D, bool CAUSAL>
hipError_t dispatch_variant(int v, const FwdParams& p, hipStream_t stream) {
  switch (v) {
    case 1: return launch_one<Tr, D, CAUSAL, 32, 4, 64, 0, 4, false>(p, stream);
    case 2: return launch_one<Tr, D, CAUSAL, 32, 4, 64, 0, 3, false>(p, stream);
    case 3: return launch_one<Tr, D, CAUSAL, 32, 4, 64, 0, 2, false>(p, stream);
    case 4: return launch_one<Tr, D, CAUSAL, 64, 4, 64, 0, 2, false>(p, stream);
    case 5:
      // 64-row ping-pong waves exist for d = 64 only (at d = 128 they would
      // spill); selected_variant never picks them for d = 128
      if constexpr (D == 64) return launch_one<Tr, D, CAUSAL, 64, 8, 64, 1, 2, false>(p, stream);
      return hipErrorInvalidValue;
    case 6:
      if constexpr (D == 64) return launch_one<Tr, D, CAUSAL, 32, 16, 64, 1, 4, false>(p, stream);
      return hipErrorInvalidValue;
    case 7:
      if constexpr (D == 64) return launch_one<Tr, D, CAUSAL, 32, 8, 64, 0, 4, false>(p, stream);
      return hipErrorInvalidValue;
    case 8:
      if constexpr (D == 128) return launch_one<Tr, D, CAUSAL, 64, 8, 32, 1, 2, false>(p, stream);
      return hipErrorInvalidValue;
    default: return launch_one<Tr, D, CAUSAL, 32, 8, 64, 1, 2, false>(p, stream);
  }
}

// Dropout: only the shapes default_variant picks for the 16-bit types
// (d = 128: ping-pong; d = 64: 32 rows per wave, or 64 without the causal mask).
template <class Tr, int D, bool CAUSAL>
hipError_t dispatch_dropout(int v, const FwdParams& p, hipStream_t stream) {
  if constexpr (D == 128) {
    if (v == 0) return launch_one<Tr, D, CAUSAL, 32, 8, 64, 1, 2, true>(p, stream);
  } else {
    if (v == 2) return launch_one<Tr, D, CAUSAL, 32, 4, 64, 0, 3, true>(p, stream);
    if constexpr (!CAUSAL) {
      if (v == 4) return launch_one<Tr, D, CAUSAL, 64, 4, 64, 0, 2, true>(p, stream);
    }
  }
  return hipErrorInvalidValue;
}

template <class Tr>
hipError_t dispatch_dtype(Dtype dt, int d, bool causal, const FwdParams& p, hipStream_t stream) {
  const bool drop = p.drop_t < 256;
  const int v = p.variant;
  if constexpr (std::is_same<Tr, TrF16>::value) {
    if (!drop && d == 64 && p.c >= 0.0625f && p.c <= 1.0f) return launch_fwd_f16_scaled(causal, p, stream);
  }
  if constexpr (!Tr::kFp8) {
    if (drop) {
      if (d == 64)
        return causal ? dispatch_dropout<Tr, 64, true>(v, p, stream) : dispatch_dropout<Tr, 64, false>(v, p, stream);
      return causal ? dispatch_dropout<Tr, 128, true>(v, p, stream) : dispatch_dropout<Tr, 128, false>(v, p, stream);
    }
  } else {
    if (drop) return hipErrorInvalidValue;
  }
  if (d == 64) return causal ? dispatch_variant<Tr, 64, true>(v, p, stream) : dispatch_variant<Tr, 64, false>(v, p, stream);
  return causal ? dispatch_variant<Tr, 128, true>(v, p, stream) : dispatch_variant<Tr, 128, false>(v, p, stream);
}

}  // namespace

// The instances of one dtype per object when FA_FWD_PART is 0, 1 or 2 (the
// build compiles this file once per dtype, side by side), the pre-scaled
// binary16 ones when it is 3; all of them when it is undefined.
#ifndef FA_FWD_PART
#define FA_FWD_PART -1
#endif
#if FA_FWD_PART < 0 || FA_FWD_PART == 0
hipError_t launch_fwd_f16(int d, bool causal, const FwdParams& p, hipStream_t stream) {
  return dispatch_dtype<TrF16>(Dtype::F16, d, causal, p, stream);
}

hipError_t launch_fwd(Dtype dt, int d, bool causal, const FwdParams& p, hipStream_t stream) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  switch (dt) {
    case Dtype::F16: return launch_fwd_f16(d, causal, p, stream);
    case Dtype::BF16: return launch_fwd_bf16(d, causal, p, stream);
    case Dtype::FP8: return launch_fwd_fp8(d, causal, p, stream);
  }
  return hipErrorInvalidValue;
}
#endif
#if FA_FWD_PART < 0 || FA_FWD_PART == 1
hipError_t launch_fwd_bf16(int d, bool causal, const FwdParams& p, hipStream_t stream) {
  return dispatch_dtype<TrBF16>(Dtype::BF16, d, causal, p, stream);
}
#endif
#if FA_FWD_PART < 0 || FA_FWD_PART == 2
hipError_t launch_fwd_fp8(int d, bool causal, const FwdParams& p, hipStream_t stream) {
  return dispatch_dtype<TrFP8>(Dtype::FP8, d, causal, p, stream);
}
#endif
#if FA_FWD_PART < 0 || FA_FWD_PART == 3
hipError_t launch_fwd_f16_scaled(bool causal, const FwdParams& p, hipStream_t stream) {
  return causal ? dispatch_variant<TrF16Scaled, 64, true>(p.variant, p, stream)
                : dispatch_variant<TrF16Scaled, 64, false>(p.variant, p, stream);
}
#endif

}  // namespace fa
