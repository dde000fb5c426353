// FlashAttention backward pass for gfx950 (MI355X, CDNA4): dQ, dK, dV from
// Q, K, V, the forward output O, its logsumexp and the output gradient dO.
//
// The probabilities are recomputed from Q, K and the saved logsumexp instead
// of being read back (the "0 MB (重计算)" attention row of the Flash
// Attention 2 memory table on page "Optimization Flash Attention 基准测试"):
//   P = exp(scale*Q K^T - lse) (masked),   dV = P^T dO,   dP = dO V^T,
//   dS = P * (dP - D) with D_i = sum_c dO_ic O_ic,   dQ = scale * dS K,
//   dK = scale * dS^T Q.
//
// Two kernels on one stream, no atomics:
//   * dQ kernel: one workgroup per block of 128 queries of one (batch, head)
//     (4 waves x 32 queries).  It writes D for its queries to the workspace,
//     streams K/V tiles of 64 keys through LDS and accumulates dQ^T = K^T dS^T
//     exactly like the forward pass accumulates O^T = V^T P^T: scores are
//     computed transposed (S^T = K Q^T, dP^T = V dO^T) so every lane owns one
//     query, dS^T feeds the matrix instruction straight from the accumulators,
//     and K^T comes from transposing LDS reads.
//   * dK/dV kernel: one workgroup per block of 128 keys (4 waves x 32 keys),
//     K and V rows held in registers, query tiles of 32 rows (Q, dO, lse, D)
//     streamed through LDS.  S = Q K^T and dP = dO V^T give every lane one
//     key; dV^T += dO^T P and dK^T += Q^T dS take P and dS from the
//     accumulators and dO^T, Q^T from transposing LDS reads.
// Masked scores are set to -inf after the scale is applied (the scale may be
// negative here), so their probabilities are exactly 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.44269504088896341f;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A 16-bit tile that is read both by rows (128-bit reads: 16 consecutive
// rows x 16 bytes per cycle) and transposed: the V layout of fa_device.h plus
// a 16-byte pad after every 4 rows.  Row r = 4a + b then starts at 64b + 16a
// bytes modulo 256 at both row sizes, so the 16 rows of a row read land on
// 16 different 4-bank groups, while each 4-row group of a transposing read
// still fills the four 64-byte quarters.  In the V layout alone rows r, r+4,
// r+8 and r+12 share their banks (a four-way conflict on every row read).
template <int RB>
struct RowsLayout {
  using V = VLayout<RB, false>;
  static_assert(4 % V::kGroupRows == 0, "the V layout's groups divide 4 rows");
  static constexpr int kGroupRows = 4;
  __host__ __device__ static constexpr int row(int r) { return V::row(r) + 16 * (r >> 2); }
  static constexpr int kGroupBytes = row(kGroupRows);  // bytes from one group to the next
};

template <int D>
struct BwdShape {
  static constexpr int kDB = D / 32;      // 32-wide blocks of the head dimension
  static constexpr int kSteps = D / 16;   // 16-wide k-steps of a product over d
  static constexpr int kRow = 2 * D;      // bytes per row (16-bit elements)
  static constexpr int kCR = kRow / 16;   // 16-byte chunks per row
  // Q, dO (dK/dV kernel) and K (dQ kernel) tiles are read by rows and
  // transposed.  At d = 128 they take the conflict-free RowsLayout (+2 %
  // without the causal mask, +6 % with it, B4 H32 N8192).  At d = 64 it
  // measured +3 % without the mask but -2 to -3 % with it (the
  // three-waves-per-SIMD causal dK/dV kernel then spills), so d = 64 keeps
  // the V layout.
  using VL = std::conditional_t<D == 128, RowsLayout<kRow>, VLayout<kRow, false>>;
  static constexpr int kGV = VL::kGroupBytes / 16;  // LDS granules per group of rows
  static constexpr int kRSK = kRow + 16;            // padded row of a tile read by rows only
};

// sum of the two 16-bit products of a packed pair, accumulated in float32
template <bool BF16>
__device__ __forceinline__ float dot_pair(u32 a, u32 b, float acc) {
  if (BF16) {
    const float a0 = __builtin_bit_cast(float, a << 16), a1 = __builtin_bit_cast(float, a & 0xFFFF0000u);
    const float b0 = __builtin_bit_cast(float, b << 16), b1 = __builtin_bit_cast(float, b & 0xFFFF0000u);
    return __builtin_fmaf(a1, b1, __builtin_fmaf(a0, b0, acc));
  }
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2, a), __builtin_bit_cast(fp16x2, b), acc, false);
}

// Direct HBM -> LDS load of `rows` rows (from row r0 of the slice) into the
// grouped, padded layout VL (see fa_device.h); NW waves share the work.
template <int D, int NW, int ROWS>
__device__ __forceinline__ void issue_rows_vl(__amdgpu_buffer_rsrc_t rs, char* dst, int r0, int wave, int lane) {
  using B = BwdShape<D>;
  constexpr int kGran = ROWS / B::VL::kGroupRows * B::kGV;
  constexpr int kBlk = (kGran + 63) / 64;
#pragma unroll
  for (int j = 0; j < (kBlk + NW - 1) / NW; ++j) {
    const int blk = wave + j * NW;
    const int g = blk * 64 + lane;
    const int grp = g / B::kGV;
    const int off = (g - grp * B::kGV) * 16;
    int r = -1, c = 0;
#pragma unroll
    for (int i = 0; i < B::VL::kGroupRows; ++i)
      if (off >= B::VL::row(i) && off < B::VL::row(i) + B::kRow) {
        r = grp * B::VL::kGroupRows + i;
        c = (off - B::VL::row(i)) / 16;
      }
    if (blk < kBlk && g < kGran && r >= 0) load_lds16(rs, dst + blk * 1024, (r0 + r) * B::kRow + c * 16);
  }
}

// The same for a tile read only by rows: one 16-byte pad granule per row.
template <int D, int NW, int ROWS>
__device__ __forceinline__ void issue_rows_k(__amdgpu_buffer_rsrc_t rs, char* dst, int r0, int wave, int lane) {
  using B = BwdShape<D>;
  constexpr int kG = B::kCR + 1;
  constexpr int kGran = ROWS * kG;
  constexpr int kBlk = (kGran + 63) / 64;
#pragma unroll
  for (int j = 0; j < (kBlk + NW - 1) / NW; ++j) {
    const int blk = wave + j * NW;
    const int g = blk * 64 + lane;
    const int r = g / kG, c = g - r * kG;
    if (blk < kBlk && g < kGran && c < B::kCR) load_lds16(rs, dst + blk * 1024, (r0 + r) * B::kRow + c * 16);
  }
}

// 128-bit operand of matrix instruction step s for row `row` of a slice,
// straight from HBM: lane (half, .) gets elements 16*s + 8*half .. +7.
template <int D>
__device__ __forceinline__ void load_row_operand(__amdgpu_buffer_rsrc_t rs, int row, int half, u32x4 (&dst)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    dst[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, row * (2 * D) + (16 * s + 8 * half) * 2, 0, 0);
}

// Transposing read of a 32-row block (rows 32*kb .. +31) of a VL tile: the A
// operand (column block db, k-step t) of a product that sums over those rows.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const char* tile, int base, int db, int kb, int t) {
  using B = BwdShape<D>;
  const int o = base + B::VL::row(32 * kb + 16 * t) + 64 * db;
  const u32x2 lo = lds_read_tr16(tile, o);
  const u32x2 hi = lds_read_tr16(tile, o + B::VL::row(8));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

template <int D>
__device__ __forceinline__ int tr_base(int lane) {
  using B = BwdShape<D>;
  const int g = lane >> 4, u = lane & 15, half = lane >> 5;
  return B::VL::row(4 * half + (u >> 2)) + 2 * (16 * (g & 1) + 4 * (u & 3));
}

// Store a d x 32 block set of transposed accumulators (lane owns one row of
// the output: a query for dQ, a key for dK/dV) as 16-bit values times `mul`.
template <bool BF16, int D>
__device__ __forceinline__ void store_rowT(char* row_ptr, const f32x16 (&acc)[D / 32], int half, float mul) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int col = 32 * db + 8 * a4 + 4 * half;
      u32x2 w;
      w[0] = pack_p<BF16>(acc[db][4 * a4 + 0] * mul, acc[db][4 * a4 + 1] * mul);
      w[1] = pack_p<BF16>(acc[db][4 * a4 + 2] * mul, acc[db][4 * a4 + 3] * mul);
      *reinterpret_cast<u32x2*>(row_ptr + col * 2) = w;
    }
}

}  // namespace

// ---------------------------------------------------------------- dQ kernel
// WPE: minimum waves per SIMD the registers are budgeted for; BC: keys per tile.
template <class Tr, int D, bool CAUSAL, int WPE, int BC>
__global__ __launch_bounds__(256, WPE) void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int NW = 4, kKB = BC / 32;
  constexpr bool kBf = Tr::kPvBf16;
  using B = BwdShape<D>;
  constexpr int kSK = BC / B::VL::kGroupRows * B::VL::kGroupBytes;  // K tile, grouped layout
  constexpr int kSV = BC * B::kRSK;                                  // V tile, padded rows
  __shared__ __attribute__((aligned(16))) char lds_k0[kSK];
  __shared__ __attribute__((aligned(16))) char lds_k1[kSK];
  __shared__ __attribute__((aligned(16))) char lds_v0[kSV];
  __shared__ __attribute__((aligned(16))) char lds_v1[kSV];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, l32 = lane & 31;
  // Causal grids at d = 64 pair query blocks n-1-i and i of a slice in one
  // workgroup, as the forward kernel does: the long block walks its keys up
  // from key 0, the short one down from its diagonal, so the workgroups of a
  // slice have equal work and read the same K/V tile at about the same time
  // (+1 to +14 %, most at small N).  At d = 128 it measured -1 to +2 %, so
  // query blocks run one per workgroup there, longest first.
  constexpr bool kPair = CAUSAL && D == 64;
  const int tile = xcd_remap(blockIdx.x, p.total_wg);
  const int per_slice = kPair ? (p.n_blocks + 1) / 2 : p.n_blocks;
  const int bh = tile / per_slice;
  const int pair = tile - bh * per_slice;
  const int n_jobs = kPair && 2 * pair + 1 < p.n_blocks ? 2 : 1;
  const int N = p.N;
  const u32 slice = (u32)N * B::kRow;
  const size_t base = (size_t)bh * N * B::kRow;
  const auto rq = make_rsrc((const char*)p.q + base, slice);
  const auto rk = make_rsrc((const char*)p.k + base, slice);
  const auto rv = make_rsrc((const char*)p.v + base, slice);
  const auto ro = make_rsrc((const char*)p.o + base, slice);
  const auto rdo = make_rsrc((const char*)p.dout + base, slice);
  const float c = p.c;

  for (int job = 0; job < n_jobs; ++job) {
    const int qt = !CAUSAL ? pair : job == 0 ? p.n_blocks - 1 - pair : pair;  // longest first
    const bool down = kPair && job == 1;  // keys from the diagonal down to key 0
    if (job > 0) __syncthreads();          // the first block's LDS stages are free again
    const int q0 = qt * kBwdRows, qw0 = q0 + wave * 32, qi = qw0 + l32;

    // this lane's query row: Q and dO as matrix operands, D = dO . O, lse
    u32x4 q16[B::kSteps], do16[B::kSteps], o16[B::kSteps];
    load_row_operand<D>(rq, qi, half, q16);
    load_row_operand<D>(rdo, qi, half, do16);
    load_row_operand<D>(ro, qi, half, o16);
    float dpart = 0.f;
#pragma unroll
    for (int s = 0; s < B::kSteps; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) dpart = dot_pair<kBf>(do16[s][e], o16[s][e], dpart);
    const float Dq = halves_sum(dpart);
    const float Lq = qi < N ? p.lse[(size_t)bh * N + qi] * kLog2e : 0.f;
    if (half == 0 && qi < N) p.delta[(size_t)bh * N + qi] = Dq;

    const int n_all = (N + BC - 1) / BC;
    const int n_kv = CAUSAL ? min(n_all, (q0 + kBwdRows - 1) / BC + 1) : n_all;
    // key tile of step i (steps are counted in the order the tiles are visited)
    auto ktile = [&](int i) __attribute__((always_inline)) { return down ? n_kv - 1 - i : i; };
    const bool has_rows = qw0 < N;

    f32x16 dqacc[B::kDB];
#pragma unroll
    for (int db = 0; db < B::kDB; ++db) dqacc[db] = f32x16{};
    const int kbase = B::VL::row(l32) + 16 * half;  // row operand of the K tile (grouped layout)
    const int vbase = l32 * B::kRSK + 16 * half;    // row operand of the V tile (padded rows)
    const int tbase = tr_base<D>(lane);

    auto step = [&](int kt, const char* lk, const char* lv) __attribute__((always_inline)) {
      if (!has_rows || (CAUSAL && ktile(kt) * BC > qw0 + 31)) return;
      f32x16 st[kKB], dpt[kKB];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        st[kb] = f32x16{};
        dpt[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < B::kSteps; ++s) {
          const u32x4 ka = lds_read_b128(lk, kbase + B::VL::row(32 * kb) + 32 * s);
          st[kb] = mfma16(ka, q16[s], st[kb], kBf);
          const u32x4 va = lds_read_b128(lv, vbase + 32 * kb * B::kRSK + 32 * s);
          dpt[kb] = mfma16(va, do16[s], dpt[kb], kBf);
        }
      }
      const int k0 = ktile(kt) * BC;
      const int lim = CAUSAL ? min(qi, N - 1) : N - 1;  // last key this query sees
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw0);
      u32x4 pb[kKB][2];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float ds[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int r = 8 * t + 2 * e + j;
              float x = __builtin_fmaf(st[kb][r], c, -Lq);
              if (need_mask) {
                const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (key > lim) x = -INFINITY;
              }
              const float pr = __builtin_amdgcn_exp2f(x);
              ds[j] = pr * (dpt[kb][r] - Dq);
            }
            pb[kb][t][e] = pack_p<kBf>(ds[0], ds[1]);
          }
#pragma unroll
      for (int db = 0; db < B::kDB; ++db)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) dqacc[db] = mfma16(tr_operand<D>(lk, tbase, db, kb, t), pb[kb][t], dqacc[db], kBf);
    };

    issue_rows_vl<D, NW, BC>(rk, lds_k0, ktile(0) * BC, wave, lane);
    issue_rows_k<D, NW, BC>(rv, lds_v0, ktile(0) * BC, wave, lane);
    for (int kt = 0; kt < n_kv; kt += 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 1 < n_kv) {
        issue_rows_vl<D, NW, BC>(rk, lds_k1, ktile(kt + 1) * BC, wave, lane);
        issue_rows_k<D, NW, BC>(rv, lds_v1, ktile(kt + 1) * BC, wave, lane);
      }
      FA_SYNC_POINT();
      step(kt, lds_k0, lds_v0);
      FA_SYNC_POINT();
      if (kt + 1 < n_kv) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 2 < n_kv) {
          issue_rows_vl<D, NW, BC>(rk, lds_k0, ktile(kt + 2) * BC, wave, lane);
          issue_rows_k<D, NW, BC>(rv, lds_v0, ktile(kt + 2) * BC, wave, lane);
        }
        FA_SYNC_POINT();
        step(kt + 1, lds_k1, lds_v1);
        FA_SYNC_POINT();
      }
    }

    if (qi < N) store_rowT<kBf, D>((char*)p.dq + base + (size_t)qi * B::kRow, dqacc, half, p.scale);
  }
}

// ------------------------------------------------------------ dK/dV kernel
// WPE: minimum waves per SIMD the registers are budgeted for (at d = 64, 3;
// at d = 128, 2 fits the kernel into 256 registers and 1 leaves it more, for
// grids too small to put two workgroups on a CU).
template <class Tr, int D, bool CAUSAL, int WPE>
__global__ __launch_bounds__(256, WPE) void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = 4, BQ = 32;
  constexpr bool kBf = Tr::kPvBf16;
  using B = BwdShape<D>;
  constexpr int kST = BQ / B::VL::kGroupRows * B::VL::kGroupBytes;  // a Q or dO tile, grouped layout
  __shared__ __attribute__((aligned(16))) char lds_q0[kST];
  __shared__ __attribute__((aligned(16))) char lds_q1[kST];
  __shared__ __attribute__((aligned(16))) char lds_d0[kST];
  __shared__ __attribute__((aligned(16))) char lds_d1[kST];
  __shared__ __attribute__((aligned(16))) float lds_ld0[2 * BQ];  // lse (natural log) then D of the tile's rows
  __shared__ __attribute__((aligned(16))) float lds_ld1[2 * BQ];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, l32 = lane & 31;
  // Causal grids at d = 64 pair key blocks i (its queries run to the end:
  // the longest) and n-1-i of a slice in one workgroup.  The long block
  // walks its query tiles down from the last one and the short block up
  // from its diagonal, so the workgroups of a slice have equal work and read
  // the same query tile at about the same time.  At d = 128 the kernel has
  // no register to spare for the second block's state (its query-tile loop
  // reloads spilled offsets), so key blocks run one per workgroup, longest
  // first, as the dQ kernel's query blocks do there.
  constexpr bool kPair = CAUSAL && D == 64;
  const int tile = xcd_remap(blockIdx.x, p.total_wg);
  const int per_slice = kPair ? (p.n_blocks + 1) / 2 : p.n_blocks;
  const int bh = tile / per_slice;
  const int pair = tile - bh * per_slice;
  const int n_jobs = kPair && 2 * pair + 1 < p.n_blocks ? 2 : 1;
  const int N = p.N;
  const u32 slice = (u32)N * B::kRow;
  const size_t base = (size_t)bh * N * B::kRow;
  const auto rq = make_rsrc((const char*)p.q + base, slice);
  const auto rk = make_rsrc((const char*)p.k + base, slice);
  const auto rv = make_rsrc((const char*)p.v + base, slice);
  const auto rdo = make_rsrc((const char*)p.dout + base, slice);
  const auto rl = make_rsrc(p.lse + (size_t)bh * N, (u32)N * 4);
  const auto rd = make_rsrc(p.delta + (size_t)bh * N, (u32)N * 4);
  const float c = p.c;
  const int n_qt = (N + BQ - 1) / BQ;

  for (int job = 0; job < n_jobs; ++job) {
    const int kblk = job == 0 ? pair : p.n_blocks - 1 - pair;
    const bool down = kPair && job == 0;  // query tiles from the last one down to the diagonal
    if (job > 0) __syncthreads();          // the first block's LDS stages are free again
    const int k0 = kblk * kBwdRows, kw0 = k0 + wave * 32, key = kw0 + l32;

    // this lane's key row of K and V as matrix operands
    u32x4 k16[B::kSteps], v16[B::kSteps];
    load_row_operand<D>(rk, key, half, k16);
    load_row_operand<D>(rv, key, half, v16);

    f32x16 dkacc[B::kDB], dvacc[B::kDB];
#pragma unroll
    for (int db = 0; db < B::kDB; ++db) {
      dkacc[db] = f32x16{};
      dvacc[db] = f32x16{};
    }
    const int rbase = B::VL::row(l32) + 16 * half;  // row operand of a Q or dO tile
    const int tbase = tr_base<D>(lane);
    const int qt0 = CAUSAL ? k0 / BQ : 0;  // earlier queries see none of this block's keys
    const int n_steps = max(n_qt - qt0, 0);
    // query tile of step i (steps are counted in the order the tiles are visited)
    auto qtile = [&](int i) __attribute__((always_inline)) { return down ? n_qt - 1 - i : qt0 + i; };
    const bool has_keys = kw0 < N;

    // wave 0 fetches the tile's 32 lse values (lanes 0..7, into dst[0..31]) and
    // its 32 D values (lanes 8..15, into dst[32..63]): a direct load writes
    // lane L's 16 bytes at dst + 16*L
    auto issue_ld = [&](int qt, float* dst) __attribute__((always_inline)) {
      if (wave == 0) {
        const int r = qt * BQ + 4 * (lane & 7);
        if (lane < 8) load_lds16(rl, (char*)dst, r * 4);
        if (lane >= 8 && lane < 16) load_lds16(rd, (char*)dst, r * 4);
      }
    };
    auto issue = [&](int qt, char* dq_tile, char* ddo_tile, float* dld) __attribute__((always_inline)) {
      issue_rows_vl<D, NW, BQ>(rq, dq_tile, qt * BQ, wave, lane);
      issue_rows_vl<D, NW, BQ>(rdo, ddo_tile, qt * BQ, wave, lane);
      issue_ld(qt, dld);
    };

    auto step = [&](int i, const char* tq, const char* tdo, const float* tld) __attribute__((always_inline)) {
      const int qb0 = qtile(i) * BQ;
      if (!has_keys || (CAUSAL && qb0 + BQ - 1 < kw0)) return;  // no query of the tile sees these keys
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < B::kSteps; ++st) {
        const u32x4 qa = lds_read_b128(tq, rbase + 32 * st);
        s = mfma16(qa, k16[st], s, kBf);
        const u32x4 da = lds_read_b128(tdo, rbase + 32 * st);
        dp = mfma16(da, v16[st], dp, kBf);
      }
      // Element r of the accumulators belongs to query row 8*(r/4) + 4*half +
      // r%4 of the tile; the four rows of group r/4 take their lse and D from
      // one 128-bit LDS read each, right where they are used.  (Whole-vector
      // casts: a bit cast of a vector element subscript reads element 0
      // whatever the index.)
      const bool need_mask = (qb0 + BQ > N) || (CAUSAL && qb0 < kw0 + 31);
      // Element r holds query qb0 + 4*half + o(r), o(r) = 8*(r/4) + r%4: it is
      // masked when o(r) >= q_end (past N) or, causal, when o(r) < k_rel (the
      // query precedes this lane's key).  Two per-lane bounds against
      // compile-time offsets, instead of each element's query index.
      const int q_end = N - qb0 - 4 * half;
      const int k_rel = key - qb0 - 4 * half;
      u32x4 pp[2], pds[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int eh = 0; eh < 2; ++eh) {
          const int g = 2 * t + eh;
          const f32x4 l4 = __builtin_bit_cast(f32x4, lds_read_b128((const char*)tld, (8 * g + 4 * half) * 4));
          const f32x4 d4 = __builtin_bit_cast(f32x4, lds_read_b128((const char*)tld, (BQ + 8 * g + 4 * half) * 4));
#pragma unroll
          for (int el = 0; el < 2; ++el) {
            const int e = 2 * eh + el;
            float pr[2], ds[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int r = 8 * t + 2 * e + j;  // = 4 * g + 2 * el + j
              float x = __builtin_fmaf(s[r], c, -l4[2 * el + j] * kLog2e);
              if (need_mask) {
                const int o = 8 * (r >> 2) + (r & 3);
                if (o >= q_end || (CAUSAL && o < k_rel)) x = -INFINITY;
              }
              pr[j] = __builtin_amdgcn_exp2f(x);
              ds[j] = pr[j] * (dp[r] - d4[2 * el + j]);
            }
            pp[t][e] = pack_p<kBf>(pr[0], pr[1]);
            pds[t][e] = pack_p<kBf>(ds[0], ds[1]);
          }
        }
#pragma unroll
      for (int db = 0; db < B::kDB; ++db)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          dvacc[db] = mfma16(tr_operand<D>(tdo, tbase, db, 0, t), pp[t], dvacc[db], kBf);
          dkacc[db] = mfma16(tr_operand<D>(tq, tbase, db, 0, t), pds[t], dkacc[db], kBf);
        }
    };

    if (n_steps > 0) issue(qtile(0), lds_q0, lds_d0, lds_ld0);
    for (int i = 0; i < n_steps; i += 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (i + 1 < n_steps) issue(qtile(i + 1), lds_q1, lds_d1, lds_ld1);
      FA_SYNC_POINT();
      step(i, lds_q0, lds_d0, lds_ld0);
      FA_SYNC_POINT();
      if (i + 1 < n_steps) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (i + 2 < n_steps) issue(qtile(i + 2), lds_q0, lds_d0, lds_ld0);
        FA_SYNC_POINT();
        step(i + 1, lds_q1, lds_d1, lds_ld1);
        FA_SYNC_POINT();
      }
    }

    // the lane's key and half-wave are recomputed here rather than kept in
    // registers through the loop (which made the causal build spill)
    const int e_lane = lane_id(), e_key = kw0 + (e_lane & 31), e_half = e_lane >> 5;
    if (e_key < N) {
      store_rowT<kBf, D>((char*)p.dk + base + (size_t)e_key * B::kRow, dkacc, e_half, p.scale);
      store_rowT<kBf, D>((char*)p.dv + base + (size_t)e_key * B::kRow, dvacc, e_half, 1.f);
    }
  }
}

namespace {

template <class Tr, int D, bool CAUSAL>
hipError_t launch_bwd_typed(const BwdParams& bp, hipStream_t stream) {
  // causal grids at d = 64: one workgroup per pair of 128-row blocks
  BwdParams p = bp;
  if (CAUSAL && D == 64) p.total_wg = (bp.n_blocks + 1) / 2 * bp.B * bp.H;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<Tr, D, CAUSAL, D == 64 ? 4 : 2, D == 64 ? 32 : 64>), dim3(p.total_wg), dim3(256), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // (dQ at d = 64: 32-key tiles fit four waves per SIMD in 128 registers,
  // bit-identical and 0-2 % faster than 64-key tiles at three waves.)
  // (256 CUs: at d = 128 two waves per SIMD pay off once there are two
  // workgroups per CU; at d = 64 the kernel fits three per SIMD, which is
  // 9 % faster than two on causal B8 H32 N4096 and the same without mask)
  if constexpr (D == 64) {
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<Tr, D, CAUSAL, 3>), dim3(p.total_wg), dim3(256), 0, stream, p);
  } else {
    if (bp.total_wg >= 512)
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<Tr, D, CAUSAL, 2>), dim3(bp.total_wg), dim3(256), 0, stream, bp);
    else
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<Tr, D, CAUSAL, 1>), dim3(bp.total_wg), dim3(256), 0, stream, bp);
  }
  return hipGetLastError();
}

template <class Tr>
hipError_t launch_bwd_dtype(int d, bool causal, const BwdParams& p, hipStream_t stream) {
  if (d == 64) return causal ? launch_bwd_typed<Tr, 64, true>(p, stream) : launch_bwd_typed<Tr, 64, false>(p, stream);
  return causal ? launch_bwd_typed<Tr, 128, true>(p, stream) : launch_bwd_typed<Tr, 128, false>(p, stream);
}

}  // namespace

// D = rowsum(dO * O) of the allocation-free entry point (fa_bwd_noalloc):
// kBwdScratchRows float32 rows (16 MiB), one copy per GPU, held until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol): the device address of each GPU's copy
// comes from hipGetSymbolAddress, once per device, below.
static __device__ __align__(256) float scratch[kBwdScratchRows];

hipError_t bwd_scratch(hipStream_t stream, float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);  // the copy on the GPU the work is enqueued on
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // the symbol's address is per device: look it up with that device current
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(ptr);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_bwd(Dtype dt, int d, bool causal, const BwdParams& p, hipStream_t stream) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  if (dt == Dtype::F16) return launch_bwd_dtype<TrF16>(d, causal, p, stream);
  if (dt == Dtype::BF16) return launch_bwd_dtype<TrBF16>(d, causal, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
