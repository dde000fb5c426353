// Tile shapes of the forward kernel and the choice among them: host logic
// shared by the C-ABI layer (which sizes the grid and reports the shape a call
// runs) and the kernel file (which holds one instance per shape).
#pragma once

#include <stdio.h>
#include <stdlib.h>

#include "fa_launch.h"

namespace fa {

struct Variant {
  int qw, nw, bc, sched, wpe;  // rows per wave, waves, keys per tile, schedule, min waves per SIMD
};
// Tile shapes compiled for every (dtype, causal); the first five for both
// head dimensions, the others for the one d64_only / d128_only name.
// FA_TILE=<qw>x<nw>x<bc>x<sched>x<wpe> selects one of them instead of the
// default (tile sweeps only; an unknown value, or a shape not compiled for
// the call's head dimension, falls back to the default).  Dropout kernels
// exist for the default shapes only, so FA_TILE is ignored with dropout.
inline constexpr Variant kVariants[] = {{32, 8, 64, 1, 2}, {32, 4, 64, 0, 4}, {32, 4, 64, 0, 3},
                                        {32, 4, 64, 0, 2}, {64, 4, 64, 0, 2}, {64, 8, 64, 1, 2},
                                        {32, 16, 64, 1, 4}, {32, 8, 64, 0, 4}, {64, 8, 32, 1, 2}};
// Shapes compiled for d = 64 only (at d = 128 they would spill).
inline constexpr bool d64_only(int v) { return v == 5 || v == 6 || v == 7; }
// Shapes compiled for d = 128 only.
inline constexpr bool d128_only(int v) { return v == 8; }
inline constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// Measured on MI355X (tile sweep under rocprofv3, interleaved A/B runs in one
// process): at d = 128 the ping-pong schedule wins for 16-bit types.  Its
// matrix phase is bound by the LDS operand reads (1 KB per instruction of a
// 32-row wave).  64-row waves with 32-key tiles cut them (to half for fp8,
// whose Q operands fit in registers, and to three quarters at 16 bits, whose
// second query block's Q operands are read from LDS): without the causal mask
// +11 % for fp8 and +6 to +8 % for the 16-bit types (B8 H32 N4096 / N8192, B4
// H32 N8192).  With the causal mask (each workgroup runs a long and a short
// query tile) the same shape wins from 4096 rows on for the 16-bit types (+1 %
// at 4096, +2 to +3 % at 8192 and 16384) and from 8192 for fp8 (+4 %); below
// that 256-row ping-pong workgroups win at 2048 rows, and the 128-row plain
// shape at two waves per SIMD at 1024 rows and fewer (+8 to +16 %) and for fp8
// below 8192.  At d = 64 the softmax's vector work per tile is as long as the
// tile's matrix work, and a single wave issues vector instructions at well
// under the SIMD's rate, so the shapes that keep more waves in their softmax
// at once win: 32 rows per wave at four waves per SIMD.  Without a causal
// mask, 8 such waves per workgroup (each K/V tile in LDS then serves 256 query
// rows, half the tile loads per row of 4 waves) below 4096 rows, and for
// binary16 below 8192; from there on 64-row ping-pong waves (twice the matrix
// work per LDS operand) win for the 16-bit types (bfloat16, whose row sums
// take twice the vector work, from 4096 rows; binary16, with Q pre-scaled,
// +2 % at 8192) and the plain 64-row shape for fp8, each by a few percent.
// With the causal mask 4-wave workgroups at four waves per SIMD win for
// bfloat16 and fp8 (for fp8 by 1 to 5 % over three waves per SIMD, 512 to
// 16384 rows; 8 waves tie for bfloat16), and for binary16 below 4096 rows;
// from 4096 rows binary16 (Q pre-scaled) gains 3 to 4 % with 8 waves (4096 to
// 16384 rows).  Packed batches of mixed lengths (N = the longest) keep
// 128-row workgroups: larger ones idle most of their waves on the short
// sequences (lengths 256..4096: 660 against 596 TFLOP/s at d = 64, 726 against
// 699 at d = 128).  Dropout kernels exist for the shapes listed in
// dispatch_dropout.
inline int default_variant(Dtype dt, int d, bool causal, int N, bool dropout, bool packed) {
  if (packed && !dropout) return d == 128 ? 3 : dt == Dtype::FP8 ? 2 : 1;
  if (d == 128) {
    if (dropout) return 0;  // the one d = 128 shape compiled with dropout
    if (!causal) return 8;
    if (dt == Dtype::FP8) return N >= 8192 ? 8 : 3;
    return N >= 4096 ? 8 : N >= 2048 ? 0 : 3;
  }
  if (dropout) return !causal && N >= 1024 ? 4 : 2;
  if (causal) return dt == Dtype::F16 && N >= 4096 ? 7 : 1;
  if (dt == Dtype::FP8) return N >= 4096 ? 4 : 7;
  return N >= (dt == Dtype::BF16 ? 4096 : 8192) ? 5 : 7;
}

inline int selected_variant(Dtype dt, int d, bool causal, int N, bool dropout, bool packed) {
  const char* env = dropout ? nullptr : getenv("FA_TILE");
  if (env) {
    Variant v{};
    if (sscanf(env, "%dx%dx%dx%dx%d", &v.qw, &v.nw, &v.bc, &v.sched, &v.wpe) == 5)
      for (int i = 0; i < kNumVariants; ++i)
        if (kVariants[i].qw == v.qw && kVariants[i].nw == v.nw && kVariants[i].bc == v.bc &&
            kVariants[i].sched == v.sched && kVariants[i].wpe == v.wpe && (!d64_only(i) || d == 64) &&
            (!d128_only(i) || d == 128))
          return i;
  }
  return default_variant(dt, d, causal, N, dropout, packed);
}

}  // namespace fa
