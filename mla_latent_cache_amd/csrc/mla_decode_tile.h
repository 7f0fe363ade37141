// Tile geometry and device helpers shared by the bf16 decode kernels
// (gfx950): the cache-row layout, the swizzled LDS placement of a 32-row
// tile, the split pieces and the 16-lane-row reductions.
#pragma once

#include "mla_common.h"

namespace mla {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kRowBytes = (kDc + kDr) * 2;  // 1152
constexpr int kTile = 32;                   // cache rows per tile
constexpr int kCBytes = kDc * 2;            // 1024: latent part c_t of a row
constexpr int kRBytes = kDr * 2;            // 128: rotary part kr_t of a row
constexpr int kCStage = kTile * kCBytes;    // latent ring stage (32 KiB)
constexpr int kRStage = kTile * kRBytes;    // rotary ring stage (4 KiB)
constexpr float kTau = 8.f;                 // lazy softmax rescale threshold (log2 units)
constexpr int kPageSize = 64;
constexpr int kKSteps = (kDc + kDr) / 32;   // 18 MFMA k-steps over [c | kr]

// One piece of a workgroup's share: rows [r0, r1) of request b (T rows in
// all) into partial slot `slot`; b (< 2^16) and slot (< 2^15) are packed
// into one non-negative int.
struct Piece {
  int b_slot, r0, r1, T;
};

__device__ __forceinline__ int sload_i32(const int32_t* p) {
  // Scalar (SMEM) load: counted by lgkmcnt, so it never forces the in-flight
  // LDS-direct loads (vmcnt, in order) to drain.
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap instructions: VALU only, no LDS round trip.
// permlane16_swap(x, x) leaves rows (0,0,2,2) / (1,1,3,3) in its two results,
// permlane32_swap(x, x) rows (0,1,0,1) / (2,3,2,3).
__device__ __forceinline__ float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS layout of a tile (no padding, 16-byte chunks XOR-swizzled per row):
// latent row r holds chunk c (0..63) at position c ^ (r & 15), rotary row r
// chunk j (0..7) at position j ^ ((r >> 1) & 7), and the tile fits in 36 KiB.
// A score-operand read (16 consecutive rows, one chunk) then reaches 64
// distinct banks per cycle; in a transposed read (ds_read_b64_tr_b16, 32
// lanes per cycle) rows r and r ^ 1 share their banks, a two-way conflict
// (the bank-conflict counter gives 0.24 on the kernel for up to 32 rows,
// which keeps this layout).  The row-owning kernel (mla_decode_rows.hip)
// keys its latent rows by 2 (r & 7) instead, which serves both reads
// without conflicts (its time did not change).
__device__ __forceinline__ int cpos(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int rpos(int r, int j) { return j ^ ((r >> 1) & 7); }

}  // namespace mla
