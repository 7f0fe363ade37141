// Device-side helpers shared by the HIP kernels of the MLA decode library.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA bf16, LDS direct loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

template <typename T> __device__ __forceinline__ float load_f(const T* p);
template <> __device__ __forceinline__ float load_f<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f<bf16>(const bf16* p) { return (float)*p; }
// Four consecutive partial-output entries, fp32 or bf16 storage.
__device__ __forceinline__ void store_part4(void* base, int64_t idx, f32x4 v, bool bf) {
  if (bf)
    *(bf16x4*)((bf16*)base + idx) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  else
    *(f32x4*)((float*)base + idx) = v;
}
template <typename T> __device__ __forceinline__ f32x4 load_part4(const T* p);
template <> __device__ __forceinline__ f32x4 load_part4<float>(const float* p) { return *(const f32x4*)p; }
template <> __device__ __forceinline__ f32x4 load_part4<bf16>(const bf16* p) {
  const bf16x4 h = *(const bf16x4*)p;
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

// Tag type of a query written as bf16 hi and lo planes ([..][2][d]: hi =
// bf16(x), lo = bf16(x - hi)); pointers of this type are cast before use.
struct SplitBf16 {};
template <typename T> __device__ __forceinline__ void store_f(T* p, float v);
template <> __device__ __forceinline__ void store_f<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f<bf16>(bf16* p, float v) { *p = (bf16)v; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// Runtime-valued vmcnt wait (the immediate must be a constant: dispatch).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;   case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;   case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;   case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;   case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;   case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break; case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break; case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break; case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break; case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break; case 19: wait_vmcnt<19>(); break;
    case 20: wait_vmcnt<20>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// Workgroup barrier without the memory fence __syncthreads() adds: the fence
// would wait for every outstanding LDS-direct load and defeat prefetching.
// Callers order their own LDS traffic with wait_lgkm0()/wait_vmcnt<>().
__device__ __forceinline__ void barrier_raw() { __builtin_amdgcn_s_barrier(); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Rotation of one adjacent feature pair (2i, 2i+1) of a rotary query by
// rel * base^(-2i/d_rope), counter-clockwise (MLA tutorial page, "Position
// Rotations Complicate the Absorption").  rel is an int64 position
// difference and the angle is formed in fp64 (positions reach 2^18, where an
// fp32 angle is off by ~0.02 rad); the rotation itself is fp32.
__device__ __forceinline__ void rope_pair(float x0, float x1, int64_t rel, int i, int d_rope, double base,
                                          float* y0, float* y1) {
  const double theta = pow(base, -2.0 * (double)i / (double)d_rope);
  double sn, cs;
  sincos((double)rel * theta, &sn, &cs);
  const float cf = (float)cs, sf = (float)sn;
  *y0 = x0 * cf - x1 * sf;
  *y1 = x0 * sf + x1 * cf;
}

// Launch a kernel and return the status of this launch itself
// (hipLaunchKernel), never an error left behind by an unrelated earlier call.
template <typename... KArgs, typename Tuple, size_t... I>
inline hipError_t launch_tuple(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Tuple& t,
                               std::index_sequence<I...>) {
  void* argv[] = {(void*)&std::get<I>(t)..., nullptr};
  return hipLaunchKernel((const void*)k, grid, block, argv, 0, stream);
}
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> t(std::forward<Args>(args)...);
  return launch_tuple(k, grid, block, stream, t, std::index_sequence_for<KArgs...>{});
}

}  // namespace mla
