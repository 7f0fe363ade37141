// The shared output projection W_O over the heads' outputs
// (MLA tutorial page, "Move the Value Expansion After the Weighted Sum": the
// value up-projection combines with each head's contribution to the final
// output projection; RedKnot-MLA abstract: the merged state goes through one
// shared output projection).
//
//   out[t][n] = sum_k x[t][k] * w_o[n][k]
//
// x is the heads' outputs back to back (k = h * d_v + i), or the weighted
// latents when w_o holds the per-head fold W_O[:, head h] U_V[h].  For few
// tokens the cost is reading W_O once (d_model x k_in bf16): the MFMA kernel
// streams each weight row exactly once per 64-token block, straight from HBM
// into registers, while the tokens' inputs are staged through LDS and shared
// by the four waves of a workgroup.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kOpRows = 64;    // output features per workgroup (16 per wave)
constexpr int kOpTok = 64;     // tokens per workgroup (four 16-token MFMA blocks)
constexpr int kOpSlab = 256;   // contraction entries per LDS slab (8 MFMA k-steps)
constexpr int kOpChunks = kOpSlab / 8;             // 16-byte chunks per token row of a slab
constexpr int kOpSlabBytes = kOpTok * kOpSlab * 2;  // 32 KiB
constexpr int kOpLoads = kOpTok * kOpChunks / 256;  // chunks each thread moves per slab

// Workgroup (features n0 .. n0 + 63, tokens t0 .. t0 + 63).  Wave w owns
// features n0 + 16 w + (0..15).  Within a slab starting at k0, lane (l16, lg)
// takes entries k0 + 64 lg + 8 j .. + 7 as the MFMA k-indices 8 lg .. 8 lg + 7
// of k-step j, for both operands (the contraction is over all k either way),
// so each lane reads 128 contiguous bytes of its weight row per slab.
//
// LDS slab: token row r (512 B) holds chunk c (entries 8 c .. 8 c + 7) at
// position c ^ (r & 15): the 16 lanes of a 16-lane group read 16 different
// rows at one chunk index, i.e. 16 distinct 16-byte bank groups.
template <typename TO>
__global__ __launch_bounds__(256) void out_proj_mfma_kernel(const bf16* __restrict__ x, const bf16* __restrict__ w,
                                                            TO* __restrict__ out, int n_tok, int k_in,
                                                            int d_model) {
  __shared__ __attribute__((aligned(16))) char xs[2][kOpSlabBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kOpRows, t0 = blockIdx.y * kOpTok;
  const int nb = min(kOpTok, n_tok - t0 + 15) / 16;  // 16-token blocks with tokens (1..4)
  const int n_slab = k_in / kOpSlab;

  // this lane's weight row (a row past d_model reads the last row; never stored)
  const int n = min(n0 + 16 * wave + l16, d_model - 1);
  const bf16* wrow = w + (int64_t)n * k_in + 64 * lg;

  // cooperative slab loads: chunk e = tid + 256 i is token e / 32, chunk e % 32
  auto load_x = [&](int s, bf16x8 (&v)[kOpLoads]) {
#pragma unroll
    for (int i = 0; i < kOpLoads; ++i) {
      const int e = tid + 256 * i, r = e / kOpChunks, c = e % kOpChunks;
      const int t = min(t0 + r, n_tok - 1);  // rows past n_tok read the last token, zeroed below
      v[i] = *(const bf16x8*)(x + (int64_t)t * k_in + (int64_t)s * kOpSlab + 8 * c);
      if (t0 + r >= n_tok) v[i] = bf16x8{};
    }
  };
  auto store_x = [&](int buf, const bf16x8 (&v)[kOpLoads]) {
#pragma unroll
    for (int i = 0; i < kOpLoads; ++i) {
      const int e = tid + 256 * i, r = e / kOpChunks, c = e % kOpChunks;
      *(bf16x8*)(xs[buf] + r * (kOpSlab * 2) + ((c ^ (r & 15)) << 4)) = v[i];
    }
  };
  auto load_w = [&](int s, bf16x8 (&a)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = *(const bf16x8*)(wrow + (int64_t)s * kOpSlab + 8 * j);
  };

  f32x4 acc[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 a_cur[8], a_nxt[8], xv[kOpLoads];
  load_x(0, xv);
  load_w(0, a_cur);
  store_x(0, xv);
  __syncthreads();
  for (int s = 0; s < n_slab; ++s) {
    const bool more = s + 1 < n_slab;
    if (more) {
      load_x(s + 1, xv);
      load_w(s + 1, a_nxt);
    }
    const char* xb = xs[s & 1];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if (tb < nb) {
        const char* xr = xb + (16 * tb + l16) * (kOpSlab * 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bf16x8 b = *(const bf16x8*)(xr + (((8 * lg + j) ^ l16) << 4));
          acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_cur[j], b, acc[tb], 0, 0, 0);
        }
      }
    }
    if (more) {
      store_x((s + 1) & 1, xv);
#pragma unroll
      for (int j = 0; j < 8; ++j) a_cur[j] = a_nxt[j];
    }
    // the next slab is in LDS, and every wave is past its reads of this one
    // (whose buffer the slab after next overwrites)
    __syncthreads();
  }

  // lane (l16, lg) holds out[t0 + 16 tb + l16][n0 + 16 wave + 4 lg + e]
  const int nf = n0 + 16 * wave + 4 * lg;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + 16 * tb + l16;
    if (tb < nb && t < n_tok) {
      TO* o = out + (int64_t)t * d_model + nf;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nf + e < d_model) store_f(o + e, acc[tb][e]);
    }
  }
}

// Any dtypes and sizes: one wave per output feature, lanes over k, fp32
// accumulation, a wave sum per token.
template <typename TX, typename TW, typename TO>
__global__ __launch_bounds__(256) void out_proj_plain_kernel(const TX* __restrict__ x, const TW* __restrict__ w,
                                                             TO* __restrict__ out, int n_tok, int k_in,
                                                             int d_model) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= d_model) return;
  const TW* wr = w + (int64_t)n * k_in;
  for (int t = blockIdx.y; t < n_tok; t += gridDim.y) {
    const TX* xr = x + (int64_t)t * k_in;
    float s = 0.f;
    for (int k = lane; k < k_in; k += 64) s += load_f(xr + k) * load_f(wr + k);
    s = wave_sum(s);
    if (lane == 0) store_f(out + (int64_t)t * d_model + n, s);
  }
}

template <typename TX, typename TW>
hipError_t plain_launch(const void* x, const void* w, void* out, bool out_bf, int n_tok, int k_in, int d_model,
                        hipStream_t stream) {
  const dim3 grid((d_model + 3) / 4, std::min(n_tok, 4096));
  if (out_bf)
    return launch(out_proj_plain_kernel<TX, TW, bf16>, grid, dim3(256), stream, (const TX*)x, (const TW*)w,
                  (bf16*)out, n_tok, k_in, d_model);
  return launch(out_proj_plain_kernel<TX, TW, float>, grid, dim3(256), stream, (const TX*)x, (const TW*)w,
                (float*)out, n_tok, k_in, d_model);
}

}  // namespace

bool out_proj_mfma_ok(const void* x, bool x_bf16, const void* w, bool w_bf16, int k_in) {
  return x_bf16 && w_bf16 && k_in % kOpSlab == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) & 15u) == 0;
}

hipError_t launch_out_proj(const void* x, bool x_bf16, const void* w, bool w_bf16, void* out, bool out_bf16,
                           int n_tok, int k_in, int d_model, hipStream_t stream) {
  if (out_proj_mfma_ok(x, x_bf16, w, w_bf16, k_in)) {
    const dim3 grid((d_model + kOpRows - 1) / kOpRows, (n_tok + kOpTok - 1) / kOpTok);
    if (out_bf16)
      return launch(out_proj_mfma_kernel<bf16>, grid, dim3(256), stream, (const bf16*)x, (const bf16*)w,
                    (bf16*)out, n_tok, k_in, d_model);
    return launch(out_proj_mfma_kernel<float>, grid, dim3(256), stream, (const bf16*)x, (const bf16*)w,
                  (float*)out, n_tok, k_in, d_model);
  }
  if (x_bf16 && w_bf16) return plain_launch<bf16, bf16>(x, w, out, out_bf16, n_tok, k_in, d_model, stream);
  if (x_bf16) return plain_launch<bf16, float>(x, w, out, out_bf16, n_tok, k_in, d_model, stream);
  if (w_bf16) return plain_launch<float, bf16>(x, w, out, out_bf16, n_tok, k_in, d_model, stream);
  return plain_launch<float, float>(x, w, out, out_bf16, n_tok, k_in, d_model, stream);
}

}  // namespace mla
