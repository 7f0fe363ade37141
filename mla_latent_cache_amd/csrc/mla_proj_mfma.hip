// Per-query projections on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16).
//
// absorb:  q_lat[t][h][j] = sum_i q_nope[t][h][i] * w_uk[h][i][j]
//          (MLA tutorial page, "Move the Key Projection Into the Query")
// out_uv:  out[t][h][v]   = sum_c o_lat[t][h][c] * w_uv[h][v][c]
//          (MLA tutorial page, "Move the Value Expansion After the Weighted Sum")
//
// Both are per head a small GEMM [n_tok x K] . [K x N] whose cost is reading
// the head's weights once (128 x 512 bf16 = 128 KiB); tokens are padded to
// 16-row MFMA blocks.  For absorb the contraction index i is the row index of
// w_uk, so the B operand (8 consecutive i per lane) is taken from an LDS copy
// of the weight slice with ds_read_b64_tr_b16; for out_uv the contraction
// index c is contiguous in both operands: the weights are loaded straight
// from HBM, the o_lat rows staged once in LDS for all the workgroup's waves.
#include "mla_common.h"
#include "mla_kernels.h"

#include <algorithm>
#include <type_traits>

namespace mla {
namespace {

constexpr int kNope = 128;        // d_nope of the bf16 fast path
constexpr int kLat = 512;         // d_c
constexpr int kAbsCols = 128;     // output columns per absorb workgroup
constexpr int kAbsLds = kAbsCols * 2 + 16;  // bytes per LDS weight row (padded)
constexpr int kAbsOut = kAbsCols + 4;       // floats per LDS row of a token block's results (padded)

// Workgroup (head h, output columns j0 .. j0 + 127) of the absorption.  An
// fp32 query (TQ = float) enters as bf16 hi + lo parts (q = hi + lo to about
// 2^-17), each multiplied by the bf16 weights with fp32 accumulation.
// QKN (QK-Norm MLA page, abstract): the content query is RMS-normalised over
// all heads of its token and weighted by g_q g_k first (the static key weight
// moved into the query); the workgroup derives each token's inverse RMS
// itself, from all n_heads * 128 entries of the token, so this suits few
// tokens; the product again enters as hi + lo parts.
template <typename TO, typename TQ = bf16, bool QKN = false>
__device__ __forceinline__ void absorb_block(const TQ* __restrict__ q_nope, const bf16* __restrict__ w_uk,
                                             TO* __restrict__ q_lat, int n_tok, int n_heads, int h, int j0,
                                             const QkArgs& qk = QkArgs{}) {
  constexpr bool QF = sizeof(TQ) == 4 || QKN;  // hi + lo parts
  __shared__ float inv_s[16];
  __shared__ __attribute__((aligned(16))) char wl[kNope * kAbsLds];
  // up to 16 tokens (one token block): the results go through LDS, the 4
  // waves writing their column blocks, then every thread storing 8
  // consecutive columns of one token (16-byte stores of whole row segments
  // instead of 2- or 4-byte ones; measured 4.65 -> 4.20 us for 4 tokens x 16
  // heads).  With more blocks each would add two barriers, which cost more
  // than the stores save (64 tokens x 128 heads: 15.1 -> 16.3 us), so those
  // store from the MFMA layout directly.
  __shared__ __attribute__((aligned(16))) float res[16 * kAbsOut];
  const bool staged = n_tok <= 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  // weight slice w_uk[h][0:128][j0:j0+128] -> LDS (row i: 256 B + pad)
  const bf16* w = w_uk + (int64_t)h * kNope * kLat + j0;
#pragma unroll
  for (int k = 0; k < kNope * (kAbsCols / 8) / 256; ++k) {  // a fixed count: all loads in flight at once
    const int e = tid + 256 * k, i = e / (kAbsCols / 8), c8 = e % (kAbsCols / 8);
    *(bf16x8*)(wl + i * kAbsLds + c8 * 16) = *(const bf16x8*)(w + (int64_t)i * kLat + c8 * 8);
  }
  __syncthreads();
  const int rq = l16 >> 2, qq = lane & 3;
  for (int t0 = 0; t0 < n_tok; t0 += 16) {
    // A operand: 16 tokens x 128 i, lane row l16, k = 32 ks + 8 lg + (0..7)
    bf16x8 qa[4], ql[QF ? 4 : 1];
    const int t = t0 + l16;
    if constexpr (QF) {
      // loads from a clamped token (always in bounds), rows past n_tok
      // zeroed afterwards: a load under the row condition compiles to a
      // branch with a full wait, one memory round trip per load
      f32x4 va[4][2];
      const int tcl = min(t, n_tok - 1);
      const bool t_ok = t < n_tok;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int64_t off = ((int64_t)tcl * n_heads + h) * kNope + 32 * ks + 8 * lg;
        if constexpr (sizeof(TQ) == 4) {
          va[ks][0] = *(const f32x4*)((const float*)q_nope + off);
          va[ks][1] = *(const f32x4*)((const float*)q_nope + off + 4);
        } else {
          const bf16x8 a = *(const bf16x8*)(q_nope + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            va[ks][0][e] = (float)a[e];
            va[ks][1][e] = (float)a[4 + e];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          va[ks][0][e] = t_ok ? va[ks][0][e] : 0.f;
          va[ks][1][e] = t_ok ? va[ks][1][e] : 0.f;
        }
      }
      if constexpr (QKN) {
        // inverse RMS of the block's tokens over all heads: wave w sums the
        // squares of tokens w, w + 4, w + 8, w + 12 with all 64 lanes, 8
        // entries per lane and load, the loads of a token issued together
        const int n_hd = n_heads * kNope;
        float ss[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tt = t0 + wave + 4 * j;
          float acc = 0.f;
          if (tt < n_tok) {
            const TQ* qt = q_nope + (int64_t)tt * n_hd;
#pragma unroll 4
            for (int i = 8 * lane; i < n_hd; i += 512) {
              if constexpr (sizeof(TQ) == 4) {
                const f32x4 a = *(const f32x4*)(qt + i), b = *(const f32x4*)(qt + i + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc += a[e] * a[e] + b[e] * b[e];
              } else {
                const bf16x8 a = *(const bf16x8*)(qt + i);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)a[e];
              }
            }
          }
          ss[j] = wave_sum(acc);
        }
        __syncthreads();  // the previous token block's factors are read
        if (lane == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) inv_s[wave + 4 * j] = 1.f / sqrtf(ss[j] / (float)n_hd + qk.eps);
        }
        __syncthreads();
        const float inv = inv_s[l16];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int gi = h * kNope + 32 * ks + 8 * lg;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            va[ks][0][e] = qk.g_q[gi + e] * qk.g_k[gi + e] * va[ks][0][e] * inv;
            va[ks][1][e] = qk.g_q[gi + 4 + e] * qk.g_k[gi + 4 + e] * va[ks][1][e] * inv;
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = e < 4 ? va[ks][0][e] : va[ks][1][e - 4];
          const bf16 hi = (bf16)v;
          qa[ks][e] = hi;
          ql[ks][e] = (bf16)(v - (float)hi);
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[ks] = t < n_tok ? *(const bf16x8*)(q_nope + ((int64_t)t * n_heads + h) * kNope + 32 * ks + 8 * lg)
                           : bf16x8{};
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int c0 = 32 * wave + 16 * cb;  // column block within the slice
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // B operand: lane col c0 + l16, k = 32 ks + 8 lg + (0..7) via two transposed reads
        const char* p0 = wl + (32 * ks + 8 * lg + rq) * kAbsLds + (c0 + 4 * qq) * 2;
        const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0));
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + 4 * kAbsLds));
        const bf16x8 wb = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], wb, acc, 0, 0, 0);
        if constexpr (QF) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[ks % (QF ? 4 : 1)], wb, acc, 0, 0, 0);
      }
      // D layout: lane holds column c0 + l16, rows (tokens) 4 lg + e
      if (staged) {
#pragma unroll
        for (int e = 0; e < 4; ++e) res[(4 * lg + e) * kAbsOut + c0 + l16] = acc[e];
        continue;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tt = t0 + 4 * lg + e;
        if (tt >= n_tok) continue;
        if constexpr (std::is_same_v<TO, SplitBf16>) {
          // hi plane, then lo plane, of the token's row
          bf16* row = (bf16*)q_lat + ((int64_t)tt * n_heads + h) * (2 * kLat);
          const bf16 hi = (bf16)acc[e];
          row[j0 + c0 + l16] = hi;
          row[kLat + j0 + c0 + l16] = (bf16)(acc[e] - (float)hi);
        } else {
          store_f(q_lat + ((int64_t)tt * n_heads + h) * kLat + j0 + c0 + l16, acc[e]);
        }
      }
    }
    if (staged) {
      __syncthreads();
      // thread: token r of the block, columns 8 c8 .. 8 c8 + 7 of the slice
      const int r = tid >> 4, c8 = tid & 15;
      const int tt = t0 + r;
      const f32x4 a = *(const f32x4*)(res + r * kAbsOut + 8 * c8);
      const f32x4 b = *(const f32x4*)(res + r * kAbsOut + 8 * c8 + 4);
      if (tt < n_tok) {
        const int64_t th = (int64_t)tt * n_heads + h;
        if constexpr (std::is_same_v<TO, SplitBf16>) {
          // hi plane, then lo plane, of the token's row
          bf16x8 hi8, lo8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = e < 4 ? a[e] : b[e - 4];
            const bf16 hi = (bf16)x;
            hi8[e] = hi;
            lo8[e] = (bf16)(x - (float)hi);
          }
          bf16* row = (bf16*)q_lat + th * (2 * kLat) + j0 + 8 * c8;
          *(bf16x8*)row = hi8;
          *(bf16x8*)(row + kLat) = lo8;
        } else if constexpr (std::is_same_v<TO, float>) {
          float* row = q_lat + th * kLat + j0 + 8 * c8;
          *(f32x4*)row = a;
          *(f32x4*)(row + 4) = b;
        } else {
          bf16x8 v8;
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = (bf16)(e < 4 ? a[e] : b[e - 4]);
          *(bf16x8*)(q_lat + th * kLat + j0 + 8 * c8) = v8;
        }
      }
    }
  }
}

template <typename TO>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const bf16* __restrict__ q_nope,
                                                          const bf16* __restrict__ w_uk, TO* __restrict__ q_lat,
                                                          int n_tok, int n_heads) {
  absorb_block(q_nope, w_uk, q_lat, n_tok, n_heads, blockIdx.x, blockIdx.y * kAbsCols);
}

// rope_relocate_q for up to kMaxShift shifts and the absorption in one launch:
// grid (heads, 4 + R); y < 4 are the absorption workgroups, y = 4 .. 4+R-1
// rotate the head's rotary query pairs (all tokens and shifts) between them.
template <typename TL, typename TR, typename TQ, bool QKN>
__global__ __launch_bounds__(256) void prepare_mfma_kernel(const TQ* __restrict__ q_nope,
                                                           const bf16* __restrict__ w_uk, TL* __restrict__ q_lat,
                                                           const bf16* __restrict__ q_pe,
                                                           const int64_t* __restrict__ pos, RopeTargets rt,
                                                           int n_tok, int n_heads, int d_rope, double base,
                                                           QkArgs qk) {
  const int h = blockIdx.x;
  if (blockIdx.y < kLat / kAbsCols) {
    absorb_block<TL, TQ, QKN>(q_nope, w_uk, q_lat, n_tok, n_heads, h, blockIdx.y * kAbsCols, qk);
    return;
  }
  const int half = d_rope / 2;
  const int per_shift = n_tok * half;
  const int r = blockIdx.y - kLat / kAbsCols, n_r = gridDim.y - kLat / kAbsCols;
  for (int idx = r * blockDim.x + threadIdx.x; idx < rt.n * per_shift; idx += n_r * blockDim.x) {
    const int k = idx / per_shift;
    const int t = (idx % per_shift) / half;
    const int i = idx % half;
    const int64_t th = (int64_t)t * n_heads + h;
    const bf16* x = q_pe + th * d_rope + 2 * i;
    float y0, y1;
    rope_pair((float)x[0], (float)x[1], pos[t] - (rt.shift[k] ? rt.shift[k][t] : 0), i, d_rope, base, &y0, &y1);
    TR* y = (TR*)rt.q_rot[k] + th * d_rope + 2 * i;
    store_f(y, y0);
    store_f(y + 1, y1);
  }
}

constexpr int kDv = 128;
constexpr int kUvTok = 32;                 // tokens per workgroup
constexpr int kUvWaves = kDv / 16;         // 8 waves, one per 16 output columns
constexpr int kUvLds = kLat * 2 + 16;      // bytes per LDS row of o_lat (padded)

// Workgroup (head h, tokens t0 .. t0 + 31): the o_lat rows of the block are
// staged in LDS once and shared by the 8 waves, wave w computing output
// columns 16 w .. 16 w + 15 with its 16 x 512 slice of w_uv as the B operand
// (64 registers, loaded before the rows so that both fetches overlap).  Each
// o_lat row is fetched once and a head's weights once per 32 tokens; the
// token blocks of a head are numbered onto one XCD (blocks h + n_heads * y,
// n_heads a multiple of 8), so their repeated weight reads meet in its L2.
template <typename TO>
__global__ __launch_bounds__(64 * kUvWaves) void out_uv_mfma_kernel(const bf16* __restrict__ o_lat,
                                                                    const bf16* __restrict__ w_uv,
                                                                    TO* __restrict__ out, int n_tok, int n_heads) {
  __shared__ __attribute__((aligned(16))) char os[kUvTok * kUvLds];
  const int h = blockIdx.x;
  const int t0 = blockIdx.y * kUvTok;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int v0 = 16 * wave;
  // B operand straight from HBM: lane col v = v0 + l16, k = 32 ks + 8 lg + (0..7)
  bf16x8 wb[16];
  const bf16* wr = w_uv + ((int64_t)h * kDv + v0 + l16) * kLat + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) wb[ks] = *(const bf16x8*)(wr + 32 * ks);
  // rows t0 .. t0 + 31 (clamped to the last token: always in bounds; rows
  // past n_tok are computed and never stored), 16 bytes per thread and load
  constexpr int kChunks = kUvTok * (kLat / 8) / (64 * kUvWaves);  // 4
  bf16x8 stage[kChunks];
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int e = tid + 64 * kUvWaves * k, r = e / (kLat / 8), c = e % (kLat / 8);
    const int t = min(t0 + r, n_tok - 1);
    stage[k] = *(const bf16x8*)(o_lat + ((int64_t)t * n_heads + h) * kLat + 8 * c);
  }
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int e = tid + 64 * kUvWaves * k, r = e / (kLat / 8), c = e % (kLat / 8);
    *(bf16x8*)(os + r * kUvLds + 16 * c) = stage[k];
  }
  __syncthreads();
#pragma unroll
  for (int tb = 0; tb < kUvTok / 16; ++tb) {
    if (t0 + 16 * tb >= n_tok) break;
    // A operand: lane row 16 tb + l16, k = 32 ks + 8 lg + (0..7)
    const char* arow = os + (16 * tb + l16) * kUvLds + 16 * lg;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 a = *(const bf16x8*)(arow + 64 * ks);
      acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wb[ks], acc[ks & 1], 0, 0, 0);
    }
    const f32x4 r = acc[0] + acc[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tt = t0 + 16 * tb + 4 * lg + e;
      if (tt < n_tok) store_f(out + ((int64_t)tt * n_heads + h) * kDv + v0 + l16, r[e]);
    }
  }
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool absorb_mfma_ok(const void* q_nope, const void* w_uk, const void* q_lat, int d_nope, int d_c) {
  return d_nope == kNope && d_c == kLat && al16(q_nope) && al16(w_uk) && al16(q_lat);
}

template <typename TL, typename TR, typename TQ>
static hipError_t prepare_launch(const void* q_nope, const void* w_uk, void* q_lat, const void* q_pe,
                                 const int64_t* pos, const RopeTargets& rt, int n_tok, int n_heads, int d_rope,
                                 double base, const QkArgs& qk, hipStream_t stream) {
  // rotation workgroups per head: one per 256 pairs (all tokens and shifts), at most 64
  const int pairs = rt.n * n_tok * (d_rope / 2);
  const int n_r = std::max(1, std::min(64, (pairs + 255) / 256));
  const dim3 grid(n_heads, kLat / kAbsCols + n_r);
  if (qk.g_q)
    return launch(prepare_mfma_kernel<TL, TR, TQ, true>, grid, dim3(256), stream, (const TQ*)q_nope,
                  (const bf16*)w_uk, (TL*)q_lat, (const bf16*)q_pe, pos, rt, n_tok, n_heads, d_rope, base, qk);
  return launch(prepare_mfma_kernel<TL, TR, TQ, false>, grid, dim3(256), stream, (const TQ*)q_nope,
                (const bf16*)w_uk, (TL*)q_lat, (const bf16*)q_pe, pos, rt, n_tok, n_heads, d_rope, base, qk);
}

template <typename TQ>
static hipError_t prepare_dispatch(const void* q_nope, const void* w_uk, void* q_lat, int lat_mode,
                                   const void* q_pe, const int64_t* pos, const RopeTargets& rt, bool rot_bf16,
                                   int n_tok, int n_heads, int d_rope, double base, const QkArgs& qk,
                                   hipStream_t stream) {
  if (lat_mode == 2 && rot_bf16)
    return prepare_launch<SplitBf16, bf16, TQ>(q_nope, w_uk, q_lat, q_pe, pos, rt, n_tok, n_heads, d_rope, base, qk,
                                               stream);
  if (lat_mode == 2)
    return prepare_launch<SplitBf16, float, TQ>(q_nope, w_uk, q_lat, q_pe, pos, rt, n_tok, n_heads, d_rope, base,
                                                qk, stream);
  const bool lat_bf16 = lat_mode == 1;
  if (lat_bf16 && rot_bf16)
    return prepare_launch<bf16, bf16, TQ>(q_nope, w_uk, q_lat, q_pe, pos, rt, n_tok, n_heads, d_rope, base, qk,
                                          stream);
  if (lat_bf16)
    return prepare_launch<bf16, float, TQ>(q_nope, w_uk, q_lat, q_pe, pos, rt, n_tok, n_heads, d_rope, base, qk,
                                           stream);
  if (rot_bf16)
    return prepare_launch<float, bf16, TQ>(q_nope, w_uk, q_lat, q_pe, pos, rt, n_tok, n_heads, d_rope, base, qk,
                                           stream);
  return prepare_launch<float, float, TQ>(q_nope, w_uk, q_lat, q_pe, pos, rt, n_tok, n_heads, d_rope, base, qk,
                                          stream);
}

hipError_t launch_prepare_mfma(const void* q_nope, bool q_f32, const void* w_uk, void* q_lat, int lat_mode,
                               const void* q_pe, const int64_t* pos, const RopeTargets& rt, bool rot_bf16, int n_tok,
                               int n_heads, int d_rope, double base, const QkArgs& qk, hipStream_t stream) {
  if (q_f32)
    return prepare_dispatch<float>(q_nope, w_uk, q_lat, lat_mode, q_pe, pos, rt, rot_bf16, n_tok, n_heads, d_rope,
                                   base, qk, stream);
  return prepare_dispatch<bf16>(q_nope, w_uk, q_lat, lat_mode, q_pe, pos, rt, rot_bf16, n_tok, n_heads, d_rope, base,
                                qk, stream);
}

hipError_t launch_absorb_mfma(const void* q_nope, const void* w_uk, void* q_lat, bool out_bf16, int n_tok,
                              int n_heads, hipStream_t stream) {
  dim3 grid(n_heads, kLat / kAbsCols);
  if (out_bf16)
    return launch(absorb_mfma_kernel<bf16>, grid, dim3(256), stream, (const bf16*)q_nope, (const bf16*)w_uk,
                       (bf16*)q_lat, n_tok, n_heads);
  else
    return launch(absorb_mfma_kernel<float>, grid, dim3(256), stream, (const bf16*)q_nope,
                       (const bf16*)w_uk, (float*)q_lat, n_tok, n_heads);
}

bool out_uv_mfma_ok(const void* o_lat, const void* w_uv, int d_c, int d_v) {
  return d_c == kLat && d_v == kDv && al16(o_lat) && al16(w_uv);
}

hipError_t launch_out_uv_mfma(const void* o_lat, const void* w_uv, void* out, bool out_bf16, int n_tok,
                              int n_heads, hipStream_t stream) {
  const dim3 grid(n_heads, (n_tok + kUvTok - 1) / kUvTok);
  if (out_bf16)
    return launch(out_uv_mfma_kernel<bf16>, grid, dim3(64 * kUvWaves), stream, (const bf16*)o_lat, (const bf16*)w_uv,
                       (bf16*)out, n_tok, n_heads);
  else
    return launch(out_uv_mfma_kernel<float>, grid, dim3(64 * kUvWaves), stream, (const bf16*)o_lat,
                       (const bf16*)w_uv, (float*)out, n_tok, n_heads);
}

}  // namespace mla
