// Per-query kernels of the MLA decode step: RoPE relocation of the query,
// key-side absorption (U_K^T q), value-side expansion (U_V o_lat) and the
// log-sum-exp merge of partial attention states.  Their cost is O(H * d)
// per query token, independent of the context length.
#include "mla_common.h"
#include "mla_kernels.h"

#include <algorithm>

#include <math.h>

namespace mla {

// ---------------------------------------------------------------------------
// RoPE relocation (MLA tutorial page, "Position Rotations Complicate the
// Absorption"; RedKnot-MLA abstract: query-side relocation).  Adjacent pairs
// (2i, 2i+1) rotate counter-clockwise by (pos - shift) * base^(-2i/d_rope)
// (rope_pair: int64 position difference, fp64 angle, fp32 rotation).
// ---------------------------------------------------------------------------
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void rope_kernel(const TI* __restrict__ q_pe, TO* __restrict__ q_rot,
                                                   const int64_t* __restrict__ pos,
                                                   const int64_t* __restrict__ shift, int n_tok,
                                                   int n_heads, int d_rope, double base) {
  const int half = d_rope / 2;
  const int64_t total = (int64_t)n_tok * n_heads * half;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx % half);
    const int64_t th = idx / half;  // token * n_heads + head
    const int t = (int)(th / n_heads);
    const int64_t rel = pos[t] - (shift ? shift[t] : 0);
    const TI* x = q_pe + th * d_rope + 2 * i;
    float y0, y1;
    rope_pair(load_f(x), load_f(x + 1), rel, i, d_rope, base, &y0, &y1);
    TO* y = q_rot + th * d_rope + 2 * i;
    store_f(y, y0);
    store_f(y + 1, y1);
  }
}

template <typename TI, typename TO>
static hipError_t rope_launch(const void* q_pe, void* q_rot, const int64_t* pos, const int64_t* shift, int n_tok,
                        int n_heads, int d_rope, double base, int blocks, hipStream_t stream) {
  return launch((rope_kernel<TI, TO>), dim3(blocks), dim3(256), stream, (const TI*)q_pe, (TO*)q_rot,
                     pos, shift, n_tok, n_heads, d_rope, base);
}

hipError_t launch_rope(const void* q_pe, bool in_bf, void* q_rot, bool out_bf, const int64_t* pos,
                       const int64_t* shift, int n_tok, int n_heads, int d_rope, double base,
                       hipStream_t stream) {
  const int64_t total = (int64_t)n_tok * n_heads * (d_rope / 2);
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (in_bf && out_bf) return rope_launch<bf16, bf16>(q_pe, q_rot, pos, shift, n_tok, n_heads, d_rope, base, blocks, stream);
  if (in_bf) return rope_launch<bf16, float>(q_pe, q_rot, pos, shift, n_tok, n_heads, d_rope, base, blocks, stream);
  if (out_bf) return rope_launch<float, bf16>(q_pe, q_rot, pos, shift, n_tok, n_heads, d_rope, base, blocks, stream);
  return rope_launch<float, float>(q_pe, q_rot, pos, shift, n_tok, n_heads, d_rope, base, blocks, stream);
}

// ---------------------------------------------------------------------------
// Key absorption (MLA tutorial page, "Move the Key Projection Into the
// Query"): q_lat[t][h][j] = sum_i w_uk[h][i][j] q_nope[t][h][i].
// Grid (heads, column blocks of 256); each thread owns one output column j and
// a chunk of TCH tokens; q_nope of the chunk is staged in LDS.  Reads each
// weight column once per token chunk (coalesced along j).
// ---------------------------------------------------------------------------
constexpr int kAbsorbTch = 16;
constexpr int kAbsorbMaxNope = 256;

template <typename T, typename TO>
__global__ __launch_bounds__(256) void absorb_kernel(const T* __restrict__ q_nope,
                                                     const T* __restrict__ w_uk, TO* __restrict__ q_lat,
                                                     int n_tok, int n_heads, int d_nope, int d_c) {
  __shared__ float qs[kAbsorbTch][kAbsorbMaxNope];
  const int h = blockIdx.x;
  const int j = blockIdx.y * 256 + threadIdx.x;
  const T* w = w_uk + (int64_t)h * d_nope * d_c;
  for (int t0 = 0; t0 < n_tok; t0 += kAbsorbTch) {
    const int nt = min(kAbsorbTch, n_tok - t0);
    __syncthreads();
    for (int e = threadIdx.x; e < nt * d_nope; e += 256) {
      const int tt = e / d_nope, i = e % d_nope;
      qs[tt][i] = load_f(q_nope + ((int64_t)(t0 + tt) * n_heads + h) * d_nope + i);
    }
    __syncthreads();
    if (j < d_c) {
      float acc[kAbsorbTch];
#pragma unroll
      for (int tt = 0; tt < kAbsorbTch; ++tt) acc[tt] = 0.f;
      for (int i = 0; i < d_nope; ++i) {
        const float wv = load_f(w + (int64_t)i * d_c + j);
#pragma unroll
        for (int tt = 0; tt < kAbsorbTch; ++tt) acc[tt] += wv * qs[tt][i];
      }
      for (int tt = 0; tt < nt; ++tt)
        store_f(q_lat + ((int64_t)(t0 + tt) * n_heads + h) * d_c + j, acc[tt]);
    }
  }
}

hipError_t launch_absorb(const void* q_nope, const void* w_uk, bool in_bf, void* q_lat, bool out_bf, int n_tok,
                         int n_heads, int d_nope, int d_c, hipStream_t stream) {
  if (in_bf && absorb_mfma_ok(q_nope, w_uk, q_lat, d_nope, d_c))
    return launch_absorb_mfma(q_nope, w_uk, q_lat, out_bf, n_tok, n_heads, stream);
  dim3 grid(n_heads, (d_c + 255) / 256);
#define MLA_ABSORB(TI, TO)                                                                                \
  return launch((absorb_kernel<TI, TO>), grid, dim3(256), stream, (const TI*)q_nope, (const TI*)w_uk, \
                     (TO*)q_lat, n_tok, n_heads, d_nope, d_c)
  if (in_bf && out_bf) MLA_ABSORB(bf16, bf16);
  if (in_bf) MLA_ABSORB(bf16, float);
  if (out_bf) MLA_ABSORB(float, bf16);
  MLA_ABSORB(float, float);
#undef MLA_ABSORB
}

// ---------------------------------------------------------------------------
// Value expansion (MLA tutorial page, "Move the Value Expansion After the
// Weighted Sum"): out[t][h][i] = sum_j w_uv[h][i][j] o_lat[t][h][j].
// One wave per (head, output row i): the weight row stays in registers, the
// wave loops over tokens with a shuffle reduction.
// ---------------------------------------------------------------------------
constexpr int kOutMaxK = 16;  // d_c <= 1024

template <typename TL, typename TW, typename TO>
__global__ __launch_bounds__(256) void out_uv_kernel(const TL* __restrict__ o_lat,
                                                     const TW* __restrict__ w_uv, TO* __restrict__ out,
                                                     int n_tok, int n_heads, int d_c, int d_v) {
  const int h = blockIdx.x;
  const int i = blockIdx.y * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (i >= d_v) return;
  const TW* w = w_uv + ((int64_t)h * d_v + i) * d_c;
  float wr[kOutMaxK];
#pragma unroll
  for (int k = 0; k < kOutMaxK; ++k) {
    const int j = lane + 64 * k;
    wr[k] = j < d_c ? load_f(w + j) : 0.f;
  }
  for (int t = 0; t < n_tok; ++t) {
    const TL* o = o_lat + ((int64_t)t * n_heads + h) * d_c;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kOutMaxK; ++k) {
      const int j = lane + 64 * k;
      if (j < d_c) acc += wr[k] * load_f(o + j);
    }
    acc = wave_sum(acc);
    if (lane == 0) store_f(out + ((int64_t)t * n_heads + h) * d_v + i, acc);
  }
}

template <typename TL, typename TW>
static hipError_t out_uv_launch(const void* o_lat, const void* w_uv, void* out, bool out_bf, int n_tok, int n_heads,
                          int d_c, int d_v, hipStream_t stream) {
  dim3 grid(n_heads, (d_v + 3) / 4);
  if (out_bf)
    return launch((out_uv_kernel<TL, TW, bf16>), grid, dim3(256), stream, (const TL*)o_lat,
                       (const TW*)w_uv, (bf16*)out, n_tok, n_heads, d_c, d_v);
  else
    return launch((out_uv_kernel<TL, TW, float>), grid, dim3(256), stream, (const TL*)o_lat,
                       (const TW*)w_uv, (float*)out, n_tok, n_heads, d_c, d_v);
}

hipError_t launch_out_uv(const void* o_lat, bool o_bf, const void* w_uv, bool w_bf, void* out, bool out_bf,
                         int n_tok, int n_heads, int d_c, int d_v, hipStream_t stream) {
  if (o_bf && w_bf && out_uv_mfma_ok(o_lat, w_uv, d_c, d_v))
    return launch_out_uv_mfma(o_lat, w_uv, out, out_bf, n_tok, n_heads, stream);
  if (o_bf && w_bf) return out_uv_launch<bf16, bf16>(o_lat, w_uv, out, out_bf, n_tok, n_heads, d_c, d_v, stream);
  if (o_bf) return out_uv_launch<bf16, float>(o_lat, w_uv, out, out_bf, n_tok, n_heads, d_c, d_v, stream);
  if (w_bf) return out_uv_launch<float, bf16>(o_lat, w_uv, out, out_bf, n_tok, n_heads, d_c, d_v, stream);
  return out_uv_launch<float, float>(o_lat, w_uv, out, out_bf, n_tok, n_heads, d_c, d_v, stream);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partial states (RedKnot-MLA abstract: the paths are
// merged before one shared output projection).  One 256-thread block per
// (row, chunk of `cols` = 128, 256 or 512 columns): wave 0 compacts the live
// slots (lse > -inf) in slot order with their weights exp(lse_j - max), so
// -inf slots are never read; the threads then split into G = 256 / (cols/4)
// slot groups of cols/4 column threads (float4 each), group g summing live
// slots g, g + G, ... with 4 loads in flight, and the G group sums are added
// in a fixed order, so the result is bitwise repeatable.  Few rows get narrow
// chunks (more blocks in flight), many rows whole-row blocks.
// ---------------------------------------------------------------------------
constexpr int kCombMaxPart = 1024;

template <typename TO, typename TP>
__global__ __launch_bounds__(256) void combine_kernel(const TP* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, int n_rows,
                                                      int n_part, int d_c, int cols, TO* __restrict__ o_lat,
                                                      float* __restrict__ lse) {
  __shared__ int live_idx[kCombMaxPart];
  __shared__ float live_w[kCombMaxPart];
  __shared__ f32x4 red[224];  // (G - 1) * cols / 4 <= 224 for cols >= 128
  __shared__ float s_inv, s_lse;
  __shared__ int s_n;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const float* lp = lse_part + (int64_t)row * n_part;
  if (tid < 64) {
    float m = -INFINITY;
    for (int j = lane; j < n_part; j += 64) m = fmaxf(m, lp[j]);
    m = wave_max(m);
    float tot = 0.f;
    int n = 0;
    for (int base = 0; base < n_part; base += 64) {
      const int j = base + lane;
      const float l = j < n_part ? lp[j] : -INFINITY;
      const bool live = l != -INFINITY;
      const float w = live ? expf(l - m) : 0.f;
      tot += w;
      const uint64_t bal = __ballot(live);
      if (live) {
        const int pos = n + __popcll(bal & ((1ull << lane) - 1));
        live_idx[pos] = j;
        live_w[pos] = w;
      }
      n += __popcll(bal);
    }
    tot = wave_sum(tot);
    if (lane == 0) {
      s_n = n;
      s_inv = n > 0 ? 1.f / tot : 0.f;
      s_lse = n > 0 ? m + logf(tot) : -INFINITY;
    }
  }
  __syncthreads();
  const int n = s_n;
  const float inv = s_inv;
  if (lse && blockIdx.y == 0 && tid == 0) lse[row] = s_lse;
  const int ct_n = cols / 4;       // column threads per group
  const int G = 256 / ct_n;        // slot groups
  const int g = tid / ct_n, ct = tid % ct_n;
  const int c = blockIdx.y * cols + 4 * ct;  // d_c is a multiple of 4: c < d_c means 4 whole columns
  const TP* op = o_part + (int64_t)row * n_part * d_c + c;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (c < d_c) {
    int i = g;
    for (; i + 3 * G < n; i += 4 * G) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = load_part4(op + (int64_t)live_idx[i + u * G] * d_c);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += live_w[i + u * G] * v[u];
    }
    for (; i < n; i += G) acc += live_w[i] * load_part4(op + (int64_t)live_idx[i] * d_c);
  }
  if (g > 0) red[(g - 1) * ct_n + ct] = acc;
  __syncthreads();
  if (g == 0 && c < d_c) {
    for (int k = 0; k < G - 1; ++k) acc += red[k * ct_n + ct];
    TO* orow = o_lat + (int64_t)row * d_c + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_f(orow + e, acc[e] * inv);
  }
}

// The same merge for many rows of 512 columns: one wave per row (four rows
// per 256-thread block), lane l owning columns 8 l .. 8 l + 7, so a live
// slot is one 16-byte load per lane (bf16 partials) and no block-wide
// synchronisation is needed.  The wave walks the live slots in slot order,
// four loads in flight, so the sum is bitwise repeatable.
template <typename TO, typename TP>
__global__ __launch_bounds__(256) void combine_rows_kernel(const TP* __restrict__ o_part,
                                                           const float* __restrict__ lse_part, int n_rows,
                                                           int n_part, TO* __restrict__ o_lat,
                                                           float* __restrict__ lse) {
  constexpr int kD = 512;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const float* lp = lse_part + (int64_t)row * n_part;
  float m = -INFINITY;
  for (int j = lane; j < n_part; j += 64) m = fmaxf(m, lp[j]);
  m = wave_max(m);
  const TP* op = o_part + (int64_t)row * n_part * kD + 8 * lane;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto load8 = [&](int j, float (&v)[8]) {
    const TP* p = op + (int64_t)j * kD;
    const f32x4 a = load_part4(p), b = load_part4(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  };
  float tot = 0.f;
  for (int base = 0; base < n_part; base += 64) {
    const int j = base + lane;
    const float l = j < n_part ? lp[j] : -INFINITY;
    const bool live = l != -INFINITY;
    const float w = live ? expf(l - m) : 0.f;
    tot += w;
    uint64_t bal = __ballot(live);
    while (bal) {
      int src[4];
      int k = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        src[u] = bal ? __ffsll((long long)bal) - 1 : -1;
        if (bal) {
          bal &= bal - 1;
          ++k;
        }
      }
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < k) load8(base + src[u], v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < k) {
          const float wu = __shfl(w, src[u]);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += wu * v[u][e];
        }
    }
  }
  tot = wave_sum(tot);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;  // tot > 0 exactly when a slot is live
  if (lse && lane == 0) lse[row] = tot > 0.f ? m + logf(tot) : -INFINITY;
  TO* orow = o_lat + (int64_t)row * kD + 8 * lane;
#pragma unroll
  for (int e = 0; e < 8; ++e) store_f(orow + e, acc[e] * inv);
}

template <typename TP>
static hipError_t combine_launch(const TP* o_part, const float* lse_part, int n_rows, int n_part, int d_c,
                                 void* o_lat, bool out_bf16, float* lse, hipStream_t stream) {
  if (d_c == 512 && n_rows >= 1024) {  // many whole rows: a wave per row
    const dim3 grid((n_rows + 3) / 4);
    if (out_bf16)
      return launch(combine_rows_kernel<bf16, TP>, grid, dim3(256), stream, o_part, lse_part, n_rows, n_part,
                    (bf16*)o_lat, lse);
    return launch(combine_rows_kernel<float, TP>, grid, dim3(256), stream, o_part, lse_part, n_rows, n_part,
                  (float*)o_lat, lse);
  }
  // chunk width: ~1024 blocks in flight for few rows, whole 512-column rows for many
  const int cols = n_rows >= 1024 ? 512 : n_rows >= 512 ? 256 : 128;
  const dim3 grid(n_rows, (d_c + cols - 1) / cols);
  if (out_bf16)
    return launch(combine_kernel<bf16, TP>, grid, dim3(256), stream, o_part, lse_part, n_rows, n_part, d_c, cols,
                  (bf16*)o_lat, lse);
  return launch(combine_kernel<float, TP>, grid, dim3(256), stream, o_part, lse_part, n_rows, n_part, d_c, cols,
                (float*)o_lat, lse);
}

hipError_t launch_combine(const void* o_part, bool part_bf16, const float* lse_part, int n_rows, int n_part,
                          int d_c, void* o_lat, bool out_bf16, float* lse, hipStream_t stream) {
  if (part_bf16)
    return combine_launch((const bf16*)o_part, lse_part, n_rows, n_part, d_c, o_lat, out_bf16, lse, stream);
  return combine_launch((const float*)o_part, lse_part, n_rows, n_part, d_c, o_lat, out_bf16, lse, stream);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge and value expansion in one pass (MLA tutorial page, "Move
// the Value Expansion After the Weighted Sum"; RedKnot-MLA abstract: the
// merged state goes through one shared output projection).  NQ 1024-thread
// blocks per (token, head) row, block q producing output columns
// [q dq, (q + 1) dq), dq = ceil(d_v / NQ); each merges the whole row (the
// repeated partial reads of a row's NQ blocks meet in L2: a row's blocks,
// and the rows of one head, are numbered onto one XCD):
//  * the head's U_V rows are loaded first (bf16, d_c = 512: thread (v, part)
//    of the TPO = 8 NQ threads of row v holds columns 64 NQ k + 8 part .. + 7,
//    k < 8 / NQ, in registers), independent of the merge, so their latency
//    overlaps it;
//  * wave 0 compacts the live slots and their weights as combine_kernel does
//    (its lse loads go out before its weight loads);
//  * 8 slot groups of 128 column threads (float4) sum the live partials and
//    the group sums are added in a fixed order into the fp32 row o (LDS),
//    stored as o_lat when asked for;
//  * out[v] = sum_c U_V[v][c] o[c]: the TPO threads of row v each take every
//    TPO-th group of 8 columns and add their sums with lane shuffles.  o
//    enters the product in fp32.
// Each row reads its head's d_v x d_c weights, so this suits few query
// tokens; many tokens use combine_kernel and the out_uv kernels.  NQ > 1
// spreads few rows over more CUs (each block is bound by what one CU can
// fetch).
// ---------------------------------------------------------------------------
template <typename TO, typename TW, bool VEC, int NQ, typename TP>
__global__ __launch_bounds__(1024) void combine_out_uv_kernel(const TP* __restrict__ o_part,
                                                              const float* __restrict__ lse_part, int n_tok,
                                                              int n_heads, int n_part, int d_c,
                                                              const TW* __restrict__ w_uv, int d_v,
                                                              TO* __restrict__ o_lat, float* __restrict__ lse,
                                                              TO* __restrict__ out) {
  constexpr int TPO = 8 * NQ;  // threads per output column
  constexpr int NW = 8 / NQ;   // bf16x8 weight chunks per thread (VEC)
  __shared__ int live_idx[kCombMaxPart];
  __shared__ float live_w[kCombMaxPart];
  __shared__ f32x4 red[7 * 128];
  __shared__ __attribute__((aligned(16))) float o_s[512];
  __shared__ float s_inv, s_lse;
  __shared__ int s_n;
  // block -> (head, token, q): consecutive items share an XCD (block b runs
  // on XCD b % 8); q fastest, then token, then head
  const int n_items = n_heads * n_tok * NQ;
  const int per = (n_items + 7) / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= n_items) return;
  const int q = item % NQ;
  const int t = (item / NQ) % n_tok;
  const int h = item / (NQ * n_tok);
  const int64_t row = (int64_t)t * n_heads + h;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int dq = (d_v + NQ - 1) / NQ;
  const int vl = tid / TPO, part = tid % TPO;  // output column (of this block's dq) and its share of d_c
  const int v = q * dq + vl;
  const bool v_ok = vl < dq && v < d_v;
  const TW* wrow = w_uv + ((int64_t)h * d_v + (v_ok ? v : 0)) * d_c;
  const float* lp = lse_part + row * n_part;
  // wave 0 issues its lse loads before the weights: loads return in order
  float lv0 = -INFINITY, lv1 = -INFINITY;
  if (tid < 64 && n_part <= 128) {
    lv0 = lane < n_part ? lp[lane] : -INFINITY;
    lv1 = lane + 64 < n_part ? lp[lane + 64] : -INFINITY;
  }
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 wv[VEC ? NW : 1];
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < NW; ++k) wv[k] = v_ok ? *(const bf16x8*)(wrow + 8 * TPO * k + 8 * part) : bf16x8{};
  }
  if (tid < 64) {
    float m = fmaxf(lv0, lv1);
    if (n_part > 128)
      for (int j = lane; j < n_part; j += 64) m = fmaxf(m, lp[j]);
    m = wave_max(m);
    float tot = 0.f;
    int n = 0;
    for (int base = 0; base < n_part; base += 64) {
      const int j = base + lane;
      const float l = n_part <= 128 ? (base == 0 ? lv0 : lv1) : j < n_part ? lp[j] : -INFINITY;
      const bool live = l != -INFINITY;
      const float w = live ? expf(l - m) : 0.f;
      tot += w;
      const uint64_t bal = __ballot(live);
      if (live) {
        const int pos = n + __popcll(bal & ((1ull << lane) - 1));
        live_idx[pos] = j;
        live_w[pos] = w;
      }
      n += __popcll(bal);
    }
    tot = wave_sum(tot);
    if (lane == 0) {
      s_n = n;
      s_inv = n > 0 ? 1.f / tot : 0.f;
      s_lse = n > 0 ? m + logf(tot) : -INFINITY;
    }
  }
  __syncthreads();
  const int n = s_n;
  const float inv = s_inv;
  if (lse && tid == 0 && q == 0) lse[row] = s_lse;
  const int g = tid >> 7, ct = tid & 127;  // 8 slot groups x 128 column threads
  const int c = 4 * ct;
  const TP* op = o_part + row * n_part * d_c + c;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (c < d_c) {
    int i = g;
    for (; i + 7 * 8 < n; i += 8 * 8) {  // 8 loads in flight: 64 live slots in one round
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = load_part4(op + (int64_t)live_idx[i + u * 8] * d_c);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += live_w[i + u * 8] * x[u];
    }
    for (; i < n; i += 8) acc += live_w[i] * load_part4(op + (int64_t)live_idx[i] * d_c);
  }
  if (g > 0) red[(g - 1) * 128 + ct] = acc;
  __syncthreads();
  if (g == 0 && c < d_c) {
    for (int k = 0; k < 7; ++k) acc += red[k * 128 + ct];
    acc *= inv;
    *(f32x4*)(o_s + c) = acc;
    if (o_lat && q == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) store_f(o_lat + row * d_c + c + e, acc[e]);
    }
  }
  __syncthreads();
  float sum = 0.f;
  if (v_ok) {
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const f32x4 a = *(const f32x4*)(o_s + 8 * TPO * k + 8 * part);
        const f32x4 b = *(const f32x4*)(o_s + 8 * TPO * k + 8 * part + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += (float)wv[k][e] * a[e] + (float)wv[k][4 + e] * b[e];
      }
    } else {
      for (int cc = part; cc < d_c; cc += TPO) sum += load_f(wrow + cc) * o_s[cc];
    }
  }
#pragma unroll
  for (int o = 1; o < TPO; o <<= 1) sum += __shfl_xor(sum, o);
  if (v_ok && part == 0) store_f(out + row * d_v + v, sum);
}

template <typename TO, typename TW, int NQ, typename TP>
static hipError_t cou_launch_nq(const TP* o_part, const float* lse_part, int n_tok, int n_heads, int n_part,
                                int d_c, const void* w_uv, int d_v, void* o_lat, float* lse, void* out,
                                hipStream_t stream) {
  const int64_t n_items = (int64_t)n_heads * n_tok * NQ;
  const dim3 grid((unsigned)(8 * ((n_items + 7) / 8)));
  if constexpr (sizeof(TW) == 2) {
    if (d_c == 512 && (reinterpret_cast<uintptr_t>(w_uv) & 15u) == 0)
      return launch(combine_out_uv_kernel<TO, TW, true, NQ, TP>, grid, dim3(1024), stream, o_part, lse_part, n_tok,
                    n_heads, n_part, d_c, (const TW*)w_uv, d_v, (TO*)o_lat, lse, (TO*)out);
  }
  return launch(combine_out_uv_kernel<TO, TW, false, NQ, TP>, grid, dim3(1024), stream, o_part, lse_part, n_tok,
                n_heads, n_part, d_c, (const TW*)w_uv, d_v, (TO*)o_lat, lse, (TO*)out);
}

// NQ: blocks per row, so that about 256 blocks (one per CU) run
template <typename TO, typename TW, typename TP>
static hipError_t cou_launch(const TP* o_part, const float* lse_part, int n_tok, int n_heads, int n_part,
                             int d_c, const void* w_uv, int d_v, void* o_lat, float* lse, void* out,
                             hipStream_t stream) {
  const int64_t rows = (int64_t)n_tok * n_heads;
  if (rows * 4 <= 256)
    return cou_launch_nq<TO, TW, 4>(o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, d_v, o_lat, lse, out,
                                    stream);
  if (rows * 2 <= 256)
    return cou_launch_nq<TO, TW, 2>(o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, d_v, o_lat, lse, out,
                                    stream);
  return cou_launch_nq<TO, TW, 1>(o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, d_v, o_lat, lse, out,
                                  stream);
}

template <typename TP>
static hipError_t cou_dispatch(const TP* o_part, const float* lse_part, int n_tok, int n_heads, int n_part, int d_c,
                               const void* w_uv, bool w_bf16, int d_v, void* o_lat, float* lse, void* out,
                               bool out_bf16, hipStream_t stream) {
  if (out_bf16 && w_bf16)
    return cou_launch<bf16, bf16>(o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, d_v, o_lat, lse, out, stream);
  if (out_bf16)
    return cou_launch<bf16, float>(o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, d_v, o_lat, lse, out, stream);
  if (w_bf16)
    return cou_launch<float, bf16>(o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, d_v, o_lat, lse, out, stream);
  return cou_launch<float, float>(o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, d_v, o_lat, lse, out, stream);
}

hipError_t launch_combine_out_uv(const void* o_part, bool part_bf16, const float* lse_part, int n_tok, int n_heads,
                                 int n_part, int d_c, const void* w_uv, bool w_bf16, int d_v, void* o_lat,
                                 float* lse, void* out, bool out_bf16, hipStream_t stream) {
  if (part_bf16)
    return cou_dispatch((const bf16*)o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, w_bf16, d_v, o_lat, lse,
                        out, out_bf16, stream);
  return cou_dispatch((const float*)o_part, lse_part, n_tok, n_heads, n_part, d_c, w_uv, w_bf16, d_v, o_lat, lse,
                      out, out_bf16, stream);
}

// ---------------------------------------------------------------------------
// int8 latent cache writer (QuantMLA abstract: a low-bit latent cache that
// attention dequantizes; here the plain per-row symmetric int8 form): one
// wave per stored row.  amax = max |c_i| over the row's d_c latent entries,
// scale = amax / 127 (IEEE fp32 quotient), code_i = the nearest integer to
// c_i / scale (fp32 quotient, ties to even) clamped to [-127, 127]; a zero
// row has scale 0 and codes 0.  The packed row is the d_c codes followed by
// the d_rope 16-bit rotary entries copied unchanged.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_latent_i8_kernel(const bf16* __restrict__ rows, int64_t n_rows,
                                                                 int d_c, int d_rope, char* __restrict__ out,
                                                                 float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < n_rows; r += (int64_t)gridDim.x * 4) {
    const int in_w = d_c + d_rope;
    const int out_w = d_c + 2 * d_rope;
    const bf16* src = rows + r * in_w;
    char* dst = out + r * out_w;
    // lane owns latent entries [8 lane, 8 lane + 8) (d_c <= 512, a multiple of 8)
    float v[8];
    const bool mine = 8 * lane < d_c;
    float amax = 0.f;
  #pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = mine ? (float)src[8 * lane + e] : 0.f;
      amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = wave_max(amax);
    const float scale = amax / 127.f;
    if (mine) {
      unsigned lo = 0, hi = 0;
  #pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = scale > 0.f ? fminf(fmaxf(rintf(v[e] / scale), -127.f), 127.f) : 0.f;
        const unsigned byte = (unsigned)((int)q & 0xff);
        if (e < 4) lo |= byte << (8 * e);
        else hi |= byte << (8 * (e - 4));
      }
      *(uint2*)(dst + 8 * lane) = uint2{lo, hi};
    }
    // rotary entries: 2 d_rope bytes in 8-byte pieces
    const unsigned short* rs = (const unsigned short*)(src + d_c);
    if (lane < d_rope / 4) {
      const unsigned short* p = rs + 4 * lane;
      unsigned lo = (unsigned)p[0] | ((unsigned)p[1] << 16), hi = (unsigned)p[2] | ((unsigned)p[3] << 16);
      *(uint2*)(dst + d_c + 8 * lane) = uint2{lo, hi};
    }
    if (lane == 0) scales[r] = scale;
  }  // rows (grid-stride: the grid is capped)
}

// Grid-stride kernels take at most this many workgroups (a launch's work-items
// must fit 32 bits per dimension).
constexpr int64_t kMaxStrideBlocks = 65536;

// ---------------------------------------------------------------------------
// int4 cache writer (QuantMLA abstract: joint INT4 caching of the content and
// rotary caches; here the plain per-row symmetric form): one wave per stored
// row, the content latent and the rotary key quantized separately.  For each
// part: scale = amax / 7 (IEEE fp32 quotient), code_i = the nearest integer to
// x_i / scale (fp32 quotient, ties to even) clamped to [-7, 7] (a zero part:
// scale 0, codes 0).  Codes are packed two per byte, entry 2j in the low
// nibble of byte j (4-bit two's complement): the packed row is d_c / 2
// content bytes then d_rope / 2 rotary bytes; scales[r] = (content, rotary).
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned pack8_i4(const float (&v)[8], float scale) {
  unsigned w = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = scale > 0.f ? fminf(fmaxf(rintf(v[e] / scale), -7.f), 7.f) : 0.f;
    w |= ((unsigned)(int)q & 0xfu) << (4 * e);
  }
  return w;
}

__global__ __launch_bounds__(256) void quantize_latent_i4_kernel(const bf16* __restrict__ rows, int64_t n_rows,
                                                                 int d_c, int d_rope, char* __restrict__ out,
                                                                 float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < n_rows; r += (int64_t)gridDim.x * 4) {
    const bf16* src = rows + r * (d_c + d_rope);
    char* dst = out + r * ((d_c + d_rope) / 2);
    // lane owns content entries [8 lane, 8 lane + 8) and rotary entries
    // [8 lane, 8 lane + 8) (d_c <= 512, d_rope <= 128, multiples of 8)
    const bool mc = 8 * lane < d_c, mr = 8 * lane < d_rope;
    float vc[8], vr[8], ac = 0.f, ar = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vc[e] = mc ? (float)src[8 * lane + e] : 0.f;
      vr[e] = mr ? (float)src[d_c + 8 * lane + e] : 0.f;
      ac = fmaxf(ac, fabsf(vc[e]));
      ar = fmaxf(ar, fabsf(vr[e]));
    }
    const float sc = wave_max(ac) / 7.f, sr = wave_max(ar) / 7.f;
    if (mc) *(unsigned*)(dst + 4 * lane) = pack8_i4(vc, sc);
    if (mr) *(unsigned*)(dst + d_c / 2 + 4 * lane) = pack8_i4(vr, sr);
    if (lane == 0) *(float2*)(scales + 2 * r) = float2{sc, sr};
  }  // rows (grid-stride: the grid is capped)
}

hipError_t launch_quantize_latent_i4(const void* rows, int64_t n_rows, int d_c, int d_rope, void* out,
                                     float* scales, hipStream_t stream) {
  const dim3 grid((unsigned)std::min<int64_t>((n_rows + 3) / 4, kMaxStrideBlocks));
  return launch(quantize_latent_i4_kernel, grid, dim3(256), stream, (const bf16*)rows, n_rows, d_c, d_rope,
                (char*)out, scales);
}

hipError_t launch_quantize_latent_i8(const void* rows, int64_t n_rows, int d_c, int d_rope, void* out,
                                     float* scales, hipStream_t stream) {
  const dim3 grid((unsigned)std::min<int64_t>((n_rows + 3) / 4, kMaxStrideBlocks));
  return launch(quantize_latent_i8_kernel, grid, dim3(256), stream, (const bf16*)rows, n_rows, d_c, d_rope,
                (char*)out, scales);
}

// ---------------------------------------------------------------------------
// QK-Norm (QK-Norm MLA page, abstract): RMSNorm after the projections, the
// statistic over a token's whole content projection.
//  * qknorm_query_kernel: one block per query token; the sum of squares over
//    all heads' q_nope, then q_out = g_q g_k q / rms (the static key weight
//    moved into the query); qknorm_query_vec_kernel is its 16-byte form.
//  * qknorm_gram_kernel: G = sum_h U_K[h]^T U_K[h] (d_c x d_c), one block per
//    row a of G, threads over b; fp32 sums over the n_heads * d_nope terms.
//  * qknorm_rinv_kernel: 16 stored rows per block, their latents in LDS;
//    thread j forms (G c)_j for the 16 rows from column j of G (G is
//    symmetric, so the reads run along rows of G), then c . G c per row and
//    1 / sqrt(c.Gc / (n_heads d_nope) + eps), the inverse RMS of the row's
//    expanded content key over all heads.
// ---------------------------------------------------------------------------
template <typename TI>
__global__ __launch_bounds__(256) void qknorm_query_kernel(const TI* __restrict__ q_nope, const float* __restrict__ g_q,
                                                           const float* __restrict__ g_k, int n_hd, float eps,
                                                           float* __restrict__ q_out) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const TI* q = q_nope + (int64_t)t * n_hd;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n_hd; i += 256) {
    const float v = load_f(q + i);
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.f / sqrtf(tot / (float)n_hd + eps);
  float* o = q_out + (int64_t)t * n_hd;
  for (int i = threadIdx.x; i < n_hd; i += 256) o[i] = g_q[i] * g_k[i] * load_f(q + i) * inv;
}

// Rows of up to 16384 entries (n_hd a multiple of 8, every pointer 16-byte
// aligned): 1024 threads, each holding two groups of 8 consecutive entries
// with their g_q and g_k in registers, so the row and both weight vectors are
// read once, in one round of loads, before the sum of squares.
template <typename TI>
__global__ __launch_bounds__(1024) void qknorm_query_reg_kernel(const TI* __restrict__ q_nope,
                                                                const float* __restrict__ g_q,
                                                                const float* __restrict__ g_k, int n_hd, float eps,
                                                                float* __restrict__ q_out) {
  constexpr int kG = 2;  // groups of 8 entries per thread
  __shared__ float red[16];
  const int t = blockIdx.x;
  const TI* q = q_nope + (int64_t)t * n_hd;
  f32x4 v[kG][2], gq[kG][2], gk[kG][2];
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    const int i = 8 * ((int)threadIdx.x + 1024 * k);
    const bool ok = i < n_hd;
    const int ic = ok ? i : 0;  // always in bounds; the group is dropped below
    if constexpr (sizeof(TI) == 4) {
      v[k][0] = *(const f32x4*)(q + ic);
      v[k][1] = *(const f32x4*)(q + ic + 4);
    } else {
      const bf16x8 b = *(const bf16x8*)(q + ic);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[k][0][e] = (float)b[e];
        v[k][1][e] = (float)b[4 + e];
      }
    }
    gq[k][0] = *(const f32x4*)(g_q + ic);
    gq[k][1] = *(const f32x4*)(g_q + ic + 4);
    gk[k][0] = *(const f32x4*)(g_k + ic);
    gk[k][1] = *(const f32x4*)(g_k + ic + 4);
    if (!ok) v[k][0] = v[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kG; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += v[k][0][e] * v[k][0][e] + v[k][1][e] * v[k][1][e];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += red[w];  // a fixed order
  const float inv = 1.f / sqrtf(tot / (float)n_hd + eps);
  float* o = q_out + (int64_t)t * n_hd;
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    const int i = 8 * ((int)threadIdx.x + 1024 * k);
    if (i >= n_hd) continue;
    f32x4 y0, y1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y0[e] = gq[k][0][e] * gk[k][0][e] * v[k][0][e] * inv;
      y1[e] = gq[k][1][e] * gk[k][1][e] * v[k][1][e] * inv;
    }
    *(f32x4*)(o + i) = y0;
    *(f32x4*)(o + i + 4) = y1;
  }
}

// The same with 8 consecutive entries per thread and load (n_hd a multiple
// of 8, every pointer 16-byte aligned): the sum of squares with four loads
// in flight per thread, then the scaled row from a second (cached) read.
template <typename TI>
__global__ __launch_bounds__(256) void qknorm_query_vec_kernel(const TI* __restrict__ q_nope,
                                                               const float* __restrict__ g_q,
                                                               const float* __restrict__ g_k, int n_hd, float eps,
                                                               float* __restrict__ q_out) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const TI* q = q_nope + (int64_t)t * n_hd;
  auto load8 = [&](int i, f32x4& a, f32x4& b) {
    if constexpr (sizeof(TI) == 4) {
      a = *(const f32x4*)(q + i);
      b = *(const f32x4*)(q + i + 4);
    } else {
      const bf16x8 v = *(const bf16x8*)(q + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = (float)v[e];
        b[e] = (float)v[4 + e];
      }
    }
  };
  float ss = 0.f;
#pragma unroll 4
  for (int i = 8 * (int)threadIdx.x; i < n_hd; i += 8 * 256) {
    f32x4 a, b;
    load8(i, a, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += a[e] * a[e] + b[e] * b[e];
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.f / sqrtf(tot / (float)n_hd + eps);
  float* o = q_out + (int64_t)t * n_hd;
#pragma unroll 2
  for (int i = 8 * (int)threadIdx.x; i < n_hd; i += 8 * 256) {
    f32x4 a, b;
    load8(i, a, b);
    const f32x4 gq0 = *(const f32x4*)(g_q + i), gq1 = *(const f32x4*)(g_q + i + 4);
    const f32x4 gk0 = *(const f32x4*)(g_k + i), gk1 = *(const f32x4*)(g_k + i + 4);
    f32x4 y0, y1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y0[e] = gq0[e] * gk0[e] * a[e] * inv;
      y1[e] = gq1[e] * gk1[e] * b[e] * inv;
    }
    *(f32x4*)(o + i) = y0;
    *(f32x4*)(o + i + 4) = y1;
  }
}

template <typename TW>
__global__ __launch_bounds__(256) void qknorm_gram_kernel(const TW* __restrict__ w_uk, int n_hd, int d_c,
                                                          float* __restrict__ gram) {
  const int a = blockIdx.x;
  for (int b = threadIdx.x; b < d_c; b += 256) {
    float acc = 0.f;
    for (int r = 0; r < n_hd; ++r) acc += load_f(w_uk + (int64_t)r * d_c + a) * load_f(w_uk + (int64_t)r * d_c + b);
    gram[(int64_t)a * d_c + b] = acc;
  }
}

template <typename TI>
__global__ __launch_bounds__(256) void qknorm_rinv_kernel(const TI* __restrict__ rows, int64_t n_rows, int row_width,
                                                          const float* __restrict__ gram, int d_c, int n_hd, float eps,
                                                          float* __restrict__ rinv) {
  constexpr int R = 16;  // rows per block
  __shared__ float cs[R][512];
  __shared__ float part[4][R];
  for (int64_t r0 = (int64_t)blockIdx.x * R; r0 < n_rows; r0 += (int64_t)gridDim.x * R) {  // grid-stride
    __syncthreads();  // the previous rows' LDS reads are done
    for (int i = threadIdx.x; i < R * d_c; i += 256) {
      const int rr = i / d_c, k = i % d_c;
      cs[rr][k] = r0 + rr < n_rows ? load_f(rows + (r0 + rr) * row_width + k) : 0.f;
    }
    __syncthreads();
    float q[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) q[rr] = 0.f;
    for (int j = threadIdx.x; j < d_c; j += 256) {
      float y[R];
#pragma unroll
      for (int rr = 0; rr < R; ++rr) y[rr] = 0.f;
      for (int k = 0; k < d_c; ++k) {
        const float gkj = gram[(int64_t)k * d_c + j];  // = G[j][k]
#pragma unroll
        for (int rr = 0; rr < R; ++rr) y[rr] += gkj * cs[rr][k];
      }
#pragma unroll
      for (int rr = 0; rr < R; ++rr) q[rr] += cs[rr][j] * y[rr];
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const float v = wave_sum(q[rr]);
      if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6][rr] = v;
    }
    __syncthreads();
    if (threadIdx.x < R && r0 + threadIdx.x < n_rows) {
      const int rr = threadIdx.x;
      const float tot = (part[0][rr] + part[1][rr]) + (part[2][rr] + part[3][rr]);
      rinv[r0 + rr] = 1.f / sqrtf(tot / (float)n_hd + eps);
    }
  }  // r0
}

hipError_t launch_qknorm_query(const void* q_nope, bool in_bf16, const float* g_q, const float* g_k, int n_tok,
                               int n_heads, int d_nope, float eps, float* q_out, hipStream_t stream) {
  const int n_hd = n_heads * d_nope;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (n_hd % 8 == 0 && n_hd <= 8 * 1024 * 2 && al16(q_nope) && al16(g_q) && al16(g_k) && al16(q_out)) {
    if (in_bf16)
      return launch(qknorm_query_reg_kernel<bf16>, dim3(n_tok), dim3(1024), stream, (const bf16*)q_nope, g_q, g_k,
                    n_hd, eps, q_out);
    return launch(qknorm_query_reg_kernel<float>, dim3(n_tok), dim3(1024), stream, (const float*)q_nope, g_q, g_k,
                  n_hd, eps, q_out);
  }
  if (n_hd % 8 == 0 && al16(q_nope) && al16(g_q) && al16(g_k) && al16(q_out)) {
    if (in_bf16)
      return launch(qknorm_query_vec_kernel<bf16>, dim3(n_tok), dim3(256), stream, (const bf16*)q_nope, g_q, g_k,
                    n_hd, eps, q_out);
    return launch(qknorm_query_vec_kernel<float>, dim3(n_tok), dim3(256), stream, (const float*)q_nope, g_q, g_k,
                  n_hd, eps, q_out);
  }
  if (in_bf16)
    return launch(qknorm_query_kernel<bf16>, dim3(n_tok), dim3(256), stream, (const bf16*)q_nope, g_q, g_k, n_hd, eps,
                  q_out);
  return launch(qknorm_query_kernel<float>, dim3(n_tok), dim3(256), stream, (const float*)q_nope, g_q, g_k, n_hd, eps,
                q_out);
}

hipError_t launch_qknorm_key_gram(const void* w_uk, bool w_bf16, int n_heads, int d_nope, int d_c, float* gram,
                                  hipStream_t stream) {
  if (w_bf16)
    return launch(qknorm_gram_kernel<bf16>, dim3(d_c), dim3(256), stream, (const bf16*)w_uk, n_heads * d_nope, d_c,
                  gram);
  return launch(qknorm_gram_kernel<float>, dim3(d_c), dim3(256), stream, (const float*)w_uk, n_heads * d_nope, d_c,
                gram);
}

hipError_t launch_qknorm_key_rinv(const void* rows, bool row_bf16, int64_t n_rows, int row_width, const float* gram,
                                  int d_c, int n_hd, float eps, float* rinv, hipStream_t stream) {
  const dim3 grid((unsigned)std::min<int64_t>((n_rows + 15) / 16, kMaxStrideBlocks));
  if (row_bf16)
    return launch(qknorm_rinv_kernel<bf16>, grid, dim3(256), stream, (const bf16*)rows, n_rows, row_width, gram, d_c,
                  n_hd, eps, rinv);
  return launch(qknorm_rinv_kernel<float>, grid, dim3(256), stream, (const float*)rows, n_rows, row_width, gram, d_c,
                n_hd, eps, rinv);
}

// ---------------------------------------------------------------------------
// Generic fp32 decode: one wave per (query row, split); split j of request b
// covers rows [j*L, min((j+1)*L, T_b)) with L = ceil(T_b / n_split).  Scores
// in fp32 against the stored latent and rotary key (absorbed form), online
// softmax, latent accumulation; writes the normalised partial and its lse.
// ---------------------------------------------------------------------------
constexpr int kF32MaxDc = 512;
constexpr int kF32MaxDr = 128;

// Index of stored row t of request b in the cache's row order (the page
// must be valid: f32_row returned non-null).
__device__ __forceinline__ int64_t f32_row_index(const SegArgs& s, int b, int t) {
  if (!s.block_table) return (int64_t)b * s.max_rows + t;
  return (int64_t)s.block_table[(int64_t)b * s.max_pages + t / s.page_size] * s.page_size + t % s.page_size;
}

__device__ __forceinline__ const float* f32_row(const SegArgs& s, int b, int t, int rw) {
  if (!s.block_table) return (const float*)s.cache + ((int64_t)b * s.max_rows + t) * rw;
  const int page = s.block_table[(int64_t)b * s.max_pages + t / s.page_size];
  if (page < 0 || page >= s.n_pages) return nullptr;
  return (const float*)s.cache + ((int64_t)page * s.page_size + t % s.page_size) * rw;
}

__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  __shared__ float qs[kF32MaxDc + kF32MaxDr];
  __shared__ float ps[64];
  const SegArgs& sg = a.seg;
  const int lane = threadIdx.x;
  const int split = blockIdx.x;
  const int row = blockIdx.y;  // over batch * s_q * head_count
  const int hc = sg.head_count;
  const int b = row / (a.s_q * hc);
  const int rem = row % (a.s_q * hc);
  const int s = rem / hc;
  const int h = sg.head_begin + rem % hc;
  const int tok = b * a.s_q + s;
  const int d_c = a.d_c, d_r = a.d_rope, rw = d_c + d_r;
  int64_t cap = sg.block_table ? (int64_t)sg.max_pages * sg.page_size : sg.max_rows;
  int T = sg.seq_lens[b];
  T = (int)max((int64_t)0, min((int64_t)T, cap));
  int vis = sg.causal ? T - a.s_q + s + 1 : T;
  vis = max(0, min(vis, T));
  const int L = (T + sg.n_split - 1) / sg.n_split;
  const int r0 = split * L;
  const int r1 = min(r0 + L, T);
  const int64_t out_row = ((int64_t)tok * a.n_heads + h) * a.n_part + sg.part_begin + split;

  const float* ql = (const float*)a.q_lat + ((int64_t)tok * a.n_heads + h) * d_c;
  const float* qr = (const float*)sg.q_rot + ((int64_t)tok * a.n_heads + h) * d_r;
  for (int d = lane; d < d_c; d += 64) qs[d] = ql[d];
  for (int d = lane; d < d_r; d += 64) qs[d_c + d] = qr[d];
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[kF32MaxDc / 64];
#pragma unroll
  for (int k = 0; k < kF32MaxDc / 64; ++k) acc[k] = 0.f;
  const int rend = min(r1, vis);
  for (int t0 = r0; t0 < rend; t0 += 64) {
    const int t = t0 + lane;
    float sc = -INFINITY;
    if (t < rend) {
      const float* rp = f32_row(sg, b, t, rw);
      if (rp) {
        float dot = 0.f, dot_r = 0.f;
        for (int d = 0; d < d_c; ++d) dot += qs[d] * rp[d];
        for (int d = d_c; d < rw; ++d) dot_r += qs[d] * rp[d];
        if (sg.row_rinv) dot *= sg.row_rinv[f32_row_index(sg, b, t)];
        sc = (dot + dot_r) * a.scale;
      }
    }
    const float mt = wave_max(sc);
    if (mt == -INFINITY) continue;  // nothing visible in this tile
    const float mn = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float p = (sc == -INFINITY) ? 0.f : expf(sc - mn);
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int k = 0; k < kF32MaxDc / 64; ++k) acc[k] *= alpha;
    ps[lane] = p;
    __syncthreads();
    const int nt = min(64, rend - t0);
    for (int jj = 0; jj < nt; ++jj) {
      const float pj = ps[jj];
      if (pj == 0.f) continue;
      const float* rp = f32_row(sg, b, t0 + jj, rw);
#pragma unroll
      for (int k = 0; k < kF32MaxDc / 64; ++k) {
        const int d = lane + 64 * k;
        if (d < d_c) acc[k] += pj * rp[d];
      }
    }
    __syncthreads();
    m = mn;
  }
  if (l > 0.f) {
    const float inv = 1.f / l;
    float* o = (float*)a.o_part + out_row * d_c;  // fp32 partials only on this path
#pragma unroll
    for (int k = 0; k < kF32MaxDc / 64; ++k) {
      const int d = lane + 64 * k;
      if (d < d_c) o[d] = acc[k] * inv;
    }
    if (lane == 0) a.lse_part[out_row] = m + logf(l);
  } else if (lane == 0) {
    a.lse_part[out_row] = -INFINITY;
  }
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.seg.n_split, a.batch * a.s_q * a.seg.head_count);
  return launch(decode_f32_kernel, grid, dim3(64), stream, a);
}

}  // namespace mla
