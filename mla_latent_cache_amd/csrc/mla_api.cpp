// C ABI of the MLA decode library: argument validation, then launches on the
// caller's stream.  Declarations and contracts: include/mla_latent.h.
#include "../../include/mla_latent.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

#include "mla_kernels.h"

namespace {

thread_local char g_err[512] = "";

mla_status fail(mla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

mla_status ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

mla_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int dt) { return dt == MLA_F32 || dt == MLA_BF16; }
// q_lat storage of the fused query kernel: 0 fp32, 1 bf16, 2 bf16 hi and lo planes
int lat_mode(int dt) { return dt == MLA_BF16X2 ? 2 : dt == MLA_BF16 ? 1 : 0; }

int cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

constexpr int kBf16Dc = 512;
// Query rows (s_q * head_count) of one bf16 segment: 64 row groups of 64.
constexpr int kBf16MaxRows = 4096;
constexpr int kBf16Dr = 64;
constexpr int kPage = 64;
// Split slots per request and segment on the bf16 path (a piece packs its
// slot into 16 bits).
constexpr int kMaxSplit = 32767;
// Query tokens per call of the query-side and output-side calls: their index
// arithmetic (tokens x rotary pairs x segment shifts) stays within 32 bits.
constexpr int kMaxTok = 1 << 20;

}  // namespace

extern "C" {

const char* mla_status_string(int st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer";
    case MLA_ERR_SHAPE: return "bad shape";
    case MLA_ERR_DTYPE: return "bad dtype";
    case MLA_ERR_ALIGN: return "misaligned pointer";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mla_last_error(void) { return g_err; }

int mla_version(void) { return 100; }

int mla_device_cu_count(void) { return cu_count(); }

int mla_decode_shares(int s_q, int head_count, int n_wg) {
  if (s_q <= 0 || head_count <= 0 || n_wg < 0 || (int64_t)s_q * head_count > kBf16MaxRows) return 0;
  const int wg = n_wg > 0 ? n_wg : cu_count();
  if (wg <= 0) return 0;
  int n_share = 0, n_rg = 0;
  mla::decode_bf16_grid(s_q * head_count, mla::decode_bf16_tile(s_q * head_count), wg, &n_share, &n_rg);
  return n_share;
}

mla_status rope_relocate_q(const void* q_pe, int in_dtype, void* q_rot, int out_dtype, const int64_t* pos,
                           const int64_t* shift, int n_tok, int n_heads, int d_rope, double base,
                           void* stream) {
  if (!q_pe || !q_rot || !pos) return fail(MLA_ERR_NULL, "rope_relocate_q: q_pe, q_rot and pos are required");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(MLA_ERR_DTYPE, "rope_relocate_q: dtypes %d, %d", in_dtype, out_dtype);
  if (n_tok < 0 || n_tok > kMaxTok || n_heads <= 0 || n_heads > 65535 || d_rope < 2 || d_rope > 128 || (d_rope & 1))
    return fail(MLA_ERR_SHAPE, "rope_relocate_q: n_tok=%d (<= %d) n_heads=%d d_rope=%d", n_tok, kMaxTok, n_heads,
                d_rope);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(MLA_ERR_SHAPE, "rope_relocate_q: base=%g", base);
  if (n_tok == 0) return ok();
  return hip_status(mla::launch_rope(q_pe, in_dtype == MLA_BF16, q_rot, out_dtype == MLA_BF16, pos, shift,
                                     n_tok, n_heads, d_rope, base, (hipStream_t)stream),
                    "rope_relocate_q launch");
}

mla_status mla_absorb_q(const void* q_nope, const void* w_uk, int in_dtype, void* q_lat, int out_dtype,
                        int n_tok, int n_heads, int d_nope, int d_c, void* stream) {
  if (!q_nope || !w_uk || !q_lat) return fail(MLA_ERR_NULL, "mla_absorb_q: null pointer");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(MLA_ERR_DTYPE, "mla_absorb_q: dtypes %d, %d", in_dtype, out_dtype);
  if (n_tok < 0 || n_tok > kMaxTok || n_heads <= 0 || d_nope <= 0 || d_nope > 256 || d_c <= 0 || d_c > 4096 ||
      n_heads > 65535)
    return fail(MLA_ERR_SHAPE, "mla_absorb_q: n_tok=%d (<= %d) n_heads=%d d_nope=%d d_c=%d", n_tok, kMaxTok, n_heads,
                d_nope, d_c);
  if (n_tok == 0) return ok();
  return hip_status(mla::launch_absorb(q_nope, w_uk, in_dtype == MLA_BF16, q_lat, out_dtype == MLA_BF16, n_tok,
                                       n_heads, d_nope, d_c, (hipStream_t)stream),
                    "mla_absorb_q launch");
}

mla_status mla_prepare_q(const void* q_nope, int q_dtype, const void* q_pe, const void* w_uk, int in_dtype,
                         void* q_lat, int lat_dtype, void* const* q_rots, const int64_t* const* shifts, int n_shift,
                         int rot_dtype, const int64_t* pos, int n_tok, int n_heads, int d_nope, int d_rope, int d_c,
                         double base, void* stream) {
  if (!q_nope || !q_pe || !w_uk || !q_lat || !pos || (n_shift > 0 && !q_rots))
    return fail(MLA_ERR_NULL, "mla_prepare_q: null pointer");
  if (!dtype_ok(q_dtype) || !dtype_ok(in_dtype) || !(dtype_ok(lat_dtype) || lat_dtype == MLA_BF16X2) ||
      !dtype_ok(rot_dtype))
    return fail(MLA_ERR_DTYPE, "mla_prepare_q: dtypes %d, %d, %d, %d", q_dtype, in_dtype, lat_dtype, rot_dtype);
  if (n_shift < 0 || n_shift > mla::kMaxShift)
    return fail(MLA_ERR_SHAPE, "mla_prepare_q: n_shift=%d (0..%d)", n_shift, mla::kMaxShift);
  for (int k = 0; k < n_shift; ++k)
    if (!q_rots[k]) return fail(MLA_ERR_NULL, "mla_prepare_q: q_rots[%d] is NULL", k);
  if (n_tok < 0 || n_tok > kMaxTok || n_heads <= 0 || n_heads > 65535 || d_nope <= 0 || d_nope > 256 || d_c <= 0 ||
      d_c > 4096 || d_rope < 2 || d_rope > 128 || (d_rope & 1))
    return fail(MLA_ERR_SHAPE, "mla_prepare_q: n_tok=%d (<= %d) n_heads=%d d_nope=%d d_rope=%d d_c=%d", n_tok,
                kMaxTok, n_heads, d_nope, d_rope, d_c);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(MLA_ERR_SHAPE, "mla_prepare_q: base=%g", base);
  const bool mfma = in_dtype == MLA_BF16 && mla::absorb_mfma_ok(q_nope, w_uk, q_lat, d_nope, d_c);
  if (q_dtype != in_dtype && !(q_dtype == MLA_F32 && mfma))
    return fail(MLA_ERR_UNSUPPORTED, "mla_prepare_q: an fp32 query with bf16 weights needs d_nope=128, d_c=512 "
                "and 16-byte aligned q_nope, w_uk and q_lat");
  if (lat_dtype == MLA_BF16X2 && !mfma)
    return fail(MLA_ERR_UNSUPPORTED, "mla_prepare_q: a split q_lat (MLA_BF16X2) needs bf16 weights, d_nope=128, "
                "d_c=512 and 16-byte aligned q_nope, w_uk and q_lat");
  if (n_tok == 0) return ok();
  const hipStream_t st = (hipStream_t)stream;
  if (mfma) {
    mla::RopeTargets rt{};
    rt.n = n_shift;
    for (int k = 0; k < n_shift; ++k) {
      rt.q_rot[k] = q_rots[k];
      rt.shift[k] = shifts ? shifts[k] : nullptr;
    }
    return hip_status(mla::launch_prepare_mfma(q_nope, q_dtype == MLA_F32, w_uk, q_lat, lat_mode(lat_dtype), q_pe,
                                               pos, rt, rot_dtype == MLA_BF16, n_tok, n_heads, d_rope, base,
                                               mla::QkArgs{}, st),
                      "mla_prepare_q launch");
  }
  // other shapes and dtypes: the two kernels one after the other
  for (int k = 0; k < n_shift; ++k) {
    const mla_status r = hip_status(mla::launch_rope(q_pe, in_dtype == MLA_BF16, q_rots[k], rot_dtype == MLA_BF16,
                                                     pos, shifts ? shifts[k] : nullptr, n_tok, n_heads, d_rope,
                                                     base, st),
                                    "mla_prepare_q rope launch");
    if (r != MLA_OK) return r;
  }
  return hip_status(mla::launch_absorb(q_nope, w_uk, in_dtype == MLA_BF16, q_lat, lat_dtype == MLA_BF16, n_tok,
                                       n_heads, d_nope, d_c, st),
                    "mla_prepare_q absorb launch");
}

mla_status mla_prepare_q_qknorm(const void* q_nope, int q_dtype, const float* g_q, const float* g_k, float eps,
                                const void* q_pe, const void* w_uk, int in_dtype, void* q_lat, int lat_dtype,
                                void* const* q_rots, const int64_t* const* shifts, int n_shift, int rot_dtype,
                                const int64_t* pos, int n_tok, int n_heads, int d_nope, int d_rope, int d_c,
                                double base, void* stream) {
  if (!q_nope || !g_q || !g_k || !q_pe || !w_uk || !q_lat || !pos || (n_shift > 0 && !q_rots))
    return fail(MLA_ERR_NULL, "mla_prepare_q_qknorm: null pointer");
  if (!dtype_ok(q_dtype) || !dtype_ok(in_dtype) || !(dtype_ok(lat_dtype) || lat_dtype == MLA_BF16X2) ||
      !dtype_ok(rot_dtype))
    return fail(MLA_ERR_DTYPE, "mla_prepare_q_qknorm: dtypes %d, %d, %d, %d", q_dtype, in_dtype, lat_dtype,
                rot_dtype);
  if (n_shift < 0 || n_shift > mla::kMaxShift)
    return fail(MLA_ERR_SHAPE, "mla_prepare_q_qknorm: n_shift=%d (0..%d)", n_shift, mla::kMaxShift);
  for (int k = 0; k < n_shift; ++k)
    if (!q_rots[k]) return fail(MLA_ERR_NULL, "mla_prepare_q_qknorm: q_rots[%d] is NULL", k);
  if (n_tok < 0 || n_tok > kMaxTok || n_heads <= 0 || n_heads > 65535 || d_rope < 2 || d_rope > 128 || (d_rope & 1))
    return fail(MLA_ERR_SHAPE, "mla_prepare_q_qknorm: n_tok=%d n_heads=%d d_rope=%d", n_tok, n_heads, d_rope);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(MLA_ERR_SHAPE, "mla_prepare_q_qknorm: base=%g", base);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MLA_ERR_SHAPE, "mla_prepare_q_qknorm: eps=%g", (double)eps);
  if (in_dtype != MLA_BF16 || !mla::absorb_mfma_ok(q_nope, w_uk, q_lat, d_nope, d_c))
    return fail(MLA_ERR_UNSUPPORTED, "mla_prepare_q_qknorm: needs bf16 w_uk and q_pe, d_nope=128, d_c=512 and "
                "16-byte aligned q_nope, w_uk and q_lat");
  if ((int64_t)n_tok * n_heads > mla::kQkFusedRows)
    return fail(MLA_ERR_UNSUPPORTED, "mla_prepare_q_qknorm: n_tok * n_heads = %lld (at most %d; use "
                "mla_qknorm_query, then mla_prepare_q)", (long long)n_tok * n_heads, mla::kQkFusedRows);
  if (n_tok == 0) return ok();
  mla::RopeTargets rt{};
  rt.n = n_shift;
  for (int k = 0; k < n_shift; ++k) {
    rt.q_rot[k] = q_rots[k];
    rt.shift[k] = shifts ? shifts[k] : nullptr;
  }
  mla::QkArgs qk;
  qk.g_q = g_q;
  qk.g_k = g_k;
  qk.eps = eps;
  return hip_status(mla::launch_prepare_mfma(q_nope, q_dtype == MLA_F32, w_uk, q_lat, lat_mode(lat_dtype), q_pe,
                                             pos, rt, rot_dtype == MLA_BF16, n_tok, n_heads, d_rope, base, qk,
                                             (hipStream_t)stream),
                    "mla_prepare_q_qknorm launch");
}

mla_status mla_out_uv(const void* o_lat, int o_dtype, const void* w_uv, int w_dtype, void* out, int out_dtype,
                      int n_tok, int n_heads, int d_c, int d_v, void* stream) {
  if (!o_lat || !w_uv || !out) return fail(MLA_ERR_NULL, "mla_out_uv: null pointer");
  if (!dtype_ok(o_dtype) || !dtype_ok(w_dtype) || !dtype_ok(out_dtype))
    return fail(MLA_ERR_DTYPE, "mla_out_uv: dtypes %d, %d, %d", o_dtype, w_dtype, out_dtype);
  if (n_tok < 0 || n_tok > kMaxTok || n_heads <= 0 || n_heads > 65535 || d_c <= 0 || d_c > 1024 || d_v <= 0 ||
      d_v > 4 * 65535)
    return fail(MLA_ERR_SHAPE, "mla_out_uv: n_tok=%d (<= %d) n_heads=%d d_c=%d d_v=%d", n_tok, kMaxTok, n_heads, d_c,
                d_v);
  if (n_tok == 0) return ok();
  return hip_status(mla::launch_out_uv(o_lat, o_dtype == MLA_BF16, w_uv, w_dtype == MLA_BF16, out,
                                       out_dtype == MLA_BF16, n_tok, n_heads, d_c, d_v, (hipStream_t)stream),
                    "mla_out_uv launch");
}

mla_status mla_out_proj(const void* x, int x_dtype, const void* w_o, int w_dtype, void* out, int out_dtype,
                        int n_tok, int k_in, int d_model, void* stream) {
  if (!x || !w_o || !out) return fail(MLA_ERR_NULL, "mla_out_proj: null pointer");
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype) || !dtype_ok(out_dtype))
    return fail(MLA_ERR_DTYPE, "mla_out_proj: dtypes %d, %d, %d", x_dtype, w_dtype, out_dtype);
  if (n_tok < 0 || n_tok > kMaxTok || k_in <= 0 || k_in > (1 << 20) || d_model <= 0 || d_model > (1 << 20))
    return fail(MLA_ERR_SHAPE, "mla_out_proj: n_tok=%d (<= %d) k_in=%d d_model=%d (each <= 2^20)", n_tok, kMaxTok,
                k_in, d_model);
  if (n_tok == 0) return ok();
  return hip_status(mla::launch_out_proj(x, x_dtype == MLA_BF16, w_o, w_dtype == MLA_BF16, out,
                                         out_dtype == MLA_BF16, n_tok, k_in, d_model, (hipStream_t)stream),
                    "mla_out_proj launch");
}

mla_status mla_combine_lse(const void* o_part, int part_dtype, const float* lse_part, int n_rows, int n_part,
                           int d_c, void* o_lat, int out_dtype, float* lse, void* stream) {
  if (!o_part || !lse_part || !o_lat) return fail(MLA_ERR_NULL, "mla_combine_lse: null pointer");
  if (!dtype_ok(out_dtype) || !dtype_ok(part_dtype))
    return fail(MLA_ERR_DTYPE, "mla_combine_lse: dtypes %d, %d", part_dtype, out_dtype);
  if (n_rows < 0 || n_rows >= (1 << 24) || n_part <= 0 || n_part > 1024 || d_c <= 0 || d_c > 4096 || (d_c & 3) ||
      ((reinterpret_cast<uintptr_t>(o_part) & 15u) != 0))
    return fail(MLA_ERR_SHAPE, "mla_combine_lse: n_rows=%d n_part=%d (<= 1024) d_c=%d (multiple of 4, "
                "o_part 16-byte aligned)", n_rows, n_part, d_c);
  if (n_rows == 0) return ok();
  return hip_status(mla::launch_combine(o_part, part_dtype == MLA_BF16, lse_part, n_rows, n_part, d_c, o_lat,
                                        out_dtype == MLA_BF16,
                                        lse, (hipStream_t)stream),
                    "mla_combine_lse launch");
}

mla_status mla_combine_out_uv(const void* o_part, int part_dtype, const float* lse_part, int n_tok, int n_heads,
                              int n_part, int d_c, const void* w_uv, int w_dtype, int d_v, void* o_lat, float* lse,
                              void* out, int out_dtype, void* stream) {
  if (!o_part || !lse_part || !w_uv || !out) return fail(MLA_ERR_NULL, "mla_combine_out_uv: null pointer");
  if (!dtype_ok(w_dtype) || !dtype_ok(out_dtype) || !dtype_ok(part_dtype))
    return fail(MLA_ERR_DTYPE, "mla_combine_out_uv: dtypes %d, %d, %d", part_dtype, w_dtype, out_dtype);
  if (n_tok < 0 || n_tok > 65535 || n_heads <= 0 || n_heads > 65535 || (int64_t)n_tok * n_heads > (1 << 21) ||
      n_part <= 0 || n_part > 1024 || d_c <= 0 || d_c > 512 || (d_c & 3) || d_v <= 0 || d_v > 128 ||
      ((reinterpret_cast<uintptr_t>(o_part) & 15u) != 0))
    return fail(MLA_ERR_SHAPE, "mla_combine_out_uv: n_tok=%d n_heads=%d (rows <= 2^21) n_part=%d (<= 1024) d_c=%d "
                "(multiple of 4, <= 512) d_v=%d (<= 128), o_part 16-byte aligned", n_tok, n_heads, n_part, d_c, d_v);
  if (n_tok == 0) return ok();
  return hip_status(mla::launch_combine_out_uv(o_part, part_dtype == MLA_BF16, lse_part, n_tok, n_heads, n_part,
                                               d_c, w_uv,
                                               w_dtype == MLA_BF16, d_v, o_lat, lse, out, out_dtype == MLA_BF16,
                                               (hipStream_t)stream),
                    "mla_combine_out_uv launch");
}

mla_status mla_quantize_latent_i8(const void* rows, int row_dtype, int64_t n_rows, int d_c, int d_rope,
                                  void* out_rows, float* scales, void* stream) {
  if (!rows || !out_rows || !scales) return fail(MLA_ERR_NULL, "mla_quantize_latent_i8: null pointer");
  if (row_dtype != MLA_BF16) return fail(MLA_ERR_DTYPE, "mla_quantize_latent_i8: rows must be bf16 (got %d)", row_dtype);
  if (n_rows < 0 || n_rows > ((int64_t)1 << 32) || d_c <= 0 || d_c > 512 || (d_c & 7) || d_rope < 0 ||
      d_rope > 128 || (d_rope & 3))
    return fail(MLA_ERR_SHAPE, "mla_quantize_latent_i8: n_rows=%lld d_c=%d (multiple of 8, <= 512) d_rope=%d "
                "(multiple of 4, <= 128)", (long long)n_rows, d_c, d_rope);
  if ((reinterpret_cast<uintptr_t>(out_rows) & 7u) != 0 || (reinterpret_cast<uintptr_t>(rows) & 7u) != 0)
    return fail(MLA_ERR_ALIGN, "mla_quantize_latent_i8: rows and out_rows must be 8-byte aligned");
  if (n_rows == 0) return ok();
  return hip_status(mla::launch_quantize_latent_i8(rows, n_rows, d_c, d_rope, out_rows, scales, (hipStream_t)stream),
                    "mla_quantize_latent_i8 launch");
}

mla_status mla_quantize_latent_i4(const void* rows, int row_dtype, int64_t n_rows, int d_c, int d_rope,
                                  void* out_rows, float* scales, void* stream) {
  if (!rows || !out_rows || !scales) return fail(MLA_ERR_NULL, "mla_quantize_latent_i4: null pointer");
  if (row_dtype != MLA_BF16) return fail(MLA_ERR_DTYPE, "mla_quantize_latent_i4: rows must be bf16 (got %d)", row_dtype);
  if (n_rows < 0 || n_rows > ((int64_t)1 << 32) || d_c <= 0 || d_c > 512 || (d_c & 7) || d_rope <= 0 ||
      d_rope > 128 || (d_rope & 7))
    return fail(MLA_ERR_SHAPE, "mla_quantize_latent_i4: n_rows=%lld d_c=%d (multiple of 8, <= 512) d_rope=%d "
                "(multiple of 8, <= 128)", (long long)n_rows, d_c, d_rope);
  if ((reinterpret_cast<uintptr_t>(out_rows) & 3u) != 0 || (reinterpret_cast<uintptr_t>(scales) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(rows) & 1u) != 0)
    return fail(MLA_ERR_ALIGN, "mla_quantize_latent_i4: out_rows 4-byte, scales 8-byte, rows 2-byte aligned");
  if (n_rows == 0) return ok();
  return hip_status(mla::launch_quantize_latent_i4(rows, n_rows, d_c, d_rope, out_rows, scales, (hipStream_t)stream),
                    "mla_quantize_latent_i4 launch");
}

mla_status mla_qknorm_query(const void* q_nope, int in_dtype, const float* g_q, const float* g_k, int n_tok,
                            int n_heads, int d_nope, double eps, float* q_out, void* stream) {
  if (!q_nope || !g_q || !g_k || !q_out) return fail(MLA_ERR_NULL, "mla_qknorm_query: null pointer");
  if (!dtype_ok(in_dtype)) return fail(MLA_ERR_DTYPE, "mla_qknorm_query: in_dtype %d", in_dtype);
  if (n_tok < 0 || n_tok > 65535 * 32 || n_heads <= 0 || d_nope <= 0 || (int64_t)n_heads * d_nope > (1 << 24) ||
      !(eps >= 0.0) || !std::isfinite(eps))
    return fail(MLA_ERR_SHAPE, "mla_qknorm_query: n_tok=%d n_heads=%d d_nope=%d eps=%g", n_tok, n_heads, d_nope, eps);
  if (n_tok == 0) return ok();
  return hip_status(mla::launch_qknorm_query(q_nope, in_dtype == MLA_BF16, g_q, g_k, n_tok, n_heads, d_nope,
                                             (float)eps, q_out, (hipStream_t)stream),
                    "mla_qknorm_query launch");
}

mla_status mla_qknorm_key_gram(const void* w_uk, int w_dtype, int n_heads, int d_nope, int d_c, float* gram,
                               void* stream) {
  if (!w_uk || !gram) return fail(MLA_ERR_NULL, "mla_qknorm_key_gram: null pointer");
  if (!dtype_ok(w_dtype)) return fail(MLA_ERR_DTYPE, "mla_qknorm_key_gram: w_dtype %d", w_dtype);
  if (n_heads <= 0 || d_nope <= 0 || (int64_t)n_heads * d_nope > (1 << 24) || d_c <= 0 || d_c > 512)
    return fail(MLA_ERR_SHAPE, "mla_qknorm_key_gram: n_heads=%d d_nope=%d d_c=%d (<= 512)", n_heads, d_nope, d_c);
  return hip_status(mla::launch_qknorm_key_gram(w_uk, w_dtype == MLA_BF16, n_heads, d_nope, d_c, gram,
                                                (hipStream_t)stream),
                    "mla_qknorm_key_gram launch");
}

mla_status mla_qknorm_key_rinv(const void* rows, int row_dtype, int64_t n_rows, int row_width, const float* gram,
                               int d_c, int n_heads, int d_nope, double eps, float* rinv, void* stream) {
  if (!rows || !gram || !rinv) return fail(MLA_ERR_NULL, "mla_qknorm_key_rinv: null pointer");
  if (!dtype_ok(row_dtype)) return fail(MLA_ERR_DTYPE, "mla_qknorm_key_rinv: row_dtype %d", row_dtype);
  if (n_rows < 0 || n_rows > ((int64_t)1 << 34) || d_c <= 0 || d_c > 512 || row_width < d_c || n_heads <= 0 ||
      d_nope <= 0 || !(eps >= 0.0) || !std::isfinite(eps))
    return fail(MLA_ERR_SHAPE, "mla_qknorm_key_rinv: n_rows=%lld row_width=%d d_c=%d (<= 512) n_heads=%d "
                "d_nope=%d eps=%g", (long long)n_rows, row_width, d_c, n_heads, d_nope, eps);
  if (n_rows == 0) return ok();
  return hip_status(mla::launch_qknorm_key_rinv(rows, row_dtype == MLA_BF16, n_rows, row_width, gram, d_c,
                                                n_heads * d_nope, (float)eps, rinv, (hipStream_t)stream),
                    "mla_qknorm_key_rinv launch");
}

mla_status mla_decode_splitkv(const mla_segment* segs, int n_segs, const void* q_lat, int q_dtype,
                              int cache_dtype, int batch, int s_q, int n_heads, int d_c, int d_rope, float scale,
                              void* o_part, int part_dtype, float* lse_part, int n_part, int n_wg, void* stream) {
  if (!segs || !q_lat || !o_part || !lse_part) return fail(MLA_ERR_NULL, "mla_decode_splitkv: null pointer");
  if (!(dtype_ok(q_dtype) || q_dtype == MLA_BF16X2) ||
      !(dtype_ok(cache_dtype) || cache_dtype == MLA_I8 || cache_dtype == MLA_I4) || !dtype_ok(part_dtype))
    return fail(MLA_ERR_DTYPE, "mla_decode_splitkv: dtypes %d, %d, %d", q_dtype, cache_dtype, part_dtype);
  const bool qx2 = q_dtype == MLA_BF16X2;
  if (qx2 && cache_dtype != MLA_BF16 && cache_dtype != MLA_I8 && cache_dtype != MLA_I4)
    return fail(MLA_ERR_UNSUPPORTED,
                "mla_decode_splitkv: a split query (MLA_BF16X2) needs a bf16, int8 or int4 cache");
  if (cache_dtype == MLA_F32 && q_dtype != MLA_F32)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_splitkv: an fp32 cache needs an fp32 query");
  if (cache_dtype == MLA_F32 && part_dtype != MLA_F32)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_splitkv: an fp32 cache writes fp32 partials");
  if (n_segs <= 0 || n_segs > 64 || batch < 0 || s_q <= 0 || n_heads <= 0 || n_part <= 0 || n_wg < 0 || n_wg > 65536)
    return fail(MLA_ERR_SHAPE, "mla_decode_splitkv: n_segs=%d batch=%d s_q=%d n_heads=%d n_part=%d n_wg=%d",
                n_segs, batch, s_q, n_heads, n_part, n_wg);
  if (!std::isfinite(scale)) return fail(MLA_ERR_SHAPE, "mla_decode_splitkv: scale is not finite");
  const bool i8 = cache_dtype == MLA_I8, i4 = cache_dtype == MLA_I4;
  const bool lowbit = i8 || i4;
  const bool bf = cache_dtype == MLA_BF16 || lowbit;  // the MFMA kernels (16-bit, int8 or int4 rows)
  const bool q32 = q_dtype == MLA_F32;
  if (lowbit && !q32 && !qx2)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_splitkv: a low-bit cache needs an fp32 or split query");
  if (bf) {
    if (d_c != kBf16Dc || d_rope != kBf16Dr)
      return fail(MLA_ERR_UNSUPPORTED, "mla_decode_splitkv: bf16 path needs d_c=512, d_rope=64 (got %d, %d)", d_c,
                  d_rope);
    if (!aligned16(q_lat) || !aligned16(o_part))
      return fail(MLA_ERR_ALIGN, "mla_decode_splitkv: q_lat and o_part must be 16-byte aligned");
  } else if (d_c <= 0 || d_c > 512 || d_rope <= 0 || d_rope > 128) {
    return fail(MLA_ERR_SHAPE, "mla_decode_splitkv: fp32 path needs d_c<=512, d_rope<=128 (got %d, %d)", d_c,
                d_rope);
  }
  // every head's slot ranges must tile [0, n_part) exactly
  std::vector<int> cover((size_t)n_heads * n_part, 0);
  for (int g = 0; g < n_segs; ++g) {
    const mla_segment& s = segs[g];
    if (!s.cache || !s.seq_lens || !s.q_rot) return fail(MLA_ERR_NULL, "segment %d: cache, seq_lens, q_rot required", g);
    if (s.head_begin < 0 || s.head_count <= 0 || s.head_begin + s.head_count > n_heads)
      return fail(MLA_ERR_SHAPE, "segment %d: heads [%d, %d) outside [0, %d)", g, s.head_begin,
                  s.head_begin + s.head_count, n_heads);
    if (s.n_split <= 0 || s.part_begin < 0 || s.part_begin + s.n_split > n_part)
      return fail(MLA_ERR_SHAPE, "segment %d: slots [%d, %d) outside [0, %d)", g, s.part_begin,
                  s.part_begin + s.n_split, n_part);
    if (s.causal != 0 && s.causal != 1) return fail(MLA_ERR_SHAPE, "segment %d: causal must be 0 or 1", g);
    if (s.block_table) {
      if (s.page_size <= 0 || s.max_pages <= 0 || s.n_pages <= 0)
        return fail(MLA_ERR_SHAPE, "segment %d: paged layout needs page_size, max_pages, n_pages > 0", g);
      if (bf && s.page_size != kPage)
        return fail(MLA_ERR_UNSUPPORTED, "segment %d: bf16 path needs page_size 64 (got %d)", g, s.page_size);
    } else if (s.max_rows <= 0 && batch > 0) {
      return fail(MLA_ERR_SHAPE, "segment %d: contiguous layout needs max_rows > 0", g);
    }
    if (bf) {
      if (!aligned16(s.cache) || !aligned16(s.q_rot))
        return fail(MLA_ERR_ALIGN, "segment %d: cache and q_rot must be 16-byte aligned", g);
      if ((int64_t)s_q * s.head_count > kBf16MaxRows)
        return fail(MLA_ERR_UNSUPPORTED, "segment %d: s_q * head_count = %d > %d", g, s_q * s.head_count,
                    kBf16MaxRows);
      if (batch > 65535 || s.n_split > kMaxSplit)
        return fail(MLA_ERR_UNSUPPORTED, "segment %d: bf16 path needs batch <= 65535 and n_split <= %d", g,
                    kMaxSplit);
      // row counts of the device-side split plan are 32-bit: bound the rows a
      // segment can hold (2^30 rows of 1152 B is far beyond device memory)
      const int64_t cap = s.block_table ? (int64_t)s.max_pages * kPage : s.max_rows;
      if (cap > ((int64_t)1 << 30) || (int64_t)batch * cap > ((int64_t)1 << 30))
        return fail(MLA_ERR_UNSUPPORTED, "segment %d: batch * rows per request = %lld exceeds 2^30", g,
                    (long long)((int64_t)batch * cap));
      if (s.row_rinv && q_dtype == MLA_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "segment %d: QK-Norm (row_rinv) needs an fp32 or split query", g);
      if ((s.row_rinv != nullptr) != (segs[0].row_rinv != nullptr))
        return fail(MLA_ERR_UNSUPPORTED, "segment %d: row_rinv must be given for every segment or for none", g);
      if (lowbit && !s.row_scale) return fail(MLA_ERR_NULL, "segment %d: a low-bit cache needs row_scale", g);
      if (lowbit && s.row_rinv)
        return fail(MLA_ERR_UNSUPPORTED, "segment %d: QK-Norm with a low-bit cache is not supported", g);
      if (i4 && (reinterpret_cast<uintptr_t>(s.row_scale) & 7u) != 0)
        return fail(MLA_ERR_ALIGN, "segment %d: int4 row_scale must be 8-byte aligned", g);
    } else if ((int64_t)batch * s_q * s.head_count > 65535 || s.n_split > 65535) {
      return fail(MLA_ERR_UNSUPPORTED, "segment %d: fp32 path grid too large", g);
    }
    if (!lowbit && s.row_scale)
      return fail(MLA_ERR_UNSUPPORTED, "segment %d: row_scale is only read with a low-bit cache", g);
    for (int h = s.head_begin; h < s.head_begin + s.head_count; ++h)
      for (int k = s.part_begin; k < s.part_begin + s.n_split; ++k) cover[(size_t)h * n_part + k]++;
  }
  for (int h = 0; h < n_heads; ++h)
    for (int k = 0; k < n_part; ++k)
      if (cover[(size_t)h * n_part + k] != 1)
        return fail(MLA_ERR_SHAPE, "head %d slot %d is covered by %d segments (must be exactly 1)", h, k,
                    cover[(size_t)h * n_part + k]);
  if (batch == 0) return ok();
  int wg = n_wg > 0 ? n_wg : cu_count();
  if (wg <= 0) return fail(MLA_ERR_HIP, "mla_decode_splitkv: could not query the device");
  std::vector<mla::SegArgs> sa((size_t)n_segs);
  const bool rows_path = bf && q32 && !lowbit;  // fp32 query, 16-bit rows
  for (int g = 0; g < n_segs; ++g) {
    const mla_segment& s = segs[g];
    sa[g] = mla::SegArgs{s.cache,     s.block_table, s.seq_lens,  s.q_rot,      s.max_rows,
                         s.page_size, s.max_pages,   s.n_pages,   s.head_begin, s.head_count,
                         s.causal,    s.part_begin,  s.n_split,   s.row_rinv,   s.row_scale};
  }
  mla::DecodeArgs a{};
  a.q_lat = q_lat;
  a.o_part = o_part;
  a.part_bf16 = part_dtype == MLA_BF16;
  a.q_split = qx2;
  a.lse_part = lse_part;
  a.batch = batch;
  a.s_q = s_q;
  a.n_heads = n_heads;
  a.d_c = d_c;
  a.d_rope = d_rope;
  a.n_part = n_part;
  a.scale = scale;
  // several segments on the row-owning path (or a low-bit cache, or a split
  // query, which only that kernel reads): one launch over all of them, the
  // grid split by each segment's share of the work
  if (lowbit || qx2 || (rows_path && n_segs > 1))
    return hip_status(mla::launch_decode_rows_multi(a, sa.data(), n_segs, wg, i4 ? 1 : i8 ? 2 : 0,
                                                    (hipStream_t)stream),
                      "mla_decode_splitkv launch");
  for (int g = 0; g < n_segs; ++g) {
    a.seg = sa[g];
    hipError_t e = bf ? mla::launch_decode_bf16(a, wg, q32, (hipStream_t)stream)
                      : mla::launch_decode_f32(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "mla_decode_splitkv launch");
  }
  return ok();
}

}  // extern "C"
