// Host-side launchers of the HIP kernels (internal; the public ABI is
// include/mla_latent.h).  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// One KV segment as the decode kernels receive it.
struct SegArgs {
  const void* cache;
  const int32_t* block_table;  // nullptr => contiguous
  const int32_t* seq_lens;
  const void* q_rot;
  int64_t max_rows;            // contiguous: rows per request in storage
  int page_size;
  int max_pages;
  int n_pages;
  int head_begin;
  int head_count;
  int causal;
  int part_begin;
  int n_split;
  const float* row_rinv;       // QK-Norm: inverse key RMS per stored row, nullptr => none
  const float* row_scale;      // int8 cache: latent scale per stored row, nullptr => 16-bit cache
};

struct DecodeArgs {
  SegArgs seg;
  const void* q_lat;
  void* o_part;       // fp32, or bf16 when part_bf16
  int part_bf16;
  int q_split;        // q_lat as bf16 hi and lo planes [..][2][d_c] (else fp32 [..][d_c])
  float* lse_part;
  int batch;
  int s_q;
  int n_heads;
  int d_c;
  int d_rope;
  int n_part;
  float scale;
};

// One launch of the row-owning decode over up to kRowsMaxSegs segments:
// segment g owns workgroups [wg_begin[g], wg_begin[g + 1]) (the last one to
// the end of the grid), cut into n_share[g] shares x n_rg[g] row groups.
constexpr int kRowsMaxSegs = 8;
struct RowsLaunch {
  DecodeArgs a;  // the call's shared arguments (a.seg unused)
  SegArgs segs[kRowsMaxSegs];
  int wg_begin[kRowsMaxSegs];
  int n_share[kRowsMaxSegs];
  int n_rg[kRowsMaxSegs];
  int rows_total[kRowsMaxSegs];
  int n_segs;
};

// Dtype flags below: true = bf16 storage, false = fp32.
hipError_t launch_rope(const void* q_pe, bool in_bf16, void* q_rot, bool out_bf16, const int64_t* pos,
                       const int64_t* shift, int n_tok, int n_heads, int d_rope, double base,
                       hipStream_t stream);
hipError_t launch_absorb(const void* q_nope, const void* w_uk, bool in_bf16, void* q_lat, bool out_bf16,
                         int n_tok, int n_heads, int d_nope, int d_c, hipStream_t stream);
hipError_t launch_out_uv(const void* o_lat, bool o_bf16, const void* w_uv, bool w_bf16, void* out,
                         bool out_bf16, int n_tok, int n_heads, int d_c, int d_v, hipStream_t stream);
// out[t][n] = sum_k x[t][k] w[n][k] (MFMA for bf16 operands, k_in % 256 == 0, 16-byte aligned)
bool out_proj_mfma_ok(const void* x, bool x_bf16, const void* w, bool w_bf16, int k_in);
hipError_t launch_out_proj(const void* x, bool x_bf16, const void* w, bool w_bf16, void* out, bool out_bf16,
                           int n_tok, int k_in, int d_model, hipStream_t stream);
// bf16 MFMA variants (d_nope = 128, d_c = 512, d_v = 128, 16-byte aligned).
bool absorb_mfma_ok(const void* q_nope, const void* w_uk, const void* q_lat, int d_nope, int d_c);

// Rotation targets of the fused query preparation (one per segment shift).
constexpr int kMaxShift = 8;
struct RopeTargets {
  void* q_rot[kMaxShift];
  const int64_t* shift[kMaxShift];
  int n;
};
// QK-Norm of the query inside the absorption (g_q == nullptr: none).  Every
// absorption workgroup reads all heads of its tokens for their RMS, so the
// fused form is bounded to n_tok * n_heads <= kQkFusedRows.
constexpr int kQkFusedRows = 512;
// QK-Norm of the query inside the absorption (g_q == nullptr: none).
struct QkArgs {
  const float* g_q = nullptr;  // [n_heads][d_nope]
  const float* g_k = nullptr;  // [n_heads][d_nope]
  float eps = 0.f;
};
// lat_mode: 0 fp32, 1 bf16, 2 bf16 hi and lo planes
hipError_t launch_prepare_mfma(const void* q_nope, bool q_f32, const void* w_uk, void* q_lat, int lat_mode,
                               const void* q_pe, const int64_t* pos, const RopeTargets& rt, bool rot_bf16, int n_tok,
                               int n_heads, int d_rope, double base, const QkArgs& qk, hipStream_t stream);
hipError_t launch_absorb_mfma(const void* q_nope, const void* w_uk, void* q_lat, bool out_bf16, int n_tok,
                              int n_heads, hipStream_t stream);
bool out_uv_mfma_ok(const void* o_lat, const void* w_uv, int d_c, int d_v);
hipError_t launch_out_uv_mfma(const void* o_lat, const void* w_uv, void* out, bool out_bf16, int n_tok,
                              int n_heads, hipStream_t stream);
hipError_t launch_combine(const void* o_part, bool part_bf16, const float* lse_part, int n_rows, int n_part,
                          int d_c, void* o_lat, bool out_bf16, float* lse, hipStream_t stream);
// Merge and value expansion of (token, head) rows in one launch (d_c <= 512,
// d_v <= 128); o_lat and lse may be null.
hipError_t launch_combine_out_uv(const void* o_part, bool part_bf16, const float* lse_part, int n_tok, int n_heads, int n_part,
                                 int d_c, const void* w_uv, bool w_bf16, int d_v, void* o_lat, float* lse,
                                 void* out, bool out_bf16, hipStream_t stream);
// int8 latent cache writer: bf16 rows [n][d_c + d_rope] -> packed rows [n][d_c + 2 d_rope] bytes + scales.
hipError_t launch_quantize_latent_i8(const void* rows, int64_t n_rows, int d_c, int d_rope, void* out,
                                     float* scales, hipStream_t stream);
hipError_t launch_quantize_latent_i4(const void* rows, int64_t n_rows, int d_c, int d_rope, void* out,
                                     float* scales, hipStream_t stream);
// QK-Norm: query scaling, the key Gram matrix and the per-row inverse RMS.
hipError_t launch_qknorm_query(const void* q_nope, bool in_bf16, const float* g_q, const float* g_k, int n_tok,
                               int n_heads, int d_nope, float eps, float* q_out, hipStream_t stream);
hipError_t launch_qknorm_key_gram(const void* w_uk, bool w_bf16, int n_heads, int d_nope, int d_c, float* gram,
                                  hipStream_t stream);
hipError_t launch_qknorm_key_rinv(const void* rows, bool row_bf16, int64_t n_rows, int row_width, const float* gram,
                                  int d_c, int n_hd, float eps, float* rinv, hipStream_t stream);
// Generic fp32 decode (any d_c <= 512, d_rope <= 128): one wave per
// (query row, split), equal-length splits per request.
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);
// bf16 MFMA decode (d_c = 512, d_rope = 64, page 64).  n_wg workgroups per
// row group; balanced split of all rows of the segment over them.
// q_f32: q_lat / q_rot are fp32 (split into bf16 hi + lo) instead of bf16.
// Low-bit caches run on the row-owning kernel (launch_decode_rows_multi).
hipError_t launch_decode_bf16(const DecodeArgs& a, int n_wg, bool q_f32, hipStream_t stream);
// Grid shape of a bf16 decode of one segment with row groups of mt rows:
// row groups and shares (n_wg workgroups per row group, a multiple of 8 when
// there are several row groups).
void decode_bf16_grid(int rows_total, int mt, int n_wg, int* n_share, int* n_rg);
// Rows of the row group the bf16 decode uses for a segment (the kernel
// chosen by launch_decode_bf16 for an fp32 query and a 16-bit cache).
int decode_bf16_tile(int rows_total);
// bf16 MFMA decode with whole query rows per wave, for segments of more than
// 32 query rows with an fp32 query, a 16-bit cache and no QK-Norm factors:
// row groups of 64 (up to 64 rows) or 128; n_wg workgroups per row group.
hipError_t launch_decode_rows(const DecodeArgs& a, int n_wg, hipStream_t stream);
// All n_segs segments (any number; kRowsMaxSegs per launch) in row-owning
// launches that split n_wg workgroups by estimated tile work; qm: the stored
// rows (0: 16-bit, 1: int4, 2: int8; low-bit rows take 64-row groups).
hipError_t launch_decode_rows_multi(const DecodeArgs& a, const SegArgs* segs, int n_segs, int n_wg, int qm,
                                    hipStream_t stream);
// Rows of that kernel's row group for a segment of rows_total query rows.
int decode_rows_tile(int rows_total);

}  // namespace mla
