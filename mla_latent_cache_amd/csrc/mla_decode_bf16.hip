// Absorbed MLA decode over a bf16 latent cache, gfx950 MFMA kernel.
//
// What it computes (MLA tutorial page, "Move the Key Projection Into the
// Query", "Position Rotations Complicate the Absorption", "Move the Value
// Expansion After the Weighted Sum"; RedKnot-MLA abstract for the segments):
// for each query row (token s, head h) of a segment and a contiguous range of
// cache rows t of one request,
//   s_t = scale * ([q_lat | q_rot] . [c_t | kr_t]),  p = softmax over the range,
//   o_part = sum_t p_t c_t  (fp32, normalised),  lse_part = ln sum_t exp(s_t).
//
// Design (MI355X, 256 CUs, 160 KiB LDS per CU, 64-lane waves):
//  * One workgroup (4 waves) owns up to MT query rows (all heads of a request
//    for the segment, or a row group of them) and streams 32-row tiles of
//    cache rows [c_t | kr_t] (576 bf16 = 1152 B) HBM -> LDS with direct-to-LDS
//    loads, 3 stages deep.  Every tile is read from HBM once and shared by all
//    MT query rows (the latent serves every head's key and value).
//  * LDS rows are padded to 73 slots of 16 B so the 16 rows one MFMA operand
//    read touches fall on distinct bank groups.
//  * QK: S^T[tokens x rows] = K_tile . [q_lat|q_rot]^T with
//    v_mfma_f32_16x16x32_bf16; query rows stay in registers; each QK wave
//    owns whole rows, so the online-softmax row max and sum are in-wave.
//  * Softmax in the exp2 domain with lazy rescaling: the running max is only
//    raised when a tile max exceeds it by more than TAU (=8, log2 units), so
//    the O rescale is almost never executed; p <= 2^TAU stays exact in fp32
//    and representable in bf16.
//  * PV: O^T[d x rows] += C_tile^T . P^T; the 512 latent columns are split over
//    the 4 waves (128 each); the C^T operand comes from ds_read_b64_tr_b16
//    transposed LDS reads, P^T from LDS.
//  * Work split: all rows of the segment (concatenated over requests) are cut
//    into equal shares, one per workgroup (balanced regardless of the length
//    mix); a share that crosses a request boundary yields several pieces.  At
//    most n_split pieces per request; unused slots get lse = -inf.  Each
//    workgroup derives its share from seq_lens on the device (no host sync).
//  * Grid: n_share workgroups per row group; the row groups of one share sit
//    on the same XCD (workgroups are dispatched round-robin over 8 XCDs) so
//    the second read of a tile hits that XCD's L2.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kRow = kDc + kDr;          // elements per cache row
constexpr int kRowBytes = kRow * 2;      // 1152
constexpr int kTile = 32;                // cache rows per tile
constexpr int kSlots = kRowBytes / 16;   // 72 16-byte chunks per row
constexpr int kSlotStride = kSlots + 1;  // 73: one pad slot per LDS row
constexpr int kLRow = kSlotStride * 16;  // 1168 bytes per LDS row
constexpr int kStageBytes = kTile * kLRow;
constexpr int kNStage = 3;
constexpr int kNDma = (kTile * kSlotStride + 63) / 64;  // 37 wave-instructions per tile
constexpr int kPStr = 80;                // bytes per P row (32 bf16 + pad)
constexpr float kTau = 8.f;
constexpr int kPageSize = 64;
constexpr int kMaxPieces = 64;

struct Piece {
  int b, r0, r1, slot;
};

// DMA instructions wave w issues for a full tile: k = w, w+4, ... < kNDma.
__device__ __forceinline__ int dma_per_wave(int w) { return (kNDma - w + 3) / 4; }

__device__ __forceinline__ int sload_i32(const int32_t* p) {
  // Scalar (SMEM) load: counted by lgkmcnt, so it never forces the in-flight
  // LDS-direct loads (vmcnt, in order) to drain.
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

template <int MT>
struct Smem {
  char stage[kNStage][kStageBytes];
  char p[2][MT * kPStr];
  float alpha[2][MT];
  float rowinv[MT];
  int flag[2][4];
  Piece pieces[kMaxPieces];
  int n_pieces;
  int base_next;
  int done;
  int red_i[8];
};

}  // namespace

// QF32: the query (q_lat, q_rot) arrives in fp32 and is split into bf16
// hi + lo parts (q = hi + lo to ~2^-17 relative), each multiplied with the
// bf16 cache tile; two MFMAs per k-step keep the score error ~1e-6 instead of
// the ~1e-3 a bf16-rounded query gives.  With a bf16 query, one MFMA.
template <int MT, bool QF32>
__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeArgs a, int n_share, int n_rg,
                                                             int rows_total) {
  constexpr int NQH = QF32 ? 2 : 1;            // query parts (hi, lo)
  constexpr int NQW = MT >= 64 ? 4 : MT / 16;  // waves that run QK + softmax
  constexpr int RW = MT / NQW;                 // query rows per QK wave (16 or 32)
  constexpr int RB = RW / 16;
  constexpr int QB = MT / 16;                  // row blocks in PV
  __shared__ __attribute__((aligned(16))) Smem<MT> sm;

  const SegArgs& sg = a.seg;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int lg = lane >> 4;  // lane group 0..3

  // ---- which share / row group this workgroup owns (XCD-aware order) ----
  int j, rg;
  if (n_rg == 1) {
    j = blockIdx.x;
    rg = 0;
  } else {
    rg = (blockIdx.x / 8) % n_rg;
    j = (blockIdx.x / (8 * n_rg)) * 8 + blockIdx.x % 8;
  }
  const int row0 = rg * MT;                       // first segment row of this group
  const int nrows = min(MT, rows_total - row0);   // rows in this group
  const int hc = sg.head_count;
  const int B = a.batch;
  const int64_t cap = sg.block_table ? (int64_t)sg.max_pages * kPageSize : sg.max_rows;
  auto clampT = [&](int t) -> int { return (int)max((int64_t)0, min((int64_t)t, cap)); };

  // ---- plan pass 1: total and longest request ----
  int tsum = 0, tmax = 0;
  for (int b = tid; b < B; b += 256) {
    const int T = clampT(sg.seq_lens[b]);
    tsum += T;
    tmax = max(tmax, T);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    tsum += __shfl_xor(tsum, o);
    tmax = max(tmax, __shfl_xor(tmax, o));
  }
  if (lane == 0) {
    sm.red_i[wave] = tsum;
    sm.red_i[4 + wave] = tmax;
  }
  __syncthreads();
  tsum = sm.red_i[0] + sm.red_i[1] + sm.red_i[2] + sm.red_i[3];
  tmax = max(max(sm.red_i[4], sm.red_i[5]), max(sm.red_i[6], sm.red_i[7]));
  const bool req_mode = sg.n_split == 1;
  int share = 0;
  if (!req_mode) {
    share = (tsum + n_share - 1) / n_share;
    share = max(share, (tmax + sg.n_split - 2) / (sg.n_split - 1));
    share = max(kTile, (share + kTile - 1) / kTile * kTile);
  }
  const int lo = j * share, hi = lo + share;
  const float sl2 = a.scale * kLog2e;

  // ---- per-row constants of the QK waves ----
  // query row handled by this lane in row block rb: local index qrow
  int vis_last[RB];   // last visible request-local row for this query row (causal), filled per piece
  int s_of[RB];
  bool rvalid[RB];
  int64_t q_off[RB];  // (tok * n_heads + h) for the row, without tok's request part
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qrow = wave * RW + rb * 16 + l16;
    const int R = row0 + qrow;
    rvalid[rb] = wave < NQW && qrow < nrows;
    const int Rc = rvalid[rb] ? R : 0;
    s_of[rb] = Rc / hc;
    q_off[rb] = (int64_t)s_of[rb] * a.n_heads + sg.head_begin + Rc % hc;
    vis_last[rb] = 0;
  }

  const char* cache = (const char*)sg.cache;

  int base = 0;  // prefix of T over requests scanned so far (wave 0)
  for (int chunk = 0;; ++chunk) {
    // ---- plan pass 2: wave 0 scans 64 requests, lists pieces, writes -inf tails ----
    if (wave == 0) {
      const int b = chunk * 64 + lane;
      const int T = b < B ? clampT(sg.seq_lens[b]) : 0;
      int incl = T;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      const int S = base + incl - T;
      bool is_piece, tail;
      int r0 = 0, r1 = 0, slot = 0, cnt = 0;
      if (req_mode) {
        is_piece = b < B && T > 0 && (b % n_share) == j;
        r1 = T;
        tail = b < B && T == 0 && (b % n_share) == j;
        cnt = 0;
      } else {
        is_piece = b < B && T > 0 && S < hi && S + T > lo;
        r0 = max(lo, S) - S;
        r1 = min(hi, S + T) - S;
        slot = j - S / share;
        const int jf = min(S / share, n_share - 1);
        cnt = T > 0 ? (S + T - 1) / share - S / share + 1 : 0;
        tail = b < B && jf == j && cnt < sg.n_split;
      }
      const uint64_t pm = __ballot(is_piece);
      if (is_piece) {
        const int pos = __popcll(pm & ((1ull << lane) - 1));
        sm.pieces[pos] = Piece{b, r0, r1, slot};
      }
      // slots a request does not use: lse = -inf (their o_part rows are never read)
      uint64_t tm = __ballot(tail);
      while (tm) {
        const int src = __ffsll((long long)tm) - 1;
        tm &= tm - 1;
        const int tb_ = __shfl(b, src);
        const int tc = __shfl(cnt, src);
        const int nsl = sg.n_split - tc;
        for (int e = lane; e < nsl * nrows; e += 64) {
          const int k = tc + e / nrows;
          const int R = row0 + e % nrows;
          const int tok = tb_ * a.s_q + R / hc;
          const int h = sg.head_begin + R % hc;
          a.lse_part[((int64_t)tok * a.n_heads + h) * a.n_part + sg.part_begin + k] = -INFINITY;
        }
      }
      const int total = __shfl(incl, 63);
      if (lane == 0) {
        sm.n_pieces = __popcll(pm);
        const int nb = base + total;
        const bool past = !req_mode && nb >= hi && j < n_share - 1;
        sm.done = (chunk * 64 + 64 >= B) || past;
      }
      base += total;
    }
    __syncthreads();
    const int n_pieces = sm.n_pieces;
    const int done = sm.done;

    for (int pi = 0; pi < n_pieces; ++pi) {
      const Piece pc = sm.pieces[pi];
      const int b = __builtin_amdgcn_readfirstlane(pc.b);
      const int pr0 = __builtin_amdgcn_readfirstlane(pc.r0);
      const int pr1 = __builtin_amdgcn_readfirstlane(pc.r1);
      const int slot = __builtin_amdgcn_readfirstlane(pc.slot);
      const int T = clampT(sg.seq_lens[b]);

      // ---- query rows into registers: [q_lat | q_rot] k-chunks of this lane ----
      bf16x8 qreg[NQH][RB][18];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int64_t qi = (int64_t)b * a.s_q * a.n_heads + q_off[rb];
        vis_last[rb] = sg.causal ? T - a.s_q + s_of[rb] : T - 1;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          const int k0 = 32 * ks + 8 * lg;
          if constexpr (QF32) {
            f32x4 v0 = f32x4{0.f, 0.f, 0.f, 0.f}, v1 = v0;
            if (rvalid[rb]) {
              const float* src = k0 < kDc ? (const float*)a.q_lat + qi * kDc + k0
                                          : (const float*)sg.q_rot + qi * kDr + (k0 - kDc);
              v0 = *(const f32x4*)src;
              v1 = *(const f32x4*)(src + 4);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = e < 4 ? v0[e] : v1[e - 4];
              const bf16 hi = (bf16)v;
              qreg[0][rb][ks][e] = hi;
              qreg[1][rb][ks][e] = (bf16)(v - (float)hi);
            }
          } else {
            qreg[0][rb][ks] = rvalid[rb]
                ? (k0 < kDc ? *(const bf16x8*)((const bf16*)a.q_lat + qi * kDc + k0)
                            : *(const bf16x8*)((const bf16*)sg.q_rot + qi * kDr + (k0 - kDc)))
                : bf16x8{};
          }
        }
      }

      // ---- tile DMA: rows [t0, t0 + nvalid) of request b into stage st ----
      const char* req_base = cache + (int64_t)b * sg.max_rows * kRowBytes;  // contiguous layout
      auto issue_tile = [&](int it) {
        const int t0 = pr0 + it * kTile;
        const int nvalid = min(kTile, pr1 - t0);
        char* st = sm.stage[it % kNStage];
        int pg0 = 0, pg1 = 0;
        if (sg.block_table) {
          const int32_t* bt = sg.block_table + (int64_t)b * sg.max_pages;
          pg0 = sload_i32(bt + t0 / kPageSize);
          pg1 = sload_i32(bt + (t0 + nvalid - 1) / kPageSize);
        }
        for (int k = wave; k < kNDma; k += 4) {
          const int slotl = k * 64 + lane;
          const int r = slotl / kSlotStride;
          const int c = slotl - r * kSlotStride;
          const bool in_tile = slotl < kTile * kSlotStride && c < kSlots;
          bool ok = in_tile && r < nvalid;
          const char* src = nullptr;
          if (ok) {
            const int t = t0 + r;
            if (sg.block_table) {
              const int pg = (t / kPageSize == t0 / kPageSize) ? pg0 : pg1;
              ok = pg >= 0 && pg < sg.n_pages;
              src = cache + ((int64_t)pg * kPageSize + (t % kPageSize)) * kRowBytes + c * 16;
            } else {
              src = req_base + (int64_t)t * kRowBytes + c * 16;
            }
          }
          if (ok) {
            __builtin_amdgcn_global_load_lds((const void*)src, (MLA_LDS void*)(st + k * 1024), 16, 0, 0);
          } else if (in_tile) {
            *(int4*)(st + slotl * 16) = int4{0, 0, 0, 0};  // rows past the piece: zeros, never stale
          }
        }
      };

      const int n_tiles = (pr1 - pr0 + kTile - 1) / kTile;
      issue_tile(0);
      if (n_tiles > 1) issue_tile(1);

      // ---- running state ----
      float m_used[RB], l_part[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        m_used[rb] = -INFINITY;
        l_part[rb] = 0.f;
      }
      f32x4 acc_o[8][QB];
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc_o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

      for (int it = 0; it < n_tiles; ++it) {
        // tile `it` landed: at most the (full) next tile's loads may remain in flight
        const bool next_full = it + 1 < n_tiles && (pr1 - (pr0 + (it + 1) * kTile)) >= kTile;
        if (next_full) {
          wait_vmcnt_dyn(dma_per_wave(wave));
        } else {
          wait_vmcnt<0>();
        }
        wait_lgkm0();
        barrier_raw();
        if (it + 2 < n_tiles) issue_tile(it + 2);

        const char* st = sm.stage[it % kNStage];
        const int t0 = pr0 + it * kTile;
        const int buf = it & 1;

        // ---------------- QK + softmax (waves < NQW) ----------------
        if (wave < NQW) {
          f32x4 sacc[2][RB];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) sacc[tb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              const bf16x8 ak = *(const bf16x8*)(st + (16 * tb + l16) * kLRow + (4 * ks + lg) * 16);
#pragma unroll
              for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int hl = 0; hl < NQH; ++hl)
                  sacc[tb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qreg[hl][rb][ks], sacc[tb][rb], 0, 0, 0);
            }
          }
          bool need_any = false;
          float alpha_r[RB];
          float pv[2][RB][4];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            float mt = -INFINITY;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int t = t0 + 16 * tb + 4 * lg + e;
                const bool v = t < pr1 && t <= vis_last[rb];
                const float s2 = v ? sacc[tb][rb][e] * sl2 : -INFINITY;
                pv[tb][rb][e] = s2;
                mt = fmaxf(mt, s2);
              }
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const bool need = mt > m_used[rb] + kTau;
            alpha_r[rb] = 1.f;
            if (need) {
              alpha_r[rb] = exp2f(m_used[rb] - mt);  // 0 when m_used was -inf
              m_used[rb] = mt;
              l_part[rb] *= alpha_r[rb];
            }
            need_any |= need;
          }
          const bool any = __ballot(need_any) != 0;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int qrow = wave * RW + rb * 16 + l16;
            float lsum = 0.f;
            bf16x4 pk[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float s2 = pv[tb][rb][e];
                const float p = s2 == -INFINITY ? 0.f : exp2f(s2 - m_used[rb]);
                lsum += p;
                pk[tb][e] = (bf16)p;
              }
            l_part[rb] += lsum;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              *(bf16x4*)(sm.p[buf] + qrow * kPStr + (16 * tb + 4 * lg) * 2) = pk[tb];
            if (lg == 0) sm.alpha[buf][qrow] = alpha_r[rb];  // read by PV if any wave rescaled
          }
          if (lane == 0) sm.flag[buf][wave] = any ? 1 : 0;
        }
        wait_lgkm0();
        barrier_raw();

        // ---------------- PV: O^T[d x rows] += C^T . P^T ----------------
        {
          int flag = 0;
#pragma unroll
          for (int w = 0; w < NQW; ++w) flag |= sm.flag[buf][w];
          bf16x8 bq[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            bq[qb] = *(const bf16x8*)(sm.p[buf] + (16 * qb + l16) * kPStr + lg * 16);
          if (flag) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              const float al = sm.alpha[buf][16 * qb + l16];
#pragma unroll
              for (int db = 0; db < 8; ++db) acc_o[db][qb] *= al;
            }
          }
          const int rq = (lane & 15) >> 2, qq = lane & 3;
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const int d0 = 128 * wave + 16 * db;
            const char* p0 = st + (8 * lg + rq) * kLRow + (d0 + 4 * qq) * 2;
            const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0));
            const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + 4 * kLRow));
            const bf16x8 ac = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc_o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ac, bq[qb], acc_o[db][qb], 0, 0, 0);
          }
        }
      }

      // ---- piece epilogue: normalise and write the partial state ----
      if (wave < NQW) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float lt = l_part[rb];
          lt += __shfl_xor(lt, 16);
          lt += __shfl_xor(lt, 32);
          const int qrow = wave * RW + rb * 16 + l16;
          const float inv = lt > 0.f ? 1.f / lt : 0.f;
          if (lg == 0) {
            sm.rowinv[qrow] = inv;
            if (rvalid[rb]) {
              const int64_t ri = (int64_t)b * a.s_q * a.n_heads + q_off[rb];
              a.lse_part[ri * a.n_part + sg.part_begin + slot] =
                  lt > 0.f ? (m_used[rb] + __log2f(lt)) * kLn2 : -INFINITY;
            }
          }
        }
      }
      wait_lgkm0();
      barrier_raw();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qrow = 16 * qb + l16;
        const float inv = sm.rowinv[qrow];
        if (qrow < nrows && inv > 0.f) {
          const int R = row0 + qrow;
          const int tok = b * a.s_q + R / hc;
          const int h = sg.head_begin + R % hc;
          float* o = a.o_part + (((int64_t)tok * a.n_heads + h) * a.n_part + sg.part_begin + slot) * kDc +
                     128 * wave + 4 * lg;
#pragma unroll
          for (int db = 0; db < 8; ++db) *(f32x4*)(o + 16 * db) = acc_o[db][qb] * inv;
        }
      }
      barrier_raw();  // stage buffers, P and rowinv are reused by the next piece
    }
    __syncthreads();
    if (done) break;
  }
}

// Row groups of at most 64 query rows: 64 keeps the query block, the O
// accumulator and the score tile in registers without spilling.
static int row_tile(int rows_total) { return rows_total <= 16 ? 16 : rows_total <= 32 ? 32 : 64; }

void decode_bf16_grid(int rows_total, int n_wg, int* n_share, int* n_rg) {
  const int mt = row_tile(rows_total);
  *n_rg = (rows_total + mt - 1) / mt;
  int ns = n_wg;
  if (*n_rg > 1) {
    ns = (n_wg / *n_rg) / 8 * 8;  // multiple of 8: the row groups of a share share an XCD
    if (ns < 8) ns = 8;
  }
  *n_share = ns < 1 ? 1 : ns;
}

template <bool QF32>
static void launch_mt(const DecodeArgs& a, int mt, dim3 grid, int n_share, int n_rg, int rows_total,
                      hipStream_t stream) {
  const dim3 block(256);
  switch (mt) {
    case 16:
      hipLaunchKernelGGL((decode_bf16_kernel<16, QF32>), grid, block, 0, stream, a, n_share, n_rg, rows_total);
      break;
    case 32:
      hipLaunchKernelGGL((decode_bf16_kernel<32, QF32>), grid, block, 0, stream, a, n_share, n_rg, rows_total);
      break;
    default:
      hipLaunchKernelGGL((decode_bf16_kernel<64, QF32>), grid, block, 0, stream, a, n_share, n_rg, rows_total);
      break;
  }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int n_wg, bool q_f32, hipStream_t stream) {
  const int rows_total = a.s_q * a.seg.head_count;
  const int mt = row_tile(rows_total);
  int n_share, n_rg;
  decode_bf16_grid(rows_total, n_wg, &n_share, &n_rg);
  const dim3 grid(n_share * n_rg);
  if (q_f32)
    launch_mt<true>(a, mt, grid, n_share, n_rg, rows_total, stream);
  else
    launch_mt<false>(a, mt, grid, n_share, n_rg, rows_total, stream);
  return hipGetLastError();
}

}  // namespace mla
