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
// Design (MI355X: 256 CUs, 4 SIMDs and 160 KiB LDS per CU, 64-lane waves):
//  * One workgroup of 8 waves (2 per SIMD) owns up to MT = 64 query rows (all
//    heads of a request for the segment, or a 64-row group of them) and
//    streams 32-row tiles of cache rows [c_t | kr_t] (576 bf16 = 1152 B)
//    HBM -> LDS with direct-to-LDS loads: latent parts into a 4-stage ring,
//    rotary parts into a 3-stage ring (3 tiles in flight).  Every tile is read
//    from HBM once and shared by all MT query rows: the latent serves every
//    head's key and value.
//  * LDS tiles are unpadded (36 KiB) with 16-byte chunks XOR-swizzled per row,
//    so the 16-row score-operand reads and the transposed reads are free of
//    bank conflicts.
//  * Wave roles, one tile apart: score waves 0..3 hold the query in registers
//    and compute S^T[tokens x rows] = K_tile . [q_lat|q_rot]^T of tile it+1 on
//    v_mfma_f32_16x16x32_bf16, the online softmax and P (bf16, in LDS).  The
//    score waves of a group split the 18 k-steps and add their partial scores
//    through LDS (one exchange barrier per tile): MT = 16, one group of four
//    k-parts; MT = 32, two groups of two; MT = 64, two groups of two waves
//    that each multiply two row blocks over half the k-steps, so each K
//    operand read serves 32 query rows.  PV waves 4..7 each own 128 latent
//    columns and accumulate O^T[d x rows] += C_tile^T . P^T of tile it, with
//    C^T from ds_read_b64_tr_b16 transposed LDS reads.  The PV waves also
//    issue all tile loads, spread between their MFMAs.
//  * An fp32 query is split into bf16 hi + lo parts (q = hi + lo to ~2^-17);
//    a bf16-rounded query alone would put ~1e-3 into the scores.  MT <= 32
//    multiplies both parts at every k-step.  MT = 64 multiplies lo only at the
//    two rotary k-steps: with delta_t = scale (lo . c_t) the neglected part of
//    a latent score, ln sum exp(s_t + delta_t) = lse + sum_t p_t delta_t +
//    O(var_p delta) = lse + scale (lo . o) + O(delta^2), so the lse gains
//    scale (lo . o) (the partial output o is at hand in the PV waves) and the
//    score MFMAs drop from 36 to 20 k-steps per row block.  The remaining lse
//    error is second order (about 1e-5 at these scales); the outputs keep a
//    first-order term of size |delta| times the spread of c over the
//    softmax, far inside their tolerance.
//  * Softmax in the exp2 domain (raw v_exp_f32) with lazy rescaling: the
//    running max only moves when a tile max exceeds it by more than TAU = 8
//    (log2 units), so the O rescale almost never runs; p <= 2^8 stays exact in
//    fp32 and representable in bf16.  Full tiles skip all masking.  Row
//    reductions over the four 16-lane rows use the gfx950 row-swap
//    instructions (VALU only).
//  * Work split: all rows of the segment (concatenated over requests) are cut
//    into equal shares, one per workgroup, whatever the length mix; a share
//    crossing a request boundary yields several pieces.  At most n_split
//    pieces per request; unused slots get lse = -inf.  Each workgroup derives
//    its share from seq_lens on the device (no host synchronisation).
//  * Grid: n_share workgroups per row group; the row groups of one share sit
//    on the same XCD (workgroups are dispatched round-robin over 8 XCDs) so
//    the second read of a tile hits that XCD's L2.
//  * Synchronisation: a raw s_barrier plus explicit vmcnt/lgkmcnt waits;
//    __syncthreads()' fence would drain the in-flight tile loads.  Every
//    branch on a wave's role is a scalar branch.
#include "mla_common.h"
#include "mla_decode_tile.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kNStage = 4;                  // latent ring: read by the score waves, then the PV waves
constexpr int kAhead = kNStage - 1;         // tiles in flight beyond the two being computed on
constexpr int kNRStage = kAhead;            // rotary ring: dead once its tile is scored
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
// wave-instructions per tile: one per latent row (64 lanes x 16 B), then 4
// for the rotary parts (8 rows x 8 chunks each)
constexpr int kNDma = kTile + kRStage / 1024;
static_assert(kNDma == 36 && kRStage % 1024 == 0, "tile geometry");
constexpr int kPStr = 80;                   // bytes per P row (32 bf16 + pad)
constexpr int kMaxPieces = 64;

// Ring geometry: the tile loads of 16-bit rows (1152 B) land directly in the
// latent ring the MFMAs read (4 stages, 3 tiles ahead).
struct Geo {
  static constexpr int RB = kRowBytes;   // cache bytes per row
  static constexpr int NST = kNStage;    // latent stages
  static constexpr int AHEAD = kAhead;   // tiles loading beyond the two in use
  static constexpr int NRST = AHEAD;     // rotary ring
  static constexpr int NDMA = kNDma;     // wave-instructions per tile
  static constexpr int LAT = kTile;      // of which latent
};

// Loads of one tile: `lim` bytes (whole rows) that are contiguous in memory
// from `src` (tiles are aligned to 32 rows inside a request and never cross a
// 64-row page).  Wave-instruction k < 32 fills latent LDS row k: lane l moves
// the chunk stored at position l, cache bytes k * 1152 + (l ^ (k & 15)) * 16.
// The next 4 fill rotary rows 8 (k - LAT) + l / 8 at position l % 8.  Rows past
// the valid ones are zero-filled so no stale value is ever read.  The four PV
// waves issue all tile loads: loader l = wave - 4 issues k = l + 4 i.
// An LDS-direct load keeps its wave busy at issue, so the score waves, which
// set the pace, issue none.
struct TileDma {
  char* cdst;       // latent ring stage
  char* rdst;       // rotary ring stage
  const char* src;  // first cache byte of the tile
  int lim;          // valid bytes at src
};

// Cache byte offset (within the tile) and LDS destination of instruction k for this lane.
__device__ __forceinline__ int dma_src_off(int k, int lane) {
  if (k < Geo::LAT) return k * kRowBytes + cpos(k, lane) * 16;
  const int r = 8 * (k - Geo::LAT) + (lane >> 3);
  return r * Geo::RB + kCBytes + rpos(r, lane & 7) * 16;
}
__device__ __forceinline__ char* dma_dst(const TileDma& d, int k) {
  return k < Geo::LAT ? d.cdst + k * 1024 : d.rdst + (k - Geo::LAT) * 1024;
}

// UNI: the loader index (hence k) is wave-uniform and held opaque in a
// scalar register, so the latent/rotary choice is a scalar branch and no
// per-instruction offset is hoisted; else it is a lane value and both sides
// run under the exec mask (fewer branches, more vector registers).
template <bool UNI>
__device__ __forceinline__ void issue_dma_one(const TileDma& d, int k, int lane) {
  // Opaque copy of the lane index: the offsets are recomputed at every
  // instruction (a few integer ops) instead of being hoisted out of the tile
  // loop and pinning registers for the whole loop.
  asm volatile("" : "+v"(lane));
  if constexpr (UNI) asm volatile("" : "+s"(k));
  const int off = dma_src_off(k, lane);
  char* dst = dma_dst(d, k);
  if (off < d.lim) {  // the lane's row is a valid row of the tile
    __builtin_amdgcn_global_load_lds((const void*)(d.src + off), (MLA_LDS void*)dst, 16, 0, 0);
  } else {
    *(int4*)(dst + lane * 16) = int4{0, 0, 0, 0};
  }
}

constexpr int kLoaders = 4;  // waves issuing tile loads (the PV waves)
constexpr int dma_per_wave() {
  static_assert(Geo::NDMA % kLoaders == 0, "every loader issues the same count");
  return Geo::NDMA / kLoaders;  // 9
}

// Loader `ld`'s i-th instruction of a tile (k = ld + 4 i): a full tile
// issues it from a uniform base plus a lane offset of two or three integer
// ops (no bounds check, every lane valid), a partial tile takes the
// bounds-checked path with zero fill.  `lane` should be opaque to the
// compiler, or it hoists the nine offsets into live registers (`ld` too with
// UNI, see issue_dma_one).
template <bool UNI>
__device__ __forceinline__ void issue_dma_fast(const TileDma& d, int ld, int i, int lane) {
  if constexpr (UNI) asm volatile("" : "+s"(ld));
  const int k = ld + kLoaders * i;
  if (d.lim == kTile * Geo::RB) {
    __builtin_amdgcn_global_load_lds((const void*)(d.src + (unsigned)dma_src_off(k, lane)),
                                     (MLA_LDS void*)dma_dst(d, k), 16, 0, 0);
  } else {
    issue_dma_one<UNI>(d, k, lane);
  }
}

// All of loader `ld`'s instructions of a tile at once.
template <bool UNI>
__device__ __forceinline__ void issue_tile_dma(const TileDma& d, int ld, int lane) {
#pragma unroll
  for (int i = 0; i < dma_per_wave(); ++i) issue_dma_one<UNI>(d, ld + kLoaders * i, lane);
}

// First byte of tile rows [t0, ...) of request b: contiguous cache, or the
// page holding row t0 (scalar load of the block-table entry; an id outside
// [0, n_pages) makes the tile read as zeros).
__device__ __forceinline__ const char* tile_src(const char* cache, const char* req_base, const int32_t* bt_row,
                                                int n_pages, int t0, bool* ok) {
  constexpr int RB = Geo::RB;
  *ok = true;
  if (!bt_row) return req_base + (int64_t)t0 * RB;
  const int pg = sload_i32(bt_row + t0 / kPageSize);
  *ok = pg >= 0 && pg < n_pages;
  return cache + ((int64_t)(*ok ? pg : 0) * kPageSize + (t0 % kPageSize)) * RB;
}

template <int MT>
struct Smem {
  using G = Geo;
  static constexpr int NRB = MT / 16;
  static constexpr int QBW = NRB == 4 ? 2 : 1;  // 16-row blocks per score wave
  static constexpr int KS = 4 / (NRB / QBW);    // k-parts (score waves) per group of QBW blocks
  char cst[G::NST][kCStage];    // 16-bit latent ring
  char rst[G::NRST][kRStage];   // rotary ring
  char p[2][MT * kPStr];         // P (bf16) of two tiles
  // exchanged partial scores [slot][tb][lane][4]: QBW = 1, k-parts 1..KS-1 of each
  // row block; QBW = 2, the partner's k-part of each row block.  After a
  // piece's last tile: the PV waves' lse corrections [PV wave][row] (MT = 64).
  float xbuf[(QBW == 1 ? NRB * (KS - 1) : NRB) * 2 * 64 * 4];
  float alpha[2][MT];
  float rowinv[MT];
  int flag[2][4];
  Piece pieces[kMaxPieces];
  int n_pieces;
  int done;
  int red_i[2 * kWaves];
};

// Loader `ld`: wait until at most `after` tiles issued after the needed one
// are still in flight; `after_full` says they are all full tiles (a partial
// tile issues fewer instructions, then everything is waited for).
__device__ __forceinline__ void wait_tiles(int after, bool after_full) {
  constexpr int W = dma_per_wave();
  if (!after_full || after == 0) {
    wait_vmcnt<0>();
  } else if (after == 1) {
    wait_vmcnt<W>();
  } else {
    wait_vmcnt<2 * W>();
  }
}

}  // namespace

// QF32: q_lat / q_rot are fp32 and split into bf16 hi + lo parts.
// QKN: QK-Norm, the latent part of every score is multiplied by the stored
// row's inverse key RMS (seg.row_rinv).
template <int MT, bool QF32, bool QKN>
__global__ __launch_bounds__(kThreads, 1) void decode_bf16_kernel(DecodeArgs a, int n_share, int n_rg,
                                                                  int rows_total) {
  constexpr int NRB = MT / 16;       // 16-row blocks
  // Score waves 0..3 form NRB / QBW groups; a group's KS waves multiply its
  // QBW row blocks, each over a part of the 18 k-steps, and add their partial
  // scores through LDS.  MT = 16: 1 group of 4 waves (one block, four k-parts);
  // MT = 32: 2 groups of 2; MT = 64: 2 groups of 2 waves that each multiply
  // two blocks over half the k-steps, so each K operand read from LDS serves
  // 32 query rows (half the LDS traffic of one block per wave).
  constexpr int QBW = NRB == 4 ? 2 : 1;
  constexpr int KS = 4 / (NRB / QBW);
  // An fp32 query is split into bf16 hi + lo parts (q = hi + lo to ~2^-17).
  // MT <= 32 multiplies both parts at every k-step (NQH = 2).  MT = 64, where
  // the score MFMAs dominate, multiplies lo only at the two rotary k-steps
  // and restores the latent lo part's share of the scores to first order in
  // the lse (LOC below, epilogue).
  // (the first-order correction needs sum_t p_t c_t to carry the latent
  // scores' weights, which QK-Norm's per-row factor breaks)
  constexpr bool LOC = QF32 && MT == 64 && !QKN;
  using G = Geo;
  constexpr bool FAC = QKN;  // a per-row factor on the latent score
  constexpr bool UNI = QKN;  // wave-uniform loader index (see pw)
  constexpr int NQH = QF32 && !LOC ? 2 : 1;
  // The KS waves of a group cut the k-steps into parts of equal MFMA count:
  // with LOC the two rotary k-steps cost two MFMAs each, so the 20 MFMA steps
  // split 10 + 10, the rotary steps at the end of the last part.
  constexpr int KCOST = LOC ? kKSteps + kDr / 32 : kKSteps;
  static_assert(!LOC || KCOST % KS == 0, "equal parts");
  constexpr int KMAX = (KCOST + KS - 1) / KS;
  constexpr int KLAST = kKSteps - (KS - 1) * (KCOST / KS);  // k-steps of the last part (LOC)
  __shared__ __attribute__((aligned(16))) Smem<MT> sm;
  static_assert(sizeof(sm.xbuf) >= 4 * MT * sizeof(float), "lse corrections fit the exchange buffer");
  static_assert(!LOC || G::NST >= 3, "two latent stages free for the lo rows after the last tile");

  // every argument field as a local value (see issue_tile_dma)
  const char* const cache = (const char*)a.seg.cache;
  const int32_t* const block_table = a.seg.block_table;
  const int32_t* const seq_lens = a.seg.seq_lens;
  const void* const q_rot_p = a.seg.q_rot;
  const void* const q_lat_p = a.q_lat;
  void* const o_part = a.o_part;
  const bool part_bf = a.part_bf16;
  float* const lse_part = a.lse_part;
  const float* const row_fac = a.seg.row_rinv;  // FAC: per stored row
  const int64_t max_rows = a.seg.max_rows;
  const int max_pages = a.seg.max_pages;
  const int n_pages = a.seg.n_pages;
  const int head_begin = a.seg.head_begin;
  const int hc = a.seg.head_count;
  const int causal = a.seg.causal;
  const int part_begin = a.seg.part_begin;
  const int n_split = a.seg.n_split;
  const int s_q = a.s_q;
  const int n_heads = a.n_heads;
  const int n_part = a.n_part;
  const int B = a.batch;
  const float scale = a.scale;
  const float sl2 = scale * kLog2e;

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
  const int row0 = rg * MT;                      // first segment row of this group
  const int nrows = min(MT, rows_total - row0);  // rows in this group
  const int64_t cap = block_table ? (int64_t)max_pages * kPageSize : max_rows;
  auto clampT = [cap](int t) -> int { return (int)max((int64_t)0, min((int64_t)t, cap)); };

  // ---- plan pass 1: total and longest request, each padded to whole tiles ----
  // (a share then starts on a tile boundary of every request it touches, and
  // no tile crosses a 64-row page).  Only wave 0 plans; with B <= 64 it takes
  // the totals from the same per-lane load its piece scan uses (one global
  // round trip and no workgroup barrier before the scan).
  auto padT = [](int t) -> int { return (t + kTile - 1) / kTile * kTile; };
  int tsum = 0, tmax = 0;
  int Tr_lane = 0;  // rows of request `lane` (wave 0, B <= 64)
  if (B <= 64) {
    if (wave == 0) {
      Tr_lane = lane < B ? clampT(seq_lens[lane]) : 0;
      tsum = padT(Tr_lane);
      tmax = tsum;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        tsum += __shfl_xor(tsum, o);
        tmax = max(tmax, __shfl_xor(tmax, o));
      }
    }
  } else {
    for (int b = tid; b < B; b += kThreads) {
      const int T = padT(clampT(seq_lens[b]));
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
      sm.red_i[kWaves + wave] = tmax;
    }
    __syncthreads();
    tsum = 0;
    tmax = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      tsum += sm.red_i[w];
      tmax = max(tmax, sm.red_i[kWaves + w]);
    }
  }
  const bool req_mode = n_split == 1;
  int share = 0;
  if (!req_mode) {
    share = (tsum + n_share - 1) / n_share;
    share = max(share, (tmax + n_split - 2) / (n_split - 1));
    share = max(kTile, (share + kTile - 1) / kTile * kTile);
  }
  const int lo = j * share, hi = lo + share;

  // ---- roles: waves 0..3 score (row block rb, k-part kp); waves 4..7 own 128 latent columns each ----
  // Role variables are wave-uniform scalars: every branch on them is a
  // scalar branch.  (Under a divergent branch with an empty EXEC mask the
  // matrix instructions would still run.)
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const bool qk_wave = wave_s < 4;
  const bool pv_wave = wave_s >= 4;
  const int grp = (wave_s & 3) / KS;   // group of a score wave: row blocks grp * QBW ..
  const int kp = (wave_s & 3) % KS;    // its part of the k-steps: [ks0, ks0 + kcnt)
  const int ks0 = LOC ? kp * (KCOST / KS) : kp * (kKSteps / KS) + min(kp, kKSteps % KS);
  const int kcnt = LOC ? (kp == KS - 1 ? KLAST : KCOST / KS) : kKSteps / KS + (kp < kKSteps % KS ? 1 : 0);
  const bool rope_part = kp == KS - 1;  // this score wave's part holds the rotary k-steps
  // the row block whose softmax this wave runs (QBW = 1: only k-part 0 runs one)
  const int rb = QBW == 1 ? grp : grp * QBW + kp;
  const bool smax_wave = QBW > 1 || kp == 0;
  const int qrow = rb * 16 + l16;    // local softmax row of this lane (score waves)
  const bool rvalid = qk_wave && qrow < nrows;
  const int Rc = rvalid ? row0 + qrow : row0;
  const int s_row = Rc / hc;
  const int64_t q_off = (int64_t)s_row * n_heads + head_begin + Rc % hc;  // without the request part
  const int s_min = row0 / hc;       // smallest token index among the group's rows
  // column slice of a PV wave and its loader index.  With a row factor (the
  // register-heaviest variants) it is the scalar copy, so the tile loads
  // branch on it (issue_dma_one); elsewhere the lane value measured faster.
  const int pw = (UNI ? wave_s : wave) - 4;

  int base = 0;  // prefix of padded T over requests scanned so far (wave 0)
  for (int chunk = 0;; ++chunk) {
    // ---- plan pass 2: wave 0 scans 64 requests, lists pieces, writes -inf tails ----
    if (wave == 0) {
      const int b = chunk * 64 + lane;
      const int Tr = B <= 64 ? Tr_lane : b < B ? clampT(seq_lens[b]) : 0;  // rows
      const int T = padT(Tr);                           // rows padded to whole tiles
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
        r1 = Tr;
        tail = b < B && T == 0 && (b % n_share) == j;
      } else {
        is_piece = b < B && T > 0 && S < hi && S + T > lo;
        r0 = max(lo, S) - S;
        r1 = min(min(hi, S + T) - S, Tr);  // a piece starting below Tr, clipped to the real rows
        slot = j - S / share;
        const int jf = min(S / share, n_share - 1);
        cnt = T > 0 ? (S + T - 1) / share - S / share + 1 : 0;
        tail = b < B && jf == j && cnt < n_split;
      }
      const uint64_t pm = __ballot(is_piece);
      if (is_piece) {
        const int pos = __popcll(pm & ((1ull << lane) - 1));
        sm.pieces[pos] = Piece{b | (slot << 16), r0, r1, Tr};
      }
      // slots a request does not use: lse = -inf (their o_part rows are never read)
      uint64_t tm = __ballot(tail);
      while (tm) {
        const int src = __ffsll((long long)tm) - 1;
        tm &= tm - 1;
        const int tb_ = __shfl(b, src);
        const int tc = __shfl(cnt, src);
        const int nsl = n_split - tc;
        for (int e = lane; e < nsl * nrows; e += 64) {
          const int k = tc + e / nrows;
          const int R = row0 + e % nrows;
          const int tok = tb_ * s_q + R / hc;
          const int h = head_begin + R % hc;
          lse_part[((int64_t)tok * n_heads + h) * n_part + part_begin + k] = -INFINITY;
        }
      }
      const int total = __shfl(incl, 63);
      if (lane == 0) {
        sm.n_pieces = __popcll(pm);
        const bool past = !req_mode && base + total >= hi && j < n_share - 1;
        sm.done = (chunk * 64 + 64 >= B) || past;
      }
      base += total;
    }
    __syncthreads();
    const int n_pieces = sm.n_pieces;
    const int done = sm.done;

    for (int pi = 0; pi < n_pieces; ++pi) {
      const Piece pc = sm.pieces[pi];
      const int b_slot = __builtin_amdgcn_readfirstlane(pc.b_slot);
      const int b = b_slot & 0xffff;
      const int slot = (int)((unsigned)b_slot >> 16);
      const int pr0 = __builtin_amdgcn_readfirstlane(pc.r0);
      const int pr1 = __builtin_amdgcn_readfirstlane(pc.r1);
      const int T = __builtin_amdgcn_readfirstlane(pc.T);
      const int vis_last = causal ? T - s_q + s_row : T - 1;  // last visible row of this lane's query
      const int vis_min = causal ? T - s_q + s_min : T - 1;   // ... of the group's first query row
      const int n_tiles = (pr1 - pr0 + kTile - 1) / kTile;
      const bool last_full = (pr1 - pr0) % kTile == 0;       // only the last tile can be partial

      const char* const req_base = cache + (int64_t)b * max_rows * G::RB;  // contiguous layout
      const int32_t* const bt_row = block_table ? block_table + (int64_t)b * max_pages : nullptr;
      // where tile `it` comes from and goes to (lim = 0: all zeros)
      auto tile_dma = [&](int it) -> TileDma {
        const int t0 = pr0 + it * kTile;
        bool ok;
        const char* src = tile_src(cache, req_base, bt_row, n_pages, t0, &ok);
        char* const cdst = sm.cst[it % G::NST];
        return TileDma{cdst, sm.rst[it % G::NRST], src, ok ? min(kTile, pr1 - t0) * G::RB : 0};
      };
      auto load_tile = [&](int it) { issue_tile_dma<UNI>(tile_dma(it), pw, lane); };

      // The two roles run separate copies of the tile loop with the same
      // barrier sequence (1 + n_tiles + 1 barriers, plus one exchange barrier
      // per scored tile when KS > 1), so the register allocator never holds
      // the query block and the O accumulator at once.
      if (qk_wave) {
        // ---- score wave: row blocks grp * QBW .. + QBW-1, k-steps [ks0, ks0 + kcnt) ----
        bf16x8 qreg[NQH][QBW][KMAX];  // [hi, lo] parts of the query (hi only with LOC / a bf16 query)
        bf16x8 qlo[QBW][2];           // LOC: lo parts of the two rotary k-steps (last part only)
#pragma unroll
        for (int j = 0; j < QBW; ++j) {
          const int row = (grp * QBW + j) * 16 + l16;
          const int Rj = row0 + row;
          const int64_t qi = (int64_t)b * s_q * n_heads + (int64_t)(Rj / hc) * n_heads + head_begin + Rj % hc;
#pragma unroll
          for (int i = 0; i < KMAX; ++i) {
            const int k0 = 32 * (ks0 + i) + 8 * lg;
            const bool in = row < nrows && i < kcnt;
            if constexpr (QF32) {
              f32x4 v0 = f32x4{0.f, 0.f, 0.f, 0.f}, v1 = v0;
              if (in) {
                const float* src = k0 < kDc ? (const float*)q_lat_p + qi * kDc + k0
                                            : (const float*)q_rot_p + qi * kDr + (k0 - kDc);
                v0 = *(const f32x4*)src;
                v1 = *(const f32x4*)(src + 4);
              }
              bf16x8 h8, l8;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float v = e < 4 ? v0[e] : v1[e - 4];
                const bf16 h = (bf16)v;
                h8[e] = h;
                l8[e] = (bf16)(v - (float)h);
              }
              qreg[0][j][i] = h8;
              if constexpr (NQH == 2) qreg[NQH - 1][j][i] = l8;
              if constexpr (LOC)
                if (i >= KLAST - 2 && i < KLAST) qlo[j][i - (KLAST - 2)] = rope_part ? l8 : bf16x8{};
            } else {
              qreg[0][j][i] = in ? (k0 < kDc ? *(const bf16x8*)((const bf16*)q_lat_p + qi * kDc + k0)
                                             : *(const bf16x8*)((const bf16*)q_rot_p + qi * kDr + (k0 - kDc)))
                                 : bf16x8{};
            }
          }
        }
        // LOC: lo part of latent query row r (lane = 8-column chunk), for the
        // lse correction
        auto lo_row = [&](int r) -> bf16x8 {
          f32x4 v0 = f32x4{0.f, 0.f, 0.f, 0.f}, v1 = v0;
          if (r < nrows) {
            const int Rr = row0 + r;
            const int64_t qi = (int64_t)b * s_q * n_heads + (int64_t)(Rr / hc) * n_heads + head_begin + Rr % hc;
            const float* src = (const float*)q_lat_p + qi * kDc + 8 * lane;
            v0 = *(const f32x4*)src;
            v1 = *(const f32x4*)(src + 4);
          }
          bf16x8 l8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = e < 4 ? v0[e] : v1[e - 4];
            l8[e] = (bf16)(v - (float)(bf16)v);
          }
          return l8;
        };
        float m_used = -INFINITY;  // running max (log2 units) of this lane's query row (k-part 0)
        float l_part = 0.f;        // this lane's share of the row's sum of p (k-part 0)

        // scores, softmax and P of tile `it`, into P / alpha / flag buffer it & 1.
        // With KS > 1 the waves of a row block exchange partial scores through
        // LDS (one extra barrier) and k-part 0 runs the softmax.
        // QK-Norm factors: the lane's 8 rows of a tile (tokens 16 tb + 4 lg +
        // e).  rinv_row: the tile's first factor (a scalar block-table load,
        // issued where no LDS access is pending), null for a page outside the
        // pool (its tile reads as zeros and takes factor 1).
        auto rinv_row = [&](int it) -> const float* {
          const int t0 = pr0 + it * kTile;
          if (!bt_row) return row_fac + (int64_t)b * max_rows + t0;
          const int pg = sload_i32(bt_row + t0 / kPageSize);
          return (pg >= 0 && pg < n_pages) ? row_fac + (int64_t)pg * kPageSize + t0 % kPageSize : nullptr;
        };
        // The loads are unconditional (a select on a loaded value would wait
        // for it here): rows past the piece repeat its last row's factor, in
        // bounds and finite, and their scores are masked later.  Returns
        // whether the factors are real (false: use 1).
        auto load_rinv = [&](int it, const float* rr, f32x4& r0v, f32x4& r1v) -> bool {
          const int lim = pr1 - 1 - (pr0 + it * kTile);  // >= 0: the tile starts inside the piece
          const float* src = rr ? rr : row_fac;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * lg + e;
            r0v[e] = src[min(t, lim)];
            r1v[e] = src[min(16 + t, lim)];
          }
          return rr != nullptr;
        };
        // scores of tile `it` with its QK-Norm factors (rf0, rf1) in
        // registers; once they are applied, the same registers receive the
        // factors of tile it+1 (applied a tile later, so the loads have time)
        auto score_tile = [&](int it, f32x4& rf0, f32x4& rf1, bool& rf_ok) {
          const char* cs = sm.cst[it % G::NST];
          const char* rs = sm.rst[it % G::NRST];
          const int t0 = pr0 + it * kTile;
          const int buf = it & 1;
          const float* rr_next = nullptr;
          if constexpr (FAC)
            if (it + 1 < n_tiles) rr_next = rinv_row(it + 1);
          // accumulators: hi and lo parts (else even and odd k-steps)
          // separately with one row block (two independent chains would stall
          // on each other), shared with two (four chains already)
          constexpr int NACC = QBW == 1 ? 2 : 1;
          f32x4 sacc[2][QBW][NACC];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int j = 0; j < QBW; ++j)
#pragma unroll
              for (int hl = 0; hl < NACC; ++hl) sacc[tb][j][hl] = f32x4{0.f, 0.f, 0.f, 0.f};
          // K operand of key block tb, k-step ks: row r = 16 tb + l16, chunk
          // 4 ks + lg (latent for ks < 16, rotary after), at its swizzled
          // position.  With xh = l16 >> 2 < 4: cpos(r, 4 ks + lg) * 16 =
          // ((ks ^ xh) << 6) + ((lg ^ l16) & 3) * 16, and (ks0 + i) ^ xh =
          // ((ks0 + (i & 3)) ^ xh) + 4 (i >> 2); so four per-lane bases cover
          // every k-step, the rest is an immediate offset.  rpos(r, j) = j ^
          // ((l16 >> 1) & 7).  The swizzle key is opaque per tile so these
          // bases are recomputed per tile rather than held across the loop.
          int xs = l16;
          asm volatile("" : "+v"(xs));
          const char* cbase = cs + l16 * kCBytes + (((lg ^ xs) & 3) << 4);
          const char* cb4[4];
#pragma unroll
          for (int n = 0; n < 4; ++n) cb4[n] = cbase + (((ks0 + n) ^ (xs >> 2)) << 6);
          const char* rbase = rs + l16 * kRBytes;
          const int xr = (xs >> 1) & 7;
          auto kop = [&](int i, int tb) -> bf16x8 {  // k-step ks0 + i
            if (ks0 + i < kDc / 32) return *(const bf16x8*)(cb4[i & 3] + tb * 16 * kCBytes + (i >> 2) * 256);
            return *(const bf16x8*)(rbase + tb * 16 * kRBytes + (((4 * (ks0 + i - kDc / 32) + lg) ^ xr) << 4));
          };
          // K operands are read kPre k-steps ahead of their MFMAs (one with two
          // row blocks per wave: eight MFMAs per k-step hide the read, and the
          // registers are needed for the query)
          constexpr int kPre = QBW == 2 ? 1 : 2;
          bf16x8 ak[kPre + 1][2];
#pragma unroll
          for (int i = 0; i < kPre; ++i)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) ak[i][tb] = kop(i, tb);
#pragma unroll
          for (int i = 0; i < KMAX; ++i) {
            if (i < kcnt) {
              if (i + kPre < kcnt) {
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) ak[(i + kPre) % (kPre + 1)][tb] = kop(i + kPre, tb);
              }
              if (FAC && ks0 + i == kDc / 32) {
                // QK-Norm: the latent part so far takes the rows' factors
                // before the rotary k-steps add to it (they take none)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                  const f32x4 f = !rf_ok ? f32x4{1.f, 1.f, 1.f, 1.f} : tb ? rf1 : rf0;
#pragma unroll
                  for (int j = 0; j < QBW; ++j)
#pragma unroll
                    for (int hl = 0; hl < NACC; ++hl) sacc[tb][j][hl] *= f;
                }
              }
#pragma unroll
              for (int hl = 0; hl < NQH; ++hl)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                  for (int j = 0; j < QBW; ++j) {
                    const int ai = (NQH == 2 ? hl : i) % NACC;
                    sacc[tb][j][ai] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ak[i % (kPre + 1)][tb], qreg[hl][j][i], sacc[tb][j][ai], 0, 0, 0);
                  }
              if constexpr (LOC) {
                if (i >= KLAST - 2 && i < KLAST && rope_part) {
#pragma unroll
                  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int j = 0; j < QBW; ++j)
                      sacc[tb][j][(i + 1) % NACC] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                          ak[i % (kPre + 1)][tb], qlo[j][i - (KLAST - 2)], sacc[tb][j][(i + 1) % NACC], 0, 0, 0);
                }
              }
            }
          }
          f32x4 sc[2][QBW];  // partial scores of this wave's k-part
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int j = 0; j < QBW; ++j) {
              sc[tb][j] = sacc[tb][j][0];
              if constexpr (NACC > 1) sc[tb][j] += sacc[tb][j][1];
            }
          if constexpr (FAC) {
            // a k-part with no rotary step applies the factors here; then the
            // next tile's factors
            if (ks0 + kcnt <= kDc / 32 && rf_ok) {
#pragma unroll
              for (int j = 0; j < QBW; ++j) {
                sc[0][j] *= rf0;
                sc[1][j] *= rf1;
              }
            }
            if (it + 1 < n_tiles) rf_ok = load_rinv(it + 1, rr_next, rf0, rf1);
          }
          f32x4 sa, sb;  // scores of the softmax block rb, all k-steps
          f32x4* xb = (f32x4*)sm.xbuf;  // [slot][tb][lane]
          if constexpr (QBW == 1) {
            sa = sc[0][0];
            sb = sc[1][0];
            if constexpr (KS > 1) {
              // k-parts 1.. of the block write, k-part 0 adds them in order
              if (kp > 0) {
                xb[((rb * (KS - 1) + kp - 1) * 2 + 0) * 64 + lane] = sa;
                xb[((rb * (KS - 1) + kp - 1) * 2 + 1) * 64 + lane] = sb;
              }
              wait_lgkm0();
              barrier_raw();
              if (kp > 0) return;
#pragma unroll
              for (int j = 0; j < KS - 1; ++j) {
                sa += xb[((rb * (KS - 1) + j) * 2 + 0) * 64 + lane];
                sb += xb[((rb * (KS - 1) + j) * 2 + 1) * 64 + lane];
              }
            }
          } else {
            // two k-parts of a group of two blocks: each wave hands its partner
            // its partial of the partner's block and adds the partner's partial
            // of its own (part 0 + part 1 either way, so bitwise identical)
            static_assert(KS == 2 && QBW == 2, "pair layout");
            const int ob = grp * 2 + (1 - kp);  // the partner's block
            xb[(ob * 2 + 0) * 64 + lane] = kp == 0 ? sc[0][1] : sc[0][0];
            xb[(ob * 2 + 1) * 64 + lane] = kp == 0 ? sc[1][1] : sc[1][0];
            wait_lgkm0();
            barrier_raw();
            sa = (kp == 0 ? sc[0][0] : sc[0][1]) + xb[(rb * 2 + 0) * 64 + lane];
            sb = (kp == 0 ? sc[1][0] : sc[1][1]) + xb[(rb * 2 + 1) * 64 + lane];
          }
          sa *= sl2;
          sb *= sl2;
          if (!(t0 + kTile <= pr1 && t0 + kTile - 1 <= vis_min)) {  // partial or causal-edge tile
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = t0 + 4 * lg + e;
              sa[e] = (t < pr1 && t <= vis_last) ? sa[e] : -INFINITY;
              sb[e] = (t + 16 < pr1 && t + 16 <= vis_last) ? sb[e] : -INFINITY;
            }
          }
          float mt = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])),
                           fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])));
          mt = rows_max(mt);
          const bool need = mt > m_used + kTau;
          float alpha = 1.f;
          if (need) {
            alpha = __builtin_amdgcn_exp2f(m_used - mt);  // 0 when m_used was -inf
            m_used = mt;
            l_part *= alpha;
          }
          const bool any = __ballot(need) != 0;
          const float msub = m_used == -INFINITY ? 0.f : m_used;
          bf16x4 pa, pb;
          float lsum = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(sa[e] - msub);  // exp2(-inf) = 0
            const float p1 = __builtin_amdgcn_exp2f(sb[e] - msub);
            lsum += p0 + p1;
            pa[e] = (bf16)p0;
            pb[e] = (bf16)p1;
          }
          l_part += lsum;
          char* prow = sm.p[buf] + qrow * kPStr + 4 * lg * 2;
          *(bf16x4*)(prow) = pa;
          *(bf16x4*)(prow + 32) = pb;
          if (lg == 0) sm.alpha[buf][qrow] = alpha;
          if (lane == 0) sm.flag[buf][rb] = any ? 1 : 0;
        };

        // QK-Norm factors of the tile being scored (1 without QK-Norm)
        f32x4 rf0 = f32x4{1.f, 1.f, 1.f, 1.f}, rf1 = rf0;
        bool rf_ok = false;
        if constexpr (FAC) rf_ok = load_rinv(0, rinv_row(0), rf0, rf1);
        // tile 0 is in LDS after the first barrier (the PV waves load)
        barrier_raw();
        score_tile(0, rf0, rf1, rf_ok);
        for (int it = 0; it < n_tiles; ++it) {
          // before barrier `it`: P(it) is written; tile it+1 is in LDS
          wait_lgkm0();
          barrier_raw();
          if (it + 1 < n_tiles) score_tile(it + 1, rf0, rf1, rf_ok);
        }
        // epilogue: 1/l of this row block's rows, and the lse
        const float lt = rows_sum(l_part);
        const float linv = lt > 0.f ? 1.f / lt : 0.f;
        if (smax_wave && lg == 0) sm.rowinv[qrow] = linv;
        const int64_t lse_i = ((int64_t)b * s_q * n_heads + q_off) * n_part + part_begin + slot;
        if constexpr (LOC) {
          // While the PV waves finish the last tile: the lo parts of the latent
          // query rows, lo = q - bf16(q) in bf16, into two free latent stages
          // (rows 0..31 / 32..63, 16-byte chunks swizzled like the tiles).
          // Score wave w takes rows 16 w .. 16 w + 15, four at a time.
          char* const lo_a = sm.cst[n_tiles % G::NST];
          char* const lo_b = sm.cst[(n_tiles + 1) % G::NST];
#pragma unroll 1
          for (int r4 = 0; r4 < MT / 4; r4 += 4)
#pragma unroll
            for (int rr = r4; rr < r4 + 4; ++rr) {
              const int r = (wave_s & 3) * (MT / 4) + rr;
              *(bf16x8*)((r < 32 ? lo_a : lo_b) + (r & 31) * kCBytes + ((lane ^ (r & 15)) << 4)) = lo_row(r);
            }
        } else {
          if (smax_wave && lg == 0 && rvalid) lse_part[lse_i] = lt > 0.f ? (m_used + __log2f(lt)) * kLn2 : -INFINITY;
        }
        wait_lgkm0();
        barrier_raw();
        wait_lgkm0();
        barrier_raw();  // the PV waves have written their lse corrections
        if constexpr (LOC) {
          // lse = ln sum exp(s_hi) + scale * sum_d lo_d o_d: the first-order
          // change of the log-sum-exp when the latent scores gain scale lo . c_t
          // (exact to second order in that term, ~1e-5 here)
          if (smax_wave && lg == 0 && rvalid) {
            const float* corr = (const float*)sm.xbuf;  // [PV wave][row]
            const float c = (corr[qrow] + corr[MT + qrow]) + (corr[2 * MT + qrow] + corr[3 * MT + qrow]);
            lse_part[lse_i] = lt > 0.f ? (m_used + __log2f(lt)) * kLn2 + scale * linv * c : -INFINITY;
          }
        }
      } else {
        // ---- PV wave (waves 4..7): 128 latent columns of all rows, and all tile loads ----
#pragma unroll
        for (int t = 0; t < G::AHEAD; ++t)
          if (t < n_tiles) load_tile(t);
        f32x4 acc_o[8][NRB];
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int q = 0; q < NRB; ++q) acc_o[db][q] = f32x4{0.f, 0.f, 0.f, 0.f};

        // O^T[d x rows] += C^T . P^T of one tile (stage `st`, P / alpha / flags
        // of its buffer) for this wave's 128 columns, with this wave's loads of
        // a later tile (into `dma_dst`) spread over the column blocks.  The LDS
        // operands arrive as restrict pointers: the compiler then knows that the
        // transposed reads never touch the stage being loaded and does not make
        // them wait for every load in flight.
        auto pv_tile = [&](const char* __restrict__ st, const char* __restrict__ pbuf,
                           const float* __restrict__ alph, const int* __restrict__ flg,
                           char* __restrict__ dma_cdst, char* __restrict__ dma_rdst, const char* dma_src,
                           int dma_lim, bool with_dma, bool with_x) {
          const TileDma dma{dma_cdst, dma_rdst, dma_src, dma_lim};
          // all C^T operands of the tile first (16 transposed reads in flight),
          // then P, the rescale flags and factors
          const int rq = l16 >> 2, qq = lane & 3;
          bf16x8 ac[8];
          // lane (16 lg + 4 rq + qq) reads 4 bf16 of rows r0 = 8 lg + rq and r0 + 4
          // at latent column 128 pw + 16 db + 4 qq, i.e. chunk c = 16 pw + 2 db +
          // qq / 2; with x = r & 15 (< 16, bit 2 clear for r0):
          // cpos(r, c) = 16 pw + 2 (db ^ (x >> 1)) + ((qq >> 1) ^ (x & 1)).
          // The swizzle key is opaque per tile (no hoisted addresses).
          const int r0 = 8 * lg + rq;
          int x0 = r0 & 15;
          asm volatile("" : "+v"(x0));
          const int x1 = x0 ^ 4;  // (r0 + 4) & 15
          const char* p0 = st + r0 * kCBytes + 256 * pw + 8 * (qq & 1) + (((qq >> 1) ^ (x0 & 1)) << 4);
          const char* p1 = st + (r0 + 4) * kCBytes + 256 * pw + 8 * (qq & 1) + (((qq >> 1) ^ (x1 & 1)) << 4);
          const int h0 = x0 >> 1, h1 = x1 >> 1;
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + ((db ^ h0) << 5)));
            const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p1 + ((db ^ h1) << 5)));
            ac[db] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          }
          int flag = 0;
#pragma unroll
          for (int r = 0; r < NRB; ++r) flag |= flg[r];
          bf16x8 bq[NRB];
#pragma unroll
          for (int q = 0; q < NRB; ++q) bq[q] = *(const bf16x8*)(pbuf + (16 * q + l16) * kPStr + lg * 16);
          // five of this wave's loads of a later tile while those reads are in
          // flight (an LDS-direct load holds the wave at issue), the other four
          // between the MFMAs
          int dlane = lane;
          asm volatile("" : "+v"(dlane));
          constexpr int kW = dma_per_wave();
          constexpr int kFirst = kW - 4;  // the rest go between the MFMAs (db = 0, 2, 4, 6)
          if (with_dma) {
#pragma unroll
            for (int i = 0; i < kFirst; ++i) issue_dma_fast<UNI>(dma, pw, i, dlane);
          }

          if (flag) {
#pragma unroll
            for (int q = 0; q < NRB; ++q) {
              const float al = alph[16 * q + l16];
#pragma unroll
              for (int db = 0; db < 8; ++db) acc_o[db][q] *= al;
            }
          }
          // the MFMAs, with loads 5..8 issued between them
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            // the score waves' mid-tile exchange barrier (their next tile): half
            // of this tile's MFMAs and loads overlap their QK, half their softmax
            if (db == 4 && with_x) barrier_raw();
            if (with_dma && db % 2 == 0) issue_dma_fast<UNI>(dma, pw, kFirst + db / 2, dlane);
#pragma unroll
            for (int q = 0; q < NRB; ++q)
              acc_o[db][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ac[db], bq[q], acc_o[db][q], 0, 0, 0);
          }
        };

        // tile 0 must be in LDS; tiles 1 .. AHEAD-1 may still be in flight
        wait_tiles(min(n_tiles - 1, G::AHEAD - 1), min(n_tiles - 1, G::AHEAD - 1) < n_tiles - 1 || last_full);
        wait_lgkm0();
        barrier_raw();
        if constexpr (KS > 1) barrier_raw();  // the score waves' exchange of tile 0
        for (int it = 0; it < n_tiles; ++it) {
          // before barrier `it`: tile it+1 is in LDS (tile it+2 may be in flight)
          if (it + 1 < n_tiles) {
            const int issued = min(it + G::AHEAD - 1, n_tiles - 1);
            wait_tiles(issued - (it + 1), issued < n_tiles - 1 || last_full);
          }
          wait_lgkm0();
          barrier_raw();
          // tile it+AHEAD goes into the stage of tile it-1, free after its PV
          const bool with_dma = it + G::AHEAD < n_tiles;
          const TileDma dma = with_dma ? tile_dma(it + G::AHEAD)
                                       : TileDma{sm.cst[(it + G::AHEAD) % G::NST], sm.rst[(it + G::AHEAD) % G::NRST],
                                                 cache, 0};
          const int buf = it & 1;
          pv_tile(sm.cst[it % G::NST], sm.p[buf], sm.alpha[buf], sm.flag[buf], dma.cdst, dma.rdst, dma.src,
                  dma.lim, with_dma, KS > 1 && it + 1 < n_tiles);
        }
        wait_lgkm0();
        barrier_raw();
        {
          const char* const lo_a = sm.cst[n_tiles % G::NST];
          const char* const lo_b = sm.cst[(n_tiles + 1) % G::NST];
#pragma unroll
          for (int q = 0; q < NRB; ++q) {
            const int qr = 16 * q + l16;
            const float inv = sm.rowinv[qr];
            if constexpr (LOC) {
              // this wave's part of sum_d lo_d acc_d for row qr: lane holds
              // columns 128 pw + 16 db + 4 lg + (0..3), chunk 16 pw + 2 db + lg / 2
              const char* lrow = (qr < 32 ? lo_a : lo_b) + (qr & 31) * kCBytes + ((lg & 1) << 3);
              float cs = 0.f;
#pragma unroll
              for (int db = 0; db < 8; ++db) {
                const bf16x4 l4 = *(const bf16x4*)(lrow + (((16 * pw + 2 * db + (lg >> 1)) ^ (qr & 15)) << 4));
#pragma unroll
                for (int e = 0; e < 4; ++e) cs += (float)l4[e] * acc_o[db][q][e];
              }
              cs = rows_sum(cs);
              if (lg == 0) ((float*)sm.xbuf)[pw * MT + qr] = cs;
            }
            if (qr < nrows && inv > 0.f) {
              const int R = row0 + qr;
              const int tok = b * s_q + R / hc;
              const int h = head_begin + R % hc;
              const int64_t o = (((int64_t)tok * n_heads + h) * n_part + part_begin + slot) * kDc + 128 * pw +
                                4 * lg;
#pragma unroll
              for (int db = 0; db < 8; ++db) store_part4(o_part, o + 16 * db, acc_o[db][q] * inv, part_bf);
            }
          }
        }
        wait_lgkm0();
        barrier_raw();  // corrections written; stage buffers, P and rowinv are reused by the next piece
      }
    }
    __syncthreads();
    if (done) break;
  }
}

// Row groups of at most 64 query rows: 64 keeps each wave's half of the query
// block, its O columns and the scores in registers without spilling.
static int row_tile(int rows_total) { return rows_total <= 16 ? 16 : rows_total <= 32 ? 32 : 64; }

int decode_bf16_tile(int rows_total) { return rows_total > 32 ? decode_rows_tile(rows_total) : row_tile(rows_total); }

void decode_bf16_grid(int rows_total, int mt, int n_wg, int* n_share, int* n_rg) {
  *n_rg = (rows_total + mt - 1) / mt;
  int ns = n_wg;
  if (*n_rg > 1) {
    ns = (n_wg / *n_rg) / 8 * 8;  // multiple of 8: the row groups of a share share an XCD
    if (ns < 8) ns = 8;
  }
  *n_share = ns < 1 ? 1 : ns;
}

template <bool QF32, bool QKN>
static hipError_t launch_mt(const DecodeArgs& a, int mt, dim3 grid, int n_share, int n_rg, int rows_total,
                            hipStream_t stream) {
  const dim3 block(kThreads);
  switch (mt) {
    case 16:
      return launch((decode_bf16_kernel<16, QF32, QKN>), grid, block, stream, a, n_share, n_rg, rows_total);
    case 32:
      return launch((decode_bf16_kernel<32, QF32, QKN>), grid, block, stream, a, n_share, n_rg, rows_total);
    default:
      return launch((decode_bf16_kernel<64, QF32, QKN>), grid, block, stream, a, n_share, n_rg, rows_total);
  }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int n_wg, bool q_f32, hipStream_t stream) {
  const int rows_total = a.s_q * a.seg.head_count;
  // more than 32 query rows with an fp32 query (with or without QK-Norm row
  // factors): whole rows per wave (mla_decode_rows.hip)
  if (rows_total > 32 && q_f32) return launch_decode_rows(a, n_wg, stream);
  const int mt = row_tile(rows_total);
  int n_share, n_rg;
  decode_bf16_grid(rows_total, mt, n_wg, &n_share, &n_rg);
  const dim3 grid(n_share * n_rg);
  // the QK-Norm variant exists for an fp32 query only (checked by the caller)
  if (q_f32 && a.seg.row_rinv) return launch_mt<true, true>(a, mt, grid, n_share, n_rg, rows_total, stream);
  if (q_f32) return launch_mt<true, false>(a, mt, grid, n_share, n_rg, rows_total, stream);
  return launch_mt<false, false>(a, mt, grid, n_share, n_rg, rows_total, stream);
}

}  // namespace mla
