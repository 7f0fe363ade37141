// Absorbed MLA decode over a bf16 latent cache for row groups of 64 and 128
// query rows, gfx950: every wave owns whole query rows.
//
// What it computes (MLA tutorial page, "Move the Key Projection Into the
// Query", "Position Rotations Complicate the Absorption", "Move the Value
// Expansion After the Weighted Sum"; RedKnot-MLA abstract for the segments):
// for each query row (token s, head h) of a segment and a contiguous range of
// cache rows t of one request,
//   s_t = scale * ([q_lat | q_rot] . [c_t | kr_t]),  p = softmax over the range,
//   o_part = sum_t p_t c_t  (fp32, normalised),  lse_part = ln sum_t exp(s_t).
//
// Design (MI355X: 256 CUs of 4 SIMDs, 160 KiB LDS and 512 KiB of registers
// per CU, 64-lane waves):
//  * One workgroup of 4 waves, one per SIMD, owns MT = 64 RB query rows (all
//    heads of a request for the segment, or a group of them); wave w owns rows
//    16 RB w .. + 16 RB - 1 completely: its query in registers, the scores of
//    its rows, their softmax, and their 512 output columns (RB = 2: 256
//    accumulator registers).  Nothing crosses between waves but the cache
//    tiles, so the only workgroup barrier is the one that recycles a ring
//    stage, once per tile.
//  * Cache rows stream in 32-row tiles [c_t | kr_t] (1152 B per row) HBM ->
//    LDS with direct-to-LDS loads: a 4-stage latent ring and a 3-stage rotary
//    ring; each wave issues a quarter of every tile's loads.  Each tile is
//    read from HBM once and serves all MT rows: for the 128 heads of a
//    DeepSeek-V3-style request that is every head at once.
//  * A wave's tile step, for its 16 RB rows, on v_mfma_f32_16x16x32_bf16:
//    QK:  S^T[32 tokens x rows] = K_tile . q^T over the 18 k-steps of [c | kr]
//         (K operand: one 16-byte LDS read per 16 tokens per k-step, shared by
//         the wave's RB row blocks);
//    PV:  O^T[512 columns x rows] += C_tile^T . P^T (C^T from two
//         ds_read_b64_tr_b16 transposed reads per 16 columns, shared by the RB
//         row blocks).
//    The softmax needs no data movement: the score accumulators hold, per
//    lane, query row l % 16 and tokens 4 (l / 16) + e and 16 + 4 (l / 16) + e,
//    and that is exactly the P^T operand of the PV product once its k order
//    is defined as those tokens (the transposed C reads are addressed to
//    match).
//  * Software pipeline, per iteration `it` after the ring barrier: the QK of
//    tile it+1, then the PV of tile it with the softmax of tile it+1 between
//    its MFMAs (the softmax of it+1 does not feed the PV of it), then the
//    rare lazy rescale of O.  So the score chain, the softmax's dependent
//    VALU/transcendental chain and both products share one instruction stream
//    per SIMD without waiting on one another.
//  * Query precision: the query is split into bf16 hi and lo parts (q_rot
//    here, from fp32; q_lat here too, or by the producer, which then stores
//    the two parts as planes so that the prologue reads only the hi plane
//    and the epilogue only the lo plane: half the bytes of the fp32 query
//    each).  The latent part is multiplied as hi only; the rotary part as
//    hi + lo.  With delta_t = lo . c_t the neglected part of a latent
//    score, log sum exp(s_t + delta_t) = lse + sum_t p_t delta_t +
//    O(var_p delta), so the lse gains scale * lo . o (o = the normalised
//    weighted latent, which each wave holds for its rows), leaving a
//    second-order error (about 1e-5 at unit-variance inputs).  The scores
//    are q . k; the softmax scale (times log2 e) enters in its exponent.
//  * Softmax in the exp2 domain with lazy rescaling: the running max moves
//    only when a tile max exceeds it by more than kRowsTau (log2 units), so
//    the O rescale almost never runs; when it does, it runs outside the tile
//    loop.
//  * Work split: the segment's rows, concatenated over requests (each padded
//    to whole tiles), are cut into equal shares, one per workgroup of a row
//    group; a share crossing request boundaries yields several pieces, each
//    written to its own partial slot (at most n_split per request; unused
//    slots get lse = -inf).  The workgroup's first wave derives the pieces from
//    seq_lens on the device.
//  * Grid: n_share workgroups per row group; the row groups of one share sit
//    on the same XCD (workgroups are dispatched round-robin over 8 XCDs), so
//    the second read of a tile hits that XCD's L2.
//  * Several segments (the offline document, the recomputed document and the
//    online tokens of the RedKnot-MLA abstract) share one launch: each gets a
//    range of workgroups sized so that all finish together under a per-tile
//    cost model, and the HBM-bound and MFMA-bound segments run side by side.
//    Within a range the shares in whole octets keep the XCD placement above;
//    the last n_share % 8 shares are placed in order.
//  * A wave whose 16 RB rows are all past the group (a group of fewer rows
//    than the workgroup holds) only moves its share of each tile and skips
//    the products, leaving the LDS and the other SIMDs' issue to the waves
//    with rows.
//  * Low-bit rows (QuantMLA abstract; 64-row groups): int8 latent codes with
//    16-bit rotary entries, or int4 latent and rotary codes, land packed in
//    LDS and every wave unpacks its 8 rows of a tile into the bf16 stages
//    (the codes are exact in bf16) one tile before their scores; the row
//    scales multiply the scores after the QK product and the weights before
//    the PV product, so the PV sums weights times dequantized rows.
//  * QK-Norm (QK-Norm MLA abstract; 16-bit rows): each stored row carries the
//    inverse RMS of its content key.  A tile's 32 factors come with its loads
//    (one more 4-byte load per wave) and multiply the latent part of the
//    scores, the rotary part apart, as the int8 scales do; they do not touch
//    the PV weights (the values are the plain latents).  The lo part's lse
//    share then carries each token's factor: the kernel also sums weights
//    times factors and takes the share as the weighted mean factor times
//    scale * lo . o, leaving the weighted covariance of the factors and the
//    lo scores, a second-order term.
#include "mla_common.h"
#include "mla_decode_tile.h"
#include "mla_kernels.h"

#include <algorithm>
#include <climits>
#include <cmath>

namespace mla {
namespace {

constexpr int kRowsThreads = 256;      // 4 waves, one per SIMD
constexpr int kRowsWaves = kRowsThreads / 64;
// Loads in flight: a CU's memory queue takes about one tile of direct-to-LDS
// loads (36 KiB) at a time, and a load issued into a full queue stalls the
// issuing wave until space frees up (measured: about 3.4k cycles per tile
// per CU at one workgroup per CU, 5.7-6 TB/s in all, with one tile or more in
// flight).  One tile ahead leaves the latency exposed behind one iteration of
// compute; so tile it+3 goes out during the PV of tile it, by when the loads
// of tile it+2 (issued one iteration earlier) have drained, and has about
// 1.5 iterations to land.
constexpr int kLatStages = 4;          // tiles it (PV), it+1 (QK), it+2, it+3 (loading)
constexpr int kRotStages = 3;          // tiles it+1 (QK), it+2, it+3
constexpr int kLoadAhead = 3;          // tiles issued before the first QK
constexpr int kTileDma = kTile + kRStage / 1024;       // 36 wave-instructions per tile
constexpr int kDmaPerWave = kTileDma / kRowsWaves;     // 9
static_assert(kTileDma % kRowsWaves == 0, "every wave issues the same share of a tile's loads");
constexpr int kRowsMaxPieces = 64;
// Cost of a piece beyond its tiles, in tiles: its prologue reads the query
// of the group's rows (fp32 latent and rotary parts, or a split query's hi
// plane and the fp32 rotary part), its epilogue reads the latent part again
// (the split query's lo plane) and writes the partial output, all at the
// CU's share of HBM bandwidth like the cache tiles (measured at 128-row
// groups: about 19 tiles with an fp32 query, as the bytes predict; 13.6 +
// 17.4 us against 2.2 us per tile, about 14, with a split query, whose bytes
// give 12).  The work split counts this many extra tiles at the start of
// every request, so a workgroup whose range crosses a request boundary (two
// pieces) takes correspondingly fewer rows.
__host__ __device__ constexpr int piece_tiles(int mt, bool part_bf16, bool q_split) {
  const int q_bytes = q_split ? kDc * 2 + kDr * 4 + kDc * 2 : (kDc + kDr) * 4 + kDc * 4;
  return (mt * (q_bytes + kDc * (part_bf16 ? 2 : 4)) + kTile * kRowBytes / 2) / (kTile * kRowBytes);
}
// Operand reads in flight ahead of their MFMAs (deeper with 16 rows per wave,
// which has registers to spare and fewer MFMAs per read to cover latency)
template <int RB> constexpr int kPvPre = RB == 1 ? 8 : 4;   // PV: column blocks of transposed reads
template <int RB> constexpr int kQkPre = RB == 1 ? 6 : 3;   // QK: k-steps of K-operand reads
// Lazy rescale threshold (log2 units): a row's running max moves only when a
// tile's max exceeds it by more than this, so weights reach 2^32 at most.
// bf16 weights and fp32 sums keep their relative precision at any magnitude
// and stay far from overflow (2^32 times 32768 rows times the largest cache
// entry), while the rescale of O, which leaves the tile loop, almost never
// runs.
constexpr float kRowsTau = 32.f;

// Instruction order of the scheduling regions of a tile step, for the
// compiler's scheduler (which otherwise issues each LDS read just before its
// MFMA and waits for it).  Groups of instruction kinds are filled in order:
constexpr int kSchedDs = 0x080, kSchedMfma = 0x008;

// int4 rows (the QuantMLA abstract's joint INT4 content and rotary caches):
// 256 bytes of latent codes and 32 of rotary codes per stored row, two fp32
// scales per row beside the cache.  A tile's codes (9 KiB) and scales land in
// LDS by direct loads, two tiles ahead; each wave then unpacks 8 of its rows
// into the bf16 stages (the codes themselves, exact small integers), one tile
// ahead of the scores, and keeps its own copy of the tile's scales.
constexpr int kI4Row = (kDc + kDr) / 2;                 // 288 bytes per stored row
constexpr int kI4Codes = kTile * kI4Row;                // 9 KiB of codes per tile
constexpr int kI4Land = kI4Codes + 256 * kRowsWaves;    // + one copy of the 32 scale pairs per wave
constexpr int kI4Dma = 4;                               // loads per wave per tile
static_assert(kI4Codes % (kRowsWaves * 256) == 0, "a wave's share of the codes is whole dword loads");

// int8 rows (the QuantMLA abstract's low-bit latent cache in its plain form):
// 512 bytes of latent codes and the 64 bf16 rotary entries per stored row,
// one fp32 scale per row beside the cache.  A tile's codes (16 KiB) and
// scales land in LDS by direct loads one tile ahead of their unpacking (two
// landing stages: a third does not fit beside the bf16 stages), its rotary
// entries go straight into the rotary ring like 16-bit rows; each wave then
// unpacks 8 of its rows into the bf16 stages (the codes, exact in bf16) and
// keeps its own copy of the tile's scales.
constexpr int kI8Row = kDc + 2 * kDr;                   // 640 bytes per stored row
constexpr int kI8Codes = kTile * kDc;                   // 16 KiB of codes per tile
constexpr int kI8Land = kI8Codes + 256 * kRowsWaves;    // + one copy of the 32 scales per wave
constexpr int kI8Dma = 6;                               // loads per wave per tile

// QM: the stored rows (0: 16-bit, 1: int4, 2: int8).  Low-bit rows land
// packed and are unpacked into three bf16 stages: tiles it (PV), it+1 (QK)
// and it+2 (unpacked into).
template <int QM, int RB, bool QKN>
struct RowsSmem {
  static constexpr int NLAT = QM ? 3 : kLatStages;
  static constexpr int NLAND = QM == 1 ? 3 : QM == 2 ? 2 : 1;
  static constexpr int LAND = QM == 1 ? kI4Land : QM == 2 ? kI8Land : 16;
  char lat[NLAT][kCStage];   // 128 KiB (96 KiB)
  char rot[kRotStages][kRStage];   // 12 KiB
  // bf16 hi parts of the rotary query of the group's rows (a wave uses only
  // its own rows): rows of 128 B, chunks placed like the rotary ring's
  char qrot[16 * RB * kRowsWaves][kRBytes];  // 16 KiB at 128-row groups
  char land[NLAND][LAND];    // int4: 30 KiB landing ring, int8: 34 KiB
  float scl[QM ? 3 : 1][kRowsWaves][QM == 1 ? 2 * kTile : QM == 2 ? kTile : 1];  // each wave's scales of a stage
  // QK-Norm: the row factors of the tiles in flight (one shared copy per
  // stage; entries 32..63 take the zeros of lanes past the tile)
  float rinv[QKN ? 3 : 1][QKN ? 64 : 1];
  Piece pieces[kRowsMaxPieces];
  int n_pieces;
  int done;
  int red[4 * kRowsWaves];
};

// Direct-to-LDS buffer load of 16 bytes per lane: LDS address = lds + 16 *
// lane, memory address = the resource's base + voffset.  A lane whose bytes
// lie past the resource's record count reads zeros, so a partial tile (or a
// page outside the pool, record count 0) needs no branch and no zero-fill
// store: its rows arrive as zeros.  Written as asm so that the compiler does
// not order later LDS reads of *other* ring stages behind these loads (it
// cannot tell the stages apart and would drain every load in flight); the
// kernel waits for each tile itself (vmcnt, in order) before the barrier
// that publishes it.  No register is written; M0 takes the LDS address, one
// wait state before the load reads it.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// int in the constant address space: uniform reads become scalar loads
typedef const __attribute__((address_space(4))) int32_t CInt;
__device__ __forceinline__ void dma16(i32x4_t rsrc, const char* lds, int voffset) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(MLA_LDS const char*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// The 4-byte form: LDS address = lds + 4 * lane.
__device__ __forceinline__ void dma4(i32x4_t rsrc, const char* lds, int voffset) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(MLA_LDS const char*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// Buffer resource over `bytes` bytes at `base` (stride 0, raw addressing;
// the third dword is the gfx9-family data-format word).
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xffff, bytes, 0x00020000};
}

// Latent rows in LDS: the 16-byte chunk c (0..63) of tile row r sits at
// position c ^ lkey(r), lkey(r) = 2 (r & 7) (rotary rows keep rpos).  The LDS
// serves a ds_read_b128 16 lanes per cycle (lanes 32 h + 4 q .. 32 h + 4 q + 3
// for the four quads q of equal bit parity) and a ds_read_b64, the transposed
// form too, 32 consecutive lanes per cycle, over 64 banks of 4 bytes (bank
// conflict counters of single lane pairs and of whole patterns).  With this
// key both operand reads below reach 64 distinct banks per cycle; the key
// r & 15 left every transposed read two-way conflicted.
__device__ __forceinline__ int lkey(int r) { return (r & 7) << 1; }
__device__ __forceinline__ int lpos(int r, int c) { return c ^ lkey(r); }

// Load i (< kDmaPerWave) of wave w's share of one tile, from the rows that
// `rsrc` covers (rows past its record count read as zeros).  Wave w fills
// latent rows k = w + 4 i (i < 8; lane l moves the chunk stored at position
// l, i.e. chunk lpos(k, l)) and, as its last load, rotary rows 8 w + l / 8
// (lane l: position l % 8, chunk (l % 8) ^ ((r >> 1) & 7)).
__device__ __forceinline__ void tile_load(i32x4_t rsrc, char* lat, char* rot, int w, int lane, int i) {
  // opaque lane copy: the offsets are recomputed per instruction instead of
  // being hoisted into registers held across the tile loop
  asm volatile("" : "+v"(lane));
  if (i < kTile / kRowsWaves) {
    const int k = w + kRowsWaves * i;
    dma16(rsrc, lat + k * kCBytes, k * kRowBytes + (lpos(k, lane) << 4));
  } else {
    const int r = 8 * w + (lane >> 3);
    dma16(rsrc, rot + w * 1024, r * kRowBytes + kCBytes + (rpos(r, lane & 7) << 4));
  }
}

// Wave w's kI4Dma loads of an int4 tile: bytes [2304 w, 2304 w + 2304) of its
// codes (two 16-byte and one 4-byte load per lane) and its 32 scale pairs
// (256 bytes, into the wave's own copy).
__device__ __forceinline__ void tile_load_i4(i32x4_t codes, i32x4_t scales, char* land, int w, int lane) {
  asm volatile("" : "+v"(lane));
  const int base = w * (kI4Codes / kRowsWaves);
  dma16(codes, land + base, base + 16 * lane);
  dma16(codes, land + base + 1024, base + 1024 + 16 * lane);
  dma4(codes, land + base + 2048, base + 2048 + 4 * lane);
  dma4(scales, land + kI4Codes + 256 * w, 4 * lane);
}

// Eight packed 4-bit codes (entry e in bits 4 e .. 4 e + 3, two's complement)
// as bf16 codes / 16 (exact; the scales carry the factor 16).  The gfx9
// signed-nibble conversion takes bits 0..3 of a byte picked by SDWA: entry
// 2k from byte k of the word, entry 2k + 1 from byte k of the word shifted
// right by 4.
template <int K>
__device__ __forceinline__ float nib16(uint32_t w) {
  float r;
  if constexpr (K == 0)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w));
  else if constexpr (K == 1)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
  else if constexpr (K == 2)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
  else
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}
constexpr float kI4Unit = 16.f;  // unpacked value = code / kI4Unit
__device__ __forceinline__ bf16x8 unpack8_i4(uint32_t wd) {
  const uint32_t hi = wd >> 4;
  bf16x8 r;
  r[0] = (bf16)nib16<0>(wd);
  r[1] = (bf16)nib16<0>(hi);
  r[2] = (bf16)nib16<1>(wd);
  r[3] = (bf16)nib16<1>(hi);
  r[4] = (bf16)nib16<2>(wd);
  r[5] = (bf16)nib16<2>(hi);
  r[6] = (bf16)nib16<3>(wd);
  r[7] = (bf16)nib16<3>(hi);
  return r;
}

// Wave w unpacks rows 8 w .. 8 w + 7 of a landed int4 tile into the bf16
// stages (latent: lane l = chunk l of each row; rotary: lane l = row 8 w +
// l / 8, chunk l % 8) and copies the tile's scales (its own landed copy) to
// its scale slot of the stage.
__device__ __forceinline__ void unpack_tile_i4(const char* __restrict__ land, char* __restrict__ lat,
                                               char* __restrict__ rot, float* __restrict__ scl, int w, int lane) {
  asm volatile("" : "+v"(lane));
  // every read first (the landing stage and the bf16 stages never overlap),
  // then the conversions and writes
  const int rr = 8 * w + (lane >> 3), j = lane & 7;
  uint32_t wd[9];
#pragma unroll
  for (int i = 0; i < 8; ++i) wd[i] = *(const uint32_t*)(land + (8 * w + i) * kI4Row + 4 * lane);
  wd[8] = *(const uint32_t*)(land + rr * kI4Row + kDc / 2 + 4 * j);
  const float sv = *(const float*)(land + kI4Codes + 256 * w + 4 * lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * w + i;
    *(bf16x8*)(lat + r * kCBytes + (lpos(r, lane) << 4)) = unpack8_i4(wd[i]);
  }
  *(bf16x8*)(rot + rr * kRBytes + (rpos(rr, j) << 4)) = unpack8_i4(wd[8]);
  scl[lane] = sv;
}

// Wave w's kI8Dma loads of an int8 tile: the codes of rows 8 w .. 8 w + 7 (two
// rows per load, into the landing stage row by row), their rotary entries
// (into the rotary ring, placed as for 16-bit rows) and the tile's 32 scales
// (into the wave's own copy; lanes past the record count read zeros).
__device__ __forceinline__ void tile_load_i8(i32x4_t rows, i32x4_t scales, char* land, char* rot, int w,
                                             int lane) {
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * w + 2 * j + (lane >> 5);
    dma16(rows, land + (8 * w + 2 * j) * kDc, r * kI8Row + 16 * (lane & 31));
  }
  const int r = 8 * w + (lane >> 3);
  dma16(rows, rot + w * 1024, r * kI8Row + kDc + (rpos(r, lane & 7) << 4));
  dma4(scales, land + kI8Codes + 256 * w, 4 * lane);
}

// Eight int8 codes (byte e = entry e, two's complement) as bf16, exact.
__device__ __forceinline__ bf16x8 unpack8_i8(uint32_t w0, uint32_t w1) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)(float)(int8_t)(w0 >> (8 * e));
    r[4 + e] = (bf16)(float)(int8_t)(w1 >> (8 * e));
  }
  return r;
}

// Wave w unpacks rows 8 w .. 8 w + 7 of a landed int8 tile into the bf16
// latent stage (lane l: chunk l, codes 8 l .. 8 l + 7, of each row) and
// copies the tile's scales (its own landed copy) to its scale slot.
__device__ __forceinline__ void unpack_tile_i8(const char* __restrict__ land, char* __restrict__ lat,
                                               float* __restrict__ scl, int w, int lane) {
  asm volatile("" : "+v"(lane));
  uint32_t wd[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 v = *(const uint2*)(land + (8 * w + i) * kDc + 8 * lane);
    wd[i][0] = v.x;
    wd[i][1] = v.y;
  }
  const float sv = *(const float*)(land + kI8Codes + 256 * w + 4 * lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * w + i;
    *(bf16x8*)(lat + r * kCBytes + (lpos(r, lane) << 4)) = unpack8_i8(wd[i][0], wd[i][1]);
  }
  if (lane < kTile) scl[lane] = sv;
}

// Score MFMAs with their accumulators in VGPRs.  Once any MFMA of a kernel
// keeps its accumulator in AGPRs (O does, all 256 of them at 32 rows per
// wave), the compiler selects the AGPR form for every MFMA, so the scores
// too would take AGPRs, and part of O would move to VGPRs and back on every
// tile.  Written as asm, the compiler sees no MFMA here and cannot insert
// the wait states that an MFMA result needs before a vector-ALU read;
// scores_ready() provides them (8, as the compiler gives this 16x16x32
// form) and orders every later read of the scores after them.  A chain of
// MFMAs into one accumulator needs none.
__device__ __forceinline__ void mfma_v(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v0(f32x4& c, const bf16x8& a, const bf16x8& b) {  // c = a . b
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(a), "v"(b));
}
template <int RB>
__device__ __forceinline__ void scores_ready(f32x4 (&s)[2][RB], f32x4 (&sr)[2][RB]) {
  asm volatile("s_nop 7" ::: "memory");
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) asm volatile("" : "+v"(s[tb][rb]), "+v"(sr[tb][rb]));
}

// Scores of one tile for the wave's RB row blocks: S^T[32 tokens x 16 rows]
// per block as two 16-token halves.  ls / rs: the tile's latent and rotary
// stages (restrict: the compiler may then order these reads freely against
// the direct-to-LDS loads in flight to other stages).  Per-lane LDS address
// parts, from an opaque copy of the lane index (so none is held across the
// loop): K operand of latent k-step ks = 4 a + n, rows 16 tb + l16, chunk
// 4 ks + lg, sits at position (4 ks + lg) ^ lkey(l16) = 16 a + 4 (n ^ (lkey
// >> 2)) + (lg ^ (lkey & 3)); rotary k-step jr: chunk 4 jr + lg at (4 jr +
// lg) ^ ((l16 >> 1) & 7).  Rows 16 + l16 share the swizzle key of row l16.
// The rotary k-steps accumulate into sr (the same array as s, except for int4
// rows, whose two parts take different scales).
template <int RB>
__device__ __forceinline__ void qk_tile(const char* __restrict__ ls, const char* __restrict__ rs,
                                        const char* __restrict__ qs, int lane, const bf16x8 (&qh)[RB][kDc / 32],
                                        const bf16x8 (&qrl)[RB][2], f32x4 (&s)[2][RB], f32x4 (&sr)[2][RB]) {
  asm volatile("" : "+v"(lane));
  const int xl = lane & 15, xg = lane >> 4;
  const char* kb[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) kb[n] = ls + xl * kCBytes + ((n ^ (lkey(xl) >> 2)) << 6) + ((xg ^ (lkey(xl) & 3)) << 4);
  const char* rb0 = rs + xl * kRBytes;
  const int xr = (xl >> 1) & 7;
  const bool split_rot = &sr[0][0] != &s[0][0];  // int4 rows: the rotary part apart
  // the rotary query's hi parts from LDS (row 16 rb + l16 of the wave's rows,
  // chunk 4 jr + lg, placed like the rotary ring), read kQrAhead latent
  // k-steps before they are needed, so that their latency hides behind those
  bf16x8 qrh[RB][2];
  constexpr int kQrAhead = 6;
  auto read_qrh = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int jr = 0; jr < 2; ++jr) {
        const int qr = 16 * rb + xl;
        qrh[rb][jr] = *(const bf16x8*)(qs + qr * kRBytes + (rpos(qr, 4 * jr + xg) << 4));
      }
  };
  // K operands of k-step ks (ks < 16 latent, then 2 rotary), read kPre
  // k-steps ahead of their MFMAs
  auto kop = [&](int ks, int tb) -> bf16x8 {
    if (ks < kDc / 32) return *(const bf16x8*)(kb[ks & 3] + (ks >> 2) * 256 + tb * 16 * kCBytes);
    return *(const bf16x8*)(rb0 + (((4 * (ks - kDc / 32) + xg) ^ xr) << 4) + tb * 16 * kRBytes);
  };
  constexpr int kPre = kQkPre<RB>;
  bf16x8 ka[kPre + 1][2];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    ka[i][0] = kop(i, 0);
    ka[i][1] = kop(i, 1);
  }
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    if (ks == kDc / 32 - kQrAhead) read_qrh();
    if (ks + kPre < kKSteps) {
      ka[(ks + kPre) % (kPre + 1)][0] = kop(ks + kPre, 0);
      ka[(ks + kPre) % (kPre + 1)][1] = kop(ks + kPre, 1);
    }
    const bf16x8 k0 = ka[ks % (kPre + 1)][0], k1 = ka[ks % (kPre + 1)][1];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (ks < kDc / 32) {
        if (ks == 0) {
          mfma_v0(s[0][rb], k0, qh[rb][ks]);
          mfma_v0(s[1][rb], k1, qh[rb][ks]);
        } else {
          mfma_v(s[0][rb], k0, qh[rb][ks]);
          mfma_v(s[1][rb], k1, qh[rb][ks]);
        }
      } else {
        const int jr = ks - kDc / 32;
        if (jr == 0 && split_rot) {
          mfma_v0(sr[0][rb], k0, qrh[rb][jr]);
          mfma_v0(sr[1][rb], k1, qrh[rb][jr]);
        } else {
          mfma_v(sr[0][rb], k0, qrh[rb][jr]);
          mfma_v(sr[1][rb], k1, qrh[rb][jr]);
        }
        mfma_v(sr[0][rb], k0, qrl[rb][jr]);
        mfma_v(sr[1][rb], k1, qrl[rb][jr]);
      }
    }
  }
  scores_ready<RB>(s, sr);
}

// O^T[512 columns x 16 rows] += C^T . P^T for the wave's RB row blocks.  The
// P^T operand of lane l holds its row's weights of tokens 4 lg + e (k = 8 lg
// + e) and 16 + 4 lg + e (k = 8 lg + 4 + e), exactly the lane's score
// registers; the C^T operand of column block db is read to match: the first
// transposed read of lane (lg, rq, qq) addresses tile row x = 4 lg + rq, the
// second row x + 16 (same swizzle key), columns 16 db + 4 qq .. + 3, i.e.
// chunk 2 db + (qq >> 1) at position 2 ((db & 7) ^ (lkey(x) >> 1)) + ((qq >> 1) ^
// (lkey(x) & 1)) (plus 16 (db >> 3)), byte 8 (qq & 1) within it; each 16-lane
// group then holds C[rows][16 db + l16].
// `load(i)` issues load i of the next tile's share after the MFMAs of column
// block kPvLoadAt[i]; `mid(db)` runs after those of block db (the next tile's
// softmax, in stages).  Each block's instructions stay in program order (a
// wave issues in order: vector-ALU work placed right after an MFMA issues
// while the MFMA runs).
constexpr int kPvLoadAt[9] = {1, 4, 8, 11, 15, 18, 22, 25, 29};
template <int RB, class Load, class Mid>
__device__ __forceinline__ void pv_tile(const char* __restrict__ ls, int lane, const bf16x8 (&p)[RB],
                                        f32x4 (&acc)[32][RB], const Load& load, const Mid& mid) {
  asm volatile("" : "+v"(lane));
  const int qq = lane & 3, rq = (lane >> 2) & 3, xg = lane >> 4;
  const int xr = 4 * xg + rq;
  const char* cb = ls + xr * kCBytes + 8 * (qq & 1) + 16 * ((qq >> 1) ^ (lkey(xr) & 1));
  const int xh = lkey(xr) >> 1;
  auto cop = [&](int db) -> bf16x8 {
    const char* pa = cb + 256 * (db >> 3) + (((db & 7) ^ xh) << 5);
    const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pa));
    const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pa + 16 * kCBytes));
    return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // C^T operands read kPvPre column blocks ahead of their MFMAs
  constexpr int kPre = kPvPre<RB>;
  bf16x8 ca[kPre + 1];
#pragma unroll
  for (int i = 0; i < kPre; ++i) ca[i] = cop(i);
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    if (db + kPre < 32) ca[(db + kPre) % (kPre + 1)] = cop(db + kPre);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      acc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[db % (kPre + 1)], p[rb], acc[db][rb], 0, 0, 0);
      asm("" : "+a"(acc[db][rb]));  // the accumulators live in AGPRs throughout
    }
    mid(db);
#pragma unroll
    for (int i = 0; i < 9; ++i)
      if (kPvLoadAt[i] == db) load(i);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// A tile's scores made ready for the softmax, in place.  Low-bit rows (QM):
// the score is s_c (latent part) + s_r (rotary part) with the row's scales,
// read from the wave's scale slot `tsc` of the tile (int4: pairs (s_c, s_r)
// per row; int8: s_c per row, the 16-bit rotary part unscaled); the latent
// scales (times the factor the unpacked codes lack) stay in `wsc` for the
// weights, which enter the PV product times them (the PV multiplies the
// codes).  Unless the whole tile is visible to every
// row of the wave (`full`), tokens past the piece or the row's causal limit
// (relative index `lim` per lane: token 4 lg + e of the first half is
// visible when e <= lim) get -inf, i.e. weight 0.  A branch on `full` is
// fine here: the softmax proper, which runs between the PV MFMAs, has none.
// QM == 2 (int8 rows: the row scale) and RF (QK-Norm: the row factor) scale
// the latent part of each score by the factor of its token; for int8 rows the
// scale also weights the token in the PV product (wsc), for QK-Norm it only
// enters the mean factor of the lse correction.
template <int RB, int QM, bool RF = false>
__device__ __forceinline__ void prep_scores(f32x4 (&s)[2][RB], const f32x4 (&sr)[2][RB], bool full,
                                            const int (&lim)[RB], const float* tsc, f32x4 (&wsc)[2]) {
  if constexpr (QM == 2 || RF) {
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
    const int lg4 = 4 * (ln >> 4);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const f32x4 sc = *(const f32x4*)(tsc + 16 * tb + lg4);  // tokens 4 lg .. 4 lg + 3 of the half
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wsc[tb][e] = sc[e];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[tb][rb][e] = sc[e] * s[tb][rb][e] + sr[tb][rb][e];
      }
    }
  }
  if constexpr (QM == 1) {
    int ln = __lane_id();
    asm volatile("" : "+v"(ln));
    const int lg4 = 4 * (ln >> 4);
    f32x4 sc[2][2];  // (tokens 4 lg .. 4 lg + 3 of each half) x (s_c, s_r) pairs
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sc[tb][0] = *(const f32x4*)(tsc + 2 * (16 * tb + lg4));
      sc[tb][1] = *(const f32x4*)(tsc + 2 * (16 * tb + lg4) + 4);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = kI4Unit * sc[tb][e >> 1][2 * (e & 1)], r = kI4Unit * sc[tb][e >> 1][2 * (e & 1) + 1];
        wsc[tb][e] = c;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[tb][rb][e] = c * s[tb][rb][e] + r * sr[tb][rb][e];
      }
  }
  if (!full) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[0][rb][e] = e <= lim[rb] ? s[0][rb][e] : -INFINITY;
        s[1][rb][e] = 16 + e <= lim[rb] ? s[1][rb][e] : -INFINITY;
      }
  }
}

// max of three (scores are finite or -inf, never NaN: no quieting of inputs,
// which fmaxf costs the compiler one extra instruction per operand here)
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// the max over the four lane groups of a row (lanes l, l + 16, l + 32, l + 48)
__device__ __forceinline__ float rows_max_raw(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max3_raw(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max3_raw(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[1]));
}

// Online softmax of one tile's prepared scores (q . k, before the softmax
// scale), in the exp2 domain: weights 2^(sl2 s - m) with sl2 = scale * log2 e,
// with lazy rescaling: the P^T operands (bf16), the factor each row's O must
// take and whether any row of the wave moved its max.  Cut into kStages short stages (per row block: the tile
// max, its reduction over the lane groups, the max update, four pairs of
// weights, the packing) that run one per PV column block, between the MFMAs
// of the previous tile's PV.
template <int RB, bool LB, bool RF = false>
struct SoftmaxStages {
  static constexpr int kPerRb = 8;
  static constexpr int kStages = kPerRb * RB;
  const f32x4 (&s)[2][RB];
  float (&m_used)[RB];
  float (&l_part)[RB];
  float (&r_part)[RB];  // RF: sum of weights times row factors (QK-Norm)
  bf16x8 (&p)[RB];
  float (&alpha)[RB];
  const f32x4 (&wsc)[2];
  float sl2;
  float mt[RB], msub[RB], lsum[RB], rsum[RB];
  bool need_any = false;

  __device__ __forceinline__ void run(int k) {
    if (k >= kStages) return;
    const int rb = k / kPerRb, st = k % kPerRb;
    const f32x4 sa = s[0][rb], sb = s[1][rb];
    if (st == 0) {
      const float m0 = max3_raw(sa[0], sa[1], sa[2]), m1 = max3_raw(sa[3], sb[0], sb[1]);
      mt[rb] = max3_raw(m0, m1, max3_raw(sb[2], sb[3], sb[3])) * sl2;  // sl2 > 0
    } else if (st == 1) {
      mt[rb] = rows_max_raw(mt[rb]);
    } else if (st == 2) {
      const bool need = mt[rb] > m_used[rb] + kRowsTau;
      const float al = need ? __builtin_amdgcn_exp2f(m_used[rb] - mt[rb]) : 1.f;  // 0 when m_used was -inf
      m_used[rb] = need ? mt[rb] : m_used[rb];
      alpha[rb] = al;
      need_any |= need;
      msub[rb] = m_used[rb] == -INFINITY ? 0.f : m_used[rb];
      lsum[rb] = 0.f;
      rsum[rb] = 0.f;
    } else if (st < 7) {
      const int e = st - 3;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], sl2, -msub[rb]));  // exp2(-inf) = 0
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[e], sl2, -msub[rb]));
      lsum[rb] += p0 + p1;
      if constexpr (RF) rsum[rb] += p0 * wsc[0][e] + p1 * wsc[1][e];
      p[rb][e] = (bf16)(LB ? p0 * wsc[0][e] : p0);
      p[rb][4 + e] = (bf16)(LB ? p1 * wsc[1][e] : p1);
    } else {
      l_part[rb] = l_part[rb] * alpha[rb] + lsum[rb];
      if constexpr (RF) r_part[rb] = r_part[rb] * alpha[rb] + rsum[rb];
      // formed here, not sunk towards their first use in the next tile
      asm volatile("" : "+v"(p[rb]), "+v"(l_part[rb]));
    }
  }
  __device__ __forceinline__ bool moved() const { return __ballot(need_any) != 0; }
};

// The whole softmax at once (the first tile of a piece)
template <int RB, bool LB, bool RF>
__device__ __forceinline__ bool softmax_tile(const f32x4 (&s)[2][RB], float (&m_used)[RB], float (&l_part)[RB],
                                             float (&r_part)[RB], bf16x8 (&p)[RB], float (&alpha)[RB],
                                             const f32x4 (&wsc)[2], float sl2) {
  SoftmaxStages<RB, LB, RF> sm{s, m_used, l_part, r_part, p, alpha, wsc, sl2};
#pragma unroll
  for (int k = 0; k < SoftmaxStages<RB, LB, RF>::kStages; ++k) sm.run(k);
  return sm.moved();
}

// O *= alpha (per row) in place in the accumulator registers, for the rare
// tile whose softmax moved a row's max.  Each entry is read, scaled and
// written back by one asm block, so the accumulators never leave their
// registers (a plain vector multiply would make the compiler hold them in
// vector registers across the whole tile loop).  The MFMAs that last wrote
// them are waited out first (the longest MFMA-result-to-read distance is
// 19 wait states).
template <int RB>
__device__ __forceinline__ void scale_acc(f32x4 (&acc)[32][RB], const float (&alpha)[RB]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < 32; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = acc[db][rb][e];
        float t;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\ts_nop 1\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(t) : "v"(alpha[rb]));
        acc[db][rb][e] = x;
      }
}

// Scores: the K operands of kQkPre k-steps ahead are in flight while a k-step's
// MFMAs issue (4 per k-step per row block pair, twice that on the two rotary
// k-steps, which multiply the hi and lo query parts).
template <int RB>
__device__ __forceinline__ void sched_qk() {
  __builtin_amdgcn_sched_group_barrier(kSchedDs, 2 * kQkPre<RB>, 0);
#pragma unroll
  for (int ks = 0; ks < kDc / 32; ++ks) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * RB, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDs, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDs, RB, 0);
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4 * RB, 0);
  __builtin_amdgcn_sched_group_barrier(kSchedDs, RB, 0);
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4 * RB, 0);
}

// a when B, else b (same type): picks an accumulator at compile time
template <bool B, class T>
__device__ __forceinline__ T& pick(T& a, T& b) {
  if constexpr (B) return a;
  return b;
}

}  // namespace

// RB: 16-row blocks per wave (1: 64-row groups, 2: 128-row groups).  QM: the
// stored rows (0: 16-bit; 1: int4, packed latent and rotary codes, two
// scales per row; 2: int8 latent codes and 16-bit rotary entries, one scale
// per row).  PB: bf16 partial outputs (a compile-time choice: a branch in
// the epilogue changes the register allocation of the tile loop).  QS: a
// split query.
template <int RB, int QM, bool PB, bool QS, bool QKN>
__global__ __launch_bounds__(kRowsThreads, 1) void decode_rows_kernel(RowsLaunch L) {
  constexpr int MT = 16 * RB * kRowsWaves;  // query rows of a row group
  constexpr int kOv = piece_tiles(MT, PB, QS) * kTile;  // a request's start, in rows of the work split
  constexpr bool LB = QM != 0;                           // low-bit rows: landed, then unpacked
  using SM = RowsSmem<QM, RB, QKN>;
  static_assert(!QKN || QM == 0, "QK-Norm row factors with 16-bit rows only");
  // loads per wave per 16-bit tile: its share of the rows, and with QK-Norm
  // one more for the tile's row factors
  constexpr int kDmaW = kDmaPerWave + (QKN ? 1 : 0);
  constexpr int NLAT = SM::NLAT;
  constexpr int RBYTES = QM == 1 ? kI4Row : QM == 2 ? kI8Row : kRowBytes;  // bytes per stored row
  __shared__ __attribute__((aligned(16))) SM sm;

  // ---- the segment of this workgroup, and its place in the segment's grid ----
  int g = 0;
  while (g + 1 < L.n_segs && (int)blockIdx.x >= L.wg_begin[g + 1]) ++g;
  const DecodeArgs& a = L.a;
  const SegArgs& sg = L.segs[g];
  const int n_share = L.n_share[g], n_rg = L.n_rg[g], rows_total = L.rows_total[g];
  const int bid = (int)blockIdx.x - L.wg_begin[g];

  const char* const cache = (const char*)sg.cache;
  const int32_t* const block_table = sg.block_table;
  const int32_t* const seq_lens = sg.seq_lens;
  const float* const q_rot = (const float*)sg.q_rot;
  const float* const q_lat = (const float*)a.q_lat;
  const float* const row_scale = sg.row_scale;
  const float* const row_rinv = sg.row_rinv;
  void* const o_part = a.o_part;
  constexpr bool part_bf = PB;
  float* const lse_part = a.lse_part;
  const int64_t max_rows = sg.max_rows;
  const int max_pages = sg.max_pages;
  const int n_pages = sg.n_pages;
  const int head_begin = sg.head_begin;
  const int hc = sg.head_count;
  const int causal = sg.causal;
  const int part_begin = sg.part_begin;
  const int n_split = sg.n_split;
  const int s_q = a.s_q;
  const int n_heads = a.n_heads;
  const int n_part = a.n_part;
  const int B = a.batch;
  const float scale = a.scale;
  const float sl2 = scale * kLog2e;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which share / row group this workgroup owns (XCD-aware order) ----
  int j, rg;
  if (n_rg == 1) {
    j = bid;
    rg = 0;
  } else if (bid < n_share / 8 * 8 * n_rg) {  // shares in whole octets: row groups on one XCD
    rg = (bid / 8) % n_rg;
    j = (bid / (8 * n_rg)) * 8 + bid % 8;
  } else {  // the last n_share % 8 shares
    const int full = n_share / 8 * 8, r = n_share - full, b2 = bid - full * n_rg;
    rg = b2 / r;
    j = full + b2 % r;
  }
  const int row0 = rg * MT;
  const int nrows = min(MT, rows_total - row0);
  const int wrow0 = 16 * RB * wave;            // first row of this wave within the group
  const bool wave_rows = wrow0 < nrows;        // wave-uniform: the wave has query rows (a wave
                                               // without rows only loads tiles)
  const int64_t cap = block_table ? (int64_t)max_pages * kPageSize : max_rows;
  auto clampT = [cap](int t) -> int { return (int)max((int64_t)0, min((int64_t)t, cap)); };
  auto padT = [](int t) -> int { return (t + kTile - 1) / kTile * kTile; };
  // a request's length in the work split: whole tiles plus the piece cost
  int ov = kOv;
  auto splitT = [padT, &ov](int t) -> int { return t > 0 ? padT(t) + ov : 0; };

  // ---- plan pass 1: total, longest and shortest request, each padded to
  // whole tiles, and the requests with rows ----
  int tsum = 0, tmax = 0, tmin = INT_MAX, nz = 0;
  auto add_req = [&](int Tr) {
    const int T = padT(Tr);
    tsum += T;
    tmax = max(tmax, T);
    tmin = min(tmin, T);
    nz += Tr > 0;
  };
  auto reduce_wave = [&]() {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      tsum += __shfl_xor(tsum, o);
      tmax = max(tmax, __shfl_xor(tmax, o));
      tmin = min(tmin, __shfl_xor(tmin, o));
      nz += __shfl_xor(nz, o);
    }
  };
  int Tr_lane = 0;
  if (B <= 64) {
    if (wave == 0) {
      Tr_lane = lane < B ? clampT(seq_lens[lane]) : 0;
      if (lane < B) add_req(Tr_lane);
      reduce_wave();
    }
  } else {
    for (int b = tid; b < B; b += kRowsThreads) add_req(clampT(seq_lens[b]));
    reduce_wave();
    if (lane == 0) {
      sm.red[wave] = tsum;
      sm.red[kRowsWaves + wave] = tmax;
      sm.red[2 * kRowsWaves + wave] = tmin;
      sm.red[3 * kRowsWaves + wave] = nz;
    }
    __syncthreads();
    tsum = nz = 0;
    tmax = 0;
    tmin = INT_MAX;
#pragma unroll
    for (int w = 0; w < kRowsWaves; ++w) {
      tsum += sm.red[w];
      tmax = max(tmax, sm.red[kRowsWaves + w]);
      tmin = min(tmin, sm.red[2 * kRowsWaves + w]);
      nz += sm.red[3 * kRowsWaves + w];
    }
  }
  const bool req_mode = n_split == 1;
  int share = 0;
  if (!req_mode) {
    // requests of one length that whole shares tile exactly keep that split
    // (one piece per share; the piece costs change nothing there, and the
    // power-of-two strides between workgroups it gives long requests stream
    // measurably faster than the shifted ones)
    const int share0 = max(kTile, ((tsum + n_share - 1) / n_share + kTile - 1) / kTile * kTile);
    if (tmin == tmax && tmax % share0 == 0) ov = 0;
    share = (tsum + nz * ov + n_share - 1) / n_share;
    // the longest request's rows span at most n_split shares
    share = max(share, (tmax + n_split - 2) / (n_split - 1));
    share = max(kTile, (share + kTile - 1) / kTile * kTile);
  }
  const int lo = j * share, hi = lo + share;

  // ---- this wave's query rows: block rb, lane row l16 (recomputed where
  // used, from an opaque lane copy, so nothing of it is held across the
  // tile loop) ----
  struct RowInfo {
    bool valid;    // the row exists
    int tok;       // query token within the request
    int64_t qoff;  // token * n_heads + head, without the request part
  };
  auto row_info = [&](int rb) -> RowInfo {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int r = wrow0 + 16 * rb + (ln & 15);
    const bool valid = r < nrows;
    const int Rr = row0 + (valid ? r : 0);  // a row past the group stands in for row0
    const int tok = Rr / hc;
    return RowInfo{valid, tok, (int64_t)tok * n_heads + head_begin + Rr % hc};
  };

  int base = 0;  // prefix of the split lengths over the requests scanned so far (wave 0)
  for (int chunk = 0;; ++chunk) {
    // ---- plan pass 2: wave 0 scans 64 requests, lists pieces, writes -inf tails ----
    if (wave == 0) {
      const int b = chunk * 64 + lane;
      const int Tr = B <= 64 ? Tr_lane : b < B ? clampT(seq_lens[b]) : 0;
      const int T = padT(Tr);
      const int V = splitT(Tr);
      int incl = V;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      // the request's rows start at S in the split's units (after its piece cost)
      const int S = base + incl - V + (V > 0 ? ov : 0);
      bool is_piece, tail;
      int r0 = 0, r1 = 0, slot = 0, cnt = 0;
      if (req_mode) {
        is_piece = b < B && T > 0 && (b % n_share) == j;
        r1 = Tr;
        tail = b < B && T == 0 && (b % n_share) == j;
      } else {
        is_piece = b < B && T > 0 && S < hi && S + T > lo;
        r0 = max(lo, S) - S;
        r1 = min(min(hi, S + T) - S, Tr);
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
          const int Rr = row0 + e % nrows;
          const int tok = tb_ * s_q + Rr / hc;
          const int h = head_begin + Rr % hc;
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
      const int n_tiles = (pr1 - pr0 + kTile - 1) / kTile;
      // last visible row of each of this lane's query rows
      int vis[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) vis[rb] = causal ? T - s_q + row_info(rb).tok : T - 1;

      const char* const req_base = cache + (int64_t)b * max_rows * RBYTES;
      // block-table row of the request, read with scalar loads (the table is
      // constant for the launch): a tile's page id is requested one
      // iteration before its loads are issued, so the round trip is hidden
      const CInt* const bt_row = block_table ? (const CInt*)(block_table + (int64_t)b * max_pages) : nullptr;
      auto page_of = [&](int it) -> int { return bt_row[(pr0 + it * kTile) / kPageSize]; };
      // resource over the rows of tile `it` (page `pg` in the paged layout);
      // a tile past the piece, or on a page outside the pool, gets record
      // count 0 and reads as zeros.  Every tile index, past the piece or not,
      // gets its kDmaPerWave loads per wave, so the loads in flight are
      // counted the same way in every iteration (they complete in order).
      // (int4 rows: also their scale pairs, indexed like the rows)
      auto tile_row = [&](int it, int pg, bool* ok) -> int64_t {
        const int t0 = pr0 + it * kTile;
        *ok = it < n_tiles;
        if (!bt_row) return (int64_t)b * max_rows + t0;
        *ok = *ok && pg >= 0 && pg < n_pages;
        return (int64_t)(*ok ? pg : 0) * kPageSize + (t0 % kPageSize);
      };
      auto tile_rsrc = [&](int it, int pg) -> i32x4_t {
        bool ok;
        const int64_t row = tile_row(it, pg, &ok);
        const int n = ok ? min(kTile, pr1 - (pr0 + it * kTile)) : 0;
        return buffer_rsrc(ok ? cache + row * RBYTES : cache, n * RBYTES);
      };
      constexpr int kSpr = QM == 1 ? 2 : 1;  // scales per stored row
      auto scale_rsrc = [&](int it, int pg) -> i32x4_t {
        bool ok;
        const int64_t row = tile_row(it, pg, &ok);
        const int n = ok ? min(kTile, pr1 - (pr0 + it * kTile)) : 0;
        return buffer_rsrc(ok ? row_scale + kSpr * row : row_scale, n * 4 * kSpr);
      };
      // QK-Norm: the row factors of tile `it` (indexed like the rows) into
      // their stage, one 4-byte load per lane of every wave (the waves write
      // the same values; each counts the load like its tile loads)
      auto load_rinv = [&](int it, int pg) {
        if constexpr (QKN) {
          bool ok;
          const int64_t row = tile_row(it, pg, &ok);
          const int n = ok ? min(kTile, pr1 - (pr0 + it * kTile)) : 0;
          int ln = lane;
          asm volatile("" : "+v"(ln));
          dma4(buffer_rsrc(ok ? row_rinv + row : row_rinv, n * 4), (const char*)sm.rinv[it % 3], 4 * ln);
        }
      };
      auto load_lb = [&](int it, int pg) {
        if constexpr (QM == 1) tile_load_i4(tile_rsrc(it, pg), scale_rsrc(it, pg), sm.land[it % 3], wave, lane);
        if constexpr (QM == 2)
          tile_load_i8(tile_rsrc(it, pg), scale_rsrc(it, pg), sm.land[it % 2], sm.rot[it % kRotStages], wave, lane);
      };
      auto unpack_lb = [&](int it) {
        if constexpr (QM == 1)
          unpack_tile_i4(sm.land[it % 3], sm.lat[it % NLAT], sm.rot[it % kRotStages], sm.scl[it % 3][wave], wave,
                         lane);
        if constexpr (QM == 2) unpack_tile_i8(sm.land[it % 2], sm.lat[it % NLAT], sm.scl[it % 3][wave], wave, lane);
      };
      // low-bit rows: loads run kLbAhead tiles ahead of the scores (int4:
      // tiles 0..2 go out first and tile 3 once tile 0 is unpacked; int8,
      // with two landing stages: tiles 0 and 1, then tile 2)
      constexpr int kLbAhead = QM == 1 ? 4 : 3;
      constexpr int kLbFirst = QM == 1 ? 3 : 2;  // tiles loaded before the first unpacking

      int pg_next = 0;  // page of the next tile to load (paged layout)
      int pg_lb = 0;    // low-bit rows: page of the tile loaded once tiles 0 and 1 are unpacked
      // ---- the first tiles go out before the query loads ----
      if constexpr (LB) {
        int pg[kLbAhead + 1];
#pragma unroll
        for (int t = 0; t <= kLbAhead; ++t) pg[t] = bt_row && t < n_tiles ? page_of(t) : 0;
#pragma unroll
        for (int t = 0; t < kLbFirst; ++t) load_lb(t, pg[t]);
        pg_lb = pg[kLbFirst];
        pg_next = pg[kLbFirst + 1];
      } else {
        int pg[kLoadAhead + 1];
#pragma unroll
        for (int t = 0; t <= kLoadAhead; ++t) pg[t] = bt_row && t < n_tiles ? page_of(t) : 0;
#pragma unroll
        for (int t = 0; t < kLoadAhead; ++t) {
          const i32x4_t rs = tile_rsrc(t, pg[t]);
#pragma unroll
          for (int i = 0; i < kDmaPerWave; ++i) tile_load(rs, sm.lat[t], sm.rot[t], wave, lane, i);
          load_rinv(t, pg[t]);
        }
        pg_next = pg[kLoadAhead];
      }

      // ---- query: latent hi parts, rotary hi + lo parts (B operands) ----
      bf16x8 qh[RB][kDc / 32];
      bf16x8 qrl[RB][2];
      char* const qrot_w = sm.qrot[16 * RB * wave];  // this wave's rows
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const RowInfo ri = row_info(rb);
        const int64_t qi = (int64_t)b * s_q * n_heads + ri.qoff;
        const float* qr = q_rot + qi * kDr + 8 * lg;
        const float* ql = q_lat + qi * kDc + 8 * lg;                   // fp32 query
        const bf16* qlh = (const bf16*)q_lat + qi * (2 * kDc) + 8 * lg;  // split query: its hi plane
        // two batches of 9 k-steps: the loads of a batch go out together
        // (unconditional: a row past the group reads row0's query), then
        // their conversions, each pinned where it is formed so the staging
        // registers die before the next batch.  The rotary part, and the
        // latent part of an fp32 query, are split here (a row past the group
        // gets zeros); a split query's hi plane is used as it is (a row past
        // the group keeps row0's: its results are never stored).  A wave
        // without rows loads them too: with the loads skipped on its path the
        // registers were undefined there, and the compiler carried the last
        // piece's query across the epilogue instead (48 VGPRs written to
        // scratch and read back in every piece at 128-row groups).
        constexpr int kBatch = kKSteps / 2;
#pragma unroll
        for (int k0 = 0; k0 < kKSteps; k0 += kBatch) {
          f32x4 v[kBatch][2];
          bf16x8 hv[kBatch];
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int ks = k0 + i;
            if (QS && ks < kDc / 32) {
              hv[i] = *(const bf16x8*)(qlh + 32 * ks);
            } else {
              const float* src = ks < kDc / 32 ? ql + 32 * ks : qr + 32 * (ks - kDc / 32);
              v[i][0] = *(const f32x4*)src;
              v[i][1] = *(const f32x4*)(src + 4);
            }
          }
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int ks = k0 + i;
            if (QS && ks < kDc / 32) {
              qh[rb][ks] = hv[i];
              asm volatile("" ::"v"(hv[i]));
              continue;
            }
            if (!ri.valid) v[i][0] = v[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 h8, l8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = v[i][e >> 2][e & 3];
              const bf16 h = (bf16)x;
              h8[e] = h;
              l8[e] = (bf16)(x - (float)h);
            }
            if (ks < kDc / 32) {
              qh[rb][ks] = h8;
              asm volatile("" ::"v"(h8));
            } else {
              const int jr = ks - kDc / 32, qr2 = 16 * rb + l16;
              *(bf16x8*)(qrot_w + qr2 * kRBytes + (rpos(qr2, 4 * jr + lg) << 4)) = h8;
              qrl[rb][jr] = l8;
              asm volatile("" ::"v"(l8));
            }
          }
        }
      }

      f32x4 acc[32][RB];  // O^T: lane holds columns 16 db + 4 lg + e of row (rb, l16)
#pragma unroll
      for (int db = 0; db < 32; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          asm("" : "+a"(acc[db][rb]));
        }
      float m_used[RB], l_part[RB], r_part[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        m_used[rb] = -INFINITY;
        l_part[rb] = 0.f;
        r_part[rb] = 0.f;
      }

      // relative index of the last visible token of tile `it` for each row
      // block, as the masked softmax takes it (block 0 of the tile: e <= lim)
      auto tile_lim = [&](int it, int (&lim)[RB]) {
        const int t0 = pr0 + it * kTile;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) lim[rb] = min(pr1 - 1, vis[rb]) - t0 - 4 * lg;
      };
      // the wave's earliest last-visible row: tile `it` needs no mask when it
      // lies inside the piece and before it
      int vis_min = vis[0];
#pragma unroll
      for (int rb = 1; rb < RB; ++rb) vis_min = min(vis_min, vis[rb]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) vis_min = min(vis_min, __shfl_xor(vis_min, o));
      vis_min = __builtin_amdgcn_readfirstlane(vis_min);
      auto tile_full = [&](int it) { return pr0 + (it + 1) * kTile <= min(pr1, vis_min + 1); };

      f32x4 sacc[2][RB];
      f32x4 racc_i4[2][RB];
      // the rotary part's accumulator (apart for low-bit rows and QK-Norm,
      // whose factors scale the latent part only)
      f32x4(&racc)[2][RB] = pick<LB || QKN>(racc_i4, sacc);
      auto scl_of = [&](int it) -> const float* {
        if constexpr (LB) return sm.scl[it % 3][wave];
        if constexpr (QKN) return sm.rinv[it % 3];
        return nullptr;
      };
      bf16x8 p[RB];
      float alpha[RB];
      int lim[RB];
      f32x4 wsc[2];  // low-bit rows: the latent scales of the current tile's tokens
      // ---- tile 0: scores and softmax ----
      if constexpr (LB) {
        // tiles 0 and 1 landed (int4: tile 2 in flight), unpacked by every
        // wave; then the next tile goes out into tile 0's landing stage
        wait_vmcnt<QM == 1 ? kI4Dma : 0>();
        wait_lgkm0();
        barrier_raw();
        unpack_lb(0);
        unpack_lb(1);
        wait_lgkm0();
        barrier_raw();
        load_lb(kLbFirst, pg_lb);
      } else {
        static_assert(kLoadAhead == 3, "tiles 1 and 2 stay in flight over tile 0");
        wait_vmcnt<2 * kDmaW>();
        wait_lgkm0();
        barrier_raw();
      }
      if (wave_rows) {
        qk_tile<RB>(sm.lat[0], sm.rot[0], qrot_w, lane, qh, qrl, sacc, racc);
        tile_lim(0, lim);
        // (its factor multiplies an empty O)
        prep_scores<RB, QM, QKN>(sacc, racc, tile_full(0), lim, scl_of(0), wsc);
        softmax_tile<RB, LB, QKN>(sacc, m_used, l_part, r_part, p, alpha, wsc, sl2);
      }
      for (int it = 0; it + 1 < n_tiles; ++it) {
        // 16-bit rows: tile it+1 in LDS (this wave's loads, with tile it+2
        // still in flight, then everyone's); every wave is past the PV of
        // tile it-1 and the scores of tile it, so their stages take tile it+3,
        // whose loads go out between the PV MFMAs of tile it.
        // Low-bit rows: tile it+2 landed (int4: tile it+3 in flight) and tile
        // it+1 unpacked; every wave is past the PV of tile it-1, the scores of
        // tile it and the unpacking of tile it+1, so tile it+2 is unpacked into
        // the stages of tile it-1 and tile it + kLbAhead lands where tile it+1
        // did (int8: its rotary entries where tile it's were).
        wait_vmcnt<QM == 1 ? kI4Dma : QM == 2 ? 0 : kDmaW>();
        wait_lgkm0();
        barrier_raw();
        const i32x4_t rs_next = tile_rsrc(it + kLoadAhead, pg_next);
        char* const lat_next = sm.lat[(it + kLoadAhead) % NLAT];
        char* const rot_next = sm.rot[(it + kLoadAhead) % kRotStages];
        auto load_next = [&](int i) {
          if constexpr (!LB) tile_load(rs_next, lat_next, rot_next, wave, lane, i);
          if (i == kDmaPerWave - 1) load_rinv(it + kLoadAhead, pg_next);
        };
        if constexpr (LB) {
          load_lb(it + kLbAhead, pg_next);
          unpack_lb(it + 2);
        }
        if (!wave_rows) {
#pragma unroll
          for (int i = 0; i < kDmaPerWave; ++i) load_next(i);
        } else {
          tile_lim(it + 1, lim);
          qk_tile<RB>(sm.lat[(it + 1) % NLAT], sm.rot[(it + 1) % kRotStages], qrot_w, lane, qh, qrl, sacc, racc);
          sched_qk<RB>();
          prep_scores<RB, QM, QKN>(sacc, racc, tile_full(it + 1), lim, scl_of(it + 1), wsc);
          __builtin_amdgcn_sched_barrier(0);
          // the PV of tile it with the softmax of tile it+1 between its MFMAs
          // (the scores die there: only the two tiles' P operands live across
          // the PV product)
          bf16x8 pn[RB];
          SoftmaxStages<RB, LB, QKN> smx{sacc, m_used, l_part, r_part, pn, alpha, wsc, sl2};
          pv_tile<RB>(sm.lat[it % NLAT], lane, p, acc, load_next, [&](int db) { smx.run(db); });
          const bool moved = smx.moved();
          __builtin_amdgcn_sched_barrier(0);
          if (moved) scale_acc<RB>(acc, alpha);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) p[rb] = pn[rb];
        }
        // the page of the tile loaded next iteration: its scalar load returns
        // during the wait at the top (not inside the score product, where it
        // would force full waits on the LDS reads)
        {
          const int t_pg = it + (LB ? kLbAhead + 1 : kLoadAhead + 1);  // the tile loaded next iteration
          if (bt_row && t_pg < n_tiles) pg_next = page_of(t_pg);
        }
      }
      // the last tile's PV (the loads past the piece, which only wrote zeros
      // into free stages, are drained too: none may land after the
      // workgroup's LDS is released)
      wait_vmcnt<0>();
      wait_lgkm0();
      barrier_raw();
      if (wave_rows) pv_tile<RB>(sm.lat[(n_tiles - 1) % NLAT], lane, p, acc, [](int) {}, [](int) {});

      // ---- epilogue: 1/l, the lse with the latent lo part's first-order
      // share, the normalised partial output.  Every load and product comes
      // before the first store: a store is counted until written, so a load
      // after it would wait for the write too. ----
      if (wave_rows) {
        float lt[RB], cs[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) lt[rb] = rows_sum(l_part[rb]);
        // sum_d lo_d acc_d over this lane's columns 16 db + 4 lg + e, per row
        // block; every query load goes out before the first product (a row
        // past the group reads row0's query)
        if constexpr (QS) {
          // the lo plane as it is: this lane's 4 columns of a block are 8
          // bytes; the loads of every row block go out together (the hi
          // parts are dead here, so their registers take them)
          uint32_t qv[RB][32][2];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int64_t qi = (int64_t)b * s_q * n_heads + row_info(rb).qoff;
            const char* qll = (const char*)((const bf16*)q_lat + qi * (2 * kDc) + kDc) + 8 * lg;
#pragma unroll
            for (int db = 0; db < 32; ++db) {
              const auto w = *(const uint2*)(qll + 32 * db);
              qv[rb][db][0] = w.x;
              qv[rb][db][1] = w.y;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            float c = 0.f;
#pragma unroll
            for (int db = 0; db < 32; ++db) {
              const uint32_t w0 = qv[rb][db][0], w1 = qv[rb][db][1];
              c += __uint_as_float(w0 << 16) * acc[db][rb][0];
              c += __uint_as_float(w0 & 0xffff0000u) * acc[db][rb][1];
              c += __uint_as_float(w1 << 16) * acc[db][rb][2];
              c += __uint_as_float(w1 & 0xffff0000u) * acc[db][rb][3];
            }
            cs[rb] = rows_sum(c) * sl2;
          }
        } else {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int64_t qi = (int64_t)b * s_q * n_heads + row_info(rb).qoff;
            const float* ql = q_lat + qi * kDc + 4 * lg;
            f32x4 qv[32];
#pragma unroll
            for (int db = 0; db < 32; ++db) qv[db] = *(const f32x4*)(ql + 16 * db);
            __builtin_amdgcn_sched_barrier(0);
            float c = 0.f;
#pragma unroll
            for (int db = 0; db < 32; ++db)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x = qv[db][e];  // the lo part as the prologue split it
                c += (float)(bf16)(x - (float)(bf16)x) * acc[db][rb][e];
              }
            cs[rb] = rows_sum(c) * sl2;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float linv = lt[rb] > 0.f ? 1.f / lt[rb] : 0.f;
          // QK-Norm: each token's lo share carries its row factor; to first
          // order that is the weighted mean factor times the lo share of o
          if constexpr (QKN) cs[rb] *= rows_sum(r_part[rb]) * linv;
          const RowInfo ri = row_info(rb);
          const int64_t lse_i = ((int64_t)b * s_q * n_heads + ri.qoff) * n_part + part_begin + slot;
          if (ri.valid && lg == 0)
            lse_part[lse_i] = lt[rb] > 0.f ? (m_used[rb] + __log2f(lt[rb]) + linv * cs[rb]) * kLn2 : -INFINITY;
          if (ri.valid && lt[rb] > 0.f) {
            const int64_t o = lse_i * kDc + 4 * lg;
#pragma unroll
            for (int db = 0; db < 32; ++db) store_part4(o_part, o + 16 * db, acc[db][rb] * linv, part_bf);
          }
        }
      }
      wait_lgkm0();
      barrier_raw();  // every wave is past its last reads of the ring before the next piece loads
    }
    __syncthreads();
    if (done) break;
  }
}

template __global__ void decode_rows_kernel<1, 0, false, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, false, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 1, false, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 2, false, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 0, false, false, true>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, false, false, true>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 0, true, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, true, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 1, true, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 2, true, false, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 0, true, false, true>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, true, false, true>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 0, false, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, false, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 1, false, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 2, false, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 0, false, true, true>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, false, true, true>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 0, true, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, true, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 1, true, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 2, true, true, false>(RowsLaunch);
template __global__ void decode_rows_kernel<1, 0, true, true, true>(RowsLaunch);
template __global__ void decode_rows_kernel<2, 0, true, true, true>(RowsLaunch);

int decode_rows_tile(int rows_total) { return rows_total <= 64 ? 64 : 128; }

namespace {

// Cost model of a segment for splitting a shared grid: its tiles (batch x row
// capacity / 32) and the cycles of one tile in its fullest row group.  A
// tile's time is mostly one wave's own chain (scores, softmax, PV, its
// loads), so it grows only a little with the number of waves that have rows
// (measured at 128-row groups: about 4.25k cycles with one such wave, 5k
// with four; at 64-row groups about 3.9k with four).
struct SegCost {
  double tiles;
  double t_tile;
  double piece;  // a piece's cost beyond its tiles, in tiles
  int batch;
  int n_rg;
};

SegCost seg_cost(const DecodeArgs& a, const SegArgs& s, int mt) {
  const int64_t cap = s.block_table ? (int64_t)s.max_pages * kPageSize : s.max_rows;
  const int rows = a.s_q * s.head_count;
  const int rpw = mt / kRowsWaves;  // rows per wave
  SegCost c;
  c.n_rg = (rows + mt - 1) / mt;
  const int busy = (std::min(rows, mt) + rpw - 1) / rpw;  // waves with rows in the fullest group
  c.t_tile = (mt == 64 ? 3400.0 + 125.0 * busy : 4000.0 + 250.0 * busy);
  c.tiles = std::max(1.0, (double)a.batch * (double)std::max<int64_t>(cap, 1) / kTile);
  c.piece = piece_tiles(mt, a.part_bf16 != 0, a.q_split != 0);
  c.batch = a.batch;
  return c;
}

template <bool PB, bool QS, bool QKN>
hipError_t launch_rows_pb(const RowsLaunch& L, int mt, int qm, int grid, hipStream_t stream) {
  const dim3 block(kRowsThreads);
  if constexpr (!QKN) {
    if (qm == 1) return launch(decode_rows_kernel<1, 1, PB, QS, false>, dim3(grid), block, stream, L);
    if (qm == 2) return launch(decode_rows_kernel<1, 2, PB, QS, false>, dim3(grid), block, stream, L);
  }
  if (mt == 64) return launch(decode_rows_kernel<1, 0, PB, QS, QKN>, dim3(grid), block, stream, L);
  return launch(decode_rows_kernel<2, 0, PB, QS, QKN>, dim3(grid), block, stream, L);
}

template <bool QKN>
hipError_t launch_rows_q(const RowsLaunch& L, int mt, int qm, int grid, hipStream_t stream) {
  if (L.a.q_split) {
    if (L.a.part_bf16) return launch_rows_pb<true, true, QKN>(L, mt, qm, grid, stream);
    return launch_rows_pb<false, true, QKN>(L, mt, qm, grid, stream);
  }
  if (L.a.part_bf16) return launch_rows_pb<true, false, QKN>(L, mt, qm, grid, stream);
  return launch_rows_pb<false, false, QKN>(L, mt, qm, grid, stream);
}

// QK-Norm row factors are given for every segment of a launch or for none
// (checked by the caller); they exist with 16-bit rows only.
hipError_t launch_rows(const RowsLaunch& L, int mt, int qm, int grid, hipStream_t stream) {
  if (L.segs[0].row_rinv) return qm ? hipErrorInvalidValue : launch_rows_q<true>(L, mt, qm, grid, stream);
  return launch_rows_q<false>(L, mt, qm, grid, stream);
}

}  // namespace

hipError_t launch_decode_rows(const DecodeArgs& a, int n_wg, hipStream_t stream) {
  return launch_decode_rows_multi(a, &a.seg, 1, n_wg, 0, stream);
}

hipError_t launch_decode_rows_multi(const DecodeArgs& a, const SegArgs* segs, int n_segs, int n_wg, int qm,
                                    hipStream_t stream) {
  for (int g0 = 0; g0 < n_segs; g0 += kRowsMaxSegs) {
    const int n = std::min(kRowsMaxSegs, n_segs - g0);
    int rows_max = 0;
    for (int g = 0; g < n; ++g) rows_max = std::max(rows_max, a.s_q * segs[g0 + g].head_count);
    const int mt = qm ? 64 : decode_rows_tile(rows_max);  // low-bit rows: 64-row groups
    RowsLaunch L{};
    L.a = a;
    L.n_segs = n;
    for (int g = 0; g < n; ++g) {
      L.segs[g] = segs[g0 + g];
      L.rows_total[g] = a.s_q * segs[g0 + g].head_count;
    }
    if (n == 1) {
      decode_bf16_grid(L.rows_total[0], mt, n_wg, &L.n_share[0], &L.n_rg[0]);
    } else {
      // shares per segment for equal finish times: the smallest time T at
      // which the shares every segment needs fit in n_wg.  A share of n
      // takes (tiles + batch x piece) / n + piece tiles (its requests' piece
      // costs spread over the shares, and its own first piece).
      SegCost c[kRowsMaxSegs];
      double hi = 1.0;
      for (int g = 0; g < n; ++g) {
        c[g] = seg_cost(a, L.segs[g], mt);
        hi = std::max(hi, (c[g].tiles + (c[g].batch + 1) * c[g].piece) * c[g].t_tile);
      }
      auto shares = [&](double T, int g) {
        const double avail = std::max(T / c[g].t_tile - c[g].piece, 1e-9);
        return (int)std::min<double>(c[g].tiles,
                                     std::max(1.0, std::ceil((c[g].tiles + c[g].batch * c[g].piece) / avail)));
      };
      auto used = [&](double T) {
        int64_t w = 0;
        for (int g = 0; g < n; ++g) w += (int64_t)shares(T, g) * c[g].n_rg;
        return w;
      };
      double lo = hi / std::max(n_wg, 1) / 4;
      for (int it = 0; it < 60; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (used(mid) <= n_wg) hi = mid; else lo = mid;
      }
      for (int g = 0; g < n; ++g) {
        L.n_share[g] = shares(hi, g);
        L.n_rg[g] = c[g].n_rg;
      }
    }
    int grid = 0;
    for (int g = 0; g < n; ++g) {
      L.wg_begin[g] = grid;
      grid += L.n_share[g] * L.n_rg[g];
    }
    const hipError_t e = launch_rows(L, mt, qm, grid, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
