// Paged absorbed-MLA decode on gfx950 MFMA for bf16 and fp8 caches,
// software pipelined across tiles.
//
// A workgroup of four waves (one per SIMD) owns a work unit: sequence b,
// split k and 128 query rows, 32 per wave. The split's cache streams through
// LDS in tiles of 32 tokens (half a page): 512 latent and 64 rope elements
// per token, the 576-element cache of PaperTrace "02 · DeepSeek-V2
// analysis", section 1.3. Every wave reads every tile.
//
// Each wave is a complete attention worker for its 32 rows on the 32x32x16
// bf16 MFMA: the absorbed queries stay in registers as the B operands of the
// score S^T[token][row] = K[token][576] Q^T (section 1.3, eq. 18; the
// 1/sqrt(192) scale is folded into the exponent), the online softmax of a
// row runs in the lane that owns it, and the latent aggregate
// U^T[dim][row] += C^T[dim][token] P^T[token][row] accumulates in the 256
// accumulation registers, reading the tile transposed (ds_read_b64_tr_b16).
// W^UV is applied afterwards (section 6.1).
//
// One wave per SIMD issues about one instruction per five cycles, so a step
// that ran the score, then the softmax, then the aggregation would leave the
// matrix unit idle through every phase boundary. Step s instead interleaves
// the aggregation of tile s with the score MFMAs of tile s + 1 in one stream
// of 68 MFMAs, and the softmax of tile s + 1 runs under the last aggregation
// MFMAs; tile s + 3 is copied into the buffer freed by tile s - 1 in the
// same step. Four tile buffers: s (aggregation), s + 1 (score), s + 2
// (landed or landing) and s + 3 (being copied).
//
// Page copies are asynchronous (global_load_lds_dwordx4, 1 KB per
// instruction), spread over the first part of the step, and every wave waits
// for its own copies with vmcnt before the barrier that publishes them. A
// copy never reads past the sequence: slots beyond its last token repeat the
// last token, and the mask gives them weight exactly 0.
//
// fp8 caches (E4M3FN codes with one fp32 scale per token) run the same
// schedule on bf16 tiles: the copies land the codes of a tile in a staging
// buffer and its scales in one of two scale buffers, both private to the
// wave that copied them (each wave copies and widens its own 8 tokens), the
// rope rows straight in the tile buffer; during the step before the tile is
// scored the wave widens its codes to bf16(scale x code) in the tile buffer,
// and each pair of rows is copied again (the next tile's) once its codes are
// in registers. Three tile buffers: s (aggregation), s + 1 (score), s + 2
// (being widened).
//
// The unit ends by writing either u = U / l and lse (one split), or partials
// for the log-sum-exp combine: bf16 u = U / l with fp32 (m, l) when the
// output is bf16, else fp32 (m, l, U).
#include <type_traits>

#include "dma.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;
constexpr int kRows = 128;                 // query rows per workgroup, 32 per wave
constexpr int kLatRow = 1024;              // bytes of one token's bf16 latent
constexpr int kRopeOff = kTile * kLatRow;  // rope rows of 128 B
constexpr int kTileBytes = kRopeOff + kTile * 128;
constexpr int kLat8 = 512;                 // bytes of one token's fp8 latent
constexpr int kStageScale = kTile * kLat8; // two buffers of staged scales follow the codes
constexpr int kStageBytes = kStageScale + 2 * kTile * 4;
constexpr int kSlots = 68;                 // MFMAs of a steady-state step

// LDS layout: tile buffers, the fp8 staging buffer, the split's page ids
// and the first kQInLds query k-steps of every wave (kept in LDS, not
// registers).
template <bool FP8>
struct Lay {
  static constexpr int kNB = FP8 ? 3 : 4;                 // tile buffers
  static constexpr int kOffStage = kNB * kTileBytes;
  static constexpr int kOffIds = kOffStage + (FP8 ? kStageBytes : 0);
  static constexpr int kQInLds = FP8 ? 7 : 2;
  static constexpr int kOffQ = kOffIds + kMaxSplitPages * 4;
  static constexpr int kLdsBytes = kOffQ + 4 * kQInLds * 1024;
  // copies per wave and tile: bf16 8 latent rows and the rope of 8 tokens;
  // fp8 4 pairs of latent rows, the rope and the scales of 8 tokens
  static constexpr int kCopies = FP8 ? 6 : 9;
  static_assert(kLdsBytes + 256 <= 163840, "LDS budget (with the barrier reduction's)");
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// LDS swizzles, chosen so that every read pattern touches each of the 64
// banks once per pass (16-B reads serve 16 lanes per pass: the 4-lane quads
// of a half-wave split by the parity of the quad index; transposed reads
// serve a half-wave per pass):
//  * latent rows (1 KB): 16-B chunk c of token t at c ^ gsw(t),
//    gsw(t) = ((t & 3) << 2) | ((t >> 2) & 3);
//  * rope rows (128 B): 16-B chunk c of token t at c ^ ((t >> 1) & 7).
__device__ __forceinline__ int gsw(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int t) { return (t >> 1) & 7; }

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Score MFMAs with VGPR accumulators (the 256 accumulation registers hold
// U). The hardware does not interlock an MFMA result against VALU reads:
// score_fence() pads the gap before the VALU reads the scores.
__device__ __forceinline__ void mfma_sc0(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_sc(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_fence(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

// Largest excess (log2 units) of a score over its row's reference maximum in
// the first pass: probabilities stay below 2^32, row sums below 2^48.
constexpr float kJump = 32.0f;

// Slot schedule of a steady-state step (68 MFMAs): two aggregation MFMAs
// whose operands are read before the step's barrier, then nine groups of
// four score MFMAs (chains A B A B: an MFMA's chain partner issued two slots
// earlier has finished) and one aggregation MFMA, then 21 aggregation MFMAs
// under which the softmax of the scored tile runs, one stage every other slot.
constexpr int kLeadG = 2;
constexpr int kGroups = 9;
constexpr int kTailFrom = kLeadG + 5 * kGroups;    // 47
__host__ __device__ constexpr bool slot_is_score(int i) {
  return i >= kLeadG && i < kTailFrom && (i - kLeadG) % 5 != 4;
}
// score k-step of a score slot / aggregation index of an aggregation slot
__host__ __device__ constexpr int slot_index(int i) {
  if (i < kLeadG) return i;
  if (i < kTailFrom) {
    const int t = (i - kLeadG) / 5, r = (i - kLeadG) % 5;
    return r < 4 ? 4 * t + r : kLeadG + t;
  }
  return kLeadG + kGroups + (i - kTailFrom);
}
constexpr int kLastScore = kTailFrom - 2;          // slot of k-step 35
// softmax stages of the scored tile: stages 0-5 (mask and maximum,
// references, the first k-step's probabilities) at every third tail slot,
// ending at the step's last slot; stages 6-9 (the second k-step's
// probabilities, first used by aggregation index 16) in the next step's
// score region
__host__ __device__ constexpr int head_stage_at(int i) {
  return (i >= kSlots - 16 && (kSlots - 1 - i) % 3 == 0) ? 5 - (kSlots - 1 - i) / 3 : -1;
}
__host__ __device__ constexpr int tail_stage_slot(int st) {
  return st == 6 ? 0 : st == 7 ? 0 : st == 8 ? 1 : 1;
}
// bf16 copy slots: op o of the step's nine copies follows MFMA 5 o + 4
__host__ __device__ constexpr int copy_at16(int i) {
  return (i >= 4 && (i - 4) % 5 == 0 && (i - 4) / 5 < 9) ? (i - 4) / 5 : -1;
}
// fp8 widening of the tile scored next, piece j (2 tokens of the wave) at
// slots 4 + 8j (read its codes and scale), 7 + 8j and 10 + 8j (widen and
// write a half); the copies: the scales (op 5) at slot 2, the rope (op 4)
// at slot 3, latent pair j (op j) at slot 7 + 8j, after the half widened
// there has consumed the pair's staged codes.
constexpr int kConvFrom = 4;
__host__ __device__ constexpr int conv_at(int i) {
  return (i >= kConvFrom && i < kConvFrom + 32 && (i - kConvFrom) % 8 < 7 &&
          (i - kConvFrom) % 8 % 3 == 0)
             ? 3 * ((i - kConvFrom) / 8) + (i - kConvFrom) % 8 / 3
             : -1;
}
__host__ __device__ constexpr int copy_at8(int i) {
  return i == 2 ? 5 : i == 3 ? 4 : (i >= 7 && (i - 7) % 8 == 0 && (i - 7) / 8 < 4) ? (i - 7) / 8 : -1;
}
// Before the read of piece j, at most five of the wave's copies may fly:
// the previous step's pairs j + 1..3 and this step's scales, rope and pairs
// 0..j - 1; so the previous step's pair j and scales have landed.
constexpr int kConvInFlight = 5;
static_assert(conv_at(4) == 0 && conv_at(7) == 1 && conv_at(10) == 2 && conv_at(12) == 3 &&
                  conv_at(34) == 11 && conv_at(36) == -1 && conv_at(5) == -1,
              "widening slots");
static_assert(copy_at8(2) == 5 && copy_at8(3) == 4 && copy_at8(7) == 0 && copy_at8(31) == 3 &&
                  copy_at8(39) == -1, "fp8 copy slots");
// the page id for the next step's copies is read from LDS after slot 30 and
// moved to a scalar after slot 40
constexpr int kIdRead = 30, kIdUse = 40;
// slot of aggregation index 15 (the last use of the first probability
// k-step) and of index 16 (the first use of the second)
constexpr int kLastP0 = kTailFrom + 15 - (kLeadG + kGroups);
constexpr int kFirstP1 = kTailFrom + 16 - (kLeadG + kGroups);
static_assert(head_stage_at(kSlots - 1) == 5 && head_stage_at(kSlots - 16) == 0, "head stages");
static_assert(kSlots - 16 > kTailFrom, "head stages follow the merged score");
static_assert(kSlots - 1 > kLastP0, "P0 is rewritten after its last use");
static_assert(tail_stage_slot(9) < kFirstP1, "P1 is complete before its first use");

// Every row of the unit gets (m, l, U) = (v, v, v): marks out-of-range
// sequences and page ids with NaN.
__device__ void write_uniform(const DecodeParams& p, int b, int k, int row0, float v) {
  const int tid = threadIdx.x;
  const int nrows = min(kRows, p.R - row0);
  for (int e = tid; e < nrows * kDc; e += kThreads) {
    const int r = row0 + e / kDc, d = e % kDc;
    if (p.n_split == 1) {
      const size_t o = ((size_t)b * p.R + r) * kDc + d;
      if (p.out_bf16) ((uint16_t*)p.out)[o] = f2bf(v);
      else ((float*)p.out)[o] = v;
    } else {
      const size_t o = (((size_t)b * p.n_split + k) * p.R + r) * kDc + d;
      if (p.part_bf16) ((uint16_t*)p.part_u)[o] = f2bf(v);
      else ((float*)p.part_u)[o] = v;
    }
  }
  for (int r = row0 + tid; r < row0 + nrows; r += kThreads) {
    if (p.n_split == 1) {
      if (p.lse) p.lse[(size_t)b * p.R + r] = v;
    } else {
      float* ml = p.part_ml + (((size_t)b * p.n_split + k) * p.R + r) * 2;
      ml[0] = v;
      ml[1] = v;
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_pipe_kernel(DecodeParams p) {
  using LY = Lay<FP8>;
  constexpr int kNB = LY::kNB;
  constexpr int kQInLds = LY::kQInLds;
  constexpr int kOffQ = LY::kOffQ;
  constexpr int kCopies = LY::kCopies;
  __shared__ __attribute__((aligned(16))) char smem_raw[LY::kLdsBytes];
  lds_char* const smem = (lds_char*)smem_raw;

  const int bid = blockIdx.x;
  const int unit = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (unit >= p.n_units) return;
  const int g_unit = unit % p.G;
  const int bk = unit / p.G;
  const int k = bk % p.n_split;
  const int b = bk / p.n_split;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(w >= 0 && w < kThreads / 64);

  const int row0 = g_unit * kRows;
  const int tok0 = k * p.split_tokens;
  const int pg_begin = tok0 / kPage;

  // ---- one round trip: the sequence length, the split's page ids and the
  // absorbed queries load together (none of the addresses depends on L) ----
  // L through a vector load (a laundered zero index): a scalar load would
  // share lgkmcnt with the kernel-argument loads, and the first wait for an
  // argument would then wait for L as well
  int zero = 0;
  asm volatile("" : "+v"(zero));
  const int L_raw = p.seq_lens[b + zero];
  const int32_t* const btrow = p.block_table + (size_t)b * p.max_pages;
  const int pg_cap = min(p.split_tokens / kPage, p.max_pages - pg_begin);   // >= the split's pages
  int idr[kMaxSplitPages / kThreads];
#pragma clang loop unroll(full)
  for (int i = 0; i < kMaxSplitPages / kThreads; ++i) {
    const int j = tid + i * kThreads;
    idr[i] = j < pg_cap ? btrow[pg_begin + j] : 0;
  }
  const int id0_raw = btrow[pg_begin];
  // Absorbed queries of the wave's 32 rows as MFMA B fragments, lane = row
  // (lane & 31), half h = lane >> 5: 32 latent k-steps (dims 16 ks + 8h..+7)
  // and 4 rope k-steps of 16.
  const int my_row = row0 + 32 * w + (lane & 31);
  const int h = lane >> 5;
  const int t32 = lane & 31;
  bf16x8_t qB[36];
  {
    const bool live = my_row < p.R;
    const size_t qrow = (size_t)b * p.R + (live ? my_row : 0);
    const uint16_t* ql = (const uint16_t*)p.q_lat + qrow * p.q_lat_stride + 8 * h;
    const uint16_t* qr = (const uint16_t*)p.q_rope + qrow * p.q_rope_stride + 8 * h;
#pragma clang loop unroll(full)
    for (int ks = 0; ks < 36; ++ks) {
      const bf16x8_t v = load_bf16x8(ks >= 32 ? qr + 16 * (ks - 32) : ql + 16 * ks);
      qB[ks] = live ? v : (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // keep these loads above the branches on L below (sunk past them, they
  // would wait a round trip for L before even being issued)
  asm volatile("" ::: "memory");

  const int L = __builtin_amdgcn_readfirstlane(L_raw);
  const int tok1 = min(tok0 + p.split_tokens, L);
  const int pg_end = (tok1 + kPage - 1) / kPage;
  const int n_tiles = (tok1 - tok0 + kTile - 1) / kTile;
  const bool seq_bad = (L < p.T) || (L > p.max_seq_len) ||
                       ((L + kPage - 1) / kPage > p.max_pages) ||
                       (pg_end - pg_begin) > kMaxSplitPages;
  if (seq_bad) {
    vm_wait<0>();
    write_uniform(p, b, k, row0, __builtin_nanf(""));
    return;
  }
  if (tok0 >= tok1) {   // split past the end of the sequence: no partial
    vm_wait<0>();
    return;
  }
  // visible-token limit of the row: s < min(L - T + t + 1, tok1)
  const int lim = min(L - p.T + (my_row < p.R ? my_row / p.H : 0) + 1, tok1);

  int* const ids = (int*)(smem_raw + LY::kOffIds);  // page ids of the split (filled below)
  // copies: latent row 4w + 16g + j takes chunk lane ^ (4j + w) (its gsw);
  // rope token 8w + lane / 8 takes chunk (lane & 7) ^ swz_rope(token)
  const uint32_t lane16 = (uint32_t)lane << 4;
  const uint32_t rope_v = (uint32_t)((lane >> 3) * 128 + (((lane & 7) ^ swz_rope(8 * w + (lane >> 3))) << 4));

  // ---- page copies ------------------------------------------------------------
  const char* const ckv_base = (const char*)p.ckv;
  const char* const kr_base = (const char*)p.kr;
  const char* const scale_base = (const char*)p.ckv_scale;
  struct TileSrc {
    const char* cp;
    const char* rp;
    const char* sp;    // fp8: the page's scales
    int lds, ssc, sb, last;
  };
  // tile jt of the split into buffer jdst: a tile past the split's end
  // re-reads the split's last tile
  auto page_slot = [&](int jt) __attribute__((always_inline)) -> int {
    return (min(jt, n_tiles - 1) * kTile) / kPage;
  };
  auto tile_src = [&](int jt, int jdst, int id) __attribute__((always_inline)) -> TileSrc {
    const int jc = min(jt, n_tiles - 1);
    const int t0 = tok0 + jc * kTile;                  // first token of the tile
    const size_t idc = (size_t)id;                     // checked in [0, n_pages)
    TileSrc ts;
    ts.cp = ckv_base + idc * (kPage * (FP8 ? kLat8 : kLatRow));
    ts.rp = kr_base + idc * (kPage * kDr * 2);
    ts.sp = FP8 ? scale_base + idc * (kPage * 4) : nullptr;
    ts.lds = (jdst % kNB) * kTileBytes;
    ts.ssc = LY::kOffStage + kStageScale + (jdst & 1) * (kTile * 4);
    ts.sb = t0 & (kPage - 1);
    ts.last = min(L - 1 - (t0 - ts.sb), kPage - 1);    // in [0, 63]
    return ts;
  };
  // copy op `op` (0-8) of a tile by this wave: ops 0-7 latent row
  // 4w + 16 (op / 4) + op % 4, op 8 the rope of tokens 8w..8w + 7. The fast
  // form assumes every slot of the tile holds a token (the copies of a row
  // group share one base, the row's offset rides in the instruction); the
  // safe form reads page slot min(sb + t, last) for slot sb + t.
  // fp8 (ops 0-5): ops 0-3 the latent codes of tokens 8w + 2 op (lanes 0-31)
  // and 8w + 2 op + 1 (lanes 32-63) into the wave's staging rows, op 4 the
  // rope rows as for bf16, op 5 the scales of tokens 8w..8w + 7 (lanes 0-7).
  auto copy_op = [&](const TileSrc& ts, int op, auto safe_c) __attribute__((always_inline)) {
    constexpr bool kSafe = decltype(safe_c)::value;
    const lds_char* const dst = smem + ts.lds;
    if constexpr (FP8) {
      if (op < 4) {
        const int t0 = 8 * w + 2 * op;
        if constexpr (!kSafe) {
          const char* const gb = ts.cp + (size_t)(ts.sb + 8 * w) * kLat8;
          const lds_char* const lb = smem + LY::kOffStage + 8 * w * kLat8;
          if (op == 0) dma_copy16_off<0>(gb, lane16, lb);
          else if (op == 1) dma_copy16_off<1024>(gb, lane16, lb);
          else if (op == 2) dma_copy16_off<2048>(gb, lane16, lb);
          else dma_copy16_off<3072>(gb, lane16, lb);
        } else {
          const int r = min(ts.sb + t0 + (lane >> 5), ts.last);
          dma_copy16_m0(ts.cp, ((uint32_t)r * kLat8) + ((uint32_t)(lane & 31) << 4),
                        smem + LY::kOffStage + t0 * kLat8);
        }
      } else if (op == 4) {
        if constexpr (!kSafe) {
          dma_copy16_m0(ts.rp + (size_t)(ts.sb + 8 * w) * 128, rope_v, dst + kRopeOff + w * 1024);
        } else {
          const int t = 8 * w + (lane >> 3);
          dma_copy16_m0(ts.rp, ((uint32_t)min(ts.sb + t, ts.last) << 7) + (rope_v & 127u),
                        dst + kRopeOff + w * 1024);
        }
      } else if (lane < 8) {
        const uint32_t r = kSafe ? (uint32_t)min(ts.sb + 8 * w + lane, ts.last)
                                 : (uint32_t)(ts.sb + 8 * w + lane);
        dma_copy4_m0(ts.sp, r << 2, smem + ts.ssc + 32 * w);
      }
      return;
    }
    if (op < 8) {
      const int g = op >> 2, j = op & 3;
      const int t0 = 4 * w + 16 * g;
      const uint32_t cv = lane16 ^ (uint32_t)((4 * j + w) << 4);
      if constexpr (!kSafe) {
        const char* const gb = ts.cp + (size_t)(ts.sb + t0) * kLatRow;
        const lds_char* const lb = dst + t0 * kLatRow;
        if (j == 0) dma_copy16_off<0>(gb, cv, lb);
        else if (j == 1) dma_copy16_off<1024>(gb, cv, lb);
        else if (j == 2) dma_copy16_off<2048>(gb, cv, lb);
        else dma_copy16_off<3072>(gb, cv, lb);
      } else {
        const int r = min(ts.sb + t0 + j, ts.last);
        dma_copy16_m0(ts.cp + (size_t)r * kLatRow, cv, dst + (t0 + j) * kLatRow);
      }
    } else {
      if constexpr (!kSafe) {
        dma_copy16_m0(ts.rp + (size_t)(ts.sb + 8 * w) * 128, rope_v, dst + kRopeOff + w * 1024);
      } else {
        const int t = 8 * w + (lane >> 3);
        dma_copy16_m0(ts.rp, ((uint32_t)min(ts.sb + t, ts.last) << 7) + (rope_v & 127u),
                      dst + kRopeOff + w * 1024);
      }
    }
  };
  auto read_id = [&](int jt) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane(ids[page_slot(jt)]);
  };
  // copy ops [op0, op1) of tile jt into buffer jdst
  auto copy_tile = [&](int jt, int jdst, int op0, int op1) __attribute__((always_inline)) {
    const TileSrc ts = tile_src(jt, jdst, read_id(jt));
#pragma clang loop unroll(full)
    for (int op = 0; op < kCopies; ++op)
      if (op >= op0 && op < op1) copy_op(ts, op, std::true_type{});
  };

  // ---- fp8 widening -------------------------------------------------------------
  // Piece j of the wave: token t = 8w + 2j + hb (hb = lane >> 5), codes
  // 16 p .. 16 p + 15 (p = lane & 31), i.e. bf16 chunks 2p and 2p + 1 of the
  // tile row. Op 3j reads the codes and the token's scale, ops 3j + 1 and
  // 3j + 2 widen and write chunk 2p + hf (hf = op - 3j - 1): bf16(scale x
  // code), in the tile's swizzled layout. The chunk's position in the row,
  // (2p + hf) ^ gsw(t), splits into a lane part X = 2p ^ 4hb and a part
  // C = 8 (j & 1) ^ ((2w + (j >> 1)) & 3) ^ hf that is uniform over the wave,
  // so the write address is (row base of 8w + hb, plus 16 X) ^ 16 C, plus
  // 2048 j: X, and the tile buffer's base (a multiple of 1 KB), leave bits
  // 4-9 to the XOR alone.
  const int cv_read = LY::kOffStage + 8 * w * kLat8 + lane * 16;   // + 1024 j
  const int cv_scale = 32 * w + 4 * (lane >> 5);                    // + scale buffer + 8 j
  const int cv_row = ((lane >> 5) << 10) + ((2 * (lane & 31)) ^ (4 * (lane >> 5))) * 16 +
                     8 * w * kLatRow;                               // + tile buffer
  u32x4_t craw = {0u, 0u, 0u, 0u};
  float csc = 0.f;
  // sa: scale buffer + cv_scale; za: tile buffer + cv_row
  auto conv_op = [&](int op, int sa, int za) __attribute__((always_inline)) {
    const int j = op / 3, part = op % 3;
    if (part == 0) {
      craw = *(const MLA_LDS u32x4_t*)(smem + cv_read + 1024 * j);
      csc = *(const MLA_LDS float*)(smem + sa + 8 * j);
      return;
    }
    const int hf = part - 1;
    typedef float f2_t __attribute__((ext_vector_type(2)));
    uint32_t o[4];
#pragma clang loop unroll(full)
    for (int d = 0; d < 2; ++d) {
      const f2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(craw[2 * hf + d], 1.0f, false);
      const f2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(craw[2 * hf + d], 1.0f, true);
      o[2 * d] = pack_bf16x2(lo[0] * csc, lo[1] * csc);
      o[2 * d + 1] = pack_bf16x2(hi[0] * csc, hi[1] * csc);
    }
    const int C = (8 * (j & 1)) ^ ((2 * w + (j >> 1)) & 3) ^ hf;
    *(MLA_LDS u32x4_t*)(smem + (za ^ (C << 4)) + 2048 * j) = (u32x4_t){o[0], o[1], o[2], o[3]};
  };
  auto conv_tile = [&](int jt) __attribute__((always_inline)) {
    const int sa = LY::kOffStage + kStageScale + (jt & 1) * (kTile * 4) + cv_scale;
    const int za = (jt % kNB) * kTileBytes + cv_row;
#pragma clang loop unroll(full)
    for (int op = 0; op < 12; ++op) conv_op(op, sa, za);
  };

  // ---- the first two tiles (both in the split's first page) go out now; a
  // bad first page id is caught with the others below, before any tile is
  // read --------------------------------------------------------------------
  const int n_pg = pg_end - pg_begin;
  const int id0 = __builtin_amdgcn_readfirstlane(id0_raw);
  const bool id0_ok = id0 >= 0 && id0 < p.n_pages;
  if (id0_ok) {
    const TileSrc t0s = tile_src(0, 0, id0), t1s = tile_src(1, 1, id0);
#pragma clang loop unroll(full)
    for (int op = 0; op < kCopies; ++op) copy_op(t0s, op, std::true_type{});
    // (fp8: tile 1's codes wait for the staging rows that tile 0's occupy)
#pragma clang loop unroll(full)
    for (int op = FP8 ? 4 : 0; op < kCopies; ++op) copy_op(t1s, op, std::true_type{});
  }
  // the group's earliest limit: tiles ending before it need no mask
  const int lim_min = min(L - p.T + min(row0, p.R - 1) / p.H + 1, tok1);

  bool bad = false;
#pragma clang loop unroll(full)
  for (int i = 0; i < kMaxSplitPages / kThreads; ++i) {
    const int j = tid + i * kThreads;
    if (j < n_pg) {
      bad |= (idr[i] < 0) || (idr[i] >= p.n_pages);
      ids[j] = idr[i];
    }
  }
  if (__syncthreads_or(bad)) {
    vm_wait<0>();                                    // the first copies land before LDS is released
    write_uniform(p, b, k, row0, __builtin_nanf(""));
    return;
  }
  // (the barrier above also published the page ids)
  const float sl = p.scale_log2;

  // ---- per-lane LDS offsets within a tile buffer ---------------------------------
  // Recomputed from a laundered lane index where needed (a few VALU
  // instructions) instead of being kept live through the passes.
  // score: latent k-step ks reads chunk 2 ks + h of token t32 at
  //   sb8[ks & 7] + 256 (ks >> 3); rope k-step r reads rb4[r]
  // aggregation: the 16-lane group G of half h reads dims 16 G + 4 (i & 3) of
  // token rows 16 kk + 4h + i / 4 (lo) and 16 kk + 8 + 4h + i / 4 (hi); dim
  // block db = 4 a + bb sits at 64 (bb ^ (i / 4)) + 256 a in the row
  struct Offs {
    int sb8[8], rb4[4], pb8[8];
  };
  auto offsets = [&]() __attribute__((always_inline)) -> Offs {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int t = ln & 31, hh = ln >> 5;
    Offs o;
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) o.sb8[j] = t * kLatRow + 16 * ((2 * j + hh) ^ gsw(t));
#pragma clang loop unroll(full)
    for (int r = 0; r < 4; ++r) o.rb4[r] = kRopeOff + t * 128 + 16 * ((2 * r + hh) ^ swz_rope(t));
    const int i = ln & 15, G = (ln >> 4) & 1;
    const int c_lo = 2 * G + ((i >> 1) & 1);
    const int tr_row = (4 * hh + (i >> 2)) * kLatRow;
#pragma clang loop unroll(full)
    for (int bb = 0; bb < 4; ++bb) {
      const int off = tr_row + 64 * (bb ^ (i >> 2)) + 8 * (i & 1);
      o.pb8[bb] = off + 16 * (c_lo ^ hh);
      o.pb8[4 + bb] = off + 8 * kLatRow + 16 * (c_lo ^ (hh + 2));
    }
    return o;
  };
  // Each row's reference maximum is fixed in the first tile, where every row
  // with a visible token in the split sees one (the split's first token is
  // visible to every row that sees any), so the latent aggregate in the MFMA
  // accumulators is never rescaled inside the loop. Should a later tile's
  // maximum exceed the reference by more than kJump (log2 units) -- or a row
  // sum overflow -- the unit runs a second pass over its tiles with every
  // reference at the true row maximum found by the first.
  f32x16_t U[16];                            // U^T: dims 32 db + 8 (q / 4) + 4h + q % 4
  float m_r, l_r;                            // reference max (log2 units); lane's share of l
  float m_true = -INFINITY;                  // running true row maximum (log2 units)

  // the query operand of score k-step ks (the first kQInLds from LDS)
  auto qop = [&](int ks) __attribute__((always_inline)) -> bf16x8_t {
    if (ks < kQInLds) return lds_read_b128(smem + kOffQ + (w * kQInLds + ks) * 1024 + lane * 16);
    return qB[ks];
  };

  // ---- score pieces -----------------------------------------------------------
  auto sfrag = [&](const Offs& o, int sbuf, int ks) __attribute__((always_inline)) -> bf16x8_t {
    if (ks >= 32) return lds_read_b128(smem + sbuf + o.rb4[ks - 32]);
    return lds_read_b128(smem + sbuf + o.sb8[ks & 7] + 256 * (ks >> 3));
  };
  auto gfrag = [&](const Offs& o, int gbuf, int e2) __attribute__((always_inline)) -> bf16x8_t {
    const int kk = e2 >> 4, db = e2 & 15;
    const int imm = 16 * kk * kLatRow + 256 * (db >> 2);
    const bf16x4_t lo = lds_read_tr16(smem + gbuf + o.pb8[db & 3] + imm);
    const bf16x4_t hi = lds_read_tr16(smem + gbuf + o.pb8[4 + (db & 3)] + imm);
    return concat(lo, hi);
  };
  // scores of tile jt -> probabilities (B operands of its two aggregation
  // k-steps: k-step kk holds the lane's values 8 kk..8 kk + 7, tokens
  // 16 kk + {4h..4h+3, 8+4h..8+4h+3}); the row sum adds the same bf16
  // values. In ten stages, so that steps can spread them between MFMAs:
  // 0 mask and maximum, 1 references, 2-5 the first k-step (P0), 6-9 the
  // second (P1) from the scores' upper half kept in Sh.
  struct SoftmaxCarry {
    float nbase, ls;
    float Sh[8];
    uint32_t pk[4];
  };
  auto prob_pair = [&](float s0, float s1, SoftmaxCarry& c, uint32_t& pk) __attribute__((always_inline)) {
    const float e0 = fast_exp2(fmaf(s0, sl, c.nbase));
    const float e1 = fast_exp2(fmaf(s1, sl, c.nbase));
    pk = pack_bf16x2(e0, e1);
    c.ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                           (bf16x2_t){(__bf16)1.0f, (__bf16)1.0f}, c.ls, false);
  };
  auto head_stage = [&](int st, f32x16_t& S, int jt, bool first, SoftmaxCarry& c, bf16x8_t& P0)
      __attribute__((always_inline)) {
    if (st == 0) {
      const int stok = tok0 + jt * kTile;
      if (stok + kTile > lim_min) {
#pragma clang loop unroll(full)
        for (int q = 0; q < 16; ++q)
          if (stok + 8 * (q >> 2) + 4 * h + (q & 3) >= lim) S[q] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(S[0], S[1]), S[2]);
#pragma clang loop unroll(full)
      for (int q = 3; q < 15; q += 2) mx = fmaxf(fmaxf(mx, S[q]), S[q + 1]);
      c.nbase = fmaxf(mx, S[15]);
    } else if (st == 1) {
      const float mx = c.nbase;
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      const float mt = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * sl;
      m_true = fmaxf(m_true, mt);
      if (first && m_r == -INFINITY) m_r = mt;        // the row's reference (U = 0)
      c.nbase = (m_r == -INFINITY) ? 0.f : -m_r;
      c.ls = 0.f;
    } else {
      const int q = 2 * (st - 2);
      prob_pair(S[q], S[q + 1], c, c.pk[q >> 1]);
      if (st == 5) {
        P0 = __builtin_bit_cast(bf16x8_t, (u32x4_t){c.pk[0], c.pk[1], c.pk[2], c.pk[3]});
#pragma clang loop unroll(full)
        for (int j = 0; j < 8; ++j) c.Sh[j] = S[8 + j];
      }
    }
  };
  auto tail_stage = [&](int st, SoftmaxCarry& c, bf16x8_t& P1) __attribute__((always_inline)) {
    const int j = 2 * (st - 6);
    prob_pair(c.Sh[j], c.Sh[j + 1], c, c.pk[j >> 1]);
    if (st == 9) {
      P1 = __builtin_bit_cast(bf16x8_t, (u32x4_t){c.pk[0], c.pk[1], c.pk[2], c.pk[3]});
      l_r += c.ls;
    }
  };

  bf16x8_t P[2];                              // probabilities of the tile being aggregated
  SoftmaxCarry carry;                         // the second half of P still to compute
  // operands of slot i are read after the MFMA of slot i - kDist; the reads
  // of a step's first kDist slots lead it (those of its aggregation MFMAs
  // before the barrier that precedes the step)
  constexpr int kDist = 3;
  static_assert(kLeadG < kDist && slot_is_score(kLeadG), "lead reads");
  bf16x8_t ring[kDist];
  int gb[8], sb[8], rb[4];                    // this step's LDS bases (aggregation, score)
  auto set_bases = [&](int gbuf, int sbuf) __attribute__((always_inline)) {
    const Offs o = offsets();
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) gb[j] = gbuf + o.pb8[j];
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) sb[j] = sbuf + o.sb8[j];
#pragma clang loop unroll(full)
    for (int r = 0; r < 4; ++r) rb[r] = sbuf + o.rb4[r];
  };
  auto sread = [&](int ks) __attribute__((always_inline)) -> bf16x8_t {
    if (ks >= 32) return lds_read_b128(smem + rb[ks - 32]);
    return lds_read_b128(smem + sb[ks & 7] + 256 * (ks >> 3));
  };
  auto gread = [&](int e2) __attribute__((always_inline)) -> bf16x8_t {
    const int kk = e2 >> 4, db = e2 & 15;
    const int imm = 16 * kk * kLatRow + 256 * (db >> 2);
    const bf16x4_t lo = lds_read_tr16(smem + gb[db & 3] + imm);
    const bf16x4_t hi = lds_read_tr16(smem + gb[4 + (db & 3)] + imm);
    return concat(lo, hi);
  };
  auto fetch = [&](int i) __attribute__((always_inline)) {
    ring[i % kDist] = slot_is_score(i) ? sread(slot_index(i)) : gread(slot_index(i));
  };
  auto lead_reads = [&]() __attribute__((always_inline)) {
#pragma clang loop unroll(full)
    for (int i = 0; i < kLeadG; ++i) fetch(i);
  };

  // the first tile of a pass: 36 score MFMAs on two chains, then the softmax
  // that fixes the references; the copies of tile 2 ride along
  auto first_step = [&]() __attribute__((always_inline)) {
    const TileSrc cts = tile_src(2, 2, read_id(2));
    const Offs o = offsets();
    bf16x8_t qL[kQInLds];
#pragma clang loop unroll(full)
    for (int j = 0; j < kQInLds; ++j) qL[j] = qop(j);
    constexpr int kRing = 7;
    bf16x8_t fr[kRing];
#pragma clang loop unroll(full)
    for (int f = 0; f < kRing; ++f) fr[f] = sfrag(o, 0, f);
    f32x16_t SA, SB;
    __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
    for (int ks = 0; ks < 36; ++ks) {
      const bf16x8_t av = fr[ks % kRing];
      f32x16_t& acc = (ks & 1) ? SB : SA;
      const bf16x8_t qv = ks < kQInLds ? qL[ks] : qB[ks];
      if (ks < 2) mfma_sc0(acc, av, qv);
      else mfma_sc(acc, av, qv);
      if (ks + kRing < 36) fr[ks % kRing] = sfrag(o, 0, ks + kRing);
      if (ks % 4 == 1 && ks / 4 < kCopies) copy_op(cts, ks / 4, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    score_fence(SA, SB);
    SA += SB;
#pragma clang loop unroll(full)
    for (int st = 0; st < 6; ++st) head_stage(st, SA, 0, true, carry, P[0]);
  };

  // steady-state step s: aggregation of tile s (bases gb, probabilities P)
  // interleaved with the scores of tile s + 1 (bases sb, rb), whose softmax
  // refills P; the copies of tile s + 3 (page id cid) go to buffer
  // (s + 3) % 4. Returns the page id for the next step's copies.
  auto step = [&](int s, int cid, auto safe_c) __attribute__((always_inline)) -> int {
    const TileSrc cts = tile_src(s + 3, s + 3, cid);
    // fp8: tile s + 2 is widened from the staging rows into its tile buffer
    const int csa = LY::kOffStage + kStageScale + ((s + 2) & 1) * (kTile * 4) + cv_scale;
    const int cza = ((s + 2) % kNB) * kTileBytes + cv_row;
    bf16x8_t qL[kQInLds];
#pragma clang loop unroll(full)
    for (int j = 0; j < kQInLds; ++j) qL[j] = qop(j);
#pragma clang loop unroll(full)
    for (int i = kLeadG; i < kDist; ++i) fetch(i);
    f32x16_t SA, SB;
    int idv = 0, nid = 0;
    __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
    for (int i = 0; i < kSlots; ++i) {
      if (slot_is_score(i)) {
        const int ks = slot_index(i);
        f32x16_t& acc = (ks & 1) ? SB : SA;
        const bf16x8_t qv = ks < kQInLds ? qL[ks] : qB[ks];
        if (ks < 2) mfma_sc0(acc, ring[i % kDist], qv);
        else mfma_sc(acc, ring[i % kDist], qv);
      } else {
        const int e2 = slot_index(i);
        U[e2 & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % kDist], P[e2 >> 4], U[e2 & 15], 0, 0, 0);
      }
      if (i + kDist < kSlots) fetch(i + kDist);
      if constexpr (FP8) {
        const int cv = conv_at(i);
        if (cv >= 0 && cv % 3 == 0) vm_wait<kConvInFlight>();   // the piece's codes and scales
        if (cv >= 0) conv_op(cv, csa, cza);
        if (copy_at8(i) >= 0) copy_op(cts, copy_at8(i), safe_c);
      } else {
        if (copy_at16(i) >= 0) copy_op(cts, copy_at16(i), safe_c);
      }
      if (i == kIdRead) idv = ids[page_slot(s + 4)];
      if (i == kIdUse) nid = __builtin_amdgcn_readfirstlane(idv);
      if (i == kLastScore + 1) score_fence(SA, SB);
      if (i == kTailFrom) SA += SB;
#pragma clang loop unroll(full)
      for (int st = 6; st < 10; ++st)
        if (tail_stage_slot(st) == i) tail_stage(st, carry, P[1]);
      if (head_stage_at(i) >= 0) head_stage(head_stage_at(i), SA, s + 1, false, carry, P[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // next step's buffers: one tile further, modulo the ring
    const int d = ((s + 1) % kNB == 0) ? -(kNB - 1) * kTileBytes : kTileBytes;
    const int d2 = ((s + 2) % kNB == 0) ? -(kNB - 1) * kTileBytes : kTileBytes;
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) gb[j] += d;
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) sb[j] += d2;
#pragma clang loop unroll(full)
    for (int r = 0; r < 4; ++r) rb[r] += d2;
    return nid;
  };

  // the last tile: its aggregation alone
  auto last_step = [&](int s) __attribute__((always_inline)) {
    const int gbuf = (s % kNB) * kTileBytes;
    const Offs o = offsets();
    constexpr int kRing = 7;
    bf16x8_t fr[kRing];
#pragma clang loop unroll(full)
    for (int e2 = 0; e2 < kRing; ++e2) fr[e2] = gfrag(o, gbuf, e2);
#pragma clang loop unroll(full)
    for (int st = 6; st < 10; ++st) tail_stage(st, carry, P[1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
    for (int e2 = 0; e2 < 32; ++e2) {
      const bf16x8_t av = fr[e2 % kRing];
      if (e2 + kRing < 32) fr[e2 % kRing] = gfrag(o, gbuf, e2 + kRing);
      U[e2 & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, P[e2 >> 4], U[e2 & 15], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma clang loop unroll(full)
    for (int db = 0; db < 16; ++db)
#pragma clang loop unroll(full)
      for (int q = 0; q < 16; ++q) U[db][q] = 0.f;
    m_r = pass == 0 ? -INFINITY : m_true;
    l_r = 0.f;
    // tiles 0 and 1 (a split of one tile re-reads it into buffer 1); the
    // first pass's went out before the queries loaded
    if (pass > 0) {
      copy_tile(0, 0, 0, kCopies);
      copy_tile(1, 1, FP8 ? 4 : 0, kCopies);
    }
    if constexpr (FP8) {
      // tiles 0 and 1 widened (each wave its own tokens) before the barrier;
      // tile 1's codes go out once tile 0's have been widened
      vm_wait<0>();
      conv_tile(0);
      copy_tile(1, 1, 0, 4);
      vm_wait<0>();
      conv_tile(1);
    } else {
      vm_wait<kCopies>();
    }
    if (pass == 0) {
      // (after the wait: an earlier store would wait for the first copies
      // before the queries were needed)
#pragma clang loop unroll(full)
      for (int ks = 0; ks < kQInLds; ++ks)
        *(MLA_LDS bf16x8_t*)(smem + kOffQ + (w * kQInLds + ks) * 1024 + lane * 16) = qB[ks];
    }
    lds_barrier();                                     // tile 0 resident
    first_step();                                      // also copies tile 2
    set_bases(0, kTileBytes);
    int cid = read_id(3);
    lead_reads();
    vm_wait<kCopies>();
    lds_barrier_keep<2 * kLeadG>();                    // tile 1 resident (bf16)
    // after step s: tile s + 2 resident (the copies of tile s + 3 may fly),
    // tile s's buffer free; the lead reads of step s + 1 may still fly
    const int n_fast = max(n_tiles - 4, 0);            // steps whose copy tile is full
    for (int s = 0; s < n_fast; ++s) {
      cid = step(s, cid, std::false_type{});
      lead_reads();
      vm_wait<kCopies>();
      lds_barrier_keep<2 * kLeadG>();
    }
    for (int s = n_fast; s + 1 < n_tiles; ++s) {
      cid = step(s, cid, std::true_type{});
      lead_reads();
      vm_wait<kCopies>();
      lds_barrier_keep<2 * kLeadG>();
    }
    last_step(n_tiles - 1);
    vm_wait<0>();   // the re-read copies land before LDS is reused
    // a second pass is needed when a row's maximum jumped past its reference
    // or a row sum left the finite range
    const bool jumped = m_true - m_r > kJump || !(l_r < INFINITY);
    if (!__syncthreads_or(jumped)) break;
  }

  // ---- finish -------------------------------------------------------------------
  float l_row;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_r), __float_as_uint(l_r), false, false);
    l_row = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const bool direct = p.n_split == 1;
  const size_t row_base = direct ? (size_t)b * p.R : ((size_t)b * p.n_split + k) * p.R;
  const bool out16 = direct ? p.out_bf16 != 0 : p.part_bf16 != 0;
  const bool normalise = direct || out16;   // fp32 partials keep U unnormalised
  const float inv = normalise ? (l_row > 0.f ? 1.f / l_row : 0.f) : 1.f;
  void* const dst = direct ? p.out : p.part_u;
  if (out16) {
    // bf16 rows through LDS (every wave's reads of the tiles ended at the
    // pass loop's last barrier): the wave writes its 32 rows of 1 KB with
    // 16-byte chunk c of row r at c ^ r, then stores one whole row per
    // instruction
    lds_char* const rows = smem + w * 32 * 1024;
#pragma clang loop unroll(full)
    for (int db = 0; db < 16; ++db) {
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j) {
        const f32x4_t v = (f32x4_t){U[db][4 * j], U[db][4 * j + 1], U[db][4 * j + 2], U[db][4 * j + 3]} * inv;
        const int c = 4 * db + j;                        // dims 32 db + 8 j .. + 7
        *(MLA_LDS u32x2_t*)(rows + t32 * 1024 + ((c ^ t32) << 4) + 8 * h) =
            (u32x2_t){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
    uint16_t* const out_rows = (uint16_t*)dst + (row_base + row0 + 32 * w) * kDc;
    const int live_rows = min(32, p.R - (row0 + 32 * w));
#pragma clang loop unroll(full)
    for (int r = 0; r < 32; ++r) {
      if (r < live_rows) {
        const u32x4_t v = *(const MLA_LDS u32x4_t*)(rows + r * 1024 + ((lane ^ r) << 4));
        *(u32x4_t*)(out_rows + r * kDc + lane * 8) = v;
      }
    }
  } else if (my_row < p.R) {
#pragma clang loop unroll(full)
    for (int db = 0; db < 16; ++db) {
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j) {
        const size_t o = (row_base + my_row) * kDc + 32 * db + 8 * j + 4 * h;
        const f32x4_t v = (f32x4_t){U[db][4 * j], U[db][4 * j + 1], U[db][4 * j + 2], U[db][4 * j + 3]} * inv;
        *(f32x4_t*)((float*)dst + o) = v;
      }
    }
  }
  if (my_row < p.R && lane < 32) {
    if (direct) {
      if (p.lse) p.lse[(size_t)b * p.R + my_row] = (m_r + log2f(l_row)) * kLn2;
    } else {
      p.part_ml[(row_base + my_row) * 2] = m_r;
      p.part_ml[(row_base + my_row) * 2 + 1] = l_row;
    }
  }
}

}  // namespace

hipError_t launch_decode_pipe(const DecodeParams& p, bool fp8, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL(decode_pipe_kernel<true>, dim3(p.per_xcd * kNumXcd), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(decode_pipe_kernel<false>, dim3(p.per_xcd * kNumXcd), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
