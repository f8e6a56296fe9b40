// Paged absorbed-MLA decode on gfx950 MFMA, for bf16 caches and for fp8
// (OCP E4M3FN) latent caches with one fp32 scale per token.
//
// A workgroup of four waves (one per SIMD) owns a work unit: sequence b,
// split k and a group of ROWS query rows (64 or 128). The split's cache
// streams through LDS in tiles of 32 tokens (half a page): 512 latent and 64
// rope elements per token, the 576-element cache of PaperTrace "02 ·
// DeepSeek-V2 analysis", section 1.3.
//
// Every wave is a complete attention worker for 32 query rows, on the
// 32x32x16 bf16 MFMA (on gfx950 the 16x16x32 form issues at about half its
// rate from one wave per SIMD). It keeps its rows' absorbed queries in
// registers (the B operands of the score), computes a tile's scores as
// S^T[token][row] = K[token][576] Q^T (section 1.3, eq. 18; the 1/sqrt(192)
// scale is folded into the exponent), runs the online softmax of its rows in
// registers (a lane owns one row; the two lane halves meet in one permlane
// swap), and accumulates the latent aggregate U^T[dim][row] += C^T[dim][token]
// P^T[token][row], reading the latent tile transposed (ds_read_b64_tr_b16 /
// _b8): each head aggregates the shared latents with its own weights and
// W^UV is applied afterwards (section 6.1). The probabilities never leave the
// registers: the score output layout is already the B operand of the
// aggregation once the transposed reads order the tokens to match. No wave
// waits for another except at the one workgroup barrier per step.
//
// With 64 rows the four waves are two row halves x two tile parities: in
// step s the waves of parity th work on tile 2s + th, so each tile is read by
// two waves and every step consumes one page; the two parities run separate
// online softmaxes, merged through LDS at the end. With 128 rows each wave
// owns a row quarter and all four read every tile, one tile per step.
//
// Page copies are asynchronous (global_load_lds_dwordx4, 1 KB per
// instruction) into a ring of tile buffers, issued by all four waves LA steps
// ahead of use and interleaved with the MFMAs; each wave waits for its own
// copies with vmcnt before the barrier that publishes them. A copy never
// reads past the sequence: slots beyond its last token repeat the last
// token, and the mask gives them weight exactly 0.
//
// fp8 latent caches stay fp8 in LDS. Every E4M3FN code is widened exactly to
// bf16 in registers before its MFMA, so the cache's own rounding is the only
// quantization on the path. The token scale multiplies the latent score in
// fp32, z = scale_s (q_lat . code_s) + q_rope . k^R_s, and is folded into the
// probability used for the aggregation, P' = p scale_s.
//
// The unit ends by writing either u = U / l and lse (one split), or partials
// for the log-sum-exp combine: bf16 u = U / l with fp32 (m, l) when the
// output is bf16, else fp32 (m, l, U).
#include "dma.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <bool FP8>
struct Geo {
  static constexpr int kLatRow = FP8 ? 512 : 1024;        // bytes of one token's latent
  static constexpr int kLatBytes = kTile * kLatRow;
  static constexpr int kRopeOff = kLatBytes;              // rope rows of 128 B (bf16)
  static constexpr int kScaleOff = kRopeOff + kTile * 128;
  static constexpr int kTileBytes = kScaleOff + (FP8 ? 256 : 0);
  static constexpr int kNumBuf = FP8 ? 6 : 4;
  static constexpr int kLatCopies = FP8 ? 16 : 32;        // 1-KB copies per tile
  static constexpr int kOffIds = kNumBuf * kTileBytes;
  static constexpr int kTilesEnd = kOffIds + kMaxSplitPages * 4;
  // end of the unit: U halves of the four waves ([wave][8 blocks][lane] x 64 B)
  // then (m, l) of the 64 rows of the two tile parities
  static constexpr int kMergeU = 4 * 32 * 1024;
  static constexpr int kOffMl = kMergeU;
  static constexpr int kMergeEnd = kOffMl + 2 * 2 * 64 * 4;
  static constexpr int kLdsBytes = kTilesEnd > kMergeEnd ? kTilesEnd : kMergeEnd;
  static_assert(kLdsBytes <= 163840, "LDS budget");
};

// LDS swizzles, chosen so that every read pattern below touches each of the
// 64 banks once per pass (16-B reads serve 16 lanes per pass: the 4-lane
// quads of a half-wave split by the parity of the quad index; 8-B and
// transposed reads serve a half-wave per pass):
//  * bf16 latent rows (1 KB): 16-B chunk c of token t at c ^ gsw(t),
//    gsw(t) = ((t & 3) << 2) | ((t >> 2) & 3). Score reads (32 tokens x one
//    chunk) and transposed reads (4 tokens x 64 B) are spread.
//  * fp8 latent rows (512 B): 16-B chunk c of token t at c ^ fsw(t), fsw a
//    bit permutation of t & 15 (bits 3,1,0,2), so score reads (32 tokens x one
//    chunk) and transposed reads (8 tokens x 32 B) are spread.
//  * rope rows (128 B): 16-B chunk c of token t at c ^ ((t >> 1) & 7).
__device__ __forceinline__ int gsw(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int fsw(int t) {
  return (t & 8) | ((t & 2) << 1) | ((t & 1) << 1) | ((t >> 2) & 1);
}
__device__ __forceinline__ int swz_rope(int t) { return (t >> 1) & 7; }

// Wait until at most N of this wave's vector-memory operations are in flight
// (6-bit vmcnt of gfx9: bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Score MFMAs (32x32x16 bf16) with their accumulators pinned to VGPRs: the
// compiler keeps the 256-register latent aggregate in AGPRs and, left to
// itself, would put every MFMA accumulator there. The hardware does not
// interlock an MFMA result against VALU reads or a VALU result against MFMA
// reads: score_fence() pads the gap before VALU reads of the scores, and the
// _v forms wait two cycles for an operand the VALU just wrote. Each chain
// has a second one interleaved with it.
__device__ __forceinline__ void mfma_sc0(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_sc(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_sc0_v(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_sc_v(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// 32 wait states between the last MFMA writing S (16 passes) and VALU reads
__device__ __forceinline__ void score_fence(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}
// 2 wait states between VALU writes of S and the MFMA that accumulates on it
__device__ __forceinline__ void valu_fence(f32x16_t& a) { asm volatile("s_nop 1" : "+v"(a)); }

// Largest excess (log2 units) of a score over its row's reference maximum in
// the first pass: probabilities stay below 2^32, row sums below 2^48.
constexpr float kJump = 32.0f;

// 8 E4M3FN bytes -> 8 bf16 (exact: every E4M3FN value is a bf16 value).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(const i32x2_t& v) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
  const bf2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
  const bf2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
  const bf2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
  return (bf16x8_t){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Every row of the unit gets (m, l, U) = (v, v, v): marks out-of-range
// sequences and page ids with NaN.
template <int ROWS>
__device__ void write_uniform(const DecodeParams& p, int b, int k, int row0, float v) {
  const int tid = threadIdx.x;
  const int nrows = min(ROWS, p.R - row0);
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

template <bool FP8, int ROWS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_split_kernel(DecodeParams p) {
  using Gm = Geo<FP8>;
  constexpr int NRB = ROWS / 32;             // 32-row blocks: 2 or 4
  constexpr int NT = 4 / NRB;                // tiles per step: 2 or 1
  constexpr int NB = Gm::kNumBuf;
  constexpr int LA = NB / NT - 1;            // copy lookahead in steps
  constexpr int kLatRow = Gm::kLatRow;
  constexpr int kTileBytes = Gm::kTileBytes;
  static_assert(NRB * NT == 4 && LA >= 1, "geometry");
  __shared__ __attribute__((aligned(16))) char smem_raw[Gm::kLdsBytes];
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
  const int rbw = w % NRB;                   // the wave's 32-row block
  const int th = w / NRB;                    // the wave's tile parity

  const int row0 = g_unit * ROWS;
  const int L = p.seq_lens[b];
  const int tok0 = k * p.split_tokens;
  const int tok1 = min(tok0 + p.split_tokens, L);
  const int pg_begin = tok0 / kPage;
  const int pg_end = (tok1 + kPage - 1) / kPage;
  const int n_tiles = (tok1 - tok0 + kTile - 1) / kTile;
  const int n_steps = (n_tiles + NT - 1) / NT;
  const bool seq_bad = (L < p.T) || (L > p.max_seq_len) ||
                       ((L + kPage - 1) / kPage > p.max_pages) ||
                       (pg_end - pg_begin) > kMaxSplitPages;
  if (seq_bad) {
    write_uniform<ROWS>(p, b, k, row0, __builtin_nanf(""));
    return;
  }
  if (tok0 >= tok1) return;   // split past the end of the sequence: no partial

  // ---- page ids of the split (global -> LDS), queries -> registers --------
  int* const ids = (int*)(smem_raw + Gm::kOffIds);
  const int32_t* const btrow = p.block_table + (size_t)b * p.max_pages;
  const int n_pg = pg_end - pg_begin;
  int idr[kMaxSplitPages / kThreads];
#pragma clang loop unroll(full)
  for (int i = 0; i < kMaxSplitPages / kThreads; ++i) {
    const int j = tid + i * kThreads;
    idr[i] = j < n_pg ? btrow[pg_begin + j] : 0;
  }

  // Absorbed queries of the wave's 32 rows as MFMA B fragments, lane = row
  // (lane & 31), half h = lane >> 5: 32 latent k-steps and 4 rope k-steps of
  // 16. bf16 k-step ks holds latent dims 16 ks + 8h..+7; fp8 pairs k-steps
  // (2p, 2p + 1) on one 16-byte read of the codes, so k-step ks holds dims
  // 32 (ks >> 1) + 16h + 8 (ks & 1)..+7.
  const int my_row = row0 + 32 * rbw + (lane & 31);
  const int hq = lane >> 5;
  bf16x8_t qB[36];
  int lim;
  {
    const bool live = my_row < p.R;
    const size_t qrow = (size_t)b * p.R + (live ? my_row : 0);
    const uint16_t* ql = (const uint16_t*)p.q_lat + qrow * kDc;
    const uint16_t* qr = (const uint16_t*)p.q_rope + qrow * kDr + 8 * hq;
#pragma clang loop unroll(full)
    for (int ks = 0; ks < 36; ++ks) {
      const uint16_t* src;
      if (ks >= 32) src = qr + 16 * (ks - 32);
      else if (FP8) src = ql + 32 * (ks >> 1) + 16 * hq + 8 * (ks & 1);
      else src = ql + 16 * ks + 8 * hq;
      const bf16x8_t v = load_bf16x8(src);
      qB[ks] = live ? v : (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
    // visible-token limit of the row: s < min(L - T + t + 1, tok1)
    const int t = live ? my_row / p.H : 0;
    lim = min(L - p.T + t + 1, tok1);
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

  // ---- per-lane offsets ---------------------------------------------------------
  // Recomputed from a laundered lane index at the top of every step (a few
  // VALU instructions) rather than kept live across the loop: the unrolled
  // reads and copies would otherwise pin dozens of registers.
  struct Lanes {
    int lane, t32, h;
    int lat_sw, rope_sw;                        // score reads of token t32
    int tr_base;                                // bf16 transposed reads: row of token 4h + i/4
    uint32_t cv[4];                             // per-lane copy source offsets (see copy_op)
    uint32_t rope_v;
  };
  auto lanes_now = [&]() __attribute__((always_inline)) -> Lanes {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    Lanes o;
    o.lane = ln;
    o.t32 = ln & 31;
    o.h = ln >> 5;
    o.lat_sw = FP8 ? fsw(o.t32) : gsw(o.t32);
    o.rope_sw = swz_rope(o.t32);
    o.tr_base = (4 * o.h + ((ln & 15) >> 2)) * kLatRow;
    // copy sources, relative to the first row of the wave's copy group (see
    // copy_op): bf16 latent rows 4w + 16g + j hold chunk c at c ^ gsw, with
    // gsw = 4j + w, so lane l fetches chunk l ^ (4j + w) of row j; fp8 row
    // pair i of rows 8w + 2i + lane / 32 takes chunk (lane & 31) ^ fsw(t) of
    // its row; rope tokens 8w + lane / 8 take chunk (lane & 7) ^ swz_rope(t)
    if constexpr (!FP8) {
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j) o.cv[j] = (uint32_t)((ln ^ (4 * j + w)) << 4);
    } else {
#pragma clang loop unroll(full)
      for (int i = 0; i < 4; ++i)
        o.cv[i] = (uint32_t)((ln >> 5) * 512 + (((ln & 31) ^ fsw(8 * w + 2 * i + (ln >> 5))) << 4));
    }
    o.rope_v = (uint32_t)((ln >> 3) * 128 + (((ln & 7) ^ swz_rope(8 * w + (ln >> 3))) << 4));
    return o;
  };

  // ---- page copies ----------------------------------------------------------
  const char* const ckv_base = (const char*)p.ckv;
  const char* const kr_base = (const char*)p.kr;
  // one tile's sources (scalar): the page's pool rows, the tile's first slot
  // in the page (0 or 32), the page's last valid slot (>= 0: a tile's page
  // always holds a token of the sequence, even when the tile itself starts
  // past the end) and the destination buffer
  struct TileSrc {
    const char* cp;
    const char* rp;
    const char* sp;
    int lds, sb, last;
    bool full;                                         // every slot holds a token
  };
  auto tile_src = [&](int jt, int id, int jdst) __attribute__((always_inline)) -> TileSrc {
    const int t0 = tok0 + jt * kTile;                  // first token of the tile
    const int sb = t0 & (kPage - 1);
    const bool ok = id >= 0 && id < p.n_pages;
    const size_t idc = ok ? (size_t)id : 0;
    TileSrc ts;
    ts.cp = ckv_base + idc * (kPage * kLatRow);
    ts.rp = kr_base + idc * (kPage * kDr * 2);
    ts.sp = FP8 ? (const char*)p.ckv_scale + idc * (kPage * 4) : nullptr;
    ts.lds = (jdst % NB) * kTileBytes;
    ts.sb = sb;
    ts.last = min(L - 1 - (t0 - sb), kPage - 1);       // in [0, 63]
    ts.full = sb + kTile - 1 <= ts.last;
    return ts;
  };
  // copy op `op` of a tile by this wave, one 1-KB (or 128-byte) copy each:
  //  bf16: ops 0-7 copy latent row 4w + 16 (op / 4) + op % 4, op 8 the rope
  //        of tokens 8w..8w + 7;
  //  fp8:  ops 0-3 copy latent rows 8w + 2 op, 8w + 2 op + 1, op 4 the rope,
  //        op 5 the 32 token scales (every wave copies the same 128 bytes, so
  //        all waves count the same number of copies).
  // The copies of a row group share one global and one LDS base (the row's
  // offset rides in the instruction). Slot sb + t reads page slot
  // min(sb + t, last), in [0, 63]: a tile that reaches past the sequence end
  // takes the per-row path.
  constexpr int kLatOps = FP8 ? 4 : 8;
  auto copy_op = [&](const Lanes& ln, const TileSrc& ts, int op) __attribute__((always_inline)) {
    const lds_char* const dst = smem + ts.lds;
    if (op < kLatOps) {
      const int g = FP8 ? 0 : op >> 2, j = op & 3;
      const int t0 = FP8 ? 8 * w : 4 * w + 16 * g;      // first row of the group
      constexpr int kStep = 1024 / kLatRow;              // rows per copy
      if (ts.full) {
        const char* const gb = ts.cp + (size_t)(ts.sb + t0) * kLatRow;
        const lds_char* const lb = dst + t0 * kLatRow;
        if (j == 0) dma_copy16_off<0>(gb, ln.cv[0], lb);
        else if (j == 1) dma_copy16_off<1024>(gb, ln.cv[1], lb);
        else if (j == 2) dma_copy16_off<2048>(gb, ln.cv[2], lb);
        else dma_copy16_off<3072>(gb, ln.cv[3], lb);
      } else {
        const int t = t0 + kStep * j + (FP8 ? (ln.lane >> 5) : 0);
        const int r = min(ts.sb + t, ts.last);
        const uint32_t v = ((uint32_t)r << (FP8 ? 9 : 10)) + (ln.cv[j] & (FP8 ? 511u : ~0u));
        dma_copy16_m0(ts.cp, v, dst + (t0 + kStep * j) * kLatRow);
      }
    } else if (op == kLatOps) {
      if (ts.full) {
        dma_copy16_m0(ts.rp + (size_t)(ts.sb + 8 * w) * 128, ln.rope_v, dst + Gm::kRopeOff + w * 1024);
      } else {
        const int t = 8 * w + (ln.lane >> 3);
        dma_copy16_m0(ts.rp, ((uint32_t)min(ts.sb + t, ts.last) << 7) + (ln.rope_v & 127u),
                      dst + Gm::kRopeOff + w * 1024);
      }
    } else if constexpr (FP8) {
      dma_copy4_m0(ts.sp, (uint32_t)min(ts.sb + (ln.lane & 31), ts.last) * 4, dst + Gm::kScaleOff);
    }
  };
  // copies per wave and tile: bf16 8 latent + 1 rope; fp8 4 latent pairs
  // + 1 rope + the scales
  constexpr int kMyCopies = FP8 ? 6 : 9;
  constexpr int kOpsPerTile = kMyCopies;
  // every step copies NT tiles: when the split's tile count is odd (64 rows),
  // the last step's second tile lies in the same page past the sequence end;
  // its slots repeat the last token and the mask gives them weight 0
  // the copies of step s into the buffers of step sdst
  auto issue_step = [&](const Lanes& ln, int s, int sdst, int id) __attribute__((always_inline)) {
#pragma clang loop unroll(full)
    for (int t = 0; t < NT; ++t) {
      const TileSrc ts = tile_src(s * NT + t, id, sdst * NT + t);
#pragma clang loop unroll(full)
      for (int op = 0; op < kOpsPerTile; ++op) copy_op(ln, ts, op);
    }
  };
  // page id of step s (both tiles of a 64-row step share one page)
  auto step_id = [&](int s) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane(ids[(s * NT * kTile) / kPage]);
  };
  static_assert((LA - 1) * NT * kMyCopies <= 63, "vmcnt range");

  if (__syncthreads_or(bad)) {
    write_uniform<ROWS>(p, b, k, row0, __builtin_nanf(""));
    return;
  }
  // (the barrier above also published the page ids)
  const float sl = p.scale_log2;

  // Each row's reference maximum is fixed at the first tile in which the row
  // sees a token, so the latent aggregate in the MFMA accumulators is never
  // rescaled inside the loop. Should a later tile's maximum exceed the
  // reference by more than kJump (log2 units) -- or a row sum overflow -- the
  // unit runs a second pass over its tiles with every reference at the true
  // row maximum found by the first, where no probability exceeds 1.
  f32x16_t U[16];                            // U^T: dims 32 db + 8 (q / 4) + 4h + q % 4
  float m_r, l_r;                            // reference max (log2 units); lane's share of l
  float m_true = -INFINITY;                  // running true row maximum (log2 units)

  // One step: the wave's tile jt = NT s + th. The copies of step s + LA are
  // interleaved with the score MFMAs (the issue of a copy can wait on the
  // copy queue). LDS reads take immediate offsets from eight per-lane bases
  // per phase: a wave64 VALU instruction costs four cycles, so per-read
  // address arithmetic would cost more than the MFMAs it feeds.
  auto step_body = [&](int s, auto first_c) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_c)::value;
    const Lanes ln = lanes_now();
    const int t32 = ln.t32, h = ln.h;
    const int jt = s * NT + th;
    const int tl_off = (jt % NB) * kTileBytes;
    const lds_char* const tl = smem + tl_off;
    const int stok = tok0 + jt * kTile;
    // Every step issues the copies of step s + LA; in the last LA steps,
    // where no such step exists, they re-read the current page (an L2 hit)
    // into the buffers of step s - 1, which nothing reads again. So every
    // step has the same copy count and no copy needs a branch.
    const bool more = s + LA < n_steps;
    const int sc = more ? s + LA : s;
    const int cid = step_id(sc);
    TileSrc cts[NT];
#pragma clang loop unroll(full)
    for (int ct = 0; ct < NT; ++ct) cts[ct] = tile_src(sc * NT + ct, cid, (s + LA) * NT + ct);
    // copy slots: after MFMA f of the step (36 score MFMAs, then 32 of the
    // aggregation), op o of the step's copies follows MFMA 68 o / kOps
    auto copy_slot = [&](int f) __attribute__((always_inline)) {
      constexpr int kOps = NT * kOpsPerTile;
#pragma clang loop unroll(full)
      for (int o = 0; o < kOps; ++o)
        if (f == (68 * o) / kOps) copy_op(ln, cts[o / kOpsPerTile], o % kOpsPerTile);
    };
    // ---------------- scores S^T[token][row] --------------------------------
    // latent k-step ks reads chunk c = 2 ks + h (bf16) or 2 (ks / 2) + h (fp8,
    // two k-steps per read) of token t32's row, swizzled c ^ sw with sw < 16:
    // row base + 16 ((2 j + h) ^ sw) + 256 q for c / 2 = 8 q + j
    const int sw = ln.lat_sw;
    int sbase[8];
#pragma clang loop unroll(full)
    for (int j = 0; j < 8; ++j) sbase[j] = tl_off + t32 * kLatRow + 16 * ((2 * j + h) ^ sw);
    auto rope_frag = [&](int r) __attribute__((always_inline)) -> bf16x8_t {
      return lds_read_b128(tl + Gm::kRopeOff + t32 * 128 + (((2 * r + h) ^ ln.rope_sw) * 16));
    };
    f32x16_t S0, S1;
    if constexpr (!FP8) {
      auto frag = [&](int ks) __attribute__((always_inline)) -> bf16x8_t {
        if (ks >= 32) return rope_frag(ks - 32);
        return lds_read_b128(smem + sbase[ks & 7] + 256 * (ks >> 3));
      };
      constexpr int kRing = 7;
      bf16x8_t ring[kRing];
#pragma clang loop unroll(full)
      for (int f = 0; f < kRing; ++f) ring[f] = frag(f);
      __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
      for (int ks = 0; ks < 36; ++ks) {
        const bf16x8_t av = ring[ks % kRing];
        f32x16_t& acc = (ks & 1) ? S1 : S0;
        if (ks < 2) mfma_sc0(acc, av, qB[ks]);
        else mfma_sc(acc, av, qB[ks]);
        if (ks + kRing < 36) ring[ks % kRing] = frag(ks + kRing);
        copy_slot(ks);
        __builtin_amdgcn_sched_barrier(0);
      }
      score_fence(S0, S1);
      S0 += S1;
    } else {
      // one 16-byte read of codes per k-step pair pp, each half widened to
      // bf16 right before its MFMA; then the token scales, then the rope
      auto frag = [&](int pp) __attribute__((always_inline)) -> bf16x8_t {
        return lds_read_b128(smem + sbase[pp & 7] + 256 * (pp >> 3));
      };
      constexpr int kRing8 = 6;
      bf16x8_t ring[kRing8];
#pragma clang loop unroll(full)
      for (int f = 0; f < kRing8; ++f) ring[f] = frag(f);
      __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
      for (int pp = 0; pp < 16; ++pp) {
        const u32x4_t raw = __builtin_bit_cast(u32x4_t, ring[pp % kRing8]);
        if (pp + kRing8 < 16) ring[pp % kRing8] = frag(pp + kRing8);
#pragma clang loop unroll(full)
        for (int half = 0; half < 2; ++half) {
          const bf16x8_t av = fp8x8_to_bf16((i32x2_t){(int)raw[2 * half], (int)raw[2 * half + 1]});
          f32x16_t& acc = half ? S1 : S0;
          if (pp == 0) mfma_sc0_v(acc, av, qB[2 * pp + half]);
          else mfma_sc_v(acc, av, qB[2 * pp + half]);
          copy_slot(2 * pp + half);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8_t rf[4];
#pragma clang loop unroll(full)
      for (int r = 0; r < 4; ++r) rf[r] = rope_frag(r);
      score_fence(S0, S1);
      // z = scale_s (q_lat . code_s) + q_rope . k^R_s: scale the latent part,
      // then accumulate the rope k-steps on top of it
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j) {
        const f32x4_t sc = *(const MLA_LDS f32x4_t*)(tl + Gm::kScaleOff + (8 * j + 4 * h) * 4);
#pragma clang loop unroll(full)
        for (int i = 0; i < 4; ++i) {
          S0[4 * j + i] = (S0[4 * j + i] + S1[4 * j + i]) * sc[i];
          S1[4 * j + i] = 0.f;
        }
      }
      valu_fence(S0);
      valu_fence(S1);
#pragma clang loop unroll(full)
      for (int r = 0; r < 4; ++r) {
        f32x16_t& acc = (r & 1) ? S1 : S0;
        mfma_sc(acc, rf[r], qB[32 + r]);
        copy_slot(32 + r);
      }
      score_fence(S0, S1);
      S0 += S1;
    }
    // ---------------- probabilities of the lane's row ----------------------------
    // lane value q is token 8 (q / 4) + 4h + q % 4 of the tile; masked only on
    // tiles that reach past the group's earliest limit
    if (stok + kTile > lim_min) {
#pragma clang loop unroll(full)
      for (int q = 0; q < 16; ++q)
        if (stok + 8 * (q >> 2) + 4 * h + (q & 3) >= lim) S0[q] = -INFINITY;
    }
    // the row maximum over the tile (both lane halves), for the running true
    // maximum -- and in the unit's first step, for the reference itself
    auto tile_max = [&]() __attribute__((always_inline)) -> float {
      float mx = fmaxf(fmaxf(S0[0], S0[1]), S0[2]);
#pragma clang loop unroll(full)
      for (int q = 3; q < 15; q += 2) mx = fmaxf(fmaxf(mx, S0[q]), S0[q + 1]);
      mx = fmaxf(mx, S0[15]);
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      return fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * sl;
    };
    if constexpr (kFirst) {
      const float mt = tile_max();
      m_true = fmaxf(m_true, mt);
      if (m_r == -INFINITY) m_r = mt;   // first tile with a visible token (U = 0)
    }
    // After the unit's first step a row either has its reference or sees no
    // token of this split at all (its later tiles only lie further right).
    const float nbase = (m_r == -INFINITY) ? 0.f : -m_r;
    // B operands of the aggregation's two k-steps: k-step kk holds the lane's
    // values 8 kk..8 kk + 7, tokens 16 kk + {4h..4h+3, 8+4h..8+4h+3}; the row
    // sum adds the same bf16 probabilities (fp8: before the token scale)
    bf16x8_t P[2];
    float ls = 0.f;
    auto probs = [&](int kk) __attribute__((always_inline)) {
      float tsc[16];   // fp8: the token scales of values 8 kk .. 8 kk + 7
      if constexpr (FP8) {
#pragma clang loop unroll(full)
        for (int j = 2 * kk; j < 2 * kk + 2; ++j) {
          const f32x4_t sc = *(const MLA_LDS f32x4_t*)(tl + Gm::kScaleOff + (8 * j + 4 * h) * 4);
#pragma clang loop unroll(full)
          for (int i = 0; i < 4; ++i) tsc[4 * j + i] = sc[i];
        }
      }
      uint32_t pk[4];
#pragma clang loop unroll(full)
      for (int q2 = 0; q2 < 4; ++q2) {
        const int q = 8 * kk + 2 * q2;
        const float e0 = fast_exp2(fmaf(S0[q], sl, nbase));
        const float e1 = fast_exp2(fmaf(S0[q + 1], sl, nbase));
        const uint32_t pl = pack_bf16x2(e0, e1);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pl),
                                             (bf16x2_t){(__bf16)1.0f, (__bf16)1.0f}, ls, false);
        pk[q2] = FP8 ? pack_bf16x2(e0 * tsc[q], e1 * tsc[q + 1]) : pl;
      }
      P[kk] = __builtin_bit_cast(bf16x8_t, (u32x4_t){pk[0], pk[1], pk[2], pk[3]});
    };
    probs(0);
    if constexpr (kFirst) probs(1);
    // ---------------- aggregation U^T[dim][row] += C^T P^T -------------------
    // 32 A fragments (32 latent dims x 16 tokens, read transposed) through a
    // ring; the two k-steps of a dim block are 16 MFMAs apart.
    //  bf16: the 16-lane group G of half h reads dims 16 G + 4 (i & 3) of
    //  token rows 16 kk + 4h + i / 4 and 16 kk + 8 + 4h + i / 4 (swizzles
    //  4 (i / 4) + h and 4 (i / 4) + 2 + h); dim block db = 4 a + b sits at
    //  64 (b ^ (i / 4)) + 256 a in the row.
    //  fp8: lane i of group G reads 8 bytes of token tau(i / 2) at chunk
    //  (2 db + G) ^ fsw(tau), i.e. 16 ((2 b8 + G) ^ fsw) + 256 a8 for
    //  db = 8 a8 + b8; k-step kk adds 16 rows.
    const int i = ln.lane & 15, G = (ln.lane >> 4) & 1;
    int pbase[8];
    if constexpr (!FP8) {
      const int c_lo = 2 * G + ((i >> 1) & 1);
#pragma clang loop unroll(full)
      for (int bb = 0; bb < 4; ++bb) {
        const int off = tl_off + ln.tr_base + 64 * (bb ^ (i >> 2)) + 8 * (i & 1);
        pbase[bb] = off + 16 * (c_lo ^ h);
        pbase[4 + bb] = off + 8 * kLatRow + 16 * (c_lo ^ (h + 2));
      }
    } else {
      const int r = i >> 1;
      const int tau = r < 4 ? 4 * h + r : 8 + 4 * h + (r - 4);
      const int fs = fsw(tau);
#pragma clang loop unroll(full)
      for (int b8 = 0; b8 < 8; ++b8) pbase[b8] = tl_off + tau * 512 + 16 * ((2 * b8 + G) ^ fs) + 8 * (i & 1);
    }
    // fp8 ring entries stay as raw codes until their MFMA (half the registers)
    using RingT = std::conditional_t<FP8, i32x2_t, bf16x8_t>;
    auto pfrag = [&](int e2) __attribute__((always_inline)) -> RingT {
      const int kk = e2 >> 4, db = e2 & 15;
      if constexpr (!FP8) {
        const int imm = 16 * kk * kLatRow + 256 * (db >> 2);
        const bf16x4_t lo = lds_read_tr16(smem + pbase[db & 3] + imm);
        const bf16x4_t hi = lds_read_tr16(smem + pbase[4 + (db & 3)] + imm);
        return concat(lo, hi);
      } else {
        const int imm = 16 * kk * 512 + 256 * (db >> 3);
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2_t*)(smem + pbase[db & 7] + imm));
      }
    };
    constexpr int kRingB = FP8 ? 10 : 7;
    RingT ringb[kRingB];
    __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
    for (int e2 = 0; e2 < kRingB; ++e2) ringb[e2] = pfrag(e2);
    __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
    for (int e2 = 0; e2 < 32; ++e2) {
      bf16x8_t av;
      if constexpr (FP8) av = fp8x8_to_bf16(ringb[e2 % kRingB]);
      else av = ringb[e2 % kRingB];
      if (e2 + kRingB < 32) ringb[e2 % kRingB] = pfrag(e2 + kRingB);
      U[e2 & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, P[e2 >> 4], U[e2 & 15], 0, 0, 0);
      if constexpr (!kFirst) {
        // the second k-step's probabilities and the tile maximum run under
        // the first k-step's MFMAs
        if (e2 == 4) probs(1);
        if (e2 == 9) m_true = fmaxf(m_true, tile_max());
      }
      copy_slot(36 + e2);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_r += ls;
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma clang loop unroll(full)
    for (int db = 0; db < 16; ++db)
#pragma clang loop unroll(full)
      for (int q = 0; q < 16; ++q) U[db][q] = 0.f;
    m_r = pass == 0 ? -INFINITY : m_true;
    l_r = 0.f;
    {
      // steps 0 .. LA - 1; a step past the end re-reads step 0 (into a
      // buffer nothing reads), so the loop's copy count stays uniform
      const Lanes ln = lanes_now();
      issue_step(ln, 0, 0, step_id(0));
      vm_wait<0>();
      for (int s = 1; s < LA; ++s) {
        const int ss = s < n_steps ? s : 0;
        issue_step(ln, ss, s, step_id(ss));
      }
    }
    lds_barrier();   // step 0 resident
    // after each step: this wave's copies of step s + 1 have landed (those of
    // the LA - 1 later steps may still fly); step s + 1 is resident and step
    // s's buffers are free after the barrier
    step_body(0, std::true_type{});
    vm_wait<(LA - 1) * NT * kMyCopies>();
    lds_barrier();
    for (int s = 1; s < n_steps; ++s) {
      step_body(s, std::false_type{});
      vm_wait<(LA - 1) * NT * kMyCopies>();
      lds_barrier();
    }
    vm_wait<0>();   // the tail's re-read copies land before LDS is reused
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
  int db_lo = 0, db_hi = 16;                 // dim blocks this wave writes
  if constexpr (NT == 2) {
    // merge the two tile parities: (m, l) of all rows, and each wave hands its
    // partner the U half that the partner finishes (th = 0: dims 0-255)
    float* const mls = (float*)(smem_raw + Gm::kOffMl);   // [th][m|l][64 rows]
    const int rr = 32 * rbw + (lane & 31);
    if (lane < 32) {
      mls[(th * 2 + 0) * 64 + rr] = m_r;
      mls[(th * 2 + 1) * 64 + rr] = l_row;
    }
    lds_char* const mine = smem + w * 32 * 1024;
    const int give = th == 0 ? 8 : 0;                       // dim blocks handed over
#pragma clang loop unroll(full)
    for (int d = 0; d < 8; ++d)
#pragma clang loop unroll(full)
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t v = {U[give + d][4 * q4], U[give + d][4 * q4 + 1], U[give + d][4 * q4 + 2],
                           U[give + d][4 * q4 + 3]};
        *(MLA_LDS f32x4_t*)(mine + ((d * 4 + q4) * 64 + lane) * 16) = v;
      }
    lds_barrier();
    const int partner = w ^ NRB;                            // same rows, other parity
    const lds_char* const theirs = smem + partner * 32 * 1024;
    db_lo = th == 0 ? 0 : 8;
    db_hi = db_lo + 8;
    const float mo = mls[((th ^ 1) * 2 + 0) * 64 + rr];
    const float lo = mls[((th ^ 1) * 2 + 1) * 64 + rr];
    const float mm = fmaxf(m_r, mo);
    const float a_me = (m_r == -INFINITY) ? 0.f : fast_exp2(m_r - mm);
    const float a_ot = (mo == -INFINITY) ? 0.f : fast_exp2(mo - mm);
    l_row = a_me * l_row + a_ot * lo;
    m_r = mm;
#pragma clang loop unroll(full)
    for (int d = 0; d < 8; ++d)
#pragma clang loop unroll(full)
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t v = *(const MLA_LDS f32x4_t*)(theirs + ((d * 4 + q4) * 64 + lane) * 16);
        const int db = db_lo + d;
#pragma clang loop unroll(full)
        for (int i = 0; i < 4; ++i) U[db][4 * q4 + i] = a_me * U[db][4 * q4 + i] + a_ot * v[i];
      }
  }
  const bool direct = p.n_split == 1;
  const size_t row_base = direct ? (size_t)b * p.R : ((size_t)b * p.n_split + k) * p.R;
  const bool out16 = direct ? p.out_bf16 != 0 : p.part_bf16 != 0;
  const bool normalise = direct || out16;   // fp32 partials keep U unnormalised
  if (my_row < p.R) {
    const float inv = normalise ? (l_row > 0.f ? 1.f / l_row : 0.f) : 1.f;
    void* const dst = direct ? p.out : p.part_u;
#pragma clang loop unroll(full)
    for (int db = 0; db < 16; ++db) {
      if (db < db_lo || db >= db_hi) continue;
#pragma clang loop unroll(full)
      for (int j = 0; j < 4; ++j) {
        const size_t o = (row_base + my_row) * kDc + 32 * db + 8 * j + 4 * hq;
        const f32x4_t v = (f32x4_t){U[db][4 * j], U[db][4 * j + 1], U[db][4 * j + 2], U[db][4 * j + 3]} * inv;
        if (out16) {
          *(u32x2_t*)((uint16_t*)dst + o) = (u32x2_t){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
          *(f32x4_t*)((float*)dst + o) = v;
        }
      }
    }
    if (lane < 32 && th == 0) {
      if (direct) {
        if (p.lse) p.lse[(size_t)b * p.R + my_row] = (m_r + log2f(l_row)) * kLn2;
      } else {
        p.part_ml[(row_base + my_row) * 2] = m_r;
        p.part_ml[(row_base + my_row) * 2 + 1] = l_row;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_split(const DecodeParams& p, int fp8, int rows, hipStream_t s) {
  const dim3 grid(p.per_xcd * kNumXcd), block(kThreads);
  if (!fp8 && rows == 64) hipLaunchKernelGGL((decode_split_kernel<false, 64>), grid, block, 0, s, p);
  else if (!fp8) hipLaunchKernelGGL((decode_split_kernel<false, 128>), grid, block, 0, s, p);
  else if (rows == 64) hipLaunchKernelGGL((decode_split_kernel<true, 64>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((decode_split_kernel<true, 128>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
