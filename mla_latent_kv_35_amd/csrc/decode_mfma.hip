// Paged absorbed-MLA decode on gfx950 MFMA, for bf16 caches and for fp8
// (OCP E4M3FN) latent caches with one fp32 scale per token.
//
// One workgroup owns a work unit (sequence b, split k, group g of 64 query
// rows) and streams the split's cache through LDS in tiles of 32 tokens
// (half a page): 512 latent + 64 rope elements per token, the 576-element
// cache of PaperTrace "02 · DeepSeek-V2 analysis", section 1.3.
//
// The workgroup's 8 waves form two teams that work one tile apart, so that on
// every SIMD one wave's softmax and LDS traffic overlap the other wave's MFMAs:
//
//  * score team (waves 0-3): wave (hh, th) holds the absorbed queries of rows
//    32*hh..+31 in registers and, for tile j, computes the scores of its 16
//    tokens S^T[token][row] = K[token][576] . Q^T[576][row] on MFMA 16x16x32,
//    exchanges per-row tile maxima with its partner wave through LDS, and
//    writes bf16 probabilities p = 2^(z - m) (log2 units, scale folded in,
//    section 1.3 eq. 18) and the rows' rescale factors to LDS;
//  * aggregation team (waves 4-7): wave v owns latent dims 128*v..+127 of all
//    64 rows and, during step j, accumulates U[row][d] += P[row][token]
//    C[token][d] for tile j-1 on MFMA, reading the latent tile transposed
//    (ds_read_b64_tr_b16) -- each head aggregates latents with its own weights
//    (section 6.1). Between its MFMA groups it issues the asynchronous copies
//    of tile j+2.
//
// Per step one workgroup barrier, X (tile j resident, P(j-1) published).
// The two score waves that split a row group's tokens exchange their tile
// maxima through LDS: each writes its maxima, then a flag holding the step
// number, and waits (bounded) for its partner's flag only, so neither the
// other pair nor the aggregation team is held up. Four tile buffers keep two
// tiles in flight while two are in use. All barriers order LDS only; the page copies are
// waited for explicitly with vmcnt by the waves that issued them. Before
// step 0 the absorbed queries pass through LDS once: each score wave loads
// half of its rows' fragments and takes the other half from its partner
// wave, while the first two tiles are already being copied.
//
// fp8 latent caches: tiles stay fp8 in LDS (half the bytes of bf16); every
// E4M3FN code is widened exactly to bf16 in registers right before its MFMA,
// so the cache's own rounding is the only quantization on the path (the
// absorbed query stays bf16: quantizing it to fp8 per row would add an error
// of about 5 % of the output on these workloads). The token scale multiplies
// the latent score in fp32, z = scale_s * (q_lat . code_s) + q_rope . k^R_s,
// and is folded into the probability for the aggregation, P' = p * scale_s,
// which reads the codes transposed (ds_read_b64_tr_b8).
//
// The split ends by writing either u = U / l and lse, or partials (m, l and
// U in fp32, or u = U / l in bf16 when the output is bf16) for the
// log-sum-exp combine kernel; bf16 rows leave through LDS in 1-KB stores.
#include "dma.h"
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 512;
constexpr int kTileTok = 32;
constexpr int kRopeTile = kTileTok * 128;           // 4096: rope rows of 128 B (bf16)
constexpr int kNumBuf = 4;
constexpr int kPStride = 64;                        // bytes per probability row (32 bf16)
constexpr int kPBytes = kRowsPerGroup * kPStride;   // 4096

// LDS tile geometry: latent rows of 1 KB (bf16) or 512 B (fp8), then the rope
// rows, then (fp8) the tile's 32 token scales in a 256-B slot.
template <bool FP8>
struct Geo {
  static constexpr int kLatRow = FP8 ? 512 : 1024;
  static constexpr int kLatTile = kTileTok * kLatRow;
  static constexpr int kScaleOff = kLatTile + kRopeTile;
  static constexpr int kTileBytes = kLatTile + kRopeTile + (FP8 ? 256 : 0);
  static constexpr int kOffP = kNumBuf * kTileBytes;        // P[2]
  static constexpr int kOffAlpha = kOffP + 2 * kPBytes;     // alpha[2][64] f32
  static constexpr int kOffRed = kOffAlpha + 2 * 64 * 4;    // tile maxima [2][64] f32
  static constexpr int kOffLsum = kOffRed + 2 * 64 * 4;     // row sums [2][64] f32
  static constexpr int kOffM = kOffLsum + 2 * 64 * 4;       // final reference max [64] f32
  // before step 0 the absorbed queries pass through LDS once per workgroup
  // (72 KB from tile buffer 2 on; bf16: buffers 2-3, fp8: also the P and
  // per-row arrays, all first written after the first step's barrier)
  static constexpr int kOffStage = 2 * kTileBytes;
  static constexpr int kStageBytes = 2 * 2 * 18 * 1024;
  static constexpr int kOffIds = (kOffM + 64 * 4 > kOffStage + kStageBytes) ? kOffM + 64 * 4
                                                                            : kOffStage + kStageBytes;
  static constexpr int kOffFlags = kOffIds + kMaxSplitPages * 4;   // per score wave: last step synced
  static constexpr int kLdsBytes = kOffFlags + 4 * 4;
  // page copies per tile per aggregation wave: bf16 8 latent rows + 1 rope
  // block; fp8 4 latent row pairs + 1 rope block (+ the scales on wave 0)
  static constexpr int kDma = FP8 ? 5 : 9;
  static_assert(kLdsBytes <= 163840, "LDS budget");
};

// The running reference max of a row only moves when a tile's max exceeds it
// by more than kLazyMax (log2 units): probabilities are then bounded by
// 2^kLazyMax, which fp32 sums and bf16 probabilities hold exactly as well,
// and the accumulator rescale runs on the first tile and on rare jumps only.
// u, l and lse do not depend on the reference.
constexpr float kLazyMax = 8.0f;

// LDS bank rules of gfx950 that the layouts below are built for (measured
// with the SQ_LDS_BANK_CONFLICT counter): ds_read_b64 and ds_read_b64_tr_*
// serve lanes 0-31 and 32-63 in one pass each over 64 banks (256 B);
// ds_read_b128 serves four passes of 16 lanes, lanes 0-31 and 32-63 apart and,
// within each half, the 4-lane quads q = lane/4 split by the parity of q's
// bits; ds_write_b64 / _b128 serve 16 / 8 consecutive lanes per pass over 32
// banks (128 B).
//
// Latent rows: 16-B chunk j of token t lives at chunk j ^ swz_lat(t & 15),
// swz_lat(s) = s3 s1 s0 0 (binary). The score team's ds_read_b128 (16 tokens
// x one chunk per k-step, tokens t and t^4 in different passes) and the
// transposed reads (4 consecutive tokens x 2 adjacent chunks per 16-lane
// group, groups 8 tokens apart, 32 lanes per pass) then touch 64 distinct
// banks per pass.
__device__ __forceinline__ int swz_lat(int s) {
  return (s & 8) | ((s & 3) << 1);
}
// Probability rows (64 B = 8 units of 8 B): unit u of row r lives at
// u ^ swz_p(r & 15), swz_p(r) = r3 r1 r2 (binary). The score team writes one
// unit per lane (16 rows per pass: 8 distinct units per row parity) and the
// aggregation team reads units 2g and 2g+1 (32 lanes per pass: rows r, r+4,
// r+8, r+12 fall in distinct unit pairs).
__device__ __forceinline__ int swz_p(int r) {
  return ((r >> 2) & 1) | (r & 2) | (((r >> 3) & 1) << 2);
}
// Rope rows (128 B): chunk j (0..7) of token t lives at chunk j ^ ((t>>1)&7).
__device__ __forceinline__ int swz_rope(int t) { return (t >> 1) & 7; }

// The split's u = U / l leaves as bf16 through an LDS staging area (the
// direct bf16 output, and bf16 partials), else as fp32 from registers.
__device__ __forceinline__ bool stage_u(const DecodeParams& p) {
  return p.n_split == 1 ? p.out_bf16 != 0 : p.part_bf16 != 0;
}
constexpr int kStagePitch = 1024 + 16;   // bf16 row of 512 + 16 B (rows 4 banks apart)

// 8 E4M3FN bytes -> 8 bf16 (exact: every E4M3FN value is a bf16 value).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(const i32x2_t& v) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
  const bf2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
  const bf2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
  const bf2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
  return (bf16x8_t){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ void write_uniform_result(const DecodeParams& p, int b, int k, int g, float v) {
  // Every row of the unit gets (m, l, U) = (v, v, v); marks out-of-range
  // sequences with NaN.
  const int tid = threadIdx.x;
  const int r0 = g * kRowsPerGroup;
  const int nrows = min(kRowsPerGroup, p.R - r0);
  for (int e = tid; e < nrows * kDc; e += kThreads) {
    const int r = r0 + e / kDc, d = e % kDc;
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
  for (int r = r0 + tid; r < r0 + nrows; r += kThreads) {
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
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mfma_kernel(DecodeParams p) {
  using Gm = Geo<FP8>;
  constexpr int kLatRow = Gm::kLatRow;
  constexpr int kLatTile = Gm::kLatTile;
  constexpr int kTileBytes = Gm::kTileBytes;
  constexpr int kOffP = Gm::kOffP, kOffAlpha = Gm::kOffAlpha, kOffRed = Gm::kOffRed;
  constexpr int kOffLsum = Gm::kOffLsum, kOffM = Gm::kOffM, kOffIds = Gm::kOffIds;
  __shared__ __attribute__((aligned(16))) char smem_raw[Gm::kLdsBytes];
  lds_char* const smem = (lds_char*)smem_raw;

  const int bid = blockIdx.x;
  const int unit = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (unit >= p.n_units) return;
  const int g = unit % p.G;
  const int bk = unit / p.G;
  const int k = bk % p.n_split;
  const int b = bk / p.n_split;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int i16 = lane & 15;
  const int G4 = lane >> 4;

  const int row0 = g * kRowsPerGroup;
  const int L = p.seq_lens[b];
  const int tok0 = k * p.split_tokens;
  const int tok1 = min(tok0 + p.split_tokens, L);
  const int pg_begin = tok0 / kPage;
  const int pg_end = (tok1 + kPage - 1) / kPage;
  const int n_tiles = (tok1 - tok0 + kTileTok - 1) / kTileTok;
  // sequence-level range checks; page ids are checked by the aggregation team
  bool expired = false;                      // a partner wait gave up (see the step loop)
  const bool seq_bad = (L < p.T) || (L > p.max_seq_len) ||
                       ((L + kPage - 1) / kPage > p.max_pages) ||
                       (pg_end - pg_begin) > kMaxSplitPages;
  int* const ids = (int*)(smem_raw + kOffIds);
  lds_char* const pbuf = smem + kOffP;
  float* const alphabuf = (float*)(smem_raw + kOffAlpha);   // [2][64]
  float* const redmax = (float*)(smem_raw + kOffRed);       // [2][64]
  float* const lsum = (float*)(smem_raw + kOffLsum);        // [2][64]
  float* const mbuf = (float*)(smem_raw + kOffM);           // [64]
  MLA_LDS int* const flags = (MLA_LDS int*)(smem + Gm::kOffFlags);
  const char* const ckv_base = (const char*)p.ckv;
  const char* const kr_base = (const char*)p.kr;

  // The two teams take fully separate code paths; both meet in the same
  // sequence of workgroup barriers.
  if (w < 4) {
    // ======================= score team ======================================
    const int hh = w & 1;    // rows 32*hh..+31
    const int th = w >> 1;   // tokens 16*th..+15 of each tile
    // Absorbed queries of the wave's 32 rows as MFMA B fragments: 16 latent
    // k-steps + 2 rope k-steps per 16-row half. The two waves of a row half
    // (th = 0, 1) each load 9 of the 18 k-steps from global memory (issued
    // before the block-table check, which they do not depend on), stage them
    // in LDS and take the partner's 9 from there, so the workgroup reads its
    // queries from memory once.
    bf16x8_t qB[2][18];
    lds_char* const stage = smem + Gm::kOffStage;
    auto stage_at = [&](int ht, int ks) __attribute__((always_inline)) -> lds_char* {
      return stage + (((hh * 2 + ht) * 18 + ks) * 64 + lane) * 16;
    };
    auto q_half = [&](auto half_c, bool from_lds) __attribute__((always_inline)) {
      constexpr int k0 = 9 * decltype(half_c)::value;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const int r = row0 + 32 * hh + 16 * ht + i16;
        const size_t qrow = (size_t)b * p.R + r;
        const uint16_t* ql = (const uint16_t*)p.q_lat + qrow * p.q_lat_stride + 8 * G4;
        const uint16_t* qr = (const uint16_t*)p.q_rope + qrow * p.q_rope_stride + 8 * G4;
#pragma unroll
        for (int kk = 0; kk < 9; ++kk) {
          const int ks = k0 + kk;
          if (from_lds) qB[ht][ks] = lds_read_b128(stage_at(ht, ks));
          else if (r >= p.R) qB[ht][ks] = (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
          else qB[ht][ks] = load_bf16x8(ks < 16 ? ql + 32 * ks : qr + 32 * (ks - 16));
        }
      }
    };
    auto q_stage = [&](auto half_c) __attribute__((always_inline)) {
      constexpr int k0 = 9 * decltype(half_c)::value;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int kk = 0; kk < 9; ++kk)
          *(MLA_LDS bf16x8_t*)stage_at(ht, k0 + kk) = qB[ht][k0 + kk];
    };
    if (th == 0) q_half(std::integral_constant<int, 0>{}, false);
    else q_half(std::integral_constant<int, 1>{}, false);
    if (seq_bad || __syncthreads_or(false)) {
      write_uniform_result(p, b, k, g, __builtin_nanf(""));
      return;
    }
    if (tok0 >= tok1) return;   // split past the end of the sequence: no partial
    if (th == 0) q_stage(std::integral_constant<int, 0>{});
    else q_stage(std::integral_constant<int, 1>{});
    if (lane == 0) flags[w] = -1;
    lds_barrier();  // (Q) both halves staged
    if (th == 0) q_half(std::integral_constant<int, 1>{}, true);
    else q_half(std::integral_constant<int, 0>{}, true);
    // visible-token limit of a row: s < min(L - T + t + 1, tok1)
    auto row_limit = [&](int rr) __attribute__((always_inline)) -> int {
      const int r = row0 + rr;
      const int t = (r < p.R) ? r / p.H : 0;
      return min(L - p.T + t + 1, tok1);
    };
    const int lim_min = row_limit(0);   // the group's first (earliest) query token
    int lim_s[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) lim_s[ht] = row_limit(32 * hh + 16 * ht + i16);
    const int fl = swz_lat(i16);     // token & 15 == i16 for this lane's A rows
    const int fr = i16 >> 1;         // rope swizzle of this lane's A rows
    float m_s[2] = {-INFINITY, -INFINITY};
    float l_s[2] = {0.f, 0.f};

    // one step: scores of tile j, then the softmax of tile j; compiled with
    // and without the causal / ragged-end mask, which only the tiles that
    // reach past the group's first row limit need
    auto step = [&](int j, auto masked_c) __attribute__((always_inline)) {
      constexpr bool kMasked = decltype(masked_c)::value;
      lds_barrier();  // (X) tile j resident
      f32x4_t S[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      const int stok0 = tok0 + j * kTileTok;   // first token of tile j
      f32x4_t tsc = {1.f, 1.f, 1.f, 1.f};       // fp8: scales of this lane's 4 tokens
      if (j < n_tiles) {
        lds_char* const tile = smem + (j % kNumBuf) * kTileBytes;
        const lds_char* const rope0 = tile + kLatTile + (16 * th + i16) * 128;
        auto rfrag = [&](int ks) __attribute__((always_inline)) -> bf16x8_t {
          return lds_read_b128(rope0 + ((4 * ks + G4) ^ fr) * 16);
        };
        if constexpr (!FP8) {
          const lds_char* const lat0 = tile + (16 * th + i16) * 1024;
          auto frag = [&](int ks) __attribute__((always_inline)) -> bf16x8_t {
            if (ks < 16)
              return lds_read_b128(lat0 + (16 * (ks >> 2) + ((4 * (ks & 3) + G4) ^ fl)) * 16);
            return rfrag(ks - 16);
          };
          constexpr int kRing = 6;
          bf16x8_t ring[kRing];
#pragma unroll
          for (int f = 0; f < kRing; ++f) ring[f] = frag(f);
          __builtin_amdgcn_sched_group_barrier(0x100, kRing, 0);
#pragma unroll
          for (int f = 0; f < 18; ++f) {
            const bf16x8_t a = ring[f % kRing];
            if (f + kRing < 18) ring[f % kRing] = frag(f + kRing);
            S[0] = mfma16x16x32(a, qB[0][f], S[0]);
            S[1] = mfma16x16x32(a, qB[1][f], S[1]);
            if (f + kRing < 18) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
        } else {
          // latent codes: 8 bytes per lane at 8-byte chunk (4*ks + G4) ^ (2*i16)
          // of token row 16*th + i16, widened to bf16 before the MFMA
          const lds_char* const lat0 = tile + (16 * th + i16) * 512;
          auto frag8 = [&](int ks) __attribute__((always_inline)) -> i32x2_t {
            return *(const MLA_LDS i32x2_t*)(lat0 + (((4 * ks + G4) ^ (2 * i16)) * 8));
          };
          constexpr int kRing = 6;
          i32x2_t ring[kRing];
#pragma unroll
          for (int f = 0; f < kRing; ++f) ring[f] = frag8(f);
          const bf16x8_t r0 = rfrag(0), r1 = rfrag(1);
          __builtin_amdgcn_sched_group_barrier(0x100, kRing + 2, 0);
          f32x4_t Sl[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int f = 0; f < 16; ++f) {
            const bf16x8_t a = fp8x8_to_bf16(ring[f % kRing]);
            if (f + kRing < 16) ring[f % kRing] = frag8(f + kRing);
            Sl[0] = mfma16x16x32(a, qB[0][f], Sl[0]);
            Sl[1] = mfma16x16x32(a, qB[1][f], Sl[1]);
            if (f + kRing < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) {
            S[ht] = mfma16x16x32(r0, qB[ht][16], S[ht]);
            S[ht] = mfma16x16x32(r1, qB[ht][17], S[ht]);
          }
          // token scales of this lane's 4 tokens on the latent part
          tsc = *(const MLA_LDS f32x4_t*)(tile + Gm::kScaleOff + (16 * th + 4 * G4) * 4);
#pragma unroll
          for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ht][i] = fmaf(Sl[ht][i], tsc[i], S[ht][i]);
        }
        // mask, tile maxima of this wave's rows; the scores stay unscaled
        // and the scale (> 0, so it commutes with max) is applied to the
        // maxima here and inside the exponent below
        float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (kMasked)
              if (stok0 + 16 * th + 4 * G4 + i >= lim_s[ht]) S[ht][i] = -INFINITY;
            mx[ht] = fmaxf(mx[ht], S[ht][i]);
          }
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          mx[ht] = wave_max16(mx[ht]) * p.scale_log2;
          if (lane < 16) redmax[th * 64 + 32 * hh + 16 * ht + lane] = mx[ht];
        }
      }
      if (j < n_tiles) {
        // the partner wave (other token half, same rows) instead of a
        // workgroup barrier: this wave's maxima are in LDS before its flag
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        if (lane == 0) *(volatile MLA_LDS int*)(flags + w) = j;
        // bounded: a wait that gives up marks the unit, whose outputs then
        // become NaN (a limit of 0 gives up at once)
        bool arrived = false;
        for (int it = 0; it < p.spin_limit; ++it) {
          if (__builtin_amdgcn_readfirstlane(*(volatile MLA_LDS int*)(flags + (w ^ 2))) == j) {
            arrived = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        expired |= !arrived;
        asm volatile("" ::: "memory");
      }
      if (j < n_tiles) {
        lds_char* const pj = pbuf + (j & 1) * kPBytes;
        float* const aj = alphabuf + (j & 1) * 64;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const int rr = 32 * hh + 16 * ht + i16;
          const float mt = fmaxf(redmax[rr], redmax[64 + rr]);
          const float mold = m_s[ht];
          const float mnew = (mt - mold > kLazyMax) ? mt : mold;   // -inf - -inf is NaN: keep
          const float base = (mnew == -INFINITY) ? 0.f : mnew;
          const float alpha = (mnew == mold) ? 1.f : fast_exp2(mold - mnew);
          m_s[ht] = mnew;
          if (th == 0 && lane < 16) aj[rr] = alpha;
          const float nb = -base, sc = p.scale_log2;
          const float e0 = fast_exp2(fmaf(S[ht][0], sc, nb)), e1 = fast_exp2(fmaf(S[ht][1], sc, nb));
          const float e2 = fast_exp2(fmaf(S[ht][2], sc, nb)), e3 = fast_exp2(fmaf(S[ht][3], sc, nb));
          uint32_t lo, hi;
          float ls;
          if constexpr (!FP8) {
            lo = pack_bf16x2(e0, e1);
            hi = pack_bf16x2(e2, e3);
            ls = bf2f(lo & 0xffff) + bf2f(lo >> 16) + bf2f(hi & 0xffff) + bf2f(hi >> 16);
          } else {
            lo = pack_bf16x2(e0 * tsc[0], e1 * tsc[1]);
            hi = pack_bf16x2(e2 * tsc[2], e3 * tsc[3]);
            ls = (e0 + e1) + (e2 + e3);
          }
          *(MLA_LDS u32x2_t*)(pj + rr * kPStride + 8 * ((4 * th + G4) ^ swz_p(i16))) = (u32x2_t){lo, hi};
          l_s[ht] = l_s[ht] * alpha + wave_sum16(ls);
        }
      }
    };
    for (int j = 0; j <= n_tiles; ++j) {
      if (tok0 + j * kTileTok + kTileTok > lim_min) step(j, std::true_type{});
      else step(j, std::false_type{});
    }
    if (lane < 16) {
      lsum[th * 64 + 32 * hh + lane] = l_s[0];
      lsum[th * 64 + 32 * hh + 16 + lane] = l_s[1];
      if (th == 0) {
        mbuf[32 * hh + lane] = m_s[0];
        mbuf[32 * hh + 16 + lane] = m_s[1];
      }
    }
    // (Z) row sums and reference maxima published; a partner wait that gave
    // up anywhere in the workgroup turns the unit's outputs into NaN
    if (__syncthreads_or(expired)) {
      write_uniform_result(p, b, k, g, __builtin_nanf(""));
      return;
    }
    if (stage_u(p)) lds_barrier();   // (W) the aggregation team's u staged
    return;
  }

  // ========================= aggregation team ===============================
  {
    bool local_bad = false;
    if (!seq_bad) {
      const int32_t* btrow = p.block_table + (size_t)b * p.max_pages;
      for (int j = pg_begin + (tid - 256); j < pg_end; j += 256) {
        const int id = btrow[j];
        local_bad |= (id < 0) || (id >= p.n_pages);
        ids[j - pg_begin] = id;
      }
    }
    if (seq_bad || __syncthreads_or(local_bad)) {
      write_uniform_result(p, b, k, g, __builtin_nanf(""));
      return;
    }
  }
  if (tok0 >= tok1) return;   // split past the end of the sequence: no partial
  const int v = w - 4;           // latent dims 128*v..+127
  // copy duties per tile: bf16 latent rows t = 4*op + v (op = 0..7); fp8
  // latent row pairs (2q, 2q+1) with q = 4*op + v (op = 0..3); then rope
  // block v; fp8 wave 0 also copies the 32 token scales.
  const int n_ops = FP8 ? (v == 0 ? 6 : 5) : 9;
  uint32_t lat_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) lat_off[q] = (uint32_t)(lane ^ swz_lat((4 * q + v) & 15)) * 16u;
  // source of tile jt: its LDS buffer, page pointers and the last valid slot
  struct TileSrc {
    lds_char* tile;
    const char* cp;
    const char* rp;
    const char* sp;
    int base_t, last;
  };
  auto tile_src = [&](int jt) __attribute__((always_inline)) -> TileSrc {
    const int t0 = tok0 + jt * kTileTok;            // first token of the tile
    const int id = __builtin_amdgcn_readfirstlane(ids[(t0 - tok0) / kPage]);
    const int base_t = t0 % kPage;                  // 0 or 32 within the page
    return TileSrc{smem + (jt % kNumBuf) * kTileBytes,
                   ckv_base + (size_t)id * (kPage * kLatRow),
                   kr_base + (size_t)id * (kPage * kDr * 2),
                   FP8 ? (const char*)p.ckv_scale + (size_t)id * (kPage * 4) : nullptr, base_t,
                   L - 1 - (t0 - base_t)};          // last valid token's page slot
  };
  auto dma_op = [&](const TileSrc& src, int op) __attribute__((always_inline)) {
    if (op < (FP8 ? 4 : 8)) {
      if constexpr (!FP8) {
        const int t = 4 * op + v;
        const int ts = min(src.base_t + t, src.last);
        dma_copy16(src.cp, (uint32_t)(ts * 1024) + lat_off[op & 3], src.tile + t * 1024);
      } else {
        const int q = 4 * op + v;                   // rows 2q (lanes 0-31), 2q+1 (32-63)
        const int t = 2 * q + (lane >> 5);
        const int ts = min(src.base_t + t, src.last);
        const int jc = (lane & 31) ^ (t & 15);      // 16-B chunk of the 512-B row
        dma_copy16(src.cp, (uint32_t)(ts * 512 + jc * 16), src.tile + 2 * q * 512);
      }
    } else if (op == (FP8 ? 4 : 8)) {
      const int t = 8 * v + (lane >> 3);
      const int ts = min(src.base_t + t, src.last);
      const int jc = (lane & 7) ^ swz_rope(t);
      dma_copy16(src.rp, (uint32_t)(ts * 128 + jc * 16), src.tile + kLatTile + v * 1024);
    } else if constexpr (FP8) {
      const int ts = min(src.base_t + (lane & 31), src.last);
      dma_copy4(src.sp, (uint32_t)(ts * 4), src.tile + Gm::kScaleOff);
    }
  };
  auto issue_tile = [&](int jt) __attribute__((always_inline)) {
    const TileSrc src = tile_src(jt);
#pragma unroll
    for (int op = 0; op < 9; ++op)
      if (op < n_ops) dma_op(src, op);
  };
  // this wave's copies of one tile must have landed: at most `pending` of the
  // next tile's copies may still be in flight
  auto wait_tile = [&](bool pending) __attribute__((always_inline)) {
    if (!pending) dma_wait<0>();
    else if (!FP8) dma_wait<9>();
    else if (v == 0) dma_wait<6>();
    else dma_wait<5>();
  };

  f32x4_t U[4][8];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) U[rt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int xq32 = 32 * (4 * (G4 & 1) + (i16 >> 2));
  const int c0 = (i16 & 3) >> 1;

  issue_tile(0);
  if (n_tiles > 1) issue_tile(1);
  lds_barrier();  // (Q) the score team's queries staged; the copies fly on
  wait_tile(n_tiles > 1);

  bf16x8_t pa[4];
  // half 0 issues copy ops 0..4 of the next-but-one tile between its MFMA
  // groups, half 1 ops 5..8 (when `more`)
  auto pv_half = [&](const lds_char* tile, int half, bool more, const TileSrc& src) __attribute__((always_inline)) {
    auto bfrag = [&](int dt) __attribute__((always_inline)) -> bf16x8_t {
      if constexpr (!FP8) {
        const lds_char* const rowA = tile + (8 * G4 + (i16 >> 2)) * 1024 + 256 * v + (i16 & 1) * 8;
        const int dx = (32 * dt) ^ xq32;              // 32 * (dt ^ xq)
        const bf16x4_t lo = lds_read_tr16(rowA + dx + 16 * c0);                  // tokens +0..3
        const bf16x4_t hi = lds_read_tr16(rowA + 4 * 1024 + dx + 16 * c0);     // tokens +4..7
        return concat(lo, hi);
      } else {
        // lane 2r+h of each 16-lane group reads 8 bytes of token 8*G4 + r at
        // latent byte 128*v + 16*dt + 8*h; the transposed read hands lane i
        // the 8 tokens of column 128*v + 16*dt + i
        const int r = i16 >> 1, h = i16 & 1;
        const int ph8 = h + 2 * (dt ^ r) + 16 * (v ^ (G4 & 1));
        const lds_char* const a = tile + (8 * G4 + r) * 512 + ph8 * 8;
        return fp8x8_to_bf16(__builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2_t*)a));
      }
    };
    constexpr int kRingB = 2;
    bf16x8_t ringb[kRingB];
#pragma unroll
    for (int e = 0; e < kRingB; ++e) ringb[e] = bfrag(4 * half + e);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kRingB, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dt = 4 * half + e;
      const bf16x8_t bv = ringb[e % kRingB];
      if (e + kRingB < 4) ringb[e % kRingB] = bfrag(dt + kRingB);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) U[rt][dt] = mfma16x16x32(pa[rt], bv, U[rt][dt]);
      if (e + kRingB < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (more) {
        if constexpr (!FP8) {
          // 9 copies: 2 + 1 + 1 + 1 in the first half, 1 + 1 + 2 in the second
          if (half == 0) {
            dma_op(src, e == 0 ? 0 : e + 1);
            if (e == 0) dma_op(src, 1);
          } else if (e < 3) {
            dma_op(src, 5 + e);
            if (e == 2) dma_op(src, 8);
          }
        } else if (half == 0 && e < 3) {
          // 5 or 6 copies, two per MFMA group
          dma_op(src, 2 * e);
          if (2 * e + 1 < n_ops) dma_op(src, 2 * e + 1);
        }
      }
    }
  };

  for (int j = 0; j <= n_tiles; ++j) {
    lds_barrier();  // (X) tile j resident; P(j-1) and alpha(j-1) published
    const bool more = j + 2 < n_tiles;
    const TileSrc src = tile_src(more ? j + 2 : 0);
    if (more && j == 0) issue_tile(j + 2);
    const lds_char* const tile = smem + ((j + kNumBuf - 1) % kNumBuf) * kTileBytes;   // tile j-1
    if (j >= 1) {
      const lds_char* const pj = pbuf + ((j - 1) & 1) * kPBytes;
      const float* const aj = alphabuf + ((j - 1) & 1) * 64;
      bool rescale = false;
      f32x4_t al[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        al[rt] = *(const f32x4_t*)(aj + 16 * rt + 4 * G4);
        rescale |= (al[rt][0] != 1.f) | (al[rt][1] != 1.f) | (al[rt][2] != 1.f) | (al[rt][3] != 1.f);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
      {
        // P row 16*rt + i16, tokens 8*G4 .. 8*G4+7 (units 2*G4, 2*G4+1)
        const lds_char* const prow = pj + (16 * rt + i16) * kPStride;
        const int sp = swz_p(i16);
        const bf16x4_t p0 = *(const MLA_LDS bf16x4_t*)(prow + 8 * ((2 * G4) ^ sp));
        const bf16x4_t p1 = *(const MLA_LDS bf16x4_t*)(prow + 8 * ((2 * G4 + 1) ^ sp));
        pa[rt] = concat(p0, p1);
      }
      if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) U[rt][dt] *= al[rt];
      }
      pv_half(tile, 0, more, src);
    }
    if (j >= 1) pv_half(tile, 1, more, src);
    // tile j+1 must be resident at the next (X); tile j+2's copies may fly on
    wait_tile(more);
  }
  // (Z) row sums and reference maxima published; a partner wait that gave
  // up anywhere in the workgroup turns the unit's outputs into NaN
  if (__syncthreads_or(expired)) {
    write_uniform_result(p, b, k, g, __builtin_nanf(""));
    return;
  }

  // ---- finish: u = U / l, or partials (m, l, U or u) ------------------------
  const bool direct = p.n_split == 1;
  const size_t row_base = direct ? (size_t)b * p.R : ((size_t)b * p.n_split + k) * p.R;
  if (stage_u(p)) {
    // bf16 u = U / l (0 for a row that saw no token of the split) into LDS
    // (the tile buffers are free after (Z)), then one 1-KB store per row
    lds_char* const stg = smem;   // [64 rows][kStagePitch]
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * rt + 4 * G4 + i;
        const float lval = lsum[rr] + lsum[64 + rr];
        // one reciprocal per row: U * (1/l) is within 1 ulp of U / l, and
        // a bf16 value v stays v (U = v * l rounds back to v)
        const float inv = lval > 0.f ? 1.f / lval : 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const float u = U[rt][dt][i] * inv;
          *(MLA_LDS uint16_t*)(stg + rr * kStagePitch + (128 * v + 16 * dt + i16) * 2) = f2bf(u);
        }
      }
    lds_barrier();  // (W) u staged
    uint16_t* const dst = direct ? (uint16_t*)p.out : (uint16_t*)p.part_u;
#pragma unroll 4
    for (int s = 0; s < 16; ++s) {
      const int rr = 16 * v + s;
      if (row0 + rr >= p.R) break;   // wave-uniform
      const u32x4_t val = *(const MLA_LDS u32x4_t*)(stg + rr * kStagePitch + lane * 16);
      *(u32x4_t*)(dst + (row_base + row0 + rr) * kDc + 8 * lane) = val;
    }
  }
  // row statistics (and fp32 u or U straight from registers)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * rt + 4 * G4 + i;
      const int r = row0 + rr;
      if (r >= p.R) continue;
      const float lval = lsum[rr] + lsum[64 + rr];
      const float mval = mbuf[rr];
      if (!stage_u(p)) {
        const size_t o = (row_base + r) * kDc + 128 * v + i16;
        float* const dst = direct ? (float*)p.out : (float*)p.part_u;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dst[o + 16 * dt] = direct ? U[rt][dt][i] / lval : U[rt][dt][i];
      }
      if (v == 0 && i16 == 0) {
        if (direct) {
          if (p.lse) p.lse[(size_t)b * p.R + r] = (mval + log2f(lval)) * kLn2;
        } else {
          p.part_ml[(row_base + r) * 2] = mval;
          p.part_ml[(row_base + r) * 2 + 1] = lval;
        }
      }
    }
}

}  // namespace

hipError_t launch_decode_mfma_fp8(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(p.per_xcd * kNumXcd), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
