// Paged absorbed-MLA decode on gfx950 bf16 MFMA.
//
// One workgroup (4 waves, 256 threads) owns a work unit (sequence b, split k,
// group g of 64 query rows). It streams the split's 64-token cache pages
// through LDS (double buffered, asynchronous 16-byte global->LDS copies) and,
// per page:
//   1. scores  S^T[token][row] = K[token][576] . Q^T[576][row] on MFMA
//      16x16x32 (the 512 latent + 64 rope features of the V2 analysis page's
//      576-element cache, section 1.3); each wave does 32 tokens x 32 rows
//      with its rows' absorbed queries held in registers;
//   2. online softmax in fp32 (log2 domain, scale folded in): per-row page
//      maxima exchanged through LDS, probabilities rounded once to bf16 and
//      staged in LDS, row sums taken from the rounded values;
//   3. aggregation U[row][d] += P[row][token] C[token][d] on MFMA with the
//      latent tile read transposed (ds_read_b64_tr_b16); each wave owns 128
//      of the 512 latent dimensions for all 64 rows (section 6.1: each head
//      aggregates latents with its own weights).
// The split ends by writing either u = U / l and lse, or fp32 partials
// (m, l, U) for the log-sum-exp combine kernel.
//
// LDS (157,696 B of gfx950's 160 KiB): two page tiles of 73,728 B (latent rows
// of 1,024 B and rope rows of 128 B, XOR-swizzled at 16-B granularity so the
// score reads and the transposed reads are bank-conflict free), the bf16
// probability tile and two small per-row exchange arrays.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kLatBytes = kPage * kDc * 2;          // 65536
constexpr int kRopeBytes = kPage * kDr * 2;         // 8192
constexpr int kTileBytes = kLatBytes + kRopeBytes;  // 73728
constexpr int kPStride = 144;                       // bytes per probability row
constexpr int kPBytes = kRowsPerGroup * kPStride;   // 9216
constexpr int kOffP = 2 * kTileBytes;               // 147456
constexpr int kOffRed = kOffP + kPBytes;            // per-row page maxima [2][64] f32
constexpr int kOffLsum = kOffRed + 2 * 64 * 4;      // per-row sums [2][64] f32
constexpr int kOffAlpha = kOffLsum + 2 * 64 * 4;    // per-row rescale factor [64] f32
constexpr int kOffM = kOffAlpha + 64 * 4;           // per-row final reference max [64] f32
constexpr int kLdsBytes = kOffM + 64 * 4;           // 158208

// The running reference max of a row only moves when a page's max exceeds it
// by more than kLazyMax (log2 units): probabilities are then bounded by
// 2^kLazyMax, which fp32 sums and bf16 probabilities hold exactly as well,
// and the accumulator rescale runs on the first page and on rare jumps only.
// u, l and lse do not depend on the reference.
constexpr float kLazyMax = 8.0f;

// Latent rows: 16-B chunk j of token t lives at chunk j ^ swz_lat(t & 15).
// swz_lat is a bijection of 0..15, so 16 consecutive tokens reading the same
// chunk hit 16 different chunk columns (all 64 banks), and for the transposed
// reads (4 consecutive tokens x 2 adjacent chunks per 16-lane group, groups
// 8 tokens apart) the 32 lanes of a pass cover 64 distinct banks.
__device__ __forceinline__ int swz_lat(int s) {
  return (s & 8) | ((s & 3) << 1) | ((s >> 2) & 1);
}
// Rope rows (128 B): chunk j (0..7) of token t lives at chunk j ^ ((t>>1)&7).
__device__ __forceinline__ int swz_rope(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ void block_sync() { __syncthreads(); }

// Issue the asynchronous copy of one cache page into an LDS tile. Tokens at
// or beyond `nvalid` (past the end of the sequence) re-read token nvalid-1 so
// the tile never holds stale or poisoned data; their weights are exactly 0.
// Wave w copies the latent rows t = 16*m + 4*w + q (m, q in 0..3), so its 16
// row copies use only 4 swizzle patterns (lane offsets lat_off[q]).
__device__ __forceinline__ void load_tile(lds_char* tile, const char* ckv_page,
                                          const char* kr_page, int nvalid, int w, int lane,
                                          const uint32_t (&lat_off)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = 16 * m + 4 * w + q;
      const int ts = min(t, nvalid - 1);
      global_to_lds16(ckv_page + (uint32_t)(ts * 1024) + lat_off[q], tile + t * 1024);
    }
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2) {
    const int m = 2 * w + m2;
    const int t = 8 * m + (lane >> 3);
    const int ts = min(t, nvalid - 1);
    const int j = (lane & 7) ^ swz_rope(t);
    global_to_lds16(kr_page + ts * 128 + j * 16, tile + kLatBytes + m * 1024);
  }
}

__device__ void write_uniform_result(const DecodeParams& p, int b, int k, int g, float mval,
                                     float lval, float uval) {
  // Every row of the unit gets (m, l, U) = (mval, lval, uval); used to mark
  // out-of-range sequences with NaN.
  const int tid = threadIdx.x;
  const int r0 = g * kRowsPerGroup;
  const int nrows = min(kRowsPerGroup, p.R - r0);
  for (int e = tid; e < nrows * kDc; e += kThreads) {
    const int r = r0 + e / kDc, d = e % kDc;
    if (p.n_split == 1) {
      const size_t o = ((size_t)b * p.R + r) * kDc + d;
      if (p.out_bf16) ((uint16_t*)p.out)[o] = f2bf(uval / lval);
      else ((float*)p.out)[o] = uval / lval;
    } else {
      p.part_u[(((size_t)b * p.n_split + k) * p.R + r) * kDc + d] = uval;
    }
  }
  for (int r = r0 + tid; r < r0 + nrows; r += kThreads) {
    if (p.n_split == 1) {
      if (p.lse) p.lse[(size_t)b * p.R + r] = (mval + log2f(lval)) * kLn2;
    } else {
      float* ml = p.part_ml + (((size_t)b * p.n_split + k) * p.R + r) * 2;
      ml[0] = mval;
      ml[1] = lval;
    }
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_bf16_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;

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
  const int hh = w & 1;     // score rows 32*hh..+31 of the group
  const int th = w >> 1;    // score tokens 32*th..+31 of each page
  const int i16 = lane & 15;
  const int G4 = lane >> 4;

  // ---- sequence and split bounds, range checks -----------------------------
  const int L = p.seq_lens[b];
  bool bad = (L < p.T) || (L > p.max_seq_len) || ((L + kPage - 1) / kPage > p.max_pages);
  const int tok0 = k * p.split_tokens;
  const int tok1 = min(tok0 + p.split_tokens, L);
  const int pg_begin = tok0 / kPage;
  const int pg_end = (tok1 + kPage - 1) / kPage;
  const int32_t* btrow = p.block_table + (size_t)b * p.max_pages;
  if (!bad) {
    bool local_bad = false;
    for (int j = pg_begin + tid; j < pg_end; j += kThreads) {
      const int id = btrow[j];
      local_bad |= (id < 0) || (id >= p.n_pages);
    }
    bad = __syncthreads_or(local_bad);
  }
  if (bad) {
    write_uniform_result(p, b, k, g, __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    return;
  }
  if (tok0 >= tok1) return;   // split past the end of the sequence: no partial

  const int row0 = g * kRowsPerGroup;
  // visible-token limit of a row: s < min(L - T + t + 1, tok1)
  auto row_limit = [&](int rr) -> int {
    const int r = row0 + rr;
    const int t = (r < p.R) ? r / p.H : 0;
    return min(L - p.T + t + 1, tok1);
  };
  // smallest limit over the group's rows (the first query token's rows)
  const int lim_min = row_limit(0);

  // ---- absorbed queries of this wave's 32 rows in registers -----------------
  bf16x8_t qB[2][18];
  int lim_s[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int rr = 32 * hh + 16 * ht + i16;
    const int r = row0 + rr;
    lim_s[ht] = row_limit(rr);
    if (r < p.R) {
      const uint16_t* ql = (const uint16_t*)p.q_lat + ((size_t)b * p.R + r) * kDc + 8 * G4;
      const uint16_t* qr = (const uint16_t*)p.q_rope + ((size_t)b * p.R + r) * kDr + 8 * G4;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qB[ht][ks] = load_bf16x8(ql + 32 * ks);
      qB[ht][16] = load_bf16x8(qr);
      qB[ht][17] = load_bf16x8(qr + 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qB[ht][ks] = (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  lds_char* const pbuf = smem + kOffP;
  float* const redmax = (float*)(smem_raw + kOffRed);   // [2][64]
  float* const lsum = (float*)(smem_raw + kOffLsum);    // [2][64]
  float* const alphabuf = (float*)(smem_raw + kOffAlpha);
  float* const mbuf = (float*)(smem_raw + kOffM);
  uint32_t lat_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) lat_off[q] = (uint32_t)(lane ^ swz_lat(4 * w + q)) * 16u;

  // per-lane swizzle constants
  const int fl = swz_lat(i16);            // score rows: token & 15 == i16
  const int fr = i16 >> 1;                // rope swizzle of score rows
  const int xq = 4 * (G4 & 1) + (i16 >> 2);
  const int c0 = (i16 & 3) >> 1;

  f32x4_t U[4][8];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) U[rt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_s[2] = {-INFINITY, -INFINITY};
  float l_s[2] = {0.f, 0.f};

  const char* ckv_base = (const char*)p.ckv;
  const char* kr_base = (const char*)p.kr;
  {
    const int id = __builtin_amdgcn_readfirstlane(btrow[pg_begin]);
    load_tile(smem, ckv_base + (size_t)id * kLatBytes, kr_base + (size_t)id * kRopeBytes,
              min(kPage, L - pg_begin * kPage), w, lane, lat_off);
  }
  // page id of the next page, fetched one iteration ahead of its use
  int id_next = (pg_begin + 1 < pg_end) ? btrow[pg_begin + 1] : 0;

  for (int pg = pg_begin; pg < pg_end; ++pg) {
    lds_char* const tile = smem + ((pg - pg_begin) & 1) * kTileBytes;
    wait_vmem();
    block_sync();  // (A) tile pg resident; previous page fully consumed
    if (pg + 1 < pg_end) {
      const int id = __builtin_amdgcn_readfirstlane(id_next);
      load_tile(smem + ((pg + 1 - pg_begin) & 1) * kTileBytes, ckv_base + (size_t)id * kLatBytes,
                kr_base + (size_t)id * kRopeBytes, min(kPage, L - (pg + 1) * kPage), w, lane,
                lat_off);
      if (pg + 2 < pg_end) id_next = btrow[pg + 2];
    }

    // ---- 1. scores: tokens 32*th + 16*tt + (4*G4 + i), rows 32*hh + 16*ht + i16
    f32x4_t S[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      S[tt][0] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      S[tt][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      const int t = 32 * th + 16 * tt + i16;
      const lds_char* latp = tile + t * 1024;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8_t a = lds_read_b128(latp + (16 * (ks >> 2) + ((4 * (ks & 3) + G4) ^ fl)) * 16);
        S[tt][0] = mfma16x16x32(a, qB[0][ks], S[tt][0]);
        S[tt][1] = mfma16x16x32(a, qB[1][ks], S[tt][1]);
      }
      const lds_char* ropep = tile + kLatBytes + t * 128;
#pragma unroll
      for (int ks = 16; ks < 18; ++ks) {
        const bf16x8_t a = lds_read_b128(ropep + ((4 * (ks - 16) + G4) ^ fr) * 16);
        S[tt][0] = mfma16x16x32(a, qB[0][ks], S[tt][0]);
        S[tt][1] = mfma16x16x32(a, qB[1][ks], S[tt][1]);
      }
    }

    const int ptok0 = pg * kPage;
    const bool masked = ptok0 + kPage > lim_min;
    float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float z = S[tt][ht][i] * p.scale_log2;
          if (masked) {
            const int s = ptok0 + 32 * th + 16 * tt + 4 * G4 + i;
            if (s >= lim_s[ht]) z = -INFINITY;
          }
          S[tt][ht][i] = z;
          mx[ht] = fmaxf(mx[ht], z);
        }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      mx[ht] = wave_max16(mx[ht]);
      if (lane < 16) redmax[th * 64 + 32 * hh + 16 * ht + lane] = mx[ht];
    }
    block_sync();  // (B) page maxima of all rows visible

    // ---- 2. softmax: probabilities of this wave's 32 tokens x 32 rows -------
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int rr = 32 * hh + 16 * ht + i16;
      const float mt = fmaxf(redmax[rr], redmax[64 + rr]);
      const float mold = m_s[ht];
      const float mnew = (mt - mold > kLazyMax) ? mt : mold;   // -inf - -inf is NaN: keep
      const float base = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = (mnew == mold) ? 1.f : fast_exp2(mold - mnew);
      m_s[ht] = mnew;
      if (th == 0 && lane < 16) alphabuf[rr] = alpha;
      float ls = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint32_t lo = pack_bf16x2(fast_exp2(S[tt][ht][0] - base), fast_exp2(S[tt][ht][1] - base));
        const uint32_t hi = pack_bf16x2(fast_exp2(S[tt][ht][2] - base), fast_exp2(S[tt][ht][3] - base));
        ls += bf2f(lo & 0xffff) + bf2f(lo >> 16) + bf2f(hi & 0xffff) + bf2f(hi >> 16);
        *(MLA_LDS u32x2_t*)(pbuf + rr * kPStride + (32 * th + 16 * tt + 4 * G4) * 2) =
            (u32x2_t){lo, hi};
      }
      l_s[ht] = l_s[ht] * alpha + wave_sum16(ls);
    }
    block_sync();  // (C) probability tile and rescale factors complete

    // ---- 3. aggregation: rows 16*rt + (4*G4 + i), dims 128*w + 16*dt + i16 --
    {
      f32x4_t al[4];
      bool rescale = false;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        al[rt] = *(const f32x4_t*)(alphabuf + 16 * rt + 4 * G4);
        rescale |= (al[rt][0] != 1.f) | (al[rt][1] != 1.f) | (al[rt][2] != 1.f) | (al[rt][3] != 1.f);
      }
      if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) U[rt][dt] *= al[rt];
      }
    }
    const int xq32 = 32 * xq;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        a[rt] = lds_read_b128(pbuf + (16 * rt + i16) * kPStride + (32 * ks + 8 * G4) * 2);
      const lds_char* rowA = tile + (32 * ks + 8 * G4 + (i16 >> 2)) * 1024 + 256 * w + (i16 & 1) * 8;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int dx = (32 * dt) ^ xq32;              // 32 * (dt ^ xq)
        const bf16x4_t lo = lds_read_tr16(rowA + dx + 16 * c0);                  // tokens +0..3
        const bf16x4_t hi = lds_read_tr16(rowA + 4 * 1024 + dx + 16 * (c0 ^ 1)); // tokens +4..7
        const bf16x8_t bv = concat(lo, hi);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) U[rt][dt] = mfma16x16x32(a[rt], bv, U[rt][dt]);
      }
    }
  }

  // ---- finish: total row sums, then u = U / l or fp32 partials ------------
  if (lane < 16) {
    lsum[th * 64 + 32 * hh + lane] = l_s[0];
    lsum[th * 64 + 32 * hh + 16 + lane] = l_s[1];
    if (th == 0) {
      mbuf[32 * hh + lane] = m_s[0];
      mbuf[32 * hh + 16 + lane] = m_s[1];
    }
  }
  block_sync();
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * rt + 4 * G4 + i;
      const int r = row0 + rr;
      if (r >= p.R) continue;
      const float lval = lsum[rr] + lsum[64 + rr];
      const float mval = mbuf[rr];
      if (p.n_split == 1) {
        const size_t o = ((size_t)b * p.R + r) * kDc + 128 * w + i16;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const float u = U[rt][dt][i] / lval;
          if (p.out_bf16) ((uint16_t*)p.out)[o + 16 * dt] = f2bf(u);
          else ((float*)p.out)[o + 16 * dt] = u;
        }
        if (p.lse && w == 0 && i16 == 0) p.lse[(size_t)b * p.R + r] = (mval + log2f(lval)) * kLn2;
      } else {
        const size_t base = ((size_t)b * p.n_split + k) * p.R + r;
        float* pu = p.part_u + base * kDc + 128 * w + i16;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) pu[16 * dt] = U[rt][dt][i];
        if (w == 0 && i16 == 0) {
          p.part_ml[base * 2] = mval;
          p.part_ml[base * 2 + 1] = lval;
        }
      }
    }
}

}  // namespace

hipError_t launch_decode_mfma_bf16(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(decode_mfma_bf16_kernel, dim3(p.per_xcd * kNumXcd), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
