// Prefill in the explicit (expanded) form (PaperTrace "02 · DeepSeek-V2
// analysis", section 6.1: with many queries per step the keys and values are
// expanded per head, K_h = [W_UK[h] c ; k^R] (128 + 64 dims) and
// V_h = W_UV[h] c (128 dims), and ordinary attention runs on them; in exact
// arithmetic it is the same function as the absorbed decode form).
//
// Causal flash attention, d_qk = 192, d_v = 128, bf16 inputs, fp32
// accumulation. One workgroup of 4 waves per (sequence b, head h, 128
// queries); wave w owns queries 32w..32w+31 of the block (two 16-query
// columns) and keeps their 192 query values in registers, so every key or
// value fragment read from LDS feeds two MFMAs. Keys and values stream
// through LDS in tiles of 64 keys, double-buffered: the next tile's direct
// global -> LDS copies are in flight during the current tile's math, with
// one workgroup barrier per tile. Per 16-key block a wave computes
//   S^T[key][query] = K[key][:] . Q^T   on v_mfma_f32_16x16x32_bf16,
// so each lane holds 4 keys x 1 query. After the online softmax (log2
// domain, scale folded into the exponent, lazily moved maximum) the lane's 4 + 4 probabilities of
// key blocks 2kk and 2kk+1 are taken as K elements 0..7 of
//   O^T[dv][query] += V^T[dv][key] . P^T[key][query]   on v_mfma_f32_16x16x32_bf16
// (a K order of our choosing: the V^T operand is read in the same order by
// two transposed reads ds_read_b64_tr_b16, keys 4g..4g+3 and 16+4g..16+4g+3).
// Query i of a sequence sits at position n_kv - n_q + i and sees keys s <= it.
#include "mla_device.h"
#include "dma.h"
#include "mla_extra.h"

namespace mla {
namespace {

constexpr int kQBlock = 128;                      // queries per workgroup, 32 per wave
constexpr int kKTile = 64;                        // keys per tile
constexpr int kThreads = 256;
constexpr int kKRow = 256;                        // bytes per k_nope / V row in LDS
constexpr int kRRow = 128;                        // bytes per k_rope row in LDS
constexpr int kOffKr = kKTile * kKRow;            // k_nope [64][256 B], k_rope [64][128 B], V
constexpr int kOffV = kOffKr + kKTile * kRRow;
constexpr int kBuf = kOffV + kKTile * kKRow;      // one tile: 40 KB
constexpr int kLds = 2 * kBuf;                    // two tiles: 80 KB (two workgroups per CU)
// The running maximum of a query moves only when a tile's maximum exceeds it
// by more than this (log2 units): weights stay below 2^8, and the O rescale
// is skipped for the many tiles that do not move it.
constexpr float kLazyMax = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// K rows: 16-B chunk c of key t lives at chunk c ^ (t & 15), so the 16 keys
// of an MFMA A fragment read 16 distinct chunks. Rope rows (128 B): chunk c
// at c ^ ((t >> 1) & 7), which spreads 16 consecutive keys over 256 B. V
// rows: 32-B block n (16 dv) of key t lives at block n ^ (t & 7), so the
// transposed reads of 8 consecutive keys hit distinct banks.
__device__ __forceinline__ int k_pos(int t, int c) { return c ^ (t & 15); }
__device__ __forceinline__ int r_pos(int t, int c) { return c ^ ((t >> 1) & 7); }
__device__ __forceinline__ int v_byte(int t, int byte) {
  return (((byte >> 5) ^ (t & 7)) << 5) | (byte & 31);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kLds];
  lds_char* const smem = (lds_char*)smem_raw;
  // every query block of one (sequence, head) runs on the same XCD, so that
  // head's keys and values (2 MB at 4096 tokens) stay in that XCD's L2;
  // within a head the blocks with the most keys (the last) go first
  const int n_qb = (p.n_q + kQBlock - 1) / kQBlock;
  int bh, qb;
  if ((p.B * p.H) % kNumXcd == 0) {
    const int x = blockIdx.x % kNumXcd, idx = blockIdx.x / kNumXcd;
    bh = kNumXcd * (idx / n_qb) + x;
    qb = n_qb - 1 - idx % n_qb;
  } else {
    bh = blockIdx.x / n_qb;
    qb = n_qb - 1 - blockIdx.x % n_qb;
  }
  const int h = bh % p.H, b = bh / p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, G4 = lane >> 4;
  const int q0 = qb * kQBlock;
  const int shift = p.n_kv - p.n_q;              // position of query i is shift + i
  const int kv_end = min(p.n_kv, shift + min(q0 + kQBlock, p.n_q));   // keys this block needs
  const int n_tiles = (kv_end + kKTile - 1) / kKTile;
  // this wave's queries: [wq0, wq1]; a wave past the end only copies
  const int wq0 = q0 + 32 * w;
  const int wq1 = min(wq0 + 31, p.n_q - 1);
  const bool active = wq0 < p.n_q;

  // copy duties per tile (keys 16w..16w+15 of the tile): 4 x 1 KB of k_nope,
  // 2 x 1 KB of k_rope, 4 x 1 KB of V; the lane's global chunk is the one the
  // swizzled layout puts at its LDS slot
  const size_t head_stride = (size_t)p.H * kKRow;                  // bytes between keys
  const char* const kn_base = (const char*)p.k_nope + ((size_t)b * p.n_kv * p.H + h) * kKRow;
  const char* const v_base = (const char*)p.v + ((size_t)b * p.n_kv * p.H + h) * kKRow;
  const char* const kr_base = (const char*)p.k_rope + (size_t)b * p.n_kv * kRRow;
  // per-lane byte offsets of the copies within a tile; keys past the end of
  // the sequence (only in its last tile) read the last key instead
  uint32_t off_k[4], off_v[4], off_r[2];
  auto copy_offsets = [&](int last) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * i + (lane >> 4), slot = lane & 15;
      const uint32_t row = (uint32_t)min(t, last) * (uint32_t)head_stride;
      off_k[i] = row + 16 * k_pos(t, slot);
      off_v[i] = row + 16 * (((slot >> 1) ^ (t & 7)) * 2 + (slot & 1));   // V chunk of this slot
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 16 * w + 8 * i + (lane >> 3), slot = lane & 7;
      off_r[i] = (uint32_t)min(t, last) * kRRow + 16 * r_pos(t, slot);
    }
  };
  copy_offsets(kKTile - 1);
  auto issue_tile = [&](int tile) __attribute__((always_inline)) {
    const int t0 = tile * kKTile;
    if (t0 + kKTile > p.n_kv) copy_offsets(p.n_kv - 1 - t0);
    lds_char* const buf = smem + (tile & 1) * kBuf;
    const char* const kn = kn_base + (size_t)t0 * head_stride;
    const char* const vv = v_base + (size_t)t0 * head_stride;
    const char* const kr = kr_base + (size_t)t0 * kRRow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma_copy16(kn, off_k[i], buf + (16 * w + 4 * i) * kKRow);
      dma_copy16(vv, off_v[i], buf + kOffV + (16 * w + 4 * i) * kKRow);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) dma_copy16(kr, off_r[i], buf + kOffKr + (16 * w + 8 * i) * kRRow);
  };
  if (n_tiles > 0) issue_tile(0);

  // this wave's queries as MFMA B fragments: [column][4 k-steps of q_nope, 2 of q_rope]
  bf16x8_t qf[2][6];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int qi = wq0 + 16 * cb + i16;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) qf[cb][ks] = (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
    if (qi < p.n_q) {
      const size_t row = ((size_t)b * p.n_q + qi) * p.H + h;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[cb][ks] = load_bf16x8((const uint16_t*)p.q_nope + row * kDh + 32 * ks + 8 * G4);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        qf[cb][4 + ks] = load_bf16x8((const uint16_t*)p.q_rope + row * kDr + 32 * ks + 8 * G4);
    }
  }

  f32x4_t o[8][2];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) o[nb][cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};   // this lane's two queries
  const float sl2 = p.scale_log2;

  //   k_nope: key 16kb + i16, chunk (4ks + G4) ^ i16 -> i16*256 + 16(G4^i16), ^ 64ks
  //   k_rope: chunk (4ks' + G4) ^ (i16 >> 1) -> i16*128 + 16(G4^(i16>>1)), ^ 64ks'
  //   V: key rows 32kk + tl and +16, tl = 4G4 + i16/4, bytes 8(i16&3) of dv
  //      block nb ^ (tl & 7) -> tl*256 + 32(tl&7) + 8(i16&3), ^ 32nb
  const uint32_t lane_kq = (uint32_t)(i16 * kKRow + 16 * (G4 ^ i16));
  const uint32_t lane_rq = (uint32_t)(i16 * kRRow + 16 * (G4 ^ (i16 >> 1)));
  const int v_tl = 4 * G4 + (i16 >> 2);
  const uint32_t lane_vq = (uint32_t)(v_tl * kKRow + 32 * (v_tl & 7) + 8 * (i16 & 3));
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * kKTile;
    dma_wait<0>();                               // this wave's copies of tile `tile` landed
    lds_barrier();                               // all copies landed; tile-1's buffer is free
    if (tile + 1 < n_tiles) issue_tile(tile + 1);
    // keys past the wave's last query are masked for all of its queries
    if (!active || t0 > shift + wq1) continue;
    // fragment addresses: the swizzles XOR bits 4..7 of a row's bytes only,
    // so a fragment's address is a per-lane base XOR a per-k-step (or per-dv-
    // block) constant plus an immediate; the bases are made opaque here so
    // that one register per base is kept instead of one per fragment
    uint32_t kq = lane_kq + (uint32_t)(tile & 1) * kBuf, rq = lane_rq + (uint32_t)(tile & 1) * kBuf;
    uint32_t vq = lane_vq + (uint32_t)(tile & 1) * kBuf;
    asm volatile("" : "+v"(kq), "+v"(rq), "+v"(vq));
    // ---- scores S^T for the 4 key blocks of the tile and both query columns
    // fragment f = (key block f / 6, k-step f % 6); a ring of kRing reads
    // stays in flight ahead of the MFMAs that consume them
    f32x4_t s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    auto kfrag = [&](int f) __attribute__((always_inline)) -> bf16x8_t {
      const int kb = f / 6, ks = f % 6;
      return lds_read_b128(ks < 4 ? smem + 16 * kKRow * kb + (kq ^ (64 * ks))
                                  : smem + kOffKr + 16 * kRRow * kb + (rq ^ (64 * (ks - 4))));
    };
    constexpr int kRing = 6;
    bf16x8_t ring[kRing];
#pragma unroll
    for (int f = 0; f < kRing; ++f) ring[f] = kfrag(f);
    __builtin_amdgcn_sched_group_barrier(0x100, kRing, 0);
#pragma unroll
    for (int f = 0; f < 24; ++f) {
      const bf16x8_t af = ring[f % kRing];
      if (f + kRing < 24) ring[f % kRing] = kfrag(f + kRing);
      s[f / 6][0] = mfma16x16x32(af, qf[0][f % 6], s[f / 6][0]);
      s[f / 6][1] = mfma16x16x32(af, qf[1][f % 6], s[f / 6][1]);
      if (f + kRing < 24) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // ---- V^T fragments for O^T += V^T P^T (two 32-key steps): fragment
    // f = (step f / 8, dv block f % 8), two transposed reads each; the first
    // kVRing are read now, under the softmax, the rest kVRing ahead of use
    auto vfrag = [&](int f) __attribute__((always_inline)) -> bf16x8_t {
      const lds_char* const lo = smem + kOffV + 32 * kKRow * (f / 8) + (vq ^ (32 * (f % 8)));
      return concat(lds_read_tr16(lo), lds_read_tr16(lo + 16 * kKRow));
    };
    constexpr int kVRing = 4;
    bf16x8_t vring[kVRing];
#pragma unroll
    for (int f = 0; f < kVRing; ++f) vring[f] = vfrag(f);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVRing, 0);
    // ---- causal mask (only tiles that reach past the wave's first query)
    if (t0 + kKTile - 1 > shift + wq0) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int qpos = shift + wq0 + 16 * cb + i16;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + 16 * kb + 4 * G4 + i > qpos) s[kb][cb][i] = -INFINITY;
      }
    }
    // ---- online softmax per query (its keys are spread over lanes l, l^16, l^32, l^48)
    bf16x4_t pb[4][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[kb][cb][i]);
      mt = wave_max16(mt) * sl2;
      const float mold = m[cb];
      const float mnew = (mt - mold > kLazyMax) ? mt : mold;   // -inf - -inf is NaN: keep
      const float base = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = mnew == mold ? 1.f : fast_exp2(mold - mnew);
      m[cb] = mnew;
      // row sum of the bf16-rounded weights (the values the MFMA multiplies)
      float ls = 0.f;
      const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint32_t lo = pack_bf16x2(fast_exp2(fmaf(s[kb][cb][0], sl2, -base)),
                                        fast_exp2(fmaf(s[kb][cb][1], sl2, -base)));
        const uint32_t hi = pack_bf16x2(fast_exp2(fmaf(s[kb][cb][2], sl2, -base)),
                                        fast_exp2(fmaf(s[kb][cb][3], sl2, -base)));
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo), ones, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi), ones, ls, false);
        pb[kb][cb] = __builtin_bit_cast(bf16x4_t, (u32x2_t){lo, hi});
      }
      l[cb] = l[cb] * alpha + wave_sum16(ls);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[nb][cb] *= alpha;
      }
    }
    // ---- O^T += V^T P^T
    bf16x8_t pB[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) pB[kk][cb] = concat(pb[2 * kk][cb], pb[2 * kk + 1][cb]);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      const bf16x8_t va = vring[f % kVRing];
      if (f + kVRing < 16) vring[f % kVRing] = vfrag(f + kVRing);
      o[f % 8][0] = mfma16x16x32(va, pB[f / 8][0], o[f % 8][0]);
      o[f % 8][1] = mfma16x16x32(va, pB[f / 8][1], o[f % 8][1]);
      if (f + kVRing < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  }

  // ---- finish: lane holds O^T[dv 16nb + 4*G4 + i][query wq0 + 16cb + i16]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int qi = wq0 + 16 * cb + i16;
    if (qi >= p.n_q) continue;
    const size_t row = ((size_t)b * p.n_q + qi) * p.H + h;
    const float inv = 1.f / l[cb];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const size_t off = row * kDh + 16 * nb + 4 * G4;
      const f32x4_t r = o[nb][cb] * inv;
      if (p.o_bf16) {
        *(u32x2_t*)((uint16_t*)p.o + off) = (u32x2_t){pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      } else {
        *(f32x4_t*)((float*)p.o + off) = r;
      }
    }
    if (p.lse && G4 == 0) p.lse[row] = (m[cb] + log2f(l[cb])) * kLn2;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  const int n_qb = (p.n_q + kQBlock - 1) / kQBlock;
  hipLaunchKernelGGL(prefill_kernel, dim3(p.B * p.H * n_qb), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
