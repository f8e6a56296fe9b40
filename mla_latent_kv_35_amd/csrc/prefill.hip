// Prefill in the explicit (expanded) form (PaperTrace "02 · DeepSeek-V2
// analysis", section 6.1: with many queries per step the keys and values are
// expanded per head, K_h = [W_UK[h] c ; k^R] (128 + 64 dims) and
// V_h = W_UV[h] c (128 dims), and ordinary attention runs on them; in exact
// arithmetic it is the same function as the absorbed decode form).
//
// Causal flash attention, d_qk = 192, d_v = 128, bf16 inputs, fp32
// accumulation. One workgroup of 4 waves per (sequence b, head h, 64
// queries); wave w owns queries 16w..16w+15 of the block and keeps their 192
// query values in registers. Keys and values stream through LDS in tiles of
// 64 keys (register-staged, the next tile's loads in flight during the
// current tile's math). Per 16-key block a wave computes
//   S^T[key][query] = K[key][:] . Q^T   on v_mfma_f32_16x16x32_bf16,
// so each lane holds 4 keys x 1 query; after the online softmax (log2
// domain, scale folded into the exponent) those 4 probabilities are exactly
// the B operand of
//   O^T[dv][query] += V^T[dv][key] . P^T[key][query]   on v_mfma_f32_16x16x16_bf16,
// with V^T read from LDS by the transposed read ds_read_b64_tr_b16.
// Query i of a sequence sits at position n_kv - n_q + i and sees keys s <= it.
#include "mla_device.h"
#include "mla_extra.h"

namespace mla {
namespace {

constexpr int kQBlock = 64;
constexpr int kKTile = 64;
constexpr int kThreads = 256;
constexpr int kRow = 256;                       // bytes per key row in each LDS region
constexpr int kOffKr = kKTile * kRow;           // k_nope [64][256 B], then k_rope, then V
constexpr int kOffV = 2 * kKTile * kRow;
constexpr int kLds = 3 * kKTile * kRow;         // 48 KB

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x16(const bf16x4_t& a, const bf16x4_t& b,
                                                const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// K rows (k_nope, and k_rope padded to 256 B): 16-B chunk c of key t lives at
// chunk c ^ (t & 15), so the 16 keys of an MFMA A fragment read 16 distinct
// chunks. V rows: 32-B block n (16 dv) of key t lives at block n ^ (t & 7),
// so the transposed reads of 8 consecutive keys hit distinct banks.
__device__ __forceinline__ int k_chunk(int t, int c) { return ((c ^ (t & 15)) << 4); }
__device__ __forceinline__ int v_byte(int t, int byte) {
  return (((byte >> 5) ^ (t & 7)) << 5) | (byte & 31);
}

__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
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
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i16 = lane & 15, G4 = lane >> 4;
  const int q0 = qb * kQBlock;
  const int shift = p.n_kv - p.n_q;              // position of query i is shift + i
  const int kv_end = min(p.n_kv, shift + min(q0 + kQBlock, p.n_q));   // keys this block needs
  const int n_tiles = (kv_end + kKTile - 1) / kKTile;

  // this wave's queries as MFMA B fragments: 4 k-steps of q_nope, 2 of q_rope
  const int qi = q0 + 16 * w + i16;              // this lane's query (B column)
  bf16x8_t qf[6];
#pragma unroll
  for (int ks = 0; ks < 6; ++ks) qf[ks] = (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
  if (qi < p.n_q) {
    const size_t row = ((size_t)b * p.n_q + qi) * p.H + h;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = load_bf16x8((const uint16_t*)p.q_nope + row * kDh + 32 * ks + 8 * G4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[4 + ks] = load_bf16x8((const uint16_t*)p.q_rope + row * kDr + 32 * ks + 8 * G4);
  }
  const int qpos = shift + qi;                   // causal limit of this lane's query

  // cooperative tile loads: 4 k_nope + 2 k_rope + 4 V chunks of 16 B per thread
  u32x4_t stg[10];
  auto load_tile = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + kThreads * i, t = e >> 4, c = e & 15;
      const int s = t0 + t;
      stg[i] = (u32x4_t){0u, 0u, 0u, 0u};
      stg[6 + i] = (u32x4_t){0u, 0u, 0u, 0u};
      if (s < p.n_kv) {
        const size_t kv = ((size_t)b * p.n_kv + s) * p.H + h;
        stg[i] = *(const u32x4_t*)((const uint16_t*)p.k_nope + kv * kDh + 8 * c);
        stg[6 + i] = *(const u32x4_t*)((const uint16_t*)p.v + kv * kDh + 8 * c);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + kThreads * i, t = e >> 3, c = e & 7;
      const int s = t0 + t;
      stg[4 + i] = (u32x4_t){0u, 0u, 0u, 0u};
      if (s < p.n_kv)
        stg[4 + i] = *(const u32x4_t*)((const uint16_t*)p.k_rope + ((size_t)b * p.n_kv + s) * kDr + 8 * c);
    }
  };
  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + kThreads * i, t = e >> 4, c = e & 15;
      *(MLA_LDS u32x4_t*)(smem + t * kRow + k_chunk(t, c)) = stg[i];
      *(MLA_LDS u32x4_t*)(smem + kOffV + t * kRow + v_byte(t, 16 * c)) = stg[6 + i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + kThreads * i, t = e >> 3, c = e & 7;
      *(MLA_LDS u32x4_t*)(smem + kOffKr + t * kRow + k_chunk(t, c)) = stg[4 + i];
    }
  };

  f32x4_t o[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;                  // this lane's query (column i16)
  const float sl2 = p.scale_log2;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * kKTile;
    if (tile + 1 < n_tiles) load_tile(t0 + kKTile);
    // ---- scores S^T for the 4 key blocks of the tile
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      const int t = 16 * kb + i16;               // this lane's key (A row)
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const lds_char* a = ks < 4 ? smem + t * kRow + k_chunk(t, 4 * ks + G4)
                                   : smem + kOffKr + t * kRow + k_chunk(t, 4 * (ks - 4) + G4);
        s[kb] = mfma16x16x32(lds_read_b128(a), qf[ks], s[kb]);
      }
    }
    // ---- causal mask (only tiles that reach past the block's first query)
    if (t0 + kKTile - 1 > shift + q0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * kb + 4 * G4 + i > qpos) s[kb][i] = -INFINITY;
    }
    // ---- online softmax for this lane's query (keys spread over lanes l, l^16, l^32, l^48)
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt * sl2);
    const float base = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - base);
    m = mnew;
    bf16x4_t pb[4];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t lo = pack_bf16x2(exp2f(fmaf(s[kb][0], sl2, -base)), exp2f(fmaf(s[kb][1], sl2, -base)));
      const uint32_t hi = pack_bf16x2(exp2f(fmaf(s[kb][2], sl2, -base)), exp2f(fmaf(s[kb][3], sl2, -base)));
      ls += (bf2f(lo & 0xffff) + bf2f(lo >> 16)) + (bf2f(hi & 0xffff) + bf2f(hi >> 16));
      pb[kb] = __builtin_bit_cast(bf16x4_t, (u32x2_t){lo, hi});
    }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l = l * alpha + ls;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[nb] *= alpha;
    // ---- O^T += V^T P^T over the 4 key blocks
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int t = 16 * kb + 4 * G4 + (i16 >> 2);   // the key row this lane addresses
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x4_t vt = lds_read_tr16(smem + kOffV + t * kRow + v_byte(t, 32 * nb + 8 * (i16 & 3)));
        o[nb] = mfma16x16x16(vt, pb[kb], o[nb]);
      }
    }
    __syncthreads();                             // every wave is done with this tile
    if (tile + 1 < n_tiles) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- finish: lane holds O^T[dv 16nb + 4*G4 + i][query qi]
  if (qi < p.n_q) {
    const size_t row = ((size_t)b * p.n_q + qi) * p.H + h;
    const float inv = 1.f / l;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const size_t off = row * kDh + 16 * nb + 4 * G4;
      if (p.o_bf16) {
        *(u32x2_t*)((uint16_t*)p.o + off) =
            (u32x2_t){pack_bf16x2(o[nb][0] * inv, o[nb][1] * inv), pack_bf16x2(o[nb][2] * inv, o[nb][3] * inv)};
      } else {
        *(f32x4_t*)((float*)p.o + off) = o[nb] * inv;
      }
    }
    if (p.lse && G4 == 0) p.lse[row] = (m + log2f(l)) * kLn2;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  const int n_qb = (p.n_q + kQBlock - 1) / kQBlock;
  hipLaunchKernelGGL(prefill_kernel, dim3(p.B * p.H * n_qb), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
