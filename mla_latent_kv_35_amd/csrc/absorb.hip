// Absorption of W^UK into the content query (PaperTrace "02 · DeepSeek-V2
// analysis", section 1.2 and section 6): q_lat[n][h][:] = W_UK[h]^T q[n][h][:],
// so the score q^T (W^UK c) becomes q_lat . c against the cached latent.
//
// bf16: one workgroup per (head h, 128-wide latent block), the blocks of one
// head on one XCD. The weight block W_UK[h][0:128][d0:d0+128] is staged in
// LDS once, with the same 16-byte XOR swizzle the decode kernel uses, and read
// transposed (ds_read_b64_tr_b16) as the K-major MFMA operand; the workgroup
// then walks the tokens in blocks of 32, staging each block's queries in LDS
// (double-buffered, the next block's loads in flight during the current
// block's MFMAs) as the other operand. fp32: plain fp32 FMA. Query row
// (n, h) starts at (n * H + h) * q_rs elements, output row at
// (n * H + h) * o_rs (packed: 128 and 512).
#include "mla_device.h"
#include "mla_extra.h"
#include "mla_internal.h"
#include "rope_body.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kTokTile = 32;

__device__ __forceinline__ int swz16(int s) { return (s & 8) | ((s & 3) << 1) | ((s >> 2) & 1); }

constexpr int kWBlock = kDh * 256;                 // the staged 128 x 128 bf16 weight block
constexpr int kQBlock = kTokTile * kDh * 2;        // one block of 32 tokens' queries: 8 KB
constexpr int kAbsorbLds = kWBlock + 2 * kQBlock;  // 48 KB: three workgroups per CU

// Query rows staged in LDS: 256 B per token, 16-byte chunk c at c ^ (t & 15),
// so the 16 tokens of an MFMA A fragment read 16 distinct bank groups.
__device__ __forceinline__ int q_chunk(int t, int c) { return c ^ (t & 15); }

template <bool OUT_BF16>
__device__ __forceinline__ void absorb_bf16_block(int bid, lds_char* smem,
                                                  const uint16_t* __restrict__ q, long q_rs,
                                                  const uint16_t* __restrict__ wuk,
                                                  void* __restrict__ out, long o_rs, int n_tok,
                                                  int H) {
  // blocks on XCD x (= bid % 8) serve the heads h with h % 8 == x
  const int x = bid % kNumXcd, idx = bid / kNumXcd;
  const int h = kNumXcd * (idx >> 2) + x;
  if (h >= H) return;
  const int d0 = 128 * (idx & 3);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i16 = lane & 15, G4 = lane >> 4;
  const int n_tb = (n_tok + kTokTile - 1) / kTokTile;

  // query chunks of token block tb this thread moves: 32 tokens x 16 chunks
  // of 16 B = 512 chunks, 2 per thread (token t = e / 16, chunk c = e % 16)
  u32x4_t qv[kQBlock / 16 / kThreads];
  auto load_q = [&](int tb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kQBlock / 16 / kThreads; ++i) {
      const int e = tid + kThreads * i, t = e >> 4, c = e & 15;
      const int n = tb * kTokTile + t;
      qv[i] = (u32x4_t){0u, 0u, 0u, 0u};
      if (n < n_tok) qv[i] = *(const u32x4_t*)(q + ((size_t)n * H + h) * q_rs + 8 * c);
    }
  };
  auto store_q = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kQBlock / 16 / kThreads; ++i) {
      const int e = tid + kThreads * i, t = e >> 4, c = e & 15;
      *(MLA_LDS u32x4_t*)(smem + kWBlock + buf * kQBlock + t * 256 + q_chunk(t, c) * 16) = qv[i];
    }
  };
  // the weight block W_UK[h][0:128][d0:d0+128] and the first queries are in
  // flight before anything waits
  const uint16_t* wh = wuk + (size_t)h * kDh * kDc + d0;
  u32x4_t wv[(kDh * 16) / kThreads];
#pragma unroll
  for (int e = 0; e < (kDh * 16) / kThreads; ++e) {
    const int idx2 = e * kThreads + tid;
    const int j = idx2 >> 4, c = idx2 & 15;
    wv[e] = *(const u32x4_t*)(wh + (size_t)j * kDc + 8 * c);
  }
  load_q(0);
  // stage the weight block: row j = 16 chunks of 16 B, chunk c at c ^ swz16(j & 15)
#pragma unroll
  for (int e = 0; e < (kDh * 16) / kThreads; ++e) {
    const int idx2 = e * kThreads + tid;
    const int j = idx2 >> 4, c = idx2 & 15;
    *(MLA_LDS u32x4_t*)(smem + j * 256 + ((c ^ swz16(j & 15)) * 16)) = wv[e];
  }
  store_q(0);
  __syncthreads();

  // B operands (K = j, N = d) for this wave's two 16-wide d tiles, kept for
  // every token block
  const int xq = 4 * (G4 & 1) + (i16 >> 2);
  const int c0 = (i16 & 3) >> 1;
  bf16x8_t bw[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int dt = 2 * w + u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const lds_char* rowA = smem + (32 * ks + 8 * G4 + (i16 >> 2)) * 256 + (i16 & 1) * 8;
      const bf16x4_t lo = lds_read_tr16(rowA + (2 * (dt ^ xq) + c0) * 16);
      const bf16x4_t hi = lds_read_tr16(rowA + 4 * 256 + (2 * (dt ^ xq) + (c0 ^ 1)) * 16);
      bw[u][ks] = concat(lo, hi);
    }
  }
  for (int tb = 0; tb < n_tb; ++tb) {
    if (tb + 1 < n_tb) load_q(tb + 1);
    const lds_char* const qs = smem + kWBlock + (tb & 1) * kQBlock;
    const int n0 = tb * kTokTile;
    const int n_tt = min(2, (n_tok - n0 + 15) >> 4);   // 16-token blocks with a live token
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt >= n_tt) break;                              // uniform
      const int t = 16 * tt + i16;
      bf16x8_t a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[ks] = lds_read_b128(qs + t * 256 + q_chunk(t, 4 * ks + G4) * 16);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(a[ks], bw[u][ks], acc);
        const int d = d0 + 16 * (2 * w + u) + i16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = n0 + 16 * tt + 4 * G4 + i;
          if (n < n_tok) {
            const size_t o = ((size_t)n * H + h) * o_rs + d;
            if (OUT_BF16) ((uint16_t*)out)[o] = f2bf(acc[i]);
            else ((float*)out)[o] = acc[i];
          }
        }
      }
    }
    if (tb + 1 < n_tb) {
      store_q((tb + 1) & 1);   // that buffer was last read in block tb-1, before the barrier
      __syncthreads();
    }
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void absorb_bf16_kernel(const uint16_t* __restrict__ q,
                                                               long q_rs,
                                                               const uint16_t* __restrict__ wuk,
                                                               void* __restrict__ out, long o_rs,
                                                               int n_tok, int H) {
  __shared__ __attribute__((aligned(16))) char smem[kAbsorbLds];
  absorb_bf16_block<OUT_BF16>(blockIdx.x, (lds_char*)smem, q, q_rs, wuk, out, o_rs, n_tok, H);
}

// The query side of one decode step in one launch: the first n_abs blocks
// absorb W_UK into the content queries exactly as absorb_bf16_kernel does,
// the rest rotate the rope queries exactly as the d_r = 64 rope kernel does
// (one block per token and 32 heads). The two halves touch disjoint buffers.
// n_abs is a multiple of 8, so the absorb blocks keep their XCD placement.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void absorb_rope_kernel(
    const uint16_t* __restrict__ q, long q_rs, const uint16_t* __restrict__ wuk,
    void* __restrict__ out, long o_rs, int n_tok, int H, int n_abs, const uint16_t* q_rope,
    VecStrides si, uint16_t* q_rot, VecStrides so, const int32_t* pos, double base,
    const double* freq) {
  __shared__ __attribute__((aligned(16))) char smem[kAbsorbLds];   // either half's LDS
  const int bid = blockIdx.x;
  if (bid < n_abs) {
    absorb_bf16_block<OUT_BF16>(bid, (lds_char*)smem, q, q_rs, wuk, out, o_rs, n_tok, H);
  } else {
    const int r = bid - n_abs, n_hb = (H + kRope64Heads - 1) / kRope64Heads;
    rope64_block<true>(r / n_hb, r % n_hb, (lds_char*)smem, q_rope, si, q_rot, so, pos, H, base,
                       freq);
  }
}

// fp32: one workgroup of 4 waves per (token, head, 256 latent dims); wave w
// sums head dims j = 32w..32w+31 for every dim d = thread (coalesced rows of
// W_UK[h]), then the four partial sums are added in a fixed order.
constexpr int kF32Dims = 256;

// part: kThreads / 64 x kF32Dims floats of LDS for the partial sums
__device__ __forceinline__ void absorb_f32_block(int nh, int y, float* part,
                                                 const float* __restrict__ q, long q_rs,
                                                 const float* __restrict__ wuk,
                                                 float* __restrict__ out, long o_rs, int H) {
  const int h = nh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d0 = y * kF32Dims;
  const float* qr = q + (size_t)nh * q_rs + 32 * w;
  const float* wh = wuk + ((size_t)h * kDh + 32 * w) * kDc + d0;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int j = 0; j < 32; ++j) {
    const float qj = qr[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(qj, wh[(size_t)j * kDc + lane + 64 * i], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[w * kF32Dims + lane + 64 * i] = acc[i];
  __syncthreads();
  const int d = threadIdx.x;
  out[(size_t)nh * o_rs + d0 + d] =
      ((part[d] + part[kF32Dims + d]) + part[2 * kF32Dims + d]) + part[3 * kF32Dims + d];
}

__global__ __launch_bounds__(kThreads) void absorb_f32_kernel(const float* __restrict__ q,
                                                              long q_rs,
                                                              const float* __restrict__ wuk,
                                                              float* __restrict__ out, long o_rs,
                                                              int H) {
  __shared__ float part[kThreads / 64 * kF32Dims];
  absorb_f32_block(blockIdx.x, blockIdx.y, part, q, q_rs, wuk, out, o_rs, H);
}

// fp32 query side in one launch: block 2*(n*H + h) + y absorbs as
// absorb_f32_kernel's block (n*H + h, y) does, the rest rotate as the fp32
// d_r = 64 rope kernel does; the two halves touch disjoint buffers.
__global__ __launch_bounds__(kThreads) void absorb_rope_f32_kernel(
    const float* __restrict__ q, long q_rs, const float* __restrict__ wuk,
    float* __restrict__ out, long o_rs, int H, int n_abs, const float* q_rope, VecStrides si,
    float* q_rot, VecStrides so, const int32_t* pos, double base, const double* freq) {
  __shared__ __attribute__((aligned(16))) float part[kThreads / 64 * kF32Dims];   // either half's LDS
  const int bid = blockIdx.x;
  if (bid < n_abs) {
    absorb_f32_block(bid >> 1, bid & 1, part, q, q_rs, wuk, out, o_rs, H);
  } else {
    const int r = bid - n_abs, n_hb = (H + kRope64Heads - 1) / kRope64Heads;
    rope64_block<false>(r / n_hb, r % n_hb, (lds_char*)part, q_rope, si, q_rot, so, pos, H, base,
                        freq);
  }
}

}  // namespace

hipError_t launch_absorb(const void* q_nope, long q_rs, const void* w_uk, void* q_lat, long o_rs,
                         int in_bf16, int out_bf16, int n_tok, int H, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (in_bf16) {
    const dim3 grid(kNumXcd * ((H + kNumXcd - 1) / kNumXcd) * 4);
    if (out_bf16)
      hipLaunchKernelGGL(absorb_bf16_kernel<true>, grid, dim3(kThreads), 0, s,
                         (const uint16_t*)q_nope, q_rs, (const uint16_t*)w_uk, q_lat, o_rs, n_tok,
                         H);
    else
      hipLaunchKernelGGL(absorb_bf16_kernel<false>, grid, dim3(kThreads), 0, s,
                         (const uint16_t*)q_nope, q_rs, (const uint16_t*)w_uk, q_lat, o_rs, n_tok,
                         H);
  } else {
    hipLaunchKernelGGL(absorb_f32_kernel, dim3(n_tok * H, kDc / kF32Dims), dim3(kThreads), 0, s,
                       (const float*)q_nope, q_rs, (const float*)w_uk, (float*)q_lat, o_rs, H);
  }
  return hipGetLastError();
}

hipError_t launch_absorb_rope(const uint16_t* q_nope, long q_rs, const uint16_t* w_uk,
                              void* q_lat, long o_rs, int out_bf16, const uint16_t* q_rope,
                              VecStrides si, uint16_t* q_rot, VecStrides so, const int32_t* pos,
                              int n_tok, int H, double base, const double* freq, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  const int n_abs = kNumXcd * ((H + kNumXcd - 1) / kNumXcd) * 4;
  const int n_rope = n_tok * ((H + kRope64Heads - 1) / kRope64Heads);
  static_assert(kRope64Threads == kThreads, "one block size for both halves");
  const dim3 grid(n_abs + n_rope);
  if (out_bf16)
    hipLaunchKernelGGL(absorb_rope_kernel<true>, grid, dim3(kThreads), 0, s, q_nope, q_rs, w_uk,
                       q_lat, o_rs, n_tok, H, n_abs, q_rope, si, q_rot, so, pos, base, freq);
  else
    hipLaunchKernelGGL(absorb_rope_kernel<false>, grid, dim3(kThreads), 0, s, q_nope, q_rs, w_uk,
                       q_lat, o_rs, n_tok, H, n_abs, q_rope, si, q_rot, so, pos, base, freq);
  return hipGetLastError();
}

}  // namespace mla

namespace mla {

hipError_t launch_absorb_rope_f32(const float* q_nope, long q_rs, const float* w_uk, float* q_lat,
                                  long o_rs, const float* q_rope, VecStrides si, float* q_rot,
                                  VecStrides so, const int32_t* pos, int n_tok, int H,
                                  double base, const double* freq, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  static_assert(kRope64Threads == kThreads, "one block size for both halves");
  static_assert(kThreads / 64 * kF32Dims * 4 >= 512, "the rope (cos, sin) table fits");
  const int n_abs = n_tok * H * (kDc / kF32Dims);
  const int n_rope = n_tok * ((H + kRope64Heads - 1) / kRope64Heads);
  hipLaunchKernelGGL(absorb_rope_f32_kernel, dim3(n_abs + n_rope), dim3(kThreads), 0, s, q_nope,
                     q_rs, w_uk, q_lat, o_rs, H, n_abs, q_rope, si, q_rot, so, pos, base, freq);
  return hipGetLastError();
}

}  // namespace mla
