// Rotary embedding body for d_r = 64 shared by the rope kernel and the fused
// absorb + rope kernel (PaperTrace "02 · DeepSeek-V2 analysis", section 1.3,
// eq. 14-15; pairs (2i, 2i+1), CSDN "DeepSeek-V3 structure and engineering",
// section 2(3)). Angles, cos and sin are fp64; the rotation is fp64, rounded
// to fp32 and then (for bf16 storage) to bf16.
#pragma once

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kRope64Threads = 256;
constexpr int kRope64Heads = 32;

// d_r = 64: one workgroup per (token, 32 heads). Lanes 0..31 build the 32
// (cos, sin) pairs of the token's position in fp64 while every thread's
// 16-byte slice of the 32 rows is already in flight; each thread then
// rotates its 4 (bf16) or 2 x 2 (fp32) pairs. In place (same memory, same
// strides) is allowed: a thread reads and writes only its own slice. Vector
// (n, h) of x_in starts at n * si.tok + h * si.head elements, of x_out at
// n * so.tok + h * so.head; each start is 16-byte aligned.

// cs_lds: 512 bytes of LDS for the token's (cos, sin) table
template <bool BF16>
__device__ __forceinline__ void rope64_block(int n, int hblk, lds_char* cs_lds, const void* x_in,
                                             VecStrides si, void* x_out, VecStrides so,
                                             const int32_t* pos, int n_heads, double base,
                                             const double* freq) {
  MLA_LDS double(*cs)[2] = (MLA_LDS double(*)[2])cs_lds;
  const int h0 = hblk * kRope64Heads;
  const int tid = threadIdx.x;
  // each 64-element row is 8 (bf16) or 16 (fp32) slices of 16 bytes
  constexpr int kSlices = BF16 ? 8 : 16;
  constexpr int kPerThread = kRope64Heads * kSlices / kRope64Threads;   // 1 or 2
  constexpr int kElt = BF16 ? 2 : 4;
  u32x4_t v[kPerThread];
  size_t off[kPerThread];   // byte offset of this thread's slice in x_out
  bool ok[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = tid + q * kRope64Threads;
    const int h = h0 + e / kSlices, c = e % kSlices;
    ok[q] = h < n_heads;
    const size_t in = ((size_t)n * si.tok + (size_t)h * si.head) * kElt + (size_t)c * 16;
    off[q] = ((size_t)n * so.tok + (size_t)h * so.head) * kElt + (size_t)c * 16;
    if (ok[q]) v[q] = *(const u32x4_t*)((const char*)x_in + in);
  }
  if (tid < 32) {
    const double theta = freq ? freq[tid] : pow(base, -2.0 * (double)tid / 64.0);
    double sn, cn;
    sincos((double)pos[n] * theta, &sn, &cn);
    cs[tid][0] = cn;
    cs[tid][1] = sn;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    if (!ok[q]) continue;
    const int c = (tid + q * kRope64Threads) % kSlices;
    u32x4_t r;
    if constexpr (BF16) {
      // 8 bf16 = pairs 4c .. 4c+3
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double x0 = bf2f(v[q][k] & 0xffff), x1 = bf2f(v[q][k] >> 16);
        const double cn = cs[4 * c + k][0], sn = cs[4 * c + k][1];
        const float y0 = (float)(x0 * cn - x1 * sn);
        const float y1 = (float)(x0 * sn + x1 * cn);
        r[k] = (uint32_t)f2bf(y0) | ((uint32_t)f2bf(y1) << 16);
      }
    } else {
      // 4 fp32 = pairs 2c, 2c+1
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const double x0 = __uint_as_float(v[q][2 * k]), x1 = __uint_as_float(v[q][2 * k + 1]);
        const double cn = cs[2 * c + k][0], sn = cs[2 * c + k][1];
        r[2 * k] = __float_as_uint((float)(x0 * cn - x1 * sn));
        r[2 * k + 1] = __float_as_uint((float)(x0 * sn + x1 * cn));
      }
    }
    *(u32x4_t*)((char*)x_out + off[q]) = r;
  }
}

}  // namespace mla
