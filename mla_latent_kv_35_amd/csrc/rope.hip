// Rotary embedding of the decoupled rope part (PaperTrace "02 · DeepSeek-V2
// analysis", section 1.3, eq. 14-15): coordinate pairs (2i, 2i+1) are rotated
// by pos * base^(-2i/d_r) (CSDN "DeepSeek-V3 structure and engineering",
// section 2(3)). Angles, cos and sin are fp64 (at position 131071 an fp32
// angle is off by up to 0.008 rad); the rotation is fp64, rounded to fp32 and
// then (for bf16 storage) to bf16.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxHalf = 128;

// d_r = 64: one workgroup per (token, 32 heads). Lanes 0..31 build the 32
// (cos, sin) pairs of the token's position in fp64 while every thread's
// 16-byte slice of the 32 rows is already in flight; each thread then
// rotates its 4 (bf16) or 2 x 2 (fp32) pairs. In place is allowed: a thread
// reads and writes only its own slice.
constexpr int kHeadsPerBlock = 32;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void rope64_kernel(const void* x_in, void* x_out,
                                                          const int32_t* pos, int n_heads,
                                                          double base, const double* freq) {
  __shared__ double cs[32][2];
  const int n = blockIdx.x;
  const int h0 = blockIdx.y * kHeadsPerBlock;
  const int tid = threadIdx.x;
  // each 64-element row is 8 (bf16) or 16 (fp32) slices of 16 bytes
  constexpr int kSlices = BF16 ? 8 : 16;
  constexpr int kPerThread = kHeadsPerBlock * kSlices / kThreads;   // 1 or 2
  u32x4_t v[kPerThread];
  size_t off[kPerThread];
  bool ok[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = tid + q * kThreads;
    const int h = h0 + e / kSlices, c = e % kSlices;
    ok[q] = h < n_heads;
    off[q] = (((size_t)n * n_heads + h) * 64) * (BF16 ? 2 : 4) + (size_t)c * 16;
    if (ok[q]) v[q] = *(const u32x4_t*)((const char*)x_in + off[q]);
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
    const int c = (tid + q * kThreads) % kSlices;
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

template <bool BF16>
__global__ __launch_bounds__(kThreads) void rope_kernel(const void* x_in, void* x_out,
                                                        const int32_t* pos, int n_heads, int d_r,
                                                        double base, const double* freq) {
  __shared__ double cs[kMaxHalf][2];
  const int n = blockIdx.x;
  const int half = d_r / 2;
  const double pn = (double)pos[n];
  for (int i = threadIdx.x; i < half; i += kThreads) {
    const double theta = freq ? freq[i] : pow(base, -2.0 * (double)i / (double)d_r);
    double s, c;
    sincos(pn * theta, &s, &c);
    cs[i][0] = c;
    cs[i][1] = s;
  }
  __syncthreads();
  const size_t row0 = (size_t)n * n_heads * d_r;
  for (int e = threadIdx.x; e < n_heads * half; e += kThreads) {
    const int h = e / half, i = e % half;
    const size_t o = row0 + (size_t)h * d_r + 2 * i;
    double x0, x1;
    if (BF16) {
      x0 = bf2f(((const uint16_t*)x_in)[o]);
      x1 = bf2f(((const uint16_t*)x_in)[o + 1]);
    } else {
      x0 = ((const float*)x_in)[o];
      x1 = ((const float*)x_in)[o + 1];
    }
    const double c = cs[i][0], s = cs[i][1];
    const float y0 = (float)(x0 * c - x1 * s);
    const float y1 = (float)(x0 * s + x1 * c);
    if (BF16) {
      ((uint16_t*)x_out)[o] = f2bf(y0);
      ((uint16_t*)x_out)[o + 1] = f2bf(y1);
    } else {
      ((float*)x_out)[o] = y0;
      ((float*)x_out)[o + 1] = y1;
    }
  }
}

}  // namespace

hipError_t launch_rope(const void* x_in, void* x_out, int bf16, const int32_t* pos, int n_tok,
                       int n_heads, int d_r, double base, const double* theta, hipStream_t s) {
  if (d_r == 64 && (((uintptr_t)x_in | (uintptr_t)x_out) & 15) == 0) {
    const dim3 grid(n_tok, (n_heads + kHeadsPerBlock - 1) / kHeadsPerBlock);
    if (bf16)
      hipLaunchKernelGGL(rope64_kernel<true>, grid, dim3(kThreads), 0, s, x_in, x_out, pos, n_heads,
                         base, theta);
    else
      hipLaunchKernelGGL(rope64_kernel<false>, grid, dim3(kThreads), 0, s, x_in, x_out, pos,
                         n_heads, base, theta);
    return hipGetLastError();
  }
  if (bf16)
    hipLaunchKernelGGL(rope_kernel<true>, dim3(n_tok), dim3(kThreads), 0, s, x_in, x_out, pos,
                       n_heads, d_r, base, theta);
  else
    hipLaunchKernelGGL(rope_kernel<false>, dim3(n_tok), dim3(kThreads), 0, s, x_in, x_out, pos,
                       n_heads, d_r, base, theta);
  return hipGetLastError();
}

}  // namespace mla
