// Rotary embedding of the decoupled rope part (PaperTrace "02 · DeepSeek-V2
// analysis", section 1.3, eq. 14-15): coordinate pairs (2i, 2i+1) are rotated
// by pos * base^(-2i/d_r) (CSDN "DeepSeek-V3 structure and engineering",
// section 2(3)). Angles, cos and sin are fp64 (at position 131071 an fp32
// angle is off by up to 0.008 rad); the rotation is fp64, rounded to fp32 and
// then (for bf16 storage) to bf16.
#include "mla_device.h"
#include "mla_internal.h"
#include "rope_body.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxHalf = 128;

template <bool BF16>
__global__ __launch_bounds__(kRope64Threads) void rope64_kernel(const void* x_in, VecStrides si,
                                                                void* x_out, VecStrides so,
                                                                const int32_t* pos, int n_heads,
                                                                double base, const double* freq) {
  __shared__ __attribute__((aligned(16))) char cs[32 * 2 * sizeof(double)];
  rope64_block<BF16>(blockIdx.x, blockIdx.y, (lds_char*)cs, x_in, si, x_out, so, pos, n_heads,
                     base, freq);
}

// any d_r and strides: one workgroup per token, one thread per pair
template <bool BF16>
__global__ __launch_bounds__(kThreads) void rope_kernel(const void* x_in, VecStrides si,
                                                        void* x_out, VecStrides so,
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
  for (int e = threadIdx.x; e < n_heads * half; e += kThreads) {
    const int h = e / half, i = e % half;
    const size_t a = (size_t)n * si.tok + (size_t)h * si.head + 2 * i;
    const size_t o = (size_t)n * so.tok + (size_t)h * so.head + 2 * i;
    double x0, x1;
    if (BF16) {
      x0 = bf2f(((const uint16_t*)x_in)[a]);
      x1 = bf2f(((const uint16_t*)x_in)[a + 1]);
    } else {
      x0 = ((const float*)x_in)[a];
      x1 = ((const float*)x_in)[a + 1];
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

hipError_t launch_rope(const void* x_in, VecStrides si, void* x_out, VecStrides so, int bf16,
                       const int32_t* pos, int n_tok, int n_heads, int d_r, double base,
                       const double* theta, hipStream_t s) {
  // every vector start 16-byte aligned: the vectorised d_r = 64 kernel
  const long elt = bf16 ? 2 : 4;
  const bool aligned = (((uintptr_t)x_in | (uintptr_t)x_out) & 15) == 0 &&
                       ((si.tok | si.head | so.tok | so.head) * elt) % 16 == 0;
  if (d_r == 64 && aligned) {
    const dim3 grid(n_tok, (n_heads + kRope64Heads - 1) / kRope64Heads);
    if (bf16)
      hipLaunchKernelGGL(rope64_kernel<true>, grid, dim3(kThreads), 0, s, x_in, si, x_out, so, pos,
                         n_heads, base, theta);
    else
      hipLaunchKernelGGL(rope64_kernel<false>, grid, dim3(kThreads), 0, s, x_in, si, x_out, so,
                         pos, n_heads, base, theta);
    return hipGetLastError();
  }
  if (bf16)
    hipLaunchKernelGGL(rope_kernel<true>, dim3(n_tok), dim3(kThreads), 0, s, x_in, si, x_out, so,
                       pos, n_heads, d_r, base, theta);
  else
    hipLaunchKernelGGL(rope_kernel<false>, dim3(n_tok), dim3(kThreads), 0, s, x_in, si, x_out, so,
                       pos, n_heads, d_r, base, theta);
  return hipGetLastError();
}

}  // namespace mla
