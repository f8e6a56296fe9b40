// Log-sum-exp merge of split-KV partials.
//
// Each split k of a row left (m_k, l_k, U_k): its max logit (log2 units), the
// sum of 2^(z - m_k) and the unnormalised latent aggregate. With
// m* = max_k m_k and w_k = 2^(m_k - m*):
//   u = (sum_k w_k U_k) / (sum_k w_k l_k),  lse = (m* + log2 sum_k w_k l_k) ln 2.
// Only splits k < ceil(L_b / split_tokens) exist (units past the end of a
// sequence write nothing); a row that sees no token of an existing split
// carries (-inf, 0, 0) there and gets weight 0. The sums run over k in
// increasing order starting from k = 0, so a single split reproduces the
// split kernel's own U / l bit for bit. Out-of-range lengths give NaN.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 128;   // 4 latent values per thread
constexpr int kMaxSplitsLds = 1024;

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  __shared__ float wsh[kMaxSplitsLds];
  __shared__ float red[kThreads / 64];
  const int row = blockIdx.x;       // b*R + r
  if (row >= p.rows) return;
  const int b = row / p.R, r = row % p.R;
  const int tid = threadIdx.x;
  const int L = p.seq_lens[b];
  const bool bad = (L < p.T) || (L > p.max_seq_len) || ((L + kPage - 1) / kPage > p.max_pages);
  if (bad) {
    const size_t o = (size_t)row * kDc + 4 * tid;
    for (int i = 0; i < 4; ++i) {
      if (p.out_bf16) ((uint16_t*)p.out)[o + i] = 0x7fc0;
      else ((float*)p.out)[o + i] = __builtin_nanf("");
    }
    if (p.lse && tid == 0) p.lse[row] = __builtin_nanf("");
    return;
  }
  const int nsp = p.n_split;                                   // split stride in memory
  const int ns = min(nsp, (L + p.split_tokens - 1) / p.split_tokens);
  auto ml = [&](int k) -> const float* {
    return p.part_ml + (((size_t)b * nsp + k) * p.R + r) * 2;
  };
  // m* = max over splits (each thread scans a strided subset, then a fixed tree)
  float mx = -INFINITY;
  for (int k = tid; k < ns; k += kThreads) mx = fmaxf(mx, ml(k)[0]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = red[0];
  for (int i = 1; i < kThreads / 64; ++i) mx = fmaxf(mx, red[i]);
  // split weights 2^(m_k - m*) into LDS
  for (int k = tid; k < ns && k < kMaxSplitsLds; k += kThreads) {
    const float mk = ml(k)[0];
    wsh[k] = (mk == -INFINITY) ? 0.f : exp2f(mk - mx);
  }
  __syncthreads();
  float lsum = wsh[0] * ml(0)[1];
  for (int k = 1; k < ns; ++k) lsum = fmaf(wsh[k], ml(k)[1], lsum);

  const int d = 4 * tid;
  const f32x4_t* pu = (const f32x4_t*)(p.part_u + (((size_t)b * nsp) * p.R + r) * kDc + d);
  const size_t kstride = (size_t)p.R * kDc / 4;
  f32x4_t acc = wsh[0] * pu[0];
  for (int k = 1; k < ns; ++k) {
    const f32x4_t v = pu[k * kstride];
    const float wk = wsh[k];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(wk, v[i], acc[i]);
  }
  const size_t o = (size_t)row * kDc + d;
  if (p.out_bf16) {
    uint16_t* out = (uint16_t*)p.out + o;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = f2bf(acc[i] / lsum);
  } else {
    float* out = (float*)p.out + o;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = acc[i] / lsum;
  }
  if (p.lse && tid == 0) p.lse[row] = (mx + log2f(lsum)) * kLn2;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.n_split > kMaxSplitsLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(p.rows), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
