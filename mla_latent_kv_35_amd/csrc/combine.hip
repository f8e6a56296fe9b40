// Log-sum-exp merge of split-KV partials.
//
// Each split k of a row left (m_k, l_k, U_k): its max logit (log2 units), the
// sum of 2^(z - m_k) and the unnormalised latent aggregate. With
// m* = max_k m_k and w_k = 2^(m_k - m*):
//   u = (sum_k w_k U_k) / (sum_k w_k l_k),  lse = (m* + log2 sum_k w_k l_k) ln 2.
// Only splits k < ceil(L_b / split_tokens) exist (units past the end of a
// sequence write nothing); a row that sees no token of an existing split
// carries (-inf, 0, 0) there and gets weight 0. The latent sums run over k
// in increasing order starting from k = 0 with w_0 * U_0, and the terms of
// dead splits in the l sum are +0, so a single split reproduces the split
// kernel's own U / l bit for bit. Out-of-range lengths give NaN.
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

// n_split <= 64: one wave per row, four rows per workgroup. Lane k holds
// split k's (m, l); the maximum and the weighted row sum are wave
// reductions. Lane i owns latent values 8i..8i+7 and accumulates the splits
// in increasing k, loading them 8 splits at a time so that 16 loads are in
// flight; w_0 = 1 for the first live split with the maximum, so one live
// split still gives U / l exactly.
constexpr int kWaveRows = 4;

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(64 * kWaveRows) void combine_wave_kernel(CombineParams p) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaveRows + wv);  // b*R + r
  if (row >= p.rows) return;                      // the whole wave leaves; no barrier below
  const int b = row / p.R, r = row % p.R;
  const int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
  const size_t o = (size_t)row * kDc + 8 * lane;
  const bool bad = (L < p.T) || (L > p.max_seq_len) || ((L + kPage - 1) / kPage > p.max_pages);
  if (bad) {
    if (p.out_bf16) {
      *(u32x4_t*)((uint16_t*)p.out + o) = (u32x4_t){0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
    } else {
      const float nan = __builtin_nanf("");
      *(f32x4_t*)((float*)p.out + o) = (f32x4_t){nan, nan, nan, nan};
      *(f32x4_t*)((float*)p.out + o + 4) = (f32x4_t){nan, nan, nan, nan};
    }
    if (p.lse && lane == 0) p.lse[row] = __builtin_nanf("");
    return;
  }
  const int nsp = p.n_split;                                   // split stride in memory
  const int ns = min(nsp, (L + p.split_tokens - 1) / p.split_tokens);
  float mk = -INFINITY, lk = 0.f;
  if (lane < ns) {
    const float* ml = p.part_ml + (((size_t)b * nsp + lane) * p.R + r) * 2;
    mk = ml[0];
    lk = ml[1];
  }
  const float mx = wave_max64(mk);
  const float wk = (mk == -INFINITY) ? 0.f : exp2f(mk - mx);
  const float lsum = wave_sum64(wk * lk);
  const float* pu = p.part_u + (((size_t)b * nsp) * p.R + r) * kDc + 8 * lane;
  const size_t kstride = (size_t)p.R * kDc;
  // split 0 is always live (L >= T >= 1)
  // split weights come from the lane that holds them (k is wave-uniform)
  const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), 0));
  f32x4_t acc0 = w0 * *(const f32x4_t*)pu;
  f32x4_t acc1 = w0 * *(const f32x4_t*)(pu + 4);
  for (int k0 = 1; k0 < ns; k0 += 8) {
    // loads of splits past the last live one repeat it (valid memory) and are
    // not accumulated
    f32x4_t v0[8], v1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const size_t off = (size_t)min(k0 + q, ns - 1) * kstride;
      v0[q] = *(const f32x4_t*)(pu + off);
      v1[q] = *(const f32x4_t*)(pu + off + 4);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (k0 + q < ns) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), k0 + q));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0[i] = fmaf(w, v0[q][i], acc0[i]);
          acc1[i] = fmaf(w, v1[q][i], acc1[i]);
        }
      }
    }
  }
  if (p.out_bf16) {
    u32x4_t ov;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ov[i] = pack_bf16x2(acc0[2 * i] / lsum, acc0[2 * i + 1] / lsum);
      ov[i + 2] = pack_bf16x2(acc1[2 * i] / lsum, acc1[2 * i + 1] / lsum);
    }
    *(u32x4_t*)((uint16_t*)p.out + o) = ov;
  } else {
    f32x4_t a, c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = acc0[i] / lsum;
      c[i] = acc1[i] / lsum;
    }
    *(f32x4_t*)((float*)p.out + o) = a;
    *(f32x4_t*)((float*)p.out + o + 4) = c;
  }
  if (p.lse && lane == 0) p.lse[row] = (mx + log2f(lsum)) * kLn2;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.n_split > kMaxSplitsLds) return hipErrorInvalidValue;
  if (p.n_split <= 64)
    hipLaunchKernelGGL(combine_wave_kernel, dim3((p.rows + kWaveRows - 1) / kWaveRows),
                       dim3(64 * kWaveRows), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel, dim3(p.rows), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
