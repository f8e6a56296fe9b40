// Paged absorbed-MLA decode for fp32 caches, fp32 arithmetic end to end.
//
// One workgroup per (sequence b, split k, query row r). Tokens of the split
// are taken 256 at a time: each thread forms one token's score
// z = (q_lat . c_s + q_rope . k^R_s) * scale (PaperTrace "02 · DeepSeek-V2
// analysis", eq. 18 over the 576 cached elements) in fp32 FMA, the chunk's
// max and exponentials update an online softmax, and each thread accumulates
// two latent dimensions of u = sum_s a_s c_s (section 6.1) over the chunk's
// tokens in increasing token order. Reductions use a fixed tree, so results
// are deterministic.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

__global__ __launch_bounds__(kThreads) void decode_simple_f32_kernel(DecodeParams p) {
  __shared__ float q[kDc + kDr];
  __shared__ float pr[kThreads];
  __shared__ int tokpage[kThreads];
  __shared__ float red[kThreads / 64];

  const int r = blockIdx.x % p.R;
  const int bk = blockIdx.x / p.R;
  const int k = bk % p.n_split;
  const int b = bk / p.n_split;
  const int tid = threadIdx.x;

  const int L = p.seq_lens[b];
  bool bad = (L < p.T) || (L > p.max_seq_len) || ((L + kPage - 1) / kPage > p.max_pages);
  const int tok0 = k * p.split_tokens;
  const int tok1 = min(tok0 + p.split_tokens, L);
  const int t = r / p.H;
  const int lim = min(L - p.T + t + 1, tok1);  // visible tokens: s < lim
  const int32_t* btrow = p.block_table + (size_t)b * p.max_pages;
  if (!bad && tok0 >= tok1) return;   // split past the end of the sequence: no partial
  if (!bad) {
    bool lb = false;
    for (int j = tok0 / kPage + tid; j < (tok1 + kPage - 1) / kPage; j += kThreads) {
      const int id = btrow[j];
      lb |= (id < 0) || (id >= p.n_pages);
    }
    bad = __syncthreads_or(lb);
  }

  float m = -INFINITY, l = 0.f, u0 = 0.f, u1 = 0.f;
  if (bad) {
    m = l = u0 = u1 = __builtin_nanf("");
  } else {
    const float* ql = (const float*)p.q_lat + ((size_t)b * p.R + r) * kDc;
    const float* qr = (const float*)p.q_rope + ((size_t)b * p.R + r) * kDr;
    for (int i = tid; i < kDc; i += kThreads) q[i] = ql[i];
    if (tid < kDr) q[kDc + tid] = qr[tid];
    __syncthreads();
    const float* ckv = (const float*)p.ckv;
    const float* kr = (const float*)p.kr;
    for (int c0 = tok0; c0 < lim; c0 += kThreads) {
      const int s = c0 + tid;
      float z = -INFINITY;
      int page = 0;
      if (s < lim) {
        page = btrow[s / kPage];
        const float* cs = ckv + ((size_t)page * kPage + s % kPage) * kDc;
        const float* ks = kr + ((size_t)page * kPage + s % kPage) * kDr;
        float acc = 0.f;
        for (int d = 0; d < kDc; ++d) acc = fmaf(q[d], cs[d], acc);
        float accr = 0.f;
        for (int d = 0; d < kDr; ++d) accr = fmaf(q[kDc + d], ks[d], accr);
        z = (acc + accr) * p.scale_log2;
      }
      const float cmax = block_reduce(z, red, true);
      const float mnew = fmaxf(m, cmax);
      const float alpha = exp2f(m - mnew);   // m = -inf on the first chunk -> 0
      const float e = (s < lim) ? exp2f(z - mnew) : 0.f;
      pr[tid] = e;
      tokpage[tid] = page;
      const float esum = block_reduce(e, red, false);  // syncs: pr visible
      l = l * alpha + esum;
      u0 *= alpha;
      u1 *= alpha;
      const int n = min(kThreads, lim - c0);
      for (int j = 0; j < n; ++j) {
        const int sj = c0 + j;
        const float* cs = ckv + ((size_t)tokpage[j] * kPage + sj % kPage) * kDc;
        u0 = fmaf(pr[j], cs[tid], u0);
        u1 = fmaf(pr[j], cs[tid + kThreads], u1);
      }
      m = mnew;
      __syncthreads();
    }
  }

  if (p.n_split == 1) {
    const size_t o = ((size_t)b * p.R + r) * kDc;
    ((float*)p.out)[o + tid] = u0 / l;
    ((float*)p.out)[o + tid + kThreads] = u1 / l;
    if (p.lse && tid == 0) p.lse[(size_t)b * p.R + r] = (m + log2f(l)) * kLn2;
  } else {
    const size_t base = ((size_t)b * p.n_split + k) * p.R + r;
    p.part_u[base * kDc + tid] = u0;
    p.part_u[base * kDc + tid + kThreads] = u1;
    if (tid == 0) {
      p.part_ml[base * 2] = m;
      p.part_ml[base * 2 + 1] = l;
    }
  }
}

}  // namespace

hipError_t launch_decode_simple_f32(const DecodeParams& p, hipStream_t s) {
  const size_t nblk = (size_t)p.B * p.n_split * p.R;
  hipLaunchKernelGGL(decode_simple_f32_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
