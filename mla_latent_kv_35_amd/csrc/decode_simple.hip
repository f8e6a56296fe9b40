// Paged absorbed-MLA decode for fp32 caches, fp32 arithmetic end to end.
//
// One workgroup of 4 waves per (sequence b, split k, query row r). The
// split's tokens go to the waves in batches of kBatch (wave w takes batches
// w, w + 4, ...). For each token a wave reads the cached row coalesced (lane i
// holds latent values 8i..8i+7 and rope value i), forms the score
// z = (q_lat . c_s + q_rope . k^R_s) * scale (PaperTrace "02 · DeepSeek-V2
// analysis", eq. 18 over the 576 cached elements) by a fixed butterfly sum,
// and folds it into the wave's online softmax; the latent aggregate
// u = sum_s a_s c_s (section 6.1) reuses the row already in registers. The
// four waves' (max, sum, aggregate) are merged by log-sum-exp in a fixed
// order, so results are deterministic. All loads of a batch are issued
// before any of them is used.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBatch = 8;

__device__ __forceinline__ float wave_sum_all(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kThreads) void decode_simple_f32_kernel(DecodeParams p) {
  __shared__ float wm[kWaves], wl[kWaves];
  __shared__ __attribute__((aligned(16))) float wu[kWaves][kDc];

  const int r = blockIdx.x % p.R;
  const int bk = blockIdx.x / p.R;
  const int k = bk % p.n_split;
  const int b = bk / p.n_split;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

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

  float m = -INFINITY, l = 0.f, u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = 0.f;
  if (!bad) {
    const size_t qi = (size_t)b * p.R + r;   // query row
    const float* qrow = (const float*)p.q_lat + qi * p.q_lat_stride + 8 * lane;
    const f32x4_t q0 = *(const f32x4_t*)qrow, q1 = *(const f32x4_t*)(qrow + 4);
    const float qr = ((const float*)p.q_rope)[qi * p.q_rope_stride + lane];
    const float* ckv = (const float*)p.ckv;
    const float* kr = (const float*)p.kr;
    for (int c0 = tok0 + kBatch * w; c0 < lim; c0 += kBatch * kWaves) {
      f32x4_t c[kBatch][2];
      float cr[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int s = min(c0 + j, lim - 1);   // past the limit: reread the last row, masked below
        const size_t row = (size_t)btrow[s / kPage] * kPage + s % kPage;
        c[j][0] = *(const f32x4_t*)(ckv + row * kDc + 8 * lane);
        c[j][1] = *(const f32x4_t*)(ckv + row * kDc + 8 * lane + 4);
        cr[j] = kr[row * kDr + lane];
      }
      float z[kBatch];
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        float acc = qr * cr[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(q0[i], c[j][0][i], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(q1[i], c[j][1][i], acc);
        z[j] = (c0 + j < lim) ? wave_sum_all(acc) * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, z[j]);
      }
      const float mnew = fmaxf(m, mt);                   // finite: token c0 is visible
      const float alpha = exp2f(m - mnew);               // m = -inf on the first batch -> 0
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] *= alpha;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float e = exp2f(z[j] - mnew);              // 0 past the limit
        l += e;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u[i] = fmaf(e, c[j][0][i], u[i]);
          u[4 + i] = fmaf(e, c[j][1][i], u[4 + i]);
        }
      }
      m = mnew;
    }
  }
  // merge the waves: M = max m_w, weights 2^(m_w - M) (0 for a wave that saw no token)
  if (lane == 0) {
    wm[w] = m;
    wl[w] = l;
  }
  *(f32x4_t*)&wu[w][8 * lane] = (f32x4_t){u[0], u[1], u[2], u[3]};
  *(f32x4_t*)&wu[w][8 * lane + 4] = (f32x4_t){u[4], u[5], u[6], u[7]};
  __syncthreads();
  float M = wm[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) M = fmaxf(M, wm[i]);
  float cw[kWaves], lsum = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    cw[i] = (wm[i] == -INFINITY) ? 0.f : exp2f(wm[i] - M);
    lsum = fmaf(cw[i], wl[i], lsum);
  }
  float U[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) acc = fmaf(cw[i], wu[i][tid + d * kThreads], acc);
    U[d] = acc;
  }
  if (bad) M = lsum = U[0] = U[1] = __builtin_nanf("");

  if (p.n_split == 1) {
    const size_t o = ((size_t)b * p.R + r) * kDc;
    ((float*)p.out)[o + tid] = U[0] / lsum;
    ((float*)p.out)[o + tid + kThreads] = U[1] / lsum;
    if (p.lse && tid == 0) p.lse[(size_t)b * p.R + r] = (M + log2f(lsum)) * kLn2;
  } else {
    const size_t base = ((size_t)b * p.n_split + k) * p.R + r;
    float* const pu = (float*)p.part_u + base * kDc;   // fp32 caches keep fp32 partials
    pu[tid] = U[0];
    pu[tid + kThreads] = U[1];
    if (tid == 0) {
      p.part_ml[base * 2] = M;
      p.part_ml[base * 2 + 1] = lsum;
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
