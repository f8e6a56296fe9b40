// Log-sum-exp merge of split-KV partials.
//
// Each split k of a row left (m_k, l_k, U_k): its max logit (log2 units), the
// sum of 2^(z - m_k) and the unnormalised latent aggregate. With
// m* = max_k m_k and w_k = 2^(m_k - m*):
//   u = (sum_k w_k U_k) / (sum_k w_k l_k),  lse = (m* + log2 sum_k w_k l_k) ln 2.
// When the output is bf16 the splits store u_k = U_k / l_k in bf16 instead
// (half the bytes), and u = sum_k a_k u_k with a_k = w_k l_k / sum_j w_j l_j.
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
  const size_t e0 = (((size_t)b * nsp) * p.R + r) * kDc + d;   // element of split 0
  const size_t kstride = (size_t)p.R * kDc;
  // split k's 4 values (bf16 partials: l_k u_k, so that acc / lsum is u)
  auto part = [&](int k) -> f32x4_t {
    if (!p.part_bf16) return *(const f32x4_t*)((const float*)p.part_u + e0 + k * kstride);
    const u32x2_t h = *(const u32x2_t*)((const uint16_t*)p.part_u + e0 + k * kstride);
    const float lk = ml(k)[1];
    return (f32x4_t){bf2f(h[0] & 0xffff), bf2f(h[0] >> 16), bf2f(h[1] & 0xffff), bf2f(h[1] >> 16)} * lk;
  };
  f32x4_t acc = wsh[0] * part(0);
  for (int k = 1; k < ns; ++k) {
    const f32x4_t v = part(k);
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

// Merge of NR rows by one wave: lane i returns u for latent values 8i..8i+7
// of each row (NaN for a sequence whose length or page count is out of
// range) and each row's lse. The rows must be wave-uniform. Every load of
// the first Q splits (their (m, l) and U, from slots clamped to the
// allocated n_split; Q = 4 when no more are allocated) is issued before the
// sequence length is known, so one memory round trip serves all NR rows;
// splits past the live count are then masked out and never accumulated. The
// sum runs over k in increasing order whatever Q is. PB: the partials are
// bf16 u_k (16 bytes per lane and split) weighted by a_k = w_k l_k / sum.
__device__ __forceinline__ void unpack_bf16x8(const u32x4_t& h, f32x4_t& lo, f32x4_t& hi) {
  lo = (f32x4_t){bf2f(h[0] & 0xffff), bf2f(h[0] >> 16), bf2f(h[1] & 0xffff), bf2f(h[1] >> 16)};
  hi = (f32x4_t){bf2f(h[2] & 0xffff), bf2f(h[2] >> 16), bf2f(h[3] & 0xffff), bf2f(h[3] >> 16)};
}

template <int NR, int Q, bool PB>
__device__ __forceinline__ void combine_rows(const CombineParams& p, const int (&row)[NR], int lane,
                                             float (&u)[NR][8], float (&lse_out)[NR]) {
  const int nsp = p.n_split;                                   // split stride in memory
  const size_t kstride = (size_t)p.R * kDc;
  int Ls[NR];
  float mk[NR], lk[NR];
  f32x4_t v0[NR][Q], v1[NR][Q];
  u32x4_t vb[NR][Q];
  const float* pu[NR];
  const uint16_t* pb[NR];
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    const int b = row[t] / p.R, r = row[t] % p.R;
    Ls[t] = p.seq_lens[b];
    const float* ml = p.part_ml + (((size_t)b * nsp + min(lane, nsp - 1)) * p.R + r) * 2;
    mk[t] = ml[0];
    lk[t] = ml[1];
    const size_t e0 = (((size_t)b * nsp) * p.R + r) * kDc + 8 * lane;
    pu[t] = (const float*)p.part_u + e0;
    pb[t] = (const uint16_t*)p.part_u + e0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const size_t off = (size_t)min(q, nsp - 1) * kstride;
      if constexpr (PB) {
        vb[t][q] = *(const u32x4_t*)(pb[t] + off);
      } else {
        v0[t][q] = *(const f32x4_t*)(pu[t] + off);
        v1[t][q] = *(const f32x4_t*)(pu[t] + off + 4);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    const int L = __builtin_amdgcn_readfirstlane(Ls[t]);
    const bool bad = (L < p.T) || (L > p.max_seq_len) || ((L + kPage - 1) / kPage > p.max_pages);
    if (bad) {
#pragma unroll
      for (int i = 0; i < 8; ++i) u[t][i] = __builtin_nanf("");
      lse_out[t] = __builtin_nanf("");
      continue;
    }
    const int ns = min(nsp, (L + p.split_tokens - 1) / p.split_tokens);
    const float m_l = lane < ns ? mk[t] : -INFINITY;
    const float l_l = lane < ns ? lk[t] : 0.f;
    const float mx = wave_max64(m_l);
    const float wk = (m_l == -INFINITY) ? 0.f : exp2f(m_l - mx);
    const float lsum = wave_sum64(wk * l_l);
    // split 0 is always live (L >= T >= 1); the split weights come from the
    // lane that holds them (k is wave-uniform); bf16 partials take
    // a_k = w_k l_k / lsum (1 for a single live split)
    const float wa = PB ? wk * l_l / lsum : wk;
    if constexpr (PB) {
#pragma unroll
      for (int q = 0; q < Q; ++q) unpack_bf16x8(vb[t][q], v0[t][q], v1[t][q]);
    }
    const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wa), 0));
    f32x4_t acc0 = w0 * v0[t][0];
    f32x4_t acc1 = w0 * v1[t][0];
#pragma unroll
    for (int q = 1; q < Q; ++q) {
      if (q < ns) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wa), q));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0[i] = fmaf(w, v0[t][q][i], acc0[i]);
          acc1[i] = fmaf(w, v1[t][q][i], acc1[i]);
        }
      }
    }
    for (int k0 = Q; k0 < ns; k0 += 8) {
      f32x4_t c0[8], c1[8];
      u32x4_t cb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const size_t off = (size_t)min(k0 + q, ns - 1) * kstride;
        if constexpr (PB) {
          cb[q] = *(const u32x4_t*)(pb[t] + off);
        } else {
          c0[q] = *(const f32x4_t*)(pu[t] + off);
          c1[q] = *(const f32x4_t*)(pu[t] + off + 4);
        }
      }
      if constexpr (PB) {
#pragma unroll
        for (int q = 0; q < 8; ++q) unpack_bf16x8(cb[q], c0[q], c1[q]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (k0 + q < ns) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wa), k0 + q));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc0[i] = fmaf(w, c0[q][i], acc0[i]);
            acc1[i] = fmaf(w, c1[q][i], acc1[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u[t][i] = PB ? acc0[i] : acc0[i] / lsum;
      u[t][4 + i] = PB ? acc1[i] : acc1[i] / lsum;
    }
    lse_out[t] = (mx + log2f(lsum)) * kLn2;
  }
}

// combine_rows with the partial format and the number of up-front loads
// (4 when no more splits are allocated) chosen at run time
template <int NR>
__device__ __forceinline__ void combine_rows_any(const CombineParams& p, const int (&row)[NR], int lane,
                                                 float (&u)[NR][8], float (&lse_out)[NR]) {
  if (p.part_bf16) {
    if (p.n_split <= 4) combine_rows<NR, 4, true>(p, row, lane, u, lse_out);
    else combine_rows<NR, 8, true>(p, row, lane, u, lse_out);
  } else {
    if (p.n_split <= 4) combine_rows<NR, 4, false>(p, row, lane, u, lse_out);
    else combine_rows<NR, 8, false>(p, row, lane, u, lse_out);
  }
}

__device__ __forceinline__ void store_u_row(const CombineParams& p, int row, int lane,
                                            const float (&u)[8], float lse) {
  const size_t o = (size_t)row * kDc + 8 * lane;
  if (p.out_bf16) {
    u32x4_t ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = pack_bf16x2(u[2 * i], u[2 * i + 1]);
    *(u32x4_t*)((uint16_t*)p.out + o) = ov;
  } else {
    *(f32x4_t*)((float*)p.out + o) = (f32x4_t){u[0], u[1], u[2], u[3]};
    *(f32x4_t*)((float*)p.out + o + 4) = (f32x4_t){u[4], u[5], u[6], u[7]};
  }
  if (p.lse && lane == 0) p.lse[row] = lse;
}

__global__ __launch_bounds__(64 * kWaveRows) void combine_wave_kernel(CombineParams p) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // block b' of the rows runs on XCD b' / per_xcd (the hardware deals blocks
  // to the 8 XCDs round-robin), the XCD whose split units wrote those rows'
  // partials when the decode placed them the same way
  const int per_xcd = gridDim.x / kNumXcd;
  const int lb = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
  const int row = __builtin_amdgcn_readfirstlane(lb * kWaveRows + wv);  // b*R + r
  if (row >= p.rows) return;                      // the whole wave leaves; no barrier below
  const int rows[1] = {row};
  float u[1][8], lse[1];
  combine_rows_any<1>(p, rows, lane, u, lse);
  store_u_row(p, row, lane, u[0], lse[0]);
}

// Combine fused with each head's value up-projection (V2 analysis page,
// section 6.1: every head first aggregates its latents with its own weights,
// then applies its own matrix, here W_UV[h]; the fused kernel the page
// mentions as the alternative order of work). One workgroup of 8 waves per
// (head h, 16 query tokens): each wave first issues its W_UV[h] fragments
// (output dims 16w..16w+15, all 512 latent dims), then merges two of the
// tokens' rows exactly as combine_wave_kernel does (one memory round trip
// for both), writes u and lse, and stages u as bf16 in LDS; after one
// barrier it computes its 16 x 16 block of o = u W_UV[h]^T on MFMA with the
// same operands and k order as out_proj, so o equals combine followed by
// out_proj bit for bit. When (head, token block) pairs alone would leave CUs
// idle, each pair gets two workgroups that split the output dims (waves 0-3
// project 64 of them; both merge the same rows and the first writes u).
constexpr int kOutTok = 16;
constexpr int kOutThreads = 512;
constexpr int kUPitch = kDc * 2 + 16;   // bf16 row + 16 B: rows start 4 banks apart

__global__ __launch_bounds__(kOutThreads) void combine_out_kernel(CombineParams p, int n_rb, int nj) {
  __shared__ __attribute__((aligned(16))) char ush_raw[kOutTok * kUPitch];
  lds_char* const ush = (lds_char*)ush_raw;
  // the row blocks of one head run on one XCD (they read the same W_UV[h])
  int h, r2;
  if (p.H % kNumXcd == 0) {
    h = (blockIdx.x / (kNumXcd * n_rb * nj)) * kNumXcd + blockIdx.x % kNumXcd;
    r2 = (blockIdx.x / kNumXcd) % (n_rb * nj);
  } else {
    h = blockIdx.x / (n_rb * nj);
    r2 = blockIdx.x % (n_rb * nj);
  }
  if (h >= p.H) return;                            // uniform over the workgroup
  const int rb = r2 / nj, jh = r2 % nj;            // token block, output-dim half
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i16 = lane & 15, G4 = lane >> 4;
  // output dims of this wave: 16 of 128, or (two workgroups per pair) waves
  // 0-3 take 16 of this workgroup's 64
  const bool projects = nj == 1 || wv < 4;         // wave-uniform
  const int jw = nj == 1 ? 16 * wv : 64 * jh + 16 * wv;
  bf16x8_t wf[16];
  if (projects) {
    const uint16_t* wrow = p.w_uv + ((size_t)h * kDh + jw + i16) * kDc + 8 * G4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) wf[ks] = load_bf16x8(wrow + 32 * ks);
  }
  const bool writes_u = p.out != nullptr && jh == 0;
  const int n0 = kOutTok * rb + 2 * wv;            // this wave's two tokens
  u32x4_t packed[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if (n0 + 1 < p.n_tok) {                          // wave-uniform
    const int rows[2] = {n0 * p.H + h, (n0 + 1) * p.H + h};
    float u[2][8], lse[2];
    combine_rows_any<2>(p, rows, lane, u, lse);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) packed[t][i] = pack_bf16x2(u[t][2 * i], u[t][2 * i + 1]);
      if (writes_u) store_u_row(p, rows[t], lane, u[t], lse[t]);
    }
  } else if (n0 < p.n_tok) {
    const int rows[1] = {n0 * p.H + h};
    float u[1][8], lse[1];
    combine_rows_any<1>(p, rows, lane, u, lse);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[0][i] = pack_bf16x2(u[0][2 * i], u[0][2 * i + 1]);
    if (writes_u) store_u_row(p, rows[0], lane, u[0], lse[0]);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
    *(MLA_LDS u32x4_t*)(ush + (2 * wv + t) * kUPitch + lane * 16) = packed[t];
  __syncthreads();
  if (!projects) return;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
    acc = mfma16x16x32(lds_read_b128(ush + i16 * kUPitch + (4 * ks + G4) * 16), wf[ks], acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = kOutTok * rb + 4 * G4 + i;
    if (n < p.n_tok) {
      const size_t off = ((size_t)n * p.H + h) * kDh + jw + i16;
      if (p.o_bf16) ((uint16_t*)p.o)[off] = f2bf(acc[i]);
      else ((float*)p.o)[off] = acc[i];
    }
  }
}

}  // namespace

hipError_t launch_combine_out(const CombineParams& p, hipStream_t s) {
  if (p.n_split > 64 || !p.w_uv || !p.o) return hipErrorInvalidValue;
  const int n_rb = (p.n_tok + kOutTok - 1) / kOutTok;
  const int nj = (int64_t)p.H * n_rb < 256 ? 2 : 1;   // split the output dims to fill the CUs
  hipLaunchKernelGGL(combine_out_kernel, dim3(p.H * n_rb * nj), dim3(kOutThreads), 0, s, p, n_rb,
                     nj);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.n_split > kMaxSplitsLds) return hipErrorInvalidValue;
  if (p.n_split <= 64)
    hipLaunchKernelGGL(combine_wave_kernel,
                       dim3(((p.rows + kWaveRows - 1) / kWaveRows + kNumXcd - 1) / kNumXcd * kNumXcd),
                       dim3(64 * kWaveRows), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel, dim3(p.rows), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
