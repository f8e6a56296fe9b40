// Per-head value up-projection after latent aggregation (PaperTrace "02 ·
// DeepSeek-V2 analysis", section 6.1: each head aggregates latents with its
// own weights first, then applies its own matrix): o[n][h][:] = W_UV[h] u[n][h][:].
//
// bf16 weights: MFMA with both operands contiguous along the reduced latent
// axis in memory (u rows and W_UV rows), so they load straight from global
// memory. fp32: plain fp32 FMA.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8_t load_row8(const void* base, size_t off, bool bf16) {
  if (bf16) return load_bf16x8((const uint16_t*)base + off);
  const f32x4_t lo = *(const f32x4_t*)((const float*)base + off);
  const f32x4_t hi = *(const f32x4_t*)((const float*)base + off + 4);
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (__bf16)lo[i];
    r[i + 4] = (__bf16)hi[i];
  }
  return r;
}

// One workgroup per (head h, 64 output dims, 32 tokens); wave w owns output
// dims 64*jb + 16*w .. +15 for the 32 tokens (two 16-token MFMA tiles). All
// of a wave's operand loads (its 16 W_UV rows and the 32 u rows) are issued
// before its first MFMA. Workgroups are placed so that the blocks of one
// head, which read the same u rows, share an XCD (and its L2).
constexpr int kTokTile = 32;

// u row of (token n, head h) starts at n * u_tok + h * u_head elements:
// (H * 512, 512) for per-head aggregates; (512, 0) for a latent shared by
// every head (the key / value expansion of prefill).
template <bool U_BF16, bool O_BF16>
__global__ __launch_bounds__(kThreads) void out_proj_bf16_kernel(const void* __restrict__ u,
                                                                 const uint16_t* __restrict__ wuv,
                                                                 void* __restrict__ o, int n_tok,
                                                                 int H, int n_tb, long u_tok,
                                                                 long u_head) {
  // blocks on XCD x (= blockIdx % 8) serve the heads h with h % 8 == x
  const int x = blockIdx.x % kNumXcd, idx = blockIdx.x / kNumXcd;
  const int per_head = 2 * n_tb;
  const int h = kNumXcd * (idx / per_head) + x;
  if (h >= H) return;
  const int tb = (idx % per_head) >> 1, jb = idx & 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i16 = lane & 15, G4 = lane >> 4;
  const int j = 64 * jb + 16 * w + i16;               // this lane's output dim (B column)
  const int n0 = tb * kTokTile;

  bf16x8_t bw[16];
  const uint16_t* wrow = wuv + ((size_t)h * kDh + j) * kDc + 8 * G4;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) bw[ks] = load_bf16x8(wrow + 32 * ks);
  bf16x8_t a[2][16];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int na = n0 + 16 * tt + i16;                // this lane's token (A row)
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      a[tt][ks] = (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
      if (na < n_tok)
        a[tt][ks] = load_row8(u, (size_t)na * u_tok + (size_t)h * u_head + 32 * ks + 8 * G4, U_BF16);
    }
  }
  f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[tt] = mfma16x16x32(a[tt][ks], bw[ks], acc[tt]);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 16 * tt + 4 * G4 + i;
      if (n < n_tok) {
        const size_t off = ((size_t)n * H + h) * kDh + j;
        if (O_BF16) ((uint16_t*)o)[off] = f2bf(acc[tt][i]);
        else ((float*)o)[off] = acc[tt][i];
      }
    }
}

// fp32: one workgroup of 4 waves per (token, head, 32 outputs); wave w
// produces 8 outputs. Lane i holds u values 8i..8i+7; each output row
// W_UV[h][j] is read coalesced (8 values per lane), the wave's 8 rows all in
// flight at once, and summed by a fixed butterfly.
constexpr int kF32Waves = 4;
constexpr int kF32Rows = 8;                                  // outputs per wave
constexpr int kF32Blocks = kDh / (kF32Waves * kF32Rows);     // workgroups per (token, head)

__global__ __launch_bounds__(64 * kF32Waves) void out_proj_f32_kernel(const float* __restrict__ u,
                                                                    const float* __restrict__ wuv,
                                                                    float* __restrict__ o, int H,
                                                                    long u_tok, long u_head) {
  const int nh = blockIdx.x;
  const int h = nh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j0 = (blockIdx.y * kF32Waves + w) * kF32Rows;     // first output of this wave
  const float* ur = u + (size_t)(nh / H) * u_tok + (size_t)h * u_head + 8 * lane;
  f32x4_t wa[kF32Rows], wb[kF32Rows];
#pragma unroll
  for (int jj = 0; jj < kF32Rows; ++jj) {
    const float* wr = wuv + ((size_t)h * kDh + j0 + jj) * kDc + 8 * lane;
    wa[jj] = *(const f32x4_t*)wr;
    wb[jj] = *(const f32x4_t*)(wr + 4);
  }
  const f32x4_t u0 = *(const f32x4_t*)ur, u1 = *(const f32x4_t*)(ur + 4);
#pragma unroll
  for (int jj = 0; jj < kF32Rows; ++jj) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(wa[jj][i], u0[i], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(wb[jj][i], u1[i], acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) o[(size_t)nh * kDh + j0 + jj] = acc;
  }
}

}  // namespace

hipError_t launch_out_proj(const void* u, const void* w_uv, void* o, int u_bf16, int w_bf16,
                           int o_bf16, int n_tok, int H, hipStream_t s) {
  return launch_out_proj_strided(u, (long)H * kDc, kDc, w_uv, o, u_bf16, w_bf16, o_bf16, n_tok, H,
                                 s);
}

hipError_t launch_out_proj_strided(const void* u, long u_tok, long u_head, const void* w_uv,
                                   void* o, int u_bf16, int w_bf16, int o_bf16, int n_tok, int H,
                                   hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (w_bf16) {
    const int n_tb = (n_tok + kTokTile - 1) / kTokTile;
    const dim3 grid(kNumXcd * ((H + kNumXcd - 1) / kNumXcd) * 2 * n_tb);
    const uint16_t* w = (const uint16_t*)w_uv;
    if (u_bf16 && o_bf16)
      hipLaunchKernelGGL((out_proj_bf16_kernel<true, true>), grid, dim3(kThreads), 0, s, u, w, o, n_tok, H, n_tb,
                         u_tok, u_head);
    else if (u_bf16)
      hipLaunchKernelGGL((out_proj_bf16_kernel<true, false>), grid, dim3(kThreads), 0, s, u, w, o, n_tok, H, n_tb,
                         u_tok, u_head);
    else if (o_bf16)
      hipLaunchKernelGGL((out_proj_bf16_kernel<false, true>), grid, dim3(kThreads), 0, s, u, w, o, n_tok, H, n_tb,
                         u_tok, u_head);
    else
      hipLaunchKernelGGL((out_proj_bf16_kernel<false, false>), grid, dim3(kThreads), 0, s, u, w, o, n_tok, H, n_tb,
                         u_tok, u_head);
  } else {
    hipLaunchKernelGGL(out_proj_f32_kernel, dim3(n_tok * H, kF32Blocks), dim3(64 * kF32Waves), 0, s,
                       (const float*)u, (const float*)w_uv, (float*)o, H, u_tok, u_head);
  }
  return hipGetLastError();
}

}  // namespace mla
