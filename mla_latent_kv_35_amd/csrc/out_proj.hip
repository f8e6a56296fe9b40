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

// One workgroup of 4 waves per (head h, 64 tokens, 128 / NJ output dims). The
// block's u rows are staged once in LDS (as bf16, 16-byte chunk c of token t
// at c ^ (t & 15), so the 16 tokens of an MFMA A fragment hit 16 distinct
// bank groups); wave w holds the W_UV[h] rows of its 32 / NJ output dims in
// registers (the MFMA B operand, contiguous along the latent axis in memory)
// and multiplies them against all 64 tokens. NJ = 1 when there are enough
// (head, token block) pairs to fill the device, else 2. Workgroups are placed
// so that the blocks of one head share an XCD (and W_UV[h] in its L2).
constexpr int kTokTile = 64;
constexpr int kUStage = kTokTile * kDc * 2;   // 64 KB

// u row of (token n, head h) starts at n * u_tok + h * u_head elements:
// (H * 512, 512) for per-head aggregates; (512, 0) for a latent shared by
// every head. o row (n, h) starts at (n * H + h) * o_rs elements.
template <bool U_BF16, bool O_BF16, int NJ, int TT>
__global__ __launch_bounds__(kThreads) void out_proj_bf16_kernel(const void* __restrict__ u,
                                                                 const uint16_t* __restrict__ wuv,
                                                                 void* __restrict__ o, long o_rs,
                                                                 int n_tok, int H, int n_tb,
                                                                 long u_tok, long u_head) {
  constexpr int JB = 2 / NJ;                          // 16-wide output blocks per wave
  __shared__ __attribute__((aligned(16))) char ush_raw[kUStage];
  lds_char* const ush = (lds_char*)ush_raw;
  // blocks on XCD x (= blockIdx % 8) serve the heads h with h % 8 == x
  const int x = blockIdx.x % kNumXcd, idx = blockIdx.x / kNumXcd;
  const int per_head = NJ * n_tb;
  const int h = kNumXcd * (idx / per_head) + x;
  if (h >= H) return;                                 // uniform over the workgroup
  const int tb = (idx % per_head) / NJ, jh = (idx % per_head) % NJ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i16 = lane & 15, G4 = lane >> 4;
  const int j0 = (kDh / NJ) * jh + 16 * JB * w;       // this wave's first output dim
  const int n0 = tb * kTokTile;                      // TT 16-token blocks from n0

  // the wave's W_UV rows, all in flight before the staging below waits
  bf16x8_t bw[JB][16];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const uint16_t* wrow = wuv + ((size_t)h * kDh + j0 + 16 * jb + i16) * kDc + 8 * G4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) bw[jb][ks] = load_bf16x8(wrow + 32 * ks);
  }
  // stage u[n0 .. n0+16*TT-1][h][:] as bf16 (zero rows past n_tok): up to
  // 16 chunks per thread, in rounds of at most 8 whose loads are all in
  // flight before their first store
  constexpr int kChunks = TT * 16 * kDc * 2 / 16 / kThreads;
  constexpr int kRound = kChunks < 8 ? kChunks : 8;
#pragma unroll
  for (int q0 = 0; q0 < kChunks; q0 += kRound) {
    bf16x8_t uv[kRound];
#pragma unroll
    for (int q = 0; q < kRound; ++q) {
      const int e = tid + kThreads * (q0 + q), t = e >> 6, c = e & 63;
      const int n = n0 + t;
      uv[q] = (bf16x8_t){0, 0, 0, 0, 0, 0, 0, 0};
      if (n < n_tok) uv[q] = load_row8(u, (size_t)n * u_tok + (size_t)h * u_head + 8 * c, U_BF16);
    }
#pragma unroll
    for (int q = 0; q < kRound; ++q) {
      const int e = tid + kThreads * (q0 + q), t = e >> 6, c = e & 63;
      *(MLA_LDS bf16x8_t*)(ush + t * (kDc * 2) + ((c & ~15) | ((c ^ t) & 15)) * 16) = uv[q];
    }
  }
  __syncthreads();
  f32x4_t acc[TT][JB];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[tt][jb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    bf16x8_t a[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = 16 * tt + i16, c = 4 * ks + G4;
      a[tt] = lds_read_b128(ush + t * (kDc * 2) + ((c & ~15) | ((c ^ t) & 15)) * 16);
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) acc[tt][jb] = mfma16x16x32(a[tt], bw[jb][ks], acc[tt][jb]);
  }
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 16 * tt + 4 * G4 + i;
        if (n < n_tok) {
          const size_t off = ((size_t)n * H + h) * o_rs + j0 + 16 * jb + i16;
          if (O_BF16) ((uint16_t*)o)[off] = f2bf(acc[tt][jb][i]);
          else ((float*)o)[off] = acc[tt][jb][i];
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
                                                                    float* __restrict__ o,
                                                                    long o_rs, int H, long u_tok,
                                                                    long u_head) {
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
    if (lane == 0) o[(size_t)nh * o_rs + j0 + jj] = acc;
  }
}

}  // namespace

hipError_t launch_out_proj(const void* u, const void* w_uv, void* o, int u_bf16, int w_bf16,
                           int o_bf16, int n_tok, int H, hipStream_t s) {
  return launch_out_proj_strided(u, (long)H * kDc, kDc, w_uv, o, kDh, u_bf16, w_bf16, o_bf16,
                                 n_tok, H, s);
}

hipError_t launch_out_proj_strided(const void* u, long u_tok, long u_head, const void* w_uv,
                                   void* o, long o_rs, int u_bf16, int w_bf16, int o_bf16,
                                   int n_tok, int H, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (w_bf16) {
    const int n_tb = (n_tok + kTokTile - 1) / kTokTile;
    const int heads = kNumXcd * ((H + kNumXcd - 1) / kNumXcd);
    // one block per (head, token block) when that fills the device, else two;
    // a single short token block computes only its live 16-token blocks
    const bool split_j = (int64_t)heads * n_tb < 256;
    const int tt = n_tb > 1 ? 4 : (n_tok <= 16 ? 1 : n_tok <= 32 ? 2 : 4);
    const dim3 grid(heads * n_tb * (split_j ? 2 : 1));
    const uint16_t* w = (const uint16_t*)w_uv;
#define MLA_OUTP_T(UB, OB, NJ)                                                                \
  if (tt == 1)                                                                                \
    hipLaunchKernelGGL((out_proj_bf16_kernel<UB, OB, NJ, 1>), grid, dim3(kThreads), 0, s, u, w, \
                       o, o_rs, n_tok, H, n_tb, u_tok, u_head);                                     \
  else if (tt == 2)                                                                           \
    hipLaunchKernelGGL((out_proj_bf16_kernel<UB, OB, NJ, 2>), grid, dim3(kThreads), 0, s, u, w, \
                       o, o_rs, n_tok, H, n_tb, u_tok, u_head);                                     \
  else                                                                                        \
    hipLaunchKernelGGL((out_proj_bf16_kernel<UB, OB, NJ, 4>), grid, dim3(kThreads), 0, s, u, w, \
                       o, o_rs, n_tok, H, n_tb, u_tok, u_head);
#define MLA_OUTP(UB, OB)  \
  if (split_j) {          \
    MLA_OUTP_T(UB, OB, 2) \
  } else {                \
    MLA_OUTP_T(UB, OB, 1) \
  }
    if (u_bf16 && o_bf16) {
      MLA_OUTP(true, true)
    } else if (u_bf16) {
      MLA_OUTP(true, false)
    } else if (o_bf16) {
      MLA_OUTP(false, true)
    } else {
      MLA_OUTP(false, false)
    }
#undef MLA_OUTP
#undef MLA_OUTP_T
  } else {
    hipLaunchKernelGGL(out_proj_f32_kernel, dim3(n_tok * H, kF32Blocks), dim3(64 * kF32Waves), 0, s,
                       (const float*)u, (const float*)w_uv, (float*)o, o_rs, H, u_tok, u_head);
  }
  return hipGetLastError();
}

}  // namespace mla
