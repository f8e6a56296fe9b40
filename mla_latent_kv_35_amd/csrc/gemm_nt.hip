// C[m][n] = sum_k A[m][k] B[n][k] on bf16 MFMA with fp32 accumulation: the
// key / value expansion of prefill (PaperTrace "02 · DeepSeek-V2 analysis",
// section 6.1), where A = the latents [n_tok][512] and B = the per-head
// up-projections flattened to [H*128][512], so C[n][h*128 + j] = W[h] c[n].
//
// One workgroup of 4 waves per 128 x 128 tile of C; wave (wm, wn) owns the
// 64 x 64 quarter (4 x 4 MFMA 16x16x32 blocks). K streams through LDS in
// chunks of 32 (one MFMA k-step), double-buffered: the next chunk's global
// loads are in flight while the current one is multiplied. LDS rows are
// 80 B apart (64 B of data + 16 B), so the 16 rows of an operand fragment
// start on 16 different bank quadruples. The C tile leaves through LDS in
// whole 256-byte row segments.
#include "dma.h"
#include "mla_device.h"
#include "mla_extra.h"

namespace mla {
namespace {

constexpr int kTile = 128;
constexpr int kKc = 32;
constexpr int kPitch = 80;                         // bytes per LDS row: 64 B of data + 16 B
constexpr int kBuf = kTile * kPitch;               // one operand chunk: 10 KB

// Tile of workgroup `bid`. The column tiles nt with nt % 8 == x run on XCD x
// (its share of B stays in that XCD's L2). Within an XCD, tiles go in groups
// of kGroupM row tiles: all of the XCD's column tiles for rows 0..7, then
// rows 8..15, ..., so the workgroups resident at one time read about 1 MB of
// A and 1.5 MB of B, which the 4 MB L2 holds.
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_of(int bid, int n_mt, int n_nt, int& mt, int& nt) {
  int x = 0, idx = bid, n_ntl = n_nt, stride = 1;
  if (n_nt % kNumXcd == 0) {
    x = bid % kNumXcd;
    idx = bid / kNumXcd;
    n_ntl = n_nt / kNumXcd;
    stride = kNumXcd;
  }
  const int group = idx / (kGroupM * n_ntl);
  const int gm0 = group * kGroupM;
  const int gsz = min(kGroupM, n_mt - gm0);
  const int r = idx - group * kGroupM * n_ntl;
  mt = gm0 + r % gsz;
  nt = stride * (r / gsz) + x;
}

template <bool A_BF16, bool C_BF16>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const void* __restrict__ A,
                                                      const uint16_t* __restrict__ Bm,
                                                      void* __restrict__ C, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * kBuf];   // A[2], B[2]
  lds_char* const smem = (lds_char*)smem_raw;
  int mt, nt;
  tile_of(blockIdx.x, (M + kTile - 1) / kTile, N / kTile, mt, nt);
  const int m0 = mt * kTile, n0 = nt * kTile;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i16 = lane & 15, G4 = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  // loads: a chunk of A (or B) is 128 rows x 64 B = 512 pieces of 16 B; 2 per thread
  u32x4_t ra[2], rb[2];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i, r = e >> 2, c = e & 3;
      const int m = m0 + r;
      ra[i] = (u32x4_t){0u, 0u, 0u, 0u};
      if (m < M) {
        if constexpr (A_BF16) {
          ra[i] = *(const u32x4_t*)((const uint16_t*)A + (size_t)m * K + k0 + 8 * c);
        } else {
          const float* src = (const float*)A + (size_t)m * K + k0 + 8 * c;
          const f32x4_t lo = *(const f32x4_t*)src, hi = *(const f32x4_t*)(src + 4);
          ra[i] = (u32x4_t){pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                            pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
        }
      }
      rb[i] = *(const u32x4_t*)(Bm + (size_t)(n0 + r) * K + k0 + 8 * c);   // N % 128 == 0
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i, r = e >> 2, c = e & 3;
      *(MLA_LDS u32x4_t*)(smem + buf * kBuf + r * kPitch + 16 * c) = ra[i];
      *(MLA_LDS u32x4_t*)(smem + (2 + buf) * kBuf + r * kPitch + 16 * c) = rb[i];
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int nk = K / kKc;
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int cur = kc & 1;
    if (kc + 1 < nk) load((kc + 1) * kKc);
#pragma unroll
    for (int ks = 0; ks < kKc / 32; ++ks) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = lds_read_b128(smem + cur * kBuf + (64 * wm + 16 * i + i16) * kPitch + 64 * ks + 16 * G4);
        b[i] = lds_read_b128(smem + (2 + cur) * kBuf + (64 * wn + 16 * i + i16) * kPitch + 64 * ks +
                             16 * G4);
      }
      // B fragments as the MFMA's A operand: the block holds C^T, so a lane
      // ends with 4 consecutive columns of one row of C
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(b[j], a[i], acc[i][j]);
    }
    if (kc + 1 < nk) store(cur ^ 1);            // the other buffer was last read one chunk ago
    __syncthreads();
  }
  // lane holds C[64wm + 16i + i16][64wn + 16j + 4*G4 + r], r = 0..3
  if constexpr (C_BF16) {
    // stage the bf16 tile in LDS (rows of 256 B + 16 B), then write whole
    // 256-byte row segments with 16-byte stores; the K loop's last barrier
    // freed the operand buffers
    constexpr int kCPitch = kTile * 2 + 16;
    static_assert(kTile * kCPitch <= 4 * kBuf, "C tile fits in the operand buffers");
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(MLA_LDS u32x2_t*)(smem + (64 * wm + 16 * i + i16) * kCPitch +
                            2 * (64 * wn + 16 * j + 4 * G4)) =
            (u32x2_t){pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                      pack_bf16x2(acc[i][j][2], acc[i][j][3])};
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kTile * kTile * 2 / 16 / 256; ++q) {
      const int e = tid + 256 * q, row = e >> 4, ch = e & 15;
      const int m = m0 + row;
      if (m < M)
        *(u32x4_t*)((uint16_t*)C + (size_t)m * N + n0 + 8 * ch) =
            *(const MLA_LDS u32x4_t*)(smem + row * kCPitch + 16 * ch);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 64 * wm + 16 * i + i16;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(f32x4_t*)((float*)C + (size_t)m * N + n0 + 64 * wn + 16 * j + 4 * G4) = acc[i][j];
    }
  }
}

// bf16 A: the operand chunks land in LDS by direct global -> LDS copies, in
// kStages buffers (two chunks in flight behind the one being multiplied, no
// registers held by loads). A copy fills 1 KB of LDS = 16 rows of 64 B, so
// rows are not padded; instead 16-B chunk c of row r sits at slot
// c ^ ((r >> 2) & 3), which keeps the 16 rows of an operand fragment on 16
// distinct bank quadruples.
constexpr int kStages = 3;
constexpr int kRowB = kKc * 2;                     // 64 B: one K chunk of a row
constexpr int kStage = 2 * kTile * kRowB;          // A rows, then B rows: 16 KB

template <bool C_BF16>
__global__ __launch_bounds__(256) void gemm_nt_dma_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ Bm,
                                                          void* __restrict__ C, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kStages * kStage];
  lds_char* const smem = (lds_char*)smem_raw;
  int mt, nt;
  tile_of(blockIdx.x, (M + kTile - 1) / kTile, N / kTile, mt, nt);
  const int m0 = mt * kTile, n0 = nt * kTile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, G4 = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  // copy q of a stage (q = 0..15, 1 KB each) fills rows 16(q & 7) .. +15 of
  // A (q < 8) or B; wave w issues q = 4w .. 4w+3, so waves 0-1 copy A and
  // 2-3 copy B. Lane l fills slot l & 3 of row l >> 2 with the chunk that
  // belongs there. Rows of A past M read row M-1 (their results are dropped).
  const bool copies_b = w >= 2;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * ((4 * w + i) & 7) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const size_t grow = copies_b ? (size_t)(n0 + row) : (size_t)min(m0 + row, M - 1);
    voff[i] = (uint32_t)((grow * K + 8 * c) * 2);
  }
  const uint16_t* const src = copies_b ? Bm : A;
  auto issue = [&](int kc) __attribute__((always_inline)) {
    lds_char* const st = smem + (kc % kStages) * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma_copy16(src + kc * kKc, voff[i], st + (4 * w + i) * 1024);
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int nk = K / kKc;
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st < nk) issue(st);
  for (int kc = 0; kc < nk; ++kc) {
    // chunk kc has landed once at most the next chunk's 4 copies are in flight
    if (kc + 1 < nk) dma_wait<4>();
    else dma_wait<0>();
    lds_barrier();                                // every wave's copies of chunk kc landed;
    if (kc + kStages - 1 < nk) issue(kc + kStages - 1);   // chunk kc-1's buffer is free
    const lds_char* const st = smem + (kc % kStages) * kStage;
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = 64 * wm + 16 * i + i16, rb = 64 * wn + 16 * i + i16;
      a[i] = lds_read_b128(st + ra * kRowB + 16 * (G4 ^ ((ra >> 2) & 3)));
      b[i] = lds_read_b128(st + kTile * kRowB + rb * kRowB + 16 * (G4 ^ ((rb >> 2) & 3)));
    }
    // B fragments as the MFMA's A operand: the block holds C^T, so a lane
    // ends with 4 consecutive columns of one row of C
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(b[j], a[i], acc[i][j]);
  }
  __syncthreads();                                // every wave is done with the stage buffers
  // lane holds C[64wm + 16i + i16][64wn + 16j + 4*G4 + r], r = 0..3
  if constexpr (C_BF16) {
    constexpr int kCPitch = kTile * 2 + 16;
    static_assert(kTile * kCPitch <= kStages * kStage, "C tile fits in the stage buffers");
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(MLA_LDS u32x2_t*)(smem + (64 * wm + 16 * i + i16) * kCPitch +
                            2 * (64 * wn + 16 * j + 4 * G4)) =
            (u32x2_t){pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                      pack_bf16x2(acc[i][j][2], acc[i][j][3])};
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kTile * kTile * 2 / 16 / 256; ++q) {
      const int e = tid + 256 * q, row = e >> 4, ch = e & 15;
      const int m = m0 + row;
      if (m < M)
        *(u32x4_t*)((uint16_t*)C + (size_t)m * N + n0 + 8 * ch) =
            *(const MLA_LDS u32x4_t*)(smem + row * kCPitch + 16 * ch);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 64 * wm + 16 * i + i16;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(f32x4_t*)((float*)C + (size_t)m * N + n0 + 64 * wn + 16 * j + 4 * G4) = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm_nt(const void* A, int a_bf16, const uint16_t* B, void* C, int c_bf16, int M,
                          int N, int K, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (N % kTile != 0 || K % kKc != 0) return hipErrorInvalidValue;
  const dim3 grid((N / kTile) * ((M + kTile - 1) / kTile));
  // direct copies take per-lane 32-bit byte offsets into A and B
  const bool dma = (int64_t)M * K * 2 < ((int64_t)1 << 31) && (int64_t)N * K * 2 < ((int64_t)1 << 31);
  if (a_bf16 && dma && c_bf16)
    hipLaunchKernelGGL(gemm_nt_dma_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)A, B, C,
                       M, N, K);
  else if (a_bf16 && dma)
    hipLaunchKernelGGL(gemm_nt_dma_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)A, B, C,
                       M, N, K);
  else if (a_bf16 && c_bf16)
    hipLaunchKernelGGL((gemm_nt_kernel<true, true>), grid, dim3(256), 0, s, A, B, C, M, N, K);
  else if (a_bf16)
    hipLaunchKernelGGL((gemm_nt_kernel<true, false>), grid, dim3(256), 0, s, A, B, C, M, N, K);
  else if (c_bf16)
    hipLaunchKernelGGL((gemm_nt_kernel<false, true>), grid, dim3(256), 0, s, A, B, C, M, N, K);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<false, false>), grid, dim3(256), 0, s, A, B, C, M, N, K);
  return hipGetLastError();
}

}  // namespace mla
