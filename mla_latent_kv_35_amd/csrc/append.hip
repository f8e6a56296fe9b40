// Cache append: each new token's 512 latent and 64 rope elements join the
// paged cache (PaperTrace "02 · DeepSeek-V2 analysis", section 1.3 and the
// token walk-through of section 6.3). The latent optionally passes through
// an RMSNorm (section 1.2) and is stored as f32, bf16 or fp8 E4M3FN with one
// fp32 scale per token; the rope key is rotated at the token's position and
// stored already rotated (section 6, third absorption condition).
//
// One wave per token, four tokens per workgroup. Lane i holds latent
// elements 8i..8i+7: the RMSNorm sum of squares and the fp8 absolute maximum
// are wave reductions in a fixed order, and each lane stores its 8 values
// with one vector store. Lanes 0-31 rotate rope pair i = lane in fp64, as the
// rope kernel does.
#include "mla_device.h"
#include "mla_extra.h"

namespace mla {
namespace {

constexpr int kTokPerBlock = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// binary32 -> OCP E4M3FN (bias 7, 3 mantissa bits, largest finite 448, no
// infinities, S.1111.111 is NaN), round to nearest even, saturating at
// +-448. Normal codes take the binary32 exponent rebiased and the top three
// mantissa bits rounded on the 20 bits below them; magnitudes under 2^-6
// are multiples of 2^-9 (subnormal codes 1..7), and rounding 7.5 * 2^-9 up
// gives 8 * 2^-9 = 2^-6, the first normal code, with the same bits.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return sign | 0x7Fu;
  uint32_t code;
  if (a >= 0x1p-6f) {
    const uint32_t au = __float_as_uint(a);
    const uint32_t e = (au >> 23) - 127u + 7u;   // >= 1 here
    const uint32_t mant = au & 0x7FFFFFu;
    uint32_t keep = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
    code = e > 15u ? 0x7Eu : (e << 3) + keep;    // a carry out of keep bumps the exponent
    if (code > 0x7Eu) code = 0x7Eu;
  } else {
    code = (uint32_t)rintf(a * 512.0f);          // exact scaling, then round half to even
  }
  return sign | code;
}

__global__ __launch_bounds__(64 * kTokPerBlock) void append_kernel(AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  if (n >= p.n_tok) return;                      // whole waves leave; no barrier below
  const int b = p.seq[n], s = p.pos[n];
  if (b < 0 || b >= p.B || s < 0 || s >= p.max_pages * kPage) return;
  const int page = p.block_table[(size_t)b * p.max_pages + s / kPage];
  if (page < 0 || page >= p.n_pages) return;
  const size_t slot = (size_t)page * kPage + s % kPage;

  // ---- latent ---------------------------------------------------------------
  float c[8];
  if (p.c_bf16) {
    const u32x4_t v = *(const u32x4_t*)((const uint16_t*)p.c_in + (size_t)n * kDc + 8 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = bf2f(v[i] & 0xffff);
      c[2 * i + 1] = bf2f(v[i] >> 16);
    }
  } else {
    const float* src = (const float*)p.c_in + (size_t)n * kDc + 8 * lane;
    const f32x4_t v0 = *(const f32x4_t*)src, v1 = *(const f32x4_t*)(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = v0[i];
      c[4 + i] = v1[i];
    }
  }
  if (p.normalize) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(c[i], c[i], ss);
    const float rms = sqrtf(wave_sum(ss) / (float)kDc + p.rms_eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c[i] = c[i] / rms;
      if (p.rms_gain) c[i] *= p.rms_gain[8 * lane + i];
    }
  }
  if (p.ckv_dt == 0) {
    float* dst = (float*)p.ckv + slot * kDc + 8 * lane;
    *(f32x4_t*)dst = (f32x4_t){c[0], c[1], c[2], c[3]};
    *(f32x4_t*)(dst + 4) = (f32x4_t){c[4], c[5], c[6], c[7]};
  } else if (p.ckv_dt == 1) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (uint32_t)f2bf(c[2 * i]) | ((uint32_t)f2bf(c[2 * i + 1]) << 16);
    *(u32x4_t*)((uint16_t*)p.ckv + slot * kDc + 8 * lane) = v;
  } else {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(c[i]));
    amax = wave_max(amax);
    const float scale = amax == 0.f ? 1.f : amax / 448.0f;
    u32x2_t v = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i >> 2] |= f32_to_e4m3fn(c[i] / scale) << (8 * (i & 3));
    *(u32x2_t*)((uint8_t*)p.ckv + slot * kDc + 8 * lane) = v;
    if (lane == 0) p.ckv_scale[slot] = scale;
  }

  // ---- rope key: pair i = lane, rotated in fp64 ------------------------------
  if (lane < kDr / 2) {
    double x0, x1;
    if (p.k_bf16) {
      const uint32_t w = ((const uint32_t*)p.k_in)[(size_t)n * (kDr / 2) + lane];
      x0 = bf2f(w & 0xffff);
      x1 = bf2f(w >> 16);
    } else {
      const float* src = (const float*)p.k_in + (size_t)n * kDr + 2 * lane;
      x0 = src[0];
      x1 = src[1];
    }
    const double theta =
        p.rope_theta ? p.rope_theta[lane] : pow(p.rope_base, -2.0 * (double)lane / (double)kDr);
    double sn, cn;
    sincos((double)s * theta, &sn, &cn);
    const float y0 = (float)(x0 * cn - x1 * sn);
    const float y1 = (float)(x0 * sn + x1 * cn);
    if (p.kr_bf16) {
      ((uint32_t*)p.kr)[slot * (kDr / 2) + lane] = (uint32_t)f2bf(y0) | ((uint32_t)f2bf(y1) << 16);
    } else {
      float* dst = (float*)p.kr + slot * kDr + 2 * lane;
      dst[0] = y0;
      dst[1] = y1;
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3((p.n_tok + kTokPerBlock - 1) / kTokPerBlock),
                     dim3(64 * kTokPerBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
