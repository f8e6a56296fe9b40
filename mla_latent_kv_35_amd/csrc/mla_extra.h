// Launch interfaces of the kernels outside the decode path: the cache
// append, the prefill attention and the expansion GEMM.
#pragma once

#include "mla_internal.h"

namespace mla {

struct AppendParams {
  const void* c_in;         // [n_tok][512] f32 or bf16
  const void* k_in;         // [n_tok][64] f32 or bf16 (not rotated)
  const float* rms_gain;    // [512] or null
  const int32_t* seq;       // [n_tok]
  const int32_t* pos;       // [n_tok]
  const int32_t* block_table;
  void* ckv;                // [n_pages][64][512]
  float* ckv_scale;         // [n_pages][64] (fp8 only)
  void* kr;                 // [n_pages][64][64]
  int n_tok, B, n_pages, max_pages;
  int c_bf16, k_bf16, kr_bf16;
  int ckv_dt;               // 0 f32, 1 bf16, 2 fp8 E4M3FN
  int normalize;
  float rms_eps;
  double rope_base;
  const double* rope_theta; // [32] or null (base^(-2i/64))
};

hipError_t launch_append(const AppendParams& p, hipStream_t s);

struct PrefillParams {
  const void* q_nope;       // [B][n_q][H][128] bf16
  const void* q_rope;       // [B][n_q][H][64] bf16, rotated
  const void* k_nope;       // [B][n_kv][H][128] bf16 (W_UK[h] c)
  const void* k_rope;       // [B][n_kv][64] bf16, rotated, shared by the heads
  const void* v;            // [B][n_kv][H][128] bf16 (W_UV[h] c)
  void* o;                  // [B][n_q][H][128]
  float* lse;               // [B][n_q][H] or null
  int B, n_q, n_kv, H;
  int o_bf16;
  float scale_log2;
};

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);
// C[M][N] = A[M][K] B[N][K]^T, B bf16, A f32 or bf16; N % 128 == 0, K % 32 == 0
hipError_t launch_gemm_nt(const void* A, int a_bf16, const uint16_t* B, void* C, int c_bf16, int M,
                          int N, int K, hipStream_t s);
// absorb (bf16 queries, bf16 W_UK) and d_r = 64 bf16 rope in one launch;
// freq null = base^(-2i/64)
// (strides as launch_absorb and launch_rope; rope vectors 16-byte aligned)
hipError_t launch_absorb_rope(const uint16_t* q_nope, long q_rs, const uint16_t* w_uk,
                              void* q_lat, long o_rs, int out_bf16, const uint16_t* q_rope,
                              VecStrides si, uint16_t* q_rot, VecStrides so, const int32_t* pos,
                              int n_tok, int H, double base, const double* freq, hipStream_t s);
// the same for fp32 queries, W_UK, q_lat and rope data
hipError_t launch_absorb_rope_f32(const float* q_nope, long q_rs, const float* w_uk, float* q_lat,
                                  long o_rs, const float* q_rope, VecStrides si, float* q_rot,
                                  VecStrides so, const int32_t* pos, int n_tok, int H,
                                  double base, const double* freq, hipStream_t s);

}  // namespace mla
