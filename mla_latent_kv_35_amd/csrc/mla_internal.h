// Internal host-side interfaces between the C ABI (mla_api.hip) and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

constexpr int kPage = 64;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDh = 128;
constexpr int kMaxSplitPages = 1024; // pages of one split (MFMA kernel keeps their ids in LDS)
constexpr int kNumXcd = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Everything a decode kernel needs; filled by the host planner.
struct DecodeParams {
  const void* q_lat;        // [B][R][512], row stride q_lat_stride elements
  const void* q_rope;       // [B][R][64], row stride q_rope_stride elements
  const void* ckv;          // [n_pages][64][512]
  const void* kr;           // [n_pages][64][64]
  const float* ckv_scale;   // [n_pages][64] (fp8 only)
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;                // [B][R][512]
  float* lse;               // [B][R] or null
  void* part_u;             // [B][n_split][R][512] (n_split > 1): fp32 U, or bf16 u = U / l
  float* part_ml;           // [B][n_split][R][2]   fp32 (m in log2 units, l)
  int part_bf16;            // partials hold bf16 u = U / l (0 where l = 0)
  int B, T, H, R;           // R = T*H query rows per sequence
  int G;                    // row groups per sequence (MFMA kernel)
  int n_split, split_tokens;
  int n_pages, max_pages, max_seq_len;
  int out_bf16;
  int n_units;              // work units actually present
  int per_xcd;              // grid = per_xcd * 8 (XCD-major unit numbering)
  float scale_log2;         // softmax_scale * log2(e)
  long q_lat_stride;        // elements between consecutive query rows of q_lat
  long q_rope_stride;       // ... and of q_rope
};

struct CombineParams {
  const void* part_u;       // as DecodeParams::part_u
  const float* part_ml;
  int part_bf16;
  void* out;
  float* lse;
  const int32_t* seq_lens;  // splits at or past L_b hold no partials
  int rows;                 // B*R
  int R, T, n_split, split_tokens;
  int max_seq_len, max_pages;
  int out_bf16;
  // fused value up-projection (combine_out): o[n][h] = W_UV[h] u[n][h]
  const uint16_t* w_uv;     // [H][128][512] bf16, or null
  void* o;                  // [n_tok][H][128]
  int o_bf16;
  int H, n_tok;             // n_tok = B*T
};




hipError_t launch_decode_simple_f32(const DecodeParams& p, hipStream_t s);
// bf16 (fp8: E4M3FN latent codes with per-token scales) latent pool, bf16
// rope pool, 128 query rows per workgroup
hipError_t launch_decode_pipe(const DecodeParams& p, bool fp8, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
// combine fused with the value up-projection; needs p.w_uv, p.o, n_split <= 64
hipError_t launch_combine_out(const CombineParams& p, hipStream_t s);

// Element strides of the (token, head) vectors of a [n_tok][heads][d] tensor:
// vector (n, h) starts at n * tok + h * head.
struct VecStrides {
  long tok, head;
};

// theta: device fp64 [d_r/2] per-pair frequencies, or null for base^(-2i/d_r)
hipError_t launch_rope(const void* x_in, VecStrides si, void* x_out, VecStrides so, int bf16,
                       const int32_t* pos, int n_tok, int n_heads, int d_r, double base,
                       const double* theta, hipStream_t s);
// q_rs, o_rs: row strides (elements between (token, head) rows) of q_nope, q_lat
hipError_t launch_absorb(const void* q_nope, long q_rs, const void* w_uk, void* q_lat, long o_rs,
                         int in_bf16, int out_bf16, int n_tok, int H, hipStream_t s);
// o[n][h][:] = W[h] u(n, h), u(n, h) at n * u_tok + h * u_head elements, o's
// (n, h) row at (n * H + h) * o_rs
hipError_t launch_out_proj_strided(const void* u, long u_tok, long u_head, const void* w_uv,
                                   void* o, long o_rs, int u_bf16, int w_bf16, int o_bf16,
                                   int n_tok, int H, hipStream_t s);
hipError_t launch_out_proj(const void* u, const void* w_uv, void* o, int u_bf16, int w_bf16,
                           int o_bf16, int n_tok, int H, hipStream_t s);

}  // namespace mla
