/*
 * mla.h -- C ABI of libmla.so: MLA absorbed decode on AMD MI355X (gfx950).
 *
 * Multi-head Latent Attention caches, per token and layer, only a joint KV
 * latent c (d_c = 512) and one decoupled RoPE key k^R (d_R = 64) that every
 * head shares (PaperTrace "02 · DeepSeek-V2 analysis", sections 1.2-1.3:
 * 576 elements per token per layer). At decode time each head's content
 * query is absorbed into the latent space through W^UK (section 1.2 and
 * section 6), scores are q_lat.c + q_rope.k^R scaled by 1/sqrt(d_h + d_R)
 * (eq. 18), softmax runs over the cached tokens, each head aggregates
 * latents u = sum_s a_s c_s, and only then applies its own W^UV (section 6.1).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers, owned by the caller, in the
 *    layout stated (row-major, last index fastest). Where a call takes
 *    strides they count ELEMENTS, 0 selects the packed layout, and a "row"
 *    is the innermost vector of one (token, head) pair: a [n][H][d] tensor
 *    with row stride r holds element (n, h, i) at (n * H + h) * r + i, so
 *    a slice of a wider per-head vector (say the first 128 of each head's
 *    192 query elements) is passed as-is. The library never allocates,
 *    frees or keeps a pointer after the call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *    is stream-ordered; the library never synchronizes.
 *  - Arguments are checked on the host before anything is launched; a bad
 *    argument returns an error status and launches nothing. A failed launch
 *    returns MLA_ERR_LAUNCH. No C++ exception crosses this ABI.
 *  - Device-side data the host cannot see (sequence lengths, block-table
 *    entries) is range-checked in the kernel: a sequence whose length or
 *    page ids are out of range gets NaN outputs instead of a memory fault.
 *  - Results are deterministic: no atomics, fixed reduction order; the
 *    order depends on logical token indices only, never on physical pages.
 *  - Calls are thread-safe. The only process-wide state is the static array
 *    of the allocation-free decode entry point.
 *
 * dtypes: MLA_F32 = IEEE binary32, MLA_BF16 = bfloat16, MLA_FP8_E4M3 = OCP
 * E4M3FN (bias 7, max 448, no infinities) with one fp32 scale per token.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2
#define MLA_PAGE_SIZE 64

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  MLA_ERR_DTYPE = 3,       /* dtype combination not supported */
  MLA_ERR_UNSUPPORTED = 4, /* shape outside what the kernels implement */
  MLA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  MLA_ERR_LAUNCH = 6       /* the HIP launch failed */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype;

/* Human-readable name of a status code (static string; never NULL). */
const char* mla_status_str(int status);

/* MLA_ABI_VERSION of the built library. */
int mla_abi_version(void);

/*
 * mla_absorb_q -- absorb W^UK into the content query.
 *   q_lat[n][h][:] = W_UK[h]^T q_nope[n][h][:]
 * i.e. q^T (W^UK c) = (W^UK^T q)^T c (V2 analysis page, section 1.2 and the
 * first absorption condition of section 6: a fixed linear map moved to the
 * query side).
 *   q_nope : [n_tok][H][d_h]  dtype q_dt (F32 or BF16), row stride
 *            q_row_stride (0: d_h)
 *   w_uk   : [H][d_h][d_c]    dtype q_dt (head h's up-projection, d_h x d_c),
 *            packed
 *   q_lat  : [n_tok][H][d_c]  dtype out_dt (F32, or BF16 when q_dt is BF16),
 *            row stride out_row_stride (0: d_c)
 * Supported: d_h = 128, d_c = 512, n_tok >= 0 (0 launches nothing), H >= 1,
 * 16-byte aligned tensors and rows (row stride x element size a multiple of
 * 16 bytes; else MLA_ERR_UNSUPPORTED). A row stride that is negative or
 * below the row length is MLA_ERR_SHAPE.
 * Accumulation is fp32; F32 inputs use fp32 FMA end to end.
 */
int mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat,
                 int q_dt, int out_dt, int n_tok, int H, int d_h, int d_c,
                 int64_t q_row_stride, int64_t out_row_stride, void* stream);

/*
 * mla_rope -- rotary position embedding of the decoupled rope query or key.
 * Coordinate pairs (2i, 2i+1) are rotated at position n (CSDN "DeepSeek-V3
 * structure and engineering", section 2(3)); the rope part is decoupled from
 * the absorbed content part (V2 analysis page, section 1.3, eq. 14-15):
 *   a = pos[n] * base^(-2i/d_r)           (angle in fp64)
 *   y[2i]   = x[2i] cos a - x[2i+1] sin a
 *   y[2i+1] = x[2i] sin a + x[2i+1] cos a
 *   x_in, x_out : [n_tok][n_heads][d_r], dtype dt (F32 or BF16); element
 *                 (n, h, i) of x_in at n * in_tok_stride +
 *                 h * in_head_stride + i, of x_out likewise with the out
 *                 strides (0: the packed n_heads * d_r and d_r). They are
 *                 disjoint, or the same memory with the same strides
 *                 (in place); x_out's vectors must not overlap one another.
 *   pos         : int32 [n_tok], positions >= 0
 * Supported: d_r even, 2 <= d_r <= 256; n_tok >= 0; any strides >= 0 (a
 * stride that is negative, or an out stride that makes output vectors
 * overlap, is MLA_ERR_SHAPE; x_in == x_out with different strides is too).
 * d_r = 64 with 16-byte aligned vectors takes a vectorised kernel.
 */
int mla_rope(const void* x_in, void* x_out, int dt, const int32_t* pos,
             int n_tok, int n_heads, int d_r, double base,
             int64_t in_tok_stride, int64_t in_head_stride,
             int64_t out_tok_stride, int64_t out_head_stride, void* stream);

/*
 * mla_rope_freq -- mla_rope with caller-given per-pair frequencies:
 *   a = pos[n] * theta[i]   (fp64), then the same rotation as mla_rope.
 *   theta : DEVICE fp64 [d_r / 2], e.g. from mla_yarn_frequencies.
 * Same layouts, strides, support and errors as mla_rope (theta NULL:
 * MLA_ERR_NULL).
 */
int mla_rope_freq(const void* x_in, void* x_out, int dt, const int32_t* pos,
                  int n_tok, int n_heads, int d_r, const double* theta,
                  int64_t in_tok_stride, int64_t in_head_stride,
                  int64_t out_tok_stride, int64_t out_head_stride, void* stream);

/*
 * mla_absorb_q_rope -- the query side of a decode step in one call: the
 * result is exactly that of mla_absorb_q(q_nope, w_uk, q_lat, ...) followed
 * by mla_rope(q_rope, q_rot, rope_dt, pos, ..., base) -- or by
 * mla_rope_freq(..., theta) when theta is not NULL -- bit for bit. The two
 * halves of the V2 analysis page's query (section 1.3, eq. 14-15: the
 * absorbed content part and the separately rotated rope part) are
 * independent, so with queries and rope data both BF16 or both F32, d_r = 64
 * and 16-byte aligned rope rows they run as one kernel launch; otherwise as
 * the two calls.
 *   q_nope, w_uk, q_lat, q_dt, out_dt, d_h, d_c, q_row_stride,
 *   out_row_stride : as mla_absorb_q (n_tok x H)
 *   q_rope, q_rot : [n_tok][H][d_r], dtype rope_dt (F32 or BF16), row
 *                   strides rope_row_stride and rot_row_stride (0: d_r;
 *                   mla_rope's token and head strides H * r and r); in place
 *                   when the same memory with the same stride
 *   pos           : int32 [n_tok]
 *   theta         : DEVICE fp64 [d_r / 2] or NULL (then base^(-2i/d_r))
 * Errors: those of mla_absorb_q and mla_rope / mla_rope_freq; nothing is
 * launched when any argument is rejected.
 */
int mla_absorb_q_rope(const void* q_nope, const void* w_uk, void* q_lat, int q_dt, int out_dt,
                      const void* q_rope, void* q_rot, int rope_dt, const int32_t* pos,
                      int n_tok, int H, int d_h, int d_c, int d_r, double base,
                      const double* theta, int64_t q_row_stride, int64_t out_row_stride,
                      int64_t rope_row_stride, int64_t rot_row_stride, void* stream);

/*
 * mla_yarn_frequencies -- YaRN frequencies of the decoupled rope part for a
 * context extended by `factor` (V2 analysis page, section 3.2: YaRN acts on
 * the 64 rope dimensions only; V2 uses factor s = 40, alpha = 1, beta = 32 on
 * a 4K original window). The pages do not print the interpolation rule; this
 * is the NTK-by-parts ramp of the YaRN method, per pair i:
 *   theta_i  = base^(-2i/d_r),  r_i = orig_len * theta_i / (2 pi)
 *              (rotations of pair i over the original window)
 *   gamma_i  = clamp((r_i - alpha) / (beta - alpha), 0, 1)
 *   theta'_i = (1 - gamma_i) * theta_i / factor + gamma_i * theta_i
 * so pairs that turn fewer than alpha times are fully interpolated, pairs
 * that turn more than beta times are unchanged. factor = 1 gives theta_i.
 *   theta : HOST fp64 [d_r / 2], written.
 * Errors: MLA_ERR_NULL (theta), MLA_ERR_SHAPE (d_r odd or outside 2..256,
 * base <= 0, factor < 1, beta <= alpha, orig_len < 1).
 */
int mla_yarn_frequencies(int d_r, double base, double factor, double alpha, double beta,
                         int orig_len, double* theta);

/*
 * mla_yarn_mscale -- YaRN attention temperature factor sqrt(1/t) =
 * coef * ln(factor) + 1 (1 for factor <= 1). V2 analysis page, section 3.2:
 * V2 uses coef = 0.0707 (about 1.26 at factor 40; the original YaRN
 * coefficient 0.1 gives about 1.37), applied through the softmax scale
 * rather than the rope cos/sin, because only the 64 rope dimensions of MLA
 * are rotated. The original scheme scales q and k each by sqrt(1/t), i.e.
 * the logits by 1/t, so the softmax scale to pass to mla_decode_paged is
 * 1/sqrt(d_h + d_r) * mla_yarn_mscale(factor, coef)^2.
 */
double mla_yarn_mscale(double factor, double coef);

/*
 * Arguments of the paged absorbed-decode kernel.
 *
 * Paged cache: token s of sequence b lives in page block_table[b][s / 64],
 * slot s % 64, of two pools that hold the 512 latent and the 64 rotated rope
 * elements of each token (the 576-element cache of the V2 analysis page,
 * section 1.3; the key is cached already rotated, section 6).
 *
 * Query rows: row (b, t, h) is query token t (0 <= t < T) of sequence b and
 * head h; it sits at position L_b - T + t and attends to tokens
 * s <= L_b - T + t (the T new tokens are already in the cache; T = 2 gives
 * the causal mask between two speculative tokens).
 */
typedef struct mla_decode_args {
  int32_t B, T, H;          /* batch, query tokens per sequence (1 or 2), heads */
  int32_t d_c, d_r;         /* latent and rope widths: must be 512 and 64 */
  int32_t page_size;        /* must be MLA_PAGE_SIZE */
  int32_t n_pages;          /* pages in each pool (bound for block-table ids) */
  int32_t max_pages_per_seq;/* row length of block_table */
  int32_t max_seq_len;      /* host upper bound on seq_lens[b] */
  int32_t q_dt;             /* dtype of q_lat and q_rope: F32 or BF16 */
  int32_t ckv_dt;           /* latent pool: F32, BF16 or FP8_E4M3 */
  int32_t kr_dt;            /* rope pool: F32 (iff ckv_dt is F32) or BF16 */
  int32_t out_dt;           /* u: F32 or BF16 */
  int32_t split_tokens;     /* 0 = auto; else a multiple of 64, at most 65536
                               (MLA_ERR_UNSUPPORTED above): split k covers
                               tokens [k*split_tokens, (k+1)*split_tokens) */
  int64_t total_tokens;     /* host hint: sum of seq_lens (0 = unknown) */
  float softmax_scale;      /* 1/sqrt(d_h + d_r) for DeepSeek-V2 (eq. 18) */
  int32_t heads_per_wg;     /* query rows (token, head pairs) per workgroup:
                               0 = the kernel's own (BF16 and FP8 pools 128,
                               F32 1; mla_decode_plan reports it), else it
                               must equal that value (MLA_ERR_UNSUPPORTED) */
  int64_t q_lat_stride;     /* row stride of q_lat (0: d_c), >= d_c */
  int64_t q_rope_stride;    /* row stride of q_rope (0: d_r), >= d_r; both
                               with rows 16-byte aligned */
  const void* q_lat;        /* [B][T][H][d_c] absorbed queries (mla_absorb_q) */
  const void* q_rope;       /* [B][T][H][d_r] rotated rope queries (mla_rope) */
  const void* ckv;          /* [n_pages][64][d_c] latent pool */
  const void* kr;           /* [n_pages][64][d_r] rotated rope-key pool */
  const float* ckv_scale;   /* [n_pages][64] fp32 per-token scale iff ckv_dt is
                               FP8_E4M3 (value = code * scale), else NULL */
  const int32_t* block_table;/* [B][max_pages_per_seq] page ids */
  const int32_t* seq_lens;  /* [B] cached length L_b incl. the T new tokens;
                               T <= L_b <= max_seq_len */
  void* out;                /* [B][T][H][d_c] u = sum_s a_s c_s, dtype out_dt */
  float* lse;               /* [B][T][H] natural-log sum of exp(scores), or NULL */
  void* workspace;          /* device scratch of workspace_bytes (split partials) */
  size_t workspace_bytes;
  /* Optional value up-projection in the same call (V2 analysis page,
   * section 6.1: each head aggregates first, then applies its own matrix):
   * o[b][t][h][:] = W_UV[h] u[b][t][h][:], exactly as mla_out_proj computes
   * it from u. With 2 to 4 splits and bf16 weights the log-sum-exp combine
   * and the projection run as one kernel (u is still written); otherwise as
   * the combine followed by the projection, with the same results. */
  const void* w_uv;         /* [H][128][d_c] dtype w_dt, or NULL: no projection */
  int32_t w_dt;             /* BF16, or F32 with F32 u and o (fp32 pools) */
  int32_t o_dt;             /* F32 or BF16 */
  void* o;                  /* [B][T][H][128] */
} mla_decode_args;

/*
 * mla_decode_plan -- host-only: the split size, split count, query rows per
 * workgroup and workspace bytes mla_decode_paged will use for these
 * arguments (pointers may be NULL; any output pointer may be NULL).
 * With more than one split, each (sequence, split, row group) produces
 * partials merged by a log-sum-exp combine kernel: fp32 (m, l) per row and
 * the split's latent aggregate, as fp32 U when out_dt is F32 and as bf16
 * u = U / l when out_dt is BF16 (bf16 and fp8 pools), so the workspace size
 * depends on out_dt.
 */
int mla_decode_plan(const mla_decode_args* args, int* split_tokens, int* n_split,
                    int* heads_per_wg, size_t* workspace_bytes);

/*
 * mla_decode_paged -- absorbed MLA decode over the paged cache (V2 analysis
 * page, sections 1.2-1.3 and 6.1):
 *   z_s  = (q_lat . c_s + q_rope . k^R_s) * softmax_scale
 *   a_s  = softmax over the visible s
 *   u    = sum_s a_s c_s            (latent-space aggregate, W^UV not applied)
 *   lse  = ln sum_s exp(z_s)
 * F32 caches run an fp32 kernel; BF16 caches run bf16 MFMA with fp32 softmax
 * and accumulation; FP8_E4M3 latents stay fp8 in HBM (half the bytes read)
 * and are widened in LDS, once per tile, to c_s = bf16(scale_s * code_s)
 * (the product in fp32, rounded to nearest even), which then takes the
 * bf16 path (q_lat is not quantized).
 */
int mla_decode_paged(const mla_decode_args* args, void* stream);

/*
 * mla_decode_paged_noalloc -- mla_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It ignores args->workspace and
 * args->workspace_bytes and keeps the split partials in a static device
 * array of MLA_NOALLOC_SCRATCH_BYTES per GPU instead, held until the process
 * ends; nothing is allocated or freed. Calls whose partials would exceed it
 * (mla_decode_plan's workspace_bytes) return MLA_ERR_WORKSPACE before any
 * launch. Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (different streams, or host threads without ordering) race.
 * Results are those of mla_decode_paged for the same arguments.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
int mla_decode_paged_noalloc(const mla_decode_args* args, void* stream);

/*
 * mla_stream_read -- diagnostic: reads `bytes` (a multiple of 16) of device
 * memory at src once with 16-byte loads and discards them, so that the
 * caller can time the read bandwidth a plain stream reaches on this GPU (the
 * reference against which the decode's cache-read rate is judged; the
 * V2 analysis page, section 1.2, puts decode at the cache-read bound). sink
 * (device, 16 bytes, 16-byte aligned) is written only in the rare case that
 * the folded loads equal a fixed sentinel. Misaligned pointers or sizes
 * return MLA_ERR_UNSUPPORTED.
 */
int mla_stream_read(const void* src, size_t bytes, void* sink, void* stream);


/*
 * mla_out_proj -- each head's value up-projection applied after aggregation
 * (V2 analysis page, section 6.1: per-head aggregation first, then the head's
 * own matrix; the heads' matrices cannot be summed):
 *   o[n][h][:] = W_UV[h] u[n][h][:]
 *   u    : [n_tok][H][d_c]  dtype u_dt (F32 or BF16), row stride
 *          u_row_stride (0: d_c)
 *   w_uv : [H][d_h][d_c]    dtype w_dt (F32 or BF16; F32 requires u_dt F32),
 *          packed
 *   o    : [n_tok][H][d_h]  dtype o_dt (F32 or BF16), row stride
 *          o_row_stride (0: d_h)
 * Supported: d_h = 128, d_c = 512, 16-byte aligned tensors and rows (else
 * MLA_ERR_UNSUPPORTED); a row stride that is negative or below the row
 * length is MLA_ERR_SHAPE. fp32 accumulation.
 */
int mla_out_proj(const void* u, const void* w_uv, void* o, int u_dt, int w_dt,
                 int o_dt, int n_tok, int H, int d_h, int d_c, int64_t u_row_stride,
                 int64_t o_row_stride, void* stream);

/*
 * Arguments of the cache append: the step that puts each new token's cache
 * entry into the paged pools before attention. Each token contributes its
 * joint KV latent c (d_c = 512) and its shared rope key k^R (d_R = 64): the
 * 576 elements that join the cache (V2 analysis page, section 1.3, and the
 * walk through one token's path in section 6.3). The latent passes through
 * an RMSNorm after the down-projection (same page, section 1.2: the report
 * puts an RMSNorm after the compressed latents; its gain is not given, so it
 * is an argument here). The rope key is rotated at the token's own position
 * and cached already rotated (section 6, third absorption condition).
 */
typedef struct mla_append_args {
  int32_t n_tok;              /* new tokens (>= 0; 0 launches nothing) */
  int32_t B;                  /* sequences = rows of block_table (>= 1) */
  int32_t d_c, d_r;           /* must be 512 and 64 */
  int32_t page_size;          /* must be 64 */
  int32_t n_pages;            /* pages in each pool (>= 1) */
  int32_t max_pages_per_seq;  /* columns of block_table (>= 1) */
  int32_t c_dt, k_dt;         /* input dtypes: F32 or BF16 */
  int32_t ckv_dt, kr_dt;      /* pool dtypes: ckv F32, BF16 or FP8_E4M3; kr F32 or BF16 */
  int32_t normalize;          /* 1: RMSNorm the latent before storing it; 0: store it as given */
  float rms_eps;              /* RMSNorm epsilon (>= 0, finite) */
  int32_t reserved0;          /* must be 0 */
  double rope_base;           /* > 0; angles pos * base^(-2i/64), as mla_rope */
  const double* rope_theta;   /* DEVICE fp64 [d_r / 2] per-pair frequencies (e.g. YaRN,
                                 mla_yarn_frequencies), or NULL for base^(-2i/64) */
  const void* c_in;           /* [n_tok][d_c] dtype c_dt: latent of each new token */
  const void* k_in;           /* [n_tok][d_r] dtype k_dt: its rope key, NOT rotated */
  const float* rms_gain;      /* [d_c] fp32 gain, or NULL for gain 1 (used iff normalize) */
  const int32_t* seq;         /* [n_tok] sequence b of each new token */
  const int32_t* pos;         /* [n_tok] its position s in the sequence */
  const int32_t* block_table; /* [B][max_pages_per_seq] page ids, as for decode */
  void* ckv;                  /* [n_pages][64][d_c] latent pool, dtype ckv_dt */
  float* ckv_scale;           /* [n_pages][64] per-token scales iff ckv_dt == FP8_E4M3 */
  void* kr;                   /* [n_pages][64][d_r] rotated-key pool, dtype kr_dt */
} mla_append_args;

/*
 * mla_cache_append -- write n_tok new tokens into the paged pools.
 * Token n goes to page block_table[seq[n]][pos[n] / 64], slot pos[n] % 64:
 *   c = c_in[n]; if normalize:
 *       c_j = c_j / sqrt(sum_j c_j^2 / 512 + rms_eps) * gain_j       (fp32)
 *   ckv[page][slot] = c stored as ckv_dt:
 *       F32 as is; BF16 rounded to nearest even;
 *       FP8_E4M3: scale = fp32(max_j |c_j|) / 448 (fp32 division; 1 when
 *       every c_j is 0), code_j = E4M3FN(fp32(c_j / scale)) rounded to
 *       nearest even and saturated at +-448, ckv_scale[page][slot] = scale
 *   kr[page][slot] = k_in[n] rotated at pos[n] (pairs (2i, 2i+1), angle,
 *       cos, sin and rotation in fp64, rounded to fp32, then to bf16 for a
 *       BF16 pool), as mla_rope computes it (mla_rope_freq when rope_theta
 *       is given).
 * With normalize = 0 and finite inputs the stored latent codes and scales
 * are exactly those of the rule above. A token whose seq, position or page
 * id is out of range writes nothing. Two tokens that address the same slot
 * race (the result is one of them, unspecified). Inputs must be finite.
 */
int mla_cache_append(const mla_append_args* args, void* stream);

/*
 * mla_expand_kv -- the expanded keys and values of prefill (V2 analysis
 * page, section 6.1: training and long-prompt prefill expand the latents per
 * head and run ordinary attention; the expansion lives only inside the
 * current block):
 *   k_nope[n][h][:] = W_UK[h] c[n],  v[n][h][:] = W_UV[h] c[n]
 *   c            : [n_tok][d_c]     dtype c_dt (F32 or BF16), the latents
 *   w_uk, w_uv   : [H][d_h][d_c]    dtype w_dt (BF16, or F32 with F32 c and outputs)
 *   k_nope, v    : [n_tok][H][d_h]  dtype out_dt (F32 or BF16)
 * Supported: d_h = 128, d_c = 512, 16-byte aligned tensors (else
 * MLA_ERR_UNSUPPORTED); fp32 accumulation (as mla_out_proj).
 */
int mla_expand_kv(const void* c, const void* w_uk, const void* w_uv, void* k_nope, void* v,
                  int c_dt, int w_dt, int out_dt, int n_tok, int H, int d_h, int d_c,
                  void* stream);

/*
 * mla_prefill_attn -- causal attention on expanded keys (V2 analysis page,
 * section 6.1; the same function as the absorbed decode in exact
 * arithmetic). Head h's key for token s is [k_nope[s][h] ; k_rope[s]]
 * (d_h + d_r = 192 values; the rope key is shared by the heads, section 1.3),
 * its value v[s][h] (128 values). Query i of sequence b sits at position
 * n_kv - n_q + i (the queries are the last n_q tokens) and attends to keys
 * s <= n_kv - n_q + i:
 *   o[b][i][h] = sum_s softmax_s(scale * (q_nope.k_nope_s + q_rope.k_rope_s)) v_s
 *   q_nope : [B][n_q][H][d_h]  BF16      q_rope : [B][n_q][H][d_r] BF16 (rotated)
 *   k_nope : [B][n_kv][H][d_h] BF16      k_rope : [B][n_kv][d_r]   BF16 (rotated)
 *   v      : [B][n_kv][H][d_h] BF16
 *   o      : [B][n_q][H][d_h]  dtype o_dt (F32 or BF16)
 *   lse    : [B][n_q][H] fp32 natural-log sum of exp(scores), or NULL
 * Supported: d_h = 128, d_r = 64, 1 <= n_q <= n_kv, H <= 65536, 16-byte
 * aligned tensors (else MLA_ERR_UNSUPPORTED). bf16 MFMA, fp32 softmax and
 * accumulation.
 */
int mla_prefill_attn(const void* q_nope, const void* q_rope, const void* k_nope,
                     const void* k_rope, const void* v, void* o, float* lse, int o_dt, int B,
                     int n_q, int n_kv, int H, int d_h, int d_r, float softmax_scale,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
