// C ABI of libmla.so: host-side argument checks, the split planner and the
// kernel launches. Declarations and semantics: include/mla.h.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "mla_extra.h"

namespace mla {
namespace {

constexpr int kNumCu = 256;           // MI355X compute units
constexpr int kMaxSplits = 1024;      // splits per sequence the combine kernel merges
constexpr size_t kWsAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool is_float_dt(int dt) { return dt == MLA_F32 || dt == MLA_BF16; }
int elt_bytes(int dt) { return dt == MLA_F32 ? 4 : dt == MLA_BF16 ? 2 : 1; }

// Strides beyond this many elements are rejected (offsets stay far inside 64 bits).
constexpr int64_t kMaxStride = int64_t(1) << 40;

// Row stride of rows `len` elements long whose starts must stay 16-byte
// aligned: 0 selects len; negative, shorter than a row or huge is a shape
// error, a misaligned one unsupported.
int row_stride(int64_t given, int len, int dt, long* out) {
  if (given < 0 || given > kMaxStride) return MLA_ERR_SHAPE;
  const int64_t r = given == 0 ? len : given;
  if (r < len) return MLA_ERR_SHAPE;
  if ((r * elt_bytes(dt)) % 16 != 0) return MLA_ERR_UNSUPPORTED;
  *out = (long)r;
  return MLA_OK;
}

// Token and head strides of rope vectors (0 selects the packed ones);
// out_vecs: the vectors are written, so they must not overlap one another
// (checked for the nested orders: heads inside tokens or tokens inside heads).
int vec_strides(int64_t tok, int64_t head, int n_tok, int n_heads, int d, bool out_vecs,
                VecStrides* st) {
  if (tok < 0 || head < 0 || tok > kMaxStride || head > kMaxStride) return MLA_ERR_SHAPE;
  st->tok = (long)(tok == 0 ? (int64_t)n_heads * d : tok);
  st->head = (long)(head == 0 ? d : head);
  if (out_vecs) {
    const int64_t t = n_tok > 1 ? st->tok : INT64_MAX, h = n_heads > 1 ? st->head : INT64_MAX;
    const bool heads_inner = h >= d && (n_tok == 1 || t >= (int64_t)(n_heads - 1) * h + d);
    const bool tokens_inner = t >= d && (n_heads == 1 || h >= (int64_t)(n_tok - 1) * t + d);
    if (!heads_inner && !tokens_inner) return MLA_ERR_SHAPE;
  }
  return MLA_OK;
}

// Rope input and output strides; the same memory must come with the same strides.
int rope_strides(const void* x_in, const void* x_out, int n_tok, int n_heads, int d_r,
                 int64_t in_tok, int64_t in_head, int64_t out_tok, int64_t out_head,
                 VecStrides* si, VecStrides* so) {
  int st = vec_strides(in_tok, in_head, n_tok, n_heads, d_r, false, si);
  if (st != MLA_OK) return st;
  st = vec_strides(out_tok, out_head, n_tok, n_heads, d_r, true, so);
  if (st != MLA_OK) return st;
  if (x_in == x_out && x_in && (si->tok != so->tok || si->head != so->head)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

// Query rows per workgroup of the decode kernel for this latent pool dtype.
int kernel_rows(int ckv_dt) { return ckv_dt == MLA_F32 ? 1 : 128; }

struct Plan {
  int split_tokens = 0;
  int n_split = 1;
  int rows = 1;           // query rows per workgroup (kernel_rows)
  int G = 1;              // row groups per sequence
  size_t part_u_bytes = 0;
  size_t ws_bytes = 0;
};

// Checks everything that does not need a device pointer.
int check_shape(const mla_decode_args* a) {
  if (!a) return MLA_ERR_NULL;
  if (a->B < 1 || a->H < 1 || a->T < 1) return MLA_ERR_SHAPE;
  if (a->T > 2) return MLA_ERR_UNSUPPORTED;
  if (a->d_c != kDc || a->d_r != kDr) return MLA_ERR_UNSUPPORTED;
  if (a->page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (a->n_pages < 1 || a->max_pages_per_seq < 1) return MLA_ERR_SHAPE;
  if (a->max_seq_len < a->T || (int64_t)a->max_seq_len > (int64_t)a->max_pages_per_seq * kPage)
    return MLA_ERR_SHAPE;
  if (a->split_tokens < 0 || a->split_tokens % kPage != 0) return MLA_ERR_SHAPE;
  if (a->split_tokens > kMaxSplitPages * kPage) return MLA_ERR_UNSUPPORTED;
  if (a->total_tokens < 0) return MLA_ERR_SHAPE;
  if (!(a->softmax_scale > 0.f) || !isfinite(a->softmax_scale)) return MLA_ERR_SHAPE;
  if ((int64_t)a->T * a->H > (1 << 20)) return MLA_ERR_UNSUPPORTED;
  // dtype combinations
  if (a->ckv_dt == MLA_F32) {
    if (a->kr_dt != MLA_F32 || a->q_dt != MLA_F32 || a->out_dt != MLA_F32) return MLA_ERR_DTYPE;
  } else if (a->ckv_dt == MLA_BF16) {
    if (a->kr_dt != MLA_BF16 || a->q_dt != MLA_BF16 || !is_float_dt(a->out_dt)) return MLA_ERR_DTYPE;
  } else if (a->ckv_dt == MLA_FP8_E4M3) {
    if (a->kr_dt != MLA_BF16 || a->q_dt != MLA_BF16 || !is_float_dt(a->out_dt)) return MLA_ERR_DTYPE;
  } else {
    return MLA_ERR_DTYPE;
  }
  if (a->heads_per_wg < 0) return MLA_ERR_SHAPE;
  if (a->heads_per_wg != 0 && a->heads_per_wg != kernel_rows(a->ckv_dt)) return MLA_ERR_UNSUPPORTED;
  long st;
  int e = row_stride(a->q_lat_stride, kDc, a->q_dt, &st);
  if (e != MLA_OK) return e;
  e = row_stride(a->q_rope_stride, kDr, a->q_dt, &st);
  if (e != MLA_OK) return e;
  return MLA_OK;
}

// Split partials are bf16 (the normalised u of each split) exactly when the
// output is bf16 and the MFMA kernel runs; fp32 outputs keep fp32 partials.
bool part_bf16(const mla_decode_args* a) { return a->out_dt == MLA_BF16 && a->ckv_dt != MLA_F32; }

Plan make_plan(const mla_decode_args* a) {
  Plan pl;
  const int64_t R = (int64_t)a->T * a->H;
  const int64_t Lmax = a->max_seq_len;
  const int64_t total = a->total_tokens > 0 ? a->total_tokens : (int64_t)a->B * Lmax;
  const int64_t pages_total = (total + kPage - 1) / kPage;
  const int64_t max_pages = (Lmax + kPage - 1) / kPage;
  pl.rows = kernel_rows(a->ckv_dt);
  pl.G = (int)((R + pl.rows - 1) / pl.rows);
  if (a->split_tokens > 0) {
    pl.split_tokens = a->split_tokens;
  } else if (a->ckv_dt == MLA_F32) {
    // fp32 kernel: one workgroup per (sequence, split, row); aim for ~4 per CU
    const int64_t want = (4 * kNumCu + a->B * R - 1) / (a->B * R);
    int64_t sp = (max_pages + want - 1) / want;
    pl.split_tokens = (int)(std::max<int64_t>(sp, 1) * kPage);
  } else {
    // MFMA kernels: units of (sequence, split, row group). Uniform batches
    // get one unit per CU; ragged ones two per CU, so that the uneven tails
    // balance (measured on the 64-sequence ragged batch: 1, 1.5, 3 and 4 per
    // CU were slower, each unit paying its own start of about 6 us)
    const bool ragged = total * 10 < (int64_t)a->B * Lmax * 9;
    const int64_t target = ragged ? 2 * kNumCu : kNumCu;
    int64_t unit_pages = (pl.G * pages_total + target - 1) / target;
    unit_pages = std::max<int64_t>(unit_pages, 4);
    unit_pages = std::min<int64_t>(unit_pages, max_pages);
    unit_pages = std::min<int64_t>(unit_pages, kMaxSplitPages);
    pl.split_tokens = (int)(unit_pages * kPage);
  }
  pl.n_split = (int)((Lmax + pl.split_tokens - 1) / pl.split_tokens);
  if (pl.n_split > 1) {
    const size_t parts = (size_t)a->B * pl.n_split * R;
    // bf16 output from a bf16 / fp8 cache: partials hold bf16 u = U / l
    const size_t elt = part_bf16(a) ? 2 : sizeof(float);
    pl.part_u_bytes = align_up(parts * kDc * elt, kWsAlign);
    pl.ws_bytes = pl.part_u_bytes + align_up(parts * 2 * sizeof(float), kWsAlign);
  }
  return pl;
}

}  // namespace
}  // namespace mla

// Scratch of the allocation-free decode entry point: one array per device,
// held until the process ends. Host code never uses the name itself (a
// host-side stand-in); the device address comes from hipGetSymbolAddress,
// once per device, with that device current.
namespace mla {
namespace {
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's scratch address, or nullptr when it cannot be had.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

const char* mla_status_str(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size is out of range or inconsistent";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unsupported dtype combination";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape outside what the kernels implement";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: kernel launch failed";
    default: return "unknown mla_status";
  }
}

int mla_abi_version(void) { return MLA_ABI_VERSION; }

namespace {
// Host checks shared by mla_absorb_q and mla_absorb_q_rope.
int check_absorb(int q_dt, int out_dt, int n_tok, int H, int d_h, int d_c, int64_t q_row_stride,
                 int64_t out_row_stride, long* q_rs, long* o_rs) {
  if (n_tok < 0 || H < 1) return MLA_ERR_SHAPE;
  if (d_h != kDh || d_c != kDc) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(q_dt) || !is_float_dt(out_dt)) return MLA_ERR_DTYPE;
  if (q_dt == MLA_F32 && out_dt != MLA_F32) return MLA_ERR_DTYPE;
  const int e = row_stride(q_row_stride, kDh, q_dt, q_rs);
  return e != MLA_OK ? e : row_stride(out_row_stride, kDc, out_dt, o_rs);
}
}  // namespace

int mla_absorb_q(const void* q_nope, const void* w_uk, void* q_lat, int q_dt, int out_dt,
                 int n_tok, int H, int d_h, int d_c, int64_t q_row_stride,
                 int64_t out_row_stride, void* stream) {
  long q_rs, o_rs;
  const int st = check_absorb(q_dt, out_dt, n_tok, H, d_h, d_c, q_row_stride, out_row_stride,
                              &q_rs, &o_rs);
  if (st != MLA_OK) return st;
  if (n_tok == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_NULL;
  if ((((uintptr_t)q_nope | (uintptr_t)w_uk | (uintptr_t)q_lat) & 15) != 0) return MLA_ERR_UNSUPPORTED;
  const hipError_t e = launch_absorb(q_nope, q_rs, w_uk, q_lat, o_rs, q_dt == MLA_BF16,
                                     out_dt == MLA_BF16, n_tok, H, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_rope(const void* x_in, void* x_out, int dt, const int32_t* pos, int n_tok, int n_heads,
             int d_r, double base, int64_t in_tok_stride, int64_t in_head_stride,
             int64_t out_tok_stride, int64_t out_head_stride, void* stream) {
  if (n_tok < 0 || n_heads < 1) return MLA_ERR_SHAPE;
  if (d_r < 2 || d_r > 256 || d_r % 2 != 0) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(dt)) return MLA_ERR_DTYPE;
  if (!(base > 0.0) || !isfinite(base)) return MLA_ERR_SHAPE;
  VecStrides si, so;
  const int st = rope_strides(x_in, x_out, n_tok, n_heads, d_r, in_tok_stride, in_head_stride,
                              out_tok_stride, out_head_stride, &si, &so);
  if (st != MLA_OK) return st;
  if (n_tok == 0) return MLA_OK;
  if (!x_in || !x_out || !pos) return MLA_ERR_NULL;
  const hipError_t e = launch_rope(x_in, si, x_out, so, dt == MLA_BF16, pos, n_tok, n_heads, d_r,
                                   base, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_rope_freq(const void* x_in, void* x_out, int dt, const int32_t* pos, int n_tok,
                  int n_heads, int d_r, const double* theta, int64_t in_tok_stride,
                  int64_t in_head_stride, int64_t out_tok_stride, int64_t out_head_stride,
                  void* stream) {
  if (n_tok < 0 || n_heads < 1) return MLA_ERR_SHAPE;
  if (d_r < 2 || d_r > 256 || d_r % 2 != 0) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(dt)) return MLA_ERR_DTYPE;
  VecStrides si, so;
  const int st = rope_strides(x_in, x_out, n_tok, n_heads, d_r, in_tok_stride, in_head_stride,
                              out_tok_stride, out_head_stride, &si, &so);
  if (st != MLA_OK) return st;
  if (n_tok == 0) return MLA_OK;
  if (!x_in || !x_out || !pos || !theta) return MLA_ERR_NULL;
  const hipError_t e = launch_rope(x_in, si, x_out, so, dt == MLA_BF16, pos, n_tok, n_heads, d_r,
                                   1.0, theta, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_absorb_q_rope(const void* q_nope, const void* w_uk, void* q_lat, int q_dt, int out_dt,
                      const void* q_rope, void* q_rot, int rope_dt, const int32_t* pos,
                      int n_tok, int H, int d_h, int d_c, int d_r, double base,
                      const double* theta, int64_t q_row_stride, int64_t out_row_stride,
                      int64_t rope_row_stride, int64_t rot_row_stride, void* stream) {
  long q_rs, o_rs;
  int st = check_absorb(q_dt, out_dt, n_tok, H, d_h, d_c, q_row_stride, out_row_stride, &q_rs,
                        &o_rs);
  if (st != MLA_OK) return st;
  if (d_r < 2 || d_r > 256 || d_r % 2 != 0) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(rope_dt)) return MLA_ERR_DTYPE;
  if (!theta && (!(base > 0.0) || !isfinite(base))) return MLA_ERR_SHAPE;
  // rope rows: token stride H * r, head stride r
  if (rope_row_stride < 0 || rot_row_stride < 0 || rope_row_stride > kMaxStride ||
      rot_row_stride > kMaxStride)
    return MLA_ERR_SHAPE;
  const int64_t rr = rope_row_stride ? rope_row_stride : d_r;
  const int64_t ro = rot_row_stride ? rot_row_stride : d_r;
  VecStrides si, so;
  st = rope_strides(q_rope, q_rot, n_tok, H, d_r, rr * H, rr, ro * H, ro, &si, &so);
  if (st != MLA_OK) return st;
  if (n_tok == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_lat || !q_rope || !q_rot || !pos) return MLA_ERR_NULL;
  if ((((uintptr_t)q_nope | (uintptr_t)w_uk | (uintptr_t)q_lat) & 15) != 0) return MLA_ERR_UNSUPPORTED;
  const hipStream_t s = (hipStream_t)stream;
  // the fused kernel's rope half reads and writes 16-byte slices
  const bool rope_vec = d_r == 64 && (((uintptr_t)q_rope | (uintptr_t)q_rot) & 15) == 0 &&
                        ((rr | ro) * elt_bytes(rope_dt)) % 16 == 0;
  hipError_t e;
  if (q_dt == MLA_BF16 && rope_dt == MLA_BF16 && rope_vec) {
    e = launch_absorb_rope((const uint16_t*)q_nope, q_rs, (const uint16_t*)w_uk, q_lat, o_rs,
                           out_dt == MLA_BF16, (const uint16_t*)q_rope, si, (uint16_t*)q_rot, so,
                           pos, n_tok, H, theta ? 1.0 : base, theta, s);
  } else if (q_dt == MLA_F32 && rope_dt == MLA_F32 && rope_vec) {
    e = launch_absorb_rope_f32((const float*)q_nope, q_rs, (const float*)w_uk, (float*)q_lat,
                               o_rs, (const float*)q_rope, si, (float*)q_rot, so, pos, n_tok, H,
                               theta ? 1.0 : base, theta, s);
  } else {
    e = launch_absorb(q_nope, q_rs, w_uk, q_lat, o_rs, q_dt == MLA_BF16, out_dt == MLA_BF16,
                      n_tok, H, s);
    if (e == hipSuccess)
      e = launch_rope(q_rope, si, q_rot, so, rope_dt == MLA_BF16, pos, n_tok, H, d_r,
                      theta ? 1.0 : base, theta, s);
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_yarn_frequencies(int d_r, double base, double factor, double alpha, double beta,
                         int orig_len, double* theta) {
  if (!theta) return MLA_ERR_NULL;
  if (d_r < 2 || d_r > 256 || d_r % 2 != 0) return MLA_ERR_SHAPE;
  if (!(base > 0.0) || !isfinite(base) || !(factor >= 1.0) || !isfinite(factor) ||
      !(beta > alpha) || !isfinite(alpha) || !isfinite(beta) || orig_len < 1)
    return MLA_ERR_SHAPE;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < d_r / 2; ++i) {
    const double th = pow(base, -2.0 * (double)i / (double)d_r);
    const double r = (double)orig_len * th / two_pi;     // rotations over the original window
    double g = (r - alpha) / (beta - alpha);
    g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
    theta[i] = (1.0 - g) * (th / factor) + g * th;
  }
  return MLA_OK;
}

double mla_yarn_mscale(double factor, double coef) {
  return factor <= 1.0 ? 1.0 : coef * log(factor) + 1.0;
}

int mla_decode_plan(const mla_decode_args* args, int* split_tokens, int* n_split,
                    int* heads_per_wg, size_t* workspace_bytes) {
  const int st = check_shape(args);
  if (st != MLA_OK) return st;
  const Plan pl = make_plan(args);
  if (pl.n_split > kMaxSplits) return MLA_ERR_UNSUPPORTED;
  if (split_tokens) *split_tokens = pl.split_tokens;
  if (n_split) *n_split = pl.n_split;
  if (heads_per_wg) *heads_per_wg = pl.rows;
  if (workspace_bytes) *workspace_bytes = pl.ws_bytes;
  return MLA_OK;
}

int mla_decode_paged(const mla_decode_args* a, void* stream) {
  const int st = check_shape(a);
  if (st != MLA_OK) return st;
  if (!a->q_lat || !a->q_rope || !a->ckv || !a->kr || !a->block_table || !a->seq_lens || !a->out)
    return MLA_ERR_NULL;
  if (a->ckv_dt == MLA_FP8_E4M3 && !a->ckv_scale) return MLA_ERR_NULL;
  const bool proj = a->w_uv != nullptr;
  if (proj) {
    if (!a->o) return MLA_ERR_NULL;
    if (!is_float_dt(a->w_dt) || !is_float_dt(a->o_dt)) return MLA_ERR_DTYPE;
    if (a->w_dt == MLA_F32 && (a->out_dt != MLA_F32 || a->o_dt != MLA_F32)) return MLA_ERR_DTYPE;
  }
  // every vector access of the decode kernels is 16 bytes wide
  const uintptr_t al = (uintptr_t)a->q_lat | (uintptr_t)a->q_rope | (uintptr_t)a->ckv |
                       (uintptr_t)a->kr | (uintptr_t)a->out |
                       (proj ? ((uintptr_t)a->w_uv | (uintptr_t)a->o) : 0);
  if (al % 16 != 0 || (uintptr_t)a->ckv_scale % 4 != 0 || (uintptr_t)a->lse % 4 != 0)
    return MLA_ERR_UNSUPPORTED;
  const Plan pl = make_plan(a);
  if (pl.n_split > kMaxSplits) return MLA_ERR_UNSUPPORTED;
  if (pl.n_split > 1) {
    if (!a->workspace || a->workspace_bytes < pl.ws_bytes) return MLA_ERR_WORKSPACE;
    if (((uintptr_t)a->workspace) % kWsAlign != 0) return MLA_ERR_WORKSPACE;
  }

  DecodeParams p{};
  p.q_lat = a->q_lat;
  p.q_rope = a->q_rope;
  p.ckv = a->ckv;
  p.kr = a->kr;
  p.ckv_scale = a->ckv_scale;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.out = a->out;
  p.lse = a->lse;
  p.part_u = pl.n_split > 1 ? a->workspace : nullptr;
  p.part_bf16 = part_bf16(a);
  p.part_ml = pl.n_split > 1 ? (float*)((char*)a->workspace + pl.part_u_bytes) : nullptr;
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.R = a->T * a->H;
  p.G = pl.G;
  p.n_split = pl.n_split;
  p.split_tokens = pl.split_tokens;
  p.n_pages = a->n_pages;
  p.max_pages = a->max_pages_per_seq;
  p.max_seq_len = a->max_seq_len;
  p.out_bf16 = a->out_dt == MLA_BF16;
  p.scale_log2 = a->softmax_scale * kLog2e;
  p.q_lat_stride = a->q_lat_stride ? (long)a->q_lat_stride : kDc;
  p.q_rope_stride = a->q_rope_stride ? (long)a->q_rope_stride : kDr;
  const int64_t units = (int64_t)a->B * pl.n_split * pl.G;
  if (units > (int64_t)1 << 30) return MLA_ERR_UNSUPPORTED;
  p.n_units = (int)units;
  p.per_xcd = (int)((units + kNumXcd - 1) / kNumXcd);

  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (a->ckv_dt == MLA_F32) e = launch_decode_simple_f32(p, s);
  else e = launch_decode_pipe(p, a->ckv_dt == MLA_FP8_E4M3, s);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  if (pl.n_split > 1) {
    CombineParams c{};
    c.part_u = p.part_u;
    c.part_ml = p.part_ml;
    c.part_bf16 = p.part_bf16;
    c.out = a->out;
    c.lse = a->lse;
    c.seq_lens = a->seq_lens;
    c.rows = a->B * p.R;
    c.R = p.R;
    c.T = a->T;
    c.n_split = pl.n_split;
    c.split_tokens = pl.split_tokens;
    c.max_seq_len = a->max_seq_len;
    c.max_pages = a->max_pages_per_seq;
    c.out_bf16 = p.out_bf16;
    // the fused combine + projection measured faster with up to 4 splits and
    // slower with 16 or 32 (its workgroups hold W_UV while they merge)
    if (proj && a->w_dt == MLA_BF16 && pl.n_split <= 4) {
      c.w_uv = (const uint16_t*)a->w_uv;
      c.o = a->o;
      c.o_bf16 = a->o_dt == MLA_BF16;
      c.H = a->H;
      c.n_tok = a->B * a->T;
      e = launch_combine_out(c, s);
      return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
    }
    e = launch_combine(c, s);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
  }
  if (proj) {
    e = launch_out_proj(a->out, a->w_uv, a->o, p.out_bf16, a->w_dt == MLA_BF16,
                        a->o_dt == MLA_BF16, a->B * a->T, a->H, s);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

int mla_decode_paged_noalloc(const mla_decode_args* args, void* stream) {
  if (!args) return MLA_ERR_NULL;
  const int st = check_shape(args);
  if (st != MLA_OK) return st;
  const Plan pl = make_plan(args);
  if (pl.n_split > 1 && pl.ws_bytes > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  void* const ws = scratch_ptr();
  if (!ws) return MLA_ERR_LAUNCH;
  mla_decode_args a = *args;
  a.workspace = ws;
  a.workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  return mla_decode_paged(&a, stream);
}


int mla_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return MLA_ERR_NULL;
  if (bytes % 16 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)sink % 16 != 0) return MLA_ERR_UNSUPPORTED;
  if (bytes == 0) return MLA_OK;
  return launch_stream_read(src, bytes, sink, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_out_proj(const void* u, const void* w_uv, void* o, int u_dt, int w_dt, int o_dt, int n_tok,
                 int H, int d_h, int d_c, int64_t u_row_stride, int64_t o_row_stride,
                 void* stream) {
  if (n_tok < 0 || H < 1) return MLA_ERR_SHAPE;
  if (d_h != kDh || d_c != kDc) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(u_dt) || !is_float_dt(w_dt) || !is_float_dt(o_dt)) return MLA_ERR_DTYPE;
  if (w_dt == MLA_F32 && (u_dt != MLA_F32 || o_dt != MLA_F32)) return MLA_ERR_DTYPE;
  long u_rs, o_rs;
  int st = row_stride(u_row_stride, kDc, u_dt, &u_rs);
  if (st == MLA_OK) st = row_stride(o_row_stride, kDh, o_dt, &o_rs);
  if (st != MLA_OK) return st;
  if (n_tok == 0) return MLA_OK;
  if (!u || !w_uv || !o) return MLA_ERR_NULL;
  if ((((uintptr_t)u | (uintptr_t)w_uv | (uintptr_t)o) & 15) != 0) return MLA_ERR_UNSUPPORTED;
  const hipError_t e = launch_out_proj_strided(u, (long)H * u_rs, u_rs, w_uv, o, o_rs,
                                               u_dt == MLA_BF16, w_dt == MLA_BF16,
                                               o_dt == MLA_BF16, n_tok, H, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_expand_kv(const void* c, const void* w_uk, const void* w_uv, void* k_nope, void* v,
                  int c_dt, int w_dt, int out_dt, int n_tok, int H, int d_h, int d_c,
                  void* stream) {
  if (n_tok < 0 || H < 1) return MLA_ERR_SHAPE;
  if (d_h != kDh || d_c != kDc) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(c_dt) || !is_float_dt(w_dt) || !is_float_dt(out_dt)) return MLA_ERR_DTYPE;
  if (w_dt == MLA_F32 && (c_dt != MLA_F32 || out_dt != MLA_F32)) return MLA_ERR_DTYPE;
  if (n_tok == 0) return MLA_OK;
  if (!c || !w_uk || !w_uv || !k_nope || !v) return MLA_ERR_NULL;
  if ((((uintptr_t)c | (uintptr_t)w_uk | (uintptr_t)w_uv | (uintptr_t)k_nope | (uintptr_t)v) & 15) != 0)
    return MLA_ERR_UNSUPPORTED;
  const hipStream_t s = (hipStream_t)stream;
  for (int i = 0; i < 2; ++i) {
    const void* w = i == 0 ? w_uk : w_uv;
    void* out = i == 0 ? k_nope : v;
    // bf16 weights: one GEMM over all heads, [n_tok][512] x [H*128][512]^T
    const hipError_t e =
        w_dt == MLA_BF16
            ? launch_gemm_nt(c, c_dt == MLA_BF16, (const uint16_t*)w, out, out_dt == MLA_BF16,
                             n_tok, H * kDh, kDc, s)
            : launch_out_proj_strided(c, kDc, 0, w, out, kDh, 0, 0, 0, n_tok, H, s);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

int mla_prefill_attn(const void* q_nope, const void* q_rope, const void* k_nope,
                     const void* k_rope, const void* v, void* o, float* lse, int o_dt, int B,
                     int n_q, int n_kv, int H, int d_h, int d_r, float softmax_scale,
                     void* stream) {
  if (B < 1 || H < 1 || n_q < 1 || n_kv < n_q) return MLA_ERR_SHAPE;
  if (d_h != kDh || d_r != kDr) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(o_dt)) return MLA_ERR_DTYPE;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  // the kernel's per-lane copy offsets (63 keys x H x 256 B) are 32-bit
  if (H > 65536 || (int64_t)B * H * ((n_q + 255) / 256) > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (!q_nope || !q_rope || !k_nope || !k_rope || !v || !o) return MLA_ERR_NULL;
  const uintptr_t al = (uintptr_t)q_nope | (uintptr_t)q_rope | (uintptr_t)k_nope |
                       (uintptr_t)k_rope | (uintptr_t)v | (uintptr_t)o;
  if (al % 16 != 0) return MLA_ERR_UNSUPPORTED;
  PrefillParams p{};
  p.q_nope = q_nope;
  p.q_rope = q_rope;
  p.k_nope = k_nope;
  p.k_rope = k_rope;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.n_q = n_q;
  p.n_kv = n_kv;
  p.H = H;
  p.o_bf16 = o_dt == MLA_BF16;
  p.scale_log2 = softmax_scale * kLog2e;
  const hipError_t e = launch_prefill(p, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_cache_append(const mla_append_args* a, void* stream) {
  if (!a) return MLA_ERR_NULL;
  if (a->n_tok < 0 || a->B < 1 || a->n_pages < 1 || a->max_pages_per_seq < 1 || a->reserved0 != 0)
    return MLA_ERR_SHAPE;
  if (a->d_c != kDc || a->d_r != kDr || a->page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (!is_float_dt(a->c_dt) || !is_float_dt(a->k_dt) || !is_float_dt(a->kr_dt) ||
      !(is_float_dt(a->ckv_dt) || a->ckv_dt == MLA_FP8_E4M3))
    return MLA_ERR_DTYPE;
  if (a->normalize != 0 && a->normalize != 1) return MLA_ERR_SHAPE;
  if (!(a->rms_eps >= 0.f) || !isfinite(a->rms_eps)) return MLA_ERR_SHAPE;
  if (!(a->rope_base > 0.0) || !isfinite(a->rope_base)) return MLA_ERR_SHAPE;
  if ((int64_t)a->max_pages_per_seq * kPage > INT32_MAX) return MLA_ERR_SHAPE;
  if (a->n_tok == 0) return MLA_OK;
  if (!a->c_in || !a->k_in || !a->seq || !a->pos || !a->block_table || !a->ckv || !a->kr)
    return MLA_ERR_NULL;
  if (a->ckv_dt == MLA_FP8_E4M3 && !a->ckv_scale) return MLA_ERR_NULL;
  // the latent rows are read and written with 16-byte (8-byte for fp8) vector accesses
  const uintptr_t al = (uintptr_t)a->c_in | (uintptr_t)a->ckv;
  if (al % (a->ckv_dt == MLA_FP8_E4M3 ? 8 : 16) != 0 || (uintptr_t)a->c_in % 16 != 0 ||
      ((uintptr_t)a->k_in | (uintptr_t)a->kr) % 4 != 0)
    return MLA_ERR_UNSUPPORTED;
  AppendParams p{};
  p.c_in = a->c_in;
  p.k_in = a->k_in;
  p.rms_gain = a->rms_gain;
  p.seq = a->seq;
  p.pos = a->pos;
  p.block_table = a->block_table;
  p.ckv = a->ckv;
  p.ckv_scale = a->ckv_scale;
  p.kr = a->kr;
  p.n_tok = a->n_tok;
  p.B = a->B;
  p.n_pages = a->n_pages;
  p.max_pages = a->max_pages_per_seq;
  p.c_bf16 = a->c_dt == MLA_BF16;
  p.k_bf16 = a->k_dt == MLA_BF16;
  p.kr_bf16 = a->kr_dt == MLA_BF16;
  p.ckv_dt = a->ckv_dt == MLA_F32 ? 0 : a->ckv_dt == MLA_BF16 ? 1 : 2;
  p.normalize = a->normalize;
  p.rms_eps = a->rms_eps;
  p.rope_base = a->rope_base;
  p.rope_theta = a->rope_theta;
  const hipError_t e = launch_append(p, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // extern "C"
