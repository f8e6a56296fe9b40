"""The C-ABI library on the host (no GPU needed): it loads, exports every symbol
include/mla.h declares, and its host-side planner and argument checks behave.
Nothing here launches a kernel: every decode call below is rejected by the
host checks before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mla_latent_kv_35_amd", "libmla.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmla.so not built")


def header_functions():
    txt = open(os.path.join(ROOT, "include", "mla.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", txt)))


@pytest.fixture(scope="module")
def B():
    from mla_latent_kv_35_amd import binding
    return binding


def test_exports_every_declared_symbol(B):
    declared = header_functions()
    assert declared == sorted(B.EXPORTED)
    lib = ctypes.CDLL(LIB)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(B):
    assert B.abi_version() == 2
    for code in range(7):
        assert B.lib().mla_status_str(code).decode().startswith("MLA_")
    assert b"unknown" in B.lib().mla_status_str(99)


def _args(mod, **kw):
    a = mod.DecodeArgs()
    a.B, a.T, a.H, a.d_c, a.d_r = 32, 1, 128, 512, 64
    a.page_size, a.n_pages, a.max_pages_per_seq, a.max_seq_len = 64, 2048, 64, 4096
    a.q_dt = a.ckv_dt = a.kr_dt = a.out_dt = mod.MLA_BF16
    a.split_tokens, a.total_tokens, a.softmax_scale = 0, 0, 192 ** -0.5
    a.heads_per_wg, a.q_lat_stride, a.q_rope_stride = 0, 0, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_plan_for_the_five_workloads(B):
    # DeepSeek-V2 layer (bf16 pool: 128-row groups): 32 (sequence, group)
    # pairs x 8 splits = 256 units
    assert B.decode_plan(_args(B))[:2] == (512, 8)
    # 128K: 4 pairs x 64 splits
    assert B.decode_plan(_args(B, B=4, n_pages=8192, max_pages_per_seq=2048,
                                   max_seq_len=131072))[:2] == (2048, 64)
    # two-token fp8: 2 row groups of 128 x 128 sequences, no split
    st, ns, ws = B.decode_plan(_args(B, B=128, T=2, ckv_dt=B.MLA_FP8_E4M3, n_pages=16384,
                                     max_pages_per_seq=128, max_seq_len=8192))
    assert ns == 1 and ws == 0
    # ragged: planned from the token total, about two units per CU
    st, ns, ws = B.decode_plan(_args(B, B=64, n_pages=16522, max_pages_per_seq=497,
                                     max_seq_len=31804, total_tokens=1055283))
    assert st % 64 == 0 and ns == -(-31804 // st)
    parts = 64 * ns * 128
    # bf16 output: bf16 u per partial row, then fp32 (m, l)
    assert ws == ((parts * 512 * 2 + 255) // 256) * 256 + ((parts * 8 + 255) // 256) * 256
    # fp32 output from the same pool: fp32 U
    _, _, ws32 = B.decode_plan(_args(B, B=64, n_pages=16522, max_pages_per_seq=497,
                                     max_seq_len=31804, total_tokens=1055283, out_dt=B.MLA_F32))
    assert ws32 == ((parts * 512 * 4 + 255) // 256) * 256 + ((parts * 8 + 255) // 256) * 256
    # fp32 tiny
    st, ns, _ = B.decode_plan(_args(B, B=1, H=16, q_dt=0, ckv_dt=0, kr_dt=0, out_dt=0,
                                    n_pages=4, max_pages_per_seq=4, max_seq_len=256))
    assert st % 64 == 0 and ns == -(-256 // st)


@pytest.mark.parametrize("field,value,status", [
    ("T", 3, 4), ("d_c", 256, 4), ("page_size", 32, 4), ("max_seq_len", 0, 2),
    ("max_seq_len", 64 * 64 + 1, 2), ("split_tokens", 100, 2), ("split_tokens", 65536 + 64, 4),
    ("heads_per_wg", -1, 2), ("heads_per_wg", 64, 4), ("heads_per_wg", 1, 4),
    ("q_lat_stride", -1, 2), ("q_lat_stride", 500, 2), ("q_lat_stride", 516, 4),
    ("q_rope_stride", -8, 2), ("q_rope_stride", 60, 2), ("q_rope_stride", 68, 4),
    ("q_lat_stride", 1 << 41, 2),
    ("softmax_scale", 0.0, 2), ("kr_dt", 0, 3), ("ckv_dt", 7, 3), ("B", 0, 2),
])
def test_plan_rejects_bad_shapes(B, field, value, status):
    # a split of at most 1024 pages (65536 tokens): the split kernel keeps its page ids in LDS
    st = B.lib().mla_decode_plan(ctypes.byref(_args(B, **{field: value})), None, None, None, None)
    assert st == status


def test_plan_reports_rows_per_workgroup_and_accepts_strides(B):
    # the kernel's own rows per workgroup: bf16 and fp8 pools 128, fp32 1
    for kw, rows in ((dict(), 128), (dict(ckv_dt=B.MLA_FP8_E4M3), 128),
                     (dict(q_dt=0, ckv_dt=0, kr_dt=0, out_dt=0), 1)):
        assert B.decode_plan_full(_args(B, **kw))[2] == rows
        # naming it explicitly is the same plan
        assert B.decode_plan_full(_args(B, heads_per_wg=rows, **kw)) == B.decode_plan_full(_args(B, **kw))
    # strided query rows (e.g. q_lat and q_rope inside one [B*T][H][576] tensor) plan alike
    assert B.decode_plan_full(_args(B, q_lat_stride=576, q_rope_stride=576)) == \
        B.decode_plan_full(_args(B))


def test_decode_rejects_before_launch(B):
    fake = 0x1000
    a = _args(B)
    # null pointers
    assert B.lib().mla_decode_paged(ctypes.byref(a), None) == 1
    for name in ("q_lat", "q_rope", "ckv", "kr", "block_table", "seq_lens", "out"):
        setattr(a, name, fake)
    # the plan needs a workspace (4 splits) and none is given
    assert B.lib().mla_decode_paged(ctypes.byref(a), None) == 5
    a.workspace, a.workspace_bytes = fake, 16
    assert B.lib().mla_decode_paged(ctypes.byref(a), None) == 5
    # fp8 without scales
    a.ckv_dt = B.MLA_FP8_E4M3
    assert B.lib().mla_decode_paged(ctypes.byref(a), None) == 1
    assert B.lib().mla_decode_paged(None, None) == 1


def test_dense_entry_points_reject_before_launch(B):
    L = B.lib()
    assert L.mla_absorb_q(None, None, None, 1, 1, 4, 128, 128, 512, 0, 0, None) == 1
    assert L.mla_absorb_q(None, None, None, 1, 1, 4, 128, 64, 512, 0, 0, None) == 4
    assert L.mla_absorb_q(None, None, None, 0, 1, 4, 128, 128, 512, 0, 0, None) == 3
    assert L.mla_absorb_q(None, None, None, 1, 1, 0, 128, 128, 512, 0, 0, None) == 0   # empty
    assert L.mla_rope(None, None, 1, None, 4, 128, 63, 10000.0, 0, 0, 0, 0, None) == 4
    assert L.mla_rope(None, None, 1, None, 4, 128, 64, -1.0, 0, 0, 0, 0, None) == 2
    assert L.mla_rope(None, None, 1, None, 4, 128, 64, 10000.0, 0, 0, 0, 0, None) == 1
    assert L.mla_out_proj(None, None, None, 1, 0, 1, 4, 128, 128, 512, 0, 0, None) == 3
    assert L.mla_out_proj(None, None, None, 1, 1, 1, -1, 128, 128, 512, 0, 0, None) == 2


def test_stride_arguments_are_checked_before_launch(B):
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    # absorb: (q_row_stride, out_row_stride); bf16 rows must stay 16-byte aligned
    absorb = lambda qs, os_: L.mla_absorb_q(None, None, None, 1, 1, 4, 8, 128, 512, qs, os_, None)
    assert absorb(192, 576) == 1          # accepted; then the null tensors are rejected
    assert absorb(-1, 0) == 2
    assert absorb(64, 0) == 2             # shorter than a 128-element row
    assert absorb(0, 500) == 2
    assert absorb(132, 0) == 4            # 264 bytes: misaligned rows
    assert absorb(0, 516) == 4
    assert absorb(1 << 41, 0) == 2
    # fp32 rows: a multiple of 4 elements
    assert L.mla_absorb_q(None, None, None, 0, 0, 4, 8, 128, 512, 132, 0, None) == 1
    assert L.mla_absorb_q(None, None, None, 0, 0, 4, 8, 128, 512, 130, 0, None) == 4
    # out_proj: (u_row_stride, o_row_stride)
    outp = lambda us, os_: L.mla_out_proj(None, None, None, 1, 1, 1, 4, 8, 128, 512, us, os_, None)
    assert outp(576, 192) == 1
    assert outp(100, 0) == 2
    assert outp(0, 120) == 2
    assert outp(0, 132) == 4
    # rope: (in_tok, in_head, out_tok, out_head), any strides >= 0; output
    # vectors must not overlap; in place needs the same strides
    rope = lambda x, y, *st: L.mla_rope(x, y, 1, None, 4, 8, 64, 1e4, *st, None)
    assert rope(None, None, 8 * 192, 192, 0, 0) == 1
    assert rope(None, None, 3, 70, 0, 0) == 1             # odd input strides are fine
    assert rope(None, None, -1, 0, 0, 0) == 2
    assert rope(None, None, 0, 0, 0, 32) == 2             # heads overlap
    assert rope(None, None, 0, 0, 256, 64) == 2           # tokens overlap
    assert rope(None, None, 0, 0, 64, 256) == 1           # tokens inside heads: disjoint
    assert rope(fake, fake, 0, 0, 8 * 192, 192) == 2      # in place with other strides
    assert rope(fake, fake, 8 * 192, 192, 8 * 192, 192) == 1
    assert L.mla_rope_freq(None, None, 1, None, 4, 8, 64, None, 0, 0, 0, 32, None) == 2
    # absorb_q_rope: (q_row, out_row, rope_row, rot_row)
    aqr = lambda *st: L.mla_absorb_q_rope(None, None, None, 1, 1, None, None, 1, None, 4, 8, 128,
                                          512, 64, 1e4, None, *st, None)
    assert aqr(192, 0, 192, 0) == 1
    assert aqr(0, 0, -64, 0) == 2
    assert aqr(0, 0, 0, 32) == 2
    assert aqr(130, 0, 0, 0) == 4


def _append_args(mod, **kw):
    a = mod.AppendArgs()
    a.n_tok, a.B, a.d_c, a.d_r, a.page_size = 4, 2, 512, 64, 64
    a.n_pages, a.max_pages_per_seq = 8, 4
    a.c_dt = a.k_dt = a.ckv_dt = a.kr_dt = mod.MLA_BF16
    a.normalize, a.rms_eps, a.reserved0, a.rope_base = 0, 0.0, 0, 10000.0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("n_tok", -1, 2), ("B", 0, 2), ("n_pages", 0, 2), ("max_pages_per_seq", 0, 2),
    ("reserved0", 1, 2), ("d_c", 256, 4), ("d_r", 32, 4), ("page_size", 16, 4),
    ("c_dt", 2, 3), ("k_dt", 2, 3), ("kr_dt", 2, 3), ("ckv_dt", 5, 3),
    ("normalize", 2, 2), ("rms_eps", -1.0, 2), ("rms_eps", float("inf"), 2),
    ("rope_base", 0.0, 2), ("max_pages_per_seq", 1 << 26, 2),
])
def test_append_rejects_bad_arguments(B, field, value, status):
    assert B.lib().mla_cache_append(ctypes.byref(_append_args(B, **{field: value})), None) == status


def test_append_rejects_before_launch(B):
    L = B.lib()
    assert L.mla_cache_append(None, None) == 1
    a = _append_args(B)
    assert L.mla_cache_append(ctypes.byref(a), None) == 1          # null tensors
    a.n_tok = 0
    assert L.mla_cache_append(ctypes.byref(a), None) == 0          # empty: no-op
    fake = 0x1000
    a = _append_args(B, ckv_dt=B.MLA_FP8_E4M3)
    for name in ("c_in", "k_in", "seq", "pos", "block_table", "ckv", "kr"):
        setattr(a, name, fake)
    assert L.mla_cache_append(ctypes.byref(a), None) == 1          # fp8 without scales
    a.ckv_dt = B.MLA_BF16
    a.c_in = fake + 8                                              # misaligned latent rows
    assert L.mla_cache_append(ctypes.byref(a), None) == 4


def test_rope_freq_rejects_before_launch(B):
    L = B.lib()
    f = lambda *a: L.mla_rope_freq(*a, 0, 0, 0, 0, None)
    assert f(None, None, 1, None, 4, 128, 63, None) == 4
    assert f(None, None, 2, None, 4, 128, 64, None) == 3
    assert f(None, None, 1, None, 4, 128, 64, None) == 1
    assert f(None, None, 1, None, 0, 128, 64, None) == 0    # empty: no-op
    assert f(None, None, 1, None, -1, 128, 64, None) == 2


def test_absorb_q_rope_rejects_before_launch(B):
    L = B.lib()
    # (q_nope, w_uk, q_lat, q_dt, out_dt, q_rope, q_rot, rope_dt, pos, n_tok, H, d_h, d_c, d_r,
    #  base, theta, four packed row strides, stream)
    f = lambda *a: L.mla_absorb_q_rope(*a[:-1], 0, 0, 0, 0, a[-1])
    assert f(None, None, None, 1, 1, None, None, 1, None, 4, 128, 128, 512, 64, 1e4, None, None) == 1
    assert f(None, None, None, 1, 1, None, None, 1, None, 4, 128, 64, 512, 64, 1e4, None, None) == 4
    assert f(None, None, None, 1, 1, None, None, 1, None, 4, 128, 128, 512, 63, 1e4, None, None) == 4
    assert f(None, None, None, 0, 1, None, None, 1, None, 4, 128, 128, 512, 64, 1e4, None, None) == 3
    assert f(None, None, None, 1, 1, None, None, 2, None, 4, 128, 128, 512, 64, 1e4, None, None) == 3
    assert f(None, None, None, 1, 1, None, None, 1, None, 4, 128, 128, 512, 64, -1., None, None) == 2
    assert f(None, None, None, 1, 1, None, None, 1, None, -1, 128, 128, 512, 64, 1e4, None, None) == 2
    assert f(None, None, None, 1, 1, None, None, 1, None, 0, 128, 128, 512, 64, 1e4, None, None) == 0


def test_dense_entry_points_reject_misaligned_pointers(B):
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    assert L.mla_absorb_q(odd, fake, fake, 0, 0, 4, 8, 128, 512, 0, 0, None) == 4
    assert L.mla_out_proj(fake, odd, fake, 0, 0, 0, 4, 8, 128, 512, 0, 0, None) == 4
    assert L.mla_expand_kv(fake, fake, fake, fake, odd, 0, 0, 0, 4, 8, 128, 512, None) == 4
    assert L.mla_absorb_q_rope(fake, fake, odd, 1, 1, fake, fake, 1, fake, 4, 8, 128, 512, 64,
                               1e4, None, 0, 0, 0, 0, None) == 4


def test_stream_read_rejects_misaligned(B):
    lib = B.lib()
    # host-side checks only: no launch happens for these
    assert lib.mla_stream_read(None, 16, 16, None) == 1    # MLA_ERR_NULL
    assert lib.mla_stream_read(16, 24, 16, None) == 4      # size not a multiple of 16
    assert lib.mla_stream_read(8, 16, 16, None) == 4       # src not 16-byte aligned
    assert lib.mla_stream_read(16, 16, 8, None) == 4       # sink not 16-byte aligned
    assert lib.mla_stream_read(16, 0, 16, None) == 0       # nothing to read
