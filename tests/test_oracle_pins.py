"""Pins that tie the CPU oracle to the pages and to mathematics other than itself.

Each test names what fixes the expected value: a value printed on the pages
(tests/golden/), a closed form, a library routine the definition reduces to,
brute force on tiny inputs, or an invariant. They are chosen so that a
dropped term, a wrong sign or index, a transposed operand or a wrong softmax
scale in the oracle fails at least one of them.
"""
import cmath
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_latent_kv_35_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# stored formats
# --------------------------------------------------------------------------

def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))


def test_e4m3fn_decode_exhaustive_vs_torch_and_format_points():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.all((np.isnan(ours) & np.isnan(ref)) | (ours == ref))
    # points fixed by the OCP E4M3FN definition
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0      # largest finite
    assert ours[0x01] == 2.0 ** -9                            # smallest subnormal
    assert ours[0x08] == 2.0 ** -6                            # smallest normal
    assert ours[0x38] == 1.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.sum(np.isnan(ours)) == 2                        # no infinities


def test_fp8_store_roundtrip_bound():
    """Generator quantisation: |x - code*scale| <= half an fp8 ulp * scale, and
    the absmax element of each token lands on +-448."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 512))
    codes, scale = synth.quantize_fp8_per_token(x)
    deq = O.stored_to_f64(codes, "fp8", scale)
    x32 = x.astype(np.float32).astype(np.float64)
    y = x32 / scale[:, None]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3)
    assert np.all(np.abs(deq - x32) <= 0.5 * ulp * scale[:, None] * (1 + 1e-6) + 1e-12)
    top = np.abs(O.e4m3fn_to_f64(codes)).max(axis=1)
    assert np.all(top == 448.0)


# --------------------------------------------------------------------------
# RoPE: pairs (2i, 2i+1) rotated at position n (CSDN page, section 2(3))
# --------------------------------------------------------------------------

POSITIONS = [0, 1, 4095, 4096, 32767, 131071]


def test_rope_identity_at_zero_and_norm_preserved():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((len(POSITIONS), 64))
    y = O.rope_rotate(x, np.array(POSITIONS))
    assert np.array_equal(y[0], x[0])
    for i in range(len(POSITIONS)):
        assert abs(np.linalg.norm(y[i]) - np.linalg.norm(x[i])) < 1e-12 * np.linalg.norm(x[i])


def test_rope_closed_form_unit_vectors():
    """A unit vector on coordinate 2i at position p goes to (cos p*th_i, sin p*th_i)
    on coordinates (2i, 2i+1), with th_i = 10000^(-2i/64); the first pair has th_0 = 1."""
    for p in POSITIONS:
        for i in (0, 1, 17, 31):
            e = np.zeros(64)
            e[2 * i] = 1.0
            y = O.rope_rotate(e[None, :], np.array([p]))[0]
            ang = p * 10000.0 ** (-(2.0 * i) / 64.0)
            assert abs(y[2 * i] - math.cos(ang)) < 1e-12
            assert abs(y[2 * i + 1] - math.sin(ang)) < 1e-12
            others = np.delete(y, [2 * i, 2 * i + 1])
            assert np.all(others == 0.0)
    e = np.zeros(64)
    e[0] = 1.0
    y = O.rope_rotate(e[None, :], np.array([1]))[0]
    assert abs(y[0] - math.cos(1.0)) < 1e-15 and abs(y[1] - math.sin(1.0)) < 1e-15


def test_rope_matches_complex_multiplication():
    """Pairing (2i, 2i+1) as the complex number x_2i + j x_2i+1, RoPE is
    multiplication by exp(j p theta_i) (textbook form)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((len(POSITIONS), 64))
    pos = np.array(POSITIONS)
    rot = np.array([[cmath.exp(1j * p * 10000.0 ** (-2.0 * i / 64.0)) for i in range(32)]
                    for p in POSITIONS])
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * rot
    y = O.rope_rotate(x, pos)
    assert np.max(np.abs(y[:, 0::2] - z.real)) < 1e-12
    assert np.max(np.abs(y[:, 1::2] - z.imag)) < 1e-12


def test_rope_relative_position():
    """<R(m) q, R(n) k> = <R(m - n) q, k>."""
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 64))
    for m, n in [(5, 3), (4095, 17), (131071, 131000), (32767, 0)]:
        lhs = O.rope_rotate(q[None], np.array([m]))[0] @ O.rope_rotate(k[None], np.array([n]))[0]
        rhs = O.rope_rotate(q[None], np.array([m - n]))[0] @ k
        assert abs(lhs - rhs) < 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))


# --------------------------------------------------------------------------
# absorption and out-projection: brute force on tiny sizes
# --------------------------------------------------------------------------

def test_absorb_and_out_proj_brute_force():
    rng = np.random.default_rng(4)
    N, H, dh, dc = 2, 3, 4, 5
    q = rng.standard_normal((N, H, dh))
    wuk = rng.standard_normal((H, dh, dc))
    wuv = rng.standard_normal((H, dh, dc))
    u = rng.standard_normal((N, H, dc))
    ql = O.absorb_q(q, wuk)
    o = O.out_proj(u, wuv)
    for n in range(N):
        for h in range(H):
            for d in range(dc):
                ref = math.fsum(wuk[h][j][d] * q[n][h][j] for j in range(dh))
                assert abs(ql[n, h, d] - ref) < 1e-12
            for j in range(dh):
                ref = math.fsum(wuv[h][j][d] * u[n][h][d] for d in range(dc))
                assert abs(o[n, h, j] - ref) < 1e-12


def test_attend_brute_force_tiny():
    """Scores, softmax, lse and the latent aggregate written out with fsum loops."""
    rng = np.random.default_rng(5)
    R, L, dc, dr = 3, 7, 6, 4
    ql, qr = rng.standard_normal((R, dc)), rng.standard_normal((R, dr))
    C, KR = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    scale = 0.37
    visible = np.array([7, 5, 1])
    m, l, U = O.attend_absorbed(ql, qr, C, KR, scale, visible)
    u, lse = O.finalize(m, l, U)
    for r in range(R):
        n = visible[r]
        z = [scale * (math.fsum(ql[r][d] * C[s][d] for d in range(dc)) +
                      math.fsum(qr[r][d] * KR[s][d] for d in range(dr))) for s in range(n)]
        den = math.fsum(math.exp(v) for v in z)
        assert abs(lse[r] - math.log(den)) < 1e-12
        for d in range(dc):
            num = math.fsum(math.exp(z[s]) * C[s][d] for s in range(n))
            assert abs(u[r, d] - num / den) < 1e-12


# --------------------------------------------------------------------------
# absorbed == explicit (V2 analysis page, section 6.1), explicit == SDPA
# --------------------------------------------------------------------------

def _explicit_for(inp, b):
    cfg = inp.cfg
    dec = O.decoded_inputs(inp)
    rows = slice(b * cfg.T, (b + 1) * cfg.T)
    pos = inp.positions[rows].astype(np.int64)
    q_rot = O.rope_rotate(dec["q_rope"][rows], pos)
    C, KR = O.sequence_cache(inp, b)
    o, A = O.explicit_mha(dec["q_nope"][rows], q_rot, C, KR, dec["w_uk"], dec["w_uv"],
                          cfg.softmax_scale, pos + 1)
    return o, A, q_rot, C, KR, dec


def test_absorbed_equals_explicit_tiny_fp32():
    inp = synth.make_inputs("tiny_fp32")
    res = O.decode_step(inp)
    o_exp, A, *_ = _explicit_for(inp, 0)
    assert rel(res[0]["o"], o_exp) < 1e-12
    assert np.allclose(A.sum(axis=-1), 1.0, atol=1e-14, rtol=0)


@pytest.mark.parametrize("T,L,permuted", [(1, 1, False), (1, 65, True), (2, 2, False), (2, 130, True)])
def test_absorbed_equals_explicit_small_shapes(T, L, permuted):
    cfg = synth.small_config(B=2, H=4, T=T, seq_len=L, permuted=permuted, q_dt="f32",
                             ckv_dt="f32", kr_dt="f32", seed=11 + L)
    inp = synth.make_inputs(cfg)
    res = O.decode_step(inp)
    for b in range(cfg.B):
        o_exp, *_ = _explicit_for(inp, b)
        assert rel(res[b]["o"], o_exp) < 1e-12


def test_explicit_equals_torch_sdpa_default_scale():
    """torch's SDPA default scale is 1/sqrt(E) with E the query width, here
    d_h + d_R = 192: the same denominator eq. 18 prescribes."""
    cfg = synth.small_config(B=1, H=4, T=1, seq_len=90, q_dt="f32", ckv_dt="f32", kr_dt="f32")
    inp = synth.make_inputs(cfg)
    o_exp, A, q_rot, C, KR, dec = _explicit_for(inp, 0)
    H = cfg.H
    q = torch.from_numpy(np.concatenate([dec["q_nope"][0:1], q_rot], axis=-1))     # [1, H, 192]
    K = np.stack([np.concatenate([C @ dec["w_uk"][h].T, KR], axis=1) for h in range(H)])
    V = np.stack([C @ dec["w_uv"][h].T for h in range(H)])
    out = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2), torch.from_numpy(K), torch.from_numpy(V))             # [H, 1, 128]
    assert rel(o_exp[0], out[:, 0, :].numpy()) < 1e-12


# --------------------------------------------------------------------------
# closed forms and special cases
# --------------------------------------------------------------------------

def _tiny(T=1, L=150, **kw):
    cfg = synth.small_config(B=1, H=4, T=T, seq_len=L, q_dt="f32", ckv_dt="f32",
                             kr_dt="f32", **kw)
    return synth.make_inputs(cfg)


def test_constant_latents_give_ones():
    """Softmax weights sum to 1, so c = 1 everywhere gives u = 1 exactly up to rounding."""
    inp = _tiny()
    inp.ckv[...] = 1.0
    res = O.decode_step(inp)
    assert np.max(np.abs(res[0]["u"] - 1.0)) < 1e-13


def test_single_token_returns_its_latent():
    inp = _tiny(L=1)
    res = O.decode_step(inp)
    C, _ = O.sequence_cache(inp, 0)
    assert np.array_equal(res[0]["u"][0], np.broadcast_to(C[0], res[0]["u"][0].shape))


def test_zero_query_gives_mean():
    inp = _tiny(L=77)
    inp.q_nope[...] = 0.0
    inp.q_rope[...] = 0.0
    res = O.decode_step(inp)
    C, _ = O.sequence_cache(inp, 0)
    assert rel(res[0]["u"][0], np.broadcast_to(C.mean(axis=0), res[0]["u"][0].shape)) < 1e-13
    assert np.allclose(res[0]["lse"], math.log(77), atol=1e-13)


@pytest.mark.parametrize("target", [0, 63, 64, 100, 149])
def test_one_hot_gather_through_rope_channel(target):
    """Only the rope channel carries signal: q_nope = 0, q_rope = 1000 e_62
    (the slowest pair, theta_31 = 10000^(-62/64), so at position 149 it turns by
    0.02 rad), k^R = 4 e_62 on the target token and 0 elsewhere. The target's
    logit exceeds the rest by ~4000/sqrt(192) ~ 288, so u = c_target."""
    inp = _tiny(L=150)
    inp.q_nope[...] = 0.0
    inp.q_rope[...] = 0.0
    inp.q_rope[:, :, 62] = 1000.0
    inp.kr[...] = 0.0
    bt = inp.block_table[0]
    inp.kr[bt[target // 64], target % 64, 62] = 4.0
    res = O.decode_step(inp)
    C, _ = O.sequence_cache(inp, 0)
    assert rel(res[0]["u"][0], np.broadcast_to(C[target], res[0]["u"][0].shape)) < 1e-12


def test_two_token_query_matches_truncated_single():
    """With T = 2, query 0 sits at position L-2 and must see exactly the cache
    truncated to L-1 tokens, i.e. a T = 1 decode on that shorter cache."""
    inp2 = _tiny(T=2, L=131)
    res2 = O.decode_step(inp2)
    cfg = inp2.cfg
    dec = O.decoded_inputs(inp2)
    C, KR = O.sequence_cache(inp2, 0)
    ql = O.absorb_q(dec["q_nope"][0:1], dec["w_uk"])[0]
    qr = O.rope_rotate(dec["q_rope"][0:1], np.array([129]))[0]
    m, l, U = O.attend_absorbed(ql, qr, C[:130], KR[:130], cfg.softmax_scale,
                                np.full(cfg.H, 130))
    u, lse = O.finalize(m, l, U)
    assert rel(res2[0]["u"][0], u) < 1e-13


@pytest.mark.parametrize("split", [64, 128, 192, 1024])
def test_split_combine_equals_unsplit(split):
    inp = _tiny(L=333, T=2)
    a = O.decode_step(inp)
    b = O.decode_step(inp, split_tokens=split)
    assert rel(b[0]["u"], a[0]["u"]) < 1e-14
    assert np.max(np.abs(b[0]["lse"] - a[0]["lse"])) < 1e-13


def test_combine_with_empty_splits():
    rng = np.random.default_rng(9)
    R, L, dc, dr = 4, 40, 8, 4
    ql, qr = rng.standard_normal((R, dc)), rng.standard_normal((R, dr))
    C, KR = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    vis = np.full(R, L)
    whole = O.finalize(*O.attend_absorbed(ql, qr, C, KR, 0.1, vis))
    parts = [O.attend_absorbed(ql, qr, C, KR, 0.1, vis, rg)
             for rg in [(0, 16), (16, 32), (32, 48), (48, 64), (64, 80)]]
    assert np.all(parts[-1][0] == -np.inf) and np.all(parts[-1][1] == 0)
    u, lse = O.combine_partials(parts)
    assert rel(u, whole[0]) < 1e-14 and np.max(np.abs(lse - whole[1])) < 1e-13


def test_block_table_permutation_invariance():
    """Same logical cache, identity pool vs permuted pool: identical outputs."""
    cfg_id = synth.small_config(B=3, H=4, seq_len=300, ragged=True, permuted=False, seed=21)
    a_inp = synth.make_inputs(cfg_id)
    b_inp = synth.make_inputs(cfg_id)
    perm = np.random.default_rng(0).permutation(b_inp.n_pages)
    inv = np.argsort(perm)
    b_inp.ckv = b_inp.ckv[inv]
    b_inp.kr = b_inp.kr[inv]
    b_inp.block_table = np.where(b_inp.block_table >= 0, perm[np.maximum(b_inp.block_table, 0)], -1)
    ra, rb = O.decode_step(a_inp), O.decode_step(b_inp)
    for b in range(cfg_id.B):
        assert np.array_equal(ra[b]["u"], rb[b]["u"])


# --------------------------------------------------------------------------
# cache accounting: values printed on the V2 analysis page
# --------------------------------------------------------------------------

def _golden():
    rows = {}
    with open(os.path.join(GOLDEN, "cache_accounting.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, val, tol, _cite = [x.strip() for x in line.split("|")]
            rows[key] = (float(val), float(tol))
    return rows


def _computed():
    GiB = 2.0 ** 30
    mla = O.mla_cache_elems_per_token_layer(512, 64)
    mha = O.mha_cache_elems_per_token_layer(128, 128)
    dsk = O.mha_cache_elems_per_token_layer(8, 128)
    tok128k = 131072
    req = O.cache_bytes(mla, 60, tok128k, 16)
    return {
        "mla_elems_per_layer": mla,
        "mla_elems_over_dh": mla / 128,
        "gqa_equivalent_groups": mla / (2 * 128),
        "mla_elems_60_layers": mla * 60,
        "lite_elems_27_layers": mla * 27,
        "mha_elems_per_layer_128x128": mha,
        "mha_over_mla_ratio": mha / mla,
        "dsk67b_elems_per_layer": dsk,
        "dsk67b_elems_per_token": dsk * 95,
        "dsk67b_kib_per_token_bf16": O.cache_bytes(dsk, 95, 1, 16) / 1024,
        "element_reduction_pct": 100 * (1 - mla * 60 / (dsk * 95)),
        "reduction_with_6bit_pct": 100 * (1 - O.cache_bytes(mla, 60, 1, 6) / O.cache_bytes(dsk, 95, 1, 16)),
        "mla_bytes_per_token_bf16": O.cache_bytes(mla, 60, 1, 16),
        "mla_kib_per_token_bf16": O.cache_bytes(mla, 60, 1, 16) / 1024,
        "request_128k_gib": req / GiB,
        "request_128k_gb_decimal": req / 1e9,
        "per_head_rope_elems_per_layer": O.per_head_rope_elems_per_token_layer(512, 64, 128),
        "per_head_rope_128k_gib": O.cache_bytes(O.per_head_rope_elems_per_token_layer(512, 64, 128), 60, tok128k, 16) / GiB,
        "no_rope_128k_gib": O.cache_bytes(O.mla_cache_elems_per_token_layer(512, 0), 60, tok128k, 16) / GiB,
        "rope_share_pct": 100 * 64 / mla,
        "rope128_128k_gib": O.cache_bytes(O.mla_cache_elems_per_token_layer(512, 128), 60, tok128k, 16) / GiB,
        "rope32_128k_gib": O.cache_bytes(O.mla_cache_elems_per_token_layer(512, 32), 60, tok128k, 16) / GiB,
        "sixbit_packed_128k_gib": O.cache_bytes(mla, 60, tok128k, 6) / GiB,
        "eightbit_container_128k_gib": O.cache_bytes(mla, 60, tok128k, 8) / GiB,
        "dsk67b_128k_gib": O.cache_bytes(dsk, 95, tok128k, 16) / GiB,
    }


def test_cache_accounting_matches_page():
    g, c = _golden(), _computed()
    assert set(g) == set(c)
    for k, (val, tol) in g.items():
        if tol == 0:
            assert c[k] == val, k
        else:
            assert abs(c[k] - val) <= tol * val + 1e-12, (k, c[k], val)


def test_decode_bytes_and_flops_per_unit():
    assert O.decode_cache_bytes_per_token("bf16", "bf16") == 1152
    assert O.decode_cache_bytes_per_token("f32", "f32") == 2304
    assert O.decode_cache_bytes_per_token("fp8", "bf16") == 644
    assert O.decode_flops_per_row_token() == 2176
