"""GPU parity of the explicit (expanded) prefill path, and the consistency
check the V2 analysis page describes in section 6.1: the expanded and the
absorbed forms are the same function in exact arithmetic, so on the same
inputs they may differ only by rounding (bf16 here), and that difference
must not grow with the sequence length.

* mla_expand_kv against W_UK[h] c and W_UV[h] c in float64;
* mla_prefill_attn against the oracle's explicit multi-head attention
  (every query row for small cases, sampled rows for larger ones), causal,
  with query blocks and key tiles that end in ragged tails; lse against the
  oracle's absorbed form (the same value in exact arithmetic);
* explicit prefill (GPU) against absorbed decode (GPU) for the last T tokens
  of paged sequences of growing length.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_35_amd import synth
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu


def row_rel(g, r):
    g = np.asarray(g, np.float64).reshape(-1, g.shape[-1])
    r = np.asarray(r, np.float64).reshape(-1, r.shape[-1])
    return float((np.abs(g - r).max(axis=1) / np.maximum(np.abs(r).max(axis=1), 1e-30)).max())


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_expand_kv_parity(mla, dt):
    rng = np.random.default_rng(81)
    n, H = 300, 16
    c = synth.store(rng.standard_normal((n, 512)), dt)
    wk = synth.store(rng.standard_normal((H, 128, 512)) / np.sqrt(512), dt)
    wv = synth.store(rng.standard_normal((H, 128, 512)) / np.sqrt(512), dt)
    k, v = mla.expand_kv(mla.to_device(c, dt), mla.to_device(wk, dt), mla.to_device(wv, dt))
    torch.cuda.synchronize()
    C = O.stored_to_f64(c, dt)
    Wk, Wv = O.stored_to_f64(wk, dt), O.stored_to_f64(wv, dt)
    tol = 1e-5 if dt == "f32" else 8e-3
    assert row_rel(host(k), np.einsum("nd,hjd->nhj", C, Wk)) <= tol
    assert row_rel(host(v), np.einsum("nd,hjd->nhj", C, Wv)) <= tol


def make_prefill(rng, B, H, n_kv):
    c = synth.store(rng.standard_normal((B, n_kv, 512)), "bf16")
    kr = synth.store(rng.standard_normal((B, n_kv, 64)), "bf16")
    wk = synth.store(rng.standard_normal((H, 128, 512)) / np.sqrt(512), "bf16")
    wv = synth.store(rng.standard_normal((H, 128, 512)) / np.sqrt(512), "bf16")
    return c, kr, wk, wv


def run_prefill(mla, c, kr, wk, wv, qn, qr, scale, out_dtype=torch.bfloat16):
    B, n_kv = c.shape[:2]
    H = wk.shape[0]
    k, v = mla.expand_kv(mla.to_device(c.reshape(B * n_kv, 512), "bf16"), mla.to_device(wk, "bf16"),
                         mla.to_device(wv, "bf16"))
    k = k.view(B, n_kv, H, 128)
    v = v.view(B, n_kv, H, 128)
    o, lse = mla.prefill_attn(mla.to_device(qn, "bf16"), mla.to_device(qr, "bf16"), k,
                              mla.to_device(kr, "bf16"), v, scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(o), lse.cpu().numpy()


@pytest.mark.parametrize("B,H,n_kv,n_q,sample", [
    (2, 16, 200, 200, None),      # full causal prefill, ragged key tile and query block
    (2, 16, 200, 37, None),       # chunked prefill: the last 37 tokens
    (1, 32, 130, 2, None),        # two speculative tokens
    (3, 16, 64, 1, None),         # one query, exactly one key tile
    (1, 128, 1000, 1000, 24),     # larger: sampled query rows
    (1, 128, 4096, 4096, 6),      # the benchmarked shape: sampled query rows
])
def test_prefill_parity(mla, B, H, n_kv, n_q, sample):
    rng = np.random.default_rng(B * 1000 + n_kv + n_q)
    c, kr, wk, wv = make_prefill(rng, B, H, n_kv)
    qn = synth.store(rng.standard_normal((B, n_q, H, 128)), "bf16")
    qr = synth.store(rng.standard_normal((B, n_q, H, 64)), "bf16")
    scale = 192 ** -0.5
    o, lse = run_prefill(mla, c, kr, wk, wv, qn, qr, scale)
    Wk, Wv = O.stored_to_f64(wk, "bf16"), O.stored_to_f64(wv, "bf16")
    for b in range(B):
        rows = np.arange(n_q) if sample is None else np.unique(np.concatenate(
            [[0, n_q - 1], rng.choice(n_q, sample, replace=False)]))
        C, KR = O.stored_to_f64(c[b], "bf16"), O.stored_to_f64(kr[b], "bf16")
        QN, QR = O.stored_to_f64(qn[b][rows], "bf16"), O.stored_to_f64(qr[b][rows], "bf16")
        visible = n_kv - n_q + rows + 1
        ref, _ = O.explicit_mha(QN, QR, C, KR, Wk, Wv, scale, visible)
        err = row_rel(o[b][rows], ref)
        assert err <= 2e-2, (b, err)
        ql = O.absorb_q(QN, Wk).reshape(len(rows) * H, -1)
        m, l, _ = O.attend_absorbed(ql, QR.reshape(len(rows) * H, -1), C, KR, scale,
                                    np.repeat(visible, H))
        assert np.abs(lse[b][rows].reshape(-1) - (m + np.log(l))).max() <= 5e-2


@pytest.mark.parametrize("B,H,n_kv,n_q", [
    (1, 20, 333, 333),            # B*H not a multiple of 8: plain workgroup order
    (3, 4, 70, 70),               # 12 heads in all, one query block each, ragged key tile
])
def test_prefill_parity_f32_output_odd_heads(mla, B, H, n_kv, n_q):
    rng = np.random.default_rng(B * 77 + H)
    c, kr, wk, wv = make_prefill(rng, B, H, n_kv)
    qn = synth.store(rng.standard_normal((B, n_q, H, 128)), "bf16")
    qr = synth.store(rng.standard_normal((B, n_q, H, 64)), "bf16")
    scale = 192 ** -0.5
    o, lse = run_prefill(mla, c, kr, wk, wv, qn, qr, scale, out_dtype=torch.float32)
    Wk, Wv = O.stored_to_f64(wk, "bf16"), O.stored_to_f64(wv, "bf16")
    for b in range(B):
        C, KR = O.stored_to_f64(c[b], "bf16"), O.stored_to_f64(kr[b], "bf16")
        QN, QR = O.stored_to_f64(qn[b], "bf16"), O.stored_to_f64(qr[b], "bf16")
        visible = n_kv - n_q + np.arange(n_q) + 1
        ref, _ = O.explicit_mha(QN, QR, C, KR, Wk, Wv, scale, visible)
        assert row_rel(o[b], ref) <= 2e-2


@pytest.mark.parametrize("T", [1, 2])
def test_explicit_prefill_equals_absorbed_decode(mla, T):
    """Section 6.1's check: the same queries and cache through both forms."""
    errs = []
    for L in (100, 1000, 4000):
        cfg = synth.small_config(f"consistency{L}", B=2, H=32, T=T, seq_len=L, ragged=False,
                                 permuted=True, seed=90 + L + T)
        inp = synth.make_inputs(cfg)
        d = mla.upload(inp)
        dec = mla.decode_step(d)
        torch.cuda.synchronize()
        o_dec = host(dec["o"]).reshape(cfg.B, T, cfg.H, 128)
        q_rot = dec["q_rot"].view(cfg.B, T, cfg.H, 64).contiguous()
        # the same sequences' latents and rotated keys, gathered out of the pages
        c = np.stack([O.gather_sequence(inp.ckv, inp.block_table[b], L) for b in range(cfg.B)])
        kr = np.stack([O.gather_sequence(inp.kr, inp.block_table[b], L) for b in range(cfg.B)])
        k, v = mla.expand_kv(mla.to_device(c.reshape(cfg.B * L, 512), "bf16"), d.w_uk, d.w_uv)
        o_pre, _ = mla.prefill_attn(d.q_nope.view(cfg.B, T, cfg.H, 128).contiguous(), q_rot,
                                    k.view(cfg.B, L, cfg.H, 128), mla.to_device(kr, "bf16"),
                                    v.view(cfg.B, L, cfg.H, 128), cfg.softmax_scale)
        torch.cuda.synchronize()
        errs.append(row_rel(host(o_pre), o_dec))
    print("explicit vs absorbed, by length:", errs)
    assert max(errs) <= 2e-2, errs
    # no systematic growth with length (a RoPE or scale-axis mismatch would grow)
    assert errs[-1] <= 4 * max(errs[0], 2e-3), errs
