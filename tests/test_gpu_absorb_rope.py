"""mla_absorb_q_rope: the absorbed content query and the rotated rope query
of one decode step from one call. It must equal mla_absorb_q followed by
mla_rope (or mla_rope_freq) bit for bit, on the fused one-launch path (bf16,
d_r = 64) and on the two-launch path it takes otherwise; the separate calls
are themselves compared with the oracle in the absorb, rope and YaRN parity
tests."""
import numpy as np
import pytest
import torch

from mla_latent_kv_35_amd import synth

pytestmark = pytest.mark.gpu


def bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy().view(np.int32)


CASES = [
    # n_tok, H, q_dt, out_dt, rope_dt, d_r, yarn
    (32, 128, "bf16", "bf16", "bf16", 64, False),     # one decode batch of the V2 layer shape
    (70, 16, "bf16", "bf16", "bf16", 64, False),      # three token tiles, ragged tail
    (5, 40, "bf16", "f32", "bf16", 64, True),         # H not a multiple of 8 or 32; YaRN
    (3, 8, "bf16", "bf16", "f32", 64, False),         # fp32 rope data: two launches
    (9, 16, "f32", "f32", "f32", 64, False),          # fp32 queries and rope: one launch
    (6, 40, "f32", "f32", "f32", 64, True),           # the same with H % 32 != 0 and YaRN
    (4, 16, "f32", "f32", "bf16", 64, False),         # fp32 queries, bf16 rope: two launches
    (4, 16, "bf16", "bf16", "bf16", 32, False),       # d_r != 64: two launches
    (1, 1, "bf16", "bf16", "bf16", 64, False),        # one token, one head
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_absorb_rope_equals_separate_calls(mla, case):
    n, H, q_dt, out_dt, rope_dt, dr, yarn = case
    rng = np.random.default_rng(n * 131 + H)
    qn = mla.to_device(synth.store(rng.standard_normal((n, H, 128)), q_dt), q_dt)
    wk = mla.to_device(synth.store(rng.standard_normal((H, 128, 512)) / np.sqrt(128), q_dt), q_dt)
    qr = mla.to_device(synth.store(rng.standard_normal((n, H, dr)), rope_dt), rope_dt)
    pos = torch.tensor(rng.integers(0, 131072, n), dtype=torch.int32, device="cuda")
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    theta = None
    if yarn:
        theta = torch.tensor(mla.yarn_frequencies(dr, 10000.0, 40.0, 1.0, 32.0, 4096),
                             dtype=torch.float64, device="cuda")
    q_lat, q_rot = mla.absorb_q_rope(qn, wk, qr, pos, 10000.0, theta=theta, out_dtype=odt)
    ref_lat = mla.absorb_q(qn, wk, out_dtype=odt)
    ref_rot = mla.rope(qr, pos) if theta is None else mla.rope_freq(qr, pos, theta)
    torch.cuda.synchronize()
    assert np.array_equal(bits(q_lat), bits(ref_lat))
    assert np.array_equal(bits(q_rot), bits(ref_rot))


def test_absorb_rope_in_place_rope(mla):
    rng = np.random.default_rng(5)
    n, H = 33, 128
    qn = mla.to_device(synth.store(rng.standard_normal((n, H, 128)), "bf16"), "bf16")
    wk = mla.to_device(synth.store(rng.standard_normal((H, 128, 512)) / np.sqrt(128), "bf16"),
                       "bf16")
    qr = mla.to_device(synth.store(rng.standard_normal((n, H, 64)), "bf16"), "bf16")
    pos = torch.arange(n, dtype=torch.int32, device="cuda") * 97
    ref_rot = mla.rope(qr, pos)
    ref_lat = mla.absorb_q(qn, wk)
    x = qr.clone()
    q_lat, q_rot = mla.absorb_q_rope(qn, wk, x, pos, q_rot=x)
    torch.cuda.synchronize()
    assert q_rot.data_ptr() == x.data_ptr()
    assert np.array_equal(bits(x), bits(ref_rot))
    assert np.array_equal(bits(q_lat), bits(ref_lat))
