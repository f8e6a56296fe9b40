"""Structure of the seeded synthetic workloads (no GPU)."""
import numpy as np
import pytest

from mla_latent_kv_35_amd import synth
from oracle import mla_oracle as O


def test_ragged_lengths_and_permuted_pool():
    cfg = synth.small_config(B=16, H=16, seq_len=700, ragged=True, permuted=True, seed=3)
    inp = synth.make_inputs(cfg)
    assert inp.seq_lens.min() >= 1 and inp.seq_lens.max() <= 700
    used = []
    for b in range(cfg.B):
        n = -(-int(inp.seq_lens[b]) // 64)
        row = inp.block_table[b]
        assert np.all(row[:n] >= 0) and np.all(row[n:] == -1)
        used.extend(row[:n].tolist())
    assert sorted(used) == list(range(inp.n_pages))         # the pool is exactly covered


def test_ragged_seed_1003_lengths():
    """The ragged workload's lengths follow from its seed alone."""
    cfg = synth.CONFIGS["ragged"]
    rng = np.random.default_rng(cfg.seed)
    lens = rng.integers(1, cfg.seq_len, size=cfg.B, endpoint=True)
    assert int(lens.sum()) == 1055283 and int(lens.min()) == 13 and int(lens.max()) == 31804


def test_unit_rms_latents_and_weight_variance():
    cfg = synth.small_config(B=2, H=8, seq_len=128, unit_rms_latent=True, seed=5)
    inp = synth.make_inputs(cfg)
    c = O.stored_to_f64(inp.ckv, "bf16")
    rms = np.sqrt(np.mean(c * c, axis=-1))
    assert np.allclose(rms, 1.0, atol=1e-2)                 # bf16 rounding only
    w = O.stored_to_f64(inp.w_uk, "bf16")
    assert abs(w.var() - 1 / 512) < 0.05 / 512


def test_fp8_cache_layout():
    cfg = synth.small_config(B=2, H=16, T=2, seq_len=100, ckv_dt="fp8", seed=6)
    inp = synth.make_inputs(cfg)
    assert inp.ckv.dtype == np.uint8 and inp.ckv_scale.shape == (inp.n_pages, 64)
    assert inp.kr.dtype == np.uint16
    assert np.array_equal(inp.positions, np.array([98, 99, 98, 99]))


def test_poisoned_tails_only_touch_unused_slots():
    cfg = synth.small_config(B=3, H=16, seq_len=150, ragged=True, seed=8)
    a = synth.make_inputs(cfg)
    b = synth.make_inputs(cfg, poison_tail=True)
    for s in range(cfg.B):
        Ca, _ = O.sequence_cache(a, s)
        Cb, _ = O.sequence_cache(b, s)
        assert np.array_equal(Ca, Cb)
    assert np.isnan(O.stored_to_f64(b.ckv, "bf16")).any()


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_config_table(name):
    cfg = synth.CONFIGS[name]
    assert cfg.d_c + cfg.d_r == 576
    assert abs(cfg.softmax_scale - 1 / np.sqrt(192)) < 1e-16
