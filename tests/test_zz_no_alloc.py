"""The allocation-free decode entry point (mla_decode_paged_noalloc) against
mla_decode_paged with a caller workspace: the same kernels on the same
inputs, so u and lse must agree bit for bit. Two calls in a row, the second
with a smaller input, so that the second reads a scratch array that still
holds the first call's partials."""
import numpy as np
import pytest
import torch

from mla_latent_kv_35_amd import synth

pytestmark = pytest.mark.gpu


def _decode_both(mla, cfg, split_tokens):
    inp = synth.make_inputs(cfg)
    d = mla.upload(inp)
    T, H = cfg.T, cfg.H
    BT = cfg.B * T
    q_lat = torch.randn((BT, H, 512), device="cuda").to(torch.bfloat16)
    q_rot = torch.randn((BT, H, 64), device="cuda").to(torch.bfloat16)
    u_ref, lse_ref = mla.decode_paged(q_lat, q_rot, d.cache, T, 0.0721, split_tokens=split_tokens)
    u = torch.full_like(u_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    mla.decode_paged_noalloc(q_lat, q_rot, d.cache, T, 0.0721, u, lse, split_tokens=split_tokens)
    torch.cuda.synchronize()
    _, n_split, ws = mla.decode_plan(mla.make_decode_args(q_lat, q_rot, d.cache, T, 0.0721, u, lse,
                                                          None, split_tokens))
    return u_ref, lse_ref, u, lse, n_split, ws


def test_noalloc_matches_workspace_entry_point(mla):
    torch.manual_seed(11)
    big = synth.small_config("noalloc_big", B=4, H=128, T=1, seq_len=3000, ragged=True, seed=21)
    small = synth.small_config("noalloc_small", B=2, H=64, T=2, seq_len=700, seed=22)
    small8 = synth.small_config("noalloc_small_fp8", B=2, H=64, T=2, seq_len=700, seed=24,
                                ckv_dt="fp8")
    for cfg, split in ((big, 256), (small, 128), (small8, 64)):
        u_ref, lse_ref, u, lse, n_split, ws = _decode_both(mla, cfg, split)
        print(cfg.name, "splits", n_split, "workspace bytes", ws)
        assert n_split > 1 and ws > 0          # the partials go through the scratch array
        assert torch.equal(u.view(torch.int16), u_ref.view(torch.int16)), cfg.name
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), cfg.name


def test_noalloc_rejects_partials_beyond_the_array(mla):
    # ws > 64 MiB: B * n_split * R * (512 * 2 + 8) bytes with one-page splits
    cfg = synth.small_config("noalloc_huge", B=16, H=128, T=1, seq_len=4096, seed=23)
    inp = synth.make_inputs(cfg)
    d = mla.upload(inp)
    q_lat = torch.zeros((cfg.B, cfg.H, 512), device="cuda", dtype=torch.bfloat16)
    q_rot = torch.zeros((cfg.B, cfg.H, 64), device="cuda", dtype=torch.bfloat16)
    u = torch.zeros((cfg.B, cfg.H, 512), device="cuda", dtype=torch.bfloat16)
    a = mla.make_decode_args(q_lat, q_rot, d.cache, 1, 0.0721, u, None, None, 64)
    _, n_split, ws = mla.decode_plan(a)
    assert ws > 64 << 20
    with pytest.raises(mla.MlaError) as e:
        mla.decode_paged_noalloc(q_lat, q_rot, d.cache, 1, 0.0721, u, None, split_tokens=64)
    assert "WORKSPACE" in str(e.value)
    assert not torch.isnan(u.float()).any()    # nothing was launched
