"""Design decisions backed by a measurement on the CPU (fp64 oracle, no GPU).

Quantizing the absorbed queries to fp8 (the operand an fp8 MFMA would need
for the latent part of the score): with an fp8 latent cache, the error of u
that the query quantization alone adds, E4M3FN with one scale per block of
the 512 latent dims, against bf16 queries. Attention output u is compared
row by row (max |u - u_ref| / max |u_ref|, the parity metric), with the
oracle's exact attention on bf16-rounded queries as the reference. The
decode keeps bf16 queries because this error alone is most of the 5e-2 fp8
tolerance."""
import numpy as np
import pytest

from mla_latent_kv_35_amd import synth
from oracle import mla_oracle as O

pytestmark = pytest.mark.timeout(300)


def _e4m3_blocks(q: np.ndarray, blk: int, pow2: bool) -> np.ndarray:
    """q rounded to E4M3FN with one scale per block of blk elements (absmax / 448;
    pow2: the scale rounded up to a power of two, as in MX formats)."""
    R, D = q.shape
    qb = q.reshape(R, D // blk, blk)
    amax = np.abs(qb).max(axis=2, keepdims=True)
    sc = np.where(amax > 0, amax / 448.0, 1.0)
    if pow2:
        sc = 2.0 ** np.ceil(np.log2(sc))
    codes = O.e4m3fn_to_f64(O.e4m3fn_round(np.asarray(qb / sc, np.float32)))
    return (codes * sc).reshape(R, D)


def _bf16(x):
    return O.bf16_bits_to_f64(O.f64_to_bf16_bits(x))


def test_fp8_query_quantization_error_fills_the_fp8_budget():
    cfg = synth.small_config("study", B=1, H=128, T=2, seq_len=8192, ckv_dt="fp8", seed=5)
    inp = synth.make_inputs(cfg)
    dec = O.decoded_inputs(inp)
    T, H = cfg.T, cfg.H
    q_lat = _bf16(O.absorb_q(dec["q_nope"][0:T], dec["w_uk"])).reshape(T * H, -1)
    pos = np.asarray(inp.positions[0:T], dtype=np.int64)
    q_rot = _bf16(O.rope_rotate(dec["q_rope"][0:T], pos, 10000.0)).reshape(T * H, -1)
    C, KR = O.sequence_cache(inp, 0)
    vis = np.repeat(pos + 1, H)
    u_ref, _ = O.finalize(*O.attend_absorbed(q_lat, q_rot, C, KR, cfg.softmax_scale, vis))

    def err(q):
        u, _ = O.finalize(*O.attend_absorbed(q, q_rot, C, KR, cfg.softmax_scale, vis))
        return float((np.abs(u - u_ref).max(axis=1) / np.abs(u_ref).max(axis=1)).max())

    e = {"bf16 (identity)": err(q_lat),
         "per row": err(_e4m3_blocks(q_lat, 512, False)),
         "per 32, fp32 scales": err(_e4m3_blocks(q_lat, 32, False)),
         "per 32, power-of-two scales": err(_e4m3_blocks(q_lat, 32, True))}
    print(e)
    assert e["bf16 (identity)"] == 0.0
    # every block-scaled fp8 query leaves under half of the 5e-2 budget for the rest
    for k in ("per row", "per 32, fp32 scales", "per 32, power-of-two scales"):
        assert e[k] > 2.5e-2, (k, e)
