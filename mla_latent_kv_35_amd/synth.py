"""Seeded synthetic inputs for MLA absorbed decode.

This module only draws random numbers and packs them into the stored form
(bit patterns of fp32 / bf16 / fp8-E4M3FN values laid out in 64-token pages
with a block table). It contains none of the attention arithmetic: no RoPE,
no absorption, no softmax. The CPU checker and the GPU path both consume
exactly the arrays returned here.

Shapes follow the DeepSeek-V2 MLA formulation: a joint KV latent of d_c = 512
per token plus one decoupled, already-rotated RoPE key of d_R = 64 shared by
all heads (PaperTrace "02 · DeepSeek-V2 analysis", sections 1.2 and 1.3;
576 cached elements per token per layer), d_h = 128 per head.

Readings of the workload descriptions that the pages leave open:

* Weights W_UK, W_UV are drawn N(0, 1/512): variance 1/512.
* "post-RMSNorm, unit RMS" latents are drawn uniformly on the sphere of
  radius sqrt(d_c): a Gaussian vector divided by its RMS.
* The cache holds the shared RoPE key already rotated (section 6, third
  absorption condition, of the same page). A rotation maps an isotropic
  Gaussian vector to an isotropic Gaussian vector, so the stored rotated key
  is drawn directly as N(0, 1); no rotation happens here.
* Rounding to bf16 and to fp8 uses torch's dtype casts (round to nearest
  even). fp8 caches use OCP E4M3FN codes with one fp32 scale per token,
  scale = fp32(absmax) / 448; an all-zero token gets scale 1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE = 64
D_C = 512
D_R = 64
D_H = 128
FP8_MAX = 448.0

F32, BF16, FP8 = "f32", "bf16", "fp8"


@dataclasses.dataclass(frozen=True)
class MlaConfig:
    name: str
    B: int
    H: int
    T: int
    seq_len: int            # uniform length, or the upper bound of a ragged draw
    ragged: bool = False    # lengths ~ Uniform[1, seq_len] (integers)
    permuted: bool = False  # block table is a random permutation of the pool
    q_dt: str = BF16        # dtype of q_nope / q_rope / weights
    ckv_dt: str = BF16      # dtype of the latent cache
    kr_dt: str = BF16       # dtype of the rotated RoPE-key cache
    unit_rms_latent: bool = False
    seed: int = 0
    d_h: int = D_H
    d_c: int = D_C
    d_r: int = D_R

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(d_h + d_R): the denominator the decoupled-RoPE concatenation uses.
        return 1.0 / math.sqrt(self.d_h + self.d_r)


# The five workloads: sizes, dtypes and structure from the benchmark description.
CONFIGS = {
    "tiny_fp32": MlaConfig("tiny_fp32", B=1, H=16, T=1, seq_len=256,
                           q_dt=F32, ckv_dt=F32, kr_dt=F32, seed=1001),
    "dsv2_layer": MlaConfig("dsv2_layer", B=32, H=128, T=1, seq_len=4096,
                            unit_rms_latent=True, seed=1002),
    "ragged": MlaConfig("ragged", B=64, H=128, T=1, seq_len=32768,
                        ragged=True, permuted=True, seed=1003),
    "long_128k": MlaConfig("long_128k", B=4, H=128, T=1, seq_len=131072, seed=1004),
    "mtp_fp8": MlaConfig("mtp_fp8", B=128, H=128, T=2, seq_len=8192,
                         ckv_dt=FP8, seed=1005),
}
CONFIG_ORDER = ["tiny_fp32", "dsv2_layer", "ragged", "long_128k", "mtp_fp8"]


def elem_bytes(dt: str) -> int:
    return {F32: 4, BF16: 2, FP8: 1}[dt]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values -> uint16 bf16 bit patterns (torch cast, round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def store(x64: np.ndarray, dt: str) -> np.ndarray:
    """fp64 draw -> stored bits of the given dtype (via fp32)."""
    x32 = x64.astype(np.float32)
    if dt == F32:
        return x32
    if dt == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(dt)


def quantize_fp8_per_token(x64: np.ndarray):
    """fp64 [..., d] -> (uint8 E4M3FN codes [..., d], fp32 scale [...]).

    scale = fp32(max |x|) / 448 (fp32 division); codes = torch cast of
    fp32(x) / scale. All-zero rows get scale 1.
    """
    x32 = x64.astype(np.float32)
    amax = np.abs(x32).max(axis=-1)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = (x32 / scale[..., None]).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


@dataclasses.dataclass
class MlaInputs:
    cfg: MlaConfig
    seq_lens: np.ndarray      # int32 [B]
    block_table: np.ndarray   # int32 [B][max_pages]; -1 for unused entries
    n_pages: int
    q_nope: np.ndarray        # [B*T][H][d_h]   stored bits (q_dt)
    q_rope: np.ndarray        # [B*T][H][d_r]   stored bits, NOT rotated
    ckv: np.ndarray           # [n_pages][64][d_c] stored bits (ckv_dt)
    kr: np.ndarray            # [n_pages][64][d_r] stored bits (kr_dt), already rotated
    ckv_scale: Optional[np.ndarray]  # fp32 [n_pages][64] iff ckv_dt == fp8
    w_uk: np.ndarray          # [H][d_h][d_c] stored bits (q_dt)
    w_uv: np.ndarray          # [H][d_h][d_c] stored bits (q_dt)
    positions: np.ndarray     # int32 [B*T]: position of each query token

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())


def _draw_lengths(cfg: MlaConfig, rng) -> np.ndarray:
    if cfg.ragged:
        return rng.integers(1, cfg.seq_len, size=cfg.B, endpoint=True).astype(np.int32)
    return np.full(cfg.B, cfg.seq_len, dtype=np.int32)


def _fill_pages(rng, n_pages: int, width: int, dt: str, unit_rms: bool,
                chunk_pages: int = 512):
    """Draw n_pages*64 token vectors of `width` values page chunk by page chunk."""
    if dt == FP8:
        codes = np.empty((n_pages, PAGE, width), dtype=np.uint8)
        scales = np.empty((n_pages, PAGE), dtype=np.float32)
    else:
        out = np.empty((n_pages, PAGE, width), dtype=np.float32 if dt == F32 else np.uint16)
    for p0 in range(0, n_pages, chunk_pages):
        p1 = min(n_pages, p0 + chunk_pages)
        x = rng.standard_normal((p1 - p0, PAGE, width))
        if unit_rms:
            x = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
        if dt == FP8:
            codes[p0:p1], scales[p0:p1] = quantize_fp8_per_token(x)
        else:
            out[p0:p1] = store(x, dt)
    if dt == FP8:
        return codes, scales
    return out, None


def make_inputs(cfg: MlaConfig | str, seed: Optional[int] = None, *,
                seq_lens: Optional[np.ndarray] = None,
                poison_tail: bool = False) -> MlaInputs:
    """Draw one workload. Fixed draw order: lengths, page permutation, q_nope,
    q_rope, latent cache, RoPE-key cache, W_UK, W_UV."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lens = _draw_lengths(cfg, rng)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
        assert lens.shape == (cfg.B,)
    pages_per_seq = (lens.astype(np.int64) + PAGE - 1) // PAGE
    max_pages = int(pages_per_seq.max())
    n_pages = int(pages_per_seq.sum())
    if cfg.permuted:
        pool = rng.permutation(n_pages).astype(np.int32)
    else:
        pool = np.arange(n_pages, dtype=np.int32)
    bt = np.full((cfg.B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(cfg.B):
        n = int(pages_per_seq[b])
        bt[b, :n] = pool[off:off + n]
        off += n

    BT = cfg.B * cfg.T
    q_nope = store(rng.standard_normal((BT, cfg.H, cfg.d_h)), cfg.q_dt)
    q_rope = store(rng.standard_normal((BT, cfg.H, cfg.d_r)), cfg.q_dt)
    ckv, ckv_scale = _fill_pages(rng, n_pages, cfg.d_c, cfg.ckv_dt, cfg.unit_rms_latent)
    kr, _ = _fill_pages(rng, n_pages, cfg.d_r, cfg.kr_dt, False)
    wstd = 1.0 / math.sqrt(cfg.d_c)
    w_uk = store(rng.standard_normal((cfg.H, cfg.d_h, cfg.d_c)) * wstd, cfg.q_dt)
    w_uv = store(rng.standard_normal((cfg.H, cfg.d_h, cfg.d_c)) * wstd, cfg.q_dt)

    # query token t of sequence b sits at position L_b - T + t (the new tokens
    # are appended to the cache before attention).
    pos = (lens[:, None].astype(np.int64) - cfg.T + np.arange(cfg.T)[None, :]).reshape(-1)
    inp = MlaInputs(cfg, lens, bt, n_pages, q_nope, q_rope, ckv, kr, ckv_scale,
                    w_uk, w_uv, pos.astype(np.int32))
    if poison_tail:
        poison_unused_slots(inp)
    return inp


def poison_unused_slots(inp: MlaInputs) -> None:
    """Write NaN into every cache slot that no sequence covers (tail slots of
    each sequence's last page). Kernels must never let them reach an output."""
    nan_bits = {F32: np.float32(np.nan), BF16: np.uint16(0x7FC0), FP8: np.uint8(0x7F)}
    for b in range(inp.cfg.B):
        L = int(inp.seq_lens[b])
        if L % PAGE:
            pg = inp.block_table[b, L // PAGE]
            inp.ckv[pg, L % PAGE:] = nan_bits[inp.cfg.ckv_dt]
            inp.kr[pg, L % PAGE:] = nan_bits[inp.cfg.kr_dt]
            if inp.ckv_scale is not None:
                inp.ckv_scale[pg, L % PAGE:] = np.float32(np.nan)


def small_config(name: str = "small", *, B=2, H=32, T=1, seq_len=200, ragged=False,
                 permuted=False, q_dt=BF16, ckv_dt=BF16, kr_dt=BF16,
                 unit_rms_latent=False, seed=7) -> MlaConfig:
    """A reduced workload with the same structure, for fast parity checks."""
    return MlaConfig(name, B=B, H=H, T=T, seq_len=seq_len, ragged=ragged,
                     permuted=permuted, q_dt=q_dt, ckv_dt=ckv_dt, kr_dt=kr_dt,
                     unit_rms_latent=unit_rms_latent, seed=seed)
