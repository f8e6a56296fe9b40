"""CPU oracle for MLA absorbed decode -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The GPU product path never calls it, and it shares no
code with the GPU path: it decodes stored bits itself and does every step in
float64 with plain numpy (matrix products are numpy's).

What it computes, and where each step is defined (pages are cited by title
and section; "the V2 analysis page" is PaperTrace "02 · DeepSeek-V2
analysis"):

* KV cache: per token only the joint latent c (d_c = 512) and one shared,
  already-rotated RoPE key k^R (d_R = 64) are kept -- V2 analysis page,
  sections 1.2 and 1.3 (576 elements per token per layer).
* Absorption: the content score q^T (W^UK c) is computed as (W^UK^T q)^T c,
  so each head's query is mapped into the latent space once -- V2 analysis
  page, section 1.2 and section 6 (linear, fixed, position-free map).
* Decoupled RoPE: a per-head rope query and the shared rope key add a second
  dot product; the sum is scaled by 1/sqrt(d_h + d_R) (eq. 18) -- V2 analysis
  page, section 1.3.
* RoPE itself rotates coordinate pairs (2i, 2i+1) at position n -- CSDN
  "DeepSeek-V3 structure and engineering", section 2(3). Frequencies
  theta_i = base^(-2i/d_R) and the rotation sign are this oracle's reading
  (the pages do not print them).
* Softmax over the cached sequence, then each head aggregates latents,
  u_i = sum_s a_{s,i} c_s, and only then applies its own W^UV -- V2 analysis
  page, section 6.1 (per-head aggregation before B_i; the B_i cannot be summed
  across heads).
* Cache append: each new token's latent (RMS-normalized, section 1.2) and its
  rope key rotated at the token's position join the paged cache -- V2
  analysis page, section 1.3, the token walk-through in section 6.3, and
  section 6 (the key is cached already rotated). The fp8 storage follows the
  per-token absmax/448 scale reading; its codes are chosen from the table of
  E4M3FN values.
* Explicit form: expand K = [W^UK c ; k^R] and V = W^UV c per head and run
  standard multi-head attention; it must equal the absorbed form up to
  rounding -- V2 analysis page, section 6.1 (training/prefill paragraph and
  the equivalence check that follows it).

Pins that tie this oracle to something other than itself live in
tests/test_oracle_pins.py. Parity unpinned: nothing here models the GPU
path's internal bf16/fp8 rounding of q_lat, of softmax weights or of split
partials.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

PAGE = 64

# ----------------------------------------------------------------------------
# Stored formats -> float64 (from the format definitions, not from a library)
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen and reinterpret."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    No infinities; S.1111.111 is NaN; exponent field 0 encodes subnormals
    m/8 * 2^(1-7). Largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.ascontiguousarray(codes).view(np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** (1 - 7)
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


def stored_to_f64(arr: np.ndarray, dt: str, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Decode stored bits; fp8 codes are multiplied by their per-token scale."""
    if dt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dt == "bf16":
        return bf16_bits_to_f64(arr)
    if dt == "fp8":
        v = e4m3fn_to_f64(arr)
        if scale is not None:
            v = v * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
        return v
    raise ValueError(dt)


# ----------------------------------------------------------------------------
# The steps of the method
# ----------------------------------------------------------------------------


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float = 10000.0,
                theta: Optional[np.ndarray] = None) -> np.ndarray:
    """Rotate pairs (x[2i], x[2i+1]) by the angle pos * base^(-2i/d), or by
    pos * theta[i] when per-pair frequencies theta are given (YaRN).

    x: [..., n, d] (or [n, d]) float64; pos: [n] integer positions, one per
    leading row of x's second-to-last axis when x is [n, d], or broadcastable
    to x[..., 0]. The rotation is (x0 cos - x1 sin, x0 sin + x1 cos).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    # theta_i = base^(-2i/d) from libm's pow, one value per pair
    if theta is None:
        theta = np.array([math.pow(base, -2.0 * i / d) for i in range(d // 2)])
    theta = np.asarray(theta, dtype=np.float64)
    assert theta.shape == (d // 2,)
    p = np.asarray(pos, dtype=np.int64)
    # cos/sin from libm (full-precision argument reduction: angles reach 1e5
    # rad at 128K positions), evaluated once per distinct position.
    uniq, inv = np.unique(p, return_inverse=True)
    ang = uniq.astype(np.float64)[:, None] * theta[None, :]
    cu = np.frompyfunc(math.cos, 1, 1)(ang).astype(np.float64)
    su = np.frompyfunc(math.sin, 1, 1)(ang).astype(np.float64)
    shape = p.shape + (1,) * (x.ndim - 1 - p.ndim) + (d // 2,)
    c = cu[inv.reshape(-1)].reshape(shape)
    s = su[inv.reshape(-1)].reshape(shape)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------
# Cache append: the 512 latent + 64 rotated rope elements of each new token
# join the cache (V2 analysis page, section 1.3 and the token walk-through of
# section 6.3); the latent is RMS-normalized after the down-projection
# (section 1.2); the rope key is cached already rotated (section 6).
# ----------------------------------------------------------------------------


def rms_normalize(c: np.ndarray, gain: Optional[np.ndarray] = None, eps: float = 0.0) -> np.ndarray:
    """RMSNorm of each row: c / sqrt(mean(c^2) + eps) * gain, in float64
    (V2 analysis page, section 1.2; the gain is not given there, so it is an
    input, 1 when absent)."""
    c = np.asarray(c, dtype=np.float64)
    r = np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)
    out = c / r
    if gain is not None:
        out = out * np.asarray(gain, dtype=np.float32).astype(np.float64)
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to binary32 (nearest even), then keep the upper 16 bits rounded to
    nearest even on the lower 16 (finite values)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = np.ascontiguousarray(x32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def e4m3fn_round(y: np.ndarray) -> np.ndarray:
    """binary32 values -> E4M3FN codes: the nearest finite E4M3FN value, ties to
    the even code (even mantissa), magnitudes above 448 saturated to 448.
    Chosen from the table of all finite values (e4m3fn_to_f64)."""
    vals = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))     # codes 0..0x7E: 0 .. 448
    yf = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(yf.astype(np.float64)), 448.0)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(yf), 0x80, 0)).astype(np.uint8)


def quantize_fp8_token(c32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token E4M3FN quantization with one fp32 scale, decided in binary32:
    scale = fp32(max_j |c_j|) / 448 (binary32 division; 1 for an all-zero row),
    code_j = E4M3FN(fp32(c_j / scale))."""
    c32 = np.asarray(c32, dtype=np.float32)
    amax = np.abs(c32).max(axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = (c32 / scale[..., None]).astype(np.float32)
    return e4m3fn_round(y), scale


def cache_append(pools: Dict[str, np.ndarray], c_in: np.ndarray, c_dt: str, k_in: np.ndarray,
                 k_dt: str, seq: np.ndarray, pos: np.ndarray, block_table: np.ndarray,
                 ckv_dt: str, kr_dt: str, normalize: bool = False,
                 gain: Optional[np.ndarray] = None, eps: float = 0.0,
                 rope_base: float = 10000.0, theta: Optional[np.ndarray] = None) -> None:
    """Write each new token into pools["ckv"], pools["kr"] (and pools["scale"]
    for fp8) in place: token n goes to page block_table[seq[n]][pos[n] // 64],
    slot pos[n] % 64; tokens whose sequence, position or page id is out of
    range are skipped. Latent: optional RMSNorm (float64), then stored as f32
    (rounded once), bf16 (via binary32) or fp8 (quantize_fp8_token of its
    binary32 value). Key: rotated at pos[n] in float64 (rope_rotate), rounded
    to binary32 and, for a bf16 pool, to bf16."""
    B, max_pages = block_table.shape
    n_pages = pools["ckv"].shape[0]
    for n in range(len(seq)):
        b, s = int(seq[n]), int(pos[n])
        if not (0 <= b < B and 0 <= s < max_pages * PAGE):
            continue
        page = int(block_table[b, s // PAGE])
        if not (0 <= page < n_pages):
            continue
        slot = s % PAGE
        c = stored_to_f64(c_in[n], c_dt)
        if normalize:
            c = rms_normalize(c, gain, eps)
        if ckv_dt == "f32":
            pools["ckv"][page, slot] = c.astype(np.float32)
        elif ckv_dt == "bf16":
            pools["ckv"][page, slot] = f64_to_bf16_bits(c)
        else:
            codes, sc = quantize_fp8_token(c.astype(np.float32))
            pools["ckv"][page, slot] = codes
            pools["scale"][page, slot] = sc
        k = rope_rotate(stored_to_f64(k_in[n], k_dt)[None, :], np.array([s]), rope_base, theta)[0]
        pools["kr"][page, slot] = k.astype(np.float32) if kr_dt == "f32" else f64_to_bf16_bits(k)


def yarn_theta(d: int, base: float, factor: float, alpha: float, beta: float,
               orig_len: int) -> np.ndarray:
    """YaRN frequencies of the rope part (V2 analysis page, section 3.2: YaRN
    acts on the 64 decoupled rope dimensions only; V2 extends a 4K window by
    factor 40 with alpha = 1, beta = 32). The pages refer elsewhere for the
    interpolation rule; this is the YaRN method's ramp over the number of
    turns r_i a pair makes across the original window: pairs with r_i <= alpha
    are slowed by the factor, pairs with r_i >= beta keep their frequency,
    pairs in between blend linearly."""
    out = np.empty(d // 2)
    for i in range(d // 2):
        th = math.pow(base, -2.0 * i / d)
        turns = orig_len * th / (2.0 * math.pi)
        g = min(1.0, max(0.0, (turns - alpha) / (beta - alpha)))
        out[i] = (1.0 - g) * (th / factor) + g * th
    return out


def yarn_mscale(factor: float, coef: float = 0.0707) -> float:
    """YaRN temperature factor sqrt(1/t) = coef ln(factor) + 1 (V2 analysis
    page, section 3.2: V2's coefficient is 0.0707, the original 0.1; the
    report's sqrt(t) is a typo for sqrt(1/t)). The pages move it onto the
    softmax scale; since the original scheme scales q and k each by it, the
    logits scale by its square (this oracle's reading)."""
    return 1.0 if factor <= 1.0 else coef * math.log(factor) + 1.0


def absorb_q(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_lat[n, h, :] = W_UK[h]^T q_nope[n, h, :].

    q_nope: [N, H, d_h]; w_uk: [H, d_h, d_c] (head h's up-projection U_h in
    R^{d_h x d_c}) -> [N, H, d_c].
    """
    N, H, dh = q_nope.shape
    out = np.empty((N, H, w_uk.shape[2]))
    for h in range(H):
        out[:, h, :] = q_nope[:, h, :] @ w_uk[h]
    return out


def out_proj(u: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o[n, h, :] = W_UV[h] u[n, h, :]; u: [N, H, d_c], w_uv: [H, d_h, d_c]."""
    N, H, dc = u.shape
    out = np.empty((N, H, w_uv.shape[1]))
    for h in range(H):
        out[:, h, :] = u[:, h, :] @ w_uv[h].T
    return out


def gather_sequence(pool: np.ndarray, block_table_row: np.ndarray, L: int) -> np.ndarray:
    """Token s of the sequence lives in page block_table_row[s // 64], slot s % 64."""
    s = np.arange(L)
    return pool[block_table_row[s // PAGE], s % PAGE]


def attend_absorbed(q_lat: np.ndarray, q_rot: np.ndarray, C: np.ndarray, KR: np.ndarray,
                    scale: float, visible: np.ndarray,
                    token_range: Optional[Tuple[int, int]] = None):
    """Absorbed-score attention over one sequence's cache.

    q_lat [R, d_c], q_rot [R, d_r]: R query rows (already absorbed / rotated).
    C [L, d_c], KR [L, d_r]: the sequence's latents and rotated rope keys.
    visible [R]: row r attends to tokens s < visible[r] (causal limit).
    token_range: restrict to tokens [s0, s1) (one split of the sequence).

    Returns (m, l, U): per row the max logit m, the sum l of exp(z - m) and
    the unnormalised latent aggregate U = sum_s exp(z_s - m) c_s. Rows with
    no visible token in the range give (-inf, 0, 0).
    """
    L = C.shape[0]
    s0, s1 = (0, L) if token_range is None else token_range
    s1 = min(s1, L)
    R = q_lat.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    U = np.zeros((R, C.shape[1]))
    if s1 <= s0:
        return m, l, U
    z = (q_lat @ C[s0:s1].T + q_rot @ KR[s0:s1].T) * scale           # [R, n]
    s_idx = np.arange(s0, s1)
    mask = s_idx[None, :] < np.asarray(visible)[:, None]
    z = np.where(mask, z, -np.inf)
    has = mask.any(axis=1)
    m = np.where(has, z.max(axis=1, initial=-np.inf), -np.inf)
    e = np.where(mask, np.exp(z - np.where(has, m, 0.0)[:, None]), 0.0)
    l = e.sum(axis=1)
    U = e @ C[s0:s1]
    return m, l, U


def finalize(m: np.ndarray, l: np.ndarray, U: np.ndarray):
    """u = U / l and lse = m + ln l."""
    return U / l[:, None], m + np.log(l)


def combine_partials(parts: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]):
    """Merge split partials (m_k, l_k, U_k) with the log-sum-exp rule:
    m* = max_k m_k, w_k = e^{m_k - m*}, u = sum w_k U_k / sum w_k l_k,
    lse = m* + ln sum w_k l_k. Empty splits (m = -inf) contribute nothing."""
    ms = np.stack([p[0] for p in parts])                             # [K, R]
    mstar = ms.max(axis=0)
    w = np.where(np.isfinite(ms), np.exp(ms - mstar[None, :]), 0.0)
    lsum = sum(w[k] * parts[k][1] for k in range(len(parts)))
    Usum = sum(w[k][:, None] * parts[k][2] for k in range(len(parts)))
    return Usum / lsum[:, None], mstar + np.log(lsum)


def split_ranges(L: int, split_tokens: int, n_split: int) -> List[Tuple[int, int]]:
    """Split k covers tokens [k*split_tokens, min((k+1)*split_tokens, L))."""
    return [(k * split_tokens, min((k + 1) * split_tokens, L)) for k in range(n_split)]


# ----------------------------------------------------------------------------
# Whole decode step over stored inputs
# ----------------------------------------------------------------------------


def _get(inp, name):
    return getattr(inp, name)


def decoded_inputs(inp) -> Dict[str, np.ndarray]:
    """Decode every stored array of an inputs object (duck-typed) to float64."""
    cfg = _get(inp, "cfg")
    out = {
        "q_nope": stored_to_f64(inp.q_nope, cfg.q_dt),
        "q_rope": stored_to_f64(inp.q_rope, cfg.q_dt),
        "w_uk": stored_to_f64(inp.w_uk, cfg.q_dt),
        "w_uv": stored_to_f64(inp.w_uv, cfg.q_dt),
    }
    return out


def sequence_cache(inp, b: int) -> Tuple[np.ndarray, np.ndarray]:
    cfg = inp.cfg
    L = int(inp.seq_lens[b])
    bt = inp.block_table[b]
    C = stored_to_f64(gather_sequence(inp.ckv, bt, L), cfg.ckv_dt,
                      None if inp.ckv_scale is None else gather_sequence(inp.ckv_scale, bt, L))
    KR = stored_to_f64(gather_sequence(inp.kr, bt, L), cfg.kr_dt)
    return C, KR


def decode_step(inp, batches: Optional[Iterable[int]] = None, rope_base: float = 10000.0,
                split_tokens: Optional[int] = None, theta: Optional[np.ndarray] = None,
                softmax_scale: Optional[float] = None):
    """The whole absorbed decode step for the chosen sequences.

    Returns dict of float64 arrays indexed by sequence b:
    q_lat [T, H, d_c], q_rot [T, H, d_r], u [T, H, d_c], lse [T, H],
    o [T, H, d_h]. With split_tokens set, each sequence is computed split by
    split and merged with combine_partials (for the split/combine pins).
    theta: per-pair rope frequencies for the query (YaRN); softmax_scale:
    replaces 1/sqrt(d_h + d_R) (YaRN temperature).
    """
    cfg = inp.cfg
    scale = cfg.softmax_scale if softmax_scale is None else softmax_scale
    T, H = cfg.T, cfg.H
    dec = decoded_inputs(inp)
    res = {}
    for b in (range(cfg.B) if batches is None else batches):
        rows = slice(b * T, (b + 1) * T)
        q_lat = absorb_q(dec["q_nope"][rows], dec["w_uk"])                  # [T, H, d_c]
        pos = np.asarray(inp.positions[rows], dtype=np.int64)
        q_rot = rope_rotate(dec["q_rope"][rows], pos, rope_base, theta)     # [T, H, d_r]
        C, KR = sequence_cache(inp, b)
        L = C.shape[0]
        visible = np.repeat(pos + 1, H)                                     # row (t,h) sees s <= pos_t
        ql = q_lat.reshape(T * H, -1)
        qr = q_rot.reshape(T * H, -1)
        if split_tokens is None:
            u, lse = finalize(*attend_absorbed(ql, qr, C, KR, scale, visible))
        else:
            n_split = -(-L // split_tokens)
            parts = [attend_absorbed(ql, qr, C, KR, scale, visible, rg)
                     for rg in split_ranges(L, split_tokens, n_split)]
            u, lse = combine_partials(parts)
        u = u.reshape(T, H, -1)
        o = out_proj(u, dec["w_uv"])
        res[b] = dict(q_lat=q_lat, q_rot=q_rot, u=u, lse=lse.reshape(T, H), o=o)
    return res


def explicit_mha(q_nope: np.ndarray, q_rot: np.ndarray, C: np.ndarray, KR: np.ndarray,
                 w_uk: np.ndarray, w_uv: np.ndarray, scale: float, visible: np.ndarray):
    """Standard multi-head attention on expanded keys and values.

    For head h: K_h[s] = [W_UK[h] c_s ; k^R_s] (d_h + d_R values),
    V_h[s] = W_UV[h] c_s, q_h = [q_nope_h ; q_rot_h]; o_h = softmax(q_h K_h^T
    * scale) V_h over the visible tokens. q_nope [R, H, d_h], q_rot [R, H, d_r]
    for R query tokens; visible [R]. Returns o [R, H, d_h] and the attention
    weights [R, H, L].
    """
    R, H, dh = q_nope.shape
    L = C.shape[0]
    o = np.zeros((R, H, dh))
    A = np.zeros((R, H, L))
    for h in range(H):
        K = np.concatenate([C @ w_uk[h].T, KR], axis=1)      # [L, d_h + d_r]
        V = C @ w_uv[h].T                                    # [L, d_h]
        for r in range(R):
            q = np.concatenate([q_nope[r, h], q_rot[r, h]])
            n = int(visible[r])
            z = (K[:n] @ q) * scale
            e = np.exp(z - z.max())
            a = e / e.sum()
            A[r, h, :n] = a
            o[r, h] = a @ V[:n]
    return o, A


# ----------------------------------------------------------------------------
# Cache-size accounting (V2 analysis page, sections 1.3 and 6.1)
# ----------------------------------------------------------------------------


def mla_cache_elems_per_token_layer(d_c: int = 512, d_r: int = 64) -> int:
    """The latent plus one shared rope key."""
    return d_c + d_r


def mha_cache_elems_per_token_layer(n_heads: int, d_h: int) -> int:
    """Keys and values for every head."""
    return 2 * n_heads * d_h


def per_head_rope_elems_per_token_layer(d_c: int, d_r: int, n_heads: int) -> int:
    """Counterfactual: a separate rope key per head instead of a shared one."""
    return d_c + n_heads * d_r


def cache_bytes(elems_per_token_layer: int, n_layers: int, n_tokens: int,
                bits_per_elem: float) -> float:
    return elems_per_token_layer * n_layers * n_tokens * bits_per_elem / 8.0


def decode_cache_bytes_per_token(ckv_dt: str, kr_dt: str, d_c: int = 512, d_r: int = 64) -> int:
    """Bytes one cached token occupies in the paged pools (fp8 adds its fp32 scale)."""
    eb = {"f32": 4, "bf16": 2, "fp8": 1}
    return d_c * eb[ckv_dt] + d_r * eb[kr_dt] + (4 if ckv_dt == "fp8" else 0)


def decode_flops_per_row_token(d_c: int = 512, d_r: int = 64) -> int:
    """Multiply-adds of one (query row, cached token) pair, counted as 2 flops:
    the latent and rope dots (d_c + d_r) and the latent aggregation (d_c)."""
    return 2 * (d_c + d_r) + 2 * d_c
