"""Benchmark of the MLA absorbed-decode hot path on one MI355X.

One step = the whole path over one batch: mla_absorb_q_rope (the absorbed
content query and the rotated rope query, one launch) ->
mla_decode_paged (split kernel, then the log-sum-exp combine fused with the
per-head value up-projection W_UV), on the
DeepSeek-V2-shaped layer B=32, H=128, S=4096, bf16 (synthetic, seeded; see
mla_latent_kv_35_amd.synth). Inputs are resident in HBM before timing starts;
the step cycles through enough replicas of the 151 MB paged cache that the
256 MB Infinity Cache cannot serve it.

Prints one JSON line: whole-step throughput (tokens/s), the decode's HBM
bandwidth on latent-cache reads, the roofline of the dominant kernel (timed
with HIP events on the stream it runs on) and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 MFMA
METRIC = "MLA decode tokens/s + achieved HBM GB/s (% of peak), B=32 H=128 S=4096 bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_{}.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="dsv2_layer")
    ap.add_argument("--replicas", type=int, default=0, help="cache copies cycled (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the CPU-oracle baseline sample (0 = skip)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times "
                         "(the known-size reference for HBM byte counters)")
    return ap.parse_args()


def copy_probe(mib: int) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}))


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("decode_pipe.hip", "combine.hip", "dma.h", "mla_device.h", "mla_internal.h"):
        with open(os.path.join(ROOT, "mla_latent_kv_35_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per decode launch of this workload from the committed
    rocprofv3 counter runs, valid only while the kernel sources are the ones
    they were taken on."""
    try:
        with open(TRAFFIC_FILE.format(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float):
    """The oracle as it stands, on whole sequences of the same workload until
    the time budget is used; tokens/s in the benchmark's unit."""
    from threadpoolctl import threadpool_info
    from oracle import mla_oracle as O
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    done, t0 = 0, time.perf_counter()
    while done < inp.cfg.B and (time.perf_counter() - t0) < budget_s:
        O.decode_step(inp, batches=[done])
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(done * inp.cfg.T / el, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {inp.cfg.B} sequences of {inp.cfg.name} "
                      f"(L={int(inp.seq_lens[0])}, H={inp.cfg.H}), float64 numpy, {el:.1f} s"}


def main():
    a = parse()
    if a.copy_probe_mb:
        copy_probe(a.copy_probe_mb)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the decode path "
              "is single-GPU by design", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from mla_latent_kv_35_amd import binding as mla, synth
    from oracle import mla_oracle as O

    torch.cuda.set_device(0)
    inp = synth.make_inputs(a.config)
    cfg = inp.cfg
    d = mla.upload(inp)
    cache_bytes = inp.total_tokens * O.decode_cache_bytes_per_token(cfg.ckv_dt, cfg.kr_dt)
    R = a.replicas or max(1, int(np.ceil(640e6 / cache_bytes)))
    caches = [d.cache]
    for _ in range(R - 1):
        c = d.cache
        caches.append(mla.PagedCache(c.ckv.clone(), c.kr.clone(),
                                     None if c.ckv_scale is None else c.ckv_scale.clone(),
                                     c.block_table.clone(), c.seq_lens.clone(), c.max_seq_len,
                                     c.total_tokens))
    stream = torch.cuda.current_stream()
    u_dtype = torch.float32 if cfg.q_dt == "f32" else torch.bfloat16
    # outputs and workspace allocated once, outside the timed region
    BT, H = cfg.B * cfg.T, cfg.H
    q_lat = torch.empty((BT, H, 512), dtype=d.q_nope.dtype, device="cuda")
    q_rot = torch.empty_like(d.q_rope)
    u = torch.empty((BT, H, 512), dtype=u_dtype, device="cuda")
    lse = torch.empty((BT, H), dtype=torch.float32, device="cuda")
    o = torch.empty((BT, H, 128), dtype=u_dtype, device="cuda")
    _, n_split, ws = mla.decode_plan(mla.make_decode_args(q_lat, q_rot, d.cache, cfg.T,
                                                          cfg.softmax_scale, out=u))
    work = torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda")

    def step(i):
        c = caches[i % R]
        mla.absorb_q_rope(d.q_nope, d.w_uk, d.q_rope, d.positions, q_lat=q_lat, q_rot=q_rot)
        # the value up-projection runs inside the decode call (fused with the
        # log-sum-exp combine when the plan splits the sequences)
        mla.decode_paged(q_lat, q_rot, c, cfg.T, cfg.softmax_scale, out=u, lse=lse,
                         workspace=work, w_uv=d.w_uv, o=o)

    def decode_only(i):
        mla.decode_paged(q_lat, q_rot, caches[i % R], cfg.T, cfg.softmax_scale, out=u, lse=lse,
                         workspace=work)

    def capture(fn, n):
        # HIP graph of n consecutive calls (no allocation or memset inside)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(n):
                fn(j)
        return g

    per_graph = R * max(1, 10 // R)
    steps = max(1, a.steps)
    n_rep, rem = divmod(steps, per_graph)
    g_step = capture(step, per_graph)
    g_rem = capture(step, rem) if rem else None
    for _ in range(max(1, -(-a.warmup // per_graph))):
        g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_rep):
        g_step.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0

    # eager launches of the same step, for reference (host launch overhead included)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    el_eager = time.perf_counter() - t1

    # dominant kernel: back-to-back decode launches, timed with events on their stream
    g_dec = capture(decode_only, per_graph)
    g_dec.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    n_dec = max(1, n_rep)
    for _ in range(n_dec):
        g_dec.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    dur_ms = {"decode": e0.elapsed_time(e1) / (n_dec * per_graph)}

    # cache append of one step's new tokens (B*T), outside the step: into a
    # pool of the same shape, at the tokens' own positions
    c0 = caches[0]
    app_cache = mla.PagedCache(torch.empty_like(c0.ckv), torch.empty_like(c0.kr),
                               None if c0.ckv_scale is None else torch.empty_like(c0.ckv_scale),
                               c0.block_table, c0.seq_lens, c0.max_seq_len, c0.total_tokens)
    gen = torch.Generator(device="cuda").manual_seed(7)
    c_new = torch.randn((BT, 512), device="cuda", generator=gen).to(torch.bfloat16)
    k_new = torch.randn((BT, 64), device="cuda", generator=gen).to(torch.bfloat16)
    seq_new = torch.arange(cfg.B, device="cuda", dtype=torch.int32).repeat_interleave(cfg.T)
    g_app = capture(lambda i: mla.cache_append(app_cache, c_new, k_new, seq_new, d.positions,
                                               normalize=True), per_graph)
    g_app.replay()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a0.record(stream)
    for _ in range(n_dec):
        g_app.replay()
    a1.record(stream)
    torch.cuda.synchronize()
    dur_ms["append"] = a0.elapsed_time(a1) / (n_dec * per_graph)

    # prefill in the explicit form, one sequence of this workload's length
    # (at most 4096) and all heads: key/value expansion, then causal attention
    prefill = None
    if cfg.q_dt == "bf16":
        n = min(cfg.seq_len, 4096)
        gen = torch.Generator(device="cuda").manual_seed(11)
        c_p = torch.randn((n, 512), device="cuda", generator=gen).to(torch.bfloat16)
        kr_p = torch.randn((1, n, 64), device="cuda", generator=gen).to(torch.bfloat16)
        qn_p = torch.randn((1, n, H, 128), device="cuda", generator=gen).to(torch.bfloat16)
        qr_p = torch.randn((1, n, H, 64), device="cuda", generator=gen).to(torch.bfloat16)
        k_p, v_p = mla.expand_kv(c_p, d.w_uk, d.w_uv)
        k_p, v_p = k_p.view(1, n, H, 128), v_p.view(1, n, H, 128)
        o_p = torch.empty((1, n, H, 128), dtype=torch.bfloat16, device="cuda")

        def timed(fn, reps=5):
            g = capture(lambda i: fn(), reps)
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(4):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / (4 * reps)

        attn_ms = timed(lambda: mla.prefill_attn(qn_p, qr_p, k_p, kr_p, v_p, cfg.softmax_scale,
                                                 want_lse=False, out=o_p))
        exp_ms = timed(lambda: mla.expand_kv(c_p, d.w_uk, d.w_uv))
        pf_flops = H * (n * (n + 1) / 2) * 2 * (192 + 128)
        prefill = {"workload": f"one sequence, n_q = n_kv = {n}, H = {H}, causal, bf16",
                   "attn_ms": round(attn_ms, 4),
                   "attn_tflops": round(pf_flops / (attn_ms * 1e-3) / 1e12, 1),
                   "mfma_frac_bf16": round(pf_flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "expand_ms": round(exp_ms, 4)}

    # context: what a plain device-to-device copy reaches on this GPU (read +
    # write bytes over time; 1 GiB each way, well past the 256 MB Infinity Cache)
    n_cp = 1 << 30
    cp_src = torch.ones(n_cp, dtype=torch.uint8, device="cuda")
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    c0e, c1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0e.record(stream)
    for _ in range(5):
        cp_dst.copy_(cp_src)
    c1e.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * n_cp * 5 / (c0e.elapsed_time(c1e) * 1e-3) / 1e9
    del cp_src, cp_dst
    # and what a plain streaming read reaches (mla_stream_read over 2 GiB: the
    # bound the decode's cache reads are held against)
    n_rp = 2 << 30
    rp_src = torch.ones(n_rp, dtype=torch.uint8, device="cuda")
    rp_sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    mla.stream_read(rp_src, rp_sink)
    r0e, r1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0e.record(stream)
    for _ in range(5):
        mla.stream_read(rp_src, rp_sink)
    r1e.record(stream)
    torch.cuda.synchronize()
    read_gbps = n_rp * 5 / (r0e.elapsed_time(r1e) * 1e-3) / 1e9
    del rp_src, rp_sink

    tokens = cfg.B * cfg.T
    value = tokens * steps / el
    dec_s = dur_ms["decode"] * 1e-3
    achieved = cache_bytes / dec_s / 1e9
    flops = inp.total_tokens * cfg.H * cfg.T * O.decode_flops_per_row_token()
    traffic = load_traffic(cfg.name)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": a.warmup,
        "ms_per_step": round(el / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8+bf16"}[cfg.ckv_dt],
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "T": cfg.T,
                   "seq_len": cfg.seq_len, "d_c": 512, "d_r": 64, "page": 64,
                   "cache_dtype": cfg.ckv_dt, "n_split": n_split, "cache_replicas": R},
        "hbm_gbps": round(achieved, 1),
        "hbm_pct_of_peak": round(100 * achieved / PEAK_HBM_GBPS, 2),
        "decode_ms": round(dur_ms["decode"], 5),
        "eager_ms_per_step": round(el_eager / steps * 1e3, 5),
        "append_ms": round(dur_ms["append"], 5),
        "prefill": prefill,
        "copy_context": {"what": "torch device-to-device copy of 1 GiB, read + write bytes / time",
                         "gbps": round(copy_gbps, 1),
                         "decode_hbm_over_copy": round(achieved / copy_gbps, 4)},
        "read_probe": {"what": "mla_stream_read of 2 GiB (16-byte loads, read only)",
                       "gbps": round(read_gbps, 1),
                       "decode_hbm_over_read": round(achieved / read_gbps, 4)},
        "launch": "hip graph of %d steps per replay" % per_graph,
        "roofline": {
            "kernel": ("mla_decode_paged: split-KV kernel (decode_pipe_kernel, bf16 and fp8 "
                       "pools) + log-sum-exp combine, timed together"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            # the counted HBM bytes (cache, queries, split partials) over the same time
            "traffic_gbps": None if traffic is None else round(traffic / dec_s / 1e9, 1),
            "algorithmic_bytes_per_launch": cache_bytes,
            "mfma_tflops": round(flops / dec_s / 1e12, 1),
            "mfma_frac_bf16": round(flops / dec_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
    }
    if a.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(inp, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
