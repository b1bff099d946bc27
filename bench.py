"""Decode-step benchmark of libspecache on one MI355X.

One step = one pass of the decode hot path over one batch of one layer:
  score_topk  (speculative row vs the low-bit copy C' -> top-k set for the next step)
  gather_fp16 (that set's 16-bit K/V rows from pinned host memory, on a side stream,
               double-buffered so it overlaps the following compute)
  decode_attn (both query rows over C' with the previous step's fetched rows substituted)
The prefill quantizer (quantize_pack) is timed separately, once per run.

Inputs are resident in HBM (C', queries) and pinned host memory (the 16-bit
cache) before the timed region starts.  Several copies of C' are rotated
between steps so that the 256 MB last-level cache does not hold them.

Prints one JSON line (see the README/DESIGN notes for the fields).

  python bench.py [--steps K] [--warmup W] [--workload mistral32k] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_attn_mistral32k_traffic.json")
ATTN_SOURCES = ("attention.hip", "mfma_frag.h", "common.h")


def attn_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_bit_kivi_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per decode_attn launch from the committed counter record, or None when
    the record is missing, is for another workload, or predates the current kernel sources."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("sources_sha256") != attn_sources_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mistral32k")
    ap.add_argument("--copies", type=int, default=0, help="C' copies rotated (0: enough for >= 512 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of the oracle sample")
    ap.add_argument("--mode", choices=("step", "copy"), default="step",
                    help="copy: a plain 1 GiB device-to-device copy, the reference for scaling the "
                         "profiler's HBM byte counters")
    return ap.parse_args()


def copy_reference(reps: int = 5):
    """A plain device copy of known size (1 GiB read + 1 GiB written per launch)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "us": us,
                      "GBs": 2 * n / (us * 1e-6) / 1e9}), flush=True)


def algorithmic_bytes_attn(cfg) -> int:
    """Bytes decode_attn must move per launch: C' (64 B per position per KV head
    at 1 bit, 96 B at 2 bits, D = 128), the k fetched 16-bit K and V rows, Q and O."""
    per_pos = 2 * (cfg.bits * cfg.head_dim // 8 + 4 * cfg.head_dim // 32)
    slices = cfg.batch * cfg.n_kv_heads
    rows = cfg.batch * cfg.n_q_heads * cfg.n_tokens
    return slices * (per_pos * cfg.seq_len + 2 * 2 * cfg.head_dim * cfg.top_k) + 2 * rows * cfg.head_dim * 2


def algorithmic_bytes_score(cfg) -> int:
    """Bytes score_topk must move per launch: the keys of C', the rank row, the top-k indices."""
    per_pos = cfg.bits * cfg.head_dim // 8 + 4 * cfg.head_dim // 32
    slices = cfg.batch * cfg.n_kv_heads
    return slices * (per_pos * cfg.seq_len + 4 * cfg.top_k) + cfg.batch * cfg.n_q_heads * cfg.head_dim * 2


def cpu_baseline(cfg, K, V, Q, budget_s: float):
    """The oracle's decode step (rank + top-k + gather + mixed attention) on a sample of
    (batch, KV head) slices, scaled to tokens/s of the whole workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    G = cfg.gqa
    slices = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_kv_heads)]
    rng = np.random.default_rng(0)
    order = [slices[i] for i in rng.permutation(len(slices))]
    spent, done = 0.0, 0
    for (b, h) in order:
        k1, v1 = K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1]
        q = Q[b:b + 1, h * G:(h + 1) * G]
        kc, kz, ks = oracle.quantize_keys(k1, cfg.bits)         # prefill: not timed
        vc, vz, vs = oracle.quantize_values(v1, cfg.bits)
        kh, vh = oracle.dequantize_keys(kc, kz, ks), oracle.dequantize_values(vc, vz, vs)
        t0 = time.perf_counter()
        idx, _ = oracle.score_topk(q, kh, 1, cfg.sm_scale, cfg.top_k)
        sk, sv = oracle.gather_rows(k1, v1, idx)
        oracle.mixed_attention(q, kh, vh, idx, sk, sv, sm_scale=cfg.sm_scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    per_slice = spent / done
    step_s = per_slice * len(slices)
    return {"value": cfg.batch / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(slices)} (batch, KV head) slices of one decode step "
                      f"({spent:.1f} s), scaled to the whole step; prefill quantization excluded",
            "seconds_per_step": step_s}


def main():
    args = parse()
    if args.mode == "copy":
        copy_reference()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; the path shards per (batch, KV head) "
                                   "slice with no exchange, see the design notes", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from decode_attention_bit_kivi_amd import (
        quantize_pack, score_topk, gather_fp16, decode_attn, empty_cache,
        score_topk_workspace_size, decode_attn_workspace_size,
    )
    from workloads import get_config, generate_all

    cfg = get_config(args.workload)
    B, Hq, Hkv, N, D, T, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim, cfg.n_tokens, cfg.top_k
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    K, V, Q, _, _, _ = generate_all(cfg)
    dev = torch.device("cuda:0")
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    k16 = torch.from_numpy(K).to(dev)
    v16 = torch.from_numpy(V).to(dev)
    hk = torch.from_numpy(K).pin_memory()
    hv = torch.from_numpy(V).pin_memory()
    q = torch.from_numpy(Q).to(dev)

    # prefill quantizer, timed on its own
    cache0 = empty_cache(B, Hkv, N, D, cfg.bits, dev)
    for _ in range(3):
        quantize_pack(k16, v16, cfg.bits, out=cache0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nq = 10
    e0.record()
    for _ in range(nq):
        quantize_pack(k16, v16, cfg.bits, out=cache0)
    e1.record()
    torch.cuda.synchronize()
    quant_us = e0.elapsed_time(e1) * 1e3 / nq

    copies = args.copies or max(3, math.ceil(512e6 / cache0.nbytes()))
    caches = [cache0] + [quantize_pack(k16, v16, cfg.bits) for _ in range(copies - 1)]
    del k16, v16
    torch.cuda.synchronize()

    ws_s = torch.empty(score_topk_workspace_size(cache0, Hq, T, k), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(decode_attn_workspace_size(cache0, Hq, T, k), dtype=torch.uint8, device=dev)
    idx_buf = [torch.zeros((B, Hkv, k), dtype=torch.int32, device=dev) for _ in range(2)]
    for i in range(2):
        idx_buf[i].copy_(torch.arange(k, dtype=torch.int32, device=dev).expand(B, Hkv, k))
    sel = [(torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev),
            torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev)) for _ in range(2)]
    out = torch.empty_like(q)
    gathered = [torch.cuda.Event() for _ in range(2)]
    scored = torch.cuda.Event()
    # step -1: fetch the initial set so the first step has rows to use
    gather_fp16(idx_buf[0], hk, hv, cfg.bits, *sel[0])
    gathered[0].record(comp)
    torch.cuda.synchronize()

    def step(i, ev=None):
        c = caches[i % copies]
        cur, nxt = i % 2, (i + 1) % 2
        if ev:
            ev["s0"].record(comp)
        score_topk(q, c, k, rank_row=1, idx_out=idx_buf[nxt], workspace=ws_s)
        if ev:
            ev["s1"].record(comp)
        scored.record(comp)
        side.wait_event(scored)
        if ev:
            ev["g0"].record(side)
        gather_fp16(idx_buf[nxt], hk, hv, cfg.bits, *sel[nxt], stream=side)
        if ev:
            ev["g1"].record(side)
        gathered[nxt].record(side)
        comp.wait_event(gathered[cur])
        if ev:
            ev["a0"].record(comp)
        decode_attn(q, c, idx_buf[cur], sel[cur][0], sel[cur][1], out=out, workspace=ws_a)
        if ev:
            ev["a1"].record(comp)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [{n: torch.cuda.Event(enable_timing=True) for n in ("s0", "s1", "g0", "g1", "a0", "a1")}
           for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(comp)
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    comp.wait_stream(side)
    t_end.record(comp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    score_us = np.array([e["s0"].elapsed_time(e["s1"]) for e in evs]) * 1e3
    gather_us = np.array([e["g0"].elapsed_time(e["g1"]) for e in evs]) * 1e3
    attn_us = np.array([e["a0"].elapsed_time(e["a1"]) for e in evs]) * 1e3

    # the same steps with the gather's result already resident: compute-only step time
    t_start.record(comp)
    for i in range(args.steps):
        c = caches[i % copies]
        score_topk(q, c, k, rank_row=1, idx_out=idx_buf[1], workspace=ws_s)
        decode_attn(q, c, idx_buf[0], sel[0][0], sel[0][1], out=out, workspace=ws_a)
    t_end.record(comp)
    torch.cuda.synchronize()
    ms_compute = t_start.elapsed_time(t_end) / args.steps

    attn_bytes = algorithmic_bytes_attn(cfg)
    attn_avg_s = float(attn_us.mean()) * 1e-6
    achieved = attn_bytes / attn_avg_s / 1e9
    score_bytes = algorithmic_bytes_score(cfg)
    gather_bytes = 2 * B * Hkv * k * D * 2

    result = {
        "metric": "decode-step attention latency + tokens/s; achieved HBM GB/s vs peak at 32K ctx",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: Mistral-7B-shaped single layer, batch {B}, {Hq} query / {Hkv} KV heads, "
                        f"head_dim {D}, context {N}, {T} query tokens, {cfg.bits}-bit K/V, group {cfg.group}, "
                        f"top-k {k} per KV head gathered from pinned host memory",
            "batch": B, "seq_len": N, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "bits": cfg.bits,
            "top_k": k, "n_tokens": T, "cache_copies_rotated": copies,
        },
        "roofline": {
            "kernel": "decode_attn (split-K attention + merge launches)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": recorded_traffic(cfg.name),
            "algorithmic_bytes_per_launch": attn_bytes,
        },
        "latency_us": {
            "step": ms_step * 1e3,
            "step_compute_only": ms_compute * 1e3,
            "exposed_gather": max(0.0, (ms_step - ms_compute) * 1e3),
            "score_topk": float(np.median(score_us)),
            "decode_attn": float(np.median(attn_us)),
            "decode_attn_mean": float(attn_us.mean()),
            "gather_fp16_side_stream": float(np.median(gather_us)),
            "quantize_pack_prefill": quant_us,
        },
        "bandwidth_GBs": {
            "decode_attn": achieved,
            "score_topk": score_bytes / (float(np.median(score_us)) * 1e-6) / 1e9,
            "gather_host_link": gather_bytes / (float(np.median(gather_us)) * 1e-6) / 1e9,
            "quantize_pack": (2 * B * Hkv * N * D * 2 + caches[0].nbytes()) / (quant_us * 1e-6) / 1e9,
        },
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host cores", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, K, V, Q, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
