"""Decode-step benchmark of libspecache on one MI355X.

One step = one layer's pass of the decode hot path over one batch:
  decode_step (both query rows over C' with this layer's fetched 16-bit rows
               substituted, and, from the same pass, the speculative row's
               ranking and top-k selection for the layer's next step)
  gather      (that selection's 16-bit K/V rows into the layer's other row
               buffer: rows the previous selection also held are copied on the
               device (gather_reuse), the others fetched from pinned host
               memory on a side stream limited to a few compute units
               (gather_fp16_missing); with --no-reuse every row is fetched)
as in the multi-layer decode loop: several layers, each with its own low-bit
cache C', selection and fetched rows, run in turn, and a layer's gather
overlaps the other layers' compute until the layer comes round again.  The
layers' C' copies together exceed the 256 MB last-level cache, so every step
reads its C' from HBM.  The layers share one pinned host copy of the 16-bit
cache (every gather still crosses the host link).  The prefill quantizer
(quantize_pack) is timed separately, once per run.

Inputs are resident in HBM (C', queries) and pinned host memory (the 16-bit
cache) before the timed region starts.  Each step of a layer takes the next of
8 fresh query draws from the workload's distribution; the planted positions
stay relevant to all of them, the rest of each top-k set is the step's own.

Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload mistral32k] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_step_mistral32k_traffic.json")
STEP_SOURCES = ("attention.hip", "attention_stream.hip", "rank.hip", "merge.h", "mfma_frag.h", "common.h")


def step_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in STEP_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_bit_kivi_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per decode_step call from the committed counter record, or None when
    the record is missing, is for another workload, or predates the current kernel sources."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("sources_sha256") != step_sources_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def round_up(x: int, m: int) -> int:
    return -(-x // m) * m


def pipeline_schedule(warmup: int, steps: int, sync_every: int):
    """Step indices of the three passes of the pipeline: (warm-up, timed, instrumented).

    A step's index picks its layer and its synchronisation group (sync_every consecutive
    indices, whose gathers are issued together after the group's last step).  Any counts are
    accepted: a pass that ends inside a group flushes that group's gathers at its end, so the
    timed pass covers exactly `steps` steps and all of their gathers; the next pass starts at
    the next whole group.  The instrumented pass (per-call events) runs whole groups only."""
    if warmup < 0 or steps < 1 or sync_every < 1:
        raise ValueError("need warmup >= 0, steps >= 1 and sync_every >= 1")
    w = list(range(warmup))
    t0 = round_up(warmup, sync_every)
    t = list(range(t0, t0 + steps))
    i0 = round_up(t0 + steps, sync_every)
    n_i = round_up(steps, sync_every)
    return w, t, list(range(i0, i0 + n_i))


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mistral32k")
    ap.add_argument("--copies", type=int, default=0, help="layers (C' copies) in turn (0: enough for >= 512 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of the oracle sample")
    ap.add_argument("--gather-cus", type=int, default=16, help="compute units of the gather stream")
    ap.add_argument("--compute-stream", choices=("exclusive", "shared"), default="exclusive",
                    help="exclusive: the compute runs on the compute units the gather stream does not use")
    ap.add_argument("--reuse", action=argparse.BooleanOptionalAction, default=True,
                    help="fetch only the rows of the new top-k not already resident (the step time of "
                         "fetching every row is reported beside it)")
    ap.add_argument("--host-copies", choices=("per-layer", "shared"), default="per-layer",
                    help="the 16-bit cache in pinned host memory: a copy per layer in turn, or one shared")
    ap.add_argument("--top-k", type=int, default=0, help="override the workload's top-k (latency-vs-k sweeps)")
    ap.add_argument("--sync-every", type=int, default=2, choices=(1, 2, 4),
                    help="steps per cross-stream synchronisation of the pipeline (at most half the layers "
                         "in turn: the gathers of a group of steps must land before the group's layers return)")
    ap.add_argument("--rank", choices=("lowbit", "mixed"), default="lowbit",
                    help="lowbit: rank against C'; mixed: by the attention row itself (fetched rows and tail in)")
    ap.add_argument("--compute-reserve", type=int, default=32,
                    help="with an exclusive compute stream: the low compute units kept from it (the "
                         "gather's among them); 32 leaves every shader engine the same number of units")
    ap.add_argument("--mode", choices=("step", "copy", "traffic-record"), default="step",
                    help="copy: a plain 1 GiB device-to-device copy, the reference for scaling the "
                         "profiler's HBM byte counters; traffic-record: write the HBM traffic record "
                         "from the four counter runs under --pmc-root (see traffic_commands)")
    ap.add_argument("--pmc-root", default="counters", help="directory holding the counter runs")
    return ap.parse_args(argv)


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


MODEL_SHAPE = {"tiny": "tiny", "llama8k": "Llama-3-8B-shaped", "mistral32k": "Mistral-7B-shaped",
               "layers32": "Llama-3-8B-shaped", "long128k": "long-context (Llama/Mistral-shaped heads)"}
TRAFFIC_KERNELS = "attn_split|attn_stream|rank_keys|rank_select|attn_merge"


def traffic_commands(root: str):
    """The runs a traffic record is made from, their counter output under `root`."""
    return [
        f"rocprofv3 --pmc FETCH_SIZE -f csv -d {root}/pmc_copy_fetch -o run -- python -u bench.py --mode copy",
        f"rocprofv3 --pmc WRITE_SIZE -f csv -d {root}/pmc_copy_write -o run -- python -u bench.py --mode copy",
        f"rocprofv3 --kernel-include-regex '{TRAFFIC_KERNELS}' --pmc FETCH_SIZE -f csv -d {root}/pmc_fetch "
        "-o run -- python -u bench.py --steps 4 --warmup 2 --no-cpu-baseline",
        f"rocprofv3 --kernel-include-regex '{TRAFFIC_KERNELS}' --pmc WRITE_SIZE -f csv -d {root}/pmc_write "
        "-o run -- python -u bench.py --steps 4 --warmup 2 --no-cpu-baseline",
        f"python bench.py --mode traffic-record --pmc-root {root}",
    ]


def _counter_rows(root: str, run: str, counter: str):
    """(queue, dispatch id, kernel name, value) of every dispatch in one rocprofv3 counter run."""
    import csv
    import glob
    files = glob.glob(os.path.join(root, run, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter collection under {os.path.join(root, run)}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Queue_Id"], int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort(key=lambda x: x[1])
    return rows


def write_traffic_record(root: str, workload: str = "mistral32k"):
    """HBM bytes per decode_step call from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for the plain 1 GiB copy.  A call is the fused-step
    split dispatch and the selection dispatches that follow it on its queue (rank_keys, for
    slices that one selection workgroup cannot hold, then rank_select)."""
    import statistics
    cal = {}
    for counter, run in (("FETCH_SIZE", "pmc_copy_fetch"), ("WRITE_SIZE", "pmc_copy_write")):
        vals = [v for _, _, name, v in _counter_rows(root, run, counter) if "copy" in name.lower()]
        cal[counter] = statistics.median(vals)
    n = 1 << 30
    scale = {"FETCH_SIZE": n / (cal["FETCH_SIZE"] * 1024), "WRITE_SIZE": n / (cal["WRITE_SIZE"] * 1024)}
    per = {}
    for counter, run in (("FETCH_SIZE", "pmc_fetch"), ("WRITE_SIZE", "pmc_write")):
        after_split = {}
        for queue, _, name, v in _counter_rows(root, run, counter):
            fused = re.search(r"attn_split_kernel<[^>]*, true, false>|attn_stream_kernel<[12]>", name)
            if fused:  # the split kernel with ranking outputs (the streamed one, or the general one)
                kind = fused.group(0)
                after_split[queue] = True
            elif after_split.get(queue) and ("rank_keys" in name or "rank_select" in name):
                kind = "rank_keys_kernel" if "rank_keys" in name else "rank_select (with the split merge)"
                if "rank_select" in name:
                    after_split[queue] = False
            else:
                if "attn_split" in name or "attn_stream" in name:
                    after_split[queue] = False
                continue
            per.setdefault(kind, {}).setdefault(counter, []).append(v)
    out = {}
    total = 0.0
    for kind, d in per.items():
        f_kib = statistics.mean(d["FETCH_SIZE"])
        w_kib = statistics.mean(d["WRITE_SIZE"])
        fb, wb = f_kib * 1024 * scale["FETCH_SIZE"], w_kib * 1024 * scale["WRITE_SIZE"]
        out[kind] = {"dispatches": len(d["FETCH_SIZE"]), "fetch_kib_raw": round(f_kib), "write_kib": round(w_kib),
                     "fetch_bytes": round(fb), "write_bytes": round(wb)}
        total += fb + wb
    from workloads import get_config
    rec = {
        "workload": workload,
        "what": "HBM bytes per specache_decode_step call: the kernels it launches (the split, then the "
                "selection: rank_select alone, or rank_keys and rank_select for slices longer than one "
                "selection workgroup holds), each dispatch taken right after a fused-step split dispatch on "
                "its queue; rocprofv3 FETCH_SIZE and WRITE_SIZE "
                "per dispatch, scaled by the same counters' reading for a plain 1 GiB device copy",
        "commands": traffic_commands(root),
        "calibration": {"copy_bytes_read": n, "copy_bytes_written": n,
                        "FETCH_SIZE_kib": round(cal["FETCH_SIZE"]), "WRITE_SIZE_kib": round(cal["WRITE_SIZE"]),
                        "fetch_scale": round(scale["FETCH_SIZE"], 4), "write_scale": round(scale["WRITE_SIZE"], 4)},
        "per_kernel": out,
        "traffic_bytes_per_launch": round(total),
        "algorithmic_bytes_per_launch": algorithmic_bytes_step(get_config(workload)),
        "sources_sha256": step_sources_hash(),
    }
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"traffic_bytes_per_launch": rec["traffic_bytes_per_launch"], "per_kernel": out}))


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence: recording it adds no system-scope
    release fence (an L2 write-back for the host's sake) to the stream, only the device-scope
    one, which is all another stream of the same GPU needs.  As a timing event it perturbs the
    calls it brackets far less than a default event (its timestamp is taken at the same point
    of the stream); with timing=False it orders streams (wait).  Called through the HIP runtime
    the process has loaded (torch's)."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded")
            cls._hip = ctypes.CDLL(paths[0])
        return cls._hip

    def __init__(self, timing: bool = True):
        import ctypes
        self._c = ctypes
        self.ev = ctypes.c_void_p()
        flags = 0x20000000 | (0 if timing else 0x2)  # hipEventDisableSystemFence [| hipEventDisableTiming]
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(flags))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self._runtime().hipEventRecord(self.ev, self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def wait(self, stream):
        """Work enqueued on `stream` after this call waits for the event's last record."""
        rc = self._runtime().hipStreamWaitEvent(self._c.c_void_p(stream.cuda_stream), self.ev, self._c.c_uint(0))
        if rc != 0:
            raise RuntimeError(f"hipStreamWaitEvent failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both completed)."""
        ms = self._c.c_float()
        rc = self._runtime().hipEventElapsedTime(self._c.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            self._runtime().hipEventDestroy(self.ev)
        except Exception:
            pass


def algorithmic_bytes_step(cfg) -> int:
    """Bytes one decode_step call must move: C' (keys and values: codes plus float16
    zero-points and scales, 64 B per position per KV head at 1 bit and D = 128, 96 B at
    2 bits), the k fetched 16-bit K and V rows and their indices, the next selection,
    the queries and the output."""
    per_pos = 2 * (cfg.bits * cfg.head_dim // 8 + 4 * cfg.head_dim // 32)
    slices = cfg.batch * cfg.n_kv_heads
    rows = cfg.batch * cfg.n_q_heads * cfg.n_tokens
    per_slice = per_pos * cfg.seq_len + (2 * 2 * cfg.head_dim + 4) * cfg.top_k + 4 * cfg.top_k
    return slices * per_slice + 2 * rows * cfg.head_dim * 2


def decode_attn_fp16_workspace_size_bytes(cfg) -> int:
    import ctypes
    from decode_attention_bit_kivi_amd import _lib
    shape = _lib.Shape(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len, cfg.bits, 32, 0)
    return int(_lib.load().specache_decode_attn_fp16_workspace_size(ctypes.byref(shape), cfg.n_tokens, 0))


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
    spent, done, passes = 0.0, 0, 0
    while spent < budget_s and passes < 50:   # cycle over the slices until the budget is spent
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
        passes += 1
    per_slice = spent / done
    step_s = per_slice * len(slices) * cfg.n_layers
    return {"value": cfg.batch / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} (batch, KV head) slice-steps ({passes} pass(es) over the {len(slices)} slices "
                      f"of one layer's decode step, {spent:.1f} s of oracle time), scaled to the whole step; "
                      f"prefill quantization excluded",
            "seconds_per_step": step_s}


# The library's streams, held past main(): torch's pinned-memory allocator records an event on
# every stream a pinned block was copied on when the block is freed, so the streams must outlive
# the pinned tensors on every way out of main() (an error included), not only the normal end.
_LIB_STREAMS = []


def main():
    args = parse()
    if args.mode == "copy":
        copy_reference()
        return
    if args.mode == "traffic-record":
        write_traffic_record(args.pmc_root, args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; the path shards per (batch, KV head) "
                                   "slice with no exchange, see the design notes", "n_gpus": args.gpus}))
        sys.exit(2)

    warm_idx, timed_idx, instr_idx = pipeline_schedule(args.warmup, args.steps, args.sync_every)

    import torch
    from decode_attention_bit_kivi_amd import (
        quantize_pack, score_topk, gather_fp16, decode_attn, decode_step, empty_cache,
        score_topk_workspace_size, decode_attn_workspace_size, decode_step_workspace_size, GatherStream,
        ComputeStream, gather_reuse, gather_fp16_missing, decode_attn_fp16,
    )
    from workloads import get_config, generate_all, generate_step_queries

    cfg = get_config(args.workload)
    if args.top_k:
        cfg = cfg.with_(top_k=args.top_k)
    B, Hq, Hkv, N, D, T, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim, cfg.n_tokens, cfg.top_k
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    K, V, Q, _, _, _ = generate_all(cfg)
    dev = torch.device("cuda:0")
    # compute on a non-default stream: the CU-limited gather stream is a blocking stream and
    # would serialize with the legacy default stream
    gather_stream = GatherStream(args.gather_cus)   # the prefetch runs on a few CUs only
    side = gather_stream.torch
    _LIB_STREAMS.append(gather_stream)
    if args.compute_stream == "exclusive":
        compute_stream = ComputeStream(max(args.compute_reserve, args.gather_cus))
        comp = compute_stream.torch
        _LIB_STREAMS.append(compute_stream)
    else:
        comp = torch.cuda.Stream()
    torch.cuda.set_stream(comp)

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

    layers = args.copies or max(3, cfg.n_layers, math.ceil(512e6 / cache0.nbytes()))
    layers = max(layers, 2 * args.sync_every)  # a group's gathers land while the next group computes
    layers = -(-layers // args.sync_every) * args.sync_every  # whole synchronisation groups
    caches = [cache0] + [quantize_pack(k16, v16, cfg.bits) for _ in range(layers - 1)]
    torch.cuda.synchronize()
    # each layer's 16-bit K and V in pinned host memory of its own (as a model offloads every
    # layer); one copy shared by all layers only when pinning that much fails
    hks, hvs = [hk], [hv]
    host_copies = "per-layer"
    if args.host_copies == "per-layer":
        try:
            for _ in range(layers - 1):
                hks.append(torch.empty(hk.shape, dtype=hk.dtype, pin_memory=True).copy_(hk))
                hvs.append(torch.empty(hv.shape, dtype=hv.dtype, pin_memory=True).copy_(hv))
        except RuntimeError as e:
            hks, hvs = [hk], [hv]
            host_copies = f"shared (pinning a copy per layer failed: {str(e).splitlines()[0][:120]})"
    else:
        host_copies = "shared"
    print(f"[bench] host copies of the 16-bit cache: {host_copies}", file=sys.stderr, flush=True)

    def host_kv(l):
        return (hks[l], hvs[l]) if len(hks) > 1 else (hk, hv)

    ws = torch.empty(decode_step_workspace_size(cache0, Hq, T, k, 0, k), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(score_topk_workspace_size(cache0, Hq, T, k), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(decode_attn_workspace_size(cache0, Hq, T, k), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    # every step of a layer takes the next of n_q fresh query draws (same distribution)
    print("[bench] drawing the step queries", file=sys.stderr, flush=True)
    n_q = 8
    qs_np = generate_step_queries(cfg, n_q)
    qs = [torch.from_numpy(qs_np[i]).to(dev) for i in range(n_q)]
    mixed = args.rank == "mixed"
    # the streams' synchronisation events: device-scope release only (both streams are on this
    # GPU); a default event's system-scope fence cost the step ~1.3 µs.  (A device-flag wait,
    # specache_flag_wait, took the gather stream's barrier off but not the step's time, and
    # cannot run where the dispatches are serialised, as under the profiler's counters.)
    gathered = [HipEvent(timing=False) for _ in range(layers)]
    stepped = [HipEvent(timing=False) for _ in range(layers)]

    def compute_then_side(slot=0):
        """Later work on the gather stream runs after everything enqueued on the compute stream."""
        stepped[slot].record(comp)
        stepped[slot].wait(side)
    sync_every = args.sync_every  # steps per cross-stream synchronisation (a divisor of the layers)

    def new_state():
        """Per layer: two selections and two row buffers in turn (the step reads one pair and
        its ranking fills the other), seeded by a pre-decoding score_topk + gather."""
        st = {"occ": [0] * layers, "idx": [], "sel": [], "fetch": [], "pending": []}
        for l in range(layers):
            i0 = score_topk(qs[n_q - 1], caches[l], k, rank_row=1, workspace=ws_s)
            st["idx"].append([i0, torch.empty_like(i0)])
            st["sel"].append([gather_fp16(i0, *host_kv(l), cfg.bits),
                              (torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev),
                               torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev))])
            st["fetch"].append(torch.empty_like(i0))
            gathered[l].record(comp)
        torch.cuda.synchronize()
        return st

    def step(st, i, reuse, ev=None):
        """Step i of the pipeline (layer i mod layers).  The streams synchronise once per
        sync_every steps: the compute stream waits for the gathers of the group of steps two
        groups back (the gather stream runs in order, so the group's event covers each of them),
        and after the group's last step the gather stream fetches the rows of the whole group."""
        def mark(name, stream):
            if ev and name in ev:
                ev[name].record(stream)

        l = i % layers
        r = st["occ"][l]
        st["occ"][l] += 1
        cur, nxt = r % 2, 1 - r % 2
        idx_c, idx_n = st["idx"][l][cur], st["idx"][l][nxt]
        sel_c, sel_n = st["sel"][l][cur], st["sel"][l][nxt]
        grp = (i // sync_every) % (layers // sync_every)  # event slot of this group
        if i % sync_every == 0:
            gathered[grp].wait(comp)
        mark("d0", comp)
        decode_step(qs[r % n_q], caches[l], k, rank_row=1, rank_mixed=mixed, idx=idx_c, k_sel=sel_c[0],
                    v_sel=sel_c[1], out=out, idx_next_out=idx_n, workspace=ws)
        mark("d1", comp)
        if reuse:  # rows of the new set already resident: device copy on the compute stream
            gather_reuse(idx_n, idx_c, sel_c[0], sel_c[1], N, k_sel=sel_n[0], v_sel=sel_n[1],
                         fetch_idx=st["fetch"][l])
        st["pending"].append((l, idx_n, sel_n))
        st["grp"] = grp
        if i % sync_every == sync_every - 1:
            flush(st, reuse, ev)

    def flush(st, reuse, ev=None):
        """The gathers of the steps enqueued since the last flush, on the gather stream after
        the compute stream's work: at the end of every group of sync_every steps, and at the
        end of a pass that stops inside a group."""
        if not st["pending"]:
            return
        grp = st["grp"]
        compute_then_side(grp)
        if ev and "g0" in ev:
            ev["g0"].record(side)
        for (pl, pidx, psel) in st["pending"]:
            if reuse:
                gather_fp16_missing(st["fetch"][pl], *host_kv(pl), psel[0], psel[1], cfg.bits, stream=side)
            else:
                gather_fp16(pidx, *host_kv(pl), cfg.bits, psel[0], psel[1], stream=side)
        if ev and "g1" in ev:
            ev["g1"].record(side)
        st["pending"] = []
        gathered[grp].record(side)

    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run_pipeline(reuse):
        """(ms per step, decode_step µs per call in the pipeline, gather µs, fetched fraction).

        The timed region holds no timing events but its own two (each timing event costs the
        stream a few µs); the per-call durations are taken in an instrumented pass after it
        (fence-free HipEvents),
        the same schedule with events around every decode_step and every gather."""
        st = new_state()
        for i in warm_idx:
            step(st, i, reuse)
        flush(st, reuse)
        torch.cuda.synchronize()
        t_start.record(comp)
        h0 = time.perf_counter()
        for i in timed_idx:
            step(st, i, reuse)
        flush(st, reuse)   # a last group cut short: its gathers are part of the timed steps
        host_enqueue_us.append((time.perf_counter() - h0) / len(timed_idx) * 1e6)  # host time to enqueue a step
        comp.wait_stream(side)
        t_end.record(comp)
        torch.cuda.synchronize()
        ms = t_start.elapsed_time(t_end) / len(timed_idx)
        fetched = None
        if reuse:
            fetched = float(np.mean([(f >= 0).float().mean().item() for f in st["fetch"]]))
        evs = [{n: HipEvent() for n in ("d0", "d1", "g0", "g1")} for _ in instr_idx]
        for i, ev in zip(instr_idx, evs):
            step(st, i, reuse, ev)
        torch.cuda.synchronize()
        d_us = np.array([e["d0"].elapsed_time(e["d1"]) for e in evs]) * 1e3
        # gathers are issued per group of sync_every steps, bracketed at the group's last step
        g_us = np.array([ev["g0"].elapsed_time(ev["g1"]) for i, ev in zip(instr_idx, evs)
                         if i % sync_every == sync_every - 1]) * 1e3 / sync_every
        return ms, d_us, g_us, fetched

    host_enqueue_us = []
    modes = ["reuse", "full"] if args.reuse else ["full"]
    runs = {}
    for m in modes:
        print(f"[bench] {m} fetch: {args.warmup} warmup + {args.steps} timed steps over {layers} layers",
              file=sys.stderr, flush=True)
        runs[m] = run_pipeline(m == "reuse")
    ms_step, step_us, gather_us, fetched = runs[modes[0]]

    # compute only (the fetched rows already resident): the fused step, then the four-call
    # form (score_topk + decode_attn) on the same inputs
    def compute_loop(fn):
        for i in range(3):
            fn(i)
        t_start.record(comp)
        for i in range(args.steps):
            fn(i)
        t_end.record(comp)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps * 1e3

    st = new_state()
    nxt = torch.empty_like(st["idx"][0][0])
    fused_us = compute_loop(lambda i: decode_step(
        qs[i % n_q], caches[i % layers], k, rank_row=1, rank_mixed=mixed, idx=st["idx"][i % layers][0],
        k_sel=st["sel"][i % layers][0][0], v_sel=st["sel"][i % layers][0][1], out=out, idx_next_out=nxt,
        workspace=ws))
    unfused_us = compute_loop(lambda i: (
        score_topk(qs[i % n_q], caches[i % layers], k, rank_row=1, idx_out=nxt, workspace=ws_s),
        decode_attn(qs[i % n_q], caches[i % layers], st["idx"][i % layers][0], st["sel"][i % layers][0][0],
                    st["sel"][i % layers][0][1], out=out, workspace=ws_a)))

    # comparators (SpeCache summary: the 16-bit decoding its throughput ratios are taken against,
    # §5 Table 3; the non-speculative serial fetch of Table 4)
    ws16 = torch.empty(decode_attn_fp16_workspace_size_bytes(cfg), dtype=torch.uint8, device=dev)
    fp16_us = compute_loop(lambda i: decode_attn_fp16(qs[i % n_q], k16, v16, out=out, workspace=ws16))
    fp16_bytes = 2 * B * Hkv * N * D * 2 + 2 * B * Hq * T * D * 2
    serial_rows = [(torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev),
                    torch.empty((B, Hkv, k, D), dtype=torch.float16, device=dev)) for _ in range(2)]
    serial_idx = torch.empty_like(st["idx"][0][0])

    def serial_step(i):
        """Rank with the real token against C', fetch its top-k (no overlap), then attend."""
        c = caches[i % layers]
        score_topk(qs[i % n_q], c, k, rank_row=0, idx_out=serial_idx, workspace=ws_s)
        compute_then_side()
        gather_fp16(serial_idx, hk, hv, cfg.bits, *serial_rows[i % 2], stream=side)
        gathered[0].record(side)
        gathered[0].wait(comp)
        decode_attn(qs[i % n_q], c, serial_idx, serial_rows[i % 2][0], serial_rows[i % 2][1], out=out,
                    workspace=ws_a)

    serial_us = compute_loop(serial_step)

    # the host link's contiguous rate: one pinned-host-to-device copy of as many bytes as the
    # gather of every top-k row moves (the pages found scattered row copies several times slower
    # than one contiguous copy)
    n_gather = 2 * B * Hkv * k * D * 2
    h_blk = torch.empty(n_gather, dtype=torch.uint8).pin_memory()
    d_blk = torch.empty(n_gather, dtype=torch.uint8, device=dev)
    h2d_us = compute_loop(lambda i: d_blk.copy_(h_blk, non_blocking=True))
    del h_blk, d_blk
    # offloading the whole layer instead (the pages' full-offload comparison): the layer's 16-bit
    # K and V copied from pinned host memory into HBM
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k16.copy_(hk, non_blocking=True)
    e0.record(comp)
    for _ in range(2):
        k16.copy_(hk, non_blocking=True)
        v16.copy_(hv, non_blocking=True)
    e1.record(comp)
    torch.cuda.synchronize()
    full_layer_us = e0.elapsed_time(e1) * 1e3 / 2

    step_bytes = algorithmic_bytes_step(cfg)
    step_avg_s = float(step_us.mean()) * 1e-6
    achieved = step_bytes / step_avg_s / 1e9
    fused_bw = step_bytes / (fused_us * 1e-6) / 1e9
    gather_bytes = 2 * B * Hkv * k * D * 2
    result = {
        "metric": "decode-step attention latency + tokens/s; achieved HBM GB/s vs peak at 32K ctx",
        # a model with several layers: one decode step runs every layer once
        "value": B / (ms_step * cfg.n_layers * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step * cfg.n_layers,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # float16 operands on the matrix cores (queries, fetched rows, expanded codes) with float32
        # accumulation; K/V stored as cfg.bits-bit codes with float16 zero-points and scales
        "dtype": "f16",
        "precision": {"queries_outputs_fetched_rows": "float16",
                      "kv_cache": f"{cfg.bits}-bit codes, float16 zero-point/scale per group of {cfg.group}",
                      "accumulation": "float32"},
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {MODEL_SHAPE.get(cfg.name, 'synthetic')} layer, batch {B}, {Hq} query / {Hkv} KV heads, "
                        f"head_dim {D}, context {N}, {T} query tokens, {cfg.bits}-bit K/V, group {cfg.group}, "
                        f"top-k {k} per KV head gathered from pinned host memory; {layers} layers in turn",
            "batch": B, "seq_len": N, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "bits": cfg.bits,
            "top_k": k, "n_tokens": T, "layers_rotated": layers, "model_layers": cfg.n_layers,
            "layer_step_ms": ms_step, "gather_stream_cus": args.gather_cus,
            "compute_stream": args.compute_stream, "rank": args.rank, "sync_every": args.sync_every,
            "fetch": "resident rows reused, only new top-k rows fetched" if args.reuse else "every top-k row fetched",
            "queries": f"fresh draws every step ({n_q} in turn), planted peak shared",
            "host_copies": host_copies,
            "compute_stream_reserved_cus": max(args.compute_reserve, args.gather_cus)
            if args.compute_stream == "exclusive" else 0,
        },
        "roofline": {
            "kernel": "decode_step (the split kernel with ranking outputs: attn_stream_kernel<1> for 1-bit "
                      "codes at head_dim 128, attn_split_kernel otherwise; then " + (
                "rank_select_pruned: r(p) of the position groups whose 8-position bound reaches the k-th "
                "rank, the top-k and the merge of the splits)" if N <= 32768 and Hq // Hkv <= 4 and k <= N // 8 else
                "rank_select forming r(p), the top-k and the merge of the splits)" if N <= 32768 and Hq // Hkv <= 4
                else "rank_keys + rank_select merging the splits)"),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": recorded_traffic(cfg.name),
            "algorithmic_bytes_per_launch": step_bytes,
        },
        "latency_us": {
            "step": ms_step * 1e3,
            "step_full_fetch": runs["full"][0] * 1e3,
            "decode_step_in_pipeline": float(np.median(step_us)),
            "decode_step_in_pipeline_mean": float(step_us.mean()),
            "decode_step_in_pipeline_p10": float(np.percentile(step_us, 10)),
            "decode_step_in_pipeline_p90": float(np.percentile(step_us, 90)),
            "gather_fp16_side_stream": float(np.median(gather_us)),
            "gather_full_fetch": float(np.median(runs["full"][2])),
            "step_compute_only_fused": fused_us,
            "step_compute_only_four_call": unfused_us,
            "exposed_gather": max(0.0, ms_step * 1e3 - fused_us),
            "quantize_pack_prefill": quant_us,
            "host_enqueue_per_step": host_enqueue_us[0],
        },
        "bandwidth_GBs": {
            "decode_step_in_pipeline": achieved,
            "decode_step_compute_only": fused_bw,
            "gather_host_link": gather_bytes / (float(np.median(runs["full"][2])) * 1e-6) / 1e9,
            "gather_host_link_whole_step": gather_bytes * (fetched if fetched is not None else 1.0)
            / (ms_step * 1e-3) / 1e9,
            "quantize_pack": (2 * B * Hkv * N * D * 2 + caches[0].nbytes()) / (quant_us * 1e-6) / 1e9,
        },
        "fetched_fraction": fetched,
        "comparators": {
            "fp16_attention_us": fp16_us,
            "fp16_attention_GBs": fp16_bytes / (fp16_us * 1e-6) / 1e9,
            "fp16_attention_tokens_per_s": B / (fp16_us * 1e-6),
            "step_speedup_vs_fp16_attention": fp16_us / (ms_step * 1e3),
            "serial_fetch_step_us": serial_us,
            "step_speedup_vs_serial_fetch": serial_us / (ms_step * 1e3),
            "contiguous_h2d_us": h2d_us,
            "full_layer_h2d_us": full_layer_us,
            "full_layer_h2d_vs_step": full_layer_us / (ms_step * 1e3),
            "contiguous_h2d_GBs": n_gather / (h2d_us * 1e-6) / 1e9,
            "gather_full_fetch_vs_contiguous_h2d": float(np.median(runs["full"][2])) / h2d_us
            if "full" in runs else None,
            "what": "fp16: attention over the whole 16-bit cache in HBM (decode_attn_fp16); serial: rank "
                    "with the real token against C', fetch its top-k without overlap, attend; contiguous "
                    "h2d: one pinned-host-to-device copy of the bytes of every top-k row; full layer h2d: "
                    "the layer's whole 16-bit K and V copied from pinned host memory",
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host cores", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, K, V, Q, args.cpu_seconds)
    print(json.dumps(result), flush=True)

    # torch's pinned-memory allocator records an event on every stream a pinned block was
    # copied on when the block is freed (hk and hv were, by the full-layer copy): free them
    # while the library's streams still exist, then destroy the streams
    del hk, hv, hks, hvs
    torch.cuda.synchronize()
    torch.cuda.set_stream(torch.cuda.default_stream())
    if args.compute_stream == "exclusive":
        compute_stream.close()
    gather_stream.close()


if __name__ == "__main__":
    main()
