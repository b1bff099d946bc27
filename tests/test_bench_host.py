"""Host checks of bench.py's bookkeeping (no GPU): the HBM traffic record built from
rocprofv3 counter runs, the algorithmic byte count, and the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from workloads import get_config  # noqa: E402

SPLIT = "void specache::(anonymous namespace)::attn_split_kernel<128, 1, 1, 2, true, false>(specache::AttnArgs, int)"
STREAM = "void specache::(anonymous namespace)::attn_stream_kernel<1>(specache::AttnArgs, int, int, long, long, int)"
PLAIN = "void specache::(anonymous namespace)::attn_stream_kernel<0>(specache::AttnArgs, int, int, long, long, int)"
KEYS = "void specache::(anonymous namespace)::rank_keys_kernel<4>(float const*)"
SELECT = "void specache::(anonymous namespace)::rank_select_resident_kernel<128>(float const*)"


def _write(root, run, rows):
    d = os.path.join(root, run, "host", "123")
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Queue_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


@pytest.mark.parametrize("split", [SPLIT, STREAM])
def test_traffic_record_scales_counters_and_keeps_only_fused_step_dispatches(tmp_path, monkeypatch, split):
    root = str(tmp_path)
    # the plain 1 GiB copy reads as 512 MiB of FETCH_SIZE and 1 GiB of WRITE_SIZE (KiB units)
    _write(root, "pmc_copy_fetch", [[1, 1, "fill", "FETCH_SIZE", 0], [2, 1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288]])
    _write(root, "pmc_copy_write", [[1, 1, "fill", "WRITE_SIZE", 1048576],
                                    [2, 1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576]])
    for counter, run, vals in (("FETCH_SIZE", "pmc_fetch", (1000, 100, 10)), ("WRITE_SIZE", "pmc_write", (500, 50, 5))):
        rows, did = [], 1
        for _ in range(3):
            for name, v in ((split, vals[0]), (KEYS, vals[1]), (SELECT, vals[2])):
                rows.append([did, 2, name, counter, v])
                did += 1
            rows.append([did, 2, KEYS, counter, 10 ** 6])  # a score_topk's rank_keys: not part of the step
            did += 1
            rows.append([did, 2, PLAIN, counter, 10 ** 6])  # decode_attn's split: not part of the step
            did += 1
            rows.append([did, 2, SELECT, counter, 10 ** 6])  # nor a selection that follows no fused split
            did += 1
        _write(root, run, rows)
    out = tmp_path / "record.json"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(out))
    bench.write_traffic_record(root)
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    per = rec["per_kernel"]
    assert per["rank_keys_kernel"]["dispatches"] == 3
    want = 1024 * (2 * (1000 + 100 + 10) + (500 + 50 + 5))
    assert rec["traffic_bytes_per_launch"] == want
    assert rec["sources_sha256"] == bench.step_sources_hash()
    assert rec["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes_step(get_config("mistral32k"))


def test_algorithmic_bytes_of_the_32k_step():
    cfg = get_config("mistral32k")
    slices, N, k = 8 * 8, 32768, 328
    want = slices * (64 * N + 516 * k + 4 * k) + 2 * (8 * 32 * 2) * 128 * 2
    assert bench.algorithmic_bytes_step(cfg) == want == 145395712


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


@pytest.mark.parametrize("steps,warmup,sync", [(20, 5, 2), (50, 10, 2), (7, 0, 4), (1, 3, 2), (21, 5, 4), (5, 5, 1)])
def test_schedule_times_exactly_the_requested_steps(steps, warmup, sync):
    """Any --steps / --warmup pair is accepted (for example --steps 20 --warmup 5 with the
    default --sync-every 2): the timed pass holds exactly `steps` steps, the passes do not
    overlap, and every pass but a cut-short one starts on a whole synchronisation group."""
    w, t, i = bench.pipeline_schedule(warmup, steps, sync)
    assert len(w) == warmup and len(t) == steps and len(i) >= steps and len(i) % sync == 0
    assert t[0] % sync == 0 and i[0] % sync == 0
    assert all(b == a + 1 for a, b in zip(t, t[1:])) and all(b == a + 1 for a, b in zip(i, i[1:]))
    assert (not w or w[-1] < t[0]) and t[-1] < i[0]


def test_steps_20_warmup_5_are_accepted():
    args = bench.parse(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert (args.gpus, args.steps, args.warmup, args.sync_every) == (1, 20, 5, 2)
    w, t, i = bench.pipeline_schedule(args.warmup, args.steps, args.sync_every)
    assert len(t) == 20 and t[0] == 6
