"""Host-side checks of the seeded input generator (no GPU)."""
import json
import os

import numpy as np

from workloads import CONFIGS, get_config, generate_all, generate_slice

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_peaks_match_calibration_record():
    with open(os.path.join(GOLDEN, "planted_peak.json")) as f:
        rec = json.load(f)
    for name in ("llama8k", "mistral32k", "layers32"):
        assert CONFIGS[name].peak == rec[name]["peak"], name


def test_generator_is_deterministic_and_slice_local():
    cfg = get_config("tiny").with_(batch=2)
    K1, V1, Q1, _, _, _ = generate_all(cfg)
    K2, V2, Q2, _, _, _ = generate_all(cfg)
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2) and np.array_equal(Q1, Q2)
    Ks, _, Qs, _, _, _ = generate_all(cfg, slices=[(1, 1)])
    assert np.array_equal(Ks[1, 1], K1[1, 1]) and not Ks[0, 0].any()
    assert np.array_equal(Qs[1, 2:4], Q1[1, 2:4])
    K3, _, _, _, _, _ = generate_all(cfg, seed=1)
    assert not np.array_equal(K3, K1)


def test_shapes_and_planted_structure():
    cfg = get_config("llama8k").with_(seq_len=1024)
    s = generate_slice(cfg, 0, 3)
    assert s.k.shape == (1024, 128) and s.k.dtype == np.float16
    assert len(s.planted) == int(np.ceil(0.005 * 1024)) and np.all(np.diff(s.planted) > 0)
    assert abs(np.linalg.norm(s.direction) - 1) < 1e-5
    big = np.abs(s.k.astype(np.float32)).max(axis=0)
    assert (big > 15).sum() == cfg.n_outlier       # the x10 outlier channels stand out


def test_config_table():
    assert set(CONFIGS) == {"tiny", "llama8k", "mistral32k", "layers32", "long128k"}
    m = CONFIGS["mistral32k"]
    assert (m.batch, m.n_q_heads, m.n_kv_heads, m.seq_len, m.head_dim, m.bits, m.top_k) == \
        (8, 32, 8, 32768, 128, 1, 328)
    assert m.top_k == int(np.ceil(0.01 * m.seq_len))


def test_step_queries_are_fresh_draws_sharing_the_planted_direction():
    from workloads import generate_step_queries, generate_slice
    cfg = get_config("llama8k").with_(batch=1)
    qs = generate_step_queries(cfg, 3)
    assert qs.shape == (3, 1, cfg.n_q_heads, cfg.n_tokens, cfg.head_dim) and qs.dtype == np.float16
    assert not np.array_equal(qs[0], qs[1])
    assert np.array_equal(qs, generate_step_queries(cfg, 3))            # seeded
    u = generate_slice(cfg, 0, 0).direction
    proj = qs[:, 0, : cfg.gqa].astype(np.float64) @ u                    # heads of KV head 0
    assert np.all(np.abs(proj.mean() - cfg.peak) < 1.0)
