"""Seeded synthetic inputs: reproducibility and the stated distributions."""
import json
import os

import numpy as np
import pytest

from datagen import (CONFIGS, bf16_bits_to_f32, config_for, f32_to_bf16_bits,
                     make_inputs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    b = f32_to_bf16_bits(x)
    y = bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert y[0] == 1.0 and y[1] == 1.0
    assert y[2] == np.float32(1.0 + 2**-7)
    assert y[3] == -2.5
    assert np.all(bf16_bits_to_f32(f32_to_bf16_bits(y)) == y)


def test_reproducible_and_shapes():
    a = make_inputs(config_for(2, T=300), seed=0)
    b = make_inputs(config_for(2, T=300), seed=0)
    for k in ("hidden", "W", "teacher_idx", "teacher_logit", "mask"):
        assert a[k].tobytes() == b[k].tobytes(), k
    c = make_inputs(config_for(2, T=300), seed=1)
    assert a["hidden"].tobytes() != c["hidden"].tobytes()
    assert a["hidden"].shape == (300, 3072) and a["hidden"].dtype == np.uint16
    assert a["W"].shape == (128256, 3072) and a["W"].dtype == np.uint16
    assert a["teacher_idx"].shape == (300, 100) and a["teacher_idx"].dtype == np.int32
    assert a["teacher_logit"].dtype == np.float32 and a["mask"].dtype == np.uint8


def test_config1_distributions():
    x = make_inputs(1, seed=0)
    cfg = CONFIGS[1]
    assert x["hidden"].dtype == np.float32 and x["W"].dtype == np.float32
    assert abs(x["W"].std() - 1 / 16) < 2e-3
    assert abs(x["hidden"].std() - 1) < 1e-2
    idx = x["teacher_idx"]
    assert idx.min() >= 0 and idx.max() < cfg.V
    assert all(len(set(r)) == cfg.K for r in idx.tolist())
    lg = x["teacher_logit"]
    assert np.all(np.diff(lg, axis=1) <= 0)
    assert abs(lg.std() - 2) < 0.1
    zeros = int((x["mask"] == 0).sum())
    # Binomial(512, 0.05): mean 25.6, sd 4.9
    assert 5 <= zeros <= 50


def test_bf16_config_distributions_and_overlap_rows():
    cfg = config_for(4, T=512, V=6000, d=256)
    x = make_inputs(cfg, seed=0)
    h = bf16_bits_to_f32(x["hidden"]).astype(np.float64)
    np.testing.assert_allclose(np.sqrt((h ** 2).mean(axis=1)), 1.0, atol=1e-2)
    w = bf16_bits_to_f32(x["W"])
    assert abs(w.std() - 0.02) < 1e-3
    # overlap rows: ids are the student's own top-K, in descending z order
    z = h @ w.astype(np.float64).T
    top = np.argsort(-z, axis=1)[:, :cfg.K]
    same = np.array([set(top[t]) == set(x["teacher_idx"][t]) for t in range(cfg.T)])
    # Bernoulli(0.3) over 512 rows: mean 154, sd 10.4
    assert 100 <= same.sum() <= 210
    # peaked rows (config 4): top logit +8 above an N(0,3) sorted draw
    gap = x["teacher_logit"][:, 0] - x["teacher_logit"][:, 1]
    assert (gap > 8).sum() >= 20


def test_pages_figures_closed_forms():
    g = json.load(open(GOLDEN))
    # the bf16 teacher-probability tensor 4 x 201,088 x 32,768 is "about 50GB"
    nbytes = g["batch"]["value"] * g["vocab_gpt_oss"]["value"] * g["seq_len_32k"]["value"] * 2
    assert abs(nbytes / 1e9 - g["teacher_tensor_bf16_gb_approx"]["value"]) < 3
    assert abs(g["isolated_dense_32k_gib"]["value"] / g["isolated_fused_32k_gib"]["value"]
               - g["isolated_reduction_x"]["value"]) < 0.05
    # the large workloads use the pages' vocabulary and cache width
    assert CONFIGS[3].V == g["vocab_gpt_oss"]["value"] == CONFIGS[5].V
    assert CONFIGS[3].K == g["teacher_top_k"]["value"]
    assert CONFIGS[3].T == g["seq_len_32k"]["value"]
