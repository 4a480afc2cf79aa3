"""The seeded input generator (CPU only): the recipe of every workload holds
(shapes, seeds, weights, masked pairs, spiked residual rows), and the
expert-sorted row layout is the grouping of a grouped GEMM2 output."""
import math

import numpy as np
import pytest

import synth


def test_same_seed_same_inputs():
    a = synth.generate(12, 16, 8, seed=5, mask_frac=0.1, spike_frac=0.2)
    b = synth.generate(12, 16, 8, seed=5, mask_frac=0.1, spike_frac=0.2)
    c = synth.generate(12, 16, 8, seed=6, mask_frac=0.1, spike_frac=0.2)
    for k in ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma"):
        assert np.array_equal(a[k], b[k]), k
    assert not np.array_equal(a["expert_out"], c["expert_out"])


@pytest.mark.parametrize("cfg", sorted(synth.CONFIGS))
def test_config_recipe(cfg):
    c = synth.CONFIGS[cfg]
    T = min(c["Ts"])
    d = synth.config_inputs(cfg, T)
    H, K = c["H"], c["K"]
    assert (d["T"], d["H"], d["K"]) == (T, H, K) and d["R"] == T * K
    assert d["expert_out"].shape == (T * K, H) and d["expert_out"].dtype == np.uint16
    assert d["perm_idx"].shape == (T, K) and d["perm_idx"].dtype == np.int32
    assert d["topk_w"].shape == (T, K) and d["topk_w"].dtype == np.float32
    for k in ("shared_out", "residual"):
        assert d[k].shape == (T, H) and d[k].dtype == np.uint16
    assert d["gamma"].shape == (H,)
    assert d["scale"] == np.float32(c["scale"]) and d["eps"] == np.float32(synth.EPS)
    valid = d["perm_idx"] >= 0
    # every row is named at most once, and only rows of expert_out
    rows = d["perm_idx"][valid]
    assert len(np.unique(rows)) == rows.size and rows.max(initial=0) < T * K
    # weights: nonnegative, each token's valid weights sum to 1 (in fp64, from fp32)
    w = d["topk_w"].astype(np.float64)
    assert (w >= 0).all() and (w[~valid] == 0).all()
    sums = w.sum(axis=1)
    has = valid.any(axis=1)
    assert np.allclose(sums[has], 1.0, atol=1e-6)
    if c["mask_frac"] > 0:
        assert (~valid).sum() == math.ceil(c["mask_frac"] * T * K)
    else:
        assert valid.all()


def test_masked_pairs_at_every_size():
    for T, m in ((1, 1), (4, 2), (64, 26)):
        d = synth.config_inputs("decode_masked", T)
        assert (d["perm_idx"] < 0).sum() == m


def test_top8_of_256_weights_descend():
    d = synth.generate(40, 16, 8, weights="top8_of_256", seed=3)
    assert (np.diff(d["topk_w"].astype(np.float64), axis=1) <= 0).all()
    e = d["experts"]
    assert e.shape == (40, 8) and e.min() >= 0 and e.max() < 256
    assert all(len(set(row)) == 8 for row in e.tolist())


def test_spiked_residual_rows():
    d = synth.generate(200, 64, 2, seed=9, spike_frac=0.01)
    assert len(d["spike_rows"]) == 2
    r = synth.bf16_bits_to_f32(d["residual"]).astype(np.float64)
    rms = np.sqrt((r * r).mean(axis=1))
    spiked = np.zeros(200, dtype=bool)
    spiked[d["spike_rows"]] = True
    # N(0, 4^2) rows against N(0, 400^2) rows
    assert rms[spiked].min() > 100 and rms[~spiked].max() < 10


def test_expert_sorted_layout():
    T, K = 96, 8
    a = synth.generate(T, 16, K, weights="top8_of_256", seed=21)
    b = synth.generate(T, 16, K, weights="top8_of_256", seed=21, layout="expert_sorted")
    for k in ("expert_out", "topk_w", "shared_out", "residual", "gamma", "experts"):
        assert np.array_equal(a[k], b[k]), k
    perm = b["perm_idx"].reshape(-1)
    assert sorted(perm.tolist()) == list(range(T * K))
    pair_of_row = np.argsort(perm)  # the (token, slot) pair each row serves
    expert_of_row = b["experts"].reshape(-1)[pair_of_row]
    token_of_row = pair_of_row // K
    assert (np.diff(expert_of_row) >= 0).all(), "rows are grouped by expert"
    same = np.diff(expert_of_row) == 0
    assert (np.diff(token_of_row)[same] > 0).all(), "tokens in order within an expert"
    with pytest.raises(ValueError):
        synth.generate(4, 16, 8, layout="expert_sorted")  # softmax_k picks no experts
    with pytest.raises(ValueError):
        synth.generate(4, 16, 8, weights="top8_of_256", layout="sideways")
