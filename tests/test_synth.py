"""The seeded input generator: determinism, bf16 exactness, target distributions."""
import numpy as np
import torch

import cce_synth as S


def test_bf16_round_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]   # exact ties go to even
    ref = torch.from_numpy(x.copy()).bfloat16().float().numpy()
    np.testing.assert_array_equal(S.bf16_round(x), ref)


def test_deterministic_and_prefix_stable():
    w = S.Workload("t", 5000, 16, 300, "bf16", 3.0, 1.1, ignore_frac=0.2, seed=7)
    a = S.make_inputs(w)
    b = S.make_inputs(w)
    for k in ("E", "C", "targets"):
        np.testing.assert_array_equal(a[k], b[k])
    c = S.make_inputs(w, N=4100)
    np.testing.assert_array_equal(c["E"], a["E"][:4100])   # rows come in fixed blocks
    assert np.array_equal(S.bf16_round(a["E"]), a["E"]) and np.array_equal(S.bf16_round(a["C"]), a["C"])


def test_zipf_and_ignore_fraction():
    w = S.Workload("t", 200000, 8, 1000, "f32", 1.0, 1.1, ignore_frac=0.2, seed=9)
    d = S.make_inputs(w)
    t = d["targets"]
    ign = t == S.IGNORE_INDEX
    assert abs(ign.mean() - 0.2) < 0.005
    p = (np.arange(1, 1001) ** -1.1)
    p /= p.sum()
    freq = np.bincount(t[~ign], minlength=1000) / (~ign).sum()
    assert abs(freq[0] - p[0]) < 0.005 and abs(freq[9] - p[9]) < 0.003
    assert t[~ign].min() >= 0 and t[~ign].max() < 1000


def test_boosted_rows_and_scale():
    w = S.Workload("t", 64, 256, 2000, "bf16", 8.0, 1.2, boost_frac=0.05, seed=3)
    d = S.make_inputs(w)
    rows = d["boosted_rows"]
    assert len(rows) == 100 and len(np.unique(rows)) == 100
    norms = np.linalg.norm(d["C"], axis=1)
    others = np.setdiff1d(np.arange(2000), rows)
    assert abs(norms[rows].mean() / norms[others].mean() - 2.0) < 0.05
    assert abs(norms[others].mean() - 8.0) < 0.3        # ||C_v|| ~ c_scale


def test_named_workloads_shapes():
    assert S.WORKLOADS["gemma2_2b_head"].N == 8192 and S.WORKLOADS["gemma2_2b_head"].V == 256000
    assert S.WORKLOADS["sparse_stress"].D == 3584
    assert S.WORKLOADS["long_seq"].ignore_frac == 0.2
    assert S.FILTER_EPS == 2.0 ** -12
