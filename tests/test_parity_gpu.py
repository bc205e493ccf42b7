"""GPU parity: libcce (HIP, gfx950) against the float64 CPU oracle, element by element, on
seeded inputs that span several 256 x 256 tiles with ragged tails, several backward vocabulary
chunks, and the degenerate cases of the method."""
import math

import numpy as np
import pytest
import torch

import cce_synth as S
import linear_cross_entropy_cce_amd as cce
import oracle
from gpu_helpers import (DEV, EPS, GRAD_TOL, II, LOSS_TOL, ROW_TOL, check_against_oracle,
                         gpu_run, log, rel, row_err, upload)

pytestmark = pytest.mark.gpu


def test_tiny_workload_fp32():
    w = S.WORKLOADS["tiny"]
    d = S.make_inputs(w)
    g = check_against_oracle(d, "f32", S.dloss_weights(1, w.N), 0.0, "tiny")
    ref, _ = oracle.forward(d["E"], d["C"], d["targets"], II)
    assert np.abs(g["loss"] - ref).max() < 1e-4    # fp32 MFMA: far inside the tolerance


SMALL = [
    # name, N, D, V, dtype, c_scale, zipf, ignore_frac, seed
    ("bf16_ragged", 300, 136, 1100, "bf16", 3.0, 1.1, 0.1, 11),
    ("bf16_tiles", 512, 256, 2048, "bf16", 3.0, 1.1, 0.0, 12),
    ("f32_ragged", 130, 36, 777, "f32", 2.0, None, 0.1, 13),
    ("bf16_k_tail", 257, 72, 300, "bf16", 2.0, 1.0, 0.2, 14),
    ("bf16_one_token", 1, 64, 300, "bf16", 3.0, None, 0.0, 15),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("eps", [0.0, EPS])
def test_small_cases(case, eps):
    name, N, D, V, dt, cs, z, ig, seed = case
    d = S.small_case(N, D, V, dt, seed, cs, z, ig)
    check_against_oracle(d, dt, S.dloss_weights(seed, N), eps, name)


def test_several_vocabulary_chunks():
    """V = 20000 (79 vocabulary tiles) spans three balanced backward chunks of 26, 26 and 27
    tiles (6656, 6656 and a ragged 6688 rows)."""
    d = S.small_case(300, 72, 20000, "bf16", 21, 3.0, 1.1, 0.05)
    assert cce.backward_chunk(300, 20000, 72, torch.bfloat16) == 27 * 256
    check_against_oracle(d, "bf16", S.dloss_weights(21, 300), EPS, "chunks")


def test_sparse_softmax_skips_blocks():
    w = S.Workload("sparse_small", 320, 128, 3000, "bf16", 12.0, 1.2, boost_frac=0.05, seed=3)
    d = S.make_inputs(w)
    g = check_against_oracle(d, "bf16", S.dloss_weights(3, 320), EPS, "sparse_small")
    assert g["skipped"] > 0


def test_far_vocabulary_blocks_are_skipped_exactly():
    """Vocabulary blocks 1 and 3 (64 wide) get logits near -200 for every token: each of
    their (token block, vocabulary block) pairs must be skipped and nothing else."""
    N, V, D = 150, 320, 64
    g = np.random.default_rng(31)
    E = S.bf16_round(np.concatenate([np.full((N, 1), 10.0), 0.1 * g.standard_normal((N, D - 1))],
                                    axis=1).astype(np.float32))
    C = 0.05 * g.standard_normal((V, D)).astype(np.float32)
    far = np.r_[64:128, 192:256]
    C[far, 0] = -20.0
    C = S.bf16_round(C)
    t = g.choice(np.setdiff1d(np.arange(V), far), size=N).astype(np.int64)
    d = {"E": E, "C": C, "targets": t}
    out = check_against_oracle(d, "bf16", np.ones(N, np.float32), EPS, "far_blocks")
    assert (out["skipped"], out["total"]) == (3 * 2, 3 * 5)


def test_zero_embeddings_give_log_v():
    N, V, D = 70, 1000, 64
    d = S.small_case(N, D, V, "bf16", 41, 3.0, 1.1, 0.0)
    d["E"][:] = 0.0
    out = gpu_run(d, "bf16", np.ones(N, np.float32), 0.0)
    assert np.abs(out["loss"] - math.log(V)).max() < 1e-5
    assert np.abs(out["dC"]).max() == 0.0
    check_against_oracle(d, "bf16", np.ones(N, np.float32), 0.0, "zero_E")


@pytest.mark.parametrize("V", [1, 2])
def test_tiny_vocabularies(V):
    d = S.small_case(70, 16, V, "bf16", 42 + V, 3.0, None, 0.1)
    g = check_against_oracle(d, "bf16", S.dloss_weights(7, 70), 0.0, f"V{V}")
    if V == 1:
        assert np.abs(g["loss"]).max() < 1e-6


def test_all_tokens_ignored():
    d = S.small_case(100, 64, 500, "bf16", 51, 3.0, 1.1, 0.0)
    d["targets"][:] = II
    out = gpu_run(d, "bf16", np.ones(100, np.float32), EPS)
    assert np.all(out["loss"] == 0.0) and np.all(out["dE"] == 0.0) and np.all(out["dC"] == 0.0)
    _, lse = oracle.forward(d["E"], d["C"], d["targets"], II)
    assert np.abs(out["lse"] - lse).max() < LOSS_TOL
    assert out["skipped"] == out["total"]   # no valid row makes any block significant


def test_dominant_logit_stays_finite():
    N, V, D = 64, 512, 64
    E = np.zeros((N, D), np.float32)
    E[np.arange(N), np.arange(N) % D] = 32.0
    C = np.zeros((V, D), np.float32)
    t = (np.arange(N) * 7 % V).astype(np.int64)
    C[t, np.arange(N) % D] = 32.0       # target logit 1024 (bf16 exact), the rest 0 or 1024
    d = {"E": E, "C": C, "targets": t}
    out = gpu_run(d, "bf16", np.ones(N, np.float32), EPS)
    assert np.all(np.isfinite(out["loss"])) and np.all(np.isfinite(out["dE"]))
    check_against_oracle(d, "bf16", np.ones(N, np.float32), EPS, "dominant")


def test_invalid_target_sets_flag_and_nan():
    d = S.small_case(40, 64, 100, "bf16", 61, 3.0, None, 0.0)
    d["targets"][5] = 100
    out = gpu_run(d, "bf16", np.ones(40, np.float32), 0.0)
    assert out["err"] == 1 and np.isnan(out["loss"][5])
    assert np.all(np.isfinite(np.delete(out["loss"], 5)))


def test_empty_batch():
    E = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    C = torch.randn((300, 64), device=DEV).to(torch.bfloat16)
    t = torch.zeros(0, dtype=torch.int64, device=DEV)
    loss, lse = cce.cce_forward(E, C, t)
    dC = torch.full((300, 64), 7.0, device=DEV)
    stats = torch.full((2,), -1, dtype=torch.int64, device=DEV)
    dE, dC = cce.cce_backward(torch.ones(0, device=DEV), E, C, t, lse, dC=dC, skip_stats=stats)
    torch.cuda.synchronize()
    assert loss.numel() == 0 and dE.numel() == 0
    assert float(dC.abs().max()) == 0.0 and stats.tolist() == [0, 0]


def test_scalar_dloss_equals_vector():
    d = S.small_case(200, 64, 900, "bf16", 71, 3.0, 1.1, 0.1)
    E, C, t = upload(d, "bf16")
    _, lse = cce.cce_forward(E, C, t)
    a = cce.cce_backward(torch.full((1,), 0.37, device=DEV), E, C, t, lse, filter_eps=EPS)
    b = cce.cce_backward(torch.full((200,), 0.37, device=DEV), E, C, t, lse, filter_eps=EPS)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_runs_are_bitwise_deterministic():
    d = S.small_case(520, 128, 9000, "bf16", 81, 3.0, 1.1, 0.1)
    w = S.dloss_weights(81, 520)
    a = gpu_run(d, "bf16", w, EPS)
    b = gpu_run(d, "bf16", w, EPS)
    for k in ("loss", "lse", "dE", "dC"):
        assert np.array_equal(a[k], b[k]), k


def test_loss_mean_matches_oracle():
    d = S.small_case(333, 72, 1500, "bf16", 91, 3.0, 1.1, 0.25)
    E, C, t = upload(d, "bf16")
    mean, nv, dE, dC = cce.cce_loss_mean(E, C, t, II, EPS)
    torch.cuda.synchronize()
    m, rE, rC, n = oracle.loss_mean(d["E"], d["C"], d["targets"], II, EPS)
    assert int(nv.item()) == n
    assert abs(float(mean.item()) - m) <= LOSS_TOL
    assert rel(dE.cpu().numpy(), rE) <= GRAD_TOL and rel(dC.cpu().numpy(), rC) <= GRAD_TOL


@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_loss_mean_over_several_token_blocks(gdt):
    """The mean call at N = 20000 (two backward token blocks, so dC adds up over the blocks in
    the mean call's own workspace), with gradients in fp32 or bf16."""
    d = S.small_case(20000, 64, 1280, "bf16", 93, 3.0, 1.1, 0.2)
    E, C, t = upload(d, "bf16")
    assert cce.backward_token_block(20000, 1280, 64, torch.bfloat16) < 20000
    mean, nv, dE, dC = cce.cce_loss_mean(E, C, t, II, EPS, grad_dtype=gdt)
    torch.cuda.synchronize()
    assert dE.dtype == gdt and dC.dtype == gdt
    m, rE, rC, n = oracle.loss_mean(d["E"], d["C"], d["targets"], II, EPS)
    _, uE, uC, _ = oracle.loss_mean(d["E"], d["C"], d["targets"], II, 0.0)
    gE, gC = dE.float().cpu().numpy(), dC.float().cpu().numpy()
    log(f"[loss mean N=20000 {gdt}] mean {abs(float(mean.item()) - m):.2e} "
        f"dE {rel(gE, rE):.2e} dC {rel(gC, rC):.2e}")
    assert int(nv.item()) == n
    assert abs(float(mean.item()) - m) <= LOSS_TOL
    assert rel(gE, rE) <= GRAD_TOL and rel(gC, rC) <= GRAD_TOL
    assert rel(gE, uE) <= GRAD_TOL and rel(gC, uC) <= GRAD_TOL
    assert row_err(gC, rC) <= ROW_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_filter_closed_form_flat_softmax(dtype):
    """A flat softmax over V = 20000 > 1/eps rows at the benchmarks' eps = 2^-12: with every
    classifier row equal, every p is 1/V < eps, so only the blocks holding a target are kept
    and the filtered gradients have a closed form (the CPU pin of the same name), far from the
    unfiltered dE = 0 -- the regime where the block filter's approximation is not small.  The
    GPU follows the closed form and the oracle, with the oracle's skip count."""
    from test_oracle import block_filter_equal_rows_closed_form
    rng = np.random.default_rng(34)
    N, V, D = 300, 20000, 64
    E = rng.standard_normal((N, D)).astype(np.float32)
    c = rng.standard_normal(D).astype(np.float32)
    if dtype == "bf16":
        E, c = S.bf16_round(E), S.bf16_round(c)
    C = np.tile(c, (V, 1))
    t = rng.integers(0, V, N).astype(np.int64)
    t[[3, 100]] = II
    d = {"E": E, "C": C, "targets": t}
    w = S.dloss_weights(34, N)
    g = gpu_run(d, dtype, w, EPS)
    eE, eC, esk = block_filter_equal_rows_closed_form(E.astype(np.float64), c.astype(np.float64),
                                                      t, w.astype(np.float64), V)
    dE, dC, (sk, tot) = oracle.backward(E, C, t, w, II, filter_eps=EPS)
    assert sk == esk and g["skipped"] == sk and g["total"] == tot
    log(f"[flat softmax {dtype}] skipped {sk}/{tot}; dE vs closed form {rel(g['dE'], eE):.2e} "
        f"dC {rel(g['dC'], eC):.2e}; oracle vs closed form dE {rel(dE, eE):.2e}")
    assert rel(dE, eE) <= 1e-9 and rel(dC, eC) <= 1e-9
    assert rel(g["dE"], eE) <= GRAD_TOL and rel(g["dC"], eC) <= GRAD_TOL
    assert row_err(g["dE"], eE) <= ROW_TOL and row_err(g["dC"], eC) <= ROW_TOL


def test_loss_mean_all_ignored_is_zero():
    d = S.small_case(64, 64, 300, "bf16", 92, 3.0, 1.1, 0.0)
    d["targets"][:] = II
    E, C, t = upload(d, "bf16")
    mean, nv, dE, dC = cce.cce_loss_mean(E, C, t, II, 0.0)
    torch.cuda.synchronize()
    assert float(mean.item()) == 0.0 and int(nv.item()) == 0
    assert float(dE.abs().max()) == 0.0 and float(dC.abs().max()) == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bf16_gradients_are_the_rounded_fp32_gradients(dtype):
    """grad_dtype = bf16: both gradients are the fp32 results rounded to nearest even, bit for
    bit (same kernels and order; dE rounded once after the last chunk)."""
    d = S.small_case(300, 72, 20000, dtype, 111, 3.0, 1.1, 0.1)
    log(f"[bf16 grads] {dtype}")
    E, C, t = upload(d, dtype)
    loss, lse = cce.cce_forward(E, C, t, II)
    dl = torch.from_numpy(S.dloss_weights(111, 300)).to(DEV)
    e32, c32 = cce.cce_backward(dl, E, C, t, lse, II, EPS)
    e16, c16 = cce.cce_backward(dl, E, C, t, lse, II, EPS, grad_dtype=torch.bfloat16)
    mean, nv, me16, mc16 = cce.cce_loss_mean(E, C, t, II, EPS, grad_dtype=torch.bfloat16)
    _, _, me32, mc32 = cce.cce_loss_mean(E, C, t, II, EPS)
    torch.cuda.synchronize()
    assert e16.dtype == torch.bfloat16 and c16.dtype == torch.bfloat16
    assert torch.equal(e16, e32.to(torch.bfloat16)) and torch.equal(c16, c32.to(torch.bfloat16))
    assert torch.equal(me16, me32.to(torch.bfloat16)) and torch.equal(mc16, mc32.to(torch.bfloat16))
    rE, rC, _ = oracle.backward(d["E"], d["C"], d["targets"], S.dloss_weights(111, 300), II,
                                filter_eps=EPS)
    assert rel(e16.float().cpu().numpy(), rE) <= GRAD_TOL
    assert rel(c16.float().cpu().numpy(), rC) <= GRAD_TOL


def test_empty_batch_bf16_gradients():
    E = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    C = torch.randn((300, 64), device=DEV).to(torch.bfloat16)
    t = torch.zeros(0, dtype=torch.int64, device=DEV)
    loss, lse = cce.cce_forward(E, C, t)
    dC = torch.full((300, 64), 7.0, device=DEV, dtype=torch.bfloat16)
    dE, dC = cce.cce_backward(torch.ones(0, device=DEV), E, C, t, lse, dC=dC,
                              grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert dE.numel() == 0 and float(dC.float().abs().max()) == 0.0


def _random_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = "bf16" if rng.random() < 0.7 else "f32"
        step = 8 if dt == "bf16" else 4
        N = int(rng.integers(1, 700))
        D = int(rng.integers(1, 41)) * step
        V = int(rng.integers(1, 5000))
        cs = float(rng.choice([1.0, 3.0, 8.0]))
        z = None if rng.random() < 0.3 else float(rng.choice([1.0, 1.1, 1.3]))
        ig = float(rng.choice([0.0, 0.1, 0.5]))
        eps = float(rng.choice([0.0, EPS, 1e-3]))
        cases.append((f"r{i}_{dt}_{N}x{D}x{V}", N, D, V, dt, cs, z, ig, eps, 500 + i))
    return cases


def _wide_random_cases(n, seed=2025):
    """Wider seeded shapes: up to 9000 tokens and 20000 vocabulary rows (several backward
    chunks), D up to 504, logit scales up to 14 (sparse softmax)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = "bf16" if rng.random() < 0.7 else "f32"
        step = 8 if dt == "bf16" else 4
        N = int(rng.choice([rng.integers(1, 300), rng.integers(300, 3000),
                            rng.integers(3000, 9000)]))
        D = int(rng.integers(1, 64)) * step
        V = int(rng.choice([rng.integers(1, 600), rng.integers(600, 9000),
                            rng.integers(9000, 20000)]))
        cs = float(rng.choice([1.0, 3.0, 8.0, 14.0]))
        z = None if rng.random() < 0.3 else float(rng.choice([1.0, 1.1, 1.3]))
        ig = float(rng.choice([0.0, 0.1, 0.5]))
        eps = float(rng.choice([0.0, EPS, 1e-3]))
        cases.append((f"w{i}_{dt}_{N}x{D}x{V}", N, D, V, dt, cs, z, ig, eps, 700 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases(12) + _wide_random_cases(12), ids=lambda c: c[0])
def test_random_shapes(case):
    """Seeded random shapes (ragged N, D and V, both dtypes, ignored rows, three thresholds)
    against the oracle with the same threshold, element by element, and, when filtered,
    against the unfiltered oracle."""
    name, N, D, V, dt, cs, z, ig, eps, seed = case
    d = S.small_case(N, D, V, dt, seed, cs, z, ig)
    check_against_oracle(d, dt, S.dloss_weights(seed, N), eps, name)


def _half_live_case(N, V, D, dtype, seed):
    """Inputs whose live 64 x 64 blocks follow a fixed pattern: token block b is "flat" (small
    logits, every softmax entry near 1/V, live everywhere) when b % 8 == 0, else it leans on
    vocabulary rows of its parity class g = (b // 2) % 2, where row v has class (v // 128) % 2:
    blocks of the same class are live, the others are negligible.  Within a 256-row tile of
    either product, many K stages have live blocks in only one 128-row half of the tile and
    others in both; targets lie in the token's own class (or anywhere for flat tokens)."""
    g = np.random.default_rng(seed)
    tb = np.arange(N) // 64
    flat = tb % 8 == 0
    cls_n = (tb // 2) % 2
    cls_v = (np.arange(V) // 128) % 2
    E = 0.3 * g.standard_normal((N, D))
    E[np.arange(N), cls_n] += np.where(flat, 0.0, 6.0)
    E[flat] *= 0.1
    C = 0.3 * g.standard_normal((V, D))
    C[np.arange(V), cls_v] += 3.0
    t = np.empty(N, np.int64)
    for c in (0, 1):
        rows = np.flatnonzero((cls_n == c) & ~flat)
        t[rows] = g.choice(np.flatnonzero(cls_v == c), size=rows.size)
    t[flat] = g.integers(0, V, size=int(flat.sum()))
    t[g.random(N) < 0.05] = II
    rnd = S.bf16_round if dtype == "bf16" else (lambda x: x)
    return {"E": rnd(E.astype(np.float32)), "C": rnd(C.astype(np.float32)), "targets": t}


@pytest.mark.parametrize("dtype,N", [("bf16", 40000), ("f32", 20000)])
def test_stages_with_one_live_half(dtype, N):
    """Backward stages whose live blocks sit in one 128-row half of a tile (only that half's
    waves multiply), mixed with stages live in both halves, and token counts whose stage lists
    take several 512-entry steps to build: element-wise parity with the oracle, and exactly the
    oracle's skipped blocks (no block is near the threshold)."""
    V, D = 1000, 64
    d = _half_live_case(N, V, D, dtype, 71)
    g = check_against_oracle(d, dtype, S.dloss_weights(71, N), EPS, f"half_live_{dtype}")
    _, _, (sk, tot) = oracle.backward(d["E"], d["C"], d["targets"],
                                      S.dloss_weights(71, N), II, filter_eps=EPS)
    assert g["skipped"] == sk and 0.3 * tot < sk < 0.6 * tot, (g["skipped"], sk, tot)


def test_vocabulary_relabelled_by_row_norm():
    """The caller-side relabelling that bench.py --vocab-order times: classifier rows sorted by
    decreasing norm and the targets mapped, which gathers the rows carrying the softmax into few
    blocks.  Loss, LSE and dE are those of the problem as given (oracle), dC is its rows in the
    new order, and more blocks are skipped than for the problem as given."""
    w = S.Workload("sparse_small", 320, 128, 3000, "bf16", 12.0, 1.2, boost_frac=0.05, seed=3)
    d = S.make_inputs(w)
    C, t = d["C"], d["targets"]
    perm = np.argsort(-np.linalg.norm(C.astype(np.float64), axis=1), kind="stable")
    rank = np.empty_like(perm)
    rank[perm] = np.arange(len(perm))
    relabelled = {"E": d["E"], "C": C[perm], "targets": np.where(t == II, t, rank[np.maximum(t, 0)])}
    wts = S.dloss_weights(3, 320)
    g0 = gpu_run(d, "bf16", wts, EPS)
    g1 = gpu_run(relabelled, "bf16", wts, EPS)
    loss, lse = oracle.forward(d["E"], C, t, II)
    dE, dC, _ = oracle.backward(d["E"], C, t, wts, II)          # unfiltered
    assert np.abs(g1["loss"] - loss).max() <= LOSS_TOL
    assert np.abs(g1["lse"] - lse).max() <= LOSS_TOL
    assert rel(g1["dE"], dE) <= GRAD_TOL, rel(g1["dE"], dE)
    assert rel(g1["dC"], dC[perm]) <= GRAD_TOL, rel(g1["dC"], dC[perm])
    log(f"[relabelled] skipped {g1['skipped']}/{g1['total']} (as given {g0['skipped']})")
    assert g1["skipped"] > g0["skipped"]


@pytest.mark.parametrize("dtype,N", [("bf16", 270000), ("f32", 140000)])
def test_many_token_blocks(dtype, N):
    """Token counts far past one backward token block (270 000 bf16 tokens: 17 blocks of at
    most 16384; 140 000 fp32 tokens: 18 blocks of at most 8192): each chunk's dC adds up over
    the blocks, here with stages live in one half, both or neither, against the oracle with
    exactly its skipped blocks."""
    V, D = 1000, 64
    d = _half_live_case(N, V, D, dtype, 73)
    w = S.dloss_weights(73, N)
    g = check_against_oracle(d, dtype, w, EPS, f"pieces_{dtype}")
    _, _, (sk, tot) = oracle.backward(d["E"], d["C"], d["targets"], w, II, filter_eps=EPS)
    assert g["skipped"] == sk, (g["skipped"], sk, tot)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_last_vocabulary_chunk_narrower_than_a_block(dtype):
    """V = 8192 + 40 (33 vocabulary tiles, two balanced chunks of 16 and 17): the last tile of
    the last chunk holds 40 rows, less than one 64-row filter block (its G tile, flags, dE
    stages and dC tile are ragged), and many targets lie in it."""
    D = 72 if dtype == "bf16" else 68
    d = S.small_case(300, D, 8192 + 40, dtype, 29, 3.0, 1.1, 0.05)
    t = d["targets"].copy()
    t[::7] = 8192 + np.arange(len(t[::7])) % 40          # targets inside the narrow chunk
    d["targets"] = t
    check_against_oracle(d, dtype, S.dloss_weights(29, 300), EPS, f"narrow_chunk_{dtype}")


def test_ignore_index_inside_the_vocabulary():
    """ignore_index may be a real token id (here 3, frequent under Zipf targets): every row
    whose target equals it is ignored (loss 0, zero dE row, no part in dC or the filter), and
    the other rows are scored as usual (the inputs hold no -100 targets)."""
    ii = 3
    d = S.small_case(400, 64, 1500, "bf16", 41, 3.0, 1.1, 0.0)
    t = d["targets"]
    assert (t == ii).sum() > 10
    w = S.dloss_weights(41, 400)
    E, C, tt = upload(d, "bf16")
    loss, lse = cce.cce_forward(E, C, tt, ii)
    dl = torch.from_numpy(w).to(DEV)
    dE, dC = cce.cce_backward(dl, E, C, tt, lse, ii, EPS)
    torch.cuda.synchronize()
    rl, rlse = oracle.forward(d["E"], d["C"], t, ii)
    rE, rC, _ = oracle.backward(d["E"], d["C"], t, w, ii)
    g_loss, g_dE = loss.cpu().numpy(), dE.cpu().numpy()
    assert np.abs(g_loss - rl).max() <= LOSS_TOL
    assert np.abs(lse.cpu().numpy() - rlse).max() <= LOSS_TOL
    assert np.all(g_loss[t == ii] == 0.0) and np.all(g_dE[t == ii] == 0.0)
    assert rel(g_dE, rE) <= GRAD_TOL and rel(dC.cpu().numpy(), rC) <= GRAD_TOL


def test_entry_floor_matches_the_oracle_rule():
    """In fp32 (G kept in fp32) with eps = 0.1 and the optional entry floor at eps / 256, the
    entries below the floor carry enough of G (4e-3 of dE) that the GPU must match the oracle's
    rule closely and differ clearly from the same oracle without the floor.  No block maximum
    lies within 1e-3 of eps, so both sides skip the same 3 of 90 blocks.  Without the argument
    the floor is off."""
    d = S.small_case(300, 64, 1100, "f32", 41, 3.0, 1.1, 0.1)
    w = S.dloss_weights(41, 300)
    eps, floor = 0.1, 0.1 / 256
    g = gpu_run(d, "f32", w, eps, entry_floor=floor)
    g0 = gpu_run(d, "f32", w, eps)
    E, C, t = d["E"], d["C"], d["targets"]
    dE1, dC1, _ = oracle.backward(E, C, t, w, II, filter_eps=eps, entry_floor=floor)
    dE0, dC0, _ = oracle.backward(E, C, t, w, II, filter_eps=eps)
    eE, eC = rel(g["dE"], dE1), rel(g["dC"], dC1)
    fE, fC = rel(dE1, dE0), rel(dC1, dC0)
    log(f"[entry floor] gpu vs oracle dE {eE:.2e} dC {eC:.2e}; floor effect dE {fE:.2e} dC {fC:.2e}")
    assert g["skipped"] == 3 and g0["skipped"] == 3
    assert eE < 1e-4 and eC < 1e-4
    assert fE > 20 * eE and fC > 20 * eC
    assert rel(g0["dE"], dE0) < 1e-4 and rel(g0["dC"], dC0) < 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_entry_floor_closed_form_equal_rows(dtype):
    """Every classifier row equal to c: every softmax entry is 1/V.  With the entry floor just
    above 1/V only the target entries survive, so dE_n = dloss_n (1/V - 1) c and
    dC_v = (1/V - 1) sum over tokens with target v of dloss_n E_n; with the floor just below
    1/V nothing is dropped and dE = 0 (rows of G sum to zero; bf16 rounding of G leaves at most
    2^-7 dloss_n |c|)."""
    N, V, D = 300, 1000, 64
    rng = np.random.default_rng(53)
    E = S.bf16_round(rng.standard_normal((N, D)).astype(np.float32))
    c = S.bf16_round(rng.standard_normal(D).astype(np.float32))
    C = np.tile(c, (V, 1))
    t = rng.integers(0, V, N)
    t[::13] = II
    w = S.dloss_weights(53, N)
    valid = t != II
    wv = np.where(valid, w, 0.0).astype(np.float64)
    onehot = np.zeros((N, V))
    onehot[np.nonzero(valid)[0], t[valid]] = 1.0
    d = {"E": E, "C": C, "targets": t}
    g = gpu_run(d, dtype, w, 0.0, entry_floor=1.01 / V)
    ref_dE = (wv * (1.0 / V - 1.0))[:, None] * c[None, :].astype(np.float64)
    ref_dC = (1.0 / V - 1.0) * (onehot * wv[:, None]).T @ E.astype(np.float64)
    eE, eC = rel(g["dE"], ref_dE), rel(g["dC"], ref_dC)
    g0 = gpu_run(d, dtype, w, 0.0, entry_floor=0.99 / V)
    resid = np.linalg.norm(g0["dE"], axis=1) / (wv * np.linalg.norm(c) + 1e-30)
    ref0_dC = ((1.0 / V) * valid[:, None] - onehot).T @ (wv[:, None] * E.astype(np.float64))
    e0C = rel(g0["dC"], ref0_dC)
    log(f"[entry floor closed form {dtype}] above 1/V: dE {eE:.2e} dC {eC:.2e}; below: "
        f"max |dE_n| / (dloss_n |c|) {resid[valid].max():.2e}, dC {e0C:.2e}")
    assert eE <= 1e-2 and eC <= 1e-2 and e0C <= 1e-2
    assert resid[valid].max() <= 2.0 ** -7


def test_bf16_gradients_over_several_token_blocks():
    """bf16 gradients when the tokens span two backward token blocks (20 000 bf16 tokens: 79
    tiles in blocks of 40 and 39) and the vocabulary two chunks: each chunk's dC adds up in
    the fp32 chunk accumulator and the last block rounds it, so both gradients are exactly the
    fp32 ones rounded to nearest even."""
    N, V, D = 20000, 9000, 64
    assert cce.backward_token_block(N, V, D, torch.bfloat16) == 40 * 256
    d = S.small_case(N, D, V, "bf16", 57, 3.0, 1.1, 0.1)
    E, C, t = upload(d, "bf16")
    loss, lse = cce.cce_forward(E, C, t, II)
    dl = torch.from_numpy(S.dloss_weights(57, N)).to(DEV)
    e32, c32 = cce.cce_backward(dl, E, C, t, lse, II, EPS)
    e16, c16 = cce.cce_backward(dl, E, C, t, lse, II, EPS, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(e16, e32.to(torch.bfloat16)) and torch.equal(c16, c32.to(torch.bfloat16))
    check_against_oracle(d, "bf16", S.dloss_weights(57, N), EPS, "two_token_blocks")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_largest_feature_dimension(dtype):
    """D = 65536, the largest the kernels take: row strides of 128 / 256 KB, 1024 K stages per
    tile, 256 dE and dC tiles along D."""
    d = S.small_case(130, 65536, 300, dtype, 43, 3.0, 1.1, 0.1)
    check_against_oracle(d, dtype, S.dloss_weights(43, 130), EPS, f"d65536_{dtype}")


def test_largest_vocabulary():
    """V = 2^24, the largest the kernels take (D = 8): 65 536 vocabulary tiles, 2048 backward
    chunks, 262 144 filter blocks.  Unfiltered, so one oracle backward suffices (~40 s)."""
    d = S.small_case(64, 8, 1 << 24, "bf16", 44, 3.0, 1.1, 0.1)
    g = check_against_oracle(d, "bf16", S.dloss_weights(44, 64), 0.0, "v2^24")
    assert g["total"] == 1 * (1 << 18) and g["skipped"] == 0


def _tile_max_oracle(E, C):
    """The largest logit x log2(e) of each 128-row x 64-token part (wave w: rows 128 (w >> 2),
    tokens 64 (w & 3)) of every 256 x 256 tile, from the oracle's logits; -inf when empty."""
    N, V = E.shape[0], C.shape[0]
    z = oracle.logits(E, C) / math.log(2.0)
    n_tb, n_vt = -(-N // 256), -(-V // 256)
    out = np.full((n_tb, n_vt, 8), -np.inf)
    for tb in range(n_tb):
        for vt in range(n_vt):
            for w in range(8):
                c0, r0 = 256 * tb + 64 * (w & 3), 256 * vt + 128 * (w >> 2)
                blk = z[c0:min(N, c0 + 64), r0:min(V, r0 + 128)]
                if blk.size:
                    out[tb, vt, w] = blk.max()
    return out.reshape(-1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tile_maxima_match_the_logits(dtype):
    """cce_forward's tile maxima against the oracle's logits (ragged N and V)."""
    d = S.small_case(300, 136, 1100, dtype, 51, 3.0, 1.1, 0.1)
    E, C, t = upload(d, dtype)
    tm = cce.tile_max_buffer(E, C)
    assert tm.numel() == 2 * 5 * 8
    loss, lse = cce.cce_forward(E, C, t, II, tile_max=tm)
    loss0, lse0 = cce.cce_forward(E, C, t, II)
    assert torch.equal(lse, lse0) and torch.equal(loss, loss0)   # the output changes nothing else
    ref = _tile_max_oracle(d["E"], d["C"])
    g = tm.cpu().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin)
    np.testing.assert_allclose(g[fin], ref[fin], rtol=1e-5, atol=1e-4)


def _far_tiles_case(dtype, seed, V=1280, far_tiles=(1, 3), N=600):
    """N tokens; the given vocabulary tiles (256 rows each) get logits near -200 for every
    token, so their G tiles can be skipped, except the one (the second far tile, token tile 0)
    that holds token 5's target."""
    D = 64
    g = np.random.default_rng(seed)
    E = np.concatenate([np.full((N, 1), 10.0), 0.1 * g.standard_normal((N, D - 1))],
                       axis=1).astype(np.float32)
    C = (0.05 * g.standard_normal((V, D))).astype(np.float32)
    far = np.concatenate([np.arange(256 * j, min(V, 256 * j + 256)) for j in far_tiles])
    C[far, 0] = -20.0
    if dtype == "bf16":
        E, C = S.bf16_round(E), S.bf16_round(C)
    t = g.choice(np.setdiff1d(np.arange(V), far), size=N).astype(np.int64)
    t[5] = 256 * far_tiles[1] + 32
    t[7] = II
    return {"E": E, "C": C, "targets": t}


FAR_LAYOUTS = {
    # V, far vocabulary tiles, N: one backward chunk; far tiles in all three chunks of
    # V = 20000 (79 tiles: chunks of tiles 0-25, 26-51, 52-78), including a chunk's first tile
    # and the ragged last tile; and 20000 tokens, two backward token blocks for bf16 inputs
    # (three for fp32), so tiles are proved negligible from the maxima of later blocks too
    "one_chunk": (1280, (1, 3), 600),
    "three_chunks": (20000, (5, 30, 26, 60, 78), 600),
    "token_blocks": (1280, (1, 3), 20000),
}


@pytest.mark.parametrize("layout", sorted(FAR_LAYOUTS))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tiles_proved_negligible_skip_their_recompute(dtype, layout):
    """With the forward's tile maxima, the backward skips the recompute of the far tiles (the
    bound holds on all far tiles but the one holding a target, checked here from the returned
    maxima; at V = 20000 the softmax is nearly uniform, about 1/V < eps, so tiles without a
    target elsewhere qualify too), also in the G tiles computed inside the fused launches of
    later chunks, and returns bitwise the same gradients and skip counts as without them, which
    match the oracle."""
    V0, far_tiles, N0 = FAR_LAYOUTS[layout]
    d = _far_tiles_case(dtype, 61, V0, far_tiles, N0)
    N, V = d["E"].shape[0], d["C"].shape[0]
    n_vt, n_tb = -(-V // 256), -(-N // 256)
    w = S.dloss_weights(61, N)
    E, C, t = upload(d, dtype)
    if layout == "token_blocks":
        assert cce.backward_token_block(N, V, E.shape[1], E.dtype) < N
    tm = cce.tile_max_buffer(E, C)
    loss, lse = cce.cce_forward(E, C, t, II, tile_max=tm)
    dl = torch.from_numpy(w).to(DEV)
    # the bound, from the returned maxima: max z log2 e - min lse log2 e over valid tokens
    tmv = tm.cpu().numpy().reshape(n_tb, n_vt, 8).max(axis=2)
    l2 = lse.cpu().numpy() / math.log(2.0)
    tt = d["targets"]
    provable = provable_far = 0
    for tb in range(n_tb):
        rows = np.arange(256 * tb, min(N, 256 * tb + 256))
        ok = tt[rows] != II
        for vt in range(n_vt):
            has_t = np.any((tt[rows][ok] >= 256 * vt) & (tt[rows][ok] < 256 * vt + 256))
            if not has_t and tmv[tb, vt] - l2[rows][ok].min() < math.log2(EPS) - 2.0 ** -10:
                provable += 1
                provable_far += vt in far_tiles
    assert provable_far == n_tb * len(far_tiles) - 1, provable_far
    out = {}
    for name, arg in (("with", tm), ("without", None)):
        stats = torch.zeros(2, dtype=torch.int64, device=DEV)
        dE, dC = cce.cce_backward(dl, E, C, t, lse, II, EPS, tile_max=arg, skip_stats=stats)
        torch.cuda.synchronize()
        out[name] = (dE.cpu().numpy(), dC.cpu().numpy(), stats.tolist())
    assert np.array_equal(out["with"][0], out["without"][0])
    assert np.array_equal(out["with"][1], out["without"][1])
    assert out["with"][2] == out["without"][2]
    dE0, dC0, (sk, tot) = oracle.backward(d["E"], d["C"], d["targets"], w, II, filter_eps=EPS)
    assert out["with"][2] == [sk, tot]
    assert rel(out["with"][0], dE0) <= GRAD_TOL and rel(out["with"][1], dC0) <= GRAD_TOL
    log(f"[far tiles {dtype}] provable {provable}, skipped {sk}/{tot}, "
        f"dE {rel(out['with'][0], dE0):.2e} dC {rel(out['with'][1], dC0):.2e}")
