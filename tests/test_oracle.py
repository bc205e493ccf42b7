"""Pins for the float64 oracle: each check ties it to something other than itself.

Sources of truth: mpmath brute force at 50 digits, central finite differences, closed forms
(all-zero E, V = 1, V = 2 logistic, equal classifier rows), torch's CPU cross-entropy and
autograd in float64 (a library routine), algebraic invariants, and a pure-Python loop for the
block filter.  tests/test_oracle_mutants.py plants mistakes in the oracle and checks that these
pins catch them."""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle

II = -100


def rand_case(seed, N, V, D, scale=1.0, ignore=()):
    g = np.random.default_rng(seed)
    E = g.standard_normal((N, D))
    C = g.standard_normal((V, D)) * scale
    t = g.integers(0, V, size=N)
    for i in ignore:
        t[i] = II
    return E, C, t


# ---------------------------------------------------------------- brute force (mpmath)
def mp_loss_lse(E, C, t):
    mpmath.mp.dps = 50
    out = []
    for n in range(E.shape[0]):
        z = [mpmath.fsum(mpmath.mpf(float(E[n, d])) * mpmath.mpf(float(C[v, d]))
                         for d in range(E.shape[1])) for v in range(C.shape[0])]
        lse = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in z))
        loss = lse - z[t[n]] if t[n] != II else mpmath.mpf(0)
        out.append((float(loss), float(lse)))
    return np.array(out)


@pytest.mark.parametrize("seed,N,V,D", [(0, 6, 11, 5), (1, 8, 7, 3), (2, 3, 2, 4), (3, 5, 1, 2)])
def test_forward_matches_mpmath(seed, N, V, D):
    E, C, t = rand_case(seed, N, V, D, scale=2.0, ignore=(1,))
    loss, lse = oracle.forward(E, C, t, II)
    ref = mp_loss_lse(E, C, t)
    np.testing.assert_allclose(loss, ref[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref[:, 1], rtol=0, atol=1e-12)
    assert loss[1] == 0.0


# ---------------------------------------------------------------- finite differences
def weighted_loss(E, C, t, w):
    loss, _ = oracle.forward(E, C, t, II)
    return float((w * loss).sum())


@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_central_differences(seed):
    N, V, D = 5, 9, 4
    E, C, t = rand_case(seed, N, V, D, ignore=(3,))
    w = np.random.default_rng(seed + 10).uniform(0.5, 1.5, N)
    dE, dC, _ = oracle.backward(E, C, t, w, II)
    h = 1e-6
    for X, dX in ((E, dE), (C, dC)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = weighted_loss(E, C, t, w)
            X[idx] = old - h
            fm = weighted_loss(E, C, t, w)
            X[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(dX, num, rtol=1e-6, atol=1e-8)
    assert np.all(dE[3] == 0.0)  # ignored row


# ---------------------------------------------------------------- library cross-check
def test_matches_torch_cross_entropy_and_autograd():
    E, C, t = rand_case(5, 40, 70, 12, scale=1.5, ignore=(0, 7, 8))
    w = np.random.default_rng(6).uniform(0.5, 1.5, 40)
    Et = torch.tensor(E, requires_grad=True)
    Ct = torch.tensor(C, requires_grad=True)
    z = Et @ Ct.T
    lt = torch.nn.functional.cross_entropy(z, torch.tensor(t), ignore_index=II, reduction="none")
    (lt * torch.tensor(w)).sum().backward()
    loss, lse = oracle.forward(E, C, t, II)
    dE, dC, _ = oracle.backward(E, C, t, w, II)
    np.testing.assert_allclose(loss, lt.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(z, 1).detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dE, Et.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dC, Ct.grad.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_zero_embeddings_closed_form():
    N, V, D = 17, 1000, 8
    g = np.random.default_rng(3)
    E = np.zeros((N, D))
    C = g.standard_normal((V, D))
    t = g.integers(0, V, N)
    w = g.uniform(0.5, 1.5, N)
    loss, lse = oracle.forward(E, C, t, II)
    np.testing.assert_allclose(loss, math.log(V), rtol=0, atol=1e-12)   # 6.907755...
    np.testing.assert_allclose(lse, math.log(V), rtol=0, atol=1e-12)
    dE, dC, _ = oracle.backward(E, C, t, w, II)
    assert np.all(dC == 0.0)
    expect = w[:, None] * (C.mean(axis=0)[None, :] - C[t])
    np.testing.assert_allclose(dE, expect, rtol=1e-10, atol=1e-12)


def test_single_class_has_zero_loss_and_gradient():
    E, C, t = rand_case(4, 6, 1, 3)
    loss, lse = oracle.forward(E, C, t, II)
    np.testing.assert_allclose(loss, 0.0, atol=1e-12)
    np.testing.assert_allclose(lse, E @ C[0], atol=1e-12)
    dE, dC, _ = oracle.backward(E, C, t, np.ones(6), II)
    np.testing.assert_allclose(dE, 0.0, atol=1e-12)
    np.testing.assert_allclose(dC, 0.0, atol=1e-12)


def test_two_classes_is_logistic_loss():
    E, C, t = rand_case(8, 30, 2, 6, scale=3.0)
    loss, _ = oracle.forward(E, C, t, II)
    z = E @ C.T
    other = z[np.arange(30), 1 - t]
    mine = z[np.arange(30), t]
    softplus = np.logaddexp(0.0, other - mine)
    np.testing.assert_allclose(loss, softplus, rtol=1e-13, atol=1e-14)


def test_equal_classifier_rows_closed_form():
    N, V, D = 12, 37, 5
    g = np.random.default_rng(9)
    E = g.standard_normal((N, D))
    C = np.tile(g.standard_normal(D), (V, 1))
    t = g.integers(0, V, N)
    w = g.uniform(0.5, 1.5, N)
    loss, _ = oracle.forward(E, C, t, II)
    np.testing.assert_allclose(loss, math.log(V), atol=1e-12)
    dE, dC, _ = oracle.backward(E, C, t, w, II)
    np.testing.assert_allclose(dE, 0.0, atol=1e-12)
    onehot = np.zeros((N, V))
    onehot[np.arange(N), t] = 1.0
    expect = (w[:, None] * (1.0 / V - onehot)).T @ E
    np.testing.assert_allclose(dC, expect, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- invariants
def test_forward_invariants():
    E, C, t = rand_case(11, 50, 300, 16, scale=2.0, ignore=(4,))
    loss, lse = oracle.forward(E, C, t, II, chunk=16, vchunk=64)
    z = E @ C.T
    zmax = z.max(axis=1)
    assert np.all(lse >= zmax - 1e-12) and np.all(lse <= zmax + math.log(300) + 1e-12)
    assert np.all(loss >= 0)
    np.testing.assert_allclose(np.exp(z - lse[:, None]).sum(axis=1), 1.0, atol=1e-12)
    # shift invariance: adding the same vector b to every classifier row shifts each token's
    # logits by a constant, which cancels in the loss
    b = np.random.default_rng(12).standard_normal(16)
    loss2, lse2 = oracle.forward(E, C + b, t, II)
    np.testing.assert_allclose(loss2, loss, atol=1e-10)
    np.testing.assert_allclose(lse2 - lse, E @ b, atol=1e-10)


def test_dominant_logit_no_overflow():
    N, V, D = 4, 50, 4
    E = 100.0 * np.eye(N, D)
    C = np.zeros((V, D))
    t = np.array([3, 5, 7, 9])
    C[t, np.arange(N)] = 10.0   # each token's target logit is 1000, all its other logits 0
    loss, lse = oracle.forward(E, C, t, II)
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(lse, 1000.0, atol=1e-12)
    np.testing.assert_allclose(loss, 0.0, atol=1e-12)


def test_gradient_invariants():
    E, C, t = rand_case(13, 64, 200, 10, scale=2.0, ignore=(5, 6))
    w = np.random.default_rng(14).uniform(0.5, 1.5, 64)
    dE, dC, _ = oracle.backward(E, C, t, w, II, chunk=64, vchunk=64)
    np.testing.assert_allclose(dC.sum(axis=0), 0.0, atol=1e-11)          # sum_v p = 1
    np.testing.assert_allclose(E.T @ dE, dC.T @ C, rtol=1e-10, atol=1e-10)  # both from one G
    dE2, dC2, _ = oracle.backward(E, C, t, 2.5 * w, II)
    np.testing.assert_allclose(dE2, 2.5 * dE, rtol=1e-12, atol=1e-13)       # linear in dloss
    np.testing.assert_allclose(dC2, 2.5 * dC, rtol=1e-12, atol=1e-13)
    dEs, dCs, _ = oracle.backward(E, C, t, 0.75, II)                        # scalar dloss
    dEv, dCv, _ = oracle.backward(E, C, t, np.full(64, 0.75), II)
    np.testing.assert_array_equal(dEs, dEv)
    np.testing.assert_array_equal(dCs, dCv)


def test_chunking_does_not_change_results():
    E, C, t = rand_case(15, 70, 130, 8, ignore=(2,))
    a = oracle.forward(E, C, t, II, chunk=256, vchunk=65536)
    b = oracle.forward(E, C, t, II, chunk=64, vchunk=64)
    np.testing.assert_allclose(a[0], b[0], atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], atol=1e-12)


def test_out_of_range_target_is_an_error():
    E, C, t = rand_case(16, 4, 10, 3)
    t[2] = 10
    with pytest.raises(ValueError):
        oracle.forward(E, C, t, II)
    t[2] = -1
    with pytest.raises(ValueError):
        oracle.forward(E, C, t, II)


# ---------------------------------------------------------------- gradient filtering
def brute_filtered_grads(E, C, t, w, eps, bn, bv, floor=0.0):
    """Plain loops: per-element p, per-block decision, the optional entry floor (never the
    target entry), then the filtered G products."""
    N, V = E.shape[0], C.shape[0]
    z = [[float(np.dot(E[n], C[v])) for v in range(V)] for n in range(N)]
    G = np.zeros((N, V))
    P = np.zeros((N, V))
    for n in range(N):
        m = max(z[n])
        s = sum(math.exp(x - m) for x in z[n])
        for v in range(V):
            P[n, v] = math.exp(z[n][v] - m) / s
            if t[n] != II:
                G[n, v] = w[n] * (P[n, v] - (1.0 if v == t[n] else 0.0))
    skipped = 0
    for i in range(0, N, bn):
        for j in range(0, V, bv):
            significant = False
            for n in range(i, min(N, i + bn)):
                if t[n] == II:
                    continue
                for v in range(j, min(V, j + bv)):
                    if P[n, v] >= eps or v == t[n]:
                        significant = True
            if not significant and eps > 0:
                skipped += 1
                G[i:i + bn, j:j + bv] = 0.0
    for n in range(N):
        for v in range(V):
            if t[n] != II and v != t[n] and P[n, v] < floor:
                G[n, v] = 0.0
    return G @ C, G.T @ E, skipped


@pytest.mark.parametrize("eps", [0.0, 2.0 ** -12, 0.02])
def test_block_filter_matches_brute_force(eps):
    E, C, t = rand_case(21, 20, 45, 6, scale=2.5, ignore=(3, 17))
    w = np.random.default_rng(22).uniform(0.5, 1.5, 20)
    dE, dC, (sk, tot) = oracle.backward(E, C, t, w, II, filter_eps=eps, block_n=4, block_v=8,
                                        chunk=8, vchunk=16)
    bE, bC, bsk = brute_filtered_grads(E, C, t, w, eps, 4, 8)
    assert sk == bsk and tot == 5 * 6
    np.testing.assert_allclose(dE, bE, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dC, bC, rtol=1e-10, atol=1e-12)
    if eps == 0.02:
        assert 0 < sk < tot  # the case exercises both outcomes


def test_entry_floor_matches_brute_force():
    """With entry_floor = f, entries below f inside kept blocks are dropped, except a row's
    target entry; the case puts row 0's target at its smallest logit, far below the floor."""
    E, C, t = rand_case(24, 16, 40, 5, scale=3.0, ignore=(9,))
    z0 = E[0] @ C.T
    t[0] = int(np.argmin(z0))
    w = np.random.default_rng(25).uniform(0.5, 1.5, 16)
    eps = 0.05
    floor = eps / 256
    dE, dC, (sk, _) = oracle.backward(E, C, t, w, II, filter_eps=eps, block_n=4, block_v=8,
                                      entry_floor=floor)
    bE, bC, bsk = brute_filtered_grads(E, C, t, w, eps, 4, 8, floor)
    assert sk == bsk
    np.testing.assert_allclose(dE, bE, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dC, bC, rtol=1e-10, atol=1e-12)
    # the case exercises the rule: the target entry of row 0 lies below the floor, and kept
    # blocks hold entries on both sides of it
    lse = np.log(np.exp(z0 - z0.max()).sum()) + z0.max()
    assert np.exp(z0[t[0]] - lse) < eps / 256
    P = np.exp(E @ C.T - oracle.forward(E, C, t, II)[1][:, None])
    neg = oracle.block_negligible(P, t, t != II, eps, 0, 0, 4, 8)
    kept = ~np.kron(neg, np.ones((4, 8), dtype=bool))[:16, :40] & (t != II)[:, None]
    assert (kept & (P < eps / 256)).sum() > 20 and (kept & (P >= eps / 256)).sum() > 20
    # without the floor the result differs by more than rounding
    nE, _, _ = brute_filtered_grads(E, C, t, w, eps, 4, 8)
    assert np.linalg.norm(dE - nE) > 1e-9 * np.linalg.norm(nE)
    # and the floor is off by default
    d0 = oracle.backward(E, C, t, w, II, filter_eps=eps, block_n=4, block_v=8)
    np.testing.assert_allclose(d0[0], nE, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("eps", [0.0, 1e-4])
def test_entry_floor_closed_form_equal_rows(eps):
    """Every classifier row equal to c: all logits of a token are equal, so every softmax entry
    is exactly 1/V.  A floor just above 1/V drops every non-target entry: G keeps only
    dloss_n (1/V - 1) at each target, so dE_n = dloss_n (1/V - 1) c and dC_v = (1/V - 1)
    sum over tokens with target v of dloss_n E_n.  A floor just below 1/V drops nothing: dE = 0
    (the row of G sums to 0) and dC_v = sum_n dloss_n (1/V - [t_n = v]) E_n.  The block filter
    (eps below 1/V) keeps every block."""
    rng = np.random.default_rng(31)
    N, V, D = 40, 250, 6
    E = rng.standard_normal((N, D))
    c = rng.standard_normal(D)
    C = np.tile(c, (V, 1))
    t = rng.integers(0, V, N)
    t[[3, 17]] = II
    w = rng.uniform(0.5, 1.5, N)
    valid = t != II
    wv = np.where(valid, w, 0.0)
    onehot = np.zeros((N, V))
    onehot[np.nonzero(valid)[0], t[valid]] = 1.0
    # floor above 1/V: only the target entries survive
    dE, dC, (sk, _) = oracle.backward(E, C, t, w, II, filter_eps=eps, entry_floor=1.01 / V)
    assert sk == 0
    np.testing.assert_allclose(dE, (wv * (1.0 / V - 1.0))[:, None] * c[None, :], rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(dC, (1.0 / V - 1.0) * (onehot * wv[:, None]).T @ E, rtol=1e-12,
                               atol=1e-12)
    # floor below 1/V: nothing is dropped
    dE, dC, _ = oracle.backward(E, C, t, w, II, filter_eps=eps, entry_floor=0.99 / V)
    np.testing.assert_allclose(dE, 0.0, atol=1e-12)
    np.testing.assert_allclose(dC, ((1.0 / V) * valid[:, None] - onehot).T @ (wv[:, None] * E),
                               rtol=1e-12, atol=1e-12)


def block_filter_equal_rows_closed_form(E, c, t, w, V, bn=64, bv=64):
    """The block filter with every classifier row equal to c and eps above 1/V: every softmax
    entry is exactly 1/V < eps, so a 64 x 64 block is kept exactly when a non-ignored token of
    its token block has its target in its vocabulary block.  Token n of block b keeps the
    K_b vocabulary rows of its block's kept vocabulary blocks: G_nv = dloss_n (1/V - [v = t_n])
    for v in K_b, else 0, so dE_n = dloss_n (|K_b| / V - 1) c and
    dC_v = sum over valid n with v in K_b(n) of dloss_n E_n / V - sum over n with t_n = v of
    dloss_n E_n.  Returns dE, dC and the number of skipped blocks."""
    N, D = E.shape
    valid = t != II
    dE = np.zeros((N, D))
    dC = np.zeros((V, D))
    n_vb = -(-V // bv)
    skipped = 0
    for b0 in range(0, N, bn):
        rows = np.arange(b0, min(N, b0 + bn))
        kept_vb = sorted({int(t[n]) // bv for n in rows if valid[n]})
        skipped += n_vb - len(kept_vb)
        K = np.concatenate([np.arange(k * bv, min(V, k * bv + bv)) for k in kept_vb]) \
            if kept_vb else np.zeros(0, dtype=np.int64)
        for n in rows:
            if not valid[n]:
                continue
            dE[n] = w[n] * (len(K) / V - 1.0) * c
            dC[K] += w[n] * E[n] / V
            dC[t[n]] -= w[n] * E[n]
    return dE, dC, skipped


def test_block_filter_closed_form_flat_softmax():
    """The block filter drops each entry below eps, not a bounded sum of them: on a flat
    softmax over V > 1/eps rows (every classifier row equal, so every p = 1/V exactly) it keeps
    only the blocks that hold a target, and the filtered gradients follow the closed form of
    block_filter_equal_rows_closed_form, far from the unfiltered dE = 0.  A threshold just
    below 1/V keeps every block and gives the unfiltered result."""
    rng = np.random.default_rng(33)
    N, V, D = 150, 200, 7          # 3 token blocks (the last ragged), 4 vocabulary blocks
    E = rng.standard_normal((N, D))
    c = rng.standard_normal(D)
    C = np.tile(c, (V, 1))
    t = rng.integers(0, V, N)
    t[:64] = rng.integers(0, 64, 64)          # token block 0 keeps vocabulary block 0 only
    t[80] = 128                                # a target on a block's first row
    t[[5, 70, 149]] = II
    t[128:150] = np.where(t[128:150] == II, II, 192 + (t[128:150] % 8))   # block 2: ragged vocab block
    w = rng.uniform(0.5, 1.5, N)
    eps = 1.5 / V
    dE, dC, (sk, tot) = oracle.backward(E, C, t, w, II, filter_eps=eps)
    eE, eC, esk = block_filter_equal_rows_closed_form(E, c, t, w, V)
    assert tot == 3 * 4 and sk == esk and sk > 0
    np.testing.assert_allclose(dE, eE, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dC, eC, rtol=1e-10, atol=1e-12)
    assert np.abs(dE[t != II]).max() > 0.1 * np.abs(c).max()   # far from the unfiltered 0
    dE0, _, (sk0, _) = oracle.backward(E, C, t, w, II, filter_eps=0.5 / V)
    assert sk0 == 0
    np.testing.assert_allclose(dE0, 0.0, atol=1e-12)


@pytest.mark.parametrize("scale,seed", [(1.0, 41), (3.0, 42), (8.0, 43)])
def test_entry_floor_dropped_mass_bounds(scale, seed):
    """Dropping a set S_n of non-target entries of row n changes dE_n by
    -dloss_n sum_{v in S_n} p[n, v] C_v and dC_v by -sum_{n: v in S_n} dloss_n p[n, v] E_n, with
    every p in S_n below the floor f; so |ddE_n| <= dloss_n f sum_v |C_v| and
    |ddC_v| <= f sum_n dloss_n |E_n| (triangle inequality).  Checked row by row for random
    cases with the floor at 1/V and at 1/(4V) (f sum_v |C_v| stays below a typical |C_v|, so
    dropping a target entry would break the bound)."""
    E, C, t = rand_case(seed, 48, 60, 8, scale=scale, ignore=(5, 30))
    w = np.random.default_rng(seed + 1).uniform(0.5, 1.5, 48)
    wv = np.where(t != II, w, 0.0)
    dE0, dC0, _ = oracle.backward(E, C, t, w, II)
    for f in (1.0 / 60, 1.0 / 240):
        dE, dC, _ = oracle.backward(E, C, t, w, II, entry_floor=f)
        bE = wv * f * np.linalg.norm(C, axis=1).sum()
        bC = f * (wv * np.linalg.norm(E, axis=1)).sum()
        assert np.all(np.linalg.norm(dE - dE0, axis=1) <= bE * (1 + 1e-9) + 1e-15)
        assert np.all(np.linalg.norm(dC - dC0, axis=1) <= bC * (1 + 1e-9) + 1e-15)
        # the case drops something
        assert np.linalg.norm(dE - dE0) > 1e-6 * np.linalg.norm(dE0)


def test_filter_eps_zero_is_bitwise_unfiltered():
    E, C, t = rand_case(23, 30, 90, 7, scale=3.0)
    w = np.ones(30)
    a = oracle.backward(E, C, t, w, II)
    b = oracle.backward(E, C, t, w, II, filter_eps=0.0, block_n=64, block_v=64)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    assert a[2][0] == 0


def test_far_vocabulary_blocks_are_skipped_exactly():
    """Vocab blocks 1 and 3 (of 5, 64 wide) get logits near -200 for every token, so every
    (token block, far vocab block) pair is negligible; targets avoid them."""
    N, V, D, bn, bv = 150, 320, 4, 64, 64
    g = np.random.default_rng(31)
    E = np.zeros((N, D))
    E[:, 0] = 10.0
    E[:, 1:] = g.standard_normal((N, D - 1)) * 0.1
    C = g.standard_normal((V, D)) * 0.05
    far = np.r_[64:128, 192:256]
    C[far, 0] = -20.0
    near = np.setdiff1d(np.arange(V), far)
    t = g.choice(near, size=N)
    dE, dC, (sk, tot) = oracle.backward(E, C, t, np.ones(N), II, filter_eps=2.0 ** -12)
    assert tot == 3 * 5
    assert sk == 3 * 2
    dE0, dC0, _ = oracle.backward(E, C, t, np.ones(N), II)
    assert np.linalg.norm(dC - dC0) / np.linalg.norm(dC0) < 1e-12
    # a target inside a far block keeps that one block (its G entry is about -1)
    t[70] = 200
    _, _, (sk2, _) = oracle.backward(E, C, t, np.ones(N), II, filter_eps=2.0 ** -12)
    assert sk2 == 3 * 2 - 1
    # the same target on an ignored row does not
    t[70] = II
    _, _, (sk3, _) = oracle.backward(E, C, t, np.ones(N), II, filter_eps=2.0 ** -12)
    assert sk3 == 3 * 2


def test_token_rows_equals_full_problem_restricted():
    E, C, t = rand_case(41, 200, 300, 6, scale=3.0, ignore=(70, 130))
    w = np.zeros(200)
    rows = np.r_[64:128, 192:200]       # one whole block and the ragged last block
    w[rows] = np.random.default_rng(42).uniform(0.5, 1.5, len(rows))
    for eps in (0.0, 0.01):
        dE, dC, (sk, _) = oracle.backward(E, C, t, w, II, filter_eps=eps)
        loss, lse = oracle.forward(E, C, t, II)
        r = oracle.token_rows(E, C, t, rows, w[rows], II, filter_eps=eps, vchunk=128)
        np.testing.assert_allclose(r["loss"], loss[rows], atol=1e-12)
        np.testing.assert_allclose(r["lse"], lse[rows], atol=1e-12)
        np.testing.assert_allclose(r["dE"], dE[rows], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(r["dC_part"], dC, rtol=1e-10, atol=1e-13)


def test_loss_mean():
    E, C, t = rand_case(51, 40, 60, 5, ignore=(1, 2, 3))
    m, dE, dC, nv = oracle.loss_mean(E, C, t, II)
    loss, _ = oracle.forward(E, C, t, II)
    assert nv == 37
    assert m == pytest.approx(loss.sum() / 37, rel=1e-14)
    bE, bC, _ = oracle.backward(E, C, t, np.full(40, 1 / 37), II)
    np.testing.assert_allclose(dE, bE, rtol=1e-14)
    np.testing.assert_allclose(dC, bC, rtol=1e-14)
    t[:] = II
    m, dE, dC, nv = oracle.loss_mean(E, C, t, II)
    assert (m, nv) == (0.0, 0) and not dE.any() and not dC.any()


def test_oracle_reproduces_its_regression_fixture():
    import json
    import os
    import cce_synth as S
    with open(os.path.join(os.path.dirname(__file__), "golden", "oracle_small_case.json")) as f:
        g = json.load(f)
    c = g["case"]
    d = S.small_case(N=c["N"], D=c["D"], V=c["V"], dtype=c["dtype"], seed=c["seed"],
                     c_scale=c["c_scale"], zipf_s=c["zipf_s"], ignore_frac=c["ignore_frac"])
    assert d["targets"].tolist() == g["targets"]
    w = S.dloss_weights(c["dloss_seed"], c["N"])
    loss, lse = oracle.forward(d["E"], d["C"], d["targets"], II)
    dE, dC, (sk, tot) = oracle.backward(d["E"], d["C"], d["targets"], w, II,
                                        filter_eps=c["filter_eps"], block_n=c["block_n"],
                                        block_v=c["block_v"], entry_floor=c["entry_floor"])
    np.testing.assert_allclose(loss, g["loss"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, g["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dE.sum(1), g["dE_rowsum"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dC.sum(1), g["dC_rowsum"], rtol=0, atol=1e-12)
    assert (sk, tot) == (g["skipped"], g["total"])
    assert 0 < sk < tot
