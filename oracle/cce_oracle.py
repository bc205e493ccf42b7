"""Plain, slow, float64 CPU oracle for the Cut Cross-Entropy (CCE) head.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its Python
binding) imports, calls or links this module.  It shares no code, constants or helpers with
the GPU path; only the seeded input generator (cce_synth) feeds both.

Citations refer to the CCE abstract, the text on the taxoreview.com page "dblp:393/3562"
(repeated word for word on page "dblp:117/4058"); "s5" means its fifth sentence.

What is computed (all in float64, logits materialised one chunk at a time, never whole):

  z[n, v]   = sum_d E[n, d] * C[v, d]                        classifier-head logits (s3)
  lse[n]    = log sum_v exp(z[n, v])                          log-sum-exp over the vocabulary (s5)
  loss[n]   = lse[n] - z[n, t[n]]  if t[n] != ignore_index, else 0
                                                              cross-entropy using only the
                                                              correct token's logit (s4, s5)
  p[n, v]   = exp(z[n, v] - lse[n])                           softmax
  G[n, v]   = dloss[n] * (p[n, v] - [v == t[n]]) for valid n, 0 for ignored n
  dE        = G @ C,     dC = G^T @ E                         gradients of sum_n dloss[n] loss[n]

Gradient filtering (s9: gradient terms too small to matter are dropped).  The pages give neither a threshold nor a granularity.  Reading used here: the
token x vocab plane is cut into aligned blocks of block_n x block_v (64 x 64 by default, the
granularity the GPU library reports); a block is negligible iff every valid token row n in it
has p[n, v] < filter_eps for every v in it AND no valid row's target lies in it.  Negligible
blocks of G are set to zero before dE and dC are formed.  filter_eps = 0 filters nothing.
Rows whose target is ignore_index have G = 0 and do not make a block significant.

Optional entry floor (an approximation on top of the block filter, off unless entry_floor > 0):
inside the blocks that are kept, a non-target entry whose p is below entry_floor is set to zero
as well; the target entry never is.  Dropping a set S_n of entries of row n changes row n of dE
by -dloss[n] sum_{v in S_n} p[n, v] C[v], so by at most dloss[n] * entry_floor * sum_v |C[v]|,
and row v of dC by at most entry_floor * sum_n dloss[n] |E[n]|.

Pins: every function here is checked in tests/test_oracle.py against mpmath brute force,
closed forms, invariants, finite differences and torch's CPU cross-entropy; the block filter
is checked against a pure-Python loop, constructed far-away blocks and the closed form of a
flat softmax (equal classifier rows, eps above 1/V: only target-holding blocks survive); the
entry floor against
the closed form of equal classifier rows (every p = 1/V exactly, so a floor just above or just
below 1/V drops every non-target entry or none) and the dropped-mass bounds above.
"""
from __future__ import annotations

import numpy as np

__all__ = ["logits", "forward", "backward", "loss_mean", "block_negligible", "entry_negligible",
           "token_rows", "validate_targets"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def validate_targets(targets, V: int, ignore_index: int) -> np.ndarray:
    """Targets must be ignore_index or inside [0, V); anything else is an error."""
    t = np.asarray(targets, dtype=np.int64)
    bad = (t != ignore_index) & ((t < 0) | (t >= V))
    if bad.any():
        raise ValueError(f"target out of range at rows {np.nonzero(bad)[0][:8].tolist()}")
    return t


def logits(E_rows, C, v0: int = 0, v1: int | None = None) -> np.ndarray:
    """z = E_rows @ C[v0:v1]^T in float64 (the matrix product is the library step)."""
    v1 = C.shape[0] if v1 is None else v1
    return _f64(E_rows) @ _f64(C[v0:v1]).T


def _rows_lse_and_target(E_rows, C, t_rows, vchunk: int):
    """LSE and target logit for a few rows, streaming over vocabulary chunks (s5: the
    log-sum-exp is taken over all logits without keeping them).  Two passes: max, then sum."""
    n = E_rows.shape[0]
    V = C.shape[0]
    m = np.full(n, -np.inf)
    for v0 in range(0, V, vchunk):
        z = logits(E_rows, C, v0, min(V, v0 + vchunk))
        m = np.maximum(m, z.max(axis=1))
    s = np.zeros(n)
    zt = np.zeros(n)
    for v0 in range(0, V, vchunk):
        v1 = min(V, v0 + vchunk)
        z = logits(E_rows, C, v0, v1)
        s += np.exp(z - m[:, None]).sum(axis=1)
        inside = (t_rows >= v0) & (t_rows < v1)
        idx = np.nonzero(inside)[0]
        zt[idx] = z[idx, t_rows[idx] - v0]
    return m + np.log(s), zt


def forward(E, C, targets, ignore_index: int = -100, chunk: int = 256, vchunk: int = 65536):
    """Per-token loss and LSE, both float64 [N].  Ignored rows: loss 0, LSE still returned."""
    N, V = E.shape[0], C.shape[0]
    t = validate_targets(targets, V, ignore_index)
    loss = np.zeros(N)
    lse = np.zeros(N)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        tr = t[n0:n1]
        l, zt = _rows_lse_and_target(E[n0:n1], C, np.where(tr == ignore_index, -1, tr), vchunk)
        lse[n0:n1] = l
        valid = tr != ignore_index
        loss[n0:n1] = np.where(valid, l - zt, 0.0)
    return loss, lse


def _dloss_vector(dloss, N: int) -> np.ndarray:
    d = _f64(dloss)
    if d.ndim == 0:
        return np.full(N, float(d))
    return d.reshape(N)


def block_negligible(P, t_rows, valid_rows, filter_eps: float, n0: int, v0: int,
                     block_n: int, block_v: int) -> np.ndarray:
    """Negligible-block mask for a probability sub-matrix P (rows n0.., columns v0..), whose
    origin is aligned to the block grid.  Returns bool [ceil(rows/bn), ceil(cols/bv)]."""
    rows, cols = P.shape
    nb, vb = -(-rows // block_n), -(-cols // block_v)
    out = np.ones((nb, vb), dtype=bool)
    if filter_eps <= 0:
        out[:] = False
        return out
    big = (P >= filter_eps) & valid_rows[:, None]
    for i in range(nb):
        r0, r1 = i * block_n, min(rows, (i + 1) * block_n)
        sig_cols = big[r0:r1].any(axis=0)
        tv = t_rows[r0:r1][valid_rows[r0:r1]] - v0
        for j in range(vb):
            c0, c1 = j * block_v, min(cols, (j + 1) * block_v)
            has_target = bool(((tv >= c0) & (tv < c1)).any())
            out[i, j] = not (sig_cols[c0:c1].any() or has_target)
    return out


def entry_negligible(P, t_rows, valid_rows, entry_floor: float, v0: int) -> np.ndarray:
    """Entries of a probability sub-matrix P (columns v0..) below entry_floor, other than each
    valid row's target entry.  Returns bool, P's shape.  Rows that are not valid are never
    marked (their G is zero anyway); entry_floor = 0 marks nothing."""
    out = (P < entry_floor) & valid_rows[:, None]
    rows = np.nonzero(valid_rows & (t_rows >= v0) & (t_rows < v0 + P.shape[1]))[0]
    out[rows, t_rows[rows] - v0] = False
    return out


def backward(E, C, targets, dloss, ignore_index: int = -100, filter_eps: float = 0.0,
             block_n: int = 64, block_v: int = 64, chunk: int = 256, vchunk: int = 65536,
             entry_floor: float = 0.0):
    """dE [N,D] and dC [V,D] in float64, plus (negligible blocks, total blocks).

    The LSE is recomputed here from E and C (the oracle never takes the GPU's LSE)."""
    N, D = E.shape
    V = C.shape[0]
    t = validate_targets(targets, V, ignore_index)
    d = _dloss_vector(dloss, N)
    assert chunk % block_n == 0 and vchunk % block_v == 0
    C64 = _f64(C)
    dE = np.zeros((N, D))
    dC = np.zeros((V, D))
    skipped = 0
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        tr = t[n0:n1]
        valid = tr != ignore_index
        E_rows = _f64(E[n0:n1])
        lse, _ = _rows_lse_and_target(E_rows, C, np.where(valid, tr, -1), vchunk)
        for v0 in range(0, V, vchunk):
            v1 = min(V, v0 + vchunk)
            z = E_rows @ C64[v0:v1].T
            P = np.exp(z - lse[:, None])
            G = P.copy()
            ridx = np.nonzero(valid & (tr >= v0) & (tr < v1))[0]
            G[ridx, tr[ridx] - v0] -= 1.0
            G *= (d[n0:n1] * valid)[:, None]
            neg = block_negligible(P, tr, valid, filter_eps, n0, v0, block_n, block_v)
            skipped += int(neg.sum())
            if neg.any():
                for i, j in zip(*np.nonzero(neg)):
                    G[i * block_n:(i + 1) * block_n, j * block_v:(j + 1) * block_v] = 0.0
            G[entry_negligible(P, tr, valid, entry_floor, v0)] = 0.0
            dE[n0:n1] += G @ C64[v0:v1]
            dC[v0:v1] += G.T @ E_rows
    total = (-(-N // block_n)) * (-(-V // block_v))
    return dE, dC, (skipped, total)


def loss_mean(E, C, targets, ignore_index: int = -100, filter_eps: float = 0.0,
              block_n: int = 64, block_v: int = 64, entry_floor: float = 0.0):
    """Mean over valid tokens of the per-token loss, and its gradients.

    Reading: the mean divides by N_valid = number of tokens whose target is not
    ignore_index; with N_valid = 0 the mean and both gradients are defined as 0."""
    loss, _ = forward(E, C, targets, ignore_index)
    t = np.asarray(targets, dtype=np.int64)
    n_valid = int((t != ignore_index).sum())
    N, D = E.shape
    if n_valid == 0:
        return 0.0, np.zeros((N, D)), np.zeros((C.shape[0], D)), 0
    mean = float(loss.sum() / n_valid)
    dE, dC, _ = backward(E, C, targets, np.full(N, 1.0 / n_valid), ignore_index, filter_eps,
                         block_n, block_v, entry_floor=entry_floor)
    return mean, dE, dC, n_valid


def token_rows(E, C, targets, rows, dloss_rows, ignore_index: int = -100,
               filter_eps=0.0, block_n: int = 64, block_v: int = 64,
               vchunk: int = 16384, entry_floor: float = 0.0, border_band: float = 1e-3):
    """The oracle restricted to a set of token rows, for checks at full size.

    rows must be a union of whole aligned token blocks (of block_n rows, the last one may be
    ragged) so that block filtering is decided exactly as on the full problem.  Returns loss,
    lse and dE for those rows, and dC_part = sum over those rows of G[n, :]^T E[n, :], which is
    the whole of dC when every other row has dloss = 0.

    filter_eps may be one threshold or a sequence of them: the gradients are then formed for
    each threshold from the same softmax values and returned in result["by_eps"][eps] (the
    top-level dE, dC_part and skipped are those of the first threshold).  For each threshold,
    "border" lists the (token block, vocabulary block) pairs that hold no valid target and whose
    largest softmax value lies within border_band of the threshold (relative): there a float32
    evaluation of the same softmax may decide the block the other way."""
    eps_list = tuple(float(e) for e in np.atleast_1d(filter_eps))
    rows = np.asarray(rows, dtype=np.int64)
    V = C.shape[0]
    D = E.shape[1]
    t = validate_targets(np.asarray(targets)[rows], V, ignore_index)
    valid = t != ignore_index
    d = _f64(dloss_rows).reshape(-1)
    E_rows = _f64(E[rows])
    C64 = _f64(C)
    loss = np.zeros(len(rows))
    lse = np.zeros(len(rows))
    per = {e: {"G": np.zeros((len(rows), V)), "skipped": 0, "border": []} for e in eps_list}
    # one aligned token block at a time, so the filter sees whole blocks; the block's logits
    # over the whole vocabulary are formed once (vocabulary chunk by chunk) and kept; the
    # filtered G of all sampled rows is kept per threshold for the two products at the end
    blk = rows // block_n
    for b in np.unique(blk):
        sel = np.nonzero(blk == b)[0]
        z = np.concatenate([logits(E_rows[sel], C64, v0, min(V, v0 + vchunk))
                            for v0 in range(0, V, vchunk)], axis=1)
        m = z.max(axis=1)
        l = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        ts = t[sel]
        vs = valid[sel]
        lse[sel] = l
        ridx = np.nonzero(vs)[0]
        loss[sel[ridx]] = l[ridx] - z[ridx, ts[ridx]]
        P = np.exp(z - l[:, None])
        del z
        G0 = P.copy()
        G0[ridx, ts[ridx]] -= 1.0
        G0 *= (d[sel] * vs)[:, None]
        G0[entry_negligible(P, ts, vs, entry_floor, 0)] = 0.0
        # largest valid-row softmax value of each vocabulary block, and the blocks that hold a
        # valid target (for the borderline list)
        nvb = -(-V // block_v)
        bmax = np.where(vs[:, None], P, 0.0)
        bmax = np.array([bmax[:, j * block_v:(j + 1) * block_v].max() for j in range(nvb)])
        has_t = np.zeros(nvb, dtype=bool)
        has_t[ts[ridx] // block_v] = True
        for e in eps_list:
            r = per[e]
            if e > 0:
                near = np.nonzero(~has_t & (np.abs(bmax - e) <= border_band * e))[0]
                r["border"] += [(int(b), int(j)) for j in near]
            G = G0.copy()
            neg = block_negligible(P, ts, vs, e, int(b) * block_n, 0, block_n, block_v)
            r["skipped"] += int(neg.sum())
            for i, j in zip(*np.nonzero(neg)):
                G[i * block_n:(i + 1) * block_n, j * block_v:(j + 1) * block_v] = 0.0
            r["G"][sel] = G
            del G
    for e in eps_list:
        r = per[e]
        G = r.pop("G")
        r["dE"] = G @ C64
        r["dC_part"] = G.T @ E_rows
        del G
    first = per[eps_list[0]]
    return {"loss": loss, "lse": lse, "dE": first["dE"], "dC_part": first["dC_part"],
            "skipped": first["skipped"], "by_eps": per}
