"""Parity at the full benchmark sizes, in the launch configuration bench.py times.

The oracle cannot materialise a full-size problem, so it checks sampled outputs exactly:
  * sampled token blocks: one 64-token block from each of 16 token tiles spread evenly over the
    grid (every tile when there are at most 16), at varying places within their tile, plus the
    last (ragged) block; loss and LSE of those tokens;
  * a backward whose upstream gradient is zero outside those blocks: then dE is zero outside
    them and dC is exactly the sampled rows' contribution, which the oracle computes for every
    vocabulary row (oracle.token_rows).  dE and dC are compared with the oracle for the same
    threshold (whole matrices and row by row, rows of borderline blocks excepted) and, with
    filtering on, with the unfiltered oracle, the definition the filter approximates;
  * the same backward with the forward's tile maxima is bitwise the backward without them;
  * a backward with a full upstream gradient: the sampled dE rows again (a row of dE depends
    only on its own token block and scales with its own dloss), plus E^T dE = dC^T C, an
    identity that holds for any G and so ties dC to dE at every size, and sum_v dC_v = 0 when
    nothing is filtered.
"""
import numpy as np
import pytest
import torch

import cce_synth as S
import linear_cross_entropy_cce_amd as cce
import oracle
from gpu_helpers import DEV, GRAD_TOL, II, LOSS_TOL, ROW_TOL, log, rel, row_err, upload

pytestmark = pytest.mark.gpu

CASES = [("gemma2_2b_head", None), ("llama3_8b_head", None), ("llama3_8b_head", 0.0),
         ("long_seq", None), ("sparse_stress", None), ("sparse_stress", 0.0)]

_cache = {}


def inputs(name):
    if name not in _cache:
        _cache.clear()
        log(f"[{name}] generating inputs")
        _cache[name] = S.make_inputs(S.WORKLOADS[name])
    return _cache[name]


def sampled_rows(N, k=16):
    """Whole aligned 64-token blocks: block (i mod 4) of each of k token tiles spread evenly
    over the grid (every tile when there are at most k), and the last block, ragged or not."""
    n_tiles = -(-N // 256)
    tiles = np.unique(np.linspace(0, n_tiles - 1, min(k, n_tiles)).round().astype(np.int64))
    blocks = {int(tb * 4 + i % 4) for i, tb in enumerate(tiles) if tb * 256 + (i % 4) * 64 < N}
    blocks.add((N - 1) // 64)
    rows = np.concatenate([np.arange(b * 64, min(N, b * 64 + 64)) for b in sorted(blocks)])
    return rows, sorted(blocks)


def excluded_rows(border, blocks, V):
    """Token rows (positions within the sample) and vocabulary rows of the borderline blocks."""
    pos = {b: i for i, b in enumerate(blocks)}
    tok, voc = set(), set()
    for tb, vb in border:
        tok.add(pos[tb])
        voc.update(range(vb * 64, min(V, vb * 64 + 64)))
    return tok, np.array(sorted(voc), dtype=np.int64)


@pytest.mark.parametrize("name,eps_override", CASES,
                         ids=[f"{n}-eps{'default' if e is None else e}" for n, e in CASES])
def test_full_size_sampled(name, eps_override):
    w = S.WORKLOADS[name]
    eps = w.filter_eps if eps_override is None else eps_override
    d = inputs(name)
    N, V = w.N, w.V
    rows, blocks = sampled_rows(N)
    log(f"[{name} eps={eps}] sampling {len(rows)} tokens in {len(blocks)} blocks: {blocks}")
    E, C, t = upload(d, w.dtype)
    tmax = cce.tile_max_buffer(E, C)
    loss, lse = cce.cce_forward(E, C, t, II, tile_max=tmax)
    wrow = S.dloss_weights(7, len(rows))
    rows_t = torch.from_numpy(rows).to(DEV)
    dl = torch.zeros(N, dtype=torch.float32, device=DEV)
    dl[rows_t] = torch.from_numpy(wrow).to(DEV)
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, eps, skip_stats=stats)
    dE_m, dC_m = cce.cce_backward(dl, E, C, t, lse, II, eps, tile_max=tmax)
    torch.cuda.synchronize()
    assert torch.equal(dE, dE_m) and torch.equal(dC, dC_m)   # the maxima change nothing
    del dE_m, dC_m
    mask = torch.ones(N, dtype=torch.bool, device=DEV)
    mask[rows_t] = False
    assert float(dE[mask].abs().max()) == 0.0
    g_loss, g_lse = loss.cpu().numpy()[rows], lse.cpu().numpy()[rows]
    g_dE = dE.cpu().numpy()[rows]
    g_dC = dC.cpu().numpy()
    log(f"[{name} eps={eps}] GPU done, running the oracle on {len(rows)} tokens")
    thresholds = (eps, 0.0) if eps > 0 else (0.0,)
    r = oracle.token_rows(d["E"], d["C"], d["targets"], rows, wrow, II, filter_eps=thresholds)
    e_loss = np.abs(g_loss - r["loss"]).max()
    assert e_loss <= LOSS_TOL, e_loss
    assert np.abs(g_lse - r["lse"]).max() <= LOSS_TOL
    assert np.all(g_loss[d["targets"][rows] == II] == 0.0)
    same = r["by_eps"][eps]
    e_dE, e_dC = rel(g_dE, same["dE"]), rel(g_dC, same["dC_part"])
    # row by row, except the rows of blocks whose decision float32 may take the other way
    tok_x, voc_x = excluded_rows(same["border"], blocks, V)
    pos = np.arange(len(rows))
    keep_t = pos[~np.isin(pos // 64, sorted(tok_x))]
    keep_v = np.setdiff1d(np.arange(V), voc_x)
    r_dE = row_err(g_dE[keep_t], same["dE"][keep_t])
    r_dC = row_err(g_dC[keep_v], same["dC_part"][keep_v])
    # rows of the last vocabulary chunk, checked on their own too
    vc = cce.backward_chunk(N, V, w.D, E.dtype)
    last = keep_v[keep_v >= V - vc]
    r_last = row_err(g_dC[last], same["dC_part"][last])
    msg = (f"[{name} eps={eps}] loss {e_loss:.2e} dE {e_dE:.2e} dC {e_dC:.2e} rows dE {r_dE:.2e} "
           f"dC {r_dC:.2e} (last chunk {r_last:.2e}); borderline blocks {len(same['border'])}; "
           f"skipped {int(stats[0])} (oracle on the sample {same['skipped']})")
    if eps > 0:
        unf = r["by_eps"][0.0]
        u_dE, u_dC = rel(g_dE, unf["dE"]), rel(g_dC, unf["dC_part"])
        msg += f"; vs unfiltered dE {u_dE:.2e} dC {u_dC:.2e}"
    log(msg)
    assert e_dE <= GRAD_TOL and e_dC <= GRAD_TOL
    assert r_dE <= ROW_TOL and r_dC <= ROW_TOL and r_last <= ROW_TOL
    if eps > 0:
        assert u_dE <= GRAD_TOL and u_dC <= GRAD_TOL

    # full upstream gradient: sampled rows again, then identities at full size
    wfull = S.dloss_weights(8, N)
    wfull_t = torch.from_numpy(wfull).to(DEV)
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    dE, dC = cce.cce_backward(wfull_t, E, C, t, lse, II, eps, tile_max=tmax, dE=dE, dC=dC,
                              skip_stats=stats)
    torch.cuda.synchronize()
    # a row of dE is linear in its own dloss and the filter does not look at dloss
    scale = (wfull[rows] / wrow)[:, None]
    f_dE = dE.cpu().numpy()[rows]
    assert rel(f_dE, same["dE"] * scale) <= GRAD_TOL
    assert row_err(f_dE[keep_t], (same["dE"] * scale)[keep_t]) <= ROW_TOL
    lhs = E.double().T @ dE.double()
    rhs = dC.double().T @ C.double()
    e_id = float((lhs - rhs).norm() / rhs.norm())
    log(f"[{name} eps={eps}] E^T dE vs dC^T C {e_id:.2e}; skipped {stats.tolist()}")
    assert e_id <= 1e-3
    if eps == 0.0:
        s = dC.double().sum(0)
        assert float(s.norm() / dC.double().abs().sum(0).norm()) <= 1e-3
        assert int(stats[0]) == 0
    assert 0 <= int(stats[0]) <= int(stats[1]) == -(-N // 64) * -(-V // 64)


def test_largest_batch_sampled():
    """N = 2^24 tokens, the largest the kernels take (D = 8, V = 64): 65 536 token tiles in
    1024 token blocks, filter flags for 262 144 token blocks.  Sampled like the benchmark
    sizes: the sampled blocks against the oracle, the rest through E^T dE = dC^T C."""
    N = 1 << 24
    d = S.small_case(N, 8, 64, "bf16", 45, 3.0, 1.1, 0.1)
    rows, blocks = sampled_rows(N)
    E, C, t = upload(d, "bf16")
    loss, lse = cce.cce_forward(E, C, t, II)
    wrow = S.dloss_weights(9, len(rows))
    dl = torch.zeros(N, dtype=torch.float32, device=DEV)
    dl[torch.from_numpy(rows).to(DEV)] = torch.from_numpy(wrow).to(DEV)
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, S.FILTER_EPS, skip_stats=stats)
    torch.cuda.synchronize()
    r = oracle.token_rows(d["E"], d["C"], d["targets"], rows, wrow, II,
                          filter_eps=(S.FILTER_EPS, 0.0))
    g_loss, g_lse = loss.cpu().numpy()[rows], lse.cpu().numpy()[rows]
    assert np.abs(g_loss - r["loss"]).max() <= LOSS_TOL
    assert np.abs(g_lse - r["lse"]).max() <= LOSS_TOL
    e_dE = rel(dE.cpu().numpy()[rows], r["dE"])
    e_dC = rel(dC.cpu().numpy(), r["dC_part"])
    u_dE = rel(dE.cpu().numpy()[rows], r["by_eps"][0.0]["dE"])
    u_dC = rel(dC.cpu().numpy(), r["by_eps"][0.0]["dC_part"])
    log(f"[N=2^24] loss {np.abs(g_loss - r['loss']).max():.2e} dE {e_dE:.2e} dC {e_dC:.2e} "
        f"vs unfiltered dE {u_dE:.2e} dC {u_dC:.2e} skipped {stats.tolist()}")
    assert e_dE <= GRAD_TOL and e_dC <= GRAD_TOL and u_dE <= GRAD_TOL and u_dC <= GRAD_TOL
    assert int(stats[1]) == (N // 64) * 1
    wfull = torch.from_numpy(S.dloss_weights(10, N)).to(DEV)
    dE, dC = cce.cce_backward(wfull, E, C, t, lse, II, 0.0, dE=dE, dC=dC)
    torch.cuda.synchronize()
    lhs = E.double().T @ dE.double()
    rhs = dC.double().T @ C.double()
    e_id = float((lhs - rhs).norm() / rhs.norm())
    s = dC.double().sum(0)
    log(f"[N=2^24] E^T dE vs dC^T C {e_id:.2e}")
    assert e_id <= 1e-3
    assert float(s.norm() / dC.double().abs().sum(0).norm()) <= 1e-3
