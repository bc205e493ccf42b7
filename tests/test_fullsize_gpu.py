"""Parity at the full benchmark sizes, in the launch configuration bench.py times.

The oracle cannot materialise a full-size problem, so it checks sampled outputs exactly:
  * loss and LSE of two whole 64-token blocks (the first and the last);
  * a backward whose upstream gradient is zero outside those blocks: then dE is zero outside
    them and dC is exactly the sampled rows' contribution, which the oracle computes for every
    vocabulary row (oracle.token_rows);
  * a backward with a full upstream gradient: the sampled dE rows again (a row of dE depends
    only on its own token block), plus E^T dE = dC^T C, an identity that holds for any G and
    so ties dC to dE at every size, and sum_v dC_v = 0 when nothing is filtered.
"""
import numpy as np
import pytest
import torch

import cce_synth as S
import linear_cross_entropy_cce_amd as cce
import oracle
from gpu_helpers import DEV, GRAD_TOL, II, LOSS_TOL, log, rel, upload

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


@pytest.mark.parametrize("name,eps_override", CASES,
                         ids=[f"{n}-eps{'default' if e is None else e}" for n, e in CASES])
def test_full_size_sampled(name, eps_override):
    w = S.WORKLOADS[name]
    eps = w.filter_eps if eps_override is None else eps_override
    d = inputs(name)
    N = w.N
    rows = np.r_[0:64, N - 64:N]
    E, C, t = upload(d, w.dtype)
    loss, lse = cce.cce_forward(E, C, t, II)
    wrow = S.dloss_weights(7, len(rows))
    dl = torch.zeros(N, dtype=torch.float32, device=DEV)
    dl[torch.from_numpy(rows).to(DEV)] = torch.from_numpy(wrow).to(DEV)
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, eps)
    torch.cuda.synchronize()
    log(f"[{name} eps={eps}] GPU done, running the oracle on {len(rows)} tokens")
    r = oracle.token_rows(d["E"], d["C"], d["targets"], rows, wrow, II, filter_eps=eps)
    g_loss, g_lse = loss.cpu().numpy()[rows], lse.cpu().numpy()[rows]
    assert np.abs(g_loss - r["loss"]).max() <= LOSS_TOL, np.abs(g_loss - r["loss"]).max()
    assert np.abs(g_lse - r["lse"]).max() <= LOSS_TOL
    mask = torch.ones(N, dtype=torch.bool, device=DEV)
    mask[torch.from_numpy(rows).to(DEV)] = False
    assert float(dE[mask].abs().max()) == 0.0
    e_dE = rel(dE.cpu().numpy()[rows], r["dE"])
    e_dC = rel(dC.cpu().numpy(), r["dC_part"])
    log(f"[{name} eps={eps}] loss {np.abs(g_loss - r['loss']).max():.2e} dE {e_dE:.2e} "
        f"dC {e_dC:.2e}")
    assert e_dE <= GRAD_TOL and e_dC <= GRAD_TOL
    del r

    # full upstream gradient: sampled rows again, then identities at full size
    wfull = S.dloss_weights(8, N)
    wfull_t = torch.from_numpy(wfull).to(DEV)
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    dE, dC = cce.cce_backward(wfull_t, E, C, t, lse, II, eps, dE=dE, dC=dC, skip_stats=stats)
    torch.cuda.synchronize()
    r = oracle.token_rows(d["E"], d["C"], d["targets"], rows, wfull[rows], II, filter_eps=eps)
    assert rel(dE.cpu().numpy()[rows], r["dE"]) <= GRAD_TOL
    lhs = E.double().T @ dE.double()
    rhs = dC.double().T @ C.double()
    e_id = float((lhs - rhs).norm() / rhs.norm())
    log(f"[{name} eps={eps}] E^T dE vs dC^T C {e_id:.2e}; skipped {stats.tolist()}")
    assert e_id <= 1e-3
    if eps == 0.0:
        s = dC.double().sum(0)
        assert float(s.norm() / dC.double().abs().sum(0).norm()) <= 1e-3
        assert int(stats[0]) == 0
    assert 0 <= int(stats[0]) <= int(stats[1]) == -(-N // 64) * -(-w.V // 64)


def test_largest_batch_sampled():
    """N = 2^24 tokens, the largest the kernels take (D = 8, V = 64): 65 536 token tiles, one
    dC tile reducing over 262 144 stages, filter flags for 262 144 token blocks.  Sampled like
    the benchmark sizes: two 64-token blocks against the oracle, the rest through E^T dE =
    dC^T C."""
    N = 1 << 24
    d = S.small_case(N, 8, 64, "bf16", 45, 3.0, 1.1, 0.1)
    rows = np.r_[0:64, N - 64:N]
    E, C, t = upload(d, "bf16")
    loss, lse = cce.cce_forward(E, C, t, II)
    wrow = S.dloss_weights(9, len(rows))
    dl = torch.zeros(N, dtype=torch.float32, device=DEV)
    dl[torch.from_numpy(rows).to(DEV)] = torch.from_numpy(wrow).to(DEV)
    stats = torch.zeros(2, dtype=torch.int64, device=DEV)
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, S.FILTER_EPS, skip_stats=stats)
    torch.cuda.synchronize()
    r = oracle.token_rows(d["E"], d["C"], d["targets"], rows, wrow, II, filter_eps=S.FILTER_EPS)
    g_loss, g_lse = loss.cpu().numpy()[rows], lse.cpu().numpy()[rows]
    assert np.abs(g_loss - r["loss"]).max() <= LOSS_TOL
    assert np.abs(g_lse - r["lse"]).max() <= LOSS_TOL
    e_dE = rel(dE.cpu().numpy()[rows], r["dE"])
    e_dC = rel(dC.cpu().numpy(), r["dC_part"])
    log(f"[N=2^24] loss {np.abs(g_loss - r['loss']).max():.2e} dE {e_dE:.2e} dC {e_dC:.2e} "
        f"skipped {stats.tolist()}")
    assert e_dE <= GRAD_TOL and e_dC <= GRAD_TOL
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
