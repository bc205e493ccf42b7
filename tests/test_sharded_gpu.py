"""Vocabulary-sharded head emulated on one GPU (cce_forward_shard / cce_merge_shards /
cce_backward_shard): the sharded results against the float64 oracle of the whole head, and
against the unsharded library call."""
import numpy as np
import pytest
import torch

import cce_synth as S
import linear_cross_entropy_cce_amd as cce
import oracle
from gpu_helpers import DEV, EPS, GRAD_TOL, II, LOSS_TOL, ROW_TOL, log, rel, row_err, upload
from linear_cross_entropy_cce_amd import sharded

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bounds", [[0, 640, 1000, 1537, 3000], [0, 1536, 3000]],
                         ids=["ragged4", "two"])
@pytest.mark.parametrize("eps", [0.0, EPS])
def test_sharded_matches_oracle(bounds, eps):
    N, D, V = 300, 72, 3000
    d = S.small_case(N, D, V, "bf16", 121, 3.0, 1.1, 0.1)
    log(f"[sharded] bounds={bounds} eps={eps}")
    E, C, t = upload(d, "bf16")
    w = S.dloss_weights(121, N)
    loss, lse, dE, dC = sharded.forward_backward(E, C, t, bounds, II, eps,
                                                 dloss=torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    rl, rlse = oracle.forward(d["E"], d["C"], d["targets"], II)
    rE, rC, _ = oracle.backward(d["E"], d["C"], d["targets"], w, II, filter_eps=0.0)
    assert np.abs(loss.cpu().numpy() - rl).max() <= LOSS_TOL
    assert np.abs(lse.cpu().numpy() - rlse).max() <= LOSS_TOL
    # filtered results (blocks aligned to each shard's rows) against the unfiltered oracle
    assert rel(dE.cpu().numpy(), rE) <= GRAD_TOL
    assert rel(dC.cpu().numpy(), rC) <= GRAD_TOL


@pytest.mark.parametrize("eps", [0.0, EPS])
def test_shards_of_several_backward_chunks(eps):
    """Shards wider than one backward vocabulary chunk (8192 rows): each of the two shards of
    V = 20000 runs two chunks, so chunk offsets inside a shard meet the shard's own offset in
    the target test and in the tile maxima."""
    N, D, V = 300, 64, 20000
    d = S.small_case(N, D, V, "bf16", 124, 3.0, 1.1, 0.1)
    bounds = [0, 9984, V]
    assert all(cce.backward_chunk(N, b - a, D, torch.bfloat16) < b - a
               for a, b in zip(bounds, bounds[1:]))
    # targets in both chunks of both shards: each chunk's first row (chunks of 19 + 20 and
    # 20 + 20 tiles), the rows on either side of the shard boundary, the last row
    for i, v in enumerate((0, 4864, 8191, 9983, 9984, 15104, 19999)):
        d["targets"][i] = v
    E, C, t = upload(d, "bf16")
    w = S.dloss_weights(124, N)
    loss, lse, dE, dC = sharded.forward_backward(E, C, t, bounds, II, eps,
                                                 dloss=torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    rl, rlse = oracle.forward(d["E"], d["C"], d["targets"], II)
    rE, rC, _ = oracle.backward(d["E"], d["C"], d["targets"], w, II, filter_eps=0.0)
    e_loss = np.abs(loss.cpu().numpy() - rl).max()
    e_dE, e_dC = rel(dE.cpu().numpy(), rE), rel(dC.cpu().numpy(), rC)
    log(f"[sharded chunks eps={eps}] loss {e_loss:.2e} dE {e_dE:.2e} dC {e_dC:.2e}")
    assert e_loss <= LOSS_TOL
    assert np.abs(lse.cpu().numpy() - rlse).max() <= LOSS_TOL
    assert e_dE <= GRAD_TOL and e_dC <= GRAD_TOL
    if eps == 0.0:
        assert row_err(dC.cpu().numpy(), rC) <= ROW_TOL


def test_sharded_equals_unsharded_closely():
    """Shards of whole 64-row blocks: same filter blocks as the unsharded call, so the results
    differ only by the rounding of the LSE merge."""
    N, D, V = 512, 128, 4096
    d = S.small_case(N, D, V, "bf16", 122, 3.0, 1.1, 0.0)
    E, C, t = upload(d, "bf16")
    b = sharded.shard_bounds(V, 4)
    assert b == [0, 1024, 2048, 3072, 4096]
    loss, lse, dE, dC = sharded.forward_backward(E, C, t, b, II, EPS)
    l1, lse1 = cce.cce_forward(E, C, t, II)
    dE1, dC1 = cce.cce_backward(torch.ones(N, device=DEV), E, C, t, lse1, II, EPS)
    torch.cuda.synchronize()
    assert (loss - l1).abs().max().item() <= 1e-5
    assert (lse - lse1).abs().max().item() <= 1e-5
    assert rel(dE.cpu().numpy(), dE1.cpu().numpy().astype(np.float64)) <= 1e-4
    assert rel(dC.cpu().numpy(), dC1.cpu().numpy().astype(np.float64)) <= 1e-4


def test_merge_flags_targets_outside_the_vocabulary():
    N, D, V = 64, 64, 640
    d = S.small_case(N, D, V, "bf16", 123, 3.0, None, 0.0)
    d["targets"][7] = V + 5
    E, C, t = upload(d, "bf16")
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    loss, lse, dE, dC = sharded.forward_backward(E, C, t, [0, 320, 640], II, 0.0, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    ln = loss.cpu().numpy()
    assert np.isnan(ln[7]) and np.all(np.isfinite(np.delete(ln, 7)))
