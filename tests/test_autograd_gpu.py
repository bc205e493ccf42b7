"""torch.autograd integration (linear_cross_entropy): gradients through autograd against the
float64 oracle for each reduction, and a short fp32 training run of a classifier head whose
loss trajectory follows the oracle's step by step."""
import numpy as np
import pytest
import torch

import cce_synth as S
import oracle
from gpu_helpers import DEV, EPS, GRAD_TOL, II, LOSS_TOL, log, rel, upload
from linear_cross_entropy_cce_amd import LinearCrossEntropy, linear_cross_entropy

pytestmark = pytest.mark.gpu


def _leaf(x):
    return x.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_autograd_gradients_match_oracle(reduction):
    N, D, V = 300, 72, 1500
    d = S.small_case(N, D, V, "bf16", 101, 3.0, 1.1, 0.15)
    log(f"[autograd {reduction}] N={N} D={D} V={V}")
    E0, C0, t = upload(d, "bf16")
    E, C = _leaf(E0), _leaf(C0)
    out = linear_cross_entropy(E, C, t, II, EPS, reduction)
    if reduction == "none":
        up = S.dloss_weights(5, N)
        out.backward(torch.from_numpy(up).to(DEV))
        w = up.astype(np.float64)
    else:
        out.backward()
        n_valid = int((d["targets"] != II).sum())
        w = np.full(N, 1.0 / n_valid if reduction == "mean" else 1.0)
    torch.cuda.synchronize()
    assert E.grad.dtype == torch.bfloat16 and C.grad.dtype == torch.bfloat16
    loss, _ = oracle.forward(d["E"], d["C"], d["targets"], II)
    dE, dC, _ = oracle.backward(d["E"], d["C"], d["targets"], w, II, filter_eps=EPS)
    got = out.detach().float().cpu().numpy()
    if reduction == "none":
        assert np.abs(got - loss).max() <= LOSS_TOL
    elif reduction == "sum":
        assert abs(float(got) - loss.sum()) <= LOSS_TOL * N
    else:
        assert abs(float(got) - loss.sum() / n_valid) <= LOSS_TOL
    # bf16 gradients (libcce rounds its fp32 results once): 2^-9 relative on top of the
    # kernel's error
    assert rel(E.grad.float().cpu().numpy(), dE) <= GRAD_TOL
    assert rel(C.grad.float().cpu().numpy(), dC) <= GRAD_TOL


def test_mean_backward_runs_once():
    d = S.small_case(64, 64, 300, "bf16", 104, 3.0, 1.1, 0.0)
    E0, C0, t = upload(d, "bf16")
    C = _leaf(C0)
    loss = linear_cross_entropy(E0, C, t, II, EPS, "mean")
    loss.backward(retain_graph=True)
    with pytest.raises(RuntimeError, match="one backward"):
        loss.backward()


def test_module_and_partial_requires_grad():
    d = S.small_case(128, 64, 700, "bf16", 102, 3.0, 1.1, 0.0)
    E0, C0, t = upload(d, "bf16")
    C = _leaf(C0)
    loss = LinearCrossEntropy(reduction="sum")(E0, C, t)
    loss.backward()
    torch.cuda.synchronize()
    assert C.grad is not None and C.grad.shape == C0.shape
    _, dC, _ = oracle.backward(d["E"], d["C"], d["targets"], np.ones(128), II,
                               filter_eps=EPS)
    assert rel(C.grad.float().cpu().numpy(), dC) <= GRAD_TOL


def test_fp32_training_run_follows_the_oracle():
    """Plain SGD on a classifier head (C learned, E fixed), fp32 on both sides: the loss after
    every step matches the oracle's trajectory (the oracle takes the same steps in float64)."""
    N, D, V, lr, steps = 256, 64, 1000, 0.5, 12
    d = S.small_case(N, D, V, "f32", 103, 1.0, 1.1, 0.1)
    E0, C0, t = upload(d, "f32")
    C = torch.nn.Parameter(C0.clone())
    opt = torch.optim.SGD([C], lr=lr)
    Cr = d["C"].astype(np.float64)
    losses, ref = [], []
    for _ in range(steps):
        opt.zero_grad()
        loss = linear_cross_entropy(E0, C, t, II, 0.0, "mean")
        loss.backward()
        opt.step()
        losses.append(float(loss.item()))
        m, _, rC, _ = oracle.loss_mean(d["E"], Cr, d["targets"], II, 0.0)
        ref.append(m)
        Cr = Cr - lr * rC
    log(f"losses {losses[0]:.4f} -> {losses[-1]:.4f} (oracle {ref[0]:.4f} -> {ref[-1]:.4f})")
    assert losses[-1] < losses[0] - 0.05
    assert np.abs(np.array(losses) - np.array(ref)).max() <= 1e-3
