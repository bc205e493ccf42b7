"""Shared helpers of the GPU parity tests (upload, run through the C ABI, compare)."""
import numpy as np
import torch

import cce_synth as S
import linear_cross_entropy_cce_amd as cce
import oracle

DEV = "cuda:0"
II = S.IGNORE_INDEX
EPS = S.FILTER_EPS
LOSS_TOL = 2e-3      # per-token loss, absolute
GRAD_TOL = 1e-2      # dE, dC relative Frobenius
ROW_TOL = 5e-2       # dE, dC row by row: |d row| <= ROW_TOL (|ref row| + ROW_ATOL rms row norm)
ROW_ATOL = 1e-3


def log(msg):
    print(msg, flush=True)


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def upload(d, dtype):
    tdt = torch_dtype(dtype)
    return (torch.from_numpy(d["E"]).to(DEV, tdt), torch.from_numpy(d["C"]).to(DEV, tdt),
            torch.from_numpy(np.ascontiguousarray(d["targets"])).to(DEV))


def rel(a, b):
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(np.asarray(a, np.float64) - b)) / (nb if nb > 0 else 1.0)


def row_err(a, b):
    """Largest row error of a against the reference b, relative to the row's own norm plus
    ROW_ATOL times the root-mean-square row norm of b (so rows far below the typical size are
    held to an absolute bound): a wrong, missing or misplaced row of a gradient shows here even
    where the whole-matrix Frobenius error hides it."""
    n = len(b)
    if n == 0:
        return 0.0
    nb, d = np.empty(n), np.empty(n)
    for i in range(0, n, 8192):   # row chunks: no full-size float64 temporaries
        bi = np.asarray(b[i:i + 8192], np.float64)
        nb[i:i + 8192] = np.linalg.norm(bi, axis=1)
        d[i:i + 8192] = np.linalg.norm(np.asarray(a[i:i + 8192], np.float64) - bi, axis=1)
    rms = float(np.sqrt(np.mean(nb ** 2)))
    den = nb + ROW_ATOL * rms
    return float(np.max(np.where(den > 0, d / np.where(den > 0, den, 1.0), d)))


def gpu_run(d, dtype, w, eps, err=False, entry_floor=0.0):
    """Forward + backward through libcce; returns numpy results and the skip statistics."""
    E, C, t = upload(d, dtype)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    loss, lse = cce.cce_forward(E, C, t, II, err_flag=flag)
    stats = torch.full((2,), -1, dtype=torch.int64, device=DEV)
    dl = torch.from_numpy(np.asarray(w, np.float32)).to(DEV)
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, eps, entry_floor=entry_floor,
                              skip_stats=stats)
    torch.cuda.synchronize()
    out = dict(loss=loss.cpu().numpy(), lse=lse.cpu().numpy(), dE=dE.cpu().numpy(),
               dC=dC.cpu().numpy(), skipped=int(stats[0]), total=int(stats[1]),
               err=int(flag.item()))
    return out


def borderline_blocks(E, C, t, eps, bn=64, bv=64, rel_band=1e-3):
    """Blocks whose decision the rounding of fp32 vs fp64 may flip: no target inside and a
    block max of the softmax within rel_band of eps (computed from the oracle's values)."""
    if eps <= 0:
        return 0
    _, lse = oracle.forward(E, C, t, II)
    N, V = E.shape[0], C.shape[0]
    count = 0
    for n0 in range(0, N, bn):
        rows = np.arange(n0, min(N, n0 + bn))
        valid = t[rows] != II
        if not valid.any():
            continue
        P = np.exp(oracle.logits(E[rows[valid]], C) - lse[rows[valid], None])
        for v0 in range(0, V, bv):
            tv = t[rows[valid]]
            if ((tv >= v0) & (tv < v0 + bv)).any():
                continue
            m = P[:, v0:v0 + bv].max()
            if abs(m - eps) <= rel_band * eps:
                count += 1
    return count


def check_against_oracle(d, dtype, w, eps, name, grad_tol=GRAD_TOL, loss_tol=LOSS_TOL,
                         vs_unfiltered=True):
    """Element-by-element comparison with the oracle's result for the same filter threshold,
    as whole matrices (relative Frobenius error) and row by row (row_err, where no block is
    borderline); a filtered result must also stay within GRAD_TOL of the unfiltered oracle,
    the definition the filter approximates.  Only thresholds above the benchmarks' 2^-12 may
    opt out of that (vs_unfiltered=False)."""
    assert vs_unfiltered or eps > EPS
    log(f"[{name}] N={d['E'].shape[0]} D={d['E'].shape[1]} V={d['C'].shape[0]} {dtype} eps={eps}")
    g = gpu_run(d, dtype, w, eps)
    E, C, t = d["E"], d["C"], d["targets"]
    loss, lse = oracle.forward(E, C, t, II)
    dE, dC, (sk, tot) = oracle.backward(E, C, t, w, II, filter_eps=eps)
    assert np.abs(g["loss"] - loss).max() <= loss_tol, np.abs(g["loss"] - loss).max()
    assert np.abs(g["lse"] - lse).max() <= loss_tol
    assert np.all(g["loss"][t == II] == 0.0)
    assert rel(g["dE"], dE) <= grad_tol, rel(g["dE"], dE)
    assert rel(g["dC"], dC) <= grad_tol, rel(g["dC"], dC)
    assert np.all(g["dE"][t == II] == 0.0)
    assert g["total"] == tot
    border = borderline_blocks(E, C, t, eps)
    assert abs(g["skipped"] - sk) <= border, (g["skipped"], sk, border)
    rE, rC = row_err(g["dE"], dE), row_err(g["dC"], dC)
    if border == 0:   # the same blocks are skipped on both sides: rows compare one to one
        assert rE <= ROW_TOL and rC <= ROW_TOL, (rE, rC)
    u = ""
    if eps > 0 and vs_unfiltered:   # also within tolerance of the unfiltered oracle
        dE0, dC0, _ = oracle.backward(E, C, t, w, II)
        uE, uC = rel(g["dE"], dE0), rel(g["dC"], dC0)
        assert uE <= GRAD_TOL and uC <= GRAD_TOL, (uE, uC)
        u = f" vs unfiltered dE {uE:.2e} dC {uC:.2e}"
    log(f"[{name}] ok: loss {np.abs(g['loss'] - loss).max():.2e} dE {rel(g['dE'], dE):.2e} "
        f"dC {rel(g['dC'], dC):.2e} rows dE {rE:.2e} dC {rC:.2e}{u} "
        f"skipped {g['skipped']}/{g['total']} (oracle {sk})")
    return g
