"""Seeded random cases through the C ABI against the oracle: shapes (N up to 40000, so several
backward token blocks; V up to 30000, so several vocabulary chunks), both input dtypes, filter
thresholds 0, 2^-12 and 1e-3, logit spreads 1 to 8, Zipf or uniform targets, ignored rows, the
forward's tile maxima on or off, fp32 or bf16 gradients, per-token or scalar dloss, whole
256-row tiles of C pushed far below the other logits (tiles the maxima prove negligible), and
the opt-in entry floor.

Criteria per case: loss and LSE to 2e-3; dE and dC to 1e-2 relative Frobenius error of the
oracle with the same threshold, plus an absolute allowance for the fp32 resolution of a target
entry p_t - 1 (about 2^-22 max(1, |lse|) per token, carried by C_t into dE and by E_n into dC),
which matters only when near-certain tokens make up the whole gradient; the block count and,
up to borderline blocks, the skip count of the oracle; with a threshold at or below 2^-12 and
where the oracle's own filter stays within 1e-3 of the unfiltered gradient (a peaked softmax),
dE and dC within 1e-2 of the unfiltered oracle too."""
import math

import numpy as np
import pytest
import torch

import cce_synth as S
import linear_cross_entropy_cce_amd as cce
import oracle
from gpu_helpers import DEV, GRAD_TOL, II, LOSS_TOL, borderline_blocks, log, rel

pytestmark = pytest.mark.gpu

N_CASES = 300
GROUPS = 6


def draw(seed):
    g = np.random.default_rng(seed)
    dtype = "bf16" if g.random() < 0.75 else "f32"
    D = int(8 * g.integers(1, 65)) if dtype == "bf16" else int(4 * g.integers(1, 129))
    V = int(round(math.exp(g.uniform(0, math.log(30000)))))
    N = int(round(math.exp(g.uniform(0, math.log(40000)))))
    while N * V * D > 3e9 and N > 1:
        N //= 2
    return dict(seed=seed, dtype=dtype, N=N, D=D, V=V,
                eps=float(g.choice([0.0, 2.0 ** -12, 1e-3])),
                c_scale=float(g.choice([1.0, 3.0, 8.0])), zipf=[None, 1.1][int(g.integers(0, 2))],
                ign=float(g.choice([0.0, 0.2])), tmax=bool(g.integers(0, 2)),
                gdt=["f32", "bf16"][int(g.integers(0, 2))], scalar=bool(g.random() < 0.2),
                far=float(g.choice([0.0, 0.0, 0.3, 0.7])),
                floor=float(g.choice([0.0, 0.0, 0.0, 1e-6, 1e-4])))


def far_tiles(d, c):
    """Pushes a random fraction c["far"] of C's 256-row tiles about 32 below every other logit
    (E[:, 0] = 8, C[v, 0] = -4 there) and moves the targets out of them."""
    g = np.random.default_rng(c["seed"] + 7)
    V = c["V"]
    far = np.nonzero(g.random(-(-V // 256)) < c["far"])[0]
    if len(far) == 0:
        return d
    E, C, tg = d["E"].copy(), d["C"].copy(), d["targets"].copy()
    E[:, 0] = 8.0
    rows = np.concatenate([np.arange(v * 256, min(V, v * 256 + 256)) for v in far])
    C[rows, 0] = -4.0
    if c["dtype"] == "bf16":
        E, C = S.bf16_round(E), S.bf16_round(C)
    near = np.setdiff1d(np.arange(V), rows)
    bad = (tg >= 0) & np.isin(tg, rows)
    tg[bad] = g.choice(near, size=int(bad.sum())) if len(near) else II
    return {"E": E, "C": C, "targets": tg}


def run_case(c):
    d = S.small_case(c["N"], c["D"], c["V"], c["dtype"], c["seed"], c["c_scale"], c["zipf"],
                     c["ign"])
    if c["far"] > 0:
        d = far_tiles(d, c)
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    E = torch.from_numpy(d["E"]).to(DEV, tdt)
    C = torch.from_numpy(d["C"]).to(DEV, tdt)
    t = torch.from_numpy(d["targets"]).to(DEV)
    N = c["N"]
    if c["scalar"]:
        w = np.full(N, 0.7, np.float32)
        dl = torch.tensor([0.7], device=DEV) if N != 1 else torch.from_numpy(w).to(DEV)
    else:
        w = S.dloss_weights(c["seed"], N)
        dl = torch.from_numpy(w).to(DEV)
    tm = cce.tile_max_buffer(E, C) if c["tmax"] else None
    loss, lse = cce.cce_forward(E, C, t, II, tile_max=tm)
    st = torch.zeros(2, dtype=torch.int64, device=DEV)
    gdt = torch.bfloat16 if c["gdt"] == "bf16" else torch.float32
    dE, dC = cce.cce_backward(dl, E, C, t, lse, II, c["eps"], tile_max=tm, grad_dtype=gdt,
                              skip_stats=st, entry_floor=c["floor"])
    torch.cuda.synchronize()
    gl, gs = loss.cpu().numpy(), lse.cpu().numpy()
    gE, gC = dE.float().cpu().numpy(), dC.float().cpu().numpy()
    tg = d["targets"]
    rl, rs = oracle.forward(d["E"], d["C"], tg, II)
    rE, rC, (sk, tot) = oracle.backward(d["E"], d["C"], tg, w, II, filter_eps=c["eps"],
                                        entry_floor=c["floor"])
    fail = []
    if np.abs(gl - rl).max() > LOSS_TOL or np.abs(gs - rs).max() > LOSS_TOL:
        fail.append("loss/lse")
    if not (np.all(gl[tg == II] == 0.0) and np.all(gE[tg == II] == 0.0)):
        fail.append("ignored rows")
    delta = np.where(tg != II, w * 2.0 ** -22 * np.maximum(1.0, np.abs(rs)), 0.0)
    cmax = float(np.linalg.norm(d["C"], axis=1).max())
    allow_e = float(np.sqrt(np.sum((2.0 * delta * cmax) ** 2)))
    allow_c = float(np.sum(2.0 * delta * np.linalg.norm(d["E"], axis=1)))
    if np.linalg.norm(gE - rE) > GRAD_TOL * np.linalg.norm(rE) + allow_e:
        fail.append(f"dE {rel(gE, rE):.2e}")
    if np.linalg.norm(gC - rC) > GRAD_TOL * np.linalg.norm(rC) + allow_c:
        fail.append(f"dC {rel(gC, rC):.2e}")
    if int(st[1]) != tot:
        fail.append("block count")
    if int(st[0]) != sk and abs(int(st[0]) - sk) > borderline_blocks(d["E"], d["C"], tg,
                                                                      c["eps"]):
        fail.append(f"skipped {int(st[0])} vs {sk}")
    if 0 < c["eps"] <= 2.0 ** -12:
        uE, uC, _ = oracle.backward(d["E"], d["C"], tg, w, II)
        if max(rel(rE, uE), rel(rC, uC)) <= 1e-3 and max(rel(gE, uE), rel(gC, uC)) > GRAD_TOL:
            fail.append(f"vs unfiltered dE {rel(gE, uE):.2e} dC {rel(gC, uC):.2e}")
    return fail


@pytest.mark.parametrize("group", range(GROUPS))
def test_random_cases_match_the_oracle(group):
    per = N_CASES // GROUPS
    seeds = range(20000 + group * per, 20000 + (group + 1) * per)
    for s in seeds:
        c = draw(s)
        fail = run_case(c)
        assert not fail, (c, fail)
    log(f"[fuzz group {group}] seeds {seeds.start}..{seeds.stop - 1}: {per} cases match")
