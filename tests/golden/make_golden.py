"""Writes oracle_small_case.json from the oracle alone (regression fixture).

Run from the repository root:  python tests/golden/make_golden.py"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import cce_synth as S  # noqa: E402
import oracle  # noqa: E402


def main():
    d = S.small_case(N=12, D=16, V=40, dtype="bf16", seed=77, c_scale=8.0, zipf_s=1.1,
                     ignore_frac=0.25)
    w = S.dloss_weights(77, 12)
    loss, lse = oracle.forward(d["E"], d["C"], d["targets"], S.IGNORE_INDEX)
    dE, dC, (sk, tot) = oracle.backward(d["E"], d["C"], d["targets"], w, S.IGNORE_INDEX,
                                        filter_eps=0.01, block_n=2, block_v=4, entry_floor=0.0)
    out = {"case": {"N": 12, "D": 16, "V": 40, "dtype": "bf16", "seed": 77, "c_scale": 8.0,
                    "zipf_s": 1.1, "ignore_frac": 0.25, "dloss_seed": 77, "filter_eps": 0.01,
                    "entry_floor": 0.0, "block_n": 2, "block_v": 4},
           "targets": d["targets"].tolist(), "loss": loss.tolist(), "lse": lse.tolist(),
           "dE_rowsum": dE.sum(axis=1).tolist(), "dC_rowsum": dC.sum(axis=1).tolist(),
           "skipped": sk, "total": tot}
    with open(os.path.join(HERE, "oracle_small_case.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
