"""Write the oracle's scale choices for the protocol samples of configs 1, 3 and 4.

The pages check their solver against exhaustive FP16 enumeration ("Verification" in the CliffQuant
README and in the W4A16-G128 model card); the oracle is that enumeration.  The synthetic configs
ask for the oracle on all of config 1 (86,016 groups), on all of config 3 or a seeded 65,536-group
subsample, and on a seeded 16,384-group sample of config 4.  Their brute force over all 31,743
scales takes minutes on a host, so this script runs it once and stores, per group and policy
(minimax, pooled), the winning bit pattern and whether the oracle's runner-up gap exceeds 1e-9
(where the GPU must return the same bits); every other value the GPU tests need (objectives at a
given scale, codes) the oracle recomputes in a moment.

Inputs come from `workloads` (seeded generators holding none of the method's arithmetic); values
come only from `oracle`.  Run from the repository root: python tests/golden/make_oracle_fixtures.py
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
GAP = 1e-9
SAMPLE_SALT = 7


def config1_groups():
    ws, ds, ps = [], [], []
    for m in range(len(W.config(1).matrices)):
        w, d, p = W.matrix_groups(*W.make_matrix(1, m))
        ws.append(w)
        ds.append(d)
        ps.append(p)
    return ws, ds, ps


def solve_and_store(name, parts, extra=None):
    t = time.time()
    out = {k: [] for k in ("mm_bits", "mm_sure", "pl_bits", "pl_sure")}
    for w, d, p in parts:
        sol = oracle.solve(w, d, p, n_threads=os.cpu_count() or 1)
        out["mm_bits"].append(sol.mm_bits.astype(np.uint16))
        out["mm_sure"].append(sol.mm_gap > GAP)
        out["pl_bits"].append(sol.pl_bits.astype(np.uint16))
        out["pl_sure"].append(sol.pl_gap > GAP)
    arrs = {k: np.concatenate(v) for k, v in out.items()}
    arrs["mm_sure"] = np.packbits(arrs["mm_sure"])
    arrs["pl_sure"] = np.packbits(arrs["pl_sure"])
    if extra:
        arrs.update(extra)
    path = os.path.join(HERE, name)
    np.savez_compressed(path, **arrs)
    print(f"{name}: {arrs['mm_bits'].size} groups in {time.time() - t:.0f} s", flush=True)


def main():
    ws, ds, ps = config1_groups()
    solve_and_store("oracle_config1_all.npz", list(zip(ws, ds, ps)))
    gids3 = W.sample_groups(3, 65536, salt=SAMPLE_SALT)
    w3, d3, _, _ = W.make_groups(3, gids3)
    solve_and_store("oracle_config3_65536.npz", [(w3, d3, w3.shape[0])], {"gids": gids3})
    gids4 = W.sample_groups(4, 16384, salt=SAMPLE_SALT)
    w4, d4, _ = W.gather_matrix_groups(4, gids4)
    solve_and_store("oracle_config4_16384.npz", [(w4, d4, w4.shape[0])], {"gids": gids4})


if __name__ == "__main__":
    main()
