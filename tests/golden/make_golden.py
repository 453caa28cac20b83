"""Write the stored expected values of the full-size parity tests.

Calls only the fp64 CPU oracle (oracle/) on the seeded workloads; nothing here
comes from the GPU path.  For each full-size configuration it stores:

  checksum      sha256 of the generated (H, W, labels): the GPU test
                regenerates the inputs and must see the same bytes
  n_valid       number of valid rows
  loss_sum      sum of the per-row losses (full fp64 forward)
  loss_valid    per-row loss of every valid row, in valid-index order (fp64)
  lse_valid     per-row logsumexp of every valid row, same order (fp64)
  vocab_ids     sampled vocabulary rows (frequent labels, the ragged last
                tile, random ids)
  dW_rows       dW[vocab_ids] for the mean loss (needs the logsumexp of every
                valid row, hence the full forward)

Per-row dH is cheap and is recomputed live by the test on sampled rows.

Usage: python tests/golden/make_golden.py [config ...]   (default 2 3 4 5)
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def vocab_sample(V: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 3, 7, 100, 1000, V // 2, V - 257, V - 2, V - 1]
    extra = rng.choice(V, 5, replace=False)
    return np.unique(np.array(fixed + extra.tolist(), dtype=np.int64))


def make(cid: int) -> None:
    t0 = time.time()
    wl = workloads.CONFIGS[cid]
    H, W, y = workloads.generate(cid)
    cs = workloads.checksum(H, W, y)
    f = oracle.forward(H, W, y, workloads.IGNORE_INDEX)
    t1 = time.time()
    vid = vocab_sample(wl.V, 7000 + cid)
    w = 1.0 / f.valid_count
    dW = oracle.rows_dW(H, W, y, f.valid_idx, f.lse[f.valid_idx], vid, w)
    out = os.path.join(HERE, f"full_config{cid}.npz")
    np.savez_compressed(out, checksum=np.array(cs), n_valid=np.array(f.valid_count),
                        loss_sum=np.array(f.loss_sum), vocab_ids=vid,
                        loss_valid=f.loss[f.valid_idx], lse_valid=f.lse[f.valid_idx],
                        dW_rows=dW.astype(np.float32))
    print(f"config {cid}: n_valid {f.valid_count} mean loss {f.loss_mean:.6f} "
          f"(forward {t1 - t0:.0f} s, total {time.time() - t0:.0f} s) -> {out}", flush=True)


if __name__ == "__main__":
    for c in [int(a) for a in sys.argv[1:]] or [2, 3, 4, 5]:
        make(c)
