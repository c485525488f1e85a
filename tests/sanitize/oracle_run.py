"""Runs every oracle function on small inputs against a sanitizer build of the
oracle (path in argv[1]), with AddressSanitizer preloaded by the caller.
numpy only (no torch), so the sanitizer sees the oracle's own memory use.
Cases: a gated layer with skewed rows (backup rows in the hybrid), tiles
holding more nonzeros than the TwELL width, a backup capacity that is too
small, and T = 1. Prints "oracle_run ok"."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle  # noqa: E402


def layer(rng, T, dm, dff):
    x = rng.standard_normal((T, dm))
    x[:, 0] = 1.0
    x[: T // 4, 0] = 3.0  # a quarter of the rows far denser than the rest
    wg = rng.standard_normal((dff, dm)) / np.sqrt(dm)
    wg[:, 0] = -1.5
    wu = rng.standard_normal((dff, dm)) / np.sqrt(dm)
    wd = rng.standard_normal((dff, dm)) / np.sqrt(dff)
    dy = rng.standard_normal((T, dm))
    return x, wg, wu, wd, dy


def main():
    oracle.load(sys.argv[1])
    oracle.set_num_threads(2)
    rng = np.random.default_rng(7)
    for T, dm, dff, W, K, max_ovf in ((37, 64, 256, 128, 16, 40), (1, 64, 384, 4, 8, 1),
                                      (20, 128, 256, 2, 6, 20)):
        x, wg, wu, wd, dy = layer(rng, T, dm, dff)
        g = oracle.gate(x, wg)
        tw = oracle.twell_pack(g, 128, W)
        y_tw = oracle.ffn_twell(x, tw, wu, wd)
        if W == 128:
            assert np.array_equal(y_tw, oracle.ffn_dense(x, wg, wu, wd))
        hy = oracle.to_hybrid(tw, K, max_ovf)
        assert not hy["capacity_exceeded"]
        y_hy = oracle.ffn_hybrid(x, hy, wu, wd)
        assert np.allclose(y_hy, y_tw, rtol=1e-12, atol=1e-12)
        oracle.bwd_hybrid(x, dy, hy, wg, wu, wd, l1=2e-5)
        oracle.bwd_dense(x, dy, wg, wu, wd, l1=2e-5)
        small = oracle.to_hybrid(tw, K, 0)
        assert small["capacity_exceeded"] == (small["n_ovf"] > 0)
    print("oracle_run ok")


if __name__ == "__main__":
    main()
