"""Write oracle_tiny_regression.npz (calls only oracle/ and seeded_inputs/)."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import seeded_inputs as si  # noqa: E402


def main():
    w = si.WORKLOADS["tiny_fwd_f32"]
    x = si.full_inputs(w)
    N = w.B * w.H
    r = lambda a: a.reshape(N, *a.shape[2:])  # noqa: E731
    meta = np.broadcast_to(x["meta_k"][None], (w.B,) + x["meta_k"].shape).reshape(N, w.n_meta, w.d)
    out = oracle.lizard_fwd(r(x["q"]), r(x["k"]), r(x["v"]), r(x["log_g"]), meta, w.window, w.alpha)
    np.savez_compressed(os.path.join(HERE, "oracle_tiny_regression.npz"),
                        y=out["y"][:, ::7], y_anchor=out["y_anchor"][:, ::7], lse=out["lse"], state=out["state"])


if __name__ == "__main__":
    main()
