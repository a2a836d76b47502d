"""Write the Lloyd codebooks of the benchmark workloads with the CPU oracle.

Runs only oracle/ (and the seeded input generator) -- never the GPU library.  The GPU test
compares qamw_codebook_train against these files bit for bit.
Usage: python tests/golden/make_codebooks.py [name ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth_inputs as synth  # noqa: E402

# name: (config index, points stream id, number of points, bits, iterations)
JOBS = {
    "cb_cfg0_k256": (0, synth.SID_POINTS, 1 << 16, 8, 20),
    "cb_cfg1_k2048": (1, synth.SID_POINTS, 1 << 20, 11, 20),
    "cb_cfg3_k128": (3, synth.SID_POINTS_K128, 1 << 20, 7, 20),
    "cb_cfg2_k2048": (2, synth.SID_POINTS, 1 << 22, 11, 50),
}


def main(names):
    orc = oracle.Oracle(oracle.build())
    for name in names:
        cfg_i, sid, n, bits, iters = JOBS[name]
        seed = synth.config(cfg_i).seed
        pts = synth.points(seed, sid, n)
        t = time.time()
        cb, trace, st = orc.lloyd(pts, bits, iters)
        assert st == 0
        np.savez(os.path.join(HERE, name + ".npz"), codebook=cb, trace=trace,
                 meta=np.array([cfg_i, sid, n, bits, iters], dtype=np.int64))
        print("%s: %d points, K=%d, %d iterations, %.1f s, final MSE %.6f" %
              (name, n, 1 << bits, iters, time.time() - t, trace[-1] / 2**32 / n), flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(JOBS))
