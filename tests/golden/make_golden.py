"""Writes the stored expected values under tests/golden/ from the oracle alone.

The pages print no worked numerical example for the spectral convolution, so
every stored value here comes from the fp64 oracle (oracle/) applied to the
seeded synthetic inputs; nothing is taken from the HIP library.

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from fft_spectral_convolution_amd.inputs import CONFIGS, make_inputs  # noqa: E402


def sample_indices(shape, count, seed):
    rng = np.random.default_rng(seed)
    return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(count)]


def main():
    cfg = CONFIGS["c1"]
    x, w = make_inputs(cfg, seed=0)
    out = oracle.spectral_conv2d_ref(x, w, cfg.mx, cfg.my)
    idx = sample_indices(out.shape, 64, 1234)
    path = os.path.join(HERE, "c1_seed0_out_samples.txt")
    with open(path, "w") as f:
        f.write("# oracle output of config c1 (2D, B=2, Cin=Cout=4, 32x32, modes 8x8, seed 0)\n")
        f.write("# written by tests/golden/make_golden.py from oracle/ only\n")
        f.write("# b o h w value\n")
        for i in idx:
            f.write("%d %d %d %d %.17g\n" % (i + (out[i],)))
    cfg = CONFIGS["c4"]
    # a small 1D case of the same recipe (the full c4 is sampled in the GPU tests)
    rng_cfg = cfg.__class__("c4s", "1d", 3, 5, 4, 1, 64, 1, 9, "normal")
    x, w = make_inputs(rng_cfg, seed=0)
    out = oracle.spectral_conv1d_ref(x, w, rng_cfg.my)
    idx = sample_indices(out.shape, 32, 99)
    path = os.path.join(HERE, "small1d_seed0_out_samples.txt")
    with open(path, "w") as f:
        f.write("# oracle output of a small 1D case (B=3, Cin=5, Cout=4, N=64, modes 9, normal x, seed 0)\n")
        f.write("# written by tests/golden/make_golden.py from oracle/ only\n")
        f.write("# b o n value\n")
        for i in idx:
            f.write("%d %d %d %.17g\n" % (i + (out[i],)))


if __name__ == "__main__":
    main()
