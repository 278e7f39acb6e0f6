"""Fit the bias column of the balanced prefill workload and store it.

The prefill workload (T = 8192 tokens, real shape) asks for near-balanced
expert loads: the busiest expert within 1.1x of the mean T*K/E = 256 rows.
Pure sampling noise leaves a max near 1.18x, so a per-expert fp32 bias column
b is fitted with the oracle's own routing:

    b <- b - eta * (load / mean - 1)      (repeated until max load <= target * mean)

starting from b = 0.  The result is written as fp32 bit patterns (hex), one
expert per line, to synth/prefill_bias_seed<seed>.txt, which the input
generators read.  Only this script (it calls nothing but oracle/ and synth/)
writes that file.

    python -m oracle.fit_prefill_bias --seed 0
"""
from __future__ import annotations

import argparse
import os

import numpy as np

from synth import gen
from .moe import LayerSpec, route


def loads(spec, x_bits, wr, b):
    ids, _ = route(spec, x_bits, wr, b)
    return np.bincount(ids.ravel(), minlength=spec.n_experts)


def fit(seed: int = 0, target: float = 1.05, eta: float = 0.1, max_iter: int = 400):
    w = gen.workload("prefill")
    spec = LayerSpec.of(w)
    x_bits, wr, _ = gen.router_inputs(w, seed, bias=np.zeros(w.n_experts, np.float32))
    mean = w.T * w.top_k / w.n_experts
    b = np.zeros(w.n_experts, np.float64)
    for it in range(max_iter):
        bf = b.astype(np.float32)
        ld = loads(spec, x_bits, wr, bf)
        ratio = ld.max() / mean
        if ratio <= target:
            return bf, it, ratio
        b = b - eta * (ld / mean - 1.0)
    raise RuntimeError(f"no fit within {max_iter} iterations (max/mean {ratio:.3f})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    b, it, ratio = fit(args.seed)
    path = gen.balanced_bias_path(args.seed)
    with open(path, "w") as f:
        f.write(f"# balanced prefill bias, seed {args.seed}: fp32 bit patterns, one per expert\n")
        f.write(f"# written by oracle/fit_prefill_bias.py after {it} iterations, max/mean {ratio:.4f}\n")
        for v in b.view(np.uint32):
            f.write(f"{int(v):08x}\n")
    print(f"wrote {path}: {it} iterations, max/mean {ratio:.4f}")


if __name__ == "__main__":
    main()
