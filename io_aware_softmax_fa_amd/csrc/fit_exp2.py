#!/usr/bin/env python3
"""Minimax polynomial for 2^f on [-1/2, 1/2] (relative error), for the
software exp2 of the attention forward's optional FMA-pipe variant.

The software exponential of the FA4 walkthrough (section 3.1.3) splits
x = n + f with n = round(x) (a Cody-Waite style split: here one step, since
n is exact and f = x - n is computed without rounding error for |x| < 2^22),
evaluates 2^f with a short polynomial in Horner form on FMAs, and scales by
2^n. This script fits that polynomial itself: a Remez exchange on the
relative error |p(f) / 2^f - 1| over [-1/2, 1/2], in float64, with the
coefficients then rounded to float32 and the error re-measured in float32
Horner evaluation on a dense grid.

    python fit_exp2.py [degree]      (default 3)

prints the float32 coefficients (c0 + c1 f + c2 f^2 + ...) as C literals and
the maximum relative error before and after rounding them.
"""
from __future__ import annotations

import sys

import numpy as np

LO, HI = -0.5, 0.5


def remez(deg: int, iters: int = 40):
    """Coefficients (low order first) minimising max |p(f) 2^-f - 1| on [LO, HI]."""
    n = deg + 2                                   # alternation points
    k = np.arange(n)
    xs = 0.5 * (LO + HI) + 0.5 * (HI - LO) * np.cos(np.pi * (n - 1 - k) / (n - 1))  # Chebyshev
    grid = np.linspace(LO, HI, 200001)
    c = None
    for _ in range(iters):
        # solve p(x_i) - 2^x_i * (1 + (-1)^i E) = 0  ->  p(x_i) - (-1)^i E 2^x_i = 2^x_i
        A = np.zeros((n, n))
        for j in range(deg + 1):
            A[:, j] = xs ** j
        A[:, -1] = -((-1.0) ** k) * np.exp2(xs)
        sol = np.linalg.solve(A, np.exp2(xs))
        c = sol[:-1]
        err = np.polyval(c[::-1], grid) / np.exp2(grid) - 1.0
        # new alternation set: the extremum of each sign run of the error
        sgn = np.sign(err)
        edges = np.flatnonzero(np.diff(sgn) != 0)
        bounds = np.concatenate(([0], edges + 1, [len(grid)]))
        ext = [b0 + int(np.argmax(np.abs(err[b0:b1]))) for b0, b1 in zip(bounds[:-1], bounds[1:])]
        if len(ext) < n:
            break
        # keep the n largest consecutive extrema
        while len(ext) > n:
            ext.pop(0 if abs(err[ext[0]]) < abs(err[ext[-1]]) else -1)
        new = grid[ext]
        if np.allclose(new, xs, atol=1e-12):
            break
        xs = new
    return c


def horner_f32(c32: np.ndarray, f: np.ndarray) -> np.ndarray:
    acc = np.full_like(f, c32[-1], dtype=np.float32)
    for cj in c32[-2::-1]:
        acc = (acc * f + cj).astype(np.float32)   # the kernel fuses this (one rounding); an upper bound
    return acc


def main(deg: int = 3):
    c = remez(deg)
    grid = np.linspace(LO, HI, 2000001)
    e64 = np.max(np.abs(np.polyval(c[::-1], grid) / np.exp2(grid) - 1.0))
    c32 = c.astype(np.float32)
    g32 = grid.astype(np.float32)
    e32 = np.max(np.abs(horner_f32(c32, g32).astype(np.float64) / np.exp2(g32.astype(np.float64)) - 1))
    print(f"degree {deg} minimax for 2^f on [{LO}, {HI}], relative error")
    for j, cj in enumerate(c32):
        print(f"  c{j} = {float(cj):.9e}f   (float64 {c[j]:.17e})")
    print(f"max relative error: {e64:.3e} (float64 coefficients), {e32:.3e} (float32 Horner)")
    return c32, e64, e32


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 3)
