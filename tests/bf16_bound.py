"""The parity bound shared by the GPU tests whose inputs give rows that see
only a few keys.

The bar is max-abs <= 1e-2 and mean-abs <= 1e-3 against the fp64 oracle,
with one derived exception: an output whose exact value has |O| >= 2 may be
off by one bf16 spacing of that value (2^-6 on [2, 4)).  Two roundings that
the method makes set that bound.  P is rounded to bf16 before P.V, which
re-weights the visible V rows by up to 2^-9 relative, so O moves by up to
2^-9 * max|v - O| before its own rounding.  O is then rounded to bf16, which
adds up to half a spacing.  On a row that sees only a few keys, with |O| in
[2, 4), the sum can pass 1e-2 (a 2-key row with |v - O| ~ 3 gives about
0.006 + 0.0078).  Below |O| = 2 one spacing is under 1e-2 and the usual bar
holds unchanged.
"""

import numpy as np

MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def bf16_spacing(x):
    """Distance between adjacent bf16 values at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)


def check(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = np.maximum(MAX_ABS, np.where(np.abs(want) >= 2.0, bf16_spacing(want), 0.0))
    mean = float(err.mean()) if err.size else 0.0
    over = int((err > MAX_ABS).sum())
    worst = float((err / bound).max(initial=0.0))
    print(f"  {what}: max_abs={err.max(initial=0):.3e} mean_abs={mean:.3e} "
          f"above 1e-2: {over} (worst {worst:.2f} of the bound)", flush=True)
    assert mean <= MEAN_ABS, f"{what}: mean {mean}"
    assert np.all(err <= bound), f"{what}: max {err.max()} at {np.argmax(err)}"
