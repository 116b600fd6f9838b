"""Tolerance used wherever floating point results are compared.

Elementwise |a - b| <= rtol * (|b| + rms(b)): relative to each reference element, plus a
floor of rtol times the reference's root-mean-square so that elements that cancel to
nearly zero are judged on the scale of the data.  rtol is 1e-2 for bf16 outputs and 1e-5
for fp32 outputs.
"""

import numpy as np

RTOL_BF16 = 1e-2
RTOL_FP32 = 1e-5


def assert_close(actual, ref, rtol):
    a = np.asarray(actual, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    rms = float(np.sqrt(np.mean(b * b))) if b.size else 0.0
    err = np.abs(a - b)
    bound = rtol * (np.abs(b) + rms)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} of {b.size} elements outside rtol={rtol}; "
                             f"first at {idx.tolist()}: {a[tuple(idx[0])]} vs {b[tuple(idx[0])]}")
