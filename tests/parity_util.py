"""Row-chunked comparison of a GPU result with the fp64 oracle.

SGMV's rows are independent (every row's update uses only its own x, y and adapter), so
the oracle evaluated on blocks of rows gives exactly the rows of the whole batch; a full
compare of a large batch then needs only one block of float64 values at a time.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

ATOL = 1e-2
RTOL = 1e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def compare_all_rows(outputs, n: int, ref_rows, dtype: str, what: str, block: int = 256):
    """Compare every element of each GPU output with the oracle, ``block`` rows at a time.

    ``outputs`` maps a label to the GPU result in storage format (numpy float16 / uint16
    bits, [n, h_out]); ``ref_rows(rows)`` returns the oracle's float64 rows.  Each block of
    the oracle serves every output.  Asserts |y - y_ref| <= ATOL + RTOL |y_ref| everywhere.
    """
    worst = {k: 0.0 for k in outputs}
    maxerr = {k: 0.0 for k in outputs}
    bad = {k: 0 for k in outputs}
    for r0 in range(0, n, block):
        rows = np.arange(r0, min(n, r0 + block))
        ref = ref_rows(rows)
        tol = ATOL + RTOL * np.abs(ref)
        for k, out in outputs.items():
            err = np.abs(oracle.decode(out[rows], dtype) - ref)
            worst[k] = max(worst[k], float(np.max(err / tol)))
            maxerr[k] = max(maxerr[k], float(err.max()))
            bad[k] += int((err > tol).sum())
    for k in outputs:
        say(f"{what} [{k}]: all {n} rows, max|err| {maxerr[k]:.3e}, worst err/tol {worst[k]:.3f}")
    for k in outputs:
        assert bad[k] == 0, f"{what} [{k}]: {bad[k]} elements outside tolerance"
