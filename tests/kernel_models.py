"""White-box models of the kernels' binary32 arithmetic, for the tests.

These restate what a kernel computes in binary32 (numpy float32 rounds to
nearest even like the kernels' VALU), so that a test can hold the kernel to
its own arithmetic where the definition alone cannot decide (degenerate
groups) and can check the error bounds the kernel relies on.  They are not
the oracle: the oracle computes the definition in float64.
"""
import numpy as np

import oracle


def butterfly_model(rows, seed, D):
    """White-box model of the in-register butterfly that 8-bit encodes run
    by default, on rows of values exact in the storage type
    (float64 [N, D]): the signed row in binary32 (exact), then log2 D
    stages of binary32 additions and subtractions in the kernel's order
    (element j of each block of 2h takes a + b, element j + h takes a - b).
    numpy's float32 arithmetic rounds to nearest even like the kernel's, so
    the model gives the kernel's unnormalized u to the bit (float64 [N, D])."""
    x = rows.astype(np.float32) * oracle.sign_vector(seed, D).astype(np.float32)
    y = x.reshape(len(x), D)
    h = 1
    while h < D:
        blk = y.reshape(len(y), D // (2 * h), 2, h)
        a, b = blk[:, :, 0, :], blk[:, :, 1, :]
        y = np.stack([a + b, a - b], axis=2).reshape(len(y), D)
        h *= 2
    return y.astype(np.float64)
