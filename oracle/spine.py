"""Row-scaled int8 dequantisation of a dense weight matrix, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Deltafin README, "Techniques / Compute": the dense (non-expert) weights are
kept as int8 with one scale per row, and a small GPU kernel fuses the int8
to fp32 conversion, the multiplication by the row's scale and the copy into
the fp32 weight buffer, bit-exact against the unfused path.  The readings
here: q is int8 [R][C] row-major, scale is float32 [R], and
out[r][c] = fp32(q[r][c] * scale[r]), one rounding of the exact product.
"""

import numpy as np


def int8_row_dequant(q, scale):
    """out float32 [R, C] = q[r, c] * scale[r], rounded once to float32.

    The product of an int8 (8 significant bits) and a float32 (24) is exact
    in float64 (53), so the cast to float32 is the single rounding.
    """
    q = np.asarray(q, dtype=np.int8)
    scale = np.asarray(scale, dtype=np.float32)
    if q.ndim != 2 or scale.shape != (q.shape[0],):
        raise ValueError("q must be [R, C] and scale [R]")
    with np.errstate(invalid="ignore", over="ignore"):
        exact = q.astype(np.float64) * scale.astype(np.float64)[:, None]
        return exact.astype(np.float32)
