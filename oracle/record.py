"""Expert record layout, parsed by the oracle itself.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Deltafin README, "Techniques / I/O and streaming" (coalesced expert fetch):
the six tensors of an expert sit contiguously, so one expert is one span of
bytes; the kimi-k3-in-c note (byte accounting) gives that span as
17,547,264 bytes.  The pages do not name the six tensors; the reading here is
{gate, up, down} x {packed E2M1 codes, E8M0 scales}, in this order:

    gate codes  [I][H/2]   gate scales [I][H/32]
    up codes    [I][H/2]   up scales   [I][H/32]
    down codes  [H][I/2]   down scales [H][I/32]

Rows are output features, the input (contraction) dimension is contiguous.
"""

import numpy as np

from .formats import mxfp4_dequant

GATE, UP, DOWN = 0, 1, 2


def matrix_bytes(rows, cols):
    """Bytes of one MXFP4 matrix: codes rows*cols/2 plus scales rows*cols/32."""
    if cols % 32:
        raise ValueError("input dimension must be a multiple of 32")
    return rows * cols // 2 + rows * cols // 32


def record_bytes(hidden, inter):
    """Bytes of one expert record (three MXFP4 matrices)."""
    return 2 * matrix_bytes(inter, hidden) + matrix_bytes(hidden, inter)


def _sections(hidden, inter):
    """(offset, shape) of the six tensors in record order."""
    out = []
    off = 0
    for rows, cols in ((inter, hidden), (inter, hidden), (hidden, inter)):
        codes = (rows, cols // 2)
        scales = (rows, cols // 32)
        out.append((off, codes))
        off += codes[0] * codes[1]
        out.append((off, scales))
        off += scales[0] * scales[1]
    return out


def split(rec, hidden, inter):
    """Views of the six tensors of one record (uint8 array of record_bytes)."""
    rec = np.asarray(rec, dtype=np.uint8).reshape(-1)
    if rec.size < record_bytes(hidden, inter):
        raise ValueError("record too short")
    views = []
    for off, shape in _sections(hidden, inter):
        n = shape[0] * shape[1]
        views.append(rec[off:off + n].reshape(shape))
    return views


def dequant_matrix(rec, hidden, inter, which):
    """float64 weights of one matrix of a record: gate/up [I,H], down [H,I]."""
    v = split(rec, hidden, inter)
    return mxfp4_dequant(v[2 * which], v[2 * which + 1])


def dequant_expert(rec, hidden, inter):
    """(Wg [I,H], Wu [I,H], Wd [H,I]) in float64."""
    return tuple(dequant_matrix(rec, hidden, inter, m) for m in (GATE, UP, DOWN))
