"""The two block layouts and the blockwise conversion between them (oracle side).

e3nn-course Lesson 12a, section 21.3 ("Data layouts in cuEquivariance and
e3nn"): a block of multiplicity m and irrep dimension 2l+1 is stored either
as an (m, 2l+1) array (``mul_ir``, multiplicity first) or as a (2l+1, m)
array (``ir_mul``, irrep component first).  The cuequivariance-torch skill
document ("Layouts and weights") adds that conversion is done per block,
never as one reshape of the whole feature vector.
"""

import numpy as np

MUL_IR = "mul_ir"
IR_MUL = "ir_mul"


def split_blocks(x, blocks, layout):
    """Split the last axis of ``x`` (shape [..., dim]) into per-block arrays
    of shape [..., 2l+1, mul] (component axis first, whatever the layout)."""
    out = []
    off = 0
    for mul, l, _ in blocks:
        d = 2 * l + 1
        seg = x[..., off:off + mul * d]
        if layout == MUL_IR:
            seg = seg.reshape(seg.shape[:-1] + (mul, d))
            seg = np.swapaxes(seg, -1, -2)
        elif layout == IR_MUL:
            seg = seg.reshape(seg.shape[:-1] + (d, mul))
        else:
            raise ValueError(f"unknown layout {layout!r}")
        out.append(seg)
        off += mul * d
    return out


def join_blocks(parts, layout):
    """Inverse of :func:`split_blocks`: per-block [..., 2l+1, mul] arrays to
    one [..., dim] array in the given layout."""
    flat = []
    for seg in parts:
        if layout == MUL_IR:
            seg = np.swapaxes(seg, -1, -2)
        elif layout != IR_MUL:
            raise ValueError(f"unknown layout {layout!r}")
        flat.append(seg.reshape(seg.shape[:-2] + (-1,)))
    return np.concatenate(flat, axis=-1)


def transpose(x, blocks, source, target):
    """Blockwise layout conversion (the TransposeIrrepsLayout of the skill
    document, "Linear: layout conversion and rotations")."""
    return join_blocks(split_blocks(x, blocks, source), target)
