"""Pure-Python scalar restatement of the reduce-scatter and all-gather
placement, used only on tiny inputs to cross-check the C oracle's indexing.

Independent of the oracle: it walks ranks and rows with dictionaries and
Python lists and rounds each add to binary32 with numpy scalars.  Readings as
in the oracle: shard rows s = ceil(d0/R), +0.0 padding, fixed rank order.
"""
import numpy as np


def _f32(bits16):
    return np.uint32(int(bits16) << 16).view(np.float32)


def rs_brute(shapes, R, grads_bits):
    """grads_bits[q][p]: flat list/array of uint16.  Returns a dict
    (r, p) -> list of float32 (the shard, padded)."""
    out = {}
    for p, shp in enumerate(shapes):
        d0 = shp[0] if len(shp) else 1
        c = 1
        for d in shp[1:]:
            c *= d
        s = -(-d0 // R)
        for r in range(R):
            shard = []
            for row in range(r * s, r * s + s):
                for col in range(c):
                    if row < d0:
                        acc = _f32(grads_bits[0][p][row * c + col])
                        with np.errstate(over="ignore"):  # IEEE overflow to inf is the result
                            for q in range(1, R):
                                acc = np.float32(acc + _f32(grads_bits[q][p][row * c + col]))
                        shard.append(acc)
                    else:
                        shard.append(np.float32(0.0))
            out[(r, p)] = shard
    return out


def ag_brute(shapes, R, gathered_bits):
    """All-gather placement by rows: returns P lists of uint16 (d0*c each):
    row i of param p comes from slot i // s, row i % s of that slot's shard
    of p."""
    d0s, cs = [], []
    for shp in shapes:
        d0s.append(shp[0] if len(shp) else 1)
        c = 1
        for d in shp[1:]:
            c *= d
        cs.append(c)
    ms = [(-(-d0 // R)) * c for d0, c in zip(d0s, cs)]
    offs, S = [], 0
    for m in ms:
        offs.append(S)
        S += m
    out = []
    for p in range(len(shapes)):
        d0, c = d0s[p], cs[p]
        s = -(-d0 // R)
        full = []
        for row in range(d0):
            r, i = divmod(row, s)
            base = r * S + offs[p] + i * c
            full.extend(int(gathered_bits[base + k]) for k in range(c))
        out.append(full)
    return out
