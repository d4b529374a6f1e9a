"""The weight-streaming layout of the E4M3 weight codes, by its definition.

Byte b of lane 16 g + r (g < 4, r < 16) of half h (0, 1) of K block kb of the
16-row fragment f sits at offset ((f Kb + kb) 2 + h) 1024 + 16 (16 g + r) + b
and holds code wq[16 f + r, 128 kb + 32 g + 16 h + b] (Kb = Kp / 128): each
16-row x 128-byte block of the codes is 2 KB in the order the 16x16x128 MFMA's
lanes hold their operand bytes, and the blocks of one 16-row band follow each
other along K.
"""

import numpy as np


def stream_order(wq):
    """Row-major codes [Np, Kp] -> the stream layout, as an [Np, Kp] byte array:
    wq viewed as axes [f, r, kb, g, h, b], laid out in the order [f, kb, h, g, r, b]."""
    Np, Kp = wq.shape
    v = wq.reshape(Np // 16, 16, Kp // 128, 4, 2, 16).transpose(0, 2, 4, 3, 1, 5)
    return np.ascontiguousarray(v).reshape(Np, Kp)
