"""The partial_out format of include/mla.h, written out with numpy for the
tests: fp16 values in the kernels' lane order, then one power-of-two descale
per (block, column quarter, head)."""
from __future__ import annotations

import numpy as np

N_HEADS, D_C = 128, 512
BLOCK_BYTES = N_HEADS * D_C * 2       # fp16 values of one (split, slot, token) block
DESC_BYTES = 4 * N_HEADS * 4          # its fp32 descales


def partial_bytes(num_splits, s_q):
    return num_splits * 2 * s_q * (BLOCK_BYTES + DESC_BYTES)


def descales(po):
    """[nb, 128, 512] -> [nb, 4 quarters, 128 heads]: 2^(e - 15) for the largest
    |value| m of the (quarter, head), m in [2^(e-1), 2^e); e >= -75."""
    m = np.abs(po).reshape(po.shape[0], N_HEADS, 4, 128).max(axis=3)
    e = np.frexp(m)[1]
    e = np.where(m > 0, np.maximum(e, -75), -75)
    return np.ldexp(1.0, e - 15).transpose(0, 2, 1)


def pack(po):
    """[splits, 2, s_q, 128, 512] partial outputs (head/column order) -> the
    partial_out bytes: the value of head 32j + 16a + r and column 16c + 4g + i
    at fp16 index 16384 j + 8 (64 c + 16 g + r) + 4 a + i of its block, its
    descale at index 128 (c / 8) + 32 j + 2 r + a of the block's descales."""
    po = np.asarray(po, np.float64)
    n, k, s = po.shape[:3]
    nb = n * k * s
    po = po.reshape(nb, N_HEADS, D_C)
    d = descales(po)                                                   # [nb, q, head]
    scaled = po / d.transpose(0, 2, 1).repeat(128, axis=2)            # column 128 q + .. -> quarter q
    v = scaled.reshape(nb, 4, 2, 16, 32, 4, 4)                         # j, a, r, c, g, i
    vals = v.transpose(0, 1, 4, 5, 3, 2, 6).astype(np.float16)         # j, c, g, r, a, i
    dsc = d.reshape(nb, 4, 4, 2, 16).transpose(0, 1, 2, 4, 3).astype(np.float32)   # q, j, r, a
    return np.concatenate([vals.reshape(-1).view(np.uint8), dsc.reshape(-1).view(np.uint8)])


def unpack(buf, num_splits, s_q):
    """partial_out bytes -> [splits, 2, s_q, 128, 512] float64."""
    nb = num_splits * 2 * s_q
    buf = np.asarray(buf, np.uint8)
    vals = buf[:nb * BLOCK_BYTES].view(np.float16).astype(np.float64).reshape(nb, 4, 32, 4, 16, 2, 4)  # j c g r a i
    dsc = buf[nb * BLOCK_BYTES:nb * (BLOCK_BYTES + DESC_BYTES)].view(np.float32).astype(np.float64)
    dsc = dsc.reshape(nb, 4, 4, 16, 2)                                  # q, j, r, a
    v = vals.transpose(0, 1, 5, 4, 2, 3, 6).reshape(nb, N_HEADS, 32, 16)   # head (j a r), c, (g i)
    d = dsc.transpose(0, 2, 4, 3, 1).reshape(nb, N_HEADS, 4)             # head (j a r), q
    v = v * d.repeat(8, axis=2)[:, :, :, None]                            # c -> quarter c / 8
    return v.reshape(num_splits, 2, s_q, N_HEADS, D_C)
