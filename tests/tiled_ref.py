"""Reference packer and unpacker for the library's tiled weight layout, written from the
layout's description in include/qmoe.h (QMOE_LAYOUT_TILES). Test infrastructure: the GPU
packing kernel is compared with pack() byte for byte, and unpack() inverts pack() from the
same description read the other way."""
from __future__ import annotations

import numpy as np

# element i of a 4-bit word sits in nibble NIBBLE_OF[i]
NIBBLE_OF = (0, 4, 1, 5, 2, 6, 3, 7)


def stack_geometry(which: str, H: int, I: int, bits: int, fusion: int, swiglu: bool = True):
    """(K, N rows of the rows-layout stack, S streams, rows per stream, fusion used)."""
    if which == "fc1":
        if swiglu and fusion != 0:
            return H, 2 * I, 2, I, fusion
        return H, I, 1, I, 0
    if which == "fc3":
        return H, I, 1, I, 0
    return I, H, 1, H, 0


def codes_of(rows_stack: np.ndarray, K: int, bits: int) -> np.ndarray:
    """uint8 [E, N, K*bits/8] -> codes [E, N, K]."""
    if bits == 8:
        return rows_stack[:, :, :K].astype(np.uint8)
    lo = rows_stack & 0x0F
    hi = rows_stack >> 4
    out = np.empty(rows_stack.shape[:2] + (2 * rows_stack.shape[2],), np.uint8)
    out[:, :, 0::2] = lo
    out[:, :, 1::2] = hi
    return out[:, :, :K]


def pack(rows_stack: np.ndarray, which: str, H: int, I: int, bits: int, fusion: int,
         swiglu: bool = True, natural: bool = False) -> np.ndarray:
    """natural: 4-bit element i in nibble i (the MX FP4 order) instead of NIBBLE_OF[i]."""
    K, N, S, R, fu = stack_geometry(which, H, I, bits, fusion, swiglu)
    E = rows_stack.shape[0]
    assert rows_stack.shape == (E, N, K * bits // 8)
    ssk = 128 if bits == 4 else 64
    NB, KT = -(-R // 16), -(-K // ssk)
    codes = codes_of(rows_stack, K, bits)
    # stream rows: [E, S, R, K], then zero-padded to [E, S, NB*16, KT*ssk]
    if fu == 1:
        sc = np.stack([codes[:, 0::2], codes[:, 1::2]], axis=1)
    elif fu == 2:
        sc = np.stack([codes[:, :R], codes[:, R:]], axis=1)
    else:
        sc = codes[:, None]
    pad = np.zeros((E, S, NB * 16, KT * ssk), np.uint8)
    pad[:, :, :R, :K] = sc
    out = np.zeros((E, S, NB, KT, 64, 16), np.uint8)  # tile (e, s, b, t), lane l, byte
    for q in range(4):
        for n in range(16):
            l = 16 * q + n
            rows = pad[:, :, n::16, :]  # row 16b + n -> [E, S, NB, KT*ssk]
            for j in range(ssk // 32):
                # elements k = t*ssk + 32j + 8q + i, i < 8 -> [E, S, NB, KT, 8]
                ks = (np.arange(KT)[:, None] * ssk + 32 * j + 8 * q + np.arange(8)[None, :])
                el = rows[:, :, :, ks]
                if bits == 4:
                    word = np.zeros(el.shape[:-1], np.uint32)
                    for i in range(8):
                        word |= el[..., i].astype(np.uint32) << np.uint32(4 * (i if natural else NIBBLE_OF[i]))
                    # the word's little-endian bytes
                    out[:, :, :, :, l, 4 * j:4 * j + 4] = np.stack(
                        [(word >> np.uint32(8 * c)) & np.uint32(0xFF) for c in range(4)],
                        axis=-1).astype(np.uint8)
                else:
                    out[:, :, :, :, l, 8 * j:8 * j + 8] = el
    return out.reshape(-1)


def unpack(packed: np.ndarray, E: int, which: str, H: int, I: int, bits: int, fusion: int,
           swiglu: bool = True, natural: bool = False) -> np.ndarray:
    """Codes [E, N, K] of the rows-layout stack, read back tile by tile, lane by lane."""
    K, N, S, R, fu = stack_geometry(which, H, I, bits, fusion, swiglu)
    ssk = 128 if bits == 4 else 64
    NB, KT = -(-R // 16), -(-K // ssk)
    t = packed.reshape(E, S, NB, KT, 64, 16)
    codes = np.zeros((E, S, NB * 16, KT * ssk), np.uint8)
    for l in range(64):
        n, q = l % 16, l // 16
        for j in range(ssk // 32):
            for i in range(8):
                k = np.arange(KT) * ssk + 32 * j + 8 * q + i
                if bits == 4:
                    p = i if natural else NIBBLE_OF[i]
                    byte = t[:, :, :, :, l, 4 * j + p // 2]
                    v = (byte >> 4) if (p % 2) else (byte & 0x0F)
                else:
                    v = t[:, :, :, :, l, 8 * j + i]
                codes[:, :, n::16, k] = v
    sc = codes[:, :, :R, :K]
    out = np.zeros((E, N, K), np.uint8)
    if fu == 1:
        out[:, 0::2], out[:, 1::2] = sc[:, 0], sc[:, 1]
    elif fu == 2:
        out[:, :R], out[:, R:] = sc[:, 0], sc[:, 1]
    else:
        out[:] = sc[:, 0]
    return out
