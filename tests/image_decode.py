"""Test-side decoder of the operand images the library writes (the layouts
include/svdq.h documents), so that the parity tests can compare what the GEMM
actually reads with the oracle's row-major codes, scales, T and L2.

Pure numpy, no arithmetic beyond unpacking: every function returns bit
patterns (uint8 / uint16) in the row-major ABI layouts."""
from __future__ import annotations

import numpy as np

INT4_BLOCK, FP4_CBLOCK, FP4_SBLOCK = 2048, 1024, 64
LR_XBLOCK, LR_WBLOCK, BIAS_BLOCK, BIAS_TAIL = 2048, 1024, 64, 1024


def _round_up(x, m):
    return (x + m - 1) // m * m


def act_layout(mode: str, M: int, K: int, rank: int) -> dict:
    """Offsets of the activation image (rows padded to 256; K split count S
    as the header gives it)."""
    G = K // 64
    RT = _round_up(M, 256) // 32
    blocks = RT * 32 // 16
    S = max(1, min(16, -(-1024 // blocks), G // 48))
    lay = dict(G=G, RT=RT, S=S, code=0)
    if mode == "int4":
        lay["lr"] = G * RT * INT4_BLOCK
    else:
        lay["scale"] = G * RT * FP4_CBLOCK
        lay["lr"] = lay["scale"] + G * RT * FP4_SBLOCK
    lay["tpart"] = lay["lr"] + (rank // 16) * RT * LR_XBLOCK
    lay["bytes"] = lay["tpart"] + (S * RT * 32 * rank * 4 if rank > 0 and S > 1 else 0)
    return lay


def weight_layout(mode: str, N: int, K: int, rank: int) -> dict:
    G = K // 64
    CT = _round_up(N, 192 if mode == "int4" else 256) // 32
    lay = dict(G=G, CT=CT, code=0)
    if mode == "int4":
        lay["lr"] = G * CT * INT4_BLOCK
    else:
        lay["scale"] = G * CT * FP4_CBLOCK
        lay["lr"] = lay["scale"] + G * CT * FP4_SBLOCK
    lay["bias"] = lay["lr"] + (rank // 16) * CT * LR_WBLOCK
    lay["bytes"] = lay["bias"] + CT * BIAS_BLOCK + BIAS_TAIL
    return lay


def _fields_to_nibbles(b24: np.ndarray) -> np.ndarray:
    """[..., 24] bytes = a little-endian 192-bit string of 32 six-bit
    sign-magnitude fields -> [..., 16] bytes of packed two's-complement
    nibbles (element 2j low).  Field = (q < 0 ? 0x20 : 0) | |q|."""
    bits = np.unpackbits(b24, axis=-1, bitorder="little")           # [..., 192]
    bits = bits.reshape(*b24.shape[:-1], 32, 6).astype(np.int64)
    f = (bits << np.arange(6)).sum(axis=-1)                           # [..., 32]
    assert np.all((f & 0x1F) <= 8), "field magnitude above 8"
    q = np.where(f & 0x20, -(f & 0x1F), f & 0x1F)
    nib = (q & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def _int4_blocks(img: np.ndarray, base: int, G: int, T: int):
    """INT4 code blocks [G][T][2048] -> (codes [T*32][K/2] uint8,
    scale dwords [T*32][G][4] uint32: slot r dword 0, 1 and slot 32 + r
    dword 0, 1)."""
    blk = img[base:base + G * T * INT4_BLOCK].reshape(G, T, INT4_BLOCK)
    halves = []
    for h in range(2):
        head = blk[:, :, 768 * h:768 * h + 512].reshape(G, T, 32, 16)
        tail = blk[:, :, 768 * h + 512:768 * h + 768].reshape(G, T, 32, 8)
        halves.append(_fields_to_nibbles(np.concatenate([head, tail], axis=-1)))  # [G][T][32][16]
    codes = np.concatenate(halves, axis=-1)                       # [G][T][32][32]
    codes = codes.transpose(1, 2, 0, 3).reshape(T * 32, G * 32)
    sc = blk[:, :, 1536:].copy().view(np.uint32).reshape(G, T, 64, 2)
    sc = np.concatenate([sc[:, :, :32, :], sc[:, :, 32:, :]], axis=-1)   # [G][T][32][4]
    return codes, sc.transpose(1, 2, 0, 3).reshape(T * 32, G, 4)


def _fp4_blocks(img: np.ndarray, code: int, scale: int, G: int, T: int):
    cb = img[code:code + G * T * FP4_CBLOCK].reshape(G, T, 2, 32, 16)     # slot = 32 h + r
    codes = cb.transpose(1, 3, 0, 2, 4).reshape(T * 32, G * 32)
    sb = img[scale:scale + G * T * FP4_SBLOCK].reshape(G, T, 2, 32)
    scales = sb.transpose(1, 3, 0, 2).reshape(T * 32, G * 2)
    return codes, scales


def decode_act_image(img: np.ndarray, mode: str, M: int, K: int, rank: int) -> dict:
    """The activation image of M rows -> codes [Mp][K/2], scales (INT4: the
    dwords of the bf16 scale operand [Mp][G][4]; FP4: E8M0 bytes
    [Mp][K/32]), T hi and lo bf16 [Mp][rank] (Mp = padded rows)."""
    lay = act_layout(mode, M, K, rank)
    img = np.asarray(img, np.uint8)
    assert img.size == lay["bytes"], (img.size, lay["bytes"])
    G, RT = lay["G"], lay["RT"]
    if mode == "int4":
        codes, scales = _int4_blocks(img, 0, G, RT)
    else:
        codes, scales = _fp4_blocks(img, 0, lay["scale"], G, RT)
    out = dict(codes=codes, scales=scales, layout=lay)
    if rank > 0:
        # [j][rt][hi/lo][slot][8 bf16]; slot = 32 a + r
        t = img[lay["lr"]:lay["tpart"]].copy().view(np.uint16).reshape(rank // 16, RT, 2, 2, 32, 8)
        # slot s = 32 a + r holds ranks 16 j + 8 a .. +7 of row r
        t = t.transpose(2, 1, 4, 0, 3, 5).reshape(2, RT * 32, rank)
        out["t_hi"], out["t_lo"] = t[0], t[1]
    return out


def decode_weight_image(img: np.ndarray, mode: str, N: int, K: int, rank: int) -> dict:
    """The prepared weight -> codes [Np][K/2], scales as in decode_act_image,
    lora_up bf16 [Np][rank], bias bf16 [Np], and the zero tail."""
    lay = weight_layout(mode, N, K, rank)
    img = np.asarray(img, np.uint8)
    assert img.size == lay["bytes"], (img.size, lay["bytes"])
    G, CT = lay["G"], lay["CT"]
    if mode == "int4":
        codes, scales = _int4_blocks(img, 0, G, CT)
    else:
        codes, scales = _fp4_blocks(img, 0, lay["scale"], G, CT)
    out = dict(codes=codes, scales=scales, layout=lay)
    if rank > 0:
        lr = img[lay["lr"]:lay["bias"]].copy().view(np.uint16).reshape(rank // 16, CT, 2, 32, 8)
        out["lora_up"] = lr.transpose(1, 3, 0, 2, 4).reshape(CT * 32, rank)
    bias_end = lay["bias"] + CT * BIAS_BLOCK
    out["bias"] = img[lay["bias"]:bias_end].copy().view(np.uint16)
    out["tail"] = img[bias_end:]
    return out
