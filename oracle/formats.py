"""Storage-format decoding, written from the format definitions.

fp8 e4m3fn (OCP 8-bit floating point, "FN" variant): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
m * 2^-9; no infinities; only S.1111.111 is NaN.  The index cache and the
index queries are stored in this format (the pages keep the index cache
resident in device memory and leave its element type open; the reading taken
is fp8 with integer values, which it represents exactly).

bf16: the upper 16 bits of an IEEE binary32.

The 656-byte fp8 latent entry (ESS concept page, the FlashTrans row: 656
bytes per token per layer; the split 512 fp8 + 16 bytes of scales + 64 bf16
is the reading taken, matching the page's per-token block size and its
83.2 % / 16.8 % split): bytes 0..511 the c_KV values as fp8 e4m3fn, bytes
512..527 four float32 scales, one per block of 128 c_KV values, bytes
528..655 the 64 k_R values as bf16.  A latent value is code value x its
block's scale; k_R is read as bf16.
"""
import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one fp8 e4m3fn byte."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)],
                        dtype=np.float64)


def decode_e4m3fn(b: np.ndarray) -> np.ndarray:
    """uint8 array of fp8 e4m3fn codes -> float64 array."""
    return E4M3FN_TABLE[np.asarray(b, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 array of bf16 bit patterns -> float64 array."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode_entries(entries: np.ndarray) -> np.ndarray:
    """uint8 656-byte entries [n][656] -> float64 latents [n][576]."""
    e = np.asarray(entries, dtype=np.uint8)
    n = e.shape[0]
    vals = decode_e4m3fn(e[:, :512]).reshape(n, 4, 128)
    scale = np.ascontiguousarray(e[:, 512:528]).view(np.float32).astype(np.float64)
    out = np.empty((n, 576), np.float64)
    out[:, :512] = (vals * scale[:, :, None]).reshape(n, 512)
    out[:, 512:] = decode_bf16(np.ascontiguousarray(e[:, 528:656]).view(np.uint16))
    return out


def encode_entries(bf16_rows: np.ndarray) -> np.ndarray:
    """bf16 latents [n][576] (uint16 bits) -> 656-byte entries [n][656], by
    the definition: per 128-value block of c_KV the scale is the smallest
    power of two s with max|x| <= 448 s (1 for an all-zero block), found by
    stepping the exponent; each value takes the finite e4m3fn code whose
    value is nearest x / s, a tie going to the even code, and -0 encodes as
    +0; k_R is copied.  Brute force over every code (slow; small inputs
    only).  Parity unpinned against the pages, which give only the entry's
    size: this is the library's reading of the 656-byte block."""
    rows = np.asarray(bf16_rows, dtype=np.uint16).reshape(-1, 576)
    n = rows.shape[0]
    x = decode_bf16(rows[:, :512]).reshape(n, 4, 128)
    out = np.zeros((n, 656), np.uint8)
    finite = np.array([c for c in range(256) if not np.isnan(E4M3FN_TABLE[c])])
    vals = E4M3FN_TABLE[finite]
    for i in range(n):
        for blk in range(4):
            amax = float(np.abs(x[i, blk]).max())
            t = 0
            if amax > 0:
                t = -160
                while amax > 448.0 * 2.0 ** t:
                    t += 1
            s = 2.0 ** t
            for c in range(128):
                v = x[i, blk, c] / s
                d = np.abs(vals - v)
                best = finite[d == d.min()]
                if len(best) > 1:          # a tie: the even code (signed zeros aside)
                    best = best[best % 2 == 0] if np.any(best % 2 == 0) else best
                code = int(best.min())
                if code == 0x80:
                    code = 0
                out[i, blk * 128 + c] = code
            out[i, 512 + 4 * blk:516 + 4 * blk] = np.frombuffer(np.float32(s).tobytes(), np.uint8)
    out[:, 528:] = np.ascontiguousarray(rows[:, 512:]).view(np.uint8).reshape(n, 128)
    return out
