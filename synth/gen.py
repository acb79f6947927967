"""Counter-keyed random streams for every input tensor of the decode path.

Every tensor is drawn from NumPy's Philox generator keyed by
(seed, tensor id, layer, request, token slot, step or chunk), so any piece can
be regenerated on its own and both the oracle and the GPU path see the same
bytes.  Long tensors indexed by position (index keys, host latents) are drawn
in chunks of CHUNK positions, each chunk its own stream, so a position range
can be produced without drawing the whole row.

Value recipes:
  * index keys k[b][s][:] and step-0 index queries: integers uniform in
    [-7, 7], stored as fp8 e4m3fn bytes (exact for these integers);
  * index queries drift as q_t = clip(round(rho * q_{t-1} + eps), -7, 7) with
    eps ~ N(0, sigma^2), sigma = sigma0 * sqrt(1 - rho^2), sigma0 = sqrt(56/3)
    (the standard deviation of the uniform integers, so that without the
    clip the spread would stay at its step-0 value; the clip trims it to
    about 3.7), rounding half to even; each (request, token slot) has its
    own chain;
  * head weights w[b][j][h]: integers uniform in [1, 4], fixed over steps;
  * absorbed queries qa[t][b][j][h][:576] ~ N(0, 0.1^2), fresh each step;
  * latents host[b][s][:576] ~ N(0, 0.5^2);
  both float tensors are rounded to bf16 (round to nearest even) and handed
  over as uint16 bit patterns.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

CHUNK = 4096

# Tensor ids for the stream keys.
_T_KEYS, _T_Q0, _T_QNOISE, _T_W, _T_QA, _T_LAT = 1, 2, 3, 4, 5, 6

# fp8 e4m3fn codes of the integers 0..7 (sign bit 0x80 for negatives).
_E4M3_OF_INT = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E],
                        dtype=np.uint8)


def _rng(*key_parts) -> np.random.Generator:
    # Philox takes a 128-bit key: pack the parts into two 64-bit words.
    parts = [int(p) & 0xFFFF for p in key_parts]
    while len(parts) < 8:
        parts.append(0)
    lo = sum(p << (16 * i) for i, p in enumerate(parts[:4]))
    hi = sum(p << (16 * i) for i, p in enumerate(parts[4:8]))
    return np.random.Generator(np.random.Philox(key=[lo, hi]))


def encode_e4m3_int(v: np.ndarray) -> np.ndarray:
    """Integers in [-7, 7] -> their exact fp8 e4m3fn byte codes."""
    v = np.asarray(v)
    if v.size and (v.min() < -7 or v.max() > 7):
        raise ValueError("only integers in [-7, 7] are encoded")
    a = np.abs(v).astype(np.int64)
    code = _E4M3_OF_INT[a]
    return np.where(v < 0, code | 0x80, code).astype(np.uint8)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


# The 656-byte latent entry of an fp8 latent cache: c_KV as 512 fp8 e4m3fn
# values, then one float32 scale per block of 128 of them (16 bytes), then
# k_R as 64 bf16 (128 bytes).  Scales are powers of two, so every stored
# value times its scale is exactly a bf16 value.
ENTRY_BYTES = 656
_E4M3_POS = np.array([(1.0 + (c & 7) / 8.0) * 2.0 ** (((c >> 3) & 15) - 7)
                      if (c >> 3) & 15 else (c & 7) * 2.0 ** -9
                      for c in range(127)])          # codes 0x00..0x7E, increasing


def encode_e4m3_rne(x: np.ndarray) -> np.ndarray:
    """float -> fp8 e4m3fn codes, round to nearest (ties to the even code),
    |x| saturated at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a), 1, 126)
    lo = hi - 1
    d_lo, d_hi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a <= _E4M3_POS[0], 0, code)
    return np.where((x < 0) & (code != 0), code | 0x80, code).astype(np.uint8)


def encode_entries(bf16_rows: np.ndarray) -> np.ndarray:
    """uint16 bf16 latents [n][576] -> uint8 656-byte entries [n][656]: each
    block of 128 c_KV values scaled by 2^ceil(log2(max|x| / 448)) (1 for an
    all-zero block) and rounded to fp8 e4m3fn; k_R kept as bf16."""
    rows = np.asarray(bf16_rows, dtype=np.uint16)
    n = rows.shape[0]
    x = (rows[:, :512].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    blocks = x.reshape(n, 4, 128)
    amax = np.abs(blocks).max(axis=2)
    e = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 0.0)
    scale = np.ldexp(1.0, e.astype(np.int64))
    q = encode_e4m3_rne(blocks / scale[:, :, None]).reshape(n, 512)
    out = np.empty((n, ENTRY_BYTES), np.uint8)
    out[:, :512] = q
    out[:, 512:528] = scale.astype(np.float32).view(np.uint8).reshape(n, 16)
    out[:, 528:] = np.ascontiguousarray(rows[:, 512:]).view(np.uint8).reshape(n, 128)
    return out


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- indexer --

def index_key_ints(wl, layer: int, b: int, s0: int = 0, s1: int = None):
    """int8 [s1-s0, d_I] integer values of the index keys of request b."""
    s1 = wl.ctx_len if s1 is None else s1
    c0, c1 = s0 // CHUNK, (s1 + CHUNK - 1) // CHUNK
    out = np.empty(((c1 - c0) * CHUNK, wl.idx_dim), np.int8)
    for c in range(c0, c1):
        r = _rng(wl.seed, _T_KEYS, layer, b, c)
        out[(c - c0) * CHUNK:(c - c0 + 1) * CHUNK] = r.integers(
            -7, 8, size=(CHUNK, wl.idx_dim), dtype=np.int8)
    off = s0 - c0 * CHUNK
    return out[off:off + (s1 - s0)]


def index_keys(wl, layer: int, b: int, s0: int = 0, s1: int = None):
    """uint8 [s1-s0, d_I] fp8 e4m3fn bytes of the index keys."""
    return encode_e4m3_int(index_key_ints(wl, layer, b, s0, s1))


def index_query_ints(wl, layer: int, b: int, j: int) -> np.ndarray:
    """int8 [T, H_I, d_I]: the drifting query chain of (request b, token j)."""
    shape = (wl.idx_heads, wl.idx_dim)
    q = np.empty((wl.steps,) + shape, np.int8)
    q[0] = _rng(wl.seed, _T_Q0, layer, b, j).integers(-7, 8, size=shape,
                                                      dtype=np.int8)
    sigma = np.sqrt(56.0 / 3.0) * np.sqrt(1.0 - wl.rho * wl.rho)
    noise = _rng(wl.seed, _T_QNOISE, layer, b, j)
    for t in range(1, wl.steps):
        eps = noise.standard_normal(shape) * sigma
        q[t] = np.clip(np.rint(wl.rho * q[t - 1] + eps), -7, 7).astype(np.int8)
    return q


def head_weights(wl, layer: int, b: int, j: int) -> np.ndarray:
    """float32 [H_I] integer head weights in [1, 4]."""
    r = _rng(wl.seed, _T_W, layer, b, j)
    return r.integers(1, 5, size=wl.idx_heads).astype(np.float32)


def index_inputs(wl, layer: int):
    """All indexer inputs of one layer.

    Returns (q_bytes uint8 [T][B][m][H_I][d_I], w float32 [B][m][H_I],
    n_vis int32 [B][m]).  The keys are drawn separately (they are large).
    """
    q = np.empty((wl.steps, wl.batch, wl.mtp, wl.idx_heads, wl.idx_dim),
                 np.uint8)
    w = np.empty((wl.batch, wl.mtp, wl.idx_heads), np.float32)
    for b in range(wl.batch):
        for j in range(wl.mtp):
            q[:, b, j] = encode_e4m3_int(index_query_ints(wl, layer, b, j))
            w[b, j] = head_weights(wl, layer, b, j)
    n_vis = np.array([[wl.n_vis(j) for j in range(wl.mtp)]] * wl.batch,
                     dtype=np.int32)
    return q, w, n_vis


def fill_index_keys(wl, layer: int, out: np.ndarray) -> np.ndarray:
    """Write all index keys of a layer into out uint8 [B][L][d_I]."""
    def job(b):
        out[b] = index_keys(wl, layer, b)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(wl.batch)))
    return out


# ------------------------------------------------------------------- MLA --

def abs_query(wl, layer: int, t: int) -> np.ndarray:
    """uint16 bf16 bits [B][m][H][576] of the absorbed queries of step t."""
    out = np.empty((wl.batch, wl.mtp, wl.mla_heads, wl.lat_dim), np.uint16)
    for b in range(wl.batch):
        for j in range(wl.mtp):
            r = _rng(wl.seed, _T_QA, layer, b, j, t)
            x = r.standard_normal((wl.mla_heads, wl.lat_dim),
                                  dtype=np.float32) * np.float32(0.1)
            out[b, j] = f32_to_bf16_bits(x)
    return out


def latents(wl, layer: int, b: int, s0: int = 0, s1: int = None):
    """uint16 bf16 bits [s1-s0][576] of the host latents of request b."""
    s1 = wl.ctx_len if s1 is None else s1
    c0, c1 = s0 // CHUNK, (s1 + CHUNK - 1) // CHUNK
    out = np.empty(((c1 - c0) * CHUNK, wl.lat_dim), np.uint16)
    for c in range(c0, c1):
        r = _rng(wl.seed, _T_LAT, layer, b, c)
        x = r.standard_normal((CHUNK, wl.lat_dim), dtype=np.float32)
        out[(c - c0) * CHUNK:(c - c0 + 1) * CHUNK] = f32_to_bf16_bits(
            x * np.float32(0.5))
    off = s0 - c0 * CHUNK
    return out[off:off + (s1 - s0)]


def latent_rows(wl, layer: int, b: int, pos: np.ndarray) -> np.ndarray:
    """uint16 [len(pos)][576]: latents of request b at the given positions,
    drawing only the chunks that hold them."""
    pos = np.asarray(pos, dtype=np.int64)
    out = np.empty((pos.size, wl.lat_dim), np.uint16)
    chunks = np.unique(pos // CHUNK)
    for c in chunks:
        sel = np.nonzero(pos // CHUNK == c)[0]
        block = latents(wl, layer, b, int(c) * CHUNK,
                        min(wl.ctx_len, (int(c) + 1) * CHUNK))
        out[sel] = block[pos[sel] - int(c) * CHUNK]
    return out


def fill_latents(wl, layer: int, out: np.ndarray) -> np.ndarray:
    """Write all host latents of a layer into out uint16 [B][L][576] (for
    example a pinned host buffer), chunk streams spread over threads."""
    nchunk = (wl.ctx_len + CHUNK - 1) // CHUNK

    def job(item):
        b, c = item
        s0, s1 = c * CHUNK, min(wl.ctx_len, (c + 1) * CHUNK)
        out[b, s0:s1] = latents(wl, layer, b, s0, s1)
    items = [(b, c) for b in range(wl.batch) for c in range(nchunk)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, items))
    return out
