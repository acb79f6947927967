"""ctypes binding of libess.so: the C ABI declared in include/ess.h, one
Python function per entry point with the same name.  Argument marshalling
only: tensors pass their device addresses, streams their HIP handles; every
step of the path runs in the library's HIP kernels.  There is no fallback:
if the library is missing or fails to load, every call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ESS_LIB names another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree libess.so.
LIB_PATH = os.environ.get("ESS_LIB") or os.path.join(HERE, "libess.so")

ESS_OK = 0
ESS_ERR_INVALID = -1
ESS_ERR_UNSUPPORTED = -2
ESS_ERR_CAPACITY = -3
ESS_ERR_HIP = -4
ESS_ERR_NOMEM = -5

ESS_MODE_FILL = 0
ESS_MODE_INLINE = 1
ESS_MODE_PREFETCH = 2

ESS_EVICT_LRU = 0
ESS_EVICT_RANDOM = 1
ESS_EVICT_SCORE = 2

EXPORTED = (
    "ess_workspace_bytes", "ess_lru_state_bytes", "ess_pool_reset",
    "ess_index_scores", "ess_topk_lookup", "ess_pool_update",
    "ess_sparse_mla_decode", "ess_sparse_mla_decode_entries", "ess_miss_copy",
    "ess_miss_copy_entries",
    "ess_decode_step",
    "ess_host_alloc", "ess_host_free", "ess_replay_evictions",
    "ess_tail_init", "ess_tail_release", "ess_append_tokens",
    "ess_prefill_ws_bytes", "ess_prefill_layers",
    "ess_pool_status", "ess_copy_async", "ess_thread_release",
    "ess_sparse_mla_decode_noalloc",
    "ess_status_string", "ess_last_error",
)


class EssError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} -> {status}: {msg}")
        self.status = status


class ess_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("mtp", ctypes.c_int32),
                ("ctx_len", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("mla_heads", ctypes.c_int32),
                ("lat_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("pool_slots", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t


class ess_layer_io(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "q_idx", "w_idx", "k_idx", "q_abs", "host_view", "pool",
        "cache_slots", "slot_pos", "lru_state", "scores", "sel_pos",
        "sel_slot", "n_sel", "row_dst", "sel_slot_post", "miss_pos",
        "miss_slot", "n_miss", "n_evict", "out", "lse", "ws")] + [
        ("ws_bytes", _S), ("host_entries", _P), ("tail_rows", _P),
        ("tail_start", _P), ("tail_block", _I)]


class ess_tail(ctypes.Structure):
    _fields_ = [("rows", _P), ("entries", _P), ("block", _I), ("batch", _I),
                ("host", ctypes.POINTER(ctypes.c_int32)), ("state_dev", _P),
                ("events", _P)]

    def _host(self, i):
        B = self.batch
        return [self.host[i * B + b] for b in range(B)]

    @property
    def first(self):
        return self._host(0)

    @property
    def n_ctx(self):
        return self._host(1)

    @property
    def start(self):
        """Host copy of every request's first tail position."""
        return self._host(2)

    @property
    def start_dev(self):
        """Device address of the per-request start array (for
        ess_layer_io.tail_start)."""
        return self.state_dev + 2 * self.batch * 4


_lib = None


def lib():
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "or python decode_lightning_indexer_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(ess_dims)
        sig = {
            "ess_workspace_bytes": (_S, [D]),
            "ess_lru_state_bytes": (_S, [D]),
            "ess_pool_reset": (_I, [D, _P, _P, _P, _P]),
            "ess_index_scores": (_I, [D, _P, _P, _P, _P, _P, _P]),
            "ess_topk_lookup": (_I, [D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
            "ess_pool_update": (_I, [D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _P, _P]),
            "ess_sparse_mla_decode": (_I, [D, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _S, _P]),
            "ess_sparse_mla_decode_entries": (_I, [D, _P, _P, _P, _P, _P, _P, _P,
                                                   _P, _P, _P, _S, _P]),
            "ess_miss_copy": (_I, [D, _I, _P, _P, _P, _P, _P, _P]),
            "ess_miss_copy_entries": (_I, [D, _I, _P, _P, _P, _P, _P, _P]),
            "ess_decode_step": (_I, [D, _I, ctypes.POINTER(ess_layer_io), _P,
                                     _I, _P, _P]),
            "ess_host_alloc": (_I, [_S, ctypes.POINTER(_P), ctypes.POINTER(_P)]),
            "ess_tail_init": (_I, [ctypes.POINTER(ess_tail), D, _P, _P, _I, _P, _P, _P]),
            "ess_tail_release": (_I, [ctypes.POINTER(ess_tail)]),
            "ess_append_tokens": (_I, [D, ctypes.POINTER(ess_tail), _P, _P, _P, _P,
                                       _P, _P, _P]),
            "ess_host_free": (_I, [_P]),
            "ess_replay_evictions": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P,
                                          ctypes.c_uint64, _I, _P, _P]),
            "ess_prefill_ws_bytes": (_S, [_I]),
            "ess_prefill_layers": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _S,
                                        _P, _P, _I, _I, _P, _P, _P]),
            "ess_pool_status": (_I, [D, _P, _P, _P]),
            "ess_sparse_mla_decode_noalloc": (_I, [D, _P, _P, _P, _P, _P, _P, _P,
                                                   _P, _P, _P]),
            "ess_copy_async": (_I, [_P, _P, _S, _P]),
            "ess_thread_release": (_I, []),
            "ess_status_string": (ctypes.c_char_p, [_I]),
            "ess_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
        # Before the interpreter exits (and so before the HIP runtime's
        # static destructors run): the main thread's stream-ordering events.
        import atexit
        atexit.register(_release_at_exit)
    return _lib


def _release_at_exit():
    if _lib is not None:
        _lib.ess_thread_release()


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, st):
    if st != ESS_OK:
        L = lib()
        raise EssError(fn, L.ess_status_string(st).decode(),
                       L.ess_last_error().decode())


def make_dims(batch, mtp, ctx_len, idx_heads, idx_dim, mla_heads, topk,
              pool_slots, softmax_scale, lat_dim=576, v_dim=512) -> ess_dims:
    return ess_dims(batch, mtp, ctx_len, idx_heads, idx_dim, mla_heads,
                    lat_dim, v_dim, topk, pool_slots, softmax_scale)


def ess_workspace_bytes(d: ess_dims) -> int:
    return lib().ess_workspace_bytes(ctypes.byref(d))


def ess_lru_state_bytes(d: ess_dims) -> int:
    return lib().ess_lru_state_bytes(ctypes.byref(d))


def ess_pool_reset(d, cache_slots, slot_pos, lru_state, stream=None):
    _check("ess_pool_reset", lib().ess_pool_reset(
        ctypes.byref(d), _ptr(cache_slots), _ptr(slot_pos), _ptr(lru_state),
        _stream(stream)))


def ess_pool_status(d, lru_state, status, stream=None):
    """status: device int32 [B][4] <- (err, compactions, updates, ring entries)."""
    _check("ess_pool_status", lib().ess_pool_status(
        ctypes.byref(d), _ptr(lru_state), _ptr(status), _stream(stream)))


def ess_copy_async(dst, src, nbytes, stream=None):
    """Copy nbytes between device memory and pinned host memory (addresses or
    tensors) on the stream."""
    _check("ess_copy_async", lib().ess_copy_async(_ptr(dst), _ptr(src), nbytes,
                                                  _stream(stream)))


def ess_thread_release():
    _check("ess_thread_release", lib().ess_thread_release())


def ess_index_scores(d, q_fp8, w, k_fp8, n_vis, scores, stream=None):
    _check("ess_index_scores", lib().ess_index_scores(
        ctypes.byref(d), _ptr(q_fp8), _ptr(w), _ptr(k_fp8), _ptr(n_vis),
        _ptr(scores), _stream(stream)))


def ess_topk_lookup(d, k, n_tok, scores, n_vis, cache_slots, sel_pos,
                    sel_slot, n_sel, ws=None, ws_bytes=0, stream=None):
    _check("ess_topk_lookup", lib().ess_topk_lookup(
        ctypes.byref(d), k, n_tok, _ptr(scores), _ptr(n_vis),
        _ptr(cache_slots), _ptr(sel_pos), _ptr(sel_slot), _ptr(n_sel),
        _ptr(ws), ws_bytes, _stream(stream)))


def ess_pool_update(d, k, n_tok, sel_pos, n_sel, cache_slots, slot_pos,
                    lru_state, miss_pos, miss_slot, n_miss, n_evict, row_dst,
                    sel_slot_post, stream=None):
    _check("ess_pool_update", lib().ess_pool_update(
        ctypes.byref(d), k, n_tok, _ptr(sel_pos), _ptr(n_sel),
        _ptr(cache_slots), _ptr(slot_pos), _ptr(lru_state), _ptr(miss_pos),
        _ptr(miss_slot), _ptr(n_miss), _ptr(n_evict), _ptr(row_dst),
        _ptr(sel_slot_post), _stream(stream)))


def ess_sparse_mla_decode(d, q_abs, sel_pos, sel_src, row_dst, n_sel, pool,
                          host_view, out, lse, ws, ws_bytes, stream=None):
    _check("ess_sparse_mla_decode", lib().ess_sparse_mla_decode(
        ctypes.byref(d), _ptr(q_abs), _ptr(sel_pos), _ptr(sel_src),
        _ptr(row_dst), _ptr(n_sel), _ptr(pool), _ptr(host_view), _ptr(out),
        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def ess_sparse_mla_decode_noalloc(d, q_abs, sel_pos, sel_src, row_dst, n_sel,
                                  pool, host_view, out, lse, stream=None):
    _check("ess_sparse_mla_decode_noalloc", lib().ess_sparse_mla_decode_noalloc(
        ctypes.byref(d), _ptr(q_abs), _ptr(sel_pos), _ptr(sel_src),
        _ptr(row_dst), _ptr(n_sel), _ptr(pool), _ptr(host_view), _ptr(out),
        _ptr(lse), _stream(stream)))


def ess_sparse_mla_decode_entries(d, q_abs, sel_pos, sel_src, row_dst, n_sel,
                                  pool, entry_view, out, lse, ws, ws_bytes,
                                  stream=None):
    _check("ess_sparse_mla_decode_entries", lib().ess_sparse_mla_decode_entries(
        ctypes.byref(d), _ptr(q_abs), _ptr(sel_pos), _ptr(sel_src),
        _ptr(row_dst), _ptr(n_sel), _ptr(pool), _ptr(entry_view), _ptr(out),
        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def ess_miss_copy(d, list_stride, miss_pos, miss_slot, n_miss, host_view,
                  pool, stream=None):
    _check("ess_miss_copy", lib().ess_miss_copy(
        ctypes.byref(d), list_stride, _ptr(miss_pos), _ptr(miss_slot),
        _ptr(n_miss), _ptr(host_view), _ptr(pool), _stream(stream)))


def ess_miss_copy_entries(d, list_stride, miss_pos, miss_slot, n_miss,
                          entry_view, pool, stream=None):
    _check("ess_miss_copy_entries", lib().ess_miss_copy_entries(
        ctypes.byref(d), list_stride, _ptr(miss_pos), _ptr(miss_slot),
        _ptr(n_miss), _ptr(entry_view), _ptr(pool), _stream(stream)))


def ess_decode_step(d, layers, n_vis, mode, stream=None, side=None):
    """layers: a sequence of ess_layer_io."""
    arr = (ess_layer_io * len(layers))(*layers)
    _check("ess_decode_step", lib().ess_decode_step(
        ctypes.byref(d), len(layers), arr, _ptr(n_vis), mode,
        _stream(stream), _stream(side) if side is not None else None))


def ess_tail_init(d, rows, block, n_ctx, state_dev, stream=None, entries=None):
    """A new ess_tail over the device tail rows [B][2*block][576]; n_ctx:
    every request's length (sequence of B ints); state_dev: device int32
    [3*B]; entries: device [B][2*block][656] for a store of fp8 entries."""
    t = ess_tail()
    arr = (ctypes.c_int32 * d.batch)(*[int(x) for x in n_ctx])
    _check("ess_tail_init", lib().ess_tail_init(
        ctypes.byref(t), ctypes.byref(d), _ptr(rows), _ptr(entries), block, arr,
        _ptr(state_dev), _stream(stream)))
    return t


def ess_tail_release(t):
    _check("ess_tail_release", lib().ess_tail_release(ctypes.byref(t)))


def ess_append_tokens(d, t, new_keys, new_lat, k_idx, n_vis, host_kv, stream=None,
                      d2h=None):
    """host_kv: the host store's CPU address (HostStore.host): bf16 rows, or
    656-byte entries when the tail has entries."""
    _check("ess_append_tokens", lib().ess_append_tokens(
        ctypes.byref(d), ctypes.byref(t), _ptr(new_keys), _ptr(new_lat),
        _ptr(k_idx), _ptr(n_vis), _ptr(host_kv), _stream(stream),
        _stream(d2h) if d2h is not None else None))


def ess_host_alloc(nbytes: int):
    """Pinned, mapped host memory: returns (host address, device view)."""
    h, dv = _P(), _P()
    _check("ess_host_alloc", lib().ess_host_alloc(nbytes, ctypes.byref(h),
                                                  ctypes.byref(dv)))
    return h.value, dv.value


def ess_host_free(host_ptr: int):
    _check("ess_host_free", lib().ess_host_free(host_ptr))


def ess_replay_evictions(policy, pool_slots, scores, sel_pos, n_sel, seed=0,
                         request=0):
    """Host replay of one request's steps under an eviction policy.
    scores float32 [T][m][L], sel_pos int32 [T][m][k], n_sel int32 [T][m]
    (NumPy arrays in host memory).  Returns (n_miss, n_evict), int32 [T]."""
    import numpy as np
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    sel_pos = np.ascontiguousarray(sel_pos, dtype=np.int32)
    n_sel = np.ascontiguousarray(n_sel, dtype=np.int32)
    T, m, L = scores.shape
    if sel_pos.shape[:2] != (T, m) or n_sel.shape != (T, m):
        raise ValueError("scores, sel_pos and n_sel disagree on steps or ways")
    n_miss = np.zeros(T, np.int32)
    n_evict = np.zeros(T, np.int32)
    _check("ess_replay_evictions", lib().ess_replay_evictions(
        policy, L, pool_slots, T, m, sel_pos.shape[2], scores.ctypes.data,
        sel_pos.ctypes.data, n_sel.ctypes.data, seed, request,
        n_miss.ctypes.data, n_evict.ctypes.data))
    return n_miss, n_evict


def ess_prefill_ws_bytes(rows: int) -> int:
    return lib().ess_prefill_ws_bytes(rows)


def ess_prefill_layers(n_layers, rows, n_hist, n_new, host_kv, new_kv, bufs,
                       layer_out, ws, onload_layer_map=None, compute_reps=1,
                       load_layer0=False, compute=None, h2d=None, d2h=None):
    """Four-buffer prefill over n_layers layers.  host_kv: host address of
    pinned [n_layers][rows][576] bf16 (from ess_host_alloc); new_kv, bufs,
    layer_out, ws: device tensors; onload_layer_map: int sequence or None.
    Returns the buffer index of every layer (numpy int32)."""
    import numpy as np
    binding = np.full(n_layers, -1, np.int32)
    m = None
    if onload_layer_map is not None:
        m = np.ascontiguousarray(onload_layer_map, dtype=np.int32)
        if m.shape != (n_layers,):
            raise ValueError("onload_layer_map needs one entry per layer")
    _check("ess_prefill_layers", lib().ess_prefill_layers(
        n_layers, rows, n_hist, n_new, _ptr(host_kv), _ptr(new_kv), _ptr(bufs),
        _ptr(layer_out), _ptr(ws), ws.numel() * ws.element_size(),
        None if m is None else m.ctypes.data, binding.ctypes.data, compute_reps,
        1 if load_layer0 else 0, _stream(compute), _stream(h2d), _stream(d2h)))
    return binding
