"""The C ABI library loads, exports every entry point include/ess.h declares,
and rejects bad arguments on the host before touching any GPU.  Runs
without a GPU: every call here fails validation before its first HIP call."""
import ctypes
import os
import re

import pytest

from decode_lightning_indexer_amd import ess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ess.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ess_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return ess.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ess.EXPORTED)


def _d(**kw):
    base = dict(batch=2, mtp=1, ctx_len=4096, idx_heads=16, idx_dim=64,
                mla_heads=16, topk=256, pool_slots=1024, softmax_scale=1 / 24)
    base.update(kw)
    return ess.make_dims(**base)


P = 0x1000   # never dereferenced: every call below fails validation first


def _status(call):
    with pytest.raises(ess.EssError) as e:
        call()
    return e.value.status


def test_sizes(L):
    d = _d()
    assert ess.ess_workspace_bytes(d) > 0
    lru = ess.ess_lru_state_bytes(d)
    assert lru >= 2 * (32 + 4 * 1024 + 8 * 4 * 1024)
    assert ess.ess_workspace_bytes(_d(lat_dim=512)) == 0


def test_null_and_bad_sizes(L):
    d = _d()
    assert _status(lambda: ess.ess_index_scores(d, 0, P, P, P, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_pool_reset(d, P, 0, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_index_scores(_d(batch=0), P, P, P, P, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_miss_copy(d, 0, P, P, P, P, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_topk_lookup(d, 8, 2, P, P, P, P, P, P, stream=0)) == "invalid argument"
    nan = _d(softmax_scale=float("nan"))
    assert _status(lambda: ess.ess_miss_copy(nan, 8, P, P, P, P, P, stream=0)) == "invalid argument"


def test_unsupported_shapes(L):
    assert _status(lambda: ess.ess_index_scores(_d(idx_dim=96), P, P, P, P, P, stream=0)) == "unsupported shape"
    assert _status(lambda: ess.ess_index_scores(_d(idx_heads=24), P, P, P, P, P, stream=0)) == "unsupported shape"
    assert _status(lambda: ess.ess_index_scores(_d(mtp=2, idx_heads=128), P, P, P, P, P, stream=0)) == "unsupported shape"
    assert _status(lambda: ess.ess_topk_lookup(_d(), 16385, 1, P, P, P, P, P, P, stream=0)) == "unsupported shape"
    assert _status(lambda: ess.ess_sparse_mla_decode(_d(mla_heads=24), P, P, P, P, P, P, P, P, P, P, 1 << 30, stream=0)) == "unsupported shape"
    assert _status(lambda: ess.ess_miss_copy(_d(lat_dim=512), 8, P, P, P, P, P, stream=0)) == "unsupported shape"


def test_capacity(L):
    d = _d(mtp=2, topk=600, pool_slots=1000)
    st = _status(lambda: ess.ess_pool_update(d, 600, 2, P, P, P, P, P, P, P, P, P, P, P, stream=0))
    assert st == "pool capacity exceeded"
    io = ess.ess_layer_io(*([P] * 22), 1 << 30)
    assert _status(lambda: ess.ess_decode_step(d, [io], P, ess.ESS_MODE_INLINE, stream=0, side=1)) == "pool capacity exceeded"


def test_workspace_too_small(L):
    # The attention needs its partials' part of the workspace (2 * 512 + 16
    # bytes per request, token, head and row chunk): one byte short is
    # refused.  The whole-step call needs all of ess_workspace_bytes.
    d = _d()
    need = ess.ess_workspace_bytes(d)
    st = _status(lambda: ess.ess_sparse_mla_decode(d, P, P, P, P, P, P, P, P, P, P, 1024, stream=0))
    assert st == "out of memory"
    msg = L.ess_last_error().decode()
    assert "workspace" in msg
    attn_need = int(msg.split("need ")[1].split()[0])
    assert attn_need <= need
    st = _status(lambda: ess.ess_sparse_mla_decode(d, P, P, P, P, P, P, P, P, P, P, attn_need - 1, stream=0))
    assert st == "out of memory"
    io = ess.ess_layer_io(*([P] * 22), need - 1)
    assert _status(lambda: ess.ess_decode_step(d, [io], P, ess.ESS_MODE_INLINE, stream=0, side=1)) == "out of memory"


def test_decode_step_argument_checks(L):
    d = _d()
    io = ess.ess_layer_io(*([P] * 22), 1 << 30)
    bad = ess.ess_layer_io(*([P] * 5 + [0] + [P] * 16), 1 << 30)
    assert _status(lambda: ess.ess_decode_step(d, [bad], P, ess.ESS_MODE_INLINE, stream=0, side=1)) == "invalid argument"
    assert _status(lambda: ess.ess_decode_step(d, [io], P, 7, stream=0, side=1)) == "invalid argument"
    assert _status(lambda: ess.ess_decode_step(d, [io], P, ess.ESS_MODE_PREFETCH, stream=5, side=5)) == "invalid argument"
    assert _status(lambda: ess.ess_decode_step(_d(pool_slots=20000, topk=256), [io], P, ess.ESS_MODE_FILL, stream=0, side=1)) == "unsupported shape"


def test_status_strings(L):
    for code, text in ((0, "ok"), (-3, "pool capacity exceeded"), (-4, "HIP runtime error")):
        assert L.ess_status_string(code).decode() == text


def _split_row_bytes(spans, k):
    # Control words (512 B) and four 2048-bin histograms, two counts per
    # span (128-byte aligned), 64 candidate keys, k winners; 256-aligned.
    win = 512 + 4 * 2048 * 4 + -(-spans * 8 // 128) * 128 + 64 * 8
    return -(-(win + 8 * k) // 256) * 256


def test_long_rows_need_a_topk_workspace(L):
    # Rows over 32768 keys with k <= 4096 select either split over
    # workgroups that exchange counts and winners through the workspace, or
    # in levels whose candidate lists (two buffers of keys and positions, k
    # per 16384-key chunk and row) sit there; the region after the
    # attention's partials holds the larger of the two, for the step's top-k
    # and for the first fill's top-C (n_tok = 1).
    short = _d(topk=2048, pool_slots=4096)
    long_ = _d(ctx_len=100000, topk=2048, pool_slots=4096)
    chunks = -(-100000 // 16384)
    step = 4 * (2 * 1) * chunks * 2048 * 4       # B=2 rows, k=2048
    fill = 4 * (2 * 1) * chunks * 4096 * 4       # k=C=4096
    split = 2 * _split_row_bytes(chunks, 4096)
    assert ess.ess_workspace_bytes(long_) - ess.ess_workspace_bytes(short) == max(step, fill, split)
    # Few candidates per chunk: the split selection's exchange area is larger.
    few = _d(batch=1, ctx_len=40000, topk=64, pool_slots=64)
    few_short = _d(batch=1, topk=64, pool_slots=64)
    lv = 4 * 1 * 3 * 64 * 4
    sp = _split_row_bytes(3, 64)
    assert sp > lv
    assert ess.ess_workspace_bytes(few) - ess.ess_workspace_bytes(few_short) == \
        -(-sp // 256) * 256
    # k > 4096 never uses levels.
    assert ess.ess_workspace_bytes(_d(ctx_len=100000, topk=8192, pool_slots=16384)) == \
        ess.ess_workspace_bytes(_d(topk=8192, pool_slots=16384))
    st = _status(lambda: ess.ess_topk_lookup(long_, 2048, 1, P, P, P, P, P, P, stream=0))
    assert st == "out of memory"
    assert "workspace" in L.ess_last_error().decode()
    st = _status(lambda: ess.ess_topk_lookup(long_, 2048, 1, P, P, P, P, P, P, P + 4, 1 << 30, stream=0))
    assert st == "invalid argument"


def test_prefill_argument_checks(L):
    import torch
    ws = torch.empty(ess.ess_prefill_ws_bytes(100), dtype=torch.uint8)   # host: never used
    small = torch.empty(16, dtype=torch.uint8)

    def call(NL=6, rows=100, n_hist=80, n_new=20, ws=ws, m=None, streams=(1, 2, 3)):
        return _status(lambda: ess.ess_prefill_layers(
            NL, rows, n_hist, n_new, P, P, P, P, ws, onload_layer_map=m,
            compute=streams[0], h2d=streams[1], d2h=streams[2]))
    assert call(n_hist=90) == "invalid argument"            # 90 + 20 > 100 rows
    assert call(NL=0) == "invalid argument"
    assert call(streams=(1, 1, 3)) == "invalid argument"
    assert call(ws=small) == "out of memory"
    assert call(m=[-1, 4, 4, -1, -1, -1]) == "invalid argument"   # layer 4 twice
    assert call(m=[-1, -1, -1, -1, -1, -1]) == "invalid argument"  # 4, 5 never loaded
    assert "not loaded" in L.ess_last_error().decode()
    assert ess.ess_prefill_ws_bytes(0) == 0
    assert ess.ess_prefill_ws_bytes(128) == 576 * 4 and ess.ess_prefill_ws_bytes(129) == 2 * 576 * 4


def test_entry_copy_argument_checks(L):
    d = _d()
    st = lambda *a: _status(lambda: ess.ess_miss_copy_entries(*a, stream=0))
    assert st(d, 0, P, P, P, P, P) == "invalid argument"          # list_stride
    assert st(d, 8, P, P, P, 0, P) == "invalid argument"          # no entries
    assert st(d, 8, P, P, P, P + 8, P) == "invalid argument"      # misaligned
    assert st(_d(lat_dim=512), 8, P, P, P, P, P) == "unsupported shape"
    # A layer with neither a bf16 store nor entries, and one whose entries
    # are misaligned, are rejected by the whole step.
    none = ess.ess_layer_io(*([P] * 4 + [0] + [P] * 17), 1 << 30, None)
    mis = ess.ess_layer_io(*([P] * 4 + [0] + [P] * 17), 1 << 30, P + 8)
    for io in (none, mis):
        assert _status(lambda: ess.ess_decode_step(d, [io], P, ess.ESS_MODE_INLINE,
                                                   stream=0, side=1)) == "invalid argument"


def test_tail_argument_checks(L):
    d = _d()
    B = d.batch
    assert _status(lambda: ess.ess_tail_init(d, 0, 8, [100] * B, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_tail_init(d, P, 0, [100] * B, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_tail_init(d, P, 8, [0] * B, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_tail_init(d, P, 8, [5000] * B, P, stream=0)) == "invalid argument"
    st = lambda dd, tt, s1, s2: _status(lambda: ess.ess_append_tokens(
        dd, tt, P, P, P, P, P, stream=s1, d2h=s2))
    assert st(d, ess.ess_tail(), 1, 2) == "invalid argument"          # not initialised
    lens = (ctypes.c_int32 * (3 * B))(*([100] * B + [100] * B + [100] * B))
    t = ess.ess_tail(P, None, 8, B, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)), P, P)
    assert st(d, t, 3, 3) == "invalid argument"                       # one stream for both
    assert st(_d(batch=3), t, 1, 2) == "invalid argument"             # batch differs
    t1 = ess.ess_tail(P, None, 1, B, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)), P, P)
    assert st(_d(mtp=2, idx_heads=16), t1, 1, 2) == "unsupported shape"   # block < mtp
    lens[B + 1] = 4096                                                # request 1 is full
    assert st(d, t, 1, 2) == "invalid argument"
    io = ess.ess_layer_io(*([P] * 22), 1 << 30, None, P, P, 0)         # tail_block 0
    assert _status(lambda: ess.ess_decode_step(d, [io], P, ess.ESS_MODE_INLINE,
                                               stream=0, side=1)) == "invalid argument"
    io = ess.ess_layer_io(*([P] * 22), 1 << 30, None, P, None, 16)     # no tail_start
    assert _status(lambda: ess.ess_decode_step(d, [io], P, ess.ESS_MODE_INLINE,
                                               stream=0, side=1)) == "invalid argument"


def test_tail_entries_must_be_aligned(L):
    d = _d()
    assert _status(lambda: ess.ess_tail_init(d, P, 8, [100] * d.batch, P, stream=0,
                                             entries=P + 8)) == "invalid argument"


def test_fill_takes_no_tail(L):
    io = ess.ess_layer_io(*([P] * 22), 1 << 30, None, P, P, 16)
    assert _status(lambda: ess.ess_decode_step(_d(), [io], P, ess.ESS_MODE_FILL,
                                               stream=0, side=1)) == "invalid argument"


def test_struct_layouts_match_the_header(tmp_path):
    # The ctypes mirrors of the ABI structs have the sizes and field offsets
    # a C compiler gives the declarations in include/ess.h.
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs gcc and the HIP headers")
    fields = {"ess_dims": ess.ess_dims, "ess_layer_io": ess.ess_layer_io, "ess_tail": ess.ess_tail}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "ess.h"', "int main(void) {"]
    for name, cls in fields.items():
        lines.append(f'  printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for name, cls in fields.items():
        assert int(got[name]) == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(cls, f).offset, (name, f)


def test_a_c_program_calls_the_library(tmp_path):
    # The library used from C with nothing but include/ess.h: a host-only
    # call (the eviction replay) on a small recorded run gives what the
    # Python binding gives, and the status strings come back.
    import shutil
    import subprocess
    import numpy as np
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs gcc and the HIP headers")
    T, m, Lc, k, C = 3, 1, 12, 4, 6
    rng = np.random.default_rng(4)
    scores = rng.standard_normal((T, m, Lc)).astype(np.float32)
    sel = np.argsort(-scores, axis=2, kind="stable")[:, :, :k].astype(np.int32)
    n_sel = np.full((T, m), k, np.int32)
    want_miss, want_ev = ess.ess_replay_evictions(ess.ESS_EVICT_LRU, C, scores, sel, n_sel)
    arr = lambda a, t: "{" + ", ".join(f"{x}{t}" for x in a.ravel().tolist()) + "}"
    src = tmp_path / "use.c"
    src.write_text(f"""#include <stdio.h>
#include "ess.h"
int main(void) {{
  const float scores[] = {arr(scores, "f")};
  const int32_t sel[] = {arr(sel, "")};
  const int32_t n_sel[] = {arr(n_sel, "")};
  int32_t n_miss[{T}], n_evict[{T}];
  ess_status s = ess_replay_evictions(ESS_EVICT_LRU, {Lc}, {C}, {T}, {m}, {k}, scores, sel,
                                      n_sel, 0, 0, n_miss, n_evict);
  printf("%s\\n", ess_status_string(s));
  for (int t = 0; t < {T}; ++t) printf("%d %d\\n", n_miss[t], n_evict[t]);
  s = ess_replay_evictions(ESS_EVICT_LRU, {Lc}, 1, {T}, {m}, {k}, scores, sel, n_sel, 0, 0,
                           n_miss, n_evict);
  printf("%s\\n", ess_status_string(s));
  return 0;
}}
""")
    libdir = os.path.join(ROOT, "decode_lightning_indexer_amd")
    exe = tmp_path / "use"
    subprocess.run([gcc, "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), ess.LIB_PATH,
                    f"-Wl,-rpath,{libdir}", "-Wl,--allow-shlib-undefined", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    assert out[0] == "ok"
    for t in range(T):
        assert out[1 + t].split() == [str(want_miss[t]), str(want_ev[t])]
    assert out[1 + T] != "ok"            # a pool smaller than k is refused


def test_pool_status_copy_and_release_checks(L):
    d = _d()
    assert _status(lambda: ess.ess_pool_status(d, 0, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_pool_status(d, P, 0, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_pool_status(_d(batch=0), P, P, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_copy_async(0, P, 16, stream=0)) == "invalid argument"
    assert _status(lambda: ess.ess_copy_async(P, 0, 16, stream=0)) == "invalid argument"
    # Zero bytes enqueue nothing; a thread that created no events releases
    # nothing.  Neither touches the GPU.
    ess.ess_copy_async(P, P, 0, stream=0)
    ess.ess_thread_release()


def test_lru_header_layout(L):
    # Per request: a 32-byte header (head, tail, free_head, epoch, cap, err,
    # compactions, pad), C int32 stamps and a ring of 4C (slot, stamp) pairs,
    # rounded up to 256 bytes; ess_pool_status reads the header fields.
    for C in (1024, 1000, 8192):
        d = _d(pool_slots=C)
        per = -(-(32 + 4 * C + 8 * 4 * C) // 256) * 256
        assert ess.ess_lru_state_bytes(d) == 2 * per


def test_long_context_is_accepted_up_to_2_28(L):
    # Contexts up to 2^28 positions pass the host checks (the kernels use
    # 64-bit offsets into every [B][L][...] array); beyond, unsupported.
    big = _d(ctx_len=(1 << 28), idx_dim=128)
    assert _status(lambda: ess.ess_index_scores(big, 0, P, P, P, P, stream=0)) == "invalid argument"
    over = _d(ctx_len=(1 << 28) + 1, idx_dim=128)
    assert _status(lambda: ess.ess_index_scores(over, P, P, P, P, P, stream=0)) == "unsupported shape"


def test_noalloc_refuses_dims_beyond_its_array(L):
    # The no-allocation attention holds 24 MiB of partials per device: dims
    # needing more are refused on the host, anything smaller passes the size
    # check (and here fails on a NULL pointer instead).
    big = _d(batch=64, mla_heads=128, topk=2048, pool_slots=4096)
    st = _status(lambda: ess.ess_sparse_mla_decode_noalloc(big, P, P, P, P, P, P, P, P, P, stream=0))
    assert st == "out of memory" and "scratch" in L.ess_last_error().decode()
    small = _d(batch=16, mla_heads=128, topk=2048, pool_slots=8192)
    st = _status(lambda: ess.ess_sparse_mla_decode_noalloc(small, P, P, P, P, P, P, 0, P, P, stream=0))
    assert st == "invalid argument"
