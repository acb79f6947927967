"""Prefill over layers with four full-layer device buffers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (FlashOffloading analysis, prefill section, Fig. 2 and
Fig. 3):
  * host memory keeps every layer's full KV history; the device holds four
    full-layer buffers: B0 bound to layer 0 for the whole prefill, B1-B3
    rotating over the later layers through a binding table;
  * a layer l >= 1: bind a free buffer and load the layer's history (H2D);
    wait for that load before the layer's attention reads; append the
    chunk's new K/V into the buffer and compute over history + new rows;
    write the updated blocks back to host (D2H); the buffer can be reused
    only once its last compute and its D2H are both done, and that release
    can start the next load;
  * the scheduling parameter onload_layer_map[i] = j: at layer i's
    scheduling point, prefetch the future layer j;
  * Fig. 3: H2D loads L1..L5 into B1, B2, B3 and then reuses B1 and B2;
    compute starts at L0 from B0 without waiting; D2H idles while the first
    buffers are still being computed;
  * exposed load time >= max(0, tau_H2D - d_on * tau_compute), d_on the
    independent layer compute between a layer's prefetch and its use (the
    same with D2H and the reuse distance); with one shared copy path the
    transfer term is tau_H2D + tau_D2H.

Readings where the pages are silent:
  * the first buffers are bound before any compute: layers 1, 2, 3 to B1,
    B2, B3 in that order (as many as there are layers);
  * layer i >= 1 releases its buffer after its compute and its D2H; the
    released buffers form a queue, and if onload_layer_map[i] = j >= 0 the
    oldest released buffer is bound to layer j (default j = i + 3; -1 =
    nothing); a map that would load a layer twice, load a layer already
    computed, or leave a layer unloaded when its turn comes is invalid;
  * layer 0's history is in B0 before the prefill starts (bound for the
    whole prefill); it writes back its new rows like every layer;
  * the stand-in compute of a layer appends the chunk's new rows after the
    history and reduces every row of the buffer to per-column sums (a
    consumer whose result shows it saw exactly history + new rows); the
    D2H writes back the new rows only (the history on host is unchanged).
"""
import numpy as np

from .formats import decode_bf16

N_BUFFERS = 4


def schedule(n_layers, onload_layer_map=None):
    """Buffer of every layer, the layer whose release freed that buffer and
    the layer at whose scheduling point the load was issued (both -1 for
    the loads bound before any compute).  A load can start once its buffer
    is released and its scheduling layer is computed.  Raises ValueError
    for an invalid map."""
    if n_layers < 1:
        raise ValueError("n_layers < 1")
    bind = [-1] * n_layers
    freed_by = [-1] * n_layers
    trigger = [-1] * n_layers
    bind[0] = 0
    free = [(b, -1) for b in range(1, N_BUFFERS)]     # (buffer, released by)
    for layer in range(1, min(N_BUFFERS, n_layers)):
        bind[layer], freed_by[layer] = free.pop(0)
    for i in range(n_layers):
        if bind[i] < 0:
            raise ValueError(f"layer {i} is not loaded when its turn comes")
        if i == 0:
            continue
        free.append((bind[i], i))
        if onload_layer_map is None:
            j = i + N_BUFFERS - 1
            if j >= n_layers:
                continue
        else:
            j = int(onload_layer_map[i])
            if j < 0:
                continue
        if j <= i or j >= n_layers or bind[j] >= 0:
            raise ValueError(f"onload_layer_map[{i}] = {j} is not a future, unloaded layer")
        bind[j], freed_by[j] = free.pop(0)
        trigger[j] = i
    return bind, freed_by, trigger


def run(host_kv, new_kv, n_hist):
    """The prefill's effect on data.  host_kv: uint16 bf16 bits
    [NL][rows][576] with rows >= n_hist + n_new; new_kv: [NL][n_new][576].
    Returns (host_after, layer_out): host_after = host_kv with every
    layer's new rows written at [n_hist, n_hist + n_new); layer_out float64
    [NL][576] = column sums over the layer's history and new rows."""
    host_kv = np.asarray(host_kv)
    new_kv = np.asarray(new_kv)
    NL, n_new = new_kv.shape[0], new_kv.shape[1]
    after = host_kv.copy()
    out = np.zeros((NL, host_kv.shape[2]), np.float64)
    for layer in range(NL):
        rows = np.concatenate([host_kv[layer, :n_hist], new_kv[layer]], axis=0)
        out[layer] = decode_bf16(rows).sum(axis=0)
        after[layer, n_hist:n_hist + n_new] = new_kv[layer]
    return after, out


def exposed_bound(tau_transfer, tau_compute, d_layers):
    """The pages' lower bound on exposed transfer time of one layer."""
    return max(0.0, tau_transfer - d_layers * tau_compute)
