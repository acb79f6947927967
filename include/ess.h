/*
 * ess.h - C ABI of the MI355X (gfx950) sparse-decode library.
 *
 * One decode step of DSA-style sparse attention over a latent cache whose
 * authoritative copy lives in pinned host memory.  Per layer and per query
 * token the step runs:
 *   1. lightning-indexer scores over every cached position  (ess_index_scores)
 *   2. top-k selection with the cache_slots lookup fused    (ess_topk_lookup)
 *   3. residency update of the hot pool (union, victims,
 *      pairing, cache_slots rewrite, copy list)              (ess_pool_update)
 *   4+5. gather of the selected latents - hits from the pool
 *      in device memory, misses straight from mapped host
 *      memory - and absorbed-MLA attention over them         (ess_sparse_mla_decode)
 * plus a standalone host->pool copy of a miss list (ess_miss_copy, and
 * ess_miss_copy_entries from 656-byte fp8 entries), a whole-step entry point
 * over several layers with side-stream prefetch (ess_decode_step), a growing
 * context with device tail blocks (ess_tail_init, ess_append_tokens), the
 * prefill four-buffer pipeline (ess_prefill_layers) and an offline replay of
 * the pool under other eviction policies (ess_replay_evictions).
 *
 * Sources: the ESS concept page ("ESS: Latent-Cache Offload", tables "dual
 * cache" and "core mechanism") and the FlashOffloading analysis
 * (hwcomputing.csdn.net; sections "cache_slots", "five steps and the MTP
 * union", "LIM: packing the index into the score", "forking inside
 * KVgather", Figs. 4-6).  Each call below names the passage it follows.
 *
 * Conventions for every call:
 *   - All array arguments are device pointers (or, for host_view, the device
 *     view of mapped pinned host memory from ess_host_alloc), owned by the
 *     caller.  The library keeps no pointer after the call returns and
 *     allocates no device memory in these calls; scratch space is a caller
 *     workspace sized by ess_workspace_bytes.
 *   - Arguments are checked on the host before anything is enqueued.  A
 *     nonzero status means nothing was enqueued; ess_last_error() holds a
 *     message.  The contents of the arrays are not checked (positions must be
 *     < ctx_len, n_vis in [1, ctx_len]); a launch failure reported by the HIP
 *     runtime returns ESS_ERR_HIP.
 *   - Every call is asynchronous on the given stream; counts such as n_sel
 *     and n_miss stay in device memory.  Calls from different host threads
 *     may run at once (on different buffers): the events a call uses to
 *     order its streams belong to the calling thread.
 *   - Layouts are row-major with the listed shapes; "bf16" arrays are passed
 *     as uint16_t bit patterns; fp8 arrays are OCP e4m3fn bytes.
 */
#ifndef ESS_H
#define ESS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem shape of one layer.
 *   batch      B  requests
 *   mtp        m  query tokens per step per request (MTP ways sharing a pool;
 *                 1 .. 4)
 *   ctx_len    L  cached positions per request (1 .. 2^28; offsets into
 *                 every [B][L][...] array are 64-bit)
 *   idx_heads  H_I indexer heads (multiple of 16; mtp*idx_heads <= 128)
 *   idx_dim    d_I indexer dimension (64 or 128)
 *   mla_heads  H  absorbed-MLA query heads (16, 32, 48, ... 128)
 *   lat_dim    576 = c_KV[512] + k_R[64]
 *   v_dim      512
 *   topk       k  (1 .. 16384)
 *   pool_slots C  hot-pool slots per request (mtp*topk <= C <= 2^20 - 2)
 *   softmax_scale  multiplies the latent dot products before the softmax */
typedef struct ess_dims {
  int32_t batch, mtp, ctx_len, idx_heads, idx_dim, mla_heads;
  int32_t lat_dim, v_dim, topk, pool_slots;
  float softmax_scale;
} ess_dims;

typedef enum ess_status {
  ESS_OK = 0,
  ESS_ERR_INVALID = -1,      /* null pointer, bad size or count            */
  ESS_ERR_UNSUPPORTED = -2,  /* shape outside what the kernels implement   */
  ESS_ERR_CAPACITY = -3,     /* union of the ways could exceed the pool    */
  ESS_ERR_HIP = -4,          /* HIP runtime error (launch or earlier fault) */
  ESS_ERR_NOMEM = -5         /* host allocation failed / workspace too small */
} ess_status;

/* Bytes of workspace the calls below need for these dims: the attention's
 * split-row partials, then (ctx_len > 32768 with topk or pool_slots <= 4096)
 * the top-k's exchange area for rows split over several workgroups or the
 * candidate lists of its levels, whichever is larger, then each token's
 * winners in position order for a step with several tokens.  One workspace
 * serves one stream at a time; it must be 16-byte aligned. */
size_t ess_workspace_bytes(const ess_dims* d);

/* Bytes of the opaque per-layer LRU state (B requests): per request a header,
 * one recency stamp per slot and a ring of (slot, stamp) entries. */
size_t ess_lru_state_bytes(const ess_dims* d);

/* Empty pool: cache_slots[B][L] = -1, slot_pos[B][C] = -1, every slot free,
 * recency ring empty.  Call before the first fill of a request batch. */
ess_status ess_pool_reset(const ess_dims* d, int32_t* cache_slots,
                          int32_t* slot_pos, void* lru_state,
                          hipStream_t stream);

/* Health of the pool state after the updates so far, per request, for
 * diagnosing caller errors (FlashOffloading analysis, "five steps and the MTP
 * union": every miss is paired with one victim, so the pool size stays C).
 * Writes status [B][4] int32 (device memory) on the stream:
 *   [0] err: 0 consistent; 1 an update found fewer victims than misses
 *       (the state was corrupted, e.g. by a foreign write): its unpaired
 *       misses are left out of the copy list, n_miss counts the paired
 *       ones only, and those rows stay unresident; 2 a selected position was
 *       outside [0, ctx_len) (it was dropped);
 *   [1] times the recency ring was compacted since ess_pool_reset;
 *   [2] updates applied since ess_pool_reset (the first fill included);
 *   [3] entries on the recency ring (live and dead). */
ess_status ess_pool_status(const ess_dims* d, const void* lru_state,
                           int32_t* status, hipStream_t stream);

/* Indexer scores (the indexer scores all L positions every step: ESS concept
 * page, "dual cache" table; score form: the DSA lightning indexer):
 *   scores[b][j][s] = sum_h w[b][j][h] * max(0, sum_d q[b][j][h][d] * k[b][s][d])
 * for s < n_vis[b][j], and -inf for n_vis[b][j] <= s < L.
 *   q_fp8   [B][m][H_I][d_I]  fp8 e4m3fn
 *   w       [B][m][H_I]       float
 *   k_fp8   [B][L][d_I]       fp8 e4m3fn (the resident index cache)
 *   n_vis   [B][m]            int32 in [1, L]
 *   scores  [B][m][L]         float (output)
 * Accumulation is fp32 via fp8 MFMA; integer-valued inputs whose partial
 * sums stay below 2^24 give exact integer scores. */
ess_status ess_index_scores(const ess_dims* d, const uint8_t* q_fp8,
                            const float* w, const uint8_t* k_fp8,
                            const int32_t* n_vis, float* scores,
                            hipStream_t stream);

/* Top-k of each of the first n_tok query tokens of every request, with the
 * residency lookup read off the winners (FlashOffloading analysis, section
 * "LIM: packing the index into the score", 20-candidate example).
 *   n_sel[b][j]    = min(k, n_vis[b][j])
 *   sel_pos[b][j][i], i < n_sel: positions of the n_sel largest scores in
 *                  rank order (score descending; equal scores: lower
 *                  position first); -1 beyond n_sel
 *   sel_slot[b][j][i] = cache_slots[b][sel_pos] before this step's update
 *                  (-1: not resident); -1 beyond n_sel
 * Inputs scores [B][m][L], n_vis [B][m], cache_slots [B][L]; outputs
 * sel_pos, sel_slot [B][n_tok][k] and n_sel [B][n_tok].  1 <= n_tok <= m,
 * 1 <= k <= 16384.  Scores must not be NaN.  Rows of at most 32768 keys,
 * and any k > 4096, select in on-chip memory (ws and ws_bytes are not used;
 * NULL and 0 are fine).  Longer rows with k <= 4096 use ws: each row is
 * split over workgroups of 16384 keys that select together, exchanging
 * counts and winners through ws (when B * n_tok * ceil(L / 16384) is at most
 * half the device's compute units), or else is reduced in levels - each
 * 16384-key chunk's top-k is written to ws as candidates until one
 * workgroup holds the row's list.  ws must then hold
 * ess_workspace_bytes(d) bytes (enough for k = d->topk with n_tok <=
 * d->mtp, and for k = d->pool_slots with n_tok = 1), else ESS_ERR_NOMEM.
 * The split selection needs all workgroups of a row resident at once; its
 * waits are bounded, and a row whose wait ran out (only possible when other
 * work holds the compute units for seconds) is returned with n_sel = 0 and
 * no selection. */
ess_status ess_topk_lookup(const ess_dims* d, int32_t k, int32_t n_tok,
                           const float* scores, const int32_t* n_vis,
                           const int32_t* cache_slots, int32_t* sel_pos,
                           int32_t* sel_slot, int32_t* n_sel, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Residency update of the hot pool for one step (FlashOffloading analysis,
 * section "five steps and the MTP union": lookup per way, union of the
 * misses, as many victims as misses from the pool minus the union, one-to-one
 * pairing and cache_slots rewrite; ESS concept page: LRU hot pool).  Per
 * request b, with U = the union of sel_pos[b][j][0..n_sel) over j < n_tok:
 *   misses M = positions of U not resident, ascending;
 *   victims  = free slots in ascending order, then resident positions outside
 *              U from the least-recently-used end (recency: the last update
 *              whose union held the position; within one update, ascending
 *              position order);
 *   M[i] is paired with victim i: cache_slots[M[i]] = slot,
 *   slot_pos[slot] = M[i]; evicted positions get cache_slots = -1.
 * Outputs per request: miss_pos[b][i], miss_slot[b][i] for i < n_miss[b]
 * (capacity n_tok*k entries per request, the copy list host -> pool),
 * n_evict[b] (victims taken from resident positions), and per row
 * [B][n_tok][k]: row_dst = the paired slot on the one row (smallest j, then
 * its row) that is the designated writer of a miss, else -1;
 * sel_slot_post = cache_slots after the update (-1 beyond n_sel).
 * The first fill is this call with n_tok = 1, k = C on an empty pool: slot i
 * receives the i-th smallest selected position.  Requires n_tok*k <= C
 * (else ESS_ERR_CAPACITY).  Calls on one lru_state must be ordered. */
ess_status ess_pool_update(const ess_dims* d, int32_t k, int32_t n_tok,
                           const int32_t* sel_pos, const int32_t* n_sel,
                           int32_t* cache_slots, int32_t* slot_pos,
                           void* lru_state, int32_t* miss_pos,
                           int32_t* miss_slot, int32_t* n_miss,
                           int32_t* n_evict, int32_t* row_dst,
                           int32_t* sel_slot_post, hipStream_t stream);

/* Gather + absorbed-MLA attention over the selected latents (ESS concept
 * page, "dual cache" table: only the top-k latents are read; FlashOffloading
 * analysis, section "forking inside KVgather": hits from device memory, misses
 * straight from pinned host memory, a miss written to its slot and the
 * on-chip tile together).  For each b, j < m, h < H, over i < n_sel[b][j]:
 *   row_i = pool[b][sel_src[i]] if sel_src[i] >= 0
 *           else host_view[b][sel_pos[i]]            (576 bf16)
 *   z_i   = softmax_scale * <q_abs[b][j][h], row_i>
 *   out[b][j][h][:] = sum_i softmax(z)_i * row_i[0:512]
 *   lse[b][j][h]    = log sum_i exp(z_i)                 (lse may be NULL)
 * If row_dst is not NULL, every miss row (sel_src[i] < 0, i < n_sel) with
 * row_dst[i] >= 0 is in pool[b][row_dst[i]] when the call's work completes
 * (that slot must be one no other selected row reads, as the slots from
 * ess_pool_update are): the attention kernel reads such a row from host
 * memory into its tile and writes it to the slot from there (one host read
 * per miss, under the attention's own work).  Every miss row, whoever
 * writes it, is read from host memory inside the attention kernel.  The
 * reduction order is the rank order in fixed chunks combined in fixed
 * order, so the result does not depend on which rows came from host
 * memory.
 *   q_abs [B][m][H][576] bf16; sel_pos, sel_src, row_dst [B][m][k];
 *   n_sel [B][m]; pool [B][C][576] bf16; host_view [B][L][576] bf16;
 *   out [B][m][H][512] float; lse [B][m][H] float. */
ess_status ess_sparse_mla_decode(const ess_dims* d, const uint16_t* q_abs,
                                 const int32_t* sel_pos,
                                 const int32_t* sel_src,
                                 const int32_t* row_dst, const int32_t* n_sel,
                                 uint16_t* pool, const uint16_t* host_view,
                                 float* out, float* lse, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* ess_sparse_mla_decode for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and result, with
 * the split-row partials in a fixed scratch array of 24 MiB that the library
 * holds on each device it runs on, from its first use there until the
 * process ends.  No allocation happens in the call.  Dims whose partials
 * exceed it (ess_workspace_bytes's attention part: 2 * 512 + 16 bytes per
 * request, token, head and row chunk) are refused with ESS_ERR_NOMEM before
 * anything is enqueued.  Every call on one device shares that device's
 * array: calls that overlap on one device (on different streams or host
 * threads) race and give wrong results; order them.  Other arguments and
 * errors as in ess_sparse_mla_decode. */
ess_status ess_sparse_mla_decode_noalloc(const ess_dims* d, const uint16_t* q_abs,
                                         const int32_t* sel_pos,
                                         const int32_t* sel_src,
                                         const int32_t* row_dst,
                                         const int32_t* n_sel, uint16_t* pool,
                                         const uint16_t* host_view, float* out,
                                         float* lse, hipStream_t stream);

/* The same with a host store of 656-byte fp8 latent entries (layout under
 * ess_miss_copy_entries): every miss row (sel_src[i] < 0) is read from
 * entry_view[b][sel_pos[i]] (656 bytes over the host link) and dequantized in
 * the attention's on-chip tile, so row_i is the dequantized entry; a
 * designated-writer miss is written to its slot as those bf16 values.
 * entry_view [B][L][656], 16-byte aligned.  Other arguments, the reduction
 * order and the errors as in ess_sparse_mla_decode. */
ess_status ess_sparse_mla_decode_entries(const ess_dims* d,
                                         const uint16_t* q_abs,
                                         const int32_t* sel_pos,
                                         const int32_t* sel_src,
                                         const int32_t* row_dst,
                                         const int32_t* n_sel, uint16_t* pool,
                                         const uint8_t* entry_view, float* out,
                                         float* lse, void* ws, size_t ws_bytes,
                                         hipStream_t stream);

/* Copy a miss list from host memory into the pool (the pages' step 5, the
 * H2D load of the copy triples; ESS concept page: small-block transfers of
 * latent entries).  For each b and i < n_miss[b]:
 *   pool[b][miss_slot[b*list_stride + i]] = host_view[b][miss_pos[b*list_stride + i]]
 * Used for the first fill. */
ess_status ess_miss_copy(const ess_dims* d, int32_t list_stride,
                         const int32_t* miss_pos, const int32_t* miss_slot,
                         const int32_t* n_miss, const uint16_t* host_view,
                         uint16_t* pool, hipStream_t stream);

/* The same copy from 656-byte fp8 latent entries (ESS concept page,
 * FlashTrans row: transfers of 656-byte blocks; the layout is this library's
 * reading of that size).  entry_view [B][L][656] bytes, 16-byte aligned,
 * mapped pinned host memory (or device memory); entry s of request b is
 *   bytes [0, 512)    c_KV as OCP e4m3fn
 *   bytes [512, 528)  four float32 scales, scale j for c_KV[128j, 128j+128)
 *   bytes [528, 656)  k_R as 64 bf16
 * For each b and i < n_miss[b], with p = miss_pos[b*list_stride + i]:
 *   pool[b][miss_slot[b*list_stride + i]][c] = bf16(e4m3(entry[p].c_KV[c]) *
 *       scale[c / 128])      for c < 512   (round to nearest even)
 *   pool[b][...][512 + r] = entry[p].k_R[r]      for r < 64
 * With power-of-two scales and products in bf16's normal range the pool row
 * is the dequantized entry exactly.  Each entry is read from host memory
 * once (656 bytes instead of a 1152-byte bf16 row). */
ess_status ess_miss_copy_entries(const ess_dims* d, int32_t list_stride,
                                 const int32_t* miss_pos,
                                 const int32_t* miss_slot,
                                 const int32_t* n_miss,
                                 const uint8_t* entry_view, uint16_t* pool,
                                 hipStream_t stream);

/* One layer's buffers for ess_decode_step.  Shapes as in the calls above;
 * miss_pos/miss_slot hold max(m*k, C) entries per request (the fill needs C);
 * sel_* and row_dst hold max(m*k, C) entries per request too. */
typedef struct ess_layer_io {
  const uint8_t* q_idx;       /* [B][m][H_I][d_I] fp8 */
  const float* w_idx;         /* [B][m][H_I] */
  const uint8_t* k_idx;       /* [B][L][d_I] fp8 */
  const uint16_t* q_abs;      /* [B][m][H][576] bf16 */
  const uint16_t* host_view;  /* [B][L][576] bf16, mapped pinned host */
  uint16_t* pool;             /* [B][C][576] bf16 */
  int32_t* cache_slots;       /* [B][L] */
  int32_t* slot_pos;          /* [B][C] */
  void* lru_state;            /* ess_lru_state_bytes */
  float* scores;              /* [B][m][L] */
  int32_t* sel_pos;           /* [B][m][k] (fill: [B][C]) */
  int32_t* sel_slot;
  int32_t* n_sel;             /* [B][m] */
  int32_t* row_dst;           /* [B][m][k] (fill: [B][C]) */
  int32_t* sel_slot_post;
  int32_t* miss_pos;          /* [B][max(m*k, C)] */
  int32_t* miss_slot;
  int32_t* n_miss;            /* [B] */
  int32_t* n_evict;           /* [B] */
  float* out;                 /* [B][m][H][512] */
  float* lse;                 /* [B][m][H] or NULL */
  void* ws;                   /* ess_workspace_bytes, one per layer */
  size_t ws_bytes;
  const uint8_t* host_entries;  /* [B][L][656] fp8 entries (mapped pinned
                                   host) or NULL.  Non-NULL: the host store
                                   holds entries instead of bf16 rows
                                   (host_view may then be NULL): the
                                   attention reads misses as entries and
                                   dequantizes them in its tile
                                   (ess_sparse_mla_decode_entries), the
                                   fill copies with ess_miss_copy_entries. */
  const uint16_t* tail_rows;  /* growing context: the tail blocks
                                 (ess_tail.rows) or NULL */
  const int32_t* tail_start;  /* device [B]: ess_tail.state_dev + 2*B; a
                                 request's positions from its start on are
                                 read from tail_rows instead of host memory */
  int32_t tail_block;         /* ess_tail.block.  ESS_MODE_FILL takes no
                                 tail (it reads every row from the host
                                 store).  With host_entries the tail must
                                 have entries too. */
} ess_layer_io;

enum {
  ESS_MODE_FILL = 0,     /* first fill: top-C of token 0, empty-pool update,
                            host -> pool copy; no attention                  */
  ESS_MODE_INLINE = 1,   /* per layer on `stream`: scores, top-k, pool update,
                            then gather + attention: the attention reads
                            each miss from host memory and writes it to its
                            slot from the tile                              */
  ESS_MODE_PREFETCH = 2  /* every layer's scores, top-k and update run ahead
                            on `side`; `stream` runs layer l's gather +
                            attention (as in ESS_MODE_INLINE) as soon as
                            layer l is selected, so layer l+1's selection
                            overlaps layer l's miss transfer and attention  */
};

/* A whole decode step over n_layers layers (ESS concept page: layer-wise
 * compute/transfer overlap; the FlashOffloading analysis's decode layer
 * order LIM -> CopySFA, Fig. 5).  n_vis [B][m] is shared by all layers.
 * In ESS_MODE_PREFETCH, `side` must be a different stream from `stream`;
 * on return all work is ordered before later work on `stream`. */
ess_status ess_decode_step(const ess_dims* d, int32_t n_layers,
                           const ess_layer_io* layers, const int32_t* n_vis,
                           int32_t mode, hipStream_t stream,
                           hipStream_t side);

/* Growing context (FlashOffloading analysis, architecture section and
 * Fig. 2: beside the C-slot hot cache the decode side keeps two tail blocks
 * of new KV; host memory holds the authoritative copy, written back by
 * block).  Each step appends every request's m tokens: their index keys go
 * to the resident index cache and their latents to the request's open tail
 * block in device memory.  When a block fills it is copied to the host store
 * on a stream of its own; its rows stay readable from the tail until the
 * block after next reuses its buffer, which first waits for that copy.  The
 * pool's residency rules do not change: a selected position from the
 * request's `start` on that misses the pool is read from its tail row
 * (device memory) instead of host memory, and written to its slot as any
 * miss.  Requests may be at different lengths.
 *
 * State of one layer's tail (fields owned by the library between
 * ess_tail_init and ess_tail_release):
 *   rows      [B][2*block][576] bf16 device memory (caller-owned); position
 *             p >= start[b] of request b lives in its row
 *             ((p / block) % 2) * block + p % block
 *   entries   NULL for a host store of bf16 rows; for a store of 656-byte
 *             fp8 entries, [B][2*block][656] device memory (caller-owned,
 *             16-byte aligned): each appended latent is quantized there
 *             (block scale = the smallest power of two s with
 *             max|c_KV| <= 448 s, 1 for an all-zero block; codes = the
 *             nearest e4m3fn value of x / s, ties to the even code; k_R
 *             as is), its tail row holds the entry dequantized, and the
 *             write-back copies entries
 *   host      [3][B] int32 host copy of (first, n_ctx, start): first = the
 *             length the tail started at (positions below it are already
 *             in the host store), n_ctx = current length, start = first
 *             position read from the tail
 *   state_dev [3][B] int32 device memory (caller-owned): the same, kept
 *             current on the stream by ess_append_tokens; the attention
 *             reads start from it (ess_layer_io.tail_start = state_dev + 2B)
 *   events    2B write-back events */
typedef struct ess_tail {
  uint16_t* rows;
  uint8_t* entries;
  int32_t block, batch;
  int32_t* host;
  int32_t* state_dev;
  void** events;
} ess_tail;

/* Start a tail for d->batch requests at lengths n_ctx[B] (host array, each
 * in [1, ctx_len]) with blocks of `block` >= 1 tokens.  Allocates the host
 * arrays and creates the events; writes state_dev and waits for that copy
 * on `stream`.  ESS_ERR_NOMEM / ESS_ERR_HIP if that fails. */
ess_status ess_tail_init(ess_tail* t, const ess_dims* d, uint16_t* rows,
                         uint8_t* entries, int32_t block, const int32_t* n_ctx,
                         int32_t* state_dev, hipStream_t stream);
/* Free the tail's host arrays and events (its copies must have completed). */
ess_status ess_tail_release(ess_tail* t);

/* Append the step's m = d->mtp tokens of every request b at positions
 * n_ctx[b] .. n_ctx[b] + m - 1:
 *   k_idx[b][n_ctx + j] = new_keys[b][j]      ([B][m][d_I] fp8 -> [B][L][d_I])
 *   tail row of n_ctx + j = new_lat[b][j]     ([B][m][576] bf16)
 *   n_vis[b][j] = n_ctx + 1 + j               (token j sees up to itself)
 * on `stream`; every tail block this fills is copied to host_store[b][p]
 * (the host store's CPU address: [B][L][576] bf16, or [B][L][656] entries
 * when the tail has entries) for its positions p >= first[b], on `d2h` (a
 * different stream).  Then n_ctx[b] += m and start[b] = max(first,
 * start of the block before the newest one), in both copies of the state.
 * Requires m <= block and n_ctx[b] + m <= ctx_len. */
ess_status ess_append_tokens(const ess_dims* d, ess_tail* t,
                             const uint8_t* new_keys, const uint16_t* new_lat,
                             uint8_t* k_idx, int32_t* n_vis, void* host_store,
                             hipStream_t stream, hipStream_t d2h);

/* Pinned host memory mapped into the device address space (write-combined
 * off; coarse-grained).  *host_ptr is the CPU address, *dev_view the address
 * kernels use.  ESS_ERR_NOMEM on failure. */
ess_status ess_host_alloc(size_t bytes, void** host_ptr, void** dev_view);
ess_status ess_host_free(void* host_ptr);

/* Bytes of device workspace ess_prefill_layers needs for buffers of `rows`
 * rows (partial sums of the stand-in compute per block of 128 rows); 0 if
 * rows < 1. */
size_t ess_prefill_ws_bytes(int32_t rows);

/* Prefill over n_layers layers with four full-layer device buffers
 * (FlashOffloading analysis, prefill section, Figs. 2 and 3): host memory
 * keeps every layer's full history; B0 (bufs[0]) stays bound to layer 0 for
 * the whole prefill and must already hold its history unless load_layer0
 * is set; B1-B3 rotate over the later layers.  Layers 1, 2, 3 are bound to
 * B1, B2, B3 before any compute; layer i >= 1 releases its buffer once its
 * compute and its write-back are done, and at layer i's scheduling point
 * the oldest released buffer is bound to layer onload_layer_map[i] (NULL:
 * i + 3 while it exists; -1: none), whose load starts once that buffer is
 * released and layer i is computed.  Per layer:
 *   load   (stream h2d): host_kv[l][0:n_hist] -> buffer (layers >= 1);
 *   compute (stream compute, after the load): new_kv[l] appended at rows
 *          [n_hist, n_hist + n_new) of the buffer, then the stand-in
 *          consumer - all n_hist + n_new rows read from the buffer once and
 *          their per-column sums taken compute_reps times on chip into
 *          layer_out[l][576] (a knob for the compute window, like a layer
 *          whose work reads its KV once; the result is the same);
 *   write-back (stream d2h, after the compute): buffer rows
 *          [n_hist, n_hist + n_new) -> host_kv[l][n_hist:].
 *   host_kv   [n_layers][rows][576] bf16 in pinned host memory (the host
 *             address from ess_host_alloc); new_kv [n_layers][n_new][576]
 *             bf16, bufs [4][rows][576] bf16, layer_out [n_layers][576]
 *             float, ws ess_prefill_ws_bytes(rows) bytes: device;
 *   onload_layer_map [n_layers], binding [n_layers] (out: the buffer of
 *             each layer, may be NULL): host arrays.
 * The three streams must differ; on return all work, write-backs included,
 * is ordered before later work on `compute`.  ESS_ERR_INVALID for bad
 * sizes, NULL pointers, equal streams or a map that loads a layer twice,
 * loads a past or bound layer, or leaves a layer unloaded at its turn. */
ess_status ess_prefill_layers(int32_t n_layers, int32_t rows, int32_t n_hist,
                              int32_t n_new, uint16_t* host_kv,
                              const uint16_t* new_kv, uint16_t* bufs,
                              float* layer_out, void* ws, size_t ws_bytes,
                              const int32_t* onload_layer_map,
                              int32_t* binding, int32_t compute_reps,
                              int32_t load_layer0, hipStream_t compute,
                              hipStream_t h2d, hipStream_t d2h);

/* Eviction policies for ess_replay_evictions. */
enum {
  ESS_EVICT_LRU = 0,     /* least recently used: the pool's own policy      */
  ESS_EVICT_RANDOM = 1,  /* uniformly random (SplitMix64 keys)               */
  ESS_EVICT_SCORE = 2    /* lowest index score of the step                   */
};

/* Offline replay of one request's decode steps through a hot pool of
 * pool_slots slots under an eviction policy (FlashOffloading analysis,
 * decode ablation, first group, and Fig. 8: the recorded per-step top-k
 * index sets replayed with only the eviction policy changed: Random, LRU,
 * Score).  A host routine: every pointer is host memory, nothing touches
 * the GPU.
 *   scores  [steps][mtp][ctx_len] float: the index scores of every step and
 *           way, -inf past a way's visible length;
 *   sel_pos [steps][mtp][topk] int32, rank order; n_sel [steps][mtp];
 *   n_miss, n_evict [steps] int32 outputs (n_evict may be NULL).
 * The pool starts from the decode's first fill (the top-min(C, visible)
 * positions of way 0 at step 0, score descending, position ascending).
 * Per step: misses = the union of the ways' selections minus the
 * residents; free slots serve misses first; each remaining miss evicts one
 * resident outside the union, the smallest by the policy's order:
 *   LRU    (last step whose union held it, position) - fill counts as the
 *          step before step 0, so this is ess_pool_update's own order;
 *   RANDOM (key, position), key = output number
 *          (request << 48 | step << 32 | position) + 1 of SplitMix64
 *          (Steele, Lea and Flood, OOPSLA 2014) seeded with `seed`;
 *   SCORE  (the largest of the position's scores over the step's ways,
 *          position).
 * The pages' fourth policy (a score threshold plus a chunk scan) is named
 * there without its rule and is not offered.  ESS_ERR_CAPACITY if a step's
 * union exceeds pool_slots, ESS_ERR_INVALID for bad sizes, NULL arrays or a
 * selected position outside [0, ctx_len); steps and request < 65536. */
ess_status ess_replay_evictions(int32_t policy, int32_t ctx_len,
                                int32_t pool_slots, int32_t steps,
                                int32_t mtp, int32_t topk,
                                const float* scores, const int32_t* sel_pos,
                                const int32_t* n_sel, uint64_t seed,
                                int32_t request, int32_t* n_miss,
                                int32_t* n_evict);

/* Asynchronous copy of `bytes` bytes on the stream between any two of
 * device memory and pinned host memory (hipMemcpyDefault: the direction
 * follows from the addresses); for callers that stage data without a HIP
 * runtime handle of their own.  0 bytes: nothing is enqueued. */
ess_status ess_copy_async(void* dst, const void* src, size_t bytes,
                          hipStream_t stream);

/* Destroy the stream-ordering events the calling thread's calls created
 * (they are otherwise kept for the thread's later calls).  Call it once the
 * thread's work has completed and before the HIP runtime is torn down
 * (e.g. at process exit, before static destructors run); a later call on
 * the thread creates new ones. */
ess_status ess_thread_release(void);

const char* ess_status_string(ess_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* ess_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ESS_H */
