// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ess.h"

namespace ess {

// Largest k the top-k and pool-update kernels hold on chip (LDS sort buffer
// of 8-byte keys: 16384 * 8 = 128 KiB of the 160 KiB per CU).
constexpr int kMaxTopk = 16384;
// The pool update packs a slot + 1 into 20 bits of its sort entries.
constexpr int kMaxPoolSlots = (1 << 20) - 2;
constexpr int kLat = 576;   // latent width: c_KV[512] + k_R[64]
constexpr int kVal = 512;   // value width

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ---- indexer ------------------------------------------------------------
// Words the indexer clears before it scores, for a selection that follows
// on the same stream (rows of `words` 32-bit words, `stride_words` apart).
struct ClearSpec {
  uint32_t* base;
  size_t stride_words;
  int words;
  int rows;
};
hipError_t launch_index_scores(const ess_dims& d, const uint8_t* q,
                               const float* w, const uint8_t* k,
                               const int32_t* n_vis, float* scores,
                               hipStream_t s, ClearSpec clr = ClearSpec{nullptr, 0, 0, 0});

// ---- top-k --------------------------------------------------------------
// Workspace of the multi-level selection of rows longer than 32768 keys
// (0 when it does not apply: short rows, or k > 4096).  With ws == nullptr
// the top-k runs one workgroup per row over the whole row.
size_t topk_ws_bytes(const ess_dims& d, int k, int n_tok);
// Each row's winners in ascending position order: position, rank and slot
// before the update, [B][n_tok][k] each (for the residency update that
// follows; pos == nullptr: none).
struct PosLists {
  int32_t* pos;
  int32_t* rank;
  int32_t* slot;
};
// Whether launch_topk can fill position lists for this k (ranked from a
// compact winner list: rows of at most 32768 keys, or levels when `levels`).
bool topk_pos_lists_fit(const ess_dims& d, int k, bool levels);
// Rows longer than 32768 keys (k <= 4096, and few enough rows) select with
// several workgroups per row that exchange counts through the workspace
// (unless `split` is false: then they select in levels, whose workgroups
// never wait for one another - the choice for a selection that runs beside
// other kernels); its control words must be zero when the selection
// starts.  split_clear tells whether a selection of (k, n_tok) over `ws`
// takes that path and which words to clear; a launch with `cleared` set
// trusts that they were (by the indexer on the same stream), otherwise it
// clears them itself.
bool split_clear(const ess_dims& d, int k, int n_tok, void* ws, ClearSpec* c);
hipError_t launch_topk(const ess_dims& d, int k, int n_tok,
                       const float* scores, const int32_t* n_vis,
                       const int32_t* cache_slots, int32_t* sel_pos,
                       int32_t* sel_slot, int32_t* n_sel, void* ws,
                       hipStream_t s, PosLists pl = PosLists{nullptr, nullptr, nullptr},
                       bool cleared = false, bool split = true);

// ---- pool ---------------------------------------------------------------
// Per-request LRU state: header, slot stamps [C], ring of (slot, stamp).
struct LruHeader {
  int32_t head;       // first unread ring entry
  int32_t tail;       // one past the last ring entry
  int32_t free_head;  // slots [free_head, C) have never been used
  int32_t epoch;      // stamp of the next update
  int32_t cap;        // ring capacity in entries
  int32_t err;        // 0 ok; 1 the victim scan ran dry (state inconsistent);
                      // 2 a selected position was outside [0, L)
  int32_t compactions;  // times the ring was compacted since the reset
  int32_t pad;
};
__host__ __device__ inline int lru_ring_cap(int C) { return 4 * C; }
inline size_t lru_bytes_per_req(int C) {
  return align_up(sizeof(LruHeader) + sizeof(int32_t) * (size_t)C +
                      2 * sizeof(int32_t) * (size_t)lru_ring_cap(C),
                  256);
}

hipError_t launch_pool_reset(const ess_dims& d, int32_t* cache_slots,
                             int32_t* slot_pos, void* lru, hipStream_t s);
// status[b][0..4) = (err, compactions, epoch, live ring entries) of request b.
hipError_t launch_pool_status(const ess_dims& d, const void* lru,
                              int32_t* status, hipStream_t s);
// hipFuncSetAttribute(MaxDynamicSharedMemorySize) once per kernel and device.
hipError_t ensure_dyn_lds(const void* fn, int bytes);
// Top-k and residency update of one query token per request in one kernel
// (select_update_fits tells when it applies).
bool select_update_fits(const ess_dims& d, int k, int n_tok);
hipError_t launch_select_update(const ess_dims& d, int k, const float* scores,
                                const int32_t* n_vis, int32_t* cache_slots,
                                int32_t* sel_pos, int32_t* sel_slot,
                                int32_t* n_sel, int32_t* slot_pos, void* lru,
                                int32_t* miss_pos, int32_t* miss_slot,
                                int32_t* n_miss, int32_t* n_evict,
                                int32_t* row_dst, int32_t* sel_slot_post,
                                void* ws, hipStream_t s, bool cleared = false,
                                bool split = true);
hipError_t launch_pool_update(const ess_dims& d, int k, int n_tok,
                              const int32_t* sel_pos, const int32_t* n_sel,
                              int32_t* cache_slots, int32_t* slot_pos,
                              void* lru, int32_t* miss_pos,
                              int32_t* miss_slot, int32_t* n_miss,
                              int32_t* n_evict, int32_t* row_dst,
                              int32_t* sel_slot_post, hipStream_t s,
                              const int32_t* sel_slot_pre = nullptr,
                              PosLists lists = PosLists{nullptr, nullptr, nullptr});

// ---- attention ----------------------------------------------------------
struct MlaPlan {
  int heads_per_wg;   // 16 * waves
  int head_groups;    // H / heads_per_wg
  int rows_per_chunk; // multiple of 64 (a tile per sub-group)
  int nchunk;         // chunks of rows per (request, token)
};
// target_wgs: workgroups to aim for (0: the whole chip, one per CU).
MlaPlan plan_sparse_mla(const ess_dims& d, int target_wgs = 0);
size_t sparse_mla_ws_bytes(const ess_dims& d, int target_wgs = 0);
// Device tail blocks of growing context: rows [B][2 * block][576] bf16;
// position p >= start[b] of request b is held in row ((p / block) & 1) *
// block + p % block.  rows == nullptr: no tail.
struct TailView {
  const uint16_t* rows;
  const int32_t* start;   // device [B]
  int block;
};

hipError_t launch_sparse_mla(const ess_dims& d, const uint16_t* q_abs,
                             const int32_t* sel_pos, const int32_t* sel_src,
                             const int32_t* row_dst, const int32_t* n_sel,
                             uint16_t* pool, const uint16_t* host,
                             float* out, float* lse, void* ws,
                             hipStream_t s, int target_wgs = 0,
                             const uint8_t* entries = nullptr,
                             TailView tail = TailView{nullptr, nullptr, 1});
// (entries non-null: misses are read from 656-byte fp8 entries [B][L][656]
// instead of host, and dequantized in the tile.)

// The same gather + attention with its partials in the library's fixed
// per-device scratch array (kNoAllocScratchBytes) instead of a workspace;
// the caller checks sparse_mla_ws_bytes(d) <= kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = (size_t)24 << 20;
hipError_t launch_sparse_mla_noalloc(const ess_dims& d, const uint16_t* q_abs,
                                     const int32_t* sel_pos, const int32_t* sel_src,
                                     const int32_t* row_dst, const int32_t* n_sel,
                                     uint16_t* pool, const uint16_t* host,
                                     float* out, float* lse, hipStream_t s);

// ---- miss copy ----------------------------------------------------------
hipError_t launch_miss_copy(const ess_dims& d, int list_stride,
                            const int32_t* miss_pos, const int32_t* miss_slot,
                            const int32_t* n_miss, const uint16_t* host,
                            uint16_t* pool, hipStream_t s);
// The same copy from 656-byte fp8 entries [B][L][656], dequantized to bf16.
hipError_t launch_entry_copy(const ess_dims& d, int list_stride,
                             const int32_t* miss_pos, const int32_t* miss_slot,
                             const int32_t* n_miss, const uint8_t* host,
                             uint16_t* pool, hipStream_t s);

// ---- growing context ----------------------------------------------------
// Append mtp tokens to every request b at positions state[B + b] ..: keys
// into k_idx [B][L][d_I], latents into the tail rows [B][2*block][576],
// n_vis [B][m] = n_ctx + 1 + j; then state[B + b] += m and state[2B + b] =
// the new first tail position.  state = device (first[B], n_ctx[B],
// start[B]).  tail_ent non-null ([B][2*block][656]): the latents are
// quantized into 656-byte entries there and the tail rows get them
// dequantized.
hipError_t launch_append_tokens(const ess_dims& d, int block,
                                const uint8_t* new_keys,
                                const uint16_t* new_lat, uint8_t* k_idx,
                                uint16_t* tail, uint8_t* tail_ent,
                                int32_t* n_vis, int32_t* state, hipStream_t s);

// ---- prefill pipeline ---------------------------------------------------
// Per-block partial sums of the stand-in layer compute for `rows` rows.
size_t prefill_ws_bytes(int rows);
// Stand-in compute of one layer on stream s: append n_new rows from
// new_rows (device) after the n_hist history rows of buf, then read the
// n_hist + n_new rows once and `reps` times reduce them on chip to
// per-column sums in out[576].
hipError_t launch_prefill_compute(const uint16_t* new_rows, int n_new,
                                  uint16_t* buf, int n_hist, int reps,
                                  float* part, float* out, hipStream_t s);

}  // namespace ess
