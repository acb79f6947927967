// Gather of the selected latents + absorbed-MLA attention over them.
//
// Pages: the main attention reads only the top-k latent entries (c_KV[512]
// + k^R each) and runs the core MLA on them (ESS concept page, "dual cache"
// table).  The fused gather forks per row between a hit, read from the pool
// in device memory, and a miss, read straight from pinned host memory; a
// miss is written to its pool slot and to the on-chip tile together, three
// memory accesses instead of four (FlashOffloading analysis, section
// "forking inside KVgather").  Here the on-chip tile is LDS, so a miss costs
// one host read plus one pool write and a hit one device read.
//
// Result independence from placement: the reduction runs over the selected
// rows in rank order, in fixed chunks of rows combined in fixed order; no
// atomics.  Which rows came from host memory changes no arithmetic.
//
// Miss handling on MI355X: a miss costs a host-link read (~55 GB/s
// measured) against an HBM read for a hit (8 TB/s), so the host link sets
// the pace.  The kernel does what the pages describe: a designated-writer
// miss is loaded from host memory into the tile like any other row, and the
// first head group of its token stores it from the tile to its pool slot.
// The host reads then run while the attention works on the rows already in
// LDS.  The workgroups of one (request, chunk) - every token and head group
// - run on one XCD close together, so a host row that another of them has
// just read comes from that XCD's L2: the second head group's reads, and a
// miss that the request's tokens share at nearby ranks, cross the link once
// (measured at 32K x 16: 4.4K misses per step take 116 us in this kernel,
// where two crossings alone would need over 180 us).  A miss row that
// another token writes is read from host memory too, never from the slot
// being written.
//
// Per workgroup: one (request, token), one group of heads, one chunk of rows.
// Each wave takes 16 heads.  With three or four head blocks (48 or 64
// heads) a wave owns all 512 value columns of its heads: one wave per SIMD,
// each scoring its heads once.  With fewer head blocks a wave owns one half
// of the value columns and the two waves of a head block compute the same
// scores (so no state is merged between waves, and the compute unit still
// runs at least four waves).  Tiles of 32 rows go from memory straight into
// LDS (gfx950's 16-byte global-to-LDS load, one 1 KB block per wave
// instruction), row-major with a 32-byte pad per row, into a ring of four
// buffers: three tiles are in flight while every wave reads the fourth,
// with one workgroup barrier per tile.  One wave per head block issues the
// tile loads; a wave waits until no more of its loads are in flight than it
// issued after the tile's (loads land in issue order, so a store issued
// between them can only make that wait longer, never end it early).  The
// miss rows are stored to their pool slots by the waves of the second
// column half, or by every wave when each owns all columns.  The queries of
// the workgroup's heads also come through LDS (two ring buffers, before the
// third and fourth tiles are issued).  Padding and unusable rows load a zero
// row.  At the end each wave writes its columns of the chunk's partial
// normalised, in fp16 scaled by a power of two per (head, half of the value
// columns) so that the half's largest magnitude lies in [0.5, 1): the stored
// values keep fp16's 11 significant bits whatever the latents' range (no
// overflow above 65504, no subnormals for small latents).  The running max
// and sum and the two scales are fp32.  The output accumulators stay in
// VGPRs (MFMA results in VGPR form, set for this file at build time): in
// accumulation registers the compiler moved all of them to VGPRs and back
// around the rescale branch on every tile (~25 % of a tile's cycles).
//   S^T[tok][h] = sum_d K[tok][d] Q[h][d]   mfma 16x16x32 bf16, A = K tile
//                                           rows from LDS, B = Q in registers
//   O^T[c][h]  += sum_tok V^T[c][tok] P[h][tok]   A = V^T, B = P in registers
// The V^T operand comes from the same row-major tile through gfx950's
// transposing LDS read (ds_read_b64_tr_b16): within a 16-lane group, lane i
// receives element i mod 4 of the 8 bytes addressed by lanes 4e + i/4, so
// pointing lane r at token 4g + r/4, columns 4(r mod 4).. gives lane i the
// column i of four tokens.  The S^T accumulator leaves each lane holding one
// head and 8 tokens; those 8 tokens are exactly the lane's reduction slice
// of the PV operand, so P never leaves registers.
// Softmax runs in the log2 domain with a running max and sum per head.
//
// With growing context the newest positions sit in two tail blocks in device
// memory until written back to the host store; a selected position from its
// request's tail.start on is loaded from its tail row like a pool row (and,
// as a miss with a writer slot, still written to that slot from the tile).
//
// With a host store of 656-byte fp8 entries (c_KV in e4m3 with one
// power-of-two scale per 128 values, k_R in bf16) a miss crosses the host
// link as its 656 bytes instead of a 1152-byte row: the load puts the raw
// entry into the last 41 slots of its tile row, and after the tile has
// landed one wave per miss row expands it in place to the 576 bf16 values
// the MFMAs and the pool write-back read (a second barrier per tile).
#include <mutex>

#include "ess_internal.h"
#include "fp8_entry.h"

namespace ess {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kTile = 32;                       // tokens per LDS tile
// Rows sit 74 slots (1184 bytes) apart: 37 whole wave loads per tile, and
// the transposing V reads (8 rows x 32 bytes per 32 lanes) fall in distinct
// banks (at 73 slots rows 0 and 7 overlap; counters showed ~43 % of the
// kernel's LDS cycles stalled on bank conflicts, now none).
constexpr int kRowSlots = kLat / 8 + 2;         // 16-byte slots per row (72 + 2 pad)
constexpr int kKStride = kRowSlots * 8;         // bf16 per row-major row (1184 B)
constexpr int kChunks16 = kLat / 8;             // 16-byte pieces per latent row (72)
constexpr int kTileLoads = (kTile * kRowSlots + 63) / 64;   // wave loads per tile (37)
constexpr int kTileSlots = kTileLoads * 64;     // slots per tile buffer (2368)
constexpr int kRing = 4;                        // tile buffers: three in flight, one read
constexpr int kMaxChunkRows = 512;              // rows per chunk held in LDS tables
constexpr int kMaxChunkTiles = kMaxChunkRows / kTile;
// Tile ring, then the rows' source addresses, the writer slots and the
// per-tile writer and fp8-entry masks.
constexpr size_t kMlaLds = (size_t)kRing * kTileSlots * 16 + (size_t)kMaxChunkRows * 8 +
                           (size_t)kMaxChunkRows * 4 + kMaxChunkTiles * 4 * 2;
static_assert(kMlaLds <= 160 * 1024, "LDS of one compute unit");
// The queries of up to 64 heads, rows laid out like tile rows, fill two
// tile buffers.
static_assert(64 * kRowSlots <= 2 * kTileSlots, "queries fit in two tile buffers");
// A miss read from a 656-byte fp8 entry lands raw in the last 41 slots of
// its tile row and is expanded in place to 576 bf16 before the tile is read.
constexpr int kRawSlot0 = kRowSlots - kEntryPieces;   // 33
static_assert(kRawSlot0 > 0, "raw entry must fit in a tile row");

// A zero latent row: the source of padding rows and unusable rows.
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[kLat] = {};

__device__ __forceinline__ v2u tr_read(const uint16_t* p) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4s*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(v2u, v);
}

// One wave instruction: lane l copies 16 bytes from `src` to LDS at
// lds_block + 16 l (lds_block is the same for the whole wave).  Issued as
// inline assembly so that the compiler does not wait for it before
// unrelated LDS reads; the caller waits (vmcnt) and synchronises before
// reading the block.
__device__ __forceinline__ void load_lds16(const void* src, const void* lds_block) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(
      const __attribute__((address_space(3))) void*)lds_block);
  // An SALU write of M0 needs one wait state before an LDS-DMA load reads it.
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(base), "v"(src) : "memory", "m0");
}

// vmcnt(N): at most N of this wave's vector-memory operations still in
// flight (expcnt, lgkmcnt unchanged).  N above the counter's 63 waits for 63,
// which is more than asked, never less.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// This wave's loads of a group have landed, given that `after` further
// groups of P loads each were issued since (loads land in issue order).
template <int P>
__device__ __forceinline__ void wait_loads(int after) {
  if (after >= 3) wait_vmcnt<3 * P>();
  else if (after == 2) wait_vmcnt<2 * P>();
  else if (after == 1) wait_vmcnt<P>();
  else wait_vmcnt<0>();
}

// Max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 of a wave (the
// lanes that hold one head), with gfx950's lane swaps: VALU operations, so
// they do not queue behind the tile reads in the LDS pipeline as lane
// shuffles would.  permlane32_swap pairs lane l with l ^ 32, permlane16_swap
// row 0 with row 1 and row 2 with row 3 (16 lanes a row); every lane ends
// with the same value.
__device__ __forceinline__ float head_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float head_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Expand the raw entry in slots kRawSlot0.. of a tile row into the row's
// 576 bf16 (one wave; lane l writes c_KV slot l, lanes 0-7 the k_R slots).
// The output overlaps raw bytes other lanes read, so every lane's reads are
// complete before any lane writes.
__device__ __forceinline__ void expand_entry_row(uint16_t* row, int lane) {
  const unsigned char* raw = reinterpret_cast<const unsigned char*>(row + kRawSlot0 * 8);
  const uint2 q8 = *reinterpret_cast<const uint2*>(raw + lane * 8);
  const float sc = *reinterpret_cast<const float*>(raw + kEntryScaleOff + (lane >> 4) * 4);
  entry_v4u kr = {0u, 0u, 0u, 0u};
  if (lane < 8) kr = *reinterpret_cast<const entry_v4u*>(raw + kEntryRopeOff + lane * 16);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const entry_v4u w = dequant8(q8.x, q8.y, sc);
  *reinterpret_cast<entry_v4u*>(row + lane * 8) = w;
  if (lane < 8) *reinterpret_cast<entry_v4u*>(row + (kVal / 8 + lane) * 8) = kr;
}

// WPS head blocks of 16 heads; CH waves per head block, each with 512 / CH
// value columns (CH = 1 or 2).
template <int WPS, int CH, bool kEnt>
__global__ __launch_bounds__(CH * WPS * 64) void sparse_mla_kernel(
    const uint16_t* __restrict__ q_abs, const int32_t* __restrict__ sel_pos,
    const int32_t* __restrict__ sel_src, const int32_t* __restrict__ row_dst,
    const int32_t* __restrict__ n_sel, uint16_t* __restrict__ pool,
    const uint16_t* __restrict__ host, const unsigned char* __restrict__ entries,
    TailView tail, _Float16* __restrict__ part_acc,
    float4* __restrict__ part_ml, int L, int C, int m, int H, int k,
    int rows_per_chunk, int nchunk, int head_groups, int n_bj,
    float scale_log2) {
  static_assert(CH == 1 || CH == 2, "one or two column parts per head block");
  constexpr int NW = CH * WPS;
  constexpr int NT = NW * 64;
  // Loads per loading wave and tile: every loading wave issues the same
  // number (repeating the tile's last block), so its count of loads in
  // flight says how many tiles are still in flight.
  constexpr int kLoadsPerWave = (kTileLoads + WPS - 1) / WPS;
  constexpr int kQRows = WPS * 16;                               // the workgroup's heads
  constexpr int kQLoads = (kQRows * kRowSlots + 63) / 64;        // wave loads of the queries
  constexpr int kQPerWave = (kQLoads + NW - 1) / NW;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // Row i of the chunk: its source address (bit 0 set for a miss read from
  // an fp8 entry, the address then 33 pieces before the entry), its writer
  // slot, and one bit per row in its tile's writer and entry masks.
  uint64_t* raddr = reinterpret_cast<uint64_t*>(smem + (size_t)kRing * kTileSlots * 8);
  int* wdst = reinterpret_cast<int*>(raddr + kMaxChunkRows);
  unsigned* wmask = reinterpret_cast<unsigned*>(wdst + kMaxChunkRows);
  unsigned* emask = wmask + kMaxChunkTiles;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ch = wave / WPS, hb = wave - ch * WPS;   // value-column part, head block
  const bool loader = ch == 0;                       // issues tile loads
  const bool storer = CH == 1 || ch == 1;            // stores miss rows
  const int g = lane >> 4, c = lane & 15;
  // Workgroup -> (token, head group, row chunk).  Consecutive workgroup ids
  // go to the 8 XCDs in turn, each with its own L2; the m * head_groups
  // workgroups of one (request, chunk) group get ids that are multiples of 8
  // apart, so they run on the same XCD close together and share the chunk's
  // rows through that L2.  Groups are numbered with the chunk slowest, the
  // chunk nearest the top-k cut first (where rows miss most); ids past the
  // last group (padding to whole rounds) exit.
  const int wg = blockIdx.x;
  const int xcd = wg & 7, round = wg >> 3;
  const int per = m * head_groups;
  const int sub = round % per;
  const int hg = sub % head_groups;
  const int grp = (round / per) * 8 + xcd;
  const int n_b = n_bj / m;
  if (grp >= n_b * nchunk) return;
  const int b = grp % n_b;
  const int chunk = nchunk - 1 - grp / n_b;
  const int bj = b * m + sub / head_groups;
  const int r0 = chunk * rows_per_chunk;
  const int rend = min(k, r0 + rows_per_chunk);    // rows the table covers
  const int h0 = hg * kQRows + hb * 16;

  const int32_t* rpos = sel_pos + (size_t)bj * k;
  const int32_t* rsrc = sel_src + (size_t)bj * k;
  const int32_t* rdst = row_dst ? row_dst + (size_t)bj * k : nullptr;
  uint16_t* pool_b = pool + (size_t)b * C * kLat;
  // Misses come from bf16 rows (host) or, with kEnt, from fp8 entries.
  const uint16_t* host_b = kEnt ? nullptr : host + (size_t)b * L * kLat;
  const unsigned char* ent_b = kEnt ? entries + (size_t)b * L * kEntryBytes : nullptr;
  // Positions from tail.start[b] on are read from the request's two tail blocks
  // in device memory (row code C + tail row) instead of host memory.
  const uint16_t* tail_b = tail.rows ? tail.rows + (size_t)b * 2 * tail.block * kLat : nullptr;
  const int tail_start = tail.rows ? tail.start[b] : INT32_MAX;

  // The zero row's address, once (not reloaded before every use).
  const uint16_t* zrow = g_zero_row;
  asm volatile("" : "+s"(zrow));

  // Row sources of the chunk, once: a hit reads its slot, a miss host
  // memory (or its tail row), a row past n_sel or with an out-of-range
  // value (caller error) the zero row.  Given writer slots, the first head
  // group stores each designated-writer miss from the tile to its slot
  // (wdst, and one bit per row in its tile's mask).  The row loads are
  // issued for the whole chunk up to k, together with the n_sel load.
  // Each wave fills 64 consecutive rows (two whole tiles, as r0 and the
  // chunk length are multiples of 64).
  const int r1 = min(min(n_sel[bj], k), r0 + rows_per_chunk);
  const int ntile = r1 > r0 ? (r1 - r0 + kTile - 1) / kTile : 0;
  const bool writer_wg = rdst != nullptr && hg == 0;
  for (int i0 = r0 + wave * 64; i0 < r0 + rows_per_chunk; i0 += NT) {
    const int i = i0 + lane;
    bool wr = false, ent = false;
    uintptr_t addr = (uintptr_t)zrow;
    if (i < rend) {
      const int src = rsrc[i], pos = rpos[i];
      const int dst = rdst ? rdst[i] : -1;
      if (i < r1) {
        if (src >= 0) {
          if (src < C) addr = (uintptr_t)(pool_b + (size_t)src * kLat);
        } else if (pos >= 0 && pos < L) {
          if (pos >= tail_start) {
            addr = (uintptr_t)(tail_b + ((size_t)((pos / tail.block) & 1) * tail.block +
                                         pos % tail.block) * kLat);
          } else if constexpr (kEnt) {
            addr = ((uintptr_t)(ent_b + (size_t)pos * kEntryBytes) - kRawSlot0 * 16) | 1u;
            ent = true;
          } else {
            addr = (uintptr_t)(host_b + (size_t)pos * kLat);
          }
          if (writer_wg && dst >= 0 && dst < C) {
            wdst[i - r0] = dst;
            wr = true;
          }
        }
      }
    }
    raddr[i - r0] = addr;
    const unsigned long long bw = __ballot(wr), be = __ballot(ent);
    if (lane == 0) {
      wmask[(i0 - r0) >> 5] = (unsigned)bw;
      wmask[((i0 - r0) >> 5) + 1] = (unsigned)(bw >> 32);
      emask[(i0 - r0) >> 5] = (unsigned)be;
      emask[((i0 - r0) >> 5) + 1] = (unsigned)(be >> 32);
    }
  }
  // (every plain global load is consumed here, before the first load into
  // LDS, so the compiler's own waits never count those)
  asm volatile("" ::"v"(r1));

  // Each of a loading wave's loads covers the same tile slots in every
  // tile: slot q = 64 j + lane holds row q / kRowSlots, piece
  // q % kRowSlots.  Kept packed per load: the row (5 bits), the piece a
  // bf16 row reads (the pad pieces and slots past the tile repeat piece 0)
  // and the piece an fp8-entry row reads, counted from 33 pieces before
  // the entry (slots before its raw pieces take its first piece; the
  // expansion overwrites them).
  unsigned lslot[kLoadsPerWave];
#pragma unroll
  for (int u = 0; u < kLoadsPerWave; ++u) {
    const int q = min(hb + u * WPS, kTileLoads - 1) * 64 + lane;
    const int row = q / kRowSlots, piece = q - row * kRowSlots;
    const int pr = row < kTile && piece < kChunks16 ? piece : 0;
    const int pe = row < kTile ? max(piece, kRawSlot0) : kRawSlot0;
    lslot[u] = (unsigned)min(row, kTile - 1) | (unsigned)pr << 5 | (unsigned)pe << 12;
  }

  // Issue the loads of tile tt into ring buffer tt % kRing (loading waves):
  // each load's row address from the table plus its piece.  The table reads
  // of all of a wave's loads are in flight together, then the loads.
  auto issue = [&](int tt) {
    uint16_t* buf = smem + (size_t)(tt & (kRing - 1)) * kTileSlots * 8;
    const uint64_t* ta = raddr + tt * kTile;
    uint64_t ra[kLoadsPerWave];
#pragma unroll
    for (int u = 0; u < kLoadsPerWave; ++u) ra[u] = ta[lslot[u] & 31u];
#pragma unroll
    for (int u = 0; u < kLoadsPerWave; ++u) {
      const int j = min(hb + u * WPS, kTileLoads - 1);
      uint64_t src;
      if constexpr (kEnt) {
        const unsigned piece = (ra[u] & 1u) ? lslot[u] >> 12 : (lslot[u] >> 5) & 127u;
        src = (ra[u] & ~(uint64_t)1) + piece * 16u;
      } else {
        src = ra[u] + ((lslot[u] >> 5) & 127u) * 16u;
      }
      load_lds16((const void*)(uintptr_t)src, buf + (size_t)j * 64 * 8);
    }
  };

  __syncthreads();            // row table visible to every wave
  // The workgroup's queries into ring buffers 2 and 3 (row h at slot
  // 74 h, like a tile row), every wave a share; then tiles 0 and 1.
  uint16_t* qbuf = smem + (size_t)2 * kTileSlots * 8;
  {
    const uint16_t* qwg = q_abs + ((size_t)bj * H + hg * kQRows) * kLat;
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int u = 0; u < kQPerWave; ++u) {
      const int j = min(wave + u * NW, kQLoads - 1);
      const int q = j * 64 + ln;
      const int row = q / kRowSlots, piece = q - row * kRowSlots;
      const int off = (piece < kChunks16 ? piece : 0) * 8;
      load_lds16(qwg + (size_t)min(row, kQRows - 1) * kLat + off, qbuf + (size_t)j * 64 * 8);
    }
  }
  if (loader) {
    if (ntile > 0) issue(0);
    if (ntile > 1) issue(1);
    wait_loads<kLoadsPerWave>(min(ntile, 2));   // the queries (tiles 0, 1 may fly)
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();            // every wave's query loads have landed
  // Lane holds Q[h0 + c][32 kk + 8 g .. + 8].
  bf16x8 qf[kLat / 32];
  {
    const uint16_t* qrow = qbuf + (size_t)(hb * 16 + c) * kKStride + g * 8;
#pragma unroll
    for (int kk = 0; kk < kLat / 32; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 32);
  }
  __syncthreads();            // queries read: buffers 2 and 3 are free
  if (loader) {
    if (ntile > 2) issue(2);
    if (ntile > 3) issue(3);
  }
  int issued = min(ntile, kRing) - 1;   // last tile issued (loading waves)

  float m_run = -__builtin_inff(), l_run = 0.f;
  constexpr int kCols = kVal / CH;      // value columns of this wave
  constexpr int kBlk = kCols / 16;      // 16-column blocks of this wave
  v4f oacc[kBlk];
#pragma unroll
  for (int nt = 0; nt < kBlk; ++nt) oacc[nt] = v4f{0.f, 0.f, 0.f, 0.f};

  // Transposed-read address of this lane within a tile half: token
  // 4 g + (c / 4), columns 4 (c % 4) .. of each 16-column group, in this
  // wave's part of the value columns.
  const int tr_off = (g * 4 + (c >> 2)) * kKStride + (c & 3) * 4 + ch * kCols;

  for (int t = 0; t < ntile; ++t) {
    if (loader) wait_loads<kLoadsPerWave>(issued - t);   // this wave's loads of tile t
    __syncthreads();          // ... and every wave's; tile t - 1 read by every wave
    if (loader && t + kRing - 1 < ntile && t + kRing - 1 > issued) {
      issue(t + kRing - 1);   // into the buffer tile t - 1 used
      issued = t + kRing - 1;
    }
    const int t0 = r0 + t * kTile;
    uint16_t* krow_w = smem + (size_t)(t & (kRing - 1)) * kTileSlots * 8;
    if constexpr (kEnt) {
      // Expand this tile's miss rows (the waves take them in turn), then
      // make them visible to every wave.
      unsigned msk = __builtin_amdgcn_readfirstlane(emask[t]);
      int n = 0;
      while (msk) {
        const int r = __builtin_ctz(msk);
        msk &= msk - 1u;
        if (n++ % NW == wave) expand_entry_row(krow_w + (size_t)r * kKStride, lane);
      }
      __syncthreads();
    }
    const uint16_t* krow = krow_w;

    // S^T for the two 16-token halves of the tile: the two accumulator
    // chains interleaved, and each step's operand reads issued kAhead steps
    // before its MFMAs, so LDS latency overlaps the matrix work.
    constexpr int kAhead = 3;
    v4f s[2];
    {
      const uint16_t* arow0 = &krow[c * kKStride + g * 8];
      const uint16_t* arow1 = arow0 + 16 * kKStride;
      v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
      bf16x8 ka[kAhead][2];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) {
        ka[i][0] = *reinterpret_cast<const bf16x8*>(arow0 + i * 32);
        ka[i][1] = *reinterpret_cast<const bf16x8*>(arow1 + i * 32);
      }
#pragma unroll
      for (int kk = 0; kk < kLat / 32; ++kk) {
        const bf16x8 a0 = ka[kk % kAhead][0], a1 = ka[kk % kAhead][1];
        if (kk + kAhead < kLat / 32) {
          ka[kk % kAhead][0] = *reinterpret_cast<const bf16x8*>(arow0 + (kk + kAhead) * 32);
          ka[kk % kAhead][1] = *reinterpret_cast<const bf16x8*>(arow1 + (kk + kAhead) * 32);
        }
        // (keeps the scheduler from moving the reads back next to their use)
        __builtin_amdgcn_sched_barrier(0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[kk], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[kk], acc1, 0, 0, 0);
      }
      s[0] = acc0;
      s[1] = acc1;
    }
    // The first V^T reads do not depend on P: issue them before the softmax.
    const uint16_t* vbase = &krow[tr_off];
    v2u vlo[kAhead], vhi[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      vlo[i] = tr_read(vbase + i * 16);
      vhi[i] = tr_read(vbase + i * 16 + 16 * kKStride);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Online softmax for head h0 + c over this tile's tokens
    // t0 + 16 mt + 4 g + r (the same in both column halves).
    float z[8];
    if (t0 + kTile <= r1) {       // a whole tile (wave-uniform)
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = s[e >> 2][e & 3] * scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = t0 + (e >> 2) * 16 + g * 4 + (e & 3);
        z[e] = tok < r1 ? s[e >> 2][e & 3] * scale_log2 : -__builtin_inff();
      }
    }
    float mx = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
    mx = head_max(mx);
    // The running maximum moves only when some head of the wave sees a tile
    // maximum more than 2^8 above it (log2 domain); otherwise every
    // p = 2^(z - m_run) stays at most 256 and the accumulators keep their
    // reference, so the rescale multiplies are skipped (the sum and the
    // accumulators always share one reference, so the result is the same).
    // (2^x below by the hardware's exp2 directly: x <= 8 here, and results
    // under 2^-126 flush to zero, far below what the sums can resolve)
    if (__ballot(mx > m_run + 8.f) != 0ull) {   // wave-uniform
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int nt = 0; nt < kBlk; ++nt) oacc[nt] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(z[e] - m_run);
      psum += p;
      pb[e] = (__bf16)p;
    }
    l_run += head_sum(psum);

    // O^T += V^T P^T over the tile for this wave's value columns; V^T
    // read transposed from the tile rows: tokens 4 g .. 4 g + 3 and
    // 16 + 4 g .. 16 + 4 g + 3, column ch kCols + nt*16 + c.  Each column
    // block's reads are issued kAhead blocks before its MFMA.
#pragma unroll
    for (int nt = 0; nt < kBlk; ++nt) {
      const v2u lo = vlo[nt % kAhead], hi = vhi[nt % kAhead];
      if (nt + kAhead < kBlk) {
        vlo[nt % kAhead] = tr_read(vbase + (nt + kAhead) * 16);
        vhi[nt % kAhead] = tr_read(vbase + (nt + kAhead) * 16 + 16 * kKStride);
      }
      __builtin_amdgcn_sched_barrier(0);
      const v4u vv = {lo[0], lo[1], hi[0], hi[1]};
      const bf16x8 va = __builtin_bit_cast(bf16x8, vv);
      oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[nt], 0, 0, 0);
    }

    // Writer rows: this tile's designated-writer misses (read from host) go
    // from the tile to their pool slots, one row per storing wave in turn.
    // Only rows below n_sel were loaded.
    if (storer && writer_wg) {
      unsigned msk = __builtin_amdgcn_readfirstlane(wmask[t]);
      if (r1 - t0 < kTile) msk &= (1u << (r1 - t0)) - 1u;
      int n = 0;
      while (msk) {
        const int r = __builtin_ctz(msk);
        msk &= msk - 1u;
        if (n++ % WPS == hb) {
          const int dst = __builtin_amdgcn_readfirstlane(wdst[t0 - r0 + r]);
          const v4u* srow = reinterpret_cast<const v4u*>(krow + r * kKStride);
          v4u* drow = reinterpret_cast<v4u*>(pool_b + (size_t)dst * kLat);
          drow[lane] = srow[lane];
          if (lane < kChunks16 - 64) drow[64 + lane] = srow[64 + lane];
        }
      }
    }
  }

  // Normalised partial: O^T rows 16 nt + 4 g + r of head h0 + c, this
  // wave's columns, one half of the value columns at a time.  The half's
  // largest magnitude (over the four lane groups that hold the head) sets a
  // power-of-two scale 2^e with amax * 2^-e in [0.5, 1); multiplying by
  // 2^-e is exact.
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  _Float16* pa = part_acc + (((size_t)bj * nchunk + chunk) * H + h0 + c) * kVal +
                 ch * kCols + g * 4;
  float* ml = reinterpret_cast<float*>(part_ml + ((size_t)bj * nchunk + chunk) * H + h0 + c);
  constexpr int kHalfBlk = kVal / 32;   // 16-column blocks per half
#pragma unroll
  for (int hh = 0; hh < kBlk / kHalfBlk; ++hh) {
    v4f fin[kHalfBlk];
#pragma unroll
    for (int u = 0; u < kHalfBlk; ++u) fin[u] = oacc[hh * kHalfBlk + u] * inv;
    float amax = 0.f;
#pragma unroll
    for (int u = 0; u < kHalfBlk; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(fin[u][r]));
    amax = head_max(amax);
    int ex = 0;
    if (amax > 0.f && amax <= 3.0e38f) (void)frexpf(amax, &ex);
    const float down = ldexpf(1.f, -ex);
#pragma unroll
    for (int u = 0; u < kHalfBlk; ++u)
      *reinterpret_cast<v4h*>(pa + (hh * kHalfBlk + u) * 16) =
          __builtin_convertvector(fin[u] * down, v4h);
    if (g == 0) ml[2 + ch + hh] = ldexpf(1.f, ex);
  }
  if (g == 0 && ch == 0) {
    ml[0] = m_run;
    ml[1] = l_run;
  }
}

// Merge the chunk partials of one (request, token, head) in chunk order;
// each partial is normalised, so its weight is 2^(m - M) times its sum, and
// its stored values are multiplied back by their half's scale.  64 threads
// per head and wave, 8 values each (16-byte fp16 loads).  With WPH waves per
// head (many chunks, few heads) wave w folds chunks [w n / WPH, (w + 1) n /
// WPH) and wave 0 then folds the waves' states in wave order; with one wave
// per head a workgroup holds 4 heads.  Chunks go in groups of 8 whose loads
// are all in flight together, folded in with a running maximum.  The order
// of every fold depends only on the shape, never on the data's placement.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
constexpr int kCombineThreads = 256;
constexpr int kCombineGroup = 8;
template <int WPH>
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(
    const _Float16* __restrict__ part_acc, const float4* __restrict__ part_ml,
    float* __restrict__ out, float* __restrict__ lse, int H, int nchunk) {
  constexpr int kHeads = kCombineThreads / 64 / WPH;   // heads per workgroup
  const int bj = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int hl = wave / WPH, w = wave % WPH;
  const int h = blockIdx.x * kHeads + hl;
  const int t = threadIdx.x & 63;
  const bool hi_half = t * 8 >= kVal / 2;      // this thread's columns' scale
  const float4* ml = part_ml + (size_t)bj * nchunk * H + h;
  const _Float16* pp = part_acc + ((size_t)bj * nchunk * H + h) * kVal + t * 8;
  const int cb = w * nchunk / WPH, ce = (w + 1) * nchunk / WPH;
  float M = -__builtin_inff(), den = 0.f;
  v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
  for (int c0 = cb; c0 < ce; c0 += kCombineGroup) {
    float4 v[kCombineGroup];
    v8h x[kCombineGroup];
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      const int ci = min(c0 + u, ce - 1);
      v[u] = ml[(size_t)ci * H];
      x[u] = *reinterpret_cast<const v8h*>(pp + (size_t)ci * H * kVal);
      if (c0 + u >= ce) v[u].y = 0.f;              // past this wave's chunks
    }
    float mg = M;
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u)
      if (v[u].y > 0.f) mg = fmaxf(mg, v[u].x);
    if (mg == -__builtin_inff()) continue;          // nothing yet
    const float sc = exp2f(M - mg);                 // 0 while M is -inf
    den *= sc;
    a0 *= sc;
    a1 *= sc;
    M = mg;
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      const float wgt = v[u].y > 0.f ? exp2f(v[u].x - M) * v[u].y : 0.f;
      const float ws = wgt * (hi_half ? v[u].w : v[u].z);
      den += wgt;
      a0 += ws * __builtin_convertvector(x[u].lo, v4f);
      a1 += ws * __builtin_convertvector(x[u].hi, v4f);
    }
  }
  if constexpr (WPH > 1) {
    // The waves' states through LDS; wave 0 of the head folds them in order.
    __shared__ float st_m[kHeads][WPH][64], st_d[kHeads][WPH][64];
    __shared__ v4f st_a[kHeads][WPH][2][64];
    st_m[hl][w][t] = M;
    st_d[hl][w][t] = den;
    st_a[hl][w][0][t] = a0;
    st_a[hl][w][1][t] = a1;
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int q = 1; q < WPH; ++q) {
      const float mq = st_m[hl][q][t], dq = st_d[hl][q][t];
      if (!(dq > 0.f)) continue;
      const float mg = fmaxf(M, mq);
      const float s0 = exp2f(M - mg), s1 = exp2f(mq - mg);   // s0 = 0 while M is -inf
      den = den * s0 + dq * s1;
      a0 = a0 * s0 + st_a[hl][q][0][t] * s1;
      a1 = a1 * s0 + st_a[hl][q][1][t] * s1;
      M = mg;
    }
  }
  const float inv = 1.f / den;
  float* op = out + ((size_t)bj * H + h) * kVal + t * 8;
  *reinterpret_cast<v4f*>(op) = a0 * inv;
  *reinterpret_cast<v4f*>(op + 4) = a1 * inv;
  if (lse && t == 0) lse[(size_t)bj * H + h] = (M + log2f(den)) * 0.69314718055994531f;
}

template <int WPS, int CH, bool kEnt>
hipError_t launch_t(const ess_dims& d, const MlaPlan& p, const uint16_t* q,
                    const int32_t* sel_pos, const int32_t* sel_src,
                    const int32_t* row_dst, const int32_t* n_sel,
                    uint16_t* pool, const uint16_t* host,
                    const unsigned char* entries, TailView tail,
                    _Float16* part_acc, float4* part_ml, hipStream_t s) {
  const float scale_log2 = d.softmax_scale * 1.4426950408889634f;
  hipError_t e = ensure_dyn_lds((const void*)sparse_mla_kernel<WPS, CH, kEnt>, (int)kMlaLds);
  if (e != hipSuccess) return e;
  // 1-D grid over (group, token, head group) in whole rounds of 8 XCDs.
  const int groups = d.batch * p.nchunk;
  const int rounds = ((groups + 7) / 8) * d.mtp * p.head_groups;
  dim3 grid(rounds * 8);
  hipLaunchKernelGGL((sparse_mla_kernel<WPS, CH, kEnt>), grid, dim3(CH * WPS * 64), kMlaLds, s, q,
                     sel_pos, sel_src, row_dst, n_sel, pool, host, entries, tail, part_acc,
                     part_ml, d.ctx_len, d.pool_slots, d.mtp, d.mla_heads,
                     d.topk, p.rows_per_chunk, p.nchunk, p.head_groups,
                     d.batch * d.mtp, scale_log2);
  return hipGetLastError();
}

}  // namespace

MlaPlan plan_sparse_mla(const ess_dims& d, int target_wgs) {
  MlaPlan p;
  const int H = d.mla_heads;
  // One workgroup per compute unit (each holds nearly all of a CU's LDS);
  // more chunks would also mean more partial traffic.
  const int target = target_wgs > 0 ? target_wgs : 256;
  // A chunk is a whole number of 64-row groups (the row table is filled 64
  // rows a wave, two tiles' writer masks at a time).
  const int max_chunks = (d.topk + 2 * kTile - 1) / (2 * kTile);
  // The most heads per workgroup (each head group reads the chunk's rows
  // again) that still gives the target number of workgroups; with few
  // requests the heads split further so more workgroups share the rows.
  p.heads_per_wg = 16;
  for (const int c : {64, 48, 32, 16}) {
    if (H % c) continue;
    p.heads_per_wg = c;
    if ((long)d.batch * d.mtp * (H / c) * max_chunks >= target) break;
  }
  p.head_groups = H / p.heads_per_wg;
  const int base = d.batch * d.mtp * p.head_groups;
  int nchunk = (target + base - 1) / base;
  const int min_chunks = (d.topk + kMaxChunkRows - 1) / kMaxChunkRows;
  if (nchunk < min_chunks) nchunk = min_chunks;   // miss list fits in LDS
  if (nchunk < 1) nchunk = 1;
  if (nchunk > max_chunks) nchunk = max_chunks;
  const int per = (d.topk + nchunk - 1) / nchunk;
  p.rows_per_chunk = (per + 2 * kTile - 1) / (2 * kTile) * (2 * kTile);
  p.nchunk = (d.topk + p.rows_per_chunk - 1) / p.rows_per_chunk;
  return p;
}

size_t sparse_mla_ws_bytes(const ess_dims& d, int target_wgs) {
  const MlaPlan p = plan_sparse_mla(d, target_wgs);
  const size_t parts = (size_t)d.batch * d.mtp * p.nchunk * d.mla_heads;
  return align_up(parts * kVal * sizeof(_Float16), 256) +
         align_up(parts * sizeof(float4), 256);
}

hipError_t launch_sparse_mla(const ess_dims& d, const uint16_t* q_abs,
                             const int32_t* sel_pos, const int32_t* sel_src,
                             const int32_t* row_dst, const int32_t* n_sel,
                             uint16_t* pool, const uint16_t* host,
                             float* out, float* lse, void* ws,
                             hipStream_t s, int target_wgs,
                             const uint8_t* entries, TailView tail) {
  const MlaPlan p = plan_sparse_mla(d, target_wgs);
  const size_t parts = (size_t)d.batch * d.mtp * p.nchunk * d.mla_heads;
  _Float16* part_acc = static_cast<_Float16*>(ws);
  float4* part_ml = reinterpret_cast<float4*>(
      static_cast<char*>(ws) + align_up(parts * kVal * sizeof(_Float16), 256));
  hipError_t e;
#define ESS_MLA_CASE(W, CH)                                                    \
  e = entries ? launch_t<W, CH, true>(d, p, q_abs, sel_pos, sel_src, row_dst, n_sel, \
                                      pool, host, entries, tail, part_acc, part_ml, s) \
              : launch_t<W, CH, false>(d, p, q_abs, sel_pos, sel_src, row_dst, n_sel, \
                                       pool, host, nullptr, tail, part_acc, part_ml, s)
  // Three or four head blocks: one wave per block with all columns; fewer:
  // two waves per block (column halves), so at least four waves run.
  switch (p.heads_per_wg / 16) {
    case 1: ESS_MLA_CASE(1, 2); break;
    case 2: ESS_MLA_CASE(2, 2); break;
    case 3: ESS_MLA_CASE(3, 1); break;
    default: ESS_MLA_CASE(4, 1); break;
  }
#undef ESS_MLA_CASE
  if (e != hipSuccess) return e;
  // Waves per head: enough that each folds about 8 chunks (one round of
  // loads), when the grid would otherwise hold few workgroups.
  const int bm = d.batch * d.mtp;
  int wph = 1;
  while (wph < 4 && p.nchunk >= 16 * wph && bm * d.mla_heads * wph < 4 * 1024) wph *= 2;
#define ESS_COMBINE(W)                                                         \
  hipLaunchKernelGGL(mla_combine_kernel<W>,                                    \
                     dim3(d.mla_heads / (kCombineThreads / 64 / W), bm),       \
                     dim3(kCombineThreads), 0, s, part_acc, part_ml, out, lse, \
                     d.mla_heads, p.nchunk)
  if (wph == 4)
    ESS_COMBINE(4);
  else if (wph == 2)
    ESS_COMBINE(2);
  else
    ESS_COMBINE(1);
#undef ESS_COMBINE
  return hipGetLastError();
}

// ---- a fixed scratch array for callers that cannot allocate -------------
//
// The attention's split-row partials in a file-scope device array instead of
// a caller workspace.  Each device the library runs on holds its own copy
// (from module load to process exit); its device address is looked up once
// per device with that device current and kept.  The array's host-side name
// is only a stand-in for the symbol: kernels get the looked-up address.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_sparse_mla_noalloc(const ess_dims& d, const uint16_t* q_abs,
                                     const int32_t* sel_pos, const int32_t* sel_src,
                                     const int32_t* row_dst, const int32_t* n_sel,
                                     uint16_t* pool, const uint16_t* host,
                                     float* out, float* lse, hipStream_t s) {
  void* ws = nullptr;
  hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_sparse_mla(d, q_abs, sel_pos, sel_src, row_dst, n_sel, pool, host,
                           out, lse, ws, s);
}

}  // namespace ess
