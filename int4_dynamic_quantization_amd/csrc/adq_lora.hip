// AddLora ("aclnnAddLora", Formulas): rows of x are grouped by their adapter
// index; each group's rows are multiplied by weightA[g, layerIdx] (shrink,
// h1 -> rank) and then by weightB[g, layerIdx] (expand, rank -> h2) and
// scale, and the result is added into columns [y_offset, y_offset + h2) of
// y.  Rows whose index lies outside [0, w) get no contribution.  Arithmetic
// is fp32 (products of 16-bit inputs are exact; Z1 stays fp32 between the two
// products); the slice is rounded once to the storage type.
//
// Tiled path, three launches on the caller's stream (two for batches of up
// to 512 rows with weightA, where each shrink workgroup groups the rows
// itself, in a fixed order, and the expand reads the table they write):
//  1. group: one workgroup builds the page's step 1 in the workspace: a
//     histogram of adapter classes, a table of tiles of up to 64 rows of one
//     class, and the rows listed class by class.  Places within a class are
//     taken with LDS atomics, so the order of rows inside a tile may vary
//     between runs; every row's result is computed from its own data in a
//     fixed order, so outputs do not.
//  2. shrink: one workgroup per (tile, slice of h1), compiled per rank (8,
//     16, 32, 64, 128; rank 8 padded to one 16-wide block), 128 k per stage.
//     The stage of weightA[g, layer] (stored [h1, rank], rank contiguous) is
//     staged in LDS transposed, so each MFMA operand is one 16-byte read; the
//     stage of x (64 rows) reaches LDS through direct-to-LDS loads in whole
//     row pieces, through a ring of LDS buffers (two stages in flight while
//     a third is multiplied; weightA one stage ahead); 4 wavefronts each take 16 rows
//     (v_mfma_f32_16x16x32_{bf16,f16}) and write fp32 partial sums to the
//     workspace.
//  3. expand: one workgroup per (16 rows of a tile, 1024 columns of the
//     slice), all workgroups of a tile on one XCD.  Each thread owns 4
//     adjacent columns: its 16 rows of y, its weightB values (rank <= 16:
//     kept in registers; larger ranks: 16 at a time, every row's sums kept
//     across the chunks) and the partial sums are all requested before
//     anything waits; Z1 = the slices' partial sums added in slice order;
//     fp32 fma chain over the ranks, fma into y, one rounding, 8-byte
//     stores.  Rows
//     without an adapter and, when out is not y, the columns outside the
//     slice are copied here.  bf16 at ranks 32, 64 and 128 takes an expand
//     on the matrix cores instead (z1 split exactly into three bf16 pieces;
//     one workgroup per 64-row tile and 512 columns).
// Generic kernel: one workgroup per row, any sizes and alignments, same
// arithmetic with block reductions in a fixed order.
#include "adq_device.h"


namespace adq {

namespace {


constexpr int kThreads = 256;         // generic, shrink and expand kernels
constexpr int kGroupThreads = 1024;   // group kernel
constexpr int kGroupBatch = 8;        // indices per thread loaded together by the group kernel
constexpr int kTile = kLoraTileRows;  // 64 rows
constexpr int kKSub = 128;            // k per shrink stage
// Transposed weightA rows in LDS: 128 k + 32 of padding (320 bytes, 16 banks
// of offset per row) with the 8-k groups of rows 8..15 (mod 16) swapped in
// pairs (group index ^ 2).  gfx950 reads 128 bits for 16 lanes per pass; for
// every lane grouping that fits the bank-conflict measurements (one half
// wave, parity of lane bits 2 and 4, possibly with bits 0 and 3) the 16
// lanes of a pass then hit 16 distinct 4-bank groups.  Ranks below 16 are
// padded to one 16-wide MFMA block with zero rows.
template <int R> constexpr int stage_k() { return kKSub; }
template <int R> constexpr int at_stride() { return stage_k<R>() + 32; }
template <int R> constexpr int padded_rank() { return R < 16 ? 16 : R; }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

template <int E>
__device__ __forceinline__ f32x4 mfma16(u16x8 a, u16x8 b, f32x4 c) {
  if constexpr (E == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Exclusive prefix of one int per thread over a workgroup of NW wavefronts,
// in thread order; `total` receives the sum.  tmp: NW ints of LDS.
template <int NW>
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, sum = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) base += tmp[w];
    sum += tmp[w];
  }
  *total = sum;
  __syncthreads();
  return base + x - v;
}

__device__ __forceinline__ int adapter_class(int32_t g, int64_t w) {
  return (g >= 0 && g < w) ? g : (int)w;
}

__host__ __device__ inline int64_t lora_max_tiles_dev(const LoraArgs& a) {
  return (a.rows + kTile - 1) / kTile + a.w + 1;
}

struct Workspace {
  int* header;      // [0]: number of tiles
  int4* table;      // per tile: {class, 0, rows, 0}
  int32_t* rows;    // per tile, 64 slots of row ids
  float* z1p;       // [ksplit][tile slot][rank] partial shrink sums
  int* hist;        // batches above kGroupRowsPerWg rows: [workgroup][class] row counts
};

__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// byte offsets of the table, the row list and the partial sums
struct WsOffsets {
  uint64_t table, rows, z1p, hist, end;
};

// Rows grouped by one workgroup of the grouping launches (8 per thread).
constexpr int64_t kGroupRowsPerWg = (int64_t)kGroupThreads * kGroupBatch;

__host__ __device__ inline WsOffsets ws_offsets(const LoraArgs& a) {
  const int64_t tiles = (a.rows + kTile - 1) / kTile + a.w + 1;
  WsOffsets o;
  o.table = 256;
  o.rows = align256(o.table + (uint64_t)tiles * 16);
  o.z1p = align256(o.rows + (uint64_t)tiles * kTile * 4);
  o.hist = align256(o.z1p +
                   (a.wa ? (uint64_t)a.ksplit * (uint64_t)tiles * kTile * (uint64_t)a.rank * 4 : 0));
  const int64_t wgs = a.rows > kGroupRowsPerWg ? (a.rows + kGroupRowsPerWg - 1) / kGroupRowsPerWg : 0;
  o.end = o.hist + (uint64_t)wgs * (uint64_t)(a.w + 1) * 4;
  return o;
}

inline Workspace ws_layout(void* base, const LoraArgs& a) {
  char* p = static_cast<char*>(base);
  const WsOffsets o = ws_offsets(a);
  Workspace w;
  w.header = reinterpret_cast<int*>(p);
  w.table = reinterpret_cast<int4*>(p + o.table);
  w.rows = reinterpret_cast<int32_t*>(p + o.rows);
  w.z1p = reinterpret_cast<float*>(p + o.z1p);
  w.hist = reinterpret_cast<int*>(p + o.hist);
  return w;
}

// ---- 1. grouping
// Batches of up to kGroupRowsPerWg rows: one workgroup counts the rows of
// each adapter class (W + 1, the last for rows without an adapter), lays out
// the tiles and places every row into its tile's slot.  Larger batches: a
// counting launch (one workgroup per kGroupRowsPerWg rows) and a placing
// launch in which each workgroup adds up the counts of the workgroups before
// it, so the rows of a class keep the order of the workgroups that hold them.

// Classes of rows base + u * kGroupThreads + tid (-1 past the end).  All
// loads are in flight before the first is used.
__device__ __forceinline__ void load_classes(const LoraArgs& a, int64_t base,
                                             int (&c)[kGroupBatch]) {
#pragma unroll
  for (int u = 0; u < kGroupBatch; ++u) {
    const int64_t i = base + (int64_t)u * kGroupThreads + threadIdx.x;
    c[u] = i < a.rows ? a.indices[i] : 0;
  }
#pragma unroll
  for (int u = 0; u < kGroupBatch; ++u) {
    const int64_t i = base + (int64_t)u * kGroupThreads + threadIdx.x;
    c[u] = i < a.rows ? adapter_class(c[u], a.w) : -1;
  }
}

// Tiles of up to kTile rows of one class, classes in order, from the row
// counts n[g] of each class: first_tile[g] for every class and, when
// `write`, the table entries and the tile count.  Rows without an adapter are
// only listed when out is not y (to be copied).
__device__ void lay_out_tiles(const LoraArgs& a, const int* n, int* first_tile, int* scan_tmp,
                              const Workspace& ws, bool write) {
  constexpr int NW = kGroupThreads / 64;
  const int tid = threadIdx.x;
  const int64_t W = a.w;
  auto placed = [&](int g) -> int { return (g < W || !a.in_place) ? n[g] : 0; };
  const int per = (int)((W + 1 + kGroupThreads - 1) / kGroupThreads);
  int tl = 0;
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g <= W) tl += (placed(g) + kTile - 1) / kTile;
  }
  int ntiles = 0;
  int tb = block_exclusive_scan<NW>(tl, scan_tmp, &ntiles);
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g <= W) {
      const int m = placed(g);
      if (write)
        for (int t = 0; t * kTile < m; ++t)
          ws.table[tb + t] = int4{g, 0, m - t * kTile < kTile ? m - t * kTile : kTile, 0};
      first_tile[g] = tb;
      tb += (m + kTile - 1) / kTile;
    }
  }
  if (write && tid == 0) ws.header[0] = ntiles;
}

// Rows base + u * kGroupThreads + tid of classes c[u] into their tiles' slots;
// cur[g] is the next position within class g.
__device__ __forceinline__ void place_rows(const LoraArgs& a, const Workspace& ws, int64_t base,
                                           const int (&c)[kGroupBatch], int* cur,
                                           const int* first_tile) {
#pragma unroll
  for (int u = 0; u < kGroupBatch; ++u) {
    if (c[u] >= 0 && (c[u] < a.w || !a.in_place)) {
      const int p = atomicAdd(&cur[c[u]], 1);
      ws.rows[(int64_t)(first_tile[c[u]] + p / kTile) * kTile + p % kTile] =
          (int32_t)(base + (int64_t)u * kGroupThreads + threadIdx.x);
    }
  }
}

__global__ void __launch_bounds__(kGroupThreads) lora_group_kernel(const LoraArgs a,
                                                                   Workspace ws) {
  __shared__ int cnt[kLoraMaxAdapters + 1];
  __shared__ int cur[kLoraMaxAdapters + 1];
  __shared__ int first_tile[kLoraMaxAdapters + 1];
  __shared__ int scan_tmp[kGroupThreads / 64];
  const int tid = threadIdx.x;
  const int64_t W = a.w;
  int c[kGroupBatch];
  load_classes(a, 0, c);
  for (int g = tid; g <= W; g += kGroupThreads) cnt[g] = 0, cur[g] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kGroupBatch; ++u)
    if (c[u] >= 0) atomicAdd(&cnt[c[u]], 1);
  __syncthreads();
  lay_out_tiles(a, cnt, first_tile, scan_tmp, ws, true);
  __syncthreads();
  place_rows(a, ws, 0, c, cur, first_tile);
}

// Larger batches, first launch: the class counts of this workgroup's rows.
__global__ void __launch_bounds__(kGroupThreads) lora_count_kernel(const LoraArgs a,
                                                                   Workspace ws) {
  __shared__ int cnt[kLoraMaxAdapters + 1];
  const int tid = threadIdx.x;
  const int64_t W = a.w;
  int c[kGroupBatch];
  load_classes(a, (int64_t)blockIdx.x * kGroupRowsPerWg, c);
  for (int g = tid; g <= W; g += kGroupThreads) cnt[g] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kGroupBatch; ++u)
    if (c[u] >= 0) atomicAdd(&cnt[c[u]], 1);
  __syncthreads();
  for (int g = tid; g <= W; g += kGroupThreads) ws.hist[(int64_t)blockIdx.x * (W + 1) + g] = cnt[g];
}

// Larger batches, second launch: class totals and this workgroup's first
// position in each class from the counts of every workgroup, the tiles
// (written by workgroup 0; every workgroup derives the same layout), then
// this workgroup's rows placed.
__global__ void __launch_bounds__(kGroupThreads) lora_place_kernel(const LoraArgs a,
                                                                   Workspace ws) {
  __shared__ int tot[kLoraMaxAdapters + 1];
  __shared__ int cur[kLoraMaxAdapters + 1];
  __shared__ int first_tile[kLoraMaxAdapters + 1];
  __shared__ int scan_tmp[kGroupThreads / 64];
  const int tid = threadIdx.x;
  const int64_t W = a.w;
  const int wg = (int)blockIdx.x, nwg = (int)gridDim.x;
  const int64_t base = (int64_t)wg * kGroupRowsPerWg;
  int c[kGroupBatch];
  load_classes(a, base, c);
  for (int g = tid; g <= W; g += kGroupThreads) {
    int total = 0, before = 0;
    for (int w0 = 0; w0 < nwg; w0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = w0 + u < nwg ? ws.hist[(int64_t)(w0 + u) * (W + 1) + g] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        total += v[u];
        if (w0 + u < wg) before += v[u];
      }
    }
    tot[g] = total;
    cur[g] = before;
  }
  __syncthreads();
  lay_out_tiles(a, tot, first_tile, scan_tmp, ws, wg == 0);
  __syncthreads();
  place_rows(a, ws, base, c, cur, first_tile);
}

// ---- 1'. grouping inside the shrink, for small batches
// One workgroup finds the rows of one tile under a stable grouping: classes
// in order, the rows of a class in index order, tiles of up to 64 rows —
// the same tile count and table shape as the grouping kernel, with a fixed
// order, so every workgroup computes the same grouping.  Up to kSmallRows
// rows (kSmallRows / kThreads per thread, thread t holding rows in index
// order).  On return (after a barrier): info[0] = the tile's class (-1 past
// the last tile), info[1] = its row count, info[2] = the tile count, and
// rows_lds[0 .. info[1]) its rows.
constexpr int kSmallRows = 512;

__device__ void group_one_tile(const LoraArgs& a, int tile, int* cnt, int* scan_tmp, int* info,
                               int64_t* rows_lds) {
  constexpr int NW = kThreads / 64;
  constexpr int RPT = kSmallRows / kThreads;
  const int tid = threadIdx.x;
  const int64_t W = a.w;
  int cls[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int64_t i = (int64_t)tid * RPT + u;
    cls[u] = i < a.rows ? adapter_class(a.indices[i], W) : -1;
  }
  for (int g = tid; g <= W; g += kThreads) cnt[g] = 0;
  if (tid == 0) info[0] = -1;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < RPT; ++u)
    if (cls[u] >= 0) atomicAdd(&cnt[cls[u]], 1);
  __syncthreads();
  // rows without an adapter are only listed when out is not y (to be copied)
  auto placed = [&](int g) -> int { return (g < W || !a.in_place) ? cnt[g] : 0; };
  const int per = (int)((W + 1 + kThreads - 1) / kThreads);
  int tl = 0;
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g <= W) tl += (placed(g) + kTile - 1) / kTile;
  }
  int ntiles = 0;
  int tb = block_exclusive_scan<NW>(tl, scan_tmp, &ntiles);
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g <= W) {
      const int nt = (placed(g) + kTile - 1) / kTile;
      if (tile >= tb && tile < tb + nt) {
        const int s = tile - tb;
        info[0] = g;
        info[1] = placed(g) - s * kTile < kTile ? placed(g) - s * kTile : kTile;
        info[3] = s;
      }
      tb += nt;
    }
  }
  if (tid == 0) info[2] = ntiles;
  __syncthreads();
  const int g = info[0], s = info[3];
  if (g < 0) return;  // uniform
  int m = 0;
#pragma unroll
  for (int u = 0; u < RPT; ++u) m += cls[u] == g;
  int total = 0;
  int r = block_exclusive_scan<NW>(m, scan_tmp, &total);  // place within the class
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    if (cls[u] == g) {
      if (r >= s * kTile && r < (s + 1) * kTile) rows_lds[r - s * kTile] = (int64_t)tid * RPT + u;
      ++r;
    }
  }
  __syncthreads();
}

// ---- 2. shrink: partial z1 over one slice of h1 for one tile
// G: the workgroup groups the rows itself (small batches, no grouping
// launch); the workgroups of slice 0 then write their tile's table entry
// and row slots, and workgroup 0 the tile count, for the expand.
template <int E, int R, bool G>
__global__ void __launch_bounds__(kThreads) lora_shrink_kernel(const LoraArgs a, Workspace ws) {
  constexpr int RP = padded_rank<R>();
  constexpr int KS = stage_k<R>();
  // x stage in LDS: 64 rows of KS k, each wave's 16-byte loads landing as
  // 1 KB pieces (RPS whole rows of CPR 16-byte chunks, lane l at byte 16 l);
  // the chunk c of row r sits at position c ^ (r % 16), so the 16-byte MFMA
  // fragment reads of 16 rows hit distinct banks
  constexpr int CPR = KS / 8, RPS = 64 / CPR, SPW = kTile / RPS / 4;
  __shared__ int64_t rows_lds[kTile];
  __shared__ __attribute__((aligned(16))) uint16_t at[RP][at_stride<R>()];
  __shared__ __attribute__((aligned(16))) uint16_t xs[kTile * KS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile = (int)(blockIdx.x / a.ksplit);
  const int ks = (int)(blockIdx.x % a.ksplit);
  if constexpr (RP > R) {  // padding rows: zero once, never staged
    for (int p = tid; p < (RP - R) * at_stride<R>(); p += kThreads)
      at[R + p / at_stride<R>()][p % at_stride<R>()] = 0;
  }
  int g, n;
  if constexpr (G) {
    __shared__ int cnt[kLoraMaxAdapters + 1];
    __shared__ int scan_tmp[kThreads / 64];
    __shared__ int info[4];
    group_one_tile(a, tile, cnt, scan_tmp, info, rows_lds);
    g = info[0], n = info[1];
    if (blockIdx.x == 0 && tid == 0) ws.header[0] = info[2];
    if (g < 0) return;  // past the last tile
    if (ks == 0) {
      if (tid == 0) ws.table[tile] = int4{g, 0, n, 0};
      if (tid < n) ws.rows[(int64_t)tile * kTile + tid] = (int32_t)rows_lds[tid];
    }
    if (g >= a.w) return;  // rows without an adapter
  } else {
    const int ntiles = ws.header[0];
    const int4 te = ws.table[tile < ntiles ? tile : 0];
    const int32_t rid = ws.rows[(int64_t)tile * kTile + tid % kTile];  // with the table
    if (tile >= ntiles) return;
    g = te.x, n = te.z;
    if (g >= a.w) return;  // rows without an adapter
    if (tid < n) rows_lds[tid] = rid;
  }
  using T = uint16_t;
  constexpr int64_t rank = R;
  const int64_t h1 = a.h1;
  constexpr int nb = RP / 16;
  const T* wa = static_cast<const T*>(a.wa) + ((g * a.l + a.layer) * h1) * rank;
  const T* x = static_cast<const T*>(a.x);
  const int64_t kc = ((h1 + a.ksplit - 1) / a.ksplit + 31) / 32 * 32;
  const int64_t k_lo = ks * kc;
  const int64_t k_hi = k_lo + kc < h1 ? k_lo + kc : h1;

  const int fi = lane & 15, fk = lane >> 4;
  const int rb = 16 * wave;  // this wavefront's rows of the tile
  f32x4 acc[nb];
#pragma unroll
  for (int b = 0; b < nb; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  // this lane's chunk of x in each of its wave's segments: byte offset of
  // the row (all ones past the tile's rows) and k of the chunk in a stage
  const rsrc_t rx = make_rsrc(x, (uint32_t)(a.rows * h1 * 2));
  uint32_t xo[SPW];
  int xk[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int r = RPS * (wave * SPW + i) + lane / CPR;
    const int c = (lane % CPR) ^ (r & 15);
    xk[i] = 8 * c;
    xo[i] = r < n ? (uint32_t)(rows_lds[r] * h1 * 2) + 16u * c : 0xFFFFFFFFu;
  }
  // Pipeline: x and weightA of stage st + 1 are requested, into registers,
  // while stage st is staged and multiplied (more stages ahead measured
  // slower: rank 16 shrink 10.95 us with one, 11.84 with two, 13.68 with
  // three on 4096 rows, h1 4096).  Stages reach LDS through ordinary LDS
  // writes, not direct-to-LDS loads: a read of LDS that such a load might
  // still be writing makes the compiler wait for all loads in flight, which
  // drained the pipeline before every stage (11.43 us).
  // x is read with the default cache policy (the streaming one measured
  // slower here: shrink 11.2 against 10.3 us on 4096 rows at rank 16).
  // Lanes with nothing to fetch (rows past the tile, k past the slice) read
  // past the end of a buffer descriptor, which yields zeros; weightA is
  // fetched by the threads that stage it only (at rank 16, half a wave: each
  // load instruction costs issue time whether or not its lanes fetch).
  // weightA stage: blocks of 8 k x 8 ranks, one per thread (threads t and
  // t + 1 take neighbouring 8-k groups of the same 8 ranks), loaded as 8
  // rows of 16 bytes, transposed in registers and written as 8 rank rows
  // of 16 bytes: 16 lanes of a row group write 16 distinct 16-byte slots
  constexpr int KG = KS / 8, NBLK = KG * (R / 8);
  static_assert(NBLK <= kThreads, "one weightA block per thread");
  const int bkg = tid % KG, brg = tid / KG;
  const bool blk = tid < NBLK;
  const rsrc_t rwa = make_rsrc(wa, (uint32_t)(h1 * rank * 2));
  auto stage_n = [&](int64_t sub) -> int {  // k of a stage inside the slice (<= 0 past it)
    const int64_t v = k_hi - sub;
    return (int)(v < KS ? (v > 0 ? v : 0) : KS);
  };
  auto load_x = [&](int64_t sub, u32x4(&xv)[SPW]) {
    const int sub_n = stage_n(sub);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const uint32_t off =
          xo[i] != 0xFFFFFFFFu && xk[i] < sub_n ? xo[i] + (uint32_t)(sub * 2) : 0xFFFFFFF0u;
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
    }
  };
  auto load_wa = [&](int64_t sub, u16x8(&w)[8]) {  // threads with a block only
    const int sub_n = stage_n(sub);
    if (blk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 8 * bkg + e;
        const uint32_t off = k < sub_n ? (uint32_t)((sub + k) * rank * 2) + 16u * brg : 0xFFFFFFF0u;
        w[e] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rwa, off, 0, 0));
      }
    }
  };
  u32x4* xs_lane = reinterpret_cast<u32x4*>(xs) + (wave * SPW * 64 + lane);
  auto stage = [&](int st, u32x4(&xv)[SPW], u16x8(&w)[8]) {
    const int64_t sub = k_lo + (int64_t)st * KS;
    const int steps = (stage_n(sub) + 31) / 32;
#pragma unroll
    for (int i = 0; i < SPW; ++i) xs_lane[i * 64] = xv[i];
    if (blk) {  // weightA staged transposed
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        u16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = w[e][q];
        const int r = 8 * brg + q;
        *reinterpret_cast<u16x8*>(&at[r][8 * (bkg ^ (((r >> 3) & 1) << 1))]) = t;
      }
    }
    load_wa(sub + KS, w);
    load_x(sub + KS, xv);
    __syncthreads();
    if (rb < n) {  // wavefront-uniform
#pragma unroll
      for (int u = 0; u < KS / 32; ++u) {
        if (u < steps) {
          const int kg = 4 * u + fk;
          const u16x8 xa = *reinterpret_cast<const u16x8*>(&xs[(rb + fi) * KS + 8 * (kg ^ fi)]);
#pragma unroll
          for (int b = 0; b < nb; ++b) {
            const int r = 16 * b + fi;
            const u16x8 bv =
                *reinterpret_cast<const u16x8*>(&at[r][8 * (kg ^ (((r >> 3) & 1) << 1))]);
            acc[b] = mfma16<E>(xa, bv, acc[b]);
          }
        }
      }
    }
    __syncthreads();  // before the next stage overwrites `at` and x
  };
  const int nst = k_hi > k_lo ? (int)((k_hi - k_lo + KS - 1) / KS) : 0;
  u32x4 xv[SPW];
  u16x8 wv[8];
  load_wa(k_lo, wv);
  load_x(k_lo, xv);
  for (int st = 0; st < nst; ++st) stage(st, xv, wv);
  wait_vmcnt<0>();  // the requests past the last stage
  // element e of lane l: row rb + 4 * (l / 16) + e, rank l % 16 (+ 16 * block)
  float* zp = ws.z1p + ((int64_t)ks * lora_max_tiles_dev(a) + tile) * kTile * rank;
#pragma unroll
  for (int b = 0; b < nb; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = rb + 4 * fk + e;
        if (i < n && 16 * b + fi < R) zp[i * rank + 16 * b + fi] = acc[b][e];
      }
}

// ---- 3. expand + accumulate for 16 rows of one tile and 1024 columns
// Thread t owns columns 4t .. 4t + 3 of the range.  All 16 rows' y values
// (8 bytes each), the thread's weightB values and the partial sums are
// requested before anything waits; then z1 (the slices' partial sums added
// in slice order) goes to LDS, and each output is one fp32 fma chain over
// the ranks, one fma into y, one rounding, an 8-byte store.
constexpr int kQRows = 16;                  // rows per workgroup
constexpr int kQuarters = kTile / kQRows;   // workgroups per tile and column range
// Threads of an expand workgroup (4 columns each): 256, or fewer for
// slices that would leave waves of a 256-thread workgroup without columns:
// 64 / 128 for up to 256 / 512 columns at ranks up to 16, 128 for up to 512
// at rank 32 (with 64 its partial sums would be fetched in 4 rounds).
__host__ __device__ constexpr int expand_threads(int64_t h2, int64_t rank) {
  if (rank <= 16) return h2 <= 256 ? 64 : h2 <= 512 ? 128 : kThreads;
  return rank <= 32 && h2 <= 512 ? 128 : kThreads;
}

template <int E, int R, int NT>
__global__ void __launch_bounds__(NT) lora_expand_kernel(const LoraArgs a, Workspace ws) {
  __shared__ __attribute__((aligned(16))) float z1[kQRows][R];
  const int tid = threadIdx.x;
  // workgroup b runs on XCD b % 8 (the dispatcher deals workgroups to the XCDs
  // in turn): all workgroups of a tile go to one XCD, so its partial sums
  // and its adapter's weightB are fetched into one L2
  const int per_tile = kQuarters * a.chunks;
  const int xcd = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
  const int tile = xcd + 8 * (j / per_tile);
  const int qt = (j % per_tile) / a.chunks;
  const int chunk = (j % per_tile) % a.chunks;
  // the tile count, the tile's entry and its row slots are read together
  // (slots past the workspace's tiles are never read: tc < max tiles)
  const int64_t mt = lora_max_tiles_dev(a);
  const int tc = tile < mt ? tile : 0;
  const int ntiles = ws.header[0];
  const int4 te = ws.table[tc];
  const int4* rq = reinterpret_cast<const int4*>(ws.rows + (int64_t)tc * kTile + qt * kQRows);
  int32_t rows[kQRows];
#pragma unroll
  for (int u = 0; u < kQRows / 4; ++u) {
    const int4 v = rq[u];
    rows[4 * u] = v.x, rows[4 * u + 1] = v.y, rows[4 * u + 2] = v.z, rows[4 * u + 3] = v.w;
  }
  if (tile >= ntiles) return;
  const int g = te.x;
  const int n = te.z - qt * kQRows < kQRows ? te.z - qt * kQRows : kQRows;
  if (n <= 0) return;
  using T = uint16_t;
  const T* y = static_cast<const T*>(a.y);
  T* out = static_cast<T*>(a.out);
  const int64_t h3 = a.h3;
  // this range's share of whole rows (copies when out is not y), in groups of 4 columns
  const int64_t ncg_row = h3 / 4;
  const int64_t per_row = (ncg_row + a.chunks - 1) / a.chunks;
  const int64_t c0 = chunk * per_row;
  const int64_t c1 = c0 + per_row < ncg_row ? c0 + per_row : ncg_row;
  if (g >= a.w) {  // rows without an adapter (listed only when out is not y): copy
    for (int i = 0; i < n; ++i) {
      const int64_t row = rows[i];
      for (int64_t c4 = c0 + tid; c4 < c1; c4 += NT)
        *reinterpret_cast<uint2*>(out + row * h3 + 4 * c4) =
            *reinterpret_cast<const uint2*>(y + row * h3 + 4 * c4);
    }
    return;
  }
  const int64_t col = (int64_t)chunk * (4 * NT) + 4 * tid;  // first column of the slice
  const bool col_ok = col < a.h2;

  // y: every row's 4 values, all loads in flight together (rows*h3*2 < 2^32);
  // lanes past the slice read nothing
  const rsrc_t ry = make_rsrc(y, (uint32_t)(a.rows * h3 * 2));
  const uint32_t col_off = col_ok ? (uint32_t)((a.y_offset + col) * 2) : 0xFFFFFFF0u;
  uint2 yv[kQRows];
#pragma unroll
  for (int i = 0; i < kQRows; ++i) {
    yv[i] = uint2{0u, 0u};
    if (i < n) {
      const uint32_t off = col_ok ? (uint32_t)(rows[i] * h3 * 2) + col_off : col_off;
      yv[i] = __builtin_bit_cast(uint2,
                                 __builtin_amdgcn_raw_buffer_load_b64(ry, off, 0, kStreamLoad));
    }
  }

  // weightB for this thread's columns (rank <= 16: held in registers),
  // issued right behind y
  constexpr int RB = R <= 16 ? R : 1;  // ranks held in registers
  const T* wb = static_cast<const T*>(a.wb) + ((g * a.l + a.layer) * R) * a.h2;
  u16x4 bwr[RB];
  if constexpr (R <= 16) {
    const rsrc_t rb = make_rsrc(wb, (uint32_t)(R * a.h2 * 2));
#pragma unroll
    for (int r = 0; r < R; ++r)
      bwr[r] = __builtin_bit_cast(
          u16x4, __builtin_amdgcn_raw_buffer_load_b64(
                     rb, col_ok ? (uint32_t)((r * a.h2 + col) * 2) : 0xFFFFFFF0u, 0, 0));
  }

  // z1 = the slices' partial sums, added in slice order (or x itself without
  // weightA).  The first kZS slices are loaded together, behind y and
  // weightB, with no wait in between; indices past the valid ones are
  // clamped to a valid slot and their values dropped.
  constexpr int ZP = (kQRows * R + NT - 1) / NT;  // elements per thread
  constexpr int kZS = ZP >= 16 ? 1 : 16 / ZP;  // slices loaded together (kZS * ZP <= 16)
  if (a.wa) {
    const int ksn = a.ksplit;
    float zs[ZP];
    int64_t zi[ZP];
#pragma unroll
    for (int u = 0; u < ZP; ++u) {
      const int t = tid + u * NT;
      const int i = t / R < n ? t / R : 0, r = t % R;
      zi[u] = ((int64_t)tile * kTile + qt * kQRows + i) * R + r;
    }
    const int64_t kstride = mt * kTile * R;
    float p[kZS][ZP];
#pragma unroll
    for (int k = 0; k < kZS; ++k)
#pragma unroll
      for (int u = 0; u < ZP; ++u) p[k][u] = ws.z1p[(k < ksn ? k : 0) * kstride + zi[u]];
    // slices past the valid ones add +0 (their bits masked off): a partial
    // sum is never -0 (the MFMA sums start from +0), so this is exact, and
    // every load is used on every path (none is sunk behind a branch)
#pragma unroll
    for (int u = 0; u < ZP; ++u) {
      zs[u] = p[0][u];
#pragma unroll
      for (int k = 1; k < kZS; ++k) {
        const uint32_t keep = k < ksn ? 0xFFFFFFFFu : 0u;
        zs[u] += __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p[k][u]) & keep);
      }
    }
    for (int k = kZS; k < ksn; ++k)
#pragma unroll
      for (int u = 0; u < ZP; ++u) zs[u] += ws.z1p[k * kstride + zi[u]];
#pragma unroll
    for (int u = 0; u < ZP; ++u) {
      const int t = tid + u * NT;
      if (t < kQRows * R) z1[t / R][t % R] = t / R < n ? zs[u] : 0.0f;
    }
  } else {
    for (int t = tid; t < kQRows * R; t += NT) {
      const int i = t / R, r = t % R;
      z1[i][r] = i < n ? widen1<E>(static_cast<const T*>(a.x)[(int64_t)rows[i] * a.h1 + r])
                       : 0.0f;
    }
  }
  __syncthreads();
  // out = y + scale * (z1 . weightB), one fp32 fma chain over the ranks in
  // rank order per output, one fma into y, one rounding
  const rsrc_t rout = make_rsrc(out, (uint32_t)(a.rows * h3 * 2));
  auto store_row = [&](int i, const float (&acc)[4]) {
    const u16x4 yq = __builtin_bit_cast(u16x4, yv[i]);
    u16x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = narrow1<E>(__builtin_fmaf(acc[q], a.scale, widen1<E>(yq[q])));
    __builtin_amdgcn_raw_buffer_store_b64(
        __builtin_bit_cast(u32x2, o), rout,
        (uint32_t)(((int64_t)rows[i] * h3 + a.y_offset + col) * 2), 0, kStreamStore);
  };
  if (col_ok) {
    if constexpr (R <= 16) {
      // weightB in registers, one row at a time
      float br[RB][4];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) br[r][q] = widen1<E>(bwr[r][q]);
#pragma unroll
      for (int i = 0; i < kQRows; ++i) {
        if (i < n) {
          float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int r4 = 0; r4 < R; r4 += 4) {
            const f32x4 zz = *reinterpret_cast<const f32x4*>(&z1[i][r4]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(zz[u], br[r4 + u][q], acc[q]);
          }
          store_row(i, acc);
        }
      }
    } else {
      // 16 ranks of weightB at a time in registers, every row's sums kept
      // across the chunks (each weightB value is read once per workgroup)
      float acc[kQRows][4];
#pragma unroll
      for (int i = 0; i < kQRows; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;
#pragma unroll 1
      for (int rc = 0; rc < R; rc += 16) {
        float b[16][4];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const u16x4 v = *reinterpret_cast<const u16x4*>(wb + (rc + r) * a.h2 + col);
#pragma unroll
          for (int q = 0; q < 4; ++q) b[r][q] = widen1<E>(v[q]);
        }
#pragma unroll
        for (int i = 0; i < kQRows; ++i) {
          if (i < n) {
#pragma unroll
            for (int r4 = 0; r4 < 16; r4 += 4) {
              const f32x4 zz = *reinterpret_cast<const f32x4*>(&z1[i][rc + r4]);
#pragma unroll
              for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  acc[i][q] = __builtin_fmaf(zz[u], b[r4 + u][q], acc[i][q]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kQRows; ++i)
        if (i < n) store_row(i, acc[i]);
    }
  }

  if (!a.in_place) {  // this range's columns outside the slice
    const int64_t s0 = a.y_offset / 4, s1 = (a.y_offset + a.h2) / 4;
    for (int i = 0; i < n; ++i) {
      const int64_t row = rows[i];
      for (int64_t c4 = c0 + tid; c4 < c1; c4 += NT)
        if (c4 < s0 || c4 >= s1)
          *reinterpret_cast<uint2*>(out + row * h3 + 4 * c4) =
              *reinterpret_cast<const uint2*>(y + row * h3 + 4 * c4);
    }
  }
}

// ---------------------------------------------------------------------------
// Expand on the matrix cores (bf16, ranks 32, 64, 128, where the fp32 sums of
// the kernel above are bound by the vector ALUs).  out[row][col] = y + scale
// * sum_r z1[row][r] weightB[r][col] as v_mfma_f32_16x16x32_bf16 products:
// each fp32 z1 value is split exactly into three bf16 pieces (hi, mid, lo;
// 8 + 8 + 8 significant bits), every product of a piece with a weightB value
// is exact, and the sums run in fp32 inside the matrix unit.
//
// One workgroup per (tile of up to 64 rows, 64 columns per wavefront of the slice), all
// workgroups of a tile on one XCD, so weightB is read once per 64 rows.  Wave
// w takes 64 columns and every 16-row block of the tile.  MFMA operand A is
// weightB: lane l reads the 4 adjacent columns c(l % 16) of 8 ranks with
// 8-byte loads straight from memory, and the q-th of the 4 columns forms the
// q-th A operand, so no transposition is needed: MFMA q yields the columns
// c(m) + q.  With c(m) below, lane l's results are row l % 16 and columns
// 8 (l / 16) + {0..7} and 32 + 8 (l / 16) + {0..7} of the wave's 64.
// Operand B is z1's pieces, staged in LDS once per workgroup as three bf16
// planes [64 rows][rank]; per chunk of 32 ranks one MFMA per piece.  y and
// out cross LDS so that memory is read and written in whole row pieces
// pieces; y is loaded after the products, which keeps the registers (and so
// the occupancy) of the kernel low.
// Wavefronts per workgroup, 64 columns each: every workgroup of a tile reads
// all of the tile's partial sums, so wider workgroups read them fewer times.
// Step time on 4096 rows, h1 4096 -> h2 4096 (bf16, 8 adapters), 4 / 8 / 16
// wavefronts: rank 32 42.5 / 40.0 / 41.9 us, rank 64 55.3 / 47.8 / 49.3,
// rank 128 70.4 / 61.1 / 63.8 (16: one workgroup per CU, 288 of them).
constexpr int kMxWaves = 8;
constexpr int kMxMinRank = 32;  // below, the kernel above is faster (measured)

// first of the 4 columns that MFMA row m of a wave's 64 columns holds
__device__ __forceinline__ int mx_col(int m) {
  return 8 * (m >> 2) + 4 * (m & 1) + 32 * ((m >> 1) & 1);
}
// piece-plane row stride in elements: rows 16 bytes apart modulo 256 bytes,
// so the 16-byte reads of 16 consecutive rows hit distinct banks
template <int R> constexpr int mx_stride() { return R + 8; }

int lora_mx_col_blocks(int64_t h2) {
  const int64_t c = (h2 + 64 * kMxWaves - 1) / (64 * kMxWaves);
  return (int)(c < 1 ? 1 : c);
}

template <int R, int NW>
__global__ void __launch_bounds__(64 * NW) lora_expand_mx_kernel(const LoraArgs a,
                                                                   Workspace ws) {
  static_assert(R >= 32 && R % 32 == 0, "ranks of 32 and above");
  constexpr int NT = 64 * NW, kMxCols = 64 * NW;  // threads, columns per workgroup
  constexpr int NP = 3, ZS = mx_stride<R>();  // pieces, plane row stride
  constexpr int RC = 32;                      // ranks per chunk
  // LDS: z1's pieces during the products, then the tile's y / out block
  // [64 rows][64 NW columns + 8] (rows 16 bytes apart modulo 256 bytes)
  constexpr int YS = kMxCols + 8;
  constexpr int kZBytes = NP * kTile * ZS * 2, kYBytes = kTile * YS * 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kZBytes > kYBytes ? kZBytes : kYBytes];
  auto zp = reinterpret_cast<uint16_t (*)[kTile][ZS]>(lds);
  auto yb = reinterpret_cast<uint16_t (*)[YS]>(lds);
  using T = uint16_t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, lq = lane >> 4;
  const int ncb = (int)((a.h2 + kMxCols - 1) / kMxCols);
  const int xcd = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
  const int tile = xcd + 8 * (j / ncb), cb = j % ncb;
  const int64_t mt = lora_max_tiles_dev(a);
  const int tc = tile < mt ? tile : 0;
  const int ntiles = ws.header[0];
  const int4 te = ws.table[tc];
  const int32_t* trows = ws.rows + (int64_t)tc * kTile;
  int32_t myrow[4];  // this lane's row in each 16-row block
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) myrow[rb] = trows[16 * rb + m];
  if (tile >= ntiles) return;
  const int g = te.x, n = te.z;
  const T* y = static_cast<const T*>(a.y);
  T* out = static_cast<T*>(a.out);
  const int64_t h3 = a.h3;
  // this workgroup's share of whole rows (copies when out is not y)
  const int64_t ncg_row = h3 / 4;
  const int64_t per_row = (ncg_row + ncb - 1) / ncb;
  const int64_t c0 = cb * per_row;
  const int64_t c1 = c0 + per_row < ncg_row ? c0 + per_row : ncg_row;
  if (g >= a.w) {  // rows without an adapter (listed only when out is not y): copy
    for (int i = 0; i < n; ++i) {
      const int64_t row = trows[i];
      for (int64_t c4 = c0 + tid; c4 < c1; c4 += NT)
        *reinterpret_cast<uint2*>(out + row * h3 + 4 * c4) =
            *reinterpret_cast<const uint2*>(y + row * h3 + 4 * c4);
    }
    return;
  }
  const int rbn = (n + 15) / 16;  // row blocks holding rows (uniform)
  const int64_t colw = (int64_t)cb * kMxCols + 64 * wave;

  // weightB: this lane's 4 columns for 8 ranks of a chunk
  const T* wb = static_cast<const T*>(a.wb) + ((g * a.l + a.layer) * R) * a.h2;
  const rsrc_t rwb = make_rsrc(wb, (uint32_t)(R * a.h2 * 2));
  const int64_t wc = colw + mx_col(m);
  const bool wok = wc < a.h2;
  const int ro = 8 * lq;  // first of the lane's 8 ranks in a chunk
  auto load_w = [&](int rc, u16x4 (&w)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = rc + ro + e;
      w[e] = __builtin_bit_cast(
          u16x4, __builtin_amdgcn_raw_buffer_load_b64(
                     rwb, wok ? (uint32_t)((r * a.h2 + wc) * 2) : 0xFFFFFFF0u, 0, 0));
    }
  };
  u16x4 wv[8];
  load_w(0, wv);

  // z1 = the slices' partial sums added in slice order (or x itself without
  // weightA), 4 ranks per access, split into its pieces in LDS; rows past
  // the tile's are zero
  constexpr int NV4 = kTile * R / 4;                         // groups of 4 ranks
  constexpr int ZP4 = (NV4 + NT - 1) / NT;       // groups per thread
  constexpr int KB = ZP4 >= 8 ? 1 : 8 / ZP4;                // slices loaded together
  f32x4 zs[ZP4];
  if (a.wa) {
    const int ksn = a.ksplit;
    const int64_t kstride = mt * kTile * R / 4;
    const f32x4* zb = reinterpret_cast<const f32x4*>(ws.z1p + (int64_t)tile * kTile * R);
    int zi[ZP4];
#pragma unroll
    for (int u = 0; u < ZP4; ++u) {
      const int v = tid + u * NT;
      zi[u] = v < NV4 && 4 * v / R < n ? v : 0;
      zs[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = 0; k0 < ksn; k0 += KB) {
      f32x4 p[KB][ZP4];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int k = k0 + kk < ksn ? k0 + kk : k0;
#pragma unroll
        for (int u = 0; u < ZP4; ++u) p[kk][u] = zb[k * kstride + zi[u]];
      }
      // slices past the valid ones add +0 (bits masked off); each component
      // is read into a scalar first (a bit cast taken straight from a vector
      // component compiled to a read of component 0)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const uint32_t keep = k0 + kk < ksn ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int u = 0; u < ZP4; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float pc = p[kk][u][c];
            zs[u][c] += __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, pc) & keep);
          }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < ZP4; ++u) {
      const int v = tid + u * NT;
      const int i = v < NV4 && 4 * v / R < n ? 4 * v / R : 0;
      const u16x4 xv = *reinterpret_cast<const u16x4*>(static_cast<const T*>(a.x) +
                                                        (int64_t)trows[i] * a.h1 + 4 * v % R);
#pragma unroll
      for (int c = 0; c < 4; ++c) zs[u][c] = widen1<kBF16>(xv[c]);
    }
  }
#pragma unroll
  for (int u = 0; u < ZP4; ++u) {
    const int v = tid + u * NT, i = 4 * v / R, r = 4 * v % R;
    if (v < NV4) {
      u16x4 hi, mid, lo;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float z = i < n ? zs[u][c] : 0.0f;
        hi[c] = narrow1<kBF16>(z);
        const float r1 = z - widen1<kBF16>(hi[c]);
        mid[c] = narrow1<kBF16>(r1);
        lo[c] = narrow1<kBF16>(r1 - widen1<kBF16>(mid[c]));
      }
      *reinterpret_cast<u16x4*>(&zp[0][i][r]) = hi;
      *reinterpret_cast<u16x4*>(&zp[1][i][r]) = mid;
      *reinterpret_cast<u16x4*>(&zp[2][i][r]) = lo;
    }
  }
  __syncthreads();

  f32x4 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[rb][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rc = 0; rc < R; rc += RC) {
    u16x4 wn[8];
    if (rc + RC < R) load_w(rc + RC, wn);  // next chunk in flight
    u16x8 av[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) av[q][e] = wv[e][q];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb < rbn) {
        u16x8 bv[NP];
#pragma unroll
        for (int pc = 0; pc < NP; ++pc)
          bv[pc] = *reinterpret_cast<const u16x8*>(&zp[pc][16 * rb + m][rc + ro]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int pc = 0; pc < NP; ++pc) acc[rb][q] = mfma16<kBF16>(av[q], bv[pc], acc[rb][q]);
      }
    }
    if (rc + RC < R) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = wn[e];
    }
  }

  // out = y + scale * sum, one rounding: y goes through LDS into the MFMA
  // layout, each lane turns its values into out in place, and the block is
  // stored row by row as it was loaded
  // y: the block's rows, 16 bytes per access, TPR threads per row (16 TPR
  // contiguous bytes), issued first.  An 8-column group that starts inside
  // the slice stays inside y's row (h3 and y_offset are multiples of 8).
  constexpr int TPR = kMxCols / 8;                     // threads per row piece
  constexpr int kYChunks = kTile * kMxCols / 8 / NT;  // 8 per thread
  const rsrc_t rout = make_rsrc(out, (uint32_t)(a.rows * h3 * 2));
  const rsrc_t ry = make_rsrc(y, (uint32_t)(a.rows * h3 * 2));
  const int64_t colb = (int64_t)cb * kMxCols + 8 * (tid % TPR);  // this thread's 8 columns
  u16x8 yv[kYChunks];
  int32_t yrow[kYChunks];
#pragma unroll
  for (int k = 0; k < kYChunks; ++k) {
    const int rs = tid / TPR + NT / TPR * k;
    yrow[k] = trows[rs];
    const bool ok = rs < n && colb < a.h2;
    yv[k] = __builtin_bit_cast(
        u16x8, __builtin_amdgcn_raw_buffer_load_b128(
                   ry, ok ? (uint32_t)((yrow[k] * h3 + a.y_offset + colb) * 2) : 0xFFFFFFF0u, 0,
                   kStreamLoad));
  }
  __syncthreads();  // every wave is done with z1's pieces
#pragma unroll
  for (int k = 0; k < kYChunks; ++k)
    *reinterpret_cast<u16x8*>(&yb[tid / TPR + NT / TPR * k][8 * (tid % TPR)]) = yv[k];
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb < rbn) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u16x8* yp = reinterpret_cast<u16x8*>(&yb[16 * rb + m][64 * wave + 8 * lq + 32 * h]);
        const u16x8 yq = *yp;
        u16x8 o;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          o[t] = narrow1<kBF16>(
              __builtin_fmaf(acc[rb][t & 3][2 * h + (t >> 2)], a.scale, widen1<kBF16>(yq[t])));
        *yp = o;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kYChunks; ++k) {
    const int rs = tid / TPR + NT / TPR * k;
    if (rs < n && colb < a.h2) {
      const u16x8 o = *reinterpret_cast<const u16x8*>(&yb[rs][8 * (tid % TPR)]);
      const uint32_t off = (uint32_t)(((int64_t)yrow[k] * h3 + a.y_offset + colb) * 2);
      if (colb + 8 <= a.h2)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rout, off, 0,
                                               kStreamStore);
      else
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(u32x2, u16x4{o[0], o[1], o[2], o[3]}), rout, off, 0, kStreamStore);
    }
  }

  if (!a.in_place) {  // this workgroup's columns outside the slice
    const int64_t s0 = a.y_offset / 4, s1 = (a.y_offset + a.h2) / 4;
    for (int i = 0; i < n; ++i) {
      const int64_t row = trows[i];
      for (int64_t c4 = c0 + tid; c4 < c1; c4 += NT)
        if (c4 < s0 || c4 >= s1)
          *reinterpret_cast<uint2*>(out + row * h3 + 4 * c4) =
              *reinterpret_cast<const uint2*>(y + row * h3 + 4 * c4);
    }
  }
}

// Sum over the workgroup in a fixed order (DPP within wavefronts, then the
// four wavefront totals in order); every thread gets the result.
__device__ float block_sum(float v, float* tmp) {
  const float s = wave_sum(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = s;
  __syncthreads();
  const float t = ((tmp[0] + tmp[1]) + tmp[2]) + tmp[3];
  __syncthreads();
  return t;
}

template <int E>
__global__ void __launch_bounds__(kThreads) lora_generic_kernel(const LoraArgs a) {
  __shared__ float z1[kLoraMaxRankGeneric];
  __shared__ float tmp[4];
  using T = uint16_t;
  const T* y = static_cast<const T*>(a.y);
  T* out = static_cast<T*>(a.out);
  const T* x = static_cast<const T*>(a.x);
  const int tid = threadIdx.x;
  for (int64_t b = blockIdx.x; b < a.rows; b += gridDim.x) {
    const int32_t g = a.indices[b];
    const bool valid = g >= 0 && g < a.w;
    const T* yr = y + b * a.h3;
    T* orow = out + b * a.h3;
    if (!a.in_place)
      for (int64_t c = tid; c < a.h3; c += kThreads)
        if (!valid || c < a.y_offset || c >= a.y_offset + a.h2) orow[c] = yr[c];
    if (!valid) continue;  // uniform per workgroup
    const T* xr = x + b * a.h1;
    if (a.wa) {
      const T* wa = static_cast<const T*>(a.wa) + ((g * a.l + a.layer) * a.h1) * a.rank;
      for (int64_t r0 = 0; r0 < a.rank; r0 += 16) {
        float p[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) p[q] = 0.0f;
        for (int64_t k = tid; k < a.h1; k += kThreads) {
          const float xv = widen1<E>(xr[k]);
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (r0 + q < a.rank) p[q] = __builtin_fmaf(xv, widen1<E>(wa[k * a.rank + r0 + q]), p[q]);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float s = block_sum(p[q], tmp);
          if (tid == 0 && r0 + q < a.rank) z1[r0 + q] = s;
        }
      }
    } else {
      for (int64_t r = tid; r < a.rank; r += kThreads) z1[r] = widen1<E>(xr[r]);
    }
    __syncthreads();
    const T* wb = static_cast<const T*>(a.wb) + ((g * a.l + a.layer) * a.rank) * a.h2;
    for (int64_t j = tid; j < a.h2; j += kThreads) {
      float z = 0.0f;
      for (int64_t r = 0; r < a.rank; ++r) z = __builtin_fmaf(z1[r], widen1<E>(wb[r * a.h2 + j]), z);
      const int64_t at = a.y_offset + j;
      orow[at] = narrow1<E>(__builtin_fmaf(z, a.scale, widen1<E>(yr[at])));
    }
    __syncthreads();  // z1 is rewritten by the next row
  }
}

template <int E, int R>
hipError_t launch_tiled(const LoraArgs& a, const Workspace& ws, hipStream_t s) {
  const int64_t tiles = lora_max_tiles(a);
  if (a.wa && a.rows <= kSmallRows) {
    // small batch: the shrink groups the rows itself (one launch fewer)
    hipLaunchKernelGGL((lora_shrink_kernel<E, R, true>), dim3((unsigned)(tiles * a.ksplit)),
                       dim3(kThreads), 0, s, a, ws);
  } else {
    if (a.rows > kGroupRowsPerWg) {
      const unsigned wgs = (unsigned)((a.rows + kGroupRowsPerWg - 1) / kGroupRowsPerWg);
      hipLaunchKernelGGL(lora_count_kernel, dim3(wgs), dim3(kGroupThreads), 0, s, a, ws);
      hipLaunchKernelGGL(lora_place_kernel, dim3(wgs), dim3(kGroupThreads), 0, s, a, ws);
    } else {
      hipLaunchKernelGGL(lora_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, a, ws);
    }
    if (a.wa)
      hipLaunchKernelGGL((lora_shrink_kernel<E, R, false>), dim3((unsigned)(tiles * a.ksplit)),
                         dim3(kThreads), 0, s, a, ws);
  }
  if constexpr (E == kBF16 && R >= kMxMinRank) {
    hipLaunchKernelGGL((lora_expand_mx_kernel<R, kMxWaves>),
                       dim3((unsigned)((tiles + 7) / 8 * 8 * lora_mx_col_blocks(a.h2))),
                       dim3(64 * kMxWaves), 0, s, a, ws);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((tiles + 7) / 8 * 8 * kQuarters * a.chunks);
  if constexpr (R <= 32) {
    const int nt = expand_threads(a.h2, R);
    if (nt == 64) {
      hipLaunchKernelGGL((lora_expand_kernel<E, R, 64>), dim3(grid), dim3(64), 0, s, a, ws);
      return hipGetLastError();
    }
    if (nt == 128) {
      hipLaunchKernelGGL((lora_expand_kernel<E, R, 128>), dim3(grid), dim3(128), 0, s, a, ws);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((lora_expand_kernel<E, R, kThreads>), dim3(grid), dim3(kThreads), 0, s, a,
                     ws);
  return hipGetLastError();
}

template <int E>
hipError_t launch_elem(const LoraArgs& a, int path, void* workspace, hipStream_t s) {
  if (path == kLoraTiled) {
    const Workspace ws = ws_layout(workspace, a);
    switch (a.rank) {
      case 8: return launch_tiled<E, 8>(a, ws, s);
      case 16: return launch_tiled<E, 16>(a, ws, s);
      case 32: return launch_tiled<E, 32>(a, ws, s);
      case 64: return launch_tiled<E, 64>(a, ws, s);
      case 128: return launch_tiled<E, 128>(a, ws, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int64_t grid = a.rows < 65536 ? a.rows : 65536;
  hipLaunchKernelGGL(lora_generic_kernel<E>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t lora_max_tiles(const LoraArgs& a) { return lora_max_tiles_dev(a); }

int lora_shrink_blocks_per_cu(const LoraArgs& a) {
  const void* fn = nullptr;
  const bool f16 = a.elem == kF16, g = a.wa && a.rows <= kSmallRows;
#define ADQ_SHRINK_FN(R_)                                                                    \
  fn = f16 ? (g ? (const void*)lora_shrink_kernel<kF16, R_, true>                          \
                : (const void*)lora_shrink_kernel<kF16, R_, false>)                         \
           : (g ? (const void*)lora_shrink_kernel<kBF16, R_, true>                         \
                : (const void*)lora_shrink_kernel<kBF16, R_, false>)
  switch (a.rank) {
    case 8: ADQ_SHRINK_FN(8); break;
    case 16: ADQ_SHRINK_FN(16); break;
    case 32: ADQ_SHRINK_FN(32); break;
    case 64: ADQ_SHRINK_FN(64); break;
    case 128: ADQ_SHRINK_FN(128); break;
    default: return 0;
  }
#undef ADQ_SHRINK_FN
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kThreads, 0) != hipSuccess)
    return 0;
  return blocks;
}

const char* lora_tiled_kernels(const LoraArgs& a) {
  const bool mx = a.elem == kBF16 && a.rank >= kMxMinRank;
  if (a.wa && a.rows <= kSmallRows) return mx ? "shrink+mfma-expand" : "shrink+expand";
  if (a.rows > kGroupRowsPerWg) {
    if (a.wa) return mx ? "count+place+shrink+mfma-expand" : "count+place+shrink+expand";
    return mx ? "count+place+mfma-expand" : "count+place+expand";
  }
  if (a.wa) return mx ? "group+shrink+mfma-expand" : "group+shrink+expand";
  return mx ? "group+mfma-expand" : "group+expand";
}

int lora_expand_chunks(int64_t h2, int64_t rank) {
  const int64_t cols = 4 * expand_threads(h2, rank);
  const int64_t c = (h2 + cols - 1) / cols;
  return (int)(c < 1 ? 1 : c);
}

uint64_t lora_workspace_bytes(const LoraArgs& a) { return ws_offsets(a).end; }

hipError_t launch_lora(const LoraArgs& a, int path, void* workspace, hipStream_t stream) {
  return a.elem == kBF16 ? launch_elem<kBF16>(a, path, workspace, stream)
                         : launch_elem<kF16>(a, path, workspace, stream);
}

}  // namespace adq
