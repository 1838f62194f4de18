// Internal interface between the C-ABI host layer (adq_api.cpp) and the
// HIP kernels (adq_row_*.hip, adq_split.hip, adq_generic.hip, adq_gemm.hip,
// adq_lora.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adq.h"

namespace adq {

enum ElemType : int { kBF16 = 0, kF16 = 1 };
// What one quantized output slot produces: nothing, INT8 codes (one per
// byte, scale = max/127) or INT4 codes (two per byte, scale = max/7).
enum QuantKind : int { kQNone = 0, kQInt8 = 1, kQInt4 = 2 };

// Everything a launch needs; passed by value as the kernel argument.
// Pointers are device addresses.  x2 == nullptr selects the single-input
// RmsNormDynamicQuant form (no add, no x_out).  Output slot 1 is always
// produced; slot 2 only when q2 != kQNone.  An absent beta reads as 0, an
// absent smooth scale as 1.
struct Args {
  const void* x1;
  const void* x2;
  const void* gamma;
  const void* beta;
  const void* smooth1;
  const void* smooth2;
  void* x_out;
  void* y1;
  void* y2;
  float* scale1;
  float* scale2;
  int64_t rows;
  int32_t n;
  float eps;
  float inv_n;  // 1/n rounded to float
};

// Kernel families.
enum Path : int { kPathRow = 1, kPathSplit = 2, kPathGeneric = 3 };

// Compile-time variant of the row and split kernels.
struct Variant {
  int elem;  // ElemType
  int nin;   // 1 or 2 inputs
  int q1;    // QuantKind of output slot 1 (never kQNone)
  int q2;    // QuantKind of output slot 2
};

// Row kernel: one workgroup per row at a time, `vpt` 8-element vectors per
// thread (1, 2 or 4), grid-strided over rows, next row prefetched; `wt`
// selects sc1 stores instead of non-temporal ones.
hipError_t launch_row(const Variant& v, int vpt, bool wt, int block, int grid, const Args& a,
                      hipStream_t stream);
int row_max_blocks_per_cu(const Variant& v, int vpt, int block);

// Split-row path: S workgroups share each row (a chunk of block * vpt
// 8-column vectors each), one batch of `batch_rows` rows at a time.
// launches 2 or 3: plain kernels hand the partial results over through the
// workspace at kernel boundaries.  launches 1: one kernel whose workgroups
// exchange them through the workspace, tagged with `tag` + b * kSplitTagStep
// for batch b (the caller reserves one tag per batch, each unique to its
// launch), waiting at most `wait_ticks` (10 ns) for each exchange before
// computing a missing partial result themselves.  `spread` places a row's
// chunks on different XCDs (tests).  The workspace takes
// split_workspace_bytes(batch_rows, splits, launches) bytes, 8-byte
// aligned, any contents.
constexpr uint64_t kSplitTagStep = 0x9E3779B97F4A7C15ULL;
struct SplitPlan {
  int vpt;
  int block;
  int splits;
  int launches;
  int64_t batch_rows;
  int spread;
  uint32_t wait_ticks;
  uint64_t tag;
};
hipError_t launch_split(const Variant& v, const SplitPlan& sp, const Args& a, void* ws,
                        hipStream_t stream);
uint64_t split_workspace_bytes(int64_t batch_rows, int splits, int launches);
int64_t split_grid(int64_t batch_rows, int splits);  // workgroups per launch
int split_exchange_blocks_per_cu(const Variant& v, int vpt, int block);
// Device address of the library's static scratch buffer
// (ADQ_STATIC_SCRATCH_BYTES) on `device`, which must be the current device;
// looked up on the first call for each device.
hipError_t split_static_scratch(int device, void** ptr);

// Generic kernel: any n (odd widths, unaligned pointers); correctness path.
hipError_t launch_generic(const Variant& v, int block, int grid, const Args& a,
                          hipStream_t stream);

// INT8 x INT8 GEMM with per-row / per-column scales (consumer of the codes).
enum GemmOut : int { kGemmOutF32 = 0, kGemmOutBF16 = 1, kGemmOutF16 = 2 };
enum GemmTile : int { kGemmTile128 = 1, kGemmTile256 = 2, kGemmTileSkinny = 3 };

struct GemmArgs {
  const int8_t* a;        // [m, k] row-major (activation codes)
  const float* a_scale;   // [m]
  const int8_t* w;        // [n, k] row-major (weight codes)
  const float* w_scale;   // [n]
  const float* bias;      // [n] or nullptr
  void* out;              // [m, n] row-major, out_type
  int64_t m, n, k;
  int32_t out_type;       // GemmOut
};

// k % 16 == 0, 16-byte aligned a and w.
hipError_t launch_w8a8(const GemmArgs& g, int tile, hipStream_t stream);

// AddLora ("aclnnAddLora", Formulas): out = y with columns
// [y_offset, y_offset + h2) of row b increased by
// scale * (x[b] . A[g, layer]) . B[g, layer], g = indices[b]; rows whose index
// lies outside [0, w) are left as y.  A is [w, l, h1, rank] (may be NULL:
// then the shrink is skipped and rank == h1), B is [w, l, rank, h2].
struct LoraArgs {
  const void* y;
  const void* x;
  const void* wa;
  const void* wb;
  const int32_t* indices;
  void* out;
  int64_t rows;
  int64_t h1, rank, h2, h3;
  int64_t w, l, layer, y_offset;
  float scale;
  int elem;      // ElemType
  int in_place;  // out == y: only the slice of rows with an adapter is written
  int ksplit;    // tiled path: slices of h1 per tile in the shrink
  int chunks;    // tiled path: column ranges per tile in the expand
};

enum LoraPath : int { kLoraTiled = 1, kLoraGeneric = 2 };
constexpr int kLoraTileRows = 64;     // rows per tile in the tiled path
constexpr int kLoraMaxAdapters = 2048;
constexpr int kLoraMaxRankTiled = 128;
constexpr int kLoraMaxRankGeneric = 1024;

// Tiled path: upper bound on the number of tiles (sum over adapter classes of
// ceil(count / 64) <= rows / 64 + w + 1), and the workspace it needs (tile
// table, grouped row order, per-slice partial shrink results).
int64_t lora_max_tiles(const LoraArgs& a);
int lora_expand_chunks(int64_t h2, int64_t rank);  // column ranges per tile in the expand
const char* lora_tiled_kernels(const LoraArgs& a);  // the tiled path's launches
int lora_shrink_blocks_per_cu(const LoraArgs& a);   // resident shrink workgroups per CU
uint64_t lora_workspace_bytes(const LoraArgs& a);
hipError_t launch_lora(const LoraArgs& a, int path, void* workspace, hipStream_t stream);

}  // namespace adq
