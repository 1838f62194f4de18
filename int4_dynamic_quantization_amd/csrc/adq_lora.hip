// AddLora ("aclnnAddLora", Formulas): rows of x are grouped by their adapter
// index; each group's rows are multiplied by weightA[g, layerIdx] (shrink,
// h1 -> rank) and then by weightB[g, layerIdx] (expand, rank -> h2) and
// scale, and the result is added into columns [y_offset, y_offset + h2) of
// y.  Rows whose index lies outside [0, w) get no contribution.  Arithmetic
// is fp32 (products of 16-bit inputs are exact; Z1 stays fp32 between the two
// products); the slice is rounded once to the storage type.
//
// Tiled kernel (the fast path): one workgroup per tile of up to 16 rows of
// one adapter, so the rows of a tile share their weights, as the page's
// step 1 regroups them.  Every workgroup derives the grouping itself from
// the index vector (histogram, prefix over the adapters' tile counts, then a
// stable ordered gather of its own rows), so a call is a single launch with
// no workspace and a deterministic result.
//  - shrink on MFMA (v_mfma_f32_16x16x32_{bf16,f16}): 16 rows x 16 ranks per
//    block, K = h1 split over the 4 wavefronts and summed in wavefront order
//    through LDS.  weightA is stored [h1, rank] (rank contiguous) while the
//    MFMA's B operand wants 8 consecutive k per lane, so each 32 x 16 block
//    goes through the wavefront's own 1 KB of LDS (one 16-byte write per
//    lane, eight 16-bit reads).
//  - expand on the vector ALU in fp32: each thread owns 4 adjacent columns
//    of the slice for all 16 rows (accumulators in registers), reads
//    weightB rows in 8-byte pieces and writes y's slice in 8-byte pieces;
//    Z1 is read from LDS by broadcast.
// Generic kernel: one workgroup per row, any sizes and alignments, same
// arithmetic with block reductions in a fixed order.
#include "adq_device.h"

namespace adq {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = kLoraTileRows;

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

// Exclusive prefix of one int per thread over the 256-thread workgroup, in
// thread order; `total` receives the sum.  tmp: 4 ints of LDS.
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
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return base + x - v;
}

__device__ __forceinline__ int adapter_class(int32_t g, int64_t w) {
  return (g >= 0 && g < w) ? g : (int)w;
}

template <int E>
__global__ void __launch_bounds__(kThreads) lora_tiled_kernel(const LoraArgs a) {
  __shared__ int cnt[kLoraMaxAdapters + 1];
  __shared__ int tstart[kLoraMaxAdapters + 1];
  __shared__ int scan_tmp[4];
  __shared__ int tile_info[2];
  __shared__ int64_t rows_lds[kTile];
  __shared__ __attribute__((aligned(16))) uint16_t wt[4][kLoraMaxRankTiled / 16][32 * 16];
  __shared__ __attribute__((aligned(16))) float part[4][kTile][kLoraMaxRankTiled];
  __shared__ __attribute__((aligned(16))) float z1[kTile][kLoraMaxRankTiled];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t W = a.w;
  const int64_t B = a.rows;

  // ---- grouping: adapter histogram, tiles per adapter and their prefix
  for (int g = tid; g <= W; g += kThreads) cnt[g] = 0;
  __syncthreads();
  const int64_t chunk = (B + kThreads - 1) / kThreads;
  const int64_t lo = tid * chunk;
  const int64_t hi = lo + chunk < B ? lo + chunk : B;
  for (int64_t i = lo; i < hi; ++i) atomicAdd(&cnt[adapter_class(a.indices[i], W)], 1);
  __syncthreads();
  auto tiles_of = [&](int g) -> int {
    if (g == W && a.in_place) return 0;  // rows without an adapter: nothing to write
    return (cnt[g] + kTile - 1) / kTile;
  };
  const int per = (int)((W + 1 + kThreads - 1) / kThreads);
  int local = 0;
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g <= W) local += tiles_of(g);
  }
  int total = 0;
  int run = block_exclusive_scan(local, scan_tmp, &total);
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g <= W) {
      tstart[g] = run;
      run += tiles_of(g);
    }
  }
  const int tile = (int)blockIdx.x;
  if (tile >= total) return;  // uniform: every thread saw the same total
  __syncthreads();
  for (int q = 0; q < per; ++q) {
    const int g = tid * per + q;
    if (g <= W && tile >= tstart[g] && tile < tstart[g] + tiles_of(g)) {
      tile_info[0] = g;
      tile_info[1] = tile - tstart[g];
    }
  }
  __syncthreads();
  const int g = tile_info[0];
  const int first = tile_info[1] * kTile;
  const int nrows = cnt[g] - first < kTile ? cnt[g] - first : kTile;

  // ---- this tile's rows: ranks [first, first + nrows) of adapter class g, in row order
  int c = 0;
  for (int64_t i = lo; i < hi; ++i) c += adapter_class(a.indices[i], W) == g;
  int dummy;
  int r = block_exclusive_scan(c, scan_tmp, &dummy);
  for (int64_t i = lo; i < hi && r < first + kTile; ++i) {
    if (adapter_class(a.indices[i], W) == g) {
      if (r >= first) rows_lds[r - first] = i;
      ++r;
    }
  }
  __syncthreads();

  using T = uint16_t;
  const T* y = static_cast<const T*>(a.y);
  T* out = static_cast<T*>(a.out);
  const int64_t h3 = a.h3;

  if (g == W) {  // no adapter (only reached when out != y): copy the rows
    for (int i = 0; i < nrows; ++i) {
      const int64_t row = rows_lds[i];
      for (int64_t c4 = tid; c4 < h3 / 4; c4 += kThreads)
        *reinterpret_cast<uint2*>(out + row * h3 + 4 * c4) =
            *reinterpret_cast<const uint2*>(y + row * h3 + 4 * c4);
    }
    return;
  }

  const int64_t rank = a.rank;
  const int nb = (int)(rank / 16);
  const T* x = static_cast<const T*>(a.x);

  // ---- shrink: z1[i][r] = sum_k x[row_i][k] * A[g, layer][k][r]
  if (a.wa) {
    const T* wa = static_cast<const T*>(a.wa) + ((g * a.l + a.layer) * a.h1) * rank;
    f32x4 acc[kLoraMaxRankTiled / 16];
#pragma unroll
    for (int b = 0; b < kLoraMaxRankTiled / 16; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int fi = lane & 15;   // A-operand row (tile row) / B-operand column (rank)
    const int fk = lane >> 4;   // which 8 of the 32 k
    const bool row_ok = fi < nrows;
    const T* xrow = x + (row_ok ? rows_lds[fi] : rows_lds[0]) * a.h1;
    const int64_t ksteps = (a.h1 + 31) / 32;
    for (int64_t s = wave; s < ksteps; s += 4) {
      const int64_t k0 = 32 * s;
      u16x8 xa = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      const int64_t kx = k0 + 8 * fk;
      if (row_ok && kx < a.h1) xa = *reinterpret_cast<const u16x8*>(xrow + kx);
      const int64_t kw = k0 + (lane >> 1);  // this lane's weight row
#pragma unroll
      for (int b = 0; b < kLoraMaxRankTiled / 16; ++b) {
        if (b < nb) {
          u16x8 wv = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
          if (kw < a.h1)
            wv = *reinterpret_cast<const u16x8*>(wa + kw * rank + 16 * b + 8 * (lane & 1));
          *reinterpret_cast<u16x8*>(&wt[wave][b][16 * (lane >> 1) + 8 * (lane & 1)]) = wv;
          u16x8 bv;
#pragma unroll
          for (int e = 0; e < 8; ++e) bv[e] = wt[wave][b][16 * (8 * fk + e) + fi];
          acc[b] = mfma16<E>(xa, bv, acc[b]);
        }
      }
    }
    // partial sums of this wavefront: element e of lane l is row 4 * (l / 16) + e, rank l % 16
#pragma unroll
    for (int b = 0; b < kLoraMaxRankTiled / 16; ++b)
      if (b < nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][4 * fk + e][16 * b + fi] = acc[b][e];
    __syncthreads();
    for (int t = tid; t < kTile * rank; t += kThreads) {
      const int i = (int)(t / rank), rr = (int)(t % rank);
      z1[i][rr] = ((part[0][i][rr] + part[1][i][rr]) + part[2][i][rr]) + part[3][i][rr];
    }
  } else {
    for (int t = tid; t < kTile * rank; t += kThreads) {
      const int i = (int)(t / rank), rr = (int)(t % rank);
      z1[i][rr] = i < nrows ? widen1<E>(x[rows_lds[i] * a.h1 + rr]) : 0.0f;
    }
  }
  __syncthreads();

  // ---- expand + accumulate: columns 4 * cg .. 4 * cg + 3 of the slice
  const T* wb = static_cast<const T*>(a.wb) + ((g * a.l + a.layer) * rank) * a.h2;
  const int64_t ncg = a.h2 / 4;
  for (int64_t cg = tid; cg < ncg; cg += kThreads) {
    float acc[kTile][4];
#pragma unroll
    for (int i = 0; i < kTile; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;
    for (int rc = 0; rc < rank; rc += 16) {
      float bw[16][4];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const u16x4 v = *reinterpret_cast<const u16x4*>(wb + (rc + rr) * a.h2 + 4 * cg);
#pragma unroll
        for (int q = 0; q < 4; ++q) bw[rr][q] = widen1<E>(v[q]);
      }
#pragma unroll
      for (int i = 0; i < kTile; ++i) {
        const f32x4* zr = reinterpret_cast<const f32x4*>(&z1[i][rc]);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 z = zr[r4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][q] = __builtin_fmaf(z[u], bw[4 * r4 + u][q], acc[i][q]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
      if (i < nrows) {
        const int64_t at = rows_lds[i] * h3 + a.y_offset + 4 * cg;
        const u16x4 yv = *reinterpret_cast<const u16x4*>(y + at);
        u16x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = narrow1<E>(__builtin_fmaf(acc[i][q], a.scale, widen1<E>(yv[q])));
        *reinterpret_cast<u16x4*>(out + at) = o;
      }
    }
  }

  // ---- out != y: the columns outside the slice are copied
  if (!a.in_place) {
    const int64_t s0 = a.y_offset / 4, s1 = (a.y_offset + a.h2) / 4;
    for (int i = 0; i < nrows; ++i) {
      const int64_t row = rows_lds[i];
      for (int64_t c4 = tid; c4 < h3 / 4; c4 += kThreads)
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

template <int E>
hipError_t launch_elem(const LoraArgs& a, int path, hipStream_t s) {
  if (path == kLoraTiled) {
    hipLaunchKernelGGL(lora_tiled_kernel<E>, dim3((unsigned)lora_tiled_grid(a)), dim3(kThreads),
                       0, s, a);
  } else {
    const int64_t grid = a.rows < 65536 ? a.rows : 65536;
    hipLaunchKernelGGL(lora_generic_kernel<E>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

int64_t lora_tiled_grid(const LoraArgs& a) {
  return (a.rows + kTile - 1) / kTile + a.w + 1;
}

hipError_t launch_lora(const LoraArgs& a, int path, hipStream_t stream) {
  return a.elem == kBF16 ? launch_elem<kBF16>(a, path, stream)
                         : launch_elem<kF16>(a, path, stream);
}

}  // namespace adq
