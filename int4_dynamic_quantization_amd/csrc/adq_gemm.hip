// INT8 x INT8 GEMM with per-row and per-column scales in the epilogue: the
// consumer of the operator's quantized output.  "aclnnAddRmsNormDynamicQuantV2"
// (Formula) defines y1Out = round(input1 / scale1Out), so input1 is
// represented by y1Out * scale1Out row by row; a linear layer with weights
// quantized per output column (w = w_q * w_scale) then computes
//
//   out[m, n] = (sum_k y1Out[m, k] * w_q[n, k]) * scale1Out[m] * w_scale[n]  (+ bias[n])
//
// with the integer sum exact in int32 (|k| <= 2^17 keeps it in range).
//
// gfx950 design: a workgroup of 2 x 2 wavefronts computes a (64*TM) x (64*TN)
// tile; each wavefront owns (32*TM) x (32*TN) outputs as TM x TN blocks of
// v_mfma_i32_32x32x32_i8.  K advances in steps of BK bytes through a double
// buffer in LDS: the next step's A and W tiles are loaded from global memory
// into registers while the current step's MFMAs run, then written to the other
// buffer; one barrier per step.  LDS rows are padded by 16 bytes so the
// 16-byte fragment reads of a wavefront hit distinct banks.  Operand
// fragments (32x32x32 int8): A[i][k] in lane i + 32 * (k / 16), byte k % 16;
// B[k][j] likewise with j; accumulator element e of lane l is
// C[(e / 4) * 8 + (l / 32) * 4 + e % 4][l % 32].
//
// Both operands are K-contiguous (activations [M, K] row-major, weights
// [N, K] row-major), so every fragment is one 16-byte read.  Tiles are dealt
// so that each XCD works on a contiguous, row-grouped range of output tiles,
// which keeps the A rows and W rows it reuses in its own L2.
#include <type_traits>

#include "adq_device.h"

namespace adq {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcdCount = 8;
constexpr int kGroupRows = 8;  // tile rows per L2 group

template <int TM, int TN, int BK>
struct GemmShape {
  static constexpr int BM = 64 * TM;
  static constexpr int BN = 64 * TN;
  static constexpr int STRIDE = BK + 16;  // LDS bytes per tile row
  static constexpr int A_CHUNKS = BM * BK / 16;  // 16-byte chunks per stage
  static constexpr int B_CHUNKS = BN * BK / 16;
  static constexpr int A_PER_THREAD = A_CHUNKS / 256;
  static constexpr int B_PER_THREAD = B_CHUNKS / 256;
  static constexpr int LDS_BYTES = 2 * (BM + BN) * STRIDE;
  static_assert(A_CHUNKS % 256 == 0 && B_CHUNKS % 256 == 0, "tile loads must split evenly");
};

template <int OUT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (OUT == kGemmOutF32) {
    static_cast<float*>(out)[idx] = v;
  } else if constexpr (OUT == kGemmOutBF16) {
    static_cast<uint16_t*>(out)[idx] = narrow1<kBF16>(v);
  } else {
    static_cast<uint16_t*>(out)[idx] = narrow1<kF16>(v);
  }
}

template <int TM, int TN, int BK, int OUT>
__global__ void __launch_bounds__(256) w8a8_kernel(const GemmArgs g) {
  using S = GemmShape<TM, TN, BK>;
  __shared__ __attribute__((aligned(16))) int8_t lds[S::LDS_BYTES];
  // buffer b: A tile at lds + b * stage, W tile right after it
  constexpr int kStage = (S::BM + S::BN) * S::STRIDE;
  auto sA = [&](int b) { return lds + b * kStage; };
  auto sB = [&](int b) { return lds + b * kStage + S::BM * S::STRIDE; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- output tile of this workgroup (XCD-contiguous, row-grouped order)
  const int64_t tiles_m = (g.m + S::BM - 1) / S::BM;
  const int64_t tiles_n = (g.n + S::BN - 1) / S::BN;
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t b = blockIdx.x;
  const int64_t per_xcd = (tiles + kXcdCount - 1) / kXcdCount;
  const int64_t t = (b % kXcdCount) * per_xcd + b / kXcdCount;
  if (t >= tiles) return;
  const int64_t group = t / (kGroupRows * tiles_n);
  const int64_t first_m = group * kGroupRows;
  const int64_t rows_in_group = tiles_m - first_m < kGroupRows ? tiles_m - first_m : kGroupRows;
  const int64_t in_group = t - group * kGroupRows * tiles_n;
  const int64_t tm = first_m + in_group % rows_in_group;
  const int64_t tn = in_group / rows_in_group;
  const int64_t m0 = tm * S::BM, n0 = tn * S::BN;

  // ---- global tile loads: buffer descriptors over this tile's rows; rows
  // past M (N) read 0; k past K is sent out of range to read 0.
  const int64_t a_rows = g.m - m0 < S::BM ? g.m - m0 : S::BM;
  const int64_t w_rows = g.n - n0 < S::BN ? g.n - n0 : S::BN;
  const rsrc_t ra = make_rsrc(g.a + m0 * g.k, (uint32_t)(a_rows * g.k));
  const rsrc_t rw = make_rsrc(g.w + n0 * g.k, (uint32_t)(w_rows * g.k));
  constexpr uint32_t kOut = 0x80000000u;  // beyond any tile descriptor
  constexpr int CPR = BK / 16;             // 16-byte chunks per tile row

  u32x4 pa[S::A_PER_THREAD], pw[S::B_PER_THREAD];
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < S::A_PER_THREAD; ++i) {
      const int c = tid + i * 256, r = c / CPR, kc = c % CPR;
      const int64_t k = k0 + kc * 16;
      const uint32_t off = k < g.k ? (uint32_t)(r * g.k + k) : kOut;
      pa[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < S::B_PER_THREAD; ++i) {
      const int c = tid + i * 256, r = c / CPR, kc = c % CPR;
      const int64_t k = k0 + kc * 16;
      const uint32_t off = k < g.k ? (uint32_t)(r * g.k + k) : kOut;
      pw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < S::A_PER_THREAD; ++i) {
      const int c = tid + i * 256, r = c / CPR, kc = c % CPR;
      *reinterpret_cast<u32x4*>(sA(buf) + r * S::STRIDE + kc * 16) = pa[i];
    }
#pragma unroll
    for (int i = 0; i < S::B_PER_THREAD; ++i) {
      const int c = tid + i * 256, r = c / CPR, kc = c % CPR;
      *reinterpret_cast<u32x4*>(sB(buf) + r * S::STRIDE + kc * 16) = pw[i];
    }
  };

  i32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = i32x16{};

  const int frag_row = lane & 31;       // row (A) or column (B) within a 32-block
  const int frag_k = (lane >> 5) * 16;  // byte offset of this lane's 16 k values
  const int64_t ksteps = (g.k + BK - 1) / BK;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int64_t s = 0; s < ksteps; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < ksteps) load_stage((s + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      i32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const i32x4*>(
            sA(buf) + (wm * 32 * TM + i * 32 + frag_row) * S::STRIDE + kk + frag_k);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const i32x4*>(
            sB(buf) + (wn * 32 * TN + j * 32 + frag_row) * S::STRIDE + kk + frag_k);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < ksteps) {
      store_stage(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: out = float(acc) * a_scale[row] * w_scale[col] (+ bias[col])
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + wn * 32 * TN + j * 32 + (lane & 31);
    const bool col_ok = col < g.n;
    const float sw = col_ok ? g.w_scale[col] : 0.0f;
    const float bias = (col_ok && g.bias) ? g.bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 32 * TM + i * 32 + (e / 4) * 8 + (lane >> 5) * 4 + (e & 3);
        if (col_ok && row < g.m) {
          const float v = (float)acc[i][j][e] * g.a_scale[row] * sw + bias;
          store_out<OUT>(g.out, row * g.n + col, v);
        }
      }
    }
  }
}

template <int TM, int TN, int BK, int OUT>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  using S = GemmShape<TM, TN, BK>;
  const int64_t tiles = ((g.m + S::BM - 1) / S::BM) * ((g.n + S::BN - 1) / S::BN);
  const int64_t per_xcd = (tiles + kXcdCount - 1) / kXcdCount;
  const int64_t grid = per_xcd * kXcdCount;
  hipLaunchKernelGGL((w8a8_kernel<TM, TN, BK, OUT>), dim3((unsigned)grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int TM, int TN, int BK>
hipError_t launch_out(const GemmArgs& g, hipStream_t s) {
  switch (g.out_type) {
    case kGemmOutF32: return launch_cfg<TM, TN, BK, kGemmOutF32>(g, s);
    case kGemmOutBF16: return launch_cfg<TM, TN, BK, kGemmOutBF16>(g, s);
    case kGemmOutF16: return launch_cfg<TM, TN, BK, kGemmOutF16>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_w8a8(const GemmArgs& g, int tile, hipStream_t stream) {
  switch (tile) {
    case kGemmTile128: return launch_out<2, 2, 128>(g, stream);
    case kGemmTile256: return launch_out<4, 4, 64>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace adq
