// Row kernel: fused (Add)RmsNorm + one or two per-row dynamic quantizations.
//
// Operator: "aclnnAddRmsNormDynamicQuantV2", Formula section (x = x1 + x2;
// y = x / Rms(x) * gamma + beta; input_k = y * smoothScale_k;
// scale_k = row_max(|input_k|) / 127 or / 7; y_k = round(input_k / scale_k))
// and "aclnnRmsNormDynamicQuant", formula section (single input).
//
// Layout: every tensor is dense row-major.  A workgroup of `block` threads
// owns a whole row at a time: thread t holds the 8-element column vectors
// t, t + block, ..., t + (VPT-1) * block, so each wavefront load or store
// instruction covers one contiguous 1 KiB (16-bit data) span.  Workgroups
// stride over rows (grid <= rows); the next row's x1/x2 are loaded into
// registers while the current row is computed, so each element of x1 and
// x2 is read from HBM exactly once and every output is written once.
//
// Per row:
//   A  load + add in fp32, store xOut (round to nearest even), sum of squares
//   -- workgroup sum (DPP + readlane per wave, LDS across waves, fixed order)
//   B  rinv = 1 / sqrt(ss / n + eps); y = fma(x * rinv, gamma, beta);
//      input_k = y * smooth_k; row max of |input_k|
//   -- workgroup max
//   C  scale_k = max_k / Q_k; code = round_half_even(input_k * (1/scale_k));
//      pack (INT8: 1 byte, INT4: 1 nibble, even column low) and store.
//
// VPT (8-column vectors per thread) is 1, 2, 4 or 8, so a row of up to 65536
// columns fits one workgroup of at most 1024 threads.  With VPT 1 or 2 the
// parameters (gamma, beta, smooth) stay in registers as packed 16-bit values
// for the whole row loop and are converted at use, and x and the quantizer
// inputs are kept between the passes.  With VPT 4 that would not fit the
// registers of 1024 threads: the parameters are read at use (from L2, they
// are shared by all rows) and x and the quantizer inputs are recomputed in
// each pass from the row's raw 16-bit data, with the same operations, so
// every pass sees the same values.  VPT 8 keeps the raw data of vectors 0-3
// in registers and of vectors 4-7 in LDS (direct-to-LDS loads; 128 KiB for
// two inputs at 1024 threads), and reads gamma and beta at use too.
#pragma once

#include <type_traits>

#include "adq_device.h"

namespace adq {

// Keeps the compiler from hoisting per-use conversions of a loop-invariant
// register out of the row loop (which would hold fp32 copies and spill).
__device__ __forceinline__ void opaque(u32x4& v) { asm volatile("" : "+v"(v)); }

// Codes of one 8-column vector into an INT8 (8 bytes) or INT4X2 (4 bytes)
// output row, at vector index j of that row.  `in` is already boosted.
template <int Q, int ST>
__device__ __forceinline__ void store_codes(const float (&in)[8], float inv, rsrc_t out,
                                            uint32_t j) {
  uint32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = code_bits(in[e], inv);
  if constexpr (Q == kQInt8) {
    __builtin_amdgcn_raw_buffer_store_b64(pack_int8x8(q), out, j * 8u, 0, ST);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(pack_int4x8(q), out, j * 4u, 0, ST);
  }
}

// WT: the stores' cache policy, non-temporal (false) or sc1 (true; chosen for
// launches that move little data).
template <int E, int NIN, int Q1, int Q2, int VPT, bool WT>
__global__ void __launch_bounds__(1024) row_kernel(const Args a) {
  static_assert(VPT == 1 || VPT == 2 || VPT == 4 || VPT == 8,
                "row kernel holds at most 64 columns per thread");
  constexpr bool kHold = VPT <= 2;  // x and the inputs kept between passes, next row prefetched
  constexpr int RV = VPT == 8 ? 4 : VPT;  // vectors whose raw data stay in registers
  constexpr bool kHoldGB = VPT <= 4;      // gamma and beta held in registers
  constexpr bool kTwo = Q2 != kQNone;
  constexpr int kQ2 = kTwo ? Q2 : kQInt8;
  constexpr int kStBulk = WT ? kWriteThroughStore : kStreamStore;
  const int tid = threadIdx.x;
  const int bs = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = bs >> 6;
  const uint32_t n = (uint32_t)a.n;
  const uint32_t row_bytes = n * 2u;  // 16-bit elements
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  const u32x4 one4 = u32x4{kOnePair<E>, kOnePair<E>, kOnePair<E>, kOnePair<E>};

  __shared__ float red_ss[16];
  __shared__ float red_mx[2][16];
  // VPT 8: raw data of vectors 4-7, input i of vector k at
  // xl[((k - 4) * NIN + i) * 1024 + thread]
  __shared__ __attribute__((aligned(16))) u32x4 xl[VPT == 8 ? (VPT - RV) * NIN * 1024 : 1];

  // This thread's 8-column vectors: j = tid + k * bs.  Vectors past the end
  // of the row read as 0 and their stores are dropped by the buffer range
  // check (the row is a whole number of 16-byte vectors).
  auto vj = [&](int k) -> uint32_t { return (uint32_t)(tid + k * bs); };

  // Parameters, kept as 16-bit pairs (1 for an absent smooth scale).
  auto load_param = [&](const void* p, int k, u32x4 absent) -> u32x4 {
    if (!p) return absent;
    return __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(p, row_bytes), vj(k) * 16u, 0, 0);
  };
  constexpr int PH = kHold ? VPT : 1;  // x / input vectors kept between passes
  // VPT 4 holds gamma and beta, and smooth1 when there is one output; the
  // smooth scales it does not hold are read at use (from L2)
  constexpr bool kHoldS1 = kHoldGB && (kHold || !kTwo);
  u32x4 pg[kHoldGB ? VPT : 1], pb[kHoldGB ? VPT : 1], p1[kHoldS1 ? VPT : 1], p2[PH];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if constexpr (kHoldGB) {
      pg[k] = load_param(a.gamma, k, zero4);
      pb[k] = load_param(a.beta, k, zero4);
    }
    if constexpr (kHoldS1) p1[k] = load_param(a.smooth1, k, one4);
    if constexpr (kHold) p2[k] = kTwo ? load_param(a.smooth2, k, one4) : zero4;
  }

  using lds_ptr = __attribute__((address_space(3))) void*;
  auto load_row = [&](int64_t row, u32x4 (&c1)[RV], u32x4 (&c2)[RV]) {
    const rsrc_t r1 = make_rsrc(row_ptr(a.x1, row, row_bytes), row_bytes);
    const rsrc_t r2 = make_rsrc(row_ptr(a.x2, row, row_bytes), row_bytes);
#pragma unroll
    for (int k = 0; k < RV; ++k) {
      c1[k] = __builtin_amdgcn_raw_buffer_load_b128(r1, vj(k) * 16u, 0, kStreamLoad);
      if constexpr (NIN == 2)
        c2[k] = __builtin_amdgcn_raw_buffer_load_b128(r2, vj(k) * 16u, 0, kStreamLoad);
    }
    // VPT 8: vectors 4-7 straight to LDS, each wave's 64 lanes as 1 KiB at
    // its own threads' slots (issued after the register loads, so waiting
    // for those does not wait for these)
    uint8_t* xl_wave = reinterpret_cast<uint8_t*>(xl) + 16 * (tid & ~63);
#pragma unroll
    for (int k = RV; k < VPT; ++k) {
      const uint32_t off = vj(k) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_ptr)(xl_wave + 16 * 1024 * ((k - RV) * NIN)),
                                               16, off, 0, 0, kStreamLoad);
      if constexpr (NIN == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r2, (lds_ptr)(xl_wave + 16 * 1024 * ((k - RV) * NIN + 1)), 16, off, 0, 0, kStreamLoad);
    }
  };

  // Rows of this workgroup: blockIdx.x, + gridDim.x, ... (strided rows
  // measured 3-9% faster than one contiguous block of rows per workgroup).
  const int64_t first = blockIdx.x;
  const int64_t rend = a.rows;
  const int64_t step = gridDim.x;
  auto clamp_row = [&](int64_t r) { return r < rend ? r : rend - 1; };

  int64_t row = first;
  if (row >= rend) return;
  u32x4 c1[RV], c2[RV];  // raw x1/x2 vectors of the row being computed (in registers)
  if constexpr (kHold) load_row(row, c1, c2);

  // One row: prefetch the next, compute and store this one, with the stores'
  // cache policy kSt.  The first row is peeled off the loop so that every
  // entry to the loop header has the same outstanding memory operations
  // (loads, then stores); the wait for the prefetched row then need not wait
  // for stores.  The last row is peeled too: its prefetch (of a row that is
  // not this workgroup's) is dead there and dropped, and its stores use sc1
  // so that the end of the kernel leaves less written data behind in the
  // caches (65536 x 5120 INT4 390.9 -> 377.8 us, 4096 x 4096 23.1 -> 21.8 us,
  // 16384 x 8192 190.7 -> 189.1 us).
  auto body = [&]<int kSt>(int64_t row) {
    // Prefetch this workgroup's next row (its last row again when there is
    // none, so the loads are unconditional).
    // (VPT 4: the registers hold no second row, so this row is loaded here)
    u32x4 n1[PH], n2[PH];
    if constexpr (kHold) load_row(clamp_row(row + step), n1, n2);
    else load_row(row, c1, c2);
    if constexpr (kHoldGB) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) opaque(pg[k]), opaque(pb[k]);
    }
    if constexpr (kHoldS1) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) opaque(p1[k]);
    }
    if constexpr (kHold) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) opaque(p2[k]);
    }
    // x of a column vector from its raw data
    auto xvec = [&](const u32x4& v1, const u32x4& v2, float (&xk)[8]) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f32x2 v = widen2<E>(v1[w]);
        if constexpr (NIN == 2) v += widen2<E>(v2[w]);
        xk[2 * w] = v.x;
        xk[2 * w + 1] = v.y;
      }
    };
    // f(k, raw x1, raw x2) for every column vector: the register-held ones
    // unrolled, those held in LDS (VPT 8) in a loop, one at a time, so that
    // their loads and parameters are not all in flight at once
    auto for_vectors = [&](auto&& f) {
#pragma unroll
      for (int k = 0; k < RV; ++k) f(k, c1[k], c2[k]);
#pragma unroll 1
      for (int k = RV; k < VPT; ++k) {
        const u32x4 v1 = xl[((k - RV) * NIN) * 1024 + tid];
        const u32x4 v2 = NIN == 2 ? xl[((k - RV) * NIN + 1) * 1024 + tid] : zero4;
        f(k, v1, v2);
      }
    };

    // ---- A: x = x1 + x2 (fp32), xOut, sum of squares
    float x[PH][8];
    float ss = 0.0f;
    const rsrc_t rxo = make_rsrc(row_ptr(a.x_out, row, row_bytes), row_bytes);
    for_vectors([&](int k, const u32x4& v1, const u32x4& v2) {
      float xk[8];
      xvec(v1, v2, xk);
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (kHold) x[k][e] = xk[e];
        acc = __builtin_fmaf(xk[e], xk[e], acc);
      }
      ss += acc;
      if constexpr (NIN == 2) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{narrow2<E>(xk[0], xk[1]), narrow2<E>(xk[2], xk[3]),
                  narrow2<E>(xk[4], xk[5]), narrow2<E>(xk[6], xk[7])},
            rxo, vj(k) * 16u, 0, kSt);
      }
    });
    ss = wave_sum(ss);
    if (lane == 0) red_ss[wave] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int w = 0; w < nwaves; ++w) tot += red_ss[w];
    const float rinv = __builtin_amdgcn_rsqf(__builtin_fmaf(tot, a.inv_n, a.eps));

    // ---- B: y = x * rinv * gamma + beta, quantizer inputs, row maxima
    // inputs of column vector k (x held or recomputed)
    auto inputs = [&](int k, const u32x4& v1, const u32x4& v2, float (&i1)[8], float (&i2)[8]) {
      float xk[8];
      if constexpr (kHold) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xk[e] = x[k][e];
      } else {
        xvec(v1, v2, xk);
      }
      u32x4 pgk, pbk, p1k, p2k = zero4;
      if constexpr (kHoldGB) pgk = pg[k], pbk = pb[k];
      else pgk = load_param(a.gamma, k, zero4), pbk = load_param(a.beta, k, zero4);
      if constexpr (kHoldS1) p1k = p1[k];
      else p1k = load_param(a.smooth1, k, one4);
      if constexpr (kTwo) {
        if constexpr (kHold) p2k = p2[k];
        else p2k = load_param(a.smooth2, k, one4);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 g = widen2<E>(pgk[w]), b = widen2<E>(pbk[w]);
        const f32x2 s1 = widen2<E>(p1k[w]);
        const float y0 = __builtin_fmaf(xk[2 * w] * rinv, g.x, b.x);
        const float y1 = __builtin_fmaf(xk[2 * w + 1] * rinv, g.y, b.y);
        i1[2 * w] = y0 * s1.x;
        i1[2 * w + 1] = y1 * s1.y;
        if constexpr (kTwo) {
          const f32x2 s2 = widen2<E>(p2k[w]);
          i2[2 * w] = y0 * s2.x;
          i2[2 * w + 1] = y1 * s2.y;
        }
      }
    };
    float in1[PH][8], in2[PH][8];
    float m1 = 0.0f, m2 = 0.0f;
    for_vectors([&](int k, const u32x4& v1, const u32x4& v2) {
      float i1[8], i2[8];
      inputs(k, v1, v2, i1, i2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        m1 = fmaxf(m1, fabsf(i1[e]));
        if constexpr (kTwo) m2 = fmaxf(m2, fabsf(i2[e]));
        if constexpr (kHold) {
          in1[k][e] = i1[e];
          if constexpr (kTwo) in2[k][e] = i2[e];
        }
      }
    });
    m1 = wave_max(m1);
    if constexpr (kTwo) m2 = wave_max(m2);
    if (lane == 0) {
      red_mx[0][wave] = m1;
      if constexpr (kTwo) red_mx[1][wave] = m2;
    }
    __syncthreads();
    float M1 = 0.0f, M2 = 0.0f;
    for (int w = 0; w < nwaves; ++w) {
      M1 = fmaxf(M1, red_mx[0][w]);
      if constexpr (kTwo) M2 = fmaxf(M2, red_mx[1][w]);
    }

    // ---- C: scales, codes, packed stores
    const RowScale r1 = row_scale<Q1>(M1);
    const RowScale r2 = row_scale<kQ2>(M2);
    if (tid == 0) {
      a.scale1[row] = r1.scale;
      if constexpr (kTwo) a.scale2[row] = r2.scale;
    }
    const uint32_t y1_bytes = Q1 == kQInt4 ? n / 2u : n;
    const rsrc_t ry1 = make_rsrc(row_ptr(a.y1, row, y1_bytes), y1_bytes);
    const uint32_t y2_bytes = kQ2 == kQInt4 ? n / 2u : n;
    const rsrc_t ry2 = make_rsrc(row_ptr(a.y2, row, kTwo ? y2_bytes : 0u), kTwo ? y2_bytes : 0u);
    if constexpr (kHold) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        apply_boost(in1[k], r1);
        if constexpr (kTwo) apply_boost(in2[k], r2);
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) store_codes<Q1, kSt>(in1[k], r1.inv, ry1, vj(k));
      if constexpr (kTwo) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) store_codes<kQ2, kSt>(in2[k], r2.inv, ry2, vj(k));
      }
    } else {
      for_vectors([&](int k, const u32x4& v1, const u32x4& v2) {
        float i1[8], i2[8];
        inputs(k, v1, v2, i1, i2);
        apply_boost(i1, r1);
        store_codes<Q1, kSt>(i1, r1.inv, ry1, vj(k));
        if constexpr (kTwo) {
          apply_boost(i2, r2);
          store_codes<kQ2, kSt>(i2, r2.inv, ry2, vj(k));
        }
      });
    }

    if constexpr (kHold) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) c1[k] = n1[k], c2[k] = n2[k];
    }
  };
  const int64_t last = first + (rend - 1 - first) / step * step;
  if (row < last) {
    body.template operator()<kStBulk>(row);
    for (row += step; row < last; row += step) body.template operator()<kStBulk>(row);
  }
  body.template operator()<kWriteThroughStore>(last);
}

// ---- launch table for one element type

template <int E, int NIN, int Q1, int Q2, int VPT, bool WT>
struct RowInst {
  static hipError_t launch(int block, int grid, const Args& a, hipStream_t s) {
    hipLaunchKernelGGL((row_kernel<E, NIN, Q1, Q2, VPT, WT>), dim3(grid), dim3(block), 0, s, a);
    return hipGetLastError();
  }
  static int occupancy(int block) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, row_kernel<E, NIN, Q1, Q2, VPT, WT>,
                                                     block, 0) != hipSuccess)
      return 0;
    return n;
  }
};

// Calls f.template operator()<Inst>() for the instance matching (nin, q1,
// q2, vpt, wt); returns false when no such instance exists.
template <int E, template <int, int, int, int, int, bool> class Inst, typename F>
bool dispatch_variant(int nin, int q1, int q2, int vpt, bool wt, F&& f) {
#define ADQ_VPT_CASES(NIN_, Q1_, Q2_)                                                     \
  switch (vpt * 2 + (wt ? 1 : 0)) {                                                       \
    case 2: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 1, false>>(); return true;      \
    case 3: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 1, true>>(); return true;       \
    case 4: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 2, false>>(); return true;      \
    case 5: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 2, true>>(); return true;       \
    case 8: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 4, false>>(); return true;      \
    case 9: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 4, true>>(); return true;       \
    case 16: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 8, false>>(); return true;     \
    case 17: f.template operator()<Inst<E, NIN_, Q1_, Q2_, 8, true>>(); return true;      \
    default: return false;                                                                \
  }
  if (nin == 1) {
    if (q2 != kQNone) return false;
    if (q1 == kQInt8) { ADQ_VPT_CASES(1, kQInt8, kQNone) }
    if (q1 == kQInt4) { ADQ_VPT_CASES(1, kQInt4, kQNone) }
    return false;
  }
  if (nin != 2) return false;
  if (q1 == kQInt8 && q2 == kQNone) { ADQ_VPT_CASES(2, kQInt8, kQNone) }
  if (q1 == kQInt4 && q2 == kQNone) { ADQ_VPT_CASES(2, kQInt4, kQNone) }
  if (q1 == kQInt8 && q2 == kQInt8) { ADQ_VPT_CASES(2, kQInt8, kQInt8) }
  if (q1 == kQInt8 && q2 == kQInt4) { ADQ_VPT_CASES(2, kQInt8, kQInt4) }
  if (q1 == kQInt4 && q2 == kQInt8) { ADQ_VPT_CASES(2, kQInt4, kQInt8) }
  if (q1 == kQInt4 && q2 == kQInt4) { ADQ_VPT_CASES(2, kQInt4, kQInt4) }
#undef ADQ_VPT_CASES
  return false;
}

// Entry points for one element type, used by launch_row() in adq_api.cpp.
#define ADQ_DEFINE_ROW_ENTRY(E, SUFFIX)                                                     \
  hipError_t launch_row_##SUFFIX(const Variant& v, int vpt, bool wt, int block, int grid,  \
                                 const Args& a, hipStream_t s) {                           \
    hipError_t err = hipErrorInvalidValue;                                                 \
    dispatch_variant<E, RowInst>(v.nin, v.q1, v.q2, vpt, wt, [&]<typename I>() {           \
      err = I::launch(block, grid, a, s);                                                  \
    });                                                                                    \
    return err;                                                                            \
  }                                                                                        \
  int row_occupancy_##SUFFIX(const Variant& v, int vpt, int block) {                       \
    int occ = 0;                                                                           \
    dispatch_variant<E, RowInst>(v.nin, v.q1, v.q2, vpt, false,                            \
                                 [&]<typename I>() { occ = I::occupancy(block); });        \
    return occ;                                                                            \
  }

}  // namespace adq
