// Split-row kernel: fused (Add)RmsNorm + dynamic quantization with S
// workgroups sharing each row, for shapes with few rows (decode steps) or
// rows longer than one workgroup holds.
//
// Operator: "aclnnAddRmsNormDynamicQuantV2", Formula section, and
// "aclnnRmsNormDynamicQuant", formula section.  Both the row sum of squares
// (inside Rms) and the row maximum (row_max) span the whole row, so the S
// workgroups of a row exchange partial results twice per row:
//   A  chunk loads, x = x1 + x2, xOut, partial sum of squares -> publish
//   -- wait for the S partial sums; add them in split order (every
//      workgroup gets the same bits, so results are deterministic)
//   B  y, quantizer inputs, partial row maxima -> publish
//   -- wait for the S partial maxima (max is exact in any order)
//   C  scales (split 0 stores them), codes, packed stores
//
// Exchange slots live in the caller's workspace and need no clearing: each
// launch carries a 64-bit epoch unique within the process, and a slot is
// two 64-bit words {epoch low half, value}, {epoch high half, value'}
// written with single-copy-atomic stores.  A reader accepts a slot only
// when both words carry this launch's halves, so a slot written by an
// earlier launch or holding unrelated data is never taken (a 64-bit match
// by chance is the only exception).  No memory fences are needed: each
// value travels in the same atomic word as its tag.
//
// All workgroups of the grid are resident at once (cooperative launch), so
// every wait ends; each wait is also bounded, and a workgroup that gives up
// records an error word in the workspace and continues.
//
// Workgroup -> (row, split) mapping keeps the S workgroups of a row on one
// XCD (workgroups are dealt to the 8 XCDs round robin), so their exchange
// stays within one L2 when the dispatcher follows that order; a wait that
// keeps failing invalidates its L2 now and then, so that a slot written
// from another XCD is still seen.
#include <type_traits>

#include "adq_device.h"

namespace adq {

namespace {

constexpr uint32_t kSpinLimit = 1u << 14;  // polls (about 2 us each) before a wait gives up
constexpr int kXcds = 8;

struct SplitArgs {
  Args a;
  uint64_t* ws;      // workspace base (header + slots)
  uint64_t epoch;    // unique per launch
  int32_t splits;    // S
  int32_t chunk;     // 8-column vectors per split (block * VPT)
  int32_t row_groups;  // grid = kXcds * row_groups * splits
};

// Workspace: 32-byte header (word 0: error flag = epoch of a launch whose
// wait timed out), then for each (row, split) two 16-byte slots (sum of
// squares; the two maxima).
__device__ __forceinline__ uint64_t* slot_ptr(const SplitArgs& p, int64_t row, int s, int phase) {
  return p.ws + 4 + ((row * p.splits + s) * 2 + phase) * 2;
}

__device__ __forceinline__ void publish(uint64_t* slot, uint64_t epoch, float v0, float v1) {
  const uint64_t w0 = ((uint64_t)__float_as_uint(v0) << 32) | (uint32_t)epoch;
  const uint64_t w1 = ((uint64_t)__float_as_uint(v1) << 32) | (uint32_t)(epoch >> 32);
  __hip_atomic_store(slot, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0, lane s < S: wait for split s's slot of this row and return its
// two values.  Returns false when the wait gave up.
__device__ __forceinline__ bool collect(const SplitArgs& p, int64_t row, int phase, int lane,
                                        float& v0, float& v1) {
  const bool mine = lane < p.splits;
  uint64_t* slot = slot_ptr(p, row, mine ? lane : 0, phase);
  const uint32_t lo = (uint32_t)p.epoch, hi = (uint32_t)(p.epoch >> 32);
  bool done = !mine;
  uint64_t w0 = 0, w1 = 0;
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (!done) {
      w0 = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w1 = __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      done = (uint32_t)w0 == lo && (uint32_t)w1 == hi;
    }
    if (__builtin_amdgcn_ballot_w64(!done) == 0) {
      v0 = __uint_as_float((uint32_t)(w0 >> 32));
      v1 = __uint_as_float((uint32_t)(w1 >> 32));
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
    // Each XCD has its own L2, and a slot polled before it was written can
    // stay cached there; the mapping keeps a row's workgroups on one XCD,
    // but only through the dispatcher's order.  After every 64 unsuccessful
    // polls (far beyond a normal wait) the wavefront invalidates its L2 so
    // that a slot written from another XCD is read afresh.
    if ((it & 63u) == 63u) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  v0 = v1 = 0.0f;
  return false;
}

template <int E, int NIN, int Q1, int Q2, int VPT>
__global__ void __launch_bounds__(1024) split_kernel(const SplitArgs p) {
  static_assert(VPT == 1 || VPT == 2, "split kernel holds at most 16 columns per thread");
  constexpr bool kTwo = Q2 != kQNone;
  constexpr int kQ2 = kTwo ? Q2 : kQInt8;
  const Args& a = p.a;
  const int tid = threadIdx.x;
  const int bs = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = bs >> 6;
  const int S = p.splits;

  // blockIdx -> (xcd, row group, split); rows xcd + 8*group, then + stride
  const int b = blockIdx.x;
  const int xcd = b % kXcds;
  const int q = b / kXcds;
  const int s = q % S;
  const int group = q / S;
  const int64_t row_stride = (int64_t)kXcds * p.row_groups;

  const uint32_t n = (uint32_t)a.n;
  const uint32_t nvec = n >> 3;
  const uint32_t v0 = (uint32_t)s * (uint32_t)p.chunk;  // first vector of this split
  const uint32_t vend = v0 + (uint32_t)p.chunk < nvec ? v0 + (uint32_t)p.chunk : nvec;
  const uint32_t chunk_bytes16 = (vend - v0) * 16u;  // bytes of 16-bit data in this split
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  const u32x4 one4 = u32x4{kOnePair<E>, kOnePair<E>, kOnePair<E>, kOnePair<E>};

  __shared__ float red_a[16], red_b[2][16];
  __shared__ float bcast[2];
  __shared__ int failed;
  if (tid == 0) failed = 0;

  uint32_t vj[VPT];  // vector index within this split's chunk
#pragma unroll
  for (int k = 0; k < VPT; ++k) vj[k] = (uint32_t)(tid + k * bs);

  auto param_rsrc = [&](const void* base) {
    return make_rsrc(static_cast<const char*>(base) + (size_t)v0 * 16u, chunk_bytes16);
  };
  u32x4 pg[VPT], pb[VPT], p1[VPT], p2[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    pg[k] = __builtin_amdgcn_raw_buffer_load_b128(param_rsrc(a.gamma), vj[k] * 16u, 0, 0);
    pb[k] = a.beta ? __builtin_amdgcn_raw_buffer_load_b128(param_rsrc(a.beta), vj[k] * 16u, 0, 0)
                   : zero4;
    // smooth absent: 1 inside the chunk, 0 past its end
    p1[k] = a.smooth1
                ? __builtin_amdgcn_raw_buffer_load_b128(param_rsrc(a.smooth1), vj[k] * 16u, 0, 0)
                : (v0 + vj[k] < vend ? one4 : zero4);
    p2[k] = !kTwo ? zero4
            : a.smooth2
                ? __builtin_amdgcn_raw_buffer_load_b128(param_rsrc(a.smooth2), vj[k] * 16u, 0, 0)
                : (v0 + vj[k] < vend ? one4 : zero4);
  }

  // the next row's chunk is requested before this row's exchanges, so its
  // loads are in flight while the workgroup waits for the other splits
  const uint32_t row_bytes = n * 2u;
  u32x4 n1[VPT], n2[VPT];
  auto load_row = [&](int64_t r) {
    const rsrc_t r1 = make_rsrc(
        static_cast<const char*>(row_ptr(a.x1, r, row_bytes)) + (size_t)v0 * 16u, chunk_bytes16);
    const rsrc_t r2 = make_rsrc(
        static_cast<const char*>(row_ptr(a.x2, r, row_bytes)) + (size_t)v0 * 16u, chunk_bytes16);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      n1[k] = __builtin_amdgcn_raw_buffer_load_b128(r1, vj[k] * 16u, 0, kStreamLoad);
      if constexpr (NIN == 2)
        n2[k] = __builtin_amdgcn_raw_buffer_load_b128(r2, vj[k] * 16u, 0, kStreamLoad);
    }
  };
  const int64_t row0 = (int64_t)group * kXcds + xcd;
  if (row0 < a.rows) load_row(row0);
  for (int64_t row = row0; row < a.rows; row += row_stride) {
    u32x4 c1[VPT], c2[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      c1[k] = n1[k];
      if constexpr (NIN == 2) c2[k] = n2[k];
    }
    if (row + row_stride < a.rows) load_row(row + row_stride);

    // ---- A
    float x[VPT][8];
    float ss = 0.0f;
    const rsrc_t rxo = make_rsrc(
        static_cast<char*>(row_ptr(a.x_out, row, row_bytes)) + (size_t)v0 * 16u, chunk_bytes16);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f32x2 v = widen2<E>(c1[k][w]);
        if constexpr (NIN == 2) v += widen2<E>(c2[k][w]);
        x[k][2 * w] = v.x;
        x[k][2 * w + 1] = v.y;
        acc = __builtin_fmaf(v.x, v.x, acc);
        acc = __builtin_fmaf(v.y, v.y, acc);
      }
      ss += acc;
      if constexpr (NIN == 2) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{narrow2<E>(x[k][0], x[k][1]), narrow2<E>(x[k][2], x[k][3]),
                  narrow2<E>(x[k][4], x[k][5]), narrow2<E>(x[k][6], x[k][7])},
            rxo, vj[k] * 16u, 0, kStreamStore);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red_a[wave] = ss;
    __syncthreads();
    if (wave == 0) {
      if (lane == 0) {
        float part = 0.0f;
        for (int w = 0; w < nwaves; ++w) part += red_a[w];
        publish(slot_ptr(p, row, s, 0), p.epoch, part, part);
      }
      float mine = 0.0f, dup = 0.0f;
      const bool ok = collect(p, row, 0, lane, mine, dup);
      float tot = 0.0f;  // in split order, the same bits in every workgroup of the row
      for (int t = 0; t < S; ++t) tot += lane_value(mine, t);
      if (lane == 0) {
        bcast[0] = tot;
        if (!ok) failed = 1;
      }
    }
    __syncthreads();
    const float rinv = __builtin_amdgcn_rsqf(__builtin_fmaf(bcast[0], a.inv_n, a.eps));

    // ---- B
    float in1[VPT][8], in2[VPT][8];
    float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 g = widen2<E>(pg[k][w]), bb = widen2<E>(pb[k][w]);
        const f32x2 s1 = widen2<E>(p1[k][w]);
        const float y0 = __builtin_fmaf(x[k][2 * w] * rinv, g.x, bb.x);
        const float y1 = __builtin_fmaf(x[k][2 * w + 1] * rinv, g.y, bb.y);
        in1[k][2 * w] = y0 * s1.x;
        in1[k][2 * w + 1] = y1 * s1.y;
        m1 = fmaxf(m1, fmaxf(fabsf(in1[k][2 * w]), fabsf(in1[k][2 * w + 1])));
        if constexpr (kTwo) {
          const f32x2 s2 = widen2<E>(p2[k][w]);
          in2[k][2 * w] = y0 * s2.x;
          in2[k][2 * w + 1] = y1 * s2.y;
          m2 = fmaxf(m2, fmaxf(fabsf(in2[k][2 * w]), fabsf(in2[k][2 * w + 1])));
        }
      }
    }
    m1 = wave_max(m1);
    if constexpr (kTwo) m2 = wave_max(m2);
    if (lane == 0) red_b[0][wave] = m1, red_b[1][wave] = m2;
    __syncthreads();
    if (wave == 0) {
      if (lane == 0) {
        float pm1 = 0.0f, pm2 = 0.0f;
        for (int w = 0; w < nwaves; ++w) pm1 = fmaxf(pm1, red_b[0][w]), pm2 = fmaxf(pm2, red_b[1][w]);
        publish(slot_ptr(p, row, s, 1), p.epoch, pm1, pm2);
      }
      float q1 = 0.0f, q2 = 0.0f;
      const bool ok = collect(p, row, 1, lane, q1, q2);
      q1 = wave_max(q1);  // lanes >= S hold 0; maxima are >= 0
      q2 = wave_max(q2);
      if (lane == 0) {
        bcast[0] = q1;
        bcast[1] = q2;
        if (!ok) failed = 1;
      }
    }
    __syncthreads();
    const float M1 = bcast[0], M2 = bcast[1];

    // ---- C
    const RowScale rs1 = row_scale<Q1>(M1);
    const RowScale rs2 = row_scale<kQ2>(M2);
    if (s == 0 && tid == 0) {
      a.scale1[row] = rs1.scale;
      if constexpr (kTwo) a.scale2[row] = rs2.scale;
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      apply_boost(in1[k], rs1);
      if constexpr (kTwo) apply_boost(in2[k], rs2);
    }
    auto codes = [&](const float (&in)[8], float inv, void* out, auto qtag) {
      constexpr int Q = decltype(qtag)::value;
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = code_bits(in[e], inv);
      return Q == kQInt8 ? pack_int8x8(c) : u32x2{pack_int4x8(c), 0u};
    };
    {
      const uint32_t ybytes = Q1 == kQInt4 ? n / 2u : n;
      const uint32_t vb = Q1 == kQInt4 ? 4u : 8u;  // bytes per vector
      const rsrc_t ry = make_rsrc(static_cast<char*>(row_ptr(a.y1, row, ybytes)) + (size_t)v0 * vb,
                                  (vend - v0) * vb);
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const u32x2 c = codes(in1[k], rs1.inv, a.y1, std::integral_constant<int, Q1>{});
        if constexpr (Q1 == kQInt8)
          __builtin_amdgcn_raw_buffer_store_b64(c, ry, vj[k] * 8u, 0, kStreamStore);
        else
          __builtin_amdgcn_raw_buffer_store_b32(c.x, ry, vj[k] * 4u, 0, kStreamStore);
      }
    }
    if constexpr (kTwo) {
      const uint32_t ybytes = kQ2 == kQInt4 ? n / 2u : n;
      const uint32_t vb = kQ2 == kQInt4 ? 4u : 8u;
      const rsrc_t ry = make_rsrc(static_cast<char*>(row_ptr(a.y2, row, ybytes)) + (size_t)v0 * vb,
                                  (vend - v0) * vb);
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const u32x2 c = codes(in2[k], rs2.inv, a.y2, std::integral_constant<int, kQ2>{});
        if constexpr (kQ2 == kQInt8)
          __builtin_amdgcn_raw_buffer_store_b64(c, ry, vj[k] * 8u, 0, kStreamStore);
        else
          __builtin_amdgcn_raw_buffer_store_b32(c.x, ry, vj[k] * 4u, 0, kStreamStore);
      }
    }
  }
  __syncthreads();
  if (tid == 0 && failed)
    __hip_atomic_store(p.ws, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int E, int NIN, int Q1, int Q2, int VPT>
struct SplitInst {
  static hipError_t launch(int block, int grid, const SplitArgs& p, hipStream_t s) {
    void* args[] = {const_cast<SplitArgs*>(&p)};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&split_kernel<E, NIN, Q1, Q2, VPT>),
                                      dim3(grid), dim3(block), args, 0, s);
  }
  static int occupancy(int block) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, split_kernel<E, NIN, Q1, Q2, VPT>, block,
                                                     0) != hipSuccess)
      return 0;
    return n;
  }
};

template <int E, typename F>
bool dispatch(int nin, int q1, int q2, int vpt, F&& f) {
#define ADQ_SPLIT_VPT(NIN_, Q1_, Q2_)                                              \
  switch (vpt) {                                                                   \
    case 1: f.template operator()<SplitInst<E, NIN_, Q1_, Q2_, 1>>(); return true; \
    case 2: f.template operator()<SplitInst<E, NIN_, Q1_, Q2_, 2>>(); return true; \
    default: return false;                                                         \
  }
  if (nin == 1) {
    if (q2 != kQNone) return false;
    if (q1 == kQInt8) { ADQ_SPLIT_VPT(1, kQInt8, kQNone) }
    if (q1 == kQInt4) { ADQ_SPLIT_VPT(1, kQInt4, kQNone) }
    return false;
  }
  if (nin != 2) return false;
  if (q1 == kQInt8 && q2 == kQNone) { ADQ_SPLIT_VPT(2, kQInt8, kQNone) }
  if (q1 == kQInt4 && q2 == kQNone) { ADQ_SPLIT_VPT(2, kQInt4, kQNone) }
  if (q1 == kQInt8 && q2 == kQInt8) { ADQ_SPLIT_VPT(2, kQInt8, kQInt8) }
  if (q1 == kQInt8 && q2 == kQInt4) { ADQ_SPLIT_VPT(2, kQInt8, kQInt4) }
  if (q1 == kQInt4 && q2 == kQInt8) { ADQ_SPLIT_VPT(2, kQInt4, kQInt8) }
  if (q1 == kQInt4 && q2 == kQInt4) { ADQ_SPLIT_VPT(2, kQInt4, kQInt4) }
#undef ADQ_SPLIT_VPT
  return false;
}

template <typename F>
bool dispatch_any(const Variant& v, int vpt, F&& f) {
  return v.elem == kBF16 ? dispatch<kBF16>(v.nin, v.q1, v.q2, vpt, f)
                         : dispatch<kF16>(v.nin, v.q1, v.q2, vpt, f);
}

}  // namespace

uint64_t split_workspace_bytes(int64_t rows, int splits) {
  return 32u + (uint64_t)rows * (uint64_t)splits * 32u;
}

int split_max_blocks_per_cu(const Variant& v, int vpt, int block) {
  int occ = 0;
  dispatch_any(v, vpt, [&]<typename I>() { occ = I::occupancy(block); });
  return occ;
}

hipError_t launch_split(const Variant& v, int vpt, int block, int splits, int row_groups,
                        const Args& a, void* ws, uint64_t epoch, hipStream_t stream) {
  if (splits < 1 || splits > 64 || row_groups < 1 || block < 64 || block > 1024 || block % 64)
    return hipErrorInvalidValue;
  SplitArgs p;
  p.a = a;
  p.ws = static_cast<uint64_t*>(ws);
  p.epoch = epoch;
  p.splits = splits;
  p.chunk = block * vpt;
  p.row_groups = row_groups;
  const int grid = kXcds * row_groups * splits;
  hipError_t err = hipErrorInvalidValue;
  dispatch_any(v, vpt, [&]<typename I>() { err = I::launch(block, grid, p, stream); });
  return err;
}

}  // namespace adq
