// Split-row path: fused (Add)RmsNorm + dynamic quantization with S
// workgroups sharing each row, for shapes whose rows are too few to occupy
// the chip one row per workgroup (decode steps) or too long for one
// workgroup to hold.
//
// Operator: "aclnnAddRmsNormDynamicQuantV2", Formula section, and
// "aclnnRmsNormDynamicQuant", formula section.  The sum of squares inside
// Rms and the row maximum (row_max) both span the whole row, so a row cut
// into S chunks needs two whole-row results before its codes exist.  They
// are handed over at kernel boundaries, never inside a launch:
//
//   K1 sumsq  workgroup (row, s): chunk s of x1, x2 -> x = x1 + x2 (fp32),
//             xOut, partial sum of squares -> ss[row][s]
//   K2 max    workgroup (row, s): total = ss[row][0] + ... + ss[row][S-1]
//             in split order (the same bits in every workgroup of the
//             row); rinv; chunk s again; quantizer inputs; partial row
//             maxima -> mx[row][s][k]
//   K3 quant  workgroup (row, s): rinv as in K2; M_k = max over
//             mx[row][.][k] (a maximum is exact in any order); scales
//             (split 0 stores them); chunk s again; codes -> y_k
//
// Two-launch form: K2 is left out and each K3 workgroup takes the row
// maxima itself over the whole row.  That costs S reads of each row from
// the cache instead of one launch.
//
// One-launch form (few rows, all S x rows workgroups of a batch on the chip
// at once): the same three steps in one kernel; each workgroup publishes its
// chunk's partial result in the workspace as two 64-bit words, each holding
// a 32-bit half of a tag unique to the launch beside the value, and reads
// the other chunks' words.  A word is taken only when it carries this
// launch's tag half (both words of a slot must), so a slot from an earlier
// launch is never taken.  Every wait is bounded: a chunk whose slot has not
// appeared within the wait budget is computed by the waiting workgroup
// itself, from the inputs, by the same code that computes its own chunk, so
// the value is the same bits either way.  Results therefore never depend on
// when (or whether) another workgroup's store becomes visible, on which XCD
// or in which order workgroups run, or on all of them being resident: only
// on each 64-bit word being read and written whole (naturally aligned 64-bit
// atomic accesses).  The tag comes from the host at each call, so this form
// is not used under graph capture (a replay would repeat the tag): a
// captured call runs the plain-launch form instead, with the same results.
//
// Every chunk is re-read from the caches (K1 loads with the default cache
// policy so the lines stay in L2 and the memory-side cache), and every
// quantizer input is recomputed from the same loaded values with the same
// fp32 operations in each kernel, so K3 quantizes exactly the values whose
// maximum K2 took.  The kernels never read a location that another
// workgroup of the same launch writes: there are no waits, no flags and no
// atomics, and the workspace needs no clearing (each kernel reads only what
// an earlier launch of the same call wrote).  Kernel boundaries on one
// stream order the launches; large inputs run as batches of rows (each
// batch's three launches before the next batch's), so the re-read chunks
// of a batch still sit in the 256 MB memory-side cache.
#include <mutex>
#include <type_traits>

#include "adq_device.h"

// Scratch memory of the entry point that allocates nothing
// (adq_add_rms_norm_dynamic_quant_v2_no_alloc): a static device array that
// every device the library runs on holds, at its own address, from module
// load until the process ends.  Host code never passes this name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[ADQ_STATIC_SCRATCH_BYTES];

namespace adq {

namespace {

constexpr int kXcds = 8;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

struct SplitArgs {
  Args a;
  float* ss;        // [rows, S] partial sums of squares
  float* mx;        // [rows, S, 2] partial row maxima (three-launch form)
  uint64_t* slots;  // [rows, S, 2 phases, 2 words] (one-launch form)
  uint64_t tag;     // one-launch form: unique to the launch
  uint32_t wait;    // one-launch form: wait budget per exchange, 10 ns ticks
  int32_t spread;   // place a row's chunks on different XCDs (tests)
  int64_t row0;     // first row of this batch
  int32_t rows;     // rows of this batch
  int32_t splits;   // S
  int32_t chunk;    // 8-column vectors per split (block * VPT)
};

// blockIdx -> (row of the batch, split).  Workgroups are dealt to the XCDs
// round robin (b % 8); the S workgroups of a row share b % 8, so in each
// launch of a batch (all with the same grid) a row's chunks are read on the
// same XCD, whose L2 then still holds them for the next launch.
struct Place {
  int32_t local;  // row within the batch
  int32_t s;      // split
  bool valid;
};

__device__ __forceinline__ Place place_of(const SplitArgs& p) {
  const int b = blockIdx.x;
  Place r;
  if (p.spread) {  // consecutive workgroups: a row's chunks on different XCDs
    r.s = b % p.splits;
    r.local = b / p.splits;
  } else {
    const int q = b / kXcds;
    r.s = q % p.splits;
    r.local = (q / p.splits) * kXcds + b % kXcds;
  }
  r.valid = r.local < p.rows;
  return r;
}

// Chunk s of a row: vectors [v0, vend) of the row's n / 8.
struct Chunk {
  uint32_t v0;
  uint32_t nv;  // vectors in the chunk (the last one may be short)
};

__device__ __forceinline__ Chunk chunk_of(const SplitArgs& p, int s) {
  const uint32_t nvec = (uint32_t)p.a.n >> 3;
  const uint32_t v0 = (uint32_t)s * (uint32_t)p.chunk;
  const uint32_t vend = v0 + (uint32_t)p.chunk < nvec ? v0 + (uint32_t)p.chunk : nvec;
  return Chunk{v0, vend - v0};
}

// Descriptor over the chunk's bytes of a row of 16-bit data (or of the
// parameter vectors when row_bytes == 0): vectors past the chunk read 0 and
// their stores are dropped.
__device__ __forceinline__ rsrc_t chunk_rsrc(const void* base, int64_t row, uint32_t row_bytes,
                                            Chunk c, uint32_t vbytes) {
  return make_rsrc(static_cast<const char*>(base) + row * (int64_t)row_bytes +
                       (size_t)c.v0 * vbytes,
                   c.nv * vbytes);
}

// Raw x1 / x2 vectors of this thread in a chunk (vector tid + k * block).
template <int NIN, int VPT>
__device__ __forceinline__ void load_x(const Args& a, int64_t row, Chunk c,
                                       const uint32_t (&vj)[VPT], u32x4 (&c1)[VPT],
                                       u32x4 (&c2)[VPT]) {
  const uint32_t row_bytes = (uint32_t)a.n * 2u;
  const rsrc_t r1 = chunk_rsrc(a.x1, row, row_bytes, c, 16u);
  const rsrc_t r2 = chunk_rsrc(NIN == 2 ? a.x2 : a.x1, row, row_bytes, c, 16u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    c1[k] = __builtin_amdgcn_raw_buffer_load_b128(r1, vj[k] * 16u, 0, 0);
    if constexpr (NIN == 2) c2[k] = __builtin_amdgcn_raw_buffer_load_b128(r2, vj[k] * 16u, 0, 0);
  }
}

// x = x1 + x2 (fp32) of one raw vector pair.
template <int E, int NIN>
__device__ __forceinline__ void xvec(const u32x4& r1, const u32x4& r2, float (&x)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f32x2 v = widen2<E>(r1[w]);
    if constexpr (NIN == 2) v += widen2<E>(r2[w]);
    x[2 * w] = v.x;
    x[2 * w + 1] = v.y;
  }
}

// Parameter vectors of a chunk (gamma, beta, smooth1, smooth2 as 16-bit
// pairs; an absent beta reads 0, an absent smooth scale 1).
template <int VPT>
struct Params {
  u32x4 g[VPT], b[VPT], s1[VPT], s2[VPT];
};

template <int E, bool TWO, int VPT>
__device__ __forceinline__ void load_params(const Args& a, Chunk c, const uint32_t (&vj)[VPT],
                                            Params<VPT>& pr) {
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  const u32x4 one4 = u32x4{kOnePair<E>, kOnePair<E>, kOnePair<E>, kOnePair<E>};
  auto ld = [&](const void* base, int k, u32x4 absent) -> u32x4 {
    if (!base) return absent;
    return __builtin_amdgcn_raw_buffer_load_b128(chunk_rsrc(base, 0, 0u, c, 16u), vj[k] * 16u,
                                                 0, 0);
  };
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    pr.g[k] = ld(a.gamma, k, zero4);
    pr.b[k] = ld(a.beta, k, zero4);
    pr.s1[k] = ld(a.smooth1, k, one4);
    pr.s2[k] = TWO ? ld(a.smooth2, k, one4) : zero4;
  }
}

// Quantizer inputs of one vector: y = fma(x * rinv, gamma, beta),
// input_k = y * smooth_k.  The same operations as in the row kernel.
template <int E, bool TWO>
__device__ __forceinline__ void inputs_of(const float (&x)[8], float rinv, const u32x4& g,
                                          const u32x4& b, const u32x4& s1, const u32x4& s2,
                                          float (&i1)[8], float (&i2)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 gg = widen2<E>(g[w]), bb = widen2<E>(b[w]), t1 = widen2<E>(s1[w]);
    const float y0 = __builtin_fmaf(x[2 * w] * rinv, gg.x, bb.x);
    const float y1 = __builtin_fmaf(x[2 * w + 1] * rinv, gg.y, bb.y);
    i1[2 * w] = y0 * t1.x;
    i1[2 * w + 1] = y1 * t1.y;
    if constexpr (TWO) {
      const f32x2 t2 = widen2<E>(s2[w]);
      i2[2 * w] = y0 * t2.x;
      i2[2 * w + 1] = y1 * t2.y;
    }
  }
}

// Workgroup sum in a fixed order (DPP + readlane per wave, waves in order).
// The leading barrier lets `red` be reused by consecutive calls.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < nwaves; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < nwaves; ++w) t = fmaxf(t, red[w]);
  return t;
}

// Partial sum of squares of a chunk from its raw vectors: one fma chain per
// thread over its vectors in order, then the workgroup sum.  Every form of
// the path computes a chunk's partial here, so it is the same bits whichever
// workgroup or kernel computes it.
template <int E, int NIN, int VPT>
__device__ __forceinline__ float chunk_sumsq(const u32x4 (&c1)[VPT], const u32x4 (&c2)[VPT],
                                             float* red) {
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float x[8];
    xvec<E, NIN>(c1[k], c2[k], x);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(x[e], x[e], acc);
    ss += acc;
  }
  return block_sum(ss, red);
}

// Partial row maxima of a chunk (both outputs; m2 is 0 with one output).
template <int E, int NIN, bool TWO, int VPT>
__device__ __forceinline__ void chunk_max(const u32x4 (&c1)[VPT], const u32x4 (&c2)[VPT],
                                          const Params<VPT>& pr, float rinv, float* red1,
                                          float* red2, float& m1, float& m2) {
  m1 = 0.0f;
  m2 = 0.0f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float x[8], i1[8], i2[8];
    xvec<E, NIN>(c1[k], c2[k], x);
    inputs_of<E, TWO>(x, rinv, pr.g[k], pr.b[k], pr.s1[k], pr.s2[k], i1, i2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      m1 = fmaxf(m1, fabsf(i1[e]));
      if constexpr (TWO) m2 = fmaxf(m2, fabsf(i2[e]));
    }
  }
  m1 = block_max(m1, red1);
  if constexpr (TWO) m2 = block_max(m2, red2);
}

// 1 / Rms of a row from its S partial sums, added in split order (the same
// bits in every workgroup of the row and in every kernel).
__device__ __forceinline__ float row_rinv(const SplitArgs& p, int32_t local, float* bcast) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const int S = p.splits;
    float tot = 0.0f;
    for (int t0 = 0; t0 < S; t0 += 64) {
      const float v = t0 + lane < S ? p.ss[(int64_t)local * S + t0 + lane] : 0.0f;
      const int cnt = S - t0 < 64 ? S - t0 : 64;
      for (int t = 0; t < cnt; ++t) tot += lane_value(v, t);
    }
    if (lane == 0) *bcast = tot;
  }
  __syncthreads();
  return __builtin_amdgcn_rsqf(__builtin_fmaf(*bcast, p.a.inv_n, p.a.eps));
}

// ---- K1: xOut and partial sums of squares

template <int E, int NIN, int VPT>
__global__ void __launch_bounds__(1024) split_sumsq_kernel(const SplitArgs p) {
  const Place pl = place_of(p);
  if (!pl.valid) return;  // the whole workgroup
  __shared__ float red[16];
  const Args& a = p.a;
  const int64_t row = p.row0 + pl.local;
  const Chunk c = chunk_of(p, pl.s);
  uint32_t vj[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) vj[k] = threadIdx.x + k * blockDim.x;
  u32x4 c1[VPT], c2[VPT];
  load_x<NIN, VPT>(a, row, c, vj, c1, c2);
  if constexpr (NIN == 2) {
    const rsrc_t rxo = chunk_rsrc(a.x_out, row, (uint32_t)a.n * 2u, c, 16u);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float x[8];
      xvec<E, NIN>(c1[k], c2[k], x);
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{narrow2<E>(x[0], x[1]), narrow2<E>(x[2], x[3]), narrow2<E>(x[4], x[5]),
                narrow2<E>(x[6], x[7])},
          rxo, vj[k] * 16u, 0, kStreamStore);
    }
  }
  const float ss = chunk_sumsq<E, NIN, VPT>(c1, c2, red);
  if (threadIdx.x == 0) p.ss[(int64_t)pl.local * p.splits + pl.s] = ss;
}

// ---- K2: partial row maxima

template <int E, int NIN, bool TWO, int VPT>
__global__ void __launch_bounds__(1024) split_max_kernel(const SplitArgs p) {
  const Place pl = place_of(p);
  if (!pl.valid) return;
  __shared__ float red[2][16];
  __shared__ float bcast;
  const Args& a = p.a;
  const int64_t row = p.row0 + pl.local;
  const Chunk c = chunk_of(p, pl.s);
  uint32_t vj[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) vj[k] = threadIdx.x + k * blockDim.x;
  u32x4 c1[VPT], c2[VPT];
  load_x<NIN, VPT>(a, row, c, vj, c1, c2);
  Params<VPT> pr;
  load_params<E, TWO, VPT>(a, c, vj, pr);
  const float rinv = row_rinv(p, pl.local, &bcast);
  float m1, m2;
  chunk_max<E, NIN, TWO, VPT>(c1, c2, pr, rinv, red[0], red[1], m1, m2);
  if (threadIdx.x == 0) {
    float* slot = p.mx + ((int64_t)pl.local * p.splits + pl.s) * 2;
    slot[0] = m1;
    slot[1] = m2;
  }
}

// ---- K3: scales and codes

template <int Q>
__device__ __forceinline__ void store_chunk_codes(const float (&in)[8], float inv, rsrc_t out,
                                                  uint32_t j) {
  uint32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = code_bits(in[e], inv);
  if constexpr (Q == kQInt8)
    __builtin_amdgcn_raw_buffer_store_b64(pack_int8x8(q), out, j * 8u, 0, kStreamStore);
  else
    __builtin_amdgcn_raw_buffer_store_b32(pack_int4x8(q), out, j * 4u, 0, kStreamStore);
}

// Row maxima over the whole row, taken by one workgroup (two-launch form):
// each thread covers vectors tid, tid + block, ... of the row, two at a
// time with all their loads in flight.  Which thread takes which vector does
// not matter: each input is computed by the same operations wherever it is
// computed, and a maximum is exact in any order.
template <int E, int NIN, bool TWO>
__device__ __forceinline__ void whole_row_max(const Args& a, int64_t row, float rinv, float& m1,
                                              float& m2) {
  const uint32_t nvec = (uint32_t)a.n >> 3;
  const Chunk all{0u, nvec};
  const uint32_t bs = blockDim.x;
  for (uint32_t base = 0; base < nvec; base += 2 * bs) {
    const uint32_t vj[2] = {base + threadIdx.x, base + bs + threadIdx.x};
    u32x4 c1[2], c2[2];
    load_x<NIN, 2>(a, row, all, vj, c1, c2);
    Params<2> pr;
    load_params<E, TWO, 2>(a, all, vj, pr);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float x[8], i1[8], i2[8];
      xvec<E, NIN>(c1[k], c2[k], x);
      inputs_of<E, TWO>(x, rinv, pr.g[k], pr.b[k], pr.s1[k], pr.s2[k], i1, i2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        m1 = fmaxf(m1, fabsf(i1[e]));
        if constexpr (TWO) m2 = fmaxf(m2, fabsf(i2[e]));
      }
    }
  }
}

template <int E, int NIN, int Q1, int Q2, int VPT, bool WHOLE>
__global__ void __launch_bounds__(1024) split_quant_kernel(const SplitArgs p) {
  constexpr bool kTwo = Q2 != kQNone;
  constexpr int kQ2 = kTwo ? Q2 : kQInt8;
  const Place pl = place_of(p);
  if (!pl.valid) return;
  __shared__ float red[2][16];
  __shared__ float bcast;
  const Args& a = p.a;
  const int64_t row = p.row0 + pl.local;
  const Chunk c = chunk_of(p, pl.s);
  uint32_t vj[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) vj[k] = threadIdx.x + k * blockDim.x;
  u32x4 c1[VPT], c2[VPT];
  load_x<NIN, VPT>(a, row, c, vj, c1, c2);
  Params<VPT> pr;
  load_params<E, kTwo, VPT>(a, c, vj, pr);
  const float rinv = row_rinv(p, pl.local, &bcast);

  float M1 = 0.0f, M2 = 0.0f;
  if constexpr (WHOLE) {
    whole_row_max<E, NIN, kTwo>(a, row, rinv, M1, M2);
    M1 = block_max(M1, red[0]);
    if constexpr (kTwo) M2 = block_max(M2, red[1]);
  } else {
    // the S partial maxima of the row, read by wave 0 and reduced in it
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const float* mx = p.mx + (int64_t)pl.local * p.splits * 2;
      for (int t = lane; t < p.splits; t += 64) {
        M1 = fmaxf(M1, mx[2 * t]);
        if constexpr (kTwo) M2 = fmaxf(M2, mx[2 * t + 1]);
      }
      M1 = wave_max(M1);
      M2 = wave_max(M2);
      if (lane == 0) red[0][0] = M1, red[1][0] = M2;
    }
    __syncthreads();
    M1 = red[0][0];
    M2 = red[1][0];
  }

  const RowScale r1 = row_scale<Q1>(M1);
  const RowScale r2 = row_scale<kQ2>(M2);
  if (pl.s == 0 && threadIdx.x == 0) {
    a.scale1[row] = r1.scale;
    if constexpr (kTwo) a.scale2[row] = r2.scale;
  }
  const uint32_t n = (uint32_t)a.n;
  const rsrc_t ry1 = chunk_rsrc(a.y1, row, Q1 == kQInt4 ? n / 2u : n, c, Q1 == kQInt4 ? 4u : 8u);
  const rsrc_t ry2 = kTwo ? chunk_rsrc(a.y2, row, kQ2 == kQInt4 ? n / 2u : n, c,
                                       kQ2 == kQInt4 ? 4u : 8u)
                          : make_rsrc(a.y1, 0u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float x[8], i1[8], i2[8];
    xvec<E, NIN>(c1[k], c2[k], x);
    inputs_of<E, kTwo>(x, rinv, pr.g[k], pr.b[k], pr.s1[k], pr.s2[k], i1, i2);
    apply_boost(i1, r1);
    store_chunk_codes<Q1>(i1, r1.inv, ry1, vj[k]);
    if constexpr (kTwo) {
      apply_boost(i2, r2);
      store_chunk_codes<kQ2>(i2, r2.inv, ry2, vj[k]);
    }
  }
}

// ---- one-launch form: in-kernel exchange with bounded waits

// Slot of (row, split, phase): two 64-bit words {tag low half, value 1},
// {tag high half, value 2}.
__device__ __forceinline__ uint64_t* xslot(const SplitArgs& p, int32_t local, int s, int phase) {
  return p.slots + (((int64_t)local * p.splits + s) * 2 + phase) * 2;
}

__device__ __forceinline__ void publish(uint64_t* slot, uint64_t tag, float v1, float v2) {
  const uint64_t w0 = ((uint64_t)__float_as_uint(v1) << 32) | (uint32_t)tag;
  const uint64_t w1 = ((uint64_t)__float_as_uint(v2) << 32) | (uint32_t)(tag >> 32);
  __hip_atomic_store(slot, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 (lane t < S, t != own split) reads the slots of the row's other
// chunks until each carries this launch's tag or the wait budget is spent.
// Writes the values found to v1[t], v2[t] (LDS) and returns, in LDS, the
// mask of chunks not found.  The own chunk's values are set by the caller.
__device__ __forceinline__ void gather(const SplitArgs& p, int32_t local, int own, int phase,
                                       float* v1, float* v2, uint64_t* missing) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int S = p.splits;
  const bool mine = lane < S && lane != own;
  uint64_t* slot = xslot(p, local, mine ? lane : own, phase);
  const uint32_t lo = (uint32_t)p.tag, hi = (uint32_t)(p.tag >> 32);
  bool done = !mine;
  uint64_t w0 = 0, w1 = 0;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    if (!done) {
      w0 = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w1 = __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      done = (uint32_t)w0 == lo && (uint32_t)w1 == hi;
    }
    if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 >= p.wait) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (mine && done) {
    v1[lane] = __uint_as_float((uint32_t)(w0 >> 32));
    v2[lane] = __uint_as_float((uint32_t)(w1 >> 32));
  }
  const uint64_t miss = __builtin_amdgcn_ballot_w64(!done);
  if (lane == 0) *missing = miss;
}

// A value every thread of the workgroup holds alike (read from LDS after a
// barrier), made a scalar so that loops over it stay uniform.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

template <int E, int NIN, int Q1, int Q2, int VPT>
__global__ void __launch_bounds__(1024) split_exchange_kernel(const SplitArgs p) {
  constexpr bool kTwo = Q2 != kQNone;
  constexpr int kQ2 = kTwo ? Q2 : kQInt8;
  const Place pl = place_of(p);
  if (!pl.valid) return;
  __shared__ float red[2][16];
  __shared__ float part1[64], part2[64];
  __shared__ uint64_t missing;
  const Args& a = p.a;
  const int S = p.splits;
  const int64_t row = p.row0 + pl.local;
  const Chunk c = chunk_of(p, pl.s);
  uint32_t vj[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) vj[k] = threadIdx.x + k * blockDim.x;
  u32x4 c1[VPT], c2[VPT];
  load_x<NIN, VPT>(a, row, c, vj, c1, c2);
  Params<VPT> pr;
  load_params<E, kTwo, VPT>(a, c, vj, pr);

  // ---- A: xOut, partial sum of squares, exchange
  if constexpr (NIN == 2) {
    const rsrc_t rxo = chunk_rsrc(a.x_out, row, (uint32_t)a.n * 2u, c, 16u);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float x[8];
      xvec<E, NIN>(c1[k], c2[k], x);
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{narrow2<E>(x[0], x[1]), narrow2<E>(x[2], x[3]), narrow2<E>(x[4], x[5]),
                narrow2<E>(x[6], x[7])},
          rxo, vj[k] * 16u, 0, kStreamStore);
    }
  }
  const float ss = chunk_sumsq<E, NIN, VPT>(c1, c2, red[0]);
  if (threadIdx.x == 0) {
    publish(xslot(p, pl.local, pl.s, 0), p.tag, ss, ss);
    part1[pl.s] = ss;
  }
  gather(p, pl.local, pl.s, 0, part1, part2, &missing);
  __syncthreads();
  for (uint64_t m = uniform64(missing); m != 0; m &= m - 1) {
    const int t = __builtin_ctzll(m);
    const Chunk ct = chunk_of(p, t);
    u32x4 t1[VPT], t2[VPT];
    load_x<NIN, VPT>(a, row, ct, vj, t1, t2);
    const float v = chunk_sumsq<E, NIN, VPT>(t1, t2, red[0]);
    if (threadIdx.x == 0) part1[t] = v;
  }
  __syncthreads();
  float tot = 0.0f;  // in split order, as in every other form
  for (int t = 0; t < S; ++t) tot += part1[t];
  const float rinv = __builtin_amdgcn_rsqf(__builtin_fmaf(tot, a.inv_n, a.eps));

  // ---- B: partial row maxima, exchange
  float m1, m2;
  chunk_max<E, NIN, kTwo, VPT>(c1, c2, pr, rinv, red[0], red[1], m1, m2);
  __syncthreads();  // every thread has read part1 (the total) before it is reused
  if (threadIdx.x == 0) {
    publish(xslot(p, pl.local, pl.s, 1), p.tag, m1, m2);
    part1[pl.s] = m1;
    part2[pl.s] = m2;
  }
  gather(p, pl.local, pl.s, 1, part1, part2, &missing);
  __syncthreads();
  for (uint64_t m = uniform64(missing); m != 0; m &= m - 1) {
    const int t = __builtin_ctzll(m);
    const Chunk ct = chunk_of(p, t);
    u32x4 t1[VPT], t2[VPT];
    load_x<NIN, VPT>(a, row, ct, vj, t1, t2);
    Params<VPT> tp;
    load_params<E, kTwo, VPT>(a, ct, vj, tp);
    float u1, u2;
    chunk_max<E, NIN, kTwo, VPT>(t1, t2, tp, rinv, red[0], red[1], u1, u2);
    if (threadIdx.x == 0) part1[t] = u1, part2[t] = u2;
  }
  __syncthreads();
  float M1 = 0.0f, M2 = 0.0f;
  for (int t = 0; t < S; ++t) {
    M1 = fmaxf(M1, part1[t]);
    if constexpr (kTwo) M2 = fmaxf(M2, part2[t]);
  }

  // ---- C: scales and codes of this chunk
  const RowScale r1 = row_scale<Q1>(M1);
  const RowScale r2 = row_scale<kQ2>(M2);
  if (pl.s == 0 && threadIdx.x == 0) {
    a.scale1[row] = r1.scale;
    if constexpr (kTwo) a.scale2[row] = r2.scale;
  }
  const uint32_t n = (uint32_t)a.n;
  const rsrc_t ry1 = chunk_rsrc(a.y1, row, Q1 == kQInt4 ? n / 2u : n, c, Q1 == kQInt4 ? 4u : 8u);
  const rsrc_t ry2 = kTwo ? chunk_rsrc(a.y2, row, kQ2 == kQInt4 ? n / 2u : n, c,
                                       kQ2 == kQInt4 ? 4u : 8u)
                          : make_rsrc(a.y1, 0u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float x[8], i1[8], i2[8];
    xvec<E, NIN>(c1[k], c2[k], x);
    inputs_of<E, kTwo>(x, rinv, pr.g[k], pr.b[k], pr.s1[k], pr.s2[k], i1, i2);
    apply_boost(i1, r1);
    store_chunk_codes<Q1>(i1, r1.inv, ry1, vj[k]);
    if constexpr (kTwo) {
      apply_boost(i2, r2);
      store_chunk_codes<kQ2>(i2, r2.inv, ry2, vj[k]);
    }
  }
}

// ---- launch tables

template <int E, int NIN, int Q1, int Q2, int VPT>
struct SplitInst {
  static constexpr bool kTwo = Q2 != kQNone;
  static hipError_t launch(int block, int grid, int launches, const SplitArgs& p,
                           hipStream_t s) {
    if (launches == 1) {
      hipLaunchKernelGGL((split_exchange_kernel<E, NIN, Q1, Q2, VPT>), dim3(grid), dim3(block),
                         0, s, p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((split_sumsq_kernel<E, NIN, VPT>), dim3(grid), dim3(block), 0, s, p);
    if (launches == 3) {
      hipLaunchKernelGGL((split_max_kernel<E, NIN, kTwo, VPT>), dim3(grid), dim3(block), 0, s, p);
      hipLaunchKernelGGL((split_quant_kernel<E, NIN, Q1, Q2, VPT, false>), dim3(grid),
                         dim3(block), 0, s, p);
    } else {
      hipLaunchKernelGGL((split_quant_kernel<E, NIN, Q1, Q2, VPT, true>), dim3(grid),
                         dim3(block), 0, s, p);
    }
    return hipGetLastError();
  }
  static int exchange_occupancy(int block) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, split_exchange_kernel<E, NIN, Q1, Q2, VPT>, block, 0) != hipSuccess)
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

}  // namespace

uint64_t split_workspace_bytes(int64_t batch_rows, int splits, int launches) {
  const uint64_t slots = (uint64_t)batch_rows * (uint64_t)splits;
  if (launches == 1) return slots * 32u;  // two phases of two 64-bit words
  const uint64_t ss = (slots * 4u + 255u) / 256u * 256u;
  return ss + (launches == 3 ? slots * 8u : 0u);
}

int64_t split_grid(int64_t batch_rows, int splits) {
  return (batch_rows + kXcds - 1) / kXcds * kXcds * splits;
}

int split_exchange_blocks_per_cu(const Variant& v, int vpt, int block) {
  int occ = 0;
  auto q = [&]<typename I>() { occ = I::exchange_occupancy(block); };
  if (v.elem == kBF16) dispatch<kBF16>(v.nin, v.q1, v.q2, vpt, q);
  else dispatch<kF16>(v.nin, v.q1, v.q2, vpt, q);
  return occ;
}

hipError_t split_static_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

hipError_t launch_split(const Variant& v, const SplitPlan& sp, const Args& a, void* ws,
                        hipStream_t stream) {
  if (sp.splits < 1 || sp.batch_rows < 1 || sp.block < 64 || sp.block > 1024 || sp.block % 64 ||
      sp.launches < 1 || sp.launches > 3 || (sp.launches == 1 && sp.splits > 64) ||
      (sp.vpt != 1 && sp.vpt != 2) || (int64_t)sp.splits * sp.block * sp.vpt < a.n / 8 ||
      split_grid(sp.batch_rows, sp.splits) > INT32_MAX)
    return hipErrorInvalidValue;
  SplitArgs p;
  p.a = a;
  p.ss = static_cast<float*>(ws);
  p.mx = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                  split_workspace_bytes(sp.batch_rows, sp.splits, 2));
  p.slots = static_cast<uint64_t*>(ws);
  p.tag = sp.tag;
  p.wait = sp.wait_ticks;
  p.spread = sp.spread;
  p.splits = sp.splits;
  p.chunk = sp.block * sp.vpt;
  hipError_t err = hipSuccess;
  for (int64_t r0 = 0; r0 < a.rows && err == hipSuccess; r0 += sp.batch_rows) {
    const int64_t rows = a.rows - r0 < sp.batch_rows ? a.rows - r0 : sp.batch_rows;
    p.row0 = r0;
    p.rows = (int32_t)rows;
    p.tag = sp.tag + (uint64_t)(r0 / sp.batch_rows) * kSplitTagStep;
    const int grid = (int)split_grid(rows, sp.splits);
    bool found = false;
    auto go = [&]<typename I>() {
      found = true;
      err = I::launch(sp.block, grid, sp.launches, p, stream);
    };
    if (v.elem == kBF16) dispatch<kBF16>(v.nin, v.q1, v.q2, sp.vpt, go);
    else dispatch<kF16>(v.nin, v.q1, v.q2, sp.vpt, go);
    if (!found) err = hipErrorInvalidValue;
  }
  return err;
}

}  // namespace adq
