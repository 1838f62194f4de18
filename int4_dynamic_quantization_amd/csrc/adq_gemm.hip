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
// Three kernels with workgroups of four wavefronts: w8a8_kernel (128 x 128
// tiles, for problems with few tiles) and w8a8_big_kernel (256 x 256 tiles,
// described at its definition), both on v_mfma_i32_32x32x32_i8, and
// w8a8_skinny_kernel (32 columns and up to 128 rows, for few rows, on
// v_mfma_i32_16x16x64_i8; described at its definition).
//
// w8a8_kernel: each wavefront owns (32*TM) x (32*TN) outputs as TM x TN MFMA
// blocks.  K advances in steps of BK bytes through a double buffer in LDS:
// the next step's A and W tiles are loaded from global memory into registers
// while the current step's MFMAs run, then written to the other buffer; one
// barrier per step.  LDS rows are padded by 16 bytes so the 16-byte fragment
// reads of a wavefront hit distinct banks.  Operand
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

// 256 x 256 tiles: K steps of 128 bytes in a 2-stage ring (measured: 64-byte
// steps with 2 stages 1262 us, 3-4 stages 1090-1118 us; 128-byte steps with
// 2 stages 1053 us on 16384 x 8192 x 8192).
constexpr int kBigTileK = 128;
constexpr int kBigTileStages = 2;

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

// ---------------------------------------------------------------------------
// 256 x 256 tiles for large problems.  Each wavefront owns 128 x 128 outputs
// (4 x 4 blocks of 32x32x32), which halves the LDS bytes read per MFMA
// compared with 64 x 64 per wavefront.  Tiles reach LDS through the buffer
// unit's direct-to-LDS path (buffer_load_dwordx4 ... lds): no staging
// registers, and a ring of STAGES buffers of BK bytes of K keeps up to
// STAGES - 1 K-steps in flight.
//
// A direct-to-LDS load writes lane l's 16 bytes at the instruction's LDS base
// + 16 * l, so a 1 KB segment holds 1024 / BK tile rows of BK / 16 chunks.
// The lane that fills position p of row r fetches chunk c = p ^ h(r) of that
// row: h(r) = (r >> 2) & 3 for BK = 64, (r >> 1) & 7 for BK = 128.  gfx950's
// LDS serves a 128-bit read in four passes of 16 lanes over 64 four-byte
// banks; measured with the LDS bank-conflict counter, a pass takes lanes
// from one half of the wavefront whose index bits 2 and 4 agree in parity
// (the fits also allow bits 0 and 3 to join that parity).  A fragment read
// has lane l on row l % 32, one chunk per half, so a pass holds 16 rows; with
// these h every pass touches 64 distinct banks for each of those lane
// groupings (measured: no conflict cycles).  Without the swizzle a pass hits
// only 16 (BK = 64) or 8 (BK = 128) banks.
template <int BK_, int STAGES>
struct BigShape {
  static constexpr int BM = 256, BN = 256, BK = BK_;
  static constexpr int SEG = 1024;                       // bytes per direct-load instruction
  static constexpr int CPR = BK / 16;                    // 16-byte chunks per tile row
  static constexpr int RPS = SEG / BK;                   // tile rows per segment
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int SEGS_PER_WAVE = A_BYTES / SEG / 4;  // per operand, 4 wavefronts
  static constexpr int LOADS = 2 * SEGS_PER_WAVE;          // per wavefront per stage
  static constexpr int NKK = BK / 32;                      // MFMA k-steps per stage
  static_assert(BK == 64 || BK == 128, "swizzle defined for 64- and 128-byte rows");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

template <int BK>
__device__ __forceinline__ int chunk_swizzle(int r) {
  return BK == 64 ? (r >> 2) & 3 : (r >> 1) & 7;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int BK, int STAGES, int OUT>
__global__ void __launch_bounds__(256) w8a8_big_kernel(const GemmArgs g) {
  using S = BigShape<BK, STAGES>;
  __shared__ __attribute__((aligned(1024))) int8_t lds[S::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

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
  const int64_t m0 = (first_m + in_group % rows_in_group) * S::BM;
  const int64_t n0 = (in_group / rows_in_group) * S::BN;

  const int64_t a_rows = g.m - m0 < S::BM ? g.m - m0 : S::BM;
  const int64_t w_rows = g.n - n0 < S::BN ? g.n - n0 : S::BN;
  const rsrc_t ra = make_rsrc(g.a + m0 * g.k, (uint32_t)(a_rows * g.k));
  const rsrc_t rw = make_rsrc(g.w + n0 * g.k, (uint32_t)(w_rows * g.k));
  constexpr uint32_t kOut = 0x80000000u;

  // this lane's source in each of the wavefront's segments: row
  // r = RPS * seg + lane / CPR (the same rows for A and W), chunk
  // c = (lane % CPR) ^ h(r)
  uint32_t src[S::SEGS_PER_WAVE];
  int src_k[S::SEGS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < S::SEGS_PER_WAVE; ++i) {
    const int r = S::RPS * (wave * S::SEGS_PER_WAVE + i) + lane / S::CPR;
    const int c = (lane % S::CPR) ^ chunk_swizzle<BK>(r);
    src[i] = (uint32_t)(r * g.k) + 16u * c;
    src_k[i] = 16 * c;
  }
  using lds_ptr = __attribute__((address_space(3))) void*;
  auto issue = [&](int64_t step, int buf) {
    const int64_t k0 = step * S::BK;
    int8_t* base = lds + buf * S::STAGE_BYTES + wave * S::SEGS_PER_WAVE * S::SEG;
#pragma unroll
    for (int i = 0; i < S::SEGS_PER_WAVE; ++i) {
      const uint32_t off = k0 + src_k[i] < g.k ? src[i] + (uint32_t)k0 : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(base + i * S::SEG), 16, off, 0, 0,
                                               0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(base + S::A_BYTES + i * S::SEG), 16,
                                               off, 0, 0, 0);
    }
  };

  i32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x16{};

  // fragment addresses (relative to a stage): row R of the A (W) tile, chunk
  // 2 * kk + lane / 32 at position chunk ^ h(R); h depends on R only through
  // lane % 32 (the block offsets are multiples of 32), so it is per lane.
  const int fr = lane & 31;
  const int hsw = chunk_swizzle<BK>(fr);
  const int fk = lane >> 5;
  int a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_off[i] = (wm * 128 + i * 32 + fr) * S::BK;
    b_off[i] = S::A_BYTES + (wn * 128 + i * 32 + fr) * S::BK;
  }

  const int64_t ksteps = (g.k + S::BK - 1) / S::BK;
  auto read = [&](const int8_t* st, int kk, i32x4* fa, i32x4* fb) {
    const int pos = 16 * (((kk * 2) + fk) ^ hsw);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const i32x4*>(st + a_off[i] + pos);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const i32x4*>(st + b_off[j] + pos);
  };
  auto mfma = [&](const i32x4* fa, const i32x4* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // Barrier without a memory fence: a fence would make every wavefront wait
  // for all of its direct-to-LDS loads, including the later stages in flight.
  // The stage about to be read is awaited explicitly: loads complete in
  // order, so it has landed once no more than the `later` stages issued after
  // it (LOADS each) are outstanding.  LDS reads of the stage being retired
  // complete (lgkmcnt) before the barrier, so after it that buffer may be
  // refilled.
  auto sync_stage = [&](int64_t later) {
    constexpr int L = S::LOADS;
    if constexpr (STAGES >= 4) {
      if (later >= 3) wait_vmcnt<3 * L>();
      else if (later == 2) wait_vmcnt<2 * L>();
      else if (later == 1) wait_vmcnt<L>();
      else wait_vmcnt<0>();
    } else if constexpr (STAGES == 3) {
      if (later >= 2) wait_vmcnt<2 * L>();
      else if (later == 1) wait_vmcnt<L>();
      else wait_vmcnt<0>();
    } else {
      if (later >= 1) wait_vmcnt<L>();
      else wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
  };
  auto min64 = [](int64_t x, int64_t y) { return x < y ? x : y; };

  // prologue: stages 0 .. STAGES-1 in flight; stage 0 visible, its first k-step read
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < ksteps) issue(s, s);
  i32x4 fa[2][4], fb[2][4];
  sync_stage(min64(STAGES - 1, ksteps - 1));
  read(lds, 0, fa[0], fb[0]);
  // One step = NKK k-steps of 32 over stage s.  Each k-step reads the next
  // k-step's fragments while its own MFMAs run; the last one first syncs on
  // stage s + 1 (issued so far: stages up to s + STAGES - 1), reads its first
  // k-step, and refills stage s's buffer, which every wavefront has finished
  // reading.  Instruction order is set with sched_group_barrier (masks 0x008
  // MFMA, 0x020 vector-memory read, 0x100 LDS read): the LDS reads and the
  // direct-to-LDS loads issue between MFMAs, in their shadow.  The last step
  // is peeled so that every loop iteration has the same waits.
  auto step = [&](int64_t s, bool last, bool refill) {
    const int buf = (int)(s % STAGES);
    const int8_t* cur = lds + buf * S::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < S::NKK; ++kk) {
      const int c = kk & 1, n = c ^ 1;
      if (kk + 1 < S::NKK) {
        read(cur, kk + 1, fa[n], fb[n]);
        mfma(fa[c], fb[c]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      } else if (!last) {
        sync_stage(min64(STAGES - 2, ksteps - 2 - s));
        read(lds + (int)((s + 1) % STAGES) * S::STAGE_BYTES, 0, fa[n], fb[n]);
        if (refill) issue(s + STAGES, buf);
        mfma(fa[c], fb[c]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, S::LOADS / 8, 0);
        }
      } else {
        mfma(fa[c], fb[c]);
      }
    }
  };
  static_assert(S::NKK % 2 == 0, "fragment sets alternate within a stage");
  int64_t s = 0;
  for (; s + STAGES < ksteps; ++s) step(s, false, true);
  for (; s + 1 < ksteps; ++s) step(s, false, false);
  step(s, true, false);

  // ---- epilogue: out = float(acc) * a_scale[row] * w_scale[col] (+ bias[col]).
  // Scales are loaded up front through range-checked buffer loads (0 past the
  // end).  Outputs go through a descriptor over this tile's rows of out (row r
  // at r * n, column n0 + c within it); the offset is sent out of range for
  // columns past N, and rows past M fall outside the descriptor.
  const rsrc_t rsa = make_rsrc(g.a_scale + m0, (uint32_t)(a_rows * 4));
  const rsrc_t rsw = make_rsrc(g.w_scale + n0, (uint32_t)(w_rows * 4));
  const rsrc_t rb = make_rsrc(g.bias ? g.bias + n0 : g.w_scale + n0,
                              g.bias ? (uint32_t)(w_rows * 4) : 0u);
  constexpr int OB = OUT == kGemmOutF32 ? 4 : 2;  // output bytes
  const rsrc_t ro = make_rsrc(static_cast<int8_t*>(g.out) + m0 * g.n * OB,
                              (uint32_t)min64(a_rows * g.n * OB, 0x7FFFFFFF));
  float sa[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = wm * 128 + i * 32 + (e / 4) * 8 + (lane >> 5) * 4 + (e & 3);
      sa[i][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, r * 4, 0, 0));
    }
  float swv[4], bv[4];
  uint32_t col_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = wn * 128 + j * 32 + (lane & 31);
    swv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsw, c * 4, 0, 0));
    bv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, c * 4, 0, 0));
    col_off[j] = n0 + c < g.n ? (uint32_t)((n0 + c) * OB) : kOut;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = wm * 128 + i * 32 + (e / 4) * 8 + (lane >> 5) * 4 + (e & 3);
      const uint32_t row_off = (uint32_t)(r * g.n * OB);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = (float)acc[i][j][e] * sa[i][e] * swv[j] + bv[j];
        const uint32_t off = col_off[j] == kOut ? kOut : row_off + col_off[j];
        if constexpr (OUT == kGemmOutF32) {
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro, off, 0,
                                                kStreamStore);
        } else {
          __builtin_amdgcn_raw_buffer_store_b16(
              narrow1<OUT == kGemmOutBF16 ? kBF16 : kF16>(v), ro, off, 0, kStreamStore);
        }
      }
    }
}

// ---- few rows: w8a8_skinny_kernel
// With few rows the product is bound by reading the weights (n x k bytes),
// and output tiles of 128 rows or more leave most CUs idle.  Here a
// workgroup owns 32 columns and all rows of a 32 * TM row block, and its four
// wavefronts split K: wavefront w takes the 128-byte K chunks w, w + 4, ...
// (two 64-byte MFMA steps each), requested D chunks ahead into a ring of
// registers straight from global memory (every load is issued, past K or
// the tile's rows it reads 0 through the buffer range check, so each wait
// counts exactly).  The products are v_mfma_i32_16x16x64_i8: its fragments
// are 16 rows of 64 contiguous bytes (lane l: row l % 16, bytes
// 16 (l / 16) .. + 16), so a fragment load touches 16 rows' cache lines,
// half as many as the 32 x 32 x 32 form's.  The four int32 partial sums of
// every output meet in LDS and are added exactly (integer addition); the
// epilogue is the same as the other kernels'.  Workgroups of one column
// block are consecutive on one XCD, so a weight block read by several row
// blocks is shared in that XCD's L2.
constexpr int kSkinnyCols = 32;
constexpr int kSkinnyChunk = 128;  // K bytes per chunk (2 MFMA steps of 64)

template <int TM> constexpr int skinny_depth() { return TM >= 4 ? 3 : 4; }

template <int TM, int OUT>
__global__ void __launch_bounds__(256) w8a8_skinny_kernel(const GemmArgs g) {
  constexpr int D = skinny_depth<TM>();
  constexpr int BM = 32 * TM;
  constexpr int RB = 2 * TM;  // 16-row blocks
  __shared__ int32_t part[4][RB][2][4][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- tile: column blocks dealt to XCDs in contiguous ranges, the row
  // blocks of a column block consecutive
  const int64_t tiles_m = (g.m + BM - 1) / BM;
  const int64_t tiles_n = (g.n + kSkinnyCols - 1) / kSkinnyCols;
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t b = blockIdx.x;
  const int64_t per_xcd = (tiles + kXcdCount - 1) / kXcdCount;
  const int64_t t = (b % kXcdCount) * per_xcd + b / kXcdCount;
  if (t >= tiles) return;
  const int64_t tn = t / tiles_m, tm = t % tiles_m;
  const int64_t m0 = tm * BM, n0 = tn * kSkinnyCols;
  const int64_t a_rows = g.m - m0 < BM ? g.m - m0 : BM;
  const int64_t w_rows = g.n - n0 < kSkinnyCols ? g.n - n0 : kSkinnyCols;
  const rsrc_t ra = make_rsrc(g.a + m0 * g.k, (uint32_t)(a_rows * g.k));
  const rsrc_t rw = make_rsrc(g.w + n0 * g.k, (uint32_t)(w_rows * g.k));
  constexpr uint32_t kOut = 0x80000000u;  // beyond any tile descriptor

  // this lane's fragment row (of a 16-row block) and its 16 bytes of each
  // 64-byte MFMA step
  const uint32_t frow = (uint32_t)(lane & 15);
  const int64_t fk = (lane >> 4) * 16;
  const int64_t nchunks = (g.k + kSkinnyChunk - 1) / kSkinnyChunk;
  const int64_t rounds = (nchunks + 3) / 4;  // chunks per wavefront (the last ones may be past K)

  i32x4 ra_[D][2][RB], rw_[D][2][2];
  auto issue = [&](int slot, int64_t round) {
    const int64_t c = round * 4 + wave;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t k = c * kSkinnyChunk + s * 64 + fk;
      const bool in = k < g.k;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        rw_[slot][s][j] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rw, in ? (uint32_t)((j * 16 + frow) * g.k + k) : kOut, 0, 0));
#pragma unroll
      for (int i = 0; i < RB; ++i)
        ra_[slot][s][i] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       ra, in ? (uint32_t)((i * 16 + frow) * g.k + k) : kOut, 0, 0));
    }
  };

  i32x4 acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i) acc[i][0] = acc[i][1] = i32x4{};
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);
  for (int64_t r = 0; r < rounds; r += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra_[d][s][i], rw_[d][s][j], acc[i][j],
                                                              0, 0, 0);
      issue(d, r + d + D);  // past the last round: reads 0, never used
    }
  }

  // ---- the four wavefronts' partial sums, added in LDS
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) part[wave][i][j][e][lane] = acc[i][j][e];
  __syncthreads();

  // ---- epilogue: out = float(sum) * a_scale[row] * w_scale[col] (+ bias[col]);
  // element e of lane l in block (i, j) is row 16 i + 4 (l / 16) + e, column
  // 16 j + l % 16
  const rsrc_t rsa = make_rsrc(g.a_scale + m0, (uint32_t)(a_rows * 4));
  const rsrc_t rsw = make_rsrc(g.w_scale + n0, (uint32_t)(w_rows * 4));
  const rsrc_t rb = make_rsrc(g.bias ? g.bias + n0 : g.w_scale + n0,
                              g.bias ? (uint32_t)(w_rows * 4) : 0u);
  constexpr int OB = OUT == kGemmOutF32 ? 4 : 2;  // output bytes
  const int64_t out_bytes = a_rows * g.n * OB;
  const rsrc_t ro = make_rsrc(static_cast<int8_t*>(g.out) + m0 * g.n * OB,
                              (uint32_t)(out_bytes < 0x7FFFFFFF ? out_bytes : 0x7FFFFFFF));
#pragma unroll
  for (int q = 0; q < 4 * TM; ++q) {
    const int idx = q * 256 + tid;  // (i, j, e, lane) of the accumulator layout
    const int i = idx >> 9, j = (idx >> 8) & 1, e = (idx >> 6) & 3;
    const int32_t sum = part[0][i][j][e][lane] + part[1][i][j][e][lane] +
                        part[2][i][j][e][lane] + part[3][i][j][e][lane];
    const int row = i * 16 + 4 * (lane >> 4) + e;
    const int col = j * 16 + (lane & 15);
    const float sa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, row * 4, 0, 0));
    const float swv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsw, col * 4, 0, 0));
    const float bv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, col * 4, 0, 0));
    const float v = (float)sum * sa * swv + bv;
    const uint32_t off = n0 + col < g.n ? (uint32_t)(row * g.n * OB) + (uint32_t)((n0 + col) * OB)
                                        : kOut;
    if constexpr (OUT == kGemmOutF32) {
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro, off, 0, kStreamStore);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16(narrow1<OUT == kGemmOutBF16 ? kBF16 : kF16>(v), ro,
                                            off, 0, kStreamStore);
    }
  }
}

template <int TM, int OUT>
hipError_t launch_skinny(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles = ((g.m + 32 * TM - 1) / (32 * TM)) * ((g.n + kSkinnyCols - 1) / kSkinnyCols);
  const int64_t grid = (tiles + kXcdCount - 1) / kXcdCount * kXcdCount;
  hipLaunchKernelGGL((w8a8_skinny_kernel<TM, OUT>), dim3((unsigned)grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int TM>
hipError_t launch_skinny_out(const GemmArgs& g, hipStream_t s) {
  switch (g.out_type) {
    case kGemmOutF32: return launch_skinny<TM, kGemmOutF32>(g, s);
    case kGemmOutBF16: return launch_skinny<TM, kGemmOutBF16>(g, s);
    case kGemmOutF16: return launch_skinny<TM, kGemmOutF16>(g, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BK, int STAGES, int OUT>
hipError_t launch_big(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles = ((g.m + 255) / 256) * ((g.n + 255) / 256);
  const int64_t grid = (tiles + kXcdCount - 1) / kXcdCount * kXcdCount;
  hipLaunchKernelGGL((w8a8_big_kernel<BK, STAGES, OUT>), dim3((unsigned)grid), dim3(256), 0, s,
                     g);
  return hipGetLastError();
}

template <int BK, int STAGES>
hipError_t launch_big_out(const GemmArgs& g, hipStream_t s) {
  switch (g.out_type) {
    case kGemmOutF32: return launch_big<BK, STAGES, kGemmOutF32>(g, s);
    case kGemmOutBF16: return launch_big<BK, STAGES, kGemmOutBF16>(g, s);
    case kGemmOutF16: return launch_big<BK, STAGES, kGemmOutF16>(g, s);
    default: return hipErrorInvalidValue;
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
    case kGemmTile256: return launch_big_out<kBigTileK, kBigTileStages>(g, stream);
    case kGemmTileSkinny:
      return g.m <= 32 ? launch_skinny_out<1>(g, stream)
             : g.m <= 64 ? launch_skinny_out<2>(g, stream)
                         : launch_skinny_out<4>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace adq
