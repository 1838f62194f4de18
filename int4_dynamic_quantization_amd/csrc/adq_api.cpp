// C-ABI of libaddrmsnorm_dq: argument validation, kernel planning and launch.
//
// Two-phase form of the operator pages ("aclnnAddRmsNormDynamicQuantV2" and
// "aclnnRmsNormDynamicQuant": a GetWorkspaceSize call that checks the
// arguments and builds an executor, then the call that runs it on a
// stream).  Output validity and the outputMask rules follow the V2 page's
// Formula cases and Constraints section.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "adq.h"
#include "adq_internal.h"

namespace adq {

hipError_t launch_row_bf16(const Variant&, int, bool, int, int, const Args&, hipStream_t);
hipError_t launch_row_f16(const Variant&, int, bool, int, int, const Args&, hipStream_t);
int row_occupancy_bf16(const Variant&, int, int);
int row_occupancy_f16(const Variant&, int, int);

hipError_t launch_row(const Variant& v, int vpt, bool wt, int block, int grid, const Args& a,
                      hipStream_t s) {
  return v.elem == kBF16 ? launch_row_bf16(v, vpt, wt, block, grid, a, s)
                         : launch_row_f16(v, vpt, wt, block, grid, a, s);
}

int row_max_blocks_per_cu(const Variant& v, int vpt, int block) {
  return v.elem == kBF16 ? row_occupancy_bf16(v, vpt, block) : row_occupancy_f16(v, vpt, block);
}

}  // namespace adq

namespace {

using adq::Args;
using adq::Variant;

thread_local std::string g_last_error;

adq_status fail(adq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

adq_status ok() {
  g_last_error.clear();
  return ADQ_OK;
}

enum Op { kOpV2 = 1, kOpRmsNorm = 2, kOpGemm = 3, kOpLora = 4 };

}  // namespace

struct adq_executor {
  int op;
  Variant var;
  Args args;
  adq::GemmArgs gemm;
  int gemm_tile;
  adq::LoraArgs lora;
  bool lora_tiled_ok;
  int64_t lora_chunk_rows;  // tiled path: rows per launch sequence
  int64_t m;
  int device;
  int cus;
  bool vector_ok;  // n % 8 == 0, aligned tensors, n small enough for the row kernel
  int path;
  int vpt;
  int block;
  int grid;
  int splits;
  int launches;        // split-row path: 1, 2 or 3 launches per batch of rows
  int plain_launches;  // split-row path: the plain form (2 or 3) a captured call runs
  int64_t batch_rows;  // split-row path: rows per batch
  int split_req;       // split-row path: requested chunks per row (0 = planner's)
  int launch_req;      // split-row path: requested launch form (0 = planner's)
  int spread;          // split-row path: a row's chunks on different XCDs (tests)
  uint32_t wait_ticks; // split-row path, one-launch form: wait budget (10 ns ticks)
  bool write_through;  // row path: sc1 stores (launches that move little data)
  uint64_t ws_bytes;
};

namespace {

int64_t numel(const adq_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

bool is_half(int32_t dt) { return dt == ADQ_F16 || dt == ADQ_BF16; }

const char* dtype_name(int32_t dt) {
  switch (dt) {
    case ADQ_F16: return "F16";
    case ADQ_BF16: return "BF16";
    case ADQ_F32: return "F32";
    case ADQ_INT8: return "INT8";
    case ADQ_INT4X2: return "INT4X2";
    case ADQ_INT32: return "INT32";
    default: return "unknown";
  }
}

// Basic well-formedness of a present tensor.
adq_status check_tensor(const adq_tensor* t, const char* name) {
  if (!t->data) return fail(ADQ_ERR_NULLPTR, "%s: data pointer is NULL", name);
  if (t->ndim < 0 || t->ndim > ADQ_MAX_DIMS)
    return fail(ADQ_ERR_PARAM_INVALID, "%s: ndim %d outside 0..%d", name, t->ndim, ADQ_MAX_DIMS);
  int64_t elems = 1;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] < 0) return fail(ADQ_ERR_PARAM_INVALID, "%s: negative dimension", name);
    if (t->shape[i] == 0)
      return fail(ADQ_ERR_PARAM_INVALID, "%s: empty tensors are not supported", name);
    // element counts stay far below int64 overflow everywhere downstream
    if (__builtin_mul_overflow(elems, t->shape[i], &elems) || elems > ((int64_t)1 << 46))
      return fail(ADQ_ERR_PARAM_INVALID, "%s: more than 2^46 elements", name);
  }
  return ADQ_OK;
}

bool same_shape(const adq_tensor* a, const adq_tensor* b) {
  if (a->ndim != b->ndim) return false;
  for (int i = 0; i < a->ndim; ++i)
    if (a->shape[i] != b->shape[i]) return false;
  return true;
}

// gamma / beta / smooth: [n], same dtype as x.
adq_status check_param(const adq_tensor* t, const char* name, int32_t dt, int64_t n) {
  adq_status st = check_tensor(t, name);
  if (st != ADQ_OK) return st;
  if (t->dtype != dt)
    return fail(ADQ_ERR_PARAM_INVALID, "%s: dtype %s differs from the input's %s", name,
                dtype_name(t->dtype), dtype_name(dt));
  if (t->ndim != 1 || t->shape[0] != n)
    return fail(ADQ_ERR_PARAM_INVALID, "%s: expected shape [%lld]", name, (long long)n);
  return ADQ_OK;
}

// A produced quantized output and its scale.
adq_status check_output(const adq_tensor* y, const adq_tensor* s, const char* yname,
                        const char* sname, const adq_tensor* x, int* qkind) {
  if (!y) return fail(ADQ_ERR_NULLPTR, "%s is required for this call", yname);
  if (!s) return fail(ADQ_ERR_NULLPTR, "%s is required for this call", sname);
  adq_status st = check_tensor(y, yname);
  if (st != ADQ_OK) return st;
  st = check_tensor(s, sname);
  if (st != ADQ_OK) return st;
  const int64_t n = x->shape[x->ndim - 1];
  if (y->dtype == ADQ_INT8) {
    *qkind = adq::kQInt8;
  } else if (y->dtype == ADQ_INT4X2) {
    *qkind = adq::kQInt4;
    if (n % 2 != 0)
      return fail(ADQ_ERR_PARAM_INVALID, "%s: INT4X2 needs an even last dimension (n = %lld)",
                  yname, (long long)n);
  } else {
    return fail(ADQ_ERR_UNSUPPORTED, "%s: dtype %s; expected INT8 or INT4X2", yname,
                dtype_name(y->dtype));
  }
  if (y->ndim != x->ndim)
    return fail(ADQ_ERR_PARAM_INVALID, "%s: rank differs from the input's", yname);
  for (int i = 0; i + 1 < x->ndim; ++i)
    if (y->shape[i] != x->shape[i])
      return fail(ADQ_ERR_PARAM_INVALID, "%s: leading dimensions differ from the input's", yname);
  const int64_t last = *qkind == adq::kQInt4 ? n / 2 : n;
  if (y->shape[y->ndim - 1] != last)
    return fail(ADQ_ERR_PARAM_INVALID, "%s: last dimension %lld, expected %lld", yname,
                (long long)y->shape[y->ndim - 1], (long long)last);
  if (s->dtype != ADQ_F32)
    return fail(ADQ_ERR_PARAM_INVALID, "%s: dtype %s; expected F32", sname,
                dtype_name(s->dtype));
  if (numel(s) != numel(x) / n)
    return fail(ADQ_ERR_PARAM_INVALID, "%s: %lld elements, expected one per row (%lld)", sname,
                (long long)numel(s), (long long)(numel(x) / n));
  return ADQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return p == nullptr || (uintptr_t)p % a == 0; }

// Bytes of a tensor's storage.
uint64_t tensor_bytes(const adq_tensor* t) {
  uint64_t esz = 2;
  if (t->dtype == ADQ_F32 || t->dtype == ADQ_INT32) esz = 4;
  else if (t->dtype == ADQ_INT8 || t->dtype == ADQ_INT4X2) esz = 1;
  return (uint64_t)numel(t) * esz;
}

bool overlaps(const adq_tensor* a, const adq_tensor* b) {
  if (!a || !b || !a->data || !b->data) return false;
  const uintptr_t a0 = (uintptr_t)a->data, b0 = (uintptr_t)b->data;
  return a0 < b0 + tensor_bytes(b) && b0 < a0 + tensor_bytes(a);
}

// Outputs must not share memory with inputs or with each other: the
// split-row and generic kernels read x1 and x2 again after xOut and the codes
// of the same row are written.
adq_status check_no_overlap(const adq_tensor* const* ins, int nin, const adq_tensor* const* outs,
                            int nout) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlaps(outs[o], ins[i]))
        return fail(ADQ_ERR_PARAM_INVALID, "an output shares memory with an input");
    for (int p = 0; p < o; ++p)
      if (overlaps(outs[o], outs[p]))
        return fail(ADQ_ERR_PARAM_INVALID, "two outputs share memory");
  }
  return ADQ_OK;
}

struct DeviceInfo {
  int cus = 0;
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

adq_status current_device(int* dev, int* cus) {
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess || d < 0) {
    (void)hipGetLastError();
    return fail(ADQ_ERR_RUNTIME, "no HIP device available");
  }
  if (d >= 64) return fail(ADQ_ERR_RUNTIME, "device index %d out of range", d);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev[d].cus == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      return fail(ADQ_ERR_RUNTIME, "cannot query the compute-unit count of device %d", d);
    }
    g_dev[d].cus = n;
  }
  *dev = d;
  *cus = g_dev[d].cus;
  return ADQ_OK;
}

int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Tags of the split-row path's one-launch form, `count` consecutive ones of
// a sequence unique within the process (a Weyl sequence with an odd step
// has period 2^64), starting from a value mixed from the clock and an
// address, so that workspace contents left by another process do not repeat
// them; one tag per batch of rows of a call.
uint64_t next_tags(uint64_t count) {
  static std::atomic<uint64_t> counter{[] {
    uint64_t z = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                 (uint64_t)(uintptr_t)&g_last_error;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
  }()};
  return counter.fetch_add(count * adq::kSplitTagStep, std::memory_order_relaxed);
}

// ---- planning constants (each measured on an MI355X; the numbers behind
// them are in the design notes of the repository)

// Row kernel: rows of up to 64 8-column vectors take one vector per thread,
// up to 2048 two, up to 4096 (32768 columns) four, up to 8192 (65536
// columns) eight, half of them held in LDS; longer rows do not fit one
// workgroup.
constexpr int64_t kRowVpt1MaxVec = 64;
constexpr int64_t kRowVpt2MaxVec = 2048;
constexpr int64_t kRowVpt4MaxVec = 4096;
constexpr int64_t kRowMaxVec = 8192;
// Rows of 3840-4096 columns in launches of at most 16 rows per CU take one
// vector per thread (480-512 threads) instead of two.  Launch to launch
// after 40 ms of launches, two vectors -> one, us: bf16 4096 x 4096 with one
// INT8 output 20.9 -> 20.0, with two 25.2 -> 23.8, 1024 rows 8.05 -> 7.6,
// 256 rows 4.13 -> 3.9, 4096 x 3840 19.6 -> 19.2; fp16 INT4 4096 x 4096
// 19.6 -> 18.9, RmsNormDynamicQuant 14.1 -> 13.8.  Not taken: 8192 rows
// and more (within 1%, RmsNormDynamicQuant 8192 x 4096 3% slower), 3584 and
// 3072 columns (2-9% slower).
constexpr int64_t kRowVpt1WideMinVec = 480;
constexpr int64_t kRowVpt1WideMaxVec = 512;
// Rows per workgroup of the row kernel, from the rows each CU has to stream.
// Fewer than 16 rows per CU, and rows of more than 8192 columns: one
// persistent wave of workgroups (every resident slot once).  Otherwise
// workgroups of a few rows each (grid-strided, each with its next row in
// flight), which the dispatcher hands to CUs as slots free up: one row when
// a row holds at most 4 KiB of input, else 8 rows for 16-32 rows per CU (4
// for rows of up to 2048 columns, whose workgroups are small), 2 for 32-64
// (and above, for rows of more than 6144 columns), and above that as many
// as make about 16 workgroups per resident slot over the launch (at least
// 3).  Swept over 1, 2, 3, 4, 6, 8, 12, 16 rows and the persistent wave on
// 50 shapes (1024-32768 columns, 4096-262144 rows, one and two INT8
// outputs, INT4, RmsNormDynamicQuant), each timed after 40 ms of launches:
// this rule is 1.1% slower than each shape's best on average (12 or 20
// workgroups per slot instead of 16: 1.2%, 1.6%); the persistent wave is
// 11.6% slower, and 24 times the slots for 16 or more rows per slot 6.5%.
// bf16 16384 x 8192 with two INT8 outputs: 182.7 us persistent, 165.0 with
// 2 rows per workgroup; fp16 65536 x 5120 INT4: 416.4 persistent, 354.8
// with 3, 343.0 with 4 (16 per slot).
constexpr int64_t kWaveRowsMaxN = 8192;
constexpr int64_t kFewRowsPerCu = 16;
constexpr int64_t kMidRowsPerCu = 32;
constexpr int64_t kManyRowsPerCu = 64;
constexpr int64_t kShortRowsMaxN = 2048;
constexpr int64_t kOneRowMaxBytes = 4096;
constexpr int64_t kWgPerSlot = 16;
constexpr int64_t kWgPerSlotMaxN = 6144;
constexpr int64_t kManyRowsMinPerWg = 3;
// Row kernel stores: sc1 instead of non-temporal when the grid is one wave
// (every workgroup resident at once) and the launch moves at most this many
// bytes; non-temporal for grids of several generations of workgroups and
// for larger launches.  Launch to launch after 40 ms of launches, bf16, nt
// against sc1, us: one wave, 4096 x 16384 two INT8 outputs (537 MB) 95.1 /
// 87.1, 2048 x 16384 51.5 / 48.9, 4096 x 4096 one output 21.3 / 20.1,
// 4096 x 8192 two 46.6 / 42.8, 8192 x 12288 (805 MB) 140.2 / 143.0; several
// generations, 16384 x 3072 one output (352 MB) 56.3 / 59.6, 12288 x 4096
// 56.4 / 58.7, 16384 x 2048 39.2 / 40.8, 8192 x 8192 75.9 / 80.3, the
// headline 16384 x 8192 165.0 / 185.6.  Exceptions measured: 8192 x 8192
// with two outputs (two generations) 90.8 / 80.4, 20000 x 2048 47.3 / 45.9.
constexpr int64_t kRowWriteThroughMaxBytes = (int64_t)640 << 20;

// Split-row path: chunks of about 512 8-column vectors (4096 columns), at
// most 1024 threads x 2 vectors (16384 columns); for few rows, no more
// chunks than give each CU one workgroup.  Measured on 1-256 rows of
// 16384 and 32768 bf16 columns (one-launch form, two INT8 outputs): 4096-
// column chunks were the fastest or within 3% of it wherever rows x chunks
// stayed within the CUs.  Plain-launch batches of rows whose x1 and x2 take
// at most 64 MiB, so that the chunks the later launches read again are
// still in the 256 MB memory-side cache.
constexpr int64_t kSplitChunkVec = 512;
constexpr int64_t kSplitMaxChunkVec = 2048;
constexpr int64_t kSplitBatchBytes = (int64_t)64 << 20;
// The two-launch form (each workgroup of the last launch takes the row
// maxima over the whole row) up to this many chunks per row and this row
// length; beyond, the three-launch form.
constexpr int64_t kSplitWholeRowMaxSplits = 8;
constexpr int64_t kSplitWholeRowMaxVec = 4096;
// One-launch form: the planner takes it when every workgroup of the call
// fits on the chip at once; a wait for another chunk's partial result gives
// up after 20 us (the waiting workgroup then computes it itself).
constexpr uint32_t kSplitWaitTicksDefault = 2000;  // 10 ns ticks
// AUTO sends rows that fit the row kernel to the split-row path when they
// are at least 16384 columns long and few enough that two or more 4096-
// column chunks per row still give each CU at most one workgroup.  Launch
// to launch, cold, one-launch form against the row kernel (bf16, two INT8
// outputs): 32 x 16384 7.0 against 9.0 us, 1 x 32768 6.7 against 10.9 us,
// 128 x 16384 8.7 against 9.9 us; at 256 rows, and for rows of 4096 or
// 8192 columns at any count, the row kernel was as fast or faster.
constexpr int64_t kFewRowsMinVec = 2048;

// Bytes one launch of the operator moves: inputs read, xOut and the codes
// and scales written (the parameter vectors aside).
int64_t launch_bytes(const adq_executor& e) {
  const int64_t n = e.args.n;
  int64_t per_row = (int64_t)e.var.nin * 2 * n + (e.var.nin == 2 ? 2 * n : 0);
  for (int q : {e.var.q1, e.var.q2})
    if (q != adq::kQNone) per_row += (q == adq::kQInt4 ? n / 2 : n) + 4;
  return e.m * per_row;
}

int64_t row_rows_per_wg(int64_t m, int64_t n, int64_t row_in_bytes, int64_t cus, int64_t slots) {
  const int64_t wave = (m + slots - 1) / slots;  // one persistent wave
  if (n > kWaveRowsMaxN || m < kFewRowsPerCu * cus) return wave;
  if (row_in_bytes <= kOneRowMaxBytes) return 1;
  if (m <= kMidRowsPerCu * cus) return n <= kShortRowsMaxN ? 4 : 8;
  if (m <= kManyRowsPerCu * cus || n > kWgPerSlotMaxN) return 2;
  const int64_t per = (m + kWgPerSlot * slots / 2) / (kWgPerSlot * slots);  // nearest
  return per > kManyRowsMinPerWg ? per : kManyRowsMinPerWg;
}

bool row_geometry(int64_t nvec, int* vpt, int* block) {
  if (nvec <= 0) return false;
  if (nvec <= kRowVpt1MaxVec) {
    *vpt = 1, *block = round_up((int)nvec, 64);
  } else if (nvec <= kRowVpt2MaxVec) {
    *vpt = 2, *block = round_up((int)((nvec + 1) / 2), 64);
  } else if (nvec <= kRowVpt4MaxVec) {
    *vpt = 4, *block = round_up((int)((nvec + 3) / 4), 64);
  } else if (nvec <= kRowMaxVec) {
    *vpt = 8, *block = round_up((int)((nvec + 7) / 8), 64);
  } else {
    return false;
  }
  return true;
}

// Split-row geometry: S chunks per row (requested, or chunks of about
// kSplitChunkVec vectors, no more per row than give each CU one workgroup
// when the rows are few), each of block x vpt vectors; the launch form
// (requested; else one launch when the call's workgroups all fit on the chip
// at once, else two or three by the rule above); rows per batch.
bool split_geometry(adq_executor* e) {
  const int64_t nvec = e->args.n / 8;
  if (nvec < 1) return false;
  int64_t S = e->split_req;
  if (S <= 0) {
    S = nvec / kSplitChunkVec;
    const int64_t fill = e->cus / e->m;  // chunks per row that still fit one per CU
    if (fill >= 1 && S > fill) S = fill;
    if (S < 1) S = 1;
  }
  if (S > nvec) S = nvec;
  const int64_t least = (nvec + kSplitMaxChunkVec - 1) / kSplitMaxChunkVec;
  if (S < least) S = least;
  const int64_t chunk = (nvec + S - 1) / S;
  int vpt = 1;
  int64_t block = round_up((int)chunk, 64);
  if (block > 1024) {
    vpt = 2;
    block = round_up((int)((chunk + 1) / 2), 64);
  }
  S = (nvec + block * vpt - 1) / (block * vpt);
  const int plain = S <= kSplitWholeRowMaxSplits && nvec <= kSplitWholeRowMaxVec ? 2 : 3;
  // one-launch form when all workgroups of the call are resident at once
  const int occ = adq::split_exchange_blocks_per_cu(e->var, vpt, (int)block);
  const int64_t capacity = (int64_t)occ * e->cus;
  int launches = e->launch_req;
  if (launches == 0)
    launches = S <= 64 && adq::split_grid(e->m, (int)S) <= capacity ? 1 : plain;
  if (launches == 1 && (S > 64 || occ <= 0)) return false;
  int64_t batch;
  if (launches == 1) {
    // batches of rows whose workgroups fit on the chip at once
    batch = capacity / S;
    if (batch >= 8) batch -= batch % 8;
  } else {
    const int64_t row_bytes = (int64_t)e->var.nin * 2 * e->args.n;
    batch = kSplitBatchBytes / row_bytes;
    if (batch >= 8) batch -= batch % 8;
  }
  if (batch < 1) batch = 1;
  if (batch > e->m) batch = e->m;
  while (batch > 1 && adq::split_grid(batch, (int)S) > INT32_MAX) batch /= 2;
  if (adq::split_grid(batch, (int)S) > INT32_MAX) return false;
  e->vpt = vpt;
  e->block = (int)block;
  e->splits = (int)S;
  e->launches = launches;
  e->plain_launches = launches == 1 ? plain : launches;
  e->batch_rows = batch;
  e->grid = (int)adq::split_grid(batch, (int)S);
  // a captured one-launch call runs the plain form on the same workspace
  uint64_t ws = adq::split_workspace_bytes(batch, (int)S, launches);
  const uint64_t ws_plain = adq::split_workspace_bytes(batch, (int)S, e->plain_launches);
  e->ws_bytes = ws > ws_plain ? ws : ws_plain;
  return true;
}

adq_status plan(adq_executor* e, int path) {
  const int64_t n = e->args.n;
  if (path == ADQ_PATH_AUTO) {
    // Row kernel when it holds a row and there are rows enough for the
    // CUs; split-row for few or long rows; generic for rows that are not
    // whole 16-byte vectors or unaligned tensors.
    int vpt = 0, block = 0;
    const bool row_ok = e->vector_ok && row_geometry(n / 8, &vpt, &block);
    int64_t few_splits = n / 8 / kSplitChunkVec;
    if (e->cus / e->m < few_splits) few_splits = e->cus / e->m;
    const bool few_rows = n / 8 >= kFewRowsMinVec && few_splits >= 2;
    if (e->vector_ok && (!row_ok || few_rows)) {
      adq_executor trial = *e;
      if (split_geometry(&trial)) path = ADQ_PATH_SPLIT;
    }
    if (path == ADQ_PATH_AUTO) path = row_ok ? ADQ_PATH_ROW : ADQ_PATH_GENERIC;
  }
  if (path == ADQ_PATH_ROW) {
    int vpt = 0, block = 0;
    if (!e->vector_ok || !row_geometry(n / 8, &vpt, &block))
      return fail(ADQ_ERR_PARAM_INVALID,
                  "row path needs n %% 8 == 0, n <= %lld and 16-byte aligned tensors",
                  (long long)(kRowMaxVec * 8));
    if (n / 8 >= kRowVpt1WideMinVec && n / 8 <= kRowVpt1WideMaxVec &&
        e->m <= kFewRowsPerCu * e->cus) {
      vpt = 1;
      block = round_up((int)(n / 8), 64);
    }
    const int occ = adq::row_max_blocks_per_cu(e->var, vpt, block);
    if (occ <= 0) return fail(ADQ_ERR_RUNTIME, "row kernel does not fit block %d", block);
    int64_t per = row_rows_per_wg(e->m, n, (int64_t)e->var.nin * 2 * n, e->cus,
                                  (int64_t)occ * e->cus);
    // a dispatch holds fewer than 2^32 work-items
    const int64_t max_grid = ((int64_t)1 << 31) / block;
    if ((e->m + per - 1) / per > max_grid) per = (e->m + max_grid - 1) / max_grid;
    e->path = ADQ_PATH_ROW;
    e->vpt = vpt;
    e->block = block;
    e->grid = (int)((e->m + per - 1) / per);
    e->write_through =
        e->grid <= (int64_t)occ * e->cus && launch_bytes(*e) <= kRowWriteThroughMaxBytes;
    e->splits = 1;
    e->launches = 1;
    e->plain_launches = 1;
    e->batch_rows = e->m;
    e->ws_bytes = 0;
    return ADQ_OK;
  }
  if (path == ADQ_PATH_GENERIC) {
    e->path = ADQ_PATH_GENERIC;
    e->vpt = 0;
    e->block = 256;
    e->grid = (int)(e->m < (int64_t)e->cus * 8 ? e->m : (int64_t)e->cus * 8);
    e->write_through = false;
    e->splits = 1;
    e->launches = 1;
    e->plain_launches = 1;
    e->batch_rows = e->m;
    e->ws_bytes = 0;
    return ADQ_OK;
  }
  if (path == ADQ_PATH_SPLIT) {
    if (!e->vector_ok)
      return fail(ADQ_ERR_PARAM_INVALID,
                  "split-row path needs n %% 8 == 0 and 16-byte aligned tensors");
    if (!split_geometry(e)) return fail(ADQ_ERR_PARAM_INVALID, "split-row geometry does not fit");
    e->path = ADQ_PATH_SPLIT;
    e->write_through = false;
    return ADQ_OK;
  }
  return fail(ADQ_ERR_PARAM_INVALID, "unknown path %d", path);
}

// Shared tail of both phase-1 calls.
adq_status finish_plan(adq_executor* proto, uint64_t* workspace_size, adq_executor** executor) {
  adq_status st = current_device(&proto->device, &proto->cus);
  if (st != ADQ_OK) return st;
  proto->wait_ticks = kSplitWaitTicksDefault;
  const Args& a = proto->args;
  proto->vector_ok = a.n % 8 == 0 && aligned(a.x1, 16) && aligned(a.x2, 16) &&
                     aligned(a.x_out, 16) && aligned(a.gamma, 16) && aligned(a.beta, 16) &&
                     aligned(a.smooth1, 16) && aligned(a.smooth2, 16) && aligned(a.y1, 8) &&
                     aligned(a.y2, 8);
  st = plan(proto, ADQ_PATH_AUTO);
  if (st != ADQ_OK) return st;
  adq_executor* e = new (std::nothrow) adq_executor(*proto);
  if (!e) return fail(ADQ_ERR_RUNTIME, "out of host memory");
  *workspace_size = e->ws_bytes;
  *executor = e;
  return ok();
}

// Rows [r0, r0 + lora_chunk_rows) of an AddLora call (fewer for the last
// range) as arguments of their own: the tiled kernels address y, out and x
// with 32-bit byte offsets, so a batch beyond 4 GiB runs as consecutive
// launch sequences over row ranges below it.  Rows are independent of one
// another, and each sequence lays its own tables out in the workspace.
adq::LoraArgs lora_part(const adq_executor& e, int64_t r0) {
  adq::LoraArgs c = e.lora;
  const int64_t left = e.lora.rows - r0;
  c.rows = left < e.lora_chunk_rows ? left : e.lora_chunk_rows;
  c.y = static_cast<const char*>(c.y) + r0 * c.h3 * 2;
  c.out = static_cast<char*>(c.out) + r0 * c.h3 * 2;
  c.x = static_cast<const char*>(c.x) + r0 * c.h1 * 2;
  c.indices += r0;
  return c;
}

adq_status run(void* workspace, uint64_t workspace_size, adq_executor* e, void* stream, int op) {
  if (!e) return fail(ADQ_ERR_NULLPTR, "executor is NULL");
  if (e->op != op) return fail(ADQ_ERR_PARAM_INVALID, "executor was built for another operator");
  if (workspace_size < e->ws_bytes || (e->ws_bytes > 0 && !workspace))
    return fail(ADQ_ERR_WORKSPACE, "workspace of %llu bytes, %llu needed",
                (unsigned long long)workspace_size, (unsigned long long)e->ws_bytes);
  if (e->ws_bytes > 0 && (uintptr_t)workspace % 8 != 0)
    return fail(ADQ_ERR_WORKSPACE, "workspace must be 8-byte aligned");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ADQ_ERR_RUNTIME, "no HIP device available");
  }
  if (cur != e->device && hipSetDevice(e->device) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ADQ_ERR_RUNTIME, "cannot select device %d", e->device);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = hipErrorInvalidValue;
  if (op == kOpGemm || op == kOpLora) {
    if (op == kOpGemm) {
      err = adq::launch_w8a8(e->gemm, e->gemm_tile, s);
    } else if (e->path == ADQ_PATH_GENERIC) {
      err = adq::launch_lora(e->lora, adq::kLoraGeneric, workspace, s);
    } else {
      err = hipSuccess;
      for (int64_t r0 = 0; r0 < e->lora.rows && err == hipSuccess; r0 += e->lora_chunk_rows)
        err = adq::launch_lora(lora_part(*e, r0), adq::kLoraTiled, workspace, s);
    }
    if (cur != e->device) (void)hipSetDevice(cur);
    if (err != hipSuccess)
      return fail(ADQ_ERR_RUNTIME, "kernel launch failed: %s", hipGetErrorString(err));
    return ok();
  }
  switch (e->path) {
    case ADQ_PATH_ROW:
      err = adq::launch_row(e->var, e->vpt, e->write_through, e->block, e->grid, e->args, s);
      break;
    case ADQ_PATH_GENERIC: err = adq::launch_generic(e->var, e->block, e->grid, e->args, s); break;
    case ADQ_PATH_SPLIT: {
      adq::SplitPlan sp{e->vpt, e->block, e->splits, e->launches, e->batch_rows, e->spread,
                        e->wait_ticks, 0};
      if (sp.launches == 1) {
        // the one-launch form's tag is made here for each call; a captured
        // call (which a replay would repeat) runs the plain form instead,
        // and so does a call whose capture state cannot be read
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
          (void)hipGetLastError();
          cs = hipStreamCaptureStatusActive;
        }
        if (cs == hipStreamCaptureStatusNone)
          sp.tag = next_tags((uint64_t)((e->m + e->batch_rows - 1) / e->batch_rows));
        else
          sp.launches = e->plain_launches;
      }
      err = adq::launch_split(e->var, sp, e->args, workspace, s);
      break;
    }
    default: break;
  }
  if (cur != e->device) (void)hipSetDevice(cur);
  if (err != hipSuccess)
    return fail(ADQ_ERR_RUNTIME, "kernel launch failed: %s", hipGetErrorString(err));
  return ok();
}

}  // namespace

extern "C" {

adq_status adq_add_rms_norm_dynamic_quant_v2_get_workspace_size(
    const adq_tensor* x1, const adq_tensor* x2, const adq_tensor* gamma,
    const adq_tensor* beta, const adq_tensor* smooth_scale1, const adq_tensor* smooth_scale2,
    double epsilon, const bool* output_mask, const adq_tensor* y1_out,
    const adq_tensor* y2_out, const adq_tensor* scale1_out, const adq_tensor* scale2_out,
    const adq_tensor* x_out, uint64_t* workspace_size, adq_executor** executor) {
  if (!workspace_size || !executor)
    return fail(ADQ_ERR_NULLPTR, "workspace_size and executor out-pointers are required");
  *executor = nullptr;
  *workspace_size = 0;
  if (!x1 || !x2 || !gamma || !x_out)
    return fail(ADQ_ERR_NULLPTR, "x1, x2, gamma and x_out are required");
  adq_status st;
  if ((st = check_tensor(x1, "x1")) != ADQ_OK) return st;
  if (!is_half(x1->dtype))
    return fail(ADQ_ERR_UNSUPPORTED, "x1: dtype %s; expected F16 or BF16", dtype_name(x1->dtype));
  if (x1->ndim < 1) return fail(ADQ_ERR_PARAM_INVALID, "x1: needs at least one dimension");
  if ((st = check_tensor(x2, "x2")) != ADQ_OK) return st;
  if ((st = check_tensor(x_out, "x_out")) != ADQ_OK) return st;
  if (x2->dtype != x1->dtype || x_out->dtype != x1->dtype)
    return fail(ADQ_ERR_PARAM_INVALID, "x2 and x_out must have x1's dtype");
  if (!same_shape(x1, x2) || !same_shape(x1, x_out))
    return fail(ADQ_ERR_PARAM_INVALID, "x1, x2 and x_out must have the same shape");
  const int64_t n = x1->shape[x1->ndim - 1];
  if (n > INT32_MAX) return fail(ADQ_ERR_PARAM_INVALID, "last dimension too large");
  if ((st = check_param(gamma, "gamma", x1->dtype, n)) != ADQ_OK) return st;
  if (beta && (st = check_param(beta, "beta", x1->dtype, n)) != ADQ_OK) return st;
  if (smooth_scale1 && (st = check_param(smooth_scale1, "smooth_scale1", x1->dtype, n)) != ADQ_OK)
    return st;
  if (smooth_scale2 && (st = check_param(smooth_scale2, "smooth_scale2", x1->dtype, n)) != ADQ_OK)
    return st;
  if (!(epsilon == epsilon) || epsilon > 3.4e38 || epsilon < -3.4e38)
    return fail(ADQ_ERR_PARAM_INVALID, "epsilon must be a finite value");

  // Which outputs exist: V2 Formula cases; Constraints rules on the mask.
  const bool has1 = smooth_scale1 != nullptr, has2 = smooth_scale2 != nullptr;
  bool act1, act2;
  if (output_mask) {
    if (has1 && !output_mask[0])
      return fail(ADQ_ERR_PARAM_INVALID, "smooth_scale1 is given, so output_mask[0] must be true");
    if (has2 && !output_mask[1])
      return fail(ADQ_ERR_PARAM_INVALID, "smooth_scale2 is given, so output_mask[1] must be true");
    if (!output_mask[0] && !output_mask[1])
      return fail(ADQ_ERR_PARAM_INVALID, "output_mask[0] and output_mask[1] cannot both be false");
    act1 = output_mask[0];
    act2 = output_mask[1];
  } else {
    if (has2 && !has1)
      return fail(ADQ_ERR_PARAM_INVALID,
                  "without output_mask, smooth_scale2 needs smooth_scale1 as well");
    act1 = true;
    act2 = has1 && has2;
  }
  int q1 = adq::kQNone, q2 = adq::kQNone;
  if (act1 && (st = check_output(y1_out, scale1_out, "y1_out", "scale1_out", x1, &q1)) != ADQ_OK)
    return st;
  if (act2 && (st = check_output(y2_out, scale2_out, "y2_out", "scale2_out", x1, &q2)) != ADQ_OK)
    return st;
  {
    const adq_tensor* ins[] = {x1, x2, gamma, beta, smooth_scale1, smooth_scale2};
    const adq_tensor* outs[] = {x_out, act1 ? y1_out : nullptr, act1 ? scale1_out : nullptr,
                                act2 ? y2_out : nullptr, act2 ? scale2_out : nullptr};
    if ((st = check_no_overlap(ins, 6, outs, 5)) != ADQ_OK) return st;
  }

  adq_executor e{};
  e.op = kOpV2;
  e.m = numel(x1) / n;
  Args& a = e.args;
  a.x1 = x1->data;
  a.x2 = x2->data;
  a.gamma = gamma->data;
  a.beta = beta ? beta->data : nullptr;
  a.x_out = x_out->data;
  a.rows = e.m;
  a.n = (int32_t)n;
  a.eps = (float)epsilon;
  a.inv_n = (float)(1.0 / (double)n);
  // The kernels always produce slot 1 and optionally slot 2; a lone second
  // output (mask [false, true]) runs in slot 1 with the second smooth scale.
  if (act1) {
    a.smooth1 = has1 ? smooth_scale1->data : nullptr;
    a.y1 = y1_out->data;
    a.scale1 = static_cast<float*>(scale1_out->data);
    if (act2) {
      a.smooth2 = has2 ? smooth_scale2->data : nullptr;
      a.y2 = y2_out->data;
      a.scale2 = static_cast<float*>(scale2_out->data);
    }
    e.var = Variant{x1->dtype == ADQ_BF16 ? adq::kBF16 : adq::kF16, 2, q1, act2 ? q2 : adq::kQNone};
  } else {
    a.smooth1 = has2 ? smooth_scale2->data : nullptr;
    a.y1 = y2_out->data;
    a.scale1 = static_cast<float*>(scale2_out->data);
    e.var = Variant{x1->dtype == ADQ_BF16 ? adq::kBF16 : adq::kF16, 2, q2, adq::kQNone};
  }
  return finish_plan(&e, workspace_size, executor);
}

adq_status adq_add_rms_norm_dynamic_quant_v2(void* workspace, uint64_t workspace_size,
                                             adq_executor* executor, void* hip_stream) {
  return run(workspace, workspace_size, executor, hip_stream, kOpV2);
}

adq_status adq_add_rms_norm_dynamic_quant_v2_no_alloc(adq_executor* executor, void* hip_stream) {
  if (!executor) return fail(ADQ_ERR_NULLPTR, "executor is NULL");
  if (executor->op != kOpV2)
    return fail(ADQ_ERR_PARAM_INVALID, "executor was built for another operator");
  if (executor->ws_bytes > ADQ_STATIC_SCRATCH_BYTES)
    return fail(ADQ_ERR_WORKSPACE,
                "this call needs %llu bytes of scratch; the library's static buffer holds %u",
                (unsigned long long)executor->ws_bytes, (unsigned)ADQ_STATIC_SCRATCH_BYTES);
  void* scratch = nullptr;
  if (executor->ws_bytes > 0) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return fail(ADQ_ERR_RUNTIME, "no HIP device available");
    }
    if (cur != executor->device && hipSetDevice(executor->device) != hipSuccess) {
      (void)hipGetLastError();
      return fail(ADQ_ERR_RUNTIME, "cannot select device %d", executor->device);
    }
    const hipError_t err = adq::split_static_scratch(executor->device, &scratch);
    if (cur != executor->device) (void)hipSetDevice(cur);
    if (err != hipSuccess) {
      (void)hipGetLastError();
      return fail(ADQ_ERR_RUNTIME, "cannot find the static scratch buffer on device %d: %s",
                  executor->device, hipGetErrorString(err));
    }
  }
  return run(scratch, ADQ_STATIC_SCRATCH_BYTES, executor, hip_stream, kOpV2);
}

adq_status adq_rms_norm_dynamic_quant_get_workspace_size(
    const adq_tensor* x, const adq_tensor* gamma, const adq_tensor* beta,
    const adq_tensor* smooth_scales, double epsilon, const adq_tensor* y_out,
    const adq_tensor* scale_out, uint64_t* workspace_size, adq_executor** executor) {
  if (!workspace_size || !executor)
    return fail(ADQ_ERR_NULLPTR, "workspace_size and executor out-pointers are required");
  *executor = nullptr;
  *workspace_size = 0;
  if (!x || !gamma) return fail(ADQ_ERR_NULLPTR, "x and gamma are required");
  adq_status st;
  if ((st = check_tensor(x, "x")) != ADQ_OK) return st;
  if (!is_half(x->dtype))
    return fail(ADQ_ERR_UNSUPPORTED, "x: dtype %s; expected F16 or BF16", dtype_name(x->dtype));
  if (x->ndim < 1) return fail(ADQ_ERR_PARAM_INVALID, "x: needs at least one dimension");
  const int64_t n = x->shape[x->ndim - 1];
  if (n > INT32_MAX) return fail(ADQ_ERR_PARAM_INVALID, "last dimension too large");
  if ((st = check_param(gamma, "gamma", x->dtype, n)) != ADQ_OK) return st;
  if (beta && (st = check_param(beta, "beta", x->dtype, n)) != ADQ_OK) return st;
  if (smooth_scales && (st = check_param(smooth_scales, "smooth_scales", x->dtype, n)) != ADQ_OK)
    return st;
  if (!(epsilon == epsilon) || epsilon > 3.4e38 || epsilon < -3.4e38)
    return fail(ADQ_ERR_PARAM_INVALID, "epsilon must be a finite value");
  int q = adq::kQNone;
  if ((st = check_output(y_out, scale_out, "y_out", "scale_out", x, &q)) != ADQ_OK) return st;
  {
    const adq_tensor* ins[] = {x, gamma, beta, smooth_scales};
    const adq_tensor* outs[] = {y_out, scale_out};
    if ((st = check_no_overlap(ins, 4, outs, 2)) != ADQ_OK) return st;
  }

  adq_executor e{};
  e.op = kOpRmsNorm;
  e.m = numel(x) / n;
  Args& a = e.args;
  a.x1 = x->data;
  a.gamma = gamma->data;
  a.beta = beta ? beta->data : nullptr;
  a.smooth1 = smooth_scales ? smooth_scales->data : nullptr;
  a.y1 = y_out->data;
  a.scale1 = static_cast<float*>(scale_out->data);
  a.rows = e.m;
  a.n = (int32_t)n;
  a.eps = (float)epsilon;
  a.inv_n = (float)(1.0 / (double)n);
  e.var = Variant{x->dtype == ADQ_BF16 ? adq::kBF16 : adq::kF16, 1, q, adq::kQNone};
  return finish_plan(&e, workspace_size, executor);
}

adq_status adq_rms_norm_dynamic_quant(void* workspace, uint64_t workspace_size,
                                      adq_executor* executor, void* hip_stream) {
  return run(workspace, workspace_size, executor, hip_stream, kOpRmsNorm);
}

// 32-column tiles for few rows (the product is then bound by reading the
// weights, and larger tiles leave CUs idle); large tiles once there are
// enough of them to occupy every compute unit
constexpr int64_t kGemmSkinnyMaxRows = 128;
static int gemm_auto_tile(const adq_executor& e) {
  if (e.gemm.m <= kGemmSkinnyMaxRows) return adq::kGemmTileSkinny;
  const int64_t big = ((e.gemm.m + 255) / 256) * ((e.gemm.n + 255) / 256);
  return big >= e.cus ? adq::kGemmTile256 : adq::kGemmTile128;
}

adq_status adq_w8a8_gemm_get_workspace_size(const adq_tensor* a, const adq_tensor* a_scale,
                                            const adq_tensor* w, const adq_tensor* w_scale,
                                            const adq_tensor* bias, const adq_tensor* out,
                                            uint64_t* workspace_size, adq_executor** executor) {
  if (!workspace_size || !executor)
    return fail(ADQ_ERR_NULLPTR, "workspace_size and executor out-pointers are required");
  *executor = nullptr;
  *workspace_size = 0;
  if (!a || !a_scale || !w || !w_scale || !out)
    return fail(ADQ_ERR_NULLPTR, "a, a_scale, w, w_scale and out are required");
  adq_status st;
  if ((st = check_tensor(a, "a")) != ADQ_OK) return st;
  if ((st = check_tensor(w, "w")) != ADQ_OK) return st;
  if ((st = check_tensor(a_scale, "a_scale")) != ADQ_OK) return st;
  if ((st = check_tensor(w_scale, "w_scale")) != ADQ_OK) return st;
  if ((st = check_tensor(out, "out")) != ADQ_OK) return st;
  if (bias && (st = check_tensor(bias, "bias")) != ADQ_OK) return st;
  if (a->dtype != ADQ_INT8 || w->dtype != ADQ_INT8)
    return fail(ADQ_ERR_UNSUPPORTED, "a and w must be INT8");
  if (a_scale->dtype != ADQ_F32 || w_scale->dtype != ADQ_F32 || (bias && bias->dtype != ADQ_F32))
    return fail(ADQ_ERR_UNSUPPORTED, "a_scale, w_scale and bias must be F32");
  int out_type;
  if (out->dtype == ADQ_F32) out_type = adq::kGemmOutF32;
  else if (out->dtype == ADQ_BF16) out_type = adq::kGemmOutBF16;
  else if (out->dtype == ADQ_F16) out_type = adq::kGemmOutF16;
  else return fail(ADQ_ERR_UNSUPPORTED, "out must be F32, BF16 or F16");
  if (a->ndim < 1 || w->ndim != 2)
    return fail(ADQ_ERR_PARAM_INVALID, "a is [..., k] and w is [n, k]");
  const int64_t k = a->shape[a->ndim - 1];
  const int64_t m = numel(a) / k;
  const int64_t n = w->shape[0];
  if (w->shape[1] != k) return fail(ADQ_ERR_PARAM_INVALID, "w must be [n, k] with a's k");
  if (k % 16 != 0) return fail(ADQ_ERR_PARAM_INVALID, "k must be a multiple of 16");
  if (k > (1 << 17)) return fail(ADQ_ERR_PARAM_INVALID, "k above 131072 could overflow int32");
  if (n > (1 << 20)) return fail(ADQ_ERR_PARAM_INVALID, "n above 1048576 is not supported");
  if (numel(a_scale) != m) return fail(ADQ_ERR_PARAM_INVALID, "a_scale needs one value per row");
  if (w_scale->ndim != 1 || w_scale->shape[0] != n)
    return fail(ADQ_ERR_PARAM_INVALID, "w_scale must be [n]");
  if (bias && (bias->ndim != 1 || bias->shape[0] != n))
    return fail(ADQ_ERR_PARAM_INVALID, "bias must be [n]");
  if (out->ndim != a->ndim) return fail(ADQ_ERR_PARAM_INVALID, "out must be [..., n]");
  for (int i = 0; i + 1 < a->ndim; ++i)
    if (out->shape[i] != a->shape[i])
      return fail(ADQ_ERR_PARAM_INVALID, "out's leading dimensions must match a's");
  if (out->shape[out->ndim - 1] != n) return fail(ADQ_ERR_PARAM_INVALID, "out must be [..., n]");
  if (!aligned(a->data, 16) || !aligned(w->data, 16))
    return fail(ADQ_ERR_PARAM_INVALID, "a and w must be 16-byte aligned");
  if (!aligned(a_scale->data, 4) || !aligned(w_scale->data, 4) ||
      (bias && !aligned(bias->data, 4)) || !aligned(out->data, out->dtype == ADQ_F32 ? 4 : 2))
    return fail(ADQ_ERR_PARAM_INVALID, "scales, bias and out must be aligned to their element size");
  adq_executor e{};
  e.op = kOpGemm;
  st = current_device(&e.device, &e.cus);
  if (st != ADQ_OK) return st;
  e.gemm.a = static_cast<const int8_t*>(a->data);
  e.gemm.a_scale = static_cast<const float*>(a_scale->data);
  e.gemm.w = static_cast<const int8_t*>(w->data);
  e.gemm.w_scale = static_cast<const float*>(w_scale->data);
  e.gemm.bias = bias ? static_cast<const float*>(bias->data) : nullptr;
  e.gemm.out = out->data;
  e.gemm.m = m;
  e.gemm.n = n;
  e.gemm.k = k;
  e.gemm.out_type = out_type;
  e.m = m;
  e.gemm_tile = gemm_auto_tile(e);
  adq_executor* ex = new (std::nothrow) adq_executor(e);
  if (!ex) return fail(ADQ_ERR_RUNTIME, "out of host memory");
  *executor = ex;
  return ok();
}

adq_status adq_w8a8_gemm(void* workspace, uint64_t workspace_size, adq_executor* executor,
                         void* hip_stream) {
  return run(workspace, workspace_size, executor, hip_stream, kOpGemm);
}

// Shrink workgroups aimed at per two CUs when h1 is cut into slices (the
// slices are further capped so that all workgroups are resident at once);
// half as many at rank 128, where every slice adds 64 x 128 partial sums
// per tile that each expand workgroup of the tile reads.  Step time on 4096
// rows, h1 4096 -> h2 4096, 8 adapters (72 tiles), slices 3 / 4 / 6 / 8:
// rank 16 40.2 / 38.9 / 37.8 / 37.8 us, rank 64 56.2 / 56.6 / 55.4 / 57.8,
// rank 128 70.3 / 74.9 / 73.6 / 78.2 (3 slices: one workgroup per CU).
constexpr int64_t kShrinkWgPerTwoCus = 3;

adq_status adq_add_lora_get_workspace_size(const adq_tensor* y, const adq_tensor* x,
                                           const adq_tensor* weight_b,
                                           const adq_tensor* indices,
                                           const adq_tensor* weight_a, int64_t layer_idx,
                                           double scale, int64_t y_offset,
                                           int64_t y_slice_size, const adq_tensor* out,
                                           uint64_t* workspace_size, adq_executor** executor) {
  if (!workspace_size || !executor)
    return fail(ADQ_ERR_NULLPTR, "workspace_size and executor out-pointers are required");
  *executor = nullptr;
  *workspace_size = 0;
  if (!y || !x || !weight_b || !indices || !out)
    return fail(ADQ_ERR_NULLPTR, "y, x, weight_b, indices and out are required");
  adq_status st;
  if ((st = check_tensor(y, "y")) != ADQ_OK) return st;
  if ((st = check_tensor(x, "x")) != ADQ_OK) return st;
  if ((st = check_tensor(weight_b, "weight_b")) != ADQ_OK) return st;
  if ((st = check_tensor(indices, "indices")) != ADQ_OK) return st;
  if ((st = check_tensor(out, "out")) != ADQ_OK) return st;
  if (weight_a && (st = check_tensor(weight_a, "weight_a")) != ADQ_OK) return st;
  if (!is_half(y->dtype))
    return fail(ADQ_ERR_UNSUPPORTED, "y: dtype %s; expected F16 or BF16", dtype_name(y->dtype));
  if (x->dtype != y->dtype || weight_b->dtype != y->dtype || out->dtype != y->dtype ||
      (weight_a && weight_a->dtype != y->dtype))
    return fail(ADQ_ERR_PARAM_INVALID, "x, weight_a, weight_b and out must have y's dtype");
  if (indices->dtype != ADQ_INT32) return fail(ADQ_ERR_UNSUPPORTED, "indices must be INT32");
  if (y->ndim < 1 || x->ndim != y->ndim)
    return fail(ADQ_ERR_PARAM_INVALID, "x and y must have the same rank (>= 1)");
  for (int i = 0; i + 1 < y->ndim; ++i)
    if (x->shape[i] != y->shape[i])
      return fail(ADQ_ERR_PARAM_INVALID, "x and y must have the same leading dimensions");
  if (!same_shape(y, out)) return fail(ADQ_ERR_PARAM_INVALID, "out must have y's shape");
  const int64_t h3 = y->shape[y->ndim - 1];
  const int64_t h1 = x->shape[x->ndim - 1];
  const int64_t rows = numel(y) / h3;
  if (numel(indices) != rows)
    return fail(ADQ_ERR_PARAM_INVALID, "indices needs one value per row (%lld)", (long long)rows);
  if (weight_b->ndim != 4) return fail(ADQ_ERR_PARAM_INVALID, "weight_b must be [W, L, rank, h2]");
  const int64_t w = weight_b->shape[0], l = weight_b->shape[1];
  const int64_t rank = weight_b->shape[2], h2 = weight_b->shape[3];
  if (weight_a) {
    if (weight_a->ndim != 4 || weight_a->shape[0] != w || weight_a->shape[1] != l ||
        weight_a->shape[2] != h1 || weight_a->shape[3] != rank)
      return fail(ADQ_ERR_PARAM_INVALID, "weight_a must be [W, L, h1, rank] = [%lld, %lld, %lld, %lld]",
                  (long long)w, (long long)l, (long long)h1, (long long)rank);
  } else if (h1 != rank) {
    return fail(ADQ_ERR_PARAM_INVALID, "without weight_a, x's last dimension must equal rank");
  }
  if (y_slice_size != h2)
    return fail(ADQ_ERR_PARAM_INVALID, "y_slice_size must equal weight_b's last dimension");
  if (y_offset < 0 || y_offset + h2 > h3)
    return fail(ADQ_ERR_PARAM_INVALID, "the slice [y_offset, y_offset + y_slice_size) must lie in y's last dimension");
  if (layer_idx < 0 || layer_idx >= l)
    return fail(ADQ_ERR_PARAM_INVALID, "layer_idx outside [0, %lld)", (long long)l);
  if (!(scale == scale) || scale > 3.4e38 || scale < -3.4e38)
    return fail(ADQ_ERR_PARAM_INVALID, "scale must be a finite value");
  if (w > adq::kLoraMaxAdapters)
    return fail(ADQ_ERR_UNSUPPORTED, "at most %d adapters", adq::kLoraMaxAdapters);
  if (rank > adq::kLoraMaxRankGeneric)
    return fail(ADQ_ERR_UNSUPPORTED, "rank above %d", adq::kLoraMaxRankGeneric);
  if (rows > INT32_MAX) return fail(ADQ_ERR_UNSUPPORTED, "too many rows");
  if (!aligned(y->data, 2) || !aligned(x->data, 2) || !aligned(weight_b->data, 2) ||
      !aligned(out->data, 2) || !aligned(indices->data, 4) ||
      (weight_a && !aligned(weight_a->data, 2)))
    return fail(ADQ_ERR_PARAM_INVALID, "misaligned tensor");
  adq_executor e{};
  e.op = kOpLora;
  st = current_device(&e.device, &e.cus);
  if (st != ADQ_OK) return st;
  adq::LoraArgs& a = e.lora;
  a.y = y->data;
  a.x = x->data;
  a.wa = weight_a ? weight_a->data : nullptr;
  a.wb = weight_b->data;
  a.indices = static_cast<const int32_t*>(indices->data);
  a.out = out->data;
  a.rows = rows;
  a.h1 = h1;
  a.rank = rank;
  a.h2 = h2;
  a.h3 = h3;
  a.w = w;
  a.l = l;
  a.layer = layer_idx;
  a.y_offset = y_offset;
  a.scale = (float)scale;
  a.elem = y->dtype == ADQ_BF16 ? adq::kBF16 : adq::kF16;
  a.in_place = out->data == y->data;
  e.m = rows;
  // Rows per launch sequence of the tiled path: y and out ([rows, h3]) and
  // x ([rows, h1]) of one sequence stay below 4 GiB.
  const int64_t below4g = ((int64_t)1 << 32) - 1;
  int64_t chunk_rows = rows;
  if (chunk_rows > below4g / (h3 * 2)) chunk_rows = below4g / (h3 * 2);
  if (weight_a && chunk_rows > below4g / (h1 * 2)) chunk_rows = below4g / (h1 * 2);
  if (chunk_rows < rows) chunk_rows -= chunk_rows % adq::kLoraTileRows;  // whole tiles
  e.lora_chunk_rows = chunk_rows;
  e.lora_tiled_ok = h1 % 8 == 0 &&
                    (rank == 8 || rank == 16 || rank == 32 || rank == 64 || rank == 128) &&
                    h2 % 4 == 0 && h3 % 8 == 0 && y_offset % 8 == 0 && aligned(x->data, 16) &&
                    (!weight_a || aligned(weight_a->data, 16)) && aligned(weight_b->data, 8) &&
                    aligned(y->data, 16) && aligned(out->data, 8) && chunk_rows >= 1 &&
                    rank * h2 * 2 < (int64_t)1 << 32 &&  // 32-bit offsets into weightB[g, layer]
                    h1 * rank * 2 < (int64_t)1 << 31;    // and into weightA[g, layer]
  {
    // Tiles are only known on the device (they depend on the index values);
    // estimate them as rows / 64 plus one partial tile per adapter in use.
    // Slices of h1 per tile (shrink) are chosen for the workgroups per CU
    // above, each slice at least 256 k; the expand takes ranges of 1024
    // columns of the slice.
    const int64_t est_tiles = (chunk_rows + adq::kLoraTileRows - 1) / adq::kLoraTileRows +
                              (w < chunk_rows ? w : chunk_rows);
    // ... but no more than fit on the chip at once (ranks whose shrink
    // holds fewer workgroups per CU would otherwise run a second round)
    const int64_t slots = kShrinkWgPerTwoCus * (int64_t)e.cus / (rank >= 128 ? 4 : 2);
    int64_t want = (slots + est_tiles - 1) / est_tiles;
    adq::LoraArgs part = a;
    part.rows = chunk_rows;
    const int64_t fit = (int64_t)adq::lora_shrink_blocks_per_cu(part) * e.cus / est_tiles;
    if (fit >= 1 && fit < want) want = fit;
    auto clamp = [](int64_t v, int64_t hi) { return (int)(v < 1 ? 1 : v > hi ? hi : v); };
    a.ksplit = clamp(want, h1 / 256 > 1 ? h1 / 256 : 1);
    a.chunks = adq::lora_expand_chunks(h2, rank);
  }
  e.path = e.lora_tiled_ok ? ADQ_PATH_AUTO : ADQ_PATH_GENERIC;
  e.ws_bytes = e.lora_tiled_ok ? adq::lora_workspace_bytes(lora_part(e, 0)) : 0;
  adq_executor* ex = new (std::nothrow) adq_executor(e);
  if (!ex) return fail(ADQ_ERR_RUNTIME, "out of host memory");
  *workspace_size = e.ws_bytes;
  *executor = ex;
  return ok();
}

adq_status adq_add_lora(void* workspace, uint64_t workspace_size, adq_executor* executor,
                        void* hip_stream) {
  return run(workspace, workspace_size, executor, hip_stream, kOpLora);
}

void adq_executor_destroy(adq_executor* executor) { delete executor; }

adq_status adq_executor_set_path(adq_executor* executor, int32_t path, uint64_t* workspace_size) {
  if (!executor || !workspace_size) return fail(ADQ_ERR_NULLPTR, "executor and workspace_size are required");
  if (executor->op == kOpGemm) {
    if (path == ADQ_PATH_AUTO) executor->gemm_tile = gemm_auto_tile(*executor);
    else if (path == ADQ_PATH_GEMM_TILE128) executor->gemm_tile = adq::kGemmTile128;
    else if (path == ADQ_PATH_GEMM_TILE256) executor->gemm_tile = adq::kGemmTile256;
    else if (path == ADQ_PATH_GEMM_TILE32) executor->gemm_tile = adq::kGemmTileSkinny;
    else return fail(ADQ_ERR_PARAM_INVALID, "a GEMM executor takes AUTO or a GEMM tile path");
    executor->path = path;
    *workspace_size = 0;
    return ok();
  }
  if (executor->op == kOpLora) {
    if (path == ADQ_PATH_AUTO) executor->path = executor->lora_tiled_ok ? ADQ_PATH_AUTO : ADQ_PATH_GENERIC;
    else if (path == ADQ_PATH_GENERIC) executor->path = ADQ_PATH_GENERIC;
    else return fail(ADQ_ERR_PARAM_INVALID, "an AddLora executor takes AUTO or GENERIC");
    executor->ws_bytes =
        executor->path == ADQ_PATH_GENERIC ? 0 : adq::lora_workspace_bytes(lora_part(*executor, 0));
    *workspace_size = executor->ws_bytes;
    return ok();
  }
  if (path == ADQ_PATH_GEMM_TILE128 || path == ADQ_PATH_GEMM_TILE256 ||
      path == ADQ_PATH_GEMM_TILE32)
    return fail(ADQ_ERR_PARAM_INVALID, "GEMM tile paths apply to GEMM executors only");
  adq_executor trial = *executor;
  adq_status st = plan(&trial, path);
  if (st != ADQ_OK) return st;
  *executor = trial;
  *workspace_size = trial.ws_bytes;
  return ok();
}

adq_status adq_executor_set_split(adq_executor* executor, const adq_split_config* config,
                                  uint64_t* workspace_size) {
  if (!executor || !config || !workspace_size)
    return fail(ADQ_ERR_NULLPTR, "executor, config and workspace_size are required");
  if (executor->op != kOpV2 && executor->op != kOpRmsNorm)
    return fail(ADQ_ERR_PARAM_INVALID, "split geometry applies to the operator's executors only");
  if (config->splits < 0 || config->launches < 0 || config->launches > 3)
    return fail(ADQ_ERR_PARAM_INVALID, "splits must be >= 0 and launches 0, 1, 2 or 3");
  if (config->launches == 1 && config->splits > 64)
    return fail(ADQ_ERR_PARAM_INVALID, "the one-launch form takes at most 64 chunks per row");
  adq_executor trial = *executor;
  trial.split_req = config->splits;
  trial.launch_req = config->launches;
  trial.spread = config->spread != 0;
  trial.wait_ticks = config->wait_us < 0 ? kSplitWaitTicksDefault
                     : config->wait_us > 1000000 ? 100000000u
                                                 : (uint32_t)config->wait_us * 100u;
  adq_status st = plan(&trial, ADQ_PATH_SPLIT);
  if (st != ADQ_OK) return st;
  if (config->splits > 0 && trial.splits != config->splits)
    return fail(ADQ_ERR_PARAM_INVALID, "%d chunks per row do not fit n = %d (nearest: %d)",
                config->splits, trial.args.n, trial.splits);
  *executor = trial;
  *workspace_size = trial.ws_bytes;
  return ok();
}

int32_t adq_executor_describe(const adq_executor* e, char* buf, uint64_t len) {
  if (!e) return -1;
  if (e->op == kOpLora) {
    if (buf && len > 0) {
      const adq::LoraArgs& a = e->lora;
      const adq::LoraArgs part = lora_part(*e, 0);
      const bool tiled = e->path != ADQ_PATH_GENERIC;
      snprintf(buf, (size_t)len,
               "path=%s rows=%lld h1=%lld rank=%lld h2=%lld h3=%lld adapters=%lld layers=%lld "
               "weight_a=%d in_place=%d ksplit=%d chunks=%d row_ranges=%lld tiles<=%lld "
               "workspace=%llu cus=%d kernels=%s",
               tiled ? "lora-tiled" : "lora-generic", (long long)a.rows, (long long)a.h1,
               (long long)a.rank, (long long)a.h2, (long long)a.h3, (long long)a.w,
               (long long)a.l, a.wa != nullptr, a.in_place, a.ksplit, a.chunks,
               tiled ? (long long)((a.rows + e->lora_chunk_rows - 1) / e->lora_chunk_rows) : 1LL,
               (long long)adq::lora_max_tiles(part), (unsigned long long)e->ws_bytes, e->cus,
               tiled ? adq::lora_tiled_kernels(part) : "generic");
    }
    return e->path;
  }
  if (e->op == kOpGemm) {
    if (buf && len > 0)
      snprintf(buf, (size_t)len, "path=gemm m=%lld n=%lld k=%lld tile=%d out=%d cus=%d",
               (long long)e->gemm.m, (long long)e->gemm.n, (long long)e->gemm.k,
               e->gemm_tile == adq::kGemmTile256 ? 256 : e->gemm_tile == adq::kGemmTileSkinny ? 32 : 128,
               e->gemm.out_type, e->cus);
    return e->path;
  }
  if (buf && len > 0) {
    static const char* names[] = {"auto", "row", "split", "generic"};
    snprintf(buf, (size_t)len,
             "path=%s elem=%s nin=%d q1=%d q2=%d rows=%lld n=%d vpt=%d block=%d grid=%d "
             "splits=%d launches=%d plain_launches=%d batch_rows=%lld spread=%d wait_us=%u "
             "store=%s workspace=%llu cus=%d",
             names[e->path & 3], e->var.elem == adq::kBF16 ? "bf16" : "fp16", e->var.nin,
             e->var.q1, e->var.q2, (long long)e->m, e->args.n, e->vpt, e->block, e->grid,
             e->splits, e->launches, e->plain_launches, (long long)e->batch_rows, e->spread,
             e->wait_ticks / 100u, e->write_through ? "sc1" : "nt",
             (unsigned long long)e->ws_bytes, e->cus);
  }
  return e->path;
}

const char* adq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
