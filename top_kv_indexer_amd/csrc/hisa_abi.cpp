// hisa_abi.cpp -- the C ABI of libhisa.so: argument checks, workspace layout
// and the kernel sequence of each call (declared in include/hisa.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "hisa.h"
#include "hisa_internal.h"

using hisa::KDims;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int launch_fail(hipError_t e, const char* what) {
  return fail(HISA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

constexpr long long kMaxElems = 1LL << 40;
constexpr int kMaxKeep = 1024;
constexpr int kMaxCandidates = 8192;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_sel(int op) { return op != HISA_OP_ATTENTION; }
bool is_att(int op) { return op == HISA_OP_ATTENTION || op == HISA_OP_DECODE_STEP; }

// Checks dims for `op` and fills the kernel-side description.
int make_kdims(int op, const hisa_dims* d, KDims* k) {
  if (!d) return fail(HISA_ERR_ARG, "dims is NULL");
  if (op < HISA_OP_BLOCK_SCORES || op > HISA_OP_DECODE_STEP) return fail(HISA_ERR_ARG, "unknown op %d", op);
  if (d->B < 1 || d->B > 65535) return fail(HISA_ERR_ARG, "B = %d must be in [1, 65535]", d->B);
  if (d->L < 1 || d->L > 524280) return fail(HISA_ERR_ARG, "L = %d must be in [1, 524280]", d->L);
  if (d->ratio < 1) return fail(HISA_ERR_ARG, "ratio = %d must be >= 1", d->ratio);
  if (d->window < 0) return fail(HISA_ERR_ARG, "window = %d must be >= 0", d->window);
  if (d->Np_cap < 1) return fail(HISA_ERR_ARG, "Np_cap = %d must be >= 1", d->Np_cap);
  // Every visible position must fit int32: t0 + L <= ratio * (Np_cap + 1).
  if ((long long)d->ratio * ((long long)d->Np_cap + 1) + d->L >= (1LL << 31))
    return fail(HISA_ERR_OVERFLOW, "ratio * (Np_cap + 1) + L overflows int32");
  KDims kd{};
  kd.B = d->B; kd.L = d->L; kd.ratio = d->ratio; kd.window = d->window; kd.topk = d->topk;
  kd.index_block = d->index_block; kd.index_keep = d->index_keep; kd.H_i = d->H_i; kd.D_i = d->D_i;
  kd.H = d->H; kd.Dk = d->Dk; kd.Dv = d->Dv; kd.Np_cap = d->Np_cap; kd.Wl_cap = d->Wl_cap; kd.kI = d->kI;
  kd.force_flat = d->mode == HISA_MODE_FORCE_FLAT;
  kd.force_dense = d->mode == HISA_MODE_FORCE_DENSE;
  kd.ratio_shift = (d->ratio > 0 && (d->ratio & (d->ratio - 1)) == 0) ? __builtin_ctz((unsigned)d->ratio) : -1;
  kd.force_path = -1;
  if (op == HISA_OP_DECODE_STEP) kd.kI = d->topk;  // the step attends to its own index row
  if (is_sel(op)) {
    if (d->idx_dtype != HISA_F32 && d->idx_dtype != HISA_BF16) return fail(HISA_ERR_DTYPE, "idx_dtype %d", d->idx_dtype);
    if (d->mode != HISA_MODE_AUTO && d->mode != HISA_MODE_FORCE_FLAT && d->mode != HISA_MODE_FORCE_DENSE)
      return fail(HISA_ERR_ARG, "mode = %d", d->mode);
    if (d->mode == HISA_MODE_FORCE_DENSE &&
        (op == HISA_OP_SELECT_DECODE || op == HISA_OP_SELECT_PREFILL || op == HISA_OP_SELECT_DECODE_CACHED ||
         op == HISA_OP_DECODE_STEP) &&
        d->topk < d->Np_cap)
      return fail(HISA_ERR_ARG, "HISA_MODE_FORCE_DENSE lists every pooled row: topk = %d must be >= Np_cap = %d",
                  d->topk, d->Np_cap);
    if (d->topk < 1) return fail(HISA_ERR_ARG, "topk = %d must be >= 1", d->topk);
    if (d->H_i < 1 || d->D_i < 1 || d->D_i > 1024) return fail(HISA_ERR_ARG, "H_i = %d, D_i = %d (need D_i in [1, 1024])", d->H_i, d->D_i);
    if (d->index_block < 0 || (d->index_block > 0 && 64 % d->index_block != 0))
      return fail(HISA_ERR_ARG, "index_block = %d must be 0 or a divisor of 64", d->index_block);
    if (d->index_keep < 1 || d->index_keep > kMaxKeep) return fail(HISA_ERR_ARG, "index_keep = %d must be in [1, %d]", d->index_keep, kMaxKeep);
    if ((long long)d->index_keep * d->index_block > kMaxCandidates)
      return fail(HISA_ERR_ARG, "index_keep * index_block = %lld exceeds %d", (long long)d->index_keep * d->index_block, kMaxCandidates);
    if (op == HISA_OP_BLOCK_SCORES && d->index_block == 0) return fail(HISA_ERR_ARG, "hisa_block_scores needs index_block > 0");
    if (op == HISA_OP_BLOCK_MEANS_UPDATE && d->index_block == 0)
      return fail(HISA_ERR_ARG, "hisa_block_means_update needs index_block > 0");
    if ((op == HISA_OP_SELECT_DECODE || op == HISA_OP_DECODE_STEP) && d->L != 1)
      return fail(HISA_ERR_ARG, "%s needs L == 1 (got %d)",
                  op == HISA_OP_SELECT_DECODE ? "hisa_select_decode" : "hisa_decode_step", d->L);
    if (op == HISA_OP_SELECT_DECODE_CACHED && (long long)d->B * d->L > 65535)
      return fail(HISA_ERR_ARG, "hisa_select_decode_cached takes at most 65535 query rows (B * L = %lld)",
                  (long long)d->B * d->L);
    const long long rows = (long long)d->B * d->L;
    if (rows * d->H_i * d->D_i > kMaxElems || (long long)d->B * d->Np_cap * d->D_i > kMaxElems ||
        rows * d->Np_cap > kMaxElems || rows * d->topk > kMaxElems)
      return fail(HISA_ERR_OVERFLOW, "selection tensors too large");
    if (d->idx_dtype == HISA_BF16 && d->D_i % 8 != 0) return fail(HISA_ERR_ARG, "bf16 keys need D_i %% 8 == 0");
    kd.nb_cap = d->index_block > 0 ? d->Np_cap / d->index_block : 0;
    kd.w_scale = (float)(1.0 / std::sqrt((double)d->H_i * (double)d->D_i));
    if (op == HISA_OP_SELECT_DECODE_CACHED && !kd.force_dense && !hisa::cached_decode_ok(kd, d->idx_dtype == HISA_BF16))
      return fail(HISA_ERR_ARG,
                  "hisa_select_decode_cached needs bf16 keys, H_i = 64, D_i = 128, index_block > 0, nb_cap <= 4096, "
                  "index_keep <= 64, topk <= index_block * index_keep <= 1024 and no forced flat scan");
  }
  if (is_att(op)) {
    if (d->attn_dtype != HISA_F32 && d->attn_dtype != HISA_BF16) return fail(HISA_ERR_DTYPE, "attn_dtype %d", d->attn_dtype);
    if (d->H < 1 || d->Dk < 1 || d->Dv < 1 || d->Dv > d->Dk) return fail(HISA_ERR_ARG, "H = %d, Dk = %d, Dv = %d (need 1 <= Dv <= Dk)", d->H, d->Dk, d->Dv);
    if (kd.kI < 0) return fail(HISA_ERR_ARG, "kI = %d must be >= 0", kd.kI);
    if (d->window > 0 && d->Wl_cap < 1) return fail(HISA_ERR_ARG, "Wl_cap = %d must be >= 1 when window > 0", d->Wl_cap);
    const long long rows = (long long)d->B * d->L;
    if (rows * d->H * d->Dk > kMaxElems || (long long)d->B * d->Np_cap * d->Dk > kMaxElems ||
        (long long)d->B * d->Wl_cap * d->Dk > kMaxElems || rows * kd.kI > kMaxElems)
      return fail(HISA_ERR_OVERFLOW, "attention tensors too large");
    if (rows > 2147483647LL) return fail(HISA_ERR_OVERFLOW, "B * L overflows the grid");
    kd.attn_scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d->Dk));
    const bool bf = d->attn_dtype == HISA_BF16;
    if (!hisa::attn_mfma_ok(kd, bf) && !hisa::attn_generic_ok(kd))
      return fail(HISA_ERR_ARG, "shape not supported: Dk = %d, window + kI = %lld (generic path needs Dk <= 1024 and window + kI <= 4096)",
                  d->Dk, (long long)d->window + kd.kI);
  }
  *k = kd;
  return HISA_OK;
}

struct Layout {
  size_t total = 0;
  size_t rep = 0, rep3 = 0, cscore = 0, scores = 0, fscore = 0, partial = 0, cnt = 0, blk = 0;
  size_t sync = 0, sel = 0;  // decode step: its sync words, and the selection's part
  int splits = 1;
};

size_t take(Layout& l, size_t bytes) {
  const size_t off = l.total;
  l.total += align256(bytes);
  return off;
}

// Which kernels the batched selection runs (hisa_select_prefill); the
// workspace holds only what they use.
// Query rows (B * L) up to which a chunk takes the cached-means kernels (one
// query row per pair of grid rows, ~21 us for 1 to 32 rows, ~0.16 us more per
// row beyond) rather than the one-row-per-wave selection (~60 us up to a
// thousand rows: each wave's chain is the same length whatever the chunk).
constexpr int kSmallRows = 192;

struct PrefillPlan {
  bool small;        // short chunk: every block mean, then the cached-means selection per row
  bool rows;         // k_select_rows: one query row per wave (block means as bf16 parts)
  bool coarse_fine;  // the coarse-score GEMM, then one workgroup per row for top-Kb + fine + top-k
  bool flat_scan;    // flat scores of every row, then the row top-k (flat sequences)
};
PrefillPlan prefill_plan(const KDims& k, bool bf) {
  PrefillPlan p;
  p.small = (long long)k.B * k.L <= kSmallRows && hisa::cached_decode_ok(k, bf);
  if (p.small) {
    p.rows = p.coarse_fine = p.flat_scan = false;
    return p;
  }
  p.rows = k.nb_cap > 0 && hisa::select_rows_ok(k, bf);
  p.coarse_fine = k.nb_cap > 0 && !p.rows;
  // The row selection also takes the flat sequences when they are short: with
  // index_block * index_keep >= topk a flat sequence has Np below that product
  // (at most 1024 where the row selection runs).  Otherwise the flat scan runs.
  p.flat_scan = !(p.rows && !k.force_flat && (long long)k.index_block * k.index_keep >= k.topk);
  return p;
}

Layout layout(int op, const hisa_dims* d, const KDims& k) {
  Layout l;
  const size_t B = (size_t)d->B, L = (size_t)d->L;
  const bool bf = d->idx_dtype == HISA_BF16;
  const size_t nb_cap = (size_t)k.nb_cap;
  switch (op) {
    case HISA_OP_BLOCK_SCORES:
      l.rep = take(l, B * nb_cap * d->D_i * sizeof(float));
      l.rep3 = hisa::idx_mfma_ok(k, bf) ? take(l, 3 * B * nb_cap * d->D_i * sizeof(uint16_t)) : 0;
      break;
    case HISA_OP_SELECT_DECODE:
      if (k.force_dense) break;  // the dense fallback only fills I
      // arrival counters first: the region callers zero once (see hisa.h)
      l.cnt = take(l, hisa::decode_counter_ints(k) * sizeof(int));
      l.fscore = take(l, B * d->Np_cap * sizeof(float));
      l.cscore = take(l, B * std::max<size_t>(nb_cap, 1) * sizeof(float));
      break;
    case HISA_OP_SELECT_DECODE_CACHED:
      if (k.force_dense) break;
      l.cnt = take(l, hisa::cached_counter_ints(k) * sizeof(int));
      l.cscore = take(l, B * std::max<size_t>(nb_cap, 1) * sizeof(float));
      l.blk = take(l, B * (size_t)d->index_keep * sizeof(int));
      l.fscore = take(l, hisa::cached_fine_floats(k) * sizeof(float));
      break;
    case HISA_OP_BLOCK_MEANS_UPDATE:
      break;
    case HISA_OP_SELECT_PREFILL: {
      if (k.force_dense) break;
      const PrefillPlan p = prefill_plan(k, bf);
      if (p.small) {
        l.rep = take(l, B * nb_cap * d->D_i * sizeof(float));
        l.cnt = take(l, hisa::cached_counter_ints(k) * sizeof(int));
        l.cscore = take(l, B * L * nb_cap * sizeof(float));
        l.blk = take(l, B * L * (size_t)d->index_keep * sizeof(int));
        l.fscore = take(l, hisa::cached_fine_floats(k) * sizeof(float));
        break;
      }
      if (nb_cap > 0) {
        l.rep = take(l, B * nb_cap * d->D_i * sizeof(float));
        l.rep3 = hisa::idx_mfma_ok(k, bf) ? take(l, 3 * B * nb_cap * d->D_i * sizeof(uint16_t)) : 0;
      }
      if (p.coarse_fine) l.cscore = take(l, B * L * nb_cap * sizeof(float));
      if (p.flat_scan) l.scores = take(l, B * L * d->Np_cap * sizeof(float));
      break;
    }
    case HISA_OP_FLAT_TOPK:
      l.scores = take(l, B * L * d->Np_cap * sizeof(float));
      break;
    case HISA_OP_ATTENTION:
      l.splits = hisa::attn_splits(k, d->attn_dtype == HISA_BF16);
      l.partial = take(l, hisa::attn_partial_bytes(k, l.splits));
      break;
    case HISA_OP_DECODE_STEP: {
      // The sync words of the one-kernel step, then hisa_select_decode's
      // workspace (counters first), then room for either kind of partials:
      // the same offsets whichever way a call runs, so the words that must
      // rest at zero never share bytes with scratch data.
      l.sync = take(l, hisa::decode_step_sync_bytes(k));
      l.sel = l.total;
      if (!k.force_dense) {
        l.cnt = take(l, hisa::decode_counter_ints(k) * sizeof(int));
        l.fscore = take(l, B * d->Np_cap * sizeof(float));
        l.cscore = take(l, B * std::max<size_t>(nb_cap, 1) * sizeof(float));
      }
      l.partial = l.total;
      l.splits = hisa::attn_splits(k, d->attn_dtype == HISA_BF16);
      take(l, std::max(hisa::decode_step_partial_bytes(k), hisa::attn_partial_bytes(k, l.splits)));
      break;
    }
  }
  return l;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

int check_ws(const Layout& l, void* ws, size_t ws_bytes) {
  if (l.total > ws_bytes) return fail(HISA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, l.total);
  if (l.total > 0 && !ws) return fail(HISA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", l.total);
  if (ws && ((uintptr_t)ws & 255)) return fail(HISA_ERR_ARG, "workspace must be 256-byte aligned");
  return HISA_OK;
}

int check_ptrs(std::initializer_list<const void*> ptrs, const char* names) {
  for (const void* p : ptrs)
    if (!p) return fail(HISA_ERR_ARG, "NULL pointer among (%s)", names);
  return HISA_OK;
}

// ---- kernel timing (opt-in tracing aid) ----
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
struct ProfTotal {
  long long launches = 0;
  double ms = 0.0;
};
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_pending;
std::vector<hipEvent_t> g_prof_pool;
std::map<std::string, ProfTotal> g_prof_totals;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  // timing only: without the system-scope fence of a default event, whose
  // cache writeback and invalidation would be timed as part of the launch
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Runs one kernel launch, bracketed by events while timing is on.
template <class F>
hipError_t timed(const char* name, hipStream_t st, F launch) {
  if (!g_prof_on) return launch();
  ProfRecord r{name, prof_event(), prof_event()};
  bool ok = r.start && r.stop && hipEventRecord(r.start, st) == hipSuccess;
  const hipError_t e = launch();
  ok = ok && hipEventRecord(r.stop, st) == hipSuccess;
  if (ok) {
    g_prof_pending.push_back(r);
  } else {  // this launch goes untimed; the events go back to the pool
    if (r.start) g_prof_pool.push_back(r.start);
    if (r.stop) g_prof_pool.push_back(r.stop);
  }
  return e;
}

// ---- library-held workspace of hisa_select_decode_noalloc
//
// A file-scope device array, one copy per GPU, held until the process ends.
// Host code never uses its name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address reaches kernels.
constexpr size_t kScratchBytes = HISA_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (taken on its first use); checks that
// `st` (NULL: the current device's null stream) runs on the current device.
int scratch_of_current_device(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HISA_ERR_ARG, "device %d is past the %d supported", dev, kMaxDevices);
  if (st) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return launch_fail(e, "hipStreamGetDevice");
    if ((int)sdev != dev)
      return fail(HISA_ERR_ARG, "the stream runs on device %d but device %d is current", (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return launch_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(HISA_ERR_LAUNCH, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HISA_OK;
}

// Compute units of the device `st` runs on (NULL: the current device).
int device_cus(hipStream_t st, int* cus) {
  static std::mutex mu;
  static int cache[kMaxDevices] = {};
  int dev = -1;
  hipError_t e;
  if (st) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    dev = (int)sdev;
  } else {
    e = hipGetDevice(&dev);
  }
  if (e != hipSuccess) return launch_fail(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(HISA_ERR_ARG, "device %d is past the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    e = hipDeviceGetAttribute(&cache[dev], hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return launch_fail(e, "hipDeviceGetAttribute");
  }
  *cus = cache[dev];
  return HISA_OK;
}

int prepare(int op, const hisa_dims* d, KDims* k, Layout* l, void* ws, size_t ws_bytes) {
  int rc = make_kdims(op, d, k);
  if (rc) return rc;
  *l = layout(op, d, *k);
  return check_ws(*l, ws, ws_bytes);
}

int attention_call(const hisa_dims* d, const void* q, const void* local_kv, const void* pooled_kv, const int32_t* I,
                   const float* sinks, const int32_t* t0, const int32_t* ring_slot, bool ring, void* out, void* ws,
                   size_t ws_bytes, void* stream);

}  // namespace

extern "C" {

const char* hisa_last_error(void) { return g_err.c_str(); }

int hisa_abi_version(void) { return HISA_ABI_VERSION; }

size_t hisa_workspace_bytes(int op, const hisa_dims* d) {
  KDims k;
  if (make_kdims(op, d, &k)) return (size_t)-1;
  return layout(op, d, k).total;
}

int hisa_block_scores(const hisa_dims* d, const void* q_idx, const float* w, const void* keys, const int32_t* t0,
                      float* cscore_out, float* rep_out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  KDims k;
  Layout l;
  int rc = prepare(HISA_OP_BLOCK_SCORES, d, &k, &l, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_ptrs({q_idx, w, keys, t0, cscore_out}, "q_idx, w, keys, t0, cscore_out"))) return rc;
  const bool bf = d->idx_dtype == HISA_BF16;
  hipStream_t st = (hipStream_t)stream;
  float* rep = rep_out ? rep_out : at<float>(ws, l.rep);
  uint16_t* rep3 = hisa::idx_mfma_ok(k, bf) ? at<uint16_t>(ws, l.rep3) : nullptr;
  hipError_t e = timed("block_mean", st, [&] { return hisa::launch_block_mean(k, bf, true, keys, t0, rep, rep3, st); });
  if (e != hipSuccess) return launch_fail(e, "block mean");
  e = timed("coarse", st, [&] { return hisa::launch_coarse(k, bf, true, q_idx, w, rep, rep3, t0, cscore_out, st); });
  if (e != hipSuccess) return launch_fail(e, "coarse scores");
  return HISA_OK;
}

int hisa_select_decode(const hisa_dims* d, const void* q_idx, const float* w, const void* keys, const int32_t* t0,
                       int32_t* I_out, int32_t* top_blk_out, int32_t* path_out, void* ws, size_t ws_bytes,
                       void* stream) {
  g_err.clear();
  KDims k;
  Layout l;
  int rc = prepare(HISA_OP_SELECT_DECODE, d, &k, &l, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_ptrs({q_idx, w, keys, t0, I_out}, "q_idx, w, keys, t0, I_out"))) return rc;
  const bool bf = d->idx_dtype == HISA_BF16;
  hipStream_t st = (hipStream_t)stream;
  if (k.force_dense) {
    hipError_t e = timed("fill_dense", st, [&] { return hisa::launch_fill_dense(k, t0, I_out, top_blk_out, path_out, st); });
    return e == hipSuccess ? HISA_OK : launch_fail(e, "dense fallback");
  }
  float* fscore = at<float>(ws, l.fscore);
  float* cscore = at<float>(ws, l.cscore);
  if (hisa::decode_fused_ok(k, bf)) {
    int* cnt = at<int>(ws, l.cnt);
    hipError_t e = timed("decode_scan_select", st, [&] {
      return hisa::launch_decode_scan(k, bf, q_idx, w, keys, t0, fscore, cscore, cnt, I_out, top_blk_out, path_out, st);
    });
    if (e != hipSuccess) return launch_fail(e, "decode scan + select");
    return HISA_OK;
  }
  hipError_t e = timed("decode_scan", st, [&] {
    return hisa::launch_decode_scan(k, bf, q_idx, w, keys, t0, fscore, cscore, nullptr, nullptr, nullptr, nullptr, st);
  });
  if (e != hipSuccess) return launch_fail(e, "decode scan");
  e = timed("decode_select", st, [&] { return hisa::launch_decode_select(k, fscore, cscore, t0, I_out, top_blk_out, path_out, st); });
  if (e != hipSuccess) return launch_fail(e, "decode select");
  return HISA_OK;
}

int hisa_select_decode_cached(const hisa_dims* d, const void* q_idx, const float* w, const void* keys, float* rep,
                              const int32_t* t0, int32_t* I_out, int32_t* top_blk_out, int32_t* path_out, void* ws,
                              size_t ws_bytes, void* stream) {
  g_err.clear();
  KDims k;
  Layout l;
  int rc = prepare(HISA_OP_SELECT_DECODE_CACHED, d, &k, &l, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_ptrs({q_idx, w, keys, rep, t0, I_out}, "q_idx, w, keys, rep, t0, I_out"))) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (k.force_dense) {
    hipError_t e = timed("fill_dense", st, [&] { return hisa::launch_fill_dense(k, t0, I_out, top_blk_out, path_out, st); });
    return e == hipSuccess ? HISA_OK : launch_fail(e, "dense fallback");
  }
  hipError_t e = timed("cached_decode", st, [&] {
    return hisa::launch_cached_decode(k, q_idx, w, keys, rep, t0, at<float>(ws, l.cscore), at<int>(ws, l.blk),
                                      at<float>(ws, l.fscore), at<int>(ws, l.cnt), I_out, top_blk_out, path_out, st);
  });
  if (e != hipSuccess) return launch_fail(e, "cached decode selection");
  return HISA_OK;
}

int hisa_block_means_update(const hisa_dims* d, const void* keys, const int32_t* t0, float* rep, void* stream) {
  g_err.clear();
  KDims k;
  int rc = make_kdims(HISA_OP_BLOCK_MEANS_UPDATE, d, &k);
  if (rc) return rc;
  if ((rc = check_ptrs({keys, t0, rep}, "keys, t0, rep"))) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed("block_means_update", st, [&] {
    return hisa::launch_rep_update(k, d->idx_dtype == HISA_BF16, false, keys, t0, rep, nullptr, 0, st);
  });
  if (e != hipSuccess) return launch_fail(e, "block means update");
  return HISA_OK;
}

int hisa_select_decode_noalloc(const hisa_dims* d, const void* q_idx, const float* w, const void* keys,
                               const int32_t* t0, int32_t* I_out, int32_t* top_blk_out, int32_t* path_out,
                               void* stream) {
  g_err.clear();
  KDims k;
  int rc = make_kdims(HISA_OP_SELECT_DECODE, d, &k);
  if (rc) return rc;
  const Layout l = layout(HISA_OP_SELECT_DECODE, d, k);
  if (l.total > kScratchBytes)
    return fail(HISA_ERR_WORKSPACE, "hisa_select_decode_noalloc holds %zu bytes of workspace; these dims need %zu",
                kScratchBytes, l.total);
  if ((rc = check_ptrs({q_idx, w, keys, t0, I_out}, "q_idx, w, keys, t0, I_out"))) return rc;
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(st, &ws))) return rc;
  // The array keeps the previous call's contents (possibly scores laid out
  // for other dims): the arrival counters start from zero on every call.
  if (!k.force_dense) {
    hipError_t e = timed("zero_counters", st, [&] {
      return hisa::launch_zero_ints(at<int>(ws, l.cnt), hisa::decode_counter_ints(k), st);
    });
    if (e != hipSuccess) return launch_fail(e, "counter clear");
  }
  return hisa_select_decode(d, q_idx, w, keys, t0, I_out, top_blk_out, path_out, ws, kScratchBytes, stream);
}

int hisa_select_prefill(const hisa_dims* d, const void* q_idx, const float* w, const void* keys, const int32_t* t0,
                        int32_t* I_out, int32_t* top_blk_out, int32_t* path_out, void* ws, size_t ws_bytes,
                        void* stream) {
  g_err.clear();
  KDims k;
  Layout l;
  int rc = prepare(HISA_OP_SELECT_PREFILL, d, &k, &l, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_ptrs({q_idx, w, keys, t0, I_out}, "q_idx, w, keys, t0, I_out"))) return rc;
  const bool bf = d->idx_dtype == HISA_BF16;
  hipStream_t st = (hipStream_t)stream;
  if (k.force_dense) {
    hipError_t e = timed("fill_dense", st, [&] { return hisa::launch_fill_dense(k, t0, I_out, top_blk_out, path_out, st); });
    return e == hipSuccess ? HISA_OK : launch_fail(e, "dense fallback");
  }
  float* cscore = nullptr;
  hipError_t e;
  // one query row per wave when the blocks and candidates fit its registers
  const PrefillPlan plan = prefill_plan(k, bf);
  if (plan.small) {
    // a short chunk (multi-token verify): every complete block's mean into
    // the workspace (its first workgroup also zeroes the arrival counters),
    // then the cached-means selection of each query row
    float* rep = at<float>(ws, l.rep);
    int* cnt = at<int>(ws, l.cnt);
    hipError_t e = timed("block_mean", st, [&] {
      return hisa::launch_rep_update(k, bf, true, keys, t0, rep, cnt, hisa::cached_counter_ints(k), st);
    });
    if (e != hipSuccess) return launch_fail(e, "block means");
    e = timed("cached_decode", st, [&] {
      return hisa::launch_cached_decode(k, q_idx, w, keys, rep, t0, at<float>(ws, l.cscore), at<int>(ws, l.blk),
                                        at<float>(ws, l.fscore), cnt, I_out, top_blk_out, path_out, st);
    });
    if (e != hipSuccess) return launch_fail(e, "short-chunk selection");
    return HISA_OK;
  }
  const bool rows = plan.rows;
  if (k.nb_cap > 0) {
    float* rep = at<float>(ws, l.rep);
    uint16_t* rep3 = hisa::idx_mfma_ok(k, bf) ? at<uint16_t>(ws, l.rep3) : nullptr;
    cscore = plan.coarse_fine ? at<float>(ws, l.cscore) : nullptr;
    e = timed("block_mean", st, [&] { return hisa::launch_block_mean(k, bf, false, keys, t0, rep, rep3, st); });
    if (e != hipSuccess) return launch_fail(e, "block mean");
    if (rows) {
      e = timed("select_rows", st, [&] {
        return hisa::launch_select_rows(k, q_idx, w, keys, rep3, t0, I_out, top_blk_out, path_out, st);
      });
      if (e != hipSuccess) return launch_fail(e, "row selection");
    } else {
      e = timed("coarse", st, [&] { return hisa::launch_coarse(k, bf, false, q_idx, w, rep, rep3, t0, cscore, st); });
      if (e != hipSuccess) return launch_fail(e, "coarse scores");
    }
  }
  if (plan.flat_scan) {
    float* scores = at<float>(ws, l.scores);
    e = timed("flat_scores", st, [&] { return hisa::launch_flat_scores(k, bf, q_idx, w, keys, t0, scores, st); });
    if (e != hipSuccess) return launch_fail(e, "flat scores");
    e = timed("topk_rows", st, [&] { return hisa::launch_topk_rows(k, scores, t0, I_out, nullptr, st); });
    if (e != hipSuccess) return launch_fail(e, "flat top-k");
  }
  if (!rows) {
    e = timed("fine", st, [&] { return hisa::launch_fine(k, bf, q_idx, w, keys, cscore, t0, I_out, top_blk_out, path_out, st); });
    if (e != hipSuccess) return launch_fail(e, "fine selection");
  }
  return HISA_OK;
}

int flat_topk_select(const hisa_dims* d, const void* q_idx, const float* w, const void* keys, const int32_t* t0,
                     int32_t* I_out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  KDims k;
  Layout l;
  int rc = prepare(HISA_OP_FLAT_TOPK, d, &k, &l, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_ptrs({q_idx, w, keys, t0, I_out}, "q_idx, w, keys, t0, I_out"))) return rc;
  const bool bf = d->idx_dtype == HISA_BF16;
  hipStream_t st = (hipStream_t)stream;
  k.force_path = hisa::PATH_FLAT;
  float* scores = at<float>(ws, l.scores);
  hipError_t e;
  if (d->L == 1 && hisa::idx_mfma_ok(k, bf)) {
    // one query row per sequence: the decode key scan scores every row (its
    // per-sequence score rows are the (B, 1, Np_cap) layout of `scores`)
    e = timed("flat_scores", st, [&] {
      return hisa::launch_decode_scan(k, bf, q_idx, w, keys, t0, scores, nullptr, nullptr, nullptr, nullptr, nullptr, st);
    });
  } else {
    e = timed("flat_scores", st, [&] { return hisa::launch_flat_scores(k, bf, q_idx, w, keys, t0, scores, st); });
  }
  if (e != hipSuccess) return launch_fail(e, "flat scores");
  e = timed("topk_rows", st, [&] { return hisa::launch_topk_rows(k, scores, t0, I_out, nullptr, st); });
  if (e != hipSuccess) return launch_fail(e, "flat top-k");
  return HISA_OK;
}

int sparse_local_pooled_attention(const hisa_dims* d, const void* q, const void* local_kv, const void* pooled_kv,
                                  const int32_t* I, const float* sinks, const int32_t* t0, void* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  g_err.clear();
  return attention_call(d, q, local_kv, pooled_kv, I, sinks, t0, nullptr, false, out, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

int attention_call(const hisa_dims* d, const void* q, const void* local_kv, const void* pooled_kv, const int32_t* I,
                   const float* sinks, const int32_t* t0, const int32_t* ring_slot, bool ring, void* out, void* ws,
                   size_t ws_bytes, void* stream) {
  KDims k;
  Layout l;
  int rc = prepare(HISA_OP_ATTENTION, d, &k, &l, ws, ws_bytes);
  if (rc) return rc;
  k.local_ring = ring ? 1 : 0;
  k.ring_slot = ring ? ring_slot : nullptr;
  if ((rc = check_ptrs({q, pooled_kv, t0, out}, "q, pooled_kv, t0, out"))) return rc;
  if (d->window > 0 && !local_kv) return fail(HISA_ERR_ARG, "local_kv is NULL with window > 0");
  if (!I && d->kI != d->Np_cap)
    return fail(HISA_ERR_ARG, "I is NULL (every pooled row) but kI = %d is not Np_cap = %d", d->kI, d->Np_cap);
  const bool bf = d->attn_dtype == HISA_BF16;
  hipStream_t st = (hipStream_t)stream;
  float* partial = l.splits > 1 ? at<float>(ws, l.partial) : nullptr;
  hipError_t e = timed("attention", st, [&] {
    return hisa::launch_attention(k, bf, q, local_kv, pooled_kv, I, sinks, t0, out, partial, l.splits, st);
  });
  if (e == hipSuccess && l.splits > 1)
    e = timed("attention_merge", st, [&] { return hisa::launch_attention_merge(k, bf, partial, sinks, out, l.splits, st); });
  if (e != hipSuccess) return launch_fail(e, "attention");
  return HISA_OK;
}

}  // namespace

extern "C" {

int sparse_local_pooled_attention_ring(const hisa_dims* d, const void* q, const void* local_ring,
                                       const void* pooled_kv, const int32_t* I, const float* sinks,
                                       const int32_t* t0, const int32_t* ring_slot, void* out, void* ws,
                                       size_t ws_bytes, void* stream) {
  g_err.clear();
  if (d && d->window > 0 && (long long)d->Wl_cap < (long long)d->window + d->L - 1)
    return fail(HISA_ERR_ARG, "a ring of Wl_cap = %d slots cannot hold window + L - 1 = %lld positions", d->Wl_cap,
                (long long)d->window + d->L - 1);
  return attention_call(d, q, local_ring, pooled_kv, I, sinks, t0, ring_slot, true, out, ws, ws_bytes, stream);
}

int hisa_decode_step(const hisa_dims* d, const void* q_idx, const float* w, const void* keys, const void* q,
                     const void* local_kv, const void* pooled_kv, const float* sinks, const int32_t* t0,
                     int32_t* I_out, int32_t* top_blk_out, int32_t* path_out, void* out, void* ws, size_t ws_bytes,
                     void* stream) {
  g_err.clear();
  KDims k;
  Layout l;
  int rc = prepare(HISA_OP_DECODE_STEP, d, &k, &l, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_ptrs({q_idx, w, keys, q, pooled_kv, t0, I_out, out}, "q_idx, w, keys, q, pooled_kv, t0, I_out, out")))
    return rc;
  if (d->window > 0 && !local_kv) return fail(HISA_ERR_ARG, "local_kv is NULL with window > 0");
  hipStream_t st = (hipStream_t)stream;
  int cus = 0;
  if ((rc = device_cus(st, &cus))) return rc;
  if (!k.force_dense && hisa::decode_step_ok(k, d->idx_dtype == HISA_BF16, d->attn_dtype == HISA_BF16, cus)) {
    float* part = at<float>(ws, l.partial);
    hipError_t e = timed("decode_step", st, [&] {
      return hisa::launch_decode_step(k, q_idx, w, keys, t0, q, local_kv, pooled_kv, sinks, at<void>(ws, l.sync),
                                      at<int>(ws, l.cnt), at<float>(ws, l.fscore), at<float>(ws, l.cscore), part,
                                      I_out, top_blk_out, path_out, st);
    });
    if (e == hipSuccess)
      e = timed("attention_merge", st, [&] {
        return hisa::launch_attention_merge(k, true, part, sinks, out, hisa::decode_step_splits(k), st);
      });
    return e == hipSuccess ? HISA_OK : launch_fail(e, "decode step");
  }
  // the selection call, then the attention call on its index row
  rc = hisa_select_decode(d, q_idx, w, keys, t0, I_out, top_blk_out, path_out, at<void>(ws, l.sel),
                          l.partial - l.sel, stream);
  if (rc) return rc;
  hisa_dims da = *d;
  da.kI = d->topk;
  return attention_call(&da, q, local_kv, pooled_kv, I_out, sinks, t0, nullptr, false, out, at<void>(ws, l.partial),
                        l.total - l.partial, stream);
}

int hisa_profile_enable(int on) {
  if (!on) {
    for (auto& r : g_prof_pending) {
      (void)hipEventSynchronize(r.stop);  // drained only; the timings are discarded
      g_prof_pool.push_back(r.start);
      g_prof_pool.push_back(r.stop);
    }
    g_prof_pending.clear();
    g_prof_totals.clear();
  }
  g_prof_on = on != 0;
  return HISA_OK;
}

int hisa_profile_collect(hisa_kernel_time* out, int max_entries) {
  for (auto& r : g_prof_pending) {
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return launch_fail(e, "profile events");
    ProfTotal& t = g_prof_totals[r.name];
    t.launches += 1;
    t.ms += ms;
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_pending.clear();
  int i = 0;
  for (const auto& kv : g_prof_totals) {
    if (out && i < max_entries) {
      std::memset(out[i].name, 0, sizeof(out[i].name));
      std::strncpy(out[i].name, kv.first.c_str(), sizeof(out[i].name) - 1);
      out[i].launches = kv.second.launches;
      out[i].total_ms = kv.second.ms;
    }
    ++i;
  }
  return i;
}

}  // extern "C"
