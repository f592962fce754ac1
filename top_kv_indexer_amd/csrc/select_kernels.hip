// select_kernels.hip -- indexer scoring and top-k selection kernels for gfx950.
//
// Method (HiSA issue, lablup/mlxcel #549, sections "Flat selection", "HiSA decode
// path", "HiSA batched path"; DSA issue, lablup/mlxcel #509, item 1):
//   score(p) = sum_h relu(q[h] . key[p]) * w[h] * H_i^-1/2 * D_i^-1/2, in f32;
//   flat: top-k over the visible rows; HiSA: top-Kb blocks by the score of the
//   block mean, then the top-k rows inside those blocks.
//
// Kernels
//   decode scan   one pass over the pooled keys of an L == 1 step: every 64-row
//                 tile gets its rows' fine scores (MFMA) and its blocks' means
//                 and coarse scores; the decode step's HBM traffic is this pass.
//   decode select one workgroup per sequence: gate, coarse top-Kb, fine top-k.
//   block mean / coarse / fine   the batched (L > 1) path: block means once,
//                 coarse scores as a GEMM over (rows x heads) x blocks, then one
//                 workgroup per query row for coarse top-Kb + fine scores + top-k.
//   flat scores + topk rows      the flat scan for any L.
// The MFMA kernels serve bf16 keys with 64 heads x 128 dims (the V4-Flash and
// V3.2 indexer shapes); other shapes and f32 inputs take plain VALU kernels.
#include <algorithm>

#include "hisa_device.h"

namespace hisa {

namespace {


__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ bf16x8 ldg8(const uint16_t* p) { return *(const bf16x8*)p; }

// ------------------------------------------------------------------ in-wave top-k

// Top-k inside one wave on register-resident keys (element r of lane l has
// order index 64r + l, ascending in block id / pooled row): a bitwise search
// finds the k-th largest key, and ballots emit the winners in ascending
// order index, ties at the threshold going to the lowest indices.
constexpr int kRowR = 16;     // keys per lane: up to 1024 blocks or candidates
constexpr int kRowKeep = 64;  // retained blocks per row

// Threshold of the top k of the wave's keys in registers r < NR (absent
// entries carry key 0; 1 <= k <= number of present entries): returns the
// k-th largest key t and `ties`, the number of keys == t inside the top k
// (taken in order index).  Radix select, most significant byte first: per
// pass the keys that still match the known prefix are counted into a
// 256-bin histogram in LDS (hist: 256 words owned by this wave), and a wave
// prefix sum over the bins, largest first, finds the byte of the k-th key.
template <int NR>
__device__ __forceinline__ uint32_t wave_topk_threshold(const uint32_t (&key)[kRowR], int k, uint32_t* hist,
                                                        int& ties) {
  const int lane = lane_id();
  uint32_t prefix = 0, mask = 0;
  int remaining = k;  // keys still to take at or below the current prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    // one wave's LDS operations complete in program order: the clear lands
    // before the adds, the adds before the read
    *(uint4*)&hist[4 * lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t u = key[r];
      if (u != 0u && (u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    // lane l holds bins 255-4l (first) .. 252-4l
    const uint4 h = *(const uint4*)&hist[252 - 4 * lane];
    const uint32_t local = h.x + h.y + h.z + h.w;
    const uint32_t incl = wave_incl_scan(local);
    const uint32_t above = incl - local;  // keys in bins above this lane's
    const bool hit = above < (uint32_t)remaining && incl >= (uint32_t)remaining;
    const int src = __builtin_ctzll(__ballot(hit));
    uint32_t acc = above, digit = 252 - 4 * lane;
    if (acc + h.w >= (uint32_t)remaining) digit = 255 - 4 * lane;
    else if ((acc += h.w) + h.z >= (uint32_t)remaining) digit = 254 - 4 * lane;
    else if ((acc += h.z) + h.y >= (uint32_t)remaining) digit = 253 - 4 * lane;
    else acc += h.y;
    digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, src);
    acc = (uint32_t)__builtin_amdgcn_readlane((int)acc, src);
    remaining -= (int)acc;
    prefix |= digit << shift;
    mask |= 0xFFu << shift;
  }
  ties = remaining;
  return prefix;
}

// emits the k winners in ascending order index: emit(slot, r)
template <int NR, class EmitF>
__device__ __forceinline__ void wave_emit_topk_n(const uint32_t (&key)[kRowR], int k, uint32_t* hist, EmitF emit) {
  int ties;
  const uint32_t t = wave_topk_threshold<NR>(key, k, hist, ties);
  int base = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const bool eq = key[r] == t;
    const uint64_t meq = __ballot(eq);
    const bool take = key[r] > t || (eq && lanes_below(meq) < ties);
    ties -= min(ties, (int)__popcll(meq));
    const uint64_t mt = __ballot(take);
    if (take) emit(base + lanes_below(mt), r);
    base += (int)__popcll(mt);
  }
}

// the same for nr <= 16 registers in use (keys of registers >= nr are 0)
template <class EmitF>
__device__ __forceinline__ void wave_emit_topk(const uint32_t (&key)[kRowR], int nr, int k, uint32_t* hist,
                                               EmitF emit) {
  if (nr <= 4) wave_emit_topk_n<4>(key, k, hist, emit);
  else if (nr <= 8) wave_emit_topk_n<8>(key, k, hist, emit);
  else wave_emit_topk_n<kRowR>(key, k, hist, emit);
}

// ------------------------------------------------------------------ decode scan

// Selection outputs of a sequence that is not scored: I = 0..Np-1 (dense) or
// -1 (invalid t0), no retained blocks.
__device__ __forceinline__ void write_unscored(const KDims& d, const SeqInfo& si, int b, int* I, int* top_blk,
                                               int* path) {
  const int lane = lane_id();
  const bool dense = si.ok && si.path == PATH_DENSE;
  for (int i = lane; i < d.topk; i += 64) I[(size_t)b * d.topk + i] = (dense && i < si.Np) ? i : -1;
  if (top_blk)
    for (int i = lane; i < d.index_keep; i += 64) top_blk[(size_t)b * d.index_keep + i] = -1;
  if (path && lane == 0) path[b] = si.path;
}


// The same for query row `row` = b * L + j of a multi-row call (path by j == 0).
__device__ __forceinline__ void write_unscored_row(const KDims& d, const SeqInfo& si, int row, int j, int b, int* I,
                                                   int* top_blk, int* path) {
  const int lane = lane_id();
  const bool dense = si.ok && si.path == PATH_DENSE;
  for (int i = lane; i < d.topk; i += 64) I[(size_t)row * d.topk + i] = (dense && i < si.Np) ? i : -1;
  if (top_blk)
    for (int i = lane; i < d.index_keep; i += 64) top_blk[(size_t)row * d.index_keep + i] = -1;
  if (path && lane == 0 && j == 0) path[b] = si.path;
}

// ---- workgroup top-k (256 threads): thread t holds element 256 r + t in
// key[r], r < NR (order index = element index, ascending in id); key 0 marks
// an absent element.
struct WgTopkSmem {
  uint32_t hist[3][256];  // rotating histograms: one barrier per radix pass
  uint32_t red[2][4];     // per-wave min and max of the present keys
  uint32_t cnt[2][16][4];  // per register and wave: keys equal to the threshold, keys taken
};

__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  u32x2 p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(p.x, p.y);
  p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(p.x, p.y);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  u32x2 p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(p.x, p.y);
  p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(p.x, p.y);
}

// Threshold of the top k present keys (1 <= k <= present count): returns t
// and `ties` such that the top k are the keys > t and the first `ties` keys
// == t in order index (kAllTies: every key == t).  Radix select that starts at the highest bit where the
// present keys differ (above it they all agree, so no pass is spent on it)
// and stops as soon as the bin holding the k-th key is taken whole.  Every
// wave evaluates the same scan of the shared histogram, so the control flow
// is uniform over the workgroup.  Its barriers (and the emitter's) order
// LDS only: loads and stores the caller has in flight stay in flight.
constexpr int kAllTies = 0x7FFFFFFF;
template <int NR, int NK>
__device__ __forceinline__ uint32_t wg_topk_threshold(const uint32_t (&key)[NK], int k, WgTopkSmem& sm, int& ties) {
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int r = 0; r < NR; ++r)
    if (key[r] != 0u) {
      mn = min(mn, key[r]);
      mx = max(mx, key[r]);
    }
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if (lane == 0) {
    sm.red[0][wv] = mn;
    sm.red[1][wv] = mx;
  }
  sm.hist[0][tid] = 0u;
  sm.hist[1][tid] = 0u;
  lds_sync();
  mn = min(min(sm.red[0][0], sm.red[0][1]), min(sm.red[0][2], sm.red[0][3]));
  mx = max(max(sm.red[1][0], sm.red[1][1]), max(sm.red[1][2], sm.red[1][3]));
  if (mn == mx) {  // every present key is equal
    ties = k;
    return mx;
  }
  int top = 31 - __builtin_clz(mn ^ mx);  // highest bit still unknown
  uint32_t mask = top == 31 ? 0u : ~0u << (top + 1);
  uint32_t prefix = mx & mask;
  int remaining = k;  // keys still to take at or below the known prefix
#pragma unroll 1
  for (int pass = 0;; ++pass) {
    const int shift = max(top - 7, 0);
    uint32_t* h = sm.hist[pass % 3];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t u = key[r];
      if (u != 0u && (u & mask) == prefix) atomicAdd(&h[(u >> shift) & 255u], 1u);
    }
    lds_sync();
    // lane l holds bins 255-4l (first) .. 252-4l
    const uint4 hv = *(const uint4*)&h[252 - 4 * lane];
    // the buffer of pass + 2: every thread finished reading it (pass - 1)
    sm.hist[(pass + 2) % 3][tid] = 0u;
    const uint32_t local = hv.x + hv.y + hv.z + hv.w;
    const uint32_t incl = wave_incl_scan(local);
    const uint32_t above = incl - local;
    const bool hit = above < (uint32_t)remaining && incl >= (uint32_t)remaining;
    const int src = __builtin_ctzll(__ballot(hit));
    uint32_t acc = above, digit = 252 - 4 * lane, inbin = hv.x;
    if (acc + hv.w >= (uint32_t)remaining) { digit = 255 - 4 * lane; inbin = hv.w; }
    else if ((acc += hv.w) + hv.z >= (uint32_t)remaining) { digit = 254 - 4 * lane; inbin = hv.z; }
    else if ((acc += hv.z) + hv.y >= (uint32_t)remaining) { digit = 253 - 4 * lane; inbin = hv.y; }
    else acc += hv.y;
    digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, src);
    acc = (uint32_t)__builtin_amdgcn_readlane((int)acc, src);
    inbin = (uint32_t)__builtin_amdgcn_readlane((int)inbin, src);
    remaining -= (int)acc;
    prefix = (prefix & ~(255u << shift)) | (digit << shift);
    mask = ~0u << shift;
    if ((uint32_t)remaining == inbin) {  // the whole bin is taken: keys >= prefix
      ties = kAllTies;
      return prefix;
    }
    if (shift == 0) {  // fully resolved: t is the k-th key, shared by inbin keys
      ties = remaining;
      return prefix;
    }
    top = shift - 1;
  }
}

// No-op publication of the threshold (see wg_emit_topk_n).
struct NoPublish {
  __device__ void operator()(uint32_t, int) const {}
};

// emits the k winners in ascending order index: emit(slot, r).  Before any
// emission, pub(t, last) runs on exactly one thread: the winners are the keys
// > t and the keys == t whose order index is <= last (INT_MAX: all of them).
template <int NR, int NK, class EmitF, class PubF = NoPublish>
__device__ __forceinline__ void wg_emit_topk_n(const uint32_t (&key)[NK], int k, WgTopkSmem& sm, EmitF emit,
                                               PubF pub = PubF()) {
  const int lane = lane_id(), wv = wave_id();
  int ties;
  const uint32_t t = wg_topk_threshold<NR>(key, k, sm, ties);
  bool take[NR];
  if (ties == kAllTies) {
#pragma unroll
    for (int r = 0; r < NR; ++r) take[r] = key[r] != 0u && key[r] >= t;
    if (threadIdx.x == 0) pub(t, 0x7FFFFFFF);
  } else {
    // ranks of the keys == t: counts per register and wave first
    uint64_t meq[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      meq[r] = __ballot(key[r] != 0u && key[r] == t);
      if (lane == 0) sm.cnt[0][r][wv] = (uint32_t)__popcll(meq[r]);
    }
    lds_sync();
    int eq_base = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      int before = eq_base, tot = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = (int)sm.cnt[0][r][u];
        before += u < wv ? c : 0;
        tot += c;
      }
      const bool eq = key[r] != 0u && key[r] == t;
      const int rank = before + lanes_below(meq[r]);
      take[r] = key[r] > t || (eq && rank < ties);
      if (eq && rank == ties - 1) pub(t, 256 * r + (int)threadIdx.x);
      eq_base += tot;
    }
  }
  uint64_t mt[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    mt[r] = __ballot(take[r]);
    if (lane == 0) sm.cnt[1][r][wv] = (uint32_t)__popcll(mt[r]);
  }
  lds_sync();
  int base = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    int before = base, tot = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = (int)sm.cnt[1][r][u];
      before += u < wv ? c : 0;
      tot += c;
    }
    if (take[r]) emit(before + lanes_below(mt[r]), r);
    base += tot;
  }
}

// the same for n <= 1024 elements (keys of elements >= n are 0)
template <class EmitF, class PubF = NoPublish>
__device__ __forceinline__ void wg_emit_topk(const uint32_t (&key)[4], int n, int k, WgTopkSmem& sm, EmitF emit,
                                             PubF pub = PubF()) {
  if (n <= 256) wg_emit_topk_n<1>(key, k, sm, emit, pub);
  else if (n <= 512) wg_emit_topk_n<2>(key, k, sm, emit, pub);
  else wg_emit_topk_n<4>(key, k, sm, emit, pub);
}
// and for n <= 4096 elements, 16 keys per thread
template <class EmitF>
__device__ __forceinline__ void wg_emit_topk16(const uint32_t (&key)[16], int n, int k, WgTopkSmem& sm, EmitF emit) {
  if (n <= 1024) wg_emit_topk_n<4>(key, k, sm, emit);
  else if (n <= 2048) wg_emit_topk_n<8>(key, k, sm, emit);
  else wg_emit_topk_n<16>(key, k, sm, emit);
}

// Decode selection of sequence b by a whole workgroup (256 threads), from the
// scan's fine scores fs (Np entries) and block scores cs (nb entries): the
// flat top-k (Np <= 1024), or the coarse top-Kb blocks (nb <= 1024, Kb <= 64)
// and the fine top-k of their C = Kb*b <= 1024 rows (HiSA issue, HiSA decode
// path).  Ids come out ascending, padded with -1.  Every thread calls it.
struct DecodeSelSmem {
  WgTopkSmem tk;
  int blk[kRowKeep];
};
__device__ __forceinline__ void decode_select_wg(const KDims& d, const SeqInfo& si, int b, const float* fs,
                                                 const float* cs, int* I, int* top_blk, int* path,
                                                 DecodeSelSmem& sm) {
  const int tid = threadIdx.x;
  int* Ib = I + (size_t)b * d.topk;
  int* blkb = top_blk ? top_blk + (size_t)b * d.index_keep : nullptr;
  for (int i = si.k + tid; i < d.topk; i += 256) Ib[i] = -1;
  if (blkb)
    for (int i = tid; i < d.index_keep; i += 256)
      if (si.path != PATH_HISA || i >= si.Kb) blkb[i] = -1;
  if (path && tid == 0) path[b] = si.path;
  uint32_t key[4];
  float v[4];
  if (si.path == PATH_FLAT) {
    const int n = si.Np;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = ld_dev(fs + min(256 * r + tid, n - 1));
    __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first wait
#pragma unroll
    for (int r = 0; r < 4; ++r) key[r] = 256 * r + tid < n ? score_key(v[r]) : 0u;
    wg_emit_topk(key, n, si.k, sm.tk, [&](int slot, int r) { Ib[slot] = 256 * r + tid; });
    return;
  }
  const int nb = si.nb;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = ld_dev(cs + min(256 * r + tid, nb - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 4; ++r) key[r] = 256 * r + tid < nb ? score_key(v[r]) : 0u;
  wg_emit_topk(key, nb, si.Kb, sm.tk, [&](int slot, int r) { sm.blk[slot] = 256 * r + tid; });
  lds_sync();
  if (blkb && tid < si.Kb) blkb[tid] = sm.blk[tid];
  const int bsz = d.index_block, lbsz = __builtin_ctz(bsz);
  const int C = si.Kb * bsz;
  // candidate cc is row blk[cc / b] * b + cc % b: every position first (LDS
  // reads back to back), then every score load
  int pos[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int cc = min(256 * r + tid, C - 1);
    pos[r] = (sm.blk[cc >> lbsz] << lbsz) + (cc & (bsz - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = ld_dev(fs + pos[r]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 4; ++r) key[r] = 256 * r + tid < C ? score_key(v[r]) : 0u;
  wg_emit_topk(key, C, si.k, sm.tk, [&](int slot, int r) { Ib[slot] = pos[r]; });
}

// relu as one instruction (v_med3): max(x, 0) for finite x
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.402823466e38f); }

// ---- pieces shared by the two decode scan kernels (bf16, H_i = 64, D_i = 128,
// index_block | 64, four waves per workgroup).  Wave w scores rows 16w ..
// 16w+15 of a 64-row slab against all 64 heads: lane (g, c) holds row 16w + c
// and MFMA step s takes dims 32s + 8g .. +7, so each load instruction reads
// one 64-byte run per row.

// q of one query row (64 heads x 256 B) into LDS: wave w moves heads 16w ..
// 16w+15, four rows per instruction, 16-byte chunks XOR-swizzled by the row
// (slot p holds chunk p ^ (h & 15)) so the operand reads are conflict free.
__device__ __forceinline__ void issue_q_lds(const uint16_t* qrow, uint16_t* s_q) {
  const int lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = wv * 16 + 4 * i + g;
    g2lds16(qrow + h * 128 + ((c ^ (h & 15)) * 8), lds_addr(s_q + (wv * 16 + 4 * i) * 128));
  }
}
__device__ __forceinline__ void read_q_lds(const uint16_t* s_q, bf16x8 (&qf)[4][4]) {
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[ht][s] = lds8(s_q + (ht * 16 + c) * 128 + (((4 * s + g) ^ c) * 8));
}
// this wave's 16 rows of a slab (rows clamped to rmax)
__device__ __forceinline__ void load_slab_rows(const uint16_t* kb, int slab, int rmax, bf16x8 (&kf)[4]) {
  const int lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int r = min(slab * 64 + wv * 16 + c, rmax);
#pragma unroll
  for (int s = 0; s < 4; ++s) kf[s] = ldg8(kb + (size_t)r * 128 + s * 32 + g * 8);
}

// Scores of one slab of sequence b: fine scores of its rows and, on the HiSA
// path, coarse scores of its blocks (all four waves call it).  MFMA gives
// D[h][row] = q_h . key_row; the fine score of a row is sum_h relu(D) w_eff.
// The block mean is linear, so q_h . rep_beta is the mean of D[h][row] over
// the block's rows: blocks of up to 16 rows are summed inside the wave,
// larger ones from per-wave partial sums exchanged through s_part[par].
// Rows past Np are scored but never stored, as are blocks past nb.
__device__ __forceinline__ void score_slab(const KDims& d, const SeqInfo& si, int b, int slab, int par,
                                           const bf16x8 (&qf)[4][4], const float (&wl)[4][4], float w_head,
                                           const bf16x8 (&kf)[4], float* fscore, float* cscore,
                                           float (*s_part)[4][64]) {
  const int lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  f32x4 acc[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][s], kf[s], acc[ht], 0, 0, 0);
  float v = 0.f;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) v += relu(acc[ht][i]) * wl[ht][i];
  v = sum_rows(v);
  const int r = slab * 64 + wv * 16 + c;
  if (g == 0 && r < si.Np) st_dev(fscore + (size_t)b * d.Np_cap + r, v);
  if (si.path != PATH_HISA) return;
  const int bsz = d.index_block;
  const float inv_b = 1.f / (float)bsz;
  if (bsz <= 16) {
    // blocks inside the wave's 16 rows: lanes c of one block share the sum
    float cv = 0.f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) cv += relu(sum_span(acc[ht][i], bsz) * inv_b) * wl[ht][i];
    cv = sum_rows(cv);
    const int beta = r / bsz;
    if (g == 0 && (c & (bsz - 1)) == 0 && beta < si.nb) st_dev(cscore + (size_t)b * d.nb_cap + beta, cv);
    return;
  }
  // blocks of 32 or 64 rows: per-head sums over this wave's rows to LDS,
  // then wave j < 64 / bsz owns block j of the slab
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    f32x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = sum_row16(acc[ht][i]);
    if (c == 0) *(f32x4*)&s_part[par][wv][ht * 16 + 4 * g] = p;
  }
  lds_sync();
  const int wpb = bsz >> 4;  // waves per block
  if (wv < 64 / bsz) {
    float sum = 0.f;
    for (int u = 0; u < wpb; ++u) sum += s_part[par][wv * wpb + u][lane];
    const float cv = wave_sum(relu(sum * inv_b) * w_head);
    const int beta = (slab * 64) / bsz + wv;
    if (lane == 0 && beta < si.nb) st_dev(cscore + (size_t)b * d.nb_cap + beta, cv);
  }
}

// Adds n to a device-scope arrival counter that completes at `total`;
// returns whether this call completed it (and then returns it to 0).
__device__ __forceinline__ bool arrive(int* c, int n, int total) {
  const int prev = __hip_atomic_fetch_add(c, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (prev + n != total) return false;
  __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Once every wave has seen its device-scope score stores acknowledged (so
// they are visible to device-scope loads anywhere), thread 0 runs `count`
// and the workgroup learns its uniform result.
template <class CountF>
__device__ __forceinline__ bool publish(CountF count, int* s_flag) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
  asm volatile("" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = count();
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_flag) != 0;
}

// Counters of the latency-bound scan: one per group of kArriveGroup slabs
// and one per sequence that counts completed groups.  Atomics on one 64-byte
// line are performed one after another (~11 ns each), so every counter has a
// line of its own (kCntStride ints) and sees at most kArriveGroup (or
// slabs / kArriveGroup) of them.
constexpr int kArriveGroup = 16;

// Shared memory of the one-slab decode scan.
struct ScanSlabSmem {
  __align__(16) uint16_t s_q[64 * 128];
  __align__(16) float s_part[2][4][64];
  DecodeSelSmem sel;
  int flag;
};

// One 64-row slab of sequence b: its rows are requested before t0 arrives
// (rows clamped to the buffer rather than to Np) and q comes into LDS in
// parallel.  With cnt != NULL the selection is fused: select(si) runs in the
// workgroup that completes the last group of the sequence's slabs, and
// unscored(si) in wave 0 of slab 0 of a dense or invalid sequence.  ngmax:
// slab-group counters per sequence.
template <class UnscoredF, class SelectF>
__device__ __forceinline__ void decode_scan_slab(const KDims& d, int b, int slab, int ngmax,
                                                 const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                                                 const uint16_t* __restrict__ keys, const int* __restrict__ t0,
                                                 float* fscore, float* cscore, int* cnt, ScanSlabSmem& sm,
                                                 UnscoredF unscored, SelectF select) {
  const int lane = lane_id(), g = lane >> 4;
  const int t0b = t0[b];  // requested first, needed after the rows arrive
  const uint16_t* kb = keys + (size_t)b * d.Np_cap * 128;
  bf16x8 kf[4];
  load_slab_rows(kb, slab, d.Np_cap - 1, kf);
  issue_q_lds(q_idx + (size_t)b * d.L * 64 * 128, sm.s_q);
  // raw head weights now, scaled after the barrier (no wait on them here)
  const float* wrow = w + (size_t)b * d.L * 64;
  float wl[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[ht][i] = wrow[ht * 16 + 4 * g + i];
  float w_head = wrow[lane];  // weight of head `lane` (block owners)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's q rows (and its keys) are in
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[ht][i] *= d.w_scale;
  w_head *= d.w_scale;
  bf16x8 qf[4][4];
  read_q_lds(sm.s_q, qf);
  const SeqInfo si = seq_info(d, t0b);
  if (!si.ok || si.path == PATH_DENSE) {
    if (cnt && slab == 0 && wave_id() == 0) unscored(si);
    return;
  }
  const int nslab = (si.Np + 63) / 64;
  if (slab >= nslab) return;  // uniform over the workgroup
  score_slab(d, si, b, slab, 0, qf, wl, w_head, kf, fscore, cscore, sm.s_part);
  if (!cnt) return;
  // cnt: B sequence counters, then B x ngmax group counters, kCntStride apart
  const int grp = slab / kArriveGroup, ngrp = (nslab + kArriveGroup - 1) / kArriveGroup;
  const bool last = publish(
      [&] {
        const int members = min(kArriveGroup, nslab - grp * kArriveGroup);
        int* c_grp = cnt + (size_t)(d.B + (size_t)b * ngmax + grp) * kCntStride;
        return arrive(c_grp, 1, members) && arrive(cnt + (size_t)b * kCntStride, 1, ngrp);
      },
      &sm.flag);
  if (last) select(si);
}

// Latency-bound decode scan (few slabs): one workgroup per 64-row slab of one
// sequence (decode_scan_slab); the completing workgroup of a sequence selects.
__global__ __launch_bounds__(256) void k_decode_scan_mfma(
    KDims d, const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ keys,
    const int* __restrict__ t0, float* fscore, float* cscore, int* cnt, int* I, int* top_blk, int* path) {
  __shared__ ScanSlabSmem sm;
  args_now(d, q_idx, w, keys, t0, fscore, cscore, cnt, I, top_blk, path);
  const int b = blockIdx.y;
  decode_scan_slab(
      d, b, blockIdx.x, (gridDim.x + kArriveGroup - 1) / kArriveGroup, q_idx, w, keys, t0, fscore, cscore, cnt, sm,
      [&](const SeqInfo& si) { write_unscored(d, si, b, I, top_blk, path); },
      [&](const SeqInfo& si) {
        decode_select_wg(d, si, b, fscore + (size_t)b * d.Np_cap, cscore + (size_t)b * d.nb_cap, I, top_blk, path,
                         sm.sel);
      });
}

// ------------------------------------------------------------------ decode step

// A whole decode step of few sequences in one launch: the selection (HiSA
// issue, HiSA decode path) and the sparse combine (HiSA issue, Consuming
// the selection: sparse combine) over bf16 keys and a 512-wide KV.
// Workgroups [0, B * nslab) are the one-slab scan above, whose completing
// workgroup selects; the others attend, one per (sequence, group of 16
// heads, split of 64 list entries).  Pooled splits s < nps take entries
// 64s .. 64s+63 of the pooled list; the remaining splits take 64-position
// pieces of the local window.  The pooled list is the HiSA candidate list
// (kept blocks ascending, rows ascending inside each) masked by the fine
// selection, or the index row I itself (flat and dense sequences).  Hand-offs
// go through device-scope memory:
//   desc[b][s]  written once the coarse stage is done (or I is complete):
//               the kept block ids of split s plus one, 13 bits each from bit
//               2 (HiSA), "read I" (list) or "empty", in the low two bits;
//   thr[b]      the fine threshold: key t (low word) and one plus the
//               candidate index of the last tie taken (high word); candidate
//               cc is selected iff its key is > t, or == t with cc <= last.
// A pooled split gathers and scores its rows as soon as its descriptor is
// out, in parallel with the fine selection, and needs the threshold only
// for its softmax.  Each split writes the split attention's partial (O / l,
// m, l) with plain stores; the split attention's merge kernel runs
// next (hand-offs inside the kernel cost a device-scope round trip each, a
// kernel boundary less than the barrier and loads a merge here would need).
// Only attention workgroups wait; every wait is bounded (err is set when one
// gives up) and the host bounds the attention grid so that it fits on the
// device beside the scan.  Every word is back to zero when the kernel ends
// (the last reader clears it).
constexpr int kStepRows = 64;       // list entries per split
constexpr int kStepPP = 72;         // P^T pitch per head (bf16): two 32-entry k-steps, padded
constexpr int kStepMaxSplits = 24;  // splits per (sequence, head group)
constexpr int kSpinMax = 1 << 20;   // polls before a wait gives up
constexpr uint64_t kDescHisa = 1, kDescList = 2, kDescEmpty = 3;

struct StepSync {
  uint64_t* desc;  // B x nps
  uint64_t* thr;   // B, one 64-byte line each
  int* seen;       // B, kCntStride apart: pooled splits done with desc and thr
  int* err;        // 1 once a wait gave up
};

struct StepAttnSmem {
  __align__(1024) uint16_t kv[kStepRows * 512];  // the split's rows, 16-byte chunks XOR-swizzled by row
  __align__(16) uint16_t p[16 * kStepPP];        // P^T operand: head, k-step, 32 entries
  float red[2][4][16];                           // per-wave head max and head sum
  int code[kStepRows];                           // row of each entry: >= 0 pooled, < 0 local row -1-code
  uint32_t live[2];                              // entries that take part
  uint64_t word;                                 // a polled word, for the whole workgroup
};

union StepSmem {
  ScanSlabSmem scan;
  StepAttnSmem attn;
};

// Polls (one thread) until the word is nonzero; 0 with err set after
// kSpinMax polls.
__device__ __forceinline__ uint64_t poll_nonzero(const uint64_t* p, int* err) {
  for (int i = 0; i < kSpinMax; ++i) {
    const uint64_t v = ld_dev_u64(p);
    if (v) return v;
    __builtin_amdgcn_s_sleep(2);
  }
  st_dev_i(err, 1);
  return 0;
}

// Outputs of a dense or invalid sequence (wave 0 of its first slab), then
// "read I" to its pooled splits once every id is stored.
__device__ __forceinline__ void step_unscored(const KDims& d, const SeqInfo& si, int b, int nps, int* I,
                                              int* top_blk, int* path, const StepSync& sy) {
  const int lane = lane_id();
  const bool dense = si.ok && si.path == PATH_DENSE;
  for (int i = lane; i < d.topk; i += 64) st_dev_i(I + (size_t)b * d.topk + i, (dense && i < si.Np) ? i : -1);
  if (top_blk)
    for (int i = lane; i < d.index_keep; i += 64) top_blk[(size_t)b * d.index_keep + i] = -1;
  if (path && lane == 0) path[b] = si.path;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: the ids are stored
  for (int s = lane; s < nps; s += 64) st_dev_u64(sy.desc + (size_t)b * nps + s, kDescList);
}

// decode_select_wg with the hand-offs: descriptors after the coarse stage
// (or after I, on the flat path) and the fine threshold before the ids.
__device__ __forceinline__ void step_select_wg(const KDims& d, const SeqInfo& si, int b, int nps, const float* fs,
                                               const float* cs, int* I, int* top_blk, int* path, DecodeSelSmem& sm,
                                               const StepSync& sy) {
  const int tid = threadIdx.x;
  int* Ib = I + (size_t)b * d.topk;
  int* blkb = top_blk ? top_blk + (size_t)b * d.index_keep : nullptr;
  uint64_t* desc = sy.desc + (size_t)b * nps;
  for (int i = si.k + tid; i < d.topk; i += 256) st_dev_i(Ib + i, -1);
  if (blkb)
    for (int i = tid; i < d.index_keep; i += 256)
      if (si.path != PATH_HISA || i >= si.Kb) blkb[i] = -1;
  if (path && tid == 0) path[b] = si.path;
  uint32_t key[4];
  float v[4];
  if (si.path == PATH_FLAT) {
    const int n = si.Np;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = ld_dev(fs + min(256 * r + tid, n - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 4; ++r) key[r] = 256 * r + tid < n ? score_key(v[r]) : 0u;
    wg_emit_topk(key, n, si.k, sm.tk, [&](int slot, int r) { st_dev_i(Ib + slot, 256 * r + tid); });
    // every wave's ids (and pads) acknowledged before the readers are told
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int s = tid; s < nps; s += 256) st_dev_u64(desc + s, kDescList);
    return;
  }
  const int nb = si.nb;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = ld_dev(cs + min(256 * r + tid, nb - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 4; ++r) key[r] = 256 * r + tid < nb ? score_key(v[r]) : 0u;
  wg_emit_topk(key, nb, si.Kb, sm.tk, [&](int slot, int r) { sm.blk[slot] = 256 * r + tid; });
  lds_sync();
  if (blkb && tid < si.Kb) blkb[tid] = sm.blk[tid];
  const int bsz = d.index_block, lbsz = __builtin_ctz(bsz);
  {
    // split s holds kept blocks s*per .. s*per + per - 1
    const int per = 64 >> lbsz;
    for (int s = tid; s < nps; s += 256) {
      uint64_t dv = kDescHisa;
      for (int j = 0; j < per; ++j)
        if (s * per + j < si.Kb) dv |= (uint64_t)(sm.blk[s * per + j] + 1) << (2 + 13 * j);
      st_dev_u64(desc + s, s * per < si.Kb ? dv : kDescEmpty);
    }
  }
  const int C = si.Kb * bsz;
  int pos[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int cc = min(256 * r + tid, C - 1);
    pos[r] = (sm.blk[cc >> lbsz] << lbsz) + (cc & (bsz - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = ld_dev(fs + pos[r]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 4; ++r) key[r] = 256 * r + tid < C ? score_key(v[r]) : 0u;
  uint64_t* thr = sy.thr + (size_t)b * (kCntStride / 2);
  wg_emit_topk(
      key, C, si.k, sm.tk, [&](int slot, int r) { Ib[slot] = pos[r]; },
      [&](uint32_t t, int last) { st_dev_u64(thr, (uint64_t)t | ((uint64_t)(min(last, 0x7FFFFFFE) + 1) << 32)); });
}

// One attention split of the decode step (the workgroup's 256 threads): 16
// heads of sequence b against up to 64 rows.
// Wave w scores rows 16w .. 16w+15 (S = K q^T, 16x16x32 MFMA, lane (g, c)
// holding rows 16w + 4g + i of head c); the softmax takes the exact maximum
// over the split's rows; O^T += V^T P^T takes V^T from the transposing LDS
// read, wave w owning value tiles w, w+4, ...; the partial (O / l in bf16, m
// and l in the log2 domain) goes to part like the split attention's.
__device__ __forceinline__ void step_attn_wg(const KDims& d, int nps, int nspl, int aw, StepAttnSmem& sm,
                                             const uint16_t* __restrict__ q, const uint16_t* __restrict__ local_kv,
                                             const uint16_t* __restrict__ pooled_kv, const float* __restrict__ sinks,
                                             const int* __restrict__ t0, const float* fscore, const int* I,
                                             float* part, const StepSync& sy) {
  constexpr int DK = 512;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int ngrp = d.H >> 4;
  // workgroup aw takes head group hg of (sequence, split) pair p, with
  // aw = 8 ngrp (p / 8) + 8 hg + p % 8: the head groups of one split are 8
  // workgroups apart, so they are dealt to one XCD (round-robin over 8) and
  // three of the four gathers of its rows find them in that XCD's L2; pairs
  // past the last are padding
  const int sg = aw / (8 * ngrp), rem = aw - sg * (8 * ngrp);
  const int hg = rem >> 3, pair = 8 * sg + (rem & 7);
  if (pair >= d.B * nspl) return;
  const int split = pair % nspl, b = pair / nspl;
  const int hbase = hg * 16;
  const bool pooled = split < nps;
  // this group's q (the B operand of the scores), requested first
  bf16x8 qf[16];
  {
    const uint16_t* qrow = q + ((size_t)b * d.H + hbase + c) * DK + g * 8;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = *(const bf16x8*)(qrow + s * 32);
  }
  const int T0 = t0[b];
  const RowPlan rp = row_plan(d, T0, 0, 0);
  // a row every live split may read (dead entries point at it)
  const int dummy = rp.n_loc > 0 ? -1 - rp.lbase : 0;
  uint64_t desc = 0;
  if (pooled) {
    if (tid == 0) sm.word = poll_nonzero(sy.desc + (size_t)b * nps + split, sy.err);
    __syncthreads();
    desc = sm.word;
  }
  const int mode = (int)(desc & 3);
  // wave 0 resolves entry `lane`
  float fsv = 0.f;
  if (wv == 0) {
    int code = dummy;
    bool present = false;
    if (rp.ok) {
      if (!pooled) {
        const int e = kStepRows * (split - nps) + lane;
        if (e < rp.n_loc) {
          present = true;
          code = -1 - local_row(d, rp, e);
        }
      } else if (mode == (int)kDescList) {
        const int e = kStepRows * split + lane;
        const int id = e < d.topk ? ld_dev_i(I + (size_t)b * d.topk + e) : -1;
        if (id >= 0 && id < rp.V) {
          present = true;
          code = id;
        }
      } else if (mode == (int)kDescHisa) {
        const int lb = __builtin_ctz(d.index_block);
        const int fld = (int)((desc >> (2 + 13 * (lane >> lb))) & 0x1FFFu);
        if (fld > 0 && fld <= d.nb_cap) {  // (a block id plus one; the bound keeps every row inside keys)
          present = true;
          code = ((fld - 1) << lb) + (lane & (d.index_block - 1));
          fsv = ld_dev(fscore + (size_t)b * d.Np_cap + code);
        }
      }
    }
    sm.code[lane] = code;
    const uint64_t m = __ballot(present);
    if (lane == 0) {
      sm.live[0] = (uint32_t)m;
      sm.live[1] = (uint32_t)(m >> 32);
    }
  }
  // orders the codes only: q and the fine scores stay in flight (a full
  // barrier would hold every wave's gather until they land)
  lds_sync();
  const uint64_t present = ((uint64_t)sm.live[1] << 32) | sm.live[0];
  const bool any = present != 0;
  const uint32_t kv_lds = lds_addr(sm.kv);
  // chunk swizzle of 1 KiB rows (as in the split attention): 16 rows with
  // distinct (r mod 16) read one chunk each from distinct slots, with the
  // LDS hash of address bits 12 and 13 folded in
  const int kvb10 = (int)((kv_lds >> 10) & 15);
  auto sw = [kvb10](int r) {
    const int t = kvb10 + (r & 15);
    return (((r & 7) << 1) | ((r >> 3) & 1)) ^ (((t >> 2) ^ (t >> 3)) & 1);
  };
  f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (any) {
    // wave w brings rows 16w .. 16w+15 from HBM straight into LDS
    const uint16_t* pooled_b = pooled_kv + (size_t)b * d.Np_cap * DK;
    const uint16_t* local_b = local_kv + (size_t)b * d.Wl_cap * DK;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = 16 * wv + u;
      const int cd = sm.code[r];
      const uint16_t* src = cd >= 0 ? pooled_b + (size_t)cd * DK : local_b + (size_t)(-1 - cd) * DK;
      g2lds16(src + (lane ^ sw(r)) * 8, kv_lds + (uint32_t)(r * DK * 2));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's rows are in LDS
    const int rr = 16 * wv + c, rsw = sw(rr);
    bf16x8 ka[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) ka[s] = *(const bf16x8*)(sm.kv + rr * DK + (((4 * s + g) ^ rsw) * 8));
    f32x4 sa[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sa[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) sa[s & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qf[s], sa[s & 3], 0, 0, 0);
    sc = (sa[0] + sa[1]) + (sa[2] + sa[3]);
  }
  // the fine selection decides which candidates take part
  uint64_t live = present;
  if (pooled) {
    if (mode == (int)kDescHisa) {
      if (tid == 0) sm.word = poll_nonzero(sy.thr + (size_t)b * (kCntStride / 2), sy.err);
      __syncthreads();
      const uint64_t th = sm.word;
      if (wv == 0) {
        const uint32_t t = (uint32_t)th, kk = score_key(fsv);
        const int last = (int)(th >> 32) - 1, cc = kStepRows * split + lane;
        const bool sel = ((present >> lane) & 1) && th != 0 && (kk > t || (kk == t && cc <= last));
        const uint64_t m = __ballot(sel);
        if (lane == 0) {
          sm.live[0] = (uint32_t)m;
          sm.live[1] = (uint32_t)(m >> 32);
        }
      }
    }
    __syncthreads();
    live = ((uint64_t)sm.live[1] << 32) | sm.live[0];
  }
  // softmax of head c over the split's rows
  const float scale = d.attn_scale_log2;
  float x[4], mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wv + 4 * g + i;
    x[i] = ((live >> r) & 1) ? sc[i] * scale : -INFINITY;
    mx = fmaxf(mx, x[i]);
  }
  mx = max_rows(mx);
  if (g == 0) sm.red[0][wv][c] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(sm.red[0][0][c], sm.red[0][1][c]), fmaxf(sm.red[0][2][c], sm.red[0][3][c]));
  const float m_sub = m == -INFINITY ? 0.f : m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_sub);
  const float ps = sum_rows((p[0] + p[1]) + (p[2] + p[3]));
  if (g == 0) sm.red[1][wv][c] = ps;
  // P^T operand of k-step kk: entry 8g + e of head c is row 32kk + 16(e/4) +
  // 4g + e%4, i.e. waves 2kk and 2kk+1 give four entries each
  uint2 pk;
  pk.x = pack_bf16x2(p[0], p[1]);
  pk.y = pack_bf16x2(p[2], p[3]);
  *(uint2*)&sm.p[c * kStepPP + (wv >> 1) * 32 + 8 * g + 4 * (wv & 1)] = pk;
  __syncthreads();  // every wave's P, sums, and rows (each wave waited for its own)
  const float l = (sm.red[1][0][c] + sm.red[1][1][c]) + (sm.red[1][2][c] + sm.red[1][3][c]);
  f32x4 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (any) {
    // transposing V reads: lane (g, c) takes rows 4g + c/4 (+16) and
    // columns 4(c%4) .. +3 of a 16-column value tile
    const int vrow = 4 * g + (c >> 2), vsw = sw(vrow);
    const bf16x8 pb0 = *(const bf16x8*)&sm.p[c * kStepPP + 8 * g];
    const bf16x8 pb1 = *(const bf16x8*)&sm.p[c * kStepPP + 32 + 8 * g];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int dt = wv + 4 * n, ch = 2 * dt + ((c & 3) >> 1);
      const int off = vrow * DK + ((ch ^ vsw) * 8) + 4 * (c & 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint16_t* base = sm.kv + kk * 32 * DK + off;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * DK));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, kk ? pb1 : pb0, acc[n], 0, 0, 0);
      }
    }
  }
  // the split's partial: O^T tile (16dt + 4g + i, head c) per lane over l, then (m, l)
  const size_t prow = ((size_t)split * d.B + b) * d.H + hbase + c;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int n = 0; n < 8; ++n) store_part4(part, prow, DK, 16 * (wv + 4 * n) + 4 * g, acc[n], inv);
  if (wv == 0 && g == 0) store_part_ml(part, prow, DK, m, l);
  if (pooled && tid == 0) {
    // done with the sequence's descriptor and threshold: the last pooled
    // split of the sequence clears them
    int* sp = sy.seen + (size_t)b * kCntStride;
    if (__hip_atomic_fetch_add(sp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == ngrp * nps) {
      for (int s = 0; s < nps; ++s) st_dev_u64(sy.desc + (size_t)b * nps + s, 0);
      st_dev_u64(sy.thr + (size_t)b * (kCntStride / 2), 0);
      st_dev_i(sp, 0);
    }
  }
}

__global__ __launch_bounds__(256) void k_decode_step(KDims d, int nslab, int nps, int nspl,
                                                     const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                                                     const uint16_t* __restrict__ keys, const int* __restrict__ t0,
                                                     const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ local_kv,
                                                     const uint16_t* __restrict__ pooled_kv,
                                                     const float* __restrict__ sinks, float* fscore, float* cscore,
                                                     int* cnt, int* I, int* top_blk, int* path, float* part,
                                                     StepSync sy) {
  __shared__ StepSmem sm;
  const int x = blockIdx.x, nscan = d.B * nslab;
  if (x < nscan) {
    args_now(d, q_idx, w, keys, t0, fscore, cscore, cnt, I, top_blk, path);
    const int b = x / nslab;
    decode_scan_slab(
        d, b, x - b * nslab, (nslab + kArriveGroup - 1) / kArriveGroup, q_idx, w, keys, t0, fscore, cscore, cnt,
        sm.scan, [&](const SeqInfo& si) { step_unscored(d, si, b, nps, I, top_blk, path, sy); },
        [&](const SeqInfo& si) {
          step_select_wg(d, si, b, nps, fscore + (size_t)b * d.Np_cap, cscore + (size_t)b * d.nb_cap, I, top_blk,
                         path, sm.scan.sel, sy);
        });
    return;
  }
  step_attn_wg(d, nps, nspl, x - nscan, sm.attn, q, local_kv, pooled_kv, sinks, t0, fscore, I, part, sy);
}

// Bandwidth-bound decode scan (many slabs, ragged batches): a persistent
// grid over the flattened list of live slabs (every sequence's slabs below
// its Np, in order).  Each workgroup takes an equal contiguous share, so
// ragged pooled counts stay balanced and q is reloaded only where the share
// crosses into the next sequence; the rows of the next two slabs stream in
// while one is scored.  With cnt != NULL each run of a sequence's slabs is
// published with one atomic (publish, arrive), and the workgroup that completes
// a sequence selects for it.  Workgroup x writes the outputs of the dense or
// invalid sequences b with b % gridDim.x == x.  B <= kStreamMaxB.
constexpr int kStreamMaxB = 1024;

__global__ __launch_bounds__(256) void k_decode_scan_stream(
    KDims d, const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ keys,
    const int* __restrict__ t0, float* fscore, float* cscore, int* cnt, int* I, int* top_blk, int* path) {
  __shared__ __align__(16) uint16_t s_q[64 * 128];
  __shared__ __align__(16) float s_part[2][4][64];
  __shared__ int s_pre[kStreamMaxB + 1];  // first flattened slab of each sequence
  __shared__ int s_t0[kStreamMaxB];       // t0 of each sequence
  __shared__ uint32_t s_wsum[4];
  __shared__ DecodeSelSmem s_sel;
  __shared__ int s_flag;
  __shared__ int s_done[kStreamMaxB];  // sequences this workgroup completed
  args_now(d, q_idx, w, keys, t0, fscore, cscore, cnt, I, top_blk, path);
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4;
  // slab counts and their prefix: thread t sums sequences 4t .. 4t+3
  {
    int n[4];
    uint32_t loc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bb = 4 * tid + u;
      n[u] = 0;
      if (bb < d.B) {
        const int t0bb = t0[bb];
        s_t0[bb] = t0bb;
        const SeqInfo sb = seq_info(d, t0bb);
        if (sb.ok && sb.path != PATH_DENSE) n[u] = (sb.Np + 63) / 64;
      }
      loc += (uint32_t)n[u];
    }
    uint32_t total;
    uint32_t run = block_excl_scan<256>(loc, s_wsum, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bb = 4 * tid + u;
      if (bb < d.B) s_pre[bb] = (int)run;
      run += (uint32_t)n[u];
    }
    // the end of the last sequence (B may be 1024, past every thread's range)
    if (tid == 0) s_pre[d.B] = (int)total;
    __syncthreads();
  }
  // outputs of the sequences that are not scored
  if (cnt && wv == 0)
    for (int bb = blockIdx.x; bb < d.B; bb += gridDim.x) {
      const SeqInfo sb = seq_info(d, s_t0[bb]);
      if (!sb.ok || sb.path == PATH_DENSE) write_unscored(d, sb, bb, I, top_blk, path);
    }
  // the prefix and t0 tables are read into scalar registers: every branch
  // and loop below is then uniform over the wave, which keeps the waits for
  // in-flight slab rows exact
  auto pre = [&](int i) { return __builtin_amdgcn_readfirstlane(s_pre[i]); };
  auto t0_of = [&](int i) { return __builtin_amdgcn_readfirstlane(s_t0[i]); };
  const int total = pre(d.B);
  const int share = (total + (int)gridDim.x - 1) / (int)gridDim.x;
  const int g_begin = min(total, (int)blockIdx.x * share), g_end = min(total, g_begin + share);
  if (g_begin >= g_end) return;
  // sequence holding flattened slab x (x < total), given that it is `from`
  // or later: the last sequence whose first slab is <= x (empty sequences
  // share their first slab with the next one, so the last is non-empty)
  auto seq_of = [&](int x, int from) {
    if (pre(from + 1) > x) return from;
    int lo = from + 1, hi = d.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre(mid) <= x) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  bf16x8 qf[4][4];
  float wl[4][4], w_head = 0.f;
  int n_done = 0;
  auto enter = [&](int bb) {  // q and the head weights of sequence bb
    __syncthreads();  // every wave is done reading the previous q
    issue_q_lds(q_idx + (size_t)bb * d.L * 64 * 128, s_q);
    const float* wrow = w + (size_t)bb * d.L * 64;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) wl[ht][i] = wrow[ht * 16 + 4 * g + i];
    w_head = wrow[lane];
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0 (the slab rows in flight land too)
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) wl[ht][i] *= d.w_scale;
    w_head *= d.w_scale;
    read_q_lds(s_q, qf);
  };
  // runs: the slabs of one sequence inside the share
  for (int x0 = g_begin, b = seq_of(g_begin, 0);;) {
    const SeqInfo si = seq_info(d, t0_of(b));
    const int first = pre(b), x1 = min(g_end, pre(b + 1)), n = __builtin_amdgcn_readfirstlane(x1 - x0);
    const uint16_t* kb = keys + (size_t)b * d.Np_cap * 128;
    // slab i of the run; past the run's end its last slab is read again (a
    // cache hit), so every step issues the same loads and each wait for a
    // slab's rows leaves the two younger slabs in flight
    auto load = [&](int i, bf16x8(&kf)[4]) { load_slab_rows(kb, x0 + min(i, n - 1) - first, si.Np - 1, kf); };
    auto score = [&](int i, const bf16x8(&kf)[4]) {
      score_slab(d, si, b, x0 + i - first, (x0 + i) & 1, qf, wl, w_head, kf, fscore, cscore, s_part);
    };
    bf16x8 k0[4], k1[4], k2[4];
    load(0, k0);
    load(1, k1);
    enter(b);
    // the three buffers take turns by name (no register copies); the loop
    // body has no exit of its own (the last one or two slabs follow it), so
    // the waits inside it count the younger slabs exactly
    int i = 0;
    for (; i + 3 <= n; i += 3) {
      load(i + 2, k2);
      score(i, k0);
      load(i + 3, k0);
      score(i + 1, k1);
      load(i + 4, k1);
      score(i + 2, k2);
    }
    if (i < n) {
      load(i + 2, k2);
      score(i, k0);
      if (i + 1 < n) {
        load(i + 3, k0);
        score(i + 1, k1);
      }
    }
    if (cnt && publish([&] { return arrive(cnt + (size_t)b * kCntStride, n, pre(b + 1) - first); }, &s_flag)) {
      if (tid == 0) s_done[n_done] = b;
      ++n_done;
    }
    if (x1 >= g_end) break;
    x0 = x1;
    b = seq_of(x0, b + 1);
  }
  // selections of the sequences this workgroup completed (after the scan,
  // so its registers are free)
  if (n_done == 0) return;
  __syncthreads();
  for (int u = 0; u < n_done; ++u) {
    const int bd = s_done[u];
    decode_select_wg(d, seq_info(d, s_t0[bd]), bd, fscore + (size_t)bd * d.Np_cap, cscore + (size_t)bd * d.nb_cap, I,
                     top_blk, path, s_sel);
    __syncthreads();  // s_sel is reused by the next selection
  }
}

// Any shape / dtype: 4 threads per row, VALU dot products.
template <typename T>
__global__ __launch_bounds__(256) void k_decode_scan_valu(KDims d, const T* __restrict__ q_idx,
                                                          const float* __restrict__ w,
                                                          const T* __restrict__ keys,
                                                          const int* __restrict__ t0,
                                                          float* __restrict__ fscore,
                                                          float* __restrict__ cscore) {
  const int b = blockIdx.y;
  const int row0 = blockIdx.x * 64;
  const SeqInfo si = seq_info(d, t0[b]);
  if (!si.ok || si.path == PATH_DENSE || row0 >= si.Np) return;
  // pre-relu dots of the slab's rows, per head, for the block scores (heads <= 64)
  __shared__ float s_dot[64 * 64];
  __shared__ float s_rep[1024];
  __shared__ float s_red[4];
  const int tid = threadIdx.x, part = tid & 3, r = tid >> 2;
  const T* qb = q_idx + (size_t)b * d.L * d.H_i * d.D_i;
  const float* wb = w + (size_t)b * d.L * d.H_i;
  const int p = row0 + r;
  const bool live = p < si.Np;
  const T* kp = keys + ((size_t)b * d.Np_cap + (live ? p : row0)) * d.D_i;
  const bool keep_dots = si.path == PATH_HISA && d.H_i <= 64;
  float tot = 0.f;
  for (int h = 0; h < d.H_i; ++h) {
    float dot = 0.f;
#pragma unroll 8
    for (int e = part; e < d.D_i; e += 4) dot += ldf(qb + (size_t)h * d.D_i + e) * ldf(kp + e);
    dot = sum_span(dot, 4);
    if (keep_dots && part == 0) s_dot[h * 64 + r] = dot;
    tot += fmaxf(dot, 0.f) * (wb[h] * d.w_scale);
  }
  if (live && part == 0) fscore[(size_t)b * d.Np_cap + p] = tot;
  if (si.path != PATH_HISA) return;
  const int bsz = d.index_block;
  if (keep_dots) {
    // The block mean is linear: q_h . rep_beta is the mean of the block's row
    // dots, so each block score comes from the dots already in LDS.
    __syncthreads();
    const int blk = tid, beta = row0 / bsz + blk;
    if (blk < 64 / bsz && beta < si.nb) {
      const float inv_b = 1.f / (float)bsz;
      float cv = 0.f;
      for (int h = 0; h < d.H_i; ++h) {
        float sum = 0.f;
        for (int rr = 0; rr < bsz; ++rr) sum += s_dot[h * 64 + blk * bsz + rr];
        cv += fmaxf(sum * inv_b, 0.f) * (wb[h] * d.w_scale);
      }
      cscore[(size_t)b * d.nb_cap + beta] = cv;
    }
    return;
  }
  for (int blk = 0; blk < 64 / bsz; ++blk) {
    const int beta = row0 / bsz + blk;
    if (beta >= si.nb) break;
    for (int e = tid; e < d.D_i; e += 256) {
      float s = 0.f;
      for (int rr = 0; rr < bsz; ++rr) s += ldf(keys + ((size_t)b * d.Np_cap + (size_t)beta * bsz + rr) * d.D_i + e);
      s_rep[e] = s / (float)bsz;
    }
    __syncthreads();
    float contrib = 0.f;
    for (int h = tid; h < d.H_i; h += 256) {
      float dot = 0.f;
      for (int e = 0; e < d.D_i; ++e) dot += ldf(qb + (size_t)h * d.D_i + e) * s_rep[e];
      contrib += fmaxf(dot, 0.f) * (wb[h] * d.w_scale);
    }
    contrib = wave_sum(contrib);
    if (lane_id() == 0) s_red[wave_id()] = contrib;
    __syncthreads();
    if (tid == 0) cscore[(size_t)b * d.nb_cap + beta] = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  }
}

// ------------------------------------------------------------------ decode select

constexpr int kMaxKeep = 1024;
constexpr int kSelectThreads = 256;
constexpr int kSelectBins = 2048;
constexpr int kSelectLdsCap = 8192;    // keys staged in LDS per pass (32 KiB)

// Stages n scores into LDS (when they fit) and returns whether it did.
template <class SrcF>
__device__ __forceinline__ bool stage_scores(float* s_sc, int n, int cap, SrcF src) {
  if (n > cap) return false;
  for (int i = threadIdx.x; i < n; i += 4 * kSelectThreads) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ii = i + u * kSelectThreads;
      v[u] = ii < n ? src(ii) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ii = i + u * kSelectThreads;
      if (ii < n) s_sc[ii] = v[u];
    }
  }
  __syncthreads();
  return true;
}

template <class ScoreF, class EmitF>
__device__ __forceinline__ void select_topk(int n, int k, ScoreF score, EmitF emit, TopkScoresSmem& sm) {
  block_topk_scores<kSelectThreads, ScoreF, EmitF, kSelectBins>(n, k, score, emit, sm);
}

// One sequence per workgroup: gate, then the flat top-k or the coarse top-Kb
// + fine top-k, reading the scan's scores through LDS.
__global__ __launch_bounds__(kSelectThreads) void k_decode_select(KDims d, int lds_cap,
                                                                  const float* __restrict__ fscore,
                                                                  const float* __restrict__ cscore,
                                                                  const int* __restrict__ t0, int* __restrict__ I,
                                                                  int* __restrict__ top_blk, int* __restrict__ path) {
  constexpr int NT = kSelectThreads;
  const int b = blockIdx.x, tid = threadIdx.x;
  const SeqInfo si = seq_info(d, t0[b]);
  extern __shared__ float s_sc[];
  __shared__ TopkScoresSmem sm;
  __shared__ int s_blk[kMaxKeep];
  int* Ib = I + (size_t)b * d.topk;
  const bool dense = si.path == PATH_DENSE;
  const int first_pad = (si.ok && !dense) ? si.k : 0;
  for (int i = tid; i < d.topk; i += NT) {
    if (dense && i < si.Np) Ib[i] = i;
    else if (i >= first_pad) Ib[i] = -1;
  }
  if (top_blk)
    for (int i = tid; i < d.index_keep; i += NT) top_blk[(size_t)b * d.index_keep + i] = -1;
  if (path && tid == 0) path[b] = si.path;
  if (!si.ok || dense) return;
  const float* fs = fscore + (size_t)b * d.Np_cap;
  if (si.path == PATH_FLAT) {
    auto emit = [&](int slot, int i) { Ib[slot] = i; };
    if (stage_scores(s_sc, si.Np, lds_cap, [&](int i) { return fs[i]; }))
      select_topk(si.Np, si.k, [&](int i) { return s_sc[i]; }, emit, sm);
    else
      select_topk(si.Np, si.k, [&](int i) { return fs[i]; }, emit, sm);
    return;
  }
  const float* cs = cscore + (size_t)b * d.nb_cap;
  auto emit_blk = [&](int slot, int i) { s_blk[slot] = i; };
  if (stage_scores(s_sc, si.nb, lds_cap, [&](int i) { return cs[i]; }))
    select_topk(si.nb, si.Kb, [&](int i) { return s_sc[i]; }, emit_blk, sm);
  else
    select_topk(si.nb, si.Kb, [&](int i) { return cs[i]; }, emit_blk, sm);
  __syncthreads();
  if (top_blk)
    for (int i = tid; i < si.Kb; i += NT) top_blk[(size_t)b * d.index_keep + i] = s_blk[i];
  const int bsz = d.index_block;
  const int C = si.Kb * bsz;
  auto pos = [&](int c) { return s_blk[c / bsz] * bsz + c % bsz; };
  stage_scores(s_sc, C, lds_cap, [&](int c) { return fs[pos(c)]; });  // C <= keep * b <= the LDS cap
  select_topk(C, si.k, [&](int c) { return s_sc[c]; }, [&](int slot, int c) { Ib[slot] = pos(c); }, sm);
}

// ------------------------------------------------------------------ batched path

// Block means (f32) and their three-part bf16 split rep = hi + mid + lo, used by
// the MFMA coarse kernel (each part times a bf16 query is exact in f32).
template <typename T>
__global__ __launch_bounds__(128) void k_block_mean(KDims d, int all_paths, const T* __restrict__ keys,
                                                    const int* __restrict__ t0, float* __restrict__ rep,
                                                    uint16_t* __restrict__ rep3) {
  const int b = blockIdx.y, beta = blockIdx.x;
  const SeqInfo si = seq_info(d, t0[b]);
  if (!all_paths && si.path != PATH_HISA) return;
  const bool live = si.ok && beta < si.nb;
  const int bsz = d.index_block;
  const size_t plane = (size_t)d.B * d.nb_cap * d.D_i;
  for (int e = threadIdx.x; e < d.D_i; e += 128) {
    float s = 0.f;
    if (live) {
      const T* kp = keys + ((size_t)b * d.Np_cap + (size_t)beta * bsz) * d.D_i + e;
#pragma unroll 16
      for (int r = 0; r < bsz; ++r) s += ldf(kp + (size_t)r * d.D_i);
      s = s / (float)bsz;
    }
    const size_t o = ((size_t)b * d.nb_cap + beta) * d.D_i + e;
    rep[o] = s;
    if (rep3) {
      const uint16_t hi = f2bf(s);
      const float r1 = s - bf2f(hi);
      const uint16_t mid = f2bf(r1);
      const uint16_t lo = f2bf(r1 - bf2f(mid));
      rep3[o] = hi;
      rep3[plane + o] = mid;
      rep3[2 * plane + o] = lo;
    }
  }
}

// Coarse scores for 4 query rows per workgroup (one per wave), 16 blocks per
// MFMA column tile, rep taken as hi + mid + lo bf16 parts.
__global__ __launch_bounds__(256) void k_coarse_mfma(KDims d, int all_paths, const uint16_t* __restrict__ q_idx,
                                                     const float* __restrict__ w,
                                                     const uint16_t* __restrict__ rep3,
                                                     const int* __restrict__ t0,
                                                     float* __restrict__ cscore) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 4 + wave_id();
  const SeqInfo si = seq_info(d, t0[b]);
  if (!all_paths && si.path != PATH_HISA) return;
  if (j >= d.L) return;
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  float* out = cscore + ((size_t)b * d.L + j) * d.nb_cap;
  if (!si.ok) {
    for (int i = lane; i < d.nb_cap; i += 64) out[i] = kNeg;
    return;
  }
  const int valid = visible(d, t0[b] + j, si.Np);
  const uint16_t* qrow = q_idx + ((size_t)b * d.L + j) * 64 * 128;
  bf16x8 qf[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[ht][s] = ldg8(qrow + (ht * 16 + c) * 128 + s * 32 + g * 8);
  float wl[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[ht][i] = w[((size_t)b * d.L + j) * 64 + ht * 16 + 4 * g + i] * d.w_scale;
  const size_t plane = (size_t)d.B * d.nb_cap * 128;
  const int nt_live = (si.nb + 15) / 16;
  for (int nt = 0; nt * 16 < d.nb_cap; ++nt) {
    const int beta = nt * 16 + c;
    float v = kNeg;
    if (nt < nt_live) {
      const int bl = min(beta, d.nb_cap - 1);
      const uint16_t* rp = rep3 + ((size_t)b * d.nb_cap + bl) * 128 + g * 8;
      f32x4 acc[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 bf = ldg8(rp + part * plane + s * 32);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht)
            acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][s], bf, acc[ht], 0, 0, 0);
        }
      float x = 0.f;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) x += fmaxf(acc[ht][i], 0.f) * wl[ht][i];
      x = sum_rows(x);
      if (beta < si.nb && beta * d.index_block < valid) v = x;
    }
    if (g == 0 && beta < d.nb_cap) out[beta] = v;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_coarse_valu(KDims d, int all_paths, const T* __restrict__ q_idx,
                                                     const float* __restrict__ w, const float* __restrict__ rep,
                                                     const int* __restrict__ t0, float* __restrict__ cscore) {
  const int b = blockIdx.y, j = blockIdx.x;
  const SeqInfo si = seq_info(d, t0[b]);
  if (!all_paths && si.path != PATH_HISA) return;
  float* out = cscore + ((size_t)b * d.L + j) * d.nb_cap;
  const int valid = si.ok ? visible(d, t0[b] + j, si.Np) : 0;
  const T* qrow = q_idx + ((size_t)b * d.L + j) * d.H_i * d.D_i;
  const float* wrow = w + ((size_t)b * d.L + j) * d.H_i;
  for (int beta = threadIdx.x; beta < d.nb_cap; beta += 256) {
    float v = kNeg;
    if (si.ok && beta < si.nb && beta * d.index_block < valid) {
      const float* rp = rep + ((size_t)b * d.nb_cap + beta) * d.D_i;
      float tot = 0.f;
      for (int h = 0; h < d.H_i; ++h) {
        float dot = 0.f;
        for (int e = 0; e < d.D_i; ++e) dot += ldf(qrow + (size_t)h * d.D_i + e) * rp[e];
        tot += fmaxf(dot, 0.f) * (wrow[h] * d.w_scale);
      }
      v = tot;
    }
    out[beta] = v;
  }
}

// Shared prologue of the fine kernels: writes the dense / invalid rows and the
// padding; returns true when the row takes the HiSA path.
__device__ __forceinline__ bool fine_prologue(const KDims& d, const SeqInfo& si, int b, int j, int* Irow,
                                              int* blkrow, int* path) {
  const bool dense = si.path == PATH_DENSE;
  if (si.path == PATH_FLAT) {
    if (blkrow)
      for (int i = threadIdx.x; i < d.index_keep; i += blockDim.x) blkrow[i] = -1;
    if (path && j == 0 && threadIdx.x == 0) path[b] = si.path;
    return false;
  }
  const int first_pad = (si.ok && !dense) ? si.k : 0;
  for (int i = threadIdx.x; i < d.topk; i += blockDim.x) {
    if (dense && i < si.Np) Irow[i] = i;
    else if (i >= first_pad) Irow[i] = -1;
  }
  if (blkrow)
    for (int i = threadIdx.x; i < d.index_keep; i += blockDim.x) blkrow[i] = -1;
  if (path && j == 0 && threadIdx.x == 0) path[b] = si.path;
  return si.ok && si.path == PATH_HISA;
}

// One query row per workgroup: coarse top-Kb, fine scores of the C = Kb*b
// candidates on MFMA (keys gathered straight from HBM/L2), fine top-k.
__global__ __launch_bounds__(256) void k_fine_mfma(KDims d, int lds_floats, const uint16_t* __restrict__ q_idx,
                                                   const float* __restrict__ w, const uint16_t* __restrict__ keys,
                                                   const float* __restrict__ cscore, const int* __restrict__ t0,
                                                   int* __restrict__ I, int* __restrict__ top_blk,
                                                   int* __restrict__ path) {
  const int b = blockIdx.y, j = blockIdx.x;
  const SeqInfo si = seq_info(d, t0[b]);
  int* Irow = I + ((size_t)b * d.L + j) * d.topk;
  int* blkrow = top_blk ? top_blk + ((size_t)b * d.L + j) * d.index_keep : nullptr;
  if (!fine_prologue(d, si, b, j, Irow, blkrow, path)) return;
  extern __shared__ float s_fs[];  // max(nb_cap, C) floats: coarse scores, then fine scores
  __shared__ TopkScoresSmem sm;
  __shared__ int s_blk[kMaxKeep];
  const int valid = visible(d, t0[b] + j, si.Np);
  const float* cs = cscore + ((size_t)b * d.L + j) * d.nb_cap;
  auto emit_blk = [&](int slot, int i) { s_blk[slot] = i; };
  if (si.nb <= lds_floats) {
    for (int i = threadIdx.x; i < si.nb; i += 256) s_fs[i] = cs[i];
    __syncthreads();
    block_topk_scores<256>(si.nb, si.Kb, [&](int i) { return s_fs[i]; }, emit_blk, sm);
  } else {
    block_topk_scores<256>(si.nb, si.Kb, [&](int i) { return cs[i]; }, emit_blk, sm);
  }
  __syncthreads();
  if (blkrow)
    for (int i = threadIdx.x; i < si.Kb; i += 256) blkrow[i] = s_blk[i];

  const int lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  // q fragments with the contiguous-64-byte k order: lane group g holds dims
  // [32g, 32g + 32); MFMA step s takes dims 32g + 8s .. 32g + 8s + 7.
  const uint16_t* qrow = q_idx + ((size_t)b * d.L + j) * 64 * 128;
  bf16x8 qf[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[ht][s] = ldg8(qrow + (ht * 16 + c) * 128 + g * 32 + s * 8);
  float wl[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[ht][i] = w[((size_t)b * d.L + j) * 64 + ht * 16 + 4 * g + i] * d.w_scale;
  const int bsz = d.index_block;
  const int C = si.Kb * bsz;
  const uint16_t* kb = keys + (size_t)b * d.Np_cap * 128;
  // Candidate tiles of 16 rows; wave w scores tiles w, w+4, ... with the keys
  // of the next three of its tiles in flight (a ring of four register sets).
  auto cand = [&](int tile) {
    const int cc = min(tile * 16 + c, C - 1);
    return s_blk[cc / bsz] * bsz + cc % bsz;
  };
  // (unconditional: past the end it re-reads the last candidate, which keeps
  // the load count per iteration fixed for the compiler's wait placement)
  auto fetch = [&](int tile, bf16x8 (&kd)[4]) {
    const uint16_t* kp = kb + (size_t)cand(tile) * 128 + g * 32;
#pragma unroll
    for (int s = 0; s < 4; ++s) kd[s] = ldg8(kp + s * 8);
  };
  auto score = [&](int tile, const bf16x8 (&kf)[4]) {
    if (tile * 16 >= C) return;
    const int cidx = tile * 16 + c;
    const int pos = cand(tile);
    f32x4 acc[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][s], kf[s], acc[ht], 0, 0, 0);
    }
    float x = 0.f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) x += fmaxf(acc[ht][i], 0.f) * wl[ht][i];
    x = sum_rows(x);
    if (g == 0 && cidx < C) s_fs[cidx] = pos < valid ? x : kNeg;
  };
  __syncthreads();  // s_fs is reused for the fine scores below
  bf16x8 k0[4], k1[4], k2[4], k3[4];
  fetch(wv, k0);
  fetch(wv + 4, k1);
  fetch(wv + 8, k2);
  for (int tile = wv; tile * 16 < C; tile += 16) {
    fetch(tile + 12, k3);
    score(tile, k0);
    fetch(tile + 16, k0);
    score(tile + 4, k1);
    fetch(tile + 20, k1);
    score(tile + 8, k2);
    fetch(tile + 24, k2);
    score(tile + 12, k3);
  }
  __syncthreads();
  block_topk_scores<256>(C, si.k, [&](int cc) { return s_fs[cc]; },
                         [&](int slot, int cc) { Irow[slot] = s_blk[cc / bsz] * bsz + cc % bsz; }, sm);
}

template <typename T>
__global__ __launch_bounds__(256) void k_fine_valu(KDims d, const T* __restrict__ q_idx, const float* __restrict__ w,
                                                   const T* __restrict__ keys, const float* __restrict__ cscore,
                                                   const int* __restrict__ t0, int* __restrict__ I,
                                                   int* __restrict__ top_blk, int* __restrict__ path) {
  const int b = blockIdx.y, j = blockIdx.x;
  const SeqInfo si = seq_info(d, t0[b]);
  int* Irow = I + ((size_t)b * d.L + j) * d.topk;
  int* blkrow = top_blk ? top_blk + ((size_t)b * d.L + j) * d.index_keep : nullptr;
  if (!fine_prologue(d, si, b, j, Irow, blkrow, path)) return;
  extern __shared__ float s_fs[];
  __shared__ TopkScoresSmem sm;
  __shared__ int s_blk[kMaxKeep];
  const int valid = visible(d, t0[b] + j, si.Np);
  const float* cs = cscore + ((size_t)b * d.L + j) * d.nb_cap;
  block_topk_scores<256>(si.nb, si.Kb, [&](int i) { return cs[i]; },
                         [&](int slot, int i) { s_blk[slot] = i; }, sm);
  __syncthreads();
  if (blkrow)
    for (int i = threadIdx.x; i < si.Kb; i += 256) blkrow[i] = s_blk[i];
  const int bsz = d.index_block;
  const int C = si.Kb * bsz;
  const T* qrow = q_idx + ((size_t)b * d.L + j) * d.H_i * d.D_i;
  const float* wrow = w + ((size_t)b * d.L + j) * d.H_i;
  for (int cc = threadIdx.x; cc < C; cc += 256) {
    const int pos = s_blk[cc / bsz] * bsz + cc % bsz;
    const T* kp = keys + ((size_t)b * d.Np_cap + pos) * d.D_i;
    float tot = 0.f;
    for (int h = 0; h < d.H_i; ++h) {
      float dot = 0.f;
      for (int e = 0; e < d.D_i; ++e) dot += ldf(qrow + (size_t)h * d.D_i + e) * ldf(kp + e);
      tot += fmaxf(dot, 0.f) * (wrow[h] * d.w_scale);
    }
    s_fs[cc] = pos < valid ? tot : kNeg;
  }
  __syncthreads();
  block_topk_scores<256>(C, si.k, [&](int cc) { return s_fs[cc]; },
                         [&](int slot, int cc) { Irow[slot] = s_blk[cc / bsz] * bsz + cc % bsz; }, sm);
}

// ------------------------------------------------------------------ batched path, one row per wave

// The whole batched HiSA selection of one query row in one wave (bf16, 64
// indexer heads of dim 128, nb <= 1024 blocks, C = Kb*b <= 1024 candidates):
// coarse block scores on MFMA (rep as three bf16 parts), coarse top-Kb,
// fine scores of the C candidates on MFMA, fine top-k.  A workgroup holds
// four query rows of one sequence; the rep tiles stream through LDS once for
// all four waves (global->LDS loads two tiles ahead), each wave's candidate
// keys come straight into registers three tiles ahead.  Both top-k steps run
// inside the wave on register-resident keys (element r of lane l has order
// index 64r + l, which is ascending in block id / pooled row): a radix
// select finds the k-th largest key, and ballots emit the winners in
// ascending id order, ties at the threshold going to the lowest ids.
__global__ __launch_bounds__(256) void k_select_rows(KDims d, const uint16_t* __restrict__ q_idx,
                                                     const float* __restrict__ w, const uint16_t* __restrict__ keys,
                                                     const uint16_t* __restrict__ rep3, const int* __restrict__ t0,
                                                     int* __restrict__ I, int* __restrict__ top_blk,
                                                     int* __restrict__ path) {
  // The coarse stage streams a ring of three 16-block tiles of rep (three
  // bf16 parts each, shared by the four waves) through LDS.  Rows are 256
  // bytes with their 16-byte chunks XOR-swizzled by the row (slot position p
  // holds chunk p ^ row), so a 16-row MFMA operand read is bank-conflict free.
  constexpr int kRepTile = 3 * 16 * 128;  // elements
  __shared__ __align__(16) uint16_t s_ring[3 * kRepTile];
  __shared__ float s_sc[4][kRowR * 64];  // per wave: coarse, then fine scores
  __shared__ int s_blk[4][kRowKeep];
  __shared__ __align__(16) uint32_t s_hist[4][256];  // per wave: top-k histogram
  const int b = blockIdx.y, wv = wave_id(), j_raw = blockIdx.x * 4 + wv;
  const bool live = j_raw < d.L;  // trailing waves of the last workgroup only help with the shared loads
  const int j = live ? j_raw : d.L - 1;
  const int lane = lane_id(), g = lane >> 4, c = lane & 15;
  const SeqInfo si = seq_info(d, t0[b]);
  int* Irow = I + ((size_t)b * d.L + j) * d.topk;
  int* blkrow = top_blk ? top_blk + ((size_t)b * d.L + j) * d.index_keep : nullptr;
  // With index_block * index_keep >= topk (and at most 1024 here) a flat
  // sequence has Np < index_block * index_keep: its row takes every pooled
  // row as a candidate of the fine stage, without the coarse stage.
  // Otherwise flat rows belong to the flat scan.
  const bool flat_here = si.path == PATH_FLAT && !d.force_flat && d.index_block * d.index_keep >= d.topk;
  if (live) {
    if (path && j == 0 && lane == 0) path[b] = si.path;
    if (blkrow)
      for (int i = lane; i < d.index_keep; i += 64) blkrow[i] = -1;
    if (si.path != PATH_FLAT || flat_here) {
      const bool dense = si.path == PATH_DENSE;
      const int first_pad = (si.ok && !dense) ? si.k : 0;
      for (int i = lane; i < d.topk; i += 64) {
        if (dense && i < si.Np) Irow[i] = i;
        else if (i >= first_pad) Irow[i] = -1;
      }
    }
  }
  if (!si.ok || (si.path != PATH_HISA && !flat_here)) return;  // uniform over the workgroup (one sequence)
  const int valid = visible(d, t0[b] + j, si.Np);
  float* sc = s_sc[wv];

  // q as the A operand (MFMA step s: dims 32s + 8g .. +7), per-head weights
  const uint16_t* qrow = q_idx + ((size_t)b * d.L + j) * 64 * 128;
  bf16x8 qf[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[ht][s] = ldg8(qrow + (ht * 16 + c) * 128 + s * 32 + g * 8);
  float wl[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[ht][i] = w[((size_t)b * d.L + j) * 64 + ht * 16 + 4 * g + i] * d.w_scale;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // q and w are in: only tile loads count on vmcnt below
  auto head_sum = [&](const f32x4 (&acc)[4]) {
    float x = 0.f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) x += fmaxf(acc[ht][i], 0.f) * wl[ht][i];
    return sum_rows(x);
  };
  // B operand of a 16-row tile in LDS: row c, MFMA step s
  auto frag = [&](const uint16_t* rows, int s) {
    return *(const bf16x8*)(rows + c * 128 + ((4 * s + g) ^ c) * 8);
  };
  auto wait_vm = [&](bool keep_one_tile, int per_tile) {
    if (!keep_one_tile) __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (per_tile == 3) __builtin_amdgcn_s_waitcnt(0x0F73);
    else __builtin_amdgcn_s_waitcnt(0x0F74);
  };

  const int bsz = d.index_block, nb = si.nb;
  const int lbsz = __builtin_ctz(bsz);
  int* blk = s_blk[wv];
  uint32_t key[kRowR];
  if (!flat_here) {
    // ---- coarse scores of blocks 16nt + c (eligible iff the block's first row is visible)
    const size_t plane = (size_t)d.B * d.nb_cap * 128;
    const int ntc = (nb + 15) / 16;
    // tile nt: wave w moves parts/rows (i = w, w+4, w+8): part i/4, rows 4(i%4) .. +3
    auto load_rep = [&](int nt) {
      uint16_t* slot = s_ring + (nt % 3) * kRepTile;
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int i = wv + 4 * u, part = i >> 2, r = 4 * (i & 3) + (lane >> 4);
        const int beta = min(nt * 16 + r, d.nb_cap - 1);
        const uint16_t* src = rep3 + part * plane + ((size_t)b * d.nb_cap + beta) * 128 + (((lane & 15) ^ r) * 8);
        g2lds16(src, lds_addr(slot + part * 2048 + 4 * (i & 3) * 128));
      }
    };
    load_rep(0);
    if (ntc > 1) load_rep(1);
    for (int nt = 0; nt < ntc; ++nt) {
      wait_vm(nt + 1 < ntc, 3);
      lds_sync();  // every wave's share of tile nt has landed; slot (nt+2)%3 is free
      if (nt + 2 < ntc) load_rep(nt + 2);
      const uint16_t* slot = s_ring + (nt % 3) * kRepTile;
      f32x4 acc[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 bf = frag(slot + part * 2048, s);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht)
            acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][s], bf, acc[ht], 0, 0, 0);
        }
      const float x = head_sum(acc);
      const int beta = nt * 16 + c;
      if (g == 0 && beta < nb) sc[beta] = beta * bsz < valid ? x : kNeg;
    }
    __syncthreads();  // the rep ring is free for the key rings
    const int nrc = (nb + 63) / 64;
#pragma unroll
    for (int r = 0; r < kRowR; ++r) {
      const int i = 64 * r + lane;
      key[r] = (r < nrc && i < nb) ? score_key(sc[i]) : 0u;
    }
    wave_emit_topk(key, nrc, si.Kb, s_hist[wv], [&](int slot, int r) { blk[slot] = 64 * r + lane; });
    if (blkrow && live)
      for (int i = lane; i < si.Kb; i += 64) blkrow[i] = blk[i];
  }

  // ---- fine scores of the C candidates: candidate cc is row blk[cc / b]*b + cc % b
  const int C = flat_here ? si.Np : si.Kb * bsz;
  const int ntf = (C + 15) / 16;
  auto cand = [&](int cc) {
    cc = min(cc, C - 1);
    return flat_here ? cc : (blk[cc >> lbsz] << lbsz) + (cc & (bsz - 1));
  };
  // B operand of candidate tile t straight from memory into registers: lane
  // (g, c) takes row cand(16t + c), dims 32s + 8g .. +7 (the k order of q),
  // and keeps the row id for the causal mask.  Four register sets keep three
  // tiles of loads in flight; past the end the last candidate is re-read, so
  // every step issues the same loads.  The MFMAs of tile t go out before the
  // epilogue (relu, head weights, head sum) of tile t-1, so the matrix and
  // vector units overlap within the wave.
  const uint16_t* kb = keys + (size_t)b * d.Np_cap * 128 + g * 8;
  struct Tile {
    bf16x8 k[4];
    int pos;
  };
  auto fetch = [&](int t, Tile& tl) {
    tl.pos = cand(t * 16 + c);
    const uint16_t* kp = kb + (size_t)tl.pos * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) tl.k[s] = ldg8(kp + s * 32);
  };
  auto mma = [&](const Tile& tl, f32x4 (&acc)[4]) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][s], tl.k[s], acc[ht], 0, 0, 0);
  };
  auto epi = [&](int t, int pos, const f32x4 (&acc)[4]) {
    if (t < 0 || t >= ntf) return;
    float x = 0.f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) x += relu(acc[ht][i]) * wl[ht][i];
    x = sum_rows(x);
    const int cidx = t * 16 + c;
    if (g == 0 && cidx < C) sc[cidx] = pos < valid ? x : kNeg;
  };
  Tile k0, k1, k2, k3;
  f32x4 accA[4], accB[4];
  int posA = 0, posB = 0;
  fetch(0, k0);
  fetch(1, k1);
  fetch(2, k2);
  for (int t = 0; t < ntf; t += 4) {
    fetch(t + 3, k3);
    mma(k0, accA);
    posA = k0.pos;
    epi(t - 1, posB, accB);
    fetch(t + 4, k0);
    mma(k1, accB);
    posB = k1.pos;
    epi(t, posA, accA);
    fetch(t + 5, k1);
    mma(k2, accA);
    posA = k2.pos;
    epi(t + 1, posB, accB);
    fetch(t + 6, k2);
    mma(k3, accB);
    posB = k3.pos;
    epi(t + 2, posA, accA);
  }
  // the last tile of the last step (t + 3)
  epi(((ntf + 3) / 4) * 4 - 1, posB, accB);
  if (!live) return;
  const int nrf = (C + 63) / 64;
#pragma unroll
  for (int r = 0; r < kRowR; ++r) {
    const int i = 64 * r + lane;
    key[r] = (r < nrf && i < C) ? score_key(sc[i]) : 0u;
  }
  wave_emit_topk(key, nrf, si.k, s_hist[wv], [&](int slot, int r) { Irow[slot] = cand(64 * r + lane); });
}

// ------------------------------------------------------------------ flat scan

constexpr int kFlatTile = 128;  // key rows per LDS tile of the flat scoring

__device__ __forceinline__ bool flat_active(const KDims& d, const SeqInfo& si) {
  return si.ok && (d.force_path == PATH_FLAT || si.path == PATH_FLAT);
}

// Scores of 8 query rows (2 per wave) against a chunk of kc keys, streamed
// through LDS in 64-row tiles, double-buffered: the next tile's rows go
// global -> LDS (1 KiB = four rows per wave instruction) while the current one
// is scored.  Rows are dense (256 B) with 16-byte chunk p of row r holding
// chunk p ^ (r & 15), so the operand reads (16 rows x one chunk) are
// conflict free.  Masked entries (p >= V) are written as -1e30.
__global__ __launch_bounds__(256, 2) void k_flat_scores_mfma(KDims d, int kc, const uint16_t* __restrict__ q_idx,
                                                          const float* __restrict__ w,
                                                          const uint16_t* __restrict__ keys,
                                                          const int* __restrict__ t0,
                                                          float* __restrict__ scores) {
  const int b = blockIdx.z;
  const SeqInfo si = seq_info(d, t0[b]);
  if (!flat_active(d, si)) return;
  const int p_begin = blockIdx.x * kc;
  if (p_begin >= si.Np) return;
  const int p_end = min(si.Np, p_begin + kc);
  const int j0 = blockIdx.y * 8;
  const int lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int jlast = min(d.L - 1, j0 + 7);
  const int Vmax = visible(d, t0[b] + jlast, si.Np);
  const int p_stop = min(p_end, Vmax);  // tiles from here on are fully masked
  int jr[2], Vr[2];
  bool live[2];
  bf16x8 qf[2][4][4];
  float wl[2][4][4];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    jr[rr] = j0 + wv * 2 + rr;
    live[rr] = jr[rr] < d.L;
    const int jj = live[rr] ? jr[rr] : 0;
    Vr[rr] = live[rr] ? visible(d, t0[b] + jj, si.Np) : 0;
    const uint16_t* qrow = q_idx + ((size_t)b * d.L + jj) * 64 * 128;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[rr][ht][s] = ldg8(qrow + (ht * 16 + c) * 128 + s * 32 + g * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) wl[rr][ht][i] = w[((size_t)b * d.L + jj) * 64 + ht * 16 + 4 * g + i] * d.w_scale;
    }
  }
  constexpr int TK = kFlatTile;  // key rows per tile
  __shared__ __align__(16) uint16_t sk[2][TK * 128];
  const uint16_t* kb = keys + (size_t)b * d.Np_cap * 128;
  const uint32_t sk_lds = lds_addr(&sk[0][0]);
  // wave w moves rows (TK/4)w .. of a tile: instruction u covers 4 rows, lane
  // l row (TK/4)w+4u+l/16 at position l%16 (rows past the chunk end read a
  // valid row whose scores are never stored)
  auto load_tile = [&](int p0, int buf) {
#pragma unroll
    for (int u = 0; u < TK / 16; ++u) {
      const int r = (TK / 4) * wv + 4 * u + (lane >> 4);
      const int ch = (lane & 15) ^ (r & 15);
      const int pr = min(p0 + r, d.Np_cap - 1);
      g2lds16(kb + (size_t)pr * 128 + ch * 8, sk_lds + (uint32_t)(buf * TK * 256 + ((TK / 4) * wv + 4 * u) * 256));
    }
  };
  if (p_begin < p_stop) load_tile(p_begin, 0);
  float* srow[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) srow[rr] = scores + ((size_t)b * d.L + (live[rr] ? jr[rr] : 0)) * d.Np_cap;
  int buf = 0;
  for (int p0 = p_begin; p0 < p_end; p0 += TK, buf ^= 1) {
    const bool compute = p0 < p_stop;
    if (compute) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's rows of the tile
    __syncthreads();  // every wave's rows are in; the other buffer is free
    if (p0 + TK < p_stop) load_tile(p0 + TK, buf ^ 1);
    constexpr int NU = TK / 8;  // units: 16 keys x one row
    float x[2][TK / 64];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int q = 0; q < TK / 64; ++q) x[rr][q] = kNeg;
    if (compute) {
      // units u: keys 16*(u/2) .. +15 of the tile against row u%2; the MFMAs
      // of unit u+1 are issued before the epilogue of unit u, and the two rows
      // share each key fragment read from LDS
      const uint16_t* skb = sk[buf];
      bf16x8 kf[4];
      f32x4 acc[2][4];
      float sv[2][4];
      auto mma = [&](int u, f32x4(&a)[4]) {
        if ((u & 1) == 0) {
          const int r = (u >> 1) * 16 + c;
#pragma unroll
          for (int s = 0; s < 4; ++s) kf[s] = lds8(skb + r * 128 + (((4 * s + g) ^ c) * 8));
        }
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) a[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int ht = 0; ht < 4; ++ht)
            a[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[u & 1][ht][s], kf[s], a[ht], 0, 0, 0);
      };
      mma(0, acc[0]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (u + 1 < NU) mma(u + 1, acc[(u + 1) & 1]);
        float v = 0.f;
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i) v += relu(acc[u & 1][ht][i]) * wl[u & 1][ht][i];
        sv[u & 1][(u >> 1) & 3] = v;
        if ((u & 7) == 7) {
          // the four 16-key groups of keys 64q .. 64q+63 are in: sum over the
          // four lane rows of all of them at once, lane 16*g + c ending with
          // key 64q + 16*g + c of the tile
          const int q = u >> 3;
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            u32x2 a = __builtin_amdgcn_permlane32_swap(__float_as_uint(sv[rr][0]), __float_as_uint(sv[rr][2]), false,
                                                       false);
            const float s02 = __uint_as_float(a.x) + __uint_as_float(a.y);
            a = __builtin_amdgcn_permlane32_swap(__float_as_uint(sv[rr][1]), __float_as_uint(sv[rr][3]), false, false);
            const float s13 = __uint_as_float(a.x) + __uint_as_float(a.y);
            a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
            const float vq = __uint_as_float(a.x) + __uint_as_float(a.y);
            if (p0 + 64 * q + lane < Vr[rr]) x[rr][q] = vq;
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < TK / 64; ++q) {
      const int p = p0 + 64 * q + lane;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        if (live[rr] && p < p_end) srow[rr][p] = x[rr][q];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_flat_scores_valu(KDims d, const T* __restrict__ q_idx,
                                                          const float* __restrict__ w, const T* __restrict__ keys,
                                                          const int* __restrict__ t0, float* __restrict__ scores) {
  const int b = blockIdx.z, j = blockIdx.y;
  const SeqInfo si = seq_info(d, t0[b]);
  if (!flat_active(d, si)) return;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= si.Np) return;
  const int valid = visible(d, t0[b] + j, si.Np);
  float v = kNeg;
  if (p < valid) {
    const T* qrow = q_idx + ((size_t)b * d.L + j) * d.H_i * d.D_i;
    const float* wrow = w + ((size_t)b * d.L + j) * d.H_i;
    const T* kp = keys + ((size_t)b * d.Np_cap + p) * d.D_i;
    float tot = 0.f;
    for (int h = 0; h < d.H_i; ++h) {
      float dot = 0.f;
      for (int e = 0; e < d.D_i; ++e) dot += ldf(qrow + (size_t)h * d.D_i + e) * ldf(kp + e);
      tot += fmaxf(dot, 0.f) * (wrow[h] * d.w_scale);
    }
    v = tot;
  }
  scores[((size_t)b * d.L + j) * d.Np_cap + p] = v;
}

constexpr int kTopkRowsThreads = 512;

// Flat top-k of one query row; the row's scores are staged in LDS when they fit.
__global__ __launch_bounds__(kTopkRowsThreads) void k_topk_rows(KDims d, int lds_cap, const float* __restrict__ scores,
                                                                const int* __restrict__ t0, int* __restrict__ I,
                                                                int* __restrict__ path) {
  const int b = blockIdx.y, j = blockIdx.x;
  const SeqInfo si = seq_info(d, t0[b]);
  int* Irow = I + ((size_t)b * d.L + j) * d.topk;
  const bool act = flat_active(d, si);
  if (d.force_path == PATH_FLAT) {
    // flat_topk_select: this kernel owns the whole output row.
    const int first_pad = act ? si.k : 0;
    for (int i = threadIdx.x; i < d.topk; i += kTopkRowsThreads)
      if (i >= first_pad) Irow[i] = -1;
    if (path && j == 0 && threadIdx.x == 0) path[b] = si.ok ? PATH_FLAT : PATH_INVALID;
  } else if (act) {
    for (int i = threadIdx.x; i < d.topk; i += kTopkRowsThreads)
      if (i >= si.k) Irow[i] = -1;
  }
  if (!act) return;
  extern __shared__ float s_row[];
  __shared__ TopkScoresSmem sm;
  const float* srow = scores + ((size_t)b * d.L + j) * d.Np_cap;
  auto emit = [&](int slot, int i) { Irow[slot] = i; };
  if (si.Np <= lds_cap) {
    for (int i = threadIdx.x; i < si.Np; i += kTopkRowsThreads) s_row[i] = srow[i];
    __syncthreads();
    block_topk_scores<kTopkRowsThreads>(si.Np, si.k, [&](int i) { return s_row[i]; }, emit, sm);
  } else {
    block_topk_scores<kTopkRowsThreads>(si.Np, si.k, [&](int i) { return srow[i]; }, emit, sm);
  }
}

// Flat top-k of one query row held in registers: 1024 threads x 32 scores
// (n <= 32768).  Element r of lane l in wave w is index 2048w + 64r + l, so a
// wave covers a contiguous index range.  The k-th element in (score desc,
// index asc) order, (kthr, ithr), is found as follows: if fewer than k scores
// are real, every real score and the lowest-index masked ones are taken;
// otherwise the real scores are counted into 2048 linear bins over [min, max]
// (narrowed to the k-th score's bin while that bin holds more than 1024
// entries), and the few entries of the k-th score's bin are ranked exactly.
// Selected: key > kthr, or key == kthr and index <= ithr; emitted in index
// order (ties at the threshold keep the lowest indices).
constexpr int kTkNT = 1024, kTkR = 32, kTkBins = 2048, kTkCand = 1024;
constexpr int kCoarseBins = 256;  // coarse key bins: the top 8 bits of score_key

struct TopkRegSmem {
  float row[kTkNT * kTkR];  // the row, staged: thread t's 32 scores, 16-byte pieces XOR-swizzled
  union {
    struct {
      uint32_t hist[kTkBins];
      float cand_s[kTkCand];
      int cand_i[kTkCand];
    };
    uint32_t h12[4096];  // coarse-bin path: histogram of 12 key bits
  };
  uint32_t wsum[16];
  float red[3][16];
  int info[8];
  uint32_t coarse[kCoarseBins];  // coarse-bin path: the sample's counts per coarse key bin
  uint32_t few[64];              // coarse-bin path: the keys under the k-th key's top 20 bits
};

// Rows of 8193..32768 scores, one workgroup per row, thread t holding the 32
// consecutive scores 32t .. 32t+31 in registers.
//  0. the coarse bin S (top 8 key bits) of the k-th key, first named by a
//     histogram of one sample per thread (the bin of the sample at the
//     scaled rank).  One pass of two float compares per score counts the
//     entries above S and in S; these own counts decide, moving S one bin up
//     or down (three tries).  S's scores go to LDS, a 12-bit histogram of
//     them narrows to 20 key bits, and the few entries under those are
//     ranked by one wave (a second 12-bit round if more than 64); ties of
//     the k-th key are taken lowest index first.  If no try holds the k-th
//     key the row goes to steps 1-3;
//  1. range [lo, hi] of the real scores (masked ones are -1e30) and their count;
//  2. fewer than k real scores: all of them plus the lowest-index masked ones;
//  3. otherwise the k-th score: a histogram of one sample per thread (indices
//     32t) over 2048 linear bins of [lo, hi] brackets it with a margin of
//     three standard deviations of the sample rank; one pass counts the
//     scores above the bracket, and if the k-th lies inside it, the exact
//     histogram rounds below only touch the scores in the bracket (else they
//     start from the whole range).  Each round bins the remaining range into
//     2048 bins and narrows to the k-th score's bin while it holds more than
//     1024 entries; then that bin's entries are ranked exactly (score desc,
//     index asc);
//  4. emission in index order: per-thread counts, a block prefix sum, and
//     each thread writes its own ids.
__global__ __launch_bounds__(kTkNT) void k_topk_rows_reg(KDims d, const float* __restrict__ scores,
                                                         const int* __restrict__ t0, int* __restrict__ I,
                                                         int* __restrict__ path) {
  __shared__ TopkRegSmem sm;
  const int b = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int t0b = t0[b];  // requested first, needed once the row's loads are out
  const float* srow = scores + ((size_t)b * d.L + j) * d.Np_cap;
  const bool staged = (d.Np_cap & 3) == 0;
  if (staged) {
    // The row goes global -> LDS in coalesced 1 KiB pieces (wave w moves
    // pieces w, w+16, ...; piece p = threads 8p .. 8p+7), the whole buffer
    // row before its length is known.  LDS position l of a piece holds the 16
    // bytes at chunk (l % 8) ^ (l / 8) of thread 8p + l / 8, so each thread's
    // eight 16-byte reads below hit distinct banks.
    const uint32_t row_lds = lds_addr(sm.row);
    const int lr = lane >> 3, lc = (lane & 7) ^ lr;
    for (int pc = wv; pc < kTkNT / 8; pc += kTkNT / 64)
      if (pc * 8 * kTkR < d.Np_cap) {
        const int src = min(pc * 8 * kTkR + lr * kTkR + lc * 4, d.Np_cap - 4);
        g2lds16(srow + src, row_lds + pc * 1024);
      }
  }
  if (tid < kCoarseBins) sm.coarse[tid] = 0;  // ordered before any add by the row's barrier
  for (int i = tid; i < 4096; i += kTkNT) sm.h12[i] = 0;  // ordered before any add by later barriers
  const SeqInfo si = seq_info(d, t0b);
  int* Irow = I + ((size_t)b * d.L + j) * d.topk;
  const bool act = flat_active(d, si);
  if (d.force_path == PATH_FLAT) {
    const int first_pad = act ? si.k : 0;
    for (int i = tid; i < d.topk; i += kTkNT)
      if (i >= first_pad) Irow[i] = -1;
    if (path && j == 0 && tid == 0) path[b] = si.ok ? PATH_FLAT : PATH_INVALID;
  } else if (act) {
    for (int i = tid; i < d.topk; i += kTkNT)
      if (i >= si.k) Irow[i] = -1;
  }
  if (!act) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: the row's LDS writes have landed
    return;
  }
  const int n = si.Np, k = si.k;
  const int i0 = kTkR * tid;  // index of v[0]
  // absent entries (index >= n) take -inf: below every real or masked score
  float v[kTkR];
  if (staged) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
    __syncthreads();
    const float* mine = sm.row + (tid >> 3) * 8 * kTkR + (tid & 7) * kTkR;
#pragma unroll
    for (int u = 0; u < kTkR / 4; ++u) {
      const float4 x = *(const float4*)(mine + 4 * (u ^ (tid & 7)));
      v[4 * u] = i0 + 4 * u < n ? x.x : -INFINITY;
      v[4 * u + 1] = i0 + 4 * u + 1 < n ? x.y : -INFINITY;
      v[4 * u + 2] = i0 + 4 * u + 2 < n ? x.z : -INFINITY;
      v[4 * u + 3] = i0 + 4 * u + 3 < n ? x.w : -INFINITY;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kTkR; ++q) v[q] = i0 + q < n ? srow[i0 + q] : -INFINITY;
  }
  // the coarse bins of one sample per thread (index 32t)
  if (i0 < n) atomicAdd(&sm.coarse[score_key(v[0]) >> 24], 1u);
  __syncthreads();
  // the selection: scores with key > kthr, and those with key == kthr at
  // index <= ithr
  uint32_t kthr = 0;
  int ithr = 0;
  // index of the r-th (1-based) entry, in index order, with pred true
  auto rth_index = [&](int r, auto pred) {
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < kTkR; ++q) m |= pred(q) ? 1u << q : 0u;
    uint32_t tot;
    const uint32_t before = block_excl_scan<kTkNT>((uint32_t)__popc(m), sm.wsum, &tot);
    if ((int)before < r && (int)before + __popc(m) >= r) {
      uint32_t x = m;
      for (int s = (int)before + 1; s < r; ++s) x &= x - 1;
      sm.info[6] = i0 + __builtin_ctz(x);
    }
    __syncthreads();
    const int res = sm.info[6];
    __syncthreads();
    return res;
  };
  bool have = false;      // kthr / ithr known
  bool all_ties = false;  // every entry with key kthr is selected
  {
    // 0. the coarse bin S (top 8 key bits) of the k-th key, first the bin of
    // the sample at the same rank, scaled; the row's own counts check it and
    // move it one bin up or down (three tries).  Every wave finds the first S
    // alone: lane l holds bins 255-4l .. 252-4l
    uint32_t hb[4], s4 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      hb[u] = sm.coarse[kCoarseBins - 1 - 4 * lane - u];
      s4 += hb[u];
    }
    const uint32_t inc = wave_incl_scan(s4);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    // the rank to find among the samples (uniform; 0: none)
    const uint32_t rt =
        k >= 1 && tot >= 1 ? (uint32_t)min((long long)tot, max(1LL, ((long long)k * tot + n - 1) / n)) : 0u;
    int S = -1;
    if (rt >= 1) {  // then exactly one lane holds the rt-th
      int Sl = -1;
      uint32_t acc = inc - s4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (acc < rt && acc + hb[u] >= rt) Sl = kCoarseBins - 1 - 4 * lane - u;
        acc += hb[u];
      }
      const uint64_t hit = __ballot(Sl >= 0);
      if (hit) S = __builtin_amdgcn_readlane(Sl, (int)__builtin_ctzll(hit));
    }
    // bin 0 holds -inf and NaN keys only: left to the exact path
    bool found = false;
    float flo = 0.f, fhi = 0.f;
    uint32_t cex = 0;
    int n_above = 0, n_in = 0;
    // counts of the entries at or above S (low half) and above S (high half),
    // each <= 32768; key >= (S << 24) <=> score >= flo and key >= ((S + 1) <<
    // 24) <=> score >= fhi (the key order is the float order; no key lies
    // past bin 255).  Moves S toward the k-th key unless it holds it.
    auto classify = [&]() {
      flo = score_of_key((uint32_t)S << 24);
      fhi = S == kCoarseBins - 1 ? __builtin_nanf("") : score_of_key((uint32_t)(S + 1) << 24);
      uint32_t c = 0;
#pragma unroll
      for (int q = 0; q < kTkR; ++q) {
        c += v[q] >= fhi ? 0x10000u : 0u;
        c += v[q] >= flo ? 1u : 0u;
      }
      uint32_t ctot;
      cex = block_excl_scan<kTkNT>(c, sm.wsum, &ctot);
      n_above = (int)(ctot >> 16);
      n_in = (int)(ctot & 0xFFFFu) - n_above;
      if (n_above >= k)
        ++S;  // uniform: the k-th key lies above S
      else if (n_above + n_in < k)
        --S;  // below S
      else
        found = true;
    };
#pragma unroll 1
    for (int attempt = 0; attempt < 3 && !found && S >= 1 && S < kCoarseBins; ++attempt) classify();
    if (found) {  // S holds the k-th key
      // S's scores into LDS (the row's copy there is no longer read: every
      // thread loaded its scores before the scan's barriers), then the
      // 4096-bin histogram of their key bits 23..12
      float* cf = sm.row;
      int pos = (int)(cex & 0xFFFFu) - (int)(cex >> 16);
#pragma unroll
      for (int q = 0; q < kTkR; ++q)
        if (v[q] >= flo && !(v[q] >= fhi)) cf[pos++] = v[q];
      if (tid == 0) sm.info[3] = 0;
      __syncthreads();
      for (int i = tid; i < n_in; i += kTkNT) atomicAdd(&sm.h12[(score_key(cf[i]) >> 12) & 4095u], 1u);
      __syncthreads();
      int r = k - n_above;  // rank of the k-th key among S's entries, from 1
      // the bin of h12 holding the r-th entry from the top: thread t reads
      // (and clears) bins 4095-4t .. 4092-4t; (bin, entries above it,
      // entries in it) come back through info[slot .. slot+2]
      auto find12 = [&](int slot, int& T, int& above, int& m) {
        const int top = 4095 - 4 * tid;
        uint32_t hx[4], sx = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          hx[u] = sm.h12[top - u];
          sm.h12[top - u] = 0;
          sx += hx[u];
        }
        uint32_t tx;
        const uint32_t ax = block_excl_scan<kTkNT>(sx, sm.wsum, &tx);
        if (ax < (uint32_t)r && ax + sx >= (uint32_t)r) {
          uint32_t acc = ax;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (acc < (uint32_t)r && acc + hx[u] >= (uint32_t)r) {
              sm.info[slot] = top - u;
              sm.info[slot + 1] = (int)acc;
              sm.info[slot + 2] = (int)hx[u];
            }
            acc += hx[u];
          }
        }
        __syncthreads();
        T = sm.info[slot];
        above = sm.info[slot + 1];
        m = sm.info[slot + 2];
      };
      int T, above, m;
      find12(0, T, above, m);
      r -= above;
      const uint32_t pre = ((uint32_t)S << 12) | (uint32_t)T;  // top 20 bits of the k-th key
      uint32_t kt;
      int mt;  // entries with key kt; the r lowest-index ones are taken
      if (m <= 64) {
        // the few entries under pre, ranked by one wave
        for (int i = tid; i < n_in; i += kTkNT) {
          const uint32_t kk = score_key(cf[i]);
          if ((kk >> 12) == pre) sm.few[atomicAdd(&sm.info[3], 1)] = kk;
        }
        __syncthreads();
        if (wv == 0) {
          const uint32_t x0 = lane < m ? sm.few[lane] : 0u;
          int gt = 0, ge = 0;
          for (int u = 0; u < m; ++u) {
            const uint32_t x = sm.few[u];
            gt += x > x0 ? 1 : 0;
            ge += x >= x0 ? 1 : 0;
          }
          if (lane < m && gt < r && ge >= r) {  // every such lane holds the same key
            sm.info[4] = (int)x0;
            sm.info[5] = r - gt;
            sm.info[6] = ge - gt;
          }
        }
        __syncthreads();
        kt = (uint32_t)sm.info[4];
        r = sm.info[5];
        mt = sm.info[6];
      } else {
        // many entries share the top 20 bits: one more 12-bit round
        for (int i = tid; i < n_in; i += kTkNT) {
          const uint32_t kk = score_key(cf[i]);
          if ((kk >> 12) == pre) atomicAdd(&sm.h12[kk & 4095u], 1u);
        }
        __syncthreads();
        int U;
        find12(4, U, above, mt);
        kt = (pre << 12) | (uint32_t)U;
        r -= above;
      }
      kthr = kt;
      all_ties = r == mt;
      ithr = all_ties ? n : rth_index(r, [&](int q) { return i0 + q < n && score_key(v[q]) == kt; });
      have = true;
    }
  }
  if (!have) {
    // 1. range of the real scores, count of masked ones
    float lo = INFINITY, hi = -INFINITY;
    int nmask = 0;
  #pragma unroll
    for (int q = 0; q < kTkR; ++q) {
      const float x = v[q];
      const bool real = x > -1e29f;
      nmask += (!real && x != -INFINITY) ? 1 : 0;
      lo = real ? fminf(lo, x) : lo;
      hi = real ? fmaxf(hi, x) : hi;
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    nmask = wave_sum_i(nmask);
    if (lane == 0) {
      sm.red[0][wv] = lo;
      sm.red[1][wv] = hi;
      sm.red[2][wv] = (float)nmask;
    }
    for (int i = tid; i < kTkBins; i += kTkNT) sm.hist[i] = 0;
    __syncthreads();
    lo = INFINITY;
    hi = -INFINITY;
    nmask = 0;
  #pragma unroll
    for (int u = 0; u < 16; ++u) {
      lo = fminf(lo, sm.red[0][u]);
      hi = fmaxf(hi, sm.red[1][u]);
      nmask += (int)sm.red[2][u];
    }
    const int nreal = n - nmask;
    if (nreal < k) {
      // every real score, then the lowest-index masked entries
      kthr = score_key(kNeg);
      ithr = rth_index(k - nreal, [&](int q) { return v[q] <= -1e29f && v[q] != -INFINITY; });
    } else {
      float blo = lo, bhi = hi;
      int need = k;  // entries still to take inside [blo, bhi]
      bool done = false;
      kthr = 0;
      ithr = 0;
      auto bins_of = [&](float rlo, float rhi, float& scale) {
        scale = (float)kTkBins / (rhi - rlo) * 0.999999f;
      };
      // the bin holding the r-th entry from the top of hist: (bin, entries above
      // it, entries in it); hist is left cleared (each thread clears the bins it
      // read; the scan's barriers order that before any later add).  info[0..2]
      // are written again only past further barriers.
      auto find_bin = [&](int r, int& T, int& above_T, int& in_T) {
        const int b0 = kTkBins - 1 - 2 * tid, b1 = kTkBins - 2 - 2 * tid;
        const uint32_t h0 = sm.hist[b0], h1 = sm.hist[b1];
        sm.hist[b0] = 0;
        sm.hist[b1] = 0;
        uint32_t tot;
        const uint32_t above = block_excl_scan<kTkNT>(h0 + h1, sm.wsum, &tot);
        if (above < (uint32_t)r && above + h0 + h1 >= (uint32_t)r) {
          const bool first = above + h0 >= (uint32_t)r;
          sm.info[0] = first ? b0 : b1;
          sm.info[1] = (int)(first ? above : above + h0);
          sm.info[2] = (int)(first ? h0 : h1);
        }
        __syncthreads();
        T = sm.info[0];
        above_T = sm.info[1];
        in_T = sm.info[2];
      };
      if (hi > lo) {
        // 3a. bracket the k-th score with one sample per thread: one scan of the
        // sample histogram gives the sample count (its total) and the bins of
        // both ends of the bracket; the histogram is cleared as it is read.
        float scale;
        bins_of(lo, hi, scale);
        const float x0 = v[0];
        if (x0 > -1e29f) atomicAdd(&sm.hist[min(kTkBins - 1, (int)((x0 - lo) * scale))], 1u);
        __syncthreads();
        const int b0 = kTkBins - 1 - 2 * tid, b1 = kTkBins - 2 - 2 * tid;
        const uint32_t h0 = sm.hist[b0], h1 = sm.hist[b1];
        sm.hist[b0] = 0;
        sm.hist[b1] = 0;
        uint32_t ns_u;
        const uint32_t above = block_excl_scan<kTkNT>(h0 + h1, sm.wsum, &ns_u);
        const int ns = (int)ns_u;
        const float target = (float)k * (float)ns / (float)nreal;
        const float margin = 3.f * sqrtf(fmaxf(target, 1.f)) + 4.f;
        const int r_hi = max(1, (int)(target - margin)), r_lo = min(ns, (int)ceilf(target + margin));
        if (ns > 0 && r_hi <= r_lo) {  // uniform
          // the bin holding the r-th sample from the top, for r = r_hi and r_lo
          auto locate = [&](int r, int slot) {
            if (above < (uint32_t)r && above + h0 + h1 >= (uint32_t)r) sm.info[slot] = above + h0 >= (uint32_t)r ? b0 : b1;
          };
          locate(r_hi, 0);
          locate(r_lo, 1);
          __syncthreads();
          const int Tt = sm.info[0], Tb = sm.info[1];
          const float clo = Tb == 0 ? lo : fmaxf(lo, lo + (float)Tb / scale);
          const float chi = Tt == kTkBins - 1 ? hi : fminf(hi, lo + (float)(Tt + 1) / scale);
          // both counts in one sum: each is at most 32768, below 2^16
          uint32_t cnt = 0;
  #pragma unroll
          for (int q = 0; q < kTkR; ++q) {
            cnt += v[q] > chi ? 1u : 0u;
            cnt += (v[q] >= clo && v[q] <= chi) ? 0x10000u : 0u;
          }
          uint32_t both;
          block_excl_scan<kTkNT>(cnt, sm.wsum, &both);  // (its barriers also order the reads of info)
          const int n_above = (int)(both & 0xFFFFu), n_in = (int)(both >> 16);
          if (n_above < k && n_above + n_in >= k && chi > clo) {
            blo = clo;
            bhi = chi;
            need = k - n_above;
          }
        }
      }
      // 3b. exact histogram rounds inside [blo, bhi]
      for (int round = 0; round < 4 && !done; ++round) {
        if (!(bhi > blo)) {
          // every remaining score equals blo: ties, lowest indices first
          kthr = score_key(blo);
          const float tv = blo;
          ithr = rth_index(need, [&](int q) { return v[q] == tv; });
          done = true;
          break;
        }
        float scale;
        bins_of(blo, bhi, scale);
        auto bin_of = [&](float x) {
          return (x < blo || x > bhi) ? -1 : min(kTkBins - 1, (int)((x - blo) * scale));
        };
        // (hist is clear: set so before the rounds, and by find_bin after each)
  #pragma unroll
        for (int q = 0; q < kTkR; ++q) {
          const int bn = bin_of(v[q]);
          if (bn >= 0) atomicAdd(&sm.hist[bn], 1u);
        }
        if (tid == 0) sm.info[3] = 0;
        __syncthreads();
        int T, above_T, mcnt;
        find_bin(need, T, above_T, mcnt);
        need -= above_T;
        if (mcnt > kTkCand) {
          // crowded bin: its range becomes the next round's
          const float nlo = blo + (float)T / scale, nhi = blo + (float)(T + 1) / scale;
          // scores exactly at the float bin edges stay inside by the clamp of bin_of
          blo = fmaxf(blo, nlo);
          bhi = fminf(bhi, nhi);
          continue;
        }
        // 3c. gather bin T's entries and rank them (score desc, index asc)
  #pragma unroll
        for (int q = 0; q < kTkR; ++q)
          if (bin_of(v[q]) == T) {
            const int slot = atomicAdd(&sm.info[3], 1);
            sm.cand_s[slot] = v[q];
            sm.cand_i[slot] = i0 + q;
          }
        __syncthreads();
        for (int t = tid; t < mcnt; t += kTkNT) {
          const uint32_t kt = score_key(sm.cand_s[t]);
          const int it = sm.cand_i[t];
          int rank = 0;
          for (int u = 0; u < mcnt; ++u) {
            const uint32_t ku = score_key(sm.cand_s[u]);
            rank += (ku > kt) || (ku == kt && sm.cand_i[u] < it);
          }
          if (rank == need - 1) {
            sm.info[4] = (int)kt;
            sm.info[5] = it;
          }
        }
        __syncthreads();
        kthr = (uint32_t)sm.info[4];
        ithr = sm.info[5];
        done = true;
      }
      if (!done) {
        // still crowded after four narrowings: the k-th score is the largest
        // value whose count from the top reaches `need`; take its ties by index
        // (exact: the crowded bin's scores are then a handful of equal values)
        kthr = score_key(blo);
        const float tv = blo;
        ithr = rth_index(need, [&](int q) { return v[q] == tv; });
      }
    }
  }
  // 4. emission in index order (float compares: the key order is the float
  // order, with -0 == +0)
  const float tv = score_of_key(kthr);
  uint32_t m = 0;
  if (all_ties) {
#pragma unroll
    for (int q = 0; q < kTkR; ++q) m |= v[q] >= tv ? 1u << q : 0u;
  } else {
#pragma unroll
    for (int q = 0; q < kTkR; ++q) {
      const bool sel = v[q] > tv || (v[q] == tv && i0 + q <= ithr);
      m |= sel ? 1u << q : 0u;
    }
  }
  uint32_t tot;
  int slot = (int)block_excl_scan<kTkNT>((uint32_t)__popc(m), sm.wsum, &tot);
  while (m) {
    const int q = __builtin_ctz(m);
    Irow[slot++] = i0 + q;
    m &= m - 1;
  }
}

// The dense fallback with the indexer switched off (HiSA issue, Implementation
// plan item 1): every row of every valid sequence lists all Np pooled rows in
// order (the host checks topk >= Np_cap), padded with -1; no block is kept.
// One workgroup per (row, sequence).
__global__ __launch_bounds__(256) void k_fill_dense(KDims d, const int* __restrict__ t0, int* I, int* top_blk,
                                                    int* path) {
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SeqInfo si = seq_info(d, t0[b]);
  const size_t row = (size_t)b * d.L + j;
  for (int i = tid; i < d.topk; i += 256) I[row * d.topk + i] = (si.ok && i < si.Np) ? i : -1;
  if (top_blk)
    for (int i = tid; i < d.index_keep; i += 256) top_blk[row * d.index_keep + i] = -1;
  if (path && j == 0 && tid == 0) path[b] = si.ok ? PATH_DENSE : PATH_INVALID;
}

// ------------------------------------------------------------------ decode on cached block means

// Decode selection that takes the block means from a caller-kept cache
// instead of re-reading every key (HiSA issue, HiSA decode path: O(nb + Kb*b)
// scores per step; The pooled stream and positions: the pooled stream grows
// in whole windows, so a complete block never changes).  Two kernels:
//   coarse (ceil(nb_cap / 16), B) x 256: the workgroup's 16 blocks are
//          staged in LDS (a block completed by this step's token averaged
//          from the keys, f32, rows in order, and written to the cache first;
//          every other block read from it), then wave w scores them against
//          heads 16w .. 16w+15 on MFMA, each f32 mean split into three bf16
//          parts (a bf16 query times a part is exact in f32).  The workgroup
//          that completes a sequence keeps its top-Kb blocks.
//   fine   (16, B) x 256: 64 candidates per workgroup (the retained blocks'
//          rows, or the rows of a flat sequence) scored on MFMA like the scan;
//          the workgroup that completes a sequence keeps the top-k.
constexpr int kCachedBlocksPerWg = 16;
constexpr int kCachedMaxNb = 4096;
constexpr int kCachedMaxCand = 1024;
constexpr int kCachedSlabs = kCachedMaxCand / 64;  // fine workgroups (64 candidates each) per query row

// Mean of the b key rows of block beta, lane l holding dims 2l and 2l+1 (64
// lanes, D_i = 128): rows summed in order in f32, then scaled by 1/b.
__device__ __forceinline__ float2 block_mean_lane(const uint16_t* kb, int beta, int bsz) {
  const uint32_t* src = (const uint32_t*)(kb + (size_t)beta * bsz * 128) + lane_id();
  float sx = 0.f, sy = 0.f;
#pragma unroll 8
  for (int r = 0; r < bsz; ++r) {
    const uint32_t v = src[r * 64];
    sx += bf_lo(v);
    sy += bf_hi(v);
  }
  const float inv = 1.f / (float)bsz;
  return make_float2(sx * inv, sy * inv);
}

// Stage 1, workgroup x of query row `row` (FUSED: the one-launch form, whose
// completing workgroup hands the kept blocks to the fine workgroups through
// desc instead of blk).
template <bool FUSED>
__device__ __forceinline__ void cached_coarse_wg(const KDims& d, const uint16_t* __restrict__ q_idx,
                                                 const float* __restrict__ w, const uint16_t* __restrict__ keys,
                                                 float* rep, const int* __restrict__ t0, float* cscore, int* blk,
                                                 int* cnt, int* I, int* top_blk, int* path, int x, int row, int ngmax,
                                                 uint64_t* desc) {
  // the workgroup's 16 block means; the row pitch of 132 floats puts the 16
  // blocks' same chunk in distinct banks for the operand reads
  __shared__ __align__(16) float s_rep[kCachedBlocksPerWg][132];
  __shared__ float s_part[4][16];
  __shared__ WgTopkSmem s_tk;
  __shared__ int s_kept[kRowKeep];
  __shared__ int s_flag;
  // one query row (b, j) per row; several rows of a sequence (a verify
  // chunk) each select on their own, with the batched masks
  const int b = row / d.L, j = row - b * d.L;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int t0b = t0[b];
  // this wave's 16 heads as the MFMA A operand (lane (g, c): head 16w + c,
  // dims 32s + 8g .. +7) and the weights of the lane's output heads
  // 16w + 4g + i, requested before t0 arrives
  bf16x8 qa[4];
  {
    const uint16_t* qrow = q_idx + ((size_t)row * 64 + 16 * wv + c) * 128 + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = *(const bf16x8*)(qrow + 32 * s);
  }
  float wl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wl[i] = w[(size_t)row * 64 + 16 * wv + 4 * g + i] * d.w_scale;
  // the cached means of blocks 4w .. 4w+3 of the workgroup, also requested
  // before t0 arrives (a block completed by this step is recomputed instead)
  const int bx0 = x * kCachedBlocksPerWg;
  const int beta0 = bx0 + 4 * wv;
  float* repb = rep + (size_t)b * d.nb_cap * 128;
  float2 mc[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) mc[jj] = *(const float2*)&repb[(size_t)min(beta0 + jj, d.nb_cap - 1) * 128 + 2 * lane];
  const SeqInfo si = seq_info(d, t0b);
  if (!si.ok || si.path == PATH_DENSE) {
    if (x == 0 && wv == 0) write_unscored_row(d, si, row, j, b, I, top_blk, path);
    return;
  }
  if (si.path != PATH_HISA) {  // flat: the fine kernel selects
    if (x == 0 && wv == 0) {
      if (top_blk)
        for (int i = lane; i < d.index_keep; i += 64) top_blk[(size_t)row * d.index_keep + i] = -1;
      if (path && lane == 0 && j == 0) path[b] = si.path;
    }
    return;
  }
  // blocks whose first row this query row cannot see score the mask value
  const int V = visible(d, t0b + j, si.Np);
  const int nwg = (si.nb + kCachedBlocksPerWg - 1) / kCachedBlocksPerWg;
  if (x >= nwg) return;
  const int bsz = d.index_block;
  // blocks completed by this step's token: the ones past the pooled rows
  // that existed before it
  const int first_new = (int)div_ratio(d, (uint32_t)t0b) / bsz;
  const uint16_t* kb = keys + (size_t)b * d.Np_cap * 128;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int beta = beta0 + jj;
    float2 m = make_float2(0.f, 0.f);  // (blocks past nb are never stored)
    if (beta < si.nb) {
      m = mc[jj];
      if (beta >= first_new) {
        m = block_mean_lane(kb, beta, bsz);
        if (row == b * d.L) *(float2*)&repb[(size_t)beta * 128 + 2 * lane] = m;  // the sequence's first row stores it
      }
    }
    *(float2*)&s_rep[4 * wv + jj][2 * lane] = m;
  }
  __syncthreads();
  // D[head][block] = q_head . rep_block: A = q, B = the block means (lane
  // (g, c): block c, dims 32s + 8g .. +7) as hi + mid + lo bf16 parts
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float4 r0 = *(const float4*)&s_rep[c][32 * s + 8 * g];
    const float4 r1 = *(const float4*)&s_rep[c][32 * s + 8 * g + 4];
    const float xv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    u32x4 hi, mid, lo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x0 = xv[2 * k], x1 = xv[2 * k + 1];
      const uint32_t hp = pack_bf16x2(x0, x1);
      const float e0 = x0 - __uint_as_float(hp << 16), e1 = x1 - __uint_as_float(hp & 0xFFFF0000u);
      const uint32_t mp = pack_bf16x2(e0, e1);
      hi[k] = hp;
      mid[k] = mp;
      lo[k] = pack_bf16x2(e0 - __uint_as_float(mp << 16), e1 - __uint_as_float(mp & 0xFFFF0000u));
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, hi), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, mid), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, lo), acc, 0, 0, 0);
  }
  // relu . w over the lane's heads 16w + 4g + i, then over the wave's 16
  // heads (lanes c, c+16, c+32, c+48), then over the four waves
  float hv = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) hv += relu(acc[i]) * wl[i];
  hv = sum_rows(hv);
  if (g == 0) s_part[wv][c] = hv;
  __syncthreads();
  if (wv == 0 && lane < 16) {
    const int beta = bx0 + lane;
    if (beta < si.nb) {
      const float cs = (s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane]);
      st_dev(cscore + (size_t)row * d.nb_cap + beta, beta * bsz < V ? cs : kNeg);
    }
  }
  // cnt: B*L row counters, then B*L x ngmax group counters
  const int nrows = d.B * d.L;
  const int grp = x / kArriveGroup, ngrp = (nwg + kArriveGroup - 1) / kArriveGroup;
  const bool last = publish(
      [&] {
        if (ngrp == 1) return arrive(cnt + (size_t)row * kCntStride, 1, nwg);  // one atomic on the path
        const int members = min(kArriveGroup, nwg - grp * kArriveGroup);
        int* c_grp = cnt + (size_t)(nrows + (size_t)row * ngmax + grp) * kCntStride;
        return arrive(c_grp, 1, members) && arrive(cnt + (size_t)row * kCntStride, 1, ngrp);
      },
      &s_flag);
  if (!last) return;
  // top-Kb of the row's nb block scores, ascending block ids
  const float* csb = cscore + (size_t)row * d.nb_cap;
  uint32_t key[16];
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = ld_dev(csb + min(256 * r + tid, si.nb - 1));
#pragma unroll
  for (int r = 0; r < 16; ++r) key[r] = 256 * r + tid < si.nb ? score_key(v[r]) : 0u;
  int* tbo = top_blk ? top_blk + (size_t)row * d.index_keep : nullptr;
  wg_emit_topk16(key, si.nb, si.Kb, s_tk, [&](int slot, int r) {
    if (FUSED) s_kept[slot] = 256 * r + tid;
    else blk[(size_t)row * d.index_keep + slot] = 256 * r + tid;
    if (tbo) tbo[slot] = 256 * r + tid;
  });
  if (tbo)
    for (int i = si.Kb + tid; i < d.index_keep; i += 256) tbo[i] = -1;
  if (path && tid == 0 && j == 0) path[b] = si.path;
  if constexpr (FUSED) {
    // one word per 64 candidates: the ids (plus one) of its 64 / b kept
    // blocks, 13 bits each, above the mode bits
    lds_sync();
    const int lbsz = __builtin_ctz(bsz), per = 64 >> lbsz;
    const int nslab = (si.Kb * bsz + 63) / 64;
    if (tid < nslab) {
      uint64_t dv = kDescHisa;
      for (int jj = 0; jj < per; ++jj)
        if (tid * per + jj < si.Kb) dv |= (uint64_t)(s_kept[tid * per + jj] + 1) << (2 + 13 * jj);
      st_dev_u64(desc + (size_t)row * kCachedSlabs + tid, dv);
    }
  }
}

// Stage 2, 64 candidates (slab) of query row `row` (FUSED: the kept blocks
// come from the completing coarse workgroup of the same launch through desc,
// polled with a bounded wait; the row's completing workgroup clears them).
template <bool FUSED>
__device__ __forceinline__ void cached_fine_wg(const KDims& d, const uint16_t* __restrict__ q_idx,
                                               const float* __restrict__ w, const uint16_t* __restrict__ keys,
                                               const int* __restrict__ t0, const int* __restrict__ blk, float* fs,
                                               int* cnt, int* I, int slab, int row, uint64_t* desc, int* err) {
  __shared__ __align__(16) uint16_t s_q[64 * 128];
  __shared__ WgTopkSmem s_tk;
  __shared__ int s_blk[kRowKeep];
  __shared__ uint64_t s_word;
  __shared__ int s_flag;
  const int b = row / d.L, j = row - b * d.L;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int t0b = t0[b];
  // the retained blocks (meaningful on the HiSA path only; always in bounds)
  const int blk_tid = (!FUSED && tid < d.index_keep) ? blk[(size_t)row * d.index_keep + tid] : 0;
  issue_q_lds(q_idx + (size_t)row * 64 * 128, s_q);
  const float* wrow = w + (size_t)row * 64;
  float wl[4][4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[ht][i] = wrow[ht * 16 + 4 * g + i];
  const SeqInfo si = seq_info(d, t0b);
  if (!si.ok || si.path == PATH_DENSE) {  // outputs written by the coarse kernel
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no global->LDS copy outlives the workgroup
    return;
  }
  const bool hisa = si.path == PATH_HISA;
  const int bsz = d.index_block, lbsz = __builtin_ctz(bsz);
  const int n = hisa ? si.Kb * bsz : si.Np;  // candidates (<= 1024)
  const int nslab = (n + 63) / 64;
  if (slab >= nslab) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no global->LDS copy outlives the workgroup
    return;
  }
  // a descriptor's block field: the id plus one (0 after a timed-out wait;
  // clamped so that every row read stays inside keys)
  auto desc_blk = [&](uint64_t dv, int jj) {
    const int fld = (int)((dv >> (2 + 13 * jj)) & 0x1FFFu);
    return min(max(fld - 1, 0), d.nb_cap - 1);
  };
  const int per = 64 >> lbsz;
  if constexpr (FUSED) {
    if (hisa) {
      if (tid == 0) s_word = poll_nonzero(desc + (size_t)row * kCachedSlabs + slab, err);
      __syncthreads();
      const uint64_t dv = s_word;
      if (tid < per) s_blk[slab * per + tid] = desc_blk(dv, tid);
    }
  } else {
    if (tid < si.Kb && hisa) s_blk[tid] = blk_tid;
  }
  __syncthreads();
  auto pos = [&](int cc) { return hisa ? (s_blk[cc >> lbsz] << lbsz) + (cc & (bsz - 1)) : cc; };
  const int cand = min(slab * 64 + wv * 16 + c, n - 1);
  const int r = pos(cand);
  const uint16_t* kr = keys + ((size_t)b * d.Np_cap + r) * 128;
  bf16x8 kf[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) kf[s4] = ldg8(kr + s4 * 32 + g * 8);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: q rows, weights and key rows are in
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[ht][i] *= d.w_scale;
  bf16x8 qf[4][4];
  read_q_lds(s_q, qf);
  f32x4 acc[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ht][s4], kf[s4], acc[ht], 0, 0, 0);
  float v = 0.f;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) v += relu(acc[ht][i]) * wl[ht][i];
  v = sum_rows(v);
  // candidates this query row cannot see score the mask value
  if (r >= visible(d, t0b + j, si.Np)) v = kNeg;
  const int cc = slab * 64 + wv * 16 + c;
  float* fsb = fs + (size_t)row * kCachedMaxCand;
  if (g == 0 && cc < n) st_dev(fsb + cc, v);
  const bool last = publish([&] { return arrive(cnt + (size_t)row * kCntStride, 1, nslab); }, &s_flag);
  if (!last) return;
  if constexpr (FUSED) {
    if (hisa) {
      // every kept block, from the row's descriptors (each fine workgroup read
      // its own before it arrived, so they are cleared here)
      if (tid < nslab) {
        uint64_t* dp = desc + (size_t)row * kCachedSlabs + tid;
        const uint64_t dv = ld_dev_u64(dp);
        for (int jj = 0; jj < per; ++jj)
          if (tid * per + jj < si.Kb) s_blk[tid * per + jj] = desc_blk(dv, jj);
        st_dev_u64(dp, 0);
      }
      __syncthreads();
    }
  }
  int* Ib = I + (size_t)row * d.topk;
  for (int i = si.k + tid; i < d.topk; i += 256) Ib[i] = -1;
  uint32_t key[4];
  float sv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) sv[rr] = ld_dev(fsb + min(256 * rr + tid, n - 1));
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) key[rr] = 256 * rr + tid < n ? score_key(sv[rr]) : 0u;
  wg_emit_topk(key, n, si.k, s_tk, [&](int slot, int rr) { Ib[slot] = pos(256 * rr + tid); });
}

// The two stages as separate launches (blk carries the kept blocks).
__global__ __launch_bounds__(256) void k_cached_coarse(KDims d, const uint16_t* __restrict__ q_idx,
                                                       const float* __restrict__ w, const uint16_t* __restrict__ keys,
                                                       float* rep, const int* __restrict__ t0, float* cscore, int* blk,
                                                       int* cnt, int* I, int* top_blk, int* path) {
  args_now(d, q_idx, w, keys, rep, t0, cscore, blk, cnt, I, top_blk, path);
  cached_coarse_wg<false>(d, q_idx, w, keys, rep, t0, cscore, blk, cnt, I, top_blk, path, blockIdx.x, blockIdx.y,
                          (gridDim.x + kArriveGroup - 1) / kArriveGroup, nullptr);
}

__global__ __launch_bounds__(256) void k_cached_fine(KDims d, const uint16_t* __restrict__ q_idx,
                                                     const float* __restrict__ w, const uint16_t* __restrict__ keys,
                                                     const int* __restrict__ t0, const int* __restrict__ blk,
                                                     float* fs, int* cnt, int* I) {
  args_now(d, q_idx, w, keys, t0, blk, fs, cnt, I);
  cached_fine_wg<false>(d, q_idx, w, keys, t0, blk, fs, cnt, I, blockIdx.x, blockIdx.y, nullptr, nullptr);
}

// Both stages in one launch (index_block >= 16, so one 64-bit word holds the
// kept blocks of 64 candidates): rows x nwg_c coarse workgroups, then rows x
// kCachedSlabs fine workgroups, which start at once (q, weights) and wait for
// their descriptor.  The coarse workgroups come first in dispatch order and
// wait for nothing, so the waiting ones cannot hold them off; every wait is
// bounded (err becomes 1 if one ever timed out).
__global__ __launch_bounds__(256) void k_cached_step(KDims d, int nwg_c, const uint16_t* __restrict__ q_idx,
                                                     const float* __restrict__ w, const uint16_t* __restrict__ keys,
                                                     float* rep, const int* __restrict__ t0, float* cscore, float* fs,
                                                     int* cnt_c, int* cnt_f, int* I, int* top_blk, int* path,
                                                     uint64_t* desc, int* err) {
  args_now(d, nwg_c, q_idx, w, keys, rep, t0, cscore, fs, cnt_c, cnt_f, I, top_blk, path, desc, err);
  const int nc = d.B * d.L * nwg_c, bid = blockIdx.x;
  if (bid < nc) {
    const int row = bid / nwg_c;
    cached_coarse_wg<true>(d, q_idx, w, keys, rep, t0, cscore, nullptr, cnt_c, I, top_blk, path, bid - row * nwg_c,
                           row, (nwg_c + kArriveGroup - 1) / kArriveGroup, desc);
    return;
  }
  const int f = bid - nc, row = f / kCachedSlabs;
  cached_fine_wg<true>(d, q_idx, w, keys, t0, nullptr, fs, cnt_f, I, f - row * kCachedSlabs, row, desc, err);
}

// Block means of the blocks completed by the step's L tokens: blocks
// [floor(floor(t0 / r) / b), floor(Np / b)) (every complete block when t0 = 0),
// rows summed in order in f32 and scaled by 1/b, as the cached decode does.
// bf16 keys with 128 dims: one wave (workgroup) per block, spread over every
// CU, lane l dims 2l and 2l+1; all b rows are requested before t0 arrives
// (block beta < nb_cap lies inside the buffer whatever t0 is), then summed in
// order, the same sum as the cached decode's (so the two give the same bits).
__global__ __launch_bounds__(64) void k_rep_update_bf16(KDims d, int all, const uint16_t* __restrict__ keys,
                                                        const int* __restrict__ t0, float* rep, int* zero_p,
                                                        int zero_n) {
  const int b = blockIdx.y, beta = blockIdx.x, lane = lane_id();
  const int t0b = t0[b];  // requested first, needed once the rows' loads are out
  const int bsz = d.index_block;
  const uint32_t* src = (const uint32_t*)(keys + ((size_t)b * d.Np_cap + (size_t)beta * bsz) * 128) + lane;
  uint32_t v[64];
#pragma unroll
  for (int r = 0; r < 64; ++r) v[r] = r < bsz ? src[r * 64] : 0u;
  // sequence 0's workgroups also zero the arrival counters of the kernels that follow
  if (zero_p && b == 0)
    for (int i = blockIdx.x * 64 + lane; i < zero_n; i += gridDim.x * 64) zero_p[i] = 0;
  const SeqInfo si = seq_info(d, t0b);
  const int first_new = all ? 0 : (int)div_ratio(d, (uint32_t)t0b) / bsz;
  if (!si.ok || beta < first_new || beta >= si.nb) return;  // uniform over the wave
  float sx = 0.f, sy = 0.f;
#pragma unroll
  for (int r = 0; r < 64; ++r)
    if (r < bsz) {
      sx += bf_lo(v[r]);
      sy += bf_hi(v[r]);
    }
  const float inv = 1.f / (float)bsz;
  *(float2*)&rep[((size_t)b * d.nb_cap + beta) * 128 + 2 * lane] = make_float2(sx * inv, sy * inv);
}

template <typename T>
__global__ __launch_bounds__(128) void k_rep_update(KDims d, int all, const T* __restrict__ keys,
                                                    const int* __restrict__ t0, float* rep, int* zero_p, int zero_n) {
  const int b = blockIdx.y, beta = blockIdx.x;
  // the first workgroup also zeroes the arrival counters of the kernels that follow
  if (zero_p && b == 0 && beta == 0)
    for (int i = threadIdx.x; i < zero_n; i += 128) zero_p[i] = 0;
  const int t0b = t0[b];
  const SeqInfo si = seq_info(d, t0b);
  if (!si.ok) return;
  const int bsz = d.index_block;
  const int first_new = all ? 0 : (int)div_ratio(d, (uint32_t)t0b) / bsz;
  if (beta < first_new || beta >= si.nb) return;
  const T* kb = keys + ((size_t)b * d.Np_cap + (size_t)beta * bsz) * d.D_i;
  const float inv = 1.f / (float)bsz;
  for (int e = threadIdx.x; e < d.D_i; e += 128) {
    float s = 0.f;
    for (int r = 0; r < bsz; ++r) s += ldf(kb + (size_t)r * d.D_i + e);
    rep[((size_t)b * d.nb_cap + beta) * d.D_i + e] = s * inv;
  }
}

// Zeroes n ints (a fill kernel rather than a memset, so a captured graph holds
// only kernel nodes).
__global__ __launch_bounds__(256) void k_zero_ints(int* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

}  // namespace

// ------------------------------------------------------------------ launchers

bool cached_decode_ok(const KDims& d, bool bf16) {
  const long long bk = (long long)d.index_keep * d.index_block;
  return idx_mfma_ok(d, bf16) && d.index_block > 0 && d.nb_cap <= kCachedMaxNb && bk <= kCachedMaxCand &&
         d.index_keep <= kRowKeep && !d.force_flat && bk >= d.topk;
}

// Counters of the cached decode: per row a coarse counter and ngmax group
// counters, then per row a fine counter, then the error line and the one-launch
// form's descriptors (rows x kCachedSlabs 64-bit words); all zero at rest.
size_t cached_counter_ints(const KDims& d) {
  const size_t rows = (size_t)d.B * d.L;
  const size_t wgs = ((size_t)d.nb_cap + kCachedBlocksPerWg - 1) / kCachedBlocksPerWg;
  const size_t ngmax = (std::max<size_t>(wgs, 1) + kArriveGroup - 1) / kArriveGroup;
  return rows * (1 + ngmax) * kCntStride + rows * kCntStride + kCntStride + rows * kCachedSlabs * 2;
}

size_t cached_fine_floats(const KDims& d) { return (size_t)d.B * d.L * kCachedMaxCand; }

hipError_t launch_cached_decode(const KDims& d, const void* q_idx, const float* w, const void* keys, float* rep,
                                const int* t0, float* cscore, int* blk, float* fs, int* cnt, int* I, int* top_blk,
                                int* path, hipStream_t st) {
  const unsigned wgs = std::max(1u, (unsigned)((d.nb_cap + kCachedBlocksPerWg - 1) / kCachedBlocksPerWg));
  const size_t ngmax = (wgs + kArriveGroup - 1) / kArriveGroup;
  const unsigned rows = (unsigned)(d.B * d.L);
  int* cnt_fine = cnt + (size_t)rows * (1 + ngmax) * kCntStride;
  if (d.index_block >= 16) {
    // one launch: a descriptor word holds the kept blocks of 64 candidates
    int* err = cnt_fine + (size_t)rows * kCntStride;
    uint64_t* desc = (uint64_t*)(err + kCntStride);
    hipLaunchKernelGGL(k_cached_step, dim3(rows * (wgs + kCachedSlabs)), dim3(256), 0, st, d, (int)wgs,
                       (const uint16_t*)q_idx, w, (const uint16_t*)keys, rep, t0, cscore, fs, cnt, cnt_fine, I,
                       top_blk, path, desc, err);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_cached_coarse, dim3(wgs, rows), dim3(256), 0, st, d, (const uint16_t*)q_idx, w,
                     (const uint16_t*)keys, rep, t0, cscore, blk, cnt, I, top_blk, path);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_cached_fine, dim3(kCachedMaxCand / 64, rows), dim3(256), 0, st, d, (const uint16_t*)q_idx, w,
                     (const uint16_t*)keys, t0, blk, fs, cnt_fine, I);
  return hipGetLastError();
}

hipError_t launch_rep_update(const KDims& d, bool bf16, bool all, const void* keys, const int* t0, float* rep,
                             int* zero_p, size_t zero_n, hipStream_t st) {
  if (d.nb_cap == 0) return hipSuccess;
  if (bf16 && d.D_i == 128)
    hipLaunchKernelGGL(k_rep_update_bf16, dim3(d.nb_cap, d.B), dim3(64), 0, st, d, (int)all,
                       (const uint16_t*)keys, t0, rep, zero_p, (int)zero_n);
  else if (bf16)
    hipLaunchKernelGGL(k_rep_update<uint16_t>, dim3(d.nb_cap, d.B), dim3(128), 0, st, d, (int)all,
                       (const uint16_t*)keys, t0, rep, zero_p, (int)zero_n);
  else
    hipLaunchKernelGGL(k_rep_update<float>, dim3(d.nb_cap, d.B), dim3(128), 0, st, d, (int)all, (const float*)keys,
                       t0, rep, zero_p, (int)zero_n);
  return hipGetLastError();
}

hipError_t launch_zero_ints(int* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_ints, dim3(blocks), dim3(256), 0, st, p, (int)n);
  return hipGetLastError();
}

hipError_t launch_fill_dense(const KDims& d, const int* t0, int* I, int* top_blk, int* path, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_dense, dim3(d.L, d.B), dim3(256), 0, st, d, t0, I, top_blk, path);
  return hipGetLastError();
}

static inline unsigned cdiv(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

bool decode_fused_ok(const KDims& d, bool bf16) {
  // every sequence's selection fits one wave: nb, C <= 1024 and Kb <= 64;
  // a flat sequence has Np <= 1024 unless the gate can send a larger one
  // there (forced flat, or b * keep < topk)
  const long long bk = (long long)d.index_keep * d.index_block;
  const bool big_flat = d.Np_cap > 64 * kRowR && (d.force_flat || bk < d.topk);
  return idx_mfma_ok(d, bf16) && d.index_block > 0 && d.nb_cap <= 64 * kRowR && bk <= 64 * kRowR &&
         d.index_keep <= kRowKeep && !big_flat;
}

hipError_t launch_decode_scan(const KDims& d, bool bf16, const void* q_idx, const float* w, const void* keys,
                              const int* t0, float* fscore, float* cscore, int* cnt, int* I, int* top_blk,
                              int* path, hipStream_t st) {
  const dim3 grid(cdiv(d.Np_cap, 64), d.B);
  if (idx_mfma_ok(d, bf16)) {
    const long long slabs = (long long)cdiv(d.Np_cap, 64) * d.B;
    if (slabs <= 1024 || d.B > kStreamMaxB) {
      // latency-bound: one workgroup per slab, rows requested before t0 is known
      hipLaunchKernelGGL(k_decode_scan_mfma, grid, dim3(256), 0, st, d, (const uint16_t*)q_idx, w,
                         (const uint16_t*)keys, t0, fscore, cscore, cnt, I, top_blk, path);
    } else {
      // bandwidth-bound: two resident workgroups per CU share the live slabs
      hipLaunchKernelGGL(k_decode_scan_stream, dim3(512), dim3(256), 0, st, d, (const uint16_t*)q_idx, w,
                         (const uint16_t*)keys, t0, fscore, cscore, cnt, I, top_blk, path);
    }
  }  else if (bf16)
    hipLaunchKernelGGL(k_decode_scan_valu<uint16_t>, grid, dim3(256), 0, st, d, (const uint16_t*)q_idx, w,
                       (const uint16_t*)keys, t0, fscore, cscore);
  else
    hipLaunchKernelGGL(k_decode_scan_valu<float>, grid, dim3(256), 0, st, d, (const float*)q_idx, w,
                       (const float*)keys, t0, fscore, cscore);
  return hipGetLastError();
}

int decode_step_pooled_splits(const KDims& d) {
  return cdiv(std::max(d.index_keep * d.index_block, d.topk), kStepRows);
}
int decode_step_splits(const KDims& d) { return decode_step_pooled_splits(d) + cdiv(d.window, kStepRows); }

// Attention workgroups of the decode step: 8 (sequence, split) pairs x H/16
// head groups per group of 8 H/16 workgroups, the last group padded.
static long long decode_step_attn_wgs(const KDims& d) {
  return 8LL * (d.H / 16) * cdiv((long long)d.B * decode_step_splits(d), 8);
}

bool decode_step_ok(const KDims& d, bool idx_bf16, bool attn_bf16, int max_attn_wgs) {
  if (!decode_fused_ok(d, idx_bf16) || d.L != 1 || d.local_ring) return false;
  // kept blocks of 16, 32 or 64 rows (a split's block ids fit one word); a
  // 512-wide bf16 KV in groups of 16 heads
  if (d.index_block < 16 || d.topk > 1024 || !attn_bf16 || d.Dk != 512 || d.Dv != 512 || d.H % 16 != 0) return false;
  const long long slabs = (long long)d.B * cdiv(d.Np_cap, 64);
  return slabs <= 1024 && decode_step_splits(d) <= kStepMaxSplits && decode_step_attn_wgs(d) <= max_attn_wgs;
}

// Sync words of the decode step, 64-byte lines: err, then per sequence seen
// and thr, then the descriptors.
namespace {
struct StepSyncLayout {
  size_t seen, thr, desc, total;
};
StepSyncLayout step_sync_layout(const KDims& d) {
  StepSyncLayout l;
  const size_t line = kCntStride * sizeof(int), B = (size_t)d.B;
  l.seen = line;
  l.thr = l.seen + B * line;
  l.desc = l.thr + B * line;
  l.total = (l.desc + B * (size_t)decode_step_pooled_splits(d) * sizeof(uint64_t) + 255) & ~(size_t)255;
  return l;
}
}  // namespace

size_t decode_step_sync_bytes(const KDims& d) { return step_sync_layout(d).total; }

size_t decode_step_partial_bytes(const KDims& d) {
  return (size_t)decode_step_splits(d) * d.B * d.H * part_row_bytes(d.Dv);
}

hipError_t launch_decode_step(const KDims& d, const void* q_idx, const float* w, const void* keys, const int* t0,
                              const void* q, const void* local_kv, const void* pooled_kv, const float* sinks,
                              void* sync, int* cnt, float* fscore, float* cscore, float* part, int* I, int* top_blk,
                              int* path, hipStream_t st) {
  const StepSyncLayout l = step_sync_layout(d);
  char* base = (char*)sync;
  StepSync sy;
  sy.err = (int*)base;
  sy.seen = (int*)(base + l.seen);
  sy.thr = (uint64_t*)(base + l.thr);
  sy.desc = (uint64_t*)(base + l.desc);
  const int nslab = cdiv(d.Np_cap, 64);
  const int nspl = decode_step_splits(d), nps = decode_step_pooled_splits(d);
  const int grid = d.B * nslab + (int)decode_step_attn_wgs(d);
  hipLaunchKernelGGL(k_decode_step, dim3(grid), dim3(256), 0, st, d, nslab, nps, nspl, (const uint16_t*)q_idx, w,
                     (const uint16_t*)keys, t0, (const uint16_t*)q, (const uint16_t*)local_kv,
                     (const uint16_t*)pooled_kv, sinks, fscore, cscore, cnt, I, top_blk, path, part, sy);
  return hipGetLastError();
}

hipError_t launch_decode_select(const KDims& d, const float* fscore, const float* cscore, const int* t0, int* I,
                                int* top_blk, int* path, hipStream_t st) {
  const int cap = std::min(kSelectLdsCap, std::max({d.nb_cap, d.index_keep * d.index_block, d.Np_cap}));
  hipLaunchKernelGGL(k_decode_select, dim3(d.B), dim3(kSelectThreads), (size_t)cap * sizeof(float), st, d, cap,
                     fscore, cscore, t0, I, top_blk, path);
  return hipGetLastError();
}

hipError_t launch_block_mean(const KDims& d, bool bf16, bool all_paths, const void* keys, const int* t0,
                             float* rep, uint16_t* rep3, hipStream_t st) {
  if (d.nb_cap == 0) return hipSuccess;
  const dim3 grid(d.nb_cap, d.B);
  if (bf16)
    hipLaunchKernelGGL(k_block_mean<uint16_t>, grid, dim3(128), 0, st, d, (int)all_paths, (const uint16_t*)keys, t0,
                       rep, rep3);
  else
    hipLaunchKernelGGL(k_block_mean<float>, grid, dim3(128), 0, st, d, (int)all_paths, (const float*)keys, t0, rep,
                       rep3);
  return hipGetLastError();
}

hipError_t launch_coarse(const KDims& d, bool bf16, bool all_paths, const void* q_idx, const float* w,
                         const float* rep, const uint16_t* rep3, const int* t0, float* cscore, hipStream_t st) {
  if (d.nb_cap == 0) return hipSuccess;
  if (idx_mfma_ok(d, bf16))
    hipLaunchKernelGGL(k_coarse_mfma, dim3(cdiv(d.L, 4), d.B), dim3(256), 0, st, d, (int)all_paths,
                       (const uint16_t*)q_idx, w, rep3, t0, cscore);
  else if (bf16)
    hipLaunchKernelGGL(k_coarse_valu<uint16_t>, dim3(d.L, d.B), dim3(256), 0, st, d, (int)all_paths,
                       (const uint16_t*)q_idx, w, rep, t0, cscore);
  else
    hipLaunchKernelGGL(k_coarse_valu<float>, dim3(d.L, d.B), dim3(256), 0, st, d, (int)all_paths,
                       (const float*)q_idx, w, rep, t0, cscore);
  return hipGetLastError();
}

bool select_rows_ok(const KDims& d, bool bf16) {
  return idx_mfma_ok(d, bf16) && d.index_block > 0 && d.nb_cap <= 64 * kRowR &&
         (long long)d.index_keep * d.index_block <= 64 * kRowR && d.index_keep <= kRowKeep;
}

hipError_t launch_select_rows(const KDims& d, const void* q_idx, const float* w, const void* keys, const uint16_t* rep3,
                              const int* t0, int* I, int* top_blk, int* path, hipStream_t st) {
  hipLaunchKernelGGL(k_select_rows, dim3(cdiv(d.L, 4), d.B), dim3(256), 0, st, d, (const uint16_t*)q_idx, w,
                     (const uint16_t*)keys, rep3, t0, I, top_blk, path);
  return hipGetLastError();
}

hipError_t launch_fine(const KDims& d, bool bf16, const void* q_idx, const float* w, const void* keys,
                       const float* cscore, const int* t0, int* I, int* top_blk, int* path, hipStream_t st) {
  // coarse scores are staged in LDS when they fit next to the fine scores
  const int lds_floats = std::max(d.index_keep * d.index_block, std::min(d.nb_cap, 12288));
  const size_t lds = (size_t)lds_floats * sizeof(float);
  const dim3 grid(d.L, d.B);
  if (idx_mfma_ok(d, bf16))
    hipLaunchKernelGGL(k_fine_mfma, grid, dim3(256), lds, st, d, lds_floats, (const uint16_t*)q_idx, w, (const uint16_t*)keys,
                       cscore, t0, I, top_blk, path);
  else if (bf16)
    hipLaunchKernelGGL(k_fine_valu<uint16_t>, grid, dim3(256), lds, st, d, (const uint16_t*)q_idx, w,
                       (const uint16_t*)keys, cscore, t0, I, top_blk, path);
  else
    hipLaunchKernelGGL(k_fine_valu<float>, grid, dim3(256), lds, st, d, (const float*)q_idx, w, (const float*)keys,
                       cscore, t0, I, top_blk, path);
  return hipGetLastError();
}

hipError_t launch_flat_scores(const KDims& d, bool bf16, const void* q_idx, const float* w, const void* keys,
                              const int* t0, float* scores, hipStream_t st) {
  if (idx_mfma_ok(d, bf16)) {
    // Few query rows: short key chunks spread the scan over the whole chip;
    // many rows: long chunks keep the queries in registers across more keys.
    const int kc = d.L <= 8 ? kFlatTile : 2048;
    hipLaunchKernelGGL(k_flat_scores_mfma, dim3(cdiv(d.Np_cap, kc), cdiv(d.L, 8), d.B), dim3(256), 0, st, d, kc,
                       (const uint16_t*)q_idx, w, (const uint16_t*)keys, t0, scores);
  } else if (bf16) {
    hipLaunchKernelGGL(k_flat_scores_valu<uint16_t>, dim3(cdiv(d.Np_cap, 256), d.L, d.B), dim3(256), 0, st, d,
                       (const uint16_t*)q_idx, w, (const uint16_t*)keys, t0, scores);
  } else {
    hipLaunchKernelGGL(k_flat_scores_valu<float>, dim3(cdiv(d.Np_cap, 256), d.L, d.B), dim3(256), 0, st, d,
                       (const float*)q_idx, w, (const float*)keys, t0, scores);
  }
  return hipGetLastError();
}

hipError_t launch_topk_rows(const KDims& d, const float* scores, const int* t0, int* I, int* path, hipStream_t st) {
  if (d.Np_cap > 8192 && d.Np_cap <= kTkNT * kTkR) {
    // long rows: scores held in registers of a 1024-thread workgroup
    hipLaunchKernelGGL(k_topk_rows_reg, dim3(d.L, d.B), dim3(kTkNT), 0, st, d, scores, t0, I, path);
    return hipGetLastError();
  }
  constexpr int kLdsCap = 32768;  // 128 KiB of keys
  const int cap = d.Np_cap <= kLdsCap ? d.Np_cap : 0;
  const size_t lds = (size_t)cap * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_topk_rows, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kLdsCap * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_topk_rows, dim3(d.L, d.B), dim3(kTopkRowsThreads), lds, st, d, cap, scores, t0, I, path);
  return hipGetLastError();
}

}  // namespace hisa
