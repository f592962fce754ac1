// hisa_device.h -- device-side helpers shared by the HiSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisa_internal.h"

namespace hisa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

constexpr float kNeg = -1e30f;  // the selection paths' finite mask value
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (inputs here are finite)
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ void stf(T* p, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void stf<uint16_t>(uint16_t* p, float v) { *p = f2bf(v); }

// Order-preserving 32-bit key of a float score: a larger score gives a larger
// key, and -0 / +0 give the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  const int lane = lane_id();
  return __popcll(mask & ((1ull << lane) - 1ull));
}

// Per-sequence facts (HiSA issue: pooled count, gate).  ok == false marks a
// sequence whose t0 breaks the buffer bounds.
struct SeqInfo {
  int Np, nb, Kb, k, path;
  bool ok;
};

__device__ __forceinline__ SeqInfo seq_info(const KDims& d, int t0) {
  SeqInfo s;
  const long long np = ((long long)t0 + d.L) / d.ratio;
  s.ok = t0 >= 0 && np <= d.Np_cap;
  s.Np = s.ok ? (int)np : 0;
  s.k = min(d.topk, s.Np);
  s.nb = d.index_block > 0 ? s.Np / d.index_block : 0;
  s.Kb = min(d.index_keep, s.nb);
  const int bk = d.index_block * d.index_keep;
  if (!s.ok) s.path = PATH_INVALID;
  else if (d.force_path >= 0) s.path = d.force_path;
  else if (s.Np <= d.topk) s.path = PATH_DENSE;
  else if (!d.force_flat && d.index_block > 0 && s.Np >= bk && bk >= s.k) s.path = PATH_HISA;
  else s.path = PATH_FLAT;
  return s;
}

__device__ __forceinline__ int visible(int t, int ratio, int Np) {
  return min(Np, (int)(((long long)t + 1) / ratio));
}

// Shared memory of block_topk.
struct TopkSmem {
  uint32_t hist[2048];
  uint32_t wtot[2][16];
  int bcast[4];
};

// Block-wide exclusive scan of one value per thread; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_w, uint32_t* total) {
  constexpr int NW = NT / 64;
  const uint32_t incl = wave_incl_scan(v);
  if (lane_id() == 63) s_w[wave_id()] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = s_w[w];
    if (w < wave_id()) before += x;
    all += x;
  }
  *total = all;
  __syncthreads();
  return before + incl - v;
}

// Top-k of n keys (larger key first; equal keys keep the lowest index), by
// radix select on 11/11/10-bit digits.  key(i) returns the 32-bit key of item
// i; emit(slot, i) is called once for each selected item, with slots
// 0..k-1 given in ascending index order.  Requires 0 <= k <= n.  All NT
// threads of the block must call it.
template <int NT, class KeyF, class EmitF>
__device__ void block_topk(int n, int k, KeyF key, EmitF emit, TopkSmem& sm) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  if (k <= 0) return;
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
  if (k < n) {
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nbins = pass == 2 ? 1024 : 2048;
      for (int i = tid; i < nbins; i += NT) sm.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t u = key(i);
        if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & (nbins - 1)], 1u);
      }
      __syncthreads();
      // Counts from the top bin down: thread t owns bins nbins-1-t*bpt-i.
      const int bpt = nbins / NT;
      uint32_t local = 0;
      for (int i = 0; i < bpt; ++i) local += sm.hist[nbins - 1 - (tid * bpt + i)];
      uint32_t tot;
      const uint32_t above = block_excl_scan<NT>(local, sm.wtot[0], &tot);
      if (above < (uint32_t)remaining && above + local >= (uint32_t)remaining) {
        uint32_t acc = above;
        for (int i = 0; i < bpt; ++i) {
          const int bin = nbins - 1 - (tid * bpt + i);
          const uint32_t c = sm.hist[bin];
          if (acc + c >= (uint32_t)remaining) {
            sm.bcast[0] = bin;
            sm.bcast[1] = (int)acc;
            sm.bcast[2] = (int)c;
            break;
          }
          acc += c;
        }
      }
      __syncthreads();
      const int digit = sm.bcast[0];
      const int cnt_above = sm.bcast[1];
      const int cnt_bin = sm.bcast[2];
      __syncthreads();
      remaining -= cnt_above;
      prefix |= (uint32_t)digit << shift;
      mask |= (uint32_t)(nbins - 1) << shift;
      if (cnt_bin == remaining) break;  // every key in this bin is selected
    }
  } else {
    remaining = n;  // everything is selected: mask 0 makes every key "equal"
  }
  // Emission in index order.  Wave w scans items [w*chunk, (w+1)*chunk).
  const int chunk = (((n + NW - 1) / NW) + 63) & ~63;
  const int wv = wave_id();
  const int lo = min(n, wv * chunk), hi = min(n, lo + chunk);
  int gt = 0, eq = 0;
  for (int i = lo + lane_id(); i < hi; i += 64) {
    const uint32_t u = key(i) & mask;
    gt += u > prefix;
    eq += u == prefix;
  }
  gt = wave_sum_i(gt);
  eq = wave_sum_i(eq);
  if (lane_id() == 0) {
    sm.wtot[0][wv] = (uint32_t)gt;
    sm.wtot[1][wv] = (uint32_t)eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wv; ++w) {
    gt_before += (int)sm.wtot[0][w];
    eq_before += (int)sm.wtot[1][w];
  }
  __syncthreads();
  int eq_run = eq_before;
  int sel_run = gt_before + min(eq_before, remaining);
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane_id();
    uint32_t u = 0;
    bool g = false, e = false;
    if (i < hi) {
      u = key(i) & mask;
      g = u > prefix;
      e = u == prefix;
    }
    const uint64_t em = __ballot(e);
    const int eq_rank = eq_run + lanes_below(em);
    const bool s = g || (e && eq_rank < remaining);
    const uint64_t sm_ = __ballot(s);
    if (s) emit(sel_run + lanes_below(sm_), i);
    eq_run += __popcll(em);
    sel_run += __popcll(sm_);
  }
}

}  // namespace hisa
