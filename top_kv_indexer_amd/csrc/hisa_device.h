// hisa_device.h -- device-side helpers shared by the HiSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisa_internal.h"

namespace hisa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;  // LDS operand of the transposing reads

constexpr float kNeg = -1e30f;  // the selection paths' finite mask value
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (inputs here are finite)
  return (uint16_t)(u >> 16);
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations (lgkmcnt 0) but leaves vector-memory loads in flight, including
// global->LDS loads into a buffer no wave reads before a full barrier.
// (__syncthreads() would wait for those loads as well.)
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane l's 16 bytes from gsrc land at LDS byte address lds_base + 16*l
// (lds_base is wave-uniform).  It is issued through inline assembly so the
// compiler does not hold later LDS accesses to other buffers behind it; the
// caller waits on vmcnt and synchronises before any wave reads the
// destination.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}
// 0 in every lane, opaque to the compiler: added to an LDS address that is
// the same in every lane, it keeps the loaded value in vector registers.
__device__ __forceinline__ int vector_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}
// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane i's bytes land at lds_base + 16 i, lds_base
// the same in every lane (it goes to the instruction through m0, which the
// compiler sets as the asm's input).  Counted on vmcnt like any vector load;
// the callers wait for it explicitly.  (As asm, the load is invisible to the
// compiler's own LDS-DMA wait insertion, which cannot tell ring slots of one
// LDS array apart and would otherwise drain every prefetch before LDS reads.)
__device__ __forceinline__ void g2lds16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// The same load as a compiler builtin, which the compiler schedules and waits
// for itself (it adds a full vmcnt wait before any LDS read it cannot tell
// apart from the load's destination): for kernels whose LDS reads it can.
__device__ __forceinline__ void g2lds16_builtin(const void* gsrc, uint32_t lds_base) {
  __builtin_amdgcn_global_load_lds(
      gsrc, (__attribute__((address_space(3))) void*)(uintptr_t)__builtin_amdgcn_readfirstlane(lds_base), 16, 0, 0);
}

// Two floats to a packed bf16 pair (low half = lo), round to nearest even, in
// one gfx950 conversion instruction.
// The low / high bf16 of a packed pair, as floats.
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
// One split partial row (see part_row_bytes): the four normalised output
// values of columns col .. col+3 (o times inv = 1 / l), and (m, l).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi);
__device__ __forceinline__ void store_part4(void* part, size_t prow, int Dv, int col, f32x4 o, float inv) {
  uint2 v;
  v.x = pack_bf16x2(o[0] * inv, o[1] * inv);
  v.y = pack_bf16x2(o[2] * inv, o[3] * inv);
  *(uint2*)((char*)part + prow * part_row_bytes(Dv) + 2 * (size_t)col) = v;
}
__device__ __forceinline__ void store_part_ml(void* part, size_t prow, int Dv, float m, float l) {
  float* ml = (float*)((char*)part + prow * part_row_bytes(Dv) + 2 * (size_t)Dv);
  ml[0] = m;
  ml[1] = l;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
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

// The float of a key (inverse of score_key; -0 comes back as +0).
__device__ __forceinline__ float score_of_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// Cross-lane reductions in registers (no LDS traffic).  Lane l = 16*g + c:
// the 16 lanes of a row share g.  DPP quad_perm / row mirrors combine lanes
// within a row; the gfx950 permlane swaps exchange whole rows (xor 16, xor 32).
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  // rows outside ROW_MASK and invalid source lanes read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Sum over aligned groups of `span` lanes within a row (span 1, 2, 4, 8, 16).
__device__ __forceinline__ float sum_span(float v, int span) {
  if (span >= 2) v += dpp_f<kDppXor1>(v);
  if (span >= 4) v += dpp_f<kDppXor2>(v);
  if (span >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (span >= 16) v += dpp_f<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float max_span8(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  return fmaxf(v, dpp_f<kDppHalfMirror>(v));
}
__device__ __forceinline__ float sum_row16(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}
__device__ __forceinline__ float max_row16(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float min_row16(float v) {
  v = fminf(v, dpp_f<kDppXor1>(v));
  v = fminf(v, dpp_f<kDppXor2>(v));
  v = fminf(v, dpp_f<kDppHalfMirror>(v));
  return fminf(v, dpp_f<kDppMirror>(v));
}
// Sum / max over the four rows (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float sum_rows(float v) {
  u32x2 p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p.x) + __uint_as_float(p.y);
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}
__device__ __forceinline__ float max_rows(float v) {
  u32x2 p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
}
__device__ __forceinline__ float min_rows(float v) {
  u32x2 p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fminf(__uint_as_float(p.x), __uint_as_float(p.y));
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(p.x), __uint_as_float(p.y));
}
__device__ __forceinline__ float wave_sum(float v) { return sum_rows(sum_row16(v)); }
__device__ __forceinline__ float wave_max(float v) { return max_rows(max_row16(v)); }
__device__ __forceinline__ float wave_min(float v) { return min_rows(min_row16(v)); }
__device__ __forceinline__ int wave_sum_i(int v) {
  v += (int)dpp_u<kDppXor1>((uint32_t)v);
  v += (int)dpp_u<kDppXor2>((uint32_t)v);
  v += (int)dpp_u<kDppHalfMirror>((uint32_t)v);
  v += (int)dpp_u<kDppMirror>((uint32_t)v);
  u32x2 p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int)(p.x + p.y);
  p = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)(p.x + p.y);
}
// Inclusive prefix sum over the 64 lanes: row-local shifts 1, 2, 4, 8, then
// row 15 -> rows 1 and 3, row 31 -> rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u<0x111>(v);
  v += dpp_u<0x112>(v);
  v += dpp_u<0x114>(v);
  v += dpp_u<0x118>(v);
  v += dpp_u<0x142, 0xA>(v);
  v += dpp_u<0x143, 0xC>(v);
  return v;
}
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  const int lane = lane_id();
  return __popcll(mask & ((1ull << lane) - 1ull));
}

// Device-scope (all XCDs) store and load of a float: written through to, and
// read from, the device's coherence point, so handing values to workgroups
// on other XCDs needs no L2 write-back.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-sequence facts (HiSA issue: pooled count, gate).  ok == false marks a
// sequence whose t0 breaks the buffer bounds.
struct SeqInfo {
  int Np, nb, Kb, k, path;
  bool ok;
};

// floor(x / ratio) for 0 <= x < 2^32: a shift for power-of-two ratios, else
// one 32-bit unsigned division
__device__ __forceinline__ uint32_t div_ratio(const KDims& d, uint32_t x) {
  return d.ratio_shift >= 0 ? x >> d.ratio_shift : x / (uint32_t)d.ratio;
}

// Every kernel argument into scalar registers at once, at the top of a
// latency-bound kernel: a kernel-argument load that misses the scalar cache
// takes ~0.6 us, and left alone the compiler issues each where it is first
// used, behind its own wait, so several of them line up one after another.
__device__ __forceinline__ void args_now(const KDims& d) {
  asm volatile("" ::"s"(d.B), "s"(d.L), "s"(d.ratio), "s"(d.window), "s"(d.topk), "s"(d.index_block),
               "s"(d.index_keep), "s"(d.H_i), "s"(d.D_i), "s"(d.H), "s"(d.Dk), "s"(d.Dv), "s"(d.Np_cap),
               "s"(d.Wl_cap), "s"(d.kI), "s"(d.force_flat), "s"(d.force_path), "s"(d.nb_cap), "s"(d.ratio_shift),
               "s"(d.w_scale), "s"(d.attn_scale_log2));
}
template <class T>
__device__ __forceinline__ void arg_now(T v) {
  asm volatile("" ::"s"(v));
}
template <class... T>
__device__ __forceinline__ void args_now(const KDims& d, T... v) {
  args_now(d);
  (arg_now(v), ...);
}

__device__ __forceinline__ SeqInfo seq_info(const KDims& d, int t0) {
  SeqInfo s;
  // t0 + L < 2^32 for any t0 >= 0 (L <= 524280): unsigned 32-bit math is exact
  const uint32_t np = t0 >= 0 ? div_ratio(d, (uint32_t)t0 + (uint32_t)d.L) : 0u;
  s.ok = t0 >= 0 && np <= (uint32_t)d.Np_cap;
  s.Np = s.ok ? (int)np : 0;
  s.k = min(d.topk, s.Np);
  s.nb = d.index_block > 0 ? s.Np / d.index_block : 0;
  s.Kb = min(d.index_keep, s.nb);
  const int bk = d.index_block * d.index_keep;
  if (!s.ok) s.path = PATH_INVALID;
  else if (d.force_path >= 0) s.path = d.force_path;
  else if (d.force_dense || s.Np <= d.topk) s.path = PATH_DENSE;
  else if (!d.force_flat && d.index_block > 0 && s.Np >= bk && bk >= s.k) s.path = PATH_HISA;
  else s.path = PATH_FLAT;
  return s;
}

// V(t) = min(Np, floor((t + 1) / ratio)) for query position t (0 for t < 0)
__device__ __forceinline__ int visible(const KDims& d, int t, int Np) {
  return t < 0 ? 0 : min(Np, (int)div_ratio(d, (uint32_t)t + 1u));
}

// Device-scope int and 64-bit stores / loads (the same coherence point as
// st_dev / ld_dev): flags and lists handed to workgroups on other XCDs.
__device__ __forceinline__ void st_dev_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev_i(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- attention row lists (the sparse combine's local and pooled rows)

// LDS slot (16-byte units) of chunk ch of a KV or q row whose swizzle is x
// (0..15): the first 64 chunks (512 dims) XOR x in their low four bits; the
// chunks past them XOR x inside the row's tail, which the row pitch rounds up
// to whole 256-byte groups.  16 rows with distinct x then read one chunk from
// 16 distinct 16-byte slots, conflict free, in the tail as in the body.
__device__ __forceinline__ int tail_pos(int ch, int x) { return ch < 64 ? (ch ^ x) : 64 + ((ch - 64) ^ x); }

struct RowPlan {
  bool ok;
  int Np, V, ls, s_lo, n_loc, n_list;
  int lbase;  // local_kv row of position s_lo (the first local entry)
};

// Ring slot of position t0[b] (ring layout only; read with t0).
__device__ __forceinline__ int ring_slot0(const KDims& d, int b, int T0) {
  if (!d.local_ring) return 0;
  if (d.ring_slot) return d.ring_slot[b];
  return T0 >= 0 ? T0 % d.Wl_cap : 0;
}

// Local rows: linear layout, row r holds position ls + r; ring layout
// (Wl_cap >= window + L - 1, checked by the host), position s sits in slot
// (S0 + s - T0) mod Wl_cap.  Either way local entry k is row lbase + k,
// wrapped once past Wl_cap (which only the ring reaches).
__device__ __forceinline__ RowPlan row_plan(const KDims& d, int T0, int S0, int j) {
  RowPlan r;
  const uint32_t np = T0 >= 0 ? div_ratio(d, (uint32_t)T0 + (uint32_t)d.L) : 0u;
  r.ls = max(0, T0 - d.window + 1);
  const bool local_ok = d.window == 0 || (d.local_ring ? (S0 >= 0 && S0 < d.Wl_cap)
                                                       : (long long)T0 + d.L - r.ls <= d.Wl_cap);
  r.ok = T0 >= 0 && np <= (uint32_t)d.Np_cap && local_ok;
  r.Np = r.ok ? (int)np : 0;
  const int t = T0 + j;
  r.V = visible(d, t, r.Np);
  r.s_lo = max(r.ls, t - d.window + 1);
  r.n_loc = (r.ok && d.window > 0) ? t - r.s_lo + 1 : 0;
  r.n_list = r.ok ? r.n_loc + d.kI : 0;
  if (d.local_ring) {
    int base = S0 + (r.s_lo - T0);  // in (-Wl_cap, 2 Wl_cap)
    base = base < 0 ? base + d.Wl_cap : (base >= d.Wl_cap ? base - d.Wl_cap : base);
    r.lbase = r.ok ? base : 0;
  } else {
    r.lbase = r.s_lo - r.ls;
  }
  return r;
}

__device__ __forceinline__ int local_row(const KDims& d, const RowPlan& rp, int k) {
  const int r = rp.lbase + k;
  return r >= d.Wl_cap ? r - d.Wl_cap : r;
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

// Shared memory of block_topk_scores.
struct TopkScoresSmem {
  TopkSmem radix;             // fallback
  float red[4][16];           // per-wave partials: min, max, masked count
  int info[8];
  float cand_s[256];
  int cand_i[256];
};

// Top-k of n float scores (larger first, equal scores keep the lowest index;
// kNeg marks masked entries, which rank below every real score), emitting
// slots 0..k-1 in ascending index order like block_topk.  Scores are bucketed
// linearly over [min, max] of the real scores into 2048 bins; everything above
// the bin that holds the k-th score is selected, and the few entries inside
// that bin are ranked exactly.  Falls back to the radix select when that bin
// holds more than 256 entries (heavy ties) or the scores are degenerate.
template <int NT, class ScoreF, class EmitF, int kTopkBins = 2048>
__device__ void block_topk_scores(int n, int k, ScoreF score, EmitF emit, TopkScoresSmem& sm) {
  static_assert(kTopkBins <= 2048 && kTopkBins % NT == 0, "bins must fit the histogram and split over threads");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  if (k <= 0) return;
  auto key_of = [&](int i) { return score_key(score(i)); };
  if (k >= n) {
    block_topk<NT>(n, k, key_of, emit, sm.radix);
    return;
  }
  // 1. range of the real scores and the masked count
  float lo = INFINITY, hi = -INFINITY;
  int nmask = 0;
  for (int i = tid; i < n; i += NT) {
    const float v = score(i);
    if (v <= -1e29f) ++nmask;
    else {
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  nmask = wave_sum_i(nmask);
  if (lane == 0) {
    sm.red[0][wv] = lo;
    sm.red[1][wv] = hi;
    sm.red[2][wv] = (float)nmask;
  }
  for (int i = tid; i < kTopkBins; i += NT) sm.radix.hist[i] = 0;
  __syncthreads();
  lo = INFINITY;
  hi = -INFINITY;
  nmask = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = fminf(lo, sm.red[0][w]);
    hi = fmaxf(hi, sm.red[1][w]);
    nmask += (int)sm.red[2][w];
  }
  const int nreal = n - nmask;
  const float scale = (float)kTopkBins / (hi - lo) * 0.999999f;
  if (nreal < k || !(hi > lo) || !(scale < 1e30f) || !(hi - lo < 1e30f)) {
    // masked entries at the boundary, or a degenerate range
    block_topk<NT>(n, k, key_of, emit, sm.radix);
    return;
  }
  // 2. histogram of real scores over linear bins (monotone in the score)
  auto bin_of = [&](float v) { return v <= -1e29f ? -1 : min(kTopkBins - 1, (int)((v - lo) * scale)); };
  for (int i = tid; i < n; i += NT) {
    const int bn = bin_of(score(i));
    if (bn >= 0) atomicAdd(&sm.radix.hist[bn], 1u);
  }
  __syncthreads();
  // 3. bin holding the k-th score, counted from the top
  const int bpt = kTopkBins / NT;
  uint32_t local = 0;
  for (int i = 0; i < bpt; ++i) local += sm.radix.hist[kTopkBins - 1 - (tid * bpt + i)];
  uint32_t tot;
  const uint32_t above = block_excl_scan<NT>(local, sm.radix.wtot[0], &tot);
  if (above < (uint32_t)k && above + local >= (uint32_t)k) {
    uint32_t acc = above;
    for (int i = 0; i < bpt; ++i) {
      const int bn = kTopkBins - 1 - (tid * bpt + i);
      const uint32_t cnt = sm.radix.hist[bn];
      if (acc + cnt >= (uint32_t)k) {
        sm.info[0] = bn;
        sm.info[1] = (int)acc;
        sm.info[2] = (int)cnt;
        break;
      }
      acc += cnt;
    }
  }
  if (tid == 0) sm.info[3] = 0;
  __syncthreads();
  const int T = sm.info[0];
  const int r = k - sm.info[1];  // entries still needed from bin T
  const int m = sm.info[2];      // entries in bin T
  if (m > 256) {
    block_topk<NT>(n, k, key_of, emit, sm.radix);
    return;
  }
  // 4. gather bin T's entries and find the r-th best of them (score desc, index asc)
  for (int i = tid; i < n; i += NT) {
    const float v = score(i);
    if (bin_of(v) == T) {
      const int slot = atomicAdd(&sm.info[3], 1);
      sm.cand_s[slot] = v;
      sm.cand_i[slot] = i;
    }
  }
  __syncthreads();
  for (int t = tid; t < m; t += NT) {
    const uint32_t kt = score_key(sm.cand_s[t]);
    const int it = sm.cand_i[t];
    int rank = 0;
    for (int j = 0; j < m; ++j) {
      const uint32_t kj = score_key(sm.cand_s[j]);
      rank += (kj > kt) || (kj == kt && sm.cand_i[j] < it);
    }
    if (rank == r - 1) {
      sm.info[4] = (int)kt;
      sm.info[5] = it;
    }
  }
  __syncthreads();
  const uint32_t kthr = (uint32_t)sm.info[4];
  const int ithr = sm.info[5];
  auto selected = [&](int i) {
    const float v = score(i);
    const int bn = bin_of(v);
    if (bn != T) return bn > T;
    const uint32_t kv = score_key(v);
    return kv > kthr || (kv == kthr && i <= ithr);
  };
  // 5. emission in index order (wave w scans a contiguous range)
  const int chunk = (((n + NW - 1) / NW) + 63) & ~63;
  const int lo_i = min(n, wv * chunk), hi_i = min(n, lo_i + chunk);
  int cnt = 0;
  for (int i = lo_i + lane; i < hi_i; i += 64) cnt += selected(i);
  cnt = wave_sum_i(cnt);
  if (lane == 0) sm.radix.wtot[0][wv] = (uint32_t)cnt;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wv; ++w) run += (int)sm.radix.wtot[0][w];
  for (int base = lo_i; base < hi_i; base += 64) {
    const int i = base + lane;
    const bool sel = i < hi_i && selected(i);
    const uint64_t bm = __ballot(sel);
    if (sel) emit(run + lanes_below(bm), i);
    run += __popcll(bm);
  }
  __syncthreads();
}

}  // namespace hisa
