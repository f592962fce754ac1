// attn_kernels.hip -- sparse local + pooled attention with per-head sinks (gfx950).
//
// Method (HiSA issue, lablup/mlxcel #549, "Consuming the selection: sparse
// combine"; DSA issue, lablup/mlxcel #509, item 3): for query row j at t = t0+j,
// one softmax over the sliding-window local rows (t - window, t] and the pooled
// rows named by I[j] that are visible (0 <= id < V(t)), with the per-head sink
// logit in the normaliser; K = V, one KV head shared by all query heads.
//
// MFMA kernel (bf16): one workgroup per (query row, KV split, 64-head group).
// Each wave owns 16 heads.  KV rows are gathered straight from HBM into LDS,
// 32 rows per tile; S^T = K Q^T (16x16x32 MFMA, A = K rows from LDS, B = q in
// registers) leaves every lane with 8 scores of one head, so the online
// softmax runs in registers; O^T += V^T P^T takes V^T from LDS with the
// gfx950 transposing LDS read and P^T straight from the S^T registers.  Split
// partials (m, l, O) are merged by a second kernel.
#include <algorithm>

#include "hisa_device.h"

namespace hisa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTile = 32;
constexpr int kChunk = 512;  // rows of the row list staged in LDS at a time

struct RowPlan {
  bool ok;
  int Np, V, ls, s_lo, n_loc, n_list;
};

__device__ __forceinline__ RowPlan row_plan(const KDims& d, int T0, int j) {
  RowPlan r;
  const long long np = ((long long)T0 + d.L) / d.ratio;
  r.ls = max(0, T0 - d.window + 1);
  r.ok = T0 >= 0 && np <= d.Np_cap && (d.window == 0 || T0 + d.L - r.ls <= d.Wl_cap);
  r.Np = r.ok ? (int)np : 0;
  const int t = T0 + j;
  r.V = visible(t, d.ratio, r.Np);
  r.s_lo = max(r.ls, t - d.window + 1);
  r.n_loc = (r.ok && d.window > 0) ? t - r.s_lo + 1 : 0;
  r.n_list = r.ok ? r.n_loc + d.kI : 0;
  return r;
}

__device__ __forceinline__ bf16x8 pack8(const float (&p)[8]) {
  u32x4 u;
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = (uint32_t)f2bf(p[2 * k]) | ((uint32_t)f2bf(p[2 * k + 1]) << 16);
  return __builtin_bit_cast(bf16x8, u);
}

// One workgroup = NHG groups of 16 heads x 2 halves of the value width = 2*NHG
// waves.  Wave (hg, dh) computes the scores of rows 16*dh..16*dh+15 of each
// 32-row tile for its 16 heads; the pair exchanges them through LDS, both run
// the same online softmax over the 32 rows, and each accumulates O for its
// half of the value columns (16 heads x DV/2 = DV/8 accumulator registers).
template <int DK, int DV, int NHG>
__global__ __launch_bounds__(NHG * 128) void k_attn_mfma(KDims d, int splits, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ local_kv,
                                                         const uint16_t* __restrict__ pooled_kv,
                                                         const int* __restrict__ I, const float* __restrict__ sinks,
                                                         const int* __restrict__ t0, uint16_t* __restrict__ out,
                                                         float* __restrict__ part) {
  constexpr int NW = NHG * 2;
  constexpr int NT = NW * 64;
  constexpr int KPD = DK + 16;  // LDS row pitch: 8 banks of skew per row for the transposing reads
  constexpr int NS = DK / 32;   // MFMA k-steps of S
  constexpr int DVH = DV / 2;   // value columns per wave
  constexpr int NO = DVH / 16;  // MFMA column tiles of O^T per wave
  constexpr int SP = 17;        // padded pitch (floats) of the score exchange rows
  static_assert(kChunk % NT == 0, "chunk rows must split evenly over the threads");
  static_assert(kTile % NW == 0, "tile rows must split evenly over the waves");
  static_assert(DK >= 512 && DK <= 1024 && DK % 8 == 0, "a KV row is one or two 64-lane 16-byte loads");
  // Two LDS tiles: rows of the next tile stream in (global -> LDS, no
  // registers) while the current one is computed.
  __shared__ __align__(16) uint16_t kv[2][kTile * KPD];
  __shared__ float s_sc[NHG][kTile * SP];
  // Row list of the current chunk: element offset of each row (>= 0 into
  // pooled_kv, ~offset into local_kv) and whether the row is live.  Dead rows
  // point at a readable row of the same sequence and are masked in the softmax.
  __shared__ long long s_off[kChunk];
  __shared__ unsigned char s_live[kChunk];

  const int split = blockIdx.x, row = blockIdx.y;
  const int b = row / d.L, j = row % d.L;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int hg = wv >> 1, dh = wv & 1;
  const int h0 = blockIdx.z * 16 * NHG + hg * 16;
  // Row list: the kI pooled ids of I first, then `window` local slots (slot
  // s holds position s_lo + s while s < n_loc).  The split geometry does not
  // depend on t0, so the index loads below go out before t0 arrives.
  const int n_geo = d.kI + d.window;
  const int per = ((n_geo + splits - 1) / splits + kTile - 1) / kTile * kTile;
  const int begin = min(n_geo, split * per), end = min(n_geo, begin + per);
  const int* Irow = I + (size_t)row * d.kI;
  constexpr int IPT = kChunk / NT;
  int idpre[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const int e = begin + tid + u * NT;
    idpre[u] = (e < end && e < d.kI) ? Irow[e] : -1;
  }
  const int T0 = t0[b];
  const RowPlan rp = row_plan(d, T0, j);
  // a row every sequence with a live row may read (dead rows point at it)
  const long long dummy = rp.n_loc > 0 ? ~(((long long)b * d.Wl_cap + (rp.s_lo - rp.ls)) * DK)
                                       : (long long)b * d.Np_cap * DK;
  const bool any_row = rp.n_loc > 0 || rp.V > 0;

  bf16x8 qf[NS];
  const uint16_t* qrow = q + ((size_t)row * d.H + h0 + c) * DK + g * 8;
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = *(const bf16x8*)(qrow + s * 32);

  float m = -INFINITY, l = 0.f;
  f32x4 acc[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int cb = any_row ? begin : end; cb < end; cb += kChunk) {
    const int ce = min(end, cb + kChunk);
    const int cpad = cb + (ce - cb + kTile - 1) / kTile * kTile;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int e = cb + tid + u * NT;
      if (e < cpad) {
        long long off = dummy;
        bool live = false;
        if (e < ce) {
          if (e < d.kI) {
            const int id = cb == begin ? idpre[u] : Irow[e];
            if (id >= 0 && id < rp.V) {
              off = ((long long)b * d.Np_cap + id) * DK;
              live = true;
            }
          } else if (e - d.kI < rp.n_loc) {
            off = ~(((long long)b * d.Wl_cap + (rp.s_lo - rp.ls + e - d.kI)) * DK);
            live = true;
          }
        }
        s_off[e - cb] = off;
        s_live[e - cb] = live;
      }
    }
    __syncthreads();
    // Tiles of 32 rows in two LDS buffers.  Wave w moves rows w, w+NW, ...:
    // one 64-lane 16-byte global->LDS load per 512 columns of a row.
    auto load_tile = [&](int tb, int buf) {
#pragma unroll
      for (int rr = 0; rr < kTile / NW; ++rr) {
        const int r = wv + rr * NW;
        const long long off = s_off[tb - cb + r];
        const uint16_t* src = (off >= 0 ? pooled_kv + off : local_kv + ~off) + lane * 8;
        uint16_t* dst = &kv[buf][r * KPD];
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        if (DK > 512 && lane < DK / 8 - 64)
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + 512),
                                           (__attribute__((address_space(3))) void*)(dst + 512), 16, 0, 0);
      }
    };
    load_tile(cb, 0);
    for (int tb = cb, it = 0; tb < ce; tb += kTile, ++it) {
      const int buf = it & 1;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile `it` have landed
      __syncthreads();                // ... and every wave's; buffer buf^1 is free
      if (tb + kTile < ce) load_tile(tb + kTile, buf ^ 1);
      const uint16_t* kvb = kv[buf];

      // S^T for rows 16*dh .. 16*dh+15 and the wave's 16 heads.
      f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s0 = 0; s0 < NS; s0 += 4) {
        bf16x8 a4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s0 + u < NS) a4[u] = *(const bf16x8*)(kvb + (dh * 16 + c) * KPD + (s0 + u) * 32 + g * 8);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s0 + u < NS) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a4[u], qf[s0 + u], st, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s_sc[hg][(dh * 16 + 4 * g + i) * SP + c] = st[i];
      __syncthreads();
      // Lane (g, c) takes head c's scores of rows 4g+i and 16+4g+i.
      float x[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mt * 16 + 4 * g + i;
          const float v = s_live[tb - cb + r] ? s_sc[hg][r * SP + c] * d.attn_scale_log2 : -INFINITY;
          x[mt * 4 + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = max_rows(tmax);
      // Lazy rescaling: the reference max m moves (and O, l are rescaled) only
      // when a head's scores exceed it by more than 2^8, so exp2(x - m) stays
      // <= 256 and the rescale of O is rare.
      if (m == -INFINITY) {
        m = tmax;
      } else if (__ballot(tmax > m + 8.f)) {
        const float m_new = fmaxf(m, tmax);
        const float alpha = exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int n = 0; n < NO; ++n) {
          acc[n][0] *= alpha;
          acc[n][1] *= alpha;
          acc[n][2] *= alpha;
          acc[n][3] *= alpha;
        }
        m = m_new;
      }
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = m == -INFINITY ? 0.f : exp2f(x[i] - m);
        psum += p[i];
      }
      psum = sum_rows(psum);
      l += psum;
      const bf16x8 pf = pack8(p);
      // O^T[dv][h] += V^T[dv][rows] P^T[rows][h] over this wave's value half.
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        const uint16_t* base = kvb + (4 * g + (c >> 2)) * KPD + dh * DVH + n * 16 + 4 * (c & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * KPD));
        const i16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pf, acc[n], 0, 0, 0);
      }
    }
  }

  const int h = h0 + c;
  if (splits == 1) {
    const float sink2 = sinks ? sinks[h] * kLog2e : -INFINITY;
    const float mf = fmaxf(m, sink2);
    float f = 0.f;
    if (mf != -INFINITY) {
      const float lf = l * exp2f(m - mf) + (sinks ? exp2f(sink2 - mf) : 0.f);
      f = lf > 0.f ? exp2f(m - mf) / lf : 0.f;
    }
    uint16_t* orow = out + ((size_t)row * d.H + h) * DV + dh * DVH + 4 * g;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      uint2 v;
      v.x = (uint32_t)f2bf(acc[n][0] * f) | ((uint32_t)f2bf(acc[n][1] * f) << 16);
      v.y = (uint32_t)f2bf(acc[n][2] * f) | ((uint32_t)f2bf(acc[n][3] * f) << 16);
      *(uint2*)(orow + n * 16) = v;
    }
  } else {
    float* pr = part + (((size_t)split * d.B * d.L + row) * d.H + h) * (DV + 2);
#pragma unroll
    for (int n = 0; n < NO; ++n) *(f32x4*)(pr + dh * DVH + n * 16 + 4 * g) = acc[n];
    if (g == 0 && dh == 0) {
      pr[DV] = m;
      pr[DV + 1] = l;
    }
  }
}

// Merge of split partials (m and l in the log2 domain), sink included.  One
// workgroup per (query row, head, 128 output columns); the first wave turns
// the splits' (m, l) into normalised weights, then every thread sums its
// column over the splits.
constexpr int kMaxSplits = 64;

template <typename T>
__global__ __launch_bounds__(128) void k_attn_merge(KDims d, int splits, const float* __restrict__ part,
                                                    const float* __restrict__ sinks, T* __restrict__ out) {
  __shared__ float s_w[kMaxSplits];
  const int row = blockIdx.x, h = blockIdx.y;
  const int e = blockIdx.z * 128 + threadIdx.x;
  const size_t stride = (size_t)d.B * d.L * d.H * (d.Dv + 2);
  const float* p0 = part + ((size_t)row * d.H + h) * (d.Dv + 2);
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float m = s < splits ? p0[s * stride + d.Dv] : -INFINITY;
    const float l = s < splits ? p0[s * stride + d.Dv + 1] : 0.f;
    const float sink2 = sinks ? sinks[h] * kLog2e : -INFINITY;
    float mf = wave_max(m);
    mf = fmaxf(mf, sink2);
    const float wgt = (mf == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - mf);
    float lf = wave_sum(l * wgt);
    if (sinks && mf != -INFINITY) lf += exp2f(sink2 - mf);
    const float inv = lf > 0.f ? 1.f / lf : 0.f;
    s_w[s] = wgt * inv;
  }
  __syncthreads();
  if (e >= d.Dv) return;
  float o = 0.f;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) o += p0[s * stride + e] * s_w[s];
  stf(out + ((size_t)row * d.H + h) * d.Dv + e, o);
}

// Any shape / dtype: one workgroup per (query row, head), two-pass softmax.
constexpr int kGenericMaxList = 4096;
constexpr int kGenericMaxDk = 1024;

template <typename T>
__global__ __launch_bounds__(256) void k_attn_valu(KDims d, const T* __restrict__ q, const T* __restrict__ local_kv,
                                                   const T* __restrict__ pooled_kv, const int* __restrict__ I,
                                                   const float* __restrict__ sinks, const int* __restrict__ t0,
                                                   T* __restrict__ out) {
  __shared__ float s_x[kGenericMaxList];
  __shared__ int s_row[kGenericMaxList];
  __shared__ float s_q[kGenericMaxDk];
  __shared__ float s_red[4];
  const int row = blockIdx.x, h = blockIdx.y;
  const int b = row / d.L, j = row % d.L, tid = threadIdx.x;
  const RowPlan rp = row_plan(d, t0[b], j);
  const int n = rp.n_list;
  const float scale = 1.0f / sqrtf((float)d.Dk);
  for (int e = tid; e < d.Dk; e += 256) s_q[e] = ldf(q + ((size_t)row * d.H + h) * d.Dk + e) * scale;
  // s_row: >= 0 pooled id, <= -2 local row -(r + 2), -1 masked
  for (int e = tid; e < n; e += 256) {
    int code = -1;
    if (e < rp.n_loc) code = -((rp.s_lo - rp.ls + e) + 2);
    else {
      const int id = I[(size_t)row * d.kI + e - rp.n_loc];
      if (id >= 0 && id < rp.V) code = id;
    }
    s_row[e] = code;
  }
  __syncthreads();
  auto row_ptr = [&](int code) -> const T* {
    return code >= 0 ? pooled_kv + ((size_t)b * d.Np_cap + code) * d.Dk
                     : local_kv + ((size_t)b * d.Wl_cap + (-code - 2)) * d.Dk;
  };
  float mx = sinks ? sinks[h] : -INFINITY;
  for (int e = tid; e < n; e += 256) {
    float x = -INFINITY;
    const int code = s_row[e];
    if (code != -1) {
      const T* kp = row_ptr(code);
      float acc = 0.f;
      for (int k = 0; k < d.Dk; ++k) acc += s_q[k] * ldf(kp + k);
      x = acc;
    }
    s_x[e] = x;
    mx = fmaxf(mx, x);
  }
  mx = wave_max(mx);
  if (lane_id() == 0) s_red[wave_id()] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  T* orow = out + ((size_t)row * d.H + h) * d.Dv;
  if (mx == -INFINITY) {
    for (int e = tid; e < d.Dv; e += 256) stf(orow + e, 0.f);
    return;
  }
  float z = 0.f;
  for (int e = tid; e < n; e += 256) {
    const float pe = s_x[e] == -INFINITY ? 0.f : expf(s_x[e] - mx);
    s_x[e] = pe;
    z += pe;
  }
  z = wave_sum(z);
  if (lane_id() == 0) s_red[wave_id()] = z;
  __syncthreads();
  z = s_red[0] + s_red[1] + s_red[2] + s_red[3] + (sinks ? expf(sinks[h] - mx) : 0.f);
  const float inv = 1.f / z;
  for (int e = tid; e < d.Dv; e += 256) {
    float o = 0.f;
    for (int r = 0; r < n; ++r) {
      const int code = s_row[r];
      if (code != -1) o += s_x[r] * ldf(row_ptr(code) + e);
    }
    stf(orow + e, o * inv);
  }
}

template <int DK, int DV>
hipError_t launch_mfma(const KDims& d, const void* q, const void* local_kv, const void* pooled_kv, const int* I,
                       const float* sinks, const int* t0, void* out, float* partial, int splits, hipStream_t st) {
  if (attn_small_groups(d)) {
    const dim3 grid(splits, d.B * d.L, d.H / 16);
    hipLaunchKernelGGL((k_attn_mfma<DK, DV, 1>), grid, dim3(128), 0, st, d, splits, (const uint16_t*)q,
                       (const uint16_t*)local_kv, (const uint16_t*)pooled_kv, I, sinks, t0, (uint16_t*)out, partial);
  } else {
    const dim3 grid(splits, d.B * d.L, d.H / 64);
    hipLaunchKernelGGL((k_attn_mfma<DK, DV, 4>), grid, dim3(512), 0, st, d, splits, (const uint16_t*)q,
                       (const uint16_t*)local_kv, (const uint16_t*)pooled_kv, I, sinks, t0, (uint16_t*)out, partial);
  }
  return hipGetLastError();
}

}  // namespace

bool attn_mfma_ok(const KDims& d, bool bf16) {
  return bf16 && d.H % 64 == 0 && ((d.Dk == 512 && d.Dv == 512) || (d.Dk == 576 && d.Dv == 576));
}

bool attn_generic_ok(const KDims& d) {
  return d.Dk <= kGenericMaxDk && (long long)d.window + d.kI <= kGenericMaxList;
}

// A handful of query rows: 16 heads per workgroup (more, smaller workgroups);
// otherwise 64 heads per workgroup, so each gathered row feeds 4x more heads.
bool attn_small_groups(const KDims& d) { return (long long)d.B * d.L * (d.H / 64) <= 8; }

int attn_splits(const KDims& d, bool bf16) {
  if (!attn_mfma_ok(d, bf16)) return 1;
  const long long work = (long long)d.B * d.L * (d.H / (attn_small_groups(d) ? 16 : 64));
  const long long n_max = (long long)d.window + d.kI;
  // at least two 32-row tiles per split, so that fetching overlaps compute
  const long long max_splits = std::max(1LL, (n_max + 2 * kTile - 1) / (2 * kTile));
  long long want = (256 + work - 1) / work;
  want = std::min(want, std::min(max_splits, (long long)kMaxSplits));
  return (int)std::max(1LL, want);
}

size_t attn_partial_bytes(const KDims& d, int splits) {
  if (splits <= 1) return 0;
  return (size_t)splits * d.B * d.L * d.H * (d.Dv + 2) * sizeof(float);
}

hipError_t launch_attention_merge(const KDims& d, bool bf16, const float* partial, const float* sinks, void* out,
                                  int splits, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(k_attn_merge<uint16_t>, dim3(d.B * d.L, d.H, (d.Dv + 127) / 128), dim3(128), 0, st, d, splits,
                       partial, sinks, (uint16_t*)out);
  else
    hipLaunchKernelGGL(k_attn_merge<float>, dim3(d.B * d.L, d.H, (d.Dv + 127) / 128), dim3(128), 0, st, d, splits,
                       partial, sinks, (float*)out);
  return hipGetLastError();
}

hipError_t launch_attention(const KDims& d, bool bf16, const void* q, const void* local_kv, const void* pooled_kv,
                            const int* I, const float* sinks, const int* t0, void* out, float* partial, int splits,
                            hipStream_t st) {
  if (attn_mfma_ok(d, bf16)) {
    if (d.Dk == 512)
      return launch_mfma<512, 512>(d, q, local_kv, pooled_kv, I, sinks, t0, out, partial, splits, st);
    return launch_mfma<576, 576>(d, q, local_kv, pooled_kv, I, sinks, t0, out, partial, splits, st);
  }
  const dim3 grid(d.B * d.L, d.H);
  if (bf16)
    hipLaunchKernelGGL(k_attn_valu<uint16_t>, grid, dim3(256), 0, st, d, (const uint16_t*)q,
                       (const uint16_t*)local_kv, (const uint16_t*)pooled_kv, I, sinks, t0, (uint16_t*)out);
  else
    hipLaunchKernelGGL(k_attn_valu<float>, grid, dim3(256), 0, st, d, (const float*)q, (const float*)local_kv,
                       (const float*)pooled_kv, I, sinks, t0, (float*)out);
  return hipGetLastError();
}

}  // namespace hisa
