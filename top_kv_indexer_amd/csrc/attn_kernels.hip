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
constexpr int kChunk = 512;  // row addresses staged in LDS at a time

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

template <int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn_mfma(KDims d, int splits, const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ local_kv,
                                                       const uint16_t* __restrict__ pooled_kv,
                                                       const int* __restrict__ I, const float* __restrict__ sinks,
                                                       const int* __restrict__ t0, uint16_t* __restrict__ out,
                                                       float* __restrict__ part) {
  constexpr int KPD = DK + 16;  // LDS row pitch: 8 banks of skew per row for the transposing reads
  constexpr int NT = NW * 64;
  constexpr int NS = DK / 32;   // MFMA k-steps of S
  constexpr int NO = DV / 16;   // MFMA column tiles of O^T
  constexpr int CPR = DK / 8;                       // 16-byte chunks per KV row
  constexpr int CPT = (kTile * CPR + NT - 1) / NT;  // chunks per thread per tile
  __shared__ __align__(16) uint16_t kv[kTile * KPD];
  __shared__ const uint16_t* s_ptr[kChunk];

  const int split = blockIdx.x, row = blockIdx.y;
  const int b = row / d.L, j = row % d.L;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int h0 = blockIdx.z * 16 * NW + wv * 16;
  const int T0 = t0[b];
  const RowPlan rp = row_plan(d, T0, j);
  const int per = (((rp.n_list + splits - 1) / splits) + kTile - 1) / kTile * kTile;
  const int begin = split * per, end = min(rp.n_list, begin + per);

  bf16x8 qf[NS];
  const uint16_t* qrow = q + ((size_t)row * d.H + h0 + c) * DK + g * 8;
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s] = *(const bf16x8*)(qrow + s * 32);

  float m = -INFINITY, l = 0.f;
  f32x4 acc[NO];
#pragma unroll
  for (int n = 0; n < NO; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int* Irow = I + (size_t)row * d.kI;
  for (int cb = begin; cb < end; cb += kChunk) {
    const int ce = min(end, cb + kChunk);
    // Row addresses of this chunk of the row list (local window, then I).
    __syncthreads();
    for (int e = cb + tid; e < ce; e += NT) {
      const uint16_t* p = nullptr;
      if (e < rp.n_loc) {
        p = local_kv + ((long long)b * d.Wl_cap + (rp.s_lo - rp.ls + e)) * DK;
      } else {
        const int id = Irow[e - rp.n_loc];
        if (id >= 0 && id < rp.V) p = pooled_kv + ((long long)b * d.Np_cap + id) * DK;
      }
      s_ptr[e - cb] = p;
    }
    __syncthreads();
    // Tiles of 32 rows; the next tile's rows are fetched into registers while
    // the current one is computed from LDS.
    uint4 reg[CPT];
    auto fetch = [&](int tb) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int ch = tid + i * NT;
        const int r = ch / CPR, seg = (ch % CPR) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ch < kTile * CPR && tb + r < ce) {
          const uint16_t* p = s_ptr[tb - cb + r];
          if (p) v = *(const uint4*)(p + seg);
        }
        reg[i] = v;
      }
    };
    fetch(cb);
    for (int tb = cb; tb < ce; tb += kTile) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int ch = tid + i * NT;
        if (ch < kTile * CPR) *(uint4*)(kv + (ch / CPR) * KPD + (ch % CPR) * 8) = reg[i];
      }
      __syncthreads();
      if (tb + kTile < ce) fetch(tb + kTile);

    // S^T[row][head] for the tile's 32 rows and the wave's 16 heads.
    f32x4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = *(const bf16x8*)(kv + (mt * 16 + c) * KPD + s * 32 + g * 8);
        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], st[mt], 0, 0, 0);
      }
    }
    // Lane (g, c) holds head c's scores of rows 4g+i (tile half 0) and 16+4g+i (half 1).
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * g + i;
        const bool live = tb + r < ce && s_ptr[tb - cb + r] != nullptr;
        const float v = live ? st[mt][i] * d.attn_scale_log2 : -INFINITY;
        x[mt * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // Lazy rescaling: the reference max m moves (and O, l are rescaled) only
    // when a head's scores exceed it by more than 2^8, so exp2(x - m) stays
    // <= 256 and the 128-register rescale of O is rare.
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
    if (m != -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = exp2f(x[i] - m);
        psum += p[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.f;
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l += psum;
    const bf16x8 pf = pack8(p);
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const uint16_t* base = kv + (4 * g + (c >> 2)) * KPD + n * 16 + 4 * (c & 3);
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
    uint16_t* orow = out + ((size_t)row * d.H + h) * DV + 4 * g;
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
    for (int n = 0; n < NO; ++n) *(f32x4*)(pr + n * 16 + 4 * g) = acc[n];
    if (g == 0) {
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
    float mf = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mf = fmaxf(mf, __shfl_xor(mf, o, 64));
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
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
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
  const dim3 grid(splits, d.B * d.L, d.H / 64);
  hipLaunchKernelGGL((k_attn_mfma<DK, DV, 4>), grid, dim3(256), 0, st, d, splits, (const uint16_t*)q,
                     (const uint16_t*)local_kv, (const uint16_t*)pooled_kv, I, sinks, t0, (uint16_t*)out, partial);
  return hipGetLastError();
}

}  // namespace

bool attn_mfma_ok(const KDims& d, bool bf16) {
  return bf16 && d.H % 64 == 0 && ((d.Dk == 512 && d.Dv == 512) || (d.Dk == 576 && d.Dv == 576));
}

bool attn_generic_ok(const KDims& d) {
  return d.Dk <= kGenericMaxDk && (long long)d.window + d.kI <= kGenericMaxList;
}

int attn_splits(const KDims& d, bool bf16) {
  if (!attn_mfma_ok(d, bf16)) return 1;
  const long long work = (long long)d.B * d.L * (d.H / 64);
  const long long n_max = (long long)min(d.window, d.Wl_cap) + d.kI;
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
