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
// partials (O / l in bf16, then m and l) are merged by a second kernel.
#include <algorithm>
#include <type_traits>

#include "hisa_device.h"

namespace hisa {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;

constexpr int kTile = 32;


// One workgroup = HW = 16*NHG heads of one query row (one KV split), NW =
// 2*NHG waves; KV tiles of 32 rows stream through a ring of NBUF LDS slots.
// Step t of the tile loop:
//  - scores of tile t+1: wave (hg, dh) computes S^T for rows 16*dh..+15 and
//    heads 16*hg..+15 (16x16x32 MFMA, A = K rows from LDS, B = q in
//    registers) into one of two score buffers;
//  - softmax of tile t (scores stored in step t-1): wave w owns heads
//    8w..8w+7 (m, l and the lazy rescale) and stores P in bf16 plus each
//    head's rescale factor;
//  - values of tile t: wave w accumulates O^T for every head of the group
//    over its own 16-column tiles of the value width (A = V^T from the gfx950
//    transposing LDS read, B = P^T), so each value column is read from LDS
//    once;
//  - the rows of tile t+NBUF-1 start streaming from global memory into LDS
//    (issued through inline assembly, so LDS reads of the other slots never
//    wait for them).
// LDS rows are a whole number of 256-byte bank rounds with the first 64
// 16-byte chunks XOR-swizzled by the row (slot position p holds chunk
// p ^ sw(row)), so the K reads (16 rows x one chunk) and the transposing V
// reads (8 rows x two chunks per half-wave) hit distinct banks.  Row
// bookkeeping is resolved once per chunk of up to 1024 rows into LDS: a
// 32-bit row code per entry (pooled row, or local row) and a 32-bit liveness
// mask per tile; wave w fetches rows RPW*w .. RPW*w + RPW-1 of each tile.
template <int DK, int DV, int NHG>
__global__ __launch_bounds__(NHG * 128) void k_attn_mfma(KDims d, int splits, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ local_kv,
                                                         const uint16_t* __restrict__ pooled_kv,
                                                         const int* __restrict__ I, const float* __restrict__ sinks,
                                                         const int* __restrict__ t0, uint16_t* __restrict__ out,
                                                         float* __restrict__ part) {
  constexpr int NW = NHG * 2;
  constexpr int NT = NW * 64;
  constexpr int HW = NHG * 16;          // heads of the workgroup
  constexpr int KPD = (DK * 2 + 255) / 256 * 128;  // LDS row pitch (elements)
  constexpr int NBUF = DK <= 512 ? 4 : 3;          // ring slots
  constexpr int NS = DK / 32;           // MFMA k-steps of S
  constexpr int NDT_ALL = DV / 16;      // 16-column tiles of the value width
  constexpr int NDT = (NDT_ALL + NW - 1) / NW;  // ... per wave (tiles w, w+NW, ...)
  constexpr int SSP = kTile + 4;        // score rows (floats) per head in LDS
  constexpr int PSP = kTile;            // P entries (bf16) per head in LDS
  constexpr int RPW = kTile / NW;       // rows of a tile each wave fetches
  constexpr int CH = 1024;              // rows of the row list resolved at a time
  constexpr int NTILE = CH / kTile;
  constexpr int IPT = CH / NT;          // chunk rows per thread
  constexpr int LPT = RPW * (DK > 512 ? 2 : 1);  // vector-memory loads per tile per wave
  constexpr int KW = 8;                 // K fragments in flight
  constexpr int OP = DV + 8;            // pitch of the staged output rows (elements)
  static_assert(HW * OP <= NBUF * kTile * KPD && HW <= 2 * kTile, "staging fits the ring");
  static_assert(RPW % 4 == 0 && CH % NT == 0, "row codes are read four at a time; a chunk splits over threads");
  static_assert(HW == 8 * NW, "each wave owns the softmax of 8 heads");
  static_assert(DV % 16 == 0 && DK >= 512 && DK <= 1024 && DK % 32 == 0, "shape");
  __shared__ __align__(1024) uint16_t kv[NBUF][kTile * KPD];
  __shared__ __align__(16) float s_sc[2][HW * SSP];
  __shared__ __align__(16) uint16_t s_p[HW * PSP];
  __shared__ __align__(16) float s_alpha[HW];
  __shared__ float s_ml[2][HW];
  __shared__ uint32_t s_tmask[NTILE];
  __shared__ __align__(16) int s_code[CH];  // row code of each entry of the current chunk

  // few, latency-bound workgroups: every argument in scalar registers at once
  if constexpr (NHG == 1) args_now(d, splits, q, local_kv, pooled_kv, I, sinks, t0, out, part);
  const int split = blockIdx.x;
  // consecutive query rows go to the same XCD (workgroups are dealt to the 8
  // XCDs round-robin), so rows sharing their local window share its L2
  const int row = [](int y, int n) {
    const int x = y & 7, qn = n >> 3, rn = n & 7;
    return x * qn + min(x, rn) + (y >> 3);
  }(blockIdx.y, d.B * d.L);
  const int b = row / d.L, j = row % d.L;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int wvs = __builtin_amdgcn_readfirstlane(wv);  // the wave index, known to be uniform
  const int hg = wv >> 1, dh = wv & 1;
  const int hbase = blockIdx.z * HW;
  const uint32_t kv_lds = lds_addr(&kv[0][0]);
  // Row swizzle of the 16-byte chunks (0..15, by the row within 16): spreads
  // the 16 rows of a key read (one chunk each) over distinct slots and the
  // row pairs of a transposing value read over distinct chunk pairs.  The
  // LDS hashes address bits 12 and 13 into bit 4 (slot bit 0); with 1 KiB
  // rows from a 1 KiB-aligned base that bit of the row's address is folded
  // in.  (1280-byte rows cross those bits inside a row and differently per
  // ring slot; there the plain swizzle is kept.)
  const int kvb10 = (int)((kv_lds >> 10) & 15);
  auto sw = [kvb10](int r) {
    const int t = kvb10 + (r & 15);
    const int hash = KPD * 2 == 1024 ? ((t >> 2) ^ (t >> 3)) & 1 : 0;
    return (((r & 7) << 1) | ((r >> 3) & 1)) ^ hash;
  };
  // scores: this wave's 16 heads of q as the B operand.  With 64 heads the
  // workgroup's head rows (contiguous in q) come in through the last two ring
  // slots, one 1 KiB global->LDS load per row (swizzled like the KV rows);
  // with 16 heads straight into registers.
  bf16x8 qf[NS];
  auto issue_q = [&]() {
    // HW <= 64 rows span ring slots NBUF-2 and NBUF-1
    const uint16_t* qg = q + ((size_t)row * d.H + hbase) * DK;
#pragma unroll
    for (int u = 0; u < HW / NW; ++u) {
      const int h = wv + NW * u;
      const uint32_t dst = kv_lds + (uint32_t)(((NBUF - 2) * kTile + h) * KPD * 2);
      g2lds16(qg + (size_t)h * DK + (lane ^ sw(h)) * 8, dst);
      if (DK > 512 && (lane ^ sw(h)) < DK / 8 - 64) g2lds16(qg + (size_t)h * DK + 512 + (lane ^ sw(h)) * 8, dst + 1024);
    }
  };
  // q fragments from LDS, once every wave's rows have landed (the caller has
  // waited for its own q loads)
  auto read_q = [&]() {
    __syncthreads();
    const uint16_t* qs = kv[NBUF - 2];
    const int hr = hg * 16 + c;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ch = 4 * s + g;
      qf[s] = *(const bf16x8*)(qs + hr * KPD + tail_pos(ch, sw(c)) * 8);
    }
    __syncthreads();  // slots NBUF-2 and NBUF-1 are free again
  };
  // Row list: the kI pooled ids of I first, then `window` local slots (slot
  // s holds position s_lo + s while s < n_loc).  The split geometry does not
  // depend on t0, so the index loads below go out before t0 arrives.
  const int n_geo = d.kI + d.window;
  const int per = ((n_geo + splits - 1) / splits + kTile - 1) / kTile * kTile;
  const int begin = min(n_geo, split * per), end = min(n_geo, begin + per);
  // no index list (I == NULL): entry e names pooled row e (dense attention)
  const int* Irow = I ? I + (size_t)row * d.kI : nullptr;
  auto id_at = [&](int e) { return Irow ? Irow[e] : e; };
  auto ident_row = [&](int u) { return tid + u * NT; };
  int id_a[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const int ea = begin + ident_row(u);
    id_a[u] = (ea < end && ea < d.kI) ? id_at(ea) : -1;
  }
  // issued before q, so waiting for it does not wait for q
  const int T0 = t0[__builtin_amdgcn_readfirstlane(b)];
  const int S0 = ring_slot0(d, __builtin_amdgcn_readfirstlane(b), T0);
  // q is requested right after the ids and t0, so its latency overlaps
  // theirs and the row bookkeeping waits only for them
  if constexpr (NHG >= 4) {
    issue_q();  // many heads per row: staged through LDS (read below)
  } else {
    const uint16_t* qrow = q + ((size_t)row * d.H + hbase + hg * 16 + c) * DK + g * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const bf16x8*)(qrow + s * 32);
  }
  // values: O^T tiles (16 value columns x 16 heads) of every head tile
  f32x4 acc[NDT][NHG];
#pragma unroll
  for (int n = 0; n < NDT; ++n)
#pragma unroll
    for (int ht = 0; ht < NHG; ++ht) acc[n][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  // softmax: lane (hq, rq) = (lane >> 3, lane & 7) holds rows 4rq..4rq+3 of head 8*wv + hq
  const int hq = lane >> 3, rq = lane & 7;
  const int hs = 8 * wv + hq;
  float m = -INFINITY, l = 0.f;
  const float scale = d.attn_scale_log2;
  // transposing V reads: lane (g, c) takes rows 4g + c/4 (+16) and columns
  // 4*(c%4) .. +3 of a 16-column value tile
  const int vrow = 4 * g + (c >> 2);
  const int vsw = sw(vrow);  // rows vrow and vrow + 16 share the swizzle
  auto vaddr = [&](int dt, int hi) {
    const int ch = 2 * dt + ((c & 3) >> 1);
    return (vrow + 16 * hi) * KPD + tail_pos(ch, vsw) * 8 + 4 * (c & 1);
  };
  // This lane's LDS element offsets inside a ring slot for the K reads of
  // every MFMA k-step and the V reads of every value tile it owns, and of
  // its 16-byte piece of each tile row the wave fetches.  They depend on the
  // lane alone.  With 16 heads (few, latency-bound workgroups) they are
  // pinned here, while the loads above are in flight, instead of being
  // computed where the compiler hoists them (after the waits); with 64 heads
  // they are formed at each use, as the compiler prefers.
  int k_el[NS], v_el[NDT][2], src_el[RPW];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int ch = 4 * s + g;
    k_el[s] = (dh * 16 + c) * KPD + tail_pos(ch, sw(c)) * 8;
    if constexpr (NHG == 1) asm volatile("" : "+v"(k_el[s]));
  }
#pragma unroll
  for (int n = 0; n < NDT; ++n)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      v_el[n][hi] = vaddr(wv + NW * n, hi);
      if constexpr (NHG == 1) asm volatile("" : "+v"(v_el[n][hi]));
    }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    src_el[r] = (lane ^ sw(RPW * wvs + r)) * 8;
    if constexpr (NHG == 1) asm volatile("" : "+v"(src_el[r]));
  }
  const RowPlan rp = row_plan(d, T0, S0, j);
  // a row every sequence with a live row may read (dead rows point at it)
  const int dummy = rp.n_loc > 0 ? -1 - rp.lbase : 0;
  const bool any_row = rp.n_loc > 0 || rp.V > 0;
  // liveness and row code of list entry e (given its pooled id when e < kI):
  // code >= 0 is pooled row `code`, code < 0 local row -1 - code
  auto resolve = [&](int e, int id, int& code) -> bool {
    code = dummy;
    if (e >= end) return false;
    if (e < d.kI) {
      if (id < 0 || id >= rp.V) return false;
      code = id;
      return true;
    }
    if (e - d.kI >= rp.n_loc) return false;
    code = -1 - local_row(d, rp, e - d.kI);
    return true;
  };
  if constexpr (NHG >= 4) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: q (and the ids) are in
    read_q();
  }

  for (int cb = any_row ? begin : end; cb < end; cb += CH) {
    const int ce = min(end, cb + CH);
    const int ntile = (ce - cb + kTile - 1) / kTile;
    __syncthreads();  // the previous chunk is done with every slot, code and mask
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      if (cb + u * NT >= ce) break;  // whole tiles past the chunk's end: never read
      const int ea = cb + ident_row(u);
      const int id = cb == begin ? id_a[u] : (ea < end && ea < d.kI ? id_at(ea) : -1);
      int code;
      const uint64_t live = __ballot(resolve(ea, id, code));
      s_code[ident_row(u)] = code;
      if (lane == 0) {
        const int t = (wv * 64 + u * NT) / kTile;
        s_tmask[t] = (uint32_t)live;
        s_tmask[t + 1] = (uint32_t)(live >> 32);
      }
    }
    __syncthreads();  // every row code of the chunk is in
    // Tile t, wave w: tile rows RPW*w .. RPW*w + RPW-1.  Their codes come
    // from LDS in one broadcast read per four rows.
    const uint16_t* pooled_b = pooled_kv + (size_t)b * d.Np_cap * DK;
    const uint16_t* local_b = local_kv + (size_t)b * d.Wl_cap * DK;
    // With 16 heads (16 rows per wave per tile) the code reads use a
    // lane-varying (always zero) offset, so the codes stay in vector
    // registers instead of being moved to scalar ones row by row; with 64
    // heads (4 rows) the scalar unit, idle there, forms the addresses.  LDS
    // destinations are plain 32-bit offsets from the ring's base.
    const int vz = NHG == 1 ? vector_zero() : 0;
    auto load_tile = [&](int t, int slot) {
      int4 code4[RPW / 4];
#pragma unroll
      for (int q4 = 0; q4 < RPW / 4; ++q4) code4[q4] = *(const int4*)&s_code[t * kTile + RPW * wvs + 4 * q4 + vz];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int4 c4 = code4[r >> 2];
        const int cd = (r & 3) == 0 ? c4.x : (r & 3) == 1 ? c4.y : (r & 3) == 2 ? c4.z : c4.w;
        const bool pooled = cd >= 0;
        const uint16_t* src = (pooled ? pooled_b : local_b) + (size_t)(uint32_t)(pooled ? cd : -1 - cd) * DK;
        const int trow = RPW * wvs + r;
        const uint32_t dst = kv_lds + (uint32_t)((slot * kTile + trow) * KPD * 2);
        g2lds16(src + (NHG == 1 ? src_el[r] : (lane ^ sw(trow)) * 8), dst);
        if (DK > 512 && (lane ^ sw(trow)) < DK / 8 - 64) g2lds16(src + 512 + (lane ^ sw(trow)) * 8, dst + 1024);
      }
    };
    auto load_k = [&](const uint16_t* kvb, int s) {  // k-step s of rows 16*dh + c
      if constexpr (NHG == 1) return *(const bf16x8*)(kvb + k_el[s]);
      const int ch = 4 * s + g;
      return *(const bf16x8*)(kvb + (dh * 16 + c) * KPD + tail_pos(ch, sw(c)) * 8);
    };
    // S^T of rows 16*dh.. for heads 16*hg.. into score buffer sb; the first
    // KW fragments arrive in ka, the rest are fetched KW steps ahead
    auto scores = [&](const uint16_t* kvb, bf16x8 (&ka)[KW], int sb) {
      // 16 heads (one wave per SIMD, latency-bound): four independent MFMA
      // chains; 64 heads: one (the other waves hide its latency)
      constexpr int NACC = NHG == 1 ? 4 : 1;
      f32x4 sa[NACC];
#pragma unroll
      for (int u = 0; u < NACC; ++u) sa[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = ka[s % KW];
        if (s + KW < NS) ka[s % KW] = load_k(kvb, s + KW);
        sa[s % NACC] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sa[s % NACC], 0, 0, 0);
      }
      f32x4 st = sa[0];
#pragma unroll
      for (int u = 1; u < NACC; ++u) st += sa[u];
      *(f32x4*)&s_sc[sb][(hg * 16 + c) * SSP + dh * 16 + 4 * g] = st;
    };
    // wait until at most `keep` tiles' loads of this wave are still in flight
    auto wait_loads = [&](int keep) {
      if (keep >= 2) __builtin_amdgcn_s_waitcnt((2 * LPT & 15) | ((2 * LPT >> 4) << 14) | 0x0F70);
      else if (keep == 1) __builtin_amdgcn_s_waitcnt((LPT & 15) | ((LPT >> 4) << 14) | 0x0F70);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
    };
    auto step = [&](int t) {
      const uint16_t* kvP = kv[t % NBUF];
      const uint16_t* kvS = kv[(t + 1) % NBUF];
      // tile t+1 must have landed; tiles t+2 .. t+NBUF-2 may still stream in
      wait_loads(min(ntile - 1, t + NBUF - 2) - (t + 1));
      lds_sync();  // every wave's tile t+1, scores of tile t, and the slot of tile t+NBUF-1 are ready
      if (t + NBUF - 1 < ntile) load_tile(t + NBUF - 1, (t + NBUF - 1) % NBUF);
      const uint32_t tmask = __builtin_amdgcn_readfirstlane(s_tmask[t]);
      const bool more = t + 1 < ntile;
      const f32x4 sv = *(const f32x4*)&s_sc[t & 1][hs * SSP + 4 * rq];
      bf16x8 ka[KW];
      if (more) {
#pragma unroll
        for (int s = 0; s < KW; ++s) ka[s] = load_k(kvS, s);
      }
      if (more) scores(kvS, ka, (t + 1) & 1);
      // softmax of head hs over rows 4rq..4rq+3 of tile t (8 lanes per head)
      {
        const uint32_t lbits = tmask >> (4 * rq);
        float x[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = ((lbits >> i) & 1u) ? sv[i] * scale : -INFINITY;
          tmax = fmaxf(tmax, x[i]);
        }
        tmax = max_span8(tmax);
        // Lazy rescaling: the reference max m moves (and O, l are rescaled)
        // only when a head's scores exceed it by more than 2^8, so exp2(x - m)
        // stays <= 256 and the rescale of O is rare.
        float alpha = 1.f;
        if (m == -INFINITY) {
          m = tmax;
        } else if (tmax > m + 8.f) {
          const float m_new = fmaxf(m, tmax);
          alpha = __builtin_amdgcn_exp2f(m - m_new);
          l *= alpha;
          m = m_new;
        }
        const float m_sub = m == -INFINITY ? 0.f : m;  // exp2(-inf) = 0 while a head has no live score
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_sub);
        l += sum_span(p[0] + p[1] + p[2] + p[3], 8);
        // P^T operand order: head row of 32 entries, entry 8*gg + e holds
        // tile row 16*(e/4) + 4*gg + e%4.
        uint2 pk;
        pk.x = pack_bf16x2(p[0], p[1]);
        pk.y = pack_bf16x2(p[2], p[3]);
        // 16-byte chunk j of head row h sits at chunk j ^ ((h >> 2) & 3), so
        // the operand reads below (rows c, c+4, c+8, c+12 at once) and these
        // writes are bank-conflict free
        *(uint2*)&s_p[hs * PSP + (((rq & 3) ^ ((hs >> 2) & 3)) * 8) + (rq >> 2) * 4] = pk;
        if (rq == 0) s_alpha[hs] = alpha;
      }
      lds_sync();
      // O^T[dv][h] += V^T[dv][rows] P^T[rows][h] over this wave's value tiles
      float al[NHG];
      bool any = false;
#pragma unroll
      for (int ht = 0; ht < NHG; ++ht) {
        al[ht] = s_alpha[ht * 16 + c];
        any |= al[ht] != 1.f;
      }
      bf16x8 pb[NHG];
#pragma unroll
      for (int ht = 0; ht < NHG; ++ht) pb[ht] = *(const bf16x8*)&s_p[(ht * 16 + c) * PSP + ((g ^ ((c >> 2) & 3)) * 8)];
      i16x4 va[NDT][2];
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const int dt = wv + NW * n;
        if (NDT * NW == NDT_ALL || dt < NDT_ALL) {
          va[n][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kvP + (NHG == 1 ? v_el[n][0] : vaddr(dt, 0))));
          va[n][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kvP + (NHG == 1 ? v_el[n][1] : vaddr(dt, 1))));
        }
      }
      if (__ballot(any)) {
#pragma unroll
        for (int n = 0; n < NDT; ++n)
#pragma unroll
          for (int ht = 0; ht < NHG; ++ht) {
            acc[n][ht][0] *= al[ht];
            acc[n][ht][1] *= al[ht];
            acc[n][ht][2] *= al[ht];
            acc[n][ht][3] *= al[ht];
          }
      }
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const int dt = wv + NW * n;
        if (NDT * NW == NDT_ALL || dt < NDT_ALL) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va[n][0], va[n][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int ht = 0; ht < NHG; ++ht)
            acc[n][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[ht], acc[n][ht], 0, 0, 0);
        }
      }
    };
    // prologue: tiles 0 .. NBUF-2 in flight, scores of tile 0
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
      if (t < ntile) load_tile(t, t);
    wait_loads(min(ntile, NBUF - 1) - 1);
    lds_sync();
    {
      bf16x8 ka[KW];
#pragma unroll
      for (int s = 0; s < KW; ++s) ka[s] = load_k(kv[0], s);
      scores(kv[0], ka, 0);
    }
    for (int t = 0; t < ntile; ++t) step(t);
  }

  // Per-head (m, l) from the softmax owners to every value wave.
  if (rq == 0) {
    s_ml[0][hs] = m;
    s_ml[1][hs] = l;
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < NHG; ++ht) {
    const int hl = ht * 16 + c, h = hbase + hl;
    const float mh = s_ml[0][hl], lh = s_ml[1][hl];
    if (splits == 1) {
      const float sink2 = sinks ? sinks[h] * kLog2e : -INFINITY;
      const float mf = fmaxf(mh, sink2);
      float f = 0.f;
      if (mf != -INFINITY) {
        const float lf = lh * exp2f(mh - mf) + (sinks ? exp2f(sink2 - mf) : 0.f);
        f = lf > 0.f ? exp2f(mh - mf) / lf : 0.f;
      }
      // staged in the (now idle) ring: head row hl, padded pitch OP
      uint16_t* orow = &kv[0][0] + hl * OP + 4 * g;
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const int dt = wv + NW * n;
        if (NDT * NW == NDT_ALL || dt < NDT_ALL) {
          uint2 v;
          v.x = pack_bf16x2(acc[n][ht][0] * f, acc[n][ht][1] * f);
          v.y = pack_bf16x2(acc[n][ht][2] * f, acc[n][ht][3] * f);
          *(uint2*)(orow + dt * 16) = v;
        }
      }
    } else {
      const size_t prow = ((size_t)split * d.B * d.L + row) * d.H + h;
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const int dt = wv + NW * n;
        if (NDT * NW == NDT_ALL || dt < NDT_ALL) store_part4(part, prow, DV, dt * 16 + 4 * g, acc[n][ht], inv);
      }
      if (wv == 0 && g == 0) store_part_ml(part, prow, DV, mh, lh);
    }
  }
  if (splits == 1) {
    // The group's HW heads are contiguous in out: copy the staged rows out in
    // 16-byte pieces, whole 128-byte lines per wave instruction.
    __syncthreads();
    uint16_t* og = out + ((size_t)row * d.H + hbase) * DV;
    constexpr int CPR = DV / 8;  // 16-byte pieces per head row
    for (int k = tid; k < HW * CPR; k += NT) {
      const int hr = k / CPR, cc = k - hr * CPR;
      *(u32x4*)(og + (size_t)k * 8) = *(const u32x4*)(&kv[0][0] + hr * OP + cc * 8);
    }
  }
}

// Many query rows (prefill; no split): one workgroup per (query row, 64
// heads), four waves, and wave w owns heads 16w .. 16w+15 from end to end,
// in the manner of flash attention with the heads in the place of query
// rows.  Per 32-row tile: S = K q^T for its heads as two 16-row MFMA blocks
// (lane (g, c) holds rows 4g+i and 16+4g+i of head c), the online softmax in
// registers (row max and sum over the four lanes of a head by lane swaps),
// and O^T += V^T P^T where P^T is the lane's own eight probabilities: the
// value MFMA's k order (entry 8g+e <-> tile row 16*(e/4) + 4g + e%4) is the
// score layout, so nothing moves between lanes or waves.  The only barrier
// per tile makes the tile's rows (fetched by all four waves, global->LDS)
// visible and frees the ring slot of the tile NBUF-1 ahead.
template <int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void k_attn_fa(KDims d, const uint16_t* __restrict__ q,
                                                                      const uint16_t* __restrict__ local_kv,
                                                                      const uint16_t* __restrict__ pooled_kv,
                                                                      const int* __restrict__ I,
                                                                      const float* __restrict__ sinks,
                                                                      const int* __restrict__ t0,
                                                                      uint16_t* __restrict__ out) {
  constexpr int NT = NW * 64, HW = NW * 16;
  constexpr int KPD = (DK * 2 + 255) / 256 * 128;  // LDS row pitch (elements)
  constexpr int NBUF = 2;                          // ring slots (LDS for two workgroups per CU at 512 wide)
  constexpr int NS = DK / 32;                      // MFMA k-steps of S
  constexpr int NDT = DV / 16;                     // 16-column value tiles (all of them, every wave)
  constexpr int RPW = kTile / NW;                  // rows of a tile each wave fetches
  constexpr int CH = 1024;                         // rows of the row list resolved at a time
  constexpr int NTILE = CH / kTile;
  constexpr int IPT = CH / NT;
  constexpr int LPT = RPW * (DK > 512 ? 2 : 1);    // vector-memory loads per tile per wave
  constexpr int KW = 4;                            // K fragments in flight (both row blocks)
  constexpr int NACC = 2;                          // accumulation chains per row block
  constexpr int PVG = 8;                           // value tiles whose reads are in flight together
  constexpr int OP = DV + 8;                       // pitch of the staged output rows (elements)
  static_assert(32 * OP <= NBUF * kTile * KPD, "32 heads' staging fits the ring");
  static_assert(RPW % 4 == 0 && CH % NT == 0, "shape of the row fetch");
  static_assert(DV % 16 == 0 && DV <= DK && DK >= 512 && DK <= 1024 && DK % 32 == 0, "shape");
  __shared__ __align__(1024) uint16_t kv[NBUF][kTile * KPD];
  __shared__ uint32_t s_tmask[NTILE];
  __shared__ __align__(16) int s_code[CH];

  const int row = [](int y, int n) {  // consecutive query rows on one XCD (shared local window)
    const int x = y & 7, qn = n >> 3, rn = n & 7;
    return x * qn + min(x, rn) + (y >> 3);
  }(blockIdx.y, d.B * d.L);
  const int b = row / d.L, j = row % d.L;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  const int hbase = blockIdx.z * HW;
  const uint32_t kv_lds = lds_addr(&kv[0][0]);
  // Row swizzle of the 16-byte chunks (0..15, by the row within 16): spreads
  // the 16 rows of a key read (one chunk each) over distinct slots and the
  // row pairs of a transposing value read over distinct chunk pairs.  The
  // LDS hashes address bits 12 and 13 into bit 4 (slot bit 0); with 1 KiB
  // rows from a 1 KiB-aligned base that bit of the row's address is folded
  // in.  (1280-byte rows cross those bits inside a row and differently per
  // ring slot; there the plain swizzle is kept.)
  const int kvb10 = (int)((kv_lds >> 10) & 15);
  auto sw = [kvb10](int r) {
    const int t = kvb10 + (r & 15);
    const int hash = KPD * 2 == 1024 ? ((t >> 2) ^ (t >> 3)) & 1 : 0;
    return (((r & 7) << 1) | ((r >> 3) & 1)) ^ hash;
  };
  const int n_geo = d.kI + d.window;
  // no index list (I == NULL): entry e names pooled row e (dense attention)
  const int* Irow = I ? I + (size_t)row * d.kI : nullptr;
  auto id_at = [&](int e) { return Irow ? Irow[e] : e; };
  int id_a[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const int ea = tid + u * NT;
    id_a[u] = (ea < n_geo && ea < d.kI) ? id_at(ea) : -1;
  }
  const int T0 = t0[__builtin_amdgcn_readfirstlane(b)];
  const int S0 = ring_slot0(d, __builtin_amdgcn_readfirstlane(b), T0);
  // this wave's 16 heads of q (the B operand of S), straight into registers
  bf16x8 qf[NS];
  {
    const uint16_t* qrow = q + ((size_t)row * d.H + hbase + 16 * wv + c) * DK + g * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const bf16x8*)(qrow + s * 32);
  }
  const RowPlan rp = row_plan(d, T0, S0, j);
  const int dummy = rp.n_loc > 0 ? -1 - rp.lbase : 0;
  const bool any_row = rp.n_loc > 0 || rp.V > 0;
  auto resolve = [&](int e, int id, int& code) -> bool {
    code = dummy;
    if (e >= n_geo) return false;
    if (e < d.kI) {
      if (id < 0 || id >= rp.V) return false;
      code = id;
      return true;
    }
    if (e - d.kI >= rp.n_loc) return false;
    code = -1 - local_row(d, rp, e - d.kI);
    return true;
  };
  // head c of this wave: running max m (log2 domain) and sum l, on all four
  // lanes that hold it
  float m = -INFINITY, l = 0.f;
  const float scale = d.attn_scale_log2;
  f32x4 acc[NDT];
#pragma unroll
  for (int n = 0; n < NDT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int vrow = 4 * g + (c >> 2);
  const int vsw = sw(vrow);
  // chunk 2dt + (c%4)/2 of row vrow (+16): as for K, the swizzle stays in
  // the low four bits, so tiles dt and dt+8 differ by 256 bytes
  auto vaddr = [&](int dt, int hi) {
    const int ch = 2 * dt + ((c & 3) >> 1);
    if (ch >= 64) return (vrow + 16 * hi) * KPD + tail_pos(ch, vsw) * 8 + 4 * (c & 1);
    return (vrow + 16 * hi) * KPD + (((2 * (dt & 7) + ((c & 3) >> 1)) ^ vsw) * 8) + (dt >> 3) * 128 + 4 * (c & 1);
  };
  const uint16_t* pooled_b = pooled_kv + (size_t)b * d.Np_cap * DK;
  const uint16_t* local_b = local_kv + (size_t)b * d.Wl_cap * DK;

  for (int cb = any_row ? 0 : n_geo; cb < n_geo; cb += CH) {
    const int ce = min(n_geo, cb + CH);
    const int ntile = (ce - cb + kTile - 1) / kTile;
    __syncthreads();  // the previous chunk is done with every slot, code and mask
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      if (cb + u * NT >= ce) break;
      const int ea = cb + tid + u * NT;
      const int id = cb == 0 ? id_a[u] : (ea < n_geo && ea < d.kI ? id_at(ea) : -1);
      int code;
      const uint64_t live = __ballot(resolve(ea, id, code));
      s_code[tid + u * NT] = code;
      if (lane == 0) {
        const int t = (wv * 64 + u * NT) / kTile;
        s_tmask[t] = (uint32_t)live;
        s_tmask[t + 1] = (uint32_t)(live >> 32);
      }
    }
    __syncthreads();  // every row code of the chunk is in
    auto load_tile = [&](int t, int slot) {
      int4 code4[RPW / 4];
#pragma unroll
      for (int q4 = 0; q4 < RPW / 4; ++q4) code4[q4] = *(const int4*)&s_code[t * kTile + RPW * wvs + 4 * q4];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int4 c4 = code4[r >> 2];
        const int cd = (r & 3) == 0 ? c4.x : (r & 3) == 1 ? c4.y : (r & 3) == 2 ? c4.z : c4.w;
        const bool pooled = cd >= 0;
        const uint16_t* src = (pooled ? pooled_b : local_b) + (size_t)(uint32_t)(pooled ? cd : -1 - cd) * DK;
        const int trow = RPW * wvs + r;
        const uint32_t dst = kv_lds + (uint32_t)((slot * kTile + trow) * KPD * 2);
        g2lds16_builtin(src + (lane ^ sw(trow)) * 8, dst);
        if (DK > 512 && (lane ^ sw(trow)) < DK / 8 - 64) g2lds16_builtin(src + 512 + (lane ^ sw(trow)) * 8, dst + 1024);
      }
    };
    auto wait_loads = [&](int keep) {  // at most `keep` later tiles' loads still in flight
      if (keep >= 2) __builtin_amdgcn_s_waitcnt((2 * LPT & 15) | ((2 * LPT >> 4) << 14) | 0x0F70);
      else if (keep == 1) __builtin_amdgcn_s_waitcnt((LPT & 15) | ((LPT >> 4) << 14) | 0x0F70);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
    };
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
      if (t < ntile) load_tile(t, t);
    for (int t = 0; t < ntile; ++t) {
      const uint16_t* kvb = kv[t % NBUF];
      wait_loads(min(ntile - 1, t + NBUF - 2) - t);
      lds_sync();  // every wave's rows of tile t are in; every wave is done with tile t-1
      if (t + NBUF - 1 < ntile) load_tile(t + NBUF - 1, (t + NBUF - 1) % NBUF);
      const uint32_t tmask = __builtin_amdgcn_readfirstlane(s_tmask[t]);
      // Lane offsets are formed here each tile from an opaque zero: hoisted
      // out of the loop they would be spilled (the accumulators and q take
      // 192 of the 256 registers) and reloaded behind full waits.
      int zl = 0;
      asm volatile("" : "+v"(zl));
      const int cz = c + zl;
      // scores: rows 16*rb + c of the tile (A) against this wave's heads (B)
      f32x4 sc[2];
      {
        f32x4 sa[2][NACC];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int u = 0; u < NACC; ++u) sa[rb][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        // chunk 4s+g of row 16rb+c: the swizzle touches only the low four
        // bits of the chunk index, so chunk (4s+g) ^ sw = 16*(s/4) + ((4*(s%4)+g) ^ sw)
        auto load_k = [&](int rb, int s) {
          const int ch = 4 * s + g;
          if (ch >= 64) return *(const bf16x8*)(kvb + (rb * 16 + cz) * KPD + tail_pos(ch, sw(cz)) * 8);
          return *(const bf16x8*)(kvb + (rb * 16 + cz) * KPD + (((4 * (s & 3) + g) ^ sw(cz)) * 8) + (s >> 2) * 128);
        };
        bf16x8 ka[2][KW / 2];
#pragma unroll
        for (int s = 0; s < KW / 2; ++s) {
          ka[0][s] = load_k(0, s);
          ka[1][s] = load_k(1, s);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a0 = ka[0][s % (KW / 2)], a1 = ka[1][s % (KW / 2)];
          if (s + KW / 2 < NS) {
            ka[0][s % (KW / 2)] = load_k(0, s + KW / 2);
            ka[1][s % (KW / 2)] = load_k(1, s + KW / 2);
          }
          sa[0][s % NACC] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[s], sa[0][s % NACC], 0, 0, 0);
          sa[1][s % NACC] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[s], sa[1][s % NACC], 0, 0, 0);
        }
        sc[0] = sa[0][0];
        sc[1] = sa[1][0];
#pragma unroll
        for (int u = 1; u < NACC; ++u) {
          sc[0] += sa[0][u];
          sc[1] += sa[1][u];
        }
      }
      // online softmax of head c over the tile's 32 rows
      float x[8];
      float tmax = -INFINITY;
      const uint32_t tb = tmask >> (4 * (g + zl));  // rows 4g+i and 16+4g+i at bits i and 16+i
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[4 * rb + i] = ((tb >> (16 * rb + i)) & 1u) ? sc[rb][i] * scale : -INFINITY;
          tmax = fmaxf(tmax, x[4 * rb + i]);
        }
      tmax = max_rows(tmax);
      // lazy rescale: the reference max moves only when exceeded by 2^8
      float alpha = 1.f;
      if (m == -INFINITY) {
        m = tmax;
      } else if (tmax > m + 8.f) {
        const float m_new = fmaxf(m, tmax);
        alpha = __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
        m = m_new;
      }
      const float m_sub = m == -INFINITY ? 0.f : m;
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(x[e] - m_sub);
        psum += p[e];
      }
      l += sum_rows(psum);
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int n = 0; n < NDT; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[n][i] *= alpha;
      }
      // P^T operand: entry e of lane (g, c) is tile row 16*(e/4) + 4g + e%4
      u32x4 pu;
#pragma unroll
      for (int k = 0; k < 4; ++k) pu[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pu);
      // O^T += V^T P^T over every 16-column value tile, PVG tiles' reads in
      // flight at a time (registers)
#pragma unroll
      for (int n0 = 0; n0 < NDT; n0 += PVG) {
#pragma unroll
        for (int n = n0; n < n0 + PVG && n < NDT; ++n) {
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kvb + zl + vaddr(n, 0)));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kvb + zl + vaddr(n, 1)));
          const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, acc[n], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // normalise (sink included) and stage the rows in the idle ring for
  // whole-line stores
  const int h = hbase + 16 * wv + c;
  const float sink2 = sinks ? sinks[h] * kLog2e : -INFINITY;
  const float mf = fmaxf(m, sink2);
  float f = 0.f;
  if (mf != -INFINITY) {
    const float lf = l * exp2f(m - mf) + (sinks ? exp2f(sink2 - mf) : 0.f);
    f = lf > 0.f ? exp2f(m - mf) / lf : 0.f;
  }
  // groups of 32 heads: waves 2h and 2h+1 stage, then all copy out
  uint16_t* og = out + ((size_t)row * d.H + hbase) * DV;
  constexpr int CPR = DV / 8;  // 16-byte pieces per head row
#pragma unroll 1
  for (int half = 0; half < NW / 2; ++half) {
    __syncthreads();  // every wave is done with the ring (or the previous half)
    if ((wv >> 1) == half) {
      uint16_t* orow = &kv[0][0] + (16 * (wv & 1) + c) * OP + 4 * g;
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        uint2 v;
        v.x = pack_bf16x2(acc[n][0] * f, acc[n][1] * f);
        v.y = pack_bf16x2(acc[n][2] * f, acc[n][3] * f);
        *(uint2*)(orow + n * 16) = v;
      }
    }
    __syncthreads();
    uint16_t* oh = og + (size_t)half * 32 * DV;
    for (int k = tid; k < 32 * CPR; k += NT) {
      const int hr = k / CPR, cc = k - hr * CPR;
      *(u32x4*)(oh + (size_t)k * 8) = *(const u32x4*)(&kv[0][0] + hr * OP + cc * 8);
    }
  }
}

// Few query rows (decode, short verify chunks; K = V rows 512 or 576 wide):
// one workgroup per (64-entry split of the row list, query row, 16 heads),
// four waves, the whole split in one pass.  Every wave resolves the split's 64
// entries (pooled ids from I, then the local window) into row codes; wave w
// brings rows 16w .. 16w+15 global->LDS and scores them against the 16 heads
// (S = K q^T, 16x16x32 MFMA, lane (g, c) holding rows 16w + 4g + i of head c);
// the softmax takes the exact maximum over the split's rows (one exchange of
// per-wave maxima and sums through LDS); P^T goes to LDS in the value MFMA's k
// order; O^T += V^T P^T reads V^T with the transposing LDS read, wave w owning
// value tiles w, w+4, ...  The partial (O / l in bf16, m and l in the log2
// domain) goes to the merge.  Rows and their 16-byte chunks are laid out as in the
// other attention kernels (the chunk swizzle by row; 576-wide rows keep their
// last eight chunks in a swizzled tail of a 1280-byte pitch).
constexpr int kSplitRows = 64;

template <int DK, int DV>
__global__ __launch_bounds__(256) void k_attn_split64(KDims d, int splits, const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ local_kv,
                                                      const uint16_t* __restrict__ pooled_kv,
                                                      const int* __restrict__ I, const int* __restrict__ t0,
                                                      float* __restrict__ part) {
  static_assert(DK == DV && (DK == 512 || DK == 576), "shape");
  constexpr int KPD = (DK * 2 + 255) / 256 * 128;  // LDS row pitch (elements)
  constexpr int NS = DK / 32;                      // MFMA k-steps of S
  constexpr int NDTW = DV / 16 / 4;                // value tiles per wave
  constexpr int PP = kSplitRows + 8;               // P^T pitch (elements) per head
  __shared__ __align__(1024) uint16_t kv[kSplitRows * KPD];
  __shared__ __align__(16) uint16_t s_p[16 * PP];
  __shared__ float s_red[2][4][16];
  args_now(d, splits, q, local_kv, pooled_kv, I, t0, part);
  // workgroup wg takes head group hg of (query row, split) pair p, with
  // wg = 8 ngrp (p / 8) + 8 hg + p % 8: the head groups of one split are 8
  // workgroups apart, so they are dealt to one XCD (round-robin over 8) and
  // share its L2 for the split's rows; pairs past the last are padding
  const int ngrp = d.H >> 4, wg = blockIdx.x;
  const int sg = wg / (8 * ngrp), rem = wg - sg * (8 * ngrp);
  const int pair = 8 * sg + (rem & 7);
  if (pair >= splits * d.B * d.L) return;
  const int split = pair % splits, row = pair / splits, hbase = (rem >> 3) * 16;
  const int b = row / d.L, j = row - b * d.L;
  const int lane = lane_id(), wv = wave_id(), g = lane >> 4, c = lane & 15;
  // this row's 16 heads of q (the B operand of S) and the split's entries of
  // the index row, requested before t0 (nothing of theirs depends on it)
  bf16x8 qf[NS];
  {
    const uint16_t* qrow = q + ((size_t)row * d.H + hbase + c) * DK + g * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const bf16x8*)(qrow + s * 32);
  }
  const int e = split * kSplitRows + lane;
  int id = -1;
  if (e < d.kI) id = I ? I[(size_t)row * d.kI + e] : e;
  const int T0 = t0[b];
  const RowPlan rp = row_plan(d, T0, ring_slot0(d, b, T0), j);
  // a row every live split may read (entries that take no part point at it)
  const int dummy = rp.n_loc > 0 ? -1 - rp.lbase : 0;
  // every wave resolves all 64 entries of the split itself (lane = entry), so
  // no wave waits on another before its gather
  int code = dummy;
  bool present = false;
  if (rp.ok) {
    if (e < d.kI) {
      if (id >= 0 && id < rp.V) {
        present = true;
        code = id;
      }
    } else if (e - d.kI < d.window && e - d.kI < rp.n_loc) {
      present = true;
      code = -1 - local_row(d, rp, e - d.kI);
    }
  }
  const uint64_t live = __ballot(present);
  const bool any = live != 0;
  const uint32_t kv_lds = lds_addr(kv);
  const int kvb10 = (int)((kv_lds >> 10) & 15);
  auto sw = [kvb10](int r) {
    const int t = kvb10 + (r & 15);
    const int hash = KPD * 2 == 1024 ? ((t >> 2) ^ (t >> 3)) & 1 : 0;
    return (((r & 7) << 1) | ((r >> 3) & 1)) ^ hash;
  };
  f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (any) {
    // wave w brings rows 16w .. 16w+15 straight into LDS
    const uint16_t* pooled_b = pooled_kv + (size_t)b * d.Np_cap * DK;
    const uint16_t* local_b = local_kv + (size_t)b * d.Wl_cap * DK;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = 16 * wv + u;
      const int cd = __builtin_amdgcn_readlane(code, r);
      const uint16_t* src = cd >= 0 ? pooled_b + (size_t)cd * DK : local_b + (size_t)(-1 - cd) * DK;
      const int x = lane ^ sw(r);
      const uint32_t dst = kv_lds + (uint32_t)(r * KPD * 2);
      g2lds16(src + x * 8, dst);
      if (DK > 512 && x < DK / 8 - 64) g2lds16(src + 512 + x * 8, dst + 1024);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's rows are in LDS
    // (each wave scores only the rows it brought)
    const int rr = 16 * wv + c, rsw = sw(rr);
    auto load_k = [&](int s) {
      const int ch = 4 * s + g;
      if (ch >= 64) return *(const bf16x8*)(kv + rr * KPD + tail_pos(ch, rsw) * 8);
      return *(const bf16x8*)(kv + rr * KPD + (((4 * (s & 3) + g) ^ rsw) * 8) + (s >> 2) * 128);
    };
    bf16x8 ka[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) ka[s] = load_k(s);
    f32x4 sa[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sa[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) sa[s & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qf[s], sa[s & 3], 0, 0, 0);
    sc = (sa[0] + sa[1]) + (sa[2] + sa[3]);
  }
  // softmax of head c over the split's rows, the exact maximum
  const float scale = d.attn_scale_log2;
  float x[4], mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wv + 4 * g + i;
    x[i] = ((live >> r) & 1) ? sc[i] * scale : -INFINITY;
    mx = fmaxf(mx, x[i]);
  }
  mx = max_rows(mx);
  if (g == 0) s_red[0][wv][c] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(s_red[0][0][c], s_red[0][1][c]), fmaxf(s_red[0][2][c], s_red[0][3][c]));
  const float m_sub = m == -INFINITY ? 0.f : m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_sub);
  const float ps = sum_rows((p[0] + p[1]) + (p[2] + p[3]));
  if (g == 0) s_red[1][wv][c] = ps;
  // P^T operand of k-step kk: entry 8g + e of head c is row 32kk + 16(e/4) +
  // 4g + e%4, i.e. waves 2kk and 2kk+1 give four entries each
  uint2 pk;
  pk.x = pack_bf16x2(p[0], p[1]);
  pk.y = pack_bf16x2(p[2], p[3]);
  *(uint2*)&s_p[c * PP + (wv >> 1) * 32 + 8 * g + 4 * (wv & 1)] = pk;
  __syncthreads();  // every wave's P, sums, and rows (each wave waited for its own)
  const float l = (s_red[1][0][c] + s_red[1][1][c]) + (s_red[1][2][c] + s_red[1][3][c]);
  f32x4 acc[NDTW];
#pragma unroll
  for (int n = 0; n < NDTW; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (any) {
    // transposing V reads: lane (g, c) takes rows 4g + c/4 (+16) and columns
    // 4(c%4) .. +3 of a 16-column value tile
    const int vrow = 4 * g + (c >> 2), vsw = sw(vrow);
    auto vaddr = [&](int dt) {
      const int ch = 2 * dt + ((c & 3) >> 1);
      if (ch >= 64) return vrow * KPD + tail_pos(ch, vsw) * 8 + 4 * (c & 1);
      return vrow * KPD + (((2 * (dt & 7) + ((c & 3) >> 1)) ^ vsw) * 8) + (dt >> 3) * 128 + 4 * (c & 1);
    };
    const bf16x8 pb0 = *(const bf16x8*)&s_p[c * PP + 8 * g];
    const bf16x8 pb1 = *(const bf16x8*)&s_p[c * PP + 32 + 8 * g];
#pragma unroll
    for (int n = 0; n < NDTW; ++n) {
      const int off = vaddr(wv + 4 * n);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint16_t* base = kv + kk * 32 * KPD + off;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * KPD));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, kk ? pb1 : pb0, acc[n], 0, 0, 0);
      }
    }
  }
  // the split's partial: O^T tile (16dt + 4g + i, head c) per lane over l, then (m, l)
  const size_t prow = ((size_t)split * d.B * d.L + row) * d.H + hbase + c;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int n = 0; n < NDTW; ++n) store_part4(part, prow, DV, 16 * (wv + 4 * n) + 4 * g, acc[n], inv);
  if (wv == 0 && g == 0) store_part_ml(part, prow, DV, m, l);
}

// Merge of split partials (part_row_bytes: O / l in bf16, then m and l in the
// log2 domain), sink included.  One workgroup per (query row, head, 256
// output columns, Dv even); the first wave turns the splits' (m, l) into
// weights exp2(m - M) l / (sum of them and the sink's), then every thread sums
// its two columns over the splits (one 4-byte load per split).  The first PRE
// splits' values are requested with (m, l), the rest after the weights (PRE
// is picked from the split count: a deeper prefetch than needed costs
// predicated loads in every thread).
constexpr int kMaxSplits = 64;

template <typename T, int PRE>
__global__ __launch_bounds__(128) void k_attn_merge(KDims d, int splits, const float* __restrict__ part,
                                                    const float* __restrict__ sinks, T* __restrict__ out) {
  __shared__ float s_w[kMaxSplits];
  args_now(d, splits, part, sinks, out);
  const int row = blockIdx.x, h = blockIdx.y;
  const int e = blockIdx.z * 256 + 2 * threadIdx.x;
  const size_t rb = part_row_bytes(d.Dv);
  const size_t stride = (size_t)d.B * d.L * d.H * rb;  // bytes between splits
  const char* p0 = (const char*)part + ((size_t)row * d.H + h) * rb;
  // the columns' partials are requested together with (m, l)
  constexpr int kPre = PRE;
  const int ec = min(e, d.Dv - 2);
  uint32_t pre[kPre];
#pragma unroll
  for (int s = 0; s < kPre; ++s) pre[s] = s < splits ? *(const uint32_t*)(p0 + s * stride + 2 * ec) : 0u;
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float* ml = (const float*)(p0 + s * stride + 2 * (size_t)d.Dv);
    const float m = s < splits ? ml[0] : -INFINITY;
    const float l = s < splits ? ml[1] : 0.f;
    const float sink2 = sinks ? sinks[h] * kLog2e : -INFINITY;
    float mf = wave_max(m);
    mf = fmaxf(mf, sink2);
    const float wgt = (mf == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - mf) * l;
    float lf = wave_sum(wgt);
    if (sinks && mf != -INFINITY) lf += exp2f(sink2 - mf);
    const float inv = lf > 0.f ? 1.f / lf : 0.f;
    s_w[s] = wgt * inv;
  }
  __syncthreads();
  if (e >= d.Dv) return;
  float ox = 0.f, oy = 0.f;
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < splits) {
      ox += bf_lo(pre[s]) * s_w[s];
      oy += bf_hi(pre[s]) * s_w[s];
    }
  for (int s = kPre; s < splits; ++s) {
    const uint32_t v = *(const uint32_t*)(p0 + s * stride + 2 * e);
    ox += bf_lo(v) * s_w[s];
    oy += bf_hi(v) * s_w[s];
  }
  T* op = out + ((size_t)row * d.H + h) * d.Dv + e;
  stf(op, ox);
  stf(op + 1, oy);
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
  const int T0 = t0[b];
  const RowPlan rp = row_plan(d, T0, ring_slot0(d, b, T0), j);
  const int n = rp.n_list;
  const float scale = 1.0f / sqrtf((float)d.Dk);
  for (int e = tid; e < d.Dk; e += 256) s_q[e] = ldf(q + ((size_t)row * d.H + h) * d.Dk + e) * scale;
  // s_row: >= 0 pooled id, <= -2 local row -(r + 2), -1 masked
  for (int e = tid; e < n; e += 256) {
    int code = -1;
    if (e < rp.n_loc) code = -(local_row(d, rp, e) + 2);
    else {
      const int id = I ? I[(size_t)row * d.kI + e - rp.n_loc] : e - rp.n_loc;
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
      // sixteen loads of the row in flight per step, four partial sums
      const T* kp = row_ptr(code);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      int k = 0;
      for (; k + 16 <= d.Dk; k += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = ldf(kp + k + u);
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u & 3] += s_q[k + u] * v[u];
      }
      for (; k < d.Dk; ++k) acc[0] += s_q[k] * ldf(kp + k);
      x = (acc[0] + acc[1]) + (acc[2] + acc[3]);
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
  // P V: with Dv < 256, G = 256 / Dv thread groups each sum every G-th row
  // (partials combined in LDS, in s_q, which the scores no longer need);
  // eight rows' loads are in flight per step
  const int G = d.Dv >= 256 ? 1 : 256 / d.Dv;
  const int span = G == 1 ? 256 : d.Dv;
  const int grp = tid / span;
  if (grp < G)
    for (int e = tid % span; e < d.Dv; e += span) {
      float o = 0.f;
      int r = grp;
      for (; r + 7 * G < n; r += 8 * G) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int code = s_row[r + u * G];
          v[u] = code != -1 ? ldf(row_ptr(code) + e) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) o += s_x[r + u * G] * v[u];
      }
      for (; r < n; r += G) {
        const int code = s_row[r];
        if (code != -1) o += s_x[r] * ldf(row_ptr(code) + e);
      }
      if (G == 1) stf(orow + e, o * inv);
      else s_q[grp * d.Dv + e] = o;
    }
  if (G == 1) return;
  __syncthreads();
  for (int e = tid; e < d.Dv; e += 256) {
    float o = 0.f;
    for (int gg = 0; gg < G; ++gg) o += s_q[gg * d.Dv + e];
    stf(orow + e, o * inv);
  }
}

template <int DK, int DV>
hipError_t launch_mfma(const KDims& d, const void* q, const void* local_kv, const void* pooled_kv, const int* I,
                       const float* sinks, const int* t0, void* out, float* partial, int splits, hipStream_t st) {
  if (attn_split64_ok(d)) {
    const dim3 grid(8 * (d.H / 16) * ((splits * d.B * d.L + 7) / 8));
    hipLaunchKernelGGL((k_attn_split64<DK, DV>), grid, dim3(256), 0, st, d, splits, (const uint16_t*)q,
                       (const uint16_t*)local_kv, (const uint16_t*)pooled_kv, I, t0, partial);
    return hipGetLastError();
  }
  if (attn_small_groups(d)) {
    const dim3 grid(splits, d.B * d.L, d.H / 16);
    hipLaunchKernelGGL((k_attn_mfma<DK, DV, 1>), grid, dim3(128), 0, st, d, splits, (const uint16_t*)q,
                       (const uint16_t*)local_kv, (const uint16_t*)pooled_kv, I, sinks, t0, (uint16_t*)out, partial);
    return hipGetLastError();
  }
  if constexpr (DK == 512) {
    // many rows, 512 wide: the flash-style kernel, 64 heads, two workgroups per CU
    if (splits == 1) {
      const dim3 grid(1, d.B * d.L, d.H / 64);
      hipLaunchKernelGGL((k_attn_fa<DK, DV, 4>), grid, dim3(256), 0, st, d, (const uint16_t*)q,
                         (const uint16_t*)local_kv, (const uint16_t*)pooled_kv, I, sinks, t0, (uint16_t*)out);
      return hipGetLastError();
    }
  }
  // (576 wide, the flash-style kernel holds one workgroup per CU, with 64
  // heads or with 128, and the kernel below is faster)
  {
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

// Up to twelve query rows' worth of 64-head groups with a row list of 2 ..
// kMaxSplits 64-entry splits: one workgroup per split (k_attn_split64, MFMA
// shapes only; its partials always go through the merge).  Measured against
// the split kernels at 64 heads x 640 entries: faster at 9 and 12 rows
// (17.7 / 19.3 against 18.9 / 20.1 us), slower from 16 rows on (26.3 against
// 23.0; 32 rows of a batch: 31.0 against 19.0), where its one workgroup per
// 64 entries and 16 heads turns into more partials than the merge pays back.
bool attn_split64_ok(const KDims& d) {
  const long long n_geo = (long long)d.kI + d.window;
  return (long long)d.B * d.L * (d.H / 64) <= 12 && n_geo > kSplitRows && n_geo <= (long long)kSplitRows * kMaxSplits;
}

int attn_splits(const KDims& d, bool bf16) {
  if (!attn_mfma_ok(d, bf16)) return 1;
  if (attn_split64_ok(d)) return std::max(1, (d.kI + d.window + kSplitRows - 1) / kSplitRows);
  const long long work = (long long)d.B * d.L * (d.H / (attn_small_groups(d) ? 16 : 64));
  const long long n_max = (long long)d.window + d.kI;
  // at least two 32-row tiles per split, so that fetching overlaps compute
  const long long max_splits = std::max(1LL, (n_max + 2 * kTile - 1) / (2 * kTile));
  // about 256 two-wave workgroups (16 heads) or 128 eight-wave ones (64
  // heads): more splits only add partials to merge
  const long long target = attn_small_groups(d) ? 256 : 128;
  long long want = (target + work - 1) / work;
  want = std::min(want, std::min(max_splits, (long long)kMaxSplits));
  return (int)std::max(1LL, want);
}

size_t attn_partial_bytes(const KDims& d, int splits) {
  if (splits <= 1) return 0;
  return (size_t)splits * d.B * d.L * d.H * part_row_bytes(d.Dv);
}

hipError_t launch_attention_merge(const KDims& d, bool bf16, const float* partial, const float* sinks, void* out,
                                  int splits, hipStream_t st) {
  if (d.Dv & 1) return hipErrorInvalidValue;  // (split attention only for 512- or 576-wide values)
  const dim3 grid(d.B * d.L, d.H, (d.Dv + 255) / 256);
  auto go = [&](auto pre) {
    constexpr int P = decltype(pre)::value;
    if (bf16)
      hipLaunchKernelGGL((k_attn_merge<uint16_t, P>), grid, dim3(128), 0, st, d, splits, partial, sinks,
                         (uint16_t*)out);
    else
      hipLaunchKernelGGL((k_attn_merge<float, P>), grid, dim3(128), 0, st, d, splits, partial, sinks, (float*)out);
  };
  if (splits <= 8) go(std::integral_constant<int, 8>{});
  else if (splits <= 24) go(std::integral_constant<int, 24>{});
  else go(std::integral_constant<int, 32>{});
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
