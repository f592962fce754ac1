// hisa_internal.h -- kernel-side problem description and launcher entry points
// shared by the host library (hisa_abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hisa {

enum { PATH_INVALID = -1, PATH_DENSE = 0, PATH_FLAT = 1, PATH_HISA = 2 };

// Plain-int copy of hisa_dims plus derived constants, passed to kernels by value.
struct KDims {
  int B, L, ratio, window, topk, index_block, index_keep;
  int H_i, D_i, H, Dk, Dv, Np_cap, Wl_cap, kI;
  int force_flat;  // HISA_MODE_FORCE_FLAT
  int force_dense; // HISA_MODE_FORCE_DENSE (the selection calls only fill I)
  int force_path;  // -1: run the gate; PATH_FLAT: flat for every valid sequence
  int nb_cap;      // Np_cap / index_block (0 when index_block == 0)
  int ratio_shift; // log2(ratio) when ratio is a power of two, else -1
  float w_scale;   // (float)(1 / sqrt(H_i * D_i)), rounded once from double
  float attn_scale_log2;  // (float)(log2(e) / sqrt(Dk))
  int local_ring;         // local_kv is a ring of Wl_cap slots (attention)
  const int* ring_slot;   // ring: slot of position t0[b] per sequence, or NULL for t0[b] mod Wl_cap
};

// Launchers (kernel files).  Each returns hipSuccess or the launch error.
// Pointers are device pointers; bf16 data is passed as uint16_t.
// Decode scan; with cnt != NULL (decode_fused_ok) it also runs the selection
// and writes I / top_blk / path, and launch_decode_select is not needed.
// cnt: decode_counter_ints(d) zeroed ints, left zeroed.
constexpr int kCntStride = 16;  // ints between arrival counters: one 64-byte line each
inline size_t decode_counter_ints(const KDims& d) {
  // B sequence counters + B x ceil(ceil(Np_cap / 64) / 16) slab-group counters
  const size_t slabs = ((size_t)d.Np_cap + 63) / 64;
  return (size_t)d.B * (1 + (slabs + 15) / 16) * kCntStride;
}
bool decode_fused_ok(const KDims& d, bool bf16);
hipError_t launch_decode_scan(const KDims& d, bool bf16, const void* q_idx, const float* w,
                              const void* keys, const int* t0, float* fscore, float* cscore,
                              int* cnt, int* I, int* top_blk, int* path, hipStream_t st);
// The decode step (selection + sparse combine) of few sequences in one
// launch up to the split partials, which launch_attention_merge (splits =
// decode_step_splits) then combines: decode_step_ok (max_attn_wgs: attention
// workgroups the device holds at once with room to spare, e.g. its CU
// count).  Workspace: the sync region (decode_step_sync_bytes, zero at first
// use and left zero; its first int becomes 1 if a hand-off ever timed out),
// the scan counters (decode_counter_ints, the same rule), fscore, cscore and
// the partials (decode_step_partial_bytes).
bool decode_step_ok(const KDims& d, bool idx_bf16, bool attn_bf16, int max_attn_wgs);
int decode_step_splits(const KDims& d);
size_t decode_step_sync_bytes(const KDims& d);
size_t decode_step_partial_bytes(const KDims& d);
hipError_t launch_decode_step(const KDims& d, const void* q_idx, const float* w, const void* keys, const int* t0,
                              const void* q, const void* local_kv, const void* pooled_kv, const float* sinks,
                              void* sync, int* cnt, float* fscore, float* cscore, float* part, int* I, int* top_blk,
                              int* path, hipStream_t st);
hipError_t launch_decode_select(const KDims& d, const float* fscore, const float* cscore,
                                const int* t0, int* I, int* top_blk, int* path, hipStream_t st);
hipError_t launch_block_mean(const KDims& d, bool bf16, bool all_paths, const void* keys,
                             const int* t0, float* rep, uint16_t* rep3, hipStream_t st);
hipError_t launch_coarse(const KDims& d, bool bf16, bool all_paths, const void* q_idx,
                         const float* w, const float* rep, const uint16_t* rep3, const int* t0,
                         float* cscore, hipStream_t st);
// Batched HiSA selection with one query row per wave (bf16 64 x 128 indexer,
// nb_cap and index_keep * index_block at most 1024).
bool select_rows_ok(const KDims& d, bool bf16);
hipError_t launch_select_rows(const KDims& d, const void* q_idx, const float* w, const void* keys,
                              const uint16_t* rep3, const int* t0, int* I, int* top_blk, int* path,
                              hipStream_t st);
hipError_t launch_fine(const KDims& d, bool bf16, const void* q_idx, const float* w,
                       const void* keys, const float* cscore, const int* t0, int* I,
                       int* top_blk, int* path, hipStream_t st);
hipError_t launch_flat_scores(const KDims& d, bool bf16, const void* q_idx, const float* w,
                              const void* keys, const int* t0, float* scores, hipStream_t st);
hipError_t launch_topk_rows(const KDims& d, const float* scores, const int* t0, int* I,
                            int* path, hipStream_t st);
// Selection on a caller-kept cache of f32 block means (B, nb_cap, D_i), one
// query row (b, j) per grid row (decode, or a short verify chunk):
// bf16 64 x 128 indexer, nb_cap <= 4096, index_keep <= 64 and
// topk <= index_block * index_keep <= 1024, not forced flat.  The coarse
// kernel also writes the means of the blocks completed by the step's token.
// cnt: cached_counter_ints(d) zeroed ints, left zeroed; cscore (B, nb_cap);
// blk (B, index_keep); fs: cached_fine_floats(d).
bool cached_decode_ok(const KDims& d, bool bf16);
size_t cached_counter_ints(const KDims& d);
size_t cached_fine_floats(const KDims& d);
hipError_t launch_cached_decode(const KDims& d, const void* q_idx, const float* w, const void* keys, float* rep,
                                const int* t0, float* cscore, int* blk, float* fs, int* cnt, int* I,
                                int* top_blk, int* path, hipStream_t st);
// Means of the blocks completed by the step's tokens (all: every complete
// block) into rep (B, nb_cap, D_i).
hipError_t launch_rep_update(const KDims& d, bool bf16, bool all, const void* keys, const int* t0, float* rep,
                             int* zero_p, size_t zero_n, hipStream_t st);
// Zeroes n ints on the stream (n < 2^31).
hipError_t launch_zero_ints(int* p, size_t n, hipStream_t st);
// The dense fallback (indexer off): I = 0..Np-1 padded with -1 on every row.
hipError_t launch_fill_dense(const KDims& d, const int* t0, int* I, int* top_blk, int* path,
                             hipStream_t st);

// Attention.  splits > 1 writes partials to ws and merges them.  The partial
// of one (split, query row, head): the split's output normalised by its own
// sum (O / l) as Dv bf16 values, then m and l (f32, the log2 domain); rows
// part_row_bytes(Dv) apart (8-byte aligned for Dv % 4 == 0).
inline constexpr size_t part_row_bytes(int Dv) { return 2 * (size_t)Dv + 8; }
int attn_splits(const KDims& d, bool bf16);
bool attn_mfma_ok(const KDims& d, bool bf16);
bool attn_generic_ok(const KDims& d);
bool attn_small_groups(const KDims& d);
bool attn_split64_ok(const KDims& d);  // (with attn_mfma_ok) few rows: one workgroup per 64-entry split
size_t attn_partial_bytes(const KDims& d, int splits);
hipError_t launch_attention(const KDims& d, bool bf16, const void* q, const void* local_kv,
                            const void* pooled_kv, const int* I, const float* sinks,
                            const int* t0, void* out, float* partial, int splits,
                            hipStream_t st);
hipError_t launch_attention_merge(const KDims& d, bool bf16, const float* partial,
                                  const float* sinks, void* out, int splits, hipStream_t st);

// Shapes with hand-tuned MFMA selection kernels.
inline bool idx_mfma_ok(const KDims& d, bool bf16) { return bf16 && d.H_i == 64 && d.D_i == 128; }

}  // namespace hisa
