/*
 * hisa.h -- C ABI of the MI355X (gfx950) HiSA sparse-selection and sparse
 * local+pooled attention library (libhisa.so).
 *
 * What it computes (the pages):
 *   [HiSA issue]  GitHub lablup/mlxcel issue #549, "feat(deepseek-v4): implement
 *                 HiSA hierarchical sparse attention": sections Conventions, The
 *                 pooled stream and positions, The indexer query and per-head
 *                 weights, Flat selection, HiSA decode path, HiSA batched path,
 *                 Consuming the selection: sparse combine, Engagement thresholds.
 *   [DSA issue]   GitHub lablup/mlxcel issue #509, "implement the DeepSeek Sparse
 *                 Attention (DSA) indexer", What needs to be built, items 1 and 3.
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major, in the axis order written at each call;
 *     the caller allocates and owns every buffer (inputs, outputs, workspace).
 *     Pointers are device pointers unless said otherwise; dims is a host pointer.
 *   - t0 is a device int32[B]: the number of tokens the layer had consumed before
 *     this step for sequence b.  Query row j sits at absolute position t0[b] + j.
 *     After the step the pooled stream holds Np_b = floor((t0[b] + L) / ratio)
 *     rows; row j sees the pooled rows p < V = min(Np_b, floor((t0[b]+j+1)/ratio)).
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = the null stream).  No
 *     call allocates, synchronises, or copies between host and device, and none
 *     keeps a pointer after it returns.  Calls on one workspace must not overlap.
 *   - Sequences whose t0 breaks the buffer bounds (t0 < 0, Np_b > Np_cap, or a
 *     local window longer than Wl_cap) are not computed: their index rows are -1,
 *     their attention rows are 0, and path_out reports HISA_PATH_INVALID.
 *   - Return value: HISA_OK or a negative HISA_ERR_*; on error nothing was
 *     enqueued and hisa_last_error() (thread-local) says why.  Nothing throws.
 *   - Which selection path a sequence takes (dense / flat / HiSA) is decided on
 *     the device per sequence; it is not an error (see hisa_dims.mode).
 */
#ifndef HISA_H
#define HISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HISA_ABI_VERSION 3

enum hisa_dtype { HISA_F32 = 0, HISA_BF16 = 1 };

/* mode: HISA_MODE_AUTO runs the gate of the HiSA issue (dense when Np <= topk;
 * HiSA when index_block > 0, Np >= index_block*index_keep and
 * index_block*index_keep >= min(topk, Np); flat otherwise).
 * The other two are the kill-switches of the HiSA issue's implementation plan
 * (item 1).  HISA_MODE_FORCE_FLAT replaces the hierarchy by the flat scan (the
 * dense case Np <= topk is kept).  HISA_MODE_FORCE_DENSE turns the indexer off
 * (the dense fallback): hisa_select_decode / hisa_select_prefill score
 * nothing and list every pooled row, I = 0..Np-1 padded with -1, so the
 * attention call attends to all of them; topk is then the width of I and must
 * be >= Np_cap (HISA_ERR_ARG otherwise), and no workspace is needed.
 * hisa_block_scores and flat_topk_select ignore the mode's switches. */
enum hisa_mode { HISA_MODE_AUTO = 0, HISA_MODE_FORCE_FLAT = 1, HISA_MODE_FORCE_DENSE = 2 };

enum hisa_path { HISA_PATH_INVALID = -1, HISA_PATH_DENSE = 0, HISA_PATH_FLAT = 1, HISA_PATH_HISA = 2 };

enum hisa_status {
  HISA_OK = 0,
  HISA_ERR_ARG = -1,       /* bad pointer, size or unsupported shape */
  HISA_ERR_DTYPE = -2,     /* unsupported dtype combination */
  HISA_ERR_WORKSPACE = -3, /* ws_bytes smaller than hisa_workspace_bytes() */
  HISA_ERR_OVERFLOW = -4,  /* a size or offset overflows the kernels' int32 indexing */
  HISA_ERR_LAUNCH = -5     /* a kernel launch failed (see hisa_last_error) */
};

enum hisa_op {
  HISA_OP_BLOCK_SCORES = 0,
  HISA_OP_SELECT_DECODE = 1,
  HISA_OP_SELECT_PREFILL = 2,
  HISA_OP_FLAT_TOPK = 3,
  HISA_OP_ATTENTION = 4,
  HISA_OP_SELECT_DECODE_CACHED = 5,
  HISA_OP_BLOCK_MEANS_UPDATE = 6,
  HISA_OP_DECODE_STEP = 7
};

/* Problem sizes (HiSA issue, Configuration table). */
typedef struct {
  int32_t B;           /* sequences */
  int32_t L;           /* query rows per sequence in this step (1 = decode) */
  int32_t ratio;       /* compress ratio r of the layer (4; 1 = per-token DSA keys) */
  int32_t window;      /* sliding_window of the local stream (128); 0 = no local stream */
  int32_t topk;        /* index_topk: pooled rows kept per query, k = min(topk, Np) */
  int32_t index_block; /* HiSA block size b in pooled rows; 0 disables the hierarchy.
                          Supported: 0 or a divisor of 64 */
  int32_t index_keep;  /* HiSA blocks kept by the coarse stage (Kb upper bound) */
  int32_t H_i, D_i;    /* indexer heads and head dim (64 x 128) */
  int32_t H, Dk, Dv;   /* main attention heads, key width, value width (Dv <= Dk) */
  int32_t Np_cap;      /* pooled rows allocated per sequence in keys / pooled_kv */
  int32_t Wl_cap;      /* local rows allocated per sequence in local_kv */
  int32_t kI;          /* width of the index rows I given to the attention call */
  int32_t mode;        /* enum hisa_mode (selection calls) */
  int32_t idx_dtype;   /* dtype of q_idx and keys: HISA_BF16 or HISA_F32 */
  int32_t attn_dtype;  /* dtype of q, local_kv, pooled_kv and out: HISA_BF16 or HISA_F32 */
} hisa_dims;

/* Common selection inputs
 *   q_idx (B, L, H_i, D_i) idx_dtype: the roped indexer query, one row per query.
 *   w     (B, L, H_i) f32: the raw weights_proj(x) output.  The library applies
 *         H_i^-1/2 * D_i^-1/2 (HiSA issue, The indexer query and per-head
 *         weights; DSA issue, item 1, Score).
 *   keys  (B, Np_cap, D_i) idx_dtype: the indexer's pooled keys (HiSA issue,
 *         The pooled stream; for ratio 1, the per-token DSA keys).  Rows at or
 *         past Np_b are never read.
 * Scores are relu(q.k) per head, weighted and summed over heads, in f32
 * (HiSA issue, Conventions).  Index outputs hold absolute pooled row ids in
 * ascending order, padded with -1; exact score ties keep the lowest id.
 */

/* The coarse stage alone (HiSA issue, HiSA decode path "coarse" and HiSA
 * batched path "coarse"): block means rep and block scores cscore, with the
 * batched eligibility mask (a block is eligible iff its first row is visible,
 * else -1e30).  nb_cap = Np_cap / index_block; index_block must be > 0.
 *   cscore_out (B, L, nb_cap) f32: entries past nb_b = floor(Np_b / b) are -1e30.
 *   rep_out    (B, nb_cap, D_i) f32 or NULL: entries past nb_b are 0. */
int hisa_block_scores(const hisa_dims* d, const void* q_idx, const float* w, const void* keys,
                      const int32_t* t0, float* cscore_out, float* rep_out, void* ws,
                      size_t ws_bytes, void* stream);

/* Single-token selection (HiSA issue, HiSA decode path; L must be 1).  The gate
 * runs per sequence: dense -> I = 0..Np-1; flat -> the flat top-k; HiSA ->
 * coarse top-Kb blocks then the fine top-k within them (the tail rows
 * [nb*b, Np) are never selected).
 * Workspace: its first B * (1 + ceil(ceil(Np_cap / 64) / 16)) * 64 bytes are
 * arrival counters of the fused scan + selection kernel.  They must be zero
 * before the first call that uses the workspace (zero-fill it once after
 * allocating it); every call leaves them zero.  The region grows with B and
 * Np_cap: before a call with a larger region than the previous calls on the
 * workspace, zero it again.  Two calls that share a workspace must not run at
 * the same time (on different streams); calls on one stream are ordered.
 *   I_out       (B, 1, topk) int32.
 *   top_blk_out (B, 1, index_keep) int32 or NULL: the retained blocks (HiSA
 *               path only, ascending; -1 elsewhere).
 *   path_out    (B) int32 or NULL: enum hisa_path per sequence. */
int hisa_select_decode(const hisa_dims* d, const void* q_idx, const float* w, const void* keys,
                       const int32_t* t0, int32_t* I_out, int32_t* top_blk_out, int32_t* path_out,
                       void* ws, size_t ws_bytes, void* stream);

/* Decode selection on cached block means (HiSA issue, HiSA decode path: the
 * coarse stage costs O(nb) scores and the fine stage O(Kb * b), so a step need
 * not read every key; The pooled stream and positions: the pooled stream only
 * grows in whole windows, so the mean of a complete block never changes).
 * Same gate, outputs and tie rule as hisa_select_decode, and L >= 1: a decode
 * step (L = 1) or a short multi-token verify chunk, whose rows each select on
 * their own with the masks of the HiSA batched path (B * L <= 65535).  The
 * block means come from rep, a caller-owned (B, nb_cap, D_i) f32 cache,
 * nb_cap = Np_cap / index_block, row beta of sequence b holding the mean of
 * its pooled key rows beta*b .. beta*b + b - 1 (rows summed in order in f32,
 * then scaled by 1/b).  Before the call rep must hold every block completed
 * before this step (all blocks below floor(floor(t0 / ratio) / index_block));
 * the call computes the blocks this step's tokens complete, if any, from the
 * keys and writes them into rep, so calling it step after step keeps the
 * cache current.  hisa_block_means_update fills a cache (e.g. after a prefill
 * chunk).  A step reads nb * D_i * 4 bytes of means and at most
 * index_keep * index_block key rows instead of all Np_b key rows.
 * Shapes: bf16 keys, H_i = 64, D_i = 128, index_block > 0, nb_cap <= 4096,
 * index_keep <= 64, topk <= index_block * index_keep <= 1024, mode not
 * HISA_MODE_FORCE_FLAT (HISA_ERR_ARG otherwise; use hisa_select_decode).
 * HISA_MODE_FORCE_DENSE behaves as in hisa_select_decode and leaves rep alone.
 * Workspace: its first part holds arrival counters and, with index_block >= 16
 * (both stages in one launch), the words that hand each row's kept blocks to
 * its fine stage, under the same rule as hisa_select_decode's counters (zero
 * before first use, left zero; zero again before a call with a larger B, L or
 * Np_cap); an int after the counters becomes 1 if such a hand-off ever timed
 * out (its bounded wait, about a second). */
int hisa_select_decode_cached(const hisa_dims* d, const void* q_idx, const float* w, const void* keys,
                              float* rep, const int32_t* t0, int32_t* I_out, int32_t* top_blk_out,
                              int32_t* path_out, void* ws, size_t ws_bytes, void* stream);

/* Block means of the blocks that the step's L tokens complete, written into
 * the cache rep (B, nb_cap, D_i) f32 of hisa_select_decode_cached: blocks beta
 * with floor(floor(t0 / ratio) / b) <= beta < floor(Np_b / b), where
 * Np_b = floor((t0 + L) / ratio).  With t0 = 0 and L the tokens so far, every
 * complete block.  Other rows of rep are left alone.  idx_dtype bf16 or f32;
 * needs index_block > 0; no workspace. */
int hisa_block_means_update(const hisa_dims* d, const void* keys, const int32_t* t0, float* rep,
                            void* stream);

/* hisa_select_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, kernels and outputs as hisa_select_decode, but
 * no caller workspace: the library keeps a HISA_DECODE_NOALLOC_MAX_BYTES
 * workspace per GPU in a static device array (held from the first call on
 * that GPU until the process ends) and zeroes its arrival counters at the
 * start of every call, so no zero-fill contract applies.  It never calls
 * hipMalloc or hipFree.
 * Limits and errors: dims whose hisa_workspace_bytes(HISA_OP_SELECT_DECODE)
 * exceeds HISA_DECODE_NOALLOC_MAX_BYTES give HISA_ERR_WORKSPACE (about
 * B * Np_cap * 4 bytes: e.g. B = 32 at Np_cap = 32768 needs 4.3 MB); the
 * stream must run on the current device (HISA_ERR_ARG otherwise).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or threads without ordering) race and must not
 * be issued; calls on one stream are ordered. */
#define HISA_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)
int hisa_select_decode_noalloc(const hisa_dims* d, const void* q_idx, const float* w, const void* keys,
                               const int32_t* t0, int32_t* I_out, int32_t* top_blk_out, int32_t* path_out,
                               void* stream);

/* Multi-row selection (HiSA issue, HiSA batched path: prefill chunks and
 * multi-token verify; any L >= 1).  Chunks of at most 192 query rows in all
 * (B * L; verify and short chunks) take the cached-means kernels of
 * hisa_select_decode_cached on block means computed into the workspace.  Per query row j: valid_len = V(t0+j);
 * blocks with b*beta >= valid_len score -1e30; candidates at or past
 * valid_len score -1e30.  Rows with fewer than k visible rows then carry
 * masked ids, which the attention call re-masks.
 *   I_out (B, L, topk), top_blk_out (B, L, index_keep) or NULL, path_out (B) or NULL. */
int hisa_select_prefill(const hisa_dims* d, const void* q_idx, const float* w, const void* keys,
                        const int32_t* t0, int32_t* I_out, int32_t* top_blk_out, int32_t* path_out,
                        void* ws, size_t ws_bytes, void* stream);

/* The flat top-k indexer (HiSA issue, Flat selection; DSA issue, item 1):
 * score every visible row, -1e30 for p >= V(t0+j), keep the top
 * k = min(topk, Np) ids.  Ignores mode and index_block.  ratio = 1 gives the
 * per-token DSA indexer.
 *   I_out (B, L, topk) int32. */
int flat_topk_select(const hisa_dims* d, const void* q_idx, const float* w, const void* keys,
                     const int32_t* t0, int32_t* I_out, void* ws, size_t ws_bytes, void* stream);

/* The sparse local+pooled combine (HiSA issue, Consuming the selection:
 * sparse combine; DSA issue, item 3: gather, not mask).  For query row j at
 * t = t0 + j and each head h: one softmax over
 *   - the local rows at positions s with t - window < s <= t, and
 *   - the pooled rows I[b, j, kk] with 0 <= id < V(t) (others are masked),
 * plus the sink logit sinks[h] in the normaliser (mass, no value); scores are
 * (q * Dk^-1/2) . row; K = V with one shared KV head; the value of a row is its
 * first Dv entries.  No visible key and no sink gives 0.
 *   q         (B, L, H, Dk) attn_dtype, already roped.
 *   local_kv  (B, Wl_cap, Dk) attn_dtype: row r holds absolute position
 *             ls + r, ls = max(0, t0[b] - window + 1); rows run through
 *             position t0[b] + L - 1.
 *   pooled_kv (B, Np_cap, Dk) attn_dtype: the attention compressor's pooled rows.
 *   I         (B, L, kI) int32: pooled ids from a selection call (or any ids),
 *             or NULL for dense attention over every visible pooled row (the
 *             sparse combine's dense branch, Np <= index_topk, and layers
 *             without an indexer such as the ratio-128 ones; HiSA issue,
 *             Dependency and Consuming the selection): kI must then equal
 *             Np_cap, and entry e of the list is pooled row e.
 *   sinks     (H) f32 or NULL.
 *   out       (B, L, H, Dv) attn_dtype. */
int sparse_local_pooled_attention(const hisa_dims* d, const void* q, const void* local_kv,
                                  const void* pooled_kv, const int32_t* I, const float* sinks,
                                  const int32_t* t0, void* out, void* ws, size_t ws_bytes,
                                  void* stream);

/* sparse_local_pooled_attention with the local window kept as a ring, the way
 * a sliding-window KV cache of fixed capacity is written (hf2q source,
 * forward_compressed_attention_rows: the window cache holds sliding_window
 * rows and each token is written at the cache's write slot).  local_ring
 * (B, Wl_cap, Dk): position s of sequence b sits in slot
 * (ring_slot[b] + s - t0[b]) mod Wl_cap, where ring_slot (B) int32 (device)
 * holds the slot of position t0[b]; ring_slot NULL means slot t0[b] mod
 * Wl_cap.  Every position the step's rows see, t0 - window + 1 .. t0 + L - 1,
 * must be present, so Wl_cap >= window + L - 1 (HISA_ERR_ARG otherwise): a
 * decode step's ring is the window itself.  A sequence whose ring_slot is
 * outside [0, Wl_cap) is not computed (output 0).  Everything else, including
 * the workspace (hisa_workspace_bytes(HISA_OP_ATTENTION, d)), is as in
 * sparse_local_pooled_attention. */
int sparse_local_pooled_attention_ring(const hisa_dims* d, const void* q, const void* local_ring,
                                       const void* pooled_kv, const int32_t* I, const float* sinks,
                                       const int32_t* t0, const int32_t* ring_slot, void* out, void* ws,
                                       size_t ws_bytes, void* stream);

/* A whole decode step: hisa_select_decode, then sparse_local_pooled_attention
 * on the index row it produced (HiSA issue, HiSA decode path, then Consuming
 * the selection: sparse combine).  L must be 1; kI is taken to be topk and
 * the local window is linear (as in sparse_local_pooled_attention).  Outputs:
 * I_out, top_blk_out (or NULL) and path_out (or NULL) exactly as
 * hisa_select_decode writes them, and out (B, 1, H, Dv) as the attention call
 * computes it on I_out, up to f32 rounding (the softmax is split and merged
 * differently).
 * For few sequences of the shapes the one-kernel step serves (bf16 keys with
 * H_i = 64, D_i = 128, index_block 16, 32 or 64, index_keep * index_block and
 * topk <= 1024; bf16 attention with Dk = Dv = 512, H a multiple of 16; at most
 * 1024 key slabs of 64 rows over the batch; S = ceil(max(index_keep *
 * index_block, topk) / 64) + ceil(window / 64) attention splits per sequence,
 * at most 24, and H/16 * 8 * ceil(B * S / 8) attention workgroups (the head
 * groups of a split on one XCD), at most the device's compute units) the step
 * is one kernel: the attention of the kept blocks gathers and
 * scores their rows as soon as the coarse stage has chosen them, while the
 * fine top-k is still running, and the local window is attended from the
 * start.  Otherwise (and under HISA_MODE_FORCE_DENSE) it runs the two calls'
 * kernels one after the other.  The selected set is hisa_select_decode's in
 * both cases.
 * Workspace (hisa_workspace_bytes(HISA_OP_DECODE_STEP, d)): its first part
 * holds synchronisation words and the arrival counters of hisa_select_decode;
 * like those counters it must be zero before the first call that uses the
 * workspace, every call leaves it zero, and it must be zeroed again before a
 * call whose B, H, Np_cap, topk, index_block or index_keep is larger than
 * those of earlier calls on it.  Its first int32 becomes 1 if one of the
 * one-kernel step's bounded waits ever gave up (never expected: that call's
 * outputs are then undefined and the region must be zeroed again).  Calls
 * that share a workspace must not overlap. */
int hisa_decode_step(const hisa_dims* d, const void* q_idx, const float* w, const void* keys, const void* q,
                     const void* local_kv, const void* pooled_kv, const float* sinks, const int32_t* t0,
                     int32_t* I_out, int32_t* top_blk_out, int32_t* path_out, void* out, void* ws,
                     size_t ws_bytes, void* stream);

/* Workspace bytes the call `op` (enum hisa_op) needs for dims d (>= 256-byte
 * aligned offsets inside); 0 when it needs none.  Returns (size_t)-1 for
 * invalid dims (see hisa_last_error). */
size_t hisa_workspace_bytes(int op, const hisa_dims* d);

/* Human-readable reason of the last error on this thread ("" if none). */
const char* hisa_last_error(void);

/* HISA_ABI_VERSION of the loaded library. */
int hisa_abi_version(void);

/* Kernel timing, a tracing aid (off by default).  While enabled, each kernel
 * the library launches is bracketed by two hipEvents recorded on the call's
 * stream (timing-only events, created with hipEventDisableSystemFence, so the
 * interval holds the launch and not a system-scope cache writeback).
 * hisa_profile_collect() waits for the recorded events, adds their
 * elapsed times to per-kernel totals, copies up to max_entries totals to out
 * and returns how many kernels have totals (or a negative HISA_ERR_*).
 * hisa_profile_enable(0) stops recording and clears the totals.  Not
 * thread-safe; do not enable it while a HIP graph is being captured. */
typedef struct {
  char name[48];      /* kernel family, e.g. "decode_scan" */
  int64_t launches;   /* launches timed since the totals were cleared */
  double total_ms;    /* sum of their event-to-event durations */
} hisa_kernel_time;

int hisa_profile_enable(int on);
int hisa_profile_collect(hisa_kernel_time* out, int max_entries);

#ifdef __cplusplus
}
#endif
#endif /* HISA_H */
