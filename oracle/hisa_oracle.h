/*
 * hisa_oracle.h -- plain CPU oracle for HiSA hierarchical sparse selection,
 * the flat top-k indexer and the sparse local+pooled combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no header, helper or constant with the HIP
 * library; it has its own dims struct and its own definitions.
 *
 * Sources (the pages):
 *   [HiSA issue]  GitHub lablup/mlxcel issue #549, "feat(deepseek-v4): implement
 *                 HiSA hierarchical sparse attention", sections Conventions,
 *                 The pooled stream and positions, The indexer query and per-head
 *                 weights, Flat selection, HiSA decode path, HiSA batched path,
 *                 Consuming the selection: sparse combine, Engagement thresholds.
 *   [DSA issue]   GitHub lablup/mlxcel issue #509, "implement the DeepSeek Sparse
 *                 Attention (DSA) indexer", section What needs to be built, item 1.
 *
 * Precision: every sum is accumulated in double.  Selection scores are then
 * rounded once to float, because the HiSA issue (Conventions) fixes selection
 * scoring at f32, and every top-k decision is taken on those float values.
 * bf16 inputs reach the oracle as floats holding the same values (exact upcast).
 *
 * All arrays are dense row-major in the axis order given at each function.
 */
#ifndef HISA_ORACLE_H
#define HISA_ORACLE_H
#ifdef __cplusplus
extern "C" {
#endif

/* Problem sizes.  Field meanings follow the HiSA issue's Configuration table:
 * topk = index_topk, index_block = b, index_keep = Kb bound, H_i/D_i = indexer
 * heads/head dim, H/Dk/Dv = main attention heads and key/value widths. */
typedef struct {
  int B, L, ratio, window, topk, index_block, index_keep;
  int H_i, D_i, H, Dk, Dv, Np_cap;
  int force_flat;  /* 1: skip the hierarchy (the "force flat scan" kill-switch) */
  int force_dense; /* 1: no indexer at all (the dense-fallback kill-switch) */
} orc_dims;

enum { ORC_PATH_DENSE = 0, ORC_PATH_FLAT = 1, ORC_PATH_HISA = 2 };

/* The large negative finite mask value of the selection paths (never -inf). */
#define ORC_NEG (-1e30f)

int orc_num_pooled(int t0, int L, int ratio);
int orc_visible(int t, int ratio, int Np);
int orc_gate(const orc_dims* d, int Np);

float orc_score(const orc_dims* d, const float* q_row, const float* w_row, const float* key);
float orc_score_rep(const orc_dims* d, const float* q_row, const float* w_row, const double* rep);
void orc_block_mean(const orc_dims* d, const float* keys_b, int beta, double* rep);
int orc_topk(const float* s, const int* ids, int n, int k, int* out);

void orc_select_row(const orc_dims* d, const float* q_row, const float* w_row,
                    const float* keys_b, int t0, int j, const int* given_blocks,
                    int* I_row, int* blk_row, int* path);
void orc_select(const orc_dims* d, const float* q, const float* w, const float* keys,
                const int* t0, int* I, int* blk, int* path);
void orc_coarse_row(const orc_dims* d, const float* q_row, const float* w_row, const float* keys_b,
                    int t0, int j, float* cscore_row);
void orc_block_scores(const orc_dims* d, const float* q, const float* w, const float* keys,
                      const int* t0, float* cscore, float* rep);
void orc_scores_of(const orc_dims* d, const float* q_row, const float* w_row,
                   const float* keys_b, int t0, int j, const int* ids, int n, float* out);

void orc_combine_row(const orc_dims* d, const float* q_row, const float* local_b,
                     const float* pooled_b, const int* I_row, int kI, const float* sinks,
                     int t0, int j, double* out);
void orc_combine(const orc_dims* d, const float* q, const float* local_kv,
                 const float* pooled_kv, const int* I, int kI, const float* sinks,
                 const int* t0, int Wl_cap, double* out);

#ifdef __cplusplus
}
#endif
#endif
