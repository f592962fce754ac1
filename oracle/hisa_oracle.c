/*
 * hisa_oracle.c -- plain, slow, obviously correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the HIP library.
 *
 * Each function follows the named passage of the pages step by step, in the
 * pages' order and notation, with no blocking, fusion or reordering:
 *   [HiSA issue]  lablup/mlxcel #549 "feat(deepseek-v4): implement HiSA
 *                 hierarchical sparse attention".
 *   [DSA issue]   lablup/mlxcel #509 "implement the DeepSeek Sparse Attention
 *                 (DSA) indexer".
 * Sums accumulate in double; selection scores are rounded once to float and
 * every top-k decision is taken on those floats (HiSA issue, Conventions:
 * selection scoring in f32).  Exact ties are broken by the lowest id, a
 * deterministic choice inside the pages' "unordered" argpartition.
 */
#include "hisa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int imin(int a, int b) { return a < b ? a : b; }
static int imax(int a, int b) { return a > b ? a : b; }

/* [HiSA issue] "The pooled stream and positions": the pooled cache advances in
 * whole windows of r tokens, so after the step's L rows (t0 + L tokens) it
 * holds floor((t0 + L) / r) rows. */
int orc_num_pooled(int t0, int L, int ratio) {
  return (int)(((long long)t0 + (long long)L) / ratio);
}

/* [HiSA issue] "The pooled stream and positions", causal visibility: a query
 * at absolute position t sees pooled rows p < V(t) = min(Np, floor((t+1)/r)). */
int orc_visible(int t, int ratio, int Np) {
  return imin(Np, (int)(((long long)t + 1) / ratio));
}

/* [HiSA issue] "HiSA decode path" / "HiSA batched path" gate conditions and the
 * "Engagement thresholds" table; the sparse-combine section's branch 2 makes
 * Np <= index_topk the dense case.  Of the two kill-switches ("Implementation
 * plan", item 1), force-flat replaces only the hierarchy and force-dense turns
 * the indexer off altogether (every pooled row goes to the combine). */
int orc_gate(const orc_dims* d, int Np) {
  int k = imin(d->topk, Np);
  long long bk = (long long)d->index_block * d->index_keep;
  if (d->force_dense) return ORC_PATH_DENSE;
  if (Np <= d->topk) return ORC_PATH_DENSE;
  if (!d->force_flat && d->index_block > 0 && Np >= bk && bk >= k) return ORC_PATH_HISA;
  return ORC_PATH_FLAT;
}

static float finish_score(double acc) {
  float s = (float)acc;
  if (s == 0.0f) s = 0.0f; /* one zero: -0 and +0 are the same score */
  return s;
}

/* [HiSA issue] "Flat selection": per indexer head, the dot product of the
 * head's query with the key, clipped below at zero; the heads are then added
 * up, each weighted by its learned weight times 1/sqrt(H_i * D_i) (the H_i
 * factor from "The indexer query and per-head weights", the D_i factor from
 * the scoring step; the DSA issue, item 1, Score, states the same product).
 * q_row is (H_i, D_i), w_row is the raw weights_proj output (H_i). */
float orc_score(const orc_dims* d, const float* q_row, const float* w_row, const float* key) {
  const double c = 1.0 / sqrt((double)d->H_i * (double)d->D_i);
  double acc = 0.0;
  for (int h = 0; h < d->H_i; h++) {
    double dot = 0.0;
    for (int e = 0; e < d->D_i; e++) dot += (double)q_row[h * d->D_i + e] * (double)key[e];
    double s = dot > 0.0 ? dot : 0.0;
    acc += s * ((double)w_row[h] * c);
  }
  return finish_score(acc);
}

/* The same head combine with a block's mean row in place of a key (HiSA
 * decode path, coarse stage); the mean is given in double. */
float orc_score_rep(const orc_dims* d, const float* q_row, const float* w_row, const double* rep) {
  const double c = 1.0 / sqrt((double)d->H_i * (double)d->D_i);
  double acc = 0.0;
  for (int h = 0; h < d->H_i; h++) {
    double dot = 0.0;
    for (int e = 0; e < d->D_i; e++) dot += (double)q_row[h * d->D_i + e] * rep[e];
    double s = dot > 0.0 ? dot : 0.0;
    acc += s * ((double)w_row[h] * c);
  }
  return finish_score(acc);
}

/* [HiSA issue] "HiSA decode path", coarse stage: block beta is the b pooled
 * rows starting at beta * b; its representative is their elementwise mean. */
void orc_block_mean(const orc_dims* d, const float* keys_b, int beta, double* rep) {
  const int b = d->index_block;
  for (int e = 0; e < d->D_i; e++) {
    double s = 0.0;
    for (int p = beta * b; p < (beta + 1) * b; p++) s += (double)keys_b[(long long)p * d->D_i + e];
    rep[e] = s / (double)b;
  }
}

typedef struct {
  float s;
  int id;
} scored_id;

static int by_score_desc_id_asc(const void* pa, const void* pb) {
  const scored_id* a = (const scored_id*)pa;
  const scored_id* b = (const scored_id*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

static int by_int_asc(const void* pa, const void* pb) {
  int a = *(const int*)pa, b = *(const int*)pb;
  return (a > b) - (a < b);
}

/* argpartition_desc(score, k)[..., :k] ([HiSA issue] "Flat selection"): the k
 * ids with the largest scores.  Full sort by (score desc, id asc); the first k
 * are written to out in ascending id order.  Returns min(k, n). */
int orc_topk(const float* s, const int* ids, int n, int k, int* out) {
  if (k > n) k = n;
  if (k <= 0) return 0;
  scored_id* v = (scored_id*)malloc(sizeof(scored_id) * (size_t)n);
  for (int i = 0; i < n; i++) {
    v[i].s = s[i];
    v[i].id = ids[i];
  }
  qsort(v, (size_t)n, sizeof(scored_id), by_score_desc_id_asc);
  for (int i = 0; i < k; i++) out[i] = v[i].id;
  qsort(out, (size_t)k, sizeof(int), by_int_asc);
  free(v);
  return k;
}

/* One query row (b, j) of the selector.  Writes I_row[topk] (absolute pooled
 * ids, ascending, -1 padded), blk_row[index_keep] (retained blocks, ascending,
 * -1 padded; only the HiSA path fills it) and the path taken.
 * given_blocks (HiSA only, may be NULL) replaces the coarse stage's choice:
 * the fine stage then runs on those Kb blocks. */
void orc_select_row(const orc_dims* d, const float* q_row, const float* w_row,
                    const float* keys_b, int t0, int j, const int* given_blocks,
                    int* I_row, int* blk_row, int* path) {
  const int Np = orc_num_pooled(t0, d->L, d->ratio);
  const int valid = orc_visible(t0 + j, d->ratio, Np); /* valid_len[b, j] */
  const int k = imin(d->topk, Np);
  const int p = orc_gate(d, Np);
  for (int i = 0; i < d->topk; i++) I_row[i] = -1;
  for (int i = 0; i < d->index_keep; i++) blk_row[i] = -1;
  *path = p;

  if (p == ORC_PATH_DENSE) {
    /* Sparse combine, branch 2: every pooled row would be selected.  (Under
     * force-dense with Np > topk the row cannot hold them all; it keeps the
     * first topk, and callers size the index row to the pooled capacity.) */
    for (int i = 0; i < Np && i < d->topk; i++) I_row[i] = i;
    return;
  }

  if (p == ORC_PATH_FLAT) {
    /* [HiSA issue] "Flat selection"; [DSA issue] item 1, Score and Select. */
    float* s = (float*)malloc(sizeof(float) * (size_t)imax(Np, 1));
    int* ids = (int*)malloc(sizeof(int) * (size_t)imax(Np, 1));
    for (int q = 0; q < Np; q++) {
      ids[q] = q;
      s[q] = q < valid ? orc_score(d, q_row, w_row, keys_b + (long long)q * d->D_i) : ORC_NEG;
    }
    orc_topk(s, ids, Np, k, I_row);
    free(s);
    free(ids);
    return;
  }

  /* [HiSA issue] "HiSA decode path" (L == 1) and "HiSA batched path" (L > 1).
   * The decode path has no masks because valid == Np for its one row, so the
   * batched masks below leave it unchanged. */
  const int b = d->index_block;
  const int nb = Np / b;
  const int Kb = imin(d->index_keep, nb);
  const int C = Kb * b;
  int* top_blk = (int*)malloc(sizeof(int) * (size_t)Kb);

  if (given_blocks) {
    for (int i = 0; i < Kb; i++) top_blk[i] = given_blocks[i];
    qsort(top_blk, (size_t)Kb, sizeof(int), by_int_asc);
  } else {
    /* Coarse stage: each block is represented by the mean of its b key rows
     * and scored like a key.  For a row of a batched step a block takes part
     * only when its first pooled row is visible to that row; the others get
     * the mask value. */
    float* cs = (float*)malloc(sizeof(float) * (size_t)nb);
    int* bid = (int*)malloc(sizeof(int) * (size_t)nb);
    double* rep = (double*)malloc(sizeof(double) * (size_t)d->D_i);
    for (int beta = 0; beta < nb; beta++) {
      bid[beta] = beta;
      if (beta * b < valid) {
        orc_block_mean(d, keys_b, beta, rep);
        cs[beta] = orc_score_rep(d, q_row, w_row, rep);
      } else {
        cs[beta] = ORC_NEG;
      }
    }
    orc_topk(cs, bid, nb, Kb, top_blk);
    free(cs);
    free(bid);
    free(rep);
  }
  for (int i = 0; i < Kb; i++) blk_row[i] = top_blk[i];

  /* Fine stage: the candidates are every row of the retained blocks, block
   * after block in ascending block order (candidate c lies in retained block
   * c / b at offset c % b inside it).  Each candidate gets its full score,
   * the ones this row cannot see get the mask value, and the k best
   * candidates are reported by their absolute pooled row ids. */
  float* fs = (float*)malloc(sizeof(float) * (size_t)C);
  int* pos = (int*)malloc(sizeof(int) * (size_t)C);
  for (int c = 0; c < C; c++) {
    pos[c] = top_blk[c / b] * b + (c % b);
    fs[c] = pos[c] < valid ? orc_score(d, q_row, w_row, keys_b + (long long)pos[c] * d->D_i) : ORC_NEG;
  }
  orc_topk(fs, pos, C, k, I_row);
  free(fs);
  free(pos);
  free(top_blk);
}

/* All rows.  q (B, L, H_i, D_i), w (B, L, H_i), keys (B, Np_cap, D_i), t0 (B).
 * I (B, L, topk), blk (B, L, index_keep), path (B, L). */
void orc_select(const orc_dims* d, const float* q, const float* w, const float* keys,
                const int* t0, int* I, int* blk, int* path) {
  const long long rows = (long long)d->B * d->L;
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < rows; r++) {
    const int b = (int)(r / d->L), j = (int)(r % d->L);
    orc_select_row(d, q + r * d->H_i * d->D_i, w + r * d->H_i,
                   keys + (long long)b * d->Np_cap * d->D_i, t0[b], j, NULL,
                   I + r * d->topk, blk + r * d->index_keep, path + r);
  }
}

/* Coarse scores of one query row (b, j): cscore[beta] for beta < nb_cap,
 * with the batched eligibility mask (beta * b >= valid_len -> -1e30) and -1e30
 * past nb.  keys_b is sequence b's (Np_cap, D_i) keys. */
void orc_coarse_row(const orc_dims* d, const float* q_row, const float* w_row, const float* keys_b,
                    int t0, int j, float* cscore_row) {
  const int b = d->index_block;
  const int nb_cap = d->Np_cap / b;
  const int Np = orc_num_pooled(t0, d->L, d->ratio);
  const int nb = Np / b;
  const int valid = orc_visible(t0 + j, d->ratio, Np);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)d->D_i);
  for (int beta = 0; beta < nb_cap; beta++) {
    float v = ORC_NEG;
    if (beta < nb && beta * b < valid) {
      orc_block_mean(d, keys_b, beta, tmp);
      v = orc_score_rep(d, q_row, w_row, tmp);
    }
    cscore_row[beta] = v;
  }
  free(tmp);
}

/* The coarse stage alone: rep (B, nb_cap, D_i) rounded to float (zeros past
 * nb) and cscore (B, L, nb_cap) from orc_coarse_row.  nb_cap = Np_cap / b. */
void orc_block_scores(const orc_dims* d, const float* q, const float* w, const float* keys,
                      const int* t0, float* cscore, float* rep) {
  const int b = d->index_block;
  const int nb_cap = d->Np_cap / b;
  const long long rows = (long long)d->B * d->L;
  if (rep) {
    for (int bb = 0; bb < d->B; bb++) {
      const int nb = orc_num_pooled(t0[bb], d->L, d->ratio) / b;
#pragma omp parallel for schedule(static)
      for (int beta = 0; beta < nb_cap; beta++) {
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d->D_i);
        float* out = rep + ((long long)bb * nb_cap + beta) * d->D_i;
        if (beta < nb) {
          orc_block_mean(d, keys + (long long)bb * d->Np_cap * d->D_i, beta, tmp);
          for (int e = 0; e < d->D_i; e++) out[e] = (float)tmp[e];
        } else {
          for (int e = 0; e < d->D_i; e++) out[e] = 0.0f;
        }
        free(tmp);
      }
    }
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < rows; r++) {
    const int bb = (int)(r / d->L), j = (int)(r % d->L);
    orc_coarse_row(d, q + r * d->H_i * d->D_i, w + r * d->H_i,
                   keys + (long long)bb * d->Np_cap * d->D_i, t0[bb], j, cscore + r * nb_cap);
  }
}

/* Scores of given pooled ids for one row, masked like the flat path (used by
 * the tests to judge near-ties).  Ids outside [0, valid_len) give -1e30. */
void orc_scores_of(const orc_dims* d, const float* q_row, const float* w_row,
                   const float* keys_b, int t0, int j, const int* ids, int n, float* out) {
  const int Np = orc_num_pooled(t0, d->L, d->ratio);
  const int valid = orc_visible(t0 + j, d->ratio, Np);
  for (int i = 0; i < n; i++) {
    const int p = ids[i];
    out[i] = (p >= 0 && p < valid) ? orc_score(d, q_row, w_row, keys_b + (long long)p * d->D_i) : ORC_NEG;
  }
}

/* [HiSA issue] "Consuming the selection: sparse combine", one query row, all
 * heads.  The logaddexp normaliser n = log(sum_local e^s + sum_pooled e^s +
 * e^sink) makes the weights exp(s - n) one softmax over the union of both
 * streams plus the sink, and the sink adds no value; it is written here as
 * that softmax, shifted by the largest logit.
 *   q_row   (H, Dk), already roped; q_s = q * Dk^-1/2.
 *   local_b (Wl_cap, Dk): local row r holds absolute position ls + r with
 *           ls = max(0, t0 - window + 1); the query at t = t0 + j sees the
 *           positions s with t - window < s <= t (sliding window incl. t).
 *   pooled_b (Np_cap, Dk): the attention compressor's pooled rows.
 *   I_row (kI): pooled ids; entries < 0 or >= V(t) are masked (the -inf
 *           re-mask of gathered invisible rows).
 *   K = V: the value of a row is its first Dv entries.  One shared KV head.
 *   sinks (H) or NULL.  With no visible key and no sink the output is 0. */
void orc_combine_row(const orc_dims* d, const float* q_row, const float* local_b,
                     const float* pooled_b, const int* I_row, int kI, const float* sinks,
                     int t0, int j, double* out) {
  const int t = t0 + j;
  const int Np = orc_num_pooled(t0, d->L, d->ratio);
  const int V = orc_visible(t, d->ratio, Np);
  const int ls = imax(0, t0 - d->window + 1);
  const int s_lo = imax(ls, t - d->window + 1);
  const int n_local = d->window > 0 ? t - s_lo + 1 : 0;
  const double scale = 1.0 / sqrt((double)d->Dk);
  const int nmax = imax(n_local + kI, 1);
  const float** rows = (const float**)malloc(sizeof(float*) * (size_t)nmax);
  double* x = (double*)malloc(sizeof(double) * (size_t)nmax);
  int n = 0;
  for (int i = 0; i < n_local; i++) rows[n++] = local_b + (long long)(s_lo - ls + i) * d->Dk;
  for (int kk = 0; kk < kI; kk++) {
    const int id = I_row[kk];
    if (id >= 0 && id < V) rows[n++] = pooled_b + (long long)id * d->Dk;
  }
  for (int h = 0; h < d->H; h++) {
    const float* qh = q_row + (long long)h * d->Dk;
    double* oh = out + (long long)h * d->Dv;
    for (int e = 0; e < d->Dv; e++) oh[e] = 0.0;
    if (n == 0 && !sinks) continue;
    double m = sinks ? (double)sinks[h] : -INFINITY;
    for (int i = 0; i < n; i++) {
      double dot = 0.0;
      for (int e = 0; e < d->Dk; e++) dot += (double)qh[e] * scale * (double)rows[i][e];
      x[i] = dot;
      if (dot > m) m = dot;
    }
    double Z = sinks ? exp((double)sinks[h] - m) : 0.0;
    for (int i = 0; i < n; i++) Z += exp(x[i] - m);
    for (int i = 0; i < n; i++) {
      const double pw = exp(x[i] - m) / Z;
      for (int e = 0; e < d->Dv; e++) oh[e] += pw * (double)rows[i][e];
    }
  }
  free(rows);
  free(x);
}

/* All rows.  q (B, L, H, Dk), local_kv (B, Wl_cap, Dk), pooled_kv (B, Np_cap, Dk),
 * I (B, L, kI), sinks (H) or NULL, t0 (B) -> out (B, L, H, Dv) in double. */
void orc_combine(const orc_dims* d, const float* q, const float* local_kv,
                 const float* pooled_kv, const int* I, int kI, const float* sinks,
                 const int* t0, int Wl_cap, double* out) {
  const long long rows = (long long)d->B * d->L;
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < rows; r++) {
    const int b = (int)(r / d->L), j = (int)(r % d->L);
    orc_combine_row(d, q + r * d->H * d->Dk, local_kv + (long long)b * Wl_cap * d->Dk,
                    pooled_kv + (long long)b * d->Np_cap * d->Dk, I + r * kI, kI, sinks,
                    t0[b], j, out + r * d->H * d->Dv);
  }
}
