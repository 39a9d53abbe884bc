/*
 * msa_oracle.c — plain, slow, fp64 CPU oracle of the MSA layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing here is part of the product path: only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark load
 * this library. It shares no code with the HIP kernels (only the seeded input
 * generator feeds both sides).
 *
 * Every quantity is the plain definition from the pages, evaluated in double
 * precision from the exact input values (fp32 or bf16 bit patterns), one query
 * row at a time, with per-row scratch only (never an N x N buffer). Rows are
 * independent, so any subset of rows can be evaluated on its own.
 *
 * Sources (web pages; cited by title and section):
 *  [Indexer]  "MSA Indexer 与 DSA Lightning Indexer 的差别" (MSA vs DSA indexer note)
 *  [KL]       "MSA 中的 KL 对齐与局部知识蒸馏" (MSA KL alignment note)
 *  [Blog]     "MiniMax Sparse Attention：教长上下文模型使用索引" (MSA blog post)
 *  [Native]   "2.4 · 训练原生稀疏" (training-native sparse attention)
 *  [Superv]   "4.1.1 · 监督与联合训练" (selector supervision and joint training)
 *
 * Readings where the pages leave a step open (each also listed in the design notes):
 *  - the forced local block counts inside k; the other k-1 slots take the best
 *    earlier blocks;
 *  - equal block scores rank the lower block index first;
 *  - with fewer than k visible blocks, all visible blocks are selected and the
 *    rest of the list is -1;
 *  - the selected ids are written in ascending order;
 *  - the main-branch softmax scale is 1/sqrt(head_dim);
 *  - query head h belongs to GQA group floor(h / G);
 *  - the teacher is normalised over the selected support J (sparse stage);
 *  - the KL mean is taken over all (batch, query, group) rows.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t batch, seqlen_kv, seqlen_q, q_start, num_q_heads, num_kv_heads;
  int32_t head_dim, idx_dim, block_size, topk, dtype; /* dtype: 0 fp32, 1 bf16 bits */
} msa_ref_shape;

enum { REF_OK = 0, REF_ERR_ARG = 1 };

/* Exact value of element idx of an fp32 or bf16 array, as a double. */
static double ld(const void* p, int dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float*)p)[idx];
  uint32_t u = ((uint32_t)((const uint16_t*)p)[idx]) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static int shape_ok(const msa_ref_shape* s) {
  if (!s) return 0;
  if (s->batch < 0 || s->seqlen_kv < 0 || s->seqlen_q < 0 || s->q_start < 0) return 0;
  if (s->num_kv_heads < 1 || s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads) return 0;
  if (s->head_dim < 1 || s->idx_dim < 1 || s->block_size < 1 || s->topk < 1) return 0;
  if ((int64_t)s->q_start + s->seqlen_q > s->seqlen_kv) return 0;
  if (s->dtype != 0 && s->dtype != 1) return 0;
  return 1;
}

static int num_blocks(const msa_ref_shape* s) {
  return (s->seqlen_kv + s->block_size - 1) / s->block_size;
}

/* ------------------------------------------------------------------------ selection */

/* Ranking of [Indexer] §2.2 with the tie rule: block a outranks block b when its
 * score is larger, or the scores are equal and a has the lower index. */
static int outranks(const double* M, int a, int b) {
  return M[a] > M[b] || (M[a] == M[b] && a < b);
}

/*
 * Block selection for one (query, group) row. M[0..L] are the block scores,
 * L = the query's own (local) block.
 *  - [Indexer] §2.2: take the top-k blocks by block score; the final recipe
 *    always includes the query's local incomplete block.
 *  - [Blog] "索引分支如何选择区块": the most recent local block is always
 *    included, even when its learned score is low.
 *  - [Blog] "系统教训": softmax preserves order, so the top-k is taken on raw
 *    scores.
 * Writes ids[0..k-1] ascending, -1 padded. *margin (optional) is the cutoff
 * margin of [Superv] eq. (9) over the non-local candidates: score of the last
 * block taken minus score of the best block left out, +inf when nothing is left
 * out.
 */
int msa_ref_topk_row(const double* M, int L, int k, int32_t* ids, double* margin) {
  if (!M || !ids || L < 0 || k < 1) return REF_ERR_ARG;
  for (int s = 0; s < k; ++s) ids[s] = -1;
  if (L + 1 <= k) {
    for (int b = 0; b <= L; ++b) ids[b] = b;
    if (margin) *margin = INFINITY;
    return REF_OK;
  }
  /* k-1 rounds of "take the best block not yet taken" among blocks 0..L-1 */
  unsigned char* taken = (unsigned char*)calloc((size_t)L, 1);
  if (!taken) return REF_ERR_ARG;
  int last = -1;
  for (int round = 0; round < k - 1; ++round) {
    int best = -1;
    for (int b = 0; b < L; ++b)
      if (!taken[b] && (best < 0 || outranks(M, b, best))) best = b;
    taken[best] = 1;
    last = best;
  }
  if (margin) {
    int next = -1;
    for (int b = 0; b < L; ++b)
      if (!taken[b] && (next < 0 || outranks(M, b, next))) next = b;
    *margin = (last >= 0 && next >= 0) ? M[last] - M[next] : INFINITY;
  }
  int n = 0;
  for (int b = 0; b < L; ++b)
    if (taken[b]) ids[n++] = b;
  ids[n++] = L; /* the forced local block is the largest index */
  free(taken);
  return REF_OK;
}

/*
 * Index logits, block scores and selection for the listed query rows.
 *  - [Indexer] §2.1: S_idx[i,j] = Q_idx[i,r] . K_idx[j] / sqrt(d_idx), with Hkv
 *    index-query heads (one per GQA group) and one shared index-key head.
 *  - [Indexer] §2.2: M[i,b] = max over tokens j of block b with j <= i.
 *  - [KL] §6: the index forward can keep a per-block log-sum-exp; block_lse
 *    (optional) is logsumexp over the same causally visible tokens of block b.
 * q_idx is compact: [nrows, Hkv, d_idx] for the listed rows; k_idx is the full
 * [B, N, d_idx]. rows[q] = b*Nq + t (NULL = all rows in order).
 * Outputs per listed row: ids [nrows, Hkv, k]; block_scores / block_lse
 * [nrows, Hkv, nb] (entries after the local block are -inf); margin [nrows, Hkv].
 */
int msa_ref_select(const msa_ref_shape* s, const void* q_idx, const void* k_idx,
                   const int64_t* rows, int64_t nrows, int32_t* ids, double* block_scores,
                   double* block_lse, double* margin, int nthreads) {
  if (!shape_ok(s) || !q_idx || !k_idx || !ids || nrows < 0) return REF_ERR_ARG;
  const int Hkv = s->num_kv_heads, di = s->idx_dim, Bk = s->block_size, k = s->topk;
  const int nb = num_blocks(s);
  const int64_t N = s->seqlen_kv, Nq = s->seqlen_q;
  const double inv_sqrt_di = 1.0 / sqrt((double)di);
  if (nthreads < 1) nthreads = 1;
  int err = 0;
#pragma omp parallel num_threads(nthreads)
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* M = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    double* ql = (double*)malloc(sizeof(double) * (size_t)di);
    if (!sc || !M || !ql) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < nrows; ++q) {
      if (err) continue;
      const int64_t row = rows ? rows[q] : q;
      const int64_t b = row / (Nq > 0 ? Nq : 1), t = row % (Nq > 0 ? Nq : 1);
      const int64_t i = s->q_start + t;
      const int L = (int)(i / Bk);
      for (int r = 0; r < Hkv; ++r) {
        for (int c = 0; c < di; ++c) ql[c] = ld(q_idx, s->dtype, (q * Hkv + r) * di + c);
        for (int64_t j = 0; j <= i; ++j) {
          double acc = 0.0;
          for (int c = 0; c < di; ++c) acc += ql[c] * ld(k_idx, s->dtype, (b * N + j) * di + c);
          sc[j] = acc * inv_sqrt_di;
        }
        for (int blk = 0; blk <= L; ++blk) {
          const int64_t j0 = (int64_t)blk * Bk;
          int64_t j1 = j0 + Bk - 1;
          if (j1 > i) j1 = i;
          double m = -INFINITY;
          for (int64_t j = j0; j <= j1; ++j) m = sc[j] > m ? sc[j] : m;
          M[blk] = m;
          if (block_lse) {
            double z = 0.0;
            for (int64_t j = j0; j <= j1; ++j) z += exp(sc[j] - m);
            block_lse[(q * Hkv + r) * nb + blk] = m + log(z);
          }
        }
        if (block_scores)
          for (int blk = 0; blk < nb; ++blk)
            block_scores[(q * Hkv + r) * nb + blk] = blk <= L ? M[blk] : -INFINITY;
        if (block_lse)
          for (int blk = L + 1; blk < nb; ++blk) block_lse[(q * Hkv + r) * nb + blk] = -INFINITY;
        double mg;
        msa_ref_topk_row(M, L, k, ids + (q * Hkv + r) * k, &mg);
        if (margin) margin[q * Hkv + r] = mg;
      }
    }
    free(sc);
    free(M);
    free(ql);
  }
  return err ? REF_ERR_ARG : REF_OK;
}

/* ------------------------------------------------------------------------ support */

/* Support J of one (query, group) row ([KL] §2): causally visible tokens
 * (j <= i) of the selected blocks, in ascending block order. Returns |J|;
 * slot[] and off[] give each token's list position and offset in its block. */
static int64_t support(const int32_t* ids, int k, int Bk, int64_t i, int64_t N, int64_t* J,
                       int* slot, int* off) {
  int64_t n = 0;
  for (int sl = 0; sl < k; ++sl) {
    const int32_t blk = ids[sl];
    if (blk < 0) continue;
    for (int o = 0; o < Bk; ++o) {
      const int64_t j = (int64_t)blk * Bk + o;
      if (j > i || j >= N) break;
      J[n] = j;
      if (slot) slot[n] = sl;
      if (off) off[n] = o;
      ++n;
    }
  }
  return n;
}

/* ------------------------------------------------------------------------ attention */

/*
 * Exact softmax attention of each query head over the selected support.
 *  - [Native] eq. (2): softmax with the denominator restricted to the selected
 *    set, output = sum of weights times values.
 *  - [Blog] "核心思想": the main branch runs standard scaled dot-product
 *    softmax attention on the tokens of the selected blocks; scale 1/sqrt(d).
 *  - [Indexer] §2.3: the G query heads of GQA group r share the group's block
 *    list and KV head r; each head keeps its own query.
 *  - [KL] §6: the forward also reports LSE_main per (query, head).
 * q is compact [nrows, Hq, d]; k, v are [B, N, Hkv, d]; ids [nrows, Hkv, k].
 * out [nrows, Hq, d], lse [nrows, Hq] (double).
 */
int msa_ref_attn(const msa_ref_shape* s, const void* q, const void* kk, const void* v,
                 const int32_t* ids, const int64_t* rows, int64_t nrows, double* out,
                 double* lse, int nthreads) {
  if (!shape_ok(s) || !q || !kk || !v || !ids || !out || nrows < 0) return REF_ERR_ARG;
  const int Hq = s->num_q_heads, Hkv = s->num_kv_heads, G = Hq / Hkv, d = s->head_dim;
  const int Bk = s->block_size, k = s->topk;
  const int64_t N = s->seqlen_kv, Nq = s->seqlen_q;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  if (nthreads < 1) nthreads = 1;
  int err = 0;
#pragma omp parallel num_threads(nthreads)
  {
    const int64_t cap = (int64_t)k * Bk;
    int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    double* sc = (double*)malloc(sizeof(double) * (size_t)cap);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!J || !sc || !o) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t qq = 0; qq < nrows; ++qq) {
      if (err) continue;
      const int64_t row = rows ? rows[qq] : qq;
      const int64_t b = row / (Nq > 0 ? Nq : 1), t = row % (Nq > 0 ? Nq : 1);
      const int64_t i = s->q_start + t;
      for (int r = 0; r < Hkv; ++r) {
        const int64_t n = support(ids + (qq * Hkv + r) * k, k, Bk, i, N, J, NULL, NULL);
        for (int h = r * G; h < (r + 1) * G; ++h) {
          double m = -INFINITY;
          for (int64_t a = 0; a < n; ++a) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
              acc += ld(q, s->dtype, (qq * Hq + h) * d + c) *
                     ld(kk, s->dtype, ((b * N + J[a]) * Hkv + r) * d + c);
            sc[a] = acc * inv_sqrt_d;
            m = sc[a] > m ? sc[a] : m;
          }
          double z = 0.0;
          for (int64_t a = 0; a < n; ++a) z += exp(sc[a] - m);
          const double LSE = m + log(z);
          for (int c = 0; c < d; ++c) o[c] = 0.0;
          for (int64_t a = 0; a < n; ++a) {
            const double w = exp(sc[a] - LSE);
            for (int c = 0; c < d; ++c) o[c] += w * ld(v, s->dtype, ((b * N + J[a]) * Hkv + r) * d + c);
          }
          for (int c = 0; c < d; ++c) out[(qq * Hq + h) * d + c] = n > 0 ? o[c] : 0.0;
          if (lse) lse[qq * Hq + h] = n > 0 ? LSE : -INFINITY;
        }
      }
    }
    free(J);
    free(sc);
    free(o);
  }
  return err ? REF_ERR_ARG : REF_OK;
}

/* ------------------------------------------------------------------------ KL alignment */

/*
 * KL alignment of one (query, group) row on a support of n tokens.
 *  s_main [G][n]: main-branch logits of the group's G heads on the support.
 *  s_idx  [n]   : index-branch logits z_j on the support.
 *  - [KL] §2.1: student P_idx = softmax of the index logits over J.
 *  - [KL] §2.2: teacher P = (1/G) sum over the group's heads of each head's
 *    own softmax over J (probabilities are averaged, not logits).
 *  - [KL] §3: D_KL(P || P_idx) = sum_j P_j log(P_j / P_idx_j); its gradient
 *    with respect to z_j is P_idx_j - P_j.
 *  - [Superv] eq. (15): p = exp(s - LSE).
 * Terms with P_j = 0 contribute 0. Writes *kl and, when dS != NULL,
 * dS[j] = P_idx_j - P_j. Optional outputs: P[n], P_idx[n], lse_idx.
 */
int msa_ref_kl_row(int G, int64_t n, const double* s_main, const double* s_idx, double* kl,
                   double* dS, double* P_out, double* Pidx_out, double* lse_idx_out) {
  if (G < 1 || n < 0 || (n > 0 && (!s_main || !s_idx)) || !kl) return REF_ERR_ARG;
  if (n == 0) {
    *kl = 0.0;
    if (lse_idx_out) *lse_idx_out = -INFINITY;
    return REF_OK;
  }
  double* P = (double*)calloc((size_t)n, sizeof(double));
  if (!P) return REF_ERR_ARG;
  for (int h = 0; h < G; ++h) {
    const double* sh = s_main + (int64_t)h * n;
    double m = -INFINITY;
    for (int64_t a = 0; a < n; ++a) m = sh[a] > m ? sh[a] : m;
    double z = 0.0;
    for (int64_t a = 0; a < n; ++a) z += exp(sh[a] - m);
    const double lse_h = m + log(z);
    for (int64_t a = 0; a < n; ++a) P[a] += exp(sh[a] - lse_h) / (double)G;
  }
  double m = -INFINITY;
  for (int64_t a = 0; a < n; ++a) m = s_idx[a] > m ? s_idx[a] : m;
  double z = 0.0;
  for (int64_t a = 0; a < n; ++a) z += exp(s_idx[a] - m);
  const double lse_idx = m + log(z);
  double acc = 0.0;
  for (int64_t a = 0; a < n; ++a) {
    const double pidx = exp(s_idx[a] - lse_idx);
    if (P[a] > 0.0) acc += P[a] * (log(P[a]) - (s_idx[a] - lse_idx));
    if (dS) dS[a] = pidx - P[a];
    if (P_out) P_out[a] = P[a];
    if (Pidx_out) Pidx_out[a] = pidx;
  }
  *kl = acc;
  if (lse_idx_out) *lse_idx_out = lse_idx;
  free(P);
  return REF_OK;
}

/*
 * KL alignment for the listed query rows ([KL] §2-§3, §6).
 * Recomputes the main logits S^(h) = q_h . k_j / sqrt(d) of the group's heads
 * and the index logits S_idx = q_idx . k_idx_j / sqrt(d_idx) on the support J
 * given by ids, then applies msa_ref_kl_row.
 * q, q_idx compact ([nrows, Hq, d], [nrows, Hkv, d_idx]); k [B,N,Hkv,d];
 * k_idx [B,N,d_idx]; ids [nrows, Hkv, k].
 * kl_rows [nrows, Hkv]; dlogits (optional) [nrows, Hkv, k, Bk] holds
 * P_idx - P at (slot, offset in block), 0 at masked or unused positions;
 * lse_idx (optional) [nrows, Hkv]; kl_mean (optional) = mean of kl_rows over
 * the listed rows and all groups ([KL] §3 averages over N*Hkv).
 * block_mass (optional) [nrows, Hkv, k]: the teacher's probability summed over
 * the support tokens of each slot's block ([KL] §8 score recall; 0 for unused
 * slots). With ids listing every block 0..floor(i/Bk) the support is the full
 * causal context ([KL] §5, warm-up) and these are the full-history block masses.
 */
int msa_ref_kl(const msa_ref_shape* s, const void* q, const void* kk, const void* q_idx,
               const void* k_idx, const int32_t* ids, const int64_t* rows, int64_t nrows,
               double* kl_rows, double* dlogits, double* lse_idx, double* kl_mean,
               double* block_mass, int nthreads) {
  if (!shape_ok(s) || !q || !kk || !q_idx || !k_idx || !ids || !kl_rows || nrows < 0)
    return REF_ERR_ARG;
  const int Hq = s->num_q_heads, Hkv = s->num_kv_heads, G = Hq / Hkv, d = s->head_dim;
  const int di = s->idx_dim, Bk = s->block_size, k = s->topk;
  const int64_t N = s->seqlen_kv, Nq = s->seqlen_q;
  const double inv_sqrt_d = 1.0 / sqrt((double)d), inv_sqrt_di = 1.0 / sqrt((double)di);
  if (nthreads < 1) nthreads = 1;
  int err = 0;
#pragma omp parallel num_threads(nthreads)
  {
    const int64_t cap = (int64_t)k * Bk;
    int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    int* slot = (int*)malloc(sizeof(int) * (size_t)cap);
    int* off = (int*)malloc(sizeof(int) * (size_t)cap);
    double* sm = (double*)malloc(sizeof(double) * (size_t)(cap * G));
    double* si = (double*)malloc(sizeof(double) * (size_t)cap);
    double* dS = (double*)malloc(sizeof(double) * (size_t)cap);
    double* Pt = (double*)malloc(sizeof(double) * (size_t)cap);
    if (!J || !slot || !off || !sm || !si || !dS || !Pt) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t qq = 0; qq < nrows; ++qq) {
      if (err) continue;
      const int64_t row = rows ? rows[qq] : qq;
      const int64_t b = row / (Nq > 0 ? Nq : 1), t = row % (Nq > 0 ? Nq : 1);
      const int64_t i = s->q_start + t;
      for (int r = 0; r < Hkv; ++r) {
        const int64_t n = support(ids + (qq * Hkv + r) * k, k, Bk, i, N, J, slot, off);
        for (int h = 0; h < G; ++h) {
          const int hq = r * G + h;
          for (int64_t a = 0; a < n; ++a) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
              acc += ld(q, s->dtype, (qq * Hq + hq) * d + c) *
                     ld(kk, s->dtype, ((b * N + J[a]) * Hkv + r) * d + c);
            sm[(int64_t)h * n + a] = acc * inv_sqrt_d;
          }
        }
        for (int64_t a = 0; a < n; ++a) {
          double acc = 0.0;
          for (int c = 0; c < di; ++c)
            acc += ld(q_idx, s->dtype, (qq * Hkv + r) * di + c) *
                   ld(k_idx, s->dtype, (b * N + J[a]) * di + c);
          si[a] = acc * inv_sqrt_di;
        }
        double kl, li;
        msa_ref_kl_row(G, n, sm, si, &kl, dS, Pt, NULL, &li);
        kl_rows[qq * Hkv + r] = kl;
        if (block_mass) {
          double* bm = block_mass + (qq * Hkv + r) * (int64_t)k;
          for (int sl = 0; sl < k; ++sl) bm[sl] = 0.0;
          for (int64_t a = 0; a < n; ++a) bm[slot[a]] += Pt[a];
        }
        if (lse_idx) lse_idx[qq * Hkv + r] = li;
        if (dlogits) {
          double* drow = dlogits + (qq * Hkv + r) * (int64_t)k * Bk;
          for (int64_t a = 0; a < (int64_t)k * Bk; ++a) drow[a] = 0.0;
          for (int64_t a = 0; a < n; ++a) drow[(int64_t)slot[a] * Bk + off[a]] = dS[a];
        }
      }
    }
    free(J);
    free(slot);
    free(off);
    free(sm);
    free(si);
    free(dS);
    free(Pt);
  }
  if (err) return REF_ERR_ARG;
  if (kl_mean) {
    double acc = 0.0;
    for (int64_t a = 0; a < nrows * Hkv; ++a) acc += kl_rows[a];
    *kl_mean = nrows > 0 ? acc / (double)(nrows * Hkv) : 0.0;
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ backward */

/*
 * Gradients of the sparse attention with the selection held fixed.
 *  - [Native] eq. (11): with alpha the softmax weights over the selected set,
 *    o the output and g = dL/do, the gradient of the logit z_s of a selected
 *    position is alpha_s g.(v_s - o); unselected positions get no gradient
 *    (eq. 12: the hard selection has zero derivative almost everywhere).
 *  - z_s = q.k_s / sqrt(d) ([Blog] "核心思想"), so dL/dq = sum_s dz_s k_s / sqrt(d),
 *    dL/dk_s = dz_s q / sqrt(d), and o = sum_s alpha_s v_s gives dL/dv_s = alpha_s g.
 *  - [Indexer] §2.3: the G heads of group r read KV head r, so k and v of group
 *    r collect the gradients of all G heads.
 * q and dout are compact [nrows, Hq, d] (dout in the input dtype); k, v are
 * [B, N, Hkv, d]; ids [nrows, Hkv, k]. Writes dq [nrows, Hq, d] and, summed
 * over the listed rows, dk and dv [B, N, Hkv, d] (double; fully overwritten;
 * both may be NULL to get dq alone). Rows run in parallel with per-thread
 * dk/dv sums added in thread order.
 */
int msa_ref_attn_bwd(const msa_ref_shape* s, const void* q, const void* kk, const void* v,
                     const int32_t* ids, const void* dout, const int64_t* rows, int64_t nrows,
                     double* dq, double* dk, double* dv, int nthreads) {
  if (!shape_ok(s) || !q || !kk || !v || !ids || !dout || !dq || nrows < 0 || (!dk != !dv))
    return REF_ERR_ARG;
  const int Hq = s->num_q_heads, Hkv = s->num_kv_heads, G = Hq / Hkv, d = s->head_dim;
  const int Bk = s->block_size, k = s->topk;
  const int64_t N = s->seqlen_kv, Nq = s->seqlen_q;
  const int64_t nkv = dk ? (int64_t)s->batch * N * Hkv * d : 0;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  if (nthreads < 1) nthreads = 1;
  double* part = nkv > 0 ? (double*)calloc((size_t)nthreads * 2 * (size_t)nkv, sizeof(double)) : NULL;
  if (!part && nkv > 0) return REF_ERR_ARG;
  int err = 0;
#pragma omp parallel num_threads(nthreads)
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* pdk = part ? part + (size_t)tid * 2 * (size_t)nkv : NULL;
    double* pdv = part ? pdk + nkv : NULL;
    const int64_t cap = (int64_t)k * Bk;
    int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
    double* z = (double*)malloc(sizeof(double) * (size_t)cap);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!J || !z || !o) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(static)
    for (int64_t qq = 0; qq < nrows; ++qq) {
      if (err) continue;
      const int64_t row = rows ? rows[qq] : qq;
      const int64_t b = row / (Nq > 0 ? Nq : 1), t = row % (Nq > 0 ? Nq : 1);
      const int64_t i = s->q_start + t;
      for (int r = 0; r < Hkv; ++r) {
        const int64_t n = support(ids + (qq * Hkv + r) * k, k, Bk, i, N, J, NULL, NULL);
        for (int h = r * G; h < (r + 1) * G; ++h) {
          double* dqh = dq + (qq * Hq + h) * d;
          for (int c = 0; c < d; ++c) dqh[c] = 0.0;
          if (n == 0) continue;
          /* forward on the support: logits, LSE, weights, output */
          double m = -INFINITY;
          for (int64_t a = 0; a < n; ++a) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
              acc += ld(q, s->dtype, (qq * Hq + h) * d + c) *
                     ld(kk, s->dtype, ((b * N + J[a]) * Hkv + r) * d + c);
            z[a] = acc * inv_sqrt_d;
            m = z[a] > m ? z[a] : m;
          }
          double zs = 0.0;
          for (int64_t a = 0; a < n; ++a) zs += exp(z[a] - m);
          const double LSE = m + log(zs);
          for (int c = 0; c < d; ++c) o[c] = 0.0;
          for (int64_t a = 0; a < n; ++a) {
            const double w = exp(z[a] - LSE);
            for (int c = 0; c < d; ++c) o[c] += w * ld(v, s->dtype, ((b * N + J[a]) * Hkv + r) * d + c);
          }
          double go = 0.0;
          for (int c = 0; c < d; ++c) go += ld(dout, s->dtype, (qq * Hq + h) * d + c) * o[c];
          /* eq. (11) per selected position, then the chain through z = q.k/sqrt(d) */
          for (int64_t a = 0; a < n; ++a) {
            const int64_t kv = ((b * N + J[a]) * Hkv + r) * d;
            const double alpha = exp(z[a] - LSE);
            double gv = 0.0;
            for (int c = 0; c < d; ++c) gv += ld(dout, s->dtype, (qq * Hq + h) * d + c) * ld(v, s->dtype, kv + c);
            const double dz = alpha * (gv - go);
            for (int c = 0; c < d; ++c) {
              const double gc = ld(dout, s->dtype, (qq * Hq + h) * d + c);
              dqh[c] += dz * ld(kk, s->dtype, kv + c) * inv_sqrt_d;
              if (pdk) {
                pdk[kv + c] += dz * ld(q, s->dtype, (qq * Hq + h) * d + c) * inv_sqrt_d;
                pdv[kv + c] += alpha * gc;
              }
            }
          }
        }
      }
    }
    free(J);
    free(z);
    free(o);
  }
  if (!err) {
    for (int64_t x = 0; x < nkv; ++x) {
      double sk = 0.0, sv = 0.0;
      for (int th = 0; th < nthreads; ++th) {
        sk += part[(size_t)th * 2 * (size_t)nkv + x];
        sv += part[(size_t)th * 2 * (size_t)nkv + nkv + x];
      }
      dk[x] = sk;
      dv[x] = sv;
    }
  }
  free(part);
  return err ? REF_ERR_ARG : REF_OK;
}

/*
 * Chain of the index-logit gradient into the index projections.
 *  - [Indexer] §2.1: S_idx[i,j] = q_idx[i,r] . k_idx[j] / sqrt(d_idx) with one
 *    k_idx head shared by every group r, so dL/dq_idx[i,r] = sum_j
 *    dS_idx[i,r,j] k_idx[j] / sqrt(d_idx) and dL/dk_idx[j] = sum over (i, r)
 *    of dS_idx[i,r,j] q_idx[i,r] / sqrt(d_idx).
 *  - [KL] §3: the gradient in the index logits is P_idx - P (dlogits, laid out
 *    [nrows, Hkv, k, Bk] by slot and offset in the slot's block, as
 *    msa_ref_kl writes it); coef carries the loss weight and the 1/(N Hkv) mean.
 * q_idx compact [nrows, Hkv, d_idx]; k_idx [B, N, d_idx]. Writes dq_idx
 * [nrows, Hkv, d_idx] and dk_idx [B, N, d_idx] summed over the listed rows
 * (double; fully overwritten). Sequential.
 */
int msa_ref_idx_bwd(const msa_ref_shape* s, const void* q_idx, const void* k_idx,
                    const int32_t* ids, const double* dlogits, double coef, const int64_t* rows,
                    int64_t nrows, double* dq_idx, double* dk_idx) {
  if (!shape_ok(s) || !q_idx || !k_idx || !ids || !dlogits || !dq_idx || !dk_idx || nrows < 0)
    return REF_ERR_ARG;
  const int Hkv = s->num_kv_heads, di = s->idx_dim, Bk = s->block_size, k = s->topk;
  const int64_t N = s->seqlen_kv, Nq = s->seqlen_q;
  const double sc = coef / sqrt((double)di);
  for (int64_t x = 0; x < (int64_t)s->batch * N * di; ++x) dk_idx[x] = 0.0;
  for (int64_t qq = 0; qq < nrows; ++qq) {
    const int64_t row = rows ? rows[qq] : qq;
    const int64_t b = row / (Nq > 0 ? Nq : 1), t = row % (Nq > 0 ? Nq : 1);
    const int64_t i = s->q_start + t;
    for (int r = 0; r < Hkv; ++r) {
      double* dqr = dq_idx + (qq * Hkv + r) * di;
      for (int c = 0; c < di; ++c) dqr[c] = 0.0;
      for (int sl = 0; sl < k; ++sl) {
        const int32_t blk = ids[(qq * Hkv + r) * k + sl];
        if (blk < 0) continue;
        for (int off = 0; off < Bk; ++off) {
          const int64_t j = (int64_t)blk * Bk + off;
          if (j > i || j >= N) break;
          const double g = dlogits[((qq * Hkv + r) * (int64_t)k + sl) * Bk + off] * sc;
          for (int c = 0; c < di; ++c) {
            dqr[c] += g * ld(k_idx, s->dtype, (b * N + j) * di + c);
            dk_idx[(b * N + j) * di + c] += g * ld(q_idx, s->dtype, (qq * Hkv + r) * di + c);
          }
        }
      }
    }
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ FP8 index scoring */

/*
 * FP8 variant of the index branch. [Indexer] §3.1 notes that the DSA indexer
 * can run in FP8; [Superv] after eq. (9) warns that a small cutoff margin lets
 * FP8 quantization flip candidates. The pages fix no format or scaling, so
 * (readings, also in the design notes):
 *  - format: OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3
 *    mantissa bits; no infinities; S.1111.111 is NaN, so the largest finite
 *    magnitude is 1.75 * 2^8 = 448; exponent field 0 holds subnormals m * 2^-9;
 *  - rounding: to the nearest E4M3 value, ties to the even code;
 *  - scales: a power of two 2^e per Q_idx row (b, t, r) and per 128-token
 *    K_idx block (b, blk): e is the smallest integer with amax <= 448 * 2^e
 *    (e = 0 when amax = 0), and the stored value is the E4M3 rounding of
 *    x * 2^-e (an exact scaling);
 *  - scores: S8_idx(i, j) = (sum_c q8_c k8_c) * 2^(e_q + e_k) / sqrt(d_idx), then
 *    the same causal block max and selection rule as msa_ref_select.
 */
static double e4m3_value(int code) {
  const int E = (code >> 3) & 15, m = code & 7;
  const double mag = E == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
  return (code & 0x80) ? -mag : mag;
}

/* Nearest E4M3 code to y (|y| <= 448), by comparing with every finite
 * non-negative code; on a tie the even code wins. */
uint8_t msa_ref_e4m3_encode(double y) {
  const double a = fabs(y);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    const double d = fabs(a - e4m3_value(c));
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

double msa_ref_e4m3_decode(uint8_t code) { return e4m3_value(code); }

/* smallest e with amax <= 448 * 2^e; 0 for amax = 0 */
int msa_ref_fp8_scale_exp(double amax) {
  if (!(amax > 0.0)) return 0;
  int e = 0;
  while (amax > ldexp(448.0, e)) ++e;
  while (amax <= ldexp(448.0, e - 1)) --e;
  return e;
}

/*
 * Quantize the index inputs: q8 [nrows, Hkv, d_idx] and q_exp [nrows, Hkv] for
 * the listed rows (q_idx compact [nrows, Hkv, d_idx]); when k8 != NULL also
 * k8 [B, N, d_idx] and k_exp [B, nb] (k_idx [B, N, d_idx]).
 */
int msa_ref_quantize_fp8(const msa_ref_shape* s, const void* q_idx, const void* k_idx,
                         int64_t nrows, uint8_t* q8, int32_t* q_exp, uint8_t* k8,
                         int32_t* k_exp, int nthreads) {
  if (!shape_ok(s) || nrows < 0 || (nrows > 0 && (!q_idx || !q8 || !q_exp)) ||
      (k8 && (!k_idx || !k_exp)))
    return REF_ERR_ARG;
  if (nthreads < 1) nthreads = 1;
  const int Hkv = s->num_kv_heads, di = s->idx_dim, Bk = s->block_size, nb = num_blocks(s);
  const int64_t N = s->seqlen_kv;
  /* rows and blocks are independent: threads split them, each writes its own outputs */
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t x = 0; x < nrows * Hkv; ++x) {
    double amax = 0.0;
    for (int c = 0; c < di; ++c) amax = fmax(amax, fabs(ld(q_idx, s->dtype, x * di + c)));
    const int e = msa_ref_fp8_scale_exp(amax);
    q_exp[x] = e;
    for (int c = 0; c < di; ++c)
      q8[x * di + c] = msa_ref_e4m3_encode(ldexp(ld(q_idx, s->dtype, x * di + c), -e));
  }
  if (k8) {
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t bb = 0; bb < (int64_t)s->batch * nb; ++bb) {
      const int64_t b = bb / nb;
      const int blk = (int)(bb % nb);
      const int64_t j0 = (int64_t)blk * Bk, j1 = j0 + Bk < N ? j0 + Bk : N;
      double amax = 0.0;
      for (int64_t j = j0; j < j1; ++j)
        for (int c = 0; c < di; ++c)
          amax = fmax(amax, fabs(ld(k_idx, s->dtype, (b * N + j) * di + c)));
      const int e = msa_ref_fp8_scale_exp(amax);
      k_exp[b * nb + blk] = e;
      for (int64_t j = j0; j < j1; ++j)
        for (int c = 0; c < di; ++c)
          k8[(b * N + j) * di + c] =
              msa_ref_e4m3_encode(ldexp(ld(k_idx, s->dtype, (b * N + j) * di + c), -e));
    }
  }
  return REF_OK;
}

/*
 * Selection from the quantized index inputs: msa_ref_select with the index
 * logits S8_idx above (exact products and sums of the E4M3 values in double).
 * q8 / q_exp compact for the listed rows; k8 [B, N, d_idx], k_exp [B, nb].
 */
int msa_ref_select_fp8(const msa_ref_shape* s, const uint8_t* q8, const int32_t* q_exp,
                       const uint8_t* k8, const int32_t* k_exp, const int64_t* rows,
                       int64_t nrows, int32_t* ids, double* block_scores, double* margin,
                       int nthreads) {
  if (!shape_ok(s) || !q8 || !q_exp || !k8 || !k_exp || !ids || nrows < 0) return REF_ERR_ARG;
  const int Hkv = s->num_kv_heads, di = s->idx_dim, Bk = s->block_size, k = s->topk;
  const int nb = num_blocks(s);
  const int64_t N = s->seqlen_kv, Nq = s->seqlen_q;
  const double inv_sqrt_di = 1.0 / sqrt((double)di);
  if (nthreads < 1) nthreads = 1;
  int err = 0;
#pragma omp parallel num_threads(nthreads)
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* M = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    double* ql = (double*)malloc(sizeof(double) * (size_t)di);
    if (!sc || !M || !ql) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < nrows; ++q) {
      if (err) continue;
      const int64_t row = rows ? rows[q] : q;
      const int64_t b = row / (Nq > 0 ? Nq : 1), t = row % (Nq > 0 ? Nq : 1);
      const int64_t i = s->q_start + t;
      const int L = (int)(i / Bk);
      for (int r = 0; r < Hkv; ++r) {
        for (int c = 0; c < di; ++c) ql[c] = e4m3_value(q8[(q * Hkv + r) * di + c]);
        for (int64_t j = 0; j <= i; ++j) {
          double acc = 0.0;
          for (int c = 0; c < di; ++c) acc += ql[c] * e4m3_value(k8[(b * N + j) * di + c]);
          const int e = q_exp[q * Hkv + r] + k_exp[b * nb + j / Bk];
          sc[j] = ldexp(acc, e) * inv_sqrt_di;
        }
        for (int blk = 0; blk <= L; ++blk) {
          const int64_t j0 = (int64_t)blk * Bk;
          int64_t j1 = j0 + Bk - 1;
          if (j1 > i) j1 = i;
          double m = -INFINITY;
          for (int64_t j = j0; j <= j1; ++j) m = sc[j] > m ? sc[j] : m;
          M[blk] = m;
        }
        if (block_scores)
          for (int blk = 0; blk < nb; ++blk)
            block_scores[(q * Hkv + r) * nb + blk] = blk <= L ? M[blk] : -INFINITY;
        double mg;
        msa_ref_topk_row(M, L, k, ids + (q * Hkv + r) * k, &mg);
        if (margin) margin[q * Hkv + r] = mg;
      }
    }
    free(sc);
    free(M);
    free(ql);
  }
  return err ? REF_ERR_ARG : REF_OK;
}
