/*
 * msa.h — C ABI of the MSA (MiniMax Sparse Attention) layer hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The path, per query position i and GQA group r:
 *   index logits  S_idx[i,j] = Q_idx[i,r] . K_idx[j] / sqrt(d_idx), one shared
 *                 K_idx head ("MSA Indexer 与 DSA Lightning Indexer 的差别"
 *                 (MSA vs DSA indexer note) §2.1);
 *   block scores  M[i,b] = max over tokens j of 128-token block b with j <= i
 *                 (same note, §2.2);
 *   selection     the query's own (local) block plus the k-1 best earlier
 *                 blocks by raw score, no softmax (same note §2.2; "MiniMax
 *                 Sparse Attention：教长上下文模型使用索引" (MSA blog), sections
 *                 on block selection and on kernel design);
 *   attention     exact causal softmax attention of the group's G query heads
 *                 over the selected blocks only ("2.4 · 训练原生稀疏"
 *                 (training-native sparse attention) eq. 2), also reporting the
 *                 log-sum-exp per (query, head) ("MSA 中的 KL 对齐与局部知识蒸馏"
 *                 (MSA KL alignment note) §6);
 *   KL alignment  teacher = per-head softmax on the selected support averaged
 *                 over the group, student = index softmax on the same support,
 *                 KL(teacher || student) and its gradient P_idx - P in the
 *                 index logits (KL alignment note §2-§3, §6).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays:
 *      q      [batch, seqlen_q, num_q_heads, head_dim]
 *      k, v   [batch, seqlen_kv, num_kv_heads, head_dim]
 *      q_idx  [batch, seqlen_q, num_kv_heads, idx_dim]
 *      k_idx  [batch, seqlen_kv, idx_dim]
 *    element type fp32 (MSA_F32) or bf16 (MSA_BF16), all of the same type.
 *  - Query row t of a sequence sits at key position i = q_start + t (prefill:
 *    q_start = 0, seqlen_q = seqlen_kv; one decode step: q_start =
 *    seqlen_kv - 1, seqlen_q = 1). Keys j <= i are visible to it.
 *  - GQA: G = num_q_heads / num_kv_heads; query head h belongs to group h / G.
 *  - Scales: 1/sqrt(idx_dim) for index logits, 1/sqrt(head_dim) for the main
 *    attention. Logarithms are natural.
 *  - The caller owns every buffer, including the workspace (size from
 *    msa_workspace_size). The library allocates no memory, keeps no pointer
 *    past a call and does not synchronise: all work is enqueued on `stream`,
 *    and buffers must stay valid until that work has run. Calls on different
 *    streams with different workspaces may run concurrently. The workspace needs
 *    no initialisation: every call writes what it reads there, so its results
 *    do not depend on the workspace's earlier contents.
 *  - Every argument is validated on the host before anything is launched; a
 *    call that returns an error has enqueued nothing. Faults inside kernels
 *    surface asynchronously on the stream.
 *  - Supported in this version: block_size 128; head_dim 64 or 128; idx_dim
 *    32 or 64; num_kv_heads 1, 2, 4 or 8; G 1, 2, 4, 8 or 16; 1 <= topk <= 32;
 *    seqlen_kv <= 262144 (at most 2048 blocks). seqlen_kv need not be a
 *    multiple of 128 (the last block may be short). Other values return
 *    MSA_ERR_UNSUPPORTED. The device must be gfx950.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_NULL = 1,        /* a required pointer is NULL */
  MSA_ERR_SHAPE = 2,       /* inconsistent shape (e.g. Hq % Hkv != 0, q_start+seqlen_q > seqlen_kv) */
  MSA_ERR_UNSUPPORTED = 3, /* valid but not supported by the library (see list above) */
  MSA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than msa_workspace_size */
  MSA_ERR_DEVICE = 5,      /* HIP error at launch, or the current device is not gfx950 */
  MSA_ERR_SCRATCH = 6      /* msa_attn_fwd_noalloc: the call needs more than its fixed scratch */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

typedef struct {
  int32_t batch;        /* sequences; 0 is allowed (nothing to do) */
  int32_t seqlen_kv;    /* N: keys per sequence */
  int32_t seqlen_q;     /* query rows per sequence; 0 is allowed */
  int32_t q_start;      /* key position of query row 0 */
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv: GQA groups, index-query heads */
  int32_t head_dim;     /* d */
  int32_t idx_dim;      /* d_idx */
  int32_t block_size;   /* Bk, must be 128 */
  int32_t topk;         /* k: blocks per (query, group), counting the forced local block */
  int32_t dtype;        /* msa_dtype of every floating-point input and of `out` */
} msa_shape;

enum {
  MSA_OP_SELECT = 0, MSA_OP_ATTN = 1, MSA_OP_KL = 2, MSA_OP_ATTN_BWD = 3, MSA_OP_IDX_BWD = 4,
  MSA_OP_KL_DENSE_BWD = 5
};

/*
 * Bytes of workspace the call `op` (MSA_OP_*) needs for `shape`; 0 for an
 * invalid shape or op. For MSA_OP_SELECT it assumes block_scores == NULL
 * (with block_scores given, the call needs no workspace).
 */
size_t msa_workspace_size(const msa_shape* shape, int op);

/*
 * msa_select — index scoring, causal block max and block selection
 * (MSA vs DSA indexer note §2.1-§2.2; MSA blog, block selection and the
 * softmax-free Top-k of its kernel section; "4.1.1 · 监督与联合训练"
 * (selector supervision) §1.2 on a fixed secondary key for ties).
 *
 *  in   q_idx, k_idx        device, layouts above
 *  out  block_ids           device int32 [batch, seqlen_q, num_kv_heads, topk]:
 *                           the local block floor(i/128) plus the topk-1
 *                           earlier blocks of largest block score; equal scores
 *                           rank the lower block index first; ascending order;
 *                           -1 in unused slots when fewer than topk blocks are
 *                           visible (all visible blocks are then selected).
 *  out  block_scores (opt)  device fp32 [batch, seqlen_q, num_kv_heads, nb],
 *                           nb = ceil(seqlen_kv/128): M[i,b] for b <= i/128;
 *                           entries past the local block are not written.
 *                           When NULL, the scores live in the workspace.
 *  out  cutoff_margin (opt) device fp32 [batch, seqlen_q, num_kv_heads]:
 *                           score of the worst selected non-local block minus
 *                           the best unselected one ("4.1.1" eq. 9); +inf when
 *                           every visible block is selected.
 *  ws   workspace of msa_workspace_size(shape, MSA_OP_SELECT) bytes (may be
 *       NULL / 0 when block_scores is given).
 */
msa_status msa_select(const msa_shape* shape, const void* q_idx, const void* k_idx,
                      int32_t* block_ids, float* block_scores, float* cutoff_margin,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_index_block_lse — the index forward with per-block log-sum-exp (KL
 * alignment note §6: the index forward keeps one LSE per block, and the
 * student's LSE_idx is their log-sum-exp over the selected blocks).
 *
 *  in   q_idx, k_idx        device, layouts above
 *  out  block_scores        device fp32 [batch, seqlen_q, num_kv_heads, nb]:
 *                           M[i,b], the same values msa_select computes
 *  out  block_lse           device fp32, same layout: log sum over the keys j
 *                           of block b with j <= i of exp(S_idx[i,j]),
 *                           S_idx = q_idx.k_idx / sqrt(d_idx)
 *  Both outputs are -inf for blocks past the row's local block. The buffers
 *  belong to the caller; no workspace. Errors as msa_select.
 */
msa_status msa_index_block_lse(const msa_shape* shape, const void* q_idx, const void* k_idx,
                               float* block_scores, float* block_lse, hipStream_t stream);

/*
 * msa_attn_fwd — exact softmax attention over the selected blocks ("2.4"
 * eq. 2 restricted to the support; MSA vs DSA indexer note §2.3: the group's
 * heads share the block list and their KV head, each keeps its own query;
 * MSA blog kernel section: KV-outer execution that loads each selected block
 * once for every query that chose it).
 *
 *  in   q, k, v             device, layouts above
 *  in   block_ids           device int32 [batch, seqlen_q, num_kv_heads, topk]
 *                           as written by msa_select (ids >= 0 must be
 *                           distinct, <= i/128, and include i/128; -1 unused)
 *  out  out                 device [batch, seqlen_q, num_q_heads, head_dim], dtype
 *  out  lse                 device fp32 [batch, seqlen_q, num_q_heads]: natural
 *                           log-sum-exp of the scaled logits over the support
 *                           (LSE_main of the KL alignment note §6)
 *  ws   workspace of msa_workspace_size(shape, MSA_OP_ATTN) bytes
 */
msa_status msa_attn_fwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                        const int32_t* block_ids, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * msa_attn_fwd_noalloc — msa_attn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and kernels, with the workspace taken
 * from a fixed device array of MSA_NOALLOC_SCRATCH_BYTES (64 MiB) that the
 * library holds on every GPU it runs on until the process ends. The call
 * allocates and frees nothing.
 *
 *  in/out  as for msa_attn_fwd (the caller passes every input and output).
 *  Errors: as msa_attn_fwd; MSA_ERR_SCRATCH (nothing launched) when
 *  msa_workspace_size(shape, MSA_OP_ATTN) exceeds MSA_NOALLOC_SCRATCH_BYTES
 *  (e.g. a decode step of 64 sequences of 131072 tokens needs 20.3 MiB, a
 *  prefill of 8192 tokens about 2 GiB); MSA_ERR_DEVICE if the scratch address
 *  cannot be resolved on the current device.
 *  Sharing: every call on one GPU uses that GPU's single scratch array and
 *  leaves its contents behind (each call clears what it needs). Calls that
 *  overlap on one GPU (other threads, or other streams whose work has not
 *  finished) race on it: serialize them, e.g. on one stream.
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
msa_status msa_attn_fwd_noalloc(const msa_shape* shape, const void* q, const void* k,
                                const void* v, const int32_t* block_ids, void* out, float* lse,
                                hipStream_t stream);

/*
 * msa_kl_align — KL alignment of the index branch on the selected support
 * (KL alignment note §2.1 student, §2.2 teacher as the group mean of the
 * heads' probabilities, §3 loss 1/(N*Hkv) sum KL(stopgrad(P) || P_idx) and
 * gradient P_idx - P, §6 probabilities rebuilt from logits and LSEs).
 *
 *  in   q, k, q_idx, k_idx  device, layouts above
 *  in   block_ids           as for msa_attn_fwd
 *  in   lse_main            device fp32 [batch, seqlen_q, num_q_heads] from
 *                           msa_attn_fwd on the same ids
 *  out  kl_rows             device fp32 [batch, seqlen_q, num_kv_heads]:
 *                           KL(P || P_idx) of each (query, group)
 *  out  kl_mean             device fp32 [1]: mean of kl_rows over every row
 *  out  dlogits_idx (opt)   device fp32 [batch, seqlen_q, num_kv_heads, topk, 128]:
 *                           P_idx - P at (slot, offset in the slot's block); 0 at
 *                           positions j > i and in unused slots. Unscaled: the
 *                           caller applies lambda, 1/(N*Hkv) and the
 *                           1/sqrt(idx_dim) of the index logits when chaining.
 *  ws   workspace of msa_workspace_size(shape, MSA_OP_KL) bytes
 */
msa_status msa_kl_align(const msa_shape* shape, const void* q, const void* k, const void* q_idx,
                        const void* k_idx, const int32_t* block_ids, const float* lse_main,
                        float* kl_rows, float* kl_mean, float* dlogits_idx, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * msa_attn_bwd — gradients of msa_attn_fwd with the selection held fixed
 * ("2.4 · 训练原生稀疏" eq. (11): the logit gradient of a selected position is
 * alpha_s g.(v_s - o); eq. (12): the hard selection itself has no gradient;
 * the same page requires the backward to stay on the selected blocks). Through
 * z = q.k / sqrt(d): dq = sum_s dz_s k_s / sqrt(d), dk_s gets dz_s q / sqrt(d)
 * and dv_s gets alpha_s g, summed over every (query, head) of the group that
 * selected the key's block.
 *
 *  in   q, k, v, block_ids  as for msa_attn_fwd (the same ids)
 *  in   out, lse            device: the outputs of msa_attn_fwd for these inputs
 *  in   dout                device [batch, seqlen_q, num_q_heads, head_dim], dtype: dL/dout
 *  out  dq                  device [batch, seqlen_q, num_q_heads, head_dim], dtype
 *  out  dk, dv              device [batch, seqlen_kv, num_kv_heads, head_dim], dtype:
 *                           the contributions of this call's query rows; keys no
 *                           row selected get 0 (fully overwritten)
 *  ws   workspace of msa_workspace_size(shape, MSA_OP_ATTN_BWD) bytes
 * Accumulation is fp32 (dk, dv through fp32 atomics, so their last bits may
 * vary from run to run). fp32 inputs need head_dim 64 (MSA_ERR_UNSUPPORTED
 * otherwise).
 */
msa_status msa_attn_bwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                        const int32_t* block_ids, const void* out, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * msa_idx_bwd — the index-logit gradient chained into the index projections
 * (MSA vs DSA indexer note §2.1: S_idx = q_idx . k_idx / sqrt(d_idx) with one
 * k_idx head shared by every group; KL alignment note §3: the index branch
 * receives only the KL gradient P_idx - P, the selection held fixed).
 *   dq_idx[i, r] = coef / sqrt(d_idx) * sum_j dlogits[i, r, j] k_idx[j]
 *   dk_idx[j]    = coef / sqrt(d_idx) * sum over (i, r) that selected j of dlogits[i, r, j] q_idx[i, r]
 *
 *  in   q_idx, k_idx        device, layouts above
 *  in   block_ids           as for msa_kl_align (the same ids)
 *  in   dlogits_idx         device fp32 [batch, seqlen_q, num_kv_heads, topk, 128] as
 *                           msa_kl_align writes it (P_idx - P; 0 off the support),
 *                           16-byte aligned
 *  in   coef                loss coefficient (e.g. lambda / (N * Hkv) for the mean KL)
 *  out  dq_idx              device [batch, seqlen_q, num_kv_heads, idx_dim], dtype
 *  out  dk_idx              device [batch, seqlen_kv, idx_dim], dtype: the
 *                           contributions of this call's query rows; keys no row
 *                           selected get 0 (fully overwritten)
 *  ws   workspace of msa_workspace_size(shape, MSA_OP_IDX_BWD) bytes
 * Accumulation is fp32 (dk_idx through fp32 atomics).
 */
msa_status msa_idx_bwd(const msa_shape* shape, const void* q_idx, const void* k_idx,
                       const int32_t* block_ids, const float* dlogits_idx, float coef,
                       void* dq_idx, void* dk_idx, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * msa_dense_lse — log-sum-exp of the main branch over the full causal context
 * (KL alignment note §5: in the warm-up stage the main branch attends to every
 * earlier token; §6: the KL needs only each branch's LSE). It stands in for the
 * LSE that a dense causal attention forward reports.
 *   lse_main[b, t, h] = log sum over j <= q_start + t of
 *                       exp(q[b, t, h] . k[b, j, floor(h / G)] / sqrt(head_dim))
 *
 *  in   q, k                device, layouts above (v is not read)
 *  out  lse_main            device fp32 [batch, seqlen_q, num_q_heads]
 * topk is not used. fp32 inputs need head_dim 64 (MSA_ERR_UNSUPPORTED
 * otherwise). No workspace. Cost is O(seqlen_q * seqlen_kv) per head.
 */
msa_status msa_dense_lse(const msa_shape* shape, const void* q, const void* k, float* lse_main,
                         hipStream_t stream);

/*
 * msa_kl_dense — KL alignment on the full causal context, the warm-up stage
 * (KL alignment note §5: support J = every j <= i; §2 student and teacher;
 * §3 KL(P || P_idx)), and the teacher's attention mass per 128-token block.
 *   P_j       = (1/G) sum over the group's heads h of exp(S_h,j - lse_main_h)
 *   P_idx_j   = exp(z_j - lse_idx), z_j = q_idx . k_idx_j / sqrt(idx_dim)
 *   kl_rows[b, t, r]       = sum over j <= i of P_j log(P_j / P_idx_j)
 *   block_mass[b, t, r, c] = sum over j in block c, j <= i, of P_j
 *
 *  in   q, k, q_idx, k_idx  device, layouts above
 *  in   lse_main            device fp32 [batch, seqlen_q, num_q_heads] over the
 *                           full causal context (msa_dense_lse)
 *  out  lse_idx             device fp32 [batch, seqlen_q, num_kv_heads]: LSE of
 *                           the index logits over j <= i
 *  out  kl_rows             device fp32 [batch, seqlen_q, num_kv_heads]
 *  out  kl_mean             device fp32 [1]: mean of kl_rows over every row
 *  out  block_mass (opt)    device fp32 [batch, seqlen_q, num_kv_heads,
 *                           ceil(seqlen_kv / 128)]; 0 for blocks after the
 *                           query's own (fully overwritten)
 * topk is not used. fp32 inputs need head_dim 64. No workspace.
 */
msa_status msa_kl_dense(const msa_shape* shape, const void* q, const void* k, const void* q_idx,
                        const void* k_idx, const float* lse_main, float* lse_idx, float* kl_rows,
                        float* kl_mean, float* block_mass, hipStream_t stream);

/*
 * msa_kl_dense_bwd — msa_kl_dense together with its gradient into the index
 * projections (KL alignment note §3: the index logits receive P_idx - P; §6:
 * the gradient is formed from the logits and the two LSEs, with no separate
 * KL forward; MSA vs DSA indexer note §2.1: one k_idx head shared by every
 * group). With dS = P_idx - P on every j <= i:
 *   dq_idx[i, r] = coef / sqrt(idx_dim) * sum_j dS[i, r, j] k_idx[j]
 *   dk_idx[j]    = coef / sqrt(idx_dim) * sum over (i, r), i >= j, of dS[i, r, j] q_idx[i, r]
 *
 *  in   q, k, q_idx, k_idx, lse_main  as for msa_kl_dense
 *  in   coef                loss coefficient (e.g. lambda / (B * N * Hkv) for the mean KL)
 *  out  lse_idx             device fp32 [batch, seqlen_q, num_kv_heads]
 *  out  kl_rows, kl_mean, block_mass (opt)  as for msa_kl_dense
 *  out  dq_idx              device [batch, seqlen_q, num_kv_heads, idx_dim], dtype
 *  out  dk_idx              device [batch, seqlen_kv, idx_dim], dtype: the
 *                           contributions of this call's query rows (overwritten)
 *  ws   workspace of msa_workspace_size(shape, MSA_OP_KL_DENSE_BWD) bytes: dS of
 *       a chunk of query rows in bf16 (at most ~2 GiB; the call loops over
 *       chunks) and an fp32 dk_idx accumulator
 * dS is rounded to bf16 and the two products run on bf16 matrix cores with
 * fp32 accumulation (fp32 inputs are rounded to bf16 for them). fp32 inputs
 * need head_dim 64.
 */
msa_status msa_kl_dense_bwd(const msa_shape* shape, const void* q, const void* k,
                            const void* q_idx, const void* k_idx, const float* lse_main,
                            float coef, float* lse_idx, float* kl_rows, float* kl_mean,
                            float* block_mass, void* dq_idx, void* dk_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * msa_block_recall — block recall and score recall of a selection against the
 * full-history teacher (KL alignment note §8; selector supervision page
 * "4.1.1 · 监督与联合训练", eq. 2 set recall and eq. 3 coverage).
 *   T = the min(topk, L + 1) blocks of largest block_mass among 0..L,
 *       L = floor(i / 128), the lower index first on equal mass
 *   block_recall[b, t, r] = |S ∩ T| / |T|, S = the row's block_ids
 *   score_recall[b, t, r] = sum of block_mass over S
 * Ids -1 (and ids outside 0..L) count as no block.
 *
 *  in   block_mass          device fp32, as msa_kl_dense writes it
 *  in   block_ids           device int32 [batch, seqlen_q, num_kv_heads, topk]
 *  out  block_recall, score_recall
 *                           device fp32 [batch, seqlen_q, num_kv_heads]
 *  out  means (opt)         device fp32 [2]: the means of the two over every row
 * No workspace.
 */
msa_status msa_block_recall(const msa_shape* shape, const float* block_mass,
                            const int32_t* block_ids, float* block_recall, float* score_recall,
                            float* means, hipStream_t stream);

/*
 * msa_index_quantize_fp8 — FP8 inputs of the index branch (MSA vs DSA indexer
 * note §3.1: the indexer's scores may run in FP8). Format OCP E4M3 (bias 7, max
 * 448, no infinities), round to nearest with ties to the even code. Scales are
 * powers of two: one per Q_idx row (b, t, r) and one per 128-token K_idx block
 * (b, c); e = the smallest integer with amax <= 448 * 2^e (0 for an all-zero
 * row or block), and the stored byte encodes x * 2^-e.
 *
 *  in   q_idx, k_idx        device, layouts above (fp32 or bf16 by dtype)
 *  out  q8 (opt)            device uint8 [batch, seqlen_q, num_kv_heads, idx_dim]
 *  out  q_exp               device int32 [batch, seqlen_q, num_kv_heads] (with q8)
 *  out  k8 (opt)            device uint8 [batch, seqlen_kv, idx_dim]
 *  out  k_exp               device int32 [batch, ceil(seqlen_kv / 128)] (with k8)
 * At least one of q8, k8. q8 and k8 must be 16-byte aligned. K_idx can be
 * quantized once (e.g. when a cache is written) and reused by later calls.
 * No workspace.
 */
msa_status msa_index_quantize_fp8(const msa_shape* shape, const void* q_idx, const void* k_idx,
                                  uint8_t* q8, int32_t* q_exp, uint8_t* k8, int32_t* k_exp,
                                  hipStream_t stream);

/*
 * msa_select_fp8 — msa_select on the FP8 index inputs: the index logits are
 * (q8 . k8 on the FP8 matrix cores) * 2^(q_exp + k_exp of the key's block) /
 * sqrt(idx_dim), then the same causal block max and the same selection rule
 * (selector supervision page, after eq. 9: a small cutoff margin is where
 * FP8 quantization flips candidates; cutoff_margin reports it per row).
 *
 *  in   q8, q_exp, k8, k_exp  as msa_index_quantize_fp8 writes them
 *  out  block_ids, block_scores (opt), cutoff_margin (opt)  as for msa_select
 *  ws   workspace of msa_workspace_size(shape, MSA_OP_SELECT) bytes (may be
 *       NULL when block_scores is given)
 * dtype is not used (the inputs are FP8).
 */
msa_status msa_select_fp8(const msa_shape* shape, const uint8_t* q8, const int32_t* q_exp,
                          const uint8_t* k8, const int32_t* k_exp, int32_t* block_ids,
                          float* block_scores, float* cutoff_margin, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* msa_status_string(msa_status status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
