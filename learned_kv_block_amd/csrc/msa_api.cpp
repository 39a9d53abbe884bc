// msa_api.cpp — the C ABI of include/msa.h: host-side validation, workspace
// layout and the launch sequence of each call. Every check runs before the
// first launch, so an error return leaves the stream untouched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "msa_dense.hpp"
#include "msa_internal.hpp"

using namespace msa;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Work items hold up to qt query rows; items_max bounds sum over buckets of
// ceil(count / qt) <= entries / qt + (non-empty buckets).
void set_item_size(Dims* d, int qt) {
  d->qt = qt;
  const int64_t per_item =
      d->entries_max / qt + (d->buckets < d->entries_max ? d->buckets : d->entries_max);
  d->items_max = per_item < d->entries_max ? per_item : d->entries_max;
}

// The bf16 attention kernel and the bf16 KL passes with G >= 8 run 256
// (query, head) rows per work item; the fp32 kernels and other KL shapes run 128.
#ifndef MSA_BWD_R16
#define MSA_BWD_R16 64
#endif

Dims for_op(Dims d, int op) {
  // bf16 attention: 256 (query, head) rows per item; 32 when no bucket can
  // hold more (Nq * G <= 32, decode), for the one-wave attention workgroups
  if (op == MSA_OP_ATTN && d.dtype == MSA_BF16) set_item_size(&d, (d.Nq * d.G <= 32 ? 32 : 256) / d.G);
  if (op == MSA_OP_KL && d.dtype == MSA_BF16 && d.G >= 8) set_item_size(&d, 256 / d.G);
  // attention backward: 64 (query, head) rows per item for bf16, 32 for fp32
  if (op == MSA_OP_ATTN_BWD) set_item_size(&d, (d.dtype == MSA_BF16 ? MSA_BWD_R16 : 32) / d.G);
  // index chain: 32 queries (of one group) per item
  if (op == MSA_OP_IDX_BWD) set_item_size(&d, 32);
  return d;
}

// Shape validation shared by all calls. Fills d on success.
msa_status make_dims(const msa_shape* s, Dims* d) {
  if (!s) return MSA_ERR_NULL;
  if (s->batch < 0 || s->seqlen_kv < 0 || s->seqlen_q < 0 || s->q_start < 0) return MSA_ERR_SHAPE;
  if (s->num_q_heads < 1 || s->num_kv_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return MSA_ERR_SHAPE;
  if (s->head_dim < 1 || s->idx_dim < 1 || s->block_size < 1 || s->topk < 1) return MSA_ERR_SHAPE;
  if ((int64_t)s->q_start + s->seqlen_q > s->seqlen_kv) return MSA_ERR_SHAPE;
  if (s->dtype != MSA_F32 && s->dtype != MSA_BF16) return MSA_ERR_SHAPE;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (s->block_size != 128) return MSA_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return MSA_ERR_UNSUPPORTED;
  if (s->idx_dim != 32 && s->idx_dim != 64) return MSA_ERR_UNSUPPORTED;
  if (s->num_kv_heads != 1 && s->num_kv_heads != 2 && s->num_kv_heads != 4 && s->num_kv_heads != 8)
    return MSA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return MSA_ERR_UNSUPPORTED;
  if (s->topk > 32) return MSA_ERR_UNSUPPORTED;
  const int nb = (s->seqlen_kv + 127) / 128;
  if (nb > 2048) return MSA_ERR_UNSUPPORTED;
  d->B = s->batch;
  d->N = s->seqlen_kv;
  d->Nq = s->seqlen_q;
  d->q_start = s->q_start;
  d->Hq = s->num_q_heads;
  d->Hkv = s->num_kv_heads;
  d->G = G;
  d->D = s->head_dim;
  d->DI = s->idx_dim;
  d->Bk = s->block_size;
  d->K = s->topk;
  d->nb = nb;
  d->dtype = s->dtype;
  d->rows = (int64_t)s->batch * s->seqlen_q;
  d->slots = d->rows * d->Hkv * d->K;
  d->nwin = (s->seqlen_q + kQueryWindow - 1) / kQueryWindow;
  d->buckets = (int64_t)s->batch * d->Hkv * d->nwin * nb;
  d->entries_max = d->rows * d->Hkv * (int64_t)(d->K < nb ? d->K : nb);
  d->num_cus = 0;
  set_item_size(d, 128 / G);
  // index ranges the kernels keep in 32-bit integers
  if (d->entries_max >= (int64_t)1 << 31 || d->buckets >= (int64_t)1 << 30 ||
      d->items_max >= (int64_t)1 << 30 || s->seqlen_q >= (1 << 25) ||
      (int64_t)s->batch * s->seqlen_q >= (int64_t)1 << 31 || d->slots + 1 >= (int64_t)1 << 31 ||
      d->rows * s->num_q_heads >= (int64_t)1 << 31)
    return MSA_ERR_UNSUPPORTED;
  if (((d->Nq + 127) / 128 > 65535) || s->batch > 65535) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

size_t elem_size(const Dims& d) { return d.dtype == MSA_BF16 ? 2 : 4; }

struct Layout {
  size_t counts, offsets, cursor, item_off, totals, items, entries, chunks;  // bucketing
  size_t cost_off, wg_start;                                            // balanced split
  size_t nchunks;  // scan chunks of 4096 buckets (+1)
  size_t opart, lpart;                                               // attention
  size_t sorted;                                                     // backward: canonical entries
  size_t drow, dqpart, slabs;                                        // attention backward
  size_t dqi_part, dki_acc;                                          // index chain
  size_t slot_lse, lse_idx, kl_part, block_sums;                     // KL
  size_t dense_ds;                                                   // full-context KL gradient
  size_t total;
};

Layout layout(const Dims& d, int op) {
  Layout L;
  std::memset(&L, 0, sizeof(L));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  if (op == MSA_OP_SELECT) {
    L.total = (size_t)d.rows * d.Hkv * d.nb * sizeof(float);
    return L;
  }
  if (op == MSA_OP_KL_DENSE_BWD) {
    L.dense_ds = take((size_t)dense_grad_ds_elems(d) * 2);
    L.dki_acc = take((size_t)d.B * d.N * d.DI * 4);
    L.total = o;
    return L;
  }
  L.counts = take(d.buckets * 4);
  L.offsets = take((d.buckets + 1) * 4);
  L.cursor = take(d.buckets * 4);
  L.item_off = take((d.buckets + 1) * 4);
  L.totals = take(16);
  L.items = take(d.items_max * 16);
  L.entries = take(d.entries_max * 4);
  L.nchunks = (size_t)(d.buckets / 4096 + 1);
  L.chunks = take(L.nchunks * 3 * 4);  // per-chunk scan sums (entries, items, cost)
  L.cost_off = take((d.buckets + 1) * 4);
  L.wg_start = take((kMaxSplit + 1) * 4);
  if (op == MSA_OP_ATTN) {
    // one extra slot: scratch target of the attention kernel's unused rows
    L.opart = take((size_t)(d.slots + 1) * d.G * d.D * elem_size(d));
    L.lpart = take((size_t)(d.slots + 1) * d.G * 4);
  } else if (op == MSA_OP_ATTN_BWD) {
    L.sorted = take(d.entries_max * 4);
    L.drow = take((size_t)d.rows * d.Hq * 4);
    // one extra slot: target of the backward kernel's unused rows
    L.dqpart = take((size_t)(d.slots + 1) * d.G * d.D * elem_size(d));
    // [bucket or workgroup run][32-row tile][dK, dV][128 keys][D] fp32
    const size_t row_tiles = (d.dtype == MSA_BF16 ? MSA_BWD_R16 : 32) / 32;
    L.slabs = take(((size_t)d.buckets + 2 * kBwdMaxGrid) * row_tiles * 2 * 128 * d.D * 4);
  } else if (op == MSA_OP_IDX_BWD) {
    L.sorted = take(d.entries_max * 4);
    // one extra slot: target of the index backward kernel's unused queries
    L.dqi_part = take((size_t)(d.slots + 1) * d.DI * 4);
    // [bucket or workgroup run][128 keys][d_idx] fp32
    L.slabs = take(((size_t)d.buckets + 2 * kBwdMaxGrid) * 128 * d.DI * 4);
  } else {
    L.slot_lse = take((size_t)d.slots * 4);
    L.lse_idx = take((size_t)d.rows * d.Hkv * 4);
    // + one spare slot and one spare 128-float row: targets of the KL kernel's
    // stores for queries past an item's count
    L.kl_part = take((size_t)(d.slots + 1 + 128) * 4);
    L.block_sums = take((size_t)((d.rows * d.Hkv + 255) / 256 + 1) * 4);
  }
  L.total = o;
  return L;
}

AttnWs carve(const Layout& L, void* ws) {
  char* p = static_cast<char*>(ws);
  AttnWs w;
  w.counts = reinterpret_cast<int32_t*>(p + L.counts);
  w.offsets = reinterpret_cast<int32_t*>(p + L.offsets);
  w.cursor = reinterpret_cast<int32_t*>(p + L.cursor);
  w.item_off = reinterpret_cast<int32_t*>(p + L.item_off);
  w.totals = reinterpret_cast<int32_t*>(p + L.totals);
  w.items = reinterpret_cast<int4*>(p + L.items);
  w.entries = reinterpret_cast<int32_t*>(p + L.entries);
  w.chunk_e = reinterpret_cast<int32_t*>(p + L.chunks);
  w.chunk_i = w.chunk_e + L.nchunks;
  w.chunk_c = w.chunk_i + L.nchunks;
  w.cost_off = reinterpret_cast<int32_t*>(p + L.cost_off);
  w.wg_start = reinterpret_cast<int32_t*>(p + L.wg_start);
  w.sorted = L.sorted ? reinterpret_cast<int32_t*>(p + L.sorted) : nullptr;
  return w;
}

msa_status check_ws(const Layout& L, void* ws, size_t bytes) {
  if (L.total == 0) return MSA_OK;
  if (!ws || bytes < L.total) return MSA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return MSA_ERR_WORKSPACE;
  return MSA_OK;
}

// The current device must be gfx950 (checked once per device); also reports
// its compute-unit count.
msa_status check_device(int* num_cus) {
  static std::atomic<int> cache[64];  // 0 unknown, -1 not gfx950, else the CU count
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return MSA_ERR_DEVICE;
  int c = cache[dev].load();
  if (c == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MSA_ERR_DEVICE;
    c = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? (prop.multiProcessorCount > 0
                                                                ? prop.multiProcessorCount
                                                                : 1)
                                                          : -1;
    cache[dev].store(c);
  }
  if (c < 0) return MSA_ERR_DEVICE;
  if (num_cus) *num_cus = c;
  return MSA_OK;
}

inline bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

msa_status attn_fwd_launch(const Dims& d, const Layout& L, const void* q, const void* k,
                           const void* v, const int32_t* block_ids, void* out, float* lse,
                           void* workspace, hipStream_t stream);

// A prefill of more than kAttnWindow queries per sequence, or of several
// sequences of at least kAttnWindowMin queries, runs the attention in windows of
// at most kAttnWindow consecutive queries of one sequence: bucketing, KV-outer
// attention and combine per window, in one window-sized workspace. The attention
// kernel's scattered partial stores and gathered Q rows then stay inside one
// window's address range (the attention kernel: 13.2 ms in one pass against
// 11.5 ms in four windows at one 131072-token sequence, 6.5 against 5.8 ms at
// 2 x 32768), and the workspace shrinks by the window count. A window is the same
// computation as a caller's chunked-prefill call (q_start shifted, batch 1); rows
// are independent.
#ifndef MSA_ATTN_WINDOW
#define MSA_ATTN_WINDOW 32768
#endif
constexpr int64_t kAttnWindow = MSA_ATTN_WINDOW;
constexpr int64_t kAttnWindowMin = 4096;

bool attn_windowed(const Dims& d) {
  return d.Nq > kAttnWindow || (d.B > 1 && d.Nq >= kAttnWindowMin);
}

// dims of the window of `len` queries starting at query `a` of one sequence
msa_status window_dims(const msa_shape* s, int64_t a, int64_t len, Dims* dw) {
  msa_shape w = *s;
  w.batch = 1;
  w.q_start = s->q_start + (int32_t)a;
  w.seqlen_q = (int32_t)len;
  const msa_status st = make_dims(&w, dw);
  if (st == MSA_OK) *dw = for_op(*dw, MSA_OP_ATTN);
  return st;
}

// the workspace layout of msa_attn_fwd: one window's when windowed
msa_status attn_layout(const msa_shape* s, const Dims& d, Layout* L) {
  if (!attn_windowed(d)) {
    *L = layout(d, MSA_OP_ATTN);
    return MSA_OK;
  }
  Dims dw;
  const msa_status st = window_dims(s, 0, d.Nq < kAttnWindow ? d.Nq : kAttnWindow, &dw);
  if (st == MSA_OK) *L = layout(dw, MSA_OP_ATTN);
  return st;
}

// msa_attn_fwd on a validated shape: one launch sequence, or one per window
msa_status attn_fwd_run(const msa_shape* s, const Dims& d, const Layout& L, const void* q,
                        const void* k, const void* v, const int32_t* block_ids, void* out,
                        float* lse, void* workspace, hipStream_t stream) {
  if (!attn_windowed(d)) return attn_fwd_launch(d, L, q, k, v, block_ids, out, lse, workspace, stream);
  const size_t es = d.dtype == MSA_BF16 ? 2 : 4;
  for (int64_t b = 0; b < d.B; ++b) {
    for (int64_t a = 0; a < d.Nq; a += kAttnWindow) {
      const int64_t len = d.Nq - a < kAttnWindow ? d.Nq - a : kAttnWindow;
      Dims dw;
      msa_status st = window_dims(s, a, len, &dw);
      if (st != MSA_OK) return st;
      dw.num_cus = d.num_cus;
      const int64_t row0 = b * d.Nq + a;  // first (batch, query) row of the window
      const size_t kvoff = (size_t)b * d.N * d.Hkv * d.D * es;
      st = attn_fwd_launch(dw, L, static_cast<const char*>(q) + (size_t)row0 * d.Hq * d.D * es,
                           static_cast<const char*>(k) + kvoff,
                           static_cast<const char*>(v) + kvoff,
                           block_ids + (size_t)row0 * d.Hkv * d.K,
                           static_cast<char*>(out) + (size_t)row0 * d.Hq * d.D * es,
                           lse + (size_t)row0 * d.Hq, workspace, stream);
      if (st != MSA_OK) return st;
    }
  }
  return MSA_OK;
}

}  // namespace

// ------------------------------------------------- fixed scratch of msa_attn_fwd_noalloc
// A device array of MSA_NOALLOC_SCRATCH_BYTES, one copy per GPU. In host code its
// name is only a stand-in: the device address is resolved once per device with
// hipGetSymbolAddress (with that device current) and only that address is used.
__device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch_addr[64];  // device address of `scratch` per device (0: unresolved)

msa_status scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MSA_ERR_DEVICE;
  void* p = g_scratch_addr[dev].load();
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_DEVICE;
    g_scratch_addr[dev].store(p);  // concurrent first calls store the same address
  }
  *ptr = p;
  return MSA_OK;
}
}  // namespace

extern "C" {

const char* msa_status_string(msa_status st) {
  switch (st) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "a required pointer is NULL";
    case MSA_ERR_SHAPE: return "inconsistent shape";
    case MSA_ERR_UNSUPPORTED: return "shape or type not supported by the library";
    case MSA_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case MSA_ERR_DEVICE: return "HIP launch error or device is not gfx950";
    case MSA_ERR_SCRATCH:
      return "workload needs more than the fixed scratch of msa_attn_fwd_noalloc (64 MiB)";
  }
  return "unknown status";
}

size_t msa_workspace_size(const msa_shape* shape, int op) {
  Dims d;
  if (make_dims(shape, &d) != MSA_OK) return 0;
  if (op != MSA_OP_SELECT && op != MSA_OP_ATTN && op != MSA_OP_KL && op != MSA_OP_ATTN_BWD &&
      op != MSA_OP_IDX_BWD && op != MSA_OP_KL_DENSE_BWD)
    return 0;
  if (op == MSA_OP_ATTN) {
    Layout L;
    return attn_layout(shape, for_op(d, op), &L) == MSA_OK ? L.total : 0;
  }
  return layout(for_op(d, op), op).total;
}

msa_status msa_select(const msa_shape* shape, const void* q_idx, const void* k_idx,
                      int32_t* block_ids, float* block_scores, float* cutoff_margin,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.rows == 0) return MSA_OK;
  if (!q_idx || !k_idx || !block_ids) return MSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(k_idx)) return MSA_ERR_SHAPE;
  float* M = block_scores;
  if (!M) {
    const Layout L = layout(d, MSA_OP_SELECT);
    if ((st = check_ws(L, workspace, workspace_bytes)) != MSA_OK) return st;
    M = static_cast<float*>(workspace);
  }
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  prof_before(MSA_K_INDEX_BLOCKMAX, stream);
  hipError_t e = launch_index_blockmax(d, q_idx, k_idx, M, stream);
  prof_after(MSA_K_INDEX_BLOCKMAX, stream);
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  prof_before(MSA_K_TOPK, stream);
  e = launch_topk(d, M, block_ids, cutoff_margin, stream);
  prof_after(MSA_K_TOPK, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_index_block_lse(const msa_shape* shape, const void* q_idx, const void* k_idx,
                               float* block_scores, float* block_lse, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.rows == 0) return MSA_OK;
  if (!q_idx || !k_idx || !block_scores || !block_lse) return MSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(k_idx)) return MSA_ERR_SHAPE;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  const int64_t n = d.rows * d.Hkv * d.nb;
  if (launch_fill_f32(block_scores, n, -INFINITY, stream) != hipSuccess ||
      launch_fill_f32(block_lse, n, -INFINITY, stream) != hipSuccess)
    return MSA_ERR_DEVICE;
  prof_before(MSA_K_INDEX_BLOCKMAX, stream);
  const hipError_t e = launch_index_block_lse(d, q_idx, k_idx, block_scores, block_lse, stream);
  prof_after(MSA_K_INDEX_BLOCKMAX, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_attn_fwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                        const int32_t* block_ids, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  d = for_op(d, MSA_OP_ATTN);
  if (d.rows == 0) return MSA_OK;
  if (!q || !k || !v || !block_ids || !out || !lse) return MSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MSA_ERR_SHAPE;
  Layout L;
  if ((st = attn_layout(shape, d, &L)) != MSA_OK) return st;
  if ((st = check_ws(L, workspace, workspace_bytes)) != MSA_OK) return st;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  return attn_fwd_run(shape, d, L, q, k, v, block_ids, out, lse, workspace, stream);
}

msa_status msa_attn_fwd_noalloc(const msa_shape* shape, const void* q, const void* k,
                                const void* v, const int32_t* block_ids, void* out, float* lse,
                                hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  d = for_op(d, MSA_OP_ATTN);
  if (d.rows == 0) return MSA_OK;
  if (!q || !k || !v || !block_ids || !out || !lse) return MSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MSA_ERR_SHAPE;
  Layout L;
  if ((st = attn_layout(shape, d, &L)) != MSA_OK) return st;
  if (L.total > MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_SCRATCH;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MSA_OK) return st;
  return attn_fwd_run(shape, d, L, q, k, v, block_ids, out, lse, ws, stream);
}

}  // extern "C"

namespace {
// the launch sequence of msa_attn_fwd on a validated shape and a workspace of L.total bytes
msa_status attn_fwd_launch(const Dims& d, const Layout& L, const void* q, const void* k,
                           const void* v, const int32_t* block_ids, void* out, float* lse,
                           void* workspace, hipStream_t stream) {
  if (decode_attn_supported(d)) {
    // one query per sequence: query-outer over the selected blocks, no workspace used
    prof_before(MSA_K_SPARSE_ATTN, stream);
    const hipError_t e = launch_decode_attn(d, q, k, v, block_ids, out, lse, stream);
    prof_after(MSA_K_SPARSE_ATTN, stream);
    return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
  }
  char* ws = static_cast<char*>(workspace);
  const AttnWs w = carve(L, workspace);
  // bf16: each row's local block is attended query-outer inside the combine,
  // so the KV-outer work lists leave it out
  const bool local_in_combine = d.dtype == MSA_BF16;
  // the persistent bf16 kernel takes cost-balanced item ranges
  const int split = d.dtype == MSA_BF16 ? (int)attn_pipe_grid(d) : 0;
  if (launch_bucketing(d, block_ids, w, local_in_combine, stream, split) != hipSuccess)
    return MSA_ERR_DEVICE;
  prof_before(MSA_K_SPARSE_ATTN, stream);
  hipError_t e = launch_sparse_attn(d, q, k, v, w, ws + L.opart,
                                    reinterpret_cast<float*>(ws + L.lpart), stream);
  prof_after(MSA_K_SPARSE_ATTN, stream);
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  prof_before(MSA_K_COMBINE, stream);
  const float* lpart = reinterpret_cast<const float*>(ws + L.lpart);
  e = local_in_combine
          ? launch_combine_local(d, q, k, v, ws + L.opart, lpart, block_ids, out, lse, stream)
          : launch_combine(d, ws + L.opart, lpart, block_ids, out, lse, stream);
  prof_after(MSA_K_COMBINE, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}
}  // namespace

extern "C" {

msa_status msa_attn_bwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                        const int32_t* block_ids, const void* out, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.dtype == MSA_F32 && d.D != 64) return MSA_ERR_UNSUPPORTED;  // LDS tiles of the fp32 kernel
  d = for_op(d, MSA_OP_ATTN_BWD);
  const int64_t nkv = (int64_t)d.B * d.N * d.Hkv * d.D;
  if (nkv > 0) {
    if (!dk || !dv) return MSA_ERR_NULL;
    if (!aligned16(dk) || !aligned16(dv)) return MSA_ERR_SHAPE;
  }
  if (d.rows > 0) {
    if (!q || !k || !v || !block_ids || !out || !lse || !dout || !dq) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
        !aligned16(dq))
      return MSA_ERR_SHAPE;
  }
  const Layout L = layout(d, MSA_OP_ATTN_BWD);
  if (d.rows > 0 && (st = check_ws(L, workspace, workspace_bytes)) != MSA_OK) return st;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  if (d.rows == 0) {  // no query row: dk = dv = 0 (the zero bit pattern of fp32 and bf16)
    const int64_t words = nkv * (int64_t)elem_size(d) / 4;
    if (launch_fill_i32(static_cast<int32_t*>(dk), words, 0, stream) != hipSuccess ||
        launch_fill_i32(static_cast<int32_t*>(dv), words, 0, stream) != hipSuccess)
      return MSA_ERR_DEVICE;
    return MSA_OK;
  }
  char* ws = static_cast<char*>(workspace);
  const AttnWs w = carve(L, workspace);
  if (launch_bucketing(d, block_ids, w, false, stream) != hipSuccess) return MSA_ERR_DEVICE;
  const hipError_t e = launch_attn_bwd(
      d, q, k, v, block_ids, out, lse, dout, w, reinterpret_cast<float*>(ws + L.drow),
      ws + L.dqpart, reinterpret_cast<float*>(ws + L.slabs), dq, dk, dv, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_idx_bwd(const msa_shape* shape, const void* q_idx, const void* k_idx,
                       const int32_t* block_ids, const float* dlogits_idx, float coef,
                       void* dq_idx, void* dk_idx, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  d = for_op(d, MSA_OP_IDX_BWD);
  const int64_t nk = (int64_t)d.B * d.N * d.DI;
  if (nk > 0) {
    if (!dk_idx) return MSA_ERR_NULL;
    if (!aligned16(dk_idx)) return MSA_ERR_SHAPE;
  }
  if (d.rows > 0) {
    if (!q_idx || !k_idx || !block_ids || !dlogits_idx || !dq_idx) return MSA_ERR_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(dq_idx) || !aligned16(dlogits_idx))
      return MSA_ERR_SHAPE;
  }
  if (!std::isfinite(coef)) return MSA_ERR_SHAPE;
  const Layout L = layout(d, MSA_OP_IDX_BWD);
  if (d.rows > 0 && (st = check_ws(L, workspace, workspace_bytes)) != MSA_OK) return st;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  if (d.rows == 0) {  // no query row: dk_idx = 0
    const int64_t words = nk * (int64_t)elem_size(d) / 4;
    return launch_fill_i32(static_cast<int32_t*>(dk_idx), words, 0, stream) == hipSuccess
               ? MSA_OK
               : MSA_ERR_DEVICE;
  }
  char* ws = static_cast<char*>(workspace);
  const AttnWs w = carve(L, workspace);
  if (launch_bucketing(d, block_ids, w, false, stream) != hipSuccess) return MSA_ERR_DEVICE;
  const hipError_t e = launch_idx_bwd(d, q_idx, k_idx, block_ids, dlogits_idx, coef, w,
                                      reinterpret_cast<float*>(ws + L.dqi_part),
                                      reinterpret_cast<float*>(ws + L.slabs), dq_idx, dk_idx,
                                      stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_kl_align(const msa_shape* shape, const void* q, const void* k, const void* q_idx,
                        const void* k_idx, const int32_t* block_ids, const float* lse_main,
                        float* kl_rows, float* kl_mean, float* dlogits_idx, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  d = for_op(d, MSA_OP_KL);
  if (!kl_mean) return MSA_ERR_NULL;
  if (d.rows > 0) {
    if (!q || !k || !q_idx || !k_idx || !block_ids || !lse_main || !kl_rows) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx) ||
        (dlogits_idx && !aligned16(dlogits_idx)))
      return MSA_ERR_SHAPE;
  }
  const Layout L = layout(d, MSA_OP_KL);
  if (d.rows > 0 && (st = check_ws(L, workspace, workspace_bytes)) != MSA_OK) return st;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  if (d.rows == 0)
    return launch_fill_f32(kl_mean, 1, 0.0f, stream) == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
  char* ws = static_cast<char*>(workspace);
  const AttnWs w = carve(L, workspace);
  if (launch_bucketing(d, block_ids, w, false, stream) != hipSuccess) return MSA_ERR_DEVICE;
  hipError_t e = launch_kl(d, q, k, q_idx, k_idx, block_ids, lse_main, w,
                           reinterpret_cast<float*>(ws + L.slot_lse),
                           reinterpret_cast<float*>(ws + L.lse_idx),
                           reinterpret_cast<float*>(ws + L.kl_part), kl_rows,
                           reinterpret_cast<float*>(ws + L.block_sums), kl_mean, dlogits_idx,
                           stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_dense_lse(const msa_shape* shape, const void* q, const void* k, float* lse_main,
                         hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.dtype == MSA_F32 && d.D != 64) return MSA_ERR_UNSUPPORTED;
  if (d.rows == 0) return MSA_OK;
  if (!q || !k || !lse_main) return MSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k)) return MSA_ERR_SHAPE;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  prof_before(MSA_K_DENSE_LSE, stream);
  const hipError_t e = launch_dense_lse(d, false, q, k, lse_main, stream);
  prof_after(MSA_K_DENSE_LSE, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_kl_dense(const msa_shape* shape, const void* q, const void* k, const void* q_idx,
                        const void* k_idx, const float* lse_main, float* lse_idx, float* kl_rows,
                        float* kl_mean, float* block_mass, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.dtype == MSA_F32 && d.D != 64) return MSA_ERR_UNSUPPORTED;
  if (!kl_mean) return MSA_ERR_NULL;
  if (d.rows > 0) {
    if (!q || !k || !q_idx || !k_idx || !lse_main || !lse_idx || !kl_rows) return MSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx))
      return MSA_ERR_SHAPE;
  }
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  if (d.rows == 0)
    return launch_fill_f32(kl_mean, 1, 0.0f, stream) == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
  if (block_mass &&
      launch_fill_f32(block_mass, d.rows * d.Hkv * d.nb, 0.0f, stream) != hipSuccess)
    return MSA_ERR_DEVICE;
  prof_before(MSA_K_DENSE_LSE_IDX, stream);
  hipError_t e = launch_dense_lse(d, true, q_idx, k_idx, lse_idx, stream);
  prof_after(MSA_K_DENSE_LSE_IDX, stream);
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  prof_before(MSA_K_KL_DENSE, stream);
  e = launch_kl_dense(d, q, k, q_idx, k_idx, lse_main, lse_idx, kl_rows, block_mass, stream);
  prof_after(MSA_K_KL_DENSE, stream);
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  e = launch_mean(kl_rows, d.rows * d.Hkv, kl_mean, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_kl_dense_bwd(const msa_shape* shape, const void* q, const void* k,
                            const void* q_idx, const void* k_idx, const float* lse_main,
                            float coef, float* lse_idx, float* kl_rows, float* kl_mean,
                            float* block_mass, void* dq_idx, void* dk_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.dtype == MSA_F32 && d.D != 64) return MSA_ERR_UNSUPPORTED;
  if (kl_mean && !kl_rows) return MSA_ERR_NULL;
  const size_t dk_bytes = (size_t)d.B * d.N * d.DI * elem_size(d);
  if (d.rows == 0) {  // no rows: dk_idx gets no contributions, the mean is 0
    if (dk_bytes > 0 && !dk_idx) return MSA_ERR_NULL;
    if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
    if (dk_bytes > 0 &&
        launch_fill_i32(static_cast<int32_t*>(dk_idx), (int64_t)(dk_bytes / 4), 0, stream) !=
            hipSuccess)
      return MSA_ERR_DEVICE;
    if (kl_mean && launch_fill_f32(kl_mean, 1, 0.0f, stream) != hipSuccess) return MSA_ERR_DEVICE;
    return MSA_OK;
  }
  if (!q || !k || !q_idx || !k_idx || !lse_main || !lse_idx || !dq_idx || !dk_idx)
    return MSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx))
    return MSA_ERR_SHAPE;
  const Layout L = layout(d, MSA_OP_KL_DENSE_BWD);
  if ((st = check_ws(L, workspace, workspace_bytes)) != MSA_OK) return st;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  if (block_mass &&
      launch_fill_f32(block_mass, d.rows * d.Hkv * d.nb, 0.0f, stream) != hipSuccess)
    return MSA_ERR_DEVICE;
  prof_before(MSA_K_DENSE_LSE_IDX, stream);
  hipError_t e = launch_dense_lse(d, true, q_idx, k_idx, lse_idx, stream);
  prof_after(MSA_K_DENSE_LSE_IDX, stream);
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  e = launch_kl_dense_grad(d, q, k, q_idx, k_idx, lse_main, lse_idx, kl_rows, block_mass, coef,
                           reinterpret_cast<bf16*>(ws + L.dense_ds),
                           reinterpret_cast<float*>(ws + L.dki_acc), dq_idx, dk_idx, stream);
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  if (kl_mean) e = launch_mean(kl_rows, d.rows * d.Hkv, kl_mean, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_block_recall(const msa_shape* shape, const float* block_mass,
                            const int32_t* block_ids, float* block_recall, float* score_recall,
                            float* means, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.rows > 0 && (!block_mass || !block_ids || !block_recall || !score_recall))
    return MSA_ERR_NULL;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  const int64_t n = d.rows * d.Hkv;
  if (n > 0) {
    prof_before(MSA_K_RECALL, stream);
    const hipError_t e = launch_recall(d, block_mass, block_ids, block_recall, score_recall, stream);
    prof_after(MSA_K_RECALL, stream);
    if (e != hipSuccess) return MSA_ERR_DEVICE;
  }
  if (means) {
    if (launch_mean(block_recall, n, means, stream) != hipSuccess ||
        launch_mean(score_recall, n, means + 1, stream) != hipSuccess)
      return MSA_ERR_DEVICE;
  }
  return MSA_OK;
}

msa_status msa_index_quantize_fp8(const msa_shape* shape, const void* q_idx, const void* k_idx,
                                  uint8_t* q8, int32_t* q_exp, uint8_t* k8, int32_t* k_exp,
                                  hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (!q8 && !k8) return MSA_ERR_NULL;
  if (q8 && d.rows > 0 && (!q_idx || !q_exp)) return MSA_ERR_NULL;
  if (k8 && d.B > 0 && d.N > 0 && (!k_idx || !k_exp)) return MSA_ERR_NULL;
  if ((q8 && !aligned16(q8)) || (k8 && !aligned16(k8))) return MSA_ERR_SHAPE;
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  prof_before(MSA_K_QUANTIZE_FP8, stream);
  const hipError_t e = launch_quantize_fp8(d, q_idx, k_idx, q8, q_exp, k8, k_exp, stream);
  prof_after(MSA_K_QUANTIZE_FP8, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

msa_status msa_select_fp8(const msa_shape* shape, const uint8_t* q8, const int32_t* q_exp,
                          const uint8_t* k8, const int32_t* k_exp, int32_t* block_ids,
                          float* block_scores, float* cutoff_margin, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  msa_status st = make_dims(shape, &d);
  if (st != MSA_OK) return st;
  if (d.rows == 0) return MSA_OK;
  if (!q8 || !q_exp || !k8 || !k_exp || !block_ids) return MSA_ERR_NULL;
  if (!aligned16(q8) || !aligned16(k8)) return MSA_ERR_SHAPE;
  float* M = block_scores;
  if (!M) {
    const Layout L = layout(d, MSA_OP_SELECT);
    if ((st = check_ws(L, workspace, workspace_bytes)) != MSA_OK) return st;
    M = static_cast<float*>(workspace);
  }
  if ((st = check_device(&d.num_cus)) != MSA_OK) return st;
  prof_before(MSA_K_INDEX_FP8, stream);
  hipError_t e = launch_index_blockmax_fp8(d, q8, q_exp, k8, k_exp, M, stream);
  prof_after(MSA_K_INDEX_FP8, stream);
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  prof_before(MSA_K_TOPK, stream);
  e = launch_topk(d, M, block_ids, cutoff_margin, stream);
  prof_after(MSA_K_TOPK, stream);
  return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
}

}  // extern "C"
