// msa_attn.hip — KV-outer sparse attention over the selected blocks.
//
// Exact softmax attention restricted to the selected support ("2.4 · 训练原生
// 稀疏" (training-native sparse attention) eq. 2), per GQA group: the group's G
// query heads share the block list and KV head r, each keeps its own query
// ("MSA Indexer 与 DSA Lightning Indexer 的差别" §2.3). Execution is KV-outer
// ("MiniMax Sparse Attention：教长上下文模型使用索引", kernel section): the
// selections are inverted into per-(batch, group, block) buckets of the query
// rows that chose the block, each block is loaded once into LDS for a chunk of
// those rows, and buckets that many rows chose (block 0, local blocks, hot
// blocks) are cut into fixed-size work items so no block becomes a straggler.
// Each (query, head, slot) gets a normalised partial output and its
// log-sum-exp; the combine merges the <= k partials of a (query, head) with
// the partition rule of "2.4" eq. (18) / "4.1.1 · 监督与联合训练" eq. (16):
// LSE = logsumexp_s LSE_s, O = sum_s exp(LSE_s - LSE) O_s.
#include "msa_internal.hpp"

namespace msa {

// ============================================================== bucketing (counting sort)
//
// bucket(b, r, w, blk) = ((b*Hkv + r)*nwin + w)*nb + blk with w = t / kQueryWindow;
// entry = (t << 6) | slot. A histogram workgroup's rows lie in one window.
// With skip_local, a row's own block floor((q_start + t)/128) gets no entry: the
// combine computes that block's attention query-outer instead.

// query rows per histogram / scatter workgroup: 64 gives a 32768-query attention
// window 512 workgroups (256 rows: 128, half the CUs idle; bucketing of the skewed
// 131072 step in four windows 0.51 -> 0.34 ms)
#ifndef MSA_BUCKET_ROWS
#define MSA_BUCKET_ROWS 64
#endif
constexpr int kBucketRows = MSA_BUCKET_ROWS;

template <bool LDSH>
__global__ void __launch_bounds__(256)
bucket_hist_kernel(const int32_t* __restrict__ ids, int Nq, int q_start, int Hkv, int K, int nb,
                   int nwin, bool skip_local, int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  const int HB = Hkv * nb;
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kBucketRows;
  const int t1 = min(Nq, t0 + kBucketRows);
  if (LDSH) {
    for (int x = threadIdx.x; x < HB; x += 256) hist[x] = 0;
    __syncthreads();
  }
  const int n = (t1 - t0) * Hkv * K;
  const int32_t* base = ids + ((size_t)(b * (size_t)Nq + t0) * Hkv) * K;
  const int w = t0 / kQueryWindow;
  // bucket of local bin x = r*nb + blk
  auto gbin = [&](int x) {
    return (((size_t)b * Hkv + x / nb) * nwin + w) * nb + x % nb;
  };
  for (int e = threadIdx.x; e < n; e += 256) {
    const int id = base[e];
    const bool local = skip_local && id == (q_start + t0 + e / (Hkv * K)) >> 7;
    if (id >= 0 && id < nb && !local) {
      const int r = (e / K) % Hkv;
      if (LDSH) atomicAdd(&hist[r * nb + id], 1);
      else atomicAdd(&counts[gbin(r * nb + id)], 1);
    }
  }
  if (LDSH) {
    __syncthreads();
    for (int x = threadIdx.x; x < HB; x += 256)
      if (hist[x]) atomicAdd(&counts[gbin(x)], hist[x]);
  }
}

// Exclusive scans of entry counts and of item counts (ceil(count / qt)) over
// all buckets, in two passes over chunks of kScanChunk buckets: chunk sums,
// then each workgroup adds the sums of the chunks before it and scans its own
// chunk. The last chunk writes the grand totals.
constexpr int kScanChunk = 4096;  // buckets per workgroup (1024 threads x 4)

__global__ void __launch_bounds__(1024)
bucket_chunk_sum_kernel(const int32_t* __restrict__ counts, int64_t nbk, int qt,
                        int32_t* __restrict__ chunk_e, int32_t* __restrict__ chunk_i,
                        int32_t* __restrict__ chunk_c) {
  __shared__ int32_t se[32], si[32], sc[32];
  const int tid = threadIdx.x;
  const int64_t lo = (int64_t)blockIdx.x * kScanChunk;
  int32_t ce = 0, ci = 0, cc = 0;
  for (int j = 0; j < kScanChunk / 1024; ++j) {
    const int64_t x = lo + j * 1024 + tid;
    if (x < nbk) {
      const int32_t c = counts[x];
      const int32_t ni = (c + qt - 1) / qt;
      ce += c;
      ci += ni;
      cc += ni * kItemCost + (ni > 0 ? kItemStartCost : 0);
    }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    ce += __shfl_xor(ce, m, 64);
    ci += __shfl_xor(ci, m, 64);
    cc += __shfl_xor(cc, m, 64);
  }
  if ((tid & 63) == 0) {
    se[tid >> 6] = ce;
    si[tid >> 6] = ci;
    sc[tid >> 6] = cc;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t te = 0, ti = 0, tc = 0;
    for (int w = 0; w < 16; ++w) {
      te += se[w];
      ti += si[w];
      tc += sc[w];
    }
    chunk_e[blockIdx.x] = te;
    chunk_i[blockIdx.x] = ti;
    chunk_c[blockIdx.x] = tc;
  }
}

__global__ void __launch_bounds__(1024)
bucket_scan_kernel(const int32_t* __restrict__ counts, int64_t nbk, int qt,
                   const int32_t* __restrict__ chunk_e, const int32_t* __restrict__ chunk_i,
                   const int32_t* __restrict__ chunk_c, int32_t* __restrict__ offsets,
                   int32_t* __restrict__ cursor, int32_t* __restrict__ item_off,
                   int32_t* __restrict__ cost_off, int32_t* __restrict__ totals,
                   int entries_max, int items_max) {
  __shared__ int32_t se[1024], si[1024], sc[1024];
  __shared__ int32_t base_e, base_i, base_c;
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  if (tid == 0) {
    int32_t be = 0, bi = 0, bc = 0;
    for (int c = 0; c < chunk; ++c) {
      be += chunk_e[c];
      bi += chunk_i[c];
      bc += chunk_c[c];
    }
    base_e = be;
    base_i = bi;
    base_c = bc;
  }
  const int64_t lo = (int64_t)chunk * kScanChunk + (int64_t)tid * (kScanChunk / 1024);
  const int64_t hi = min(nbk, lo + kScanChunk / 1024);
  int32_t ce = 0, ci = 0, cc = 0;
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t c = counts[x];
    const int32_t ni = (c + qt - 1) / qt;
    ce += c;
    ci += ni;
    cc += ni * kItemCost + (ni > 0 ? kItemStartCost : 0);
  }
  se[tid] = ce;
  si[tid] = ci;
  sc[tid] = cc;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t ae = tid >= off ? se[tid - off] : 0;
    const int32_t ai = tid >= off ? si[tid - off] : 0;
    const int32_t ac = tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    se[tid] += ae;
    si[tid] += ai;
    sc[tid] += ac;
    __syncthreads();
  }
  // exclusive
  int32_t re = base_e + se[tid] - ce, ri = base_i + si[tid] - ci, rc = base_c + sc[tid] - cc;
  for (int64_t x = lo; x < hi; ++x) {
    const int32_t c = counts[x];
    const int32_t ni = (c + qt - 1) / qt;
    offsets[x] = re;
    cursor[x] = re;
    item_off[x] = ri;
    cost_off[x] = rc;
    re += c;
    ri += ni;
    rc += ni * kItemCost + (ni > 0 ? kItemStartCost : 0);
  }
  if (chunk == (int)gridDim.x - 1 && tid == 1023) {
    const int32_t te = base_e + se[1023], ti = base_i + si[1023], tc = base_c + sc[1023];
    offsets[nbk] = te;
    item_off[nbk] = ti;
    cost_off[nbk] = tc;
    // both bounds hold for valid ids; clamping keeps malformed ids from
    // indexing past the work arrays
    totals[0] = min(te, entries_max);
    totals[1] = min(ti, items_max);
    totals[2] = tc;
    totals[3] = 0;  // no balanced split until wg_split_kernel writes one
  }
}

template <bool LDSH>
__global__ void __launch_bounds__(256)
bucket_scatter_kernel(const int32_t* __restrict__ ids, int Nq, int q_start, int Hkv, int K, int nb,
                      int nwin, bool skip_local, int32_t* __restrict__ cursor,
                      int32_t* __restrict__ entries, int entries_max) {
  extern __shared__ int32_t sh[];
  const int HB = Hkv * nb;
  int32_t* hist = sh;
  int32_t* base = sh + (LDSH ? HB : 0);
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kBucketRows;
  const int t1 = min(Nq, t0 + kBucketRows);
  const int n = (t1 - t0) * Hkv * K;
  const int32_t* idp = ids + ((size_t)(b * (size_t)Nq + t0) * Hkv) * K;
  const int w = t0 / kQueryWindow;
  auto gbin = [&](int x) {
    return (((size_t)b * Hkv + x / nb) * nwin + w) * nb + x % nb;
  };
  if (LDSH) {
    for (int x = threadIdx.x; x < HB; x += 256) hist[x] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += 256) {
      const int id = idp[e];
      const bool local = skip_local && id == (q_start + t0 + e / (Hkv * K)) >> 7;
      if (id >= 0 && id < nb && !local) atomicAdd(&hist[((e / K) % Hkv) * nb + id], 1);
    }
    __syncthreads();
    for (int x = threadIdx.x; x < HB; x += 256) {
      const int c = hist[x];
      base[x] = c ? atomicAdd(&cursor[gbin(x)], c) : 0;
      hist[x] = 0;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < n; e += 256) {
    const int id = idp[e];
    const bool local = skip_local && id == (q_start + t0 + e / (Hkv * K)) >> 7;
    if (id >= 0 && id < nb && !local) {
      const int bin = ((e / K) % Hkv) * nb + id;
      const int p = LDSH ? base[bin] + atomicAdd(&hist[bin], 1) : atomicAdd(&cursor[gbin(bin)], 1);
      const int t = t0 + e / (Hkv * K);
      if (p < entries_max) entries[p] = (t << 6) | (e % K);  // bound holds for valid ids
    }
  }
}

// One thread per work item: item = (bucket, first entry, count <= qt).
__global__ void __launch_bounds__(256)
work_items_kernel(const int32_t* __restrict__ item_off, const int32_t* __restrict__ offsets,
                  const int32_t* __restrict__ cost_off, const int32_t* __restrict__ totals,
                  int64_t nbk, int qt, int4* __restrict__ items) {
  const int it = blockIdx.x * 256 + threadIdx.x;
  if (it >= totals[1]) return;
  int64_t lo = 0, hi = nbk - 1;  // largest bkt with item_off[bkt] <= it
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (item_off[mid] <= it) lo = mid;
    else hi = mid - 1;
  }
  const int64_t bkt = lo;
  const int local = it - item_off[bkt];
  const int start = offsets[bkt] + local * qt;
  const int cnt = max(0, min(min(qt, offsets[bkt + 1] - start), totals[0] - start));
  // work cost before the item: a bucket's first item costs kItemCost + kItemStartCost
  const int cost = cost_off[bkt] + (local == 0 ? 0 : kItemStartCost + local * kItemCost);
  items[it] = make_int4((int)bkt, start, cnt, cost);
}

// Balanced ranges of a persistent kernel of R workgroups: range r holds the items
// whose work cost before them lies in [r C / R, (r+1) C / R), C the total cost
// (costs increase along the item list, so the ranges are contiguous and partition
// it). Item i writes wg_start[r] = i for every r in (range(i-1), range(i)]; the
// end sentinel i = total closes the last ranges. Every entry 0..R has one writer.
__global__ void __launch_bounds__(256)
wg_split_kernel(const int4* __restrict__ items, int32_t* __restrict__ totals, int R,
                int32_t* __restrict__ wg_start) {
  const int total = totals[1];
  const int64_t C = totals[2];
  for (int i = blockIdx.x * 256 + threadIdx.x; i <= total; i += gridDim.x * 256) {
    const int ri = i < total ? (int)((int64_t)items[i].w * R / C) : R;
    const int rp = i > 0 ? (int)((int64_t)items[i - 1].w * R / C) : -1;
    for (int r = rp + 1; r <= ri; ++r) wg_start[r] = i;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) totals[3] = R;
}

// One query per sequence (decode): a row's valid ids are distinct, so every
// (batch, group, block) bucket holds one entry and each entry is its own work
// item; one workgroup compacts them in order, skipping empty slots (and the
// local block with skip_local).
constexpr int64_t kDirectMax = 1 << 15;  // slots one workgroup compacts (32 passes)

__global__ void __launch_bounds__(1024)
direct_items_kernel(const int32_t* __restrict__ ids, int64_t nrows, int K, int nb, int nwin,
                    int q_start, bool skip_local, int32_t* __restrict__ entries,
                    int4* __restrict__ items, int32_t* __restrict__ totals) {
  __shared__ int wsum[16];
  __shared__ int wbase[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = q_start / 128;
  const int64_t n = nrows * K;
  int base = 0;
  for (int64_t e0 = 0; e0 < n; e0 += 1024) {
    const int64_t e = e0 + tid;
    const int id = e < n ? ids[e] : -1;
    const bool valid = id >= 0 && id < nb && !(skip_local && id == L);
    const uint64_t bal = __ballot(valid);
    const int before = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int w = 0; w < 16; ++w) {
        wbase[w] = acc;
        acc += wsum[w];
      }
      wsum[0] = acc;  // the chunk's total, read after the next barrier
    }
    __syncthreads();
    if (valid) {
      const int pos = base + wbase[wave] + before;
      const int64_t row = e / K;  // (b, r) of Nq = 1
      entries[pos] = (int)(e % K);  // (t = 0) << 6 | slot
      items[pos] = make_int4((int)(row * nwin * nb + id), pos, 1, 0);
    }
    base += wsum[0];
    __syncthreads();
  }
  if (tid == 0) {
    totals[0] = base;
    totals[1] = base;
    totals[2] = base;
    totals[3] = 0;  // no balanced split: one-entry items are split by count
  }
}

// Canonical order inside each bucket, for the backward's fixed summation order.
// A bucket's entries come from distinct rows t (the valid ids of a row are
// distinct), so row order is a total order: one workgroup per bucket marks the
// rows present in an LDS bitmap (kSortWords words, 32 * kSortWords rows per
// pass) and writes each entry at its rank, the number of present rows below
// its own (prefix popcounts). If the ranks do not account for every entry (two
// entries of one row: ids repeated in a row, which msa_select never produces)
// the bucket is copied in scatter order, so the output is always a
// permutation of the input.
constexpr int kSortWords = 4096;

__global__ void __launch_bounds__(256)
bucket_sort_kernel(const int32_t* __restrict__ offsets, int64_t nbk, int Nq, int entries_max,
                   const int32_t* __restrict__ src, int32_t* __restrict__ dst) {
  __shared__ uint32_t bits[kSortWords];
  __shared__ int32_t pref[kSortWords];
  __shared__ int32_t wsum[4];
  constexpr int WPT = kSortWords / 256;  // words per thread in the scan
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int64_t bkt = blockIdx.x; bkt < nbk; bkt += gridDim.x) {
    const int lo = min(offsets[bkt], entries_max), hi = min(offsets[bkt + 1], entries_max);
    if (hi - lo <= 1) {
      if (hi - lo == 1 && tid == 0) dst[lo] = src[lo];
      continue;  // uniform
    }
    int placed = 0;
    for (int tb = 0; tb < Nq; tb += 32 * kSortWords) {
      const int nw = min(kSortWords, (Nq - tb + 31) / 32);  // words used in this pass
      for (int x = tid; x < nw; x += 256) bits[x] = 0u;
      __syncthreads();
      for (int e = lo + tid; e < hi; e += 256) {
        const int t = (src[e] >> 6) - tb;
        if (t >= 0 && t < 32 * nw) atomicOr(&bits[t >> 5], 1u << (t & 31));
      }
      __syncthreads();
      int c[WPT], sum = 0;
#pragma unroll
      for (int j = 0; j < WPT; ++j) {
        const int x = tid * WPT + j;
        c[j] = x < nw ? __popc(bits[x]) : 0;
        sum += c[j];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (lane == 63) wsum[wave] = incl;
      __syncthreads();
      int run = incl - sum;
      for (int v = 0; v < wave; ++v) run += wsum[v];
      const int pass_total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
#pragma unroll
      for (int j = 0; j < WPT; ++j) {
        const int x = tid * WPT + j;
        if (x < nw) pref[x] = run;
        run += c[j];
      }
      __syncthreads();
      for (int e = lo + tid; e < hi; e += 256) {
        const int v = src[e];
        const int t = (v >> 6) - tb;
        if (t >= 0 && t < 32 * nw) {
          const int rank = placed + pref[t >> 5] + __popc(bits[t >> 5] & ((1u << (t & 31)) - 1u));
          if (rank < hi - lo) dst[lo + rank] = v;
        }
      }
      placed += pass_total;
      __syncthreads();  // bitmap, prefix and wsum are rewritten by the next pass
    }
    if (placed != hi - lo) {  // uniform: not a set of distinct rows
      for (int e = lo + tid; e < hi; e += 256) dst[e] = src[e];
    }
  }
}

static size_t bucket_lds_bytes(const Dims& d, int arrays) {
  return (size_t)arrays * d.Hkv * d.nb * sizeof(int32_t);
}
static bool bucket_use_lds(const Dims& d) { return bucket_lds_bytes(d, 2) <= 64 * 1024; }

hipError_t launch_bucketing(const Dims& d, const int32_t* ids, const AttnWs& w, bool skip_local,
                            hipStream_t s, int split_grid) {
  hipError_t e;
  // the direct path records no per-bucket offsets, which the canonical order needs
  if (!w.sorted && d.Nq == 1 && d.rows > 0 && d.items_max >= d.entries_max &&
      d.rows * d.Hkv * d.K <= kDirectMax) {
    prof_before(MSA_K_BUCKET_HIST, s);
    direct_items_kernel<<<1, 1024, 0, s>>>(ids, d.rows * d.Hkv, d.K, d.nb, d.nwin, d.q_start,
                                           skip_local, w.entries, w.items, w.totals);
    prof_after(MSA_K_BUCKET_HIST, s);
    return hipGetLastError();
  }
  if ((e = launch_fill_i32(w.counts, d.buckets, 0, s)) != hipSuccess) return e;
  const unsigned nchunks = (unsigned)((d.buckets + kScanChunk - 1) / kScanChunk);
  auto scan = [&](int entries_max, int items_max) {
    bucket_chunk_sum_kernel<<<nchunks, 1024, 0, s>>>(w.counts, d.buckets, d.qt, w.chunk_e,
                                                     w.chunk_i, w.chunk_c);
    bucket_scan_kernel<<<nchunks, 1024, 0, s>>>(w.counts, d.buckets, d.qt, w.chunk_e,
                                                w.chunk_i, w.chunk_c, w.offsets, w.cursor,
                                                w.item_off, w.cost_off, w.totals, entries_max,
                                                items_max);
  };
  if (d.rows == 0) {
    scan(0, 0);
    return hipGetLastError();
  }
  const dim3 grid((d.Nq + kBucketRows - 1) / kBucketRows, d.B);
  const bool lds = bucket_use_lds(d);
  prof_before(MSA_K_BUCKET_HIST, s);
  if (lds)
    bucket_hist_kernel<true><<<grid, 256, bucket_lds_bytes(d, 1), s>>>(
        ids, d.Nq, d.q_start, d.Hkv, d.K, d.nb, d.nwin, skip_local, w.counts);
  else
    bucket_hist_kernel<false><<<grid, 256, 0, s>>>(ids, d.Nq, d.q_start, d.Hkv, d.K, d.nb,
                                                   d.nwin, skip_local, w.counts);
  prof_after(MSA_K_BUCKET_HIST, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_before(MSA_K_BUCKET_SCAN, s);
  scan((int)d.entries_max, (int)d.items_max);
  prof_after(MSA_K_BUCKET_SCAN, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_before(MSA_K_BUCKET_SCATTER, s);
  if (lds)
    bucket_scatter_kernel<true><<<grid, 256, bucket_lds_bytes(d, 2), s>>>(
        ids, d.Nq, d.q_start, d.Hkv, d.K, d.nb, d.nwin, skip_local, w.cursor, w.entries,
        (int)d.entries_max);
  else
    bucket_scatter_kernel<false><<<grid, 256, 0, s>>>(ids, d.Nq, d.q_start, d.Hkv, d.K, d.nb,
                                                     d.nwin, skip_local, w.cursor, w.entries,
                                                     (int)d.entries_max);
  prof_after(MSA_K_BUCKET_SCATTER, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (w.sorted && d.buckets > 0) {
    prof_before(MSA_K_BUCKET_SORT, s);
    bucket_sort_kernel<<<(unsigned)std::min<int64_t>(d.buckets, 4096), 256, 0, s>>>(
        w.offsets, d.buckets, d.Nq, (int)d.entries_max, w.entries, w.sorted);
    prof_after(MSA_K_BUCKET_SORT, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (d.items_max > 0) {
    prof_before(MSA_K_WORK_ITEMS, s);
    work_items_kernel<<<(unsigned)((d.items_max + 255) / 256), 256, 0, s>>>(
        w.item_off, w.offsets, w.cost_off, w.totals, d.buckets, d.qt, w.items);
    if (split_grid > 0 && split_grid <= kMaxSplit)
      wg_split_kernel<<<(unsigned)std::min<int64_t>((d.items_max + 256) / 256, 1024), 256, 0,
                        s>>>(w.items, w.totals, split_grid, w.wg_start);
    prof_after(MSA_K_WORK_ITEMS, s);
  }
  return hipGetLastError();
}

// ============================================================== sparse attention (KV-outer)
//
// One workgroup (4 waves) per work item: a 128-token K/V block of group r and
// up to QT = 128/G query rows that selected it, i.e. 128 (query, head) rows,
// 32 per wave. K and V are staged in LDS row-major.
//   S^T = K Q^T   A = K rows from LDS, B = the wave's Q rows (registers);
//                 each lane then holds 64 keys of one (query, head) row, so
//                 the row max / sum are in-lane plus one exchange.
//   O^T = V^T P^T B = P^T straight from the S^T accumulator (the key set a
//                 lane holds is the k-set it supplies); A = V^T, read from the
//                 row-major V tile with gfx950's transposing LDS read
//                 (ds_read_b64_tr_b16: each 16-lane group reads a 4-key x
//                 16-d tile and lane j receives the 4 keys of column j).
//                 fp32 inputs have no transposing read and stage V^T instead.
// Blocks past a query's position are masked (j > i) only where needed.
// The item -> workgroup mapping keeps consecutive items (same K/V block) on
// the same XCD: workgroup id g runs on XCD g % 8.

template <typename T> struct AttnPad;
template <> struct AttnPad<bf16> { static constexpr int K = 8, V = 8; };
template <> struct AttnPad<float> { static constexpr int K = 4, V = 2; };


// A operand of O^T = V^T P^T for k-step st and d tile dt from row-major V:
// elements 0..3 = V[16st + 4h + 0..3][d], 4..7 = V[16st + 4h + 8..11][d],
// d = 32dt + l32.
template <int LDV>
__device__ __forceinline__ bf16x8 v_frag_tr(const bf16* Vs, int st, int dt, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int krow = 16 * st + 4 * (g >> 1) + (s >> 2);
  const int dcol = dt * 32 + 16 * (g & 1) + 4 * (s & 3);
  typedef __attribute__((address_space(3))) short4v lds_short4;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(Vs + krow * LDV + dcol));
  const short4v hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(Vs + (krow + 8) * LDV + dcol));
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = l4[e];
    r[4 + e] = h4[e];
  }
  return r;
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(256, 2)
sparse_attn_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const int4* __restrict__ items, const int32_t* __restrict__ entries,
                   const int32_t* __restrict__ totals, T* __restrict__ opart,
                   float* __restrict__ lpart, int N, int Nq, int q_start, int Hkv, int nb,
                   int nbw, int topk, float scale_log2) {
  constexpr bool TR = sizeof(T) == 2;  // bf16: row-major V + transposing reads
  constexpr int KSD = D / 16;          // k-steps over the head dim
  constexpr int DT = D / 32;           // 32-wide output d tiles
  constexpr int PK = AttnPad<T>::K, PV = AttnPad<T>::V;
  constexpr int LDV = TR ? D + PV : 128 + PV;
  __shared__ T Ks[128][D + PK];
  __shared__ T Vs[(TR ? 128 : D) * LDV];

  // XCD-aware item order: XCD x = g % 8 takes a contiguous range of items.
  const int total = totals[1];
  const int per = (total + 7) / 8;
  const int g = blockIdx.x;
  const int it = (g & 7) * per + (g >> 3);
  if ((g >> 3) >= per || it >= total) return;

  const int4 item = items[it];
  const int bkt = item.x, start = item.y, cnt = item.z;
  const int blk = bkt % nb;
  const int br = bkt / nbw;
  const int r = br % Hkv;
  const int b = br / Hkv;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int row = 32 * wave + l32;  // (query, head) row of the item
  const int qi = row / G;
  const int hg = row % G;
  const bool rv = qi < cnt;
  const int ent = rv ? entries[start + qi] : 0;
  const int t = ent >> 6, slot = ent & 63;
  const int i_row = q_start + t;
  const int Hq = Hkv * G;
  // this lane's Q fragments are requested before the K/V staging
  vec8<T> qf[KSD];
  {
    const T* qp = q + ((size_t)(b * (size_t)Nq + t) * Hq + r * G + hg) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) qf[ks] = rv ? ld8<T>(qp + 16 * ks) : zero8<T>();
  }
  // stage K and V
  const size_t kvrow = (size_t)Hkv * D;
  const T* kb = k + ((size_t)b * N + (size_t)blk * 128) * kvrow + (size_t)r * D;
  const T* vb = v + ((size_t)b * N + (size_t)blk * 128) * kvrow + (size_t)r * D;
  const int nvalid = min(128, N - blk * 128);
  constexpr int CH = D / 8;  // 8-element chunks per row
  for (int c = tid; c < 128 * CH; c += 256) {
    const int kr = c / CH, dc = c % CH;
    st8<T>(&Ks[kr][dc * 8], kr < nvalid ? ld8<T>(kb + kr * kvrow + dc * 8) : zero8<T>());
    if (TR) st8<T>(&Vs[kr * LDV + dc * 8], kr < nvalid ? ld8<T>(vb + kr * kvrow + dc * 8)
                                                     : zero8<T>());
  }
  if (!TR) {
    for (int c = tid; c < 128 * CH; c += 256) {
      const int kr = c % 128, dc = c / 128;
      const vec8<T> x = kr < nvalid ? ld8<T>(vb + kr * kvrow + dc * 8) : zero8<T>();
#pragma unroll
      for (int e = 0; e < 8; ++e) Vs[(dc * 8 + e) * LDV + kr] = x[e];
    }
  }
  __syncthreads();

  f32x16 sacc[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
      mma(sacc[kt], ld8<T>(&Ks[kt * 32 + l32][16 * ks + 8 * h]), qf[ks]);
  }
  // softmax over the 128 keys of this block, in the log2 domain
  const bool need_mask = blk * 128 + 127 > i_row;
  // the same arithmetic, in the same order, as the persistent kernel: a row
  // gets identical P, O and LSE whichever kernel processes it
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    if (need_mask) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (blk * 128 + kt * 32 + drow(e, h) > i_row) sacc[kt][e] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 16; e += 2) mx = vmax(vmax(mx, sacc[kt][e]), sacc[kt][e + 1]);
  }
  mx = vmax(mx, shfl_xor_f(mx, 32));
  const float mxs = mx * scale_log2;
  float ls = 0.0f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], scale_log2, -mxs));
      sacc[kt][e] = p;
      ls += p;
    }
  }
  ls += shfl_xor_f(ls, 32);

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.0f;
#pragma unroll
  for (int st = 0; st < 8; ++st) {  // 16 keys per step: elements 8*(st%2).. of tile st/2
    vec8<T> pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = cvt<T>(sacc[st >> 1][8 * (st & 1) + e]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      vec8<T> vf;
      if constexpr (TR) {
        vf = v_frag_tr<LDV>(reinterpret_cast<const bf16*>(Vs), st, dt, lane);
      } else {
        const int key0 = 16 * st + 4 * h;  // keys key0..key0+3 and key0+8..key0+11
        const T* vp = &Vs[(dt * 32 + l32) * LDV + key0];
        const vec4<T> lo = ld4<T>(vp), hi = ld4<T>(vp + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[e] = lo[e];
          vf[4 + e] = hi[e];
        }
      }
      mma(oacc[dt], vf, pf);
    }
  }
  if (rv) {
    const float inv = 1.0f / ls;
    const size_t entry = ((size_t)(b * (size_t)Nq + t) * Hkv + r) * topk + slot;
    T* op = opart + (entry * G + hg) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        vec4<T> o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = cvt<T>(oacc[dt][4 * jg + e] * inv);
        st4<T>(op + dt * 32 + 8 * jg + 4 * h, o);
      }
    }
    if (h == 0) lpart[entry * G + hg] = (mxs + __log2f(ls)) * kLn2;
  }
}

// ------------------------------------------------------------ bf16: persistent, pipelined
//
// One workgroup of 8 waves per CU, looping over a contiguous range of work
// items of its XCD (consecutive items mostly share one K/V block). A work item
// is 256 (query, head) rows, 32 per wave.
//  - K and V of a block are copied HBM/L2 -> LDS with global_load_lds (16 B per
//    lane) only when the next item needs a different block.
//  - The MFMA operand layouts tie a lane to one (query, head) row, so a direct
//    load or store of Q or O would touch 32 rows per instruction. Both go
//    through a per-wave LDS region instead: the next item's Q rows are loaded
//    row-contiguously (1 KB per instruction) and re-read as fragments, and the
//    output tile is written to LDS and stored row-contiguously. The memory
//    address path, not the matrix cores, is otherwise the limit.
// LDS tiles are row-major without padding; the 16-byte chunk c of row rho is
// stored at chunk c ^ swz(rho) (patterns below).

// Partials are written once and read once, long after: stream them past the
// caches (non-temporal stores in the attention kernel, loads in the combine).
#ifndef MSA_NT_LOAD
#define MSA_NT_LOAD 1
#endif
#ifndef MSA_NT_STORE
#define MSA_NT_STORE 1
#endif

// NWV waves per workgroup, 32 (query, head) rows each: 8 for prefill (one
// workgroup per CU); 1 when a bucket holds at most 32/G queries (decode), so
// that two workgroups share a CU and one's K/V copy overlaps the other's work.
template <int D, int G, int NWV>
__global__ void __launch_bounds__(64 * NWV, 1)
sparse_attn_pipe_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                        const bf16* __restrict__ v, const int4* __restrict__ items,
                        const int32_t* __restrict__ entries, const int32_t* __restrict__ totals,
                        const int32_t* __restrict__ wg_start,
                        bf16* __restrict__ opart, float* __restrict__ lpart, int N, int Nq,
                        int q_start, int Hkv, int nb, int nbw, int topk, float scale_log2,
                        size_t dummy_entry) {
  constexpr int KSD = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;                             // 16-byte chunks per row
  constexpr int TILE = 128 * D;                          // elements per K or V tile
  constexpr int LOADS = 128 * CPR / (64 * NWV);   // global_load_lds per wave per tile
  constexpr int LDW = D + 8;                             // staging row stride (elements)
  constexpr int RCH = 32 * CPR / 64;                     // row chunks per lane per wave tile
  __shared__ bf16 Kb[TILE];
  __shared__ bf16 Vb[TILE];
  __shared__ bf16 Wst[NWV][32 * LDW];
  typedef __attribute__((address_space(3))) void lds_void;

  // Workgroup g runs on XCD g % 8. XCD x takes the x-th eighth of the item list and
  // its workgroups contiguous ranges of it, so consecutive items (one block) share an
  // XCD's L2: range r = x * (gridDim.x / 8) + g / 8, cut by work cost when the
  // bucketing wrote a split for this grid (balances the K/V reloads), else by count.
  const int total = totals[1];
  const int nwg_x = gridDim.x / 8;  // workgroups per XCD (gridDim.x is a multiple of 8)
  const int x = blockIdx.x & 7, gx = blockIdx.x >> 3;
  int i0, i1;
  if (totals[3] == (int)gridDim.x) {
    const int rg = x * nwg_x + gx;
    i0 = wg_start[rg];
    i1 = wg_start[rg + 1];
  } else {
    const int per_x = (total + 7) / 8;
    const int x0 = x * per_x, x1 = min(total, x0 + per_x);
    const int per_wg = (per_x + nwg_x - 1) / nwg_x;
    i0 = x0 + gx * per_wg;
    i1 = min(x1, i0 + per_wg);
  }
  if (i0 >= i1) return;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = 32 * wave + l32;
  const int qi = row / G, hg = row % G;
  const int Hq = Hkv * G;
  const size_t kvrow = (size_t)Hkv * D;
  bf16* const W = Wst[wave];
  // One 1 KB row-contiguous access covers RPI rows. With G >= RPI they belong
  // to one query, so their addresses are a wave-uniform base plus a
  // lane-constant offset; the entries of the wave's QPW queries are read as
  // scalars.
  constexpr int RPI = 64 / CPR;
  constexpr bool kUniformRows = G >= RPI;
  constexpr int QPW = kUniformRows ? 32 / G : 1;  // queries per wave
  const int qw0 = (32 * wave) / G;                // first query of the wave in an item

  // async copy of the K and V tiles of bucket `bkt`
  auto stage = [&](int bkt) {
    const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
    const int nvalid = min(128, N - blk * 128);
    const size_t base = ((size_t)b * N + (size_t)blk * 128) * kvrow + (size_t)r * D;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int p = (wave * LOADS + j) * 64 + lane;  // 16-byte LDS position in the tile
      const int rho = p / CPR, cs = p % CPR;
      const size_t rowbase = base + (size_t)min(rho, nvalid - 1) * kvrow;
      const size_t srck = rowbase + 8 * (cs ^ swz_k<D>(rho));
      const size_t srcv = rowbase + 8 * (cs ^ swz_v<D>(rho));
      __builtin_amdgcn_global_load_lds((const void*)(k + srck),
                                       (lds_void*)(&Kb[(wave * LOADS + j) * 512]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(v + srcv),
                                       (lds_void*)(&Vb[(wave * LOADS + j) * 512]), 16, 0, 0);
    }
  };
  // Row-contiguous load of the wave's 32 Q rows of an item: lane chunk
  // c = lane + 64*u covers row c / CPR, 16-byte chunk c % CPR. `ent_row` is
  // the entry of this lane's MFMA row (row l32); rows are fetched by shuffle.
  auto load_q_rows = [&](int bkt, int ent_row, const int* es, vec8<bf16>* raw) {
    const int br = bkt / nbw, r = br % Hkv, b = br / Hkv;
    if constexpr (kUniformRows) {
      // Q row of (query j of the wave, head 0 of group r); < 2^31 (checked by the caller)
      int qrow[QPW];
#pragma unroll
      for (int j = 0; j < QPW; ++j) qrow[j] = ((b * Nq + (es[j] >> 6)) * Hkv + r) * G;
#pragma unroll
      for (int u = 0; u < RCH; ++u) {
        const int j = (RPI * u) / G, hd = (RPI * u) % G;  // 32*wave is a multiple of G
        const bf16* base = q + (size_t)(uint32_t)qrow[j] * D + hd * D;
        raw[u] = ld8<bf16>(base + (lane / CPR) * D + 8 * (lane % CPR));
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < RCH; ++u) {
      const int c = lane + 64 * u;
      const int rr = c / CPR;  // row within the wave tile
      const int e = __shfl(ent_row, rr, 64);
      const int rg = 32 * wave + rr;
      raw[u] = ld8<bf16>(q + ((size_t)(b * (size_t)Nq + (e >> 6)) * Hq + r * G + rg % G) * D +
                         8 * (c % CPR));
    }
  };
  // raw rows -> staging region -> MFMA B fragments (lane row l32, k-half h)
  auto rows_to_frags = [&](const vec8<bf16>* raw, vec8<bf16>* qf) {
#pragma unroll
    for (int u = 0; u < RCH; ++u) {
      const int c = lane + 64 * u;
      st8<bf16>(W + (c / CPR) * LDW + 8 * (c % CPR), raw[u]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) qf[ks] = ld8<bf16>(W + l32 * LDW + 16 * ks + 8 * h);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  };

  // Every load reads a clamped, in-bounds address and is issued
  // unconditionally: rows past an item's count compute on a valid but unused
  // query and are stored to a scratch slot.
  const int ent_last = max(0, totals[0] - 1);
  auto entry_of = [&](const int4& itm) { return entries[min(itm.y + qi, ent_last)]; };
  // entries of the wave's queries of an item (uniform loads)
  auto wave_entries = [&](const int4& itm, int* es) {
#pragma unroll
    for (int j = 0; j < QPW; ++j) es[j] = entries[min(itm.y + qw0 + j, ent_last)];
  };

  // prologue: item i0 staged and its Q fragments ready. Prefetch depths:
  // descriptors three items ahead, row entries two, Q rows one.
  int4 cur = items[i0];
  stage(cur.x);
  int ent = entry_of(cur);
  int es[QPW];
  wave_entries(cur, es);
  vec8<bf16> qf[KSD];
  {
    vec8<bf16> raw[RCH];
    load_q_rows(cur.x, ent, es, raw);
    rows_to_frags(raw, qf);
  }
  int4 nxt = items[min(i0 + 1, i1 - 1)];
  int4 nxt2 = items[min(i0 + 2, i1 - 1)];
  int ent_n = entry_of(nxt);
  int es_n[QPW];
  wave_entries(nxt, es_n);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = i0; it < i1; ++it) {
    const int bkt = cur.x, cnt = cur.z;
    const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
    const bool have_next = it + 1 < i1;
    // ---- requests for later items (unconditional, clamped)
    const int ent_n2 = entry_of(nxt2);
    int es_n2[QPW];
    wave_entries(nxt2, es_n2);
    const int4 nxt3 = items[min(it + 3, i1 - 1)];
    vec8<bf16> qraw[RCH];
    load_q_rows(nxt.x, ent_n, es_n, qraw);

    // ---- S^T = K Q^T for the current item
    const bool rv = qi < cnt;
    const int t = ent >> 6, slot = ent & 63;
    const int i_row = q_start + t;
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.0f;
      const int rho = kt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
        mma(sacc[kt], ld8<bf16>(Kb + tile_off<D, false>(rho, 16 * ks + 8 * h)), qf[ks]);
    }
    // ---- softmax over the block's 128 keys (log2 domain)
    float mx = -INFINITY;
    const bool need_mask = blk * 128 + 127 > i_row;
    if (__any(need_mask)) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (blk * 128 + kt * 32 + drow(e, h) > i_row) sacc[kt][e] = -INFINITY;
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = vmax(vmax(mx, sacc[kt][e]), sacc[kt][e + 1]);
    mx = vmax(mx, shfl_xor_f(mx, 32));
    const float mxs = mx * scale_log2;
    float ls = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], scale_log2, -mxs));
        sacc[kt][e] = p;
        ls += p;
      }
    }
    ls += shfl_xor_f(ls, 32);
    // ---- O^T = V^T P^T
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.0f;
    typedef __attribute__((address_space(3))) short4v lds_short4;
    const int g16 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      vec8<bf16> pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = cvt<bf16>(sacc[st >> 1][8 * (st & 1) + e]);
      const int krow = 16 * st + 4 * (g16 >> 1) + (s16 >> 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int dcol = dt * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4*)(Vb + tile_off<D, true>(krow, dcol)));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4*)(Vb + tile_off<D, true>(krow + 8, dcol)));
        const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
        bf16x8 vf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[e] = l4[e];
          vf[4 + e] = h4[e];
        }
        mma(oacc[dt], vf, pf);
      }
    }
    // ---- partial output: O tile -> staging region -> row-contiguous stores.
    // Rows past the item's count go to the scratch slot `dummy_entry`.
    {
      const float inv = 1.0f / ls;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          vec4<bf16> o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = cvt<bf16>(oacc[dt][4 * jg + e] * inv);
          st4<bf16>(W + l32 * LDW + dt * 32 + 8 * jg + 4 * h, o);
        }
      }
      const size_t my_entry =
          rv ? ((size_t)(b * (size_t)Nq + t) * Hkv + r) * topk + slot : dummy_entry;
      lpart[my_entry * G + hg] = (mxs + __log2f(ls)) * kLn2;  // both lane halves hold it
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      if constexpr (kUniformRows) {
        // slot of query j of the wave (the scratch slot past the item's count); < 2^31
        int oslot[QPW];
#pragma unroll
        for (int j = 0; j < QPW; ++j)
          oslot[j] = qw0 + j < cnt ? ((b * Nq + (es[j] >> 6)) * Hkv + r) * topk + (es[j] & 63)
                                   : (int)dummy_entry;
#pragma unroll
        for (int u = 0; u < RCH; ++u) {
          const int j = (RPI * u) / G, hd = (RPI * u) % G;  // 32*wave is a multiple of G
          bf16* base = opart + (size_t)(uint32_t)oslot[j] * (G * D) + hd * D;
#if MSA_NT_STORE
          st8_nt<bf16>(base + (lane / CPR) * D + 8 * (lane % CPR),
                       ld8<bf16>(W + (RPI * u + lane / CPR) * LDW + 8 * (lane % CPR)));
#else
          st8<bf16>(base + (lane / CPR) * D + 8 * (lane % CPR),
                    ld8<bf16>(W + (RPI * u + lane / CPR) * LDW + 8 * (lane % CPR)));
#endif
        }
      } else {
#pragma unroll
        for (int u = 0; u < RCH; ++u) {
          const int c = lane + 64 * u;
          const int rr = c / CPR;
          const int e = __shfl(ent, rr, 64);
          const int rg = 32 * wave + rr;
          const bool ok = rg / G < cnt;
          const size_t entry =
              ok ? ((size_t)(b * (size_t)Nq + (e >> 6)) * Hkv + r) * topk + (e & 63) : dummy_entry;
          st8<bf16>(opart + (entry * G + rg % G) * D + 8 * (c % CPR),
                    ld8<bf16>(W + rr * LDW + 8 * (c % CPR)));
        }
      }
    }
    // ---- next item's Q fragments (the staging region is free again)
    vec8<bf16> qn[KSD];
    rows_to_frags(qraw, qn);
    // ---- a new block for the next item: reload the tiles once every wave is
    // done with the current ones (uniform: all waves see the same items).
    if (have_next && nxt.x != bkt) {
      __syncthreads();
      stage(nxt.x);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    cur = nxt;
    nxt = nxt2;
    nxt2 = nxt3;
    ent = ent_n;
    ent_n = ent_n2;
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      es[j] = es_n[j];
      es_n[j] = es_n2[j];
    }
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) qf[ks] = qn[ks];
  }
}

template <typename T, int D>
static hipError_t attn_dispatch_g(const Dims& d, const void* q, const void* k, const void* v,
                                  const AttnWs& w, void* opart, float* lpart, hipStream_t s) {
  const unsigned grid = (unsigned)(d.items_max + 8);
  const float scale_log2 = (float)(1.0 / sqrt((double)D) * 1.4426950408889634);
#define MSA_ATTN_CASE(GG)                                                                     \
  case GG:                                                                                    \
    sparse_attn_kernel<T, D, GG><<<grid, 256, 0, s>>>(                                        \
        (const T*)q, (const T*)k, (const T*)v, w.items, w.entries, w.totals, (T*)opart, lpart, \
        d.N, d.Nq, d.q_start, d.Hkv, d.nb, d.nb * d.nwin, d.K, scale_log2);                   \
    break;
  switch (d.G) {
    MSA_ATTN_CASE(1)
    MSA_ATTN_CASE(2)
    MSA_ATTN_CASE(4)
    MSA_ATTN_CASE(8)
    MSA_ATTN_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MSA_ATTN_CASE
  return hipGetLastError();
}

unsigned attn_pipe_grid(const Dims& d) {
  const bool one_wave = d.qt * d.G <= 32;
  return (unsigned)((((one_wave ? 2 : 1) * d.num_cus + 7) / 8) * 8);
}

template <int D>
static hipError_t attn_pipe_dispatch_g(const Dims& d, const void* q, const void* k, const void* v,
                                       const AttnWs& w, void* opart, float* lpart, hipStream_t s) {
  // persistent grid, a multiple of 8 (one share per XCD): one 8-wave workgroup
  // per CU, or two 1-wave workgroups per CU for items of at most 32/G queries
  const bool one_wave = d.qt * d.G <= 32;
  const unsigned grid = attn_pipe_grid(d);
  const float scale_log2 = (float)(1.0 / sqrt((double)D) * 1.4426950408889634);
#define MSA_PIPE_LAUNCH(GG, NW)                                                                 \
  sparse_attn_pipe_kernel<D, GG, NW><<<grid, 64 * NW, 0, s>>>(                                 \
      (const bf16*)q, (const bf16*)k, (const bf16*)v, w.items, w.entries, w.totals,            \
      w.wg_start, (bf16*)opart, lpart, d.N, d.Nq, d.q_start, d.Hkv, d.nb, d.nb * d.nwin, d.K,  \
      scale_log2,                                                                              \
      (size_t)d.slots)
#define MSA_PIPE_CASE(GG)                                                                       \
  case GG:                                                                                      \
    if (one_wave)                                                                               \
      MSA_PIPE_LAUNCH(GG, 1);                                                                   \
    else                                                                                        \
      MSA_PIPE_LAUNCH(GG, 8);                                                                   \
    break;
  switch (d.G) {
    MSA_PIPE_CASE(1)
    MSA_PIPE_CASE(2)
    MSA_PIPE_CASE(4)
    MSA_PIPE_CASE(8)
    MSA_PIPE_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MSA_PIPE_CASE
#undef MSA_PIPE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const Dims& d, const void* q, const void* k, const void* v,
                              const AttnWs& w, void* opart, float* lpart, hipStream_t s) {
  if (d.items_max == 0) return hipSuccess;
  if (d.dtype == MSA_BF16) {
    if (d.D == 128) return attn_pipe_dispatch_g<128>(d, q, k, v, w, opart, lpart, s);
    if (d.D == 64) return attn_pipe_dispatch_g<64>(d, q, k, v, w, opart, lpart, s);
  } else {
    if (d.D == 128) return attn_dispatch_g<float, 128>(d, q, k, v, w, opart, lpart, s);
    if (d.D == 64) return attn_dispatch_g<float, 64>(d, q, k, v, w, opart, lpart, s);
  }
  return hipErrorInvalidValue;
}

// ============================================================== LSE combine
//
// One wave per (query row, group). The partials of a (query, group) are
// contiguous, [slot][head in group][d], and so is the group's output row.
//  1. Lane-per-head layout (64/G lanes per head): each lane reads the slot
//     LSEs of its head, forms L = log sum_s exp(lse_s) and the merge weights
//     w_s = exp(lse_s - L), and one lane per head stores them in a per-wave
//     LDS table [head][slot].
//  2. Lane unit u = lane + 64c (8 elements) of a slot block: every load and
//     the output store move 64 consecutive units (1 KB in bf16) per
//     instruction. Slots without a block (id < 0) are skipped by a
//     wave-uniform branch, so their (never written) partials are not used.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
combine_kernel(const T* __restrict__ opart, const float* __restrict__ lpart,
               const int32_t* __restrict__ ids, T* __restrict__ out, float* __restrict__ lse,
               int64_t rows, int Hkv, int topk) {
  constexpr int UPH = D / 8;            // units per head row
  constexpr int UPS = G * UPH;          // units per slot block
  constexpr int NCH = (UPS + 63) / 64;  // units per lane
  constexpr int LPH = 64 / G;           // lanes per head in the weight phase
  constexpr int SMAX = 32;
  __shared__ float wt[4][G][SMAX + 1];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t rr = (int64_t)blockIdx.x * 4 + wave;  // (row, group), uniform
  if (rr >= rows * Hkv) return;
  const int lane = threadIdx.x & 63;
  const size_t e0 = (size_t)rr * topk;
  const int32_t* id = ids + e0;

  // 1. weights
  const int hg = lane / LPH;
  float lsv[SMAX];
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    if (s < topk) {
      lsv[s] = id[s] >= 0 ? lpart[(e0 + s) * G + hg] : -INFINITY;
      m = vmax(m, lsv[s]);
    }
  }
  float z = 0.0f;
#pragma unroll
  for (int s = 0; s < SMAX; ++s)
    if (s < topk) z += __expf(lsv[s] - m);
  const float L = m + __logf(z);
  if (lane % LPH == 0) {
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (s < topk) wt[wave][hg][s] = __expf(lsv[s] - L);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the table is written
  __builtin_amdgcn_wave_barrier();

  // 2. weighted sum of the slot blocks
  float acc[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.0f;
  const T* op = opart + e0 * (size_t)(G * D);
  bool ok[NCH];
  int hd[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int u = lane + 64 * c;
    ok[c] = UPS % 64 == 0 || u < UPS;
    hd[c] = ok[c] ? u / UPH : 0;
  }
  for (int s0 = 0; s0 < topk; s0 += 4) {
    vec8<T> o[4][NCH];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = min(s0 + j, topk - 1);  // in bounds; repeats are skipped below
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (ok[c]) {
#if MSA_NT_LOAD
          o[j][c] = ld8_nt<T>(op + (size_t)sl * (G * D) + 8 * (lane + 64 * c));
#else
          o[j][c] = ld8<T>(op + (size_t)sl * (G * D) + 8 * (lane + 64 * c));
#endif
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (s0 + j >= topk || id[s0 + j] < 0) continue;  // uniform
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!ok[c]) continue;
        const float w = wt[wave][hd[c]][s0 + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] += w * (float)o[j][c][e];
      }
    }
  }
  const int r = (int)(rr % Hkv);
  const int64_t row = rr / Hkv;
  T* dst = out + ((size_t)row * Hkv + r) * (size_t)(G * D);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (!ok[c]) continue;
    vec8<T> res;
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = cvt<T>(acc[c][e]);
    st8<T>(dst + 8 * (lane + 64 * c), res);
  }
  if (lane % LPH == 0) lse[((size_t)row * Hkv + r) * G + hg] = L;
}

// ============================================================== local block + combine (bf16)
//
// The local block floor(i/128) is the one selected block that a row sees only
// in part (causal mask), and every query of a block selects it. Its attention
// therefore runs query-outer here, inside the combine, instead of as KV-outer
// work items (the bucketing skips it): no gathered Q rows and no partial
// written and read back for it.
// Workgroup = one (128-token block L, group r): K and V of the block are
// copied to LDS once (global_load_lds, swizzled as in the KV-outer kernel) and
// serve the block's QW-query tiles (RW = QW*G (query, head) rows, 32 per
// wave). A wave owns the same 32 rows of every tile, i.e. QPW = 32/G queries
// per tile, and works through its queries in order:
//  A. at a query that opens a tile: S^T = K Q^T with the causal mask,
//     softmax, O^T = V^T P^T for the wave's 32 rows; the normalised O (bf16)
//     and its LSE go to the wave's rows of an LDS region.
//  B. per query, eq. (16)/(18): the slot LSEs (the local one from LDS) give
//     L and the weights w_s = exp(LSE_s - L), kept in a per-wave LDS table;
//     the accumulator starts with the local O (from LDS), then the non-local
//     partials stream in: lane unit u = lane + 64c (8 elements) of a slot
//     block, so every load moves 64 consecutive units.
// The partial loads form one continuous stream per wave: a query always has
// NE = SMAX stream entries (entry k is the k-th non-local slot; entries past
// the row's slots repeat its last one and are not accumulated), so entry k
// sits in ring position k % W, and the loads run W entries ahead across query
// and tile boundaries. Everything else a query needs is loaded early enough
// not to stall the stream: the next query's slot ids and LSEs during the
// current one, the next tile's Q fragments (registers) when the tile's last
// query starts. (A global_load_lds copy of Q would make the compiler hold
// every later LDS read until all vector loads land.)
// Only the K/V copy needs a workgroup barrier.

// partial entries in flight per wave, in units of 4 loads per lane: one 4 KB
// entry at G = 16, d = 128 (two measured 0.5 ms slower at the skewed 131072
// shape: more reads in flight leave the output writes waiting longer)
#ifndef MSA_CL_W4
#define MSA_CL_W4 1
#endif

template <int D, int G, int SMAX>
__global__ void __launch_bounds__(G == 1 ? 256 : 512, 1)
combine_local_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                     const bf16* __restrict__ v, const bf16* __restrict__ opart,
                     const float* __restrict__ lpart, const int32_t* __restrict__ ids,
                     bf16* __restrict__ out, float* __restrict__ lse, int N, int Nq, int q_start,
                     int Hkv, int topk, float scale_log2) {
  constexpr int QW = G == 1 ? 128 : 256 / G;  // positions per tile
  constexpr int RW = QW * G;                  // (query, head) rows per tile
  constexpr int NWV = RW / 32;                // waves
  constexpr int QPW = 32 / G;                 // queries of a wave's 32 rows
  constexpr int KSD = D / 16, DT = D / 32, CPR = D / 8;
  constexpr int TILE = 128 * D;
  constexpr int LOADS = 128 * CPR / (64 * NWV);  // global_load_lds per wave for K (and V)
  constexpr int UPH = D / 8;                     // 8-element units per head row
  constexpr int UPS = G * UPH;                   // units per slot block
  constexpr int NCH = (UPS + 63) / 64;           // units per lane
  constexpr int LPH = 64 / G;                    // lanes per head in the weight phase
  constexpr int NE = SMAX;                       // stream entries per query
  constexpr int W = MSA_CL_W4 * 4 / NCH;  // entries in flight per wave (W * NCH loads)
  static_assert(NE % W == 0 && SMAX <= 64, "ring layout");
  __shared__ __attribute__((aligned(16))) bf16 kv[2 * TILE];
  __shared__ __attribute__((aligned(16))) bf16 Ob[RW * D];  // chunk c of row rho at c ^ (rho % CPR)
  __shared__ float lse_loc[RW];
  __shared__ __attribute__((aligned(16))) float wt[NWV][SMAX * G];  // per-wave weights [slot][head]
  bf16* const Kb = kv;
  bf16* const Vb = kv + TILE;
  typedef __attribute__((address_space(3))) void lds_void;
  typedef __attribute__((address_space(3))) short4v lds_short4;

  const int b = blockIdx.z, r = blockIdx.x;
  const int L = q_start / 128 + (int)blockIdx.y;  // this workgroup's block
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = Hkv * G;
  const size_t kvrow = (size_t)Hkv * D;
  // positions of the block that are rows of this call
  const int p_lo = max(L * 128, q_start), p_hi = min(L * 128 + 128, q_start + Nq);
  const int tile_lo = (p_lo - L * 128) / QW, tile_hi = (p_hi - 1 - L * 128) / QW;

  // The wave's queries qi, in order; qi -> position apos(qi). Positions grow
  // with qi, so the rows of this call are one range [qi_lo, qi_hi].
  auto apos = [&](int qi) { return L * 128 + (qi / QPW) * QW + wave * QPW + qi % QPW; };
  int qi_lo = 1 << 30, qi_hi = -1;
  for (int qi = tile_lo * QPW; qi < (tile_hi + 1) * QPW; ++qi) {
    const int a = apos(qi);
    if (a >= p_lo && a < p_hi) {
      qi_lo = min(qi_lo, qi);
      qi_hi = qi;
    }
  }
  // Q fragments of this lane's MFMA row of a tile (rows outside the call read a
  // valid Q row and are never stored)
  auto load_q = [&](int tile, vec8<bf16>* qf) {
    const int rq = 32 * wave + l32;
    const int a = L * 128 + tile * QW + rq / G;
    const int t_row = min(max(a - q_start, 0), Nq - 1);
    const bf16* qrow = q + ((size_t)(b * (size_t)Nq + t_row) * Hq + r * G + rq % G) * D;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) qf[ks] = ld8<bf16>(qrow + 16 * ks + 8 * h);
  };
  {  // K and V of block L (rows past N read row N-1: masked)
    const int nvalid = min(128, N - L * 128);
    const size_t base = ((size_t)b * N + (size_t)L * 128) * kvrow + (size_t)r * D;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int p = (wave * LOADS + j) * 64 + lane;  // 16-byte LDS position in the tile
      const int rho = p / CPR, cs = p % CPR;
      const size_t rowbase = base + (size_t)min(rho, nvalid - 1) * kvrow;
      __builtin_amdgcn_global_load_lds((const void*)(k + rowbase + 8 * (cs ^ swz_k<D>(rho))),
                                       (lds_void*)(&Kb[(wave * LOADS + j) * 512]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(v + rowbase + 8 * (cs ^ swz_v<D>(rho))),
                                       (lds_void*)(&Vb[(wave * LOADS + j) * 512]), 16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  if (qi_hi < 0) return;  // uniform; no barrier follows

  // ---- per-query slot table (uniform values)
  auto row_e0 = [&](int qi) {  // first (query, group, slot) entry of the row
    const int t = apos(min(qi, qi_hi)) - q_start;
    return (((size_t)b * Nq + t) * Hkv + r) * (size_t)topk;
  };
  // lane s < topk holds slot s's block id
  auto load_ids = [&](int qi) {
    const size_t e0 = row_e0(qi);
    return ids[e0 + min(lane, topk - 1)];
  };
  struct Desc {
    size_t e0;
    int loc;        // slot of the local block (topk if absent)
    int nsl;        // non-local slots
    uint64_t used;  // bit s: slot s holds a block
  };
  auto make_desc = [&](int qi, int32_t idv) {
    Desc d;
    d.e0 = row_e0(qi);
    const uint64_t isloc = __ballot(lane < topk && idv == L);
    d.used = __ballot(lane < topk && idv >= 0);
    d.loc = isloc ? (int)__builtin_ctzll(isloc) : topk;
    d.nsl = d.loc < topk ? topk - 1 : topk;
    return d;
  };
  auto slot_of = [&](const Desc& d, int e) { return e + (e >= d.loc ? 1 : 0); };
  auto entry_valid = [&](const Desc& d, int e) {
    return e < d.nsl && ((d.used >> slot_of(d, e)) & 1);
  };
  // address of stream entry e (entries past the row's slots repeat the last one)
  auto entry_ptr = [&](const Desc& d, int e) {
    const int sl = d.nsl > 0 ? slot_of(d, min(e, d.nsl - 1)) : 0;
    return opart + (d.e0 + (size_t)sl) * (size_t)(G * D);
  };
  bool ok[NCH];
  int hd[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int u = lane + 64 * c;
    ok[c] = UPS % 64 == 0 || u < UPS;
    hd[c] = ok[c] ? u / UPH : 0;
  }
  const int hg = lane / LPH;
  vec8<bf16> o[W][NCH];
  auto issue = [&](int j, const Desc& d, int e) {
    const bf16* p = entry_ptr(d, e);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (ok[c]) o[j][c] = ld8_nt<bf16>(p + 8 * (lane + 64 * c));
  };
  // A row's slot LSEs ([topk][G] floats, contiguous). With G >= 4, lane l
  // holds elements 256c + 4l + j (one 16-byte load per c): slot
  // (256c + 4l) / G, head (4l + j) % G, so the lanes of one head differ in
  // the lane bits from G/4 up. Otherwise lane-per-head, one slot per value.
  constexpr bool kPack = G >= 4;
  constexpr int NCL = kPack ? (SMAX * G + 255) / 256 : SMAX;
  constexpr int NLV = kPack ? 4 : 1;
  auto load_lse = [&](size_t e0, float (*x)[NLV]) {
    if constexpr (kPack) {
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        const int f = min(256 * c + 4 * lane, topk * G - 4);
        const vec4<float> v4 = ld4<float>(lpart + e0 * G + f);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[c][j] = v4[j];
      }
    } else {
#pragma unroll
      for (int s = 0; s < SMAX; ++s) x[s][0] = lpart[(e0 + (size_t)min(s, topk - 1)) * G + hg];
    }
  };

  // ---- phase A: the local block's attention for the wave's rows of a tile
  const int rho_q = 32 * wave + l32;  // this lane's MFMA row in a tile
  const int g16 = lane >> 4, s16 = lane & 15;
  auto phase_a = [&](int tile, const vec8<bf16>* qf) {
    const int a_row = L * 128 + tile * QW + rho_q / G;
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.0f;
      const int rho = kt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
        mma(sacc[kt], ld8<bf16>(Kb + tile_off<D, false>(rho, 16 * ks + 8 * h)), qf[ks]);
    }
    // causal mask: key kt*32 + drow(e, h) of the block lies past the row when
    // its lane-free part kt*32 + drow(e, 0) exceeds thr (compile-time
    // constants against one register)
    const int thr = a_row - L * 128 - 4 * h;
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kt * 32 + drow(e, 0) > thr) sacc[kt][e] = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = vmax(vmax(mx, sacc[kt][e]), sacc[kt][e + 1]);
    }
    mx = vmax(mx, shfl_xor_f(mx, 32));
    const float mxs = mx * scale_log2;
    float ls = 0.0f;
    vec8<bf16> pf[8];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], scale_log2, -mxs));
        ls += pe;
        pf[2 * kt + e / 8][e % 8] = cvt<bf16>(pe);
      }
    }
    ls += shfl_xor_f(ls, 32);
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.0f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int krow = 16 * st + 4 * (g16 >> 1) + (s16 >> 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int dcol = dt * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4*)(Vb + tile_off<D, true>(krow, dcol)));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4*)(Vb + tile_off<D, true>(krow + 8, dcol)));
        const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
        bf16x8 vf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[e] = l4[e];
          vf[4 + e] = h4[e];
        }
        mma(oacc[dt], vf, pf[st]);
      }
    }
    const float inv = 1.0f / ls;
    const int sw = rho_q % CPR;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        vec4<bf16> ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = cvt<bf16>(oacc[dt][4 * jg + e] * inv);
        st4<bf16>(Ob + rho_q * D + 8 * ((dt * 4 + jg) ^ sw) + 4 * h, ov);
      }
    }
    lse_loc[rho_q] = (mxs + __log2f(ls)) * kLn2;  // both lane halves hold it
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): the wave's O rows are in LDS
    __builtin_amdgcn_wave_barrier();
  };

  // ---- the stream
  vec8<bf16> qf[KSD];
  load_q(qi_lo / QPW, qf);
  int32_t id_cur = load_ids(qi_lo);
  Desc dc = make_desc(qi_lo, id_cur);
  float lsv[NCL][NLV];
  load_lse(dc.e0, lsv);
#pragma unroll
  for (int j = 0; j < W; ++j) issue(j, dc, j);

  for (int qi = qi_lo; qi <= qi_hi; ++qi) {
    const int i = qi % QPW;  // query within the wave's rows of its tile
    if (i == 0 || qi == qi_lo) phase_a(qi / QPW, qf);  // uniform
    // the next query's slot ids and LSEs (clamped past the last query)
    const int32_t id_n = load_ids(qi + 1);
    float lsv_n[NCL][NLV];
    load_lse(row_e0(qi + 1), lsv_n);

    // weights: LSE = logsumexp of the slot LSEs, w_s = exp(LSE_s - LSE)
    const int orow0 = (wave * QPW + i) * G;  // the query's first row in a tile
    float Lw[NLV];
    if constexpr (kPack) {
      const int hh0 = (4 * lane) % G;  // heads hh0 .. hh0+3
      const vec4<float> lloc = ld4<float>(&lse_loc[orow0 + hh0]);
      float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        const int f = 256 * c + 4 * lane, sl = f / G;
        const int sid = __shfl(id_cur, min(sl, 63), 64);
        const bool used = f < topk * G && sid >= 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lsv[c][j] = used ? (sid == L ? lloc[j] : lsv[c][j]) : -INFINITY;
          m[j] = vmax(m[j], lsv[c][j]);
        }
      }
#pragma unroll
      for (int msk = G / 4; msk < 64; msk *= 2)
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = vmax(m[j], shfl_xor_f(m[j], msk));
      float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NCL; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] += __expf(lsv[c][j] - m[j]);
#pragma unroll
      for (int msk = G / 4; msk < 64; msk *= 2)
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] += shfl_xor_f(z[j], msk);
#pragma unroll
      for (int j = 0; j < 4; ++j) Lw[j] = m[j] + __logf(z[j]);
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        const int f = 256 * c + 4 * lane;
        if (f < SMAX * G) {
          vec4<float> w4;
#pragma unroll
          for (int j = 0; j < 4; ++j) w4[j] = __expf(lsv[c][j] - Lw[j]);
          st4<float>(&wt[wave][f], w4);
        }
      }
    } else {
      const float lloc = lse_loc[orow0 + hg];
      float m = -INFINITY;
#pragma unroll
      for (int s = 0; s < SMAX; ++s) {
        const int sid = __builtin_amdgcn_readlane(id_cur, s);
        lsv[s][0] = (s < topk && sid >= 0) ? (sid == L ? lloc : lsv[s][0]) : -INFINITY;
        m = vmax(m, lsv[s][0]);
      }
      float z = 0.0f;
#pragma unroll
      for (int s = 0; s < SMAX; ++s) z += __expf(lsv[s][0] - m);
      Lw[0] = m + __logf(z);
      if (lane % LPH == 0) {
#pragma unroll
        for (int s = 0; s < SMAX; ++s) wt[wave][s * G + hg] = __expf(lsv[s][0] - Lw[0]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the table is written
    __builtin_amdgcn_wave_barrier();

    // the accumulator starts with the local slot's share (its O from LDS)
    float acc[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[c][x] = 0.0f;
    if (dc.loc < topk) {  // uniform
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!ok[c]) continue;
        const int u = lane + 64 * c;
        const int orow = orow0 + hd[c];
        const float w = wt[wave][dc.loc * G + hd[c]];
        const vec8<bf16> ol = ld8<bf16>(Ob + orow * D + 8 * ((u % UPH) ^ (orow % CPR)));
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[c][x] = w * (float)ol[x];
      }
    }
    if (i == QPW - 1) load_q(min(qi + 1, qi_hi) / QPW, qf);  // uniform: the next tile's Q

    Desc dn;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int j = e % W;
      if (e == NE - W) dn = make_desc(qi + 1, id_n);
      if (entry_valid(dc, e)) {  // uniform
        const int sl = slot_of(dc, e);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          if (!ok[c]) continue;
          const float w = wt[wave][sl * G + hd[c]];
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[c][x] += w * (float)o[j][c][x];
        }
      }
      // refill ring position j: W entries ahead, into the next query
      if (e + W < NE)
        issue(j, dc, e + W);
      else
        issue(j, dn, e + W - NE);
    }
    const int t = apos(qi) - q_start;
    // the query's output replaces its local O rows in Ob (read for the last time
    // above); the wave writes its finished queries of the tile together (8 KB
    // bursts instead of 4 KB between the partial reads: HBM loses less to
    // turning between reads and writes), before the next tile's phase A
    // overwrites Ob
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (!ok[c]) continue;
      const int u = lane + 64 * c, orow = orow0 + hd[c];
      vec8<bf16> res;
#pragma unroll
      for (int x = 0; x < 8; ++x) res[x] = cvt<bf16>(acc[c][x]);
      st8<bf16>(Ob + orow * D + 8 * ((u % UPH) ^ (orow % CPR)), res);
    }
    if (i == QPW - 1 || qi == qi_hi) {  // uniform
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the rows are in LDS
      __builtin_amdgcn_wave_barrier();
      for (int qq = max(qi_lo, qi - i); qq <= qi; ++qq) {
        const int orq = (wave * QPW + qq % QPW) * G;
        bf16* dq = out + ((size_t)(b * (size_t)Nq + (apos(qq) - q_start)) * Hq + r * G) * D;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          if (!ok[c]) continue;
          const int u = lane + 64 * c, orow = orq + hd[c];
          st8_nt<bf16>(dq + 8 * u, ld8<bf16>(Ob + orow * D + 8 * ((u % UPH) ^ (orow % CPR))));
        }
      }
    }
    if constexpr (kPack) {  // lanes of slot 0 hold every head once
      if (4 * lane < G) {
        vec4<float> l4;
#pragma unroll
        for (int j = 0; j < 4; ++j) l4[j] = Lw[j];
        st4<float>(&lse[((size_t)b * Nq + t) * Hq + r * G + 4 * lane], l4);
      }
    } else if (lane % LPH == 0) {
      lse[((size_t)b * Nq + t) * Hq + r * G + hg] = Lw[0];
    }

    dc = dn;
    id_cur = id_n;
#pragma unroll
    for (int c = 0; c < NCL; ++c)
#pragma unroll
      for (int j = 0; j < NLV; ++j) lsv[c][j] = lsv_n[c][j];
  }
  // the ring's last W loads (the repeated last row) drain before the wave ends
}

template <int D>
static hipError_t combine_local_dispatch_g(const Dims& d, const void* q, const void* k,
                                           const void* v, const void* opart, const float* lpart,
                                           const int32_t* ids, void* out, float* lse,
                                           hipStream_t s) {
  const float scale_log2 = (float)(1.0 / sqrt((double)D) * 1.4426950408889634);
  const int nblk = (d.q_start + d.Nq - 1) / 128 - d.q_start / 128 + 1;
  // grid (group, block, batch): the groups of a block run side by side
  const dim3 grid((unsigned)d.Hkv, (unsigned)nblk, (unsigned)d.B);
#define MSA_CL_CASE(GG)                                                                        \
  case GG: {                                                                                   \
    constexpr int NT = GG == 1 ? 256 : 512;                                                    \
    if (d.K <= 16)                                                                             \
      combine_local_kernel<D, GG, 16><<<grid, NT, 0, s>>>(                                     \
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)opart, lpart, ids,      \
          (bf16*)out, lse, d.N, d.Nq, d.q_start, d.Hkv, d.K, scale_log2);                      \
    else                                                                                       \
      combine_local_kernel<D, GG, 32><<<grid, NT, 0, s>>>(                                     \
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)opart, lpart, ids,      \
          (bf16*)out, lse, d.N, d.Nq, d.q_start, d.Hkv, d.K, scale_log2);                      \
    break;                                                                                     \
  }
  switch (d.G) {
    MSA_CL_CASE(1)
    MSA_CL_CASE(2)
    MSA_CL_CASE(4)
    MSA_CL_CASE(8)
    MSA_CL_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MSA_CL_CASE
  return hipGetLastError();
}

hipError_t launch_combine_local(const Dims& d, const void* q, const void* k, const void* v,
                                const void* opart, const float* lpart, const int32_t* ids,
                                void* out, float* lse, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  if (d.dtype != MSA_BF16) return hipErrorInvalidValue;
  if (d.D == 128) return combine_local_dispatch_g<128>(d, q, k, v, opart, lpart, ids, out, lse, s);
  if (d.D == 64) return combine_local_dispatch_g<64>(d, q, k, v, opart, lpart, ids, out, lse, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t combine_dispatch_g(const Dims& d, const void* opart, const float* lpart,
                                     const int32_t* ids, void* out, float* lse, hipStream_t s) {
  const unsigned grid = (unsigned)((d.rows * d.Hkv + 3) / 4);
#define MSA_COMB_CASE(GG)                                                                   \
  case GG:                                                                                  \
    combine_kernel<T, D, GG><<<grid, 256, 0, s>>>((const T*)opart, lpart, ids, (T*)out, lse, \
                                                  d.rows, d.Hkv, d.K);                      \
    break;
  switch (d.G) {
    MSA_COMB_CASE(1)
    MSA_COMB_CASE(2)
    MSA_COMB_CASE(4)
    MSA_COMB_CASE(8)
    MSA_COMB_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MSA_COMB_CASE
  return hipGetLastError();
}

hipError_t launch_combine(const Dims& d, const void* opart, const float* lpart,
                          const int32_t* ids, void* out, float* lse, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  if (d.dtype == MSA_BF16) {
    if (d.D == 128) return combine_dispatch_g<bf16, 128>(d, opart, lpart, ids, out, lse, s);
    if (d.D == 64) return combine_dispatch_g<bf16, 64>(d, opart, lpart, ids, out, lse, s);
  } else {
    if (d.D == 128) return combine_dispatch_g<float, 128>(d, opart, lpart, ids, out, lse, s);
    if (d.D == 64) return combine_dispatch_g<float, 64>(d, opart, lpart, ids, out, lse, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
