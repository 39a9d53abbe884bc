// msa_kl.hip — KL alignment of the index branch on the selected support.
//
// "MSA 中的 KL 对齐与局部知识蒸馏" (MSA KL alignment note):
//   §2.1 student P_idx = softmax of the index logits over the support J;
//   §2.2 teacher P = (1/G) sum over the group's heads of each head's softmax
//        over J (probabilities averaged, not logits);
//   §3   KL(P || P_idx) per (query, group), loss = mean over N*Hkv rows,
//        gradient in the index logits = P_idx - P;
//   §6   probabilities are rebuilt from logits and the two LSEs
//        (p = exp(s - LSE), also "4.1.1 · 监督与联合训练" eq. 15), LSE_main
//        coming from the sparse forward; the work per KV tile is uneven, which
//        the shared KV-outer work list (fixed-size items of hot buckets) absorbs.
// Passes, all over the attention work items (one 128-token block of group r,
// up to 128/G query rows):
//   A  index logits on the block -> per-(query, slot) log-sum-exp;
//   B  logsumexp over slots -> LSE_idx per (query, group); zero dS rows of
//      unused slots;
//   C  main logits of the G heads (MFMA) -> teacher P; index logits -> P_idx;
//      dS = P_idx - P per token, KL partial per (query, slot);
//   D  KL per row (fixed slot order) and the mean (fixed-order tree).
#include "msa_internal.hpp"

namespace msa {

template <typename T> struct KlPad;
template <> struct KlPad<bf16> { static constexpr int K = 8; };
template <> struct KlPad<float> { static constexpr int K = 4; };

// Index logits S_idx^T = K_idx_blk Q_idx^T for the item's queries. Wave w
// owns keys [32w, 32w+32); column tile ct holds queries 32ct..32ct+31.
// Writes z = S_idx (natural scale, fp32) to zs[q][key] in LDS.
template <typename T, int DI, int QT>
__device__ __forceinline__ void item_index_logits(const T* __restrict__ q_idx,
                                                  const T* __restrict__ k_idx, int b, int r,
                                                  int blk, int N, int Nq, int Hkv, int cnt,
                                                  const int* s_t, float (*zs)[128 + 4],
                                                  float scale) {
  constexpr int KS = DI / 16;
  constexpr int CT = (QT + 31) / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int j = blk * 128 + 32 * wave + l32;
  vec8<T> af[KS];
  const T* kp = k_idx + ((size_t)b * N + j) * DI + 8 * h;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) af[ks] = j < N ? ld8<T>(kp + 16 * ks) : zero8<T>();
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int qi = ct * 32 + l32;
    const bool qv = qi < cnt;
    const int t = qv ? s_t[qi] : 0;
    const T* qp = q_idx + ((size_t)(b * (size_t)Nq + t) * Hkv + r) * DI + 8 * h;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) mma(acc, af[ks], qv ? ld8<T>(qp + 16 * ks) : zero8<T>());
    if (qi < QT) {
#pragma unroll
      for (int e = 0; e < 16; ++e) zs[qi][32 * wave + drow(e, h)] = acc[e] * scale;
    }
  }
}

// ---------------------------------------------------------------- pass A
template <typename T, int DI, int QT>
__global__ void __launch_bounds__(256)
kl_idx_stats_kernel(const T* __restrict__ q_idx, const T* __restrict__ k_idx,
                    const int4* __restrict__ items, const int32_t* __restrict__ entries,
                    const int32_t* __restrict__ totals, float* __restrict__ slot_lse, int N,
                    int Nq, int q_start, int Hkv, int nb, int nbw, int topk) {
  __shared__ float zs[QT][128 + 4];
  __shared__ int s_t[QT], s_s[QT];
  const int total = totals[1];
  const int per = (total + 7) / 8;
  const int g = blockIdx.x;
  const int it = (g & 7) * per + (g >> 3);
  if ((g >> 3) >= per || it >= total) return;
  const int4 item = items[it];
  const int bkt = item.x, start = item.y, cnt = item.z;
  const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
  const int tid = threadIdx.x;
  if (tid < QT) {
    const int e = tid < cnt ? entries[start + tid] : 0;
    s_t[tid] = e >> 6;
    s_s[tid] = e & 63;
  }
  __syncthreads();
  item_index_logits<T, DI, QT>(q_idx, k_idx, b, r, blk, N, Nq, Hkv, cnt, s_t, zs,
                               1.0f / sqrtf((float)DI));
  __syncthreads();
  // one thread per query: logsumexp over the visible tokens of the block
  if (tid < cnt) {
    const int i = q_start + s_t[tid];
    const int last = min(127, i - blk * 128);
    float m = -INFINITY;
    for (int key = 0; key <= last; ++key) m = fmaxf(m, zs[tid][key]);
    float z = 0.0f;
    for (int key = 0; key <= last; ++key) z += __expf(zs[tid][key] - m);
    const size_t entry = ((size_t)(b * (size_t)Nq + s_t[tid]) * Hkv + r) * topk + s_s[tid];
    slot_lse[entry] = m + __logf(z);
  }
}

// ---------------------------------------------------------------- pass B
__global__ void __launch_bounds__(256)
kl_idx_lse_kernel(const int32_t* __restrict__ ids, const float* __restrict__ slot_lse,
                  float* __restrict__ lse_idx, float* __restrict__ dlogits, int64_t nrows,
                  int topk) {
  const int64_t rr = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, group)
  if (rr >= nrows) return;
  const int32_t* id = ids + rr * topk;
  float m = -INFINITY;
  for (int s = 0; s < topk; ++s)
    if (id[s] >= 0) m = fmaxf(m, slot_lse[rr * topk + s]);
  float z = 0.0f;
  for (int s = 0; s < topk; ++s)
    if (id[s] >= 0) z += __expf(slot_lse[rr * topk + s] - m);
  lse_idx[rr] = m + __logf(z);
  if (dlogits) {
    for (int s = 0; s < topk; ++s) {
      if (id[s] >= 0) continue;
      float4* p = reinterpret_cast<float4*>(dlogits + (rr * topk + s) * 128);
      for (int x = 0; x < 32; ++x) p[x] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ---------------------------------------------------------------- pass C
//
// S = Q K^T with the wave's 32 (query, head) rows as GEMM rows: A = Q
// fragments (registers), B = K block from LDS. Lane element e holds row
// drow(e, h), key column l32 of tile kt. The G heads of one query sit in RPQ
// consecutive elements of a lane (plus the other lane half when G >= 8), so
// the teacher's head average is an in-lane sum (+ one exchange).
template <typename T, int D, int DI, int G>
__global__ void __launch_bounds__(256, 2)
kl_main_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ q_idx,
               const T* __restrict__ k_idx, const float* __restrict__ lse_main,
               const float* __restrict__ lse_idx, const int4* __restrict__ items,
               const int32_t* __restrict__ entries, const int32_t* __restrict__ totals,
               float* __restrict__ kl_part, float* __restrict__ dlogits, int N, int Nq,
               int q_start, int Hkv, int nb, int nbw, int topk, float scale_log2) {
  constexpr int QT = 128 / G;
  constexpr int KSD = D / 16;
  constexpr int PK = KlPad<T>::K;
  constexpr bool PARTNER = G >= 8;
  constexpr int RPQ = PARTNER ? G / 2 : G;  // rows of one query per lane
  constexpr int NLQ = 16 / RPQ;             // queries per lane
  __shared__ T Ks[128][D + PK];
  __shared__ float zs[QT][128 + 4];
  __shared__ int s_t[QT], s_s[QT];
  __shared__ float s_li[QT];

  const int total = totals[1];
  const int per = (total + 7) / 8;
  const int g = blockIdx.x;
  const int it = (g & 7) * per + (g >> 3);
  if ((g >> 3) >= per || it >= total) return;
  const int4 item = items[it];
  const int bkt = item.x, start = item.y, cnt = item.z;
  const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
  const int tid = threadIdx.x;
  if (tid < QT) {
    const int e = tid < cnt ? entries[start + tid] : 0;
    const int t = e >> 6;
    s_t[tid] = t;
    s_s[tid] = e & 63;
    s_li[tid] = tid < cnt ? lse_idx[(size_t)(b * (size_t)Nq + t) * Hkv + r] : 0.0f;
  }
  const size_t kvrow = (size_t)Hkv * D;
  const T* kb = k + ((size_t)b * N + (size_t)blk * 128) * kvrow + (size_t)r * D;
  const int nvalid = min(128, N - blk * 128);
  constexpr int CH = D / 8;
  for (int c = tid; c < 128 * CH; c += 256) {
    const int kr = c / CH, dc = c % CH;
    st8<T>(&Ks[kr][dc * 8], kr < nvalid ? ld8<T>(kb + kr * kvrow + dc * 8) : zero8<T>());
  }
  __syncthreads();
  item_index_logits<T, DI, QT>(q_idx, k_idx, b, r, blk, N, Nq, Hkv, cnt, s_t, zs,
                               1.0f / sqrtf((float)DI));
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int Hq = Hkv * G;
  // A operand: this lane's Q row (wave row l32) for the MFMA rows
  const int arow = 32 * wave + l32;
  const int aqi = arow / G;
  const bool av = aqi < cnt;
  const int at = av ? s_t[aqi] : 0;
  vec8<T> qf[KSD];
  {
    const T* qp = q + ((size_t)(b * (size_t)Nq + at) * Hq + r * G + arow % G) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) qf[ks] = av ? ld8<T>(qp + 16 * ks) : zero8<T>();
  }
  // per-element (row) data: LSE_main of the row's head in the log2 domain
  float lm2[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = 32 * wave + drow(e, h);
    const int qi = row / G;
    lm2[e] = qi < cnt
                 ? lse_main[(size_t)(b * (size_t)Nq + s_t[qi]) * Hq + r * G + row % G] * kLog2e
                 : 0.0f;
  }
  // per query of this lane: position, log2 LSE_idx, gradient row base; all in
  // the log2 domain (raw v_exp_f32 / v_log_f32, scales folded into FMAs)
  int q_i[NLQ];
  float li2[NLQ];
  float* dbase[NLQ];
  bool qown[NLQ];
#pragma unroll
  for (int lq = 0; lq < NLQ; ++lq) {
    const int row = 32 * wave + drow(lq * RPQ, h);
    const int qi = row / G;
    qown[lq] = qi < cnt && (!PARTNER || h == 0);
    const int qc = qi < cnt ? qi : 0;
    const int t = s_t[qc];
    q_i[lq] = q_start + t;
    li2[lq] = s_li[qc] * kLog2e;
    const size_t entry = ((size_t)(b * (size_t)Nq + t) * Hkv + r) * topk + s_s[qc];
    dbase[lq] = dlogits ? dlogits + entry * 128 : nullptr;
  }
  float klacc[NLQ];
#pragma unroll
  for (int lq = 0; lq < NLQ; ++lq) klacc[lq] = 0.0f;
  const float inv_g = 1.0f / (float)G;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
      mma(acc, qf[ks], ld8<T>(&Ks[kt * 32 + l32][16 * ks + 8 * h]));
    const int key = kt * 32 + l32;
    const int tok = blk * 128 + key;
#pragma unroll
    for (int lq = 0; lq < NLQ; ++lq) {
      // teacher: mean over the group's heads of exp(S - LSE_main)
      float P = 0.0f;
#pragma unroll
      for (int e = lq * RPQ; e < (lq + 1) * RPQ; ++e)
        P += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e], scale_log2, -lm2[e]));
      if (PARTNER) P += shfl_xor_f(P, 32);
      P *= inv_g;
      const int qi = (32 * wave + drow(lq * RPQ, h)) / G;
      const float lpi2 = __builtin_fmaf(zs[qi < cnt ? qi : 0][key], kLog2e, -li2[lq]);  // log2 P_idx
      const bool vis = tok <= q_i[lq];
      const float dS = vis ? __builtin_amdgcn_exp2f(lpi2) - P : 0.0f;
      // P below the smallest normal float adds nothing to P log P (and v_log_f32
      // may treat it as 0)
      const float kt_term =
          (vis && P >= 1.17549435e-38f) ? P * (__builtin_amdgcn_logf(P) - lpi2) : 0.0f;
      if (qown[lq]) {
        klacc[lq] += kt_term;
        if (dlogits) dbase[lq][key] = dS;
      }
    }
  }
  // reduce the KL partial of each query over the 32 key columns of a lane half
#pragma unroll
  for (int lq = 0; lq < NLQ; ++lq) {
    float v = klacc[lq] * kLn2;  // log2 -> natural log
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
    const int row = 32 * wave + drow(lq * RPQ, h);
    const int qi = row / G;
    if (l32 == 0 && qown[lq]) {
      const size_t entry = ((size_t)(b * (size_t)Nq + s_t[qi]) * Hkv + r) * topk + s_s[qi];
      kl_part[entry] = v;
    }
  }
}

// ---------------------------------------------------------------- pass C, bf16, G >= 8
//
// Persistent: one workgroup of 8 waves per CU over a contiguous range of its
// XCD's items (as the KV-outer attention kernel); an item is 256 (query,
// head) rows = 256/G queries of one block, 32 rows per wave.
//  - K and K_idx of the block are copied to LDS (global_load_lds, swizzled)
//    only when the next item needs another block.
//  - Q rows are loaded row-contiguously one item ahead and turned into MFMA A
//    fragments through a per-wave LDS region.
//  - Index logits of the item's queries: waves 0-3 form 32 keys x the item's
//    queries each (MFMA) into a double-buffered LDS table; one workgroup
//    barrier per item.
//  - S = Q K^T, keys in lanes: the teacher is the mean over the group's heads
//    of exp(S - LSE_main), an in-lane sum plus one exchange of lane halves;
//    student, KL and dS in the log2 domain; dS rows are streamed out.
constexpr int kKlWaves = 8;

template <int D, int DI, int G, bool DL>
__global__ void __launch_bounds__(512, 1)
kl_main_pipe_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                    const bf16* __restrict__ q_idx, const bf16* __restrict__ k_idx,
                    const float* __restrict__ lse_main, const float* __restrict__ lse_idx,
                    const int4* __restrict__ items, const int32_t* __restrict__ entries,
                    const int32_t* __restrict__ totals, float* __restrict__ kl_part,
                    float* __restrict__ dlogits, int N, int Nq, int q_start, int Hkv, int nb,
                    int nbw, int topk, int nslots, float scale_log2, float zscale_log2) {
  static_assert(G >= 8, "two lane halves per query");
  constexpr int QT = 256 / G;            // queries per item
  constexpr int KSD = D / 16, KSI = DI / 16;
  constexpr int CPR = D / 8, CPI = DI / 8;
  constexpr int TILE = 128 * D, ITILE = 128 * DI;
  constexpr int LOADS = 128 * CPR / (64 * kKlWaves);
  constexpr int ILOADS = 128 * CPI / (64 * kKlWaves);
  constexpr int LDW = D + 8;
  constexpr int RCH = 32 * CPR / 64;     // Q row chunks per lane per wave tile
  constexpr int RPI = 64 / CPR;          // rows per 1 KB access
  static_assert(G >= RPI, "rows of one access belong to one query");
  constexpr int QPW = 32 / G;            // queries per wave
  constexpr int RPQ = G / 2;             // rows of one query per lane
  constexpr int NLQ = 16 / RPQ;          // queries per lane (= QPW)
  __shared__ bf16 Kb[TILE];
  __shared__ bf16 KIb[ITILE];
  __shared__ bf16 Wst[kKlWaves][32 * LDW];
  __shared__ float zs[2][QT][128 + 4];
  typedef __attribute__((address_space(3))) void lds_void;

  const int total = totals[1];
  const int nwg_x = gridDim.x / 8;
  const int x = blockIdx.x & 7, gx = blockIdx.x >> 3;
  const int per_x = (total + 7) / 8;
  const int x0 = x * per_x, x1 = min(total, x0 + per_x);
  const int per_wg = (per_x + nwg_x - 1) / nwg_x;
  const int i0 = x0 + gx * per_wg, i1 = min(x1, i0 + per_wg);
  if (i0 >= i1) return;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t kvrow = (size_t)Hkv * D;
  bf16* const W = Wst[wave];
  const int qw0 = wave * QPW;  // first query of the wave in an item
  const int ent_last = max(0, totals[0] - 1);

  auto stage = [&](int bkt) {
    const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
    const int nvalid = min(128, N - blk * 128);
    const size_t base = ((size_t)b * N + (size_t)blk * 128) * kvrow + (size_t)r * D;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int p = (wave * LOADS + j) * 64 + lane;
      const int rho = p / CPR, cs = p % CPR;
      const size_t src = base + (size_t)min(rho, nvalid - 1) * kvrow + 8 * (cs ^ swz_k<D>(rho));
      __builtin_amdgcn_global_load_lds((const void*)(k + src),
                                       (lds_void*)(&Kb[(wave * LOADS + j) * 512]), 16, 0, 0);
    }
    const size_t ibase = ((size_t)b * N + (size_t)blk * 128) * DI;
#pragma unroll
    for (int j = 0; j < ILOADS; ++j) {
      const int p = (wave * ILOADS + j) * 64 + lane;
      const int rho = p / CPI, cs = p % CPI;
      const size_t src = ibase + (size_t)min(rho, nvalid - 1) * DI + 8 * (cs ^ swz_k<DI>(rho));
      __builtin_amdgcn_global_load_lds((const void*)(k_idx + src),
                                       (lds_void*)(&KIb[(wave * ILOADS + j) * 512]), 16, 0, 0);
    }
  };
  auto wave_entries = [&](const int4& itm, int* es) {
#pragma unroll
    for (int j = 0; j < QPW; ++j) es[j] = entries[min(itm.y + qw0 + j, ent_last)];
  };
  // index-logit operand of an item: lane l32 < QT takes query l32 (others
  // repeat query 0); every wave loads it, so no load sits under a branch
  auto z_entry = [&](const int4& itm) {
    const int qi = l32 < QT ? l32 : 0;
    return entries[min(itm.y + min(qi, itm.z - 1), ent_last)];
  };
  auto load_qz = [&](const int4& itm, int ez, vec8<bf16>* qz) {
    const int br = itm.x / nbw, r = br % Hkv, b = br / Hkv;
    const bf16* qp = q_idx + (((size_t)b * Nq + (ez >> 6)) * Hkv + r) * DI + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) qz[ks] = ld8<bf16>(qp + 16 * ks);
  };
  // Q rows of the wave's queries (row-contiguous) and LSE_main of its rows
  auto load_rows = [&](int bkt, const int* es, vec8<bf16>* raw, float* lm2) {
    const int br = bkt / nbw, r = br % Hkv, b = br / Hkv;
#pragma unroll
    for (int u = 0; u < RCH; ++u) {
      const int j = (RPI * u) / G, hd = (RPI * u) % G;
      const bf16* base = q + (((size_t)b * Nq + (es[j] >> 6)) * Hkv + r) * (size_t)(G * D) + hd * D;
      raw[u] = ld8<bf16>(base + (lane / CPR) * D + 8 * (lane % CPR));
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = drow(e, h);  // row within the wave
      const int j = row / G;
      lm2[e] = lse_main[(((size_t)b * Nq + (es[j] >> 6)) * Hkv + r) * G + row % G] * kLog2e;
    }
  };
  auto rows_to_frags = [&](const vec8<bf16>* raw, vec8<bf16>* qf) {
#pragma unroll
    for (int u = 0; u < RCH; ++u) {
      const int c = lane + 64 * u;
      st8<bf16>(W + (c / CPR) * LDW + 8 * (c % CPR), raw[u]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) qf[ks] = ld8<bf16>(W + l32 * LDW + 16 * ks + 8 * h);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  };

  int4 cur = items[i0];
  stage(cur.x);
  int es[QPW];
  wave_entries(cur, es);
  vec8<bf16> qf[KSD];
  float lm2[16];
  {
    vec8<bf16> raw[RCH];
    load_rows(cur.x, es, raw, lm2);
    rows_to_frags(raw, qf);
  }
  int4 nxt = items[min(i0 + 1, i1 - 1)];
  int es_n[QPW];
  wave_entries(nxt, es_n);
  int ez_n = z_entry(nxt);
  vec8<bf16> qz[KSI];
  load_qz(cur, z_entry(cur), qz);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const float inv_g = 1.0f / (float)G;
  for (int it = i0; it < i1; ++it) {
    const int bkt = cur.x, cnt = cur.z;
    const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
    const int buf = (it - i0) & 1;
    const bool have_next = it + 1 < i1;
    const int4 nxt2 = items[min(it + 2, i1 - 1)];
    // q_idx operand of the next item (its entry was loaded one item earlier)
    vec8<bf16> qz_n[KSI];
    load_qz(nxt, ez_n, qz_n);
    int es_n2[QPW];
    wave_entries(nxt2, es_n2);
    const int ez_n2 = z_entry(nxt2);
    vec8<bf16> qraw[RCH];
    float lm2_n[16];
    load_rows(nxt.x, es_n, qraw, lm2_n);

    // ---- S = Q K^T
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
        mma(sacc[kt], qf[ks], ld8<bf16>(Kb + tile_off<D, false>(kt * 32 + l32, 16 * ks + 8 * h)));
    }
    // ---- index logits of the item's queries (waves 0-3: keys 32w..32w+31)
    if (wave < 4) {
      f32x16 zacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) zacc[i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks)
        mma(zacc, ld8<bf16>(KIb + tile_off<DI, false>(32 * wave + l32, 16 * ks + 8 * h)), qz[ks]);
      if (l32 < QT) {
#pragma unroll
        for (int i = 0; i < 16; ++i) zs[buf][l32][32 * wave + drow(i, h)] = zacc[i] * zscale_log2;
      }
    }
    // per query of the lane: position, log2 LSE_idx, KL slot and gradient row.
    // Both lane halves hold the same values and store them to the same
    // addresses; a query past cnt writes to the spare slot and row past the
    // last slot. No store sits under a branch, so the waits for the loads
    // issued before them can count them.
    int q_i[NLQ];
    float li2[NLQ];
    int kslot[NLQ];
    float* dptr[NLQ];
#pragma unroll
    for (int lq = 0; lq < NLQ; ++lq) {
      const int t = es[lq] >> 6;
      const bool qv = qw0 + lq < cnt;
      q_i[lq] = q_start + t;
      const size_t rg = ((size_t)b * Nq + t) * Hkv + r;
      li2[lq] = lse_idx[rg] * kLog2e;
      kslot[lq] = qv ? (int)(rg * topk + (es[lq] & 63)) : nslots;
      dptr[lq] = DL ? (qv ? dlogits + (size_t)kslot[lq] * 128 : kl_part + nslots + 1) : nullptr;
    }
    __syncthreads();  // the index-logit table of this item is complete
    float klacc[NLQ];
#pragma unroll
    for (int lq = 0; lq < NLQ; ++lq) klacc[lq] = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = kt * 32 + l32;
      const int tok = blk * 128 + key;
#pragma unroll
      for (int lq = 0; lq < NLQ; ++lq) {
        float P = 0.0f;
#pragma unroll
        for (int e = lq * RPQ; e < (lq + 1) * RPQ; ++e)
          P += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], scale_log2, -lm2[e]));
        P += shfl_xor_f(P, 32);
        P *= inv_g;
        const float lpi2 = zs[buf][qw0 + lq][key] - li2[lq];  // log2 P_idx
        const bool vis = tok <= q_i[lq];
        const float dS = vis ? __builtin_amdgcn_exp2f(lpi2) - P : 0.0f;
        const float term =
            (vis && P >= 1.17549435e-38f) ? P * (__builtin_amdgcn_logf(P) - lpi2) : 0.0f;
        klacc[lq] += term;
        if constexpr (DL) __builtin_nontemporal_store(dS, dptr[lq] + key);
      }
    }
#pragma unroll
    for (int lq = 0; lq < NLQ; ++lq) {
      float v = klacc[lq] * kLn2;
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
      kl_part[kslot[lq]] = v;
    }
    // ---- next item's Q fragments
    rows_to_frags(qraw, qf);
    if (have_next && nxt.x != bkt) {
      __syncthreads();
      stage(nxt.x);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    cur = nxt;
    nxt = nxt2;
    ez_n = ez_n2;
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) qz[ks] = qz_n[ks];
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      es[j] = es_n[j];
      es_n[j] = es_n2[j];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) lm2[e] = lm2_n[e];
  }
}

// ---------------------------------------------------------------- pass D
__global__ void __launch_bounds__(256)
kl_reduce_kernel(const int32_t* __restrict__ ids, const float* __restrict__ kl_part,
                 float* __restrict__ kl_rows, float* __restrict__ block_sums, int64_t nrows,
                 int topk) {
  __shared__ float red[256];
  const int64_t rr = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float v = 0.0f;
  if (rr < nrows) {
    const int32_t* id = ids + rr * topk;
    for (int s = 0; s < topk; ++s)
      if (id[s] >= 0) v += kl_part[rr * topk + s];
    kl_rows[rr] = v;
  }
  red[threadIdx.x] = v;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) block_sums[blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(256)
kl_mean_kernel(const float* __restrict__ block_sums, int64_t nblocks, int64_t nrows,
               float* __restrict__ kl_mean) {
  __shared__ double red[256];
  double v = 0.0;
  for (int64_t x = threadIdx.x; x < nblocks; x += 256) v += (double)block_sums[x];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *kl_mean = nrows > 0 ? (float)(red[0] / (double)nrows) : 0.0f;
}

// ---------------------------------------------------------------- launch

template <typename T, int D, int DI, int G>
static hipError_t kl_run(const Dims& d, const void* q, const void* k, const void* q_idx,
                         const void* k_idx, const int32_t* ids, const float* lse_main,
                         const AttnWs& w, float* slot_lse, float* lse_idx, float* kl_part,
                         float* kl_rows, float* block_sums, float* kl_mean, float* dlogits,
                         hipStream_t s) {
  const unsigned grid = (unsigned)(d.items_max + 8);
  const int64_t nrows = d.rows * d.Hkv;
  // bf16 with G >= 8: 256-row items and the persistent main pass
  constexpr bool kPipe = sizeof(T) == 2 && G >= 8;
  constexpr int QT = kPipe ? 256 / G : 128 / G;
  if (d.items_max > 0) {
    prof_before(MSA_K_KL_IDX_STATS, s);
    kl_idx_stats_kernel<T, DI, QT><<<grid, 256, 0, s>>>(
        (const T*)q_idx, (const T*)k_idx, w.items, w.entries, w.totals, slot_lse, d.N, d.Nq,
        d.q_start, d.Hkv, d.nb, d.nb * d.nwin, d.K);
    prof_after(MSA_K_KL_IDX_STATS, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned rgrid = (unsigned)((nrows + 255) / 256);
  if (nrows > 0) {
    prof_before(MSA_K_KL_IDX_LSE, s);
    kl_idx_lse_kernel<<<rgrid, 256, 0, s>>>(ids, slot_lse, lse_idx, dlogits, nrows, d.K);
    prof_after(MSA_K_KL_IDX_LSE, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (d.items_max > 0) {
    const float scale_log2 = (float)(1.0 / sqrt((double)D) * 1.4426950408889634);
    prof_before(MSA_K_KL_MAIN, s);
    if constexpr (kPipe) {
      // one workgroup per CU, a multiple of 8 (one share per XCD)
      const unsigned pgrid = (unsigned)(((d.num_cus + 7) / 8) * 8);
      const float zscale_log2 = (float)(1.0 / sqrt((double)DI) * 1.4426950408889634);
      // kl_part holds one spare slot and one spare 128-float gradient row past
      // the last slot (targets of the stores of queries past an item's count)
      if (dlogits)
        kl_main_pipe_kernel<D, DI, G, true><<<pgrid, 64 * kKlWaves, 0, s>>>(
            (const bf16*)q, (const bf16*)k, (const bf16*)q_idx, (const bf16*)k_idx, lse_main,
            lse_idx, w.items, w.entries, w.totals, kl_part, dlogits, d.N, d.Nq, d.q_start,
            d.Hkv, d.nb, d.nb * d.nwin, d.K, (int)d.slots, scale_log2, zscale_log2);
      else
        kl_main_pipe_kernel<D, DI, G, false><<<pgrid, 64 * kKlWaves, 0, s>>>(
            (const bf16*)q, (const bf16*)k, (const bf16*)q_idx, (const bf16*)k_idx, lse_main,
            lse_idx, w.items, w.entries, w.totals, kl_part, dlogits, d.N, d.Nq, d.q_start,
            d.Hkv, d.nb, d.nb * d.nwin, d.K, (int)d.slots, scale_log2, zscale_log2);
    } else {
      kl_main_kernel<T, D, DI, G><<<grid, 256, 0, s>>>(
          (const T*)q, (const T*)k, (const T*)q_idx, (const T*)k_idx, lse_main, lse_idx,
          w.items, w.entries, w.totals, kl_part, dlogits, d.N, d.Nq, d.q_start, d.Hkv, d.nb,
          d.nb * d.nwin, d.K, scale_log2);
    }
    prof_after(MSA_K_KL_MAIN, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nrows > 0) {
    prof_before(MSA_K_KL_REDUCE, s);
    kl_reduce_kernel<<<rgrid, 256, 0, s>>>(ids, kl_part, kl_rows, block_sums, nrows, d.K);
    prof_after(MSA_K_KL_REDUCE, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  kl_mean_kernel<<<1, 256, 0, s>>>(block_sums, nrows > 0 ? (int64_t)rgrid : 0, nrows, kl_mean);
  return hipGetLastError();
}

template <typename T, int D, int DI>
static hipError_t kl_dispatch_g(const Dims& d, const void* q, const void* k, const void* qi,
                                const void* ki, const int32_t* ids, const float* lm,
                                const AttnWs& w, float* sl, float* li, float* kp, float* kr,
                                float* bs, float* km, float* dl, hipStream_t s) {
  switch (d.G) {
    case 1: return kl_run<T, D, DI, 1>(d, q, k, qi, ki, ids, lm, w, sl, li, kp, kr, bs, km, dl, s);
    case 2: return kl_run<T, D, DI, 2>(d, q, k, qi, ki, ids, lm, w, sl, li, kp, kr, bs, km, dl, s);
    case 4: return kl_run<T, D, DI, 4>(d, q, k, qi, ki, ids, lm, w, sl, li, kp, kr, bs, km, dl, s);
    case 8: return kl_run<T, D, DI, 8>(d, q, k, qi, ki, ids, lm, w, sl, li, kp, kr, bs, km, dl, s);
    case 16: return kl_run<T, D, DI, 16>(d, q, k, qi, ki, ids, lm, w, sl, li, kp, kr, bs, km, dl, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t kl_dispatch_di(const Dims& d, const void* q, const void* k, const void* qi,
                                 const void* ki, const int32_t* ids, const float* lm,
                                 const AttnWs& w, float* sl, float* li, float* kp, float* kr,
                                 float* bs, float* km, float* dl, hipStream_t s) {
  if (d.DI == 64) return kl_dispatch_g<T, D, 64>(d, q, k, qi, ki, ids, lm, w, sl, li, kp, kr, bs, km, dl, s);
  if (d.DI == 32) return kl_dispatch_g<T, D, 32>(d, q, k, qi, ki, ids, lm, w, sl, li, kp, kr, bs, km, dl, s);
  return hipErrorInvalidValue;
}

hipError_t launch_kl(const Dims& d, const void* q, const void* k, const void* q_idx,
                     const void* k_idx, const int32_t* ids, const float* lse_main,
                     const AttnWs& w, float* slot_lse, float* lse_idx, float* kl_part,
                     float* kl_rows, float* block_sums, float* kl_mean, float* dlogits,
                     hipStream_t s) {
  if (d.dtype == MSA_BF16) {
    if (d.D == 128) return kl_dispatch_di<bf16, 128>(d, q, k, q_idx, k_idx, ids, lse_main, w, slot_lse, lse_idx, kl_part, kl_rows, block_sums, kl_mean, dlogits, s);
    if (d.D == 64) return kl_dispatch_di<bf16, 64>(d, q, k, q_idx, k_idx, ids, lse_main, w, slot_lse, lse_idx, kl_part, kl_rows, block_sums, kl_mean, dlogits, s);
  } else {
    if (d.D == 128) return kl_dispatch_di<float, 128>(d, q, k, q_idx, k_idx, ids, lse_main, w, slot_lse, lse_idx, kl_part, kl_rows, block_sums, kl_mean, dlogits, s);
    if (d.D == 64) return kl_dispatch_di<float, 64>(d, q, k, q_idx, k_idx, ids, lse_main, w, slot_lse, lse_idx, kl_part, kl_rows, block_sums, kl_mean, dlogits, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
