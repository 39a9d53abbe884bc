// msa_bwd.hip — backward of the sparse attention over the selected blocks,
// and the chain of the index-logit gradient into the index projections.
//
// The selection is held fixed ("2.4 · 训练原生稀疏" (training-native sparse
// attention) eq. (12): the hard top-k has zero derivative almost everywhere),
// and every step stays on the selected support (same page: a backward that
// rebuilds the full score matrix would pay the quadratic cost again). With
// alpha the softmax weights of a (query, head) over its support, o its output
// and g = dL/do, eq. (11) gives the logit gradient dz_s = alpha_s g.(v_s - o)
// = P (dP - D) with dP = g.v_s and D = g.o; then, through z = q.k / sqrt(d),
//   dq = sum_s dz_s k_s / sqrt(d),  dk_s += dz_s q / sqrt(d),  dv_s += alpha_s g.
//
// Execution is KV-outer like the forward: the (query, slot) pairs are inverted
// into per-(batch, group, block) buckets (the counting sort of msa_attn.hip,
// local block included) and cut into items of 64 (query, head) rows (32 in
// fp32). A persistent workgroup walks a contiguous range of items; each wave
// owns one (32-key quarter of the current block, 32-row tile of the item) pair
// and keeps its keys' dK and dV in registers across the consecutive items of a
// bucket. dQ gets one partial per (query, slot), summed per row afterwards.
//
// Every sum has a fixed order, so the backward is bitwise repeatable: the
// entries of a bucket are in row order (bucket_sort_kernel), hence so are its
// items; a workgroup's run of items of one bucket writes its fp32 dK, dV sums
// (one slab per 32-row tile) to the bucket's slab when the run is the whole
// bucket, else to one of the workgroup's two slabs (its first and last run;
// only those can be shared with a neighbour); the finalize kernel adds a
// bucket's slabs in item order and writes dK, dV (zero for unselected keys).
#include "msa_internal.hpp"

namespace msa {

// D[row, h] = dO . O (fp32). D/8 consecutive lanes share a (row, head), 8
// elements each, so a wave reads whole rows; the partial sums meet by shuffles.
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_rowdot_kernel(const T* __restrict__ out, const T* __restrict__ dout, int64_t n,
                  float* __restrict__ drow) {
  constexpr int L = D / 8;
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lanes per row");
  const int64_t x = (int64_t)blockIdx.x * (256 / L) + threadIdx.x / L;
  const int c = threadIdx.x % L;
  float acc = 0.0f;
  if (x < n) {
    const vec8<T> a = ld8<T>(out + x * D + 8 * c), b = ld8<T>(dout + x * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) acc += shfl_xor_f(acc, m);
  if (x < n && c == 0) drow[x] = acc;
}

// persistent grid of the backward kernels: per_cu workgroups per CU, at most
// kBwdMaxGrid (the workspace holds two slabs per workgroup)
static int bwd_grid(const Dims& d, int per_cu = 1) {
  const int g = ((d.num_cus * per_cu + 7) / 8) * 8;
  return g < kBwdMaxGrid ? g : kBwdMaxGrid;
}
// the index backward's workgroups hold 60 KB of LDS and 185 registers per lane:
// two per CU hide each other's load latency (2.78 -> 2.10 ms at 2 x 32768)
#ifndef MSA_IDXBWD_PER_CU
#define MSA_IDXBWD_PER_CU 2
#endif

// (query, head) rows per work item: 64 for bf16; 32 for fp32, whose tiles
// also keep transposed copies in LDS
#ifndef MSA_BWD_R16
#define MSA_BWD_R16 64
#endif
#ifndef MSA_BWD_KT16
#define MSA_BWD_KT16 1
#endif
template <typename T>
constexpr int bwd_rows() {
  return sizeof(T) == 2 ? MSA_BWD_R16 : 32;
}
// one wave per (32-key quarter of the block, 32-row tile of the item)
template <typename T>
constexpr int bwd_threads() {
  return 64 * 4 * (bwd_rows<T>() / 32);
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(bwd_threads<T>(), 1)
attn_bwd_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                const T* __restrict__ dout, const float* __restrict__ lse,
                const float* __restrict__ rowdot, const int4* __restrict__ items,
                const int32_t* __restrict__ entries, const int32_t* __restrict__ totals,
                T* __restrict__ dqpart, float* __restrict__ slabs, int nbk, int N, int Nq,
                int q_start, int Hkv, int nb, int nbw, int topk, int nslots, float scale) {
  constexpr int R = bwd_rows<T>();  // (query, head) rows per item
  constexpr int RT = R / 32;        // 32-row tiles per item
  constexpr int NT = bwd_threads<T>();
  // bf16: the X^T operands (Q^T, dO^T, K^T) come from the row-major tiles
  // through the transposing LDS read; fp32 keeps transposed copies
  constexpr bool kTr = sizeof(T) == 2;
  constexpr bool kKT = !kTr || MSA_BWD_KT16;  // K^T copy in LDS for dQ
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LK = D + PAD;    // row stride of the row-major K, V, Q, dO tiles
  constexpr int LT = 128 + PAD;  // row stride of K^T [D][128] and of dS [R][128]
  constexpr int LR = R + PAD;    // row stride of Q^T, dO^T [D][R]
  constexpr int KSD = D / 16, DT = D / 32, CH = D / 8;
  __shared__ __attribute__((aligned(16))) T Ks[128 * LK];
  __shared__ __attribute__((aligned(16))) T Vs[128 * LK];
  __shared__ __attribute__((aligned(16))) T KT[kKT ? D * LT : 8];
  __shared__ __attribute__((aligned(16))) T Qs[R * LK];
  __shared__ __attribute__((aligned(16))) T dOs[R * LK];
  __shared__ __attribute__((aligned(16))) T QT[kTr ? 8 : D * LR];
  __shared__ __attribute__((aligned(16))) T dOT[kTr ? 8 : D * LR];
  __shared__ __attribute__((aligned(16))) T dSs[R * LT];
  // per-row data of the item, one array so that one address serves all four:
  // [0, R) LSE in the log2 domain, [R, 2R) D = rowsum(dO o O) (both fp32 bits),
  // [2R, 3R) position i, [3R, 4R) (query, slot) index of the row's dQ partial
  __shared__ __attribute__((aligned(16))) int rowd_s[4 * R];
  int* const lse_s = rowd_s;
  int* const d_s = rowd_s + R;
  int* const irow_s = rowd_s + 2 * R;
  int* const slot_s = rowd_s + 3 * R;

  // contiguous item range of this workgroup inside its XCD's share
  const int total = totals[1];
  const ItemSplit split(total, gridDim.x);
  int i0, i1;
  split.range(blockIdx.x, &i0, &i1);
  if (i0 >= i1) return;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = w & 3, rt = w >> 2;  // key quarter, row tile of phase 1
  const int Hq = Hkv * G;
  const size_t kvrow = (size_t)Hkv * D;
  const float sl2 = scale * kLog2e;

  // dK^T, dV^T of keys 32kw + l32 from this wave's row tile: element e is
  // d = 32dt + drow(e, h); the waves of the other row tiles hold the rest
  f32x16 dka[DT], dva[DT];
  auto zero_acc = [&]() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dka[dt][e] = 0.0f;
        dva[dt][e] = 0.0f;
      }
  };
  // the run [ra, rb) of bucket bkt ends: its sums go to the bucket's slab, or
  // to this workgroup's first- or last-run slab when a neighbour holds items
  // of the same bucket; slab layout [row tile][dK, dV][128 keys][D] fp32
  // (the buckets a neighbour may share: that of the item before the range and
  // that of the item after it)
  const int bkt_prev = __builtin_amdgcn_readfirstlane(i0 > 0 ? items[i0 - 1].x : -1);
  const int bkt_next = __builtin_amdgcn_readfirstlane(i1 < total ? items[i1].x : -1);
  auto flush = [&](int bkt, int ra, int rb) {
    const bool shared = (ra == i0 && bkt_prev == bkt) || (rb == i1 && bkt_next == bkt);
    const size_t slab = shared ? (size_t)nbk + 2 * blockIdx.x + (ra == i0 ? 0 : 1) : (size_t)bkt;
    float* const pk = slabs + ((slab * RT + rt) * 2) * 128 * D + (size_t)(32 * kw + l32) * D;
    float* const pv = pk + 128 * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dka[dt] *= scale;
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // elements 4j..4j+3: d = 32dt + 8j + 4h + 0..3
        const int dd = 32 * dt + 8 * j + 4 * h;
        *reinterpret_cast<f32x4*>(pk + dd) =
            f32x4{dka[dt][4 * j], dka[dt][4 * j + 1], dka[dt][4 * j + 2], dka[dt][4 * j + 3]};
        *reinterpret_cast<f32x4*>(pv + dd) =
            f32x4{dva[dt][4 * j], dva[dt][4 * j + 1], dva[dt][4 * j + 2], dva[dt][4 * j + 3]};
      }
    }
  };
  // two 4-element runs of a contiguous row: k-indices {16c+4h+0..3, 16c+8+4h+0..3},
  // the rows (or keys) an accumulator's elements 8c..8c+7 hold
  auto frag_rows = [&](const T* row, int c) {
    const vec4<T> lo = ld4<T>(row + 16 * c + 4 * h), hi = ld4<T>(row + 16 * c + 8 + 4 * h);
    vec8<T> a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = lo[e];
      a[4 + e] = hi[e];
    }
    return a;
  };
  // X^T fragment (d x rows) of a row-major [.][LK] tile: d tile dt, rows 16c..16c+15,
  // by the transposing LDS read (16-lane groups: output lane j gets element j of 4
  // consecutive rows), with the k-set of frag_rows (bf16 only)
  typedef __attribute__((address_space(3))) short4v lds_short4;
  const int g16 = lane >> 4, s16 = lane & 15;
  auto frag_tr = [&](const T* tile, int c, int dt) {
    const int krow = 16 * c + 4 * (g16 >> 1) + (s16 >> 2);
    const int dcol = dt * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);
    const short4v lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tile + krow * LK + dcol));
    const short4v hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tile + (krow + 8) * LK + dcol));
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
    vec8<T> a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = l4[e];
      a[4 + e] = h4[e];
    }
    return a;
  };

  // rows of an item -> registers (issued one item ahead): chunk c = tid + NT u
  // covers row c / CH, 8-element chunk c % CH
  constexpr int RU = R * CH / NT;
  static_assert(R * CH % NT == 0 && R <= NT, "row chunks");
  vec8<T> qr[RU], gr[RU];
  float lr = 0.0f, dr = 0.0f;
  int ir = -1, sr = nslots;
  // the entries of an item's rows, loaded one item ahead of the rows themselves:
  // en[u] for chunk u's row, er for row tid % R (rows past cnt: a valid row)
  int en[RU], er;
  auto load_ents = [&](int it) {
    const int4 itm = items[it];
    const int start = itm.y, cnt = itm.z;
#pragma unroll
    for (int u = 0; u < RU; ++u)
      en[u] = entries[start + min((tid + NT * u) / CH / G, cnt - 1)];
    er = entries[start + min((tid % R) / G, cnt - 1)];
  };
  // Every lane loads (lanes past R repeat a row), so no load sits under a branch
  // and the waits for them count a fixed number of later memory operations.
  auto load_rows = [&](int it) {
    const int4 itm = items[it];
    const int bkt = itm.x, cnt = itm.z;
    const int br = bkt / nbw, r = br % Hkv, b = br / Hkv;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int c = tid + NT * u;
      const int rho = c / CH, dc = c % CH;
      const int t = en[u] >> 6;
      const size_t off = ((size_t)(b * (size_t)Nq + t) * Hq + r * G + rho % G) * D + 8 * dc;
      qr[u] = ld8<T>(q + off);
      gr[u] = ld8<T>(dout + off);
    }
    const int rho = tid % R, j = rho / G, t = er >> 6;
    const size_t rr = (size_t)(b * (size_t)Nq + t) * Hq + r * G + rho % G;
    lr = lse[rr];
    dr = rowdot[rr];
    ir = j < cnt ? q_start + t : -1;  // an unused row masks every key: P = dS = 0
    // slot indices stay below 2^31 (checked by the caller); an unused row writes
    // its (zero) dQ partial to the spare slot past the last
    sr = j < cnt ? (int)((((size_t)b * Nq + t) * Hkv + r) * topk + (er & 63)) : nslots;
  };

  zero_acc();
  int cur = -1, run0 = i0;
  load_ents(i0);
  load_rows(i0);
  load_ents(min(i0 + 1, i1 - 1));
  for (int it = i0; it < i1; ++it) {
    const int bkt = items[it].x;
    const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
    __syncthreads();  // every wave is done with the previous item's tiles
    if (bkt != cur) {  // uniform
      if (cur >= 0) flush(cur, run0, it);
      zero_acc();
      cur = bkt;
      run0 = it;
      // K and V of block blk (row-major; fp32 also K^T); rows past N are zero
      for (int c = tid; c < 128 * CH; c += NT) {
        const int rho = c / CH, dc = c % CH;
        const int key = blk * 128 + rho;
        vec8<T> kk = zero8<T>(), vv = zero8<T>();
        if (key < N) {
          const size_t off = ((size_t)b * N + key) * kvrow + (size_t)r * D + 8 * dc;
          kk = ld8<T>(k + off);
          vv = ld8<T>(v + off);
        }
        st8<T>(Ks + rho * LK + 8 * dc, kk);
        st8<T>(Vs + rho * LK + 8 * dc, vv);
        if constexpr (kKT) {
#pragma unroll
          for (int e = 0; e < 8; ++e) KT[(8 * dc + e) * LT + rho] = kk[e];
        }
      }
    }
    // the item's rows (row rho = query rho / G of the item, head rho % G), prefetched
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int c = tid + NT * u;
      const int rho = c / CH, dc = c % CH;
      st8<T>(Qs + rho * LK + 8 * dc, qr[u]);
      st8<T>(dOs + rho * LK + 8 * dc, gr[u]);
      if constexpr (!kTr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          QT[(8 * dc + e) * LR + rho] = qr[u][e];
          dOT[(8 * dc + e) * LR + rho] = gr[u][e];
        }
      }
    }
    if (tid < R) {
      lse_s[tid] = __float_as_int(lr * kLog2e);
      d_s[tid] = __float_as_int(dr);
      irow_s[tid] = ir;
      slot_s[tid] = sr;
    }
    load_rows(min(it + 1, i1 - 1));  // the next item's rows land during this item
    load_ents(min(it + 2, i1 - 1));
    __syncthreads();

    // ---- phase 1: keys 32kw..32kw+31 and rows 32rt..32rt+31 of the item:
    // S = Q K^T, dP = dO V^T (rows x keys), P = exp(S - LSE) on the support,
    // dS = P (dP - D); dV^T += dO^T P, dK^T += Q^T dS
    const int key = blk * 128 + 32 * kw + l32;
    {
      f32x16 sacc, pacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[e] = 0.0f;
        pacc[e] = 0.0f;
      }
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const vec8<T> kf = ld8<T>(Ks + (32 * kw + l32) * LK + 16 * ks + 8 * h);
        const vec8<T> vf = ld8<T>(Vs + (32 * kw + l32) * LK + 16 * ks + 8 * h);
        mma(sacc, ld8<T>(Qs + (32 * rt + l32) * LK + 16 * ks + 8 * h), kf);
        mma(pacc, ld8<T>(dOs + (32 * rt + l32) * LK + 16 * ks + 8 * h), vf);
      }
      // the lane's 16 rows are 4 runs of 4 consecutive rows 8j + 4h + 0..3 (element
      // e = 4j + x is row 8j + 4h + x): their per-row data in 16-byte reads, one run
      // at a time; the exponential is unconditional and selected. P and dS go
      // straight into the operands of the dV, dK products (elements 8c..8c+7).
      vec8<T> pf[2], sf[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = 32 * rt + 8 * j + 4 * h;
        const f32x4 a = __builtin_bit_cast(f32x4, *reinterpret_cast<const i32x4*>(lse_s + r0));
        const f32x4 c = __builtin_bit_cast(f32x4, *reinterpret_cast<const i32x4*>(d_s + r0));
        const i32x4 g = *reinterpret_cast<const i32x4*>(irow_s + r0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int e = 4 * j + x;
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], sl2, -a[x]));
          const float pv = key <= g[x] ? pe : 0.0f;
          const float dv = pv * (pacc[e] - c[x]);
          dSs[(r0 + x) * LT + 32 * kw + l32] = cvt<T>(dv);
          pf[e >> 3][e & 7] = cvt<T>(pv);
          sf[e >> 3][e & 7] = cvt<T>(dv);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          if constexpr (kTr) {
            mma(dva[dt], frag_tr(dOs, 2 * rt + c, dt), pf[c]);
            mma(dka[dt], frag_tr(Qs, 2 * rt + c, dt), sf[c]);
          } else {
            mma(dva[dt], frag_rows(dOT + (32 * dt + l32) * LR + 32 * rt, c), pf[c]);
            mma(dka[dt], frag_rows(QT + (32 * dt + l32) * LR + 32 * rt, c), sf[c]);
          }
        }
      }
    }
    __syncthreads();  // dS of every wave's keys is in LDS

    // ---- phase 2: dQ = dS K (rows x d); wave w takes row tile w / DT and
    // d columns 32(w % DT)..+31
    if (RT * DT * 64 >= NT || w < RT * DT) {  // uniform
      const int dq_t = w % DT, rq = w / DT;
      {
        f32x16 qacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) qacc[e] = 0.0f;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) {
          if constexpr (!kKT)
            mma(qacc, frag_rows(dSs + (32 * rq + l32) * LT, kc), frag_tr(Ks, kc, dq_t));
          else
            mma(qacc, ld8<T>(dSs + (32 * rq + l32) * LT + 16 * kc + 8 * h),
                ld8<T>(KT + (32 * dq_t + l32) * LT + 16 * kc + 8 * h));
        }
        // into the Q tile, unused since the dK products (rows 32rq + drow(e, h))
#pragma unroll
        for (int e = 0; e < 16; ++e)
          Qs[(32 * rq + drow(e, h)) * LK + 32 * dq_t + l32] = cvt<T>(qacc[e] * scale);
      }
    }
    __syncthreads();  // the item's dQ rows are complete
    // each row's dQ goes out as the (query, slot) partial in whole-row chunks;
    // an unused row writes the spare slot past the last
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int c = tid + NT * u;
      const int rho = c / CH, dc = c % CH;
      st8<T>(dqpart + ((size_t)slot_s[rho] * G + rho % G) * D + 8 * dc,
             ld8<T>(Qs + rho * LK + 8 * dc));
    }
  }
  if (cur >= 0) flush(cur, run0, i1);
}

// dK, dV of one bucket's 128 keys (one workgroup per bucket, grid-stride): the
// sum of its slabs in item order (workgroup by workgroup, row tile by row
// tile), zero when no row selected the block. Keys past N are not written.
template <typename T, int D, int RT>
__global__ void __launch_bounds__(256)
attn_bwd_finalize_kernel(const float* __restrict__ slabs, const int32_t* __restrict__ item_off,
                         const int32_t* __restrict__ totals,
                         int nbk, int grid, int N, int Hkv, int nb, int nbw, T* __restrict__ dk,
                         T* __restrict__ dv) {
  constexpr int C4 = 128 * D / 4;  // 4-element chunks of a [128][D] slab
  const int total = totals[1];
  const ItemSplit split(total, grid);
  for (int bkt = blockIdx.x; bkt < nbk; bkt += gridDim.x) {
    const int blk = bkt % nb, br = bkt / nbw, r = br % Hkv, b = br / Hkv;
    const int ia = min(item_off[bkt], total), ib = min(item_off[bkt + 1], total);
    for (int c = threadIdx.x; c < C4; c += 256) {
      const int kl = c / (D / 4), dd = 4 * (c % (D / 4));
      const int key = blk * 128 + kl;
      if (key >= N) continue;
      f32x4 sk = {0.0f, 0.0f, 0.0f, 0.0f}, sv = {0.0f, 0.0f, 0.0f, 0.0f};
      if (ia < ib) {
        const int wa = split.owner(ia);
        int wa0, wa1;
        split.range(wa, &wa0, &wa1);
        if (ib <= wa1) {  // the whole bucket is one workgroup's run: the bucket's slab
          for (int rt = 0; rt < RT; ++rt) {
            const float* p = slabs + (((size_t)bkt * RT + rt) * 2) * 128 * D + (size_t)kl * D + dd;
            sk += *reinterpret_cast<const f32x4*>(p);
            sv += *reinterpret_cast<const f32x4*>(p + 128 * D);
          }
        } else {  // runs of consecutive workgroups, in item order
          for (int it = ia; it < ib;) {
            const int wg = split.owner(it);
            int w0, w1;
            split.range(wg, &w0, &w1);
            const size_t slab = (size_t)nbk + 2 * wg + (it == w0 ? 0 : 1);
            for (int rt = 0; rt < RT; ++rt) {
              const float* p = slabs + ((slab * RT + rt) * 2) * 128 * D + (size_t)kl * D + dd;
              sk += *reinterpret_cast<const f32x4*>(p);
              sv += *reinterpret_cast<const f32x4*>(p + 128 * D);
            }
            it = w1;
          }
        }
      }
      const size_t o = (((size_t)b * N + key) * Hkv + r) * D + dd;
      vec4<T> ok, ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ok[e] = cvt<T>(sk[e]);
        ov[e] = cvt<T>(sv[e]);
      }
      st4<T>(dk + o, ok);
      st4<T>(dv + o, ov);
    }
  }
}

// dq[row, r*G + hh] = sum over the row's used slots of the slot partials
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
dq_sum_kernel(const T* __restrict__ dqpart, const int32_t* __restrict__ ids, int64_t nrg,
              int topk, T* __restrict__ dq) {
  constexpr int CH = D / 8;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row*Hkv + r, hh, chunk)
  if (x >= nrg * G * CH) return;
  const int ch = (int)(x % CH);
  const int hh = (int)((x / CH) % G);
  const int64_t rg = x / (CH * G);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // Every slot's partial is loaded (the buffer holds all of them) and an unused
  // slot's, never written, is dropped by a select: no branch stands between the
  // loads, so they are all in flight together.
#pragma unroll 16
  for (int s = 0; s < topk; ++s) {
    const bool used = ids[rg * topk + s] >= 0;
    const vec8<T> a = ld8_nt<T>(dqpart + ((rg * topk + s) * G + hh) * D + 8 * ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += used ? (float)a[e] : 0.0f;
  }
  vec8<T> res;
#pragma unroll
  for (int e = 0; e < 8; ++e) res[e] = cvt<T>(acc[e]);
  st8<T>(dq + (rg * G + hh) * D + 8 * ch, res);
}


template <typename T>
__global__ void __launch_bounds__(256)
f32_to_kernel(const float* __restrict__ src, int64_t n, T* __restrict__ dst) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * 256)
    dst[x] = cvt<T>(src[x]);
}

// ============================================================== index chain
//
// dlogits = P_idx - P in the index logits (the KL pass), on the selected
// support; S_idx = q_idx . k_idx / sqrt(d_idx) with one k_idx head shared by
// every group (indexer note §2.1), so
//   dq_idx[i, r] = c/sqrt(d_idx) sum_j dl[i, r, j] k_idx[j],
//   dk_idx[j]    = c/sqrt(d_idx) sum over (i, r) that selected j of dl[i, r, j] q_idx[i, r],
// c = the caller's loss coefficient. Same buckets as the attention (items of up
// to 32 queries of one (batch, group, block), entries in row order); a
// persistent workgroup (4 waves) keeps the block's dk_idx in registers across
// the bucket's items (wave w: keys 32w..32w+31) and writes it to a slab at the
// end of each run, as the attention backward does; the finalize kernel adds,
// per key, the buckets of every group in group order (each bucket's slabs in
// item order). dq_idx gets one fp32 partial per (query, slot), summed per row
// afterwards. Products use fp32 matrix cores (dlogits are fp32).
template <typename T, int DI>
__global__ void __launch_bounds__(256, 1)
idx_bwd_kernel(const T* __restrict__ qi, const T* __restrict__ ki, const float* __restrict__ dl,
               const int4* __restrict__ items, const int32_t* __restrict__ entries,
               const int32_t* __restrict__ totals, float* __restrict__ dqpart,
               float* __restrict__ slabs, int nbk, int N, int Nq, int Hkv, int nb, int nbw,
               int topk, int nslots, float coef) {
  constexpr int Q = 32;         // queries per item
  constexpr int LKT = 128 + 4;  // row stride of K_idx^T [DI][128] and of dl [Q][128]
  constexpr int LQ = Q + 4;     // row stride of Q_idx^T [DI][Q]
  constexpr int DIT = DI / 32;
  __shared__ __attribute__((aligned(16))) float KIT[DI * LKT];
  __shared__ __attribute__((aligned(16))) float DLs[Q * LKT];
  __shared__ __attribute__((aligned(16))) float QIT[DI * LQ];
  __shared__ __attribute__((aligned(16))) int slot_s[Q];  // (query, slot) of each query's partial

  const int total = totals[1];
  const ItemSplit split(total, gridDim.x);
  int i0, i1;
  split.range(blockIdx.x, &i0, &i1);
  if (i0 >= i1) return;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x16 dka[DIT];  // dk_idx^T: d rows 32dt + drow(e, h), key column 32w + l32
  auto zero_acc = [&]() {
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dka[dt][e] = 0.0f;
  };
  // the run [ra, rb) of bucket bkt ends: [128 keys][DI] fp32 slab, chosen as in
  // the attention backward. The buckets a neighbour may share (those of the items
  // just outside the range) are read once here: with the test written inline in
  // the item loop, the compiled flush inside the loop dropped the comparison of
  // the previous item's bucket and sent the first run of a range that opens a
  // bucket to the shared slab, leaving the bucket's own slab unwritten.
  const int bkt_prev = __builtin_amdgcn_readfirstlane(i0 > 0 ? items[i0 - 1].x : -1);
  const int bkt_next = __builtin_amdgcn_readfirstlane(i1 < total ? items[i1].x : -1);
  auto flush = [&](int bkt, int ra, int rb) {
    const bool shared = (ra == i0 && bkt_prev == bkt) || (rb == i1 && bkt_next == bkt);
    const size_t slab = shared ? (size_t)nbk + 2 * blockIdx.x + (ra == i0 ? 0 : 1) : (size_t)bkt;
    float* const row = slabs + (slab * 128 + 32 * w + l32) * DI;
#pragma unroll
    for (int dt = 0; dt < DIT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)  // elements 4j..4j+3: d = 32dt + 8j + 4h + 0..3
        *reinterpret_cast<f32x4*>(row + 32 * dt + 8 * j + 4 * h) =
            f32x4{dka[dt][4 * j] * coef, dka[dt][4 * j + 1] * coef, dka[dt][4 * j + 2] * coef,
                  dka[dt][4 * j + 3] * coef};
  };

  // the item's dl rows (4 floats per chunk) and Q_idx rows, loaded one item
  // ahead; the entries that address them one item earlier still. Every lane
  // loads (rows past cnt repeat a valid row), so no load sits under a branch.
  constexpr int DU = Q * 128 / 4 / 256;  // dl chunks per thread
  constexpr int QU = (Q * DI + 255) / 256;  // Q_idx values per thread
  vec4<float> dlr[DU];
  float qir[QU];
  int edl[DU], eqi[QU], es;
  int sr = nslots;
  auto load_ents = [&](int it) {
    const int4 itm = items[it];
    const int start = itm.y, cnt = itm.z;
#pragma unroll
    for (int u = 0; u < DU; ++u) edl[u] = entries[start + min((tid + 256 * u) / 32, cnt - 1)];
#pragma unroll
    for (int u = 0; u < QU; ++u)
      eqi[u] = entries[start + min(min(tid + 256 * u, Q * DI - 1) / DI, cnt - 1)];
    es = entries[start + min(tid % Q, cnt - 1)];
  };
  auto load_rows = [&](int it) {
    const int4 itm = items[it];
    const int bkt = itm.x, cnt = itm.z;
    const int br = bkt / nbw, r = br % Hkv, b = br / Hkv;
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int o4 = (tid + 256 * u) % 32, ent = edl[u];  // rows past cnt: zeroed when stored
      dlr[u] = ld4<float>(dl + (((size_t)b * Nq + (ent >> 6)) * Hkv + r) * topk * 128 +
                          (ent & 63) * 128 + 4 * o4);
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int dd = min(tid + 256 * u, Q * DI - 1) % DI;
      qir[u] = (float)qi[(((size_t)b * Nq + (eqi[u] >> 6)) * Hkv + r) * DI + dd];
    }
    // slot indices stay below 2^31 (checked by the caller); a query past cnt
    // writes its (zero) partial to the spare slot past the last
    sr = tid % Q < cnt ? (int)((((size_t)b * Nq + (es >> 6)) * Hkv + r) * topk + (es & 63))
                       : nslots;
  };

  zero_acc();
  int cur = -1, run0 = i0;
  load_ents(i0);
  load_rows(i0);
  load_ents(min(i0 + 1, i1 - 1));
  for (int it = i0; it < i1; ++it) {
    const int4 itm = items[it];
    const int bkt = itm.x, cnt = itm.z;
    const int blk = bkt % nb, b = bkt / nbw / Hkv;
    __syncthreads();
    if (bkt != cur) {  // uniform
      if (cur >= 0) flush(cur, run0, it);
      zero_acc();
      cur = bkt;
      run0 = it;
      for (int c = tid; c < 128 * DI; c += 256) {  // K_idx^T of the block, keys past N zero
        const int key = c / DI, dd = c % DI;
        const int kk = blk * 128 + key;
        KIT[dd * LKT + key] = kk < N ? (float)ki[((size_t)b * N + kk) * DI + dd] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < DU; ++u) {  // dl rows (zero past cnt)
      const int c = tid + 256 * u;
      const int j = c / 32, o4 = c % 32;
      vec4<float> val = dlr[u];
      if (j >= cnt) val = vec4<float>{0.0f, 0.0f, 0.0f, 0.0f};
      st4<float>(DLs + j * LKT + 4 * o4, val);
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {  // Q_idx^T of the item's queries (zero past cnt)
      const int c = tid + 256 * u;
      if (Q * DI % 256 == 0 || c < Q * DI) {  // no branch when the chunks fill every thread
        const int j = c / DI, dd = c % DI;
        QIT[dd * LQ + j] = j < cnt ? qir[u] : 0.0f;
      }
    }
    if (tid < Q) slot_s[tid] = sr;
    load_rows(min(it + 1, i1 - 1));  // the next item's rows land during this item
    load_ents(min(it + 2, i1 - 1));
    __syncthreads();
    // dq_idx partial of the item's queries: dl (Q x 128) K_idx (128 x DI); wave w < DIT
    if (w < DIT) {  // uniform
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        mma(acc, ld8<float>(DLs + l32 * LKT + 16 * kc + 8 * h),
            ld8<float>(KIT + (32 * w + l32) * LKT + 16 * kc + 8 * h));
      // the lane's queries 8jj + 4h + 0..3: their slots in 16-byte reads
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const i32x4 sl = *reinterpret_cast<const i32x4*>(slot_s + 8 * jj + 4 * h);
#pragma unroll
        for (int x = 0; x < 4; ++x)
          dqpart[(size_t)sl[x] * DI + 32 * w + l32] = acc[4 * jj + x] * coef;
      }
    }
    // dk_idx^T of keys 32w..: Q_idx^T (DI x Q) dl (Q x keys); the B fragment is 8
    // queries of the lane's key column, read from the row-major dl tile (consecutive
    // lanes, consecutive keys: no bank conflicts)
#pragma unroll
    for (int kc = 0; kc < Q / 16; ++kc) {
      vec8<float> bcol;
#pragma unroll
      for (int e = 0; e < 8; ++e) bcol[e] = DLs[(16 * kc + 8 * h + e) * LKT + 32 * w + l32];
#pragma unroll
      for (int dt = 0; dt < DIT; ++dt)
        mma(dka[dt], ld8<float>(QIT + (32 * dt + l32) * LQ + 16 * kc + 8 * h), bcol);
    }
  }
  if (cur >= 0) flush(cur, run0, i1);
}

// dk_idx of one (batch, block)'s 128 keys (one workgroup each, grid-stride):
// the groups' buckets in group order, each the sum of its slabs in item order;
// zero when no row of any group selected the block. Keys past N are not written.
template <typename T, int DI>
__global__ void __launch_bounds__(256)
idx_bwd_finalize_kernel(const float* __restrict__ slabs, const int32_t* __restrict__ item_off,
                        const int32_t* __restrict__ totals, int nbk, int grid, int B, int N,
                        int Hkv, int nb, int nbw, T* __restrict__ dk) {
  constexpr int C4 = 128 * DI / 4;
  const int total = totals[1];
  const ItemSplit split(total, grid);
  for (int bb = blockIdx.x; bb < B * nb; bb += gridDim.x) {
    const int b = bb / nb, blk = bb % nb;
    for (int c = threadIdx.x; c < C4; c += 256) {
      const int kl = c / (DI / 4), dd = 4 * (c % (DI / 4));
      const int key = blk * 128 + kl;
      if (key >= N) continue;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int r = 0; r < Hkv; ++r) {
        const int bkt = (b * Hkv + r) * nbw + blk;
        const int ia = min(item_off[bkt], total), ib = min(item_off[bkt + 1], total);
        if (ia >= ib) continue;
        const int wa = split.owner(ia);
        int wa0, wa1;
        split.range(wa, &wa0, &wa1);
        f32x4 sb = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ib <= wa1) {
          sb = *reinterpret_cast<const f32x4*>(slabs + ((size_t)bkt * 128 + kl) * DI + dd);
        } else {
          for (int it = ia; it < ib;) {
            const int wg = split.owner(it);
            int w0, w1;
            split.range(wg, &w0, &w1);
            const size_t slab = (size_t)nbk + 2 * wg + (it == w0 ? 0 : 1);
            sb += *reinterpret_cast<const f32x4*>(slabs + (slab * 128 + kl) * DI + dd);
            it = w1;
          }
        }
        acc += sb;
      }
      vec4<T> o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = cvt<T>(acc[e]);
      st4<T>(dk + ((size_t)b * N + key) * DI + dd, o);
    }
  }
}

// dq_idx[row, r] = sum over the row's used slots of the slot partials; a thread
// sums 4 consecutive elements, loading every slot and dropping unused ones
// (never written) by a select, so that the loads are all in flight together
template <typename T, int DI>
__global__ void __launch_bounds__(256)
dqi_sum_kernel(const float* __restrict__ dqpart, const int32_t* __restrict__ ids, int64_t nrg,
               int topk, T* __restrict__ dq) {
  constexpr int C4 = DI / 4;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row*Hkv + r, 4-element chunk)
  if (x >= nrg * C4) return;
  const int64_t rg = x / C4;
  const int cc = (int)(x % C4);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
  for (int s = 0; s < topk; ++s) {
    const bool used = ids[rg * topk + s] >= 0;
    const float4 a = *reinterpret_cast<const float4*>(dqpart + (rg * topk + s) * DI + 4 * cc);
    acc.x += used ? a.x : 0.0f;
    acc.y += used ? a.y : 0.0f;
    acc.z += used ? a.z : 0.0f;
    acc.w += used ? a.w : 0.0f;
  }
  T* o = dq + rg * DI + 4 * cc;
  o[0] = cvt<T>(acc.x);
  o[1] = cvt<T>(acc.y);
  o[2] = cvt<T>(acc.z);
  o[3] = cvt<T>(acc.w);
}

template <typename T, int DI>
static hipError_t idx_bwd_run(const Dims& d, const void* qi, const void* ki, const int32_t* ids,
                              const float* dl, float coef, const AttnWs& w, float* dqpart,
                              float* slabs, void* dq, void* dk, hipStream_t s) {
  hipError_t e;
  const int grid = bwd_grid(d, MSA_IDXBWD_PER_CU);
  const float c = coef / sqrtf((float)DI);
  const int nbk = (int)d.buckets, nbw = d.nb * d.nwin;
  prof_before(MSA_K_IDX_BWD, s);
  idx_bwd_kernel<T, DI><<<grid, 256, 0, s>>>((const T*)qi, (const T*)ki, dl, w.items, w.sorted,
                                             w.totals, dqpart, slabs, nbk, d.N, d.Nq, d.Hkv,
                                             d.nb, nbw, d.K, (int)d.slots, c);
  prof_after(MSA_K_IDX_BWD, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nrg = d.rows * d.Hkv;
  dqi_sum_kernel<T, DI><<<(unsigned)((nrg * (DI / 4) + 255) / 256), 256, 0, s>>>(
      dqpart, ids, nrg, d.K, (T*)dq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nbb = (int64_t)d.B * d.nb;
  if (nbb > 0) {
    prof_before(MSA_K_BWD_FINALIZE, s);
    idx_bwd_finalize_kernel<T, DI><<<(unsigned)std::min<int64_t>(nbb, 4096), 256, 0, s>>>(
        slabs, w.item_off, w.totals, nbk, grid, d.B, d.N, d.Hkv, d.nb, nbw, (T*)dk);
    prof_after(MSA_K_BWD_FINALIZE, s);
  }
  return hipGetLastError();
}

hipError_t launch_idx_bwd(const Dims& d, const void* qi, const void* ki, const int32_t* ids,
                          const float* dl, float coef, const AttnWs& w, float* dqpart,
                          float* slabs, void* dq, void* dk, hipStream_t s) {
  if (d.nwin != 1 || !w.sorted) return hipErrorInvalidValue;  // one bucket per (b, group, block)
  if (d.dtype == MSA_BF16) {
    if (d.DI == 64) return idx_bwd_run<bf16, 64>(d, qi, ki, ids, dl, coef, w, dqpart, slabs, dq, dk, s);
    if (d.DI == 32) return idx_bwd_run<bf16, 32>(d, qi, ki, ids, dl, coef, w, dqpart, slabs, dq, dk, s);
  } else {
    if (d.DI == 64) return idx_bwd_run<float, 64>(d, qi, ki, ids, dl, coef, w, dqpart, slabs, dq, dk, s);
    if (d.DI == 32) return idx_bwd_run<float, 32>(d, qi, ki, ids, dl, coef, w, dqpart, slabs, dq, dk, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t bwd_run(const Dims& d, const void* q, const void* k, const void* v,
                          const int32_t* ids, const void* out, const float* lse,
                          const void* dout, const AttnWs& w,
                          float* drow, void* dqpart, float* slabs, void* dq,
                          void* dk, void* dv, hipStream_t s) {
  hipError_t e;
  const int64_t nrh = d.rows * d.Hq;
  bwd_rowdot_kernel<T, D><<<(unsigned)((nrh + 256 / (D / 8) - 1) / (256 / (D / 8))), 256, 0, s>>>(
      (const T*)out, (const T*)dout, nrh, drow);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int grid = bwd_grid(d);
  const float scale = (float)(1.0 / sqrt((double)D));
  const int64_t nrg = d.rows * d.Hkv;
  const unsigned sgrid = (unsigned)((nrg * d.G * (D / 8) + 255) / 256);
  const int nbk = (int)d.buckets, nbw = d.nb * d.nwin;
#define MSA_BWD_CASE(GG)                                                                        \
  case GG:                                                                                      \
    prof_before(MSA_K_ATTN_BWD, s);                                                             \
    attn_bwd_kernel<T, D, GG><<<grid, bwd_threads<T>(), 0, s>>>(                                \
        (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse, drow, w.items, w.sorted,    \
        w.totals, (T*)dqpart, slabs, nbk, d.N, d.Nq, d.q_start, d.Hkv, d.nb, nbw, d.K,          \
        (int)d.slots, scale);                                                                   \
    prof_after(MSA_K_ATTN_BWD, s);                                                              \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                        \
    if (nrg > 0)                                                                                \
      dq_sum_kernel<T, D, GG><<<sgrid, 256, 0, s>>>((const T*)dqpart, ids, nrg, d.K,         \
                                                    (T*)dq);                                    \
    break;
  switch (d.G) {
    MSA_BWD_CASE(1)
    MSA_BWD_CASE(2)
    MSA_BWD_CASE(4)
    MSA_BWD_CASE(8)
    MSA_BWD_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MSA_BWD_CASE
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nbk > 0) {
    prof_before(MSA_K_BWD_FINALIZE, s);
    attn_bwd_finalize_kernel<T, D, bwd_rows<T>() / 32>
        <<<(unsigned)std::min(nbk, 4096), 256, 0, s>>>(slabs, w.item_off, w.totals,
                                                       nbk, grid, d.N, d.Hkv, d.nb, nbw,
                                                       (T*)dk, (T*)dv);
    prof_after(MSA_K_BWD_FINALIZE, s);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const Dims& d, const void* q, const void* k, const void* v,
                           const int32_t* ids, const void* out, const float* lse,
                           const void* dout, const AttnWs& w,
                           float* drow, void* dqpart, float* slabs, void* dq,
                           void* dk, void* dv, hipStream_t s) {
  if (d.nwin != 1 || !w.sorted) return hipErrorInvalidValue;  // one bucket per (b, group, block)
  if (d.dtype == MSA_BF16) {
    if (d.D == 128)
      return bwd_run<bf16, 128>(d, q, k, v, ids, out, lse, dout, w, drow, dqpart, slabs, dq, dk,
                                dv, s);
    if (d.D == 64)
      return bwd_run<bf16, 64>(d, q, k, v, ids, out, lse, dout, w, drow, dqpart, slabs, dq, dk,
                               dv, s);
  } else if (d.D == 64) {
    return bwd_run<float, 64>(d, q, k, v, ids, out, lse, dout, w, drow, dqpart, slabs, dq, dk,
                              dv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
