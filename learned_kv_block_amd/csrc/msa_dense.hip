// msa_dense.hip — the warm-up stage of the index branch on the full causal context.
//
// "MSA 中的 KL 对齐与局部知识蒸馏" (MSA KL alignment note):
//   §5  before Top-k routing is switched on, the main branch attends to the
//       whole causal history and the KL support J is the full causal context;
//   §6  each branch only has to provide its log-sum-exp: probabilities are
//       rebuilt as p = exp(s - LSE) ("4.1.1 · 监督与联合训练" eq. 15);
//   §8  block recall (how many of the teacher's best blocks the selection
//       holds) and score recall (the teacher mass the selected blocks cover;
//       "4.1.1 · 监督与联合训练" eq. 2 and eq. 3).
// Nothing here is O(k): every kernel streams the causal history 128 keys at a
// time and keeps the N x N score matrix in registers.
//
//   dense_lse_kernel  causal LSE of either branch, query-outer: keys through a
//                     double-buffered LDS tile, online (max, sum) per row;
//   kl_dense_kernel   KL(P || P_idx) per (query, group) on the full causal
//                     context, and the teacher's mass per 128-token block;
//   recall_kernel     block recall and score recall of a selection against
//                     the teacher's block masses;
//   mean_kernel       fixed-order mean of a vector (one workgroup).
#include <type_traits>

#include "msa_dense.hpp"

namespace msa {

// Task order of the query-outer kernels: task = (tile rank u, pair) with the
// pairs (b, y) innermost — y the KV group, or 0 for the index branch — and the
// tiles from the longest (latest queries, most key blocks) to the shortest.
// The hardware hands workgroups to the 8 XCDs round robin, so when the number
// of pairs divides 8 (or 8 divides it) each XCD keeps the same pairs, and the
// workgroups resident on an XCD at one time are tiles of nearly the same
// length that started together: they stream the same key head in lockstep and
// share its blocks in L2 (a balanced zig-zag order with contiguous per-XCD
// ranges measured 27% slower for the same work). Longest first also leaves
// the short tiles to fill the end of the launch.
struct Task {
  int b, y, tile;
};

// row stride (elements) of the bf16 dS rows of the gradient chain: N rounded
// up to 8, so that every row starts 16-byte aligned
__host__ __device__ __forceinline__ int ds_stride(int N) { return (N + 7) & ~7; }
__device__ __forceinline__ bool task_of(int ntasks, int ntiles, int ngroups, Task* t) {
  const int g = blockIdx.x;
  if (g >= ntasks) return false;
  const int npairs = ntasks / ntiles;
  const int u = g / npairs, pair = g - u * npairs;
  t->tile = ntiles - 1 - u;
  t->b = pair / ngroups;
  t->y = pair - t->b * ngroups;
  return true;
}
static unsigned task_grid(int ntasks) { return (unsigned)ntasks; }

// One 128-key tile of a key head ([128][DK], row j0 + r at base + (j0 + r) * stride)
// moved global -> registers -> swizzled LDS by the NT threads of a workgroup.
// Rows at or past N repeat row N - 1; such keys are after every query and masked.
// Chunk c of row r sits at c ^ (idx_swz(r) & (CPR - 1)): with 16 chunks per row
// (a row is one 256-byte bank row), the 16 rows one LDS cycle serves land in 16
// distinct 4-bank groups (a 3-bit swizzle would pair them: 2-way conflicts).
template <typename T, int DK, int NT>
struct KeyStage {
  static constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  static constexpr int CPR = DK / EPC;        // chunks per row
  static constexpr int SWM = CPR - 1;
  static_assert(CPR <= 16, "swizzle of up to 16 chunks");
  static constexpr int CH = 128 * CPR / NT;   // chunks per thread
  static_assert((128 * CPR) % NT == 0, "tile shape");
  i32x4 raw[CH];
  __device__ __forceinline__ void load(const T* base, size_t stride, int j0, int N, int tid) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int x = tid + NT * u, r = x / CPR, c = x % CPR;
      const int j = min(j0 + r, N - 1);
      raw[u] = *reinterpret_cast<const i32x4*>(base + (size_t)j * stride + c * EPC);
    }
  }
  __device__ __forceinline__ void store(i32x4* dst, int tid) const {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int x = tid + NT * u, r = x / CPR, c = x % CPR;
      dst[r * CPR + (c ^ (idx_swz(r) & SWM))] = raw[u];
    }
  }
};

// MFMA fragment (8 elements) of row r of a
// KeyStage tile: chunk c0 (and c0 + 1 for fp32) of the row
template <typename T, int CPR>
__device__ __forceinline__ vec8<T> key_frag(const i32x4* tile, int r, int c0) {
  const i32x4* row = tile + r * CPR;
  const int s = idx_swz(r) & (CPR - 1);
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(vec8<T>, row[c0 ^ s]);
  } else {
    const i32x4 lo = row[c0 ^ s], hi = row[(c0 + 1) ^ s];
    f32x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = __int_as_float(lo[e]);
      v[4 + e] = __int_as_float(hi[e]);
    }
    return v;
  }
}

// ============================================================== causal LSE
//
// LSE[b, t, y*R + u] = log sum_{j <= i} exp(q[b, t, y*R + u] . key_y[j] / sqrt(D)),
// i = q_start + t. Main branch: R = G query heads of group y read KV head y.
// Index branch: R = Hkv index heads, y = 0, all reading the one K_idx head.
// Workgroup = RT = 64*NW consecutive rows (QT = RT/R queries) of one pair;
// wave w owns rows [64w, 64w+64) as two 32-column MFMA B tiles held in
// registers. The product is formed transposed (32 keys as rows), so each lane
// holds 16 keys of one row and the online max / sum stay in the lane; the two
// lane halves are merged once at the end. All exponentials are base 2 with
// the scale folded into one FMA.
template <typename T, int D, int R, int NW>
__global__ void __launch_bounds__(64 * NW)
dense_lse_kernel(const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ lse,
                 int N, int Nq, int q_start, int qrows, int kstride, int ngroups, int ntiles,
                 int ntasks, float scale_log2) {
  constexpr int NT = 64 * NW, RT = 64 * NW, QT = RT / R, KS = D / 16;
  using Stage = KeyStage<T, D, NT>;
  constexpr int CPR = Stage::CPR, EPC = Stage::EPC;
  static_assert(RT % R == 0, "rows of a query stay in one tile");
  __shared__ i32x4 kbuf[2][128 * CPR];

  Task tk;
  if (!task_of(ntasks, ntiles, ngroups, &tk)) return;
  const int b = tk.b, y = tk.y, t0 = tk.tile * QT;
  const int t_last = min(Nq, t0 + QT) - 1;
  const int kb_last = (q_start + t_last) >> 7;
  // first block holding a key after the tile's first query
  const int kb_mask = min((q_start + t0 + 1) >> 7, kb_last + 1);
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const T* kbase = k + (size_t)b * N * kstride + (size_t)y * D;

  Stage st;
  st.load(kbase, kstride, 0, N, tid);
  vec8<T> qf[2][KS];
  int i_row[2];
  size_t orow[2];
  bool ovalid[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int rho = 64 * wave + 32 * ct + l32;
    const int tq = t0 + rho / R, u = rho % R;
    const int tc = min(tq, Nq - 1);
    orow[ct] = ((size_t)b * Nq + tc) * qrows + (size_t)y * R + u;
    ovalid[ct] = tq < Nq;
    i_row[ct] = q_start + tc;
    const T* qp = q + orow[ct] * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ct][ks] = ld8<T>(qp + 16 * ks);
  }
  st.store(kbuf[0], tid);
  if (kb_last >= 1) st.load(kbase, kstride, 128, N, tid);
  __syncthreads();

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
  auto key_tile = [&](auto masked, const i32x4* tile, int kb, int kt) {
    vec8<T> af[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) af[ks] = key_frag<T, CPR>(tile, 32 * kt + l32, (16 * ks + 8 * h) / EPC);
    f32x16 acc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ct][e] = 0.0f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) mma(acc[ct], af[ks], qf[ct][ks]);
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 128 + 32 * kt + drow(e, h) > i_row[ct]) acc[ct][e] = -INFINITY;
      }
      float mt = vmax(acc[ct][0], acc[ct][1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2) mt = vmax(vmax(mt, acc[ct][e]), acc[ct][e + 1]);
      const float mn = vmax(m[ct], mt * scale_log2);
      const float mref = mn == -INFINITY ? 0.0f : mn;
      float s = l[ct] * __builtin_amdgcn_exp2f(m[ct] - mref);
#pragma unroll
      for (int e = 0; e < 16; ++e) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[ct][e], scale_log2, -mref));
      l[ct] = s;
      m[ct] = mn;
    }
  };
  auto block = [&](auto masked, int kb) {
    const int cur = kb & 1;
    if (kb + 1 <= kb_last) {
      st.store(kbuf[cur ^ 1], tid);  // last read before the previous barrier
      if (kb + 2 <= kb_last) st.load(kbase, kstride, (kb + 2) * 128, N, tid);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) key_tile(masked, kbuf[cur], kb, kt);
    __syncthreads();
  };
  int kb = 0;
  for (; kb < kb_mask; ++kb) block(std::false_type(), kb);
  for (; kb <= kb_last; ++kb) block(std::true_type(), kb);

#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float mo = shfl_xor_f(m[ct], 32), lo = shfl_xor_f(l[ct], 32);
    const float M = vmax(m[ct], mo);
    const float Mr = M == -INFINITY ? 0.0f : M;
    const float L = l[ct] * __builtin_amdgcn_exp2f(m[ct] - Mr) + lo * __builtin_amdgcn_exp2f(mo - Mr);
    if (h == 0 && ovalid[ct]) lse[orow[ct]] = (Mr + __builtin_amdgcn_logf(L)) * kLn2;
  }
}

// ============================================================== KL on the full causal context
//
// Per (query, group) row, with J = {j <= i}:
//   P_j     = (1/G) sum over the group's heads of exp(S_h,j - LSE_main,h)
//   log P_idx_j = z_j - LSE_idx,   z_j = q_idx . k_idx_j / sqrt(d_idx)
//   KL      = sum_j P_j (log P_j - log P_idx_j)         (terms with P_j = 0 vanish)
//   mass_b  = sum over the keys of block b of P_j
// Workgroup = RT = 32*NW rows (QT = RT/G queries x the G heads of group y) of
// one pair; the product S = Q K^T has the wave's 32 rows as MFMA rows (Q in
// registers) and 32 keys in the lanes, so the G heads of a query sit in G
// elements of a lane (G/2 plus the other lane half for G >= 8) and the teacher
// average is an in-lane sum plus at most one exchange. For G >= 8 the two lane
// halves then split the queries, so the per-(query, key) work is not repeated.
// The index logits use the same layout: the query's q_idx row is repeated on
// each of its head rows and multiplied by the K_idx tile.
template <typename T, int D, int DI, int G, int NW>
__global__ void __launch_bounds__(64 * NW)
kl_dense_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ q_idx,
                const T* __restrict__ k_idx, const float* __restrict__ lse_main,
                const float* __restrict__ lse_idx, float* __restrict__ kl_rows,
                float* __restrict__ mass, bf16* __restrict__ ds, int N, int Nq, int q_start,
                int t_begin, int t_end, int Hkv, int nb, int ntiles, int ntasks, float sc2,
                float zc2) {
  constexpr int NT = 64 * NW, RT = 32 * NW, QT = RT / G, KS = D / 16, KSI = DI / 16;
  constexpr bool PARTNER = G >= 8;
  constexpr int RPQ = PARTNER ? G / 2 : G;  // rows of one query per lane
  constexpr int NLQ = 16 / RPQ;             // queries per lane (before the split)
  constexpr int OWN = PARTNER ? NLQ / 2 : NLQ;
  constexpr int QPW = 32 / G;               // queries per wave
  using SK = KeyStage<T, D, NT>;
  using SI = KeyStage<T, DI, NT>;
  __shared__ i32x4 kbuf[2][128 * SK::CPR];
  __shared__ i32x4 ibuf[2][128 * SI::CPR];

  Task tk;
  if (!task_of(ntasks, ntiles, Hkv, &tk)) return;
  const int b = tk.b, r = tk.y, t0 = t_begin + tk.tile * QT;
  const int t_last = min(t_end, t0 + QT) - 1;
  const int kb_last = (q_start + t_last) >> 7;
  const int kb_mask = min((q_start + t0 + 1) >> 7, kb_last + 1);
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = Hkv * G;
  const size_t kstride = (size_t)Hkv * D;
  const T* kbase = k + (size_t)b * N * kstride + (size_t)r * D;
  const T* ibase = k_idx + (size_t)b * N * DI;

  SK sk;
  SI si;
  sk.load(kbase, kstride, 0, N, tid);
  si.load(ibase, DI, 0, N, tid);
  // A fragments: MFMA row l32 = wave row 32w + l32 = (query, head)
  vec8<T> qf[KS], qif[KSI];
  {
    const int rho = 32 * wave + l32;
    const int tc = min(t0 + rho / G, t_end - 1);
    const T* qp = q + (((size_t)b * Nq + tc) * Hq + (size_t)r * G + rho % G) * D + 8 * h;
    const T* qip = q_idx + (((size_t)b * Nq + tc) * Hkv + r) * DI + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = ld8<T>(qp + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) qif[ks] = ld8<T>(qip + 16 * ks);
  }
  // LSE_main (log2 domain) of the row of each accumulator element
  float lm2[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int rho = 32 * wave + drow(e, h);
    const int tc = min(t0 + rho / G, t_end - 1);
    lm2[e] = lse_main[((size_t)b * Nq + tc) * Hq + (size_t)r * G + rho % G] * kLog2e;
  }
  // the lane's own queries
  int i_q[OWN];
  float li2[OWN];
  size_t grow[OWN], dsr[OWN];
  bool qv[OWN];
#pragma unroll
  for (int m = 0; m < OWN; ++m) {
    const int wq = PARTNER ? 2 * m + h : drow(m * RPQ, h) / G;  // query within the wave
    const int tq = t0 + wave * QPW + wq;
    const int tc = min(tq, t_end - 1);
    qv[m] = tq < t_end;
    i_q[m] = q_start + tc;
    grow[m] = ((size_t)b * Nq + tc) * Hkv + r;
    li2[m] = lse_idx[grow[m]] * kLog2e;
    dsr[m] = (((size_t)b * (t_end - t_begin) + (tc - t_begin)) * Hkv + r) * (size_t)ds_stride(N);
  }
  sk.store(kbuf[0], tid);
  si.store(ibuf[0], tid);
  if (kb_last >= 1) {
    sk.load(kbase, kstride, 128, N, tid);
    si.load(ibase, DI, 128, N, tid);
  }
  __syncthreads();

  const float inv_g = 1.0f / (float)G;
  float klacc[OWN], macc[OWN];
#pragma unroll
  for (int m = 0; m < OWN; ++m) klacc[m] = macc[m] = 0.0f;

  auto key_tile = [&](auto masked, const i32x4* ktile, const i32x4* itile, int kb, int kt) {
    f32x16 s, z;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = z[e] = 0.0f;
    {
      vec8<T> bf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bf[ks] = key_frag<T, SK::CPR>(ktile, 32 * kt + l32, (16 * ks + 8 * h) / SK::EPC);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(s, qf[ks], bf[ks]);
    }
    {
      vec8<T> bi[KSI];
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks)
        bi[ks] = key_frag<T, SI::CPR>(itile, 32 * kt + l32, (16 * ks + 8 * h) / SI::EPC);
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks) mma(z, qif[ks], bi[ks]);
    }
    float part[NLQ];
#pragma unroll
    for (int lq = 0; lq < NLQ; ++lq) {
      float p = 0.0f;
#pragma unroll
      for (int e = lq * RPQ; e < (lq + 1) * RPQ; ++e)
        p += __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sc2, -lm2[e]));
      part[lq] = p;
    }
    const int key = kb * 128 + 32 * kt + l32;
#pragma unroll
    for (int m = 0; m < OWN; ++m) {
      float P, zz;
      if constexpr (PARTNER) {
        // half h keeps query 2m + h; the other half's partial sum comes across
        const float send = h ? part[2 * m] : part[2 * m + 1];
        const float recv = shfl_xor_f(send, 32);
        P = (h ? part[2 * m + 1] : part[2 * m]) + recv;
        zz = h ? z[(2 * m + 1) * RPQ] : z[2 * m * RPQ];
      } else {
        P = part[m];
        zz = z[m * RPQ];
      }
      P *= inv_g;
      const bool vis = !decltype(masked)::value || key <= i_q[m];
      P = vis ? P : 0.0f;
      const float lpi2 = __builtin_fmaf(zz, zc2, -li2[m]);  // log2 P_idx
      // P below the smallest normal float adds nothing (and v_log_f32 may read it as 0)
      klacc[m] += P >= 1.17549435e-38f ? P * (__builtin_amdgcn_logf(P) - lpi2) : 0.0f;
      macc[m] += P;
      if (ds && qv[m] && key < N)
        ds[dsr[m] + key] = (bf16)(vis ? __builtin_amdgcn_exp2f(lpi2) - P : 0.0f);
    }
  };
  auto block = [&](auto masked, int kb) {
    const int cur = kb & 1;
    if (kb + 1 <= kb_last) {
      sk.store(kbuf[cur ^ 1], tid);
      si.store(ibuf[cur ^ 1], tid);
      if (kb + 2 <= kb_last) {
        sk.load(kbase, kstride, (kb + 2) * 128, N, tid);
        si.load(ibase, DI, (kb + 2) * 128, N, tid);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) key_tile(masked, kbuf[cur], ibuf[cur], kb, kt);
    if (mass) {
#pragma unroll
      for (int m = 0; m < OWN; ++m) {
        float v = macc[m];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) v += shfl_xor_f(v, o);
        if (l32 == 0 && qv[m] && kb <= (i_q[m] >> 7)) mass[grow[m] * nb + kb] = v;
        macc[m] = 0.0f;
      }
    }
    __syncthreads();
  };
  int kb = 0;
  for (; kb < kb_mask; ++kb) block(std::false_type(), kb);
  for (; kb <= kb_last; ++kb) block(std::true_type(), kb);

#pragma unroll
  for (int m = 0; m < OWN; ++m) {
    float v = klacc[m] * kLn2;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += shfl_xor_f(v, o);
    if (kl_rows && l32 == 0 && qv[m]) kl_rows[grow[m]] = v;
  }
}

// KL pass for G >= 8, with the index logits formed once per workgroup. The
// workgroup's QT <= 32 queries fit one 32-column MFMA tile, so waves 0-3 form
// z = S_idx of one 32-key tile each (K_idx tile x Q_idx^T) into a
// double-buffered LDS table, a block ahead: K_idx is staged one block ahead
// of K, and the table for block kb+1 is written while block kb is consumed.
// The registers this frees let each wave issue the MFMAs of key tile kt+1
// before the exponentials of tile kt. Same arithmetic as kl_dense_kernel.
template <typename T, int D, int DI, int G, int NW>
__global__ void __launch_bounds__(64 * NW)
kl_dense_zt_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ q_idx,
                   const T* __restrict__ k_idx, const float* __restrict__ lse_main,
                   const float* __restrict__ lse_idx, float* __restrict__ kl_rows,
                   float* __restrict__ mass, bf16* __restrict__ ds, int N, int Nq,
                   int q_start, int t_begin, int t_end, int Hkv, int nb, int ntiles, int ntasks,
                   float sc2, float zc2) {
  constexpr int NT = 64 * NW, RT = 32 * NW, QT = RT / G, KS = D / 16, KSI = DI / 16;
  static_assert(G >= 8 && QT <= 32 && NW >= 4, "one table tile, four table waves");
  constexpr int RPQ = G / 2;    // rows of one query per lane
  constexpr int NLQ = 16 / RPQ; // queries per lane before the split
  constexpr int OWN = NLQ / 2;  // queries per lane after it
  constexpr int QPW = 32 / G;   // queries per wave
  constexpr int ZST = 128 + 4;  // table row stride (floats)
  using SK = KeyStage<T, D, NT>;
  using SI = KeyStage<T, DI, NT>;
  __shared__ i32x4 kbuf[2][128 * SK::CPR];
  __shared__ i32x4 ibuf[2][128 * SI::CPR];
  __shared__ float zs[2][QT * ZST];

  Task tk;
  if (!task_of(ntasks, ntiles, Hkv, &tk)) return;
  const int b = tk.b, r = tk.y, t0 = t_begin + tk.tile * QT;
  const int t_last = min(t_end, t0 + QT) - 1;
  const int kb_last = (q_start + t_last) >> 7;
  const int kb_mask = min((q_start + t0 + 1) >> 7, kb_last + 1);
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = Hkv * G;
  const size_t kstride = (size_t)Hkv * D;
  const T* kbase = k + (size_t)b * N * kstride + (size_t)r * D;
  const T* ibase = k_idx + (size_t)b * N * DI;

  SK sk;
  SI si;
  sk.load(kbase, kstride, 0, N, tid);
  si.load(ibase, DI, 0, N, tid);
  // A fragments of S = Q K^T: MFMA row l32 = wave row 32w + l32 = (query, head)
  vec8<T> qf[KS];
  {
    const int rho = 32 * wave + l32;
    const int tc = min(t0 + rho / G, t_end - 1);
    const T* qp = q + (((size_t)b * Nq + tc) * Hq + (size_t)r * G + rho % G) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = ld8<T>(qp + 16 * ks);
  }
  // B fragments of the table (waves 0-3): column l32 = query t0 + l32; columns
  // past the tile's queries repeat a valid row and are never stored
  vec8<T> qit[KSI];
  if (wave < 4) {
    const int tc = min(t0 + min(l32, QT - 1), t_end - 1);
    const T* qip = q_idx + (((size_t)b * Nq + tc) * Hkv + r) * DI + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) qit[ks] = ld8<T>(qip + 16 * ks);
  }
  float lm2[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int rho = 32 * wave + drow(e, h);
    const int tc = min(t0 + rho / G, t_end - 1);
    lm2[e] = lse_main[((size_t)b * Nq + tc) * Hq + (size_t)r * G + rho % G] * kLog2e;
  }
  int i_q[OWN], zrow[OWN];
  float li2[OWN];
  size_t grow[OWN], dsr[OWN];
  bool qv[OWN];
#pragma unroll
  for (int m = 0; m < OWN; ++m) {
    const int wq = wave * QPW + 2 * m + h;  // query within the workgroup
    const int tq = t0 + wq;
    const int tc = min(tq, t_end - 1);
    zrow[m] = wq * ZST;
    qv[m] = tq < t_end;
    i_q[m] = q_start + tc;
    grow[m] = ((size_t)b * Nq + tc) * Hkv + r;
    li2[m] = lse_idx[grow[m]] * kLog2e;
    dsr[m] = (((size_t)b * (t_end - t_begin) + (tc - t_begin)) * Hkv + r) * (size_t)ds_stride(N);
  }

  auto ztile = [&](int buf, const i32x4* itile) {
    vec8<T> af[KSI];
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks)
      af[ks] = key_frag<T, SI::CPR>(itile, 32 * wave + l32, (16 * ks + 8 * h) / SI::EPC);
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) mma(acc, af[ks], qit[ks]);
    if (l32 < QT) {
#pragma unroll
      for (int e = 0; e < 16; ++e) zs[buf][l32 * ZST + 32 * wave + drow(e, h)] = acc[e] * zc2;
    }
  };

  sk.store(kbuf[0], tid);
  si.store(ibuf[0], tid);
  if (kb_last >= 1) {
    sk.load(kbase, kstride, 128, N, tid);
    si.load(ibase, DI, 128, N, tid);
  }
  __syncthreads();
  if (wave < 4) ztile(0, ibuf[0]);
  if (kb_last >= 1) {
    si.store(ibuf[1], tid);
    if (kb_last >= 2) si.load(ibase, DI, 256, N, tid);
  }
  __syncthreads();  // table of block 0 and K_idx of block 1 in LDS

  const float inv_g = 1.0f / (float)G;
  float klacc[OWN], macc[OWN];
#pragma unroll
  for (int m = 0; m < OWN; ++m) klacc[m] = macc[m] = 0.0f;

  auto smma = [&](f32x16& s, const i32x4* ktile, int kt) {
    vec8<T> bf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bf[ks] = key_frag<T, SK::CPR>(ktile, 32 * kt + l32, (16 * ks + 8 * h) / SK::EPC);
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) mma(s, qf[ks], bf[ks]);
  };
  auto vtile = [&](auto masked, const f32x16& s, const float* zt, int kb, int kt) {
    float part[NLQ];
#pragma unroll
    for (int lq = 0; lq < NLQ; ++lq) {
      float p = 0.0f;
#pragma unroll
      for (int e = lq * RPQ; e < (lq + 1) * RPQ; ++e)
        p += __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sc2, -lm2[e]));
      part[lq] = p;
    }
    const int kk = 32 * kt + l32;
#pragma unroll
    for (int m = 0; m < OWN; ++m) {
      const float send = h ? part[2 * m] : part[2 * m + 1];
      const float recv = shfl_xor_f(send, 32);
      float P = ((h ? part[2 * m + 1] : part[2 * m]) + recv) * inv_g;
      const bool vis = !decltype(masked)::value || kb * 128 + kk <= i_q[m];
      P = vis ? P : 0.0f;
      const float lpi2 = zt[zrow[m] + kk] - li2[m];  // log2 P_idx
      klacc[m] += P >= 1.17549435e-38f ? P * (__builtin_amdgcn_logf(P) - lpi2) : 0.0f;
      macc[m] += P;
      if (ds && qv[m] && kb * 128 + kk < N)
        ds[dsr[m] + kb * 128 + kk] = (bf16)(vis ? __builtin_amdgcn_exp2f(lpi2) - P : 0.0f);
    }
  };
  auto block = [&](auto masked, int kb) {
    const int cur = kb & 1;
    if (kb + 1 <= kb_last) {
      sk.store(kbuf[cur ^ 1], tid);
      if (kb + 2 <= kb_last) sk.load(kbase, kstride, (kb + 2) * 128, N, tid);
      if (wave < 4) ztile(cur ^ 1, ibuf[cur ^ 1]);
      if (kb + 2 <= kb_last) {
        si.store(ibuf[cur], tid);  // block kb's K_idx was last read for its table
        if (kb + 3 <= kb_last) si.load(ibase, DI, (kb + 3) * 128, N, tid);
      }
    }
    const i32x4* kt_lds = kbuf[cur];
    const float* zt = zs[cur];
    f32x16 sa, sb;
    smma(sa, kt_lds, 0);
    smma(sb, kt_lds, 1);
    vtile(masked, sa, zt, kb, 0);
    smma(sa, kt_lds, 2);
    vtile(masked, sb, zt, kb, 1);
    smma(sb, kt_lds, 3);
    vtile(masked, sa, zt, kb, 2);
    vtile(masked, sb, zt, kb, 3);
    if (mass) {
#pragma unroll
      for (int m = 0; m < OWN; ++m) {
        float v = macc[m];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) v += shfl_xor_f(v, o);
        if (l32 == 0 && qv[m] && kb <= (i_q[m] >> 7)) mass[grow[m] * nb + kb] = v;
        macc[m] = 0.0f;
      }
    }
    __syncthreads();
  };
  int kb = 0;
  for (; kb < kb_mask; ++kb) block(std::false_type(), kb);
  for (; kb <= kb_last; ++kb) block(std::true_type(), kb);

#pragma unroll
  for (int m = 0; m < OWN; ++m) {
    float v = klacc[m] * kLn2;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += shfl_xor_f(v, o);
    if (kl_rows && l32 == 0 && qv[m]) kl_rows[grow[m]] = v;
  }
}

// ============================================================== KL gradient chain
//
// KL note §3: the index logits receive P_idx - P; through z = q_idx . k_idx /
// sqrt(d_idx) with one shared k_idx head (indexer note §2.1),
//   dq_idx[i, r] = coef / sqrt(d_idx) * sum_{j <= i} dS[i, r, j] k_idx[j]
//   dk_idx[j]    = coef / sqrt(d_idx) * sum over (i, r), i >= j, of dS[i, r, j] q_idx[i, r].
// The KL pass writes dS in bf16 for a chunk of query rows ([B, chunk, Hkv, N]);
// the two products below run on bf16 matrix cores with fp32 accumulation.
// Operands with the reduction index along rows of a row-major tile come from
// the transposing LDS read (16-lane groups receive element j of 4 consecutive
// rows); the other operand takes the same k-set {16c+4h+0..3, 16c+8+4h+0..3}
// from a contiguous row.

typedef __attribute__((address_space(3))) short4v lds_short4;

// X^T fragment (32 columns x 16 rows) of a row-major bf16 LDS tile with row
// stride LD: columns 32*ct.., rows 16c..16c+15, k-set as above
template <int LD>
__device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int c, int ct, int lane) {
  const int g16 = lane >> 4, s16 = lane & 15;
  const int krow = 16 * c + 4 * (g16 >> 1) + (s16 >> 2);
  const int col = ct * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tile + krow * LD + col));
  const short4v hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tile + (krow + 8) * LD + col));
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = l4[e];
    a[4 + e] = h4[e];
  }
  return a;
}

template <typename T>
__device__ __forceinline__ bf16x8 to_bf16x8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return ld8<bf16>(reinterpret_cast<const bf16*>(p));
  } else {
    const f32x8 v = ld8<float>(p);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    return o;
  }
}

// dq_idx rows of a chunk. Workgroup = 128 consecutive chunk rows (t, r) of one
// batch; wave w takes rows 32w..32w+31 as the columns of D^T = K_idx^T . dS^T.
// Per 128-key block, the K_idx block and the rows' dS on it are loaded
// row-contiguously (16 lanes per 256-byte dS row segment) one block ahead and
// staged through LDS. Keys after a row's query are masked when the dS
// fragments are read (select, so unwritten parts of the dS rows are never used).
template <typename T, int DI>
__global__ void __launch_bounds__(256)
dense_dq_idx_kernel(const bf16* __restrict__ ds, const T* __restrict__ k_idx,
                    T* __restrict__ dq, int N, int Nq, int q_start, int t_begin, int t_end,
                    int Hkv, int tiles_b, float scale) {
  constexpr int LK = DI + 8;
  constexpr int LS = 128 + 8;  // row stride of the dS tile
  constexpr int DT = DI / 32;
  __shared__ __attribute__((aligned(16))) bf16 kt[128 * LK];
  __shared__ __attribute__((aligned(16))) bf16 dst[128 * LS];
  const int rows_b = (t_end - t_begin) * Hkv;
  const int b = blockIdx.x / tiles_b, rho0 = (blockIdx.x % tiles_b) * 128;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = tid >> 6;
  const int rho = rho0 + 32 * wave + l32;
  const int rc = min(rho, rows_b - 1);
  const int t = t_begin + rc / Hkv, r = rc % Hkv;
  const int i = q_start + t;
  const int rlast = min(rho0 + 127, rows_b - 1);
  const int kb_last = (q_start + t_begin + rlast / Hkv) >> 7;
  const T* kbase = k_idx + (size_t)b * N * DI;

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;
  }
  // next block's K_idx chunks and dS row segments (global -> registers)
  constexpr int KCH = 128 * DI / 8 / 256;
  constexpr int SCH = 128 * 16 / 256;
  bf16x8 kraw[KCH], sraw[SCH];
  // Loads without branches (a guarded load joins the unguarded path and the
  // wait after the join drains every load in flight): rows past the chunk read
  // its last row (their dq_idx is never written); a dS row holds ds_stride(N)
  // >= N elements and a segment starts at a multiple of 8, so a segment past
  // the row reads the row's last one. Keys past N are after every query, so the
  // select below zeroes their dS, and the K_idx row they meet (row N-1) is finite.
  const int seg_max = ds_stride(N) - 8;
  auto prefetch = [&](int kb) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int x = tid + 256 * u, row = x / (DI / 8), c = x % (DI / 8);
      const int j = min(kb * 128 + row, N - 1);
      kraw[u] = to_bf16x8<T>(kbase + (size_t)j * DI + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < SCH; ++u) {
      const int x = tid + 256 * u, rr = x / 16, c = x % 16;
      const bf16* p = ds + ((size_t)b * rows_b + min(rho0 + rr, rows_b - 1)) * ds_stride(N);
      sraw[u] = ld8<bf16>(p + min(kb * 128 + 8 * c, seg_max));
    }
  };
  prefetch(0);
  for (int kb = 0; kb <= kb_last; ++kb) {
    __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int x = tid + 256 * u, row = x / (DI / 8), c = x % (DI / 8);
      *reinterpret_cast<bf16x8*>(kt + row * LK + 8 * c) = kraw[u];
    }
#pragma unroll
    for (int u = 0; u < SCH; ++u) {
      const int x = tid + 256 * u, rr = x / 16, c = x % 16;
      *reinterpret_cast<bf16x8*>(dst + rr * LS + 8 * c) = sraw[u];
    }
    __syncthreads();
    if (kb + 1 <= kb_last) prefetch(kb + 1);
    // B fragments: the lane's row, keys {16c + 4h + 0..3, 16c + 8 + 4h + 0..3}
    // (the k-set of the transposing read of K_idx); keys after the row's query
    // are masked (select)
    const bf16* srow = dst + (32 * wave + l32) * LS;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x4 lo = ld4<bf16>(srow + 16 * c + 4 * h), hi = ld4<bf16>(srow + 16 * c + 8 + 4 * h);
      const int key0 = kb * 128 + 16 * c + 4 * h;
      bf16x8 bfr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bfr[e] = key0 + e <= i ? lo[e] : (bf16)0.0f;
        bfr[4 + e] = key0 + 8 + e <= i ? hi[e] : (bf16)0.0f;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) mma(acc[dt], frag_tr<LK>(kt, c, dt, lane), bfr);
    }
  }
  if (rho < rows_b) {
    T* out = dq + (((size_t)b * Nq + t) * Hkv + r) * DI;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) out[32 * dt + drow(e, h)] = (T)(acc[dt][e] * scale);
    }
  }
}

// dk_idx of one 128-key block over the chunk's rows whose query sees the
// block (i >= 128 blk). D^T = Q_idx^T . dS: both operands by the transposing
// read of 64-row LDS tiles (q_idx rows; the same rows' dS on the block's keys).
// Wave w produces key tile w. The chunks of a call add up in an fp32
// accumulator (one workgroup per block, so no atomics); the last chunk writes
// dk_idx. dS of rows whose query is before a key is 0 (written by the KL pass).
template <typename T, int DI>
__global__ void __launch_bounds__(256)
dense_dk_idx_kernel(const bf16* __restrict__ ds, const T* __restrict__ q_idx,
                    float* __restrict__ dk_acc, T* __restrict__ dk, int N, int Nq, int q_start,
                    int t_begin, int t_end, int Hkv, int nb, float scale, int first, int last) {
  constexpr int RT = 64, LQ = DI + 8, LS = 128 + 8;
  constexpr int DT = DI / 32;
  __shared__ __attribute__((aligned(16))) bf16 qs[RT * LQ];
  __shared__ __attribute__((aligned(16))) bf16 dss[RT * LS];
  const int blk = blockIdx.x % nb, b = blockIdx.x / nb;
  const int rows_b = (t_end - t_begin) * Hkv;
  const int t_first = max(t_begin, 128 * blk - q_start);
  const int rho_first = (t_first - t_begin) * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = tid >> 6;

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;
  }
  // next row tile (global -> registers): q_idx rows and the rows' dS on the block
  constexpr int QCH = RT * DI / 8 / 256, SCH = RT * 16 / 256;
  bf16x8 qraw[QCH], sraw[SCH];
  // Loads without branches (a guarded load joins the unguarded path and the
  // wait after the join drains every load in flight): rows past the chunk read
  // its last row, and their q_idx rows are zeroed when the tile is stored, so
  // they add nothing; dS runs past a row's ds_stride(N) elements read its last
  // run (key0 is a multiple of 8): those keys are >= N, and their dk columns are
  // never written.
  const int srun_max = ds_stride(N) - 8;
  auto prefetch = [&](int rho0) {
#pragma unroll
    for (int u = 0; u < QCH; ++u) {
      const int x = tid + 256 * u, rr = x / (DI / 8), c = x % (DI / 8);
      const int rho = min(rho0 + rr, rows_b - 1);
      const size_t row = ((size_t)b * Nq + t_begin + rho / Hkv) * Hkv + rho % Hkv;
      qraw[u] = to_bf16x8<T>(q_idx + row * DI + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < SCH; ++u) {
      const int x = tid + 256 * u, rr = x / 16, c = x % 16;
      const int rho = min(rho0 + rr, rows_b - 1);
      const bf16* p = ds + ((size_t)b * rows_b + rho) * ds_stride(N);
      sraw[u] = ld8<bf16>(p + min(blk * 128 + 8 * c, srun_max));
    }
  };
  if (rho_first < rows_b) prefetch(rho_first);
  for (int rho0 = rho_first; rho0 < rows_b; rho0 += RT) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int u = 0; u < QCH; ++u) {
      const int x = tid + 256 * u, rr = x / (DI / 8), c = x % (DI / 8);
      bf16x8 v = qraw[u];
      if (rho0 + rr >= rows_b) {  // a row past the chunk adds nothing
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)0.0f;
      }
      *reinterpret_cast<bf16x8*>(qs + rr * LQ + 8 * c) = v;
    }
#pragma unroll
    for (int u = 0; u < SCH; ++u) {
      const int x = tid + 256 * u, rr = x / 16, c = x % 16;
      *reinterpret_cast<bf16x8*>(dss + rr * LS + 8 * c) = sraw[u];
    }
    __syncthreads();
    if (rho0 + RT < rows_b) prefetch(rho0 + RT);
#pragma unroll
    for (int c = 0; c < RT / 16; ++c) {
      const bf16x8 bfr = frag_tr<LS>(dss, c, wave, lane);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) mma(acc[dt], frag_tr<LQ>(qs, c, dt, lane), bfr);
    }
  }
  const int j = blk * 128 + 32 * wave + l32;
  if (j < N) {
    const size_t base = ((size_t)b * N + j) * DI;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const size_t x = base + 32 * dt + drow(e, h);
        float v = acc[dt][e];
        if (!first) v += dk_acc[x];
        if (last) {
          dk[x] = (T)(v * scale);
        } else {
          dk_acc[x] = v;
        }
      }
    }
  }
}

// ============================================================== recall
//
// One wavefront per (b, t, r) row. T = the teacher's top min(k, L+1) blocks
// among the visible blocks 0..L (L = the query's local block) by block mass,
// the lower index first on equal mass. A selected block is in T when fewer
// than |T| visible blocks outrank it. block recall = |S ∩ T| / |T|;
// score recall = the mass on S (ids -1 and ids outside 0..L count as empty).
__global__ void __launch_bounds__(256)
recall_kernel(const float* __restrict__ mass, const int32_t* __restrict__ ids,
              float* __restrict__ brec, float* __restrict__ srec, int64_t nrows, int Nq,
              int q_start, int Hkv, int nb, int topk) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int t = (int)((row / Hkv) % Nq);
  const int L = (q_start + t) >> 7;
  const int tsz = min(topk, L + 1);
  const float* mr = mass + row * nb;
  const int32_t* id = ids + row * topk;
  int hits = 0;
  float score = 0.0f;
  for (int s = 0; s < topk; ++s) {
    const int blk = id[s];
    if (blk < 0 || blk > L) continue;
    const float v = mr[blk];
    int above = 0;
    for (int c = lane; c <= L; c += 64) {
      const float x = mr[c];
      above += (x > v || (x == v && c < blk)) ? 1 : 0;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) above += __shfl_xor(above, o, 64);
    hits += above < tsz ? 1 : 0;
    score += v;
  }
  if (lane == 0) {
    brec[row] = (float)hits / (float)tsz;
    srec[row] = score;
  }
}

// mean of x[0..n) in a fixed order (fp64 partial sums), one workgroup
__global__ void __launch_bounds__(1024)
mean_kernel(const float* __restrict__ x, int64_t n, float* __restrict__ out) {
  __shared__ double red[1024];
  double v = 0.0;
  for (int64_t a = threadIdx.x; a < n; a += 1024) v += (double)x[a];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = n > 0 ? (float)(red[0] / (double)n) : 0.0f;
}

// ============================================================== launch

constexpr int kDenseWaves = 8;

template <typename T, int D, int R>
static hipError_t lse_run(const Dims& d, const void* q, const void* k, float* lse, int qrows,
                          int kstride, int ngroups, hipStream_t s) {
  constexpr int QT = 64 * kDenseWaves / R;
  const int ntiles = (d.Nq + QT - 1) / QT;
  const int ntasks = ntiles * d.B * ngroups;
  if (ntasks == 0) return hipSuccess;
  const float scale_log2 = (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634);
  dense_lse_kernel<T, D, R, kDenseWaves><<<task_grid(ntasks), 64 * kDenseWaves, 0, s>>>(
      (const T*)q, (const T*)k, lse, d.N, d.Nq, d.q_start, qrows, kstride, ngroups, ntiles,
      ntasks, scale_log2);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t lse_by_r(const Dims& d, int R, const void* q, const void* k, float* lse,
                           int qrows, int kstride, int ngroups, hipStream_t s) {
  switch (R) {
    case 1: return lse_run<T, D, 1>(d, q, k, lse, qrows, kstride, ngroups, s);
    case 2: return lse_run<T, D, 2>(d, q, k, lse, qrows, kstride, ngroups, s);
    case 4: return lse_run<T, D, 4>(d, q, k, lse, qrows, kstride, ngroups, s);
    case 8: return lse_run<T, D, 8>(d, q, k, lse, qrows, kstride, ngroups, s);
    case 16: return lse_run<T, D, 16>(d, q, k, lse, qrows, kstride, ngroups, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t lse_by_dim(const Dims& d, int dim, int R, const void* q, const void* k,
                             float* lse, int qrows, int kstride, int ngroups, hipStream_t s) {
  if (dim == 64) return lse_by_r<T, 64>(d, R, q, k, lse, qrows, kstride, ngroups, s);
  if (dim == 32) return lse_by_r<T, 32>(d, R, q, k, lse, qrows, kstride, ngroups, s);
  if constexpr (sizeof(T) == 2) {
    if (dim == 128) return lse_by_r<T, 128>(d, R, q, k, lse, qrows, kstride, ngroups, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dense_lse(const Dims& d, bool index_branch, const void* q, const void* k,
                            float* lse, hipStream_t s) {
  // main: G heads per group, K head y at offset y*D of a [Hkv*D] key row;
  // index: Hkv heads per query, all on the one [DI] key row
  const int dim = index_branch ? d.DI : d.D;
  const int R = index_branch ? d.Hkv : d.G;
  const int qrows = index_branch ? d.Hkv : d.Hq;
  const int kstride = index_branch ? d.DI : d.Hkv * d.D;
  const int ngroups = index_branch ? 1 : d.Hkv;
  if (d.dtype == MSA_BF16) return lse_by_dim<bf16>(d, dim, R, q, k, lse, qrows, kstride, ngroups, s);
  return lse_by_dim<float>(d, dim, R, q, k, lse, qrows, kstride, ngroups, s);
}

struct DenseKlArgs {
  const void *q, *k, *qi, *ki;
  const float *lse_main, *lse_idx;
  float *kl_rows, *mass;
  bf16* ds;
  int t_begin, t_end;
};

template <typename T, int D, int DI, int G>
static hipError_t kl_dense_run(const Dims& d, const DenseKlArgs& a, hipStream_t s) {
  constexpr int QT = 32 * kDenseWaves / G;
  const int ntiles = (a.t_end - a.t_begin + QT - 1) / QT;
  const int ntasks = ntiles * d.B * d.Hkv;
  if (ntasks == 0) return hipSuccess;
  const float sc2 = (float)(1.0 / std::sqrt((double)D) * 1.4426950408889634);
  const float zc2 = (float)(1.0 / std::sqrt((double)DI) * 1.4426950408889634);
  if constexpr (G >= 8 && sizeof(T) == 2) {  // fp32 tiles would not fit LDS with the table
    kl_dense_zt_kernel<T, D, DI, G, kDenseWaves><<<task_grid(ntasks), 64 * kDenseWaves, 0, s>>>(
        (const T*)a.q, (const T*)a.k, (const T*)a.qi, (const T*)a.ki, a.lse_main, a.lse_idx,
        a.kl_rows, a.mass, a.ds, d.N, d.Nq, d.q_start, a.t_begin, a.t_end, d.Hkv, d.nb, ntiles,
        ntasks, sc2, zc2);
  } else {
    kl_dense_kernel<T, D, DI, G, kDenseWaves><<<task_grid(ntasks), 64 * kDenseWaves, 0, s>>>(
        (const T*)a.q, (const T*)a.k, (const T*)a.qi, (const T*)a.ki, a.lse_main, a.lse_idx,
        a.kl_rows, a.mass, a.ds, d.N, d.Nq, d.q_start, a.t_begin, a.t_end, d.Hkv, d.nb, ntiles,
        ntasks, sc2, zc2);
  }
  return hipGetLastError();
}

template <typename T, int D, int DI>
static hipError_t kl_dense_by_g(const Dims& d, const DenseKlArgs& a, hipStream_t s) {
  switch (d.G) {
    case 1: return kl_dense_run<T, D, DI, 1>(d, a, s);
    case 2: return kl_dense_run<T, D, DI, 2>(d, a, s);
    case 4: return kl_dense_run<T, D, DI, 4>(d, a, s);
    case 8: return kl_dense_run<T, D, DI, 8>(d, a, s);
    case 16: return kl_dense_run<T, D, DI, 16>(d, a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t kl_dense_by_di(const Dims& d, const DenseKlArgs& a, hipStream_t s) {
  if (d.DI == 64) return kl_dense_by_g<T, D, 64>(d, a, s);
  if (d.DI == 32) return kl_dense_by_g<T, D, 32>(d, a, s);
  return hipErrorInvalidValue;
}

static hipError_t kl_dense_dispatch(const Dims& d, const DenseKlArgs& a, hipStream_t s) {
  if (d.dtype == MSA_BF16) {
    if (d.D == 128) return kl_dense_by_di<bf16, 128>(d, a, s);
    if (d.D == 64) return kl_dense_by_di<bf16, 64>(d, a, s);
  } else if (d.D == 64) {
    return kl_dense_by_di<float, 64>(d, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_kl_dense(const Dims& d, const void* q, const void* k, const void* q_idx,
                           const void* k_idx, const float* lse_main, const float* lse_idx,
                           float* kl_rows, float* mass, hipStream_t s) {
  const DenseKlArgs a{q, k, q_idx, k_idx, lse_main, lse_idx, kl_rows, mass, nullptr, 0, d.Nq};
  return kl_dense_dispatch(d, a, s);
}

// Rows per chunk of the gradient chain: a multiple of 256 query positions
// (every KL tile lies in one chunk) with at most ~2 GiB of bf16 dS per chunk.
int dense_grad_chunk(const Dims& d) {
  const int64_t per_t = (int64_t)d.B * d.Hkv * ds_stride(d.N) * 2;
  int64_t ch = per_t > 0 ? ((int64_t)1 << 31) / per_t : d.Nq;
  ch = ch / 256 * 256;
  if (ch < 256) ch = 256;
  const int64_t all = ((int64_t)d.Nq + 255) / 256 * 256;
  return (int)(ch < all ? ch : all);
}

template <typename T, int DI>
static hipError_t chain_run(const Dims& d, const bf16* ds, const void* qi, const void* ki,
                            float* dk_acc, void* dq, void* dk, int t_begin, int t_end, float scale,
                            bool first, bool last, hipStream_t s) {
  const int rows_b = (t_end - t_begin) * d.Hkv;
  const int tiles_b = (rows_b + 127) / 128;
  if (tiles_b > 0) {
    dense_dq_idx_kernel<T, DI><<<(unsigned)(tiles_b * d.B), 256, 0, s>>>(
        ds, (const T*)ki, (T*)dq, d.N, d.Nq, d.q_start, t_begin, t_end, d.Hkv, tiles_b, scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dense_dk_idx_kernel<T, DI><<<(unsigned)(d.nb * d.B), 256, 0, s>>>(
      ds, (const T*)qi, dk_acc, (T*)dk, d.N, d.Nq, d.q_start, t_begin, t_end, d.Hkv, d.nb, scale,
      first ? 1 : 0, last ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_kl_dense_grad(const Dims& d, const void* q, const void* k, const void* q_idx,
                                const void* k_idx, const float* lse_main, const float* lse_idx,
                                float* kl_rows, float* mass, float coef, bf16* ds,
                                float* dk_acc, void* dq_idx, void* dk_idx, hipStream_t s) {
  const int chunk = dense_grad_chunk(d);
  const float scale = (float)((double)coef / std::sqrt((double)d.DI));
  for (int t0 = 0; t0 < d.Nq; t0 += chunk) {
    const int t1 = t0 + chunk < d.Nq ? t0 + chunk : d.Nq;
    const DenseKlArgs a{q, k, q_idx, k_idx, lse_main, lse_idx, kl_rows, mass, ds, t0, t1};
    prof_before(MSA_K_KL_DENSE, s);
    hipError_t e = kl_dense_dispatch(d, a, s);
    prof_after(MSA_K_KL_DENSE, s);
    if (e != hipSuccess) return e;
    const bool first = t0 == 0, last = t1 == d.Nq;
    prof_before(MSA_K_KL_DENSE_CHAIN, s);
    if (d.dtype == MSA_BF16) {
      e = d.DI == 64 ? chain_run<bf16, 64>(d, ds, q_idx, k_idx, dk_acc, dq_idx, dk_idx, t0, t1,
                                           scale, first, last, s)
                     : chain_run<bf16, 32>(d, ds, q_idx, k_idx, dk_acc, dq_idx, dk_idx, t0, t1,
                                           scale, first, last, s);
    } else {
      e = d.DI == 64 ? chain_run<float, 64>(d, ds, q_idx, k_idx, dk_acc, dq_idx, dk_idx, t0, t1,
                                            scale, first, last, s)
                     : chain_run<float, 32>(d, ds, q_idx, k_idx, dk_acc, dq_idx, dk_idx, t0, t1,
                                            scale, first, last, s);
    }
    prof_after(MSA_K_KL_DENSE_CHAIN, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_recall(const Dims& d, const float* mass, const int32_t* ids, float* brec,
                         float* srec, hipStream_t s) {
  const int64_t nrows = d.rows * d.Hkv;
  if (nrows == 0) return hipSuccess;
  recall_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, s>>>(mass, ids, brec, srec, nrows, d.Nq,
                                                            d.q_start, d.Hkv, d.nb, d.K);
  return hipGetLastError();
}

hipError_t launch_mean(const float* x, int64_t n, float* out, hipStream_t s) {
  mean_kernel<<<1, 1024, 0, s>>>(x, n, out);
  return hipGetLastError();
}

}  // namespace msa
