// msa_decode.hip — attention of one query per sequence (a decode step), query-outer.
//
// The same restricted softmax as the KV-outer path ("2.4 · 训练原生稀疏" eq. 2 on
// the selected support; the group's G heads share its block list and KV head,
// "MSA Indexer 与 DSA Lightning Indexer 的差别" §2.3), ordered for one query
// row per sequence: with a single query there is nothing to share a block
// with, so instead of inverting the selection into buckets, writing a
// partial per slot and merging the partials in a second kernel, one workgroup
// per (sequence, group) streams that row's selected blocks once and keeps a
// running (max, sum, output) per head, merged with the partition rule of
// "2.4" eq. (18) / "4.1.1 · 监督与联合训练" eq. (16).
//
// Workgroup: 4 waves; wave w owns keys 32w .. 32w+31 of every block and runs
// its own online softmax over them. The block's K and V sit in one LDS tile;
// the next block is loaded into registers during the current one and written
// to the tile between two barriers. At the end the four per-wave states merge
// through LDS: M = max_w m_w, O = sum_w e^(m_w - M) O_w / sum_w e^(m_w - M) l_w,
// LSE = M + log sum_w e^(m_w - M) l_w.
//
// Matrix products use the 16x16x32 bf16 instruction with the G heads (padded
// to 16 rows) as the rows (lane l, c = l % 16, g = l / 16):
//   S^T(keys x heads) = K Q^T:  A = K[16kt + c][32ks + 8g + e], B = Q[head c][32ks + 8g + e];
//                               lane (c, g) gets keys 16kt + 4g + j of head c.
//   O^T(d x heads) = V^T P^T:   the wave's 32 keys are one k-step; its B operand is the
//                               lane's own P (keys 32w + 4g + j and 32w + 16 + 4g + j),
//                               A = V[those keys][16dt + c] from two transposing LDS reads.
#include "msa_internal.hpp"

namespace msa {

namespace {

typedef float f32x4d __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void mma16d(f32x4d& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// reductions over the four lanes of a head (lanes c, c+16, c+32, c+48)
__device__ __forceinline__ float max4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// [128][D] bf16 tile, 16-byte chunk c of row rho stored at chunk c ^ swz(rho):
// K fragment reads (16 rows, one chunk) and transposing V reads (16 rows,
// 32 B) both spread over the banks.
template <int D>
__device__ __forceinline__ int dk_off(int rho, int col) {
  constexpr int CPR = D / 8;
  return rho * D + 8 * ((col >> 3) ^ (rho & (CPR - 1))) + (col & 7);
}
template <int D>
__device__ __forceinline__ int dv_off(int rho, int col) {
  constexpr int CPR = D / 8;
  return rho * D + 8 * ((col >> 3) ^ ((2 * rho) & (CPR - 1))) + (col & 7);
}

template <int D, int G>
__global__ void __launch_bounds__(256, 2)
decode_attn_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                   const bf16* __restrict__ v, const int32_t* __restrict__ ids,
                   bf16* __restrict__ out, float* __restrict__ lse, int N, int q_start, int Hkv,
                   int nb, int topk, float scale_log2) {
  constexpr int KS = D / 32;          // k-steps of S^T over d
  constexpr int DT = D / 16;          // d tiles of O^T
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int LD = 128 * CPR / 256; // 16-byte chunks per thread per tile (K or V)
  static_assert(G <= 16, "heads of a group are the rows of one 16-row tile");
  __shared__ bf16 Kt[128 * D];
  __shared__ bf16 Vt[128 * D];
  typedef __attribute__((address_space(3))) short4v lds_short4;

  const int row = blockIdx.x;             // (b, r) with one query per sequence
  const int r = row % Hkv, b = row / Hkv;
  const int i = q_start;                  // the query's position
  const int L = i / 128;                  // its local block
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, g = lane >> 4;
  const int wave = tid >> 6;
  const int Hq = Hkv * G;
  const size_t kvrow = (size_t)Hkv * D;
  const int32_t* rid = ids + (size_t)row * topk;

  // raw chunks of block blk for this thread: chunk p = tid + 256u of the tile
  i32x4 rk[LD], rv[LD];
  auto load_block = [&](int blk) {
    const int nvalid = min(128, N - blk * 128);
    const char* kb = reinterpret_cast<const char*>(k + ((size_t)b * N + (size_t)blk * 128) * kvrow +
                                                   (size_t)r * D);
    const char* vb = reinterpret_cast<const char*>(v + ((size_t)b * N + (size_t)blk * 128) * kvrow +
                                                   (size_t)r * D);
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int p = tid + 256 * u, rho = p / CPR, cs = p % CPR;
      const size_t off = (size_t)min(rho, nvalid - 1) * kvrow * 2 + (size_t)cs * 16;
      rk[u] = *reinterpret_cast<const i32x4*>(kb + off);
      rv[u] = *reinterpret_cast<const i32x4*>(vb + off);
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int p = tid + 256 * u, rho = p / CPR, cs = p % CPR;
      *reinterpret_cast<i32x4*>(&Kt[dk_off<D>(rho, cs * 8)]) = rk[u];
      *reinterpret_cast<i32x4*>(&Vt[dv_off<D>(rho, cs * 8)]) = rv[u];
    }
  };
  // next valid selected block after slot s (-1: none); ids are ascending, -1 padded
  auto next_slot = [&](int s) {
    for (++s; s < topk; ++s) {
      const int id = rid[s];
      if (id >= 0 && id <= L && id < nb) return s;
    }
    return -1;
  };

  // Q^T fragments of the group's heads (rows past G are zero)
  bf16x8 qf[KS];
  {
    const bf16* qp = q + ((size_t)b * Hq + (size_t)r * G + (c < G ? c : 0)) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = c < G ? ld8<bf16>(qp + 32 * ks) : zero8<bf16>();
  }

  float m_run = -INFINITY, l_run = 0.0f;  // log2 domain, per head (all four lanes hold it)
  f32x4d O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x4d{0.0f, 0.0f, 0.0f, 0.0f};

  int s = next_slot(-1);
  if (s >= 0) load_block(rid[s]);
  while (s >= 0) {
    const int blk = rid[s];
    __syncthreads();  // every wave is done with the previous block's tile
    store_block();
    const int sn = next_slot(s);
    __syncthreads();  // the tile holds block blk
    if (sn >= 0) load_block(rid[sn]);  // in flight during this block's products

    // S^T for the wave's two key tiles
    f32x4d S[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      S[h2] = f32x4d{0.0f, 0.0f, 0.0f, 0.0f};
      const int kt = 2 * wave + h2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        mma16d(S[h2], ld8<bf16>(Kt + dk_off<D>(16 * kt + c, 32 * ks + 8 * g)), qf[ks]);
    }
    // causal mask (the local block: keys past the query)
    float mx = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = blk * 128 + 16 * (2 * wave + h2) + 4 * g + j;
        if (key > i) S[h2][j] = -INFINITY;
        mx = vmax(mx, S[h2][j]);
      }
    const float m_new = vmax(m_run, max4(mx) * scale_log2);
    // a head with no visible key yet keeps m = -inf; its terms are all zero
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ls = 0.0f;
    bf16x8 pf;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[h2][j], scale_log2, -m_use));
        ls += p;
        pf[4 * h2 + j] = cvt<bf16>(p);
      }
    l_run = l_run * alpha + sum4(ls);
    m_run = m_new;
    // O^T += V^T P^T over the wave's 32 keys
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int krow = 32 * wave + 4 * g + (c >> 2), dcol = 16 * dt + 4 * (c & 3);
      const short4v lo =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(Vt + dv_off<D>(krow, dcol)));
      const short4v hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(Vt + dv_off<D>(krow + 16, dcol)));
      const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
      bf16x8 vf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[e] = l4[e];
        vf[4 + e] = h4[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) O[dt][e] *= alpha;
      mma16d(O[dt], vf, pf);
    }
    s = sn;
  }

  // ---- merge the four waves' states through LDS (the K tile is free now)
  __syncthreads();
  float* ms = reinterpret_cast<float*>(Kt);       // [4][16]: m (log2 domain)
  float* lsm = ms + 64;                            // [4][16]: l
  float* os = reinterpret_cast<float*>(Vt);       // [4][16][D]: unnormalised O
  if (g == 0) {
    ms[wave * 16 + c] = m_run;
    lsm[wave * 16 + c] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) os[(wave * 16 + c) * D + 16 * dt + 4 * g + e] = O[dt][e];
  __syncthreads();
  // thread t: head hd = t / 16 (< G), d range (t % 16) * D/16 .. +D/16
  const int hd = tid >> 4, part = tid & 15;
  if (hd < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = vmax(M, ms[w * 16 + hd]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    float wgt[4], l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wgt[w] = __builtin_amdgcn_exp2f(ms[w * 16 + hd] - Mu);
      l += wgt[w] * lsm[w * 16 + hd];
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // l = 0 only for an empty selection
    constexpr int PER = D / 16;                      // 8 (d = 128) or 4 (d = 64) per thread
    bf16* op = out + ((size_t)b * Hq + (size_t)r * G + hd) * D + part * PER;
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += wgt[w] * os[(w * 16 + hd) * D + part * PER + e];
      o[e] = acc * inv;
    }
    if constexpr (PER == 8) {
      bf16x8 o8;
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = cvt<bf16>(o[e]);
      st8<bf16>(op, o8);
    } else {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = cvt<bf16>(o[e]);
      st4<bf16>(op, o4);
    }
    if (part == 0) lse[(size_t)b * Hq + (size_t)r * G + hd] = (Mu + __log2f(l)) * kLn2;
  }
}

template <int D>
hipError_t decode_dispatch_g(const Dims& d, const void* q, const void* k, const void* v,
                             const int32_t* ids, void* out, float* lse, hipStream_t s) {
  const unsigned grid = (unsigned)(d.B * d.Hkv);
  const float scale_log2 = (float)(1.0 / sqrt((double)D) * 1.4426950408889634);
#define MSA_DEC_CASE(GG)                                                                       \
  case GG:                                                                                     \
    decode_attn_kernel<D, GG><<<grid, 256, 0, s>>>((const bf16*)q, (const bf16*)k,             \
                                                   (const bf16*)v, ids, (bf16*)out, lse, d.N,  \
                                                   d.q_start, d.Hkv, d.nb, d.K, scale_log2);   \
    break;
  switch (d.G) {
    MSA_DEC_CASE(1)
    MSA_DEC_CASE(2)
    MSA_DEC_CASE(4)
    MSA_DEC_CASE(8)
    MSA_DEC_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MSA_DEC_CASE
  return hipGetLastError();
}

// ------------------------------------------------------------ index scan of a decode step
//
// With one query per sequence the index GEMM has only Hkv rows per sequence, so
// it is a stream over K_idx (one 128-key block = 16 KB at d_idx = 64). Each wave
// takes 8 consecutive blocks of one sequence and loads their K_idx fragments
// straight from HBM into registers, one block ahead of the products (no LDS, no
// barrier); 8 blocks per wave keep ~8K waves in flight at the 64 x 131072 decode
// shape (nontemporal loads measured slower). The products are those of the prefill index kernel — the same
// 32x32x16 instruction, K_idx rows as A (lane l: key 32kt + l%32, d 16ks + 8h .. +7,
// h = l/32), the Hkv index-query rows as B columns (zero past Hkv), k-steps in
// the same order — so every block score is bit-identical to the prefill one.
#ifndef MSA_DIDX_CB
#define MSA_DIDX_CB 8
#endif

template <int DI>
__global__ void __launch_bounds__(256, 2)
decode_index_kernel(const bf16* __restrict__ q_idx, const bf16* __restrict__ k_idx,
                    float* __restrict__ M, int N, int q_start, int Hkv, int nb, int chunks,
                    int total_waves, float scale) {
  constexpr int KS = DI / 16;   // k-steps of 16
  constexpr int NF = 4 * KS;    // fragments per block: 4 key tiles x KS
  constexpr int CB = MSA_DIDX_CB;  // blocks per wave
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int gw = blockIdx.x * 4 + wave;  // (sequence, chunk) of this wave
  const int b = gw / chunks, ch = gw % chunks;
  const int i = q_start, L = i / 128;
  const int kb0 = ch * CB;
  if (gw >= total_waves) return;  // the last workgroup may have spare waves
  if (kb0 > L) return;
  const int kb1 = min(kb0 + CB - 1, L);
  // B operand: column l32 = index-query row r = l32 (< Hkv), d 16ks + 8h .. +7
  bf16x8 qf[KS];
  {
    const bf16* qp = q_idx + ((size_t)b * Hkv + (l32 < Hkv ? l32 : 0)) * DI + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = l32 < Hkv ? ld8<bf16>(qp + 16 * ks) : zero8<bf16>();
  }
  const bf16* kb = k_idx + (size_t)b * N * DI;
  auto load = [&](int blk, bf16x8* f) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = min(blk * 128 + 32 * kt + l32, N - 1);  // keys past N are masked
      const bf16* p = kb + (size_t)key * DI + 8 * h;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) f[kt * KS + ks] = ld8<bf16>(p + 16 * ks);
    }
  };
  float* mrow = M + (size_t)b * Hkv * nb;  // row r of sequence b: mrow + r * nb
  auto block = [&](int blk, const bf16x8* f) {
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(acc, f[kt * KS + ks], qf[ks]);
      if (blk == L) {  // the local block: keys after the query are masked
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (blk * 128 + 32 * kt + drow(e, h) > i) acc[e] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 16; e += 2) m = vmax(vmax(m, acc[e]), acc[e + 1]);
    }
    m = vmax(m, shfl_xor_f(m, 32));
    if (h == 0 && l32 < Hkv) mrow[(size_t)l32 * nb + blk] = m * scale;  // scale > 0: commutes
  };
  bf16x8 fa[NF], fb[NF];
  load(kb0, fa);
  for (int blk = kb0; blk <= kb1; blk += 2) {
    if (blk + 1 <= kb1) load(blk + 1, fb);
    block(blk, fa);
    if (blk + 1 > kb1) break;
    if (blk + 2 <= kb1) load(blk + 2, fa);
    block(blk + 1, fb);
  }
}

}  // namespace

bool decode_index_supported(const Dims& d) {
  return d.dtype == MSA_BF16 && d.Nq == 1 && (d.DI == 64 || d.DI == 32) && d.Hkv <= 8;
}

hipError_t launch_decode_index(const Dims& d, const void* q_idx, const void* k_idx, float* M,
                               hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  const int L = d.q_start / 128;
  const int chunks = (L + MSA_DIDX_CB) / MSA_DIDX_CB;  // MSA_DIDX_CB blocks per wave
  const unsigned grid = (unsigned)((d.B * chunks + 3) / 4);
  const float scale = 1.0f / sqrtf((float)d.DI);
  if (d.DI == 64)
    decode_index_kernel<64><<<grid, 256, 0, s>>>((const bf16*)q_idx, (const bf16*)k_idx, M, d.N,
                                                 d.q_start, d.Hkv, d.nb, chunks, d.B * chunks,
                                                 scale);
  else
    decode_index_kernel<32><<<grid, 256, 0, s>>>((const bf16*)q_idx, (const bf16*)k_idx, M, d.N,
                                                 d.q_start, d.Hkv, d.nb, chunks, d.B * chunks,
                                                 scale);
  return hipGetLastError();
}

bool decode_attn_supported(const Dims& d) {
  return d.dtype == MSA_BF16 && d.Nq == 1 && (d.D == 128 || d.D == 64) && d.G <= 16;
}

hipError_t launch_decode_attn(const Dims& d, const void* q, const void* k, const void* v,
                              const int32_t* ids, void* out, float* lse, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  if (d.D == 128) return decode_dispatch_g<128>(d, q, k, v, ids, out, lse, s);
  if (d.D == 64) return decode_dispatch_g<64>(d, q, k, v, ids, out, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace msa
