// msa_select.hip — index scoring with fused causal block max, and block Top-k.
//
// Index branch of "MSA Indexer 与 DSA Lightning Indexer 的差别" (MSA vs DSA
// indexer note): §2.1 scores S_idx = Q_idx . K_idx^T / sqrt(d_idx) with one
// shared K_idx head; §2.2 block score M[i,b] = max of S_idx over the tokens
// j <= i of 128-token block b, then Top-k blocks with the query's local block
// always included. "MiniMax Sparse Attention：教长上下文模型使用索引" (MSA blog),
// kernel section: the Top-k runs on raw scores (softmax keeps the order).
#include "msa_internal.hpp"

namespace msa {

// ============================================================== fill kernels

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x)
    p[x] = v;
}
__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x)
    p[x] = v;
}
static unsigned fill_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<fill_grid(n), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_f32_kernel<<<fill_grid(n), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

// ============================================================== index GEMM + block max
//
// Workgroup = one tile of QT = 128/HKV consecutive query rows (all HKV groups:
// 128 GEMM rows, contiguous in Q_idx) x a chunk of kIdxChunk key blocks.
// Wave w owns keys [32w, 32w+32) of each 128-key block. The product is formed
// transposed, D = K_idx_tile (keys as rows) * Q_idx_tile^T, so each lane holds
// 16 keys of one GEMM row and a wave's part of the block max is an in-lane
// reduction plus one exchange with the other lane half. The four waves' parts
// of every block of the chunk meet in LDS after a single barrier per chunk.
//  - MFMA fragments tie a lane to one row, so a direct fragment load touches
//    32 rows per instruction. Q_idx and K_idx are instead read row-contiguously
//    (1 KB per instruction) and re-read as fragments from LDS.
//  - Two accumulator sets: the MFMAs of block kb+1 are in flight while the
//    VALU runs the max epilogue of block kb; raw K_idx rows are loaded two
//    blocks ahead.
// The N x N score matrix never leaves registers; one fp32 per (row, block) is
// written, a row's blocks of the chunk contiguously.

constexpr int kIdxChunk = 8;

template <typename T, int DI, int HKV>
__global__ void __launch_bounds__(256, 2)
index_blockmax_kernel(const T* __restrict__ q_idx, const T* __restrict__ k_idx,
                      float* __restrict__ M, int N, int Nq, int q_start, int nb, int ntiles,
                      float scale) {
  constexpr int QT = 128 / HKV;
  constexpr int KS = DI / 16;
  constexpr int CB = kIdxChunk;
  constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int CPR = DI / EPC;            // chunks per row
  constexpr int LDQ = DI + 2 * EPC;        // staging row stride (elements), breaks bank aliasing
  constexpr int QCH = 128 * CPR / 256;     // Q_idx chunks per thread
  constexpr int KCH = 32 * CPR / 64;       // K_idx chunks per lane per block
  __shared__ float red_m[CB][4][128];
  __shared__ T qs[128 * LDQ];
  __shared__ T kst[4][32 * LDQ];

  const int tile = ntiles - 1 - (int)blockIdx.y;  // longest rows first
  const int b = blockIdx.z;
  const int t0 = tile * QT;
  const int t_last = min(Nq, t0 + QT) - 1;
  const int i_first = q_start + t0;
  const int i_last = q_start + t_last;
  const int kb0 = (int)blockIdx.x * CB;
  if (kb0 * 128 > i_last) return;  // whole workgroup: chunk is after every row's window
  const int kb1 = min(kb0 + CB - 1, i_last / 128);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;

  // Q_idx tile: 128 rows (query t0 + row/HKV, group row%HKV) are contiguous.
  // Rows past the last query read a valid row and are never stored.
  {
    const size_t rbase = (size_t)(b * (size_t)Nq) * HKV;
    const size_t rmax = rbase + (size_t)Nq * HKV - 1;
#pragma unroll
    for (int u = 0; u < QCH; ++u) {
      const int c = tid + 256 * u, row = c / CPR, ch = c % CPR;
      const size_t grow = min(rbase + (size_t)t0 * HKV + row, rmax);
      st8<T>(&qs[row * LDQ + ch * EPC], ld8<T>(q_idx + grow * DI + ch * EPC));
    }
  }
  __syncthreads();
  vec8<T> qf[4][KS];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ct][ks] = ld8<T>(&qs[(32 * ct + l32) * LDQ + 16 * ks + 8 * h]);

  // raw K_idx rows of this wave's 32 keys of block kb (keys past N read row N-1;
  // every such key is > i for all rows and is masked)
  const T* kb_base = k_idx + (size_t)b * N * DI;
  T* const kw = kst[wave];
  auto load_raw = [&](int kb, vec8<T>* raw) {
    const int kc = min(kb, kb1);
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = lane + 64 * u, row = c / CPR, ch = c % CPR;
      const int j = min(kc * 128 + 32 * wave + row, N - 1);
      raw[u] = ld8<T>(kb_base + (size_t)j * DI + ch * EPC);
    }
  };
  auto raw_to_frags = [&](const vec8<T>* raw, vec8<T>* f) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = lane + 64 * u;
      st8<T>(&kw[(c / CPR) * LDQ + (c % CPR) * EPC], raw[u]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) f[ks] = ld8<T>(&kw[l32 * LDQ + 16 * ks + 8 * h]);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  };
  auto mma_blk = [&](const vec8<T>* f, f32x16* acc) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ct][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(acc[ct], f[ks], qf[ct][ks]);
    }
  };
  // causal mask, per-wave block max, partial result to LDS
  auto epilogue = [&](f32x16* acc, int kb) {
    const bool need_mask = (kb * 128 + 127 > i_first);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int row = 32 * ct + l32;
      const int i_row = q_start + t0 + row / HKV;
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 128 + 32 * wave + drow(e, h) > i_row) acc[ct][e] = -INFINITY;
      }
      float m = acc[ct][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) m = fmaxf(m, acc[ct][e]);
      m = fmaxf(m, shfl_xor_f(m, 32));
      if (h == 0) red_m[kb - kb0][wave][row] = m;
    }
  };

  vec8<T> raw0[KCH], raw1[KCH], f[KS];
  f32x16 acc0[4], acc1[4];
  load_raw(kb0, raw0);
  load_raw(kb0 + 1, raw1);
  raw_to_frags(raw0, f);
  mma_blk(f, acc0);
  load_raw(kb0 + 2, raw0);
  for (int kb = kb0; kb <= kb1; kb += 2) {
    // acc0: block kb; raw1: block kb+1; raw0: block kb+2 (in flight)
    if (kb + 1 <= kb1) {
      raw_to_frags(raw1, f);
      load_raw(kb + 3, raw1);
      mma_blk(f, acc1);
    }
    epilogue(acc0, kb);
    if (kb + 1 > kb1) break;
    // acc1: block kb+1; raw0: block kb+2; raw1: block kb+3
    if (kb + 2 <= kb1) {
      raw_to_frags(raw0, f);
      load_raw(kb + 4, raw0);
      mma_blk(f, acc0);
    }
    epilogue(acc1, kb + 1);
  }
  __syncthreads();
  // combine the four waves: thread = (row, block of the chunk)
  const int nblk = kb1 - kb0 + 1;
  for (int x = tid; x < 128 * nblk; x += 256) {
    const int row = x / nblk, kk = x % nblk;  // a row's blocks are contiguous in M
    const int tq = t0 + row / HKV;
    const int r = row % HKV;
    if (tq >= Nq || kb0 + kk > (q_start + tq) / 128) continue;
    const float m = fmaxf(fmaxf(red_m[kk][0][row], red_m[kk][1][row]),
                          fmaxf(red_m[kk][2][row], red_m[kk][3][row]));
    const size_t o = ((size_t)(b * (size_t)Nq + tq) * HKV + r) * nb + kb0 + kk;
    M[o] = m * scale;  // scale > 0 commutes with max
  }
}

template <typename T, int DI, int HKV>
static hipError_t index_dispatch(const Dims& d, const void* qi, const void* ki, float* M,
                                 hipStream_t s) {
  constexpr int QT = 128 / HKV;
  const int ntiles = (d.Nq + QT - 1) / QT;
  const int nchunks = (d.nb + kIdxChunk - 1) / kIdxChunk;
  if (ntiles == 0 || d.B == 0) return hipSuccess;
  dim3 grid(nchunks, ntiles, d.B);
  const float scale = 1.0f / sqrtf((float)DI);
  index_blockmax_kernel<T, DI, HKV><<<grid, 256, 0, s>>>((const T*)qi, (const T*)ki, M, d.N, d.Nq,
                                                         d.q_start, d.nb, ntiles, scale);
  return hipGetLastError();
}

template <typename T, int DI>
static hipError_t index_dispatch_hkv(const Dims& d, const void* qi, const void* ki, float* M,
                                     hipStream_t s) {
  switch (d.Hkv) {
    case 1: return index_dispatch<T, DI, 1>(d, qi, ki, M, s);
    case 2: return index_dispatch<T, DI, 2>(d, qi, ki, M, s);
    case 4: return index_dispatch<T, DI, 4>(d, qi, ki, M, s);
    case 8: return index_dispatch<T, DI, 8>(d, qi, ki, M, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_index_blockmax(const Dims& d, const void* q_idx, const void* k_idx, float* M,
                                 hipStream_t s) {
  if (d.dtype == MSA_BF16) {
    if (d.DI == 64) return index_dispatch_hkv<bf16, 64>(d, q_idx, k_idx, M, s);
    if (d.DI == 32) return index_dispatch_hkv<bf16, 32>(d, q_idx, k_idx, M, s);
  } else {
    if (d.DI == 64) return index_dispatch_hkv<float, 64>(d, q_idx, k_idx, M, s);
    if (d.DI == 32) return index_dispatch_hkv<float, 32>(d, q_idx, k_idx, M, s);
  }
  return hipErrorInvalidValue;
}

// ============================================================== block Top-k
//
// One wavefront per (b, t, r) row of block scores M[0..L], L = local block.
// Keys are 64-bit: (order-preserving bits of the score) << 32 | ~block, so a
// larger key means a higher score, or an equal score and a lower block index;
// every key is distinct. Lane l owns blocks v*64 + l (coalesced loads).
//  1. T = the (k-1)-th largest per-lane maximum score (bitonic sort of the 64
//     lane maxima). Every block of the true top-(k-1) scores >= T, and at
//     least k-1 blocks do, so the blocks with score >= T are the candidates.
//  2. Candidates are compacted into LDS in (v, lane) order = ascending block.
//  3. Each candidate's exact rank among candidates gives the selection; the
//     selected ones keep their ascending order; the local block L (the
//     largest visible index) goes last.
// If ties make the candidate list overflow LDS, a k-1 round wave-argmax
// fallback gives the same (exact) result.

__device__ __forceinline__ uint32_t ord_f32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_of_ord(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t make_key(float score, int blk) {
  return ((uint64_t)ord_f32(score) << 32) | (uint64_t)(uint32_t)(~(uint32_t)blk);
}
__device__ __forceinline__ int key_blk(uint64_t key) { return (int)(~(uint32_t)(key & 0xffffffffull)); }
__device__ __forceinline__ float key_score(uint64_t key) { return f32_of_ord((uint32_t)(key >> 32)); }
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m, 64), hi = __shfl_xor((uint32_t)(x >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t y = shfl_xor_u64(x, m);
    x = y > x ? y : x;
  }
  return x;
}
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kTopkMax = 32;

template <int V>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ M, int64_t nrows, int Nq, int q_start, int Hkv, int nb,
            int k, int32_t* __restrict__ ids, float* __restrict__ margin) {
  constexpr int CMAX = (kTopkMax - 1) * V;
  __shared__ uint64_t cand[4][CMAX];
  __shared__ uint64_t msel[4][2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= nrows) return;  // wave-uniform; the kernel has no workgroup barrier
  const int t = (int)((row / Hkv) % Nq);
  const int i = q_start + t;
  const int L = i / 128;
  int32_t* out = ids + row * k;
  if (L + 1 <= k) {  // every visible block is selected
    for (int s = lane; s < k; s += 64) out[s] = s <= L ? s : -1;
    if (margin && lane == 0) margin[row] = INFINITY;
    return;
  }
  const float* mr = M + row * (int64_t)nb;
  uint64_t key[V];
  uint32_t lmax = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int blk = v * 64 + lane;
    if (blk < L) {
      const float sc = mr[blk];
      key[v] = make_key(sc, blk);
      lmax = max(lmax, ord_f32(sc));
    } else {
      key[v] = 0;  // not a candidate (every real key is > 0)
    }
  }
  // 1. threshold from the lane maxima: bitonic sort, descending
  uint32_t x = lmax;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t y = __shfl_xor(x, stride, 64);
      const bool lower = (lane & stride) == 0;
      const bool desc = (lane & size) == 0;
      const uint32_t hi = max(x, y), lo = min(x, y);
      x = (lower == desc) ? hi : lo;
    }
  }
  const uint32_t T = __shfl(x, k - 2, 64);

  // 2. count candidates
  int C = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const bool c = key[v] != 0 && (uint32_t)(key[v] >> 32) >= T;
    C += __popcll(__ballot(c));
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t worst_sel = 0, best_unsel = 0;
  if (C <= CMAX) {
    int base = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const bool c = key[v] != 0 && (uint32_t)(key[v] >> 32) >= T;
      const uint64_t bal = __ballot(c);
      if (c) cand[wave][base + __popcll(bal & lt_mask)] = key[v];
      base += __popcll(bal);
    }
    if (margin && lane < 2) msel[wave][lane] = 0;
    wave_sync();
    // 3. exact ranks among candidates
    int pos_base = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const bool have = c < C;
      const uint64_t kc = have ? cand[wave][c] : 0;
      int rank = 0;
      for (int c2 = 0; c2 < C; ++c2) rank += cand[wave][c2] > kc;
      const bool sel = have && rank < k - 1;
      const uint64_t bal = __ballot(sel);
      if (sel) out[pos_base + __popcll(bal & lt_mask)] = key_blk(kc);
      pos_base += __popcll(bal);
      if (margin && have) {
        if (rank == k - 2) msel[wave][0] = kc;
        if (rank == k - 1) msel[wave][1] = kc;
      }
    }
    if (margin) {
      wave_sync();
      worst_sel = msel[wave][0];
      best_unsel = msel[wave][1];
      uint64_t nc = 0;  // best non-candidate
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const bool c = key[v] != 0 && (uint32_t)(key[v] >> 32) >= T;
        if (!c && key[v] > nc) nc = key[v];
      }
      nc = wave_max_u64(nc);
      best_unsel = nc > best_unsel ? nc : best_unsel;
    }
  } else {
    // fallback: k-1 rounds of wave argmax over all blocks
    uint32_t taken = 0;
    for (int round = 0; round < k - 1; ++round) {
      uint64_t bestl = 0;
      int bestv = -1;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (!((taken >> v) & 1u) && key[v] > bestl) { bestl = key[v]; bestv = v; }
      const uint64_t best = wave_max_u64(bestl);
      if (bestv >= 0 && bestl == best) taken |= 1u << bestv;
      if (round == k - 2) worst_sel = best;
    }
    int base = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const bool sel = (taken >> v) & 1u;
      const uint64_t bal = __ballot(sel);
      if (sel) out[base + __popcll(bal & lt_mask)] = v * 64 + lane;
      base += __popcll(bal);
    }
    uint64_t nc = 0;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (!((taken >> v) & 1u) && key[v] > nc) nc = key[v];
    best_unsel = wave_max_u64(nc);
  }
  if (lane == 0) {
    out[k - 1] = L;
    if (margin)
      margin[row] = best_unsel ? key_score(worst_sel) - key_score(best_unsel) : INFINITY;
  }
}

hipError_t launch_topk(const Dims& d, const float* M, int32_t* ids, float* margin, hipStream_t s) {
  const int64_t nrows = d.rows * d.Hkv;
  if (nrows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((nrows + 3) / 4);
  const int vneed = (d.nb + 63) / 64;
  if (vneed <= 4)
    topk_kernel<4><<<grid, 256, 0, s>>>(M, nrows, d.Nq, d.q_start, d.Hkv, d.nb, d.K, ids, margin);
  else if (vneed <= 16)
    topk_kernel<16><<<grid, 256, 0, s>>>(M, nrows, d.Nq, d.q_start, d.Hkv, d.nb, d.K, ids, margin);
  else if (vneed <= 32)
    topk_kernel<32><<<grid, 256, 0, s>>>(M, nrows, d.Nq, d.q_start, d.Hkv, d.nb, d.K, ids, margin);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
