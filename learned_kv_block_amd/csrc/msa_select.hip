// msa_select.hip — index scoring with fused causal block max, and block Top-k.
//
// Index branch of "MSA Indexer 与 DSA Lightning Indexer 的差别" (MSA vs DSA
// indexer note): §2.1 scores S_idx = Q_idx . K_idx^T / sqrt(d_idx) with one
// shared K_idx head; §2.2 block score M[i,b] = max of S_idx over the tokens
// j <= i of 128-token block b, then Top-k blocks with the query's local block
// always included. "MiniMax Sparse Attention：教长上下文模型使用索引" (MSA blog),
// kernel section: the Top-k runs on raw scores (softmax keeps the order).
#include <type_traits>

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
// Workgroup = one tile of RT = 32*CT*NW consecutive GEMM rows (QT = RT/HKV
// queries x all HKV groups; the rows are contiguous in Q_idx) x a chunk of CB
// key blocks. Wave w owns CT row tiles of 32 GEMM rows, [32CTw, 32CT(w+1)):
// its Q_idx rows stay in registers as MFMA B fragments for the whole chunk,
// and every K_idx fragment read from LDS feeds CT MFMAs. Each 128-key block of
// K_idx is read from HBM/L2 once per workgroup, row-contiguously, and shared by
// all NW waves through a double-buffered LDS tile (one barrier per block).
// The product is formed transposed, D = K_idx_tile (32 keys as rows) x
// Q_idx^T, so a lane holds 16 keys of one GEMM row and the block max is an
// in-lane reduction over the four key tiles plus one exchange between the two
// lane halves. Block maxima of the chunk are collected in LDS and written row
// by row (CB contiguous floats per row) at the end: the N x N score matrix
// never leaves registers.
//
// LDS tiles hold 16-byte chunks; chunk c of row r sits at position
// c ^ swz(r) inside the row, so that the 32 rows a fragment read touches (and
// the rows a store touches) spread over all banks.

// LSE: also the per-block log-sum-exp of the index logits over the block's
// keys j <= i (a running max and sum per key tile, the two lane halves merged
// at the block's end), written to BL beside the block maxima.
// bf16 with CT <= 3 runs two waves per SIMD (256 registers each), CT = 4 one
// wave per SIMD with the 512 registers of a lone wave.
template <typename T, int DI, int HKV, int NW, int CT, int CB, bool LSE>
__global__ void __launch_bounds__(64 * NW, sizeof(T) != 2 ? 1 : CT == 2 ? 8 / NW : CT == 3 ? 2 : 1)
index_blockmax_kernel(const T* __restrict__ q_idx, const T* __restrict__ k_idx,
                      float* __restrict__ M, float* __restrict__ BL, int N, int Nq, int q_start,
                      int nb, float scale) {
  constexpr int NT = 64 * NW;
  constexpr int RT = 32 * CT * NW;         // GEMM rows per tile
  constexpr int QT = RT / HKV;             // queries per tile
  constexpr int KS = DI / 16;
  constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int CPR = DI / EPC;            // chunks per row
  constexpr int SWM = (CPR < 8 ? CPR : 8) - 1;
  constexpr int KCH = 128 * CPR / NT;      // K_idx chunks per thread per block
  constexpr int QCH = 32 * CPR / 64;       // Q_idx chunks per lane per 32-row half
  constexpr int MST = CB + 1;              // block-max row stride (floats): empty column + CB
  constexpr int QBYTES = NW * 32 * CPR * 16;
  constexpr int MBYTES = RT * MST * 4 * (LSE ? 2 : 1);  // block maxima (then block LSEs)
  constexpr int UBYTES = QBYTES > MBYTES ? QBYTES : MBYTES;
  static_assert((128 * CPR) % NT == 0 && (32 * CPR) % 64 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) char ubuf[UBYTES];  // Q_idx staging, then block maxima
  __shared__ i32x4 kbuf[2][128 * CPR];

  const int tile = blockIdx.x;
  const int b = blockIdx.z;
  const int t0 = tile * QT;
  if (t0 >= Nq) return;
  const int t_last = min(Nq, t0 + QT) - 1;
  const int i_last = q_start + t_last;
  const int kb0 = (int)blockIdx.y * CB;
  if (kb0 * 128 > i_last) return;  // whole workgroup: chunk is after every row's window
  const int kb1 = min(kb0 + CB - 1, i_last >> 7);

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // raw K_idx chunks of block kb (keys past N read row N-1; every such key is
  // > i for all rows and is masked)
  const char* kbase = reinterpret_cast<const char*>(k_idx + (size_t)b * N * DI);
  i32x4 raw[KCH];
  auto load_raw = [&](int kb) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int q = tid + NT * u, r = q / CPR, c = q % CPR;
      const int j = min(kb * 128 + r, N - 1);
      raw[u] = *reinterpret_cast<const i32x4*>(kbase + ((size_t)j * CPR + c) * 16);
    }
  };
  auto store_raw = [&](i32x4* dst) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int q = tid + NT * u, r = q / CPR, c = q % CPR;
      dst[r * CPR + (c ^ (idx_swz(r) & SWM))] = raw[u];
    }
  };
  load_raw(kb0);

  // Q_idx: the wave's 32*CT rows, in CT tiles of 32 rows staged through LDS.
  // Rows past the last query read a valid row and are never stored.
  vec8<T> qf[CT][KS];
  {
    i32x4* qs = reinterpret_cast<i32x4*>(ubuf) + wave * 32 * CPR;
    const char* qbase = reinterpret_cast<const char*>(q_idx);
    const size_t rbase = (size_t)b * Nq * HKV;
    const size_t rmax = rbase + (size_t)Nq * HKV - 1;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int u = 0; u < QCH; ++u) {
        const int q = lane + 64 * u, r = q / CPR, c = q % CPR;
        const size_t grow = min(rbase + (size_t)t0 * HKV + wave * 32 * CT + 32 * ct + r, rmax);
        qs[r * CPR + (c ^ (idx_swz(r) & SWM))] =
            *reinterpret_cast<const i32x4*>(qbase + (grow * CPR + c) * 16);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ct][ks] = lds_frag<T, CPR>(qs, l32, (16 * ks + 8 * h) / EPC);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  }
  store_raw(kbuf[0]);
  if (kb0 + 1 <= kb1) load_raw(kb0 + 1);
  __syncthreads();  // block kb0 is in LDS; every wave has its Q fragments

  float* mbuf = reinterpret_cast<float*>(ubuf);
  float* lbuf = mbuf + RT * MST;  // LSE only
  const float c2 = scale * kLog2e;  // exp(scale * s) = exp2(c2 * s)
  const int row0 = wave * 32 * CT;  // first GEMM row of the wave
  int i_row[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) i_row[ct] = q_start + t0 + (row0 + 32 * ct + l32) / HKV;

  // One key tile (32 keys) of the block: D^T tiles for the wave's CT row tiles.
  auto mma_tile = [&](const i32x4* tile, int kt, f32x16* acc) {
    vec8<T> af[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) af[ks] = lds_frag<T, CPR>(tile, 32 * kt + l32, (16 * ks + 8 * h) / EPC);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ct][e] = 0.0f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) mma(acc[ct], af[ks], qf[ct][ks]);
    }
  };
  // causal mask (MASK) and running in-lane block max (LSE: and the sum of
  // exp(scale (s - max))) of one key tile
  float l[CT] = {};
  auto reduce_tile = [&](auto masked, f32x16* acc, float* m, int kb, int kt) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 128 + 32 * kt + drow(e, h) > i_row[ct]) acc[ct][e] = -INFINITY;
      }
      float x = m[ct];
#pragma unroll
      for (int e = 0; e < 16; e += 2) x = vmax(vmax(x, acc[ct][e]), acc[ct][e + 1]);
      if constexpr (LSE) {
        const float mu = x == -INFINITY ? 0.0f : x;  // all masked so far: every term is 0
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f((acc[ct][e] - mu) * c2);
        l[ct] = l[ct] * __builtin_amdgcn_exp2f((m[ct] - mu) * c2) + sum;
      }
      m[ct] = x;
    }
  };
  // block kb's maxima -> LDS column kb - kb0 + 1 (column 0 takes the empty
  // block before kb0); both lane halves hold the value and store it
  auto finish_block = [&](float* m, int kb) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float mo = shfl_xor_f(m[ct], 32);
      const float x = vmax(m[ct], mo);
      mbuf[(row0 + 32 * ct + l32) * MST + (kb - kb0 + 1)] = x;
      if constexpr (LSE) {
        const float lo = shfl_xor_f(l[ct], 32);
        const float mu = x == -INFINITY ? 0.0f : x;
        const float z = l[ct] * __builtin_amdgcn_exp2f((m[ct] - mu) * c2) +
                        lo * __builtin_amdgcn_exp2f((mo - mu) * c2);
        // ln sum exp(scale s) = scale max + ln z
        lbuf[(row0 + 32 * ct + l32) * MST + (kb - kb0 + 1)] =
            x == -INFINITY ? -INFINITY : (x * c2 + __builtin_amdgcn_logf(z)) * kLn2;
        l[ct] = 0.0f;
      }
    }
  };

  // Software pipeline: the MFMAs of key tile kt+1 are issued before the VALU
  // reduces tile kt; tile 3 of a block is reduced under tile 0 of the next.
  // The body is branch-free so that the two streams can interleave; blocks
  // that need the causal mask (the tile's last one or two) run in a second loop.
  f32x16 accA[CT], accB[CT];
  float m[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int e = 0; e < 16; ++e) accB[ct][e] = -INFINITY;
    m[ct] = -INFINITY;
  }
  auto block_body = [&](auto masked, int kb) {
    const int cur = (kb - kb0) & 1;
    if (kb + 1 <= kb1) {
      store_raw(kbuf[cur ^ 1]);  // last read in the previous iteration, before its barrier
      if (kb + 2 <= kb1) load_raw(kb + 2);
    }
    const i32x4* kt_lds = kbuf[cur];
    mma_tile(kt_lds, 0, accA);
    reduce_tile(masked, accB, m, kb - 1, 3);
    finish_block(m, kb - 1);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) m[ct] = -INFINITY;
    mma_tile(kt_lds, 1, accB);
    reduce_tile(masked, accA, m, kb, 0);
    mma_tile(kt_lds, 2, accA);
    reduce_tile(masked, accB, m, kb, 1);
    mma_tile(kt_lds, 3, accB);
    reduce_tile(masked, accA, m, kb, 2);
    __syncthreads();  // next block is in LDS; this block's tile may be overwritten
  };
  // first block with a key after the tile's first query
  const int kb_mask = min(max(kb0, (q_start + t0 + 1) >> 7), kb1 + 1);
  int kb = kb0;
  for (; kb < kb_mask; ++kb) block_body(std::false_type(), kb);
  for (; kb <= kb1; ++kb) block_body(std::true_type(), kb);
  reduce_tile(std::true_type(), accB, m, kb1, 3);
  finish_block(m, kb1);
  __syncthreads();

  // write the chunk's block maxima, CB contiguous floats per row
  const int nblk = kb1 - kb0 + 1;
  const size_t grow0 = ((size_t)b * Nq + t0) * HKV;
  for (int x = tid; x < RT * nblk; x += NT) {
    const int row = x / nblk, kk = x - row * nblk;
    const int tq = t0 + row / HKV;
    if (tq >= Nq || kb0 + kk > ((q_start + tq) >> 7)) continue;
    M[(grow0 + row) * nb + kb0 + kk] = mbuf[row * MST + kk + 1] * scale;  // scale > 0 commutes with max
    if constexpr (LSE) BL[(grow0 + row) * nb + kb0 + kk] = lbuf[row * MST + kk + 1];
  }
}

// bf16 tiles: 8 waves of 96 GEMM rows (768 rows per workgroup). Against 64
// rows per wave this cuts the LDS fragment reads per MFMA by a third
// (3.80 -> 3.70 ms at the skewed 131072 shape); 128 rows per wave spill at two
// waves per SIMD and lose latency hiding at one.
#ifndef MSA_IDX_CT
#define MSA_IDX_CT 3
#endif
#ifndef MSA_IDX_NW
#define MSA_IDX_NW 8
#endif
#ifndef MSA_IDX_CB
#define MSA_IDX_CB 32
#endif

template <typename T, int DI, int HKV, int NW, int CT, bool LSE>
static hipError_t index_launch(const Dims& d, const void* qi, const void* ki, float* M, float* BL,
                               hipStream_t s) {
  constexpr int CB = LSE ? 16 : MSA_IDX_CB;  // LSE: two LDS staging arrays
  constexpr int QT = 32 * CT * NW / HKV;
  const int ntiles = (d.Nq + QT - 1) / QT;
  const int nchunks = (d.nb + CB - 1) / CB;
  if (ntiles == 0 || d.B == 0) return hipSuccess;
  dim3 grid(ntiles, nchunks, d.B);
  const float scale = 1.0f / sqrtf((float)DI);
  index_blockmax_kernel<T, DI, HKV, NW, CT, CB, LSE><<<grid, 64 * NW, 0, s>>>(
      (const T*)qi, (const T*)ki, M, BL, d.N, d.Nq, d.q_start, d.nb, scale);
  return hipGetLastError();
}

template <typename T, int DI, int HKV, bool LSE>
static hipError_t index_dispatch(const Dims& d, const void* qi, const void* ki, float* M,
                                 float* BL, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    // fp32 tiles: LDS and register limits
    return index_launch<T, DI, HKV, 4, 2, LSE>(d, qi, ki, M, BL, s);
  } else {
    // a decode step has a few rows per sequence: one-wave tiles (64 rows)
    // instead of 768-row tiles keep the MFMA work near the rows that exist
    if ((int64_t)d.Nq * HKV <= 64) return index_launch<T, DI, HKV, 1, 2, LSE>(d, qi, ki, M, BL, s);
    // the block-LSE pass keeps 64 rows per wave: its running sums do not fit
    // the registers of more
    constexpr int CT = LSE ? 2 : MSA_IDX_CT;
    return index_launch<T, DI, HKV, LSE ? 8 : MSA_IDX_NW, CT, LSE>(d, qi, ki, M, BL, s);
  }
}

template <typename T, int DI, bool LSE>
static hipError_t index_dispatch_hkv(const Dims& d, const void* qi, const void* ki, float* M,
                                     float* BL, hipStream_t s) {
  switch (d.Hkv) {
    case 1: return index_dispatch<T, DI, 1, LSE>(d, qi, ki, M, BL, s);
    case 2: return index_dispatch<T, DI, 2, LSE>(d, qi, ki, M, BL, s);
    case 4: return index_dispatch<T, DI, 4, LSE>(d, qi, ki, M, BL, s);
    case 8: return index_dispatch<T, DI, 8, LSE>(d, qi, ki, M, BL, s);
  }
  return hipErrorInvalidValue;
}

template <bool LSE>
static hipError_t index_dispatch_all(const Dims& d, const void* q_idx, const void* k_idx,
                                     float* M, float* BL, hipStream_t s) {
  if (d.dtype == MSA_BF16) {
    if (d.DI == 64) return index_dispatch_hkv<bf16, 64, LSE>(d, q_idx, k_idx, M, BL, s);
    if (d.DI == 32) return index_dispatch_hkv<bf16, 32, LSE>(d, q_idx, k_idx, M, BL, s);
  } else {
    if (d.DI == 64) return index_dispatch_hkv<float, 64, LSE>(d, q_idx, k_idx, M, BL, s);
    if (d.DI == 32) return index_dispatch_hkv<float, 32, LSE>(d, q_idx, k_idx, M, BL, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_index_blockmax(const Dims& d, const void* q_idx, const void* k_idx, float* M,
                                 hipStream_t s) {
  if (decode_index_supported(d)) return launch_decode_index(d, q_idx, k_idx, M, s);
  return index_dispatch_all<false>(d, q_idx, k_idx, M, nullptr, s);
}

hipError_t launch_index_block_lse(const Dims& d, const void* q_idx, const void* k_idx, float* M,
                                  float* BL, hipStream_t s) {
  return index_dispatch_all<true>(d, q_idx, k_idx, M, BL, s);
}

// ============================================================== block Top-k
//
// One wavefront per (b, t, r) row of block scores M[0..L], L = local block.
// Keys are 64-bit: (order-preserving bits of the score) << 32 | ~block, so a
// larger key means a higher score, or an equal score and a lower block index;
// every key is distinct. Lane l owns blocks v*64 + l; the scores are read with
// buffer loads whose range ends at block L, so blocks past it need no branch.
//  1. T = the (k-1)-th largest per-lane maximum score, found by bisection on
//     its order-preserving bits (one ballot per bit, stopping as soon as
//     exactly k-1 lane maxima are >= T). Every block of the true top-(k-1)
//     scores >= T, and at least k-1 blocks do, so the blocks with score >= T
//     are the candidates.
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

constexpr int kCandMax = 128;  // candidates ranked exactly (two passes of 64)

// One (query, group) row with L candidate blocks, VV*64 >= L: lane l holds
// blocks v*64 + l, v < VV.
// NF: the first NF groups v are known to lie below L (64*NF < L), so only the
// others need the -inf select.
template <int VV, int NF>
__device__ __forceinline__ void topk_row(const float* __restrict__ M, int64_t row, int L, int nb,
                                         int k, int32_t* __restrict__ out,
                                         float* __restrict__ margin, uint64_t* __restrict__ candw,
                                         uint64_t* __restrict__ mselw, int lane) {
  constexpr int V = VV;
  // scores of the candidate blocks 0..L-1; loads past block L-1 return 0
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(M + row * (int64_t)nb), 0, L * 4, 0x00020000);
  float x[V];
  float lm = -INFINITY;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float raw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (v * 64 + lane) * 4, 0, 0));
    x[v] = (v < NF || v * 64 + lane < L) ? raw : -INFINITY;
  }
#pragma unroll
  for (int v = 0; v + 1 < V; v += 2) lm = vmax(vmax(lm, x[v]), x[v + 1]);
  if constexpr (V % 2) lm = vmax(lm, x[V - 1]);
  // 1. threshold: bisection on the order-preserving bits of the lane maxima
  const uint32_t om = ord_f32(lm);
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t tt = T | (1u << bit);
    const int cnt = __popcll(__ballot(om >= tt));
    if (cnt >= k - 1) {
      T = tt;
      if (cnt == k - 1) break;
    }
  }
  // ord(x) >= T implies x >= Tf; the float test may add a signed-zero tie,
  // which the exact ranking below handles
  const float Tf = f32_of_ord(T);

  // 2. compact the candidates (positions past kCandMax go to the sink; C
  // counts them all, and a list that overflowed is not used)
  int C = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const bool c = x[v] >= Tf;
    const uint64_t bal = __ballot(c);
    if (bal) {  // uniform
      const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      candw[(c && pos < kCandMax) ? pos : kCandMax] = make_key(x[v] + 0.0f, v * 64 + lane);  // -0 -> +0
      C += __popcll(bal);
    }
  }
  uint64_t worst_sel = 0, best_unsel = 0;
  if (C <= kCandMax) {
    if (margin && lane < 2) mselw[lane] = 0;
    wave_sync();
    // 3. exact ranks among candidates
    int pos_base = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const bool have = c < C;
      const uint64_t kc = have ? candw[c] : 0;
      int rank = 0;
      for (int c2 = 0; c2 < C; ++c2) rank += candw[c2] > kc;
      const bool sel = have && rank < k - 1;
      const uint64_t bal = __ballot(sel);
      if (sel)
        out[pos_base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] =
            key_blk(kc);
      pos_base += __popcll(bal);
      if (margin && have) {
        if (rank == k - 2) mselw[0] = kc;
        if (rank == k - 1) mselw[1] = kc;
      }
    }
    if (margin) {
      wave_sync();
      worst_sel = mselw[0];
      best_unsel = mselw[1];
      uint64_t nc = 0;  // best non-candidate
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const uint64_t kv = x[v] > -INFINITY ? make_key(x[v] + 0.0f, v * 64 + lane) : 0;
        if (!(x[v] >= Tf) && kv > nc) nc = kv;
      }
      nc = wave_max_u64(nc);
      best_unsel = nc > best_unsel ? nc : best_unsel;
    }
  } else {
    // fallback: k-1 rounds of wave argmax over all blocks
    uint64_t key[V];
#pragma unroll
    for (int v = 0; v < V; ++v) key[v] = x[v] > -INFINITY ? make_key(x[v] + 0.0f, v * 64 + lane) : 0;
    uint32_t taken = 0;
    for (int round = 0; round < k - 1; ++round) {
      uint64_t bestl = 0;
      int bestv = -1;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (!((taken >> v) & 1u) && key[v] > bestl) {
          bestl = key[v];
          bestv = v;
        }
      const uint64_t best = wave_max_u64(bestl);
      if (bestv >= 0 && bestl == best) taken |= 1u << bestv;
      if (round == k - 2) worst_sel = best;
    }
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
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
      // +inf when nothing competes for a slot: k = 1 (no slot besides the local block) or
      // no candidate left out
      margin[row] = (k > 1 && best_unsel) ? key_score(worst_sel) - key_score(best_unsel)
                                          : INFINITY;
  }
}

template <int VV, int STEP, int V>
__device__ __forceinline__ void topk_row_fit(const float* __restrict__ M, int64_t row, int L, int nb,
                                             int k, int32_t* __restrict__ out,
                                             float* __restrict__ margin, uint64_t* __restrict__ candw,
                                             uint64_t* __restrict__ mselw, int lane) {
  // here L > (VV - STEP) * 64: the first VV - STEP groups are whole
  constexpr int NF = VV > STEP ? VV - STEP : 0;
  if constexpr (VV >= V) {
    topk_row<V, NF>(M, row, L, nb, k, out, margin, candw, mselw, lane);
  } else {
    if (L <= VV * 64)  // uniform
      topk_row<VV, NF>(M, row, L, nb, k, out, margin, candw, mselw, lane);
    else
      topk_row_fit<VV + STEP, STEP, V>(M, row, L, nb, k, out, margin, candw, mselw, lane);
  }
}

template <int V>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ M, int64_t nrows, int Nq, int q_start, int Hkv, int nb,
            int k, int32_t* __restrict__ ids, float* __restrict__ margin) {
  __shared__ uint64_t cand[4][kCandMax + 1];  // + a sink for non-candidate lanes
  __shared__ uint64_t msel[4][2];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
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
  // L, and with it the register count of the row, is uniform per wave
  constexpr int STEP = V >= 16 ? V / 4 : V;
  topk_row_fit<STEP, STEP, V>(M, row, L, nb, k, out, margin, cand[wave], msel[wave], lane);
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
