// msa_fp8.hip — FP8 (OCP E4M3) index scoring with fused causal block max.
//
// "MSA Indexer 与 DSA Lightning Indexer 的差别" (MSA vs DSA indexer note) §3.1:
// the DSA indexer's scores can run in FP8; §2.1-§2.2: S_idx = q_idx . k_idx /
// sqrt(d_idx) and the causal block max. "4.1.1 · 监督与联合训练" (selector
// supervision) after eq. (9): a small cutoff margin lets FP8 quantization flip
// candidates, which the churn report of the FP8 path measures.
//
// Scaling: a power of two 2^e per Q_idx row and per 128-token K_idx block, e the
// smallest integer with amax <= 448 * 2^e; the stored byte is the E4M3 value
// nearest to x * 2^-e (ties to the even code). Both scales are powers of two
// and positive, so they commute with the block max: the kernel takes the max
// of the raw FP8 dot products and scales once per (row, block).
//
// gfx950 matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in
// format 0 (E4M3, decoded with bias 7) and unit block scales (E8M0 127): one
// instruction covers d_idx = 64 for a 32-key x 32-row tile, where bf16 needs four.
#include <type_traits>

#include "msa_internal.hpp"

namespace msa {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- quantization

// E4M3 code of y, |y| <= 448 (larger magnitudes saturate to 448): round to
// nearest with ties to the even code, from the fp32 bit fields.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t sgn = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  const uint32_t ua = __float_as_uint(a);
  const int E = (int)(ua >> 23) - 127;
  uint32_t code;
  if (E < -6) {
    // below the smallest normal (2^-6): multiples of 2^-9; code 8 is 2^-6 itself
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t m = ua & 0x7FFFFFu;
    uint32_t keep = m >> 20;
    const uint32_t rest = m & 0xFFFFFu;
    keep += (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u;
    code = ((uint32_t)(E + 7) << 3) + keep;  // a mantissa carry moves to the next binade
  }
  return sgn | code;
}

// smallest e with amax <= 448 * 2^e (0 for amax = 0): amax = f * 2^x with
// f in [0.5, 1) and 448 = 0.875 * 2^9
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int x;
  const float f = frexpf(amax, &x);
  return f <= 0.875f ? x - 9 : x - 8;
}

template <typename T> __device__ __forceinline__ float to_f(T v) { return (float)v; }

// Q_idx rows: 16 lanes per row, DI/16 elements per lane; 4 rows per wave.
template <typename T, int DI>
__global__ void __launch_bounds__(256)
quantize_rows_kernel(const T* __restrict__ x, uint8_t* __restrict__ q8,
                     int32_t* __restrict__ q_exp, int64_t nrows) {
  constexpr int EPL = DI / 16;
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  if (row >= nrows) return;  // whole 16-lane groups
  const T* p = x + row * DI + sub * EPL;
  float v[EPL];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    v[e] = to_f(p[e]);
    amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  const int ex = fp8_scale_exp(amax);
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) packed |= e4m3_rne(ldexpf(v[e], -ex)) << (8 * e);
  if constexpr (EPL == 4) {
    *reinterpret_cast<uint32_t*>(q8 + row * DI + sub * 4) = packed;
  } else {
    *reinterpret_cast<uint16_t*>(q8 + row * DI + sub * 2) = (uint16_t)packed;
  }
  if (sub == 0) q_exp[row] = ex;
}

// K_idx blocks: one workgroup per (batch, 128-token block); 8 elements per
// thread per pass; rows at or past N are neither read nor written.
template <typename T, int DI>
__global__ void __launch_bounds__(256)
quantize_blocks_kernel(const T* __restrict__ x, uint8_t* __restrict__ k8,
                       int32_t* __restrict__ k_exp, int N, int nb) {
  constexpr int CH = 128 * DI / 8;            // 8-element chunks per block
  constexpr int PER = (CH + 255) / 256;
  __shared__ float red[4];
  const int blk = blockIdx.x, b = blockIdx.y;
  const int nrow = min(128, N - blk * 128);
  const size_t base = ((size_t)b * N + (size_t)blk * 128) * DI;
  float v[PER][8];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = threadIdx.x + 256 * u;
    const bool ok = c < CH && c / (DI / 8) < nrow;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[u][e] = ok ? to_f(x[base + (size_t)c * 8 + e]) : 0.0f;
      amax = fmaxf(amax, fabsf(v[u][e]));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int ex = fp8_scale_exp(amax);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = threadIdx.x + 256 * u;
    if (c < CH && c / (DI / 8) < nrow) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= e4m3_rne(ldexpf(v[u][e], -ex)) << (8 * e);
        hi |= e4m3_rne(ldexpf(v[u][4 + e], -ex)) << (8 * e);
      }
      *reinterpret_cast<uint2*>(k8 + base + (size_t)c * 8) = make_uint2(lo, hi);
    }
  }
  if (threadIdx.x == 0) k_exp[(size_t)b * nb + blk] = ex;
}

// ---------------------------------------------------------------- index GEMM + block max
//
// The bf16 kernel's structure with FP8 operands: a workgroup owns RT = 32*CT*NW
// consecutive GEMM rows (QT = RT/HKV queries x all HKV groups) and a chunk of CB
// key blocks; wave w keeps its 32*CT Q8 rows as CT 32-column B operands
// (32 bytes per lane: lane half h holds bytes 32h..32h+31 of its row; zero for
// d_idx = 32, h = 1). Each 128-key K8 block goes global -> registers -> swizzled
// LDS, double-buffered, one barrier per block. D^T = K8_tile (32 keys) x Q8^T,
// so a lane holds 16 keys of one row; the block max is in-lane plus one
// lane-half exchange. Maxima are collected in LDS and scaled on the way out.
template <int DI, int HKV, int NW, int CT, int CB>
__global__ void __launch_bounds__(64 * NW, NW == 8 ? 1 : 8 / NW)
index_blockmax_fp8_kernel(const uint8_t* __restrict__ q8, const int32_t* __restrict__ q_exp,
                          const uint8_t* __restrict__ k8, const int32_t* __restrict__ k_exp,
                          float* __restrict__ M, int N, int Nq, int q_start, int nb,
                          float inv_sqrt_di) {
  constexpr int NT = 64 * NW, RT = 32 * CT * NW, QT = RT / HKV;
  constexpr int CPR = DI / 16;  // 16-byte chunks per row
  constexpr int SWM = CPR - 1;
  constexpr int NCH = 128 * CPR;
  constexpr int KCH = (NCH + NT - 1) / NT;
  constexpr int MST = CB + 1;
  static_assert(CPR == 2 || CPR == 4, "d_idx 32 or 64");
  __shared__ float mbuf[RT * MST];
  __shared__ i32x4 kbuf[2][NCH];

  const int tile = blockIdx.x, b = blockIdx.z;
  const int t0 = tile * QT;
  if (t0 >= Nq) return;
  const int t_last = min(Nq, t0 + QT) - 1;
  const int i_last = q_start + t_last;
  const int kb0 = (int)blockIdx.y * CB;
  if (kb0 * 128 > i_last) return;
  const int kb1 = min(kb0 + CB - 1, i_last >> 7);
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const uint8_t* kbase = k8 + (size_t)b * N * DI;
  i32x4 raw[KCH];
  auto load_raw = [&](int kb) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int x = tid + NT * u;
      if (NCH % NT == 0 || x < NCH) {
        const int r = x / CPR, c = x % CPR;
        const int j = min(kb * 128 + r, N - 1);
        raw[u] = *reinterpret_cast<const i32x4*>(kbase + (size_t)j * DI + c * 16);
      }
    }
  };
  auto store_raw = [&](i32x4* dst) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int x = tid + NT * u;
      if (NCH % NT == 0 || x < NCH) {
        const int r = x / CPR, c = x % CPR;
        dst[r * CPR + (c ^ (idx_swz(r) & SWM))] = raw[u];
      }
    }
  };
  load_raw(kb0);

  i32x8 qf[CT];
  {
    const size_t rbase = (size_t)b * Nq * HKV;
    const size_t rmax = rbase + (size_t)Nq * HKV - 1;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const size_t grow = min(rbase + (size_t)t0 * HKV + 32 * CT * wave + 32 * ct + l32, rmax);
      i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (DI == 64 || h == 0) {
        const i32x4* p = reinterpret_cast<const i32x4*>(q8 + grow * DI + 32 * h);
        lo = p[0];
        hi = p[1];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ct][e] = lo[e];
        qf[ct][4 + e] = hi[e];
      }
    }
  }
  store_raw(kbuf[0]);
  if (kb0 + 1 <= kb1) load_raw(kb0 + 1);
  __syncthreads();

  const int row0 = wave * 32 * CT;
  int i_row[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) i_row[ct] = q_start + t0 + (row0 + 32 * ct + l32) / HKV;

  auto mma_tile = [&](const i32x4* ktile, int kt, f32x16* acc) {
    i32x8 af;
    if (DI == 64 || h == 0) {
      const int rho = 32 * kt + l32;
      const i32x4* rowp = ktile + rho * CPR;
      const int s = idx_swz(rho) & SWM;
      const i32x4 lo = rowp[(2 * h) ^ s], hi = rowp[(2 * h + 1) ^ s];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        af[e] = lo[e];
        af[4 + e] = hi[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) af[e] = 0;
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x16 z;
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = 0.0f;
      acc[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, qf[ct], z, 0, 0, 0, 127, 0, 127);
    }
  };
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
      m[ct] = x;
    }
  };
  auto finish_block = [&](float* m, int kb) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float x = vmax(m[ct], shfl_xor_f(m[ct], 32));
      mbuf[(row0 + 32 * ct + l32) * MST + (kb - kb0 + 1)] = x;
    }
  };

  // MFMAs of key tile kt+1 are issued before the max of tile kt (as in bf16)
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
      store_raw(kbuf[cur ^ 1]);
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
    __syncthreads();
  };
  const int kb_mask = min(max(kb0, (q_start + t0 + 1) >> 7), kb1 + 1);
  int kb = kb0;
  for (; kb < kb_mask; ++kb) block_body(std::false_type(), kb);
  for (; kb <= kb1; ++kb) block_body(std::true_type(), kb);
  reduce_tile(std::true_type(), accB, m, kb1, 3);
  finish_block(m, kb1);
  __syncthreads();

  const int nblk = kb1 - kb0 + 1;
  const size_t grow0 = ((size_t)b * Nq + t0) * HKV;
  for (int x = tid; x < RT * nblk; x += NT) {
    const int row = x / nblk, kk = x - row * nblk;
    const int tq = t0 + row / HKV;
    if (tq >= Nq || kb0 + kk > ((q_start + tq) >> 7)) continue;
    const int ex = q_exp[grow0 + row] + k_exp[(size_t)b * nb + kb0 + kk];
    M[(grow0 + row) * nb + kb0 + kk] = mbuf[row * MST + kk + 1] * ldexpf(inv_sqrt_di, ex);
  }
}

// ---------------------------------------------------------------- launch

template <typename T, int DI>
static hipError_t quantize_run(const Dims& d, const void* qi, const void* ki, uint8_t* q8,
                               int32_t* qe, uint8_t* k8, int32_t* ke, hipStream_t s) {
  const int64_t nrows = d.rows * d.Hkv;
  if (q8 && nrows > 0) {
    quantize_rows_kernel<T, DI><<<(unsigned)((nrows + 15) / 16), 256, 0, s>>>((const T*)qi, q8, qe,
                                                                              nrows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (k8 && d.B > 0 && d.nb > 0) {
    quantize_blocks_kernel<T, DI><<<dim3(d.nb, d.B), 256, 0, s>>>((const T*)ki, k8, ke, d.N, d.nb);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_quantize_fp8(const Dims& d, const void* q_idx, const void* k_idx, uint8_t* q8,
                               int32_t* q_exp, uint8_t* k8, int32_t* k_exp, hipStream_t s) {
  if (d.dtype == MSA_BF16) {
    if (d.DI == 64) return quantize_run<bf16, 64>(d, q_idx, k_idx, q8, q_exp, k8, k_exp, s);
    if (d.DI == 32) return quantize_run<bf16, 32>(d, q_idx, k_idx, q8, q_exp, k8, k_exp, s);
  } else {
    if (d.DI == 64) return quantize_run<float, 64>(d, q_idx, k_idx, q8, q_exp, k8, k_exp, s);
    if (d.DI == 32) return quantize_run<float, 32>(d, q_idx, k_idx, q8, q_exp, k8, k_exp, s);
  }
  return hipErrorInvalidValue;
}

#ifndef MSA_FP8_CB
#define MSA_FP8_CB 32
#endif
#ifndef MSA_FP8_NW
#define MSA_FP8_NW 4
#endif
// 96 GEMM rows per wave (three 32-row B operands per K8 fragment read from
// LDS): 2.31 -> 2.14 ms at the skewed 131072 shape against 64 rows; two
// 384-row workgroups per CU beat one of 768 rows (2.33 ms)
#ifndef MSA_FP8_CT
#define MSA_FP8_CT 3
#endif
constexpr int kFp8Cb = MSA_FP8_CB;

template <int DI, int HKV, int NW, int CT>
static hipError_t fp8_index_launch(const Dims& d, const uint8_t* q8, const int32_t* qe,
                                   const uint8_t* k8, const int32_t* ke, float* M, hipStream_t s) {
  constexpr int QT = 32 * CT * NW / HKV;
  const int ntiles = (d.Nq + QT - 1) / QT;
  const int nchunks = (d.nb + kFp8Cb - 1) / kFp8Cb;
  if (ntiles == 0 || d.B == 0) return hipSuccess;
  index_blockmax_fp8_kernel<DI, HKV, NW, CT, kFp8Cb><<<dim3(ntiles, nchunks, d.B), 64 * NW, 0, s>>>(
      q8, qe, k8, ke, M, d.N, d.Nq, d.q_start, d.nb, (float)(1.0 / std::sqrt((double)DI)));
  return hipGetLastError();
}

template <int DI, int HKV>
static hipError_t fp8_index_nw(const Dims& d, const uint8_t* q8, const int32_t* qe,
                               const uint8_t* k8, const int32_t* ke, float* M, hipStream_t s) {
  // one-wave tiles when a sequence has at most 64 GEMM rows (decode)
  if ((int64_t)d.Nq * HKV <= 64) return fp8_index_launch<DI, HKV, 1, 2>(d, q8, qe, k8, ke, M, s);
  return fp8_index_launch<DI, HKV, MSA_FP8_NW, MSA_FP8_CT>(d, q8, qe, k8, ke, M, s);
}

template <int DI>
static hipError_t fp8_index_hkv(const Dims& d, const uint8_t* q8, const int32_t* qe,
                                const uint8_t* k8, const int32_t* ke, float* M, hipStream_t s) {
  switch (d.Hkv) {
    case 1: return fp8_index_nw<DI, 1>(d, q8, qe, k8, ke, M, s);
    case 2: return fp8_index_nw<DI, 2>(d, q8, qe, k8, ke, M, s);
    case 4: return fp8_index_nw<DI, 4>(d, q8, qe, k8, ke, M, s);
    case 8: return fp8_index_nw<DI, 8>(d, q8, qe, k8, ke, M, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- decode scan
//
// One query per sequence: the register-streamed scan of the bf16 decode step
// (each wave takes 8 consecutive blocks of one sequence and loads a block's
// fragments straight from HBM, one block ahead of its products; no LDS, no
// barrier) on the FP8 operands. Each key tile is the tiled kernel's single
// 32x32x64 instruction on the same bytes (lane l: K8 row 32kt + l%32, bytes
// 32h .. 32h+31, h = l/32; the Hkv index-query rows as B columns, zero past
// Hkv), and the maxima are scaled the same way, so the block scores equal the
// tiled kernel's bit for bit.
template <int DI>
__global__ void __launch_bounds__(256, 2)
decode_index_fp8_kernel(const uint8_t* __restrict__ q8, const int32_t* __restrict__ q_exp,
                        const uint8_t* __restrict__ k8, const int32_t* __restrict__ k_exp,
                        float* __restrict__ M, int N, int q_start, int Hkv, int nb, int chunks,
                        int total_waves, float inv_sqrt_di) {
  constexpr int CB = 8;  // blocks per wave
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int gw = blockIdx.x * 4 + wave;
  if (gw >= total_waves) return;  // the last workgroup may have spare waves
  const int b = gw / chunks, ch = gw % chunks;
  const int i = q_start, L = i / 128;
  const int kb0 = ch * CB;
  if (kb0 > L) return;
  const int kb1 = min(kb0 + CB - 1, L);
  const bool on = DI == 64 || h == 0;  // d_idx = 32: the upper lane half holds zeros
  i32x8 qf;
  {
    i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (on && l32 < Hkv) {
      const i32x4* p = reinterpret_cast<const i32x4*>(q8 + ((size_t)b * Hkv + l32) * DI + 32 * h);
      lo = p[0];
      hi = p[1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[e] = lo[e];
      qf[4 + e] = hi[e];
    }
  }
  const uint8_t* kbase = k8 + (size_t)b * N * DI;
  auto load = [&](int blk, i32x4* f) {  // f[2kt], f[2kt + 1]: the lane's 32 bytes of tile kt
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = min(blk * 128 + 32 * kt + l32, N - 1);  // keys past N are masked
      if (on) {
        const i32x4* p = reinterpret_cast<const i32x4*>(kbase + (size_t)key * DI + 32 * h);
        f[2 * kt] = p[0];
        f[2 * kt + 1] = p[1];
      } else {
        f[2 * kt] = i32x4{0, 0, 0, 0};
        f[2 * kt + 1] = i32x4{0, 0, 0, 0};
      }
    }
  };
  float* mrow = M + (size_t)b * Hkv * nb;  // row r of sequence b: mrow + r * nb
  auto block = [&](int blk, const i32x4* f) {
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      i32x8 af;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        af[e] = f[2 * kt][e];
        af[4 + e] = f[2 * kt + 1][e];
      }
      f32x16 z;
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = 0.0f;
      f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, qf, z, 0, 0, 0, 127, 0, 127);
      if (blk == L) {  // the local block: keys after the query are masked
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (blk * 128 + 32 * kt + drow(e, h) > i) acc[e] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 16; e += 2) m = vmax(vmax(m, acc[e]), acc[e + 1]);
    }
    m = vmax(m, shfl_xor_f(m, 32));
    if (h == 0 && l32 < Hkv) {
      const int ex = q_exp[(size_t)b * Hkv + l32] + k_exp[(size_t)b * nb + blk];
      mrow[(size_t)l32 * nb + blk] = m * ldexpf(inv_sqrt_di, ex);
    }
  };
  i32x4 fa[8], fb[8];
  load(kb0, fa);
  for (int blk = kb0; blk <= kb1; blk += 2) {
    if (blk + 1 <= kb1) load(blk + 1, fb);
    block(blk, fa);
    if (blk + 1 > kb1) break;
    if (blk + 2 <= kb1) load(blk + 2, fa);
    block(blk + 1, fb);
  }
}

template <int DI>
static hipError_t fp8_decode_launch(const Dims& d, const uint8_t* q8, const int32_t* qe,
                                    const uint8_t* k8, const int32_t* ke, float* M,
                                    hipStream_t s) {
  const int L = d.q_start / 128;
  const int chunks = (L + 8) / 8;  // 8 blocks per wave
  const int total = d.B * chunks;
  decode_index_fp8_kernel<DI><<<(unsigned)((total + 3) / 4), 256, 0, s>>>(
      q8, qe, k8, ke, M, d.N, d.q_start, d.Hkv, d.nb, chunks, total,
      (float)(1.0 / std::sqrt((double)DI)));  // the tiled kernel's constant
  return hipGetLastError();
}

hipError_t launch_index_blockmax_fp8(const Dims& d, const uint8_t* q8, const int32_t* q_exp,
                                     const uint8_t* k8, const int32_t* k_exp, float* M,
                                     hipStream_t s) {
  if (d.Nq == 1 && d.rows > 0 && d.Hkv <= 32) {  // one query per sequence: the decode scan
    if (d.DI == 64) return fp8_decode_launch<64>(d, q8, q_exp, k8, k_exp, M, s);
    if (d.DI == 32) return fp8_decode_launch<32>(d, q8, q_exp, k8, k_exp, M, s);
  }
  if (d.DI == 64) return fp8_index_hkv<64>(d, q8, q_exp, k8, k_exp, M, s);
  if (d.DI == 32) return fp8_index_hkv<32>(d, q8, q_exp, k8, k_exp, M, s);
  return hipErrorInvalidValue;
}

}  // namespace msa
