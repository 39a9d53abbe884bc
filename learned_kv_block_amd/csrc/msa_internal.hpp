// msa_internal.hpp — shared definitions of the MSA HIP kernels (gfx950).
//
// Matrix-core conventions used by every kernel
// --------------------------------------------
// All dense contractions use the 32x32 MFMA tile: D(32x32, fp32) += A(32x16) * B(16x32).
//   bf16 inputs: one v_mfma_f32_32x32x16_bf16.
//   fp32 inputs: eight v_mfma_f32_32x32x2_f32 over the same 16-wide k range.
// Lane l (0..63), half h = l/32, l32 = l%32:
//   A fragment: A[row = l32][k in K(h)]   (8 values, contiguous in memory)
//   B fragment: B[k in K(h)][col = l32]   (8 values)
//   D element e (0..15): row = 8*(e/4) + 4*h + (e%4), col = l32.
// K(h) is the set of 8 k-indices a lane supplies. A and B use the same set,
// so any fixed assignment of k-indices to (h, element) gives the same sum;
// the kernels use that freedom to feed a D tile straight back as a B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"
#include "msa_timing.h"

namespace msa {

typedef __bf16 bf16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));  // ds_read_tr16_b64 result

template <typename T> struct V8;
template <> struct V8<bf16> { typedef bf16x8 type; };
template <> struct V8<float> { typedef f32x8 type; };
template <typename T> struct V4;
template <> struct V4<bf16> { typedef bf16x4 type; };
template <> struct V4<float> { typedef f32x4 type; };
template <typename T> using vec8 = typename V8<T>::type;
template <typename T> using vec4 = typename V4<T>::type;

__device__ __forceinline__ void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ vec8<T> zero8() {
  vec8<T> z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (T)0.0f;
  return z;
}
template <typename T> __device__ __forceinline__ vec8<T> ld8(const T* p) {
  return *reinterpret_cast<const vec8<T>*>(p);
}
template <typename T> __device__ __forceinline__ void st8(T* p, const vec8<T>& v) {
  *reinterpret_cast<vec8<T>*>(p) = v;
}
// Streaming (non-temporal) access for data touched once.
template <typename T> __device__ __forceinline__ vec8<T> ld8_nt(const T* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const vec8<T>*>(p));
}
template <typename T> __device__ __forceinline__ void st8_nt(T* p, const vec8<T>& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<vec8<T>*>(p));
}
template <typename T> __device__ __forceinline__ vec4<T> ld4(const T* p) {
  return *reinterpret_cast<const vec4<T>*>(p);
}
template <typename T> __device__ __forceinline__ void st4(T* p, const vec4<T>& v) {
  *reinterpret_cast<vec4<T>*>(p) = v;
}
template <typename T> __device__ __forceinline__ T cvt(float x) { return (T)x; }

// D-tile row of element e for lane half h.
__device__ __forceinline__ constexpr int drow(int e, int h) { return 8 * (e / 4) + 4 * h + (e % 4); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// NaN-propagating maximum. Unlike fmaxf it needs no quieting of its operands,
// and chains m = vmax(vmax(m, a), b) become one v_maximum3_f32 per two inputs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ---- swizzled [128][D] bf16 K/V tiles in LDS (16-byte chunk c of row rho at c ^ swz(rho))
// K fragment reads touch one chunk of 16 consecutive rows; the transposing V
// reads touch 4 chunks of 4 consecutive rows. Each tile gets its own XOR
// pattern so that both access shapes spread over all 64 LDS banks.
template <int D>
__device__ __forceinline__ int swz_k(int rho) {
  return rho & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int rho) {
  return D == 128 ? 4 * (rho & 3) : 2 * (rho & 3);
}
// element offset of (row, col) in a swizzled [128][D] tile
template <int D, bool IS_V>
__device__ __forceinline__ int tile_off(int rho, int col) {
  const int sw = IS_V ? swz_v<D>(rho) : swz_k<D>(rho);
  return rho * D + 8 * ((col >> 3) ^ sw) + (col & 7);
}

// ---- LDS tiles of 16-byte chunks: chunk c of row r sits at c ^ (idx_swz(r) & M),
// M = min(chunks per row, 8) - 1, so that 32-row fragment reads and row-wise
// stores spread over all banks.
__device__ __forceinline__ int idx_swz(int r) { return r ^ (r >> 3); }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

template <typename T, int CPR>
__device__ __forceinline__ vec8<T> lds_frag(const i32x4* tile, int r, int c0) {
  constexpr int M = (CPR < 8 ? CPR : 8) - 1;
  const i32x4* row = tile + r * CPR;
  const int s = idx_swz(r) & M;
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

// The persistent kernels' split of the work items over a grid of workgroups
// (a multiple of 8; workgroup w runs on XCD w % 8): each XCD gets an equal
// contiguous share, cut into equal contiguous ranges of its workgroups in
// order. owner(it) is the workgroup whose range holds item it (total > 0).
struct ItemSplit {
  int total, nwg_x, per_x, per_wg;
  __device__ ItemSplit(int total_items, int grid)
      : total(total_items), nwg_x(grid / 8), per_x((total_items + 7) / 8),
        per_wg((per_x + nwg_x - 1) / nwg_x) {}
  __device__ void range(int wg, int* i0, int* i1) const {
    const int x = wg & 7, gx = wg >> 3;
    const int x0 = x * per_x, x1 = min(total, x0 + per_x);
    *i0 = x0 + gx * per_wg;
    *i1 = min(x1, *i0 + per_wg);
  }
  __device__ int owner(int it) const {
    const int x = it / per_x;
    return ((it - x * per_x) / per_wg) * 8 + x;
  }
};

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------- host side

struct Dims {
  int B, N, Nq, q_start, Hq, Hkv, G, D, DI, Bk, K, nb, dtype;
  int64_t rows;     // B * Nq query rows
  int64_t slots;    // B * Nq * Hkv * K (selection slots)
  int64_t buckets;  // B * Hkv * nb
  int64_t entries_max;  // upper bound of used slots
  int64_t items_max;    // upper bound of attention work items
  int nwin;             // query windows of kQueryWindow rows per sequence
  int qt;               // queries per work item: 256/G (bf16 attention), else 128/G
  int num_cus;          // compute units of the device (persistent grids)
};

// Work items are ordered by (batch, group, query window, block): the rows of
// one window of kQueryWindow queries are revisited by many consecutive items
// and stay in L2 / Infinity Cache. Bucket id = ((b*Hkv + r)*nwin + w)*nb + blk.
#ifndef MSA_QUERY_WINDOW
#define MSA_QUERY_WINDOW (1 << 30)  // one window: plain (batch, group, block) order
#endif
constexpr int kQueryWindow = MSA_QUERY_WINDOW;
// Work cost of the persistent attention's items for the range split: kItemCost
// units per item and kItemStartCost more for the first item of a bucket, whose K/V
// tiles a workgroup must load behind a barrier and a full drain of its memory
// operations. Per-workgroup timings under a split by item count showed the late
// blocks of each group (small buckets, up to 20x more K/V reloads per workgroup)
// finishing last; at the skewed 131072-token step, start/item cost ratios of
// 0 (count split), 0.25, 0.5, 1, 1.5, 2, 4, 8, 16 gave attention times of
// 11.66, 11.58, 11.31, 11.12, 11.17, 11.51, 11.74, 12.29, 12.99 ms.
#ifndef MSA_ITEM_START_COST
#define MSA_ITEM_START_COST 1
#endif
#ifndef MSA_ITEM_COST
#define MSA_ITEM_COST 1
#endif
constexpr int kItemStartCost = MSA_ITEM_START_COST;
constexpr int kItemCost = MSA_ITEM_COST;
constexpr int kMaxSplit = 2048;  // workgroup ranges the balanced split can describe

// Backward: at most this many persistent workgroups (a multiple of 8; two per
// CU on 256 CUs). The dK/dV (and dk_idx) sums of a run of items of one bucket
// go to fp32 slabs of 128 keys: one per bucket, plus two per workgroup for the
// runs it shares with a neighbour.
constexpr int kBwdMaxGrid = 512;

// Workspace of the attention and KL calls (bucketing + partials).
struct AttnWs {
  int32_t* counts;    // [buckets]
  int32_t* offsets;   // [buckets + 1]
  int32_t* cursor;    // [buckets]
  int32_t* item_off;  // [buckets + 1]
  int32_t* totals;    // [4]: entries, items, work cost, grid of the balanced split (0: none)
  int4* items;        // [items_max]: bucket, first entry, count, work cost before it
  int32_t* entries;   // [entries_max]: (t << 6) | slot
  int32_t* chunk_e;   // [buckets / 4096 + 1]: entry count per scan chunk
  int32_t* chunk_i;   // [buckets / 4096 + 1]: item count per scan chunk
  int32_t* chunk_c;   // [buckets / 4096 + 1]: work cost per scan chunk
  int32_t* cost_off;  // [buckets + 1]: exclusive prefix of the work cost of each bucket
  int32_t* wg_start;  // [kMaxSplit + 1]: first item of each balanced workgroup range
  // [entries_max] or null: when set, bucketing also writes the entries here in
  // row order inside each bucket (the order the backward sums in)
  int32_t* sorted;
};

// Launch hooks around each kernel (kernel ids MSA_K_* of msa_timing.h). The
// product library links no-ops (msa_prof_off.cpp); the measurement build links
// the event-recording hook (msa_timing.cpp).
void prof_before(int kernel, hipStream_t s);
void prof_after(int kernel, hipStream_t s);

// ---------------------------------------------------------------- launchers (return hipError_t)
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);

hipError_t launch_index_blockmax(const Dims& d, const void* q_idx, const void* k_idx, float* M,
                                 hipStream_t s);
hipError_t launch_topk(const Dims& d, const float* M, int32_t* ids, float* margin, hipStream_t s);
// the tiled index kernel that also writes each causal block's log-sum-exp to BL
hipError_t launch_index_block_lse(const Dims& d, const void* q_idx, const void* k_idx, float* M,
                                  float* BL, hipStream_t s);
// bf16 with one query per sequence: a register-streamed scan of K_idx whose block
// scores are bit-identical to those of the tiled index kernel
bool decode_index_supported(const Dims& d);
hipError_t launch_decode_index(const Dims& d, const void* q_idx, const void* k_idx, float* M,
                               hipStream_t s);

// split_grid > 0: also cut the items into split_grid cost-balanced contiguous
// ranges (wg_start, totals[3] = split_grid) for a persistent kernel of that grid
hipError_t launch_bucketing(const Dims& d, const int32_t* ids, const AttnWs& w, bool skip_local,
                            hipStream_t s, int split_grid = 0);
// grid of the persistent bf16 attention kernel for d
unsigned attn_pipe_grid(const Dims& d);
hipError_t launch_sparse_attn(const Dims& d, const void* q, const void* k, const void* v,
                              const AttnWs& w, void* opart, float* lpart, hipStream_t s);
hipError_t launch_combine(const Dims& d, const void* opart, const float* lpart,
                          const int32_t* ids, void* out, float* lse, hipStream_t s);
// bf16 with one query per sequence (a decode step): query-outer attention of each
// (sequence, group) over its selected blocks, written straight to out / lse
bool decode_attn_supported(const Dims& d);
hipError_t launch_decode_attn(const Dims& d, const void* q, const void* k, const void* v,
                              const int32_t* ids, void* out, float* lse, hipStream_t s);
// bf16: attention of each row's local block (query-outer) fused with the combine
hipError_t launch_combine_local(const Dims& d, const void* q, const void* k, const void* v,
                                const void* opart, const float* lpart, const int32_t* ids,
                                void* out, float* lse, hipStream_t s);

hipError_t launch_attn_bwd(const Dims& d, const void* q, const void* k, const void* v,
                           const int32_t* ids, const void* out, const float* lse,
                           const void* dout, const AttnWs& w, float* drow, void* dqpart,
                           float* slabs, void* dq, void* dk, void* dv, hipStream_t s);
hipError_t launch_idx_bwd(const Dims& d, const void* qi, const void* ki, const int32_t* ids,
                          const float* dl, float coef, const AttnWs& w, float* dqpart,
                          float* slabs, void* dq, void* dk, hipStream_t s);
hipError_t launch_kl(const Dims& d, const void* q, const void* k, const void* q_idx,
                     const void* k_idx, const int32_t* ids, const float* lse_main,
                     const AttnWs& w, float* idx_stats, float* lse_idx, float* kl_part,
                     float* kl_rows, float* kl_block_sums, float* kl_mean, float* dlogits,
                     hipStream_t s);

// warm-up stage on the full causal context
hipError_t launch_dense_lse(const Dims& d, bool index_branch, const void* q, const void* k,
                            float* lse, hipStream_t s);
hipError_t launch_kl_dense(const Dims& d, const void* q, const void* k, const void* q_idx,
                           const void* k_idx, const float* lse_main, const float* lse_idx,
                           float* kl_rows, float* mass, hipStream_t s);
hipError_t launch_recall(const Dims& d, const float* mass, const int32_t* ids, float* brec,
                         float* srec, hipStream_t s);
hipError_t launch_mean(const float* x, int64_t n, float* out, hipStream_t s);

// FP8 (E4M3) index branch
hipError_t launch_quantize_fp8(const Dims& d, const void* q_idx, const void* k_idx, uint8_t* q8,
                               int32_t* q_exp, uint8_t* k8, int32_t* k_exp, hipStream_t s);
hipError_t launch_index_blockmax_fp8(const Dims& d, const uint8_t* q8, const int32_t* q_exp,
                                     const uint8_t* k8, const int32_t* k_exp, float* M,
                                     hipStream_t s);

}  // namespace msa
