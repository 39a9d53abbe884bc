// msa_dense.hpp — host entry points of the gradient of the full-context KL
// (msa_dense.hip), shared with the C ABI layer.
#pragma once

#include "msa_internal.hpp"

namespace msa {

// rows per chunk of the gradient chain (a multiple of 256 query positions)
int dense_grad_chunk(const Dims& d);
// bf16 elements of one chunk of dS rows (row stride N rounded up to 8)
inline int64_t dense_grad_ds_elems(const Dims& d) {
  return (int64_t)d.B * dense_grad_chunk(d) * d.Hkv * (int64_t)((d.N + 7) & ~7);
}
hipError_t launch_kl_dense_grad(const Dims& d, const void* q, const void* k, const void* q_idx,
                                const void* k_idx, const float* lse_main, const float* lse_idx,
                                float* kl_rows, float* mass, float coef, bf16* ds,
                                float* dk_acc, void* dq_idx, void* dk_idx, hipStream_t s);

}  // namespace msa
