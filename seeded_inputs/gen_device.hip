/*
 * gen_device.hip — device build of the seeded input generator (msa_gen.h), so
 * that tensors of several GiB are produced in place on the GPU. Test and
 * benchmark infrastructure; holds no arithmetic of the method. Bit-identical
 * to gen_host.c by construction (integer hashing and IEEE conversions only).
 * Built with: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off -shared -fPIC.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "msa_gen.h"

enum { GEN_F32 = 0, GEN_BF16 = 1 };

__global__ void __launch_bounds__(256)
msa_gen_fill_kernel(uint64_t key, int dtype, int64_t ncols, int64_t row0, int64_t n_elems,
                    double scale, const double* __restrict__ shift,
                    const uint8_t* __restrict__ flags, void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n_elems; q += stride) {
    const int64_t r = q / ncols;
    const int64_t c = q - r * ncols;
    const uint64_t e = (uint64_t)(row0 + r) * (uint64_t)ncols + (uint64_t)c;
    const double x = msa_gen_normal(key, e);
    const int boosted = flags ? (flags[r] != 0) : 0;
    const double y = msa_gen_affine(x, scale, boosted ? shift[c] : 0.0);
    const float f = (float)y;
    if (dtype == GEN_F32) {
      ((float*)out)[q] = f;
    } else {
      ((uint16_t*)out)[q] = msa_gen_bf16_rne(f);
    }
  }
}

/*
 * Device counterpart of msa_gen_fill_host for a contiguous row range:
 * writes rows [row0, row0+nrows) of the [*, ncols] view to out (device).
 * shift (device, ncols doubles) and flags (device, nrows bytes) may be NULL
 * together. Returns 0, -1 on a bad argument, -2 on a launch error.
 */
extern "C" int msa_gen_fill_device(uint64_t seed, uint32_t tid, int dtype, int64_t ncols,
                                   int64_t row0, int64_t nrows, double scale,
                                   const double* shift, const uint8_t* flags, void* out,
                                   hipStream_t stream) {
  if (!out || ncols <= 0 || nrows < 0 || (dtype != GEN_F32 && dtype != GEN_BF16)) return -1;
  if (flags && !shift) return -1;
  const int64_t n = nrows * ncols;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  msa_gen_fill_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      msa_gen_key(seed, tid), dtype, ncols, row0, n, scale, shift, flags, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
