/*
 * gen_host.c — host build of the seeded input generator (msa_gen.h).
 * Test and benchmark infrastructure; holds no arithmetic of the method.
 * Built with: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include "msa_gen.h"

enum { GEN_F32 = 0, GEN_BF16 = 1 };

/*
 * View the tensor as [total_rows, ncols]. Writes `nrows` rows: row rows[q]
 * (or row0 + q when rows == NULL) goes to out[q*ncols ...]. Element (row, c)
 * is generator element e = row*ncols + c. Where flags != NULL and flags[q] != 0
 * the value gets shift[c] added before rounding.
 * Returns 0, or -1 on a bad argument.
 */
int msa_gen_fill_host(uint64_t seed, uint32_t tid, int dtype, int64_t ncols,
                      const int64_t* rows, int64_t row0, int64_t nrows,
                      double scale, const double* shift, const uint8_t* flags,
                      void* out, int nthreads) {
  if (!out || ncols <= 0 || nrows < 0 || (dtype != GEN_F32 && dtype != GEN_BF16)) return -1;
  if (flags && !shift) return -1;
  const uint64_t key = msa_gen_key(seed, tid);
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t q = 0; q < nrows; ++q) {
    const int64_t row = rows ? rows[q] : row0 + q;
    const int boosted = flags ? (flags[q] != 0) : 0;
    for (int64_t c = 0; c < ncols; ++c) {
      const uint64_t e = (uint64_t)row * (uint64_t)ncols + (uint64_t)c;
      const double x = msa_gen_normal(key, e);
      const double y = msa_gen_affine(x, scale, boosted ? shift[c] : 0.0);
      const float f = (float)y;
      if (dtype == GEN_F32) {
        ((float*)out)[q * ncols + c] = f;
      } else {
        ((uint16_t*)out)[q * ncols + c] = msa_gen_bf16_rne(f);
      }
    }
  }
  return 0;
}

/* out[q] = msa_gen_bits(key(seed, tid), e) with e = rows[q] (or e0 + q when rows == NULL). */
int msa_gen_bits_host(uint64_t seed, uint32_t tid, const int64_t* rows, uint64_t e0, int64_t n,
                      uint64_t* out) {
  if (!out || n < 0) return -1;
  const uint64_t key = msa_gen_key(seed, tid);
  for (int64_t q = 0; q < n; ++q)
    out[q] = msa_gen_bits(key, rows ? (uint64_t)rows[q] : e0 + (uint64_t)q);
  return 0;
}

/* out[q] = msa_gen_normal(key(seed, tid), e0 + q) in double, before any scaling or rounding. */
int msa_gen_normals_host(uint64_t seed, uint32_t tid, uint64_t e0, int64_t n, double* out) {
  if (!out || n < 0) return -1;
  const uint64_t key = msa_gen_key(seed, tid);
  for (int64_t q = 0; q < n; ++q) out[q] = msa_gen_normal(key, e0 + (uint64_t)q);
  return 0;
}
