/*
 * msa_gen.h — seeded, counter-based synthetic input generator.
 *
 * Test and benchmark infrastructure shared by the CPU oracle side and the GPU
 * side. It holds no arithmetic of the attention method: it only turns
 * (seed, tensor id, element index) into a number and rounds it to the storage
 * type. Any element can be regenerated on its own, so a checker can rebuild
 * exactly the rows it samples, and the host and device builds of this header
 * give identical bits (integer hashing, one exact int->double conversion, one
 * IEEE double multiply-add, IEEE round-to-nearest-even conversions only).
 *
 * Definition of element e of tensor (seed, tid):
 *   key   = mix64((seed << 8) | tid)
 *   h_m   = mix64(key + 6*e + m),  m = 0..5           (six 64-bit hashes)
 *   S     = sum of the twelve 32-bit halves of h_0..h_5 (an integer < 2^36)
 *   x     = (S + 6 - 6*2^32) * 2^-32                   (exact in double)
 * x is the Irwin-Hall sum of twelve uniforms on (0,1) minus 6: mean 0,
 * variance 1, support (-6, 6), the textbook approximation of N(0,1).
 *   y     = x * scale + shift                           (double, one FMA-free
 *                                                        multiply then add)
 *   fp32  = (float) y                                   (round to nearest even)
 *   bf16  = round-to-nearest-even of the fp32 value to its top 16 bits
 *
 * mix64 is the SplitMix64 output function (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), with the constants
 * of the public-domain splitmix64 reference by S. Vigna.
 */
#ifndef MSA_GEN_H
#define MSA_GEN_H

#include <stdint.h>

#if defined(__HIPCC__)
#define MSA_GEN_FN __host__ __device__ static inline
#else
#define MSA_GEN_FN static inline
#endif

MSA_GEN_FN uint64_t msa_gen_mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

MSA_GEN_FN uint64_t msa_gen_key(uint64_t seed, uint32_t tid) {
  return msa_gen_mix64((seed << 8) | (uint64_t)(tid & 0xffu));
}

/* Irwin-Hall(12) - 6 for element e of the stream `key`. */
MSA_GEN_FN double msa_gen_normal(uint64_t key, uint64_t e) {
  uint64_t s = 0;
  for (int m = 0; m < 6; ++m) {
    uint64_t h = msa_gen_mix64(key + 6ull * e + (uint64_t)m);
    s += (h & 0xffffffffull) + (h >> 32);
  }
  int64_t n = (int64_t)s + 6 - 6ll * 4294967296ll;
  /* 2^-32 is exact; so is the product (|n| < 2^36). */
  return (double)n * 2.3283064365386962890625e-10;
}

/* One raw 64-bit hash of element e (used for seeded bits and integer draws). */
MSA_GEN_FN uint64_t msa_gen_bits(uint64_t key, uint64_t e) {
  return msa_gen_mix64(key + e);
}

MSA_GEN_FN uint32_t msa_gen_f32_bits(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}

/* Round-to-nearest-even of a finite fp32 value to bf16 (its top 16 bits). */
MSA_GEN_FN uint16_t msa_gen_bf16_rne(float f) {
  uint32_t u = msa_gen_f32_bits(f);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* y = x*scale + shift, evaluated as two separately rounded double operations.
 * Every file that includes this header is built with -ffp-contract=off so that
 * neither compiler fuses the pair into one FMA. */
MSA_GEN_FN double msa_gen_affine(double x, double scale, double shift) {
  double p = x * scale;
  return p + shift;
}

#endif /* MSA_GEN_H */
