/*
 * Seeded synthetic input generator shared by the tests, the bench and the
 * oracle harness.  It holds no decode arithmetic: it only draws numbers.
 *
 * Counter-based generator: Philox4x32-10 as defined by Salmon, Moraes, Dror
 * and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).  Element i
 * of a tensor is a pure function of (seed, stream, i), so every draw is
 * independent of thread count and host.  Normals come from the Box-Muller
 * transform of two 32-bit uniforms; bf16 outputs are rounded to nearest even.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static inline uint32_t mulhilo(uint32_t a, uint32_t b, uint32_t* hi) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  return (uint32_t)p;
}

/* Philox4x32 with 10 rounds: counter ctr[4], key (k0, k1). */
static void philox4x32_10(const uint32_t ctr_in[4], uint32_t k0, uint32_t k1, uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, hi1;
    uint32_t lo0 = mulhilo(0xD2511F53u, c0, &hi0);
    uint32_t lo1 = mulhilo(0xCD9E8D57u, c2, &hi1);
    uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void block4(uint64_t seed, uint64_t stream, uint64_t j, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
  philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), out);
}

/* Four normals per Philox block: Box-Muller on (x0,x1) and (x2,x3). */
static inline void normal4(uint64_t seed, uint64_t stream, uint64_t j, double z[4]) {
  uint32_t x[4];
  block4(seed, stream, j, x);
  const double two_pi = 6.283185307179586476925286766559;
  for (int p = 0; p < 2; ++p) {
    double u1 = ((double)x[2 * p] + 1.0) * (1.0 / 4294967296.0);  /* (0, 1] */
    double u2 = (double)x[2 * p + 1] * (1.0 / 4294967296.0);       /* [0, 1) */
    double rad = sqrt(-2.0 * log(u1));
    z[2 * p] = rad * cos(two_pi * u2);
    z[2 * p + 1] = rad * sin(two_pi * u2);
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = {f};
  if ((v.u & 0x7F800000u) == 0x7F800000u && (v.u & 0x007FFFFFu)) return (uint16_t)((v.u >> 16) | 0x40u);
  uint32_t bias = 0x7FFFu + ((v.u >> 16) & 1u);
  return (uint16_t)((v.u + bias) >> 16);
}

/* out[i] = bf16(mean + std * N(0,1)) for i in [0, n) of the (seed, stream) tensor. */
void synth_normal_bf16(uint16_t* out, size_t n, uint64_t seed, uint64_t stream, double mean, double stdv) {
  size_t nb = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (size_t j = 0; j < nb; ++j) {
    double z[4];
    normal4(seed, stream, j, z);
    for (int c = 0; c < 4; ++c) {
      size_t i = j * 4 + c;
      if (i < n) out[i] = f32_to_bf16_rne((float)(mean + stdv * z[c]));
    }
  }
}

void synth_normal_f32(float* out, size_t n, uint64_t seed, uint64_t stream, double mean, double stdv) {
  size_t nb = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (size_t j = 0; j < nb; ++j) {
    double z[4];
    normal4(seed, stream, j, z);
    for (int c = 0; c < 4; ++c) {
      size_t i = j * 4 + c;
      if (i < n) out[i] = (float)(mean + stdv * z[c]);
    }
  }
}

/* out[i] = bf16(lo + (hi - lo) * U[0,1)). */
void synth_uniform_bf16(uint16_t* out, size_t n, uint64_t seed, uint64_t stream, double lo, double hi) {
  size_t nb = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (size_t j = 0; j < nb; ++j) {
    uint32_t x[4];
    block4(seed, stream, j, x);
    for (int c = 0; c < 4; ++c) {
      size_t i = j * 4 + c;
      if (i < n) out[i] = f32_to_bf16_rne((float)(lo + (hi - lo) * ((double)x[c] * (1.0 / 4294967296.0))));
    }
  }
}

/* Raw 32-bit draws (for token ids, context lengths, permutations). */
void synth_u32(uint32_t* out, size_t n, uint64_t seed, uint64_t stream) {
  size_t nb = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (size_t j = 0; j < nb; ++j) {
    uint32_t x[4];
    block4(seed, stream, j, x);
    for (int c = 0; c < 4; ++c) {
      size_t i = j * 4 + c;
      if (i < n) out[i] = x[c];
    }
  }
}

/* Random OCP E4M3 fp8 weight codes, one 32-bit draw x each: sign = bit 31, mantissa = bits 28-30,
 * exponent field 14 - t with t the number of trailing zero bits of x (capped at 14), so field e has
 * probability 2^(e-15) -- a magnitude spread falling off by halves below the top, as a zero-mean
 * bell-shaped draw does -- reaching zero and subnormal codes at field 0 and never field 15 (no
 * NaN codes).  The generator only assembles bits; it decodes nothing. */
void synth_fp8_codes(uint8_t* out, size_t n, uint64_t seed, uint64_t stream) {
  size_t nb = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (size_t j = 0; j < nb; ++j) {
    uint32_t x[4];
    block4(seed, stream, j, x);
    for (int c = 0; c < 4; ++c) {
      size_t i = j * 4 + c;
      if (i >= n) continue;
      uint32_t t = (uint32_t)__builtin_ctz(x[c] | (1u << 14));
      out[i] = (uint8_t)(((x[c] >> 31) << 7) | ((14u - t) << 3) | ((x[c] >> 28) & 7u));
    }
  }
}

/* Philox block for known-answer tests of the generator itself. */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  philox4x32_10(ctr, key[0], key[1], out);
}
