/*
 * Seeded synthetic inputs shared by the CPU oracle tests and the GPU path's tests and bench.
 *
 * This header defines the input generator only; it holds none of the decoder's arithmetic.
 * It compiles as plain C (gcc, for the host library libfx.so) and as HIP device code (for the
 * GPU fill library libfx_gpu.so), so both sides draw bit-identical values.  Build both with
 * -ffp-contract=off: the only floating-point steps are one f32 multiply and one f32 add, and
 * they must round separately on both sides.
 *
 * Generator, from its published definitions:
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 *     OOPSLA 2014): state advances by the golden-ratio increment 0x9E3779B97F4A7C15 and each
 *     output is the state passed through the variant-13 finaliser used by Java's SplittableRandom.
 *     Draw i of a stream with key k is mix(k + (i + 1) * golden), i.e. the (i+1)-th output of a
 *     SplitMix64 sequence seeded with k, so any element can be drawn independently (counter-based).
 *   - Normal variates by the Irwin-Hall sum of twelve uniforms minus six (the classic
 *     approximation to N(0,1): mean 0, variance 1, support +-6).  Each uniform is a 16-bit lane of
 *     a draw, so one variate uses draws 3i, 3i+1, 3i+2 and the sum is an exact integer.
 *   - bf16 by round-to-nearest-even of the f32 value (no NaN or infinity can arise here).
 */
#ifndef FX_CORE_H
#define FX_CORE_H
#include <stdint.h>

#if defined(__HIPCC__)
#define FX_FN __host__ __device__ static inline
#else
#define FX_FN static inline
#endif

#define FX_GOLDEN 0x9E3779B97F4A7C15ull

FX_FN uint64_t fx_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Key of an independent stream: the seed and the stream id pass through the finaliser. */
FX_FN uint64_t fx_stream_key(uint64_t seed, uint64_t stream) {
  return fx_mix64(fx_mix64(seed) ^ fx_mix64(stream + FX_GOLDEN));
}

/* Draw i of the stream: the (i+1)-th SplitMix64 output after seeding with key. */
FX_FN uint64_t fx_draw(uint64_t key, uint64_t i) { return fx_mix64(key + (i + 1ull) * FX_GOLDEN); }

/* Irwin-Hall(12) - 6 from the twelve 16-bit lanes of draws 3i..3i+2; exact in f32. */
FX_FN float fx_std_normal(uint64_t key, uint64_t i) {
  int32_t s = 0;
  for (int j = 0; j < 3; ++j) {
    uint64_t u = fx_draw(key, 3ull * i + (uint64_t)j);
    s += (int32_t)(u & 0xFFFF) + (int32_t)((u >> 16) & 0xFFFF) + (int32_t)((u >> 32) & 0xFFFF) +
         (int32_t)(u >> 48);
  }
  /* 12 * 32767.5 = 393210 is the exact mean of the sum. */
  return (float)(s - 393210) * (1.0f / 65536.0f);
}

FX_FN uint32_t fx_f32_bits(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}

/* f32 -> bf16 bits, round to nearest, ties to even. */
FX_FN uint16_t fx_bf16_rne(float f) {
  uint32_t u = fx_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* N(0, sigma^2) weight element in bf16. */
FX_FN uint16_t fx_normal_bf16(uint64_t key, uint64_t i, float sigma) {
  float z = fx_std_normal(key, i);
  float w = z * sigma;
  return fx_bf16_rne(w);
}

/* Norm gain 1 + N(0, sigma^2) in bf16 (sigma = 0 gives exactly 1). */
FX_FN uint16_t fx_gain_bf16(uint64_t key, uint64_t i, float sigma) {
  float z = fx_std_normal(key, i);
  float d = z * sigma;
  float g = 1.0f + d;
  return fx_bf16_rne(g);
}

/* Uniform token in [0, vocab) by the multiply-shift map of the draw's top 32 bits. */
FX_FN int32_t fx_token(uint64_t key, uint64_t i, uint32_t vocab) {
  uint64_t hi = fx_draw(key, i) >> 32;
  return (int32_t)((hi * (uint64_t)vocab) >> 32);
}

#endif
