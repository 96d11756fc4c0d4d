/* Host entry points of the seeded input generator (see fx_core.h). OpenMP over elements only:
 * every element is drawn independently, so the thread count never changes a value. */
#include <stdint.h>
#include "fx_core.h"

void fx_fill_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, float sigma,
                         uint16_t* out) {
  uint64_t key = fx_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = fx_normal_bf16(key, offset + (uint64_t)i, sigma);
}

void fx_fill_gain_bf16(uint64_t seed, uint64_t stream, uint64_t n, float sigma, uint16_t* out) {
  uint64_t key = fx_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = fx_gain_bf16(key, (uint64_t)i, sigma);
}

void fx_fill_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, float* out) {
  uint64_t key = fx_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = fx_std_normal(key, offset + (uint64_t)i);
}

void fx_fill_tokens(uint64_t seed, uint64_t stream, uint64_t n, uint32_t vocab, int32_t* out) {
  uint64_t key = fx_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = fx_token(key, (uint64_t)i, vocab);
}

uint64_t fx_splitmix64_next(uint64_t* state) {
  *state += FX_GOLDEN;
  return fx_mix64(*state);
}

/* FNV-1a 64 over bytes: weight checksums recorded with every bench result. */
uint64_t fx_fnv1a64(const uint8_t* p, uint64_t n) {
  uint64_t h = 0xCBF29CE484222325ull;
  for (uint64_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}
