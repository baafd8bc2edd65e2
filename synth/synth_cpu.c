/*
 * synth_cpu.c - host build of the seeded input generator (see synth_rng.h).
 * Fills host buffers with synthetic normal values; rows of a [rows, V] tensor
 * are addressed by their global element index, so any subset of rows can be
 * regenerated on its own.  Holds no part of the loss method.
 */
#include "synth_rng.h"

#include <stddef.h>

enum { SYNTH_F32 = 0, SYNTH_BF16 = 1 };

/* out[i] = N(0, stdev^2) element (offset + i) of stream (seed, stream),
 * i in [0, n), stored as binary32 (dtype 0) or bfloat16 bits (dtype 1). */
int synth_cpu_fill_normal(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                          double stdev, int dtype, void* out) {
  if (n < 0 || out == NULL || (dtype != SYNTH_F32 && dtype != SYNTH_BF16)) return -1;
  const uint64_t key = synth_key(seed, stream);
  if (dtype == SYNTH_F32) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) o[i] = synth_normal_f32(key, offset + (uint64_t)i, stdev);
  } else {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
      o[i] = synth_f32_to_bf16(synth_normal_f32(key, offset + (uint64_t)i, stdev));
  }
  return 0;
}

/* Same as synth_cpu_fill_normal for a list of rows of a [*, row_len] tensor:
 * out row k = generated row rows[k]. */
int synth_cpu_fill_normal_rows(uint64_t seed, uint64_t stream, const int64_t* rows,
                               int64_t nrows, int64_t row_len, double stdev, int dtype,
                               void* out) {
  if (nrows < 0 || row_len < 0 || rows == NULL || out == NULL) return -1;
  if (dtype != SYNTH_F32 && dtype != SYNTH_BF16) return -1;
  const uint64_t key = synth_key(seed, stream);
  const size_t esz = dtype == SYNTH_F32 ? 4 : 2;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nrows; ++k) {
    const uint64_t base = (uint64_t)rows[k] * (uint64_t)row_len;
    char* dst = (char*)out + (size_t)k * (size_t)row_len * esz;
    for (int64_t i = 0; i < row_len; ++i) {
      float f = synth_normal_f32(key, base + (uint64_t)i, stdev);
      if (dtype == SYNTH_F32)
        ((float*)dst)[i] = f;
      else
        ((uint16_t*)dst)[i] = synth_f32_to_bf16(f);
    }
  }
  return 0;
}
