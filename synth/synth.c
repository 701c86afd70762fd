/*
 * Seeded, counter-based generator of synthetic attention inputs.
 *
 * This file holds none of the attention method's arithmetic: it only draws
 * standard normal numbers and applies an affine map (scale, offset) chosen by
 * the caller.  Every draw is a pure function of (seed, config, stream, index),
 * so results do not depend on thread count or evaluation order.
 *
 *   r(i)   = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)       (SplitMix64 step)
 *   u(i)   = ((r(i) >> 11) + 1) * 2^-53                      uniform in (0, 1]
 *   z(i)   = sqrt(-2 ln u(2i)) * cos(2 pi u(2i+1))           Box-Muller, fp64
 *   key    = mix64(mix64(mix64(seed) ^ config) ^ stream)
 *
 * mix64 is the SplitMix64 output function (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).
 */
#include <math.h>
#include <stdint.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t config, uint64_t stream) {
  return mix64(mix64(mix64(seed) ^ config) ^ stream);
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double unit(uint64_t r) {
  return (double)((r >> 11) + 1) * 0x1.0p-53;
}

static inline double normal_at(uint64_t key, int64_t i) {
  const double u1 = unit(draw(key, 2 * (uint64_t)i));
  const double u2 = unit(draw(key, 2 * (uint64_t)i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* Raw 64-bit draws r(start .. start+count-1). */
void synth_u64(uint64_t seed, uint64_t config, uint64_t stream, int64_t start,
               int64_t count, uint64_t* out) {
  const uint64_t key = stream_key(seed, config, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = draw(key, (uint64_t)(start + i));
}

/* Standard normals z(start .. start+count-1) in fp64. */
void synth_normal_f64(uint64_t seed, uint64_t config, uint64_t stream, int64_t start,
                      int64_t count, double* out) {
  const uint64_t key = stream_key(seed, config, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = normal_at(key, start + i);
}

/*
 * out[i] = (float)(sigma * z(i) * chan_scale[i % period] + chan_offset[i % period])
 * for i in [0, count).  chan_scale / chan_offset may be NULL (1 and 0).
 * With a row-major [B, N, H, D] tensor and period = H*D, i % period is the
 * (head, channel) index, so the per-channel terms are shared by all tokens
 * and batch entries.
 */
void synth_fill_f32(uint64_t seed, uint64_t config, uint64_t stream, int64_t count,
                    double sigma, const double* chan_scale, const double* chan_offset,
                    int64_t period, float* out) {
  const uint64_t key = stream_key(seed, config, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    const int64_t c = period > 0 ? i % period : 0;
    double x = sigma * normal_at(key, i);
    if (chan_scale) x *= chan_scale[c];
    if (chan_offset) x += chan_offset[c];
    out[i] = (float)x;
  }
}
