/*
 * Seeded synthetic-input generator shared by the GPU path's tests/bench and the CPU oracle.
 *
 * It holds none of the method's arithmetic: it only draws numbers.  Every stream is
 * counter-based, so any slice [offset, offset+count) of a tensor can be produced on its
 * own and in parallel, and the bytes depend only on (seed, stream id, element index).
 *
 *   SplitMix64 (Steele, Lea, Flood: "Fast splittable pseudorandom number generators",
 *   OOPSLA 2014): output i of the stream with key k is mix64(k + (i + 1) * GAMMA).
 *   Uniform (0,1): ((z >> 11) + 0.5) * 2^-53.
 *   Normal: Box-Muller (1958) on the pair (u1, u2) = (U(2p), U(2p+1)), element 2p takes
 *   r*cos(2*pi*u2), element 2p+1 takes r*sin(2*pi*u2), r = sqrt(-2 ln u1), in fp64,
 *   then rounded to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* The key of stream `stream` under `seed`: two SplitMix64 steps so that nearby
 * (seed, stream) pairs give unrelated keys. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed * GAMMA + 0x632BE59BD9B4E019ULL) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline double unit(uint64_t z) { return ((double)(z >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

uint64_t wl_u64(uint64_t seed, uint64_t stream, uint64_t i) { return draw(stream_key(seed, stream), i); }

void wl_uniform_f32(uint64_t seed, uint64_t stream, int64_t offset, int64_t count, float lo, float hi,
                    float* out) {
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    double u = unit(draw(key, (uint64_t)(offset + i)));
    out[i] = (float)((double)lo + ((double)hi - (double)lo) * u);
  }
}

void wl_normal_f32(uint64_t seed, uint64_t stream, int64_t offset, int64_t count, float* out) {
  const uint64_t key = stream_key(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint64_t e = (uint64_t)(offset + i);
    uint64_t p = e >> 1;
    double u1 = unit(draw(key, 2 * p));
    double u2 = unit(draw(key, 2 * p + 1));
    double r = sqrt(-2.0 * log(u1));
    double v = (e & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
    out[i] = (float)v;
  }
}

/* Round fp32 values to the nearest bfloat16 (ties to even) in place, keeping them as fp32
 * bit patterns with the low 16 bits cleared.  This fixes the input's storage type; finite
 * inputs only. */
void wl_round_bf16(float* x, int64_t count) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint32_t u;
    memcpy(&u, &x[i], 4);
    uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
    memcpy(&x[i], &u, 4);
  }
}

/* Multiply the listed channels of a [rows][dim] fp32 block by `factor` in place. */
void wl_scale_channels(float* x, int64_t rows, int dim, const int32_t* channels, int n_channels,
                       float factor) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < n_channels; ++c) x[r * dim + channels[c]] *= factor;
}
