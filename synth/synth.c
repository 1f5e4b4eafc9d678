/*
 * synth.c -- seeded synthetic inputs for the MoE FFN layer.
 *
 * Shared by the tests, the benchmark and the oracle's callers; it holds none
 * of the layer's arithmetic (no quantisation codec, no routing rule, no
 * product).  Every value is a pure function of (seed, stream, index), so any
 * slice of any tensor can be regenerated on its own.
 *
 * Generator: splitmix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants of S. Vigna's
 * reference splitmix64.c).  The state of a stream advances by the golden
 * gamma 0x9e3779b97f4a7c15 and each output is the 64-bit finaliser of the
 * state, so the i-th output is directly mix64(base + (i + 1) * gamma).
 * Normals: Box-Muller (1958) on the two 32-bit halves of one draw.
 */
#include <math.h>
#include <stdint.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
  return mix64((seed << 32) ^ (stream & 0xffffffffULL));
}

static inline uint64_t draw(uint64_t base, uint64_t i) {
  return mix64(base + (i + 1) * 0x9e3779b97f4a7c15ULL);
}

/* (0, 1): 32 high bits, offset by half a step so 0 is never produced. */
static inline double unit_open(uint32_t v) { return ((double)v + 0.5) * (1.0 / 4294967296.0); }

uint64_t synth_draw(uint64_t seed, uint64_t stream, uint64_t i) {
  return draw(stream_base(seed, stream), i);
}

/* out[i] = lo + floor(span * U) with U the high 32 bits / 2^32. */
void synth_bytes(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, uint32_t lo,
                 uint32_t span, uint8_t* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t r = draw(base, offset + (uint64_t)i);
    uint32_t hi = (uint32_t)(r >> 32);
    out[i] = (uint8_t)(lo + (uint32_t)(((uint64_t)hi * span) >> 32));
  }
}

static inline double normal_from(uint64_t r) {
  double u1 = unit_open((uint32_t)(r >> 32));
  double u2 = unit_open((uint32_t)r);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                      float* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * normal_from(draw(base, offset + (uint64_t)i)));
}

/* Normal drawn in double, rounded to fp32, then to bfloat16 (nearest, ties
 * to even) -- the input format of activations and router weights. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                       uint16_t* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float f = (float)(sigma * normal_from(draw(base, offset + (uint64_t)i)));
    union {
      float f;
      uint32_t u;
    } c;
    c.f = f;
    uint32_t u = c.u;
    u += 0x7fffu + ((u >> 16) & 1u);
    out[i] = (uint16_t)(u >> 16);
  }
}

/* Uniform (0, 1) doubles. */
void synth_uniform(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unit_open((uint32_t)(draw(base, offset + (uint64_t)i) >> 32));
}
