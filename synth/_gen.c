/*
 * Seeded synthetic-input generator (counter-based, multithreaded).
 *
 * Holds none of the decode method's arithmetic: it only draws the random
 * tensors (weights, seeded K/V history, int4 codes) that both the CPU oracle
 * and the GPU path consume. Every element is a pure function of
 * (seed, stream, index), so any slice can be regenerated independently and
 * the result does not depend on the thread count.
 *
 * Hash: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), applied to a
 * counter. Normals: Box-Muller transform on two 32-bit uniforms from one
 * 64-bit hash; element 2i takes the cosine branch and 2i+1 the sine branch
 * of hash i. bf16 rounding is round-to-nearest-even of the fp32 value.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t sm64_mix(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27; z *= 0x94D049BB133111EBULL;
  z ^= z >> 31; return z;
}

static inline uint64_t counter_hash(uint64_t key, uint64_t i) {
  return sm64_mix(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return sm64_mix(sm64_mix(seed ^ 0x6A09E667F3BCC909ULL) + sm64_mix(stream + 0x3C6EF372FE94F82BULL));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static inline void normal_pair(uint64_t h, double* z0, double* z1) {
  /* u1 in (0,1], u2 in [0,1) */
  double u1 = ((double)(h >> 32) + 1.0) * (1.0 / 4294967296.0);
  double u2 = (double)(h & 0xFFFFFFFFu) * (1.0 / 4294967296.0);
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925 * u2;
  *z0 = r * cos(a);
  *z1 = r * sin(a);
}

typedef struct {
  int kind;            /* 0 normal bf16, 1 normal f32, 2 uniform u32 below n_range, 3 uniform f64, 4 uniform u8 below n_range */
  uint64_t key, begin, end, offset;
  double mean, std;
  uint64_t n_range;
  void* out;
} job_t;

/* Element e of the output is element (offset + e) of the stream. */
static void run_range(const job_t* j) {
  uint64_t i = j->begin;
  const uint64_t o = j->offset;
  if (j->kind == 0 || j->kind == 1) {
    for (; i < j->end; ++i) {
      uint64_t c = o + i;
      double z0, z1;
      normal_pair(counter_hash(j->key, c >> 1), &z0, &z1);
      double z = (c & 1) ? z1 : z0;
      float v = (float)(j->mean + j->std * z);
      if (j->kind == 0) ((uint16_t*)j->out)[i] = f32_to_bf16_rne(v);
      else ((float*)j->out)[i] = v;
    }
  } else if (j->kind == 2 || j->kind == 4) {
    for (; i < j->end; ++i) {
      uint64_t h = counter_hash(j->key, o + i);
      /* multiply-shift reduction to [0, n_range) (Lemire) on the high 32 bits */
      uint32_t r = (uint32_t)(((h >> 32) * j->n_range) >> 32);
      if (j->kind == 2) ((uint32_t*)j->out)[i] = r;
      else ((uint8_t*)j->out)[i] = (uint8_t)r;
    }
  } else {
    for (; i < j->end; ++i) {
      uint64_t h = counter_hash(j->key, o + i);
      ((double*)j->out)[i] = (double)(h >> 11) * (1.0 / 9007199254740992.0);
    }
  }
}

static void* thread_main(void* arg) { run_range((const job_t*)arg); return 0; }

static void run(int kind, uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, double mean,
                double std, uint64_t n_range, void* out, int threads) {
  job_t jobs[256]; pthread_t tid[256];
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (n < (uint64_t)threads * 65536u) threads = 1;
  uint64_t key = stream_key(seed, stream);
  uint64_t chunk = (n + threads - 1) / threads;
  chunk = (chunk + 1) & ~(uint64_t)1;
  for (int t = 0; t < threads; ++t) {
    uint64_t b = (uint64_t)t * chunk, e = b + chunk;
    if (b > n) b = n;
    if (e > n) e = n;
    jobs[t] = (job_t){kind, key, b, e, offset, mean, std, n_range, out};
  }
  for (int t = 1; t < threads; ++t) pthread_create(&tid[t], 0, thread_main, &jobs[t]);
  run_range(&jobs[0]);
  for (int t = 1; t < threads; ++t) pthread_join(tid[t], 0);
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, double mean,
                       double std, uint16_t* out, int threads) {
  run(0, seed, stream, offset, n, mean, std, 0, out, threads);
}
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, double mean,
                      double std, float* out, int threads) {
  run(1, seed, stream, offset, n, mean, std, 0, out, threads);
}
void synth_uniform_u32(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, uint64_t n_range,
                       uint32_t* out, int threads) {
  run(2, seed, stream, offset, n, 0, 0, n_range, out, threads);
}
void synth_uniform_u8(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, uint64_t n_range,
                      uint8_t* out, int threads) {
  run(4, seed, stream, offset, n, 0, 0, n_range, out, threads);
}
void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, double* out,
                       int threads) {
  run(3, seed, stream, offset, n, 0, 0, 0, out, threads);
}
