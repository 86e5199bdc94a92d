/*
 * Seeded, counter-based synthetic inputs for the AllReduce workloads.
 *
 * This module is shared by the CPU oracle's tests and by the GPU path's tests
 * and bench, and by nothing else.  It holds no part of the reduction: it only
 * turns (seed, stream, rank, element index) into a value of the requested
 * element type, so any window of any rank's buffer can be regenerated exactly.
 *
 * Generator: the splitmix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) applied to a
 * Weyl sequence, used counter-style: draw(key, c) = mix64(key + (c+1)*G).
 * Normals: Box-Muller in binary64 (Box and Muller, 1958), one pair of draws
 * per pair of elements (even element takes the cosine branch, odd the sine).
 * Uniform integers: lo + floor(u * (hi-lo+1)) with u the top 32 bits / 2^32.
 * Rounding to the element type: binary64 -> binary32 by the C conversion
 * (round to nearest even), then binary32 -> binary16 / bfloat16 by
 * round-to-nearest-even on the bit pattern.
 *
 * Element type codes: 0 fp32, 1 fp16, 2 bf16, 3 int32, 4 int8.
 * Distribution codes: 0 uniform integers in [p0, p1], 1 normal N(0, p0) with
 * p0 the standard deviation.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define SYN_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream, uint64_t rank) {
  return mix64(mix64(mix64(seed + SYN_GOLDEN) ^ stream) + rank * SYN_GOLDEN);
}

static inline uint64_t draw(uint64_t key, uint64_t ctr) {
  return mix64(key + (ctr + 1) * SYN_GOLDEN);
}

static inline uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* binary32 -> bfloat16, round to nearest even on the bit pattern. */
static uint16_t syn_to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* binary32 -> binary16, round to nearest even (normals, subnormals, inf). */
static uint16_t syn_to_f16(float f) {
  uint32_t u = f32_bits(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7e00u;
  if (a >= 0x47800000u) return sign | 0x7c00u; /* >= 65536: inf */
  int e = (int)(a >> 23) - 127;
  uint32_t m = (a & 0x7fffffu) | 0x800000u;
  if (a < 0x00800000u) return sign; /* binary32 subnormal: far below half of fp16's least subnormal */
  int shift;
  uint32_t base;
  if (e < -14) { /* result is subnormal or zero: unit 2^-24 */
    shift = -e - 1; /* value / 2^-24 = m * 2^(e+1) */
    base = 0;
    if (shift > 31) return sign;
  } else {
    shift = 13;
    base = (uint32_t)(e + 15) << 10;
    m &= 0x7fffffu;
  }
  uint32_t q = m >> shift;
  uint32_t rem = m & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  return (uint16_t)(sign | (base + q)); /* a carry into the exponent is the correct result */
}

typedef struct {
  void* out;
  int dtype, dist;
  double p0, p1;
  uint64_t key, first, n;
} job_t;

static void store(void* out, int dtype, uint64_t i, double v) {
  switch (dtype) {
    case 0: ((float*)out)[i] = (float)v; break;
    case 1: ((uint16_t*)out)[i] = syn_to_f16((float)v); break;
    case 2: ((uint16_t*)out)[i] = syn_to_bf16((float)v); break;
    case 3: ((int32_t*)out)[i] = (int32_t)v; break;
    case 4: ((int8_t*)out)[i] = (int8_t)v; break;
    default: break;
  }
}

static void run_job(const job_t* j) {
  const double two_pi = 6.283185307179586476925286766559;
  for (uint64_t i = 0; i < j->n; ++i) {
    uint64_t idx = j->first + i;
    double v;
    if (j->dist == 0) {
      double lo = j->p0, hi = j->p1;
      double span = hi - lo + 1.0;
      double u = (double)(draw(j->key, idx) >> 32) * (1.0 / 4294967296.0);
      v = lo + floor(u * span);
      if (v > hi) v = hi;
    } else {
      uint64_t pair = idx >> 1;
      double u1 = ((double)(draw(j->key, 2 * pair) >> 11) + 1.0) * (1.0 / 9007199254740992.0);
      double u2 = (double)(draw(j->key, 2 * pair + 1) >> 11) * (1.0 / 9007199254740992.0);
      double r = sqrt(-2.0 * log(u1));
      double th = two_pi * u2;
      v = j->p0 * ((idx & 1) ? r * sin(th) : r * cos(th));
    }
    store(j->out, j->dtype, i, v);
  }
}

static void* thread_main(void* arg) {
  run_job((const job_t*)arg);
  return NULL;
}

static size_t esize(int dtype) {
  switch (dtype) {
    case 0: return 4;
    case 1: return 2;
    case 2: return 2;
    case 3: return 4;
    case 4: return 1;
    default: return 0;
  }
}

/* Fill out[0..n) with elements first..first+n-1 of the (seed, stream, rank)
 * sequence.  Returns 0, or -1 on a bad argument. */
int synth_fill(void* out, int dtype, int dist, double p0, double p1, uint64_t seed,
               uint64_t stream, uint64_t rank, uint64_t first, uint64_t n, int nthreads) {
  if (esize(dtype) == 0 || (dist != 0 && dist != 1) || (n > 0 && out == NULL)) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < (1u << 16)) nthreads = 1;
  job_t jobs[64];
  pthread_t th[64];
  uint64_t key = synth_key(seed, stream, rank);
  uint64_t chunk = (n + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t b = (uint64_t)t * chunk;
    if (b >= n) break;
    uint64_t e = b + chunk < n ? b + chunk : n;
    jobs[t].out = (char*)out + b * esize(dtype);
    jobs[t].dtype = dtype;
    jobs[t].dist = dist;
    jobs[t].p0 = p0;
    jobs[t].p1 = p1;
    jobs[t].key = key;
    jobs[t].first = first + b;
    jobs[t].n = e - b;
    if (t == 0) continue;
    if (pthread_create(&th[t], NULL, thread_main, &jobs[t]) != 0) {
      run_job(&jobs[t]);
      th[t] = 0;
    }
    started = t;
  }
  run_job(&jobs[0]);
  for (int t = 1; t <= started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
  return 0;
}
