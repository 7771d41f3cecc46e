/*
 * Seeded synthetic inputs for the offloaded MoE layer step.
 *
 * This module only *makes inputs*: expert weight records, router weights and
 * biases, and token hidden states.  It holds none of the layer's own
 * arithmetic (no routing, no cache bookkeeping, no FFN).  Both the CPU oracle
 * and the GPU library consume the bytes it writes; neither links this file.
 *
 * Randomness: Philox4x32-10, the counter-based generator published by
 * Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
 * (SC'11).  Every value is a pure function of (seed, stream, index), so any
 * expert of any layer can be regenerated on its own and in parallel.
 * Normals come from the Box-Muller transform on pairs of 24-bit uniforms.
 *
 * Counter = (block_lo, block_hi, stream_lo, stream_hi), key = (seed_lo, seed_hi);
 * block b yields normals 4b .. 4b+3 of that stream.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void syn_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void draw4(uint64_t seed, uint64_t stream, uint64_t block, uint32_t r[4]) {
  uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  syn_philox4x32_10(ctr, key, r);
}

static inline void normals4(uint64_t seed, uint64_t stream, uint64_t block, float z[4]) {
  uint32_t r[4];
  draw4(seed, stream, block, r);
  const float two_pi = 6.28318530717958647692f;
  for (int p = 0; p < 2; ++p) {
    float u1 = (float)((r[2 * p] >> 8) + 1u) * (1.0f / 16777216.0f); /* (0, 1] */
    float u2 = (float)(r[2 * p + 1] >> 8) * (1.0f / 16777216.0f);    /* [0, 1) */
    float rad = sqrtf(-2.0f * logf(u1));
    float ang = two_pi * u2;
    z[2 * p] = rad * cosf(ang);
    z[2 * p + 1] = rad * sinf(ang);
  }
}

/* normal number `idx` of a stream */
static inline float normal_at(uint64_t seed, uint64_t stream, uint64_t idx) {
  float z[4];
  normals4(seed, stream, idx >> 2, z);
  return z[idx & 3];
}

/* ---- stream ids ---- */
enum { KIND_EXPERT = 1, KIND_ROUTER_W = 2, KIND_ROUTER_PERM = 3, KIND_AR1 = 4, KIND_IID = 5, KIND_SHARED = 6 };

static uint64_t stream_id(uint64_t kind, uint64_t layer, uint64_t item, uint64_t part) {
  return (kind << 56) | ((layer & 0xFFFFu) << 40) | ((item & 0xFFFFFFFFu) << 8) | (part & 0xFFu);
}

/* ---- narrow encodings used to store generated values ---- */
static inline uint16_t to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* OCP 8-bit E4M3 (the "fn" variant: bias 7, no infinities, 0x7F/0xFF NaN,
 * largest finite 448), round to nearest even, saturating. */
static uint8_t to_e4m3_rne_sat(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  float a = fabsf(v);
  if (isnan(a)) return sign | 0x7F;
  if (a >= 448.0f) return sign | 0x7E;
  if (a < 0.015625f) { /* below 2^-6: subnormal grid of 2^-9 */
    float m = nearbyintf(a * 512.0f); /* 0..8; 8 is the smallest normal, code 0x08 */
    return sign | (uint8_t)m;
  }
  int e2;
  frexpf(a, &e2);
  int E = e2 - 1;                           /* a in [2^E, 2^(E+1)) */
  float m = nearbyintf((ldexpf(a, -E) - 1.0f) * 8.0f);
  if (m == 8.0f) { m = 0.0f; E += 1; }
  if (E > 8 || (E == 8 && m > 6.0f)) return sign | 0x7E;
  return sign | (uint8_t)(((E + 7) << 3) | (int)m);
}

/* ---- public generators ---- */

void syn_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, float sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = sigma * normal_at(seed, stream, first + (uint64_t)i);
}

void syn_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, float sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = to_bf16_rne(sigma * normal_at(seed, stream, first + (uint64_t)i));
}

void syn_encode_bf16(const float* in, uint64_t n, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = to_bf16_rne(in[i]);
}

void syn_encode_e4m3(const float* in, uint64_t n, uint8_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = to_e4m3_rne_sat(in[i]);
}

/* OCP MX v1.0 FP4 (E2M1) code of v: round to nearest, ties to the code with an
 * even mantissa bit, magnitudes above 6 saturate to 6. */
static uint8_t to_e2m1_rne_sat(float v) {
  static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  float a = fabsf(v);
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    float d = fabsf(a - mag[c]), db = fabsf(a - mag[best]);
    if (d < db || (d == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)((v < 0.0f && best != 0 ? 8 : 0) | best);
}

/* weight dtype codes: 0 = fp32, 1 = bf16, 2 = fp8 e4m3 with 128x128 fp32 block
 * scales, 3 = MXFP4 (E2M1 codes, two per byte, E8M0 scale per 32 weights of a row) */
uint64_t syn_record_bytes(int wdt, int H, int F) {
  uint64_t n = 3ull * (uint64_t)H * (uint64_t)F;
  if (wdt == 0) return 4 * n;
  if (wdt == 1) return 2 * n;
  if (wdt == 3) return n / 2 + n / 32;
  return n + 3ull * (uint64_t)(H / 128) * (uint64_t)(F / 128) * 4ull;
}

/* Fill one weight matrix [R][C] (row-major) of one expert into dst.
 * fp8: per 128x128 block, scale = amax/448 and q = e4m3(w/scale); the scales
 * ([R/128][C/128], fp32) go to sdst.
 * MXFP4 (OCP MX v1.0 conversion): per 32 weights of a row, shared exponent
 * floor(log2(amax)) - 2 (2 = E2M1's largest exponent), X = 2^that,
 * q = e2m1(w / X); the E8M0 bytes ([R][C/32]) go to sdst. */
static void fill_matrix(uint64_t seed, uint64_t stream, int R, int C, int wdt, float sigma, uint8_t* dst, void* sdst) {
  if (wdt == 3) {
    uint8_t* sc = (uint8_t*)sdst;
    for (int r = 0; r < R; ++r)
      for (int cb = 0; cb < C / 32; ++cb) {
        uint64_t base = (uint64_t)r * (uint64_t)C + (uint64_t)cb * 32;
        float w[32], amax = 0.0f;
        for (int c = 0; c < 32; c += 4) {
          float z[4];
          normals4(seed, stream, (base + (uint64_t)c) >> 2, z);
          for (int q = 0; q < 4; ++q) {
            w[c + q] = sigma * z[q];
            if (fabsf(w[c + q]) > amax) amax = fabsf(w[c + q]);
          }
        }
        int e2 = 0;
        if (amax > 0.0f) {
          frexpf(amax, &e2); /* amax in [2^(e2-1), 2^e2) */
          e2 = e2 - 1 - 2;
        }
        if (e2 < -127) e2 = -127;
        if (e2 > 127) e2 = 127;
        sc[(uint64_t)r * (uint64_t)(C / 32) + (uint64_t)cb] = (uint8_t)(e2 + 127);
        const float inv = ldexpf(1.0f, -e2);
        for (int c = 0; c < 32; c += 2) {
          uint8_t lo = to_e2m1_rne_sat(w[c] * inv), hi = to_e2m1_rne_sat(w[c + 1] * inv);
          dst[(base + (uint64_t)c) / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
  } else if (wdt == 0) {
    float* o = (float*)dst;
    for (int64_t i = 0; i < (int64_t)R * C; i += 4) {
      float z[4];
      normals4(seed, stream, (uint64_t)i >> 2, z);
      for (int q = 0; q < 4 && i + q < (int64_t)R * C; ++q) o[i + q] = sigma * z[q];
    }
  } else if (wdt == 1) {
    uint16_t* o = (uint16_t*)dst;
    for (int64_t i = 0; i < (int64_t)R * C; i += 4) {
      float z[4];
      normals4(seed, stream, (uint64_t)i >> 2, z);
      for (int q = 0; q < 4 && i + q < (int64_t)R * C; ++q) o[i + q] = to_bf16_rne(sigma * z[q]);
    }
  } else {
    int RB = R / 128, CB = C / 128;
    static const int B = 128;
    float blk[128 * 128];
    for (int rb = 0; rb < RB; ++rb)
      for (int cb = 0; cb < CB; ++cb) {
        float amax = 0.0f;
        for (int r = 0; r < B; ++r) {
          uint64_t base = (uint64_t)(rb * B + r) * (uint64_t)C + (uint64_t)cb * B;
          for (int c = 0; c < B; c += 4) {
            float z[4];
            normals4(seed, stream, (base + (uint64_t)c) >> 2, z);
            for (int q = 0; q < 4; ++q) {
              float w = sigma * z[q];
              blk[r * B + c + q] = w;
              if (fabsf(w) > amax) amax = fabsf(w);
            }
          }
        }
        float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        ((float*)sdst)[rb * CB + cb] = scale;
        for (int r = 0; r < B; ++r) {
          uint8_t* orow = dst + (uint64_t)(rb * B + r) * (uint64_t)C + (uint64_t)cb * B;
          for (int c = 0; c < B; ++c) orow[c] = to_e4m3_rne_sat(blk[r * B + c] / scale);
        }
      }
  }
}

/* Expert records e0 .. e0+count-1 of `layer` into dst (record i at dst + i*stride).
 * Record = [gate F x H | up F x H | down H x F | scales (fp8, MXFP4): gate, up, down].
 * shared != 0 draws the layer's shared expert instead (count must be 1). */
void syn_fill_records(uint64_t seed, int layer, int e0, int count, int H, int F, int wdt, float sigma,
                      uint8_t* dst, uint64_t stride, int shared) {
  uint64_t esz = wdt == 0 ? 4 : (wdt == 1 ? 2 : 1);
  uint64_t mat = wdt == 3 ? (uint64_t)H * (uint64_t)F / 2 : (uint64_t)H * (uint64_t)F * esz;
  uint64_t nsc = (uint64_t)(H / 128) * (uint64_t)(F / 128);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int i = 0; i < count; ++i)
    for (int part = 0; part < 3; ++part) {
      uint8_t* rec = dst + (uint64_t)i * stride;
      uint64_t sid = stream_id(shared ? KIND_SHARED : KIND_EXPERT, (uint64_t)layer, (uint64_t)(e0 + i), (uint64_t)part);
      int R = part < 2 ? F : H, C = part < 2 ? H : F;
      void* sc = wdt == 2   ? (void*)((float*)(rec + 3 * mat) + (uint64_t)part * nsc)
                 : wdt == 3 ? (void*)(rec + 3 * mat + (uint64_t)part * ((uint64_t)H * (uint64_t)F / 32))
                            : NULL;
      fill_matrix(seed, sid, R, C, wdt, sigma, rec + (uint64_t)part * mat, sc);
    }
}

/* Router of `layer`: W[E][H] ~ N(0, sigma) (fp32 or bf16) and bias[E].
 * zipf_s > 0: a seeded permutation ranks the experts 1..E and
 * bias_e = -zipf_s * ln(rank_e), so softmax(bias) is the Zipf(zipf_s) law.
 * zipf_s == 0: bias = 0. */
void syn_router(uint64_t seed, int layer, int E, int H, int wdt, float sigma, double zipf_s, void* w, float* bias) {
  uint64_t sid = stream_id(KIND_ROUTER_W, (uint64_t)layer, 0, 0);
  if (wdt == 0) syn_normal_f32(seed, sid, 0, (uint64_t)E * H, sigma, (float*)w);
  else syn_normal_bf16(seed, sid, 0, (uint64_t)E * H, sigma, (uint16_t*)w);
  if (zipf_s <= 0.0) {
    for (int e = 0; e < E; ++e) bias[e] = 0.0f;
    return;
  }
  int perm[4096];
  for (int e = 0; e < E; ++e) perm[e] = e;
  uint64_t pid = stream_id(KIND_ROUTER_PERM, (uint64_t)layer, 0, 0);
  for (int i = E - 1; i > 0; --i) { /* Fisher-Yates */
    uint32_t r[4];
    draw4(seed, pid, (uint64_t)i, r);
    int j = (int)(((uint64_t)r[0] * (uint64_t)(i + 1)) >> 32);
    int t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
  for (int pos = 0; pos < E; ++pos) bias[perm[pos]] = (float)(-zipf_s * log((double)(pos + 1)));
}

/* Token hidden states for `steps` decode steps of a batch of T sequences,
 * out[steps][T][H] in activation dtype adt (0 fp32, else bf16).
 * rho > 0: AR(1) per sequence, h_0 = eps_0, h_s = rho h_{s-1} + sqrt(1-rho^2) eps_s
 * (unit stationary variance; the state is kept unrounded in double).
 * rho == 0: i.i.d. N(0,1). `tag` separates independent streams. */
void syn_tokens(uint64_t seed, uint64_t tag, int T, int H, int steps, double rho, int adt, void* out) {
  double c = sqrt(1.0 - rho * rho);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    uint64_t sid = stream_id(rho > 0.0 ? KIND_AR1 : KIND_IID, tag, (uint64_t)t, 0);
    for (int i = 0; i < H; ++i) {
      double h = 0.0;
      for (int s = 0; s < steps; ++s) {
        double eps = (double)normal_at(seed, sid, (uint64_t)s * (uint64_t)H + (uint64_t)i);
        h = (rho > 0.0 && s > 0) ? rho * h + c * eps : eps;
        uint64_t o = ((uint64_t)s * T + t) * (uint64_t)H + (uint64_t)i;
        if (adt == 0) ((float*)out)[o] = (float)h;
        else ((uint16_t*)out)[o] = to_bf16_rne((float)h);
      }
    }
  }
}
