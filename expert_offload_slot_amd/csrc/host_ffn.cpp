// Expert FFN on the host CPU for cold experts: the misses of a call are
// computed from their records in host DRAM instead of crossing the host link.
//
// npu-offload README, intro, "Results" (where the time goes: the CPU's cold
// experts are bound by DRAM bandwidth) and "Architecture" (hot experts on the
// accelerator and cold experts on the host run in parallel per layer; only
// activations cross PCIe, weights never move).
//
// Work is split by weight rows, so every weight byte is read from DRAM once per
// call and meets every token routed to its expert while it sits in cache:
//   phase 1: (cold expert, block of F rows)  gate/up dot products, h = silu(g) * u
//   phase 2: (cold expert, block of H rows)  down dot products into the output rows
// Dot products accumulate in fp32 over 16 interleaved lanes: with AVX-512 (picked
// when the library loads) two weight rows at a time, one register per (row,
// token), fused multiply-adds, codes widened in registers; otherwise the same sums
// in portable C++.  A persistent
// pool of worker threads claims blocks from an atomic counter.
#include <immintrin.h>
#include <math.h>
#include <sched.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/moe_offload.h"
#include "host_ffn.h"

namespace moe {
namespace {


// ---------------------------------------------------------------- weight formats
// e4m3 ("fn": bias 7, no infinities, S.1111.111 is NaN) and E2M1 values, built
// from their bit fields when the library loads.
struct Tables {
  float e4m3[256];
  float e2m1[16];
  // the bf16 bits of the 128 e4m3 magnitudes (every e4m3 value is a bf16 value: 3 mantissa bits, exponents
  // 2^-9 .. 2^8); the NaN code's entry is the quiet NaN
  alignas(64) uint16_t e4m3_bf16[128];
  Tables() {
    for (int c = 0; c < 256; ++c) {
      const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
      float v;
      if (e == 15 && m == 7) v = NAN;
      else if (e == 0) v = ldexpf((float)m / 8.0f, -6);
      else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
      e4m3[c] = s ? -v : v;
    }
    for (int c = 0; c < 128; ++c) {
      uint32_t u;
      memcpy(&u, &e4m3[c], 4);
      e4m3_bf16[c] = (uint16_t)(u >> 16);
    }
    for (int c = 0; c < 16; ++c) {
      const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
      const float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
      e2m1[c] = s ? -v : v;
    }
  }
};
const Tables g_tab;

inline float bf16_to_f32(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

inline float e8m0_to_f32(uint8_t e) {
  if (e == 255) return NAN;
  if (e == 0) return ldexpf(1.0f, -127);
  const uint32_t u = (uint32_t)e << 23;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// One weight row of C columns (codes at w; fp8: block scales `sc` per 128
// columns; MXFP4: E8M0 bytes `sc` per 32 columns) times nt activation rows
// a[t] (fp32, C long): acc[t] = sum_c W[c] a[t][c], 16 lanes per row (one
// AVX-512 register per token).  The AVX-512 versions keep the nt accumulators in
// registers; the portable versions do the same sums lane by lane.
constexpr int kLanes = 16;
constexpr int kMaxTok = 8;  // activation rows per pass

// ---- portable
void dot_f32_p(const float* w, int C, const float* const* a, int nt, float* acc) {
  for (int t = 0; t < nt; ++t) {
    float l[kLanes] = {};
    for (int c = 0; c < C; c += kLanes)
      for (int i = 0; i < kLanes; ++i) l[i] += w[c + i] * a[t][c + i];
    float s = 0.f;
    for (int i = 0; i < kLanes; ++i) s += l[i];
    acc[t] = s;
  }
}

template <typename Dec>
void dot_dec_p(const Dec& dec, int C, int block, const float* sc, const float* const* a, int nt, float* acc) {
  for (int t = 0; t < nt; ++t) acc[t] = 0.f;
  for (int c0 = 0; c0 < C; c0 += block) {
    for (int t = 0; t < nt; ++t) {
      float l[kLanes] = {};
      for (int c = c0; c < c0 + block; c += kLanes)
        for (int i = 0; i < kLanes; ++i) l[i] += dec(c + i) * a[t][c + i];
      float p = 0.f;
      for (int i = 0; i < kLanes; ++i) p += l[i];
      acc[t] += (sc ? sc[c0 / block] : 1.0f) * p;
    }
  }
}

// ---- AVX-512
#define MOE_AVX512 __attribute__((target("avx512f")))
#define MOE_AVX512BW __attribute__((target("avx512f,avx512bw")))
const bool g_avx512bw = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");

MOE_AVX512 inline float hsum(__m512 v) { return _mm512_reduce_add_ps(v); }

// 16 bf16 -> 16 fp32
MOE_AVX512 inline __m512 ld_bf16(const uint16_t* w) {
  const __m256i b = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(w));
  return _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(b), 16));
}

// 16 e4m3 codes -> 16 fp32: sign, then exponent + 120 into place for normals,
// m * 2^-9 for subnormals, NaN for the two NaN codes
MOE_AVX512 inline __m512 ld_e4m3(const uint8_t* w) {
  const __m512i u = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(w)));
  const __m512i em = _mm512_and_si512(u, _mm512_set1_epi32(0x7f));
  const __m512i sign = _mm512_slli_epi32(_mm512_and_si512(u, _mm512_set1_epi32(0x80)), 24);
  const __m512i norm = _mm512_add_epi32(_mm512_slli_epi32(em, 20), _mm512_set1_epi32(120 << 23));
  const __m512 sub = _mm512_mul_ps(_mm512_cvtepi32_ps(em), _mm512_set1_ps(1.0f / 512.0f));
  const __mmask16 is_sub = _mm512_cmplt_epi32_mask(em, _mm512_set1_epi32(8));
  const __mmask16 is_nan = _mm512_cmpeq_epi32_mask(em, _mm512_set1_epi32(0x7f));
  __m512i bits = _mm512_mask_mov_epi32(norm, is_sub, _mm512_castps_si512(sub));
  bits = _mm512_mask_mov_epi32(bits, is_nan, _mm512_set1_epi32(0x7fc00000));
  return _mm512_castsi512_ps(_mm512_or_si512(bits, sign));
}

// NR weight rows (ld(r, c): 16 weights of row r from column c) against NT activation
// rows: each activation chunk is loaded once for the NR rows, so with two rows the
// loop issues 10 loads per 16 fused multiply-adds instead of 9 per 8.  Every (row,
// token) sum keeps its own register and the same order as one row at a time.
template <int NR, int NT, typename Load, typename Scale>
MOE_AVX512 inline void dot_blocks(const Load& ld, const Scale& scale, int C, int block, const float* const* a,
                                  float* acc) {
  float out[NR][NT] = {};
  for (int c0 = 0; c0 < C; c0 += block) {
    __m512 l[NR][NT];
    for (int r = 0; r < NR; ++r)
      for (int t = 0; t < NT; ++t) l[r][t] = _mm512_setzero_ps();
    for (int c = c0; c < c0 + block; c += kLanes) {
      __m512 av[NT];
      for (int t = 0; t < NT; ++t) av[t] = _mm512_loadu_ps(a[t] + c);
      for (int r = 0; r < NR; ++r) {
        const __m512 wv = ld(r, c);
        for (int t = 0; t < NT; ++t) l[r][t] = _mm512_fmadd_ps(wv, av[t], l[r][t]);
      }
    }
    for (int r = 0; r < NR; ++r) {
      const float sc = scale(r, c0);
      for (int t = 0; t < NT; ++t) out[r][t] += sc * hsum(l[r][t]);
    }
  }
  for (int r = 0; r < NR; ++r)
    for (int t = 0; t < NT; ++t) acc[r * kMaxTok + t] = out[r][t];
}

// MXFP4 rows: 32 weights (16 code bytes, one E8M0 block) per step.  The nibbles are split and
// interleaved as bytes, widened once, and looked up in the E2M1 table times the block's scale (a power
// of two, so each entry is exact and equal to the value times the scale); the same products summed in
// the same order as 16 weights at a time with the scale applied after the lookup.
template <int NR, int NT>
MOE_AVX512 inline void dot_blocks_mx4(const uint8_t* w, const uint8_t* sc, int C, const float* const* a,
                                      float* acc) {
  const __m512 table = _mm512_loadu_ps(g_tab.e2m1);
  const __m128i m4 = _mm_set1_epi8(15);
  __m512 l[NR][NT];
  for (int r = 0; r < NR; ++r)
    for (int t = 0; t < NT; ++t) l[r][t] = _mm512_setzero_ps();
  for (int c = 0; c < C; c += 2 * kLanes) {
    __m512 av0[NT], av1[NT];
    for (int t = 0; t < NT; ++t) {
      av0[t] = _mm512_loadu_ps(a[t] + c);
      av1[t] = _mm512_loadu_ps(a[t] + c + kLanes);
    }
    for (int r = 0; r < NR; ++r) {
      const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i*>(w + ((size_t)r * C + c) / 2));
      const __m128i lo = _mm_and_si128(b, m4), hi = _mm_and_si128(_mm_srli_epi16(b, 4), m4);
      const __m512 ts = _mm512_mul_ps(table, _mm512_set1_ps(e8m0_to_f32(sc[(size_t)r * (C / 32) + c / 32])));
      const __m512 w0 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpacklo_epi8(lo, hi)), ts);
      const __m512 w1 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpackhi_epi8(lo, hi)), ts);
      for (int t = 0; t < NT; ++t) {
        l[r][t] = _mm512_fmadd_ps(w0, av0[t], l[r][t]);
        l[r][t] = _mm512_fmadd_ps(w1, av1[t], l[r][t]);
      }
    }
  }
  for (int r = 0; r < NR; ++r)
    for (int t = 0; t < NT; ++t) acc[r * kMaxTok + t] = 0.0f + hsum(l[r][t]);
}

// 32 e4m3 codes -> 32 fp32 (v0: the first 16): the magnitudes looked up as bf16 bits in two 64-entry
// halves of the 128-entry table (vpermi2w), the sign bit put in place, then widened; the same values as
// ld_e4m3, exactly
MOE_AVX512BW inline void ld_e4m3_32(const uint8_t* w, const __m512i (&t)[4], __m512& v0, __m512& v1) {
  const __m512i u = _mm512_cvtepu8_epi16(_mm256_loadu_si256(reinterpret_cast<const __m256i*>(w)));
  const __m512i em = _mm512_and_si512(u, _mm512_set1_epi16(0x7f));
  const __m512i r0 = _mm512_permutex2var_epi16(t[0], em, t[1]);  // magnitudes 0..63 (index bits 0-5)
  const __m512i r1 = _mm512_permutex2var_epi16(t[2], em, t[3]);  // 64..127
  __m512i b = _mm512_mask_blend_epi16(_mm512_test_epi16_mask(em, _mm512_set1_epi16(64)), r0, r1);
  b = _mm512_or_si512(b, _mm512_slli_epi16(_mm512_and_si512(u, _mm512_set1_epi16(0x80)), 8));
  v0 = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(_mm512_castsi512_si256(b)), 16));
  v1 = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(_mm512_extracti64x4_epi64(b, 1)), 16));
}

// fp8 rows with 128 x 128 block scales, 32 weights per step: the same products, sums and scaling, in the
// same order, as dot_blocks with ld_e4m3 (16 at a time, one scale per 128 columns)
template <int NR, int NT>
MOE_AVX512BW inline void dot_blocks_fp8(const uint8_t* w, const float* sc, int C, const float* const* a, float* acc) {
  __m512i t[4];
  for (int i = 0; i < 4; ++i) t[i] = _mm512_load_si512(g_tab.e4m3_bf16 + 32 * i);
  float out[NR][NT] = {};
  for (int c0 = 0; c0 < C; c0 += 128) {
    __m512 l[NR][NT];
    for (int r = 0; r < NR; ++r)
      for (int t_ = 0; t_ < NT; ++t_) l[r][t_] = _mm512_setzero_ps();
    for (int c = c0; c < c0 + 128; c += 2 * kLanes) {
      __m512 av0[NT], av1[NT];
      for (int t_ = 0; t_ < NT; ++t_) {
        av0[t_] = _mm512_loadu_ps(a[t_] + c);
        av1[t_] = _mm512_loadu_ps(a[t_] + c + kLanes);
      }
      for (int r = 0; r < NR; ++r) {
        __m512 w0, w1;
        ld_e4m3_32(w + (size_t)r * C + c, t, w0, w1);
        for (int t_ = 0; t_ < NT; ++t_) {
          l[r][t_] = _mm512_fmadd_ps(w0, av0[t_], l[r][t_]);
          l[r][t_] = _mm512_fmadd_ps(w1, av1[t_], l[r][t_]);
        }
      }
    }
    for (int r = 0; r < NR; ++r) {
      const float s = sc[c0 / 128];
      for (int t_ = 0; t_ < NT; ++t_) out[r][t_] += s * hsum(l[r][t_]);
    }
  }
  for (int r = 0; r < NR; ++r)
    for (int t_ = 0; t_ < NT; ++t_) acc[r * kMaxTok + t_] = out[r][t_];
}

template <int NR>
MOE_AVX512BW void dot_fp8_any(const uint8_t* w, const float* sc, int C, const float* const* a, int nt, float* acc) {
  switch (nt) {
    case 1: dot_blocks_fp8<NR, 1>(w, sc, C, a, acc); return;
    case 2: dot_blocks_fp8<NR, 2>(w, sc, C, a, acc); return;
    case 3: dot_blocks_fp8<NR, 3>(w, sc, C, a, acc); return;
    case 4: dot_blocks_fp8<NR, 4>(w, sc, C, a, acc); return;
    case 5: dot_blocks_fp8<NR, 5>(w, sc, C, a, acc); return;
    case 6: dot_blocks_fp8<NR, 6>(w, sc, C, a, acc); return;
    case 7: dot_blocks_fp8<NR, 7>(w, sc, C, a, acc); return;
    default: dot_blocks_fp8<NR, 8>(w, sc, C, a, acc); return;
  }
}

template <int NR>
MOE_AVX512 void dot_mx4_any(const uint8_t* w, const uint8_t* sc, int C, const float* const* a, int nt, float* acc) {
  switch (nt) {
    case 1: dot_blocks_mx4<NR, 1>(w, sc, C, a, acc); return;
    case 2: dot_blocks_mx4<NR, 2>(w, sc, C, a, acc); return;
    case 3: dot_blocks_mx4<NR, 3>(w, sc, C, a, acc); return;
    case 4: dot_blocks_mx4<NR, 4>(w, sc, C, a, acc); return;
    case 5: dot_blocks_mx4<NR, 5>(w, sc, C, a, acc); return;
    case 6: dot_blocks_mx4<NR, 6>(w, sc, C, a, acc); return;
    case 7: dot_blocks_mx4<NR, 7>(w, sc, C, a, acc); return;
    default: dot_blocks_mx4<NR, 8>(w, sc, C, a, acc); return;
  }
}

template <int NR, typename Load, typename Scale>
MOE_AVX512 void dot_any(const Load& ld, const Scale& scale, int C, int block, const float* const* a, int nt,
                        float* acc) {
  switch (nt) {
    case 1: dot_blocks<NR, 1>(ld, scale, C, block, a, acc); return;
    case 2: dot_blocks<NR, 2>(ld, scale, C, block, a, acc); return;
    case 3: dot_blocks<NR, 3>(ld, scale, C, block, a, acc); return;
    case 4: dot_blocks<NR, 4>(ld, scale, C, block, a, acc); return;
    case 5: dot_blocks<NR, 5>(ld, scale, C, block, a, acc); return;
    case 6: dot_blocks<NR, 6>(ld, scale, C, block, a, acc); return;
    case 7: dot_blocks<NR, 7>(ld, scale, C, block, a, acc); return;
    default: dot_blocks<NR, 8>(ld, scale, C, block, a, acc); return;
  }
}

// nr (1 or 2) consecutive rows, row stride C weights; acc[r * kMaxTok + t]
template <int NR>
MOE_AVX512 void dot_rows_v(const uint8_t* w, int dtype, const void* sc, int C, const float* const* a, int nt,
                           float* acc) {
  const auto one = [](int, int) MOE_AVX512 { return 1.0f; };
  switch (dtype) {
    case MOE_F32: {
      const float* wf = reinterpret_cast<const float*>(w);
      dot_any<NR>([&](int r, int c) MOE_AVX512 { return _mm512_loadu_ps(wf + (size_t)r * C + c); }, one, C, C, a,
                  nt, acc);
      return;
    }
    case MOE_BF16: {
      const uint16_t* wb = reinterpret_cast<const uint16_t*>(w);
      dot_any<NR>([&](int r, int c) MOE_AVX512 { return ld_bf16(wb + (size_t)r * C + c); }, one, C, C, a, nt, acc);
      return;
    }
    case MOE_FP8_E4M3_B128: {  // the rows share their 128-row block's scales
      const float* s = reinterpret_cast<const float*>(sc);
      if (g_avx512bw) {
        dot_fp8_any<NR>(w, s, C, a, nt, acc);
        return;
      }
      dot_any<NR>([&](int r, int c) MOE_AVX512 { return ld_e4m3(w + (size_t)r * C + c); },
                  [&](int, int c0) MOE_AVX512 { return s[c0 / 128]; }, C, 128, a, nt, acc);
      return;
    }
    default:  // MXFP4: E8M0 bytes per 32 columns of each row
      dot_mx4_any<NR>(w, reinterpret_cast<const uint8_t*>(sc), C, a, nt, acc);
      return;
  }
}

const bool g_avx512 = __builtin_cpu_supports("avx512f");

void dot_f32(const float* w, int C, const float* const* a, int nt, float* acc) { dot_f32_p(w, C, a, nt, acc); }
void dot_bf16(const uint16_t* w, int C, const float* const* a, int nt, float* acc) {
  dot_dec_p([&](int c) { return bf16_to_f32(w[c]); }, C, C, nullptr, a, nt, acc);
}
void dot_fp8(const uint8_t* w, const float* sc, int C, const float* const* a, int nt, float* acc) {
  dot_dec_p([&](int c) { return g_tab.e4m3[w[c]]; }, C, 128, sc, a, nt, acc);
}
void dot_mx4(const uint8_t* w, const uint8_t* sc, int C, const float* const* a, int nt, float* acc) {
  dot_dec_p([&](int c) { return g_tab.e2m1[(w[c / 2] >> (4 * (c & 1))) & 15] * e8m0_to_f32(sc[c / 32]); }, C, C,
            nullptr, a, nt, acc);
}

// rows r .. r + nr - 1 (nr 1 or 2; r even when nr is 2) of matrix m (0 gate, 1 up: [F][H];
// 2 down: [H][F]) of a record against nt activation rows; acc[i * kMaxTok + t]
void dot_rows(const uint8_t* rec, int dtype, int H, int F, int m, int r, int nr, const float* const* a, int nt,
              float* acc) {
  const uint64_t n = (uint64_t)F * H;
  const int C = m == 2 ? F : H;
  const uint8_t* w;
  const void* sc = nullptr;
  switch (dtype) {
    case MOE_F32: w = rec + 4 * (m * n + (uint64_t)r * C); break;
    case MOE_BF16: w = rec + 2 * (m * n + (uint64_t)r * C); break;
    case MOE_FP8_E4M3_B128: {
      const float* scales = reinterpret_cast<const float*>(rec + 3 * n);
      const uint64_t per = (uint64_t)(F / 128) * (H / 128);
      w = rec + m * n + (uint64_t)r * C;
      sc = scales + m * per + (uint64_t)(r / 128) * (C / 128);
      break;
    }
    default: {  // MOE_MXFP4
      const uint8_t* scales = rec + 3 * n / 2;
      w = rec + (m * n + (uint64_t)r * C) / 2;
      sc = scales + m * (n / 32) + (uint64_t)r * (C / 32);
      break;
    }
  }
  if (g_avx512) {
    if (nr == 2) dot_rows_v<2>(w, dtype, sc, C, a, nt, acc);
    else dot_rows_v<1>(w, dtype, sc, C, a, nt, acc);
    return;
  }
  for (int i = 0; i < nr; ++i) {
    float* o = acc + i * kMaxTok;
    switch (dtype) {
      case MOE_F32: dot_f32(reinterpret_cast<const float*>(w) + (uint64_t)i * C, C, a, nt, o); break;
      case MOE_BF16: dot_bf16(reinterpret_cast<const uint16_t*>(w) + (uint64_t)i * C, C, a, nt, o); break;
      case MOE_FP8_E4M3_B128: dot_fp8(w + (uint64_t)i * C, reinterpret_cast<const float*>(sc), C, a, nt, o); break;
      default:
        dot_mx4(w + (uint64_t)i * C / 2, reinterpret_cast<const uint8_t*>(sc) + (uint64_t)i * (C / 32), C, a, nt,
                o);
        break;
    }
  }
}

// ---------------------------------------------------------------- worker pool
// A call is one parallel region (both phases, ordered per expert by counters),
// issued once per layer and lasting a few hundred microseconds, so waking
// sleeping threads for it (futex round trips, one thread after another) would
// cost as much as the work.  Workers therefore poll a generation counter for a
// while after each region, yielding the CPU between polls so that a busy host
// loses nothing to them, and only then sleep on a condition variable.  The
// caller works too and waits for the region's last item the same way.
class Pool {
 public:
  Pool() {
    cpu_set_t set;
    int n = 0;
    if (sched_getaffinity(0, sizeof set, &set) == 0) n = CPU_COUNT(&set);
    if (n <= 0) n = (int)std::thread::hardware_concurrency();
    nthreads_ = std::max(1, n);
    for (int i = 1; i < nthreads_; ++i) workers_.emplace_back([this] { loop(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_.store(true);
      gen_.fetch_add(1);
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
  }
  int threads() const { return nthreads_; }

  // runs fn(i) for i in [0, n) on every thread of the pool and the caller; returns when all are done
  void run(int n, const std::function<void(int)>& fn) {
    if (n <= 0) return;
    std::unique_lock<std::mutex> call(call_mu_);  // one parallel region at a time
    fn_ = &fn;
    n_ = n;
    next_.store(0);
    pending_.store((int)workers_.size());
    gen_.fetch_add(1);  // sequentially consistent: ordered before the sleeper count is read
    if (sleepers_.load() > 0) {
      std::lock_guard<std::mutex> lk(mu_);
      cv_.notify_all();
    }
    work();
    while (pending_.load(std::memory_order_acquire) > 0) sched_yield();
    fn_ = nullptr;
  }

 private:
  static constexpr int64_t kPollNs = 2000000;  // poll this long after a region before sleeping

  void work() {
    for (int i = next_.fetch_add(1); i < n_; i = next_.fetch_add(1)) (*fn_)(i);
  }
  void loop() {
    uint64_t seen = 0;  // the generation at construction: a region may start before this thread runs
    for (;;) {
      const auto t0 = std::chrono::steady_clock::now();
      uint32_t polls = 0;
      while (gen_.load(std::memory_order_acquire) == seen) {
        sched_yield();
        if ((++polls & 63) == 0 &&
            std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count() >
                kPollNs) {
          std::unique_lock<std::mutex> lk(mu_);
          sleepers_.fetch_add(1);  // sequentially consistent: ordered before gen_ is read again
          cv_.wait(lk, [&] { return gen_.load() != seen; });
          sleepers_.fetch_sub(1);
          break;
        }
      }
      seen = gen_.load(std::memory_order_acquire);
      if (stop_.load()) return;
      work();
      pending_.fetch_sub(1, std::memory_order_acq_rel);
    }
  }
  int nthreads_ = 1;
  std::vector<std::thread> workers_;
  std::mutex mu_, call_mu_;
  std::condition_variable cv_;
  const std::function<void(int)>* fn_ = nullptr;
  int n_ = 0;
  std::atomic<int> next_{0}, pending_{0}, sleepers_{0};
  std::atomic<uint64_t> gen_{0};
  std::atomic<bool> stop_{false};
};

Pool& pool() {
  static Pool p;  // created on first use, joined when the library unloads
  return p;
}

}  // namespace

int host_threads() { return pool().threads(); }

void host_cold_ffn(const HostFfnJob& j) {
  const int H = j.H, F = j.F, n = j.T * j.k;
  // group the cold pairs by expert (ascending expert id, pairs in call order)
  std::vector<int> order;
  for (int p = 0; p < n; ++p)
    if (j.sid[p] >= j.S + j.E && j.sid[p] < j.S + 2 * j.E) order.push_back(p);
  if (order.empty()) return;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return j.sid[a] < j.sid[b]; });
  struct Group {
    int e, first, count;
  };
  std::vector<Group> groups;
  for (int i = 0; i < (int)order.size(); ++i) {
    const int e = j.sid[order[i]] - j.S - j.E;
    if (groups.empty() || groups.back().e != e) groups.push_back({e, i, 0});
    groups.back().count += 1;
  }
  // activations as fp32 rows, and the h rows of every cold pair
  std::vector<float> xf((size_t)j.T * H);
  for (size_t i = 0; i < xf.size(); ++i)
    xf[i] = j.dtype == MOE_F32 ? reinterpret_cast<const float*>(j.x)[i]
                               : bf16_to_f32(reinterpret_cast<const uint16_t*>(j.x)[i]);
  std::vector<float> hbuf((size_t)order.size() * F);
  constexpr int kRowsF = 16, kRowsH = 32;  // weight rows per block
  const int bf = F / kRowsF, bh = (H + kRowsH - 1) / kRowsH;
  // phase 1: gate/up rows of each cold expert against its tokens (kMaxTok at a time)
  pool().run((int)groups.size() * bf, [&](int item) {
    const Group& g = groups[item / bf];
    const int f0 = (item % bf) * kRowsF;
    const uint8_t* rec = j.host + (uint64_t)g.e * j.stride;
    for (int t0 = 0; t0 < g.count; t0 += kMaxTok) {
      const int nt = std::min(kMaxTok, g.count - t0);
      const float* a[kMaxTok];
      for (int t = 0; t < nt; ++t) a[t] = xf.data() + (size_t)(order[g.first + t0 + t] / j.k) * H;
      for (int f = f0; f < f0 + kRowsF; f += 2) {  // two rows at a time (kRowsF is even)
        float gv[2 * kMaxTok], uv[2 * kMaxTok];
        dot_rows(rec, j.dtype, H, F, 0, f, 2, a, nt, gv);
        dot_rows(rec, j.dtype, H, F, 1, f, 2, a, nt, uv);
        for (int i = 0; i < 2; ++i)
          for (int t = 0; t < nt; ++t) {
            const float gg = gv[i * kMaxTok + t], uu = uv[i * kMaxTok + t];
            hbuf[(size_t)(g.first + t0 + t) * F + f + i] = gg / (1.0f + expf(-gg)) * uu;
          }
      }
    }
  });
  // phase 2: down rows of each cold expert against its h rows, into the output rows
  pool().run((int)groups.size() * bh, [&](int item) {
    const Group& g = groups[item / bh];
    const int r0 = (item % bh) * kRowsH, r1 = std::min(H, r0 + kRowsH);
    const uint8_t* rec = j.host + (uint64_t)g.e * j.stride;
    for (int t0 = 0; t0 < g.count; t0 += kMaxTok) {
      const int nt = std::min(kMaxTok, g.count - t0);
      const float* a[kMaxTok];
      for (int t = 0; t < nt; ++t) a[t] = hbuf.data() + (size_t)(g.first + t0 + t) * F;
      for (int r = r0; r < r1; r += 2) {  // two rows at a time (H, r0 and r1 are even)
        const int nr = std::min(2, r1 - r);
        float o[2 * kMaxTok];
        dot_rows(rec, j.dtype, H, F, 2, r, nr, a, nt, o);
        for (int i = 0; i < nr; ++i)
          for (int t = 0; t < nt; ++t) j.out[(size_t)order[g.first + t0 + t] * H + r + i] = o[i * kMaxTok + t];
      }
    }
  });
}

// ---------------------------------------------------------------- decode-chain server
class ColdServer {
 public:
  ColdServer(const ColdChainLayer* layers, int L, int T, uint64_t xrow, const ColdChainIo& io)
      : layers_(layers, layers + L), L_(L), T_(T), xrow_(xrow), io_(io), last_(L) {
    for (int l = 0; l < L; ++l) last_[l] = __atomic_load_n(&io_.req[l], __ATOMIC_ACQUIRE);
    thread_ = std::thread([this] { loop(); });
  }
  ~ColdServer() {
    stop_.store(true);
    thread_.join();
  }

 private:
  void loop() {
    using clk = std::chrono::steady_clock;
    auto idle_since = clk::now();
    while (!stop_.load(std::memory_order_relaxed)) {
      bool did = false;
      for (int l = 0; l < L_; ++l) {
        const uint32_t r = __atomic_load_n(&io_.req[l], __ATOMIC_ACQUIRE);
        if (r == last_[l]) continue;
        // request r of layer l: its indices and activations were stored before r was
        const ColdChainLayer& c = layers_[l];
        HostFfnJob j;
        j.host = c.host;
        j.stride = c.stride;
        j.dtype = c.dtype;
        j.H = c.H;
        j.F = c.F;
        j.x = io_.x + (size_t)l * T_ * xrow_;
        j.T = T_;
        j.k = c.k;
        j.sid = io_.sid + (size_t)l * T_ * c.k;
        j.S = c.S;
        j.E = c.E;
        j.out = io_.out + (size_t)l * T_ * c.k * c.H;
        host_cold_ffn(j);
        __atomic_store_n(&io_.done[l], r, __ATOMIC_RELEASE);  // after the rows
        last_[l] = r;
        did = true;
      }
      const auto now = clk::now();
      if (did) {
        idle_since = now;
      } else if (now - idle_since > std::chrono::milliseconds(50)) {
        std::this_thread::sleep_for(std::chrono::microseconds(100));
      } else {
        _mm_pause();
      }
    }
  }

  std::vector<ColdChainLayer> layers_;
  int L_, T_;
  uint64_t xrow_;
  ColdChainIo io_;
  std::vector<uint32_t> last_;
  std::atomic<bool> stop_{false};
  std::thread thread_;
};

ColdServer* cold_server_start(const ColdChainLayer* layers, int L, int T, uint64_t xrow, const ColdChainIo& io) {
  try {
    return new ColdServer(layers, L, T, xrow, io);
  } catch (...) {
    return nullptr;
  }
}

void cold_server_stop(ColdServer* s) { delete s; }

}  // namespace moe
