/*
 * CPU ORACLE for the offloaded Mixture-of-Experts layer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this.  It is plain and slow on
 * purpose, shares no code with the GPU library, and the GPU library never
 * calls it.
 *
 * Sources ("the pages"):
 *   [xinfer]   xinfer-ai 0.14.6 docs/moe_offload.md (my.diffend.io npm diff page),
 *              sections "How it works" (Decode, Prefill, slot tensors) and the
 *              opening paragraph (how many experts sit on the GPU changes neither
 *              the routing nor the numerics).
 *   [freetoken] FreeToken issue #677 "prefetch the next layer's experts from a router
 *              lookahead during offloaded decode", section "Proposal"
 *              (Lookahead, Install, Correctness constraint), and "Measured" (the
 *              scored-eviction baseline).
 *   [moe-inf]  MoE-Infinity README, "Overview" and "Key Features" (the
 *              activation-aware expert cache).
 *   [npu]      npu-offload README, intro, "Architecture" and "Results" (cold
 *              experts computed by the host CPU; profile-guided placement).
 * Where the pages are silent the plainest reading is taken; each such reading is
 * marked READING below and listed in the design notes.
 *
 * Precision: every floating-point step runs in double, except the router
 * logits and the pre-norm.  The logits' fp32 value decides an integer (the
 * top-k ids), so they are computed in the GPU kernel's precision with one
 * fixed summation order (READING, see orc_router_logits); the order is part of
 * the specification.  The pre-norm is glue outside the method whose output is
 * a quantised code; its binary32 order is fixed the same way (READING, see
 * orc_rmsnorm).
 *
 * Build: gcc -O2 -ffp-contract=off (no fast-math; denormals kept).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* weight dtype codes */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_MXFP4 = 3 };
/* descriptor modes */
enum { ORC_SLOTS = 0, ORC_STAGED = 1, ORC_STAGED_ALL = 2, ORC_COLD = 3 };
/* error codes */
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENAN = -2 };

/* ------------------------------------------------------------------ */
/* number formats                                                     */
/* ------------------------------------------------------------------ */

/* bf16 -> double: the 16 bits are the top half of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* double -> bf16, round to nearest, ties to even, computed on the exact value
 * (no intermediate rounding to binary32). */
uint16_t orc_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  /* largest finite bf16 = (2 - 2^-7) * 2^127; halfway to 2^128 rounds to inf */
  if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7F80;
  int e;
  frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  if (E < -126) E = -126;       /* subnormal range: fixed quantum 2^-133 */
  double q = ldexp(1.0, E - 7); /* spacing of bf16 values near a */
  double m = nearbyint(a / q);  /* a/q is exact (power-of-two scaling); RNE */
  double r = m * q;
  float f = (float)r;           /* exactly representable */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

/* OCP 8-bit floating point, E4M3 ("fn": bias 7, no infinities, S.1111.111 = NaN).
 * Normal: (-1)^s 2^(e-7) (1 + m/8); subnormal (e = 0): (-1)^s 2^-6 (m/8). */
double orc_fp8_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP Microscaling (MX) v1.0 FP4 element, E2M1: sign bit 3, exponent bits 2:1
 * with bias 1, mantissa bit 0, no infinities or NaN.  Normal (e > 0):
 * (-1)^s 2^(e-1) (1 + m/2); subnormal (e = 0): (-1)^s (m/2).  Magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double orc_e2m1_to_f64(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* MX shared scale, E8M0: 2^(e - 127); e = 255 is NaN. */
double orc_e8m0_to_f64(uint8_t e) {
  if (e == 255) return NAN;
  return ldexp(1.0, (int)e - 127);
}

static double load_w(const uint8_t* base, int wdt, size_t i) {
  if (wdt == ORC_F32) { float f; memcpy(&f, base + 4 * i, 4); return (double)f; }
  if (wdt == ORC_BF16) { uint16_t b; memcpy(&b, base + 2 * i, 2); return orc_bf16_to_f64(b); }
  return orc_fp8_to_f64(base[i]);
}

/* activation dtype follows the weights: fp32 for fp32 weights, bf16 otherwise */
static double load_act(const void* x, int wdt, size_t i) {
  if (wdt == ORC_F32) return (double)((const float*)x)[i];
  return orc_bf16_to_f64(((const uint16_t*)x)[i]);
}

static void store_act(void* y, int wdt, size_t i, double v) {
  if (wdt == ORC_F32) ((float*)y)[i] = (float)v; /* C conversion rounds to nearest even */
  else ((uint16_t*)y)[i] = orc_f64_to_bf16(v);
}

/* record = [gate F x H | up F x H | down H x F | scales gate, up, down]
 *   fp32 / bf16: no scales;
 *   fp8:   one byte per weight, fp32 scale per 128 x 128 block;
 *   MXFP4: two E2M1 codes per byte (element 2i in the low nibble, 2i + 1 in
 *          the high nibble, row-major), one E8M0 scale per 32 consecutive
 *          weights of a row ([rows][cols / 32] bytes per matrix). */
size_t orc_record_bytes(int wdt, int H, int F) {
  size_t n = 3 * (size_t)H * (size_t)F;
  if (wdt == ORC_F32) return 4 * n;
  if (wdt == ORC_BF16) return 2 * n;
  if (wdt == ORC_MXFP4) return n / 2 + n / 32;
  return n + 3 * (size_t)(H / 128) * (size_t)(F / 128) * 4;
}

/* ------------------------------------------------------------------ */
/* router: logits, top-k, renormalised softmax weights                 */
/* ------------------------------------------------------------------ */

/* Router logits l[t][e] = sum_i x[t][i] Wr[e][i] + b[e].
 * READING (the pages give no formula, only "routing"): the sum is taken in
 * binary32 with one fixed order, so that the integer top-k decision is the
 * same on any machine that follows it:
 *   - the H inputs are split into chunks of 8 consecutive elements;
 *     64 lanes; lane L owns chunks L, L+64, L+128, ... in ascending order;
 *   - each lane starts at +0 and accumulates acc = fma(x_i, w_i, acc)
 *     (one rounding per step) over its chunks, elements in ascending i;
 *   - lanes are combined pairwise, p[L] = p[L] + p[L xor o] for
 *     o = 32, 16, 8, 4, 2, 1 (all lanes end with the same value);
 *   - finally l = p[0] + b[e], rounded to binary32.
 * Inputs (bf16 or fp32) are widened exactly.  H must be a multiple of 8. */
void orc_router_logits(const void* x, const void* wr, int wdt, const float* bias, int T, int E, int H,
                       float* logits) {
  /* tokens are independent; threads only split them (each logit's arithmetic is unchanged) */
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      float p[64];
      for (int L = 0; L < 64; ++L) {
        float acc = 0.0f;
        for (int c = L; c * 8 < H; c += 64)
          for (int q = 0; q < 8; ++q) {
            int i = c * 8 + q;
            float xv = (float)load_act(x, wdt, (size_t)t * H + i);
            float wv = (float)load_w((const uint8_t*)wr, wdt == ORC_F32 ? ORC_F32 : ORC_BF16, (size_t)e * H + i);
            acc = fmaf(xv, wv, acc);
          }
        p[L] = acc;
      }
      for (int o = 32; o >= 1; o >>= 1) {
        float n[64];
        for (int L = 0; L < 64; ++L) n[L] = p[L] + p[L ^ o];
        memcpy(p, n, sizeof p);
      }
      logits[(size_t)t * E + e] = p[0] + bias[e];
    }
}

/* Top-k and weights for each token.
 * READING: experts are ordered by (logit descending, id ascending) and the
 * first k are taken; position j follows that order (ties go to the lower id).
 * Weights are the softmax over all E logits renormalised over the k chosen,
 * which equals w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), in double.
 * Returns ORC_ENAN if any logit is NaN. */
int orc_topk(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e)
      if (isnan(l[e])) return ORC_ENAN;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: equal logits keep the lower id */
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    free(taken);
    double l0 = (double)l[ids[(size_t)t * k]];
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp((double)l[ids[(size_t)t * k + j]] - l0);
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - l0) / z;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* per-layer LRU expert-slot cache                                     */
/* ------------------------------------------------------------------ */
/*
 * [xinfer] "How it works", Decode: a per-layer LRU table on the GPU; routed
 * experts are looked up, misses get the least-recently-used slots, expert ids
 * are rewritten to slot ids, and the missing experts are copied from pinned
 * host memory into their slots.  Prefill: a call that touches more distinct
 * experts than there are slots stages the layer in a staging buffer instead.
 *
 * READING of the rules the page leaves open (all integer, so bit-exact):
 *   state: expert_of[S] (-1 = free), slot_of[E] (-1 = not resident),
 *          last_use[S], tick; the cache starts empty with tick = 0.
 *   ensure(ids):
 *     1. tick += 1;  D = sorted distinct ids;  R = resident experts.
 *     2. |D| <= S (SLOTS): M = D \ R ascending.  Eligible victims are the
 *        slots whose expert is not in D, ordered by the key
 *        (occupied, last_use, slot): free slots first, then the least
 *        recently used, ties to the lower slot.  M[i] goes to victim i; the
 *        evicted expert leaves the map.  Every e in D gets last_use = tick.
 *        slot_ids = slot_of[id].  Copy list = (M[i], victim i).
 *     3. more misses than eligible victims, i.e. |D| > S when no slot is
 *        pinned (STAGED; not on the page, which stages whole layers for
 *        prefill only): hits as in 2.  The eligible victims, in the same
 *        order, are fewer than the misses; the misses claim them in install
 *        order (pairs routed to e descending, best top-k position ascending,
 *        id ascending; see orc_install) and every miss left over is copied
 *        to staging record e and read at S + e for this call only.  Every e
 *        of D holding a slot gets last_use = tick.  Copy list = (e, its slot
 *        or S + e) for e in D \ R ascending.  So a batch wider than the
 *        cache still leaves its most used experts resident for the next call.
 *   A record index r < S names slot r; r >= S names staging record r - S.
 *   Prefetch install ([freetoken] "Install"): see orc_install.
 *
 * Scored eviction (READING of the baseline policy [freetoken] "Measured"
 * names, "scored eviction", whose only stated rule is that installed slots
 * start at usage 0 and go first): each slot keeps a usage score, the number
 * of ensure calls that routed to its expert since it was loaded (per call,
 * like the LRU clock), saturating at 2^20 - 1; a slot's score is 0 when an
 * expert is loaded or installed into it.  With policy ORC_SCORED the victim
 * key is (occupied, score, last_use, slot): least used first, then least
 * recently used, then the lower slot.  Everything else is as above.
 *
 * Activation-aware eviction (READING of [moe-infinity] "Overview" and "Key
 * Features": the cache keeps the experts that are activated most often on the
 * GPU; the page gives no rule beyond that): every expert keeps an activation
 * count, the number of ensure calls that routed to it since the cache was
 * created (per call, saturating at 2^20 - 1), which survives eviction and
 * reloading.  With policy ORC_FREQ the victim key is (occupied, never used
 * since install (last_use = 0) first, activation count of the held expert,
 * last_use, slot): installed slots still go first as the prefetch rule asks,
 * then the least activated expert, then the least recently used, then the
 * lower slot.  Installs and pins do not count as activations.
 *
 * Host-computed cold experts (READING of [npu-offload] intro, "Results" and
 * "Architecture": hot experts stay in accelerator memory, the host CPU computes
 * the cold ones from host DRAM, only activations cross the link and weights
 * never move): with the cold mode on, an ensure call loads nothing.  D, the
 * hits and their last_use / score / activation updates are as above, and every
 * routed expert's activation count advances; a miss keeps no slot, takes no
 * victim and is read at record index S + E + e (host record e) for this call.
 * Copy list = {COLD, |misses|, (e, S + E + e) for e in D \ R ascending}.  The
 * table is otherwise unchanged; there is no overflow.  Counters: calls, hits,
 * and cold (the misses computed on the host).
 *
 * Split mode (READING: the same pages, with the host and the link working at
 * once, each on part of a call's misses): ensure runs as above, and of the
 * misses a call wider than the cache stages for itself only (they keep no
 * slot), the last round(n_staged * q / 256) in ascending id are read at
 * S + E + e (computed on the host) instead of staging; q in [0, 256] is the
 * host's share.  The copy list keeps mode STAGED and lists them with their
 * S + E + e index; counters: staged_copies counts the staged ones left, cold
 * the host's.  Calls that do not overflow are unchanged.
 */
enum { ORC_LRU = 0, ORC_SCORED = 1, ORC_FREQ = 2 };
#define ORC_SCORE_MAX ((1u << 20) - 1u)

typedef struct {
  int E, S;
  int policy;
  int32_t* slot_of;
  int32_t* expert_of;
  uint64_t* last_use;
  uint32_t* score;
  uint32_t* act;         /* [E] activation count (ORC_FREQ key; kept under every policy) */
  unsigned char* pinned; /* [S] profile-guided placement: never a victim */
  int cold;              /* 1: misses are computed on the host, never loaded; 2: split (cold_q) */
  int cold_q;            /* split mode: the host's share of the staged misses, in 1/256 */
  uint64_t tick;
  /* cumulative counters */
  uint64_t calls, hits, misses, staged_calls, staged_copies, prefetch_installs, prefetch_hits, cold_misses;
} orc_cache;

orc_cache* orc_cache_new(int E, int S) {
  if (E <= 0 || S <= 0 || S > E) return NULL;
  orc_cache* c = (orc_cache*)calloc(1, sizeof(orc_cache));
  c->E = E;
  c->S = S;
  c->slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  c->expert_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  c->last_use = (uint64_t*)calloc((size_t)S, sizeof(uint64_t));
  c->score = (uint32_t*)calloc((size_t)S, sizeof(uint32_t));
  c->act = (uint32_t*)calloc((size_t)E, sizeof(uint32_t));
  c->pinned = (unsigned char*)calloc((size_t)S, 1);
  for (int e = 0; e < E; ++e) c->slot_of[e] = -1;
  for (int s = 0; s < S; ++s) c->expert_of[s] = -1;
  return c;
}

void orc_cache_free(orc_cache* c) {
  if (!c) return;
  free(c->slot_of);
  free(c->expert_of);
  free(c->last_use);
  free(c->score);
  free(c->act);
  free(c->pinned);
  free(c);
}

void orc_cache_set_policy(orc_cache* c, int policy) {
  c->policy = (policy == ORC_SCORED || policy == ORC_FREQ) ? policy : ORC_LRU;
}

void orc_cache_set_cold(orc_cache* c, int on) { c->cold = on != 0; }

void orc_cache_set_split(orc_cache* c, int q) {
  c->cold = 2;
  c->cold_q = q < 0 ? 0 : (q > 256 ? 256 : q);
}

void orc_cache_act(const orc_cache* c, uint32_t* act) { memcpy(act, c->act, sizeof(uint32_t) * (size_t)c->E); }

void orc_cache_scores(const orc_cache* c, uint32_t* score) {
  memcpy(score, c->score, sizeof(uint32_t) * (size_t)c->S);
}

void orc_cache_pinned(const orc_cache* c, int32_t* pinned) {
  for (int s = 0; s < c->S; ++s) pinned[s] = c->pinned[s];
}

void orc_cache_state(const orc_cache* c, int32_t* slot_of, int32_t* expert_of, uint64_t* last_use, uint64_t* tick) {
  if (slot_of) memcpy(slot_of, c->slot_of, sizeof(int32_t) * (size_t)c->E);
  if (expert_of) memcpy(expert_of, c->expert_of, sizeof(int32_t) * (size_t)c->S);
  if (last_use) memcpy(last_use, c->last_use, sizeof(uint64_t) * (size_t)c->S);
  if (tick) *tick = c->tick;
}

/* counters: calls, hits, misses, staged_calls, staged_copies, prefetch_installs, prefetch_hits, cold */
void orc_cache_counters(const orc_cache* c, uint64_t out[8]) {
  out[0] = c->calls; out[1] = c->hits; out[2] = c->misses; out[3] = c->staged_calls;
  out[4] = c->staged_copies; out[5] = c->prefetch_installs; out[6] = c->prefetch_hits; out[7] = c->cold_misses;
}

/* does slot a come before slot b in victim order?  LRU (occupied, last_use, slot); scored (occupied,
 * score, last_use, slot); activation-aware (occupied, last_use != 0, activation count, last_use, slot) */
static int victim_before(const orc_cache* c, int a, int b) {
  int oa = c->expert_of[a] >= 0, ob = c->expert_of[b] >= 0;
  if (oa != ob) return oa < ob;
  if (c->policy == ORC_SCORED && c->score[a] != c->score[b]) return c->score[a] < c->score[b];
  if (c->policy == ORC_FREQ && oa) { /* both occupied */
    int ua = c->last_use[a] != 0, ub = c->last_use[b] != 0;
    if (ua != ub) return ua < ub;
    uint32_t fa = c->act[c->expert_of[a]], fb = c->act[c->expert_of[b]];
    if (fa != fb) return fa < fb;
  }
  if (c->last_use[a] != c->last_use[b]) return c->last_use[a] < c->last_use[b];
  return a < b;
}

/* eligible slots (not pinned, protect[expert] == 0) sorted into victim order; returns how many */
static int victim_order(const orc_cache* c, const unsigned char* protect, int* order) {
  int n = 0;
  for (int s = 0; s < c->S; ++s) {
    int e = c->expert_of[s];
    if (c->pinned[s] || (e >= 0 && protect[e])) continue;
    /* insertion sort: plain and obviously ordered */
    int pos = n++;
    while (pos > 0 && victim_before(c, s, order[pos - 1])) {
      order[pos] = order[pos - 1];
      --pos;
    }
    order[pos] = s;
  }
  return n;
}

/* does expert a come before expert b in install order (count desc, best asc, id asc)? */
static int install_before(const int* cnt, const int* best, int a, int b) {
  if (cnt[a] != cnt[b]) return cnt[a] > cnt[b];
  if (best[a] != best[b]) return best[a] < best[b];
  return a < b;
}

/* desc layout: desc[0] = mode, desc[1] = count, then count pairs (expert, record index).
 * ids: n = T*k routed ids, k per token.  Returns ORC_EINVAL (state untouched) on an id
 * outside [0, E). */
int orc_ensure(orc_cache* c, const int32_t* ids, int n, int k, int32_t* slot_ids, int32_t* desc) {
  if (k <= 0 || n % k != 0) return ORC_EINVAL;
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->E) return ORC_EINVAL;
  int E = c->E, S = c->S;
  c->tick += 1;
  c->calls += 1;
  unsigned char* inD = (unsigned char*)calloc((size_t)E, 1);
  unsigned char* miss = (unsigned char*)calloc((size_t)E, 1);
  int nd = 0, nm = 0;
  for (int i = 0; i < n; ++i)
    if (!inD[ids[i]]) { inD[ids[i]] = 1; ++nd; }
  /* hits are the experts of D resident before the call */
  for (int e = 0; e < E; ++e) {
    if (!inD[e]) continue;
    int s = c->slot_of[e];
    if (s >= 0) {
      c->hits += 1;
      if (c->last_use[s] == 0) c->prefetch_hits += 1; /* installed by prefetch, first use */
    } else {
      miss[e] = 1;
      ++nm;
    }
  }
  if (c->cold == 1) { /* nothing loads: hits are used in place, misses are read from the host */
    for (int e = 0; e < E; ++e) {
      if (!inD[e]) continue;
      int s = c->slot_of[e];
      if (s >= 0) {
        c->last_use[s] = c->tick;
        if (c->score[s] < ORC_SCORE_MAX) c->score[s] += 1;
      }
      if (c->act[e] < ORC_SCORE_MAX) c->act[e] += 1;
    }
    int count = 0;
    for (int e = 0; e < E; ++e) {
      if (!miss[e]) continue;
      desc[2 + 2 * count] = e;
      desc[3 + 2 * count] = S + E + e;
      ++count;
    }
    for (int i = 0; i < n; ++i) {
      int e = ids[i];
      slot_ids[i] = c->slot_of[e] >= 0 ? c->slot_of[e] : S + E + e;
    }
    desc[0] = ORC_COLD;
    desc[1] = count;
    c->cold_misses += (uint64_t)nm;
    free(miss);
    free(inD);
    return ORC_OK;
  }
  /* the eligible slots in victim order; the call overflows when the misses
   * outnumber them (without pinned slots: exactly when |D| > S) */
  int* order = (int*)malloc(sizeof(int) * (size_t)S);
  int nv = victim_order(c, inD, order);
  int over = nm > nv;
  /* the order in which the misses claim the eligible slots */
  int* claim = (int*)malloc(sizeof(int) * (size_t)(nm > 0 ? nm : 1));
  int nc = 0;
  if (!over) {
    for (int e = 0; e < E; ++e)
      if (miss[e]) claim[nc++] = e;
  } else {
    int* cnt = (int*)calloc((size_t)E, sizeof(int));
    int* best = (int*)malloc(sizeof(int) * (size_t)E);
    for (int e = 0; e < E; ++e) best[e] = k;
    for (int i = 0; i < n; ++i) {
      int e = ids[i];
      cnt[e] += 1;
      if (i % k < best[e]) best[e] = i % k;
    }
    for (int e = 0; e < E; ++e) {
      if (!miss[e]) continue;
      int pos = nc++;
      while (pos > 0 && install_before(cnt, best, e, claim[pos - 1])) {
        claim[pos] = claim[pos - 1];
        --pos;
      }
      claim[pos] = e;
    }
    free(cnt);
    free(best);
  }
  int ns = nm < nv ? nm : nv;
  for (int r = 0; r < ns; ++r) {
    int v = order[r], e = claim[r];
    int old = c->expert_of[v];
    if (old >= 0) c->slot_of[old] = -1;
    c->expert_of[v] = e;
    c->slot_of[e] = v;
    c->score[v] = 0;
  }
  for (int e = 0; e < E; ++e)
    if (inD[e] && c->slot_of[e] >= 0) {
      int s = c->slot_of[e];
      c->last_use[s] = c->tick;
      if (c->score[s] < ORC_SCORE_MAX) c->score[s] += 1;
    }
  for (int e = 0; e < E; ++e) /* every routed expert, resident or staged, was activated by this call */
    if (inD[e] && c->act[e] < ORC_SCORE_MAX) c->act[e] += 1;
  /* split mode (READING): the host takes its share q/256 of the call's whole link work, every miss
   * (slot claims included), but only from the staged ones, the last n_host in ascending id */
  unsigned char* host_e = (unsigned char*)calloc((size_t)E, 1);
  int n_host = 0;
  if (over && c->cold == 2) {
    int n_staged = nm - ns;
    n_host = (nm * c->cold_q + 128) / 256;
    if (n_host > n_staged) n_host = n_staged;
    int seen = 0;
    for (int e = 0; e < E; ++e) {
      if (!miss[e] || c->slot_of[e] >= 0) continue; /* a staged miss */
      if (seen >= n_staged - n_host) host_e[e] = 1;
      ++seen;
    }
  }
  int count = 0;
  for (int e = 0; e < E; ++e) {
    if (!miss[e]) continue;
    desc[2 + 2 * count] = e;
    desc[3 + 2 * count] = c->slot_of[e] >= 0 ? c->slot_of[e] : (host_e[e] ? S + E + e : S + e);
    ++count;
  }
  for (int i = 0; i < n; ++i) {
    int e = ids[i];
    slot_ids[i] = c->slot_of[e] >= 0 ? c->slot_of[e] : (host_e[e] ? S + E + e : S + e);
  }
  desc[0] = over ? ORC_STAGED : ORC_SLOTS;
  desc[1] = count;
  c->misses += (uint64_t)ns;
  if (over) {
    c->staged_calls += 1;
    c->staged_copies += (uint64_t)(nm - ns - n_host);
    c->cold_misses += (uint64_t)n_host;
  }
  free(host_e);
  free(order);
  free(claim);
  free(miss);
  free(inD);
  return ORC_OK;
}

/* Whole-layer staging ([xinfer] "Prefill"): every routed id is rewritten to
 * staging record S + id; the caller copies the whole layer to staging.  The
 * slot state is untouched apart from tick.  desc = {STAGED_ALL, E, (e, S+e)...}. */
int orc_stage_all(orc_cache* c, const int32_t* ids, int n, int32_t* slot_ids, int32_t* desc) {
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->E) return ORC_EINVAL;
  c->tick += 1;
  c->calls += 1;
  c->staged_calls += 1;
  c->staged_copies += (uint64_t)c->E;
  for (int i = 0; i < n; ++i) slot_ids[i] = c->S + ids[i];
  desc[0] = ORC_STAGED_ALL;
  desc[1] = c->E;
  for (int e = 0; e < c->E; ++e) {
    desc[2 + 2 * e] = e;
    desc[3 + 2 * e] = c->S + e;
  }
  return ORC_OK;
}

/* number of distinct ids (the prefill staging decision compares it with S) */
int orc_distinct(const int32_t* ids, int n, int E) {
  unsigned char* seen = (unsigned char*)calloc((size_t)E, 1);
  int nd = 0;
  for (int i = 0; i < n; ++i)
    if (ids[i] >= 0 && ids[i] < E && !seen[ids[i]]) { seen[ids[i]] = 1; ++nd; }
  free(seen);
  return nd;
}

/* Prefetch install, [freetoken] "Install": up to max_n predicted experts that
 * are not resident become low-priority entries: kept resident at usage 0, so
 * they are the first victims.  READING:
 *   P = distinct predicted ids (pred: T rows of k ids, in top-k position order);
 *   candidates = P \ R ordered by (number of tokens predicting e descending,
 *                best top-k position ascending, id ascending);
 *   victims = slots whose expert is not in P, in the ensure's victim order;
 *   n = min(max_n, #candidates, #victims); candidate i goes to victim i with
 *   last_use = 0 (demand ticks start at 1, so these go first among occupied
 *   slots).  tick is unchanged.  desc = {SLOTS, n, (e, slot)...}. */
int orc_install(orc_cache* c, const int32_t* pred, int T, int k, int max_n, int32_t* desc) {
  int n_all = T * k;
  for (int i = 0; i < n_all; ++i)
    if (pred[i] < 0 || pred[i] >= c->E) return ORC_EINVAL;
  int E = c->E;
  int* cnt = (int*)calloc((size_t)E, sizeof(int));
  int* best = (int*)malloc(sizeof(int) * (size_t)E);
  unsigned char* inP = (unsigned char*)calloc((size_t)E, 1);
  for (int e = 0; e < E; ++e) best[e] = k;
  for (int t = 0; t < T; ++t) {
    /* a token names an expert at most once in its top-k */
    for (int j = 0; j < k; ++j) {
      int e = pred[t * k + j];
      cnt[e] += 1;
      if (j < best[e]) best[e] = j;
      inP[e] = 1;
    }
  }
  int* cand = (int*)malloc(sizeof(int) * (size_t)E);
  int nc = 0;
  for (int e = 0; e < E; ++e) {
    if (!inP[e] || c->slot_of[e] >= 0) continue;
    int pos = nc++;
    while (pos > 0 && install_before(cnt, best, e, cand[pos - 1])) {
      cand[pos] = cand[pos - 1];
      --pos;
    }
    cand[pos] = e;
  }
  int* order = (int*)malloc(sizeof(int) * (size_t)c->S);
  int nv = victim_order(c, inP, order);
  int n = max_n;
  if (nc < n) n = nc;
  if (nv < n) n = nv;
  if (n < 0) n = 0;
  for (int i = 0; i < n; ++i) {
    int v = order[i], e = cand[i];
    int old = c->expert_of[v];
    if (old >= 0) c->slot_of[old] = -1;
    c->expert_of[v] = e;
    c->slot_of[e] = v;
    c->last_use[v] = 0;
    c->score[v] = 0;
    desc[2 + 2 * i] = e;
    desc[3 + 2 * i] = v;
  }
  desc[0] = ORC_SLOTS;
  desc[1] = n;
  c->prefetch_installs += (uint64_t)n;
  free(cnt); free(best); free(inP); free(cand); free(order);
  return ORC_OK;
}

/* Profile-guided placement (READING of [npu-offload] "PolyStrata" placement,
 * a static hot set from a routing profile, mixed with the dynamic cache):
 * pin(P) makes the distinct experts P resident and never-evicted, replacing
 * any earlier pinned set.  Pinned slots are never victims of ensure or
 * install; they are used (last_use, score) like any other slot.  Steps:
 *   1. unpin every slot; experts of P already resident keep their slot and
 *      are pinned there;
 *   2. the others, ascending id, take victims in the ensure order among the
 *      slots not pinned and not holding an expert of P; each is pinned with
 *      last_use = tick (the clock does not advance) and score 0;
 *   3. desc = {SLOTS, n, (expert, slot)...} for the loads.
 * 0 <= |P| <= S - k_max is the caller's bound (so a call of k experts always
 * finds slots); here |P| <= S.  ORC_EINVAL (nothing changed) on an id out of
 * range or repeated. */
int orc_pin(orc_cache* c, const int32_t* experts, int n, int32_t* desc) {
  int E = c->E, S = c->S;
  if (n < 0 || n > S) return ORC_EINVAL;
  unsigned char* inP = (unsigned char*)calloc((size_t)E, 1);
  for (int i = 0; i < n; ++i) {
    if (experts[i] < 0 || experts[i] >= E || inP[experts[i]]) {
      free(inP);
      return ORC_EINVAL;
    }
    inP[experts[i]] = 1;
  }
  for (int s = 0; s < S; ++s) c->pinned[s] = 0;
  for (int e = 0; e < E; ++e)
    if (inP[e] && c->slot_of[e] >= 0) c->pinned[c->slot_of[e]] = 1;
  int* order = (int*)malloc(sizeof(int) * (size_t)S);
  int nv = victim_order(c, inP, order);
  int count = 0;
  for (int e = 0; e < E; ++e) {
    if (!inP[e] || c->slot_of[e] >= 0) continue;
    if (count >= nv) break; /* cannot happen for |P| <= S */
    int v = order[count];
    int old = c->expert_of[v];
    if (old >= 0) c->slot_of[old] = -1;
    c->expert_of[v] = e;
    c->slot_of[e] = v;
    c->last_use[v] = c->tick;
    c->score[v] = 0;
    c->pinned[v] = 1;
    desc[2 + 2 * count] = e;
    desc[3 + 2 * count] = v;
    ++count;
  }
  desc[0] = ORC_SLOTS;
  desc[1] = count;
  free(order);
  free(inP);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* copy (byte for byte) and the expert FFN                             */
/* ------------------------------------------------------------------ */

/* Apply a copy list: record r := host record e, into slots (r < S) or staging
 * (r >= S).  Strides are the distances between consecutive records. */
void orc_copy(const int32_t* desc, int S, const uint8_t* host, size_t host_stride, uint8_t* slots, uint8_t* staging,
              size_t dev_stride, size_t record_bytes) {
  if (desc[0] == ORC_COLD) return; /* cold experts stay on the host: nothing moves (split mode: the caller
                                       leaves the host-computed entries out of the list) */
  int count = desc[1];
  for (int i = 0; i < count; ++i) {
    int e = desc[2 + 2 * i], r = desc[3 + 2 * i];
    uint8_t* dst = r < S ? slots + (size_t)r * dev_stride : staging + (size_t)(r - S) * dev_stride;
    memcpy(dst, host + (size_t)e * host_stride, record_bytes);
  }
}

/* weight W[n][kk] of a [R][C] matrix at byte offset `off` of a record (fp8, MXFP4: times its scale) */
static double weight_at(const uint8_t* rec, int wdt, size_t off, size_t scale_off, int C, int n, int kk) {
  if (wdt == ORC_MXFP4) {
    size_t i = (size_t)n * C + kk;
    uint8_t code = (uint8_t)((rec[off + i / 2] >> (4 * (i & 1))) & 15);
    return orc_e2m1_to_f64(code) * orc_e8m0_to_f64(rec[scale_off + (size_t)n * (size_t)(C / 32) + (size_t)(kk / 32)]);
  }
  double v = load_w(rec + off, wdt, (size_t)n * C + kk);
  if (wdt == ORC_FP8) {
    float s;
    memcpy(&s, rec + scale_off + 4 * ((size_t)(n / 128) * (size_t)(C / 128) + (size_t)(kk / 128)), 4);
    v *= (double)s;
  }
  return v;
}

/* One expert on one token, [xinfer] slot tensors / the usual gated MLP:
 *   g = Wg x, u = Wu x (F each), h = silu(g) * u with silu(z) = z / (1 + e^-z),
 *   o = Wd h (H).  Everything in double on exactly widened operands. */
static void expert_ffn(const uint8_t* rec, int wdt, int H, int F, const double* x, double* h, double* o) {
  size_t esz = wdt == ORC_F32 ? 4 : (wdt == ORC_BF16 ? 2 : 1);
  size_t mat = wdt == ORC_MXFP4 ? (size_t)H * F / 2 : (size_t)H * F * esz;
  size_t nsc = wdt == ORC_MXFP4 ? (size_t)H * F / 32 : (size_t)(H / 128) * (size_t)(F / 128) * 4;
  size_t sc0 = 3 * mat;
#pragma omp parallel for schedule(static)
  for (int f = 0; f < F; ++f) {
    double g = 0.0, u = 0.0;
    for (int i = 0; i < H; ++i) {
      g += weight_at(rec, wdt, 0, sc0, H, f, i) * x[i];
      u += weight_at(rec, wdt, mat, sc0 + nsc, H, f, i) * x[i];
    }
    h[f] = g / (1.0 + exp(-g)) * u;
  }
#pragma omp parallel for schedule(static)
  for (int r = 0; r < H; ++r) {
    double acc = 0.0;
    for (int f = 0; f < F; ++f) acc += weight_at(rec, wdt, 2 * mat, sc0 + 2 * nsc, F, r, f) * h[f];
    o[r] = acc;
  }
}

/* Layer output for T tokens:
 *   y_t = sum_{j<k} w[t][j] * FFN(record of (t, j), x_t)   (in order j = 0..k-1)
 *         + FFN(shared record, x_t) if `shared` is non-null (READING: the
 *           always-resident shared expert is ungated, weight 1),
 * rounded once to the activation dtype (fp32 for fp32 weights, else bf16).
 * recs[t*k + j] points at the record that (t, j) reads.
 * y64 (optional) receives the unrounded double sums. */
void orc_ffn(const void* x, int wdt, int H, int F, int T, int k, const uint8_t* const* recs, const double* w,
             const uint8_t* shared, void* y, double* y64) {
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* hb = (double*)malloc(sizeof(double) * (size_t)F);
  double* ob = (double*)malloc(sizeof(double) * (size_t)H);
  double* acc = (double*)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; ++t) {
    for (int i = 0; i < H; ++i) xv[i] = load_act(x, wdt, (size_t)t * H + i);
    for (int i = 0; i < H; ++i) acc[i] = 0.0;
    for (int j = 0; j < k; ++j) {
      expert_ffn(recs[(size_t)t * k + j], wdt, H, F, xv, hb, ob);
      double wj = w[(size_t)t * k + j];
      for (int i = 0; i < H; ++i) acc[i] += wj * ob[i];
    }
    if (shared) {
      expert_ffn(shared, wdt, H, F, xv, hb, ob);
      for (int i = 0; i < H; ++i) acc[i] += ob[i];
    }
    for (int i = 0; i < H; ++i) {
      store_act(y, wdt, (size_t)t * H + i, acc[i]);
      if (y64) y64[(size_t)t * H + i] = acc[i];
    }
  }
  free(xv); free(hb); free(ob); free(acc);
}

/* Resolve record indices (slot ids) to record pointers: r < S -> slots, else staging. */
void orc_resolve(const int32_t* slot_ids, int n, int S, int E, const uint8_t* slots, const uint8_t* staging,
                 const uint8_t* host, size_t stride, const uint8_t** recs) {
  for (int i = 0; i < n; ++i) {
    int r = slot_ids[i];
    if (r < S) recs[i] = slots + (size_t)r * stride;
    else if (r < S + E) recs[i] = staging + (size_t)(r - S) * stride;
    else recs[i] = host + (size_t)(r - S - E) * stride; /* a cold expert: its host record */
  }
}

/* Residual stream between layers (READING): the MoE block adds its output to
 * the stream, x_next = x + y, rounded once to the activation dtype, with y
 * already rounded. */
void orc_residual(const void* x, const void* y, int wdt, size_t n, void* out) {
  for (size_t i = 0; i < n; ++i) store_act(out, wdt, i, load_act(x, wdt, i) + load_act(y, wdt, i));
}

/* Input of each MoE block (READING): the stream normalised to unit root mean
 * square per token, xn = x / sqrt(mean(x^2) + eps), no learned scale, rounded
 * once to the activation dtype.  The pages describe no norm; without one the
 * residual stream of a 48-layer chain of gated FFNs with N(0, 0.02) weights
 * grows until it overflows, while the pre-norm block of the model family the
 * configurations are shaped after keeps it bounded.
 * The norm is glue around the layer, so its arithmetic is fixed here the way
 * the router logits' is (READING): binary32 throughout, in one order, so that
 * the activation codes it produces are a definition rather than a tolerance:
 *   - 256 partial sums; partial i takes the 8-element chunks c = i, i + 256, ...
 *     in ascending order and accumulates v*v with fused multiply-adds in
 *     element order;
 *   - the partials form four groups of 64; within a group, an xor butterfly:
 *     for o = 32, 16, ..., 1, partial l becomes partial l + partial (l ^ o);
 *   - the four group sums are added left to right;
 *   - inv = 1 / sqrt(sum / H + eps), each operation correctly rounded;
 *   - xn = x * inv in binary32, then rounded once to the activation dtype. */
void orc_rmsnorm(const void* x, int wdt, int T, int H, double eps, void* out) {
  const float epsf = (float)eps;
  for (int t = 0; t < T; ++t) {
    const size_t base = (size_t)t * H;
    float part[256], grp[4];
    for (int i = 0; i < 256; ++i) {
      float ss = 0.0f;
      for (int c = i; c * 8 < H; c += 256)
        for (int q = 0; q < 8; ++q) {
          const float v = (float)load_act(x, wdt, base + (size_t)c * 8 + q);
          ss = fmaf(v, v, ss);
        }
      part[i] = ss;
    }
    for (int g = 0; g < 4; ++g) {
      float a[64], b[64];
      memcpy(a, part + 64 * g, sizeof a);
      for (int o = 32; o >= 1; o >>= 1) {
        for (int l = 0; l < 64; ++l) b[l] = a[l] + a[l ^ o];
        memcpy(a, b, sizeof a);
      }
      grp[g] = a[0];
    }
    const float tot = ((grp[0] + grp[1]) + grp[2]) + grp[3];
    const float inv = 1.0f / sqrtf(tot / (float)H + epsf);
    for (int i = 0; i < H; ++i)
      store_act(out, wdt, base + i, (double)((float)load_act(x, wdt, base + i) * inv));
  }
}

/* threads the OpenMP loops above use (for reporting how the oracle was timed) */
int orc_threads(void) { return omp_get_max_threads(); }

/* threads for the parallel loops from now on (n < 1: all the host's processors) */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : omp_get_num_procs()); }
