/*
 * moe_offload.h — C ABI of the offloaded Mixture-of-Experts layer step on
 * one MI355X (gfx950).
 *
 * One handle = one MoE layer.  Every routed expert of the layer lives in a
 * pinned, device-mapped host store; the layer keeps `num_slots` of them in a
 * device slot tensor [num_slots, record] with a least-recently-used table.
 * A decode call is:
 *
 *     moe_route_topk   -> ids[T,k], w[T,k]
 *     moe_slot_ensure  -> slot_ids[T,k]    (LRU lookup, victim choice, id rewrite,
 *                                           copy list and miss count in device memory)
 *     moe_copy_misses  -> missing records copied from mapped host memory
 *     moe_slot_ffn     -> y[T,H] (and optionally x + y)
 *
 * All four are asynchronous on the caller's stream, never synchronise the
 * host and use launch shapes that depend only on the handle and T, so a
 * whole decode step can be captured once in a HIP graph and replayed.
 *
 * Sources (cited by section):
 *   xinfer-ai 0.14.6, docs/moe_offload.md (npm diff page on my.diffend.io):
 *     "How it works" — Decode (per-layer LRU table on the GPU, least-recently-used
 *     slots for misses, expert ids rewritten to slot ids, a second kernel copying
 *     the missing experts from device-mapped pinned host memory, fixed launch
 *     shapes with the miss count read from device memory, graph capture without
 *     host sync), Prefill (whole-layer staging when a call touches more distinct
 *     experts than slots), and the GEMM reading [num_slots, N, K] instead of
 *     [num_experts, N, K]; "Supported" — every [E, ...] tensor (weights and scales)
 *     in host RAM, inputs outside the supported set rejected with an explanatory
 *     message; the opening paragraph — the share of experts kept on the GPU
 *     alters neither the routing nor the numerics.
 *   FreeToken issue #677, "Proposal" — router lookahead, install of predicted
 *     experts as low-priority slots (usage 0, first evicted), copy on a side
 *     stream, every slot-map writer on the compute stream.
 *
 * Conventions
 *   - Return value: 0 on success, a negative MOE_E* code on failure; the
 *     message of the last failure on this host thread is moe_offload_last_error().
 *     No call aborts or throws across the ABI.
 *   - Errors found on the device (an expert id outside [0, E), a NaN router
 *     logit, an audit failure) cannot be returned by asynchronous calls; they
 *     set a sticky error word in the handle, reported by moe_offload_stats()
 *     (which synchronises) and cleared by moe_offload_reset().  A call that
 *     finds a bad id changes no slot state and writes an empty copy list.
 *   - Pointers named `*_dev` or described as device pointers must be device
 *     (or device-mapped) memory owned by the caller and valid until the work
 *     queued on `stream` has finished.  `stream` is a hipStream_t passed as
 *     void*; NULL means the null stream.
 *   - One host thread at a time per handle.  Calls on one handle are ordered
 *     by the caller's streams: the slot table has exactly one writer
 *     (moe_slot_ensure, moe_prefill_stage, moe_prefetch_install), which must
 *     all be issued on the same (compute) stream.
 *
 * Record layout (one expert, `record_bytes`, records `record_stride` apart):
 *     gate [F][H] | up [F][H] | down [H][F] | (fp8, MXFP4) scales
 *   rows are contiguous along the reduction dimension; elements are fp32,
 *   bf16, fp8 e4m3 (OCP "fn": bias 7, no infinities), or MXFP4.  fp8 records
 *   end with fp32 block scales, one per 128 x 128 block, row-major: gate
 *   [F/128][H/128], up [F/128][H/128], down [H/128][F/128]; weight =
 *   decode(q) * scale.  MXFP4 (OCP Microscaling v1.0): E2M1 codes, two per
 *   byte, element 2i of a row in the low nibble; then E8M0 scale bytes, one per
 *   32 consecutive weights of a row: gate [F][H/32], up [F][H/32], down
 *   [H][F/32]; weight = e2m1(q) * 2^(e - 127).
 *
 * Record index ("slot id") space used by slot_ids:
 *   r in [0, S)          slot r of the slot tensor
 *   r in [S, S + E)      staging record r - S (expert r - S staged for this call)
 *   r in [S + E, S + 2E) cold mode: expert r - S - E, computed by the host CPU from its host record
 */
#ifndef MOE_OFFLOAD_H
#define MOE_OFFLOAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_offload moe_offload;

/* weight/activation formats */
enum moe_dtype {
  MOE_F32 = 0,            /* fp32 weights, fp32 activations */
  MOE_BF16 = 1,           /* bf16 weights, bf16 activations */
  MOE_FP8_E4M3_B128 = 2,  /* fp8 e4m3 weights + fp32 128x128 block scales, bf16 activations */
  MOE_MXFP4 = 3           /* MXFP4 weights (E2M1 + E8M0 per 32), bf16 activations; H, F multiples of 256 */
};

/* return codes */
enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument (shape, size, null pointer, S < k, ...) */
  MOE_ENOMEM = -2,        /* device or pinned host allocation failed */
  MOE_EHIP = -3,          /* a HIP runtime call failed */
  MOE_EUNSUPPORTED = -4,  /* a dtype or shape the library does not handle */
  MOE_EDEVICE = -5        /* a sticky device-side error is set (see stats.error) */
};

/* bits of moe_stats.error (sticky, device-side) */
enum {
  MOE_DEV_ERR_BAD_ID = 1,     /* a routed or predicted id outside [0, E) */
  MOE_DEV_ERR_NAN = 2,        /* a NaN router logit (selection then treats it as -inf) */
  MOE_DEV_ERR_AUDIT = 4,      /* audit mode: slot maps not mutually inverse, or a needed expert not resident */
  MOE_DEV_ERR_HOST_TIMEOUT = 8 /* a decode chain gave up waiting (half a second or more) for the host's rows of a
                                  cold-mode layer; that call's host-computed outputs are stale */
};
/* (A call with more pairs than max_tokens * top_k cannot reach the device: every
 * entry point rejects T > max_tokens with MOE_EINVAL before it launches.) */

/* creation flags */
enum {
  MOE_FLAG_AUDIT = 1,          /* check the slot table after every ensure/install (sets MOE_DEV_ERR_AUDIT) */
  MOE_FLAG_HOST_COHERENT = 2,  /* fine-grained (coherent) host store instead of coarse-grained */
  MOE_FLAG_SCORED = 4,         /* scored eviction: victims by (occupied, usage score, last_use, slot) */
  MOE_FLAG_FREQ = 8            /* activation-aware eviction (MoE-Infinity README, "Overview": the cache keeps
                                  the most often activated experts): victims by (occupied, installed and
                                  unused first, activation count of the held expert, last_use, slot); the
                                  count of an expert is the number of ensure calls that routed to it since
                                  create or reset (saturating at 2^20 - 1), kept across evictions.
                                  Exclusive with MOE_FLAG_SCORED. */
};

typedef struct {
  int32_t num_experts;   /* E, 1..1024 */
  int32_t num_slots;     /* S, top_k <= S <= E (xinfer-ai docs, "Options": the slot count never falls
                            below what one token's top-k needs) */
  int32_t hidden;        /* H, multiple of 64 for MOE_F32, of 128 otherwise */
  int32_t ffn;           /* F, multiple of 64 for MOE_F32, of 128 otherwise */
  int32_t top_k;         /* k, 1..16 */
  int32_t dtype;         /* enum moe_dtype */
  int32_t max_tokens;    /* largest T of any call, 1..65536 */
  int32_t device;        /* HIP device ordinal */
  uint32_t flags;        /* MOE_FLAG_* */
  /* Optional sharing between the layers of one model (all calls of the
   * sharing handles on one stream).  The owner must outlive every sharer.
   *   share_host:    read this handle's host store instead of allocating one
   *                  (same E, dtype, H, F).  Used when host RAM cannot hold
   *                  every layer: layers then alias the same expert bytes.
   *   share_staging: use this handle's staging buffer (same E, dtype, H, F). */
  const moe_offload* share_host;
  const moe_offload* share_staging;
} moe_offload_desc;

typedef struct {
  uint64_t calls;             /* ensure + prefill-stage calls */
  uint64_t hits;              /* distinct routed experts found resident */
  uint64_t misses;            /* demand misses copied into slots */
  uint64_t staged_calls;      /* calls with more distinct experts than slots */
  uint64_t staged_copies;     /* misses of those calls copied into staging */
  uint64_t prefetch_installs; /* experts installed by moe_prefetch_install */
  uint64_t prefetch_hits;     /* installed experts found by a later ensure before any other use */
  uint64_t bytes_copied;      /* bytes moved host -> device by this handle */
  uint64_t tick;              /* LRU clock (ensure and stage calls) */
  int32_t error;              /* sticky MOE_DEV_ERR_* bits */
  int32_t resident;           /* experts currently resident in slots */
  uint64_t cold_misses;       /* misses computed on the host in cold or split mode */
} moe_stats;

/* Device addresses and sizes of the handle's state, for inspection and tests.
 * The arrays are owned by the handle; writing them is allowed only for
 * fault-injection tests of the audit mode. */
typedef struct {
  int32_t* slot_of;       /* [E]  slot of each expert, -1 = not resident */
  int32_t* expert_of;     /* [S]  expert in each slot, -1 = free */
  uint64_t* last_use;     /* [S]  tick of last use; 0 = never used (free or prefetched) */
  int32_t* copy_list;     /* [2 + 2*max(S,E)]  {mode, count, (expert, record index) x count} */
  int32_t* prefetch_list; /* [2 + 2*S]         {0, count, (expert, slot) x count} */
  void* slots;            /* device [S, record_stride] */
  void* staging;          /* device [E, record_stride] */
  void* host;             /* host store [E, record_stride] (host address) */
  void* host_dev;         /* the same store as a device address */
  void* ffn_h;            /* FFN workspace: h rows [max_tokens*(k+1)][F] (bf16, fp32 for MOE_F32) */
  float* ffn_part;        /* FFN workspace: per-(t, j) expert outputs [max_tokens*(k+1)][H] fp32 */
  int32_t* ffn_groups;    /* FFN workspace: {records, list, starts, pair ids} of the last call */
  size_t record_bytes;
  size_t record_stride;
  int32_t E, S, H, F, k, dtype, max_tokens, device;
  uint32_t* score;        /* [S]  usage score: ensure calls routed to the slot's expert since it was loaded
                             (saturating at 2^20 - 1); kept under both policies, used by MOE_FLAG_SCORED */
  int32_t* pinned;        /* [S]  1: the slot's expert is pinned (moe_offload_pin), never a victim */
  uint32_t* act;          /* [E]  activation count per expert (ensure calls routing to it; kept under every
                             policy, used by MOE_FLAG_FREQ) */
} moe_info;

/* copy-list modes (copy_list[0]); MOE_MODE_COLD: the listed misses are computed on the host
 * (record index S + E + e), nothing is copied */
enum { MOE_MODE_SLOTS = 0, MOE_MODE_STAGED = 1, MOE_MODE_STAGED_ALL = 2, MOE_MODE_COLD = 3 };

/* Create one layer's handle: pinned mapped host store [E, record_stride]
 * (contents undefined until the caller writes it), slot tensor, slot table
 * (empty cache, tick 0), copy lists, staging buffer [E, record_stride],
 * workspaces and counters.  Later calls never allocate.
 * Errors: MOE_EINVAL (shape/limits), MOE_EUNSUPPORTED (dtype), MOE_ENOMEM, MOE_EHIP. */
int moe_offload_create(const moe_offload_desc* desc, moe_offload** out);

/* Slot count for automatic sizing (xinfer-ai 0.14.6 docs/moe_offload.md,
 * "Options", `auto`: after loading, every layer's slots grow by the same
 * amount into the free device memory, leaving a reserve for the KV cache and
 * workspaces).  For `layers` handles created with *d (num_slots ignored):
 *   S = min(E, floor((free - reserve - staging - layers * state) / (layers * record_stride)))
 * where staging is one [E, record_stride] buffer (share_staging != 0: the
 * layers share one, as moe_offload_desc.share_staging allows) or one per layer,
 * and state is a handle's state block (tables, lists, workspaces) at its
 * largest.  free_bytes = 0: the device's free memory now (hipMemGetInfo on
 * d->device); otherwise the given figure, and no device is touched.
 *   *slots_out: the S to pass to moe_offload_create for every layer.
 * Errors: MOE_EINVAL / MOE_EUNSUPPORTED (the descriptor, layers < 1),
 * MOE_ENOMEM when not even top_k slots per layer fit (*slots_out = top_k),
 * MOE_EHIP. */
int moe_offload_auto_slots(const moe_offload_desc* d, int32_t layers, int32_t share_staging, uint64_t reserve_bytes,
                           uint64_t free_bytes, int32_t* slots_out);

/* Synchronise the device, free everything the handle owns.  Null-safe. */
void moe_offload_destroy(moe_offload* h);

/* The host store, so the caller can write expert records in place
 * (record e at host + e * record_stride).  Host address; pinned, mapped. */
int moe_offload_host_records(moe_offload* h, void** host, size_t* record_stride, size_t* record_bytes);

/* Router (xinfer-ai 0.14.6 docs/moe_offload.md, "How it works", Decode: the
 * routed experts of each call are what the slot table is asked for; opening
 * paragraph: slot placement leaves this routing untouched).
 * Logits l = x Wr^T + b (binary32, one fixed summation order: chunks
 * of 8 elements, 64 lanes each owning every 64th chunk, an FMA chain per lane,
 * an xor-butterfly over the lanes, then + b), top-k by (logit descending, id
 * ascending), weights = softmax over the k chosen logits.
 *   x:        device [T, H], fp32 (MOE_F32) or bf16
 *   w_router: device [E, H], fp32 (MOE_F32) or bf16
 *   bias:     device [E] fp32
 *   ids:      device [T, k] int32 (out);  w: device [T, k] fp32 (out)
 * 1 <= T <= max_tokens.  Asynchronous, capture-safe. */
int moe_route_topk(moe_offload* h, const void* x, const void* w_router, const float* bias, int32_t T,
                   int32_t* ids, float* w, void* stream);

/* LRU slot table update for one call (xinfer-ai 0.14.6 docs/moe_offload.md,
 * "How it works", Decode: look-up in a per-layer LRU table on the GPU,
 * least-recently-used slots for the misses, expert ids rewritten to slot ids,
 * the miss count left in device memory, a fixed launch shape; single workgroup):
 * D = distinct ids.  Victims are the slots not holding an expert of D, in
 * (free first, then least recently used, then lowest slot) order; with
 * MOE_FLAG_SCORED, (free first, then lowest usage score, then least recently
 * used, then lowest slot), the score counting the calls that routed to the
 * slot's expert since it was loaded.  Every slot used by the call gets
 * last_use = tick and its score incremented (a slot just loaded: 1).
 * |D| <= S: misses (ascending id) take the victims; copy list
 * {SLOTS, |misses|, (expert, slot)...}.  |D| > S (decode batches wider than
 * the cache; the page stages whole layers only for prefill): the victims are
 * fewer than the misses and go to the misses routed by most pairs (then best
 * top-k position, then lowest id); every other miss e is staged for this call
 * and read at S + e; copy list {STAGED, |misses|, (expert, slot or S + e)...}
 * in ascending expert id.  Residents are read in place, ids are rewritten to
 * record indices, and every expert of D holding a slot becomes most recent.
 *   ids: device [T, k] int32;  slot_ids: device [T, k] int32 (out).
 * Asynchronous, capture-safe; the table's only writer besides install/stage. */
int moe_slot_ensure(moe_offload* h, const int32_t* ids, int32_t T, int32_t* slot_ids, void* stream);

/* Miss copy (xinfer-ai 0.14.6 docs/moe_offload.md, "How it works", Decode: a
 * second kernel moves the missing experts from device-mapped pinned host
 * memory into their slots, its launch shape fixed and its count read on the
 * device).
 * Copy the current copy list's records from the mapped host store into slots
 * or staging with 16-byte loads (fixed grid; the count is read on the device,
 * an empty list costs one empty launch).  No-op for MOE_MODE_STAGED_ALL.
 * Asynchronous, capture-safe. */
int moe_copy_misses(moe_offload* h, void* stream);

/* Expert FFN and combine over the slot tensor (xinfer-ai 0.14.6
 * docs/moe_offload.md, "How it works": the expert GEMMs read [num_slots, N, K]
 * slot tensors in place of [num_experts, N, K]):
 *   y_t = sum_j w[t][j] * Wd_r silu(Wg_r x_t) * (Wu_r x_t)   (j = 0..k-1 in order)
 *         + the same FFN of shared_record on x_t (weight 1) if shared_record != NULL,
 *   r = slot_ids[t][j] (slot or staging record), rounded once to the activation dtype.
 *   x: device [T, H]; slot_ids: device [T, k]; w: device [T, k] fp32;
 *   shared_record: NULL or a device record (same layout/dtype, caller-owned, always resident);
 *   y: device [T, H] (out);
 *   x_next: NULL or device [T, H] (out) = round(residual + y), the residual stream after
 *           the block; residual: device [T, H], or NULL to add to x itself.
 * Results do not depend on which slot holds an expert or on S.
 * Asynchronous, capture-safe. */
int moe_slot_ffn(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int32_t T,
                 const void* shared_record, void* y, const void* residual, void* x_next, void* stream);

/* Kernel pair of the expert FFN for calls of 2 to 64 tokens (xinfer-ai docs,
 * "How it works": decode and prefill are the same grouped FFN; which kernels
 * run is an implementation choice that never changes which experts are used).
 *   MOE_FFN_AUTO (the default): the grouped MFMA GEMM when T * k >= c * E, with
 *     c = 5 for bf16, 1 for MXFP4 and 1/8 for fp8 (the measured crossovers: the
 *     decode kernels read each weight row once per 8-token group of a record,
 *     the GEMM once per tile of up to 80 pairs), else the pair-dot decode
 *     kernels;
 *   MOE_FFN_DECODE: always the decode kernels;  MOE_FFN_GEMM: always the GEMM.
 * Calls of one token always take the single-token kernels, calls above 64
 * tokens the GEMM, fp32 layers their fp32 kernels.  The choice depends on T
 * and the handle only, never on S or on residency, so outputs stay bitwise
 * independent of the slot count; the two pairs differ in summation order, so
 * their outputs agree within the usual tolerance, not bit for bit.  Only the
 * decode kernels read missed records through (decode chain).  Host-side
 * setting; a decode chain keeps the kernels it captured at its first run.
 * Errors: MOE_EINVAL (unknown path). */
enum { MOE_FFN_AUTO = 0, MOE_FFN_DECODE = 1, MOE_FFN_GEMM = 2 };
int moe_offload_set_ffn_path(moe_offload* h, int32_t path);

/* Workgroup size of the grouped GEMM (the kernels of prefill-sized calls,
 * xinfer-ai docs, "How it works", Prefill; an implementation choice).  Each
 * wavefront owns 16 rows of gate and of up (32 of down) and every pair of a
 * token tile, so a workgroup of 8 wavefronts fetches each tile's token rows
 * once per 128 rows of gate and up (256 of down) instead of once per 64 (128),
 * and has the registers to load them two K slices ahead, but holds one
 * workgroup per compute unit, too few for small calls.
 *   0 (the default): 8 wavefronts when the call has at least 1024 work items
 *     of theirs, counted as (T * k / 64) token tiles times (F / 128) row tiles
 *     for gate/up, (H / 256) for down (about four per compute unit), else 4
 *     (measured: DeepSeek-V3- and Mixtral-shaped 2048-token calls 10 to 20 %
 *     faster, 64-token calls 7 to 45 % slower);
 *   4 or 8: always that many (down keeps 4 when H is not a multiple of 256).
 * Every output element sums the same products in the same order either way:
 * outputs are bitwise identical.  Host-side setting.
 * Errors: MOE_EINVAL (waves not 0, 4 or 8). */
int moe_offload_set_gemm_waves(moe_offload* h, int32_t waves);

/* Host-computed cold experts (npu-offload README, intro and "Architecture":
 * hot experts stay in accelerator memory, the host CPU computes the cold ones
 * from host DRAM in parallel, only activations cross the link; "Results", where
 * the time goes: the CPU's share is bound by DRAM bandwidth).
 * In cold mode an ensure call loads nothing: hits are used in place (last_use,
 * usage score and activation count as usual), each miss e keeps no slot, takes
 * no victim and is read at record index S + E + e; the copy list is
 * {MOE_MODE_COLD, |misses|, (e, S + E + e)...} in ascending id and the copy
 * kernel moves nothing; stats.cold_misses counts them.
 *   mode: MOE_COLD_OFF, MOE_COLD_ON, or MOE_COLD_AUTO: measure, for one record
 *         of this layer, the host FFN at one token (on the library's worker
 *         threads) against a pinned host-to-device copy of the record, and turn
 *         the cold mode on when the host is faster (the layer's misses then go
 *         to the CPU instead of over the link);
 *         or MOE_COLD_SPLIT: the same measurement, then split mode with the
 *         host's share q = round(256 * link / (cpu + link)) (moe_offload_set_split).
 *   chosen (may be NULL): the resulting mode (0 off, 1 on), or for MOE_COLD_SPLIT
 *         the share q in [0, 256];
 *   cpu_us, link_us (may be NULL): the two measured times per record (AUTO and
 *         SPLIT; 0 otherwise).
 * Cold mode freezes the resident set (nothing is loaded while it is on), so
 * switch it on once the cache has warmed over the link or been pinned to a
 * profiled hot set; from an empty cache every expert stays cold.
 * Host-synchronising on `stream`; the flag is written on the device in stream
 * order, so issue it on the compute stream between calls.  Switching on the
 * first time allocates the pinned host buffers the cold FFN uses (max_tokens
 * rows).  While the mode is on, the FFN must be moe_slot_ffn_host_cold
 * (moe_slot_ffn refuses the handle with MOE_EINVAL) or a decode chain, which
 * computes the host's share on a thread of its own (moe_chain_run).
 * Errors: MOE_EINVAL, MOE_ENOMEM, MOE_EHIP. */
enum { MOE_COLD_OFF = 0, MOE_COLD_ON = 1, MOE_COLD_AUTO = 2, MOE_COLD_SPLIT = 3 };
int moe_offload_set_cold(moe_offload* h, int32_t mode, void* stream, int32_t* chosen, double* cpu_us,
                         double* link_us);

/* Split mode (same pages: the host's DRAM-bound FFN and the host link are two
 * independent channels out of host memory; a call wider than the cache uses
 * both).  Calls that fit the cache are unchanged (mode SLOTS).  In a call that
 * overflows (mode STAGED), slot claims, victims, usage updates and copy-list
 * order are unchanged; of the n staged misses (those that got no slot), the
 * last h = min(n, floor((m * q + 128) / 256)) in ascending id, m being all the
 * call's misses (the link's whole work), are computed on the host:
 * their record index is S + E + e in slot_ids and in the copy list, the copy
 * kernel skips them, stats.staged_copies counts the other n - h and
 * stats.cold_misses the h.
 *   q: the host's share of the call's misses in 1/256, in [0, 256] (0: every
 *      staged miss crosses the link, as with the mode off; 256: none does).
 * While split mode is on the FFN must be moe_slot_ffn_host_cold, and the
 * activations x it receives must already be final when the call's
 * moe_slot_ensure is enqueued (they are whenever x fed moe_route_topk before
 * it): the host reads the call's indices and activations on a stream of its
 * own as soon as the ensure has run, so its share overlaps the copy kernel.
 * A call of at most S - P pairs (P: the size of the pinned set) cannot
 * overflow: moe_slot_ffn_host_cold runs it as moe_slot_ffn would, with no host
 * round trip, and its outputs are those of moe_slot_ffn bit for bit.
 * Host-synchronising on `stream`; MOE_COLD_OFF (moe_offload_set_cold) ends it.
 * Errors: MOE_EINVAL (q outside [0, 256]), MOE_ENOMEM, MOE_EHIP. */
int moe_offload_set_split(moe_offload* h, int32_t q, void* stream);

/* The expert FFN of a cold-mode call (same arguments and results as
 * moe_slot_ffn): the GPU computes the resident experts while the host CPU
 * computes every pair whose record index is S + E + e from expert e's host
 * record (fp32 sums; h kept in fp32), then the host's rows join the GPU's in
 * the same top-k weighted combine.  Host-synchronising (it waits for the
 * call's indices and activations), not capturable.  Outputs match the plain
 * definition within the same tolerance as the GPU path, not bit for bit.
 * Errors: as moe_slot_ffn; MOE_EINVAL if the cold mode was never switched on. */
int moe_slot_ffn_host_cold(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int32_t T,
                           const void* shared_record, void* y, const void* residual, void* x_next, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): moe_slot_ffn with the
 * same arguments and the same results, bit for bit, whose workspace (the
 * grouping of the call's pairs by record, the h rows and the fp32 per-choice
 * outputs) lives in one file-scope device array of MOE_NOALLOC_SCRATCH_BYTES
 * per GPU instead of the handle's workspace.  The array's device address is
 * looked up once per device by moe_offload_create; this call allocates and
 * frees nothing.  Every call on one GPU shares that array: calls that overlap
 * on one GPU (other streams, other handles, other host threads) race and
 * must be ordered by the caller.  Nothing in it needs to start at zero.
 * Errors: as moe_slot_ffn, and MOE_EINVAL when the call's workspace,
 * 256-aligned (4 x (32 x (min(T k, S + E) + 2) + T k + min(T k, S + E) + 2)
 * bytes) + (T k + T) F (2, or 4 for MOE_F32) + 4 (T k + T) H bytes, exceeds
 * MOE_NOALLOC_SCRATCH_BYTES. */
#define MOE_NOALLOC_SCRATCH_BYTES (32ull << 20)
int moe_slot_ffn_noalloc(moe_offload* h, const void* x, const int32_t* slot_ids, const float* w, int32_t T,
                         const void* shared_record, void* y, const void* residual, void* x_next, void* stream);

/* Per-token RMS normalisation, out = round(x / sqrt(mean(x^2) + eps)) (fp32 arithmetic,
 * no learned scale): the input of each MoE block in the decode-step chain.  The pages
 * describe no norm; it is the library's reading of the inter-layer glue (a 48-layer
 * residual chain of gated FFNs without one overflows).
 *   x, out: device [T, H], fp32 (MOE_F32) or bf16 (otherwise); H a multiple of 8.
 * Asynchronous, capture-safe. */
int moe_rmsnorm(const void* x, void* out, int32_t T, int32_t H, int32_t dtype, float eps, void* stream);

/* Prefill entry (xinfer-ai 0.14.6 docs/moe_offload.md, "How it works",
 * Prefill: a call needing more distinct experts than the layer has slots gets
 * the whole layer copied into a staging buffer by a pinned asynchronous copy,
 * and the GEMMs read the staging buffer).
 * Host-synchronising, not capturable: count the distinct ids
 * of the call.  More than S: copy the whole layer host -> staging with an
 * asynchronous DMA copy, rewrite ids to S + id, copy list {STAGED_ALL, E, ...},
 * slot table untouched (tick advances), *staged_out = 1.  Otherwise run
 * moe_slot_ensure + moe_copy_misses, *staged_out = 0.
 *   ids: device [T, k]; slot_ids: device [T, k] (out); staged_out: host int32 (may be NULL).
 * Returns MOE_EDEVICE (nothing queued) if an id is out of range. */
int moe_prefill_stage(moe_offload* h, const int32_t* ids, int32_t T, int32_t* slot_ids, int32_t* staged_out,
                      void* stream);

/* Router-lookahead prefetch, install half (FreeToken #677 "Install"): for
 * the predicted ids of the *next* layer (this handle), take up to max_n
 * predicted experts that are not resident, ordered by (number of tokens
 * predicting them desc, best top-k position asc, id asc), and place them in
 * victim slots (same order as ensure, never a slot holding a predicted
 * expert) with last_use = 0 and usage score 0, i.e. evicted first.  Writes the prefetch copy
 * list.  Must be issued on the compute stream (single slot-table writer).
 *   pred_ids: device [T, k] int32.  0 <= max_n <= S. */
int moe_prefetch_install(moe_offload* h, const int32_t* pred_ids, int32_t T, int32_t max_n, void* stream);

/* Profile-guided placement (npu-offload README, PolyStrata placement: a hot
 * set from a routing profile, here mixed with the dynamic cache): make the n
 * distinct experts experts_dev[0..n) resident and pinned, replacing any
 * earlier pinned set.  Pinned slots are never victims of ensure or install
 * and are used like any other slot.  Members already resident are pinned in
 * place; the others (ascending id) take victims in the ensure order among
 * slots not pinned and not holding a member, with last_use = the current
 * tick and score 0, and are copied in (the copy list is reused).  With pins,
 * an ensure call overflows when its misses outnumber the unpinned victims.
 *   experts_dev: device int32 [n];  0 <= n <= S - k (else MOE_EINVAL).
 * An id out of range or repeated: nothing changes, the sticky bad-id bit is
 * set.  Asynchronous; a slot-table writer: issue it on the compute stream. */
int moe_offload_pin(moe_offload* h, const int32_t* experts_dev, int32_t n, void* stream);

/* Prefetch copy (FreeToken issue #677, "Proposal", Install: the installed
 * experts move on a separate stream, and the layer's own miss copy is ordered
 * after them).  Copies the prefetch copy list's records from the mapped host
 * store into their slots; it may run on a side stream after an event that
 * follows the install, and this layer's FFN (and demand copy) must wait for it.
 * Asynchronous, capture-safe. */
int moe_copy_prefetch(moe_offload* h, void* stream);

/* Synchronise the device and read the counters and the sticky error word. */
int moe_offload_stats(moe_offload* h, moe_stats* out);

/* Empty the cache (all slots free and unpinned, tick 0), zero the counters
 * and the sticky error word, on `stream`. */
int moe_offload_reset(moe_offload* h, void* stream);

/* Fill `out` with the device addresses and sizes of the handle's state. */
int moe_offload_query(const moe_offload* h, moe_info* out);

/* Message of the last failing call on this host thread ("" if none). */
const char* moe_offload_last_error(void);

/* ------------------------------------------------------------------ */
/* Per-kernel timing (opt-in, for measurement).                        */
/* ------------------------------------------------------------------ */
/* Not from the pages: a measurement aid.  While profiling is on, every
 * kernel the handle launches on a stream that is not being captured is
 * bracketed by two HIP events recorded on that same stream; the elapsed times
 * accumulate per kernel kind.  The host waits for a kind's previous pair only
 * when it records the next pair of that kind (or when the times are read).
 * Launches inside graph capture are not timed. */
enum moe_kernel_kind {
  MOE_K_LOGITS = 0,   /* router logits */
  MOE_K_TOPK = 1,     /* top-k + weights (moe_route_topk) */
  MOE_K_DECIDE = 2,   /* fused decode control: top-k + ensure + grouping (chain) */
  MOE_K_ENSURE = 3,   /* moe_slot_ensure, moe_offload_pin */
  MOE_K_INSTALL = 4,  /* moe_prefetch_install */
  MOE_K_COPY = 5,     /* demand / staging / pin copy (moe_copy_misses, prefill, moe_offload_pin) */
  MOE_K_PF_COPY = 6,  /* prefetch copy (moe_copy_prefetch) */
  MOE_K_GROUP = 7,    /* FFN grouping by record */
  MOE_K_GATEUP = 8,   /* FFN gate/up + SiLU */
  MOE_K_DOWN = 9,     /* FFN down projection */
  MOE_K_COMBINE = 10, /* top-k weighted combine (+ residual, + next norm) */
  MOE_K_STAGE = 11,   /* prefill: distinct count, whole-layer id rewrite */
  MOE_K_N = 12
};

typedef struct {
  double ms[MOE_K_N];          /* summed event time per kind, milliseconds */
  uint64_t launches[MOE_K_N];  /* timed launches per kind */
} moe_kernel_times;

/* enable != 0: start (or restart) timing with zeroed sums; 0: stop.  The
 * first call with enable != 0 creates the handle's events.
 * Errors: MOE_EINVAL, MOE_EHIP. */
int moe_offload_profile(moe_offload* h, int32_t enable);

/* Wait for the pending event pairs and read the sums. */
int moe_offload_kernel_times(moe_offload* h, moe_kernel_times* out);

/* ------------------------------------------------------------------ */
/* Decode-step chain: L layers captured once into one HIP graph.       */
/* ------------------------------------------------------------------ */
/* xinfer-ai 0.14.6 docs/moe_offload.md, "How it works", Decode: the offloaded
 * decode step stays inside a captured graph with no host synchronisation.
 * For l = 0 .. L-1 the chain issues, on one compute stream,
 *     xn_l = rmsnorm(x_l) -> route(layer l, xn_l) -> ensure -> copy -> ffn(xn_l) -> y_l,
 *     x_{l+1} = round(x_l + y_l)
 * (a pre-norm residual stream between MoE layers; no other sublayer is modelled).
 * prefetch_n > 0 builds the router-lookahead variant (FreeToken issue #677,
 * "Proposal"): layer l's router (l >= 1) also runs on layer l-1's router input
 * xn_{l-1}, and layer l-1's control step installs up to prefetch_n of the
 * predicted experts into layer l (every slot-table writer stays on the compute
 * stream).  The installed records move on a separate copy stream, started
 * once layer l-1's own missed records are in hand (after its copy launch; with
 * read-through, after its control step, so it shares the link with that
 * layer's FFN launches, which fetch its misses themselves; starting it after
 * those launches instead was measured slower on the same tokens); nothing of
 * layer l that reads slots starts before that copy has finished.  All streams
 * have the default priority.
 *
 * The chain owns its activation buffers (device):
 *   x      [L+1][T][H]  x[0] is the step input (caller writes it before run), x[l+1] = x[l] + y[l]
 *   xn     [L][T][H]    rmsnorm(x[l]) (eps 1e-6): layer l's router and expert input
 *   y      [L][T][H]    layer outputs before the residual add
 *   ids    [L][T][k] int32, w [L][T][k] fp32, slot_ids [L][T][k] int32
 *   pred   [L][T][k] int32 lookahead predictions (prefetch variant; row l = prediction for layer l)
 * Activations are fp32 for MOE_F32 layers, bf16 otherwise.
 *   layers:        L handles (same H, k, dtype; T <= each max_tokens); not owned
 *   w_router:      L device pointers [E][H]; bias: L device pointers [E] fp32 (caller-owned)
 *   shared_records: NULL or L device pointers (each may be NULL)
 * Errors: MOE_EINVAL, MOE_ENOMEM, MOE_EHIP. */
typedef struct moe_chain moe_chain;

typedef struct {
  void* x;
  void* xn;
  void* y;
  int32_t* ids;
  float* w;
  int32_t* slot_ids;
  int32_t* pred;
  size_t act_bytes;   /* bytes per activation element (4 or 2) */
} moe_chain_buffers;

int moe_chain_create(moe_offload* const* layers, int32_t L, const void* const* w_router, const float* const* bias,
                     const void* const* shared_records, int32_t T, int32_t prefetch_n, moe_chain** out);

/* Device addresses of the chain's buffers. */
int moe_chain_get_buffers(const moe_chain* c, moe_chain_buffers* out);

/* One decode step: launch the captured graph on `stream` (captured on the
 * first call; later calls only launch).  Asynchronous.
 * Layers in cold or split mode (moe_offload_set_cold) join the step: the
 * graph publishes each call that has host-computed pairs (record index
 * S + E + e) into pinned host memory, a host thread of the chain computes
 * those pairs (the host FFN of moe_slot_ffn_host_cold), and the graph waits
 * for its rows before the layer's combine, with no host synchronisation.
 * Which layers take part is fixed when the graph is captured (cold mode, or
 * split mode with calls of more than S - P pairs); a run that finds another
 * set synchronises the device and captures again.  The host thread starts
 * with the first such run and polls until moe_chain_destroy (every 100 us
 * after 50 ms without work).  If the host does not answer within half a
 * second or so, the step goes on with stale rows and sets
 * MOE_DEV_ERR_HOST_TIMEOUT.
 * Errors: MOE_EINVAL (null chain; a layer in cold or split mode together
 * with the lookahead prefetch), MOE_ENOMEM, MOE_EHIP. */
int moe_chain_run(moe_chain* c, void* stream);

/* The same step issued call by call on `stream` (no graph), for profiling
 * and for checking the graph against eager execution (cold and split layers
 * as in moe_chain_run). */
int moe_chain_run_eager(moe_chain* c, void* stream);

/* Read-through of decode misses (default on).  The pages move a missed
 * expert into its slot and then run the expert GEMMs on the slot
 * (xinfer-ai 0.14.6 docs/moe_offload.md, "How it works", Decode).  On: a
 * chain whose T is 1, or 2 to 64 with T * top_k <= 256 (bf16, fp8 and
 * MXFP4 layers), launches no copy kernel; its gate/up and down launches read each
 * record of the ensure's copy list from the device-mapped host store and
 * store every byte they read into the record's slot (or, for the overflow of
 * a call wider than the cache, its staging record), so the resident experts
 * compute while the missed ones cross the host link.  Off: the copy kernel
 * moves the misses first.  Slots, tables, counters and outputs are the same
 * either way; only the launches differ.  Changing the setting synchronises
 * the device and drops the captured graph (the next moe_chain_run captures
 * again).  Other T and fp32 layers always use the copy kernel.  Errors:
 * MOE_EINVAL (null chain), MOE_EHIP. */
int moe_chain_set_read_through(moe_chain* c, int on);

/* Synchronise and free the chain's graph, streams, events and buffers.  Null-safe. */
void moe_chain_destroy(moe_chain* c);

#ifdef __cplusplus
}
#endif
#endif /* MOE_OFFLOAD_H */
