/*
 * ckv.h -- C ABI of the certified quantized-KV decode attention library
 * (HIP, gfx950 / MI355X).
 *
 * The method is the one described on the page "Runtime-Certified
 * Bounded-Error Quantized Attention" (gist.science paper 2605.20868,
 * technical summary).  Section tags used below:
 *   [Meth-1]  Methodology 1, tiered storage with deterministic fallback
 *   [Meth-2]  Methodology 2, two-term error decomposition
 *   [Meth-3]  Methodology 3, adaptive precision and the fallback ladder
 *   [Contrib] Key contributions
 *   [Results] Experimental results
 *
 * Conventions for every entry point:
 *   - Pointers are plain host or device addresses as stated per argument;
 *     the library never takes ownership of caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *   - Errors are returned as ckv_status; nothing is thrown across the ABI.
 *     On error a message is available from ckv_last_error() (per thread).
 *     CKV_EHIP means a HIP runtime call failed; the HIP error text is in
 *     the message.
 *   - One cache must not be used from two host threads or two streams at
 *     the same time.
 *   - FP16 data is IEEE binary16, passed as 16-bit patterns.
 */
#ifndef CKV_H
#define CKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CKV_OK = 0,
    CKV_EINVAL = 1, /* bad argument (shape, pointer, layer/sequence index)   */
    CKV_ENOMEM = 2, /* device or pinned host allocation failed               */
    CKV_EHIP = 3,   /* a HIP runtime call failed                             */
    CKV_ERANGE = 4, /* appending would exceed max_context                    */
    CKV_ESTATE = 5  /* call not valid in the current state (e.g. empty seq)  */
} ckv_status;

typedef struct ckv_cache ckv_cache;

/* Shape of a cache.  head_dim must be 64 or 128; n_q_heads a multiple of
 * n_kv_heads with n_q_heads / n_kv_heads <= 8; max_context >= 1.  Blocks
 * are 64 tokens; INT4 value groups are 32 channels. */
typedef struct {
    int n_layers;
    int max_batch;    /* sequences per layer                               */
    int n_q_heads;
    int n_kv_heads;
    int head_dim;
    int max_context;  /* tokens per sequence                               */
    int device;       /* HIP device ordinal                                */
    int v_bits;       /* value code width: 4 (the design's asymmetric cache:
                         INT8 keys, INT4 values; 0 also means 4) or 8 (the
                         symmetric cache configuration of [Results]: values
                         at the keys' width, the same per-token 32-channel
                         groups with 255 levels, one code per byte)       */
} ckv_config;

/* Thresholds of the certified decode step [Meth-3, Results].
 * tau_cov: coverage of the estimated attention mass by the blocks whose
 *   FP16 keys are paged in (the page's example: 0.995), in [0, 1].  0 pages
 *   no FP16 keys: with k_tol and v_tol infinite the step is plain quantized
 *   attention (INT8 keys, INT4 values) and E_key, E_val bound its error.
 * k_tol / v_tol: tolerances on E_key / E_val, in output units.
 * rank_tol: the rank check fails when more than floor(rank_tol * K*(K*-1)/2)
 *   pairs of promoted blocks are ordered differently by INT8 and FP16 keys.
 * sm_scale: softmax scale applied to q.k.
 * f_layer: a layer (per sequence) falls back whole when more than
 *   f_layer * n_q_heads heads fell back on their own.
 * n_widen: maximum number of rung-1 widenings (each halves 1 - tau).
 * v_cap_blocks: maximum FP16-value blocks per head (<= 0: no cap). */
typedef struct {
    float tau_cov, k_tol, v_tol, rank_tol, sm_scale, f_layer;
    int n_widen, v_cap_blocks;
} ckv_thresholds;

/* Per (sequence, q head) outcome of a decode step [Meth-2, Meth-3].
 * e_key, e_val, tv_bound: certified bounds (0 for heads that fell back,
 *   whose output is exact dense attention).
 * tau_final: coverage after rung-1 widening.
 * kstar: blocks with FP16 keys; n_v_promoted: blocks with FP16 values.
 * rank_ok: 1 consistent, 0 inconsistent, -1 not run (layer fell back
 *   before paging).  n_discordant: discordant pair count.
 * rung_max: highest rung reached (0..4); rung_mask: bit r set for every
 *   rung r reached. */
typedef struct {
    float e_key, e_val, tv_bound, tau_final;
    int kstar, n_v_promoted, rank_ok, rung_max, rung_mask, n_discordant;
} ckv_head_report;

/* Create a cache: tier 1 (codes, metadata, annotations) in device memory,
 * tier 2 (FP16 originals) in pinned host memory [Meth-1], plus staging and
 * scratch.  *out receives the handle.  Errors: EINVAL, ENOMEM, EHIP. */
ckv_status ckv_create(const ckv_config *cfg, ckv_cache **out);

/* Free everything the cache owns.  NULL is accepted. */
void ckv_destroy(ckv_cache *c);

/* Forget every token of sequence `seq` in all layers.  Errors: EINVAL. */
ckv_status ckv_reset_sequence(ckv_cache *c, int seq);

/* Append n_tokens tokens to (layer, seq) [Meth-1].
 * k_fp16, v_fp16: [n_tokens][n_kv_heads][head_dim] binary16, in device
 *   memory if src_on_device, else in host memory; read before return.
 * Every completed 64-token block is quantized (INT8 keys with a per-channel
 * scale/offset per block, INT4 values (INT8 when v_bits = 8) with a
 * scale/offset per token and 32-channel group, the block's value-error
 * annotation); tokens of an
 * unfinished block stay FP16 on the device.  Completed blocks are copied to
 * the FP16 tier in host memory (an unfinished block is read from its device
 * copy until it completes).  The call synchronizes `stream`.
 * Errors: EINVAL, ERANGE (would exceed max_context), EHIP. */
ckv_status ckv_append_kv(ckv_cache *c, int layer, int seq, const void *k_fp16,
                         const void *v_fp16, int n_tokens, int src_on_device, void *stream);

/* Append one decode token to each of sequences 0..batch-1 of `layer`
 * [Meth-1]: the same result as ckv_append_kv with n_tokens = 1 for each
 * sequence in turn, in one pass over the batch (the decode step's append).
 * k_fp16, v_fp16: [batch][n_kv_heads][head_dim] binary16, in device memory
 * if src_on_device, else in host memory; read before return.  A block that
 * the token completes is quantized and written to the FP16 tier.  The call
 * synchronizes `stream`.  Errors: EINVAL, ERANGE (a sequence would exceed
 * max_context; nothing is appended), EHIP. */
ckv_status ckv_append_token(ckv_cache *c, int layer, int batch, const void *k_fp16,
                            const void *v_fp16, int src_on_device, void *stream);

/* Certified decode attention for sequences 0..batch-1 of `layer`
 * [Meth-2, Meth-3, Contrib].
 * q_fp16: device, [batch][n_q_heads][head_dim] binary16.
 * th: host pointer to the thresholds.
 * out: device, [batch][n_q_heads][head_dim] FP32 attention output.
 * report: host, [batch][n_q_heads].
 * Steps: INT8 scoring pass over tier 1; top-K* selection covering tau_cov
 * of the estimated mass; E_key / E_val from quantities tracked on the
 * device only; rungs 1-2; FP16 keys (and values of rung 2) paged from
 * tier 2 with hipMemcpyAsync on a side stream while the tail is processed;
 * rank-consistency check; rungs 3-4 page full FP16 KV and recompute dense.
 * The call returns after the report is on the host (the ladder needs host
 * round trips).  Every sequence must hold >= 1 token.
 * Errors: EINVAL, ESTATE (empty sequence), EHIP.  On error `out` is
 * unspecified and every report has rung_max = -1. */
ckv_status ckv_certified_decode_attention(ckv_cache *c, int layer, const void *q_fp16, int batch,
                                          const ckv_thresholds *th, float *out,
                                          ckv_head_report *report, void *stream);

/* Exact dense decode attention over caller-provided device FP16 K/V, the
 * fast dense baseline the certified step is measured against [Results].
 * k, v: device binary16 in the block layout
 *   [batch][n_kv_heads][n_tokens/64][64 * head_dim], where a K block is
 *   [head_dim/8][64 tokens][8 channels] and a V block [head_dim][64 tokens];
 * n_tokens: a multiple of 64, at most the cache's max_context;
 * q: device [batch][n_q_heads][head_dim] binary16; out: device FP32
 * [batch][n_q_heads][head_dim].  Uses the cache's shape (heads, head_dim)
 * and scratch; stream-ordered, returns without synchronizing.
 * Errors: EINVAL, EHIP. */
ckv_status ckv_dense_decode_attention(ckv_cache *c, const void *k, const void *v, int n_tokens,
                                      const void *q_fp16, int batch, float sm_scale, float *out,
                                      void *stream);

/* The same exact dense decode attention as ckv_dense_decode_attention,
 * without a cache and without allocating anything: for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc).  No hipMalloc, hipFree or other
 * allocating call is made.
 * k, v, n_tokens, q_fp16, batch, sm_scale, out: as for
 *   ckv_dense_decode_attention (device pointers, the same block layout).
 * n_q_heads, n_kv_heads, head_dim: the head shape (head_dim 64 or 128,
 *   n_q_heads / n_kv_heads in {1, 2, 4, 8}).
 * Runs on the calling thread's current device; `stream` must belong to it.
 * The split partials live in a static 4 MiB device array per GPU, held
 * until the process ends: batch * n_q_heads * (head_dim + 2) * 4 bytes must
 * not exceed it (batch * n_q_heads <= 7710 at head_dim 128), otherwise
 * CKV_EINVAL; longer contexts use longer splits.  Every call on one GPU
 * shares that array, and each call writes every partial it reads, so no
 * state carries over; calls that overlap on one GPU (other streams or
 * threads) race.  Stream-ordered, returns without synchronizing.
 * Errors: EINVAL, EHIP. */
ckv_status ckv_dense_decode_attention_noalloc(const void *k, const void *v, int n_tokens,
                                              const void *q_fp16, int batch, int n_q_heads,
                                              int n_kv_heads, int head_dim, float sm_scale,
                                              float *out, void *stream);

/* Bytes held: tier 1 + partial blocks + staging + scratch on the device,
 * tier 2 in pinned host memory. */
ckv_status ckv_footprint(const ckv_cache *c, size_t *dev_bytes, size_t *host_bytes,
                         size_t *tier1_bytes);

/* Tokens currently held by (layer, seq). */
ckv_status ckv_seq_length(const ckv_cache *c, int layer, int seq, int *n_tokens);

/* Message of the last failed call on this thread ("" if none). */
const char *ckv_last_error(void);

/* ---- introspection (tests and benchmarks) ------------------------------ */

/* Tier-1 contents of one block, in token-major layout:
 * k_code [64][d] u8, k_s, k_z [d] binary16, v_code [64][d/2] u8 (low nibble
 * = even channel; [64][d] when v_bits = 8), v_s, v_z [64][d/32] binary16,
 * eta [1] FP32.  Host
 * pointers; any may be NULL.  Errors: EINVAL (block not complete), EHIP. */
ckv_status ckv_export_block(ckv_cache *c, int layer, int seq, int kv_head, int block,
                            uint8_t *k_code, uint16_t *k_s, uint16_t *k_z, uint8_t *v_code,
                            uint16_t *v_s, uint16_t *v_z, float *eta);

/* Intermediates of the last decode step (host pointers, may be NULL), for
 * batch rows 0..batch-1, with Np = N + (partial block ? 1 : 0) slots per
 * head where N = full blocks of the longest sequence in the batch:
 *   score  [batch][n_q_heads][Np*64] FP32  INT8 scores (partial: FP16)
 *   bstat  [batch][n_q_heads][Np][4] FP32  block max, l, Delta, rho
 *   mref   [batch][n_q_heads] FP32         largest estimated score
 *   mfx    [batch][n_q_heads][Np] u64      fixed-point estimated masses
 *   sel    [batch][n_kv_heads][Np] u32     bit j: P of head j of the
 *                                          group, bit 8+j: VP of head j
 *                                          (first N entries of each row)
 *   m16fx  [batch][n_q_heads][Np] u64      fixed-point FP16 masses on P
 *                                          (not written for a sequence at
 *                                          rung 4 before paging)
 *                                          (first N entries of each row)
 *   bounds [batch][n_q_heads][4] FP64      mu, TV, E_key, E_val
 *   seq_flags [batch] int                  bit0 rung 4 before paging,
 *                                          bit1 rung 4 after the rank check
 * Entries past a shorter sequence's own tokens (score) or slots (the
 * per-block arrays) are not defined.
 * np_out receives Np.  Errors: ESTATE (no step yet), EINVAL, EHIP. */
ckv_status ckv_export_step(ckv_cache *c, int batch, int *np_out, float *score, float *bstat,
                           float *mref, uint64_t *mfx, uint32_t *sel, uint64_t *m16fx,
                           double *bounds, int *seq_flags);

/* Device-resident FP16 block cache across steps (a "next" step beyond the
 * page's design, which names host-to-device paging traffic as the main
 * overhead): FP16 K and V blocks paged in for layer l stay in HBM for the
 * following steps of layer l, so a block is copied from tier 2 at most once
 * while it stays complete (blocks are immutable; ckv_reset_sequence drops a
 * sequence's blocks).  Layers 0 .. m-1 get a persistent mirror of their
 * staging area, m = min(n_layers, max_bytes / (2 * max_batch * n_kv_heads *
 * ceil(max_context/64) * 64 * head_dim * 2 bytes)); the other layers page
 * every step as before.  *layers receives m.  Results are identical with and
 * without the cache.  Errors: EINVAL (null cache), ESTATE (already enabled),
 * ENOMEM (device memory: the layers mirrored so far stay enabled). */
ckv_status ckv_enable_fp16_cache(ckv_cache *c, size_t max_bytes, int *layers);

/* Paging by the device instead of host-issued copies (a measured
 * alternative to the design's hipMemcpyAsync paging): a kernel reads the
 * listed FP16 blocks straight from tier 2 (pinned host memory mapped into
 * the device's address space) into the staging area: only the needed
 * blocks cross the host link (no gap fill) and there is no per-copy cost.
 * Results are identical.  Layers with the FP16 cache enabled, sequences
 * skipped by rung 4 before paging and the dense fallback keep using the
 * copies.  enable: 0 host copies (default), 1 device paging.
 * Errors: EINVAL (null cache). */
ckv_status ckv_set_device_paging(ckv_cache *c, int enable);

/* Staged paging (an implementation choice for the host-issued paging of
 * [Meth-1]; the page issues one copy per block), on by default: host
 * threads pack the listed FP16 blocks of a step, and only those, into 4 MiB
 * chunks of a ring in pinned host memory (16 chunks); each chunk crosses the
 * host link in one hipMemcpyAsync on a paging stream, straight into packed
 * staging areas in listing order (for a layer with the persistent FP16 cache:
 * into a device ring slot, and a kernel moves its blocks to their
 * block-indexed staging slots).  Runs of consecutive listed blocks of at
 * least a chunk's bytes are copied directly, one copy each.  Switched off,
 * the blocks are copied as runs of consecutive blocks, small gaps filled, one
 * copy per run.  The results
 * are identical either way.  threads: 0 switches it off, 1 .. 64 the packing
 * threads (held by the cache until it is destroyed or this is called again;
 * ckv_create starts min(8, half the host's CPUs), at least 1).  The first switch
 * on (in ckv_create) allocates the ring, about 64 MiB of pinned host and of
 * device memory, kept until ckv_destroy, and reads every page of tier 2 once
 * so that the packing takes no page faults.  Waits for the device to finish.
 * CKV_EINVAL for threads outside 0 .. 64, CKV_ENOMEM when the ring or the
 * threads cannot be had.  Device paging, when on, takes precedence. */
ckv_status ckv_set_staged_paging(ckv_cache *c, int threads);

/* Profile of the decode steps since profiling was enabled (enabling resets
 * it).  Phases: 0 scoring pass (K1), 1 selection (K2), 2 tail pass (K3),
 * 3 page-in (the host-to-device copies on the paging streams), 4 promoted
 * value pass over INT4 values (K4a), 5 fallback (the time it adds: from the
 * end of the step's own paging on the first paging stream to the end of the
 * dense recompute; its blocks are paged right behind the step's own, as soon
 * as the rank check's verdicts reach the host),
 * 6 the whole step on the host wall clock, 7 rank check + merge (K4b, two
 * launches), 8 FP16-key scoring of the promoted blocks (K4a keys),
 * 9 promoted value pass over FP16 values (K4a; with packed staged paging
 * two launches, the pairs whose FP16 values land before the last chunk and
 * then the rest, their spans added).  The kernel phases (0, 1,
 * 2, 4, 7, 8, 9) are each kernel's own execution span, its first wave's
 * start to its last wave's end on the device's constant-rate wall clock,
 * stamped by the kernel (a few atomics per workgroup); phases 3 and 5 are
 * timed with HIP events on the streams they run on.  Block counts are what
 * the passes read, summed over steps: a block is one (sequence, kv head,
 * 64 tokens).  Profiling adds per step a kernel that folds the clock slots
 * into one start and one end per timed launch (and re-arms them), a 160-byte
 * copy back, and a few events.  Enabling it arms the slots and waits for
 * that copy; CKV_EHIP if it fails. */
typedef struct {
    double ms[10];          /* accumulated milliseconds per phase            */
    int counts[10];         /* timed occurrences per phase                   */
    int steps;              /* decode steps profiled                         */
    uint64_t bytes_paged;   /* tier 2 -> staging bytes (staged paging: with
                               the chunk headers; run copies: with filled
                               gaps)                                         */
    uint64_t copies;        /* host-to-device copies issued (staged paging:
                               chunks and direct runs)                       */
    uint64_t q8_blocks;     /* blocks read by the scoring pass               */
    uint64_t tail_blocks;   /* blocks read by the tail pass (INT4 values)    */
    uint64_t k16_blocks;    /* FP16 key blocks read by the promoted pass     */
    uint64_t v16_blocks;    /* FP16 value blocks read by the promoted pass   */
    uint64_t int4p_blocks;  /* INT4 value blocks read by the promoted pass   */
    uint64_t dense_blocks;  /* FP16 K+V blocks read by the dense fallback    */
    double gather_lead_ms;  /* device paging only: summed over its steps, the
                               K gather's first wave start minus the
                               selection kernel's last wave end (device
                               clock; the host's round trip is not in it)  */
    int gather_steps;       /* steps that paged by the device                */
    int staged_threads;     /* the cache's packing threads now (0: staged
                               paging off)                                   */
} ckv_profile;

ckv_status ckv_set_profiling(ckv_cache *c, int enable);
ckv_status ckv_get_profile(const ckv_cache *c, ckv_profile *p);

/* Measurement aid (not part of the decode step): a streaming read of
 * `bytes` of device memory at dev_buf, enqueued on `stream` (a hipStream_t;
 * NULL: the null stream).  Wave w reads wave_kib KiB (4, 8 or 16) at byte
 * offset w * wave_kib KiB as 16-byte loads per lane, all requested before any
 * is used: the load shape of the scoring pass (8 KiB of key codes per wave)
 * and of the FP16-key pass (16 KiB per block).  Timing it over a buffer much
 * larger than the device's last-level cache gives the read rate these passes
 * are measured against.  dev_sink: one device word, written only if the fold
 * of the loaded words takes one particular value (it keeps the loads).  The
 * caller owns both buffers; bytes must be a positive multiple of wave_kib KiB.
 * Errors: EINVAL (null pointer, wave_kib, bytes), EHIP (launch failure). */
ckv_status ckv_read_probe(const void *dev_buf, size_t bytes, int wave_kib, unsigned *dev_sink, void *stream);

/* Fault injection for tests of the error path of a decode step: the host-to-
 * device paging copy issued after `after_copies` further copies (0: the
 * next one) is not issued and reports failure, as a failed hipMemcpyAsync
 * would; the injection then clears itself.  < 0 clears it.  The step that
 * meets it returns CKV_EHIP with every report at rung_max = -1 and forgets
 * which blocks of the layer are staged, so the next step pages them again
 * and is computed as if the failed step had not happened.  Device paging
 * (ckv_set_device_paging) issues no copies for the listed blocks.
 * Errors: EINVAL (null cache). */
ckv_status ckv_inject_paging_fault(ckv_cache *c, int after_copies);

#ifdef __cplusplus
}
#endif
#endif
