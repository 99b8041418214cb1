/*
 * h2o.h -- C ABI of the MI355X (gfx950) Heavy-Hitter Oracle (H2O) KV-cache library.
 *
 * Citations ("H2O §x") refer to the page "H2O: Heavy-Hitter Oracle for
 * Efficient Generative Inference of Large Language Models" (paperlayer.ai
 * source-linked summary of arXiv 2306.14048v3), section x.
 *
 * The problem (H2O §2 "Problem formulation", §D "Cache eviction"): every
 * (batch, head) pair keeps a cache of exactly k = k_heavy + k_recent slots;
 * between two consecutive decode steps at most one cached token is evicted,
 * chosen from normalised attention accumulated over the steps (H2O §1, §4.1,
 * §B.2: accumulated, not averaged). Prefill reduces the prompt to heavy
 * hitters plus recent tokens (H2O §A "Pseudocode", "System Details").
 *
 * Conventions shared by every call
 *  - Device memory is owned by the caller. The library never allocates or
 *    frees device memory; all device pointers must be 16-byte aligned and the
 *    tensors dense and contiguous in the layouts stated below (outermost
 *    dimension first).
 *  - "dtype" is the element type of the K/V cache and of every query, key and
 *    value handed in (h2o_dtype). Scores, outputs and column sums are fp32.
 *  - Every call that takes a stream enqueues its work asynchronously on that
 *    stream (a hipStream_t; NULL is the null stream) and returns without
 *    waiting, except h2o_cache_state when it copies to the host. Calls on one
 *    cache must be issued in order on one stream.
 *  - Argument errors are detected before anything is launched: the call
 *    returns a non-zero h2o_status, changes nothing, and h2o_last_error()
 *    returns a message. A HIP launch error returns H2O_EDEVICE. No C++
 *    exception crosses this interface.
 *  - All functions are thread-safe with respect to different caches.
 */
#ifndef H2O_MI355X_H
#define H2O_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* h2o_stream_t; /* a hipStream_t */

/* Status codes are small positive integers (0 = success). */
typedef enum {
  H2O_OK = 0,
  H2O_EINVAL = 1,     /* null pointer, bad size, unsupported dtype or head dim */
  H2O_ESTATE = 2,     /* cache not initialised, or call not allowed in its state */
  H2O_EWORKSPACE = 3, /* prefill workspace missing or too small */
  H2O_EDEVICE = 4     /* the HIP runtime reported an error */
} h2o_status;

typedef enum { H2O_F32 = 0, H2O_BF16 = 1, H2O_F16 = 2 } h2o_dtype;

/*
 * What a cached token is worth keeping (the largest values are kept at
 * prefill, the smallest eligible one is evicted at decode; ties go by
 * position, the later one being kept):
 *   ACCUMULATED - its accumulated attention score (H2O, §4.1);
 *   AVERAGED    - that score divided by the number of queries that attended
 *                 to it, t - pos + 1 (the variant H2O §B.2 reports as worse);
 *   POSITION    - minus its position: the first k_heavy tokens stay as
 *                 attention sinks and the newest token outside the recent
 *                 window leaves (StreamingLLM's sink-plus-window cache).
 */
typedef enum { H2O_POLICY_ACCUMULATED = 0, H2O_POLICY_AVERAGED = 1, H2O_POLICY_POSITION = 2 } h2o_policy;

/*
 * Storage of a cache's keys and values:
 *   NONE       - rows in the cache dtype, as handed in;
 *   U8, U4, U2 - b = 8, 4 or 2-bit codes (H2O combined with quantisation,
 *          H2O §5 "Ablation and Extended Evaluations"; keys per channel and
 *          values per token, down to 2 bits, after the KIVI abstract on the
 *          page "Discoveries (cursor 150)"). With L = 2^b - 1: keys use one
 *          affine grid per (batch, head, channel), fixed by the prompt: mn_c
 *          and mx_c are the prompt's smallest and largest key values in
 *          channel c and scale_c = (mx_c - mn_c) / L. Values use one grid per
 *          cached row over its own d values. A value x is stored as the code
 *          rint((x - mn) / scale) clamped to [0, L] (0 if scale = 0), all in
 *          fp32 with IEEE rounding and ties to even, and read as
 *          code * scale + mn. A row of head_dim codes takes head_dim * b / 8
 *          bytes; channel c sits in byte c * b / 8 at bit offset
 *          b * (c mod 8/b), low bits first. A decode token attends to its own
 *          key and value at full precision; it is quantised when written into
 *          its slot.
 */
typedef enum { H2O_QUANT_NONE = 0, H2O_QUANT_U8 = 1, H2O_QUANT_U4 = 2, H2O_QUANT_U2 = 3 } h2o_quant;

/* Size limits that the library checks (H2O_EINVAL beyond them). */
#define H2O_MAX_SLOTS 8192      /* k = k_heavy + k_recent */
#define H2O_MAX_PROMPT 1048576  /* n */

/*
 * Cache descriptor: a plain host struct filled by h2o_cache_init. It records
 * the shape and the caller-owned device tensors of one layer's cache:
 *   K, V  : [batch][heads][k][head_dim] dtype, slot-indexed rows
 *   score : [batch][heads][k] fp32, accumulated normalised attention per slot
 *   pos   : [batch][heads][k] int32, sequence position held by the slot, -1 = empty
 * and the host counter t_next (position of the next decode token). The number
 * of occupied slots is always n_used = min(k, t_next), the same for all heads;
 * slots [0, n_used) are the occupied ones.
 * Slot layout after prefill: heavy hitters in ascending position in slots
 * [0, k_heavy), the recent window in ascending position in [k_heavy, k) (H2O §A
 * "System Details"); a prompt no longer than k fills slots 0..n-1 in order. A
 * decode step writes the new token into the evicted slot, or into slot n_used
 * while the cache is not full. Fields are read-only for the caller.
 */
typedef struct {
  int32_t batch, heads, head_dim;
  int32_t k_heavy, k_recent;
  int32_t dtype;    /* h2o_dtype */
  int32_t policy;   /* h2o_policy */
  float scale;      /* softmax scale applied to q.k (1/sqrt(head_dim) usually) */
  void* K;
  void* V;
  float* score;
  int32_t* pos;
  int32_t n_used;   /* min(k, t_next) */
  int32_t t_next;
  int64_t steps;    /* decode steps taken since init */
  uint32_t magic;   /* set by h2o_cache_init */
  int32_t quant;    /* h2o_quant */
  float* k_qparam;  /* U8/U4/U2 only (NULL otherwise): [batch][heads][2][head_dim] fp32, key grid scale_c then mn_c */
  float* v_qparam;  /* U8/U4/U2 only (NULL otherwise): [batch][heads][k][2] fp32, value grid (scale, mn) of each slot */
} h2o_cache;

/* Host view of a cache's counters (see h2o_cache_state). */
typedef struct {
  int32_t n_used, t_next, k, k_heavy, k_recent;
  int32_t reserved;
  int64_t steps;
} h2o_state;

/*
 * Fill *cache and clear the device state: pos = -1, score = 0 for every slot
 * (K and V are left as they are), t_next = 0.
 * Requires batch, heads >= 1; head_dim in {64, 128}; k_heavy >= 0;
 * k_recent >= 0 with k = k_heavy + k_recent >= 1 and k <= H2O_MAX_SLOTS;
 * policy an h2o_policy; scale finite and > 0; non-null device pointers.
 * k_heavy = 0 is the recent-window ("Local") cache; k_recent = 0 keeps heavy
 * hitters only (H2O §5 ablations) and lets the new token compete for a slot.
 */
h2o_status h2o_cache_init(h2o_cache* cache, int32_t batch, int32_t heads, int32_t head_dim,
                          int32_t k_heavy, int32_t k_recent, int32_t policy, int32_t dtype,
                          float scale, void* K, void* V, float* score, int32_t* pos,
                          h2o_stream_t stream);

/*
 * As h2o_cache_init, for a cache stored as codes (quant = H2O_QUANT_U8,
 * H2O_QUANT_U4 or H2O_QUANT_U2, b = 8, 4 or 2 bits, see h2o_quant). dtype is
 * that of the queries, keys and values handed to prefill and decode; the
 * cache holds
 *   Kq, Vq   : [batch][heads][k][head_dim * b / 8] uint8 packed codes,
 *              slot-indexed rows
 *   k_qparam : [batch][heads][2][head_dim] fp32 (scales, then minima),
 *              written by prefill
 *   v_qparam : [batch][heads][k][2] fp32 (scale, minimum of each row)
 * with score and pos as for h2o_cache_init. Kq, Vq, k_qparam and v_qparam
 * must be 16-byte aligned. The prompt handed to prefill must have n >= 1
 * (it fixes the key grids). h2o_decode_step_split does not take such a cache.
 * Errors: H2O_EINVAL for an unknown quant value or a missing buffer, plus
 * those of h2o_cache_init.
 */
h2o_status h2o_cache_init_quant(h2o_cache* cache, int32_t batch, int32_t heads, int32_t head_dim,
                                int32_t k_heavy, int32_t k_recent, int32_t policy, int32_t dtype,
                                float scale, int32_t quant, uint8_t* Kq, uint8_t* Vq, float* k_qparam,
                                float* v_qparam, float* score, int32_t* pos, h2o_stream_t stream);

/*
 * Bytes of device workspace h2o_prefill_select, h2o_prefill_attention and
 * h2o_prefill_select_lse need for a prompt of n tokens (0 for an invalid
 * shape): each prompt row's log normaliser, then the column sums when the
 * caller does not ask for them. Sizing only: the pages describe no memory
 * layout, so no passage defines this call.
 */
size_t h2o_prefill_workspace_bytes(int32_t batch, int32_t heads, int32_t n);

/*
 * Prefill scoring and selection (H2O §A "Pseudocode"; attention as in H2O §D
 * "Recursive attention").
 *   Q, Kp, Vp : [batch][heads][n][head_dim] dtype, the prompt's queries, keys, values
 * For every (b,h): c_j = sum over prompt rows i >= j of softmax_j'(scale*q_i.k_j')[j]
 * (causal, own position included). If n <= k every position is kept in slots
 * 0..n-1; otherwise the recent window n-k_recent..n-1 is kept together with
 * the k_heavy positions in [0, n-k_recent) whose (value, j) are largest, the
 * value being the policy's (c_j; c_j / (n - j); or -j), so equal values keep
 * the later position. Kept slots get K/V rows copied from the prompt and
 * score = c_j; unused slots get pos = -1, score = 0.
 * Afterwards t_next = n.
 *   workspace  : device buffer of at least h2o_prefill_workspace_bytes(...) bytes
 *   colsum_out : optional [batch][heads][n] fp32 device buffer receiving c, or NULL
 * The cache must be freshly initialised (t_next == 0). n may be 0.
 */
h2o_status h2o_prefill_select(h2o_cache* cache, const void* Q, const void* Kp, const void* Vp,
                              int32_t n, void* workspace, size_t workspace_bytes,
                              float* colsum_out, h2o_stream_t stream);

/*
 * h2o_prefill_select that also returns the prompt's own causal attention
 * (H2O §D "Recursive attention": o_i = sum_{j<=i} softmax_j(scale*q_i.k_j) v_j
 * with its normaliser D_i), so that a model's prefill attention and the H2O
 * scoring share the first QK^T pass and H2O's extra cost is the column-sum
 * pass alone:
 *   out     : [batch][heads][n][head_dim] fp32, o_i (required when n > 0)
 *   lse_out : optional [batch][heads][n] fp32, log sum_{j<=i} exp(scale*q_i.k_j)
 *             (natural log), or NULL
 * Everything else as for h2o_prefill_select.
 */
h2o_status h2o_prefill_attention(h2o_cache* cache, const void* Q, const void* Kp, const void* Vp,
                                 int32_t n, void* workspace, size_t workspace_bytes, float* out,
                                 float* lse_out, float* colsum_out, h2o_stream_t stream);

/*
 * h2o_prefill_select for a caller whose own attention kernel already produced
 * each prompt row's log normaliser:
 *   lse : [batch][heads][n] fp32 device, log sum_{j<=i} exp(scale*q_i.k_j)
 *         (natural log, the cache's scale), e.g. the log-sum-exp a fused
 *         attention forward emits.
 * Only the column-sum pass forms QK^T; its terms are exp(scale*q_i.k_j - lse_i),
 * so the column sums are exact for the normalisers given.
 */
h2o_status h2o_prefill_select_lse(h2o_cache* cache, const void* Q, const void* Kp, const void* Vp,
                                  int32_t n, const float* lse, void* workspace, size_t workspace_bytes,
                                  float* colsum_out, h2o_stream_t stream);

/*
 * One decode step at position t = t_next for every (b,h) (H2O §D "Recursive
 * attention" then "Cache eviction"; H2O §2 "Problem formulation"):
 *   q, k_new, v_new : [batch][heads][head_dim] dtype, the new token
 *   out             : [batch][heads][head_dim] fp32, attention output
 *   evicted_pos     : [batch][heads] int32, the evicted position; -1 when
 *                     the cache was not full; -2 when it was full but no slot
 *                     was eligible, which a cache driven only through this
 *                     interface never is (a caller that rewrote pos
 *                     inconsistently): then no slot is written
 * 1. p = softmax over the occupied slots plus the new token itself of scale*q.k.
 * 2. out = sum p_a V_a + p_new v_new.
 * 3. score_a += p_a for every occupied slot.
 * 4. If the cache is full (n_used == k), the victim is the candidate with the
 *    smallest (value, pos) among slots with pos <= t - k_recent, the value
 *    being the policy's (see h2o_policy); with k_recent = 0 the new token is
 *    a candidate too. Exactly one token is evicted. Otherwise nothing is
 *    evicted and the slot is n_used.
 * 5. The freed slot receives k_new, v_new, pos = t, score = p_new, unless the
 *    new token itself was evicted (then evicted_pos = t and no slot changes
 *    except for the scores of step 3); t_next = t + 1.
 * A cache stored as codes must have been prefilled first (its key grids come
 * from the prompt): with t_next == 0 it returns H2O_ESTATE.
 * Inputs are not scanned for NaN or Inf. A NaN in a head's q or k_new makes
 * that head's scores and output NaN (one in v_new, its output); its eviction
 * is still an eligible slot (a NaN score orders above every number and equal
 * keys fall to the older position), and no other head is affected.
 */
h2o_status h2o_decode_step(h2o_cache* cache, const void* q, const void* k_new, const void* v_new,
                           float* out, int32_t* evicted_pos, h2o_stream_t stream);

/*
 * Bytes of device workspace h2o_decode_step_split needs for a cache of
 * batch x heads heads, head_dim and k = k_heavy + k_recent slots (0 for an
 * invalid shape). The workspace holds the step's logits [batch][heads][k] and
 * up to ceil(k/64) chunk partials per head; it carries nothing from one call
 * to the next. Sizing only: no passage on the pages defines this call.
 */
size_t h2o_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t k);

/*
 * The decode step of h2o_decode_step, same arguments, same results (up to the
 * fp32 summation order of the softmax), with every head's occupied slots cut
 * into chunks of chunk_rows rows, each streamed by its own wave, so that few
 * (batch, head) pairs with long caches still fill the GPU. A second kernel
 * merges the chunks' partial softmax sums per head (H2O §D "Recursive
 * attention"), updates the scores and evicts (H2O §2 "Problem formulation",
 * §D "Cache eviction").
 *   chunk_rows : 0 lets the library choose (about two waves per SIMD in
 *                total); otherwise a positive multiple of 64 (a value above
 *                k rounded up to 64 is taken as that: one chunk per head)
 *   workspace  : device buffer of at least h2o_decode_workspace_bytes(...)
 *                bytes, 256-byte aligned, used only while the call's work
 *                runs on the stream (calls sharing one workspace must be
 *                issued in order on one stream).
 * For many heads with short caches h2o_decode_step is the faster call.
 */
h2o_status h2o_decode_step_split(h2o_cache* cache, const void* q, const void* k_new, const void* v_new,
                                 float* out, int32_t* evicted_pos, int32_t chunk_rows, void* workspace,
                                 size_t workspace_bytes, h2o_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * h2o_decode_step_split with the same arguments and results, whose workspace
 * is instead an array of H2O_SPLIT_SCRATCH_BYTES bytes inside the library,
 * one per GPU, held until the process ends. Its address is looked up once per
 * device, by h2o_cache_init (or by this call's first use on a device no cache
 * was initialised on). A shape whose workspace, h2o_decode_workspace_bytes,
 * exceeds H2O_SPLIT_SCRATCH_BYTES returns H2O_EWORKSPACE before anything is
 * launched. The call allocates nothing. Every call on one GPU shares that
 * GPU's array, so calls whose work can overlap on one GPU (unordered streams,
 * several threads) race: issue them in order on one stream. Nothing in the
 * array needs to start at zero (each call writes every entry it reads).
 */
#define H2O_SPLIT_SCRATCH_BYTES (16u << 20)
h2o_status h2o_decode_step_split_noalloc(h2o_cache* cache, const void* q, const void* k_new, const void* v_new,
                                         float* out, int32_t* evicted_pos, int32_t chunk_rows,
                                         h2o_stream_t stream);

/*
 * Export the cache state (checkpoint, inspection): the fixed-size set of
 * cached positions and their accumulated scores, S_i and the scores that
 * drive the next eviction in H2O §2 "Problem formulation" and §D "Cache
 * eviction". The pages define no checkpoint call; this one is bookkeeping
 * around that state. Fills *state from the host counters. If pos_host and/or
 * score_host are non-null ([batch][heads][k] host arrays), the device arrays
 * are copied into them and the call waits for the stream; otherwise it does
 * not touch the device.
 */
h2o_status h2o_cache_state(const h2o_cache* cache, h2o_state* state, int32_t* pos_host,
                           float* score_host, h2o_stream_t stream);

/*
 * Restore the host counter after the caller has written K, V, score and pos
 * (and, for a cache of codes, both grids) back into the device tensors:
 * resume from a checkpoint, or resynchronise from another implementation.
 * Sets t_next and n_used = min(k, t_next). The counterpart of
 * h2o_cache_state; no passage on the pages defines it.
 */
h2o_status h2o_cache_restore(h2o_cache* cache, int32_t t_next, int64_t steps);

/*
 * Plain decode attention over a contiguous full cache, without scores or
 * eviction (the no-eviction comparator of the same step):
 *   q : [batch][heads][head_dim], Kc, Vc : [batch][heads][len][head_dim] dtype
 *   out : [batch][heads][head_dim] fp32, out = softmax(scale*q.Kc) Vc over len rows.
 */
h2o_status h2o_fullcache_decode(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype,
                                float scale, int32_t len, const void* q, const void* Kc,
                                const void* Vc, float* out, h2o_stream_t stream);

/*
 * Message for the last non-OK status returned on the calling thread (error
 * reporting; no passage on the pages defines it).
 */
const char* h2o_last_error(void);

/*
 * 16 hex digits identifying the sources the library was built from (a
 * SHA-256 prefix over its kernel sources and this header), so that a caller
 * can refuse a binary older than its sources. Build identification; no
 * passage on the pages defines it.
 */
const char* h2o_build_digest(void);

#ifdef __cplusplus
}
#endif
#endif /* H2O_MI355X_H */
