// C ABI of the H2O KV-cache library: validation, host-side counters, launches.
// The entry points and their contracts are declared in include/h2o.h.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/h2o.h"
#include "launch.h"
#include "prefill_launch.h"

namespace {

constexpr uint32_t kMagic = 0x48324F31u;  // "H2O1"
thread_local char g_err[512] = "";

h2o_status fail(h2o_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

h2o_status device_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return H2O_OK;
  return fail(H2O_EDEVICE, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Bits per code of a quantised cache.
int code_bits(int32_t quant) { return quant == H2O_QUANT_U8 ? 8 : quant == H2O_QUANT_U4 ? 4 : 2; }

h2o_status check_cache(const h2o_cache* c) {
  if (!c) return fail(H2O_EINVAL, "cache is NULL");
  if (c->magic != kMagic) return fail(H2O_ESTATE, "cache descriptor was not initialised by h2o_cache_init");
  return H2O_OK;
}

size_t lse_ld(int32_t n) { return (size_t(n) + 63) & ~size_t(63); }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Split decode: chunks are whole multiples of 64 rows, so a head has at most
// ceil(k / 64) of them.
constexpr int kSplitRows = 64;
size_t split_cmax(int32_t k) { return (size_t(k) + kSplitRows - 1) / kSplitRows; }
static_assert((H2O_MAX_SLOTS + kSplitRows - 1) / kSplitRows <= h2o::kMaxChunks, "split chunk capacity");

h2o_status init_cache(h2o_cache* cache, int32_t batch, int32_t heads, int32_t head_dim, int32_t k_heavy,
                      int32_t k_recent, int32_t policy, int32_t dtype, float scale, void* K, void* V, float* score,
                      int32_t* pos, int32_t quant, float* k_qparam, float* v_qparam, h2o_stream_t stream) {
  if (!cache) return fail(H2O_EINVAL, "cache is NULL");
  if (batch < 1 || heads < 1) return fail(H2O_EINVAL, "batch and heads must be >= 1");
  if (int64_t(batch) * heads > (int64_t(1) << 31) - 1) return fail(H2O_EINVAL, "batch*heads too large");
  if (head_dim != 64 && head_dim != 128) return fail(H2O_EINVAL, "head_dim %d not supported (64, 128)", head_dim);
  if (dtype != H2O_F32 && dtype != H2O_BF16 && dtype != H2O_F16) return fail(H2O_EINVAL, "unknown dtype %d", dtype);
  if (k_heavy < 0) return fail(H2O_EINVAL, "k_heavy must be >= 0");
  if (k_recent < 0) return fail(H2O_EINVAL, "k_recent must be >= 0");
  if (int64_t(k_heavy) + k_recent < 1) return fail(H2O_EINVAL, "k = k_heavy + k_recent must be >= 1");
  if (policy != H2O_POLICY_ACCUMULATED && policy != H2O_POLICY_AVERAGED && policy != H2O_POLICY_POSITION)
    return fail(H2O_EINVAL, "unknown policy %d", policy);
  if (int64_t(k_heavy) + k_recent > H2O_MAX_SLOTS)
    return fail(H2O_EINVAL, "k = %lld exceeds %d slots", (long long)k_heavy + k_recent, H2O_MAX_SLOTS);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(H2O_EINVAL, "scale must be finite and > 0");
  if (!K || !V || !score || !pos) return fail(H2O_EINVAL, "K, V, score and pos must be non-NULL");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(score, 4) || !aligned(pos, 4))
    return fail(H2O_EINVAL, "K and V must be 16-byte aligned, score and pos 4-byte aligned");

  h2o_cache c{};
  c.batch = batch;
  c.heads = heads;
  c.head_dim = head_dim;
  c.k_heavy = k_heavy;
  c.k_recent = k_recent;
  c.dtype = dtype;
  c.policy = policy;
  c.scale = scale;
  c.K = K;
  c.V = V;
  c.score = score;
  c.pos = pos;
  c.n_used = 0;
  c.t_next = 0;
  c.steps = 0;
  c.magic = kMagic;
  c.quant = quant;
  c.k_qparam = k_qparam;
  c.v_qparam = v_qparam;
  const int64_t count = int64_t(batch) * heads * (k_heavy + k_recent);
  h2o_status st = device_status(
      h2o::launch_cache_clear(score, pos, count, static_cast<hipStream_t>(stream)), "h2o_cache_init");
  if (st != H2O_OK) return st;
  // Set-up of h2o_decode_step_split_noalloc on this device: the address of
  // the library's own workspace, so that the step itself makes no runtime
  // call that could allocate.
  void* scratch = nullptr;
  st = device_status(h2o::split_scratch(&scratch), "h2o_cache_init");
  if (st != H2O_OK) return st;
  *cache = c;
  return H2O_OK;
}

h2o_status prefill(h2o_cache* cache, const void* Q, const void* Kp, const void* Vp, int32_t n, void* workspace,
                   size_t workspace_bytes, float* colsum_out, int32_t pass1, float* out, float* lse_out,
                   const float* lse_in, h2o_stream_t stream, const char* who) {
  h2o_status st = check_cache(cache);
  if (st != H2O_OK) return st;
  if (cache->t_next != 0) return fail(H2O_ESTATE, "prefill needs a freshly initialised cache (t_next = %d)", cache->t_next);
  if (n < 0 || n > H2O_MAX_PROMPT) return fail(H2O_EINVAL, "prompt length %d out of range [0, %d]", n, H2O_MAX_PROMPT);
  if (n == 0 && cache->quant != H2O_QUANT_NONE)
    return fail(H2O_EINVAL, "a cache stored as codes needs a prompt of at least one token (it fixes the key grids)");
  if (n == 0) return H2O_OK;  // nothing to score; the cleared cache is the result
  if (!Q || !Kp || !Vp) return fail(H2O_EINVAL, "Q, K and V must be non-NULL");
  if (!aligned(Q, 16) || !aligned(Kp, 16) || !aligned(Vp, 16))
    return fail(H2O_EINVAL, "Q, K and V must be 16-byte aligned");
  const size_t need = h2o_prefill_workspace_bytes(cache->batch, cache->heads, n);
  if (!workspace || workspace_bytes < need)
    return fail(H2O_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (!aligned(workspace, 256)) return fail(H2O_EWORKSPACE, "workspace must be 256-byte aligned");
  if (colsum_out && !aligned(colsum_out, 4)) return fail(H2O_EINVAL, "colsum_out must be 4-byte aligned");

  const int G = cache->batch * cache->heads;
  h2o::PrefillArgs a{};
  a.Q = Q;
  a.K = Kp;
  a.V = Vp;
  a.lse2 = static_cast<float*>(workspace);
  a.colsum = colsum_out ? colsum_out
                        : reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                   align256(size_t(G) * lse_ld(n) * sizeof(float)));
  a.cK = cache->K;
  a.cV = cache->V;
  a.cscore = cache->score;
  a.cpos = cache->pos;
  a.n = n;
  a.k_heavy = cache->k_heavy;
  a.k_recent = cache->k_recent;
  a.policy = cache->policy;
  a.c = cache->scale * h2o::kLog2e;
  a.quant = cache->quant;
  a.kq_param = cache->k_qparam;
  a.vq_param = cache->v_qparam;
  a.pass1 = pass1;
  a.out = out;
  a.lse_out = lse_out;
  a.lse_in = lse_in;
  st = device_status(h2o::launch_prefill(cache->dtype, cache->head_dim, G, a, static_cast<hipStream_t>(stream)),
                     who);
  if (st != H2O_OK) return st;
  const int32_t k = cache->k_heavy + cache->k_recent;
  cache->t_next = n;
  cache->n_used = n < k ? n : k;
  return H2O_OK;
}

// The split decode step with its workspace already chosen (the caller's, or
// the library's own array for h2o_decode_step_split_noalloc).
h2o_status split_step(h2o_cache* cache, const void* q, const void* k_new, const void* v_new, float* out,
                      int32_t* evicted_pos, int32_t chunk_rows, void* workspace, size_t workspace_bytes,
                      h2o_stream_t stream, const char* who) {
  h2o_status st = check_cache(cache);
  if (st != H2O_OK) return st;
  if (!q || !k_new || !v_new || !out || !evicted_pos)
    return fail(H2O_EINVAL, "q, k_new, v_new, out and evicted_pos must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16) || !aligned(evicted_pos, 4))
    return fail(H2O_EINVAL, "q, k_new, v_new, out must be 16-byte aligned; evicted_pos 4-byte aligned");
  if (cache->quant != H2O_QUANT_NONE) return fail(H2O_EINVAL, "split decode takes caches stored in their dtype only");
  if (chunk_rows < 0 || chunk_rows % kSplitRows != 0)
    return fail(H2O_EINVAL, "chunk_rows must be 0 or a positive multiple of %d", kSplitRows);
  const int32_t k = cache->k_heavy + cache->k_recent;
  const size_t need = h2o_decode_workspace_bytes(cache->batch, cache->heads, cache->head_dim, k);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(H2O_EWORKSPACE, "split decode needs a 256-byte aligned workspace of %zu bytes", need);
  if (cache->t_next == INT32_MAX) return fail(H2O_ESTATE, "position counter exhausted");

  const int G = cache->batch * cache->heads;
  const int nu = cache->n_used;
  int L = chunk_rows;
  if (L == 0) {
    // About two waves per SIMD in total, at least one 64-row chunk each.
    const int64_t target = int64_t(h2o::cu_count()) * 4 * 2;
    const int64_t per = (int64_t(G) * nu + target - 1) / target;
    L = int(((per + kSplitRows - 1) / kSplitRows) * kSplitRows);
    if (L < kSplitRows) L = kSplitRows;
  }
  // A chunk longer than the cache is one chunk per head (and keeps the
  // chunk kernel's LDS, 4 bytes per row, within 32 KiB).
  const int Lmax = int(split_cmax(k)) * kSplitRows;
  if (L > Lmax) L = Lmax;
  const int chunks = nu > 0 ? (nu + L - 1) / L : 1;
  if (size_t(chunks) > split_cmax(k)) return fail(H2O_EINVAL, "chunk_rows %d too small for k = %d", L, k);

  h2o::DecodeArgs a{};
  a.K = cache->K;
  a.V = cache->V;
  a.K_w = cache->K;
  a.V_w = cache->V;
  a.score = cache->score;
  a.pos = cache->pos;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  a.evicted = evicted_pos;
  a.k = k;
  a.n_used = nu;
  a.t = cache->t_next;
  a.k_recent = cache->k_recent;
  a.policy = cache->policy;
  a.c = cache->scale * h2o::kLog2e;
  char* ws = static_cast<char*>(workspace);
  const size_t cmax = split_cmax(k);
  h2o::SplitArgs w{};
  w.logit = reinterpret_cast<float*>(ws);
  ws += align256(size_t(G) * k * sizeof(float));
  w.part_ml = reinterpret_cast<float*>(ws);
  ws += align256(size_t(G) * cmax * 2 * sizeof(float));
  w.part_acc = reinterpret_cast<float*>(ws);
  w.chunk_len = L;
  w.chunks = chunks;
  w.cmax = int(cmax);
  st = device_status(h2o::launch_decode_split(cache->dtype, cache->head_dim, G, a, w, static_cast<hipStream_t>(stream)),
                     who);
  if (st != H2O_OK) return st;
  cache->t_next += 1;
  cache->n_used = cache->n_used < k ? cache->n_used + 1 : k;
  cache->steps += 1;
  return H2O_OK;
}

}  // namespace

extern "C" {

const char* h2o_last_error(void) { return g_err; }

#ifndef H2O_SOURCE_DIGEST
#define H2O_SOURCE_DIGEST "unknown"
#endif
const char* h2o_build_digest(void) { return H2O_SOURCE_DIGEST; }

h2o_status h2o_cache_init(h2o_cache* cache, int32_t batch, int32_t heads, int32_t head_dim,
                          int32_t k_heavy, int32_t k_recent, int32_t policy, int32_t dtype, float scale,
                          void* K, void* V, float* score, int32_t* pos, h2o_stream_t stream) {
  return init_cache(cache, batch, heads, head_dim, k_heavy, k_recent, policy, dtype, scale, K, V, score, pos,
                    H2O_QUANT_NONE, nullptr, nullptr, stream);
}

h2o_status h2o_cache_init_quant(h2o_cache* cache, int32_t batch, int32_t heads, int32_t head_dim,
                                int32_t k_heavy, int32_t k_recent, int32_t policy, int32_t dtype, float scale,
                                int32_t quant, uint8_t* Kq, uint8_t* Vq, float* k_qparam, float* v_qparam,
                                float* score, int32_t* pos, h2o_stream_t stream) {
  if (quant != H2O_QUANT_U8 && quant != H2O_QUANT_U4 && quant != H2O_QUANT_U2)
    return fail(H2O_EINVAL, "unknown code format %d (H2O_QUANT_U8, _U4 or _U2)", quant);
  if (!k_qparam || !v_qparam) return fail(H2O_EINVAL, "k_qparam and v_qparam must be non-NULL");
  if (!aligned(k_qparam, 16) || !aligned(v_qparam, 16))
    return fail(H2O_EINVAL, "k_qparam and v_qparam must be 16-byte aligned");
  return init_cache(cache, batch, heads, head_dim, k_heavy, k_recent, policy, dtype, scale, Kq, Vq, score, pos,
                    quant, k_qparam, v_qparam, stream);
}

size_t h2o_prefill_workspace_bytes(int32_t batch, int32_t heads, int32_t n) {
  if (batch < 1 || heads < 1 || n < 0) return 0;
  const size_t G = size_t(batch) * heads;
  return align256(G * lse_ld(n) * sizeof(float)) + align256(G * size_t(n) * sizeof(float));
}

h2o_status h2o_prefill_select(h2o_cache* cache, const void* Q, const void* Kp, const void* Vp,
                              int32_t n, void* workspace, size_t workspace_bytes, float* colsum_out,
                              h2o_stream_t stream) {
  return prefill(cache, Q, Kp, Vp, n, workspace, workspace_bytes, colsum_out, h2o::PASS1_LSE, nullptr, nullptr,
                 nullptr, stream, "h2o_prefill_select");
}

h2o_status h2o_prefill_attention(h2o_cache* cache, const void* Q, const void* Kp, const void* Vp, int32_t n,
                                 void* workspace, size_t workspace_bytes, float* out, float* lse_out,
                                 float* colsum_out, h2o_stream_t stream) {
  if (n > 0 && !out) return fail(H2O_EINVAL, "out must be non-NULL");
  if (out && !aligned(out, 16)) return fail(H2O_EINVAL, "out must be 16-byte aligned");
  if (lse_out && !aligned(lse_out, 4)) return fail(H2O_EINVAL, "lse_out must be 4-byte aligned");
  return prefill(cache, Q, Kp, Vp, n, workspace, workspace_bytes, colsum_out, h2o::PASS1_ATTENTION, out, lse_out,
                 nullptr, stream, "h2o_prefill_attention");
}

h2o_status h2o_prefill_select_lse(h2o_cache* cache, const void* Q, const void* Kp, const void* Vp, int32_t n,
                                  const float* lse, void* workspace, size_t workspace_bytes, float* colsum_out,
                                  h2o_stream_t stream) {
  if (n > 0 && !lse) return fail(H2O_EINVAL, "lse must be non-NULL");
  if (lse && !aligned(lse, 4)) return fail(H2O_EINVAL, "lse must be 4-byte aligned");
  return prefill(cache, Q, Kp, Vp, n, workspace, workspace_bytes, colsum_out, h2o::PASS1_GIVEN, nullptr, nullptr,
                 lse, stream, "h2o_prefill_select_lse");
}

h2o_status h2o_decode_step(h2o_cache* cache, const void* q, const void* k_new, const void* v_new,
                           float* out, int32_t* evicted_pos, h2o_stream_t stream) {
  h2o_status st = check_cache(cache);
  if (st != H2O_OK) return st;
  if (!q || !k_new || !v_new || !out || !evicted_pos)
    return fail(H2O_EINVAL, "q, k_new, v_new, out and evicted_pos must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16) || !aligned(evicted_pos, 4))
    return fail(H2O_EINVAL, "q, k_new, v_new, out must be 16-byte aligned; evicted_pos 4-byte aligned");
  if (cache->t_next == INT32_MAX) return fail(H2O_ESTATE, "position counter exhausted");
  if (cache->quant != H2O_QUANT_NONE && cache->t_next == 0)
    return fail(H2O_ESTATE, "a cache stored as codes must be prefilled first: its key grids come from the prompt");

  const int32_t k = cache->k_heavy + cache->k_recent;
  h2o::DecodeArgs a{};
  a.K = cache->K;
  a.V = cache->V;
  a.K_w = cache->K;
  a.V_w = cache->V;
  a.score = cache->score;
  a.pos = cache->pos;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  a.evicted = evicted_pos;
  a.k = k;
  a.n_used = cache->n_used;
  a.t = cache->t_next;
  a.k_recent = cache->k_recent;
  a.policy = cache->policy;
  a.c = cache->scale * h2o::kLog2e;
  a.k_qparam = cache->k_qparam;
  a.v_qparam = cache->v_qparam;
  const int G = cache->batch * cache->heads;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = device_status(cache->quant != H2O_QUANT_NONE
                         ? h2o::launch_decode_quant(code_bits(cache->quant), cache->dtype, cache->head_dim, G, a, s)
                         : h2o::launch_decode(cache->dtype, cache->head_dim, G, a, s),
                     "h2o_decode_step");
  if (st != H2O_OK) return st;
  cache->t_next += 1;
  cache->n_used = cache->n_used < k ? cache->n_used + 1 : k;
  cache->steps += 1;
  return H2O_OK;
}

size_t h2o_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t k) {
  if (batch < 1 || heads < 1 || k < 1 || k > H2O_MAX_SLOTS || (head_dim != 64 && head_dim != 128)) return 0;
  const size_t G = size_t(batch) * heads;
  const size_t cmax = split_cmax(k);
  return align256(G * k * sizeof(float)) + align256(G * cmax * 2 * sizeof(float)) +
         align256(G * cmax * head_dim * sizeof(float));
}

h2o_status h2o_decode_step_split(h2o_cache* cache, const void* q, const void* k_new, const void* v_new,
                                 float* out, int32_t* evicted_pos, int32_t chunk_rows, void* workspace,
                                 size_t workspace_bytes, h2o_stream_t stream) {
  return split_step(cache, q, k_new, v_new, out, evicted_pos, chunk_rows, workspace, workspace_bytes, stream,
                    "h2o_decode_step_split");
}

h2o_status h2o_decode_step_split_noalloc(h2o_cache* cache, const void* q, const void* k_new, const void* v_new,
                                         float* out, int32_t* evicted_pos, int32_t chunk_rows,
                                         h2o_stream_t stream) {
  h2o_status st = check_cache(cache);
  if (st != H2O_OK) return st;
  const int32_t k = cache->k_heavy + cache->k_recent;
  const size_t need = h2o_decode_workspace_bytes(cache->batch, cache->heads, cache->head_dim, k);
  if (need > H2O_SPLIT_SCRATCH_BYTES)
    return fail(H2O_EWORKSPACE, "this shape needs %zu bytes of split-decode workspace, above the library's own %u",
                need, H2O_SPLIT_SCRATCH_BYTES);
  void* ws = nullptr;
  st = device_status(h2o::split_scratch(&ws), "h2o_decode_step_split_noalloc");
  if (st != H2O_OK) return st;
  return split_step(cache, q, k_new, v_new, out, evicted_pos, chunk_rows, ws, H2O_SPLIT_SCRATCH_BYTES, stream,
                    "h2o_decode_step_split_noalloc");
}

h2o_status h2o_cache_state(const h2o_cache* cache, h2o_state* state, int32_t* pos_host,
                           float* score_host, h2o_stream_t stream) {
  h2o_status st = check_cache(cache);
  if (st != H2O_OK) return st;
  if (!state) return fail(H2O_EINVAL, "state is NULL");
  const int32_t k = cache->k_heavy + cache->k_recent;
  const size_t count = size_t(cache->batch) * cache->heads * k;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pos_host) {
    st = device_status(hipMemcpyAsync(pos_host, cache->pos, count * sizeof(int32_t), hipMemcpyDeviceToHost, s),
                       "h2o_cache_state");
    if (st != H2O_OK) return st;
  }
  if (score_host) {
    st = device_status(hipMemcpyAsync(score_host, cache->score, count * sizeof(float), hipMemcpyDeviceToHost, s),
                       "h2o_cache_state");
    if (st != H2O_OK) return st;
  }
  if (pos_host || score_host) {
    st = device_status(hipStreamSynchronize(s), "h2o_cache_state");
    if (st != H2O_OK) return st;
  }
  state->n_used = cache->n_used;
  state->t_next = cache->t_next;
  state->k = k;
  state->k_heavy = cache->k_heavy;
  state->k_recent = cache->k_recent;
  state->reserved = 0;
  state->steps = cache->steps;
  return H2O_OK;
}

h2o_status h2o_cache_restore(h2o_cache* cache, int32_t t_next, int64_t steps) {
  h2o_status st = check_cache(cache);
  if (st != H2O_OK) return st;
  if (t_next < 0 || t_next == INT32_MAX) return fail(H2O_EINVAL, "t_next %d out of range", t_next);
  if (steps < 0) return fail(H2O_EINVAL, "steps must be >= 0");
  const int32_t k = cache->k_heavy + cache->k_recent;
  cache->t_next = t_next;
  cache->n_used = t_next < k ? t_next : k;
  cache->steps = steps;
  return H2O_OK;
}

h2o_status h2o_fullcache_decode(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype, float scale,
                                int32_t len, const void* q, const void* Kc, const void* Vc, float* out,
                                h2o_stream_t stream) {
  if (batch < 1 || heads < 1) return fail(H2O_EINVAL, "batch and heads must be >= 1");
  if (int64_t(batch) * heads > (int64_t(1) << 31) - 1) return fail(H2O_EINVAL, "batch*heads too large");
  if (head_dim != 64 && head_dim != 128) return fail(H2O_EINVAL, "head_dim %d not supported (64, 128)", head_dim);
  if (dtype != H2O_F32 && dtype != H2O_BF16 && dtype != H2O_F16) return fail(H2O_EINVAL, "unknown dtype %d", dtype);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(H2O_EINVAL, "scale must be finite and > 0");
  if (len < 1) return fail(H2O_EINVAL, "len must be >= 1");
  if (!q || !Kc || !Vc || !out) return fail(H2O_EINVAL, "q, K, V and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(Kc, 16) || !aligned(Vc, 16) || !aligned(out, 16))
    return fail(H2O_EINVAL, "q, K, V and out must be 16-byte aligned");
  h2o::DecodeArgs a{};
  a.K = Kc;
  a.V = Vc;
  a.q = q;
  a.out = out;
  a.k = len;
  a.n_used = len;
  a.c = scale * h2o::kLog2e;
  return device_status(h2o::launch_fullcache(dtype, head_dim, batch * heads, a, static_cast<hipStream_t>(stream)),
                       "h2o_fullcache_decode");
}

}  // extern "C"
