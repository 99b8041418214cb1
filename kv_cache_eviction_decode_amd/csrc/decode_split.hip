// Split H2O decode step for gfx950: few (batch, head) pairs, long caches.
//
// Citations ("H2O §x") refer to the page "H2O: Heavy-Hitter Oracle for
// Efficient Generative Inference of Large Language Models" (paperlayer.ai
// summary of arXiv 2306.14048v3).
//
// The step is the fused one (attention of the new token over the occupied
// slots and itself, H2O §D "Recursive attention"; accumulation of the
// normalised attention into every slot's score, §1 and §B.2; at most one
// eviction, the smallest (value, pos) outside the recent window, §2 "Problem
// formulation" and §D "Cache eviction"; insert into the freed slot). What
// changes is the work split, so that a handful of heads still puts thousands
// of waves on the chip:
//
//   decode_chunk_kernel  - the occupied slots of a head are cut into chunks
//     of chunk_len rows, each streamed by its own wave; a chunk leaves its
//     logits and its online-softmax partial (max m_c, sum l_c, unnormalised
//     P.V) in the workspace.
//   decode_merge_kernel  - one 512-thread workgroup per head merges the
//     partials (M = max(m_c, s_new), Z = sum l_c 2^(m_c - M) + 2^(s_new - M)),
//     writes the output, adds 2^(logit - M)/Z to every slot's score, picks the
//     victim and inserts the new token.
//
// The kernel boundary orders the two (the chunks of a head run on different
// XCDs, whose L2 caches are only made coherent at kernel boundaries), so both
// kernels use plain, vectorised loads and stores and nothing waits on another
// workgroup. A single-kernel variant in which the last chunk to arrive does
// the merge was measured slower: one wave per head is too little parallelism
// for the merge, and the cross-XCD hand-over needs write-through stores or an
// L2 write-back, whose latency sits on the critical path.

#include <mutex>

#include "../../include/h2o.h"
#include "h2o_device.h"
#include "launch.h"

namespace h2o {
namespace {

// Workspace of h2o_decode_step_split_noalloc: one array per GPU, held for the
// life of the process. Host code never uses this name as an address (on the
// host it is only a stand-in for the symbol); it uses the device address
// that hipGetSymbolAddress returns, kept per device by split_scratch().
static __device__ __align__(256) char scratch[H2O_SPLIT_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Merge workgroup: 512 threads, 4 slots each per round (256 threads: 2% slower at
// one sequence of 32 heads x 2048 slots, 1024 threads: 7% slower).
constexpr int kMergeThreads = 512;
constexpr int kMergeWaves = kMergeThreads / 64;

// One wave per (head, chunk); block b is chunk b % chunks of head b / chunks.
//   UB: 1 KiB wave-loads of K (and as many of V) per batch; two batches in flight.
template <int DT, int D, int UB>
__global__ __launch_bounds__(64, 2) void decode_chunk_kernel(DecodeArgs a, SplitArgs w) {
  using S = Shape<DT, D, 1>;
  extern __shared__ float sm_lg[];  // [chunk_len] logits of this chunk, base-2 units
  const int lane = threadIdx.x;
  const int grp = lane / S::LPR;
  const int sub = lane % S::LPR;
  const int head = blockIdx.x / w.chunks;
  const int chunk = blockIdx.x - head * w.chunks;
  const int nu = a.n_used;
  const int r0 = chunk * w.chunk_len;
  const int r1 = min(r0 + w.chunk_len, nu);
  const int rows = r1 > r0 ? r1 - r0 : 0;
  const int nb = (rows + S::RPU * UB - 1) / (S::RPU * UB);  // batches in this chunk
  const size_t hrow = size_t(head) * a.k;
  const char* Kh = static_cast<const char*>(a.K) + hrow * S::ROW + sub * 16;
  const char* Vh = static_cast<const char*>(a.V) + hrow * S::ROW + sub * 16;
  const uint4 q = ld16(static_cast<const char*>(a.q) + size_t(head) * S::ROW + sub * 16);

  // Unconditional loads (rows past the chunk are clamped to its last row and
  // masked), as in the fused kernel: the wait counts stay exact.
  auto issue = [&](uint4 (&kb)[UB], uint4 (&vb)[UB], int b) {
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const int row = min(r0 + (b * UB + j) * S::RPU + grp, r1 - 1);
      kb[j] = ldnt16(Kh + size_t(row) * S::ROW);
      vb[j] = ldnt16(Vh + size_t(row) * S::ROW);
    }
  };
  float m = kNegInf, l = 0.f;
  float acc[S::EPL];
#pragma unroll
  for (int e = 0; e < S::EPL; ++e) acc[e] = 0.f;
  auto compute = [&](const uint4 (&kc)[UB], const uint4 (&vc)[UB], int b) {
    float s[UB];
    float bm = kNegInf;
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const int row = r0 + (b * UB + j) * S::RPU + grp;
      const float x = group_sum<S::LPR>(dot16<DT>(q, kc[j])) * a.c;
      s[j] = row < r1 ? x : kNegInf;
      bm = fmaxf(bm, s[j]);
      if (sub == 0 && row < r1) sm_lg[row - r0] = s[j];
    }
    if (bm != kNegInf) {
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) acc[e] *= alpha;
#pragma unroll
      for (int j = 0; j < UB; ++j) {
        const float p = fast_exp2(s[j] - mn);
        l += p;
        float v[S::EPL];
        Unpack<DT>::run(vc[j], v);
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) acc[e] = fmaf(p, v[e], acc[e]);
      }
      m = mn;
    }
  };

  if (nb > 0) {
    uint4 kA[UB], vA[UB], kB[UB], vB[UB];
    issue(kA, vA, 0);
    for (int b = 0; b < nb; b += 2) {
      set_wave_priority(3 - (4 * b) / nb);  // lagging waves of a SIMD issue first
      issue(kB, vB, b + 1);
      compute(kA, vA, b);
      issue(kA, vA, b + 2);
      compute(kB, vB, b + 1);
    }
  }

  // Logits were parked in LDS while streaming (global stores between the loads
  // would hold up the loads' wait counts); they leave in coalesced stores.
  __syncthreads();
  float* lg_g = w.logit + hrow + r0;
  for (int i = lane; i < rows; i += 64) lg_g[i] = sm_lg[i];

  const float mc = across_groups<S::LPR>(m, OpMax());
  const float wg = mc == kNegInf ? 0.f : fast_exp2(m - mc);  // empty chunk: all zero
  const float lc = across_groups<S::LPR>(l * wg, OpAdd());
#pragma unroll
  for (int e = 0; e < S::EPL; ++e) acc[e] = across_groups<S::LPR>(acc[e] * wg, OpAdd());
  const size_t part = size_t(head) * w.cmax + chunk;
  if (grp == 0) {
    float* pa = w.part_acc + part * D + sub * S::EPL;
#pragma unroll
    for (int e = 0; e < S::EPL; e += 4)
      *reinterpret_cast<float4*>(pa + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
  if (lane == 0) *reinterpret_cast<float2*>(w.part_ml + 2 * part) = make_float2(mc, lc);
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  return across_groups<16>(x, OpMax());
}

template <int DT> __device__ __forceinline__ float load_elem(const void* p, size_t i);
template <> __device__ __forceinline__ float load_elem<DT_F32>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load_elem<DT_BF16>(const void* p, size_t i) {
  return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
}
template <> __device__ __forceinline__ float load_elem<DT_F16>(const void* p, size_t i) {
  return float(static_cast<const _Float16*>(p)[i]);
}

// One workgroup per head. Every load the merge needs for up to 2048 slots
// is issued before the first one is used.
template <int DT, int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a, SplitArgs w) {
  using S = Shape<DT, D, 1>;
  constexpr int LPC = D / 4;                // threads per partial row (16 bytes each)
  constexpr int RPL = kMergeThreads / LPC;  // partial rows per block-wide load
  constexpr int NB = kMaxChunks / RPL;      // block-wide loads covering every chunk
  constexpr int U = 4;                      // slots per thread per round
  static_assert(kMaxChunks <= kMergeThreads, "one chunk maximum per thread");
  __shared__ float sm_red[kMergeWaves];
  __shared__ __attribute__((aligned(16))) float sm_acc[kMergeWaves][D];
  __shared__ uint64_t sm_key[kMergeWaves];
  __shared__ int sm_victim, sm_evicted;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int head = blockIdx.x;
  const int nu = a.n_used;
  const int C = w.chunks;
  const size_t hrow = size_t(head) * a.k;
  const float* pml = w.part_ml + size_t(head) * w.cmax * 2;
  const float* pacc = w.part_acc + size_t(head) * w.cmax * D;
  const float* lg_g = w.logit + hrow;
  float* sc_g = a.score + hrow;
  int32_t* pos_g = a.pos + hrow;

  // ---- loads -----------------------------------------------------------------------
  const int sub = lane % S::LPR;
  const size_t hoff = size_t(head) * S::ROW + sub * 16;
  const uint4 q = ld16(static_cast<const char*>(a.q) + hoff);
  const uint4 kn = ld16(static_cast<const char*>(a.k_new) + hoff);
  const uint4 vn = ld16(static_cast<const char*>(a.v_new) + hoff);
  const float2 ml = *reinterpret_cast<const float2*>(pml + 2 * min(tid, C - 1));
  const int col = 4 * (tid % LPC);
  const int crow = tid / LPC;
  float4 pv[NB];
  float mx[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int c = min(crow + RPL * i, C - 1);
    pv[i] = *reinterpret_cast<const float4*>(pacc + size_t(c) * D + col);
    mx[i] = pml[2 * c];
  }
  float vo[4];  // the new value at this thread's output columns
#pragma unroll
  for (int e = 0; e < 4; ++e) vo[e] = load_elem<DT>(a.v_new, size_t(head) * D + col + e);
  float lg[U], sc[U];
  int ps[U];
  auto load_slots = [&](int base) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int slot = min(base + tid + kMergeThreads * i, nu - 1);
      lg[i] = lg_g[slot];
      sc[i] = sc_g[slot];
      ps[i] = pos_g[slot];
    }
  };
  if (nu > 0) load_slots(0);

  // ---- M, Z and the output ---------------------------------------------------------
  const float s_new = group_sum<S::LPR>(dot16<DT>(q, kn)) * a.c;
  float M = wave_max(fmaxf(s_new, tid < C ? ml.x : kNegInf));
  if (lane == 0) sm_red[wave] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMergeWaves; ++i) M = fmaxf(M, sm_red[i]);
  __syncthreads();
  const float lw_own = tid < C ? ml.y * fast_exp2(ml.x - M) : 0.f;  // an empty chunk has m = -inf
  const float lw_wave = group_sum<64>(lw_own);
  if (lane == 0) sm_red[wave] = lw_wave;
  // P.V: the weighted partial rows, then the RPL row groups summed (lanes, LDS).
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (crow + RPL * i < C) {
      const float wc = fast_exp2(mx[i] - M);
      o[0] = fmaf(wc, pv[i].x, o[0]);
      o[1] = fmaf(wc, pv[i].y, o[1]);
      o[2] = fmaf(wc, pv[i].z, o[2]);
      o[3] = fmaf(wc, pv[i].w, o[3]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = across_groups<LPC>(o[e], OpAdd());
  if (lane < LPC) *reinterpret_cast<float4*>(&sm_acc[wave][col]) = make_float4(o[0], o[1], o[2], o[3]);
  __syncthreads();
  float lw = 0.f;
#pragma unroll
  for (int i = 0; i < kMergeWaves; ++i) lw += sm_red[i];
  const float w_new = fast_exp2(s_new - M);
  const float invZ = 1.0f / (lw + w_new);
  if (tid < LPC) {
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = 0.f;
#pragma unroll
      for (int v = 0; v < kMergeWaves; ++v) x += sm_acc[v][col + e];
      r[e] = fmaf(w_new, vo[e], x) * invZ;
    }
    *reinterpret_cast<float4*>(a.out + size_t(head) * D + col) = make_float4(r[0], r[1], r[2], r[3]);
  }

  // ---- accumulate scores, pick the victim ------------------------------------------
  const float p_new = w_new * invZ;
  const bool full = nu == a.k;
  const int lim = a.t - a.k_recent;  // eligible iff pos <= t - k_recent
  uint64_t best = ~0ull;
  int best_slot = -1, best_pos = -1;
  for (int base = 0; base < nu; base += kMergeThreads * U) {
    if (base > 0) load_slots(base);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int slot = base + tid + kMergeThreads * i;
      if (slot < nu) {
        const float v = sc[i] + fast_exp2(lg[i] - M) * invZ;
        sc_g[slot] = v;
        if (full && ps[i] <= lim) {
          const uint64_t key = evict_key(v, ps[i], a.t, a.policy);
          if (key < best) {
            best = key;
            best_slot = slot;
            best_pos = ps[i];
          }
        }
      }
    }
  }
  // Without a recent window the new token competes too (slot k = "itself").
  if (full && a.k_recent == 0 && tid == 0) {
    const uint64_t key = evict_key(p_new, a.t, a.t, a.policy);
    if (key < best) {
      best = key;
      best_slot = a.k;
      best_pos = a.t;
    }
  }
  int victim = nu;  // not full: the next free slot
  int evicted = -1;
  if (full) {
    const uint64_t wmin = wave_min_u64(best);
    if (lane == 0) sm_key[wave] = wmin;
    if (tid == 0) {
      sm_victim = -1;  // no eligible slot: the caller's state is inconsistent
      sm_evicted = -2;
    }
    __syncthreads();
    uint64_t gmin = sm_key[0];
#pragma unroll
    for (int i = 1; i < kMergeWaves; ++i) gmin = min64(gmin, sm_key[i]);
    // Keys are unique (positions are), so exactly one thread holds the minimum.
    if (gmin != ~0ull && best == gmin) {
      sm_victim = best_slot;
      sm_evicted = best_pos;
    }
    __syncthreads();
    victim = sm_victim;
    evicted = sm_evicted;
  }

  // ---- insert the new token (unless it was the one evicted) -------------------------
  // The slot's score and pos are written by the thread that updated it above.
  if (victim >= 0 && victim < a.k) {
    if (tid == victim % kMergeThreads) {
      sc_g[victim] = p_new;
      pos_g[victim] = a.t;
    }
    if (tid < S::LPR) {
      st16(static_cast<char*>(a.K_w) + (hrow + victim) * S::ROW + sub * 16, kn);
      st16(static_cast<char*>(a.V_w) + (hrow + victim) * S::ROW + sub * 16, vn);
    }
  }
  if (tid == 0) a.evicted[head] = evicted;
}

template <int DT, int D>
hipError_t launch_split_typed(int G, const DecodeArgs& a, const SplitArgs& w, hipStream_t s) {
  constexpr int UB = 4;  // 4-deep batches, as in the fused kernels
  const int64_t blocks = int64_t(G) * w.chunks;
  const size_t shmem = size_t(w.chunk_len) * sizeof(float);
  hipLaunchKernelGGL((decode_chunk_kernel<DT, D, UB>), dim3(uint32_t(blocks)), dim3(64), shmem, s, a, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<DT, D>), dim3(G), dim3(kMergeThreads), 0, s, a, w);
  return hipGetLastError();
}

}  // namespace

hipError_t split_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_split(int dtype, int head_dim, int G, const DecodeArgs& a, const SplitArgs& w,
                               hipStream_t s) {
  if (G <= 0) return hipSuccess;
  switch (dtype * 1000 + head_dim) {
    case DT_F32 * 1000 + 64: return launch_split_typed<DT_F32, 64>(G, a, w, s);
    case DT_F32 * 1000 + 128: return launch_split_typed<DT_F32, 128>(G, a, w, s);
    case DT_BF16 * 1000 + 64: return launch_split_typed<DT_BF16, 64>(G, a, w, s);
    case DT_BF16 * 1000 + 128: return launch_split_typed<DT_BF16, 128>(G, a, w, s);
    case DT_F16 * 1000 + 64: return launch_split_typed<DT_F16, 64>(G, a, w, s);
    case DT_F16 * 1000 + 128: return launch_split_typed<DT_F16, 128>(G, a, w, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace h2o
