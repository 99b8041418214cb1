// Fused H2O decode step for gfx950.
//
// Citations ("H2O §x") refer to the page "H2O: Heavy-Hitter Oracle for
// Efficient Generative Inference of Large Language Models" (paperlayer.ai
// summary of arXiv 2306.14048v3).
//
// One workgroup (4 waves) per (batch, head). The step is a matrix-vector
// product over k cached rows, so it is HBM-bound and uses VALU dot products,
// not MFMA. Rows are streamed with 16-byte loads: a row of d elements is read
// by LPR = d*bytes/16 consecutive lanes, so one wave-wide load covers RPU =
// 64/LPR consecutive rows (1 KiB, fully coalesced). Each lane group keeps its
// own online-softmax partial (running max m, sum l, and its slice of the
// P.V accumulator) over the rows it streamed, so K and V loads of a batch are
// issued together and no cross-lane traffic is needed inside the loop except
// the DPP reduction of each row's dot product. Raw logits (base-2 units) are
// parked in LDS; after the partials are merged, the exact probability of every
// slot is known and the accumulated scores are updated (H2O §1 "Greedy
// algorithm for low-cost policy", §B.2: accumulated, not averaged).
//
// The victim is the slot with the smallest (score, pos) key among slots
// outside the recent window (H2O §2 "Problem formulation": one eviction at
// most; §D "Cache eviction"), found with a wave shuffle min and an LDS merge.
// The new token then takes the victim's slot (or slot n_used while the cache
// is not full).

#include "h2o_device.h"
#include "launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int DT, int D>
struct Shape {
  static constexpr int E = Elem<DT>::bytes;
  static constexpr int ROW = D * E;      // bytes per cache row
  static constexpr int LPR = ROW / 16;   // lanes per row
  static constexpr int RPU = 64 / LPR;   // rows per wave-wide load
  static constexpr int EPL = 16 / E;     // elements per lane
  static constexpr int NP = kWaves * RPU;  // online-softmax partials per workgroup
  static_assert(LPR >= 4 && LPR <= 64, "row must span 4..64 lanes");
};

// SCORED = true: the H2O step. SCORED = false: plain attention over a
// contiguous cache of n_used rows (no new token, no scores, no eviction).
template <int DT, int D, int UB, int PF, bool SCORED>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using S = Shape<DT, D>;
  __shared__ float sm_m[S::NP];
  __shared__ float sm_l[S::NP];
  __shared__ __attribute__((aligned(16))) float sm_acc[S::NP][D];
  __shared__ float sm_vnew[D];
  __shared__ uint64_t sm_key[kWaves];
  __shared__ int sm_slot[kWaves];
  extern __shared__ float sm_logit[];  // [n_used] logits in base-2 units (scored)

  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane / S::LPR;
  const int sub = lane % S::LPR;
  const int part = wave * S::RPU + grp;
  const int nu = a.n_used;
  const size_t head_rows = size_t(head) * a.k;

  const char* Kh = static_cast<const char*>(a.K) + head_rows * S::ROW + sub * 16;
  const char* Vh = static_cast<const char*>(a.V) + head_rows * S::ROW + sub * 16;
  const uint4 qv = ld16(static_cast<const char*>(a.q) + size_t(head) * S::ROW + sub * 16);

  uint4 kn = make_uint4(0, 0, 0, 0), vn = make_uint4(0, 0, 0, 0);
  float sc_pf[PF];
  int pos_pf[PF];
  if constexpr (SCORED) {
    kn = ld16(static_cast<const char*>(a.k_new) + size_t(head) * S::ROW + sub * 16);
    vn = ld16(static_cast<const char*>(a.v_new) + size_t(head) * S::ROW + sub * 16);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int slot = tid + i * kThreads;
      sc_pf[i] = 0.f;
      pos_pf[i] = 0;
      if (slot < nu) {
        sc_pf[i] = a.score[head_rows + slot];
        pos_pf[i] = a.pos[head_rows + slot];
      }
    }
  }

  // ---- stream K and V rows: per-group online softmax -------------------------
  float m = kNegInf, l = 0.f;
  float acc[S::EPL];
#pragma unroll
  for (int e = 0; e < S::EPL; ++e) acc[e] = 0.f;

  const int units = (nu + S::RPU - 1) / S::RPU;
  for (int u0 = wave; u0 < units; u0 += kWaves * UB) {
    uint4 kr[UB], vr[UB];
    int row[UB];
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      row[j] = (u0 + kWaves * j) * S::RPU + grp;
      kr[j] = make_uint4(0, 0, 0, 0);
      vr[j] = make_uint4(0, 0, 0, 0);
      if (row[j] < nu) {
        kr[j] = ld16(Kh + size_t(row[j]) * S::ROW);
        vr[j] = ld16(Vh + size_t(row[j]) * S::ROW);
      }
    }
    float s[UB];
    float bm = kNegInf;
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const float x = group_sum<S::LPR>(dot16<DT>(qv, kr[j])) * a.c;
      s[j] = row[j] < nu ? x : kNegInf;
      bm = fmaxf(bm, s[j]);
    }
    if constexpr (SCORED) {
#pragma unroll
      for (int j = 0; j < UB; ++j)
        if (sub == 0 && row[j] < nu) sm_logit[row[j]] = s[j];
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
        Unpack<DT>::run(vr[j], v);
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) acc[e] = fmaf(p, v[e], acc[e]);
      }
      m = mn;
    }
  }

  // ---- merge the partials ----------------------------------------------------
  if (sub == 0) {
    sm_m[part] = m;
    sm_l[part] = l;
  }
#pragma unroll
  for (int e = 0; e < S::EPL; e += 4)
    *reinterpret_cast<float4*>(&sm_acc[part][sub * S::EPL + e]) =
        make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);

  float s_new = kNegInf;
  if constexpr (SCORED) {
    s_new = group_sum<S::LPR>(dot16<DT>(qv, kn)) * a.c;
    if (wave == 0 && grp == 0) {
      float v[S::EPL];
      Unpack<DT>::run(vn, v);
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) sm_vnew[sub * S::EPL + e] = v[e];
    }
  }
  __syncthreads();

  float M = s_new;
#pragma unroll
  for (int p = 0; p < S::NP; ++p) M = fmaxf(M, sm_m[p]);
  float Z = fast_exp2(s_new - M);
  float w[S::NP];
#pragma unroll
  for (int p = 0; p < S::NP; ++p) {
    w[p] = fast_exp2(sm_m[p] - M);
    Z = fmaf(sm_l[p], w[p], Z);
  }
  const float invZ = 1.0f / Z;

  if (tid < D) {
    float o = SCORED ? fast_exp2(s_new - M) * sm_vnew[tid] : 0.f;
#pragma unroll
    for (int p = 0; p < S::NP; ++p) o = fmaf(sm_acc[p][tid], w[p], o);
    a.out[size_t(head) * D + tid] = o * invZ;
  }

  if constexpr (SCORED) {
    // ---- accumulate scores, pick the victim ----------------------------------
    const float p_new = fast_exp2(s_new - M) * invZ;
    const bool full = nu == a.k;
    const int lim = a.t - a.k_recent;  // eligible iff pos <= t - k_recent
    float* sc_g = a.score + head_rows;
    int32_t* pos_g = a.pos + head_rows;
    uint64_t best = ~0ull;
    int best_slot = -1;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int slot = tid + i * kThreads;
      if (slot < nu) {
        const float sc = sc_pf[i] + fast_exp2(sm_logit[slot] - M) * invZ;
        sc_g[slot] = sc;
        if (full && pos_pf[i] <= lim) {
          const uint64_t key = score_pos_key(sc, pos_pf[i]);
          if (key < best) {
            best = key;
            best_slot = slot;
          }
        }
      }
    }
    for (int slot = tid + PF * kThreads; slot < nu; slot += kThreads) {
      const float sc = sc_g[slot] + fast_exp2(sm_logit[slot] - M) * invZ;
      const int ps = pos_g[slot];
      sc_g[slot] = sc;
      if (full && ps <= lim) {
        const uint64_t key = score_pos_key(sc, ps);
        if (key < best) {
          best = key;
          best_slot = slot;
        }
      }
    }

    int victim = nu;  // not full: the next free slot
    int evicted = -1;
    if (full) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t ok = __shfl_xor(best, off);
        const int os = __shfl_xor(best_slot, off);
        if (ok < best) {
          best = ok;
          best_slot = os;
        }
      }
      if (lane == 0) {
        sm_key[wave] = best;
        sm_slot[wave] = best_slot;
      }
      __syncthreads();
      best = sm_key[0];
      best_slot = sm_slot[0];
#pragma unroll
      for (int wv = 1; wv < kWaves; ++wv) {
        if (sm_key[wv] < best) {
          best = sm_key[wv];
          best_slot = sm_slot[wv];
        }
      }
      victim = best_slot;
      // A full cache always has k_heavy + 1 eligible slots; if the caller's
      // state broke that invariant nothing is written and -2 is reported.
      evicted = victim >= 0 ? int(uint32_t(best & 0xffffffffu)) : -2;
    }

    // ---- insert the new token --------------------------------------------------
    if (victim >= 0) {
      if (tid == victim % kThreads) {  // the thread that owns the slot's score
        sc_g[victim] = p_new;
        pos_g[victim] = a.t;
      }
      if (wave == 0 && grp == 0) {
        st16(static_cast<char*>(a.K_w) + (head_rows + victim) * S::ROW + sub * 16, kn);
        st16(static_cast<char*>(a.V_w) + (head_rows + victim) * S::ROW + sub * 16, vn);
      }
    }
    if (tid == 0) a.evicted[head] = evicted;
  }
}

template <int DT, int D, bool SCORED>
hipError_t launch_typed(int G, const DecodeArgs& a, hipStream_t s) {
  constexpr int UB = 8;
  constexpr int PF = 4;
  const size_t shmem = SCORED ? size_t(a.k) * sizeof(float) : 0;
  hipLaunchKernelGGL((decode_kernel<DT, D, UB, PF, SCORED>), dim3(G), dim3(kThreads), shmem, s, a);
  return hipGetLastError();
}

template <bool SCORED>
hipError_t dispatch(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s) {
  if (G <= 0) return hipSuccess;
  switch (dtype * 1000 + head_dim) {
    case DT_F32 * 1000 + 64: return launch_typed<DT_F32, 64, SCORED>(G, a, s);
    case DT_F32 * 1000 + 128: return launch_typed<DT_F32, 128, SCORED>(G, a, s);
    case DT_BF16 * 1000 + 64: return launch_typed<DT_BF16, 64, SCORED>(G, a, s);
    case DT_BF16 * 1000 + 128: return launch_typed<DT_BF16, 128, SCORED>(G, a, s);
    case DT_F16 * 1000 + 64: return launch_typed<DT_F16, 64, SCORED>(G, a, s);
    case DT_F16 * 1000 + 128: return launch_typed<DT_F16, 128, SCORED>(G, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s) {
  return dispatch<true>(dtype, head_dim, G, a, s);
}

hipError_t launch_fullcache(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s) {
  return dispatch<false>(dtype, head_dim, G, a, s);
}

}  // namespace h2o
