// Fused H2O decode step for gfx950.
//
// Citations ("H2O §x") refer to the page "H2O: Heavy-Hitter Oracle for
// Efficient Generative Inference of Large Language Models" (paperlayer.ai
// summary of arXiv 2306.14048v3).
//
// The step is a matrix-vector product over the k cached rows of every
// (batch, head), so it is HBM-bound and uses VALU dot products, not MFMA.
// Rows are streamed with 16-byte loads: a row of d elements is read by
// LPR = d*bytes/16 consecutive lanes, so one wave-wide load covers RPU =
// 64/LPR consecutive rows (1 KiB, fully coalesced). Each lane group keeps its
// own online-softmax partial (running max m, sum l and its slice of the P.V
// accumulator) over the rows it streamed, so K and V loads are issued
// together and the only cross-lane work inside the loop is the DPP reduction
// of each row's dot product. Raw logits (base-2 units) are parked in LDS;
// once the partials are merged the exact probability of every slot is known
// and the accumulated scores are updated (H2O §1 "Greedy algorithm for
// low-cost policy", §B.2: accumulated, not averaged). The victim is the slot
// with the smallest (score, pos) key among slots outside the recent window
// (H2O §2 "Problem formulation": one eviction at most; §D "Cache eviction");
// the new token then takes the victim's slot (or slot n_used while the cache
// is not full).
//
// Two launch shapes share this arithmetic:
//   decode_wave_kernel - one wave per head, persistent, double-buffered, all
//     reductions inside the wave (DPP, v_permlane*_swap); used when there are
//     enough heads to give every SIMD at least one wave.
//   decode_kernel      - one 8-wave workgroup per head with an LDS merge; used
//     for few heads with long caches.

#include "h2o_device.h"
#include "launch.h"

namespace h2o {
namespace {

// SCORED = true: the H2O step. SCORED = false: plain attention over a
// contiguous cache of n_used rows (no new token, no scores, no eviction).
//   WAVES: waves per workgroup (the head's rows are split over them)
//   UB:    1 KiB wave-loads of K (and as many of V) issued together per batch
//   PF:    score/pos entries per thread prefetched at kernel start
//   MINW:  occupancy hint (waves per SIMD) for the register budget
template <int DT, int D, int WAVES, int UB, int PF, int MINW, bool SCORED>
__global__ __launch_bounds__(WAVES * 64, MINW) void decode_kernel(DecodeArgs a) {
  using S = Shape<DT, D, WAVES>;
  constexpr int kThreads = WAVES * 64;
  constexpr int kWaves = WAVES;
  __shared__ float sm_m[S::NP];
  __shared__ float sm_l[S::NP];
  __shared__ __attribute__((aligned(16))) float sm_acc[S::NP][D];
  __shared__ float sm_vnew[D];
  __shared__ uint64_t sm_key[kWaves];
  __shared__ int sm_slot[kWaves];
  __shared__ int sm_epos[kWaves];
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
        kr[j] = ldnt16(Kh + size_t(row[j]) * S::ROW);
        vr[j] = ldnt16(Vh + size_t(row[j]) * S::ROW);
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

  for (int dd = tid; dd < D; dd += kThreads) {
    float o = SCORED ? fast_exp2(s_new - M) * sm_vnew[dd] : 0.f;
#pragma unroll
    for (int p = 0; p < S::NP; ++p) o = fmaf(sm_acc[p][dd], w[p], o);
    a.out[size_t(head) * D + dd] = o * invZ;
  }

  if constexpr (SCORED) {
    // ---- accumulate scores, pick the victim ----------------------------------
    const float p_new = fast_exp2(s_new - M) * invZ;
    const bool full = nu == a.k;
    const int lim = a.t - a.k_recent;  // eligible iff pos <= t - k_recent
    float* sc_g = a.score + head_rows;
    int32_t* pos_g = a.pos + head_rows;
    uint64_t best = ~0ull;
    int best_slot = -1, best_pos = -1;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int slot = tid + i * kThreads;
      if (slot < nu) {
        const float sc = sc_pf[i] + fast_exp2(sm_logit[slot] - M) * invZ;
        sc_g[slot] = sc;
        if (full && pos_pf[i] <= lim) {
          const uint64_t key = evict_key(sc, pos_pf[i], a.t, a.policy);
          if (key < best) {
            best = key;
            best_slot = slot;
            best_pos = pos_pf[i];
          }
        }
      }
    }
    for (int slot = tid + PF * kThreads; slot < nu; slot += kThreads) {
      const float sc = sc_g[slot] + fast_exp2(sm_logit[slot] - M) * invZ;
      const int ps = pos_g[slot];
      sc_g[slot] = sc;
      if (full && ps <= lim) {
        const uint64_t key = evict_key(sc, ps, a.t, a.policy);
        if (key < best) {
          best = key;
          best_slot = slot;
          best_pos = ps;
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
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t ok = __shfl_xor(best, off);
        const int os = __shfl_xor(best_slot, off);
        const int op = __shfl_xor(best_pos, off);
        if (ok < best) {
          best = ok;
          best_slot = os;
          best_pos = op;
        }
      }
      if (lane == 0) {
        sm_key[wave] = best;
        sm_slot[wave] = best_slot;
        sm_epos[wave] = best_pos;
      }
      __syncthreads();
      best = sm_key[0];
      best_slot = sm_slot[0];
      best_pos = sm_epos[0];
#pragma unroll
      for (int wv = 1; wv < kWaves; ++wv) {
        if (sm_key[wv] < best) {
          best = sm_key[wv];
          best_slot = sm_slot[wv];
          best_pos = sm_epos[wv];
        }
      }
      // A full cache always has an eligible candidate; if the caller's state
      // broke that invariant nothing is written and -2 is reported.
      victim = best == ~0ull ? -1 : best_slot;
      evicted = best == ~0ull ? -2 : best_pos;
    }

    // ---- insert the new token (unless it was the one evicted) -----------------
    if (victim >= 0 && victim < a.k) {
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

template <int DT, int D, int PF>
struct HeadInputs {
  uint4 q, kn, vn;
  float sc[PF];
  int pos[PF];
};

template <int DT, int D, int UB, int PF, int MINW, bool SCORED, bool FAIR = true>
__global__ __launch_bounds__(64, MINW) void decode_wave_kernel(DecodeArgs a, int G) {
  using S = Shape<DT, D, 1>;
  extern __shared__ float sm_logit[];  // [k] logits of the current head, base-2 units
  const int lane = threadIdx.x;
  const int grp = lane / S::LPR;
  const int sub = lane % S::LPR;
  const int nu = a.n_used;
  const int units = (nu + S::RPU - 1) / S::RPU;
  const int nb = (units + UB - 1) / UB;  // batches per head
  const size_t kstride = size_t(a.k) * S::ROW;

  int head = blockIdx.x;
  if (head >= G) return;

  auto load_head = [&](HeadInputs<DT, D, PF>& h, int hd) {
    const size_t off = size_t(hd) * S::ROW + sub * 16;
    h.q = ld16(static_cast<const char*>(a.q) + off);
    if constexpr (SCORED) {
      h.kn = ld16(static_cast<const char*>(a.k_new) + off);
      h.vn = ld16(static_cast<const char*>(a.v_new) + off);
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        const int slot = lane + 64 * i;
        h.sc[i] = 0.f;
        h.pos[i] = 0;
        if (slot < nu) {
          h.sc[i] = a.score[size_t(hd) * a.k + slot];
          h.pos[i] = a.pos[size_t(hd) * a.k + slot];
        }
      }
    }
  };
  // Loads are unconditional (rows past n_used are clamped to the last occupied
  // row and masked out of the softmax): exec-masked loads would need their
  // destination registers zeroed first, which forces a wait on the batch
  // still in flight and serialises the pipeline. Only called when nu >= 1.
  auto issue = [&](uint4 (&kb)[UB], uint4 (&vb)[UB], int hd, int b) {
    const char* Kh = static_cast<const char*>(a.K) + hd * kstride + sub * 16;
    const char* Vh = static_cast<const char*>(a.V) + hd * kstride + sub * 16;
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const int row = min((b * UB + j) * S::RPU + grp, nu - 1);
      kb[j] = ldnt16(Kh + size_t(row) * S::ROW);
      vb[j] = ldnt16(Vh + size_t(row) * S::ROW);
    }
  };

  HeadInputs<DT, D, PF> cur;
  uint4 kA[UB], vA[UB], kB[UB], vB[UB];
  float m, l;
  float acc[S::EPL];

  auto compute = [&](const uint4 (&kc)[UB], const uint4 (&vc)[UB], int b) {
    float s[UB];
    float bm = kNegInf;
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const int row = (b * UB + j) * S::RPU + grp;
      const float x = group_sum<S::LPR>(dot16<DT>(cur.q, kc[j])) * a.c;
      s[j] = row < nu ? x : kNegInf;
      bm = fmaxf(bm, s[j]);
      if constexpr (SCORED) {
        if (sub == 0 && row < nu) sm_logit[row] = s[j];
      }
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
  auto epilogue = [&]() {
    const size_t hrow = size_t(head) * a.k;
    // Logits of this lane's slots do not depend on the merge: fetch them first.
    float lg[PF];
    if constexpr (SCORED) {
#pragma unroll
      for (int i = 0; i < PF; ++i) lg[i] = (lane + 64 * i < nu) ? sm_logit[lane + 64 * i] : kNegInf;
    }
    float s_new = kNegInf;
    if constexpr (SCORED) s_new = group_sum<S::LPR>(dot16<DT>(cur.q, cur.kn)) * a.c;
    // Merge the lane-group partials: an all-reduce across groups.
    const float M = fmaxf(across_groups<S::LPR>(m, OpMax()), s_new);
    const float w = fast_exp2(m - M);
    const float lw = across_groups<S::LPR>(l * w, OpAdd());
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) acc[e] = across_groups<S::LPR>(acc[e] * w, OpAdd());
    const float w_new = fast_exp2(s_new - M);
    const float invZ = 1.0f / (lw + w_new);
    if (grp == 0) {
      float o[S::EPL];
      if constexpr (SCORED) {
        float v[S::EPL];
        Unpack<DT>::run(cur.vn, v);
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) o[e] = fmaf(w_new, v[e], acc[e]) * invZ;
      } else {
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) o[e] = acc[e] * invZ;
      }
      float* op = a.out + size_t(head) * D + sub * S::EPL;
#pragma unroll
      for (int e = 0; e < S::EPL; e += 4)
        *reinterpret_cast<float4*>(op + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    }
    if constexpr (SCORED) {
      const float p_new = w_new * invZ;
      const bool full = nu == a.k;
      const int lim = a.t - a.k_recent;
      float* sc_g = a.score + hrow;
      int32_t* pos_g = a.pos + hrow;
      uint64_t best = ~0ull;
      int best_slot = -1, best_pos = -1;
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        const int slot = lane + 64 * i;
        if (slot < nu) {
          const float sc = cur.sc[i] + fast_exp2(lg[i] - M) * invZ;
          sc_g[slot] = sc;
          if (full && cur.pos[i] <= lim) {
            const uint64_t key = evict_key(sc, cur.pos[i], a.t, a.policy);
            if (key < best) {
              best = key;
              best_slot = slot;
              best_pos = cur.pos[i];
            }
          }
        }
      }
      for (int slot = lane + 64 * PF; slot < nu; slot += 64) {
        const float sc = sc_g[slot] + fast_exp2(sm_logit[slot] - M) * invZ;
        const int ps = pos_g[slot];
        sc_g[slot] = sc;
        if (full && ps <= lim) {
          const uint64_t key = evict_key(sc, ps, a.t, a.policy);
          if (key < best) {
            best = key;
            best_slot = slot;
            best_pos = ps;
          }
        }
      }
      // Without a recent window the new token competes too (slot k = "itself").
      if (full && a.k_recent == 0 && lane == 0) {
        const uint64_t key = evict_key(p_new, a.t, a.t, a.policy);
        if (key < best) {
          best = key;
          best_slot = a.k;
          best_pos = a.t;
        }
      }
      int victim = nu;
      int evicted = -1;
      if (full) {
        const uint64_t gmin = wave_min_u64(best);
        // Keys are unique (positions are), so exactly one lane holds the minimum.
        const uint64_t owners = __ballot(best == gmin && gmin != ~0ull);
        if (owners) {
          const int owner = __ffsll((unsigned long long)owners) - 1;
          victim = __builtin_amdgcn_readlane(best_slot, owner);
          evicted = __builtin_amdgcn_readlane(best_pos, owner);
        } else {
          victim = -1;  // no eligible slot: the caller's state is inconsistent
          evicted = -2;
        }
      }
      if (victim >= 0 && victim < a.k) {
        if (lane == victim % 64) {
          sc_g[victim] = p_new;
          pos_g[victim] = a.t;
        }
        if (grp == 0) {
          st16(static_cast<char*>(a.K_w) + (hrow + victim) * S::ROW + sub * 16, cur.kn);
          st16(static_cast<char*>(a.V_w) + (hrow + victim) * S::ROW + sub * 16, cur.vn);
        }
      }
      if (lane == 0) a.evicted[head] = evicted;
    }
  };

  for (; head < G; head += gridDim.x) {
    load_head(cur, head);
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) acc[e] = 0.f;
    // Two batches in flight: B is issued before A is consumed, A before B.
    // Issues are unconditional so that every path through the loop has the
    // same loads outstanding (the wait counts stay exact); a batch past the
    // end re-reads the last occupied row, an L2 hit, and is masked out.
    if (nb > 0) {
      issue(kA, vA, head, 0);
      for (int b = 0; b < nb; b += 2) {
        // Fair share of the memory pipe between the waves of a SIMD: the
        // arbiter favours the oldest wave, which would stream its head first
        // and leave the others starved until the end. Priority falls as a
        // wave's progress rises, so lagging waves issue first.
        if constexpr (FAIR) set_wave_priority(3 - (4 * b) / nb);
        issue(kB, vB, head, b + 1);
        compute(kA, vA, b);
        issue(kA, vA, head, b + 2);
        compute(kB, vB, b + 1);
      }
    }
    epilogue();
  }
}


template <int DT, int D, bool SCORED>
hipError_t launch_typed(int G, const DecodeArgs& a, hipStream_t s) {
  const size_t shmem = SCORED ? size_t(a.k) * sizeof(float) : 0;
  constexpr int WMINW = 2;  // waves per SIMD the wave kernel is built for
  const int resident = cu_count() * 4 * WMINW;
  if (G >= resident / 2) {
    // 4 wave-loads per batch (two batches in flight): 2% faster than 8 at the
    // OPT-6.7B, OPT-30B and large-batch shapes.
    // Score/pos entries prefetched with the head's inputs: 4 per lane covers
    // 256 slots; larger caches take 8, so that the epilogue loads nothing
    // from HBM up to 512 slots (OPT-30B shape, 410 slots: 62.0 -> 61.4 us).
    constexpr int UB = 4;
    // With more heads than two waves per SIMD, the grid fills a third: the
    // scored kernel's 140-157 registers leave room for it, and one wave's
    // epilogue then overlaps the others' streams (large-batch layer, 8192
    // heads: 187.5 -> 185.5 us; a grid balanced to exactly three heads per
    // wave measured 188.6 us).
    const int grid = G < resident ? G : (SCORED ? (G < resident * 3 / 2 ? G : resident * 3 / 2) : resident);
    if (a.k > 256)
      hipLaunchKernelGGL((decode_wave_kernel<DT, D, UB, 8, WMINW, SCORED>), dim3(grid), dim3(64), shmem, s, a, G);
    else
      hipLaunchKernelGGL((decode_wave_kernel<DT, D, UB, 4, WMINW, SCORED>), dim3(grid), dim3(64), shmem, s, a, G);
  } else {
    // Few heads: spread each head over an 8-wave workgroup instead (two
    // waves per SIMD; against 4 waves: 32 heads x 2048 slots 33.5 -> 23.8 us,
    // 256 heads 46.5 -> 44.4 us; 16 waves is slower). With a workgroup per
    // CU or more, 4-deep batches are best; with fewer, each workgroup needs
    // the deeper batches to keep enough bytes in flight.
    constexpr int WAVES = 8, PF = 4, MINW = 2;
    if (G >= cu_count())
      hipLaunchKernelGGL((decode_kernel<DT, D, WAVES, 4, PF, MINW, SCORED>), dim3(G), dim3(WAVES * 64), shmem, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<DT, D, WAVES, 8, PF, MINW, SCORED>), dim3(G), dim3(WAVES * 64), shmem, s, a);
  }
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

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

hipError_t launch_decode(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s) {
  return dispatch<true>(dtype, head_dim, G, a, s);
}

hipError_t launch_fullcache(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s) {
  return dispatch<false>(dtype, head_dim, G, a, s);
}

}  // namespace h2o
