// H2O decode step over a cache stored as 8-, 4- or 2-bit codes, for gfx950.
//
// Citations ("H2O §x") refer to the page "H2O: Heavy-Hitter Oracle for
// Efficient Generative Inference of Large Language Models" (paperlayer.ai
// summary of arXiv 2306.14048v3); the code format (keys on per-channel grids,
// values on per-token grids) follows the KIVI abstract on the page
// "Discoveries (cursor 150)" and is described with h2o_quant in the C header.
//
// The step is the fused one of decode.hip (attention of the new token over
// the occupied slots and itself, H2O §D "Recursive attention"; accumulated
// scores, §1 and §B.2; at most one eviction outside the recent window, §2
// "Problem formulation", §D "Cache eviction"; insert into the freed slot),
// reading codes instead of rows. The grids fold into the arithmetic instead
// of being applied per element:
//   q.k_a   = sum_c q_c (s_c code_ac + mn_c) = sum_c (q_c s_c) code_ac + sum_c q_c mn_c,
//             so each head pre-scales q by the key grid once and adds one bias;
//   p_a v_a = (p_a s_a) code_a + (p_a mn_a) 1, so the P.V accumulator takes
//             p_a s_a per row and a separate sum of p_a mn_a.
// A row of d codes is read by d/16 lanes (16 codes, 2 * BITS bytes, each),
// one wave per head, persistent over heads, two batches of rows in flight as
// in the wave kernel of decode.hip (an 8-wave workgroup per head when there
// are few heads); narrower codes take more rows per batch.
// The new token's key and value are quantised on insert.

#include "h2o_device.h"
#include "lane_codes.h"
#include "launch.h"

namespace h2o {
namespace {

// 16 consecutive elements of a dtype row: raw 16-byte chunks, then fp32.
template <int DT> struct Raw16 {
  static constexpr int E = Elem<DT>::bytes, EPC = 16 / E, N = 16 / EPC;  // chunks of EPC elements
  uint4 w[N];
  __device__ __forceinline__ void load(const void* row, int first) {
    const char* p = static_cast<const char*>(row) + size_t(first) * E;
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = ld16(p + 16 * i);
  }
  __device__ __forceinline__ void unpack(float (&x)[16]) const {
#pragma unroll
    for (int i = 0; i < N; ++i) Unpack<DT>::run(w[i], x + EPC * i);
  }
};

// The softmax reference of a lane group moves only when a batch's maximum
// exceeds it by more than this (base 2; probabilities stay below 2^8), and
// the accumulators are rescaled only when some lane of the wave moved it,
// which after a head's first batches is rare. Numerator and normaliser share
// the reference, so the result is the same.
constexpr float kLazyRef = 8.0f;

// One wave per head.
//   BITS: code width; UB: wave-loads of codes (K and V, 128 * BITS bytes each)
//   per batch; PF: score/pos entries per lane prefetched with the head's inputs.
template <int DT, int D, int BITS, int UB, int PF>
__global__ __launch_bounds__(64, 2) void decode_quant_kernel(DecodeArgs a, int G) {
  using LC = LaneCodes<BITS>;
  using CT = typename LC::T;
  constexpr int LPR = D / 16;          // lanes per row of codes
  constexpr int RPU = 64 / LPR;        // rows per wave-wide load
  constexpr int RB = D * BITS / 8;     // bytes per code row
  constexpr int CB = 2 * BITS;         // code bytes per lane
  extern __shared__ float sm_logit[];  // [k] logits of the current head, base-2 units
  const int lane = threadIdx.x;
  const int grp = lane / LPR;
  const int sub = lane % LPR;
  const int c0 = sub * 16;  // this lane's channels
  const int nu = a.n_used;
  const int units = (nu + RPU - 1) / RPU;
  const int nb = (units + UB - 1) / UB;

  for (int head = blockIdx.x; head < G; head += gridDim.x) {
    const size_t hrow = size_t(head) * a.k;
    // ---- head inputs: q folded with the key grid, the new token, scores ---------------
    // Everything the epilogue needs is loaded here, so that no load sits on
    // the head's critical path after the stream.
    const size_t hoff = size_t(head) * D * Elem<DT>::bytes;
    Raw16<DT> q_raw, kn_raw, vn_raw;
    q_raw.load(static_cast<const char*>(a.q) + hoff, c0);
    kn_raw.load(static_cast<const char*>(a.k_new) + hoff, c0);
    vn_raw.load(static_cast<const char*>(a.v_new) + hoff, c0);
    const float4* kg4 = reinterpret_cast<const float4*>(a.k_qparam + size_t(head) * 2 * D + c0);
    float4 ks4[4], km4[4];  // this lane's key grids
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ks4[i] = kg4[i];
      km4[i] = kg4[D / 4 + i];
    }
    // The head's first batch of codes goes out right behind its inputs, so
    // that its latency overlaps the folding of q and the quantisation below.
    const uint8_t* Kh = static_cast<const uint8_t*>(a.K) + hrow * RB;
    const uint8_t* Vh = static_cast<const uint8_t*>(a.V) + hrow * RB;
    const float2* vg = reinterpret_cast<const float2*>(a.v_qparam) + hrow;
    // Loads are unconditional (rows past the occupied ones read as zeros,
    // range-checked by the buffer load, and are masked) so that the
    // compiler's wait counts stay exact: a conditional first batch makes it
    // wait for every load before the quantisation below. A batch's offsets
    // are one vector add from the lane's constant; each unit's is an
    // immediate on top.
    const auto Kr = rows_rsrc(Kh, nu * RB);
    const auto Vr = rows_rsrc(Vh, nu * RB);
    const auto Gr = rows_rsrc(vg, nu * 8);
    const uint32_t lane_off = uint32_t(grp * RB + sub * CB), lane_goff = uint32_t(grp * 8);
    auto issue = [&](CT (&kb)[UB], CT (&vb)[UB], float2 (&gb)[UB], int b) {
      const uint32_t off = lane_off + uint32_t(b * UB * RPU * RB), goff = lane_goff + uint32_t(b * UB * RPU * 8);
#pragma unroll
      for (int j = 0; j < UB; ++j) {
        kb[j] = LC::load(Kr, off + j * RPU * RB);
        vb[j] = LC::load(Vr, off + j * RPU * RB);
        gb[j] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(Gr, goff + j * RPU * 8, 0, 0));
      }
    };
    CT kA[UB], vA[UB], kB[UB], vB[UB];
    float2 gA[UB], gB[UB];
    issue(kA, vA, gA, 0);
    const float* ks = reinterpret_cast<const float*>(ks4);
    const float* km = reinterpret_cast<const float*>(km4);
    float qs[16];
    float bias;
    {
      float q[16];
      q_raw.unpack(q);
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        qs[i] = q[i] * ks[i] * a.c * LC::inv_weight(i);  // codes come weighted
        part = fmaf(q[i], km[i], part);
      }
      bias = group_sum<LPR>(part) * a.c;
    }
    // The new token's codes do not depend on the step's attention, only the
    // slot they go to does: quantise now, while the first rows are in flight
    // (32 correctly rounded divisions per lane off the epilogue's path).
    CT kn_codes, vn_codes;
    float vs, vmn;
    {
      float kn[16], vn[16];
      kn_raw.unpack(kn);
      vn_raw.unpack(vn);
      vmn = vn[0];
      float vmx = vn[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        vmn = fminf(vmn, vn[i]);
        vmx = fmaxf(vmx, vn[i]);
      }
      vmn = lane_group<LPR>(vmn, OpMin());
      vmx = lane_group<LPR>(vmx, OpMax());
      vs = grid_scale<BITS>(vmn, vmx);
      uint32_t kc[16], vc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        kc[i] = quantize_code<BITS>(kn[i], ks[i], km[i]);
        vc[i] = quantize_code<BITS>(vn[i], vs, vmn);
      }
      kn_codes = LC::pack(kc);
      vn_codes = LC::pack(vc);
    }
    float sc_pf[PF];
    int pos_pf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int slot = lane + 64 * i;
      sc_pf[i] = 0.f;
      pos_pf[i] = 0;
      if (slot < nu) {
        sc_pf[i] = a.score[hrow + slot];
        pos_pf[i] = a.pos[hrow + slot];
      }
    }

    // ---- stream the codes: per lane-group online softmax -------------------------------
    float m = kNegInf, l = 0.f, pm = 0.f;  // pm: sum of p * value-grid minimum
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    auto compute = [&](const CT (&kb)[UB], const CT (&vb)[UB], const float2 (&gb)[UB], int b) {
      float s[UB];
      float bm = kNegInf;
#pragma unroll
      for (int j = 0; j < UB; ++j) {
        const int row = (b * UB + j) * RPU + grp;
        float c[16];
        LC::to_float(kb[j], c);
        float x4[4] = {0.f, 0.f, 0.f, 0.f};  // four short chains instead of one long one
#pragma unroll
        for (int i = 0; i < 16; ++i) x4[i % 4] = fmaf(qs[i], c[i], x4[i % 4]);
        const float x = group_sum<LPR>((x4[0] + x4[1]) + (x4[2] + x4[3])) + bias;
        s[j] = row < nu ? x : kNegInf;
        bm = fmaxf(bm, s[j]);
        if (sub == 0 && row < nu) sm_logit[row] = s[j];
      }
      if (bm != kNegInf) {
        const bool raise = bm > m + kLazyRef;  // always on a group's first rows (m = -inf)
        if (__ballot(raise)) {
          const float mn = raise ? bm : m;
          const float alpha = fast_exp2(m - mn);
          l *= alpha;
          pm *= alpha;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[i] *= alpha;
          m = mn;
        }
#pragma unroll
        for (int j = 0; j < UB; ++j) {
          const float p = fast_exp2(s[j] - m);
          l += p;
          pm = fmaf(p, gb[j].y, pm);
          const float ps = p * gb[j].x;
          float c[16];
          LC::to_float(vb[j], c);
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[i] = fmaf(ps, c[i], acc[i]);
        }
      }
    };
    if (nb > 0) {
      for (int b = 0; b < nb; b += 2) {
        set_wave_priority(3 - (4 * b) / nb);  // lagging waves of a SIMD issue first
        issue(kB, vB, gB, b + 1);
        compute(kA, vA, gA, b);
        issue(kA, vA, gA, b + 2);
        compute(kB, vB, gB, b + 1);
      }
    }

    // ---- merge the lane groups, output -------------------------------------------------
    float qf[16], kn[16], vn[16];
    q_raw.unpack(qf);
    kn_raw.unpack(kn);
    vn_raw.unpack(vn);
    float sn = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sn = fmaf(qf[i], kn[i], sn);
    const float s_new = group_sum<LPR>(sn) * a.c;  // the new token at full precision
    const float M = fmaxf(across_groups<LPR>(m, OpMax()), s_new);
    const float w = fast_exp2(m - M);
    const float lw = across_groups<LPR>(l * w, OpAdd());
    const float pmw = across_groups<LPR>(pm * w, OpAdd());
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = across_groups<LPR>(acc[i] * (w * LC::inv_weight(i)), OpAdd());
    const float w_new = fast_exp2(s_new - M);
    const float invZ = 1.0f / (lw + w_new);
    if (grp == 0) {
      float* op = a.out + size_t(head) * D + c0;
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (acc[i + e] + pmw + w_new * vn[i + e]) * invZ;
        *reinterpret_cast<float4*>(op + i) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }

    // ---- accumulate scores, pick the victim ------------------------------------------
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

    // ---- insert the new token, quantised ---------------------------------------------
    if (victim >= 0 && victim < a.k) {
      if (lane == victim % 64) {
        sc_g[victim] = p_new;
        pos_g[victim] = a.t;
      }
      if (grp == 0) {
        LC::store(static_cast<uint8_t*>(a.K_w) + (hrow + victim) * RB + sub * CB, kn_codes);
        LC::store(static_cast<uint8_t*>(a.V_w) + (hrow + victim) * RB + sub * CB, vn_codes);
        if (sub == 0) reinterpret_cast<float2*>(a.v_qparam)[hrow + victim] = make_float2(vs, vmn);
      }
    }
    if (lane == 0) a.evicted[head] = evicted;
  }
}

// Few heads: one WAVES-wave workgroup per head. Wave w streams units w,
// w + WAVES, ... of the head's rows with the same per-lane-group online
// softmax as the wave kernel; each wave merges its lane groups, the waves'
// partials are merged through LDS, and all threads share the score update
// and the victim search (per-wave minima, then a minimum over the waves).
template <int DT, int D, int BITS, int WAVES, int UB, int PF>
__global__ __launch_bounds__(WAVES * 64, 2) void decode_quant_wg_kernel(DecodeArgs a) {
  using LC = LaneCodes<BITS>;
  using CT = typename LC::T;
  constexpr int LPR = D / 16;
  constexpr int RPU = 64 / LPR;
  constexpr int RB = D * BITS / 8;
  constexpr int CB = 2 * BITS;
  constexpr int NT = WAVES * 64;
  extern __shared__ float sm_logit[];  // [k] logits of the head, base-2 units
  __shared__ float sm_m[WAVES], sm_l[WAVES], sm_pm[WAVES];
  __shared__ __attribute__((aligned(16))) float sm_acc[WAVES][D];
  __shared__ uint64_t sm_key[WAVES];
  __shared__ int sm_slot[WAVES], sm_epos[WAVES];

  const int head = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPR, sub = lane % LPR;
  const int c0 = sub * 16;
  const int nu = a.n_used;
  const size_t hrow = size_t(head) * a.k;
  const size_t hoff = size_t(head) * D * Elem<DT>::bytes;

  // ---- head inputs: q folded with the key grid, the new token, scores -----------------
  Raw16<DT> q_raw, kn_raw, vn_raw;
  q_raw.load(static_cast<const char*>(a.q) + hoff, c0);
  kn_raw.load(static_cast<const char*>(a.k_new) + hoff, c0);
  vn_raw.load(static_cast<const char*>(a.v_new) + hoff, c0);
  const float4* kg4 = reinterpret_cast<const float4*>(a.k_qparam + size_t(head) * 2 * D + c0);
  float4 ks4[4], km4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ks4[i] = kg4[i];
    km4[i] = kg4[D / 4 + i];
  }
  const float* ks = reinterpret_cast<const float*>(ks4);
  const float* km = reinterpret_cast<const float*>(km4);
  float qs[16];
  float bias;
  {
    float q[16];
    q_raw.unpack(q);
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      qs[i] = q[i] * ks[i] * a.c * LC::inv_weight(i);  // codes come weighted
      part = fmaf(q[i], km[i], part);
    }
    bias = group_sum<LPR>(part) * a.c;
  }
  // Codes of the new token (only wave 0 writes them), computed while the
  // first rows are in flight.
  CT kn_codes{}, vn_codes{};
  float vs = 0.f, vmn = 0.f;
  if (wave == 0) {
    float kn[16], vn[16];
    kn_raw.unpack(kn);
    vn_raw.unpack(vn);
    vmn = vn[0];
    float vmx = vn[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      vmn = fminf(vmn, vn[i]);
      vmx = fmaxf(vmx, vn[i]);
    }
    vmn = lane_group<LPR>(vmn, OpMin());
    vmx = lane_group<LPR>(vmx, OpMax());
    vs = grid_scale<BITS>(vmn, vmx);
    uint32_t kc[16], vc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      kc[i] = quantize_code<BITS>(kn[i], ks[i], km[i]);
      vc[i] = quantize_code<BITS>(vn[i], vs, vmn);
    }
    kn_codes = LC::pack(kc);
    vn_codes = LC::pack(vc);
  }
  float sc_pf[PF];
  int pos_pf[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int slot = tid + NT * i;
    sc_pf[i] = 0.f;
    pos_pf[i] = 0;
    if (slot < nu) {
      sc_pf[i] = a.score[hrow + slot];
      pos_pf[i] = a.pos[hrow + slot];
    }
  }

  // ---- stream this wave's rows -------------------------------------------------------
  const uint8_t* Kh = static_cast<const uint8_t*>(a.K) + hrow * RB;
  const uint8_t* Vh = static_cast<const uint8_t*>(a.V) + hrow * RB;
  const float2* vg = reinterpret_cast<const float2*>(a.v_qparam) + hrow;
  float m = kNegInf, l = 0.f, pm = 0.f;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int units = (nu + RPU - 1) / RPU;
  const int nb = (units + WAVES * UB - 1) / (WAVES * UB);  // batches per wave
  auto row_of = [&](int b, int j) { return ((b * UB + j) * WAVES + wave) * RPU + grp; };
  // As in the wave kernel: the head's rows as buffer resources (rows past
  // the occupied ones read as zeros), one vector add per batch.
  const int lrow = wave * RPU + grp;  // the lane's row within a unit of WAVES waves
  const auto Kr = rows_rsrc(Kh, nu * RB);
  const auto Vr = rows_rsrc(Vh, nu * RB);
  const auto Gr = rows_rsrc(vg, nu * 8);
  const uint32_t lane_off = uint32_t(lrow * RB + sub * CB), lane_goff = uint32_t(lrow * 8);
  // 8- and 4-bit codes keep pointer loads clamped to the last occupied row:
  // at 256 heads x 2048 slots the buffer form measured 8 bits 27.38 -> 27.80
  // us and 4 bits 20.83 -> 21.32 us, against 2 bits 18.26 -> 17.35 us.
  constexpr bool kBufferRows = BITS == 2;
  auto issue = [&](CT (&kb)[UB], CT (&vb)[UB], float2 (&gb)[UB], int b) {
    const uint32_t off = lane_off + uint32_t(b * UB * WAVES * RPU * RB), goff = lane_goff + uint32_t(b * UB * WAVES * RPU * 8);
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      if constexpr (kBufferRows) {
        kb[j] = LC::load(Kr, off + j * WAVES * RPU * RB);
        vb[j] = LC::load(Vr, off + j * WAVES * RPU * RB);
        gb[j] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(Gr, goff + j * WAVES * RPU * 8, 0, 0));
      } else {
        const int row = min(row_of(b, j), nu - 1);
        kb[j] = LC::load(Kh + size_t(row) * RB + sub * CB);
        vb[j] = LC::load(Vh + size_t(row) * RB + sub * CB);
        gb[j] = vg[row];
      }
    }
  };
  auto compute = [&](const CT (&kb)[UB], const CT (&vb)[UB], const float2 (&gb)[UB], int b) {
    float s[UB];
    float bm = kNegInf;
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const int row = row_of(b, j);
      float c[16];
      LC::to_float(kb[j], c);
      float x4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) x4[i % 4] = fmaf(qs[i], c[i], x4[i % 4]);
      const float x = group_sum<LPR>((x4[0] + x4[1]) + (x4[2] + x4[3])) + bias;
      s[j] = row < nu ? x : kNegInf;
      bm = fmaxf(bm, s[j]);
      if (sub == 0 && row < nu) sm_logit[row] = s[j];
    }
    if (bm != kNegInf) {
      const bool raise = bm > m + kLazyRef;  // always on a group's first rows (m = -inf)
      if (__ballot(raise)) {
        const float mn = raise ? bm : m;
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
        pm *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] *= alpha;
        m = mn;
      }
#pragma unroll
      for (int j = 0; j < UB; ++j) {
        const float p = fast_exp2(s[j] - m);
        l += p;
        pm = fmaf(p, gb[j].y, pm);
        const float ps = p * gb[j].x;
        float c[16];
        LC::to_float(vb[j], c);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = fmaf(ps, c[i], acc[i]);
      }
    }
  };
  if (nu > 0) {
    CT kA[UB], vA[UB], kB[UB], vB[UB];
    float2 gA[UB], gB[UB];
    issue(kA, vA, gA, 0);
    for (int b = 0; b < nb; b += 2) {
      issue(kB, vB, gB, b + 1);
      compute(kA, vA, gA, b);
      issue(kA, vA, gA, b + 2);
      compute(kB, vB, gB, b + 1);
    }
  }

  // ---- merge: lane groups inside the wave, then the waves through LDS -----------------
  float qf[16], kn[16], vn[16];
  q_raw.unpack(qf);
  kn_raw.unpack(kn);
  vn_raw.unpack(vn);
  float sn = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sn = fmaf(qf[i], kn[i], sn);
  const float s_new = group_sum<LPR>(sn) * a.c;  // the new token at full precision
  // Every wave's reference includes s_new, so it is finite even for a wave
  // that streamed no occupied row.
  const float Mw = fmaxf(across_groups<LPR>(m, OpMax()), s_new);
  const float w = fast_exp2(m - Mw);
  const float lw = across_groups<LPR>(l * w, OpAdd());
  const float pmw = across_groups<LPR>(pm * w, OpAdd());
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = across_groups<LPR>(acc[i] * (w * LC::inv_weight(i)), OpAdd());
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<float4*>(&sm_acc[wave][c0 + i]) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  }
  if (lane == 0) {
    sm_m[wave] = Mw;
    sm_l[wave] = lw;
    sm_pm[wave] = pmw;
  }
  __syncthreads();
  float M = sm_m[0];
#pragma unroll
  for (int v = 1; v < WAVES; ++v) M = fmaxf(M, sm_m[v]);
  float f[WAVES];
  float Z = 0.f, PM = 0.f;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) {
    f[v] = fast_exp2(sm_m[v] - M);
    Z = fmaf(sm_l[v], f[v], Z);
    PM = fmaf(sm_pm[v], f[v], PM);
  }
  const float w_new = fast_exp2(s_new - M);
  const float invZ = 1.0f / (Z + w_new);
  if (wave == 0 && grp == 0) {
    float* op = a.out + size_t(head) * D + c0;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = 0.f;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) x = fmaf(sm_acc[v][c0 + i + e], f[v], x);
        o[e] = (x + PM + w_new * vn[i + e]) * invZ;
      }
      *reinterpret_cast<float4*>(op + i) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }

  // ---- accumulate scores, pick the victim ----------------------------------------------
  const float p_new = w_new * invZ;
  const bool full = nu == a.k;
  const int lim = a.t - a.k_recent;
  float* sc_g = a.score + hrow;
  int32_t* pos_g = a.pos + hrow;
  uint64_t best = ~0ull;
  int best_slot = -1, best_pos = -1;
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int slot = tid + NT * i;
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
  for (int slot = tid + NT * PF; slot < nu; slot += NT) {
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
  int victim = nu;
  int evicted = -1;
  if (full) {
    const uint64_t gmin = wave_min_u64(best);
    // Keys are unique (positions are), so at most one lane holds the minimum.
    const uint64_t owners = __ballot(best == gmin && gmin != ~0ull);
    if (lane == 0) {
      sm_key[wave] = gmin;
      sm_slot[wave] = -1;
      sm_epos[wave] = -2;
    }
    if (owners) {
      const int owner = __ffsll((unsigned long long)owners) - 1;
      const int vslot = __builtin_amdgcn_readlane(best_slot, owner);
      const int vpos = __builtin_amdgcn_readlane(best_pos, owner);
      if (lane == 0) {
        sm_slot[wave] = vslot;
        sm_epos[wave] = vpos;
      }
    }
  }
  __syncthreads();
  if (full) {
    uint64_t k_best = sm_key[0];
    int vb = 0;
#pragma unroll
    for (int v = 1; v < WAVES; ++v)
      if (sm_key[v] < k_best) {
        k_best = sm_key[v];
        vb = v;
      }
    // A full cache always has an eligible candidate; if the caller's state
    // broke that invariant nothing is written and -2 is reported.
    victim = k_best == ~0ull ? -1 : sm_slot[vb];
    evicted = k_best == ~0ull ? -2 : sm_epos[vb];
  }

  // ---- insert the new token, quantised ---------------------------------------------------
  if (victim >= 0 && victim < a.k) {
    if (tid == victim % NT) {
      sc_g[victim] = p_new;
      pos_g[victim] = a.t;
    }
    if (wave == 0 && grp == 0) {
      LC::store(static_cast<uint8_t*>(a.K_w) + (hrow + victim) * RB + sub * CB, kn_codes);
      LC::store(static_cast<uint8_t*>(a.V_w) + (hrow + victim) * RB + sub * CB, vn_codes);
      if (sub == 0) reinterpret_cast<float2*>(a.v_qparam)[hrow + victim] = make_float2(vs, vmn);
    }
  }
  if (tid == 0) a.evicted[head] = evicted;
}

template <int DT, int D, int BITS>
hipError_t launch_typed(int G, const DecodeArgs& a, hipStream_t s) {
  // K and V codes per batch: 2 KiB at 8 and 4 bits (2 or 4 wave-loads), 1 KiB
  // at 2 bits (4 wave-loads; 8 would spill registers).
  constexpr int UB = BITS == 8 ? 2 : 4, PF = 4, MINW = 2;
  const int resident = cu_count() * 4 * MINW;
  const size_t shmem = size_t(a.k) * sizeof(float);
  if (G >= resident / 2) {
    const int grid = G < resident ? G : resident;
    hipLaunchKernelGGL((decode_quant_kernel<DT, D, BITS, UB, PF>), dim3(grid), dim3(64), shmem, s, a, G);
  } else {
    // Few heads: an 8-wave workgroup per head, as for caches of rows.
    constexpr int WAVES = 8;
    hipLaunchKernelGGL((decode_quant_wg_kernel<DT, D, BITS, WAVES, UB, PF>), dim3(G), dim3(WAVES * 64), shmem, s,
                       a);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t dispatch(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s) {
  switch (dtype * 1000 + head_dim) {
    case DT_F32 * 1000 + 64: return launch_typed<DT_F32, 64, BITS>(G, a, s);
    case DT_F32 * 1000 + 128: return launch_typed<DT_F32, 128, BITS>(G, a, s);
    case DT_BF16 * 1000 + 64: return launch_typed<DT_BF16, 64, BITS>(G, a, s);
    case DT_BF16 * 1000 + 128: return launch_typed<DT_BF16, 128, BITS>(G, a, s);
    case DT_F16 * 1000 + 64: return launch_typed<DT_F16, 64, BITS>(G, a, s);
    case DT_F16 * 1000 + 128: return launch_typed<DT_F16, 128, BITS>(G, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_quant(int bits, int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s) {
  if (G <= 0) return hipSuccess;
  switch (bits) {
    case 8: return dispatch<8>(dtype, head_dim, G, a, s);
    case 4: return dispatch<4>(dtype, head_dim, G, a, s);
    case 2: return dispatch<2>(dtype, head_dim, G, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace h2o
