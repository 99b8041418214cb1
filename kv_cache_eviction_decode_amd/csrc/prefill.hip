// H2O prefill scoring and selection for gfx950.
//
// Citations ("H2O §x") refer to the page "H2O: Heavy-Hitter Oracle for
// Efficient Generative Inference of Large Language Models" (paperlayer.ai
// summary of arXiv 2306.14048v3).
//
// For every (batch, head) the prompt's causal attention matrix P (row i is a
// softmax over keys j <= i, H2O §D "Recursive attention") is reduced to its
// column sums c_j, the accumulated attention each prompt token receives
// (H2O §1, §4.1). c needs each row's final normaliser, so QK^T is formed
// twice, both times on MFMA (v_mfma_f32_32x32x16_{bf16,f16}), with the operand
// shared by a workgroup staged through LDS:
//
//   pass 1 (rowlse):  lse2_i = log2 sum_j 2^(c * s_ij), keys streamed per query
//                     block; the tile is computed transposed (keys x queries)
//                     so each lane owns one query column and reduces in-lane.
//   pass 2 (colsum):  c_j = sum_i 2^(c * s_ij - lse2_i), queries streamed per key
//                     block; each workgroup owns its key columns, so the sums
//                     need no atomics and are deterministic.
//
// Then one workgroup per head selects the k_heavy largest (c_j, j) among
// positions before the recent window with an MSB-first radix select on the
// score bits, compacts them in ascending position order together with the
// recent window (H2O §A "Pseudocode", "System Details") and copies the K/V
// rows into the cache slots.

#include <type_traits>

#include "../../include/h2o.h"
#include "h2o_device.h"
#include "launch.h"
#include "prefill_launch.h"

namespace h2o {
namespace {

// Blocks are dispatched round-robin over the 8 XCDs. Remap so that XCD x runs
// a contiguous range of logical blocks (the same heads), keeping each head's
// K and Q tiles in one XCD's L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int grid) {
  const int per = grid >> 3;  // grid is padded to a multiple of 8
  return (bid & 7) * per + (bid >> 3);
}

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data
// format, no swizzle): untyped loads, range-checked against the record count.
constexpr int kBufferWord3 = 0x00020000;

template <int DT> struct MfmaOp;
template <> struct MfmaOp<DT_BF16> {
  __device__ __forceinline__ static f32x16 run(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct MfmaOp<DT_F16> {
  __device__ __forceinline__ static f32x16 run(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// 32x32x16 MFMA operand/result layout (wave64): lane l supplies row (l % 32)
// of A and column (l % 32) of B, each with the 8 contiguous k values
// 8*(l/32) .. 8*(l/32)+7. Result element j (0..15) of lane l is
// D[8*(j/4) + 4*(l/32) + j%4][l % 32].
__device__ __forceinline__ int mfma_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

// ---------------------------------------------------------------- LDS-staged passes
// Both passes form 64x64 score tiles per wave per iteration (4 accumulators of
// 32x32, 32 MFMAs). The operand that the NW waves of a workgroup share (K
// rows in pass 1, Q rows in pass 2) is staged through LDS in 64-row tiles:
// each thread fetches its share of the next tile into registers while the
// current tile is consumed, then writes it to the other LDS buffer (one
// barrier per tile). Rows are padded by 16 bytes in LDS so that the 32 rows one MFMA
// operand read touches fall into distinct banks.
template <int DT, int D, int NW = 4>
struct Tile64 {
  static constexpr int E = Elem<DT>::bytes;
  static constexpr int ROW = D * E;       // bytes per row in global memory
  static constexpr int CH = ROW / 16;     // 16-byte chunks per row
  static constexpr int RS = ROW + 16;     // padded LDS row stride
  static constexpr int BYTES = 64 * RS;   // one 64-row tile
  static constexpr int CPT = CH / NW;     // chunks per thread (NW waves, 64 rows)
  static constexpr int RPI = 64 / CH;     // rows one wave-wide 16-byte access covers
  static constexpr int KS = D / 16;       // MFMA k-steps per row
  static_assert(CPT >= 1, "tile too small for the workgroup");

  // Thread (wave w, lane l) moves chunk l % CH of rows (64/NW)w + i*RPI + l / CH:
  // each wave-wide access is 1 KiB of consecutive rows in global memory, and
  // consecutive lanes write consecutive 16-byte chunks of one LDS row (no
  // bank conflicts).
  __device__ __forceinline__ static int my_row(int i) {
    return (threadIdx.x >> 6) * (64 / NW) + i * RPI + (threadIdx.x & 63) / CH;
  }
  __device__ __forceinline__ static int my_chunk() { return (threadIdx.x & 63) % CH; }

  // A head's n rows as a buffer resource: loads past row n - 1 return zeros
  // (range-checked by the load itself), so tiles need no clamping.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rows(const char* head_base, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(head_base), 0, n * ROW, kBufferWord3);
  }
  // Fetch rows [r0, r0 + 64) of `src` into registers (zeros past the end).
  __device__ __forceinline__ static void fetch(uint4 (&r)[CPT], __amdgpu_buffer_rsrc_t src, int r0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t off = uint32_t((r0 + my_row(i)) * ROW + my_chunk() * 16);
      r[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, 0));
    }
  }
  __device__ __forceinline__ static void store(char* lds, const uint4 (&r)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *reinterpret_cast<uint4*>(lds + my_row(i) * RS + my_chunk() * 16) = r[i];
  }
  // MFMA operand fragment: row (32*blk + lane%32), k-step ks.
  __device__ __forceinline__ static uint4 frag(const char* lds, int blk, int ks, int lane) {
    return *reinterpret_cast<const uint4*>(lds + (blk * 32 + (lane & 31)) * RS + (ks * 2 + (lane >> 5)) * 16);
  }
};

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Wait for every outstanding vector-memory load. Used once, after the
// register-resident MFMA operands are loaded: without it the wait-count pass
// cannot tell at the tile loop's header that those loads are done and waits
// for the next tile's prefetch inside the MFMA chain, exposing its latency.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Block pairing of the causal passes. Workgroup pr (0 <= pr < (nblk + 1) / 2)
// takes the block with the (pr+1)-th longest causal extent, nblk - 1 - pr,
// and then the block returned here (-1: none). Block b spans b + 1 block
// lengths of keys. With an even count the partner of nblk - 1 - pr is pr,
// and each workgroup spans nblk + 1; with an odd count the longest block
// runs alone and the rest pair as (nblk - 1 - pr, pr - 1), each pair
// spanning nblk, the longest block's extent.
__device__ __forceinline__ int pair_partner(int nblk, int pr) { return (nblk & 1) ? pr - 1 : pr; }

// Pass 1: lse2_i = log2 sum_{j<=i} 2^(c*s_ij). Workgroup = 64 * NW queries (64
// per wave); keys streamed in 64-row LDS tiles. The transposed tile (keys x
// queries) gives each lane one query column, so the row statistics are
// in-lane until the final merge of the two lane halves.
//
// Each lane keeps a reference r (log2 domain) and l = sum 2^(c*s - r). r is
// the maximum of the first tile the lane sees, and stays fixed while a
// tile's partial sum stays below 2^64 (every term below 2^58 of the
// reference): then a score costs one FMA, one exp2 and one add, with no
// max. A tile whose sum overflows that bound, or the first tile, takes the
// exact path instead: tile maximum, rescale of l, new reference. The sum is
// the same up to fp32 rounding whatever the reference, since fp32 keeps its
// relative precision over the whole range involved.
//
// Key tiles below the workgroup's first query are visible to all of its
// queries and run without the causal mask; only the last NW tiles (the
// diagonal) test positions, and there a wave skips the MFMAs and the exp
// work of every 32x32 quarter that lies wholly above the diagonal.
template <int DT, int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void rowlse_lds(PrefillArgs a, int nblk, int G, int ld_lse, int paired) {
  using T = Tile64<DT, D, NW>;
  constexpr int QBLK = 64 * NW;  // queries per workgroup
  __shared__ __attribute__((aligned(16))) char lds[2][T::BYTES];
  const int per_head = paired ? (nblk + 1) / 2 : nblk;
  const int L = xcd_logical_block(blockIdx.x, gridDim.x);
  if (L >= G * per_head) return;  // uniform over the workgroup
  const int head = L / per_head;
  const int pr = L % per_head;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lh = lane >> 5;
  const int n = a.n;
  const char* Qh = static_cast<const char*>(a.Q) + size_t(head) * n * T::ROW;
  const char* Kh = static_cast<const char*>(a.K) + size_t(head) * n * T::ROW;
  const auto Kr = T::rows(Kh, n);
  const float c = a.c;

  // Paired: query block nblk - 1 - pr, then block pair_partner(pr): the two
  // causal extents add up to that of the longest block (odd count) or to
  // one block more (even count), so every workgroup carries the same work.
  // Otherwise block nblk - 1 - pr alone (longest causal extent first).
  for (int seg = 0; seg < 2; ++seg) {
    const int qb = seg == 0 ? nblk - 1 - pr : pair_partner(nblk, pr);
    if (seg == 1 && (!paired || qb < 0)) break;
    const int wg_q0 = qb * QBLK;
    // The wave's 64 queries are two 32-row halves of the block, w and
    // 2NW - 1 - w: on the causal diagonal every wave then sees the same
    // number of keys, so no wave waits at the tile barrier while another
    // finishes a longer diagonal.
    const int qh[2] = {wg_q0 + 32 * wave, wg_q0 + 32 * (2 * NW - 1 - wave)};

    // The first key tile is fetched together with the query fragments, so the
    // prologue waits for one memory latency, not two.
    uint4 nx[T::CPT];
    T::fetch(nx, Kr, 0);
    uint4 qf[2][T::KS];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = min(qh[cb] + (lane & 31), n - 1);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) qf[cb][ks] = ld16(Qh + size_t(r) * T::ROW + (ks * 16 + lh * 8) * T::E);
    }
    wait_vmem_all();
    float ref[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
    const int ntiles = min(wg_q0 + QBLK - 1, n - 1) / 64 + 1;
    const int nfull = min(wg_q0 / 64, ntiles);  // tiles with every key <= the workgroup's first query
    T::store(lds[0], nx);
    __syncthreads();

    // Adds half cb's scores of the tile (both 32-key halves, or the first
    // only when the second lies wholly past the queries).
    auto accumulate = [&](const f32x16 (&acc)[2][2], int cb, auto both_halves) {
      constexpr bool BOTH = decltype(both_halves)::value;
      const float nr = -ref[cb];
      float t0 = 0.f, t1 = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        t0 += fast_exp2(fmaf(acc[0][cb][j], c, nr));
        if constexpr (BOTH) t1 += fast_exp2(fmaf(acc[1][cb][j], c, nr));
      }
      const float t = t0 + t1;
      if (t <= 0x1p64f) {
        l[cb] += t;
      } else {  // first tile (reference -inf), or a score far above the reference; also NaN
        float tm = kNegInf;
#pragma unroll
        for (int j = 0; j < 16; j += 2) tm = max3f(tm, acc[0][cb][j], acc[0][cb][j + 1]);
        if constexpr (BOTH) {
#pragma unroll
          for (int j = 0; j < 16; j += 2) tm = max3f(tm, acc[1][cb][j], acc[1][cb][j + 1]);
        }
        const float rn = fmaxf(ref[cb], tm * c);
        if (rn != kNegInf) {
          float u0 = 0.f, u1 = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            u0 += fast_exp2(fmaf(acc[0][cb][j], c, -rn));
            if constexpr (BOTH) u1 += fast_exp2(fmaf(acc[1][cb][j], c, -rn));
          }
          l[cb] = fmaf(l[cb], fast_exp2(ref[cb] - rn), u0 + u1);
          ref[cb] = rn;
        }
      }
    };

    auto step = [&](int kt, auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
      if (kt + 1 < ntiles) T::fetch(nx, Kr, (kt + 1) * 64);
      const char* buf = lds[kt & 1];
      const int key0 = kt * 64;
      // vis[kb][cb]: the 32 keys key0 + 32kb.. reach some query of half cb
      // (past the prompt's end a half has no queries). The second query half
      // lies after the first, so vis[kb][0] implies vis[kb][1], and the
      // second key half lies after the first, so vis[1][cb] implies vis[0][cb].
      bool vis[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) vis[kb][cb] = !MASKED || key0 + 32 * kb <= min(qh[cb] + 31, n - 1);
      // The MFMA chain issues at raised priority, so that while this wave
      // feeds the matrix unit the other wave of the SIMD fills the gaps with
      // its exp/sum work instead of delaying the chain (long prompts: 5%).
      __builtin_amdgcn_s_setprio(1);
      f32x16 acc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!vis[kb][0] && !vis[kb][1]) continue;
        uint4 af[T::KS];
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) af[ks] = T::frag(buf, kb, ks, lane);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          if (!vis[kb][cb]) continue;
          acc[kb][cb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < T::KS; ++ks) acc[kb][cb] = MfmaOp<DT>::run(af[ks], qf[cb][ks], acc[kb][cb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // acc[kb][cb][j] = s(query qh[cb] + lane%32, key key0 + 32kb + mfma_row(j))
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if (!vis[0][cb]) continue;
        if constexpr (MASKED) {
          // Keys and query halves are 32-aligned, so a quarter is cut by the
          // diagonal only when it starts at the half's first query.
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (vis[kb][cb] && key0 + 32 * kb == qh[cb]) {
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (mfma_row(j, lane) > (lane & 31)) acc[kb][cb][j] = kNegInf;
            }
        }
        if (vis[1][cb])
          accumulate(acc, cb, std::true_type{});
        else
          accumulate(acc, cb, std::false_type{});
      }
      if (kt + 1 < ntiles) T::store(lds[(kt + 1) & 1], nx);
      __syncthreads();
    };
    for (int kt = 0; kt < nfull; ++kt) step(kt, std::false_type{});
    for (int kt = nfull; kt < ntiles; ++kt) step(kt, std::true_type{});
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float ro = __shfl_xor(ref[cb], 32);
      const float lo = __shfl_xor(l[cb], 32);
      const float M = fmaxf(ref[cb], ro);
      const float Lsum = l[cb] * fast_exp2(ref[cb] - M) + lo * fast_exp2(ro - M);
      const int qi = qh[cb] + (lane & 31);
      if (lh == 0 && qi < n) a.lse2[size_t(head) * ld_lse + qi] = M + fast_log2(Lsum);
    }
  }
}

// ---------------------------------------------------------------- pass 1 with output
// Eight probabilities as one 16-byte MFMA operand of the input type.
template <int DT> __device__ __forceinline__ uint4 pack8(const float* p);
template <> __device__ __forceinline__ uint4 pack8<DT_BF16>(const float* p) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)p[i];
  return __builtin_bit_cast(uint4, v);
}
template <> __device__ __forceinline__ uint4 pack8<DT_F16>(const float* p) {
  f16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (_Float16)p[i];
  return __builtin_bit_cast(uint4, v);
}

// Pass 1 emitting the prompt's own attention output O = P V as well as
// lse2 (H2O §D "Recursive attention": o_i together with its normaliser D_i).
// The S^T tiles are those of rowlse_lds; the probabilities of a 16-key group
// held by a lane are exactly the 8 k values the lane supplies as the B
// operand of O^T = V^T P^T (k slot 8h+i <-> key 16g + 8(i/4) + 4h + i%4), so P
// never leaves registers; V^T comes from a transposed LDS tile. The softmax
// keeps one reference per query column, shared by both lane halves (their
// probabilities meet in one P.V output column): as in rowlse_lds, the first
// tile's maximum, kept while the tile's sum over both halves stays below
// 2^64 (2^15 for fp16 inputs, whose P operand must stay finite in fp16), so
// no maximum is taken per tile. A tile beyond that bound (or the
// first) takes the exact path for its queries, and the O accumulators are
// rescaled only when some lane of the wave did, which after the first tiles
// is rare. Numerator and denominator share the reference, so the result is
// exact up to rounding.

// Workgroup of NWV waves (8, or 4 for short prompts) of 32 queries sharing
// the K and V tiles of 32 NWV queries: a wave's O accumulators (d x 32), S
// tile and query fragments fit in half the register file, so two waves run
// per SIMD and the softmax of one overlaps the other's MFMAs (64 queries per
// wave at one wave per SIMD ran 1.4x slower). V is staged in LDS as it is in memory (key rows) and its
// MFMA A operands (channel rows) are read with gfx950's transposing LDS
// read; a V tile transposed while staging took 2-byte LDS writes that
// collided on banks.
template <int DT, int D, int NWV>
struct VTile8 {
  using T = Tile64<DT, D, NWV>;
  static constexpr int RS = T::ROW + 32;  // bytes per key row: 4 consecutive rows fall 8 banks apart
  static constexpr int BYTES = 64 * RS;
  __device__ __forceinline__ static void store(char* lds, const uint4 (&r)[T::CPT]) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i)
      *reinterpret_cast<uint4*>(lds + T::my_row(i) * RS + T::my_chunk() * 16) = r[i];
  }
  // A operand of the P.V MFMA for 32-channel block db and 16-key group g:
  // channel 32db + lane%32, keys 16g + 4h + {0..3} then 16g + 8 + 4h + {0..3}
  // (h = lane/32). The transposing LDS read gives lane i of each 16-lane group
  // element i%4 of the 8-byte rows read by lanes i/4, i/4 + 4, i/4 + 8 and
  // i/4 + 12 of the group, so lane s reads key row 16g + 4h + s/4 (+8) at
  // channel 32db + 16 * (group % 2) + 4 * (s % 4).
  __device__ __forceinline__ static uint4 frag(const char* lds, int db, int g, int lane) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const int s = lane & 15;
    const int row = 16 * g + 4 * (lane >> 5) + (s >> 2);
    const int ch = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const char* p = lds + row * RS + ch * 2;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 8 * RS));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return make_uint4(l2.x, l2.y, h2.x, h2.y);
  }
};

template <int DT, int D, int NWV>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void rowattn8_lds(PrefillArgs a, int nblk, int G, int ld_lse, int paired) {
  using T = Tile64<DT, D, NWV>;
  using VT = VTile8<DT, D, NWV>;
  constexpr int QBLK = 32 * NWV;  // queries per workgroup
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) char lds_k[2][T::BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v[2][VT::BYTES];
  const int per_head = paired ? (nblk + 1) / 2 : nblk;
  const int L = xcd_logical_block(blockIdx.x, gridDim.x);
  if (L >= G * per_head) return;  // uniform over the workgroup
  const int head = L / per_head;
  const int pr = L % per_head;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lh = lane >> 5;
  const int n = a.n;
  const char* Qh = static_cast<const char*>(a.Q) + size_t(head) * n * T::ROW;
  const char* Kh = static_cast<const char*>(a.K) + size_t(head) * n * T::ROW;
  const char* Vh = static_cast<const char*>(a.V) + size_t(head) * n * T::ROW;
  const auto Kr = T::rows(Kh, n);
  const auto Vr = T::rows(Vh, n);
  const float c = a.c;

  // Blocks nblk - 1 - pr and pair_partner(pr) in turn when paired (as in
  // rowlse_lds), else block nblk - 1 - pr alone (longest causal extent first).
  for (int seg = 0; seg < 2; ++seg) {
    const int qb = seg == 0 ? nblk - 1 - pr : pair_partner(nblk, pr);
    if (seg == 1 && (!paired || qb < 0)) break;
    const int wg_q0 = qb * QBLK;
    const int q0 = wg_q0 + wave * 32;

    // The first key and value tiles are fetched together with the query
    // fragments (one memory latency in the prologue, not two).
    uint4 nk[T::CPT], nv[T::CPT];
    T::fetch(nk, Kr, 0);
    T::fetch(nv, Vr, 0);
    uint4 qf[T::KS];
    {
      const int r = min(q0 + (lane & 31), n - 1);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) qf[ks] = ld16(Qh + size_t(r) * T::ROW + (ks * 16 + lh * 8) * T::E);
    }
    wait_vmem_all();
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float ref = kNegInf, l = 0.f;
    const int ntiles = min(wg_q0 + QBLK - 1, n - 1) / 64 + 1;
    T::store(lds_k[0], nk);
    VT::store(lds_v[0], nv);
    __syncthreads();
    const int qi = q0 + (lane & 31);
    // Key tiles below the workgroup's first query need no causal mask.
    const int nfull = min(wg_q0 / 64, ntiles);
    auto step = [&](int kt, auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
      if (kt + 1 < ntiles) {
        T::fetch(nk, Kr, (kt + 1) * 64);
        T::fetch(nv, Vr, (kt + 1) * 64);
      }
      const char* kbuf = lds_k[kt & 1];
      const char* vbuf = lds_v[kt & 1];
      const int key0 = kt * 64;
      if (!MASKED || key0 <= min(q0 + 31, n - 1)) {  // every query of this wave sees key0
        f32x16 acc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          acc[kb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < T::KS; ++ks) acc[kb] = MfmaOp<DT>::run(T::frag(kbuf, kb, ks, lane), qf[ks], acc[kb]);
        }
        // acc[kb][j] = s(query qi, key key0 + 32kb + mfma_row(j))
        if constexpr (MASKED) {
          if (key0 + 63 > q0) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (key0 + kb * 32 + mfma_row(j, lane) > qi) acc[kb][j] = kNegInf;
          }
        }
        // Probabilities against the query's reference (base 2, shared by the
        // two lane halves that hold the query's keys).
        float p[2][16];
        float t = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            p[kb][j] = fast_exp2(fmaf(acc[kb][j], c, -ref));
            t += p[kb][j];
          }
        // P feeds the MFMA in the input type: fp16 must stay below its 65504
        // limit, bf16 has fp32's range.
        constexpr float kBound = DT == DT_F16 ? 0x1p15f : 0x1p64f;
        const bool redo = !(t + __shfl_xor(t, 32) <= kBound);  // first tile, far above, or NaN
        if (__ballot(redo)) {
          float tm = kNegInf;
#pragma unroll
          for (int j = 0; j < 16; j += 2) tm = max3f(tm, acc[0][j], acc[0][j + 1]);
#pragma unroll
          for (int j = 0; j < 16; j += 2) tm = max3f(tm, acc[1][j], acc[1][j + 1]);
          const float tmax = fmaxf(tm, __shfl_xor(tm, 32)) * c;
          float rn = redo ? fmaxf(ref, tmax) : ref;
          if (rn == kNegInf) rn = 0.f;  // no visible key yet: nothing to scale
          const float alpha = fast_exp2(ref - rn);  // 1 where the reference stays
          if (redo) {
            t = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int j = 0; j < 16; ++j) {
                p[kb][j] = fast_exp2(fmaf(acc[kb][j], c, -rn));
                t += p[kb][j];
              }
          }
          l *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db] *= alpha;
          ref = rn;
        }
        l += t;
        uint4 pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          pb[kb][0] = pack8<DT>(p[kb]);
          pb[kb][1] = pack8<DT>(p[kb] + 8);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              o[db] = MfmaOp<DT>::run(VT::frag(vbuf, db, kb * 2 + g, lane), pb[kb][g], o[db]);
      }
      if (kt + 1 < ntiles) {
        T::store(lds_k[(kt + 1) & 1], nk);
        VT::store(lds_v[(kt + 1) & 1], nv);
      }
      __syncthreads();
    };
    for (int kt = 0; kt < nfull; ++kt) step(kt, std::false_type{});
    for (int kt = nfull; kt < ntiles; ++kt) step(kt, std::true_type{});
    const float lt = l + __shfl_xor(l, 32);  // both halves share the reference maximum
    if (qi < n) {
      const float lse2 = ref + fast_log2(lt);
      if (lh == 0) {
        a.lse2[size_t(head) * ld_lse + qi] = lse2;
        if (a.lse_out) a.lse_out[size_t(head) * n + qi] = lse2 * 0.6931471805599453f;
      }
      const float inv = 1.0f / lt;
      float* orow = a.out + (size_t(head) * n + qi) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<float4*>(orow + db * 32 + 8 * jj + 4 * lh) =
              make_float4(o[db][4 * jj] * inv, o[db][4 * jj + 1] * inv, o[db][4 * jj + 2] * inv, o[db][4 * jj + 3] * inv);
    }
  }
}

// Pass 2: c_j = sum_{i>=j} 2^(c*s_ij - lse2_i). Workgroup = 64 * NW keys (64
// per wave, held in registers as MFMA B operands); queries streamed in 64-row LDS
// tiles together with their lse2. Each lane owns one key column; the tile
// partial of 32 values is added with compensation. On the first NW query
// tiles (the diagonal) a wave skips every 32x32 quarter whose queries all
// precede its keys.
template <int DT, int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void colsum_lds(PrefillArgs a, int nblk, int G, int ld_lse, int paired) {
  using T = Tile64<DT, D, NW>;
  constexpr int KBLK = 64 * NW;  // keys per workgroup
  __shared__ __attribute__((aligned(16))) char lds[2][T::BYTES];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][64];
  const int per_head = paired ? (nblk + 1) / 2 : nblk;
  const int L = xcd_logical_block(blockIdx.x, gridDim.x);
  if (L >= G * per_head) return;
  const int head = L / per_head;
  const int pr = L % per_head;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lh = lane >> 5;
  const int n = a.n;
  const char* Qh = static_cast<const char*>(a.Q) + size_t(head) * n * T::ROW;
  const char* Kh = static_cast<const char*>(a.K) + size_t(head) * n * T::ROW;
  const auto Qr = T::rows(Qh, n);
  const float* lse = a.lse2 + size_t(head) * ld_lse;
  const float c = a.c;

  // Paired: key block pr, then block nblk - 1 - pair_partner(pr) (the same
  // total number of query tiles for every workgroup, as for the query blocks
  // of rowlse_lds). Otherwise block pr alone (most query tiles first).
  for (int seg = 0; seg < 2; ++seg) {
    const int partner = pair_partner(nblk, pr);
    const int kblk = seg == 0 ? pr : nblk - 1 - partner;
    if (seg == 1 && (!paired || partner < 0)) break;
    const int wg_k0 = kblk * KBLK;
    // The wave's 64 keys are two 32-row halves of the block, w and
    // 2NW - 1 - w, so that on the causal diagonal every wave sees the same
    // number of queries (as the query halves of rowlse_lds).
    const int kh[2] = {wg_k0 + 32 * wave, wg_k0 + 32 * (2 * NW - 1 - wave)};

    const int t0 = wg_k0 / 64;
    const int ntiles = (n + 63) / 64;
    uint4 nx[T::CPT];
    float nl = 0.f;
    // Rows past the prompt get lse = +inf, so their terms are exp2(-inf) = 0
    // without a per-element test.
    auto fetch = [&](int qt) {
      T::fetch(nx, Qr, qt * 64);
      if (threadIdx.x < 64) {
        const int q = qt * 64 + threadIdx.x;
        nl = q < n ? lse[q] : __builtin_huge_valf();
      }
    };
    auto store = [&](int buf) {
      T::store(lds[buf], nx);
      if (threadIdx.x < 64) lds_lse[buf][threadIdx.x] = nl;
    };
    // The first query tile is fetched together with the key fragments, so the
    // prologue waits for one memory latency, not two.
    fetch(t0);
    uint4 kf[2][T::KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = min(kh[kb] + (lane & 31), n - 1);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) kf[kb][ks] = ld16(Kh + size_t(r) * T::ROW + (ks * 16 + lh * 8) * T::E);
    }
    wait_vmem_all();
    float sum[2] = {0.f, 0.f}, comp[2] = {0.f, 0.f};
    store(0);
    __syncthreads();
    auto step = [&](int qt, auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
      const int cur = (qt - t0) & 1;
      if (qt + 1 < ntiles) fetch(qt + 1);
      const int qrow0 = qt * 64;
      // vis[qb][kb]: some query of the 32 from qrow0 + 32qb sees a key of
      // half kb (a half wholly past the prompt's end sees none). Later query
      // halves see more, so vis[0][kb] implies vis[1][kb]; the second key
      // half lies after the first, so vis[qb][1] implies vis[qb][0].
      bool vis[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) vis[qb][kb] = !MASKED || (kh[kb] < n && qrow0 + 32 * qb + 31 >= kh[kb]);
      const char* buf = lds[cur];
      __builtin_amdgcn_s_setprio(1);  // as in rowlse_lds (neutral here, kept for symmetry)
      f32x16 acc[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (!vis[qb][0] && !vis[qb][1]) continue;
        uint4 af[T::KS];
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) af[ks] = T::frag(buf, qb, ks, lane);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (!vis[qb][kb]) continue;
          acc[qb][kb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < T::KS; ++ks) acc[qb][kb] = MfmaOp<DT>::run(af[ks], kf[kb][ks], acc[qb][kb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // acc[qb][kb][j] = s(query qrow0 + 32qb + mfma_row(j), key kh[kb] + lane%32)
      float lq[2][16];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float4 v = *reinterpret_cast<const float4*>(&lds_lse[cur][qb * 32 + 8 * jj + 4 * lh]);
          lq[qb][4 * jj] = v.x;
          lq[qb][4 * jj + 1] = v.y;
          lq[qb][4 * jj + 2] = v.z;
          lq[qb][4 * jj + 3] = v.w;
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!vis[1][kb]) continue;
        if constexpr (MASKED) {
          // 32-aligned halves: a quarter is cut by the diagonal only when
          // its queries start at the key half's first key.
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            if (vis[qb][kb] && qrow0 + 32 * qb == kh[kb]) {
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (mfma_row(j, lane) < (lane & 31)) acc[qb][kb][j] = kNegInf;
            }
        }
        float t = 0.f, t2 = 0.f;
        if (vis[0][kb]) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            t += fast_exp2(fmaf(acc[0][kb][j], c, -lq[0][j]));
            t2 += fast_exp2(fmaf(acc[1][kb][j], c, -lq[1][j]));
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) t2 += fast_exp2(fmaf(acc[1][kb][j], c, -lq[1][j]));
        }
        t += t2;
        const float y = t - comp[kb];
        const float s2 = sum[kb] + y;
        comp[kb] = (s2 - sum[kb]) - y;
        sum[kb] = s2;
      }
      if (qt + 1 < ntiles) store(cur ^ 1);
      __syncthreads();
    };
    // Query tiles [t0, t0 + NW) hold the diagonal of some wave of the
    // workgroup; every later tile is visible to all of its keys.
    const int tdiag = min(t0 + NW, ntiles);
    for (int qt = t0; qt < tdiag; ++qt) step(qt, std::true_type{});
    for (int qt = tdiag; qt < ntiles; ++qt) step(qt, std::false_type{});
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float mine = sum[kb] - comp[kb];
      const float other = __shfl_xor(mine, 32);
      const int kj = kh[kb] + (lane & 31);
      if (lh == 0 && kj < n) a.colsum[size_t(head) * n + kj] = mine + other;
    }
  }
}

// ---------------------------------------------------------------- fp32 (VALU)
// fp32 operands run on the vector ALU. A workgroup of 256 lanes owns 64 rows of
// one head (queries in the row passes, keys in the column pass): the four lanes
// of a quad share a row, lane s holding float4 columns s, s+4, s+8, ... of it in
// registers. The other operand streams through LDS 32 rows at a time, fetched
// into registers one tile ahead. For a group of four streamed rows, lane s
// forms the partial dot product of its columns with row (r ^ s) as its r-th
// value; two quad swaps then leave lane s holding the full score against row s
// of the group, so every score is finished in exactly one lane and the softmax
// arithmetic is not repeated across the quad.
constexpr int kF32Threads = 256;
constexpr int kF32Rows = kF32Threads / 4;  // rows owned by a workgroup
constexpr int kF32Tile = 32;               // streamed rows per LDS tile
// Heads x prompt rows from which the column pass and the row pass without
// output give each quad two rows (1024 two-row workgroups fill the chip).
constexpr int64_t kF32TwoRowsMin = int64_t(1024) * 2 * kF32Rows;

template <int D> struct F32Layout {
  static constexpr int C4 = D / 16;                   // float4 columns per lane
  static constexpr int TILE4 = kF32Tile * D / 4;      // float4 per LDS tile
  static constexpr int LOADS = TILE4 / kF32Threads;   // float4 per lane per tile
  static_assert(TILE4 % kF32Threads == 0, "tile must split evenly over the workgroup");
};

// One lane's columns of row r of a [n][D] matrix (zeros past n).
template <int D>
__device__ __forceinline__ void f32_row(float4 (&x)[F32Layout<D>::C4], const float* X, int r, int n, int s) {
  const float4* row = reinterpret_cast<const float4*>(X + size_t(r) * D);
#pragma unroll
  for (int m = 0; m < F32Layout<D>::C4; ++m) x[m] = r < n ? row[4 * m + s] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Streamed rows [r0, r0 + kF32Tile) of a [n][D] matrix into registers, zeros past n.
template <int D>
__device__ __forceinline__ void f32_fetch(float4 (&buf)[F32Layout<D>::LOADS], const float* X, int r0, int n) {
#pragma unroll
  for (int l = 0; l < F32Layout<D>::LOADS; ++l) {
    const int idx = threadIdx.x + l * kF32Threads, r = r0 + idx / (D / 4);
    buf[l] = r < n ? reinterpret_cast<const float4*>(X + size_t(r) * D)[idx % (D / 4)]
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int D>
__device__ __forceinline__ void f32_store(float4* tile, const float4 (&buf)[F32Layout<D>::LOADS]) {
#pragma unroll
  for (int l = 0; l < F32Layout<D>::LOADS; ++l) tile[threadIdx.x + l * kF32Threads] = buf[l];
}

__device__ __forceinline__ float dot4(float4 x, float4 y, float acc) {
  return fmaf(x.w, y.w, fmaf(x.z, y.z, fmaf(x.y, y.y, fmaf(x.x, y.x, acc))));
}

// Lane s of each quad: dot product of the quad's row with streamed row 4g + s.
template <int D>
__device__ __forceinline__ float quad_score(const float4 (&x)[F32Layout<D>::C4], const float4* tile, int g, int s) {
  float u[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float4* row = tile + (4 * g + (r ^ s)) * (D / 4) + s;
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < F32Layout<D>::C4; ++m) acc = dot4(x[m], row[4 * m], acc);
    u[r] = acc;
  }
  const float k0 = u[0] + dpp<kQuadSwap1>(u[1]);  // rows s and s ^ 2, two lanes each
  const float k1 = u[2] + dpp<kQuadSwap1>(u[3]);
  return k0 + dpp<kQuadSwap2>(k1);
}

__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  return fmaxf(x, dpp<kQuadSwap2>(x));
}

// Value of lane R of the quad, in every lane of it.
template <int R> __device__ __forceinline__ float quad_bcast(float x) { return dpp<R * 0x55>(x); }

// R query rows per quad (rows r, r + 64, ...): each streamed float4 read from
// LDS then feeds 4R FMAs, for prompts long enough to keep the chip busy with
// 64R-row workgroups. All scores of a tile in one pass: lane s gets, for each
// of its R rows, the score against streamed row 4g + s in out[h][g]. The
// next streamed row's reads are issued ahead of the current row's FMAs in
// program order (two register buffers); pinning that order with a scheduling
// barrier raised the register count to two waves per SIMD and was 8% slower.
template <int D, int R>
__device__ __forceinline__ void tile_scores(const float4 (&x)[R][F32Layout<D>::C4], const float4* tile, int s,
                                            float (&out)[R][kF32Tile / 4]) {
  constexpr int C4 = F32Layout<D>::C4;
  constexpr int NR = kF32Tile;  // (group, r) pairs per tile
  float4 y[2][C4];
  auto load = [&](float4 (&dst)[C4], int gr) {
    const float4* row = tile + (4 * (gr >> 2) + ((gr & 3) ^ s)) * (D / 4) + s;
#pragma unroll
    for (int m = 0; m < C4; ++m) dst[m] = row[4 * m];
  };
  load(y[0], 0);
  float u[R][4];
#pragma unroll
  for (int gr = 0; gr < NR; ++gr) {
    if (gr + 1 < NR) load(y[(gr + 1) & 1], gr + 1);
    const int r = gr & 3;
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < C4; ++m) acc = dot4(x[h][m], y[gr & 1][m], acc);
      u[h][r] = acc;
    }
    if (r == 3) {
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float k0 = u[h][0] + dpp<kQuadSwap1>(u[h][1]);  // rows s and s ^ 2, two lanes each
        const float k1 = u[h][2] + dpp<kQuadSwap1>(u[h][3]);
        out[h][gr >> 2] = k0 + dpp<kQuadSwap2>(k1);
      }
    }
  }
}

// Pass 1, fp32: per-row log2-sum-exp2 of the scaled causal scores.
template <int D, int R>
__global__ __launch_bounds__(kF32Threads) void rowlse_f32(PrefillArgs a, int nblk, int ld_lse, int paired) {
  using L = F32Layout<D>;
  constexpr int ROWS = R * kF32Rows;  // query rows per workgroup
  __shared__ float4 tile[L::TILE4];
  const int per_head = paired ? (nblk + 1) / 2 : nblk;
  const int head = blockIdx.x / per_head;
  const int pr = blockIdx.x % per_head;
  const int n = a.n, s = threadIdx.x & 3;
  const float* Q = static_cast<const float*>(a.Q) + size_t(head) * n * D;
  const float* K = static_cast<const float*>(a.K) + size_t(head) * n * D;
  const float c = a.c;
  // Row blocks nblk - 1 - pr, then pair_partner(pr) when paired (as in
  // rowlse_lds); unpaired, the longest rows first.
  for (int seg = 0; seg < 2; ++seg) {
    const int qb = seg == 0 ? nblk - 1 - pr : pair_partner(nblk, pr);
    if (seg == 1 && (!paired || qb < 0)) break;
    const int i0 = qb * ROWS + (threadIdx.x >> 2);  // rows i0 + h * kF32Rows
    float4 q[R][L::C4];
#pragma unroll
    for (int h = 0; h < R; ++h) f32_row<D>(q[h], Q, i0 + h * kF32Rows, n, s);
    const int ntiles = (min(n, (qb + 1) * ROWS) + kF32Tile - 1) / kF32Tile;
    float4 buf[L::LOADS];
    f32_fetch<D>(buf, K, 0, n);
    float m[R], l[R];
#pragma unroll
    for (int h = 0; h < R; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
    }
    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();
      f32_store<D>(tile, buf);
      __syncthreads();
      if (t + 1 < ntiles) f32_fetch<D>(buf, K, (t + 1) * kF32Tile, n);
      float sc[R][kF32Tile / 4];
      tile_scores<D, R>(q, tile, s, sc);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int g = 0; g < kF32Tile / 4; ++g) sc[h][g] *= c;
      if (t * kF32Tile + kF32Tile - 1 > qb * ROWS) {
#pragma unroll
        for (int h = 0; h < R; ++h)
#pragma unroll
          for (int g = 0; g < kF32Tile / 4; ++g)
            if (t * kF32Tile + 4 * g + s > i0 + h * kF32Rows) sc[h][g] = kNegInf;
      }
#pragma unroll
      for (int h = 0; h < R; ++h) {
        float mt = sc[h][0];
#pragma unroll
        for (int g = 1; g < kF32Tile / 4; ++g) mt = fmaxf(mt, sc[h][g]);
        const float mn = fmaxf(m[h], mt), ms = mn == kNegInf ? 0.f : mn;
        float p = 0.f;
#pragma unroll
        for (int g = 0; g < kF32Tile / 4; ++g) p += fast_exp2(sc[h][g] - ms);
        l[h] = fmaf(l[h], fast_exp2(m[h] - ms), p);
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const int i = i0 + h * kF32Rows;
      const float M = quad_max(m[h]);  // finite: key i lies in the row of lane i % 4
      const float total = group_sum<4>(l[h] * fast_exp2(m[h] - M));
      if (s == 0 && i < n) a.lse2[size_t(head) * ld_lse + i] = M + fast_log2(total);
    }
  }
}

// Pass 1 with output, fp32: the quad keeps one running maximum so that its
// four lanes can accumulate their columns of the output row together.
template <int D>
__global__ __launch_bounds__(kF32Threads) void rowattn_f32(PrefillArgs a, int nblk, int ld_lse, int paired) {
  using L = F32Layout<D>;
  __shared__ float4 ktile[L::TILE4];
  __shared__ float4 vtile[L::TILE4];
  const int per_head = paired ? (nblk + 1) / 2 : nblk;
  const int head = blockIdx.x / per_head;
  const int pr = blockIdx.x % per_head;
  const int n = a.n, s = threadIdx.x & 3;
  const float* Q = static_cast<const float*>(a.Q) + size_t(head) * n * D;
  const float* K = static_cast<const float*>(a.K) + size_t(head) * n * D;
  const float* V = static_cast<const float*>(a.V) + size_t(head) * n * D;
  const float c = a.c;
  for (int seg = 0; seg < 2; ++seg) {  // row blocks as in rowlse_f32
    const int qb = seg == 0 ? nblk - 1 - pr : pair_partner(nblk, pr);
    if (seg == 1 && (!paired || qb < 0)) break;
    const int i = qb * kF32Rows + (threadIdx.x >> 2);
    float4 q[L::C4], o[L::C4];
    f32_row<D>(q, Q, i, n, s);
#pragma unroll
    for (int e = 0; e < L::C4; ++e) o[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int ntiles = (min(n, (qb + 1) * kF32Rows) + kF32Tile - 1) / kF32Tile;
    float4 kbuf[L::LOADS], vbuf[L::LOADS];
    f32_fetch<D>(kbuf, K, 0, n);
    f32_fetch<D>(vbuf, V, 0, n);
    float m = kNegInf, l = 0.f;
    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();
      f32_store<D>(ktile, kbuf);
      f32_store<D>(vtile, vbuf);
      __syncthreads();
      if (t + 1 < ntiles) {
        f32_fetch<D>(kbuf, K, (t + 1) * kF32Tile, n);
        f32_fetch<D>(vbuf, V, (t + 1) * kF32Tile, n);
      }
      float sc[kF32Tile / 4];
#pragma unroll
      for (int g = 0; g < kF32Tile / 4; ++g) sc[g] = quad_score<D>(q, ktile, g, s) * c;
      if (t * kF32Tile + kF32Tile - 1 > qb * kF32Rows) {
#pragma unroll
        for (int g = 0; g < kF32Tile / 4; ++g)
          if (t * kF32Tile + 4 * g + s > i) sc[g] = kNegInf;
      }
      float mt = sc[0];
#pragma unroll
      for (int g = 1; g < kF32Tile / 4; ++g) mt = fmaxf(mt, sc[g]);
      const float mn = fmaxf(m, quad_max(mt)), ms = mn == kNegInf ? 0.f : mn;
      const float alpha = fast_exp2(m - ms);
      float psum = 0.f;
#pragma unroll
      for (int g = 0; g < kF32Tile / 4; ++g) {
        sc[g] = fast_exp2(sc[g] - ms);
        psum += sc[g];
      }
      l = fmaf(l, alpha, psum);
#pragma unroll
      for (int e = 0; e < L::C4; ++e) {
        o[e].x *= alpha;
        o[e].y *= alpha;
        o[e].z *= alpha;
        o[e].w *= alpha;
      }
#pragma unroll
      for (int g = 0; g < kF32Tile / 4; ++g) {
        const float p[4] = {quad_bcast<0>(sc[g]), quad_bcast<1>(sc[g]), quad_bcast<2>(sc[g]), quad_bcast<3>(sc[g])};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4* row = vtile + (4 * g + r) * (D / 4) + s;
#pragma unroll
          for (int e = 0; e < L::C4; ++e) {
            const float4 y = row[4 * e];
            o[e].x = fmaf(p[r], y.x, o[e].x);
            o[e].y = fmaf(p[r], y.y, o[e].y);
            o[e].z = fmaf(p[r], y.z, o[e].z);
            o[e].w = fmaf(p[r], y.w, o[e].w);
          }
        }
      }
      m = mn;
    }
    const float total = group_sum<4>(l);
    if (i < n) {  // no early return: the next row block's tiles need every thread at the barriers
      const float lse2 = m + fast_log2(total);
      if (s == 0) {
        a.lse2[size_t(head) * ld_lse + i] = lse2;
        if (a.lse_out) a.lse_out[size_t(head) * n + i] = lse2 * 0.6931471805599453f;
      }
      const float inv = 1.0f / total;
      float4* orow = reinterpret_cast<float4*>(a.out + (size_t(head) * n + i) * D);
#pragma unroll
      for (int e = 0; e < L::C4; ++e) orow[4 * e + s] = make_float4(o[e].x * inv, o[e].y * inv, o[e].z * inv, o[e].w * inv);
    }
  }
}

// Pass 1 replaced by the caller's natural-log normalisers: lse2 = lse * log2(e).
__global__ void lse_from_natural(PrefillArgs a, int G, int ld_lse) {
  const int64_t total = int64_t(G) * a.n;
  for (int64_t x = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; x < total; x += int64_t(gridDim.x) * blockDim.x) {
    const int64_t g = x / a.n, i = x % a.n;
    a.lse2[g * ld_lse + i] = a.lse_in[x] * kLog2e;
  }
}

// Pass 2, fp32: a workgroup owns 64R keys (R per quad: keys j, j + 64, ...)
// and streams the queries at and after its first key, with their
// normalisers, through LDS.
template <int D, int R>
__global__ __launch_bounds__(kF32Threads) void colsum_f32(PrefillArgs a, int nblk, int ld_lse, int paired) {
  using L = F32Layout<D>;
  constexpr int ROWS = R * kF32Rows;  // keys per workgroup
  __shared__ float4 tile[L::TILE4];
  __shared__ float ltile[kF32Tile];
  const int per_head = paired ? (nblk + 1) / 2 : nblk;
  const int head = blockIdx.x / per_head;
  const int pr = blockIdx.x % per_head;
  const int n = a.n, s = threadIdx.x & 3;
  const float* Q = static_cast<const float*>(a.Q) + size_t(head) * n * D;
  const float* K = static_cast<const float*>(a.K) + size_t(head) * n * D;
  const float* lse = a.lse2 + size_t(head) * ld_lse;
  const float c = a.c;
  // Key block pr (block 0 streams the most queries), then, when paired,
  // block nblk - 1 - pair_partner(pr) (as in colsum_lds).
  for (int seg = 0; seg < 2; ++seg) {
    const int partner = pair_partner(nblk, pr);
    const int kb = seg == 0 ? pr : nblk - 1 - partner;
    if (seg == 1 && (!paired || partner < 0)) break;
    const int k0 = kb * ROWS, j0 = k0 + (threadIdx.x >> 2);  // keys j0 + h * kF32Rows
    float4 kr[R][L::C4];
#pragma unroll
    for (int h = 0; h < R; ++h) f32_row<D>(kr[h], K, j0 + h * kF32Rows, n, s);
    const int t0 = k0 / kF32Tile, ntiles = (n + kF32Tile - 1) / kF32Tile;
    float4 buf[L::LOADS];
    f32_fetch<D>(buf, Q, t0 * kF32Tile, n);
    const int lr = threadIdx.x < kF32Tile ? t0 * kF32Tile + threadIdx.x : n;
    float lbuf = lr < n ? lse[lr] : 0.f;
    float sum[R], comp[R];
#pragma unroll
    for (int h = 0; h < R; ++h) {
      sum[h] = 0.f;
      comp[h] = 0.f;
    }
    for (int t = t0; t < ntiles; ++t) {
      __syncthreads();
      f32_store<D>(tile, buf);
      if (threadIdx.x < kF32Tile) ltile[threadIdx.x] = lbuf;
      __syncthreads();
      if (t + 1 < ntiles) {
        f32_fetch<D>(buf, Q, (t + 1) * kF32Tile, n);
        const int r = threadIdx.x < kF32Tile ? (t + 1) * kF32Tile + threadIdx.x : n;
        lbuf = r < n ? lse[r] : 0.f;
      }
      const bool edge = t * kF32Tile < k0 + ROWS || (t + 1) * kF32Tile > n;
      float sc[R][kF32Tile / 4];
      tile_scores<D, R>(kr, tile, s, sc);
#pragma unroll
      for (int g = 0; g < kF32Tile / 4; ++g) {
        float v[R];
#pragma unroll
        for (int h = 0; h < R; ++h) v[h] = sc[h][g];
        const float lq = ltile[4 * g + s];
        const int qi = t * kF32Tile + 4 * g + s;
#pragma unroll
        for (int h = 0; h < R; ++h) {
          float p = fast_exp2(fmaf(v[h], c, -lq));
          if (edge && (qi < j0 + h * kF32Rows || qi >= n)) p = 0.f;
          const float y = p - comp[h];
          const float u = sum[h] + y;
          comp[h] = (u - sum[h]) - y;
          sum[h] = u;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const int j = j0 + h * kF32Rows;
      const float total = group_sum<4>(sum[h] - comp[h]);
      if (s == 0 && j < n) a.colsum[size_t(head) * n + j] = total;
    }
  }
}

// ---------------------------------------------------------------- select + gather
// 512 threads, the slot list sized to k in dynamic LDS (1 KiB at k = 256):
// several heads' workgroups share a CU. Against 1024 threads and a list sized
// for the largest cache: prompt 1024 prefill 1.04 -> 1.01 ms, 1920 2.38 ->
// 2.35 ms, 16384 unchanged (256 threads: 1% slower there).
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;

__device__ int block_exclusive_scan(int v, int* sm_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sm_wave[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = sm_wave[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// N consecutive BITS-wide codes (the first channel a multiple of 8 / BITS),
// packed low bits first into N * BITS / 8 bytes (1 to 8).
template <int N, int BITS> __device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t (&c)[N]) {
  static_assert((N == 4 || N == 8) && (BITS == 8 || BITS == 4 || BITS == 2), "4 or 8 codes of 8, 4 or 2 bits");
  uint64_t w = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) w |= uint64_t(c[i]) << (BITS * i);
  constexpr int bytes = N * BITS / 8;
  if constexpr (bytes == 8) *reinterpret_cast<uint2*>(p) = make_uint2(uint32_t(w), uint32_t(w >> 32));
  else if constexpr (bytes == 4) *reinterpret_cast<uint32_t*>(p) = uint32_t(w);
  else if constexpr (bytes == 2) *reinterpret_cast<uint16_t*>(p) = uint16_t(w);
  else *p = uint8_t(w);
}

// BITS = 0: the cache holds rows in the input dtype; 8, 4, 2: packed codes.
template <int DT, int D, int BITS>
__global__ __launch_bounds__(kSelThreads) void select_gather(PrefillArgs a) {
  constexpr int E = Elem<DT>::bytes, ROW = D * E, LPR = ROW / 16;
  extern __shared__ int slot_pos[];  // [k]
  __shared__ int hist[256];
  __shared__ int sm_wave[kSelWaves];
  __shared__ int sm_digit, sm_above, sm_P;

  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = a.n, kh = a.k_heavy, kr = a.k_recent, k = kh + kr;
  const float* col = a.colsum + size_t(head) * n;
  // Retention value of candidate j at the last prompt row, as float bits
  // (monotone: values are >= 0). Accumulated: c_j; averaged: c_j / (n - j).
  auto vbits = [&](int j) -> uint32_t {
    const float c = col[j];
    return __float_as_uint(a.policy == POLICY_AVERAGED ? c / float(n - j) : c);
  };

  if (n <= k) {
    for (int s = tid; s < k; s += kSelThreads) slot_pos[s] = s < n ? s : -1;
  } else if (a.policy == POLICY_POSITION) {
    // The earliest positions are the most valuable: they are the sinks.
    for (int s = tid; s < kh; s += kSelThreads) slot_pos[s] = s;
    for (int s = tid; s < kr; s += kSelThreads) slot_pos[kh + s] = n - kr + s;
  } else {
    const int C = n - kr;  // heavy-hitter candidates: positions [0, C)
    uint32_t T = 0;
    int P = C;
    if (kh > 0) {
      uint32_t prefix = 0, pmask = 0;
      int need = kh;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < C; j += kSelThreads) {
          const uint32_t b = vbits(j);
          if ((b & pmask) == prefix) atomicAdd(&hist[(b >> shift) & 255], 1);
        }
        __syncthreads();
        // digit d scanned from the top: v = hist[255 - tid]
        const int v = tid < 256 ? hist[255 - tid] : 0;
        int tot;
        const int above = block_exclusive_scan(v, sm_wave, tot);
        if (tid < 256 && above < need && above + v >= need) {
          sm_digit = 255 - tid;
          sm_above = above;
        }
        __syncthreads();
        need -= sm_above;
        prefix |= uint32_t(sm_digit) << shift;
        pmask |= 255u << shift;
        __syncthreads();
      }
      T = prefix;
      // Ties at T: keep the `need` of them with the largest positions.
      int taken = 0;
      for (int base = ((C - 1) / kSelThreads) * kSelThreads; base >= 0; base -= kSelThreads) {
        const int j = base + tid;
        const int tie = (j < C && vbits(j) == T) ? 1 : 0;
        int tot;
        const int below = block_exclusive_scan(tie, sm_wave, tot);
        const int above = tot - below - tie;  // ties in this chunk after j
        if (tie && taken + above == need - 1) sm_P = j;
        __syncthreads();
        if (taken + tot >= need) break;
        taken += tot;
      }
      P = sm_P;
    }
    // Compact the selected candidates in ascending position order.
    int base_slot = 0;
    for (int base = 0; base < C; base += kSelThreads) {
      const int j = base + tid;
      int sel = 0;
      if (kh > 0 && j < C) {
        const uint32_t b = vbits(j);
        sel = (b > T || (b == T && j >= P)) ? 1 : 0;
      }
      int tot;
      const int off = block_exclusive_scan(sel, sm_wave, tot);
      if (sel && base_slot + off < kh) slot_pos[base_slot + off] = j;
      base_slot += tot;
    }
    for (int s = tid; s < kr; s += kSelThreads) slot_pos[kh + s] = n - kr + s;
  }
  __syncthreads();

  const size_t hk = size_t(head) * k;
  for (int s = tid; s < k; s += kSelThreads) {
    const int p = slot_pos[s];
    a.cpos[hk + s] = p;
    a.cscore[hk + s] = p >= 0 ? col[p] : 0.f;
  }
  const int filled = min(n, k);
  const int sub = tid % LPR;
  const char* Kp = static_cast<const char*>(a.K) + size_t(head) * n * ROW + sub * 16;
  const char* Vp = static_cast<const char*>(a.V) + size_t(head) * n * ROW + sub * 16;
  if constexpr (BITS > 0) {
    // Codes: each lane quantises its EPL elements of the row; keys on the
    // head's channel grids, values on the row's own grid.
    constexpr int EPL = 16 / E;
    constexpr int RB = D * BITS / 8;          // bytes per code row
    constexpr int LB = EPL * BITS / 8;        // code bytes per lane
    const float* kg = a.kq_param + size_t(head) * 2 * D + sub * EPL;
    float ks[EPL], km[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      ks[e] = kg[e];
      km[e] = kg[D + e];
    }
    uint8_t* cK = static_cast<uint8_t*>(a.cK) + hk * RB + sub * LB;
    uint8_t* cV = static_cast<uint8_t*>(a.cV) + hk * RB + sub * LB;
    for (int s = tid / LPR; s < filled; s += kSelThreads / LPR) {
      const int p = slot_pos[s];
      if (p < 0 || p >= n) continue;  // cannot happen for a consistent selection
      const size_t src = size_t(p) * ROW;
      float x[EPL], v[EPL];
      Unpack<DT>::run(ldnt16(Kp + src), x);
      Unpack<DT>::run(ldnt16(Vp + src), v);
      uint32_t kc[EPL], vc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) kc[e] = quantize_code<BITS>(x[e], ks[e], km[e]);
      float vmn = v[0], vmx = v[0];
#pragma unroll
      for (int e = 1; e < EPL; ++e) {
        vmn = fminf(vmn, v[e]);
        vmx = fmaxf(vmx, v[e]);
      }
      vmn = lane_group<LPR>(vmn, OpMin());
      vmx = lane_group<LPR>(vmx, OpMax());
      const float vs = grid_scale<BITS>(vmn, vmx);
#pragma unroll
      for (int e = 0; e < EPL; ++e) vc[e] = quantize_code<BITS>(v[e], vs, vmn);
      store_codes<EPL, BITS>(cK + size_t(s) * RB, kc);
      store_codes<EPL, BITS>(cV + size_t(s) * RB, vc);
      if (sub == 0) *reinterpret_cast<float2*>(a.vq_param + (hk + s) * 2) = make_float2(vs, vmn);
    }
  } else {
    char* cK = static_cast<char*>(a.cK) + hk * ROW + sub * 16;
    char* cV = static_cast<char*>(a.cV) + hk * ROW + sub * 16;
    for (int s = tid / LPR; s < filled; s += kSelThreads / LPR) {
      const int p = slot_pos[s];
      if (p < 0 || p >= n) continue;  // cannot happen for a consistent selection
      const size_t src = size_t(p) * ROW;
      st16(cK + size_t(s) * ROW, ldnt16(Kp + src));
      st16(cV + size_t(s) * ROW, ldnt16(Vp + src));
    }
  }
}

// Key grids of a cache stored as BITS-wide codes: per (head, channel), the
// smallest and largest prompt key, scale = (mx - mn) / (2^BITS - 1). One
// workgroup per head.
template <int DT, int D, int BITS>
__global__ __launch_bounds__(256) void key_grid(PrefillArgs a) {
  constexpr int E = Elem<DT>::bytes, ROW = D * E, LPR = ROW / 16, EPL = 16 / E, RPP = 256 / LPR;
  __shared__ float sm_mn[RPP][D + 1];
  __shared__ float sm_mx[RPP][D + 1];
  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int sub = tid % LPR, r = tid / LPR;
  const char* Kp = static_cast<const char*>(a.K) + size_t(head) * a.n * ROW + sub * 16;
  float mn[EPL], mx[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    mn[e] = __builtin_huge_valf();
    mx[e] = -__builtin_huge_valf();
  }
  for (int j = r; j < a.n; j += RPP) {
    float x[EPL];
    Unpack<DT>::run(ld16(Kp + size_t(j) * ROW), x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      mn[e] = fminf(mn[e], x[e]);
      mx[e] = fmaxf(mx[e], x[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    sm_mn[r][sub * EPL + e] = mn[e];
    sm_mx[r][sub * EPL + e] = mx[e];
  }
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    float lo = sm_mn[0][c], hi = sm_mx[0][c];
    for (int i = 1; i < RPP; ++i) {
      lo = fminf(lo, sm_mn[i][c]);
      hi = fmaxf(hi, sm_mx[i][c]);
    }
    float* kg = a.kq_param + size_t(head) * 2 * D;
    kg[c] = grid_scale<BITS>(lo, hi);
    kg[D + c] = lo;
  }
}

__global__ void cache_clear(float* score, int32_t* pos, int64_t count) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * blockDim.x) {
    score[i] = 0.f;
    pos[i] = -1;
  }
}

int pad8(int x) { return (x + 7) & ~7; }

// Whether the prefill passes pair a head's blocks in one workgroup (see
// pair_partner): every workgroup then carries the same work (scoring, prompt
// 1024: 1.00-1.04 -> 0.93-0.95 ms; 1536: -7%; 2048: -4%; 4096: -5%; with the
// prompt's attention output, 1024: -9%, 2048: -7%, 4096: -4%).
int pair_blocks(int nblk) { return nblk >= 2 ? 1 : 0; }

template <int DT, int D>
hipError_t prefill_typed(int G, const PrefillArgs& a, hipStream_t s) {
  const int ld_lse = (a.n + 63) & ~63;
  if (a.pass1 == PASS1_GIVEN) {
    int64_t blocks = (int64_t(G) * a.n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(lse_from_natural, dim3(unsigned(blocks)), dim3(256), 0, s, a, G, ld_lse);
  }
  if constexpr (DT == DT_F32) {
    const int nblk = (a.n + kF32Rows - 1) / kF32Rows;
    // Two rows per quad once the prompt gives every CU several 128-row
    // workgroups; below that, one row keeps the workgroup count up.
    const bool two = int64_t(G) * a.n >= kF32TwoRowsMin;
    const int nblk2 = (a.n + 2 * kF32Rows - 1) / (2 * kF32Rows);
    const int p1 = pair_blocks(nblk), p2 = pair_blocks(nblk2);
    const int wg1 = p1 ? (nblk + 1) / 2 : nblk, wg2 = p2 ? (nblk2 + 1) / 2 : nblk2;  // workgroups per head
    if (a.pass1 == PASS1_LSE) {
      if (two)
        hipLaunchKernelGGL((rowlse_f32<D, 2>), dim3(G * wg2), dim3(kF32Threads), 0, s, a, nblk2, ld_lse, p2);
      else
        hipLaunchKernelGGL((rowlse_f32<D, 1>), dim3(G * wg1), dim3(kF32Threads), 0, s, a, nblk, ld_lse, p1);
    } else if (a.pass1 == PASS1_ATTENTION) {
      hipLaunchKernelGGL((rowattn_f32<D>), dim3(G * wg1), dim3(kF32Threads), 0, s, a, nblk, ld_lse, p1);
    }
    if (two)
      hipLaunchKernelGGL((colsum_f32<D, 2>), dim3(G * wg2), dim3(kF32Threads), 0, s, a, nblk2, ld_lse, p2);
    else
      hipLaunchKernelGGL((colsum_f32<D, 1>), dim3(G * wg1), dim3(kF32Threads), 0, s, a, nblk, ld_lse, p1);
  } else {
    const int nblk = (a.n + 255) / 256;
    if (a.pass1 == PASS1_ATTENTION) {
      // Prompts under 2048 tokens: 4-wave workgroups of 128 queries, two
      // per CU, so that fewer waves idle on the causal diagonal (1152: 1.88
      // -> 1.70 ms; 1920: -4%; 1024: -1%; 2048 measured 0.6% slower).
      if (a.n < 2048) {
        const int nb = (a.n + 127) / 128, paired = pair_blocks(nb);
        hipLaunchKernelGGL((rowattn8_lds<DT, D, 4>), dim3(pad8(G * (paired ? (nb + 1) / 2 : nb))), dim3(256), 0, s, a, nb, G,
                           ld_lse, paired);
      } else {
        const int paired = pair_blocks(nblk);
        hipLaunchKernelGGL((rowattn8_lds<DT, D, 8>), dim3(pad8(G * (paired ? (nblk + 1) / 2 : nblk))), dim3(512), 0, s, a, nblk,
                           G, ld_lse, paired);
      }
    }
    // Prompts up to 2048 tokens: 2-wave workgroups (128 queries or keys), so
    // that more, shorter workgroups overlap their prologues and fewer waves
    // idle on the causal diagonal (prompt 1024: 10% faster, 1920: 11%);
    // longer prompts keep 4 waves sharing each staged tile (4096: 5% faster,
    // 8192: 5%).
    if (a.n <= 2048) {
      const int nb = (a.n + 127) / 128;
      const int paired = pair_blocks(nb);
      const int per_head = paired ? (nb + 1) / 2 : nb;
      if (a.pass1 == PASS1_LSE)
        hipLaunchKernelGGL((rowlse_lds<DT, D, 2>), dim3(pad8(G * per_head)), dim3(128), 0, s, a, nb, G, ld_lse, paired);
      hipLaunchKernelGGL((colsum_lds<DT, D, 2>), dim3(pad8(G * per_head)), dim3(128), 0, s, a, nb, G, ld_lse, paired);
    } else {
      const int paired = pair_blocks(nblk);
      const int per_head = paired ? (nblk + 1) / 2 : nblk;
      if (a.pass1 == PASS1_LSE)
        hipLaunchKernelGGL((rowlse_lds<DT, D, 4>), dim3(pad8(G * per_head)), dim3(256), 0, s, a, nblk, G, ld_lse, paired);
      hipLaunchKernelGGL((colsum_lds<DT, D, 4>), dim3(pad8(G * per_head)), dim3(256), 0, s, a, nblk, G, ld_lse, paired);
    }
  }
  switch (a.quant) {
    case H2O_QUANT_NONE:
      hipLaunchKernelGGL((select_gather<DT, D, 0>), dim3(G), dim3(kSelThreads), size_t(a.k_heavy + a.k_recent) * sizeof(int), s, a);
      break;
    case H2O_QUANT_U8:
      hipLaunchKernelGGL((key_grid<DT, D, 8>), dim3(G), dim3(256), 0, s, a);
      hipLaunchKernelGGL((select_gather<DT, D, 8>), dim3(G), dim3(kSelThreads), size_t(a.k_heavy + a.k_recent) * sizeof(int), s, a);
      break;
    case H2O_QUANT_U4:
      hipLaunchKernelGGL((key_grid<DT, D, 4>), dim3(G), dim3(256), 0, s, a);
      hipLaunchKernelGGL((select_gather<DT, D, 4>), dim3(G), dim3(kSelThreads), size_t(a.k_heavy + a.k_recent) * sizeof(int), s, a);
      break;
    case H2O_QUANT_U2:
      hipLaunchKernelGGL((key_grid<DT, D, 2>), dim3(G), dim3(256), 0, s, a);
      hipLaunchKernelGGL((select_gather<DT, D, 2>), dim3(G), dim3(kSelThreads), size_t(a.k_heavy + a.k_recent) * sizeof(int), s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(int dtype, int head_dim, int G, const PrefillArgs& a, hipStream_t s) {
  if (G <= 0 || a.n <= 0) return hipSuccess;
  switch (dtype * 1000 + head_dim) {
    case DT_F32 * 1000 + 64: return prefill_typed<DT_F32, 64>(G, a, s);
    case DT_F32 * 1000 + 128: return prefill_typed<DT_F32, 128>(G, a, s);
    case DT_BF16 * 1000 + 64: return prefill_typed<DT_BF16, 64>(G, a, s);
    case DT_BF16 * 1000 + 128: return prefill_typed<DT_BF16, 128>(G, a, s);
    case DT_F16 * 1000 + 64: return prefill_typed<DT_F16, 64>(G, a, s);
    case DT_F16 * 1000 + 128: return prefill_typed<DT_F16, 128>(G, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_cache_clear(float* score, int32_t* pos, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(cache_clear, dim3(unsigned(blocks)), dim3(256), 0, s, score, pos, count);
  return hipGetLastError();
}

}  // namespace h2o
