// TTT-Linear forward on the gfx950 matrix cores: d = 64, mini-batch b = 16, causal,
// bf16 Q/K/V/Z, fp32 state; and, on the same machinery, the exact delta rule (b = 1).
//
// Method (wmrh.cn summary of Sun et al. 2024, section 1.2.2, mini-batch TTT and its dual
// form; gradient (W k - v) k^T from the "Fast weights" page, section 1).  For a chunk with
// rows Q, K, V (16 x 64) and chunk-start weights W, with R = K W^T - V:
//     Z = Q W^T - eta * tril(Q K^T) R        (tril keeps the diagonal: z_t sees its own
//     W <- W - eta * R^T K                    update)
// which equals the per-token recurrence up to floating-point order.
//
// Delta rule ("Fast weights" page, section 1: W_t = W_{t-1} + eta (v_t - W_{t-1} k_t) k_t^T,
// z_t = W_t q_t), processed 16 tokens at a time exactly.  Inside a chunk starting from W,
// the prediction errors u_t = v_t - W_{t-1} k_t satisfy
//     u_t = (v_t - W k_t) - eta * sum_{s<t} (k_t . k_s) u_s,
// i.e. (I + eta stril(K K^T)) U = -(K W^T - V).  With Tm = (I + eta stril(K K^T))^-1 and
// R = Tm (K W^T - V) = -U, the chunk's outputs and update are the mini-batch formulas
// above with this R (z_t = W q_t + eta sum_{s<=t} (q_t . k_s) u_s; W <- W + eta U^T K).
// Tm depends only on K; delta_tmat_kernel computes it for every chunk beforehand.
//
// Mapping.  One workgroup of 4 waves per (batch, head) chain.  The linear model is
// separable by output row (row i of W only needs v[i]), so wave w owns rows 16w..16w+15 of
// W and never exchanges state with the other waves.  A fifth wave streams Q/K/V chunks into
// an LDS ring with direct-to-LDS buffer loads (no registers are spent on data in flight);
// one barrier per group of 4 chunks publishes chunks and recycles slots.  The compute
// waves read the next chunk's operands while they compute the current one and store their
// 16 columns of Z directly.
// Within a wave everything stays in registers, in the layouts the MFMA operands need:
//   * the fp32 state W^T (64 x 16) is 4 accumulator tiles of v_mfma_f32_16x16x32_bf16;
//   * its bf16 copy is, lane for lane, the B operand of R = K W^T and the A operand of
//     Z^T = W Q^T, with K and Q read from LDS in the matching order;
//   * R comes out with tokens as rows, which is the B operand of the rank-16 update
//     W^T += K^T (-eta R) and the A operand of the in-chunk correction (-eta R^T) P^T;
//   * P^T = K Q^T comes out as the B operand of that correction;
//   * -V enters R's accumulator through an MFMA with -I, which turns a row read of V into
//     the accumulator layout;
//   * products that contract over the 16 tokens use the same 16x16x32 instruction with the
//     upper half of one operand zero.
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;
constexpr int kB = 16;          // tokens per chunk

struct ChunkRegs {
  u32x4 ka0, ka1;  // K[t = n][16 g + 0..7], K[n][16 g + 8..15]: the two A operands of K W^T
  u32x4 qb0, qb1;  // Q[n][16 g + 0..7], Q[n][16 g + 8..15]
  uint32_t kt[4][2];  // kt[e][h] = K[4 g + e][c0 + 8 h .. + 1],  c0 = 16 (n / 4) + 2 (n % 4)
  u32x2 vv;        // V[n][i0 + 4 g .. 4 g + 3]
  u32x2 tm;        // delta rule: Tm[n][4 g .. 4 g + 3] (A operand of R = Tm R0)
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ bf16x8_t bf(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }

// LDS tiles.  A tile is one 16 x 64 bf16 chunk of one tensor (16 rows of 128 bytes = 8
// pieces of 16 bytes).  Piece x of row t is stored at piece index t * 8 + (x ^ (t & 7)), so
// the row-strided operand reads of a wave spread over the banks.
constexpr int kTileBytes = kB * kD * 2;
constexpr int kTmBytes = kB * kB * 2;  // one 16 x 16 bf16 Tm matrix of the delta rule
// Ring of kSlots chunk slots, published kGroup chunks per barrier.  The loader issues
// kLoads loads per chunk (6, or 7 with Tm) and before barrier g waits until the chunks the
// compute waves read in group g have landed, leaving kSlots - 2 kGroup chunks in flight;
// the 6-bit vmcnt bounds that count.
constexpr int kGroup = 4;
template <bool kDelta> struct Ring {
  static constexpr int kLoads = kDelta ? 7 : 6;
  static constexpr int kSlots = 14;
  static constexpr int kSlotBytes = 3 * kTileBytes + (kDelta ? 1024 : 0);
  static_assert(kLoads * (kSlots - 1 - kGroup) < 64, "vmcnt is 6 bits");
  static_assert(kSlots >= 2 * kGroup, "ring too small for the group");
};
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ int swz(int t, int x) { return t * 8 + (x ^ (t & 7)); }

template <typename T>
__device__ __forceinline__ T lds_load(const lds_char* base, int byte) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(base + byte);
}
template <typename T>
__device__ __forceinline__ void lds_store(lds_char* base, int byte, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(base + byte) = v;
}

// Per-lane byte offsets inside a tile, fixed for the whole kernel.
struct LaneOffsets {
  int ka0, ka1;    // row n, pieces 2g and 2g+1
  int kt[4][2];    // row 4g+e, piece 2 (n / 4) + h, dword n % 4
  int vv;          // row n, piece 2w + g / 2, second half when g is odd
  int tm;          // Tm tile (row-major, unswizzled): row n, columns 4g .. 4g + 3
};

// Reads a chunk's operands from its ring slot (Q tile at +0, K at +kTileBytes, V at
// +2 kTileBytes).  Only compute waves run this, and their code path issues no
// direct-to-LDS loads, so the compiler's own lgkmcnt waits order the reads.
template <bool kDelta>
__device__ __forceinline__ void read_chunk(ChunkRegs& r, const lds_char* slot, const LaneOffsets& o) {
  const lds_char* q = slot;
  const lds_char* k = slot + kTileBytes;
  const lds_char* v = slot + 2 * kTileBytes;
  r.ka0 = lds_load<u32x4>(k, o.ka0);
  r.ka1 = lds_load<u32x4>(k, o.ka1);
  r.qb0 = lds_load<u32x4>(q, o.ka0);
  r.qb1 = lds_load<u32x4>(q, o.ka1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.kt[e][0] = lds_load<uint32_t>(k, o.kt[e][0]);
    r.kt[e][1] = lds_load<uint32_t>(k, o.kt[e][1]);
  }
  r.vv = lds_load<u32x2>(v, o.vv);
  if (kDelta) r.tm = lds_load<u32x2>(slot + 3 * kTileBytes, o.tm);
}

// State: four fp32 accumulator tiles of W^T.  Tile jb = 2 h + p, row m of the tile holds
// input index j = 16 (m / 4) + 2 (m % 4) + 8 h + p, column n holds output row i0 + n; so
// lane (g, n), element e of tile 2h+p is W[i0 + n][16 g + 8 h + 2 e + p].
struct WState {
  float4_t t0, t1, t2, t3;
};

// Chunk-independent constants of a lane.
struct LaneConst {
  bf16x8_t neg_eye;        // -I as a padded B operand: slot s < 4 of lane (g, n) is row 4g+s
  uint32_t pmask0, pmask1; // causal mask of P^T on packed bf16 pairs (row 4g+e kept if <= n)
  float neta;
};

// One chunk.  Every accumulation chain uses the one opcode v_mfma_f32_16x16x32_bf16 and
// the K = 16 products are zero-padded (chaining a 16x16x16 result into a 16x16x32
// accumulator input was observed to read stale accumulator values on gfx950).  Returns Z^T
// for the lane (4 consecutive output features of token n) packed as bf16.
template <bool kDelta>
__device__ __forceinline__ u32x2 chunk_step(WState& w, const ChunkRegs& r, const LaneConst& lc) {
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const bf16x8_t ka0 = bf(r.ka0), ka1 = bf(r.ka1), qb0 = bf(r.qb0), qb1 = bf(r.qb1);
  // bf16 copy of the chunk-start W^T in the B layout of K W^T: operand h, dword e holds
  // j = 16 g + 8 h + 2 e + {0, 1}, matching the K row reads.
  const bf16x8_t wb0 = as_bf16x8(pack_bf16(w.t0[0], w.t1[0]), pack_bf16(w.t0[1], w.t1[1]),
                                 pack_bf16(w.t0[2], w.t1[2]), pack_bf16(w.t0[3], w.t1[3]));
  const bf16x8_t wb1 = as_bf16x8(pack_bf16(w.t2[0], w.t3[0]), pack_bf16(w.t2[1], w.t3[1]),
                                 pack_bf16(w.t2[2], w.t3[2]), pack_bf16(w.t2[3], w.t3[3]));
  // R = K W^T - V (rows: tokens 4g+e, column: output feature i0 + n)
  const u32x4 vpad = {r.vv.x, r.vv.y, 0u, 0u};
  float4_t racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(vpad), lc.neg_eye, zero, 0, 0, 0);
  racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, wb0, racc, 0, 0, 0);
  racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, wb1, racc, 0, 0, 0);
  if (kDelta) {
    // delta rule: R <- Tm R (Tm in the padded A layout, R0 in bf16 as the B operand)
    const u32x4 r0b = {pack_bf16(racc[0], racc[1]), pack_bf16(racc[2], racc[3]), 0u, 0u};
    const u32x4 tma = {r.tm.x, r.tm.y, 0u, 0u};
    racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(tma), bf(r0b), zero, 0, 0, 0);
  }
  // Z^T = W Q^T (first part) and P^T = K Q^T, independent of R
  float4_t zacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb0, qb0, zero, 0, 0, 0);
  zacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb1, qb1, zacc, 0, 0, 0);
  float4_t pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qb0, zero, 0, 0, 0);
  pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qb1, pacc, 0, 0, 0);
  // K^T gathers for the update: tile 2h+p, lane (g, n), slot e = K[4g+e][c0 + 8h + p]
  const u32x4 kt0 = {__builtin_amdgcn_perm(r.kt[1][0], r.kt[0][0], kLo),
                     __builtin_amdgcn_perm(r.kt[3][0], r.kt[2][0], kLo), 0u, 0u};
  const u32x4 kt1 = {__builtin_amdgcn_perm(r.kt[1][0], r.kt[0][0], kHi),
                     __builtin_amdgcn_perm(r.kt[3][0], r.kt[2][0], kHi), 0u, 0u};
  const u32x4 kt2 = {__builtin_amdgcn_perm(r.kt[1][1], r.kt[0][1], kLo),
                     __builtin_amdgcn_perm(r.kt[3][1], r.kt[2][1], kLo), 0u, 0u};
  const u32x4 kt3 = {__builtin_amdgcn_perm(r.kt[1][1], r.kt[0][1], kHi),
                     __builtin_amdgcn_perm(r.kt[3][1], r.kt[2][1], kHi), 0u, 0u};
  // -eta R as a padded bf16 operand
  const u32x4 rbu = {pack_bf16(lc.neta * racc[0], lc.neta * racc[1]),
                     pack_bf16(lc.neta * racc[2], lc.neta * racc[3]), 0u, 0u};
  const bf16x8_t rb = bf(rbu);
  // W^T += K^T (-eta R)
  w.t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(kt0), rb, w.t0, 0, 0, 0);
  w.t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(kt1), rb, w.t1, 0, 0, 0);
  w.t2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(kt2), rb, w.t2, 0, 0, 0);
  w.t3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(kt3), rb, w.t3, 0, 0, 0);
  // Z^T += (-eta R)^T P^T with the causal mask applied to the packed pairs of P^T
  const u32x4 pbu = {pack_bf16(pacc[0], pacc[1]) & lc.pmask0,
                     pack_bf16(pacc[2], pacc[3]) & lc.pmask1, 0u, 0u};
  zacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb, bf(pbu), zacc, 0, 0, 0);
  const u32x2 out = {pack_bf16(zacc[0], zacc[1]), pack_bf16(zacc[2], zacc[3])};
  return out;
}

// Buffer resource over one chunk of a sequence: base at the chunk, range = bytes left, so
// rows past the end read as zero and stores to them are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int left) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, left > 0 ? left : 0,
                                           0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS traffic only: this wave's LDS writes are complete, then all
// waves meet.  (The fence of __syncthreads() would also drain every outstanding global
// load, i.e. the whole prefetch ring; the loads that the barrier publishes are waited for
// explicitly with wait_vmcnt.  The compiler does not order LDS reads after direct-to-LDS
// loads by itself, so that explicit wait is what makes the data visible.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unconstrained
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

constexpr int kComputeWaves = 4;
constexpr int kThreads = 64 * (kComputeWaves + 1);

template <bool kDelta>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void linear_mfma_kernel(
    LinearArgs a, const bf16* tmat) {
  using RG = Ring<kDelta>;
  constexpr int kRing = RG::kSlots;
  __shared__ __attribute__((aligned(16))) char ring_mem[kRing * RG::kSlotBytes];
  lds_char* ring = (lds_char*)(ring_mem);

  const int chain = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int seq_bytes = T * kD * 2;  // < 2^31: checked by linear_mfma_supported
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;

  if (wv == kComputeWaves) {
    // Loader wave: streams Q, K, V of chunk c into ring slot c % kRing with direct-to-LDS
    // loads, 6 instructions per chunk (2 per tensor, 8 rows each).  Lane l fills piece l
    // of a half tile: row 8 hh + l / 8 at swizzled position l % 8, which holds global
    // piece (l % 8) ^ (l / 8) of that row.  Barrier b publishes chunk b (b = 0 before the
    // loop, then chunk c + 1 at barrier c) and frees the slot of chunk c.
    const char* src[3] = {reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0),
                          reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0),
                          reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0)};
    const int lrow = lane >> 3;
    const int lglob = lrow * 128 + (((lane & 7) ^ lrow) * 16);
    const char* tsrc = reinterpret_cast<const char*>(tmat) +
                       (kDelta ? static_cast<size_t>(chain) * nchunks * kTmBytes : 0);
    auto issue = [&](int c) {
      const int off = c * kTileBytes;
      lds_char* dst = ring + (c % kRing) * RG::kSlotBytes;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(src[t] + off, seq_bytes - off);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + t * kTileBytes, 16, lglob, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + t * kTileBytes + 1024, 16, lglob + 1024, 0, 0, 0);
      }
      if (kDelta) {
        // Tm of chunk c: 512 bytes read by lanes 0..31; lanes 32..63 are out of range and
        // fill the unused second half of the 1 KB area with zeros.
        const __amdgpu_buffer_rsrc_t rs =
            chunk_rsrc(tsrc + static_cast<size_t>(c) * kTmBytes, c < nchunks ? kTmBytes : 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + 3 * kTileBytes, 16, lane * 16, 0, 0, 0);
      }
    };
    // The compute waves read chunk 0 after barrier 0 and chunks kGroup g + 1 .. kGroup g +
    // kGroup between barriers g and g + 1.  So barrier g publishes the chunks up to
    // kGroup g + kGroup, and from g = 1 on it frees the slots of the chunks up to kGroup g,
    // after which the loader refills the ring up to chunk kGroup g + kRing.
    // Barrier 0 frees nothing; the wait before barrier 1 leaves chunks kGroup + kGroup + 1 ..
    // kRing - 1 in flight, later waits leave kRing - 2 kGroup chunks in flight.
    const int ngroups = (nchunks + kGroup - 1) / kGroup;
    for (int c = 0; c < kRing; ++c) issue(c);
    wait_vmcnt<RG::kLoads * (kRing - 1 - kGroup)>();
    lds_barrier();
    if (ngroups > 1) {
      wait_vmcnt<RG::kLoads * (kRing - 1 - 2 * kGroup)>();
      lds_barrier();
#pragma unroll
      for (int x = 0; x <= kGroup; ++x) issue(kRing + x);
    }
    for (int grp = 2; grp < ngroups; ++grp) {
      wait_vmcnt<RG::kLoads * (kRing - 2 * kGroup)>();
      lds_barrier();
#pragma unroll
      for (int x = 1; x <= kGroup; ++x) issue(kGroup * (grp - 1) + kRing + x);
    }
    wait_vmcnt<0>();  // no load outlives the wave
    return;
  }

  // Compute waves: wave w owns output rows 16w .. 16w + 15.
  const int g = lane >> 4;
  const int n = lane & 15;
  const int i0 = 16 * wv;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
  const float* w0 = a.w0 + bi * a.w0_batch_stride + static_cast<long long>(hi) * kD * kD;

  // state: element e of tile 2h+p = W[i0 + n][16 g + 8 h + 2 e + p]
  WState wacc;
  {
    const float* wr = w0 + (i0 + n) * kD + 16 * g;
    const float4_t f0 = *reinterpret_cast<const float4_t*>(wr);
    const float4_t f1 = *reinterpret_cast<const float4_t*>(wr + 4);
    const float4_t f2 = *reinterpret_cast<const float4_t*>(wr + 8);
    const float4_t f3 = *reinterpret_cast<const float4_t*>(wr + 12);
    wacc.t0 = float4_t{f0[0], f0[2], f1[0], f1[2]};
    wacc.t1 = float4_t{f0[1], f0[3], f1[1], f1[3]};
    wacc.t2 = float4_t{f2[0], f2[2], f3[0], f3[2]};
    wacc.t3 = float4_t{f2[1], f2[3], f3[1], f3[3]};
  }
  LaneConst lc;
  {
    const uint32_t one_neg = 0xBF80u;  // bf16 -1.0
    const u32x4 eye = {(4 * g + 0 == n ? one_neg : 0u) | (4 * g + 1 == n ? one_neg << 16 : 0u),
                       (4 * g + 2 == n ? one_neg : 0u) | (4 * g + 3 == n ? one_neg << 16 : 0u),
                       0u, 0u};
    lc.neg_eye = bf(eye);
    lc.pmask0 = (4 * g + 0 <= n ? 0x0000FFFFu : 0u) | (4 * g + 1 <= n ? 0xFFFF0000u : 0u);
    lc.pmask1 = (4 * g + 2 <= n ? 0x0000FFFFu : 0u) | (4 * g + 3 <= n ? 0xFFFF0000u : 0u);
    lc.neta = -a.eta;
  }
  LaneOffsets o;
  o.ka0 = swz(n, 2 * g) * 16;
  o.ka1 = swz(n, 2 * g + 1) * 16;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int h = 0; h < 2; ++h) o.kt[e][h] = swz(4 * g + e, 2 * (n >> 2) + h) * 16 + 4 * (n & 3);
  o.vv = swz(n, 2 * wv + (g >> 1)) * 16 + 8 * (g & 1);
  o.tm = n * 32 + 8 * g;

  // Step c: compute chunk c from registers read in step c - 1 while reading chunk c + 1,
  // and store this wave's 16 columns of Z_c (8 bytes per lane; rows past T are dropped by
  // the buffer range).  Chunks past the end read as zeros and leave the state unchanged.
  const int zoff = n * 128 + 2 * (i0 + 4 * g);
  auto step = [&](int c, ChunkRegs& cur, ChunkRegs& nxt) {
    __builtin_amdgcn_sched_barrier(0);  // keep steps apart (register pressure)
    read_chunk<kDelta>(nxt, ring + ((c + 1) % kRing) * RG::kSlotBytes, o);
    const u32x2 zz = chunk_step<kDelta>(wacc, cur, lc);
    const int off = c * kTileBytes;
    __builtin_amdgcn_raw_buffer_store_b64(zz, chunk_rsrc(z + off, seq_bytes - off), zoff, 0, 0);
  };
  const int ngroups = (nchunks + kGroup - 1) / kGroup;
  lds_barrier();  // barrier 0: chunks 0 .. kGroup published
  ChunkRegs ra, rb;
  read_chunk<kDelta>(ra, ring, o);
  for (int grp = 0; grp < ngroups; ++grp) {
    if (grp > 0) lds_barrier();
    const int c = grp * kGroup;
    static_assert(kGroup == 4, "the group below is written out for 4 chunks");
    step(c + 0, ra, rb);
    step(c + 1, rb, ra);
    step(c + 2, ra, rb);
    step(c + 3, rb, ra);
  }

  if (a.w_out) {
    float* wr = a.w_out + static_cast<size_t>(chain) * kD * kD + (i0 + n) * kD + 16 * g;
    *reinterpret_cast<float4_t*>(wr) = float4_t{wacc.t0[0], wacc.t1[0], wacc.t0[1], wacc.t1[1]};
    *reinterpret_cast<float4_t*>(wr + 4) = float4_t{wacc.t0[2], wacc.t1[2], wacc.t0[3], wacc.t1[3]};
    *reinterpret_cast<float4_t*>(wr + 8) = float4_t{wacc.t2[0], wacc.t3[0], wacc.t2[1], wacc.t3[1]};
    *reinterpret_cast<float4_t*>(wr + 12) = float4_t{wacc.t2[2], wacc.t3[2], wacc.t2[3], wacc.t3[3]};
  }
}

}  // namespace

static bool mfma_shape_ok(const LinearArgs& a) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  // 16-byte vector loads of tokens and of the fp32 state rows
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.z, 16) &&
                       al(a.w0, 16) && (a.w0_batch_stride % 4) == 0 &&
                       (a.w_out == nullptr || al(a.w_out, 16));
  // byte offsets inside one sequence are 32-bit
  const bool fits = static_cast<long long>(a.T) * kD * 2 + 2LL * kTileBytes * 16 < 0x7fffffffLL;
  return a.d == kD && a.T > 0 && aligned && fits;
}

bool linear_mfma_supported(const LinearArgs& a, bool bf16_io) {
  return bf16_io && a.chunk == kB && a.causal == 1 && mfma_shape_ok(a);
}

hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  if (nchains > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_mfma_kernel<false>, dim3(static_cast<unsigned>(nchains)), dim3(kThreads),
                     0, s, a, static_cast<const bf16*>(nullptr));
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ delta rule

// Tm = (I + eta stril(K K^T))^-1 for every chunk of every chain, in bf16, row-major
// [chain][chunk][16][16].  One group of 16 lanes per chunk (16 chunks per workgroup):
// lane j first computes column j of the strictly lower Gram matrix, then column j of Tm by
// forward substitution, Tm[t][j] = [t == j] - eta sum_{s<t} (k_t . k_s) Tm[s][j].  Rows past
// the end of the sequence have zero keys, so their rows of Tm are unit rows.
__global__ __launch_bounds__(256) void delta_tmat_kernel(const bf16* __restrict__ k, bf16* __restrict__ tm,
                                                         int T, int nchunks, long long total, float eta) {
  __shared__ float ks[16][kB][kD + 1];
  __shared__ float gram[16][kB][kB + 1];
  const int grp = threadIdx.x >> 4;   // chunk within the workgroup
  const int j = threadIdx.x & 15;
  const long long id = static_cast<long long>(blockIdx.x) * 16 + grp;
  const bool valid = id < total;
  const long long chain = valid ? id / nchunks : 0;
  const int c = valid ? static_cast<int>(id - chain * nchunks) : 0;
  const bf16* kc = k + (static_cast<size_t>(chain) * T + static_cast<size_t>(c) * kB) * kD;
  // lane j loads row j of the chunk (zero past the end of the sequence)
  const bool row_in = valid && c * kB + j < T;
  for (int x = 0; x < kD; ++x) ks[grp][j][x] = row_in ? static_cast<float>(kc[j * kD + x]) : 0.0f;
  __syncthreads();
  for (int t = 0; t < kB; ++t) {
    float acc = 0.0f;
    if (t > j)
      for (int x = 0; x < kD; ++x) acc += ks[grp][t][x] * ks[grp][j][x];
    gram[grp][t][j] = acc;
  }
  __syncthreads();
  float col[kB];
#pragma unroll
  for (int t = 0; t < kB; ++t) {
    float acc = (t == j) ? 1.0f : 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < t; ++s2) acc -= eta * gram[grp][t][s2] * col[s2];
    col[t] = acc;
  }
  if (valid) {
    bf16* out = tm + static_cast<size_t>(id) * kB * kB;
#pragma unroll
    for (int t = 0; t < kB; ++t) out[t * kB + j] = static_cast<bf16>(col[t]);
  }
}

bool delta_fast_supported(const LinearArgs& a, bool bf16_io) {
  return bf16_io && mfma_shape_ok(a);
}

size_t delta_workspace_bytes(const LinearArgs& a) {
  const long long nchunks = (a.T + kB - 1) / kB;
  return static_cast<size_t>(a.B) * a.H * nchunks * kTmBytes;
}

hipError_t launch_delta_fast(const LinearArgs& a, void* workspace, hipStream_t s) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  const int nchunks = (a.T + kB - 1) / kB;
  const long long total = nchains * nchunks;
  const long long nblocks = (total + 15) / 16;
  if (nchains > 0x7fffffffLL || nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  bf16* tm = static_cast<bf16*>(workspace);
  hipLaunchKernelGGL(delta_tmat_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(256), 0, s,
                     static_cast<const bf16*>(a.k), tm, a.T, nchunks, total, a.eta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(linear_mfma_kernel<true>, dim3(static_cast<unsigned>(nchains)), dim3(kThreads),
                     0, s, a, static_cast<const bf16*>(tm));
  return hipGetLastError();
}

}  // namespace ttt
