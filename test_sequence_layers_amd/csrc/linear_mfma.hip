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
// Mapping.  The linear model is separable by output row (row i of W only needs v[i]), so a
// (batch, head) chain is split over kSplit = 2 workgroups of 32 output rows each; within a
// workgroup, wave w owns 16 rows and never exchanges state with the other wave.  The two
// workgroups of a chain get block indices that are equal mod 8, which places them on the
// same XCD, so their reads of the chain's Q and K meet in one L2.  Per chunk, each wave
// issues about 60 instructions; with one wave per SIMD that issue rate, not memory, bounds
// the kernel, and the split lets 192 CUs work instead of 96.
// A third wave streams chunks into an LDS ring with direct-to-LDS buffer loads (no
// registers are spent on data in flight); one barrier per group of 4 chunks publishes
// chunks and recycles slots.  The compute waves read the next chunk's operands while they
// compute the current one and store their 16 columns of Z directly.  The loop is unrolled
// over the whole ring, so every LDS address is a per-lane base plus an immediate.
// Within a wave everything stays in registers, in the layouts the MFMA operands need:
//   * the fp32 state W^T (64 x 16) is 4 accumulator tiles; tile t = 2 kb + hf, row m holds
//     input index j = 32 kb + 8 (m / 4) + 4 hf + m % 4, so lane (g, n) holds the four
//     consecutive inputs 32 kb + 8 g + 4 hf + e of output row i0 + n;
//   * its bf16 copy (tiles 2 kb and 2 kb + 1 side by side) is, lane for lane, the B operand
//     of R = K W^T and the A operand of Z^T = W Q^T for input block kb, with K and Q read
//     as 16-byte row pieces;
//   * R comes out with tokens as rows, which is the B operand of the rank-16 update
//     W^T += K^T (-eta R) (16x16x16 MFMA) and the A operand of the in-chunk correction
//     (-eta R^T) P^T;
//   * the K^T operand of the update is read with the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16): within 16 lanes, lane i receives element i % 4 of the 8 bytes
//     fetched by lane 4 s + i / 4, so lanes that fetch 4 consecutive inputs of token rows
//     4 g .. 4 g + 3 hand each lane the 4 tokens of one input column;
//   * P^T = K Q^T comes out as the B operand of that correction;
//   * -V enters R's accumulator through an MFMA with -I, which turns a row read of V into
//     the accumulator layout;
//   * every accumulator is written by one MFMA opcode only (chaining a 16x16x16 result into
//     a 16x16x32 accumulator input was observed to read stale values on gfx950); products
//     over the 16 tokens that share an accumulator with 16x16x32 products use 16x16x32
//     with the upper half of one operand zero.
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kD = 64;
constexpr int kB = 16;                 // tokens per chunk
constexpr int kTileBytes = kB * kD * 2;  // one 16 x 64 bf16 chunk of one tensor
constexpr int kTmBytes = kB * kB * 2;  // one 16 x 16 bf16 Tm matrix of the delta rule
constexpr int kComputeWaves = 2;
constexpr int kSplit = 4 / kComputeWaves;  // workgroups per chain
constexpr int kThreads = 64 * (kComputeWaves + 1);
constexpr int kHalfCols = kD / kSplit;  // output rows (= V columns) per workgroup

// LDS ring of kRing slots, published kGroup chunks per barrier.  Slot layout: Q tile at 0
// and K tile at 2 KB (16 rows of 128 bytes, 16-byte pieces swizzled by row), this
// workgroup's 32 V columns at 4 KB (16 rows of 64 bytes, swizzled), and for the delta
// rule the chunk's Tm (512 bytes, row-major, then 512 bytes of zeros) at 5 KB.  The
// loader issues kLoads direct-to-LDS loads per chunk; its waits before barriers are
// bounded by the 6-bit vmcnt (a smaller count than needed only waits longer).
constexpr int kGroup = 4;
constexpr int kRing = 16;
constexpr int kVOff = 2 * kTileBytes;
constexpr int kTmOff = kVOff + kB * kHalfCols * 2;
// (Plain constants: a dependent static member passed to the direct-to-LDS load builtin
// kept the host compiler from emitting the kernel's launch stub.)
template <bool kDelta> struct Ring {
  static constexpr int kLoads = kDelta ? 6 : 5;
  static constexpr int kSlotBytes = kTmOff + (kDelta ? 2 * kTmBytes : 0);
  static constexpr int clampw(int nchunks) {
    return nchunks * kLoads < 64 ? nchunks * kLoads : (63 / kLoads) * kLoads;
  }
  static constexpr int kWait0 = clampw(kRing - 1 - kGroup);
  static constexpr int kWait1 = clampw(kRing - 1 - 2 * kGroup);
  static constexpr int kWaitN = clampw(kRing - 2 * kGroup);
};

// Swizzle of the 128-byte Q/K rows: logical 16-byte piece p of row r sits at piece
// p ^ sig(r).  sig is a bijection on r mod 8, so the 8 lanes of a 16-byte row read (rows
// n .. n + 7, one logical piece) hit 8 different bank groups; and it flips bit 2 of the
// piece index between the rows 4 g + s of a transposing read, which keeps that read at
// two lanes per bank pair (the minimum for 8-byte reads at a fixed half of a piece).
__device__ __forceinline__ int sig(int r) { return ((r & 1) << 2) | ((r >> 1) & 3); }
__device__ __forceinline__ int swz(int r, int p) { return r * 8 + (p ^ sig(r)); }
// Swizzle of the 64-byte V rows: piece p of row r at p ^ ((r / 2) % 4).
__device__ __forceinline__ int vswz(int r, int p) { return r * 4 + (p ^ ((r >> 1) & 3)); }

__device__ __forceinline__ bf16x8_t bf8(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }
__device__ __forceinline__ bf16x4_t bf4(const u32x2& x) { return __builtin_bit_cast(bf16x4_t, x); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
template <typename T>
__device__ __forceinline__ T lds_load(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
__device__ __forceinline__ u32x2 lds_load_tr(const lds_char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

struct ChunkRegs {
  u32x4 ka0, ka1;          // K[t = n][8 g + 0..7], K[n][32 + 8 g + 0..7]
  u32x4 qb0, qb1;          // Q[n][8 g + 0..7], Q[n][32 + 8 g + 0..7]
  u32x2 kt0, kt1, kt2, kt3;  // tile t: K[4 g + s][j_t(n)], s = 0..3 (A operand of the update)
  u32x2 vv;                // V[n][i0 + 4 g .. 4 g + 3]
  u32x2 tm;                // delta rule: Tm[n][4 g .. 4 g + 3] (from the stored Tm^T)
};

// Per-lane byte offsets inside a slot, fixed for the whole kernel.
struct LaneOffsets {
  int ka0, ka1;  // row n, pieces g and 4 + g
  int kt0, kt1;  // transposing reads: row 4 g + n / 4, pieces n % 4 and 4 + n % 4
  int vv;        // V row n, columns i0 - 32 part + 4 g
  int tm;        // Tm row n, columns 4 g
};

// Reads a chunk's operands from its ring slot.  Only compute waves run this, and their code
// path issues no direct-to-LDS loads, so the compiler's own lgkmcnt waits order the reads.
template <bool kDelta>
__device__ __forceinline__ void read_chunk(ChunkRegs& r, const lds_char* slot, const LaneOffsets& o) {
  const lds_char* q = slot;
  const lds_char* k = slot + kTileBytes;
  r.ka0 = lds_load<u32x4>(k + o.ka0);
  r.ka1 = lds_load<u32x4>(k + o.ka1);
  r.qb0 = lds_load<u32x4>(q + o.ka0);
  r.qb1 = lds_load<u32x4>(q + o.ka1);
  r.kt0 = lds_load_tr(k + o.kt0);
  r.kt1 = lds_load_tr(k + o.kt0 + 8);
  r.kt2 = lds_load_tr(k + o.kt1);
  r.kt3 = lds_load_tr(k + o.kt1 + 8);
  r.vv = lds_load<u32x2>(slot + kVOff + o.vv);
  if (kDelta) r.tm = lds_load_tr(slot + kTmOff + o.tm);
}

struct WState {
  float4_t t0, t1, t2, t3;
};

// Chunk-independent constants of a lane.
struct LaneConst {
  bf16x8_t neg_eye;        // -I as a padded B operand: slot s < 4 of lane (g, n) is row 4g+s
  uint32_t pmask0, pmask1; // causal mask of P^T on packed bf16 pairs (row 4g+e kept if <= n)
  float neta;
};

#define MFMA32 __builtin_amdgcn_mfma_f32_16x16x32_bf16
#define MFMA16 __builtin_amdgcn_mfma_f32_16x16x16bf16_1k

// One chunk.  Returns Z^T for the lane (4 consecutive output features of token n) as bf16.
template <bool kDelta>
__device__ __forceinline__ u32x2 chunk_step(WState& w, const ChunkRegs& r, const LaneConst& lc) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // bf16 W^T: operand kb holds inputs 32 kb + 8 g + 0..7 of output row i0 + n
  const u32x4 wb0u = {pack_bf16(w.t0[0], w.t0[1]), pack_bf16(w.t0[2], w.t0[3]),
                      pack_bf16(w.t1[0], w.t1[1]), pack_bf16(w.t1[2], w.t1[3])};
  const u32x4 wb1u = {pack_bf16(w.t2[0], w.t2[1]), pack_bf16(w.t2[2], w.t2[3]),
                      pack_bf16(w.t3[0], w.t3[1]), pack_bf16(w.t3[2], w.t3[3])};
  const bf16x8_t wb0 = bf8(wb0u), wb1 = bf8(wb1u);
  // R = K W^T - V (rows: tokens 4 g + e, column: output feature i0 + n)
  const u32x4 vpad = {r.vv.x, r.vv.y, 0u, 0u};
  float4_t racc = MFMA32(bf8(vpad), lc.neg_eye, zero, 0, 0, 0);
  racc = MFMA32(bf8(r.ka0), wb0, racc, 0, 0, 0);
  racc = MFMA32(bf8(r.ka1), wb1, racc, 0, 0, 0);
  if (kDelta) {
    // delta rule: R <- Tm R (Tm in the padded A layout, R in bf16 as the B operand)
    const u32x4 r0b = {pack_bf16(racc[0], racc[1]), pack_bf16(racc[2], racc[3]), 0u, 0u};
    const u32x4 tma = {r.tm.x, r.tm.y, 0u, 0u};
    racc = MFMA32(bf8(tma), bf8(r0b), zero, 0, 0, 0);
  }
  // Z^T = W Q^T (first part) and P^T = K Q^T, independent of R
  float4_t zacc = MFMA32(wb0, bf8(r.qb0), zero, 0, 0, 0);
  zacc = MFMA32(wb1, bf8(r.qb1), zacc, 0, 0, 0);
  float4_t pacc = MFMA32(bf8(r.ka0), bf8(r.qb0), zero, 0, 0, 0);
  pacc = MFMA32(bf8(r.ka1), bf8(r.qb1), pacc, 0, 0, 0);
  // W^T += K^T (-eta R)
  const u32x2 rn = {pack_bf16(lc.neta * racc[0], lc.neta * racc[1]),
                    pack_bf16(lc.neta * racc[2], lc.neta * racc[3])};
  w.t0 = MFMA16(bf4(r.kt0), bf4(rn), w.t0, 0, 0, 0);
  w.t1 = MFMA16(bf4(r.kt1), bf4(rn), w.t1, 0, 0, 0);
  w.t2 = MFMA16(bf4(r.kt2), bf4(rn), w.t2, 0, 0, 0);
  w.t3 = MFMA16(bf4(r.kt3), bf4(rn), w.t3, 0, 0, 0);
  // Z^T += (-eta R)^T P^T with the causal mask applied to the packed pairs of P^T
  const u32x4 pm = {pack_bf16(pacc[0], pacc[1]) & lc.pmask0,
                    pack_bf16(pacc[2], pacc[3]) & lc.pmask1, 0u, 0u};
  const u32x4 rn4 = {rn.x, rn.y, 0u, 0u};
  zacc = MFMA32(bf8(rn4), bf8(pm), zacc, 0, 0, 0);
  const u32x2 out = {pack_bf16(zacc[0], zacc[1]), pack_bf16(zacc[2], zacc[3])};
  return out;
}

// Buffer resource over the rest of a sequence: base at a chunk, range = bytes left, so rows
// past the end read as zero and stores to them are dropped.
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

// Workgroup barrier for LDS traffic only: this wave's LDS reads are complete, then all
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

template <bool kDelta>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void linear_mfma_kernel(
    LinearArgs a, const bf16* tmat) {
  using RG = Ring<kDelta>;
  __shared__ __attribute__((aligned(16))) char ring_mem[kRing * RG::kSlotBytes];
  lds_char* ring = (lds_char*)(ring_mem);

  // blockIdx = 8 kSplit (chain / 8) + 8 part + chain % 8: the parts of a chain share an XCD
  const int bidx = blockIdx.x;
  const int part = (bidx >> 3) % kSplit;
  const int chain = (bidx / (8 * kSplit)) * 8 + (bidx & 7);
  if (chain >= a.B * a.H) return;  // padding block of the last group of 8 chains
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int ngroups = (nchunks + kGroup - 1) / kGroup;
  const int seq_bytes = T * kD * 2;  // < 2^31: checked by linear_mfma_supported
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;

  if (wv == kComputeWaves) {
    // Loader wave: streams chunk c into ring slot c % kRing with direct-to-LDS loads.  Lane
    // l of a Q/K half tile fills physical piece l % 8 of row 8 hh + l / 8, i.e. loads that
    // row's logical piece (l % 8) ^ sig(l / 8); lane l of the V load fills physical piece
    // l % 4 of row l / 4 from this workgroup's 64-byte half of the V row.
    const char* qsrc = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
    const char* ksrc = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
    const char* vsrc = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
    const int lrow = lane >> 3;
    const int lglob = lrow * 128 + (((lane & 7) ^ sig(lrow)) * 16);
    const int vrow = lane >> 2;
    const int vglob = vrow * 128 + part * (kHalfCols * 2) + (((lane & 3) ^ ((vrow >> 1) & 3)) * 16);
    const char* tsrc = reinterpret_cast<const char*>(tmat) +
                       (kDelta ? static_cast<size_t>(chain) * nchunks * kTmBytes : 0);
    auto issue = [&](int c) {
      const int off = c * kTileBytes;
      lds_char* dst = ring + (c % kRing) * RG::kSlotBytes;
      const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(qsrc + off, seq_bytes - off);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dst, 16, lglob, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dst + 1024, 16, lglob + 1024, 0, 0, 0);
      const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(ksrc + off, seq_bytes - off);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + kTileBytes, 16, lglob, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + kTileBytes + 1024, 16, lglob + 1024, 0, 0, 0);
      const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(vsrc + off, seq_bytes - off);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + kVOff, 16, vglob, 0, 0, 0);
      if (kDelta) {
        // Tm^T of chunk c: 512 bytes read by lanes 0..31; lanes 32..63 are out of range
        // and fill the second half of the 1 KB area with zeros.
        const __amdgpu_buffer_rsrc_t rs =
            chunk_rsrc(tsrc + static_cast<size_t>(c) * kTmBytes, c < nchunks ? kTmBytes : 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + kTmOff, 16, lane * 16, 0, 0, 0);
      }
    };
    // The compute waves read chunk 0 after barrier 0 and chunks kGroup g + 1 .. kGroup g +
    // kGroup between barriers g and g + 1.  So barrier g publishes the chunks up to
    // kGroup g + kGroup, and from g = 1 on it frees the slots of the chunks up to kGroup g,
    // after which the loader refills the ring up to chunk kGroup g + kRing.  Barrier 0
    // frees nothing.
    for (int c = 0; c < kRing; ++c) issue(c);
    wait_vmcnt<RG::kWait0>();
    lds_barrier();
    if (ngroups > 1) {
      wait_vmcnt<RG::kWait1>();
      lds_barrier();
#pragma unroll
      for (int x = 0; x <= kGroup; ++x) issue(kRing + x);
    }
    for (int grp = 2; grp < ngroups; ++grp) {
      wait_vmcnt<RG::kWaitN>();
      lds_barrier();
#pragma unroll
      for (int x = 1; x <= kGroup; ++x) issue(kGroup * (grp - 1) + kRing + x);
    }
    wait_vmcnt<0>();  // no load outlives the wave
    return;
  }

  // Compute waves: wave w of part p owns output rows i0 .. i0 + 15, i0 = 32 p + 16 w.
  const int g = lane >> 4;
  const int n = lane & 15;
  const int i0 = kHalfCols * part + 16 * wv;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
  const float* w0 = a.w0 + bi * a.w0_batch_stride + static_cast<long long>(hi) * kD * kD;

  WState wacc;
  {
    const float* wr = w0 + (i0 + n) * kD + 8 * g;
    wacc.t0 = *reinterpret_cast<const float4_t*>(wr);
    wacc.t1 = *reinterpret_cast<const float4_t*>(wr + 4);
    wacc.t2 = *reinterpret_cast<const float4_t*>(wr + 32);
    wacc.t3 = *reinterpret_cast<const float4_t*>(wr + 36);
  }
  LaneConst lc;
  {
    const uint32_t one_neg = 0xBF80u;  // bf16 -1.0
    const u32x4 eye = {(4 * g + 0 == n ? one_neg : 0u) | (4 * g + 1 == n ? one_neg << 16 : 0u),
                       (4 * g + 2 == n ? one_neg : 0u) | (4 * g + 3 == n ? one_neg << 16 : 0u),
                       0u, 0u};
    lc.neg_eye = bf8(eye);
    lc.pmask0 = (4 * g + 0 <= n ? 0x0000FFFFu : 0u) | (4 * g + 1 <= n ? 0xFFFF0000u : 0u);
    lc.pmask1 = (4 * g + 2 <= n ? 0x0000FFFFu : 0u) | (4 * g + 3 <= n ? 0xFFFF0000u : 0u);
    lc.neta = -a.eta;
  }
  LaneOffsets o;
  o.ka0 = swz(n, g) * 16;
  o.ka1 = swz(n, 4 + g) * 16;
  o.kt0 = swz(4 * g + (n >> 2), n & 3) * 16;
  o.kt1 = swz(4 * g + (n >> 2), 4 + (n & 3)) * 16;
  o.vv = vswz(n, 2 * wv + (g >> 1)) * 16 + 8 * (g & 1);
  o.tm = (4 * g + (n >> 2)) * 32 + 8 * (n & 3);

  // Step c: compute chunk c from registers read in step c - 1 while reading chunk c + 1,
  // and store this wave's 16 columns of Z_c (8 bytes per lane; rows past T are dropped by
  // the buffer range).  Chunks past the end read as zeros and leave the state unchanged.
  // The Z stores of a block of kRing chunks share one buffer resource, rebased once per
  // block; the lane offsets of the block's chunks are precomputed, so a step's store needs
  // no address arithmetic (the range check on the lane offset still drops rows past T).
  const int zoff = n * 128 + 2 * (i0 + 4 * g);
  int zo[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) zo[i] = zoff + i * kTileBytes;
  lds_barrier();  // barrier 0: chunks 0 .. kGroup published
  ChunkRegs ra, rb;
  read_chunk<kDelta>(ra, ring, o);
  for (int gbase = 0; gbase < ngroups; gbase += kRing / kGroup) {
    const int boff = gbase * kGroup * kTileBytes;
    const __amdgpu_buffer_rsrc_t zrs = chunk_rsrc(z + boff, seq_bytes - boff);
#pragma unroll
    for (int gg = 0; gg < kRing / kGroup; ++gg) {
      const int grp = gbase + gg;
      if (grp >= ngroups) break;
      if (grp > 0) lds_barrier();
#pragma unroll
      for (int x = 0; x < kGroup; ++x) {
        const int nslot = (gg * kGroup + x + 1) % kRing;  // compile-time slot of chunk c + 1
        ChunkRegs& cur = (x & 1) ? rb : ra;
        ChunkRegs& nxt = (x & 1) ? ra : rb;
        __builtin_amdgcn_sched_barrier(0);  // keep steps apart (register pressure)
        read_chunk<kDelta>(nxt, ring + nslot * RG::kSlotBytes, o);
        const u32x2 zz = chunk_step<kDelta>(wacc, cur, lc);
        __builtin_amdgcn_raw_buffer_store_b64(zz, zrs, zo[gg * kGroup + x], 0, 0);
      }
    }
  }

  if (a.w_out) {
    float* wr = a.w_out + static_cast<size_t>(chain) * kD * kD + (i0 + n) * kD + 8 * g;
    *reinterpret_cast<float4_t*>(wr) = wacc.t0;
    *reinterpret_cast<float4_t*>(wr + 4) = wacc.t1;
    *reinterpret_cast<float4_t*>(wr + 32) = wacc.t2;
    *reinterpret_cast<float4_t*>(wr + 36) = wacc.t3;
  }
}

}  // namespace

static bool mfma_shape_ok(const LinearArgs& a) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  // 16-byte vector loads of tokens and of the fp32 state rows
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.z, 16) &&
                       al(a.w0, 16) && (a.w0_batch_stride % 4) == 0 &&
                       (a.w_out == nullptr || al(a.w_out, 16));
  // byte offsets inside one sequence, including the loads the ring issues past the end,
  // are 32-bit
  const bool fits = static_cast<long long>(a.T) * kD * 2 + 2LL * kTileBytes * (kRing + 2 * kGroup) < 0x7fffffffLL;
  return a.d == kD && a.T > 0 && aligned && fits;
}

static long long mfma_grid(const LinearArgs& a) {
  const long long nchains = static_cast<long long>(a.B) * a.H;
  return (nchains + 7) / 8 * 8 * kSplit;
}

bool linear_mfma_supported(const LinearArgs& a, bool bf16_io) {
  return bf16_io && a.chunk == kB && a.causal == 1 && mfma_shape_ok(a);
}

hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s) {
  const long long nblocks = mfma_grid(a);
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_mfma_kernel<false>, dim3(static_cast<unsigned>(nblocks)), dim3(kThreads),
                     0, s, a, static_cast<const bf16*>(nullptr));
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ delta rule

// Tm = (I + eta stril(K K^T))^-1 for every chunk of every chain, stored transposed in bf16:
// [chain][chunk][j][t] = Tm[t][j] (row j of the stored tile is column j of Tm).  One wave
// per 4 chunks: the wave forms the Gram matrix G = K K^T of each chunk with two MFMAs (K
// rows loaded straight into the operand layout; the A and B operands of K K^T are the same
// registers), stages L = eta stril(G) in LDS, and then lane (q, j) solves column j of chunk
// q by forward substitution in fp32, Tm[t][j] = [t == j] - sum_{s<t} L[t][s] Tm[s][j]
// (the 16 lanes of a chunk read the same L row, a broadcast).  Rows past the end of the
// sequence have zero keys, so their rows of Tm are unit rows.
constexpr int kTmWaves = 4;
constexpr int kTmChunksPerWave = 4;
__global__ __launch_bounds__(64 * kTmWaves) void delta_tmat_kernel(const bf16* __restrict__ k, bf16* __restrict__ tmt,
                                                                 int T, int nchunks, long long total, float eta) {
  __shared__ float ls[kTmWaves][kTmChunksPerWave][kB][kB];
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const long long id0 = (static_cast<long long>(blockIdx.x) * kTmWaves + wv) * kTmChunksPerWave;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < kTmChunksPerWave; ++q) {
    const long long id = id0 + q;  // uniform in the wave
    float4_t gacc = zero;
    if (id < total) {
      const long long chain = id / nchunks;
      const int c = static_cast<int>(id - chain * nchunks);
      const bf16* kc = k + (static_cast<size_t>(chain) * T + static_cast<size_t>(c) * kB) * kD;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kc), 0, (T - c * kB) * kD * 2, 0x00020000);
      // lane (g, n): K[n][8 g .. 8 g + 7] and K[n][32 + 8 g ..]; rows past T read as zero
      const u32x4 k0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, n * 128 + 16 * g, 0, 0));
      const u32x4 k1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, n * 128 + 64 + 16 * g, 0, 0));
      gacc = MFMA32(bf8(k0), bf8(k0), zero, 0, 0, 0);
      gacc = MFMA32(bf8(k1), bf8(k1), gacc, 0, 0, 0);
    }
    // lane (g, n) holds G[4 g + e][n]; keep the strict lower triangle, scaled by eta
#pragma unroll
    for (int e = 0; e < 4; ++e) ls[wv][q][4 * g + e][n] = (n < 4 * g + e) ? eta * gacc[e] : 0.0f;
  }
  __syncthreads();
  // lane (q, j): column j of chunk q
  const int q = g;
  const int j = n;
  const float* lq = &ls[wv][q][0][0];
  float x[kB];
#pragma unroll
  for (int t = 0; t < kB; ++t) {
    float acc = (t == j) ? 1.0f : 0.0f;
#pragma unroll
    for (int s4 = 0; s4 < t; s4 += 4) {
      const float4_t l4 = *reinterpret_cast<const float4_t*>(lq + t * kB + s4);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (s4 + u < t) acc -= l4[u] * x[s4 + u];
    }
    x[t] = acc;
  }
  const long long id = id0 + q;
  if (id < total) {
    u32x4 lo, hi;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lo[u] = pack_bf16(x[2 * u], x[2 * u + 1]);
      hi[u] = pack_bf16(x[8 + 2 * u], x[8 + 2 * u + 1]);
    }
    u32x4* out = reinterpret_cast<u32x4*>(tmt + static_cast<size_t>(id) * kB * kB + j * kB);
    out[0] = lo;
    out[1] = hi;
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
  constexpr int kPerBlock = kTmWaves * kTmChunksPerWave;
  const long long nblocks = (total + kPerBlock - 1) / kPerBlock;
  if (nchains > 0x7fffffffLL || nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  bf16* tm = static_cast<bf16*>(workspace);
  hipLaunchKernelGGL(delta_tmat_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(64 * kTmWaves), 0, s,
                     static_cast<const bf16*>(a.k), tm, a.T, nchunks, total, a.eta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nmain = mfma_grid(a);
  if (nmain > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_mfma_kernel<true>, dim3(static_cast<unsigned>(nmain)), dim3(kThreads),
                     0, s, a, static_cast<const bf16*>(tm));
  return hipGetLastError();
}

}  // namespace ttt
