// TTT-Linear forward on the gfx950 matrix cores: d = 64, mini-batch b = 16, causal,
// bf16 Q/K/V/Z, fp32 state; and, on the same machinery, the exact delta rule (b = 1).
//
// Method (wmrh.cn summary of Sun et al. 2024, section 1.2.2, mini-batch TTT and its dual
// form; gradient (W k - v) k^T from the "Fast weights" page, section 1; with the negative
// dot-product loss of the blog page, section TTT / 如何理解, the gradient is -v k^T and
// R = -V below).  For a chunk with rows Q, K, V (16 x 64) and chunk-start weights W, with
// R = K W^T - V:
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
// workgroup, chain wave w owns 16 rows and never exchanges state with the other chain wave.
// The two workgroups of a chain get block indices that are equal mod 8, which places them
// on the same XCD, so their reads of the chain's Q and K meet in one L2.
// Work per workgroup, each on its own SIMD:
//   * two chain waves run the state recursion only, two chunks per step (below), and hand
//     each pair's bf16 start state and -eta R to an output wave through LDS;
//   * two output waves form each chunk's Z one group of chunks later and store it;
//   * a loader wave streams chunks into an LDS ring with direct-to-LDS buffer loads (no
//     registers are spent on data in flight).  What bounds the kernel is this stream: a
//     compute unit takes in at most about 38 GB/s (one 128-byte line per ~7 cycles, with
//     the non-temporal policy), and a chunk costs a workgroup 48 lines (Q, K and V; the V
//     half-rows cost whole lines).
// One barrier per group of 4 chunks publishes chunks and handoffs and recycles ring slots and
// handoff buffers.  The chain waves read a pair's operands one step ahead.  Loops are
// unrolled over the whole ring, so every LDS address is a per-lane base plus an immediate.
//
// Two chunks per step.  From W = W_c, R_c = K_c W^T - V_c and, since W_{c+1} = W - eta R_c^T
// K_c, R_{c+1} = (K_{c+1} W^T - V_{c+1}) + (K_{c+1} K_c^T)(-eta R_c) (delta rule: Tm times
// each bracket); then one update W <- W - eta [R_c; R_{c+1}]^T [K_c; K_{c+1}] over 32
// tokens.  So the state, its bf16 copy and the update are touched once per pair, and Z of
// the second chunk is Q W_c^T + (Q K_c^T)(-eta R_c) + tril(Q K^T)(-eta R_{c+1}).
// Within a wave everything stays in registers, in the layouts the MFMA operands need:
//   * the fp32 state W^T (64 x 16) is 4 accumulator tiles; tile t = 2 kb + hf, row m holds
//     input index j = 32 kb + 8 (m / 4) + 4 hf + m % 4, so lane (g, n) holds the four
//     consecutive inputs 32 kb + 8 g + 4 hf + e of output row i0 + n;
//   * its bf16 copy (tiles 2 kb and 2 kb + 1 side by side) is, lane for lane, the B operand
//     of R = K W^T and the A operand of Z^T = W Q^T for input block kb, with K and Q read
//     as 16-byte row pieces;
//   * R comes out with tokens as rows: as bf16 pairs it is the B operand (over tokens) of
//     the state update and of M (-eta R_c), and the A operand of the output corrections
//     (-eta R^T) P^T (the handoff stores the bf16 operands lane by lane, so the output wave
//     gets them in the same layouts);
//   * the K^T operands of the update are read with the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16): within 16 lanes, lane i receives element i % 4 of the 8 bytes
//     fetched by lane 4 s + i / 4, so lanes that fetch 4 consecutive inputs of token rows
//     4 g .. 4 g + 3 hand each lane the 4 tokens of one input column; the pair's two
//     chunks fill slots 0..3 and 4..7 of one K = 32 operand;
//   * M^T = K_c K_{c+1}^T, P^T = K Q^T and (K_c Q^T) come out in the layout of the A or B
//     operands that use them;
//   * -V enters R's accumulator through an MFMA with -I, which turns a row read of V into
//     the accumulator layout;
//   * every accumulator is written by one MFMA opcode only (chaining a 16x16x16 result into
//     a 16x16x32 accumulator input was observed to read stale values on gfx950); products
//     over the 16 tokens of a chunk use 16x16x32 with the upper half of one operand zero.
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
constexpr int kChainWaves = 2;
constexpr int kOutWaves = kChainWaves;
// Waves of a workgroup: 0, 1 chain; 2, 3 output (first chunk of each pair); 4, 5 loaders;
// 6, 7 output (second chunk of each pair).  Waves are placed on the four SIMDs in turn, so
// each chain wave shares its SIMD with a loader and the four output waves share the other
// two.  Each output wave forms all of the workgroup's 32 Z columns of its chunk, so that one
// 16-byte store per lane writes the chunk's rows (a compute unit's memory pipeline pays per
// row piece touched, and loads and stores share it).  Two loader waves (Q and V; K with the rate factors and Tm^T): one wave issues a
// direct-to-LDS load only every ~70 cycles, so a compute unit streams about twice as fast
// from two waves as from one.
constexpr int kLoaderWave = kChainWaves + kOutWaves;  // first loader wave
constexpr int kLoaderWaves = 2;
constexpr int kSplit = 4 / kChainWaves;  // workgroups per chain
constexpr int kThreads = 64 * (kLoaderWave + kLoaderWaves + kOutWaves);
constexpr int kHalfCols = kD / kSplit;  // output rows (= V columns) per workgroup

// LDS ring of kRing slots, published kGroup chunks per barrier.  Slot layout: Q tile at 0
// and K tile at 2 KB (16 rows of 128 bytes, 16-byte pieces swizzled by row), this
// workgroup's 32 V columns at 4 KB (16 rows of 64 bytes, swizzled), and for the delta
// rule the chunk's Tm^T (512 bytes, row-major) after that; with per-token rates, the
// chunk's 16 rate factors (64 bytes) sit between V and Tm^T.  Loader wave p issues
// loads(p) direct-to-LDS loads of every chunk, so the same chunk counts bound each
// loader's waits before barriers, times its own loads per chunk and capped by the 6-bit
// vmcnt (a smaller count than needed only waits longer).
// Barrier b publishes the chunks that the chain waves read after it (up to kGroup b +
// kGroup + 1) and frees the slots of the chunks that the output waves finished before it (up
// to kGroup b - kGroup - 1); the loader then refills up to kRing chunks past that.
constexpr int kGroup = 4;
constexpr int kVOff = 2 * kTileBytes;
constexpr int kEtaOff = kVOff + kB * kHalfCols * 2;  // per-token rate factors (64 bytes)
constexpr int kEtaBytes = kB * 4;
constexpr int kTmOffNoRates = kEtaOff;
constexpr int kTmOffRates = kEtaOff + kEtaBytes;
// (Plain constants: a dependent static member passed to the direct-to-LDS load builtin
// kept the host compiler from emitting the kernel's launch stub.)
template <bool kDelta, bool kTok> struct Ring {
  static constexpr int kRing = kDelta && kTok ? 20 : 24;  // within 160 KB of LDS
  static constexpr int kSlotBytes = (kTok ? kTmOffRates : kTmOffNoRates) + (kDelta ? kTmBytes : 0);
  // loads per chunk of loader wave p: Q tile (2) and V half tile (1); K tile (2), rates, Tm^T
  static constexpr int loads(int p) { return p == 0 ? 3 : 2 + (kTok ? 1 : 0) + (kDelta ? 1 : 0); }
  static constexpr int clampw(int nchunks, int per) {
    return nchunks * per < 64 ? nchunks * per : (63 / per) * per;
  }
  template <int P> static constexpr int kWait0 = clampw(kRing - 2 - kGroup, loads(P));
  template <int P> static constexpr int kWait1 = clampw(kRing - 2 - 2 * kGroup, loads(P));
  template <int P> static constexpr int kWaitN = clampw(kRing - 2 - 3 * kGroup, loads(P));
  static_assert(kRing % kGroup == 0 && kRing - 2 - 3 * kGroup >= 0, "ring too small");
};
constexpr int kRingMax = 24;
// Cache policy of the streaming loads and of the Z stores: non-temporal (each byte is read
// once per workgroup, and Z is not read back).
constexpr int kNT = 2;

// Handoff from a chain wave to its output wave, per pair of chunks: the bf16 W^T operands
// of the pair's start state (two 16-byte pieces per lane) and -eta R of both chunks (8 bytes
// per lane each), lane-major.  Two buffers of one group each, by group parity: the chain
// waves fill one while the output waves read the other.
constexpr int kHandW1 = 64 * 16;
constexpr int kHandR0 = 2 * 64 * 16;
constexpr int kHandR1 = kHandR0 + 64 * 8;
constexpr int kHandPair = kHandR1 + 64 * 8;
constexpr int kHandWave = (kGroup / 2) * kHandPair;
constexpr int kHandGroup = kChainWaves * kHandWave;
constexpr int kHandBytes = 2 * kHandGroup;
// Per output wave, 1 KB that restages its chunk's 16 x 32 Z block row-major for the store.
constexpr int kStageBytes = 4 * kB * kHalfCols * 2;

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
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
template <typename T>
__device__ __forceinline__ T lds_load(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ void lds_store(lds_char* p, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(p) = v;
}
__device__ __forceinline__ u32x2 lds_load_tr(const lds_char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// A pair of chunks' operands for a chain wave, read one pair ahead: K rows, V columns, the
// K^T gathers and, for the delta rule, Tm.
struct PairRegs {
  u32x4 k[2][2];   // chunk e: K[n][8 g + 0..7], K[n][32 + 8 g + 0..7]
  u32x2 v[2];      // chunk e: V[n][i0 + 4 g .. + 3]
  u32x2 kt[2][4];  // chunk e, tile t: K[4 g + s][j_t(n)], s = 0..3
  u32x2 tm[2];     // delta rule: chunk e's Tm[n][4 g .. 4 g + 3] (from the stored Tm^T)
  float4_t et[2];  // per-token rates: chunk e's factors of tokens 4 g .. 4 g + 3
};

// Per-lane byte offsets inside a slot, fixed for the whole kernel.
struct LaneOffsets {
  int ka0, ka1;  // row n, pieces g and 4 + g
  int kt0, kt1;  // transposing reads: row 4 g + n / 4, pieces n % 4 and 4 + n % 4
  int vv;        // V row n, columns i0 - 32 part + 4 g
  int tm;        // Tm row n, columns 4 g
  int et;        // rate factors of tokens 4 g .. 4 g + 3
};

// Ring reads of the chain waves.  Only chain waves run this, and their code path issues no
// direct-to-LDS loads, so the compiler's own lgkmcnt waits order the reads.
template <bool kDelta, bool kTok>
__device__ __forceinline__ void read_pair(PairRegs& r, const lds_char* s0, const lds_char* s1, const LaneOffsets& o) {
  constexpr int kTmOff = kTok ? kTmOffRates : kTmOffNoRates;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const lds_char* slot = e ? s1 : s0;
    const lds_char* k = slot + kTileBytes;
    r.k[e][0] = lds_load<u32x4>(k + o.ka0);
    r.k[e][1] = lds_load<u32x4>(k + o.ka1);
    r.v[e] = lds_load<u32x2>(slot + kVOff + o.vv);
    r.kt[e][0] = lds_load_tr(k + o.kt0);
    r.kt[e][1] = lds_load_tr(k + o.kt0 + 8);
    r.kt[e][2] = lds_load_tr(k + o.kt1);
    r.kt[e][3] = lds_load_tr(k + o.kt1 + 8);
    if (kDelta) r.tm[e] = lds_load_tr(slot + kTmOff + o.tm);
    if (kTok) r.et[e] = lds_load<float4_t>(slot + kEtaOff + o.et);
  }
}

struct WState {
  float4_t t0, t1, t2, t3;
};

// Chunk-independent constants of a lane.
struct LaneConst {
  bf16x8_t neg_eye;        // -I as a padded B operand: slot s < 4 of lane (g, n) is row 4g+s
  float neta;
};

#define MFMA32 __builtin_amdgcn_mfma_f32_16x16x32_bf16

// -V + K W^T for one chunk: V row n enters the accumulator through an MFMA with -I.
__device__ __forceinline__ float4_t kw_minus_v(const u32x4& k0, const u32x4& k1, const u32x2& vv,
                                              const bf16x8_t& wb0, const bf16x8_t& wb1, const LaneConst& lc) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const u32x4 vpad = {vv.x, vv.y, 0u, 0u};
  float4_t acc = MFMA32(bf8(vpad), lc.neg_eye, zero, 0, 0, 0);
  acc = MFMA32(bf8(k0), wb0, acc, 0, 0, 0);
  return MFMA32(bf8(k1), wb1, acc, 0, 0, 0);
}
// Delta rule: R = Tm X, with X in bf16 as the B operand and Tm in the padded A layout.
__device__ __forceinline__ float4_t tm_apply(const u32x2& tm, const float4_t& x) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const u32x4 xb = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), 0u, 0u};
  const u32x4 tma = {tm.x, tm.y, 0u, 0u};
  return MFMA32(bf8(tma), bf8(xb), zero, 0, 0, 0);
}
__device__ __forceinline__ u32x2 neg_eta_bf16(const float4_t& r, float neta) {
  const u32x2 x = {pack_bf16(neta * r[0], neta * r[1]), pack_bf16(neta * r[2], neta * r[3])};
  return x;
}
// -eta_t R with a rate factor per row (token 4 g + e)
__device__ __forceinline__ u32x2 neg_eta_bf16(const float4_t& r, float neta, const float4_t& et) {
  const u32x2 x = {pack_bf16((neta * et[0]) * r[0], (neta * et[1]) * r[1]),
                   pack_bf16((neta * et[2]) * r[2], (neta * et[3]) * r[3])};
  return x;
}

// Chunks c, c + 1 (c even) of the state recursion, from W = W_c:
//   R_c     = K_c W^T - V_c
//   R_{c+1} = K_{c+1} W_{c+1}^T - V_{c+1} = (K_{c+1} W^T - V_{c+1}) + M (-eta R_c),
//             M = K_{c+1} K_c^T, because W_{c+1} = W - eta R_c^T K_c
//   W_{c+2} = W - eta [R_c; R_{c+1}]^T [K_c; K_{c+1}]   (one K = 32 MFMA per state tile)
// (delta rule: each R is Tm times the bracket).  Only the second R waits for the first; the
// state update and its bf16 copy happen once per pair.  Hands off the bf16 W_c and
// -eta R_c, -eta R_{c+1} to the output wave (pair area h; lw = 16 lane, lr = 8 lane).
template <bool kDelta, bool kTok, bool kDot>
__device__ __forceinline__ void pair_step(WState& w, const PairRegs& r, const LaneConst& lc, lds_char* h, int lw,
                                          int lr) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const u32x4 wb0u = {pack_bf16(w.t0[0], w.t0[1]), pack_bf16(w.t0[2], w.t0[3]),
                      pack_bf16(w.t1[0], w.t1[1]), pack_bf16(w.t1[2], w.t1[3])};
  const u32x4 wb1u = {pack_bf16(w.t2[0], w.t2[1]), pack_bf16(w.t2[2], w.t2[3]),
                      pack_bf16(w.t3[0], w.t3[1]), pack_bf16(w.t3[2], w.t3[3])};
  const bf16x8_t wb0 = bf8(wb0u), wb1 = bf8(wb1u);
  float4_t r0, r1;
  u32x2 rn0, rn1;
  if (kDot) {
    // dot-product loss: the error term is -v whatever W is, so neither R needs the state
    const u32x4 vpad0 = {r.v[0].x, r.v[0].y, 0u, 0u}, vpad1 = {r.v[1].x, r.v[1].y, 0u, 0u};
    r0 = MFMA32(bf8(vpad0), lc.neg_eye, zero, 0, 0, 0);
    r1 = MFMA32(bf8(vpad1), lc.neg_eye, zero, 0, 0, 0);
    rn0 = kTok ? neg_eta_bf16(r0, lc.neta, r.et[0]) : neg_eta_bf16(r0, lc.neta);
    rn1 = kTok ? neg_eta_bf16(r1, lc.neta, r.et[1]) : neg_eta_bf16(r1, lc.neta);
  } else {
    r0 = kw_minus_v(r.k[0][0], r.k[0][1], r.v[0], wb0, wb1, lc);
    const float4_t a1 = kw_minus_v(r.k[1][0], r.k[1][1], r.v[1], wb0, wb1, lc);
    // M^T = K_c K_{c+1}^T in the C layout is M as the A operand: lane (g, n) = M[n][4 g + s]
    float4_t mt = MFMA32(bf8(r.k[0][0]), bf8(r.k[1][0]), zero, 0, 0, 0);
    mt = MFMA32(bf8(r.k[0][1]), bf8(r.k[1][1]), mt, 0, 0, 0);
    if (kDelta) r0 = tm_apply(r.tm[0], r0);
    rn0 = kTok ? neg_eta_bf16(r0, lc.neta, r.et[0]) : neg_eta_bf16(r0, lc.neta);
    const u32x4 mpad = {pack_bf16(mt[0], mt[1]), pack_bf16(mt[2], mt[3]), 0u, 0u};
    const u32x4 rpad0 = {rn0.x, rn0.y, 0u, 0u};
    r1 = MFMA32(bf8(mpad), bf8(rpad0), a1, 0, 0, 0);
    if (kDelta) r1 = tm_apply(r.tm[1], r1);
    rn1 = kTok ? neg_eta_bf16(r1, lc.neta, r.et[1]) : neg_eta_bf16(r1, lc.neta);
  }
  lds_store<u32x4>(h + lw, wb0u);
  lds_store<u32x4>(h + kHandW1 + lw, wb1u);
  lds_store<u32x2>(h + kHandR0 + lr, rn0);
  lds_store<u32x2>(h + kHandR1 + lr, rn1);
  // W^T += K^T (-eta R) over the pair's 32 tokens: slots 0..3 chunk c, 4..7 chunk c + 1
  const u32x4 rr = {rn0.x, rn0.y, rn1.x, rn1.y};
  const u32x4 k0 = {r.kt[0][0].x, r.kt[0][0].y, r.kt[1][0].x, r.kt[1][0].y};
  const u32x4 k1 = {r.kt[0][1].x, r.kt[0][1].y, r.kt[1][1].x, r.kt[1][1].y};
  const u32x4 k2 = {r.kt[0][2].x, r.kt[0][2].y, r.kt[1][2].x, r.kt[1][2].y};
  const u32x4 k3 = {r.kt[0][3].x, r.kt[0][3].y, r.kt[1][3].x, r.kt[1][3].y};
  w.t0 = MFMA32(bf8(k0), bf8(rr), w.t0, 0, 0, 0);
  w.t1 = MFMA32(bf8(k1), bf8(rr), w.t1, 0, 0, 0);
  w.t2 = MFMA32(bf8(k2), bf8(rr), w.t2, 0, 0, 0);
  w.t3 = MFMA32(bf8(k3), bf8(rr), w.t3, 0, 0, 0);
}

// One chunk's output from the pair's handoff h and the chunk's ring slot:
//   Z^T = W Q^T + (-eta R)^T P^T,  P^T = K Q^T with the causal mask on its packed pairs.
// For the second chunk of a pair W is the pair's start state W_c and the first chunk's
// update enters as (-eta R_c)^T (K_c Q^T) (kprev: K_c's slot).  Returns Z^T for the lane (4
// consecutive output features of token n) as bf16.
template <bool kOdd>
__device__ __forceinline__ u32x2 out_step(const lds_char* slot, const lds_char* kprev, const lds_char* h, int ka0,
                                          int ka1, int lw, int lr, uint32_t pmask0, uint32_t pmask1) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const lds_char* q = slot;
  const lds_char* k = slot + kTileBytes;
  const bf16x8_t qb0 = bf8(lds_load<u32x4>(q + ka0)), qb1 = bf8(lds_load<u32x4>(q + ka1));
  const bf16x8_t kb0 = bf8(lds_load<u32x4>(k + ka0)), kb1 = bf8(lds_load<u32x4>(k + ka1));
  const bf16x8_t wb0 = bf8(lds_load<u32x4>(h + lw)), wb1 = bf8(lds_load<u32x4>(h + kHandW1 + lw));
  const u32x2 rn = lds_load<u32x2>(h + (kOdd ? kHandR1 : kHandR0) + lr);
  float4_t zacc = MFMA32(wb0, qb0, zero, 0, 0, 0);
  zacc = MFMA32(wb1, qb1, zacc, 0, 0, 0);
  float4_t pacc = MFMA32(kb0, qb0, zero, 0, 0, 0);
  pacc = MFMA32(kb1, qb1, pacc, 0, 0, 0);
  if (kOdd) {
    const lds_char* kp = kprev + kTileBytes;
    const bf16x8_t kp0 = bf8(lds_load<u32x4>(kp + ka0)), kp1 = bf8(lds_load<u32x4>(kp + ka1));
    const u32x2 rp = lds_load<u32x2>(h + kHandR0 + lr);
    float4_t xacc = MFMA32(kp0, qb0, zero, 0, 0, 0);
    xacc = MFMA32(kp1, qb1, xacc, 0, 0, 0);
    const u32x4 xm = {pack_bf16(xacc[0], xacc[1]), pack_bf16(xacc[2], xacc[3]), 0u, 0u};
    const u32x4 rp4 = {rp.x, rp.y, 0u, 0u};
    zacc = MFMA32(bf8(rp4), bf8(xm), zacc, 0, 0, 0);
  }
  const u32x4 pm = {pack_bf16(pacc[0], pacc[1]) & pmask0, pack_bf16(pacc[2], pacc[3]) & pmask1, 0u, 0u};
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

template <int P> struct IntTag {
  static constexpr int value = P;
};

template <bool kDelta, bool kTok, bool kDot>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void linear_mfma_kernel(
    LinearArgs a, const bf16* tmat) {
  using RG = Ring<kDelta, kTok>;
  constexpr int kTmOff = kTok ? kTmOffRates : kTmOffNoRates;
  constexpr int kRing = RG::kRing;
  __shared__ __attribute__((aligned(16))) char lds_mem[kRing * RG::kSlotBytes + kHandBytes + kStageBytes];
  lds_char* ring = (lds_char*)(lds_mem);
  lds_char* hand = ring + kRing * RG::kSlotBytes;
  lds_char* stage = hand + kHandBytes;

  // blockIdx = 8 kSplit (chain / 8) + 8 part + chain % 8: the parts of a chain share an XCD
  const int bidx = blockIdx.x;
  const int part = (bidx >> 3) % kSplit;
  const int chain = (bidx / (8 * kSplit)) * 8 + (bidx & 7);
  if (chain >= a.B * a.H) return;  // padding block of the last group of 8 chains
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int T = a.T;
  const int nchunks = (T + kB - 1) / kB;
  const int ngroups = (nchunks + kGroup - 1) / kGroup;
  const int seq_bytes = T * kD * 2;  // < 2^31: checked by linear_mfma_supported
  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const int lw = 16 * lane, lr = 8 * lane;  // lane offsets in a handoff
  // Every wave meets barriers 0 .. ngroups.  Chain waves compute group grp (chunks kGroup grp
  // .. + kGroup - 1) between barriers grp and grp + 1 and hand it off; output waves finish it
  // between barriers grp + 1 and grp + 2.

  if (wv >= kLoaderWave && wv < kLoaderWave + kLoaderWaves) {
    // Loader waves: stream chunk c into ring slot c % kRing with direct-to-LDS loads, wave
    // kLoaderWave + p taking part p of every chunk (Q tile and V half tile; K tile with the
    // rate factors and Tm^T).  Lane l of a Q/K half tile fills physical piece l % 8 of row
    // 8 hh + l / 8, i.e. loads that row's logical piece (l % 8) ^ sig(l / 8); lane l of the
    // V load fills physical piece l % 4 of row l / 4 from this workgroup's 64-byte half of
    // the V row.
    const char* qsrc = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
    const char* ksrc = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
    const char* vsrc = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
    const int lrow = lane >> 3;
    const int lglob = lrow * 128 + (((lane & 7) ^ sig(lrow)) * 16);
    const int vrow = lane >> 2;
    const int vglob = vrow * 128 + part * (kHalfCols * 2) + (((lane & 3) ^ ((vrow >> 1) & 3)) * 16);
    const char* tsrc = reinterpret_cast<const char*>(tmat) +
                       (kDelta ? static_cast<size_t>(chain) * nchunks * kTmBytes : 0);
    const char* esrc = kTok ? reinterpret_cast<const char*>(a.eta_tok + static_cast<size_t>(chain) * T) : nullptr;
    // Chain waves read chunks 0, 1 after barrier 0 and chunks up to kGroup b + kGroup + 1
    // after barrier b (one pair ahead); output waves read chunks kGroup (b - 1) .. kGroup b - 1 after barrier
    // b.  So barrier b must publish the chunks up to kGroup b + kGroup + 1, and from b = 2 on it
    // frees the slots of the chunks up to kGroup b - kGroup - 1 (barriers 0 and 1 free
    // nothing), after which each loader refills the ring up to chunk kGroup b - kGroup - 1 +
    // kRing.
    auto stream = [&](auto part_tag) {
      constexpr int P = decltype(part_tag)::value;
      auto issue = [&](int c) {
        const int off = c * kTileBytes;
        lds_char* dst = ring + (c % kRing) * RG::kSlotBytes;
        const __amdgpu_buffer_rsrc_t rs = chunk_rsrc((P == 0 ? qsrc : ksrc) + off, seq_bytes - off);
        lds_char* d = dst + P * kTileBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, lglob, 0, 0, kNT);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d + 1024, 16, lglob + 1024, 0, 0, kNT);
        if constexpr (P == 0) {
          const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(vsrc + off, seq_bytes - off);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + kVOff, 16, vglob, 0, 0, kNT);
        } else {
          if (kTok && lane < kB) {
            // rate factors of chunk c's tokens: 4 bytes per lane (zeros past the end)
            const __amdgpu_buffer_rsrc_t re = chunk_rsrc(esrc + c * kEtaBytes, T * 4 - c * kEtaBytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(re, dst + kEtaOff, 4, lane * 4, 0, 0, kNT);
          }
          if (kDelta && lane < 32) {
            // Tm^T of chunk c: 512 bytes, 16 per lane (zeros past the last chunk)
            const __amdgpu_buffer_rsrc_t rs =
                chunk_rsrc(tsrc + static_cast<size_t>(c) * kTmBytes, c < nchunks ? kTmBytes : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + kTmOff, 16, lane * 16, 0, 0, kNT);
          }
        }
      };
      for (int c = 0; c < kRing; ++c) issue(c);
      wait_vmcnt<RG::template kWait0<P>>();
      lds_barrier();  // barrier 0
      wait_vmcnt<RG::template kWait1<P>>();
      lds_barrier();  // barrier 1
      for (int b = 2; b <= ngroups; ++b) {
        wait_vmcnt<RG::template kWaitN<P>>();
        lds_barrier();  // barrier b
        if (b < ngroups) {
#pragma unroll
          for (int x = 0; x < kGroup; ++x) issue(kGroup * b - 2 * kGroup + kRing + x);
        }
      }
    };
    if (wv == kLoaderWave) {
      stream(IntTag<0>{});
    } else {
      stream(IntTag<1>{});
    }
    wait_vmcnt<0>();  // no load outlives the wave
    return;
  }

  LaneOffsets o;
  o.ka0 = swz(n, g) * 16;
  o.ka1 = swz(n, 4 + g) * 16;

  if (wv >= kChainWaves) {
    // Output wave (pr, hf): chunk hf of pair pr of every group, Z columns 32 part .. + 31 (the
    // row blocks of both chain waves).  Lane (g, n) holds token n, columns 16 ow + 4 g .. + 3
    // of block ow; the wave restages the two blocks row-major in its own 1 KB of LDS and
    // stores 16 bytes per lane, 64 bytes of each of the chunk's 16 rows, non-temporal like
    // the loads (rows past T are dropped by the buffer range).  The stores of a block of kRing chunks share one buffer
    // resource, rebased once per block.
    const int pr = wv & 1;
    const bool hf = wv >= kLoaderWave + kLoaderWaves;
    lds_char* zst = stage + (pr + (hf ? 2 : 0)) * (kStageBytes / 4);
    char* z = reinterpret_cast<char*>(static_cast<bf16*>(a.z) + tok0);
    const uint32_t pmask0 = (4 * g + 0 <= n ? 0x0000FFFFu : 0u) | (4 * g + 1 <= n ? 0xFFFF0000u : 0u);
    const uint32_t pmask1 = (4 * g + 2 <= n ? 0x0000FFFFu : 0u) | (4 * g + 3 <= n ? 0xFFFF0000u : 0u);
    const int zw = n * (kHalfCols * 2) + 8 * g;  // restage offset of block 0 (block 1: + 32)
    const int zoff = (lane >> 2) * 128 + part * (kHalfCols * 2) + (lane & 3) * 16 + (hf ? kTileBytes : 0);
    lds_barrier();  // barrier 0
    for (int gbase = 0; gbase < ngroups; gbase += kRing / kGroup) {
      const int boff = gbase * kGroup * kTileBytes;
      const __amdgpu_buffer_rsrc_t zrs = chunk_rsrc(z + boff, seq_bytes - boff);
#pragma unroll
      for (int gg = 0; gg < kRing / kGroup; ++gg) {
        const int grp = gbase + gg;
        if (grp >= ngroups) break;
        lds_barrier();  // barrier grp + 1: group grp's handoffs are complete
        const int slot = gg * kGroup + 2 * pr;  // chunk kGroup grp + 2 pr, mod kRing
        const lds_char* s0 = ring + slot * RG::kSlotBytes;
        const lds_char* hp0 = hand + (grp & 1) * kHandGroup + pr * kHandPair;
        const lds_char* hp1 = hp0 + kHandWave;
        u32x2 za, zb;
        if (!hf) {
          za = out_step<false>(s0, s0, hp0, o.ka0, o.ka1, lw, lr, pmask0, pmask1);
          zb = out_step<false>(s0, s0, hp1, o.ka0, o.ka1, lw, lr, pmask0, pmask1);
        } else {
          za = out_step<true>(s0 + RG::kSlotBytes, s0, hp0, o.ka0, o.ka1, lw, lr, pmask0, pmask1);
          zb = out_step<true>(s0 + RG::kSlotBytes, s0, hp1, o.ka0, o.ka1, lw, lr, pmask0, pmask1);
        }
        lds_store<u32x2>(zst + zw, za);
        lds_store<u32x2>(zst + zw + 32, zb);
        __asm__ __volatile__("" ::: "memory");  // the wave's LDS accesses execute in order
        const u32x4 zr = lds_load<u32x4>(zst + 16 * lane);
        __builtin_amdgcn_raw_buffer_store_b128(zr, zrs, zoff + slot * kTileBytes, 0, kNT);
      }
    }
    return;
  }

  // Chain waves: wave w of part p owns output rows i0 .. i0 + 15, i0 = 32 p + 16 w.
  const int i0 = kHalfCols * part + 16 * wv;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
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
    lc.neta = -a.eta;
  }
  o.kt0 = swz(4 * g + (n >> 2), n & 3) * 16;
  o.kt1 = swz(4 * g + (n >> 2), 4 + (n & 3)) * 16;
  o.vv = vswz(n, 2 * wv + (g >> 1)) * 16 + 8 * (g & 1);
  o.tm = (4 * g + (n >> 2)) * 32 + 8 * (n & 3);
  o.et = 16 * g;

  // Pair step p computes chunks 2p, 2p + 1 from registers read in step p - 1 while reading
  // chunks 2p + 2, 2p + 3.  Chunks past the end read as zeros and leave the state unchanged.
  lds_char* hw = hand + wv * kHandWave;
  lds_barrier();  // barrier 0: chunks 0 .. kGroup + 1 published
  PairRegs ra, rb;
  read_pair<kDelta, kTok>(ra, ring, ring + RG::kSlotBytes, o);
  for (int gbase = 0; gbase < ngroups; gbase += kRing / kGroup) {
#pragma unroll
    for (int gg = 0; gg < kRing / kGroup; ++gg) {
      const int grp = gbase + gg;
      if (grp >= ngroups) break;
      if (grp > 0) lds_barrier();  // barrier grp
      lds_char* hg = hw + (grp & 1) * kHandGroup;
#pragma unroll
      for (int x = 0; x < kGroup; x += 2) {
        const int s2 = (gg * kGroup + x + 2) % kRing;  // compile-time slots of chunks c + 2, c + 3
        const int s3 = (gg * kGroup + x + 3) % kRing;
        const PairRegs& cur = (x & 2) ? rb : ra;
        PairRegs& nxt = (x & 2) ? ra : rb;
        __builtin_amdgcn_sched_barrier(0);  // keep steps apart (register pressure)
        read_pair<kDelta, kTok>(nxt, ring + s2 * RG::kSlotBytes, ring + s3 * RG::kSlotBytes, o);
        pair_step<kDelta, kTok, kDot>(wacc, cur, lc, hg + (x / 2) * kHandPair, lw, lr);
      }
    }
  }
  lds_barrier();  // barrier ngroups: the last group's handoffs are complete

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
  const bool fits = static_cast<long long>(a.T) * kD * 2 + 2LL * kTileBytes * (kRingMax + 2 * kGroup) < 0x7fffffffLL;
  return a.d == kD && a.T > 0 && a.ln_w == nullptr && aligned && fits;
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
  const dim3 grid(static_cast<unsigned>(nblocks)), block(kThreads);
  const bf16* none = nullptr;
  if (a.dot_loss) {
    if (a.eta_tok)
      hipLaunchKernelGGL((linear_mfma_kernel<false, true, true>), grid, block, 0, s, a, none);
    else
      hipLaunchKernelGGL((linear_mfma_kernel<false, false, true>), grid, block, 0, s, a, none);
  } else {
    if (a.eta_tok)
      hipLaunchKernelGGL((linear_mfma_kernel<false, true, false>), grid, block, 0, s, a, none);
    else
      hipLaunchKernelGGL((linear_mfma_kernel<false, false, false>), grid, block, 0, s, a, none);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ delta rule

// Tm = (I + eta stril(K K^T) diag(eta_tok))^-1 for every chunk of every chain (diag(eta_tok)
// = I without per-token rates: the write of token s carries its own rate, so column s of
// the strict lower triangle is scaled by it), stored transposed in bf16:
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
                                                                 int T, int nchunks, long long total, float eta,
                                                                 const float* __restrict__ etok) {
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
    float rate = eta;
    if (id < total) {
      const long long chain = id / nchunks;
      const int c = static_cast<int>(id - chain * nchunks);
      if (etok) {  // uniform: rate factor of token n of the chunk (zero past T)
        const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(etok + static_cast<size_t>(chain) * T + static_cast<size_t>(c) * kB), 0,
            (T - c * kB) * 4, 0x00020000);
        rate = eta * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, n * 4, 0, 0));
      }
      const bf16* kc = k + (static_cast<size_t>(chain) * T + static_cast<size_t>(c) * kB) * kD;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(kc), 0, (T - c * kB) * kD * 2, 0x00020000);
      // lane (g, n): K[n][8 g .. 8 g + 7] and K[n][32 + 8 g ..]; rows past T read as zero
      const u32x4 k0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, n * 128 + 16 * g, 0, 0));
      const u32x4 k1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, n * 128 + 64 + 16 * g, 0, 0));
      gacc = MFMA32(bf8(k0), bf8(k0), zero, 0, 0, 0);
      gacc = MFMA32(bf8(k1), bf8(k1), gacc, 0, 0, 0);
    }
    // lane (g, n) holds G[4 g + e][n]; keep the strict lower triangle, scaled by the rate of
    // token n (column)
#pragma unroll
    for (int e = 0; e < 4; ++e) ls[wv][q][4 * g + e][n] = (n < 4 * g + e) ? rate * gacc[e] : 0.0f;
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
                     static_cast<const bf16*>(a.k), tm, a.T, nchunks, total, a.eta, a.eta_tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nmain = mfma_grid(a);
  if (nmain > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.eta_tok)
    hipLaunchKernelGGL((linear_mfma_kernel<true, true, false>), dim3(static_cast<unsigned>(nmain)), dim3(kThreads),
                       0, s, a, static_cast<const bf16*>(tm));
  else
    hipLaunchKernelGGL((linear_mfma_kernel<true, false, false>), dim3(static_cast<unsigned>(nmain)), dim3(kThreads),
                       0, s, a, static_cast<const bf16*>(tm));
  return hipGetLastError();
}

}  // namespace ttt
