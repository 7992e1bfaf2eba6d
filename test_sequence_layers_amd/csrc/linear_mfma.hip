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
// The same holds for a pair of chunks taken as one block of 32 tokens: the kernel applies
// the pair's 32 x 32 Tm = I + N at once, R = X + N X (X = K W^T - V of both chunks, exact
// in fp32, plus a correction with bf16 operands).  N depends only on K (and the rates), so
// two Tm waves of the workgroup compute it one group of chunks ahead, from the K tiles in
// the ring (tm_pair below), and hand it to the chain waves through LDS; nothing is read
// from or written to global memory for it.
//
// Mapping.  The linear model is separable by output row (row i of W only needs v[i]), so a
// (batch, head) chain is split over kSplit = 2 workgroups of 32 output rows each; within a
// workgroup, chain wave w owns 16 rows and never exchanges state with the other chain wave.
// The two workgroups of a chain get block indices that are equal mod 8, which places them
// on the same XCD, so their reads of the chain's Q and K meet in one L2.
// Work per workgroup (the wave roles are listed in Waves<> below):
//   * two chain waves run the state recursion only, two chunks per step (below), and hand
//     each pair's bf16 start state and -eta R to the output waves through LDS;
//   * four output waves form each chunk's Z one group of chunks later and store it;
//   * two loader waves stream chunks into an LDS ring with direct-to-LDS buffer loads (no
//     registers are spent on data in flight).  A compute unit takes in about 38 GB/s from
//     one loader wave (one 128-byte line per ~7 cycles, with the non-temporal policy), and
//     a chunk costs a workgroup 48 lines (Q, K and V; the V half-rows cost whole lines);
//   * for the delta rule, two Tm waves form the pair inverses of the next group of chunks.
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
constexpr int kChainWaves = 2;
constexpr int kOutWaves = kChainWaves;
// Waves of a workgroup (Waves<> below): two chain waves, four output waves (two for the first
// chunk of each pair, two for the second), two loaders, and for the delta rule two Tm waves
// and two idle ones.  Waves are placed on the four SIMDs in turn (wave w on SIMD w % 4); each
// chain wave shares its SIMD only with a loader (and, for the delta rule, an idle wave), and
// each delta Tm wave shares its SIMD with two output waves.
// Each output wave forms all of the workgroup's 32 Z columns of its chunk, so that one
// 16-byte store per lane writes the chunk's rows (a compute unit's memory pipeline pays per
// row piece touched, and loads and stores share it).  Two loader waves (Q and V; K with the
// rate factors): one wave issues a direct-to-LDS load only every ~70 cycles, so a compute
// unit streams about twice as fast from two waves as from one.
constexpr int kLoaderWave = kChainWaves + kOutWaves;  // first loader wave
constexpr int kLoaderWaves = 2;
constexpr int kSplit = 4 / kChainWaves;  // workgroups per chain
constexpr int kThreads = 64 * (kLoaderWave + kLoaderWaves + kOutWaves);
constexpr int kHalfCols = kD / kSplit;  // output rows (= V columns) per workgroup

// LDS ring of kRing slots, published kGroup chunks per barrier.  Slot layout: Q tile at 0
// and K tile at 2 KB (16 rows of 128 bytes, 16-byte pieces swizzled by row), this
// workgroup's 32 V columns at 4 KB (16 rows of 64 bytes, swizzled); with per-token rates,
// the chunk's 16 rate factors (64 bytes) after V.  Loader wave p issues loads(p)
// direct-to-LDS loads of every chunk, so the same chunk counts bound each loader's waits
// before barriers, times its own loads per chunk and capped by the 6-bit vmcnt (a smaller
// count than needed only waits longer).
// Barrier b publishes the chunks that the chain waves read after it (up to kGroup b +
// kGroup + 1; for the delta rule kAhead = 2 more, the next group that the Tm wave works on)
// and frees the slots of the chunks that the output waves finished before it (up to
// kGroup b - kGroup - 1); the loader then refills up to kRing chunks past that.
constexpr int kGroup = 4;
constexpr int kVOff = 2 * kTileBytes;
constexpr int kEtaOff = kVOff + kB * kHalfCols * 2;  // per-token rate factors (64 bytes)
constexpr int kEtaBytes = kB * 4;
constexpr int kSlotPlain = kEtaOff;
constexpr int kSlotRates = kEtaOff + kEtaBytes;
// (Plain constants: a dependent static member passed to the direct-to-LDS load builtin
// kept the host compiler from emitting the kernel's launch stub.)
template <bool kDelta, bool kTok> struct Ring {
  static constexpr int kRing = 24;  // within 160 KB of LDS
  static constexpr int kSlotBytes = kTok ? kSlotRates : kSlotPlain;
  static constexpr int kAhead = kDelta ? 2 : 0;
  // loads per chunk of loader wave p: Q tile (2) and V half tile (1); K tile (2) and rates
  static constexpr int loads(int p) { return p == 0 ? 3 : 2 + (kTok ? 1 : 0); }
  static constexpr int clampw(int nchunks, int per) {
    return nchunks * per < 64 ? nchunks * per : (63 / per) * per;
  }
  template <int P> static constexpr int kWait0 = clampw(kRing - 2 - kGroup - kAhead, loads(P));
  template <int P> static constexpr int kWait1 = clampw(kRing - 2 - 2 * kGroup - kAhead, loads(P));
  template <int P> static constexpr int kWaitN = clampw(kRing - 2 - 3 * kGroup - kAhead, loads(P));
  static_assert(kRing % kGroup == 0 && kRing - 2 - 3 * kGroup - kAhead >= 0, "ring too small");
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
// Delta rule: the pair correction operands N (per pair: N00 over the first chunk's tokens, 8
// bytes per lane, then [N10 | N11] over both chunks' tokens, 16 bytes per lane), two groups
// by group parity (the Tm waves fill one while the chain waves read the other).
constexpr int kNPair = 64 * 8 + 64 * 16;
constexpr int kNGroup = (kGroup / 2) * kNPair;
constexpr int kNBytes = 2 * kNGroup;

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
  float4_t et[2];  // per-token rates: chunk e's factors of tokens 4 g .. 4 g + 3
};

// Per-lane byte offsets inside a slot, fixed for the whole kernel.
struct LaneOffsets {
  int ka0, ka1;  // row n, pieces g and 4 + g
  int kt0, kt1;  // transposing reads: row 4 g + n / 4, pieces n % 4 and 4 + n % 4
  int vv;        // V row n, columns i0 - 32 part + 4 g
  int et;        // rate factors of tokens 4 g .. 4 g + 3
};

// Ring reads of the chain waves.  Only chain waves run this, and their code path issues no
// direct-to-LDS loads, so the compiler's own lgkmcnt waits order the reads.
template <bool kTok>
__device__ __forceinline__ void read_pair(PairRegs& r, const lds_char* s0, const lds_char* s1, const LaneOffsets& o) {
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
// Only the second R waits for the first; the state update and its bf16 copy happen once per
// pair.  Delta rule: with X_e = K_e W^T - V_e of both chunks, the pair's R = X + N X in one
// step (N = Tm - I of the pair's 32 tokens, from the Tm wave: n00 over chunk c's tokens,
// n1 over both chunks'): R_c = X_c + N00 X_c, R_{c+1} = X_{c+1} + N10 X_c + N11 X_{c+1}.
// Hands off the bf16 W_c and -eta R_c, -eta R_{c+1} to the output wave (pair area h;
// lw = 16 lane, lr = 8 lane).
template <bool kDelta, bool kTok, bool kDot>
__device__ __forceinline__ void pair_step(WState& w, const PairRegs& r, const LaneConst& lc, lds_char* h, int lw,
                                          int lr, const lds_char* nb) {
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
  } else if (kDelta) {
    const u32x2 n00 = lds_load<u32x2>(nb + 8 * (lr >> 3));
    const u32x4 n1 = lds_load<u32x4>(nb + 512 + 16 * (lr >> 3));
    const float4_t x0 = kw_minus_v(r.k[0][0], r.k[0][1], r.v[0], wb0, wb1, lc);
    const float4_t x1 = kw_minus_v(r.k[1][0], r.k[1][1], r.v[1], wb0, wb1, lc);
    const uint32_t xa = pack_bf16(x0[0], x0[1]), xb = pack_bf16(x0[2], x0[3]);
    const u32x4 b0 = {xa, xb, 0u, 0u};
    const u32x4 b1 = {xa, xb, pack_bf16(x1[0], x1[1]), pack_bf16(x1[2], x1[3])};
    const u32x4 a0 = {n00.x, n00.y, 0u, 0u};
    r0 = MFMA32(bf8(a0), bf8(b0), x0, 0, 0, 0);
    r1 = MFMA32(bf8(n1), bf8(b1), x1, 0, 0, 0);
    rn0 = kTok ? neg_eta_bf16(r0, lc.neta, r.et[0]) : neg_eta_bf16(r0, lc.neta);
    rn1 = kTok ? neg_eta_bf16(r1, lc.neta, r.et[1]) : neg_eta_bf16(r1, lc.neta);
  } else {
    r0 = kw_minus_v(r.k[0][0], r.k[0][1], r.v[0], wb0, wb1, lc);
    const float4_t a1 = kw_minus_v(r.k[1][0], r.k[1][1], r.v[1], wb0, wb1, lc);
    // M^T = K_c K_{c+1}^T in the C layout is M as the A operand: lane (g, n) = M[n][4 g + s]
    float4_t mt = MFMA32(bf8(r.k[0][0]), bf8(r.k[1][0]), zero, 0, 0, 0);
    mt = MFMA32(bf8(r.k[0][1]), bf8(r.k[1][1]), mt, 0, 0, 0);
    rn0 = kTok ? neg_eta_bf16(r0, lc.neta, r.et[0]) : neg_eta_bf16(r0, lc.neta);
    const u32x4 mpad = {pack_bf16(mt[0], mt[1]), pack_bf16(mt[2], mt[3]), 0u, 0u};
    const u32x4 rpad0 = {rn0.x, rn0.y, 0u, 0u};
    r1 = MFMA32(bf8(mpad), bf8(rpad0), a1, 0, 0, 0);
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

// Delta rule, a Tm wave's work for one pair of chunks (a group has two pairs, one per Tm
// wave).  The pair's 32 tokens form one block (our derivation from the per-token write,
// exact algebra): with L = eta stril(K K^T) diag(rates) over the 32 tokens, Tm = (I + L)^-1
// is block lower triangular, its diagonal blocks T00, T11 are unit lower triangular (the
// inverses of the chunks' own I + L_qq) and T10 = -T11 L10 T00.  It writes N = Tm - I as the
// chain waves' A operands, lane-major: N00 over the first chunk's tokens (8 bytes per lane,
// row n, columns 4 g .. 4 g + 3) and [N10 | N11] over both chunks' tokens (16 bytes).
// A chunk's L is strictly lower triangular, so L^16 = 0 and
//     (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8)
// (each factor (I + L^(2^i)) times (I - L^(2^i)) leaves I - L^(2^(i+1))): three squarings and
// three products, all bf16 MFMAs with fp32 accumulation, entirely in registers.  Every
// matrix M is kept as two C-layout tiles, M (lane (g, n): M[4 g + e][n]) and M^T (lane (g, n):
// M[n][4 g + e]); the C layout of M is the B operand of a product over M's rows and the C
// layout of M^T the A operand over its columns, so (XY) = mfma(X^T, Y) and
// (XY)^T = mfma(Y, X^T).  L and L^T come from one Gram tile (K K^T is symmetric).
struct TmIn {
  u32x4 k[2][2];   // chunk q's K rows for lane (g, n): K[n][8 g .. + 7], K[n][32 + 8 g .. + 7]
  float4_t r4[2];  // chunk q's rates of tokens 4 g .. 4 g + 3 (ones without rates)
  float rn[2];     // chunk q's rate of token n
};
__device__ __forceinline__ u32x4 pk4(const float4_t& x) {
  const u32x4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), 0u, 0u};
  return u;
}
// T_q = (I + L_q)^-1 as the tiles T_q and T_q^T
__device__ __forceinline__ void tm_block(const u32x4& k0, const u32x4& k1, const float4_t& r4, float rn, float eta,
                                         int g, int n, float4_t& tC, float4_t& tT) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float4_t gq = MFMA32(bf8(k0), bf8(k0), zero, 0, 0, 0);
  gq = MFMA32(bf8(k1), bf8(k1), gq, 0, 0, 0);
  float4_t aC, aT, iC;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * g + e;
    aC[e] = (n < row) ? (eta * rn) * gq[e] : 0.0f;     // L[row][n], column rate r_n
    aT[e] = (row < n) ? (eta * r4[e]) * gq[e] : 0.0f;  // L[n][row] = eta r_row G[n][row]
    iC[e] = (row == n) ? 1.0f : 0.0f;
  }
  const u32x4 aCb = pk4(aC), aTb = pk4(aT);
  const float4_t a2C = MFMA32(bf8(aTb), bf8(aCb), zero, 0, 0, 0);
  const float4_t a2T = MFMA32(bf8(aCb), bf8(aTb), zero, 0, 0, 0);
  const u32x4 a2Cb = pk4(a2C), a2Tb = pk4(a2T);
  const float4_t a4C = MFMA32(bf8(a2Tb), bf8(a2Cb), zero, 0, 0, 0);
  const float4_t a4T = MFMA32(bf8(a2Cb), bf8(a2Tb), zero, 0, 0, 0);
  const u32x4 a4Cb = pk4(a4C), a4Tb = pk4(a4T);
  const float4_t a8C = MFMA32(bf8(a4Tb), bf8(a4Cb), zero, 0, 0, 0);
  const float4_t imaC = iC - aC, imaT = iC - aT;  // I - L and its transpose
  const u32x4 imaTb = pk4(imaT);
  const float4_t p1C = MFMA32(bf8(imaTb), bf8(a2Cb), imaC, 0, 0, 0);  // (I - L)(I + L^2)
  const float4_t p1T = MFMA32(bf8(a2Cb), bf8(imaTb), imaT, 0, 0, 0);
  const u32x4 p1Tb = pk4(p1T);
  const float4_t p2C = MFMA32(bf8(p1Tb), bf8(a4Cb), p1C, 0, 0, 0);  // ... (I + L^4)
  const float4_t p2T = MFMA32(bf8(a4Cb), bf8(p1Tb), p1T, 0, 0, 0);
  const u32x4 p2Tb = pk4(p2T), a8Cb = pk4(a8C);
  tC = MFMA32(bf8(p2Tb), bf8(a8Cb), p2C, 0, 0, 0);  // ... (I + L^8)
  tT = MFMA32(bf8(a8Cb), bf8(p2Tb), p2T, 0, 0, 0);
}
__device__ __forceinline__ void tm_pair(const TmIn& in, lds_char* nbuf, float eta, int lane) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const int g = lane >> 4;
  const int n = lane & 15;
  float4_t t0C, t0T, t1C, t1T;
  tm_block(in.k[0][0], in.k[0][1], in.r4[0], in.rn[0], eta, g, n, t0C, t0T);
  tm_block(in.k[1][0], in.k[1][1], in.r4[1], in.rn[1], eta, g, n, t1C, t1T);
  (void)t1C;
  // K_0 K_1^T in the C layout: lane (g, n) = G10[n][4 g + e], G10 = K_1 K_0^T, so the A
  // operand of L10 = eta G10 diag(rates of chunk 0) over chunk 0's tokens
  float4_t gt = MFMA32(bf8(in.k[0][0]), bf8(in.k[1][0]), zero, 0, 0, 0);
  gt = MFMA32(bf8(in.k[0][1]), bf8(in.k[1][1]), gt, 0, 0, 0);
  const float4_t r0 = in.r4[0];
  const u32x4 l10 = {pack_bf16(eta * r0[0] * gt[0], eta * r0[1] * gt[1]),
                     pack_bf16(eta * r0[2] * gt[2], eta * r0[3] * gt[3]), 0u, 0u};
  // P = L10 T00; T10^T = -(P^T)(T11^T), whose C layout is T10 as the A operand
  const float4_t pp = MFMA32(bf8(l10), bf8(pk4(t0C)), zero, 0, 0, 0);
  const u32x4 pa = {pack_bf16(-pp[0], -pp[1]), pack_bf16(-pp[2], -pp[3]), 0u, 0u};
  const u32x4 t11r = pk4(t1T);  // T11[n][4 g + e]
  const float4_t t10 = MFMA32(bf8(pa), bf8(t11r), zero, 0, 0, 0);
  // N = T - I over rows n, columns 4 g + e: T is unit lower triangular, so keep 4 g + e < n
  const uint32_t sm0 = (4 * g + 0 < n ? 0x0000FFFFu : 0u) | (4 * g + 1 < n ? 0xFFFF0000u : 0u);
  const uint32_t sm1 = (4 * g + 2 < n ? 0x0000FFFFu : 0u) | (4 * g + 3 < n ? 0xFFFF0000u : 0u);
  const u32x4 t00r = pk4(t0T);
  const u32x2 n00 = {t00r.x & sm0, t00r.y & sm1};
  const u32x4 n1 = {pack_bf16(t10[0], t10[1]), pack_bf16(t10[2], t10[3]), t11r.x & sm0, t11r.y & sm1};
  lds_store<u32x2>(nbuf + 8 * lane, n00);
  lds_store<u32x4>(nbuf + 512 + 16 * lane, n1);
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

// Roles of the waves (wave w runs on SIMD w % 4).  Plain: chain waves 0, 1; output waves
// 2, 3, 6, 7; loaders 4, 5.  The delta rule adds two Tm waves (one per pair of a group) and
// keeps them off the chain waves' SIMDs: chain waves 1, 2, each with a loader (5, 6) and an
// idle wave (9, 10: barriers only); Tm waves 0, 3, each with two output waves (4, 8 and 7, 11).
template <bool kDelta> struct Waves {
  static constexpr int kCount = kDelta ? 12 : kThreads / 64;
  static constexpr int kPerSimdMax = (kCount + 3) / 4;
  static constexpr int chain(int w) { return kDelta ? (w == 1 ? 0 : w == 2 ? 1 : -1) : (w < 2 ? w : -1); }
  static constexpr int loader(int w) { return kDelta ? (w == 5 ? 0 : w == 6 ? 1 : -1) : (w == 4 ? 0 : w == 5 ? 1 : -1); }
  // output wave (pr, hf) as pr + 2 hf
  static constexpr int output(int w) {
    return kDelta ? (w == 4 ? 0 : w == 7 ? 1 : w == 8 ? 2 : w == 11 ? 3 : -1)
                  : (w == 2 ? 0 : w == 3 ? 1 : w == 6 ? 2 : w == 7 ? 3 : -1);
  }
  // Tm wave for pair p of each group
  static constexpr int tm(int w) { return kDelta ? (w == 0 ? 0 : w == 3 ? 1 : -1) : -1; }
  static constexpr bool idle(int w) { return kDelta && (w == 9 || w == 10); }
};

template <bool kDelta, bool kTok, bool kDot>
__global__ __launch_bounds__(64 * Waves<kDelta>::kCount) __attribute__((amdgpu_waves_per_eu(
    Waves<kDelta>::kPerSimdMax - 1, Waves<kDelta>::kPerSimdMax))) void linear_mfma_kernel(LinearArgs a) {
  using RG = Ring<kDelta, kTok>;
  constexpr int kRing = RG::kRing;
  constexpr int kExtra = kDelta ? kNBytes : 0;
  __shared__ __attribute__((aligned(16))) char lds_mem[kRing * RG::kSlotBytes + kHandBytes + kStageBytes + kExtra];
  lds_char* ring = (lds_char*)(lds_mem);
  lds_char* hand = ring + kRing * RG::kSlotBytes;
  lds_char* stage = hand + kHandBytes;
  lds_char* nring = stage + kStageBytes;  // delta rule: N operands, then the Tm wave's scratch

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

  using WR = Waves<kDelta>;
  if (WR::loader(wv) >= 0) {
    // Loader waves: stream chunk c into ring slot c % kRing with direct-to-LDS loads, wave
    // loader wave p taking part p of every chunk (Q tile and V half tile; K tile with the
    // rate factors).  Lane l of a Q/K half tile fills physical piece l % 8 of row
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
    const char* esrc = kTok ? reinterpret_cast<const char*>(a.eta_tok + static_cast<size_t>(chain) * T) : nullptr;
    // Chain waves read chunks 0, 1 after barrier 0 and chunks up to kGroup b + kGroup + 1
    // after barrier b (one pair ahead); the delta rule's Tm wave reads chunks kGroup (b + 1) ..
    // kGroup b + 2 kGroup - 1 after barrier b; output waves read chunks kGroup (b - 1) .. kGroup b - 1
    // after barrier b.  So barrier b must publish the chunks up to kGroup b + kGroup + 1 + kAhead,
    // and from b = 2 on it frees the slots of the chunks up to kGroup b - kGroup - 1 (barriers 0
    // and 1 free nothing), after which each loader refills the ring up to chunk
    // kGroup b - kGroup - 1 + kRing.
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
    if (WR::loader(wv) == 0) {
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

  if (WR::idle(wv)) {
    for (int b = 0; b <= ngroups; ++b) lds_barrier();  // barriers 0 .. ngroups
    return;
  }
  if (WR::tm(wv) >= 0) {
    // Tm wave for pair tp of every group: the pair corrections N of group 0 from global memory
    // before barrier 0, then of group grp + 1 from the ring between barriers grp and grp + 1
    // (published at barrier grp), into N buffer (grp + 1) & 1, which the chain waves read
    // after barrier grp + 1.
    const int tp = WR::tm(wv);
    const float eta = a.eta;
    const float* etok = kTok ? a.eta_tok + static_cast<size_t>(chain) * T : nullptr;
    {
      const char* ksrc = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
      TmIn in;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = 2 * tp + q;
        const int off = c * kTileBytes;
        const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(ksrc + off, seq_bytes - off);
        in.k[q][0] = __builtin_amdgcn_raw_buffer_load_b128(rk, n * 128 + 16 * g, 0, 0);
        in.k[q][1] = __builtin_amdgcn_raw_buffer_load_b128(rk, n * 128 + 64 + 16 * g, 0, 0);
        in.r4[q] = float4_t{1.0f, 1.0f, 1.0f, 1.0f};
        in.rn[q] = 1.0f;
        if (kTok) {
          const __amdgpu_buffer_rsrc_t re = chunk_rsrc(etok + c * kB, (T - c * kB) * 4);
          in.r4[q] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(re, 16 * g, 0, 0));
          in.rn[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, 4 * n, 0, 0));
        }
      }
      tm_pair(in, nring + tp * kNPair, eta, lane);
    }
    lds_barrier();  // barrier 0
    for (int grp = 0; grp < ngroups; ++grp) {
      if (grp + 1 < ngroups) {
        const int c0 = kGroup * (grp + 1) + 2 * tp;
        TmIn in;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const lds_char* slot = ring + ((c0 + q) % kRing) * RG::kSlotBytes;
          in.k[q][0] = lds_load<u32x4>(slot + kTileBytes + o.ka0);
          in.k[q][1] = lds_load<u32x4>(slot + kTileBytes + o.ka1);
          in.r4[q] = kTok ? lds_load<float4_t>(slot + kEtaOff + 16 * g) : float4_t{1.0f, 1.0f, 1.0f, 1.0f};
          in.rn[q] = kTok ? lds_load<float>(slot + kEtaOff + 4 * n) : 1.0f;
        }
        tm_pair(in, nring + ((grp + 1) & 1) * kNGroup + tp * kNPair, eta, lane);
      }
      lds_barrier();  // barrier grp + 1
    }
    return;
  }

  if (WR::chain(wv) < 0) {
    // Output wave (pr, hf): chunk hf of pair pr of every group, Z columns 32 part .. + 31 (the
    // row blocks of both chain waves).  Lane (g, n) holds token n, columns 16 ow + 4 g .. + 3
    // of block ow; the wave restages the two blocks row-major in its own 1 KB of LDS and
    // stores 16 bytes per lane, 64 bytes of each of the chunk's 16 rows, non-temporal like
    // the loads (rows past T are dropped by the buffer range).  The stores of a block of kRing chunks share one buffer
    // resource, rebased once per block.
    const int pr = WR::output(wv) & 1;
    const bool hf = WR::output(wv) >= 2;
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
  const int cw = WR::chain(wv);
  const int i0 = kHalfCols * part + 16 * cw;
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
  o.vv = vswz(n, 2 * cw + (g >> 1)) * 16 + 8 * (g & 1);
  o.et = 16 * g;

  // Pair step p computes chunks 2p, 2p + 1 from registers read in step p - 1 while reading
  // chunks 2p + 2, 2p + 3.  Chunks past the end read as zeros and leave the state unchanged.
  lds_char* hw = hand + cw * kHandWave;
  lds_barrier();  // barrier 0: chunks 0 .. kGroup + 1 published
  PairRegs ra, rb;
  read_pair<kTok>(ra, ring, ring + RG::kSlotBytes, o);
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
        read_pair<kTok>(nxt, ring + s2 * RG::kSlotBytes, ring + s3 * RG::kSlotBytes, o);
        pair_step<kDelta, kTok, kDot>(wacc, cur, lc, hg + (x / 2) * kHandPair, lw, lr,
                                      nring + (grp & 1) * kNGroup + (x / 2) * kNPair);
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
  if (a.dot_loss) {
    if (a.eta_tok)
      hipLaunchKernelGGL((linear_mfma_kernel<false, true, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((linear_mfma_kernel<false, false, true>), grid, block, 0, s, a);
  } else {
    if (a.eta_tok)
      hipLaunchKernelGGL((linear_mfma_kernel<false, true, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((linear_mfma_kernel<false, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ delta rule

bool delta_fast_supported(const LinearArgs& a, bool bf16_io) {
  return bf16_io && mfma_shape_ok(a);
}

hipError_t launch_delta_fast(const LinearArgs& a, hipStream_t s) {
  const long long nmain = mfma_grid(a);
  if (nmain > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nmain)), block(64 * Waves<true>::kCount);
  if (a.eta_tok)
    hipLaunchKernelGGL((linear_mfma_kernel<true, true, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((linear_mfma_kernel<true, false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
