// TTT-Linear forward on the gfx950 matrix cores: d = 64, mini-batch b = 16, causal,
// bf16 Q/K/V/Z, fp32 state.
//
// Method (wmrh.cn summary of Sun et al. 2024, section 1.2.2, mini-batch TTT and its dual
// form; gradient (W k - v) k^T from the "Fast weights" page, section 1).  For a chunk with
// rows Q, K, V (16 x 64) and chunk-start weights W, with R = K W^T - V:
//     Z = Q W^T - eta * tril(Q K^T) R        (tril keeps the diagonal: z_t sees its own
//     W <- W - eta * R^T K                    update)
// which equals the per-token recurrence up to floating-point order.
//
// Mapping.  The linear model is separable by output row: row i of W only needs v[i].  One
// wave (one workgroup) owns 16 rows i0..i0+15 of one (batch, head) chain, so a chain is 4
// independent waves that never communicate; workgroup ids are ordered so that the four
// waves of a chain land on the same XCD and share its L2 for the Q/K re-reads.
// Within the wave everything stays in registers, in the layouts the MFMA operands need:
//   * the fp32 state W^T (64 x 16) is 4 accumulator tiles of v_mfma_f32_16x16x32_bf16;
//     tile jb, accumulator row m holds input index j = 4 m + jb;
//   * its bf16 copy is, lane for lane, the B operand of R = K W^T and the A operand of
//     Z^T = W Q^T (v_mfma_f32_16x16x32_bf16), with K and Q loaded in the matching order;
//   * R comes out with tokens as rows, which is the B operand of the rank-16 update
//     W^T += K^T (-eta R) and the A operand of the in-chunk correction (-eta R^T) P^T;
//   * P^T = K Q^T comes out as the B operand of that correction;
//   * -V enters R's accumulator through an MFMA with -I, which turns a row-major load of
//     V into the accumulator layout;
//   * products that contract over the 16 tokens use the same 16x16x32 instruction with the
//     upper half of every operand zero (see chunk_step);
//   * Z^T comes out with 4 consecutive output features per lane: one 8-byte store.
// Q/K/V of the next kPrefetch chunks are in flight in registers while a chunk computes.
#include "common.hpp"

namespace ttt {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;
constexpr int kB = 16;          // tokens per chunk
constexpr int kSlices = 4;      // waves (16 output rows each) per chain
constexpr int kPrefetch = 4;    // chunks in flight per wave

struct ChunkRegs {
  u32x4 ka0, ka1;  // K[t = n][16 g + 0..7], K[n][16 g + 8..15]: the two A operands of K W^T
  u32x4 qb0, qb1;  // Q[n][16 g + 0..7], Q[n][16 g + 8..15]
  uint32_t kt[4][2];  // kt[e][h] = K[4 g + e][c0 + 8 h .. + 1],  c0 = 16 (n / 4) + 2 (n % 4)
  u32x2 vv;        // V[n][i0 + 4 g .. 4 g + 3]
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

// Per-lane byte offsets inside a chunk (16 rows of 128 bytes), fixed for the whole kernel.
struct LaneOffsets {
  uint32_t row;      // n * 128 + 32 g          (K / Q operand rows)
  uint32_t kt[4];    // (4 g + e) * 128 + 2 c0
  uint32_t vz;       // n * 128 + 2 (i0 + 4 g)  (V load and Z store)
};

// Buffer resource over one chunk: base at the chunk, range = bytes left in the sequence,
// so rows past the end of the sequence read as zero and stores to them are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int left) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, left > 0 ? left : 0, 0x00020000);
}


__device__ __forceinline__ void load_chunk(ChunkRegs& r, __amdgpu_buffer_rsrc_t q,
                                           __amdgpu_buffer_rsrc_t k, __amdgpu_buffer_rsrc_t v,
                                           const LaneOffsets& o) {
  r.ka0 = __builtin_amdgcn_raw_buffer_load_b128(k, o.row, 0, 0);
  r.ka1 = __builtin_amdgcn_raw_buffer_load_b128(k, o.row + 16, 0, 0);
  r.qb0 = __builtin_amdgcn_raw_buffer_load_b128(q, o.row, 0, 0);
  r.qb1 = __builtin_amdgcn_raw_buffer_load_b128(q, o.row + 16, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.kt[e][0] = __builtin_amdgcn_raw_buffer_load_b32(k, o.kt[e], 0, 0);
    r.kt[e][1] = __builtin_amdgcn_raw_buffer_load_b32(k, o.kt[e] + 16, 0, 0);
  }
  r.vv = __builtin_amdgcn_raw_buffer_load_b64(v, o.vz, 0, 0);
}

// State: four fp32 accumulator tiles of W^T.  Tile jb = 2 h + p, row m of the tile holds
// input index j = 16 (m / 4) + 2 (m % 4) + 8 h + p, column n holds output row i0 + n; so
// lane (g, n), element e of tile 2h+p is W[i0 + n][16 g + 8 h + 2 e + p].
struct WState {
  float4_t t0, t1, t2, t3;
};

// Per-chunk values that do not depend on W, computed one chunk ahead.
struct Ahead {
  float4_t vneg;   // -V in the accumulator layout of R (rows t = 4g+e, column i0 + n)
  u32x4 pb;        // masked P^T = tril(Q K^T)^T as a padded bf16 B operand
  u32x4 kt0, kt1, kt2, kt3;  // K^T tiles (padded A operands of the update)
};

__device__ __forceinline__ bf16x8_t bf(const u32x4& x) { return __builtin_bit_cast(bf16x8_t, x); }

// Chunk-independent constants of a lane.
struct LaneConst {
  bf16x8_t neg_eye;        // -I as a padded B operand: slot s < 4 of lane (g, n) is row 4g+s
  uint32_t pmask0, pmask1; // causal mask of P^T on packed bf16 pairs (row 4g+e kept if <= n)
  float neta;
};

// W-independent work of a chunk: -V via an MFMA with -I, P^T = K Q^T with the causal mask,
// and the K^T gathers for the update.  Every accumulation chain in this file uses the one
// opcode v_mfma_f32_16x16x32_bf16 and the K = 16 products are zero-padded (chaining a
// 16x16x16 result into a 16x16x32 accumulator input was observed to read stale
// accumulator values on gfx950).
__device__ __forceinline__ void prepare(Ahead& a, const ChunkRegs& r, const LaneConst& lc) {
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const bf16x8_t ka0 = __builtin_bit_cast(bf16x8_t, r.ka0);
  const bf16x8_t ka1 = __builtin_bit_cast(bf16x8_t, r.ka1);
  const bf16x8_t qb0 = __builtin_bit_cast(bf16x8_t, r.qb0);
  const bf16x8_t qb1 = __builtin_bit_cast(bf16x8_t, r.qb1);
  const u32x4 vpad = {r.vv.x, r.vv.y, 0u, 0u};
  a.vneg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(vpad), lc.neg_eye, zero, 0, 0, 0);
  float4_t pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qb0, zero, 0, 0, 0);
  pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qb1, pacc, 0, 0, 0);
  a.kt0 = u32x4{__builtin_amdgcn_perm(r.kt[1][0], r.kt[0][0], kLo),
                __builtin_amdgcn_perm(r.kt[3][0], r.kt[2][0], kLo), 0u, 0u};
  a.kt1 = u32x4{__builtin_amdgcn_perm(r.kt[1][0], r.kt[0][0], kHi),
                __builtin_amdgcn_perm(r.kt[3][0], r.kt[2][0], kHi), 0u, 0u};
  a.kt2 = u32x4{__builtin_amdgcn_perm(r.kt[1][1], r.kt[0][1], kLo),
                __builtin_amdgcn_perm(r.kt[3][1], r.kt[2][1], kLo), 0u, 0u};
  a.kt3 = u32x4{__builtin_amdgcn_perm(r.kt[1][1], r.kt[0][1], kHi),
                __builtin_amdgcn_perm(r.kt[3][1], r.kt[2][1], kHi), 0u, 0u};
  a.pb = u32x4{pack_bf16(pacc[0], pacc[1]) & lc.pmask0, pack_bf16(pacc[2], pacc[3]) & lc.pmask1,
               0u, 0u};
}

// One chunk on the serial chain W -> R -> W, with the current chunk's output and the next
// chunk's W-independent work placed in the latency gaps.  Returns Z^T for the lane (4
// consecutive output features of token n) packed as bf16.  Scheduling barriers fix the
// phase order; inside a phase the compiler may reorder.
__device__ __forceinline__ u32x2 chunk_step(WState& w, Ahead& cur, Ahead& nxt_out,
                                            const ChunkRegs& r, const ChunkRegs& rn,
                                            const LaneConst& lc) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // bf16 copy of the chunk-start W^T in the B layout of K W^T: operand h, dword e holds
  // j = 16 g + 8 h + 2 e + {0, 1}, matching the contiguous K row loads.
  const bf16x8_t wb0 = as_bf16x8(pack_bf16(w.t0[0], w.t1[0]), pack_bf16(w.t0[1], w.t1[1]),
                                 pack_bf16(w.t0[2], w.t1[2]), pack_bf16(w.t0[3], w.t1[3]));
  const bf16x8_t wb1 = as_bf16x8(pack_bf16(w.t2[0], w.t3[0]), pack_bf16(w.t2[1], w.t3[1]),
                                 pack_bf16(w.t2[2], w.t3[2]), pack_bf16(w.t2[3], w.t3[3]));
  __builtin_amdgcn_sched_barrier(0);
  // R = K W^T - V (chain), then Z^T = W Q^T (off chain; fills the matrix pipe)
  float4_t racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, r.ka0), wb0, cur.vneg, 0, 0, 0);
  racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.ka1), wb1, racc,
                                                 0, 0, 0);
  float4_t zacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb0, __builtin_bit_cast(bf16x8_t, r.qb0),
                                                          zero, 0, 0, 0);
  zacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb1, __builtin_bit_cast(bf16x8_t, r.qb1), zacc,
                                                 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  // -eta R as a padded bf16 operand (chain)
  const u32x4 rbu = {pack_bf16(lc.neta * racc[0], lc.neta * racc[1]),
                     pack_bf16(lc.neta * racc[2], lc.neta * racc[3]), 0u, 0u};
  const bf16x8_t rb = bf(rbu);
  __builtin_amdgcn_sched_barrier(0);
  // W^T += K^T (-eta R) (chain), then the in-chunk correction Z^T += (-eta R)^T P^T
  w.t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(cur.kt0), rb, w.t0, 0, 0, 0);
  w.t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(cur.kt1), rb, w.t1, 0, 0, 0);
  w.t2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(cur.kt2), rb, w.t2, 0, 0, 0);
  w.t3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(cur.kt3), rb, w.t3, 0, 0, 0);
  zacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rb, bf(cur.pb), zacc, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  // next chunk's W-independent work (off chain)
  prepare(nxt_out, rn, lc);
  __builtin_amdgcn_sched_barrier(0);
  const u32x2 out = {pack_bf16(zacc[0], zacc[1]), pack_bf16(zacc[2], zacc[3])};
  return out;
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void linear_mfma_kernel(
    LinearArgs a, int nchains) {
  // Workgroup id -> (chain, slice): the 4 slices of a chain share id % 8 (one XCD).
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int rr = id >> 3;
  const int chain = (rr >> 2) * 8 + xcd;
  const int slice = rr & 3;
  if (chain >= nchains) return;

  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int i0 = 16 * slice;
  const int bi = chain / a.H;
  const int hi = chain - bi * a.H;
  const int T = a.T;
  const float neta = -a.eta;

  const size_t tok0 = static_cast<size_t>(chain) * static_cast<size_t>(T) * kD;
  const char* q = reinterpret_cast<const char*>(static_cast<const bf16*>(a.q) + tok0);
  const char* k = reinterpret_cast<const char*>(static_cast<const bf16*>(a.k) + tok0);
  const char* v = reinterpret_cast<const char*>(static_cast<const bf16*>(a.v) + tok0);
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
  o.row = n * 128 + 32 * g;
  const int c0 = 16 * (n >> 2) + 2 * (n & 3);
#pragma unroll
  for (int e = 0; e < 4; ++e) o.kt[e] = (4 * g + e) * 128 + 2 * c0;
  o.vz = n * 128 + 2 * (i0 + 4 * g);

  // All chunks go through one loop; chunks past the end of the sequence read zeros (their
  // residuals and updates are exactly zero) and their stores are dropped, which also
  // handles a ragged last chunk.  The loop runs whole rounds of kPrefetch chunks over a
  // ring of named register sets (no array, so nothing is demoted to memory).  Scheduling
  // barriers between chunks keep the compiler from hoisting work above a chunk's loads'
  // consumers, which would force a wait for the newest loads.
  static_assert(kPrefetch == 4, "the ring below is written out for 4 slots");
  constexpr int kChunkBytes = kB * kD * 2;
  const int seq_bytes = T * kD * 2;  // < 2^31: checked by linear_mfma_supported
  const int nchunks = (T + kB - 1) / kB;
  const int nrounds = (nchunks + kPrefetch - 1) / kPrefetch;
  ChunkRegs r0, r1, r2, r3;
  Ahead ah0, ah1;
#define TTT_LOAD(R, C)                                                              \
  {                                                                                 \
    const int off_ = (C) * kChunkBytes;                                             \
    load_chunk(R, chunk_rsrc(q + off_, seq_bytes - off_), chunk_rsrc(k + off_, seq_bytes - off_), \
               chunk_rsrc(v + off_, seq_bytes - off_), o);                          \
  }
  // chunk C is in ring slot R with its look-ahead values in A; RN holds chunk C+1 and AN
  // receives its look-ahead values.
#define TTT_STEP(R, RN, A, AN, C)                                                   \
  {                                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                              \
    const u32x2 zz_ = chunk_step(wacc, A, AN, R, RN, lc);                           \
    TTT_LOAD(R, (C) + kPrefetch)                                                    \
    const int zo_ = (C) * kChunkBytes;                                              \
    __builtin_amdgcn_raw_buffer_store_b64(zz_, chunk_rsrc(z + zo_, seq_bytes - zo_), o.vz, 0, 0); \
  }
  // Prologue loads in ring order (the loop-head wait must also hold on entry).
  TTT_LOAD(r0, 0)
  __builtin_amdgcn_sched_barrier(0);
  TTT_LOAD(r1, 1)
  __builtin_amdgcn_sched_barrier(0);
  TTT_LOAD(r2, 2)
  __builtin_amdgcn_sched_barrier(0);
  TTT_LOAD(r3, 3)
  __builtin_amdgcn_sched_barrier(0);
  prepare(ah0, r0, lc);
  for (int round = 0; round < nrounds; ++round) {
    const int c = round * kPrefetch;
    TTT_STEP(r0, r1, ah0, ah1, c + 0)
    TTT_STEP(r1, r2, ah1, ah0, c + 1)
    TTT_STEP(r2, r3, ah0, ah1, c + 2)
    TTT_STEP(r3, r0, ah1, ah0, c + 3)
  }
#undef TTT_LOAD
#undef TTT_STEP

  if (a.w_out) {
    float* wr = a.w_out + static_cast<size_t>(chain) * kD * kD + (i0 + n) * kD + 16 * g;
    *reinterpret_cast<float4_t*>(wr) = float4_t{wacc.t0[0], wacc.t1[0], wacc.t0[1], wacc.t1[1]};
    *reinterpret_cast<float4_t*>(wr + 4) = float4_t{wacc.t0[2], wacc.t1[2], wacc.t0[3], wacc.t1[3]};
    *reinterpret_cast<float4_t*>(wr + 8) = float4_t{wacc.t2[0], wacc.t3[0], wacc.t2[1], wacc.t3[1]};
    *reinterpret_cast<float4_t*>(wr + 12) = float4_t{wacc.t2[2], wacc.t3[2], wacc.t2[3], wacc.t3[3]};
  }
}

}  // namespace

bool linear_mfma_supported(const LinearArgs& a, bool bf16_io) {
  auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
  // 16-byte vector loads of tokens and of the fp32 state rows
  const bool aligned = al(a.q, 16) && al(a.k, 16) && al(a.v, 16) && al(a.z, 16) &&
                       al(a.w0, 16) && (a.w0_batch_stride % 4) == 0 &&
                       (a.w_out == nullptr || al(a.w_out, 16));
  // byte offsets inside one sequence are 32-bit
  const bool fits = static_cast<long long>(a.T) * kD * 2 + 2LL * kB * kD * 2 * kPrefetch < 0x7fffffffLL;
  return bf16_io && a.d == kD && a.chunk == kB && a.causal == 1 && a.T > 0 && aligned && fits;
}

hipError_t launch_linear_mfma(const LinearArgs& a, hipStream_t s) {
  const int nchains = a.B * a.H;
  const long long groups8 = (static_cast<long long>(nchains) + 7) / 8;
  const long long nwg = groups8 * 8 * kSlices;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_mfma_kernel, dim3(static_cast<unsigned>(nwg)), dim3(64), 0, s, a,
                     nchains);
  return hipGetLastError();
}

}  // namespace ttt
