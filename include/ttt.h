/*
 * ttt.h - C ABI of libttt.so, the MI355X (gfx950) TTT-layer forward pass.
 *
 * The method (test-time training layers): a small inner model f(k; W) is trained inside
 * the sequence by gradient descent on the reconstruction loss 1/2 ||f(k; W) - v||^2 and
 * every output reads the trained model, z_t = f(q_t; W_t).  Tokens are processed in
 * mini-batches ("chunks") of b consecutive tokens: every gradient of a chunk is taken at
 * the weights left by the previous chunk, and W_t = W_chunk - eta * sum_{s<=t} grad l_s.
 * b = 1 is the delta rule, one chunk of all tokens is batch gradient descent.
 *   - update / output rule: blog page "TTT: Test-Time Training", section TTT (general
 *     form); page "5.1 Fast weights and TTT layers", opening formula and section 1;
 *   - mini-batch rule: wmrh.cn summary of Sun et al. 2024, section 1.2.2 (mini-batch TTT);
 *   - non-causal full-batch use: ViT3 news page, section 1 (inner training setup).
 *
 * Conventions shared by every entry point
 *   - Token tensors q, k, v, z are dense row-major [B][H][T][d] in the I/O dtype
 *     (TTT_F32 = float32, TTT_BF16 = bfloat16).  They are device pointers (HIP global
 *     memory) owned by the caller; outputs must not overlap inputs.
 *   - States are float32, row-major, f(k; W) = W k with W[d_out][d_in]:
 *       linear: W [d][d];   MLP: W1 [dh][d], W2 [d][dh]  (f(k) = W2 SiLU(W1 k)).
 *     The initial state of (batch b, head h) starts at  base + b * batch_stride +
 *     h * (state size); batch_stride 0 shares one [H][...] state across the batch.
 *   - Final-state outputs (w_out, w1_out, w2_out) are dense [B][H][...] float32, or NULL.
 *   - eta is the scalar inner learning rate; chunk >= 1 (a chunk longer than T is one
 *     chunk of T tokens; when T is not a multiple of chunk the last chunk is shorter).
 *   - eta_tok (optional, NULL for none): per-token rate factors, float32 [B][H][T], a device
 *     pointer owned by the caller, 4-byte aligned.  Token t of (b, h) then learns at rate
 *     eta * eta_tok[(b H + h) T + t], and in a mini-batch each token's gradient carries its
 *     own rate: W_t = W_chunk - sum_{s<=t} eta_s grad l_s.  The "Fast weights" page writes
 *     the step with a per-step rate (opening formula); the wmrh.cn summary, section 2.2.3,
 *     makes it a function of the token, eta_base * sigmoid(theta . x_t), which a caller
 *     passes as eta = eta_base and eta_tok = sigmoid(theta . x_t).  The factors are read as
 *     they are (not validated on the host; non-finite factors give non-finite outputs).
 *   - loss (ttt_linear_fwd, ttt_mlp_fwd): TTT_LOSS_MSE, the reconstruction loss
 *     1/2 ||f(k; W) - v||^2 ("Fast weights" page, opening formula), or TTT_LOSS_DOT, the
 *     negative dot product -v^T f(k; W) (blog page, section TTT / 如何理解; the ViT3 news
 *     page, section 2, uses it for the vision model).  With TTT_LOSS_DOT the error term
 *     f(k; W) - v of every gradient becomes -v, so the gradients no longer depend on W.
 *   - epochs (ttt_linear_fwd, ttt_mlp_fwd): passes of mini-batch GD over all chunks, in
 *     order, each starting from the weights the previous pass left, before the outputs are
 *     read (ViT3 news page, observation 2 and its figure on inner batch size and epochs).
 *     epochs >= 1; epochs > 1 requires causal = 0 (TTT_E_INVALID otherwise), since a second
 *     pass would let a causal output see later tokens.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream).  Calls are
 *     asynchronous, never synchronise, keep no pointer after returning and are thread-safe;
 *     any workspace a call needs is allocated and released in stream order on `stream`,
 *     from a memory pool of the library's own per device that keeps the blocks it has
 *     handed out (so repeated calls map no new pages); that memory, at most the largest
 *     workspace in use at once, stays with the process until it ends.
 *   - Arguments are validated on the host before any HIP call.  Return values:
 *       TTT_OK             work enqueued;
 *       TTT_E_INVALID      a null required pointer, a non-positive size, chunk < 1, a
 *                          non-finite eta, a misaligned eta_tok, an unknown dtype or loss,
 *                          epochs < 1 (or > 1 with causal = 1), or a size overflow;
 *       TTT_E_UNSUPPORTED  a valid combination with no kernel (see each function);
 *       TTT_E_HIP          a HIP runtime error (launch failure, workspace allocation);
 *       TTT_E_NONFINITE    only with the finite check on (ttt_set_check_finite below): the
 *                          call ran and one of its outputs holds a NaN or an infinity.
 *     ttt_last_error() returns the calling thread's message for the last non-OK status.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* ttt_stream_t; /* identical to hipStream_t */

enum { TTT_OK = 0, TTT_E_INVALID = -1, TTT_E_UNSUPPORTED = -2, TTT_E_HIP = -3, TTT_E_NONFINITE = -4 };
enum { TTT_F32 = 0, TTT_BF16 = 1 };
enum { TTT_LOSS_MSE = 0, TTT_LOSS_DOT = 1 };

/*
 * TTT-Linear forward: f(k; W) = W k, reconstruction loss, mini-batch GD of size `chunk`.
 * Gradient (W k - v) k^T ("Fast weights" page, section 1).  causal = 1: z_t = W_t q_t with
 * W_t including the token's own update; causal = 0: every chunk is trained first (for
 * `epochs` passes) and all queries read the final W (ViT3 news page, section 1).
 *   q, k, v  [B][H][T][d] io_dtype            z      [B][H][T][d] io_dtype (out)
 *   w0       float32, per (b, h) a [d][d]     w_out  [B][H][d][d] float32 (out) or NULL
 * Supported: d in {16, 32, 64}, any chunk, both dtypes, causal 0/1.  T may be 0 (then z is
 * untouched and w_out receives the initial state).
 */
int ttt_linear_fwd(const void* q, const void* k, const void* v,
                   const float* w0, long long w0_batch_stride,
                   void* z, float* w_out,
                   int B, int H, int T, int d, int chunk, int causal, float eta,
                   const float* eta_tok, int loss, int epochs, int io_dtype,
                   ttt_stream_t stream);

/*
 * TTT-MLP forward: f(k; W1, W2) = W2 SiLU(W1 k) with hidden width dh, no bias (ViT3 news
 * page, section 2: 2-layer SiLU inner MLP), reconstruction loss, mini-batch GD.
 *   w1  float32, per (b, h) a [dh][d];  w2  float32, per (b, h) a [d][dh]; both use
 *   w_batch_stride as the distance between batch elements (0 = shared across the batch).
 *   w1_out [B][H][dh][d], w2_out [B][H][d][dh] float32 (out) or NULL.
 * Supported: d in {16, 32, 64}, 1 <= dh <= 512, any chunk, both dtypes, causal 0/1.
 * Some shapes use a device workspace that the call allocates and frees in stream order on
 * `stream` (hipMallocFromPoolAsync on the library's pool / hipFreeAsync; TTT_E_HIP if the
 * allocation fails).
 */
int ttt_mlp_fwd(const void* q, const void* k, const void* v,
                const float* w1, const float* w2, long long w_batch_stride,
                void* z, float* w1_out, float* w2_out,
                int B, int H, int T, int d, int dh, int chunk, int causal, float eta,
                const float* eta_tok, int loss, int epochs, int io_dtype,
                ttt_stream_t stream);

/*
 * The paper's instantiation of the inner model (wmrh.cn summary of Sun et al. 2024, section
 * 2.2.1: layer norm and a residual connection are always included, for stability):
 *   f(x) = x + LN(f_res(x)),   LN(y) = ln_weight * (y - mean(y)) / sqrt(var(y) + ln_eps) + ln_bias
 * over the d features of a token (biased variance).  ttt_linear_ln_fwd: f_res(x) = W x (the
 * paper's TTT-Linear); ttt_mlp_ln_fwd: f_res(x) = W2 GELU(W1 x) with GELU(u) = u Phi(u), Phi
 * the standard normal CDF (the paper's TTT-MLP, hidden width dh, 4 d in the paper).  The
 * loss, the update and output rules and every other argument are those of ttt_linear_fwd /
 * ttt_mlp_fwd; only W (W1, W2) is trained, the layer norm's parameters are fixed.
 *   ln_weight, ln_bias  float32 [H][d] device pointers (one gain and bias per head, shared
 *                       over the batch), owned by the caller;  ln_eps > 0 and finite.
 * Supported: as ttt_linear_fwd / ttt_mlp_fwd.  The causal d = 64, chunk 16, bf16 shape runs on
 * matrix-core kernels (and, for the MLP, hidden width 256), every other shape on the
 * vector-ALU kernels.
 * TTT_E_INVALID additionally for a null ln_weight / ln_bias or a bad ln_eps.
 */
int ttt_linear_ln_fwd(const void* q, const void* k, const void* v,
                      const float* w0, long long w0_batch_stride,
                      const float* ln_weight, const float* ln_bias, float ln_eps,
                      void* z, float* w_out,
                      int B, int H, int T, int d, int chunk, int causal, float eta,
                      const float* eta_tok, int loss, int epochs, int io_dtype,
                      ttt_stream_t stream);

int ttt_mlp_ln_fwd(const void* q, const void* k, const void* v,
                   const float* w1, const float* w2, long long w_batch_stride,
                   const float* ln_weight, const float* ln_bias, float ln_eps,
                   void* z, float* w1_out, float* w2_out,
                   int B, int H, int T, int d, int dh, int chunk, int causal, float eta,
                   const float* eta_tok, int loss, int epochs, int io_dtype,
                   ttt_stream_t stream);

/*
 * ttt_mlp_fwd / ttt_mlp_ln_fwd with a workspace owned by the caller, for the causal
 * d = 64, dh = 256, chunk 16, bf16 shape.  The layer's recursion (the gradients of the keys
 * and the state updates, wmrh.cn summary of Sun et al. 2024, section 1.2.2) does not depend
 * on the queries, so a kernel with two workgroups per (b, h) runs it on one compute unit and
 * forms the outputs on a second, which replays the same state updates from the operands the
 * first hands over through the workspace (18 KB per chunk of 16 tokens).  Results are
 * bit-identical to ttt_mlp_fwd / ttt_mlp_ln_fwd.
 *   workspace        device memory of at least ttt_mlp_fwd_workspace_size(...) bytes,
 *                    256-byte aligned, owned by the caller; its contents need no
 *                    initialisation and are left undefined.  One workspace serves one call
 *                    at a time: calls that may overlap (different streams) need their own.
 *   workspace_bytes  its size.
 * With workspace == NULL, for any other shape (for which ttt_mlp_fwd_workspace_size
 * returns 0), or with pointers the matrix-core kernels cannot take (q, k, v, z, w1, w2 and
 * the output states 16-byte aligned, w_batch_stride a multiple of 4, eta_tok 4-byte
 * aligned, as for ttt_mlp_fwd's matrix-core path), the call is ttt_mlp_fwd /
 * ttt_mlp_ln_fwd.  The call allocates nothing on the two-workgroup path.  TTT_E_INVALID
 * additionally for a workspace that is too small or misaligned.  Should the outputs' workgroup of a sequence ever wait past a bound (about a
 * second) for the operands, it fills that sequence's remaining outputs with NaN instead of
 * hanging (never observed: the recursion's workgroups are dispatched first and never wait).
 */
size_t ttt_mlp_fwd_workspace_size(int B, int H, int T, int d, int dh, int chunk, int causal,
                                  int io_dtype);
int ttt_mlp_fwd_ws(const void* q, const void* k, const void* v,
                   const float* w1, const float* w2, long long w_batch_stride,
                   void* z, float* w1_out, float* w2_out,
                   int B, int H, int T, int d, int dh, int chunk, int causal, float eta,
                   const float* eta_tok, int loss, int epochs, int io_dtype,
                   void* workspace, size_t workspace_bytes, ttt_stream_t stream);
int ttt_mlp_ln_fwd_ws(const void* q, const void* k, const void* v,
                      const float* w1, const float* w2, long long w_batch_stride,
                      const float* ln_weight, const float* ln_bias, float ln_eps,
                      void* z, float* w1_out, float* w2_out,
                      int B, int H, int T, int d, int dh, int chunk, int causal, float eta,
                      const float* eta_tok, int loss, int epochs, int io_dtype,
                      void* workspace, size_t workspace_bytes, ttt_stream_t stream);

/*
 * Delta rule (mini-batch of one token, causal): W_t = W_{t-1} + eta_t (v_t - W_{t-1} k_t) k_t^T,
 * z_t = W_t q_t ("Fast weights" page, section 1), eta_t = eta or eta * eta_tok[t].  Same
 * arguments as ttt_linear_fwd without chunk / causal.  Supported: d in {16, 32, 64}, both
 * dtypes.  No workspace: the call allocates nothing.
 */
int delta_rule_fwd(const void* q, const void* k, const void* v,
                   const float* w0, long long w0_batch_stride,
                   void* z, float* w_out,
                   int B, int H, int T, int d, float eta, const float* eta_tok,
                   int io_dtype, ttt_stream_t stream);

/*
 * Backward pass of the causal TTT-Linear layer: the gradients the outer loop needs to train
 * the projections, the initial state and per-token rates through the inner updates
 * (wmrh.cn summary of Sun et al. 2024, sections 2.2 and 2.2.3; "Fast weights" page, opening
 * paragraph).  For the forward call ttt_linear_fwd(q, k, v, w0, ..., chunk, causal = 1, eta,
 * eta_tok, loss, 1) (loss TTT_LOSS_MSE or TTT_LOSS_DOT) and upstream gradients dz of z and
 * dw_out of the final state, writes
 *   dq, dk, dv  [B][H][T][d] io_dtype (out)
 *   dw0         [B][H][d][d] float32 (out): per (b, h) sequence; when w0 is shared over the
 *               batch (w0_batch_stride 0) its gradient is the sum of dw0 over b.
 *   deta_tok    [B][H][T] float32 (out) or NULL: the gradient of the per-token rate factors
 *               eta_tok [B][H][T] (or NULL: the scalar rate); needs eta_tok.
 *   dz          [B][H][T][d] io_dtype;  dw_out [B][H][d][d] float32 or NULL (zero).
 * Supported: d in {16, 32, 64}, chunks of at most 16 tokens (min(chunk, T) <= 16), both
 * dtypes.  The call recomputes the forward pass and keeps its chunk-start states in a
 * stream-ordered workspace: bf16 on the matrix cores (d = 64, chunk 16, bf16, with q, k, v,
 * dz, dq, dk, dv, dw0, dw_out and w0 16-byte aligned and w0_batch_stride a multiple of 4;
 * B*H*ceil(T/16)*8 KB), else float32 (B*H*ceil(T/chunk)*d*d*4 bytes).  chunk = 1 (the delta
 * rule) runs the exact chunked form 16 tokens at a time on the matrix cores in fp32, keeping
 * per 16 tokens the float32 state and the chunk's two 16 x 16 matrices (B*H*ceil(T/16)*
 * (d*d + 512)*4 bytes).  T = 0 copies dw_out to dw0 (zeros without it).
 */
int ttt_linear_bwd(const void* q, const void* k, const void* v,
                   const float* w0, long long w0_batch_stride,
                   const void* dz, const float* dw_out,
                   void* dq, void* dk, void* dv, float* dw0,
                   int B, int H, int T, int d, int chunk, float eta,
                   const float* eta_tok, float* deta_tok, int loss,
                   int io_dtype, ttt_stream_t stream);

/*
 * ttt_linear_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc): the same
 * arguments, results and supported shapes, but the chunk-start state history lives in a
 * fixed scratch array of the library (64 MiB, one per GPU, held until the process ends)
 * instead of a stream-ordered workspace, and the call allocates nothing.  A call whose
 * history would exceed it (matrix-core path: B*H*ceil(T/16)*8 KB; vector-ALU path:
 * B*H*ceil(T/chunk)*d*d*4 bytes; chunk 1: B*H*ceil(T/16)*(d*d + 512)*4 bytes) returns
 * TTT_E_UNSUPPORTED.  Every call on one GPU shares the
 * array: calls that overlap on one GPU (on different streams) race and must be ordered by the
 * caller.
 */
int ttt_linear_bwd_noalloc(const void* q, const void* k, const void* v,
                           const float* w0, long long w0_batch_stride,
                           const void* dz, const float* dw_out,
                           void* dq, void* dk, void* dv, float* dw0,
                           int B, int H, int T, int d, int chunk, float eta,
                           const float* eta_tok, float* deta_tok, int loss,
                           int io_dtype, ttt_stream_t stream);

/*
 * Backward pass of the causal TTT-MLP layer (f(k) = W2 SiLU(W1 k)), the MLP counterpart of
 * ttt_linear_bwd.  For the forward call ttt_mlp_fwd(q, k, v, w1, w2, ..., chunk, causal = 1,
 * eta, eta_tok, loss, 1) (loss TTT_LOSS_MSE or TTT_LOSS_DOT; any other value is
 * TTT_E_INVALID) and upstream gradients dz of z and dw1_out, dw2_out of the final states,
 * writes
 *   dq, dk, dv  [B][H][T][d] io_dtype (out)
 *   dw1 [B][H][dh][d], dw2 [B][H][d][dh] float32 (out), per (b, h) sequence (sum over b for a
 *               state shared over the batch).
 *   deta_tok    [B][H][T] float32 (out) or NULL: the gradient of the per-token rate factors
 *               eta_tok [B][H][T] (or NULL: the scalar rate); needs eta_tok.
 *   dz [B][H][T][d] io_dtype;  dw1_out, dw2_out float32 of the same shapes as dw1, dw2, or
 *   NULL (zero).
 * Supported: d in {16, 32, 64}, 1 <= dh <= 256, chunks of at most 16 tokens, both dtypes.  The
 * call recomputes the forward pass and keeps its chunk-start states in a stream-ordered
 * workspace: bf16 with d = 64, dh = 256, chunk = 16, TTT_LOSS_MSE, no eta_tok and 16-byte
 * aligned buffers (matrix cores; B*H*ceil(T/16)*64 KB), else float32 (B*H*ceil(T/chunk)*2*d*dh*4 bytes, plus the
 * forward's 4*d*dh*4 bytes per sequence).  T = 0 copies dw1_out, dw2_out to dw1, dw2 (zeros
 * without them).
 */
int ttt_mlp_bwd(const void* q, const void* k, const void* v,
                const float* w1, const float* w2, long long w_batch_stride,
                const void* dz, const float* dw1_out, const float* dw2_out,
                void* dq, void* dk, void* dv, float* dw1, float* dw2,
                int B, int H, int T, int d, int dh, int chunk, float eta,
                const float* eta_tok, float* deta_tok,
                int loss, int io_dtype, ttt_stream_t stream);

/*
 * Backward pass of the paper's causal TTT-Linear layer, f(x) = x + LN(W x) (wmrh.cn summary
 * of Sun et al. 2024, section 2.2.1), the counterpart of ttt_linear_bwd for the forward call
 * ttt_linear_ln_fwd(q, k, v, w0, ..., ln_weight, ln_bias, ln_eps, ..., chunk, causal = 1,
 * eta, eta_tok, loss, 1).  Besides dq, dk, dv, dw0 and deta_tok (as ttt_linear_bwd) writes
 *   dln_weight, dln_bias  [B][H][d] float32 (out): the gradients of the layer norm's gain and
 *               bias, per (b, h) sequence (sum over b for the per-head parameters).
 * Supported: d in {16, 32, 64}, chunks of at most 16 tokens, either loss, both dtypes, on the
 * vector ALUs; the call recomputes the forward pass and keeps its float32 chunk-start states
 * in a stream-ordered workspace (B*H*ceil(T/chunk)*d*d*4 bytes).  T = 0 copies dw_out to dw0
 * and zeroes dln_weight, dln_bias.
 */
int ttt_linear_ln_bwd(const void* q, const void* k, const void* v,
                      const float* w0, long long w0_batch_stride,
                      const float* ln_weight, const float* ln_bias, float ln_eps,
                      const void* dz, const float* dw_out,
                      void* dq, void* dk, void* dv, float* dw0,
                      float* dln_weight, float* dln_bias,
                      int B, int H, int T, int d, int chunk, float eta,
                      const float* eta_tok, float* deta_tok, int loss,
                      int io_dtype, ttt_stream_t stream);

/*
 * Backward pass of the paper's causal TTT-MLP layer, f(x) = x + LN(W2 GELU(W1 x)), the
 * counterpart of ttt_mlp_bwd for the forward call ttt_mlp_ln_fwd(q, k, v, w1, w2, ...,
 * ln_weight, ln_bias, ln_eps, ..., chunk, causal = 1, eta, eta_tok, loss, 1).  Besides dq,
 * dk, dv, dw1, dw2 and deta_tok (as ttt_mlp_bwd) writes dln_weight, dln_bias [B][H][d]
 * float32 (out), per (b, h) sequence.  Supported: d in {16, 32, 64}, 1 <= dh <= 256, chunks
 * of at most 16 tokens, either loss, both dtypes, on the vector ALUs; the call recomputes the
 * forward pass and keeps its float32 chunk-start states in a stream-ordered workspace
 * (B*H*ceil(T/chunk)*2*d*dh*4 bytes, plus the forward's 4*d*dh*4 bytes per sequence).
 * T = 0 copies dw1_out, dw2_out and zeroes dln_weight, dln_bias.
 */
int ttt_mlp_ln_bwd(const void* q, const void* k, const void* v,
                   const float* w1, const float* w2, long long w_batch_stride,
                   const float* ln_weight, const float* ln_bias, float ln_eps,
                   const void* dz, const float* dw1_out, const float* dw2_out,
                   void* dq, void* dk, void* dv, float* dw1, float* dw2,
                   float* dln_weight, float* dln_bias,
                   int B, int H, int T, int d, int dh, int chunk, float eta,
                   const float* eta_tok, float* deta_tok, int loss,
                   int io_dtype, ttt_stream_t stream);

/*
 * Backward pass of the non-causal TTT layers: the layer trains on every pair first (steps of
 * mini-batch GD over the chunks, `epochs` passes) and then every query reads the final
 * weights (ViT3 news page, section 1, observation 2); the outer loop trains the projections,
 * the initial state and the rates through those steps (wmrh.cn summary of Sun et al. 2024,
 * sections 2.2 and 2.2.3; "Fast weights" page, section 2).  For the forward call
 * ttt_linear_fwd(q, k, v, w0, ..., chunk, causal = 0, eta, eta_tok, loss, epochs), resp.
 * ttt_mlp_fwd(q, k, v, w1, w2, ..., chunk, causal = 0, eta, eta_tok, loss, epochs), and the
 * upstream gradients dz of z and dw_out (dw1_out, dw2_out) of the final states, writes
 *   dq, dk, dv  [B][H][T][d] io_dtype (out)
 *   dw0 [B][H][d][d] (linear) or dw1 [B][H][dh][d], dw2 [B][H][d][dh] (MLP), float32 (out),
 *               per (b, h) sequence (sum over b for a state shared over the batch)
 *   deta_tok    [B][H][T] float32 (out) or NULL: the gradient of the per-token rate factors
 *               eta_tok (needs eta_tok)
 *   dz [B][H][T][d] io_dtype;  dw_out / dw1_out, dw2_out float32 or NULL (zero).
 * Supported: d in {16, 32, 64}, 1 <= dh <= 256 (MLP, SiLU), any chunk >= 1 and epochs >= 1,
 * TTT_LOSS_MSE or TTT_LOSS_DOT, both dtypes, on the vector ALUs (one workgroup per sequence).
 * The call keeps every step-start state and fp32 accumulators of dk, dv and deta_tok in a
 * stream-ordered workspace of B*H*((S+1)*state + 2*T*d + T)*4 bytes, S = ceil(T/chunk)*epochs
 * steps and state = d*d (linear) or 2*d*dh (MLP) floats.  One exception: d = 64 (and dh = 64
 * for the MLP), bf16, one full-batch step (chunk >= T, epochs = 1), 16 <= T <= 256 and
 * 16-byte aligned q, k, v, dz, dq, dk, dv, states and state gradients (batch stride a
 * multiple of 4) runs on the matrix cores with no workspace.  T = 0 copies the upstream state
 * gradients (zeros without them).
 */
int ttt_linear_nc_bwd(const void* q, const void* k, const void* v,
                      const float* w0, long long w0_batch_stride,
                      const void* dz, const float* dw_out,
                      void* dq, void* dk, void* dv, float* dw0,
                      int B, int H, int T, int d, int chunk, int epochs, float eta,
                      const float* eta_tok, float* deta_tok, int loss,
                      int io_dtype, ttt_stream_t stream);
int ttt_mlp_nc_bwd(const void* q, const void* k, const void* v,
                   const float* w1, const float* w2, long long w_batch_stride,
                   const void* dz, const float* dw1_out, const float* dw2_out,
                   void* dq, void* dk, void* dv, float* dw1, float* dw2,
                   int B, int H, int T, int d, int dh, int chunk, int epochs, float eta,
                   const float* eta_tok, float* deta_tok, int loss,
                   int io_dtype, ttt_stream_t stream);

/* Message for the calling thread's last non-OK status ("" if none).  Owned by the library;
   valid until the thread's next call into it. */
const char* ttt_last_error(void);

/*
 * Finite check of the outputs, for debugging (no page describes it; a layer whose inner
 * updates diverge, as the raw-key MLP workloads do at large rates, fills its outputs with
 * NaN or infinities, and this names where).  When it is on, every call that would return
 * TTT_OK then scans each of its outputs on its stream (z, final states, gradients; token
 * outputs only when T > 0), waits for the stream, and returns TTT_E_NONFINITE with the
 * first output holding a NaN or an infinity named in ttt_last_error().  Calls with the
 * check on are therefore synchronous, and calls with it on that overlap on one GPU share
 * that GPU's flags and can report each other's outputs.  Off by default; a non-empty
 * environment variable TTT_CHECK_FINITE other than "0" turns it on for the process.
 * ttt_set_check_finite(on) sets it for the process (nonzero = on) and returns the previous
 * setting; ttt_get_check_finite() returns the current one (1 or 0).  Neither touches the GPU.
 */
int ttt_set_check_finite(int on);
int ttt_get_check_finite(void);

/*
 * Debug switches of the two-workgroup MLP kernel (ttt_mlp_fwd_ws, ttt_mlp_ln_fwd_ws), for
 * tests of its paths that a normal run does not take; set for the process, read at each
 * call.  TTT_SPLIT_FORMAL: hand off with agent-scope release and acquire on every chunk, the
 * path taken when the two workgroups of a sequence sit on different XCCs (results are
 * identical, the call is slower).  TTT_SPLIT_TEST_ABORT: the output workgroups wait for a
 * tag the recursion never writes, with a bound of 64 polls, so that they take the failure
 * path at once: every z of the call is NaN, the final states are right, and the call returns
 * TTT_OK.  Returns the previous flags; 0 turns both off.
 */
enum { TTT_SPLIT_FORMAL = 1, TTT_SPLIT_TEST_ABORT = 2 };
int ttt_set_split_debug(int flags);

/* ABI version of this header (incremented on any incompatible change). */
int ttt_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
