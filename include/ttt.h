/*
 * ttt.h -- C ABI of the TTT-layer forward library for AMD Instinct MI355X (gfx950).
 *
 * A TTT ("test-time training") layer keeps, per attention head, a small inner model W that is
 * trained at inference time on the layer's keys and values and then applied to its queries
 * (ViT^3 review on techloop.online, "core idea" section: train F on (K, V), obtain W*, output
 * F_{W*}(Q); TTT-Linear / TTT-MLP abstract: the hidden state is a model and its update rule a
 * step of self-supervised learning). Each entry point below runs one layer forward.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes and layout.  q, k, v and o are [B, N, H, D] row-major with D contiguous, i.e. token n of
 *   batch b holds the H heads' D-vectors back to back (C = H*D channels, as a QKV projection
 *   emits them). Element type is `dt`: TTT_BF16 (bfloat16) or TTT_F32.
 *   Inner states are always fp32, row-major, rows = input features: the linear model predicts
 *   k . W with W [D, D]; the MLP predicts GELU(k . W1) . W2 with W1 [D, Dh], W2 [Dh, D].
 *   An initial state pointer covers [H, ...] when its batch stride is 0 (one state shared by
 *   all batch elements) or [B, H, ...] when the stride (in elements) is at least
 *   H * (elements of one head's state) and a multiple of 4, which keeps each batch element's
 *   states 16-byte aligned.
 * Loss and step.  Per token l(W) = 1/2 ||f_W(k) - v||^2; a step over n tokens is
 *   W <- W - (eta/n) * sum of the n per-token gradients (gradient-descent update rule of the
 *   Vision-TTT summary on gist.science, "Methodologie" item 1; mini-batches of item 3).
 * Pointers.  q, k, v, o, w*, w*_out and workspace are DEVICE pointers owned by the caller;
 *   nothing is retained after return and the library never allocates memory. `stream` is a
 *   hipStream_t (NULL = the default stream). All work is enqueued asynchronously on it; results
 *   are valid once the stream has synchronised. No host synchronisation happens inside.
 * Aliasing.  q == k is allowed (Vision-TTT shares its Q/K projection); o and the *_out states
 *   must not overlap any input or each other.
 * Alignment.  q, k, v, o must be 16-byte aligned; states and workspace 16-byte aligned.
 * Errors.  Every argument is validated before anything is enqueued; on error nothing is
 *   enqueued and no output is touched.
 *     TTT_ERR_INVALID      null pointer, non-positive size, N not a multiple of chunk,
 *                          misaligned pointer or batch stride, overlapping output, non-finite eta
 *     TTT_ERR_UNSUPPORTED  D not in {16, 32, 64}; chunk not in {16, 32, 64};
 *                          TTT-MLP with Dh not a multiple of 64 in [64, 1024]
 *     TTT_ERR_WORKSPACE    workspace_bytes < ttt_workspace_size(...)
 *     TTT_ERR_HIP          a HIP launch error reported right after enqueueing
 * Workspace.  Scratch device memory of at least ttt_workspace_size(...) bytes (may be NULL when
 *   that size is 0). It needs no initialisation and holds garbage afterwards. Calls that share
 *   one workspace must be ordered on one stream; calls on different streams need separate
 *   workspaces.
 * Precision.  TTT_F32 computes in fp32 throughout (plain FMA, no reduced-precision operands).
 *   TTT_BF16 reads and writes bf16 (round-to-nearest-even on output), keeps the state and every
 *   accumulator in fp32, and feeds 16-bit operands to the matrix cores: bf16, except in
 *   ttt_mlp_forward's products on the W2 side (hidden activations, W2, residuals), which take
 *   fp16 operands (more mantissa bits) while the values converted stay inside the ranges that
 *   ttt_mlp_forward states; chains whose values leave them are recomputed with bf16 operands.
 * Threads.  Entry points are reentrant and keep no state between calls. How a call splits its work
 *   (token splits, scan segments) is a function of its sizes only, never of the device it runs
 *   on, so workspace sizes and results are the same on every device.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTT_OK = 0,
  TTT_ERR_INVALID = 1,
  TTT_ERR_UNSUPPORTED = 2,
  TTT_ERR_WORKSPACE = 3,
  TTT_ERR_HIP = 4
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

typedef enum {
  TTT_OP_FULLBATCH = 0,
  TTT_OP_CAUSAL = 1,
  TTT_OP_BIDIR = 2,
  TTT_OP_MLP = 3,
  TTT_OP_FULLBATCH_BWD = 4,
  TTT_OP_BIDIR2D = 5,
  TTT_OP_CAUSAL_BWD = 6,
  TTT_OP_BIDIR_BWD = 7
} ttt_op;

/*
 * Single-epoch, full-batch inner step (ViT^3 review on techloop.online, design-space study: one
 * epoch, full batch, inner learning rate 1.0). Per (b, h):
 *   W* = W0 - (eta/N) K^T (K W0 - V),   O = Q W*.
 * w_out (nullable): fp32 [B, H, D, D] receives W*.
 */
ttt_status ttt_forward_fullbatch(ttt_dtype dt, int B, int H, int N, int D, float eta,
                                 const void* q, const void* k, const void* v,
                                 const float* w0, long long w0_batch_stride,
                                 void* o, float* w_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of ttt_forward_fullbatch for the outer training loop: given d_o = dL/dO, the
 * gradients of L with respect to q, k, v and W0, in closed form (the pages' authors also write
 * the inner gradient by hand: ViT^3 review on techloop.online, section on the official code).
 * With s = eta/N, W* as in the forward, G = Q^T dO and M = W0 G^T + G W0^T, per (b, h):
 *   dQ = dO W*^T,   dK = -s (K M - V G^T),   dV = s K G,   dW0 = G - s (K^T K) G.
 * d_o, d_q, d_k, d_v: [B, N, H, D] of dtype dt; d_w0: fp32 [B, H, D, D], per batch element even
 * when W0 is shared (w0_batch_stride 0): the caller then sums it over the batch. Outputs must not
 * overlap any input or each other. Workspace: ttt_workspace_size(TTT_OP_FULLBATCH_BWD, ...).
 */
ttt_status ttt_backward_fullbatch(ttt_dtype dt, int B, int H, int N, int D, float eta,
                                  const void* q, const void* k, const void* v,
                                  const float* w0, long long w0_batch_stride, const void* d_o,
                                  void* d_q, void* d_k, void* d_v, float* d_w0,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Several full-batch epochs before the read-out (ViT^3 review on techloop.online, design-space
 * study: how many epochs one inner update runs). Per (b, h), from W_0 = W0:
 *   W_{e+1} = W_e - (eta/N) K^T (K W_e - V)   for e < epochs,   O = Q W_epochs.
 * epochs = 1 is ttt_forward_fullbatch. The epochs reuse the one pass over K and V (K^T K and K^T V
 * are summed once), so their cost is a few d x d products per (b, h). epochs < 1 is
 * TTT_ERR_INVALID, above 256 TTT_ERR_UNSUPPORTED. Workspace as for ttt_forward_fullbatch.
 */
ttt_status ttt_forward_fullbatch_epochs(ttt_dtype dt, int B, int H, int N, int D, int epochs,
                                        float eta, const void* q, const void* k, const void* v,
                                        const float* w0, long long w0_batch_stride,
                                        void* o, float* w_out,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal mini-batch TTT-Linear (TTT-Linear / TTT-MLP abstract; mini-batches of b = chunk tokens,
 * Vision-TTT summary "Methodologie" item 3). Per (b, h), for consecutive chunks c of b tokens
 * with start state W_s:
 *   o_i = q_i (W_s - (eta/b) sum_{j <= i in c} k_j^T (k_j W_s - v_j))     (own token included)
 *   W_next = W_s - (eta/b) K_c^T (K_c W_s - V_c).
 * w_out (nullable): fp32 [B, H, D, D] receives the state after the last chunk, so a sequence can
 * be continued by a later call with w0 = w_out and w0_batch_stride = H*D*D.
 */
ttt_status ttt_forward_chunked_causal(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                      float eta, const void* q, const void* k, const void* v,
                                      const float* w0, long long w0_batch_stride,
                                      void* o, float* w_out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of ttt_forward_chunked_causal for the outer training loop: given d_o = dL/dO, the
 * gradients of L with respect to q, k, v and W0 (closed form, in the style of the hand-written
 * inner gradient of the ViT^3 review on techloop.online, section on the official code). Per chunk
 * with start state W, a = eta/b, E = K W - V, S = tril(Q K^T) and lam = dL/d(the state the chunk
 * hands on):
 *   dE = -a (S^T dO + K lam),   dS = -a tril(dO E^T),
 *   dQ = dO W^T + dS K,   dK = dE W^T + dS^T Q - a E lam^T,   dV = -dE,
 *   dL/dW (for the chunk before) = lam + Q^T dO + K^T dE.
 * Arguments as for ttt_backward_fullbatch plus chunk (16, 32 or 64, dividing N): d_o, d_q, d_k,
 * d_v [B, N, H, D] of dtype dt; d_w0 fp32 [B, H, D, D] per batch element (summed by the caller
 * when W0 is shared). No gradient flows in through the end state (w_out of the forward). Outputs
 * must not overlap any input or each other. Workspace: ttt_workspace_size(TTT_OP_CAUSAL_BWD, ...,
 * chunk), which may be 0 (then workspace may be NULL).
 */
ttt_status ttt_backward_chunked_causal(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                       float eta, const void* q, const void* k, const void* v,
                                       const float* w0, long long w0_batch_stride,
                                       const void* d_o, void* d_q, void* d_k, void* d_v,
                                       float* d_w0, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * Bidirectional chunked scan (Vision-TTT summary on gist.science, "Methodologie" item 2: tokens
 * are scanned forwards and backwards; item 3: mini-batches). Per (b, h): a forward scan over
 * chunks of b tokens, W_c = W_{c-1} - (eta/b) K_c^T (K_c W_{c-1} - V_c) from W_{-1} = W0, reads
 * out each chunk after its own update (non-causal inside the chunk), O^f_c = Q_c W_c; a second
 * scan does the same on the token-reversed sequence from the same W0; the output is
 *   O = O^f + (reverse-scan outputs put back in token order).
 * w_out (nullable): fp32 [2, B, H, D, D]: [0] the forward scan's end state, [1] the reverse's.
 */
ttt_status ttt_forward_chunked_bidir(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                     float eta, const void* q, const void* k, const void* v,
                                     const float* w0, long long w0_batch_stride,
                                     void* o, float* w_out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of ttt_forward_chunked_bidir: the gradients of both scans summed (each reads the
 * same q, k, v and W0 and receives the same d_o). Each scan reads out after its chunk's update, so
 * per chunk (in that scan's order) with lam' = lam + Q^T dO and W_c the state after the chunk:
 *   dE = -a K lam',   dQ = dO W_c^T,   dK = dE W^T - a E lam'^T,   dV = -dE,
 *   dL/dW (for the chunk before) = lam' + K^T dE.
 * Arguments, layouts and errors as for ttt_backward_chunked_causal; workspace:
 * ttt_workspace_size(TTT_OP_BIDIR_BWD, ..., chunk) (nonzero: it holds one scan's partial sums).
 */
ttt_status ttt_backward_chunked_bidir(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                      float eta, const void* q, const void* k, const void* v,
                                      const float* w0, long long w0_batch_stride,
                                      const void* d_o, void* d_q, void* d_k, void* d_v,
                                      float* d_w0, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * 2-D bidirectional layer: the bidirectional scan of ttt_forward_chunked_bidir over the tokens in
 * raster order plus the same scan over the tokens in column order (top to bottom, column by
 * column: the Vision-TTT summary on gist.science, "De Oplossing", has the scanner read the image
 * top to bottom as well), summed; all four directions start from W0. The N = height * width
 * tokens of each batch element are an image in raster order (token i * width + j is pixel (i, j)).
 * w_out (nullable): fp32 [4, B, H, D, D]: raster forward end, raster reverse end, column forward
 * end, column reverse end. Workspace: ttt_workspace_size(TTT_OP_BIDIR2D, ..., N, D, 0, chunk) with
 * N = height * width: for bf16 I/O the scans' own workspace (the column-order scan reads q, k, v in
 * place and adds its output into o; null is accepted when the size is 0), for fp32 I/O also
 * column-order copies of the inputs and output. The column-order sum is rounded once: o = bf16(raster
 * result + column result), each term as the bidirectional scan rounds it.
 */
ttt_status ttt_forward_chunked_bidir2d(ttt_dtype dt, int B, int H, int height, int width, int D,
                                       int chunk, float eta, const void* q, const void* k,
                                       const void* v, const float* w0, long long w0_batch_stride,
                                       void* o, float* w_out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal mini-batch TTT-MLP (TTT-Linear / TTT-MLP abstract: the hidden state is a two-layer
 * MLP). f(x) = GELU(x W1) W2 with exact erf GELU and no bias. Per (b, h) and chunk c with start
 * state (W1_s, W2_s): token i is read out with (W1_s, W2_s) - (eta/b) * sum_{j <= i in c} of the
 * per-token gradients at the start state; the chunk hands on the state after all b gradients.
 * w1_0: fp32 [H, D, Dh] (stride 0) or [B, H, D, Dh]; w2_0: fp32 [H, Dh, D] or [B, H, Dh, D];
 * w_batch_stride: elements between consecutive batch elements' states, 0 or at least H*D*Dh (a
 * multiple of 4); it applies to both w1_0 and w2_0, which hold D*Dh elements per head.
 * w1_out / w2_out (nullable): fp32 [B, H, D, Dh] / [B, H, Dh, D] end states.
 * Sizes: D in {16, 32, 64}, Dh a multiple of 64 in [64, 1024], chunk in {16, 32, 64}. bf16 I/O with
 * (D, Dh, chunk) = (64, 256, 16) runs on the matrix cores with the state held in registers, the
 * forward chain of each (b, h) on one CU and the read-outs beside it on other CUs from per-chunk
 * intermediates and state checkpoints kept in the workspace (about (N / 16) * 20 KiB plus
 * (N / 1024 + 4) * 128 KiB per (b, h): the size ttt_workspace_size returns). On that path a
 * workspace of at least B*H ints but less than that size runs the single-workgroup schedule
 * instead (forward and read-outs in one workgroup per (b, h), about 13 % slower at 4 x 8192 x 12),
 * for sequences whose intermediates the caller cannot hold; bf16
 * I/O with D = 64, chunk = 16 and Dh = 512, 768 or 1024 runs on the matrix cores with the fp32 state
 * in the workspace (bf16 operands, fp32 accumulation); every other size, and fp32 I/O, runs in
 * plain fp32 arithmetic with the state in the workspace.
 * Operand ranges (bf16 I/O, (D, Dh, chunk) = (64, 256, 16)): the products on the W2 side take
 * fp16 operands while the hidden pre-activations stay at least 2^-10 in magnitude (per lane of a
 * wave and chunk, unless all zero) and either within sqrt 2 or with GELU outputs within 32, the W2
 * state's largest magnitude (checked every 32 chunks and at the end) is in [2^-10, 2^15], and the
 * state stays finite; the read-outs check their own pre-activations and GELU outputs the same way.
 * A (batch, head) chain that leaves these ranges is recomputed in full by a last kernel with bf16
 * operands (fp32's exponent range); the workspace then holds, as its first B*H ints, a nonzero
 * value for each recomputed chain (bit 0: the forward chain, bit 1: a read-out) and 0 for the
 * others.
 * Precision: TTT_F32 keeps everything in fp32 (no reduced-precision operands).
 */
ttt_status ttt_mlp_forward(ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk, float eta,
                           const void* q, const void* k, const void* v,
                           const float* w1_0, const float* w2_0, long long w_batch_stride,
                           void* o, float* w1_out, float* w2_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Depth-wise 3x3 convolution over the token grid, the Conv2d preprocessing applied to a scan's
 * training data before the scan (Vision-TTT summary on gist.science, "Methodologie" item 2) and
 * ViT^3's depth-wise branch (ViT^3 review on techloop.online, "TTT Block" section). x and y are
 * [B, height * width, C] (tokens in raster order, channels contiguous: the [B, N, H, D] layout of
 * q, k, v with C = H * D) of dtype dt; weight fp32 [C, 3, 3]; bias fp32 [C] or NULL. With zero
 * padding of one token on each side,
 *   y[b, i, j, c] = bias[c] + sum_{u, v = 0..2} weight[c, u, v] x[b, i + u - 1, j + v - 1, c]
 * (cross-correlation, as convolution layers compute it), accumulated in fp32 and rounded to dt.
 * C must be a multiple of 4 and one image row (width * C elements) at most 2^31 - 1 bytes; x, y and
 * weight 16-byte aligned, bias 4-byte aligned; y must not overlap x, weight or bias. No workspace.
 */
ttt_status ttt_dwconv3x3(ttt_dtype dt, int B, int height, int width, int C, const void* x,
                         const float* weight, const float* bias, void* y, void* stream);

/*
 * ViT^3 block epilogue (ViT^3 review on techloop.online, "TTT Block" section and the section on the
 * official code: a GLU-style main branch and a 3x3 depth-wise convolution branch in parallel, their
 * outputs concatenated and projected back to the block's width). Per token m:
 *   y[m] = [o[m] * sigmoid(gate[m]), xconv[m]] w_proj^T + bias
 * o, gate, xconv: [M, C] (e.g. M = B * N tokens of the TTT layer's output, its gate, and the
 * convolution branch from ttt_dwconv3x3); w_proj: [C_out, 2C] (a linear layer's [out, in] layout),
 * all of dtype dt; bias fp32 [C_out] or NULL; y: [M, C_out] of dtype dt. bf16 accumulates in fp32
 * on the matrix cores (the gated values are rounded to bf16 as operands). C must be a multiple of
 * 32, C_out of 64; pointers 16-byte aligned (bias 4-byte); y must not overlap an input.
 */
ttt_status ttt_block_epilogue(ttt_dtype dt, int M, int C, int C_out, const void* o,
                              const void* gate, const void* xconv, const void* w_proj,
                              const float* bias, void* y, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): ttt_forward_fullbatch without a workspace argument.
 * Its scratch is a static device array of TTT_NOALLOC_SCRATCH_BYTES per device, which each device
 * the library runs on holds until the process ends; nothing is allocated or freed by the call.
 * Results are bit-identical to ttt_forward_fullbatch's. Every argument is validated as there;
 * calls whose ttt_workspace_size(TTT_OP_FULLBATCH, ...) exceeds TTT_NOALLOC_SCRATCH_BYTES return
 * TTT_ERR_WORKSPACE with nothing enqueued. `stream` must belong to the current device, whose
 * scratch is used; its address is looked up on the first call on that device (TTT_ERR_HIP if
 * that fails). All calls on one device share its scratch and keep no state in it between calls:
 * calls that overlap in time on one device (different streams, or host threads without ordering)
 * race on it and must not be made.
 */
#define TTT_NOALLOC_SCRATCH_BYTES (32u << 20)
ttt_status ttt_forward_fullbatch_noalloc(ttt_dtype dt, int B, int H, int N, int D, float eta,
                                         const void* q, const void* k, const void* v,
                                         const float* w0, long long w0_batch_stride,
                                         void* o, float* w_out, void* stream);

/* Bytes of workspace an entry point needs for these sizes (0 when none; chunk and Dh are
 * ignored where they do not apply). Returns 0 also for unsupported sizes. */
size_t ttt_workspace_size(ttt_op op, ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk);

/* Static, human-readable name of a status code. */
const char* ttt_status_string(ttt_status s);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
