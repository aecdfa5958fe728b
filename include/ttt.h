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
 *                          TTT-MLP with (D, Dh) other than (64, 256); TTT-MLP with fp32 I/O
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
 *   fp16 operands (more mantissa bits; those values stay far inside fp16's range).
 * Threads.  Entry points are reentrant. The only state kept between calls is a per-device cache
 *   of kernel occupancy figures (the chunked scans size their segment plan from it), filled on a
 *   device's first call through atomics.
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

typedef enum { TTT_OP_FULLBATCH = 0, TTT_OP_CAUSAL = 1, TTT_OP_BIDIR = 2, TTT_OP_MLP = 3 } ttt_op;

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
 * Causal mini-batch TTT-MLP (TTT-Linear / TTT-MLP abstract: the hidden state is a two-layer
 * MLP). f(x) = GELU(x W1) W2 with exact erf GELU and no bias. Per (b, h) and chunk c with start
 * state (W1_s, W2_s): token i is read out with (W1_s, W2_s) - (eta/b) * sum_{j <= i in c} of the
 * per-token gradients at the start state; the chunk hands on the state after all b gradients.
 * w1_0: fp32 [H, D, Dh] (stride 0) or [B, H, D, Dh]; w2_0: fp32 [H, Dh, D] or [B, H, Dh, D];
 * w_batch_stride: elements between consecutive batch elements' states, 0 or at least H*D*Dh (a
 * multiple of 4); it applies to both w1_0 and w2_0, which hold D*Dh elements per head.
 * w1_out / w2_out (nullable): fp32 [B, H, D, Dh] / [B, H, Dh, D] end states.
 */
ttt_status ttt_mlp_forward(ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk, float eta,
                           const void* q, const void* k, const void* v,
                           const float* w1_0, const float* w2_0, long long w_batch_stride,
                           void* o, float* w1_out, float* w2_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace an entry point needs for these sizes (0 when none; chunk and Dh are
 * ignored where they do not apply). Returns 0 also for unsupported sizes. */
size_t ttt_workspace_size(ttt_op op, ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk);

/* Static, human-readable name of a status code. */
const char* ttt_status_string(ttt_status s);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H_ */
