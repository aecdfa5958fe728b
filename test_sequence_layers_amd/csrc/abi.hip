// C ABI of the TTT-layer forward library: argument validation, workspace sizing and dispatch.
// Every check runs before anything is enqueued, so a failed call leaves the outputs untouched.
#include <math.h>
#include <stdint.h>

#include "../../include/ttt.h"
#include "internal.hpp"

namespace {

using ttt::round_up;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlaps(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int D) { return D == 16 || D == 32 || D == 64; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }

size_t elem_size(ttt_dtype dt) { return dt == TTT_BF16 ? 2 : 4; }

// Byte extent of an fp32 state array with per-head size `per_head` floats.
size_t state_bytes(int B, int H, size_t per_head, long long stride) {
  const size_t one = (size_t)H * per_head;
  if (stride == 0) return one * sizeof(float);
  return ((size_t)(B - 1) * (size_t)stride + one) * sizeof(float);
}

// Common validation of the TTT-Linear entry points. Returns TTT_OK or the first failure.
ttt_status check_linear(ttt_op op, ttt_dtype dt, int B, int H, int N, int D, int chunk,
                        float eta, const void* q, const void* k, const void* v, const float* w0,
                        long long w0s, const void* o, const float* w_out, const void* ws,
                        size_t ws_bytes) {
  if (dt != TTT_F32 && dt != TTT_BF16) return TTT_ERR_INVALID;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return TTT_ERR_INVALID;
  if (!isfinite(eta)) return TTT_ERR_INVALID;
  if (!q || !k || !v || !w0 || !o) return TTT_ERR_INVALID;
  if (!supported_d(D)) return TTT_ERR_UNSUPPORTED;
  if (op != TTT_OP_FULLBATCH) {
    if (chunk <= 0) return TTT_ERR_INVALID;
    if (!supported_chunk(chunk)) return TTT_ERR_UNSUPPORTED;
    if (N % chunk != 0) return TTT_ERR_INVALID;
  }
  if ((long long)B * H > 65535) return TTT_ERR_UNSUPPORTED;
  const long long head = (long long)H * D * D;
  // A per-batch stride keeps every batch element's states 16-byte aligned, as the kernels' vector
  // loads of them require.
  if (w0s != 0 && (w0s < head || w0s % 4 != 0)) return TTT_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(w0))
    return TTT_ERR_INVALID;
  if (w_out && !aligned16(w_out)) return TTT_ERR_INVALID;
  const size_t act = (size_t)B * N * H * D * elem_size(dt);
  const Range rq = range_of(q, act), rk = range_of(k, act), rv = range_of(v, act);
  const Range ro = range_of(o, act), rw0 = range_of(w0, state_bytes(B, H, (size_t)D * D, w0s));
  if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rw0))
    return TTT_ERR_INVALID;
  if (w_out) {
    const size_t nst = op == TTT_OP_BIDIR ? 2 : 1;
    const Range rwo = range_of(w_out, nst * (size_t)B * H * D * D * sizeof(float));
    if (overlaps(rwo, rq) || overlaps(rwo, rk) || overlaps(rwo, rv) || overlaps(rwo, ro) ||
        overlaps(rwo, rw0))
      return TTT_ERR_INVALID;
  }
  const size_t need = ttt_workspace_size(op, dt, B, H, N, D, 0, chunk);
  if (need > 0) {
    if (!ws || ws_bytes < need) return TTT_ERR_WORKSPACE;
    if (!aligned16(ws)) return TTT_ERR_INVALID;
    const Range rws = range_of(ws, need);
    if (overlaps(rws, rq) || overlaps(rws, rk) || overlaps(rws, rv) || overlaps(rws, ro) ||
        overlaps(rws, rw0))
      return TTT_ERR_INVALID;
    if (w_out && overlaps(rws, range_of(w_out, (op == TTT_OP_BIDIR ? 2 : 1) * (size_t)B * H * D * D * 4)))
      return TTT_ERR_INVALID;
  }
  return TTT_OK;
}

ttt_status from_hip(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_HIP; }

}  // namespace

extern "C" {

size_t ttt_workspace_size(ttt_op op, ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk) {
  if (B <= 0 || H <= 0 || N <= 0 || !supported_d(D)) return 0;
  if (dt != TTT_F32 && dt != TTT_BF16) return 0;
  const bool bf = dt == TTT_BF16;
  switch (op) {
    case TTT_OP_FULLBATCH:
      return round_up(ttt::fb_workspace_bytes(bf, B, H, N, D), 256);
    case TTT_OP_CAUSAL:
    case TTT_OP_BIDIR:
      if (!supported_chunk(chunk) || N % chunk != 0) return 0;
      return round_up(ttt::chunked_workspace_bytes(op == TTT_OP_BIDIR, bf, B, H, N, D, chunk), 256);
    case TTT_OP_MLP:
      if (chunk <= 0 || N % chunk != 0) return 0;
      return round_up(ttt::mlp_workspace_bytes(B, H, N, D, Dh, chunk), 256);
  }
  return 0;
}

const char* ttt_status_string(ttt_status s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_ERR_INVALID: return "invalid argument";
    case TTT_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case TTT_ERR_WORKSPACE: return "workspace missing or too small";
    case TTT_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

ttt_status ttt_forward_fullbatch(ttt_dtype dt, int B, int H, int N, int D, float eta,
                                 const void* q, const void* k, const void* v, const float* w0,
                                 long long w0_batch_stride, void* o, float* w_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const ttt_status st = check_linear(TTT_OP_FULLBATCH, dt, B, H, N, D, 0, eta, q, k, v, w0,
                                     w0_batch_stride, o, w_out, workspace, workspace_bytes);
  if (st != TTT_OK) return st;
  return from_hip(ttt::fb_launch(dt == TTT_BF16, B, H, N, D, eta, q, k, v, w0, w0_batch_stride,
                                 o, w_out, workspace, static_cast<hipStream_t>(stream)));
}

ttt_status ttt_forward_chunked_causal(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                      float eta, const void* q, const void* k, const void* v,
                                      const float* w0, long long w0_batch_stride, void* o,
                                      float* w_out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  const ttt_status st = check_linear(TTT_OP_CAUSAL, dt, B, H, N, D, chunk, eta, q, k, v, w0,
                                     w0_batch_stride, o, w_out, workspace, workspace_bytes);
  if (st != TTT_OK) return st;
  return from_hip(ttt::chunked_launch(false, dt == TTT_BF16, B, H, N, D, chunk, eta, q, k, v, w0,
                                      w0_batch_stride, o, w_out, workspace,
                                      static_cast<hipStream_t>(stream)));
}

ttt_status ttt_forward_chunked_bidir(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                     float eta, const void* q, const void* k, const void* v,
                                     const float* w0, long long w0_batch_stride, void* o,
                                     float* w_out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  const ttt_status st = check_linear(TTT_OP_BIDIR, dt, B, H, N, D, chunk, eta, q, k, v, w0,
                                     w0_batch_stride, o, w_out, workspace, workspace_bytes);
  if (st != TTT_OK) return st;
  return from_hip(ttt::chunked_launch(true, dt == TTT_BF16, B, H, N, D, chunk, eta, q, k, v, w0,
                                      w0_batch_stride, o, w_out, workspace,
                                      static_cast<hipStream_t>(stream)));
}

ttt_status ttt_mlp_forward(ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk, float eta,
                           const void* q, const void* k, const void* v, const float* w1_0,
                           const float* w2_0, long long w_batch_stride, void* o, float* w1_out,
                           float* w2_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (dt != TTT_F32 && dt != TTT_BF16) return TTT_ERR_INVALID;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || Dh <= 0 || chunk <= 0) return TTT_ERR_INVALID;
  if (!isfinite(eta)) return TTT_ERR_INVALID;
  if (!q || !k || !v || !w1_0 || !w2_0 || !o) return TTT_ERR_INVALID;
  if (dt != TTT_BF16 || D != 64 || Dh != 256 || chunk != 16) return TTT_ERR_UNSUPPORTED;
  if (N % chunk != 0) return TTT_ERR_INVALID;
  const long long head = (long long)H * D * Dh;
  if (w_batch_stride != 0 && (w_batch_stride < head || w_batch_stride % 4 != 0)) return TTT_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(w1_0) ||
      !aligned16(w2_0))
    return TTT_ERR_INVALID;
  if ((w1_out && !aligned16(w1_out)) || (w2_out && !aligned16(w2_out))) return TTT_ERR_INVALID;
  const size_t act = (size_t)B * N * H * D * elem_size(dt);
  const Range rq = range_of(q, act), rk = range_of(k, act), rv = range_of(v, act);
  const Range ro = range_of(o, act);
  const size_t wb = state_bytes(B, H, (size_t)D * Dh, w_batch_stride);
  const Range r1 = range_of(w1_0, wb), r2 = range_of(w2_0, wb);
  if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, r1) ||
      overlaps(ro, r2))
    return TTT_ERR_INVALID;
  const size_t ob = (size_t)B * H * D * Dh * sizeof(float);
  const Range outs[2] = {range_of(w1_out, w1_out ? ob : 0), range_of(w2_out, w2_out ? ob : 0)};
  for (int i = 0; i < 2; ++i) {
    if (outs[i].hi == outs[i].lo) continue;
    if (overlaps(outs[i], rq) || overlaps(outs[i], rk) || overlaps(outs[i], rv) ||
        overlaps(outs[i], ro) || overlaps(outs[i], r1) || overlaps(outs[i], r2))
      return TTT_ERR_INVALID;
  }
  if (w1_out && w2_out && overlaps(outs[0], outs[1])) return TTT_ERR_INVALID;
  const size_t need = ttt_workspace_size(TTT_OP_MLP, dt, B, H, N, D, Dh, chunk);
  if (need > 0 && (!workspace || workspace_bytes < need)) return TTT_ERR_WORKSPACE;
  return from_hip(ttt::mlp_launch(B, H, N, D, Dh, chunk, eta, q, k, v, w1_0, w2_0,
                                  w_batch_stride, o, w1_out, w2_out, workspace,
                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
