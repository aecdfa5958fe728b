// C ABI of the TTT-layer forward library: argument validation, workspace sizing and dispatch.
// Every check runs before anything is enqueued, so a failed call leaves the outputs untouched.
#include <math.h>
#include <stdint.h>

#include <mutex>

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

// Common validation of the TTT-Linear entry points. Returns TTT_OK or the first failure. With
// check_ws false the workspace arguments are ignored (the caller supplies scratch of its own).
ttt_status check_linear(ttt_op op, ttt_dtype dt, int B, int H, int N, int D, int chunk,
                        float eta, const void* q, const void* k, const void* v, const float* w0,
                        long long w0s, const void* o, const float* w_out, const void* ws,
                        size_t ws_bytes, bool check_ws = true) {
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
  if (check_ws && need > 0) {
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

// Validation of the backward entry points: the forward's checks of q, k, v, w0 and one
// [B, N, H, D] output (d_q), then d_o, the other outputs, the workspace and every overlap.
ttt_status check_backward(ttt_op op, ttt_dtype dt, int B, int H, int N, int D, int chunk,
                          float eta, const void* q, const void* k, const void* v, const float* w0,
                          long long w0s, const void* d_o, const void* d_q, const void* d_k,
                          const void* d_v, const float* d_w0, const void* ws, size_t ws_bytes) {
  const ttt_op fwd = op == TTT_OP_FULLBATCH_BWD ? TTT_OP_FULLBATCH
                                                : (op == TTT_OP_CAUSAL_BWD ? TTT_OP_CAUSAL : TTT_OP_BIDIR);
  ttt_status st = check_linear(fwd, dt, B, H, N, D, chunk, eta, q, k, v, w0, w0s, d_q, nullptr,
                               nullptr, 0, false);
  if (st != TTT_OK) return st;
  if (!d_o || !d_k || !d_v || !d_w0) return TTT_ERR_INVALID;
  if (!aligned16(d_o) || !aligned16(d_k) || !aligned16(d_v) || !aligned16(d_w0))
    return TTT_ERR_INVALID;
  const size_t act = (size_t)B * N * H * D * elem_size(dt);
  const Range ins[5] = {range_of(q, act), range_of(k, act), range_of(v, act), range_of(d_o, act),
                        range_of(w0, state_bytes(B, H, (size_t)D * D, w0s))};
  const Range outs[4] = {range_of(d_q, act), range_of(d_k, act), range_of(d_v, act),
                         range_of(d_w0, (size_t)B * H * D * D * sizeof(float))};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], ins[j])) return TTT_ERR_INVALID;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return TTT_ERR_INVALID;
  }
  const size_t need = ttt_workspace_size(op, dt, B, H, N, D, 0, chunk);
  if (need > 0) {
    if (!ws || ws_bytes < need) return TTT_ERR_WORKSPACE;
    if (!aligned16(ws)) return TTT_ERR_INVALID;
    const Range rws = range_of(ws, need);
    for (int j = 0; j < 5; ++j)
      if (overlaps(rws, ins[j])) return TTT_ERR_INVALID;
    for (int i = 0; i < 4; ++i)
      if (overlaps(rws, outs[i])) return TTT_ERR_INVALID;
  }
  return TTT_OK;
}

// Scratch of ttt_forward_fullbatch_noalloc: one static array per device, never allocated or freed
// by the library (each device holds it until the process ends). In host code `scratch` only names
// the symbol; its device address is looked up once per device with that device current, and only
// that address is ever handed to kernels.
__device__ __align__(256) unsigned char scratch[TTT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device (null until looked up)

// Device address of the current device's scratch, or null if it cannot be had.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t ttt_workspace_size(ttt_op op, ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk) {
  if (B <= 0 || H <= 0 || N <= 0 || !supported_d(D)) return 0;
  if (dt != TTT_F32 && dt != TTT_BF16) return 0;
  const bool bf = dt == TTT_BF16;
  switch (op) {
    case TTT_OP_FULLBATCH:
      return round_up(ttt::fb_workspace_bytes(bf, B, H, N, D), 256);
    case TTT_OP_FULLBATCH_BWD:
      return round_up(ttt::fbb_workspace_bytes(bf, B, H, N, D), 256);
    case TTT_OP_CAUSAL_BWD:
    case TTT_OP_BIDIR_BWD:
      if (!supported_chunk(chunk) || N % chunk != 0) return 0;
      return round_up(ttt::chunked_bwd_workspace_bytes(op == TTT_OP_BIDIR_BWD, bf, B, H, N, D, chunk), 256);
    case TTT_OP_CAUSAL:
    case TTT_OP_BIDIR:
      if (!supported_chunk(chunk) || N % chunk != 0) return 0;
      return round_up(ttt::chunked_workspace_bytes(op == TTT_OP_BIDIR, bf, B, H, N, D, chunk), 256);
    case TTT_OP_BIDIR2D: {
      if (!supported_chunk(chunk) || N % chunk != 0) return 0;
      const size_t scan = round_up(ttt::chunked_workspace_bytes(true, bf, B, H, N, D, chunk), 256);
      if (bf) return scan;  // bf16: the column-order scan reads and adds in place
      const size_t act = round_up((size_t)B * N * H * D * elem_size(dt), 256);
      return 4 * act + scan;  // fp32: column-order copies of q, k, v and of the output, then the scans'
    }
    case TTT_OP_MLP:
      if (!ttt::mlp_supported(D, Dh, chunk) || N % chunk != 0) return 0;
      return round_up(ttt::mlp_workspace_bytes(bf, B, H, N, D, Dh, chunk), 256);
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
  return ttt_forward_fullbatch_epochs(dt, B, H, N, D, 1, eta, q, k, v, w0, w0_batch_stride, o,
                                      w_out, workspace, workspace_bytes, stream);
}

ttt_status ttt_forward_fullbatch_epochs(ttt_dtype dt, int B, int H, int N, int D, int epochs,
                                        float eta, const void* q, const void* k, const void* v,
                                        const float* w0, long long w0_batch_stride, void* o,
                                        float* w_out, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  const ttt_status st = check_linear(TTT_OP_FULLBATCH, dt, B, H, N, D, 0, eta, q, k, v, w0,
                                     w0_batch_stride, o, w_out, workspace, workspace_bytes);
  if (st != TTT_OK) return st;
  if (epochs < 1) return TTT_ERR_INVALID;
  if (epochs > 256) return TTT_ERR_UNSUPPORTED;
  return from_hip(ttt::fb_launch(dt == TTT_BF16, B, H, N, D, epochs, eta, q, k, v, w0,
                                 w0_batch_stride, o, w_out, workspace,
                                 static_cast<hipStream_t>(stream)));
}

ttt_status ttt_backward_fullbatch(ttt_dtype dt, int B, int H, int N, int D, float eta,
                                  const void* q, const void* k, const void* v, const float* w0,
                                  long long w0_batch_stride, const void* d_o, void* d_q,
                                  void* d_k, void* d_v, float* d_w0, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  const ttt_status st = check_backward(TTT_OP_FULLBATCH_BWD, dt, B, H, N, D, 0, eta, q, k, v, w0,
                                       w0_batch_stride, d_o, d_q, d_k, d_v, d_w0, workspace,
                                       workspace_bytes);
  if (st != TTT_OK) return st;
  return from_hip(ttt::fbb_launch(dt == TTT_BF16, B, H, N, D, eta, q, k, v, w0, w0_batch_stride,
                                  d_o, d_q, d_k, d_v, d_w0, workspace,
                                  static_cast<hipStream_t>(stream)));
}

ttt_status ttt_backward_chunked_causal(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                       float eta, const void* q, const void* k, const void* v,
                                       const float* w0, long long w0_batch_stride,
                                       const void* d_o, void* d_q, void* d_k, void* d_v,
                                       float* d_w0, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  const ttt_status st = check_backward(TTT_OP_CAUSAL_BWD, dt, B, H, N, D, chunk, eta, q, k, v, w0,
                                       w0_batch_stride, d_o, d_q, d_k, d_v, d_w0, workspace,
                                       workspace_bytes);
  if (st != TTT_OK) return st;
  return from_hip(ttt::chunked_bwd_launch(false, dt == TTT_BF16, B, H, N, D, chunk, eta, q, k, v,
                                          w0, w0_batch_stride, d_o, d_q, d_k, d_v, d_w0,
                                          workspace, static_cast<hipStream_t>(stream)));
}

ttt_status ttt_backward_chunked_bidir(ttt_dtype dt, int B, int H, int N, int D, int chunk,
                                      float eta, const void* q, const void* k, const void* v,
                                      const float* w0, long long w0_batch_stride,
                                      const void* d_o, void* d_q, void* d_k, void* d_v,
                                      float* d_w0, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  const ttt_status st = check_backward(TTT_OP_BIDIR_BWD, dt, B, H, N, D, chunk, eta, q, k, v, w0,
                                       w0_batch_stride, d_o, d_q, d_k, d_v, d_w0, workspace,
                                       workspace_bytes);
  if (st != TTT_OK) return st;
  return from_hip(ttt::chunked_bwd_launch(true, dt == TTT_BF16, B, H, N, D, chunk, eta, q, k, v,
                                          w0, w0_batch_stride, d_o, d_q, d_k, d_v, d_w0,
                                          workspace, static_cast<hipStream_t>(stream)));
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

ttt_status ttt_forward_chunked_bidir2d(ttt_dtype dt, int B, int H, int height, int width, int D,
                                       int chunk, float eta, const void* q, const void* k,
                                       const void* v, const float* w0, long long w0_batch_stride,
                                       void* o, float* w_out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (height <= 0 || width <= 0) return TTT_ERR_INVALID;
  if ((long long)height * width > 0x7fffffffll) return TTT_ERR_UNSUPPORTED;
  const int N = height * width;
  // The bidirectional checks cover the inputs, o and the first two w_out states; the column scan
  // writes the other two.
  ttt_status st = check_linear(TTT_OP_BIDIR, dt, B, H, N, D, chunk, eta, q, k, v, w0,
                               w0_batch_stride, o, w_out, nullptr, 0, false);
  if (st != TTT_OK) return st;
  const size_t act = (size_t)B * N * H * D * elem_size(dt);
  const size_t dd = (size_t)B * H * D * D;
  const Range rq = range_of(q, act), rk = range_of(k, act), rv = range_of(v, act);
  const Range rw0 = range_of(w0, state_bytes(B, H, (size_t)D * D, w0_batch_stride));
  if (w_out) {
    const Range rwo = range_of(w_out, 4 * dd * sizeof(float));
    if (overlaps(rwo, rq) || overlaps(rwo, rk) || overlaps(rwo, rv) || overlaps(rwo, rw0) ||
        overlaps(rwo, range_of(o, act)))
      return TTT_ERR_INVALID;
  }
  const size_t need = ttt_workspace_size(TTT_OP_BIDIR2D, dt, B, H, N, D, 0, chunk);
  if (need > 0) {  // (a bf16 call whose scans are one segment each needs none)
    if (!workspace || workspace_bytes < need) return TTT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TTT_ERR_INVALID;
    const Range rws = range_of(workspace, need);
    if (overlaps(rws, rq) || overlaps(rws, rk) || overlaps(rws, rv) || overlaps(rws, rw0) ||
        overlaps(rws, range_of(o, act)) || (w_out && overlaps(rws, range_of(w_out, 4 * dd * 4))))
      return TTT_ERR_INVALID;
  }
  const bool bf = dt == TTT_BF16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf) {  // the raster-order scan writes o, the column-order one reads in place and adds into o
    hipError_t e = ttt::chunked_launch(true, true, B, H, N, D, chunk, eta, q, k, v, w0, w0_batch_stride, o,
                                       w_out, workspace, s);
    if (e == hipSuccess)
      e = ttt::chunked_bidir_cols_launch(B, H, height, width, D, chunk, eta, q, k, v, w0, w0_batch_stride, o,
                                         w_out ? w_out + 2 * dd : nullptr, workspace, s);
    return from_hip(e);
  }
  // fp32 workspace: q, k, v and the output in column order, then the scans' own workspace.
  char* wsb = static_cast<char*>(workspace);
  const size_t actp = round_up(act, 256);
  void* qt = wsb;
  void* kt = wsb + actp;
  void* vt = wsb + 2 * actp;
  void* ot = wsb + 3 * actp;
  void* scan_ws = wsb + 4 * actp;
  const void* srcs[3] = {q, k, v};
  void* dsts[3] = {qt, kt, vt};
  hipError_t e = ttt::gather_columns_launch(bf, B, height, width, H * D, srcs, dsts, 3, s);
  if (e == hipSuccess)
    e = ttt::chunked_launch(true, bf, B, H, N, D, chunk, eta, q, k, v, w0, w0_batch_stride, o, w_out,
                            scan_ws, s);
  if (e == hipSuccess)
    e = ttt::chunked_launch(true, bf, B, H, N, D, chunk, eta, qt, kt, vt, w0, w0_batch_stride, ot,
                            w_out ? w_out + 2 * dd : nullptr, scan_ws, s);
  if (e == hipSuccess) e = ttt::add_columns_launch(bf, B, height, width, H * D, ot, o, s);
  return from_hip(e);
}

ttt_status ttt_mlp_forward(ttt_dtype dt, int B, int H, int N, int D, int Dh, int chunk, float eta,
                           const void* q, const void* k, const void* v, const float* w1_0,
                           const float* w2_0, long long w_batch_stride, void* o, float* w1_out,
                           float* w2_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (dt != TTT_F32 && dt != TTT_BF16) return TTT_ERR_INVALID;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || Dh <= 0 || chunk <= 0) return TTT_ERR_INVALID;
  if (!isfinite(eta)) return TTT_ERR_INVALID;
  if (!q || !k || !v || !w1_0 || !w2_0 || !o) return TTT_ERR_INVALID;
  if (!ttt::mlp_supported(D, Dh, chunk)) return TTT_ERR_UNSUPPORTED;
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
  // ttt_workspace_size's figure runs the fastest schedule; on the matrix-core path a workspace of at
  // least one int per chain, but less than that, runs the single-workgroup schedule.
  const size_t full = ttt_workspace_size(TTT_OP_MLP, dt, B, H, N, D, Dh, chunk);
  const size_t least = ttt::mlp_min_workspace_bytes(dt == TTT_BF16, B, H, N, D, Dh, chunk);
  const size_t need = workspace_bytes >= full ? full : least;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return TTT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TTT_ERR_INVALID;
    const Range rws = range_of(workspace, need);
    if (overlaps(rws, rq) || overlaps(rws, rk) || overlaps(rws, rv) || overlaps(rws, ro) ||
        overlaps(rws, r1) || overlaps(rws, r2) || overlaps(rws, outs[0]) || overlaps(rws, outs[1]))
      return TTT_ERR_INVALID;
  }
  return from_hip(ttt::mlp_launch(dt == TTT_BF16, B, H, N, D, Dh, chunk, eta, q, k, v, w1_0, w2_0,
                                  w_batch_stride, o, w1_out, w2_out, workspace, need,
                                  static_cast<hipStream_t>(stream)));
}

ttt_status ttt_dwconv3x3(ttt_dtype dt, int B, int height, int width, int C, const void* x,
                         const float* weight, const float* bias, void* y, void* stream) {
  if (dt != TTT_F32 && dt != TTT_BF16) return TTT_ERR_INVALID;
  if (B <= 0 || height <= 0 || width <= 0 || C <= 0) return TTT_ERR_INVALID;
  if (!x || !weight || !y) return TTT_ERR_INVALID;
  if (C % 4 != 0) return TTT_ERR_UNSUPPORTED;
  // (one image row's bytes must fit the 32-bit range of a buffer resource)
  if (B > 65535 || height > 65535 || (long long)width * C * elem_size(dt) > 0x7fffffffll)
    return TTT_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || !aligned16(weight) ||
      (bias && (reinterpret_cast<uintptr_t>(bias) & 3u)))
    return TTT_ERR_INVALID;
  const size_t act = (size_t)B * height * width * C * elem_size(dt);
  const Range ry = range_of(y, act);
  if (overlaps(ry, range_of(x, act)) || overlaps(ry, range_of(weight, (size_t)C * 9 * sizeof(float))) ||
      (bias && overlaps(ry, range_of(bias, (size_t)C * sizeof(float)))))
    return TTT_ERR_INVALID;
  return from_hip(ttt::dwconv_launch(dt == TTT_BF16, B, height, width, C, x, weight, bias, y,
                                     static_cast<hipStream_t>(stream)));
}

ttt_status ttt_block_epilogue(ttt_dtype dt, int M, int C, int C_out, const void* o,
                              const void* gate, const void* xconv, const void* w_proj,
                              const float* bias, void* y, void* stream) {
  if (dt != TTT_F32 && dt != TTT_BF16) return TTT_ERR_INVALID;
  if (M <= 0 || C <= 0 || C_out <= 0) return TTT_ERR_INVALID;
  if (!o || !gate || !xconv || !w_proj || !y) return TTT_ERR_INVALID;
  if (C % 32 != 0 || C_out % 64 != 0 || C > 4096 || C_out > 65535 * 64) return TTT_ERR_UNSUPPORTED;
  if ((long long)M * (C > C_out ? C : C_out) > (1ll << 40)) return TTT_ERR_UNSUPPORTED;
  if (!aligned16(o) || !aligned16(gate) || !aligned16(xconv) || !aligned16(w_proj) || !aligned16(y) ||
      (bias && (reinterpret_cast<uintptr_t>(bias) & 3u)))
    return TTT_ERR_INVALID;
  const size_t es = elem_size(dt);
  const Range ry = range_of(y, (size_t)M * C_out * es);
  if (overlaps(ry, range_of(o, (size_t)M * C * es)) || overlaps(ry, range_of(gate, (size_t)M * C * es)) ||
      overlaps(ry, range_of(xconv, (size_t)M * C * es)) ||
      overlaps(ry, range_of(w_proj, (size_t)C_out * 2 * C * es)) ||
      (bias && overlaps(ry, range_of(bias, (size_t)C_out * sizeof(float)))))
    return TTT_ERR_INVALID;
  return from_hip(ttt::epilogue_launch(dt == TTT_BF16, M, C, C_out, o, gate, xconv, w_proj, bias, y,
                                       static_cast<hipStream_t>(stream)));
}

ttt_status ttt_forward_fullbatch_noalloc(ttt_dtype dt, int B, int H, int N, int D, float eta,
                                         const void* q, const void* k, const void* v,
                                         const float* w0, long long w0_batch_stride, void* o,
                                         float* w_out, void* stream) {
  const ttt_status st = check_linear(TTT_OP_FULLBATCH, dt, B, H, N, D, 0, eta, q, k, v, w0,
                                     w0_batch_stride, o, w_out, nullptr, 0, false);
  if (st != TTT_OK) return st;
  const size_t need = ttt_workspace_size(TTT_OP_FULLBATCH, dt, B, H, N, D, 0, 0);
  if (need > (size_t)TTT_NOALLOC_SCRATCH_BYTES) return TTT_ERR_WORKSPACE;
  void* ws = scratch_of_current_device();
  if (!ws) return TTT_ERR_HIP;
  return from_hip(ttt::fb_launch(dt == TTT_BF16, B, H, N, D, 1, eta, q, k, v, w0,
                                 w0_batch_stride, o, w_out, ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
