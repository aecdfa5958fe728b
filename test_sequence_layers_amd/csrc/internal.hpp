// Host-side interface between the C ABI layer (abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ttt {

// Round x up to a multiple of m.
inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// ---- full-batch -----------------------------------------------------------------------------
struct FbPlan {
  int splits;           // token splits per (b, h) for the gradient reduction
  int tokens_per_split; // multiple of the 64-token tile
};
FbPlan fb_plan(int B, int H, int N, int D);
size_t fb_workspace_bytes(bool bf16_io, int B, int H, int N, int D);
hipError_t fb_launch(bool bf16_io, int B, int H, int N, int D, float eta, const void* q,
                     const void* k, const void* v, const float* w0, long long w0_bstride, void* o,
                     float* w_out, void* ws, hipStream_t st);

// ---- chunked TTT-Linear (causal and bidirectional) ------------------------------------------
size_t chunked_workspace_bytes(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk);
hipError_t chunked_launch(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk,
                          float eta, const void* q, const void* k, const void* v, const float* w0,
                          long long w0_bstride, void* o, float* w_out, void* ws, hipStream_t st);

// ---- TTT-MLP --------------------------------------------------------------------------------
size_t mlp_workspace_bytes(int B, int H, int N, int D, int Dh, int chunk);
hipError_t mlp_launch(int B, int H, int N, int D, int Dh, int chunk, float eta, const void* q,
                      const void* k, const void* v, const float* w1, const float* w2,
                      long long w_bstride, void* o, float* w1_out, float* w2_out, void* ws,
                      hipStream_t st);

}  // namespace ttt
