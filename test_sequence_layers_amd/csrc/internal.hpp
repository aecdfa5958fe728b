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
hipError_t fb_launch(bool bf16_io, int B, int H, int N, int D, int epochs, float eta,
                     const void* q, const void* k, const void* v, const float* w0,
                     long long w0_bstride, void* o, float* w_out, void* ws, hipStream_t st);

size_t fbb_workspace_bytes(bool bf16_io, int B, int H, int N, int D);
hipError_t fbb_launch(bool bf16_io, int B, int H, int N, int D, float eta, const void* q,
                      const void* k, const void* v, const float* w0, long long w0_bstride,
                      const void* d_o, void* d_q, void* d_k, void* d_v, float* d_w0, void* ws,
                      hipStream_t st);

// ---- chunked TTT-Linear (causal and bidirectional) ------------------------------------------
size_t chunked_workspace_bytes(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk);
hipError_t chunked_launch(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk,
                          float eta, const void* q, const void* k, const void* v, const float* w0,
                          long long w0_bstride, void* o, float* w_out, void* ws, hipStream_t st);
// bf16 bidirectional scan over the column order of a Hg x Wg token grid, reading q, k, v in place
// (raster layout) and adding its output into o (which holds the raster-order scan's); the workspace
// is chunked_workspace_bytes(true, true, B, H, Hg * Wg, D, chunk).
hipError_t chunked_bidir_cols_launch(int B, int H, int Hg, int Wg, int D, int chunk, float eta,
                                     const void* q, const void* k, const void* v, const float* w0,
                                     long long w0_bstride, void* o, float* w_out, void* ws, hipStream_t st);
size_t chunked_bwd_workspace_bytes(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk);
hipError_t chunked_bwd_launch(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk,
                              float eta, const void* q, const void* k, const void* v,
                              const float* w0, long long w0_bstride, const void* d_o, void* d_q,
                              void* d_k, void* d_v, float* d_w0, void* ws, hipStream_t st);

// ---- TTT-MLP --------------------------------------------------------------------------------
bool mlp_supported(int D, int Dh, int chunk);
size_t mlp_workspace_bytes(bool bf16_io, int B, int H, int N, int D, int Dh, int chunk);
size_t mlp_min_workspace_bytes(bool bf16_io, int B, int H, int N, int D, int Dh, int chunk);
hipError_t mlp_launch(bool bf16_io, int B, int H, int N, int D, int Dh, int chunk, float eta,
                      const void* q, const void* k, const void* v, const float* w1,
                      const float* w2, long long w_bstride, void* o, float* w1_out,
                      float* w2_out, void* ws, size_t ws_bytes, hipStream_t st);

// ---- token-grid permutations (column order) ---------------------------------------------------
hipError_t gather_columns_launch(bool bf16_io, int B, int Hg, int Wg, int C,
                                 const void* const src[3], void* const dst[3], int count,
                                 hipStream_t st);
hipError_t add_columns_launch(bool bf16_io, int B, int Hg, int Wg, int C, const void* ot, void* o,
                              hipStream_t st);

// ---- ViT^3 block epilogue ---------------------------------------------------------------------
hipError_t epilogue_launch(bool bf16_io, int M, int C, int Cout, const void* o, const void* gate,
                           const void* xc, const void* wo, const float* bias, void* y,
                           hipStream_t st);

// ---- depth-wise 3x3 convolution over the token grid ------------------------------------------
hipError_t dwconv_launch(bool bf16_io, int B, int Hi, int Wi, int C, const void* x,
                         const float* w, const float* bias, void* y, hipStream_t st);

}  // namespace ttt
