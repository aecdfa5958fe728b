// Token-grid permutations for the column-order scans of the 2-D bidirectional layer (Vision-TTT
// summary on gist.science, "De Oplossing": the scanner also reads the image top to bottom).
// A sequence of N = height * width tokens in raster order, [B, N, C] with C channels contiguous,
// is read in column order (top to bottom, column by column) by moving whole token rows: token
// (i, j) goes from raster index i * width + j to column index j * height + i. Each thread moves
// one 16-byte piece of a token row, so every access is a contiguous run of a row: HBM-bound,
// coalesced, no LDS.
#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kGridThreads = 256;

// dst[t] = src[t] in column order, for the tensors t = blockIdx.z (up to three at once).
__global__ __launch_bounds__(kGridThreads) void gather_columns(const uint4* __restrict__ s0,
                                                               const uint4* __restrict__ s1,
                                                               const uint4* __restrict__ s2,
                                                               uint4* __restrict__ d0,
                                                               uint4* __restrict__ d1,
                                                               uint4* __restrict__ d2, int Hg,
                                                               int Wg, int pieces) {
  const long long e = (long long)blockIdx.x * kGridThreads + threadIdx.x;  // piece of this image
  const long long N = (long long)Hg * Wg;
  if (e >= N * pieces) return;
  const int p = (int)(e / pieces), c = (int)(e % pieces);  // destination token (column order)
  const int j = p / Hg, i = p % Hg;
  const long long img = (long long)blockIdx.y * N * pieces;
  const long long src = img + ((long long)i * Wg + j) * pieces + c;
  const long long dst = img + (long long)p * pieces + c;
  const uint4* s = blockIdx.z == 0 ? s0 : (blockIdx.z == 1 ? s1 : s2);
  uint4* d = blockIdx.z == 0 ? d0 : (blockIdx.z == 1 ? d1 : d2);
  d[dst] = s[src];
}

// o[raster token] += ot[the same token in column order], 8 bf16 (or 4 fp32) values a piece, the
// sum rounded once.
template <class T>
__global__ __launch_bounds__(kGridThreads) void add_columns(const T* __restrict__ ot,
                                                            T* __restrict__ o, int Hg, int Wg,
                                                            int pieces) {
  constexpr int V = 16 / sizeof(T);
  const long long e = (long long)blockIdx.x * kGridThreads + threadIdx.x;
  const long long N = (long long)Hg * Wg;
  if (e >= N * pieces) return;
  const int p = (int)(e / pieces), c = (int)(e % pieces);  // raster token p = i * Wg + j
  const int i = p / Wg, j = p % Wg;
  const long long img = (long long)blockIdx.y * N * pieces;
  const long long dst = (img + (long long)p * pieces + c) * V;
  const long long src = (img + ((long long)j * Hg + i) * pieces + c) * V;
  if constexpr (sizeof(T) == 2) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + dst);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(ot + src);
    f32x4 lo, hi;
    for (int t = 0; t < 4; ++t) {
      lo[t] = (float)a[t] + (float)b[t];
      hi[t] = (float)a[4 + t] + (float)b[4 + t];
    }
    *reinterpret_cast<bf16x8*>(o + dst) = cat8(to_bf16x4(lo), to_bf16x4(hi));
  } else {
    float4 a = *reinterpret_cast<const float4*>(o + dst);
    const float4 b = *reinterpret_cast<const float4*>(ot + src);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    *reinterpret_cast<float4*>(o + dst) = a;
  }
}

}  // namespace

hipError_t gather_columns_launch(bool bf16_io, int B, int Hg, int Wg, int C, const void* const src[3],
                                 void* const dst[3], int count, hipStream_t st) {
  const int pieces = C * (bf16_io ? 2 : 4) / 16;
  const long long n = (long long)Hg * Wg * pieces;
  const dim3 grid((unsigned)((n + kGridThreads - 1) / kGridThreads), (unsigned)B, (unsigned)count);
  hipLaunchKernelGGL(gather_columns, grid, dim3(kGridThreads), 0, st, (const uint4*)src[0],
                     (const uint4*)src[count > 1 ? 1 : 0], (const uint4*)src[count > 2 ? 2 : 0],
                     (uint4*)dst[0], (uint4*)dst[count > 1 ? 1 : 0], (uint4*)dst[count > 2 ? 2 : 0], Hg,
                     Wg, pieces);
  return hipGetLastError();
}

hipError_t add_columns_launch(bool bf16_io, int B, int Hg, int Wg, int C, const void* ot, void* o,
                              hipStream_t st) {
  const int pieces = C * (bf16_io ? 2 : 4) / 16;
  const long long n = (long long)Hg * Wg * pieces;
  const dim3 grid((unsigned)((n + kGridThreads - 1) / kGridThreads), (unsigned)B);
  if (bf16_io)
    hipLaunchKernelGGL(add_columns<bf16>, grid, dim3(kGridThreads), 0, st, (const bf16*)ot, (bf16*)o, Hg,
                       Wg, pieces);
  else
    hipLaunchKernelGGL(add_columns<float>, grid, dim3(kGridThreads), 0, st, (const float*)ot, (float*)o,
                       Hg, Wg, pieces);
  return hipGetLastError();
}

}  // namespace ttt
