// ViT^3 block epilogue (ViT^3 review on techloop.online, "TTT Block" section and the section on the
// official code: a GLU-style main branch and a 3x3 depth-wise convolution branch run in parallel,
// their outputs are concatenated and projected back to the block's width). Per token:
//   y = [O * sigmoid(G), X] Wo^T + b,   Wo [C_out, 2C] (a linear layer's [out, in] layout),
// with O the TTT layer's output, G the gate (the sigmoid of the original gated linear unit) and X
// the convolution branch's output, all [M, C] row-major.
//
// bf16: a GEMM whose activation operand is formed while it is staged. Workgroup tile: 64 tokens x
// 64 outputs, the contraction (K = 2C) in blocks of 64 through double-buffered LDS, one barrier a
// block; the next block's pieces are loaded into registers while the current one is multiplied.
// The matrix-core A operand is Wo (rows = outputs) and B the activations (columns = tokens), so
// lane (r, g) ends with 4 adjacent outputs of token r; the output tile is written out through LDS
// as whole 128-byte rows. At the workloads' widths
// (C = 64..192) the arithmetic intensity is about 50-100 flop/byte, below the ridge point: bound
// by reading O, G, X and writing y. fp32: plain FMA, one thread per output element.
#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kEpThreads = 256;
constexpr int kEpTok = 64, kEpOut = 64, kEpK = 64;
constexpr int kEpP = kEpK + 8;  // LDS row pitch (elements): 144 bytes

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }

__device__ __forceinline__ uint4 pack_bf16x8(const float* v) {
  const f32x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
  return __builtin_bit_cast(uint4, cat8(to_bf16x4(lo), to_bf16x4(hi)));
}
__device__ __forceinline__ void unpack_bf16x8(uint4 u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__global__ __launch_bounds__(kEpThreads) void epilogue_bf16(
    const bf16* __restrict__ o, const bf16* __restrict__ gate, const bf16* __restrict__ xc,
    const bf16* __restrict__ wo, const float* __restrict__ bias, bf16* __restrict__ y, int M,
    int C, int Cout) {
  __shared__ __align__(16) bf16 sA[2][kEpTok * kEpP];  // activations [token][k]
  __shared__ __align__(16) bf16 sW[2][kEpOut * kEpP];  // Wo [out][k]
  const int m0 = blockIdx.x * kEpTok, n0 = blockIdx.y * kEpOut;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int K = 2 * C, nkb = K / kEpK;
  const int tid = threadIdx.x;
  // Each thread stages pieces (row, 8-wide column) p = tid and tid + 256 of each 64 x 64 block.
  uint4 ra[2], rw[2];
  auto load = [&](int kb) {
    for (int u = 0; u < 2; ++u) {
      const int p = tid + u * kEpThreads, row = p >> 3, kk = kb * kEpK + (p & 7) * 8;
      const int tok = m0 + row;
      float v[8];
      if (tok < M) {
        if (kk < C) {  // gated main branch O * sigmoid(G)
          float a[8], b[8];
          unpack_bf16x8(ld16(o + (long long)tok * C + kk), a);
          unpack_bf16x8(ld16(gate + (long long)tok * C + kk), b);
          for (int i = 0; i < 8; ++i) v[i] = a[i] * sigmoidf_(b[i]);
          ra[u] = pack_bf16x8(v);
        } else {       // convolution branch
          ra[u] = ld16(xc + (long long)tok * C + (kk - C));
        }
      } else {
        ra[u] = make_uint4(0u, 0u, 0u, 0u);
      }
      rw[u] = ld16(wo + (long long)(n0 + row) * K + kk);
    }
  };
  auto store = [&](int buf) {
    for (int u = 0; u < 2; ++u) {
      const int p = tid + u * kEpThreads, row = p >> 3, c8 = (p & 7) * 8;
      *reinterpret_cast<uint4*>(&sA[buf][row * kEpP + c8]) = ra[u];
      *reinterpret_cast<uint4*>(&sW[buf][row * kEpP + c8]) = rw[u];
    }
  };
  f32x4 acc[4];
  for (int t = 0; t < 4; ++t) acc[t] = zero4();
  load(0);
  store(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load(kb + 1);
    for (int ks = 0; ks < kEpK / 32; ++ks) {
      const bf16x8 a = ld8(&sW[buf][(16 * w + r) * kEpP + 32 * ks + 8 * g]);  // outputs 16w + r
      for (int t = 0; t < 4; ++t)
        acc[t] = mma32(a, ld8(&sA[buf][(16 * t + r) * kEpP + 32 * ks + 8 * g]), acc[t]);  // tokens 16t + r
    }
    if (kb + 1 < nkb) store(buf ^ 1);
    __syncthreads();
  }
  // lane (r, g) of tile t holds y[token m0 + 16t + r][outputs n0 + 16w + 4g .. + 3]. The 64 x 64 tile
  // goes through LDS (sA[0], free after the loop's last barrier), so that y is written as whole
  // rows: 16-byte pieces, 8 lanes to a token's 128 bytes, with the nontemporal hint.
  const int oc = 16 * w + 4 * g;
  f32x4 bs = zero4();
  if (bias)
    for (int j = 0; j < 4; ++j) bs[j] = bias[n0 + oc + j];
  bf16* sY = sA[0];
  for (int t = 0; t < 4; ++t) *reinterpret_cast<bf16x4*>(&sY[(16 * t + r) * kEpP + oc]) = to_bf16x4(acc[t] + bs);
  __syncthreads();
  for (int u = 0; u < 2; ++u) {
    const int p = tid + u * kEpThreads, row = p >> 3, c8 = (p & 7) * 8, tok = m0 + row;
    if (tok < M) st16_out(y + (long long)tok * Cout + n0 + c8, ld16(&sY[row * kEpP + c8]));
  }
}

__global__ __launch_bounds__(kEpThreads) void epilogue_f32(const float* __restrict__ o,
                                                           const float* __restrict__ gate,
                                                           const float* __restrict__ xc,
                                                           const float* __restrict__ wo,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ y, int M, int C,
                                                           int Cout) {
  const long long e = (long long)blockIdx.x * kEpThreads + threadIdx.x;
  if (e >= (long long)M * Cout) return;
  const int tok = (int)(e / Cout), n = (int)(e % Cout);
  const float* row = wo + (long long)n * 2 * C;
  float acc = bias ? bias[n] : 0.f;
  for (int k = 0; k < C; ++k) {
    const long long i = (long long)tok * C + k;
    acc = fmaf(o[i] * sigmoidf_(gate[i]), row[k], acc);
  }
  for (int k = 0; k < C; ++k) acc = fmaf(xc[(long long)tok * C + k], row[C + k], acc);
  y[e] = acc;
}

}  // namespace

hipError_t epilogue_launch(bool bf16_io, int M, int C, int Cout, const void* o, const void* gate,
                           const void* xc, const void* wo, const float* bias, void* y,
                           hipStream_t st) {
  if (bf16_io) {
    const dim3 grid((unsigned)((M + kEpTok - 1) / kEpTok), (unsigned)(Cout / kEpOut));
    hipLaunchKernelGGL(epilogue_bf16, grid, dim3(kEpThreads), 0, st, (const bf16*)o, (const bf16*)gate,
                       (const bf16*)xc, (const bf16*)wo, bias, (bf16*)y, M, C, Cout);
  } else {
    const long long n = (long long)M * Cout;
    hipLaunchKernelGGL(epilogue_f32, dim3((unsigned)((n + kEpThreads - 1) / kEpThreads)), dim3(kEpThreads), 0,
                       st, (const float*)o, (const float*)gate, (const float*)xc, (const float*)wo, bias,
                       (float*)y, M, C, Cout);
  }
  return hipGetLastError();
}

}  // namespace ttt
