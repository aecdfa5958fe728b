// Causal mini-batch TTT-MLP forward (TTT-Linear / TTT-MLP abstract: the hidden state is a
// two-layer MLP trained by a self-supervised step; mini-batches: Vision-TTT summary on
// gist.science, "Methodologie" item 3).
//
// Inner model f(x) = GELU(x W1) W2, W1 [D, Dh], W2 [Dh, D], loss 1/2 ||f(k) - v||^2 per token.
// Per chunk of b tokens with start state (W1, W2), all gradients taken at the start state
// (dual form of the primal per-token definition):
//   Z1 = K W1, X2 = GELU(Z1), E = X2 W2 - V, D1 = (E W2^T) * GELU'(Z1)
//   Z1q = Q W1 - a tril(Q K^T) D1,  X2q = GELU(Z1q),  O = X2q W2 - a tril(X2q X2^T) E
//   W1 <- W1 - a K^T D1,  W2 <- W2 - a X2^T E,   a = eta / b, tril keeps the diagonal.
//
// One workgroup per (batch, head), 8 waves; wave w owns hidden units [32w, 32w + 32): its slice
// of W1 (columns), of W2 (rows) and a second copy of its W2 slice in transposed accumulator
// layout (needed as the operand of E W2^T). All three stay in MFMA accumulator registers for the
// whole sequence and are updated in place by MFMA. The per-chunk products are computed
// transposed (hidden x token) so each product's accumulator tile feeds the next product's B
// operand directly; only the small per-chunk activations (X2, D1, E: tokens x features, bf16) go
// through LDS for transposes. Cross-wave sums over the hidden dimension (Z2 and the read-out)
// use LDS in a fixed wave order, so results are deterministic.
#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kD = 64;        // feature dim
constexpr int kDh = 256;      // hidden width
constexpr int kCh = 16;       // tokens per chunk
constexpr int kWaves = 8;
constexpr int kHw = kDh / kWaves;  // hidden units per wave
constexpr int kNh = kHw / 16;      // 16-unit hidden tiles per wave
constexpr int kP = kD + 8;         // pitch of the K/V/Q tiles (elements)
constexpr int kPt = 24;            // pitch of [row][token] tiles (16 tokens + pad)

__device__ __forceinline__ float gelu_f(float x) {
  return 0.5f * x * (1.f + erff(x * 0.70710678118654752440f));
}
// d/dx x Phi(x) = Phi(x) + x phi(x)
__device__ __forceinline__ float gelu_d(float x) {
  return 0.5f * (1.f + erff(x * 0.70710678118654752440f)) +
         x * expf(-0.5f * x * x) * 0.39894228040143267794f;
}

__device__ __forceinline__ bf16x8 cat_tiles(f32x4 lo, f32x4 hi) {
  return cat8(to_bf16x4(lo), to_bf16x4(hi));
}

__global__ __launch_bounds__(kWaves * 64, 1) void mlp_fwd_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out) {
  __shared__ __align__(16) bf16 sK[kCh * kP];
  __shared__ __align__(16) bf16 sV[kCh * kP];
  __shared__ __align__(16) bf16 sQ[kCh * kP];
  __shared__ __align__(16) bf16 sX2[kWaves * kHw * kPt];  // -a X2^T per wave, [hidden][token]
  __shared__ __align__(16) bf16 sD1[kWaves * kHw * kPt];  // -a D1^T per wave, [hidden][token]
  __shared__ __align__(16) bf16 sE[kD * kPt];             // E^T, [feature][token]
  __shared__ __align__(16) f32x4 sRed[kWaves * 5 * 64];   // per-wave partial tiles, lane-private

  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const long long ts = (long long)H * kD;
  const float* W1g = w1 + b * wbs + (long long)h * kD * kDh;
  const float* W2g = w2 + b * wbs + (long long)h * kDh * kD;
  const int hid0 = kHw * w;

  // W1t[m][n]:  W1[16m + 4g + j][hid0 + 16n + r]   (rows: features, cols: hidden)
  // W2t[n][o]:  W2[hid0 + 16n + 4g + j][16o + r]   (rows: hidden,   cols: outputs)
  // W2x[o][n]:  W2[hid0 + 16n + r][16o + 4g + j]   (the same slice, transposed layout)
  f32x4 W1t[4][kNh], W2t[kNh][4], W2x[4][kNh];
  for (int m = 0; m < 4; ++m)
    for (int n = 0; n < kNh; ++n)
      for (int j = 0; j < 4; ++j) {
        W1t[m][n][j] = W1g[(16 * m + 4 * g + j) * kDh + hid0 + 16 * n + r];
        W2t[n][m][j] = W2g[(hid0 + 16 * n + 4 * g + j) * kD + 16 * m + r];
        W2x[m][n][j] = W2g[(hid0 + 16 * n + r) * kD + 16 * m + 4 * g + j];
      }

  bf16* myX2 = sX2 + w * kHw * kPt;
  bf16* myD1 = sD1 + w * kHw * kPt;
  const int C = N / kCh;
  const long long head0 = (long long)b * N * ts + (long long)h * kD;

  for (int c = 0; c < C; ++c) {
    const long long tok0 = head0 + (long long)c * kCh * ts;
    __syncthreads();
    {  // stage K, V, Q: 16 rows x 8 chunks of 16 B each
      const int t = threadIdx.x;
      const int row = (t & 127) >> 3, col = (t & 7) * 8;
      const bf16* src = t < 128 ? k : (t < 256 ? v : q);
      bf16* dst = t < 128 ? sK : (t < 256 ? sV : sQ);
      if (t < 384) st16(&dst[row * kP + col], ld16(src + tok0 + row * ts + col));
    }
    __syncthreads();

    // Z1^T, Z1q^T (hidden x token): A = W1^T from W1t, B = K^T / Q^T rows (c-layout k map).
    f32x4 Z1[kNh], Z1q[kNh];
    bf16x8 kb[2], qb[2];
    for (int ks = 0; ks < 2; ++ks) {
      const bf16* pk = &sK[r * kP + 32 * ks + 4 * g];
      const bf16* pq = &sQ[r * kP + 32 * ks + 4 * g];
      kb[ks] = cat8(ld4(pk), ld4(pk + 16));
      qb[ks] = cat8(ld4(pq), ld4(pq + 16));
    }
    for (int n = 0; n < kNh; ++n) {
      Z1[n] = zero4();
      Z1q[n] = zero4();
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 aw = cat_tiles(W1t[2 * ks][n], W1t[2 * ks + 1][n]);
        Z1[n] = mma32(aw, kb[ks], Z1[n]);
        Z1q[n] = mma32(aw, qb[ks], Z1q[n]);
      }
    }
    // Mt[t' = 4g + j][t = r] = k_t' . q_t
    f32x4 Mt = zero4();
    for (int ks = 0; ks < 2; ++ks)
      Mt = mma32(ld8(&sK[r * kP + 32 * ks + 8 * g]), ld8(&sQ[r * kP + 32 * ks + 8 * g]), Mt);

    f32x4 X2[kNh], Gp[kNh];
    for (int n = 0; n < kNh; ++n)
      for (int j = 0; j < 4; ++j) {
        X2[n][j] = gelu_f(Z1[n][j]);
        Gp[n][j] = gelu_d(Z1[n][j]);
      }

    // Z2^T partial (output x token) over this wave's hidden slice: A = W2^T (from W2t), B = X2^T.
    for (int o2 = 0; o2 < 4; ++o2) {
      f32x4 acc = zero4();
      for (int kh = 0; kh < kNh / 2; ++kh)
        acc = mma32(cat_tiles(W2t[2 * kh][o2], W2t[2 * kh + 1][o2]),
                    cat_tiles(X2[2 * kh], X2[2 * kh + 1]), acc);
      sRed[(w * 5 + o2) * 64 + l] = acc;
    }
    __syncthreads();

    // E^T = sum over waves (fixed order) of Z2^T - V^T, all four output tiles.
    f32x4 Et[4];
    for (int o2 = 0; o2 < 4; ++o2) {
      f32x4 s = sRed[o2 * 64 + l];
      for (int ww = 1; ww < kWaves; ++ww) s = s + sRed[(ww * 5 + o2) * 64 + l];
      const bf16x4 vv = ld4(&sV[r * kP + 16 * o2 + 4 * g]);
      for (int j = 0; j < 4; ++j) Et[o2][j] = s[j] - (float)vv[j];
      if (o2 == w)
        for (int j = 0; j < 4; ++j) sE[(16 * o2 + 4 * g + j) * kPt + r] = (bf16)Et[o2][j];
    }
    for (int n = 0; n < kNh; ++n)
      for (int j = 0; j < 4; ++j) myX2[(16 * n + 4 * g + j) * kPt + r] = (bf16)(-a * X2[n][j]);

    // dX2^T = W2 E^T (hidden x token): A = W2 rows (from W2x), B = E^T. D1^T = dX2^T * GELU'(Z1^T).
    for (int n = 0; n < kNh; ++n) {
      f32x4 acc = zero4();
      for (int ko = 0; ko < 2; ++ko)
        acc = mma32(cat_tiles(W2x[2 * ko][n], W2x[2 * ko + 1][n]),
                    cat_tiles(Et[2 * ko], Et[2 * ko + 1]), acc);
      for (int j = 0; j < 4; ++j) myD1[(16 * n + 4 * g + j) * kPt + r] = (bf16)(-a * acc[j] * Gp[n][j]);
    }
    __syncthreads();

    // Z1q^T += (-a D1^T) tril(Q K^T)^T: A = D1^T rows (LDS), B = Mt with t' <= t kept.
    f32x4 Mm = Mt;
    for (int j = 0; j < 4; ++j)
      if (4 * g + j > r) Mm[j] = 0.f;
    const bf16x4 Mb = to_bf16x4(Mm);
    f32x4 X2q[kNh];
    for (int n = 0; n < kNh; ++n) {
      Z1q[n] = mma16(ld4(&myD1[(16 * n + r) * kPt + 4 * g]), Mb, Z1q[n]);
      for (int j = 0; j < 4; ++j) X2q[n][j] = gelu_f(Z1q[n][j]);
    }

    // O^T partial = W2^T X2q^T, and N2^T partial = X2 X2q^T (token x token), this wave's hidden slice.
    for (int o2 = 0; o2 < 4; ++o2) {
      f32x4 acc = zero4();
      for (int kh = 0; kh < kNh / 2; ++kh)
        acc = mma32(cat_tiles(W2t[2 * kh][o2], W2t[2 * kh + 1][o2]),
                    cat_tiles(X2q[2 * kh], X2q[2 * kh + 1]), acc);
      sRed[(w * 5 + o2) * 64 + l] = acc;
    }
    {
      f32x4 acc = zero4();
      for (int kh = 0; kh < kNh / 2; ++kh)
        acc = mma32(cat_tiles(X2[2 * kh], X2[2 * kh + 1]), cat_tiles(X2q[2 * kh], X2q[2 * kh + 1]), acc);
      sRed[(w * 5 + 4) * 64 + l] = acc;
    }
    __syncthreads();

    // Wave w finishes output tile w: O^T = sum of partials - a E^T tril(X2q X2^T)^T; store.
    for (int o2 = 0; o2 < 4; ++o2) {
      if (o2 != w) continue;
      f32x4 s = sRed[o2 * 64 + l];
      f32x4 n2 = sRed[4 * 64 + l];
      for (int ww = 1; ww < kWaves; ++ww) {
        s = s + sRed[(ww * 5 + o2) * 64 + l];
        n2 = n2 + sRed[(ww * 5 + 4) * 64 + l];
      }
      for (int j = 0; j < 4; ++j)
        if (4 * g + j > r) n2[j] = 0.f;
      s = mma16(ld4(&sE[(16 * o2 + r) * kPt + 4 * g]), to_bf16x4_scaled(n2, -a), s);
      *reinterpret_cast<bf16x4*>(o + tok0 + r * ts + 16 * o2 + 4 * g) = to_bf16x4(s);
    }

    // State updates at the end of the chunk (the read-out above used the start state).
    for (int n = 0; n < kNh; ++n) {
      const bf16x4 d1 = ld4(&myD1[(16 * n + r) * kPt + 4 * g]);   // (-a D1)[t][hidden]
      const bf16x4 x2 = ld4(&myX2[(16 * n + r) * kPt + 4 * g]);   // (-a X2)[t][hidden]
      for (int m = 0; m < 4; ++m)  // W1 += K^T (-a D1)
        W1t[m][n] = mma16(ld4_col(&sK[(4 * g) * kP + 16 * m + r], kP), d1, W1t[m][n]);
      for (int o2 = 0; o2 < 4; ++o2) {
        const bf16x4 e = ld4(&sE[(16 * o2 + r) * kPt + 4 * g]);  // E[t][out]
        W2t[n][o2] = mma16(x2, e, W2t[n][o2]);   // W2   += (-a X2)^T E
        W2x[o2][n] = mma16(e, x2, W2x[o2][n]);   // W2^T += E^T (-a X2)
      }
    }
  }

  const long long bhl = bh;
  if (w1_out) {
    float* dst = w1_out + bhl * kD * kDh;
    for (int m = 0; m < 4; ++m)
      for (int n = 0; n < kNh; ++n)
        for (int j = 0; j < 4; ++j) dst[(16 * m + 4 * g + j) * kDh + hid0 + 16 * n + r] = W1t[m][n][j];
  }
  if (w2_out) {
    float* dst = w2_out + bhl * kDh * kD;
    for (int n = 0; n < kNh; ++n)
      for (int o2 = 0; o2 < 4; ++o2)
        for (int j = 0; j < 4; ++j) dst[(hid0 + 16 * n + 4 * g + j) * kD + 16 * o2 + r] = W2t[n][o2][j];
  }
}

}  // namespace

size_t mlp_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t mlp_launch(int B, int H, int N, int D, int Dh, int chunk, float eta, const void* q,
                      const void* k, const void* v, const float* w1, const float* w2,
                      long long wbs, void* o, float* w1_out, float* w2_out, void*, hipStream_t st) {
  if (D != kD || Dh != kDh || chunk != kCh) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mlp_fwd_bf16, dim3(B * H), dim3(kWaves * 64), 0, st, (const bf16*)q, (const bf16*)k,
                     (const bf16*)v, w1, w2, wbs, H, N, eta / (float)chunk, (bf16*)o, w1_out,
                     w2_out);
  return hipGetLastError();
}

}  // namespace ttt
