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
// use LDS in a fixed wave order, so results are deterministic. K, V, Q of a chunk are staged
// through double-buffered LDS; the next chunk's loads are issued before the current chunk's work.
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
__device__ __forceinline__ bf16x8 cat_tiles(f32x4 lo, f32x4 hi) {
  return cat8(to_bf16x4(lo), to_bf16x4(hi));
}

__global__ __launch_bounds__(kWaves * 64, 1) void mlp_fwd_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out) {
  __shared__ __align__(16) bf16 sKVQ[2][3][kCh * kP];
  __shared__ __align__(16) bf16 sX2[kWaves * kHw * kPt];  // -a X2^T per wave, [hidden][token]
  __shared__ __align__(16) bf16 sD1[kWaves * kHw * kPt];  // -a D1^T per wave, [hidden][token]
  __shared__ __align__(16) bf16 sE[kD * kPt];             // E^T, [feature][token]
  __shared__ __align__(16) f32x4 sRed[kWaves * 5 * 64];   // per-wave partial tiles, lane-private
  __shared__ __align__(16) bf16x4 sEt[4 * 64];            // E^T tiles, lane-private accumulator layout

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

  // Staging: threads 0..383 each move one 16-byte piece of K, V or Q (16 rows x 8 pieces each).
  // Chunk c is read from LDS buffer c & 1; chunk c + 1 is loaded into registers at the start of
  // iteration c and written to the other buffer at its end.
  const int t = threadIdx.x;
  const int prow = (t & 127) >> 3, pcol = (t & 7) * 8, which = t >> 7;
  const bf16* psrc = t < 128 ? k : (t < 256 ? v : q);
  if (t < 384) st16(&sKVQ[0][which][prow * kP + pcol], ld16(psrc + head0 + prow * ts + pcol));

  for (int c = 0; c < C; ++c) {
    const long long tok0 = head0 + (long long)c * kCh * ts;
    const bf16* sK = sKVQ[c & 1][0];
    const bf16* sV = sKVQ[c & 1][1];
    const bf16* sQ = sKVQ[c & 1][2];
    uint4 pf = make_uint4(0u, 0u, 0u, 0u);
    const bool pre = t < 384 && c + 1 < C;
    if (pre) pf = ld16(psrc + tok0 + kCh * ts + prow * ts + pcol);
    __syncthreads();

    // Z1^T (hidden x token): A = W1^T from W1t, B = K^T rows (c-layout k map).
    f32x4 X2[kNh], Gp[kNh];
    {
      bf16x8 kb[2];
      for (int ks = 0; ks < 2; ++ks) {
        const bf16* pk = &sK[r * kP + 32 * ks + 4 * g];
        kb[ks] = cat8(ld4(pk), ld4(pk + 16));
      }
      for (int n = 0; n < kNh; ++n) {
        f32x4 z = zero4();
        for (int ks = 0; ks < 2; ++ks) z = mma32(cat_tiles(W1t[2 * ks][n], W1t[2 * ks + 1][n]), kb[ks], z);
        for (int j = 0; j < 4; ++j) {
          const float x = z[j];
          const float cdf = 0.5f * (1.f + erff(x * 0.70710678118654752440f));
          X2[n][j] = x * cdf;                                                       // GELU
          Gp[n][j] = cdf + x * expf(-0.5f * x * x) * 0.39894228040143267794f;      // GELU'
        }
      }
    }

    // Z2^T partial (output x token) over this wave's hidden slice: A = W2^T (from W2t), B = X2^T.
    for (int o2 = 0; o2 < 4; ++o2) {
      f32x4 acc = zero4();
      for (int kh = 0; kh < kNh / 2; ++kh)
        acc = mma32(cat_tiles(W2t[2 * kh][o2], W2t[2 * kh + 1][o2]),
                    cat_tiles(X2[2 * kh], X2[2 * kh + 1]), acc);
      sRed[(w * 5 + o2) * 64 + l] = acc;
    }
    for (int n = 0; n < kNh; ++n)
      for (int j = 0; j < 4; ++j) myX2[(16 * n + 4 * g + j) * kPt + r] = (bf16)(-a * X2[n][j]);
    __syncthreads();

    // Waves 0..3: E^T tile w = sum over waves (fixed order) of Z2^T - V^T; shared as bf16 twice:
    // [feature][token] rows (sE) and the lane-private accumulator layout (sEt).
    if (w < 4) {
      f32x4 s = sRed[w * 64 + l];
      for (int ww = 1; ww < kWaves; ++ww) s = s + sRed[(ww * 5 + w) * 64 + l];
      const bf16x4 vv = ld4(&sV[r * kP + 16 * w + 4 * g]);
      bf16x4 eb;
      for (int j = 0; j < 4; ++j) {
        eb[j] = (bf16)(s[j] - (float)vv[j]);
        sE[(16 * w + 4 * g + j) * kPt + r] = eb[j];
      }
      sEt[w * 64 + l] = eb;
    }
    __syncthreads();

    // dX2^T = W2 E^T (hidden x token): A = W2 rows (from W2x), B = E^T. D1^T = dX2^T * GELU'(Z1^T).
    {
      bf16x8 eb[2];
      for (int ko = 0; ko < 2; ++ko) eb[ko] = cat8(sEt[(2 * ko) * 64 + l], sEt[(2 * ko + 1) * 64 + l]);
      for (int n = 0; n < kNh; ++n) {
        f32x4 acc = zero4();
        for (int ko = 0; ko < 2; ++ko) acc = mma32(cat_tiles(W2x[2 * ko][n], W2x[2 * ko + 1][n]), eb[ko], acc);
        for (int j = 0; j < 4; ++j) myD1[(16 * n + 4 * g + j) * kPt + r] = (bf16)(-a * acc[j] * Gp[n][j]);
      }
    }
    // The wave reads its D1 rows back across lanes below. A wave-local LDS wait was measured to be
    // insufficient here (nondeterministic results), so this is a full workgroup barrier.
    __syncthreads();
    // Read-out. Mt[t' = 4g + j][t = r] = k_t' . q_t, kept for t' <= t.
    f32x4 Mt = zero4();
    for (int ks = 0; ks < 2; ++ks)
      Mt = mma32(ld8(&sK[r * kP + 32 * ks + 8 * g]), ld8(&sQ[r * kP + 32 * ks + 8 * g]), Mt);
    for (int j = 0; j < 4; ++j)
      if (4 * g + j > r) Mt[j] = 0.f;
    const bf16x4 Mb = to_bf16x4(Mt);
    // Z1q^T = W1^T Q^T + (-a D1^T) tril(Q K^T)^T (the wave's own D1 rows, written above).
    f32x4 X2q[kNh];
    {
      bf16x8 qb[2];
      for (int ks = 0; ks < 2; ++ks) {
        const bf16* pq = &sQ[r * kP + 32 * ks + 4 * g];
        qb[ks] = cat8(ld4(pq), ld4(pq + 16));
      }
      for (int n = 0; n < kNh; ++n) {
        f32x4 z = zero4();
        for (int ks = 0; ks < 2; ++ks) z = mma32(cat_tiles(W1t[2 * ks][n], W1t[2 * ks + 1][n]), qb[ks], z);
        z = mma16(ld4(&myD1[(16 * n + r) * kPt + 4 * g]), Mb, z);
        for (int j = 0; j < 4; ++j) X2q[n][j] = gelu_f(z[j]);
      }
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

    // Waves 0..3 finish output tile w: O^T = sum of partials - a E^T tril(X2q X2^T)^T; store.
    if (w < 4) {
      f32x4 s = sRed[w * 64 + l];
      f32x4 n2 = sRed[4 * 64 + l];
      for (int ww = 1; ww < kWaves; ++ww) {
        s = s + sRed[(ww * 5 + w) * 64 + l];
        n2 = n2 + sRed[(ww * 5 + 4) * 64 + l];
      }
      for (int j = 0; j < 4; ++j)
        if (4 * g + j > r) n2[j] = 0.f;
      s = mma16(ld4(&sE[(16 * w + r) * kPt + 4 * g]), to_bf16x4_scaled(n2, -a), s);
      *reinterpret_cast<bf16x4*>(o + tok0 + r * ts + 16 * w + 4 * g) = to_bf16x4(s);
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
    if (pre) st16(&sKVQ[(c + 1) & 1][which][prow * kP + pcol], pf);
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
