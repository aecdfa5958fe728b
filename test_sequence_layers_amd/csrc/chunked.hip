// Chunked TTT-Linear forward: causal mini-batch TTT-Linear and the bidirectional scan.
//
// Per (batch, head) and chunk c of b tokens with start state W_s (mini-batch gradient descent,
// Vision-TTT summary on gist.science, "Methodologie" items 1 and 3):
//   E_c    = K_c W_s - V_c                       residuals at the chunk's start state
//   W_next = W_s - (eta/b) K_c^T E_c             one averaged gradient step
// Causal read-out (TTT-Linear; token i sees the gradients of tokens j <= i of its chunk):
//   O_c = Q_c W_s - (eta/b) tril(Q_c K_c^T) E_c  (dual form of q_i (W_s - (eta/b) sum_{j<=i} ...))
// Bidirectional read-out (Vision-TTT, "Methodologie" item 2): each chunk is read out after its own
// update by a forward scan and by a scan of the reversed sequence from the same W0; the two are
// summed: O_c = Q_c (W^f_c + W^r_c), where W^r_c is the reverse scan's state after chunk c.
//
// The d output columns of W are independent regressions (column j of the update only involves
// column j of W and V), so wave w of a workgroup owns columns [16w, 16w + 16) of the state and
// keeps them in MFMA accumulator layout for the whole scan; no state ever leaves registers
// between chunks. K, V, Q of one chunk are staged through LDS.
#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

enum ScanMode { kCausal = 0, kReverseStore = 1, kForwardBoth = 2 };

// Stage a [CH x D] bf16 tile (token stride ts) into LDS with row pitch P.
template <int D, int CH, int P, int NTH>
__device__ __forceinline__ void stage_chunk(bf16* dst, const bf16* src, long long ts) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < CH * CPR; c += NTH) {
    const int row = c / CPR, col = (c % CPR) * 8;
    st16(dst + row * P + col, ld16(src + row * ts + col));
  }
}

// Write a [CH x D] bf16 tile from LDS to global memory.
template <int D, int CH, int P, int NTH>
__device__ __forceinline__ void store_chunk(bf16* dst, const bf16* src, long long ts) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < CH * CPR; c += NTH) {
    const int row = c / CPR, col = (c % CPR) * 8;
    st16(dst + row * ts + col, ld16(src + row * P + col));
  }
}

// A operand: 16 rows of a row-major LDS tile (pitch P) starting at `row0`, features
// [32ks, 32ks + 32) in the c-layout k map (matching a state held in C layout).
template <int P>
__device__ __forceinline__ bf16x8 a_rows_clayout(const bf16* t, int row0, int ks, int r, int g) {
  const bf16* p = t + (row0 + r) * P + 32 * ks + 4 * g;
  return cat8(ld4(p), ld4(p + 16));
}

// B operand from a state held in C layout (tiles m = 2ks, 2ks + 1 cover features 32ks..32ks+31).
__device__ __forceinline__ bf16x8 b_state(const f32x4* W, int ks) {
  return cat8(to_bf16x4(W[2 * ks]), to_bf16x4(W[2 * ks + 1]));
}

// Y[16 tokens x 16 cols] = X_rows(row0..row0+15) . W[:, cols] + init, contraction over D.
template <int D, int P>
__device__ __forceinline__ f32x4 rows_times_state(const bf16* X, int row0, const f32x4* W,
                                                  f32x4 init, int r, int g) {
  if constexpr (D >= 32) {
    for (int ks = 0; ks < D / 32; ++ks) init = mma32(a_rows_clayout<P>(X, row0, ks, r, g), b_state(W, ks), init);
  } else {
    init = mma16(ld4(X + (row0 + r) * P + 4 * g), to_bf16x4(W[0]), init);
  }
  return init;
}

template <int D, int CH, int MODE>
__global__ __launch_bounds__(D / 16 * 64) void chunk_scan_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w0, long long w0_bstride, int H, int N, float a,
    float* __restrict__ states, bf16* __restrict__ o, float* __restrict__ w_out) {
  constexpr int P = D + 8;
  constexpr int NT = D / 16;   // waves = column tiles = row tiles
  constexpr int NP = CH / 16;  // 16-token tiles per chunk
  constexpr int NTH = NT * 64;
  __shared__ __align__(16) bf16 sK[CH * P];
  __shared__ __align__(16) bf16 sV[CH * P];
  __shared__ __align__(16) bf16 sQ[CH * P];
  __shared__ __align__(16) bf16 sO[CH * P];

  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int C = N / CH;
  const long long ts = (long long)H * D;
  const long long dd = (long long)D * D;
  const float* W0 = w0 + b * w0_bstride + h * dd;

  f32x4 W[NT];  // W[16m + 4g + j][16w + r]
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j) W[m][j] = W0[(16 * m + 4 * g + j) * D + 16 * w + r];

  const long long head0 = (long long)b * N * ts + (long long)h * D;
  float* st_bh = states ? states + bh * (long long)C * dd : nullptr;

  for (int it = 0; it < C; ++it) {
    const int c = (MODE == kReverseStore) ? C - 1 - it : it;
    const long long tok0 = head0 + (long long)c * CH * ts;
    __syncthreads();
    stage_chunk<D, CH, P, NTH>(sK, k + tok0, ts);
    stage_chunk<D, CH, P, NTH>(sV, v + tok0, ts);
    if (MODE != kReverseStore) stage_chunk<D, CH, P, NTH>(sQ, q + tok0, ts);
    __syncthreads();

    // E_p = K_p W_s - V_p for the wave's 16 columns (C layout: row = token 16p + 4g + j).
    f32x4 E[NP];
    for (int p = 0; p < NP; ++p) {
      f32x4 init;
      for (int j = 0; j < 4; ++j) init[j] = -(float)sV[(16 * p + 4 * g + j) * P + 16 * w + r];
      E[p] = rows_times_state<D, P>(sK, 16 * p, W, init, r, g);
    }

    if constexpr (MODE == kCausal) {
      // O_p = Q_p W_s - a * sum_{p' <= p} tril(P_{p p'}) E_{p'},  P = Q K^T.
      for (int p = 0; p < NP; ++p) {
        f32x4 acc = rows_times_state<D, P>(sQ, 16 * p, W, zero4(), r, g);
        for (int pp = 0; pp <= p; ++pp) {
          // Pt[t' = 16pp + 4g + j][t = 16p + r] = k_t' . q_t
          f32x4 pt = zero4();
          if constexpr (D >= 32) {
            for (int ks = 0; ks < D / 32; ++ks)
              pt = mma32(ld8(&sK[(16 * pp + r) * P + 32 * ks + 8 * g]),
                         ld8(&sQ[(16 * p + r) * P + 32 * ks + 8 * g]), pt);
          } else {
            pt = mma16(ld4(&sK[(16 * pp + r) * P + 4 * g]), ld4(&sQ[(16 * p + r) * P + 4 * g]), pt);
          }
          if (pp == p)
            for (int j = 0; j < 4; ++j)
              if (4 * g + j > r) pt[j] = 0.f;
          // A = -a P (row t = lane r, k = t' = 4g + j), B = E_{p'} (k = t', column = lane r).
          acc = mma16(to_bf16x4_scaled(pt, -a), to_bf16x4(E[pp]), acc);
        }
        for (int j = 0; j < 4; ++j) sO[(16 * p + 4 * g + j) * P + 16 * w + r] = (bf16)acc[j];
      }
    }

    // W += (-a K^T) E: A = K^T (row = feature 16m + r, k = token 16p + 4g + j), B = -a E_p.
    for (int p = 0; p < NP; ++p) {
      const bf16x4 eb = to_bf16x4_scaled(E[p], -a);
      for (int m = 0; m < NT; ++m)
        W[m] = mma16(ld4_col(&sK[(16 * p + 4 * g) * P + 16 * m + r], P), eb, W[m]);
    }

    if constexpr (MODE == kReverseStore) {
      f32x4* dst = reinterpret_cast<f32x4*>(st_bh + c * dd);
      for (int m = 0; m < NT; ++m) dst[(w * NT + m) * 64 + l] = W[m];
    }
    if constexpr (MODE == kForwardBoth) {
      const f32x4* src = reinterpret_cast<const f32x4*>(st_bh + c * dd);
      f32x4 Ws[NT];
      for (int m = 0; m < NT; ++m) Ws[m] = W[m] + src[(w * NT + m) * 64 + l];
      for (int p = 0; p < NP; ++p) {
        const f32x4 acc = rows_times_state<D, P>(sQ, 16 * p, Ws, zero4(), r, g);
        for (int j = 0; j < 4; ++j) sO[(16 * p + 4 * g + j) * P + 16 * w + r] = (bf16)acc[j];
      }
    }
    if constexpr (MODE != kReverseStore) {
      __syncthreads();
      store_chunk<D, CH, P, NTH>(o + tok0, sO, ts);
    }
  }

  if (w_out) {
    float* dst = w_out + (MODE == kReverseStore ? (long long)gridDim.x * dd : 0) + bh * dd;
    for (int m = 0; m < NT; ++m)
      for (int j = 0; j < 4; ++j) dst[(16 * m + 4 * g + j) * D + 16 * w + r] = W[m][j];
  }
}

// ---------------------------------------------------------------- fp32 I/O, plain FMA
// One workgroup per (b, h); the state lives in LDS and tokens are processed one by one in the
// primal form (weights of each token materialised), in true fp32.
template <int D, int MODE>
__global__ __launch_bounds__(256) void chunk_scan_f32(const float* __restrict__ q,
                                                      const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      const float* __restrict__ w0,
                                                      long long w0_bstride, int H, int N, int CH,
                                                      float a, float* __restrict__ states,
                                                      float* __restrict__ o,
                                                      float* __restrict__ w_out) {
  __shared__ float sW[D][D + 1], sS[D][D + 1];
  __shared__ float sk[D], sq[D], se[D];
  constexpr int PER = (D * D + 255) / 256;
  const int bh = blockIdx.x, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int C = N / CH;
  const long long ts = (long long)H * D, dd = (long long)D * D;
  const float* W0 = w0 + b * w0_bstride + h * dd;
  for (int e = tid; e < D * D; e += 256) sW[e / D][e % D] = W0[e];
  const long long head0 = (long long)b * N * ts + (long long)h * D;
  float* st_bh = states ? states + bh * (long long)C * dd : nullptr;
  for (int it = 0; it < C; ++it) {
    const int c = (MODE == kReverseStore) ? C - 1 - it : it;
    for (int e = tid; e < D * D; e += 256) sS[e / D][e % D] = 0.f;
    __syncthreads();
    for (int i = 0; i < CH; ++i) {
      const long long off = head0 + ((long long)c * CH + i) * ts;
      if (tid < D) {
        sk[tid] = k[off + tid];
        sq[tid] = (MODE == kReverseStore) ? 0.f : q[off + tid];
      }
      __syncthreads();
      if (tid < D) {  // e = k W_s - v
        float acc = -v[off + tid];
        for (int j = 0; j < D; ++j) acc = fmaf(sk[j], sW[j][tid], acc);
        se[tid] = acc;
      }
      __syncthreads();
      for (int u = 0; u < PER; ++u) {  // S += k^T e
        const int e = tid + 256 * u;
        if (e < D * D) sS[e / D][e % D] = fmaf(sk[e / D], se[e % D], sS[e / D][e % D]);
      }
      __syncthreads();
      if (MODE == kCausal && tid < D) {  // o_i = q_i (W_s - a S_i)
        float acc = 0.f;
        for (int j = 0; j < D; ++j) acc = fmaf(sq[j], fmaf(-a, sS[j][tid], sW[j][tid]), acc);
        o[off + tid] = acc;
      }
      __syncthreads();
    }
    for (int e = tid; e < D * D; e += 256) sW[e / D][e % D] = fmaf(-a, sS[e / D][e % D], sW[e / D][e % D]);
    __syncthreads();
    if (MODE == kReverseStore)
      for (int e = tid; e < D * D; e += 256) st_bh[c * dd + e] = sW[e / D][e % D];
    if (MODE == kForwardBoth) {
      for (int e = tid; e < D * D; e += 256) sS[e / D][e % D] = sW[e / D][e % D] + st_bh[c * dd + e];
      __syncthreads();
      for (int e = tid; e < CH * D; e += 256) {
        const int i = e / D, col = e % D;
        const long long off = head0 + ((long long)c * CH + i) * ts;
        float acc = 0.f;
        for (int j = 0; j < D; ++j) acc = fmaf(q[off + j], sS[j][col], acc);
        o[off + col] = acc;
      }
    }
    __syncthreads();
  }
  if (w_out) {
    float* dst = w_out + (MODE == kReverseStore ? (long long)gridDim.x * dd : 0) + bh * dd;
    for (int e = tid; e < D * D; e += 256) dst[e] = sW[e / D][e % D];
  }
}

template <int D, int CH>
hipError_t launch_bf16(bool bidir, int B, int H, int N, float a, const void* q, const void* k,
                       const void* v, const float* w0, long long w0s, void* o, float* w_out,
                       void* ws, hipStream_t st) {
  const int BH = B * H;
  const dim3 grid(BH), block(D / 16 * 64);
  if (!bidir) {
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kCausal>), grid, block, 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, nullptr, (bf16*)o, w_out);
  } else {
    float* states = static_cast<float*>(ws);
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kReverseStore>), grid, block, 0, st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, states,
                       (bf16*)o, w_out);
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kForwardBoth>), grid, block, 0, st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, states,
                       (bf16*)o, w_out);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(bool bidir, int B, int H, int N, int CH, float a, const void* q,
                      const void* k, const void* v, const float* w0, long long w0s, void* o,
                      float* w_out, void* ws, hipStream_t st) {
  const int BH = B * H;
  if (!bidir) {
    hipLaunchKernelGGL((chunk_scan_f32<D, kCausal>), dim3(BH), dim3(256), 0, st, (const float*)q,
                       (const float*)k, (const float*)v, w0, w0s, H, N, CH, a, nullptr,
                       (float*)o, w_out);
  } else {
    float* states = static_cast<float*>(ws);
    hipLaunchKernelGGL((chunk_scan_f32<D, kReverseStore>), dim3(BH), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, w0, w0s, H, N, CH, a,
                       states, (float*)o, w_out);
    hipLaunchKernelGGL((chunk_scan_f32<D, kForwardBoth>), dim3(BH), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, w0, w0s, H, N, CH, a,
                       states, (float*)o, w_out);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(bool bidir, int B, int H, int N, int CH, float a, const void* q,
                         const void* k, const void* v, const float* w0, long long w0s, void* o,
                         float* w_out, void* ws, hipStream_t st) {
  switch (CH) {
    case 16: return launch_bf16<D, 16>(bidir, B, H, N, a, q, k, v, w0, w0s, o, w_out, ws, st);
    case 32: return launch_bf16<D, 32>(bidir, B, H, N, a, q, k, v, w0, w0s, o, w_out, ws, st);
    case 64: return launch_bf16<D, 64>(bidir, B, H, N, a, q, k, v, w0, w0s, o, w_out, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t chunked_workspace_bytes(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk) {
  (void)bf16_io;
  (void)chunk;
  if (!bidir) return 0;
  // reverse-scan state after every chunk: C * D * D fp32 per (b, h)
  return (size_t)B * H * (size_t)N / (size_t)chunk * D * D * sizeof(float);
}

hipError_t chunked_launch(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk,
                          float eta, const void* q, const void* k, const void* v, const float* w0,
                          long long w0s, void* o, float* w_out, void* ws, hipStream_t st) {
  const float a = eta / (float)chunk;
  if (bf16_io) {
    switch (D) {
      case 16: return launch_bf16_d<16>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st);
      case 32: return launch_bf16_d<32>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st);
      case 64: return launch_bf16_d<64>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (D) {
    case 16: return launch_f32<16>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st);
    case 32: return launch_f32<32>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st);
    case 64: return launch_f32<64>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
