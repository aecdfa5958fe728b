// Full-batch single-step TTT-Linear forward (ViT^3 review on techloop.online, design-space study:
// single epoch, full batch, inner learning rate 1.0; "core idea": train on (K, V), read out Q):
//   W* = W0 - (eta/N) K^T (K W0 - V),  O = Q W*   for every (batch, head).
//
// Three launches on the caller's stream:
//   1. fb_partial: grid (splits, B*H). Each workgroup streams a token range of one (b, h) through
//      LDS and accumulates the partial gradient G_s = K_s^T (K_s W0 - V_s) with MFMA.
//   2. fb_reduce:  grid (B*H). Sums the split partials in a fixed order (deterministic) and forms W*.
//   3. fb_readout: grid (splits, B*H). Streams Q and writes O = Q W*.
// HBM traffic is the algorithmic Q, K, V read plus the O write; the partials are d x d fp32 per
// split and stay in L2 / Infinity Cache.
#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kTile = 64;      // tokens per staged tile (bf16 path)
constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kTileF = 32;     // tokens per staged tile (fp32 path)

// Stage a [64 x D] bf16 tile into LDS (row pitch P); rows >= valid become zeros, which adds
// nothing to K^T (K W0 - V).
template <int D, int P>
__device__ __forceinline__ void stage_bf16(bf16* dst, const bf16* src, long long ts, int valid) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < kTile * CPR; c += kThreads) {
    const int row = c / CPR, col = (c % CPR) * 8;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (row < valid) val = ld16(src + row * ts + col);
    st16(dst + row * P + col, val);
  }
}

// ---------------------------------------------------------------- bf16 I/O, MFMA
template <int D>
__global__ __launch_bounds__(kThreads) void fb_partial_bf16(
    const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ w0,
    long long w0_bstride, int H, int N, int tps, int S, float* __restrict__ partial) {
  constexpr int P = D + 8;     // LDS row pitch (elements); +16 B keeps row reads conflict-free
  constexpr int NT = D / 16;   // 16-column tiles of W / G
  constexpr int WPT = 4 / NT;  // waves sharing one column tile; they split the 16-token sub-tiles
  __shared__ __align__(16) bf16 sK[kTile * P];
  __shared__ __align__(16) bf16 sV[kTile * P];
  __shared__ float sG[4 * D * 16];

  const int s = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh % H;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int n = w % NT, tw = w / NT;
  const long long ts = (long long)H * D;
  const float* W0 = w0 + b * w0_bstride + (long long)h * D * D;

  // B operand fragments of W0[:, 16n .. 16n+16), contiguous k map.
  constexpr int KS = D >= 32 ? D / 32 : 1;
  bf16x8 wb[KS];
  bf16x4 wb4;
  if constexpr (D >= 32) {
    for (int ks = 0; ks < KS; ++ks)
      for (int i = 0; i < 8; ++i) wb[ks][i] = (bf16)W0[(32 * ks + 8 * g + i) * D + 16 * n + r];
  } else {
    for (int i = 0; i < 4; ++i) wb4[i] = (bf16)W0[(4 * g + i) * D + 16 * n + r];
  }

  f32x4 G[NT];
  for (int m = 0; m < NT; ++m) G[m] = zero4();

  const long long base = ((long long)b * N + n0) * ts + (long long)h * D;
  for (int t0 = n0; t0 < n1; t0 += kTile) {
    __syncthreads();
    stage_bf16<D, P>(sK, k + base + (long long)(t0 - n0) * ts, ts, n1 - t0);
    stage_bf16<D, P>(sV, v + base + (long long)(t0 - n0) * ts, ts, n1 - t0);
    __syncthreads();
    for (int p = tw; p < 4; p += WPT) {
      // E = K W0 - V on 16 tokens x 16 columns (C layout: row = token 16p + 4g + j).
      f32x4 e;
      for (int j = 0; j < 4; ++j) e[j] = -(float)sV[(16 * p + 4 * g + j) * P + 16 * n + r];
      if constexpr (D >= 32) {
        for (int ks = 0; ks < KS; ++ks) e = mma32(ld8(&sK[(16 * p + r) * P + 32 * ks + 8 * g]), wb[ks], e);
      } else {
        e = mma16(ld4(&sK[(16 * p + r) * P + 4 * g]), wb4, e);
      }
      // G[:, n] += K^T E: E's C layout is already the B operand (k = token 4g + j).
      const bf16x4 eb = to_bf16x4(e);
      for (int m = 0; m < NT; ++m)
        G[m] = mma16(ld4_col(&sK[(16 * p + 4 * g) * P + 16 * m + r], P), eb, G[m]);
    }
  }
  // Sum the waves that share a column tile, in a fixed order.
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j) sG[(w * D + 16 * m + 4 * g + j) * 16 + r] = G[m][j];
  __syncthreads();
  float* out = partial + ((long long)bh * S + s) * D * D;
  for (int e = threadIdx.x; e < D * D; e += kThreads) {
    const int i = e / D, c = e % D, nn = c / 16, rr = c % 16;
    float acc = 0.f;
    for (int t = 0; t < WPT; ++t) acc += sG[((t * NT + nn) * D + i) * 16 + rr];
    out[e] = acc;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void fb_readout_bf16(const bf16* __restrict__ q,
                                                            const float* __restrict__ wstar, int H,
                                                            int N, int tps, bf16* __restrict__ o) {
  constexpr int NT = D / 16;
  constexpr int KS = D >= 32 ? D / 32 : 1;
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const float* W = wstar + (long long)bh * D * D;
  const long long ts = (long long)H * D;

  // O^T = W*^T Q^T: A = W*^T (lane: row c = 16n + r, k = feature), B = Q^T (lane: token column).
  bf16x8 wa[NT][KS];
  bf16x4 wa4[NT];
  for (int n = 0; n < NT; ++n) {
    if constexpr (D >= 32) {
      for (int ks = 0; ks < KS; ++ks)
        for (int i = 0; i < 8; ++i) wa[n][ks][i] = (bf16)W[(32 * ks + 8 * g + i) * D + 16 * n + r];
    } else {
      for (int i = 0; i < 4; ++i) wa4[n][i] = (bf16)W[(4 * g + i) * D + 16 * n + r];
    }
  }
  for (int t0 = n0 + 16 * w; t0 < n1; t0 += 64) {
    const int t = t0 + r;
    const bool ok = t < n1;
    const bf16* qrow = q + ((long long)b * N + (ok ? t : t0)) * ts + (long long)h * D;
    bf16* orow = o + ((long long)b * N + (ok ? t : t0)) * ts + (long long)h * D;
    if constexpr (D >= 32) {
      bf16x8 qb[KS];
      for (int ks = 0; ks < KS; ++ks) qb[ks] = ld8(qrow + 32 * ks + 8 * g);
      for (int n = 0; n < NT; ++n) {
        f32x4 acc = zero4();
        for (int ks = 0; ks < KS; ++ks) acc = mma32(wa[n][ks], qb[ks], acc);
        if (ok) *reinterpret_cast<bf16x4*>(orow + 16 * n + 4 * g) = to_bf16x4(acc);
      }
    } else {
      const bf16x4 qb = ld4(qrow + 4 * g);
      f32x4 acc = mma16(wa4[0], qb, zero4());
      if (ok) *reinterpret_cast<bf16x4*>(orow + 4 * g) = to_bf16x4(acc);
    }
  }
}

// ---------------------------------------------------------------- fp32 I/O, plain FMA
template <int D>
__global__ __launch_bounds__(kThreads) void fb_partial_f32(const float* __restrict__ k,
                                                           const float* __restrict__ v,
                                                           const float* __restrict__ w0,
                                                           long long w0_bstride, int H, int N,
                                                           int tps, int S,
                                                           float* __restrict__ partial) {
  __shared__ float sK[kTileF][D + 1], sE[kTileF][D + 1], sW[D][D + 1];
  constexpr int PER = (D * D + kThreads - 1) / kThreads;
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const long long ts = (long long)H * D;
  const float* W0 = w0 + b * w0_bstride + (long long)h * D * D;
  for (int e = threadIdx.x; e < D * D; e += kThreads) sW[e / D][e % D] = W0[e];
  float G[PER];
  for (int u = 0; u < PER; ++u) G[u] = 0.f;
  for (int t0 = n0; t0 < n1; t0 += kTileF) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTileF * D; e += kThreads) {
      const int t = e / D, c = e % D;
      const bool ok = t0 + t < n1;
      const long long off = ((long long)b * N + t0 + t) * ts + (long long)h * D + c;
      sK[t][c] = ok ? k[off] : 0.f;
      sE[t][c] = ok ? v[off] : 0.f;
    }
    __syncthreads();
    // E = K W0 - V, in place over the V tile (each thread touches only its own elements).
    for (int e = threadIdx.x; e < kTileF * D; e += kThreads) {
      const int t = e / D, c = e % D;
      float acc = -sE[t][c];
      for (int i = 0; i < D; ++i) acc = fmaf(sK[t][i], sW[i][c], acc);
      sE[t][c] = acc;
    }
    __syncthreads();
    for (int u = 0; u < PER; ++u) {
      const int e = threadIdx.x + kThreads * u;
      if (e < D * D) {
        const int i = e / D, c = e % D;
        float acc = G[u];
        for (int t = 0; t < kTileF; ++t) acc = fmaf(sK[t][i], sE[t][c], acc);
        G[u] = acc;
      }
    }
  }
  float* out = partial + ((long long)bh * S + s) * D * D;
  for (int u = 0; u < PER; ++u) {
    const int e = threadIdx.x + kThreads * u;
    if (e < D * D) out[e] = G[u];
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void fb_readout_f32(const float* __restrict__ q,
                                                           const float* __restrict__ wstar, int H,
                                                           int N, int tps, float* __restrict__ o) {
  __shared__ float sQ[kTileF][D + 1], sW[D][D + 1];
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const long long ts = (long long)H * D;
  const float* W = wstar + (long long)bh * D * D;
  for (int e = threadIdx.x; e < D * D; e += kThreads) sW[e / D][e % D] = W[e];
  for (int t0 = n0; t0 < n1; t0 += kTileF) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTileF * D; e += kThreads) {
      const int t = e / D, c = e % D;
      sQ[t][c] = (t0 + t < n1) ? q[((long long)b * N + t0 + t) * ts + (long long)h * D + c] : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kTileF * D; e += kThreads) {
      const int t = e / D, c = e % D;
      if (t0 + t >= n1) continue;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc = fmaf(sQ[t][i], sW[i][c], acc);
      o[((long long)b * N + t0 + t) * ts + (long long)h * D + c] = acc;
    }
  }
}

// ---------------------------------------------------------------- shared reduction
__global__ __launch_bounds__(kThreads) void fb_reduce(const float* __restrict__ partial, int S,
                                                      const float* __restrict__ w0,
                                                      long long w0_bstride, int H, int D,
                                                      float scale, float* __restrict__ wstar,
                                                      float* __restrict__ w_out) {
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const long long dd = (long long)D * D;
  const float* W0 = w0 + b * w0_bstride + h * dd;
  const float* pp = partial + bh * S * dd;
  for (int e = threadIdx.x; e < D * D; e += kThreads) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc += pp[s * dd + e];
    const float wv = W0[e] - scale * acc;
    wstar[bh * dd + e] = wv;
    if (w_out) w_out[bh * dd + e] = wv;
  }
}

template <int D>
hipError_t fb_launch_d(bool bf16_io, int B, int H, int N, float eta, const void* q, const void* k,
                       const void* v, const float* w0, long long w0s, void* o, float* w_out,
                       void* ws, hipStream_t st) {
  const FbPlan pl = fb_plan(B, H, N, D);
  const int BH = B * H;
  float* partial = static_cast<float*>(ws);
  float* wstar = partial + (size_t)BH * pl.splits * D * D;
  const dim3 grid(pl.splits, BH);
  if (bf16_io) {
    hipLaunchKernelGGL(fb_partial_bf16<D>, grid, dim3(kThreads), 0, st, (const bf16*)k,
                       (const bf16*)v, w0, w0s, H, N, pl.tokens_per_split, pl.splits, partial);
  } else {
    hipLaunchKernelGGL(fb_partial_f32<D>, grid, dim3(kThreads), 0, st, (const float*)k,
                       (const float*)v, w0, w0s, H, N, pl.tokens_per_split, pl.splits, partial);
  }
  hipLaunchKernelGGL(fb_reduce, dim3(BH), dim3(kThreads), 0, st, partial, pl.splits, w0, w0s, H,
                     D, eta / (float)N, wstar, w_out);
  if (bf16_io) {
    hipLaunchKernelGGL(fb_readout_bf16<D>, grid, dim3(kThreads), 0, st, (const bf16*)q, wstar, H,
                       N, pl.tokens_per_split, (bf16*)o);
  } else {
    hipLaunchKernelGGL(fb_readout_f32<D>, grid, dim3(kThreads), 0, st, (const float*)q, wstar, H,
                       N, pl.tokens_per_split, (float*)o);
  }
  return hipGetLastError();
}

}  // namespace

FbPlan fb_plan(int B, int H, int N, int D) {
  (void)D;
  const int BH = B * H;
  const int tiles = (N + kTile - 1) / kTile;
  // Aim for about 1024 workgroups (4 per CU on 256 CUs), never below one 64-token tile each.
  int splits = (1024 + BH - 1) / BH;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int tiles_per = (tiles + splits - 1) / splits;
  FbPlan p;
  p.tokens_per_split = tiles_per * kTile;
  p.splits = (N + p.tokens_per_split - 1) / p.tokens_per_split;
  return p;
}

size_t fb_workspace_bytes(int B, int H, int N, int D) {
  const FbPlan p = fb_plan(B, H, N, D);
  const size_t dd = (size_t)D * D * sizeof(float);
  return (size_t)B * H * p.splits * dd + (size_t)B * H * dd;
}

hipError_t fb_launch(bool bf16_io, int B, int H, int N, int D, float eta, const void* q,
                     const void* k, const void* v, const float* w0, long long w0s, void* o,
                     float* w_out, void* ws, hipStream_t st) {
  switch (D) {
    case 16: return fb_launch_d<16>(bf16_io, B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 32: return fb_launch_d<32>(bf16_io, B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 64: return fb_launch_d<64>(bf16_io, B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
