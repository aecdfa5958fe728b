// Full-batch single-step TTT-Linear forward (ViT^3 review on techloop.online, design-space study:
// single epoch, full batch, inner learning rate 1.0; "core idea": train on (K, V), read out Q):
//   W* = W0 - (eta/N) K^T (K W0 - V),  O = Q W*   for every (batch, head).
//
// bf16 I/O: two launches. Heads whose D-vectors are adjacent in a token row are grouped up to
// 128 bytes per row (2 heads of 32, 4 of 16, 1 of 64), so every staged row is a full, contiguous
// cache line. Work items are (group, token split), one per workgroup; a group's items share an
// XCD.
//   fb_partial_bf16: stream K, V tiles (double-buffered LDS, up to four tiles in flight in
//                    registers) and accumulate the split's K_s^T K_s and K_s^T V_s with MFMA
//                    (operands by LDS transpose reads); since K^T (K W0 - V) = (K^T K) W0 - K^T V,
//                    these two sums carry the gradient;
//   fb_readout_bf16: form W* = W0 - (eta/N) (sum_s K_s^T K_s W0 - sum_s K_s^T V_s) from the
//                    group's split records (fixed order: deterministic) into LDS, then stream Q
//                    through wave-private LDS tiles, one wave per 16-token block, and write
//                    O = Q W*.
// HBM traffic is the algorithmic Q, K, V read plus the O write; the split records are two d x d
// fp32 matrices per split and stay in L2 / Infinity Cache.
//
// fp32 I/O: three plain-FMA launches (partial gradients, fixed-order reduction, read-out).
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kTile = 64;      // tokens per staged tile (bf16 path)
constexpr int kThreads = 256;  // 4 waves per workgroup
// Register sets per thread for staged tiles (bf16 path): a split's first tile_sets(D) tiles are
// all in flight from the start, and tile it + tile_sets(D) loads as soon as tile it has moved to
// LDS. The plan keeps splits within that many tiles where the workgroup count allows, so that a
// workgroup waits for HBM about once. (Two for D = 64, whose MFMA operands need the registers.)
constexpr int tile_sets(int D) { return D >= 64 ? 2 : 4; }
constexpr int kTileF = 32;     // tokens per staged tile (fp32 path)

// ---------------------------------------------------------------- bf16 I/O, MFMA
// Shared geometry of the bf16 kernels: a head group of HG heads of D features (COLS <= 64
// channels, one 128-byte row per token), (head, 16-column) pairs spread over the 4 waves.
template <int D, int HG>
struct Geo {
  static constexpr int NT = D / 16;
  static constexpr int COLS = HG * D;
  static constexpr int PAIRS = COLS / 16;
  static constexpr int WPP = 4 / PAIRS;  // waves per pair; they split the 16-token sub-tiles
  static constexpr int P = COLS + 8;     // LDS row pitch (elements)
  static constexpr int CPR = COLS / 8;   // 16-byte pieces per row
  static constexpr int PIECES = kTile * CPR;
  static constexpr int PER = (PIECES + kThreads - 1) / kThreads;
  static constexpr int KS = D >= 32 ? D / 32 : 1;
};

// Register <-> LDS staging of one 64-token tile of a head group (rows past n1 read as zeros).
template <class G>
struct Stager {
  const bf16* src;
  long long base, ts;
  int n1;
  __device__ __forceinline__ void load(uint4* regs, int t0) const {
    for (int i = 0; i < G::PER; ++i) {
      const int c = threadIdx.x + i * kThreads;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (G::PIECES % kThreads == 0 || c < G::PIECES) {
        const int row = c / G::CPR, col = (c % G::CPR) * 8;
        if (t0 + row < n1) val = ld16(src + base + (long long)(t0 + row) * ts + col);
      }
      regs[i] = val;
    }
  }
  __device__ __forceinline__ static void store(bf16* dst, const uint4* regs) {
    for (int i = 0; i < G::PER; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (G::PIECES % kThreads == 0 || c < G::PIECES) st16(dst + (c / G::CPR) * G::P + (c % G::CPR) * 8, regs[i]);
    }
  }
};

// W* for the read-out is stored in bf16 as the read-out's MFMA A operands (W*^T tiles), so that
// a lane loads each operand with one access. Operand (head hl, column tile n, k step ks), lane
// l = r + 16g, element i holds W*[kb * ks + e * g + i][16n + r] with e = 8 (D >= 32, k steps of
// 32) or e = 4 (D = 16, one k step of 16), kb = 4e.
template <int D>
constexpr int kOpElems = D >= 32 ? 8 : 4;

template <int D>
__device__ __forceinline__ int wstar_operand_offset(int hl, int row, int col) {
  constexpr int NT = D / 16, E = kOpElems<D>, KS = D / (4 * E);
  return (((hl * NT + col / 16) * KS + row / (4 * E)) * 64 + col % 16 + 16 * ((row % (4 * E)) / E)) * E +
         row % E;
}

// Row block m of W* = W0 - scale ((K^T K) W0 - K^T V) for head hl of a group, from the summed
// accumulator tiles acc[0 .. NT) = (c, m) of K^T K and acc[NT .. 2NT) = (m, n) of K^T V. By
// symmetry, tile (c, m) of K^T K in accumulator layout is the A operand of rows 16m.. and k block
// c. (The 16x16x16 products keep their own accumulators: they must not take a 16x16x32 result as
// their accumulator input.) Writes the read-out operands and, if w_out is set, W* in fp32.
template <int D>
__device__ __forceinline__ void wstar_rows(const f32x4* acc, int hl, int m, const float* W0,
                                           float scale, bf16* wop_grp, float* w_out, int r, int g) {
  constexpr int NT = D / 16;
  bf16x4 ka[NT];
  for (int c = 0; c < NT; ++c) ka[c] = to_bf16x4(acc[c]);
  for (int n = 0; n < NT; ++n) {
    f32x4 gw = zero4();
    for (int c = 0; c < NT; ++c) {
      bf16x4 wb;  // B operand: W0[16c + 4g + i][16n + r]
      for (int i = 0; i < 4; ++i) wb[i] = (bf16)W0[(16 * c + 4 * g + i) * D + 16 * n + r];
      gw = mma16(ka[c], wb, gw);
    }
    for (int j = 0; j < 4; ++j) {  // W*[16m + 4g + j][16n + r]
      const int row = 16 * m + 4 * g + j, col = 16 * n + r;
      const float wv = W0[row * D + col] - scale * (gw[j] - acc[NT + n][j]);
      wop_grp[wstar_operand_offset<D>(hl, row, col)] = (bf16)wv;
      if (w_out) w_out[row * D + col] = wv;
    }
  }
}

// Blocks of one launch go to the 8 XCDs in turn (block i to XCD i mod 8); the work items of a
// group are given to blocks of one XCD, so that its L2 serves the group's split records to all
// of them.
__device__ __forceinline__ int xcd_item(int i, int items) {
  const int q = items / 8, rem = items % 8, x = i % 8;
  return x * q + min(x, rem) + i / 8;
}

// 1. Gradient sums of one token split of one head group: the split's gradient at W0 is
// K_s^T (K_s W0 - V_s) = (K_s^T K_s) W0 - K_s^T V_s, so the kernel accumulates K_s^T K_s and
// K_s^T V_s over the split's tokens, every MFMA operand read from LDS by transpose reads
// (contraction over tokens); W0 is applied once per group by the reduction. Wave w owns task
// (head, 16-row block m); waves sharing a task split the 32-token steps. K^T K is symmetric, so
// the wave accumulates its column block m, tiles (c, m) in accumulator layout, which are the A
// operands of row block m, k block c, in the product with W0.
template <int D, int HG>
__global__ __launch_bounds__(kThreads, 4) void fb_partial_bf16(
    const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ w0,
    long long w0_bstride, int H, int N, int S, int tps, float* __restrict__ partial) {
  using G = Geo<D, HG>;
  constexpr int NT = G::NT;
  constexpr long long DD = (long long)D * D;
  constexpr int TASKS = HG * NT;  // (head, 16-row block) of G_s
  constexpr int WPT = 4 / TASKS;  // waves per task
  __shared__ __align__(16) bf16 sK[2][kTile * G::P];
  __shared__ __align__(16) bf16 sV[2][kTile * G::P];
  static_assert(TASKS * WPT == 4, "tasks divide the waves");
  static_assert(sizeof(float) * (4 - TASKS) * 2 * NT * 256 <= sizeof(bf16) * 2 * kTile * G::P,
                "sums of the waves sharing a task fit in sK");
  float* sG = reinterpret_cast<float*>(&sK[0][0]);

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int grp = item / S, s = item % S;
  const int b = grp / (H / HG), h0 = (grp % (H / HG)) * HG;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const int ntiles = (n1 - n0 + kTile - 1) / kTile;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int task = w % TASKS, tw = w / TASKS;
  const int hl = task / NT, m = task % NT;  // head within the group, row block
  const long long ts = (long long)H * D;
  const long long base = (long long)b * N * ts + (long long)h0 * D;
  const Stager<G> stk{k, base, ts, n1}, stv{v, base, ts, n1};

  f32x4 kk[NT], kv[NT];  // tiles (c, m) of K^T K and (m, n) of K^T V
  for (int c = 0; c < NT; ++c) kk[c] = kv[c] = zero4();
  constexpr int SETS = tile_sets(D);
  struct Regs {
    uint4 k[G::PER], v[G::PER];
  } sets[SETS];
  auto load = [&](Regs& R, int it) {
    stk.load(R.k, n0 + it * kTile);
    stv.load(R.v, n0 + it * kTile);
  };
#pragma unroll
  for (int u = 0; u < SETS; ++u)
    if (u < ntiles) load(sets[u], u);
  auto step = [&](int it, Regs& R) {
    const int buf = it & 1;
    Stager<G>::store(sK[buf], R.k);
    Stager<G>::store(sV[buf], R.v);
    if (it + SETS < ntiles) load(R, it + SETS);
    __syncthreads();
    const bf16* tK = sK[buf] + hl * D;
    const bf16* tV = sV[buf] + hl * D;
    for (int ks = tw; ks < kTile / 32; ks += WPT) {
      // Operands over 32 tokens, k map {4g + j} u {16 + 4g + j}: lane (r, g) holds column r.
      const bf16* k0 = tK + 32 * ks * G::P;
      const bf16* v0 = tV + 32 * ks * G::P;
      // (Block m is read on its own: m varies by wave, and indexing registers with it would
      // become select chains.)
      const bf16x8 km = cat8(tile_tr(k0 + 16 * m, G::P, l), tile_tr(k0 + 16 * G::P + 16 * m, G::P, l));
      bf16x8 tk[NT], tv[NT];
      for (int c = 0; c < NT; ++c) {
        tk[c] = cat8(tile_tr(k0 + 16 * c, G::P, l), tile_tr(k0 + 16 * G::P + 16 * c, G::P, l));
        tv[c] = cat8(tile_tr(v0 + 16 * c, G::P, l), tile_tr(v0 + 16 * G::P + 16 * c, G::P, l));
      }
      for (int c = 0; c < NT; ++c) kk[c] = mma32(tk[c], km, kk[c]);
      for (int n = 0; n < NT; ++n) kv[n] = mma32(km, tv[n], kv[n]);
    }
  };
  for (int it = 0; it < ntiles; it += SETS) {
#pragma unroll
    for (int u = 0; u < SETS; ++u)
      if (it + u < ntiles) step(it + u, sets[u]);
  }
  // The split's partial record holds, per task (head, row block m), the accumulator tiles
  // (c, m) of K^T K then (m, n) of K^T V, lane by lane (16 bytes a lane, coalesced). Waves
  // sharing a task add theirs first through sK, in a fixed order.
  float* part = partial + ((long long)grp * S + s) * (2 * HG * D * D) + (long long)task * (2 * NT * 256);
  if constexpr (WPT > 1) {
    __syncthreads();  // tile buffers free
    if (tw > 0)
      for (int c = 0; c < NT; ++c) {
        *reinterpret_cast<f32x4*>(sG + (((w - TASKS) * 2 * NT + c) * 64 + l) * 4) = kk[c];
        *reinterpret_cast<f32x4*>(sG + (((w - TASKS) * 2 * NT + NT + c) * 64 + l) * 4) = kv[c];
      }
    __syncthreads();
    if (tw == 0)
      for (int t = 1; t < WPT; ++t) {
        const int wt = (t - 1) * TASKS + task;
        for (int c = 0; c < NT; ++c) {
          kk[c] += *reinterpret_cast<const f32x4*>(sG + ((wt * 2 * NT + c) * 64 + l) * 4);
          kv[c] += *reinterpret_cast<const f32x4*>(sG + ((wt * 2 * NT + NT + c) * 64 + l) * 4);
        }
      }
  }
  if (tw == 0)
    for (int c = 0; c < NT; ++c) {
      *reinterpret_cast<f32x4*>(part + (c * 64 + l) * 4) = kk[c];
      *reinterpret_cast<f32x4*>(part + ((NT + c) * 64 + l) * 4) = kv[c];
    }
}

// 2. O = Q W*, computed as O^T = W*^T Q^T (lane (r, g) gets 4 adjacent outputs of token r).
// Each workgroup first forms its group's W* = W0 - (eta/N) ((sum_s K_s^T K_s) W0 - sum_s K_s^T V_s)
// from the split records (wave (task, tw) sums the task's tiles of splits tw, tw + WPT, ...; the
// waves of a task add theirs in a fixed order, so every workgroup of a group gets the same W*),
// with its first Q blocks already in flight; the work items of a group share an XCD (xcd_item).
// W* goes to LDS as the read-out's MFMA operands (wstar_rows).
// Then each wave streams its own 16-token blocks of the split (blocks w, w + 4, ...), kReadSets
// of them in flight, through a wave-private LDS tile: full-row 16-byte pieces to and from HBM,
// operand-shaped pieces to and from the matrix cores. No workgroup barriers in that loop: a wave's
// LDS operations execute in order, and a wavefront-scope fence keeps the compiler from reordering
// them.
constexpr int kReadSets = 4;

template <int D, int HG>
__global__ __launch_bounds__(kThreads) void fb_readout_bf16(
    const bf16* __restrict__ q, const float* __restrict__ partial, const float* __restrict__ w0,
    long long w0_bstride, int H, int N, int S, int tps, float scale, bf16* __restrict__ o,
    float* __restrict__ w_out) {
  using G = Geo<D, HG>;
  constexpr int NT = D / 16, E = kOpElems<D>, KS = D / (4 * E);
  constexpr long long DD = (long long)D * D;
  constexpr int TASKS = HG * NT, WPT = 4 / TASKS, T2 = 2 * NT;
  constexpr int BP = 16 * G::CPR;       // 16-byte pieces of a 16-token block
  constexpr int PPL = (BP + 63) / 64;   // pieces per lane
  constexpr int WPER = (HG * D * D + kThreads - 1) / kThreads;
  __shared__ __align__(16) bf16 sQ[4][16 * G::P];
  __shared__ __align__(16) bf16 sO[4][16 * G::P];
  __shared__ __align__(16) float sW0[HG * D * D];
  __shared__ __align__(16) bf16 sWop[HG * D * D];
  __shared__ f32x4 sSum[(4 - TASKS) > 0 ? (4 - TASKS) : 1][T2][64];
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int grp = item / S, s = item % S;
  const int b = grp / (H / HG), h0 = (grp % (H / HG)) * HG;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int task = w % TASKS, tw = w / TASKS, hl = task / NT, m = task % NT;
  const int blocks = (n1 - n0 + 15) / 16;
  const int mine = blocks > w ? (blocks - w + 3) / 4 : 0;
  const long long ts = (long long)H * D;
  const long long base = (long long)b * N * ts + (long long)h0 * D;
  bf16* myQ = sQ[w];
  bf16* myO = sO[w];

  struct Regs {
    uint4 x[PPL];
  } sets[kReadSets];
  auto valid = [&](int c) { return BP % 64 == 0 || c < BP; };
  auto load = [&](Regs& R, int i) {
    const int t0 = n0 + 16 * (w + 4 * i);
    for (int u = 0; u < PPL; ++u) {
      const int c = l + 64 * u, row = c / G::CPR;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (valid(c) && t0 + row < n1) v = ld16(q + base + (t0 + row) * ts + (c % G::CPR) * 8);
      R.x[u] = v;
    }
  };
#pragma unroll
  for (int u = 0; u < kReadSets; ++u)
    if (u < mine) load(sets[u], u);

  // W* of the group, while those loads are in flight.
  {
    const float* W0g = w0 + b * w0_bstride + (long long)h0 * DD;  // the group's heads, contiguous
    float w0v[WPER];
    for (int i = 0; i < WPER; ++i) {
      const int e = threadIdx.x + i * kThreads;
      w0v[i] = (HG * D * D) % kThreads == 0 || e < HG * D * D ? W0g[e] : 0.f;
    }
    const float* pt = partial + (long long)grp * S * (2 * HG * DD) + (long long)task * (T2 * 256) + l * 4;
    f32x4 acc[T2];
    for (int t = 0; t < T2; ++t) acc[t] = zero4();
    constexpr int UB = T2 >= 8 ? 2 : 4;  // splits in flight (16 tiles of loads)
    for (int s0 = tw; s0 < S; s0 += UB * WPT) {
      f32x4 x[UB][T2];
      for (int u = 0; u < UB; ++u) {
        const int sp = s0 + u * WPT;
        for (int t = 0; t < T2; ++t)
          x[u][t] = sp < S ? *reinterpret_cast<const f32x4*>(pt + (long long)sp * (2 * HG * DD) + t * 256) : zero4();
      }
      for (int u = 0; u < UB; ++u)
        for (int t = 0; t < T2; ++t) acc[t] += x[u][t];
    }
    for (int i = 0; i < WPER; ++i) {
      const int e = threadIdx.x + i * kThreads;
      if ((HG * D * D) % kThreads == 0 || e < HG * D * D) sW0[e] = w0v[i];
    }
    if constexpr (WPT > 1) {
      if (tw > 0)
        for (int t = 0; t < T2; ++t) sSum[w - TASKS][t][l] = acc[t];
    }
    __syncthreads();
    if (tw == 0) {
      if constexpr (WPT > 1)
        for (int u = 1; u < WPT; ++u)
          for (int t = 0; t < T2; ++t) acc[t] += sSum[(u - 1) * TASKS + task][t][l];
      wstar_rows<D>(acc, hl, m, sW0 + hl * DD, scale, sWop,
                    (w_out && s == 0) ? w_out + ((long long)b * H + h0 + hl) * DD : nullptr, r, g);
    }
    __syncthreads();
  }
  using Op = typename std::conditional<(D >= 32), bf16x8, bf16x4>::type;
  Op wa[HG][NT][KS];  // A operands W*^T
  for (int hl2 = 0; hl2 < HG; ++hl2)
    for (int n = 0; n < NT; ++n)
      for (int ks = 0; ks < KS; ++ks)
        wa[hl2][n][ks] = *reinterpret_cast<const Op*>(sWop + (((hl2 * NT + n) * KS + ks) * 64 + l) * E);

  auto step = [&](int i, Regs& R) {
    const int t0 = n0 + 16 * (w + 4 * i);
    for (int u = 0; u < PPL; ++u) {
      const int c = l + 64 * u;
      if (valid(c)) st16(myQ + (c / G::CPR) * G::P + (c % G::CPR) * 8, R.x[u]);
    }
    if (i + kReadSets < mine) load(R, i + kReadSets);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (int hl = 0; hl < HG; ++hl)
      for (int n = 0; n < NT; ++n) {
        f32x4 acc = zero4();
        for (int ks = 0; ks < KS; ++ks) {
          const Op qb = *reinterpret_cast<const Op*>(myQ + r * G::P + hl * D + 4 * E * ks + E * g);
          if constexpr (D >= 32) acc = mma32(wa[hl][n][ks], qb, acc);
          else acc = mma16(wa[hl][n][ks], qb, acc);
        }
        *reinterpret_cast<bf16x4*>(myO + r * G::P + hl * D + 16 * n + 4 * g) = to_bf16x4(acc);
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (int u = 0; u < PPL; ++u) {
      const int c = l + 64 * u, row = c / G::CPR;
      if (valid(c) && t0 + row < n1)
        st16(o + base + (t0 + row) * ts + (c % G::CPR) * 8, ld16(myO + row * G::P + (c % G::CPR) * 8));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  };
  for (int i = 0; i < mine; i += kReadSets) {
#pragma unroll
    for (int u = 0; u < kReadSets; ++u)
      if (i + u < mine) step(i + u, sets[u]);
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

// Heads per group: the largest power of two dividing H whose D-vectors fit in one 128-byte row
// (1, 2 or 4: the group's (head, 16-column) pairs must divide the 4 waves).
int head_group(int H, int D) {
  int hg = 64 / D;
  while (hg > 1 && H % hg != 0) hg /= 2;
  return hg;
}

FbPlan plan_splits(int groups, int N, int sets) {
  const int tiles = (N + kTile - 1) / kTile;
  // Aim for about 512 workgroups (two per CU: the streaming rate of 256 CUs), never below one
  // 64-token tile each; more splits (up to 4096 workgroups) where that keeps every split within
  // 2 * sets tiles (the in-flight register sets, refilled once). At most 16 splits per group:
  // every read-out workgroup sums all of its group's split records, so that work grows with the
  // split count (16 groups of 16384 tokens: 36 us with 32 splits, 29 us with 16, 31 with 12, 33
  // with 20). With 256 groups or more, the groups alone fill the CUs: only as many splits as the
  // register sets need (64 x 196 tokens, 6 heads of 64: 20.2 -> 17.6 us with 1 split instead of 2).
  int splits = (512 + groups - 1) / groups;
  const int need = (tiles + 2 * sets - 1) / (2 * sets);
  if (splits < need && (long long)groups * need <= 4096) splits = need;
  if (groups >= 256) splits = need;
  if (splits > 16) splits = 16;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int tiles_per = (tiles + splits - 1) / splits;
  FbPlan p;
  p.tokens_per_split = tiles_per * kTile;
  p.splits = (N + p.tokens_per_split - 1) / p.tokens_per_split;
  return p;
}

template <int D, int HG>
hipError_t launch_bf16(int B, int H, int N, float eta, const void* q, const void* k, const void* v,
                       const float* w0, long long w0s, void* o, float* w_out, void* ws,
                       hipStream_t st) {
  const int groups = B * (H / HG);
  const FbPlan pl = plan_splits(groups, N, tile_sets(D));
  float* partial = static_cast<float*>(ws);
  const int items = groups * pl.splits;
  const float scale = eta / (float)N;
  hipLaunchKernelGGL((fb_partial_bf16<D, HG>), dim3(items), dim3(kThreads), 0, st, (const bf16*)k,
                     (const bf16*)v, w0, w0s, H, N, pl.splits, pl.tokens_per_split, partial);
  hipLaunchKernelGGL((fb_readout_bf16<D, HG>), dim3(items), dim3(kThreads), 0, st, (const bf16*)q,
                     partial, w0, w0s, H, N, pl.splits, pl.tokens_per_split, scale, (bf16*)o, w_out);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(int B, int H, int N, float eta, const void* q, const void* k, const void* v,
                      const float* w0, long long w0s, void* o, float* w_out, void* ws,
                      hipStream_t st) {
  const int BH = B * H;
  const FbPlan pl = plan_splits(BH, N, 1);
  float* partial = static_cast<float*>(ws);
  float* wstar = partial + (size_t)BH * pl.splits * D * D;
  const dim3 grid(pl.splits, BH);
  hipLaunchKernelGGL(fb_partial_f32<D>, grid, dim3(kThreads), 0, st, (const float*)k,
                     (const float*)v, w0, w0s, H, N, pl.tokens_per_split, pl.splits, partial);
  hipLaunchKernelGGL(fb_reduce, dim3(BH), dim3(kThreads), 0, st, partial, pl.splits, w0, w0s, H,
                     D, eta / (float)N, wstar, w_out);
  hipLaunchKernelGGL(fb_readout_f32<D>, grid, dim3(kThreads), 0, st, (const float*)q, wstar, H,
                     N, pl.tokens_per_split, (float*)o);
  return hipGetLastError();
}

}  // namespace

FbPlan fb_plan(int B, int H, int N, int D) {
  return plan_splits(B * (H / head_group(H, D)), N, tile_sets(D));
}

size_t fb_workspace_bytes(bool bf16_io, int B, int H, int N, int D) {
  const size_t dd = (size_t)D * D * sizeof(float);
  if (!bf16_io) {
    const FbPlan p = plan_splits(B * H, N, 1);
    return (size_t)B * H * p.splits * dd + (size_t)B * H * dd;
  }
  const int hg = head_group(H, D);
  const int groups = B * (H / hg);
  const FbPlan p = plan_splits(groups, N, tile_sets(D));
  return (size_t)groups * p.splits * 2 * hg * dd;
}

hipError_t fb_launch(bool bf16_io, int B, int H, int N, int D, float eta, const void* q,
                     const void* k, const void* v, const float* w0, long long w0s, void* o,
                     float* w_out, void* ws, hipStream_t st) {
  if (!bf16_io) {
    switch (D) {
      case 16: return launch_f32<16>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
      case 32: return launch_f32<32>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
      case 64: return launch_f32<64>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
      default: return hipErrorInvalidValue;
    }
  }
  const int hg = head_group(H, D);
  switch (D * 8 + hg) {
    case 64 * 8 + 1: return launch_bf16<64, 1>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 32 * 8 + 2: return launch_bf16<32, 2>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 32 * 8 + 1: return launch_bf16<32, 1>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 16 * 8 + 4: return launch_bf16<16, 4>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 16 * 8 + 2: return launch_bf16<16, 2>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 16 * 8 + 1: return launch_bf16<16, 1>(B, H, N, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
