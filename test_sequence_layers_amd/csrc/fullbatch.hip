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
// fp32 matrices per split and stay in L2 / Infinity Cache. When the plan gives each group one
// split (many groups of few tokens, e.g. 64 images of 196 tokens), fb_fused_bf16 does both in one
// launch, the sums kept in registers: no records, one launch fewer.
//
// fp32 I/O: three plain-FMA launches (the splits' K^T K and K^T V, a fixed-order reduction that
// also runs the epochs, read-out).
//
// Several epochs (ViT^3 review, design-space study: epochs per inner update) reuse the same sums:
// epoch e takes W_{e+1} = W_e - (eta/N) ((K^T K) W_e - K^T V), a few small products per (b, h)
// in the read-out kernel, with no further pass over K and V.
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
// STREAM: loads with the nontemporal hint (the forward's split-sum launch, which reads K and V once:
// measured faster with the inputs in HBM and in the caches alike; the one-launch kernel, whose Q
// loads are in flight beside them, and the backward's split sums were slower with it when the
// inputs were cached).
template <class G, bool STREAM = false>
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
        if (t0 + row < n1) {
          const bf16* p = src + base + (long long)(t0 + row) * ts + col;
          val = STREAM ? ld16_stream(p) : ld16(p);
        }
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

// W* for the read-out is stored as the read-out's MFMA A operands (W*^T tiles), so that a lane
// loads each operand with one access, in two bf16 parts: hi = bf16(W*) and lo = bf16(W* - hi). The
// read-out multiplies by both (same-shape products into one fp32 accumulator), so W* enters with
// about 16 significant bits instead of bf16's 8: the read-out is bound by HBM, not by the matrix
// cores. Operand (head hl, column tile n, k step ks), lane l = r + 16g, element i holds
// W*[kb * ks + e * g + i][16n + r] with e = 8 (D >= 32, k steps of 32) or e = 4 (D = 16, one k
// step of 16), kb = 4e; the lo part follows the hi part at an offset of HG d^2 elements.
template <int D>
constexpr int kOpElems = D >= 32 ? 8 : 4;

template <int D>
__device__ __forceinline__ int wstar_operand_offset(int hl, int row, int col) {
  constexpr int NT = D / 16, E = kOpElems<D>, KS = D / (4 * E);
  return (((hl * NT + col / 16) * KS + row / (4 * E)) * 64 + col % 16 + 16 * ((row % (4 * E)) / E)) * E +
         row % E;
}

// A head's state W in LDS for the product (K^T K) W: its bf16 transpose, rows of pitch D + 8
// (WbT[col][row]), so that each MFMA B operand of W (lane (r, g): W[16c + 4g + i][16n + r], i < 4)
// is one 8-byte read. The fp32 W itself stays in the registers of the waves that own its rows.
template <int D>
constexpr int kWtPitch = D + 8;

// Row block m of W (tiles (m, n), accumulator layout: lane (r, g) holds W[16m + 4g + j][16n + r]):
// loaded from HBM (w: the head's d x d matrix) and stored to LDS as part of W's bf16 transpose.
template <int D>
__device__ __forceinline__ void load_rows(const float* __restrict__ w, int m, int r, int g, f32x4 (&wr)[D / 16]) {
  for (int n = 0; n < D / 16; ++n)
    for (int j = 0; j < 4; ++j) wr[n][j] = w[(16 * m + 4 * g + j) * D + 16 * n + r];
}
template <int D>
__device__ __forceinline__ void put_rows_t(const f32x4 (&wr)[D / 16], int m, int r, int g, bf16* wbt) {
  for (int n = 0; n < D / 16; ++n)
    *reinterpret_cast<bf16x4*>(wbt + (16 * n + r) * kWtPitch<D> + 16 * m + 4 * g) = to_bf16x4(wr[n]);
}

// One epoch for row block m of head hl of a group: W1 = W - scale ((K^T K) W - K^T V), from the
// summed accumulator tiles acc[0 .. NT) = (c, m) of K^T K and acc[NT .. 2NT) = (m, n) of K^T V,
// the row block wr of W (replaced by W1's) and W's bf16 transpose wbt (all rows). By symmetry,
// tile (c, m) of K^T K in accumulator layout is the A operand of rows 16m.. and k block c. (The
// 16x16x16 products keep their own accumulators: they must not take a 16x16x32 result as their
// accumulator input.) Writes, where set: the read-out operands (8-byte pieces: a lane's four
// rows of a column are adjacent there), W1 in fp32 to w_out, W1's bf16 transpose to nbt (the next
// epoch's wbt).
template <int D>
__device__ __forceinline__ void wstar_rows(const f32x4* acc, int hl, int m, f32x4 (&wr)[D / 16],
                                           const bf16* wbt, float scale, bf16* wop_grp, int lo_offset,
                                           float* w_out, bf16* nbt, int r, int g) {
  constexpr int NT = D / 16;
  bf16x4 ka[NT];
  for (int c = 0; c < NT; ++c) ka[c] = to_bf16x4(acc[c]);
  for (int n = 0; n < NT; ++n) {
    f32x4 gw = zero4();
    for (int c = 0; c < NT; ++c) gw = mma16(ka[c], ld4(wbt + (16 * n + r) * kWtPitch<D> + 16 * c + 4 * g), gw);
    f32x4 wv;  // W1[16m + 4g + j][16n + r]
    for (int j = 0; j < 4; ++j) wv[j] = wr[n][j] - scale * (gw[j] - acc[NT + n][j]);
    wr[n] = wv;
    if (wop_grp) {
      const bf16x4 hi = to_bf16x4(wv);
      f32x4 rest;
      for (int j = 0; j < 4; ++j) rest[j] = wv[j] - (float)hi[j];
      const int off = wstar_operand_offset<D>(hl, 16 * m + 4 * g, 16 * n + r);
      *reinterpret_cast<bf16x4*>(wop_grp + off) = hi;
      *reinterpret_cast<bf16x4*>(wop_grp + lo_offset + off) = to_bf16x4(rest);
    }
    if (w_out)
      for (int j = 0; j < 4; ++j) w_out[(16 * m + 4 * g + j) * D + 16 * n + r] = wv[j];
  }
  if (nbt) put_rows_t<D>(wr, m, r, g, nbt);
}

// Blocks of one launch go to the 8 XCDs in turn (block i to XCD i mod 8); the work items of a
// group are given to blocks of one XCD, so that its L2 serves the group's split records to all
// of them.
__device__ __forceinline__ int xcd_item(int i, int items) {
  const int q = items / 8, rem = items % 8, x = i % 8;
  return x * q + min(x, rem) + i / 8;
}

// Gradient sums over tokens [n0, n1) of one head group: the gradient at W0 of those tokens is
// K_s^T (K_s W0 - V_s) = (K_s^T K_s) W0 - K_s^T V_s, so K_s^T K_s and K_s^T V_s are accumulated,
// every MFMA operand read from LDS by transpose reads (contraction over tokens); W0 is applied
// once per group, when W* is formed. Wave w owns task (head hl, 16-row block m); waves sharing a
// task split the 32-token steps. K^T K is symmetric, so the wave accumulates its column block m,
// tiles (c, m) in accumulator layout, which are the A operands of row block m, k block c, in the
// product with W0. The tiles stream through the double-buffered sK, sV ([2][kTile * P] each).
template <int D, int HG, bool STREAM>
__device__ __forceinline__ void gram_sums(const bf16* __restrict__ k, const bf16* __restrict__ v,
                                          long long base, long long ts, int n0, int n1, bf16* sK,
                                          bf16* sV, f32x4 (&kk)[D / 16], f32x4 (&kv)[D / 16]) {
  using G = Geo<D, HG>;
  constexpr int NT = G::NT;
  constexpr int TASKS = HG * NT;  // (head, 16-row block) of G_s
  constexpr int WPT = 4 / TASKS;  // waves per task
  static_assert(TASKS * WPT == 4, "tasks divide the waves");
  const int ntiles = (n1 - n0 + kTile - 1) / kTile;
  const int w = wave_id(), l = lane_id();
  const int task = w % TASKS, tw = w / TASKS;
  const int hl = task / NT, m = task % NT;  // head within the group, row block
  const Stager<G, STREAM> stk{k, base, ts, n1}, stv{v, base, ts, n1};

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
    bf16* bK = sK + (it & 1) * (kTile * G::P);
    bf16* bV = sV + (it & 1) * (kTile * G::P);
    Stager<G, STREAM>::store(bK, R.k);
    Stager<G, STREAM>::store(bV, R.v);
    if (it + SETS < ntiles) load(R, it + SETS);
    __syncthreads();
    const bf16* tK = bK + hl * D;
    const bf16* tV = bV + hl * D;
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
}

// Waves sharing a task (when a group has fewer than four tasks) add their sums into those of the
// task's wave tw = 0, in a fixed order, through sG ((4 - TASKS) * 2 NT fp32 tiles of 64 lanes; it
// may alias the tile buffers of gram_sums: the first barrier frees them).
template <int D, int HG>
__device__ __forceinline__ void task_sum(float* sG, f32x4 (&kk)[D / 16], f32x4 (&kv)[D / 16]) {
  constexpr int NT = D / 16, TASKS = HG * NT, WPT = 4 / TASKS;
  if constexpr (WPT > 1) {
    const int w = wave_id(), l = lane_id(), task = w % TASKS, tw = w / TASKS;
    __syncthreads();
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
}

// 1. Gradient sums of one token split of one head group (gram_sums); the split's record holds,
// per task (head, row block m), the accumulator tiles (c, m) of K^T K then (m, n) of K^T V, lane
// by lane (16 bytes a lane, coalesced).
template <int D, int HG, bool STREAM>
__global__ __launch_bounds__(kThreads, 4) void fb_partial_bf16(
    const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ w0,
    long long w0_bstride, int H, int N, int S, int tps, float* __restrict__ partial) {
  using G = Geo<D, HG>;
  constexpr int NT = G::NT;
  constexpr int TASKS = HG * NT;
  __shared__ __align__(16) bf16 sK[2][kTile * G::P];
  __shared__ __align__(16) bf16 sV[2][kTile * G::P];
  static_assert(sizeof(float) * (4 - TASKS) * 2 * NT * 256 <= sizeof(bf16) * 2 * kTile * G::P,
                "sums of the waves sharing a task fit in sK");

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int grp = item / S, s = item % S;
  const int b = grp / (H / HG), h0 = (grp % (H / HG)) * HG;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const int w = wave_id(), l = lane_id();
  const int task = w % TASKS, tw = w / TASKS;
  const long long ts = (long long)H * D;
  const long long base = (long long)b * N * ts + (long long)h0 * D;

  f32x4 kk[NT], kv[NT];  // tiles (c, m) of K^T K and (m, n) of K^T V
  gram_sums<D, HG, STREAM>(k, v, base, ts, n0, n1, &sK[0][0], &sV[0][0], kk, kv);
  task_sum<D, HG>(reinterpret_cast<float*>(&sK[0][0]), kk, kv);
  float* part = partial + ((long long)grp * S + s) * (2 * HG * D * D) + (long long)task * (2 * NT * 256);
  if (tw == 0)
    for (int c = 0; c < NT; ++c) {
      *reinterpret_cast<f32x4*>(part + (c * 64 + l) * 4) = kk[c];
      *reinterpret_cast<f32x4*>(part + ((NT + c) * 64 + l) * 4) = kv[c];
    }
}

// W* of the group from the summed tiles acc of the waves tw = 0 (acc[0 .. NT): tiles (c, m) of
// K^T K, acc[NT .. 2NT): tiles (m, n) of K^T V) and their row blocks wr of W0 (load_rows). Epoch e
// takes W_{e+1} = W_e - scale ((K^T K) W_e - K^T V) with W_e's bf16 transpose in wbt[e & 1]
// (HG heads of d rows of pitch kWtPitch each; the first stored here); the last epoch writes the
// read-out operands sWop (hi, then lo) and, where w_out_grp is set, W* in fp32 (the group's heads,
// contiguous). Starts and ends with a barrier.
template <int D, int HG>
__device__ __forceinline__ void form_wstar(const f32x4* acc, f32x4 (&wr)[D / 16], bf16* wbt0, bf16* wbt1,
                                           bf16* sWop, float scale, int epochs, float* w_out_grp) {
  constexpr int NT = D / 16, TASKS = HG * NT;
  constexpr long long DD = (long long)D * D;
  constexpr int WT = D * kWtPitch<D>;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int task = w % TASKS, tw = w / TASKS, hl = task / NT, m = task % NT;
  if (tw == 0) put_rows_t<D>(wr, m, r, g, wbt0 + hl * WT);
  __syncthreads();
  for (int e = 0; e < epochs; ++e) {
    const bool last = e + 1 == epochs;
    bf16* cur = (e & 1) ? wbt1 : wbt0;
    bf16* nxt = (e & 1) ? wbt0 : wbt1;
    if (tw == 0)
      wstar_rows<D>(acc, hl, m, wr, cur + hl * WT, scale, last ? sWop : nullptr, HG * D * D,
                    (last && w_out_grp) ? w_out_grp + hl * DD : nullptr, last ? nullptr : nxt + hl * WT, r, g);
    __syncthreads();
  }
}

// A wave's 16-token blocks of Q within [n0, n1) (blocks w, w + 4, ...), loaded as full-row 16-byte
// pieces into register sets.
constexpr int kReadSets = 4;

template <int D, int HG>
struct QBlocks {
  using G = Geo<D, HG>;
  static constexpr int BP = 16 * G::CPR;      // 16-byte pieces of a 16-token block
  static constexpr int PPL = (BP + 63) / 64;  // pieces per lane
  struct Regs {
    uint4 x[PPL];
  };
  const bf16* q;
  long long base, ts;
  int n0, n1, w, l, mine;
  __device__ __forceinline__ QBlocks(const bf16* q_, long long base_, long long ts_, int n0_, int n1_)
      : q(q_), base(base_), ts(ts_), n0(n0_), n1(n1_), w(wave_id()), l(lane_id()) {
    const int blocks = (n1 - n0 + 15) / 16;
    mine = blocks > w ? (blocks - w + 3) / 4 : 0;
  }
  __device__ __forceinline__ static bool valid(int c) { return BP % 64 == 0 || c < BP; }
  __device__ __forceinline__ void load(Regs& R, int i) const {
    const int t0 = n0 + 16 * (w + 4 * i);
    for (int u = 0; u < PPL; ++u) {
      const int c = l + 64 * u, row = c / G::CPR;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (valid(c) && t0 + row < n1) x = ld16(q + base + (t0 + row) * ts + (c % G::CPR) * 8);
      R.x[u] = x;
    }
  }
  __device__ __forceinline__ void load_first(Regs (&sets)[kReadSets]) const {
#pragma unroll
    for (int u = 0; u < kReadSets; ++u)
      if (u < mine) load(sets[u], u);
  }
};

// O = Q W* for a wave's blocks, computed as O^T = W*^T Q^T (lane (r, g) gets 4 adjacent outputs of
// token r), from the read-out operands sWop (wstar_rows) and the blocks' register sets (the first
// kReadSets already loaded), kReadSets blocks in flight, through the wave-private LDS tiles myQ,
// myO: full-row 16-byte pieces to and from HBM, operand-shaped pieces to and from the matrix
// cores. No workgroup barriers: a wave's LDS operations execute in order, and a wavefront-scope
// fence keeps the compiler from reordering them.
template <int D, int HG>
__device__ __forceinline__ void readout_blocks(const QBlocks<D, HG>& qb, typename QBlocks<D, HG>::Regs (&sets)[kReadSets],
                                               const bf16* sWop, bf16* myQ, bf16* myO, bf16* __restrict__ o) {
  using G = Geo<D, HG>;
  using QB = QBlocks<D, HG>;
  constexpr int NT = D / 16, E = kOpElems<D>, KS = D / (4 * E);
  const int l = qb.l, r = l & 15, g = l >> 4;
  using Op = typename std::conditional<(D >= 32), bf16x8, bf16x4>::type;
  Op wa[HG][NT][KS], wl[HG][NT][KS];  // A operands W*^T, hi and lo parts
  for (int hl2 = 0; hl2 < HG; ++hl2)
    for (int n = 0; n < NT; ++n)
      for (int ks = 0; ks < KS; ++ks) {
        const int off = (((hl2 * NT + n) * KS + ks) * 64 + l) * E;
        wa[hl2][n][ks] = *reinterpret_cast<const Op*>(sWop + off);
        wl[hl2][n][ks] = *reinterpret_cast<const Op*>(sWop + HG * D * D + off);
      }

  auto step = [&](int i, typename QB::Regs& R) {
    const int t0 = qb.n0 + 16 * (qb.w + 4 * i);
    for (int u = 0; u < QB::PPL; ++u) {
      const int c = l + 64 * u;
      if (QB::valid(c)) st16(myQ + (c / G::CPR) * G::P + (c % G::CPR) * 8, R.x[u]);
    }
    if (i + kReadSets < qb.mine) qb.load(R, i + kReadSets);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (int hl = 0; hl < HG; ++hl)
      for (int n = 0; n < NT; ++n) {
        f32x4 acc = zero4();
        for (int ks = 0; ks < KS; ++ks) {
          const Op qv = *reinterpret_cast<const Op*>(myQ + r * G::P + hl * D + 4 * E * ks + E * g);
          if constexpr (D >= 32) acc = mma32(wl[hl][n][ks], qv, mma32(wa[hl][n][ks], qv, acc));
          else acc = mma16(wl[hl][n][ks], qv, mma16(wa[hl][n][ks], qv, acc));
        }
        *reinterpret_cast<bf16x4*>(myO + r * G::P + hl * D + 16 * n + 4 * g) = to_bf16x4(acc);
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (int u = 0; u < QB::PPL; ++u) {
      const int c = l + 64 * u, row = c / G::CPR;
      if (QB::valid(c) && t0 + row < qb.n1)
        st16_out(o + qb.base + (t0 + row) * qb.ts + (c % G::CPR) * 8, ld16(myO + row * G::P + (c % G::CPR) * 8));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  };
  for (int i = 0; i < qb.mine; i += kReadSets) {
#pragma unroll
    for (int u = 0; u < kReadSets; ++u)
      if (i + u < qb.mine) step(i + u, sets[u]);
  }
}

// 2. O = Q W* for one token split. Each workgroup first forms its group's
// W* = W0 - (eta/N) ((sum_s K_s^T K_s) W0 - sum_s K_s^T V_s) from the split records (wave
// (task, tw) sums the task's tiles of splits tw, tw + WPT, ...; the waves of a task add theirs in
// a fixed order, so every workgroup of a group gets the same W*), with its first Q blocks already
// in flight; the work items of a group share an XCD (xcd_item). Then readout_blocks.
template <int D, int HG>
__global__ __launch_bounds__(kThreads) void fb_readout_bf16(
    const bf16* __restrict__ q, const float* __restrict__ partial, const float* __restrict__ w0,
    long long w0_bstride, int H, int N, int S, int tps, float scale, int epochs,
    bf16* __restrict__ o, float* __restrict__ w_out) {
  using G = Geo<D, HG>;
  constexpr int NT = D / 16;
  constexpr long long DD = (long long)D * D;
  constexpr int TASKS = HG * NT, WPT = 4 / TASKS, T2 = 2 * NT;
  __shared__ __align__(16) bf16 sQ[4][16 * G::P];
  __shared__ __align__(16) bf16 sO[4][16 * G::P];
  __shared__ __align__(16) bf16 sWt[2][HG * D * kWtPitch<D>];  // W_e^T in bf16, by epoch parity
  __shared__ __align__(16) bf16 sWop[2 * HG * D * D];  // hi, then lo
  __shared__ f32x4 sSum[(4 - TASKS) > 0 ? (4 - TASKS) : 1][T2][64];
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int grp = item / S, s = item % S;
  const int b = grp / (H / HG), h0 = (grp % (H / HG)) * HG;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const int w = wave_id(), l = lane_id();
  const int task = w % TASKS, tw = w / TASKS, hl = task / NT, m = task % NT;
  const long long ts = (long long)H * D;
  const long long base = (long long)b * N * ts + (long long)h0 * D;

  const QBlocks<D, HG> qb(q, base, ts, n0, n1);
  typename QBlocks<D, HG>::Regs sets[kReadSets];
  qb.load_first(sets);

  // W* of the group, while those loads are in flight.
  f32x4 wr[NT];
  if (tw == 0) load_rows<D>(w0 + b * w0_bstride + (long long)(h0 + hl) * DD, m, l & 15, l >> 4, wr);
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
  if constexpr (WPT > 1) {
    if (tw > 0)
      for (int t = 0; t < T2; ++t) sSum[w - TASKS][t][l] = acc[t];
    __syncthreads();
    if (tw == 0)
      for (int u = 1; u < WPT; ++u)
        for (int t = 0; t < T2; ++t) acc[t] += sSum[(u - 1) * TASKS + task][t][l];
  }
  form_wstar<D, HG>(acc, wr, sWt[0], sWt[1], &sWop[0], scale, epochs,
                    (w_out && s == 0) ? w_out + ((long long)b * H + h0) * DD : nullptr);
  readout_blocks<D, HG>(qb, sets, sWop, sQ[w], sO[w], o);
}

// 1 + 2 in one launch, for plans with one split per group (many groups of few tokens, e.g. 64
// images x 196 tokens x 6 heads of 64): one workgroup per group sums K^T K and K^T V over all of
// the group's tokens (gram_sums, with the group's Q blocks and W0 already in flight), forms W*
// from the sums in its registers and reads out Q. No split records, one launch instead of two;
// the same arithmetic as the two launches with one split (a record sum from zero adds nothing).
// The read-out's LDS buffers reuse those of the sums.
template <int D, int HG>
struct FusedLds {
  using G = Geo<D, HG>;
  static constexpr int kTileB = kTile * G::P * 2;  // bytes of one staged 64-token tile
  static constexpr int kBlockB = 16 * G::P * 2;    // bytes of one wave's 16-token tile
  static constexpr int kWtB = HG * D * kWtPitch<D> * 2;  // bytes of the group's W^T (bf16)
  static constexpr int kSums = 4 * kTileB;                // sK[2], sV[2]
  static constexpr int kQ = 0, kO = 4 * kBlockB, kWop = 8 * kBlockB;
  static constexpr int kReadout = kWop + 2 * HG * D * D * 2;
  // W^T by epoch parity: beside the other buffers (stored while the sums' tiles may still be read)
  static constexpr int kWt = (kSums > kReadout ? kSums : kReadout);
  static constexpr int kBytes = kWt + 2 * kWtB;
};

template <int D, int HG>
__global__ __launch_bounds__(kThreads, 2) void fb_fused_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w0, long long w0_bstride, int H, int N, float scale, int epochs,
    bf16* __restrict__ o, float* __restrict__ w_out) {
  using G = Geo<D, HG>;
  using L = FusedLds<D, HG>;
  constexpr int NT = D / 16;
  constexpr long long DD = (long long)D * D;
  static_assert(sizeof(float) * (4 - HG * NT) * 2 * NT * 256 <= 2 * L::kTileB, "task sums fit in sK");
  __shared__ __align__(16) unsigned char smem[L::kBytes];
  bf16* sK = reinterpret_cast<bf16*>(smem);
  bf16* sV = reinterpret_cast<bf16*>(smem + 2 * L::kTileB);
  const int grp = blockIdx.x;
  const int b = grp / (H / HG), h0 = (grp % (H / HG)) * HG;
  const int w = wave_id(), l = lane_id();
  const int task = w % (HG * NT), tw = w / (HG * NT), hl = task / NT, m = task % NT;
  const long long ts = (long long)H * D;
  const long long base = (long long)b * N * ts + (long long)h0 * D;

  const QBlocks<D, HG> qb(q, base, ts, 0, N);
  typename QBlocks<D, HG>::Regs sets[kReadSets];
  qb.load_first(sets);
  f32x4 wr[NT];
  if (tw == 0) load_rows<D>(w0 + b * w0_bstride + (long long)(h0 + hl) * DD, m, l & 15, l >> 4, wr);

  f32x4 acc[2 * NT];  // tiles (c, m) of K^T K, then (m, n) of K^T V
  {
    f32x4 kk[NT], kv[NT];
    gram_sums<D, HG, false>(k, v, base, ts, 0, N, sK, sV, kk, kv);
    task_sum<D, HG>(reinterpret_cast<float*>(sK), kk, kv);
    for (int c = 0; c < NT; ++c) {
      acc[c] = kk[c];
      acc[NT + c] = kv[c];
    }
  }
  // (form_wstar's first barrier also ends every read of the tile buffers and task sums, which the
  // read-out's buffers reuse)
  bf16* sWop = reinterpret_cast<bf16*>(smem + L::kWop);
  form_wstar<D, HG>(acc, wr, reinterpret_cast<bf16*>(smem + L::kWt), reinterpret_cast<bf16*>(smem + L::kWt + L::kWtB),
                    sWop, scale, epochs, w_out ? w_out + ((long long)b * H + h0) * DD : nullptr);
  readout_blocks<D, HG>(qb, sets, sWop, reinterpret_cast<bf16*>(smem + L::kQ + w * L::kBlockB),
                        reinterpret_cast<bf16*>(smem + L::kO + w * L::kBlockB), o);
}

// ---------------------------------------------------------------- fp32 I/O, plain FMA
// Per (b, h, split): the split's K^T K and K^T V (plain fp32 FMA), as in the bf16 path.
template <int D>
__global__ __launch_bounds__(kThreads) void fb_partial_f32(const float* __restrict__ k,
                                                           const float* __restrict__ v, int H,
                                                           int N, int tps, int S,
                                                           float* __restrict__ partial) {
  __shared__ float sK[kTileF][D + 1], sV[kTileF][D + 1];
  constexpr int PER = (D * D + kThreads - 1) / kThreads;
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int n0 = s * tps, n1 = min(N, n0 + tps);
  const long long ts = (long long)H * D;
  float kk[PER], kv[PER];
  for (int u = 0; u < PER; ++u) kk[u] = kv[u] = 0.f;
  for (int t0 = n0; t0 < n1; t0 += kTileF) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTileF * D; e += kThreads) {
      const int t = e / D, c = e % D;
      const bool ok = t0 + t < n1;
      const long long off = ((long long)b * N + t0 + t) * ts + (long long)h * D + c;
      sK[t][c] = ok ? k[off] : 0.f;
      sV[t][c] = ok ? v[off] : 0.f;
    }
    __syncthreads();
    for (int u = 0; u < PER; ++u) {
      const int e = threadIdx.x + kThreads * u;
      if (e < D * D) {
        const int i = e / D, c = e % D;
        float a = kk[u], bb = kv[u];
        for (int t = 0; t < kTileF; ++t) {
          a = fmaf(sK[t][i], sK[t][c], a);
          bb = fmaf(sK[t][i], sV[t][c], bb);
        }
        kk[u] = a;
        kv[u] = bb;
      }
    }
  }
  float* out = partial + ((long long)bh * S + s) * 2 * D * D;
  for (int u = 0; u < PER; ++u) {
    const int e = threadIdx.x + kThreads * u;
    if (e < D * D) {
      out[e] = kk[u];
      out[D * D + e] = kv[u];
    }
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

// ---------------------------------------------------------------- fp32 reduction and epochs
// Per (b, h): sums the splits' K^T K and K^T V in a fixed order, then runs the epochs
// W <- W - scale ((K^T K) W - K^T V) from W0 in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void fb_reduce_f32(const float* __restrict__ partial, int S,
                                                          const float* __restrict__ w0,
                                                          long long w0_bstride, int H, float scale,
                                                          int epochs, float* __restrict__ wstar,
                                                          float* __restrict__ w_out) {
  __shared__ float sKK[D][D + 1], sKV[D][D + 1], sW[2][D][D + 1];
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const long long dd = (long long)D * D;
  const float* W0 = w0 + b * w0_bstride + h * dd;
  const float* pp = partial + (long long)bh * S * 2 * dd;
  for (int e = threadIdx.x; e < D * D; e += kThreads) {
    float a = 0.f, c = 0.f;
    for (int s = 0; s < S; ++s) {
      a += pp[s * 2 * dd + e];
      c += pp[s * 2 * dd + dd + e];
    }
    sKK[e / D][e % D] = a;
    sKV[e / D][e % D] = c;
    sW[0][e / D][e % D] = W0[e];
  }
  __syncthreads();
  int cur = 0;
  for (int ep = 0; ep < epochs; ++ep) {
    for (int e = threadIdx.x; e < D * D; e += kThreads) {
      const int i = e / D, c = e % D;
      float gw = 0.f;
      for (int kq = 0; kq < D; ++kq) gw = fmaf(sKK[i][kq], sW[cur][kq][c], gw);
      sW[cur ^ 1][i][c] = sW[cur][i][c] - scale * (gw - sKV[i][c]);
    }
    __syncthreads();
    cur ^= 1;
  }
  for (int e = threadIdx.x; e < D * D; e += kThreads) {
    const float wv = sW[cur][e / D][e % D];
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
hipError_t launch_bf16(int B, int H, int N, int epochs, float eta, const void* q, const void* k,
                       const void* v, const float* w0, long long w0s, void* o, float* w_out,
                       void* ws, hipStream_t st) {
  const int groups = B * (H / HG);
  const FbPlan pl = plan_splits(groups, N, tile_sets(D));
  float* partial = static_cast<float*>(ws);
  const int items = groups * pl.splits;
  const float scale = eta / (float)N;
  if (pl.splits == 1) {  // no split records: one launch (the workspace is not used)
    hipLaunchKernelGGL((fb_fused_bf16<D, HG>), dim3(groups), dim3(kThreads), 0, st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, w0, w0s, H, N, scale, epochs, (bf16*)o, w_out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fb_partial_bf16<D, HG, true>), dim3(items), dim3(kThreads), 0, st, (const bf16*)k,
                     (const bf16*)v, w0, w0s, H, N, pl.splits, pl.tokens_per_split, partial);
  hipLaunchKernelGGL((fb_readout_bf16<D, HG>), dim3(items), dim3(kThreads), 0, st, (const bf16*)q,
                     partial, w0, w0s, H, N, pl.splits, pl.tokens_per_split, scale, epochs, (bf16*)o,
                     w_out);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(int B, int H, int N, int epochs, float eta, const void* q, const void* k,
                      const void* v, const float* w0, long long w0s, void* o, float* w_out,
                      void* ws, hipStream_t st) {
  const int BH = B * H;
  const FbPlan pl = plan_splits(BH, N, 1);
  float* partial = static_cast<float*>(ws);
  float* wstar = partial + (size_t)BH * pl.splits * 2 * D * D;
  const dim3 grid(pl.splits, BH);
  hipLaunchKernelGGL(fb_partial_f32<D>, grid, dim3(kThreads), 0, st, (const float*)k,
                     (const float*)v, H, N, pl.tokens_per_split, pl.splits, partial);
  hipLaunchKernelGGL(fb_reduce_f32<D>, dim3(BH), dim3(kThreads), 0, st, partial, pl.splits, w0, w0s,
                     H, eta / (float)N, epochs, wstar, w_out);
  hipLaunchKernelGGL(fb_readout_f32<D>, grid, dim3(kThreads), 0, st, (const float*)q, wstar, H,
                     N, pl.tokens_per_split, (float*)o);
  return hipGetLastError();
}


// ---------------------------------------------------------------- backward (outer-loop gradients)
// Given dO, the gradients of the one-step layer (closed form; the pages' authors likewise write
// the inner gradient by hand, ViT^3 review, section on the official code). With s = eta/N,
// W* = W0 - s ((K^T K) W0 - K^T V), G = Q^T dO and M = W0 G^T + G W0^T:
//   dQ = dO W*^T,   dV = s K G,   dK = -s (K M - V G^T),   dW0 = G - s (K^T K) G.
// Three launches after the sums (the partial kernels above, run on (K, V) for K^T K and K^T V
// and on (Q, dO), whose second product is G):
//   fbb_finish: per (b, h), the fixed-order sums of the split records, then W*, dW0 and M in
//               LDS (plain fp32), written out as the token kernel's four operand matrices
//               A_q = W*, A_v = s G^T, A_k1 = -s M, A_k2 = s G (bf16 MFMA tiles, or fp32);
//   fbb_tokens: per 16-token tile, dQ^T = A_q dO^T, dV^T = A_v K^T, dK^T = A_k1 K^T + A_k2 V^T.
constexpr int kBwdMats = 4;

// One workgroup per (b, h). rec_kv / rec_qd: the group's split records (bf16 path) or the
// (b, h)'s (fp32 path: per split K^T K then K^T V, row-major). ops: the four operand matrices.
template <int D, int HG, bool BF16>
__global__ __launch_bounds__(kThreads) void fbb_finish(const float* __restrict__ rec_kv,
                                                       const float* __restrict__ rec_qd,
                                                       const float* __restrict__ w0,
                                                       long long w0_bstride, int H, int S,
                                                       float s_eta, void* __restrict__ ops,
                                                       float* __restrict__ d_w0) {
  __shared__ float sKK[D][D + 1], sKV[D][D + 1], sG[D][D + 1], sW0[D][D + 1];
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const long long DD = (long long)D * D;
  const float* W0 = w0 + b * w0_bstride + h * DD;
  if constexpr (BF16) {
    // The head's part of a split record is 2 d^2 contiguous floats (its tasks' tiles), laid out
    // alike in every split: sum it in split order over 16-byte pieces (the loads of 8 splits in
    // flight at once), then scatter each element to its (row, column).
    constexpr int NT = D / 16, TASK = 2 * NT * 256, U = 8;
    const int grp = b * (H / HG) + h / HG, hl = h % HG;
    const long long rstride = 2LL * HG * DD;  // floats per split record of the group
    const float* rk = rec_kv + (long long)grp * S * rstride + (long long)hl * 2 * DD;
    const float* rq = rec_qd + (long long)grp * S * rstride + (long long)hl * 2 * DD;
    for (int o4 = threadIdx.x; o4 < 2 * DD / 4; o4 += kThreads) {
      f32x4 ak = zero4(), aq = zero4();
      for (int sp0 = 0; sp0 < S; sp0 += U) {
        f32x4 bk[U], bq[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (sp0 + u < S) {
            bk[u] = *reinterpret_cast<const f32x4*>(rk + (sp0 + u) * rstride + 4 * o4);
            bq[u] = *reinterpret_cast<const f32x4*>(rq + (sp0 + u) * rstride + 4 * o4);
          }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (sp0 + u < S) {
            ak += bk[u];
            aq += bq[u];
          }
      }
      // offset 4 o4 + jj: task tl, tile tt, lane r + 16 g, element jj (the record layout)
      const int tl = (4 * o4) / TASK, rem = (4 * o4) % TASK, tt = rem / 256, lane = (rem % 256) / 4;
      const int r = lane % 16, g = lane / 16;
      for (int jj = 0; jj < 4; ++jj) {
        if (tt < NT) {  // K^T K tile (c = tt, m = tl)
          sKK[16 * tt + 4 * g + jj][16 * tl + r] = ak[jj];
        } else {        // K^T V and Q^T dO tiles (m = tl, n = tt - NT)
          sKV[16 * tl + 4 * g + jj][16 * (tt - NT) + r] = ak[jj];
          sG[16 * tl + 4 * g + jj][16 * (tt - NT) + r] = aq[jj];
        }
      }
    }
    for (int e = threadIdx.x; e < D * D; e += kThreads) sW0[e / D][e % D] = W0[e];
  }
  if constexpr (!BF16) {  // per (b, h, split): K^T K then K^T V (or Q^T Q then Q^T dO), row-major
    for (int e = threadIdx.x; e < D * D; e += kThreads) {
      const int i = e / D, j = e % D;
      float kk = 0.f, kv = 0.f, gq = 0.f;
      for (int sp = 0; sp < S; ++sp) {
        const long long base = ((long long)bh * S + sp) * 2 * DD;
        kk += rec_kv[base + e];
        kv += rec_kv[base + DD + e];
        gq += rec_qd[base + DD + e];
      }
      sKK[i][j] = kk;
      sKV[i][j] = kv;
      sG[i][j] = gq;
      sW0[i][j] = W0[e];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < D * D; e += kThreads) {
    const int i = e / D, j = e % D;
    float kw = 0.f, kg = 0.f, m = 0.f;
    for (int c = 0; c < D; ++c) {
      kw = fmaf(sKK[i][c], sW0[c][j], kw);
      kg = fmaf(sKK[i][c], sG[c][j], kg);
      m = fmaf(sW0[i][c], sG[j][c], fmaf(sG[i][c], sW0[j][c], m));
    }
    const float ws = sW0[i][j] - s_eta * (kw - sKV[i][j]);
    d_w0[(long long)bh * DD + e] = sG[i][j] - s_eta * kg;
    // A_q = W*, A_v = s G^T, A_k1 = -s M, A_k2 = s G, element (row i, k = j)
    const float a[kBwdMats] = {ws, s_eta * sG[j][i], -s_eta * m, s_eta * sG[i][j]};
    for (int mat = 0; mat < kBwdMats; ++mat) {
      if constexpr (BF16) {
        // operand tile (column tile n = i / 16, k step ks), lane r + 16 g, element ii
        constexpr int E = D >= 32 ? 8 : 4, KS = D >= 32 ? D / 32 : 1;
        const int n = i / 16, r = i % 16, ks = j / (4 * E), g = (j % (4 * E)) / E, ii = j % E;
        bf16* dst = static_cast<bf16*>(ops) + (long long)bh * kBwdMats * DD + mat * DD;
        dst[((n * KS + ks) * 64 + r + 16 * g) * E + ii] = (bf16)a[mat];
      } else {
        static_cast<float*>(ops)[(long long)bh * kBwdMats * DD + mat * DD + e] = a[mat];
      }
    }
  }
}

// bf16: one workgroup per (256-token block, b, h); wave w handles 16-token tiles w, w + 4, ... of
// the block. Operands of the four matrices are staged in LDS (lane order); each tile's dO, K, V
// rows are the B operands (lane (r, g): token r, features 8g.. of a 32-feature k step, one 16-byte
// load), and the results come out transposed (lane (r, g): 4 adjacent output features of token r,
// one 8-byte store).
constexpr int kBwdTok = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void fbb_tokens_bf16(
    const bf16* __restrict__ d_o, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ ops, int H, int N, bf16* __restrict__ d_q, bf16* __restrict__ d_k,
    bf16* __restrict__ d_v) {
  constexpr int NT = D / 16, E = D >= 32 ? 8 : 4, KS = D >= 32 ? D / 32 : 1;
  constexpr int DD = D * D;
  typedef typename std::conditional<(D >= 32), bf16x8, bf16x4>::type Op;
  __shared__ __align__(16) bf16 sOps[kBwdMats * DD];
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const bf16* src = ops + (long long)bh * kBwdMats * DD;
  for (int e = threadIdx.x * 8; e < kBwdMats * DD; e += kThreads * 8)
    *reinterpret_cast<uint4*>(&sOps[e]) = *reinterpret_cast<const uint4*>(&src[e]);
  __syncthreads();
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;
  auto mma = [](Op a, Op bb, f32x4 c) {
    if constexpr (D >= 32) return mma32(a, bb, c);
    else return mma16(a, bb, c);
  };
  auto aop = [&](int mat, int n, int ks) {
    return *reinterpret_cast<const Op*>(&sOps[mat * DD + ((n * KS + ks) * 64 + l) * E]);
  };
  for (int tile = w; tile * 16 < kBwdTok; tile += 4) {
    const int t0 = blockIdx.x * kBwdTok + tile * 16;
    if (t0 >= N) break;
    const bool ok = t0 + r < N;
    const long long row = head0 + (long long)(t0 + r) * ts;
    Op xo[KS], xk[KS], xv[KS];
    for (int ks = 0; ks < KS; ++ks) {
      const int col = ks * 4 * E + E * g;
      xo[ks] = ok ? *reinterpret_cast<const Op*>(d_o + row + col) : Op{};
      xk[ks] = ok ? *reinterpret_cast<const Op*>(k + row + col) : Op{};
      xv[ks] = ok ? *reinterpret_cast<const Op*>(v + row + col) : Op{};
    }
    for (int n = 0; n < NT; ++n) {
      f32x4 aq = zero4(), av = zero4(), ak = zero4();
      for (int ks = 0; ks < KS; ++ks) {
        aq = mma(aop(0, n, ks), xo[ks], aq);
        av = mma(aop(1, n, ks), xk[ks], av);
        ak = mma(aop(2, n, ks), xk[ks], ak);
        ak = mma(aop(3, n, ks), xv[ks], ak);
      }
      if (ok) {
        const long long o = row + 16 * n + 4 * g;
        *reinterpret_cast<bf16x4*>(d_q + o) = to_bf16x4(aq);
        *reinterpret_cast<bf16x4*>(d_v + o) = to_bf16x4(av);
        *reinterpret_cast<bf16x4*>(d_k + o) = to_bf16x4(ak);
      }
    }
  }
}

// fp32: plain FMA, one workgroup per (256-token block, b, h); the matrices in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void fbb_tokens_f32(
    const float* __restrict__ d_o, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ ops, int H, int N, float* __restrict__ d_q, float* __restrict__ d_k,
    float* __restrict__ d_v) {
  __shared__ float sA[kBwdMats][D][D + 1];
  __shared__ float sX[3][kTileF][D + 1];
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const float* src = ops + (long long)bh * kBwdMats * D * D;
  for (int e = threadIdx.x; e < kBwdMats * D * D; e += kThreads) sA[e / (D * D)][(e / D) % D][e % D] = src[e];
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;
  for (int t0 = blockIdx.x * kBwdTok; t0 < min(N, (int)(blockIdx.x + 1) * kBwdTok); t0 += kTileF) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTileF * D; e += kThreads) {
      const int t = e / D, c = e % D;
      const bool ok = t0 + t < N;
      const long long off = head0 + (long long)(t0 + t) * ts + c;
      sX[0][t][c] = ok ? d_o[off] : 0.f;
      sX[1][t][c] = ok ? k[off] : 0.f;
      sX[2][t][c] = ok ? v[off] : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kTileF * D; e += kThreads) {
      const int t = e / D, i = e % D;
      if (t0 + t >= N) continue;
      float q = 0.f, vv = 0.f, kk = 0.f;
      for (int j = 0; j < D; ++j) {
        q = fmaf(sA[0][i][j], sX[0][t][j], q);
        vv = fmaf(sA[1][i][j], sX[1][t][j], vv);
        kk = fmaf(sA[2][i][j], sX[1][t][j], fmaf(sA[3][i][j], sX[2][t][j], kk));
      }
      const long long off = head0 + (long long)(t0 + t) * ts + i;
      d_q[off] = q;
      d_v[off] = vv;
      d_k[off] = kk;
    }
  }
}

template <int D, int HG>
hipError_t launch_bwd_bf16(int B, int H, int N, float eta, const void* q, const void* k,
                           const void* v, const float* w0, long long w0s, const void* d_o,
                           void* d_q, void* d_k, void* d_v, float* d_w0, void* ws,
                           hipStream_t st) {
  const int groups = B * (H / HG);
  const FbPlan pl = plan_splits(groups, N, tile_sets(D));
  const size_t rec = (size_t)groups * pl.splits * 2 * HG * D * D;  // floats per record set
  float* rkv = static_cast<float*>(ws);
  float* rqd = rkv + rec;
  bf16* ops = reinterpret_cast<bf16*>(rqd + rec);
  const int items = groups * pl.splits;
  hipLaunchKernelGGL((fb_partial_bf16<D, HG, false>), dim3(items), dim3(kThreads), 0, st, (const bf16*)k,
                     (const bf16*)v, w0, w0s, H, N, pl.splits, pl.tokens_per_split, rkv);
  hipLaunchKernelGGL((fb_partial_bf16<D, HG, false>), dim3(items), dim3(kThreads), 0, st, (const bf16*)q,
                     (const bf16*)d_o, w0, w0s, H, N, pl.splits, pl.tokens_per_split, rqd);
  hipLaunchKernelGGL((fbb_finish<D, HG, true>), dim3(B * H), dim3(kThreads), 0, st, rkv, rqd, w0, w0s,
                     H, pl.splits, eta / (float)N, (void*)ops, d_w0);
  hipLaunchKernelGGL((fbb_tokens_bf16<D>), dim3((N + kBwdTok - 1) / kBwdTok, B * H), dim3(kThreads), 0,
                     st, (const bf16*)d_o, (const bf16*)k, (const bf16*)v, (const bf16*)ops, H, N,
                     (bf16*)d_q, (bf16*)d_k, (bf16*)d_v);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_f32(int B, int H, int N, float eta, const void* q, const void* k,
                          const void* v, const float* w0, long long w0s, const void* d_o,
                          void* d_q, void* d_k, void* d_v, float* d_w0, void* ws, hipStream_t st) {
  const int BH = B * H;
  const FbPlan pl = plan_splits(BH, N, 1);
  const size_t rec = (size_t)BH * pl.splits * 2 * D * D;
  float* rkv = static_cast<float*>(ws);
  float* rqd = rkv + rec;
  float* ops = rqd + rec;
  const dim3 grid(pl.splits, BH);
  hipLaunchKernelGGL(fb_partial_f32<D>, grid, dim3(kThreads), 0, st, (const float*)k, (const float*)v,
                     H, N, pl.tokens_per_split, pl.splits, rkv);
  hipLaunchKernelGGL(fb_partial_f32<D>, grid, dim3(kThreads), 0, st, (const float*)q, (const float*)d_o,
                     H, N, pl.tokens_per_split, pl.splits, rqd);
  hipLaunchKernelGGL((fbb_finish<D, 1, false>), dim3(BH), dim3(kThreads), 0, st, rkv, rqd, w0, w0s, H,
                     pl.splits, eta / (float)N, (void*)ops, d_w0);
  hipLaunchKernelGGL(fbb_tokens_f32<D>, dim3((N + kBwdTok - 1) / kBwdTok, BH), dim3(kThreads), 0, st,
                     (const float*)d_o, (const float*)k, (const float*)v, (const float*)ops, H, N,
                     (float*)d_q, (float*)d_k, (float*)d_v);
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
    return (size_t)B * H * p.splits * 2 * dd + (size_t)B * H * dd;
  }
  const int hg = head_group(H, D);
  const int groups = B * (H / hg);
  const FbPlan p = plan_splits(groups, N, tile_sets(D));
  return (size_t)groups * p.splits * 2 * hg * dd;
}

hipError_t fb_launch(bool bf16_io, int B, int H, int N, int D, int epochs, float eta,
                     const void* q, const void* k, const void* v, const float* w0, long long w0s,
                     void* o, float* w_out, void* ws, hipStream_t st) {
  const int E = epochs;
  if (!bf16_io) {
    switch (D) {
      case 16: return launch_f32<16>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
      case 32: return launch_f32<32>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
      case 64: return launch_f32<64>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
      default: return hipErrorInvalidValue;
    }
  }
  const int hg = head_group(H, D);
  switch (D * 8 + hg) {
    case 64 * 8 + 1: return launch_bf16<64, 1>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 32 * 8 + 2: return launch_bf16<32, 2>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 32 * 8 + 1: return launch_bf16<32, 1>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 16 * 8 + 4: return launch_bf16<16, 4>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 16 * 8 + 2: return launch_bf16<16, 2>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    case 16 * 8 + 1: return launch_bf16<16, 1>(B, H, N, E, eta, q, k, v, w0, w0s, o, w_out, ws, st);
    default: return hipErrorInvalidValue;
  }
}

size_t fbb_workspace_bytes(bool bf16_io, int B, int H, int N, int D) {
  const size_t dd = (size_t)D * D;
  if (!bf16_io) {
    const FbPlan p = plan_splits(B * H, N, 1);
    return (2 * (size_t)B * H * p.splits * 2 * dd + (size_t)B * H * kBwdMats * dd) * sizeof(float);
  }
  const int hg = head_group(H, D);
  const int groups = B * (H / hg);
  const FbPlan p = plan_splits(groups, N, tile_sets(D));
  return 2 * (size_t)groups * p.splits * 2 * hg * dd * sizeof(float) + (size_t)B * H * kBwdMats * dd * 2;
}

hipError_t fbb_launch(bool bf16_io, int B, int H, int N, int D, float eta, const void* q,
                      const void* k, const void* v, const float* w0, long long w0s,
                      const void* d_o, void* d_q, void* d_k, void* d_v, float* d_w0, void* ws,
                      hipStream_t st) {
  if (!bf16_io) {
    switch (D) {
      case 16: return launch_bwd_f32<16>(B, H, N, eta, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
      case 32: return launch_bwd_f32<32>(B, H, N, eta, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
      case 64: return launch_bwd_f32<64>(B, H, N, eta, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
      default: return hipErrorInvalidValue;
    }
  }
  const int hg = head_group(H, D);
  switch (D * 8 + hg) {
#define TTT_BWD(DV, HGV)                                                                          \
  case DV * 8 + HGV:                                                                             \
    return launch_bwd_bf16<DV, HGV>(B, H, N, eta, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
    TTT_BWD(64, 1)
    TTT_BWD(32, 2)
    TTT_BWD(32, 1)
    TTT_BWD(16, 4)
    TTT_BWD(16, 2)
    TTT_BWD(16, 1)
#undef TTT_BWD
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
