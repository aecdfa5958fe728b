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
// Parallel structure. The chunk step is affine in the state: W -> A_c W + B_c with
// A_c = I - a K_c^T K_c and B_c = a K_c^T V_c (a = eta/b). A run of chunks (a "segment") therefore
// composes to one affine map, and the sequence is processed in three launches:
//   1. chunk_compose: one workgroup per (segment, b, h) composes its segment's map by scanning
//      the 2D-column state [P | R] from [I | 0] (columns are independent regressions). It stores
//      Dev = I - P (the small deviation, which keeps bf16 operands accurate) and R. Every A_c is
//      symmetric, so the reverse scan's composite of the segment is Dev^T; its offset
//      R_rev = a sum_c (K_c P_{c-1})^T V_c is accumulated alongside.
//   2. chunk_prefix: one single-wave workgroup per (b, h, direction, 16-column tile) folds the
//      segment maps in order from W0 and stores every segment's entry state
//      (W <- W - Dev W + R per segment).
//   3. chunk_scan: one workgroup per (segment, b, h) rescans its segment from its true entry
//      state and writes the outputs. For the bidirectional scan it first runs the reverse scan
//      over its chunks, keeping each W^r_c (bf16) in LDS, then the forward scan with the read-out.
// A single segment (short sequences) skips launches 1 and 2.
//
// Inside every kernel, wave w owns columns [16w, 16w + 16) of its state (the columns of W are
// independent regressions), held in MFMA accumulator layout; the chunk's K, V, Q are staged
// through LDS with the next chunk prefetched into registers.
#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

enum ScanMode { kCausal = 0, kBidir = 1 };

// Segment map record of one (b, h, segment, direction): -Dev as bf16 (the MFMA operand of the
// prefix fold, already negated) followed by R as fp32; kMapFloats<D> floats in all. Records and
// segment entry states are stored as MFMA register tiles, so that each lane moves its operands
// with 16-byte accesses:
//  - state tiles (R and the entry states, fp32): tile (column tile n, row tile m) holds, for lane
//    l = r + 16g, rows 16m + 4g + j (j < 4) of column 16n + r, contiguous (the accumulator layout);
//  - -Dev tiles (bf16): the A operand of the fold's product. Tile (row tile m, k slot ks) holds,
//    for lane l = r + 16g, row 16m + r at k = 32ks + 4g + i and 32ks + 16 + 4g + i (i < 4); for
//    D = 16 only k = 4g + i.
template <int D>
constexpr int kMapFloats = D * D / 2 + D * D;
template <int D>
constexpr int kDevElems = D >= 32 ? 8 : 4;

template <int D>
__device__ __forceinline__ long long state_tile(int n, int m, int l) {  // float offset
  return ((long long)(n * (D / 16) + m) * 64 + l) * 4;
}

template <int D>
__device__ __forceinline__ int dev_offset(int row, int kcol) {  // bf16 offset of -Dev[row][kcol]
  constexpr int KS = D >= 32 ? D / 32 : 1;
  const int kk = kcol & 31, half = kk >> 4, gg = (kk & 15) >> 2;
  return (((row >> 4) * KS + (kcol >> 5)) * 64 + (row & 15) + 16 * gg) * kDevElems<D> + (kk & 3) +
         4 * half;
}

// Row pitch (elements) of the [token][feature] LDS tiles. For d = 64 it is 76 (152 bytes = 38 banks of 4 bytes): the
// two 8-byte reads 32 bytes apart that form a c-layout operand, the row reads and the transpose reads then hit
// distinct banks (a 144-byte pitch makes the paired reads of rows r and r + 2 collide). Rows are then only 8-byte
// aligned, so tiles move through LDS in 8-byte pieces.
template <int D>
constexpr int lds_pitch() { return D == 64 ? 76 : D + 8; }
// 16 bytes between registers and an LDS row that may be only 8-byte aligned.
__device__ __forceinline__ void st16_lds8(bf16* p, uint4 v) {
  reinterpret_cast<uint2*>(p)[0] = make_uint2(v.x, v.y);
  reinterpret_cast<uint2*>(p)[1] = make_uint2(v.z, v.w);
}
__device__ __forceinline__ uint4 ld16_lds8(const bf16* p) {
  const uint2 a = reinterpret_cast<const uint2*>(p)[0], b = reinterpret_cast<const uint2*>(p)[1];
  return make_uint4(a.x, a.y, b.x, b.y);
}

// LDS bytes available for the reverse states of one bidirectional scan segment: 80 KB holds 10
// states of d = 64 and leaves room for double-buffered 64-token tiles (one barrier per chunk).
constexpr int kRevLdsBytes = 80 * 1024;
template <int D>
constexpr int max_seg_len() { return kRevLdsBytes / (D * D * 2); }

// ---------------------------------------------------------------- staging with prefetch
// The [CH x D] bf16 tiles of NTS tensors of one chunk move HBM -> registers -> LDS (row pitch P).
// The workgroup's threads form G groups; group j holds the chunks whose step index is j mod G: it
// loads a chunk G steps before the step that uses it and stores it to LDS at the start of that
// step, so each load has G steps to arrive with one register set per thread. A thread's 16-byte
// pieces sit at fixed offsets within a chunk tile, computed once; when a tile spans whole waves,
// the tensor of a piece is the same across the wave, and choosing its base pointer is scalar work.
template <int D, int CH, int NTH, int NTS, int G, int P>
struct ChunkStager {
  static_assert(NTH % G == 0 && NTS >= 1 && NTS <= 3, "staging geometry");
  static constexpr int CPR = D / 8;  // 16-byte pieces per row
  static constexpr int TILE = CH * CPR;
  static constexpr int PIECES = NTS * TILE;
  static constexpr int GT = NTH / G;  // threads per group
  static constexpr int PER = (PIECES + GT - 1) / GT;
  static constexpr bool kUniform = TILE % 64 == 0 && GT % 64 == 0;
  uint4 v[PER];
  int group;
  int sel[PER], goff[PER], loff[PER];
  __device__ __forceinline__ explicit ChunkStager(long long ts) : group(threadIdx.x / GT) {
    const int idx = threadIdx.x % GT;
    for (int i = 0; i < PER; ++i) {
      const int p = idx + i * GT, rem = p % TILE;
      sel[i] = kUniform ? __builtin_amdgcn_readfirstlane(p / TILE) : p / TILE;
      goff[i] = (int)((rem / CPR) * ts) + (rem % CPR) * 8;
      loff[i] = (rem / CPR) * P + (rem % CPR) * 8;
    }
  }
  __device__ __forceinline__ bool mine(int step) const { return step % G == group; }
  __device__ __forceinline__ bool valid(int i) const {
    return PIECES % GT == 0 || (int)(threadIdx.x % GT) + i * GT < PIECES;
  }
  // t0, t1, t2: the chunk's first row in each tensor.
  __device__ __forceinline__ void load(const bf16* t0, const bf16* t1, const bf16* t2) {
    for (int i = 0; i < PER; ++i)
      if (valid(i)) {
        const bf16* src = sel[i] == 0 ? t0 : (sel[i] == 1 ? t1 : t2);
        v[i] = ld16(src + goff[i]);
      }
  }
  __device__ __forceinline__ void store(bf16* d0, bf16* d1, bf16* d2) const {
    for (int i = 0; i < PER; ++i)
      if (valid(i)) {
        bf16* dst = sel[i] == 0 ? d0 : (sel[i] == 1 ? d1 : d2);
        st16_lds8(dst + loff[i], v[i]);
      }
  }
};

// Prefetch groups: 16-token chunks leave half of the threads idle for one chunk's tiles, so two
// groups stage alternate chunks two steps ahead at no register cost.
template <int CH>
constexpr int stage_groups() { return CH == 16 ? 2 : 1; }

template <int D, int CH, int P, int NTH>
__device__ __forceinline__ void store_chunk(bf16* dst, const bf16* src, long long ts) {
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < CH * CPR; c += NTH) {
    const int row = c / CPR, col = (c % CPR) * 8;
    st16(dst + row * ts + col, ld16_lds8(src + row * P + col));
  }
}

// ---------------------------------------------------------------- MFMA building blocks
// B operand from a state held in C layout (tiles m = 2ks, 2ks + 1 cover features 32ks..32ks+31).
__device__ __forceinline__ bf16x8 b_state(const f32x4* W, int ks) {
  return cat8(to_bf16x4(W[2 * ks]), to_bf16x4(W[2 * ks + 1]));
}

// Y[16 rows x 16 cols] = X_rows(row0..row0+15) . W[:, cols] + init, contraction over D; the A
// operand reads X rows from LDS in the c-layout k map that matches W's accumulator layout.
template <int D, int P>
__device__ __forceinline__ f32x4 rows_times_state(const bf16* X, int row0, const f32x4* W,
                                                  f32x4 init, int r, int g) {
  if constexpr (D >= 32) {
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16* p = X + (row0 + r) * P + 32 * ks + 4 * g;
      init = mma32(cat8(ld4(p), ld4(p + 16)), b_state(W, ks), init);
    }
  } else {
    init = mma16(ld4(X + (row0 + r) * P + 4 * g), to_bf16x4(W[0]), init);
  }
  return init;
}

// The transpose of the above without init: Y^T[16 cols x 16 rows] = W[:, cols]^T X_rows^T. The
// state tiles in accumulator layout are the A operand of W^T; lane (r, g) gets the 4 adjacent
// columns 4g.. of row row0 + r (one 8-byte store).
template <int D, int P>
__device__ __forceinline__ f32x4 state_times_rows(const bf16* X, int row0, const f32x4* W, int r,
                                                  int g) {
  f32x4 acc = zero4();
  if constexpr (D >= 32) {
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16* p = X + (row0 + r) * P + 32 * ks + 4 * g;
      acc = mma32(b_state(W, ks), cat8(ld4(p), ld4(p + 16)), acc);
    }
  } else {
    acc = mma16(to_bf16x4(W[0]), ld4(X + (row0 + r) * P + 4 * g), acc);
  }
  return acc;
}

// W[:, cols] += K^T (-a E): A = K^T (row = feature 16m + r, k = token 16p + 4g + j, by LDS
// transpose reads), B = -a E_p (accumulator layout). Chunks of 32 tokens or more contract 32 tokens
// per product (k map {4g + j} u {16 + 4g + j} on both operands).
template <int D, int NP, int P>
__device__ __forceinline__ void update_state(f32x4* W, const f32x4* E, const bf16* sK, float a,
                                             int l) {
  if constexpr (NP == 1) {
    const bf16x4 eb = to_bf16x4_scaled(E[0], -a);
    for (int m = 0; m < D / 16; ++m) W[m] = mma16(tile_tr(&sK[16 * m], P, l), eb, W[m]);
  } else {
    for (int p = 0; p < NP; p += 2) {
      const bf16x8 eb = cat8(to_bf16x4_scaled(E[p], -a), to_bf16x4_scaled(E[p + 1], -a));
      for (int m = 0; m < D / 16; ++m) {
        const bf16x8 kt = cat8(tile_tr(&sK[16 * p * P + 16 * m], P, l), tile_tr(&sK[16 * (p + 1) * P + 16 * m], P, l));
        W[m] = mma32(kt, eb, W[m]);
      }
    }
  }
}

// E_p = K_p W - V_p[:, 16*vcol ..] for every 16-token tile p (V skipped when vcol < 0).
template <int D, int NP, int P>
__device__ __forceinline__ void residuals(f32x4* E, const f32x4* W, const bf16* sK,
                                          const bf16* sV, int vcol, int r, int g, int l) {
  for (int p = 0; p < NP; ++p) {
    f32x4 init = zero4();
    if (vcol >= 0) {  // -V tile in accumulator layout, by an LDS transpose read
      const bf16x4 vt = tile_tr(&sV[16 * p * P + 16 * vcol], P, l);
      for (int j = 0; j < 4; ++j) init[j] = -(float)vt[j];
    }
    E[p] = rows_times_state<D, P>(sK, 16 * p, W, init, r, g);
  }
}

// ---------------------------------------------------------------- 1. compose
template <int D, int CH, bool BIDIR>
__global__ __launch_bounds__(D / 8 * 64) void chunk_compose_bf16(
    const bf16* __restrict__ k, const bf16* __restrict__ v, int H, int N, float a, int S, int L,
    float* __restrict__ comp) {
  constexpr int P = lds_pitch<D>(), NT = D / 16, NP = CH / 16, NTH = 2 * NT * 64;
  constexpr long long DD = (long long)D * D;
  // Double-buffered chunk tiles: chunk c is staged while other waves may still read chunk c - 1,
  // so one barrier per chunk suffices.
  __shared__ __align__(16) bf16 sKb[2][CH * P];
  __shared__ __align__(16) bf16 sVb[2][CH * P];

  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const bool pwave = w < NT;        // P columns (init I, no V); else R columns (init 0, V)
  const int col = pwave ? w : w - NT;
  const int C = N / CH;
  const int lo = s * L, hi = min(C, lo + L);
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;

  f32x4 X[NT], RR[NT];
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j) {
      X[m][j] = (pwave && 16 * m + 4 * g + j == 16 * col + r) ? 1.f : 0.f;
      RR[m][j] = 0.f;
    }

  constexpr int G = stage_groups<CH>();
  ChunkStager<D, CH, NTH, 2, G, P> st(ts);
  const long long cs = (long long)CH * ts;  // elements between consecutive chunks
  const bf16* kn = k + head0 + lo * cs;     // chunk lo + j (j < G), then chunk c + G
  const bf16* vn = v + head0 + lo * cs;
  for (int j = 0; j < G; ++j, kn += cs, vn += cs)
    if (lo + j < hi && st.mine(j)) st.load(kn, vn, nullptr);
  for (int c = lo; c < hi; ++c, kn += cs, vn += cs) {
    bf16* sK = sKb[(c - lo) & 1];
    bf16* sV = sVb[(c - lo) & 1];
    if (st.mine(c - lo)) {
      st.store(sK, sV, nullptr);
      if (c + G < hi) st.load(kn, vn, nullptr);
    }
    __syncthreads();
    f32x4 Y[NP];
    residuals<D, NP, P>(Y, X, sK, sV, pwave ? -1 : col, r, g, l);
    if constexpr (BIDIR) {
      if (pwave) {  // R_rev[16col + i][16n + .] += a (K_c P_{c-1})^T V_c
        if constexpr (NP == 1) {
          const bf16x4 ya = to_bf16x4_scaled(Y[0], a);
          for (int n = 0; n < NT; ++n) RR[n] = mma16(ya, tile_tr(&sV[16 * n], P, l), RR[n]);
        } else {  // 32 tokens per product, k map {4g + j} u {16 + 4g + j}
          for (int p = 0; p < NP; p += 2) {
            const bf16x8 ya = cat8(to_bf16x4_scaled(Y[p], a), to_bf16x4_scaled(Y[p + 1], a));
            for (int n = 0; n < NT; ++n)
              RR[n] = mma32(ya, cat8(tile_tr(&sV[16 * p * P + 16 * n], P, l),
                                     tile_tr(&sV[16 * (p + 1) * P + 16 * n], P, l)), RR[n]);
          }
        }
      }
    }
    update_state<D, NP, P>(X, Y, sK, a, l);
  }

  // comp[(bh * S + s)] holds the forward map record and, for the bidirectional scan, the
  // reverse one (-Dev_r = -Dev_f^T, R_rev).
  float* rec = comp + ((long long)bh * S + s) * (BIDIR ? 2 : 1) * kMapFloats<D>;
  bf16* ndev_f = reinterpret_cast<bf16*>(rec);
  float* r_f = rec + DD / 2;
  bf16* ndev_r = reinterpret_cast<bf16*>(rec + kMapFloats<D>);
  float* r_r = rec + kMapFloats<D> + DD / 2;
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * m + 4 * g + j, cc = 16 * col + r;
      if (pwave) {
        const bf16 nd = (bf16)(X[m][j] - (row == cc ? 1.f : 0.f));  // -Dev = P - I
        ndev_f[dev_offset<D>(row, cc)] = nd;
        if constexpr (BIDIR) ndev_r[dev_offset<D>(cc, row)] = nd;  // Dev_r = Dev_f^T
      }
    }
  if (!pwave)
    for (int m = 0; m < NT; ++m) *reinterpret_cast<f32x4*>(r_f + state_tile<D>(col, m, l)) = X[m];
  if constexpr (BIDIR) {
    if (pwave)  // RR[n] is R_rev's tile (column tile n, row tile col)
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(r_r + state_tile<D>(n, col, l)) = RR[n];
  }
}

// ---------------------------------------------------------------- 2. prefix over segments
// The columns of W are independent regressions, so the fold over the segment maps,
// W[:, cols] <- W[:, cols] + (-Dev) W[:, cols] + R[:, cols], runs as one single-wave workgroup
// per (b, h, direction, 16-column tile), storing each segment's entry state. Its speed is the
// latency of one step (a few dependent products), so there is no LDS and no barrier: each lane
// loads its own operands of a map record (rows of -Dev, its R entries) straight into registers,
// kPrefixSets steps ahead, rotating through kPrefixSets register sets.
constexpr int kPrefixSets = 4;

template <int D>
struct PrefixOperands {
  static constexpr int NT = D / 16, KS = D >= 32 ? D / 32 : 1;
  bf16x8 dev[NT][KS];  // -Dev tiles (D >= 32)
  bf16x4 dev16;        // -Dev tile for D = 16
  f32x4 rr[NT];        // R tiles (column tile col, row tile m)
  __device__ __forceinline__ void load(const float* rec, int col, int l) {
    const bf16* nd = reinterpret_cast<const bf16*>(rec);
    const float* R = rec + D * D / 2;
    if constexpr (D >= 32) {
      for (int m = 0; m < NT; ++m)
        for (int ks = 0; ks < KS; ++ks)
          dev[m][ks] = *reinterpret_cast<const bf16x8*>(nd + ((m * KS + ks) * 64 + l) * 8);
    } else {
      dev16 = *reinterpret_cast<const bf16x4*>(nd + l * 4);
    }
    for (int m = 0; m < NT; ++m) rr[m] = *reinterpret_cast<const f32x4*>(R + state_tile<D>(col, m, l));
  }
};

template <int D, bool BIDIR>
__global__ __launch_bounds__(64) void chunk_prefix(const float* __restrict__ w0,
                                                   long long w0_bstride, int H, int S,
                                                   const float* __restrict__ comp,
                                                   float* __restrict__ win) {
  constexpr int NT = D / 16;
  constexpr long long DD = (long long)D * D;
  const int bh = blockIdx.x, dir = blockIdx.y, col = blockIdx.z, b = bh / H, h = bh % H;
  const int BH = gridDim.x;
  const int l = threadIdx.x, r = l & 15, g = l >> 4;
  const int nrec = BIDIR ? 2 : 1;
  auto record = [&](int i) {  // map record of the i-th fold step
    const int s = dir == 0 ? i : S - 1 - i;
    return comp + (((long long)bh * S + s) * nrec + dir) * kMapFloats<D>;
  };

  const float* W0 = w0 + b * w0_bstride + h * DD;
  f32x4 W[NT];  // W[16m + 4g + j][16 col + r]
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j) W[m][j] = W0[(16 * m + 4 * g + j) * D + 16 * col + r];
  float* dst_base = win + ((long long)dir * BH + bh) * S * DD;
  const int steps = S - 1;  // maps applied: segments 0 .. S-2 in fold order
  PrefixOperands<D> set0, set1, set2, set3;
  set0.load(record(0), col, l);
  set1.load(record(min(1, S - 1)), col, l);
  set2.load(record(min(2, S - 1)), col, l);
  set3.load(record(min(3, S - 1)), col, l);
  auto store = [&](int i) {  // entry state of the i-th segment in fold order
    float* dst = dst_base + (dir == 0 ? i : S - 1 - i) * DD;
    for (int m = 0; m < NT; ++m) *reinterpret_cast<f32x4*>(dst + state_tile<D>(col, m, l)) = W[m];
  };
  auto step = [&](int i, PrefixOperands<D>& op) {  // applies map i, stores entry state i + 1
    f32x4 acc[NT];
    for (int m = 0; m < NT; ++m) acc[m] = W[m] + op.rr[m];
    for (int m = 0; m < NT; ++m) {
      if constexpr (D >= 32) {
        for (int ks = 0; ks < D / 32; ++ks) acc[m] = mma32(op.dev[m][ks], b_state(W, ks), acc[m]);
      } else {
        acc[m] = mma16(op.dev16, to_bf16x4(W[0]), acc[m]);
      }
    }
    for (int m = 0; m < NT; ++m) W[m] = acc[m];
    store(i + 1);
    // Unconditional (clamped to the last record, which exists) so that every step issues the
    // same memory operations and the compiler's waits stay kPrefixSets steps behind the loads.
    op.load(record(min(i + kPrefixSets, S - 1)), col, l);
  };
  store(0);
  int i = 0;
  for (; i + kPrefixSets <= steps; i += kPrefixSets) {
    step(i, set0);
    step(i + 1, set1);
    step(i + 2, set2);
    step(i + 3, set3);
  }
  if (i < steps) step(i, set0);
  if (i + 1 < steps) step(i + 1, set1);
  if (i + 2 < steps) step(i + 2, set2);
}

// ---------------------------------------------------------------- 3. segment scan
template <int D, int CH, int MODE>
__global__ __launch_bounds__(D / 16 * 64) void chunk_scan_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w0, long long w0_bstride, int H, int N, float a, int S, int L,
    const float* __restrict__ win, bf16* __restrict__ o, float* __restrict__ w_out) {
  constexpr int P = lds_pitch<D>();
  constexpr int NT = D / 16;   // waves = column tiles = row tiles
  constexpr int NP = CH / 16;  // 16-token tiles per chunk
  constexpr int NTH = NT * 64;
  constexpr long long DD = (long long)D * D;
  constexpr int LMAX = MODE == kBidir ? max_seg_len<D>() : 1;
  constexpr int WR_BYTES = MODE == kBidir ? LMAX * NT * NT * 64 * 8 : 8;
  // Chunk tiles (K, V, Q, O) are double-buffered when LDS allows (one barrier per chunk: chunk c
  // is staged while other waves may still read chunk c - 1, and chunk c - 1's O tile is written
  // out after chunk c's barrier); otherwise single buffers with three barriers per chunk.
  constexpr int NBUF = WR_BYTES + 2 * 4 * CH * P * 2 <= 160 * 1024 ? 2 : 1;
  __shared__ __align__(16) bf16 sKb[NBUF][CH * P];
  __shared__ __align__(16) bf16 sVb[NBUF][CH * P];
  __shared__ __align__(16) bf16 sQb[NBUF][CH * P];
  __shared__ __align__(16) bf16 sOb[NBUF][CH * P];
  __shared__ __align__(16) bf16x4 sWr[WR_BYTES / 8];

  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int BH = gridDim.y;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int C = N / CH;
  const int lo = s * L, hi = min(C, lo + L);
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;

  // Entry state of this segment (C layout): W0 for a single segment, else the prefix pass's
  // state tiles.
  auto entry = [&](int dir, f32x4* W) {
    if (S == 1) {
      const float* src = w0 + b * w0_bstride + h * DD;
      for (int m = 0; m < NT; ++m)
        for (int j = 0; j < 4; ++j) W[m][j] = src[(16 * m + 4 * g + j) * D + 16 * w + r];
    } else {
      const float* src = win + (((long long)dir * BH + bh) * S + s) * DD;
      for (int m = 0; m < NT; ++m) W[m] = *reinterpret_cast<const f32x4*>(src + state_tile<D>(w, m, l));
    }
  };
  // The entry state comes from global memory. Waiting for those loads here, once, keeps the
  // compiler's wait tracking from treating the state registers as possibly still in flight inside
  // the chunk loop, where it would otherwise wait for every outstanding load (the chunk prefetch
  // included) before each use of the state.
  auto entry_done = [] { __builtin_amdgcn_s_waitcnt(0); };
  auto save = [&](float* dst, const f32x4* W) {
    for (int m = 0; m < NT; ++m)
      for (int j = 0; j < 4; ++j) dst[(16 * m + 4 * g + j) * D + 16 * w + r] = W[m][j];
  };

  f32x4 W[NT];
  constexpr int G = stage_groups<CH>();
  const bf16* qb = q + head0;
  const bf16* kb = k + head0;
  const bf16* vb = v + head0;
  const long long cs = (long long)CH * ts;  // elements between consecutive chunks

  if constexpr (MODE == kBidir) {
    // Reverse scan over the segment's chunks (last to first), keeping each W^r_c in LDS.
    entry(1, W);
    entry_done();
    ChunkStager<D, CH, NTH, 2, G, P> sr(ts);
    const bf16* kn = kb + (hi - 1) * cs;  // chunk hi - 1 - j (j < G), then chunk c - G
    const bf16* vn = vb + (hi - 1) * cs;
    for (int j = 0; j < G; ++j, kn -= cs, vn -= cs)
      if (hi - 1 - j >= lo && sr.mine(j)) sr.load(kn, vn, nullptr);
    for (int c = hi - 1; c >= lo; --c, kn -= cs, vn -= cs) {
      const int buf = NBUF == 2 ? (hi - 1 - c) & 1 : 0;
      bf16* sK = sKb[buf];
      bf16* sV = sVb[buf];
      if (NBUF == 1) __syncthreads();
      if (sr.mine(hi - 1 - c)) {
        sr.store(sK, sV, nullptr);
        if (c - G >= lo) sr.load(kn, vn, nullptr);
      }
      __syncthreads();
      f32x4 E[NP];
      residuals<D, NP, P>(E, W, sK, sV, w, r, g, l);
      update_state<D, NP, P>(W, E, sK, a, l);
      for (int m = 0; m < NT; ++m) sWr[(((c - lo) * NT + w) * NT + m) * 64 + l] = to_bf16x4(W[m]);
    }
    if (s == 0 && w_out) save(w_out + (long long)BH * DD + bh * DD, W);
  }

  // Forward scan over the segment with the read-out. (For the bidirectional scan, the barrier
  // below orders the reverse pass's last tile reads before the first forward store.)
  if (MODE == kBidir) __syncthreads();
  entry(0, W);
  entry_done();
  ChunkStager<D, CH, NTH, 3, G, P> sf(ts);
  const bf16* kn = kb + lo * cs;  // chunk lo + j (j < G), then chunk c + G
  const bf16* vn = vb + lo * cs;
  const bf16* qn = qb + lo * cs;
  for (int j = 0; j < G; ++j, kn += cs, vn += cs, qn += cs)
    if (lo + j < hi && sf.mine(j)) sf.load(kn, vn, qn);
  for (int c = lo; c < hi; ++c, kn += cs, vn += cs, qn += cs) {
    const long long tok0 = head0 + (long long)c * CH * ts;
    const int buf = NBUF == 2 ? (c - lo) & 1 : 0;
    bf16* sK = sKb[buf];
    bf16* sV = sVb[buf];
    bf16* sQ = sQb[buf];
    bf16* sO = sOb[buf];
    if (NBUF == 1) __syncthreads();
    if (sf.mine(c - lo)) {
      sf.store(sK, sV, sQ);
      if (c + G < hi) sf.load(kn, vn, qn);
    }
    __syncthreads();
    if (NBUF == 2 && c > lo) store_chunk<D, CH, P, NTH>(o + tok0 - CH * ts, sOb[buf ^ 1], ts);

    f32x4 E[NP];
    residuals<D, NP, P>(E, W, sK, sV, w, r, g, l);

    if constexpr (MODE == kCausal) {
      // O_p = Q_p W_s - a * sum_{p' <= p} tril(P_{p p'}) E_{p'},  P = Q K^T, computed transposed
      // (lane (r, g) gets columns 16w + 4g.. of token 16p + r: one 8-byte store).
      for (int p = 0; p < NP; ++p) {
        // W_s^T Q_p^T and the masked term get separate accumulators: a 16x16x16 product must not
        // accumulate onto a 16x16x32 product's result (on gfx950 that chain read a stale value).
        const f32x4 qw = state_times_rows<D, P>(sQ, 16 * p, W, r, g);
        f32x4 acc = zero4();
        for (int pp = 0; pp <= p; ++pp) {
          // Pt[t' = 16pp + 4g + j][t = 16p + r] = k_t' . q_t
          f32x4 pt = zero4();
          if constexpr (D >= 32) {
            for (int ks = 0; ks < D / 32; ++ks)
              pt = mma32(cat8(ld4(&sK[(16 * pp + r) * P + 32 * ks + 4 * g]), ld4(&sK[(16 * pp + r) * P + 32 * ks + 16 + 4 * g])),
                         cat8(ld4(&sQ[(16 * p + r) * P + 32 * ks + 4 * g]), ld4(&sQ[(16 * p + r) * P + 32 * ks + 16 + 4 * g])), pt);
          } else {
            pt = mma16(ld4(&sK[(16 * pp + r) * P + 4 * g]), ld4(&sQ[(16 * p + r) * P + 4 * g]), pt);
          }
          if (pp == p)
            for (int j = 0; j < 4; ++j)
              if (4 * g + j > r) pt[j] = 0.f;
          // A = E_{p'}^T (row = column 16w + r, k = t' = 4g + j), B = -a P^T (k = t', n = t = r).
          acc = mma16(to_bf16x4(E[pp]), to_bf16x4_scaled(pt, -a), acc);
        }
        *reinterpret_cast<bf16x4*>(&sO[(16 * p + r) * P + 16 * w + 4 * g]) = to_bf16x4(qw + acc);
      }
      update_state<D, NP, P>(W, E, sK, a, l);
    } else {
      update_state<D, NP, P>(W, E, sK, a, l);
      f32x4 Ws[NT];
      for (int m = 0; m < NT; ++m) {
        const bf16x4 wr = sWr[(((c - lo) * NT + w) * NT + m) * 64 + l];
        for (int j = 0; j < 4; ++j) Ws[m][j] = W[m][j] + (float)wr[j];
      }
      for (int p = 0; p < NP; ++p)  // transposed: columns 16w + 4g.. of token 16p + r
        *reinterpret_cast<bf16x4*>(&sO[(16 * p + r) * P + 16 * w + 4 * g]) =
            to_bf16x4(state_times_rows<D, P>(sQ, 16 * p, Ws, r, g));
    }
    if (NBUF == 1) {
      __syncthreads();
      store_chunk<D, CH, P, NTH>(o + tok0, sO, ts);
    }
  }
  if (NBUF == 2) {  // the last chunk's O tile
    __syncthreads();
    store_chunk<D, CH, P, NTH>(o + head0 + (long long)(hi - 1) * CH * ts, sOb[(hi - 1 - lo) & 1], ts);
  }
  if (s == S - 1 && w_out) save(w_out + bh * DD, W);
}

// ---------------------------------------------------------------- fp32 I/O, plain FMA
// One workgroup per (b, h); the state lives in LDS and tokens are processed one by one in the
// primal form (weights of each token materialised), in true fp32. The reverse scan of the
// bidirectional variant stores its per-chunk states in the workspace.
enum F32Mode { kF32Causal = 0, kF32ReverseStore = 1, kF32ForwardBoth = 2 };

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
    const int c = (MODE == kF32ReverseStore) ? C - 1 - it : it;
    for (int e = tid; e < D * D; e += 256) sS[e / D][e % D] = 0.f;
    __syncthreads();
    for (int i = 0; i < CH; ++i) {
      const long long off = head0 + ((long long)c * CH + i) * ts;
      if (tid < D) {
        sk[tid] = k[off + tid];
        sq[tid] = (MODE == kF32ReverseStore) ? 0.f : q[off + tid];
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
      if (MODE == kF32Causal && tid < D) {  // o_i = q_i (W_s - a S_i)
        float acc = 0.f;
        for (int j = 0; j < D; ++j) acc = fmaf(sq[j], fmaf(-a, sS[j][tid], sW[j][tid]), acc);
        o[off + tid] = acc;
      }
      __syncthreads();
    }
    for (int e = tid; e < D * D; e += 256) sW[e / D][e % D] = fmaf(-a, sS[e / D][e % D], sW[e / D][e % D]);
    __syncthreads();
    if (MODE == kF32ReverseStore)
      for (int e = tid; e < D * D; e += 256) st_bh[c * dd + e] = sW[e / D][e % D];
    if (MODE == kF32ForwardBoth) {
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
    float* dst = w_out + (MODE == kF32ReverseStore ? (long long)gridDim.x * dd : 0) + bh * dd;
    for (int e = tid; e < D * D; e += 256) dst[e] = sW[e / D][e % D];
  }
}

// ---------------------------------------------------------------- planning and launch
struct ChunkPlan {
  int S, L;  // segments per (b, h) and chunks per segment
};

// Resident workgroups of the segment kernels. The compose and scan kernels walk their segment's
// chunks one after another (latency-bound), so the plan sizes the grid to be resident in one round:
// a partial second round would double their time. The plan is a pure function of the call's sizes
// and of fixed constants, never of the device the call runs on, so that the workspace size and the
// rounding path (the output bits) are the same everywhere:
//  - kPlanCUs: the 256 compute units of an MI355X (a device with fewer only runs the grid in more
//    rounds);
//  - the waves per SIMD each compiled kernel sustains on gfx950, the compiler's occupancy figure
//    (it accounts for the kernel's VGPR and LDS use), indexed [log2(D / 16)][log2(CH / 16)][bidir];
//    tests/test_codegen.py checks these tables against the compiler's resource report of the
//    current sources.
// A kernel of w waves per workgroup then keeps floor(4 * occupancy / w) workgroups on a CU (at most
// kMaxGroupsPerCU), and the plan takes the smaller figure of compose and scan.
constexpr int kPlanCUs = 256;
constexpr int kMaxGroupsPerCU = 16;
constexpr int kComposeOcc[3][3][2] = {{{8, 8}, {8, 8}, {7, 6}},   // D = 16: CH = 16, 32, 64
                                      {{8, 8}, {8, 8}, {7, 5}},   // D = 32
                                      {{8, 6}, {7, 5}, {6, 4}}};  // D = 64
constexpr int kScanOcc[3][3][2] = {{{7, 1}, {4, 1}, {2, 1}},
                                   {{7, 1}, {4, 1}, {2, 1}},
                                   {{5, 1}, {4, 1}, {2, 1}}};

constexpr int log2_16(int x) { return x == 16 ? 0 : (x == 32 ? 1 : 2); }

template <int D, int CH>
int groups_per_cu(bool bidir) {
  const int comp = 4 * kComposeOcc[log2_16(D)][log2_16(CH)][bidir] / (D / 8);
  const int scan = 4 * kScanOcc[log2_16(D)][log2_16(CH)][bidir] / (D / 16);
  const int n = comp < scan ? comp : scan;
  return n < 1 ? 1 : (n > kMaxGroupsPerCU ? kMaxGroupsPerCU : n);
}

template <int D, int CH>
ChunkPlan chunk_plan_dc(bool bidir, int B, int H, int N) {
  const int C = N / CH;
  const int BH = B * H;
  const int slots = kPlanCUs * groups_per_cu<D, CH>(bidir);  // workgroups resident at once
  int S = slots / BH;                       // segments per (b, h): one resident round
  if (S > C / 4) S = C / 4;                 // keep at least 4 chunks per segment
  if (S < 1) S = 1;
  int L = (C + S - 1) / S;
  if (bidir && L > max_seg_len<D>()) L = max_seg_len<D>();
  S = (C + L - 1) / L;
  return ChunkPlan{S, L};
}

template <int D>
ChunkPlan chunk_plan_d(bool bidir, int B, int H, int N, int CH) {
  switch (CH) {
    case 16: return chunk_plan_dc<D, 16>(bidir, B, H, N);
    case 32: return chunk_plan_dc<D, 32>(bidir, B, H, N);
    default: return chunk_plan_dc<D, 64>(bidir, B, H, N);
  }
}

ChunkPlan chunk_plan(bool bidir, int B, int H, int N, int D, int CH) {
  switch (D) {
    case 16: return chunk_plan_d<16>(bidir, B, H, N, CH);
    case 32: return chunk_plan_d<32>(bidir, B, H, N, CH);
    default: return chunk_plan_d<64>(bidir, B, H, N, CH);
  }
}

template <int D, int CH>
hipError_t launch_bf16(bool bidir, int B, int H, int N, float a, const void* q, const void* k,
                       const void* v, const float* w0, long long w0s, void* o, float* w_out,
                       void* ws, hipStream_t st) {
  const int BH = B * H;
  const ChunkPlan pl = chunk_plan(bidir, B, H, N, D, CH);
  const long long DD = (long long)D * D;
  float* comp = static_cast<float*>(ws);
  float* win = comp + (long long)BH * pl.S * (bidir ? 2 : 1) * kMapFloats<D>;
  if (pl.S > 1) {
    if (bidir) {
      hipLaunchKernelGGL((chunk_compose_bf16<D, CH, true>), dim3(pl.S, BH), dim3(D / 8 * 64), 0, st,
                         (const bf16*)k, (const bf16*)v, H, N, a, pl.S, pl.L, comp);
      hipLaunchKernelGGL((chunk_prefix<D, true>), dim3(BH, 2, D / 16), dim3(64), 0, st, w0, w0s, H,
                         pl.S, comp, win);
    } else {
      hipLaunchKernelGGL((chunk_compose_bf16<D, CH, false>), dim3(pl.S, BH), dim3(D / 8 * 64), 0,
                         st, (const bf16*)k, (const bf16*)v, H, N, a, pl.S, pl.L, comp);
      hipLaunchKernelGGL((chunk_prefix<D, false>), dim3(BH, 1, D / 16), dim3(64), 0, st, w0, w0s,
                         H, pl.S, comp, win);
    }
  }
  if (bidir) {
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kBidir>), dim3(pl.S, BH), dim3(D / 16 * 64), 0, st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, pl.S,
                       pl.L, win, (bf16*)o, w_out);
  } else {
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kCausal>), dim3(pl.S, BH), dim3(D / 16 * 64), 0,
                       st, (const bf16*)q, (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, pl.S,
                       pl.L, win, (bf16*)o, w_out);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(bool bidir, int B, int H, int N, int CH, float a, const void* q,
                      const void* k, const void* v, const float* w0, long long w0s, void* o,
                      float* w_out, void* ws, hipStream_t st) {
  const int BH = B * H;
  if (!bidir) {
    hipLaunchKernelGGL((chunk_scan_f32<D, kF32Causal>), dim3(BH), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, w0, w0s, H, N, CH, a,
                       nullptr, (float*)o, w_out);
  } else {
    float* states = static_cast<float*>(ws);
    hipLaunchKernelGGL((chunk_scan_f32<D, kF32ReverseStore>), dim3(BH), dim3(256), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, w0, w0s, H, N, CH, a,
                       states, (float*)o, w_out);
    hipLaunchKernelGGL((chunk_scan_f32<D, kF32ForwardBoth>), dim3(BH), dim3(256), 0, st,
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
  const size_t BH = (size_t)B * H, DD = (size_t)D * D;
  if (!bf16_io) {
    if (!bidir) return 0;
    // fp32 path: reverse-scan state after every chunk, C * D * D fp32 per (b, h)
    return BH * ((size_t)N / (size_t)chunk) * DD * sizeof(float);
  }
  const ChunkPlan pl = chunk_plan(bidir, B, H, N, D, chunk);
  if (pl.S == 1) return 0;
  // segment map records (-Dev bf16 + R fp32, per direction) + entry states per direction
  const size_t ndir = bidir ? 2 : 1;
  return BH * pl.S * ndir * (DD / 2 + DD) * sizeof(float) + BH * pl.S * ndir * DD * sizeof(float);
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
