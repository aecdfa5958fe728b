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

// ---------------------------------------------------------------- column order of a token grid
// The 2-D scan (Vision-TTT summary, "De Oplossing": the scanner also reads top to bottom) runs the
// bidirectional scan a second time over the tokens of a height x width grid in column order:
// position p' of that sequence is the raster token (p' mod height) * width + p' / height. The
// column-order kernels read and write the raster tensors in place through this map. ColPos follows
// one row of a chunk tile from chunk to chunk (p' moves by a fixed step, forward or back) with one
// conditional wrap and no division.
struct ColMap {
  int hg, wg;
};
struct ColPos {
  int i, j;  // grid row and column of the tracked token
  __device__ __forceinline__ void init(int pp, ColMap m) {
    pp = pp < 0 ? 0 : pp;
    j = pp / m.hg;
    i = pp - j * m.hg;
  }
  // p' += step (di = step mod hg, dj = step / hg), or p' -= step
  __device__ __forceinline__ void fwd(int di, int dj, ColMap m) {
    i += di;
    j += dj;
    if (i >= m.hg) {
      i -= m.hg;
      ++j;
    }
  }
  __device__ __forceinline__ void back(int di, int dj, ColMap m) {
    i -= di;
    j -= dj;
    if (i < 0) {
      i += m.hg;
      --j;
    }
  }
  __device__ __forceinline__ long long token(ColMap m) const { return (long long)i * m.wg + j; }
};

// ---------------------------------------------------------------- staging with prefetch
// The [CH x D] bf16 tiles of NTS tensors of one chunk move HBM -> registers -> LDS (row pitch P).
// The workgroup's threads form G groups; group j holds the chunks whose step index is j mod G: it
// loads a chunk G steps before the step that uses it and stores it to LDS at the start of that
// step, so each load has G steps to arrive with one register set per thread. A thread's 16-byte
// pieces sit at fixed offsets within a chunk tile, computed once; when a tile spans whole waves,
// the tensor of a piece is the same across the wave, and choosing its base pointer is scalar work.
// COLS: the tile rows come from the column map instead (ChunkStager::track, load_cols): each piece
// keeps its row's grid position for the next chunk its group loads.
template <int D, int CH, int NTH, int NTS, int G, int P, bool COLS = false>
struct ChunkStager {
  static_assert(NTH % G == 0 && NTS >= 1 && NTS <= 4, "staging geometry");
  static constexpr int CPR = D / 8;  // 16-byte pieces per row
  static constexpr int TILE = CH * CPR;
  static constexpr int PIECES = NTS * TILE;
  static constexpr int GT = NTH / G;  // threads per group
  static constexpr int PER = (PIECES + GT - 1) / GT;
  static constexpr bool kUniform = TILE % 64 == 0 && GT % 64 == 0;
  uint4 v[PER];
  int group;
  int sel[PER], goff[PER], loff[PER];
  ColPos pos[COLS ? PER : 1];  // COLS: grid position of the piece's row in the group's next chunk
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
  // COLS: start at chunk c of the column-order sequence (this thread's group's first load).
  __device__ __forceinline__ void track(int c, ColMap m) {
    for (int i = 0; i < PER; ++i) pos[i].init(c * CH + ((threadIdx.x % GT) + i * GT) % TILE / CPR, m);
  }
  // COLS: load the tracked chunk from the head base pointers t0 .. t3 (raster layout), then move
  // every piece G chunks on (dir > 0) or back (dir < 0).
  __device__ __forceinline__ void load_cols(const bf16* t0, const bf16* t1, const bf16* t2, const bf16* t3,
                                            ColMap m, long long ts, int dir) {
    const int di = (G * CH) % m.hg, dj = (G * CH) / m.hg;
    for (int i = 0; i < PER; ++i) {
      if (valid(i)) {
        const bf16* src = sel[i] == 0 ? t0 : (sel[i] == 1 ? t1 : (sel[i] == 2 ? t2 : t3));
        const int col = (((threadIdx.x % GT) + i * GT) % TILE % CPR) * 8;
        v[i] = ld16(src + pos[i].token(m) * ts + col);
      }
      if (dir > 0) pos[i].fwd(di, dj, m);
      else pos[i].back(di, dj, m);
    }
  }
  // t0 .. t3: the chunk's first row in each tensor (unused ones may be null).
  __device__ __forceinline__ void load(const bf16* t0, const bf16* t1, const bf16* t2,
                                       const bf16* t3 = nullptr) {
    for (int i = 0; i < PER; ++i)
      if (valid(i)) {
        const bf16* src = sel[i] == 0 ? t0 : (sel[i] == 1 ? t1 : (sel[i] == 2 ? t2 : t3));
        v[i] = ld16(src + goff[i]);
      }
  }
  __device__ __forceinline__ void store(bf16* d0, bf16* d1, bf16* d2, bf16* d3 = nullptr) const {
    for (int i = 0; i < PER; ++i)
      if (valid(i)) {
        bf16* dst = sel[i] == 0 ? d0 : (sel[i] == 1 ? d1 : (sel[i] == 2 ? d2 : d3));
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

// The O tile of a column-order chunk (bf16 in LDS, row pitch P) added into the raster output, which
// already holds the raster-order scan's result: o[token] = bf16(o[token] + tile), summed in fp32 and
// rounded once. Each thread tracks the rows of its pieces (tid, tid + NTH, ...) from chunk to chunk;
// the chunks are stored in order.
template <int D, int CH, int P, int NTH>
struct ColStore {
  static constexpr int CPR = D / 8, PIECES = CH * CPR, PER = (PIECES + NTH - 1) / NTH;
  ColPos pos[PER];
  __device__ __forceinline__ static bool valid(int k) { return PIECES % NTH == 0 || (int)threadIdx.x + k * NTH < PIECES; }
  __device__ __forceinline__ void track(int c, ColMap m) {
    for (int k = 0; k < PER; ++k) pos[k].init(c * CH + ((int)threadIdx.x + k * NTH) / CPR, m);
  }
  __device__ __forceinline__ void add(bf16* o_head, const bf16* src, long long ts, ColMap m) {
    const int di = CH % m.hg, dj = CH / m.hg;
    for (int k = 0; k < PER; ++k) {
      if (valid(k)) {
        const int c = threadIdx.x + k * NTH, row = c / CPR, col = (c % CPR) * 8;
        bf16* dst = o_head + pos[k].token(m) * ts + col;
        const bf16x8 a = ld8(dst);
        const bf16x8 b = __builtin_bit_cast(bf16x8, ld16_lds8(src + row * P + col));
        f32x4 lo, hi;
        for (int t = 0; t < 4; ++t) {
          lo[t] = (float)a[t] + (float)b[t];
          hi[t] = (float)a[4 + t] + (float)b[4 + t];
        }
        st16(dst, __builtin_bit_cast(uint4, cat8(to_bf16x4(lo), to_bf16x4(hi))));
      }
      pos[k].fwd(di, dj, m);
    }
  }
};

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
// Wave w owns column tile w of both halves of the state [P | R]: the P tile (from I, no V) and the
// R tile (from 0, with V). The two tiles share their operands of K (the rows for the residuals, the
// transpose reads for the update), so each wave reads the chunk's K tile from LDS once for both,
// and the workgroup has D / 16 waves.
template <int D, int CH, bool BIDIR, bool COLS = false>
__global__ __launch_bounds__(D / 16 * 64) void chunk_compose_bf16(
    const bf16* __restrict__ k, const bf16* __restrict__ v, int H, int N, float a, int S, int L,
    float* __restrict__ comp, ColMap cmap) {
  constexpr int P = lds_pitch<D>(), NT = D / 16, NP = CH / 16, NTH = NT * 64;
  constexpr long long DD = (long long)D * D;
  // Double-buffered chunk tiles: chunk c is staged while other waves may still read chunk c - 1,
  // so one barrier per chunk suffices.
  __shared__ __align__(16) bf16 sKb[2][CH * P];
  __shared__ __align__(16) bf16 sVb[2][CH * P];

  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int col = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int C = N / CH;
  const int lo = s * L, hi = min(C, lo + L);
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;

  f32x4 XP[NT], XR[NT], RR[NT];
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j) {
      XP[m][j] = 16 * m + 4 * g + j == 16 * col + r ? 1.f : 0.f;
      XR[m][j] = 0.f;
      RR[m][j] = 0.f;
    }

  constexpr int G = stage_groups<CH>();
  ChunkStager<D, CH, NTH, 2, G, P, COLS> st(ts);
  const long long cs = (long long)CH * ts;  // elements between consecutive chunks
  const bf16* kn = k + head0 + lo * cs;     // chunk lo + j (j < G), then chunk c + G
  const bf16* vn = v + head0 + lo * cs;
  if constexpr (COLS) st.track(lo + st.group, cmap);
  auto load_next = [&]() {
    if constexpr (COLS) st.load_cols(k + head0, v + head0, nullptr, nullptr, cmap, ts, 1);
    else st.load(kn, vn, nullptr);
  };
  for (int j = 0; j < G; ++j, kn += cs, vn += cs)
    if (lo + j < hi && st.mine(j)) load_next();
  for (int c = lo; c < hi; ++c, kn += cs, vn += cs) {
    bf16* sK = sKb[(c - lo) & 1];
    bf16* sV = sVb[(c - lo) & 1];
    if (st.mine(c - lo)) {
      st.store(sK, sV, nullptr);
      if (c + G < hi) load_next();
    }
    __syncthreads();
    // Residuals of both tiles: YP_p = K_p P, YR_p = K_p R - V_p[:, 16 col ..].
    f32x4 YP[NP], YR[NP];
    for (int p = 0; p < NP; ++p) {
      const bf16x4 vt = tile_tr(&sV[16 * p * P + 16 * col], P, l);  // V tile, accumulator layout
      f32x4 yp = zero4(), yr;
      for (int j = 0; j < 4; ++j) yr[j] = -(float)vt[j];
      if constexpr (D >= 32) {
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16* pk = sK + (16 * p + r) * P + 32 * ks + 4 * g;
          const bf16x8 ka = cat8(ld4(pk), ld4(pk + 16));
          yp = mma32(ka, b_state(XP, ks), yp);
          yr = mma32(ka, b_state(XR, ks), yr);
        }
      } else {
        const bf16x4 ka = ld4(sK + (16 * p + r) * P + 4 * g);
        yp = mma16(ka, to_bf16x4(XP[0]), yp);
        yr = mma16(ka, to_bf16x4(XR[0]), yr);
      }
      YP[p] = yp;
      YR[p] = yr;
    }
    if constexpr (BIDIR) {  // R_rev[16col + i][16n + .] += a (K_c P_{c-1})^T V_c
      if constexpr (NP == 1) {
        const bf16x4 ya = to_bf16x4_scaled(YP[0], a);
        for (int n = 0; n < NT; ++n) RR[n] = mma16(ya, tile_tr(&sV[16 * n], P, l), RR[n]);
      } else {  // 32 tokens per product, k map {4g + j} u {16 + 4g + j}
        for (int p = 0; p < NP; p += 2) {
          const bf16x8 ya = cat8(to_bf16x4_scaled(YP[p], a), to_bf16x4_scaled(YP[p + 1], a));
          for (int n = 0; n < NT; ++n)
            RR[n] = mma32(ya, cat8(tile_tr(&sV[16 * p * P + 16 * n], P, l),
                                   tile_tr(&sV[16 * (p + 1) * P + 16 * n], P, l)), RR[n]);
        }
      }
    }
    // [P | R] += K^T (-a [YP | YR]): the transpose reads of K serve both tiles.
    if constexpr (NP == 1) {
      const bf16x4 ep = to_bf16x4_scaled(YP[0], -a), er = to_bf16x4_scaled(YR[0], -a);
      for (int m = 0; m < NT; ++m) {
        const bf16x4 kt = tile_tr(&sK[16 * m], P, l);
        XP[m] = mma16(kt, ep, XP[m]);
        XR[m] = mma16(kt, er, XR[m]);
      }
    } else {
      for (int p = 0; p < NP; p += 2) {
        const bf16x8 ep = cat8(to_bf16x4_scaled(YP[p], -a), to_bf16x4_scaled(YP[p + 1], -a));
        const bf16x8 er = cat8(to_bf16x4_scaled(YR[p], -a), to_bf16x4_scaled(YR[p + 1], -a));
        for (int m = 0; m < NT; ++m) {
          const bf16x8 kt = cat8(tile_tr(&sK[16 * p * P + 16 * m], P, l), tile_tr(&sK[16 * (p + 1) * P + 16 * m], P, l));
          XP[m] = mma32(kt, ep, XP[m]);
          XR[m] = mma32(kt, er, XR[m]);
        }
      }
    }
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
      const bf16 nd = (bf16)(XP[m][j] - (row == cc ? 1.f : 0.f));  // -Dev = P - I
      ndev_f[dev_offset<D>(row, cc)] = nd;
      if constexpr (BIDIR) ndev_r[dev_offset<D>(cc, row)] = nd;  // Dev_r = Dev_f^T
    }
  for (int m = 0; m < NT; ++m) *reinterpret_cast<f32x4*>(r_f + state_tile<D>(col, m, l)) = XR[m];
  if constexpr (BIDIR)  // RR[n] is R_rev's tile (column tile n, row tile col)
    for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(r_r + state_tile<D>(n, col, l)) = RR[n];
}

// ---------------------------------------------------------------- 2. prefix over segments
// The columns of W are independent regressions, so the fold over the segment maps,
// W[:, cols] <- W[:, cols] + (-Dev) W[:, cols] + R[:, cols], runs as one single-wave workgroup
// per (b, h, record slot, 16-column tile), storing each segment's entry state. A segment carries
// NREC map records: even slots are folded first segment to last, odd slots last to first; slots
// below n_init start from W0, the others from zero (the backward pass folds its adjoint maps,
// which start from a zero gradient, beside the forward maps). Its speed is the
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

template <int D, int NREC>
__global__ __launch_bounds__(64) void chunk_prefix(const float* __restrict__ w0,
                                                   long long w0_bstride, int n_init, int H, int S,
                                                   const float* __restrict__ comp,
                                                   float* __restrict__ win) {
  constexpr int NT = D / 16;
  constexpr long long DD = (long long)D * D;
  const int bh = blockIdx.x, slot = blockIdx.y, col = blockIdx.z, b = bh / H, h = bh % H;
  const int BH = gridDim.x;
  const int l = threadIdx.x, r = l & 15, g = l >> 4;
  const bool rev = slot & 1;
  auto record = [&](int i) {  // map record of the i-th fold step
    const int s = rev ? S - 1 - i : i;
    return comp + (((long long)bh * S + s) * NREC + slot) * kMapFloats<D>;
  };

  const float* W0 = w0 + b * w0_bstride + h * DD;
  f32x4 W[NT];  // W[16m + 4g + j][16 col + r]
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j)
      W[m][j] = slot < n_init ? W0[(16 * m + 4 * g + j) * D + 16 * col + r] : 0.f;
  float* dst_base = win + ((long long)slot * BH + bh) * S * DD;
  const int steps = S - 1;  // maps applied: segments 0 .. S-2 in fold order
  PrefixOperands<D> set0, set1, set2, set3;
  set0.load(record(0), col, l);
  set1.load(record(min(1, S - 1)), col, l);
  set2.load(record(min(2, S - 1)), col, l);
  set3.load(record(min(3, S - 1)), col, l);
  auto store = [&](int i) {  // entry state of the i-th segment in fold order
    float* dst = dst_base + (rev ? S - 1 - i : i) * DD;
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
template <int D, int CH, int MODE, bool COLS = false>
__global__ __launch_bounds__(D / 16 * 64) void chunk_scan_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w0, long long w0_bstride, int H, int N, float a, int S, int L,
    const float* __restrict__ win, bf16* __restrict__ o, float* __restrict__ w_out, ColMap cmap) {
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
    ChunkStager<D, CH, NTH, 2, G, P, COLS> sr(ts);
    const bf16* kn = kb + (hi - 1) * cs;  // chunk hi - 1 - j (j < G), then chunk c - G
    const bf16* vn = vb + (hi - 1) * cs;
    if constexpr (COLS) sr.track(hi - 1 - sr.group, cmap);
    auto load_next = [&]() {
      if constexpr (COLS) sr.load_cols(kb, vb, nullptr, nullptr, cmap, ts, -1);
      else sr.load(kn, vn, nullptr);
    };
    for (int j = 0; j < G; ++j, kn -= cs, vn -= cs)
      if (hi - 1 - j >= lo && sr.mine(j)) load_next();
    for (int c = hi - 1; c >= lo; --c, kn -= cs, vn -= cs) {
      const int buf = NBUF == 2 ? (hi - 1 - c) & 1 : 0;
      bf16* sK = sKb[buf];
      bf16* sV = sVb[buf];
      if (NBUF == 1) __syncthreads();
      if (sr.mine(hi - 1 - c)) {
        sr.store(sK, sV, nullptr);
        if (c - G >= lo) load_next();
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
  ChunkStager<D, CH, NTH, 3, G, P, COLS> sf(ts);
  const bf16* kn = kb + lo * cs;  // chunk lo + j (j < G), then chunk c + G
  const bf16* vn = vb + lo * cs;
  const bf16* qn = qb + lo * cs;
  if constexpr (COLS) sf.track(lo + sf.group, cmap);
  ColStore<D, CH, P, NTH> ost;  // COLS: the O tiles' rows (chunks lo, lo + 1, ...)
  if constexpr (COLS) ost.track(lo, cmap);
  auto load_next = [&]() {
    if constexpr (COLS) sf.load_cols(kb, vb, qb, nullptr, cmap, ts, 1);
    else sf.load(kn, vn, qn);
  };
  for (int j = 0; j < G; ++j, kn += cs, vn += cs, qn += cs)
    if (lo + j < hi && sf.mine(j)) load_next();
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
      if (c + G < hi) load_next();
    }
    __syncthreads();
    if (NBUF == 2 && c > lo) {
      if constexpr (COLS) ost.add(o + head0, sOb[buf ^ 1], ts, cmap);
      else store_chunk<D, CH, P, NTH>(o + tok0 - CH * ts, sOb[buf ^ 1], ts);
    }

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
      if constexpr (COLS) ost.add(o + head0, sO, ts, cmap);
      else store_chunk<D, CH, P, NTH>(o + tok0, sO, ts);
    }
  }
  if (NBUF == 2) {  // the last chunk's O tile
    __syncthreads();
    if constexpr (COLS) ost.add(o + head0, sOb[(hi - 1 - lo) & 1], ts, cmap);
    else store_chunk<D, CH, P, NTH>(o + head0 + (long long)(hi - 1) * CH * ts, sOb[(hi - 1 - lo) & 1], ts);
  }
  if (s == S - 1 && w_out) save(w_out + bh * DD, W);
}

// ---------------------------------------------------------------- fp32 I/O, plain FMA
// The fp32 path takes the same decomposition as the bf16 kernels (the plan's segments, composed
// maps stored as -Dev = P - I and R, the prefix fold, per-segment rescans with the dual-form causal
// read-out), in fp32 FMA with workgroup-wide loops over LDS tiles, so that the fp32 parity bound
// checks that algebra itself. Records hold -Dev and R in fp32 (kF32MapFloats per direction).
template <int D>
constexpr int kF32MapFloats = 2 * D * D;
constexpr int kF32Threads = 256;

// Y[t][j] = sum_k X[t][k] M[k][j] - (Vt ? Vt[t][j] : 0) for t < rows (LDS tiles, row pitch D + 1).
template <int D>
__device__ __forceinline__ void f32_rows_times(float* Y, const float* X, const float* M, const float* Vt,
                                               int rows) {
  constexpr int DP = D + 1;
  for (int e = threadIdx.x; e < rows * D; e += kF32Threads) {
    const int t = e / D, j = e % D;
    float acc = Vt ? -Vt[t * DP + j] : 0.f;
    for (int k = 0; k < D; ++k) acc = fmaf(X[t * DP + k], M[k * DP + j], acc);
    Y[t * DP + j] = acc;
  }
}

// M[i][j] += s sum_t X[t][i] Y[t][j] over t < rows.
template <int D>
__device__ __forceinline__ void f32_add_xt_y(float* M, const float* X, const float* Y, float s, int rows) {
  constexpr int DP = D + 1;
  for (int e = threadIdx.x; e < D * D; e += kF32Threads) {
    const int i = e / D, j = e % D;
    float acc = 0.f;
    for (int t = 0; t < rows; ++t) acc = fmaf(X[t * DP + i], Y[t * DP + j], acc);
    M[i * DP + j] = fmaf(s, acc, M[i * DP + j]);
  }
}

template <int D>
__device__ __forceinline__ void f32_load_rows(float* dst, const float* src, long long ts, int rows) {
  constexpr int DP = D + 1;
  for (int e = threadIdx.x; e < rows * D; e += kF32Threads) dst[(e / D) * DP + e % D] = src[(e / D) * ts + e % D];
}

// 1. compose: the segment's forward map W -> P W + R (and, bidirectional, the reversed scan's
// offset R_rev = a sum_c (K_c P_{c-1})^T V_c), from P = I, R = 0.
template <int D, bool BIDIR>
__global__ __launch_bounds__(kF32Threads) void chunk_compose_f32(const float* __restrict__ k,
                                                                 const float* __restrict__ v, int H,
                                                                 int N, int CH, float a, int S, int L,
                                                                 float* __restrict__ comp) {
  constexpr int DP = D + 1;
  __shared__ float sK[64 * DP], sV[64 * DP], sY[64 * DP], sYR[64 * DP];
  __shared__ float sP[D * DP], sR[D * DP], sRR[BIDIR ? D * DP : 1];
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int C = N / CH, lo = s * L, hi = min(C, lo + L);
  const long long ts = (long long)H * D, head0 = (long long)b * N * ts + (long long)h * D;
  for (int e = tid; e < D * D; e += kF32Threads) {
    sP[(e / D) * DP + e % D] = (e / D == e % D) ? 1.f : 0.f;
    sR[(e / D) * DP + e % D] = 0.f;
    if (BIDIR) sRR[(e / D) * DP + e % D] = 0.f;
  }
  for (int c = lo; c < hi; ++c) {
    __syncthreads();
    f32_load_rows<D>(sK, k + head0 + (long long)c * CH * ts, ts, CH);
    f32_load_rows<D>(sV, v + head0 + (long long)c * CH * ts, ts, CH);
    __syncthreads();
    f32_rows_times<D>(sY, sK, sP, nullptr, CH);  // K P
    f32_rows_times<D>(sYR, sK, sR, sV, CH);      // K R - V
    __syncthreads();
    if (BIDIR) f32_add_xt_y<D>(sRR, sY, sV, a, CH);
    f32_add_xt_y<D>(sP, sK, sY, -a, CH);
    f32_add_xt_y<D>(sR, sK, sYR, -a, CH);
  }
  __syncthreads();
  float* rec = comp + ((long long)bh * S + s) * (BIDIR ? 2 : 1) * kF32MapFloats<D>;
  for (int e = tid; e < D * D; e += kF32Threads) {
    const int i = e / D, j = e % D;
    const float nd = sP[i * DP + j] - (i == j ? 1.f : 0.f);  // -Dev = P - I
    rec[e] = nd;
    rec[D * D + e] = sR[i * DP + j];
    if (BIDIR) {
      rec[kF32MapFloats<D> + j * D + i] = nd;  // -Dev_r = -Dev^T
      rec[kF32MapFloats<D> + D * D + e] = sRR[i * DP + j];
    }
  }
}

// 2. prefix: per (b, h, direction), W <- W + (-Dev) W + R over the segments in fold order
// (reversed for direction 1), storing every segment's entry state.
template <int D, bool BIDIR>
__global__ __launch_bounds__(kF32Threads) void chunk_prefix_f32(const float* __restrict__ w0,
                                                                long long w0_bstride, int H, int S,
                                                                const float* __restrict__ comp,
                                                                float* __restrict__ win) {
  constexpr int DP = D + 1;
  __shared__ float sW[D * DP], sT[D * DP];
  const int bh = blockIdx.x, dir = blockIdx.y, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int BH = gridDim.x;
  const long long DD = (long long)D * D;
  const float* W0 = w0 + b * w0_bstride + h * DD;
  for (int e = tid; e < D * D; e += kF32Threads) sW[(e / D) * DP + e % D] = W0[e];
  float* dst = win + ((long long)dir * BH + bh) * S * DD;
  for (int i = 0; i < S; ++i) {
    const int sg = dir == 0 ? i : S - 1 - i;
    __syncthreads();
    for (int e = tid; e < D * D; e += kF32Threads) dst[sg * DD + e] = sW[(e / D) * DP + e % D];
    if (i == S - 1) break;
    const float* rec = comp + ((long long)bh * S + sg) * (BIDIR ? 2 : 1) * kF32MapFloats<D> + dir * kF32MapFloats<D>;
    for (int e = tid; e < D * D; e += kF32Threads) {
      const int r = e / D, c = e % D;
      float acc = rec[D * D + e];
      for (int k2 = 0; k2 < D; ++k2) acc = fmaf(rec[r * D + k2], sW[k2 * DP + c], acc);
      sT[r * DP + c] = acc;
    }
    __syncthreads();
    for (int e = tid; e < D * D; e += kF32Threads) sW[(e / D) * DP + e % D] += sT[(e / D) * DP + e % D];
  }
}

// 3. scan: per (segment, b, h), from the segment's entry state. Causal: O = Q W - a tril(Q K^T) E,
// W <- W - a K^T E. Bidirectional: the reversed scan over the segment stores each W^r_c in
// `rstates`, then the forward scan reads out O = Q (W^f_c + W^r_c).
template <int D, int MODE>
__global__ __launch_bounds__(kF32Threads) void chunk_scan_dual_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ w0, long long w0_bstride, int H, int N, int CH, float a, int S, int L,
    const float* __restrict__ win, float* __restrict__ rstates, float* __restrict__ o,
    float* __restrict__ w_out) {
  constexpr int DP = D + 1;
  __shared__ float sK[64 * DP], sV[64 * DP], sQ[64 * DP], sE[64 * DP];
  __shared__ float sW[D * DP], sS[64 * 65];
  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int BH = gridDim.y;
  const int C = N / CH, lo = s * L, hi = min(C, lo + L);
  const long long ts = (long long)H * D, head0 = (long long)b * N * ts + (long long)h * D;
  const long long DD = (long long)D * D;
  auto entry = [&](int dir) {
    const float* src = S == 1 ? w0 + b * w0_bstride + h * DD : win + (((long long)dir * BH + bh) * S + s) * DD;
    for (int e = tid; e < D * D; e += kF32Threads) sW[(e / D) * DP + e % D] = src[e];
  };
  auto step = [&](int c, bool with_q) {  // stage chunk c, E = K W - V, W <- W - a K^T E (after use)
    __syncthreads();
    f32_load_rows<D>(sK, k + head0 + (long long)c * CH * ts, ts, CH);
    f32_load_rows<D>(sV, v + head0 + (long long)c * CH * ts, ts, CH);
    if (with_q) f32_load_rows<D>(sQ, q + head0 + (long long)c * CH * ts, ts, CH);
    __syncthreads();
    f32_rows_times<D>(sE, sK, sW, sV, CH);
    __syncthreads();
  };
  float* rs_bh = MODE == kBidir ? rstates + (long long)bh * C * DD : nullptr;
  if (MODE == kBidir) {
    entry(1);
    for (int c = hi - 1; c >= lo; --c) {
      step(c, false);
      f32_add_xt_y<D>(sW, sK, sE, -a, CH);
      __syncthreads();
      for (int e = tid; e < D * D; e += kF32Threads) rs_bh[c * DD + e] = sW[(e / D) * DP + e % D];
    }
    __syncthreads();
    if (s == 0 && w_out)
      for (int e = tid; e < D * D; e += kF32Threads) w_out[(long long)BH * DD + bh * DD + e] = sW[(e / D) * DP + e % D];
  }
  entry(0);
  for (int c = lo; c < hi; ++c) {
    step(c, true);
    float* oc = o + head0 + (long long)c * CH * ts;
    if (MODE == kCausal) {
      for (int e = tid; e < CH * CH; e += kF32Threads) {  // S = tril(Q K^T)
        const int t = e / CH, u = e % CH;
        float acc = 0.f;
        if (u <= t)
          for (int kk = 0; kk < D; ++kk) acc = fmaf(sQ[t * DP + kk], sK[u * DP + kk], acc);
        sS[t * 65 + u] = acc;
      }
      __syncthreads();
      for (int e = tid; e < CH * D; e += kF32Threads) {  // O = Q W - a S E
        const int t = e / D, j = e % D;
        float qw = 0.f, se = 0.f;
        for (int kk = 0; kk < D; ++kk) qw = fmaf(sQ[t * DP + kk], sW[kk * DP + j], qw);
        for (int u = 0; u <= t; ++u) se = fmaf(sS[t * 65 + u], sE[u * DP + j], se);
        oc[t * ts + j] = fmaf(-a, se, qw);
      }
      __syncthreads();
      f32_add_xt_y<D>(sW, sK, sE, -a, CH);
    } else {
      f32_add_xt_y<D>(sW, sK, sE, -a, CH);
      __syncthreads();
      for (int e = tid; e < CH * D; e += kF32Threads) {  // O = Q (W^f_c + W^r_c)
        const int t = e / D, j = e % D;
        float acc = 0.f;
        for (int kk = 0; kk < D; ++kk) acc = fmaf(sQ[t * DP + kk], sW[kk * DP + j] + rs_bh[c * DD + kk * D + j], acc);
        oc[t * ts + j] = acc;
      }
    }
  }
  __syncthreads();
  if (s == S - 1 && w_out)
    for (int e = tid; e < D * D; e += kF32Threads) w_out[bh * DD + e] = sW[(e / D) * DP + e % D];
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
// kMaxGroupsPerCU), and the plan takes the smaller figure of compose and scan, and at most
// kPlanWavesPerCU waves of them per CU. Compose and scan are walks of dependent chunk steps whose
// CU throughput (chunk steps per us) stays about flat above three 4-wave workgroups per CU, while
// every extra segment adds a step to the prefix fold: for the causal layer of 2 x 16384 x 12 heads
// (d = 64, b = 16) S = 41 segments (4 workgroups per CU) measured 82.4 us cold and S = 32 (3 per CU)
// 76.4 us, and a sweep of S from 16 to 41 put 28-32 best.
constexpr int kPlanCUs = 256;
constexpr int kMaxGroupsPerCU = 16;
constexpr int kPlanWavesPerCU = 12;
constexpr int kComposeOcc[3][3][2] = {{{8, 8}, {7, 6}, {4, 4}},   // D = 16: CH = 16, 32, 64
                                      {{7, 5}, {5, 4}, {4, 3}},   // D = 32
                                      {{4, 4}, {4, 3}, {3, 2}}};  // D = 64
constexpr int kScanOcc[3][3][2] = {{{7, 1}, {4, 1}, {2, 1}},
                                   {{7, 1}, {4, 1}, {2, 1}},
                                   {{5, 1}, {4, 1}, {2, 1}}};

constexpr int log2_16(int x) { return x == 16 ? 0 : (x == 32 ? 1 : 2); }

template <int D, int CH>
int groups_per_cu(bool bidir) {
  const int comp = 4 * kComposeOcc[log2_16(D)][log2_16(CH)][bidir] / (D / 16);
  const int scan = 4 * kScanOcc[log2_16(D)][log2_16(CH)][bidir] / (D / 16);
  int n = comp < scan ? comp : scan;
  if (n > kPlanWavesPerCU / (D / 16)) n = kPlanWavesPerCU / (D / 16);
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

// cols: the bidirectional scan over the column order of a token grid, added into o (null: raster order).
template <int D, int CH>
hipError_t launch_bf16(bool bidir, int B, int H, int N, float a, const void* q, const void* k,
                       const void* v, const float* w0, long long w0s, void* o, float* w_out,
                       void* ws, hipStream_t st, const ColMap* cols) {
  const int BH = B * H;
  const ChunkPlan pl = chunk_plan(bidir, B, H, N, D, CH);
  const long long DD = (long long)D * D;
  float* comp = static_cast<float*>(ws);
  float* win = comp + (long long)BH * pl.S * (bidir ? 2 : 1) * kMapFloats<D>;
  const ColMap cm = cols ? *cols : ColMap{1, 1};
  if (pl.S > 1) {
    if (bidir) {
      if (cols)
        hipLaunchKernelGGL((chunk_compose_bf16<D, CH, true, true>), dim3(pl.S, BH), dim3(D / 16 * 64), 0, st,
                           (const bf16*)k, (const bf16*)v, H, N, a, pl.S, pl.L, comp, cm);
      else
        hipLaunchKernelGGL((chunk_compose_bf16<D, CH, true>), dim3(pl.S, BH), dim3(D / 16 * 64), 0, st,
                           (const bf16*)k, (const bf16*)v, H, N, a, pl.S, pl.L, comp, cm);
      hipLaunchKernelGGL((chunk_prefix<D, 2>), dim3(BH, 2, D / 16), dim3(64), 0, st, w0, w0s, 2, H,
                         pl.S, comp, win);
    } else {
      hipLaunchKernelGGL((chunk_compose_bf16<D, CH, false>), dim3(pl.S, BH), dim3(D / 16 * 64), 0,
                         st, (const bf16*)k, (const bf16*)v, H, N, a, pl.S, pl.L, comp, cm);
      hipLaunchKernelGGL((chunk_prefix<D, 1>), dim3(BH, 1, D / 16), dim3(64), 0, st, w0, w0s, 1,
                         H, pl.S, comp, win);
    }
  }
  if (bidir && cols) {
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kBidir, true>), dim3(pl.S, BH), dim3(D / 16 * 64), 0, st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, pl.S,
                       pl.L, win, (bf16*)o, w_out, cm);
  } else if (bidir) {
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kBidir>), dim3(pl.S, BH), dim3(D / 16 * 64), 0, st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, pl.S,
                       pl.L, win, (bf16*)o, w_out, cm);
  } else {
    hipLaunchKernelGGL((chunk_scan_bf16<D, CH, kCausal>), dim3(pl.S, BH), dim3(D / 16 * 64), 0,
                       st, (const bf16*)q, (const bf16*)k, (const bf16*)v, w0, w0s, H, N, a, pl.S,
                       pl.L, win, (bf16*)o, w_out, cm);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(bool bidir, int B, int H, int N, int CH, float a, const void* q,
                      const void* k, const void* v, const float* w0, long long w0s, void* o,
                      float* w_out, void* ws, hipStream_t st) {
  const int BH = B * H;
  const ChunkPlan pl = chunk_plan(bidir, B, H, N, D, CH);
  const long long DD = (long long)D * D;
  const int ndir = bidir ? 2 : 1;
  float* comp = static_cast<float*>(ws);
  float* win = comp + (pl.S > 1 ? (long long)BH * pl.S * ndir * kF32MapFloats<D> : 0);
  float* rstates = win + (pl.S > 1 ? (long long)ndir * BH * pl.S * DD : 0);
  const float *Q = (const float*)q, *K = (const float*)k, *V = (const float*)v;
  if (pl.S > 1) {
    if (bidir) {
      hipLaunchKernelGGL((chunk_compose_f32<D, true>), dim3(pl.S, BH), dim3(kF32Threads), 0, st, K, V, H, N, CH, a,
                         pl.S, pl.L, comp);
      hipLaunchKernelGGL((chunk_prefix_f32<D, true>), dim3(BH, 2), dim3(kF32Threads), 0, st, w0, w0s, H, pl.S,
                         comp, win);
    } else {
      hipLaunchKernelGGL((chunk_compose_f32<D, false>), dim3(pl.S, BH), dim3(kF32Threads), 0, st, K, V, H, N, CH,
                         a, pl.S, pl.L, comp);
      hipLaunchKernelGGL((chunk_prefix_f32<D, false>), dim3(BH, 1), dim3(kF32Threads), 0, st, w0, w0s, H, pl.S,
                         comp, win);
    }
  }
  if (bidir)
    hipLaunchKernelGGL((chunk_scan_dual_f32<D, kBidir>), dim3(pl.S, BH), dim3(kF32Threads), 0, st, Q, K, V, w0,
                       w0s, H, N, CH, a, pl.S, pl.L, win, rstates, (float*)o, w_out);
  else
    hipLaunchKernelGGL((chunk_scan_dual_f32<D, kCausal>), dim3(pl.S, BH), dim3(kF32Threads), 0, st, Q, K, V, w0,
                       w0s, H, N, CH, a, pl.S, pl.L, win, rstates, (float*)o, w_out);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(bool bidir, int B, int H, int N, int CH, float a, const void* q,
                         const void* k, const void* v, const float* w0, long long w0s, void* o,
                         float* w_out, void* ws, hipStream_t st, const ColMap* cols = nullptr) {
  switch (CH) {
    case 16: return launch_bf16<D, 16>(bidir, B, H, N, a, q, k, v, w0, w0s, o, w_out, ws, st, cols);
    case 32: return launch_bf16<D, 32>(bidir, B, H, N, a, q, k, v, w0, w0s, o, w_out, ws, st, cols);
    case 64: return launch_bf16<D, 64>(bidir, B, H, N, a, q, k, v, w0, w0s, o, w_out, ws, st, cols);
    default: return hipErrorInvalidValue;
  }
}

// ================================================================ backward (outer-loop gradients)
// Gradients of the chunked layers for the outer training loop (the pages' authors write the inner
// gradient by hand rather than by autograd: ViT^3 review, section on the official code; the outer
// gradient here is derived in the same closed-form style). One scan direction, chunk c in the
// scan's order with start state W (= W_{c-1}), a = eta/b, E = K W - V and the read-out
//   O = Q W - a (M o Q K^T) E,   M = tril (causal) or all ones (read-out after the chunk's update,
//                                    i.e. O = Q W_c with W_c = W - a K^T E),
// and lam = dL/dW_c from the chunks after c (zero after the last). Then
//   dE = -a (S^T dO + K lam),  S = M o (Q K^T)      dS = -a M o (dO E^T)
//   dQ = dO W^T + dS K        dK = dE W^T + dS^T Q - a E lam^T        dV = -dE
//   dL/dW_{c-1} = lam + Q^T dO + K^T dE.
// For the read-out after the update the same reads, with lam' = lam + Q^T dO:
//   dE = -a K lam',  dQ = dO W_c^T,  dK = dE W^T - a E lam'^T,  dL/dW_{c-1} = lam' + K^T dE.
// The adjoint step lam -> A_c lam + U_c is affine with the forward map's linear part A_c =
// I - a K^T K (symmetric), so a segment's adjoint map is the forward composite transposed plus an
// offset, and the prefix fold carries the adjoints beside the forward states:
//   1. chunk_compose_bwd: per (segment, b, h), the forward map (as in the forward pass) and the
//      adjoint offsets: for a forward-ordered scan U = sum_c P_{c-1}^T U_c (P_{c-1} the forward
//      composite before chunk c; U_c = (Q_c - a S_c K_c)^T dO_c, which is (Q_c A_c)^T dO_c for the
//      all-ones mask); for the reversed scan of the bidirectional layer, whose adjoint runs over
//      the chunks in forward order, mu <- A_c (mu + Q_c^T dO_c).
//   2. chunk_prefix over the records: forward entry states and adjoints at every segment's end.
//   3. chunk_bwd_scan: per (segment, b, h), the forward states over the segment into an LDS ring
//      (bf16, the operand precision), then the chunks in reverse scan order with the formulas
//      above. The bidirectional layer runs it once per direction: the reversed scan writes fp32
//      partial gradients, the forward scan adds them before rounding.

// Record slots of the backward (a segment's maps): causal: 0 forward map, 1 adjoint map;
// bidirectional: 0 forward, 1 reversed-scan forward, 2 reversed-scan adjoint, 3 forward adjoint.
// Even slots are folded first segment to last, odd slots last to first.

// Y^T[16 cols x 16 rows] = W[:, col0..col0+15]^T X_rows^T with W a row-major bf16 tile in LDS
// (row pitch PW): lane (r, g) gets sum_k W[k][col0 + 4g + j] X[row0 + r][k]. The A operand (W's
// columns) comes from LDS transpose reads.
template <int D, int P, int PW>
__device__ __forceinline__ f32x4 ldsstate_times_rows(const bf16* Wl, int col0, const bf16* X,
                                                     int row0, f32x4 acc, int r, int g, int l) {
  if constexpr (D >= 32) {
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16* p = X + (row0 + r) * P + 32 * ks + 4 * g;
      acc = mma32(cat8(tile_tr(&Wl[(32 * ks) * PW + col0], PW, l), tile_tr(&Wl[(32 * ks + 16) * PW + col0], PW, l)),
                  cat8(ld4(p), ld4(p + 16)), acc);
    }
  } else {
    acc = mma16(tile_tr(&Wl[col0], PW, l), ld4(X + (row0 + r) * P + 4 * g), acc);
  }
  return acc;
}

// C[16 x 16] += A_rows(arow0..) . B_rows(brow0..)^T, contraction over the D features: lane (r, g)
// gets sum_k A[arow0 + 4g + j][k] B[brow0 + r][k] (A and B row-major bf16 in LDS).
template <int D, int PA, int PB>
__device__ __forceinline__ f32x4 rows_dot_rows(const bf16* A, int arow0, const bf16* Bm, int brow0,
                                               f32x4 acc, int r, int g) {
  if constexpr (D >= 32) {
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16* pa = A + (arow0 + r) * PA + 32 * ks + 4 * g;
      const bf16* pb = Bm + (brow0 + r) * PB + 32 * ks + 4 * g;
      acc = mma32(cat8(ld4(pa), ld4(pa + 16)), cat8(ld4(pb), ld4(pb + 16)), acc);
    }
  } else {
    acc = mma16(ld4(A + (arow0 + r) * PA + 4 * g), ld4(Bm + (brow0 + r) * PB + 4 * g), acc);
  }
  return acc;
}

// X[:, 16col..] += A^T B[:, 16col..] over the chunk's tokens, A and B [CH x D] tiles in LDS (A^T
// and B both by transpose reads). 16-token chunks use 16x16x16 products, longer ones 16x16x32
// (the same shapes as update_state, so the two may accumulate into the same registers).
template <int D, int NP, int P>
__device__ __forceinline__ void add_at_b(f32x4* X, const bf16* A, const bf16* Bm, int col, int l) {
  if constexpr (NP == 1) {
    const bf16x4 bt = tile_tr(&Bm[16 * col], P, l);
    for (int m = 0; m < D / 16; ++m) X[m] = mma16(tile_tr(&A[16 * m], P, l), bt, X[m]);
  } else {
    for (int p = 0; p < NP; p += 2) {
      const bf16x8 bt = cat8(tile_tr(&Bm[16 * p * P + 16 * col], P, l), tile_tr(&Bm[16 * (p + 1) * P + 16 * col], P, l));
      for (int m = 0; m < D / 16; ++m)
        X[m] = mma32(cat8(tile_tr(&A[16 * p * P + 16 * m], P, l), tile_tr(&A[16 * (p + 1) * P + 16 * m], P, l)), bt, X[m]);
    }
  }
}

// Acc[n] (row tile col, column tile n) += Z^T B[:, 16n..], Z the [CH x 16] C-layout tiles of one
// wave (rows = tokens), B a [CH x D] LDS tile: the R_rev accumulation pattern of the compose.
template <int D, int NP, int P>
__device__ __forceinline__ void add_zt_b(f32x4* Acc, const f32x4* Z, const bf16* Bm, float scale,
                                         int l) {
  if constexpr (NP == 1) {
    const bf16x4 za = to_bf16x4_scaled(Z[0], scale);
    for (int n = 0; n < D / 16; ++n) Acc[n] = mma16(za, tile_tr(&Bm[16 * n], P, l), Acc[n]);
  } else {
    for (int p = 0; p < NP; p += 2) {
      const bf16x8 za = cat8(to_bf16x4_scaled(Z[p], scale), to_bf16x4_scaled(Z[p + 1], scale));
      for (int n = 0; n < D / 16; ++n)
        Acc[n] = mma32(za, cat8(tile_tr(&Bm[16 * p * P + 16 * n], P, l), tile_tr(&Bm[16 * (p + 1) * P + 16 * n], P, l)), Acc[n]);
    }
  }
}

// ---------------------------------------------------------------- B1. compose (backward)
// Waves: role 0 holds P columns [16col, 16col + 16) (from I) and accumulates row tile col of the
// forward scan's adjoint offset (and, bidirectional, of R_rev); role 1 holds R columns (from 0);
// role 2 (bidirectional) holds columns of the reversed scan's adjoint offset.
template <int D, int CH, bool BIDIR>
__global__ __launch_bounds__((BIDIR ? 3 : 2) * (D / 16) * 64) void chunk_compose_bwd_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ d_o, int H, int N, float a, int S, int L, float* __restrict__ comp) {
  constexpr int P = lds_pitch<D>(), NT = D / 16, NP = CH / 16, NTH = (BIDIR ? 3 : 2) * NT * 64;
  constexpr int NREC = BIDIR ? 4 : 2;
  constexpr long long DD = (long long)D * D;
  __shared__ __align__(16) bf16 sKb[2][CH * P];
  __shared__ __align__(16) bf16 sVb[2][CH * P];
  __shared__ __align__(16) bf16 sQb[2][CH * P];
  __shared__ __align__(16) bf16 sDb[2][CH * P];

  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int role = w / NT, col = w % NT;
  const int C = N / CH;
  const int lo = s * L, hi = min(C, lo + L);
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;

  f32x4 X[NT], RR[NT], UT[NT];
  for (int m = 0; m < NT; ++m)
    for (int j = 0; j < 4; ++j) {
      X[m][j] = (role == 0 && 16 * m + 4 * g + j == 16 * col + r) ? 1.f : 0.f;
      RR[m][j] = 0.f;
      UT[m][j] = 0.f;
    }

  constexpr int G = stage_groups<CH>();
  ChunkStager<D, CH, NTH, 4, G, P> st(ts);
  const long long cs = (long long)CH * ts;
  const bf16* kn = k + head0 + lo * cs;
  const bf16* vn = v + head0 + lo * cs;
  const bf16* qn = q + head0 + lo * cs;
  const bf16* dn = d_o + head0 + lo * cs;
  for (int j = 0; j < G; ++j, kn += cs, vn += cs, qn += cs, dn += cs)
    if (lo + j < hi && st.mine(j)) st.load(kn, vn, qn, dn);
  for (int c = lo; c < hi; ++c, kn += cs, vn += cs, qn += cs, dn += cs) {
    bf16* sK = sKb[(c - lo) & 1];
    bf16* sV = sVb[(c - lo) & 1];
    bf16* sQ = sQb[(c - lo) & 1];
    bf16* sD = sDb[(c - lo) & 1];
    if (st.mine(c - lo)) {
      st.store(sK, sV, sQ, sD);
      if (c + G < hi) st.load(kn, vn, qn, dn);
    }
    __syncthreads();
    f32x4 Y[NP];
    if (role == 0) {
      residuals<D, NP, P>(Y, X, sK, sV, -1, r, g, l);  // K_c P_{c-1}
      f32x4 Z[NP];
      if constexpr (!BIDIR) {
        // Z = Q_c P_{c-1} - a tril(Q_c K_c^T) K_c P_{c-1}
        for (int p = 0; p < NP; ++p) {
          const f32x4 zq = rows_times_state<D, P>(sQ, 16 * p, X, zero4(), r, g);
          f32x4 acc = zero4();
          for (int pp = 0; pp <= p; ++pp) {
            // pt[t' = 16pp + 4g + j][t = 16p + r] = k_t' . q_t: the A operand S[t][t']
            f32x4 pt = rows_dot_rows<D, P, P>(sK, 16 * pp, sQ, 16 * p, zero4(), r, g);
            if (pp == p)
              for (int j = 0; j < 4; ++j)
                if (4 * g + j > r) pt[j] = 0.f;
            acc = mma16(to_bf16x4_scaled(pt, -a), to_bf16x4(Y[pp]), acc);
          }
          Z[p] = zq + acc;
        }
        add_zt_b<D, NP, P>(UT, Z, sD, 1.f, l);
        update_state<D, NP, P>(X, Y, sK, a, l);
      } else {
        add_zt_b<D, NP, P>(RR, Y, sV, a, l);  // R_rev += a (K_c P_{c-1})^T V_c
        update_state<D, NP, P>(X, Y, sK, a, l);
        for (int p = 0; p < NP; ++p) Z[p] = rows_times_state<D, P>(sQ, 16 * p, X, zero4(), r, g);
        add_zt_b<D, NP, P>(UT, Z, sD, 1.f, l);  // U += (Q_c P_c)^T dO_c
      }
    } else if (role == 1) {
      residuals<D, NP, P>(Y, X, sK, sV, col, r, g, l);
      update_state<D, NP, P>(X, Y, sK, a, l);
    } else {  // mu <- A_c (mu + Q_c^T dO_c)
      add_at_b<D, NP, P>(X, sQ, sD, col, l);
      residuals<D, NP, P>(Y, X, sK, sV, -1, r, g, l);
      update_state<D, NP, P>(X, Y, sK, a, l);
    }
  }

  float* rec = comp + ((long long)bh * S + s) * NREC * kMapFloats<D>;
  auto ndev = [&](int slot) { return reinterpret_cast<bf16*>(rec + slot * kMapFloats<D>); };
  auto roff = [&](int slot) { return rec + slot * kMapFloats<D> + DD / 2; };
  if (role == 0) {
    for (int m = 0; m < NT; ++m)
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * m + 4 * g + j, cc = 16 * col + r;
        const bf16 nd = (bf16)(X[m][j] - (row == cc ? 1.f : 0.f));  // -Dev = P - I
        ndev(0)[dev_offset<D>(row, cc)] = nd;
        ndev(1)[dev_offset<D>(cc, row)] = nd;
        if constexpr (BIDIR) {
          ndev(2)[dev_offset<D>(row, cc)] = nd;
          ndev(3)[dev_offset<D>(cc, row)] = nd;
        }
      }
    // UT[n] / RR[n]: tile (column tile n, row tile col) of the offsets
    for (int n = 0; n < NT; ++n)
      *reinterpret_cast<f32x4*>(roff(BIDIR ? 3 : 1) + state_tile<D>(n, col, l)) = UT[n];
    if constexpr (BIDIR)
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(roff(1) + state_tile<D>(n, col, l)) = RR[n];
  } else {
    float* dst = roff(role == 1 ? 0 : 2);
    for (int m = 0; m < NT; ++m) *reinterpret_cast<f32x4*>(dst + state_tile<D>(col, m, l)) = X[m];
  }
}

// ---------------------------------------------------------------- B3. segment scan (backward)
// LDS of the backward scan: five [CH x D] tiles (K; V, then E; Q; dO; dE), -a lam (row-major) and
// two row-major state tiles (this chunk's start state and the next chunk's, which is this chunk's
// end state). The segment's forward states go to a per-segment ring in the workspace as bf16
// accumulator-layout tiles: each wave writes its own columns in the states pass and reads back
// only what it wrote, so the ring needs no cross-wave ordering; segments are as long as the plan
// wants, with no LDS bound.
template <int D>
constexpr long long kRingState = (long long)D * D;  // bf16 elements per state in the ring

// Output modes: write bf16; write fp32 partials (reversed scan of the bidirectional layer); add the
// partials and write bf16 (its forward scan, launched after).
enum BwdOut { kOutBf16 = 0, kOutPartial = 1, kOutAddPartial = 2 };

template <int D, int CH, bool CAUSAL>
__global__ __launch_bounds__(D / 16 * 64) void chunk_bwd_scan_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ d_o, const float* __restrict__ w0, long long w0_bstride, int H, int N,
    float a, int S, int L, const float* __restrict__ win, bf16* __restrict__ wring, int dir,
    int fwd_slot, int adj_slot, int out_mode, float* __restrict__ part, bf16* __restrict__ dq,
    bf16* __restrict__ dk, bf16* __restrict__ dv, float* __restrict__ d_w0) {
  constexpr int P = lds_pitch<D>(), PW = P;
  constexpr int NT = D / 16, NP = CH / 16, NTH = NT * 64;
  constexpr long long DD = (long long)D * D;
  __shared__ __align__(16) bf16 sK[CH * P];
  __shared__ __align__(16) bf16 sV[CH * P];  // V in the states pass, E in the gradient pass
  __shared__ __align__(16) bf16 sQ[CH * P];
  __shared__ __align__(16) bf16 sD[CH * P];
  __shared__ __align__(16) bf16 sDE[CH * P];
  __shared__ __align__(16) bf16 sL[D * PW];
  __shared__ __align__(16) bf16 sW[2][D * PW];
  bf16* const sE = sV;

  const int s = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int BH = gridDim.y;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int C = N / CH;
  const int lo = s * L, hi = min(C, lo + L), n = hi - lo;
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;
  const long long cs = (long long)CH * ts;
  // chunk at scan position pos of this segment
  auto chunk_at = [&](int pos) { return dir == 0 ? lo + pos : hi - 1 - pos; };
  const long long step = dir == 0 ? cs : -cs;  // pointer step to the next scan position

  auto entry = [&](int slot, f32x4* X) {
    if (S == 1) {
      const float* src = w0 + b * w0_bstride + h * DD;
      for (int m = 0; m < NT; ++m)
        for (int j = 0; j < 4; ++j) X[m][j] = slot == fwd_slot ? src[(16 * m + 4 * g + j) * D + 16 * w + r] : 0.f;
    } else {
      const float* src = win + (((long long)slot * BH + bh) * S + s) * DD;
      for (int m = 0; m < NT; ++m) X[m] = *reinterpret_cast<const f32x4*>(src + state_tile<D>(w, m, l));
    }
  };
  auto put_state = [&](bf16* dst, const f32x4* X, float scale) {  // row-major bf16, this wave's columns
    for (int m = 0; m < NT; ++m)
      for (int j = 0; j < 4; ++j) dst[(16 * m + 4 * g + j) * PW + 16 * w + r] = (bf16)(X[m][j] * scale);
  };
  // The segment's ring: state pos at ring_seg + pos * D * D, tile (wave w, row tile m) lane by lane.
  bf16* const ring_seg = wring + ((long long)bh * S + s) * (L + 1) * kRingState<D>;
  auto ring_put = [&](int pos, const f32x4* X) {
    for (int m = 0; m < NT; ++m)
      *reinterpret_cast<bf16x4*>(ring_seg + pos * kRingState<D> + ((w * NT + m) * 64 + l) * 4) = to_bf16x4(X[m]);
  };
  auto ring_get = [&](int pos, bf16x4* T) {
    for (int m = 0; m < NT; ++m)
      T[m] = *reinterpret_cast<const bf16x4*>(ring_seg + pos * kRingState<D> + ((w * NT + m) * 64 + l) * 4);
  };
  auto put_tiles = [&](bf16* dst, const bf16x4* T) {  // row-major, this wave's columns
    for (int m = 0; m < NT; ++m)
      for (int j = 0; j < 4; ++j) dst[(16 * m + 4 * g + j) * PW + 16 * w + r] = T[m][j];
  };
  constexpr int G = stage_groups<CH>();

  // ---- states pass: the segment's chunks in scan order from its entry state
  f32x4 W[NT];
  entry(fwd_slot, W);
  __builtin_amdgcn_s_waitcnt(0);
  {
    ChunkStager<D, CH, NTH, 2, G, P> sa(ts);
    const bf16* kn = k + head0 + chunk_at(0) * cs;
    const bf16* vn = v + head0 + chunk_at(0) * cs;
    for (int j = 0; j < G; ++j, kn += step, vn += step)
      if (j < n && sa.mine(j)) sa.load(kn, vn, nullptr);
    for (int pos = 0; pos < n; ++pos, kn += step, vn += step) {
      __syncthreads();
      if (sa.mine(pos)) {
        sa.store(sK, sV, nullptr);
        if (pos + G < n) sa.load(kn, vn, nullptr);
      }
      __syncthreads();
      ring_put(pos, W);
      f32x4 E[NP];
      residuals<D, NP, P>(E, W, sK, sV, w, r, g, l);
      update_state<D, NP, P>(W, E, sK, a, l);
    }
    if (!CAUSAL) ring_put(n, W);
  }

  // ---- gradient pass: the chunks in reverse scan order
  f32x4 lam[NT];
  entry(adj_slot, lam);
  __builtin_amdgcn_s_waitcnt(0);
  ChunkStager<D, CH, NTH, 4, G, P> sb(ts);
  const bf16* kn = k + head0 + chunk_at(n - 1) * cs;
  const bf16* vn = v + head0 + chunk_at(n - 1) * cs;
  const bf16* qn = q + head0 + chunk_at(n - 1) * cs;
  const bf16* dn = d_o + head0 + chunk_at(n - 1) * cs;
  for (int j = 0; j < G; ++j, kn -= step, vn -= step, qn -= step, dn -= step)
    if (j < n && sb.mine(j)) sb.load(kn, vn, qn, dn);
  // State tiles: sW[it & 1] holds this chunk's start state; the other buffer, the previous
  // iteration's start state, is this chunk's end state (read-out after the update). Each wave
  // fetches its own ring tiles one chunk ahead.
  bf16x4 wt[NT];
  if (!CAUSAL) {
    ring_get(n, wt);
    put_tiles(sW[1], wt);
  }
  ring_get(n - 1, wt);
  for (int it = 0; it < n; ++it, kn -= step, vn -= step, qn -= step, dn -= step) {
    const int pos = n - 1 - it;
    const long long tok0 = head0 + (long long)chunk_at(pos) * cs;
    bf16* const Wp = sW[it & 1];
    const bf16* const Wn = CAUSAL ? Wp : sW[(it + 1) & 1];
    // V is staged into the E tile's buffer; each lane reads its own V values from there before
    // overwriting them with E (same rows and columns).
    __syncthreads();
    if (sb.mine(it)) {
      sb.store(sK, sV, sQ, sD);
      if (it + G < n) sb.load(kn, vn, qn, dn);
    }
    put_tiles(Wp, wt);
    if (pos > 0) ring_get(pos - 1, wt);
    __syncthreads();

    // E^T and dE^T for this wave's 16 features: lane (r, g) holds features 16w + 4g + j of token
    // 16p + r.
    f32x4 Et[NP], dEt[NP];
    for (int p = 0; p < NP; ++p) {
      const bf16x4 vv = ld4(&sV[(16 * p + r) * P + 16 * w + 4 * g]);
      f32x4 init;
      for (int j = 0; j < 4; ++j) init[j] = -(float)vv[j];
      Et[p] = ldsstate_times_rows<D, P, PW>(Wp, 16 * w, sK, 16 * p, init, r, g, l);
    }
    if (!CAUSAL) add_at_b<D, NP, P>(lam, sQ, sD, w, l);  // lam' = lam + Q^T dO
    for (int p = 0; p < NP; ++p) {
      const f32x4 kl = state_times_rows<D, P>(sK, 16 * p, lam, r, g);
      f32x4 sd = zero4();
      if constexpr (CAUSAL) {
        // sum over t >= t' of S[t][t'] dO[t][col]: A = dO^T (tile pp), B[t][t'] = q_t . k_t'
        for (int pp = p; pp < NP; ++pp) {
          f32x4 st = rows_dot_rows<D, P, P>(sQ, 16 * pp, sK, 16 * p, zero4(), r, g);
          if (pp == p)
            for (int j = 0; j < 4; ++j)
              if (r > 4 * g + j) st[j] = 0.f;
          sd = mma16(tile_tr(&sD[16 * pp * P + 16 * w], P, l), to_bf16x4(st), sd);
        }
      }
      dEt[p] = (kl + sd) * (-a);
    }
    for (int p = 0; p < NP; ++p) {
      *reinterpret_cast<bf16x4*>(&sE[(16 * p + r) * P + 16 * w + 4 * g]) = to_bf16x4(Et[p]);
      *reinterpret_cast<bf16x4*>(&sDE[(16 * p + r) * P + 16 * w + 4 * g]) = to_bf16x4(dEt[p]);
    }
    put_state(sL, lam, -a);
    __syncthreads();

    // Gradients of this wave's 16 features of every token, transposed (lane (r, g): features
    // 16w + 4g + j of token 16p + r).
    for (int p = 0; p < NP; ++p) {
      f32x4 gq = rows_dot_rows<D, PW, P>(Wn, 16 * w, sD, 16 * p, zero4(), r, g);
      f32x4 gk = rows_dot_rows<D, PW, P>(Wp, 16 * w, sDE, 16 * p, zero4(), r, g);
      gk = rows_dot_rows<D, PW, P>(sL, 16 * w, sE, 16 * p, gk, r, g);
      if constexpr (CAUSAL) {
        f32x4 cq = zero4(), ck = zero4();
        for (int pp = 0; pp <= p; ++pp) {  // dQ += dS K: B[t'][t] = -a E_t' . dO_t, t' <= t
          f32x4 et = rows_dot_rows<D, P, P>(sE, 16 * pp, sD, 16 * p, zero4(), r, g);
          if (pp == p)
            for (int j = 0; j < 4; ++j)
              if (4 * g + j > r) et[j] = 0.f;
          cq = mma16(tile_tr(&sK[16 * pp * P + 16 * w], P, l), to_bf16x4_scaled(et, -a), cq);
        }
        for (int pp = p; pp < NP; ++pp) {  // dK += dS^T Q: B[t][t'] = -a dO_t . E_t', t' <= t
          f32x4 de = rows_dot_rows<D, P, P>(sD, 16 * pp, sE, 16 * p, zero4(), r, g);
          if (pp == p)
            for (int j = 0; j < 4; ++j)
              if (r > 4 * g + j) de[j] = 0.f;
          ck = mma16(tile_tr(&sQ[16 * pp * P + 16 * w], P, l), to_bf16x4_scaled(de, -a), ck);
        }
        gq += cq;
        gk += ck;
      }
      const f32x4 gv = -dEt[p];
      const long long off = tok0 + (long long)(16 * p + r) * ts + 16 * w + 4 * g;
      if (out_mode == kOutPartial) {
        const long long act = (long long)gridDim.y / H * N * ts;  // elements of one [B, N, H, D] tensor
        *reinterpret_cast<f32x4*>(part + off) = gq;
        *reinterpret_cast<f32x4*>(part + act + off) = gk;
        *reinterpret_cast<f32x4*>(part + 2 * act + off) = gv;
      } else {
        f32x4 oq = gq, ok = gk, ov = gv;
        if (out_mode == kOutAddPartial) {
          const long long act = (long long)gridDim.y / H * N * ts;
          oq += *reinterpret_cast<const f32x4*>(part + off);
          ok += *reinterpret_cast<const f32x4*>(part + act + off);
          ov += *reinterpret_cast<const f32x4*>(part + 2 * act + off);
        }
        *reinterpret_cast<bf16x4*>(dq + off) = to_bf16x4(oq);
        *reinterpret_cast<bf16x4*>(dk + off) = to_bf16x4(ok);
        *reinterpret_cast<bf16x4*>(dv + off) = to_bf16x4(ov);
      }
    }
    if (CAUSAL) add_at_b<D, NP, P>(lam, sQ, sD, w, l);
    add_at_b<D, NP, P>(lam, sK, sDE, w, l);
  }
  // The segment holding the scan's first chunk ends the adjoint: dL/dW0 of this direction.
  if (s == (dir == 0 ? 0 : S - 1)) {
    float* dst = d_w0 + (long long)bh * DD;
    for (int m = 0; m < NT; ++m)
      for (int j = 0; j < 4; ++j) {
        float* e = dst + (16 * m + 4 * g + j) * D + 16 * w + r;
        *e = out_mode == kOutAddPartial ? *e + lam[m][j] : lam[m][j];
      }
  }
}

// ---------------------------------------------------------------- backward, fp32 I/O, plain FMA
// One workgroup per (b, h) and scan direction pass; the states of the scan (C + 1 of them) go to
// the workspace, the gradient pass reads them back. Same algebra as the bf16 kernels, in fp32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void chunk_bwd_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ d_o, const float* __restrict__ w0, long long w0_bstride, int H,
    int N, int CH, float a, int dir, float* __restrict__ states, bool accumulate,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ d_w0) {
  constexpr int DP = D + 1;
  __shared__ float sW[D * DP], sLam[D * DP];
  __shared__ float sK[64 * DP], sQ[64 * DP], sD[64 * DP], sE[64 * DP], sDE[64 * DP];
  __shared__ float sS[64 * 65];
  const int bh = blockIdx.x, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int C = N / CH;
  const long long ts = (long long)H * D, dd = (long long)D * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;
  float* st = states + (long long)bh * (C + 1) * dd;
  auto chunk_at = [&](int pos) { return dir == 0 ? pos : C - 1 - pos; };
  auto load_tile = [&](float* dst, const float* src, int c) {
    for (int e = tid; e < CH * D; e += 256) dst[(e / D) * DP + e % D] = src[head0 + ((long long)c * CH + e / D) * ts + e % D];
  };
  const float* W0 = w0 + b * w0_bstride + h * dd;
  for (int e = tid; e < D * D; e += 256) sW[(e / D) * DP + e % D] = W0[e];
  __syncthreads();
  // states pass
  for (int pos = 0; pos < C; ++pos) {
    const int c = chunk_at(pos);
    for (int e = tid; e < D * D; e += 256) st[pos * dd + e] = sW[(e / D) * DP + e % D];
    load_tile(sK, k, c);
    __syncthreads();
    for (int e = tid; e < CH * D; e += 256) {  // E = K W - V
      const int t = e / D, j = e % D;
      float acc = -v[head0 + ((long long)c * CH + t) * ts + j];
      for (int kk = 0; kk < D; ++kk) acc = fmaf(sK[t * DP + kk], sW[kk * DP + j], acc);
      sE[t * DP + j] = acc;
    }
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) {  // W -= a K^T E
      const int i = e / D, j = e % D;
      float acc = 0.f;
      for (int t = 0; t < CH; ++t) acc = fmaf(sK[t * DP + i], sE[t * DP + j], acc);
      sW[i * DP + j] = fmaf(-a, acc, sW[i * DP + j]);
    }
    __syncthreads();
  }
  for (int e = tid; e < D * D; e += 256) {
    st[C * dd + e] = sW[(e / D) * DP + e % D];
    sLam[(e / D) * DP + e % D] = 0.f;
  }
  __syncthreads();
  // gradient pass
  for (int pos = C - 1; pos >= 0; --pos) {
    const int c = chunk_at(pos);
    const float* Wp = st + pos * dd;
    const float* Wn = st + (CAUSAL ? pos : pos + 1) * dd;
    load_tile(sK, k, c);
    load_tile(sQ, q, c);
    load_tile(sD, d_o, c);
    for (int e = tid; e < D * D; e += 256) sW[(e / D) * DP + e % D] = Wp[e];
    __syncthreads();
    for (int e = tid; e < CH * D; e += 256) {  // E = K W - V
      const int t = e / D, j = e % D;
      float acc = -v[head0 + ((long long)c * CH + t) * ts + j];
      for (int kk = 0; kk < D; ++kk) acc = fmaf(sK[t * DP + kk], sW[kk * DP + j], acc);
      sE[t * DP + j] = acc;
    }
    for (int e = tid; e < CH * CH; e += 256) {  // S[t][t'] = q_t . k_t' (masked below)
      const int t = e / CH, u = e % CH;
      float acc = 0.f;
      for (int kk = 0; kk < D; ++kk) acc = fmaf(sQ[t * DP + kk], sK[u * DP + kk], acc);
      sS[t * 65 + u] = acc;
    }
    if (!CAUSAL) {
      for (int e = tid; e < D * D; e += 256) {  // lam' = lam + Q^T dO
        const int i = e / D, j = e % D;
        float acc = sLam[i * DP + j];
        for (int t = 0; t < CH; ++t) acc = fmaf(sQ[t * DP + i], sD[t * DP + j], acc);
        sLam[i * DP + j] = acc;
      }
    }
    __syncthreads();
    for (int e = tid; e < CH * D; e += 256) {  // dE = -a (S^T dO + K lam)
      const int t = e / D, j = e % D;
      float acc = 0.f;
      for (int kk = 0; kk < D; ++kk) acc = fmaf(sK[t * DP + kk], sLam[kk * DP + j], acc);
      if (CAUSAL)
        for (int u = t; u < CH; ++u) acc = fmaf(sS[u * 65 + t], sD[u * DP + j], acc);
      sDE[t * DP + j] = -a * acc;
    }
    __syncthreads();
    if (CAUSAL) {
      for (int e = tid; e < CH * CH; e += 256) {  // dS[t][t'] = -a dO_t . E_t', t' <= t
        const int t = e / CH, u = e % CH;
        float acc = 0.f;
        if (u <= t)
          for (int kk = 0; kk < D; ++kk) acc = fmaf(sD[t * DP + kk], sE[u * DP + kk], acc);
        sS[t * 65 + u] = -a * acc;
      }
      __syncthreads();
    }
    for (int e = tid; e < CH * D; e += 256) {
      const int t = e / D, i = e % D;
      const long long off = head0 + ((long long)c * CH + t) * ts + i;
      float gq = 0.f, gk = 0.f;
      for (int j = 0; j < D; ++j) {
        gq = fmaf(sD[t * DP + j], Wn[i * D + j], gq);
        gk = fmaf(sDE[t * DP + j], sW[i * DP + j], gk);
        gk = fmaf(-a * sE[t * DP + j], sLam[i * DP + j], gk);
      }
      if (CAUSAL) {
        for (int u = 0; u <= t; ++u) gq = fmaf(sS[t * 65 + u], sK[u * DP + i], gq);
        for (int u = t; u < CH; ++u) gk = fmaf(sS[u * 65 + t], sQ[u * DP + i], gk);
      }
      const float gv = -sDE[t * DP + i];
      dq[off] = accumulate ? dq[off] + gq : gq;
      dk[off] = accumulate ? dk[off] + gk : gk;
      dv[off] = accumulate ? dv[off] + gv : gv;
    }
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) {  // lam <- lam (+ Q^T dO) + K^T dE
      const int i = e / D, j = e % D;
      float acc = sLam[i * DP + j];
      for (int t = 0; t < CH; ++t) {
        if (CAUSAL) acc = fmaf(sQ[t * DP + i], sD[t * DP + j], acc);
        acc = fmaf(sK[t * DP + i], sDE[t * DP + j], acc);
      }
      sLam[i * DP + j] = acc;
    }
    __syncthreads();
  }
  float* dst = d_w0 + (long long)bh * dd;
  for (int e = tid; e < D * D; e += 256) dst[e] = accumulate ? dst[e] + sLam[(e / D) * DP + e % D] : sLam[(e / D) * DP + e % D];
}

// ---------------------------------------------------------------- backward planning and launch
struct BwdPlan {
  int S, L;
};

// Segments as for the forward scans: the grid resident in one round (two workgroups of the segment
// scan per CU: its LDS and registers allow two at d = 64), at least 4 chunks per segment.
constexpr int kBwdGroupsPerCU = 2;

BwdPlan bwd_plan(int B, int H, int N, int CH) {
  const int C = N / CH;
  const int BH = B * H;
  int S = kPlanCUs * kBwdGroupsPerCU / BH;
  if (S > C / 4) S = C / 4;
  if (S < 1) S = 1;
  const int L = (C + S - 1) / S;
  S = (C + L - 1) / L;
  return BwdPlan{S, L};
}

template <int D, int CH>
hipError_t launch_bwd_bf16(bool bidir, int B, int H, int N, float a, const void* q, const void* k,
                           const void* v, const float* w0, long long w0s, const void* d_o,
                           void* dq, void* dk, void* dv, float* d_w0, void* ws, hipStream_t st) {
  const int BH = B * H;
  const BwdPlan pl = bwd_plan(B, H, N, CH);
  const int nrec = bidir ? 4 : 2;
  const long long DD = (long long)D * D;
  float* comp = static_cast<float*>(ws);
  float* win = comp + (pl.S > 1 ? (long long)BH * pl.S * nrec * kMapFloats<D> : 0);
  bf16* wring = reinterpret_cast<bf16*>(win + (pl.S > 1 ? (long long)nrec * BH * pl.S * DD : 0));
  float* part = reinterpret_cast<float*>(wring + (long long)BH * pl.S * (pl.L + 1) * kRingState<D>);
  const bf16 *Q = (const bf16*)q, *K = (const bf16*)k, *V = (const bf16*)v, *DO = (const bf16*)d_o;
  bf16 *GQ = (bf16*)dq, *GK = (bf16*)dk, *GV = (bf16*)dv;
  const dim3 grid(pl.S, BH), block(D / 16 * 64);
  if (!bidir) {
    if (pl.S > 1) {
      hipLaunchKernelGGL((chunk_compose_bwd_bf16<D, CH, false>), dim3(pl.S, BH), dim3(2 * D / 16 * 64), 0,
                         st, Q, K, V, DO, H, N, a, pl.S, pl.L, comp);
      hipLaunchKernelGGL((chunk_prefix<D, 2>), dim3(BH, 2, D / 16), dim3(64), 0, st, w0, w0s, 1, H,
                         pl.S, comp, win);
    }
    hipLaunchKernelGGL((chunk_bwd_scan_bf16<D, CH, true>), grid, block, 0, st, Q, K, V, DO, w0, w0s,
                       H, N, a, pl.S, pl.L, win, wring, 0, 0, 1, (int)kOutBf16, part, GQ, GK, GV, d_w0);
    return hipGetLastError();
  }
  if (pl.S > 1) {
    hipLaunchKernelGGL((chunk_compose_bwd_bf16<D, CH, true>), dim3(pl.S, BH), dim3(3 * D / 16 * 64), 0,
                       st, Q, K, V, DO, H, N, a, pl.S, pl.L, comp);
    hipLaunchKernelGGL((chunk_prefix<D, 4>), dim3(BH, 4, D / 16), dim3(64), 0, st, w0, w0s, 2, H,
                       pl.S, comp, win);
  }
  // reversed scan: forward states in slot 1, its adjoints in slot 2; then the forward scan
  hipLaunchKernelGGL((chunk_bwd_scan_bf16<D, CH, false>), grid, block, 0, st, Q, K, V, DO, w0, w0s,
                     H, N, a, pl.S, pl.L, win, wring, 1, 1, 2, (int)kOutPartial, part, GQ, GK, GV, d_w0);
  hipLaunchKernelGGL((chunk_bwd_scan_bf16<D, CH, false>), grid, block, 0, st, Q, K, V, DO, w0, w0s,
                     H, N, a, pl.S, pl.L, win, wring, 0, 0, 3, (int)kOutAddPartial, part, GQ, GK, GV, d_w0);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_bf16_d(bool bidir, int B, int H, int N, int CH, float a, const void* q,
                             const void* k, const void* v, const float* w0, long long w0s,
                             const void* d_o, void* dq, void* dk, void* dv, float* d_w0, void* ws,
                             hipStream_t st) {
  switch (CH) {
    case 16: return launch_bwd_bf16<D, 16>(bidir, B, H, N, a, q, k, v, w0, w0s, d_o, dq, dk, dv, d_w0, ws, st);
    case 32: return launch_bwd_bf16<D, 32>(bidir, B, H, N, a, q, k, v, w0, w0s, d_o, dq, dk, dv, d_w0, ws, st);
    case 64: return launch_bwd_bf16<D, 64>(bidir, B, H, N, a, q, k, v, w0, w0s, d_o, dq, dk, dv, d_w0, ws, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_bwd_f32(bool bidir, int B, int H, int N, int CH, float a, const void* q,
                          const void* k, const void* v, const float* w0, long long w0s,
                          const void* d_o, void* dq, void* dk, void* dv, float* d_w0, void* ws,
                          hipStream_t st) {
  const int BH = B * H;
  float* states = static_cast<float*>(ws);
  const float *Q = (const float*)q, *K = (const float*)k, *V = (const float*)v, *DO = (const float*)d_o;
  float *GQ = (float*)dq, *GK = (float*)dk, *GV = (float*)dv;
  if (!bidir) {
    hipLaunchKernelGGL((chunk_bwd_f32<D, true>), dim3(BH), dim3(256), 0, st, Q, K, V, DO, w0, w0s, H,
                       N, CH, a, 0, states, false, GQ, GK, GV, d_w0);
  } else {
    hipLaunchKernelGGL((chunk_bwd_f32<D, false>), dim3(BH), dim3(256), 0, st, Q, K, V, DO, w0, w0s, H,
                       N, CH, a, 1, states, false, GQ, GK, GV, d_w0);
    hipLaunchKernelGGL((chunk_bwd_f32<D, false>), dim3(BH), dim3(256), 0, st, Q, K, V, DO, w0, w0s, H,
                       N, CH, a, 0, states, true, GQ, GK, GV, d_w0);
  }
  return hipGetLastError();
}

}  // namespace

size_t chunked_workspace_bytes(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk) {
  const size_t BH = (size_t)B * H, DD = (size_t)D * D;
  const ChunkPlan pl = chunk_plan(bidir, B, H, N, D, chunk);
  if (!bf16_io) {
    // fp32 path: map records (-Dev and R, fp32) and entry states per direction, and for the
    // bidirectional scan the reversed scan's state after every chunk (C * D * D per (b, h))
    const size_t ndir = bidir ? 2 : 1;
    size_t bytes = pl.S > 1 ? BH * pl.S * ndir * 2 * DD * sizeof(float) + ndir * BH * pl.S * DD * sizeof(float) : 0;
    if (bidir) bytes += BH * ((size_t)N / (size_t)chunk) * DD * sizeof(float);
    return bytes;
  }
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

hipError_t chunked_bidir_cols_launch(int B, int H, int Hg, int Wg, int D, int chunk, float eta,
                                     const void* q, const void* k, const void* v, const float* w0,
                                     long long w0s, void* o, float* w_out, void* ws, hipStream_t st) {
  const float a = eta / (float)chunk;
  const int N = Hg * Wg;
  const ColMap cm{Hg, Wg};
  switch (D) {
    case 16: return launch_bf16_d<16>(true, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st, &cm);
    case 32: return launch_bf16_d<32>(true, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st, &cm);
    case 64: return launch_bf16_d<64>(true, B, H, N, chunk, a, q, k, v, w0, w0s, o, w_out, ws, st, &cm);
    default: return hipErrorInvalidValue;
  }
}

size_t chunked_bwd_workspace_bytes(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk) {
  const size_t BH = (size_t)B * H, DD = (size_t)D * D, C = (size_t)N / (size_t)chunk;
  // fp32: the scan's C + 1 states per (b, h)
  if (!bf16_io) return BH * (C + 1) * DD * sizeof(float);
  const BwdPlan pl = bwd_plan(B, H, N, chunk);
  const size_t nrec = bidir ? 4 : 2;
  size_t bytes = 0;
  if (pl.S > 1)  // map records (-Dev bf16 + offset fp32) and the folded states, per slot
    bytes += BH * pl.S * nrec * (DD / 2 + DD) * sizeof(float) + nrec * BH * pl.S * DD * sizeof(float);
  bytes += BH * pl.S * (pl.L + 1) * DD * 2;  // the segments' forward states, bf16
  if (bidir)  // the reversed scan's fp32 partial dq, dk, dv
    bytes += 3 * (size_t)B * N * H * D * sizeof(float);
  return bytes;
}

hipError_t chunked_bwd_launch(bool bidir, bool bf16_io, int B, int H, int N, int D, int chunk,
                              float eta, const void* q, const void* k, const void* v,
                              const float* w0, long long w0s, const void* d_o, void* d_q,
                              void* d_k, void* d_v, float* d_w0, void* ws, hipStream_t st) {
  const float a = eta / (float)chunk;
  if (bf16_io) {
    switch (D) {
      case 16: return launch_bwd_bf16_d<16>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
      case 32: return launch_bwd_bf16_d<32>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
      case 64: return launch_bwd_bf16_d<64>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (D) {
    case 16: return launch_bwd_f32<16>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
    case 32: return launch_bwd_f32<32>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
    case 64: return launch_bwd_f32<64>(bidir, B, H, N, chunk, a, q, k, v, w0, w0s, d_o, d_q, d_k, d_v, d_w0, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttt
