// Causal mini-batch TTT-MLP forward (TTT-Linear / TTT-MLP abstract: the hidden state is a
// two-layer MLP trained by a self-supervised step; mini-batches: Vision-TTT summary on
// gist.science, "Methodologie" item 3).
//
// Inner model f(x) = GELU(x W1) W2, W1 [D, Dh], W2 [Dh, D], loss 1/2 ||f(k) - v||^2 per token.
// Per chunk of b tokens with start state (W1, W2), all gradients taken at the start state:
//   Z1 = K W1, X2 = GELU(Z1), E = X2 W2 - V, D1 = (E W2^T) * GELU'(Z1)
//   W1' = W1 - a K^T D1,  W2' = W2 - a X2^T E,   a = eta / b
// and token t is read out with the start state minus a times the gradients of tokens t' <= t.
// Written with the END state of the chunk (W1', W2') this read-out is
//   Z1q = Q W1' + a striu(Q K^T) D1,  X2q = GELU(Z1q),  O = X2q W2' + a striu(X2q X2^T) E
// (striu keeps t' > t), which is the same quantity: Q W1 - a tril(Q K^T) D1 = Q W1' + a (Q K^T -
// tril(Q K^T)) D1. The end state of chunk c is the start state of chunk c + 1, so the read-out of
// chunk c is computed in the same pass as chunk c + 1's forward, sharing its weight operands.
//
// One workgroup per (batch, head), 8 waves; wave w owns hidden units [32w, 32w + 32): its slice
// of W1 (columns), of W2 (rows) and a second copy of its W2 slice in transposed accumulator
// layout (the operand of E W2^T). All three stay in MFMA accumulator registers for the whole
// sequence and are updated in place by MFMA. Z1, X2 and D1 are produced as [token][hidden]
// accumulator tiles, which are directly the operands of the weight updates; the transposed
// operands of K and E (contractions over tokens) come from LDS by gfx950 transpose reads, and
// X2^T (for the contraction over hidden units) is a product with an identity tile. The
// cross-wave sums over hidden units (Z2 and the read-out) go through LDS in a fixed wave order,
// so results are deterministic. The steps between the first and the last have both a read-out
// and a forward, known at compile time, so that their products and GELUs share basic blocks and
// interleave. E is kept as -a E (a = eta / b), so that -a D1 and the weight updates' operands come
// out of the products with the right sign (no separate negations). Operand precision: the
// products on the W1 side (inputs K, Q and D1) take bf16 operands, those on the W2 side (X2, W2,
// E, X2 X2^T) fp16 ones, which the packed fp16 GELU path produces directly; all accumulate in fp32. Two workgroup barriers per
// chunk; K, V, Q are staged through a four-deep LDS ring: each chunk's global loads are issued
// three chunks ahead into one of two alternating register sets and stored to LDS two chunks ahead.
//
// No 16x16x16 product accumulates onto the result of a 16x16x32 product: on gfx950 such a
// mixed-shape accumulator chain was measured to read a stale accumulator (wrong results that
// depended on the instruction schedule), so terms of different shapes get separate accumulators
// and are added in registers.
#include <type_traits>

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
// Pitch of [token][feature] tiles (elements): 152 bytes = 38 banks, so the paired 8-byte operand
// reads (32 bytes apart), the row reads and the transpose reads hit distinct banks. Rows are only
// 8-byte aligned: staging stores go in 8-byte pieces.
constexpr int kP = kD + 12;
constexpr int kRing = 4;           // K/V/Q staging depth
constexpr int kSlots = 8;          // partial tiles per wave: Z2^T x4, O^T x4

constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kNegHalfLog2e = -0.72134752044448170368f;  // -log2(e) / 2
constexpr float kLog2InvSqrt2Pi = -1.32574806473615935f;   // log2(1 / sqrt(2 pi))

// GELU(x) = x Phi(x) with Phi(x) = (1 + erf(x / sqrt 2)) / 2 (exact erf form) and
// GELU'(x) = Phi(x) + x phi(x), phi the standard normal density.
// Fast path, used when every argument of the wave's GELUs in a chunk step has x^2 <= 2
// (|x / sqrt 2| <= 1): erf(u) = u P(u^2)
// with P the degree-3 least-squares polynomial for erf(u)/u on u^2 in [0, 1] (fitted on Chebyshev
// nodes; max abs error of erf 2.7e-5 in fp32 Horner form), so Phi(x) = 1/2 + x R(x^2) with
// R(t) = P(t / 2) / (2 sqrt 2). It runs in packed fp16 (below); its GELU and GELU' stay within
// 1.1e-3 of the exact values, about the rounding of a bf16 operand. Otherwise fp32 with the
// library erf and exp2.
constexpr float kErfP[4] = {1.128350616f, -0.3751908541f, 0.1079747304f, -0.0184600465f};
constexpr float kInvTwoSqrt2 = 0.35355339059327376220f;
constexpr float kR0 = kErfP[0] * kInvTwoSqrt2, kR1 = kErfP[1] * kInvTwoSqrt2 / 2.f,
                kR2 = kErfP[2] * kInvTwoSqrt2 / 4.f, kR3 = kErfP[3] * kInvTwoSqrt2 / 8.f;

__device__ __forceinline__ float cdf_fast(float x, float t) {  // t = x * x <= 2
  float r = fmaf(kR3, t, kR2);
  r = fmaf(r, t, kR1);
  r = fmaf(r, t, kR0);
  return fmaf(x, r, 0.5f);
}
__device__ __forceinline__ float cdf_lib(float x) { return 0.5f * (1.f + erff(x * kInvSqrt2)); }

__device__ __forceinline__ bf16x8 cat_tiles(f32x4 lo, f32x4 hi) {
  return cat8(to_bf16x4(lo), to_bf16x4(hi));
}

// fp16 operands for the products on the W2 side (X2, W2, E and the X2 X2^T terms): three more
// mantissa bits than bf16, and the packed fp16 arithmetic of the fast GELU path yields them
// directly (no conversions). Their range (|x| < 65504) is far above these activations.
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mmah32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mmah16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) {  // round to nearest even, two per instruction
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f16x2 lo = __builtin_convertvector(f32x2{x[0], x[1]}, f16x2);
  const f16x2 hi = __builtin_convertvector(f32x2{x[2], x[3]}, f16x2);
  return __builtin_bit_cast(f16x4, make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)));
}
__device__ __forceinline__ f16x8 cat8h(f16x4 lo, f16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 cat_tiles_h(f32x4 lo, f32x4 hi) { return cat8h(to_f16x4(lo), to_f16x4(hi)); }
__device__ __forceinline__ f16x4 ld4h(const f16* p) { return *reinterpret_cast<const f16x4*>(p); }
__device__ __forceinline__ f16x4 tile_tr_h(const f16* base, int pitch, int l) {  // as tile_tr
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int u = l & 15;
  const f16* p = base + (4 * (l >> 4) + (u >> 2)) * pitch + 4 * (u & 3);
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

// Fast GELU path in packed fp16 (|x| <= sqrt 2): Phi(x) = 1/2 + x R(t) as above, and
// GELU'(x) = 1/2 + x S(t), t = x^2, with S the degree-3 least-squares polynomial for
// (Phi(x) - 1/2) / x + phi(x) on t in [0, 2] (Chebyshev nodes; max abs error of GELU' 1.2e-4).
constexpr float kS0 = 0.7977905544868868f, kS1 = -0.26441428752463436f, kS2 = 0.0557860757632853f,
                kS3 = -0.0059361438042217956f;
__device__ __forceinline__ f16x4 splat(float v) { return (f16x4)(f16)v; }
__device__ __forceinline__ f16x4 fmah(f16x4 a, f16x4 b, f16x4 c) { return __builtin_elementwise_fma(a, b, c); }
__device__ __forceinline__ f16x4 cdf_fast_h(f16x4 x, f16x4 t) {
  f16x4 r = fmah(splat(kR3), t, splat(kR2));
  r = fmah(r, t, splat(kR1));
  r = fmah(r, t, splat(kR0));
  return fmah(x, r, splat(0.5f));
}
__device__ __forceinline__ f16x4 slope_fast_h(f16x4 x, f16x4 t) {
  f16x4 r = fmah(splat(kS3), t, splat(kS2));
  r = fmah(r, t, splat(kS1));
  r = fmah(r, t, splat(kS0));
  return fmah(x, r, splat(0.5f));
}

__device__ __forceinline__ void st16_lds8(bf16* p, uint4 v) {
  reinterpret_cast<uint2*>(p)[0] = make_uint2(v.x, v.y);
  reinterpret_cast<uint2*>(p)[1] = make_uint2(v.z, v.w);
}

__global__ __launch_bounds__(kWaves * 64, 1) void mlp_fwd_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out) {
  __shared__ __align__(16) bf16 sKVQ[kRing][3][kCh * kP];
  __shared__ __align__(16) f16 sE[2][kCh * kP];            // -a E [token][out] (fp16)
  __shared__ __align__(16) f32x4 sRed[kWaves * kSlots * 64];  // lane-private partial tiles

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
  f16x4 ident;  // identity tile as the B operand: lane holds I[4g + i][r]
  for (int i = 0; i < 4; ++i) ident[i] = (f16)(4 * g + i == r ? 1.f : 0.f);

  const int C = N / kCh;
  const long long head0 = (long long)b * N * ts + (long long)h * kD;
  // Staging: threads 0..383 each move one 16-byte piece of K, V or Q (16 rows x 8 pieces each).
  const int t = threadIdx.x;
  const int prow = (t & 127) >> 3, pcol = (t & 7) * 8, which = t >> 7;
  const bf16* psrc = (t < 128 ? k : (t < 256 ? v : q)) + head0 + prow * ts + pcol;
  uint4 pfA = make_uint4(0u, 0u, 0u, 0u), pfB = make_uint4(0u, 0u, 0u, 0u);
  if (t < 384) {
    st16_lds8(&sKVQ[0][which][prow * kP + pcol], ld16(psrc));
    if (C > 1) st16_lds8(&sKVQ[1][which][prow * kP + pcol], ld16(psrc + kCh * ts));
    if (C > 2) pfB = ld16(psrc + 2 * kCh * ts);
  }
  __syncthreads();

  bf16x4 d1p[kNh];  // -a D1 of the previous chunk, [token][hidden] tiles
  f16x8 x2tp;       // X2^T of the previous chunk, [hidden][token] tiles (both, c-layout k map)
  for (int n = 0; n < kNh; ++n) d1p[n] = bf16x4{};
  x2tp = f16x8{};

  // One chunk step: forward of chunk c, read-out of chunk c - 1. pf_cur holds chunk c + 2 (loaded
  // one step earlier); chunk c + 3 is loaded into pf_next.
  auto step = [&](const int c, uint4& pf_next, const uint4& pf_cur, auto rd_tag, auto fwd_tag) {
    constexpr bool rd = decltype(rd_tag)::value;    // read-out of chunk c - 1
    constexpr bool fwd = decltype(fwd_tag)::value;  // forward of chunk c
    if (t < 384 && c + 3 < C) pf_next = ld16(psrc + (long long)(c + 3) * kCh * ts);
    const bf16* sK = sKVQ[c % kRing][0];
    const bf16* sV = sKVQ[c % kRing][1];
    const bf16* sKp = sKVQ[(c + kRing - 1) % kRing][0];  // chunk c - 1
    const bf16* sQp = sKVQ[(c + kRing - 1) % kRing][2];
    f16* sEc = sE[c & 1];
    const f16* sEp = sE[(c + 1) & 1];  // -a E of chunk c - 1

    // ---------------- phase 1: products with the current weights. The read-out of chunk c - 1
    // and the forward of chunk c are independent; their products, GELUs and remaining products
    // are grouped so that one basic block holds both chains.
    bf16x8 w1b[2][kNh];  // W1 tiles (k = features, c-layout k map)
    for (int ks = 0; ks < 2; ++ks)
      for (int n = 0; n < kNh; ++n) w1b[ks][n] = cat_tiles(W1t[2 * ks][n], W1t[2 * ks + 1][n]);
    f32x4 Z1q[kNh];  // read-out: Z1q^T [hidden][token]
    f32x4 Z1[kNh];   // forward: Z1 [token][hidden]
    f16x4 x2qh[kNh], x2b[kNh], gph[kNh];  // GELU(Z1q), GELU(Z1), GELU'(Z1) as fp16 tiles
    if constexpr (rd) {
      // M[t'][t] = k_t' . q_t of chunk c - 1, kept for t' > t.
      f32x4 mt = zero4();
      for (int ks = 0; ks < 2; ++ks)
        mt = mma32(cat8(ld4(&sKp[r * kP + 32 * ks + 4 * g]), ld4(&sKp[r * kP + 32 * ks + 16 + 4 * g])),
                   cat8(ld4(&sQp[r * kP + 32 * ks + 4 * g]), ld4(&sQp[r * kP + 32 * ks + 16 + 4 * g])), mt);
      for (int j = 0; j < 4; ++j) mt[j] = 4 * g + j <= r ? 0.f : -mt[j];
      const bf16x4 mb = to_bf16x4(mt);  // -M, t' > t kept (the carried D1 is -a D1)
      // Z1q^T = W1^T Q^T + a D1^T M = W1^T Q^T + (-a D1)^T (-M).
      for (int n = 0; n < kNh; ++n) {
        f32x4 z = zero4();
        for (int ks = 0; ks < 2; ++ks) {
          const bf16* pq = &sQp[r * kP + 32 * ks + 4 * g];
          z = mma32(w1b[ks][n], cat8(ld4(pq), ld4(pq + 16)), z);
        }
        // (-a D1)^T (-M) as a 16x16x32 product with the upper k half zero in both operands, so that
        // it chains onto the same-shape accumulator (a 16x16x16 product must not).
        Z1q[n] = mma32(cat8(d1p[n], bf16x4{}), cat8(mb, bf16x4{}), z);
      }
    }
    if constexpr (fwd) {
      // Z1 = K W1: A = K rows (c-layout k map), B = W1 tiles.
      for (int n = 0; n < kNh; ++n) {
        f32x4 z = zero4();
        for (int ks = 0; ks < 2; ++ks) {
          const bf16* pk = &sK[r * kP + 32 * ks + 4 * g];
          z = mma32(cat8(ld4(pk), ld4(pk + 16)), w1b[ks][n], z);
        }
        Z1[n] = z;
      }
    }
    {  // GELU of both chains, one fast-path decision for the wave
      f16x4 zq[kNh], zf[kNh], tq[kNh], tf[kNh];
      f16x4 tm = splat(0.f);
      for (int n = 0; n < kNh; ++n) {
        if constexpr (rd) {
          zq[n] = to_f16x4(Z1q[n]);
          tq[n] = zq[n] * zq[n];
          tm = __builtin_elementwise_max(tm, tq[n]);
        }
        if constexpr (fwd) {
          zf[n] = to_f16x4(Z1[n]);
          tf[n] = zf[n] * zf[n];
          tm = __builtin_elementwise_max(tm, tf[n]);
        }
      }
      const float tmax = fmaxf(fmaxf((float)tm[0], (float)tm[1]), fmaxf((float)tm[2], (float)tm[3]));
      if (!__any(!(tmax <= 2.f))) {
        for (int n = 0; n < kNh; ++n) {
          if constexpr (rd) x2qh[n] = zq[n] * cdf_fast_h(zq[n], tq[n]);
          if constexpr (fwd) {
            x2b[n] = zf[n] * cdf_fast_h(zf[n], tf[n]);
            gph[n] = slope_fast_h(zf[n], tf[n]);
          }
        }
      } else {  // fp32 with the library erf
        for (int n = 0; n < kNh; ++n) {
          f32x4 xq, xf, gp;
          for (int j = 0; j < 4; ++j) {
            if constexpr (rd) xq[j] = Z1q[n][j] * cdf_lib(Z1q[n][j]);
            if constexpr (fwd) {
              const float x = Z1[n][j], cdf = cdf_lib(x);
              xf[j] = x * cdf;
              gp[j] = fmaf(x, __builtin_amdgcn_exp2f(fmaf(x * x, kNegHalfLog2e, kLog2InvSqrt2Pi)), cdf);
            }
          }
          if constexpr (rd) x2qh[n] = to_f16x4(xq);
          if constexpr (fwd) {
            x2b[n] = to_f16x4(xf);
            gph[n] = to_f16x4(gp);
          }
        }
      }
    }
    f16x8 x2q;
    f16x4 n2b;
    if constexpr (rd) {
      x2q = cat8h(x2qh[0], x2qh[1]);
      // (with the previous chunk's X2^T, before the forward below replaces it)
      f32x4 n2 = mmah32(x2tp, x2q, zero4());  // [t'][t] = sum_h X2[t'][h] X2q[t][h]
      for (int j = 0; j < 4; ++j) n2[j] = 4 * g + j <= r ? 0.f : -n2[j];
      n2b = to_f16x4(n2);  // (-a is in the stored E)
    }
    if constexpr (fwd) {
      f32x4 xt[kNh];
      for (int n = 0; n < kNh; ++n) xt[n] = mmah16(x2b[n], ident, zero4());  // X2^T [hidden][token]
      x2tp = cat_tiles_h(xt[0], xt[1]);
    }
    f16x8 w2a[4];  // W2^T tiles (k = this wave's hidden units), for both products below
    for (int o2 = 0; o2 < 4; ++o2) w2a[o2] = cat_tiles_h(W2t[0][o2], W2t[1][o2]);
    if constexpr (rd) {
      // This wave's share of O^T [out][token]: W2^T X2q^T over its hidden units, plus
      // (a E)^T striu(X2q X2^T)^T = (-a E)^T (-striu(X2q X2^T))^T with X2q X2^T summed over the
      // same units (t' > t kept), the latter as a 16x16x32 product with a zero upper k half
      // (same-shape chain).
      for (int o2 = 0; o2 < 4; ++o2) {
        const f32x4 ow = mmah32(w2a[o2], x2q, zero4());
        sRed[(w * kSlots + 4 + o2) * 64 + l] =
            mmah32(cat8h(tile_tr_h(&sEp[16 * o2], kP, l), f16x4{}), cat8h(n2b, f16x4{}), ow);  // A = (-a E)^T
      }
    }
    if constexpr (fwd) {
      // Z2^T partial [out][token] over this wave's hidden units.
      for (int o2 = 0; o2 < 4; ++o2) sRed[(w * kSlots + o2) * 64 + l] = mmah32(w2a[o2], x2tp, zero4());
    }
    __syncthreads();

    // ---------------- phase 2: cross-wave sums (fixed wave order)
    if (fwd && w < 4) {  // E^T tile w = Z2^T - V^T, stored as -a E [token][out]
      // All nine LDS reads are issued before the adds (the compiler otherwise keeps only two or
      // three of them in flight, and this phase is their latency).
      f32x4 pt[kWaves];
      for (int ww = 0; ww < kWaves; ++ww) pt[ww] = sRed[(ww * kSlots + w) * 64 + l];
      const bf16x4 vv = ld4(&sV[r * kP + 16 * w + 4 * g]);
      __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
      f32x4 s = pt[0];
      for (int ww = 1; ww < kWaves; ++ww) s = s + pt[ww];
      f32x4 e;
      for (int j = 0; j < 4; ++j) e[j] = a * ((float)vv[j] - s[j]);
      *reinterpret_cast<f16x4*>(&sEc[r * kP + 16 * w + 4 * g]) = to_f16x4(e);
    }
    if (rd && w >= 4) {  // O^T tile of chunk c - 1 = sum of the waves' shares
      const int o4 = w - 4;
      f32x4 pt[kWaves];
      for (int ww = 0; ww < kWaves; ++ww) pt[ww] = sRed[(ww * kSlots + 4 + o4) * 64 + l];
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      f32x4 s = pt[0];
      for (int ww = 1; ww < kWaves; ++ww) s = s + pt[ww];
      const long long tokp = head0 + (long long)(c - 1) * kCh * ts;
      *reinterpret_cast<bf16x4*>(o + tokp + r * ts + 16 * o4 + 4 * g) = to_bf16x4(s);
    }
    __syncthreads();

    // ---------------- phase 3: backward and state update of chunk c
    if (fwd) {
      // -a dX2 [token][hidden] = (-a E) W2^T: A = -a E rows (c-layout k map), B = W2x tiles.
      f16x8 ea[2];
      for (int ko = 0; ko < 2; ++ko) {
        const f16* pe = &sEc[r * kP + 32 * ko + 4 * g];
        ea[ko] = cat8h(ld4h(pe), ld4h(pe + 16));
      }
      for (int n = 0; n < kNh; ++n) {
        f32x4 acc = zero4();
        for (int ko = 0; ko < 2; ++ko) acc = mmah32(ea[ko], cat_tiles_h(W2x[2 * ko][n], W2x[2 * ko + 1][n]), acc);
        f32x4 d1;  // -a D1
        for (int j = 0; j < 4; ++j) d1[j] = acc[j] * (float)gph[n][j];
        d1p[n] = to_bf16x4(d1);
      }
      // W1 += K^T (-a D1): A = K^T (row feature, k token; LDS transpose read), B = -a D1.
      for (int m = 0; m < 4; ++m) {
        const bf16x4 kt = tile_tr(&sK[16 * m], kP, l);
        for (int n = 0; n < kNh; ++n) W1t[m][n] = mma16(kt, d1p[n], W1t[m][n]);
      }
      // W2 += X2^T (-a E) and W2^T += (-a E)^T X2: -a E's transposed tiles give both operands.
      for (int o2 = 0; o2 < 4; ++o2) {
        const f16x4 e = tile_tr_h(&sEc[16 * o2], kP, l);
        for (int n = 0; n < kNh; ++n) {
          W2t[n][o2] = mmah16(x2b[n], e, W2t[n][o2]);
          W2x[o2][n] = mmah16(e, x2b[n], W2x[o2][n]);
        }
      }
    }
    if (t < 384 && c + 2 < C) st16_lds8(&sKVQ[(c + 2) % kRing][which][prow * kP + pcol], pf_cur);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Step 0 has no read-out, step C no forward; the steps between have both (two per trip: the
  // register sets swap roles).
  if (C > 0) step(0, pfA, pfB, F_{}, T_{});
  int c = 1;
  for (; c + 1 < C; c += 2) {
    step(c, pfB, pfA, T_{}, T_{});
    step(c + 1, pfA, pfB, T_{}, T_{});
  }
  if (c < C) {
    step(c, pfB, pfA, T_{}, T_{});
    step(c + 1, pfA, pfB, T_{}, F_{});
  } else {
    step(c, pfB, pfA, T_{}, F_{});
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
