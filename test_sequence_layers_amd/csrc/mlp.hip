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
// so results are deterministic. E is kept as -a E (a = eta / b), so that -a D1 and the weight
// updates' operands come out of the products with the right sign (no separate negations). Two
// workgroup barriers per chunk; K, V (and Q) are staged through a four-deep LDS ring: each chunk's
// global loads are issued three chunks ahead into one of two alternating register sets and stored
// to LDS two chunks ahead.
//
// Schedule. The forward chain (the state updates) is sequential per (b, h), and only 48 chains
// exist at the reference shape, so it holds 48 of the 256 CUs. The read-outs do not feed the chain:
// the chain workgroup stores, per chunk, the -a D1 and X2 tiles of each wave and the -a E tile,
// and at each segment start a checkpoint of its state; read-out workgroups on other CUs replay a
// segment's state updates from its checkpoint with those tiles (the chain's own products, so the
// same states bit for bit) and read each chunk out with its end state (the end-state form above).
// Both roles share one launch (chain workgroups first, so that they are dispatched before any
// read-out workgroup waits on them; see mlp_fwd_fused). Without the read-outs in its steps the
// chain runs 785 us instead of 945 at 4 x 8192 x 12 heads. The steps between the first and the last
// of the generic single-workgroup form (used by the bf16 recomputation) have both a read-out and a
// forward, known at compile time, so that their products and GELUs share basic blocks and
// interleave.
//
// Operand precision. The products on the W1 side (inputs K, Q and D1) take bf16 operands. Those
// on the W2 side (X2, X2q, W2, E and X2q X2^T) take fp16 operands in the first launch: three more
// mantissa bits than bf16, and the packed fp16 GELU path produces them directly. fp16 covers
// magnitudes 2^-14 .. 65504 at full precision, so that launch checks, per wave and step, the
// values it converts: the hidden pre-activations (each lane's largest magnitude at least 2^-10
// unless all are zero, and at most sqrt 2 for the polynomial GELU; GELU outputs at most 32 in
// magnitude otherwise, so that the 32-unit sums of X2q X2^T stay below 32768) and, every 32 chunks
// and at the end, the W2 slice (largest magnitude in [2^-10, 2^15], or zero). The -a E tiles are
// not checked in the steps: an fp16 overflow there turns the W2 update and, through D1, the W1
// update into inf or NaN, which a final check of the whole state catches. Nor do they need a lower
// bound: -a E only enters as a correction added to a term without it (the W2 update to W2, the
// read-out's correction to X2q W2, through D1 the W1 update to W1), so its rounding error below
// fp16's normal range (at most 2^-25 a value) stays negligible beside them when a = eta / b is
// small, and inputs or weights small enough to make those terms small too fail the other checks.
// A (batch,
// head) chain that fails any check (in its forward chain or in a read-out) is flagged in the
// workspace, and a last launch recomputes exactly the flagged chains in the single-workgroup form
// with bf16 operands on the W2 side (bf16 has fp32's exponent range) and the fp32 GELU; every other
// chain returns at once. All products accumulate in fp32.
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
// Fast path, used when every argument of the wave's GELUs in a chunk step has |x| <= sqrt 2
// (rounded down to fp16, so x^2 <= 2 and |x / sqrt 2| <= 1): erf(u) = u P(u^2)
// with P the degree-3 least-squares polynomial for erf(u)/u on u^2 in [0, 1] (fitted on Chebyshev
// nodes; max abs error of erf 2.7e-5 in fp32 Horner form), so Phi(x) = 1/2 + x R(x^2) with
// R(t) = P(t / 2) / (2 sqrt 2). It runs in packed fp16 (below); its GELU and GELU' stay within
// 1.1e-3 of the exact values, about the rounding of a bf16 operand. Otherwise fp32 with the
// library erf and exp2.
constexpr float kErfP[4] = {1.128350616f, -0.3751908541f, 0.1079747304f, -0.0184600465f};
constexpr float kInvTwoSqrt2 = 0.35355339059327376220f;
constexpr float kSqrt2h = 1.4140625f;  // sqrt 2 rounded down to fp16: the fast path's bound on |x|
constexpr uint32_t kZLoBits = 0x3A800000u;  // float bits of 2^-10
constexpr uint32_t kZHiBits = 0x3FB50000u;  // float bits of 1.4140625
constexpr float kR0 = kErfP[0] * kInvTwoSqrt2, kR1 = kErfP[1] * kInvTwoSqrt2 / 2.f,
                kR2 = kErfP[2] * kInvTwoSqrt2 / 4.f, kR3 = kErfP[3] * kInvTwoSqrt2 / 8.f;

__device__ __forceinline__ float cdf_lib(float x) { return 0.5f * (1.f + erff(x * kInvSqrt2)); }

__device__ __forceinline__ bf16x8 cat_tiles(f32x4 lo, f32x4 hi) {
  return cat8(to_bf16x4(lo), to_bf16x4(hi));
}

// fp16 operands for the products on the W2 side (X2, W2, E and the X2 X2^T terms): three more
// mantissa bits than bf16, and the packed fp16 arithmetic of the fast GELU path yields them
// directly (no conversions). The kernel checks that the values it converts stay inside fp16's
// range (header comment).
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

// The operand type of the products on the W2 side: fp16 (first launch) or bf16 (recomputation of
// the chains whose values left fp16's range).
template <bool F16>
struct W2Side;
template <>
struct W2Side<true> {
  typedef f16 elem;
  typedef f16x4 x4;
  typedef f16x8 x8;
  static __device__ __forceinline__ f32x4 mma32(x8 a, x8 b, f32x4 c) { return mmah32(a, b, c); }
  static __device__ __forceinline__ f32x4 mma16(x4 a, x4 b, f32x4 c) { return mmah16(a, b, c); }
  static __device__ __forceinline__ x4 cvt(f32x4 x) { return to_f16x4(x); }
  static __device__ __forceinline__ x8 cat(x4 lo, x4 hi) { return cat8h(lo, hi); }
  static __device__ __forceinline__ x4 ld(const elem* p) { return ld4h(p); }
  static __device__ __forceinline__ x4 tr(const elem* base, int pitch, int l) { return tile_tr_h(base, pitch, l); }
};
template <>
struct W2Side<false> {
  typedef bf16 elem;
  typedef bf16x4 x4;
  typedef bf16x8 x8;
  static __device__ __forceinline__ f32x4 mma32(x8 a, x8 b, f32x4 c) { return ttt::mma32(a, b, c); }
  static __device__ __forceinline__ f32x4 mma16(x4 a, x4 b, f32x4 c) { return ttt::mma16(a, b, c); }
  static __device__ __forceinline__ x4 cvt(f32x4 x) { return to_bf16x4(x); }
  static __device__ __forceinline__ x8 cat(x4 lo, x4 hi) { return cat8(lo, hi); }
  static __device__ __forceinline__ x4 ld(const elem* p) { return ld4(p); }
  static __device__ __forceinline__ x4 tr(const elem* base, int pitch, int l) { return tile_tr(base, pitch, l); }
};

// Largest magnitude among the four values (NaN compares as not in any range below).
__device__ __forceinline__ float absmax4(f32x4 x) {
  return fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
}
// True when, over the wave, the largest magnitude m (one per lane) is outside [lo, hi] while not all
// values are zero, or is not a number.
__device__ __forceinline__ bool wave_out_of_range(float m, float lo, float hi) {
  return __any(!(m <= hi)) || (__any(m > 0.f) && !__any(m >= lo));
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

// The workgroup's shared memory, used by both passes of a chain.
struct MlpLds {
  bf16 kvq[kRing][3][kCh * kP];     // K, V, Q staging ring
  unsigned short e[2][kCh * kP];    // -a E [token][out], fp16 or bf16 bits
  f32x4 red[kWaves * kSlots * 64];  // lane-private partial tiles
  int bad;
};

// Intermediates of the split schedule (SPLIT), per (b, h) chain in the workspace: for every chunk the
// -a D1 tiles of every thread's wave (bf16x4 x 2 per thread), then the X2 tiles (fp16x4 x 2), so
// that each store instruction writes whole lines, for
// every chunk the -a E tile (four 16 x 16 tiles, lane l of wave w < 4 holds tile w's accumulator
// fragment: 8 bytes; waves 4-7 store zeros to slots of their own, so that every wave issues the
// same memory operations), and at the start of every read-out segment a checkpoint of the state (each
// thread's W1 and W2 tiles: 16 fp32x4).
// Segments: kSegLong chunks each, except that the last (up to kSegLong) chunks are cut into
// segments of kSegTail, so that little read-out work is left when the chain ends; every segment end
// is a publication of the chain (a wait for its stores and an L2 write-back), which is why the
// other segments are long.
constexpr int kSegLong = 64;
constexpr int kSegTail = 16;
constexpr int kReadoutWorkers = 96;  // read-out workgroups of the fused launch (48, 64, 96, 128, 192 measured: 96 best)
struct SegPlan {
  int C, R, nlong;  // chunks; start of the tail region; segments before it
  __host__ __device__ explicit SegPlan(int C_) : C(C_), R((C_ - 1) / kSegLong * kSegLong), nlong((C_ - 1) / kSegLong) {}
  __host__ __device__ int count() const { return nlong + (C - R + kSegTail - 1) / kSegTail; }
  __host__ __device__ int lo(int s) const { return s < nlong ? s * kSegLong : R + (s - nlong) * kSegTail; }
  __host__ __device__ int hi(int s) const { return min(C, s < nlong ? (s + 1) * kSegLong : R + (s - nlong + 1) * kSegTail); }
  // the segment that starts at chunk c, or -1
  __host__ __device__ int starting_at(int c) const {
    if (c < R) return c % kSegLong == 0 ? c / kSegLong : -1;
    return (c - R) % kSegTail == 0 ? nlong + (c - R) / kSegTail : -1;
  }
  __host__ __device__ bool is_end(int done) const {
    return done <= R ? done % kSegLong == 0 : ((done - R) % kSegTail == 0 || done == C);
  }
};
// The intermediates are stored with the nontemporal hint: the chain never reads them back, and
// fewer dirty lines are left in the L2 for each publication's write-back (measured 898 -> 881 us).
__device__ __forceinline__ void st8_out(void* p, uint2 v) {
  typedef unsigned u32x2_nt __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(__builtin_bit_cast(u32x2_nt, v), reinterpret_cast<u32x2_nt*>(p));
}
struct MlpSplitWs {
  uint4* inter;   // [bh][chunk][D1, X2][thread]
  uint2* etile;   // [bh][chunk][8 waves][64 lanes] (slots of waves 4-7 unused)
  f32x4* ckpt;    // [bh][segment][thread][16]
  int* progress;  // [bh]: chunks whose intermediates are published (release, agent scope)
};
__host__ __device__ inline long long mlp_inter_uint4(int C) { return (long long)C * kWaves * 64 * 2; }
__host__ __device__ inline long long mlp_etile_uint2(int C) { return (long long)C * 8 * 64; }
__host__ __device__ inline long long mlp_ckpt_f32x4(int C) { return (long long)SegPlan(C).count() * kWaves * 64 * 16; }

// One (b, h) chain. F16: fp16 operands on the W2 side with range checks; returns true (the same in
// every thread) when a check failed. !F16: bf16 operands, no checks; returns false.
// SPLIT (with F16): the forward chain only, no read-out and no Q staging; each step stores its
// intermediates and at each segment start the state into sw, from which the read-out workgroups compute the
// read-outs of all chunks in parallel.
template <bool F16, bool SPLIT = false>
__device__ __forceinline__ bool mlp_chain(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out,
    MlpLds& lds, MlpSplitWs sw = MlpSplitWs{}) {
  static_assert(!SPLIT || F16, "the split schedule runs the fp16 pass");
  using S = W2Side<F16>;
  using x4 = typename S::x4;
  using x8 = typename S::x8;
  using GpT = typename std::conditional<F16, f16x4, f32x4>::type;  // GELU'(Z1) tiles
  auto& sKVQ = lds.kvq;
  auto sE = reinterpret_cast<typename S::elem(*)[kCh * kP]>(lds.e);
  f32x4* const sRed = lds.red;
  int& sBad = lds.bad;

  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const long long ts = (long long)H * kD;
  const float* W1g = w1 + b * wbs + (long long)h * kD * kDh;
  const float* W2g = w2 + b * wbs + (long long)h * kDh * kD;
  const int hid0 = kHw * w;
  bool bad = false;  // wave-uniform: a value converted to fp16 left the checked range
  if (F16 && threadIdx.x == 0) sBad = 0;

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
  x4 ident;  // identity tile as the B operand: lane holds I[4g + i][r]
  for (int i = 0; i < 4; ++i) ident[i] = (typename S::elem)(4 * g + i == r ? 1.f : 0.f);

  const int C = N / kCh;
  const long long head0 = (long long)b * N * ts + (long long)h * kD;
  // Staging: every thread moves one 16-byte piece of K, V or Q per chunk (16 rows x 8 pieces each);
  // threads 384..511 repeat the Q pieces of threads 256..383 (same source, same LDS address, same
  // value). Chunk indices past the end are clamped to the last chunk. So every wave issues the same
  // loads on every step, and the compiler's wait before a staged piece's LDS write counts only the
  // memory operations issued after its load: no wait drains the loads in flight or the O stores.
  const int t = threadIdx.x, u = SPLIT ? (t & 255) : (t < 384 ? t : t - 128);
  const int prow = (u & 127) >> 3, pcol = (u & 7) * 8, which = u >> 7;
  const bf16* psrc = (u < 128 ? k : (u < 256 ? v : q)) + head0 + prow * ts + pcol;
  bf16* const pdst = &sKVQ[0][which][prow * kP + pcol];
  auto chunk_src = [&](int cc) { return psrc + (long long)min(cc, C - 1) * kCh * ts; };
  st16_lds8(pdst, ld16(psrc));
  uint4 pfA = ld16(chunk_src(1)), pfB = ld16(chunk_src(2));  // chunks 1 and 2
  __syncthreads();

  const long long bhs = blockIdx.x;
  uint4* const inter = sw.inter + bhs * mlp_inter_uint4(C) + t;
  uint2* const etile = sw.etile + bhs * mlp_etile_uint2(C) + 64 * w + l;
  f32x4* const ckpt = sw.ckpt + bhs * mlp_ckpt_f32x4(C) + 16 * t;
  bf16x4 d1p[kNh];  // -a D1 of the previous chunk, [token][hidden] tiles
  x8 x2tp;          // X2^T of the previous chunk, [hidden][token] tiles (both, c-layout k map)
  for (int n = 0; n < kNh; ++n) d1p[n] = bf16x4{};
  x2tp = x8{};

  // One chunk step: forward of chunk c, read-out of chunk c - 1. pf holds chunk c + 1 (loaded two
  // steps earlier); at the end of phase 1 it goes to its ring slot and is reloaded with chunk c + 3.
  auto step = [&](const int c, uint4& pf, auto rd_tag, auto fwd_tag) {
    constexpr bool rd = decltype(rd_tag)::value;    // read-out of chunk c - 1
    constexpr bool fwd = decltype(fwd_tag)::value;  // forward of chunk c
    const bf16* sK = sKVQ[c % kRing][0];
    const bf16* sV = sKVQ[c % kRing][1];
    const bf16* sKp = sKVQ[(c + kRing - 1) % kRing][0];  // chunk c - 1
    const bf16* sQp = sKVQ[(c + kRing - 1) % kRing][2];
    typename S::elem* sEc = sE[c & 1];
    const typename S::elem* sEp = sE[(c + 1) & 1];  // -a E of chunk c - 1

    // ---------------- phase 1: products with the current weights. The read-out of chunk c - 1
    // and the forward of chunk c are independent; their products, GELUs and remaining products
    // are grouped so that one basic block holds both chains.
    if constexpr (SPLIT) {
      const int sg = SegPlan(C).starting_at(c);
      if (sg >= 0) {  // the chunk's start state
        f32x4* dst = ckpt + (long long)sg * kWaves * 64 * 16;
        for (int m = 0; m < 4; ++m)
          for (int n = 0; n < kNh; ++n) dst[m * kNh + n] = W1t[m][n];
        for (int n = 0; n < kNh; ++n)
          for (int o2 = 0; o2 < 4; ++o2) dst[8 + n * 4 + o2] = W2t[n][o2];
      }
    }
    bf16x8 w1b[2][kNh];  // W1 tiles (k = features, c-layout k map)
    for (int ks = 0; ks < 2; ++ks)
      for (int n = 0; n < kNh; ++n) w1b[ks][n] = cat_tiles(W1t[2 * ks][n], W1t[2 * ks + 1][n]);
    f32x4 Z1q[kNh];  // read-out: Z1q^T [hidden][token]
    f32x4 Z1[kNh];   // forward: Z1 [token][hidden]
    x4 x2qh[kNh], x2b[kNh];  // GELU(Z1q), GELU(Z1) as W2-side operand tiles
    GpT gph[kNh];            // GELU'(Z1)
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
    // GELU of both chains. fp32 with the library erf, for the recomputation, or when a hidden
    // pre-activation of the wave's step exceeds sqrt 2 in magnitude; otherwise the packed fp16
    // polynomials.
    auto gelu_lib = [&](auto& xq_out, auto& xf_out, auto& gp_out, float& xm) {
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
        if constexpr (rd) {
          xq_out[n] = S::cvt(xq);
          xm = fmaxf(xm, absmax4(xq));
        }
        if constexpr (fwd) {
          xf_out[n] = S::cvt(xf);
          xm = fmaxf(xm, absmax4(xf));
          if constexpr (F16) gp_out[n] = to_f16x4(gp);
          else gp_out[n] = gp;
        }
      }
    };
    if constexpr (F16) {
      float zm = 0.f;  // largest |pre-activation| of the lane
      for (int n = 0; n < kNh; ++n) {
        if constexpr (rd) zm = fmaxf(zm, absmax4(Z1q[n]));
        if constexpr (fwd) zm = fmaxf(zm, absmax4(Z1[n]));
      }
      // Polynomial path when every lane's largest |pre-activation| is in [2^-10, sqrt 2]: one
      // unsigned compare of the float bits (monotonic for non-negative floats; NaN fails it).
      // Below 2^-10 the GELU outputs would sit near fp16's subnormal range, so the other path
      // flags such lanes (all-zero lanes are exact).
      const bool poly = __float_as_uint(zm) - kZLoBits <= kZHiBits - kZLoBits;
      if (!__any(!poly)) {
        for (int n = 0; n < kNh; ++n) {
          if constexpr (rd) {
            const f16x4 zq = to_f16x4(Z1q[n]), tq = zq * zq;
            x2qh[n] = zq * cdf_fast_h(zq, tq);
          }
          if constexpr (fwd) {
            const f16x4 zf = to_f16x4(Z1[n]), tf = zf * zf;
            x2b[n] = zf * cdf_fast_h(zf, tf);
            gph[n] = slope_fast_h(zf, tf);
          }
        }
      } else {
        float xm = 0.f;
        gelu_lib(x2qh, x2b, gph, xm);
        // |X2|, |X2q| <= 32 keeps them and the 32-unit sums of X2q X2^T inside fp16.
        bad |= __any(!(xm <= 32.f)) || __any(zm > 0.f && zm < 0x1p-10f);
      }
    } else {
      float xm = 0.f;
      gelu_lib(x2qh, x2b, gph, xm);
    }
    x8 x2q;
    x4 n2b;
    if constexpr (rd) {
      x2q = S::cat(x2qh[0], x2qh[1]);
      // (with the previous chunk's X2^T, before the forward below replaces it)
      f32x4 n2 = S::mma32(x2tp, x2q, zero4());  // [t'][t] = sum_h X2[t'][h] X2q[t][h]
      for (int j = 0; j < 4; ++j) n2[j] = 4 * g + j <= r ? 0.f : -n2[j];
      n2b = S::cvt(n2);  // (-a is in the stored E)
    }
    if constexpr (fwd) {
      f32x4 xt[kNh];
      for (int n = 0; n < kNh; ++n) xt[n] = S::mma16(x2b[n], ident, zero4());  // X2^T [hidden][token]
      x2tp = S::cat(S::cvt(xt[0]), S::cvt(xt[1]));
      if constexpr (SPLIT) {
        const uint2 x0 = __builtin_bit_cast(uint2, x2b[0]), x1 = __builtin_bit_cast(uint2, x2b[1]);
        st16_out(&inter[((long long)c * 2 + 1) * kWaves * 64], make_uint4(x0.x, x0.y, x1.x, x1.y));
      }
    }
    x8 w2a[4];  // W2^T tiles (k = this wave's hidden units), for both products below
    for (int o2 = 0; o2 < 4; ++o2) w2a[o2] = S::cat(S::cvt(W2t[0][o2]), S::cvt(W2t[1][o2]));
    if constexpr (rd) {
      // This wave's share of O^T [out][token]: W2^T X2q^T over its hidden units, plus
      // (a E)^T striu(X2q X2^T)^T = (-a E)^T (-striu(X2q X2^T))^T with X2q X2^T summed over the
      // same units (t' > t kept), the latter as a 16x16x32 product with a zero upper k half
      // (same-shape chain).
      for (int o2 = 0; o2 < 4; ++o2) {
        const f32x4 ow = S::mma32(w2a[o2], x2q, zero4());
        sRed[(w * kSlots + 4 + o2) * 64 + l] =
            S::mma32(S::cat(S::tr(&sEp[16 * o2], kP, l), x4{}), S::cat(n2b, x4{}), ow);  // A = (-a E)^T
      }
    }
    if constexpr (fwd) {
      // Z2^T partial [out][token] over this wave's hidden units.
      for (int o2 = 0; o2 < 4; ++o2) sRed[(w * kSlots + o2) * 64 + l] = S::mma32(w2a[o2], x2tp, zero4());
    }
    if constexpr (F16 && fwd) {
      if ((c & 31) == 0) {  // the W2 slice, every 32 chunks (here, where the barrier ends the block)
        float wm = 0.f;
        for (int n = 0; n < kNh; ++n)
          for (int o2 = 0; o2 < 4; ++o2) wm = fmaxf(wm, absmax4(W2t[n][o2]));
        bad |= wave_out_of_range(wm, 0x1p-10f, 0x1p15f);
      }
    }
    // Chunk c + 1 into its slot, which no wave reads in this step (slots c and c - 1 are in use;
    // past the end the slot receives a repeat of the last chunk, which no step reads).
    st16_lds8(pdst + ((c + 1) % kRing) * (3 * kCh * kP), pf);
    pf = ld16(chunk_src(c + 3));
    __syncthreads();

    // ---------------- phase 2: cross-wave sums (fixed wave order)
    // (SPLIT: waves 4-7 have no read-out sums here; instead of repeating waves 0-3's sums they
    // store zeros to their own slots, so that every wave issues the same memory operations:
    // measured 0.847 -> 0.828 ms)
    if (fwd && SPLIT && w >= 4) st8_out(&etile[(long long)c * 8 * 64], make_uint2(0u, 0u));
    if (fwd && w < 4) {  // E^T tile w = Z2^T - V^T, stored as -a E [token][out]
      const int we = w;
      // All nine LDS reads are issued before the adds (the compiler otherwise keeps only two or
      // three of them in flight, and this phase is their latency).
      f32x4 pt[kWaves];
      for (int ww = 0; ww < kWaves; ++ww) pt[ww] = sRed[(ww * kSlots + we) * 64 + l];
      const bf16x4 vv = ld4(&sV[r * kP + 16 * we + 4 * g]);
      __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
      f32x4 s = pt[0];
      for (int ww = 1; ww < kWaves; ++ww) s = s + pt[ww];
      f32x4 e;
      for (int j = 0; j < 4; ++j) e[j] = a * ((float)vv[j] - s[j]);
      const x4 eh = S::cvt(e);
      *reinterpret_cast<x4*>(&sEc[r * kP + 16 * we + 4 * g]) = eh;
      if constexpr (SPLIT) st8_out(&etile[(long long)c * 8 * 64], __builtin_bit_cast(uint2, eh));
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
      x8 ea[2];
      for (int ko = 0; ko < 2; ++ko) {
        const typename S::elem* pe = &sEc[r * kP + 32 * ko + 4 * g];
        ea[ko] = S::cat(S::ld(pe), S::ld(pe + 16));
      }
      for (int n = 0; n < kNh; ++n) {
        f32x4 acc = zero4();
        for (int ko = 0; ko < 2; ++ko)
          acc = S::mma32(ea[ko], S::cat(S::cvt(W2x[2 * ko][n]), S::cvt(W2x[2 * ko + 1][n])), acc);
        f32x4 d1;  // -a D1
        for (int j = 0; j < 4; ++j) d1[j] = acc[j] * (float)gph[n][j];
        d1p[n] = to_bf16x4(d1);
      }
      if constexpr (SPLIT) {
        const uint2 d0 = __builtin_bit_cast(uint2, d1p[0]), d1 = __builtin_bit_cast(uint2, d1p[1]);
        st16_out(&inter[(long long)c * 2 * kWaves * 64], make_uint4(d0.x, d0.y, d1.x, d1.y));
      }
      // W1 += K^T (-a D1): A = K^T (row feature, k token; LDS transpose read), B = -a D1.
      for (int m = 0; m < 4; ++m) {
        const bf16x4 kt = tile_tr(&sK[16 * m], kP, l);
        for (int n = 0; n < kNh; ++n) W1t[m][n] = mma16(kt, d1p[n], W1t[m][n]);
      }
      // W2 += X2^T (-a E) and W2^T += (-a E)^T X2: -a E's transposed tiles give both operands.
      for (int o2 = 0; o2 < 4; ++o2) {
        const x4 e = S::tr(&sEc[16 * o2], kP, l);
        for (int n = 0; n < kNh; ++n) {
          W2t[n][o2] = S::mma16(x2b[n], e, W2t[n][o2]);
          W2x[o2][n] = S::mma16(e, x2b[n], W2x[o2][n]);
        }
      }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Step 0 has no read-out, step C no forward; the steps between have both (two per trip: even
  // steps stage from pfA, odd ones from pfB). SPLIT: forward steps only.
  if constexpr (SPLIT) {
    // At each segment end (SegPlan) the count of finished chunks is published for the
    // read-out workgroups: every wave waits for its own stores, and after the barrier one release at
    // agent scope (which writes the CU's L2 back) covers the whole workgroup's stores.
    const SegPlan plan(C);
    auto publish = [&](int done) {
      if (plan.is_end(done)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t == 0) __hip_atomic_store(sw.progress + bhs, done, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    int c = 0;
    for (; c + 1 < C; c += 2) {
      step(c, pfA, F_{}, T_{});
      publish(c + 1);
      step(c + 1, pfB, F_{}, T_{});
      publish(c + 2);
    }
    if (c < C) {
      step(c, pfA, F_{}, T_{});
      publish(c + 1);
    }
  } else {
    step(0, pfA, F_{}, T_{});
    int c = 1;
    for (; c + 1 < C; c += 2) {
      step(c, pfB, T_{}, T_{});
      step(c + 1, pfA, T_{}, T_{});
    }
    if (c < C) {
      step(c, pfB, T_{}, T_{});
      step(c + 1, pfA, T_{}, F_{});
    } else {
      step(c, pfB, T_{}, F_{});
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
  if constexpr (F16) {
    // The state must have stayed finite and W2 in range: an fp16 overflow of a -a E tile (whose
    // values the steps do not check) reaches W2 through its update and W1 through D1 as inf or NaN.
    float sm = 0.f, wm = 0.f;
    for (int m = 0; m < 4; ++m)
      for (int n = 0; n < kNh; ++n) {
        sm = fmaxf(sm, absmax4(W1t[m][n]));
        sm = fmaxf(sm, absmax4(W2x[m][n]));
        wm = fmaxf(wm, absmax4(W2t[n][m]));
      }
    bad |= wave_out_of_range(wm, 0x1p-10f, 0x1p15f) || __any(!(sm <= 3.0e38f));
    if (bad && l == 0) sBad = 1;  // (every writer stores the same value)
    __syncthreads();
    return sBad != 0;
  }
  return false;
}

// The bf16 pass as a call of its own: compiled apart from the kernel, it leaves the fp16 pass's code
// as it is when that pass is the whole kernel.
__device__ __noinline__ void mlp_chain_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out,
    MlpLds& lds) {
  mlp_chain<false>(q, k, v, w1, w2, wbs, H, N, a, o, w1_out, w2_out, lds);
}

// The fast path in three launches (split schedule):
//  1. mlp_clear zeroes the chains' flags and published-chunk counts.
//  2. mlp_fwd_fused: workgroups 0 .. BH-1 run the forward chains (one per (b, h); the fp16 pass
//     without read-outs), storing their intermediates and checkpoints and publishing their progress
//     at each segment end (SegPlan); the next n_workers workgroups take the read-out segments in order
//     (segment-major: task = segment * BH + bh, worker j takes tasks j, j + n_workers, ...), each
//     waiting until its chain has published the segment. The chain workgroups have the lowest ids,
//     so they are dispatched before any read-out workgroup, never wait, and every wait ends; a wait
//     is also bounded (then the chain is flagged and recomputed). With 48 chains on 48 CUs the
//     read-outs run beside the chains on other CUs.
//  3. mlp_fixup_bf16 recomputes in full (bf16 W2-side operands, read-outs and end states) every
//     chain that a range check flagged, in the forward chain (bit 0), in a read-out (bit 1) or by a
//     wait that timed out (bit 2).
// The single-workgroup schedule, for callers whose workspace holds only the flags (one int per
// chain): the fp16 pass with the read-outs in the chain's own steps, and only when a range check
// failed the bf16 pass over the same chain (its outputs replace the first pass's); flags[bh]
// records which.
__global__ __launch_bounds__(kWaves * 64, 1) void mlp_fwd_single(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out,
    int* __restrict__ flags) {
  __shared__ __align__(16) MlpLds lds;
  const bool bad = mlp_chain<true>(q, k, v, w1, w2, wbs, H, N, a, o, w1_out, w2_out, lds);
  if (threadIdx.x == 0) flags[blockIdx.x] = bad ? 1 : 0;
  if (bad) {
    __syncthreads();  // every wave is done with the first pass's shared memory
    mlp_chain_bf16(q, k, v, w1, w2, wbs, H, N, a, o, w1_out, w2_out, lds);
  }
}

__global__ void mlp_clear(int* __restrict__ flags, int* __restrict__ progress, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    flags[i] = 0;
    progress[i] = 0;
  }
}

struct MlpReadoutLds {
  bf16 kq[2][2][kCh * kP];         // [parity][K, Q][token][feature]
  f16 e[2][kCh * kP];              // [parity] -a E [token][out]
  f32x4 red[2][kWaves * 4 * 64];   // [parity] O^T partial tiles, lane-private
};
struct MlpChunkRegs {
  uint4 kq;      // this thread's 16-byte piece of the K or Q tile
  uint4 d1, x2;  // -a D1 and X2 tiles of the thread's wave
  uint2 e;       // -a E fragment of tile w & 3
};

// Reads out segment seg of chain bh; returns true (in every thread of a wave that saw it) when a
// value left the range its fp16 operands allow.
__device__ __forceinline__ bool readout_segment(
    int seg, int bh, const bf16* __restrict__ q, const bf16* __restrict__ k, int H, int N, float a,
    bf16* __restrict__ o, const MlpSplitWs& sw, MlpReadoutLds& lds) {
  using S = W2Side<true>;
  const int b = bh / H, h = bh % H;
  const int t = threadIdx.x, w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const int C = N / kCh;
  const SegPlan plan(C);
  const int c0 = plan.lo(seg), c1 = plan.hi(seg);
  const long long ts = (long long)H * kD;
  const long long head0 = (long long)b * N * ts + (long long)h * kD;

  f32x4 W1t[4][kNh], W2t[kNh][4];  // layouts as in mlp_chain
  {
    const f32x4* ck = sw.ckpt + (long long)bh * mlp_ckpt_f32x4(C) + (long long)seg * kWaves * 64 * 16 + 16 * t;
    for (int m = 0; m < 4; ++m)
      for (int n = 0; n < kNh; ++n) W1t[m][n] = ck[m * kNh + n];
    for (int n = 0; n < kNh; ++n)
      for (int o2 = 0; o2 < 4; ++o2) W2t[n][o2] = ck[8 + n * 4 + o2];
  }
  const uint4* inter = sw.inter + (long long)bh * mlp_inter_uint4(C) + t;
  const uint2* etile = sw.etile + (long long)bh * mlp_etile_uint2(C) + 64 * (w & 3) + l;
  // Threads 0..255 move one 16-byte piece of K or Q per chunk; 256..511 repeat them (same source and
  // LDS address), so that every wave issues the same loads.
  const int u = t & 255, prow = (u & 127) >> 3, pcol = (u & 7) * 8, which = u >> 7;
  const bf16* psrc = (which == 0 ? k : q) + head0 + prow * ts + pcol;
  const int poff = which * kCh * kP + prow * kP + pcol;  // within lds.kq[parity]
  auto load = [&](int cc, MlpChunkRegs& d) {  // chunk indices past the segment repeat its last chunk
    cc = min(cc, c1 - 1);
    d.kq = ld16(psrc + (long long)cc * kCh * ts);
    const uint4* pi = inter + (long long)cc * 2 * kWaves * 64;
    d.d1 = pi[0];
    d.x2 = pi[kWaves * 64];
    d.e = etile[(long long)cc * 8 * 64];
  };
  auto to_lds = [&](int parity, const MlpChunkRegs& d) {
    st16_lds8(&lds.kq[parity][0][0] + poff, d.kq);
    *reinterpret_cast<uint2*>(&lds.e[parity][r * kP + 16 * (w & 3) + 4 * g]) = d.e;
  };
  f16x4 ident;  // identity tile as the B operand: lane holds I[4g + i][r]
  for (int i = 0; i < 4; ++i) ident[i] = (f16)(4 * g + i == r ? 1.f : 0.f);

  MlpChunkRegs set0, set1;  // data of the even and of the odd chunks
  load(c0, set0);
  load(c0 + 1, set1);
  to_lds(0, set0);  // c0 is even (segment lengths are)
  __syncthreads();
  bool bad = false;

  auto step = [&](const int c, MlpChunkRegs& cur, MlpChunkRegs& nxt) {
    const int p = c & 1;
    const bf16* sK = lds.kq[p][0];
    const bf16* sQ = lds.kq[p][1];
    const f16* sE = lds.e[p];
    f32x4* const sRed = lds.red[p];
    bf16x4 d1p[kNh];
    f16x4 x2b[kNh];
    {
      const uint2 d0 = make_uint2(cur.d1.x, cur.d1.y), d1 = make_uint2(cur.d1.z, cur.d1.w);
      d1p[0] = __builtin_bit_cast(bf16x4, d0);
      d1p[1] = __builtin_bit_cast(bf16x4, d1);
      const uint2 x0 = make_uint2(cur.x2.x, cur.x2.y), x1 = make_uint2(cur.x2.z, cur.x2.w);
      x2b[0] = __builtin_bit_cast(f16x4, x0);
      x2b[1] = __builtin_bit_cast(f16x4, x1);
    }
    // The chunk's state update (the forward chain's phase 3 products): W1 += K^T (-a D1),
    // W2 += X2^T (-a E).
    for (int m = 0; m < 4; ++m) {
      const bf16x4 kt = tile_tr(&sK[16 * m], kP, l);
      for (int n = 0; n < kNh; ++n) W1t[m][n] = mma16(kt, d1p[n], W1t[m][n]);
    }
    for (int o2 = 0; o2 < 4; ++o2) {
      const f16x4 e = S::tr(&sE[16 * o2], kP, l);
      for (int n = 0; n < kNh; ++n) W2t[n][o2] = S::mma16(x2b[n], e, W2t[n][o2]);
    }
    // Read-out with the end state.
    bf16x8 w1b[2][kNh];
    for (int ks = 0; ks < 2; ++ks)
      for (int n = 0; n < kNh; ++n) w1b[ks][n] = cat_tiles(W1t[2 * ks][n], W1t[2 * ks + 1][n]);
    f32x4 mt = zero4();  // M[t'][t] = k_t' . q_t, kept for t' > t
    for (int ks = 0; ks < 2; ++ks)
      mt = mma32(cat8(ld4(&sK[r * kP + 32 * ks + 4 * g]), ld4(&sK[r * kP + 32 * ks + 16 + 4 * g])),
                 cat8(ld4(&sQ[r * kP + 32 * ks + 4 * g]), ld4(&sQ[r * kP + 32 * ks + 16 + 4 * g])), mt);
    for (int j = 0; j < 4; ++j) mt[j] = 4 * g + j <= r ? 0.f : -mt[j];
    const bf16x4 mb = to_bf16x4(mt);  // -M (the stored D1 is -a D1)
    f32x4 Z1q[kNh];  // Z1q^T [hidden][token] = W1^T Q^T + (-a D1)^T (-M)
    for (int n = 0; n < kNh; ++n) {
      f32x4 z = zero4();
      for (int ks = 0; ks < 2; ++ks) {
        const bf16* pq = &sQ[r * kP + 32 * ks + 4 * g];
        z = mma32(w1b[ks][n], cat8(ld4(pq), ld4(pq + 16)), z);
      }
      Z1q[n] = mma32(cat8(d1p[n], bf16x4{}), cat8(mb, bf16x4{}), z);
    }
    f16x4 x2qh[kNh];
    float zm = 0.f;
    for (int n = 0; n < kNh; ++n) zm = fmaxf(zm, absmax4(Z1q[n]));
    const bool poly = __float_as_uint(zm) - kZLoBits <= kZHiBits - kZLoBits;
    if (!__any(!poly)) {
      for (int n = 0; n < kNh; ++n) {
        const f16x4 zq = to_f16x4(Z1q[n]), tq = zq * zq;
        x2qh[n] = zq * cdf_fast_h(zq, tq);
      }
    } else {
      float xm = 0.f;
      for (int n = 0; n < kNh; ++n) {
        f32x4 xq;
        for (int j = 0; j < 4; ++j) xq[j] = Z1q[n][j] * cdf_lib(Z1q[n][j]);
        x2qh[n] = to_f16x4(xq);
        xm = fmaxf(xm, absmax4(xq));
      }
      bad |= __any(!(xm <= 32.f)) || __any(zm > 0.f && zm < 0x1p-10f);
    }
    const f16x8 x2q = cat8h(x2qh[0], x2qh[1]);
    f32x4 xt[kNh];
    for (int n = 0; n < kNh; ++n) xt[n] = S::mma16(x2b[n], ident, zero4());  // X2^T [hidden][token]
    const f16x8 x2tp = cat8h(to_f16x4(xt[0]), to_f16x4(xt[1]));
    f32x4 n2 = S::mma32(x2tp, x2q, zero4());  // [t'][t] = sum_h X2[t'][h] X2q[t][h]
    for (int j = 0; j < 4; ++j) n2[j] = 4 * g + j <= r ? 0.f : -n2[j];
    const f16x4 n2b = to_f16x4(n2);
    for (int o2 = 0; o2 < 4; ++o2) {
      const f16x8 w2a = cat8h(to_f16x4(W2t[0][o2]), to_f16x4(W2t[1][o2]));
      const f32x4 ow = S::mma32(w2a, x2q, zero4());
      sRed[(w * 4 + o2) * 64 + l] = S::mma32(cat8h(S::tr(&sE[16 * o2], kP, l), f16x4{}), cat8h(n2b, f16x4{}), ow);
    }
    // Chunk c + 1 into the other parity's buffers (last read in step c - 1), chunk c + 2 into cur.
    to_lds(p ^ 1, nxt);
    load(c + 2, cur);
    __syncthreads();
    if (w >= 4) {  // O^T tile w - 4 of chunk c = the sum of the waves' shares (fixed order)
      const int o4 = w - 4;
      f32x4 pt[kWaves];
      for (int ww = 0; ww < kWaves; ++ww) pt[ww] = sRed[(ww * 4 + o4) * 64 + l];
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      f32x4 sum = pt[0];
      for (int ww = 1; ww < kWaves; ++ww) sum = sum + pt[ww];
      const long long tok = head0 + (long long)c * kCh * ts;
      *reinterpret_cast<bf16x4*>(o + tok + r * ts + 16 * o4 + 4 * g) = to_bf16x4(sum);
    }
  };
  int c = c0;
  for (; c + 1 < c1; c += 2) {
    step(c, set0, set1);
    step(c + 1, set1, set0);
  }
  if (c < c1) step(c, set0, set1);
  return bad;
}

union MlpFusedLds {
  MlpLds chain;
  MlpReadoutLds readout;
};

__global__ __launch_bounds__(kWaves * 64, 1) void mlp_fwd_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out,
    int* __restrict__ flags, MlpSplitWs sw, int BH) {
  __shared__ __align__(16) MlpFusedLds lds;
  __shared__ int s_wait;
  if ((int)blockIdx.x < BH) {
    const bool bad = mlp_chain<true, true>(q, k, v, w1, w2, wbs, H, N, a, o, w1_out, w2_out, lds.chain, sw);
    if (bad && threadIdx.x == 0) atomicOr(flags + blockIdx.x, 1);
    return;
  }
  const int C = N / kCh;
  const SegPlan plan(C);
  const int tasks = plan.count() * BH;
  const int workers = gridDim.x - BH;
  // Bound on one wait (s_sleep polls of about a microsecond): far beyond the chain's own time.
  const int max_polls = 64 * C + (1 << 20);
  for (int task = blockIdx.x - BH; task < tasks; task += workers) {
    const int seg = task / BH, bh = task % BH;
    const int need = plan.hi(seg);
    if (threadIdx.x == 0) {
      int polls = 0;
      // Relaxed polls (an acquire per poll would invalidate the L2 each time); one acquire fence
      // after the wait orders the loads of the published data.
      while (__hip_atomic_load(sw.progress + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need &&
             polls < max_polls) {
        __builtin_amdgcn_s_sleep(16);
        ++polls;
      }
      // The polling thread's acquire pairs with the chain's release; the barrier orders the other
      // waves after it, and each wave's own acquire fence drops its stale cache lines.
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      s_wait = polls < max_polls ? 0 : 1;
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (s_wait) {
      if (threadIdx.x == 0) atomicOr(flags + bh, 4);
    } else {
      const bool bad = readout_segment(seg, bh, q, k, H, N, a, o, sw, lds.readout);
      if (bad && lane_id() == 0) atomicOr(flags + bh, 2);
    }
    __syncthreads();  // the workgroup's shared memory is free for the next task
  }
}

// Launch 3: the flagged chains, recomputed in full with bf16 W2-side operands (read-outs and end
// states); every other workgroup returns at once.
__global__ __launch_bounds__(kWaves * 64, 1) void mlp_fixup_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out,
    const int* __restrict__ flags) {
  __shared__ __align__(16) MlpLds lds;
  if (flags[blockIdx.x] == 0) return;
  mlp_chain_bf16(q, k, v, w1, w2, wbs, H, N, a, o, w1_out, w2_out, lds);
}


// ---------------------------------------------------------------- wide inner model, matrix cores
// The layer for bf16 I/O, D = 64, b = 16 and hidden widths of 2 to 4 blocks of 256 units (ViT^3
// review, design-space study: a wider inner model). One workgroup of 8 waves per (batch, head), as
// above, but the state (W1 and W2, 2 D Dh fp32 values) no longer fits in registers: it lives in the
// workspace in fp32, in layouts chosen so that each lane moves its MFMA operands and update tiles as
// 16-byte pieces: W1^T [Dh][D], W2 [Dh][D] and a second copy W2^T [D][Dh] (the operand layouts of
// X2 W2 and of E W2^T differ). In each block of 256 hidden units wave w owns units [32w, 32w + 32),
// and every state element is loaded and stored by the same lane (initial copy, operands, updates,
// final copy), so the waves share no state. Per chunk, with the start state (W1, W2) and the read-
// out in the start-state dual form (one state per chunk step):
//   forward, per block:  Z1 = K W1; X2 = GELU(Z1) and GELU'(Z1) kept in registers; the Z2^T partial
//                        accumulates W2^T X2^T over the blocks;
//   cross-wave sum:      -a E = a (V - Z2)  (LDS, fixed wave order);
//   per block:           -a D1 = ((-a E) W2^T) * GELU'(Z1);
//                        Z1q^T = W1^T Q^T + (-a D1)^T tril(Q K^T)^T, X2q = GELU(Z1q),
//                        O^T partial += W2^T X2q^T + (-a E)^T tril(X2q X2^T)^T;
//   cross-wave sum:      O;
//   update, per block:   W1 += K^T (-a D1), W2 += X2^T (-a E) (both copies).
// tril keeps t' <= t. All products take bf16 operands (fp32's exponent range: no range checks) and
// accumulate in fp32; GELU is the erf form in fp32 (cdf_as: erf within 1.5e-7).
constexpr int kWideBlock = 256;  // hidden units per block (8 waves x 32)

// GELU and GELU' in fp32 without the library erf (whose range branches and long polynomials would
// dominate this kernel's instruction count): erf by Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26, erf(u) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^(-u^2) with
// t = 1 / (1 + p u), u >= 0 (absolute error at most 1.5e-7), extended as an odd function. With
// u = |x| / sqrt 2 the factor e^(-u^2) = e^(-x^2 / 2) also gives the normal density of
// GELU'(x) = Phi(x) + x phi(x). One exp2, one reciprocal, no branch.
constexpr float kAsP = 0.3275911f, kAsA1 = 0.254829592f, kAsA2 = -0.284496736f, kAsA3 = 1.421413741f,
                kAsA4 = -1.453152027f, kAsA5 = 1.061405429f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;
__device__ __forceinline__ float cdf_as(float x, float& e) {  // Phi(x); e = e^(-x^2 / 2)
  e = __builtin_amdgcn_exp2f(x * x * kNegHalfLog2e);
  const float t = __builtin_amdgcn_rcpf(fmaf(kAsP, fabsf(x) * kInvSqrt2, 1.f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, kAsA5, kAsA4), kAsA3), kAsA2), kAsA1);
  return 0.5f + copysignf(0.5f * fmaf(-poly, e, 1.f), x);
}

__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4f(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

template <int NB>
__global__ __launch_bounds__(kWaves * 64, 1) void mlp_fwd_wide(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N,
    float a, bf16* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out,
    float* __restrict__ ws) {
  constexpr int Dh = NB * kWideBlock;
  __shared__ __align__(16) bf16 sKVQ[2][3][kCh * kP];
  __shared__ __align__(16) bf16 sE[kCh * kP];                 // -a E [token][out]
  __shared__ __align__(16) f32x4 sRed[kWaves * kSlots * 64];  // lane-private partial tiles

  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int w = wave_id(), l = lane_id(), r = l & 15, g = l >> 4;
  const long long ts = (long long)H * kD;
  const float* W1g = w1 + b * wbs + (long long)h * kD * Dh;  // [D][Dh]
  const float* W2g = w2 + b * wbs + (long long)h * Dh * kD;  // [Dh][D]
  float* W1T = ws + (long long)bh * 3 * kD * Dh;             // [Dh][D]
  float* W2s = W1T + kD * Dh;                                // [Dh][D]
  float* W2T = W2s + kD * Dh;                                // [D][Dh]

  // The lane's state tiles (the same elements its operand loads and updates touch):
  //   W1 [feature 16m + 4g + j][unit u0 + 16n + r]  at W1T[(u0 + 16n + r) D + 16m + 4g + j]
  //   W2 [unit u0 + 16n + 4g + j][out 16o + r]      at W2T[(16o + r) Dh + u0 + 16n + 4g + j]
  //   W2 [unit u0 + 16n + r][out 16o + 4g + j]      at W2s[(u0 + 16n + r) D + 16o + 4g + j]
  for (int nb = 0; nb < NB; ++nb) {
    const int u0 = nb * kWideBlock + kHw * w;
    for (int n = 0; n < kNh; ++n) {
      const int u = u0 + 16 * n + r;
      for (int m = 0; m < 4; ++m) {
        f32x4 t1, t2;
        for (int j = 0; j < 4; ++j) {
          t1[j] = W1g[(16 * m + 4 * g + j) * Dh + u];
          t2[j] = W2g[(u0 + 16 * n + 4 * g + j) * kD + 16 * m + r];
        }
        st4f(W1T + (long long)u * kD + 16 * m + 4 * g, t1);
        st4f(W2T + (long long)(16 * m + r) * Dh + u0 + 16 * n + 4 * g, t2);
        st4f(W2s + (long long)u * kD + 16 * m + 4 * g, ld4f(W2g + (long long)u * kD + 16 * m + 4 * g));
      }
    }
  }
  const bf16x4 ident = identity_b(r, g);

  const int C = N / kCh;
  const long long head0 = (long long)b * N * ts + (long long)h * kD;
  // Staging: threads 0..383 each move one 16-byte piece of K, V or Q (16 rows x 8 pieces each), one
  // chunk ahead through a register.
  const int t = threadIdx.x;
  const int prow = (t & 127) >> 3, pcol = (t & 7) * 8, which = t >> 7;
  const bf16* psrc = (t < 128 ? k : (t < 256 ? v : q)) + head0 + prow * ts + pcol;
  if (t < 384) st16_lds8(&sKVQ[0][which][prow * kP + pcol], ld16(psrc));
  __syncthreads();

  for (int c = 0; c < C; ++c) {
    const int cb = c & 1;
    uint4 pf = make_uint4(0u, 0u, 0u, 0u);
    if (t < 384 && c + 1 < C) pf = ld16(psrc + (long long)(c + 1) * kCh * ts);
    const bf16* sK = sKVQ[cb][0];
    const bf16* sV = sKVQ[cb][1];
    const bf16* sQ = sKVQ[cb][2];

    // ---------------- forward
    bf16x4 x2b[NB][kNh];  // X2 [token 4g + j][unit 16n + r]
    bf16x8 x2t[NB];       // X2^T as a B operand (k = units, n = token)
    f32x4 gpr[NB][kNh];   // GELU'(Z1), same layout as X2
    f32x4 zacc[4];        // Z2^T partial [out][token] over this wave's units
    for (int o2 = 0; o2 < 4; ++o2) zacc[o2] = zero4();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int u0 = nb * kWideBlock + kHw * w;
      for (int n = 0; n < kNh; ++n) {
        const float* p = W1T + (long long)(u0 + 16 * n + r) * kD + 4 * g;
        f32x4 z = zero4();
        for (int ks = 0; ks < 2; ++ks) {
          const bf16* pk = &sK[r * kP + 32 * ks + 4 * g];
          z = mma32(cat8(ld4(pk), ld4(pk + 16)), cat_tiles(ld4f(p + 32 * ks), ld4f(p + 32 * ks + 16)), z);
        }
        f32x4 xf, gp;
        for (int j = 0; j < 4; ++j) {
          float e;
          const float x = z[j], cdf = cdf_as(x, e);
          xf[j] = x * cdf;
          gp[j] = fmaf(x * e, kInvSqrt2Pi, cdf);
        }
        x2b[nb][n] = to_bf16x4(xf);
        gpr[nb][n] = gp;
      }
      f32x4 xt[kNh];
      for (int n = 0; n < kNh; ++n) xt[n] = mma16(x2b[nb][n], ident, zero4());  // [unit][token]
      x2t[nb] = cat_tiles(xt[0], xt[1]);
      for (int o2 = 0; o2 < 4; ++o2) {
        const float* p = W2T + (long long)(16 * o2 + r) * Dh + u0 + 4 * g;
        zacc[o2] = mma32(cat_tiles(ld4f(p), ld4f(p + 16)), x2t[nb], zacc[o2]);
      }
    }
    for (int o2 = 0; o2 < 4; ++o2) sRed[(w * kSlots + o2) * 64 + l] = zacc[o2];
    __syncthreads();
    if (w < 4) {  // E^T tile w = Z2^T - V^T, stored as -a E [token][out]
      f32x4 pt[kWaves];
      for (int ww = 0; ww < kWaves; ++ww) pt[ww] = sRed[(ww * kSlots + w) * 64 + l];
      const bf16x4 vv = ld4(&sV[r * kP + 16 * w + 4 * g]);
      f32x4 s = pt[0];
      for (int ww = 1; ww < kWaves; ++ww) s = s + pt[ww];
      f32x4 e;
      for (int j = 0; j < 4; ++j) e[j] = a * ((float)vv[j] - s[j]);
      *reinterpret_cast<bf16x4*>(&sE[r * kP + 16 * w + 4 * g]) = to_bf16x4(e);
    }
    __syncthreads();

    // ---------------- backward and read-out
    bf16x8 ea[2];  // -a E rows (k = outputs)
    for (int ko = 0; ko < 2; ++ko) {
      const bf16* pe = &sE[r * kP + 32 * ko + 4 * g];
      ea[ko] = cat8(ld4(pe), ld4(pe + 16));
    }
    bf16x4 et[4];  // (-a E)^T tiles: lane (r, g) holds -a E[token 4g + j][out 16o + r]
    for (int o2 = 0; o2 < 4; ++o2) et[o2] = tile_tr(&sE[16 * o2], kP, l);
    // M[t'][t] = k_t' . q_t, kept for t' <= t
    f32x4 mt = zero4();
    for (int ks = 0; ks < 2; ++ks)
      mt = mma32(cat8(ld4(&sK[r * kP + 32 * ks + 4 * g]), ld4(&sK[r * kP + 32 * ks + 16 + 4 * g])),
                 cat8(ld4(&sQ[r * kP + 32 * ks + 4 * g]), ld4(&sQ[r * kP + 32 * ks + 16 + 4 * g])), mt);
    for (int j = 0; j < 4; ++j) mt[j] = 4 * g + j <= r ? mt[j] : 0.f;
    const bf16x4 mb = to_bf16x4(mt);
    bf16x4 d1b[NB][kNh];  // -a D1 [token][unit]
    f32x4 oacc[4];        // O^T partial [out][token]
    for (int o2 = 0; o2 < 4; ++o2) oacc[o2] = zero4();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int u0 = nb * kWideBlock + kHw * w;
      f32x4 zq[kNh];
      for (int n = 0; n < kNh; ++n) {
        // -a dX2 = (-a E) W2^T: B = W2 [k = out][n = unit]
        const float* p2 = W2s + (long long)(u0 + 16 * n + r) * kD + 4 * g;
        f32x4 acc = zero4();
        for (int ko = 0; ko < 2; ++ko)
          acc = mma32(ea[ko], cat_tiles(ld4f(p2 + 32 * ko), ld4f(p2 + 32 * ko + 16)), acc);
        f32x4 d1;
        for (int j = 0; j < 4; ++j) d1[j] = acc[j] * gpr[nb][n][j];
        d1b[nb][n] = to_bf16x4(d1);
        // Z1q^T = W1^T Q^T + (-a D1)^T M: A = W1 tiles as W1^T (rows = units), B = Q rows; the
        // correction as a 16x16x32 product with a zero upper k half (same-shape chain)
        const float* p1 = W1T + (long long)(u0 + 16 * n + r) * kD + 4 * g;
        f32x4 z = zero4();
        for (int ks = 0; ks < 2; ++ks) {
          const bf16* pq = &sQ[r * kP + 32 * ks + 4 * g];
          z = mma32(cat_tiles(ld4f(p1 + 32 * ks), ld4f(p1 + 32 * ks + 16)), cat8(ld4(pq), ld4(pq + 16)), z);
        }
        zq[n] = mma32(cat8(d1b[nb][n], bf16x4{}), cat8(mb, bf16x4{}), z);  // [unit][token]
      }
      bf16x4 xq[kNh];
      for (int n = 0; n < kNh; ++n) {
        f32x4 x;
        for (int j = 0; j < 4; ++j) {
          float e;
          x[j] = zq[n][j] * cdf_as(zq[n][j], e);
        }
        xq[n] = to_bf16x4(x);
      }
      const bf16x8 x2q = cat8(xq[0], xq[1]);  // B operand (k = units, n = token)
      f32x4 n2 = mma32(x2t[nb], x2q, zero4());  // [t'][t] = sum over the units of X2[t'] X2q[t]
      for (int j = 0; j < 4; ++j) n2[j] = 4 * g + j <= r ? n2[j] : 0.f;
      const bf16x4 n2b = to_bf16x4(n2);
      for (int o2 = 0; o2 < 4; ++o2) {
        const float* p = W2T + (long long)(16 * o2 + r) * Dh + u0 + 4 * g;
        oacc[o2] = mma32(cat_tiles(ld4f(p), ld4f(p + 16)), x2q, oacc[o2]);
        oacc[o2] = mma32(cat8(et[o2], bf16x4{}), cat8(n2b, bf16x4{}), oacc[o2]);
      }
    }
    for (int o2 = 0; o2 < 4; ++o2) sRed[(w * kSlots + 4 + o2) * 64 + l] = oacc[o2];
    __syncthreads();
    if (w >= 4) {  // O^T tile w - 4 = sum of the waves' shares
      const int o4 = w - 4;
      f32x4 pt[kWaves];
      for (int ww = 0; ww < kWaves; ++ww) pt[ww] = sRed[(ww * kSlots + 4 + o4) * 64 + l];
      f32x4 s = pt[0];
      for (int ww = 1; ww < kWaves; ++ww) s = s + pt[ww];
      const long long tok = head0 + (long long)c * kCh * ts;
      *reinterpret_cast<bf16x4*>(o + tok + r * ts + 16 * o4 + 4 * g) = to_bf16x4(s);
    }

    // ---------------- update (lane-private state tiles)
    bf16x4 kt[4];  // K^T tiles: lane (r, g) holds K[token 4g + j][feature 16m + r]
    for (int m = 0; m < 4; ++m) kt[m] = tile_tr(&sK[16 * m], kP, l);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int u0 = nb * kWideBlock + kHw * w;
      for (int n = 0; n < kNh; ++n) {
        float* p1 = W1T + (long long)(u0 + 16 * n + r) * kD + 4 * g;
        for (int m = 0; m < 4; ++m) st4f(p1 + 16 * m, mma16(kt[m], d1b[nb][n], ld4f(p1 + 16 * m)));
        for (int o2 = 0; o2 < 4; ++o2) {
          float* pa = W2T + (long long)(16 * o2 + r) * Dh + u0 + 16 * n + 4 * g;
          st4f(pa, mma16(x2b[nb][n], et[o2], ld4f(pa)));
          float* pb = W2s + (long long)(u0 + 16 * n + r) * kD + 16 * o2 + 4 * g;
          st4f(pb, mma16(et[o2], x2b[nb][n], ld4f(pb)));
        }
      }
    }
    if (t < 384 && c + 1 < C) st16_lds8(&sKVQ[cb ^ 1][which][prow * kP + pcol], pf);
    __syncthreads();
  }

  // End states from the lane's own tiles.
  for (int nb = 0; nb < NB; ++nb) {
    const int u0 = nb * kWideBlock + kHw * w;
    for (int n = 0; n < kNh; ++n) {
      const int u = u0 + 16 * n + r;
      for (int m = 0; m < 4; ++m) {
        if (w1_out) {
          const f32x4 t1 = ld4f(W1T + (long long)u * kD + 16 * m + 4 * g);
          for (int j = 0; j < 4; ++j) w1_out[(long long)bh * kD * Dh + (16 * m + 4 * g + j) * Dh + u] = t1[j];
        }
        if (w2_out)
          st4f(w2_out + (long long)bh * Dh * kD + (long long)u * kD + 16 * m + 4 * g,
               ld4f(W2s + (long long)u * kD + 16 * m + 4 * g));
      }
    }
  }
}

// ---------------------------------------------------------------- any size, fp32 arithmetic
// The same layer for every other supported size (D in {16, 32, 64}, Dh a multiple of 64 up to
// 1024, b in {16, 32, 64}) and for fp32 I/O, in plain fp32 FMA arithmetic (the exact erf GELU of
// the C library), one workgroup per (batch, head). Each chunk is computed from its start state
// (W1, W2) in the dual form of the per-token read-out:
//   Z1 = K W1, X2 = GELU(Z1), E = X2 W2 - V, D1 = (E W2^T) * GELU'(Z1)
//   Z1q = Q W1 - a tril(Q K^T) D1, X2q = GELU(Z1q), O = X2q W2 - a tril(X2q X2^T) E
//   W1 -= a K^T D1, W2 -= a X2^T E
// (tril keeps j <= i, so token i sees the gradients of tokens j <= i). The state lives in the
// workspace; so do the [Dh, b] intermediates, stored hidden-unit-major so that a thread owning a
// hidden unit reads and writes its b values contiguously. Work is laid out so that the state
// streams once per pass: a thread owns hidden unit j for the passes over W1's column j and W2's row
// j (Z1 and Q W1; D1, X2q and the W1 update; the W2 update), and the contractions over the hidden
// units (E, O) give each thread an output feature and a share of the hidden units, the partial sums
// reduced through LDS in a fixed order. The chunk's K, V, Q, E and the masked b x b products are in
// LDS. Per chain the workspace holds 2 D Dh + 4 b Dh floats.
constexpr int kGenThreads = 256;
constexpr int kGenTB = 16;  // tokens per block of the E and O partial sums

__device__ __forceinline__ float gelu_f32(float x) { return x * cdf_lib(x); }
__device__ __forceinline__ float gelu_prime_f32(float x) {
  return cdf_lib(x) + x * expf(-0.5f * x * x) * 0.39894228040143267794f;  // Phi(x) + x phi(x)
}
template <class T>
__device__ __forceinline__ float load_io(const T* p) { return (float)*p; }
template <class T>
__device__ __forceinline__ void store_io(T* p, float v) { *p = (T)v; }

template <class T, int D, int CH>
__global__ __launch_bounds__(kGenThreads) void mlp_fwd_generic(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ w2, long long wbs, int H, int N, int Dh,
    float a, T* __restrict__ o, float* __restrict__ w1_out, float* __restrict__ w2_out,
    float* __restrict__ ws) {
  // DP: LDS row pitch; 16-byte rows, so that the unrolled broadcast reads of a row vectorise
  constexpr int DP = D + 4, G = kGenThreads / D;  // G hidden-unit groups of the E / O partial sums
  __shared__ __align__(16) float sK[CH * DP], sV[CH * DP], sQ[CH * DP], sE[CH * DP];
  __shared__ float sM[CH * (CH + 1)], sN2[CH * (CH + 1)];
  __shared__ float sPart[kGenThreads * (kGenTB + 1)];
  const int bh = blockIdx.x, b = bh / H, h = bh % H, tid = threadIdx.x;
  const long long DDh = (long long)D * Dh, BDh = (long long)CH * Dh;
  float* W1 = ws + (long long)bh * (2 * DDh + 4 * BDh);  // [D][Dh]
  float* W2 = W1 + DDh;                                  // [Dh][D]
  float* X2T = W2 + DDh;                                 // [Dh][CH]: GELU(Z1)
  float* GPT = X2T + BDh;                                // [Dh][CH]: GELU'(Z1)
  float* XQT = GPT + BDh;                                // [Dh][CH]: Q W1, then X2q
  float* D1T = XQT + BDh;                                // [Dh][CH]: D1
  const float* W1g = w1 + b * wbs + (long long)h * DDh;
  const float* W2g = w2 + b * wbs + (long long)h * DDh;
  for (long long e = tid; e < DDh; e += kGenThreads) {
    W1[e] = W1g[e];
    W2[e] = W2g[e];
  }
  const long long ts = (long long)H * D;
  const long long head0 = (long long)b * N * ts + (long long)h * D;
  const int f = tid % D, jg = tid / D;  // output feature and hidden-unit group of the partial sums

  // P[t][f] = sum_j XT[j][tb + t] W2[j][f] over the chunk's tokens tb .. tb + 15, reduced over the
  // groups in order; calls out(t, f, value) for each.
  auto hidden_contraction = [&](const float* XT, auto out) {
    for (int tb = 0; tb < CH; tb += kGenTB) {
      float acc[kGenTB];
#pragma unroll
      for (int t = 0; t < kGenTB; ++t) acc[t] = 0.f;
      for (int j = jg; j < Dh; j += G) {
        const float w = W2[(long long)j * D + f];
        const f32x4* x = reinterpret_cast<const f32x4*>(XT + (long long)j * CH + tb);
#pragma unroll
        for (int t4 = 0; t4 < kGenTB / 4; ++t4) {
          const f32x4 xv = x[t4];
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[4 * t4 + u] = fmaf(xv[u], w, acc[4 * t4 + u]);
        }
      }
#pragma unroll
      for (int t = 0; t < kGenTB; ++t) sPart[tid * (kGenTB + 1) + t] = acc[t];
      __syncthreads();
      for (int e = tid; e < kGenTB * D; e += kGenThreads) {
        const int t = e / D, ff = e % D;
        float sum = 0.f;
        for (int g = 0; g < G; ++g) sum += sPart[(g * D + ff) * (kGenTB + 1) + t];
        out(tb + t, ff, sum);
      }
      __syncthreads();
    }
  };

  __syncthreads();
  for (int c0 = 0; c0 < N; c0 += CH) {
    for (int e = tid; e < CH * D; e += kGenThreads) {
      const int t = e / D, ff = e % D;
      const long long off = head0 + (long long)(c0 + t) * ts + ff;
      sK[t * DP + ff] = load_io(k + off);
      sV[t * DP + ff] = load_io(v + off);
      sQ[t * DP + ff] = load_io(q + off);
    }
    __syncthreads();
    // Z1 = K W1 (X2, GELU'), Q W1, column by column of W1; M = tril(Q K^T)
    for (int j = tid; j < Dh; j += kGenThreads) {
      float wc[D];
#pragma unroll
      for (int ff = 0; ff < D; ++ff) wc[ff] = W1[(long long)ff * Dh + j];
#pragma unroll 1
      for (int t = 0; t < CH; ++t) {
        float z = 0.f, zq = 0.f;
#pragma unroll
        for (int ff = 0; ff < D; ++ff) {
          z = fmaf(sK[t * DP + ff], wc[ff], z);
          zq = fmaf(sQ[t * DP + ff], wc[ff], zq);
        }
        X2T[(long long)j * CH + t] = gelu_f32(z);
        GPT[(long long)j * CH + t] = gelu_prime_f32(z);
        XQT[(long long)j * CH + t] = zq;
      }
    }
    for (int e = tid; e < CH * CH; e += kGenThreads) {
      const int i = e / CH, u = e % CH;
      float m = 0.f;
      if (u <= i)
        for (int ff = 0; ff < D; ++ff) m = fmaf(sQ[i * DP + ff], sK[u * DP + ff], m);
      sM[i * (CH + 1) + u] = m;
    }
    __syncthreads();
    // E = X2 W2 - V
    hidden_contraction(X2T, [&](int t, int ff, float sum) { sE[t * DP + ff] = sum - sV[t * DP + ff]; });
    // per hidden unit j: D1 = (E W2^T) * GELU'(Z1); X2q = GELU(Q W1 - a M D1); W1[:, j] -= a K^T D1
    for (int j = tid; j < Dh; j += kGenThreads) {
      float* d1 = D1T + (long long)j * CH;
      float* xq = XQT + (long long)j * CH;
      {
        float wr[D];
#pragma unroll
        for (int ff = 0; ff < D; ++ff) wr[ff] = W2[(long long)j * D + ff];
#pragma unroll 1
        for (int t = 0; t < CH; ++t) {
          float g = 0.f;
#pragma unroll
          for (int ff = 0; ff < D; ++ff) g = fmaf(sE[t * DP + ff], wr[ff], g);
          d1[t] = g * GPT[(long long)j * CH + t];
        }
      }
#pragma unroll 1
      for (int t = 0; t < CH; ++t) {
        float corr = 0.f;
        for (int u = 0; u <= t; ++u) corr = fmaf(sM[t * (CH + 1) + u], d1[u], corr);
        xq[t] = gelu_f32(fmaf(-a, corr, xq[t]));
      }
      float gk[D];
#pragma unroll
      for (int ff = 0; ff < D; ++ff) gk[ff] = 0.f;
#pragma unroll 1
      for (int t = 0; t < CH; ++t) {
        const float dt = d1[t];
#pragma unroll
        for (int ff = 0; ff < D; ++ff) gk[ff] = fmaf(sK[t * DP + ff], dt, gk[ff]);
      }
#pragma unroll
      for (int ff = 0; ff < D; ++ff) W1[(long long)ff * Dh + j] = fmaf(-a, gk[ff], W1[(long long)ff * Dh + j]);
    }
    __syncthreads();
    // N2 = tril(X2q X2^T)
    for (int e = tid; e < CH * CH; e += kGenThreads) {
      const int i = e / CH, u = e % CH;
      float m = 0.f;
      if (u <= i)
        for (int j = 0; j < Dh; ++j) m = fmaf(XQT[(long long)j * CH + i], X2T[(long long)j * CH + u], m);
      sN2[i * (CH + 1) + u] = m;
    }
    __syncthreads();
    // O = X2q W2 - a N2 E
    T* oc = o + head0 + (long long)c0 * ts;
    hidden_contraction(XQT, [&](int t, int ff, float sum) {
      float corr = 0.f;
      for (int u = 0; u <= t; ++u) corr = fmaf(sN2[t * (CH + 1) + u], sE[u * DP + ff], corr);
      store_io(oc + (long long)t * ts + ff, fmaf(-a, corr, sum));
    });
    // W2[j, :] -= a X2[:, j]^T E (every read of the start state W2 is done: the last barrier above)
    for (int j = tid; j < Dh; j += kGenThreads) {
      float g[D];
#pragma unroll
      for (int ff = 0; ff < D; ++ff) g[ff] = 0.f;
#pragma unroll 1
      for (int t = 0; t < CH; ++t) {
        const float xt = X2T[(long long)j * CH + t];
#pragma unroll
        for (int ff = 0; ff < D; ++ff) g[ff] = fmaf(xt, sE[t * DP + ff], g[ff]);
      }
#pragma unroll
      for (int ff = 0; ff < D; ++ff) W2[(long long)j * D + ff] = fmaf(-a, g[ff], W2[(long long)j * D + ff]);
    }
    __syncthreads();
  }
  if (w1_out)
    for (long long e = tid; e < DDh; e += kGenThreads) w1_out[(long long)bh * DDh + e] = W1[e];
  if (w2_out)
    for (long long e = tid; e < DDh; e += kGenThreads) w2_out[(long long)bh * DDh + e] = W2[e];
}

template <class T, int D>
void launch_generic_d(int BH, int H, int N, int Dh, int CH, float a, const void* q, const void* k,
                      const void* v, const float* w1, const float* w2, long long wbs, void* o,
                      float* w1_out, float* w2_out, float* ws, hipStream_t st) {
  const T *Q = (const T*)q, *K = (const T*)k, *V = (const T*)v;
  switch (CH) {
    case 16:
      hipLaunchKernelGGL((mlp_fwd_generic<T, D, 16>), dim3(BH), dim3(kGenThreads), 0, st, Q, K, V, w1, w2, wbs, H,
                         N, Dh, a, (T*)o, w1_out, w2_out, ws);
      break;
    case 32:
      hipLaunchKernelGGL((mlp_fwd_generic<T, D, 32>), dim3(BH), dim3(kGenThreads), 0, st, Q, K, V, w1, w2, wbs, H,
                         N, Dh, a, (T*)o, w1_out, w2_out, ws);
      break;
    default:
      hipLaunchKernelGGL((mlp_fwd_generic<T, D, 64>), dim3(BH), dim3(kGenThreads), 0, st, Q, K, V, w1, w2, wbs, H,
                         N, Dh, a, (T*)o, w1_out, w2_out, ws);
  }
}

template <class T>
void launch_generic(int BH, int H, int N, int D, int Dh, int CH, float a, const void* q, const void* k,
                    const void* v, const float* w1, const float* w2, long long wbs, void* o, float* w1_out,
                    float* w2_out, float* ws, hipStream_t st) {
  switch (D) {
    case 16: launch_generic_d<T, 16>(BH, H, N, Dh, CH, a, q, k, v, w1, w2, wbs, o, w1_out, w2_out, ws, st); break;
    case 32: launch_generic_d<T, 32>(BH, H, N, Dh, CH, a, q, k, v, w1, w2, wbs, o, w1_out, w2_out, ws, st); break;
    default: launch_generic_d<T, 64>(BH, H, N, Dh, CH, a, q, k, v, w1, w2, wbs, o, w1_out, w2_out, ws, st);
  }
}

}  // namespace

bool mlp_fast_path(bool bf16_io, int D, int Dh, int chunk) {
  return bf16_io && D == kD && Dh == kDh && chunk == kCh;
}
// The matrix-core kernel with the state in the workspace: 2 to 4 blocks of 256 hidden units.
bool mlp_wide_path(bool bf16_io, int D, int Dh, int chunk) {
  return bf16_io && D == kD && chunk == kCh && Dh % kWideBlock == 0 && Dh >= 2 * kWideBlock && Dh <= 4 * kWideBlock;
}

bool mlp_supported(int D, int Dh, int chunk) {
  if (D != 16 && D != 32 && D != 64) return false;
  if (chunk != 16 && chunk != 32 && chunk != 64) return false;
  return Dh >= 64 && Dh <= 1024 && Dh % 64 == 0;
}

// Fast path: one flag per (batch, head) chain, then the split schedule's intermediates and
// checkpoints (MlpSplitWs), each part 256-byte aligned. Otherwise the state and intermediates per
// chain.
struct MlpSplitLayout {
  size_t flags, progress, inter, etile, ckpt, total;
};
MlpSplitLayout mlp_split_layout(int BH, int N) {
  const int C = N / kCh;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  MlpSplitLayout L;
  L.flags = 0;
  L.progress = up((size_t)BH * sizeof(int));
  L.inter = L.progress + up((size_t)BH * sizeof(int));
  L.etile = L.inter + up((size_t)BH * mlp_inter_uint4(C) * sizeof(uint4));
  L.ckpt = L.etile + up((size_t)BH * mlp_etile_uint2(C) * sizeof(uint2));
  L.total = L.ckpt + up((size_t)BH * mlp_ckpt_f32x4(C) * sizeof(f32x4));
  return L;
}
size_t mlp_workspace_bytes(bool bf16_io, int B, int H, int N, int D, int Dh, int chunk) {
  if (mlp_fast_path(bf16_io, D, Dh, chunk)) return mlp_split_layout(B * H, N).total;
  return mlp_min_workspace_bytes(bf16_io, B, H, N, D, Dh, chunk);
}
// The least workspace a call accepts: on the fast path the single-workgroup schedule's flags.
size_t mlp_min_workspace_bytes(bool bf16_io, int B, int H, int N, int D, int Dh, int chunk) {
  if (mlp_fast_path(bf16_io, D, Dh, chunk)) return (size_t)B * H * sizeof(int);
  if (mlp_wide_path(bf16_io, D, Dh, chunk)) return (size_t)B * H * 3 * (size_t)D * Dh * sizeof(float);
  return (size_t)B * H * (2 * (size_t)D * Dh + 4 * (size_t)chunk * Dh) * sizeof(float);
}

hipError_t mlp_launch(bool bf16_io, int B, int H, int N, int D, int Dh, int chunk, float eta,
                      const void* q, const void* k, const void* v, const float* w1,
                      const float* w2, long long wbs, void* o, float* w1_out, float* w2_out,
                      void* ws, size_t ws_bytes, hipStream_t st) {
  const float a = eta / (float)chunk;
  if (mlp_wide_path(bf16_io, D, Dh, chunk)) {
    const int nb = Dh / kWideBlock;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(B * H), dim3(kWaves * 64), 0, st, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, w1, w2, wbs, H, N, a, (bf16*)o, w1_out, w2_out, static_cast<float*>(ws));
    };
    if (nb == 2) go(mlp_fwd_wide<2>);
    else if (nb == 3) go(mlp_fwd_wide<3>);
    else go(mlp_fwd_wide<4>);
    return hipGetLastError();
  }
  if (!mlp_fast_path(bf16_io, D, Dh, chunk)) {
    if (!mlp_supported(D, Dh, chunk)) return hipErrorInvalidValue;
    if (bf16_io)
      launch_generic<bf16>(B * H, H, N, D, Dh, chunk, a, q, k, v, w1, w2, wbs, o, w1_out, w2_out,
                           static_cast<float*>(ws), st);
    else
      launch_generic<float>(B * H, H, N, D, Dh, chunk, a, q, k, v, w1, w2, wbs, o, w1_out, w2_out,
                            static_cast<float*>(ws), st);
    return hipGetLastError();
  }
  const MlpSplitLayout L = mlp_split_layout(B * H, N);
  if (ws_bytes < L.total) {  // the single-workgroup schedule
    hipLaunchKernelGGL(mlp_fwd_single, dim3(B * H), dim3(kWaves * 64), 0, st, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, w1, w2, wbs, H, N, a, (bf16*)o, w1_out, w2_out, static_cast<int*>(ws));
    return hipGetLastError();
  }
  char* base = static_cast<char*>(ws);
  int* flags = reinterpret_cast<int*>(base + L.flags);
  int* progress = reinterpret_cast<int*>(base + L.progress);
  const MlpSplitWs sw{reinterpret_cast<uint4*>(base + L.inter), reinterpret_cast<uint2*>(base + L.etile),
                      reinterpret_cast<f32x4*>(base + L.ckpt), progress};
  const int BH = B * H, tasks = SegPlan(N / kCh).count() * BH;
  const int workers = tasks < kReadoutWorkers ? tasks : kReadoutWorkers;
  hipLaunchKernelGGL(mlp_clear, dim3((BH + 255) / 256), dim3(256), 0, st, flags, progress, BH);
  hipLaunchKernelGGL(mlp_fwd_fused, dim3(BH + workers), dim3(kWaves * 64), 0, st, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, w1, w2, wbs, H, N, a, (bf16*)o, w1_out, w2_out,
                     flags, sw, BH);
  hipLaunchKernelGGL(mlp_fixup_bf16, dim3(B * H), dim3(kWaves * 64), 0, st, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, w1, w2, wbs, H, N, a, (bf16*)o, w1_out, w2_out,
                     (const int*)flags);
  return hipGetLastError();
}

}  // namespace ttt
