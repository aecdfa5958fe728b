// Depth-wise 3x3 convolution over the token grid: the Conv2d preprocessing that Vision-TTT
// applies before its scan (Vision-TTT summary on gist.science, "Methodologie" item 2) and the
// depth-wise branch of ViT^3's block (ViT^3 review on techloop.online, "TTT Block" section).
// A sequence of N = height * width tokens in raster order, [B, N, C] with C channels contiguous
// (the [B, N, H, D] layout of q, k, v with C = H * D), is an image of height x width pixels; each
// channel has its own 3x3 kernel and bias, with zero padding:
//   y[b, i, j, c] = bias[c] + sum_{u, v in 0..2} w[c, u, v] x[b, i + u - 1, j + v - 1, c].
//
// 9 multiply-adds per element read and written: without packed fp32 arithmetic the vector ALUs
// are about as busy as HBM, so the kernel keeps every instruction that is not one of those
// multiply-adds or a bf16 widening out of the loop, and overlaps loads, arithmetic and stores
// inside each wave. Each thread owns one piece of a token row (4 channels) in a strip of output
// rows and streams down the strip, prefetching three input rows ahead. Loads go through one
// buffer resource per image row, so the zero padding costs no instruction: loads outside the row,
// and every load of a row outside the image, return zero in hardware. Adjacent threads hold
// adjacent pieces, so a wave's three loads of a row (columns j - 1, j, j + 1) are contiguous runs
// that mostly hit in the L1 cache after the first. No LDS, no barriers.
#include "device.hpp"
#include "internal.hpp"

namespace ttt {
namespace {

constexpr int kConvThreads = 256;

// Buffer resource of one image row: loads at byte offsets outside [0, bytes) return zero, which
// is the convolution's zero padding (the piece left of token 0 and right of the last token, and
// whole rows outside the image, given bytes = 0). gfx9 descriptor word 3: 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef int i32x4 __attribute__((ext_vector_type(4)));

// One piece: 4 channels of a token (8 bytes of bf16, 16 of fp32), loaded raw and widened to fp32
// only for the arithmetic.
template <class T>
struct Io4;
template <>
struct Io4<bf16> {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef i32x2 Raw;
  static constexpr int kBytes = 8;
  static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  }
  static __device__ __forceinline__ void widen(const Raw& v, float* out) {
    for (int i = 0; i < 2; ++i) {
      const uint32_t u = (uint32_t)v[i];
      out[2 * i] = __uint_as_float(u << 16);
      out[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(char* p, const float* v) {
    *reinterpret_cast<bf16x4*>(p) = to_bf16x4(f32x4{v[0], v[1], v[2], v[3]});
  }
};
template <>
struct Io4<float> {
  typedef i32x4 Raw;
  static constexpr int kBytes = 16;
  static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
  static __device__ __forceinline__ void widen(const Raw& v, float* out) {
    for (int i = 0; i < 4; ++i) out[i] = __int_as_float(v[i]);
  }
  static __device__ __forceinline__ void store(char* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// A row of the image is Wi * CG pieces (CG = C / 4), piece P = j * CG + (channel group); the
// pieces of token j - 1 and j + 1 in the same channels are P - CG and P + CG. Thread P of
// workgroup (blockIdx.x, blockIdx.y) owns piece P of the output rows of strip blockIdx.y,
// [RS blockIdx.y, RS blockIdx.y + RS), and streams down the strip's input rows (one halo row
// above and below): every input row adds kernel row 2 to output row ii - 1 (then complete), row 1
// to output row ii and row 0 to output row ii + 1, in a ring of three accumulator rows; the raw
// loads of the next three input rows are issued before the current three are computed.
template <class T>
__global__ __launch_bounds__(kConvThreads) void dwconv3x3_kernel(const T* __restrict__ x,
                                                                 const float* __restrict__ w,
                                                                 const float* __restrict__ bias,
                                                                 T* __restrict__ y, int Hi, int Wi,
                                                                 int C, int RS) {
  using IO = Io4<T>;
  using Raw = typename IO::Raw;
  constexpr int PB = IO::kBytes;
  const int CG = C / 4;
  const int rowp = Wi * CG;  // pieces per image row
  const int P = blockIdx.x * kConvThreads + threadIdx.x;
  if (P >= rowp) return;  // (no barriers in this kernel)
  const int r0 = blockIdx.y * RS, r1 = min(Hi, r0 + RS);  // output rows [r0, r1)
  const int n_in = r1 - r0 + 2;                             // input rows r0 - 1 .. r1
  const uint32_t rowbytes = (uint32_t)rowp * PB;
  const char* xb = reinterpret_cast<const char*>(x) + (long long)blockIdx.z * Hi * rowbytes;
  char* yb = reinterpret_cast<char*>(y) + (long long)blockIdx.z * Hi * rowbytes;
  // Byte offsets in a row of this piece and of its left and right neighbours; a negative one
  // wraps to a huge unsigned offset, which the row's buffer resource reads as zero.
  const uint32_t oc = (uint32_t)P * PB, ol = oc - (uint32_t)CG * PB, orr = oc + (uint32_t)CG * PB;
  // Input row ii (uniform across the workgroup); rows outside the image and below the strip's
  // halo read as zero.
  auto load_row = [&](int ii, Raw* r) {
    const bool in = ii >= 0 && ii < Hi && ii <= r1;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(xb + (long long)(in ? ii : 0) * rowbytes, in ? rowbytes : 0u);
    r[0] = IO::load(rs, ol);
    r[1] = IO::load(rs, oc);
    r[2] = IO::load(rs, orr);
  };
  Raw nxt[3][3];
  for (int q = 0; q < 3; ++q) load_row(r0 - 1 + q, nxt[q]);

  const int c0 = (P % CG) * 4;
  float wt[3][3][4], bs[4];
  {
    const float4* wp = reinterpret_cast<const float4*>(w + c0 * 9);  // 36 contiguous floats
    float wl[36];
    for (int i = 0; i < 9; ++i) {
      const float4 f = wp[i];
      wl[4 * i] = f.x; wl[4 * i + 1] = f.y; wl[4 * i + 2] = f.z; wl[4 * i + 3] = f.w;
    }
    for (int k = 0; k < 4; ++k) {
      for (int u = 0; u < 3; ++u)
        for (int v = 0; v < 3; ++v) wt[u][v][k] = wl[k * 9 + u * 3 + v];
      bs[k] = bias ? bias[c0 + k] : 0.f;
    }
  }
  float acc[3][4];
  for (int s = 0; s < 3; ++s)
    for (int k = 0; k < 4; ++k) acc[s][k] = bs[k];
  // Three input rows per trip, so that the ring's slot roles are the same in every trip.
  for (int tb = 0; tb < n_in; tb += 3) {
    Raw cur[3][3];
    for (int q = 0; q < 3; ++q)
      for (int v = 0; v < 3; ++v) cur[q][v] = nxt[q][v];
    for (int q = 0; q < 3; ++q) load_row(r0 + 2 + tb + q, nxt[q]);  // rows of the next trip
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int t = tb + q, o = r0 - 2 + t;  // output row complete after this input row
      float* am = acc[q];
      float* a0 = acc[(q + 1) % 3];
      float* ap = acc[(q + 2) % 3];
      float xv[3][4];
      for (int v = 0; v < 3; ++v) IO::widen(cur[q][v], xv[v]);
      for (int v = 0; v < 3; ++v)
        for (int k = 0; k < 4; ++k) {
          am[k] = fmaf(wt[2][v][k], xv[v][k], am[k]);
          a0[k] = fmaf(wt[1][v][k], xv[v][k], a0[k]);
          ap[k] = fmaf(wt[0][v][k], xv[v][k], ap[k]);
        }
      if (o >= r0 && o < r1) IO::store(yb + (long long)o * rowbytes + oc, am);
      for (int k = 0; k < 4; ++k) am[k] = bs[k];  // the slot becomes output row o + 3
    }
  }
}

template <class T>
hipError_t launch_conv(int B, int Hi, int Wi, int C, const void* x, const float* w,
                       const float* bias, void* y, hipStream_t st) {
  const long long pieces = (long long)Wi * (C / 4);
  const int gx = (int)((pieces + kConvThreads - 1) / kConvThreads);
  // Strips of rows: enough workgroups for about 640 (two waves per SIMD of 256 CUs would be 512),
  // at least 4 rows each so that the halo rows stay a small share.
  int strips = (int)((640 + (long long)gx * B - 1) / ((long long)gx * B));
  if (strips > (Hi + 3) / 4) strips = (Hi + 3) / 4;
  if (strips < 1) strips = 1;
  const int RS = (Hi + strips - 1) / strips;
  const dim3 grid((unsigned)gx, (unsigned)((Hi + RS - 1) / RS), (unsigned)B);
  hipLaunchKernelGGL(dwconv3x3_kernel<T>, grid, dim3(kConvThreads), 0, st, (const T*)x, w, bias, (T*)y,
                     Hi, Wi, C, RS);
  return hipGetLastError();
}

}  // namespace

hipError_t dwconv_launch(bool bf16_io, int B, int Hi, int Wi, int C, const void* x,
                         const float* w, const float* bias, void* y, hipStream_t st) {
  return bf16_io ? launch_conv<bf16>(B, Hi, Wi, C, x, w, bias, y, st)
                 : launch_conv<float>(B, Hi, Wi, C, x, w, bias, y, st);
}

}  // namespace ttt
