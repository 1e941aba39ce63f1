// Decode kernels: one new token per sequence. Both are matrix-vector products
// bound by reading the weights from HBM once per call: the gate/up weights
// (shared by the batch) and each sequence's fp32 fast weight. One wave per
// output row for gate/up, four per output row for the apply; lanes stride the
// row in 8-element (16- or 32-byte) vectors, several in flight, and reduce
// with cross-lane shuffles. Rounding matches the prefill path: z is
// rounded to the storage type, and on the bf16 path the fast weight is
// rounded to bf16 before the product, as the prefill apply reads a bf16 copy.
#include "internal.h"

namespace ipttt {
namespace {

constexpr int MAXB = 8;  // sequences per pass of the gate/up kernel

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(__bf16 v) { return (float)v; }
template <typename T>
__device__ __forceinline__ T from_f(float v);
template <>
__device__ __forceinline__ float from_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 from_f<__bf16>(float v) { return (__bf16)v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// 8 consecutive elements p[k .. k+7] as floats: 16-byte vector loads when all
// 8 are inside the row (k + 8 <= n) and p + k is 16-byte aligned, else element
// by element (zero past n).
template <typename T>
__device__ __forceinline__ void load8(const T *p, int k, int n, float (&v)[8]) {
  if (k + 8 <= n && ((uintptr_t)(p + k) & 15u) == 0) {
    if constexpr (sizeof(T) == 2) {
      typedef __bf16 b8 __attribute__((ext_vector_type(8)));
      const b8 x = *(const b8 *)(p + k);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = (float)x[q];
    } else {
      const float4 a = *(const float4 *)(p + k), b = *(const float4 *)(p + k + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = k + q < n ? to_f(p[k + q]) : 0.f;
  }
}

// Pieces of 8 elements per lane whose loads are issued before any is used: a
// GEMV is bound by the bytes in flight, and one piece per lane at a time (2 KB
// per wave) leaves HBM idle at these occupancies.
constexpr int UNROLL = 4;

// 8 elements p[0 .. 7] as floats with 16-byte vector loads (p 16-byte aligned,
// all 8 in range)
template <typename T>
__device__ __forceinline__ void load8v(const T *p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 b8 __attribute__((ext_vector_type(8)));
    const b8 x = *(const b8 *)p;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (float)x[q];
  } else {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ bool aligned16(const T *p) {
  return ((uintptr_t)p & 15u) == 0;
}

// one wave per d_ff row f; sequences [b0, b0 + NB)
template <typename T, int NB>
__global__ __launch_bounds__(256) void k_dec_gateup(const T *__restrict__ x, int64_t x_stride,
                                                    int b0, int d, int F,
                                                    const T *__restrict__ wg,
                                                    const T *__restrict__ wu, T *__restrict__ z) {
  const int f = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (f >= F) return;
  // fewer pieces in flight for larger batches (their x rows take the registers)
  constexpr int U = NB <= 2 ? UNROLL : NB <= 4 ? 2 : 1;
  float g[NB] = {}, u[NB] = {};
  const T *gr = wg + (int64_t)f * d, *ur = wu + (int64_t)f * d;
  auto piece = [&](int k, const float (&wgv)[8], const float (&wuv)[8], bool vec) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float xv[8];
      const T *xr = x + (int64_t)(b0 + b) * x_stride;
      if (vec)
        load8v(xr + k, xv);
      else
        load8(xr, k, d, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[b] = fmaf(xv[e], wgv[e], g[b]);
        u[b] = fmaf(xv[e], wuv[e], u[b]);
      }
    }
  };
  // whole groups of U pieces with unchecked vector loads (wave-uniform test),
  // then the rest one checked piece at a time
  const bool vec = (d % 8) == 0 && (x_stride % 8) == 0 && aligned16(gr) && aligned16(ur) &&
                   aligned16(x + (int64_t)b0 * x_stride);
  int kb = 0;
  if (vec)
    for (; kb + 8 * 64 * U <= d; kb += 8 * 64 * U) {
      float wgv[U][8], wuv[U][8];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        load8v(gr + kb + 8 * 64 * q + 8 * lane, wgv[q]);
        load8v(ur + kb + 8 * 64 * q + 8 * lane, wuv[q]);
      }
#pragma unroll
      for (int q = 0; q < U; ++q) piece(kb + 8 * 64 * q + 8 * lane, wgv[q], wuv[q], true);
    }
  for (; kb < d; kb += 8 * 64) {
    float wgv[8], wuv[8];
    const int k = kb + 8 * lane;
    load8(gr, k, d, wgv);
    load8(ur, k, d, wuv);
    piece(k, wgv, wuv, false);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float gs = wave_sum(g[b]), us = wave_sum(u[b]);
    if (lane == 0) z[(int64_t)(b0 + b) * F + f] = from_f<T>(gs / (1.f + expf(-gs)) * us);
  }
}

// one block of 4 waves per (sequence b, output column c): wave w takes the
// 512-element pieces w, w + 4, ... of the row, two at a time, and the four
// partial sums meet in LDS
template <typename T>
__global__ __launch_bounds__(256) void k_dec_apply(const T *__restrict__ z,
                                                   const float *__restrict__ w, int d, int F,
                                                   float *__restrict__ o) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = row / d, c = row % d;
  const float *wr = w + ((int64_t)b * d + c) * F;
  const T *zr = z + (int64_t)b * F;
  float acc = 0.f;
  auto piece = [&](const float (&wv)[8], const float (&zv)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(zv[e], to_f(from_f<T>(wv[e])), acc);
  };
  const int npieces = (F + 511) / 512, nfull = F / 512;
  const bool vec = (F % 8) == 0 && aligned16(wr) && aligned16(zr);
  int p = wave;
  if (vec)
    for (; p + 4 < nfull; p += 8) {  // pieces p and p + 4, both whole
      float wv[2][8], zv[2][8];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        load8v(wr + (p + 4 * q) * 512 + 8 * lane, wv[q]);
        load8v(zr + (p + 4 * q) * 512 + 8 * lane, zv[q]);
      }
      piece(wv[0], zv[0]);
      piece(wv[1], zv[1]);
    }
  for (; p < npieces; p += 4) {
    float wv[8], zv[8];
    load8(wr, p * 512 + 8 * lane, F, wv);
    load8(zr, p * 512 + 8 * lane, F, zv);
    piece(wv, zv);
  }
  acc = wave_sum(acc);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) o[(int64_t)b * d + c] = (part[0] + part[1]) + (part[2] + part[3]);
}

}  // namespace

template <typename T, int NB>
static void launch_dec_gateup(const T *x, int64_t x_stride, int b0, int d, int F, const T *wg,
                              const T *wu, T *z, hipStream_t st) {
  hipLaunchKernelGGL((k_dec_gateup<T, NB>), dim3((unsigned)((F + 3) / 4)), dim3(256), 0, st, x,
                     x_stride, b0, d, F, wg, wu, z);
}

template <typename T>
hipError_t dec_gateup(const T *x, int64_t x_stride, int batch, int d, int F, const T *wg,
                      const T *wu, T *z, hipStream_t st) {
  for (int b0 = 0; b0 < batch; b0 += MAXB) {
    switch (min(MAXB, batch - b0)) {
      case 1: launch_dec_gateup<T, 1>(x, x_stride, b0, d, F, wg, wu, z, st); break;
      case 2: launch_dec_gateup<T, 2>(x, x_stride, b0, d, F, wg, wu, z, st); break;
      case 3: launch_dec_gateup<T, 3>(x, x_stride, b0, d, F, wg, wu, z, st); break;
      case 4: launch_dec_gateup<T, 4>(x, x_stride, b0, d, F, wg, wu, z, st); break;
      case 5: launch_dec_gateup<T, 5>(x, x_stride, b0, d, F, wg, wu, z, st); break;
      case 6: launch_dec_gateup<T, 6>(x, x_stride, b0, d, F, wg, wu, z, st); break;
      case 7: launch_dec_gateup<T, 7>(x, x_stride, b0, d, F, wg, wu, z, st); break;
      default: launch_dec_gateup<T, MAXB>(x, x_stride, b0, d, F, wg, wu, z, st); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
hipError_t dec_apply(const T *z, const float *w, int batch, int d, int F, float *o,
                     hipStream_t st) {
  const int64_t rows = (int64_t)batch * d;
  hipLaunchKernelGGL(k_dec_apply<T>, dim3((unsigned)rows), dim3(256), 0, st, z, w, d, F, o);
  return hipGetLastError();
}

template hipError_t dec_gateup<float>(const float *, int64_t, int, int, int, const float *,
                                      const float *, float *, hipStream_t);
template hipError_t dec_gateup<__bf16>(const __bf16 *, int64_t, int, int, int, const __bf16 *,
                                       const __bf16 *, __bf16 *, hipStream_t);
template hipError_t dec_apply<float>(const float *, const float *, int, int, int, float *,
                                     hipStream_t);
template hipError_t dec_apply<__bf16>(const __bf16 *, const float *, int, int, int, float *,
                                      hipStream_t);

}  // namespace ipttt
