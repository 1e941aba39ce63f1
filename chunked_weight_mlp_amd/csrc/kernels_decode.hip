// Decode kernels: one new token per sequence. Both are matrix-vector products
// bound by reading the weights from HBM once per call: the gate/up weights
// (shared by the batch) and each sequence's fp32 fast weight. One wave per
// output row; lanes stride the row in 8-element (16- or 32-byte) vectors and
// reduce with cross-lane shuffles. Rounding matches the prefill path: z is
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

// one wave per d_ff row f; sequences [b0, b0 + nb)
template <typename T>
__global__ __launch_bounds__(256) void k_dec_gateup(const T *__restrict__ x, int64_t x_stride,
                                                    int b0, int nb, int d, int F,
                                                    const T *__restrict__ wg,
                                                    const T *__restrict__ wu, T *__restrict__ z) {
  const int f = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (f >= F) return;
  float g[MAXB] = {}, u[MAXB] = {};
  const T *gr = wg + (int64_t)f * d, *ur = wu + (int64_t)f * d;
  for (int k = 8 * lane; k < d; k += 8 * 64) {
    float wgv[8], wuv[8];
    load8(gr, k, d, wgv);
    load8(ur, k, d, wuv);
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
      if (b >= nb) break;
      float xv[8];
      load8(x + (int64_t)(b0 + b) * x_stride, k, d, xv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        g[b] = fmaf(xv[q], wgv[q], g[b]);
        u[b] = fmaf(xv[q], wuv[q], u[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < MAXB; ++b) {
    if (b >= nb) break;
    const float gs = wave_sum(g[b]), us = wave_sum(u[b]);
    if (lane == 0) z[(int64_t)(b0 + b) * F + f] = from_f<T>(gs / (1.f + expf(-gs)) * us);
  }
}

// one wave per (sequence b, output column c): 8 fast-weight entries per lane
// per step, read as two 16-byte vectors
template <typename T>
__global__ __launch_bounds__(256) void k_dec_apply(const T *__restrict__ z,
                                                   const float *__restrict__ w, int batch, int d,
                                                   int F, float *__restrict__ o) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= batch * d) return;
  const int b = row / d, c = row % d;
  const float *wr = w + ((int64_t)b * d + c) * F;
  const T *zr = z + (int64_t)b * F;
  float acc = 0.f;
  for (int f = 8 * lane; f < F; f += 8 * 64) {
    float wv[8], zv[8];
    load8(wr, f, F, wv);
    load8(zr, f, F, zv);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = fmaf(zv[q], to_f(from_f<T>(wv[q])), acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) o[(int64_t)b * d + c] = acc;
}

}  // namespace

template <typename T>
hipError_t dec_gateup(const T *x, int64_t x_stride, int batch, int d, int F, const T *wg,
                      const T *wu, T *z, hipStream_t st) {
  for (int b0 = 0; b0 < batch; b0 += MAXB) {
    hipLaunchKernelGGL(k_dec_gateup<T>, dim3((unsigned)((F + 3) / 4)), dim3(256), 0, st, x,
                       x_stride, b0, min(MAXB, batch - b0), d, F, wg, wu, z);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
hipError_t dec_apply(const T *z, const float *w, int batch, int d, int F, float *o,
                     hipStream_t st) {
  const int64_t rows = (int64_t)batch * d;
  hipLaunchKernelGGL(k_dec_apply<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, z, w,
                     batch, d, F, o);
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
