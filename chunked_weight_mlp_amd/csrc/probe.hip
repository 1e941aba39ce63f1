// Measurement-only micro-benchmarks of the chip's achievable rates, against
// which the layer's kernels are reported: MFMA issue with no memory traffic
// (two waves per SIMD, independent accumulators), a streaming read, LDS reads
// and direct copies from L2 into LDS. Built into its own library
// (libipttt_probe.so, include/ipttt_probe.h), apart from the layer library.
#include <hip/hip_runtime.h>

#include "../../include/ipttt_probe.h"

namespace ipttt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;

// operands built from the thread index and a runtime seed, so nothing folds
__device__ __forceinline__ void probe_operands(float seed, bf16x8 &a, bf16x8 &b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b[i] = (__bf16)(seed * (float)(i + 1));
  }
}

// 8 independent 16 x 16 x 32 accumulators, 8 MFMAs per iteration. Issued as
// asm on VGPR accumulators: written with the builtin, this loop gets
// accumulator moves between register files every iteration (the layer's
// kernels do not), which would measure those instead of the MFMA pipe. Each
// chain's previous MFMA is 8 issues back, beyond any dependency window; the
// s_nops before the sum let the last ones finish.
#define PROBE_MFMA16(c) \
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b))
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma16(float *out, int64_t iters,
                                                                float seed) {
  bf16x8 a, b;
  probe_operands(seed, a, b);
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int64_t it = 0; it < iters; ++it) {
    PROBE_MFMA16(c0);
    PROBE_MFMA16(c1);
    PROBE_MFMA16(c2);
    PROBE_MFMA16(c3);
    PROBE_MFMA16(c4);
    PROBE_MFMA16(c5);
    PROBE_MFMA16(c6);
    PROBE_MFMA16(c7);
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  const f32x4 t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = t[0] + t[1] + t[2] + t[3];
}
#undef PROBE_MFMA16

// 4 independent 32 x 32 x 16 accumulators, 4 MFMAs per iteration
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma32(float *out, int64_t iters,
                                                                float seed) {
  bf16x8 a, b;
  probe_operands(seed, a, b);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const f32x16 t = c0 + c1 + c2 + c3;
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = t[0] + t[5] + t[10] + t[15];
}

// streams n 16-byte pieces, four loads in flight per thread, and folds them
// into one value per thread (stored so the loads are kept)
__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const uint4 *__restrict__ src,
                                                              unsigned *__restrict__ out,
                                                              int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

// LDS reads: two 256-thread blocks per CU (two waves per SIMD) each fill 32 KB
// of LDS, then read it n times over in 16-byte pieces (four per thread per
// iteration, a wave's 64 pieces contiguous, so no bank conflicts), folded into
// one value per thread (stored so the reads are kept)
constexpr int kProbeLdsBytes = 32 * 1024;
__global__ __launch_bounds__(kProbeThreads) void k_probe_lds(unsigned *__restrict__ out,
                                                             int64_t iters) {
  __shared__ uint4 buf[kProbeLdsBytes / 16];
  constexpr int N = kProbeLdsBytes / 16;
  for (int i = threadIdx.x; i < N; i += kProbeThreads)
    buf[i] = uint4{(unsigned)i, (unsigned)i * 3u, (unsigned)i * 5u, (unsigned)i * 7u};
  __syncthreads();
  unsigned acc = 0;
  for (int64_t it = 0; it < iters; ++it) {
    const int base = (int)((it * 4 * kProbeThreads) % N);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 v = buf[(base + k * kProbeThreads + threadIdx.x) % N];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    asm volatile("" ::: "memory");  // each iteration's reads stay in it
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}
// Direct global -> LDS copies from L2: four-wave blocks, two per CU, each copy
// 8 KB per wave and iteration (eight 1 KB global_load_lds_dwordx4) from a
// 64 KB window of src into a two-half 32 KB LDS ring, with two iterations in
// flight; the 64 windows (4 MiB) stay in L2 after the first pass.
typedef __attribute__((address_space(3))) void probe_lds_t;
typedef __attribute__((address_space(1))) const void probe_gbl_t;
__global__ __launch_bounds__(kProbeThreads) void k_probe_copy(const char *__restrict__ src,
                                                              int64_t iters) {
  __shared__ __attribute__((aligned(1024))) char ring[32768];
  constexpr int NW = kProbeThreads / 64;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char *win = src + (int64_t)(blockIdx.x % 64) * 65536;
  for (int64_t it = 0; it < iters; ++it) {
    char *half = ring + (it & 1) * 16384;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t off = ((it * 8 + i) * 1024 + wave * 8192) % 65536;
      __builtin_amdgcn_global_load_lds((probe_gbl_t *)(win + off + lane * 16),
                                       (probe_lds_t *)(half + ((i * NW + wave) % 16) * 1024), 16,
                                       0, 0);
    }
    // the previous iteration's copies landed (this one's 8 may still fly)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
}  // namespace

constexpr size_t kCopyWindowBytes = (size_t)64 * 65536;  // 64 windows of 64 KB

}  // namespace ipttt

extern "C" int ipttt_probe(int32_t kind, int64_t n, const void *src, size_t src_bytes, void *dst,
                           size_t dst_bytes, double *work, void *hip_stream) {
  using namespace ipttt;
  constexpr int kOk = 0, kInvalid = -1, kHip = -3;
  if (kind < IPTTT_PROBE_MFMA16 || kind > IPTTT_PROBE_COPY || n < 1 || !dst || !work ||
      ((uintptr_t)dst & 15))
    return kInvalid;
  const bool needs_src = kind == IPTTT_PROBE_READ || kind == IPTTT_PROBE_COPY;
  if (needs_src && (!src || ((uintptr_t)src & 15))) return kInvalid;
  if (kind == IPTTT_PROBE_READ && (n % 16 || (size_t)n > src_bytes)) return kInvalid;
  if (kind == IPTTT_PROBE_COPY && src_bytes < kCopyWindowBytes) return kInvalid;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return kHip;
  hipStream_t st = (hipStream_t)hip_stream;
  const int64_t blocks2 = 2 * (int64_t)cus;  // 8 waves per CU: two per SIMD
  const size_t out2 = (size_t)blocks2 * kProbeThreads * 4;
  if (kind == IPTTT_PROBE_MFMA16 || kind == IPTTT_PROBE_MFMA32) {
    if (dst_bytes < out2) return kInvalid;
    const int64_t waves = blocks2 * (kProbeThreads / 64);
    if (kind == IPTTT_PROBE_MFMA16) {
      hipLaunchKernelGGL(k_probe_mfma16, dim3((unsigned)blocks2), dim3(kProbeThreads), 0, st,
                         (float *)dst, n, 1e-3f);
      *work = (double)n * 8 * (2.0 * 16 * 16 * 32) * waves;
    } else {
      hipLaunchKernelGGL(k_probe_mfma32, dim3((unsigned)blocks2), dim3(kProbeThreads), 0, st,
                         (float *)dst, n, 1e-3f);
      *work = (double)n * 4 * (2.0 * 32 * 32 * 16) * waves;
    }
  } else if (kind == IPTTT_PROBE_COPY) {
    hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)blocks2), dim3(kProbeThreads), 0, st,
                       (const char *)src, n);
    *work = (double)n * 8 * 1024 * (kProbeThreads / 64) * blocks2;
  } else if (kind == IPTTT_PROBE_LDS) {
    if (dst_bytes < out2) return kInvalid;
    hipLaunchKernelGGL(k_probe_lds, dim3((unsigned)blocks2), dim3(kProbeThreads), 0, st,
                       (unsigned *)dst, n);
    *work = (double)n * 4 * 16 * kProbeThreads * blocks2;
  } else {  // read: n bytes from src, one 32-bit value per thread to dst
    const int64_t blocks = 8 * (int64_t)cus;
    if (dst_bytes < (size_t)blocks * kProbeThreads * 4) return kInvalid;
    hipLaunchKernelGGL(k_probe_read, dim3((unsigned)blocks), dim3(kProbeThreads), 0, st,
                       (const uint4 *)src, (unsigned *)dst, n / 16);
    *work = (double)n;
  }
  return hipGetLastError() == hipSuccess ? kOk : kHip;
}
