// Generic kernels of the fast-weight prefill: LDS-tiled fp32 FMA, storage in
// fp32 or bf16. They run every fp32 layer and, on request, bf16 layers (as a
// cross-check of the MFMA kernels). Each block computes a 64x64 output tile
// with 256 threads, 4x4 outputs per thread, K staged through LDS 16 at a time.
#include "internal.h"

namespace ipttt {
namespace {

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(__bf16 v) { return (float)v; }
template <typename T>
__device__ __forceinline__ T from_f(float v);
template <>
__device__ __forceinline__ float from_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 from_f<__bf16>(float v) { return (__bf16)v; }  // RNE

// Row p of a chunk-padded slab -> token index within the sequence, or -1 for a pad row.
__device__ __forceinline__ int64_t slab_row_token(const Slab &s, int64_t p) {
  const int64_t j = p / s.Bp, i = p % s.Bp;
  if (i >= s.B || j >= s.nc) return -1;
  const int64_t t = s.tok0 + j * s.B + i;
  return t < s.L ? t : -1;
}

constexpr int TILE = 64, TK = 16, NT = 256;

// C[m][n] = sum_k A[m][k] B[n][k]; both operands K-contiguous. Op supplies the
// per-batch operand pointers and the epilogue.
template <typename TA, typename TB, class Op>
__global__ __launch_bounds__(NT) void k_gemm_nt(Op op, int M, int N, int K) {
  const int bz = blockIdx.z;
  const TA *A = op.a(bz);
  const TB *Bm = op.b(bz);
  const int64_t lda = op.lda, ldb = op.ldb;
  const int m0 = blockIdx.y * TILE, n0 = blockIdx.x * TILE;
  __shared__ float As[TK][TILE + 1], Bs[TK][TILE + 1];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + q * NT, r = idx / TK, kk = idx % TK;
      const int m = m0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < M && k < K) ? to_f(A[(int64_t)m * lda + k]) : 0.f;
      Bs[kk][r] = (n < N && k < K) ? to_f(Bm[(int64_t)n * ldb + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty + 16 * i];
        b[i] = Bs[kk][tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(a[i], b[jj], acc[i][jj]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * jj;
      if (m < M && n < N) op.store(bz, m, n, acc[i][jj]);
    }
}

// Z = SiLU(X W_g) * (X W_u) over the slab's padded rows; writes Z and Zt.
template <typename T>
__global__ __launch_bounds__(NT) void k_gateup_gen(Slab s, const T *x, const T *wg, const T *wu,
                                                   T *z, T *zt) {
  const int n_seq = blockIdx.z;
  const int d = s.d, F = s.F;
  const int64_t P = (int64_t)s.nc * s.Bp;
  const int64_t p0 = (int64_t)blockIdx.y * TILE;
  const int f0 = blockIdx.x * TILE;
  const T *xs = x + n_seq * s.x_seq_stride;
  __shared__ float As[TK][TILE + 1], Gs[TK][TILE + 1], Us[TK][TILE + 1];
  __shared__ int64_t rowtok[TILE];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  if (tid < TILE) rowtok[tid] = (p0 + tid < P) ? slab_row_token(s, p0 + tid) : -1;
  __syncthreads();
  float ag[4][4] = {}, au[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += TK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + q * NT, r = idx / TK, kk = idx % TK, k = k0 + kk;
      const int64_t t = rowtok[r];
      As[kk][r] = (t >= 0 && k < d) ? to_f(xs[t * d + k]) : 0.f;
      const int f = f0 + r;
      Gs[kk][r] = (f < F && k < d) ? to_f(wg[(int64_t)f * d + k]) : 0.f;
      Us[kk][r] = (f < F && k < d) ? to_f(wu[(int64_t)f * d + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], g[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty + 16 * i];
        g[i] = Gs[kk][tx + 16 * i];
        u[i] = Us[kk][tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          ag[i][jj] = fmaf(a[i], g[jj], ag[i][jj]);
          au[i][jj] = fmaf(a[i], u[jj], au[i][jj]);
        }
    }
    __syncthreads();
  }
  T *zs = z + (int64_t)n_seq * s.Lp * F;
  T *zts = zt + (int64_t)n_seq * F * s.Lp;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t p = p0 + ty + 16 * i;
      const int f = f0 + tx + 16 * jj;
      if (p < P && f < F) {
        const float g = ag[i][jj];
        const float zz = g / (1.f + expf(-g)) * au[i][jj];
        const T v = from_f<T>(zz);
        zs[p * F + f] = v;
        zts[(int64_t)f * s.Lp + p] = v;
      }
    }
}

// C[p][c] = sum_j conv_w[c][j] E[t + j][c], zero past the chunk end (pad rows: 0).
template <typename T>
__global__ void k_conv_gen(Slab s, const T *e, const T *cw, T *c) {
  const int n_seq = blockIdx.y;
  const int64_t P = (int64_t)s.nc * s.Bp;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= P * s.d) return;
  const int64_t p = idx / s.d;
  const int ch = (int)(idx % s.d);
  float acc = 0.f;
  const int64_t t = slab_row_token(s, p);
  if (t >= 0) {
    const int64_t j = p / s.Bp, i = p % s.Bp;
    const int64_t chunk_end = min(s.tok0 + (j + 1) * s.B, s.L);
    const T *es = e + n_seq * s.x_seq_stride;
    for (int q = 0; q < s.Kc; ++q) {
      if (t + q < chunk_end) acc = fmaf(to_f(cw[ch * s.Kc + q]), to_f(es[(t + q) * s.d + ch]), acc);
    }
    (void)i;
  }
  c[(int64_t)n_seq * s.Lp * s.d + p * s.d + ch] = from_f<T>(acc);
}

template <typename T>
__global__ void k_snapshot_gen(int64_t n_elem, const float *w, T *snap, int64_t snap_stride) {
  const int n_seq = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_elem) snap[n_seq * snap_stride + i] = from_f<T>(w[n_seq * n_elem + i]);
}

// ---- epilogue ops --------------------------------------------------------
template <typename T>
struct ProjOp {  // Vt[n][c'][p] = scale * sum_c C[n][p][c] proj[c'][c]
  const T *c;
  const T *proj;
  T *vt;
  int64_t lda, ldb, Lp;
  int d;
  float scale;
  __device__ const T *a(int bz) const { return c + (int64_t)bz * Lp * d; }
  __device__ const T *b(int) const { return proj; }
  __device__ void store(int bz, int m, int n, float acc) const {
    vt[(int64_t)bz * d * Lp + (int64_t)n * Lp + m] = from_f<T>(scale * acc);
  }
};

template <typename T>
struct ApplyOp {  // O rows of chunk j = sum_f Z[p][f] S_j[c][f]; mse: Rt = eta (V - O)
  Slab s;
  int j0, nj;
  const T *z, *snap, *vt;
  int64_t snap_seq_stride, snap_chunk_stride;
  float *o;
  T *rt;
  int64_t lda, ldb;
  __device__ const T *a(int bz) const {
    const int n = bz / nj, j = j0 + bz % nj;
    return z + (int64_t)n * s.Lp * s.F + (int64_t)j * s.Bp * s.F;
  }
  __device__ const T *b(int bz) const {
    const int n = bz / nj, jl = bz % nj;
    return snap + n * snap_seq_stride + jl * snap_chunk_stride;
  }
  __device__ void store(int bz, int m, int c, float acc) const {
    const int n = bz / nj, j = j0 + bz % nj;
    const int64_t t = s.tok0 + (int64_t)j * s.B + m;
    const bool valid = m < s.B && t < s.L;
    if (valid && o) o[n * s.x_seq_stride + t * s.d + c] = acc;
    if (rt) {
      float r = 0.f;
      if (valid) r = s.eta * (to_f(vt[(int64_t)n * s.d * s.Lp + (int64_t)c * s.Lp + (int64_t)j * s.Bp + m]) - acc);
      rt[(int64_t)n * s.d * s.Bp + (int64_t)c * s.Bp + m] = from_f<T>(r);
    }
  }
};

template <typename T>
struct UpdateOp {  // W[n][c][f] += sum_t A[n][c][t] Zt[n][f][t]; snapshot of the new W
  const T *a_base, *zt;
  int64_t a_seq_stride, zt_seq_stride;
  float *w;
  T *snap;
  int64_t snap_seq_stride;
  int64_t lda, ldb;
  int F;
  int64_t dF;
  __device__ const T *a(int bz) const { return a_base + bz * a_seq_stride; }
  __device__ const T *b(int bz) const { return zt + bz * zt_seq_stride; }
  __device__ void store(int bz, int c, int f, float acc) const {
    float *wp = w + bz * dF + (int64_t)c * F + f;
    const float nw = *wp + acc;
    *wp = nw;
    if (snap) snap[bz * snap_seq_stride + (int64_t)c * F + f] = from_f<T>(nw);
  }
};

inline dim3 gemm_grid(int64_t M, int64_t N, int batch) {
  return dim3((unsigned)((N + TILE - 1) / TILE), (unsigned)((M + TILE - 1) / TILE), (unsigned)batch);
}

}  // namespace

template <typename T>
hipError_t gen_gateup(const Slab &s, const T *x, const Weights &w, const WsPtrs &ws,
                      hipStream_t st) {
  const int64_t P = (int64_t)s.nc * s.Bp;
  hipLaunchKernelGGL(k_gateup_gen<T>, gemm_grid(P, s.F, s.n_seq), dim3(NT), 0, st, s, x,
                     (const T *)w.w_gate, (const T *)w.w_up, (T *)ws.z, (T *)ws.zt);
  return hipGetLastError();
}

template <typename T>
hipError_t gen_conv(const Slab &s, const T *e, const Weights &w, const WsPtrs &ws,
                    hipStream_t st) {
  const int64_t P = (int64_t)s.nc * s.Bp;
  const int64_t n = P * s.d;
  hipLaunchKernelGGL(k_conv_gen<T>, dim3((unsigned)((n + 255) / 256), (unsigned)s.n_seq),
                     dim3(256), 0, st, s, e, (const T *)w.conv_w, (T *)ws.c);
  return hipGetLastError();
}

template <typename T>
hipError_t gen_proj(const Slab &s, const Weights &w, const WsPtrs &ws, hipStream_t st) {
  const int64_t P = (int64_t)s.nc * s.Bp;
  ProjOp<T> op{(const T *)ws.c, (const T *)w.proj, (T *)ws.vt, s.d, s.d, s.Lp, s.d,
               s.mse ? 1.f : s.eta};
  hipLaunchKernelGGL((k_gemm_nt<T, T, ProjOp<T>>), gemm_grid(P, s.d, s.n_seq), dim3(NT), 0, st,
                     op, (int)P, s.d, s.d);
  return hipGetLastError();
}

template <typename T>
hipError_t gen_snapshot(const Slab &s, const float *w_state, T *snap, int64_t snap_seq_stride,
                        hipStream_t st) {
  const int64_t n = (int64_t)s.d * s.F;
  hipLaunchKernelGGL(k_snapshot_gen<T>, dim3((unsigned)((n + 255) / 256), (unsigned)s.n_seq),
                     dim3(256), 0, st, n, w_state, snap, snap_seq_stride);
  return hipGetLastError();
}

template <typename T>
hipError_t gen_update(const Slab &s, int j, const T *a, int64_t a_ld, int64_t a_seq_stride,
                      const WsPtrs &ws, float *w_state, T *snap_out, int64_t snap_seq_stride,
                      hipStream_t st) {
  UpdateOp<T> op{a, (const T *)ws.zt + (int64_t)j * s.Bp, a_seq_stride, (int64_t)s.F * s.Lp,
                 w_state, snap_out, snap_seq_stride, a_ld, s.Lp, s.F, (int64_t)s.d * s.F};
  hipLaunchKernelGGL((k_gemm_nt<T, T, UpdateOp<T>>), gemm_grid(s.d, s.F, s.n_seq), dim3(NT), 0,
                     st, op, s.d, s.F, s.Bp);
  return hipGetLastError();
}

template <typename T>
hipError_t gen_apply(const Slab &s, int j0, int nj, const T *snap, int64_t snap_seq_stride,
                     int64_t snap_chunk_stride, const WsPtrs &ws, float *o, hipStream_t st) {
  ApplyOp<T> op{s, j0, nj, (const T *)ws.z, snap, (const T *)ws.vt, snap_seq_stride,
                snap_chunk_stride, o, s.mse ? (T *)ws.rt : nullptr, s.F, s.F};
  hipLaunchKernelGGL((k_gemm_nt<T, T, ApplyOp<T>>), gemm_grid(s.Bp, s.d, s.n_seq * nj), dim3(NT),
                     0, st, op, s.Bp, s.d, s.F);
  return hipGetLastError();
}

#define IPTTT_INST(T)                                                                          \
  template hipError_t gen_gateup<T>(const Slab &, const T *, const Weights &, const WsPtrs &, \
                                    hipStream_t);                                              \
  template hipError_t gen_conv<T>(const Slab &, const T *, const Weights &, const WsPtrs &,   \
                                  hipStream_t);                                                \
  template hipError_t gen_proj<T>(const Slab &, const Weights &, const WsPtrs &, hipStream_t); \
  template hipError_t gen_snapshot<T>(const Slab &, const float *, T *, int64_t, hipStream_t); \
  template hipError_t gen_update<T>(const Slab &, int, const T *, int64_t, int64_t,           \
                                    const WsPtrs &, float *, T *, int64_t, hipStream_t);      \
  template hipError_t gen_apply<T>(const Slab &, int, int, const T *, int64_t, int64_t,       \
                                   const WsPtrs &, float *, hipStream_t);
IPTTT_INST(float)
IPTTT_INST(__bf16)
#undef IPTTT_INST

}  // namespace ipttt
