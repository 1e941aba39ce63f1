// bf16 MFMA kernels of the fast-weight prefill for gfx950 (CDNA4).
//
// All four dense contractions share one block shape: 256 threads = 4 waves as
// 2 x 2, a 256 x 128 output tile per block, 128 x 64 per wave as 8 x 4 tiles of
// v_mfma_f32_16x16x32_bf16, K staged through LDS 32 at a time in two buffers.
// Both operands are K-contiguous in memory ("NT"): a lane's MFMA operand is
// 8 consecutive K values (one 16-byte LDS read). LDS rows are padded from 64 to
// 80 bytes so that the 16-byte fragment reads of 8 (or 16) consecutive lanes
// fall on distinct banks.
//
// 16x16x32 operand layout used here: lane l supplies row (l % 16) of A and
// column (l % 16) of B, each with K values 8*(l / 16) .. 8*(l / 16) + 7; the
// result lane l holds rows 4*(l / 16) + r, r = 0..3, of column (l % 16). Any
// consistent assignment of K values to (lane group, slot) gives the same sum.
//
// Kernels:
//   k_gateup   Z = SiLU(X W_g) * (X W_u)   M = slab rows, N = d_ff (64 gate +
//              64 up columns per block), K = d. Writes Z and Zt.
//   k_proj     Vt = scale * (C Proj)^T       M = slab rows, N = d, K = d.
//   k_apply    O = Z_j S_j                   M = chunk rows, N = d, K = d_ff,
//              batched over (sequence, chunk); MSE also writes
//              Rt = eta (V - O)^T.
//   k_update   W^T tile (256 d_ff x 128 d, fp32) held in the accumulators across
//              the chunks of a slab: per chunk, optionally write the bf16
//              snapshot S_j, then accumulate Zt_j . Vt_j over the chunk's tokens.
#include "internal.h"

namespace ipttt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 128, BK = 32;
constexpr int PITCH = BK + 8;                 // LDS row pitch in bf16 (80 bytes)
constexpr int NTHR = 256;
constexpr int A_PIECES = BM * (BK / 8) / NTHR;  // 16-byte loads per thread per step (4)
constexpr int B_PIECES = BN * (BK / 8) / NTHR;  // (2)
constexpr int A_STAGE = BM * PITCH, B_STAGE = BN * PITCH;
constexpr int MI = 8, NJ = 4;                 // 16x16 tiles per wave

struct Smem {
  __bf16 a[2][A_STAGE];
  __bf16 b[2][B_STAGE];
};

__device__ __forceinline__ uint4 ld16(const __bf16 *p) { return *(const uint4 *)p; }

// Logical block index: the hardware hands consecutive workgroups to the 8 XCDs
// in turn; give each XCD a contiguous range of logical tiles so that tiles
// that share operands also share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int x = bid % 8, q = bid / 8;
  return x * per + min(x, rem) + q;
}

// Per-thread loader state: the rows this thread copies into LDS (row index
// (tid / 4) + 64 i) and the 8-element K offset (tid % 4).
template <int NP>
struct RowLoader {
  const __bf16 *ptr[NP];  // row base (already offset to K = 0), nullptr = zero row
  uint4 v[NP];
  __device__ __forceinline__ void fetch(int k0, int q) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      v[i] = ptr[i] ? ld16(ptr[i] + k0 + 8 * q) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void stash(__bf16 *stage, int r0, int q) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) *(uint4 *)(stage + (r0 + 64 * i) * PITCH + 8 * q) = v[i];
  }
};

// One K-step of MFMAs for a wave: A rows arow0 + 16 i, B rows brow[j].
__device__ __forceinline__ void mma_step(const __bf16 *As, const __bf16 *Bs, int arow0,
                                         const int (&brow)[NJ], int lane, f32x4 (&acc)[MI][NJ]) {
  const int r = lane & 15, kq = 8 * (lane >> 4);
  bf16x8 a[MI], b[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) b[j] = *(const bf16x8 *)(Bs + (brow[j] + r) * PITCH + kq);
#pragma unroll
  for (int i = 0; i < MI; ++i) a[i] = *(const bf16x8 *)(As + (arow0 + 16 * i + r) * PITCH + kq);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Full K loop over nk steps with double-buffered LDS.
__device__ __forceinline__ void kloop(Smem &sm, RowLoader<A_PIECES> &la, RowLoader<B_PIECES> &lb,
                                      int nk, int tid, int arow0, const int (&brow)[NJ],
                                      f32x4 (&acc)[MI][NJ]) {
  const int lane = tid & 63, r0 = tid >> 2, q = tid & 3;
  la.fetch(0, q);
  lb.fetch(0, q);
  la.stash(sm.a[0], r0, q);
  lb.stash(sm.b[0], r0, q);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    if (s + 1 < nk) {
      la.fetch((s + 1) * BK, q);
      lb.fetch((s + 1) * BK, q);
    }
    mma_step(sm.a[cur], sm.b[cur], arow0, brow, lane, acc);
    if (s + 1 < nk) {
      la.stash(sm.a[cur ^ 1], r0, q);
      lb.stash(sm.b[cur ^ 1], r0, q);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MI][NJ]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Tile order inside a grid of (nm x nn) tiles: groups of GM row tiles, column
// tile slowest within a group, so neighbouring blocks share both operands.
__device__ __forceinline__ void tile_of(int id, int nm, int nn, int &tm, int &tn) {
  constexpr int GM = 8;
  const int group = id / (GM * nn);
  const int first = group * GM;
  const int gm = min(GM, nm - first);
  const int in = id % (GM * nn);
  tm = first + in % gm;
  tn = in / gm;
}

__device__ __forceinline__ int64_t slab_row_token(const Slab &s, int64_t p) {
  const int64_t j = p / s.Bp, i = p % s.Bp;
  if (i >= s.B || j >= s.nc) return -1;
  const int64_t t = s.tok0 + j * s.B + i;
  return t < s.L ? t : -1;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NTHR) void k_gateup(Slab s, const __bf16 *__restrict__ x,
                                                 const __bf16 *__restrict__ wg,
                                                 const __bf16 *__restrict__ wu,
                                                 __bf16 *__restrict__ z, __bf16 *__restrict__ zt) {
  __shared__ Smem sm;
  const int P = s.nc * s.Bp;
  const int nm = (P + BM - 1) / BM, nn = (s.F + 63) / 64;
  const int per_seq = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int n_seq = id / per_seq;
  int tm, tn;
  tile_of(id % per_seq, nm, nn, tm, tn);
  const int m0 = tm * BM, f0 = tn * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int r0 = tid >> 2;

  RowLoader<A_PIECES> la;
  RowLoader<B_PIECES> lb;
  const __bf16 *xs = x + n_seq * s.x_seq_stride;
#pragma unroll
  for (int i = 0; i < A_PIECES; ++i) {
    const int p = m0 + r0 + 64 * i;
    const int64_t t = p < P ? slab_row_token(s, p) : -1;
    la.ptr[i] = t >= 0 ? xs + t * s.d : nullptr;
  }
  // B rows 0..63: gate rows f0.., 64..127: up rows f0..
#pragma unroll
  for (int i = 0; i < B_PIECES; ++i) {
    const int rr = r0 + 64 * i;
    const int f = f0 + (rr & 63);
    lb.ptr[i] = f < s.F ? (rr < 64 ? wg : wu) + (int64_t)f * s.d : nullptr;
  }
  const int brow[NJ] = {wn * 32, wn * 32 + 16, 64 + wn * 32, 64 + wn * 32 + 16};
  f32x4 acc[MI][NJ];
  zero_acc(acc);
  kloop(sm, la, lb, s.d / BK, tid, wm * 128, brow, acc);

  __bf16 *zs = z + (int64_t)n_seq * s.Lp * s.F;
  __bf16 *zts = zt + (int64_t)n_seq * s.F * s.Lp;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = m0 + wm * 128 + 16 * i + 4 * (lane >> 4);
      const int f = f0 + wn * 32 + 16 * j + (lane & 15);
      if (p < P && f < s.F) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = acc[i][j][r], u = acc[i][j + 2][r];
          v[r] = (__bf16)(g / (1.f + __expf(-g)) * u);
        }
        *(bf16x4 *)(zts + (int64_t)f * s.Lp + p) = v;
#pragma unroll
        for (int r = 0; r < 4; ++r) zs[(int64_t)(p + r) * s.F + f] = v[r];
      }
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NTHR) void k_proj(Slab s, const __bf16 *__restrict__ c,
                                               const __bf16 *__restrict__ proj,
                                               __bf16 *__restrict__ vt, float scale) {
  __shared__ Smem sm;
  const int P = s.nc * s.Bp;
  const int nm = (P + BM - 1) / BM, nn = (s.d + BN - 1) / BN;
  const int per_seq = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int n_seq = id / per_seq;
  int tm, tn;
  tile_of(id % per_seq, nm, nn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int r0 = tid >> 2;
  RowLoader<A_PIECES> la;
  RowLoader<B_PIECES> lb;
  const __bf16 *cs = c + (int64_t)n_seq * s.Lp * s.d;
#pragma unroll
  for (int i = 0; i < A_PIECES; ++i) {
    const int p = m0 + r0 + 64 * i;
    la.ptr[i] = p < P ? cs + (int64_t)p * s.d : nullptr;
  }
#pragma unroll
  for (int i = 0; i < B_PIECES; ++i) {
    const int n = n0 + r0 + 64 * i;
    lb.ptr[i] = n < s.d ? proj + (int64_t)n * s.d : nullptr;
  }
  const int brow[NJ] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  f32x4 acc[MI][NJ];
  zero_acc(acc);
  kloop(sm, la, lb, s.d / BK, tid, wm * 128, brow, acc);

  __bf16 *vts = vt + (int64_t)n_seq * s.d * s.Lp;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int p = m0 + wm * 128 + 16 * i + 4 * (lane >> 4);
      const int n = n0 + wn * 64 + 16 * j + (lane & 15);
      if (p < P && n < s.d) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(scale * acc[i][j][r]);
        *(bf16x4 *)(vts + (int64_t)n * s.Lp + p) = v;
      }
    }
}

// ---------------------------------------------------------------------------
// O rows of chunks [j0, j0 + nj) of every sequence: O_j = Z_j S_j^T-stored.
__global__ __launch_bounds__(NTHR) void k_apply(Slab s, int j0, int nj, const __bf16 *__restrict__ z,
                                                const __bf16 *__restrict__ snap,
                                                int64_t snap_seq_stride, int64_t snap_chunk_stride,
                                                float *__restrict__ o, const __bf16 *__restrict__ vt,
                                                __bf16 *__restrict__ rt) {
  __shared__ Smem sm;
  const int nm = (s.Bp + BM - 1) / BM, nn = (s.d + BN - 1) / BN;
  const int per_chunk = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bz = id / per_chunk;
  const int n_seq = bz / nj, jl = bz % nj, j = j0 + jl;
  int tm, tn;
  tile_of(id % per_chunk, nm, nn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int r0 = tid >> 2;
  RowLoader<A_PIECES> la;
  RowLoader<B_PIECES> lb;
  const __bf16 *zs = z + (int64_t)n_seq * s.Lp * s.F + (int64_t)j * s.Bp * s.F;
  const __bf16 *ss = snap + n_seq * snap_seq_stride + jl * snap_chunk_stride;
#pragma unroll
  for (int i = 0; i < A_PIECES; ++i) {
    const int m = m0 + r0 + 64 * i;
    la.ptr[i] = m < s.Bp ? zs + (int64_t)m * s.F : nullptr;
  }
#pragma unroll
  for (int i = 0; i < B_PIECES; ++i) {
    const int n = n0 + r0 + 64 * i;
    lb.ptr[i] = n < s.d ? ss + (int64_t)n * s.F : nullptr;
  }
  const int brow[NJ] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  f32x4 acc[MI][NJ];
  zero_acc(acc);
  kloop(sm, la, lb, s.F / BK, tid, wm * 128, brow, acc);

  const int64_t chunk_tok0 = s.tok0 + (int64_t)j * s.B;
  float *os = o + n_seq * s.x_seq_stride;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int m = m0 + wm * 128 + 16 * i + 4 * (lane >> 4);
      const int n = n0 + wn * 64 + 16 * jj + (lane & 15);
      if (n >= s.d || m >= s.Bp) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = chunk_tok0 + m + r;
        if (m + r < s.B && t < s.L) os[t * s.d + n] = acc[i][jj][r];
      }
      if (rt) {
        const bf16x4 v = *(const bf16x4 *)(vt + (int64_t)n_seq * s.d * s.Lp + (int64_t)n * s.Lp +
                                           (int64_t)j * s.Bp + m);
        bf16x4 rv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t t = chunk_tok0 + m + r;
          const bool valid = m + r < s.B && t < s.L;
          rv[r] = (__bf16)(valid ? s.eta * ((float)v[r] - acc[i][jj][r]) : 0.f);
        }
        *(bf16x4 *)(rt + (int64_t)n_seq * s.d * s.Bp + (int64_t)n * s.Bp + m) = rv;
      }
    }
}

// ---------------------------------------------------------------------------
// W^T tile update: rows f (d_ff), columns c (d), K = tokens. The fp32 tile
// lives in the accumulators for all chunks [j_first, j_first + n_chunks).
// a_src = Zt (rows f, token-contiguous), b_src = Vt or Rt (rows c).
// snap_each_chunk: write S[j] = bf16(W) before chunk j's accumulation;
// snap_after: write S = bf16(W) after the last chunk.
__global__ __launch_bounds__(NTHR) void k_update(Slab s, int j_first, int n_chunks,
                                                 const __bf16 *__restrict__ zt,
                                                 const __bf16 *__restrict__ bsrc, int64_t b_ld,
                                                 int64_t b_seq_stride, int64_t b_chunk_stride,
                                                 float *__restrict__ w, __bf16 *__restrict__ snap,
                                                 int64_t snap_seq_stride, int64_t snap_chunk_stride,
                                                 int snap_each_chunk, int snap_after) {
  __shared__ Smem sm;
  const int nm = (s.F + BM - 1) / BM, nn = (s.d + BN - 1) / BN;
  const int per_seq = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int n_seq = id / per_seq;
  int tm, tn;
  tile_of(id % per_seq, nm, nn, tm, tn);
  const int f0 = tm * BM, c0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int r0 = tid >> 2, q = tid & 3;
  const int64_t dF = (int64_t)s.d * s.F;
  float *ws = w + n_seq * dF;

  // accumulators <- W tile: lane holds W^T[c][f .. f+3]
  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int f = f0 + wm * 128 + 16 * i + 4 * (lane >> 4);
      const int c = c0 + wn * 64 + 16 * jj + (lane & 15);
      acc[i][jj] = (f < s.F && c < s.d) ? *(const f32x4 *)(ws + (int64_t)c * s.F + f)
                                         : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  auto write_snap = [&](__bf16 *dst) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int f = f0 + wm * 128 + 16 * i + 4 * (lane >> 4);
        const int c = c0 + wn * 64 + 16 * jj + (lane & 15);
        if (f < s.F && c < s.d) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)acc[i][jj][r];
          *(bf16x4 *)(dst + (int64_t)c * s.F + f) = v;
        }
      }
  };

  RowLoader<A_PIECES> la;
  RowLoader<B_PIECES> lb;
  const int brow[NJ] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  const int steps = s.Bp / BK;
  for (int jc = 0; jc < n_chunks; ++jc) {
    const int j = j_first + jc;
    if (snap_each_chunk) write_snap(snap + n_seq * snap_seq_stride + jc * snap_chunk_stride);
#pragma unroll
    for (int i = 0; i < A_PIECES; ++i) {
      const int f = f0 + r0 + 64 * i;
      la.ptr[i] = f < s.F ? zt + (int64_t)n_seq * s.F * s.Lp + (int64_t)f * s.Lp + (int64_t)j * s.Bp
                          : nullptr;
    }
#pragma unroll
    for (int i = 0; i < B_PIECES; ++i) {
      const int c = c0 + r0 + 64 * i;
      lb.ptr[i] = c < s.d ? bsrc + n_seq * b_seq_stride + (int64_t)c * b_ld + jc * b_chunk_stride
                          : nullptr;
    }
    kloop(sm, la, lb, steps, tid, wm * 128, brow, acc);
  }
  if (snap_after) write_snap(snap + n_seq * snap_seq_stride);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int f = f0 + wm * 128 + 16 * i + 4 * (lane >> 4);
      const int c = c0 + wn * 64 + 16 * jj + (lane & 15);
      if (f < s.F && c < s.d) *(f32x4 *)(ws + (int64_t)c * s.F + f) = acc[i][jj];
    }
}

inline unsigned blocks(int64_t n) { return (unsigned)n; }

}  // namespace

bool mfma_supported(int d, int F) { return d % BK == 0 && F % BK == 0; }

hipError_t mf_gateup(const Slab &s, const __bf16 *x, const Weights &w, const WsPtrs &ws,
                     hipStream_t st) {
  const int64_t P = (int64_t)s.nc * s.Bp;
  const int64_t nb = ((P + BM - 1) / BM) * ((s.F + 63) / 64) * s.n_seq;
  hipLaunchKernelGGL(k_gateup, dim3(blocks(nb)), dim3(NTHR), 0, st, s, x, (const __bf16 *)w.w_gate,
                     (const __bf16 *)w.w_up, (__bf16 *)ws.z, (__bf16 *)ws.zt);
  return hipGetLastError();
}

hipError_t mf_proj(const Slab &s, const Weights &w, const WsPtrs &ws, hipStream_t st) {
  const int64_t P = (int64_t)s.nc * s.Bp;
  const int64_t nb = ((P + BM - 1) / BM) * ((s.d + BN - 1) / BN) * s.n_seq;
  hipLaunchKernelGGL(k_proj, dim3(blocks(nb)), dim3(NTHR), 0, st, s, (const __bf16 *)ws.c,
                     (const __bf16 *)w.proj, (__bf16 *)ws.vt, s.mse ? 1.f : s.eta);
  return hipGetLastError();
}

hipError_t mf_apply(const Slab &s, int j0, int nj, const WsPtrs &ws, float *o, hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  const int64_t snap_seq = s.mse ? dF : (int64_t)s.nc_cap * dF;
  const int64_t snap_chunk = s.mse ? 0 : dF;
  const __bf16 *snap = (const __bf16 *)ws.s + (s.mse ? 0 : (int64_t)j0 * dF);
  const int64_t nb = ((s.Bp + BM - 1) / BM) * ((s.d + BN - 1) / BN) * (int64_t)nj * s.n_seq;
  hipLaunchKernelGGL(k_apply, dim3(blocks(nb)), dim3(NTHR), 0, st, s, j0, nj,
                     (const __bf16 *)ws.z, snap, snap_seq, snap_chunk, o, (const __bf16 *)ws.vt,
                     s.mse ? (__bf16 *)ws.rt : nullptr);
  return hipGetLastError();
}

hipError_t mf_update_scan(const Slab &s, const WsPtrs &ws, float *w_state, hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  const int64_t nb = ((s.F + BM - 1) / BM) * ((s.d + BN - 1) / BN) * s.n_seq;
  // B operand: Vt rows c, chunk jc at column offset jc * Bp
  hipLaunchKernelGGL(k_update, dim3(blocks(nb)), dim3(NTHR), 0, st, s, 0, s.nc,
                     (const __bf16 *)ws.zt, (const __bf16 *)ws.vt, s.Lp, (int64_t)s.d * s.Lp,
                     (int64_t)s.Bp, w_state, (__bf16 *)ws.s, (int64_t)s.nc_cap * dF, dF, 1, 0);
  return hipGetLastError();
}

hipError_t mf_update_one(const Slab &s, int j, const WsPtrs &ws, float *w_state, hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  const int64_t nb = ((s.F + BM - 1) / BM) * ((s.d + BN - 1) / BN) * s.n_seq;
  // B operand: Rt [n][d][Bp] of chunk j
  hipLaunchKernelGGL(k_update, dim3(blocks(nb)), dim3(NTHR), 0, st, s, j, 1,
                     (const __bf16 *)ws.zt, (const __bf16 *)ws.rt, (int64_t)s.Bp,
                     (int64_t)s.d * s.Bp, (int64_t)0, w_state, (__bf16 *)ws.s, dF, (int64_t)0, 0, 1);
  return hipGetLastError();
}

}  // namespace ipttt
