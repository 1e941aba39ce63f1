// Backward of the fast-weight scan, bf16 MFMA path (gfx950).
//
// The gradient pass reruns the forward scan (gate/up with its pre-activations,
// conv, projection, update scan with one W snapshot per chunk), then:
//   dOt = bf16(dO)^T                         transpose, chunk-padded rows
//   reverse scan  G += Z_j^T dO_j, last chunk to first, T_j = bf16(G_{j+1})
//   dZ_j = dO_j W_j^T + (eta V_j) G_{j+1}^T  -> dA, dU through SiLU gating
//   dV_j = eta Z_j G_{j+1}
//   dC = dV Proj^T, dProj = C^T dV            (summed over sequences)
//   dX = dA W_g^T + dU W_u^T, dW_g = X^T dA, dW_u = X^T dU
//   dE, dconv: the conv's adjoint inside each chunk
//   dW_0 = G after the first chunk, summed over sequences
// Every contraction runs on one MFMA GEMM kernel (k_gemm) whose operands may
// each be stored K-contiguous or K-major, with up to two K phases summed into
// the same accumulators, a two-level batch (sequence, chunk) and K split into
// segments (one per sequence) for the weight gradients. The epilogue is a
// functor that receives four consecutive output rows of one column.
#include <algorithm>
#include <type_traits>

#include "mfma_common.h"

namespace ipttt {
namespace mfma {

// One operand of one K phase. Element (row r, k) of a K-contiguous operand is
// p[r * ld + k]; of a K-major operand, p[k * ld + r]. Batch item (b1, b2) and
// K segment g add b1 * s1 + b2 * s2 + g * sseg. Rows (K-contiguous) or columns
// (K-major) at or past lim are clamped in bounds; the outputs they feed are
// outside the problem and never written.
struct GOp {
  const __bf16 *p;
  int64_t ld, s1, s2, sseg, lim;
};
struct GPhase {
  GOp a, b;
  int K;  // per segment, a multiple of BK
};
struct GProb {
  int M, N;       // output rows and columns per batch item
  int nb1, nb2;   // batch = nb1 x nb2 items
  int nseg;       // K segments summed into one output
  int nph;        // 1 or 2 phases
  GPhase ph[2];
};

// Epilogues that read memory (In, load, store) get their loads issued for
// part of a tile at a time before any of that part's stores: a store with a lane
// predicate makes every later load wait for it, so loads interleaved with
// stores would cost one memory round trip per output group.
template <class E, class = void>
struct EpiLoads : std::false_type {};
template <class E>
struct EpiLoads<E, std::void_t<typename E::In>> : std::true_type {};

template <class C, bool TA, bool TB, class Epi>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_gemm(
    GProb g, Epi epi) {
  using GL = GLoaders<C, TA, TB>;
  static_assert(GL::SMEM * 2 <= 160 * 1024, "LDS overflow");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[GL::SMEM];
  using M = typename C::M;
  const int nm = (g.M + C::BM - 1) / C::BM, nn = (g.N + C::BN - 1) / C::BN;
  const int per = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per, b1 = b / g.nb2, b2 = b % g.nb2;
  int tm, tn;
  tile_of<C::GM>(id % per, nm, nn, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r0 = tid / C::KP;
  int brow[C::NJ];
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj) brow[jj] = wn * C::WTN + C::FM * jj;
  typename C::acc_t acc[C::MI][C::NJ];
  zero_acc<C>(acc);
  typename GL::LA la;
  typename GL::LB lb;
#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
    if (ph >= g.nph) break;
    const GOp A = g.ph[ph].a, Bo = g.ph[ph].b;
    for (int sg = 0; sg < g.nseg; ++sg) {
      const __bf16 *pa = A.p + b1 * A.s1 + b2 * A.s2 + sg * A.sseg;
      const __bf16 *pb = Bo.p + b1 * Bo.s1 + b2 * Bo.s2 + sg * Bo.sseg;
      if constexpr (!TA && !TB && C::SWZ) {
        // both operands K-contiguous: direct LDS copies into swizzled rows,
        // pipelined fragments interleaved with the MFMAs
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        DmaLoader<C, C::BM> da;
        DmaLoader<C, C::BN> db;
        da.init(wv, lane, [&](int r) { return pa + min((int64_t)m0 + r, A.lim - 1) * A.ld; });
        db.init(wv, lane, [&](int r) { return pb + min((int64_t)n0 + r, Bo.lim - 1) * Bo.ld; });
        kloop_dma_pl<C, 2, true>(
            smem, da, db, g.ph[ph].K / C::BK, wv, lane, wm * C::WTM, brow, acc,
            [](int st, int64_t &ka, int64_t &kb) { ka = kb = (int64_t)st * C::BK; }, [](int) {},
            [](int) {});
        continue;
      }
      if constexpr (TA) {
        la.ld = A.ld;
#pragma unroll
        for (int i = 0; i < GL::LA::NP; ++i)
          la.ptr[i] = pa + (int64_t)GL::LA::krow(tid, i) * A.ld +
                      min((int64_t)m0 + GL::LA::col(tid, i), A.lim - 8);
      } else {
#pragma unroll
        for (int i = 0; i < C::A_PIECES; ++i)
          la.ptr[i] = pa + min((int64_t)m0 + r0 + C::RPP * i, A.lim - 1) * A.ld;
      }
      if constexpr (TB) {
        lb.ld = Bo.ld;
#pragma unroll
        for (int i = 0; i < GL::LB::NP; ++i)
          lb.ptr[i] = pb + (int64_t)GL::LB::krow(tid, i) * Bo.ld +
                      min((int64_t)n0 + GL::LB::col(tid, i), Bo.lim - 8);
      } else {
#pragma unroll
        for (int i = 0; i < C::B_PIECES; ++i)
          lb.ptr[i] = pb + min((int64_t)n0 + r0 + C::RPP * i, Bo.lim - 1) * Bo.ld;
      }
      if constexpr (C::WM * C::WN >= 8)  // two waves per SIMD: interleaved loop
        kloop_g_il<C, TA, TB>(smem, la, lb, g.ph[ph].K / C::BK, tid, wm * C::WTM, brow, acc);
      else
        kloop_g<C, TA, TB>(smem, la, lb, g.ph[ph].K / C::BK, tid, wm * C::WTM, brow, acc);
    }
  }
  if constexpr (EpiLoads<Epi>::value) {
    // row tiles loaded together: half the wave tile at one wave per SIMD, a
    // quarter at two (whose 256 registers hold less beside the accumulators)
    constexpr int H = C::WM * C::WN >= 8 ? C::MI / 4 : C::MI / 2;
    static_assert(C::MI % 4 == 0, "quarters of the wave tile");
#pragma unroll
    for (int h0 = 0; h0 < C::MI; h0 += H) {
      typename Epi::In in[H][C::NJ][M::NG];
#pragma unroll
      for (int i = 0; i < H; ++i)
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
          for (int q = 0; q < M::NG; ++q) {
            // clamped in bounds and loaded unconditionally (M is a multiple of 4)
            const int m = min(m0 + wm * C::WTM + C::FM * (h0 + i) + M::rrow(lane, q), g.M - 4);
            const int n = min(n0 + wn * C::WTN + C::FM * jj + M::rcol(lane), g.N - 1);
            in[i][jj][q] = epi.load(b1, b2, m, n);
          }
#pragma unroll
      for (int i = 0; i < H; ++i)
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
          for (int q = 0; q < M::NG; ++q) {
            const int m = m0 + wm * C::WTM + C::FM * (h0 + i) + M::rrow(lane, q);
            const int n = n0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
            if (m < g.M && n < g.N) epi.store(b1, b2, m, n, get4(acc[h0 + i][jj], q), in[i][jj][q]);
          }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
        for (int q = 0; q < M::NG; ++q) {
          const int m = m0 + wm * C::WTM + C::FM * i + M::rrow(lane, q);
          const int n = n0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
          if (m < g.M && n < g.N) epi(b1, b2, m, n, get4(acc[i][jj], q));
        }
  }
}

// ---- epilogues (m .. m + 3 are consecutive output rows, n one column) -------

// dZ of chunk b2 of sequence b1 -> dA = dZ U SiLU'(A), dU = dZ SiLU(A), from
// the pre-activations; all [n][F][Lp] bf16, row n = f, column = slab row.
struct EpiDZ {
  const __bf16 *at, *ut;
  __bf16 *dat, *dut;
  int64_t seq_stride, Lp;
  int Bp;
  struct In {
    bf16x4 a, u;
  };
  __device__ int64_t offset(int b1, int b2, int m, int n) const {
    return b1 * seq_stride + n * Lp + (int64_t)b2 * Bp + m;
  }
  __device__ In load(int b1, int b2, int m, int n) const {
    const int64_t off = offset(b1, b2, m, n);
    return {*(const bf16x4 *)(at + off), *(const bf16x4 *)(ut + off)};
  }
  __device__ void store(int b1, int b2, int m, int n, f32x4 v, In in) const {
    const int64_t off = offset(b1, b2, m, n);
    bf16x4 da, du;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float A = (float)in.a[r], U = (float)in.u[r];
      const float sg = fast_sigmoid(A);
      da[r] = (__bf16)(v[r] * U * sg * (1.f + A * (1.f - sg)));
      du[r] = (__bf16)(v[r] * A * sg);
    }
    *(bf16x4 *)(dat + off) = da;
    *(bf16x4 *)(dut + off) = du;
  }
};

// scale * acc -> bf16 [n][d][Lp], row n = channel, column = slab row of chunk b2.
struct EpiRowsT {
  __bf16 *out;
  int64_t seq_stride, Lp;
  int Bp;
  float scale;
  __device__ void operator()(int b1, int b2, int m, int n, f32x4 v) const {
    bf16x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = (__bf16)(scale * v[r]);
    *(bf16x4 *)(out + b1 * seq_stride + n * Lp + (int64_t)b2 * Bp + m) = o;
  }
};

// fp32 out[b1 * s1][row][col], row-major with pitch ld; b2 picks out0 / out1.
struct EpiRows {
  float *out0, *out1;
  int64_t s1, ld;
  __device__ void operator()(int b1, int b2, int m, int n, f32x4 v) const {
    float *o = (b2 ? out1 : out0) + b1 * s1;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[(int64_t)(m + r) * ld + n] = v[r];
  }
};

// MSE rule, chunk at column col0: P = Z_j G_{j+1} -> dY = dO - eta P and
// dV = eta P, both bf16 [n][d][Lp] (row n = channel), dO read from dOt.
struct EpiMseP {
  const __bf16 *dot;
  __bf16 *dyt, *dvt;
  int64_t seq_stride, Lp, col0;
  float eta;
  struct In {
    bf16x4 o;
  };
  __device__ In load(int b1, int, int m, int n) const {
    return {*(const bf16x4 *)(dot + b1 * seq_stride + n * Lp + col0 + m)};
  }
  __device__ void store(int b1, int, int m, int n, f32x4 v, In in) const {
    const int64_t off = b1 * seq_stride + n * Lp + col0 + m;
    bf16x4 dy, dv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dy[r] = (__bf16)((float)in.o[r] - eta * v[r]);
      dv[r] = (__bf16)(eta * v[r]);
    }
    *(bf16x4 *)(dyt + off) = dy;
    *(bf16x4 *)(dvt + off) = dv;
  }
};

// fp32 partial sums: out[b2 * s2][row][col], pitch ld (one slice of a split K).
struct EpiRowsSplit {
  float *out;
  int64_t s2, ld;
  __device__ void operator()(int, int b2, int m, int n, f32x4 v) const {
    float *o = out + b2 * s2;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[(int64_t)(m + r) * ld + n] = v[r];
  }
};

// fp32 out[seq][token][col] for slab rows that are tokens (padding rows dropped).
struct EpiTok {
  float *out;
  Slab s;
  __device__ void operator()(int b1, int, int m, int n, f32x4 v) const {
    const int jc = m / s.Bp, ic = m - jc * s.Bp;
    const int64_t t0 = s.tok0 + (int64_t)jc * s.B + ic;
    float *o = out + b1 * s.x_seq_stride;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (jc < s.nc && ic + r < s.B && t0 + r < s.L) o[(t0 + r) * s.d + n] = v[r];
  }
};

template <class C, bool TA, bool TB, class Epi>
hipError_t launch_gemm(const GProb &g, const Epi &epi, hipStream_t st) {
  const int64_t nb = (int64_t)((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN) * g.nb1 *
                     g.nb2;
  if (nb <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm<C, TA, TB, Epi>), dim3((unsigned)nb), dim3(C::NTHR), 0, st, g, epi);
  return hipGetLastError();
}

// transposed operands: K-major rows padded by 16 elements (conflict-free
// transposing reads, as for the forward's apply)
using BwCfg = Cfg<2, 4, 64, 16, 16, 16>;
using BwSmallCfg = Cfg<1, 2, 64, 16, 16, 16>;  // chunk-batched problems with short chunks
using BwNTCfg = Cfg<2, 4, 64, 16, 0, 8>;       // both operands K-contiguous: direct copies

// ---- elementwise / vector kernels --------------------------------------------

// in [n][L][d] token rows (TI = float or bf16) -> out bf16 [n][d][Lp] with the
// slab's chunk-padded columns (padding columns 0). 64 x 64 tiles through LDS.
template <typename TI>
__global__ __launch_bounds__(256) void k_transpose(Slab s, const TI *__restrict__ in,
                                                   __bf16 *__restrict__ out) {
  __shared__ float tile[64][65];
  const int P = s.nc * s.Bp;
  const int tp = blockIdx.x, tc = blockIdx.y, n_seq = blockIdx.z;
  const int p0 = tp * 64, c0 = tc * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const TI *src = in + n_seq * s.x_seq_stride;
  for (int r = ty; r < 64; r += 4) {
    const int p = p0 + r, c = c0 + tx;
    float v = 0.f;
    if (p < P && c < s.d) {
      const int64_t t = slab_row_token(s, p);
      if (t >= 0) v = (float)src[t * s.d + c];
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  __bf16 *dst = out + (int64_t)n_seq * s.d * s.Lp;
  for (int r = ty; r < 64; r += 4) {
    const int c = c0 + r, p = p0 + tx;
    if (c < s.d && p < P) dst[(int64_t)c * s.Lp + p] = (__bf16)tile[tx][r];
  }
}

// Adjoint of the chunk-padded depthwise conv. A thread owns 8 channels and
// CONV_BW_RUN slab rows of one chunk: dE[t] = sum_q w[q] dC[t - q] (rows before
// the chunk start contribute nothing), and its share of dconv[c][q] =
// sum_t dC[t] E[t + q] (E zero past the chunk end) goes to part[run][c][q].
constexpr int CONV_BW_RUN = kConvBwRun;

template <int KC>
__global__ __launch_bounds__(256) void k_conv_bwd(Slab s, const float *__restrict__ dc,
                                                  const __bf16 *__restrict__ e,
                                                  const __bf16 *__restrict__ cw,
                                                  float *__restrict__ de,
                                                  float *__restrict__ part) {
  const int groups = s.d / 8;
  const int64_t runs_per_seq = (int64_t)s.nc * (s.Bp / CONV_BW_RUN);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= runs_per_seq * groups * s.n_seq) return;
  const int g = (int)(gid % groups);
  const int64_t run = (gid / groups) % runs_per_seq;
  const int n_seq = (int)(gid / groups / runs_per_seq);
  const int64_t p0 = run * CONV_BW_RUN;
  const int64_t j = p0 / s.Bp, i0 = p0 % s.Bp;
  const int64_t cs = s.tok0 + j * s.B;
  const int64_t ce = min(cs + (int64_t)s.B, s.L);
  const int ch = 8 * g;
  float w[KC][8];
#pragma unroll
  for (int q = 0; q < KC; ++q)
#pragma unroll
    for (int k = 0; k < 8; ++k) w[q][k] = (float)cw[(ch + k) * KC + q];
  // dC rows i0 - (KC - 1) .. i0 + RUN - 1 of the chunk (zero before its start)
  float dcw[CONV_BW_RUN + KC - 1][8];
  const float *dcs = dc + (int64_t)n_seq * s.Lp * s.d + (j * s.Bp) * s.d + ch;
#pragma unroll
  for (int r = 0; r < CONV_BW_RUN + KC - 1; ++r) {
    const int64_t i = i0 - (KC - 1) + r;
#pragma unroll
    for (int k = 0; k < 8; ++k) dcw[r][k] = i >= 0 ? dcs[i * s.d + k] : 0.f;
  }
  const __bf16 *es = e + n_seq * s.x_seq_stride + ch;
  float acc[KC][8];
#pragma unroll
  for (int q = 0; q < KC; ++q)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[q][k] = 0.f;
  float *des = de + n_seq * s.x_seq_stride + ch;
#pragma unroll
  for (int r = 0; r < CONV_BW_RUN; ++r) {
    const int64_t t = cs + i0 + r;
    const bool real = i0 + r < s.B && t < ce;
    // dE at this row: taps q read dC at row - q
    if (real) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < KC; ++q) a = fmaf(w[q][k], dcw[r + KC - 1 - q][k], a);
        des[t * s.d + k] = a;
      }
    }
    // dconv: dC at this row times E at row + q (inside the chunk)
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const bool in = i0 + r + q < s.B && t + q < ce;
      if (in) {
        const bf16x8 ev = *(const bf16x8 *)(es + (t + q) * s.d);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[q][k] = fmaf(dcw[r + KC - 1][k], (float)ev[k], acc[q][k]);
      }
    }
  }
  float *pp = part + ((int64_t)n_seq * runs_per_seq + run) * s.d * KC + (int64_t)ch * KC;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int q = 0; q < KC; ++q) pp[k * KC + q] = acc[q][k];
}

// Row group y of gridDim.y: out[y * len + i] = sum over its rows r of
// in[r * len + i], rows in ascending order (a fixed summation order).
__global__ __launch_bounds__(256) void k_sum_rows(const float *__restrict__ in, int64_t rows,
                                                 int64_t len, float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= len) return;
  const int64_t per = (rows + gridDim.y - 1) / gridDim.y;
  const int64_t r0 = blockIdx.y * per, r1 = min(rows, r0 + per);
  float a = 0.f;
  for (int64_t r = r0; r < r1; ++r) a += in[r * len + i];
  out[blockIdx.y * len + i] = a;
}

__global__ __launch_bounds__(256) void k_fill(float *__restrict__ p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace mfma

// ---- host wrappers -------------------------------------------------------------
using namespace mfma;

namespace {
GOp kcontig(const __bf16 *p, int64_t ld, int64_t lim, int64_t s1 = 0, int64_t s2 = 0,
            int64_t sseg = 0) {
  return GOp{p, ld, s1, s2, sseg, lim};
}
GOp kmajor(const __bf16 *p, int64_t ld, int64_t lim, int64_t s1 = 0, int64_t s2 = 0,
           int64_t sseg = 0) {
  return GOp{p, ld, s1, s2, sseg, lim};
}
}  // namespace

hipError_t bw_transpose_f32(const Slab &s, const float *in, __bf16 *out, hipStream_t st) {
  const int P = s.nc * s.Bp;
  hipLaunchKernelGGL(k_transpose<float>, dim3((P + 63) / 64, (s.d + 63) / 64, s.n_seq), dim3(256), 0,
                     st, s, in, out);
  return hipGetLastError();
}
hipError_t bw_transpose_bf16(const Slab &s, const __bf16 *in, __bf16 *out, hipStream_t st) {
  const int P = s.nc * s.Bp;
  hipLaunchKernelGGL(k_transpose<__bf16>, dim3((P + 63) / 64, (s.d + 63) / 64, s.n_seq), dim3(256),
                     0, st, s, in, out);
  return hipGetLastError();
}

hipError_t bw_dz(const Slab &s, const BwBufs &b, const __bf16 *a0, const __bf16 *a1,
                 hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  GProb g{};
  g.M = s.Bp;
  g.N = s.F;
  g.nb1 = s.n_seq;
  g.nb2 = s.nc;
  g.nseg = 1;
  g.nph = 2;
  // phase 0: dY_j W_j^T (A = a0 columns of chunk j, B = S_j [d][F], both K-major);
  // dY = dO for the linear rule
  g.ph[0].a = kmajor(a0, s.Lp, s.Bp, (int64_t)s.d * s.Lp, s.Bp);
  g.ph[0].b = kmajor(b.snap_w, s.F, s.F, (int64_t)s.nc_cap * dF, dF);
  g.ph[0].K = s.d;
  // phase 1: a1_j G_{j+1}^T with a1 = eta V (linear) or eta (V - O) = -eta R (MSE)
  g.ph[1].a = kmajor(a1, s.Lp, s.Bp, (int64_t)s.d * s.Lp, s.Bp);
  g.ph[1].b = kmajor(b.snap_g, s.F, s.F, (int64_t)s.nc_cap * dF, dF);
  g.ph[1].K = s.d;
  EpiDZ e{b.at, b.ut, b.dat, b.dut, (int64_t)s.F * s.Lp, s.Lp, s.Bp};
  if (s.Bp < BwCfg::BM) return launch_gemm<BwSmallCfg, true, true>(g, e, st);
  return launch_gemm<BwCfg, true, true>(g, e, st);
}

hipError_t bw_dv(const Slab &s, const BwBufs &b, hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  GProb g{};
  g.M = s.Bp;
  g.N = s.d;
  g.nb1 = s.n_seq;
  g.nb2 = s.nc;
  g.nseg = 1;
  g.nph = 1;
  // eta Z_j G_{j+1}: A = Zt columns of chunk j (K-major), B = T_j rows c (K-contiguous over f)
  g.ph[0].a = kmajor(b.zt, s.Lp, s.Bp, (int64_t)s.F * s.Lp, s.Bp);
  g.ph[0].b = kcontig(b.snap_g, s.F, s.d, (int64_t)s.nc_cap * dF, dF);
  g.ph[0].K = s.F;
  EpiRowsT e{b.dvt, (int64_t)s.d * s.Lp, s.Lp, s.Bp, s.eta};
  if (s.Bp < BwCfg::BM) return launch_gemm<BwSmallCfg, true, false>(g, e, st);
  return launch_gemm<BwCfg, true, false>(g, e, st);
}

hipError_t bw_mse_p(const Slab &s, int j, const BwBufs &b, hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  GProb g{};
  g.M = s.Bp;
  g.N = s.d;
  g.nb1 = s.n_seq;
  g.nb2 = 1;
  g.nseg = 1;
  g.nph = 1;
  // Z_j G_{j+1}: A = Zt columns of chunk j (K-major), B = T_j rows c (K-contiguous over f)
  g.ph[0].a = kmajor(b.zt + (int64_t)j * s.Bp, s.Lp, s.Bp, (int64_t)s.F * s.Lp);
  g.ph[0].b = kcontig(b.snap_g + (int64_t)j * dF, s.F, s.d, (int64_t)s.nc_cap * dF);
  g.ph[0].K = s.F;
  EpiMseP e{b.dot, b.dyt, b.dvt, (int64_t)s.d * s.Lp, s.Lp, (int64_t)j * s.Bp, s.eta};
  const int64_t big = ((s.Bp + BwCfg::BM - 1) / BwCfg::BM) * ((s.d + BwCfg::BN - 1) / BwCfg::BN) *
                      s.n_seq;
  if (big < 512) return launch_gemm<BwSmallCfg, true, false>(g, e, st);
  return launch_gemm<BwCfg, true, false>(g, e, st);
}

hipError_t bw_dc(const Slab &s, const BwBufs &b, const void *proj, hipStream_t st) {
  GProb g{};
  g.M = s.nc * s.Bp;
  g.N = s.d;
  g.nb1 = s.n_seq;
  g.nb2 = 1;
  g.nseg = 1;
  g.nph = 1;
  // dC[t][i] = sum_c dV[t][c] proj[c][i]: A = dVt (K-major), B = proj rows c (K-major over i)
  g.ph[0].a = kmajor(b.dvt, s.Lp, s.Lp, (int64_t)s.d * s.Lp);
  g.ph[0].b = kmajor((const __bf16 *)proj, s.d, s.d);
  g.ph[0].K = s.d;
  EpiRows e{b.dc, nullptr, s.Lp * s.d, s.d};
  return launch_gemm<BwCfg, true, true>(g, e, st);
}

hipError_t bw_dx(const Slab &s, const BwBufs &b, const void *wg, const void *wu, float *dx,
                 hipStream_t st) {
  GProb g{};
  g.M = s.nc * s.Bp;
  g.N = s.d;
  g.nb1 = s.n_seq;
  g.nb2 = 1;
  g.nseg = 1;
  g.nph = 2;
  // dX[t][i] = sum_f dA[t][f] w_gate[f][i] + dU[t][f] w_up[f][i]
  g.ph[0].a = kmajor(b.dat, s.Lp, s.Lp, (int64_t)s.F * s.Lp);
  g.ph[0].b = kmajor((const __bf16 *)wg, s.d, s.d);
  g.ph[0].K = s.F;
  g.ph[1].a = kmajor(b.dut, s.Lp, s.Lp, (int64_t)s.F * s.Lp);
  g.ph[1].b = kmajor((const __bf16 *)wu, s.d, s.d);
  g.ph[1].K = s.F;
  EpiTok e{dx, s};
  return launch_gemm<BwCfg, true, true>(g, e, st);
}

hipError_t bw_dw(const Slab &s, const BwBufs &b, float *dwg, float *dwu, hipStream_t st) {
  GProb g{};
  g.M = s.F;
  g.N = s.d;
  g.nb1 = 1;
  g.nb2 = 2;  // gate, up
  g.nseg = s.n_seq;
  g.nph = 1;
  // dW[f][i] = sum over tokens of all sequences dA[t][f] X[t][i]; dUt follows dAt
  g.ph[0].a = kcontig(b.dat, s.Lp, s.F, 0, b.dut - b.dat, (int64_t)s.F * s.Lp);
  g.ph[0].b = kcontig(b.xt, s.Lp, s.d, 0, 0, (int64_t)s.d * s.Lp);
  g.ph[0].K = (int)s.Lp;
  EpiRows e{dwg, dwu, 0, s.d};
  return launch_gemm<BwNTCfg, false, false>(g, e, st);
}

int bw_dproj_splits(const Slab &s) {
  int sp = kDprojSplits;
  while (sp > 1 && (s.Lp / BwCfg::BK) % sp) sp /= 2;
  return sp;
}

hipError_t bw_dproj(const Slab &s, const BwBufs &b, float *dproj, hipStream_t st) {
  // d x d outputs are too few tiles to fill the GPU: K (tokens) is split into
  // sp slices whose partial sums are added in a fixed order afterwards
  const int sp = bw_dproj_splits(s);
  const int64_t kp = s.Lp / sp;
  GProb g{};
  g.M = s.d;
  g.N = s.d;
  g.nb1 = 1;
  g.nb2 = sp;
  g.nseg = s.n_seq;
  g.nph = 1;
  // dproj[c][i] = sum over tokens dV[t][c] C[t][i]: A = dVt rows c, B = C (K-major over i)
  g.ph[0].a = kcontig(b.dvt, s.Lp, s.d, 0, kp, (int64_t)s.d * s.Lp);
  g.ph[0].b = kmajor(b.c, s.d, s.d, 0, kp * s.d, s.Lp * s.d);
  g.ph[0].K = (int)kp;
  const int64_t dd = (int64_t)s.d * s.d;
  EpiRowsSplit e{b.dproj_part, dd, s.d};
  hipError_t err = launch_gemm<BwCfg, false, true>(g, e, st);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_sum_rows, dim3((unsigned)((dd + 255) / 256)), dim3(256), 0, st,
                     (const float *)b.dproj_part, (int64_t)sp, dd, dproj);
  return hipGetLastError();
}

int64_t bw_conv_runs(const Slab &s) { return (int64_t)s.n_seq * s.nc * (s.Bp / CONV_BW_RUN); }

hipError_t bw_conv(const Slab &s, const BwBufs &b, const __bf16 *e, const void *conv_w, float *de,
                   float *dconv, hipStream_t st) {
  const int64_t total = bw_conv_runs(s) * (s.d / 8);
  const unsigned grid = (unsigned)((total + 255) / 256);
  const __bf16 *cw = (const __bf16 *)conv_w;
  switch (s.Kc) {
#define BW_CONV_CASE(K) \
  case K: hipLaunchKernelGGL(k_conv_bwd<K>, dim3(grid), dim3(256), 0, st, s, b.dc, e, cw, de, b.part); break;
    BW_CONV_CASE(1) BW_CONV_CASE(2) BW_CONV_CASE(3) BW_CONV_CASE(4)
    BW_CONV_CASE(5) BW_CONV_CASE(6) BW_CONV_CASE(7) BW_CONV_CASE(8)
#undef BW_CONV_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // partial sums of the runs: in row groups, then the groups (fixed order)
  const int64_t len = (int64_t)s.d * s.Kc;
  const int64_t runs = bw_conv_runs(s);
  const int groups = (int)std::min<int64_t>(kConvSumGroups, runs);
  hipLaunchKernelGGL(k_sum_rows, dim3((unsigned)((len + 255) / 256), groups), dim3(256), 0, st,
                     (const float *)b.part, runs, len, b.part2);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_sum_rows, dim3((unsigned)((len + 255) / 256)), dim3(256), 0, st,
                     (const float *)b.part2, (int64_t)groups, len, dconv);
  return hipGetLastError();
}
static_assert(kChunkAlign % CONV_BW_RUN == 0, "conv runs must not cross a chunk");

hipError_t bw_sum_seq(const float *in, int n, int64_t len, float *out, hipStream_t st) {
  hipLaunchKernelGGL(k_sum_rows, dim3((unsigned)((len + 255) / 256)), dim3(256), 0, st, in,
                     (int64_t)n, len, out);
  return hipGetLastError();
}

hipError_t bw_fill(float *p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace ipttt
