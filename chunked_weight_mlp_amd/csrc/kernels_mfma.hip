// bf16 MFMA kernels of the fast-weight prefill for gfx950 (CDNA4).
//
// All the dense contractions share one block structure, templated on the
// wave grid, the K step, the MFMA shape and the wave tile (Cfg): WM x WN
// waves, each computing a 128 x WTN output tile from FM x FM MFMA tiles
// (v_mfma_f32_32x32x16_bf16 or v_mfma_f32_16x16x32_bf16), so a block covers
// (128 WM) x (WTN WN). K is staged through LDS BK at a time in two buffers
// (three in the update), the next steps' copies in flight while a step runs
// on MFMA. gate/up, proj and the update fill the buffers with direct
// global-to-LDS copies into unpadded rows whose 16-byte pieces are
// XOR-swizzled (kslot) and load each MFMA sub-step's fragments into registers
// behind the previous sub-step's MFMAs. The apply, the Gram and the MSE
// corrections stage through registers into padded rows (PAD / PADT
// elements): their K-major operands are read with transposing LDS reads, which
// the compiler makes wait for every direct copy in flight. A K-contiguous
// operand gives each lane 8 consecutive K values with one 16-byte LDS read; a
// K-major one is read with ds_read_b64_tr_b16. Shapes, paddings and staging
// were picked by timing on MI355X.
//
// Kernels:
//   k_gateup   Z = SiLU(X W_g) * (X W_u)   M = slab rows, N = d_ff (half the
//              block's B rows are gate rows, half up rows), K = d. Writes Zt
//              (rows of d_ff, token-contiguous), the only copy of Z.
//   k_proj     Vt = scale * (C Proj)^T     M = slab rows, N = d, K = d.
//   k_apply    O = Z_q S_q (+ P_q (eta V_q))  M = rows of a group of G
//              chunks, N = d, K = d_ff (then the group's earlier tokens),
//              batched over (sequence, group); A comes from Zt (then P^T)
//              through LDS transpose reads, B from the blocked copy S_q. The
//              MSE rule also writes Rt = eta (V - O)^T of the group's rows.
//   k_mse_fix  MSE rule, chunk jl of a group: O += P R over the group's
//              earlier chunks' final residuals, then Rt of the chunk.
//   k_gram     P^T = block-causal Z_q Z_q^T of each group (G > 1), both
//              operands read transposed; only the tiles the apply reads.
//   k_update   W^T tile (BM d_ff rows x BN d columns, fp32) held in the
//              accumulators across the chunks of a slab, one K loop over all
//              of them: per group of G chunks, optionally the bf16 snapshot
//              S_q (streamed out over the group's K steps, blocked layout),
//              then Zt . Vt over the group's tokens.
//   k_snapshot_blk  bf16 blocked copy of W (the MSE rule's first group).
//   k_conv     depthwise conv of E, vector loads, sliding window.

#include <algorithm>
#include <atomic>

#include "mfma_common.h"

namespace ipttt {
namespace mfma {

// ---------------------------------------------------------------------------
// Runs a GEMM kernel's tiles (logical ids 0 .. ntiles - 1) with both operands
// staged by direct copies: init(id) points the loaders at tile id,
// epilogue(id) writes it from the accumulators. PERS: persistent blocks (one
// per CU) walk their XCD's tiles as one stream of K steps
// (kloop_dma_pl_tiles). The hardware hands block b to XCD b % 8; that XCD's
// blocks share its contiguous range of logical tiles, block k of them taking
// tiles lo + k, lo + k + nbx, ..., so concurrent blocks hold neighbouring
// tiles. Otherwise one tile per block, numbered by xcd_remap.
template <class C, bool PERS, class Init, class Epi>
__device__ __forceinline__ void run_tiles(__bf16 *smem, DmaLoader<C, C::BM> &la,
                                          DmaLoader<C, C::BN> &lb, int ntiles, int nk, int wave,
                                          int lane, int arow0, const int (&brow)[C::NJ],
                                          typename C::acc_t (&acc)[C::MI][C::NJ], Init init,
                                          Epi epilogue) {
  const auto koff = [](int st, int64_t &ka, int64_t &kb) { ka = kb = (int64_t)st * C::BK; };
  if constexpr (PERS) {
    const int xc = blockIdx.x % 8, k = blockIdx.x / 8;
    const int nbx = gridDim.x / 8 + (xc < (int)(gridDim.x % 8));
    const int per = ntiles / 8, rem = ntiles % 8;
    const int lo = xc * per + min(xc, rem), hi = lo + per + (xc < rem);
    const int nt = hi - lo - k > 0 ? (hi - lo - k + nbx - 1) / nbx : 0;
    if (nt == 0) return;
    kloop_dma_pl_tiles<C, 2, true, C::MI + C::NJ>(
        smem, la, lb, nt, nk, wave, acc,
        [&](const __bf16 *As, const __bf16 *Bs, int u, Frags<C> &f) __attribute__((always_inline)) {
          load_frags<C>(As, Bs, u, arow0, brow, lane, f);
        },
        koff, [&](int t) __attribute__((always_inline)) { init(lo + k + t * nbx); },
        [&](int t) __attribute__((always_inline)) { epilogue(lo + k + t * nbx); });
  } else {
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    init(id);
    zero_acc<C>(acc);
    kloop_dma_pl<C, 2, true>(smem, la, lb, nk, wave, lane, arow0, brow, acc, koff, [](int) {},
                             [](int) {});
    epilogue(id);
  }
}

// ---------------------------------------------------------------------------
// PERS: persistent blocks (one per CU), each running a range of its XCD's
// tiles back to back through kloop_dma_pl_tiles; otherwise one tile per block.
// PRE: also write the pre-activations (at, ut) for the backward.
template <class C, bool PERS, bool PRE>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_gateup(
    Slab s, const __bf16 *__restrict__ x, const __bf16 *__restrict__ wg,
    const __bf16 *__restrict__ wu, __bf16 *__restrict__ zt, __bf16 *__restrict__ at,
    __bf16 *__restrict__ ut) {
  static_assert(C::SMEM_ELEMS * 2 <= 160 * 1024, "LDS overflow");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[C::SMEM_ELEMS];
  using M = typename C::M;
  constexpr int FT = C::BN / 2;  // d_ff columns per block
  const int P = s.nc * s.Bp;
  const int nm = (P + C::BM - 1) / C::BM, nn = (s.F + FT - 1) / FT;
  const int per_seq = nm * nn;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  // tile of logical index id: sequence, first slab row, first d_ff column
  const auto tile = [&](int id, int &n_seq, int &m0, int &f0) __attribute__((always_inline)) {
    n_seq = id / per_seq;
    int tm, tn;
    tile_of<C::GM>(id % per_seq, nm, nn, tm, tn);
    m0 = tm * C::BM;
    f0 = tn * FT;
  };

  // A rows: the slab rows' tokens of X; B rows [0, FT): gate rows f0..,
  // [FT, 2 FT): the matching up rows
  DmaLoader<C, C::BM> la;
  DmaLoader<C, C::BN> lb;
  const auto init = [&](int id) __attribute__((always_inline)) {
    int n_seq, m0, f0;
    tile(id, n_seq, m0, f0);
    const __bf16 *xs = x + n_seq * s.x_seq_stride;
    la.init(wave, lane, [&](int r) {
      const int p = m0 + r;
      const int64_t t = p < P ? slab_row_token(s, p) : -1;
      return xs + (t >= 0 ? t : 0) * s.d;
    });
    lb.init(wave, lane, [&](int rr) {
      const int f = f0 + (rr < FT ? rr : rr - FT);
      return (rr < FT ? wg : wu) + (int64_t)(f < s.F ? f : 0) * s.d;
    });
  };
  // a wave's first NJ/2 B tiles are gate rows, the other NJ/2 the matching up rows
  constexpr int HJ = C::NJ / 2;
  constexpr int WF = C::WTN / 2;  // d_ff columns per wave
  int brow[C::NJ];
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    brow[j] = wn * WF + C::FM * j;
    brow[j + HJ] = FT + wn * WF + C::FM * j;
  }
  typename C::acc_t acc[C::MI][C::NJ];

  const auto epilogue = [&](int id) __attribute__((always_inline)) {
    int n_seq, m0, f0;
    tile(id, n_seq, m0, f0);
    __bf16 *zts = zt + (int64_t)n_seq * s.F * s.Lp;
    // Row tiles i and i + 1 together: lane l holds rows (tokens) 4 (l / 16) ..
    // + 3 of each at its column f; swapping between lane groups l / 16 = 0 <-> 1
    // and 2 <-> 3 leaves every lane 8 consecutive tokens of its column, one
    // 16-byte store (Bp and P are multiples of 64, so an 8-row group is wholly
    // inside or outside the slab).
    static_assert(M::NG == 1 && C::MI % 2 == 0, "pairs of 16-row tiles");
    const int gq = lane >> 4;
    const auto swap8 = [](bf16x4 a, bf16x4 b) __attribute__((always_inline)) {
      const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
      const auto x = __builtin_amdgcn_permlane16_swap(ua.x, ub.x, false, false);
      const auto y = __builtin_amdgcn_permlane16_swap(ua.y, ub.y, false, false);
      return uint4{x[0], y[0], x[1], y[1]};
    };
    // tiles wholly inside the slab, the sequence and d_ff: no per-row masks and
    // no store predicates (a predicated store would also wait for the next
    // tile's copies in flight)
    const bool full = s.B == s.Bp && m0 + C::BM <= P && s.tok0 + m0 + C::BM <= s.L &&
                      f0 + FT <= s.F;
    const auto tile_out = [&](auto full_tag) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
      for (int i = 0; i < C::MI; i += 2) {
        // rows p .. p + 3 of each tile lie in one chunk (Bp is a multiple of 4);
        // chunk-padding rows and tokens past the sequence end are exact zeros
        bool real[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (FULL) {
#pragma unroll
            for (int r = 0; r < 4; ++r) real[h][r] = true;
            continue;
          }
          const int p = m0 + wm * C::WTM + C::FM * (i + h) + M::rrow(lane, 0);
          if (s.B == s.Bp) {  // no padding rows: slab row p is token tok0 + p
            const int64_t t0 = s.tok0 + p;
#pragma unroll
            for (int r = 0; r < 4; ++r) real[h][r] = p < P && t0 + r < s.L;
          } else {
            const int jc = p / s.Bp, ic = p - jc * s.Bp;
            const int64_t t0 = s.tok0 + (int64_t)jc * s.B + ic;
#pragma unroll
            for (int r = 0; r < 4; ++r) real[h][r] = jc < s.nc && ic + r < s.B && t0 + r < s.L;
          }
        }
        const int pl = m0 + wm * C::WTM + C::FM * i + 8 * (gq >> 1) + C::FM * (gq & 1);
#pragma unroll
        for (int j = 0; j < HJ; ++j) {
          const int f = f0 + wn * WF + C::FM * j + M::rcol(lane);
          bf16x4 v[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 gv = get4(acc[i + h][j], 0), uv = get4(acc[i + h][j + HJ], 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)  // SiLU(a) = a sigmoid(a)
              v[h][r] = (__bf16)(real[h][r] ? gv[r] * fast_sigmoid(gv[r]) * uv[r] : 0.f);
          }
          const uint4 z = swap8(v[0], v[1]);
          if (FULL || (pl < P && f < s.F)) *(uint4 *)(zts + (int64_t)f * s.Lp + pl) = z;
          if constexpr (PRE) {  // pre-activations, for the backward
            bf16x4 va[2], vu[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4 gv = get4(acc[i + h][j], 0), uv = get4(acc[i + h][j + HJ], 0);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                va[h][r] = (__bf16)(real[h][r] ? gv[r] : 0.f);
                vu[h][r] = (__bf16)(real[h][r] ? uv[r] : 0.f);
              }
            }
            const uint4 za = swap8(va[0], va[1]), zu = swap8(vu[0], vu[1]);
            const int64_t off = (int64_t)n_seq * s.F * s.Lp + (int64_t)f * s.Lp + pl;
            if (FULL || (pl < P && f < s.F)) {
              *(uint4 *)(at + off) = za;
              *(uint4 *)(ut + off) = zu;
            }
          }
        }
      }
    };
    if (full)
      tile_out(std::true_type());
    else
      tile_out(std::false_type());
  };

  run_tiles<C, PERS>(smem, la, lb, per_seq * s.n_seq, s.d / C::BK, wave, lane, wm * C::WTM, brow,
                     acc, init, epilogue);
}

// ---------------------------------------------------------------------------
template <class C, bool PERS>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_proj(
    Slab s, const __bf16 *__restrict__ c, const __bf16 *__restrict__ proj,
    __bf16 *__restrict__ vt, float scale) {
  static_assert(C::SMEM_ELEMS * 2 <= 160 * 1024, "LDS overflow");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[C::SMEM_ELEMS];
  using M = typename C::M;
  const int P = s.nc * s.Bp;
  const int nm = (P + C::BM - 1) / C::BM, nn = (s.d + C::BN - 1) / C::BN;
  const int per_seq = nm * nn;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const auto tile = [&](int id, int &n_seq, int &m0, int &n0) __attribute__((always_inline)) {
    n_seq = id / per_seq;
    int tm, tn;
    tile_of<C::GM>(id % per_seq, nm, nn, tm, tn);
    m0 = tm * C::BM;
    n0 = tn * C::BN;
  };
  DmaLoader<C, C::BM> la;
  DmaLoader<C, C::BN> lb;
  const auto init = [&](int id) __attribute__((always_inline)) {
    int n_seq, m0, n0;
    tile(id, n_seq, m0, n0);
    const __bf16 *cs = c + (int64_t)n_seq * s.Lp * s.d;
    la.init(wave, lane, [&](int r) { return cs + (int64_t)(m0 + r < P ? m0 + r : 0) * s.d; });
    lb.init(wave, lane, [&](int r) { return proj + (int64_t)(n0 + r < s.d ? n0 + r : 0) * s.d; });
  };
  int brow[C::NJ];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) brow[j] = wn * C::WTN + C::FM * j;
  typename C::acc_t acc[C::MI][C::NJ];
  const auto epilogue = [&](int id) __attribute__((always_inline)) {
    int n_seq, m0, n0;
    tile(id, n_seq, m0, n0);
    __bf16 *vts = vt + (int64_t)n_seq * s.d * s.Lp;
    // Row tiles i and i + 1 together, their halves swapped between lane groups
    // (as gate/up's Zt): each lane stores 8 consecutive tokens of its column n.
    static_assert(M::NG == 1 && C::MI % 2 == 0, "pairs of 16-row tiles");
    const int gq = lane >> 4;
    // tiles wholly inside the slab and d store without predicates (a
    // predicated store would also wait for the next tile's copies in flight)
    const bool full = m0 + C::BM <= P && n0 + C::BN <= s.d;
    const auto tile_out = [&](auto full_tag) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
      for (int i = 0; i < C::MI; i += 2) {
        const int pl = m0 + wm * C::WTM + C::FM * i + 8 * (gq >> 1) + C::FM * (gq & 1);
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          const int n = n0 + wn * C::WTN + C::FM * j + M::rcol(lane);
          bf16x4 v[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 a4 = get4(acc[i + h][j], 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[h][r] = (__bf16)(scale * a4[r]);
          }
          const uint2 ua = __builtin_bit_cast(uint2, v[0]), ub = __builtin_bit_cast(uint2, v[1]);
          const auto x = __builtin_amdgcn_permlane16_swap(ua.x, ub.x, false, false);
          const auto y = __builtin_amdgcn_permlane16_swap(ua.y, ub.y, false, false);
          const uint4 z{x[0], y[0], x[1], y[1]};
          if (FULL || (pl < P && n < s.d)) *(uint4 *)(vts + (int64_t)n * s.Lp + pl) = z;
        }
      }
    };
    if (full)
      tile_out(std::true_type());
    else
      tile_out(std::false_type());
  };
  run_tiles<C, PERS>(smem, la, lb, per_seq * s.n_seq, s.d / C::BK, wave, lane, wm * C::WTM, brow,
                     acc, init, epilogue);
}

// ---------------------------------------------------------------------------
// Layout of the forward's bf16 copies S of the fast weight (BLK): blocks of 8
// consecutive d_ff values, element (c, f) at ((f / 8) d + c) 8 + f % 8. The
// update writes S from the accumulators, where 16 consecutive lanes hold 8
// consecutive f each for 16 consecutive columns c: one 256-byte run here,
// against 16 separate 16-byte pieces (half cache lines) in the row-major
// [d][F] layout, whose partial-line writes completed slowly enough to hold
// up the update's later waits. The apply's snapshot loads stay whole lines
// (8 consecutive c of one block of f). Otherwise row-major.
template <bool BLK>
__device__ __forceinline__ int64_t snap_offset(const Slab &s, int c, int f) {
  if constexpr (BLK)
    return ((int64_t)(f >> 3) * s.d + c) * 8 + (f & 7);
  else
    return (int64_t)c * s.F + f;
}
// S = bf16(W) in the blocked layout, for every sequence of the slab (the MSE
// rule's first copy; the update writes the later ones). A block converts 16
// rows c x 256 columns f through LDS: rows read whole, blocks of f written as
// 256-byte runs of 16 consecutive c.
__global__ __launch_bounds__(256) void k_snapshot_blk(Slab s, const float *__restrict__ w,
                                                      __bf16 *__restrict__ snap,
                                                      int64_t snap_seq_stride) {
  constexpr int TC = 16, TF = 256;
  __shared__ __attribute__((aligned(16))) __bf16 tile[TC][TF + 8];
  const int c0 = blockIdx.x * TC, f0 = blockIdx.y * TF, n_seq = blockIdx.z;
  const int t = threadIdx.x;
  const float *ws = w + (int64_t)n_seq * s.d * s.F;
  {  // thread t: rows c0 + t / 64 + 4 i, 4 columns from f0 + 4 (t % 64): each wave
     // reads 1 KB of one row per load, all four loads in flight together
    const int f = f0 + 4 * (t % 64);
    f32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + t / 64 + 4 * i;
      v[i] = (c < s.d && f < s.F) ? *(const f32x4 *)(ws + (int64_t)c * s.F + f)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 b;
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = (__bf16)v[i][r];
      *(bf16x4 *)&tile[t / 64 + 4 * i][4 * (t % 64)] = b;
    }
  }
  __syncthreads();
  __bf16 *ss = snap + n_seq * snap_seq_stride;
#pragma unroll
  for (int k = 0; k < TC * TF / 8 / 256; ++k) {  // piece p: column c0 + p % 16, block p / 16
    const int p = t + 256 * k;
    const int c = c0 + p % TC, f = f0 + 8 * (p / TC);
    if (c < s.d && f < s.F)
      *(bf16x8 *)(ss + snap_offset<true>(s, c, f)) = *(const bf16x8 *)&tile[p % TC][8 * (p / TC)];
  }
}

// ---------------------------------------------------------------------------
// O rows of chunk groups [q0, q0 + nq) of every sequence (G = 1: one chunk per
// group): O = Z S_q over the group's rows (S_q stored output-major, d rows of
// d_ff), plus, when pt is given, the updates of the group's earlier chunks as
// P (eta V), P^T read from the Gram buffer. The MSE rule (pt null) also writes
// Rt = eta (V - O)^T.
// BLK: the snapshots are in the blocked layout of snap_offset (the forward's),
// else row-major [d][F] (the backward's).
template <class C, bool IL, bool BLK>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_apply(
    Slab s, int q0, int nq, const __bf16 *__restrict__ zt, const __bf16 *__restrict__ snap,
    int64_t snap_seq_stride, int64_t snap_group_stride, const __bf16 *__restrict__ pt,
    int64_t pt_seq_stride, float *__restrict__ o, const __bf16 *__restrict__ vt,
    __bf16 *__restrict__ rt, int64_t rt_seq_stride, int64_t rt_ld) {
  static_assert(C::SMEM_T_ELEMS * 2 <= 160 * 1024, "LDS overflow");
  static_assert(kChunkAlign % C::BK == 0, "chunk starts must be whole K steps");
  __shared__ __bf16 smem[C::SMEM_T_ELEMS];
  using M = typename C::M;
  using LA = LoaderT<C, C::BM>;
  const int RG = s.G * s.Bp;  // rows of a full group
  const int nm = (RG + C::BM - 1) / C::BM, nn = (s.d + C::BN - 1) / C::BN;
  const int per_group = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bz = id / per_group;
  const int n_seq = bz / nq, ql = bz % nq, q = q0 + ql;
  int tm, tn;
  tile_of<C::GM>(id % per_group, nm, nn, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int j_first = q * s.G;                    // the group's first chunk in the slab
  const int R = min(s.G, s.nc - j_first) * s.Bp;  // its rows (the slab's last group may be short)
  if (m0 >= R) return;
  const int64_t row0 = (int64_t)j_first * s.Bp;  // its first slab row
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r0 = tid / C::KP;
  int brow[C::NJ];
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj) brow[jj] = wn * C::WTN + C::FM * jj;
  typename C::acc_t acc[C::MI][C::NJ];
  zero_acc<C>(acc);
  const __bf16 *zts = zt + (int64_t)n_seq * s.F * s.Lp;
  const __bf16 *ss = snap + n_seq * snap_seq_stride + ql * snap_group_stride;
  const __bf16 *vts = vt + (int64_t)n_seq * s.d * s.Lp;
  // rows of the tile see the group's tokens before their own chunk (G > 1);
  // the tile's last chunk starts at cs_last, so the second K phase runs over
  // group rows [0, cs_last), where P is zero until a row's chunk is complete.
  const int cs_last = (min(m0 + C::BM, R) - 1) / s.Bp * s.Bp;
  const __bf16 *pts = pt ? pt + n_seq * pt_seq_stride + (int64_t)q * RG * RG : nullptr;
  // A = Z read from Zt (token-contiguous rows of d_ff): K row f, M columns =
  // the group's slab rows. Columns past the workspace rows are clamped in
  // bounds; the rows they feed are past the group and are dropped.
  LA la;
  la.ld = s.Lp;
#pragma unroll
  for (int i = 0; i < LA::NP; ++i)
    la.ptr[i] = zts + (int64_t)LA::krow(tid, i) * s.Lp + min(row0 + m0 + LA::col(tid, i), s.Lp - 8);
  {
    using LS = typename std::conditional<BLK, BlockLoader<C, C::B_PIECES>,
                                         Loader<C, C::B_PIECES>>::type;
    LS lb;
    int lr0 = r0;
    if constexpr (BLK) {
      lb.assign(tid);
      lr0 = lb.r0;
      lb.blk = (int64_t)8 * s.d;
    }
#pragma unroll
    for (int i = 0; i < C::B_PIECES; ++i) {
      const int n = n0 + lr0 + C::RPP * i;
      if constexpr (BLK)
        lb.ptr[i] = ss + (int64_t)(n < s.d ? n : 0) * 8;
      else
        lb.ptr[i] = ss + (int64_t)(n < s.d ? n : 0) * s.F;
    }
    if constexpr (IL)
      kloop_g_il<C, true, false>(smem, la, lb, s.F / C::BK, tid, wm * C::WTM, brow, acc);
    else
      kloop_t<C>(smem, la, lb, s.F / C::BK, tid, wm * C::WTM, brow, acc);
  }

  if (pts && cs_last > 0) {
    Loader<C, C::B_PIECES> lb;
    la.ld = RG;
#pragma unroll
    for (int i = 0; i < LA::NP; ++i)
      la.ptr[i] = pts + (int64_t)LA::krow(tid, i) * RG + min(m0 + LA::col(tid, i), RG - 8);
#pragma unroll
    for (int i = 0; i < C::B_PIECES; ++i) {
      const int n = n0 + r0 + C::RPP * i;
      lb.ptr[i] = vts + (int64_t)(n < s.d ? n : 0) * s.Lp + row0;
    }
    if constexpr (IL)
      kloop_g_il<C, true, false>(smem, la, lb, cs_last / C::BK, tid, wm * C::WTM, brow, acc);
    else
      kloop_t<C>(smem, la, lb, cs_last / C::BK, tid, wm * C::WTM, brow, acc);
  }

  float *os = o ? o + n_seq * s.x_seq_stride : nullptr;  // nullptr: residual only
  // the residual's V for the whole tile before any store (clamped in bounds,
  // loaded unconditionally), so one wait covers every load
  bf16x4 vb[C::MI][M::NG][C::NJ];
  if (rt) {
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int g = 0; g < M::NG; ++g) {
        const int m = min(m0 + wm * C::WTM + C::FM * i + M::rrow(lane, g), R - 4);
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj) {
          const int n = min(n0 + wn * C::WTN + C::FM * jj + M::rcol(lane), s.d - 1);
          vb[i][g][jj] = *(const bf16x4 *)(vts + (int64_t)n * s.Lp + row0 + m);
        }
      }
  }
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int g = 0; g < M::NG; ++g) {
      // rows m .. m + 3 share one chunk (Bp is a multiple of 4)
      const int m = m0 + wm * C::WTM + C::FM * i + M::rrow(lane, g);
      const int jc = m / s.Bp, ic = m - jc * s.Bp;
      const int64_t t0 = s.tok0 + (int64_t)(j_first + jc) * s.B + ic;
      bool valid[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) valid[r] = ic + r < s.B && t0 + r < s.L;
      if (m >= R) continue;
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj) {
        const int n = n0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
        if (n >= s.d) continue;
        const f32x4 a4 = get4(acc[i][jj], g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (os && valid[r]) os[(t0 + r) * s.d + n] = a4[r];
        if (rt) {
          const bf16x4 v = vb[i][g][jj];
          bf16x4 rv;
#pragma unroll
          for (int r = 0; r < 4; ++r) rv[r] = (__bf16)(valid[r] ? s.eta * ((float)v[r] - a4[r]) : 0.f);
          *(bf16x4 *)(rt + n_seq * rt_seq_stride + n * rt_ld + m) = rv;
        }
      }
    }
}

// ---------------------------------------------------------------------------
// MSE rule over chunk groups (G > 1), chunk jl >= 1 of group q of every
// sequence. The apply wrote the group's rows O = Z S_q (S_q: W at the group's
// first chunk) and Rt = eta (V - O)^T from them, which is final for chunk 0.
// Chunk jl adds what the group's earlier chunks changed in W: with R_i their
// final residuals, W_jl = W_q + sum over i < jl of Z_i^T R_i, so
//   O_jl = Z_jl S_q + sum over group rows s of earlier chunks of (z_m . z_s) R_s,
// the Gram term read from P^T (block-causal, as the linear rule's). Then
// Rt = eta (V - O)^T for the chunk's rows, which chunks after it read.
// A = P^T (rows s, K-major), B = Rt rows c (token-contiguous, pitch G Bp).
template <class C, bool IL>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_mse_fix(
    Slab s, int q, int jl, const __bf16 *__restrict__ pt, int64_t pt_seq_stride,
    const __bf16 *__restrict__ vt, __bf16 *__restrict__ rt, int64_t rt_seq_stride,
    float *__restrict__ o) {
  static_assert(C::SMEM_T_ELEMS * 2 <= 160 * 1024, "LDS overflow");
  static_assert(kChunkAlign % C::BK == 0, "chunk starts must be whole K steps");
  __shared__ __bf16 smem[C::SMEM_T_ELEMS];
  using M = typename C::M;
  using LA = LoaderT<C, C::BM>;
  const int RG = s.G * s.Bp;  // rows of a full group
  const int nm = (s.Bp + C::BM - 1) / C::BM, nn = (s.d + C::BN - 1) / C::BN;
  const int per_seq = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int n_seq = id / per_seq;
  int tm, tn;
  tile_of<C::GM>(id % per_seq, nm, nn, tm, tn);
  const int cs = jl * s.Bp;           // the chunk's first group row = rows of earlier chunks
  const int m0 = cs + tm * C::BM, n0 = tn * C::BN;
  const int mend = cs + s.Bp;         // rows past the chunk belong to the next one
  const int j_first = q * s.G;
  const int64_t row0 = (int64_t)j_first * s.Bp;  // the group's first slab row
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int r0 = tid / C::KP;
  int brow[C::NJ];
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj) brow[jj] = wn * C::WTN + C::FM * jj;
  typename C::acc_t acc[C::MI][C::NJ];
  zero_acc<C>(acc);
  const __bf16 *pts = pt + n_seq * pt_seq_stride + (int64_t)q * RG * RG;
  __bf16 *rts = rt + n_seq * rt_seq_stride;
  const __bf16 *vts = vt + (int64_t)n_seq * s.d * s.Lp;
  {
    LA la;
    la.ld = RG;
#pragma unroll
    for (int i = 0; i < LA::NP; ++i)
      la.ptr[i] = pts + (int64_t)LA::krow(tid, i) * RG + min(m0 + LA::col(tid, i), RG - 8);
    Loader<C, C::B_PIECES> lb;
#pragma unroll
    for (int i = 0; i < C::B_PIECES; ++i) {
      const int n = n0 + r0 + C::RPP * i;
      lb.ptr[i] = rts + (int64_t)(n < s.d ? n : 0) * RG;
    }
    if constexpr (IL)
      kloop_g_il<C, true, false>(smem, la, lb, cs / C::BK, tid, wm * C::WTM, brow, acc);
    else
      kloop_t<C>(smem, la, lb, cs / C::BK, tid, wm * C::WTM, brow, acc);
  }

  float *os = o + n_seq * s.x_seq_stride;
  if constexpr (C::WM * C::WN < 8) {  // one wave per SIMD: registers for the whole tile
    // every load of the tile (O and V, clamped in bounds, unconditional) before
    // any store, so one wait covers them all; rows and columns out of range are
    // never stored
    static_assert(M::NG == 1, "one 4-row group per accumulator tile");
    f32x4 ob[C::MI][C::NJ];
    bf16x4 vb[C::MI][C::NJ];
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int m = min(m0 + wm * C::WTM + C::FM * i + M::rrow(lane, 0), mend - 4);
      const int64_t t0 = s.tok0 + (int64_t)(j_first + jl) * s.B + (m - cs);
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj) {
        const int n = min(n0 + wn * C::WTN + C::FM * jj + M::rcol(lane), s.d - 1);
        vb[i][jj] = *(const bf16x4 *)(vts + (int64_t)n * s.Lp + row0 + m);
#pragma unroll
        for (int r = 0; r < 4; ++r) ob[i][jj][r] = os[min(t0 + r, s.L - 1) * s.d + n];
      }
    }
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      // rows m .. m + 3 share one chunk (Bp is a multiple of 4)
      const int m = m0 + wm * C::WTM + C::FM * i + M::rrow(lane, 0);
      if (m >= mend) continue;
      const int ic = m - cs;
      const int64_t t0 = s.tok0 + (int64_t)(j_first + jl) * s.B + ic;
      bool valid[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) valid[r] = ic + r < s.B && t0 + r < s.L;
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj) {
        const int n = n0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
        if (n >= s.d) continue;
        const f32x4 a4 = get4(acc[i][jj], 0);
        bf16x4 rv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ov = ob[i][jj][r] + a4[r];
          if (valid[r]) os[(t0 + r) * s.d + n] = ov;
          rv[r] = (__bf16)(valid[r] ? s.eta * ((float)vb[i][jj][r] - ov) : 0.f);
        }
        *(bf16x4 *)(rts + (int64_t)n * RG + m) = rv;
      }
    }
  } else {  // two waves per SIMD: a row tile at a time
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int g = 0; g < M::NG; ++g) {
        // rows m .. m + 3 share one chunk (Bp is a multiple of 4)
        const int m = m0 + wm * C::WTM + C::FM * i + M::rrow(lane, g);
        if (m >= mend) continue;
        const int ic = m - cs;
        const int64_t t0 = s.tok0 + (int64_t)(j_first + jl) * s.B + ic;
        bool valid[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) valid[r] = ic + r < s.B && t0 + r < s.L;
        // every load of the row tile before its stores, so one wait covers them
        f32x4 ob[C::NJ];
        bf16x4 vb[C::NJ];
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj) {
          // clamped in bounds and loaded unconditionally; rows and columns out of
          // range are never stored
          const int n = min(n0 + wn * C::WTN + C::FM * jj + M::rcol(lane), s.d - 1);
          vb[jj] = *(const bf16x4 *)(vts + (int64_t)n * s.Lp + row0 + m);
#pragma unroll
          for (int r = 0; r < 4; ++r) ob[jj][r] = os[min(t0 + r, s.L - 1) * s.d + n];
        }
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj) {
          const int n = n0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
          if (n >= s.d) continue;
          const f32x4 a4 = get4(acc[i][jj], g);
          bf16x4 rv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ov = ob[jj][r] + a4[r];
            if (valid[r]) os[(t0 + r) * s.d + n] = ov;
            rv[r] = (__bf16)(valid[r] ? s.eta * ((float)vb[jj][r] - ov) : 0.f);
          }
          *(bf16x4 *)(rts + (int64_t)n * RG + m) = rv;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Block-causal Gram of chunk groups [0, ng) of the slab: P^T[s][m] = z_m . z_s
// (a sum over d_ff) when group row s lies in an earlier chunk than group row
// m, else 0. A = Zt columns m, B = Zt columns s, both K-major (rows of d_ff)
// in memory and read through transposing LDS reads. Only the tiles the apply
// reads are computed: s below the first row of the m tile's last chunk.
template <class C>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_gram(
    Slab s, int ng, const __bf16 *__restrict__ zt, __bf16 *__restrict__ pt,
    int64_t pt_seq_stride) {
  static_assert(C::SMEM_TT_ELEMS * 2 <= 160 * 1024, "LDS overflow");
  __shared__ __bf16 smem[C::SMEM_TT_ELEMS];
  using M = typename C::M;
  using LA = LoaderT<C, C::BM>;
  using LB = LoaderT<C, C::BN>;
  const int RG = s.G * s.Bp;
  const int nm = (RG + C::BM - 1) / C::BM, nn = (RG + C::BN - 1) / C::BN;
  const int per_group = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bz = id / per_group;
  const int n_seq = bz / ng, q = bz % ng;
  const int tm = (id % per_group) / nn, tn = (id % per_group) % nn;
  const int m0 = tm * C::BM, s0 = tn * C::BN;
  const int j_first = q * s.G;
  const int R = min(s.G, s.nc - j_first) * s.Bp;
  if (m0 >= R) return;
  const int cs_last = (min(m0 + C::BM, R) - 1) / s.Bp * s.Bp;
  if (s0 >= cs_last) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t row0 = (int64_t)j_first * s.Bp;
  const __bf16 *zts = zt + (int64_t)n_seq * s.F * s.Lp;
  LA la;
  LB lb;
  la.ld = lb.ld = s.Lp;
#pragma unroll
  for (int i = 0; i < LA::NP; ++i)
    la.ptr[i] = zts + (int64_t)LA::krow(tid, i) * s.Lp + min(row0 + m0 + LA::col(tid, i), s.Lp - 8);
#pragma unroll
  for (int i = 0; i < LB::NP; ++i)
    lb.ptr[i] = zts + (int64_t)LB::krow(tid, i) * s.Lp + min(row0 + s0 + LB::col(tid, i), s.Lp - 8);
  int brow[C::NJ];
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj) brow[jj] = wn * C::WTN + C::FM * jj;
  typename C::acc_t acc[C::MI][C::NJ];
  zero_acc<C>(acc);
  if constexpr (C::WM * C::WN >= 8)  // two waves per SIMD: interleaved loop
    kloop_g_il<C, true, true>(smem, la, lb, s.F / C::BK, tid, wm * C::WTM, brow, acc);
  else
    kloop_tt<C>(smem, la, lb, s.F / C::BK, tid, wm * C::WTM, brow, acc);

  __bf16 *pts = pt + n_seq * pt_seq_stride + (int64_t)q * RG * RG;
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
      for (int g = 0; g < M::NG; ++g) {
        const int m = m0 + wm * C::WTM + C::FM * i + M::rrow(lane, g);
        const int sc = s0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
        if (m < RG && sc < RG) {
          const f32x4 a4 = get4(acc[i][jj], g);
          const bool earlier = sc / s.Bp < m / s.Bp;  // rows m .. m + 3 share a chunk
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)(earlier ? a4[r] : 0.f);
          *(bf16x4 *)(pts + (int64_t)sc * RG + m) = v;
        }
      }
}

// ---------------------------------------------------------------------------
// W^T tile update: rows f (d_ff), columns c (d), K = tokens. The fp32 tile
// lives in the accumulators for chunks [j_first, j_first + n_chunks), taken G
// at a time (one K loop per group of G chunks, whose rows are contiguous).
// A operand = Zt (rows f, token-contiguous); B operand = Vt or Rt (rows c).
// snap_each_group: write S[g] = bf16(W) before group g's accumulation;
// snap_after: write S = bf16(W) after the last chunk. reverse (G = 1): walk
// the chunks last to first, snapshot S[j] before chunk j (the backward's
// G_{j+1}). BLK: snapshots in the blocked layout snap_offset describes (the
// forward's, read by the apply), else row-major [d][F] (the backward's).
// FULL: every tile lies inside the matrix (d_ff and d whole multiples of the
// tile), so no store tests its bounds: a predicated store inside the K loop
// also waits for every copy in flight.
template <class C, bool BLK, bool FULL>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_update(
    Slab s, int j_first, int n_chunks, int G, const __bf16 *__restrict__ zt,
    const __bf16 *__restrict__ bsrc, int64_t b_ld, int64_t b_seq_stride, int64_t b_chunk_stride,
    float *__restrict__ w, __bf16 *__restrict__ snap, int64_t snap_seq_stride,
    int64_t snap_group_stride, int snap_each_group, int snap_after, int reverse) {
  // three copy stages of the 128 x 256 tile (144 KB, one block per CU): each
  // stage's copies are issued two K steps ahead of its fragment reads
  constexpr int NSU = 3;
  static_assert(C::SMEM_ELEMS / 2 * NSU * 2 <= 160 * 1024, "LDS overflow");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[C::SMEM_ELEMS / 2 * NSU];
  using M = typename C::M;
  const int nm = (s.F + C::BM - 1) / C::BM, nn = (s.d + C::BN - 1) / C::BN;
  const int per_seq = nm * nn;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int n_seq = id / per_seq;
  int tm, tn;
  tile_of<C::GM>(id % per_seq, nm, nn, tm, tn);
  const int f0 = tm * C::BM, c0 = tn * C::BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t dF = (int64_t)s.d * s.F;
  float *ws = w + n_seq * dF;

  // accumulators <- W tile: each group of 4 accumulator rows is W^T[c][f .. f+3]
  typename C::acc_t acc[C::MI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
      for (int g = 0; g < M::NG; ++g) {
        const int f = f0 + wm * C::WTM + C::FM * i + M::rrow(lane, g);
        const int c = c0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
        set4(acc[i][jj], g,
             (f < s.F && c < s.d) ? *(const f32x4 *)(ws + (int64_t)c * s.F + f)
                                  : f32x4{0.f, 0.f, 0.f, 0.f});
      }
  auto write_snap = [&](__bf16 *dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
        for (int g = 0; g < M::NG; ++g) {
          const int f = f0 + wm * C::WTM + C::FM * i + M::rrow(lane, g);
          const int c = c0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
          if (FULL || (f < s.F && c < s.d)) {
            const f32x4 a4 = get4(acc[i][jj], g);
            bf16x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (__bf16)a4[r];
            *(bf16x4 *)(dst + snap_offset<BLK>(s, c, f)) = v;
          }
        }
  };

  // A rows: Zt rows f (token-contiguous); B rows: bsrc rows c. One K loop over
  // every step of the chunks; step st is K step r of chunk jc (walked last to
  // first when reverse).
  const __bf16 *zts = zt + (int64_t)n_seq * s.F * s.Lp;
  const __bf16 *bs = bsrc + n_seq * b_seq_stride;
  DmaLoader<C, C::BM> la;
  DmaLoader<C, C::BN> lb;
  la.init(wave, lane, [&](int r) { return zts + (int64_t)(f0 + r < s.F ? f0 + r : 0) * s.Lp; });
  lb.init(wave, lane, [&](int r) { return bs + (int64_t)(c0 + r < s.d ? c0 + r : 0) * b_ld; });
  int brow[C::NJ];
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj) brow[jj] = wn * C::WTN + C::FM * jj;
  const int spc = s.Bp / C::BK;  // K steps per chunk
  const int spg = G * spc;       // K steps per group
  // koff is called for steps 0, 1, 2, ... in order: walk (chunk, step) counters
  int kq = 0, kr = 0;
  auto koff = [&](int, int64_t &ka, int64_t &kb) __attribute__((always_inline)) {
    const int jc = reverse ? n_chunks - 1 - kq : kq;
    ka = (int64_t)(j_first + jc) * s.Bp + kr * C::BK;
    kb = (int64_t)jc * b_chunk_stride + kr * C::BK;
    if (++kr == spc) {
      kr = 0;
      ++kq;
    }
  };
  // Per-group snapshots: at the group's first K step the tile is rounded to
  // bf16 into registers (NSP pieces of 4 values per lane); the pieces then go
  // out in NSLOT slots at evenly spaced steps of the group (after the step's
  // barrier), so the copies stream out behind the MFMAs instead of stalling
  // every block at the same step. A slot holds the PPS row tiles i of one
  // column tile jj: whole 128-byte lines of the d_ff-contiguous snapshot rows.
  // Slots a short last group has not reached are stored after the loop;
  // groups of fewer than NSLOT steps store the whole tile at their first step.
  // Four slots (a whole column tile each) timed best; 8 and 16 smaller slots
  // were up to 2% and 5% slower.
  constexpr int NSP = C::MI * C::NJ * M::NG, NSLOT = 4, PPS = NSP / NSLOT;
  static_assert(M::NG == 1 && C::MI % PPS == 0 && C::NJ * (C::MI / PPS) == NSLOT,
                "snapshot slots must be whole column tiles of PPS row tiles");
  uint2 sbuf[NSP];
  __bf16 *sdst = snap + n_seq * snap_seq_stride;  // the pending snapshot
  const int cl = c0 + wn * C::WTN + M::rcol(lane);
  auto slot_piece = [](int k, int e) { return ((k / C::NJ) * PPS + e) * C::NJ + k % C::NJ; };
  // Pieces q0, q1 of row tiles i and i + 1 of one column tile: lane l holds 4
  // values (d_ff 4 (l / 16) ..) of each; swapping between lane groups
  // l / 16 = 0 <-> 1 and 2 <-> 3 leaves every lane 8 consecutive values of its
  // row, one 16-byte store (64 contiguous bytes per row per instruction).
  auto store_pair = [&](int q0, int q1) __attribute__((always_inline)) {
    const int i = q0 / (C::NJ * M::NG), jj = q0 / M::NG % C::NJ;
    const auto x = __builtin_amdgcn_permlane16_swap(sbuf[q0].x, sbuf[q1].x, false, false);
    const auto y = __builtin_amdgcn_permlane16_swap(sbuf[q0].y, sbuf[q1].y, false, false);
    const uint4 v{x[0], y[0], x[1], y[1]};
    const int gq = lane >> 4;
    const int f = f0 + wm * C::WTM + C::FM * i + 8 * (gq >> 1) + C::FM * (gq & 1);
    const int c = cl + C::FM * jj;
    if (FULL || (f < s.F && c < s.d)) *(uint4 *)(sdst + snap_offset<BLK>(s, c, f)) = v;
  };
  static_assert(PPS % 2 == 0 && C::FM == 16, "slots store pairs of 16-row tiles");
  auto store_slot = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NSLOT; ++k)
      if (slot == k)
#pragma unroll
        for (int e = 0; e < PPS; e += 2) store_pair(slot_piece(k, e), slot_piece(k, e + 1));
  };
  int gr = 0, gq = 0;            // K step within the group, group (walk order)
  int nslot = NSLOT, nstep = 0;  // next slot to store and the group step it is due at
  auto pre = [&](int) __attribute__((always_inline)) {
    if (!snap_each_group || gr != 0) return;
    const int g = reverse ? n_chunks - 1 - gq : gq;  // reverse walks single chunks (G = 1)
    sdst = snap + n_seq * snap_seq_stride + (int64_t)g * snap_group_stride;
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
        for (int g2 = 0; g2 < M::NG; ++g2) {
          const f32x4 a4 = get4(acc[i][jj], g2);
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)a4[e];
          sbuf[(i * C::NJ + jj) * M::NG + g2] = __builtin_bit_cast(uint2, v);
        }
    if (spg >= NSLOT) {
      nslot = 0;
      nstep = 0;
    } else {
#pragma unroll
      for (int k = 0; k < NSLOT; ++k) store_slot(k);
    }
  };
  auto post = [&](int) __attribute__((always_inline)) {
    if (!snap_each_group) return;
    if (nslot < NSLOT && gr == nstep) {
      store_slot(nslot);
      ++nslot;
      nstep = nslot * spg / NSLOT;
    }
    if (++gr == spg) {
      gr = 0;
      ++gq;
    }
  };
  const int nk = n_chunks * spc;
  kloop_dma_pl<C, NSU, true>(smem, la, lb, nk, wave, lane, wm * C::WTM, brow, acc, koff, pre, post);
#pragma unroll
  for (int k = 0; k < NSLOT; ++k)
    if (k >= nslot) store_slot(k);
  // after the last chunk: the next slot when the groups have their own copies
  if (snap_after)
    write_snap(snap + n_seq * snap_seq_stride +
               (snap_each_group ? (int64_t)((n_chunks + G - 1) / G) * snap_group_stride : 0));
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int jj = 0; jj < C::NJ; ++jj)
#pragma unroll
      for (int g = 0; g < M::NG; ++g) {
        const int f = f0 + wm * C::WTM + C::FM * i + M::rrow(lane, g);
        const int c = c0 + wn * C::WTN + C::FM * jj + M::rcol(lane);
        if (FULL || (f < s.F && c < s.d)) *(f32x4 *)(ws + (int64_t)c * s.F + f) = get4(acc[i][jj], g);
      }
}

// ---------------------------------------------------------------------------
// Depthwise conv of the token embeddings, bf16 path: C[p][c] = sum_j w[c][j]
// E[t + j][c] with E taken as 0 past the chunk's end (pad rows: 0). A thread
// owns 8 channels (one 16-byte vector) over RUN consecutive rows of one chunk
// and keeps the KC-row window in registers, so each E row is read about once.
// Arithmetic in fp32, result rounded to bf16.
constexpr int CONV_RUN = 16;

template <int KC>
__global__ __launch_bounds__(256) void k_conv(Slab s, const __bf16 *__restrict__ e,
                                              const __bf16 *__restrict__ cw,
                                              __bf16 *__restrict__ c) {
  const int groups = s.d / 8;
  const int64_t runs_per_seq = (int64_t)s.nc * (s.Bp / CONV_RUN);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = runs_per_seq * groups * s.n_seq;
  if (gid >= total) return;
  const int g = (int)(gid % groups);
  const int64_t run = (gid / groups) % runs_per_seq;
  const int n_seq = (int)(gid / groups / runs_per_seq);
  const int64_t p0 = run * CONV_RUN;
  const int64_t j = p0 / s.Bp, i0 = p0 % s.Bp;
  const int64_t cs = s.tok0 + j * s.B;               // chunk's first token
  const int64_t ce = min(cs + (int64_t)s.B, s.L);    // one past its last token
  const int ch = 8 * g;
  float w[KC][8];
#pragma unroll
  for (int q = 0; q < KC; ++q)
#pragma unroll
    for (int k = 0; k < 8; ++k) w[q][k] = (float)cw[(ch + k) * KC + q];
  const __bf16 *es = e + n_seq * s.x_seq_stride + ch;
  bf16x8 win[CONV_RUN + KC - 1];
#pragma unroll
  for (int r = 0; r < CONV_RUN + KC - 1; ++r) {
    const int64_t t = cs + i0 + r;
    const bool in = (i0 + r < s.B) && t < ce;
    win[r] = in ? *(const bf16x8 *)(es + t * s.d) : bf16x8{};
  }
  __bf16 *cp = c + (int64_t)n_seq * s.Lp * s.d + p0 * s.d + ch;
#pragma unroll
  for (int i = 0; i < CONV_RUN; ++i) {
    const bool real = (i0 + i < s.B) && (cs + i0 + i < ce);
    bf16x8 out;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = 0.f;
#pragma unroll
      for (int q = 0; q < KC; ++q) a = fmaf(w[q][k], (float)win[i + q][k], a);
      out[k] = (__bf16)(real ? a : 0.f);
    }
    *(bf16x8 *)(cp + (int64_t)i * s.d) = out;
  }
}

// ---- launchers (templated on the block configuration) ---------------------
// Compute units of the current device, cached per device (relaxed atomics:
// handles may launch from several threads; every writer stores the same value).
inline int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n < 1) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// persistent kernels run one block per CU (their stages fill most of a CU's LDS)
template <class C, bool PERS>
hipError_t launch_gateup(const Slab &s, const __bf16 *x, const Weights &w, const WsPtrs &ws,
                         hipStream_t st, __bf16 *at = nullptr, __bf16 *ut = nullptr) {
  const int64_t P = (int64_t)s.nc * s.Bp;
  const int64_t ntiles =
      ((P + C::BM - 1) / C::BM) * ((s.F + C::BN / 2 - 1) / (C::BN / 2)) * s.n_seq;
  const int64_t nb = PERS ? std::min<int64_t>(ntiles, device_cus()) : ntiles;
  if (at)
    hipLaunchKernelGGL((k_gateup<C, PERS, true>), dim3((unsigned)nb), dim3(C::NTHR), 0, st, s, x,
                       (const __bf16 *)w.w_gate, (const __bf16 *)w.w_up, (__bf16 *)ws.zt, at, ut);
  else
    hipLaunchKernelGGL((k_gateup<C, PERS, false>), dim3((unsigned)nb), dim3(C::NTHR), 0, st, s, x,
                       (const __bf16 *)w.w_gate, (const __bf16 *)w.w_up, (__bf16 *)ws.zt, at, ut);
  return hipGetLastError();
}

template <class C, bool PERS>
hipError_t launch_proj(const Slab &s, const Weights &w, const WsPtrs &ws, hipStream_t st) {
  const int64_t P = (int64_t)s.nc * s.Bp;
  const int64_t ntiles = ((P + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  const int64_t nb = PERS ? std::min<int64_t>(ntiles, device_cus()) : ntiles;
  hipLaunchKernelGGL((k_proj<C, PERS>), dim3((unsigned)nb), dim3(C::NTHR), 0, st, s,
                     (const __bf16 *)ws.c, (const __bf16 *)w.proj, (__bf16 *)ws.vt,
                     s.mse ? 1.f : s.eta);
  return hipGetLastError();
}

// Groups of the slab: ceil(nc / G).
inline int slab_groups(const Slab &s) { return (s.nc + s.G - 1) / s.G; }

// Apply with every operand explicit: snapshot q0 + i at snap + n * snap_seq +
// i * snap_group; residual (MSE) to rt + n * rt_seq + c * rt_ld + row.
// IL: the interleaved loop for blocks of two waves per SIMD (eight-wave blocks)
template <class C, bool BLK, bool IL = (C::WM * C::WN >= 8)>
hipError_t launch_apply_x(const Slab &s, int q0, int nq, const __bf16 *zt, const __bf16 *snap,
                          int64_t snap_seq, int64_t snap_group, const __bf16 *pt, float *o,
                          const __bf16 *vt, __bf16 *rt, int64_t rt_seq, int64_t rt_ld,
                          hipStream_t st) {
  const int64_t RG = (int64_t)s.G * s.Bp;
  const int64_t nb = ((RG + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * nq * s.n_seq;
  hipLaunchKernelGGL((k_apply<C, IL, BLK>), dim3((unsigned)nb), dim3(C::NTHR), 0, st, s, q0, nq, zt, snap,
                     snap_seq, snap_group, pt, (int64_t)s.ng_cap * RG * RG, o, vt, rt, rt_seq,
                     rt_ld);
  return hipGetLastError();
}

template <class C>
hipError_t launch_apply(const Slab &s, int q0, int nq, const WsPtrs &ws, float *o,
                        hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  const int64_t snap_seq = s.mse ? dF : (int64_t)s.ng_cap * dF;
  const int64_t snap_group = s.mse ? 0 : dF;
  const __bf16 *snap = (const __bf16 *)ws.s + (s.mse ? 0 : (int64_t)q0 * dF);
  return launch_apply_x<C, true>(s, q0, nq, (const __bf16 *)ws.zt, snap, snap_seq, snap_group,
                           s.G > 1 ? (const __bf16 *)ws.p : nullptr, o, (const __bf16 *)ws.vt,
                           s.mse ? (__bf16 *)ws.rt : nullptr, (int64_t)s.d * s.Bp, s.Bp, st);
}

template <class C>
hipError_t launch_gram(const Slab &s, const WsPtrs &ws, hipStream_t st) {
  const int64_t RG = (int64_t)s.G * s.Bp;
  const int ng = slab_groups(s);
  const int64_t nb = ((RG + C::BM - 1) / C::BM) * ((RG + C::BN - 1) / C::BN) * ng * s.n_seq;
  hipLaunchKernelGGL(k_gram<C>, dim3((unsigned)nb), dim3(C::NTHR), 0, st, s, ng,
                     (const __bf16 *)ws.zt, (__bf16 *)ws.p, (int64_t)s.ng_cap * RG * RG);
  return hipGetLastError();
}

// Launches k_update over nb tiles, in its FULL form when the tiles cover d_ff
// and d exactly.
template <class C, bool BLK, class... Args>
hipError_t launch_k_update(const Slab &s, int64_t nb, hipStream_t st, Args... args) {
  if (s.F % C::BM == 0 && s.d % C::BN == 0)
    hipLaunchKernelGGL((k_update<C, BLK, true>), dim3((unsigned)nb), dim3(C::NTHR), 0, st, s,
                       args...);
  else
    hipLaunchKernelGGL((k_update<C, BLK, false>), dim3((unsigned)nb), dim3(C::NTHR), 0, st, s,
                       args...);
  return hipGetLastError();
}

template <class C, bool BLK>
hipError_t launch_update_scan(const Slab &s, const WsPtrs &ws, float *w_state, hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  const int64_t nb = ((s.F + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  // B operand: Vt rows c; chunk jc starts jc * Bp tokens along the row
  return launch_k_update<C, BLK>(s, nb, st, 0, s.nc, s.G, (const __bf16 *)ws.zt,
                                 (const __bf16 *)ws.vt, s.Lp, (int64_t)s.d * s.Lp, (int64_t)s.Bp,
                                 w_state, (__bf16 *)ws.s, (int64_t)s.ng_cap * dF, dF, 1, 0, 0);
}

// MSE rule over chunk groups: W += sum over the chunks of group q of
// Zt_j . Rt_j (Rt [n][d][G Bp], the group's rows), then S = bf16(W).
template <class C>
hipError_t launch_update_group(const Slab &s, int q, const WsPtrs &ws, float *w_state,
                               hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F, RG = (int64_t)s.G * s.Bp;
  const int j_first = q * s.G, n_chunks = std::min(s.G, s.nc - j_first);
  const int64_t nb = ((s.F + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  return launch_k_update<C, true>(s, nb, st, j_first, n_chunks, 1, (const __bf16 *)ws.zt,
                                  (const __bf16 *)ws.rt, RG, s.d * RG, (int64_t)s.Bp, w_state,
                                  (__bf16 *)ws.s, dF, (int64_t)0, 0, 1, 0);
}

// Backward scan: G (fp32, [n][d][F] like W) += Zt_j . Bt_j over the chunks in
// reverse, writing snap[n][j] = bf16(G) before chunk j. Bt rows c are
// token-contiguous with the slab's row layout (pitch Lp).
template <class C>
hipError_t launch_update_reverse(const Slab &s, const __bf16 *zt, const __bf16 *bt, float *g,
                                 __bf16 *snap, hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  const int64_t nb = ((s.F + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  return launch_k_update<C, false>(s, nb, st, 0, s.nc, 1, zt, bt, s.Lp, (int64_t)s.d * s.Lp,
                                   (int64_t)s.Bp, g, snap, (int64_t)s.nc_cap * dF, dF, 1, 0, 1);
}

template <class C>
hipError_t launch_update_one(const Slab &s, int j, const WsPtrs &ws, float *w_state,
                             hipStream_t st) {
  const int64_t dF = (int64_t)s.d * s.F;
  const int64_t nb = ((s.F + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  // B operand: Rt [n][d][Bp] of chunk j
  return launch_k_update<C, true>(s, nb, st, j, 1, 1, (const __bf16 *)ws.zt,
                                  (const __bf16 *)ws.rt, (int64_t)s.Bp, (int64_t)s.d * s.Bp,
                                  (int64_t)0, w_state, (__bf16 *)ws.s, dF, (int64_t)0, 0, 1, 0);
}

template <int KC>
hipError_t launch_conv(const Slab &s, const __bf16 *e, const Weights &w, const WsPtrs &ws,
                       hipStream_t st) {
  const int64_t total = (int64_t)s.nc * (s.Bp / CONV_RUN) * (s.d / 8) * s.n_seq;
  hipLaunchKernelGGL(k_conv<KC>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, s, e,
                     (const __bf16 *)w.conv_w, (__bf16 *)ws.c);
  return hipGetLastError();
}
static_assert(kChunkAlign % CONV_RUN == 0, "conv runs must not cross a chunk");

// Block shapes, MFMA shapes, LDS row layouts and stage-write points chosen by
// timing on MI355X at the 4B layer shape (d 2560, d_ff 9728, 16 chunks of
// 1024), alternating candidates within one run.
using GateUpCfg = Cfg<2, 4, 64, 16, 0, 8, 1, 4>;   // direct LDS copies, swizzled rows
using ProjCfg = Cfg<2, 4, 64, 16, 0, 8, 1, 8>;     // direct LDS copies, swizzled rows
// K-major (transposed) rows are padded by 16 elements: the four K rows one
// 16-lane transposing read touches then start 8 banks apart and never share a
// bank (a pad of 8 leaves every such read 2-way conflicted); trow_off moves the
// rows the other 16 lanes of the same 32 read onto the other half of the banks.
using ApplyCfg = Cfg<2, 4, 64, 16, 16, 16>;
using ApplySmallCfg = Cfg<1, 2, 64, 16, 16, 16>;  // when ApplyCfg would leave most CUs idle
using UpdateCfg = Cfg<1, 4, 64, 16, 0, 8, 1, 16>;  // direct copies, pipelined, interleaved fragments
using GramCfg = Cfg<2, 4, 64, 16, 16, 16>;
static_assert(kChunkAlign % UpdateCfg::BK == 0, "chunk pitch must be whole update K steps");
// The Gram computes, per m tile, the columns the apply's m tiles read: its m
// tiles must be unions of whole apply m tiles.
static_assert(GramCfg::BM % ApplyCfg::BM == 0 && GramCfg::BM % ApplySmallCfg::BM == 0,
              "Gram and apply row tiles must nest");

}  // namespace mfma

bool mfma_supported(int d, int F) { return d % 64 == 0 && F % 64 == 0; }

hipError_t mf_conv(const Slab &s, const __bf16 *e, const Weights &w, const WsPtrs &ws,
                   hipStream_t st) {
  switch (s.Kc) {
    case 1: return mfma::launch_conv<1>(s, e, w, ws, st);
    case 2: return mfma::launch_conv<2>(s, e, w, ws, st);
    case 3: return mfma::launch_conv<3>(s, e, w, ws, st);
    case 4: return mfma::launch_conv<4>(s, e, w, ws, st);
    case 5: return mfma::launch_conv<5>(s, e, w, ws, st);
    case 6: return mfma::launch_conv<6>(s, e, w, ws, st);
    case 7: return mfma::launch_conv<7>(s, e, w, ws, st);
    case 8: return mfma::launch_conv<8>(s, e, w, ws, st);
  }
  return hipErrorInvalidValue;
}
hipError_t mf_gateup(const Slab &s, const __bf16 *x, const Weights &w, const WsPtrs &ws,
                     hipStream_t st) {
  return mfma::launch_gateup<mfma::GateUpCfg, true>(s, x, w, ws, st);
}
hipError_t mf_proj(const Slab &s, const Weights &w, const WsPtrs &ws, hipStream_t st) {
  return mfma::launch_proj<mfma::ProjCfg, true>(s, w, ws, st);
}
hipError_t mf_apply(const Slab &s, int q0, int nq, const WsPtrs &ws, float *o, hipStream_t st) {
  using C = mfma::ApplyCfg;
  const int64_t big_blocks = (((int64_t)s.G * s.Bp + C::BM - 1) / C::BM) *
                             ((s.d + C::BN - 1) / C::BN) * (int64_t)nq * s.n_seq;
  if (big_blocks < 512) return mfma::launch_apply<mfma::ApplySmallCfg>(s, q0, nq, ws, o, st);
  return mfma::launch_apply<C>(s, q0, nq, ws, o, st);
}
hipError_t mf_apply_mse_group(const Slab &s, int q, const WsPtrs &ws, float *o, hipStream_t st) {
  using C = mfma::ApplyCfg;
  const int64_t RG = (int64_t)s.G * s.Bp, dF = (int64_t)s.d * s.F;
  const int64_t big_blocks = ((RG + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  const __bf16 *zt = (const __bf16 *)ws.zt, *snap = (const __bf16 *)ws.s,
               *vt = (const __bf16 *)ws.vt;
  __bf16 *rt = (__bf16 *)ws.rt;
  if (big_blocks < 512)
    return mfma::launch_apply_x<mfma::ApplySmallCfg, true>(s, q, 1, zt, snap, dF, 0, nullptr, o, vt,
                                                           rt, s.d * RG, RG, st);
  return mfma::launch_apply_x<C, true>(s, q, 1, zt, snap, dF, 0, nullptr, o, vt, rt, s.d * RG, RG,
                                       st);
}
hipError_t mf_mse_fix(const Slab &s, int q, int jl, const WsPtrs &ws, float *o, hipStream_t st) {
  using C = mfma::ApplyCfg;
  using CS = mfma::ApplySmallCfg;
  const int64_t RG = (int64_t)s.G * s.Bp;
  const int64_t big_blocks = ((s.Bp + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  const __bf16 *pt = (const __bf16 *)ws.p, *vt = (const __bf16 *)ws.vt;
  __bf16 *rt = (__bf16 *)ws.rt;
  const int64_t pseq = (int64_t)s.ng_cap * RG * RG;
  if (big_blocks < 512) {
    const int64_t nb = ((s.Bp + CS::BM - 1) / CS::BM) * ((s.d + CS::BN - 1) / CS::BN) * s.n_seq;
    hipLaunchKernelGGL((mfma::k_mse_fix<CS, (CS::WM * CS::WN >= 8)>), dim3((unsigned)nb),
                       dim3(CS::NTHR), 0, st, s, q, jl, pt, pseq, vt, rt, s.d * RG, o);
  } else {
    hipLaunchKernelGGL((mfma::k_mse_fix<C, (C::WM * C::WN >= 8)>), dim3((unsigned)big_blocks),
                       dim3(C::NTHR), 0, st, s, q, jl, pt, pseq, vt, rt, s.d * RG, o);
  }
  return hipGetLastError();
}
hipError_t mf_update_group(const Slab &s, int q, const WsPtrs &ws, float *w_state,
                           hipStream_t st) {
  return mfma::launch_update_group<mfma::UpdateCfg>(s, q, ws, w_state, st);
}
hipError_t mf_apply_mse_chunk(const Slab &s, int j, const __bf16 *zt, const __bf16 *snap,
                              int64_t snap_seq, const __bf16 *vt, __bf16 *rt, int64_t rt_seq,
                              int64_t rt_ld, hipStream_t st) {
  using C = mfma::ApplyCfg;
  const int64_t big_blocks = ((s.Bp + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  if (big_blocks < 512)
    return mfma::launch_apply_x<mfma::ApplySmallCfg, false>(s, j, 1, zt, snap, snap_seq, 0, nullptr,
                                                            nullptr, vt, rt, rt_seq, rt_ld, st);
  return mfma::launch_apply_x<C, false>(s, j, 1, zt, snap, snap_seq, 0, nullptr, nullptr, vt, rt,
                                        rt_seq, rt_ld, st);
}
hipError_t mf_apply_mse_group_rm(const Slab &s, int q, const __bf16 *zt, const __bf16 *snap,
                                 int64_t snap_seq, const __bf16 *vt, float *o, __bf16 *rt,
                                 hipStream_t st) {
  using C = mfma::ApplyCfg;
  const int64_t RG = (int64_t)s.G * s.Bp;
  const int64_t big_blocks = ((RG + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  if (big_blocks < 512)
    return mfma::launch_apply_x<mfma::ApplySmallCfg, false>(s, q, 1, zt, snap, snap_seq, 0, nullptr,
                                                            o, vt, rt, s.d * RG, RG, st);
  return mfma::launch_apply_x<C, false>(s, q, 1, zt, snap, snap_seq, 0, nullptr, o, vt, rt,
                                        s.d * RG, RG, st);
}
hipError_t mf_update_group_rm(const Slab &s, int q, const __bf16 *zt, const __bf16 *rt, float *w,
                              __bf16 *snap, int64_t snap_seq, hipStream_t st) {
  using C = mfma::UpdateCfg;
  const int64_t dF = (int64_t)s.d * s.F, RG = (int64_t)s.G * s.Bp;
  const int j_first = q * s.G, n_chunks = std::min(s.G, s.nc - j_first);
  const int64_t nb = ((s.F + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  // one copy group per chunk (G = 1 inside the launch), the B operand the
  // group's Rt rows (chunk jc at jc Bp)
  return mfma::launch_k_update<C, false>(s, nb, st, j_first, n_chunks, 1, zt, rt, RG, s.d * RG,
                                         (int64_t)s.Bp, w, snap, snap_seq, dF, 1,
                                         j_first + n_chunks < s.nc ? 1 : 0, 0);
}
hipError_t mf_update_chunk(const Slab &s, int j, const __bf16 *zt, const __bf16 *bsrc,
                           int64_t b_ld, int64_t b_seq, float *w, __bf16 *snap_after,
                           int64_t snap_seq, hipStream_t st) {
  using C = mfma::UpdateCfg;
  const int64_t nb = ((s.F + C::BM - 1) / C::BM) * ((s.d + C::BN - 1) / C::BN) * s.n_seq;
  return mfma::launch_k_update<C, false>(s, nb, st, j, 1, 1, zt, bsrc, b_ld, b_seq, (int64_t)0, w,
                                         snap_after, snap_seq, (int64_t)0, 0, snap_after ? 1 : 0,
                                         0);
}
hipError_t mf_snapshot(const Slab &s, const float *w_state, __bf16 *snap, int64_t snap_seq_stride,
                       hipStream_t st) {
  hipLaunchKernelGGL(mfma::k_snapshot_blk, dim3((unsigned)(s.d / 16), (unsigned)((s.F + 255) / 256),
                                                (unsigned)s.n_seq),
                     dim3(256), 0, st, s, w_state, snap, snap_seq_stride);
  return hipGetLastError();
}
hipError_t mf_gram(const Slab &s, const WsPtrs &ws, hipStream_t st) {
  return mfma::launch_gram<mfma::GramCfg>(s, ws, st);
}
hipError_t mf_update_scan(const Slab &s, const WsPtrs &ws, float *w_state, bool blocked,
                          hipStream_t st) {
  if (blocked) return mfma::launch_update_scan<mfma::UpdateCfg, true>(s, ws, w_state, st);
  return mfma::launch_update_scan<mfma::UpdateCfg, false>(s, ws, w_state, st);
}
hipError_t mf_update_one(const Slab &s, int j, const WsPtrs &ws, float *w_state, hipStream_t st) {
  return mfma::launch_update_one<mfma::UpdateCfg>(s, j, ws, w_state, st);
}
hipError_t mf_gateup_pre(const Slab &s, const __bf16 *x, const Weights &w, const WsPtrs &ws,
                         __bf16 *at, __bf16 *ut, hipStream_t st) {
  return mfma::launch_gateup<mfma::GateUpCfg, true>(s, x, w, ws, st, at, ut);
}
hipError_t mf_update_reverse(const Slab &s, const __bf16 *zt, const __bf16 *bt, float *g,
                             __bf16 *snap, hipStream_t st) {
  return mfma::launch_update_reverse<mfma::UpdateCfg>(s, zt, bt, g, snap, st);
}

}  // namespace ipttt
