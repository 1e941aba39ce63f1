// MFMA building blocks shared by the bf16 kernels (gfx950 / CDNA4): MFMA tile
// shapes and their lane maps, the block configuration Cfg, register-staged
// global -> LDS loaders for K-contiguous and K-major (transposed) operands and
// direct global -> LDS copies for K-contiguous ones, one LDS stage of MFMAs for
// each operand layout, the double-buffered K loops (register-staged; direct
// copies with pipelined fragments, per tile or persistent), XCD-aware block numbering
// and the slab row -> token map. Device code only; included by the .hip files
// that build kernels from these pieces.
#pragma once

#include <type_traits>

#include "internal.h"

namespace ipttt {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// MFMA tile shapes. Operand: lane l supplies row orow(l) of A (column of B) and
// K values okoff(l) .. okoff(l) + 7 of one MFMA K step (K wide). Result: the
// lane holds NG groups of 4 consecutive rows, group g starting at row
// rrow(l, g), all in column rcol(l). Any consistent assignment of K values to
// (lane, slot) gives the same sum; the row and column maps are the hardware's.
template <int FM>
struct Mfma;
template <>
struct Mfma<16> {
  typedef f32x4 acc_t;
  static constexpr int K = 32, NG = 1;
  __device__ static __forceinline__ acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int orow(int l) { return l & 15; }
  __device__ static __forceinline__ int okoff(int l) { return 8 * (l >> 4); }
  __device__ static __forceinline__ int rrow(int l, int) { return 4 * (l >> 4); }
  __device__ static __forceinline__ int rcol(int l) { return l & 15; }
  // transposed-A source address of lane l (see mma_stage_t)
  __device__ static __forceinline__ int tr_row(int l) { return 8 * (l >> 4) + (l & 15) / 4; }
  __device__ static __forceinline__ int tr_col(int l) { return 4 * (l & 3); }
};
template <>
struct Mfma<32> {
  typedef f32x16 acc_t;
  static constexpr int K = 16, NG = 4;
  __device__ static __forceinline__ acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int orow(int l) { return l & 31; }
  __device__ static __forceinline__ int okoff(int l) { return 8 * (l >> 5); }
  __device__ static __forceinline__ int rrow(int l, int g) { return 8 * g + 4 * (l >> 5); }
  __device__ static __forceinline__ int rcol(int l) { return l & 31; }
  __device__ static __forceinline__ int tr_row(int l) { return 8 * (l >> 5) + (l & 15) / 4; }
  __device__ static __forceinline__ int tr_col(int l) { return 16 * ((l >> 4) & 1) + 4 * (l & 3); }
};

__device__ __forceinline__ f32x4 get4(const f32x4 &a, int) { return a; }
__device__ __forceinline__ f32x4 get4(const f32x16 &a, int g) {
  return f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
}
__device__ __forceinline__ void set4(f32x4 &a, int, f32x4 v) { a = v; }
__device__ __forceinline__ void set4(f32x16 &a, int g, f32x4 v) {
  a[4 * g] = v[0];
  a[4 * g + 1] = v[1];
  a[4 * g + 2] = v[2];
  a[4 * g + 3] = v[3];
}

template <int WM_, int WN_, int BK_, int FM_ = 32, int PAD_ = 16, int PADT_ = 8, int OCC_ = 1,
          int GM_ = 8, int WTN_ = 64, int MID_ = 0>
struct Cfg {
  static constexpr int WM = WM_, WN = WN_, BK = BK_, FM = FM_;
  // MFMA sub-steps of a K step done before the next step's LDS writes (0: all;
  // the writes then follow the whole step's MFMAs)
  static constexpr int MID = MID_;
  static constexpr int GM = GM_;  // row tiles per group in the tile order (tile_of)
  static constexpr int OCC = OCC_;  // waves per SIMD the register allocation must allow
  using M = Mfma<FM>;
  using acc_t = typename M::acc_t;
  static constexpr int WTM = 128, WTN = WTN_;  // wave tile
  static constexpr int MI = WTM / FM, NJ = WTN / FM;
  static constexpr int BM = WTM * WM, BN = WTN * WN;
  static constexpr int NTHR = 64 * WM * WN;
  static constexpr int PITCH = BK + PAD_;  // LDS row pitch in bf16
  // PAD_ = 0: unpadded rows with the 16-byte pieces of row r stored XOR-permuted
  // (piece q at slot q ^ swz(r)), so that the 16 rows one fragment read touches
  // and the rows one stage write touches fall on distinct banks.
  static constexpr bool SWZ = PAD_ == 0;
  static constexpr int KP = BK / 8;        // 16-byte pieces per row per step
  static constexpr int RPP = NTHR / KP;    // rows covered by one pass of all threads
  static constexpr int A_PIECES = BM / RPP;
  static constexpr int B_PIECES = BN / RPP;
  static constexpr int A_STAGE = BM * PITCH, B_STAGE = BN * PITCH;
  static constexpr int SMEM_ELEMS = 2 * (A_STAGE + B_STAGE);
  // A held K-major in LDS ([BK rows of K][BM columns of M]) for an A operand
  // stored M-contiguous in memory; a stage also holds the 64-element shift of
  // each run of 8 K rows (trow_off).
  static constexpr int PITCH_T = BM + PADT_;
  static constexpr int AT_PIECES = BK * (BM / 8) / NTHR;
  static constexpr int AT_STAGE = BK * PITCH_T + 64 * (BK / 8);
  static constexpr int SMEM_T_ELEMS = 2 * (AT_STAGE + B_STAGE);
  // both operands K-major ([BK rows of K][BM or BN columns])
  static constexpr int PITCH_TB = BN + PADT_;
  static constexpr int BT_STAGE = BK * PITCH_TB + 64 * (BK / 8);
  static constexpr int SMEM_TT_ELEMS = 2 * (AT_STAGE + BT_STAGE);
  static_assert(BK % 32 == 0 && BM % RPP == 0 && BN % RPP == 0, "bad tile config");
  static_assert(PAD_ % 8 == 0 && PADT_ % 4 == 0, "LDS rows must keep 16 / 8-byte alignment");
  static_assert(!SWZ || (BK == 32 || BK == 64), "swizzled rows need 128 / BK rows per bank span");
  static_assert((BK * (BM / 8)) % NTHR == 0 && (BK * (BN / 8)) % NTHR == 0,
                "bad transposed tile config");
};

__device__ __forceinline__ uint4 ld16(const __bf16 *p) { return *(const uint4 *)p; }

// Logistic sigmoid 1 / (1 + e^-a) with the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each in fp32, far below the bf16 rounding
// every use here ends in); a correctly rounded reciprocal expands to a full
// division sequence per element.
__device__ __forceinline__ float fast_sigmoid(float a) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-a));
}

// Logical block index: the hardware hands consecutive workgroups to the 8 XCDs
// in turn; give each XCD a contiguous range of logical tiles so that tiles
// that share operands also share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int x = bid % 8, q = bid / 8;
  return x * per + min(x, rem) + q;
}

// Tile order inside a grid of (nm x nn) tiles: groups of GM row tiles, column
// tile slowest within a group, so neighbouring blocks share both operands.
template <int GM>
__device__ __forceinline__ void tile_of(int id, int nm, int nn, int &tm, int &tn) {
  const int group = id / (GM * nn);
  const int first = group * GM;
  const int gm = min(GM, nm - first);
  const int in = id % (GM * nn);
  tm = first + in % gm;
  tn = in / gm;
}

// LDS element offset within row `row` of K offset k (a multiple of 8) for a
// K-contiguous operand tile: k itself, or with the 16-byte piece index XORed
// by a function of the row (Cfg::SWZ). 128 / BK consecutive rows cover the 64
// banks once, so the XOR key counts in units of that many rows.
template <class C>
__device__ __forceinline__ int kslot(int row, int k) {
  if constexpr (C::SWZ) {
    constexpr int rows_per_span = 128 / C::BK;
    return k ^ (8 * ((row / rows_per_span) & (C::KP - 1)));
  } else {
    return k;
  }
}

// Per-thread loader: the rows this thread copies into LDS (row (tid / KP) +
// RPP i, 16-byte piece tid % KP). Rows outside the matrix point at a valid row
// of it: every load is unconditional and nothing consumes the loaded value
// before it is stored to LDS, so the loads of the next step stay in flight
// behind the current step's MFMAs. The rows they feed are masked at the
// epilogue (each output row or column depends only on its own operand row).
template <class C, int NP>
struct Loader {
  const __bf16 *ptr[NP];
  uint4 v[NP];
  __device__ __forceinline__ void fetch(int k0, int q) {
#pragma unroll
    for (int i = 0; i < NP; ++i) v[i] = ld16(ptr[i] + k0 + 8 * q);
  }
  __device__ __forceinline__ void stash(__bf16 *stage, int r0, int q) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int row = r0 + C::RPP * i;
      *(uint4 *)(stage + row * C::PITCH + kslot<C>(row, 8 * q)) = v[i];
    }
  }
};

// Per-thread loader of a K-contiguous operand stored in blocks of 8 K values
// (element (n, k) at ((k / 8) * rows + n) * 8 + k % 8, the layout of the
// forward's fast-weight copies): piece q of the K step at k0 of row n is the
// 16 bytes of block k0 / 8 + q. It fills the same LDS tile as Loader, but a
// thread's (row, piece) is its own (r0, q below, not the ones the K loop
// passes): each 16 lanes take rows r .. r + 7 of pieces q, q + 1, two whole
// 128-byte lines of the blocked layout, and each 8 lanes take 4 rows of both
// pieces, which land on distinct LDS banks at a 160-byte row pitch.
template <class C, int NP>
struct BlockLoader {
  static_assert(C::KP % 2 == 0 && C::RPP % 8 == 0 && C::NTHR % (8 * C::KP) == 0,
                "BlockLoader lane map");
  const __bf16 *ptr[NP];  // row r0 + RPP i of block 0: base + 8 (r0 + RPP i)
  int64_t blk;            // elements between consecutive blocks (8 x rows)
  int r0, q;
  uint4 v[NP];
  __device__ __forceinline__ void assign(int tid) {
    const int l16 = tid % 16, g = tid / 16;
    q = 2 * (g % (C::KP / 2)) + (l16 / 4) % 2;
    r0 = 8 * (g / (C::KP / 2)) + l16 % 4 + 4 * (l16 / 8);
  }
  __device__ __forceinline__ void fetch(int k0, int) {
#pragma unroll
    for (int i = 0; i < NP; ++i) v[i] = ld16(ptr[i] + (int64_t)(k0 / 8 + q) * blk);
  }
  __device__ __forceinline__ void stash(__bf16 *stage, int, int) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int row = r0 + C::RPP * i;
      *(uint4 *)(stage + row * C::PITCH + kslot<C>(row, 8 * q)) = v[i];
    }
  }
};

// MFMA sub-steps [U0, U1) of one LDS stage (all of them by default).
template <class C, int U0 = 0, int U1 = C::BK / C::M::K>
__device__ __forceinline__ void mma_stage(const __bf16 *As, const __bf16 *Bs, int arow0,
                                          const int (&brow)[C::NJ], int lane,
                                          typename C::acc_t (&acc)[C::MI][C::NJ]) {
  using M = typename C::M;
  const int r = M::orow(lane), kq = M::okoff(lane);
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    bf16x8 a[C::MI], b[C::NJ];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
      b[j] = *(const bf16x8 *)(Bs + (brow[j] + r) * C::PITCH + kslot<C>(brow[j] + r, M::K * u + kq));
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
      a[i] = *(const bf16x8 *)(As + (arow0 + C::FM * i + r) * C::PITCH +
                               kslot<C>(arow0 + C::FM * i + r, M::K * u + kq));
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) acc[i][j] = M::mma(a[i], b[j], acc[i][j]);
  }
}

// ---- A operand stored M-contiguous (K-major rows) ---------------------------
// Start of K row r in a K-major LDS tile of COLS columns. The hardware serves
// a transposing read 32 lanes (256 bytes, all 64 banks) at a time, and the
// second 16-lane group of each 32 reads the K rows 8 below the first group's
// (the next 8 K values of its MFMA operand). At the padded pitch alone those
// rows start on the same banks (8 rows of 8 banks each: 64); shifting every
// run of 8 K rows by a further 64 elements (128 bytes, half the banks) puts
// the two groups on disjoint halves. Tiles narrower than 128 columns keep
// plain rows.
template <int COLS>
__device__ __forceinline__ int trow_off(int r, int pitch) {
  if constexpr (COLS >= 128) return r * pitch + 64 * (r >> 3); else return r * pitch;
}

// The tile is copied into LDS as BK rows of BM elements; each MFMA A fragment
// (8 consecutive K values of one M row per lane) is assembled from two
// ds_read_b64_tr_b16. That instruction works on groups of 16 lanes: lane i of
// a group receives element (i % 4) of the 8-byte chunk read by lane 4 j + i / 4
// of the group, for j = 0..3. Source lane p therefore points at K row (p / 4)
// and M columns 4 (p % 4) .. + 3 of a 4 x 16 block, and lane i gets that
// block's column i: 4 consecutive K values of M row i (tr_row / tr_col place
// each 16-lane group on the rows and K values its MFMA operand needs).
// COLS = BM for the A operand, BN for a B operand stored N-contiguous (its
// fragments are read the same way, the MFMA B layout mirroring A's).
template <class C, int COLS>
struct LoaderT {
  static constexpr int NP = C::BK * (COLS / 8) / C::NTHR;
  static constexpr int PITCH = COLS + (C::PITCH_T - C::BM);
  const __bf16 *ptr[NP];  // piece i's K row start, offset to its columns
  int64_t ld;             // elements between K rows
  uint4 v[NP];
  // the K row and first column of piece i of thread tid within a step
  __device__ static __forceinline__ int krow(int tid, int i) { return (tid + i * C::NTHR) / (COLS / 8); }
  __device__ static __forceinline__ int col(int tid, int i) { return 8 * ((tid + i * C::NTHR) % (COLS / 8)); }
  __device__ __forceinline__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < NP; ++i) v[i] = ld16(ptr[i] + (int64_t)k0 * ld);
  }
  __device__ __forceinline__ void stash(__bf16 *stage, int tid) const {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      *(uint4 *)(stage + trow_off<COLS>(krow(tid, i), PITCH) + col(tid, i)) = v[i];
  }
};

__device__ __forceinline__ v4i16 ds_read_tr16(const __bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
}

// One MFMA operand fragment (8 K values of one row) from a K-major LDS tile
// of row pitch `pitch`, via two transposing reads.
template <class M, int COLS>
__device__ __forceinline__ bf16x8 frag_t(const __bf16 *tile, int pitch, int u, int col0, int trr,
                                         int trc) {
  // K u is a multiple of 8, so the row offset splits into a constant and the lane's part
  const __bf16 *base =
      tile + trow_off<COLS>(M::K * u, pitch) + trow_off<COLS>(trr, pitch) + col0 + trc;
  const v4i16 lo = ds_read_tr16(base), hi = ds_read_tr16(base + 4 * pitch);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// TB = false: B tile row-major [BN][BK] (K-contiguous); true: K-major like A.
template <class C, bool TB, int U0 = 0, int U1 = C::BK / C::M::K>
__device__ __forceinline__ void mma_stage_t(const __bf16 *At, const __bf16 *Bs, int arow0,
                                            const int (&brow)[C::NJ], int lane,
                                            typename C::acc_t (&acc)[C::MI][C::NJ]) {
  using M = typename C::M;
  const int r = M::orow(lane), kq = M::okoff(lane);
  const int trr = M::tr_row(lane), trc = M::tr_col(lane);
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    bf16x8 a[C::MI], b[C::NJ];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
      b[j] = TB ? frag_t<M, C::BN>(Bs, C::PITCH_TB, u, brow[j], trr, trc)
                : *(const bf16x8 *)(Bs + (brow[j] + r) * C::PITCH +
                                    kslot<C>(brow[j] + r, M::K * u + kq));
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
      a[i] = frag_t<M, C::BM>(At, C::PITCH_T, u, arow0 + C::FM * i, trr, trc);
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) acc[i][j] = M::mma(a[i], b[j], acc[i][j]);
  }
}

// Sub-steps of a K step done before the next step's LDS writes (Cfg::MID).
template <class C>
constexpr int mid_step() {
  constexpr int NU = C::BK / C::M::K;
  return (C::MID > 0 && C::MID < NU) ? C::MID : NU;
}

// Register-staged K loops over nk steps of BK with double-buffered LDS: the
// next step's global loads go to registers before this step's MFMAs and to
// LDS after them (or after MID sub-steps). Stage addresses are formed
// arithmetically from the __shared__ base so the compiler keeps them in the
// LDS address space (ds_read / ds_write, not flat).
// A K-major (transposed) operand and a K-contiguous B operand (the apply):
template <class C, class LB>
__device__ __forceinline__ void kloop_t(__bf16 *smem, LoaderT<C, C::BM> &la, LB &lb, int nk,
                                        int tid, int arow0,
                                        const int (&brow)[C::NJ],
                                        typename C::acc_t (&acc)[C::MI][C::NJ]) {
  __bf16 *const Bbase = smem + 2 * C::AT_STAGE;
  const int lane = tid & 63, r0 = tid / C::KP, q = tid % C::KP;
  la.fetch(0);
  lb.fetch(0, q);
  la.stash(smem, tid);
  lb.stash(Bbase, r0, q);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    if (s + 1 < nk) {
      la.fetch((s + 1) * C::BK);
      lb.fetch((s + 1) * C::BK, q);
    }
    mma_stage_t<C, false, 0, mid_step<C>()>(smem + cur * C::AT_STAGE, Bbase + cur * C::B_STAGE,
                                             arow0, brow, lane, acc);
    if (s + 1 < nk) {
      la.stash(smem + (cur ^ 1) * C::AT_STAGE, tid);
      lb.stash(Bbase + (cur ^ 1) * C::B_STAGE, r0, q);
    }
    mma_stage_t<C, false, mid_step<C>()>(smem + cur * C::AT_STAGE, Bbase + cur * C::B_STAGE, arow0,
                                         brow, lane, acc);
    __syncthreads();
  }
}

// Both operands K-major in memory (the Gram product of Zt with itself).
template <class C>
__device__ __forceinline__ void kloop_tt(__bf16 *smem, LoaderT<C, C::BM> &la,
                                         LoaderT<C, C::BN> &lb, int nk, int tid, int arow0,
                                         const int (&brow)[C::NJ],
                                         typename C::acc_t (&acc)[C::MI][C::NJ]) {
  __bf16 *const Bbase = smem + 2 * C::AT_STAGE;
  const int lane = tid & 63;
  la.fetch(0);
  lb.fetch(0);
  la.stash(smem, tid);
  lb.stash(Bbase, tid);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    if (s + 1 < nk) {
      la.fetch((s + 1) * C::BK);
      lb.fetch((s + 1) * C::BK);
    }
    mma_stage_t<C, true, 0, mid_step<C>()>(smem + cur * C::AT_STAGE, Bbase + cur * C::BT_STAGE,
                                            arow0, brow, lane, acc);
    if (s + 1 < nk) {
      la.stash(smem + (cur ^ 1) * C::AT_STAGE, tid);
      lb.stash(Bbase + (cur ^ 1) * C::BT_STAGE, tid);
    }
    mma_stage_t<C, true, mid_step<C>()>(smem + cur * C::AT_STAGE, Bbase + cur * C::BT_STAGE, arow0,
                                        brow, lane, acc);
    __syncthreads();
  }
}

template <class C>
__device__ __forceinline__ void zero_acc(typename C::acc_t (&acc)[C::MI][C::NJ]) {
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = typename C::acc_t{};
}

// ---- any operand layout: TA / TB = A / B stored K-major (M- / N-contiguous) --
template <class C, bool TA, bool TB>
struct GLoaders {
  using LA = typename std::conditional<TA, LoaderT<C, C::BM>, Loader<C, C::A_PIECES>>::type;
  using LB = typename std::conditional<TB, LoaderT<C, C::BN>, Loader<C, C::B_PIECES>>::type;
  static constexpr int A_ST = TA ? C::AT_STAGE : C::A_STAGE;
  static constexpr int B_ST = TB ? C::BT_STAGE : C::B_STAGE;
  static constexpr int SMEM = 2 * (A_ST + B_ST);
};

template <class C, int NP>
__device__ __forceinline__ void gfetch(Loader<C, NP> &l, int k0, int q) { l.fetch(k0, q); }
template <class C, int COLS>
__device__ __forceinline__ void gfetch(LoaderT<C, COLS> &l, int k0, int) { l.fetch(k0); }
template <class C, int NP>
__device__ __forceinline__ void gstash(const Loader<C, NP> &l, __bf16 *st, int, int r0, int q) {
  l.stash(st, r0, q);
}
template <class C, int NP>
__device__ __forceinline__ void gfetch(BlockLoader<C, NP> &l, int k0, int q) { l.fetch(k0, q); }
template <class C, int NP>
__device__ __forceinline__ void gstash(const BlockLoader<C, NP> &l, __bf16 *st, int, int r0,
                                       int q) {
  l.stash(st, r0, q);
}
template <class C, int COLS>
__device__ __forceinline__ void gstash(const LoaderT<C, COLS> &l, __bf16 *st, int tid, int, int) {
  l.stash(st, tid);
}

template <class C, bool TA, bool TB, int U0 = 0, int U1 = C::BK / C::M::K>
__device__ __forceinline__ void mma_stage_g(const __bf16 *As, const __bf16 *Bs, int arow0,
                                            const int (&brow)[C::NJ], int lane,
                                            typename C::acc_t (&acc)[C::MI][C::NJ]) {
  using M = typename C::M;
  const int r = M::orow(lane), kq = M::okoff(lane);
  const int trr = M::tr_row(lane), trc = M::tr_col(lane);
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    bf16x8 a[C::MI], b[C::NJ];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
      b[j] = TB ? frag_t<M, C::BN>(Bs, C::PITCH_TB, u, brow[j], trr, trc)
                : *(const bf16x8 *)(Bs + (brow[j] + r) * C::PITCH +
                                    kslot<C>(brow[j] + r, M::K * u + kq));
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
      a[i] = TA ? frag_t<M, C::BM>(As, C::PITCH_T, u, arow0 + C::FM * i, trr, trc)
                : *(const bf16x8 *)(As + (arow0 + C::FM * i + r) * C::PITCH +
                                    kslot<C>(arow0 + C::FM * i + r, M::K * u + kq));
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) acc[i][j] = M::mma(a[i], b[j], acc[i][j]);
  }
}

template <class C, bool TA, bool TB>
__device__ __forceinline__ void kloop_g(__bf16 *smem, typename GLoaders<C, TA, TB>::LA &la,
                                        typename GLoaders<C, TA, TB>::LB &lb, int nk, int tid,
                                        int arow0, const int (&brow)[C::NJ],
                                        typename C::acc_t (&acc)[C::MI][C::NJ]) {
  using GL = GLoaders<C, TA, TB>;
  __bf16 *const Bbase = smem + 2 * GL::A_ST;
  const int lane = tid & 63, r0 = tid / C::KP, q = tid % C::KP;
  gfetch(la, 0, q);
  gfetch(lb, 0, q);
  gstash(la, smem, tid, r0, q);
  gstash(lb, Bbase, tid, r0, q);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    if (s + 1 < nk) {
      gfetch(la, (s + 1) * C::BK, q);
      gfetch(lb, (s + 1) * C::BK, q);
    }
    mma_stage_g<C, TA, TB, 0, mid_step<C>()>(smem + cur * GL::A_ST, Bbase + cur * GL::B_ST, arow0,
                                              brow, lane, acc);
    if (s + 1 < nk) {
      gstash(la, smem + (cur ^ 1) * GL::A_ST, tid, r0, q);
      gstash(lb, Bbase + (cur ^ 1) * GL::B_ST, tid, r0, q);
    }
    mma_stage_g<C, TA, TB, mid_step<C>()>(smem + cur * GL::A_ST, Bbase + cur * GL::B_ST, arow0,
                                          brow, lane, acc);
    __syncthreads();
  }
}

// kloop_g with each step's memory work spread among its MFMAs, for blocks of
// two waves per SIMD: the next step's global loads between the first
// sub-steps' MFMAs, its LDS writes between the last sub-step's MFMAs (all
// waves leave each barrier together, so bursts of memory instructions before
// or after the MFMAs leave the SIMDs idle). The last step (no next stage) is
// peeled, so each main-loop step is one block. Same arithmetic as kloop_g.
template <class C, bool TA, bool TB, class LA, class LB>
__device__ __forceinline__ void kloop_g_il(__bf16 *smem, LA &la, LB &lb, int nk, int tid,
                                           int arow0, const int (&brow)[C::NJ],
                                           typename C::acc_t (&acc)[C::MI][C::NJ]) {
  using GL = GLoaders<C, TA, TB>;
  constexpr int NU = C::BK / C::M::K;
  static_assert(NU >= 2, "two or more MFMA sub-steps per stage");
  constexpr int NVA = TA ? LoaderT<C, C::BM>::NP : C::A_PIECES;
  constexpr int NVB = TB ? LoaderT<C, C::BN>::NP : C::B_PIECES;
  constexpr int NV = NVA + NVB;  // global loads (and LDS writes) per step
  static_assert(NV <= C::MI * C::NJ, "more memory instructions than MFMAs to hide them");
  __bf16 *const Bbase = smem + 2 * GL::A_ST;
  const int lane = tid & 63, r0 = tid / C::KP, q = tid % C::KP;
  gfetch(la, 0, q);
  gfetch(lb, 0, q);
  gstash(la, smem, tid, r0, q);
  gstash(lb, Bbase, tid, r0, q);
  __syncthreads();
  const auto step = [&](int s, auto more) __attribute__((always_inline)) {
    constexpr bool MORE = decltype(more)::value;
    const int cur = s & 1;
    if constexpr (MORE) {
      gfetch(la, (s + 1) * C::BK, q);
      gfetch(lb, (s + 1) * C::BK, q);
    }
    mma_stage_g<C, TA, TB, 0, NU - 1>(smem + cur * GL::A_ST, Bbase + cur * GL::B_ST, arow0, brow,
                                      lane, acc);
    if constexpr (MORE) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    mma_stage_g<C, TA, TB, NU - 1>(smem + cur * GL::A_ST, Bbase + cur * GL::B_ST, arow0, brow,
                                   lane, acc);
    if constexpr (MORE) {
      gstash(la, smem + (cur ^ 1) * GL::A_ST, tid, r0, q);
      gstash(lb, Bbase + (cur ^ 1) * GL::B_ST, tid, r0, q);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  int s = 0;
  for (; s + 1 < nk; ++s) step(s, std::true_type());
  if (s < nk) step(s, std::false_type());
}

// ---- direct global -> LDS loads (K-contiguous operands, swizzled rows) -------
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory into LDS
// at a wave-uniform base + 16 x lane without passing through registers, so the
// K loop needs no staging registers and no LDS write instructions. The copies
// are counted by vmcnt; the loops below wait for them explicitly (vector
// memory loads complete in issue order) and then pass a block barrier.

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_cvoid_t;

// Wait until at most N vector-memory operations of this wave are outstanding.
// The memory clobber keeps LDS reads of the landed stage below it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block barrier after this wave's LDS reads have completed: after it no wave
// still reads a stage that the next copies overwrite.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Copies ROWS rows x BK elements of one operand per stage. One instruction
// fills 1 KB = RPI rows; instruction i of wave w fills rows (i NW + w) RPI ..
// + RPI. Lane l writes row (l / KP), LDS slot (l % KP); the swizzled layout
// puts logical piece kslot(row, slot) there (the XOR is its own inverse), so
// the lane loads that piece. Rows outside the matrix point at a valid row
// (masked at the epilogue, as with the register loaders).
template <class C, int ROWS>
struct DmaLoader {
  static constexpr int NW = C::NTHR / 64;
  static constexpr int RPI = 512 / C::BK;
  static constexpr int NI = ROWS / (RPI * NW);  // instructions per wave per stage
  static_assert(C::SWZ, "direct LDS copies need unpadded (swizzled) rows");
  static_assert(ROWS % (RPI * NW) == 0, "rows must split evenly over the waves");
  static constexpr int STAGE = ROWS * C::BK;  // elements per stage
  const __bf16 *ptr[NI];  // this lane's source at K offset 0
  // rowptr(r): start of tile row r (K offset 0)
  template <class RowPtr>
  __device__ __forceinline__ void init(int wave, int lane, RowPtr rowptr) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (i * NW + wave) * RPI + lane / C::KP;
      ptr[i] = rowptr(row) + kslot<C>(row, 8 * (lane % C::KP));
    }
  }
  // wave must be wave-uniform (readfirstlane), as the LDS base is
  __device__ __forceinline__ void issue(__bf16 *stage, int wave, int64_t koff) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_global_load_lds((gbl_cvoid_t *)(ptr[i] + koff),
                                       (lds_void_t *)(stage + (i * NW + wave) * RPI * C::BK), 16, 0,
                                       0);
  }
};

// The operand fragments of one MFMA sub-step (K = M::K) of a stage.
template <class C>
struct Frags {
  bf16x8 a[C::MI], b[C::NJ];
};
template <class C>
__device__ __forceinline__ void load_frags(const __bf16 *As, const __bf16 *Bs, int u, int arow0,
                                           const int (&brow)[C::NJ], int lane, Frags<C> &f) {
  using M = typename C::M;
  const int r = M::orow(lane), kq = M::okoff(lane);
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
    f.b[j] = *(const bf16x8 *)(Bs + (brow[j] + r) * C::PITCH +
                               kslot<C>(brow[j] + r, M::K * u + kq));
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
    f.a[i] = *(const bf16x8 *)(As + (arow0 + C::FM * i + r) * C::PITCH +
                               kslot<C>(arow0 + C::FM * i + r, M::K * u + kq));
}
template <class C>
__device__ __forceinline__ void mma_frags(const Frags<C> &f,
                                          typename C::acc_t (&acc)[C::MI][C::NJ]) {
  using M = typename C::M;
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = M::mma(f.a[i], f.b[j], acc[i][j]);
}
// An asm statement that reads f: the compiler waits for f's loads before it.
// After a direct LDS copy the compiler's next LDS wait drains every LDS read
// in flight; placed where f is known to have landed, this absorbs that wait,
// so the MFMAs that follow do not also wait for the next prefetch.
template <class C>
__device__ __forceinline__ void touch(const Frags<C> &f) {
#pragma unroll
  for (int i = 0; i < C::MI; ++i) asm volatile("" ::"v"(f.a[i]));
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) asm volatile("" ::"v"(f.b[j]));
}

// Scheduling pattern for one MFMA sub-step: NV direct copies, then ND LDS
// fragment reads, each issued between two of the NM MFMAs, so that the issue of
// the memory instructions hides under MFMA execution instead of delaying the
// first MFMA (all waves leave a barrier together, so no other wave has MFMAs
// ready to fill that gap). Applies to the scheduling region it ends.
template <int NV, int ND, int NM>
__device__ __forceinline__ void interleave_mfma() {
  static_assert(NV + ND <= NM, "more memory instructions than MFMAs to hide them");
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - NV - ND, 0);
}

// Software-pipelined K loop: the fragments of sub-step u + 1 load while
// sub-step u's MFMAs run, and the barrier sits between a stage's last fragment
// loads and its last MFMAs, so the next stage's first fragments and the
// refill of the stage just consumed load behind those MFMAs. NS stages are
// filled by direct copies NS steps ahead; the last NS steps (no refill) run as
// a peeled tail, so every step of the main loop is one straight block. IL:
// the copies and fragment reads are interleaved with the MFMAs (two waves per
// SIMD, where all waves leave each barrier together); otherwise they are all
// issued ahead of the MFMAs (one wave per SIMD, measured faster there).
// pre(s) runs before step s's MFMAs (the accumulators then hold steps
// 0 .. s - 1) and post(s) after step s's barrier, ahead of the refill (the
// next step's vmcnt wait covers any global stores it issues).
// ldf(As, Bs, u, f) reads sub-step u's fragments of a stage; ND is the number
// of LDS read instructions it issues.
template <class C, int NS, bool IL, int ND, class LA, class LB, class Ldf, class Koff, class Pre,
          class Post>
__device__ __forceinline__ void kloop_dma_pl(__bf16 *smem, const LA &la, const LB &lb, int nk,
                                             int wave, typename C::acc_t (&acc)[C::MI][C::NJ],
                                             Ldf ldf, Koff koff, Pre pre, Post post) {
  constexpr int NU = C::BK / C::M::K;
  static_assert(NU >= 2, "two or more MFMA sub-steps per stage");
  constexpr int AS = LA::STAGE, ST = AS + LB::STAGE;
  constexpr int IPW = LA::NI + LB::NI;
  constexpr int NFR = ND, NMF = C::MI * C::NJ;
  int64_t ka, kb;
#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < nk) {
      koff(p, ka, kb);
      la.issue(smem + p * ST, wave, ka);
      lb.issue(smem + p * ST + AS, wave, kb);
    }
  if (NS - 1 < nk)
    wait_vm<(NS - 1) * IPW>();
  else
    wait_vm<0>();
  lds_barrier();
  Frags<C> f[2];
  ldf(smem, smem + AS, 0, f[0]);
  // keep this load apart from the loop's prefetch (the compiler would
  // otherwise merge the two into one load at the loop head)
#pragma unroll
  for (int i = 0; i < C::MI; ++i) asm volatile("" : "+v"(f[0].a[i]));
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) asm volatile("" : "+v"(f[0].b[j]));
  int cur = 0;
  const auto step = [&](int s, auto refill) __attribute__((always_inline)) {
    constexpr bool RF = decltype(refill)::value;
    const __bf16 *st = smem + cur * ST;
#pragma unroll
    for (int u = 0; u + 1 < NU; ++u) {
      touch<C>(f[u & 1]);
      ldf(st, st + AS, u + 1, f[(u + 1) & 1]);
      if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
      if (u == 0) pre(s);
      mma_frags<C>(f[u & 1], acc);
      if constexpr (IL) interleave_mfma<0, NFR, NMF>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s + NS - 1 < nk)
      wait_vm<(NS - 2) * IPW>();  // step s + 1 landed
    else
      wait_vm<0>();
    lds_barrier();
    touch<C>(f[(NU - 1) & 1]);
    post(s);
    if constexpr (RF) {  // refill this step's stage
      koff(s + NS, ka, kb);
      la.issue(smem + cur * ST, wave, ka);
      lb.issue(smem + cur * ST + AS, wave, kb);
    }
    cur = cur + 1 == NS ? 0 : cur + 1;
    // the next step's first fragments (after the last step: an unused read of
    // a valid stage)
    ldf(smem + cur * ST, smem + cur * ST + AS, 0, f[NU & 1]);
    if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
    mma_frags<C>(f[(NU - 1) & 1], acc);
    if constexpr (IL) interleave_mfma<RF ? IPW : 0, NFR, NMF>();
    __builtin_amdgcn_sched_barrier(0);
  };
  int s = 0;
  for (; s < nk - NS; ++s) step(s, std::true_type());
  for (; s < nk; ++s) step(s, std::false_type());
  lds_barrier();
}

// Persistent form of kloop_dma_pl: the block runs nt tiles of nk K steps each
// as one stream of nt nk steps. Copies run NS steps ahead across tile
// boundaries, so a tile's first stages land during the previous tile's last
// steps, and epi(t) (tile t's epilogue, from the accumulators) runs between
// tile t's last MFMAs and tile t + 1's first, with t + 1's first fragments
// already in registers; its stores stay in flight over t + 1's first MFMA
// sub-step (the next vmcnt wait covers them).
// next(t) points the loaders at tile t (called before tile t's first copy);
// koff(s, ka, kb) gives step s's offsets within a tile.
template <class C, int NS, bool IL, int ND, class LA, class LB, class Ldf, class Koff, class Next,
          class Epi>
__device__ __forceinline__ void kloop_dma_pl_tiles(__bf16 *smem, LA &la, LB &lb, int nt, int nk,
                                                   int wave,
                                                   typename C::acc_t (&acc)[C::MI][C::NJ],
                                                   Ldf ldf, Koff koff, Next next, Epi epi) {
  constexpr int NU = C::BK / C::M::K;
  static_assert(NU >= 2, "two or more MFMA sub-steps per stage");
  constexpr int AS = LA::STAGE, ST = AS + LB::STAGE;
  constexpr int IPW = LA::NI + LB::NI;
  constexpr int NFR = ND, NMF = C::MI * C::NJ;
  const int total = nt * nk;
  int lt = 0, ls = 0;  // tile and step of the next copy
  const auto advance = [&]() __attribute__((always_inline)) {
    if (ls == nk && lt + 1 < nt) {  // the next copy starts the next tile
      ls = 0;
      next(++lt);
    }
  };
  int64_t ka, kb;
  next(0);
#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < total) {
      koff(ls++, ka, kb);
      la.issue(smem + p * ST, wave, ka);
      lb.issue(smem + p * ST + AS, wave, kb);
      advance();
    }
  if (NS - 1 < total)
    wait_vm<(NS - 1) * IPW>();
  else
    wait_vm<0>();
  lds_barrier();
  zero_acc<C>(acc);
  Frags<C> f[2];
  ldf(smem, smem + AS, 0, f[0]);
#pragma unroll
  for (int i = 0; i < C::MI; ++i) asm volatile("" : "+v"(f[0].a[i]));
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) asm volatile("" : "+v"(f[0].b[j]));
  int cur = 0, ct = 0, cs = 0;  // stage, tile and step being computed
  const auto step = [&](int g, auto refill) __attribute__((always_inline)) {
    constexpr bool RF = decltype(refill)::value;
    const __bf16 *st = smem + cur * ST;
#pragma unroll
    for (int u = 0; u + 1 < NU; ++u) {
      touch<C>(f[u & 1]);
      ldf(st, st + AS, u + 1, f[(u + 1) & 1]);
      if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
      mma_frags<C>(f[u & 1], acc);
      if constexpr (IL) interleave_mfma<0, NFR, NMF>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (g + NS - 1 < total)
      wait_vm<(NS - 2) * IPW>();  // step g + 1 landed
    else
      wait_vm<0>();
    lds_barrier();
    touch<C>(f[(NU - 1) & 1]);
    if constexpr (RF) {  // refill this step's stage with step g + NS
      koff(ls++, ka, kb);
      la.issue(smem + cur * ST, wave, ka);
      lb.issue(smem + cur * ST + AS, wave, kb);
    }
    cur = cur + 1 == NS ? 0 : cur + 1;
    ldf(smem + cur * ST, smem + cur * ST + AS, 0, f[NU & 1]);
    if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
    mma_frags<C>(f[(NU - 1) & 1], acc);
    if constexpr (IL) interleave_mfma<RF ? IPW : 0, NFR, NMF>();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RF) advance();
    if (++cs == nk) {
      epi(ct);
      zero_acc<C>(acc);
      cs = 0;
      ++ct;
    }
  };
  int g = 0;
  for (; g < total - NS; ++g) step(g, std::true_type());
  for (; g < total; ++g) step(g, std::false_type());
  lds_barrier();
}

// Both operands K-contiguous (swizzled rows).
template <class C, int NS, bool IL, class Koff, class Pre, class Post>
__device__ __forceinline__ void kloop_dma_pl(__bf16 *smem, const DmaLoader<C, C::BM> &la,
                                             const DmaLoader<C, C::BN> &lb, int nk, int wave,
                                             int lane, int arow0, const int (&brow)[C::NJ],
                                             typename C::acc_t (&acc)[C::MI][C::NJ], Koff koff,
                                             Pre pre, Post post) {
  kloop_dma_pl<C, NS, IL, C::MI + C::NJ>(
      smem, la, lb, nk, wave, acc,
      [&](const __bf16 *As, const __bf16 *Bs, int u, Frags<C> &f) __attribute__((always_inline)) {
        load_frags<C>(As, Bs, u, arow0, brow, lane, f);
      },
      koff, pre, post);
}

// Token of slab row p (slab rows fit in 32 bits), or -1 for a padding row.
__device__ __forceinline__ int64_t slab_row_token(const Slab &s, int p) {
  if (s.B == s.Bp) {  // no padding rows: no divide
    const int64_t t = s.tok0 + p;
    return p < s.nc * s.Bp && t < s.L ? t : -1;
  }
  const int j = p / s.Bp, i = p - j * s.Bp;
  if (i >= s.B || j >= s.nc) return -1;
  const int64_t t = s.tok0 + (int64_t)j * s.B + i;
  return t < s.L ? t : -1;
}

}  // namespace mfma
}  // namespace ipttt
