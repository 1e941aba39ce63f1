// Internal declarations shared by the host library (ipttt.cpp) and the kernel
// translation units. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ipttt.h"

namespace ipttt {

// Rows of a slab are chunk-padded: chunk j of the slab occupies rows
// [j*Bp, j*Bp + B) and rows [j*Bp + B, (j+1)*Bp) are zero padding, so every
// chunk starts on a 64-row boundary (one K step of the MFMA update).
constexpr int kChunkAlign = 64;

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Geometry of one slab of a prefill call.
struct Slab {
  int n_seq;        // sequences in the call
  int d, F, Kc;     // widths, conv taps
  int B, Bp;        // chunk, padded chunk pitch
  int nc;           // chunks in this slab
  int nc_cap;       // chunks the workspace is laid out for (row pitch = nc_cap*Bp)
  int G;            // chunks per group sharing one W snapshot (1: one per chunk)
  int ng_cap;       // groups the workspace is laid out for = ceil(nc_cap / G)
  int64_t Lp;       // padded rows per sequence in the workspace = nc_cap * Bp
  int64_t tok0;     // first token of the slab within each sequence
  int64_t L;        // tokens per sequence in the call
  int64_t x_seq_stride;  // elements between sequences in x / e / o (= L_total * d)
  float eta;
  int mse;
};

// Byte offsets of the workspace buffers (all 256-byte aligned).
struct WsLayout {
  size_t z, zt, c, vt, s, rt, p, total;
};

// Largest rows per chunk group (G * Bp) of the chunk-parallel scan.
constexpr int kMaxGroupRows = 4096;

// Size of the fixed per-device scratch area that ipttt_prefill_layer_noalloc
// uses as its workspace (scratch.hip).
constexpr size_t kScratchBytes = IPTTT_NOALLOC_SCRATCH_BYTES;
// Device address of the current device's scratch area (looked up on the first
// call per device, then cached); *out = nullptr on failure.
hipError_t scratch_setup(void **out);

// need_z: the token-major copy of Z (read by the generic apply only).
// G: chunks per group (bf16 MFMA path; 1 on the generic path).
WsLayout ws_layout(int elem, int n_seq, int d, int F, int Bp, int nc_cap, int G, int mse,
                   int need_z);

// Pointers into the workspace for one call.
struct WsPtrs {
  void *z;   // [n][Lp][F]      Z, token-major (generic path only)
  void *zt;  // [n][F][Lp]      Z transposed (token-contiguous)
  void *c;   // [n][Lp][d]      conv output
  void *vt;  // [n][d][Lp]      target V transposed; eta*V for the linear rule
  void *s;   // linear: [n][ng_cap][d][F] W snapshot per group; mse: [n][d][F]
  void *rt;  // mse: [n][d][Bp] eta*(V - O) of the current chunk, transposed
  void *p;   // G > 1: [n][ng_cap][G Bp][G Bp] block-causal Gram, P^T[s][m] = z_m . z_s
};

struct Weights {
  const void *w_gate, *w_up, *proj, *conv_w;
};

// ---- generic kernels (fp32 and bf16 storage, fp32 FMA) --------------------
template <typename T>
hipError_t gen_gateup(const Slab &s, const T *x, const Weights &w, const WsPtrs &ws,
                      hipStream_t st);
template <typename T>
hipError_t gen_conv(const Slab &s, const T *e, const Weights &w, const WsPtrs &ws,
                    hipStream_t st);
template <typename T>
hipError_t gen_proj(const Slab &s, const Weights &w, const WsPtrs &ws, hipStream_t st);
template <typename T>
hipError_t gen_snapshot(const Slab &s, const float *w_state, T *snap, int64_t snap_seq_stride,
                        hipStream_t st);
// W[c][f] += sum_t A[c][t] Zt[f][t] over one chunk j; optional snapshot of the new W.
template <typename T>
hipError_t gen_update(const Slab &s, int j, const T *a, int64_t a_ld, int64_t a_seq_stride,
                      const WsPtrs &ws, float *w_state, T *snap_out, int64_t snap_seq_stride,
                      hipStream_t st);
// O rows of chunks [j0, j0+nj) from snapshots; mse also writes rt (nj must be 1).
template <typename T>
hipError_t gen_apply(const Slab &s, int j0, int nj, const T *snap, int64_t snap_seq_stride,
                     int64_t snap_chunk_stride, const WsPtrs &ws, float *o, hipStream_t st);

// ---- decode (one token per sequence) -----------------------------------------
// z[b][f] = T(SiLU(x_b . W_g[f]) * (x_b . W_u[f])) for b < batch; x_b = x + b * x_stride.
template <typename T>
hipError_t dec_gateup(const T *x, int64_t x_stride, int batch, int d, int F, const T *wg,
                      const T *wu, T *z, hipStream_t st);
// o[b][c] = sum_f z[b][f] * T(W[b][c][f]) (W stored [batch][d][F] fp32).
template <typename T>
hipError_t dec_apply(const T *z, const float *w, int batch, int d, int F, float *o,
                     hipStream_t st);

// ---- MFMA kernels (bf16 storage, gfx950) ----------------------------------
bool mfma_supported(int d, int F);
hipError_t mf_gateup(const Slab &s, const __bf16 *x, const Weights &w, const WsPtrs &ws,
                     hipStream_t st);
hipError_t mf_conv(const Slab &s, const __bf16 *e, const Weights &w, const WsPtrs &ws,
                   hipStream_t st);
hipError_t mf_proj(const Slab &s, const Weights &w, const WsPtrs &ws, hipStream_t st);
// Linear rule: for each group q of G chunks of the slab, write snapshot
// S[q] = bf16(W) then W += sum over the group's tokens of z_t^T (eta v_t); W
// stays in registers across the slab. blocked: S in the layout of mf_snapshot
// (what mf_apply reads), else row-major [d][F] (what the backward reads).
hipError_t mf_update_scan(const Slab &s, const WsPtrs &ws, float *w_state, bool blocked,
                          hipStream_t st);
// G > 1: masked Gram of every group of the slab, P^T[s][m] = z_m . z_s when
// token s lies in an earlier chunk of the group than token m, else 0.
hipError_t mf_gram(const Slab &s, const WsPtrs &ws, hipStream_t st);
// S = bf16(W) in the blocked layout the MFMA apply reads (element (c, f) at
// ((f / 8) d + c) 8 + f % 8), every sequence of the slab: the MSE rule's first
// copy of a call.
hipError_t mf_snapshot(const Slab &s, const float *w_state, __bf16 *snap, int64_t snap_seq_stride,
                       hipStream_t st);
// MSE rule, one chunk j: W += Rt Zt_j^T-contract, snapshot S = bf16(new W) in
// the layout of mf_snapshot.
hipError_t mf_update_one(const Slab &s, int j, const WsPtrs &ws, float *w_state,
                         hipStream_t st);
// MSE rule over chunk groups (G > 1), group q: O = Z S for the group's rows (S:
// W at its first chunk) and Rt = eta (V - O)^T ([n][d][G Bp]) from them; then
// mf_mse_fix for its chunks jl = 1 .. in order (O += the Gram term over the
// earlier chunks' residuals, Rt of the chunk's rows), then mf_update_group
// (W += Zt Rt over the group's chunks, S = bf16(W)).
hipError_t mf_apply_mse_group(const Slab &s, int q, const WsPtrs &ws, float *o, hipStream_t st);
hipError_t mf_mse_fix(const Slab &s, int q, int jl, const WsPtrs &ws, float *o, hipStream_t st);
hipError_t mf_update_group(const Slab &s, int q, const WsPtrs &ws, float *w_state,
                           hipStream_t st);
// O rows of groups [q0, q0 + nq) (G = 1: chunks): O = Z S_q (S in the layout
// of mf_snapshot), plus P (eta V) when G > 1; the MSE rule (G = 1, nq = 1)
// also writes Rt.
hipError_t mf_apply(const Slab &s, int q0, int nq, const WsPtrs &ws, float *o,
                    hipStream_t st);

// Gate/up that also writes the pre-activations At = X W_g, Ut = X W_u
// ([n][F][Lp] bf16, padding rows 0), for the backward.
hipError_t mf_gateup_pre(const Slab &s, const __bf16 *x, const Weights &w, const WsPtrs &ws,
                         __bf16 *at, __bf16 *ut, hipStream_t st);
// Backward scan over all chunks of the slab, last to first: snap[n][j] =
// bf16(G) (G_{j+1}), then G += Zt_j . Bt_j; g is fp32 [n][d][F].
hipError_t mf_update_reverse(const Slab &s, const __bf16 *zt, const __bf16 *bt, float *g,
                             __bf16 *snap, hipStream_t st);

// One chunk j of the MSE rule with explicit buffers (the backward's recompute):
// apply with the snapshot at snap (+ n * snap_seq), writing only the residual
// eta (V - O) to rt + n * rt_seq + c * rt_ld + row (rt pre-offset to chunk j);
// and W += Zt_j . B_j with B = bsrc (+ n * b_seq, rows c at b_ld, pre-offset
// to chunk j), then snap_after = bf16(W) when non-null.
hipError_t mf_apply_mse_chunk(const Slab &s, int j, const __bf16 *zt, const __bf16 *snap,
                              int64_t snap_seq, const __bf16 *vt, __bf16 *rt, int64_t rt_seq,
                              int64_t rt_ld, hipStream_t st);
hipError_t mf_update_chunk(const Slab &s, int j, const __bf16 *zt, const __bf16 *bsrc,
                           int64_t b_ld, int64_t b_seq, float *w, __bf16 *snap_after,
                           int64_t snap_seq, hipStream_t st);
// Group q of the MSE rule with explicit buffers and row-major copies of W (the
// backward's recompute over chunk groups, s.G chunks each): the apply of the
// group's rows from snap (+ n * snap_seq, W at the group's first chunk),
// writing O (o + n * s.x_seq_stride, token rows) and Rt = eta (V - O)^T to rt
// ([n][d][G Bp], the group's rows), after which mf_mse_fix corrects chunks
// 1 .. of the group; then the group's update W += Zt . Rt with a row-major
// copy of W before each of its chunks at snap + j dF (j = 0 .. chunks - 1, the
// first one unchanged) and, when more chunks follow, the copy after its last
// chunk at the next slot.
hipError_t mf_apply_mse_group_rm(const Slab &s, int q, const __bf16 *zt, const __bf16 *snap,
                                 int64_t snap_seq, const __bf16 *vt, float *o, __bf16 *rt,
                                 hipStream_t st);
hipError_t mf_update_group_rm(const Slab &s, int q, const __bf16 *zt, const __bf16 *rt, float *w,
                              __bf16 *snap, int64_t snap_seq, hipStream_t st);

// ---- backward (bf16 MFMA path, one slab holding the whole sequence) -----------
struct BwBufs {
  const __bf16 *zt, *at, *ut;  // [n][F][Lp] Z, X W_g, X W_u (token-contiguous)
  const __bf16 *c, *vt;        // [n][Lp][d] conv output; [n][d][Lp] eta V
  const __bf16 *snap_w;        // [n][nc][d][F] W_j, the weight chunk j applied
  const __bf16 *snap_g;        // [n][nc][d][F] G_{j+1} = dL/dW_{j+1}
  const __bf16 *dot, *xt;      // [n][d][Lp] dO and X, transposed
  __bf16 *dat, *dut;           // [n][F][Lp] dA, dU (dut directly follows dat)
  __bf16 *dvt;                 // [n][d][Lp] dV
  __bf16 *dyt;                 // MSE: [n][d][Lp] dY = dO - eta Z G (gradient reaching Z W)
  const __bf16 *rt;            // MSE: [n][d][Lp] eta (V - O) of every chunk
  float *dc;                   // [n][Lp][d] dC
  float *part;                 // [conv runs][d][Kc] partial conv-weight gradients
  float *part2;                // [kConvSumGroups][d][Kc] their sums by row group
  float *dproj_part;           // [kDprojSplits][d][d] split-K partial dProj
};
constexpr int kConvSumGroups = 64;
constexpr int kConvBwRun = 16;  // slab rows per thread of the conv adjoint
constexpr int kDprojSplits = 8;
hipError_t bw_transpose_f32(const Slab &s, const float *in, __bf16 *out, hipStream_t st);
hipError_t bw_transpose_bf16(const Slab &s, const __bf16 *in, __bf16 *out, hipStream_t st);
// dZ = a0 W_j^T + a1 G_{j+1}^T: (dO, eta V) for the linear rule, (dY, eta (V - O)) for MSE
hipError_t bw_dz(const Slab &s, const BwBufs &b, const __bf16 *a0, const __bf16 *a1,
                 hipStream_t st);
// MSE rule, chunk j: dY_j, dV_j from P = Z_j G_{j+1}
hipError_t bw_mse_p(const Slab &s, int j, const BwBufs &b, hipStream_t st);
hipError_t bw_dv(const Slab &s, const BwBufs &b, hipStream_t st);
hipError_t bw_dc(const Slab &s, const BwBufs &b, const void *proj, hipStream_t st);
hipError_t bw_dx(const Slab &s, const BwBufs &b, const void *wg, const void *wu, float *dx,
                 hipStream_t st);
hipError_t bw_dw(const Slab &s, const BwBufs &b, float *dwg, float *dwu, hipStream_t st);
hipError_t bw_dproj(const Slab &s, const BwBufs &b, float *dproj, hipStream_t st);
int64_t bw_conv_runs(const Slab &s);
int bw_dproj_splits(const Slab &s);
hipError_t bw_conv(const Slab &s, const BwBufs &b, const __bf16 *e, const void *conv_w, float *de,
                   float *dconv, hipStream_t st);
hipError_t bw_sum_seq(const float *in, int n, int64_t len, float *out, hipStream_t st);
hipError_t bw_fill(float *p, int64_t n, float v, hipStream_t st);


}  // namespace ipttt
