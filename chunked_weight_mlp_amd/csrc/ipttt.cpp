// Host side of libipttt: argument validation, workspace planning and the
// chunk-scan launch sequence. Kernels live in kernels_*.hip.
//
// Linear rule, per slab of chunks (all sequences of the call at once), the
// chunks taken in groups of G (G = 1: plain chunk scan):
//   gate/up -> Z, Zt;  conv -> C;  proj -> Vt = eta * V
//   update scan: snapshot S_q = W before group q, then W += eta Z_q^T V_q
//   Gram (G > 1): P_q = block-causal Z_q Z_q^T (token s of an earlier chunk
//   of the group than token t, else 0)
//   apply (batched over groups): O_q = Z_q S_q + P_q (eta V_q)
// The update of one W tile never needs another tile, and the apply of group q
// needs only S_q and the group's own Z and V, so applying every group after
// the scan is the same computation as applying each chunk before its update:
// for chunk k of group q, W_k = S_q + eta sum over the group's earlier chunks
// of Z_j^T V_j, and Z_k W_k expands to the two terms above.
// MSE rule, per chunk: apply with S = W (current) -> O_j and Rt = eta (V - O_j);
// update W += Z_j^T Rt and refresh S.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

struct ipttt_layer {
  ipttt_layer_desc desc;
  std::vector<uint8_t> was_reset;
  bool mfma;
  // per-kernel timing (ipttt_profile_begin / _end); no_events: the current call
  // must not create or record events (the allocation-free entry point)
  bool prof = false;
  bool no_events = false;
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> spare;
  std::vector<hipEvent_t> all_events;
};

namespace {

thread_local std::string g_last_error;

ipttt_status fail(ipttt_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(ipttt_status_str(s)) + ": " + buf;
  return s;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int elem_size(ipttt_dtype t) { return t == IPTTT_BF16 ? 2 : 4; }

ipttt_status check_sizes(const ipttt_layer_desc *d) {
  if (!d) return fail(IPTTT_E_INVALID, "descriptor is NULL");
  if (d->d <= 0 || d->d_ff <= 0) return fail(IPTTT_E_INVALID, "d=%d d_ff=%d must be > 0", d->d, d->d_ff);
  if (d->d > (1 << 16) || d->d_ff > (1 << 18))
    return fail(IPTTT_E_UNSUPPORTED, "d=%d d_ff=%d exceed 65536 / 262144", d->d, d->d_ff);
  if (d->chunk <= 0) return fail(IPTTT_E_INVALID, "chunk=%d must be > 0", d->chunk);
  if (d->chunk > (1 << 16)) return fail(IPTTT_E_UNSUPPORTED, "chunk=%d exceeds 65536", d->chunk);
  if (d->conv_k <= 0) return fail(IPTTT_E_INVALID, "conv_k=%d must be > 0", d->conv_k);
  if (d->conv_k > 8) return fail(IPTTT_E_UNSUPPORTED, "conv_k=%d exceeds 8", d->conv_k);
  if (d->max_batch <= 0) return fail(IPTTT_E_INVALID, "max_batch=%d must be > 0", d->max_batch);
  if (d->in_dtype != IPTTT_F32 && d->in_dtype != IPTTT_BF16)
    return fail(IPTTT_E_UNSUPPORTED, "in_dtype=%d", (int)d->in_dtype);
  if (d->update != IPTTT_UPDATE_LINEAR && d->update != IPTTT_UPDATE_MSE)
    return fail(IPTTT_E_UNSUPPORTED, "update=%d", (int)d->update);
  if (!(d->eta == d->eta) || d->eta > 3.0e38f || d->eta < -3.0e38f)
    return fail(IPTTT_E_INVALID, "eta is not finite");
  if (d->flags & ~IPTTT_FLAG_GENERIC_KERNELS) return fail(IPTTT_E_INVALID, "unknown flags 0x%x", d->flags);
  if (d->group_chunks < 0) return fail(IPTTT_E_INVALID, "group_chunks=%d must be >= 0", d->group_chunks);
  if ((int64_t)d->group_chunks * ipttt::round_up(d->chunk, ipttt::kChunkAlign) > ipttt::kMaxGroupRows)
    return fail(IPTTT_E_UNSUPPORTED, "group_chunks=%d: %d chunk-padded rows per group exceed %d",
                d->group_chunks,
                (int)(d->group_chunks * ipttt::round_up(d->chunk, ipttt::kChunkAlign)),
                ipttt::kMaxGroupRows);
  return IPTTT_OK;
}

int chunk_pitch(int B) { return (int)ipttt::round_up(B, ipttt::kChunkAlign); }

bool use_mfma(const ipttt_layer_desc *d) {
  return d->in_dtype == IPTTT_BF16 && !(d->flags & IPTTT_FLAG_GENERIC_KERNELS) &&
         ipttt::mfma_supported(d->d, d->d_ff);
}

// Chunk-padded rows per group when the descriptor leaves the choice to the
// library: enough to give the apply full-height tiles and cut the W snapshots
// to one per 1024 rows.
constexpr int kDefaultGroupRows = 1024;

// The MSE rule's default: its groups trade the Gram term (a cost growing with
// the group) against streaming W through HBM once per group.
constexpr int kDefaultMseGroupRows = 2048;

// Chunks per group of the chunk-parallel scan (bf16 MFMA path); 1 elsewhere.
// A slab of n chunks uses min(G, n).
int group_chunks(const ipttt_layer_desc *d) {
  if (!use_mfma(d)) return 1;
  if (d->group_chunks > 0) return d->group_chunks;
  const int rows = d->update == IPTTT_UPDATE_MSE ? kDefaultMseGroupRows : kDefaultGroupRows;
  return std::max(1, rows / chunk_pitch(d->chunk));
}

ipttt_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return IPTTT_OK;
  return fail(IPTTT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TRY_HIP(expr, what)                                    \
  do {                                                         \
    ipttt_status _s = hip_status((expr), (what));              \
    if (_s != IPTTT_OK) return _s;                             \
  } while (0)

// Records an event pair around one launch when the handle is profiling.
struct ProfScope {
  ipttt_layer *h;
  int kind;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  static hipEvent_t take(ipttt_layer *h) {
    if (!h->spare.empty()) {
      hipEvent_t e = h->spare.back();
      h->spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    h->all_events.push_back(e);
    return e;
  }
  ProfScope(ipttt_layer *h_, int kind_, hipStream_t st_) : h(h_), kind(kind_), st(st_) {
    if (!h->prof || h->no_events) return;
    a = take(h);
    b = take(h);
    if (a && b) (void)hipEventRecord(a, st);  // best effort: a failed record shows as a zero time
  }
  ~ProfScope() {
    if (!h->prof || h->no_events || !a || !b) return;
    (void)hipEventRecord(b, st);
    h->recs.push_back({kind, a, b});
  }
};

#define LAUNCH(kind, expr, what)                                   \
  do {                                                             \
    ProfScope _ps(h, (kind), st);                                  \
    TRY_HIP((expr), (what));                                       \
  } while (0)

}  // namespace

namespace ipttt {

WsLayout ws_layout(int elem, int n_seq, int d, int F, int Bp, int nc_cap, int G, int mse,
                   int need_z) {
  WsLayout w{};
  const size_t Lp = (size_t)nc_cap * Bp;
  const size_t ng = (size_t)(nc_cap + G - 1) / G, RG = (size_t)G * Bp;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  w.z = take(need_z ? (size_t)n_seq * Lp * F * elem : 0);
  w.zt = take((size_t)n_seq * F * Lp * elem);
  w.c = take((size_t)n_seq * Lp * d * elem);
  w.vt = take((size_t)n_seq * d * Lp * elem);
  w.s = take((size_t)n_seq * (mse ? 1 : ng) * d * F * elem);
  w.rt = mse ? take((size_t)n_seq * d * RG * elem) : off;
  w.p = G > 1 ? take((size_t)n_seq * ng * RG * RG * elem) : off;
  w.total = off;
  return w;
}

}  // namespace ipttt

extern "C" {

const char *ipttt_status_str(ipttt_status s) {
  switch (s) {
    case IPTTT_OK: return "IPTTT_OK";
    case IPTTT_E_INVALID: return "IPTTT_E_INVALID";
    case IPTTT_E_UNSUPPORTED: return "IPTTT_E_UNSUPPORTED";
    case IPTTT_E_HIP: return "IPTTT_E_HIP";
    case IPTTT_E_STATE: return "IPTTT_E_STATE";
    case IPTTT_E_WORKSPACE: return "IPTTT_E_WORKSPACE";
  }
  return "IPTTT_E_UNKNOWN";
}

const char *ipttt_last_error(void) { return g_last_error.c_str(); }

size_t ipttt_workspace_bytes(const ipttt_layer_desc *desc, int32_t batch, int32_t slab_chunks) {
  std::string saved = g_last_error;
  ipttt_status s = check_sizes(desc);
  g_last_error = saved;
  if (s != IPTTT_OK || batch < 1 || slab_chunks < 1) return 0;
  return ipttt::ws_layout(elem_size(desc->in_dtype), batch, desc->d, desc->d_ff,
                          chunk_pitch(desc->chunk), slab_chunks,
                          std::min(group_chunks(desc), (int)slab_chunks),
                          desc->update == IPTTT_UPDATE_MSE, !use_mfma(desc))
      .total;
}

ipttt_status ipttt_init(const ipttt_layer_desc *desc, ipttt_layer **out) {
  if (!out) return fail(IPTTT_E_INVALID, "out is NULL");
  *out = nullptr;
  ipttt_status s = check_sizes(desc);
  if (s != IPTTT_OK) return s;
  const void *ptrs[] = {desc->w_gate, desc->w_up, desc->proj, desc->conv_w, desc->w0,
                        desc->w_state, desc->workspace};
  const char *names[] = {"w_gate", "w_up", "proj", "conv_w", "w0", "w_state", "workspace"};
  for (int i = 0; i < 7; ++i) {
    if (!ptrs[i]) return fail(IPTTT_E_INVALID, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(IPTTT_E_INVALID, "%s is not 16-byte aligned", names[i]);
  }
  if (((uintptr_t)desc->workspace & 255u) != 0)
    return fail(IPTTT_E_INVALID, "workspace is not 256-byte aligned");
  if (desc->workspace_bytes < ipttt_workspace_bytes(desc, 1, 1))
    return fail(IPTTT_E_WORKSPACE, "workspace_bytes=%zu below the %zu bytes of one chunk of one sequence",
                desc->workspace_bytes, ipttt_workspace_bytes(desc, 1, 1));
  ipttt_layer *h = new (std::nothrow) ipttt_layer;
  if (!h) return fail(IPTTT_E_INVALID, "out of host memory");
  h->desc = *desc;
  h->was_reset.assign((size_t)desc->max_batch, 0);
  h->mfma = use_mfma(desc);
  // set-up of the allocation-free prefill's scratch area on the current device;
  // a failure here (no device yet) is retried, and reported, by that entry point
  void *scr = nullptr;
  (void)ipttt::scratch_setup(&scr);
  *out = h;
  return IPTTT_OK;
}

void ipttt_destroy(ipttt_layer *h) {
  if (!h) return;
  for (hipEvent_t e : h->all_events) (void)hipEventDestroy(e);
  delete h;
}

ipttt_status ipttt_profile_begin(ipttt_layer *h) {
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  for (auto &r : h->recs) {
    h->spare.push_back(r.a);
    h->spare.push_back(r.b);
  }
  h->recs.clear();
  h->prof = true;
  return IPTTT_OK;
}

ipttt_status ipttt_profile_end(ipttt_layer *h, int32_t *launches, double *ms) {
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  if (!launches || !ms) return fail(IPTTT_E_INVALID, "launches and ms must be non-NULL");
  for (int k = 0; k < IPTTT_K_COUNT; ++k) {
    launches[k] = 0;
    ms[k] = 0.0;
  }
  h->prof = false;
  ipttt_status st = IPTTT_OK;
  for (auto &r : h->recs) {
    float t = 0.f;
    if (st == IPTTT_OK) {
      st = hip_status(hipEventSynchronize(r.b), "event synchronize");
      if (st == IPTTT_OK) st = hip_status(hipEventElapsedTime(&t, r.a, r.b), "event elapsed time");
    }
    launches[r.kind] += 1;
    ms[r.kind] += t;
    h->spare.push_back(r.a);
    h->spare.push_back(r.b);
  }
  h->recs.clear();
  return st;
}

ipttt_status ipttt_reset_fast_weights(ipttt_layer *h, int32_t first_seq, int32_t n_seq,
                                      void *hip_stream) {
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  const ipttt_layer_desc &d = h->desc;
  if (first_seq < 0 || n_seq < 0 || (int64_t)first_seq + n_seq > d.max_batch)
    return fail(IPTTT_E_INVALID, "sequences [%d, %d) outside [0, %d)", first_seq, first_seq + n_seq,
                d.max_batch);
  const size_t bytes = (size_t)d.d * d.d_ff * sizeof(float);
  hipStream_t st = (hipStream_t)hip_stream;
  for (int32_t i = 0; i < n_seq; ++i)
    TRY_HIP(hipMemcpyAsync(d.w_state + (size_t)(first_seq + i) * d.d * d.d_ff, d.w0, bytes,
                           hipMemcpyDeviceToDevice, st),
            "reset copy");
  for (int32_t i = 0; i < n_seq; ++i) h->was_reset[(size_t)(first_seq + i)] = 1;
  return IPTTT_OK;
}

}  // extern "C"

namespace {

// Runs the scan over `L` tokens of `n_seq` sequences whose state slots start
// at `slot0`. x / e / o point at token 0 of the first sequence; sequences are
// `seq_stride` elements apart. o == nullptr runs the updates only (the
// outputs of those tokens were produced elsewhere, e.g. token by token).
template <typename T>
ipttt_status run_scan(ipttt_layer *h, const T *x, const T *e, float *o, int slot0, int n_seq,
                      int64_t L, int64_t seq_stride, void *ws_base, size_t ws_bytes,
                      hipStream_t st) {
  using namespace ipttt;
  const ipttt_layer_desc &d = h->desc;
  const int elem = (int)sizeof(T);
  const int mse = d.update == IPTTT_UPDATE_MSE;
  const int B = d.chunk, Bp = chunk_pitch(B);
  const int64_t K = (L + B - 1) / B;
  const int G_max = group_chunks(&d);
  // workspace of a slab of n chunks (its groups hold min(G_max, n) chunks);
  // non-decreasing in n, so the largest slab that fits is found by bisection
  auto layout = [&](int64_t n) {
    return ws_layout(elem, n_seq, d.d, d.d_ff, Bp, (int)n, (int)std::min<int64_t>(G_max, n), mse,
                     !h->mfma);
  };
  // slab rows are indexed in 32 bits on the device
  int64_t lo = 1, hi = std::min<int64_t>(K, ((int64_t)1 << 30) / Bp);
  if (layout(1).total > ws_bytes)
    return fail(IPTTT_E_WORKSPACE, "workspace of %zu bytes cannot hold one chunk of %d sequences (%zu)",
                ws_bytes, n_seq, layout(1).total);
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (layout(mid).total <= ws_bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int G = (int)std::min<int64_t>(G_max, lo);
  // slabs of whole groups unless one slab covers the call
  const int nc_cap = (int)(lo < K ? lo / G * G : lo);
  const WsLayout lay = ws_layout(elem, n_seq, d.d, d.d_ff, Bp, nc_cap, G, mse, !h->mfma);
  char *base = (char *)ws_base;
  WsPtrs ws{base + lay.z,  base + lay.zt, base + lay.c, base + lay.vt,
            base + lay.s,  base + lay.rt, base + lay.p};
  Weights w{d.w_gate, d.w_up, d.proj, d.conv_w};
  float *wst = d.w_state + (size_t)slot0 * d.d * d.d_ff;
  const int64_t dF = (int64_t)d.d * d.d_ff;
  const int64_t snap_seq_stride = mse ? dF : (int64_t)nc_cap * dF;

  for (int64_t k0 = 0; k0 < K; k0 += nc_cap) {
    Slab s{};
    s.n_seq = n_seq;
    s.d = d.d;
    s.F = d.d_ff;
    s.Kc = d.conv_k;
    s.B = B;
    s.Bp = Bp;
    s.nc = (int)std::min<int64_t>(nc_cap, K - k0);
    s.nc_cap = nc_cap;
    s.G = G;
    s.ng_cap = (nc_cap + G - 1) / G;
    s.Lp = (int64_t)nc_cap * Bp;
    s.tok0 = k0 * B;
    s.L = L;
    s.x_seq_stride = seq_stride;
    s.eta = d.eta;
    s.mse = mse;
    if (h->mfma) {
      LAUNCH(IPTTT_K_GATEUP, mf_gateup(s, (const __bf16 *)x, w, ws, st), "gate/up launch");
      LAUNCH(IPTTT_K_CONV, mf_conv(s, (const __bf16 *)e, w, ws, st), "conv launch");
      LAUNCH(IPTTT_K_PROJ, mf_proj(s, w, ws, st), "proj launch");
      if (!mse) {
        LAUNCH(IPTTT_K_UPDATE, mf_update_scan(s, ws, wst, true, st), "update scan launch");
        if (o) {
          if (G > 1) LAUNCH(IPTTT_K_GRAM, mf_gram(s, ws, st), "Gram launch");
          LAUNCH(IPTTT_K_APPLY, mf_apply(s, 0, (s.nc + G - 1) / G, ws, o, st), "apply launch");
        }
      } else {
        if (k0 == 0)
          LAUNCH(IPTTT_K_SNAPSHOT, mf_snapshot(s, wst, (__bf16 *)ws.s, snap_seq_stride, st),
                 "snapshot launch");
        if (G > 1 && o) {
          // chunk groups: one apply, the chunks' Gram corrections in order, one update
          LAUNCH(IPTTT_K_GRAM, mf_gram(s, ws, st), "Gram launch");
          for (int q = 0; q * G < s.nc; ++q) {
            LAUNCH(IPTTT_K_APPLY, mf_apply_mse_group(s, q, ws, o, st), "apply launch");
            for (int jl = 1; jl < G && q * G + jl < s.nc; ++jl)
              LAUNCH(IPTTT_K_MSE_FIX, mf_mse_fix(s, q, jl, ws, o, st), "MSE correction launch");
            LAUNCH(IPTTT_K_UPDATE, mf_update_group(s, q, ws, wst, st), "update launch");
          }
        } else {
          // chunk by chunk (also when only the updates are wanted: the groups'
          // corrections need the outputs)
          s.G = 1;
          s.ng_cap = nc_cap;
          for (int j = 0; j < s.nc; ++j) {
            LAUNCH(IPTTT_K_APPLY, mf_apply(s, j, 1, ws, o, st), "apply launch");
            LAUNCH(IPTTT_K_UPDATE, mf_update_one(s, j, ws, wst, st), "update launch");
          }
        }
      }
    } else {
      LAUNCH(IPTTT_K_GATEUP, gen_gateup<T>(s, x, w, ws, st), "gate/up launch");
      LAUNCH(IPTTT_K_CONV, gen_conv<T>(s, e, w, ws, st), "conv launch");
      LAUNCH(IPTTT_K_PROJ, gen_proj<T>(s, w, ws, st), "proj launch");
      T *S = (T *)ws.s;
      if (!mse) {
        LAUNCH(IPTTT_K_SNAPSHOT, gen_snapshot<T>(s, wst, S, snap_seq_stride, st), "snapshot launch");
        for (int j = 0; j < s.nc; ++j) {
          T *next = (j + 1 < s.nc) ? S + (int64_t)(j + 1) * dF : nullptr;
          LAUNCH(IPTTT_K_UPDATE,
                 gen_update<T>(s, j, (const T *)ws.vt + (int64_t)j * Bp, s.Lp,
                               (int64_t)d.d * s.Lp, ws, wst, next, snap_seq_stride, st),
                 "update launch");
        }
        if (o) LAUNCH(IPTTT_K_APPLY, gen_apply<T>(s, 0, s.nc, S, snap_seq_stride, dF, ws, o, st), "apply launch");
      } else {
        if (k0 == 0) LAUNCH(IPTTT_K_SNAPSHOT, gen_snapshot<T>(s, wst, S, snap_seq_stride, st), "snapshot launch");
        for (int j = 0; j < s.nc; ++j) {
          LAUNCH(IPTTT_K_APPLY, gen_apply<T>(s, j, 1, S, snap_seq_stride, 0, ws, o, st), "apply launch");
          LAUNCH(IPTTT_K_UPDATE,
                 gen_update<T>(s, j, (const T *)ws.rt, Bp, (int64_t)d.d * Bp, ws, wst, S,
                               snap_seq_stride, st),
                 "update launch");
        }
      }
    }
  }
  return IPTTT_OK;
}

ipttt_status check_call(ipttt_layer *h, const void *x, const void *e, const float *o) {
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  if (!x || !e || !o) return fail(IPTTT_E_INVALID, "x, e and o must be non-NULL");
  // the MFMA path moves x and e in 16-byte vectors
  const size_t align = h->mfma ? 16 : (size_t)elem_size(h->desc.in_dtype);
  if (((uintptr_t)x % align) || ((uintptr_t)e % align) || ((uintptr_t)o % 4))
    return fail(IPTTT_E_INVALID, "x / e must be %zu-byte aligned and o 4-byte aligned", align);
  return IPTTT_OK;
}

// ws_base == nullptr: the descriptor's workspace
ipttt_status dispatch(ipttt_layer *h, const void *x, const void *e, float *o, int slot0, int n_seq,
                      int64_t L, int64_t seq_stride, hipStream_t st, void *ws_base = nullptr,
                      size_t ws_bytes = 0) {
  if (!ws_base) {
    ws_base = h->desc.workspace;
    ws_bytes = h->desc.workspace_bytes;
  }
  if (h->desc.in_dtype == IPTTT_BF16)
    return run_scan<__bf16>(h, (const __bf16 *)x, (const __bf16 *)e, o, slot0, n_seq, L, seq_stride,
                            ws_base, ws_bytes, st);
  return run_scan<float>(h, (const float *)x, (const float *)e, o, slot0, n_seq, L, seq_stride,
                         ws_base, ws_bytes, st);
}

// The checks every prefill entry point makes before any device work.
ipttt_status check_prefill(ipttt_layer *h, const void *x, const void *e, const float *o,
                           int32_t batch, int64_t seq_len) {
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  if (batch < 0 || seq_len < 0)
    return fail(IPTTT_E_INVALID, "batch=%d seq_len=%lld must be >= 0", batch, (long long)seq_len);
  if (batch > h->desc.max_batch)
    return fail(IPTTT_E_INVALID, "batch=%d exceeds max_batch=%d", batch, h->desc.max_batch);
  if (batch == 0 || seq_len == 0) return IPTTT_OK;
  ipttt_status s = check_call(h, x, e, o);
  if (s != IPTTT_OK) return s;
  if (seq_len > ((int64_t)1 << 40) / h->desc.d) return fail(IPTTT_E_UNSUPPORTED, "seq_len too large");
  for (int32_t i = 0; i < batch; ++i)
    if (!h->was_reset[(size_t)i]) return fail(IPTTT_E_STATE, "sequence %d was never reset", i);
  return IPTTT_OK;
}

// ---- backward ---------------------------------------------------------------

bool bw_supported(const ipttt_layer_desc *d) { return use_mfma(d); }

struct BwLayout {
  size_t zt, at, ut, c, vt, wscr, gscr, snap_w, snap_g, dot, xt, dat, dut, dvt, dc, part, part2,
      dproj_part, dyt, rt, p, oscr, rtg, total;
  int G;  // chunks per group of the MSE recompute (1: chunk by chunk)
};

// Workspace of the backward: the whole sequence in one slab of K chunks.
BwLayout bw_layout(const ipttt_layer_desc &d, int n, int64_t L) {
  BwLayout w{};
  const size_t Bp = (size_t)chunk_pitch(d.chunk), K = (size_t)((L + d.chunk - 1) / d.chunk);
  const size_t Lp = K * Bp, F = (size_t)d.d_ff, D = (size_t)d.d, N = (size_t)n;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (size_t)ipttt::round_up((int64_t)bytes, 256);
    return o;
  };
  w.zt = take(N * F * Lp * 2);
  w.at = take(N * F * Lp * 2);
  w.ut = take(N * F * Lp * 2);
  w.c = take(N * Lp * D * 2);
  w.vt = take(N * D * Lp * 2);
  w.wscr = take(N * D * F * 4);
  w.gscr = take(N * D * F * 4);
  w.snap_w = take(N * K * D * F * 2);
  w.snap_g = take(N * K * D * F * 2);
  w.dot = take(N * D * Lp * 2);
  w.xt = take(N * D * Lp * 2);
  w.dat = take(N * F * Lp * 2);
  w.dut = take(N * F * Lp * 2);
  w.dvt = take(N * D * Lp * 2);
  w.dc = take(N * Lp * D * 4);
  w.part = take(N * K * (Bp / ipttt::kConvBwRun) * D * (size_t)d.conv_k * 4);
  w.part2 = take((size_t)ipttt::kConvSumGroups * D * (size_t)d.conv_k * 4);
  w.dproj_part = take((size_t)ipttt::kDprojSplits * D * D * 4);
  const bool mse = d.update == IPTTT_UPDATE_MSE;
  w.dyt = take(mse ? N * D * Lp * 2 : 0);
  w.rt = take(mse ? N * D * Lp * 2 : 0);
  // the MSE recompute over chunk groups: block-causal Gram, O of every token,
  // the current group's residuals
  w.G = mse ? (int)std::min<size_t>((size_t)group_chunks(&d), K) : 1;
  const size_t G = (size_t)w.G, ng = (K + G - 1) / G, RG = G * Bp;
  w.p = take(w.G > 1 ? N * ng * RG * RG * 2 : 0);
  w.oscr = take(w.G > 1 ? N * (size_t)L * D * 4 : 0);
  w.rtg = take(w.G > 1 ? N * D * RG * 2 : 0);
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

ipttt_status ipttt_prefill_layer(ipttt_layer *h, const void *x, const void *e, float *o,
                                 int32_t batch, int64_t seq_len, void *hip_stream) {
  ipttt_status s = check_prefill(h, x, e, o, batch, seq_len);
  if (s != IPTTT_OK || batch == 0 || seq_len == 0) return s;
  return dispatch(h, x, e, o, 0, batch, seq_len, seq_len * h->desc.d, (hipStream_t)hip_stream);
}

ipttt_status ipttt_prefill_layer_noalloc(ipttt_layer *h, const void *x, const void *e, float *o,
                                         int32_t batch, int64_t seq_len, void *hip_stream) {
  ipttt_status s = check_prefill(h, x, e, o, batch, seq_len);
  if (s != IPTTT_OK || batch == 0 || seq_len == 0) return s;
  const ipttt_layer_desc &d = h->desc;
  const int mse = d.update == IPTTT_UPDATE_MSE;
  const size_t one = ipttt::ws_layout(elem_size(d.in_dtype), batch, d.d, d.d_ff,
                                      chunk_pitch(d.chunk), 1, 1, mse, !h->mfma)
                         .total;
  if (one > ipttt::kScratchBytes)
    return fail(IPTTT_E_WORKSPACE,
                "one chunk of %d sequences needs %zu bytes of workspace, above the fixed %zu-byte "
                "scratch area of the allocation-free prefill",
                batch, one, ipttt::kScratchBytes);
  void *scr = nullptr;
  TRY_HIP(ipttt::scratch_setup(&scr), "scratch area lookup");
  h->no_events = true;
  s = dispatch(h, x, e, o, 0, batch, seq_len, seq_len * d.d, (hipStream_t)hip_stream, scr,
               ipttt::kScratchBytes);
  h->no_events = false;
  return s;
}

ipttt_status ipttt_decode_step(ipttt_layer *h, const void *x, const void *e, int64_t seq_stride,
                               int32_t pos, float *o, int32_t batch, void *hip_stream) {
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  const ipttt_layer_desc &d = h->desc;
  if (batch < 0 || batch > d.max_batch)
    return fail(IPTTT_E_INVALID, "batch=%d outside [0, %d]", batch, d.max_batch);
  if (pos < 0 || pos >= d.chunk)
    return fail(IPTTT_E_INVALID, "pos=%d outside [0, chunk=%d)", pos, d.chunk);
  if (batch == 0) return IPTTT_OK;
  ipttt_status s = check_call(h, x, e, o);
  if (s != IPTTT_OK) return s;
  if (batch > 1 && seq_stride < (int64_t)(pos + 1) * d.d)
    return fail(IPTTT_E_INVALID, "seq_stride=%lld shorter than the %d rows of the chunk so far",
                (long long)seq_stride, pos + 1);
  if (seq_stride % 8) return fail(IPTTT_E_INVALID, "seq_stride must be a multiple of 8 elements");
  for (int32_t i = 0; i < batch; ++i)
    if (!h->was_reset[(size_t)i]) return fail(IPTTT_E_STATE, "sequence %d was never reset", i);
  const size_t el = (size_t)elem_size(d.in_dtype);
  if ((size_t)batch * d.d_ff * el > d.workspace_bytes)
    return fail(IPTTT_E_WORKSPACE, "workspace too small for %d decode activations", batch);
  hipStream_t st = (hipStream_t)hip_stream;
  const char *xt = (const char *)x + (size_t)pos * d.d * el;
  if (d.in_dtype == IPTTT_BF16) {
    __bf16 *z = (__bf16 *)d.workspace;
    LAUNCH(IPTTT_K_GATEUP,
           ipttt::dec_gateup<__bf16>((const __bf16 *)xt, seq_stride, batch, d.d, d.d_ff,
                                     (const __bf16 *)d.w_gate, (const __bf16 *)d.w_up, z, st),
           "decode gate/up launch");
    LAUNCH(IPTTT_K_APPLY, ipttt::dec_apply<__bf16>(z, d.w_state, batch, d.d, d.d_ff, o, st),
           "decode apply launch");
  } else {
    float *z = (float *)d.workspace;
    LAUNCH(IPTTT_K_GATEUP,
           ipttt::dec_gateup<float>((const float *)xt, seq_stride, batch, d.d, d.d_ff,
                                    (const float *)d.w_gate, (const float *)d.w_up, z, st),
           "decode gate/up launch");
    LAUNCH(IPTTT_K_APPLY, ipttt::dec_apply<float>(z, d.w_state, batch, d.d, d.d_ff, o, st),
           "decode apply launch");
  }
  if (pos + 1 == d.chunk)  // chunk complete: its update, as prefill would run it
    return dispatch(h, x, e, nullptr, 0, batch, d.chunk, seq_stride, st);
  return IPTTT_OK;
}

size_t ipttt_backward_workspace_bytes(const ipttt_layer_desc *desc, int32_t batch,
                                      int64_t seq_len) {
  std::string saved = g_last_error;
  ipttt_status s = check_sizes(desc);
  g_last_error = saved;
  if (s != IPTTT_OK || batch < 1 || seq_len < 1 || !bw_supported(desc)) return 0;
  if ((seq_len + desc->chunk - 1) / desc->chunk * chunk_pitch(desc->chunk) > ((int64_t)1 << 30))
    return 0;
  return bw_layout(*desc, batch, seq_len).total;
}

ipttt_status ipttt_backward_layer(ipttt_layer *h, const void *x, const void *e, const float *d_o,
                                  const float *d_wfinal, int32_t batch, int64_t seq_len,
                                  const ipttt_grads *grads, void *workspace,
                                  size_t workspace_bytes, void *hip_stream) {
  using namespace ipttt;
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  const ipttt_layer_desc &d = h->desc;
  if (!bw_supported(&d))
    return fail(IPTTT_E_UNSUPPORTED, "backward runs on bf16 MFMA layers");
  if (batch < 1 || seq_len < 1)
    return fail(IPTTT_E_INVALID, "batch=%d seq_len=%lld must be >= 1", batch, (long long)seq_len);
  if (batch > d.max_batch)
    return fail(IPTTT_E_INVALID, "batch=%d exceeds max_batch=%d", batch, d.max_batch);
  ipttt_status s = check_call(h, x, e, d_o);
  if (s != IPTTT_OK) return s;
  if (!grads) return fail(IPTTT_E_INVALID, "grads is NULL");
  float *outs[] = {grads->dx, grads->de, grads->dw_gate, grads->dw_up, grads->dproj,
                   grads->dconv_w, grads->dw0};
  const char *onames[] = {"dx", "de", "dw_gate", "dw_up", "dproj", "dconv_w", "dw0"};
  for (int i = 0; i < 7; ++i)
    if (!outs[i] || ((uintptr_t)outs[i] & 3u))
      return fail(IPTTT_E_INVALID, "grads->%s is NULL or not 4-byte aligned", onames[i]);
  if (d_wfinal && ((uintptr_t)d_wfinal & 3u))
    return fail(IPTTT_E_INVALID, "d_wfinal is not 4-byte aligned");
  const int B = d.chunk, Bp = chunk_pitch(B);
  const int64_t K = (seq_len + B - 1) / B;
  if (K * Bp > ((int64_t)1 << 30)) return fail(IPTTT_E_UNSUPPORTED, "seq_len too large");
  if (!workspace || ((uintptr_t)workspace & 255u))
    return fail(IPTTT_E_INVALID, "workspace is NULL or not 256-byte aligned");
  const BwLayout lay = bw_layout(d, batch, seq_len);
  if (workspace_bytes < lay.total)
    return fail(IPTTT_E_WORKSPACE, "workspace_bytes=%zu below the %zu bytes this backward needs",
                workspace_bytes, lay.total);

  hipStream_t st = (hipStream_t)hip_stream;
  char *base = (char *)workspace;
  Slab sl{};
  sl.n_seq = batch;
  sl.d = d.d;
  sl.F = d.d_ff;
  sl.Kc = d.conv_k;
  sl.B = B;
  sl.Bp = Bp;
  sl.nc = (int)K;
  sl.nc_cap = (int)K;
  sl.G = 1;
  sl.ng_cap = (int)K;
  sl.Lp = K * Bp;
  sl.tok0 = 0;
  sl.L = seq_len;
  sl.x_seq_stride = seq_len * d.d;
  sl.eta = d.eta;
  const bool mse = d.update == IPTTT_UPDATE_MSE;
  sl.mse = mse ? 1 : 0;
  WsPtrs ws{nullptr, base + lay.zt, base + lay.c, base + lay.vt, base + lay.snap_w, nullptr, nullptr};
  Weights w{d.w_gate, d.w_up, d.proj, d.conv_w};
  BwBufs bb{};
  bb.zt = (const __bf16 *)(base + lay.zt);
  bb.at = (const __bf16 *)(base + lay.at);
  bb.ut = (const __bf16 *)(base + lay.ut);
  bb.c = (const __bf16 *)(base + lay.c);
  bb.vt = (const __bf16 *)(base + lay.vt);
  bb.snap_w = (const __bf16 *)(base + lay.snap_w);
  bb.snap_g = (const __bf16 *)(base + lay.snap_g);
  bb.dot = (const __bf16 *)(base + lay.dot);
  bb.xt = (const __bf16 *)(base + lay.xt);
  bb.dat = (__bf16 *)(base + lay.dat);
  bb.dut = (__bf16 *)(base + lay.dut);
  bb.dvt = (__bf16 *)(base + lay.dvt);
  bb.dc = (float *)(base + lay.dc);
  bb.part = (float *)(base + lay.part);
  bb.part2 = (float *)(base + lay.part2);
  bb.dproj_part = (float *)(base + lay.dproj_part);
  bb.dyt = (__bf16 *)(base + lay.dyt);
  bb.rt = (const __bf16 *)(base + lay.rt);
  float *wscr = (float *)(base + lay.wscr), *gscr = (float *)(base + lay.gscr);
  const size_t dF = (size_t)d.d * d.d_ff;

  // forward recompute from w0: Z with its pre-activations, eta V, W_j per chunk
  for (int32_t i = 0; i < batch; ++i)
    TRY_HIP(hipMemcpyAsync(wscr + i * dF, d.w0, dF * sizeof(float), hipMemcpyDeviceToDevice, st),
            "w0 copy");
  LAUNCH(IPTTT_K_GATEUP,
         mf_gateup_pre(sl, (const __bf16 *)x, w, ws, (__bf16 *)(base + lay.at),
                       (__bf16 *)(base + lay.ut), st),
         "gate/up launch");
  LAUNCH(IPTTT_K_CONV, mf_conv(sl, (const __bf16 *)e, w, ws, st), "conv launch");
  LAUNCH(IPTTT_K_PROJ, mf_proj(sl, w, ws, st), "proj launch");
  const int64_t sseq = K * (int64_t)dF;  // snapshot pitch between sequences
  __bf16 *snap_w = (__bf16 *)(base + lay.snap_w), *snap_g = (__bf16 *)(base + lay.snap_g);
  __bf16 *rt = (__bf16 *)(base + lay.rt);
  const int64_t tstride = (int64_t)d.d * sl.Lp;  // [n][d][Lp] pitch between sequences
  if (!mse) {
    LAUNCH(IPTTT_K_UPDATE, mf_update_scan(sl, ws, wscr, false, st), "update scan launch");
  } else if (lay.G > 1) {
    // chunk groups, as the forward: per group one apply (from W at its first
    // chunk), the Gram corrections of its later chunks, one update that keeps
    // a row-major W per chunk; the group's residuals then go to their place
    // in the token-contiguous Rt the reverse pass reads
    Slab sg = sl;
    sg.G = lay.G;
    sg.ng_cap = (int)((K + lay.G - 1) / lay.G);
    const int64_t RG = (int64_t)lay.G * Bp;
    __bf16 *rtg = (__bf16 *)(base + lay.rtg);
    float *oscr = (float *)(base + lay.oscr);
    WsPtrs wsg{nullptr, base + lay.zt, nullptr, base + lay.vt, nullptr, rtg, base + lay.p};
    LAUNCH(IPTTT_K_SNAPSHOT, gen_snapshot<__bf16>(sl, wscr, snap_w, sseq, st), "snapshot launch");
    LAUNCH(IPTTT_K_GRAM, mf_gram(sg, wsg, st), "Gram launch");
    for (int q = 0; (int64_t)q * lay.G < K; ++q) {
      const int64_t j0 = (int64_t)q * lay.G, nq = std::min<int64_t>(lay.G, K - j0);
      LAUNCH(IPTTT_K_APPLY,
             mf_apply_mse_group_rm(sg, q, bb.zt, snap_w + j0 * dF, sseq, bb.vt, oscr, rtg, st),
             "apply launch");
      for (int jl = 1; jl < nq; ++jl)
        LAUNCH(IPTTT_K_MSE_FIX, mf_mse_fix(sg, q, jl, wsg, oscr, st), "MSE correction launch");
      LAUNCH(IPTTT_K_UPDATE, mf_update_group_rm(sg, q, bb.zt, rtg, wscr, snap_w + j0 * dF, sseq, st),
             "update launch");
      TRY_HIP(hipMemcpy2DAsync(rt + j0 * Bp, (size_t)sl.Lp * 2, rtg, (size_t)RG * 2,
                               (size_t)(nq * Bp) * 2, (size_t)batch * d.d, hipMemcpyDeviceToDevice,
                               st),
              "residual copy");
    }
  } else {
    // chunk by chunk: W_j kept per chunk, residual eta (V - O_j) kept per chunk
    LAUNCH(IPTTT_K_SNAPSHOT, gen_snapshot<__bf16>(sl, wscr, snap_w, sseq, st), "snapshot launch");
    for (int64_t j = 0; j < K; ++j) {
      LAUNCH(IPTTT_K_APPLY,
             mf_apply_mse_chunk(sl, (int)j, bb.zt, snap_w + j * dF, sseq, bb.vt, rt + j * Bp,
                                tstride, sl.Lp, st),
             "apply launch");
      LAUNCH(IPTTT_K_UPDATE,
             mf_update_chunk(sl, (int)j, bb.zt, rt + j * Bp, sl.Lp, tstride, wscr,
                             j + 1 < K ? snap_w + (j + 1) * dF : nullptr, sseq, st),
             "update launch");
    }
  }
  // reverse scan: G_{j+1} per chunk, G_0 = dL/dW_0 per sequence
  LAUNCH(IPTTT_K_BW_MISC, bw_transpose_f32(sl, d_o, (__bf16 *)bb.dot, st), "dO transpose launch");
  LAUNCH(IPTTT_K_BW_MISC, bw_transpose_bf16(sl, (const __bf16 *)x, (__bf16 *)bb.xt, st),
         "x transpose launch");
  if (d_wfinal)
    TRY_HIP(hipMemcpyAsync(gscr, d_wfinal, batch * dF * sizeof(float), hipMemcpyDeviceToDevice, st),
            "d_wfinal copy");
  else
    LAUNCH(IPTTT_K_BW_MISC, bw_fill(gscr, (int64_t)(batch * dF), 0.f, st), "fill launch");
  if (!mse) {
    LAUNCH(IPTTT_K_BW_SCAN, mf_update_reverse(sl, bb.zt, bb.dot, gscr, snap_g, st),
           "reverse scan launch");
    // per-chunk gradients, then the slow weights
    LAUNCH(IPTTT_K_BW_DZ, bw_dz(sl, bb, bb.dot, bb.vt, st), "dZ launch");
    LAUNCH(IPTTT_K_BW_DV, bw_dv(sl, bb, st), "dV launch");
  } else {
    // chunk by chunk in reverse: T_j = G_{j+1}; dY_j = dO_j - eta Z_j G_{j+1},
    // dV_j = eta Z_j G_{j+1}; G_j = G_{j+1} + Z_j^T dY_j
    LAUNCH(IPTTT_K_BW_MISC, gen_snapshot<__bf16>(sl, gscr, snap_g + (K - 1) * dF, sseq, st),
           "snapshot launch");
    for (int64_t j = K - 1; j >= 0; --j) {
      LAUNCH(IPTTT_K_BW_DV, bw_mse_p(sl, (int)j, bb, st), "dY launch");
      LAUNCH(IPTTT_K_BW_SCAN,
             mf_update_chunk(sl, (int)j, bb.zt, bb.dyt + j * Bp, sl.Lp, tstride, gscr,
                             j > 0 ? snap_g + (j - 1) * dF : nullptr, sseq, st),
             "backward update launch");
    }
    LAUNCH(IPTTT_K_BW_DZ, bw_dz(sl, bb, bb.dyt, bb.rt, st), "dZ launch");
  }
  LAUNCH(IPTTT_K_BW_SMALL, bw_dc(sl, bb, d.proj, st), "dC launch");
  LAUNCH(IPTTT_K_BW_SMALL,
         bw_conv(sl, bb, (const __bf16 *)e, d.conv_w, grads->de, grads->dconv_w, st),
         "conv adjoint launch");
  LAUNCH(IPTTT_K_BW_DX, bw_dx(sl, bb, d.w_gate, d.w_up, grads->dx, st), "dX launch");
  LAUNCH(IPTTT_K_BW_DW, bw_dw(sl, bb, grads->dw_gate, grads->dw_up, st), "dW launch");
  LAUNCH(IPTTT_K_BW_SMALL, bw_dproj(sl, bb, grads->dproj, st), "dProj launch");
  LAUNCH(IPTTT_K_BW_SMALL, bw_sum_seq(gscr, batch, (int64_t)dF, grads->dw0, st), "dW0 launch");
  return IPTTT_OK;
}

ipttt_status ipttt_prefill_packed(ipttt_layer *h, const void *x, const void *e, float *o,
                                  int32_t slot, int64_t seq_len, const int64_t *doc_starts,
                                  int32_t n_docs, void *hip_stream) {
  if (!h) return fail(IPTTT_E_INVALID, "handle is NULL");
  if (slot < 0 || slot >= h->desc.max_batch)
    return fail(IPTTT_E_INVALID, "slot=%d outside [0, %d)", slot, h->desc.max_batch);
  if (seq_len < 0 || n_docs < 0) return fail(IPTTT_E_INVALID, "seq_len and n_docs must be >= 0");
  if (n_docs > 0 && !doc_starts) return fail(IPTTT_E_INVALID, "doc_starts is NULL");
  for (int32_t i = 0; i < n_docs; ++i) {
    if (doc_starts[i] <= 0 || doc_starts[i] >= seq_len)
      return fail(IPTTT_E_INVALID, "doc_starts[%d]=%lld outside (0, %lld)", i, (long long)doc_starts[i],
                  (long long)seq_len);
    if (i > 0 && doc_starts[i] <= doc_starts[i - 1])
      return fail(IPTTT_E_INVALID, "doc_starts must be strictly ascending");
  }
  if (seq_len == 0) return IPTTT_OK;
  ipttt_status s = check_call(h, x, e, o);
  if (s != IPTTT_OK) return s;
  if (!h->was_reset[(size_t)slot]) return fail(IPTTT_E_STATE, "sequence %d was never reset", slot);
  const ipttt_layer_desc &d = h->desc;
  const size_t el = (size_t)elem_size(d.in_dtype);
  hipStream_t st = (hipStream_t)hip_stream;
  int64_t a = 0;
  for (int32_t i = 0; i <= n_docs; ++i) {
    const int64_t b = i < n_docs ? doc_starts[i] : seq_len;
    if (i > 0)
      TRY_HIP(hipMemcpyAsync(d.w_state + (size_t)slot * d.d * d.d_ff, d.w0,
                             (size_t)d.d * d.d_ff * sizeof(float), hipMemcpyDeviceToDevice, st),
              "reset copy");
    s = dispatch(h, (const char *)x + (size_t)a * d.d * el, (const char *)e + (size_t)a * d.d * el,
                 o + (size_t)a * d.d, slot, 1, b - a, (b - a) * d.d, st);
    if (s != IPTTT_OK) return s;
    a = b;
  }
  return IPTTT_OK;
}

}  // extern "C"
