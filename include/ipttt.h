/*
 * ipttt.h: C ABI of libipttt, the MI355X (gfx950) fast-weight prefill of
 * In-Place Test-Time Training.
 *
 * What it computes. A gated MLP, MLP(x) = (SiLU(x W_g) (x) (x W_u)) W_o, whose
 * down projection W_o is a per-sequence fast weight W (explainer page
 * "In-Place Test-Time Training：让大语言模型在推理时原地进化…", §2.1). The
 * prefill walks each sequence in chunks of B tokens, k ascending (same page,
 * §2.2 and Fig. 1; analysis page "大模型长文本核心架构全解析…", 第三板斧):
 *
 *   Z_k = SiLU(X_k W_g) * (X_k W_u)           intermediate activation
 *   C_k[t, c] = sum_j conv_w[c, j] E[t + j, c]  depthwise conv over the token
 *             embeddings E, taps looking forward, zero past the chunk's end
 *   V_k = C_k Proj                            LM-aligned target (explainer §2.3)
 *   O_k = Z_k W_k                             apply with the current W
 *   W_{k+1} = W_k + eta Z_k^T V_k             linear update (explainer §2.3)
 *   W_{k+1} = W_k - eta Z_k^T (O_k - V_k)     MSE update (analysis page, 第二板斧)
 *
 * A last chunk shorter than B (seq_len not a multiple of B) is applied and
 * updated like any other; its conv pad starts at its own end. Each prefill
 * call starts a new chunk at its first token; the state W carries over.
 *
 * Layouts. Row-major. Every weight matrix is stored OUTPUT-major, row r holding
 * the weights that produce output feature r (the nn.Linear convention); in the
 * row-vector notation above the stored array is the transpose:
 *   w_gate, w_up  [d_ff][d]     w_gate[j*d + i] = W_g[i][j]
 *   proj          [d][d]        proj[j*d + i]   = Proj[i][j]
 *   conv_w        [d][conv_k]   conv_w[c*conv_k + j] is tap j of channel c
 *   w0            [d][d_ff]     fp32, W_0 transposed (the pretrained W_o)
 *   w_state       [max_batch][d][d_ff]  fp32, W transposed, one per sequence
 *   x, e          [batch][seq_len][d]   in_dtype
 *   o             [batch][seq_len][d]   fp32
 *
 * Arithmetic. in_dtype IPTTT_F32: fp32 throughout. in_dtype IPTTT_BF16: bf16
 * operands on bf16 MFMA with fp32 accumulation; Z, the conv output, V and the
 * copy of W that the apply reads are rounded to nearest-even bf16; W stays
 * fp32; the conv runs in fp32.
 *
 * Ownership. The caller allocates every device buffer (weights, w0, w_state,
 * x, e, o and the workspace) and keeps it alive while the handle uses it; the
 * library borrows the pointers and never allocates or frees device memory.
 * The handle owns host metadata only.
 *
 * Errors. Every function returns a status and never throws across the ABI.
 * Arguments are validated before any device work, so a rejected call has no
 * device side effects. HIP launch errors map to IPTTT_E_HIP; faults inside a
 * kernel surface at the caller's next synchronisation. ipttt_last_error()
 * gives a thread-local message for the last failure.
 *
 * Concurrency. All device work of a call is enqueued on the given HIP stream
 * (NULL = the null stream); the library never synchronises the host. A handle
 * is not thread-safe; distinct handles are. Calls that share a workspace must
 * be ordered on one stream.
 */
#ifndef IPTTT_H
#define IPTTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ipttt_layer ipttt_layer; /* opaque, host-side only */

typedef enum {
  IPTTT_OK = 0,
  IPTTT_E_INVALID = -1,     /* bad argument: null pointer, size <= 0, misalignment */
  IPTTT_E_UNSUPPORTED = -2, /* valid but not implemented (e.g. conv_k > 8)         */
  IPTTT_E_HIP = -3,         /* a HIP runtime call or kernel launch failed          */
  IPTTT_E_STATE = -4,       /* a sequence's fast weight was never reset            */
  IPTTT_E_WORKSPACE = -5    /* workspace too small for one chunk of this batch     */
} ipttt_status;

typedef enum { IPTTT_F32 = 0, IPTTT_BF16 = 1 } ipttt_dtype;

typedef enum { IPTTT_UPDATE_LINEAR = 0, IPTTT_UPDATE_MSE = 1 } ipttt_update;

/* Flags. IPTTT_FLAG_GENERIC_KERNELS runs bf16 layers on the generic LDS-tiled
 * FMA kernels instead of the MFMA kernels (same results up to fp32 summation
 * order); fp32 layers always use them. */
#define IPTTT_FLAG_GENERIC_KERNELS 1u

/* Chunk groups (bf16 MFMA path). The linear update is associative, a plain
 * sum of per-chunk terms (explainer page §2.3), so a group of G consecutive
 * chunks can share one copy of W: with W_q the fast weight at the group's
 * first chunk,
 *   O_t = z_t W_q + sum over earlier-chunk tokens s of the group of
 *         (z_t . z_s) eta v_s,
 * which is O_k = Z_k W_k for every chunk k of the group. The scan then keeps
 * one bf16 copy of W per group instead of per chunk, and the apply adds the
 * block-causal Gram term. The MSE rule (analysis page, 第二板斧) groups the
 * same way with the residuals r_s = eta (v_s - o_s) of the earlier chunks in
 * place of eta v_s; those are final only once their own chunk is, so the
 * chunks of a group are corrected in order, and W is updated once per group.
 * group_chunks sets G (1 gives the plain chunk scan; G * round_up(chunk, 64)
 * must not exceed 4096); 0 lets the library choose, about 1024 chunk-padded
 * rows per group for the linear rule and 2048 for the MSE rule. Results agree
 * with the plain scan up to bf16 rounding. The generic kernels ignore the
 * field. */
typedef struct {
  int32_t d;           /* model width (columns of X, E, O)                       */
  int32_t d_ff;        /* MLP width F (rows of the fast weight's input side)     */
  int32_t conv_k;      /* conv taps per channel, 1..8                            */
  int32_t chunk;       /* chunk size B >= 1                                      */
  int32_t max_batch;   /* number of fast-weight states in w_state                */
  float eta;           /* step size of the update                                */
  ipttt_update update; /* linear or MSE rule                                     */
  ipttt_dtype in_dtype;/* dtype of x, e, w_gate, w_up, proj, conv_w              */
  uint32_t flags;      /* IPTTT_FLAG_*                                           */
  int32_t group_chunks;/* chunks per group of the chunk-parallel scan (the
                          note above); 0 = library choice, 1 = chunk by chunk */
  const void *w_gate;  /* [d_ff][d]                                              */
  const void *w_up;    /* [d_ff][d]                                              */
  const void *proj;    /* [d][d]                                                 */
  const void *conv_w;  /* [d][conv_k]                                            */
  const float *w0;     /* [d][d_ff] fp32: reset source                           */
  float *w_state;      /* [max_batch][d][d_ff] fp32: mutated by prefill          */
  void *workspace;     /* device scratch, 256-byte aligned                       */
  size_t workspace_bytes;
} ipttt_layer_desc;

/* Bytes of workspace that let one prefill call on `batch` sequences process
 * `slab_chunks` chunks per pass (a call makes ceil(chunks / slab_chunks)
 * passes; more chunks per pass means fewer round trips of W through memory).
 * Returns 0 if the descriptor's sizes are invalid or batch / slab_chunks < 1.
 * Pointers in `desc` are not read. */
size_t ipttt_workspace_bytes(const ipttt_layer_desc *desc, int32_t batch, int32_t slab_chunks);

/* Validates the descriptor (sizes, dtypes, non-null and 16-byte aligned device
 * pointers, workspace pointer and size) and returns a handle in *out. No
 * device work (it looks up, on the current device, the address of the scratch
 * area of ipttt_prefill_layer_noalloc). Every sequence starts "never reset":
 * reset it before prefill. */
ipttt_status ipttt_init(const ipttt_layer_desc *desc, ipttt_layer **out);

/* Prefill of sequences 0..batch-1 (state slots 0..batch-1), seq_len tokens
 * each, continuing from each slot's current W: writes o and advances
 * w_state. batch == 0 or seq_len == 0 is a successful no-op. Fails with
 * IPTTT_E_STATE if a slot in range was never reset, IPTTT_E_WORKSPACE if the
 * workspace cannot hold one chunk of `batch` sequences, IPTTT_E_INVALID for
 * batch > max_batch, null or misaligned pointers (x and e must be 16-byte
 * aligned on the bf16 MFMA path, element-aligned otherwise; o 4-byte). */
ipttt_status ipttt_prefill_layer(ipttt_layer *h, const void *x, const void *e, float *o,
                                 int32_t batch, int64_t seq_len, void *hip_stream);

/* Allocation-free prefill, for callers that cannot allocate device memory
 * (code under HIP stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation as ipttt_prefill_layer, with its workspace
 * in a fixed scratch area of IPTTT_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every device it runs on (a static device array, alive until the
 * process ends) instead of the descriptor's workspace. It calls no hipMalloc,
 * hipFree or other allocating routine and records no profiling events; the
 * caller still passes x, e, o and the handle's w_state. Longer sequences run
 * in several passes over the scratch area (W stays exact between them, as with
 * a small workspace); a call whose single chunk of `batch` sequences needs more
 * than the scratch area returns IPTTT_E_WORKSPACE. Every call on one device
 * shares that device's scratch area, which keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap on one device,
 * from any handle, stream or thread, race and must be ordered by the caller.
 * The scratch address is looked up with the current device current, at
 * ipttt_init and, for another device, at the first call there. Same validation
 * and error codes as ipttt_prefill_layer, plus IPTTT_E_HIP if the lookup fails. */
#define IPTTT_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
ipttt_status ipttt_prefill_layer_noalloc(ipttt_layer *h, const void *x, const void *e, float *o,
                                         int32_t batch, int64_t seq_len, void *hip_stream);

/* Prefill of ONE sequence holding several packed documents (state slot
 * `slot`). The fast weight goes back to w0 at every document start (explainer
 * page §3.2, boundary reset): doc_starts lists n_docs token positions in
 * ascending order (host memory); position 0 is implied and entries outside
 * (0, seq_len) are rejected. A new chunk begins at every document start, so no
 * chunk, and no conv pad, spans two documents. The first document continues
 * from the slot's current W. */
ipttt_status ipttt_prefill_packed(ipttt_layer *h, const void *x, const void *e, float *o,
                                  int32_t slot, int64_t seq_len, const int64_t *doc_starts,
                                  int32_t n_docs, void *hip_stream);

/* Decode: one new token for each of sequences 0..batch-1, all at the same
 * position inside their current chunk (the step after prefill while the fast
 * weight keeps adapting, explainer page §6). The caller keeps the chunk in
 * progress: x and e point at its first token for sequence 0, sequence i's
 * chunk starts seq_stride elements later, rows are d apart, and rows
 * 0..pos hold the chunk so far with the new token at row pos (0 <= pos < B).
 * Writes o[batch][d] fp32 = z W_k for the new token, where z is its gated
 * activation and W_k the fast weight of the chunk (the last update happened
 * at the chunk's start). When pos == B - 1 the chunk is complete and its
 * update W_{k+1} = W_k + eta Z^T V (or the MSE rule) runs from rows 0..B-1,
 * exactly as prefill would. The chunk must start on a chunk boundary of the
 * scan (after a reset, a completed chunk, or a prefill call). Same
 * validation and error codes as ipttt_prefill_layer. */
ipttt_status ipttt_decode_step(ipttt_layer *h, const void *x, const void *e, int64_t seq_stride,
                               int32_t pos, float *o, int32_t batch, void *hip_stream);

/* Backward (training through the layer: continued training of a pretrained
 * model and pretraining from scratch, explainer page §4.1 and §4.2). For a
 * prefill of sequences 0..batch-1 that each start from w0, seq_len tokens
 * each, and a scalar loss with gradient d_o = dL/dO ([batch][seq_len][d]
 * fp32) and d_wfinal = dL/dW_final ([batch][d][d_ff] fp32 in the w_state
 * layout, or NULL for zero), computes the gradients with respect to the
 * inputs and the slow weights, differentiating through every update of the
 * scan (eta is not trained). The forward is recomputed inside the call from
 * x, e and w0; w_state and the layer's workspace are not touched. Every
 * output is fp32 and overwritten:
 *   dx, de     [batch][seq_len][d]
 *   dw_gate, dw_up [d_ff][d]   dproj [d][d]   dconv_w [d][conv_k]   (layouts of
 *   dw0 [d][d_ff]                           the weights, summed over the batch)
 * workspace: device scratch of ipttt_backward_workspace_bytes() bytes,
 * 256-byte aligned, exclusively the call's until it completes on the stream.
 * Both update rules; the MSE rule runs its reverse pass chunk by chunk (each
 * chunk's dL/dW_j needs the next chunk's). Supported: bf16 layers on the MFMA
 * path; other layers return IPTTT_E_UNSUPPORTED. Same pointer and size
 * validation as prefill. */
typedef struct {
  float *dx, *de;
  float *dw_gate, *dw_up;
  float *dproj;
  float *dconv_w;
  float *dw0;
} ipttt_grads;

/* Workspace bytes of ipttt_backward_layer for `batch` sequences of seq_len
 * tokens; 0 if the sizes are invalid or the layer's backward is unsupported.
 * Pointers in `desc` are not read. */
size_t ipttt_backward_workspace_bytes(const ipttt_layer_desc *desc, int32_t batch,
                                      int64_t seq_len);

ipttt_status ipttt_backward_layer(ipttt_layer *h, const void *x, const void *e, const float *d_o,
                                  const float *d_wfinal, int32_t batch, int64_t seq_len,
                                  const ipttt_grads *grads, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/* w_state[s] := w0 bitwise for s in first_seq..first_seq+n_seq-1 (document
 * boundary, explainer page §3.2) and marks those slots as reset. */
ipttt_status ipttt_reset_fast_weights(ipttt_layer *h, int32_t first_seq, int32_t n_seq,
                                      void *hip_stream);

/* Per-kernel timing. Between ipttt_profile_begin and ipttt_profile_end the
 * handle records a HIP event pair on the call's stream around every kernel
 * launch; results are unchanged. Events are created on first use and freed by
 * ipttt_destroy. */
typedef enum {
  IPTTT_K_GATEUP = 0,   /* Z = SiLU(X W_g) * (X W_u)                 */
  IPTTT_K_CONV = 1,     /* chunk-padded depthwise conv of E          */
  IPTTT_K_PROJ = 2,     /* V = C Proj                                */
  IPTTT_K_UPDATE = 3,   /* W += eta Z^T V (scan) or the MSE update   */
  IPTTT_K_APPLY = 4,    /* O = Z W_k                                 */
  IPTTT_K_SNAPSHOT = 5, /* bf16 / fp32 copy of W read by the apply   */
  IPTTT_K_GRAM = 6,     /* block-causal Z Z^T of a chunk group       */
  IPTTT_K_BW_SCAN = 7,  /* backward: G += Z^T dO, chunks in reverse  */
  IPTTT_K_BW_DZ = 8,    /* backward: dZ -> dA, dU                    */
  IPTTT_K_BW_DV = 9,    /* backward: dV = eta Z G                    */
  IPTTT_K_BW_DX = 10,   /* backward: dX                              */
  IPTTT_K_BW_DW = 11,   /* backward: dW_gate, dW_up                  */
  IPTTT_K_BW_SMALL = 12,/* backward: dC, dProj, conv adjoint, dW_0   */
  IPTTT_K_BW_MISC = 13, /* backward: transposes, fills, copies       */
  IPTTT_K_MSE_FIX = 14, /* MSE rule, chunk groups: Gram correction   */
  IPTTT_K_COUNT = 15
} ipttt_kernel;

ipttt_status ipttt_profile_begin(ipttt_layer *h);

/* Waits for the recorded events, writes the number of launches and their summed
 * milliseconds per kernel kind into launches[IPTTT_K_COUNT] and
 * ms[IPTTT_K_COUNT] (host arrays), and stops recording. */
ipttt_status ipttt_profile_end(ipttt_layer *h, int32_t *launches, double *ms);

/* Frees the handle (host memory only). NULL is ignored. */
void ipttt_destroy(ipttt_layer *h);

/* Static name of a status code. */
const char *ipttt_status_str(ipttt_status s);

/* Thread-local message describing this thread's last failed call ("" if none). */
const char *ipttt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IPTTT_H */
