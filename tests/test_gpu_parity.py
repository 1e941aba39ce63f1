"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bars (relative Frobenius error of O and of the final fast weight):
  fp32 path: 1e-4      bf16-input / fp32-accumulate path: 2e-2
Bitwise: run-to-run determinism, token-level causality, continuation across
calls, slab splits, batch independence and reset.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from chunked_weight_mlp_amd import ipttt as B
from parity_check import ChunkErrors, check_chunks, check_weights, report

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_fro(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def make_layer(w: wl.Workload, weights, flags=0, max_batch=None, slab_chunks=None,
               workspace_bytes=None, group_chunks=0):
    dev = {k: v.to(DEV) for k, v in weights.items()}
    return B.Layer(**dev, chunk=w.chunk, eta=w.eta, update=w.update,
                   max_batch=max_batch or w.n_seq, slab_chunks=slab_chunks,
                   max_seq_len=w.seq_len, workspace_bytes=workspace_bytes, flags=flags,
                   group_chunks=group_chunks)


def gpu_run(layer, x, e, reset=True):
    if reset:
        layer.reset()
    o = layer.prefill(x.to(DEV), e.to(DEV))
    torch.cuda.synchronize()
    return o


def w_pages(layer, n):
    """Final fast weights in the pages' orientation [n, F, d], float64."""
    return layer.w_state[:n].detach().to("cpu", torch.float64).numpy().transpose(0, 2, 1)


def oracle_run(w, x, e, weights, W_start=None):
    ow = wl.to_oracle(weights)
    X = x.to(torch.float64).numpy()
    E = e.to(torch.float64).numpy()
    return oracle.prefill(X, E, ow["W_g"], ow["W_u"], ow["conv_w"], ow["Proj"],
                          ow["W_0"] if W_start is None else W_start, w.eta, w.chunk, update=w.update)


def check_against_oracle(w, flags=0, n_seq=None, seq_len=None, slab_chunks=None, seed=0,
                         group_chunks=0):
    weights = wl.make_weights(w, seed_offset=seed)
    x, e = wl.make_inputs(w, seq_len=seq_len, n_seq=n_seq, seed_offset=seed)
    N, L = x.shape[0], x.shape[1]
    say(f"[parity] {w.name} N={N} L={L} B={w.chunk} d={w.d} F={w.d_ff} {w.dtype} {w.update} "
        f"flags={flags} slab={slab_chunks} group={group_chunks}")
    layer = make_layer(w.replace(n_seq=N, seq_len=L), weights, flags=flags, slab_chunks=slab_chunks,
                       group_chunks=group_chunks)
    o = gpu_run(layer, x, e).to("cpu", torch.float64).numpy()
    Wg = w_pages(layer, N)
    O_ref, W_ref = oracle_run(w, x, e, weights)
    assert np.isfinite(o).all()
    eo = check_chunks(o, O_ref, w.chunk, TOL[w.dtype], "parity")
    ew = check_weights(Wg, W_ref, TOL[w.dtype], "parity")
    return eo, ew


TINY = wl.WORKLOADS["tiny_d64_f256_L1024_B128_fp32"]
W4B = wl.WORKLOADS["qwen3_4b_L32k_B512"]
W15 = wl.WORKLOADS["pretrain_1p5b_8x16k_B512_mse"]


def test_tiny_fp32_full_size():
    check_against_oracle(TINY)


@pytest.mark.parametrize("L,Bc,N,update", [
    (1000, 128, 2, "linear"),   # ragged last chunk, two sequences
    (37, 5, 1, "linear"),       # chunk not a multiple of 32, ragged
    (130, 64, 3, "mse"),
    (1, 16, 1, "linear"),       # a single token
    (70, 1, 1, "linear"),       # one token per chunk
    (300, 300, 1, "mse"),       # single chunk
    (200, 512, 1, "linear"),    # chunk longer than the sequence
])
def test_fp32_edges(L, Bc, N, update):
    w = TINY.replace(chunk=Bc, update=update, eta=0.02 if update == "linear" else 0.01)
    check_against_oracle(w, n_seq=N, seq_len=L)


BF16_SMALL = wl.Workload("bf16_d256_f640", 2, 256, 640, 1000, 128, "bf16", 1e-2, "linear")


@pytest.mark.parametrize("flags", [0, B.IPTTT_FLAG_GENERIC_KERNELS], ids=["mfma", "generic"])
@pytest.mark.parametrize("update", ["linear", "mse"])
@pytest.mark.parametrize("L,Bc", [(1000, 128), (777, 96), (2048, 1024), (64, 64)])
def test_bf16_small_shapes(flags, update, L, Bc):
    w = BF16_SMALL.replace(chunk=Bc, update=update, eta=1e-2 if update == "linear" else 2e-3)
    check_against_oracle(w, flags=flags, seq_len=L)


def test_bf16_persistent_uneven_tiles():
    """Persistent gate/up and proj blocks with tile counts that do not split
    evenly over the 8 XCDs: d_ff 4224 and 4224 slab rows give 17 x 33 = 561
    gate/up tiles (2-3 per block, one XCD with a tile more), proj 17 x 2 = 34."""
    w = BF16_SMALL.replace(d=512, d_ff=4224, chunk=128)
    check_against_oracle(w, n_seq=1, seq_len=33 * 128)


@pytest.mark.parametrize("update", ["linear", "mse"])
def test_bf16_partial_tiles(update):
    """d 320 and d_ff 576 (multiples of 64, not of 128 or 256): the last row and
    column tiles of gate/up, proj, the update scan and the apply are partial, so
    their bounds checks (loads clamped to a valid row, stores skipped) run."""
    w = BF16_SMALL.replace(d=320, d_ff=576, update=update,
                           eta=1e-2 if update == "linear" else 2e-3)
    check_against_oracle(w, n_seq=2, seq_len=700)


@pytest.mark.parametrize("Kc,Bc,L,update", [
    (1, 64, 194, "linear"),   # one tap
    (3, 2, 41, "linear"),     # chunks of 2 tokens, shorter than the filter
    (3, 128, 257, "mse"),     # 1-token tail
    (8, 5, 67, "linear"),     # 8 taps over 5-token chunks, 2-token tail
    (8, 64, 130, "mse"),      # 2-token tail
])
def test_bf16_conv_taps(Kc, Bc, L, update):
    """The conv with 1, 3 and 8 taps per channel (each a kernel instance of its
    own), including chunks and ragged tails shorter than the filter, whose taps
    past the chunk's end read the zero pad."""
    w = BF16_SMALL.replace(chunk=Bc, conv_k=Kc, update=update,
                           eta=1e-2 if update == "linear" else 2e-3)
    check_against_oracle(w, n_seq=1, seq_len=L)


def test_bf16_multi_slab():
    """A workspace for 3 chunks forces several passes over a 9-chunk sequence."""
    check_against_oracle(BF16_SMALL.replace(chunk=64), seq_len=9 * 64 - 5, slab_chunks=3)


@pytest.mark.parametrize("Bc,G,L,N", [
    (64, 0, 2000, 2),     # default group (16 chunks), ragged last chunk, two groups
    (96, 3, 1000, 1),     # 384 group rows: not a multiple of the apply's row tile
    (128, 5, 3000, 2),    # a short last group (4 of 5 chunks)
    (200, 2, 1500, 1),    # padding rows inside every chunk
    (64, 64, 4096 + 37, 1),  # the largest group (4096 rows) and a one-chunk last group
    (64, 4, 100, 1),      # fewer chunks than a group
])
def test_bf16_chunk_groups(Bc, G, L, N):
    """Chunk-parallel form: one W snapshot per group of G chunks, the group's
    earlier chunks added through the block-causal Gram product."""
    check_against_oracle(BF16_SMALL.replace(chunk=Bc), n_seq=N, seq_len=L, group_chunks=G)


@pytest.mark.parametrize("Bc,G,L,N", [
    (64, 0, 2000, 2),     # default group (32 chunks): 31 corrections, ragged last chunk
    (96, 3, 1000, 1),     # 384 group rows: not a multiple of the apply's row tile
    (128, 5, 3000, 2),    # a short last group (4 of 5 chunks)
    (200, 2, 1500, 1),    # padding rows inside every chunk
    (64, 64, 4096 + 37, 1),  # the largest group (4096 rows) and a one-chunk last group
    (64, 4, 100, 1),      # fewer chunks than a group
])
def test_bf16_mse_chunk_groups(Bc, G, L, N):
    """MSE rule over chunk groups: O of a group from W at its first chunk, each
    later chunk corrected by the Gram term over the earlier chunks' residuals,
    one update per group."""
    w = BF16_SMALL.replace(chunk=Bc, update="mse", eta=2e-3)
    check_against_oracle(w, n_seq=N, seq_len=L, group_chunks=G)


@pytest.mark.parametrize("N", [2, 3, 4])
def test_mse_batch_entry_points_bitwise(N):
    """MSE chunk groups over several sequences: every sequence's output and
    final fast weight from ipttt_prefill_layer equal, bit for bit, those of the
    allocation-free entry point (same kernels and grouping, workspace in the
    library's scratch area); N = 2 is also checked against the oracle chunk by
    chunk."""
    w = BF16_SMALL.replace(chunk=64, update="mse", eta=2e-3, n_seq=N, seq_len=1500)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights, group_chunks=4)   # 24 chunks: 6 groups
    try:
        xd, ed = x.to(DEV), e.to(DEV)
        runs = []
        for fn in (B.ipttt_prefill_layer, B.ipttt_prefill_layer_noalloc):
            layer.reset()
            o = torch.full((N, w.seq_len, w.d), float("nan"), dtype=torch.float32, device=DEV)
            fn(layer.handle, xd, ed, o, N, w.seq_len)
            torch.cuda.synchronize()
            runs.append((o.cpu(), layer.w_state[:N].cpu()))
        (o_reg, w_reg), (o_na, w_na) = runs
        assert torch.isfinite(o_reg).all()
        assert torch.equal(o_reg, o_na)
        assert torch.equal(w_reg, w_na)
        if N == 2:
            O_ref, W_ref = oracle_run(w, x, e, weights)
            check_chunks(o_reg.double().numpy(), O_ref, w.chunk, TOL[w.dtype], "entry points")
            check_weights(w_reg.double().numpy().transpose(0, 2, 1), W_ref, TOL[w.dtype],
                          "entry points")
    finally:
        layer.close()


def test_bf16_chunk_groups_multi_slab():
    """A workspace for 7 chunks with groups of 3: slabs of 6 chunks (whole groups)."""
    check_against_oracle(BF16_SMALL.replace(chunk=64), seq_len=20 * 64 - 9, slab_chunks=7,
                         group_chunks=3)


@pytest.mark.parametrize("update,w_tol", [("linear", 1e-5), ("mse", 1e-2)])
def test_chunk_groups_match_plain_scan(update, w_tol):
    """Grouped and plain scans differ only by rounding: O agrees to bf16 level.
    With the linear rule the final weight is a sum of the same products and
    agrees very closely; with the MSE rule each update multiplies bf16
    residuals, which the two forms round differently, so W agrees at the bf16
    level both show against the oracle (about 3e-3)."""
    w = BF16_SMALL.replace(chunk=64, n_seq=1, seq_len=1500, update=update,
                           eta=1e-2 if update == "linear" else 2e-3)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    outs = []
    for g in (1, 8):
        layer = make_layer(w, weights, group_chunks=g)
        outs.append((gpu_run(layer, x, e).double().cpu().numpy(), w_pages(layer, 1)))
        layer.close()
    eo = rel_fro(outs[1][0], outs[0][0])
    ew = rel_fro(outs[1][1], outs[0][1])
    say(f"[groups] {update} grouped vs plain: rel O={eo:.3e} W={ew:.3e}")
    assert eo <= 1e-2 and ew <= w_tol


def test_qwen3_4b_shape_two_chunks_and_tail():
    check_against_oracle(W4B.replace(chunk=1024), n_seq=1, seq_len=2 * 1024 + 100)


def test_pretrain_1p5b_mse_shape():
    check_against_oracle(W15, n_seq=2, seq_len=512 + 512 + 37)


@pytest.mark.parametrize("Bc", [64, 256, 512, 1024, 4096])
def test_chunk_sweep_vs_prefix_form(Bc):
    """4B-shaped layer at several chunk sizes against the oracle's prefix-sum form."""
    w = wl.WORKLOADS[f"qwen3_4b_L64k_B{Bc}"]
    L = 1024
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w, seq_len=L)
    say(f"[sweep] B={Bc} L={L}")
    layer = make_layer(w.replace(seq_len=L), weights)
    o = gpu_run(layer, x, e).to("cpu", torch.float64).numpy()
    ow = wl.to_oracle(weights)
    O_ref, W_ref = oracle.prefill_prefix_form(x.double().numpy(), e.double().numpy(), ow["W_g"],
                                              ow["W_u"], ow["conv_w"], ow["Proj"], ow["W_0"], w.eta, Bc)
    check_chunks(o, O_ref, Bc, TOL["bf16"], f"sweep B={Bc}")
    check_weights(w_pages(layer, 1), W_ref, TOL["bf16"], f"sweep B={Bc}")


def _bitwise_pair(layer_a, layer_b, x, e):
    oa = gpu_run(layer_a, x, e)
    ob = gpu_run(layer_b, x, e)
    return oa, ob


def test_determinism_and_reset():
    w = BF16_SMALL.replace(seq_len=1000)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights)
    o1 = gpu_run(layer, x, e).clone()
    w1 = layer.w_state.clone()
    o2 = gpu_run(layer, x, e)   # reset puts W_0 back: same result bit for bit
    assert torch.equal(o1, o2)
    assert torch.equal(w1, layer.w_state)


def test_causality_bitwise():
    w = BF16_SMALL.replace(n_seq=1, seq_len=640, chunk=128)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights)
    o = gpu_run(layer, x, e).clone()
    for p in (1, 127, 128, 129, 300):
        x2, e2 = x.clone(), e.clone()
        x2[:, p:] += 1.0
        e2[:, p:] -= 1.0
        o2 = gpu_run(layer, x2, e2)
        assert torch.equal(o2[:, :p], o[:, :p]), p
        assert not torch.equal(o2[:, p:], o[:, p:])
    for k in range(4):  # target of chunk k is first used by chunk k+1
        e3 = e.clone()
        e3[:, k * 128:(k + 1) * 128] += 1.0
        o3 = gpu_run(layer, x, e3)
        assert torch.equal(o3[:, :(k + 1) * 128], o[:, :(k + 1) * 128]), k
        assert not torch.equal(o3[:, (k + 1) * 128:], o[:, (k + 1) * 128:])


@pytest.mark.parametrize("update,group", [("linear", 1), ("linear", 2), ("mse", 1), ("mse", 2)])
def test_continuation_bitwise(update, group):
    """The first call ends on a chunk boundary (and, grouped, on a group
    boundary), so two calls run the same arithmetic as one."""
    w = BF16_SMALL.replace(n_seq=2, seq_len=5 * 128 + 50, update=update, eta=2e-3)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights, group_chunks=group)
    o = gpu_run(layer, x, e).clone()
    wf = layer.w_state.clone()
    layer.reset()
    xd, ed = x.to(DEV), e.to(DEV)
    o1 = layer.prefill(xd[:, :256].contiguous(), ed[:, :256].contiguous())
    o2 = layer.prefill(xd[:, 256:].contiguous(), ed[:, 256:].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], 1), o)
    assert torch.equal(layer.w_state, wf)


def test_batch_independence_bitwise():
    w = BF16_SMALL.replace(n_seq=3, seq_len=400)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights)
    o = gpu_run(layer, x, e).clone()
    x2, e2 = x.clone(), e.clone()
    x2[[0, 2]] += 0.5
    e2[[0, 2]] -= 0.5
    o2 = gpu_run(layer, x2, e2)
    assert torch.equal(o2[1], o[1])


@pytest.mark.parametrize("update,Bc,L,starts", [
    ("linear", 128, 900, [200, 333, 700]),
    ("mse", 64, 1500, [200, 333, 1100]),   # documents of 3-12 chunks: MSE chunk groups per document
])
def test_packed_documents(update, Bc, L, starts):
    w = BF16_SMALL.replace(n_seq=1, seq_len=L, chunk=Bc, update=update,
                           eta=1e-2 if update == "linear" else 2e-3)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights)
    layer.reset()
    o = layer.prefill_packed(x[0].to(DEV), e[0].to(DEV), starts)
    torch.cuda.synchronize()
    ow = wl.to_oracle(weights)
    O_ref, W_ref = oracle.prefill_with_resets(x[0].double().numpy(), e[0].double().numpy(), ow["W_g"],
                                              ow["W_u"], ow["conv_w"], ow["Proj"], ow["W_0"], w.eta,
                                              w.chunk, starts, update=update)
    # chunks restart at every document start
    ce = ChunkErrors("packed")
    og = o.double().cpu().numpy()
    bounds = [0, *starts, w.seq_len]
    for i in range(len(bounds) - 1):
        a, b = bounds[i], bounds[i + 1]
        for k, (s, t) in enumerate(oracle.chunk_ranges(b - a, w.chunk)):
            ce.add(i, k, a + s, og[a + s:a + t], O_ref[a + s:a + t])
    ce.check(TOL["bf16"])
    check_weights(w_pages(layer, 1), W_ref[None], TOL["bf16"], "packed")


def test_profile_records_every_kernel():
    w = BF16_SMALL.replace(n_seq=1, seq_len=512)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights)
    layer.reset()
    B.ipttt_profile_begin(layer.handle)
    layer.prefill(x.to(DEV), e.to(DEV))
    prof = B.ipttt_profile_end(layer.handle)
    for k in ("gateup", "conv", "proj", "update", "apply"):
        assert prof[k][0] >= 1 and prof[k][1] > 0, (k, prof)


@pytest.mark.parametrize("dtype,update", [("bf16", "linear"), ("bf16", "mse"), ("f32", "linear")])
def test_decode_token_by_token(dtype, update):
    """Decode T tokens one at a time (two sequences), with an earlier prefill of
    one chunk: outputs of every token and the weight after the last completed
    chunk against the oracle's token-at-a-time continuation."""
    Bc, d, F = 64, 256, 640
    w = wl.Workload("decode", 2, d, F, 64 + 2 * Bc + 9, Bc, dtype, 1e-2 if update == "linear" else 2e-3,
                    update)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    layer = make_layer(w, weights)
    layer.reset()
    xd, ed = x.to(DEV), e.to(DEV)
    o_pre = layer.prefill(xd[:, :64].contiguous(), ed[:, :64].contiguous())
    xc = torch.zeros((2, Bc, d), dtype=xd.dtype, device=DEV)
    ec = torch.zeros_like(xc)
    outs = []
    for t in range(64, w.seq_len):
        pos = (t - 64) % Bc
        xc[:, pos] = xd[:, t]
        ec[:, pos] = ed[:, t]
        outs.append(layer.decode_step(xc, ec, pos))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1).double().cpu().numpy()
    ow = wl.to_oracle(weights)
    X, E = x.double().numpy(), e.double().numpy()
    tol = TOL[dtype]
    W_ref = []
    for n in range(2):
        O_ref, W_after = oracle.decode_steps(X[n], E[n], ow["W_g"], ow["W_u"], ow["conv_w"], ow["Proj"],
                                             ow["W_0"], w.eta, Bc, update=update)
        # the decoded tokens start on a chunk boundary (position 64)
        check_chunks(o_dec[n][None], O_ref[None, 64:], Bc, tol, f"decode {dtype} {update} seq {n}")
        check_chunks(o_pre[n].double().cpu().numpy()[None], O_ref[None, :64], Bc, tol,
                     f"decode prefill {dtype} {update} seq {n}")
        W_ref.append(W_after)
    ew = rel_fro(w_pages(layer, 2), np.stack(W_ref))
    report(f"[decode] {dtype} {update}: rel_fro W={ew:.3e}")
    assert ew <= tol
