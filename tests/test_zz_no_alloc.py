"""The allocation-free prefill (ipttt_prefill_layer_noalloc: workspace in the
library's fixed per-device scratch area) against the regular entry point
(ipttt_prefill_layer: the descriptor's workspace), through the C ABI.

Each case makes two calls in a row on one handle, the second with a smaller
input, each compared with the regular entry point on the same inputs: every
chunk's O and every final fast weight within the bf16 bar (2e-2 relative
Frobenius error; the kernels are the same, so the results are expected to be
bit-identical unless the scratch area changes the chunk grouping). The scratch
area keeps the previous call's contents, so the second, smaller call also
checks that nothing relies on it starting at zero. A batch whose single chunk
needs more than the scratch area is rejected before any device work.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from chunked_weight_mlp_amd import ipttt as B
from parity_check import check_chunks, check_weights, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def both(layer, x, e):
    """(o, W) from the regular entry point, then from the allocation-free one."""
    n, L = x.shape[0], x.shape[1]
    out = []
    for fn in (B.ipttt_prefill_layer, B.ipttt_prefill_layer_noalloc):
        layer.reset()
        o = torch.full((n, L, x.shape[2]), float("nan"), dtype=torch.float32, device=DEV)
        fn(layer.handle, x, e, o, n, L)
        torch.cuda.synchronize()
        out.append((o.double().cpu().numpy(), layer.w_state[:n].double().cpu().numpy()))
    return out


@pytest.mark.parametrize("shape,update,calls", [
    # 4B-shaped layer: one chunk needs ~80 MB, so the 256 MiB scratch area runs
    # the 9-chunk call in several passes; then a 3-chunk call
    ((2560, 9728, 1024), "linear", [(1, 8 * 1024 + 300), (1, 2 * 1024 + 5)]),
    ((256, 640, 128), "linear", [(2, 1500), (1, 333)]),
    ((256, 640, 64), "linear", [(2, 2100), (2, 77)]),     # chunk groups of 16
    ((256, 640, 128), "mse", [(2, 1000), (1, 260)]),
])
def test_noalloc_matches_prefill_layer(shape, update, calls):
    d, F, Bc = shape
    w = wl.Workload("noalloc", max(n for n, _ in calls), d, F, max(L for _, L in calls), Bc, "bf16",
                    1e-3 if d > 1000 else (1e-2 if update == "linear" else 2e-3), update)
    weights = {k: v.to(DEV) for k, v in wl.make_weights(w).items()}
    layer = B.Layer(**weights, chunk=Bc, eta=w.eta, update=update, max_batch=w.n_seq,
                    max_seq_len=w.seq_len)
    try:
        for i, (n, L) in enumerate(calls):
            x, e = wl.make_inputs(w, seq_len=L, n_seq=n, seed_offset=i)
            (o_ref, w_ref), (o_na, w_na) = both(layer, x.to(DEV), e.to(DEV))
            same = np.array_equal(o_ref, o_na) and np.array_equal(w_ref, w_na)
            say(f"[noalloc] d={d} F={F} B={Bc} {update} call {i}: N={n} L={L}, bit-identical={same}")
            assert np.isfinite(o_na).all()
            check_chunks(o_na, o_ref, Bc, TOL, f"noalloc call {i}")
            check_weights(w_na.transpose(0, 2, 1), w_ref.transpose(0, 2, 1), TOL, f"noalloc call {i}")
    finally:
        layer.close()


def test_noalloc_rejects_batches_beyond_the_scratch_area():
    """One 4096-token chunk of two 4B-shaped sequences needs more workspace than
    the fixed scratch area holds: IPTTT_E_WORKSPACE, nothing written."""
    w = wl.Workload("noalloc_big", 2, 2560, 9728, 4096, 4096, "bf16", 1e-3, "linear")
    need = B.ipttt_workspace_bytes(B.LayerDesc(d=w.d, d_ff=w.d_ff, conv_k=4, chunk=w.chunk,
                                               max_batch=2, eta=w.eta, update=0, in_dtype=1), 2, 1)
    assert need > B.IPTTT_NOALLOC_SCRATCH_BYTES
    weights = {k: v.to(DEV) for k, v in wl.make_weights(w).items()}
    layer = B.Layer(**weights, chunk=w.chunk, eta=w.eta, max_batch=2, slab_chunks=1)
    try:
        layer.reset()
        x = torch.zeros((2, 64, w.d), dtype=torch.bfloat16, device=DEV)
        o = torch.full((2, 64, w.d), 7.0, dtype=torch.float32, device=DEV)
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_layer_noalloc(layer.handle, x, x, o, 2, 64)
        assert ei.value.status == B.IPTTT_E_WORKSPACE and "scratch" in str(ei.value)
        torch.cuda.synchronize()
        assert bool((o == 7.0).all())
        # one sequence fits
        B.ipttt_prefill_layer_noalloc(layer.handle, x[:1].contiguous(), x[:1].contiguous(), o[:1], 1, 64)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o[0]).all())
    finally:
        layer.close()
