"""C-ABI checks that need no GPU: the library loads, exports every function that
include/ipttt.h declares, the descriptor layout agrees with the C compiler's, and
every argument error is reported before any device work."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from chunked_weight_mlp_amd import ipttt as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ipttt.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libipttt.so is not built: run __graft_entry__.build()")
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ipttt_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (ipttt_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        assert hasattr(lib, f)


def test_descriptor_layout_matches_c(tmp_path):
    fields = [f for f, _ in B.LayerDesc._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){",
           'printf("%zu\\n", sizeof(ipttt_layer_desc));']
    src += [f'printf("%zu\\n", offsetof(ipttt_layer_desc, {f}));' for f in fields]
    src += ["return 0;}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(c), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(B.LayerDesc)
    assert vals[1:] == [getattr(B.LayerDesc, f).offset for f in fields]


def test_status_strings(lib):
    for code, name in [(0, "IPTTT_OK"), (-1, "IPTTT_E_INVALID"), (-2, "IPTTT_E_UNSUPPORTED"),
                       (-3, "IPTTT_E_HIP"), (-4, "IPTTT_E_STATE"), (-5, "IPTTT_E_WORKSPACE")]:
        assert B.ipttt_status_str(code) == name
    assert B.ipttt_status_str(7) == "IPTTT_E_UNKNOWN"


# --- fake device memory: aligned host buffers; nothing below touches the device ---

class FakeMem:
    def __init__(self):
        self.bufs = []

    def ptr(self, nbytes=4096, offset=0):
        b = ctypes.create_string_buffer(nbytes + 512)
        self.bufs.append(b)
        return (ctypes.addressof(b) + 255) // 256 * 256 + offset


def make_desc(mem, ws_bytes=None, **kw):
    d = dict(d=64, d_ff=256, conv_k=4, chunk=128, max_batch=2, eta=0.01, update=0, in_dtype=1,
             flags=0)
    d.update(kw)
    desc = B.LayerDesc(**d)
    for f in ("w_gate", "w_up", "proj", "conv_w", "w0", "w_state"):
        setattr(desc, f, mem.ptr())
    need = B.ipttt_workspace_bytes(desc, 1, 1)
    desc.workspace_bytes = need if ws_bytes is None else ws_bytes
    desc.workspace = mem.ptr()
    return desc


def init_status(desc):
    h = ctypes.c_void_p()
    s = B.load().ipttt_init(ctypes.byref(desc) if desc is not None else None, ctypes.byref(h))
    if s == 0:
        B.ipttt_destroy(h)
    return s


def test_workspace_bytes(lib):
    mem = FakeMem()
    desc = make_desc(mem)
    one = B.ipttt_workspace_bytes(desc, 1, 1)
    assert one > 0
    assert B.ipttt_workspace_bytes(desc, 1, 4) > one
    assert B.ipttt_workspace_bytes(desc, 2, 1) > one
    assert B.ipttt_workspace_bytes(desc, 0, 1) == 0
    assert B.ipttt_workspace_bytes(desc, 1, 0) == 0
    assert B.ipttt_workspace_bytes(make_desc(mem, d=0), 1, 1) == 0
    mse = make_desc(mem, update=1)
    assert B.ipttt_workspace_bytes(mse, 1, 4) > 0


def test_workspace_bytes_of_chunk_groups(lib):
    """Groups of G chunks share one W snapshot and add a (G Bp)^2 Gram buffer
    (linear rule); the MSE rule's groups add the Gram buffer and residual rows."""
    mem = FakeMem()
    d, F, Bc = 64, 256, 64
    el = 2
    snap = d * F * el
    plain = B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=1), 1, 8)
    grouped = B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=4), 1, 8)
    # 8 snapshots -> 2, plus 2 groups of (4 * 64)^2 Gram entries
    assert grouped - plain == -6 * snap + 2 * (4 * Bc) ** 2 * el
    # a slab shorter than a group uses groups of the slab's length
    one = B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=4), 1, 1)
    assert one == B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=1), 1, 1)
    # default: about 1024 padded rows per group (16 chunks of 64)
    auto = B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=0), 1, 32)
    g16 = B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=16), 1, 32)
    assert auto == g16
    # the generic kernels and fp32 layers keep one snapshot per chunk
    for kw in (dict(flags=B.IPTTT_FLAG_GENERIC_KERNELS), dict(in_dtype=0)):
        assert (B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=4, **kw), 1, 8) ==
                B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=1, **kw), 1, 8))
    # the MSE rule keeps one copy of W either way; its groups hold the residuals
    # of all their rows (d x G Bp) and the Gram buffer
    mse1 = B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=1, update=1), 1, 8)
    mse4 = B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=4, update=1), 1, 8)
    assert mse4 - mse1 == 3 * d * Bc * el + 2 * (4 * Bc) ** 2 * el
    # default: about 2048 padded rows per group (32 chunks of 64)
    assert (B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=0, update=1), 1, 64) ==
            B.ipttt_workspace_bytes(make_desc(mem, chunk=Bc, group_chunks=32, update=1), 1, 64))


@pytest.mark.parametrize("kw,status", [
    (dict(d=0), B.IPTTT_E_INVALID),
    (dict(d_ff=-3), B.IPTTT_E_INVALID),
    (dict(chunk=0), B.IPTTT_E_INVALID),
    (dict(conv_k=0), B.IPTTT_E_INVALID),
    (dict(conv_k=9), B.IPTTT_E_UNSUPPORTED),
    (dict(max_batch=0), B.IPTTT_E_INVALID),
    (dict(in_dtype=5), B.IPTTT_E_UNSUPPORTED),
    (dict(update=3), B.IPTTT_E_UNSUPPORTED),
    (dict(flags=0x80), B.IPTTT_E_INVALID),
    (dict(eta=float("nan")), B.IPTTT_E_INVALID),
    (dict(eta=float("inf")), B.IPTTT_E_INVALID),
    (dict(group_chunks=-1), B.IPTTT_E_INVALID),
    (dict(group_chunks=33), B.IPTTT_E_UNSUPPORTED),   # 33 x 128 padded rows > 4096
])
def test_init_rejects_bad_sizes(lib, kw, status):
    mem = FakeMem()
    assert init_status(make_desc(mem, **kw)) == status
    assert B.ipttt_last_error().startswith(B.ipttt_status_str(status))


def test_init_rejects_null_and_misaligned_pointers(lib):
    mem = FakeMem()
    assert init_status(None) == B.IPTTT_E_INVALID
    for f in ("w_gate", "w_up", "proj", "conv_w", "w0", "w_state", "workspace"):
        desc = make_desc(mem)
        setattr(desc, f, None)
        assert init_status(desc) == B.IPTTT_E_INVALID
        assert f in B.ipttt_last_error()
        desc = make_desc(mem)
        setattr(desc, f, getattr(desc, f) + 8)
        assert init_status(desc) == B.IPTTT_E_INVALID
    desc = make_desc(mem)
    desc.workspace = desc.workspace + 64  # 16- but not 256-byte aligned
    assert init_status(desc) == B.IPTTT_E_INVALID
    assert lib.ipttt_init(ctypes.byref(make_desc(mem)), None) == B.IPTTT_E_INVALID


def test_init_rejects_small_workspace(lib):
    mem = FakeMem()
    desc = make_desc(mem)
    desc.workspace_bytes -= 1
    assert init_status(desc) == B.IPTTT_E_WORKSPACE


def test_prefill_errors_before_device_work(lib):
    mem = FakeMem()
    desc = make_desc(mem)
    h = B.ipttt_init(desc)
    x, e, o = mem.ptr(), mem.ptr(), mem.ptr()
    try:
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_layer(h, x, e, o, 3, 128, stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID and "max_batch" in str(ei.value)
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_layer(h, x, e, o, 1, 128, stream=0)
        assert ei.value.status == B.IPTTT_E_STATE and "never reset" in str(ei.value)
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_layer(h, x, e, o, -1, 128, stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_layer(h, None, e, o, 1, 128, stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_layer(h, x + 1, e, o, 1, 128, stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID
        # empty calls are successful no-ops
        B.ipttt_prefill_layer(h, x, e, o, 0, 128, stream=0)
        B.ipttt_prefill_layer(h, x, e, o, 1, 0, stream=0)
        # packed documents
        for starts in ([0], [128], [5, 5], [9, 3], [-1]):
            with pytest.raises(B.IptttError) as ei:
                B.ipttt_prefill_packed(h, x, e, o, 0, 128, starts, stream=0)
            assert ei.value.status == B.IPTTT_E_INVALID
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_packed(h, x, e, o, 0, 128, [7], stream=0)
        assert ei.value.status == B.IPTTT_E_STATE
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_prefill_packed(h, x, e, o, 2, 128, [], stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID
        # reset range
        for first, n in ((-1, 1), (0, 3), (2, 1), (1, -1)):
            with pytest.raises(B.IptttError) as ei:
                B.ipttt_reset_fast_weights(h, first, n, stream=0)
            assert ei.value.status == B.IPTTT_E_INVALID
        B.ipttt_reset_fast_weights(h, 1, 0, stream=0)  # empty range: no device work
    finally:
        B.ipttt_destroy(h)
    B.ipttt_destroy(None)


def test_null_handle(lib):
    assert lib.ipttt_prefill_layer(None, None, None, None, 1, 1, None) == B.IPTTT_E_INVALID
    assert lib.ipttt_prefill_layer_noalloc(None, None, None, None, 1, 1, None) == B.IPTTT_E_INVALID
    assert lib.ipttt_reset_fast_weights(None, 0, 1, None) == B.IPTTT_E_INVALID
    assert lib.ipttt_prefill_packed(None, None, None, None, 0, 1, None, 0, None) == B.IPTTT_E_INVALID


def test_decode_errors_before_device_work(lib):
    mem = FakeMem()
    desc = make_desc(mem)
    h = B.ipttt_init(desc)
    x, e, o = mem.ptr(), mem.ptr(), mem.ptr()
    try:
        for pos in (-1, 128):
            with pytest.raises(B.IptttError) as ei:
                B.ipttt_decode_step(h, x, e, 128 * 64, pos, o, 1, stream=0)
            assert ei.value.status == B.IPTTT_E_INVALID and "pos" in str(ei.value)
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_decode_step(h, x, e, 128 * 64, 0, o, 3, stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_decode_step(h, x, e, 64, 5, o, 2, stream=0)   # stride shorter than the chunk so far
        assert ei.value.status == B.IPTTT_E_INVALID
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_decode_step(h, x, e, 128 * 64, 3, o, 1, stream=0)
        assert ei.value.status == B.IPTTT_E_STATE
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_decode_step(h, None, e, 128 * 64, 3, o, 1, stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID
        B.ipttt_decode_step(h, x, e, 128 * 64, 3, o, 0, stream=0)   # empty batch: no-op
    finally:
        B.ipttt_destroy(h)


def test_backward_workspace_bytes(lib):
    mem = FakeMem()
    desc = make_desc(mem)
    one = B.ipttt_backward_workspace_bytes(desc, 1, 128)
    assert one > 0
    assert B.ipttt_backward_workspace_bytes(desc, 2, 128) > one
    assert B.ipttt_backward_workspace_bytes(desc, 1, 129) > one
    assert B.ipttt_backward_workspace_bytes(desc, 0, 128) == 0
    assert B.ipttt_backward_workspace_bytes(desc, 1, 0) == 0
    # only bf16 layers on the MFMA path have a backward (either rule)
    assert B.ipttt_backward_workspace_bytes(make_desc(mem, update=1), 1, 128) > one
    for kw in (dict(in_dtype=0), dict(flags=B.IPTTT_FLAG_GENERIC_KERNELS)):
        assert B.ipttt_backward_workspace_bytes(make_desc(mem, **kw), 1, 128) == 0


def test_backward_errors_before_device_work(lib):
    mem = FakeMem()
    names = [k for k, _ in B.Grads._fields_]

    def grads(**over):
        g = {k: mem.ptr() for k in names}
        g.update(over)
        return g

    desc = make_desc(mem)
    h = B.ipttt_init(desc)
    x, e, do = mem.ptr(), mem.ptr(), mem.ptr()
    need = B.ipttt_backward_workspace_bytes(desc, 1, 128)
    ws = mem.ptr(64)
    try:
        def call(batch=1, L=128, g=None, w=ws, wb=need, xx=x, dd=do, dwf=None):
            return B.ipttt_backward_layer(h, xx, e, dd, dwf, batch, L, g or grads(), w, wb, stream=0)

        for kw, status in ((dict(batch=0), B.IPTTT_E_INVALID), (dict(L=0), B.IPTTT_E_INVALID),
                           (dict(batch=3), B.IPTTT_E_INVALID), (dict(xx=x + 2), B.IPTTT_E_INVALID),
                           (dict(dd=None), B.IPTTT_E_INVALID), (dict(w=None), B.IPTTT_E_INVALID),
                           (dict(w=ws + 64), B.IPTTT_E_INVALID),
                           (dict(wb=need - 1), B.IPTTT_E_WORKSPACE),
                           (dict(dwf=do + 2), B.IPTTT_E_INVALID)):
            with pytest.raises(B.IptttError) as ei:
                call(**kw)
            assert ei.value.status == status, kw
        for k in names:
            for bad in (None, mem.ptr() + 2):
                with pytest.raises(B.IptttError) as ei:
                    call(g=grads(**{k: bad}))
                assert ei.value.status == B.IPTTT_E_INVALID and k in str(ei.value)
        with pytest.raises(B.IptttError) as ei:
            B.ipttt_backward_layer(h, x, e, do, None, 1, 128, None, ws, need, stream=0)
        assert ei.value.status == B.IPTTT_E_INVALID
    finally:
        B.ipttt_destroy(h)
    for kw in (dict(in_dtype=0), dict(flags=B.IPTTT_FLAG_GENERIC_KERNELS)):
        h = B.ipttt_init(make_desc(mem, **kw))
        try:
            with pytest.raises(B.IptttError) as ei:
                B.ipttt_backward_layer(h, x, e, do, None, 1, 128, grads(), ws, 1 << 30, stream=0)
            assert ei.value.status == B.IPTTT_E_UNSUPPORTED
        finally:
            B.ipttt_destroy(h)
    assert lib.ipttt_backward_layer(None, None, None, None, None, 1, 1, None, None, 0, None) == \
        B.IPTTT_E_INVALID


def test_probe_library_errors_before_device_work():
    """The measurement library (its own ABI, include/ipttt_probe.h) rejects bad
    arguments, including sources shorter than a probe reads, before touching
    the device."""
    from chunked_weight_mlp_amd import probe as P
    if not os.path.exists(P.LIB_PATH):
        pytest.fail("libipttt_probe.so is not built: run __graft_entry__.build()")
    lib = P.load()
    hdr = open(os.path.join(ROOT, "include", "ipttt_probe.h")).read()
    assert sorted(set(re.findall(r"\b(ipttt_[a-z_]+)\s*\(", re.sub(r"/\*.*?\*/", "", hdr,
                                                                     flags=re.S)))) == list(P.EXPORTS)
    mem = FakeMem()
    buf = mem.ptr()
    big = 1 << 20
    for kind, n, src, src_bytes, dst, work_ok in (
            (7, 10, None, 0, buf, True),                          # unknown kind
            (P.IPTTT_PROBE_MFMA16, 0, None, 0, buf, True),        # n < 1
            (P.IPTTT_PROBE_MFMA32, 10, None, 0, None, True),      # no dst
            (P.IPTTT_PROBE_MFMA32, 10, None, 0, buf + 8, True),   # misaligned dst
            (P.IPTTT_PROBE_READ, 16, None, big, buf, True),       # read without src
            (P.IPTTT_PROBE_READ, 32, buf, 16, buf, True),         # reads past src
            (P.IPTTT_PROBE_READ, 24, buf, big, buf, True),        # n not a multiple of 16
            (P.IPTTT_PROBE_LDS, 0, None, 0, buf, True),           # n < 1
            (P.IPTTT_PROBE_LDS, 10, None, 0, None, True),         # no dst
            (P.IPTTT_PROBE_COPY, 10, None, 4 << 20, buf, True),   # copy without src
            (P.IPTTT_PROBE_COPY, 10, buf + 8, 4 << 20, buf, True),  # misaligned src
            (P.IPTTT_PROBE_COPY, 10, buf, (4 << 20) - 16, buf, True),  # src below 4 MiB
            (P.IPTTT_PROBE_MFMA16, 10, None, 0, buf, False)):     # no work
        work = ctypes.byref(ctypes.c_double()) if work_ok else None
        assert lib.ipttt_probe(kind, n, src, src_bytes, dst, 1 << 20, work, None) == \
            B.IPTTT_E_INVALID, (kind, n, src_bytes)
