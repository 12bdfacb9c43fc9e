"""Host-only checks of the C ABI (no GPU): the library loads, exports every
entry point include/mtp_draft.h declares, and its host-side validation returns
the documented status codes before anything would be enqueued."""
import ctypes
import os
import re

import pytest
import torch

import mtp_draft_head_embed_amd as mtp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtp_draft.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(mtp_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 9, names
    L = mtp.lib()
    for n in names:
        assert hasattr(L, n), n
        # and the Python binding carries the same name
        assert hasattr(mtp, n), n


def test_status_strings():
    for code in range(8):
        assert mtp.mtp_status_str(code)
    assert mtp.mtp_status_str(99) == "unknown status"


def test_workspace_bytes():
    assert mtp.mtp_workspace_bytes(6144, 154880, 1) > 6144 * 2
    assert mtp.mtp_workspace_bytes(6144, 154880, 16) > mtp.mtp_workspace_bytes(6144, 154880, 1)
    for bad in [(0, 10, 1), (8, 10, 1), (8208, 10, 1), (24, 10, 1), (16, 0, 1), (16, 10, 0),
                (16, 10, 65), (16, 2 ** 24 + 1, 1)]:
        assert mtp.mtp_workspace_bytes(*bad) == 0, bad
    assert mtp.mtp_workspace_bytes(16, 1, 1) > 0
    assert mtp.mtp_workspace_bytes(8192, 2 ** 24, 64) > 0


def _fake_weights(H=64, V=100, eps=1e-6, **over):
    base = 0x10000
    vals = dict(embed=base, enorm_w=base * 2, hnorm_w=base * 3, head_norm_w=base * 4,
                eh_proj=base * 5, lm_head=base * 6)
    vals.update(over)
    return mtp._Weights(H, V, ctypes.c_float(eps), *[vals[k] for k in
                        ("embed", "enorm_w", "hnorm_w", "head_norm_w", "eh_proj", "lm_head")])


def _validate(w, fp8=0, q=0x70000, scale=0x80000, batch=2, tokens=0x90000, hidden=0xA0000,
              draft=0xB0000, logits=0xC0000, ws=0xD0000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = mtp.mtp_workspace_bytes(w.hidden, w.vocab, max(batch, 1)) or 1 << 20
    P = ctypes.c_void_p
    return mtp.lib().mtp_validate_draft_args(
        ctypes.byref(w) if w is not None else None, fp8, P(q) if q else None,
        P(scale) if scale else None, batch, P(tokens) if tokens else None,
        P(hidden) if hidden else None, P(draft) if draft else None,
        P(logits) if logits else None, P(ws) if ws else None, ws_bytes)


def test_validation_ok():
    assert _validate(_fake_weights()) == mtp.MTP_OK
    assert _validate(_fake_weights(), fp8=1) == mtp.MTP_OK
    assert _validate(_fake_weights(), logits=0) == mtp.MTP_OK          # logits optional
    assert _validate(_fake_weights(lm_head=0), fp8=1) == mtp.MTP_OK    # FP8 needs no lm_head


@pytest.mark.parametrize("kw,code", [
    (dict(tokens=0), mtp.MTP_ERR_NULL),
    (dict(hidden=0), mtp.MTP_ERR_NULL),
    (dict(draft=0), mtp.MTP_ERR_NULL),
    (dict(fp8=1, q=0), mtp.MTP_ERR_NULL),
    (dict(fp8=1, scale=0), mtp.MTP_ERR_NULL),
    (dict(ws=0), mtp.MTP_ERR_WORKSPACE),
    (dict(ws_bytes=16), mtp.MTP_ERR_WORKSPACE),
    (dict(tokens=0x90004), mtp.MTP_ERR_ALIGN),
    (dict(logits=0xC0002), mtp.MTP_ERR_ALIGN),
    (dict(ws=0xD0008), mtp.MTP_ERR_ALIGN),
    (dict(batch=0), mtp.MTP_ERR_SHAPE),
    (dict(batch=65), mtp.MTP_ERR_SHAPE),
])
def test_validation_errors(kw, code):
    assert _validate(_fake_weights(), **kw) == code


@pytest.mark.parametrize("over,code", [
    (dict(H=0), mtp.MTP_ERR_SHAPE), (dict(H=8), mtp.MTP_ERR_SHAPE),
    (dict(H=40), mtp.MTP_ERR_SHAPE), (dict(H=8208), mtp.MTP_ERR_SHAPE),
    (dict(V=0), mtp.MTP_ERR_SHAPE), (dict(V=-5), mtp.MTP_ERR_SHAPE),
    (dict(embed=0), mtp.MTP_ERR_NULL), (dict(eh_proj=0), mtp.MTP_ERR_NULL),
    (dict(lm_head=0), mtp.MTP_ERR_NULL), (dict(head_norm_w=0x40008), mtp.MTP_ERR_ALIGN),
])
def test_validation_weight_errors(over, code):
    H, V = over.pop("H", 64), over.pop("V", 100)
    w = _fake_weights(H=H, V=V, **over)
    assert _validate(w, ws_bytes=1 << 24) == code


def test_validation_null_weights():
    assert _validate(None, ws_bytes=1 << 20) == mtp.MTP_ERR_NULL


def test_binding_refuses_host_tensors():
    """Host tensors never reach the library: the binding raises first."""
    H, V = 16, 8
    t = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mtp.mtp_weights(t(V, H), t(H), t(H), t(H), t(H, 2 * H), t(V, H), 1e-6)


def test_context_workspace_bytes():
    assert mtp.mtp_context_workspace_bytes(6144, 1) > 0
    assert mtp.mtp_context_workspace_bytes(6144, 4096) >= 4096 * 6144 * 4
    for bad in [(6144, 0), (6144, 65537), (8, 10), (8208, 10)]:
        assert mtp.mtp_context_workspace_bytes(*bad) == 0, bad


def test_chain_workspace_and_validation():
    """Chained drafts: workspace = the sweep's plus two block outputs; a step
    count out of range or a workspace sized for one sweep is refused before
    anything is enqueued (fake device addresses are never touched)."""
    H, V, B = 64, 100, 2
    one = mtp.mtp_workspace_bytes(H, V, B)
    ch = mtp.mtp_chain_workspace_bytes(H, V, B)
    assert ch >= one + 2 * B * H * 2
    assert mtp.mtp_chain_workspace_bytes(8, V, B) == 0
    w = _fake_weights(H, V)
    P = ctypes.c_void_p
    args = lambda steps, nbytes: (ctypes.byref(w), steps, B, P(0x90000), P(0xA0000), P(0xB0000),
                                  None, P(0xD0000), nbytes, None)
    L = mtp.lib()
    assert L.mtp_draft_chain_bf16(*args(0, ch)) == mtp.MTP_ERR_SHAPE
    assert L.mtp_draft_chain_bf16(*args(65, ch)) == mtp.MTP_ERR_SHAPE
    assert L.mtp_draft_chain_bf16(*args(3, one)) == mtp.MTP_ERR_WORKSPACE
    assert L.mtp_draft_chain_fp8w(ctypes.byref(w), None, P(0x80000), 3, B, P(0x90000),
                                  P(0xA0000), P(0xB0000), None, P(0xD0000), ch,
                                  None) == mtp.MTP_ERR_NULL


def test_probe_argument_errors():
    """The streaming-read probe rejects bad arguments on the host, before any
    launch."""
    L = mtp.lib()
    P = ctypes.c_void_p
    assert L.mtp_probe_stream_read(None, 1024, P(0x1000), 2, None) == mtp.MTP_ERR_NULL
    assert L.mtp_probe_stream_read(P(0x1000), 1024, None, 2, None) == mtp.MTP_ERR_NULL
    assert L.mtp_probe_stream_read(P(0x1000), 0, P(0x2000), 2, None) == mtp.MTP_ERR_SHAPE
    assert L.mtp_probe_stream_read(P(0x1000), 1000, P(0x2000), 2, None) == mtp.MTP_ERR_SHAPE
    assert L.mtp_probe_stream_read(P(0x1000), 1024, P(0x2000), 0, None) == mtp.MTP_ERR_SHAPE
    assert L.mtp_probe_stream_read(P(0x1000), 1024, P(0x2000), 17, None) == mtp.MTP_ERR_SHAPE
    assert L.mtp_probe_stream_read(P(0x1008), 1024, P(0x2000), 2, None) == mtp.MTP_ERR_ALIGN
    assert L.mtp_probe_stream_read(P(0x1000), 1024, P(0x2002), 2, None) == mtp.MTP_ERR_ALIGN
    assert L.mtp_probe_fp8_convert(None, None) == mtp.MTP_ERR_NULL
    assert L.mtp_probe_fp8_convert(P(0x2002), None) == mtp.MTP_ERR_ALIGN


def test_static_entry_host_errors():
    """The allocation-free call rejects shapes whose workspace exceeds its
    static scratch, and bad arguments, before any device call."""
    L = mtp.lib()
    P = ctypes.c_void_p

    def call(w, q=None, s=None, batch=2, tokens=0x90000, hidden=0xA0000, draft=0xB0000):
        return L.mtp_draft_static(ctypes.byref(w) if w is not None else None,
                                  P(q) if q else None, P(s) if s else None, batch,
                                  P(tokens) if tokens else None, P(hidden) if hidden else None,
                                  P(draft) if draft else None, None, None)
    big = _fake_weights(H=8192, V=1000)
    assert mtp.mtp_workspace_bytes(8192, 1000, 64) > mtp.MTP_STATIC_SCRATCH_BYTES
    assert call(big, batch=64) == mtp.MTP_ERR_SCRATCH
    assert mtp.mtp_workspace_bytes(6144, 154880, 32) <= mtp.MTP_STATIC_SCRATCH_BYTES
    w = _fake_weights()
    assert call(None) == mtp.MTP_ERR_NULL
    assert call(w, q=0x70000) == mtp.MTP_ERR_NULL          # q without scale
    assert call(w, s=0x80000) == mtp.MTP_ERR_NULL          # scale without q
    assert call(w, tokens=0) == mtp.MTP_ERR_NULL
    assert call(w, hidden=0xA0008) == mtp.MTP_ERR_ALIGN
    assert call(w, batch=0) == mtp.MTP_ERR_SHAPE
    assert call(_fake_weights(lm_head=0)) == mtp.MTP_ERR_NULL  # the BF16 head needs lm_head
    assert "static scratch" in mtp.mtp_status_str(mtp.MTP_ERR_SCRATCH)


def test_library_imports_no_allocator():
    """No entry point can allocate: the library does not even import the HIP
    runtime's allocation functions."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", mtp.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert any(sym.startswith("hipLaunchKernel") or sym == "hipGetLastError" for sym in syms)
    bad = [sym for sym in syms if sym.startswith(("hipMalloc", "hipFree", "hipHostMalloc",
                                                  "hipHostFree", "hipExtMalloc", "hipMemAlloc"))]
    assert not bad, bad
