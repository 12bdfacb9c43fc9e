"""Python binding of libmtpdraft.so (the MTP draft sweep on MI355X / gfx950).

Argument marshalling only: every function here has the name of a C entry point
in include/mtp_draft.h, checks that the torch tensors it is handed are device
tensors of the right dtype and at least the size the call will touch, and
passes their addresses and the current HIP stream through ctypes.  Every step
of the sweep runs in the library's HIP kernels; there is no fallback.  If the
shared library is missing and cannot be built, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "MTP_OK", "MTP_ERR_NULL", "MTP_ERR_SHAPE", "MTP_ERR_ALIGN", "MTP_ERR_WORKSPACE",
    "MTP_ERR_NONFINITE", "MTP_ERR_HIP", "MTP_ERR_SCRATCH", "MTP_STATIC_SCRATCH_BYTES",
    "MTP_DRAFT_INVALID", "MtpError", "mtp_weights",
    "lib", "lib_path", "mtp_workspace_bytes", "mtp_validate_draft_args",
    "mtp_quantize_head_fp8", "mtp_draft_bf16", "mtp_draft_fp8w", "mtp_front", "mtp_head_bf16",
    "mtp_head_fp8w", "mtp_status_str", "new_workspace", "mtp_context_workspace_bytes",
    "mtp_context_rows", "mtp_probe_stream_read", "mtp_probe_fp8_convert", "mtp_draft_static",
]

MTP_OK, MTP_ERR_NULL, MTP_ERR_SHAPE, MTP_ERR_ALIGN = 0, 1, 2, 3
MTP_ERR_WORKSPACE, MTP_ERR_NONFINITE, MTP_ERR_HIP, MTP_ERR_SCRATCH = 4, 5, 6, 7
MTP_STATIC_SCRATCH_BYTES = 16 << 20
MTP_DRAFT_INVALID = 0xFFFFFFFF

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmtpdraft.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB_PATH


class MtpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({mtp_status_str(status)})")


class _Weights(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("embed", ctypes.c_void_p), ("enorm_w", ctypes.c_void_p), ("hnorm_w", ctypes.c_void_p),
        ("head_norm_w", ctypes.c_void_p), ("eh_proj", ctypes.c_void_p),
        ("lm_head", ctypes.c_void_p),
    ]


def lib():
    """Load libmtpdraft.so (building it with hipcc only if it is absent)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        W = ctypes.POINTER(_Weights)
        sigs = {
            "mtp_workspace_bytes": ([i32, i32, i32], sz),
            "mtp_validate_draft_args": ([W, ctypes.c_int, P, P, i32, P, P, P, P, P, sz], ctypes.c_int),
            "mtp_quantize_head_fp8": ([P, i32, i32, P, P, P, sz, P], ctypes.c_int),
            "mtp_draft_bf16": ([W, i32, P, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_draft_fp8w": ([W, P, P, i32, P, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_draft_static": ([W, P, P, i32, P, P, P, P, P], ctypes.c_int),
            "mtp_front": ([W, i32, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_head_bf16": ([W, i32, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_head_fp8w": ([W, P, P, i32, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "mtp_context_workspace_bytes": ([i32, i32], sz),
            "mtp_context_rows": ([W, i32, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_chain_workspace_bytes": ([i32, i32, i32], sz),
            "mtp_draft_chain_bf16": ([W, i32, i32, P, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_draft_chain_fp8w": ([W, P, P, i32, i32, P, P, P, P, P, sz, P], ctypes.c_int),
            "mtp_probe_stream_read": ([P, sz, P, i32, P], ctypes.c_int),
            "mtp_probe_fp8_convert": ([P, P], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
        return L


def mtp_status_str(status: int) -> str:
    return lib().mtp_status_str(int(status)).decode()


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _dev(t: torch.Tensor | None, name: str, dtype: torch.dtype, min_numel: int,
         optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {min_numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc: int, where: str):
    if rc != MTP_OK:
        raise MtpError(rc, where)


class mtp_weights:
    """The C struct ``mtp_weights`` plus references to the tensors it points
    at (so they stay alive as long as this object).  All tensors are BF16 on
    the device: embed [V][H], enorm_w/hnorm_w/head_norm_w [H], eh_proj [H][2H],
    lm_head [V][H] (may be None when only the FP8 head is used)."""

    def __init__(self, embed, enorm_w, hnorm_w, head_norm_w, eh_proj, lm_head, rms_eps: float):
        V, H = embed.shape
        bf = torch.bfloat16
        self.hidden, self.vocab, self.rms_eps = int(H), int(V), float(rms_eps)
        self._keep = (embed, enorm_w, hnorm_w, head_norm_w, eh_proj, lm_head)
        self.c = _Weights(
            self.hidden, self.vocab, ctypes.c_float(self.rms_eps),
            _dev(embed, "embed", bf, V * H), _dev(enorm_w, "enorm_w", bf, H),
            _dev(hnorm_w, "hnorm_w", bf, H), _dev(head_norm_w, "head_norm_w", bf, H),
            _dev(eh_proj, "eh_proj", bf, 2 * H * H),
            _dev(lm_head, "lm_head", bf, V * H, optional=True),
        )

    def ref(self):
        return ctypes.byref(self.c)


def mtp_workspace_bytes(hidden: int, vocab: int, batch: int) -> int:
    return int(lib().mtp_workspace_bytes(hidden, vocab, batch))


def new_workspace(hidden: int, vocab: int, batch: int, device="cuda") -> torch.Tensor:
    n = mtp_workspace_bytes(hidden, vocab, batch)
    if n == 0:
        raise MtpError(MTP_ERR_SHAPE, "new_workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mtp_validate_draft_args(w: mtp_weights, fp8: bool, q, scale, batch: int, tokens, hidden,
                            draft, logits, workspace) -> int:
    """Host-only check (touches no device); returns the status code."""
    def addr(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())
    return int(lib().mtp_validate_draft_args(
        w.ref(), int(bool(fp8)), addr(q), addr(scale), batch, addr(tokens), addr(hidden),
        addr(draft), addr(logits), addr(workspace),
        0 if workspace is None else workspace.numel()))


def mtp_quantize_head_fp8(lm_head, vocab: int, hidden: int, q, scale, workspace,
                          stream=None) -> None:
    """Fill q (uint8 [V][H]) and scale (float32 [V]); raises MtpError with
    status MTP_ERR_NONFINITE when a weight is NaN or Inf."""
    n = vocab * hidden
    rc = lib().mtp_quantize_head_fp8(
        _dev(lm_head, "lm_head", torch.bfloat16, n), vocab, hidden,
        _dev(q, "q", torch.uint8, n), _dev(scale, "scale", torch.float32, vocab),
        _dev(workspace, "workspace", torch.uint8, 256), workspace.numel(), _stream(stream))
    _check(rc, "mtp_quantize_head_fp8")


def _draft_common(w, batch, tokens, hidden, draft, logits, workspace):
    H, V = w.hidden, w.vocab
    return (
        _dev(tokens, "tokens", torch.int32, batch) if tokens.dtype == torch.int32
        else _dev(tokens, "tokens", torch.uint32, batch),
        _dev(hidden, "hidden", torch.bfloat16, batch * H),
        _dev(draft, "draft", torch.int32, batch) if draft.dtype == torch.int32
        else _dev(draft, "draft", torch.uint32, batch),
        _dev(logits, "logits", torch.bfloat16, batch * V, optional=True),
        _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(),
    )


def mtp_draft_bf16(w: mtp_weights, batch: int, tokens, hidden, draft, logits, workspace,
                   stream=None) -> None:
    """Enqueue one draft per sequence (BF16 lm_head).  tokens/draft are
    int32 or uint32 [B] device tensors (u32 semantics), hidden BF16 [B][H],
    logits BF16 [B][V] or None."""
    t, h, d, lg, ws, nws = _draft_common(w, batch, tokens, hidden, draft, logits, workspace)
    _check(lib().mtp_draft_bf16(w.ref(), batch, t, h, d, lg, ws, nws, _stream(stream)),
           "mtp_draft_bf16")


def mtp_draft_fp8w(w: mtp_weights, q, scale, batch: int, tokens, hidden, draft, logits,
                   workspace, stream=None) -> None:
    t, h, d, lg, ws, nws = _draft_common(w, batch, tokens, hidden, draft, logits, workspace)
    n = w.vocab * w.hidden
    _check(lib().mtp_draft_fp8w(w.ref(), _dev(q, "q", torch.uint8, n),
                                _dev(scale, "scale", torch.float32, w.vocab), batch, t, h, d, lg,
                                ws, nws, _stream(stream)), "mtp_draft_fp8w")


def mtp_draft_static(w: mtp_weights, q, scale, batch: int, tokens, hidden, draft, logits,
                     stream=None) -> None:
    """The allocation-free draft call: the BF16 head when q and scale are
    None, else the FP8 copy; the library's static scratch replaces the
    workspace (calls that overlap on one GPU race)."""
    H, V = w.hidden, w.vocab
    t = (_dev(tokens, "tokens", torch.int32, batch) if tokens.dtype == torch.int32
         else _dev(tokens, "tokens", torch.uint32, batch))
    d = (_dev(draft, "draft", torch.int32, batch) if draft.dtype == torch.int32
         else _dev(draft, "draft", torch.uint32, batch))
    n = V * H
    _check(lib().mtp_draft_static(
        w.ref(), _dev(q, "q", torch.uint8, n, optional=True),
        _dev(scale, "scale", torch.float32, V, optional=True), batch, t,
        _dev(hidden, "hidden", torch.bfloat16, batch * H), d,
        _dev(logits, "logits", torch.bfloat16, batch * V, optional=True), _stream(stream)),
        "mtp_draft_static")


def mtp_front(w: mtp_weights, batch: int, tokens, hidden, x, workspace, stream=None) -> None:
    H = w.hidden
    t = (_dev(tokens, "tokens", torch.int32, batch) if tokens.dtype == torch.int32
         else _dev(tokens, "tokens", torch.uint32, batch))
    _check(lib().mtp_front(w.ref(), batch, t, _dev(hidden, "hidden", torch.bfloat16, batch * H),
                           _dev(x, "x", torch.bfloat16, batch * H),
                           _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(),
                           _stream(stream)), "mtp_front")


def mtp_head_bf16(w: mtp_weights, batch: int, x, draft, logits, workspace, stream=None) -> None:
    H, V = w.hidden, w.vocab
    d = (_dev(draft, "draft", torch.int32, batch) if draft.dtype == torch.int32
         else _dev(draft, "draft", torch.uint32, batch))
    _check(lib().mtp_head_bf16(w.ref(), batch, _dev(x, "x", torch.bfloat16, batch * H), d,
                               _dev(logits, "logits", torch.bfloat16, batch * V, optional=True),
                               _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(),
                               _stream(stream)), "mtp_head_bf16")


def mtp_head_fp8w(w: mtp_weights, q, scale, batch: int, x, draft, logits, workspace,
                  stream=None) -> None:
    H, V = w.hidden, w.vocab
    d = (_dev(draft, "draft", torch.int32, batch) if draft.dtype == torch.int32
         else _dev(draft, "draft", torch.uint32, batch))
    _check(lib().mtp_head_fp8w(w.ref(), _dev(q, "q", torch.uint8, V * H),
                               _dev(scale, "scale", torch.float32, V), batch,
                               _dev(x, "x", torch.bfloat16, batch * H), d,
                               _dev(logits, "logits", torch.bfloat16, batch * V, optional=True),
                               _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(),
                               _stream(stream)), "mtp_head_fp8w")


def mtp_context_workspace_bytes(hidden: int, rows: int) -> int:
    return int(lib().mtp_context_workspace_bytes(hidden, rows))


def mtp_context_rows(w: mtp_weights, rows: int, tokens, hiddens, x, workspace,
                     stream=None) -> None:
    """Enqueue the front half for T context rows: row r pairs the embedding of
    tokens[r + 1] with hiddens[r].  tokens int32/uint32 [T + 1], hiddens BF16
    [T][H], x BF16 [T][H] (written)."""
    H = w.hidden
    t = (_dev(tokens, "tokens", torch.int32, rows + 1) if tokens.dtype == torch.int32
         else _dev(tokens, "tokens", torch.uint32, rows + 1))
    _check(lib().mtp_context_rows(w.ref(), rows, t,
                                  _dev(hiddens, "hiddens", torch.bfloat16, rows * H),
                                  _dev(x, "x", torch.bfloat16, rows * H),
                                  _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(),
                                  _stream(stream)), "mtp_context_rows")


def mtp_chain_workspace_bytes(hidden: int, vocab: int, batch: int) -> int:
    return int(lib().mtp_chain_workspace_bytes(hidden, vocab, batch))


def _chain_common(w, steps, batch, tokens, hidden, drafts, logits, workspace):
    H, V = w.hidden, w.vocab
    return (
        _dev(tokens, "tokens", torch.int32, batch) if tokens.dtype == torch.int32
        else _dev(tokens, "tokens", torch.uint32, batch),
        _dev(hidden, "hidden", torch.bfloat16, batch * H),
        _dev(drafts, "drafts", torch.int32, steps * batch) if drafts.dtype == torch.int32
        else _dev(drafts, "drafts", torch.uint32, steps * batch),
        _dev(logits, "logits", torch.bfloat16, steps * batch * V, optional=True),
        _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(),
    )


def mtp_draft_chain_bf16(w: mtp_weights, steps: int, batch: int, tokens, hidden, drafts, logits,
                         workspace, stream=None) -> None:
    """Enqueue `steps` chained drafts per sequence (BF16 lm_head): step k + 1
    takes step k's draft and block output.  drafts int32/uint32 [K][B],
    logits BF16 [K][B][V] or None."""
    t, h, d, lg, ws, nws = _chain_common(w, steps, batch, tokens, hidden, drafts, logits,
                                         workspace)
    _check(lib().mtp_draft_chain_bf16(w.ref(), steps, batch, t, h, d, lg, ws, nws,
                                      _stream(stream)), "mtp_draft_chain_bf16")


def mtp_draft_chain_fp8w(w: mtp_weights, q, scale, steps: int, batch: int, tokens, hidden,
                         drafts, logits, workspace, stream=None) -> None:
    """As mtp_draft_chain_bf16 with the FP8 copy of lm_head (q, scale)."""
    t, h, d, lg, ws, nws = _chain_common(w, steps, batch, tokens, hidden, drafts, logits,
                                         workspace)
    n = w.vocab * w.hidden
    _check(lib().mtp_draft_chain_fp8w(w.ref(), _dev(q, "q", torch.uint8, n),
                                      _dev(scale, "scale", torch.float32, w.vocab), steps, batch,
                                      t, h, d, lg, ws, nws, _stream(stream)),
           "mtp_draft_chain_fp8w")


def mtp_probe_stream_read(buf, out, wg_per_cu: int = 2, stream=None) -> None:
    """A plain streaming read of the device tensor `buf` (a measurement aid:
    the practical HBM ceiling the weight sweeps are compared with).  `out` is
    a device int32/uint32 tensor of at least one element."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    o = (_dev(out, "out", torch.int32, 1) if out.dtype == torch.int32
         else _dev(out, "out", torch.uint32, 1))
    _check(lib().mtp_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, o,
                                       int(wg_per_cu), _stream(stream)), "mtp_probe_stream_read")


def mtp_probe_fp8_convert(result, stream=None) -> None:
    """Check the hardware FP32 -> E4M3FN convert on every float of magnitude
    <= 448; result (int32 or uint32 [2] device tensor) receives the number of
    values whose code differs from round half to even, and the number checked."""
    r = (_dev(result, "result", torch.int32, 2) if result.dtype == torch.int32
         else _dev(result, "result", torch.uint32, 2))
    _check(lib().mtp_probe_fp8_convert(r, _stream(stream)), "mtp_probe_fp8_convert")
