"""FP64 CPU oracle for the MTP draft sweep -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never reaches it, and
it shares no code with the HIP path: the arithmetic lives in ``oracle.c`` (plain
C, built with ``gcc -O2 -ffp-contract=off``), this module only marshals numpy
arrays into it and chains the steps in the order the draft formula gives them.

Sources: metrale API docs, ``metrale_model_arch/glm5next_mtp_head.rs`` (module
doc: the draft formula; ``forward_one``: gather by row pointer, enorm, hnorm,
concat, ``dense_gemv`` eh_proj, ``shared_head.norm``, ``dense_gemv`` /
``dense_gemv_fp8w`` lm_head, ``argmax_bf16``; the ``head_fp8`` field doc: the FP8
E4M3 drafting copy) and ``metrale_model_arch/glm5next_layer/mod.rs`` (module
invariants: ``rms_norm_vanilla`` is ``x * w / rms``).

The MTP block between eh_proj and the head is taken as the identity: the pages
describe it only as "DSA + routed MoE" (parity unpinned for that step by
construction; there is nothing to compute).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point this at another build of oracle.c (a sanitizer build).
_LIB_OVERRIDE = os.environ.get("MTP_ORACLE_LIB")

GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
           "-shared", "-fPIC", "-pthread", _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_from_double.argtypes = [ctypes.c_double]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_rmsnorm.argtypes = [P, P, i64, ctypes.c_float, P]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm_unrounded.argtypes = [P, P, i64, ctypes.c_float, P]
        L.orc_rmsnorm_unrounded.restype = None
        L.orc_front.argtypes = [P, i64, i64, ctypes.c_uint32, P, P, P, ctypes.c_float, P]
        L.orc_front.restype = ctypes.c_int
        L.orc_gemv_bf16.argtypes = [P, i64, i64, P, P, ctypes.c_int]
        L.orc_gemv_bf16.restype = None
        L.orc_gemv_fp8.argtypes = [P, P, i64, i64, P, P, ctypes.c_int]
        L.orc_gemv_fp8.restype = None
        L.orc_round_bf16.argtypes = [P, i64, P]
        L.orc_round_bf16.restype = None
        L.orc_argmax_bf16.argtypes = [P, i64]
        L.orc_argmax_bf16.restype = i64
        L.orc_quantize_fp8.argtypes = [P, i64, i64, P, P, ctypes.c_int]
        L.orc_quantize_fp8.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def host_cores() -> dict:
    """What this process may run on: os.cpu_count(), the CPU affinity mask and
    the cgroup CPU quota (in cores, None when unlimited)."""
    info = {"os_cpu_count": os.cpu_count() or 1,
            "affinity": len(os.sched_getaffinity(0)), "cgroup_quota_cores": None}
    for path, split in (("/sys/fs/cgroup/cpu.max", None),
                        ("/sys/fs/cgroup/cpu/cpu.cfs_quota_us", "/sys/fs/cgroup/cpu/cpu.cfs_period_us")):
        try:
            if split is None:
                quota, period = open(path).read().split()
            else:
                quota, period = open(path).read().strip(), open(split).read().strip()
            if quota not in ("max", "-1"):
                info["cgroup_quota_cores"] = -(-int(quota) // int(period))
            break
        except (OSError, ValueError):
            continue
    return info


# A one-GPU host grants a process about 16 host cores, whatever the machine has.
THREAD_CAP = 16


def default_threads() -> int:
    """Threads for the row-parallel loops: the cores this process may use
    (affinity, cgroup quota), at most THREAD_CAP."""
    h = host_cores()
    n = min(h["os_cpu_count"], h["affinity"], h["cgroup_quota_cores"] or h["affinity"])
    return max(1, min(THREAD_CAP, n))


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns (uint16) to float64."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_from_f64(x) -> np.ndarray:
    """Correctly rounded (RNE) float64 -> BF16 bits, one value at a time in C."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_round_bf16(_p(x), x.size, _p(out))
    return out


def e4m3_encode(y: float) -> int:
    return int(lib().orc_e4m3_encode(float(y)))


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


# --------------------------------------------------------------------------
# Steps of the sweep (each cites the passage it follows in oracle.c)
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(w), x.size, ctypes.c_float(eps), _p(out))
    return out


def rmsnorm_unrounded(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """The norm's outputs in FP64 before their BF16 rounding (rmsnorm rounds
    exactly these values)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    out = np.empty(x.size, dtype=np.float64)
    lib().orc_rmsnorm_unrounded(_p(x), _p(w), x.size, ctypes.c_float(eps), _p(out))
    return out


def front_unrounded(embed, token: int, hidden, enorm_w, hnorm_w, eps: float):
    """[enorm(embed[token]) | hnorm(hidden)] in FP64 before the BF16 rounding
    of the concat; None when token >= V."""
    V, H = embed.shape
    if int(token) >= V:
        return None
    e = np.ascontiguousarray(embed[int(token)])
    return np.concatenate([rmsnorm_unrounded(e, enorm_w, eps),
                           rmsnorm_unrounded(np.ascontiguousarray(hidden), hnorm_w, eps)])


def front(embed, token: int, hidden, enorm_w, hnorm_w, eps: float):
    """concat = [enorm(embed[token]) | hnorm(hidden)]; None when token >= V."""
    V, H = embed.shape
    concat = np.empty(2 * H, dtype=np.uint16)
    rc = lib().orc_front(_p(embed), V, H, int(token), _p(np.ascontiguousarray(hidden)),
                         _p(enorm_w), _p(hnorm_w), ctypes.c_float(eps), _p(concat))
    return None if rc != 0 else concat


def gemv_bf16(W: np.ndarray, x: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """Unrounded FP64 y = W @ x, W BF16 row-major [n][k]."""
    n, k = W.shape
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.size == k
    out = np.empty(n, dtype=np.float64)
    lib().orc_gemv_bf16(_p(W), n, k, _p(x), _p(out), nthreads or default_threads())
    return out


def gemv_fp8(q: np.ndarray, s: np.ndarray, x: np.ndarray, nthreads: int | None = None):
    """Unrounded FP64 y_v = s_v * sum_j dec(q[v][j]) * x_j."""
    n, k = q.shape
    x = np.ascontiguousarray(x, dtype=np.uint16)
    s = np.ascontiguousarray(s, dtype=np.float32)
    assert x.size == k and s.size == n
    out = np.empty(n, dtype=np.float64)
    lib().orc_gemv_fp8(_p(q), _p(s), n, k, _p(x), _p(out), nthreads or default_threads())
    return out


def argmax_bf16(logits: np.ndarray) -> int:
    logits = np.ascontiguousarray(logits, dtype=np.uint16)
    return int(lib().orc_argmax_bf16(_p(logits), logits.size))


def quantize_fp8(L: np.ndarray, nthreads: int | None = None):
    """Per-row amax/448 E4M3FN copy of a BF16 [V][H] matrix.

    Returns (q uint8 [V][H], s float32 [V]), or None when a weight is not finite.
    """
    V, H = L.shape
    L = np.ascontiguousarray(L, dtype=np.uint16)
    q = np.empty((V, H), dtype=np.uint8)
    s = np.empty(V, dtype=np.float32)
    rc = lib().orc_quantize_fp8(_p(L), V, H, _p(q), _p(s), nthreads or default_threads())
    return None if rc != 0 else (q, s)


def draft(w: dict, token: int, hidden: np.ndarray, fp8: tuple | None = None,
          nthreads: int | None = None) -> dict | None:
    """One draft for one sequence, every intermediate kept.

    ``w`` holds BF16 bit arrays: embed [V][H], enorm_w, hnorm_w, head_norm_w [H],
    eh_proj [H][2H], lm_head [V][H], and rms_eps.  With ``fp8=(q, s)`` the head
    reads the FP8 copy instead of lm_head.  Returns None when token >= V.

    x = eh_proj(concat(enorm(embed[token]), hnorm(hidden)))   (block = identity)
    logits = lm_head(shared_head.norm(x)); draft = argmax(logits)
    """
    eps = float(w["rms_eps"])
    concat = front(w["embed"], token, hidden, w["enorm_w"], w["hnorm_w"], eps)
    if concat is None:
        return None
    concat_un = front_unrounded(w["embed"], token, hidden, w["enorm_w"], w["hnorm_w"], eps)
    x_un = gemv_bf16(w["eh_proj"], concat, nthreads)
    x = bf16_from_f64(x_un)
    xn = rmsnorm(x, w["head_norm_w"], eps)
    if fp8 is None:
        o = gemv_bf16(w["lm_head"], xn, nthreads)
    else:
        o = gemv_fp8(fp8[0], fp8[1], xn, nthreads)
    logits = bf16_from_f64(o)
    return {"concat": concat, "concat_unrounded": concat_un, "x_unrounded": x_un, "x": x,
            "xn": xn, "o": o,
            "logits": logits, "draft": argmax_bf16(logits)}


def context_rows(w: dict, tokens: np.ndarray, hiddens: np.ndarray,
                 nthreads: int | None = None) -> dict:
    """Context rows (glm5next_mtp_head.rs, `rows_impl`): row r pairs the
    embedding of tokens[r + 1] with hiddens[r] and runs enorm, hnorm, concat and
    eh_proj.  Returns ``x`` as BF16 bits [T][H], ``x_unrounded`` (FP64), the
    BF16 ``concat`` rows [T][2H] and ``concat_unrounded`` (FP64, before that
    rounding); all zero in a row whose tokens[r + 1] is out of range (the
    library leaves such a row unspecified)."""
    T = hiddens.shape[0]
    assert tokens.size == T + 1
    H = w["embed"].shape[1]
    x = np.zeros((T, H), dtype=np.uint16)
    x_un = np.zeros((T, H), dtype=np.float64)
    concat = np.zeros((T, 2 * H), dtype=np.uint16)
    concat_un = np.zeros((T, 2 * H), dtype=np.float64)
    for r in range(T):
        c = front(w["embed"], int(tokens[r + 1]), hiddens[r], w["enorm_w"], w["hnorm_w"],
                  float(w["rms_eps"]))
        if c is not None:
            concat[r] = c
            concat_un[r] = front_unrounded(w["embed"], int(tokens[r + 1]), hiddens[r],
                                           w["enorm_w"], w["hnorm_w"], float(w["rms_eps"]))
            x_un[r] = gemv_bf16(w["eh_proj"], c, nthreads)
            x[r] = bf16_from_f64(x_un[r])
    return {"x": x, "x_unrounded": x_un, "concat": concat, "concat_unrounded": concat_un}


def draft_chain(w: dict, token: int, hidden: np.ndarray, steps: int, fp8: tuple | None = None,
                nthreads: int | None = None) -> list:
    """Chained drafts for one sequence: ``steps`` calls of ``draft``, step k + 1
    taking step k's draft as its token and step k's block output x (BF16 bits)
    as its hidden.  The pages show that a propose call writes several drafts
    (glm5next_mtp_head.rs, the state's ``last_drafted``), each one
    ``forward_one(token, hidden_in)``; which hidden is fed back is not shown,
    and the block output is taken (the block being the identity).  Returns the
    per-step results of ``draft``; a None entry (token out of range) ends the
    chain, every later draft being invalid too."""
    out = []
    tok, hid = int(token), np.ascontiguousarray(hidden, dtype=np.uint16)
    for _ in range(steps):
        r = draft(w, tok, hid, fp8, nthreads)
        out.append(r)
        if r is None:
            break
        tok, hid = r["draft"], r["x"]
    return out
