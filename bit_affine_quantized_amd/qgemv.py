"""ctypes binding of libqgemv.so (include/qgemv.h), argument marshalling only.

The module-level functions carry the C names and take plain integers
(device pointers) or torch tensors (their ``data_ptr()`` is passed).  Every
step of the product runs in the library's HIP kernels; nothing here computes.
Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

QGEMV_OK = 0
QGEMV_E_ARG, QGEMV_E_BITS, QGEMV_E_GROUP, QGEMV_E_SHAPE, QGEMV_E_STRIDE = -1, -2, -3, -4, -5
QGEMV_E_ALIGN, QGEMV_E_WINDOW, QGEMV_E_ALIAS, QGEMV_E_NOKERNEL, QGEMV_E_HIP = -6, -7, -8, -9, -10
QGEMV_E_INDEX = -11
QGEMV_EPI_NONE, QGEMV_EPI_RELU2 = 0, 1
QGEMV_ARITH_AUTO, QGEMV_ARITH_DOT, QGEMV_ARITH_MFMA, QGEMV_ARITH_WIDE = 0, 1, 2, 3
QGEMV_MAX_WINDOW = 16
QGEMV_MAX_PROMPT = 65

_lib = None
_lock = threading.Lock()


class QgemvError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what}: {qgemv_strerror(status)}")
        self.status = status


class qgemv_desc(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("n_experts", ctypes.c_int32), ("w", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


QGEMV_MAX_RUNS, QGEMV_MAX_MEMBERS = 8, 4


class qgemv_run_spec(ctypes.Structure):
    _fields_ = [("w", qgemv_desc), ("n_members", ctypes.c_int32),
                ("member_rows", ctypes.c_int64 * QGEMV_MAX_MEMBERS),
                ("member_cols", ctypes.c_int64 * QGEMV_MAX_MEMBERS)]


def load(path: str | None = None):
    """The loaded library; raises if it is not built (no fallback exists).
    QGEMV_LIB names another build of the same library (e.g. a tuning build)."""
    global _lib
    path = path or os.environ.get("QGEMV_LIB") or LIB_PATH
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise ImportError(f"libqgemv.so is not built ({path}); run __graft_entry__.build()")
            lib = ctypes.CDLL(path)
            p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            lib.qgemv_create.argtypes = [ctypes.POINTER(qgemv_desc), ctypes.POINTER(p)]
            lib.qgemv_create.restype = ctypes.c_int
            lib.qgemv_create_arith.argtypes = [ctypes.POINTER(qgemv_desc), i32, ctypes.POINTER(p)]
            lib.qgemv_create_arith.restype = ctypes.c_int
            lib.qgemv_arith.argtypes = [p]
            lib.qgemv_arith.restype = ctypes.c_int
            lib.qgemv_mfma_codes.argtypes = [i32, i32]
            lib.qgemv_mfma_codes.restype = ctypes.c_int64
            lib.qgemv_destroy.argtypes = [p]
            lib.qgemv_destroy.restype = None
            lib.qgemv_run.argtypes = [p, p, i32, p, i32, p]
            lib.qgemv_run.restype = ctypes.c_int
            lib.qgemv_run_strided.argtypes = [p, p, i32, p, i64, i32, p]
            lib.qgemv_run_strided.restype = ctypes.c_int
            lib.qgemv_run_indexed.argtypes = [p, p, i32, p, i32, p, i32, p]
            lib.qgemv_run_indexed.restype = ctypes.c_int
            lib.qgemv_check_indices.argtypes = [p, p, i32, i32, p]
            lib.qgemv_check_indices.restype = ctypes.c_int
            lib.qgemv_run_gateup.argtypes = [p, p, p, i32, p, i64, p]
            lib.qgemv_run_gateup.restype = ctypes.c_int
            lib.qgemv_run_gateup_indexed.argtypes = [p, p, p, i32, p, i32, p, p]
            lib.qgemv_run_gateup_indexed.restype = ctypes.c_int
            lib.qgemv_common_width.argtypes = [p, p, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
            lib.qgemv_common_width.restype = ctypes.c_int
            lib.qgemv_widen.argtypes = [ctypes.POINTER(qgemv_desc), i32, i32, p, p, p, p]
            lib.qgemv_widen.restype = ctypes.c_int
            lib.qgemv_debug_unpack.argtypes = [p, i32, p, p]
            lib.qgemv_debug_unpack.restype = ctypes.c_int
            lib.qgemv_strerror.argtypes = [ctypes.c_int]
            lib.qgemv_strerror.restype = ctypes.c_char_p
            lib.qgemv_query.argtypes = [p, ctypes.POINTER(ctypes.c_int64 * 6)]
            lib.qgemv_query.restype = ctypes.c_int
            lib.qgemv_stack_create.argtypes = [ctypes.POINTER(qgemv_run_spec), i32, i64, ctypes.POINTER(p)]
            lib.qgemv_stack_create.restype = ctypes.c_int
            lib.qgemv_stack_run.argtypes = [p, p, i32, p, i32, p]
            lib.qgemv_stack_run.restype = ctypes.c_int
            lib.qgemv_stack_destroy.argtypes = [p]
            lib.qgemv_stack_destroy.restype = None
            _lib = lib
    return _lib


def _addr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- the C entry points, same names -----------------------------------------

def qgemv_strerror(status: int) -> str:
    return load().qgemv_strerror(status).decode()


def qgemv_create(bits, group, n, k, w, scales, biases, n_experts=1):
    """Returns (status, handle); handle is None on a refusal."""
    d = qgemv_desc(bits, group, n, k, n_experts, _addr(w), _addr(scales), _addr(biases))
    h = ctypes.c_void_p()
    rc = load().qgemv_create(ctypes.byref(d), ctypes.byref(h))
    return rc, (h.value if rc == QGEMV_OK else None)


def qgemv_create_arith(bits, group, n, k, w, scales, biases, arith, n_experts=1):
    """As qgemv_create with the arithmetic chosen (QGEMV_ARITH_*)."""
    d = qgemv_desc(bits, group, n, k, n_experts, _addr(w), _addr(scales), _addr(biases))
    h = ctypes.c_void_p()
    rc = load().qgemv_create_arith(ctypes.byref(d), arith, ctypes.byref(h))
    return rc, (h.value if rc == QGEMV_OK else None)


def qgemv_arith(h) -> int:
    return load().qgemv_arith(h)


def qgemv_mfma_codes(bits, group) -> int:
    return load().qgemv_mfma_codes(bits, group)


def qgemv_destroy(h) -> None:
    load().qgemv_destroy(h)


def qgemv_run(h, x, m, y, epi=QGEMV_EPI_NONE, stream=None) -> int:
    return load().qgemv_run(h, _addr(x), m, _addr(y), epi, _stream(stream))


def qgemv_run_strided(h, x, m, y, ldy, epi=QGEMV_EPI_NONE, stream=None) -> int:
    return load().qgemv_run_strided(h, _addr(x), m, _addr(y), ldy, epi, _stream(stream))


def qgemv_run_indexed(h, x, m, idx, slots, y, epi=QGEMV_EPI_NONE, stream=None) -> int:
    return load().qgemv_run_indexed(h, _addr(x), m, _addr(idx), slots, _addr(y), epi, _stream(stream))


def qgemv_check_indices(h, idx, m, slots, stream=None) -> int:
    return load().qgemv_check_indices(h, _addr(idx), m, slots, _stream(stream))


def qgemv_run_gateup(gate, up, x, m, y, ldy, stream=None) -> int:
    return load().qgemv_run_gateup(gate, up, _addr(x), m, _addr(y), ldy, _stream(stream))


def qgemv_run_gateup_indexed(gate, up, x, m, idx, slots, y, stream=None) -> int:
    return load().qgemv_run_gateup_indexed(gate, up, _addr(x), m, _addr(idx), slots, _addr(y), _stream(stream))


def qgemv_common_width(bits, groups):
    """Returns (status, bits, group) for lists of member bits and groups."""
    n = len(bits)
    ab = (ctypes.c_int32 * max(1, n))(*bits)
    ag = (ctypes.c_int32 * max(1, n))(*groups)
    ob, og = ctypes.c_int32(), ctypes.c_int32()
    rc = load().qgemv_common_width(ctypes.addressof(ab), ctypes.addressof(ag), n, ctypes.byref(ob), ctypes.byref(og))
    return rc, ob.value, og.value


def qgemv_widen(bits, group, n, k, w, scales, biases, bits_out, group_out, w_out, scales_out, biases_out,
                n_experts=1, stream=None) -> int:
    d = qgemv_desc(bits, group, n, k, n_experts, _addr(w), _addr(scales), _addr(biases))
    return load().qgemv_widen(ctypes.byref(d), bits_out, group_out, _addr(w_out), _addr(scales_out),
                              _addr(biases_out), _stream(stream))


def qgemv_debug_unpack(h, expert, codes, stream=None) -> int:
    return load().qgemv_debug_unpack(h, expert, _addr(codes), _stream(stream))


def qgemv_query(h):
    out = (ctypes.c_int64 * 6)()
    rc = load().qgemv_query(h, ctypes.byref(out))
    return rc, list(out)


def qgemv_stack_create(runs, ldy):
    """runs: list of dicts with bits, group, n, k, w, scales, biases and
    members = [(rows, first_column), ...].  Returns (status, handle)."""
    arr = (qgemv_run_spec * max(1, len(runs)))()
    for i, r in enumerate(runs):
        arr[i].w = qgemv_desc(r["bits"], r["group"], r["n"], r["k"], 1, _addr(r["w"]),
                              _addr(r["scales"]), _addr(r["biases"]))
        members = r["members"]
        arr[i].n_members = len(members)
        for j, (rows, col) in enumerate(members[:QGEMV_MAX_MEMBERS]):
            arr[i].member_rows[j] = rows
            arr[i].member_cols[j] = col
    h = ctypes.c_void_p()
    rc = load().qgemv_stack_create(arr, len(runs), ldy, ctypes.byref(h))
    return rc, (h.value if rc == QGEMV_OK else None)


def qgemv_stack_run(h, x, m, y, epi=QGEMV_EPI_NONE, stream=None) -> int:
    return load().qgemv_stack_run(h, _addr(x), m, _addr(y), epi, _stream(stream))


def qgemv_stack_destroy(h) -> None:
    load().qgemv_stack_destroy(h)


# ---- convenience wrapper over torch device tensors ---------------------------

class Matrix:
    """One handle over torch device tensors (kept alive with the handle).

    w: int32/uint32 [E][N][K*bits/32]; scales, biases: int16/bf16 [E][N][K/G];
    x: bf16 (or int16 bits) [M][K]; y: float32.  Statuses other than
    QGEMV_OK raise QgemvError."""

    def __init__(self, bits, group, n, k, w, scales, biases, n_experts=1, arith=QGEMV_ARITH_AUTO):
        self.bits, self.group, self.n, self.k, self.n_experts = bits, group, n, k, n_experts
        self._keep = (w, scales, biases)
        rc, h = qgemv_create_arith(bits, group, n, k, w, scales, biases, arith, n_experts)
        if rc != QGEMV_OK:
            raise QgemvError("qgemv_create_arith", rc)
        self.h = h
        self.arith = qgemv_arith(h)

    def _chk(self, rc, what):
        if rc != QGEMV_OK:
            raise QgemvError(what, rc)

    def run(self, x, y, m=None, epi=QGEMV_EPI_NONE, stream=None):
        m = x.shape[0] if m is None else m
        self._chk(qgemv_run(self.h, x, m, y, epi, stream), "qgemv_run")
        return y

    def run_strided(self, x, y, ldy, m=None, epi=QGEMV_EPI_NONE, stream=None):
        m = x.shape[0] if m is None else m
        self._chk(qgemv_run_strided(self.h, x, m, y, ldy, epi, stream), "qgemv_run_strided")
        return y

    def run_indexed(self, x, idx, y, epi=QGEMV_EPI_NONE, stream=None):
        m, slots = idx.shape
        self._chk(qgemv_run_indexed(self.h, x, m, idx, slots, y, epi, stream), "qgemv_run_indexed")
        return y

    def debug_unpack(self, codes, expert=0, stream=None):
        self._chk(qgemv_debug_unpack(self.h, expert, codes, stream), "qgemv_debug_unpack")
        return codes

    def query(self):
        rc, out = qgemv_query(self.h)
        self._chk(rc, "qgemv_query")
        return out

    def close(self):
        if getattr(self, "h", None):
            qgemv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Stack:
    """A fused stack over torch device tensors (kept alive with the handle)."""

    def __init__(self, runs, ldy):
        self._keep = [(r["w"], r["scales"], r["biases"]) for r in runs]
        self.ldy = ldy
        rc, h = qgemv_stack_create(runs, ldy)
        if rc != QGEMV_OK:
            raise QgemvError("qgemv_stack_create", rc)
        self.h = h

    def run(self, x, y, m=None, epi=QGEMV_EPI_NONE, stream=None):
        m = x.shape[0] if m is None else m
        rc = qgemv_stack_run(self.h, x, m, y, epi, stream)
        if rc != QGEMV_OK:
            raise QgemvError("qgemv_stack_run", rc)
        return y

    def close(self):
        if getattr(self, "h", None):
            qgemv_stack_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
