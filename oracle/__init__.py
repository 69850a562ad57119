"""CPU oracle for the MLX-affine quantized row product (test infrastructure).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the product path
(``bit_affine_quantized_amd``) never does, and the two share no code.

The arithmetic lives in ``qgemv_oracle.c`` (plain C, fp64).  This module
compiles it with gcc, marshals numpy arrays to it, and states the acceptance
bounds.  Every function cites the passage it follows; page titles:

  P788 = "Qwen3.8-Flash-Next faster kernels in Zig engine - #788"
  P774 = "Qwen3.8-Flash-Next support for oQ in Zig engine - #774"

Parity status of each function is stated in its docstring ("pinned by ...").
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qgemv_oracle.c")
BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-shared", "-fPIC"]

_lib = None
_lock = threading.Lock()


def build(source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_check_shape.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64]
    lib.oracle_check_shape.restype = ctypes.c_int
    lib.oracle_unpack.argtypes = [ctypes.c_int, i64, i64, p, p]
    lib.oracle_unpack.restype = ctypes.c_int
    lib.oracle_gemv.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, p, p, p, i64, p,
                                ctypes.c_double, i64, i64, i64, p, p, p]
    lib.oracle_gemv.restype = ctypes.c_int
    lib.oracle_relu2.argtypes = [p, i64, p]
    lib.oracle_relu2.restype = None
    lib.oracle_silu_gateup.argtypes = [p, p, i64, p]
    lib.oracle_silu_gateup.restype = None
    return lib


def load(path: str | None = None):
    """Load the compiled oracle, building it first if it is not built."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            # QGEMV_ORACLE_LIB points the tests at another build of the oracle
            # (the mutation check builds deliberately broken copies).
            alt = os.environ.get("QGEMV_ORACLE_LIB")
            if alt:
                _lib = _bind(ctypes.CDLL(alt))
            else:
                if not os.path.exists(LIB_PATH):
                    build()
                _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# --------------------------------------------------------------------------
# the method, step by step
# --------------------------------------------------------------------------

def check_shape(bits: int, group: int, n: int, k: int, lib=None) -> int:
    """0 if admitted.  Rules: widths 2/3/4/5/6/8 and groups 32/64/128 (P774,
    "What this changes", item 2: admission reads MLX affine 2, 3, 4, 5, 6 or
    8 bits in groups of 32, 64 or 128); the group divides K; a row ends on a
    32-bit word (P788, commit "...row kernel at every MLX width")."""
    lib = lib or load()
    return lib.oracle_check_shape(bits, group, n, k)


def unpack(words: np.ndarray, bits: int, n: int, k: int, lib=None) -> np.ndarray:
    """codes[n][k]: code k = bits [k*b, k*b+b) of the row's little-endian
    bitstream, low code first (P788, commit "...row kernel at every MLX
    width").  Pinned by hand-packed bytes and a bit-by-bit brute force."""
    lib = lib or load()
    w = np.ascontiguousarray(words, dtype=np.uint32).reshape(n, -1)
    out = np.empty((n, k), dtype=np.uint8)
    rc = lib.oracle_unpack(bits, n, k, _ptr(w), _ptr(out))
    if rc:
        raise ValueError(f"oracle_unpack refused (status {rc})")
    return out


def gemv(words, scales, biases, x, bits: int, group: int, n: int, k: int,
         scale_mult: float = 1.0, rows=None, threads: int = 1, lib=None):
    """fp64 y, abs and terms, each [M][N] (columns outside ``rows`` are NaN).

    w = s*q + bias per group, y = sum_k w*x summed in fp64 (P788, commit
    "tf-affine-ref": the reference dequantizes the same codes in float64 and
    multiplies in float64).  ``scale_mult`` = 1.01 gives the negative control
    with scales 1% off (same commit).  ``rows`` = (n0, n1) limits the columns
    computed; ``threads`` splits them over host threads (ctypes releases the
    GIL, the arithmetic per column is unchanged).  Pinned by one-hot,
    closed-form, exact-rational and exact-representable cases."""
    lib = lib or load()
    w = np.ascontiguousarray(words, dtype=np.uint32).reshape(n, -1)
    s = np.ascontiguousarray(scales, dtype=np.uint16).reshape(n, k // group)
    b = np.ascontiguousarray(biases, dtype=np.uint16).reshape(n, k // group)
    xx = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, k)
    m = xx.shape[0]
    n0, n1 = (0, n) if rows is None else rows
    y = np.full((m, n), np.nan)
    a = np.full((m, n), np.nan)
    t = np.full((m, n), np.nan)

    def part(lo, hi):
        rc = lib.oracle_gemv(bits, group, n, k, _ptr(w), _ptr(s), _ptr(b), m, _ptr(xx),
                             float(scale_mult), lo, hi, n, _ptr(y), _ptr(a), _ptr(t))
        if rc:
            raise ValueError(f"oracle_gemv refused (status {rc})")

    if threads <= 1 or n1 - n0 < 2 * threads:
        part(n0, n1)
    else:
        edges = np.linspace(n0, n1, threads + 1).astype(np.int64)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: part(int(edges[i]), int(edges[i + 1])), range(threads)))
    return y, a, t


def relu2(y: np.ndarray, lib=None) -> np.ndarray:
    """relu2 epilogue in fp64: y*y where y > 0, NaN passes, else +0 (P788,
    commit "...row kernel at every MLX width", option relu2)."""
    lib = lib or load()
    yy = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty_like(yy)
    lib.oracle_relu2(_ptr(yy), yy.size, _ptr(out))
    return out


def silu_gateup(g: np.ndarray, u: np.ndarray, lib=None) -> np.ndarray:
    """Gate/up pair in fp64: silu(g) * u, silu(g) = g / (1 + exp(-g)) (the
    experts' "gate/up (through silu)" class, P788 "tf-flashnext-widths").
    Pinned by tests/test_oracle_pins.py against g * (1 + tanh(g/2)) / 2."""
    lib = lib or load()
    gg = np.ascontiguousarray(g, dtype=np.float64)
    uu = np.ascontiguousarray(u, dtype=np.float64)
    assert gg.shape == uu.shape
    out = np.empty_like(gg)
    lib.oracle_silu_gateup(_ptr(gg), _ptr(uu), gg.size, _ptr(out))
    return out


def gemv_indexed(words, scales, biases, x, idx, bits, group, n, k, scale_mult=1.0,
                 threads: int = 1, lib=None):
    """Indexed slots: output (i, s) is row i times the expert idx[i, s]
    (P788, commit "...row kernel at every MLX width", option "indexed
    slots"; commit "tf-affine-ref": the one-expert gather).
    Returns y, abs, terms as [M][S][N]."""
    idx = np.asarray(idx)
    m, slots = idx.shape
    y = np.empty((m, slots, n))
    a = np.empty((m, slots, n))
    t = np.empty((m, slots, n))
    for i in range(m):
        for sl in range(slots):
            e = int(idx[i, sl])
            yy, aa, tt = gemv(words[e], scales[e], biases[e], x[i:i + 1], bits, group, n, k,
                              scale_mult, threads=threads, lib=lib)
            y[i, sl], a[i, sl], t[i, sl] = yy[0], aa[0], tt[0]
    return y, a, t


# --------------------------------------------------------------------------
# acceptance bounds
# --------------------------------------------------------------------------

U32 = 2.0 ** -24  # unit roundoff of fp32


def tol_y(abs64: np.ndarray, k: int) -> np.ndarray:
    """Acceptance for fp32 outputs: |y - y64| <= K * 2^-24 * sum|w*x| + 1e-7."""
    return k * U32 * abs64 + 1e-7


def tol_pages(terms64: np.ndarray, group: int, k: int) -> np.ndarray:
    """Diagnostic bound of P788, commit "tf-affine-ref": (group + K/group + 8)
    fp32 roundings of the summed terms' magnitudes (the extra bf16 ulp there
    applies to bf16 outputs only; these outputs are fp32)."""
    return (group + k // group + 8) * U32 * terms64


def tol_relu2(y64: np.ndarray, tol: np.ndarray) -> np.ndarray:
    """Bound for relu2 outputs given the bound E on y: the change of y*y
    under |dy| <= E, plus one fp32 rounding of the product."""
    ay = np.abs(y64)
    return tol * (2.0 * ay + tol) + U32 * (ay + tol) ** 2


SILU_SLOPE = 1.0999   # max |d silu / dg| (about 1.0998, at g = 2.3994)


def tol_gateup(g64: np.ndarray, u64: np.ndarray, tol_g: np.ndarray, tol_u: np.ndarray) -> np.ndarray:
    """Bound for fp32 silu(g) * u given the bounds E_g, E_u on g and u:
    |silu(G) - silu(g)| <= SILU_SLOPE * E_g; the fp32 evaluation
    g / (1 + exp(-g)) adds at most 4 roundings (exp within 2 ulp, the add,
    the divide), E_s = 4u * A + SILU_SLOPE * E_g with A = |silu(g)| +
    SILU_SLOPE * E_g; then the product: A' * E_u + |u| * E_s + u * A' *
    (|u| + E_u), A' = |silu(g)| + E_s, u = 2^-24."""
    s64 = np.abs(silu_gateup(g64, np.ones_like(g64)))
    a = s64 + SILU_SLOPE * tol_g
    e_s = 4.0 * U32 * a + SILU_SLOPE * tol_g
    a2 = s64 + e_s
    au = np.abs(u64)
    return a2 * tol_u + au * e_s + U32 * a2 * (au + tol_u)


def worst_fraction(err: np.ndarray, tol: np.ndarray) -> float:
    """Largest err/bound over all outputs (the pages report the worst column's
    error as a fraction of its bound: P774, "FP64 per class")."""
    return float(np.max(err / tol)) if err.size else 0.0
