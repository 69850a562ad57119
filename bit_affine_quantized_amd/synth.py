"""Seeded synthetic inputs for the MLX-affine quantized row product.

This module draws inputs and nothing else: it holds none of the product's
arithmetic (no unpacking, no dequantization, no dot product). It serves the
CPU oracle, the GPU tests and the benchmark alike, so that both sides see the
same bytes.

What it draws, following the check programs described on "Qwen3.8-Flash-Next
faster kernels in Zig engine - #788" (commit "tf-affine-ref": seeded synthetic
codes, scales, biases and inputs, packed as MLX affine):

* codes: every bit of each row's bitstream is an independent fair coin, drawn
  as uniform 32-bit words.  A b-bit field of independent fair bits is uniform
  over [0, 2^b - 1], so every code is uniform over its full range.
* scales ~ U(0.005, 0.02) and biases ~ U(-0.1, 0.1), one pair per group,
  drawn in fp64 and rounded to bf16 (fp64 -> fp32 -> bf16, round to nearest
  even at each step).
* activations x ~ N(0, 1), drawn in fp64 and rounded the same way.
* wide-range activations (one parity case): sign * (1 + j/128) * 2^e with j
  uniform over 0..127, e uniform over -24..24 and a fair sign, rounded the
  same way, so that a 32-code unit's fp32 dot rounds.
* expert routing: for every activation row, 8 distinct expert slots drawn
  without replacement, kept in the order drawn.

Draw order per matrix: code words (row-major), scales, biases; then the
activation window; then the routing table.

Storage layout (the format every consumer reads):
  words  uint32 [E][N][K*bits/32]  little-endian words; row n of expert e is
         one contiguous bitstream, code k at bits [k*bits, k*bits+bits)
         counted from bit 0 of the row's first word (low code first).
  scales, biases  uint16 (bf16 bits) [E][N][K/group]
  x      uint16 (bf16 bits) [M][K]

``pack_codes`` writes given codes into that layout, for structured test
inputs (sweep patterns, exact cases); it is the format's encoder and is
pinned against hand-packed bytes derived from the pages' rule.
"""

from __future__ import annotations

import numpy as np

BITS = (2, 3, 4, 5, 6, 8)
GROUPS = (32, 64, 128)
PAIRS = tuple((b, g) for b in BITS for g in GROUPS)


# --------------------------------------------------------------------------
# bf16 encoding of draws
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest, ties to even.

    Inputs are finite (no NaN handling is needed for these draws)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def to_bf16_bits(a) -> np.ndarray:
    """fp64 draws -> bf16 bit patterns (fp64 -> fp32 RNE -> bf16 RNE)."""
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float64).astype(np.float32))


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# format encoder (structured inputs only)
# --------------------------------------------------------------------------

def row_words(k: int, bits: int) -> int:
    if (k * bits) % 32:
        raise ValueError("a row of K codes must end on a 32-bit word")
    return k * bits // 32


def pack_codes(codes, bits: int) -> np.ndarray:
    """codes uint8 [..., K] (each < 2^bits) -> words uint32 [..., K*bits/32].

    Bit j of code k lands at bit k*bits + j of the row's bitstream; the
    bitstream is cut into little-endian 32-bit words."""
    codes = np.asarray(codes)
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range for width")
    k = codes.shape[-1]
    nw = row_words(k, bits)
    planes = [(codes >> j) & 1 for j in range(bits)]          # [..., K] each
    stream = np.stack(planes, axis=-1).astype(np.uint8)       # [..., K, bits]
    stream = stream.reshape(codes.shape[:-1] + (k * bits,))
    raw = np.packbits(stream, axis=-1, bitorder="little")     # [..., K*bits/8]
    raw = np.ascontiguousarray(raw)
    return raw.view("<u4").reshape(codes.shape[:-1] + (nw,)).astype(np.uint32)


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------

def draw_words(rng, shape, k: int, bits: int) -> np.ndarray:
    nw = row_words(k, bits)
    return rng.integers(0, 1 << 32, size=tuple(shape) + (nw,), dtype=np.uint64).astype(np.uint32)


def draw_scales(rng, shape) -> np.ndarray:
    return to_bf16_bits(rng.uniform(0.005, 0.02, size=shape))


def draw_biases(rng, shape) -> np.ndarray:
    return to_bf16_bits(rng.uniform(-0.1, 0.1, size=shape))


def draw_x(rng, m: int, k: int) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal(size=(m, k)))


def draw_x_wide(rng, m: int, k: int, span: int = 48) -> np.ndarray:
    """Activations whose magnitudes spread over 2^(+-span/2) with random
    signs, so that a 32-code unit's fp32 dot rounds (normal draws keep most
    unit dots exact)."""
    mant = 1.0 + rng.integers(0, 128, size=(m, k)) / 128.0
    expo = rng.integers(-(span // 2), span // 2 + 1, size=(m, k))
    sign = np.where(rng.integers(0, 2, size=(m, k)) == 1, -1.0, 1.0)
    return to_bf16_bits(sign * np.ldexp(mant, expo))


def draw_routes(rng, m: int, slots: int, n_experts: int) -> np.ndarray:
    idx = np.empty((m, slots), dtype=np.int32)
    for i in range(m):
        idx[i] = rng.choice(n_experts, size=slots, replace=False)
    return idx


def matrix(seed: int, bits: int, group: int, n: int, k: int, m: int = 0,
           n_experts: int = 1) -> dict:
    """One quantized matrix (or expert stack) and an optional window.

    Returns a dict with words [E][N][W], scales/biases [E][N][K/G] and,
    when m > 0, x [m][K].  With n_experts == 1 the leading E axis is dropped.
    """
    if k % group:
        raise ValueError("K must be a multiple of the group")
    rng = np.random.default_rng(seed)
    lead = (n_experts, n) if n_experts > 1 else (n,)
    words = draw_words(rng, lead, k, bits)
    scales = draw_scales(rng, lead + (k // group,))
    biases = draw_biases(rng, lead + (k // group,))
    out = dict(bits=bits, group=group, n=n, k=k, n_experts=n_experts,
               words=words, scales=scales, biases=biases)
    if m:
        out["x"] = draw_x(rng, m, k)
    out["rng"] = rng
    return out


# --------------------------------------------------------------------------
# the workloads (shapes and value distributions of the pages' decode shapes)
# --------------------------------------------------------------------------

SWEEP_N = SWEEP_K = 4096
SWEEP_WINDOWS = (1, 2, 3, 8, 16)
LMHEAD_N, LMHEAD_K, LMHEAD_BITS, LMHEAD_GROUP = 248320, 2048, 6, 32
STACK_K = 2048
# (bits, group, columns, first output column) of each run; output row stride 8288
STACK_RUNS = ((4, 64, 2048, 0), (5, 128, 6192, 2048), (6, 64, 48, 8240))
STACK_LDY = 8288
EXPERTS_E, EXPERTS_N, EXPERTS_K, EXPERTS_BITS, EXPERTS_GROUP = 128, 1024, 2048, 4, 64
EXPERTS_M, EXPERTS_SLOTS = 16, 8


def single(m: int = 1, seed: int = 0) -> dict:
    """N = K = 2048, 4-bit codes, group 64, one activation row, seed 0."""
    return matrix(seed, 4, 64, 2048, 2048, m)


def sweep_seed(bits: int, group: int) -> int:
    return 2000 + 100 * bits + group


def sweep(bits: int, group: int, m: int = 16, n: int = SWEEP_N, k: int = SWEEP_K) -> dict:
    """N = K = 4096 at one width/group pair, windows of up to 16 rows."""
    return matrix(sweep_seed(bits, group), bits, group, n, k, m)


def lmhead(m: int = 1, seed: int = 4000) -> dict:
    """LM-head-sized matrix: N = 248320, K = 2048, 6-bit codes, group 32."""
    return matrix(seed, LMHEAD_BITS, LMHEAD_GROUP, LMHEAD_N, LMHEAD_K, m)


def stack(m: int = 1, seed: int = 3000) -> dict:
    """Fused mixed-width projection stack at K = 2048: three runs written into
    one output row of 8288 columns through the row stride."""
    rng = np.random.default_rng(seed)
    runs = []
    for bits, group, n, col in STACK_RUNS:
        words = draw_words(rng, (n,), STACK_K, bits)
        scales = draw_scales(rng, (n, STACK_K // group))
        biases = draw_biases(rng, (n, STACK_K // group))
        runs.append(dict(bits=bits, group=group, n=n, k=STACK_K, col=col,
                         words=words, scales=scales, biases=biases))
    x = draw_x(rng, m, STACK_K)
    return dict(runs=runs, x=x, ldy=STACK_LDY, k=STACK_K)


def experts(seed: int = 5000, m: int = EXPERTS_M, slots: int = EXPERTS_SLOTS,
            n_experts: int = EXPERTS_E, n: int = EXPERTS_N) -> dict:
    """Indexed expert stack: 128 experts of 1024 x 2048 at 4-bit/group 64,
    16 activation rows each routed to 8 distinct expert slots."""
    d = matrix(seed, EXPERTS_BITS, EXPERTS_GROUP, n, EXPERTS_K, m, n_experts)
    d["idx"] = draw_routes(d["rng"], m, slots, n_experts)
    d["slots"] = slots
    return d


# --------------------------------------------------------------------------
# structured inputs for exactness cases
# --------------------------------------------------------------------------

def sweep_codes(n: int, k: int, bits: int) -> np.ndarray:
    """q[n,k] = (7k + k//32 + n) mod 2^bits: every value at every bit offset
    of a 32-bit word once K reaches 32 * 2^bits."""
    kk = np.arange(k)[None, :]
    nn = np.arange(n)[:, None]
    return ((7 * kk + kk // 32 + nn) % (1 << bits)).astype(np.uint8)


def exact_case(seed: int, bits: int, group: int, n: int, k: int, m: int) -> dict:
    """Inputs on which every fp32 summation order is exact.

    scales in {2^-8, 2^-7, 2^-6}, biases multiples of 2^-8 with |bias| <= 1/8,
    x in {-1, 0, 1}: every partial sum is a multiple of 2^-8 below 2^15."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, size=(n, k), dtype=np.int64).astype(np.uint8)
    scales = to_bf16_bits(2.0 ** -rng.integers(6, 9, size=(n, k // group)))
    biases = to_bf16_bits(rng.integers(-32, 33, size=(n, k // group)) / 256.0)
    x = to_bf16_bits(rng.integers(-1, 2, size=(m, k)).astype(np.float64))
    return dict(bits=bits, group=group, n=n, k=k, n_experts=1, codes=codes,
                words=pack_codes(codes, bits), scales=scales, biases=biases, x=x)
