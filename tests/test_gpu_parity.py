"""GPU parity of the HIP row product against the CPU oracle, through the C ABI.

Bars (fp32 outputs):
  * unpacked codes: bit for bit equal to the oracle's, every width;
  * outputs: |y - y64| <= K * 2^-24 * sum|w*x| + 1e-7 (y64, sum from the oracle);
  * relu2: within the bound that y's bound implies, and bit for bit equal to
    fp32 y*y of the plain call;
  * a row alone equals the same row in windows of 2 to 16 rows at every
    position, bit for bit; strided and indexed outputs equal the plain call
    bit for bit; a repeat gives the same bytes;
  * the two matrix-core forms give the same bits, also with activations whose
    unit dots round (the library's choice mixes them by window);
  * exact-representable inputs give y == y64 exactly;
  * scales 1% off (negative control) exceed the pages' bound.
"""

import os

import numpy as np
import pytest

import oracle
from bit_affine_quantized_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from bit_affine_quantized_amd import qgemv  # noqa: E402

THREADS = max(1, min(16, os.cpu_count() or 1))
PAIRS = list(synth.PAIRS)
DEV = "cuda"


def dev(a: np.ndarray):
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16,
            np.dtype(np.int32): np.int32, np.dtype(np.uint8): np.uint8}[a.dtype]
    return torch.from_numpy(a.view(view)).to(DEV)


# both arithmetic forms of a handle, each held to the same bars
ARITHS = [qgemv.QGEMV_ARITH_DOT, qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_WIDE]
ARITH_IDS = ["dot", "mfma", "wide"]
arith_param = pytest.mark.parametrize("arith", ARITHS, ids=ARITH_IDS)
# the two matrix-core forms (prompt windows, gate/up pairs)
MC = [qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_WIDE]
mc_param = pytest.mark.parametrize("arith", MC, ids=["mfma", "wide"])


def matrix_of(d, expert=None, arith=qgemv.QGEMV_ARITH_AUTO):
    w, s, b = d["words"], d["scales"], d["biases"]
    if expert is not None:
        w, s, b = w[expert], s[expert], b[expert]
    tw, ts, tb = dev(w), dev(s), dev(b)
    return qgemv.Matrix(d["bits"], d["group"], d["n"], d["k"], tw, ts, tb, arith=arith)


def run(mat, xt, m=None, epi=0):
    m = xt.shape[0] if m is None else m
    y = torch.empty((m, mat.n), dtype=torch.float32, device=DEV)
    mat.run(xt[:m], y, m=m, epi=epi)
    return y


def bits_equal(a, b) -> bool:
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def check_bound(y_gpu: np.ndarray, y64, a64, k, label=""):
    err = np.abs(y_gpu.astype(np.float64) - y64)
    tol = oracle.tol_y(a64, k)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, f"{label}: {len(bad)} outputs outside the bound, first {bad[:3].tolist()}, " \
                          f"worst err/bound {oracle.worst_fraction(err, tol):.3f}"
    return oracle.worst_fraction(err, tol)


def print_case(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,group", PAIRS)
def test_unpacked_codes_bit_exact(bits, group):
    print_case("unpack", bits, group)
    n, k = 24, 4096
    d = synth.matrix(synth.sweep_seed(bits, group) + 1, bits, group, n, k)
    mat = matrix_of(d)
    codes = torch.empty((n, k), dtype=torch.uint8, device=DEV)
    mat.debug_unpack(codes)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.unpack(d["words"], bits, n, k))
    # every value at every bit offset of a word
    kk = 32 * (1 << bits)
    kk = ((kk + group - 1) // group) * group
    sc = synth.sweep_codes(3, kk, bits)
    words = synth.pack_codes(sc, bits)
    ones = synth.to_bf16_bits(np.ones((3, kk // group)))
    m2 = qgemv.Matrix(bits, group, 3, kk, dev(words), dev(ones), dev(ones))
    c2 = torch.empty((3, kk), dtype=torch.uint8, device=DEV)
    m2.debug_unpack(c2)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), oracle.unpack(words, bits, 3, kk))
    assert np.array_equal(c2.cpu().numpy(), sc)


# ---------------------------------------------------------------------------
# the width sweep: N = K = 4096 at every pair, a 16-row window
# ---------------------------------------------------------------------------

@arith_param
@pytest.mark.parametrize("bits,group", PAIRS)
def test_sweep_within_bound(bits, group, arith):
    print_case("sweep", bits, group, arith)
    d = synth.sweep(bits, group, m=16)
    n, k = d["n"], d["k"]
    mat = matrix_of(d, arith=arith)
    assert mat.arith == arith
    xt = dev(d["x"])
    y16 = run(mat, xt).cpu().numpy()
    y64, a64, t64 = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k,
                                threads=THREADS)
    frac = check_bound(y16, y64, a64, k, f"{bits}/{group}")
    pages = oracle.worst_fraction(np.abs(y16 - y64), oracle.tol_pages(t64, group, k))
    print_case(f"  worst err/bound {frac:.4f}; of the pages' bound {pages:.4f}")
    # negative control: scales 1% off must exceed the pages' bound (row 0)
    yb, _, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"][:1], bits, group, n, k,
                           scale_mult=1.01, threads=THREADS)
    ctrl = oracle.worst_fraction(np.abs(y16[:1] - yb), oracle.tol_pages(t64[:1], group, k))
    assert ctrl > 1.0, f"negative control only {ctrl:.3f} of the bound"


@pytest.mark.parametrize("arith", ARITHS + [qgemv.QGEMV_ARITH_AUTO], ids=ARITH_IDS + ["auto"])
@pytest.mark.parametrize("bits,group", PAIRS)
def test_window_invariance(bits, group, arith):
    """Every row of a 64-row pool alone equals itself at every position of
    every window of 2 to 16 rows, bit for bit (the pages check windows of 1,
    2, 3, 4, 5, 8, 9, 16, 17 and 33 rows against one call; 17 and 33 are
    prompt windows, tested separately)."""
    print_case("windows", bits, group, arith)
    d = synth.sweep(bits, group, m=0)
    rng = np.random.default_rng(synth.sweep_seed(bits, group) + 7)
    pool = dev(synth.draw_x(rng, 64, d["k"]))
    mat = matrix_of(d, arith=arith)
    alone = torch.empty((64, d["n"]), dtype=torch.float32, device=DEV)
    for r in range(64):
        mat.run(pool[r:r + 1], alone[r:r + 1], m=1)
    for m in range(2, 17):
        y = torch.empty((64 - m + 1, m, d["n"]), dtype=torch.float32, device=DEV)
        for s0 in range(0, 64 - m + 1):
            mat.run(pool[s0:s0 + m], y[s0], m=m)
        want = torch.stack([alone[s0:s0 + m] for s0 in range(0, 64 - m + 1)])
        if not bits_equal(y, want):
            bad = [s0 for s0 in range(0, 64 - m + 1) if not bits_equal(y[s0], want[s0])]
            raise AssertionError(f"window {m} differs at positions {bad[:8]}")


@pytest.mark.parametrize("bits,group", PAIRS)
def test_matrix_core_forms_agree_bit_for_bit(bits, group):
    """The block-diagonal and wide forms give the same bits with activations
    whose unit dots round (magnitudes over 2^+-24, mixed signs): the matrix
    cores sum a 16x16x32 product's K as four 8-wide steps in order, which is
    what the block-diagonal form's four chained products do.  The library's
    choice runs block-diagonal kernels up to 8 rows and wide ones above, so a
    row keeps its bits in every window; both stay within the bound."""
    print_case("forms", bits, group)
    d = synth.sweep(bits, group, m=0, n=512, k=2048)
    rng = np.random.default_rng(synth.sweep_seed(bits, group) + 11)
    x = synth.draw_x_wide(rng, 16, d["k"])
    xt = dev(x)
    mats = {a: matrix_of(d, arith=a) for a in (qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_WIDE,
                                             qgemv.QGEMV_ARITH_AUTO)}
    alone = torch.empty((16, d["n"]), dtype=torch.float32, device=DEV)
    for r in range(16):
        mats[qgemv.QGEMV_ARITH_MFMA].run(xt[r:r + 1], alone[r:r + 1], m=1)
    for m in (1, 4, 8, 9, 16):
        for a, mat in mats.items():
            y = run(mat, xt, m=m)
            assert bits_equal(y, alone[:m]), f"form {a} at {m} rows differs from the 1-row block-diagonal call"
    y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], x, bits, group, d["n"], d["k"],
                              threads=THREADS)
    check_bound(alone.cpu().numpy(), y64, a64, d["k"], f"{bits}/{group} wide-range activations")


@mc_param
@pytest.mark.parametrize("bits,group", [(6, 32), (4, 64), (3, 128), (8, 32), (2, 64), (5, 64)])
def test_prompt_windows(bits, group, arith):
    """Matrix-core forms: windows of 17-65 rows (passes of 16) give every row
    the bits it has alone, and stay within the bound; the dot form refuses
    them."""
    print_case("prompt", bits, group, arith)
    n, k = 1000, 2048
    d = synth.matrix(7000 + bits * 10 + group, bits, group, n, k)
    rng = np.random.default_rng(7100 + bits * 10 + group)
    pool_np = synth.draw_x(rng, 80, k)
    pool = dev(pool_np)
    mat = matrix_of(d, arith=arith)
    alone = torch.empty((80, n), dtype=torch.float32, device=DEV)
    for r in range(80):
        mat.run(pool[r:r + 1], alone[r:r + 1], m=1)
    for m in (17, 33, 65):
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        for s0 in (0, 15 if m < 65 else 7):
            mat.run(pool[s0:s0 + m], y, m=m)
            assert bits_equal(y, alone[s0:s0 + m]), f"window {m} at {s0}"
    # y holds the last 65-row window, pool rows 7..71
    y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], pool_np[7:72], bits, group, n, k,
                              threads=THREADS)
    check_bound(y.cpu().numpy(), y64, a64, k, f"prompt {bits}/{group}")
    dot = matrix_of(d, arith=qgemv.QGEMV_ARITH_DOT)
    with pytest.raises(qgemv.QgemvError, match="QGEMV_E_WINDOW"):
        dot.run(pool[:17], torch.empty((17, n), dtype=torch.float32, device=DEV), m=17)


GATEUP = [(6, 32, 1003, 2048), (4, 64, 1024, 2048), (3, 128, 100, 1024), (8, 32, 48, 512),
          (2, 64, 300, 2048), (5, 32, 17, 1024)]


def _gateup_pair(bits, group, n, k, m, seed, n_experts=1):
    dg = synth.matrix(seed, bits, group, n, k, m, n_experts=n_experts)
    du = synth.matrix(seed + 1, bits, group, n, k, n_experts=n_experts)
    return dg, du


@mc_param
@pytest.mark.parametrize("bits,group,n,k", GATEUP)
def test_gateup_pair(bits, group, n, k, arith):
    """y = silu(g) * u in one dispatch over the gate and up matrices: within
    a few fp32 roundings of fp64 silu over the plain calls' own g and u, within
    the bound against the oracle, and each row's bits the same in every
    window and position."""
    print_case("gateup", bits, group, n, k, arith)
    dg, du = _gateup_pair(bits, group, n, k, 16, 7500 + bits * 10 + group)
    gate = matrix_of(dg, arith=arith)
    up = matrix_of(du, arith=arith)
    xt = dev(dg["x"])
    rows = {}
    for m in (1, 5, 16):
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        assert qgemv.qgemv_run_gateup(gate.h, up.h, xt, m, y, n) == qgemv.QGEMV_OK
        g = run(gate, xt, m).cpu().numpy().astype(np.float64)
        u = run(up, xt, m).cpu().numpy().astype(np.float64)
        yc = y.cpu().numpy()
        ref = oracle.silu_gateup(g, u)
        # a few fp32 roundings; below g = -88.7 exp(-g) overflows fp32 and
        # silu(g) (under 1e-36 |g| there) evaluates to 0
        floor = 1e-30 * (1.0 + np.abs(u))
        assert np.all(np.abs(yc - ref) <= 8 * oracle.U32 * np.abs(ref) + floor), f"m={m}"
        g64, ag, _ = oracle.gemv(dg["words"], dg["scales"], dg["biases"], dg["x"][:m], bits, group, n, k)
        u64, au, _ = oracle.gemv(du["words"], du["scales"], du["biases"], dg["x"][:m], bits, group, n, k)
        tol = oracle.tol_gateup(g64, u64, oracle.tol_y(ag, k), oracle.tol_y(au, k))
        err = np.abs(yc - oracle.silu_gateup(g64, u64))
        assert np.all(err <= tol), f"m={m}: worst err/bound {oracle.worst_fraction(err, tol):.3f}"
        rows[m] = y
    for m in (5, 16):
        assert bits_equal(rows[m][:1], rows[1])
    y1 = torch.empty((1, n), dtype=torch.float32, device=DEV)
    for r in (3, 15):
        assert qgemv.qgemv_run_gateup(gate.h, up.h, xt[r:r + 1], 1, y1, n) == qgemv.QGEMV_OK
        assert bits_equal(y1[0], rows[16][r])
    # strided: gaps keep their bytes
    ldy = n + 5
    sentinel = torch.full((5, ldy), 0x7FC0BEEF, dtype=torch.int32, device=DEV)
    ys = sentinel.clone().view(torch.float32)
    assert qgemv.qgemv_run_gateup(gate.h, up.h, xt, 5, ys.view(-1)[2:], ldy) == qgemv.QGEMV_OK
    assert bits_equal(ys[:, 2:2 + n], rows[5])
    gap = torch.ones((5, ldy), dtype=torch.bool, device=DEV)
    gap[:, 2:2 + n] = False
    assert torch.equal(ys.view(torch.int32)[gap], sentinel[gap])


@mc_param
def test_gateup_indexed_and_refusals(arith):
    """Indexed gate/up: each (row, slot) equals the pair call on that expert's
    own gate and up handles; unequal shapes and the dot form are refused."""
    bits, group, n, k, e = 3, 64, 300, 1024, 6
    dg, du = _gateup_pair(bits, group, n, k, 9, 7700, n_experts=e)
    idx = np.array([[1, 1, 2], [1, 0, 5], [1, 3, 3], [1, 2, 0], [1, 4, 4],
                    [1, 5, 1], [0, 0, 0], [2, 1, 4], [3, 3, 1]], dtype=np.int32)
    tg = [dev(dg[key]) for key in ("words", "scales", "biases")]
    tu = [dev(du[key]) for key in ("words", "scales", "biases")]
    mf = arith
    gate = qgemv.Matrix(bits, group, n, k, *tg, n_experts=e, arith=mf)
    up = qgemv.Matrix(bits, group, n, k, *tu, n_experts=e, arith=mf)
    xt = dev(dg["x"])
    y = torch.empty((9, 3, n), dtype=torch.float32, device=DEV)
    assert qgemv.qgemv_run_gateup_indexed(gate.h, up.h, xt, 9, dev(idx), 3, y.view(-1)) == qgemv.QGEMV_OK
    y1 = torch.empty((1, n), dtype=torch.float32, device=DEV)
    views = {}
    for i in range(9):
        for s_ in range(3):
            ex = int(idx[i, s_])
            if ex not in views:
                views[ex] = (qgemv.Matrix(bits, group, n, k, tg[0][ex], tg[1][ex], tg[2][ex], arith=mf),
                             qgemv.Matrix(bits, group, n, k, tu[0][ex], tu[1][ex], tu[2][ex], arith=mf))
            vg, vu = views[ex]
            assert qgemv.qgemv_run_gateup(vg.h, vu.h, xt[i:i + 1], 1, y1, n) == qgemv.QGEMV_OK
            assert bits_equal(y1[0], y[i, s_]), (i, s_)
    # refusals
    dot_g = qgemv.Matrix(bits, group, n, k, tg[0][0], tg[1][0], tg[2][0], arith=qgemv.QGEMV_ARITH_DOT)
    dot_u = qgemv.Matrix(bits, group, n, k, tu[0][0], tu[1][0], tu[2][0], arith=qgemv.QGEMV_ARITH_DOT)
    assert qgemv.qgemv_run_gateup(dot_g.h, dot_u.h, xt, 1, y1, n) == qgemv.QGEMV_E_NOKERNEL
    vg0, _ = views[0]
    narrow = qgemv.Matrix(bits, group, n - 1, k, tu[0][0], tu[1][0], tu[2][0], arith=mf)
    assert qgemv.qgemv_run_gateup(vg0.h, narrow.h, xt, 1, y1, n) == qgemv.QGEMV_E_SHAPE


@mc_param
@pytest.mark.parametrize("k", [20480, 40960])
def test_indexed_narrow_windows_at_large_k(k, arith):
    """At K = 20480 four staged routed rows no longer fit one block's LDS, so
    indexed calls stage 2 rows a pass, and at K = 40960 one: the indexed
    kernels of those windows, each expert taking several passes.  Every (row,
    slot), plain and as a gate/up pair, equals the call on that expert's own
    handles bit for bit."""
    print_case("indexed large k", k, arith)
    bits, group, n, e = 4, 64, 40, 3
    dg, du = _gateup_pair(bits, group, n, k, 5, 7900 + k // 1024, n_experts=e)
    idx = np.array([[0, 2], [1, 1], [2, 0], [1, 2], [0, 0]], dtype=np.int32)
    tg = [dev(dg[key]) for key in ("words", "scales", "biases")]
    tu = [dev(du[key]) for key in ("words", "scales", "biases")]
    gate = qgemv.Matrix(bits, group, n, k, *tg, n_experts=e, arith=arith)
    up = qgemv.Matrix(bits, group, n, k, *tu, n_experts=e, arith=arith)
    xt = dev(dg["x"])
    ti = dev(idx)
    y = torch.empty((5, 2, n), dtype=torch.float32, device=DEV)
    yp = torch.empty((5, 2, n), dtype=torch.float32, device=DEV)
    gate.run_indexed(xt, ti, y.view(-1))
    assert qgemv.qgemv_run_gateup_indexed(gate.h, up.h, xt, 5, ti, 2, yp.view(-1)) == qgemv.QGEMV_OK
    y1 = torch.empty((1, n), dtype=torch.float32, device=DEV)
    for ex in range(e):
        vg = qgemv.Matrix(bits, group, n, k, tg[0][ex], tg[1][ex], tg[2][ex], arith=arith)
        vu = qgemv.Matrix(bits, group, n, k, tu[0][ex], tu[1][ex], tu[2][ex], arith=arith)
        for i, s_ in zip(*np.nonzero(idx == ex)):
            assert bits_equal(run(vg, xt[i:i + 1])[0], y[i, s_]), (ex, i, s_)
            assert qgemv.qgemv_run_gateup(vg.h, vu.h, xt[i:i + 1], 1, y1, n) == qgemv.QGEMV_OK
            assert bits_equal(y1[0], yp[i, s_]), (ex, i, s_)


def _dequant64(words, scales, biases, bits, group, n, k):
    q = oracle.unpack(words, bits, n, k).astype(np.float64)
    s = synth.bf16_bits_to_f32(scales).astype(np.float64)
    b = synth.bf16_bits_to_f32(biases).astype(np.float64)
    g = np.arange(k) // group
    return s[:, g] * q + b[:, g]


WIDEN = [(bi, gi, bo, go) for bi in (2, 3, 4, 5, 6, 8) for bo in (2, 3, 4, 5, 6, 8) if bo >= bi
         for gi in (32, 64, 128) for go in (32, 64, 128) if gi % go == 0]


def test_widen_is_exact():
    """For each source width, each target of at least as many bits, and each
    target group dividing the source group, the fp64 dequantized values are
    identical bit for bit (both experts of a two-expert stack); a target equal
    to the source returns identical bytes."""
    n, k, e = 6, 1024, 2
    for (bi, gi, bo, go) in WIDEN:
        d = synth.matrix(9100 + bi * 1000 + gi + bo * 7 + go, bi, gi, n, k, n_experts=e)
        tw, ts, tb = dev(d["words"]), dev(d["scales"]), dev(d["biases"])
        wo = torch.zeros((e, n, k * bo // 32), dtype=torch.int32, device=DEV)
        so = torch.zeros((e, n, k // go), dtype=torch.int16, device=DEV)
        bo_ = torch.zeros((e, n, k // go), dtype=torch.int16, device=DEV)
        rc = qgemv.qgemv_widen(bi, gi, n, k, tw, ts, tb, bo, go, wo, so, bo_, n_experts=e)
        assert rc == qgemv.QGEMV_OK, qgemv.qgemv_strerror(rc)
        torch.cuda.synchronize()
        w2 = wo.cpu().numpy().view(np.uint32)
        s2, b2 = so.cpu().numpy().view(np.uint16), bo_.cpu().numpy().view(np.uint16)
        for x in range(e):
            a = _dequant64(d["words"][x], d["scales"][x], d["biases"][x], bi, gi, n, k)
            c = _dequant64(w2[x], s2[x], b2[x], bo, go, n, k)
            assert np.array_equal(a.view(np.int64), c.view(np.int64)), (bi, gi, bo, go, x)
        if (bi, gi) == (bo, go):
            assert np.array_equal(w2, d["words"]) and np.array_equal(s2, d["scales"])


def test_widen_fused_members_in_order_and_products():
    """Two members of different widths, widened to their common width one call
    each into consecutive rows of one matrix, keep their values in order; the
    widened matrices' products, in every arithmetic form, meet the bound
    around the source's fp64 product (the dequantized values are the same; a
    smaller group re-associates the fp32 sums, so bit equality with the
    source's product is not expected)."""
    k = 2048
    members = [(4, 64, 100), (5, 128, 48)]
    rc, cb, cg = qgemv.qgemv_common_width([m[0] for m in members], [m[1] for m in members])
    assert (rc, cb, cg) == (0, 5, 64)
    rows = sum(m[2] for m in members)
    wo = torch.zeros((rows, k * cb // 32), dtype=torch.int32, device=DEV)
    so = torch.zeros((rows, k // cg), dtype=torch.int16, device=DEV)
    bo = torch.zeros((rows, k // cg), dtype=torch.int16, device=DEV)
    r0, srcs = 0, []
    for i, (bits, group, n) in enumerate(members):
        d = synth.matrix(9500 + i, bits, group, n, k)
        srcs.append(d)
        rc = qgemv.qgemv_widen(bits, group, n, k, dev(d["words"]), dev(d["scales"]), dev(d["biases"]),
                               cb, cg, wo[r0:], so[r0:], bo[r0:])
        assert rc == qgemv.QGEMV_OK
        r0 += n
    torch.cuda.synchronize()
    full = _dequant64(wo.cpu().numpy().view(np.uint32), so.cpu().numpy().view(np.uint16),
                      bo.cpu().numpy().view(np.uint16), cb, cg, rows, k)
    r0 = 0
    for (bits, group, n), d in zip(members, srcs):
        a = _dequant64(d["words"], d["scales"], d["biases"], bits, group, n, k)
        assert np.array_equal(a.view(np.int64), full[r0:r0 + n].view(np.int64))
        r0 += n
    # products of widened handles against the source's fp64 product
    for (bi, gi, bo_, go) in [(3, 64, 6, 32), (5, 128, 8, 64), (2, 128, 4, 128)]:
        n = 520
        d = synth.matrix(9600 + bi, bi, gi, n, k, 8)
        y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bi, gi, n, k)
        tw, ts, tb = dev(d["words"]), dev(d["scales"]), dev(d["biases"])
        w2 = torch.zeros((n, k * bo_ // 32), dtype=torch.int32, device=DEV)
        s2 = torch.zeros((n, k // go), dtype=torch.int16, device=DEV)
        b2 = torch.zeros((n, k // go), dtype=torch.int16, device=DEV)
        assert qgemv.qgemv_widen(bi, gi, n, k, tw, ts, tb, bo_, go, w2, s2, b2) == qgemv.QGEMV_OK
        xt = dev(d["x"])
        for arith in ARITHS:
            wid = qgemv.Matrix(bo_, go, n, k, w2, s2, b2, arith=arith)
            for m in (1, 8):
                y = run(wid, xt, m).cpu().numpy()
                check_bound(y, y64[:m], a64[:m], k, f"widen {bi}/{gi}->{bo_}/{go} arith {arith} m {m}")


@arith_param
@pytest.mark.parametrize("bits,group", PAIRS)
def test_exact_representable_inputs(bits, group, arith):
    """s in {2^-8, 2^-7, 2^-6}, bias a multiple of 2^-8, x in {-1, 0, 1}: every
    summation order is exact, so y must equal y64 exactly."""
    n, k = 72, 4096
    d = synth.exact_case(9000 + bits * 10 + group, bits, group, n, k, 16)
    mat = matrix_of(d, arith=arith)
    xt = dev(d["x"])
    y64, _, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k)
    for m in (1, 16):
        y = run(mat, xt, m).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, y64[:m]), f"m={m}"


# ---------------------------------------------------------------------------
# epilogue, stride, repeat, NaN
# ---------------------------------------------------------------------------

@arith_param
@pytest.mark.parametrize("bits,group", [(2, 32), (3, 64), (4, 64), (5, 128), (6, 32), (8, 128)])
def test_relu2_and_strided(bits, group, arith):
    print_case("relu2/strided", bits, group, arith)
    n, k = 1000, 2048      # ragged against every tile size
    d = synth.matrix(6000 + bits * 10 + group, bits, group, n, k, 8)
    mat = matrix_of(d, arith=arith)
    xt = dev(d["x"])
    y = run(mat, xt)
    r = run(mat, xt, epi=qgemv.QGEMV_EPI_RELU2)
    want = torch.where(y > 0, y * y, torch.zeros_like(y))
    assert bits_equal(r, want)
    r1 = run(mat, xt[3:4], epi=qgemv.QGEMV_EPI_RELU2)
    assert bits_equal(r1[0], r[3])
    y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k)
    tol = oracle.tol_relu2(y64, oracle.tol_y(a64, k))
    r64 = oracle.relu2(y64)
    assert np.all(np.abs(r.cpu().numpy() - r64) <= tol)
    # strided: a sentinel-filled wider output; gaps must keep their bytes
    ldy = n + 37
    sentinel = torch.full((8, ldy), 0x7FC0BEEF, dtype=torch.int32, device=DEV)
    ys = sentinel.clone().view(torch.float32)
    col = 5
    flat = ys.view(-1)[col:]
    mat.run_strided(xt, flat, ldy)
    assert bits_equal(ys[:, col:col + n], y)
    gap = torch.ones((8, ldy), dtype=torch.bool, device=DEV)
    gap[:, col:col + n] = False
    assert torch.equal(ys.view(torch.int32)[gap], sentinel[gap])
    # repeat: the same bytes
    y2 = run(mat, xt)
    assert bits_equal(y, y2)


@arith_param
def test_nan_row_stays_in_its_row(arith):
    bits, group, n, k = 4, 64, 512, 2048
    d = synth.matrix(77, bits, group, n, k, 3)
    x = d["x"].copy()
    x[1, 100] = 0x7FC0  # bf16 NaN
    mat = matrix_of(d, arith=arith)
    y = run(mat, dev(x)).cpu().numpy()
    yc = run(mat, dev(d["x"])).cpu().numpy()
    assert np.all(np.isnan(y[1]))
    assert np.array_equal(y[0].view(np.int32), yc[0].view(np.int32))
    assert np.array_equal(y[2].view(np.int32), yc[2].view(np.int32))


def test_refusals_leave_output_untouched():
    bits, group, n, k = 4, 64, 256, 2048
    d = synth.matrix(78, bits, group, n, k, 2)
    mat = matrix_of(d)
    xt = dev(d["x"])
    y = torch.full((2, n), 3.0, device=DEV)
    assert qgemv.qgemv_run(mat.h, xt, 0, y) == qgemv.QGEMV_OK
    assert qgemv.qgemv_run(mat.h, xt, qgemv.QGEMV_MAX_PROMPT + 1, y) == qgemv.QGEMV_E_WINDOW
    assert qgemv.qgemv_run_strided(mat.h, xt, 2, y, n - 1) == qgemv.QGEMV_E_STRIDE
    assert qgemv.qgemv_run(mat.h, xt, 2, xt) == qgemv.QGEMV_E_ALIAS
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)


# ---------------------------------------------------------------------------
# edge shapes: narrow, ragged, tiny K (one-unit geometry), one column
# ---------------------------------------------------------------------------

EDGE = [(6, 64, 48, 2048), (5, 128, 6192, 2048), (4, 32, 1, 2048), (3, 32, 33, 32),
        (5, 32, 65, 96), (6, 64, 17, 192), (2, 128, 129, 384), (8, 32, 3, 32), (3, 128, 40, 4096 + 128),
        # the shortest rows of the matrix-core form, N ragged against 16-column waves
        (4, 128, 1, 128), (8, 32, 17, 128), (2, 64, 100, 256), (6, 32, 1, 256), (3, 64, 33, 512),
        (5, 128, 31, 1024), (4, 32, 1000, 384)]


@arith_param
@pytest.mark.parametrize("bits,group,n,k", EDGE)
def test_edge_shapes(bits, group, n, k, arith):
    print_case("edge", bits, group, n, k, arith)
    d = synth.matrix(8000 + n + k, bits, group, n, k, 3)
    if arith in MC and k % qgemv.qgemv_mfma_codes(bits, group):
        with pytest.raises(qgemv.QgemvError, match="QGEMV_E_NOKERNEL"):
            matrix_of(d, arith=arith)
        return
    mat = matrix_of(d, arith=arith)
    xt = dev(d["x"])
    y3 = run(mat, xt)
    y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k)
    check_bound(y3.cpu().numpy(), y64, a64, k, f"edge {bits}/{group} {n}x{k}")
    for r in range(3):
        assert bits_equal(run(mat, xt[r:r + 1])[0], y3[r])
    codes = torch.empty((n, k), dtype=torch.uint8, device=DEV)
    mat.debug_unpack(codes)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.unpack(d["words"], bits, n, k))


# ---------------------------------------------------------------------------
# the named workloads at full size
# ---------------------------------------------------------------------------

def test_single_matrix_config():
    d = synth.single(m=1)
    n, k, bits, group = d["n"], d["k"], d["bits"], d["group"]
    mat = matrix_of(d)
    y = run(mat, dev(d["x"])).cpu().numpy()
    y64, a64, t64 = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k)
    frac = check_bound(y, y64, a64, k, "single")
    yb, _, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k, scale_mult=1.01)
    assert oracle.worst_fraction(np.abs(y - yb), oracle.tol_pages(t64, group, k)) > 1.0
    print_case(f"single: worst err/bound {frac:.4f}")


@pytest.mark.parametrize("m", [1, 16])
def test_stack_config(m):
    """Three runs (4/64 x 2048, 5/128 x 6192, 6/64 x 48) written by strided
    calls into one 8288-column output row."""
    st = synth.stack(m=m)
    k, ldy = st["k"], st["ldy"]
    xt = dev(st["x"])
    y = torch.full((m, ldy), float("nan"), device=DEV)
    flat = y.view(-1)
    mats = []
    for run_ in st["runs"]:
        d = dict(run_, n_experts=1)
        mat = matrix_of(d)
        mats.append(mat)
        mat.run_strided(xt, flat[run_["col"]:], ldy)
    for run_, mat in zip(st["runs"], mats):
        n, col = run_["n"], run_["col"]
        plain = run(mat, xt)
        assert bits_equal(y[:, col:col + n], plain)
        y64, a64, _ = oracle.gemv(run_["words"], run_["scales"], run_["biases"], st["x"],
                                  run_["bits"], run_["group"], n, k, threads=THREADS)
        check_bound(y[:, col:col + n].cpu().numpy(), y64, a64, k, f"stack run at {col}")
    assert not torch.any(torch.isnan(y))


@pytest.fixture(scope="module")
def lmhead():
    d = synth.lmhead(m=16)
    tw, ts, tb = dev(d["words"]), dev(d["scales"]), dev(d["biases"])
    d["mats"] = {a: qgemv.Matrix(d["bits"], d["group"], d["n"], d["k"], tw, ts, tb, arith=a)
                 for a in ARITHS + [qgemv.QGEMV_ARITH_AUTO]}
    d["xt"] = dev(d["x"])
    return d


@arith_param
def test_lmhead_every_column_one_row(lmhead, arith):
    """The 1-row LM head (the workload the benchmark times) against the
    threaded oracle at every one of its 248,320 columns."""
    d = lmhead
    n, k, bits, group = d["n"], d["k"], d["bits"], d["group"]
    y = run(d["mats"][arith], d["xt"], 1).cpu().numpy()
    if "y64_m1" not in d:
        d["y64_m1"] = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"][:1], bits, group, n, k,
                                  threads=THREADS)
    y64, a64, _ = d["y64_m1"]
    frac = check_bound(y, y64, a64, k, f"lmhead every column arith={arith}")
    print_case(f"  lmhead, all {n} columns: worst err/bound {frac:.4f}")


# about 2,200 tiles of 64 columns: more than the resident blocks of the
# whole chip (at most a few per CU), so each block walks several
MULTI_TILE = [(6, 32, 140000, 512), (4, 64, 141000, 256), (5, 128, 140100, 1024), (3, 32, 139900, 1024),
              (2, 128, 140007, 512), (8, 64, 140033, 256)]


@arith_param
@pytest.mark.parametrize("bits,group,n,k", MULTI_TILE)
def test_blocks_walking_several_tiles(bits, group, n, k, arith):
    """Shapes with more column tiles than the resident grid holds, so that
    every block walks several tiles and reuses its staged window: every
    column against the oracle at 1 and 4 rows, and the 4-row window's rows
    equal to their 1-row calls bit for bit."""
    print_case("multi-tile", bits, group, n, k, arith)
    d = synth.matrix(8800 + bits * 10 + group, bits, group, n, k, 4)
    mat = matrix_of(d, arith=arith)
    xt = dev(d["x"])
    y4 = run(mat, xt)
    y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k, threads=THREADS)
    check_bound(y4.cpu().numpy(), y64, a64, k, f"multi-tile {bits}/{group} {n}x{k}")
    for r in range(4):
        assert bits_equal(run(mat, xt[r:r + 1])[0], y4[r]), f"row {r}"


@mc_param
def test_many_tiles_consecutive_calls(arith):
    """Matrix-core plain and strided calls with more column tiles than the
    resident blocks hold: their rows equal those of a 17-row prompt window
    (two passes over the tiles) bit for bit; consecutive calls on a large and
    then a smaller matrix, and a strided call, write every column, and the
    strided call leaves its gaps untouched."""
    print_case("many tiles, consecutive calls", arith)
    big = synth.matrix(8900, 6, 32, 100000, 512, 17)
    small = synth.matrix(8901, 4, 64, 70001, 256, 3)
    mb, ms = matrix_of(big, arith=arith), matrix_of(small, arith=arith)
    xb, xs = dev(big["x"]), dev(small["x"])
    y17 = run(mb, xb, 17)                           # two passes of window rows
    sent = 0x7FC0BEEF
    for rep in range(3):
        yb = torch.full((2, 100000), sent, dtype=torch.int32, device=DEV).view(torch.float32)
        mb.run(xb[:2], yb, m=2)
        ys = torch.full((3, 70001), sent, dtype=torch.int32, device=DEV).view(torch.float32)
        ms.run(xs, ys, m=3)
        y1 = run(mb, xb[5:6], 1)
        assert bits_equal(yb, y17[:2]), rep
        assert bits_equal(y1[0], y17[5]), rep
        assert not torch.any(ys.view(torch.int32) == sent), rep
    y64, a64, _ = oracle.gemv(small["words"], small["scales"], small["biases"], small["x"], 4, 64, 70001, 256,
                              threads=THREADS)
    check_bound(ys.cpu().numpy(), y64, a64, 256, "many tiles, smaller matrix")
    # strided: gaps untouched, columns equal the plain call's
    ldy = 100003
    wide = torch.full((2, ldy), sent, dtype=torch.int32, device=DEV)
    yw = wide.clone().view(torch.float32)
    mb.run_strided(xb[:2], yw.view(-1)[2:], ldy, m=2)
    assert bits_equal(yw[:, 2:2 + 100000], y17[:2])
    gap = torch.ones((2, ldy), dtype=torch.bool, device=DEV)
    gap[:, 2:2 + 100000] = False
    assert torch.equal(yw.view(torch.int32)[gap], wide[gap])


# (bits, group, K): every width and both scale layouts at K = 2048, the 5-bit
# blocks of 7 and 8 waves, and rows of 3, 6 and 8 two-group stages
HANDOUT = [(2, 32, 2048), (3, 64, 2048), (4, 64, 2048), (4, 128, 2048), (5, 32, 2048), (5, 128, 2048),
           (6, 32, 2048), (8, 64, 2048), (8, 128, 2048), (4, 64, 1536), (8, 32, 1536), (2, 128, 3072),
           (4, 64, 4096)]


@mc_param
@pytest.mark.parametrize("bits,group,k", HANDOUT)
def test_unit_handout_equals_tile_walk(bits, group, k, arith):
    """A matrix of 100,000 columns runs the kernels that hand out 16-column
    units inside one block per CU (2-, 4- and 8-bit codes two load groups a
    stage); its first 40,000 columns, as a matrix of their own, run the tile
    walk with no K split.  The shared columns agree bit for bit at 1, 4 and 16
    rows, with activations whose unit dots round; sampled columns are held
    to the oracle's bound; the relu2 epilogue and a strided output of the
    large matrix hold the plain call's bits, and the gaps keep their bytes."""
    print_case("unit handout vs tile walk", bits, group, k, arith)
    n, n_small = 100000, 40000
    rng = np.random.default_rng(9100 + 10 * bits + group + k)
    words = synth.draw_words(rng, (n,), k, bits)
    scales = synth.draw_scales(rng, (n, k // group))
    biases = synth.draw_biases(rng, (n, k // group))
    x = synth.draw_x_wide(rng, 16, k)
    tw, ts, tb = dev(words), dev(scales), dev(biases)
    big = qgemv.Matrix(bits, group, n, k, tw, ts, tb, arith=arith)
    small = qgemv.Matrix(bits, group, n_small, k, tw[:n_small], ts[:n_small], tb[:n_small], arith=arith)
    xt = dev(x)
    cols = np.unique(np.concatenate([np.arange(0, n, 997), [n_small - 1, n_small, n - 1]]))
    y64, a64, _ = oracle.gemv(words[cols], scales[cols], biases[cols], x, bits, group, len(cols), k,
                              threads=THREADS)
    for m in (1, 4, 16):
        yb, ys = run(big, xt, m), run(small, xt, m)
        assert bits_equal(yb[:, :n_small], ys), f"m={m}"
        check_bound(yb.cpu().numpy()[:, cols], y64[:m], a64[:m], k, f"unit handout {bits}/{group} m={m}")
    # the same kernels with the relu2 epilogue and through an output row
    # stride: relu2 of the plain call's bits, gaps untouched
    r = run(big, xt, 4, epi=qgemv.QGEMV_EPI_RELU2)
    assert bits_equal(r, torch.where(yb[:4] > 0, yb[:4] * yb[:4], torch.zeros_like(yb[:4])))
    ldy, col = n + 19, 3
    sentinel = torch.full((4, ldy), 0x7FC0BEEF, dtype=torch.int32, device=DEV)
    yw = sentinel.clone().view(torch.float32)
    big.run_strided(xt[:4], yw.view(-1)[col:], ldy, m=4)
    assert bits_equal(yw[:, col:col + n], yb[:4])
    gap = torch.ones((4, ldy), dtype=torch.bool, device=DEV)
    gap[:, col:col + n] = False
    assert torch.equal(yw.view(torch.int32)[gap], sentinel[gap])


@mc_param
@pytest.mark.parametrize("bits,group", [(2, 32), (3, 64), (4, 64), (5, 32), (5, 128), (6, 32), (8, 128)])
def test_four_wave_blocks_equal_eight(bits, group, arith):
    """Small matrices run 8- and 16-row windows of the tile walk in blocks of
    4 waves (blocks of 8 would cover at most half the CUs).  At K = 2048 a
    4096-column matrix and a larger one split K alike (in 4 parts, or in 2
    for 3- and 5-bit codes, whose rows hold two load groups), and the first
    takes 4-wave blocks, the second (8192 columns, or 16384 at a split of 2)
    8-wave ones.  The larger matrix's first 4096 columns are the smaller
    matrix: they agree bit for bit at 8 and 16 rows (and at a 12-row window),
    with activations whose unit dots round, and the 4096-column outputs stay
    within the oracle's bound."""
    print_case("4-wave blocks", bits, group, arith)
    n, k, n_small = (16384 if bits in (3, 5) else 8192), 2048, 4096
    rng = np.random.default_rng(9400 + 10 * bits + group)
    words = synth.draw_words(rng, (n,), k, bits)
    scales = synth.draw_scales(rng, (n, k // group))
    biases = synth.draw_biases(rng, (n, k // group))
    x = synth.draw_x_wide(rng, 16, k)
    tw, ts, tb = dev(words), dev(scales), dev(biases)
    big = qgemv.Matrix(bits, group, n, k, tw, ts, tb, arith=arith)
    small = qgemv.Matrix(bits, group, n_small, k, tw[:n_small], ts[:n_small], tb[:n_small], arith=arith)
    xt = dev(x)
    y64, a64, _ = oracle.gemv(words[:n_small], scales[:n_small], biases[:n_small], x, bits, group, n_small, k,
                              threads=THREADS)
    for m in (8, 12, 16):
        ys = run(small, xt, m)
        assert bits_equal(run(big, xt, m)[:, :n_small], ys), f"m={m}"
        check_bound(ys.cpu().numpy(), y64[:m], a64[:m], k, f"4-wave blocks {bits}/{group} m={m}")


@pytest.mark.parametrize("bits,group", [(8, 32), (4, 128)])
def test_unit_handout_scales_only_4_byte_aligned(bits, group):
    """The unit-handout kernels load a stage's two groups' dword scales of a
    column at once (16 bytes at 8/32, 8 at 4/128), so they need 16- or
    8-byte aligned scale and bias arrays; with arrays 4 bytes off that, a
    large matrix takes the tile walk, and its outputs hold the same bits as
    with aligned arrays."""
    print_case("unit handout, scales 4 bytes off", bits, group)
    n, k = 100000, 2048
    rng = np.random.default_rng(9300 + bits + group)
    words = synth.draw_words(rng, (n,), k, bits)
    scales = synth.draw_scales(rng, (n, k // group))
    biases = synth.draw_biases(rng, (n, k // group))
    x = synth.draw_x_wide(rng, 4, k)
    tw, xt = dev(words), dev(x)

    def shifted(a):
        # the same values from 4 bytes past a 256-byte aligned allocation
        t = torch.zeros(a.size + 2, dtype=torch.int16, device=DEV)
        t[2:] = dev(a).view(-1)
        return t[2:].view(a.shape)

    aligned = qgemv.Matrix(bits, group, n, k, tw, dev(scales), dev(biases))
    ss, bb = shifted(scales), shifted(biases)
    assert ss.data_ptr() % 16 == 4 and bb.data_ptr() % 16 == 4
    off = qgemv.Matrix(bits, group, n, k, tw, ss, bb)
    for m in (1, 4):
        assert bits_equal(run(aligned, xt, m), run(off, xt, m)), f"m={m}"


@pytest.mark.parametrize("arith", ARITHS + [qgemv.QGEMV_ARITH_AUTO], ids=ARITH_IDS + ["auto"])
@pytest.mark.parametrize("m", [1, 8, 16])
def test_lmhead_sampled(lmhead, m, arith):
    d = lmhead
    n, k, bits, group = d["n"], d["k"], d["bits"], d["group"]
    mat = d["mats"][arith]
    y = run(mat, d["xt"], m)
    rng = np.random.default_rng(m)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                     rng.integers(0, n, 384)]))
    y64, a64, _ = oracle.gemv(d["words"][cols], d["scales"][cols], d["biases"][cols], d["x"][:m],
                              bits, group, len(cols), k, threads=THREADS)
    check_bound(y[:, cols].cpu().numpy(), y64, a64, k, f"lmhead m={m}")
    # the same rows alone, at full size
    for r in sorted({0, m - 1, m // 2}):
        assert bits_equal(run(mat, d["xt"][r:r + 1])[0], y[r])


@pytest.fixture(scope="module")
def experts():
    d = synth.experts()
    d["tw"], d["ts"], d["tb"] = dev(d["words"]), dev(d["scales"]), dev(d["biases"])
    return d


@arith_param
@pytest.mark.parametrize("epi", [0, 1])
def test_indexed_experts_config(experts, epi, arith):
    d = experts
    n, k, m, slots = d["n"], d["k"], d["idx"].shape[0], d["idx"].shape[1]
    xt = dev(d["x"])
    it = dev(d["idx"])
    y = torch.empty((m, slots, n), dtype=torch.float32, device=DEV)
    mat = qgemv.Matrix(d["bits"], d["group"], n, k, d["tw"], d["ts"], d["tb"], n_experts=d["n_experts"],
                       arith=arith)
    mat.run_indexed(xt, it, y.view(-1), epi=epi)
    # each (row, slot) equals the plain call on the expert's own handle
    wpr = d["words"].shape[-1]
    gpr = d["scales"].shape[-1]
    views = {}
    for i in range(m):
        for s in range(slots):
            e = int(d["idx"][i, s])
            if e not in views:
                views[e] = qgemv.Matrix(d["bits"], d["group"], n, k, d["tw"][e], d["ts"][e], d["tb"][e],
                                        arith=arith)
            yp = run(views[e], xt[i:i + 1], epi=epi)
            assert bits_equal(yp[0], y[i, s]), (i, s, e)
    assert wpr and gpr
    y64, a64, _ = oracle.gemv_indexed(d["words"], d["scales"], d["biases"], d["x"], d["idx"],
                                      d["bits"], d["group"], n, k, threads=THREADS)
    tol = oracle.tol_y(a64, k)
    got = y.cpu().numpy()
    if epi:
        tol = oracle.tol_relu2(y64, tol)
        y64 = oracle.relu2(y64)
    assert np.all(np.abs(got - y64) <= tol)


@arith_param
def test_indexed_out_of_range_slots_write_nothing(arith):
    """idx values outside [0, n_experts) (-1, n_experts, large) are a caller
    precondition: the kernels only match valid expert ids, so such slots keep
    their bytes and every other slot equals the plain call on its expert's
    own handle; the checked mode names the table QGEMV_E_INDEX.  Indexed
    gate/up pairs likewise (matrix-core forms)."""
    bits, group, n, k, e = 4, 64, 200, 1024, 5
    d = synth.matrix(4300, bits, group, n, k, 6, n_experts=e)
    idx = np.array([[0, -1, 4], [e, 2, 2], [1, 3, 1 << 20], [-7, -1, e], [4, 0, 3], [2, e + 1, 1]],
                   dtype=np.int32)
    tw, ts, tb = dev(d["words"]), dev(d["scales"]), dev(d["biases"])
    mat = qgemv.Matrix(bits, group, n, k, tw, ts, tb, n_experts=e, arith=arith)
    xt = dev(d["x"])
    ti = dev(idx)
    sentinel = torch.full((6, 3, n), 0x7FC0BEEF, dtype=torch.int32, device=DEV)
    y = sentinel.clone().view(torch.float32)
    mat.run_indexed(xt, ti, y.view(-1), epi=qgemv.QGEMV_EPI_RELU2)
    views = {}
    for i in range(6):
        for s_ in range(3):
            ex = int(idx[i, s_])
            if not 0 <= ex < e:
                assert torch.equal(y[i, s_].view(torch.int32), sentinel[i, s_]), (i, s_, ex)
                continue
            if ex not in views:
                views[ex] = qgemv.Matrix(bits, group, n, k, tw[ex], ts[ex], tb[ex], arith=arith)
            assert bits_equal(run(views[ex], xt[i:i + 1], epi=qgemv.QGEMV_EPI_RELU2)[0], y[i, s_]), (i, s_)
    assert qgemv.qgemv_check_indices(mat.h, ti, 6, 3) == qgemv.QGEMV_E_INDEX
    good = dev(np.clip(idx, 0, e - 1).astype(np.int32))
    assert qgemv.qgemv_check_indices(mat.h, good, 6, 3) == qgemv.QGEMV_OK
    if arith == qgemv.QGEMV_ARITH_DOT:
        return
    du = synth.matrix(4301, bits, group, n, k, n_experts=e)
    tu = [dev(du[key]) for key in ("words", "scales", "biases")]
    up = qgemv.Matrix(bits, group, n, k, *tu, n_experts=e, arith=arith)
    yp = sentinel.clone().view(torch.float32)
    assert qgemv.qgemv_run_gateup_indexed(mat.h, up.h, xt, 6, ti, 3, yp.view(-1)) == qgemv.QGEMV_OK
    y1 = torch.empty((1, n), dtype=torch.float32, device=DEV)
    for i in range(6):
        for s_ in range(3):
            ex = int(idx[i, s_])
            if not 0 <= ex < e:
                assert torch.equal(yp[i, s_].view(torch.int32), sentinel[i, s_]), (i, s_, ex)
                continue
            vu = qgemv.Matrix(bits, group, n, k, tu[0][ex], tu[1][ex], tu[2][ex], arith=arith)
            assert qgemv.qgemv_run_gateup(views[ex].h, vu.h, xt[i:i + 1], 1, y1, n) == qgemv.QGEMV_OK
            assert bits_equal(y1[0], yp[i, s_]), (i, s_)


@arith_param
def test_indexed_small_stack_repeats_and_duplicates(arith):
    """A routing table that names one expert twice in a row and gives one
    expert more rows than one staging pass holds."""
    bits, group, n, k, e = 3, 64, 300, 1024, 6
    d = synth.matrix(4242, bits, group, n, k, 9, n_experts=e)
    idx = np.array([[1, 1, 2], [1, 0, 5], [1, 3, 3], [1, 2, 0], [1, 4, 4],
                    [1, 5, 1], [0, 0, 0], [2, 1, 4], [3, 3, 1]], dtype=np.int32)
    tw, ts, tb = dev(d["words"]), dev(d["scales"]), dev(d["biases"])
    mat = qgemv.Matrix(bits, group, n, k, tw, ts, tb, n_experts=e, arith=arith)
    xt = dev(d["x"])
    y = torch.empty((9, 3, n), dtype=torch.float32, device=DEV)
    mat.run_indexed(xt, dev(idx), y.view(-1))
    for i in range(9):
        for s in range(3):
            ex = int(idx[i, s])
            v = qgemv.Matrix(bits, group, n, k, tw[ex], ts[ex], tb[ex], arith=arith)
            assert bits_equal(run(v, xt[i:i + 1])[0], y[i, s]), (i, s)


# ---------------------------------------------------------------------------
# fused stacks: one dispatch, each member equal to its run's strided call
# ---------------------------------------------------------------------------

def _offset_by_one(a: np.ndarray):
    """A device copy of a bf16 array that starts 2 bytes into its buffer (so
    it is 2-byte but not 4-byte aligned)."""
    buf = torch.zeros(a.size + 1, dtype=torch.int16, device=DEV)
    buf[1:] = dev(a.reshape(-1))
    return buf[1:]


def _stack_runs(specs, k, seed):
    """specs: [(bits, group, [(rows, col), ...])] or (..., misaligned): with
    misaligned true the run's scales and biases are only 2-byte aligned.
    Returns runs for qgemv.Stack plus the host copies."""
    runs, host = [], []
    for i, spec in enumerate(specs):
        bits, group, members = spec[:3]
        mis = len(spec) > 3 and spec[3]
        n = sum(r for r, _ in members)
        d = synth.matrix(seed + i, bits, group, n, k)
        host.append(d)
        put = _offset_by_one if mis else dev
        runs.append(dict(bits=bits, group=group, n=n, k=k, w=dev(d["words"]), scales=put(d["scales"]),
                         biases=put(d["biases"]), members=members))
    return runs, host


def _check_stack(specs, k, ldy, m, seed, epi=0):
    runs, host = _stack_runs(specs, k, seed)
    rng = np.random.default_rng(seed)
    x = synth.draw_x(rng, m, k)
    xt = dev(x)
    st = qgemv.Stack(runs, ldy)
    sentinel = torch.full((m, ldy), 0x7FC0BEEF, dtype=torch.int32, device=DEV)
    y = sentinel.clone().view(torch.float32)
    st.run(xt, y.view(-1), epi=epi)
    covered = torch.zeros((m, ldy), dtype=torch.bool, device=DEV)
    for r, d in zip(runs, host):
        mat = qgemv.Matrix(r["bits"], r["group"], r["n"], k, r["w"], r["scales"], r["biases"])
        plain = run(mat, xt, epi=epi)
        row0 = 0
        for rows, col in r["members"]:
            assert bits_equal(y[:, col:col + rows], plain[:, row0:row0 + rows]), (r["bits"], col)
            covered[:, col:col + rows] = True
            row0 += rows
        y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], x, r["bits"], r["group"], r["n"], k,
                                  threads=THREADS)
        if not epi:
            check_bound(plain.cpu().numpy(), y64, a64, k, f"stack run {r['bits']}/{r['group']}")
    assert torch.equal(y.view(torch.int32)[~covered], sentinel[~covered])


@pytest.mark.parametrize("m", [1, 16])
def test_fused_stack_config(m):
    """The stack workload in one dispatch: 4/64 x 2048 at column 0, the 5/128
    run of two members (6144 + 48) at 2048, 6/64 x 48 at 8240; ldy 8288."""
    print_case("fused stack", m)
    specs = [(4, 64, [(2048, 0)]), (5, 128, [(6144, 2048), (48, 8192)]), (6, 64, [(48, 8240)])]
    _check_stack(specs, synth.STACK_K, synth.STACK_LDY, m, 3100 + m)


def test_fused_stack_column_map_gaps():
    """Members of one run placed apart, runs interleaved, gaps untouched."""
    specs = [(5, 128, [(6144, 2100), (48, 8400)]), (4, 64, [(2048, 0)]), (6, 64, [(48, 8300)])]
    _check_stack(specs, 2048, 9000, 3, 3200)


@pytest.mark.parametrize("epi", [0, 1])
def test_fused_stack_all_widths(epi):
    """Every width in one stack, members of different sizes, K = 4096."""
    specs = [(2, 32, [(300, 5000)]), (3, 64, [(128, 0), (72, 4000)]), (4, 128, [(512, 200)]),
             (5, 32, [(64, 712)]), (6, 128, [(1000, 3000)]), (8, 64, [(256, 776), (16, 1100)])]
    _check_stack(specs, 4096, 5400, 5, 3300 + epi, epi)


def test_fused_stack_both_forms():
    """A stack whose runs take both arithmetic forms, so that one call makes
    both dispatches: at K = 65536 the 3- and 6-bit runs' windows no longer fit
    the matrix-core form's LDS and take the dot form, while the 4-bit run
    keeps the matrix cores.  Each member equals its run's own call."""
    k = 65536
    specs = [(4, 64, [(200, 0)]), (6, 64, [(72, 300), (24, 200)]), (3, 64, [(96, 400)])]
    fake = (0x1000000, 0x20000000, 0x30000000)
    forms = []
    for bits, group, members in specs:
        rc, h = qgemv.qgemv_create_arith(bits, group, sum(r for r, _ in members), k, *fake,
                                         qgemv.QGEMV_ARITH_AUTO, 1)
        assert rc == qgemv.QGEMV_OK
        forms.append(qgemv.qgemv_arith(h))
        qgemv.qgemv_destroy(h)
    assert forms == [qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_DOT, qgemv.QGEMV_ARITH_DOT], forms
    print_case("fused stack, both forms", k)
    _check_stack(specs, k, 520, 1, 3400)


def test_fused_stack_dot_runs_by_alignment():
    """At K = 2048 a stack's runs whose scales and biases are only 2-byte
    aligned (which the matrix-core form does not take) run in the dot form,
    the others on the matrix cores: two dispatches, each member equal to its
    run's own call, gaps untouched."""
    k = 2048
    specs = [(4, 64, [(200, 0)]), (6, 64, [(72, 300), (24, 200)], True), (3, 64, [(96, 400)], True),
             (5, 128, [(600, 520)])]
    runs, _ = _stack_runs(specs, k, 3450)
    forms = [qgemv.Matrix(r["bits"], r["group"], r["n"], k, r["w"], r["scales"], r["biases"]).arith for r in runs]
    assert forms == [qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_DOT, qgemv.QGEMV_ARITH_DOT,
                     qgemv.QGEMV_ARITH_MFMA], forms
    print_case("fused stack, runs of both forms by alignment", k)
    _check_stack(specs, k, 1200, 3, 3450)


# ---------------------------------------------------------------------------
# seeded random shapes across widths, groups, forms and windows
# ---------------------------------------------------------------------------

def _random_cases(count=40, seed=20260):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        bits, group = PAIRS[int(rng.integers(len(PAIRS)))]
        arith = ARITHS[int(rng.integers(len(ARITHS)))]
        step = qgemv.qgemv_mfma_codes(bits, group) if arith != qgemv.QGEMV_ARITH_DOT else group
        k = step * int(rng.integers(1, max(2, 4096 // step) + 1))
        n = int(rng.integers(1, 2600))
        top = qgemv.QGEMV_MAX_PROMPT if arith != qgemv.QGEMV_ARITH_DOT else qgemv.QGEMV_MAX_WINDOW
        m = int(rng.integers(1, top + 1))
        if n * k * m > 12_000_000 or k > 4096:
            continue
        cases.append((bits, group, n, k, m, arith, int(rng.integers(1 << 30))))
    return cases


def _random_auto_cases(count=24, seed=20261):
    """The library's choice at matrix-core shapes, windows of 1 to 65 rows;
    every other case with activations whose unit dots round."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        bits, group = PAIRS[int(rng.integers(len(PAIRS)))]
        step = qgemv.qgemv_mfma_codes(bits, group)
        k = step * int(rng.integers(1, max(2, 4096 // step) + 1))
        n = int(rng.integers(1, 2600))
        m = int(rng.integers(1, qgemv.QGEMV_MAX_PROMPT + 1))
        if n * k * m > 12_000_000 or k > 4096:
            continue
        cases.append((bits, group, n, k, m, qgemv.QGEMV_ARITH_AUTO, int(rng.integers(1 << 30)), len(cases) % 2 == 1))
    return cases


@pytest.mark.parametrize("bits,group,n,k,m,arith,seed,wide_x",
                         [c + (False,) for c in _random_cases()] + _random_auto_cases())
def test_random_shapes(bits, group, n, k, m, arith, seed, wide_x):
    """Random (seeded) shapes: ragged N, every admissible K of the form up to
    4096, windows up to the form's limit (the library's choice too, which
    mixes the block-diagonal and wide kernels by window, some with
    activations over 2^+-24).  Outputs meet the bound; two rows equal their
    1-row calls bit for bit; a strided call equals the plain one and leaves
    the gaps untouched."""
    print_case("random", bits, group, n, k, m, arith, seed, "wide-range x" if wide_x else "")
    d = synth.matrix(seed, bits, group, n, k, m)
    if wide_x:
        d["x"] = synth.draw_x_wide(np.random.default_rng(seed + 1), m, k)
    try:
        mat = matrix_of(d, arith=arith)
    except qgemv.QgemvError as e:
        # the dot form's fast and generic kernels take every admitted K; a
        # window too wide for LDS is the only refusal expected here
        assert arith == qgemv.QGEMV_ARITH_DOT and "WINDOW" in str(e), str(e)
        return
    xt = dev(d["x"])
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    try:
        mat.run(xt, y, m=m)
    except qgemv.QgemvError as e:
        assert arith == qgemv.QGEMV_ARITH_DOT and "QGEMV_E_WINDOW" in str(e), str(e)
        return
    y64, a64, _ = oracle.gemv(d["words"], d["scales"], d["biases"], d["x"], bits, group, n, k, threads=THREADS)
    check_bound(y.cpu().numpy(), y64, a64, k, f"random {bits}/{group} {n}x{k} m={m} arith={arith}")
    for r in sorted({0, m - 1, m // 2}):
        assert bits_equal(run(mat, xt[r:r + 1])[0], y[r]), f"row {r}"
    ldy = n + 3
    sentinel = torch.full((m, ldy), 0x7FC0BEEF, dtype=torch.int32, device=DEV)
    ys = sentinel.clone().view(torch.float32)
    mat.run_strided(xt, ys.view(-1)[1:], ldy, m=m)
    assert bits_equal(ys[:, 1:1 + n], y)
    gap = torch.ones((m, ldy), dtype=torch.bool, device=DEV)
    gap[:, 1:1 + n] = False
    assert torch.equal(ys.view(torch.int32)[gap], sentinel[gap])


# ---------------------------------------------------------------------------
# HIP graph capture: launch-bound callers replay captured calls
# ---------------------------------------------------------------------------

def test_graph_replay_equals_eager():
    """Plain, strided, fused-stack, indexed (relu2) and many-tile plain calls
    captured in one
    HIP graph and replayed three times, with eager calls and output resets
    between the replays: every replay's outputs equal the eager calls' bit for
    bit, and the strided call's gaps keep their bytes (the library records no
    memset or host work into a graph)."""
    print_case("graph replay")
    k = 2048
    d1 = synth.matrix(8100, 6, 32, 1000, k, 3)
    plain = matrix_of(d1)
    x1 = dev(d1["x"])
    d2 = synth.matrix(8101, 4, 64, 256, k)
    strided = matrix_of(d2)
    ldy = 300
    specs = [(4, 64, [(256, 0)]), (5, 128, [(192, 256), (8, 500)]), (6, 64, [(48, 448)])]
    runs, _ = _stack_runs(specs, k, 8102)
    stack = qgemv.Stack(runs, 512)
    bits, group, n, ke, e = 3, 64, 300, 1024, 6
    d3 = synth.matrix(8103, bits, group, n, ke, 9, n_experts=e)
    experts = qgemv.Matrix(bits, group, n, ke, dev(d3["words"]), dev(d3["scales"]), dev(d3["biases"]),
                           n_experts=e)
    x3 = dev(d3["x"])
    idx = dev(np.array([[1, 1, 2], [1, 0, 5], [1, 3, 3], [1, 2, 0], [1, 4, 4],
                        [1, 5, 1], [0, 0, 0], [2, 1, 4], [3, 3, 1]], dtype=np.int32))
    sentinel = torch.full((3, ldy), 0x7FC0BEEF, dtype=torch.int32, device=DEV)
    gap = torch.ones((3, ldy), dtype=torch.bool, device=DEV)
    gap[:, 10:10 + 256] = False
    # a matrix of more column tiles than the resident blocks hold
    d4 = synth.matrix(8104, 6, 32, 90000, 512, 3)
    many = matrix_of(d4)
    x4 = dev(d4["x"])

    def outputs():
        return (torch.empty((3, 1000), dtype=torch.float32, device=DEV),
                sentinel.clone().view(torch.float32),
                torch.zeros((3, 512), dtype=torch.float32, device=DEV),
                torch.empty((9, 3, n), dtype=torch.float32, device=DEV),
                torch.empty((3, 90000), dtype=torch.float32, device=DEV))

    def launch(outs, s):
        yp, ys, yk, yi, yd = outs
        assert qgemv.qgemv_run(plain.h, x1, 3, yp, 0, s) == qgemv.QGEMV_OK
        assert qgemv.qgemv_run_strided(strided.h, x1, 3, ys.view(-1)[10:], ldy, 0, s) == qgemv.QGEMV_OK
        assert qgemv.qgemv_stack_run(stack.h, x1, 3, yk, 0, s) == qgemv.QGEMV_OK
        assert qgemv.qgemv_run_indexed(experts.h, x3, 9, idx, 3, yi.view(-1), qgemv.QGEMV_EPI_RELU2, s) \
            == qgemv.QGEMV_OK
        assert qgemv.qgemv_run(many.h, x4, 3, yd, 0, s) == qgemv.QGEMV_OK

    eager = outputs()
    launch(eager, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    graphed = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(graphed, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(graphed, torch.cuda.current_stream().cuda_stream)
    other = outputs()
    for rep in range(3):
        # back to each output's initial bytes (the stack's output starts at
        # zero, so its unwritten columns are checked too)
        graphed[0].view(torch.int32).fill_(0x7FC0BEEF)
        graphed[1].view(torch.int32).copy_(sentinel)
        graphed[2].zero_()
        graphed[3].view(torch.int32).fill_(0x7FC0BEEF)
        graphed[4].view(torch.int32).fill_(0x7FC0BEEF)
        launch(other, torch.cuda.current_stream().cuda_stream)   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, graphed):
            assert bits_equal(a, b), rep
        assert torch.equal(graphed[1].view(torch.int32)[gap], sentinel[gap]), rep
