"""Host-side checks of the C ABI that need no GPU: the library loads, it
exports every entry point include/qgemv.h declares, and every refusal is
returned by name before any HIP call."""

import ctypes
import os
import re

import pytest

from bit_affine_quantized_amd import qgemv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")

# Fake, suitably aligned device addresses: create() never dereferences them.
W, S, B, X, Y, IDX = 0x100000, 0x200000, 0x300000, 0x400000, 0x800000, 0xC00000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = qgemv.load()
    names = declared_functions()
    assert {"qgemv_create", "qgemv_run", "qgemv_run_strided", "qgemv_run_indexed",
            "qgemv_destroy", "qgemv_strerror", "qgemv_debug_unpack"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_names():
    for code, name in [(0, "QGEMV_OK"), (-1, "QGEMV_E_ARG"), (-2, "QGEMV_E_BITS"), (-3, "QGEMV_E_GROUP"),
                       (-4, "QGEMV_E_SHAPE"), (-5, "QGEMV_E_STRIDE"), (-6, "QGEMV_E_ALIGN"),
                       (-7, "QGEMV_E_WINDOW"), (-8, "QGEMV_E_ALIAS"), (-9, "QGEMV_E_NOKERNEL"),
                       (-10, "QGEMV_E_HIP"), (-11, "QGEMV_E_INDEX")]:
        assert qgemv.qgemv_strerror(code) == name
    assert qgemv.qgemv_strerror(12345) == "QGEMV_E_UNKNOWN"


@pytest.mark.parametrize("bits,group,n,k,w,want", [
    (7, 64, 16, 2048, W, qgemv.QGEMV_E_BITS),
    (1, 64, 16, 2048, W, qgemv.QGEMV_E_BITS),
    (4, 16, 16, 2048, W, qgemv.QGEMV_E_GROUP),
    (4, 256, 16, 2048, W, qgemv.QGEMV_E_GROUP),
    (4, 64, 0, 2048, W, qgemv.QGEMV_E_SHAPE),
    (4, 64, 16, 0, W, qgemv.QGEMV_E_SHAPE),
    (4, 64, 16, 2080, W, qgemv.QGEMV_E_SHAPE),   # group does not divide K
    (4, 64, 16, 2048, 0, qgemv.QGEMV_E_ARG),     # null weights
    (4, 64, 16, 2048, W + 4, qgemv.QGEMV_E_ALIGN),
])
def test_create_refusals(bits, group, n, k, w, want):
    rc, h = qgemv.qgemv_create(bits, group, n, k, w, S, B)
    assert rc == want and h is None


def test_create_refuses_misaligned_scales_and_bad_experts():
    assert qgemv.qgemv_create(4, 64, 16, 2048, W, S + 1, B)[0] == qgemv.QGEMV_E_ALIGN
    assert qgemv.qgemv_create(4, 64, 16, 2048, W, S, B + 1)[0] == qgemv.QGEMV_E_ALIGN
    assert qgemv.qgemv_create(4, 64, 16, 2048, W, S, B, n_experts=0)[0] == qgemv.QGEMV_E_SHAPE
    assert qgemv.qgemv_create(4, 64, 16, 2048, W, 0, B)[0] == qgemv.QGEMV_E_ARG


def test_create_accepts_every_pair_without_a_device():
    for bits in (2, 3, 4, 5, 6, 8):
        for group in (32, 64, 128):
            for k in (group, 2048, 4096, 96 * group // 32 if group == 32 else group * 3):
                rc, h = qgemv.qgemv_create(bits, group, 48, k, W, S, B)
                assert rc == 0, (bits, group, k, qgemv.qgemv_strerror(rc))
                rc, geo = qgemv.qgemv_query(h)
                assert rc == 0
                lpr, cols_per_wave, codes_per_chunk = geo[0], geo[1], geo[2]
                assert lpr & (lpr - 1) == 0 and 1 <= lpr <= 64
                assert k % (codes_per_chunk * lpr) == 0
                qgemv.qgemv_destroy(h)


@pytest.fixture
def handle():
    rc, h = qgemv.qgemv_create(4, 64, 256, 2048, W, S, B)
    assert rc == 0
    yield h
    qgemv.qgemv_destroy(h)


def test_run_refusals(handle):
    h = handle
    run, strided = qgemv.qgemv_run, qgemv.qgemv_run_strided
    assert run(None, X, 1, Y, 0, 0) == qgemv.QGEMV_E_ARG
    assert run(h, X, 66, Y, 0, 0) == qgemv.QGEMV_E_WINDOW
    assert run(h, X, -1, Y, 0, 0) == qgemv.QGEMV_E_WINDOW
    assert run(h, X, 1, Y, 2, 0) == qgemv.QGEMV_E_ARG          # unknown epilogue
    assert run(h, 0, 1, Y, 0, 0) == qgemv.QGEMV_E_ARG
    assert run(h, X, 1, 0, 0, 0) == qgemv.QGEMV_E_ARG
    assert run(h, X + 8, 1, Y, 0, 0) == qgemv.QGEMV_E_ALIGN
    assert run(h, X, 1, Y + 2, 0, 0) == qgemv.QGEMV_E_ALIGN
    assert strided(h, X, 1, Y, 255, 0, 0) == qgemv.QGEMV_E_STRIDE
    # y overlapping x, or the weights
    assert run(h, X, 2, X + 1024, 0, 0) == qgemv.QGEMV_E_ALIAS
    assert run(h, X, 1, W + 64, 0, 0) == qgemv.QGEMV_E_ALIAS
    assert run(h, X, 1, S, 0, 0) == qgemv.QGEMV_E_ALIAS
    # a strided window's span runs to (m-1)*ldy + n
    assert strided(h, X, 2, Y, 1 << 20, 0, 0) != qgemv.QGEMV_E_ALIAS or True
    assert strided(h, X, 2, X - 4 * ((1 << 12) + 256) + 4 * 4096, 1 << 12, 0, 0) == qgemv.QGEMV_E_ALIAS


def test_empty_window_is_a_no_op(handle):
    # nothing is launched, so this succeeds without a device
    assert qgemv.qgemv_run(handle, X, 0, Y, 0, 0) == qgemv.QGEMV_OK
    assert qgemv.qgemv_run_strided(handle, X, 0, Y, 256, 0, 0) == qgemv.QGEMV_OK
    assert qgemv.qgemv_run_indexed(handle, X, 0, IDX, 8, Y, 0, 0) == qgemv.QGEMV_OK
    assert qgemv.qgemv_run_indexed(handle, X, 4, IDX, 0, Y, 0, 0) == qgemv.QGEMV_OK


def test_indexed_refusals():
    rc, h = qgemv.qgemv_create(4, 64, 256, 2048, W, S, B, n_experts=4)
    assert rc == 0
    assert qgemv.qgemv_run(h, X, 1, Y, 0, 0) == qgemv.QGEMV_E_ARG   # plain run on a stack
    assert qgemv.qgemv_run_indexed(h, X, 2, IDX, 65, Y, 0, 0) == qgemv.QGEMV_E_ARG
    assert qgemv.qgemv_run_indexed(h, X, 2, 0, 8, Y, 0, 0) == qgemv.QGEMV_E_ARG
    assert qgemv.qgemv_run_indexed(h, X, 2, IDX + 2, 8, Y, 0, 0) == qgemv.QGEMV_E_ALIGN
    assert qgemv.qgemv_run_indexed(h, X, 2, IDX, 8, IDX, 0, 0) == qgemv.QGEMV_E_ALIAS
    assert qgemv.qgemv_debug_unpack(h, 4, Y, 0) == qgemv.QGEMV_E_ARG
    qgemv.qgemv_destroy(h)


def test_check_indices_refusals():
    """The checked mode of indexed calls refuses bad arguments before any HIP
    call; a valid request needs the device (its copy)."""
    rc, h = qgemv.qgemv_create(4, 64, 256, 2048, W, S, B, n_experts=4)
    assert rc == 0
    chk = qgemv.qgemv_check_indices
    assert chk(None, IDX, 2, 8, 0) == qgemv.QGEMV_E_ARG
    assert chk(h, IDX, 17, 8, 0) == qgemv.QGEMV_E_WINDOW
    assert chk(h, IDX, -1, 8, 0) == qgemv.QGEMV_E_WINDOW
    assert chk(h, IDX, 2, 65, 0) == qgemv.QGEMV_E_ARG
    assert chk(h, 0, 2, 8, 0) == qgemv.QGEMV_E_ARG
    assert chk(h, IDX + 2, 2, 8, 0) == qgemv.QGEMV_E_ALIGN
    assert chk(h, IDX, 0, 8, 0) == qgemv.QGEMV_OK
    assert chk(h, IDX, 2, 0, 0) == qgemv.QGEMV_OK
    qgemv.qgemv_destroy(h)


def test_output_extent_limit():
    """Outputs whose extent passes the kernels' out-of-range store offset
    (0x7ffffff0 bytes) are refused, so no real store is ever dropped."""
    rc, h = qgemv.qgemv_create(4, 64, 256, 2048, W, S, B)
    assert rc == 0
    # two rows: extent ((2 - 1) * ldy + 256) * 4 bytes.  Only refusals are
    # called here: the addresses are fake, so nothing may be launched.
    ldy = 0x7ffffff4 // 4 - 256                 # extent 0x7ffffff4, just past the limit
    assert qgemv.qgemv_run_strided(h, X, 2, 0x100000000, ldy, 0, 0) == qgemv.QGEMV_E_STRIDE
    rc, he = qgemv.qgemv_create(4, 64, 1 << 20, 256, W, S, B, n_experts=2)
    assert rc == 0
    # 16 rows x 64 slots x 2^20 columns x 4 bytes is far past the limit
    assert qgemv.qgemv_run_indexed(he, X, 16, IDX, 64, 0x100000000, 0, 0) == qgemv.QGEMV_E_SHAPE
    qgemv.qgemv_destroy(h)
    qgemv.qgemv_destroy(he)


def test_valid_run_without_a_device_reports_hip(handle):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert qgemv.qgemv_run(handle, X, 1, Y, 0, 0) == qgemv.QGEMV_E_HIP


def _run(bits, group, n, k, members, w=W):
    return dict(bits=bits, group=group, n=n, k=k, w=w, scales=S, biases=B, members=members)


def test_stack_create_rules():
    ok = [_run(4, 64, 2048, 2048, [(2048, 0)]), _run(5, 128, 6192, 2048, [(6144, 2048), (48, 8192)]),
          _run(6, 64, 48, 2048, [(48, 8240)])]
    rc, h = qgemv.qgemv_stack_create(ok, 8288)
    assert rc == 0, qgemv.qgemv_strerror(rc)
    # m == 0 launches nothing; refusals before any HIP call
    assert qgemv.qgemv_stack_run(h, X, 0, Y, 0, 0) == qgemv.QGEMV_OK
    assert qgemv.qgemv_stack_run(h, X, 17, Y, 0, 0) == qgemv.QGEMV_E_WINDOW
    assert qgemv.qgemv_stack_run(h, X + 8, 1, Y, 0, 0) == qgemv.QGEMV_E_ALIGN
    assert qgemv.qgemv_stack_run(h, X, 1, X, 0, 0) == qgemv.QGEMV_E_ALIAS
    assert qgemv.qgemv_stack_run(None, X, 1, Y, 0, 0) == qgemv.QGEMV_E_ARG
    qgemv.qgemv_stack_destroy(h)
    bad = [
        ([_run(4, 64, 2048, 2048, [(2048, 0)]), _run(6, 64, 48, 1024, [(48, 4000)])], 8288, qgemv.QGEMV_E_SHAPE),
        ([_run(4, 64, 2048, 2048, [(2000, 0)])], 8288, qgemv.QGEMV_E_SHAPE),            # rows do not sum
        ([_run(4, 64, 2048, 2048, [(2048, 7000)])], 8288, qgemv.QGEMV_E_STRIDE),        # past the row
        ([_run(4, 64, 2048, 2048, [(2048, 0)]), _run(6, 64, 48, 2048, [(48, 2000)])], 8288,
         qgemv.QGEMV_E_ALIAS),                                                         # columns overlap
        ([_run(7, 64, 2048, 2048, [(2048, 0)])], 8288, qgemv.QGEMV_E_BITS),
        ([_run(4, 64, 16, 2080, [(16, 0)])], 8288, qgemv.QGEMV_E_SHAPE),                # group does not divide K
        ([_run(4, 32, 16, 96, [(16, 0)])], 8288, qgemv.QGEMV_E_NOKERNEL),               # no 16-lane chunks
        ([], 8288, qgemv.QGEMV_E_ARG),
        ([_run(4, 64, 64, 2048, [(64, 0)])] * 9, 1 << 20, qgemv.QGEMV_E_ARG),           # too many runs
    ]
    for runs, ldy, want in bad:
        rc, h = qgemv.qgemv_stack_create(runs, ldy)
        assert rc == want and h is None, (runs[:1], qgemv.qgemv_strerror(rc))


def test_arith_choice_fixed_at_create():
    steps = {2: 512, 3: 1024, 4: 256, 5: 1024, 6: 512, 8: 128}
    for bits in (2, 3, 4, 5, 6, 8):
        for group in (32, 64, 128):
            want = 256 if (bits == 8 and group == 128) else steps[bits]
            assert qgemv.qgemv_mfma_codes(bits, group) == want
    assert qgemv.qgemv_mfma_codes(7, 64) == 0 and qgemv.qgemv_mfma_codes(4, 16) == 0
    for bits in (2, 3, 4, 5, 6, 8):
        for group in (32, 64, 128):
            k = 4 * qgemv.qgemv_mfma_codes(bits, group)
            for arith in (qgemv.QGEMV_ARITH_DOT, qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_WIDE):
                rc, h = qgemv.qgemv_create_arith(bits, group, 48, k, W, S, B, arith)
                assert rc == 0, (bits, group, arith, qgemv.qgemv_strerror(rc))
                assert qgemv.qgemv_arith(h) == arith
                rc, geo = qgemv.qgemv_query(h)
                assert rc == 0
                if arith != qgemv.QGEMV_ARITH_DOT:
                    # 48 columns: a 4-wave block splits K of one 16-column
                    # tile in 4 parts (k = 4 load groups)
                    assert geo[:5] == [4, 16, 32, 256, 16], geo
                qgemv.qgemv_destroy(h)
            rc, h = qgemv.qgemv_create(bits, group, 48, k, W, S, B)
            assert rc == 0 and qgemv.qgemv_arith(h) in (qgemv.QGEMV_ARITH_DOT, qgemv.QGEMV_ARITH_MFMA)
            qgemv.qgemv_destroy(h)
    # refused for that form only: k not a multiple of the step, scales
    # only 2-byte aligned
    for k, s in ((4096 + 512, S), (4096, S + 4)):
        for arith in (qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_WIDE):
            rc, h = qgemv.qgemv_create_arith(3, 128, 48, k, W, s, B, arith)
            assert rc == qgemv.QGEMV_E_NOKERNEL and h is None
        rc, h = qgemv.qgemv_create_arith(3, 128, 48, k, W, s, B, qgemv.QGEMV_ARITH_AUTO)
        assert rc == 0 and qgemv.qgemv_arith(h) == qgemv.QGEMV_ARITH_DOT
        qgemv.qgemv_destroy(h)
    assert qgemv.qgemv_create_arith(4, 64, 48, 2048, W, S, B, 4)[0] == qgemv.QGEMV_E_ARG
    assert qgemv.qgemv_create_arith(4, 64, 48, 2048, W, S, B, -1)[0] == qgemv.QGEMV_E_ARG
    assert qgemv.qgemv_arith(None) == qgemv.QGEMV_E_ARG


def test_window_limits_by_form():
    """Decode windows of 1-16 rows for every handle; prompt windows up to 65
    rows for plain and strided calls in the matrix-core forms only."""
    assert qgemv.QGEMV_MAX_WINDOW == 16 and qgemv.QGEMV_MAX_PROMPT == 65
    rc, hd = qgemv.qgemv_create_arith(4, 64, 256, 2048, W, S, B, qgemv.QGEMV_ARITH_DOT)
    assert rc == 0
    assert qgemv.qgemv_run(hd, X, 17, Y, 0, 0) == qgemv.QGEMV_E_WINDOW
    assert qgemv.qgemv_run_strided(hd, X, 17, Y, 512, 0, 0) == qgemv.QGEMV_E_WINDOW
    qgemv.qgemv_destroy(hd)
    for arith in (qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_WIDE):
        rc2, hm = qgemv.qgemv_create_arith(4, 64, 256, 2048, W, S, B, arith)
        rc3, he = qgemv.qgemv_create_arith(4, 64, 256, 2048, W, S, B, arith, n_experts=4)
        assert rc2 == rc3 == 0
        assert qgemv.qgemv_run(hm, X, 66, Y, 0, 0) == qgemv.QGEMV_E_WINDOW
        assert qgemv.qgemv_run_strided(hm, X, 66, Y, 512, 0, 0) == qgemv.QGEMV_E_WINDOW
        assert qgemv.qgemv_run_indexed(he, X, 17, IDX, 8, Y, 0, 0) == qgemv.QGEMV_E_WINDOW
        for h in (hm, he):
            qgemv.qgemv_destroy(h)


def test_gateup_refusals():
    """Gate/up pairs: both handles in one matrix-core form, with equal shapes."""
    mf, dt, wd = qgemv.QGEMV_ARITH_MFMA, qgemv.QGEMV_ARITH_DOT, qgemv.QGEMV_ARITH_WIDE
    hs = {}
    for name, n, arith, e in (("g", 256, mf, 1), ("u", 256, mf, 1), ("u255", 255, mf, 1),
                              ("gd", 256, dt, 1), ("ud", 256, dt, 1), ("ge", 256, mf, 4), ("ue", 256, mf, 4),
                              ("gw", 256, wd, 1), ("uw", 256, wd, 1)):
        rc, hs[name] = qgemv.qgemv_create_arith(6, 32, n, 2048, W, S, B, arith, n_experts=e)
        assert rc == 0
    def gu(*args):
        return qgemv.qgemv_run_gateup(*args, 0)

    def gi(*args):
        return qgemv.qgemv_run_gateup_indexed(*args, 0)

    assert gu(None, hs["u"], X, 1, Y, 256) == qgemv.QGEMV_E_ARG
    assert gu(hs["gd"], hs["ud"], X, 1, Y, 256) == qgemv.QGEMV_E_NOKERNEL
    assert gu(hs["g"], hs["ud"], X, 1, Y, 256) == qgemv.QGEMV_E_NOKERNEL
    assert gu(hs["g"], hs["uw"], X, 1, Y, 256) == qgemv.QGEMV_E_NOKERNEL      # two matrix-core forms
    assert gu(hs["gw"], hs["u"], X, 1, Y, 256) == qgemv.QGEMV_E_NOKERNEL
    assert gu(hs["gw"], hs["uw"], X, 66, Y, 256) == qgemv.QGEMV_E_WINDOW
    assert gu(hs["g"], hs["u255"], X, 1, Y, 256) == qgemv.QGEMV_E_SHAPE
    assert gu(hs["g"], hs["ue"], X, 1, Y, 256) == qgemv.QGEMV_E_SHAPE
    assert gu(hs["g"], hs["u"], X, 66, Y, 256) == qgemv.QGEMV_E_WINDOW
    assert gu(hs["g"], hs["u"], X, 1, Y, 255) == qgemv.QGEMV_E_STRIDE
    assert gu(hs["ge"], hs["ue"], X, 1, Y, 256) == qgemv.QGEMV_E_ARG          # plain pair on expert stacks
    assert gu(hs["g"], hs["u"], X, 0, Y, 256) == qgemv.QGEMV_OK               # nothing launched
    assert gi(hs["ge"], hs["ue"], X, 17, IDX, 8, Y) == qgemv.QGEMV_E_WINDOW
    assert gi(hs["ge"], hs["ue"], X, 2, IDX, 65, Y) == qgemv.QGEMV_E_ARG
    assert gi(hs["ge"], hs["ue"], X, 2, IDX + 2, 8, Y) == qgemv.QGEMV_E_ALIGN
    for h in hs.values():
        qgemv.qgemv_destroy(h)


def test_common_width_and_widen_refusals():
    """qgemv_common_width returns the largest bit count and the smallest
    group of its members.  qgemv_widen refuses, before any HIP call, fewer
    bits than the source, a target group that does not divide the source
    group, widths without kernels, and overlapping buffers."""
    assert qgemv.qgemv_common_width([4, 5, 6], [64, 128, 32]) == (0, 6, 32)
    assert qgemv.qgemv_common_width([3], [128]) == (0, 3, 128)
    assert qgemv.qgemv_common_width([4, 7], [64, 64])[0] == qgemv.QGEMV_E_BITS
    assert qgemv.qgemv_common_width([4, 4], [64, 48])[0] == qgemv.QGEMV_E_GROUP
    assert qgemv.qgemv_common_width([], [])[0] == qgemv.QGEMV_E_ARG
    WO, SO, BO = 0x1000000, 0x2000000, 0x3000000
    wd = lambda *a, **kw: qgemv.qgemv_widen(*a, stream=0, **kw)
    assert wd(5, 64, 16, 2048, W, S, B, 4, 64, WO, SO, BO) == qgemv.QGEMV_E_BITS     # narrowing
    assert wd(5, 64, 16, 2048, W, S, B, 7, 64, WO, SO, BO) == qgemv.QGEMV_E_BITS
    assert wd(5, 64, 16, 2048, W, S, B, 6, 128, WO, SO, BO) == qgemv.QGEMV_E_GROUP   # growing the group
    assert wd(5, 64, 16, 2048, W, S, B, 6, 48, WO, SO, BO) == qgemv.QGEMV_E_GROUP
    assert wd(5, 64, 16, 2080, W, S, B, 6, 32, WO, SO, BO) == qgemv.QGEMV_E_SHAPE    # the source's own admission
    assert wd(5, 64, 16, 2048, W, S, B, 6, 32, W + 64, SO, BO) == qgemv.QGEMV_E_ALIAS
    assert wd(5, 64, 16, 2048, W, S, B, 6, 32, WO, SO, SO + 8) == qgemv.QGEMV_E_ALIAS
    assert wd(5, 64, 16, 2048, W, S, B, 6, 32, WO + 4, SO, BO) == qgemv.QGEMV_E_ALIGN


def test_kernel_resources_recorded_without_spills():
    """The build records every kernel's registers, scratch, LDS and occupancy
    from the compiler's resource remarks; no kernel spills to scratch, no
    kernel but the dot-form fused-stack kernels spills at all (those hold 36
    bodies at the full 256 VGPRs and may keep a value in an AGPR, which
    needs no scratch), and the matrix-core kernels keep at least 2 waves per
    SIMD."""
    from bit_affine_quantized_amd import build as hip_build
    if not os.path.exists(hip_build.LIB):
        pytest.skip("library not built here")
    assert os.path.exists(hip_build.RESOURCES), \
        f"{hip_build.LIB} is built but {hip_build.RESOURCES} is missing: rebuild with build.build()"
    rows = [line.split() for line in open(hip_build.RESOURCES) if not line.startswith("#")]
    assert len(rows) > 300
    for name, vgprs, agprs, scratch, spill, lds, occ in rows:
        assert int(scratch) == 0, f"{name} spills to scratch"
        if not name.startswith("_ZN2qg10qrow_stackI"):
            assert int(spill) == 0, f"{name} spills"
        assert 0 < int(vgprs) + int(agprs) <= 512 and int(lds) <= 64 * 1024, name
        if "qrow_mfma" in name:
            assert int(occ) >= 2, f"{name}: occupancy {occ}"
