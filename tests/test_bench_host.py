"""Host checks of bench.py's measurement plumbing (no GPU): the one-GPU
refusal, the algorithmic bytes of the workloads against their stated sizes,
and the rule that a counter summary applies only to the machine code it was
taken on."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run_bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run_bench(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_matrix_workload_shape():
    assert bench.parse_shape("5,64,131072,2048") == (5, 64, 131072, 2048)
    for bad in (None, "5,64,131072", "7,64,1024,2048", "4,48,1024,2048", "4,64,0,2048", "4,64,1024,96"):
        with pytest.raises(ValueError):
            bench.parse_shape(bad)
    # refused before any GPU work, with the reason on stderr
    r = _run_bench("--workload", "matrix", "--shape", "4,48,1024,2048")
    assert r.returncode == 2 and "4/48" in r.stderr
    r = _run_bench("--workload", "matrix")
    assert r.returncode == 2 and "--shape" in r.stderr
    r = _run_bench("--shape", "4,64,1024,2048")
    assert r.returncode == 2 and "--workload matrix" in r.stderr


def test_algorithmic_bytes_match_the_stated_sizes():
    # the 1-row LM head: 381,419,520 B of codes, 63,569,920 B of bf16 scales
    # and biases, 4,096 B of activations, 993,280 B of fp32 outputs
    assert bench.algorithmic_bytes([(6, 32, 248320)], 1, 2048, 248320) == 445986816
    assert bench.algorithmic_bytes([(6, 32, 248320)], 0, 2048, 0) == 381419520 + 63569920
    # per output column at K = 2048: 1,792 B (6/32), 1,152 B (4/64), 1,344 B (5/128)
    for bits, group, per_col in ((6, 32, 1792), (4, 64, 1152), (5, 128, 1344)):
        assert bench.algorithmic_bytes([(bits, group, 1)], 0, 2048, 0) == per_col
    # the fused stack at 1 row moves about 10.8 MB: three runs, one 8288-column row
    stack = bench.algorithmic_bytes([(4, 64, 2048), (5, 128, 6192), (6, 64, 48)], 1, 2048, 8288)
    assert stack == 2048 * 1152 + 6192 * 1344 + 48 * 1536 + 48 * 128 + 4096 + 8288 * 4
    assert 10.7e6 < stack < 10.9e6
    # an indexed call adds its routing table
    assert bench.algorithmic_bytes([(4, 64, 1024)], 16, 2048, 8 * 1024, 16 * 8 * 4) == \
        1024 * 1152 + 16 * 2048 * 2 + 16 * 8 * 1024 * 4 + 512


def test_traffic_applies_only_to_its_machine_code(tmp_path, monkeypatch):
    if not os.path.exists(bench.LIB_DEFAULT):
        pytest.skip("library not built here")
    monkeypatch.delenv("QGEMV_LIB", raising=False)
    sha = bench.kernel_hash()
    assert len(sha) == 16 and int(sha, 16) >= 0
    # the hash covers the kernels' machine code, in the library's .hip_fatbin section
    with open(bench.LIB_DEFAULT, "rb") as f:
        assert bench._elf_section(f.read(), ".hip_fatbin") is not None
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.read_traffic("lmhead_m1") is None
    (tmp_path / "counters_lmhead_m1.txt").write_text(
        f"# test\nkernel_sha: {sha}\nhbm_bytes_per_launch: 447000000\n")
    assert bench.read_traffic("lmhead_m1") == 447000000
    other = "0" * 16 if sha != "0" * 16 else "1" * 16
    (tmp_path / "counters_lmhead_m1.txt").write_text(
        f"kernel_sha: {other}\nhbm_bytes_per_launch: 447000000\n")
    assert bench.read_traffic("lmhead_m1") is None


def _patched(tmp_path, name, section, data, fb_off, obj_index, needle=None):
    """A copy of the library with one byte changed inside one section of one
    GPU code object (at `needle` if given, else in the section's middle)."""
    objs = bench.code_objects(data[fb_off[0]:fb_off[0] + fb_off[1]])
    obj = objs[obj_index]
    obj_at = data.index(obj, fb_off[0])
    off, size = bench._elf_section_range(obj, section)
    at = obj.index(needle, off) if needle else off + size // 2
    assert off <= at < off + size
    out = bytearray(data)
    out[obj_at + at] ^= 0x01
    path = tmp_path / name
    path.write_bytes(bytes(out))
    return str(path)


def test_kernel_hash_ignores_path_derived_names(tmp_path):
    """The hash covers each GPU code object's .text only: changing a byte of a
    compiler-made, path-derived symbol name (a code object's .strtab, where
    the __hip_cuid_ names live) keeps it, changing a byte of machine code
    does not."""
    if not os.path.exists(bench.LIB_DEFAULT):
        pytest.skip("library not built here")
    with open(bench.LIB_DEFAULT, "rb") as f:
        data = f.read()
    fb = bench._elf_section_range(data, ".hip_fatbin")
    objs = bench.code_objects(data[fb[0]:fb[0] + fb[1]])
    assert len(objs) >= 17                         # one per translation unit
    base = bench.kernel_hash(bench.LIB_DEFAULT)
    i = next(j for j, o in enumerate(objs) if b"__hip_cuid_" in o)
    name_changed = _patched(tmp_path, "names.so", ".strtab", data, fb, i, needle=b"__hip_cuid_")
    assert bench.kernel_hash(name_changed) == base
    code_changed = _patched(tmp_path, "code.so", ".text", data, fb, i)
    assert bench.kernel_hash(code_changed) != base
