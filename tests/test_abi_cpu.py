"""The C ABI library without a GPU: it loads, exports every declared symbol,
rejects bad arguments on the host before touching the device, and its
launch grids and indexes stay inside their buffers (host-side replay)."""

import ctypes
import os
import re
import subprocess

import pytest

import newton_schulz_07_amd as ns

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ns_hip.h")
FAKE_IN = 0x10000000
FAKE_OUT = 0x20000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ns_[a-z_]+)\s*\(", text)))


def test_header_declares_what_the_binding_wraps():
    assert declared_functions() == sorted(ns.SIGNATURES)


def test_library_loads_and_exports_every_declared_symbol():
    lib = ns.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def call(batch=1, rows=256, cols=512, dtype=1, steps=5, inp=FAKE_IN, out=FAKE_OUT):
    return ns.lib().ns_orthogonalize(ctypes.c_void_p(inp), ctypes.c_void_p(out), batch, rows, cols, dtype,
                                     steps, 3.4445, -4.775, 2.0315, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(inp=0), 1),                      # NULL in
    (dict(out=0), 1),                      # NULL out
    (dict(rows=0), 1),
    (dict(cols=-8), 1),
    (dict(batch=-1), 1),
    (dict(steps=-1), 1),
    (dict(rows=65536, cols=65536), 1),     # slice of 2^32 elements
    (dict(rows=16384, cols=32768), 1),     # 2^29 elements: over the 2 GiB fp32 slice limit
    (dict(dtype=2), 2),
    (dict(dtype=-1), 2),
    (dict(inp=FAKE_IN + 8), 3),            # not 16-byte aligned
    (dict(out=FAKE_IN + 256 * 512), 1),    # partial overlap with in
])
def test_argument_errors_are_reported_before_any_launch(kwargs, status):
    st = call(**kwargs)
    assert st == status
    assert ns.lib().ns_last_error().decode() != ""
    assert ns.lib().ns_status_string(st).decode().startswith("NS_ERR")


@pytest.mark.parametrize("rows,cols", [(260, 512), (256, 100), (1, 1), (9, 13)])
def test_dims_not_multiple_of_8_pass_the_argument_checks(rows, cols):
    # ns_orthogonalize pads such shapes (stage exports still refuse them);
    # without a GPU the call gets as far as the device query
    st = call(rows=rows, cols=cols)
    assert st not in (1, 2, 3), ns.lib().ns_last_error().decode()
    pr, pc = -(-rows // 8) * 8, -(-cols // 8) * 8
    assert ns.ns_workspace_bytes(2, rows, cols, 1) >= ns.ns_workspace_bytes(2, pr, pc, 1) + 2 * 2 * pr * pc * 2


def test_empty_batch_is_a_no_op():
    assert call(batch=0) == 0
    assert call(batch=0, inp=FAKE_IN, out=FAKE_IN) == 0


def test_stage_argument_errors():
    L = ns.lib()
    vp = ctypes.c_void_p
    big = FAKE_OUT + (1 << 24)
    assert L.ns_stage_gram(vp(FAKE_IN), vp(0), vp(FAKE_OUT), 1, 64, 64, 1, None) == 1
    assert L.ns_stage_poly(vp(FAKE_IN), vp(FAKE_OUT), vp(FAKE_IN), vp(FAKE_OUT), 1, 64, 1, 1.0, 0.0, 0.0, None) == 1
    assert L.ns_stage_update(vp(FAKE_IN), vp(FAKE_OUT), vp(big), vp(FAKE_IN), 1, 64, 64, 1, None) == 1  # overlap
    assert L.ns_stage_update(vp(FAKE_IN), vp(FAKE_OUT), None, vp(big), 1, 64, 64, 1, None) == 1  # NULL c_diag
    assert L.ns_stage_normalize(vp(FAKE_IN), vp(FAKE_OUT), None, 1, 63, 64, 1, None) == 3
    assert L.ns_stage_normalize(vp(FAKE_IN), vp(FAKE_OUT), None, 0, 64, 64, 1, None) == 0


def test_workspace_bytes():
    L = ns.lib()
    # temporary X + two m x m matrices + two fp32 diagonals + norm partials
    b, r, c = 128, 1536, 2048
    ws = L.ns_workspace_bytes(b, r, c, 1)
    assert ws >= b * r * c * 2 + 2 * b * r * r * 2 + 2 * b * r * 4
    assert ws < 1.01 * (b * r * c * 2 + 2 * b * r * r * 2) + (1 << 20)
    assert L.ns_workspace_bytes(1, 14336, 4096, 1) == L.ns_workspace_bytes(1, 4096, 14336, 1)
    assert L.ns_workspace_bytes(1, 10, 16, 1) > L.ns_workspace_bytes(1, 16, 16, 1)  # padded copies
    assert L.ns_workspace_bytes(1, 0, 16, 1) == 0  # invalid shape
    assert L.ns_workspace_bytes(1, 16, 16, 7) == 0  # invalid dtype


def test_timing_query_rejects_bad_kind():
    L = ns.lib()
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert L.ns_timing_query(99, ctypes.byref(ms), ctypes.byref(n)) == 1
    assert L.ns_timing_reset() == 0
    assert L.ns_timing_query(2, ctypes.byref(ms), ctypes.byref(n)) == 0 and n.value == 0
    for every, offset in ((0, 0), (5, 5), (5, -1), (-1, 0)):
        assert L.ns_timing_sample(every, offset) == 1, (every, offset)
    assert L.ns_timing_sample(5, 2) == 0
    assert L.ns_timing_sample(1, 0) == 0


def test_peak_calibration_argument_errors():
    # every check runs before the device is touched
    L = ns.lib()
    tf, mhz = ctypes.c_double(), ctypes.c_double()
    assert L.ns_peak_mfma(7, 1024, ctypes.byref(tf), ctypes.byref(mhz), None) == 2  # NS_ERR_DTYPE
    assert L.ns_peak_mfma(1, 1024, None, ctypes.byref(mhz), None) == 1
    assert L.ns_peak_mfma(1, 1024, ctypes.byref(tf), None, None) == 1
    for iters in (0, 3, 1026, (1 << 30) + 4):
        assert L.ns_peak_mfma(1, iters, ctypes.byref(tf), ctypes.byref(mhz), None) == 1, iters
        assert "iters" in L.ns_last_error().decode()


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        ns.orthogonalize(torch.zeros(8, 8))


@pytest.fixture(scope="module")
def boundscheck():
    import __graft_entry__
    return __graft_entry__.build_boundscheck()


@pytest.mark.parametrize("case", [
    "1 1 256 512 5", "0 1 256 512 5",        # the small workload, both dtypes
    "1 3 264 520 5", "0 3 264 520 3",        # ragged tails, batch, wide
    "1 2 520 264 4", "0 2 520 264 1",        # tall
    "1 1 8 8 1", "1 1 8 2048 5", "1 4 2048 8 2", "1 1 136 136 5",
    "1 1 40 24 0",                           # zero steps
    "1 16 384 512 5", "1 2 1040 336 5",      # batched, tall, several tiles
    # stacks whose Gram stores only its lower block triangle (256 and 128
    # Gram tiles): every read of A must hit an element the Gram wrote
    "1 400 264 520 2", "1 200 520 264 2",
    # rows or cols not a multiple of 8: zero-padded copies in and out
    "1 3 100 37 3", "0 2 33 17 2", "1 1 1 1 2", "1 2 9 2051 1", "0 1 5 3 0",
])
def test_launch_indexes_stay_in_bounds(boundscheck, case):
    r = subprocess.run([boundscheck] + case.split(), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "violations=0" in r.stdout


# ------------------------------------------------- grouped calls (several stacks)

def gcall(shapes, ins=None, outs=None, dtype=1, steps=5, n=None):
    n = len(shapes) if n is None else n
    k = len(shapes)
    ins = ins if ins is not None else [FAKE_IN + (i << 28) for i in range(k)]
    outs = outs if outs is not None else [FAKE_OUT + (i << 32) for i in range(k)]
    arr = lambda t, v: (t * max(k, 1))(*v) if k else None
    b, r, c = ([s[j] for s in shapes] for j in range(3))
    return ns.lib().ns_orthogonalize_grouped(n, arr(ctypes.c_void_p, ins), arr(ctypes.c_void_p, outs),
                                             arr(ctypes.c_int64, b), arr(ctypes.c_int64, r),
                                             arr(ctypes.c_int64, c), dtype, steps, 3.4445, -4.775, 2.0315, None)


def test_grouped_empty_calls_are_no_ops():
    assert gcall([]) == 0
    assert gcall([(0, 64, 64), (0, 8, 8)], ins=[0, 0], outs=[0, 0]) == 0  # skipped stacks: NULL allowed


@pytest.mark.parametrize("kwargs,status,where", [
    (dict(shapes=[(1, 64, 64)], n=-1), 1, "n_groups"),
    (dict(shapes=[(1, 64, 64)], n=4097), 1, "n_groups"),
    (dict(shapes=[(1, 64, 64), (1, 0, 64)]), 1, "stack 1"),
    (dict(shapes=[(1, 64, 64), (70000, 8, 8)]), 1, "stack 1"),
    (dict(shapes=[(1, 64, 64)], dtype=5), 2, "dtype"),
    (dict(shapes=[(1, 64, 64), (1, 64, 64)], ins=[FAKE_IN, FAKE_IN + 8]), 3, "stack 1"),
    (dict(shapes=[(1, 64, 64)], ins=[0]), 1, "stack 0"),
    (dict(shapes=[(1, 64, 64)], outs=[FAKE_IN + 64]), 1, "stack 0"),          # partial overlap in/out
    (dict(shapes=[(1, 64, 64), (1, 64, 64)], outs=[FAKE_OUT, FAKE_IN + (1 << 28)]), 1, "overlaps"),  # out0 = in1
    (dict(shapes=[(1, 64, 64), (1, 64, 64)], outs=[FAKE_OUT, FAKE_OUT + 4096]), 1, "overlaps"),      # out0 ~ out1
    (dict(shapes=[(1, 64, 64)], steps=-1), 1, "ns_steps"),
])
def test_grouped_argument_errors(kwargs, status, where):
    st = gcall(**kwargs)
    assert st == status
    assert where in ns.lib().ns_last_error().decode()


def test_grouped_in_place_and_odd_shapes_pass_the_checks():
    st = gcall([(2, 264, 520), (3, 100, 37)], outs=[FAKE_IN, FAKE_IN + (1 << 28)])
    assert st not in (1, 2, 3), ns.lib().ns_last_error().decode()


def test_grouped_workspace_is_the_sum_of_the_stacks():
    shapes = [(2, 264, 520), (3, 520, 264), (1, 100, 37), (0, 64, 64), (16, 1536, 2048)]
    single = [ns.ns_workspace_bytes(b, r, c, 1) if b else 0 for b, r, c in shapes]
    assert ns.ns_workspace_bytes_grouped(shapes, 1) == sum(-(-s // 256) * 256 for s in single)
    assert ns.ns_workspace_bytes_grouped([(1, 0, 8)], 1) == 0
    assert ns.ns_workspace_bytes_grouped(shapes, 3) == 0


@pytest.mark.parametrize("case", [
    "1 3 2 264 520 3 520 264 1 100 37",          # wide, tall and padded stacks together
    "0 2 2 264 520 3 520 264 1 33 17",
    "1 2 200 264 520 200 520 264",               # lower-triangle A, 128 Gram tiles in both orientations
    "1 2 400 264 520 200 520 264",               # 256 Gram tiles (wide) beside 128 (tall)
    "1 2 6 264 520 200 520 264",                 # a 192-tile wide Gram beside 128 tall tiles
    "1 1 " + " ".join(f"{1 + i % 3} {8 + 8 * i} {16 + 8 * ((i * 7) % 13)}" for i in range(20)),  # 20 stacks
    "1 0 2 64 64 1 9 13",                        # ns_steps = 0
])
def test_grouped_launch_indexes_stay_in_bounds(boundscheck, case):
    r = subprocess.run([boundscheck, "--group"] + case.split(), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "violations=0" in r.stdout


def test_noalloc_rejects_bad_arguments_and_oversized_calls_before_any_launch():
    L = ns.lib()

    def noalloc(batch=1, rows=256, cols=512, dtype=1, steps=5, inp=FAKE_IN, out=FAKE_OUT):
        return L.ns_orthogonalize_noalloc(ctypes.c_void_p(inp), ctypes.c_void_p(out), batch, rows, cols, dtype,
                                          steps, 3.4445, -4.775, 2.0315, None)
    assert noalloc(inp=0) == 1
    assert noalloc(steps=-1) == 1
    assert noalloc(dtype=3) == 2
    assert noalloc(out=FAKE_OUT + 4) == 3
    assert noalloc(batch=0) == 0  # nothing to do, nothing touched
    # the fixed scratch is 256 MiB: 8192^2 bf16 needs 384 MiB, 128 x 1536 x 2048 about 1.9 GiB
    for shape in ((1, 8192, 8192), (128, 1536, 2048)):
        assert ns.ns_workspace_bytes(*shape, 1) > ns.NS_NOALLOC_SCRATCH_BYTES
        assert noalloc(*shape, out=FAKE_IN + 0x100000000) == 7  # out past the end of in
        assert "fixed scratch" in L.ns_last_error().decode()
    assert L.ns_status_string(7).decode().startswith("NS_ERR_SCRATCH")
    assert ns.ns_workspace_bytes(1, 4096, 4096, 1) <= ns.NS_NOALLOC_SCRATCH_BYTES


def test_missing_library_fails_loudly(monkeypatch):
    # no fallback: without the built library every call raises
    monkeypatch.setattr(ns, "LIB_PATH", "/nonexistent/libns_hip.so")
    monkeypatch.setattr(ns, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        ns.lib()
    with pytest.raises(RuntimeError, match="not built"):
        ns.ns_workspace_bytes(1, 64, 64, 1)


@pytest.mark.parametrize("call", ["orthogonalize", "orthogonalize_grouped", "ns_orthogonalize_noalloc"])
def test_host_tensors_are_refused(call):
    # the path runs on the GPU only: a host tensor is an error, never computed on the CPU
    import torch
    x = torch.randn(2, 16, 24)
    with pytest.raises(ValueError, match="GPU tensor"):
        if call == "orthogonalize":
            ns.orthogonalize(x)
        elif call == "orthogonalize_grouped":
            ns.orthogonalize_grouped([x])
        else:
            ns.ns_orthogonalize_noalloc(x, torch.empty_like(x))
