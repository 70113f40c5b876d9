"""Host-side checks of the C-ABI library (no GPU needed, no compute launched).

* the library loads and exports every function include/flce.h declares, and
  the benchmark's probe library every function include/flce_probe.h declares;
* the chunk policy reproduces every geometry the pages print;
* workspace sizing follows the slab formula and is flat in BT for an
  explicit chunk size;
* invalid arguments are rejected on the host before any launch.
"""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _header_functions(header="flce.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z0-9_]+)\s*\(", src)))


def test_header_and_exports_agree(flce_lib):
    declared = _header_functions()
    assert sorted(flce_lib.EXPORTS) == declared
    lib = flce_lib.load()
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_exported_symbols_in_dynamic_table(flce_lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", flce_lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in _header_functions():
        assert name in syms


def test_probe_library_exports_its_header(flce_lib):
    import ctypes
    import subprocess
    path = os.path.join(os.path.dirname(flce_lib.LIB_PATH), "libflce_probe.so")
    declared = _header_functions("flce_probe.h")
    assert declared == ["flce_probe_mfma16_loop", "flce_probe_mfma_loop", "flce_probe_mfma_threads",
                        "flce_probe_read_stream", "flce_probe_stream_threads"]
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert set(declared) <= syms
    lib = ctypes.CDLL(path)
    assert lib.flce_probe_mfma_threads() == 512
    assert lib.flce_probe_stream_threads() == 256
    # invalid arguments are refused before any launch
    for f in (lib.flce_probe_mfma_loop, lib.flce_probe_mfma16_loop):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.flce_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    far = 1 << 44
    for loop in (lib.flce_probe_mfma_loop, lib.flce_probe_mfma16_loop):
        assert loop(far, 16, far, 511, 1, 1, None) == 1   # sink too small
        assert loop(far, 8, far, 512, 1, 1, None) == 1    # no whole fragment
        assert loop(None, 16, far, 512, 1, 1, None) == 1
        assert loop(far, 16, far, 512, 1, -1, None) == 1  # negative iteration count
    assert lib.flce_probe_read_stream(far, 24, far, 4096, 1, None) == 1   # not a multiple of 16
    assert lib.flce_probe_read_stream(far, 32, far, 4095, 1, None) == 1   # sink too small


def test_status_and_kernel_names(flce_lib):
    assert flce_lib.flce_status_string(0) == "FLCE_OK"
    assert flce_lib.flce_status_string(-3).startswith("FLCE_E_TARGET")
    n = len(flce_lib.KERNEL_KINDS)
    assert [flce_lib.flce_kernel_name(k) for k in range(n)] == flce_lib.KERNEL_KINDS
    assert flce_lib.flce_kernel_name(n) == "unknown"


# ------------------------------------------------------------- chunk policy
def test_heuristic_geometry_matches_pages(flce_lib):
    geo = json.load(open(os.path.join(GOLDEN, "chunk_geometry.json")))
    for g in geo["heuristic"]:
        c = flce_lib.flce_chunk_size(g["BT"], g["H"], g["V"], 0, g["C"])
        assert c == g["chunk_size"], g
        assert -(-g["BT"] // c) == g["num_chunks"], g


def test_slab_bytes_match_pages(flce_lib):
    geo = json.load(open(os.path.join(GOLDEN, "chunk_geometry.json")))
    for g in geo["slab_bytes"]:
        c = flce_lib.flce_chunk_size(g["BT"], g["H"], g["V"], 0, g["C"])
        assert c * g["V"] * g["itemsize"] == g["bytes"]


def test_explicit_chunk_size_floor_and_clamp(flce_lib):
    geo = json.load(open(os.path.join(GOLDEN, "chunk_geometry.json")))
    for g in geo["explicit"]:
        assert flce_lib.flce_chunk_size(g["BT"], 4096, 128256, g["requested"], 1) == g["chunk_size"]
    assert flce_lib.flce_chunk_size(300, 128, 1000, 512, 1) == 300   # clamp to BT
    assert flce_lib.flce_chunk_size(300, 128, 1000, 1, 1) == 1
    assert flce_lib.flce_chunk_size(0, 128, 1000, 64, 1) == 1         # empty batch
    assert flce_lib.flce_chunk_size(300, 128, 1000, 0, 0) == -1        # C must be >= 1
    assert flce_lib.flce_chunk_size(300, 0, 1000, 64, 1) == -1
    assert flce_lib.flce_chunk_size(-1, 128, 1000, 64, 1) == -1


def test_skip_whole_chunks_geometry(flce_lib):
    """40 rows at chunk 16: 0/1/8/24/40 ignored -> 3/3/2/1/0 logits GEMMs (count = ceil(N/c))."""
    g = json.load(open(os.path.join(GOLDEN, "chunk_geometry.json")))["skip_whole_chunks"]
    c = flce_lib.flce_chunk_size(g["BT"], 64, 100, g["chunk_size"], 1)
    assert c == 16
    for ign, gemms in zip(g["ignored"], g["logits_gemms"]):
        assert -(-(g["BT"] - ign) // c) == gemms


def test_workspace_flat_in_bt_for_explicit_chunk(flce_lib):
    H, V = 5376, 262144
    a = flce_lib.flce_workspace_bytes(8192, H, V, flce_lib.BF16, 256, 1)
    b = flce_lib.flce_workspace_bytes(32768, H, V, flce_lib.BF16, 256, 1)
    slab = 256 * V * 2
    assert a >= slab and b >= slab
    # only the 8 bytes per row of index and per-row loss grow with BT
    assert b - a <= 8 * (32768 - 8192) + 4 * 256
    # the heuristic's slab grows with BT (chunk 256 -> 1024)
    h8 = flce_lib.flce_workspace_bytes(8192, H, V, flce_lib.BF16, 0, 1)
    h32 = flce_lib.flce_workspace_bytes(32768, H, V, flce_lib.BF16, 0, 1)
    assert h32 - h8 >= (1024 - 256) * V * 2


def test_workspace_invalid_arguments(flce_lib):
    assert flce_lib.flce_workspace_bytes(128, 64, 100, 7, 64, 1) == 0
    assert flce_lib.flce_workspace_bytes(128, 0, 100, 0, 64, 1) == 0


# ------------------------------------------------ rejected before any launch
# Fake, disjoint device addresses (never dereferenced: every call below fails
# on the host before anything is enqueued).
FAKE = dict(X=0x10000, W=0x20000, targets=0x30000, loss=0x40000, dX=0x50000, dW=0x60000,
            workspace=0x70000)


def _call(flce_lib, **kw):
    a = dict(X=FAKE["X"], W=FAKE["W"], targets=FAKE["targets"], BT=4, H=64, V=10,
             dtype=flce_lib.BF16, ignore_index=-100, reduction=0, chunk_size=0,
             chunk_mem_const=1, accum_dtype=flce_lib.BF16, frozen_weight=0, accumulate_dw=0,
             grad_output=None, loss=FAKE["loss"], dX=FAKE["dX"], dW=FAKE["dW"],
             workspace=FAKE["workspace"], workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return flce_lib.flce_fwd_bwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), -2),
    (dict(accum_dtype=1), -2),                 # bf16 operands, fp16 dW
    (dict(reduction=3), -1),
    (dict(H=60), -1),                          # H must be a multiple of 8
    (dict(H=0), -1),
    (dict(H=(1 << 20) + 8), -1),               # at most 2^20 hidden units
    (dict(V=0), -1),
    (dict(BT=-1), -1),
    (dict(loss=None), -1),
    (dict(loss=None, reduction=2), -1),        # none needs [BT] unless BT = 0
    (dict(dW=None), -1),                       # trained weight needs dW
    (dict(X=None), -1),
    (dict(X=FAKE["X"] + 2), -1),               # misaligned
    (dict(workspace=None), -1),
    (dict(workspace=FAKE["workspace"] + 16), -1),  # workspace must be 256-byte aligned
    (dict(workspace_bytes=1), -4),
    (dict(chunk_mem_const=0), -1),
    (dict(frozen_weight=2), -1),
])
def test_invalid_arguments_rejected_on_host(flce_lib, kw, status):
    assert _call(flce_lib, **kw) == status


@pytest.mark.parametrize("kw", [
    dict(dX=FAKE["X"] + 256),                  # grad_input over the inputs
    dict(dW=FAKE["W"]),                        # grad_weight onto the weight
    dict(loss=FAKE["workspace"] + 64),         # loss inside the workspace
    dict(loss=FAKE["targets"] + 16),           # loss over the targets
    dict(dX=FAKE["dW"] + 512),                 # two outputs overlapping
    dict(workspace=FAKE["dX"]),                # workspace over an output
    dict(grad_output=FAKE["loss"], reduction=2),  # per-token upstream gradient over the loss
])
def test_overlapping_buffers_rejected_on_host(flce_lib, kw):
    """A written buffer overlapping any other buffer of the call is refused
    before any launch.  The workspace is declared too small as well, so that a
    missed check would stop at the workspace check (FLCE_E_WORKSPACE) rather
    than enqueue anything."""
    assert _call(flce_lib, workspace_bytes=1) == -4  # the addresses alone are fine
    assert _call(flce_lib, workspace_bytes=1, **kw) == -1
    # frozen: dW is not written, so it may sit anywhere
    assert _call(flce_lib, workspace_bytes=1, frozen_weight=1, dW=FAKE["W"]) == -4


# Disjoint fake addresses 1 TiB apart, for the large shapes below (never
# dereferenced: the workspace is always declared too small).
FAR = {k: (i + 1) << 40 for i, k in enumerate(FAKE)}


@pytest.mark.parametrize("kw,status", [
    (dict(V=4194296), -4),                        # 256 slab rows of bf16 fit one 32-bit range
    (dict(V=4194304), -1),                        # ... and no longer
    (dict(V=2097144, dtype=0, accum_dtype=0), -4),
    (dict(V=2097152, dtype=0, accum_dtype=0), -1),
    (dict(V=4194304, frozen_weight=1, dW=None), -1),  # grad_input still reads the slab
    (dict(BT=1 << 20, H=2048, chunk_size=1024), -4),  # X of 4 GiB: rows gathered per chunk
    (dict(BT=1 << 20, H=2048, chunk_size=1 << 20, frozen_weight=1, dW=None), -4),  # 4 GiB chunk
])
def test_size_limits_on_host(flce_lib, kw, status):
    """The 32-bit buffer ranges of one GEMM tile bound V and the chunk, not X."""
    a = dict(FAR, BT=4, H=64, V=10, dtype=flce_lib.BF16, ignore_index=-100, reduction=0,
             chunk_size=0, chunk_mem_const=1, accum_dtype=flce_lib.BF16, frozen_weight=0,
             accumulate_dw=0, grad_output=None, workspace_bytes=1, stream=None)
    a.update(kw)
    assert flce_lib.flce_fwd_bwd(**a) == status


def test_noalloc_rejects_oversized_calls_on_host(flce_lib):
    """The no-allocation entry point refuses, before any HIP call, a call
    whose workspace would not fit its static scratch, and bad dtypes."""
    a = dict(FAR, BT=8192, H=4096, V=128256, dtype=flce_lib.BF16, ignore_index=-100,
             reduction=0, chunk_size=2048, chunk_mem_const=1, accum_dtype=flce_lib.F32,
             frozen_weight=0, accumulate_dw=0, grad_output=None, stream=None)
    a.pop("workspace")
    assert flce_lib.flce_workspace_bytes(8192, 4096, 128256, flce_lib.BF16, 2048, 1) > \
        flce_lib.SCRATCH_BYTES
    assert flce_lib.flce_fwd_bwd_ex_noalloc(**a) == -4
    assert "static scratch" in flce_lib.flce_last_error()
    assert flce_lib.flce_fwd_bwd_ex_noalloc(**dict(a, dtype=7)) == -2
    assert flce_lib.flce_fwd_bwd_ex_noalloc(**dict(a, H=0)) == -1


def test_row_index_offset(flce_lib):
    """The labelled-row index sits 256-byte aligned inside the workspace, with
    room for BT int32 entries, for every option set."""
    O = flce_lib.FlceOptions
    for args in [(8192, 4096, 128256, flce_lib.BF16, 2048, 1), (300, 96, 700, flce_lib.F32, 64, 1),
                 (1, 8, 1, flce_lib.F16, 0, 1), (1 << 20, 2048, 1000, flce_lib.BF16, 1024, 1)]:
        for opt in (None, O(1), O(0, None, 16, 0.0, 16, 16, 16)):
            off = flce_lib.flce_workspace_row_index_offset(*args, opt)
            ws = flce_lib.flce_workspace_bytes_ex(*args, opt)
            assert off % 256 == 0 and off + 4 * args[0] <= ws, (args, off, ws)
    assert flce_lib.flce_workspace_row_index_offset(128, 64, 100, 7, 64, 1, None) == 2 ** 64 - 1
    assert flce_lib.flce_workspace_row_index_offset(128, 0, 100, 0, 64, 1, None) == 2 ** 64 - 1


# ----------------------------------------------------------------- options
def test_workspace_ex_follows_options(flce_lib):
    """No options: the plain size.  Loss only: no slab.  Extras: small additions."""
    O = flce_lib.FlceOptions
    args = (8192, 4096, 128256, flce_lib.BF16, 2048, 1)
    plain = flce_lib.flce_workspace_bytes(*args)
    assert flce_lib.flce_workspace_bytes_ex(*args, None) == plain
    assert flce_lib.flce_workspace_bytes_ex(*args, O()) == plain
    fwd = flce_lib.flce_workspace_bytes_ex(*args, O(1))
    assert fwd < plain - 2048 * 128256 * 2  # the [c, V] slab is gone
    ex = flce_lib.flce_workspace_bytes_ex(*args, O(0, None, 16, 0.0, 16, 16, 16))
    assert plain < ex < plain * 1.2


def test_invalid_options_rejected_on_host(flce_lib):
    """Bad options fail before any launch.  The workspace is too small on
    purpose: a missed check would still stop at the workspace check, before
    anything is enqueued on the fake pointers."""
    O = flce_lib.FlceOptions
    ws = 1
    base = dict(X=FAKE["X"], W=FAKE["W"], targets=FAKE["targets"], BT=4, H=8, V=16,
                dtype=flce_lib.F32, ignore_index=-100, reduction=flce_lib.MEAN, chunk_size=4,
                chunk_mem_const=1, accum_dtype=flce_lib.F32, frozen_weight=0, accumulate_dw=0,
                grad_output=None, loss=FAKE["loss"], dX=FAKE["dX"], dW=FAKE["dW"],
                workspace=FAKE["workspace"], workspace_bytes=ws, stream=None)
    assert flce_lib.flce_fwd_bwd_ex(*base.values(), None, O()) == -4  # only the workspace is short
    for bad in (O(2), O(0, 8), O(0, None, 8), O(0, None, None, -1.0), O(0, None, None, float("nan")),
                O(0, None, None, 0.0, None, None, 4)):
        rc = flce_lib.flce_fwd_bwd_ex(*base.values(), None, bad)
        assert rc == -1, (bad.forward_only, rc)


# ------------------------------------------------------ MI355X chunk policy
POLICY_SHAPES = [  # BT, H, V, dtype, accum, frozen
    (8192, 4096, 128256, 2, 0, 0), (16384, 4096, 32000, 2, 2, 0), (16384, 4096, 32000, 0, 0, 0),
    (8192, 5376, 262144, 2, 2, 0), (32768, 5376, 262144, 2, 2, 0), (8192, 2048, 151936, 2, 2, 1),
    (256, 128, 1024, 0, 0, 0), (100, 64, 50, 1, 0, 0)]


@pytest.mark.parametrize("shape", POLICY_SHAPES)
def test_policy_is_a_clamped_power_of_two_within_budget(flce_lib, shape):
    BT, H, V, dt, adt, fr = shape
    s = 4 if dt == 0 else 2
    for budget in (0, 1 << 28, 1 << 33):
        c = flce_lib.flce_chunk_size_mi355x(BT, H, V, dt, adt, fr, budget)
        assert 1 <= c <= BT
        assert c == BT or (c & (c - 1)) == 0
        assert c == 1 or c * V * s <= (budget or (2 << 30))


def test_policy_monotone_in_budget_and_work(flce_lib):
    f = flce_lib.flce_chunk_size_mi355x
    cs = [f(8192, 4096, 128256, 2, 0, 0, b) for b in (1 << 24, 1 << 26, 1 << 28, 1 << 30, 0)]
    assert cs == sorted(cs)
    # freezing the weight removes the dW traffic, so a smaller chunk suffices
    assert f(8192, 2048, 151936, 2, 2, 1, 0) <= f(8192, 2048, 151936, 2, 2, 0, 0)


def test_policy_choices_at_benchmark_shapes(flce_lib):
    """The model's choices (validated by bench.py --chunk-sweep on MI355X)."""
    f = flce_lib.flce_chunk_size_mi355x
    assert f(8192, 4096, 128256, 2, 0, 0, 0) == 4096
    assert f(8192, 4096, 128256, 2, 0, 0, 1 << 28) == 1024  # 256 MiB slab budget
    assert f(16384, 4096, 32000, 2, 2, 0, 0) == 4096


def test_policy_rejects_invalid_arguments(flce_lib):
    f = flce_lib.flce_chunk_size_mi355x
    assert f(-1, 8, 8, 2, 2, 0, 0) == -1
    assert f(8, 0, 8, 2, 2, 0, 0) == -1
    assert f(8, 8, 8, 7, 7, 0, 0) == -1
    assert f(8, 8, 8, 2, 1, 0, 0) == -1  # bf16 operands with an fp16 accumulator


def test_profile_kind_mask_is_checked(flce_lib):
    """flce_profile_begin_kinds rejects an empty mask and unknown kinds; an open
    profile with nothing launched closes with zero counts (no HIP call)."""
    lib = flce_lib.load()
    assert lib.flce_profile_begin_kinds(0) == -1  # FLCE_E_ARG
    assert lib.flce_profile_begin_kinds(1 << len(flce_lib.KERNEL_KINDS)) == -1
    assert flce_lib.flce_profile_begin_kinds(["dw_gemm", "logits_gemm"]) == 0
    prof = flce_lib.flce_profile_end()
    assert all(v == (0, 0.0) for v in prof.values())
    assert flce_lib.flce_profile_begin() == 0
    flce_lib.flce_profile_end()
    with pytest.raises(flce_lib.FlceError):
        flce_lib.flce_profile_end()  # none open


def test_none_over_zero_rows_needs_no_loss_buffer(flce_lib):
    """Reduction none over BT = 0 rows has an empty loss vector: a NULL loss is
    accepted, and with a frozen weight nothing at all is enqueued."""
    assert _call(flce_lib, BT=0, reduction=2, loss=None, frozen_weight=1, dW=None) == 0
    assert _call(flce_lib, BT=0, reduction=0, loss=None, frozen_weight=1, dW=None) == -1
