"""CPU checks of the C ABI: the library loads and exports every declared entry
point, and the host-side validator, layout adapter and chunk planner behave
(built with g++ under AddressSanitizer/UBSan, no GPU involved)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcp.h")
CSRC = os.path.join(ROOT, "context_lse_merge_amd", "csrc")
LIB = os.path.join(ROOT, "context_lse_merge_amd", "libdcp.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dcp_workspace_create", "dcp_workspace_destroy", "dcp_lse_combine", "dcp_last_error",
              "dcp_status_string"):
        assert n in names


def test_library_loads_and_exports_every_declared_symbol():
    assert os.path.exists(LIB), "libdcp.so is not built"
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, "declared in dcp.h but not exported: %s" % missing
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dcp_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_binding_imports_and_status_strings():
    import context_lse_merge_amd as dcp
    assert dcp.dcp_status_string(dcp.DCP_ERR_STREAM) == "DCP_ERR_STREAM"
    assert dcp.dcp_status_string(12345) == "DCP_ERR_UNKNOWN"
    assert dcp.DCP_HEAD_DIM == 512


def test_workspace_errors_through_the_binding():
    import context_lse_merge_amd as dcp
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_workspace_create(0, 16, 4, stream=0x1000)
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG and "capacity" in str(e.value)
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_workspace_create(8, 16, 4, d=128, stream=0x1000)
    assert e.value.status == dcp.DCP_ERR_LAYOUT
    fake = 0x7 << 40          # a device address the library stores but never touches
    ws = dcp.dcp_workspace_create(8, 16, 4, stream=0x1000, buf=fake, buf_bytes=dcp.dcp_workspace_size(8, 16, 4))
    assert ws.handle
    dcp.dcp_workspace_set_load_policy(ws, dcp.DCP_LOAD_CACHED)
    dcp.dcp_workspace_set_load_policy(ws, dcp.DCP_LOAD_STREAMING)
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_workspace_set_load_policy(ws, 7)
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG and "policy" in str(e.value)
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_workspace_create(8, 16, 4, dtype=5, stream=0x1000)
    assert e.value.status == dcp.DCP_ERR_LAYOUT
    dcp.dcp_workspace_destroy(ws)
    assert ws.handle is None


def test_workspace_buffer_size_and_rejection_through_the_binding():
    """dcp_workspace_size is the landing zone's size (capacity x h_local x cp rows of D bf16/fp16 values plus one
    fp32 LSE each, regions rounded to 256 bytes); create rejects a missing, smaller or misaligned buffer before
    making anything."""
    import context_lse_merge_amd as dcp
    fake = 0x7 << 40
    for cap, hl, cp, dt in ((128, 16, 4, dcp.DCP_DTYPE_BF16), (3, 5, 3, dcp.DCP_DTYPE_FP16), (1, 1, 1, 0)):
        rows = cap * hl * cp
        want = (rows * 1024 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
        n = dcp.dcp_workspace_size(cap, hl, cp, dtype=dt)
        assert n == want
        ws = dcp.dcp_workspace_create(cap, hl, cp, dtype=dt, stream=0x1000, buf=fake, buf_bytes=n)
        ws.close()
        with pytest.raises(dcp.DcpError) as e:
            dcp.dcp_workspace_create(cap, hl, cp, dtype=dt, stream=0x1000, buf=fake, buf_bytes=n - 1)
        assert e.value.status == dcp.DCP_ERR_WORKSPACE and "dcp_workspace_size" in str(e.value)
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_workspace_create(8, 16, 4, stream=0x1000, buf=0, buf_bytes=1 << 30)
    assert e.value.status == dcp.DCP_ERR_WORKSPACE
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_workspace_create(8, 16, 4, stream=0x1000, buf=fake + 8, buf_bytes=1 << 30)
    assert e.value.status == dcp.DCP_ERR_ALIGN
    assert dcp.dcp_workspace_size(128, 16, 4) == 128 * 16 * 4 * (1024 + 4)


def test_varlen_scratch_size_limits_through_the_binding():
    import context_lse_merge_amd as dcp
    assert dcp.dcp_mla_partial_decode_varlen_scratch_size(0, 128, 1 << 30, 4) == 0
    assert dcp.dcp_mla_partial_decode_varlen_scratch_size(4, 128, 1 << 30, 4) > 0
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_mla_partial_decode_varlen_scratch_size(4, 128, (1 << 30) + 1, 4)
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG and "max_seq_len" in str(e.value)
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_mla_partial_decode_varlen_scratch_size(1 << 24, 128, 4096, 4)
    assert e.value.status == dcp.DCP_ERR_INVALID_ARG


def test_host_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "host_plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "host_plan_check.cpp"), os.path.join(CSRC, "dcp_host.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    # a library preloaded by the environment may sit before the ASan runtime
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stderr + r.stdout
    assert "host plan checks passed" in r.stdout


def test_noalloc_static_scratch_covers_every_fixed_length_shape():
    """dcp_mla_partial_decode_noalloc keeps the split partials in a static array of DCP_NOALLOC_SCRATCH_BYTES:
    over a grid of shapes that includes the largest case (255 row-block x shard units, two splits each), the
    scratch dcp_mla_partial_decode needs never exceeds it, and the largest case needs exactly that much."""
    import context_lse_merge_amd as dcp
    cap = dcp.DCP_NOALLOC_SCRATCH_BYTES
    worst = 0
    for cp in (1, 2, 3, 4, 5, 7, 8, 13, 16, 31, 64):
        for hq in (1, 7, 16, 100, 128, 129, 200, 256):
            for B in list(range(1, 40)) + [51, 63, 64, 65, 127, 128, 255, 256, 257, 1000]:
                for T in (0, 1, 31, 255, 256, 257, 511, 2560, 4097, 32768, 131072, 1 << 20):
                    worst = max(worst, dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp))
    assert worst == cap == dcp.dcp_mla_partial_decode_scratch_size(51, 128, 2560, 5)
