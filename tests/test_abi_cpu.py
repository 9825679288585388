"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point that include/csa2.h declares, and rejects bad arguments before any
HIP call (every call below fails validation, so nothing is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

import hierarchical_sparse_attention_csa2_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = csa2.load_library()
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", csa2.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (csa2_\w+)", out))
    assert set(names) <= exported
    assert set(csa2.EXPORTED) == set(names)


def test_status_strings():
    assert csa2.status_string(0) == "ok"
    assert "invalid" in csa2.status_string(-1)
    assert "workspace" in csa2.status_string(-3)
    assert csa2.status_string(12345) == "unknown status"


NULL = None
P = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def test_validation_rejects_before_launch():
    L = csa2.load_library()
    # index_scan: NULL inputs, bad sizes
    assert L.csa2_index_scan(NULL, P, P, P, P, 1, 1, 16, NULL, P, NULL, NULL) == -1
    assert L.csa2_index_scan(P, P, P, P, P, 0, 1, 16, NULL, P, NULL, NULL) == -1
    assert L.csa2_index_scan(P, P, P, P, P, 1, 0, 16, NULL, P, NULL, NULL) == -1
    assert L.csa2_index_scan(P, P, P, P, P, 1, 1, 0, NULL, P, NULL, NULL) == -1
    assert L.csa2_index_scan(P, P, P, P, P, 1, 1, 16, NULL, NULL, NULL, NULL) == -1
    # select_blocks
    assert L.csa2_select_blocks(P, NULL, 2, P, 1, 0, P, 0, NULL, NULL) == -1
    assert L.csa2_select_blocks(P, NULL, 2, P, 1, 4, P, 2, NULL, NULL) == -1
    assert L.csa2_select_blocks(P, NULL, 0, P, 1, 4, P, 0, NULL, NULL) == -1
    # index_pool
    assert L.csa2_index_pool(P, P, P, P, NULL, 4, P, 1, 1, 16, P, NULL) == -1
    assert L.csa2_index_pool(P, P, P, P, P, 0, P, 1, 1, 16, P, NULL) == -1
    # topk
    assert L.csa2_topk(NULL, P, 4, P, 1, 8, P, NULL) == -1
    assert L.csa2_topk(P, P, 4, P, 1, -1, P, NULL) == -1
    assert L.csa2_topk(P, P, 4, P, 0, 8, P, NULL) == -1
    assert L.csa2_topk(P, P, 4, P, 1, 0, P, NULL) == 0          # k = 0: nothing to do
    # index_full: workspace too small, missing idx
    assert L.csa2_index_full(P, P, P, P, P, 1, 1, 64, 4, 8, NULL, NULL, P, P, NULL, 0, NULL) == -3
    assert L.csa2_index_full(P, P, P, P, P, 1, 1, 64, 4, 8, NULL, NULL, P, NULL, P, 1 << 20, NULL) == -1
    assert L.csa2_index_full(P, P, P, P, P, 1, 1, 64, 0, 8, NULL, NULL, P, P, P, 1 << 20, NULL) == -1
    # sparse_attn: unsupported head counts, bad window, missing workspace
    f = ctypes.c_float(0.04)
    assert L.csa2_sparse_attn(P, P, P, P, 8, P, P, P, 4, 1, 1, 64, 24, 8, f, P, P, 1 << 20, NULL) == -2
    assert L.csa2_sparse_attn(P, P, P, P, 8, P, P, P, 4, 1, 1, 64, 128, 8, f, P, P, 1 << 20, NULL) == -2
    assert L.csa2_sparse_attn(P, P, P, P, 8, P, P, P, 9, 1, 1, 64, 64, 8, f, P, P, 1 << 20, NULL) == -1
    assert L.csa2_sparse_attn(P, P, P, NULL, 8, P, P, P, 4, 1, 1, 64, 64, 8, f, P, P, 1 << 20, NULL) == -1
    assert L.csa2_sparse_attn(P, P, P, P, 512, P, P, P, 128, 1, 1, 64, 64, 128, f, P, NULL, 0, NULL) == -3
    assert L.csa2_sparse_attn(P, P, P, P, 8, P, P, P, 4, 1, 1, 64, 64, 8, ctypes.c_float(float("nan")), P, P,
                              1 << 20, NULL) == -1


def test_validation_rejects_misaligned_pointers():
    """Tensor pointers must be 16-byte aligned; the check runs before any launch."""
    L = csa2.load_library()
    Q = ctypes.c_void_p(0x1004)
    f = ctypes.c_float(0.04)
    assert L.csa2_index_scan(Q, P, P, P, P, 1, 1, 16, NULL, P, NULL, NULL) == -1
    assert L.csa2_index_scan(P, P, P, P, P, 1, 1, 16, NULL, Q, NULL, NULL) == -1
    assert L.csa2_select_blocks(P, Q, 2, P, 1, 4, P, 0, NULL, NULL) == -1
    assert L.csa2_index_pool(P, P, Q, P, P, 4, P, 1, 1, 16, P, NULL) == -1
    assert L.csa2_topk(P, NULL, 4, P, 1, 8, Q, NULL) == -1
    assert L.csa2_index_full(P, P, P, P, P, 1, 1, 64, 4, 8, NULL, NULL, P, P, Q, 1 << 20, NULL) == -1
    assert L.csa2_sparse_attn(Q, P, P, P, 8, P, P, P, 4, 1, 1, 64, 64, 8, f, P, P, 1 << 20, NULL) == -1
    assert L.csa2_sparse_attn(P, P, P, P, 8, P, P, P, 4, 1, 1, 64, 64, 8, f, Q, P, 1 << 20, NULL) == -1


def test_cache_write_validation():
    """The cache-write entry points check sizes, NULLs and alignment before any launch."""
    L = csa2.load_library()
    Q = ctypes.c_void_p(0x1004)
    # D must be a power of two in [32, 16384]; ratio in [1, 64]; weights needed for ratio > 1
    assert L.csa2_cache_write_mxfp4(P, P, 4, 2, 96, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(P, P, 4, 2, 16, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(P, P, 4, 2, 32768, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(P, P, 4, 0, 128, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(P, P, 4, 65, 128, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(P, NULL, 4, 2, 128, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(P, P, -1, 2, 128, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(NULL, P, 4, 2, 128, P, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(P, P, 4, 2, 128, NULL, P, NULL) == -1
    assert L.csa2_cache_write_mxfp4(Q, P, 4, 2, 128, P, P, NULL) == -1                    # x: 16 bytes
    assert L.csa2_cache_write_mxfp4(P, ctypes.c_void_p(0x1002), 4, 2, 128, P, P, NULL) == -1   # w: 4 bytes
    assert L.csa2_cache_write_mxfp4(P, P, 4, 2, 128, ctypes.c_void_p(0x1001), P, NULL) == -1   # codes: 2 bytes
    # nothing to write: no launch, success (ratio 1 may omit the weights)
    assert L.csa2_cache_write_mxfp4(P, NULL, 0, 1, 128, P, P, NULL) == 0
    assert L.csa2_cache_write_e4m3(P, 6, P, NULL) == -1
    assert L.csa2_cache_write_e4m3(P, -4, P, NULL) == -1
    assert L.csa2_cache_write_e4m3(NULL, 8, P, NULL) == -1
    assert L.csa2_cache_write_e4m3(Q, 8, P, NULL) == -1
    assert L.csa2_cache_write_e4m3(P, 8, ctypes.c_void_p(0x1002), NULL) == -1
    assert L.csa2_cache_write_e4m3(P, 0, P, NULL) == 0
    assert L.csa2_cache_write_e4m3(NULL, 0, NULL, NULL) == 0
    assert L.csa2_cache_write_mxfp4(NULL, NULL, 0, 2, 128, NULL, NULL, NULL) == 0


def test_workspace_bytes():
    L = csa2.load_library()
    # index_full: block maxima + the first k blocks + their scores
    n = csa2.csa2_workspace_bytes(csa2.CSA2_OP_INDEX_FULL, 4, 1, 524288, 0, 512)
    assert n >= 4 * 65536 * 4 + 4 * 512 * 4 + 4 * 4096 * 4
    assert csa2.csa2_workspace_bytes(csa2.CSA2_OP_INDEX_FULL, 0, 1, 16, 0, 8) == 0
    assert csa2.csa2_workspace_bytes(99, 1, 1, 16, 0, 8) == 0
    # attention: split partials only when a row is split over several workgroups
    a = csa2.csa2_workspace_bytes(csa2.CSA2_OP_SPARSE_ATTN, 4, 1, 0, 64, 640)
    assert a > 0 and a % (64 * 514 * 4) == 0
    assert csa2.csa2_workspace_bytes(csa2.CSA2_OP_SPARSE_ATTN, 4, 1, 0, 24, 640) == 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 64), dtype=torch.uint8)
    with pytest.raises(ValueError):
        csa2.csa2_index_scan(x, x, x, x, torch.zeros(1, dtype=torch.int32), 1, 1, 1,
                             torch.zeros((1, 1), dtype=torch.float32))


def test_header_is_plain_c_and_links(tmp_path):
    """include/csa2.h compiles as C99 (no C++ constructs), a C program that
    references every entry point links against libcsa2.so, and it runs: the
    host-side answers (status strings, workspace sizes, argument errors
    returned before any launch) reach a C caller unchanged."""
    import shutil

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = _declared()
    src = tmp_path / "use_csa2.c"
    body = "\n".join(f"    (void)&{n};" for n in names)
    checks = r"""
    if (csa2_workspace_bytes(CSA2_OP_INDEX_FULL, 4, 1, 524288, 0, 512) == 0) return 2;
    if (csa2_workspace_bytes(99, 1, 1, 1, 0, 1) != 0) return 3;
    if (csa2_index_scan(NULL, NULL, NULL, NULL, NULL, 1, 1, 1, NULL, NULL, NULL, NULL) != CSA2_ERR_INVALID)
        return 4;
    if (csa2_sparse_attn(NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, 0, 1, 1, 1, 64, 0, 1.0f, NULL, NULL, 0,
                         NULL) != CSA2_ERR_INVALID)
        return 5;
    if (csa2_cache_write_e4m3(NULL, 0, NULL, NULL) != CSA2_OK) return 6;
    printf("%s|%s\n", csa2_status_string(CSA2_OK), csa2_status_string(CSA2_ERR_WORKSPACE));
"""
    src.write_text('#include "csa2.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   "int main(void) {\n" + body + "\n" + checks + "    return 0;\n}\n")
    exe = tmp_path / "use_csa2"
    libdir = os.path.dirname(csa2.LIB_PATH)
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                          str(src), "-o", str(exe), "-L", libdir, "-l:libcsa2.so", f"-Wl,-rpath,{libdir}"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stderr)
    assert run.stdout.strip() == "ok|workspace missing or too small"
