"""CPU checks of the C ABI: the library loads, exports every function that
include/rope_attn.h declares, and rejects invalid arguments before any HIP
call (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rope_attn.h", "gram_select.h")]


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:rope_attn|gram)_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    from bwd_rope_apply_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("librope_attn.so is not built: run `python -m bwd_rope_apply_amd.build`")
    return _lib.load()


def test_header_declares_the_entry_points():
    assert _declared() == ["gram_cascade", "gram_cascade_workspace_bytes", "gram_select",
                           "gram_select_stages", "gram_select_workspace_bytes",
                           "rope_attn_bwd", "rope_attn_bwd_ex", "rope_attn_bwd_stages",
                           "rope_attn_bwd_workspace_bytes", "rope_attn_bwd_workspace_bytes_min",
                           "rope_attn_fwd", "rope_attn_fwd_ex", "rope_attn_fwd_noalloc",
                           "rope_attn_fwd_stages", "rope_attn_fwd_workspace_bytes",
                           "rope_attn_status_string", "rope_attn_workspace_flags"]


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_workspace_queries(lib):
    assert lib.rope_attn_fwd_workspace_bytes(1, 32, 8192, 128, 1, 1) > 0
    assert lib.rope_attn_bwd_workspace_bytes(1, 32, 8192, 128, 1, 1) > 0
    assert lib.rope_attn_fwd_workspace_bytes(1, 1, 16, 96, 1, 1) == 0   # bad D
    assert lib.rope_attn_bwd_workspace_bytes(0, 1, 16, 64, 1, 1) == 0   # bad B
    assert lib.rope_attn_bwd_workspace_bytes(1, 1, 16, 64, 7, 1) == 0   # bad dtype


A = 4096  # any 16-byte aligned non-null value; validation fails before use


@pytest.mark.parametrize("args,status", [
    ((None, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 1, A, 1 << 30, None), -1),
    ((A, A, A, A, A, 1, 1, 16, 96, 1, 1e4, None, 1, A, 1 << 30, None), -2),
    ((A, A, A, A, A, 1, 0, 16, 64, 1, 1e4, None, 1, A, 1 << 30, None), -2),
    ((A, A, A, A, A, 1, 1, 16, 64, 5, 1e4, None, 1, A, 1 << 30, None), -3),
    ((A + 2, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 1, A, 1 << 30, None), -4),
    ((A, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 1, A, 16, None), -5),
    ((A, A, A, A, A, 1, 1, 16, 64, 1, 0.0, None, 1, A, 1 << 30, None), -7),
    ((A, A, A, A, A, 1, 1, 16, 64, 1, float("nan"), None, 1, A, 1 << 30, None), -7),
    ((A, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 2, A, 1 << 30, None), -7),
    ((A, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 1, None, 1 << 30, None), -1),
])
def test_fwd_validation(lib, args, status):
    assert lib.rope_attn_fwd(*args) == status


@pytest.mark.parametrize("fields,status", [
    ((-1, 0.0, 0), -7), ((33, 0.0, 0), -7), ((0, -0.5, 0), -7), ((0, float("inf"), 0), -7),
    ((0, float("nan"), 0), -7), ((0, 0.0, -3), -7), ((0, 0.0, (1 << 30) - 8), -7),
])
def test_options_validation(lib, fields, status):
    """Invalid frequency-schedule options are rejected before any launch
    (D = 64: unrotated_pairs in [0, 32]; N = 16)."""
    import ctypes
    from bwd_rope_apply_amd import _lib
    op = _lib.Options(*fields)
    args = (A, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 1, A, 1 << 30, None)
    assert lib.rope_attn_fwd_ex(63, ctypes.addressof(op), *args) == status
    bargs = [A] * 10 + [1, 1, 16, 64, 1, 1e4, None, 1, A, 1 << 30, None]
    assert lib.rope_attn_bwd_ex(63, ctypes.addressof(op), *bargs) == status


def test_bwd_validation(lib):
    ok = [A] * 10 + [1, 1, 16, 64, 1, 1e4, None, 1, A, 1 << 30, None]
    bad = list(ok)
    bad[6] = None  # dq
    assert lib.rope_attn_bwd(*bad) == -1
    bad = list(ok)
    bad[9] = A + 4  # dalpha misaligned
    assert lib.rope_attn_bwd(*bad) == -4
    bad = list(ok)
    bad[19] = 8  # workspace too small
    assert lib.rope_attn_bwd(*bad) == -5


def test_status_strings(lib):
    for s in range(-7, 1):
        assert lib.rope_attn_status_string(s)
    assert lib.rope_attn_status_string(-99) == b"unknown status"


@pytest.mark.parametrize("N,ptr,idx,nnz,status", [
    (65537, A, A, 4, -2),      # more than 512 blocks per head
    (256, A, A, -1, -7),       # negative entry count
    (256, A, None, 3, -7),     # entries without an index array
    (256, A + 2, A, 4, -4),    # misaligned offsets
    (256, A, A + 1, 4, -4),    # misaligned indices
])
def test_block_list_validation(lib, N, ptr, idx, nnz, status):
    """Invalid block lists are rejected before any launch (D = 64)."""
    import ctypes
    from bwd_rope_apply_amd import _lib
    op = _lib.Options(0, 0.0, 0, ptr, idx, nnz)
    args = (A, A, A, A, A, 1, 1, N, 64, 1, 1e4, None, 1, A, 1 << 40, None)
    assert lib.rope_attn_fwd_ex(63, ctypes.addressof(op), *args) == status
    bargs = [A] * 10 + [1, 1, N, 64, 1, 1e4, None, 1, A, 1 << 40, None]
    assert lib.rope_attn_bwd_ex(63, ctypes.addressof(op), *bargs) == status


def _panel_bytes(B, H, N, causal):
    """fp16 dS panels: one per 256-query block, [keys][256]; under the causal
    mask panel b keeps keys 0 .. 256 (b + 1) - 1."""
    n = -(-N // 256)
    per_head = 256 * 256 * n * (n + 1) // 2 if causal else n * 256 * 256 * n
    return 2 * B * H * per_head


def test_workspace_panels(lib):
    """The full backward workspace adds the dS panels (bf16, up to 16 GiB),
    at the end of the layout; the minimal one is the recomputing layout."""
    for B, H, N, causal in ((1, 32, 8192, 1), (2, 3, 1000, 0), (1, 1, 1, 1), (1, 8, 32768, 1)):
        full = lib.rope_attn_bwd_workspace_bytes(B, H, N, 128, 1, causal)
        lo = lib.rope_attn_bwd_workspace_bytes_min(B, H, N, 128, 1, causal)
        pb = _panel_bytes(B, H, N, causal)
        assert full - lo == (pb + 255) // 256 * 256, (B, H, N, causal)
        assert lo > lib.rope_attn_fwd_workspace_bytes(B, H, N, 128, 1, causal)
    # fp32 inputs and D = 64 never use panels; above 16 GiB of panels neither does bf16
    assert (lib.rope_attn_bwd_workspace_bytes(1, 8, 32768, 64, 1, 1)
            == lib.rope_attn_bwd_workspace_bytes_min(1, 8, 32768, 64, 1, 1))
    assert (lib.rope_attn_bwd_workspace_bytes(1, 4, 4096, 64, 0, 1)
            == lib.rope_attn_bwd_workspace_bytes_min(1, 4, 4096, 64, 0, 1))
    assert _panel_bytes(1, 64, 32768, 1) > 16 << 30
    assert (lib.rope_attn_bwd_workspace_bytes(1, 64, 32768, 128, 1, 1)
            == lib.rope_attn_bwd_workspace_bytes_min(1, 64, 32768, 128, 1, 1))
    assert lib.rope_attn_bwd_workspace_bytes_min(1, 1, 16, 96, 1, 1) == 0   # bad D


def test_workspace_covers_block_lists(lib):
    """The workspace queries take no options, so their size must hold the
    block-list layout too (visibility mask, and the dQ/dK/dV slots for the
    one-block exact corner) at lengths where the dense corner is larger."""
    for N in (256, 8192, 20000, 65536):
        f = lib.rope_attn_fwd_workspace_bytes(1, 4, N, 128, 1, 1)
        b = lib.rope_attn_bwd_workspace_bytes(1, 4, N, 128, 1, 1)
        nb = (N + 127) // 128
        assert f >= 4 * 4 * nb * ((nb + 31) // 32)
        assert b > f


def test_gram_workspace_queries(lib):
    assert lib.gram_select_workspace_bytes(1, 8192, 4096) >= 8 * 8192
    assert lib.gram_cascade_workspace_bytes(8192, 4096) >= 17 * 8192
    assert lib.gram_select_workspace_bytes(1, 512, 100) == 0        # d not a multiple of 64
    assert lib.gram_select_workspace_bytes(0, 512, 768) == 0
    assert lib.gram_select_workspace_bytes(1, 1 << 21, 64) == 0     # T > 2^20
    assert lib.gram_cascade_workspace_bytes(1 << 16, 1 << 16) == 0  # T d > 2^31


W_ = 1 << 30


@pytest.mark.parametrize("args,status", [
    ((None, 1, 64, 64, 1, 0.3, A, A, None, A, W_, None), -1),      # x
    ((A, 1, 64, 64, 1, 0.3, None, A, None, A, W_, None), -1),      # max_cos
    ((A, 1, 64, 64, 3, 0.3, A, A, None, A, W_, None), -3),         # dtype
    ((A, 1, 64, 96, 1, 0.3, A, A, None, A, W_, None), -2),         # d
    ((A, 1, 0, 64, 1, 0.3, A, A, None, A, W_, None), -2),          # T
    ((A, 1, 64, 64, 1, -0.1, A, A, None, A, W_, None), -7),        # tau < 0
    ((A, 1, 64, 64, 1, float("nan"), A, A, None, A, W_, None), -7),
    ((A + 8, 1, 64, 64, 1, 0.3, A, A, None, A, W_, None), -4),     # x alignment
    ((A, 1, 64, 64, 1, 0.3, A + 2, A, None, A, W_, None), -4),     # max_cos alignment
    ((A, 1, 64, 64, 1, 0.3, A, A, None, A + 16, W_, None), -4),    # workspace alignment
    ((A, 1, 64, 64, 1, 0.3, A, A, None, A, 16, None), -5),         # workspace size
])
def test_gram_select_validation(lib, args, status):
    assert lib.gram_select(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, 64, 64, 1, 0.3, None, A, A, None, A, W_, None), -1),      # prev
    ((A, 64, 64, 2, float("inf"), A, A, A, None, A, W_, None), -7),
    ((A, 64, 128, 0, 0.3, A, A, A, None, A, W_, None), -3),
    ((A, 64, 64, 1, 0.3, A, A, A, None, A, 64, None), -5),
])
def test_gram_cascade_validation(lib, args, status):
    assert lib.gram_cascade(*args) == status


def test_headers_compile_as_plain_c(tmp_path):
    """Both headers are C: a C99 translation unit that includes them and
    takes the address of every declared function compiles without warnings."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use.c"
    names = _declared()
    src.write_text('#include "rope_attn.h"\n#include "gram_select.h"\n'
                   "typedef void (*fn)(void);\n"
                   "fn table[] = {" + ", ".join(f"(fn)&{n}" for n in names) + "};\n"
                   "int main(void) { return table[0] == 0; }\n")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        f"-I{os.path.join(ROOT, 'include')}", "-c", str(src), "-o", str(tmp_path / "use.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_workspace_flags_validation(lib):
    """The range-flag query rejects a NULL, misaligned or too small workspace
    and a NULL result pointer before any HIP call."""
    v = ctypes.c_uint(7)
    assert lib.rope_attn_workspace_flags(None, 1 << 20, ctypes.byref(v), None) == -1
    assert lib.rope_attn_workspace_flags(A, 1 << 20, None, None) == -1
    assert lib.rope_attn_workspace_flags(A + 4, 1 << 20, ctypes.byref(v), None) == -4
    assert lib.rope_attn_workspace_flags(A, 2, ctypes.byref(v), None) == -5
    assert v.value == 7


def test_binding_checks_caller_tensors():
    """The binding rejects caller-supplied tensors of the wrong shape, dtype,
    layout or device before anything reaches the library (CPU tensors here:
    each check is hit in order, the device check last)."""
    import torch
    from bwd_rope_apply_amd import _lib
    dev = torch.device("cuda", 0)
    ok = torch.zeros(2, 3, dtype=torch.float32)
    cases = [
        (torch.zeros(2, 4), "shape"),
        (torch.zeros(2, 3, dtype=torch.bfloat16), "float32"),
        (torch.zeros(3, 2).t(), "not contiguous"),
        (ok, "device tensor"),
    ]
    for t, msg in cases:
        with pytest.raises(ValueError, match=msg):
            _lib._check_tensor("out", t, (2, 3), torch.float32, dev)
    with pytest.raises(ValueError, match="contiguous"):
        _lib._workspace(torch.zeros(8, 2, dtype=torch.uint8).t(), 16, dev)
    with pytest.raises(ValueError, match="device tensor"):
        _lib._workspace(torch.zeros(16, dtype=torch.uint8), 16, dev)
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        _lib.fwd(q, q, q, 1e4)


def test_noalloc_validation(lib):
    """The no-allocation forward validates like the forward and rejects a
    problem larger than its fixed array before any HIP call."""
    assert lib.rope_attn_fwd_noalloc(A, A, A, A, A, 1, 1, 16, 96, 1, 1e4, None, 1, None) == -2
    assert lib.rope_attn_fwd_noalloc(A, A, A, A, A, 1, 1, 16, 64, 9, 1e4, None, 1, None) == -3
    assert lib.rope_attn_fwd_noalloc(None, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 1, None) == -1
    # 1 x 64 x 8192 x 128 bf16 needs ~390 MiB of workspace, past the 64 MiB array
    assert lib.rope_attn_fwd_noalloc(A, A, A, A, A, 1, 64, 8192, 128, 1, 1e4, None, 1, None) == -5
    # base and causal are checked before the device's array is looked up
    assert lib.rope_attn_fwd_noalloc(A, A, A, A, A, 1, 1, 16, 64, 1, 0.0, None, 1, None) == -7
    assert lib.rope_attn_fwd_noalloc(A, A, A, A, A, 1, 1, 16, 64, 1, float("nan"), None, 1, None) == -7
    assert lib.rope_attn_fwd_noalloc(A, A, A, A, A, 1, 1, 16, 64, 1, 1e4, None, 2, None) == -7
