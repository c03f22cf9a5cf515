"""The C ABI without a GPU: the library loads, exports what ``include/w4a16.h``
declares, the ctypes struct matches the C layout, and host-side validation
rejects bad arguments before anything is enqueued.

Only argument combinations that fail validation are passed with placeholder
pointers, so no kernel is ever launched here.
"""

import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

from weight_only_int4_rtn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
FAKE = 0x100000   # 16-byte aligned placeholder address, never dereferenced
MISALIGNED = 0x100004


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        import weight_only_int4_rtn_amd.build as b
        b.build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_abi_version_and_status_strings(L):
    assert L.w4a16_abi_version() == _lib.ABI_VERSION == 3
    assert _lib.status_string(0) == "W4A16_OK"
    assert _lib.status_string(3) == "W4A16_ERR_WORKSPACE"
    assert _lib.status_string(99) == "W4A16_UNKNOWN_STATUS"


def test_struct_layout_matches_c_compiler():
    fields = [f[0] for f in _lib.MoeArgs._fields_]
    prog = "#include <stdio.h>\n#include <stddef.h>\n#include \"w4a16.h\"\nint main(void){\n"
    prog += 'printf("%zu\\n", sizeof(moe_w4a16_args));\n'
    for f in fields:
        prog += f'printf("%zu\\n", offsetof(moe_w4a16_args, {f}));\n'
    prog += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == C.sizeof(_lib.MoeArgs)
    assert got[1:] == [getattr(_lib.MoeArgs, f).offset for f in fields]


def base_args(T=1, H=2048, I=512, E=256, k=8, bits=4):
    a = _lib.MoeArgs()
    a.T, a.H, a.I, a.E, a.top_k, a.bits, a.group = T, H, I, E, k, bits, 128
    for i, f in enumerate(("x", "router_logits", "w13", "s13", "w2", "s2", "y")):
        setattr(a, f, FAKE + 0x1000 * i)
    return a


def forward_status(L, a):
    return L.moe_w4a16_forward(C.byref(a), None)


@pytest.mark.parametrize("field,value,expect", [
    ("bits", 5, _lib.W4A16_ERR_INVALID_ARG),
    ("group", 64, _lib.W4A16_ERR_INVALID_ARG),
    ("H", 2000, _lib.W4A16_ERR_INVALID_ARG),
    ("I", 100, _lib.W4A16_ERR_INVALID_ARG),
    ("top_k", 0, _lib.W4A16_ERR_INVALID_ARG),
    ("top_k", 300, _lib.W4A16_ERR_INVALID_ARG),
    ("top_k", 17, _lib.W4A16_ERR_UNSUPPORTED),
    ("E", 0, _lib.W4A16_ERR_INVALID_ARG),
    ("E", 2048, _lib.W4A16_ERR_UNSUPPORTED),
    ("T", -1, _lib.W4A16_ERR_INVALID_ARG),
    ("H", 32768, _lib.W4A16_ERR_UNSUPPORTED),
    ("x", 0, _lib.W4A16_ERR_INVALID_ARG),
    ("y", 0, _lib.W4A16_ERR_INVALID_ARG),
    ("w13", MISALIGNED, _lib.W4A16_ERR_INVALID_ARG),
    ("shared_bits", 3, _lib.W4A16_ERR_INVALID_ARG),
])
def test_forward_rejects_bad_arguments(L, field, value, expect):
    a = base_args()
    setattr(a, field, value)
    assert forward_status(L, a) == expect
    assert _lib.last_error()


def test_forward_rejects_missing_ids_and_small_workspace(L):
    a = base_args()
    a.router_logits = None
    assert forward_status(L, a) == _lib.W4A16_ERR_INVALID_ARG
    a = base_args()
    need = L.moe_w4a16_workspace_size(C.byref(a))
    assert need > 0
    a.workspace, a.workspace_bytes = FAKE + 0x10000, need - 1
    assert forward_status(L, a) == _lib.W4A16_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = None, need
    assert forward_status(L, a) == _lib.W4A16_ERR_WORKSPACE
    a = base_args()
    a.y = a.x
    a.workspace, a.workspace_bytes = FAKE + 0x10000, need
    assert forward_status(L, a) == _lib.W4A16_ERR_INVALID_ARG
    a = base_args()
    a.shared_bits, a.shared_I = 8, 512
    assert forward_status(L, a) == _lib.W4A16_ERR_INVALID_ARG   # shared pointers missing


def test_forward_zero_tokens_is_a_noop(L):
    a = base_args(T=0)
    for f in ("x", "router_logits", "w13", "s13", "w2", "s2", "y"):
        setattr(a, f, None)
    assert forward_status(L, a) == _lib.W4A16_OK


def test_workspace_init_validation(L):
    """Rejections happen on the host; nothing is enqueued (no GPU here)."""
    assert L.moe_w4a16_workspace_init(None, 1 << 20, None) == _lib.W4A16_ERR_INVALID_ARG
    assert L.moe_w4a16_workspace_init(C.c_void_p(MISALIGNED), 1 << 20, None) == _lib.W4A16_ERR_INVALID_ARG
    assert L.moe_w4a16_workspace_init(C.c_void_p(FAKE), _lib.WORKSPACE_HEAD_BYTES - 1, None) == _lib.W4A16_ERR_WORKSPACE
    assert str(_lib.WORKSPACE_HEAD_BYTES) in _lib.last_error()


def test_workspace_head_size_matches_header():
    hdr = open(HEADER).read()
    m = re.search(r"#define W4A16_WORKSPACE_HEAD_BYTES (\d+)", hdr)
    assert m and int(m.group(1)) == _lib.WORKSPACE_HEAD_BYTES


def test_workspace_size(L):
    sizes = {}
    for T in (1, 32, 64, 65, 8192):
        sizes[T] = L.moe_w4a16_workspace_size(C.byref(base_args(T=T)))
        assert sizes[T] > 0 and sizes[T] % 256 == 0
    assert sizes[1] < sizes[32] < sizes[8192]
    # the gate/up output of 8192 x 8 pairs alone is 64 MiB of bf16
    assert sizes[8192] >= 8192 * 8 * 512 * 2
    bad = base_args()
    bad.bits = 3
    assert L.moe_w4a16_workspace_size(C.byref(bad)) == 0
    sh = base_args(T=4)
    sh.shared_bits, sh.shared_I = 8, 512
    assert L.moe_w4a16_workspace_size(C.byref(sh)) > L.moe_w4a16_workspace_size(C.byref(base_args(T=4)))


@pytest.mark.parametrize("args,expect", [
    ((FAKE, 0, 1, 8, 256, 5, 128), _lib.W4A16_ERR_INVALID_ARG),     # bits
    ((FAKE, 0, 1, 8, 256, 4, 64), _lib.W4A16_ERR_INVALID_ARG),      # group
    ((FAKE, 0, 1, 8, 200, 4, 128), _lib.W4A16_ERR_INVALID_ARG),     # cols % 128
    ((FAKE, 2, 1, 8, 256, 4, 128), _lib.W4A16_ERR_INVALID_ARG),     # dtype
    ((None, 0, 1, 8, 256, 4, 128), _lib.W4A16_ERR_INVALID_ARG),     # NULL w
    ((MISALIGNED, 0, 1, 8, 256, 4, 128), _lib.W4A16_ERR_INVALID_ARG),
    ((FAKE, 0, -1, 8, 256, 4, 128), _lib.W4A16_ERR_INVALID_ARG),
    ((None, 0, 0, 8, 256, 4, 128), _lib.W4A16_OK),                  # nothing to do
])
def test_quantize_validation(L, args, expect):
    w, dt, n, r, c, bits, group = args
    packed = None if w is None else FAKE
    st = L.rtn_quantize_pack(w, dt, n, r, c, bits, group, packed, packed, None)
    assert st == expect
