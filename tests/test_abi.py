"""The C ABI without a GPU: the library loads, exports what ``include/w4a16.h``
declares, the ctypes struct matches the C layout, and host-side validation
rejects bad arguments before anything is enqueued.

Only argument combinations that fail validation are passed with placeholder
pointers, so no kernel is ever launched here.
"""

import ast
import ctypes as C
import os
import re
import subprocess
import sys
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
    assert L.w4a16_abi_version() == _lib.ABI_VERSION == 7
    assert _lib.status_string(0) == "W4A16_OK"
    assert _lib.status_string(3) == "W4A16_ERR_WORKSPACE"
    assert _lib.status_string(5) == "W4A16_ERR_TIMEOUT"
    assert _lib.status_string(99) == "W4A16_UNKNOWN_STATUS"


@pytest.mark.parametrize("cstruct,ctype", [(_lib.MoeArgs, "moe_w4a16_args"), (_lib.LinearArgs, "w4a16_linear_args")])
def test_struct_layout_matches_c_compiler(cstruct, ctype):
    fields = [f[0] for f in cstruct._fields_]
    prog = "#include <stdio.h>\n#include <stddef.h>\n#include \"w4a16.h\"\nint main(void){\n"
    prog += f'printf("%zu\\n", sizeof({ctype}));\n'
    for f in fields:
        prog += f'printf("%zu\\n", offsetof({ctype}, {f}));\n'
    prog += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == C.sizeof(cstruct)
    assert got[1:] == [getattr(cstruct, f).offset for f in fields]


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
    need = L.moe_w4a16_workspace_size(a.T, a.H, a.I, a.E, a.top_k, 0)
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
        sizes[T] = L.moe_w4a16_workspace_size(T, 2048, 512, 256, 8, 0)
        assert sizes[T] > 0 and sizes[T] % 256 == 0
    assert sizes[1] < sizes[32] < sizes[8192]
    # the gate/up output of 8192 x 8 pairs alone is 64 MiB of bf16
    assert sizes[8192] >= 8192 * 8 * 512 * 2
    for bad in ((1, 2000, 512, 256, 8, 0), (1, 2048, 100, 256, 8, 0), (1, 2048, 512, 256, 0, 0),
                (1, 2048, 512, 8, 9, 0), (-1, 2048, 512, 256, 8, 0), (1, 2048, 512, 256, 8, 100),
                (1, 2048, 512, 256, 8, -128)):
        assert L.moe_w4a16_workspace_size(*bad) == 0, bad
        assert _lib.last_error()
    assert L.moe_w4a16_workspace_size(4, 2048, 512, 256, 8, 512) > L.moe_w4a16_workspace_size(4, 2048, 512, 256, 8, 0)


def test_workspace_check_validation(L):
    """Host-side rejections of the time-out check (no GPU call is reached)."""
    assert L.moe_w4a16_workspace_check(None, 1 << 20, None) == _lib.W4A16_ERR_INVALID_ARG
    assert L.moe_w4a16_workspace_check(C.c_void_p(MISALIGNED), 1 << 20, None) == _lib.W4A16_ERR_INVALID_ARG
    assert L.moe_w4a16_workspace_check(C.c_void_p(FAKE), 100, None) == _lib.W4A16_ERR_WORKSPACE


def test_error_offset_matches_header():
    hdr = open(HEADER).read()
    m = re.search(r"#define W4A16_WORKSPACE_ERROR_OFFSET (\d+)", hdr)
    assert m and int(m.group(1)) == _lib.WORKSPACE_ERROR_OFFSET
    assert _lib.WORKSPACE_ERROR_OFFSET + 4 <= _lib.WORKSPACE_HEAD_BYTES


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


def test_binding_shape_checks_on_the_host():
    """The binding's shape rules (run before any call into the library), on meta tensors."""
    import torch
    import weight_only_int4_rtn_amd as w4
    m = dict(device="meta")
    E, H, I = 8, 256, 128
    good = (torch.empty((E, 2 * I, H // 8), dtype=torch.int32, **m), torch.empty((E, 2 * I, H // 128), **m),
            torch.empty((E, H, I // 8), dtype=torch.int32, **m), torch.empty((E, H, I // 128), **m))
    assert w4._check_experts(*good, 4, H) == (E, I)
    with pytest.raises(ValueError):
        w4._check_experts(*good, 8, H)                     # 8-bit codes need twice the words
    with pytest.raises(ValueError):
        w4._check_experts(*good, 4, H + 128)               # another hidden size
    with pytest.raises(ValueError):
        w4._check_experts(*good, 3, H)
    bad_s2 = torch.empty((E, H, 2), **m)
    with pytest.raises(ValueError):
        w4._check_experts(good[0], good[1], good[2], bad_s2, 4, H)
    with pytest.raises(ValueError):
        w4._shape(torch.empty((3, H), **m), "out", (4, H))
    w4._shape(None, "residual", (4, H))                  # absent optional tensors pass


@pytest.mark.parametrize("fn,args,expect", [
    ("fp8", (FAKE, 0, 1, 8, 254), _lib.W4A16_ERR_INVALID_ARG),          # cols % 4
    ("fp8", (FAKE, 3, 1, 8, 256), _lib.W4A16_ERR_INVALID_ARG),          # dtype
    ("fp8", (None, 0, 1, 8, 256), _lib.W4A16_ERR_INVALID_ARG),          # NULL w
    ("fp8", (MISALIGNED, 0, 1, 8, 256), _lib.W4A16_ERR_INVALID_ARG),
    ("fp8", (None, 0, 0, 8, 256), _lib.W4A16_OK),                       # nothing to do
    ("mx", (FAKE, 0, 1, 8, 48, 1), _lib.W4A16_ERR_INVALID_ARG),         # cols % 32
    ("mx", (FAKE, 0, 1, 8, 256, 2), _lib.W4A16_ERR_INVALID_ARG),        # method
    ("mx", (FAKE, 0, -1, 8, 256, 1), _lib.W4A16_ERR_INVALID_ARG),
    ("mx", (None, 1, 2, 0, 256, 0), _lib.W4A16_OK),
])
def test_format_quantizer_validation(L, fn, args, expect):
    if fn == "fp8":
        w, dt, n, r, c = args
        st = L.fp8_quantize_pack(w, dt, n, r, c, None if w is None else FAKE, None if w is None else FAKE, None)
    else:
        w, dt, n, r, c, m = args
        st = L.mxfp4_quantize_pack(w, dt, n, r, c, m, None if w is None else FAKE, None if w is None else FAKE, None)
    assert st == expect


@pytest.mark.parametrize("fmt,bits,expect", [(1, 4, _lib.W4A16_ERR_INVALID_ARG), (2, 8, _lib.W4A16_ERR_INVALID_ARG),
                                             (3, 4, _lib.W4A16_ERR_INVALID_ARG), (-1, 4, _lib.W4A16_ERR_INVALID_ARG)])
def test_forward_rejects_bad_weight_format(L, fmt, bits, expect):
    a = base_args(bits=bits)
    a.weight_format = fmt
    assert forward_status(L, a) == expect


def test_linear_validation(L):
    def args(T=4, K=2048, N=512, bits=8, fmt=0):
        a = _lib.LinearArgs()
        a.T, a.K, a.N, a.bits, a.group, a.weight_format = T, K, N, bits, 128, fmt
        a.x, a.w, a.s, a.y = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
        return a
    for kw, expect in ((dict(K=2000), _lib.W4A16_ERR_INVALID_ARG), (dict(N=100), _lib.W4A16_ERR_INVALID_ARG),
                       (dict(bits=5), _lib.W4A16_ERR_INVALID_ARG), (dict(fmt=1, bits=4), _lib.W4A16_ERR_INVALID_ARG),
                       (dict(K=16384), _lib.W4A16_ERR_UNSUPPORTED), (dict(T=-1), _lib.W4A16_ERR_INVALID_ARG)):
        assert L.w4a16_linear(C.byref(args(**kw)), None) == expect, kw
    a = args()
    need = L.w4a16_linear_workspace_size(4, 2048, 512)
    assert need > 0
    a.workspace, a.workspace_bytes = FAKE + 0x10000, need - 1
    assert L.w4a16_linear(C.byref(a), None) == _lib.W4A16_ERR_WORKSPACE
    a = args()
    a.y = a.x
    a.workspace, a.workspace_bytes = FAKE + 0x10000, need
    assert L.w4a16_linear(C.byref(a), None) == _lib.W4A16_ERR_INVALID_ARG
    assert L.w4a16_linear(C.byref(args(T=0)), None) == _lib.W4A16_OK
    assert L.w4a16_linear_workspace_size(1, 100, 512) == 0


def test_one_hip_runtime_whatever_the_import_order():
    """Loading the library before anything imports torch still maps a single HIP runtime
    (torch's): two runtimes in one process leave the library's own without the GPU."""
    code = ("import weight_only_int4_rtn_amd as w4\n"
            "w4._lib.lib()\n"
            "import torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    runtimes = ast.literal_eval(out.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes
