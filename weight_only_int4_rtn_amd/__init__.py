"""W4A16 routed-expert MoE for MI355X (gfx950): Python binding of ``libw4a16.so``.

The functions here only marshal torch tensors into the C ABI of
``include/w4a16.h`` (pointers, sizes, the current HIP stream); every step of the
computation runs in the library's HIP kernels.  Tensors must be contiguous and on
the GPU.  bf16 data is passed as ``torch.bfloat16`` (or its bit pattern as
``torch.int16`` / ``torch.uint16``).
"""

from __future__ import annotations

import ctypes as C

from . import _lib
from ._lib import W4A16Error, MoeArgs  # noqa: F401

__all__ = ["rtn_quantize_pack", "moe_w4a16_forward", "moe_w4a16_forward_timed", "moe_w4a16_workspace_size",
           "moe_w4a16_workspace_init", "new_workspace",
           "MoeCall", "w4a16_abi_version", "W4A16Error", "library_path"]

GROUP = 128


def library_path() -> str:
    return _lib.LIB_PATH


def w4a16_abi_version() -> int:
    return _lib.lib().w4a16_abi_version()


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _need(t, name, dtypes, device=None):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16) + ((torch.uint16,) if hasattr(torch, "uint16") else ())


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def rtn_quantize_pack(w, bits: int = 4, group: int = GROUP, packed=None, scales=None, stream=None):
    """Quantize ``w[..., rows, cols]`` (fp32 or bf16, on the GPU) with symmetric RTN.

    Returns ``(packed int32 [..., rows, cols*bits/32], scales bf16 [..., rows, cols/128])``.
    """
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16))
    if w.dim() < 2:
        raise ValueError("w must have at least 2 dims")
    rows, cols = w.shape[-2], w.shape[-1]
    n_mats = w.numel() // max(1, rows * cols) if rows * cols else 0
    lead = tuple(w.shape[:-1])
    if packed is None:
        packed = torch.empty(lead + (cols * bits // 32,), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty(lead + (cols // group if group else 0,), dtype=torch.bfloat16, device=w.device)
    _need(packed, "packed", (torch.int32,), w.device)
    _need(scales, "scales", _bf16_types(), w.device)
    dt = _lib.W4A16_F32 if w.dtype == torch.float32 else _lib.W4A16_BF16
    st = _lib.lib().rtn_quantize_pack(_ptr(w), dt, n_mats, rows, cols, bits, group, _ptr(packed), _ptr(scales),
                                      _stream(w.device, stream))
    _lib.check(st, "rtn_quantize_pack")
    return packed, scales


def _args(x, w13, s13, w2, s2, top_k, bits, router_logits, topk_ids, topk_w, shared, residual, out,
          counts, offsets, sorted_pairs, workspace):
    a = MoeArgs()
    T, H = x.shape
    E, twoI = w13.shape[0], w13.shape[1]
    a.T, a.H, a.I, a.E, a.top_k = T, H, twoI // 2, E, top_k
    a.bits, a.group = bits, GROUP
    a.x, a.router_logits = _ptr(x), _ptr(router_logits)
    a.w13, a.s13, a.w2, a.s2 = _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2)
    if shared is not None:
        a.shared_bits = shared["bits"]
        a.shared_I = shared["w13"].shape[0] // 2
        a.shared_w13, a.shared_s13 = _ptr(shared["w13"]), _ptr(shared["s13"])
        a.shared_w2, a.shared_s2 = _ptr(shared["w2"]), _ptr(shared["s2"])
    a.residual, a.y = _ptr(residual), _ptr(out)
    a.topk_ids, a.topk_w = _ptr(topk_ids), _ptr(topk_w)
    a.expert_counts, a.expert_offsets, a.sorted_pairs = _ptr(counts), _ptr(offsets), _ptr(sorted_pairs)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def moe_w4a16_workspace_size(T: int, H: int, I: int, E: int, top_k: int, shared_bits: int = 0,
                             shared_I: int = 0) -> int:
    """Bytes of device workspace :func:`moe_w4a16_forward` needs for these shapes."""
    a = MoeArgs()
    a.T, a.H, a.I, a.E, a.top_k, a.bits, a.group = T, H, I, E, top_k, 4, GROUP
    a.shared_bits, a.shared_I = shared_bits, shared_I
    n = _lib.lib().moe_w4a16_workspace_size(C.byref(a))
    if n == 0:
        raise W4A16Error(_lib.W4A16_ERR_INVALID_ARG, "moe_w4a16_workspace_size", _lib.last_error())
    return n


def moe_w4a16_workspace_init(workspace, stream=None):
    """Zero the head of a workspace (once, before its first forward; a zero-filled
    allocation needs nothing).  ``workspace`` is a uint8 device tensor."""
    torch = _torch()
    _need(workspace, "workspace", (torch.uint8,))
    st = _lib.lib().moe_w4a16_workspace_init(C.c_void_p(workspace.data_ptr()), workspace.numel(),
                                             _stream(workspace.device, stream))
    _lib.check(st, "moe_w4a16_workspace_init")
    return workspace


def new_workspace(nbytes: int, device):
    """A device workspace of ``nbytes`` bytes ready for :func:`moe_w4a16_forward`."""
    torch = _torch()
    return moe_w4a16_workspace_init(torch.empty((max(int(nbytes), _lib.WORKSPACE_HEAD_BYTES),), dtype=torch.uint8,
                                                device=device))


def moe_w4a16_forward(x, w13, s13, w2, s2, *, top_k: int, bits: int = 4, router_logits=None,
                      topk_ids=None, topk_w=None, shared=None, residual=None, out=None, workspace=None,
                      routing_out: bool = False, stream=None, _timed=None):
    """One routed-expert MoE FFN on the GPU.

    ``x`` bf16 ``[T, H]``; ``w13`` int32 ``[E, 2I, H*bits/32]`` and ``s13`` bf16
    ``[E, 2I, H/128]`` (gate rows then up rows); ``w2`` int32 ``[E, H, I*bits/32]``,
    ``s2`` bf16 ``[E, H, I/128]``.  Either ``router_logits`` fp32 ``[T, E]`` or both
    ``topk_ids`` int32 and ``topk_w`` fp32 ``[T, top_k]``.  ``shared`` is an optional dict
    ``{w13, s13, w2, s2, bits}`` of one always-on expert.  Returns ``y`` bf16 ``[T, H]``,
    and with ``routing_out`` also a dict of the routing outputs (ids, w, counts, offsets,
    sorted_pairs).
    """
    torch = _torch()
    bf = _bf16_types()
    _need(x, "x", bf)
    dev = x.device
    for name, t, dt in (("w13", w13, (torch.int32,)), ("s13", s13, bf), ("w2", w2, (torch.int32,)),
                        ("s2", s2, bf)):
        _need(t, name, dt, dev)
    if x.dim() != 2 or w13.dim() != 3 or w2.dim() != 3:
        raise ValueError("x must be 2-D and w13, w2 3-D")
    T, H = x.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    if router_logits is not None:
        _need(router_logits, "router_logits", (torch.float32,), dev)
        if tuple(router_logits.shape) != (T, E):
            raise ValueError("router_logits must be [T, E]")
    else:
        _need(topk_ids, "topk_ids", (torch.int32,), dev)
        _need(topk_w, "topk_w", (torch.float32,), dev)
    if shared is not None:
        for name in ("w13", "s13", "w2", "s2"):
            _need(shared[name], "shared." + name, (torch.int32,) if name[0] == "w" else bf, dev)
    if residual is not None:
        _need(residual, "residual", bf, dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", bf, dev)
    routing = {}
    counts = offsets = sorted_pairs = None
    if routing_out:
        if router_logits is not None:
            topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
            topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
        counts = torch.empty((E,), dtype=torch.int32, device=dev)
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        sorted_pairs = torch.empty((T * top_k,), dtype=torch.int32, device=dev)
        routing = dict(ids=topk_ids, w=topk_w, counts=counts, offsets=offsets, sorted_pairs=sorted_pairs)
    if workspace is None:
        sb = shared["bits"] if shared is not None else 0
        sI = shared["w13"].shape[0] // 2 if shared is not None else 0
        n = moe_w4a16_workspace_size(T, H, I, E, top_k, sb, sI) if T > 0 else 0
        workspace = torch.zeros((max(n, 1),), dtype=torch.uint8, device=dev)   # zero head: see workspace_init
    a = _args(x, w13, s13, w2, s2, top_k, bits, router_logits, topk_ids, topk_w, shared, residual, out,
              counts, offsets, sorted_pairs, workspace)
    if _timed is None:
        st = _lib.lib().moe_w4a16_forward(C.byref(a), _stream(dev, stream))
        _lib.check(st, "moe_w4a16_forward")
    else:
        n = C.c_int(0)
        ms = (C.c_float * 16)()
        names = (C.c_char_p * 16)()
        st = _lib.lib().moe_w4a16_forward_timed(C.byref(a), _stream(dev, stream), 16, ms, names, C.byref(n))
        _lib.check(st, "moe_w4a16_forward_timed")
        _timed.extend((names[i].decode(), float(ms[i])) for i in range(n.value))
    return (out, routing) if routing_out else out


def moe_w4a16_forward_timed(*args, **kwargs):
    """:func:`moe_w4a16_forward` that also returns ``[(kernel name, ms), ...]`` measured
    with HIP events around each kernel (synchronises the stream)."""
    timings = []
    res = moe_w4a16_forward(*args, _timed=timings, **kwargs)
    return res, timings


class MoeCall:
    """A prepared :func:`moe_w4a16_forward` for repeated calls with fixed shapes, weights
    and workspace (a decode loop): everything is validated once here, and each call
    only sets the per-call pointers (activations, logits, residual, output) before
    calling the library.  Tensors passed per call must have the shapes, dtypes and
    device given at construction.
    """

    def __init__(self, x, w13, s13, w2, s2, *, top_k: int, bits: int = 4, shared=None, workspace=None,
                 stream=None):
        torch = _torch()
        bf = _bf16_types()
        _need(x, "x", bf)
        dev = x.device
        for name, t, dt in (("w13", w13, (torch.int32,)), ("s13", s13, bf), ("w2", w2, (torch.int32,)),
                            ("s2", s2, bf)):
            _need(t, name, dt, dev)
        self.T, self.H = x.shape
        self.E, self.top_k = w13.shape[0], top_k
        sb = shared["bits"] if shared is not None else 0
        sI = shared["w13"].shape[0] // 2 if shared is not None else 0
        if shared is not None:
            for name in ("w13", "s13", "w2", "s2"):
                _need(shared[name], "shared." + name, (torch.int32,) if name[0] == "w" else bf, dev)
        need = moe_w4a16_workspace_size(self.T, self.H, w13.shape[1] // 2, self.E, top_k, sb, sI)
        if workspace is None:
            workspace = new_workspace(need, dev)
        _need(workspace, "workspace", (torch.uint8,), dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace needs {need} bytes")
        self._keep = (w13, s13, w2, s2, shared, workspace)
        self.args = _args(x, w13, s13, w2, s2, top_k, bits, None, None, None, shared, None, None, None, None, None,
                          workspace)
        self.device = dev
        self.stream = None if stream is None else _stream(dev, stream)   # None: the current stream per call
        self._fn = _lib.lib().moe_w4a16_forward
        self._ref = C.byref(self.args)

    def __call__(self, x, out, router_logits=None, topk_ids=None, topk_w=None, residual=None):
        a = self.args
        a.x = x.data_ptr()
        a.y = out.data_ptr()
        a.router_logits = None if router_logits is None else router_logits.data_ptr()
        a.topk_ids = None if topk_ids is None else topk_ids.data_ptr()
        a.topk_w = None if topk_w is None else topk_w.data_ptr()
        a.residual = None if residual is None else residual.data_ptr()
        st = self._fn(self._ref, self.stream if self.stream is not None else
                      C.c_void_p(_torch().cuda.current_stream(self.device).cuda_stream))
        if st:
            _lib.check(st, "moe_w4a16_forward")
        return out
