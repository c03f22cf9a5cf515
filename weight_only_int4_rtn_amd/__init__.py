"""W4A16 routed-expert MoE for MI355X (gfx950): Python binding of ``libw4a16.so``.

The functions here only marshal torch tensors into the C ABI of
``include/w4a16.h`` (pointers, sizes, the current HIP stream); every step of the
computation runs in the library's HIP kernels.  Tensors must be contiguous and on
the GPU.  bf16 data is passed as ``torch.bfloat16`` (or its bit pattern as
``torch.int16`` / ``torch.uint16``).  Every tensor's shape is checked against the
others before anything is enqueued (the C ABI sees raw pointers and cannot); a
mismatch raises ``ValueError``.

Streams: with ``stream=s`` every tensor the binding allocates (outputs, routing
tensors, a temporary workspace) is allocated and initialised on ``s`` itself, so it is
ordered before the kernels and returns to the caching allocator on that stream.
"""

from __future__ import annotations

import contextlib
import ctypes as C

from . import _lib
from ._lib import W4A16Error, MoeArgs  # noqa: F401

__all__ = ["stream_read", "rtn_quantize_pack", "fp8_quantize_pack", "mxfp4_quantize_pack", "moe_w4a16_forward", "moe_w4a16_forward_timed", "moe_w4a16_workspace_size",
           "moe_w4a16_workspace_init", "moe_w4a16_workspace_check", "new_workspace", "w4a16_linear",
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


def _on(stream):
    """Context in which allocations and torch work go to ``stream`` (None: unchanged)."""
    return _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_bits(bits, name="bits"):
    if bits not in (4, 8):
        raise ValueError(f"{name} = {bits}, must be 4 or 8")


def _check_experts(w13, s13, w2, s2, bits, H, fmt="int"):
    """Shapes of a routed-expert bank for code width ``bits``, hidden size ``H`` and
    weight format ``fmt`` (int / fp8 / mxfp4): returns (E, I)."""
    _check_bits(bits)
    if fmt not in _lib.FORMATS:
        raise ValueError(f"weight_format {fmt!r}: one of {tuple(_lib.FORMATS)}")
    if (fmt == "fp8" and bits != 8) or (fmt == "mxfp4" and bits != 4):
        raise ValueError(f"{fmt} experts have {8 if fmt == 'fp8' else 4}-bit codes, not {bits}")
    if w13.dim() != 3 or w2.dim() != 3:
        raise ValueError("w13 and w2 must be 3-D")
    E, twoI = w13.shape[0], w13.shape[1]
    if twoI % 2 or H % GROUP or (twoI // 2) % GROUP:
        raise ValueError(f"H = {H} and I = {twoI / 2} must be multiples of {GROUP}")
    I = twoI // 2
    _shape(w13, "w13", (E, 2 * I, H * bits // 32))
    _shape(w2, "w2", (E, H, I * bits // 32))
    if fmt == "int":
        _shape(s13, "s13", (E, 2 * I, H // GROUP))
        _shape(s2, "s2", (E, H, I // GROUP))
    elif fmt == "fp8":
        _shape(s13, "s13", (E, 2 * I))
        _shape(s2, "s2", (E, H))
    else:
        _shape(s13, "s13", (E, 2 * I, H // 32))
        _shape(s2, "s2", (E, H, I // 32))
    return E, I


def _scale_types(fmt):
    torch = _torch()
    return _bf16_types() if fmt == "int" else (torch.float32,) if fmt == "fp8" else (torch.uint8,)


def _check_shared(shared, H, dev):
    """Validates the shared-expert dict; returns (bits, intermediate size)."""
    torch = _torch()
    bf = _bf16_types()
    for name in ("w13", "s13", "w2", "s2", "bits"):
        if name not in shared:
            raise ValueError(f"shared.{name} is required")
    for name in ("w13", "s13", "w2", "s2"):
        _need(shared[name], "shared." + name, (torch.int32,) if name[0] == "w" else bf, dev)
    sb = shared["bits"]
    _check_bits(sb, "shared.bits")
    if shared["w13"].dim() != 2 or shared["w13"].shape[0] % (2 * GROUP):
        raise ValueError("shared.w13 must be [2 * shared_I, H * bits / 32] with shared_I a multiple of 128")
    sI = shared["w13"].shape[0] // 2
    _shape(shared["w13"], "shared.w13", (2 * sI, H * sb // 32))
    _shape(shared["s13"], "shared.s13", (2 * sI, H // GROUP))
    _shape(shared["w2"], "shared.w2", (H, sI * sb // 32))
    _shape(shared["s2"], "shared.s2", (H, sI // GROUP))
    return sb, sI


def rtn_quantize_pack(w, bits: int = 4, group: int = GROUP, packed=None, scales=None, stream=None):
    """Quantize ``w[..., rows, cols]`` (fp32 or bf16, on the GPU) with symmetric RTN.

    Returns ``(packed int32 [..., rows, cols*bits/32], scales bf16 [..., rows, cols/128])``.
    """
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16))
    if w.dim() < 2:
        raise ValueError("w must have at least 2 dims")
    _check_bits(bits)
    if group != GROUP:
        raise ValueError(f"group = {group}, only {GROUP} is supported")
    rows, cols = w.shape[-2], w.shape[-1]
    if cols % GROUP:
        raise ValueError(f"cols = {cols} is not a multiple of {GROUP}")
    n_mats = w.numel() // max(1, rows * cols) if rows * cols else 0
    lead = tuple(w.shape[:-1])
    with _on(stream):
        if packed is None:
            packed = torch.empty(lead + (cols * bits // 32,), dtype=torch.int32, device=w.device)
        if scales is None:
            scales = torch.empty(lead + (cols // group,), dtype=torch.bfloat16, device=w.device)
    _need(packed, "packed", (torch.int32,), w.device)
    _need(scales, "scales", _bf16_types(), w.device)
    _shape(packed, "packed", lead + (cols * bits // 32,))
    _shape(scales, "scales", lead + (cols // group,))
    dt = _lib.W4A16_F32 if w.dtype == torch.float32 else _lib.W4A16_BF16
    st = _lib.lib().rtn_quantize_pack(_ptr(w), dt, n_mats, rows, cols, bits, group, _ptr(packed), _ptr(scales),
                                      _stream(w.device, stream))
    _lib.check(st, "rtn_quantize_pack")
    return packed, scales


def _quantize_common(w, col_mult):
    torch = _torch()
    _need(w, "w", (torch.float32, torch.bfloat16))
    if w.dim() < 2:
        raise ValueError("w must have at least 2 dims")
    rows, cols = w.shape[-2], w.shape[-1]
    if cols % col_mult:
        raise ValueError(f"cols = {cols} is not a multiple of {col_mult}")
    n_mats = w.numel() // max(1, rows * cols) if rows * cols else 0
    dt = _lib.W4A16_F32 if w.dtype == torch.float32 else _lib.W4A16_BF16
    return rows, cols, n_mats, tuple(w.shape[:-1]), dt


def fp8_quantize_pack(w, packed=None, scales=None, stream=None):
    """Per-output-channel FP8 E4M3 of ``w[..., rows, cols]`` (fp32 or bf16, on the GPU).

    Returns ``(packed int32 [..., rows, cols/4], scales fp32 [..., rows])``.
    """
    torch = _torch()
    rows, cols, n_mats, lead, dt = _quantize_common(w, 4)
    with _on(stream):
        if packed is None:
            packed = torch.empty(lead + (cols // 4,), dtype=torch.int32, device=w.device)
        if scales is None:
            scales = torch.empty(lead, dtype=torch.float32, device=w.device)
    _need(packed, "packed", (torch.int32,), w.device)
    _need(scales, "scales", (torch.float32,), w.device)
    _shape(packed, "packed", lead + (cols // 4,))
    _shape(scales, "scales", lead)
    st = _lib.lib().fp8_quantize_pack(_ptr(w), dt, n_mats, rows, cols, _ptr(packed), _ptr(scales),
                                      _stream(w.device, stream))
    _lib.check(st, "fp8_quantize_pack")
    return packed, scales


def mxfp4_quantize_pack(w, method: str = "mse", packed=None, scales=None, stream=None):
    """MXFP4 of ``w[..., rows, cols]``: E2M1 codes and one E8M0 scale per 32 columns, the
    scale exponent by weight-MSE search (``mse``) or round-to-nearest (``rtn``).

    Returns ``(packed int32 [..., rows, cols/8], scales uint8 [..., rows, cols/32])``.
    """
    torch = _torch()
    if method not in _lib.MXFP4_METHODS:
        raise ValueError(f"method {method!r}: one of {tuple(_lib.MXFP4_METHODS)}")
    rows, cols, n_mats, lead, dt = _quantize_common(w, 32)
    with _on(stream):
        if packed is None:
            packed = torch.empty(lead + (cols // 8,), dtype=torch.int32, device=w.device)
        if scales is None:
            scales = torch.empty(lead + (cols // 32,), dtype=torch.uint8, device=w.device)
    _need(packed, "packed", (torch.int32,), w.device)
    _need(scales, "scales", (torch.uint8,), w.device)
    _shape(packed, "packed", lead + (cols // 8,))
    _shape(scales, "scales", lead + (cols // 32,))
    st = _lib.lib().mxfp4_quantize_pack(_ptr(w), dt, n_mats, rows, cols, _lib.MXFP4_METHODS[method], _ptr(packed),
                                        _ptr(scales), _stream(w.device, stream))
    _lib.check(st, "mxfp4_quantize_pack")
    return packed, scales


def _args(x, w13, s13, w2, s2, top_k, bits, router_logits, topk_ids, topk_w, shared, residual, out,
          counts, offsets, sorted_pairs, workspace, router_w=None, shared_gate_w=None, logits_out=None,
          gate_out=None, weight_format="int", cooperative=True):
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
    a.router_w, a.shared_gate_w = _ptr(router_w), _ptr(shared_gate_w)
    a.logits_out, a.shared_gate_out = _ptr(logits_out), _ptr(gate_out)
    a.weight_format = _lib.FORMATS[weight_format]
    a.flags = 0 if cooperative else _lib.W4A16_FLAG_NO_COOPERATIVE
    return a


def moe_w4a16_workspace_size(T: int, H: int, I: int, E: int, top_k: int, shared_bits: int = 0,
                             shared_I: int = 0) -> int:
    """Bytes of device workspace :func:`moe_w4a16_forward` needs for these shapes
    (``shared_I`` counts only when ``shared_bits`` is non-zero)."""
    n = _lib.lib().moe_w4a16_workspace_size(T, H, I, E, top_k, shared_I if shared_bits else 0)
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


def moe_w4a16_workspace_check(workspace, stream=None) -> bool:
    """Synchronise ``stream`` and report whether a single-launch wait timed out on this
    workspace since the last check (True: it did, and the head has been reset; the
    outputs of the forwards since then hold NaN rows).  Never raises for a time-out."""
    torch = _torch()
    _need(workspace, "workspace", (torch.uint8,))
    st = _lib.lib().moe_w4a16_workspace_check(C.c_void_p(workspace.data_ptr()), workspace.numel(),
                                              _stream(workspace.device, stream))
    if st == _lib.W4A16_ERR_TIMEOUT:
        return True
    _lib.check(st, "moe_w4a16_workspace_check")
    return False


def new_workspace(nbytes: int, device, stream=None):
    """A device workspace of ``nbytes`` bytes ready for :func:`moe_w4a16_forward`,
    allocated and initialised on ``stream`` (default: the current stream)."""
    torch = _torch()
    with _on(stream):
        ws = torch.empty((max(int(nbytes), _lib.WORKSPACE_HEAD_BYTES),), dtype=torch.uint8, device=device)
        return moe_w4a16_workspace_init(ws)


def moe_w4a16_forward(x, w13, s13, w2, s2, *, top_k: int, bits: int = 4, router_logits=None,
                      topk_ids=None, topk_w=None, shared=None, residual=None, out=None, workspace=None,
                      routing_out: bool = False, stream=None, router_w=None, shared_gate_w=None,
                      weight_format: str = "int", cooperative: bool = True, _timed=None):
    """One routed-expert MoE FFN on the GPU.

    ``x`` bf16 ``[T, H]``; ``w13`` int32 ``[E, 2I, H*bits/32]`` and ``s13`` bf16
    ``[E, 2I, H/128]`` (gate rows then up rows); ``w2`` int32 ``[E, H, I*bits/32]``,
    ``s2`` bf16 ``[E, H, I/128]``.  Either ``router_logits`` fp32 ``[T, E]`` or both
    ``topk_ids`` int32 and ``topk_w`` fp32 ``[T, top_k]``.  ``shared`` is an optional dict
    ``{w13, s13, w2, s2, bits}`` of one always-on expert.  Returns ``y`` bf16 ``[T, H]``,
    and with ``routing_out`` also a dict of the routing outputs (ids, w, counts, offsets,
    sorted_pairs).

    ``router_w`` bf16 ``[E, H]`` computes the logits from ``x`` (then ``router_logits``
    must be None); ``shared_gate_w`` bf16 ``[H]`` scales the shared expert's output per
    token by ``sigmoid(x . shared_gate_w)``.  With ``routing_out`` the routing dict then
    also holds ``logits`` fp32 ``[T, E]`` and ``shared_gate`` fp32 ``[T]``.

    ``weight_format`` ``fp8`` (bits 8) or ``mxfp4`` (bits 4) takes routed experts packed by
    :func:`fp8_quantize_pack` / :func:`mxfp4_quantize_pack`: ``s13``/``s2`` are then fp32
    ``[E, 2I]`` / ``[E, H]`` row scales, or uint8 E8M0 ``[E, 2I, H/32]`` / ``[E, H, I/32]``.

    ``cooperative=False`` keeps to launches whose workgroups never wait for each other
    (``W4A16_FLAG_NO_COOPERATIVE``; 1- and 2-token batches then skip the single-launch
    kernel): for callers that share the GPU with other work.
    """
    torch = _torch()
    bf = _bf16_types()
    _need(x, "x", bf)
    dev = x.device
    if weight_format not in _lib.FORMATS:
        raise ValueError(f"weight_format {weight_format!r}: one of {tuple(_lib.FORMATS)}")
    sdt = _scale_types(weight_format)
    for name, t, dt in (("w13", w13, (torch.int32,)), ("s13", s13, sdt), ("w2", w2, (torch.int32,)),
                        ("s2", s2, sdt)):
        _need(t, name, dt, dev)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [T, H]")
    T, H = x.shape
    E, I = _check_experts(w13, s13, w2, s2, bits, H, weight_format)
    if not 1 <= top_k <= E:
        raise ValueError(f"top_k = {top_k} not in [1, E = {E}]")
    if router_w is not None:
        if router_logits is not None:
            raise ValueError("router_w and router_logits are exclusive")
        _need(router_w, "router_w", bf, dev)
        _shape(router_w, "router_w", (E, H))
    elif router_logits is not None:
        _need(router_logits, "router_logits", (torch.float32,), dev)
        _shape(router_logits, "router_logits", (T, E))
    else:
        _need(topk_ids, "topk_ids", (torch.int32,), dev)
        _need(topk_w, "topk_w", (torch.float32,), dev)
        _shape(topk_ids, "topk_ids", (T, top_k))
        _shape(topk_w, "topk_w", (T, top_k))
    sb = sI = 0
    if shared is not None:
        sb, sI = _check_shared(shared, H, dev)
    if shared_gate_w is not None:
        if shared is None:
            raise ValueError("shared_gate_w needs a shared expert")
        _need(shared_gate_w, "shared_gate_w", bf, dev)
        _shape(shared_gate_w, "shared_gate_w", (H,))
    if residual is not None:
        _need(residual, "residual", bf, dev)
        _shape(residual, "residual", (T, H))
    if out is not None:
        _need(out, "out", bf, dev)
        _shape(out, "out", (T, H))
    need = moe_w4a16_workspace_size(T, H, I, E, top_k, sb, sI) if T > 0 else 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,), dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    routing = {}
    counts = offsets = sorted_pairs = logits_out = gate_out = None
    with _on(stream):   # everything allocated here is ordered before the kernels on `stream`
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        if routing_out:
            if router_w is not None:
                logits_out = torch.empty((T, E), dtype=torch.float32, device=dev)
            if shared_gate_w is not None:
                gate_out = torch.empty((T,), dtype=torch.float32, device=dev)
            if router_logits is not None or router_w is not None:
                topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
                topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
            counts = torch.empty((E,), dtype=torch.int32, device=dev)
            offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
            sorted_pairs = torch.empty((T * top_k,), dtype=torch.int32, device=dev)
            routing = dict(ids=topk_ids, w=topk_w, counts=counts, offsets=offsets, sorted_pairs=sorted_pairs)
            if logits_out is not None:
                routing["logits"] = logits_out
            if gate_out is not None:
                routing["shared_gate"] = gate_out
        if workspace is None:
            workspace = torch.zeros((max(need, 1),), dtype=torch.uint8, device=dev)   # zero head: see workspace_init
        a = _args(x, w13, s13, w2, s2, top_k, bits, router_logits, topk_ids, topk_w, shared, residual, out,
                  counts, offsets, sorted_pairs, workspace, router_w, shared_gate_w, logits_out, gate_out,
                  weight_format, cooperative)
        if _timed is None:
            st = _lib.lib().moe_w4a16_forward(C.byref(a), _stream(dev, None))
            _lib.check(st, "moe_w4a16_forward")
        else:
            n = C.c_int(0)
            ms = (C.c_float * 16)()
            names = (C.c_char_p * 16)()
            st = _lib.lib().moe_w4a16_forward_timed(C.byref(a), _stream(dev, None), 16, ms, names, C.byref(n))
            _lib.check(st, "moe_w4a16_forward_timed")
            _timed.extend((names[i].decode(), float(ms[i])) for i in range(n.value))
    return (out, routing) if routing_out else out


def w4a16_linear(x, w, s, *, bits: int = 8, weight_format: str = "int", residual=None, out=None, workspace=None,
                 stream=None):
    """Dense projection ``y = x . W^T (+ residual)`` with ``W`` packed ``[N, K*bits/32]``
    and its scales (INT: bf16 ``[N, K/128]``; fp8: fp32 ``[N]``; mxfp4: uint8 ``[N, K/32]``),
    on the expert down-projection kernels.  ``x`` bf16 ``[T, K]``; returns bf16 ``[T, N]``."""
    torch = _torch()
    bf = _bf16_types()
    _need(x, "x", bf)
    dev = x.device
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x and w must be 2-D")
    _check_bits(bits)
    if weight_format not in _lib.FORMATS:
        raise ValueError(f"weight_format {weight_format!r}: one of {tuple(_lib.FORMATS)}")
    T, K = x.shape
    N = w.shape[0]
    if K % GROUP or N % GROUP:
        raise ValueError(f"K = {K} and N = {N} must be multiples of {GROUP}")
    _need(w, "w", (torch.int32,), dev)
    _need(s, "s", _scale_types(weight_format), dev)
    _shape(w, "w", (N, K * bits // 32))
    _shape(s, "s", (N, K // GROUP) if weight_format == "int" else (N,) if weight_format == "fp8" else (N, K // 32))
    if residual is not None:
        _need(residual, "residual", bf, dev)
        _shape(residual, "residual", (T, N))
    if out is not None:
        _need(out, "out", bf, dev)
        _shape(out, "out", (T, N))
    need = _lib.lib().w4a16_linear_workspace_size(T, K, N) if T > 0 else 0
    if T > 0 and need == 0:
        raise W4A16Error(_lib.W4A16_ERR_INVALID_ARG, "w4a16_linear_workspace_size", _lib.last_error())
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,), dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    with _on(stream):
        if out is None:
            out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        a = _lib.LinearArgs()
        a.T, a.K, a.N = T, K, N
        a.bits, a.group, a.weight_format = bits, GROUP, _lib.FORMATS[weight_format]
        a.x, a.w, a.s, a.residual, a.y = _ptr(x), _ptr(w), _ptr(s), _ptr(residual), _ptr(out)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
        st = _lib.lib().w4a16_linear(C.byref(a), _stream(dev, None))
        _lib.check(st, "w4a16_linear")
    return out


def moe_w4a16_forward_timed(*args, **kwargs):
    """:func:`moe_w4a16_forward` that also returns ``[(kernel name, ms), ...]`` measured
    with HIP events around each kernel (synchronises the stream)."""
    timings = []
    res = moe_w4a16_forward(*args, _timed=timings, **kwargs)
    return res, timings


class MoeCall:
    """A prepared :func:`moe_w4a16_forward` for repeated calls with fixed shapes, weights
    and workspace (a decode loop): everything is validated once here, and each call
    checks only the per-call tensors' shapes and sets their pointers (activations,
    logits or ids, residual, output) before calling the library.
    """

    def __init__(self, x, w13, s13, w2, s2, *, top_k: int, bits: int = 4, shared=None, workspace=None,
                 stream=None, router_w=None, shared_gate_w=None, weight_format: str = "int",
                 cooperative: bool = True):
        torch = _torch()
        bf = _bf16_types()
        _need(x, "x", bf)
        dev = x.device
        if weight_format not in _lib.FORMATS:
            raise ValueError(f"weight_format {weight_format!r}: one of {tuple(_lib.FORMATS)}")
        sdt = _scale_types(weight_format)
        for name, t, dt in (("w13", w13, (torch.int32,)), ("s13", s13, sdt), ("w2", w2, (torch.int32,)),
                            ("s2", s2, sdt)):
            _need(t, name, dt, dev)
        if x.dim() != 2:
            raise ValueError("x must be 2-D [T, H]")
        self.T, self.H = x.shape
        self.E, I = _check_experts(w13, s13, w2, s2, bits, self.H, weight_format)
        if not 1 <= top_k <= self.E:
            raise ValueError(f"top_k = {top_k} not in [1, E = {self.E}]")
        self.top_k = top_k
        sb = sI = 0
        if shared is not None:
            sb, sI = _check_shared(shared, self.H, dev)
        if router_w is not None:
            _need(router_w, "router_w", bf, dev)
            _shape(router_w, "router_w", (self.E, self.H))
        if shared_gate_w is not None:
            if shared is None:
                raise ValueError("shared_gate_w needs a shared expert")
            _need(shared_gate_w, "shared_gate_w", bf, dev)
            _shape(shared_gate_w, "shared_gate_w", (self.H,))
        self.self_routed = router_w is not None
        need = moe_w4a16_workspace_size(self.T, self.H, I, self.E, top_k, sb, sI)
        if workspace is None:
            workspace = new_workspace(need, dev, stream)
        _need(workspace, "workspace", (torch.uint8,), dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace needs {need} bytes")
        self._keep = (w13, s13, w2, s2, shared, workspace, router_w, shared_gate_w)
        self.workspace = workspace
        self.args = _args(x, w13, s13, w2, s2, top_k, bits, None, None, None, shared, None, None, None, None, None,
                          workspace, router_w, shared_gate_w, weight_format=weight_format,
                          cooperative=cooperative)
        self.device = dev
        self.stream = None if stream is None else _stream(dev, stream)   # None: the current stream per call
        self._fn = _lib.lib().moe_w4a16_forward
        self._ref = C.byref(self.args)
        self._th = (self.T, self.H)
        self._tk = (self.T, self.top_k)
        self._te = (self.T, self.E)

    def __call__(self, x, out, router_logits=None, topk_ids=None, topk_w=None, residual=None):
        torch = _torch()
        if (x.shape != self._th or out.shape != self._th or x.element_size() != 2 or out.element_size() != 2
                or not (x.is_contiguous() and out.is_contiguous())):
            raise ValueError(f"x and out must be contiguous 16-bit {self._th}")
        if self.self_routed:
            if router_logits is not None or topk_ids is not None:
                raise ValueError("this call computes its logits from x (router_w): pass no logits or ids")
        elif router_logits is not None:
            if router_logits.shape != self._te or router_logits.dtype != torch.float32:
                raise ValueError(f"router_logits must be fp32 {self._te}")
        elif (topk_ids is None or topk_w is None or topk_ids.shape != self._tk or topk_w.shape != self._tk
              or topk_ids.dtype != torch.int32 or topk_w.dtype != torch.float32):
            raise ValueError(f"topk_ids (int32) and topk_w (fp32) must be {self._tk} when router_logits is None")
        if residual is not None and (residual.shape != self._th or residual.element_size() != 2):
            raise ValueError(f"residual must be 16-bit {self._th}")
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


def stream_read(buf, sink, stream=None) -> None:
    """A plain streaming read of ``buf`` (a contiguous device tensor of a multiple of 16
    bytes): the XOR of its 32-bit words is XOR-ed into ``sink`` (one int32 on the same
    device).  The measurement aid ``w4a16_stream_read``."""
    if not (buf.is_cuda and sink.is_cuda and buf.device == sink.device):
        raise ValueError("stream_read: buf and sink must be tensors on one GPU")
    if not buf.is_contiguous() or sink.dtype != _torch().int32 or sink.numel() != 1:
        raise ValueError("stream_read: contiguous buf and a one-element int32 sink")
    nbytes = buf.numel() * buf.element_size()
    st = _lib.lib().w4a16_stream_read(C.c_void_p(buf.data_ptr()), nbytes, C.c_void_p(sink.data_ptr()),
                                      _stream(buf.device, stream))
    _lib.check(st, "w4a16_stream_read")
