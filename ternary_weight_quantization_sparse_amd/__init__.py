"""Sherry 1.25-bit ternary linear layer for MI355X (gfx950).

Thin Python binding over libsherry (include/sherry.h).  Functions take torch
CUDA (HIP) tensors, allocate outputs and workspaces with torch, and pass raw
device pointers plus the current stream to the C ABI.  Every step of the
computation runs in the library's HIP kernels.

The method: "Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
Fine-grained Sparsification" (3:4 ternary blocks, 5-bit codes, Sparse-AbsMean
scales) and the SherryNMQuant / SherryLinear listings of "Sherry, Tequila and
Fairies in Python", section 1.1.
"""

from __future__ import annotations

from dataclasses import dataclass

from . import _lib
from ._lib import SherryError, check, load  # noqa: F401

__all__ = [
    "PackedWeight", "quantize_pack", "unpack", "gemv", "gemm", "packed_bytes", "num_scales",
    "workspace_bytes", "SherryError", "load", "fake_quant", "fake_quant_ste", "gemv_batched",
    "FusedWeight", "quantize_pack_fused", "gemv_fused", "arenas_lambda", "arenas_gemm",
    "compare_repack", "compare_gemv", "gemm_fused", "quantize_pack_noalloc",
]


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on_stream(stream):
    """Context in which the binding allocates its temporaries: the caller's
    stream when one is given, so the caching allocator never hands a
    workspace or a copy to another stream while the kernels still use it."""
    import contextlib
    return _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _gran(granularity) -> int:
    if isinstance(granularity, int):
        return granularity
    try:
        return _lib.GRANULARITY[granularity]
    except KeyError:
        raise ValueError(f"unsupported granularity: {granularity!r}") from None


def _need_gpu(t, name, device=None):
    """Every tensor handed to the library must live on the GPU (and on the
    same one as the weight): the kernels dereference its address."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_out(t, name, dtype, numel, device):
    """A caller-supplied output: right dtype and device, contiguous, at least
    ``numel`` elements (the library cannot see buffer sizes)."""
    _need_gpu(t, name, device)
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")


def _check_pw(pw):
    """Packed planes and scales of the sizes their shape implies."""
    torch = _torch()
    _need_gpu(pw.packed, "packed")
    _need_gpu(pw.alpha, "alpha", pw.packed.device)
    lib = load()
    nbytes = int(lib.sherry_packed_bytes(pw.n, pw.k))
    nsc = int(lib.sherry_num_scales(pw.n, pw.k, _gran(pw.granularity), pw.group_size))
    if pw.packed.dtype != torch.uint8 or not pw.packed.is_contiguous() or pw.packed.numel() < nbytes:
        raise ValueError(f"packed must be a contiguous uint8 tensor of {nbytes} bytes")
    if pw.alpha.dtype != torch.float32 or not pw.alpha.is_contiguous() or pw.alpha.numel() < max(nsc, 0):
        raise ValueError(f"alpha must be a contiguous float32 tensor of {nsc} scales")


def _activations(x, k, device, rank=2):
    """bf16 activations [rows, K] on the weight's device (a copy only if x is
    not contiguous)."""
    torch = _torch()
    _need_gpu(x, "x", device)
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    if x.dim() != rank or x.shape[-1] != k:
        raise ValueError(f"x must be [rows, {k}], got {tuple(x.shape)}")
    return x.contiguous()


def packed_bytes(n: int, k: int) -> int:
    return int(load().sherry_packed_bytes(n, k))


def num_scales(n: int, k: int, granularity="per_group", group_size: int = 128) -> int:
    return int(load().sherry_num_scales(n, k, _gran(granularity), group_size))


def workspace_bytes(op: int, n: int, k: int, granularity="per_group", group_size: int = 128,
                    batch_or_m: int = 1, count: int = 1) -> int:
    v = int(load().sherry_workspace_bytes(op, n, k, _gran(granularity), group_size, batch_or_m, count))
    if v == (1 << 64) - 1:
        raise ValueError("invalid arguments for sherry_workspace_bytes")
    return v


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    torch = _torch()
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class PackedWeight:
    """Packed planes + scales of one [N, K] weight (the offline artifact)."""
    packed: object          # torch.uint8 [N*K*5/32]
    alpha: object           # torch.float32 [num_scales]
    n: int
    k: int
    granularity: str = "per_group"
    group_size: int = 128


def quantize_pack(w, granularity: str = "per_group", group_size: int = 128, stream=None) -> PackedWeight:
    """Sparse-AbsMean quantize + pack of a latent weight ``w`` [N, K] (fp32 or
    bf16, CUDA)."""
    torch = _torch()
    if w.dim() != 2:
        raise ValueError("Sherry quantization expects a 2-D weight")
    _need_gpu(w, "w")
    n, k = w.shape
    gran = _gran(granularity)
    dtype = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}.get(w.dtype)
    if dtype is None:
        raise ValueError("w must be float32 or bfloat16")
    lib = load()
    nbytes = int(lib.sherry_packed_bytes(n, k))
    nsc = int(lib.sherry_num_scales(n, k, gran, group_size))
    ws_bytes = int(lib.sherry_workspace_bytes(_lib.OP_QUANTIZE_PACK, n, k, gran, group_size, 1, 1))
    with _on_stream(stream):
        w = w.contiguous()
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
        alpha = torch.empty(max(nsc, 1), dtype=torch.float32, device=w.device)
        ws = _workspace(ws_bytes if ws_bytes != (1 << 64) - 1 else 0, w.device)
        check(lib.sherry_quantize_pack(n, k, gran, group_size, _ptr(w), dtype, _ptr(packed), _ptr(alpha),
                                       _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return PackedWeight(packed[:nbytes], alpha[:nsc], n, k, granularity, group_size)


def quantize_pack_noalloc(w, packed, alpha, granularity: str = "per_group", group_size: int = 128,
                          stream=None) -> PackedWeight:
    """quantize_pack into caller-provided ``packed`` (uint8, packed_bytes)
    and ``alpha`` (float32, num_scales) through the library's allocation-free
    entry point: no memory is allocated (the workspace is the library's static
    device buffer), so the call can run under HIP graph capture.  ``w`` must
    be contiguous.  Calls that overlap on one device race on that buffer."""
    torch = _torch()
    if w.dim() != 2:
        raise ValueError("Sherry quantization expects a 2-D weight")
    _need_gpu(w, "w")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous (no copy is made)")
    n, k = w.shape
    gran = _gran(granularity)
    dtype = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}.get(w.dtype)
    if dtype is None:
        raise ValueError("w must be float32 or bfloat16")
    lib = load()
    nbytes = int(lib.sherry_packed_bytes(n, k))
    nsc = int(lib.sherry_num_scales(n, k, gran, group_size))
    _need_out(packed, "packed", torch.uint8, nbytes, w.device)
    _need_out(alpha, "alpha", torch.float32, nsc, w.device)
    with torch.cuda.device(w.device):
        check(lib.sherry_quantize_pack_noalloc(n, k, gran, group_size, _ptr(w), dtype, _ptr(packed), _ptr(alpha),
                                               _stream(stream)))
    return PackedWeight(packed[:nbytes], alpha[:nsc], n, k, granularity, group_size)


def fake_quant(w, granularity: str = "per_group", group_size: int = 128, out_dtype=None, stream=None):
    """Quantize -> dequantize forward of a latent weight ``w`` [N, K] (fp32 or
    bf16, CUDA): returns (T*alpha dense [N, K], alpha).  ``out_dtype`` defaults
    to w's dtype (fp32 exact, bf16 rounded to nearest even)."""
    torch = _torch()
    if w.dim() != 2:
        raise ValueError("Sherry quantization expects a 2-D weight")
    _need_gpu(w, "w")
    n, k = w.shape
    gran = _gran(granularity)
    dtype = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}.get(w.dtype)
    if dtype is None:
        raise ValueError("w must be float32 or bfloat16")
    odt = w.dtype if out_dtype is None else out_dtype
    ocode = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}.get(odt)
    if ocode is None:
        raise ValueError("out_dtype must be float32 or bfloat16")
    lib = load()
    nsc = int(lib.sherry_num_scales(n, k, gran, group_size))
    ws_bytes = int(lib.sherry_workspace_bytes(_lib.OP_FAKE_QUANT, n, k, gran, group_size, 1, 1))
    with _on_stream(stream):
        w = w.contiguous()
        out = torch.empty((n, k), dtype=odt, device=w.device)
        alpha = torch.empty(max(nsc, 1), dtype=torch.float32, device=w.device)
        ws = _workspace(ws_bytes if ws_bytes != (1 << 64) - 1 else 0, w.device)
        check(lib.sherry_fake_quant(n, k, gran, group_size, _ptr(w), dtype, _ptr(out), ocode, _ptr(alpha),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out, alpha[:nsc]


def _make_ste():
    torch = _torch()

    class SherryFakeQuantSTE(torch.autograd.Function):
        """Forward: T*alpha from the latent weight (one fused kernel for
        per_group 128).  Backward: the straight-through estimator -- the
        gradient of the dequantized weight is passed to the latent weight
        unchanged ("Sherry, Tequila and Fairies in Python", section 1.1,
        SherryNMQuant.backward)."""

        @staticmethod
        def forward(ctx, w, granularity="per_group", group_size=128):
            out, _ = fake_quant(w, granularity, group_size)
            return out

        @staticmethod
        def backward(ctx, grad_out):
            return grad_out, None, None

    return SherryFakeQuantSTE


_STE = None


def fake_quant_ste(w, granularity: str = "per_group", group_size: int = 128):
    """Differentiable fake quantization for quantization-aware training:
    forward T*alpha, backward identity (straight-through)."""
    global _STE
    if _STE is None:
        _STE = _make_ste()
    return _STE.apply(w, granularity, group_size)


def unpack(pw: PackedWeight, out_dtype="int8", stream=None):
    """Decode to int8 T, fp32 T*alpha or bf16 RNE(T*alpha), [N, K]."""
    torch = _torch()
    tdt, code = {"int8": (torch.int8, _lib.I8), "float32": (torch.float32, _lib.F32),
                 "bfloat16": (torch.bfloat16, _lib.BF16)}[str(out_dtype).replace("torch.", "")]
    _check_pw(pw)
    with _on_stream(stream):
        out = torch.empty((pw.n, pw.k), dtype=tdt, device=pw.packed.device)
        check(load().sherry_unpack(pw.n, pw.k, _gran(pw.granularity), pw.group_size, _ptr(pw.packed),
                                   _ptr(pw.alpha), _ptr(out), code, _stream(stream)))
    return out


_Y_DTYPES = {"bfloat16": _lib.BF16, "float32": _lib.F32}


def _y_dtype(y_dtype):
    torch = _torch()
    key = str(y_dtype).replace("torch.", "")
    if key not in _Y_DTYPES:
        raise ValueError("y_dtype must be bfloat16 or float32")
    return getattr(torch, key), _Y_DTYPES[key]


def gemv(pw: PackedWeight, x, y_dtype="bfloat16", stream=None, out=None):
    """y = x @ (T*alpha)^T for a decode batch ``x`` [B, K] bf16 (B = 1..16)."""
    torch = _torch()
    _check_pw(pw)
    dev = pw.packed.device
    if x.dim() == 1:
        x = x.unsqueeze(0)
    ydt, code = _y_dtype(y_dtype)
    gran = _gran(pw.granularity)
    lib = load()
    with _on_stream(stream):
        x = _activations(x, pw.k, dev)
        b = x.shape[0]
        if out is not None:
            _need_out(out, "out", ydt, b * pw.n, dev)
        y = out if out is not None else torch.empty((b, pw.n), dtype=ydt, device=dev)
        ws_bytes = int(lib.sherry_workspace_bytes(_lib.OP_GEMV, pw.n, pw.k, gran, pw.group_size, b, 1))
        ws = _workspace(ws_bytes if ws_bytes != (1 << 64) - 1 else 0, dev)
        check(lib.sherry_gemv(pw.n, pw.k, gran, pw.group_size, _ptr(pw.packed), _ptr(pw.alpha), _ptr(x), b,
                              _ptr(y), code, 1, 0, 0, 0, _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(stream)))
    return y


def arenas_lambda(step: int, total_steps: int, lambda0: float) -> float:
    """Cosine-annealed residual weight of the Arenas forward (lambda0 at step
    0, 0 at ``total_steps`` and after), computed by the library's
    ``sherry_arenas_lambda``."""
    return float(load().sherry_arenas_lambda(int(step), int(total_steps), float(lambda0)))


def arenas_gemm(pw: PackedWeight, w, lam: float, x, stream=None, out=None):
    """Arenas training forward Y = X (T*alpha)^T + lam * X W^T for prefill
    activations ``x`` [M, K] bf16 and the latent weight ``w`` [N, K] (bf16;
    an fp32 master weight is rounded to bf16 here) -> [M, N] bf16."""
    torch = _torch()
    _check_pw(pw)
    dev = pw.packed.device
    if tuple(w.shape) != (pw.n, pw.k):
        raise ValueError("w must be [N, K] of the packed weight")
    _need_gpu(w, "w", dev)
    gran = _gran(pw.granularity)
    lib = load()
    with _on_stream(stream):
        x = _activations(x, pw.k, dev)
        wb = w.to(torch.bfloat16).contiguous()
        m = x.shape[0]
        if out is not None:
            _need_out(out, "out", torch.bfloat16, m * pw.n, dev)
        y = out if out is not None else torch.empty((m, pw.n), dtype=torch.bfloat16, device=dev)
        ws_bytes = int(lib.sherry_workspace_bytes(_lib.OP_ARENAS_GEMM, pw.n, pw.k, gran, pw.group_size, m, 1))
        ws = _workspace(ws_bytes if ws_bytes != (1 << 64) - 1 else 0, dev)
        check(lib.sherry_arenas_gemm(pw.n, pw.k, gran, pw.group_size, _ptr(pw.packed), _ptr(pw.alpha), _ptr(wb),
                                     float(lam), _ptr(x), m, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(stream)))
    return y


def compare_repack(pw: PackedWeight, fmt: int, stream=None):
    """Re-encode a packed weight as padded 2-bit (fmt 0) or three weights in 5
    bits (fmt 1): the comparison packings of the same ternary matrix."""
    torch = _torch()
    _check_pw(pw)
    lib = load()
    nbytes = int(lib.sherry_compare_bytes(fmt, pw.n, pw.k))
    if nbytes == 0:
        raise ValueError("invalid comparison format or shape")
    with _on_stream(stream):
        out = torch.empty(nbytes, dtype=torch.uint8, device=pw.packed.device)
        check(lib.sherry_compare_repack(fmt, pw.n, pw.k, _ptr(pw.packed), _ptr(out), _stream(stream)))
    return out


def compare_gemv(fmt: int, planes, alpha, n: int, k: int, x, count: int = 1, planes_stride: int = 0,
                 alpha_stride: int = 0, y=None, y_stride: int = 0, stream=None):
    """Batch-1 GEMV over a comparison packing with per-channel scales."""
    torch = _torch()
    lib = load()
    nbytes = int(lib.sherry_compare_bytes(fmt, n, k))
    if nbytes == 0:
        raise ValueError("invalid comparison format or shape")
    if count < 1:
        raise ValueError("count must be >= 1")
    _need_out(planes, "planes", torch.uint8, (count - 1) * planes_stride + nbytes, planes.device)
    dev = planes.device
    _need_out(alpha, "alpha", torch.float32, (count - 1) * alpha_stride + n, dev)
    if x.dim() == 2:
        x = x.reshape(-1)
    with _on_stream(stream):
        x = _activations(x, k, dev, rank=1)
        if y is None:
            y = torch.empty((count, n), dtype=torch.bfloat16, device=dev)
            y_stride = n
        else:
            _need_out(y, "y", torch.bfloat16, (count - 1) * y_stride + n, dev)
        check(lib.sherry_compare_gemv(fmt, n, k, _ptr(planes), _ptr(alpha), _ptr(x), _ptr(y), count,
                                      planes_stride, alpha_stride, y_stride, _stream(stream)))
    return y


@dataclass
class FusedWeight:
    """Several linears that read the same activations (q/k/v, gate/up) packed
    as one weight of their stacked rows, so one GEMV launch -- and one set of
    activation tables per workgroup -- serves all of them."""
    pw: PackedWeight
    sizes: tuple            # rows of each member, in order


def quantize_pack_fused(weights, granularity: str = "per_group", group_size: int = 128,
                        stream=None) -> FusedWeight:
    """Pack [N_i, K] latent weights as one [sum N_i, K] weight.  The scales of
    per_group / per_channel are row-local, so every member gets exactly the
    codes and scales of packing it alone; per_tensor would share one scale
    across the members (a different model) and is refused."""
    torch = _torch()
    if str(granularity) == "per_tensor" or _gran(granularity) == _lib.PER_TENSOR:
        raise ValueError("fused packing needs row-local scales (per_group or per_channel)")
    ks = {int(w.shape[1]) for w in weights}
    if len(ks) != 1:
        raise ValueError("fused members must share K")
    with _on_stream(stream):
        w = torch.cat([t.contiguous() for t in weights], dim=0)
    pw = quantize_pack(w, granularity, group_size, stream)
    return FusedWeight(pw, tuple(int(t.shape[0]) for t in weights))


def gemv_fused(fw: FusedWeight, x, y_dtype="bfloat16", stream=None, out=None):
    """One launch for all members; returns one [B, N_i] view per member."""
    y = gemv(fw.pw, x, y_dtype, stream, out)
    return list(y.split(list(fw.sizes), dim=1))


def gemm_fused(fw: FusedWeight, x, stream=None, out=None):
    """Prefill product for all members in one launch; one [M, N_i] view per member."""
    y = gemm(fw.pw, x, stream, out)
    return list(y.split(list(fw.sizes), dim=1))


def gemv_batched(packed_all, alpha_all, n: int, k: int, x, count: int, packed_stride: int,
                 alpha_stride: int, granularity="per_group", group_size: int = 128,
                 y_dtype="bfloat16", y=None, y_stride=None, ws=None, stream=None):
    """One launch over ``count`` same-shape packed matrices that share ``x``:
    matrix c reads ``packed_all`` at byte c*packed_stride and ``alpha_all`` at
    element c*alpha_stride, and writes y[c]."""
    torch = _torch()
    gran = _gran(granularity)
    lib = load()
    nbytes = int(lib.sherry_packed_bytes(n, k))
    nsc = int(lib.sherry_num_scales(n, k, gran, group_size))
    if nbytes == 0 or nsc < 0:
        raise ValueError("invalid shape, granularity or group size")
    if count < 1:
        raise ValueError("count must be >= 1")
    dev = packed_all.device
    _need_out(packed_all, "packed_all", torch.uint8, (count - 1) * packed_stride + nbytes, dev)
    _need_out(alpha_all, "alpha_all", torch.float32, (count - 1) * alpha_stride + nsc, dev)
    if x.dim() == 1:
        x = x.unsqueeze(0)
    ydt, code = _y_dtype(y_dtype)
    with _on_stream(stream):
        x = _activations(x, k, dev)
        b = x.shape[0]
        if y_stride is None:
            y_stride = b * n
        if y is None:
            y = torch.empty((count, y_stride), dtype=ydt, device=dev)
        else:
            _need_out(y, "y", ydt, (count - 1) * y_stride + b * n, dev)
        ws_bytes = int(lib.sherry_workspace_bytes(_lib.OP_GEMV, n, k, gran, group_size, b, count))
        if ws_bytes == (1 << 64) - 1:
            raise ValueError("invalid batch or count")
        if ws is None:
            ws = _workspace(ws_bytes, dev)
        elif ws_bytes:
            _need_out(ws, "ws", torch.uint8, ws_bytes, dev)
        check(lib.sherry_gemv(n, k, gran, group_size, _ptr(packed_all), _ptr(alpha_all), _ptr(x), b, _ptr(y),
                              code, count, packed_stride, alpha_stride, y_stride, _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream)))
    return y


def gemm(pw: PackedWeight, x, stream=None, out=None):
    """Y = X @ (T*alpha)^T for prefill activations ``x`` [M, K] bf16 -> [M, N] bf16."""
    torch = _torch()
    _check_pw(pw)
    dev = pw.packed.device
    gran = _gran(pw.granularity)
    lib = load()
    with _on_stream(stream):
        x = _activations(x, pw.k, dev)
        m = x.shape[0]
        if out is not None:
            _need_out(out, "out", torch.bfloat16, m * pw.n, dev)
        y = out if out is not None else torch.empty((m, pw.n), dtype=torch.bfloat16, device=dev)
        ws_bytes = int(lib.sherry_workspace_bytes(_lib.OP_GEMM, pw.n, pw.k, gran, pw.group_size, m, 1))
        ws = _workspace(ws_bytes if ws_bytes != (1 << 64) - 1 else 0, dev)
        check(lib.sherry_gemm(pw.n, pw.k, gran, pw.group_size, _ptr(pw.packed), _ptr(pw.alpha), _ptr(x), m,
                              _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return y
