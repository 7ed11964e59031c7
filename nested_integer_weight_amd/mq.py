"""Torch-facing binding of libmq: argument marshalling only.

Every step of the layer (packing, slicing, dequantization, contraction) runs in
the HIP kernels of libmq.so; PyTorch supplies device memory and the current
stream.  Tensors must be contiguous CUDA (HIP) tensors on one device.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field

import torch

from . import _lib
from ._lib import MQ_BF16, MQ_F16, MQ_F32, MQ_PREFIX, MQ_ROUND, MQ_ROUND_EXTRA, MqError, NPLANES  # noqa: F401

RULES = {"prefix": MQ_PREFIX, "round": MQ_ROUND, "extra": MQ_ROUND_EXTRA,
         MQ_PREFIX: MQ_PREFIX, MQ_ROUND: MQ_ROUND, MQ_ROUND_EXTRA: MQ_ROUND_EXTRA}
_DTYPES = {torch.float16: MQ_F16, torch.bfloat16: MQ_BF16, torch.float32: MQ_F32}


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need_cuda(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def plane_bytes(n: int, k: int, plane: int) -> int:
    return int(_lib.lib().mq_plane_bytes(n, k, plane))


def planes_needed(r: int, rule) -> int:
    return int(_lib.lib().mq_planes_needed(r, RULES[rule]))


def workspace_bytes(m: int, n: int, k: int) -> int:
    return int(_lib.lib().mq_linear_workspace_bytes(m, n, k))


@dataclass
class Packed:
    """A packed parent: five bit-plane buffers (uint8 CUDA tensors, or None
    when a plane is not resident)."""
    n: int
    k: int
    planes: list
    _c: _lib.MqPacked = field(default=None, repr=False)

    def cstruct(self) -> _lib.MqPacked:
        if self._c is None:
            c = _lib.MqPacked()
            c.n, c.k = self.n, self.k
            for p in range(NPLANES):
                c.plane[p] = None if self.planes[p] is None else self.planes[p].data_ptr()
            self._c = c
        return self._c

    def truncated(self, r: int, rule="prefix") -> "Packed":
        """A view holding only the planes a width-r call reads (the rest None)."""
        np_ = planes_needed(r, rule)
        return Packed(self.n, self.k, [p if i < np_ else None for i, p in enumerate(self.planes)])

    @property
    def device(self):
        return next(p.device for p in self.planes if p is not None)


def alloc_planes(n: int, k: int, device) -> list:
    return [torch.empty(plane_bytes(n, k, p), dtype=torch.uint8, device=device) for p in range(NPLANES)]


def pack_parent(codes: torch.Tensor, out: list | None = None) -> Packed:
    """codes: uint8 [n, k] CUDA tensor of 8-bit parent codes -> Packed."""
    _need_cuda(codes, "codes", torch.uint8)
    if codes.dim() != 2:
        raise ValueError("codes must be [n, k]")
    n, k = codes.shape
    planes = out if out is not None else alloc_planes(n, k, codes.device)
    pk = Packed(n, k, planes)
    _lib.check(_lib.lib().mq_pack_parent(_ptr(codes), n, k, ctypes.byref(pk.cstruct()), _stream(codes.device)),
               "mq_pack_parent")
    return pk


class Workspace:
    """Split-k workspace memory owned by the caller: one buffer per (device,
    stream), so calls on different streams never share partial sums.

    A buffer that is too small is replaced by a larger one, but the replaced
    buffer stays allocated for the lifetime of this object: a HIP graph
    captured earlier still holds its address and writes to it on replay."""

    def __init__(self):
        self._buf = {}
        self._retired = []

    def get(self, nbytes: int, device) -> torch.Tensor | None:
        if nbytes <= 0:
            return None
        dev = torch.device(device)
        key = (dev, torch.cuda.current_stream(dev).cuda_stream)
        b = self._buf.get(key)
        if b is None or b.numel() < nbytes:
            if b is not None:
                self._retired.append(b)
            b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            self._buf[key] = b
        return b


_default_ws = Workspace()


def _check_layer_args(x, packed, scales, zeros, group):
    _need_cuda(x, "x")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    if x.dim() != 2 or x.shape[1] != packed.k:
        raise ValueError(f"x must be [m, {packed.k}]")
    _need_cuda(scales, "scales", torch.float16)
    _need_cuda(zeros, "zeros", torch.float16)
    g = packed.k // group if group > 0 and packed.k % group == 0 else -1
    if scales.shape != (packed.n, g) or zeros.shape != (packed.n, g):
        raise ValueError(f"scales/zeros must be [{packed.n}, {g}]")


def linear(x: torch.Tensor, packed: Packed, r: int, rule, group: int, scales: torch.Tensor,
           zeros: torch.Tensor, out: torch.Tensor | None = None, workspace: Workspace | None = _default_ws
           ) -> torch.Tensor:
    """y[m, n] = x . dequant(slice_r(Q))^T, y in x's dtype."""
    _check_layer_args(x, packed, scales, zeros, group)
    m = x.shape[0]
    y = out if out is not None else torch.empty((m, packed.n), dtype=x.dtype, device=x.device)
    _need_cuda(y, "out", x.dtype)
    ws = None
    if workspace is not None and m > 0:
        ws = workspace.get(workspace_bytes(m, packed.n, packed.k), x.device)
    _lib.check(_lib.lib().mq_linear(_ptr(x), _DTYPES[x.dtype], m, ctypes.byref(packed.cstruct()), r, RULES[rule],
                                    group, _ptr(scales), _ptr(zeros), _ptr(y), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(x.device)), "mq_linear")
    return y


def linear_noalloc(x: torch.Tensor, packed: Packed, r: int, rule, group: int, scales: torch.Tensor,
                   zeros: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """linear() with the split-k workspace taken from the library's static
    per-device scratch (no device allocation by the library; `out` is the
    caller's).  Calls that overlap in time on one device share the scratch."""
    _check_layer_args(x, packed, scales, zeros, group)
    _need_cuda(out, "out", x.dtype)
    if out.shape != (x.shape[0], packed.n):
        raise ValueError(f"out must be [{x.shape[0]}, {packed.n}]")
    _lib.check(_lib.lib().mq_linear_noalloc(_ptr(x), _DTYPES[x.dtype], x.shape[0], ctypes.byref(packed.cstruct()), r,
                                            RULES[rule], group, _ptr(scales), _ptr(zeros), _ptr(out),
                                            _stream(x.device)), "mq_linear_noalloc")
    return out


@dataclass
class Call:
    x: torch.Tensor
    packed: Packed
    r: int
    rule: object
    group: int
    scales: torch.Tensor
    zeros: torch.Tensor
    out: torch.Tensor | None = None


class PreparedCalls:
    """A fixed list of calls checked and marshalled into the C-ABI call array
    once; run() issues them with one mq_linear_mixed call.  For serving loops
    that repeat the same calls on the same buffers: the tensors (inputs,
    planes, scales, zero points, outputs) must stay alive and keep their
    storage; their contents may change between runs."""

    def __init__(self, calls: list, workspace: Workspace | None = _default_ws):
        self.n = len(calls)
        self.outs = []
        self._workspace = workspace
        if not calls:
            return
        self.dev = calls[0].x.device
        self._arr = (_lib.MqCall * len(calls))()
        self._keep = []
        for i, c in enumerate(calls):
            _check_layer_args(c.x, c.packed, c.scales, c.zeros, c.group)
            m = c.x.shape[0]
            y = c.out if c.out is not None else torch.empty((m, c.packed.n), dtype=c.x.dtype, device=self.dev)
            _need_cuda(y, "out", c.x.dtype)
            self.outs.append(y)
            self._keep.append((c.x, c.scales, c.zeros, y, c.packed))
            e = self._arr[i]
            e.x = c.x.data_ptr()
            e.x_dtype = _DTYPES[c.x.dtype]
            e.m = m
            e.w = ctypes.pointer(c.packed.cstruct())
            e.r = c.r
            e.rule = RULES[c.rule]
            e.group = c.group
            e.scales = c.scales.data_ptr()
            e.zeros = c.zeros.data_ptr()
            e.y = y.data_ptr()
        self._ws_need = int(_lib.lib().mq_linear_mixed_workspace_bytes(self._arr, self.n))
        self._failed = ctypes.c_int32(-1)

    def run(self) -> list:
        if not self.n:
            return []
        ws = self._workspace.get(self._ws_need, self.dev) if self._workspace is not None else None
        st = _lib.lib().mq_linear_mixed(self._arr, self.n, _ptr(ws), 0 if ws is None else ws.numel(),
                                        ctypes.byref(self._failed), _stream(self.dev))
        if st != 0:
            raise MqError(st, f"mq_linear_mixed (call {self._failed.value})")
        return self.outs


def linear_mixed(calls: list, workspace: Workspace | None = _default_ws) -> list:
    """Mix'n'Match: each call at its own width, in order on the current stream."""
    return PreparedCalls(calls, workspace).run()


def slice_codes(packed: Packed, r: int, rule) -> torch.Tensor:
    out = torch.empty((packed.n, packed.k), dtype=torch.uint8, device=packed.device)
    _lib.check(_lib.lib().mq_slice_codes(ctypes.byref(packed.cstruct()), r, RULES[rule], _ptr(out),
                                         _stream(out.device)), "mq_slice_codes")
    return out


def dequant(packed: Packed, r: int, rule, group: int, scales: torch.Tensor, zeros: torch.Tensor,
            dtype=torch.float32) -> torch.Tensor:
    _need_cuda(scales, "scales", torch.float16)
    _need_cuda(zeros, "zeros", torch.float16)
    out = torch.empty((packed.n, packed.k), dtype=dtype, device=packed.device)
    _lib.check(_lib.lib().mq_dequant(ctypes.byref(packed.cstruct()), r, RULES[rule], group, _ptr(scales),
                                     _ptr(zeros), _DTYPES[dtype], _ptr(out), _stream(out.device)), "mq_dequant")
    return out


def produce_parent(w: torch.Tensor, group: int, widths, lambdas, rule="prefix", n_grid: int = 80,
                   grid_den: int = 100):
    """Nested parent of fp32 weights w [n, k]: scale search and cross-width
    code choice in the library.  Returns (codes uint8 [n, k], scales fp16
    [n, k/group], zeros fp16 [n, k/group]) on w's device."""
    _need_cuda(w, "w", torch.float32)
    if w.dim() != 2:
        raise ValueError("w must be [n, k]")
    n, k = w.shape
    widths = [int(r) for r in widths]
    lambdas = [float(v) for v in lambdas]
    if len(widths) != len(lambdas):
        raise ValueError("widths and lambdas differ in length")
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    g = max(k // group, 1) if group > 0 else 1
    scales = torch.empty((n, g), dtype=torch.float16, device=w.device)
    zeros = torch.empty((n, g), dtype=torch.float16, device=w.device)
    wa = (ctypes.c_int32 * max(len(widths), 1))(*widths)
    la = (ctypes.c_float * max(len(lambdas), 1))(*lambdas)
    _lib.check(_lib.lib().mq_produce_parent(_ptr(w), n, k, group, wa, la, len(widths), RULES[rule], n_grid,
                                            grid_den, _ptr(codes), _ptr(scales), _ptr(zeros), _stream(w.device)),
               "mq_produce_parent")
    return codes, scales, zeros
