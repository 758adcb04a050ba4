"""Python face of the C ABI: torch tensors in, device pointers and sizes out.

Every step of the layer runs in the HIP library; this module only checks tensor
shapes/dtypes, allocates outputs and the workspace with torch, and passes pointers
and the current HIP stream.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_PATHS = {"auto": _lib.MOE_PATH_AUTO, "gemv": _lib.MOE_PATH_GEMV, "gemm": _lib.MOE_PATH_GEMM}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def device_supported(device: int = 0):
    lib = _lib.load()
    buf = ctypes.create_string_buffer(64)
    ok = lib.moe_device_supported(device, buf, 64)
    return bool(ok), buf.value.decode()


def kernel_scale_shape(groups: int, n: int, k: int):
    """Shape of the kernel-layout scales: [G][ceil(K/128)][ceil(N/64)][16][4][4]."""
    return (groups, (k // 32 + 3) // 4, (n + 63) // 64, 16, 4, 4)


def pack_fp4(codes: torch.Tensor, scales: torch.Tensor, stream=None):
    """Checkpoint layout (codes [G][N][K/2], scales [G][N][K/32]) -> kernel layout
    (codes [G][K/32][N][16], scales as ``kernel_scale_shape``), by the library's pack kernel."""
    lib = _lib.load()
    g, n, half_k = codes.shape
    k = 2 * half_k
    if tuple(scales.shape) != (g, n, k // 32) or codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise ValueError("pack_fp4 wants uint8 codes [G][N][K/2] and scales [G][N][K/32]")
    if not (codes.is_cuda and scales.is_cuda and codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("pack_fp4 wants contiguous CUDA tensors")
    out_c = torch.empty((g, k // 32, n, 16), dtype=torch.uint8, device=codes.device)
    out_s = torch.empty(kernel_scale_shape(g, n, k), dtype=torch.uint8, device=codes.device)
    _lib.check(lib.moe_pack_fp4(_ptr(codes), _ptr(scales), _ptr(out_c), _ptr(out_s), g, n, k,
                                _stream_handle(stream)), lib)
    return out_c, out_s


def pack_fp8(codes: torch.Tensor, stream=None) -> torch.Tensor:
    """FP8 E4M3 codes in the checkpoint layout [G][N][K] (uint8) -> the kernel layout
    [G][K/128][N][128], by the library's pack kernel.  Block scales need no repacking."""
    lib = _lib.load()
    g, n, k = codes.shape
    if codes.dtype != torch.uint8 or not codes.is_cuda or not codes.is_contiguous() or k % 128:
        raise ValueError("pack_fp8 wants contiguous uint8 CUDA codes [G][N][K] with K a multiple of 128")
    out = torch.empty((g, k // 128, n, 128), dtype=torch.uint8, device=codes.device)
    _lib.check(lib.moe_pack_fp8(_ptr(codes), _ptr(out), g, n, k, _stream_handle(stream)), lib)
    return out


class MoeLayer:
    """One routed FP4-expert MoE layer over borrowed device weights.

    ``gate``/``up``/``down`` are (codes, scales) uint8 CUDA tensors in the kernel
    layout: codes [G][K/32][N][16], scales ``kernel_scale_shape`` (see ``pack_fp4``),
    G = E + S groups.  With ``shared_fp8`` = dict(gate=(codes, scales), up=..., down=...)
    the shared expert is FP8 E4M3 instead (codes in the kernel layout of ``pack_fp8``,
    float32 scales [N/128][K/128]) and the FP4 arrays hold the E routed experts only.
    The library keeps only pointers, so this object holds references to keep them alive.
    """

    def __init__(self, w_router: torch.Tensor, gate, up, down, top_k: int, n_shared: int = 1,
                 router_bias: Optional[torch.Tensor] = None, path: str = "auto", shared_fp8: Optional[dict] = None,
                 routed_scale: float = 1.0, host_weights: bool = False):
        self.lib = _lib.load()
        e, h = w_router.shape
        g, hb, inter, sixteen = gate[0].shape
        fp4_groups = e if shared_fp8 is not None else e + n_shared
        if g != fp4_groups or hb * 32 != h or sixteen != 16:
            raise ValueError(f"gate codes {tuple(gate[0].shape)} do not match E={e}, S={n_shared}, H={h}")
        f8 = {}
        if shared_fp8 is not None:
            for name, n, k in (("gate", inter, h), ("up", inter, h), ("down", h, inter)):
                c, sc = shared_fp8[name]
                if tuple(c.shape) != (k // 128, n, 128) or c.dtype != torch.uint8 or not c.is_cuda:
                    raise ValueError(f"shared FP8 {name} codes {tuple(c.shape)}, expected {(k // 128, n, 128)}")
                if tuple(sc.shape) != (n // 128, k // 128) or sc.dtype != torch.float32 or not sc.is_cuda:
                    raise ValueError(f"shared FP8 {name} scales {tuple(sc.shape)}, expected {(n // 128, k // 128)}")
                if not c.is_contiguous() or not sc.is_contiguous():
                    raise ValueError(f"shared FP8 {name} tensors must be contiguous")
                f8[f"shared_{name}_fp8"] = _ptr(c)
                f8[f"shared_{name}_fp8_scales"] = _ptr(sc)
        for name, (c, s), n, k in (("gate", gate, inter, h), ("up", up, inter, h), ("down", down, h, inter)):
            if tuple(c.shape) != (g, k // 32, n, 16) or tuple(s.shape) != kernel_scale_shape(g, n, k):
                raise ValueError(f"{name} weights: codes {tuple(c.shape)} / scales {tuple(s.shape)}, "
                                 f"expected {(g, k // 32, n, 16)} / {(g, k // 32, n)} (kernel layout)")
            if c.dtype != torch.uint8 or s.dtype != torch.uint8:
                raise ValueError(f"{name} weights must be uint8 tensors")
            if host_weights and not (c.is_pinned() and s.is_pinned()):
                raise ValueError(f"{name} weights must be pinned host tensors (host_weights=True: an expert bank)")
            if not host_weights and not (c.is_cuda and s.is_cuda):
                raise ValueError(f"{name} weights must be CUDA tensors")
            if not c.is_contiguous() or not s.is_contiguous():
                raise ValueError(f"{name} weights must be contiguous")
        if w_router.dtype != torch.float32 or not w_router.is_cuda or not w_router.is_contiguous():
            raise ValueError("w_router must be a contiguous float32 CUDA tensor")
        if router_bias is not None and (router_bias.dtype != torch.float32 or router_bias.numel() != e
                                        or not router_bias.is_cuda):
            raise ValueError("router_bias must be a float32 CUDA tensor of E values")
        self.hidden, self.n_experts, self.top_k, self.n_shared, self.inter = h, e, top_k, n_shared, inter
        self.device = w_router.device
        self._keep = (w_router, gate, up, down, router_bias, shared_fp8)
        desc = _lib.LayerDesc(
            abi_version=_lib.MOE_ABI_VERSION, hidden=h, n_experts=e, top_k=top_k, n_shared=n_shared,
            inter=inter, path=_PATHS[path], device=w_router.device.index or 0, block=32,
            flags=_lib.MOE_SHARED_FP8 if shared_fp8 is not None else 0, routed_scale=routed_scale, reserved=0,
            w_router=_ptr(w_router), router_bias=_ptr(router_bias),
            gate_codes=_ptr(gate[0]), gate_scales=_ptr(gate[1]), up_codes=_ptr(up[0]),
            up_scales=_ptr(up[1]), down_codes=_ptr(down[0]), down_scales=_ptr(down[1]), **f8)
        handle = ctypes.c_void_p()
        _lib.check(self.lib.moe_layer_create(ctypes.byref(desc), ctypes.byref(handle)), self.lib)
        self._h = handle

    def close(self):
        if getattr(self, "_h", None):
            self.lib.moe_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -------------------------------------------------------------------------------
    def workspace_bytes(self, max_tokens: int) -> int:
        return int(self.lib.moe_workspace_bytes(self._h, max_tokens))

    def workspace(self, max_tokens: int) -> torch.Tensor:
        """A zero-filled workspace (the library's control words must start at zero)."""
        return torch.zeros(self.workspace_bytes(max_tokens), dtype=torch.uint8, device=self.device)

    def route_buffers(self, tokens: int) -> dict:
        d, k, e = self.device, self.top_k, self.n_experts
        return dict(idx=torch.empty((tokens, k), dtype=torch.int32, device=d),
                    weight=torch.empty((tokens, k), dtype=torch.float32, device=d),
                    counts=torch.empty(e, dtype=torch.int32, device=d),
                    offsets=torch.empty(e + 1, dtype=torch.int32, device=d),
                    perm=torch.empty(tokens * k, dtype=torch.int32, device=d))

    @staticmethod
    def _route_struct(r: dict) -> _lib.RouteOut:
        return _lib.RouteOut(idx=_ptr(r["idx"]), weight=_ptr(r["weight"]), counts=_ptr(r["counts"]),
                             offsets=_ptr(r["offsets"]), perm=_ptr(r["perm"]))

    def _check_x(self, x: torch.Tensor) -> int:
        if x.dim() != 2 or x.shape[1] != self.hidden or x.element_size() != 2 or not x.is_cuda:
            raise ValueError(f"x must be a [T][{self.hidden}] bf16 CUDA tensor")
        if not x.is_contiguous():
            raise ValueError("x must be contiguous")
        return x.shape[0]

    def route(self, x: torch.Tensor, workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
              stream=None) -> dict:
        t = self._check_x(x)
        out = out if out is not None else self.route_buffers(t)
        ws = workspace if workspace is not None else self.workspace(t)
        rs = self._route_struct(out)
        _lib.check(self.lib.moe_route(self._h, _ptr(x), t, ctypes.byref(rs), _ptr(ws), ws.numel(),
                                      _stream_handle(stream)), self.lib)
        return out

    def forward(self, x: torch.Tensor, workspace: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                route: Optional[dict] = None, stream=None) -> torch.Tensor:
        t = self._check_x(x)
        if y is None:
            y = torch.empty((t, self.hidden), dtype=torch.float32, device=self.device)
        ws = workspace if workspace is not None else self.workspace(t)
        rs = self._route_struct(route) if route is not None else None
        _lib.check(self.lib.moe_forward(self._h, _ptr(x), t, _ptr(y), ctypes.byref(rs) if rs is not None else None,
                                        _ptr(ws), ws.numel(), _stream_handle(stream)), self.lib)
        return y

    def forward_noalloc(self, x: torch.Tensor, y: torch.Tensor, route: Optional[dict] = None,
                        stream=None) -> torch.Tensor:
        """forward with the workspace in the library's per-device scratch array: nothing is
        allocated, so the caller passes the output too."""
        t = self._check_x(x)
        if y.shape != (t, self.hidden) or y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous():
            raise ValueError(f"y must be a contiguous [{t}][{self.hidden}] float32 CUDA tensor")
        rs = self._route_struct(route) if route is not None else None
        _lib.check(self.lib.moe_forward_noalloc(self._h, _ptr(x), t, _ptr(y),
                                                ctypes.byref(rs) if rs is not None else None,
                                                _stream_handle(stream)), self.lib)
        return y

    __call__ = forward


# ---- partial-residency expert bank --------------------------------------------------------

class MoeBank:
    """HBM expert slots filled on demand from a layer whose FP4 weights are pinned host tensors
    (``MoeLayer(..., host_weights=True)``): ``forward`` routes on the device, waits for the
    routing counts, uploads the missing active experts in refill groups of ``group`` and runs the
    grouped-GEMM expert kernels of each refill group as soon as its uploads are in."""

    def __init__(self, layer: "MoeLayer", n_slots: int, group: int):
        self.lib = _lib.load()
        self.layer = layer
        h = ctypes.c_void_p()
        _lib.check(self.lib.moe_bank_create(layer._h, n_slots, group, ctypes.byref(h)), self.lib)
        self._h = h.value

    def forward(self, x: torch.Tensor, workspace: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                route: Optional[dict] = None, stream=None) -> torch.Tensor:
        L = self.layer
        t = L._check_x(x)
        if y is None:
            y = torch.empty((t, L.hidden), dtype=torch.float32, device=L.device)
        ws = workspace if workspace is not None else L.workspace(t)
        rs = L._route_struct(route) if route is not None else None
        _lib.check(self.lib.moe_bank_forward(self._h, _ptr(x), t, _ptr(y), ctypes.byref(rs) if rs is not None else None,
                                             _ptr(ws), ws.numel(), _stream_handle(stream)), self.lib)
        return y

    def stats(self) -> dict:
        out = (ctypes.c_int64 * 5)()
        _lib.check(self.lib.moe_bank_stats(self._h, out), self.lib)
        return dict(calls=out[0], resident_hits=out[1], uploads=out[2], bytes_uploaded=out[3], refill_groups=out[4])

    def close(self):
        if getattr(self, "_h", None):
            self.lib.moe_bank_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- chained decode ----------------------------------------------------------------------

def _f32_cuda(t, shape, what):
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be a contiguous float32 CUDA tensor of shape {tuple(shape)}")


def residual_rmsnorm(h_src: torch.Tensor, y: Optional[torch.Tensor] = None, h_dst: Optional[torch.Tensor] = None,
                     norm_weight: Optional[torch.Tensor] = None, eps: float = 1e-6, x: Optional[torch.Tensor] = None,
                     stream=None):
    """The join between two layers (one library call): h_dst = h_src + y when y is given, and
    x = bf16(RMSNorm(h) * norm_weight) when x is given; returns x."""
    lib = _lib.load()
    t, h = h_src.shape
    _f32_cuda(h_src, (t, h), "h_src")
    for name, a in (("y", y), ("h_dst", h_dst)):
        if a is not None:
            _f32_cuda(a, (t, h), name)
    if norm_weight is not None:
        _f32_cuda(norm_weight, (h,), "norm_weight")
    if x is not None and (x.element_size() != 2 or not x.is_cuda or not x.is_contiguous() or tuple(x.shape) != (t, h)):
        raise ValueError(f"x must be a contiguous [{t}][{h}] 16-bit CUDA tensor")
    _lib.check(lib.moe_residual_rmsnorm(_ptr(h_src), _ptr(y), _ptr(h_dst), _ptr(norm_weight), eps, _ptr(x), t, h,
                                        _stream_handle(stream)), lib)
    return x


class MoeChain:
    """Layers recorded into one HIP graph by the library and replayed by ``run``.

    ``residual=True``: the chained decode -- layer l's input x[l] = bf16(RMSNorm(h_l) * norm_weight[l]),
    y[l] = layer l (x[l]), h_{l+1} = h_l + y[l], from ``h_in`` to ``h_out``.  ``residual=False``: the
    layers one after another on the inputs the caller writes into ``x`` (independent calls).  The
    buffers are allocated here (x [L][T][H] int16 bf16 bits, y [L][T][H] float32, h_in/h_out
    [T][H] float32) and are the graph's: write inputs into ``h_in`` (or ``x``) in place."""

    def __init__(self, layers, tokens: int, residual: bool = True, norm_weight=None, eps: float = 1e-6,
                 routes: bool = False):
        self.lib = _lib.load()
        if not layers:
            raise ValueError("a chain needs at least one layer")
        self.layers = list(layers)
        h, dev = self.layers[0].hidden, self.layers[0].device
        n, t = len(self.layers), tokens
        self.hidden, self.tokens, self.device, self.residual = h, t, dev, residual
        self.x = torch.zeros((n, t, h), dtype=torch.int16, device=dev)
        self.y = torch.zeros((n, t, h), dtype=torch.float32, device=dev)
        self.h_in = torch.zeros((t, h), dtype=torch.float32, device=dev) if residual else None
        self.h_out = torch.zeros((t, h), dtype=torch.float32, device=dev) if residual else None
        self.routes = [l.route_buffers(t) for l in self.layers] if routes else None
        self.workspace = torch.zeros(max(l.workspace_bytes(t) for l in self.layers), dtype=torch.uint8, device=dev)
        self.norm_weight = list(norm_weight) if norm_weight is not None else None
        if self.norm_weight is not None:
            if len(self.norm_weight) != n:
                raise ValueError("one norm weight per layer")
            for g in self.norm_weight:
                if g is not None:
                    _f32_cuda(g, (h,), "norm weight")
        lp = (ctypes.c_void_p * n)(*[l._h for l in self.layers])
        gp = None
        if self.norm_weight is not None:
            gp = (ctypes.c_void_p * n)(*[_ptr(g) for g in self.norm_weight])
        rp = None
        if self.routes is not None:
            rp = (_lib.RouteOut * n)(*[MoeLayer._route_struct(r) for r in self.routes])
        self._arrays = (lp, gp, rp)
        desc = _lib.ChainDesc(abi_version=_lib.MOE_ABI_VERSION, n_layers=n, tokens=t,
                              flags=_lib.MOE_CHAIN_RESIDUAL if residual else 0, eps=eps, reserved=0,
                              layers=ctypes.cast(lp, ctypes.POINTER(ctypes.c_void_p)),
                              norm_weight=ctypes.cast(gp, ctypes.POINTER(ctypes.c_void_p)) if gp is not None else None,
                              h_in=_ptr(self.h_in), h_out=_ptr(self.h_out), x=_ptr(self.x), y=_ptr(self.y),
                              routes=ctypes.cast(rp, ctypes.POINTER(_lib.RouteOut)) if rp is not None else None,
                              workspace=_ptr(self.workspace), workspace_bytes=self.workspace.numel())
        torch.cuda.synchronize(dev)        # the zeroed buffers exist before the graph names them
        h_ = ctypes.c_void_p()
        _lib.check(self.lib.moe_chain_create(ctypes.byref(desc), ctypes.byref(h_)), self.lib)
        self._h = h_.value

    def run(self, stream=None):
        _lib.check(self.lib.moe_chain_run(self._h, _stream_handle(stream)), self.lib)

    def close(self):
        if getattr(self, "_h", None):
            self.lib.moe_chain_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- kernel timing ---------------------------------------------------------------------

def timing_enable(on: bool = True):
    _lib.load().moe_timing_enable(1 if on else 0)


def timing_reset():
    _lib.load().moe_timing_reset()


def timing_read() -> dict:
    """{kernel name: (launches, total_ms)} since the last reset (waits for the recorded events)."""
    lib = _lib.load()
    cap = 64
    names = (ctypes.c_char_p * cap)()
    launches = (ctypes.c_int64 * cap)()
    ms = (ctypes.c_double * cap)()
    n = lib.moe_timing_read(names, launches, ms, cap)
    return {names[i].decode(): (int(launches[i]), float(ms[i])) for i in range(min(n, cap))}
