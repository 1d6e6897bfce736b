"""Python binding of the joint RoPE attention library (libflux_attn.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/flux_attn.h``.  PyTorch supplies device
memory and the stream.  There is no CPU fallback: if the shared library is
missing, loading raises ``FluxAttnError``.

    plan = Plan(batch=1, num_heads=24, head_dim=128, max_tokens=8704)
    out = plan.forward(q, k, v, segment_tokens=[512, 4096, 4096], pos_ids=pos)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflux_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "flux_attn.h")

OK, INVALID_ARGUMENT, UNSUPPORTED, DEVICE_ERROR, OUT_OF_MEMORY = 0, 1, 2, 3, 4
BF16, FP8_E4M3 = 0, 1
_MODES = ("joint", "segment_local")


class FluxAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("max_segments", ctypes.c_int32),
        ("rope_axes_dim", ctypes.c_int32 * 3),
        ("rope_theta", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


_lib = None
_vp, _i32, _i32p, _fp = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libflux_attn.so (built by ``python -m diffusion_transformer_joint_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FluxAttnError(DEVICE_ERROR, f"{p} is missing: build it with "
                            "`python -m diffusion_transformer_joint_amd.build`")
    # torch ships its own HIP runtime under the same soname; load it first so
    # that the library binds to that one instead of pulling in a second copy.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    cp = ctypes.POINTER(Config)
    sig = {
        "flux_attn_default_config": ([cp, _i32, _i32, _i32, _i32], ctypes.c_int),
        "flux_attn_validate_config": ([cp], ctypes.c_int),
        "flux_attn_validate_forward": ([cp, _vp, _vp, _vp, _vp, _i32p, _i32, _vp, _vp], ctypes.c_int),
        "flux_attn_create": ([cp, ctypes.POINTER(_vp)], ctypes.c_int),
        "flux_attn_forward": ([_vp, _vp, _vp, _vp, _vp, _i32p, _i32, _vp, _vp, _vp], ctypes.c_int),
        "flux_attn_forward_segment_local": ([_vp, _vp, _vp, _vp, _vp, _i32p, _i32, _vp, _vp, _vp], ctypes.c_int),
        "flux_attn_forward_noalloc": ([cp, _vp, _vp, _vp, _vp, _i32p, _i32, _vp, _vp, _vp], ctypes.c_int),
        "flux_attn_get_config": ([_vp, cp], ctypes.c_int),
        "flux_attn_destroy": ([_vp], ctypes.c_int),
        "flux_attn_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "flux_attn_last_error": ([], ctypes.c_char_p),
        "flux_attn_abi_version": ([], ctypes.c_int),
        "flux_attn_timing_enable": ([_vp, _i32], ctypes.c_int),
        "flux_attn_schedule": ([_i32, _i32, _i32, _i32, _i32, _i32p, _i32p, _i32p, _i32p], ctypes.c_int),
        "flux_attn_timing_read": ([_vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                   ctypes.POINTER(ctypes.c_double), _i32, _i32p], ctypes.c_int),
        "flux_attn_block_mask": ([_vp, _vp, _vp, _i32p, _i32, _vp, ctypes.c_float, _vp, _vp], ctypes.c_int),
        "flux_attn_block_mask_pooled": ([_vp, _vp, _vp, _i32p, _i32, _vp, ctypes.c_float, _vp, _vp], ctypes.c_int),
        "flux_attn_forward_sparse": ([_vp, _vp, _vp, _vp, _i32p, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
        "flux_attn_forward_lse": ([_vp, _vp, _vp, _vp, _i32p, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
        "flux_attn_backward": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32p, _i32, _vp, _vp, _vp, _vp, _vp],
                               ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    if path is None:
        _lib = lib
    return lib


def header_functions(header: str = HEADER_PATH) -> list:
    """Names of the functions include/flux_attn.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"\b(flux_attn_[a-z_0-9]+)\s*\(", text)))


def last_error() -> str:
    return load_library().flux_attn_last_error().decode()


def check(status: int, what: str = "flux_attn") -> None:
    if status != OK:
        lib = load_library()
        raise FluxAttnError(status, f"{what}: {lib.flux_attn_status_string(status).decode()}: "
                            f"{lib.flux_attn_last_error().decode()}")


def default_config(batch: int, num_heads: int, head_dim: int, max_tokens: int, dtype: str = "bf16",
                   rope_axes_dim: Optional[Sequence[int]] = None, rope_theta: float = 10000.0,
                   softmax_scale: float = 0.0, max_segments: int = 12) -> Config:
    lib = load_library()
    cfg = Config()
    check(lib.flux_attn_default_config(ctypes.byref(cfg), batch, num_heads, head_dim, max_tokens),
          "default_config")
    if rope_axes_dim is not None:
        for i in range(3):
            cfg.rope_axes_dim[i] = int(rope_axes_dim[i])
    cfg.rope_theta = rope_theta
    cfg.softmax_scale = softmax_scale
    cfg.max_segments = max_segments
    cfg.dtype = {"bf16": BF16, "fp8": FP8_E4M3, "fp8_e4m3": FP8_E4M3}[dtype]
    return cfg


def schedule(tiles: int, kv_tiles: int, num_cus: int, max_pieces: int, head_dim: int = 128) -> dict:
    """The library's work split for one launch (host-side policy, no GPU needed)."""
    lib = load_library()
    out = [ctypes.c_int32() for _ in range(4)]
    check(lib.flux_attn_schedule(tiles, kv_tiles, num_cus, max_pieces, head_dim, *[ctypes.byref(x) for x in out]),
          "schedule")
    return dict(zip(("whole_tiles", "split_tiles", "split", "grid"), (x.value for x in out)))


def _i32_array(values: Sequence[int]):
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr


def _device_tensor(name, t, device, shape=None, dtype=None):
    """Reject a tensor the kernels cannot address: not on ``device``, not
    contiguous, or of the wrong shape or dtype.  The C side cannot tell a host
    pointer from a device pointer, so this is the only guard against handing a
    kernel host memory."""
    if not t.is_cuda or t.device != device:
        raise FluxAttnError(INVALID_ARGUMENT, f"{name} must be a tensor on {device} (got {t.device})")
    if not t.is_contiguous():
        raise FluxAttnError(INVALID_ARGUMENT, f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise FluxAttnError(INVALID_ARGUMENT, f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise FluxAttnError(INVALID_ARGUMENT, f"{name} has dtype {t.dtype}, expected {dtype}")


NOALLOC_SCRATCH_BYTES = 32 << 20   # FLUX_ATTN_NOALLOC_SCRATCH_BYTES


def forward_noalloc(config: Config, q, k, v, segment_tokens: Sequence[int], pos_ids, out, scales=None,
                    stream=None):
    """Joint attention through ``flux_attn_forward_noalloc``: no plan and no
    device allocation (the library's static scratch holds the RoPE table and
    split partials).  ``config`` comes from ``default_config``; the tensors are
    as for ``Plan.forward`` and ``out`` must be given.  Returns out."""
    import torch

    fp8 = config.dtype == FP8_E4M3
    want = (torch.uint8, torch.float8_e4m3fn) if fp8 else torch.bfloat16
    n = int(sum(segment_tokens))
    shape = (config.batch, n, config.num_heads, config.head_dim)
    if not q.is_cuda:
        raise FluxAttnError(INVALID_ARGUMENT, f"q must be a device tensor (got {q.device})")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _device_tensor(name, t, q.device, shape, want)
    _device_tensor("pos_ids", pos_ids, q.device, (n, 3), torch.int32)
    _device_tensor("out", out, q.device, shape, torch.bfloat16)
    sp = None
    if scales is not None:
        _device_tensor("scales", scales, q.device, (3, config.batch, config.num_heads), torch.float32)
        sp = scales.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load_library()
    segs = _i32_array(segment_tokens)
    check(lib.flux_attn_forward_noalloc(ctypes.byref(config), q.data_ptr(), k.data_ptr(), v.data_ptr(), sp, segs,
                                        len(segment_tokens), pos_ids.data_ptr(), out.data_ptr(),
                                        stream.cuda_stream), "forward_noalloc")
    return out


class Plan:
    """A plan for one configuration; owns the library's device workspace."""

    def __init__(self, batch: int, num_heads: int, head_dim: int, max_tokens: int, dtype: str = "bf16",
                 rope_axes_dim: Optional[Sequence[int]] = None, rope_theta: float = 10000.0,
                 softmax_scale: float = 0.0, max_segments: int = 12):
        self._lib = load_library()
        self.config = default_config(batch, num_heads, head_dim, max_tokens, dtype, rope_axes_dim,
                                     rope_theta, softmax_scale, max_segments)
        handle = ctypes.c_void_p()
        check(self._lib.flux_attn_create(ctypes.byref(self.config), ctypes.byref(handle)), "create")
        self._handle = handle

    @property
    def fp8(self) -> bool:
        return self.config.dtype == FP8_E4M3

    def forward(self, q, k, v, segment_tokens: Sequence[int], pos_ids, out=None, scales=None,
                mode: str = "joint", stream=None):
        """Attention over torch device tensors on ``stream`` (default: current stream).

        q, k, v: [B, N, H, D] contiguous bf16 (or uint8 / float8_e4m3fn codes for an
        FP8 plan); pos_ids: [N, 3] int32; scales: [3, B, H] float32 (FP8 only);
        out: optional [B, N, H, D] bf16 destination.  mode "joint" calls
        flux_attn_forward, "segment_local" flux_attn_forward_segment_local.
        Returns out.
        """
        import torch

        if mode not in _MODES:
            raise FluxAttnError(INVALID_ARGUMENT, f"unknown mode {mode!r}")
        want = (torch.uint8, torch.float8_e4m3fn) if self.fp8 else torch.bfloat16
        n, shape = self._check_qkv(q, k, v, segment_tokens, pos_ids, want)
        c = self.config
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
        else:
            _device_tensor("out", out, q.device, shape, torch.bfloat16)
        sp = None
        if scales is not None:
            _device_tensor("scales", scales, q.device, (3, c.batch, c.num_heads), torch.float32)
            sp = scales.data_ptr()
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        segs = _i32_array(segment_tokens)
        fn = self._lib.flux_attn_forward if mode == "joint" else self._lib.flux_attn_forward_segment_local
        check(fn(self._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), sp, segs, len(segment_tokens),
                 pos_ids.data_ptr(), out.data_ptr(), stream.cuda_stream), mode)
        return out

    def _check_qkv(self, q, k, v, segment_tokens, pos_ids, want=None):
        import torch
        if self._handle is None:
            raise FluxAttnError(INVALID_ARGUMENT, "plan is closed")
        want = torch.bfloat16 if want is None else want
        n = int(sum(segment_tokens))
        c = self.config
        shape = (c.batch, n, c.num_heads, c.head_dim)
        if not q.is_cuda:
            raise FluxAttnError(INVALID_ARGUMENT, f"q must be a device tensor (got {q.device})")
        for name, t in (("q", q), ("k", k), ("v", v)):
            _device_tensor(name, t, q.device, shape, want)
        _device_tensor("pos_ids", pos_ids, q.device, (n, 3), torch.int32)
        return n, shape

    def mask_shape(self, n_tokens: int) -> tuple:
        """Shape of a tile mask: [B, H, ceil(N/256), ceil(N/64)]."""
        c = self.config
        return (c.batch, c.num_heads, (n_tokens + 255) // 256, (n_tokens + 63) // 64)

    def block_mask(self, q, k, segment_tokens: Sequence[int], pos_ids, tau: float, mask=None, stream=None,
                   rule: str = "bound"):
        """Tile mask (uint8 [B, H, QT, KT]) for threshold tau: rule "bound"
        (flux_attn_block_mask, the score-bound rule) or "pooled"
        (flux_attn_block_mask_pooled)."""
        if rule not in ("bound", "pooled"):
            raise FluxAttnError(INVALID_ARGUMENT, f"unknown rule {rule!r}")
        import torch
        n, _ = self._check_qkv(q, k, k, segment_tokens, pos_ids)
        ms = self.mask_shape(n)
        if mask is None:
            mask = torch.empty(ms, dtype=torch.uint8, device=q.device)
        else:
            _device_tensor("mask", mask, q.device, ms, torch.uint8)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        segs = _i32_array(segment_tokens)
        fn = self._lib.flux_attn_block_mask if rule == "bound" else self._lib.flux_attn_block_mask_pooled
        check(fn(self._handle, q.data_ptr(), k.data_ptr(), segs, len(segment_tokens), pos_ids.data_ptr(),
                 float(tau), mask.data_ptr(), stream.cuda_stream), f"block_mask ({rule})")
        return mask

    def forward_sparse(self, q, k, v, segment_tokens: Sequence[int], pos_ids, mask, out=None, stream=None):
        """Attention over the kept tiles of ``mask`` (uint8 [B, H, QT, KT]).  Returns out."""
        import torch
        n, shape = self._check_qkv(q, k, v, segment_tokens, pos_ids)
        ms = self.mask_shape(n)
        _device_tensor("mask", mask, q.device, ms, torch.uint8)
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
        else:
            _device_tensor("out", out, q.device, shape, torch.bfloat16)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        segs = _i32_array(segment_tokens)
        check(self._lib.flux_attn_forward_sparse(self._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), segs,
                                                 len(segment_tokens), pos_ids.data_ptr(), mask.data_ptr(),
                                                 out.data_ptr(), stream.cuda_stream), "forward_sparse")
        return out

    def forward_lse(self, q, k, v, segment_tokens: Sequence[int], pos_ids, out=None, lse=None, stream=None):
        """Joint forward that also returns the row log-sum-exp ([B, H, N] float32).  Returns (out, lse)."""
        import torch
        n, shape = self._check_qkv(q, k, v, segment_tokens, pos_ids)
        c = self.config
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=q.device)
        else:
            _device_tensor("out", out, q.device, shape, torch.bfloat16)
        ls = (c.batch, c.num_heads, n)
        if lse is None:
            lse = torch.empty(ls, dtype=torch.float32, device=q.device)
        else:
            _device_tensor("lse", lse, q.device, ls, torch.float32)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        segs = _i32_array(segment_tokens)
        check(self._lib.flux_attn_forward_lse(self._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), segs,
                                              len(segment_tokens), pos_ids.data_ptr(), out.data_ptr(),
                                              lse.data_ptr(), stream.cuda_stream), "forward_lse")
        return out, lse

    def backward(self, q, k, v, out, dout, lse, segment_tokens: Sequence[int], pos_ids, stream=None):
        """Gradients (dq, dk, dv) of the joint attention for upstream gradient dout."""
        import torch
        n, shape = self._check_qkv(q, k, v, segment_tokens, pos_ids)
        c = self.config
        for name, t in (("out", out), ("dout", dout)):
            _device_tensor(name, t, q.device, shape, torch.bfloat16)
        _device_tensor("lse", lse, q.device, (c.batch, c.num_heads, n), torch.float32)
        dq, dk, dv = (torch.empty(shape, dtype=torch.bfloat16, device=q.device) for _ in range(3))
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        segs = _i32_array(segment_tokens)
        check(self._lib.flux_attn_backward(self._handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           dout.data_ptr(), lse.data_ptr(), segs, len(segment_tokens),
                                           pos_ids.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                           stream.cuda_stream), "backward")
        return dq, dk, dv

    def timing_enable(self, capacity: int) -> None:
        """Record the attention kernel's duration for the next ``capacity`` forwards."""
        check(self._lib.flux_attn_timing_enable(self._handle, int(capacity)), "timing_enable")

    def timing_read(self, max_count: int = 4096, with_merge: bool = False):
        """Durations (ms) of the attention kernels recorded since timing_enable/last read.

        with_merge: return a dict instead: "attn_ms" (attention kernel),
        "total_ms" (attention kernel plus the merge of its split pieces) and
        "clock_mhz" (average shader clock of the timed attention kernels)."""
        buf = (ctypes.c_float * max_count)()
        tot = (ctypes.c_float * max_count)()
        mhz = ctypes.c_double(0.0)
        n = ctypes.c_int32(0)
        check(self._lib.flux_attn_timing_read(self._handle, buf, tot, ctypes.byref(mhz), max_count, ctypes.byref(n)),
              "timing_read")
        attn = [buf[i] for i in range(n.value)]
        if not with_merge:
            return attn
        return {"attn_ms": attn, "total_ms": [tot[i] for i in range(n.value)], "clock_mhz": mhz.value}

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None:
            h, self._handle = self._handle, None
            check(self._lib.flux_attn_destroy(h), "destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
