"""Python binding of the C ABI in include/moe_layout.h, with the same names.

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), outputs are allocated with torch when the caller passes none,
and the call goes to the HIP library on torch's current stream.  Every step
of the path runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import MoeTuning, lib

MOE_F32, MOE_BF16 = 0, 1
MOE_I32, MOE_I64 = 0, 1
STATUS_BAD_EXPERT, STATUS_BAD_POSITION = 1, 2

FIELDS = {  # name -> (id, dtype, shape as a function of (T,K,E,P,R))
    "num_tokens_per_expert": (0, torch.int32, lambda T, K, E, P, R: (E,)),
    "num_tokens_per_rank": (1, torch.int32, lambda T, K, E, P, R: (P,)),
    "is_token_in_rank": (2, torch.uint8, lambda T, K, E, P, R: (T, P)),
    "expert_offset": (3, torch.int32, lambda T, K, E, P, R: (E + 1,)),
    "rank_offset": (4, torch.int32, lambda T, K, E, P, R: (P + 1,)),
    "send_offset": (5, torch.int32, lambda T, K, E, P, R: (P + 1,)),
    "token_slot": (6, torch.int32, lambda T, K, E, P, R: (T, P)),
    "recv_pos": (7, torch.int32, lambda T, K, E, P, R: (T, K)),
    "recv_token": (8, torch.int32, lambda T, K, E, P, R: (R,)),
    "recv_k": (9, torch.int32, lambda T, K, E, P, R: (R,)),
    "status": (10, torch.int32, lambda T, K, E, P, R: (1,)),
    "send_token": (11, torch.int32, lambda T, K, E, P, R: (T * min(K, P),)),
}


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib().moe_strerror(code).decode()
        super().__init__(f"{where}: {msg} (status {code})")
        self.code = code


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise MoeError(rc, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"rows must be float32 or bfloat16, got {t.dtype}")


# Argument marshalling is on every call's host path (a few microseconds per
# call matter for small batches), so pointers and streams go to ctypes as
# plain integers and devices are compared by index.

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    """torch's current stream on `device`, as a raw hipStream_t.  The raw
    query returns the same stream as torch.cuda.current_stream(device)
    (stream contexts included) in a few percent of its time."""
    if _RAW_STREAM is not None:
        return _RAW_STREAM(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, device, shape=None, dtype=None):
    if t.get_device() != device.index:  # -1 for a host tensor
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def moe_workspace_size(T: int, K: int, E: int, P: int, pad_multiple: int = 1) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size_padded(T, K, E, P, pad_multiple, ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


_SIZES = {}  # (T, K, E, P, pad_multiple) -> workspace bytes (pure host functions of the shape)
_SIZES_MAX = 4096  # a job with many distinct token counts starts the cache over past this


def _workspace_bytes(T, K, E, P, pad):
    key = (T, K, E, P, pad)
    v = _SIZES.get(key)
    if v is None:
        if len(_SIZES) >= _SIZES_MAX:
            _SIZES.clear()
        v = _SIZES[key] = moe_workspace_size(T, K, E, P, pad)
    return v


class Handle:
    """Opaque layout handle plus the device workspace its arrays live in."""

    def __init__(self, chunks_per_lane: int = 0, nontemporal: int = 2, waves_per_block: int = 0,
                 layout_pairs: int = 0, pad_multiple: int = 1, gather_mode: int = 0):
        tun = MoeTuning(chunks_per_lane, nontemporal, waves_per_block, layout_pairs, gather_mode)
        h = ctypes.c_void_p()
        _check(lib().moe_handle_create_padded(ctypes.byref(h), ctypes.byref(tun), int(pad_multiple)),
               "moe_handle_create")
        self._h = h
        self.pad_multiple = int(pad_multiple)  # fixed for the handle's life
        self.workspace: Optional[torch.Tensor] = None
        self.T = self.K = self.E = self.P = self.R = None
        self.device = None
        # Layouts computed on this handle so far.  The C handle only ever
        # holds its latest layout, so a backward pass checks that the layout
        # its forward used is still the one in place.
        self.generation = 0

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                lib().moe_handle_destroy(h)
            except Exception:
                pass
            self._h = None

    @property
    def ptr(self) -> ctypes.c_void_p:
        return self._h

    def field(self, name: str) -> torch.Tensor:
        """A view (no copy, no sync) of one handle field inside the workspace."""
        fid, dt, shape = FIELDS[name]
        p = ctypes.c_void_p()
        n = ctypes.c_size_t()
        _check(lib().moe_handle_field(self._h, fid, ctypes.byref(p), ctypes.byref(n)), "moe_handle_field")
        off = (p.value or 0) - self.workspace.data_ptr()
        raw = self.workspace[off:off + n.value]
        return raw.view(dt).reshape(shape(self.T, self.K, self.E, self.P, self.R))

    def check(self) -> int:
        """Synchronises the current stream and returns the device status bits."""
        if self.device is None:
            raise RuntimeError("moe_handle_check: the handle has no layout yet")
        v = ctypes.c_int(0)
        _check(lib().moe_handle_check(self._h, _stream(self.device), ctypes.byref(v)), "moe_handle_check")
        return v.value


def moe_layout(topk_idx: torch.Tensor, num_experts: int, num_partitions: int,
               handle: Optional[Handle] = None, workspace: Optional[torch.Tensor] = None) -> Handle:
    """Layout of one routing decision; returns the handle (see moe_layout.h)."""
    return _layout("moe_layout", topk_idx, num_experts, num_partitions, handle, workspace)


def moe_layout_noalloc(topk_idx: torch.Tensor, num_experts: int, num_partitions: int,
                       handle: Optional[Handle] = None, workspace: Optional[torch.Tensor] = None) -> Handle:
    """moe_layout whose histogram scratch is the library's static per-GPU array
    (see moe_layout.h).  The library call allocates nothing; this wrapper
    allocates only when it has to create the workspace, so a caller that passes
    one, or reuses the handle's, allocates nothing at all (graph capture)."""
    return _layout("moe_layout_noalloc", topk_idx, num_experts, num_partitions, handle, workspace)


def _layout(entry, topk_idx, num_experts, num_partitions, handle, workspace) -> Handle:
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, K]")
    dev = topk_idx.device
    _need(topk_idx, "topk_idx", dev)
    if topk_idx.dtype == torch.int32:
        itype = MOE_I32
    elif topk_idx.dtype == torch.int64:
        itype = MOE_I64
    else:
        raise TypeError("topk_idx must be int32 or int64")
    T, K = topk_idx.shape
    E, P = int(num_experts), int(num_partitions)
    h = handle if handle is not None else Handle()
    if workspace is None:
        need = _workspace_bytes(T, K, E, P, h.pad_multiple)
        ws = h.workspace
        if ws is None or ws.numel() < need or ws.get_device() != dev.index:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", dev, dtype=torch.uint8)
        ws = workspace  # the library checks its size
    _check(getattr(lib(), entry)(h.ptr, _ptr(topk_idx), itype, T, K, E, P, _ptr(ws), ws.numel(),
                                 _stream(dev)), entry)
    if (h.T, h.K, h.E, h.P) != (T, K, E, P) or h.R is None:
        n = ctypes.c_int64(0)
        _check(lib().moe_recv_capacity(h.ptr, ctypes.byref(n)), "moe_recv_capacity")
        h.R = n.value  # receive rows: T*K, plus the padding capacity of a padded handle
    h.workspace, h.T, h.K, h.E, h.P, h.device = ws, T, K, E, P, dev
    h.generation += 1
    return h


def moe_recv_capacity(handle: Handle) -> int:
    """Rows of a receive buffer for the handle's layout: T*K + E*(pad_multiple-1)."""
    return handle.R


def moe_dispatch(handle: Handle, x: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                 scale_rows: bool = False, recv: Optional[torch.Tensor] = None,
                 recv_scores=None):
    """recv[recv_pos[t,k]] = x[t] (scaled by w[t,k] if scale_rows).

    recv_scores: None (not produced), True (allocate) or a float32 [R] tensor.
    Returns (recv, recv_scores or None)."""
    h = handle
    dev = h.device
    T, K = h.T, h.K
    _need(x, "x", dev)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError(f"x must be [{T}, H]")
    H = x.shape[1]
    dt = _dtype_code(x)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", dev, (T, K), torch.float32)
    R = h.R
    if recv is None:
        recv = torch.empty((R, H), dtype=x.dtype, device=dev)
    _need(recv, "recv", dev, (R, H), x.dtype)
    if recv_scores is True:
        recv_scores = torch.empty(R, dtype=torch.float32, device=dev)
    elif recv_scores is False:
        recv_scores = None
    if recv_scores is not None:
        _need(recv_scores, "recv_scores", dev, (R,), torch.float32)
    _check(lib().moe_dispatch(h.ptr, _ptr(x), dt, H, _ptr(topk_weights), int(bool(scale_rows)),
                              _ptr(recv), _ptr(recv_scores), _stream(dev)), "moe_dispatch")
    return recv, recv_scores


def moe_combine(handle: Handle, y: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = sum_k [w[t,k] *] y[recv_pos[t,k]] (float32, k order)."""
    h = handle
    dev = h.device
    T, K = h.T, h.K
    _need(y, "y", dev)
    if y.dim() != 2 or y.shape[0] != h.R:
        raise ValueError(f"y must be [{h.R}, H]")
    H = y.shape[1]
    dt = _dtype_code(y)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", dev, (T, K), torch.float32)
    if out is None:
        out = torch.empty((T, H), dtype=y.dtype, device=dev)
    _need(out, "out", dev, (T, H), y.dtype)
    _check(lib().moe_combine(h.ptr, _ptr(y), dt, H, _ptr(topk_weights), _ptr(out), _stream(dev)),
           "moe_combine")
    return out


def moe_combine_bwd(handle: Handle, grad_out: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None, grad_y: Optional[torch.Tensor] = None,
                    grad_w=None):
    """grad_y[recv_pos[t,k]] = [w[t,k] *] grad_out[t]; grad_w[t,k] = <grad_out[t], y[row]>.

    grad_y: None (allocate), False (rows not produced: grad_w only) or a tensor.
    grad_w: None (not produced), True (allocate) or a float32 [T,K] tensor.
    Returns (grad_y, grad_w or None)."""
    h = handle
    dev = h.device
    T, K = h.T, h.K
    _need(grad_out, "grad_out", dev)
    if grad_out.dim() != 2 or grad_out.shape[0] != T:
        raise ValueError(f"grad_out must be [{T}, H]")
    H = grad_out.shape[1]
    dt = _dtype_code(grad_out)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", dev, (T, K), torch.float32)
    if y is not None:
        _need(y, "y", dev, (h.R, H), grad_out.dtype)
    if grad_y is None:
        grad_y = torch.empty((h.R, H), dtype=grad_out.dtype, device=dev)
    elif grad_y is False:
        grad_y = None  # router-weight gradient only
    if grad_y is not None:
        _need(grad_y, "grad_y", dev, (h.R, H), grad_out.dtype)
    if grad_w is True:
        grad_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    elif grad_w is False:
        grad_w = None
    if grad_w is not None:
        _need(grad_w, "grad_w", dev, (T, K), torch.float32)
    _check(lib().moe_combine_bwd(h.ptr, _ptr(grad_out), dt, H, _ptr(topk_weights), _ptr(y),
                                 _ptr(grad_y), _ptr(grad_w), _stream(dev)), "moe_combine_bwd")
    return grad_y, grad_w


def moe_dispatch_bwd(handle: Handle, grad_recv: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                     x: Optional[torch.Tensor] = None, grad_x: Optional[torch.Tensor] = None,
                     grad_s=None):
    """grad_x[t] = sum_k [w[t,k] *] grad_recv[recv_pos[t,k]]; grad_s[t,k] = <grad_recv[row], x[t]>.

    Pass topk_weights iff the forward dispatch scaled its rows.
    grad_x: None (allocate), False (rows not produced: grad_s only) or a tensor.
    grad_s: None, True (allocate) or a float32 [T,K] tensor.
    Returns (grad_x, grad_s or None)."""
    h = handle
    dev = h.device
    T, K = h.T, h.K
    _need(grad_recv, "grad_recv", dev)
    if grad_recv.dim() != 2 or grad_recv.shape[0] != h.R:
        raise ValueError(f"grad_recv must be [{h.R}, H]")
    H = grad_recv.shape[1]
    dt = _dtype_code(grad_recv)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", dev, (T, K), torch.float32)
    if x is not None:
        _need(x, "x", dev, (T, H), grad_recv.dtype)
    if grad_x is None:
        grad_x = torch.empty((T, H), dtype=grad_recv.dtype, device=dev)
    elif grad_x is False:
        grad_x = None  # score gradient only
    if grad_x is not None:
        _need(grad_x, "grad_x", dev, (T, H), grad_recv.dtype)
    if grad_s is True:
        grad_s = torch.empty((T, K), dtype=torch.float32, device=dev)
    elif grad_s is False:
        grad_s = None
    if grad_s is not None:
        _need(grad_s, "grad_s", dev, (T, K), torch.float32)
    _check(lib().moe_dispatch_bwd(h.ptr, _ptr(grad_recv), dt, H, _ptr(topk_weights), _ptr(x),
                                  _ptr(grad_x), _ptr(grad_s), _stream(dev)), "moe_dispatch_bwd")
    return grad_x, grad_s


# ---- staged exchange ---------------------------------------------------------

def moe_send_capacity(handle: Handle) -> int:
    """Rows a send buffer must hold: T * min(K, P)."""
    n = ctypes.c_int64(0)
    _check(lib().moe_send_capacity(handle.ptr, ctypes.byref(n)), "moe_send_capacity")
    return n.value


def _send_buf(handle: Handle, t: Optional[torch.Tensor], H: int, dtype, name: str):
    cap = moe_send_capacity(handle)
    if t is None:
        return torch.empty((cap, H), dtype=dtype, device=handle.device)
    _need(t, name, handle.device, dtype=dtype)
    if t.dim() != 2 or t.shape[1] != H or t.shape[0] < cap:
        raise ValueError(f"{name} must be [>= {cap}, {H}]")
    return t


def moe_send(handle: Handle, x: torch.Tensor, send: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Source side of a staged dispatch: send[send_offset[r] + token_slot[t,r]] = x[t]."""
    h = handle
    _need(x, "x", h.device)
    if x.dim() != 2 or x.shape[0] != h.T:
        raise ValueError(f"x must be [{h.T}, H]")
    H = x.shape[1]
    send = _send_buf(h, send, H, x.dtype, "send")
    _check(lib().moe_send(h.ptr, _ptr(x), _dtype_code(x), H, _ptr(send), send.shape[0],
                          _stream(h.device)), "moe_send")
    return send


def moe_expand(handle: Handle, send: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
               scale_rows: bool = False, recv: Optional[torch.Tensor] = None, recv_scores=None):
    """Receiver side of a staged dispatch; returns (recv, recv_scores or None)."""
    h = handle
    _need(send, "send", h.device)
    H = send.shape[1]
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", h.device, (h.T, h.K), torch.float32)
    if recv is None:
        recv = torch.empty((h.R, H), dtype=send.dtype, device=h.device)
    _need(recv, "recv", h.device, (h.R, H), send.dtype)
    if recv_scores is True:
        recv_scores = torch.empty(h.R, dtype=torch.float32, device=h.device)
    elif recv_scores is False:
        recv_scores = None
    if recv_scores is not None:
        _need(recv_scores, "recv_scores", h.device, (h.R,), torch.float32)
    _check(lib().moe_expand(h.ptr, _ptr(send), _dtype_code(send), H, send.shape[0], _ptr(topk_weights),
                            int(bool(scale_rows)), _ptr(recv), _ptr(recv_scores), _stream(h.device)),
           "moe_expand")
    return recv, recv_scores


def moe_reduce_partitions(handle: Handle, y: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                          partial: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Receiver side of the two-level combine: one partial row per send row."""
    h = handle
    _need(y, "y", h.device)
    if y.dim() != 2 or y.shape[0] != h.R:
        raise ValueError(f"y must be [{h.R}, H]")
    H = y.shape[1]
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", h.device, (h.T, h.K), torch.float32)
    partial = _send_buf(h, partial, H, y.dtype, "partial")
    _check(lib().moe_reduce_partitions(h.ptr, _ptr(y), _dtype_code(y), H, _ptr(topk_weights),
                                       _ptr(partial), partial.shape[0], _stream(h.device)),
           "moe_reduce_partitions")
    return partial


def moe_combine_partitions(handle: Handle, partial: torch.Tensor,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Source side of the two-level combine: partitions added in ascending order."""
    h = handle
    _need(partial, "partial", h.device)
    H = partial.shape[1]
    if out is None:
        out = torch.empty((h.T, H), dtype=partial.dtype, device=h.device)
    _need(out, "out", h.device, (h.T, H), partial.dtype)
    _check(lib().moe_combine_partitions(h.ptr, _ptr(partial), _dtype_code(partial), H, partial.shape[0],
                                        _ptr(out), _stream(h.device)), "moe_combine_partitions")
    return out


class CuBudgetStream:
    """A HIP stream restricted to compute units [cu_first, cu_first + cu_count)
    (moe_stream_create_cu_budget), usable as a torch stream (`.stream`)."""

    def __init__(self, cu_first: int, cu_count: int, device=None):
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        with torch.cuda.device(dev):
            s = ctypes.c_void_p()
            _check(lib().moe_stream_create_cu_budget(int(cu_first), int(cu_count), ctypes.byref(s)),
                   "moe_stream_create_cu_budget")
        self._s = s
        self.cu_first, self.cu_count = int(cu_first), int(cu_count)
        self.stream = torch.cuda.ExternalStream(s.value, device=dev)

    def close(self):
        if getattr(self, "_s", None) is not None and self._s.value:
            self.stream.synchronize()
            lib().moe_stream_destroy(self._s)
            self._s = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_time_next_kernel(h: Handle, start: Optional[int], stop: Optional[int]) -> None:
    """Measurement hook: the next kernel a row call on ``h`` launches binds
    the raw ``hipEvent_t`` handle ``stop`` (an integer) to its completion
    and, when ``start`` is given, records ``start`` just before it.
    One-shot; ``None, None`` disarms."""
    _check(lib().moe_time_next_kernel(h.ptr, start, stop), "moe_time_next_kernel")


def moe_bench_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """Plain device copy (calibration kernel for HBM traffic counters)."""
    if dst.numel() * dst.element_size() != src.numel() * src.element_size():
        raise ValueError("size mismatch")
    _check(lib().moe_bench_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(),
                                _stream(src.device)), "moe_bench_copy")
