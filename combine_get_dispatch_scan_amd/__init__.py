"""Python binding of libmoe_ep: MoE dispatch / combine on one MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
``libmoe_ep.so`` (built from ``csrc/`` for gfx950); PyTorch supplies device
memory and the stream.  There is no CPU fallback: if the library is missing
the calls raise.

Two layers:

* ``ep_*`` -- one function per C entry point of ``include/moe_ep.h``, same
  names and arguments (device pointers as ints, the stream as a handle).
* ``get_dispatch_layout`` / ``dispatch`` / ``dispatch_cached`` / ``combine`` /
  ``dispatch_backward`` / ``combine_backward`` / ``handle_recv_counts`` -- the
  same calls on torch tensors: they allocate
  the outputs with ``torch.empty`` on the tensors' device and launch on torch's
  current stream.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

from . import _build

LIB_PATH = _build.LIB_PATH

EP_OK = 0
EP_EINVAL = -1
EP_EHIP = -2
EP_ECAPACITY = -3
EP_EIDS = -4
EP_HANDLE_MAGIC = 0x31485045
EP_MAX_LL_TOKENS = 256
EP_NOALLOC_SCRATCH_BYTES = 81920


class EpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe_ep error {code}: {msg}")
        self.code = code


class ep_handle_t(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("stage", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_partitions", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("use_fp8", ctypes.c_int32),
        ("capacity_rows", ctypes.c_int32),
        ("has_weights", ctypes.c_int32),
        ("num_chunks", ctypes.c_int32),
        ("static_cap", ctypes.c_int32),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
        ("expert_offset", ctypes.c_void_p),
        ("slot", ctypes.c_void_p),
        ("src_token", ctypes.c_void_p),
        ("weights", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("pair_code", ctypes.c_void_p),
        ("chunk_base", ctypes.c_void_p),
        ("chunk_pcnt", ctypes.c_void_p),
        ("chunk_inv", ctypes.c_void_p),
        ("chunk_cnt", ctypes.c_void_p),
        ("expert_alignment", ctypes.c_int32),
        ("scale_ld", ctypes.c_int32),
        ("fp8_input", ctypes.c_int32),
        ("dispatch_seq", ctypes.c_int32),
    ]


_lib = None

# C entry points and their ctypes signatures
_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "ep_version": ([], _I),
    "ep_last_error": ([], ctypes.c_char_p),
    "ep_workspace_bytes": ([_I, _I, _I, _I], ctypes.c_size_t),
    "ep_get_dispatch_layout": ([_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                ctypes.POINTER(ep_handle_t), _P], _I),
    "ep_dispatch": ([_P, _P, _I, _I, _P, _P, _I, ctypes.POINTER(ep_handle_t), _P], _I),
    "ep_dispatch_cached": ([_P, ctypes.POINTER(ep_handle_t), _P, _P, _P], _I),
    "ep_get_dispatch_layout_aligned": ([_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                        ctypes.POINTER(ep_handle_t), _P], _I),
    "ep_dispatch_ex": ([_P, _P, _P, _I, _I, _I, _P, _P, _I, ctypes.POINTER(ep_handle_t), _P], _I),
    "ep_dispatch_cached_ex": ([_P, _P, ctypes.POINTER(ep_handle_t), _P, _P, _P], _I),
    "ep_combine_fp8": ([_P, _P, ctypes.POINTER(ep_handle_t), _P, _P, _P], _I),
    "ep_dispatch_backward_fp8": ([_P, _P, ctypes.POINTER(ep_handle_t), _P, _P], _I),
    "ep_low_latency_dispatch": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                 _P, ctypes.c_size_t, ctypes.POINTER(ep_handle_t), _P], _I),
    "ep_low_latency_dispatch_noalloc": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P,
                                         _P, ctypes.POINTER(ep_handle_t), _P], _I),
    "ep_combine": ([_P, ctypes.POINTER(ep_handle_t), _P, _P, _P], _I),
    "ep_dispatch_backward": ([_P, ctypes.POINTER(ep_handle_t), _P, _P], _I),
    "ep_combine_backward": ([_P, _P, ctypes.POINTER(ep_handle_t), _P, _P, _P, _P], _I),
    "ep_handle_recv_counts": ([ctypes.POINTER(ep_handle_t), _P, _P, _P], _I),
    "ep_handle_recv_counts_async": ([ctypes.POINTER(ep_handle_t), _P, _P], _I),
    "ep_recv_counts_decode": ([ctypes.POINTER(ep_handle_t), _P, _P, _P], _I),
    "ep_e4m3fn_encode": ([_P, _P, ctypes.c_int64, _P], _I),
    "ep_rank_routing": ([_P, _I, _I, _I, _I, _P, _P], _I),
    "ep_pack_metadata": ([_P, _P, _I, _I, _P, ctypes.POINTER(ep_handle_t), _P, _P, _P], _I),
}


def load():
    """Load libmoe_ep.so (raises if it has not been built).

    torch, when installed, is imported first: its HIP libraries load the HIP
    runtime torch ships, and the library then binds to that same runtime (it
    asks for the runtime by its soname).  Loaded the other way round, torch
    would load a second HIP runtime into the process, and the two do not
    share the device."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc: int, ok=(EP_OK,)):
    if rc not in ok:
        raise EpError(rc, load().ep_last_error().decode())
    return rc


# ----------------------------------------------------------------------------
# the C entry points
# ----------------------------------------------------------------------------

def ep_version() -> int:
    return load().ep_version()


def ep_last_error() -> str:
    return load().ep_last_error().decode()


def ep_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int, num_partitions: int) -> int:
    return load().ep_workspace_bytes(num_tokens, num_topk, num_experts, num_partitions)


def ep_get_dispatch_layout(topk_idx, num_tokens, num_topk, num_experts, num_partitions,
                           num_tokens_per_partition, num_tokens_per_expert,
                           is_token_in_partition, num_invalid, ws, ws_bytes, handle, stream) -> int:
    return load().ep_get_dispatch_layout(topk_idx, num_tokens, num_topk, num_experts,
                                         num_partitions, num_tokens_per_partition,
                                         num_tokens_per_expert, is_token_in_partition,
                                         num_invalid, ws, ws_bytes, ctypes.byref(handle), stream)


def ep_dispatch(x, topk_weights, hidden, use_fp8, recv_x, recv_scales, capacity_rows, handle,
                stream) -> int:
    return load().ep_dispatch(x, topk_weights, hidden, int(use_fp8), recv_x, recv_scales,
                              capacity_rows, ctypes.byref(handle), stream)


def ep_low_latency_dispatch(x, topk_idx, topk_weights, num_tokens, hidden, num_topk, num_experts,
                            num_partitions, use_fp8, num_max_tokens, recv_x, recv_scales,
                            num_tokens_per_partition, num_tokens_per_expert,
                            is_token_in_partition, num_invalid, ws, ws_bytes, handle,
                            stream) -> int:
    return load().ep_low_latency_dispatch(x, topk_idx, topk_weights, num_tokens, hidden, num_topk,
                                          num_experts, num_partitions, int(use_fp8),
                                          num_max_tokens, recv_x, recv_scales,
                                          num_tokens_per_partition, num_tokens_per_expert,
                                          is_token_in_partition, num_invalid, ws, ws_bytes,
                                          ctypes.byref(handle), stream)


def ep_low_latency_dispatch_noalloc(x, topk_idx, topk_weights, num_tokens, hidden, num_topk,
                                    num_experts, num_partitions, use_fp8, num_max_tokens, recv_x,
                                    recv_scales, num_tokens_per_partition, num_tokens_per_expert,
                                    is_token_in_partition, num_invalid, handle, stream) -> int:
    return load().ep_low_latency_dispatch_noalloc(x, topk_idx, topk_weights, num_tokens, hidden,
                                                  num_topk, num_experts, num_partitions,
                                                  int(use_fp8), num_max_tokens, recv_x, recv_scales,
                                                  num_tokens_per_partition, num_tokens_per_expert,
                                                  is_token_in_partition, num_invalid,
                                                  ctypes.byref(handle), stream)


def ep_get_dispatch_layout_aligned(topk_idx, num_tokens, num_topk, num_experts, num_partitions,
                                   expert_alignment, num_tokens_per_partition,
                                   num_tokens_per_expert, is_token_in_partition, num_invalid, ws,
                                   ws_bytes, handle, stream) -> int:
    return load().ep_get_dispatch_layout_aligned(topk_idx, num_tokens, num_topk, num_experts,
                                                 num_partitions, expert_alignment,
                                                 num_tokens_per_partition, num_tokens_per_expert,
                                                 is_token_in_partition, num_invalid, ws, ws_bytes,
                                                 ctypes.byref(handle), stream)


def ep_dispatch_ex(x, x_scales, topk_weights, hidden, use_fp8, scale_ld, recv_x, recv_scales,
                   capacity_rows, handle, stream) -> int:
    return load().ep_dispatch_ex(x, x_scales, topk_weights, hidden, int(use_fp8), scale_ld, recv_x,
                                 recv_scales, capacity_rows, ctypes.byref(handle), stream)


def ep_dispatch_cached_ex(x, x_scales, handle, recv_x, recv_scales, stream) -> int:
    return load().ep_dispatch_cached_ex(x, x_scales, ctypes.byref(handle), recv_x, recv_scales,
                                        stream)


def ep_dispatch_cached(x, handle, recv_x, recv_scales, stream) -> int:
    return load().ep_dispatch_cached(x, ctypes.byref(handle), recv_x, recv_scales, stream)


def ep_combine(y, handle, topk_weights, out, stream) -> int:
    return load().ep_combine(y, ctypes.byref(handle), topk_weights, out, stream)


def ep_combine_fp8(y, y_scales, handle, topk_weights, out, stream) -> int:
    return load().ep_combine_fp8(y, y_scales, ctypes.byref(handle), topk_weights, out, stream)


def ep_dispatch_backward_fp8(grad_recv, grad_scales, handle, grad_x, stream) -> int:
    return load().ep_dispatch_backward_fp8(grad_recv, grad_scales, ctypes.byref(handle), grad_x,
                                           stream)


def ep_dispatch_backward(grad_recv, handle, grad_x, stream) -> int:
    return load().ep_dispatch_backward(grad_recv, ctypes.byref(handle), grad_x, stream)


def ep_combine_backward(grad_out, y, handle, topk_weights, grad_y, grad_w, stream) -> int:
    return load().ep_combine_backward(grad_out, y, ctypes.byref(handle), topk_weights, grad_y,
                                      grad_w, stream)


def ep_handle_recv_counts(handle, host_counts, host_num_recv, stream) -> int:
    return load().ep_handle_recv_counts(ctypes.byref(handle), host_counts, host_num_recv, stream)


def ep_handle_recv_counts_async(handle, host_buf, stream) -> int:
    return load().ep_handle_recv_counts_async(ctypes.byref(handle), host_buf, stream)


def ep_recv_counts_decode(handle, host_buf, host_counts, host_num_recv) -> int:
    return load().ep_recv_counts_decode(ctypes.byref(handle), host_buf, host_counts, host_num_recv)


def ep_e4m3fn_encode(inp, out, n, stream) -> int:
    return load().ep_e4m3fn_encode(inp, out, n, stream)


# ----------------------------------------------------------------------------
# the same calls on torch tensors
# ----------------------------------------------------------------------------

def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_KINDS = {}


def _kinds():
    """Element types the library accepts, by the C type it reads."""
    if not _KINDS:
        import torch
        _KINDS.update(bf16=(torch.bfloat16,), fp8=(torch.float8_e4m3fn, torch.uint8),
                      f32=(torch.float32,), i64=(torch.int64,), i32=(torch.int32,),
                      u8=(torch.uint8,))
    return _KINDS


def _ptr(t, kind: Optional[str] = None, name: str = "tensor") -> Optional[int]:
    """Device address of a tensor the library reads or writes densely.  It
    must be a GPU tensor, contiguous (rows without gaps) and, when ``kind``
    names one, of an element type the call takes; anything else raises
    before the call."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous: the library reads and writes rows densely")
    if kind is not None and t.dtype not in _kinds()[kind]:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in _kinds()[kind])}, got {t.dtype}")
    return t.data_ptr()


@dataclass
class Handle:
    """Routing metadata of one dispatch (wraps ep_handle_t and keeps the
    workspace it points into alive).  num_recv is the number of dispatched
    pairs once handle_recv_counts has read it (None before)."""
    c: ep_handle_t
    ws: object
    num_recv: Optional[int] = None

    @property
    def num_tokens(self):
        return self.c.num_tokens

    @property
    def num_topk(self):
        return self.c.num_topk

    @property
    def hidden(self):
        return self.c.hidden

    def _view(self, field, n, dtype):
        import torch
        ptr = getattr(self.c, field)
        if n == 0 or not ptr:
            return torch.empty(0, dtype=dtype, device=self.ws.device)
        off = ptr - self.ws.data_ptr()
        return self.ws[off:off + n * 4].view(dtype)

    @property
    def slot(self):
        import torch
        return self._view("slot", self.num_tokens * self.num_topk, torch.int32).view(self.num_tokens, self.num_topk)

    @property
    def src_token(self):
        import torch
        return self._view("src_token", self.num_tokens * self.num_topk, torch.int32)

    @property
    def expert_offset(self):
        import torch
        return self._view("expert_offset", self.c.num_experts + 1, torch.int32)

    @property
    def weights(self):
        import torch
        return self._view("weights", self.num_tokens * self.num_topk, torch.float32).view(self.num_tokens, self.num_topk)


@dataclass
class Layout:
    num_tokens_per_partition: object
    num_tokens_per_expert: object
    is_token_in_partition: object
    num_invalid: object
    handle: Handle


def get_dispatch_layout(topk_idx, num_experts: int, num_partitions: int, ws=None,
                        expert_alignment: int = 1) -> Layout:
    """topk_idx: int64 [T, K] on the GPU.  Returns the counts, the mask and a
    handle for ``dispatch``.  ``ws`` (uint8, >= ep_workspace_bytes) may be
    passed to reuse a workspace.  expert_alignment > 1 rounds each expert's
    block of receive rows up to a multiple of it (zeroed padding rows)."""
    import torch
    T, K = topk_idx.shape
    dev = topk_idx.device
    nbytes = ep_workspace_bytes(T, K, num_experts, num_partitions)
    if nbytes == 0:
        raise EpError(EP_EINVAL, f"invalid dims T={T} K={K} E={num_experts} P={num_partitions}")
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ntpp = torch.empty(num_partitions, dtype=torch.int32, device=dev)
    ntpe = torch.empty(num_experts, dtype=torch.int32, device=dev)
    itip = torch.empty((T, num_partitions), dtype=torch.uint8, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    h = ep_handle_t()
    _check(ep_get_dispatch_layout_aligned(_ptr(topk_idx.contiguous(), "i64", "topk_idx"), T, K, num_experts,
                                          num_partitions, int(expert_alignment), _ptr(ntpp),
                                          _ptr(ntpe), _ptr(itip), _ptr(ninv), _ptr(ws, "u8", "ws"), ws.numel(),
                                          h, _stream()))
    return Layout(ntpp, ntpe, itip, ninv, Handle(h, ws))


def dispatch(x, topk_weights, layout: Layout, use_fp8: bool, capacity_rows: Optional[int] = None,
             x_scales=None, column_major_scales: bool = False):
    """x: bf16 [T, H] (or, with x_scales fp32 [T, H/128], E4M3FN codes [T, H]
    passed through unchanged); topk_weights: fp32 [T, K] or None.
    Returns (recv_x, recv_scales or None, handle).  recv_x is float8_e4m3fn
    [capacity, H] in FP8 mode, else bf16 [capacity, H]; capacity defaults to
    the worst case T*K (+ E*(A-1) for an aligned layout), so no host sync.
    column_major_scales stores recv_scales as [H/128, ld], ld = capacity
    rounded up to a multiple of 4."""
    import torch
    h = layout.handle
    T, H = x.shape
    K = h.num_topk
    A = max(1, h.c.expert_alignment)
    cap = T * K + h.c.num_experts * (A - 1) if capacity_rows is None else int(capacity_rows)
    dev = x.device
    scale_ld = 0
    if use_fp8:
        recv = torch.empty((cap, H), dtype=torch.float8_e4m3fn, device=dev)
        if column_major_scales:
            scale_ld = (cap + 3) // 4 * 4
            scales = torch.empty((H // 128, scale_ld), dtype=torch.float32, device=dev)
        else:
            scales = torch.empty((cap, H // 128), dtype=torch.float32, device=dev)
    else:
        recv = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        scales = None
    _check(ep_dispatch_ex(_ptr(x, "fp8" if x_scales is not None else "bf16", "x"),
                          _ptr(x_scales, "f32", "x_scales"), _ptr(topk_weights, "f32", "topk_weights"),
                          H, int(use_fp8), scale_ld, _ptr(recv), _ptr(scales), cap, h.c, _stream()))
    return recv, scales, h


def low_latency_dispatch(x, topk_idx, topk_weights, num_experts: int, num_partitions: int,
                         num_max_tokens: int, use_fp8: bool, ws=None, out=None):
    """One-launch dispatch for decode batches (T <= 256) into a static
    per-expert layout: expert e's rows are [e*cap, (e+1)*cap).  Returns
    (recv_x [E*cap, H], recv_scales or None, Layout).  ``out`` may pass
    preallocated (recv_x, recv_scales, Layout) to reuse (e.g. under graph
    capture)."""
    import torch
    T, H = x.shape
    K = topk_idx.shape[1]
    topk_idx = topk_idx.contiguous()
    E, P, cap = num_experts, num_partitions, num_max_tokens
    dev = x.device
    if out is None:
        if ws is None:
            ws = torch.empty(ep_workspace_bytes(T, K, E, P), dtype=torch.uint8, device=dev)
        lay = Layout(torch.empty(P, dtype=torch.int32, device=dev),
                     torch.empty(E, dtype=torch.int32, device=dev),
                     torch.empty((T, P), dtype=torch.uint8, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev), Handle(ep_handle_t(), ws))
        if use_fp8:
            recv = torch.empty((E * cap, H), dtype=torch.float8_e4m3fn, device=dev)
            scales = torch.empty((E * cap, H // 128), dtype=torch.float32, device=dev)
        else:
            recv = torch.empty((E * cap, H), dtype=torch.bfloat16, device=dev)
            scales = None
    else:
        recv, scales, lay = out
    h = lay.handle
    _check(ep_low_latency_dispatch(_ptr(x, "bf16", "x"), _ptr(topk_idx, "i64", "topk_idx"),
                                   _ptr(topk_weights, "f32", "topk_weights"), T, H, K, E, P,
                                   int(use_fp8), cap, _ptr(recv, "fp8" if use_fp8 else "bf16", "recv_x"),
                                   _ptr(scales, "f32", "recv_scales"),
                                   _ptr(lay.num_tokens_per_partition),
                                   _ptr(lay.num_tokens_per_expert),
                                   _ptr(lay.is_token_in_partition), _ptr(lay.num_invalid),
                                   _ptr(h.ws), h.ws.numel(), h.c, _stream()))
    return recv, scales, lay


def dispatch_cached(x, handle: Handle, recv_x=None, recv_scales=None, x_scales=None):
    """Re-send new rows along a dispatched handle's routing (same options:
    x_scales exactly when the handle was dispatched from FP8 input)."""
    import torch
    c = handle.c
    cap, H = c.capacity_rows, c.hidden
    if recv_x is None:
        recv_x = torch.empty((cap, H), dtype=torch.float8_e4m3fn if c.use_fp8 else torch.bfloat16,
                             device=x.device)
    if c.use_fp8 and recv_scales is None:
        shape = (H // 128, c.scale_ld) if c.scale_ld else (cap, H // 128)
        recv_scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check(ep_dispatch_cached_ex(_ptr(x, "fp8" if (x_scales is not None or c.fp8_input) else "bf16", "x"),
                                 _ptr(x_scales, "f32", "x_scales"),
                                 c, _ptr(recv_x, "fp8" if c.use_fp8 else "bf16", "recv_x"),
                                 _ptr(recv_scales, "f32", "recv_scales"), _stream()))
    return recv_x, recv_scales


def combine(y, handle: Handle, topk_weights=None, out=None):
    """y: bf16 [rows, H] in dispatch's receive order.  Returns bf16 [T, H]."""
    import torch
    c = handle.c
    if out is None:
        out = torch.empty((c.num_tokens, c.hidden), dtype=torch.bfloat16, device=y.device)
    _check(ep_combine(_ptr(y, "bf16", "y"), c, _ptr(topk_weights, "f32", "topk_weights"),
                      _ptr(out, "bf16", "out"), _stream()))
    return out


def combine_fp8(y, y_scales, handle: Handle, topk_weights=None, out=None):
    """y: float8_e4m3fn (or uint8) [rows, H] with fp32 scales [rows, H/128], in
    dispatch's receive order.  Returns bf16 [T, H]."""
    import torch
    c = handle.c
    if out is None:
        out = torch.empty((c.num_tokens, c.hidden), dtype=torch.bfloat16, device=y.device)
    _check(ep_combine_fp8(_ptr(y, "fp8", "y"), _ptr(y_scales, "f32", "y_scales"), c,
                          _ptr(topk_weights, "f32", "topk_weights"), _ptr(out, "bf16", "out"), _stream()))
    return out


def dispatch_backward_fp8(grad_recv, grad_scales, handle: Handle, grad_x=None):
    """grad_recv: float8_e4m3fn [rows, H] + fp32 scales [rows, H/128].
    Returns grad_x bf16 [T, H]."""
    import torch
    c = handle.c
    if grad_x is None:
        grad_x = torch.empty((c.num_tokens, c.hidden), dtype=torch.bfloat16, device=grad_recv.device)
    _check(ep_dispatch_backward_fp8(_ptr(grad_recv, "fp8", "grad_recv"), _ptr(grad_scales, "f32", "grad_scales"),
                                    c, _ptr(grad_x, "bf16", "grad_x"), _stream()))
    return grad_x


def dispatch_backward(grad_recv, handle: Handle, grad_x=None):
    """grad_recv: bf16 [rows, H] in the receive order.  Returns grad_x bf16 [T, H]."""
    import torch
    c = handle.c
    if grad_x is None:
        grad_x = torch.empty((c.num_tokens, c.hidden), dtype=torch.bfloat16, device=grad_recv.device)
    _check(ep_dispatch_backward(_ptr(grad_recv, "bf16", "grad_recv"), c, _ptr(grad_x, "bf16", "grad_x"),
                                _stream()))
    return grad_x


def combine_backward(grad_out, handle: Handle, y=None, topk_weights=None, grad_y=None):
    """grad_out: bf16 [T, H].  Returns (grad_y bf16 [capacity, H], grad_w fp32
    [T, K] or None when y is None).  Rows of grad_y that no pair maps to are
    left as allocated."""
    import torch
    c = handle.c
    dev = grad_out.device
    if grad_y is None:
        grad_y = torch.empty((c.capacity_rows, c.hidden), dtype=torch.bfloat16, device=dev)
    grad_w = None if y is None else torch.empty((c.num_tokens, c.num_topk), dtype=torch.float32,
                                                device=dev)
    _check(ep_combine_backward(_ptr(grad_out, "bf16", "grad_out"), _ptr(y, "bf16", "y"), c,
                               _ptr(topk_weights, "f32", "topk_weights"), _ptr(grad_y, "bf16", "grad_y"),
                               _ptr(grad_w, "f32", "grad_w"), _stream()))
    return grad_y, grad_w


def handle_recv_counts(handle: Handle):
    """Synchronises the current stream.  Returns (counts list[E], N, status)
    where status is EP_OK, EP_ECAPACITY or EP_EIDS."""
    E = handle.c.num_experts
    counts = (ctypes.c_int32 * E)()
    n = ctypes.c_int32(0)
    rc = _check(ep_handle_recv_counts(handle.c, counts, ctypes.byref(n), _stream()),
                ok=(EP_OK, EP_ECAPACITY, EP_EIDS))
    handle.num_recv = int(n.value)
    return list(counts), int(n.value), rc


def handle_recv_counts_async(handle: Handle, host_buf):
    """Enqueue the count readback into ``host_buf`` (int32 [E+5], pinned CPU
    tensor) without waiting.  Wait on an event recorded after this call, then
    call ``recv_counts_decode``."""
    _check(ep_handle_recv_counts_async(handle.c, host_buf.data_ptr(), _stream()))


def recv_counts_decode(handle: Handle, host_buf):
    """Returns (counts list[E], N, status) from a filled ``host_buf``."""
    E = handle.c.num_experts
    counts = (ctypes.c_int32 * E)()
    n = ctypes.c_int32(0)
    rc = _check(ep_recv_counts_decode(handle.c, host_buf.data_ptr(), counts, ctypes.byref(n)),
                ok=(EP_OK, EP_ECAPACITY, EP_EIDS))
    return list(counts), int(n.value), rc


def e4m3fn_encode(v):
    """fp32 tensor -> uint8 codes with the device encoder."""
    import torch
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check(ep_e4m3fn_encode(_ptr(v.contiguous(), "f32", "v"), _ptr(out), v.numel(), _stream()))
    return out


# ----------------------------------------------------------------------------
# expert parallelism over ranks, one rank's share
# ----------------------------------------------------------------------------

def ep_rank_routing(topk_idx, num_tokens, num_topk, num_experts, num_partitions, part_idx,
                    stream) -> int:
    return load().ep_rank_routing(topk_idx, num_tokens, num_topk, num_experts, num_partitions,
                                  part_idx, stream)


def ep_pack_metadata(topk_idx, topk_weights, num_topk, num_experts, part_idx, pack_handle,
                     local_idx, local_w, stream) -> int:
    return load().ep_pack_metadata(topk_idx, topk_weights, num_topk, num_experts, part_idx,
                                   ctypes.byref(pack_handle), local_idx, local_w, stream)


def rank_routing(topk_idx, num_experts: int, num_partitions: int):
    """Each token's distinct destination ranks, ascending, then -1: int64
    [T, min(K, P)] on the GPU."""
    import torch
    T, K = topk_idx.shape
    part = torch.empty((T, min(K, num_partitions)), dtype=torch.int64, device=topk_idx.device)
    _check(ep_rank_routing(_ptr(topk_idx.contiguous(), "i64", "topk_idx"), T, K, num_experts,
                           num_partitions, _ptr(part), _stream()))
    return part


def pack_for_ranks(x, topk_idx, topk_weights, num_experts: int, num_partitions: int,
                   use_fp8: bool = True):
    """The sender's side: rows packed destination-major (ascending token within
    each destination, one row per (token, destination)) with their metadata.
    Returns (send_x, send_scales or None, local_idx int64 [capacity, K],
    local_w fp32 [capacity, K], pack Layout, part_idx); the pack layout's
    num_tokens_per_expert[p] is the row count for destination p."""
    import torch
    part = rank_routing(topk_idx, num_experts, num_partitions)
    lay = get_dispatch_layout(part, num_partitions, num_partitions)
    send_x, send_scales, h = dispatch(x, None, lay, use_fp8)
    K = topk_idx.shape[1]
    cap = h.c.capacity_rows
    local_idx = torch.full((cap, K), -1, dtype=torch.int64, device=x.device)
    local_w = torch.zeros((cap, K), dtype=torch.float32, device=x.device)
    _check(ep_pack_metadata(_ptr(topk_idx.contiguous(), "i64", "topk_idx"),
                            _ptr(topk_weights.contiguous(), "f32", "topk_weights"), K,
                            num_experts, _ptr(part), h.c, _ptr(local_idx), _ptr(local_w),
                            _stream()))
    return send_x, send_scales, local_idx, local_w, lay, part
