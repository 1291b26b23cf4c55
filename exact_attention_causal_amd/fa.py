"""ctypes binding of the gfx950 attention library (include/fa.h).

The functions named like the C entry points (fa_fwd, fa_fwd_workspace_size,
fa_fwd_ws, fa_bwd_preprocess, fa_bwd_workspace_size, fa_bwd, fa_bwd_noalloc,
fa_fwd_partial, fa_merge, fa_bwd_partial, fa_get_plan, fa_strerror) only
marshal arguments: tensors
become device pointers, the stream becomes HIP's stream handle, and the status
code comes back unchanged.  ``forward`` / ``backward`` / ``attention_fwd_bwd``
are conveniences that allocate outputs with PyTorch (device memory is the
only thing PyTorch provides here) and raise on a non-zero status.

There is no fallback: if the shared library has not been built, or the
tensors are not on a GPU, every call raises.
"""
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# FA_LIB_PATH selects another build of the library (the host-sanitized build of
# build_sanitized.py, loaded with the sanitizer runtime preloaded)
LIB_PATH = os.environ.get("FA_LIB_PATH") or os.path.join(HERE, "libfa_mi355x.so")

FA_F32 = 0
FA_BF16 = 1
FA_OK = 0
FA_EINVAL = -1
FA_EUNSUPPORTED = -2
FA_EALIGN = -3
FA_EWORKSPACE = -4
FA_EHIP = -5
FA_ESCRATCH = -6

#: head dimensions with built kernels
HEAD_DIMS = (16, 32, 64, 80, 96, 128)

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


class Plan(ctypes.Structure):
    """fa_plan: the tile configuration the library picks for a problem (include/fa.h)."""
    _fields_ = [("num_cu", ctypes.c_int), ("fwd_block_queries", ctypes.c_int),
                ("fwd_key_groups", ctypes.c_int), ("fwd_key_tile", ctypes.c_int),
                ("fwd_band", ctypes.c_int),
                ("bwd_chunks", ctypes.c_int), ("bwd_chunk_rows", ctypes.c_int)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class FaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status}: {fa_strerror(status)}")


def load_library():
    """Load libfa_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_attention_causal_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_fwd.restype = _i
    lib.fa_fwd_workspace_size.argtypes = [_i, _i, _i, _i, _i]
    lib.fa_fwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_ws.argtypes = [_vp] * 6 + [ctypes.c_size_t, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_fwd_ws.restype = _i
    lib.fa_bwd_preprocess.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    lib.fa_bwd_preprocess.restype = _i
    lib.fa_bwd_workspace_size.argtypes = [_i, _i, _i, _i, _i]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [_vp] * 10 + [ctypes.c_size_t, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_bwd.restype = _i
    lib.fa_fwd_partial.argtypes = [_vp] * 5 + [_i] * 5 + [_f, _i, _i, _i, _i, _vp]
    lib.fa_fwd_partial.restype = _i
    lib.fa_merge.argtypes = [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp]
    lib.fa_merge.restype = _i
    lib.fa_bwd_partial.argtypes = [_vp] * 9 + [_i] * 6 + [_f, _i, _i, _i, _vp]
    lib.fa_bwd_partial.restype = _i
    lib.fa_bwd_noalloc.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_bwd_noalloc.restype = _i
    lib.fa_get_plan.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(Plan)]
    lib.fa_get_plan.restype = _i
    lib.fa_strerror.argtypes = [_i]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _on_stream(stream):
    """Context making the stream of a stream argument (a torch stream or a raw HIP
    handle; None: the current stream) current for torch's allocations and copies."""
    if stream is None or isinstance(stream, torch.cuda.Stream):
        return torch.cuda.stream(stream)
    return torch.cuda.stream(torch.cuda.ExternalStream(int(stream)))


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------- C entry points ---

def fa_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype, stream=None):
    return load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D,
                                 float(scale), int(causal), int(dtype), _stream(stream))


def fa_fwd_workspace_size(B, H, S, D, dtype):
    return int(load_library().fa_fwd_workspace_size(B, H, S, D, int(dtype)))


def fa_fwd_ws(q, k, v, o, lse, workspace, workspace_bytes, B, H, S, D, scale, causal, dtype,
              stream=None):
    return load_library().fa_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                    int(workspace_bytes), B, H, S, D, float(scale), int(causal),
                                    int(dtype), _stream(stream))


def fa_bwd_preprocess(o, dout, delta, B, H, S, D, dtype, stream=None):
    return load_library().fa_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(delta), B, H, S, D,
                                            int(dtype), _stream(stream))


def fa_bwd_workspace_size(B, H, S, D, dtype):
    return int(load_library().fa_bwd_workspace_size(B, H, S, D, int(dtype)))


def fa_bwd(q, k, v, dout, lse, delta, dq, dk, dv, workspace, workspace_bytes, B, H, S, D, scale,
           causal, dtype, stream=None):
    return load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                 int(workspace_bytes), B, H, S, D, float(scale), int(causal),
                                 int(dtype), _stream(stream))


def fa_bwd_noalloc(q, k, v, dout, lse, delta, dq, dk, dv, B, H, S, D, scale, causal, dtype,
                   stream=None):
    return load_library().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                         _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), B, H, S, D,
                                         float(scale), int(causal), int(dtype), _stream(stream))


def fa_get_plan(B, H, S, D, dtype, num_cu=0):
    """(status, Plan) for a problem on a device with num_cu compute units (0: the current one)."""
    plan = Plan()
    rc = load_library().fa_get_plan(B, H, S, D, int(dtype), int(num_cu), ctypes.byref(plan))
    return rc, plan


def fa_fwd_partial(q, k, v, o_parts, lse_parts, B, H, Sq, Sk, D, scale, causal, q_offset, n_split,
                   dtype, stream=None):
    return load_library().fa_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o_parts), _ptr(lse_parts),
                                         B, H, Sq, Sk, D, float(scale), int(causal), int(q_offset),
                                         int(n_split), int(dtype), _stream(stream))


def fa_merge(o_parts, lse_parts, n_parts, o, lse, B, H, S, D, dtype, stream=None):
    return load_library().fa_merge(_ptr(o_parts), _ptr(lse_parts), int(n_parts), _ptr(o), _ptr(lse),
                                   B, H, S, D, int(dtype), _stream(stream))


def fa_bwd_partial(q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, accumulate, B, H, Sq, Sk, D,
                   scale, causal, q_offset, dtype, stream=None):
    return load_library().fa_bwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                         _ptr(delta), _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc),
                                         int(accumulate), B, H, Sq, Sk, D, float(scale),
                                         int(causal), int(q_offset), int(dtype), _stream(stream))


def fa_strerror(status):
    return load_library().fa_strerror(int(status)).decode()


# ------------------------------------------------------------ helpers ---

def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return FA_BF16
    if t == torch.float32:
        return FA_F32
    raise ValueError(f"unsupported dtype {t}")


def _check(status, where):
    if status != FA_OK:
        raise FaError(status, where)


def _shape(q):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("expected [B, H, S, D] tensors")
    return tuple(q.shape)


def _like(name, x, shape, dtype, device, contiguous=False):
    """Raise ValueError unless x has this shape, dtype and device (and, for a buffer the
    library writes into, is contiguous): the kernels take every size from q, so a
    mismatched tensor would be read or written out of its bounds."""
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if x.dtype != dtype:
        raise ValueError(f"{name} has dtype {x.dtype}, expected {dtype}")
    if x.device != device:
        raise ValueError(f"{name} is on {x.device}, expected {device}")
    if contiguous and not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous (the library writes it in place)")


def _on_gpu(x):
    if not x.is_cuda:
        raise ValueError("tensors must be on a GPU (there is no CPU path)")


def _workspace(workspace, device):
    if not isinstance(workspace, torch.Tensor) or workspace.device != device \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace.numel() * workspace.element_size()


def forward(q, k, v, causal=True, scale=None, out=None, lse=None, workspace=None, stream=None):
    """O, L for [B, H, S, D] q, k, v (bf16 or fp32, same shape) on the GPU.

    A caller's ``out`` ([B, H, S, D], q's dtype) and ``lse`` ([B, H, S] fp32) must be
    contiguous tensors on q's device; they are overwritten.  ``workspace``: None
    allocates what fa_fwd_workspace_size asks for and calls fa_fwd_ws (which splits
    the keys of few-tile problems); False calls fa_fwd; a contiguous tensor on q's
    device is passed to fa_fwd_ws as it is.
    """
    B, H, S, D = _shape(q)
    code = dtype_code(q.dtype)
    for n, x in (("k", k), ("v", v)):
        _like(n, x, q.shape, q.dtype, q.device)
    if out is not None:
        _like("out", out, q.shape, q.dtype, q.device, contiguous=True)
    if lse is not None:
        _like("lse", lse, (B, H, S), torch.float32, q.device, contiguous=True)
    ws_bytes = 0
    if workspace is not None and workspace is not False:
        ws_bytes = _workspace(workspace, q.device)
    _on_gpu(q)
    # temporaries, contiguous copies and outputs are allocated on the stream the
    # kernels run on, so the caching allocator never reuses them early
    with _on_stream(stream):
        q, k, v = (x.contiguous() for x in (q, k, v))
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, S), device=q.device, dtype=torch.float32)
        if workspace is False:
            _check(fa_fwd(q, k, v, out, lse, B, H, S, D, scale, causal, code, stream), "fa_fwd")
            return out, lse
        if workspace is None:
            ws_bytes = fa_fwd_workspace_size(B, H, S, D, code)
            if ws_bytes > 0:
                workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
        _check(fa_fwd_ws(q, k, v, out, lse, workspace, ws_bytes, B, H, S, D, scale, causal, code, stream),
               "fa_fwd_ws")
        return out, lse


def backward(q, k, v, o, lse, dout, causal=True, scale=None, delta=None, grads=None,
             workspace=None, stream=None):
    """dQ, dK, dV (and delta) for the forward pass that produced o, lse.

    q, k, v, o, dout share one shape and dtype; lse is [B, H, S] fp32.  A caller's
    ``delta`` ([B, H, S] fp32), ``grads`` (three tensors shaped and typed like q) and
    ``workspace`` must be contiguous tensors on q's device.
    """
    B, H, S, D = _shape(q)
    code = dtype_code(q.dtype)
    for n, x in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _like(n, x, q.shape, q.dtype, q.device)
    _like("lse", lse, (B, H, S), torch.float32, q.device)
    if delta is not None:
        _like("delta", delta, (B, H, S), torch.float32, q.device, contiguous=True)
    if grads is not None:
        if len(grads) != 3:
            raise ValueError("grads must be (dq, dk, dv)")
        for n, x in zip(("dq", "dk", "dv"), grads):
            _like(n, x, q.shape, q.dtype, q.device, contiguous=True)
    if workspace is not None:
        ws_bytes = _workspace(workspace, q.device)
    _on_gpu(q)
    # temporaries, contiguous copies and outputs are allocated on the stream the
    # kernels run on, so the caching allocator never reuses them early
    with _on_stream(stream):
        q, k, v, o, dout, lse = (x.contiguous() for x in (q, k, v, o, dout, lse))
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        if delta is None:
            delta = torch.empty((B, H, S), device=q.device, dtype=torch.float32)
        if grads is None:
            grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        dq, dk, dv = grads
        _check(fa_bwd_preprocess(o, dout, delta, B, H, S, D, code, stream), "fa_bwd_preprocess")
        if workspace is None:
            ws_bytes = fa_bwd_workspace_size(B, H, S, D, code)
            if ws_bytes:
                workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
        # (a caller's smaller workspace disables the split backward)
        _check(fa_bwd(q, k, v, dout, lse, delta, dq, dk, dv, workspace, ws_bytes, B, H, S, D, scale,
                      causal, code, stream), "fa_bwd")
        return dq, dk, dv, delta


def split_chunk(Sk, n_split):
    """Keys per chunk of fa_fwd_partial: 64 * ceil(Sk / (64 * n_split))."""
    return 64 * ((Sk + 64 * n_split - 1) // (64 * n_split))


def _keys(q, k, v):
    """Sk of key/value tensors that match q [B, H, Sq, D] in B, H, D, dtype and device."""
    B, H, _, D = _shape(q)
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("expected [B, H, Sk, D] keys")
    Sk = k.shape[2]
    for n, x in (("k", k), ("v", v)):
        _like(n, x, (B, H, Sk, D), q.dtype, q.device)
    return Sk


def forward_partial(q, k, v, causal=True, scale=None, q_offset=0, n_split=1, stream=None):
    """fp32 (O, L) of q [B,H,Sq,D] over each key chunk of k, v [B,H,Sk,D].

    Returns o_parts [n_split, B, H, Sq, D] and lse_parts [n_split, B, H, Sq]; query i
    sits q_offset positions after key 0 (see fa_fwd_partial in include/fa.h).
    """
    B, H, Sq, D = _shape(q)
    code = dtype_code(q.dtype)
    Sk = _keys(q, k, v)
    _on_gpu(q)
    # temporaries, contiguous copies and outputs are allocated on the stream the
    # kernels run on, so the caching allocator never reuses them early
    with _on_stream(stream):
        q, k, v = (x.contiguous() for x in (q, k, v))
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        o_parts = torch.empty((n_split, B, H, Sq, D), device=q.device, dtype=torch.float32)
        lse_parts = torch.empty((n_split, B, H, Sq), device=q.device, dtype=torch.float32)
        _check(fa_fwd_partial(q, k, v, o_parts, lse_parts, B, H, Sq, Sk, D, scale, causal, q_offset,
                              n_split, code, stream), "fa_fwd_partial")
        return o_parts, lse_parts


def merge(o_parts, lse_parts, dtype=torch.bfloat16, stream=None):
    """Merge [n, B, H, S, D] fp32 partial outputs and [n, B, H, S] L into (O in dtype, L)."""
    if not isinstance(o_parts, torch.Tensor) or o_parts.dim() != 5:
        raise ValueError("expected [n, B, H, S, D] partial outputs")
    n, B, H, S, D = o_parts.shape
    code = dtype_code(dtype)
    _like("o_parts", o_parts, o_parts.shape, torch.float32, o_parts.device)
    _like("lse_parts", lse_parts, (n, B, H, S), torch.float32, o_parts.device)
    _on_gpu(o_parts)
    # temporaries, contiguous copies and outputs are allocated on the stream the
    # kernels run on, so the caching allocator never reuses them early
    with _on_stream(stream):
        o_parts, lse_parts = o_parts.contiguous(), lse_parts.contiguous()
        o = torch.empty((B, H, S, D), device=o_parts.device, dtype=dtype)
        lse = torch.empty((B, H, S), device=o_parts.device, dtype=torch.float32)
        _check(fa_merge(o_parts, lse_parts, n, o, lse, B, H, S, D, code, stream), "fa_merge")
        return o, lse


def forward_split_kv(q, k, v, n_split, causal=True, scale=None, stream=None):
    """Self-attention forward with the keys split over n_split chunks, then merged."""
    o_parts, lse_parts = forward_partial(q, k, v, causal, scale, 0, n_split, stream)
    return merge(o_parts, lse_parts, q.dtype, stream)


def backward_partial(q, k, v, dout, lse, delta, causal=True, scale=None, q_offset=0, grads=None,
                     stream=None):
    """fp32 gradient contributions of the key set k, v [B,H,Sk,D] for q, dout [B,H,Sq,D].

    lse and delta [B,H,Sq] are the whole attention's L and Delta; query i sits q_offset
    positions after key 0 (see fa_bwd_partial in include/fa.h).  With grads = (dq, dk, dv)
    (fp32) the contributions are added to them; otherwise new tensors are returned.
    """
    B, H, Sq, D = _shape(q)
    code = dtype_code(q.dtype)
    Sk = _keys(q, k, v)
    _like("dout", dout, q.shape, q.dtype, q.device)
    _like("lse", lse, (B, H, Sq), torch.float32, q.device)
    _like("delta", delta, (B, H, Sq), torch.float32, q.device)
    accumulate = grads is not None
    if grads is not None:
        if len(grads) != 3:
            raise ValueError("grads must be (dq, dk, dv)")
        for n, x, shp in zip(("dq", "dk", "dv"), grads, ((B, H, Sq, D), (B, H, Sk, D), (B, H, Sk, D))):
            _like(n, x, shp, torch.float32, q.device, contiguous=True)
    _on_gpu(q)
    # temporaries, contiguous copies and outputs are allocated on the stream the
    # kernels run on, so the caching allocator never reuses them early
    with _on_stream(stream):
        q, k, v, dout = (x.contiguous() for x in (q, k, v, dout))
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        if grads is None:
            f32 = dict(device=q.device, dtype=torch.float32)
            grads = (torch.empty((B, H, Sq, D), **f32), torch.empty((B, H, Sk, D), **f32),
                     torch.empty((B, H, Sk, D), **f32))
        dq, dk, dv = grads
        _check(fa_bwd_partial(q, k, v, dout, lse.contiguous(), delta.contiguous(), dq, dk, dv,
                              accumulate, B, H, Sq, Sk, D, scale, causal, q_offset,
                              code, stream), "fa_bwd_partial")
        return dq, dk, dv


# ------------------------------------------------------------- autograd ---

class FlashAttention(torch.autograd.Function):
    """Attention as a differentiable op (CS336 Assignment 2 handout, section 4.2.2 (a)).

    forward(q, k, v, is_causal=False, scale=None) returns O and keeps only
    q, k, v, O and the logsumexp L for the backward, which recomputes P from L
    (handout Algorithm 2).  Inputs are [B, H, S, D] or [B, S, D] (one head)
    bf16 or fp32 GPU tensors; the default scale is 1/sqrt(D).
    """

    @staticmethod
    def forward(ctx, q, k, v, is_causal=False, scale=None):
        three = q.dim() == 3
        if three:
            q, k, v = (x.unsqueeze(1) for x in (q, k, v))
        o, lse = forward(q, k, v, causal=bool(is_causal), scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.is_causal, ctx.scale, ctx.three = bool(is_causal), scale, three
        return o.squeeze(1) if three else o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if ctx.three:
            do = do.unsqueeze(1)
        dq, dk, dv, _ = backward(q, k, v, o, lse, do, causal=ctx.is_causal, scale=ctx.scale)
        if ctx.three:
            dq, dk, dv = (x.squeeze(1) for x in (dq, dk, dv))
        return dq, dk, dv, None, None


def flash_attention(q, k, v, is_causal=False, scale=None):
    """Differentiable attention through the HIP kernels (see FlashAttention)."""
    return FlashAttention.apply(q, k, v, is_causal, scale)
