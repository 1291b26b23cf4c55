"""ctypes binding of the gfx950 attention library (include/fa.h).

The functions named like the C entry points (fa_fwd, fa_bwd_preprocess,
fa_bwd_workspace_size, fa_bwd, fa_fwd_partial, fa_merge, fa_bwd_partial, fa_strerror) only marshal arguments: tensors
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
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")

FA_F32 = 0
FA_BF16 = 1
FA_OK = 0
FA_EINVAL = -1
FA_EUNSUPPORTED = -2
FA_EALIGN = -3
FA_EWORKSPACE = -4
FA_EHIP = -5

#: head dimensions with built kernels
HEAD_DIMS = (16, 32, 64, 80, 96, 128)

_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


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
    if q.dim() != 4:
        raise ValueError("expected [B, H, S, D] tensors")
    if not q.is_cuda:
        raise ValueError("tensors must be on a GPU (there is no CPU path)")
    return tuple(q.shape)


def forward(q, k, v, causal=True, scale=None, out=None, lse=None, stream=None):
    """O, L for contiguous [B, H, S, D] q, k, v (bf16 or fp32) on the GPU."""
    B, H, S, D = _shape(q)
    q, k, v = (x.contiguous() for x in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), device=q.device, dtype=torch.float32)
    _check(fa_fwd(q, k, v, out, lse, B, H, S, D, scale, causal, dtype_code(q.dtype), stream),
           "fa_fwd")
    return out, lse


def backward(q, k, v, o, lse, dout, causal=True, scale=None, delta=None, grads=None,
             workspace=None, stream=None):
    """dQ, dK, dV (and delta) for the forward pass that produced o, lse."""
    B, H, S, D = _shape(q)
    q, k, v, o, dout = (x.contiguous() for x in (q, k, v, o, dout))
    code = dtype_code(q.dtype)
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
    else:  # a caller's workspace (a smaller one disables the split backward)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(fa_bwd(q, k, v, dout, lse, delta, dq, dk, dv, workspace, ws_bytes, B, H, S, D, scale,
                  causal, code, stream), "fa_bwd")
    return dq, dk, dv, delta


def split_chunk(Sk, n_split):
    """Keys per chunk of fa_fwd_partial: 64 * ceil(Sk / (64 * n_split))."""
    return 64 * ((Sk + 64 * n_split - 1) // (64 * n_split))


def forward_partial(q, k, v, causal=True, scale=None, q_offset=0, n_split=1, stream=None):
    """fp32 (O, L) of q [B,H,Sq,D] over each key chunk of k, v [B,H,Sk,D].

    Returns o_parts [n_split, B, H, Sq, D] and lse_parts [n_split, B, H, Sq]; query i
    sits q_offset positions after key 0 (see fa_fwd_partial in include/fa.h).
    """
    B, H, Sq, D = _shape(q)
    Sk = k.shape[2]
    q, k, v = (x.contiguous() for x in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o_parts = torch.empty((n_split, B, H, Sq, D), device=q.device, dtype=torch.float32)
    lse_parts = torch.empty((n_split, B, H, Sq), device=q.device, dtype=torch.float32)
    _check(fa_fwd_partial(q, k, v, o_parts, lse_parts, B, H, Sq, Sk, D, scale, causal, q_offset,
                          n_split, dtype_code(q.dtype), stream), "fa_fwd_partial")
    return o_parts, lse_parts


def merge(o_parts, lse_parts, dtype=torch.bfloat16, stream=None):
    """Merge [n, B, H, S, D] fp32 partial outputs and [n, B, H, S] L into (O in dtype, L)."""
    n, B, H, S, D = o_parts.shape
    if not o_parts.is_cuda:
        raise ValueError("tensors must be on a GPU (there is no CPU path)")
    o_parts, lse_parts = o_parts.contiguous(), lse_parts.contiguous()
    o = torch.empty((B, H, S, D), device=o_parts.device, dtype=dtype)
    lse = torch.empty((B, H, S), device=o_parts.device, dtype=torch.float32)
    _check(fa_merge(o_parts, lse_parts, n, o, lse, B, H, S, D, dtype_code(dtype), stream), "fa_merge")
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
    Sk = k.shape[2]
    q, k, v, dout = (x.contiguous() for x in (q, k, v, dout))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    accumulate = grads is not None
    if grads is None:
        f32 = dict(device=q.device, dtype=torch.float32)
        grads = (torch.empty((B, H, Sq, D), **f32), torch.empty((B, H, Sk, D), **f32),
                 torch.empty((B, H, Sk, D), **f32))
    dq, dk, dv = grads
    for g in grads:
        if g.dtype != torch.float32 or not g.is_contiguous():
            raise ValueError("gradient accumulators must be contiguous fp32 tensors")
    _check(fa_bwd_partial(q, k, v, dout, lse.contiguous(), delta.contiguous(), dq, dk, dv,
                          accumulate, B, H, Sq, Sk, D, scale, causal, q_offset,
                          dtype_code(q.dtype), stream), "fa_bwd_partial")
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
