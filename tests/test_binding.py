"""The Python binding rejects mismatched tensors before anything reaches the library.

The kernels take every size from q, so a key tensor of another length, a
caller's output of the wrong shape or dtype, or tensors on different devices
would be read or written out of their bounds on the GPU.  Each case here is
refused with ValueError on the host (CPU tensors: the checks run before the
device check, so these tests need no GPU and launch nothing).
"""
import pytest
import torch

fa = pytest.importorskip("exact_attention_causal_amd.fa")

B, H, S, D = 1, 2, 64, 16


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def qkv(dtype=torch.bfloat16):
    return t(B, H, S, D, dtype=dtype), t(B, H, S, D, dtype=dtype), t(B, H, S, D, dtype=dtype)


def raises(match, f, *a, **kw):
    with pytest.raises(ValueError, match=match):
        f(*a, **kw)


def test_forward_mismatches():
    q, k, v = qkv()
    raises("k has shape", fa.forward, q, t(B, H, S - 1, D), v)           # shorter keys
    raises("v has shape", fa.forward, q, k, t(B, H, S, D + 16))
    raises("k has dtype", fa.forward, q, k.float(), v)                   # fp32 k with bf16 q
    raises("out has shape", fa.forward, q, k, v, out=t(B, H, S, D // 2))
    raises("out has dtype", fa.forward, q, k, v, out=t(B, H, S, D, dtype=torch.float32))
    raises("out must be contiguous", fa.forward, q, k, v, out=t(B, H, D, S).transpose(2, 3))
    raises("lse has shape", fa.forward, q, k, v, lse=t(B, H, S + 1, dtype=torch.float32))
    raises("lse has dtype", fa.forward, q, k, v, lse=t(B, H, S))
    raises(r"expected \[B, H, S, D\]", fa.forward, t(H, S, D), k, v)
    raises("unsupported dtype", fa.forward, *(x.half() for x in (q, k, v)))
    raises("workspace must be", fa.forward, q, k, v, workspace=b"\0" * 64)
    # consistent tensors reach the device check (there is no CPU path)
    raises("must be on a GPU", fa.forward, q, k, v)


def test_backward_mismatches():
    q, k, v = qkv()
    o, do = t(B, H, S, D), t(B, H, S, D)
    lse = t(B, H, S, dtype=torch.float32)
    g = (t(B, H, S, D), t(B, H, S, D), t(B, H, S, D))
    raises("k has shape", fa.backward, q, t(B, H, 2 * S, D), v, o, lse, do)
    raises("o has dtype", fa.backward, q, k, v, o.float(), lse, do)
    raises("dout has shape", fa.backward, q, k, v, o, lse, t(B, H, S, D + 16))
    raises("lse has shape", fa.backward, q, k, v, o, t(B, H, S - 1, dtype=torch.float32), do)
    raises("lse has dtype", fa.backward, q, k, v, o, lse.bfloat16(), do)
    raises("delta has shape", fa.backward, q, k, v, o, lse, do, delta=t(B, H, 1, dtype=torch.float32))
    raises("dk has shape", fa.backward, q, k, v, o, lse, do, grads=(g[0], t(B, H, S - 1, D), g[2]))
    raises("dv has dtype", fa.backward, q, k, v, o, lse, do, grads=(g[0], g[1], g[2].float()))
    raises("dq must be contiguous", fa.backward, q, k, v, o, lse, do,
           grads=(t(B, H, D, S).transpose(2, 3), g[1], g[2]))
    raises("grads must be", fa.backward, q, k, v, o, lse, do, grads=g[:2])
    raises("workspace must be", fa.backward, q, k, v, o, lse, do, workspace=b"\0" * 64)
    raises("must be on a GPU", fa.backward, q, k, v, o, lse, do)


def test_partial_and_merge_mismatches():
    q = t(B, H, S, D)
    k, v = t(B, H, 3 * S, D), t(B, H, 3 * S, D)
    raises("v has shape", fa.forward_partial, q, k, t(B, H, 2 * S, D))
    raises("k has shape", fa.forward_partial, q, t(B, H + 1, 3 * S, D), v)
    raises("k has dtype", fa.forward_partial, q, k.float(), v.float())
    raises("must be on a GPU", fa.forward_partial, q, k, v)

    op, lp = t(3, B, H, S, D, dtype=torch.float32), t(3, B, H, S, dtype=torch.float32)
    raises("lse_parts has shape", fa.merge, op, t(2, B, H, S, dtype=torch.float32))
    raises("o_parts has dtype", fa.merge, op.bfloat16(), lp)
    raises(r"expected \[n, B, H, S, D\]", fa.merge, t(B, H, S, D, dtype=torch.float32), lp)
    raises("must be on a GPU", fa.merge, op, lp)

    do = t(B, H, S, D)
    lse, delta = t(B, H, S, dtype=torch.float32), t(B, H, S, dtype=torch.float32)
    f32 = dict(dtype=torch.float32)
    raises("dout has shape", fa.backward_partial, q, k, v, t(B, H, 3 * S, D), lse, delta)
    raises("delta has shape", fa.backward_partial, q, k, v, do, lse, t(B, H, 3 * S, **f32))
    raises("dk has shape", fa.backward_partial, q, k, v, do, lse, delta,
           grads=(t(B, H, S, D, **f32), t(B, H, S, D, **f32), t(B, H, 3 * S, D, **f32)))
    raises("dq has dtype", fa.backward_partial, q, k, v, do, lse, delta,
           grads=(t(B, H, S, D), t(B, H, 3 * S, D, **f32), t(B, H, 3 * S, D, **f32)))
    raises("must be on a GPU", fa.backward_partial, q, k, v, do, lse, delta)
