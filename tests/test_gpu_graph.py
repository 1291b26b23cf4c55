"""A whole forward+backward step captured as a HIP graph and replayed.

fa_fwd (or fa_fwd_ws with a workspace the caller holds), fa_bwd_preprocess and
fa_bwd (with a workspace the caller holds) or fa_bwd_noalloc allocate nothing,
synchronise nothing and enqueue only kernels on the caller's stream, so one
step can be captured (torch.cuda.graph drives the capture on its own stream)
and replayed.  A replay re-runs the step on whatever the captured buffers hold
at that moment.  The kernels are deterministic (no atomics, sums in a fixed
order), so every replay must equal the eager step bit for bit: replays
separated by eager work and synchronisations, and a replay after new values
are copied into the captured inputs.  Outputs are overwritten with NaN before
each replay, so a replay that skipped a kernel fails.
"""
import math

import pytest
import torch

from exact_attention_causal_amd import fa
from exact_attention_causal_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

# (B, H, S, D, dtype, forward entry point, backward entry point)
CASES = [
    (4, 12, 512, 64, "bf16", "fa_fwd", "fa_bwd"),            # many heads
    (1, 1, 4096, 128, "bf16", "fa_fwd_ws", "fa_bwd"),        # one head: split forward and backward
    (1, 2, 257, 64, "f32", "fa_fwd", "fa_bwd"),              # fp32, ragged length
    (2, 1, 3000, 64, "f32", "fa_fwd_ws", "fa_bwd"),          # fp32 split forward and backward
    (2, 3, 1000, 80, "bf16", "fa_fwd", "fa_bwd_noalloc"),    # the allocation-free backward, 16-row tails
]
NAMES = ("o", "lse", "delta", "dq", "dk", "dv")


class Step:
    """Preallocated buffers of one step and the calls that enqueue it on the current stream."""

    def __init__(self, B, H, S, D, dtype, fwd, bwd, seed):
        dev = torch.device("cuda:0")
        self.dims = (B, H, S, D)
        self.code = fa.FA_BF16 if dtype == "bf16" else fa.FA_F32
        self.scale = 1.0 / math.sqrt(D)
        self.fwd, self.bwd = fwd, bwd
        self.inputs = [x.to(dev) for x in make_inputs(B, H, S, D, dtype, seed=seed)]
        q = self.inputs[0]
        self.o, self.dq, self.dk, self.dv = (torch.empty_like(q) for _ in range(4))
        self.lse = torch.empty((B, H, S), device=dev, dtype=torch.float32)
        self.delta = torch.empty_like(self.lse)
        self.ws_bytes = fa.fa_bwd_workspace_size(B, H, S, D, self.code)
        self.ws = torch.empty(max(self.ws_bytes, 1), device=dev, dtype=torch.uint8)
        self.fws_bytes = fa.fa_fwd_workspace_size(B, H, S, D, self.code)
        assert fwd == "fa_fwd" or self.fws_bytes > 0   # (the fa_fwd_ws cases do split)
        self.fws = torch.empty(max(self.fws_bytes, 1), device=dev, dtype=torch.uint8)

    def outputs(self):
        return (self.o, self.lse, self.delta, self.dq, self.dk, self.dv)

    def run(self):
        B, H, S, D = self.dims
        q, k, v, do = self.inputs
        if self.fwd == "fa_fwd":
            rc = fa.fa_fwd(q, k, v, self.o, self.lse, B, H, S, D, self.scale, 1, self.code)
        else:
            rc = fa.fa_fwd_ws(q, k, v, self.o, self.lse, self.fws, self.fws_bytes, B, H, S, D,
                              self.scale, 1, self.code)
        assert rc == 0, fa.fa_strerror(rc)
        rc = fa.fa_bwd_preprocess(self.o, do, self.delta, B, H, S, D, self.code)
        assert rc == 0, fa.fa_strerror(rc)
        if self.bwd == "fa_bwd":
            rc = fa.fa_bwd(q, k, v, do, self.lse, self.delta, self.dq, self.dk, self.dv, self.ws,
                           self.ws_bytes, B, H, S, D, self.scale, 1, self.code)
        else:
            rc = fa.fa_bwd_noalloc(q, k, v, do, self.lse, self.delta, self.dq, self.dk, self.dv,
                                   B, H, S, D, self.scale, 1, self.code)
        assert rc == 0, fa.fa_strerror(rc)

    def poison(self):
        for t in self.outputs():
            t.fill_(float("nan"))


def assert_same(got, want, what):
    for name, a, b in zip(NAMES, got, want):
        assert torch.equal(a, b), f"{what}: {name} differs from the eager step"


@pytest.mark.parametrize("B,H,S,D,dtype,fwd,bwd", CASES)
def test_step_graph_replays_match_eager(B, H, S, D, dtype, fwd, bwd):
    print(f"[graph] B={B} H={H} S={S} D={D} dtype={dtype} {fwd} {bwd}", flush=True)
    dev = torch.device("cuda:0")
    st = Step(B, H, S, D, dtype, fwd, bwd, seed=31)
    st.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in st.outputs()]
    assert all(torch.isfinite(t).all() for t in ref[3:])

    st.poison()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work of the program's own between replays
        x = torch.randn(384, 384, device=dev)
        assert torch.isfinite((x @ x).sum()).item()
        st.poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(st.outputs(), ref, f"replay {rep}")

    # new values in the captured inputs: the replay computes on them
    for t, x in zip(st.inputs, make_inputs(B, H, S, D, dtype, seed=32)):
        t.copy_(x.to(dev))
    st.run()
    torch.cuda.synchronize()
    ref2 = [t.clone() for t in st.outputs()]
    assert not torch.equal(ref2[0], ref[0])
    st.poison()
    g.replay()
    torch.cuda.synchronize()
    assert_same(st.outputs(), ref2, "replay on new inputs")
