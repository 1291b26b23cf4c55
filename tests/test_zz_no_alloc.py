"""fa_bwd_noalloc (the backward without a workspace argument) against fa_bwd.

Both go through the C ABI on the same inputs.  Calls follow each other on one
GPU, so each later call finds the device scratch as the earlier one left it;
the second call is smaller than the first.  Where both entry points choose the
same split of the backward, the results must be bit-identical; where the
fixed scratch holds fewer partials than a full workspace (the long one-head
case), they differ only in the order of fp32 sums and are compared at the
tolerances of the oracle comparisons.  The small cases are also compared with
the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_causal_amd import fa
from exact_attention_causal_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": dict(o=2e-2, grad=5e-2), "f32": dict(o=1e-4, grad=1e-4)}


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) / max(float(np.max(np.abs(b))), 1e-300)


def run(B, H, S, D, dtype, seed, with_oracle, causal=True):
    print(f"[no-alloc] B={B} H={H} S={S} D={D} dtype={dtype} seed={seed} causal={causal}", flush=True)
    dev = torch.device("cuda:0")
    code = fa.FA_BF16 if dtype == "bf16" else fa.FA_F32
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = make_inputs(B, H, S, D, dtype, seed=seed)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    dq_r, dk_r, dv_r, delta = fa.backward(qd, kd, vd, o, lse, dod, causal=causal)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    rc = fa.fa_bwd_noalloc(qd, kd, vd, dod, lse, delta, dq, dk, dv, B, H, S, D, scale, int(causal), code)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    torch.cuda.synchronize()

    # the split each entry point takes: fa_bwd with a full workspace (the plan) against the
    # split whose partials fit beside the base-2 L in the 64 MiB scratch
    _, plan = fa.fa_get_plan(B, H, S, D, code, 0)
    rows_bytes = (B * H * S * 4 + 255) // 256 * 256
    part = 3 * plan.bwd_chunks * B * H * S * D * 4 if plan.bwd_chunks > 1 else 0
    same_split = rows_bytes + part <= 64 << 20
    for n, got, ref in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        g, r = got.double().cpu().numpy(), ref.double().cpu().numpy()
        assert np.all(np.isfinite(g)), n
        if same_split:
            assert np.array_equal(g, r), (n, rel(g, r))
        else:
            assert rel(g, r) <= TOL[dtype]["grad"], (n, rel(g, r))
    print(f"[no-alloc] chunks {plan.bwd_chunks}, same split: {same_split}", flush=True)
    if with_oracle:
        ref = oracle.backward(*(x.double().numpy() for x in (q, k, v, do)), causal=causal)
        for n, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            e = rel(got.double().cpu().numpy(), ref[n])
            assert e <= TOL[dtype]["grad"], (n, e)


def test_noalloc_matches_fa_bwd_on_consecutive_calls():
    # split backward (8 chunks fit the scratch), then a smaller problem (3 chunks)
    run(1, 2, 1500, 128, "bf16", seed=701, with_oracle=True)
    run(1, 1, 300, 64, "bf16", seed=702, with_oracle=True)
    # fp32 (split into 6 chunks), then smaller again (2 chunks, the second of one row)
    run(2, 2, 333, 80, "f32", seed=703, with_oracle=True)
    run(1, 1, 65, 32, "f32", seed=704, with_oracle=True)


def test_noalloc_with_fewer_chunks_than_fa_bwd():
    # one head of 65536: a full workspace holds 2 chunks of partials (200 MB), the scratch none
    run(1, 1, 65536, 128, "bf16", seed=705, with_oracle=False)
    run(1, 3, 4096, 80, "bf16", seed=706, with_oracle=True)


def test_noalloc_non_causal():
    # without the mask (the split takes it into account): bf16 at CU/2 tiles (2 chunks, where the
    # causal plan asks for 3), then a smaller fp32 problem (4 chunks of 64 rows)
    run(1, 8, 4096, 64, "bf16", seed=707, with_oracle=True, causal=False)
    run(1, 2, 200, 80, "f32", seed=708, with_oracle=True, causal=False)
