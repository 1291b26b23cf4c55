"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Error metric (per tensor): max |gpu - oracle| / max |oracle|; L is compared
in absolute terms.  Bounds: bf16 O 2e-2, dQ/dK/dV 5e-2; fp32 O and grads
1e-4; L 1e-3 absolute.

Small and mid workloads are compared element by element on every output.
The two long workloads (S = 16000, D = 80 and S = 65536, D = 128) run in the
launch configuration the benchmark times; the oracle evaluates a seeded
sample of query rows (O, L, dQ) and of key rows (dK, dV, which need the
oracle's own L and D for every later query of that head), and whole-tensor
identities that hold at any size are checked on all rows.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_causal_amd import fa
from exact_attention_causal_amd.inputs import (WORKLOADS, make_inputs, sample_head_rows,
                                               workload_inputs)

pytestmark = pytest.mark.gpu

TOL = {
    "bf16": dict(o=2e-2, grad=5e-2, lse=1e-3),
    "f32": dict(o=1e-4, grad=1e-4, lse=1e-3),
}


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    denom = float(np.max(np.abs(b))) if b.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return float(np.max(np.abs(a - b))) / denom


def absdiff(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    fa.load_library()
    return torch.device("cuda:0")


def run_gpu(q, k, v, do, causal=True, scale=None):
    """fwd + preprocess + bwd through the C ABI; returns CPU fp64 numpy arrays."""
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    out = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)
    return {n: t.double().cpu().numpy() for n, t in out.items()}


def check_full(q, k, v, do, dtype, causal=True, scale=None, label=""):
    print(f"[parity] {label} shape={tuple(q.shape)} dtype={dtype} causal={causal}", flush=True)
    g = run_gpu(q, k, v, do, causal, scale)
    r = oracle.backward(*(x.double().numpy() for x in (q, k, v, do)), scale=scale,
                        causal=causal)
    return compare(g, r, dtype, label)


def compare(g, r, dtype, label):
    tol = TOL[dtype]
    errs = dict(o=rel(g["o"], r["o"]), lse=absdiff(g["lse"], r["lse"]),
                dq=rel(g["dq"], r["dq"]), dk=rel(g["dk"], r["dk"]), dv=rel(g["dv"], r["dv"]),
                delta=rel(g["delta"], r["delta_o"]))
    print(f"[parity] {label} errors {errs}", flush=True)
    assert errs["o"] <= tol["o"], errs
    assert errs["lse"] <= tol["lse"], errs
    for n in ("dq", "dk", "dv"):
        assert errs[n] <= tol["grad"], (n, errs)
    # delta is the fp32 rowsum of the GPU's own (rounded) O; it must sit inside the grad budget
    assert errs["delta"] <= tol["grad"], errs
    return errs


# --------------------------------------------------------- the workloads ---

@pytest.mark.parametrize("name", ["f32_b1h2_s128_d64", "bf16_b4h12_s512_d64",
                                  "bf16_b4h16_s2048_d64_peaky"])
def test_workload_full(name):
    w = WORKLOADS[name]
    q, k, v, do = workload_inputs(w)
    check_full(q, k, v, do, w.dtype, causal=True, scale=w.scale, label=name)


def _sampled_check(w, heads=4, per_head=64):
    """Sampled oracle comparison at full size (the benchmark's launch shapes).

    A few seeded heads, a seeded set of rows in each (always the sequence ends and tile
    edges): O, L and dQ at those query rows and dK, dV at the same key rows.  dK_j and
    dV_j sum over every query i >= j, so the oracle first computes its own L and D for
    every row of each sampled head.  Whole-tensor identities cover every row.
    """
    print(f"[parity] sampled {w.name}: {heads} heads x {per_head} rows", flush=True)
    q, k, v, do = workload_inputs(w)
    g = run_gpu(q, k, v, do, causal=True, scale=w.scale)
    tol = TOL[w.dtype]
    qn, kn, vn, don = (x.double().numpy().reshape(w.B * w.H, w.S, w.D) for x in (q, k, v, do))
    go = {n: g[n].reshape(w.B * w.H, w.S, -1) for n in ("o", "dq", "dk", "dv")}
    glse = g["lse"].reshape(w.B * w.H, w.S)

    ref = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    got = {n: [] for n in ref}
    for hh, rows in sample_head_rows(w.B * w.H, w.S, heads, per_head):
        print(f"[parity] sampled {w.name}: head {hh} oracle statistics", flush=True)
        lse_full, del_full = oracle.head_stats(qn[hh], kn[hh], vn[hh], don[hh], scale=w.scale)
        o, lse, dq = oracle.rows(qn[hh], kn[hh], vn[hh], don[hh], rows, scale=w.scale)
        dk, dv = oracle.cols(qn[hh], kn[hh], vn[hh], don[hh], lse_full, del_full, rows,
                             scale=w.scale)
        assert np.max(np.abs(lse - lse_full[rows])) <= 1e-12   # the two oracle paths agree
        for n, r, gg in (("o", o, go["o"][hh][rows]), ("lse", lse, glse[hh][rows]),
                         ("dq", dq, go["dq"][hh][rows]), ("dk", dk, go["dk"][hh][rows]),
                         ("dv", dv, go["dv"][hh][rows])):
            ref[n].append(r)
            got[n].append(gg)
    cat = lambda x: np.concatenate(x)
    errs = dict(o=rel(cat(got["o"]), cat(ref["o"])), lse=absdiff(cat(got["lse"]), cat(ref["lse"])),
                dq=rel(cat(got["dq"]), cat(ref["dq"])), dk=rel(cat(got["dk"]), cat(ref["dk"])),
                dv=rel(cat(got["dv"]), cat(ref["dv"])))

    # whole-tensor identities (every row): sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per head
    # (each residual relative to the sum of magnitudes it is made of)
    dk_sum = go["dk"].sum(axis=1)
    dv_sum = go["dv"].sum(axis=1)
    do_sum = don.sum(axis=1)
    errs["sum_dk"] = float(np.max(np.abs(dk_sum) / np.abs(go["dk"]).sum(axis=1)))
    errs["sum_dv"] = float(np.max(np.abs(dv_sum - do_sum) / np.abs(go["dv"]).sum(axis=1)))
    print(f"[parity] sampled {w.name} errors {errs}", flush=True)
    assert errs["o"] <= tol["o"], errs
    assert errs["lse"] <= tol["lse"], errs
    for n in ("dq", "dk", "dv"):
        assert errs[n] <= tol["grad"], (n, errs)
    assert errs["sum_dk"] <= tol["grad"], errs
    assert errs["sum_dv"] <= tol["grad"], errs
    assert np.all(np.isfinite(g["o"])) and np.all(np.isfinite(g["dq"]))
    assert np.all(np.isfinite(g["dk"])) and np.all(np.isfinite(g["dv"]))


def test_workload_s16000_d80_sampled():
    _sampled_check(WORKLOADS["bf16_b1h32_s16000_d80"])


@pytest.mark.slow
def test_workload_s65536_d128_sampled():
    # 4 heads x 64 rows; each head's full L and D from the oracle (about 10 s a head on 16 cores)
    _sampled_check(WORKLOADS["bf16_b1h16_s65536_d128"])


@pytest.mark.slow
def test_tensors_beyond_2_31_elements():
    """65536 heads of 256 x 128: each tensor holds 2^31 elements (4 GiB in bf16), so the last
    heads lie past every 32-bit element offset.  Heads at the start, middle and end of every
    output are compared with the oracle element by element."""
    dev = torch.device("cuda:0")
    B, H, S, D = 1, 65536, 256, 128
    assert B * H * S * D == 1 << 31
    g = torch.Generator(device=dev).manual_seed(1500)
    q, k, v, do = (torch.randn((B, H, S, D), device=dev, generator=g).to(torch.bfloat16)
                   for _ in range(4))
    print(f"[parity] 2^31-element tensors B={B} H={H} S={S} D={D}", flush=True)
    o, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv, delta = fa.backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    heads = [0, 1, H // 2, H - 2, H - 1]
    pick = lambda t: t[:, heads].double().cpu().numpy()
    r = oracle.backward(*(pick(x) for x in (q, k, v, do)), causal=True)
    g_ = dict(o=pick(o), lse=pick(lse), dq=pick(dq), dk=pick(dk), dv=pick(dv), delta=pick(delta))
    compare(g_, r, "bf16", "2^31 elements, heads " + str(heads))


# ------------------------------------------------------ edges and tails ---

@pytest.mark.parametrize("S", [1, 2, 15, 17, 31, 33, 63, 65, 127, 129, 200, 257])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sequence_tails(S, dtype):
    q, k, v, do = make_inputs(1, 2, S, 64, dtype, seed=100 + S)
    check_full(q, k, v, do, dtype, causal=True, label=f"tail S={S}")


@pytest.mark.parametrize("S", [1, 31, 65, 129, 255, 257, 511])
@pytest.mark.parametrize("D", [80, 128])
def test_sequence_tails_wide_heads(S, D):
    # ragged query tiles (64 rows) and key tiles (256 keys) of the bf16 key-outer pass at the
    # head dims with their own tilings (D = 128: -V^T in LDS, two stages)
    q, k, v, do = make_inputs(1, 2, S, D, "bf16", seed=1600 + S + D)
    check_full(q, k, v, do, "bf16", causal=True, label=f"tail S={S} D={D}")


@pytest.mark.parametrize("H,S,D,causal", [(1, 700, 64, False), (2, 333, 96, False), (1, 1, 128, False),
                                          (3, 100, 80, False), (1, 40, 128, True),
                                          (128, 512, 128, True), (192, 512, 128, True), (193, 512, 128, True),
                                          (256, 512, 64, True), (257, 512, 64, True)])
def test_two_key_groups(H, S, D, causal):
    # a bf16 forward with few 256-query tiles per CU (D >= 64) splits each 128-query tile's keys
    # over two wave groups and merges their m, l and O at the end: one key tile (the second group
    # has none), non-causal rows, ragged tails; at D = 128, 192 heads x 512 rows is the largest
    # such launch (384 tiles, 1.5 per CU), 193 x 512 the smallest past it (one group); at D = 64
    # the limit is 512 tiles (256 heads)
    q, k, v, do = make_inputs(1, H, S, D, "bf16", seed=2100 + H + S + D)
    check_full(q, k, v, do, "bf16", causal=causal, label=f"two key groups H={H} S={S} D={D} causal={causal}")


@pytest.mark.parametrize("D", [16, 32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_dims(D, dtype):
    q, k, v, do = make_inputs(2, 2, 300, D, dtype, seed=200 + D)
    check_full(q, k, v, do, dtype, causal=True, label=f"D={D}")


@pytest.mark.parametrize("D", [16, 32, 64, 80, 96, 128])
def test_head_dims_many_query_tiles(D):
    # 512 heads x 520 rows: a many-head launch (two key groups in the bf16
    # forward at D >= 64, more than one dK/dV tile per CU, so no split).  Heads
    # are independent, so the oracle checks a spread of them.  (The 512-query
    # D = 128 forward tile needs S >= 16384: see the tests of its orders below.)
    q, k, v, do = make_inputs(1, 512, 520, D, "bf16", seed=400 + D)
    print(f"[parity] many query tiles D={D} shape={tuple(q.shape)}", flush=True)
    g = run_gpu(q, k, v, do)
    heads = [0, 1, 255, 510, 511]
    r = oracle.backward(*(x[:, heads].double().numpy() for x in (q, k, v, do)), causal=True)
    gs = {n: a[:, heads] for n, a in g.items()}
    compare(gs, r, "bf16", f"many query tiles D={D}")


@pytest.mark.parametrize("S,D", [(1, 64), (100, 64), (256, 80), (333, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noncausal(S, D, dtype):
    q, k, v, do = make_inputs(1, 3, S, D, dtype, seed=300 + S)
    check_full(q, k, v, do, dtype, causal=False, label=f"noncausal S={S} D={D}")


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("f32", False)])
def test_autograd_function(dtype, causal):
    # the differentiable op: gradients of sum(W * O) equal the oracle's dQ, dK, dV for dO = W
    q, k, v, w = make_inputs(2, 3, 150, 64, dtype, seed=500)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev).requires_grad_(True) for x in (q, k, v))
    o = fa.flash_attention(qd, kd, vd, is_causal=causal)
    (o.float() * w.to(dev).float()).sum().backward()
    torch.cuda.synchronize()
    r = oracle.backward(*(x.double().numpy() for x in (q, k, v, w)), causal=causal)
    tol = TOL[dtype]
    assert rel(o.detach().double().cpu().numpy(), r["o"]) <= tol["o"]
    for n, t in (("dq", qd), ("dk", kd), ("dv", vd)):
        assert rel(t.grad.double().cpu().numpy(), r[n]) <= tol["grad"], n


def test_autograd_function_single_head_layout():
    # [B, S, D] inputs (no head axis) are one head each
    q, k, v, w = make_inputs(3, 1, 77, 32, "bf16", seed=501)
    dev = torch.device("cuda:0")
    q3, k3, v3 = (x[:, 0].to(dev).requires_grad_(True) for x in (q, k, v))
    o = fa.flash_attention(q3, k3, v3, is_causal=True)
    assert o.shape == q3.shape
    (o.float() * w[:, 0].to(dev).float()).sum().backward()
    r = oracle.backward(*(x.double().numpy() for x in (q, k, v, w)), causal=True)
    assert rel(o.detach().double().cpu().numpy(), r["o"][:, 0]) <= TOL["bf16"]["o"]
    assert rel(q3.grad.double().cpu().numpy(), r["dq"][:, 0]) <= TOL["bf16"]["grad"]


# ------------------------------------- shifted / split keys and the merge ---

def _check_partial(g_o, g_l, r_o, r_l, dtype, label):
    """Compare fp32 partial (O, L) with the oracle; empty rows must be exactly (0, -inf)."""
    empty = np.isneginf(r_l)
    assert np.array_equal(np.isneginf(g_l), empty), label
    assert np.all(g_o[empty] == 0.0), label
    if (~empty).any():
        eo = rel(g_o[~empty], r_o[~empty])
        el = absdiff(g_l[~empty], r_l[~empty])
        print(f"[parity] {label} errors o={eo:.3g} lse={el:.3g}", flush=True)
        assert eo <= TOL[dtype]["o"], (label, eo)
        assert el <= TOL[dtype]["lse"], (label, el)


@pytest.mark.parametrize("Sq,Sk,off,causal", [
    (100, 300, 200, 1),    # queries after most keys (one shard against an earlier one)
    (300, 100, -50, 1),    # early queries see no key
    (77, 77, 0, 1),        # plain causal self-attention
    (200, 130, 1000, 1),   # every key allowed
    (64, 200, -64, 1),     # no query sees any key
    (90, 130, 0, 0),       # no mask
])
@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 80), ("bf16", 80)])
def test_fwd_partial_shifted(Sq, Sk, off, causal, dtype, D):
    dev = torch.device("cuda:0")
    q, _, _, _ = make_inputs(2, 2, Sq, D, dtype, seed=600 + Sq)
    _, k, v, _ = make_inputs(2, 2, Sk, D, dtype, seed=700 + Sk)
    op, lp = fa.forward_partial(q.to(dev), k.to(dev), v.to(dev), causal=bool(causal), q_offset=off)
    torch.cuda.synchronize()
    r_o, r_l = oracle.forward_offset(*(x.double().numpy() for x in (q, k, v)), q_offset=off,
                                     causal=bool(causal))
    _check_partial(op[0].double().cpu().numpy(), lp[0].double().cpu().numpy(), r_o, r_l, dtype,
                   f"partial Sq={Sq} Sk={Sk} off={off} causal={causal} D={D}")


@pytest.mark.parametrize("n_split", [2, 3, 7])
def test_fwd_partial_split_chunks(n_split):
    # every chunk's (O, L) is attention over that chunk's keys at their positions
    dev = torch.device("cuda:0")
    Sq, Sk, off, D = 150, 333, 120, 64
    q, _, _, _ = make_inputs(1, 3, Sq, D, "bf16", seed=800)
    _, k, v, _ = make_inputs(1, 3, Sk, D, "bf16", seed=801)
    op, lp = fa.forward_partial(q.to(dev), k.to(dev), v.to(dev), causal=True, q_offset=off,
                                n_split=n_split)
    torch.cuda.synchronize()
    c = fa.split_chunk(Sk, n_split)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    for s_ in range(n_split):
        a, b = min(s_ * c, Sk), min((s_ + 1) * c, Sk)
        if a == b:   # a chunk past the keys is empty for every row
            assert torch.all(op[s_] == 0) and torch.all(torch.isneginf(lp[s_]))
            continue
        r_o, r_l = oracle.forward_offset(qn, kn[:, :, a:b], vn[:, :, a:b], q_offset=off - a,
                                         causal=True)
        _check_partial(op[s_].double().cpu().numpy(), lp[s_].double().cpu().numpy(), r_o, r_l,
                       "bf16", f"split {s_}/{n_split}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_merge_matches_oracle(dtype):
    dev = torch.device("cuda:0")
    g = torch.Generator("cpu").manual_seed(900)
    n, B, H, S, D = 4, 2, 3, 50, 80
    o_parts = torch.randn(n, B, H, S, D, generator=g)
    lse_parts = torch.randn(n, B, H, S, generator=g) * 3.0
    lse_parts[1, 0, 0, :10] = float("-inf")            # a part empty on some rows
    o_parts[1, 0, 0, :10] = 0.0
    lse_parts[:, 1, 2, 7] = float("-inf")              # a row empty in every part
    o_parts[:, 1, 2, 7] = 0.0
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o, lse = fa.merge(o_parts.to(dev), lse_parts.to(dev), tdt)
    torch.cuda.synchronize()
    r_o, r_l = oracle.merge(o_parts.double().numpy(), lse_parts.double().numpy())
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert go[1, 2, 7].tolist() == [0.0] * D and np.isneginf(gl[1, 2, 7])
    fin = ~np.isneginf(r_l)
    assert np.array_equal(np.isneginf(gl), ~fin)
    # fp32 merge arithmetic: 1e-5 relative on an fp32 output, bf16 rounding otherwise
    assert rel(go, r_o) <= (1e-5 if dtype == "f32" else 8e-3)
    assert absdiff(gl[fin], r_l[fin]) <= 1e-5


@pytest.mark.parametrize("n_split,S,D", [(4, 700, 64), (9, 2000, 128), (2, 100, 80)])
def test_split_kv_forward_end_to_end(n_split, S, D):
    dev = torch.device("cuda:0")
    q, k, v, _ = make_inputs(2, 3, S, D, "bf16", seed=1000 + S)
    o, lse = fa.forward_split_kv(q.to(dev), k.to(dev), v.to(dev), n_split)
    o1, l1 = fa.forward(q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    r_o, r_l = oracle.forward(*(x.double().numpy() for x in (q, k, v)), causal=True)
    assert rel(o.double().cpu().numpy(), r_o) <= TOL["bf16"]["o"]
    assert absdiff(lse.double().cpu().numpy(), r_l) <= TOL["bf16"]["lse"]
    # the split path and the one-pass forward agree to bf16 rounding of O
    assert rel(o.double().cpu().numpy(), o1.double().cpu().numpy()) <= 1e-2


# ------------------------------------------------ forward with a workspace ---

def _fwd_ws(q, k, v, causal, ws_bytes=None):
    """fa_fwd_ws through the C ABI with a workspace of ws_bytes (None: the size query's)."""
    B, H, S, D = q.shape
    code = fa.FA_BF16 if q.dtype == torch.bfloat16 else fa.FA_F32
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, S), float("nan"), device=dev)
    if ws_bytes is None:
        ws_bytes = fa.fa_fwd_workspace_size(B, H, S, D, code)
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    rc = fa.fa_fwd_ws(qd, kd, vd, o, lse, ws if ws_bytes else None, ws_bytes, B, H, S, D,
                      1.0 / np.sqrt(D), causal, code)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    o1 = torch.full_like(qd, float("nan"))
    l1 = torch.full((B, H, S), float("nan"), device=dev)
    rc = fa.fa_fwd(qd, kd, vd, o1, l1, B, H, S, D, 1.0 / np.sqrt(D), causal, code)
    assert rc == fa.FA_OK
    torch.cuda.synchronize()
    return o, lse, o1, l1


@pytest.mark.parametrize("B,H,S,D,dtype,causal", [
    (1, 1, 4096, 128, "bf16", 1),   # 16 tiles: 8 key chunks
    (1, 3, 2100, 64, "bf16", 1),    # 27 tiles, ragged: 7 chunks of 320 keys
    (2, 1, 1000, 80, "f32", 1),     # 8 tiles: 8 chunks of 128 keys (16-row tails)
    (1, 2, 777, 32, "f32", 0),      # non-causal, ragged: 7 chunks
    (1, 4, 4096, 64, "f32", 1),     # 64 tiles at S >= 4096: 16 chunks
    (1, 1, 4096, 16, "bf16", 1),    # 8 chunks, 16-row output tails
    (1, 1, 4096, 80, "bf16", 1),    # 8 chunks, 16-row output tails
    (1, 2, 3000, 96, "bf16", 1),    # 8 chunks of 384 keys
    (1, 1, 2500, 32, "bf16", 0),    # non-causal: 8 chunks of 320 keys
    (1, 1, 2048, 128, "f32", 1),    # 16 chunks of 128 keys (the fp32 D = 128 chunk tile)
    (1, 2, 1500, 96, "f32", 1),     # 12 chunks of 128 keys
    (1, 4, 8192, 128, "f32", 0),    # non-causal, 256 tiles of 128 queries: 2 chunks
    (1, 4, 8192, 32, "bf16", 1),    # D <= 32, 128 tiles: 6 chunks
    (1, 2, 6000, 16, "bf16", 0),    # D <= 32 non-causal, ragged, 48 tiles: 4 chunks
    (1, 5, 16400, 32, "bf16", 0),   # D <= 32 non-causal, ragged, 325 tiles, S >= 16384: 2 chunks
    (1, 10, 5000, 16, "bf16", 1),   # D <= 32, ragged, 200 tiles: 6 chunks
    (1, 12, 5000, 32, "f32", 1),    # fp32 D <= 32, ragged, 240 tiles: 8 chunks
    (1, 2, 16300, 80, "bf16", 1),   # D >= 64, ragged, 128 tiles (CU/2): 3 chunks
])
def test_fwd_ws_split_matches_oracle(B, H, S, D, dtype, causal):
    code = fa.FA_BF16 if dtype == "bf16" else fa.FA_F32
    nb = fa.fa_fwd_workspace_size(B, H, S, D, code)
    assert nb > 0
    print(f"[parity] fa_fwd_ws B={B} H={H} S={S} D={D} {dtype} causal={causal} ws={nb}", flush=True)
    q, k, v, _ = make_inputs(B, H, S, D, dtype, seed=1300 + S)
    o, lse, o1, l1 = _fwd_ws(q, k, v, causal)
    r_o, r_l = oracle.forward(*(x.double().numpy() for x in (q, k, v)), causal=bool(causal))
    go, gl = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert rel(go, r_o) <= TOL[dtype]["o"], rel(go, r_o)
    assert absdiff(gl, r_l) <= TOL[dtype]["lse"], absdiff(gl, r_l)
    # the same attention as fa_fwd, up to the order of fp32 sums (and bf16 rounding of O)
    assert rel(go, o1.double().cpu().numpy()) <= (1e-5 if dtype == "f32" else 1e-2)


def test_fwd_ws_runs_as_fa_fwd_without_a_split():
    # no split wanted (many tiles), no workspace, or one too small for two chunks:
    # bit-identical to fa_fwd
    q, k, v, _ = make_inputs(1, 16, 1024, 64, "bf16", seed=1401)
    assert fa.fa_fwd_workspace_size(1, 16, 1024, 64, fa.FA_BF16) == 0
    o, lse, o1, l1 = _fwd_ws(q, k, v, 1)
    assert torch.equal(o, o1) and torch.equal(lse, l1)
    q, k, v, _ = make_inputs(1, 1, 4096, 128, "bf16", seed=1402)
    for nb in (0, 4096 * 129 * 4):   # none; one chunk's worth (two do not fit)
        o, lse, o1, l1 = _fwd_ws(q, k, v, 1, ws_bytes=nb)
        assert torch.equal(o, o1) and torch.equal(lse, l1), nb


def test_fwd_ws_with_a_partial_workspace():
    # a workspace for 3 of the 8 chunks the size query asks for takes 3 chunks
    B, H, S, D = 1, 1, 4096, 128
    q, k, v, _ = make_inputs(B, H, S, D, "bf16", seed=1403)
    nb = 3 * S * D * 4 + 3 * S * 4 + 512
    o, lse, o1, _ = _fwd_ws(q, k, v, 1, ws_bytes=nb)
    r_o, r_l = oracle.forward(*(x.double().numpy() for x in (q, k, v)), causal=True)
    assert rel(o.double().cpu().numpy(), r_o) <= TOL["bf16"]["o"]
    assert absdiff(lse.double().cpu().numpy(), r_l) <= TOL["bf16"]["lse"]
    assert not torch.equal(o, o1)   # (it did split)


def test_fwd_ws_is_deterministic():
    q, k, v, _ = make_inputs(2, 1, 3000, 64, "f32", seed=1404)
    first = _fwd_ws(q, k, v, 1)[:2]
    for _ in range(2):
        again = _fwd_ws(q, k, v, 1)[:2]
        assert all(torch.equal(a, b) for a, b in zip(first, again))


# ------------------------------------------- key-set backward and the ring ---

def _stats_over(q, k, v, do, off, causal):
    """fp64 L and Delta of attention over k, v (the oracle's), as fp32 inputs for the GPU."""
    o, lse = oracle.forward_offset(q, k, v, q_offset=off, causal=causal)
    delta = np.einsum("bhsd,bhsd->bhs", o, do)
    return lse, delta


@pytest.mark.parametrize("Sq,Sk,off,causal", [
    (100, 300, 200, 1),    # queries after most keys
    (300, 100, -50, 1),    # early queries see no key (L = -inf rows)
    (129, 129, 0, 1),      # causal self-attention with a ragged tail
    (200, 130, 1000, 1),   # every key allowed
    (64, 200, -64, 1),     # no query sees any key: contributions are exactly zero
    (90, 230, 0, 0),       # no mask
    (1, 1, 0, 1),          # one query, one key
])
@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 80), ("bf16", 16), ("bf16", 80)])
def test_bwd_partial_shifted(Sq, Sk, off, causal, dtype, D):
    dev = torch.device("cuda:0")
    q, _, _, do = make_inputs(2, 2, Sq, D, dtype, seed=1100 + Sq)
    _, k, v, _ = make_inputs(2, 2, Sk, D, dtype, seed=1200 + Sk)
    qn, kn, vn, don = (x.double().numpy() for x in (q, k, v, do))
    lse, delta = _stats_over(qn, kn, vn, don, off, bool(causal))
    label = f"bwd partial Sq={Sq} Sk={Sk} off={off} causal={causal} {dtype} D={D}"
    print(f"[parity] {label}", flush=True)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).float().to(dev)
    dq, dk, dv = fa.backward_partial(q.to(dev), k.to(dev), v.to(dev), do.to(dev), f32(lse), f32(delta),
                                     causal=bool(causal), q_offset=off)
    torch.cuda.synchronize()
    r = oracle.backward_partial(qn, kn, vn, don, lse, delta, q_offset=off, causal=bool(causal))
    no_pair = bool(causal) and off <= -Sq     # the mask allows no (query, key) pair
    for name, g_, r_ in zip(("dq", "dk", "dv"), (dq, dk, dv), r):
        g_ = g_.double().cpu().numpy()
        if no_pair:
            assert not np.any(g_), (label, name)   # exact zeros where nothing contributes
            continue
        if np.max(np.abs(r_)) <= 1e-9:
            # zero by cancellation (one key: P = 1 and Delta = dP, so dS = 0); the kernel's
            # fp32 dP - Delta of unit-scale inputs leaves rounding residue only
            assert np.max(np.abs(g_)) <= 1e-4, (label, name)
            continue
        e = rel(g_, r_)
        print(f"[parity] {label} {name} err={e:.3g}", flush=True)
        assert e <= TOL[dtype]["grad"], (label, name, e)


@pytest.mark.parametrize("D", [64, 80])
def test_bwd_partial_accumulates(D):
    # accumulate = 1 adds the contributions to what the buffers hold; 0 overwrites
    # (D = 80 also covers the 16-row output tails)
    dev = torch.device("cuda:0")
    Sq, Sk, off = 150, 333, 120
    q, _, _, do = make_inputs(1, 3, Sq, D, "bf16", seed=1300)
    _, k, v, _ = make_inputs(1, 3, Sk, D, "bf16", seed=1301)
    qn, kn, vn, don = (x.double().numpy() for x in (q, k, v, do))
    lse, delta = _stats_over(qn, kn, vn, don, off, True)
    args = [x.to(dev) for x in (q, k, v, do)] + [torch.from_numpy(x).float().to(dev) for x in (lse, delta)]
    g = torch.Generator("cpu").manual_seed(1302)
    base = [torch.randn(shape, generator=g) for shape in ((1, 3, Sq, D), (1, 3, Sk, D), (1, 3, Sk, D))]
    acc = [b.clone().to(dev) for b in base]
    fa.backward_partial(*args, causal=True, q_offset=off, grads=tuple(acc))
    fresh = fa.backward_partial(*args, causal=True, q_offset=off)
    torch.cuda.synchronize()
    for a_, b_, f_ in zip(acc, base, fresh):
        # the only rounding between the two is the final fp32 add
        assert torch.allclose(a_.cpu() - b_, f_.cpu(), rtol=1e-6, atol=1e-5)
    # a key set no query sees leaves accumulators untouched
    acc2 = [b.clone().to(dev) for b in base]
    fa.backward_partial(*args, causal=True, q_offset=-Sq, grads=tuple(acc2))
    torch.cuda.synchronize()
    for a_, b_ in zip(acc2, base):
        assert torch.equal(a_.cpu(), b_)


def _shards(S, R):
    edges = [round(i * S / R) for i in range(R + 1)]
    return list(zip(edges[:-1], edges[1:]))


@pytest.mark.parametrize("S,R,D,skip_masked", [(1000, 3, 64, True), (777, 4, 128, False),
                                                (4096, 4, 128, True)])
def test_ring_schedule_matches_full_attention(S, R, D, skip_masked):
    """Sequence sharded R ways: every query shard meets every key shard (as on a ring of R
    devices, here in one process), forward parts merged, backward contributions accumulated
    with the merged L and Delta; the result is the full causal attention and its gradients."""
    dev = torch.device("cuda:0")
    B, H = 1, 2
    q, k, v, do = make_inputs(B, H, S, D, "bf16", seed=1400 + S)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    sh = _shards(S, R)
    outs, lses = [], []
    for qa, qe in sh:
        parts = [fa.forward_partial(qd[:, :, qa:qe], kd[:, :, ka:ke], vd[:, :, ka:ke], causal=True,
                                    q_offset=qa - ka)
                 for ka, ke in sh if not (skip_masked and ka > qe - 1)]
        o_i, l_i = fa.merge(torch.cat([p[0] for p in parts]), torch.cat([p[1] for p in parts]),
                            torch.bfloat16)
        outs.append(o_i)
        lses.append(l_i)
    f32 = dict(device=dev, dtype=torch.float32)
    dq = torch.zeros((B, H, S, D), **f32)
    dk = torch.zeros((B, H, S, D), **f32)
    dv = torch.zeros((B, H, S, D), **f32)
    for i, (qa, qe) in enumerate(sh):
        delta = torch.empty((B, H, qe - qa), **f32)
        assert fa.fa_bwd_preprocess(outs[i].contiguous(), dod[:, :, qa:qe].contiguous(), delta, B, H,
                                    qe - qa, D, fa.FA_BF16) == 0
        for ka, ke in sh:
            if skip_masked and ka > qe - 1:
                continue
            gq = dq[:, :, qa:qe].contiguous()
            gk = dk[:, :, ka:ke].contiguous()
            gv = dv[:, :, ka:ke].contiguous()
            fa.backward_partial(qd[:, :, qa:qe], kd[:, :, ka:ke], vd[:, :, ka:ke], dod[:, :, qa:qe],
                                lses[i], delta, causal=True, q_offset=qa - ka, grads=(gq, gk, gv))
            dq[:, :, qa:qe] = gq
            dk[:, :, ka:ke] = gk
            dv[:, :, ka:ke] = gv
    torch.cuda.synchronize()
    r = oracle.backward(*(x.double().numpy() for x in (q, k, v, do)), causal=True)
    g = dict(o=torch.cat(outs, 2), lse=torch.cat(lses, 2), dq=dq, dk=dk, dv=dv)
    g = {n: t.double().cpu().numpy() for n, t in g.items()}
    errs = dict(o=rel(g["o"], r["o"]), lse=absdiff(g["lse"], r["lse"]),
                **{n: rel(g[n], r[n]) for n in ("dq", "dk", "dv")})
    print(f"[parity] ring S={S} R={R} D={D} errors {errs}", flush=True)
    assert errs["o"] <= TOL["bf16"]["o"] and errs["lse"] <= TOL["bf16"]["lse"], errs
    for n in ("dq", "dk", "dv"):
        assert errs[n] <= TOL["bf16"]["grad"], (n, errs)


def _random_cases(seed, n):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        yield dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), S=int(rng.integers(1, 700)),
                   D=int(rng.choice([16, 32, 64, 80, 96, 128])), causal=bool(rng.integers(0, 2)),
                   seed=int(rng.integers(0, 1 << 30)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", list(_random_cases(1700, 10)), ids=lambda c: "B{B}H{H}S{S}D{D}c{causal:d}".format(**c))
def test_random_shapes(case, dtype):
    """Seeded random shapes (ragged S, every head dim, causal or not) through the whole path."""
    c = case
    q, k, v, do = make_inputs(c["B"], c["H"], c["S"], c["D"], dtype, seed=c["seed"])
    check_full(q, k, v, do, dtype, causal=c["causal"], label=f"random {c}")


@pytest.mark.parametrize("case", list(range(12)))
def test_random_key_sets(case):
    """Seeded random query/key shard sizes and offsets through the key-set forward and backward:
    the shifted forward against the oracle, and the backward contributions against the oracle's
    with the same L and Delta.  The 12 cases take every head dimension in both dtypes."""
    rng = np.random.default_rng(1800 + case)
    dev = torch.device("cuda:0")
    Sq, Sk = int(rng.integers(1, 400)), int(rng.integers(1, 400))
    off = int(rng.integers(-Sq - 20, Sk + 20))
    D = (16, 32, 64, 80, 96, 128)[case % 6]
    dtype = "bf16" if case < 6 else "f32"
    causal = bool(rng.integers(0, 4))          # mostly causal
    q, _, _, do = make_inputs(1, 2, Sq, D, dtype, seed=1900 + case)
    _, k, v, _ = make_inputs(1, 2, Sk, D, dtype, seed=2000 + case)
    qn, kn, vn, don = (x.double().numpy() for x in (q, k, v, do))
    label = f"key set Sq={Sq} Sk={Sk} off={off} D={D} {dtype} causal={causal}"
    print(f"[parity] {label}", flush=True)
    op, lp = fa.forward_partial(q.to(dev), k.to(dev), v.to(dev), causal=causal, q_offset=off)
    torch.cuda.synchronize()
    r_o, r_l = oracle.forward_offset(qn, kn, vn, q_offset=off, causal=causal)
    _check_partial(op[0].double().cpu().numpy(), lp[0].double().cpu().numpy(), r_o, r_l, dtype, label)
    delta = np.einsum("bhsd,bhsd->bhs", r_o, don)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).float().to(dev)
    g = fa.backward_partial(q.to(dev), k.to(dev), v.to(dev), do.to(dev), f32(r_l), f32(delta),
                            causal=causal, q_offset=off)
    torch.cuda.synchronize()
    r = oracle.backward_partial(qn, kn, vn, don, r_l, delta, q_offset=off, causal=causal)
    for name, g_, r_ in zip(("dq", "dk", "dv"), g, r):
        g_ = g_.double().cpu().numpy()
        if np.max(np.abs(r_)) <= 1e-9:
            # nothing contributes (no allowed pair) or cancellation (a single key)
            assert np.max(np.abs(g_)) <= 1e-4, (label, name)
            continue
        e = rel(g_, r_)
        assert e <= TOL[dtype]["grad"], (label, name, e)


def test_custom_scale_and_peaky_scores():
    q, k, v, do = make_inputs(1, 2, 257, 64, "bf16", seed=7, qk_mult=3.0)
    check_full(q, k, v, do, "bf16", causal=True, scale=0.3, label="scale=0.3 peaky")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("slope,jump", [(0.065, 0.0), (0.4, 0.0), (0.0, 150.0), (0.02, 90.0)])
def test_rising_scores(slope, jump, dtype):
    """Scores that rise along the keys, so the running row maximum has to move
    tile after tile.

    Key j scores about slope*j (natural-log units), plus `jump` from the middle
    key on.  slope 0.065 lifts each 64-key tile by about 4 (6 in base 2): its
    probabilities against the maximum so far sum past 2^8 while each stays
    below it.  slope 0.4 lifts each tile by about 25.  Jumps of 90 and 150
    make the exponentials against the maximum before them overflow to inf.
    """
    B, H, S, D = 1, 2, 777, 64
    g = torch.Generator("cpu").manual_seed(31)
    u = torch.randn(D, generator=g)
    u = u / u.norm()
    pos = torch.arange(S, dtype=torch.float32)
    a = slope * pos + jump * (pos >= S // 2).float()
    # scale 1/8 and q . k_j = 8 a_j: the score of key j is about a_j.  The keys
    # also get a part orthogonal to the queries' direction, as large as a_j:
    # without it the keys a row attends to share one large component, and
    # dQ = scale * sum_j dS_ij k_j (whose dS sum to zero over j) would be a
    # near-total cancellation that no bf16 path computes to 5e-2.
    q = 8.0 * u + 0.05 * torch.randn(B, H, S, D, generator=g)
    w = torch.randn(B, H, S, D, generator=g)
    w = w - (w @ u)[..., None] * u
    k = a[:, None] * u + (0.5 * a + 1.0)[:, None] * w
    v, do = (torch.randn(B, H, S, D, generator=g) for _ in range(2))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, do = (x.to(tdt) for x in (q, k, v, do))
    check_full(q, k, v, do, dtype, causal=True, label=f"rising slope={slope} jump={jump}")
    check_full(q, k, v, do, dtype, causal=False, label=f"rising slope={slope} jump={jump} non-causal")
    if dtype == "bf16":
        # the shifted-key forward over three key chunks, merged
        dev = torch.device("cuda:0")
        o, lse = fa.forward_split_kv(q.to(dev), k.to(dev), v.to(dev), 3)
        torch.cuda.synchronize()
        r_o, r_l = oracle.forward(*(x.double().numpy() for x in (q, k, v)), causal=True)
        assert rel(o.double().cpu().numpy(), r_o) <= TOL["bf16"]["o"]
        assert absdiff(lse.double().cpu().numpy(), r_l) <= TOL["bf16"]["lse"]


def test_rising_scores_wide_tile():
    """The same on the 64-queries-per-wave forward tile (bf16, D = 128, enough
    query tiles to select it): scores rise by about 4.8 per 32-key tile over
    the first 1024 keys (7 in base 2: the tile's sums pass 2^8, each
    probability stays below it), then jump by 100 at key 3000 (overflow)."""
    B, H, S, D = 1, 128, 4096, 128
    g = torch.Generator("cpu").manual_seed(41)
    u = torch.randn(D, generator=g)
    u = u / u.norm()
    pos = torch.arange(S, dtype=torch.float32)
    a = 0.152 * torch.clamp(pos, max=1024.0) + 100.0 * (pos >= 3000).float()
    # default scale 1/sqrt(D) and q . k_j = sqrt(D) a_j: the score of key j is about a_j
    q = D ** 0.5 * u + 0.05 * torch.randn(B, H, S, D, generator=g)
    k = a[:, None] * u + 0.05 * torch.randn(B, H, S, D, generator=g)
    v = torch.randn(B, H, S, D, generator=g)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    dev = torch.device("cuda:0")
    print("[parity] rising scores, wide forward tile", flush=True)
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    for hh in (0, 77):
        r_o, r_l = oracle.forward(*(x[:, hh:hh + 1].double().numpy() for x in (q, k, v)),
                                  causal=True)
        assert rel(o[:, hh:hh + 1].double().cpu().numpy(), r_o) <= TOL["bf16"]["o"], hh
        assert absdiff(lse[:, hh:hh + 1].double().cpu().numpy(), r_l) <= TOL["bf16"]["lse"], hh


@pytest.mark.parametrize("B,H,S,D,causal", [(1, 1, 300, 64, True), (1, 1, 1000, 80, True),
                                             (1, 2, 4097, 128, True), (1, 1, 777, 16, False),
                                             (2, 1, 2000, 96, True), (1, 1, 257, 128, True),
                                             (3, 1, 520, 64, True), (1, 1, 8192, 64, True),
                                             (1, 8, 4096, 64, True), (1, 8, 4096, 16, True),
                                             (1, 32, 2048, 16, False), (1, 8, 4096, 64, False)])
def test_split_backward(B, H, S, D, causal):
    """bf16 problems with few key tiles per CU: the backward runs each pass in
    chunks side by side and sums the fp32 partials (a fixed order, so still
    bit-reproducible); the forward of these shapes (D >= 64) runs two key
    groups per workgroup and merges them."""
    assert fa.fa_bwd_workspace_size(B, H, S, D, fa.FA_BF16) > ((B * H * S * 4 + 255) // 256) * 256
    q, k, v, do = make_inputs(B, H, S, D, "bf16", seed=2100 + S)
    check_full(q, k, v, do, "bf16", causal=causal, label=f"split backward B={B} H={H} S={S} D={D}")
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    first = fa.backward(qd, kd, vd, o, lse, dod, causal=causal)
    again = fa.backward(qd, kd, vd, o, lse, dod, causal=causal)
    for a_, b_ in zip(first, again):
        assert torch.equal(a_, b_)
    # a workspace holding only the base-2 L runs the unsplit backward: the same gradients
    # up to the order of fp32 sums
    small = torch.empty(((B * H * S * 4 + 255) // 256) * 256, device=dev, dtype=torch.uint8)
    plain = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, workspace=small)
    torch.cuda.synchronize()
    for a_, b_ in zip(first[:3], plain[:3]):
        assert rel(a_.double().cpu().numpy(), b_.double().cpu().numpy()) <= 1e-2


def test_first_query_and_identical_keys():
    """Closed forms on the GPU: O_0 = V_0; identical keys give the causal prefix mean."""
    S, D = 300, 64
    q, k1, v, _ = make_inputs(1, 2, 1, D, "f32", seed=11)
    q, _, v, _ = make_inputs(1, 2, S, D, "f32", seed=11)
    k = k1.expand(1, 2, S, D).contiguous()
    dev = torch.device("cuda:0")
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), causal=True)
    o = o.double().cpu()
    prefix = torch.cumsum(v.double(), dim=2) / torch.arange(1, S + 1, dtype=torch.float64)[:, None]
    assert torch.max(torch.abs(o - prefix)).item() <= 1e-4
    assert torch.max(torch.abs(o[:, :, 0] - v[:, :, 0].double())).item() <= 1e-6


def test_noncontiguous_inputs():
    q, k, v, do = make_inputs(1, 130, 2, 64, "bf16", seed=12)   # [B, S, H, D] drawn
    qt, kt, vt, dot = (x.transpose(1, 2) for x in (q, k, v, do))  # -> [B, H, S, D] views
    check_full(qt, kt, vt, dot, "bf16", causal=True, label="non-contiguous")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_is_deterministic(dtype):
    # (both split: 4 heads of 1000 rows have few dK/dV tiles for the CUs)
    q, k, v, do = make_inputs(1, 4, 1000, 80, dtype, seed=13)
    rc, plan = fa.fa_get_plan(1, 4, 1000, 80, fa.FA_BF16 if dtype == "bf16" else fa.FA_F32, 0)
    assert rc == 0 and plan.bwd_chunks > 1, plan.as_dict()
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd)
    first = fa.backward(qd, kd, vd, o, lse, dod)
    for _ in range(3):
        again = fa.backward(qd, kd, vd, o, lse, dod)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_forward_on_a_side_stream():
    q, k, v, do = make_inputs(2, 2, 200, 64, "bf16", seed=14)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    ref, _ = fa.forward(qd, kd, vd)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, _ = fa.forward(qd, kd, vd, stream=s)
    s.synchronize()
    assert torch.equal(o, ref)


@pytest.mark.parametrize("raw_handle", [False, True])
def test_helpers_on_a_stream_that_is_not_current(raw_handle):
    # forward/backward given a stream other than the current one: their workspaces
    # (a split forward and a split backward at one head), copies and outputs are
    # allocated on that stream; results equal the current-stream ones bit for bit
    B, H, S, D = 1, 1, 8192, 128
    assert fa.fa_fwd_workspace_size(B, H, S, D, fa.FA_BF16) > 0
    assert fa.fa_bwd_workspace_size(B, H, S, D, fa.FA_BF16) > 4 * B * H * S
    print(f"[parity] helpers on a side stream, raw handle={raw_handle}", flush=True)
    q, k, v, do = make_inputs(B, H, S, D, "bf16", seed=15)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    ref_o, ref_l = fa.forward(qd, kd, vd)
    ref_g = fa.backward(qd, kd, vd, ref_o, ref_l, dod)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    st = s.cuda_stream if raw_handle else s
    s.wait_stream(torch.cuda.current_stream())
    o, lse = fa.forward(qd, kd, vd, stream=st)
    g = fa.backward(qd, kd, vd, o, lse, dod, stream=st)
    # the current stream allocates and writes while the side stream may still run
    junk = [torch.full((1 << 22,), float(i), device=dev) for i in range(8)]
    s.synchronize()
    del junk
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
    for a, b in zip(g, ref_g):
        assert torch.equal(a, b)


# ------------------------------------------- workgroup order of the forward ---

def _banded_forward(B, H, S, heads, rows=None, causal=True, banded=True):
    """Forward through a launch that takes the 512-query D=128 tile, in the banded XCD order
    (B*H a multiple of 8) or the consecutive one; outputs start as NaN so a (head, tile) the
    order skipped shows."""
    D = 128
    rc, plan = fa.fa_get_plan(B, H, S, D, fa.FA_BF16, 0)
    assert rc == 0 and plan.fwd_block_queries == 512 and (plan.fwd_band > 0) == banded, plan.as_dict()
    print(f"[parity] banded forward B={B} H={H} S={S} band={plan.fwd_band} causal={causal}", flush=True)
    q, k, v, do = make_inputs(B, H, S, D, "bf16", seed=900 + H)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, S), float("nan"), device=dev)
    fa.forward(qd, kd, vd, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    on = o.double().cpu().numpy().reshape(B * H, S, D)
    ln = lse.double().cpu().numpy().reshape(B * H, S)
    qn, kn, vn, don = (x.double().numpy().reshape(B * H, S, D) for x in (q, k, v, do))
    ro, rl, go, gl = [], [], [], []
    for hh in heads:
        rr = list(range(S)) if rows is None else rows
        o_ref, l_ref, _ = oracle.rows(qn[hh], kn[hh], vn[hh], don[hh], rr, causal=causal)
        ro.append(o_ref); rl.append(l_ref); go.append(on[hh][rr]); gl.append(ln[hh][rr])
    eo = rel(np.concatenate(go), np.concatenate(ro))
    el = absdiff(np.concatenate(gl), np.concatenate(rl))
    print(f"[parity] banded forward errors o={eo:.3e} lse={el:.3e}", flush=True)
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("causal", [True, False])
def test_banded_order_partial_bands(causal):
    # 32 heads of 33 query tiles (the last one ragged): every XCD's heads fall in partial bands of
    # 64; every (head, tile) is checked finite, sampled rows (all tile edges) against the oracle
    S = 16384 + 100
    edges = [r for t in range(0, S, 512) for r in (t, t + 1, t + 511) if r < S]
    rows = sorted(set(edges + [S - 2, S - 1] + list(np.random.default_rng(33).integers(0, S, 24))))
    _banded_forward(2, 16, S, heads=[0, 1, 7, 8, 9, 23, 31], rows=rows, causal=causal)


def test_512_query_tile_consecutive_order():
    # 33 heads (not a multiple of the 8 XCDs): the 512-query tile in the consecutive order,
    # 33 tiles per head with a ragged last one of 37 rows
    S = 16384 + 37
    edges = [r for t in range(0, S, 512) for r in (t, t + 511) if r < S]
    rows = sorted(set(edges + [S - 2, S - 1] + list(np.random.default_rng(34).integers(0, S, 16))))
    _banded_forward(1, 33, S, heads=[0, 16, 32], rows=rows, banded=False)


@pytest.mark.slow
def test_banded_order_full_bands_and_remainder():
    # 8 heads of 129 query tiles: two full bands of 64 and a one-tile remainder per head
    S = 64 * 1024 + 300
    rows = [0, 1, 511, 512, 32767, 32768, 65535, 65536, S - 300, S - 2, S - 1]
    _banded_forward(1, 8, S, heads=[0, 3, 7], rows=rows)


# ------------------------------------------------ tile selection on the device ---

def test_plan_uses_the_device_cu_count():
    n = torch.cuda.get_device_properties(0).multi_processor_count
    rc, plan = fa.fa_get_plan(1, 16, 65536, 128, fa.FA_BF16, 0)
    assert rc == 0 and plan.num_cu == n, (rc, plan.as_dict(), n)
    rc2, explicit = fa.fa_get_plan(1, 16, 65536, 128, fa.FA_BF16, n)
    assert rc2 == 0 and explicit.as_dict() == plan.as_dict()


@pytest.mark.parametrize("B,H,S,chunks", [(2, 4, 2048, 3), (1, 1, 3000, 8)])
def test_fp32_split_backward_d128(B, H, S, chunks):
    # fp32 D = 128: the dQ pass on 4-wave workgroups, split over key chunks (3: a chunk count
    # that does not divide the tiles), the pair dK/dV kernel over query chunks
    D = 128
    rc, plan = fa.fa_get_plan(B, H, S, D, fa.FA_F32, 0)
    assert rc == 0 and plan.bwd_chunks == chunks, plan.as_dict()
    q, k, v, do = make_inputs(B, H, S, D, "f32", seed=815 + S)
    check_full(q, k, v, do, "f32", causal=True, label=f"fp32 D=128 split backward B={B} H={H} S={S}")


@pytest.mark.parametrize("B,H,S,D,chunks", [(1, 1, 200, 80, 4), (1, 2, 97, 64, 2), (2, 3, 256, 128, 4)])
def test_fp32_split_backward_short(B, H, S, D, chunks):
    # fp32 at S <= 256: chunks of 64 rows (a ragged last one), causal and not
    rc, plan = fa.fa_get_plan(B, H, S, D, fa.FA_F32, 0)
    assert rc == 0 and plan.bwd_chunks == chunks, plan.as_dict()
    q, k, v, do = make_inputs(B, H, S, D, "f32", seed=840 + S)
    for causal in (True, False):
        check_full(q, k, v, do, "f32", causal=causal, label=f"fp32 short split B={B} H={H} S={S} D={D} {causal}")


def test_fp32_split_backward_one_head():
    # one fp32 head: the pair dK/dV kernel over 8 query chunks and dQ over 8 key chunks (ragged
    # last chunk), fp32 partials summed; element by element against the oracle at 1e-4
    B, H, S, D = 1, 1, 2000, 64
    rc, plan = fa.fa_get_plan(B, H, S, D, fa.FA_F32, 0)
    assert rc == 0 and plan.bwd_chunks == 8, plan.as_dict()
    q, k, v, do = make_inputs(B, H, S, D, "f32", seed=812)
    check_full(q, k, v, do, "f32", causal=True, label="fp32 split backward")


def test_backward_with_a_partial_split_workspace():
    """A workspace that holds the partials of fewer chunks than fa_bwd_workspace_size asks for
    takes as many chunks as fit; the gradients still match the oracle."""
    B, H, S, D = 1, 1, 4096, 128
    rc, plan = fa.fa_get_plan(B, H, S, D, fa.FA_BF16, 0)
    assert rc == 0 and plan.bwd_chunks >= 4, plan.as_dict()
    q, k, v, do = make_inputs(B, H, S, D, "bf16", seed=811)
    r = oracle.backward(*(x.double().numpy() for x in (q, k, v, do)), causal=True)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=True)
    base = (B * H * S * 4 + 255) // 256 * 256
    per_chunk = 3 * B * H * S * D * 4
    outs = {}
    for chunks in (plan.bwd_chunks, 3, 2, 1):
        print(f"[parity] split backward with a workspace for {chunks} chunk(s)", flush=True)
        ws = torch.empty(base + (per_chunk * chunks if chunks > 1 else 0), device=dev, dtype=torch.uint8)
        dq, dk, dv, _ = fa.backward(qd, kd, vd, o, lse, dod, causal=True, workspace=ws)
        torch.cuda.synchronize()
        g = {n: t.double().cpu().numpy() for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
        for n in g:
            assert rel(g[n], r[n]) <= TOL["bf16"]["grad"], (chunks, n, rel(g[n], r[n]))
        outs[chunks] = g
    # different chunk counts sum the same contributions in a different order
    for n in ("dq", "dk", "dv"):
        assert rel(outs[2][n], outs[1][n]) <= 1e-2
