"""Pins for the fp64 CPU oracle (no GPU).

The oracle is only trusted because these checks tie it to things other than
itself: a hand-worked example, central finite differences of its own forward,
closed forms of the definition, softmax invariants, the two-block merge rule of
the ring-attention page, and PyTorch's float64 CPU attention with autograd.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_causal_amd.inputs import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(x):
    if isinstance(x, list):
        return [_val(t) for t in x]
    if isinstance(x, str):
        if x == "ln3":
            return math.log(3.0)
        if x == "ln4":
            return math.log(4.0)
        if x == "0.75*ln3":
            return 0.75 * math.log(3.0)
        raise ValueError(x)
    return float(x)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- golden ---

def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_s2_d1.json")) as f:
        g = json.load(f)
    inp = {k: np.array(_val(v)) for k, v in g["inputs"].items() if k != "scale"}
    exp = {k: np.array(_val(v)) for k, v in g["expected"].items()}
    scale = g["inputs"]["scale"]
    o, lse = oracle.forward(inp["q"], inp["k"], inp["v"], scale=scale, causal=True)
    np.testing.assert_allclose(o, exp["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, exp["lse"], rtol=0, atol=1e-14)
    r = oracle.backward(inp["q"], inp["k"], inp["v"], inp["do"], scale=scale, causal=True)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r[name], exp[name], rtol=0, atol=1e-14, err_msg=name)
    np.testing.assert_allclose(r["delta_p"], exp["delta"], atol=1e-14)
    np.testing.assert_allclose(r["delta_o"], exp["delta"], atol=1e-14)


# ------------------------------------------------------- finite differences ---

@pytest.mark.parametrize("S,D,causal", [(1, 3, True), (2, 4, True), (5, 3, True),
                                        (7, 8, True), (5, 4, False), (7, 3, False)])
def test_gradients_central_differences(S, D, causal):
    """Loss = sum(W o O); oracle analytic grads vs central differences of its forward."""
    H = 2
    q, k, v, w = (_rand((1, H, S, D), s) for s in (11, 12, 13, 14))
    scale = 1.0 / math.sqrt(D)
    r = oracle.backward(q, k, v, w, scale=scale, causal=causal)

    def loss(qq, kk, vv):
        o, _ = oracle.forward(qq, kk, vv, scale=scale, causal=causal)
        return float(np.sum(w * o))

    h = 1e-6
    for name, x, g in (("dq", q, r["dq"]), ("dk", k, r["dk"]), ("dv", v, r["dv"])):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = [q, k, v]; args_m = [q, k, v]
            pos = {"dq": 0, "dk": 1, "dv": 2}[name]
            args_p[pos] = xp; args_m[pos] = xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        denom = max(1.0, float(np.max(np.abs(num))))
        err = float(np.max(np.abs(num - g))) / denom
        assert err <= 1e-6, f"{name}: rel err {err}"


# ------------------------------------------------------------ closed forms ---

def test_query_zero_sees_only_key_zero():
    q, k, v = (_rand((2, 3, 9, 5), s) for s in (1, 2, 3))
    scale = 0.37
    o, lse = oracle.forward(q, k, v, scale=scale, causal=True)
    np.testing.assert_allclose(o[..., 0, :], v[..., 0, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[..., 0], scale * np.sum(q[..., 0, :] * k[..., 0, :], -1),
                               rtol=0, atol=1e-13)


def test_identical_keys_give_causal_prefix_mean():
    S, D = 11, 6
    q = _rand((1, 2, S, D), 4)
    v = _rand((1, 2, S, D), 5)
    kvec = _rand((1, 2, 1, D), 6)
    k = np.broadcast_to(kvec, (1, 2, S, D)).copy()
    scale = 1 / math.sqrt(D)
    o, lse = oracle.forward(q, k, v, scale=scale, causal=True)
    counts = np.arange(1, S + 1)[:, None]
    prefix_mean = np.cumsum(v, axis=-2) / counts
    np.testing.assert_allclose(o, prefix_mean, rtol=0, atol=1e-13)
    want_lse = scale * np.sum(q * kvec, -1) + np.log(np.arange(1, S + 1))
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-13)


def test_single_token():
    q, k, v, do = (_rand((2, 2, 1, 4), s) for s in (7, 8, 9, 10))
    r = oracle.backward(q, k, v, do, causal=True)
    np.testing.assert_allclose(r["o"], v, atol=1e-15)
    np.testing.assert_allclose(r["dv"], do, atol=1e-15)
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-15)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-15)


def test_noncausal_uniform_scores_average_all_values():
    """Q = 0 makes every score equal: O is the plain mean of V, L = ln Sk."""
    S, D = 6, 3
    q = np.zeros((1, 1, S, D))
    k = _rand((1, 1, S, D), 20)
    v = _rand((1, 1, S, D), 21)
    o, lse = oracle.forward(q, k, v, causal=False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (S, D)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(S), atol=1e-14)


# -------------------------------------------------------------- invariants ---

@pytest.mark.parametrize("causal", [True, False])
def test_probability_rows(causal):
    S, D = 13, 4
    q, k = _rand((S, D), 30), _rand((S, D), 31) * 3
    P = oracle.probs(q, k, causal=causal)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.all(P >= 0)
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)
        assert np.all(np.diag(P) > 0)


def test_backward_identities():
    S, D = 17, 5
    q, k, v, do = (_rand((2, 2, S, D), s) for s in (40, 41, 42, 43))
    r = oracle.backward(q, k, v, do, causal=True)
    # both forms of Delta agree (handout: rowsum(P o dP) = rowsum(O o dO))
    np.testing.assert_allclose(r["delta_p"], r["delta_o"], rtol=0, atol=1e-12)
    # shifting every key by one vector changes no softmax -> sum_j dK_j = 0
    np.testing.assert_allclose(r["dk"].sum(-2), 0.0, atol=1e-12)
    # shifting every value by c shifts every output by c -> sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(r["dv"].sum(-2), do.sum(-2), atol=1e-12)
    # scaling the scores through Q or through `scale` is the same function
    o1, l1 = oracle.forward(q, k, v, scale=0.3, causal=True)
    o2, l2 = oracle.forward(q * 3.0, k, v, scale=0.1, causal=True)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


# --------------------------------------------------- two-block merge rule ---

def _merge(o_l, lse_l, o_r, lse_r):
    """Combine two partial (O, L) results over disjoint key sets.

    Ring-attention page ("online attention"): with m = max(m_l, m_r) the
    merged output is (B_l e^{m_l-m} o_l + B_r e^{m_r-m} o_r) / (B_l e^{m_l-m}
    + B_r e^{m_r-m}); B e^m is exp(L) for each part.
    """
    m = np.maximum(lse_l, lse_r)
    a = np.exp(lse_l - m)
    b = np.exp(lse_r - m)
    o = (a[..., None] * o_l + b[..., None] * o_r) / (a + b)[..., None]
    return o, m + np.log(a + b)


def test_split_kv_merge_noncausal():
    Sq, Sk, D, split = 9, 14, 6, 5
    q = _rand((2, Sq, D), 50)
    k, v = _rand((2, Sk, D), 51), _rand((2, Sk, D), 52)
    o, lse = oracle.forward(q, k, v, causal=False)
    ol, ll = oracle.forward(q, k[:, :split], v[:, :split], causal=False, scale=1 / math.sqrt(D))
    orr, lr = oracle.forward(q, k[:, split:], v[:, split:], causal=False, scale=1 / math.sqrt(D))
    om, lm = _merge(ol, ll, orr, lr)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lm, lse, rtol=1e-12, atol=1e-12)


def test_split_kv_merge_causal():
    """Rows i >= s see keys [0, s) (all) and [s, i] (causal on the trailing block)."""
    S, D, s = 16, 4, 6
    q, k, v = (_rand((3, S, D), t) for t in (60, 61, 62))
    sc = 1 / math.sqrt(D)
    o, lse = oracle.forward(q, k, v, causal=True, scale=sc)
    ol, ll = oracle.forward(q[:, s:], k[:, :s], v[:, :s], causal=False, scale=sc)
    orr, lr = oracle.forward(q[:, s:], k[:, s:], v[:, s:], causal=True, scale=sc)
    om, lm = _merge(ol, ll, orr, lr)
    np.testing.assert_allclose(om, o[:, s:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lm, lse[:, s:], rtol=1e-12, atol=1e-12)
    o0, l0 = oracle.forward(q[:, :s], k[:, :s], v[:, :s], causal=True, scale=sc)
    np.testing.assert_allclose(o0, o[:, :s], atol=1e-14)
    np.testing.assert_allclose(l0, lse[:, :s], atol=1e-14)


# ------------------------------------- shifted queries and the n-way merge ---

def _torch_shifted(q, k, v, q_offset, causal, scale):
    """fp64 torch attention with an explicitly built shifted causal mask."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    s = (qt @ kt.transpose(-1, -2)) * scale
    Sq, Sk = q.shape[-2], k.shape[-2]
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        s = s.masked_fill(j > i + q_offset, float("-inf"))
    return (torch.softmax(s, -1) @ vt).numpy(), torch.logsumexp(s, -1).numpy()


@pytest.mark.parametrize("Sq,Sk,off", [(7, 11, 0), (7, 11, 4), (9, 6, -3), (5, 8, 20), (6, 6, -6)])
def test_shifted_forward_matches_torch_with_explicit_mask(Sq, Sk, off):
    D = 5
    q, k, v = _rand((2, Sq, D), 70), _rand((2, Sk, D), 71), _rand((2, Sk, D), 72)
    sc = 1 / math.sqrt(D)
    o, lse = oracle.forward_offset(q, k, v, q_offset=off, scale=sc, causal=True)
    ot, lt = _torch_shifted(q, k, v, off, True, sc)
    empty = np.arange(Sq) + off < 0          # rows that allow no key
    np.testing.assert_allclose(o[:, ~empty], ot[:, ~empty], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, ~empty], lt[:, ~empty], rtol=0, atol=1e-12)
    assert np.all(o[:, empty] == 0.0) and np.all(np.isneginf(lse[:, empty]))
    # offset 0 with equal lengths is the plain causal forward; without the mask nothing shifts
    if Sq == Sk and off == 0:
        o0, l0 = oracle.forward(q, k, v, scale=sc, causal=True)
        np.testing.assert_array_equal(o, o0)
    on, ln = oracle.forward_offset(q, k, v, q_offset=off, scale=sc, causal=False)
    of, lf = oracle.forward(q, k, v, scale=sc, causal=False)
    np.testing.assert_array_equal(on, of)
    np.testing.assert_array_equal(ln, lf)


@pytest.mark.parametrize("causal", [True, False])
def test_nway_merge_of_key_chunks_is_full_attention(causal):
    """Three key chunks at their positions, merged, equal attention over all keys."""
    Sq, Sk, D, q_pos = 12, 17, 4, 5           # query i sits at position q_pos + i
    q, k, v = _rand((3, Sq, D), 80), _rand((3, Sk, D), 81), _rand((3, Sk, D), 82)
    sc = 1 / math.sqrt(D)
    o, lse = oracle.forward_offset(q, k, v, q_offset=q_pos, scale=sc, causal=causal)
    bounds = [0, 6, 13, Sk]
    parts = [oracle.forward_offset(q, k[:, a:b], v[:, a:b], q_offset=q_pos - a, scale=sc,
                                   causal=causal) for a, b in zip(bounds[:-1], bounds[1:])]
    om, lm = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(om, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lse, rtol=0, atol=1e-12)
    ot, lt = _torch_shifted(q, k, v, q_pos, causal, sc)
    np.testing.assert_allclose(om, ot, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lt, rtol=0, atol=1e-12)


def test_merge_closed_forms():
    o1, l1 = _rand((2, 5, 3), 90), _rand((2, 5), 91)
    # one part: unchanged
    om, lm = oracle.merge(o1[None], l1[None])
    np.testing.assert_allclose(om, o1, atol=1e-15)
    np.testing.assert_allclose(lm, l1, atol=1e-15)
    # an empty part (O = 0, L = -inf) changes nothing
    empty_o, empty_l = np.zeros_like(o1), np.full_like(l1, -np.inf)
    om, lm = oracle.merge(np.stack([o1, empty_o]), np.stack([l1, empty_l]))
    np.testing.assert_allclose(om, o1, atol=1e-15)
    np.testing.assert_allclose(lm, l1, atol=1e-15)
    # the same part twice: same output, L + ln 2
    om, lm = oracle.merge(np.stack([o1, o1]), np.stack([l1, l1]))
    np.testing.assert_allclose(om, o1, atol=1e-14)
    np.testing.assert_allclose(lm, l1 + math.log(2.0), atol=1e-14)
    # all parts empty: the row stays empty
    om, lm = oracle.merge(np.stack([empty_o, empty_o]), np.stack([empty_l, empty_l]))
    assert np.all(om == 0.0) and np.all(np.isneginf(lm))
    # agrees with the two-block rule written above for two parts
    o2, l2 = _rand((2, 5, 3), 92), _rand((2, 5), 93)
    om, lm = oracle.merge(np.stack([o1, o2]), np.stack([l1, l2]))
    ref_o, ref_l = _merge(o1, l1, o2, l2)
    np.testing.assert_allclose(om, ref_o, atol=1e-14)
    np.testing.assert_allclose(lm, ref_l, atol=1e-14)


def _torch_shifted_grads(q, k, v, do, q_offset, causal, scale):
    """fp64 torch autograd of attention with an explicitly built shifted mask."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True) for x in (q, k, v))
    s = (qt @ kt.transpose(-1, -2)) * scale
    if causal:
        i = torch.arange(q.shape[-2])[:, None]
        j = torch.arange(k.shape[-2])[None, :]
        s = s.masked_fill(j > i + q_offset, float("-inf"))
    o = torch.softmax(s, -1) @ vt
    o.backward(torch.from_numpy(np.ascontiguousarray(do)))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_key_set_backward_sums_to_the_full_backward(causal):
    """Query and key shards at their positions: the per-pair contributions, with the full
    L and D, add up to the gradients of the whole attention (torch autograd)."""
    S, D = 19, 4
    q, k, v, do = (_rand((2, S, D), t) for t in (110, 111, 112, 113))
    sc = 1 / math.sqrt(D)
    r = oracle.backward(q, k, v, do, scale=sc, causal=causal)
    dq_t, dk_t, dv_t = _torch_shifted_grads(q, k, v, do, 0, causal, sc)
    np.testing.assert_allclose(r["dq"], dq_t, rtol=0, atol=1e-12)
    qb, kb = [0, 7, S], [0, 5, 12, S]      # query shards and key sets
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for qa, qe in zip(qb[:-1], qb[1:]):
        for ka, ke in zip(kb[:-1], kb[1:]):
            gq, gk, gv = oracle.backward_partial(q[:, qa:qe], k[:, ka:ke], v[:, ka:ke],
                                                 do[:, qa:qe], r["lse"][:, qa:qe],
                                                 r["delta_o"][:, qa:qe], q_offset=qa - ka,
                                                 scale=sc, causal=causal)
            dq[:, qa:qe] += gq
            dk[:, ka:ke] += gk
            dv[:, ka:ke] += gv
    np.testing.assert_allclose(dq, dq_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, dk_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv_t, rtol=0, atol=1e-12)


def test_key_set_backward_special_cases():
    S, D = 9, 3
    q, k, v, do = (_rand((1, S, D), t) for t in (120, 121, 122, 123))
    sc = 1 / math.sqrt(D)
    r = oracle.backward(q, k, v, do, scale=sc, causal=True)
    # one set holding every key at offset 0 is the whole backward
    gq, gk, gv = oracle.backward_partial(q, k, v, do, r["lse"], r["delta_o"], 0, sc, True)
    np.testing.assert_allclose(gq, r["dq"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gk, r["dk"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gv, r["dv"], rtol=0, atol=1e-13)
    # keys that no query may see contribute nothing; rows with L = -inf contribute nothing
    gq, gk, gv = oracle.backward_partial(q, k, v, do, r["lse"], r["delta_o"], -S, sc, True)
    assert not gq.any() and not gk.any() and not gv.any()
    lse = r["lse"].copy()
    lse[:] = -np.inf
    gq, gk, gv = oracle.backward_partial(q, k, v, do, lse, r["delta_o"], 0, sc, True)
    assert not gq.any() and not gk.any() and not gv.any()


# ---------------------------------------- library routine (torch fp64 CPU) ---

@pytest.mark.parametrize("S,D,causal,mult", [(33, 16, True, 1.0), (64, 8, True, 3.0),
                                             (20, 12, False, 1.0)])
def test_matches_torch_float64_attention_and_autograd(S, D, causal, mult):
    torch.manual_seed(0)
    q, k, v, do = (torch.randn(2, 3, S, D, dtype=torch.float64) for _ in range(4))
    q = q * mult
    k = k * mult
    scale = 1 / math.sqrt(D)
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    s = (qt @ kt.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    lse_t = torch.logsumexp(s, -1)
    ot = torch.softmax(s, -1) @ vt
    ot.backward(do)
    r = oracle.backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), scale=scale, causal=causal)
    np.testing.assert_allclose(r["o"], ot.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse_t.detach().numpy(), rtol=0, atol=1e-12)
    for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), rtol=0, atol=1e-11, err_msg=name)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    np.testing.assert_allclose(r["o"], ref.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------- sampled mode ---

def test_sampled_mode_matches_full_backward():
    S, D = 70, 8
    q, k, v, do = (x.double().numpy()[0, 0] for x in make_inputs(1, 1, S, D, "f32", seed=3))
    r = oracle.backward(q, k, v, do, causal=True)
    lse, delta = oracle.head_stats(q, k, v, do)
    np.testing.assert_allclose(lse, r["lse"], atol=1e-13)
    np.testing.assert_allclose(delta, r["delta_o"], atol=1e-13)
    idx = [0, 1, 31, 32, 69]
    o, l, dq = oracle.rows(q, k, v, do, idx)
    np.testing.assert_allclose(o, r["o"][idx], atol=1e-13)
    np.testing.assert_allclose(l, r["lse"][idx], atol=1e-13)
    np.testing.assert_allclose(dq, r["dq"][idx], atol=1e-12)
    dk, dv = oracle.cols(q, k, v, do, lse, delta, idx)
    np.testing.assert_allclose(dk, r["dk"][idx], atol=1e-12)
    np.testing.assert_allclose(dv, r["dv"][idx], atol=1e-12)


def test_input_generator_is_seeded_and_cast():
    a = make_inputs(1, 2, 8, 4, "bf16", seed=7)
    b = make_inputs(1, 2, 8, 4, "bf16", seed=7)
    c = make_inputs(1, 2, 8, 4, "bf16", seed=8)
    assert all(x.dtype == torch.bfloat16 for x in a)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[0], c[0])
