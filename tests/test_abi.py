"""C-ABI contract checks that run without a GPU.

The library must load, export every entry point include/fa.h declares, and
reject invalid arguments synchronously, before any device work.  Every call
below carries at least one invalid argument, so nothing is ever launched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("exact_attention_causal_amd.fa")

# fake device addresses: never dereferenced, because each call fails validation
P = 0x100000          # 16-byte aligned
MIS = 0x100008        # 8-byte aligned only


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa_mi355x.so is not built (run __graft_entry__.build())")
    return fa.load_library()


def test_header_declares_the_entry_points():
    assert _declared_functions() == ["fa_bwd", "fa_bwd_noalloc", "fa_bwd_partial", "fa_bwd_preprocess",
                                     "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_partial",
                                     "fa_fwd_workspace_size", "fa_fwd_ws", "fa_get_plan", "fa_merge",
                                     "fa_strerror"]


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(fa.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert fa.fa_strerror(code) and "unknown" not in fa.fa_strerror(code)
    assert fa.fa_strerror(0) == "success"
    assert "unknown" in fa.fa_strerror(17)


def test_workspace_size(lib):
    # one fp32 per row (the base-2 copy of lse), rounded up to 256 bytes; 0 for invalid sizes
    assert fa.fa_bwd_workspace_size(1, 16, 65536, 128, fa.FA_BF16) == 16 * 65536 * 4
    assert fa.fa_bwd_workspace_size(4, 12, 512, 64, fa.FA_F32) == 48 * 512 * 4 + 3 * 2 * 48 * 512 * 64 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 3, 64, fa.FA_BF16) == 256
    assert fa.fa_bwd_workspace_size(1, 1, 0, 64, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 128, 72, fa.FA_BF16) == 0
    # bf16 with fewer than 512 key tiles of 256 (S > 256): + 3*n*B*H*S*D fp32 partials of the
    # split backward, n <= 8 chunks of whole 64-row tiles, at most 256 MiB of partials
    assert fa.fa_bwd_workspace_size(1, 1, 8192, 128, fa.FA_BF16) == 8192 * 4 + 3 * 8 * 8192 * 128 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 65536, 128, fa.FA_BF16) == 65536 * 4 + 3 * 2 * 65536 * 128 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 1000, 80, fa.FA_BF16) == 4096 + 3 * 8 * 1000 * 80 * 4
    # fp32: 128-key dK/dV workgroups, split more readily (64 tiles: 8 chunks at D = 64, 4 at D = 128)
    assert fa.fa_bwd_workspace_size(1, 1, 8192, 64, fa.FA_F32) == 8192 * 4 + 3 * 8 * 8192 * 64 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 8192, 128, fa.FA_F32) == 8192 * 4 + 3 * 4 * 8192 * 128 * 4
    assert fa.fa_bwd_workspace_size(4, 32, 8192, 128, fa.FA_F32) == 128 * 8192 * 4  # 8192 tiles
    assert fa.fa_bwd_workspace_size(2, 16, 8192, 128, fa.FA_BF16) == 32 * 8192 * 4   # enough tiles


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, S=128, D=64, scale=0.125, causal=1,
             dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd(**a)


def _pre(**kw):
    a = dict(o=P, dout=P, delta=P, B=1, H=2, S=128, D=64, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_bwd_preprocess(**a)


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, dout=P, lse=P, delta=P, dq=P, dk=P, dv=P, workspace=P,
             workspace_bytes=1 << 20, B=1, H=2, S=128, D=64, scale=0.125, causal=1, dtype=fa.FA_BF16,
             stream=0)
    a.update(kw)
    return fa.fa_bwd(**a)


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), fa.FA_EINVAL), (dict(lse=None), fa.FA_EINVAL),
    (dict(B=0), fa.FA_EINVAL), (dict(H=-1), fa.FA_EINVAL), (dict(S=0), fa.FA_EINVAL),
    (dict(causal=2), fa.FA_EINVAL), (dict(scale=0.0), fa.FA_EINVAL),
    (dict(scale=-0.1), fa.FA_EINVAL), (dict(scale=float("nan")), fa.FA_EINVAL),
    (dict(scale=float("inf")), fa.FA_EINVAL),
    (dict(D=72), fa.FA_EUNSUPPORTED), (dict(D=256), fa.FA_EUNSUPPORTED),
    (dict(dtype=7), fa.FA_EUNSUPPORTED),
    (dict(q=MIS), fa.FA_EALIGN), (dict(o=MIS), fa.FA_EALIGN), (dict(lse=MIS), fa.FA_EALIGN),
    (dict(B=1 << 20, H=1 << 10, S=1 << 20, D=128), fa.FA_EINVAL),
    (dict(S=(1 << 30) + 1, D=16), fa.FA_EINVAL),
])
def test_fwd_rejects(lib, bad, code):
    assert _fwd(**bad) == code
    # fa_fwd_ws checks the same arguments first (with and without a workspace)
    assert _fwd_ws(**bad) == code
    assert _fwd_ws(workspace=None, workspace_bytes=0, **bad) == code


def _fwd_ws(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, workspace=P, workspace_bytes=1 << 20, B=1, H=2, S=128, D=64,
             scale=0.125, causal=1, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd_ws(**a)


def test_fwd_ws_rejects_a_misaligned_workspace(lib):
    assert _fwd_ws(workspace=MIS) == fa.FA_EALIGN


def test_fwd_workspace_size(lib):
    # 0 where fa_fwd_ws runs as fa_fwd; else n chunks of fp32 partial O and L (two regions,
    # each rounded up to 256 bytes)
    assert fa.fa_fwd_workspace_size(1, 16, 65536, 128, fa.FA_BF16) == 0      # many tiles
    assert fa.fa_fwd_workspace_size(1, 1, 1024, 128, fa.FA_BF16) == 0        # bf16: S < 2048
    # bf16, one head of 4096 (16 tiles of 256): 8 chunks
    assert fa.fa_fwd_workspace_size(1, 1, 4096, 128, fa.FA_BF16) == 8 * 4096 * 128 * 4 + 8 * 4096 * 4
    # bf16, 48 tiles: 4 chunks
    assert fa.fa_fwd_workspace_size(1, 3, 4096, 64, fa.FA_BF16) == 4 * 3 * 4096 * 64 * 4 + 4 * 3 * 4096 * 4
    # bf16 D <= 32 (no two-group tile), S >= 4096: 6 (causal) chunks up to one tile per CU, and up
    # to two from S = 16384 on
    for B, H, S, D in [(1, 1, 32768, 16), (1, 4, 8192, 32), (1, 16, 4096, 16), (1, 8, 16384, 32)]:
        assert fa.fa_fwd_workspace_size(B, H, S, D, fa.FA_BF16) == 6 * B * H * S * D * 4 + 6 * B * H * S * 4
    assert fa.fa_fwd_workspace_size(1, 32, 2048, 16, fa.FA_BF16) == 0    # S < 4096
    assert fa.fa_fwd_workspace_size(1, 16, 8192, 32, fa.FA_BF16) == 0    # 512 tiles, S < 16384
    assert fa.fa_fwd_workspace_size(1, 4, 8192, 64, fa.FA_BF16) == 3 * 4 * 8192 * 64 * 4 + 3 * 4 * 8192 * 4  # CU/2
    assert fa.fa_fwd_workspace_size(1, 8, 8192, 64, fa.FA_BF16) == 0     # D = 64, 256 tiles: two key groups
    assert fa.fa_fwd_workspace_size(1, 8, 4096, 128, fa.FA_BF16) == 0    # CU/2 tiles, S < 8192
    # fp32, 32 tiles: ceil(256/32) = 8 chunks; 64 tiles at S >= 4096: 16; 256 tiles: 2
    assert fa.fa_fwd_workspace_size(1, 1, 8192, 64, fa.FA_F32) == 8 * 8192 * 64 * 4 + 8 * 8192 * 4
    assert fa.fa_fwd_workspace_size(1, 4, 4096, 64, fa.FA_F32) == 16 * 4 * 4096 * 64 * 4 + 16 * 4 * 4096 * 4
    assert fa.fa_fwd_workspace_size(1, 16, 4096, 64, fa.FA_F32) == 2 * 16 * 4096 * 64 * 4 + 2 * 16 * 4096 * 4
    assert fa.fa_fwd_workspace_size(1, 16, 4096, 32, fa.FA_F32) == 8 * 16 * 4096 * 32 * 4 + 8 * 16 * 4096 * 4  # D <= 32
    # fp32, one head of 512: ceil(256/2) = 128 wanted, at most S/64 = 8 chunks of 64 keys
    assert fa.fa_fwd_workspace_size(1, 1, 512, 64, fa.FA_F32) == 8 * 512 * 64 * 4 + 8 * 512 * 4
    # fp32 D = 128 counts tiles of 128 queries: 16 tiles: 256/16 = 16 chunks; 64: 4; 128: 3;
    # 256 (causal): 2
    assert fa.fa_fwd_workspace_size(1, 1, 2048, 128, fa.FA_F32) == 16 * 2048 * 128 * 4 + 16 * 2048 * 4
    assert fa.fa_fwd_workspace_size(1, 1, 8192, 128, fa.FA_F32) == 4 * 8192 * 128 * 4 + 4 * 8192 * 4
    assert fa.fa_fwd_workspace_size(2, 4, 2048, 128, fa.FA_F32) == 3 * 8 * 2048 * 128 * 4 + 3 * 8 * 2048 * 4
    assert fa.fa_fwd_workspace_size(1, 1, 32768, 128, fa.FA_F32) == 2 * 32768 * 128 * 4 + 2 * 32768 * 4
    assert fa.fa_fwd_workspace_size(1, 1, 65536, 128, fa.FA_F32) == 2 * 65536 * 128 * 4 + 2 * 65536 * 4  # 512
    assert fa.fa_fwd_workspace_size(1, 2, 65536, 128, fa.FA_F32) == 0   # 1024 tiles
    assert fa.fa_fwd_workspace_size(1, 1, 0, 64, fa.FA_BF16) == 0
    assert fa.fa_fwd_workspace_size(1, 1, 128, 72, fa.FA_BF16) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(o=None), fa.FA_EINVAL), (dict(delta=None), fa.FA_EINVAL), (dict(S=-5), fa.FA_EINVAL),
    (dict(D=48), fa.FA_EUNSUPPORTED), (dict(dtype=3), fa.FA_EUNSUPPORTED),
    (dict(dout=MIS), fa.FA_EALIGN), (dict(delta=P + 4), fa.FA_EALIGN),
])
def test_preprocess_rejects(lib, bad, code):
    assert _pre(**bad) == code


@pytest.mark.parametrize("bad,code", [
    (dict(dq=None), fa.FA_EINVAL), (dict(delta=None), fa.FA_EINVAL), (dict(H=0), fa.FA_EINVAL),
    (dict(causal=-1), fa.FA_EINVAL), (dict(scale=float("-inf")), fa.FA_EINVAL),
    (dict(D=100), fa.FA_EUNSUPPORTED), (dict(dtype=2), fa.FA_EUNSUPPORTED), (dict(S=(1 << 30) + 64), fa.FA_EINVAL),
    (dict(dk=MIS), fa.FA_EALIGN), (dict(lse=P + 2), fa.FA_EALIGN),
    (dict(workspace=None), fa.FA_EINVAL), (dict(workspace=MIS), fa.FA_EALIGN),
    (dict(workspace_bytes=2 * 128 * 4 - 1), fa.FA_EWORKSPACE), (dict(workspace_bytes=0), fa.FA_EWORKSPACE),
])
def test_bwd_rejects(lib, bad, code):
    assert _bwd(**bad) == code


def _part(**kw):
    a = dict(q=P, k=P, v=P, o_parts=P, lse_parts=P, B=1, H=2, Sq=100, Sk=300, D=64, scale=0.125,
             causal=1, q_offset=200, n_split=3, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd_partial(**a)


def _merge(**kw):
    a = dict(o_parts=P, lse_parts=P, n_parts=3, o=P, lse=P, B=1, H=2, S=100, D=64,
             dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_merge(**a)


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), fa.FA_EINVAL), (dict(lse_parts=None), fa.FA_EINVAL), (dict(Sq=0), fa.FA_EINVAL),
    (dict(Sk=-1), fa.FA_EINVAL), (dict(n_split=0), fa.FA_EINVAL), (dict(n_split=70000), fa.FA_EINVAL),
    (dict(causal=3), fa.FA_EINVAL), (dict(scale=0.0), fa.FA_EINVAL), (dict(Sk=(1 << 29) + 1), fa.FA_EINVAL),
    (dict(B=1 << 16, H=1 << 10, Sq=1 << 20, D=128, n_split=1000), fa.FA_EINVAL),
    (dict(D=40), fa.FA_EUNSUPPORTED), (dict(dtype=5), fa.FA_EUNSUPPORTED),
    (dict(o_parts=MIS), fa.FA_EALIGN), (dict(k=MIS), fa.FA_EALIGN),
])
def test_fwd_partial_rejects(lib, bad, code):
    assert _part(**bad) == code


@pytest.mark.parametrize("bad,code", [
    (dict(o=None), fa.FA_EINVAL), (dict(lse_parts=None), fa.FA_EINVAL), (dict(n_parts=0), fa.FA_EINVAL),
    (dict(S=0), fa.FA_EINVAL), (dict(B=1 << 16, H=1 << 10, S=1 << 20, D=128, n_parts=1000), fa.FA_EINVAL),
    (dict(D=24), fa.FA_EUNSUPPORTED), (dict(dtype=9), fa.FA_EUNSUPPORTED),
    (dict(lse=MIS), fa.FA_EALIGN), (dict(o_parts=P + 8), fa.FA_EALIGN),
])
def test_merge_rejects(lib, bad, code):
    assert _merge(**bad) == code


def _bpart(**kw):
    a = dict(q=P, k=P, v=P, dout=P, lse=P, delta=P, dq_acc=P, dk_acc=P, dv_acc=P, accumulate=1,
             B=1, H=2, Sq=100, Sk=300, D=64, scale=0.125, causal=1, q_offset=200,
             dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_bwd_partial(**a)


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), fa.FA_EINVAL), (dict(delta=None), fa.FA_EINVAL), (dict(dv_acc=None), fa.FA_EINVAL),
    (dict(Sq=0), fa.FA_EINVAL), (dict(Sk=-3), fa.FA_EINVAL), (dict(accumulate=2), fa.FA_EINVAL),
    (dict(accumulate=-1), fa.FA_EINVAL), (dict(causal=5), fa.FA_EINVAL), (dict(scale=float("nan")), fa.FA_EINVAL),
    (dict(Sq=(1 << 29) + 1), fa.FA_EINVAL), (dict(Sk=(1 << 29) + 1), fa.FA_EINVAL), (dict(B=1 << 20, H=1 << 10, Sk=1 << 20, D=128), fa.FA_EINVAL),
    (dict(D=112), fa.FA_EUNSUPPORTED), (dict(dtype=4), fa.FA_EUNSUPPORTED),
    (dict(dk_acc=MIS), fa.FA_EALIGN), (dict(lse=P + 4), fa.FA_EALIGN), (dict(dout=MIS), fa.FA_EALIGN),
])
def test_bwd_partial_rejects(lib, bad, code):
    assert _bpart(**bad) == code


def test_split_chunk_rule():
    # 64-key multiples covering Sk in n_split chunks (the last one may be short or empty)
    for Sk, n in ((300, 3), (64, 1), (65, 2), (1, 4), (65536, 7)):
        c = fa.split_chunk(Sk, n)
        assert c % 64 == 0 and c * n >= Sk and c * (n - 1) < Sk + 64 * n


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def _noalloc(**kw):
    a = dict(q=P, k=P, v=P, dout=P, lse=P, delta=P, dq=P, dk=P, dv=P, B=1, H=2, S=128, D=64,
             scale=0.125, causal=1, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_bwd_noalloc(**a)


@pytest.mark.parametrize("bad,code", [
    (dict(q=None), fa.FA_EINVAL), (dict(dv=None), fa.FA_EINVAL), (dict(B=0), fa.FA_EINVAL),
    (dict(causal=2), fa.FA_EINVAL), (dict(scale=0.0), fa.FA_EINVAL),
    (dict(D=72), fa.FA_EUNSUPPORTED), (dict(dtype=3), fa.FA_EUNSUPPORTED),
    (dict(dq=MIS), fa.FA_EALIGN), (dict(lse=P + 4), fa.FA_EALIGN),
    # the fixed scratch holds the base-2 lse of at most 2^24 rows
    (dict(B=1, H=257, S=65536, D=64), fa.FA_ESCRATCH), (dict(B=2, H=1, S=(1 << 23) + 1, D=16), fa.FA_ESCRATCH),
])
def test_bwd_noalloc_rejects(lib, bad, code):
    assert _noalloc(**bad) == code


def _plan(B, H, S, D, dtype, ncu):
    rc, p = fa.fa_get_plan(B, H, S, D, dtype, ncu)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    assert p.num_cu == ncu
    return p


def test_plan_thresholds_follow_the_cu_count(lib):
    """Tile selection is a function of the device's compute units: every threshold moves with them."""
    bf, f32 = fa.FA_BF16, fa.FA_F32
    # S=65536, D=128, 16 heads: 2048 tiles of 512 queries = 8 per CU on 256 CUs (64 queries per
    # wave, S >= 16384); below 2 per CU (1024 CUs) the 256-query tile; at 1.5 tiles of 256 per CU
    # or fewer (2731 CUs and up) two key groups on 128-query tiles
    p = _plan(1, 16, 65536, 128, bf, 256)
    assert (p.fwd_block_queries, p.fwd_key_tile, p.fwd_band) == (512, 32, 64)   # 16 heads: banded order
    assert _plan(1, 12, 65536, 128, bf, 256).fwd_band == 0    # 12 heads do not split over 8 XCDs
    assert _plan(1, 32, 16000, 80, bf, 256).fwd_band == 0     # D = 80: consecutive heads
    assert _plan(1, 16, 65536, 128, bf, 1024).fwd_block_queries == 512   # exactly 2 per CU
    assert _plan(1, 16, 65536, 128, bf, 1025).fwd_block_queries == 256
    assert _plan(1, 64, 8192, 128, bf, 256).fwd_block_queries == 256     # 4 per CU, but S < 16384
    assert _plan(1, 64, 1024, 128, bf, 256).fwd_key_groups == 1          # one tile per CU, S < 2048
    assert _plan(1, 32, 2048, 128, bf, 256).fwd_key_groups == 2          # one tile per CU, S >= 2048
    assert _plan(1, 16, 65536, 128, bf, 2730).fwd_key_groups == 1        # 4096 > 1.5 * 2730
    p = _plan(1, 16, 65536, 128, bf, 2731)
    assert (p.fwd_block_queries, p.fwd_key_groups, p.fwd_key_tile) == (128, 2, 32)
    # D <= 80: two key groups up to one tile of 256 per CU, and up to 2 from S = 4096 on
    assert _plan(1, 32, 2048, 64, bf, 256).fwd_key_groups == 2          # 256 tiles
    assert _plan(1, 64, 2048, 64, bf, 256).fwd_key_groups == 1          # 512 tiles, S < 4096
    # (32 heads of 16000: 2016 tiles)
    assert _plan(1, 32, 16000, 80, bf, 1007).fwd_key_groups == 1
    p = _plan(1, 32, 16000, 80, bf, 1008)
    assert (p.fwd_block_queries, p.fwd_key_groups, p.fwd_key_tile) == (128, 2, 64)
    p = _plan(1, 32, 16000, 80, bf, 256)
    assert (p.fwd_block_queries, p.fwd_key_groups, p.fwd_key_tile) == (256, 1, 64)
    # fp32 never takes the bf16-only tiles; wide fp32 heads use 32-key tiles
    p = _plan(1, 1, 4096, 128, f32, 256)
    assert (p.fwd_block_queries, p.fwd_key_groups, p.fwd_key_tile, p.bwd_chunks) == (256, 1, 32, 8)
    # fp32 split: t = B*H*ceil(S/128) dK/dV workgroups; 8 chunks up to CU/4 or S/32, 4 up to CU/2,
    # 2 up to 2 CU
    assert _plan(1, 16, 1024, 64, f32, 256).bwd_chunks == 4     # t = 128
    assert _plan(1, 32, 1024, 64, f32, 256).bwd_chunks == 2     # t = 256
    assert _plan(1, 4, 8192, 64, f32, 256).bwd_chunks == 8      # t = 256 <= S/32
    assert _plan(1, 32, 4096, 64, f32, 256).bwd_chunks == 1     # t = 1024
    # fp32 D = 128 (4-wave dQ workgroups): 8 up to CU/8, 4 up to CU/4, 3 up to CU/2, 2 up to 2 CU
    assert _plan(1, 1, 4096, 128, f32, 256).bwd_chunks == 8     # t = 32
    assert _plan(1, 1, 8192, 128, f32, 256).bwd_chunks == 4     # t = 64
    assert _plan(2, 4, 2048, 128, f32, 256).bwd_chunks == 3     # t = 128
    assert _plan(1, 4, 8192, 128, f32, 256).bwd_chunks == 2     # t = 256 (S/32 no longer counts)
    assert _plan(1, 8, 8192, 128, f32, 256).bwd_chunks == 2     # t = 512
    assert _plan(1, 16, 8192, 128, f32, 256).bwd_chunks == 1    # t = 1024
    # fp32 at S <= 256: chunks of 64 rows up to CU/2 tiles, none from S <= 64 or past CU/2
    p = _plan(1, 1, 200, 80, f32, 256)
    assert (p.bwd_chunks, p.bwd_chunk_rows) == (4, 64)
    assert _plan(4, 16, 256, 64, f32, 256).bwd_chunks == 4      # t = 128
    assert _plan(8, 16, 256, 64, f32, 256).bwd_chunks == 1      # t = 256
    assert _plan(1, 1, 64, 64, f32, 256).bwd_chunks == 1
    assert _plan(1, 1, 256, 64, bf, 256).bwd_chunks == 1        # bf16: S <= 256 never splits
    # split backward: below one dK/dV tile of 256 keys per CU, n = ceil(CU / tiles) <= 8 chunks;
    # one to two tiles per CU: 2 chunks from S = 4096 on; S <= 512: 4 chunks below CU/16 tiles
    p = _plan(1, 1, 8192, 128, bf, 256)          # 32 tiles: 8 wanted
    assert (p.bwd_chunks, p.bwd_chunk_rows) == (8, 1024)
    p = _plan(1, 16, 1024, 128, bf, 256)         # 64 tiles: 4
    assert (p.bwd_chunks, p.bwd_chunk_rows) == (4, 256)
    p = _plan(1, 1, 8192, 128, bf, 32)           # 32 tiles on 32 CUs, S >= 4096: 2
    assert (p.bwd_chunks, p.bwd_chunk_rows) == (2, 4096)
    assert _plan(4, 16, 1024, 64, bf, 256).bwd_chunks == 1  # 256 tiles on 256 CUs, S < 4096
    assert _plan(1, 1, 8192, 128, bf, 16).bwd_chunks == 1   # already 2 tiles per CU
    p = _plan(1, 1, 512, 64, bf, 256)            # S <= 512, 2 tiles: 4 chunks of 128 rows
    assert (p.bwd_chunks, p.bwd_chunk_rows) == (4, 128)
    assert _plan(4, 12, 512, 64, bf, 256).bwd_chunks == 1   # S <= 512, 96 tiles: the partials cost more
    assert _plan(1, 2, 16384, 64, bf, 256).bwd_chunks == 3  # CU/2 tiles, S >= 4096: at least 3 chunks
    assert _plan(1, 32, 1024, 64, bf, 256).bwd_chunks == 2  # CU/2 tiles, S < 4096: ceil(CU / tiles)
    assert _plan(1, 3, 16384, 128, bf, 256).bwd_chunks == 2  # 192 tiles: 2
    assert _plan(1, 4, 16384, 16, bf, 256).bwd_chunks == 8  # D = 16 (two workgroups per CU), S >= 4096
    assert _plan(1, 32, 2048, 16, bf, 256).bwd_chunks == 3  # D = 16, S < 4096
    assert _plan(2, 32, 4096, 16, bf, 256).bwd_chunks == 1  # D = 16, 1024 tiles
    p = _plan(1, 1, 65536, 128, bf, 256)         # 256 tiles: 2 wanted, 2 fit in 256 MiB
    assert (p.bwd_chunks, p.bwd_chunk_rows) == (2, 32768)
    assert _plan(1, 1, 65536, 128, bf, 128).bwd_chunks == 1
    assert _plan(1, 1, 65536, 128, bf, 4096).bwd_chunks == 2     # 32 wanted; the partials cap at 2
    assert _plan(1, 16, 65536, 128, bf, 4096).bwd_chunks == 1    # partials of 2 chunks: 1.5 GiB


def test_plan_rejects(lib):
    assert fa.fa_get_plan(1, 1, 0, 64, fa.FA_BF16, 256)[0] == fa.FA_EINVAL
    assert fa.fa_get_plan(1, 1, 128, 72, fa.FA_BF16, 256)[0] == fa.FA_EUNSUPPORTED
    assert fa.load_library().fa_get_plan(1, 1, 128, 64, 1, 256, None) == fa.FA_EINVAL


def test_header_is_plain_c(tmp_path):
    """include/fa.h declares a C ABI: a C99 translation unit that calls every entry point
    compiles against it (and so does C++)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(r'''
#include "fa.h"
int use(void *p, hipStream_t st) {
    fa_plan plan;
    int rc = fa_get_plan(1, 2, 128, 64, FA_BF16, 256, &plan);
    rc |= fa_fwd(p, p, p, p, (float *)p, 1, 2, 128, 64, 0.125f, 1, FA_BF16, st);
    rc |= fa_bwd_preprocess(p, p, (float *)p, 1, 2, 128, 64, FA_BF16, st);
    size_t ws = fa_bwd_workspace_size(1, 2, 128, 64, FA_BF16);
    rc |= fa_bwd(p, p, p, p, (const float *)p, (const float *)p, p, p, p, p, ws, 1, 2, 128, 64, 0.125f, 1,
                 FA_BF16, st);
    rc |= fa_bwd_noalloc(p, p, p, p, (const float *)p, (const float *)p, p, p, p, 1, 2, 128, 64, 0.125f, 1,
                         FA_F32, st);
    rc |= fa_fwd_partial(p, p, p, (float *)p, (float *)p, 1, 2, 128, 256, 64, 0.125f, 1, 128, 2, FA_BF16, st);
    rc |= fa_merge((const float *)p, (const float *)p, 2, p, (float *)p, 1, 2, 128, 64, FA_BF16, st);
    rc |= fa_bwd_partial(p, p, p, p, (const float *)p, (const float *)p, (float *)p, (float *)p, (float *)p, 0,
                         1, 2, 128, 256, 64, 0.125f, 1, 128, FA_BF16, st);
    return rc + (fa_strerror(rc) != 0) + plan.num_cu;
}
''')
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        r = subprocess.run([cc, "-x", lang, std, "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                            "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
