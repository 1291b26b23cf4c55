"""The build module's resource report (CPU: hipcc cross-compiles for gfx950).

kernel_label turns this library's kernel symbols into readable names; the
report compiles device code with the library's flags and reads the
compiler's per-kernel remarks.
"""
import os

import pytest

from exact_attention_causal_amd import build


@pytest.mark.parametrize("sym,label", [
    ("_ZN2fa10fwd_kernelIDF16bNS_7FwdTileIDF16bLi128ELi2ELi32ELi8ELi1EEEDF16bLb0EEEvPKT_S5_S5_PT1_PfNS_8FwdShapeE",
     "fwd_kernel<bf16, FwdTile<bf16, 128, 2, 32, 8, 1>, bf16, false>"),
    ("_ZN2fa12dkdv1_kernelIDF16bNS_7KvTile1IDF16bLi128ELi8ELb1ELi2ELi2ELi4EEEDF16bLb0EEEvPKT_S5_S5_S5_PKfS7_PT1_"
     "S9_NS_8BwdShapeE", "dkdv1_kernel<bf16, KvTile1<bf16, 128, 8, true, 2, 2, 4>, bf16, false>"),
    ("_ZN2fa9dq_kernelIfNS_5QTileIfLi80ELi1ELi64ELi8EEEfLb1EEEvPKT_S5_S5_S5_PKfS7_PT1_NS_8BwdShapeE",
     "dq_kernel<float, QTile<float, 80, 1, 64, 8>, float, true>"),
    ("_ZN2fa12delta_kernelIDF16bLi128EEEvPKT_S3_Pfx", "delta_kernel<bf16, 128>"),
    ("_ZN2fa1kILin5EEEvv", "k<-5>"),
    ("_ZN2fa11lse2_kernelEPKfPfx", "lse2_kernel"),
    ("_Z3fooi", "_Z3fooi"),                               # not in namespace fa: unchanged
    ("_ZN2fa10fwd_kernelIDF16bNS_7FwdTileIQ", "_ZN2fa10fwd_kernelIDF16bNS_7FwdTileIQ"),  # malformed: unchanged
])
def test_kernel_label(sym, label):
    assert build.kernel_label(sym) == label


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_resource_report_of_one_source(monkeypatch):
    # one small translation unit keeps this quick; the report parses every
    # kernel the compiler remarks on
    monkeypatch.setattr(build, "SOURCES", ["fa_merge.hip"])
    rows = build.resources()
    names = {r["name"] for r in rows}
    assert {"merge_kernel<bf16, 128>", "merge_kernel<float, 80>"} <= names
    for r in rows:
        assert r["source"] == "fa_merge.hip"
        assert 0 < r["vgprs"] <= 512 and r["agprs"] >= 0
        assert r["spills"] == 0 and r["scratch"] == 0 and r["lds"] == 0
        assert 1 <= r["waves_per_simd"] <= 8
    only = build.resources("merge_kernel<bf16, 128>")
    assert [r["name"] for r in only] == ["merge_kernel<bf16, 128>"]


def test_peak_library_rejects_bad_arguments():
    # the matrix-core microbenchmark library (bench.py --peak): argument checks and the FLOP
    # count, no launch
    import ctypes
    if not os.path.exists(build.PEAK_LIB):
        pytest.fail("libfa_peak.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(build.PEAK_LIB)
    lib.fa_peak_mfma.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_peak_mfma_flop.argtypes = [ctypes.c_int] * 3
    lib.fa_peak_mfma_flop.restype = ctypes.c_double
    out = 0x100000
    for dtype, mode, blocks, iters, ptr in [(3, 0, 1, 1, out), (-1, 0, 1, 1, out), (1, 3, 1, 1, out), (1, 0, 0, 1, out),
                                            (1, 0, 1, 0, out), (0, 0, 1, 1, None), (1, 0, (1 << 22) + 1, 1, out)]:
        assert lib.fa_peak_mfma(dtype, mode, blocks, iters, ptr, None) == -1
    # 4 waves x 16 instructions per round: 32768 FLOP each (bf16 32x32x16), 16384 (bf16
    # 16x16x32), 4096 (fp32 32x32x2)
    assert lib.fa_peak_mfma_flop(1, 3, 5) == 3 * 4 * 5 * 16 * 32768
    assert lib.fa_peak_mfma_flop(2, 3, 5) == 3 * 4 * 5 * 16 * 16384
    assert lib.fa_peak_mfma_flop(0, 3, 5) == 3 * 4 * 5 * 16 * 4096
    assert lib.fa_peak_mfma_flop(3, 3, 5) == 0
