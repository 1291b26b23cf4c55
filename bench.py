"""Benchmark: causal attention forward and forward+backward on one MI355X.

One step = the whole hot path over one batch of seeded synthetic inputs that
are already resident in HBM: fa_fwd (O, L), fa_bwd_preprocess (D) and fa_bwd
(dQ, dK, dV), all through the C ABI on one stream.  Throughput counts the
algorithmic causal FLOPs, 4*D per allowed (query, key) pair for the forward
and 14*D per pair for forward+backward (five contractions in the backward;
recomputation, masked halves of diagonal tiles and head-dimension padding are
not counted).

Prints one JSON line.  `roofline` covers the forward kernel (one kernel per
fa_fwd call, timed with HIP events on the stream it runs on);
`roofline_bwd` covers the backward launch pair of fa_bwd.  `cpu_baseline`
times the fp64 CPU oracle on a bounded slice of the same workload.
"""
import argparse
import json
import statistics
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_causal_amd import fa  # noqa: E402
from exact_attention_causal_amd.inputs import WORKLOADS, workload_inputs  # noqa: E402

METRIC = "causal attention fwd & fwd+bwd TFLOP/s (bf16) + % of MFMA peak, 1 GPU"
PEAK_BF16 = 2516.6   # TFLOP/s, dense bf16 matrix cores (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_F32 = 157.3     # TFLOP/s, dense fp32 matrix cores
DEFAULT_WORKLOAD = "bf16_b1h16_s65536_d128"
# the other workload with a throughput target (S >= 16k), timed beside the headline one
EXTRA_WORKLOADS = ("bf16_b1h32_s16000_d80",)

# HBM traffic of one forward-kernel launch on each long workload, from two
# rocprofv3 --pmc passes (FETCH_SIZE x 2.0 and WRITE_SIZE x 1.0, the factors a
# plain 1 GiB copy calibrates; profiles/attn_bf16_*.md), keyed
# by a hash of every source the forward kernel and its launch plan compile
# from: once one changes, the figure is stale and reported as null until the
# counters are taken again.
FWD_TRAFFIC = {"sources_sha1": "9827a2ffe460393ce388154c73575108f1256afb",
               "bytes": {"bf16_b1h16_s65536_d128": 4669211296, "bf16_b1h32_s16000_d80": 2103765536}}
FWD_SOURCES = ("exact_attention_causal_amd/csrc/fa_fwd.hip", "exact_attention_causal_amd/csrc/fa_common.hpp",
               "exact_attention_causal_amd/csrc/fa_launch.hpp")


def fwd_sources_sha1():
    import hashlib
    h = hashlib.sha1()
    for f in FWD_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (not also the other long workload)")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the sampled oracle check of the timed step's outputs")
    ap.add_argument("--cpu-tokens", type=int, default=12288,
                    help="sequence prefix the CPU oracle baseline runs on")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; "
                         "its HBM counters calibrate the traffic figures")
    ap.add_argument("--hold", type=float, default=0.0, metavar="SECONDS",
                    help="only run the --hold-entry entry point back to back for SECONDS "
                         "(for sampling clocks and board power alongside) and exit")
    ap.add_argument("--hold-entry", default="fwd", choices=("fwd", "bwd"))
    ap.add_argument("--split-kv", type=int, default=0, metavar="N",
                    help="only time the split-KV forward of the workload (fa_fwd_partial over N key "
                         "chunks, then fa_merge) and print its own JSON line: the partial forward "
                         "against the matrix-core peak, the merge against HBM bandwidth")
    ap.add_argument("--vs-materialised", action="store_true",
                    help="time and peak memory of fwd+bwd against attention with the S x S matrix "
                         "materialised (fp32 PyTorch ops), batch 8, one head")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the benchmark sweep (B=1, H=1, S = 128 .. 65536 in powers of "
                         "two, D in 16/32/64/128, bf16 and fp32, causal and not), print a "
                         "markdown table and exit")
    ap.add_argument("--shapes", action="store_true",
                    help="only time forward and forward+backward (bf16, causal) on a list of common "
                         "training shapes, print a markdown table and exit")
    ap.add_argument("--peak", action="store_true",
                    help="only run the matrix-core microbenchmark (libfa_peak.so): bf16 32x32x16, 16x16x32 and "
                         "fp32 32x32x2 MFMA loops with no memory traffic, on zero, constant and "
                         "random operands; print one JSON line per case and exit")
    ap.add_argument("--graph", action="store_true",
                    help="only time whole fwd+bwd steps launched one call at a time against the "
                         "same step captured once as a HIP graph and replayed, on the small "
                         "workloads and one-head shapes; print a markdown table and exit")
    return ap.parse_args()


def cpu_baseline(w, q, k, v, do, tokens):
    """fp64 oracle forward+backward on the first `tokens` positions of every head.

    Causal attention restricted to a prefix of the sequence is the same
    computation on a smaller triangle, so its FLOP rate is the oracle's rate
    on this workload's shapes and head dimension.
    """
    import oracle
    S = min(tokens, w.S)
    sl = [x[:, :, :S].double().numpy() for x in (q, k, v, do)]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    t0 = time.perf_counter()
    oracle.backward(*sl, scale=w.scale, causal=True, nthreads=threads)
    dt = time.perf_counter() - t0
    pairs = w.B * w.H * S * (S + 1) // 2
    return {"value": 14 * w.D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": dt, "cpu_model": cpu_model(),
            "sample": f"fp64 oracle fwd+bwd on the first {S} tokens of all {w.B * w.H} heads "
                      f"(causal prefix of the same Q/K/V/dO), 14*D*pairs FLOPs / wall time"}


def cpu_model():
    """The host CPU's model name (as lscpu reports it, read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def sampled_errors(w, cpu_in, outs, heads=1, per_head=64):
    """Errors of one step's outputs against the fp64 oracle on seeded rows of a few heads.

    O, L and dQ at the sampled query rows, dK and dV at the same key rows (with the
    oracle's own L and D for every row of the sampled heads); max |gpu - oracle| /
    max |oracle| per tensor, L in absolute terms.
    """
    import numpy as np
    import oracle
    from exact_attention_causal_amd.inputs import sample_head_rows
    BH = w.B * w.H
    qn, kn, vn, don = (x.reshape(BH, w.S, w.D) for x in cpu_in)
    samples = sample_head_rows(BH, w.S, heads, per_head)
    ref = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    got = {n: [] for n in ref}
    for hh, rows in samples:
        qh, kh, vh, dh = (x[hh].double().numpy() for x in (qn, kn, vn, don))
        lse_full, del_full = oracle.head_stats(qh, kh, vh, dh, scale=w.scale)
        o, lse, dq = oracle.rows(qh, kh, vh, dh, rows, scale=w.scale)
        dk, dv = oracle.cols(qh, kh, vh, dh, lse_full, del_full, rows, scale=w.scale)
        for n, r in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            ref[n].append(r)
            t = outs[n].reshape(BH, w.S, -1)[hh][rows] if n != "lse" else outs[n].reshape(BH, w.S)[hh][rows]
            got[n].append(t.double().cpu().numpy())
    err = {}
    for n in ref:
        a, b = np.concatenate(got[n]), np.concatenate(ref[n])
        d = float(np.max(np.abs(a - b)))
        err[n] = d if n == "lse" else d / float(np.max(np.abs(b)))
    tol = {"o": 2e-2, "lse": 1e-3, "dq": 5e-2, "dk": 5e-2, "dv": 5e-2} if w.dtype == "bf16" else \
        {"o": 1e-4, "lse": 1e-3, "dq": 1e-4, "dk": 1e-4, "dv": 1e-4}
    return {"max_err": {n: float(f"{e:.3e}") for n, e in err.items()},
            "tolerance": tol, "within_tolerance": all(err[n] <= tol[n] for n in err),
            "sample": f"{len(samples)} seeded head(s) x {per_head} rows (sequence ends and tile edges "
                      f"included) of the last timed step; O, L, dQ at those query rows, dK, dV at "
                      f"the same key rows; errors relative to the oracle's max |x| (L absolute)",
            "heads": [h for h, _ in samples]}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def split_kv(dev, w, n_split, steps, warmup, with_cpu):
    """Split-KV forward of one workload: fa_fwd_partial over n_split key chunks + fa_merge.

    The partial forward does the same 4*D*pairs FLOPs as fa_fwd (rated against the
    matrix-core peak); the merge is bound by HBM: it reads n_split fp32 partial
    outputs and logsumexps and writes O and L (rated against 8 TB/s).
    """
    fa.load_library()
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
    B, H, S, D = w.shape
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    q, k, v, _ = workload_inputs(w)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    op = torch.empty((n_split, B, H, S, D), device=dev, dtype=torch.float32)
    lp = torch.empty((n_split, B, H, S), device=dev, dtype=torch.float32)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, S), device=dev, dtype=torch.float32)

    def part():
        rc = fa.fa_fwd_partial(qd, kd, vd, op, lp, B, H, S, S, D, w.scale, 1, 0, n_split, code, sh)
        assert rc == 0, fa.fa_strerror(rc)

    def merge():
        rc = fa.fa_merge(op, lp, n_split, o, lse, B, H, S, D, code, sh)
        assert rc == 0, fa.fa_strerror(rc)

    for _ in range(warmup):
        part(); merge()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream); part(); e[1].record(stream); merge(); e[2].record(stream)
    torch.cuda.synchronize()
    t_part = statistics.median(e[0].elapsed_time(e[1]) for e in ev)
    t_merge = statistics.median(e[1].elapsed_time(e[2]) for e in ev)
    pairs = w.causal_pairs()
    tf = 4 * D * pairs / (t_part * 1e-3) / 1e12
    esize = 2 if w.dtype == "bf16" else 4
    mbytes = n_split * B * H * S * (D + 1) * 4 + B * H * S * (D * esize + 4)
    gbs = mbytes / (t_merge * 1e-3) / 1e9
    peak = PEAK_BF16 if w.dtype == "bf16" else PEAK_F32
    rec = {"mode": "split_kv_forward", "config": {"workload": w.name, "n_split": n_split},
           "steps": steps, "warmup": warmup,
           "ms": {"fwd_partial": round(t_part, 4), "merge": round(t_merge, 4),
                  "total": round(t_part + t_merge, 4)},
           "fwd_tflops": round(4 * D * pairs / ((t_part + t_merge) * 1e-3) / 1e12, 2),
           "roofline_partial": {"kernel": "fwd_kernel (fa_fwd_partial)", "bound": "mfma",
                                "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                                "frac": round(tf / peak, 4)},
           "roofline_merge": {"kernel": "merge_kernel (fa_merge)", "bound": "hbm",
                              "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                              "frac": round(gbs / 8000.0, 4), "algorithmic_bytes": mbytes}}
    if with_cpu:
        # the oracle's merge of the same kind of parts on the first heads (a bounded sample)
        import numpy as np
        import oracle
        hs = max(1, min(B * H, (1 << 28) // (n_split * S * D)))
        opn = op.view(n_split, B * H, S, D)[:, :hs].double().cpu().numpy()
        lpn = lp.view(n_split, B * H, S)[:, :hs].double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.merge(opn, lpn)
        dt = time.perf_counter() - t0
        nb = n_split * hs * S * (D + 1) * 8 + hs * S * (D + 1) * 8
        rec["cpu_baseline"] = {"value": round(nb / dt / 1e9, 3), "unit": "GB/s (fp64)",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count(),
                               "kind": "oracle", "seconds": dt,
                               "sample": f"fp64 oracle merge of the same {n_split} parts for {hs} of "
                                         f"{B * H} heads"}
    print(json.dumps(rec), flush=True)


def hold(dev, w, seconds, entry):
    """Run one entry point (fa_fwd, or fa_bwd_preprocess + fa_bwd) back to back for `seconds`
    (to sample clocks and board power beside it) and print the mean time per call."""
    fa.load_library()
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
    B, H, S, D = w.shape
    q, k, v, do = (x.to(dev) for x in workload_inputs(w))
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_size(B, H, S, D, code)
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    sh = torch.cuda.current_stream(dev).cuda_stream

    def f():
        if entry == "fwd":
            rc = fa.fa_fwd(q, k, v, o, lse, B, H, S, D, w.scale, 1, code, sh)
        else:
            rc = fa.fa_bwd_preprocess(o, do, delta, B, H, S, D, code, sh) or \
                fa.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, ws, ws_bytes, B, H, S, D, w.scale, 1, code, sh)
        if rc != 0:
            raise RuntimeError(fa.fa_strerror(rc))

    f()
    torch.cuda.synchronize()
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            f()
        torch.cuda.synchronize()
        n += 5
    print(json.dumps({"hold_entry": entry, "calls": n,
                      "ms_per_call": round((time.perf_counter() - t0) * 1e3 / n, 3)}), flush=True)


def sweep(dev):
    """Latency sweep over the grid of the handout's FlashAttention-2 benchmark.

    One head (B=1, H=1) per point, as in that benchmark; times are medians of
    HIP-event times over repeated calls after about 20 ms of warm-up calls.  fwd = fa_fwd_ws (fa_fwd
    with the workspace its size query asks for: it splits the keys of few-tile
    problems); fwd+bwd = that + fa_bwd_preprocess + fa_bwd.
    """
    from exact_attention_causal_amd.inputs import make_inputs
    fa.load_library()
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    rows = []
    print("| dtype | causal | D | S | fwd ms | fwd+bwd ms | fwd TFLOP/s | fwd+bwd TFLOP/s | "
          "split-KV fwd ms (chunks) | step peak MiB | one S×S fp32 matrix MiB |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for dtype in ("bf16", "f32"):
        code = fa.FA_BF16 if dtype == "bf16" else fa.FA_F32
        for causal in (1, 0):
            for D in (16, 32, 64, 128):
                for e in range(7, 17):
                    S = 1 << e
                    q, k, v, do = (x.to(dev) for x in make_inputs(1, 1, S, D, dtype, seed=e))
                    o = torch.empty_like(q)
                    lse = torch.empty((1, 1, S), device=dev, dtype=torch.float32)
                    delta = torch.empty_like(lse)
                    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                    ws_bytes = fa.fa_bwd_workspace_size(1, 1, S, D, code)
                    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
                    fws_bytes = fa.fa_fwd_workspace_size(1, 1, S, D, code)
                    fws = torch.empty(max(fws_bytes, 1), device=dev, dtype=torch.uint8)
                    scale = 1.0 / math.sqrt(D)

                    def fwd():
                        rc = fa.fa_fwd_ws(q, k, v, o, lse, fws, fws_bytes, 1, 1, S, D, scale, causal,
                                          code, sh)
                        assert rc == 0, fa.fa_strerror(rc)

                    def step():
                        fwd()
                        rc = fa.fa_bwd_preprocess(o, do, delta, 1, 1, S, D, code, sh)
                        assert rc == 0, fa.fa_strerror(rc)
                        rc = fa.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, ws, ws_bytes, 1, 1, S, D,
                                       scale, causal, code, sh)
                        assert rc == 0, fa.fa_strerror(rc)

                    def timed(f, n):
                        # warm-up: at least 3 calls and about 20 ms of them, so the
                        # GPU holds its working clock before the timed calls
                        t0, calls = time.perf_counter(), 0
                        while calls < 3 or time.perf_counter() - t0 < 0.02:
                            f()
                            calls += 1
                            if calls % 8 == 0:
                                torch.cuda.synchronize()
                        torch.cuda.synchronize()
                        ts = []
                        for _ in range(n):
                            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                            a.record(stream)
                            f()
                            b.record(stream)
                            ts.append((a, b))
                        torch.cuda.synchronize()
                        return statistics.median(x.elapsed_time(y) for x, y in ts)

                    # split-KV forward: keys cut into chunks so that about eight
                    # workgroups per CU exist, then merged (fa_fwd_partial + fa_merge)
                    n_split = max(1, min(64, (8 * 256) // max(1, (S + 255) // 256), S // 256))
                    op = torch.empty((n_split, 1, 1, S, D), device=dev, dtype=torch.float32)
                    lp = torch.empty((n_split, 1, 1, S), device=dev, dtype=torch.float32)

                    def fwd_split():
                        rc = fa.fa_fwd_partial(q, k, v, op, lp, 1, 1, S, S, D, scale, causal, 0,
                                               n_split, code, sh)
                        assert rc == 0, fa.fa_strerror(rc)
                        rc = fa.fa_merge(op, lp, n_split, o, lse, 1, 1, S, D, code, sh)
                        assert rc == 0, fa.fa_strerror(rc)

                    n = 10 if S >= 16384 else 30
                    t_f, t_s, t_sp = timed(fwd, n), timed(step, n), timed(fwd_split, n)
                    # memory of one fwd+bwd step over the inputs already held: the
                    # outputs, L, D and the backward's workspace (no S x S matrix
                    # exists at any point)
                    del op, lp
                    torch.cuda.synchronize()
                    base = torch.cuda.memory_allocated()
                    torch.cuda.reset_peak_memory_stats()
                    step()
                    torch.cuda.synchronize()
                    peak = (torch.cuda.max_memory_allocated() - base) / 2**20
                    # (this step's buffers were allocated before `base`; report all of them)
                    peak += sum(t.numel() * t.element_size()
                                for t in (o, lse, delta, dq, dk, dv, ws)) / 2**20 + fws_bytes / 2**20
                    sxs = S * S * 4 / 2**20
                    pairs = S * (S + 1) // 2 if causal else S * S
                    tf_f = 4 * D * pairs / (t_f * 1e-3) / 1e12
                    tf_s = 14 * D * pairs / (t_s * 1e-3) / 1e12
                    rows.append(dict(dtype=dtype, causal=causal, D=D, S=S, fwd_ms=t_f, step_ms=t_s,
                                     split_ms=t_sp, n_split=n_split, peak_mib=peak))
                    print(f"| {dtype} | {causal} | {D} | {S} | {t_f:.4f} | {t_s:.4f} | {tf_f:.1f} | "
                          f"{tf_s:.1f} | {t_sp:.4f} ({n_split}) | {peak:.2f} | {sxs:.1f} |", flush=True)
    return rows


# common training shapes: (B, H, S, D)
SHAPES = [(8, 32, 2048, 128), (4, 32, 4096, 128), (2, 32, 8192, 128), (1, 32, 16384, 128),
          (1, 64, 8192, 128), (16, 16, 2048, 64), (8, 16, 4096, 64), (4, 40, 4096, 80),
          (2, 24, 8192, 96), (1, 8, 32768, 128)]


def shapes(dev):
    """Forward and forward+backward throughput (bf16, causal) on common training shapes:
    fwd = fa_fwd_ws (with the workspace its size query asks for), fwd+bwd = that +
    fa_bwd_preprocess + fa_bwd; after about 100 ms of warm-up, the median over 5 batches of
    back-to-back calls (HIP events around each batch)."""
    from exact_attention_causal_amd.inputs import make_inputs
    fa.load_library()
    print("| B | H | S | D | fwd ms | fwd TFLOP/s (% of peak) | fwd+bwd ms | fwd+bwd TFLOP/s (% of peak) |")
    print("|---|---|---|---|---|---|---|---|")
    rows = []
    for B, H, S, D in SHAPES:
        code = fa.FA_BF16
        q, k, v, do = (x.to(dev) for x in make_inputs(B, H, S, D, "bf16", seed=11))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, S), device=dev, dtype=torch.float32)
        delta = torch.empty_like(lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = fa.fa_bwd_workspace_size(B, H, S, D, code)
        ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
        fws_bytes = fa.fa_fwd_workspace_size(B, H, S, D, code)
        fws = torch.empty(max(fws_bytes, 1), device=dev, dtype=torch.uint8)
        scale = 1.0 / math.sqrt(D)

        def fwd():
            rc = fa.fa_fwd_ws(q, k, v, o, lse, fws, fws_bytes, B, H, S, D, scale, 1, code)
            assert rc == 0, fa.fa_strerror(rc)

        def step():
            fwd()
            rc = fa.fa_bwd_preprocess(o, do, delta, B, H, S, D, code)
            rc = rc or fa.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, ws, ws_bytes, B, H, S, D, scale, 1, code)
            assert rc == 0, fa.fa_strerror(rc)

        def timed(f):
            # about 100 ms of warm-up (the clock settles), then the median over 5 batches of
            # back-to-back calls, each batch about 20 ms
            f()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            f()
            torch.cuda.synchronize()
            one = max(time.perf_counter() - t0, 1e-5)
            for _ in range(int(0.1 / one) + 1):
                f()
            n = int(0.02 / one) + 1
            ts = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(n):
                    f()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) / n)
            return statistics.median(ts)

        t_f, t_s = timed(fwd), timed(step)
        pairs = B * H * S * (S + 1) // 2
        tf_f = 4 * D * pairs / (t_f * 1e-3) / 1e12
        tf_s = 14 * D * pairs / (t_s * 1e-3) / 1e12
        rows.append(dict(B=B, H=H, S=S, D=D, fwd_ms=round(t_f, 4), step_ms=round(t_s, 4)))
        print(f"| {B} | {H} | {S} | {D} | {t_f:.3f} | {tf_f:.0f} ({100 * tf_f / PEAK_BF16:.1f} %) | "
              f"{t_s:.3f} | {tf_s:.0f} ({100 * tf_s / PEAK_BF16:.1f} %) |", flush=True)
        del q, k, v, do, o, lse, delta, dq, dk, dv, ws, fws
        torch.cuda.empty_cache()
    print(json.dumps({"shapes": rows}), flush=True)
    return rows


def graph_steps(dev):
    """Step time with the step's five kernels launched call by call (through the
    Python binding, as a Python caller does) against one replay of the same step
    captured as a HIP graph.  Times are per step over back-to-back steps between
    two HIP events (median of 5 repetitions), so launch overhead that the GPU
    cannot hide behind earlier work shows up in the first column.  fa_fwd,
    fa_bwd_preprocess and fa_bwd with a caller-held workspace allocate nothing,
    so the step is capturable as is; every replay matches the eager step bit for
    bit (tests/test_gpu_graph.py)."""
    from exact_attention_causal_amd.inputs import Workload, make_inputs
    fa.load_library()
    shapes = [WORKLOADS[n] for n in ("f32_b1h2_s128_d64", "bf16_b4h12_s512_d64", "bf16_b4h16_s2048_d64_peaky")]
    shapes += [Workload(f"bf16_b1h1_s{S}_d128", "bf16", 1, 1, S, 128, seed=7) for S in (256, 1024, 4096)]
    print("| workload | eager step ms | graph replay ms | speed-up | graph fwd+bwd TFLOP/s |")
    print("|---|---|---|---|---|")
    rows = []
    for w in shapes:
        B, H, S, D = w.shape
        code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
        q, k, v, do = (x.to(dev) for x in make_inputs(B, H, S, D, w.dtype, seed=w.seed, qk_mult=w.qk_mult))
        o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
        lse = torch.empty((B, H, S), device=dev, dtype=torch.float32)
        delta = torch.empty_like(lse)
        ws_bytes = fa.fa_bwd_workspace_size(B, H, S, D, code)
        ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)

        def step():
            rc = fa.fa_fwd(q, k, v, o, lse, B, H, S, D, w.scale, 1, code)
            rc = rc or fa.fa_bwd_preprocess(o, do, delta, B, H, S, D, code)
            rc = rc or fa.fa_bwd(q, k, v, do, lse, delta, dq, dk, dv, ws, ws_bytes, B, H, S, D,
                                 w.scale, 1, code)
            if rc != 0:
                raise RuntimeError(fa.fa_strerror(rc))

        for _ in range(5):
            step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()

        def per_step(f, n=50):
            ts = []
            for _ in range(5):
                f()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(n):
                    f()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) / n)
            return statistics.median(ts)

        t_e, t_g = per_step(step), per_step(g.replay)
        tf = 14 * D * w.causal_pairs() / (t_g * 1e-3) / 1e12
        rows.append({"workload": w.name, "eager_ms": round(t_e, 5), "graph_ms": round(t_g, 5)})
        print(f"| {w.name} | {t_e:.4f} | {t_g:.4f} | {t_e / t_g:.2f}x | {tf:.1f} |", flush=True)
        del g
    print(json.dumps({"graph_steps": rows}), flush=True)
    return rows


def vs_materialised(dev):
    """One forward+backward of this library against attention with the S x S matrix materialised.

    The comparator is the composed attention the pages benchmark first (scores, causal mask,
    softmax and the value product as separate PyTorch ops on the GPU, differentiated by
    autograd), in fp32.  Grid of the pages' attention benchmark: batch 8, one head,
    D in {16, 32, 64, 128}, S in {256, ..., 16384}.  Times are medians of HIP-event times;
    "peak MiB" is what one step allocates beyond its inputs (outputs and gradients included).
    """
    from exact_attention_causal_amd.inputs import make_inputs
    fa.load_library()
    stream = torch.cuda.current_stream(dev)
    B, H = 8, 1

    def measure(f, n=5):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        f()
        torch.cuda.synchronize()
        peak = (torch.cuda.max_memory_allocated() - base) / 2**20
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return statistics.median(x.elapsed_time(y) for x, y in ts), peak

    print("| D | S | materialised fp32 fwd+bwd ms | materialised peak MiB | this library fp32 ms | "
          "fp32 peak MiB | this library bf16 ms | bf16 peak MiB |")
    print("|---|---|---|---|---|---|---|---|")
    for D in (16, 32, 64, 128):
        for S in (256, 1024, 4096, 8192, 16384):
            scale = 1.0 / math.sqrt(D)
            q, k, v, do = (x.to(dev) for x in make_inputs(B, H, S, D, "f32", seed=2000 + S + D))
            mask = torch.ones((S, S), dtype=torch.bool, device=dev).triu(1)

            def composed():
                qg, kg, vg = (x.detach().requires_grad_(True) for x in (q, k, v))
                sc = torch.matmul(qg, kg.transpose(-1, -2)) * scale
                p = torch.softmax(sc.masked_fill(mask, float("-inf")), dim=-1)
                torch.matmul(p, vg).backward(do)
                return qg.grad, kg.grad, vg.grad

            try:
                t_m, m_m = measure(composed)
                mat = f"{t_m:.3f} | {m_m:.1f}"
            except torch.cuda.OutOfMemoryError:
                mat = "OOM | OOM"
            del mask
            torch.cuda.empty_cache()
            cells = []
            for dt in (torch.float32, torch.bfloat16):
                qd, kd, vd, dod = (x.to(dt) for x in (q, k, v, do))

                def flash():
                    o, lse = fa.forward(qd, kd, vd, causal=True, scale=scale)
                    return fa.backward(qd, kd, vd, o, lse, dod, causal=True, scale=scale)

                t_f, m_f = measure(flash)
                cells.append(f"{t_f:.3f} | {m_f:.1f}")
            print(f"| {D} | {S} | {mat} | {cells[0]} | {cells[1]} |", flush=True)
            del q, k, v, do
            torch.cuda.empty_cache()


PUBLISHED_PEAK = {"bf16": 2516.6, "fp32": 157.3}   # dense MFMA TFLOP/s, 2.4 GHz


def peak(dev):
    """Matrix-core throughput with no memory traffic: per dtype and operand kind, the mean
    over 10 launches after 5 warm-up launches (HIP events on the launching stream)."""
    import ctypes
    from exact_attention_causal_amd import build as fab
    if not os.path.exists(fab.PEAK_LIB):
        raise RuntimeError(f"{fab.PEAK_LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(fab.PEAK_LIB)
    lib.fa_peak_mfma.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_peak_mfma.restype = ctypes.c_int
    lib.fa_peak_mfma_flop.argtypes = [ctypes.c_int] * 3
    lib.fa_peak_mfma_flop.restype = ctypes.c_double
    # (launches of 4-19 ms; 16384 bf16 workgroups keep the last round of waves short)
    out = torch.empty(16384 * 256, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    forms = {0: "32x32x2", 1: "32x32x16", 2: "16x16x32"}
    for name, code, blocks, iters in (("bf16", 1, 16384, 1024), ("bf16", 2, 16384, 2048), ("fp32", 0, 4096, 512)):
        for mode, operands in enumerate(("zeros", "constant", "random N(0,1)")):
            launch = lambda: lib.fa_peak_mfma(code, mode, blocks, iters, out.data_ptr(), stream.cuda_stream)
            for _ in range(5):
                assert launch() == 0
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(10):
                assert launch() == 0
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 10
            tf = lib.fa_peak_mfma_flop(code, blocks, iters) / (ms * 1e-3) / 1e12
            print(json.dumps({"peak": f"mfma {name} {forms[code]}",
                              "operands": operands, "blocks": blocks, "iters": iters, "ms": round(ms, 4),
                              "tflops": round(tf, 1),
                              "published": PUBLISHED_PEAK[name], "frac": round(tf / PUBLISHED_PEAK[name], 4)}),
                  flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no communication, so one GPU is measured)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return
    if args.sweep:
        sweep(dev)
        return
    if args.vs_materialised:
        vs_materialised(dev)
        return
    if args.graph:
        graph_steps(dev)
        return
    if args.peak:
        peak(dev)
        return
    if args.shapes:
        shapes(dev)
        return
    if args.hold > 0:
        hold(dev, WORKLOADS[args.workload], args.hold, args.hold_entry)
        return
    if args.split_kv:
        split_kv(dev, WORKLOADS[args.workload], args.split_kv, args.steps, args.warmup,
                 not args.no_cpu_baseline)
        return
    fa.load_library()
    w = WORKLOADS[args.workload]
    rec, cpu_in, outs = time_workload(dev, w, args.steps, args.warmup, headline=True)
    extra = [n for n in EXTRA_WORKLOADS if n != w.name] if not args.no_extra else []
    side = {}
    for name in extra:
        wx = WORKLOADS[name]
        r, cin, o = time_workload(dev, wx, args.steps, args.warmup, headline=False)
        side[name] = (wx, r, cin, o)
    if not args.no_check:
        log(f"sampled oracle check of {w.name}")
        rec["check"] = sampled_errors(w, cpu_in, outs)
    for name, (wx, r, cin, o) in side.items():
        if not args.no_check:
            log(f"sampled oracle check of {name}")
            r["check"] = sampled_errors(wx, cin, o)
        rec.setdefault("workloads", {})[name] = r
    del outs, side
    if not args.no_cpu_baseline:
        log("cpu oracle baseline")
        rec["cpu_baseline"] = cpu_baseline(w, *cpu_in, args.cpu_tokens)
    print(json.dumps(rec), flush=True)


def time_workload(dev, w, steps, warmup, headline):
    """Warm up, then time `steps` whole steps (fa_fwd + fa_bwd_preprocess + fa_bwd) of one
    workload on one stream.  Returns (record, CPU inputs, outputs of the last step)."""
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
    B, H, S, D = w.shape

    log(f"generating inputs for {w.name}")
    q, k, v, do = workload_inputs(w)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, S), device=dev, dtype=torch.float32)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws_bytes = fa.fa_bwd_workspace_size(B, H, S, D, code)
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {fa.fa_strerror(rc)}")

    def fwd():
        check(fa.fa_fwd(qd, kd, vd, o, lse, B, H, S, D, w.scale, 1, code, sh), "fa_fwd")

    def pre():
        check(fa.fa_bwd_preprocess(o, dod, delta, B, H, S, D, code, sh), "fa_bwd_preprocess")

    def bwd():
        check(fa.fa_bwd(qd, kd, vd, dod, lse, delta, dq, dk, dv, ws, ws_bytes, B, H, S, D,
                        w.scale, 1, code, sh), "fa_bwd")

    log(f"warmup {w.name}")
    for _ in range(warmup):
        fwd(); pre(); bwd()
    torch.cuda.synchronize()
    log(f"timing {steps} steps of {w.name}")

    # timed region: K whole steps, with per-entry-point events on the same stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        pre()
        ev[i][2].record(stream)
        bwd()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_fwd = [e[0].elapsed_time(e[1]) for e in ev]
    per_pre = [e[1].elapsed_time(e[2]) for e in ev]
    per_bwd = [e[2].elapsed_time(e[3]) for e in ev]
    per_step = [e[0].elapsed_time(e[3]) for e in ev]
    t_fwd = sum(per_fwd) / steps
    t_pre = sum(per_pre) / steps
    t_bwd = sum(per_bwd) / steps
    ms_step = wall * 1e3 / steps

    pairs = w.causal_pairs()
    f_fwd = 4 * D * pairs
    f_all = 14 * D * pairs
    peak = PEAK_BF16 if w.dtype == "bf16" else PEAK_F32
    value = f_all / (ms_step * 1e-3) / 1e12
    fwd_tf = f_fwd / (t_fwd * 1e-3) / 1e12
    bwd_tf = 10 * D * pairs / (t_bwd * 1e-3) / 1e12
    esize = 2 if w.dtype == "bf16" else 4
    tensor = B * H * S * D * esize
    _, plan = fa.fa_get_plan(B, H, S, D, code, 0)
    config = {"workload": w.name, "B": B, "H": H, "S": S, "D": D, "causal": True,
              "scale": w.scale, "seed": w.seed, "qk_mult": w.qk_mult, "plan": plan.as_dict()}
    timing = {
        "ms_per_step": round(ms_step, 4),
        "fwd_bwd_tflops": round(value, 2),
        "frac_of_peak": round(value / peak, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_frac_of_peak": round(fwd_tf / peak, 4),
        "ms": {"fwd": round(t_fwd, 4), "bwd_preprocess": round(t_pre, 4), "bwd": round(t_bwd, 4)},
        "ms_event_stats": {n: {"median": round(statistics.median(x), 4), "min": round(min(x), 4),
                               "max": round(max(x), 4)}
                           for n, x in (("step", per_step), ("fwd", per_fwd), ("bwd", per_bwd))},
        "roofline": {"kernel": "fwd_kernel (fa_fwd)", "bound": "mfma", "achieved": round(fwd_tf, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(fwd_tf / peak, 4),
                     "traffic": (FWD_TRAFFIC["bytes"].get(w.name)
                                 if FWD_TRAFFIC["sources_sha1"] == fwd_sources_sha1() else None),
                     "algorithmic_per_launch": {"flop": f_fwd, "bytes": 4 * tensor + 4 * B * H * S}},
        "roofline_bwd": {"kernel": "dK/dV + dQ kernels (fa_bwd)", "bound": "mfma",
                         "achieved": round(bwd_tf, 2), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(bwd_tf / peak, 4)},
    }
    if headline:
        rec = {
            "metric": METRIC,
            "value": round(value, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": w.dtype,
            "data": "synthetic (seeded i.i.d. N(0,1) Q, K, V, dO)",
            "config": config,
        }
        timing.pop("ms_per_step")
        timing.pop("fwd_bwd_tflops")
        rec.update(timing)
    else:
        rec = {"config": config, "steps": steps, "warmup": warmup, **timing}
    log(f"{w.name}: {ms_step:.3f} ms/step, {value:.1f} TFLOP/s fwd+bwd, {fwd_tf:.1f} TFLOP/s fwd")
    outs = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    return rec, (q, k, v, do), outs


if __name__ == "__main__":
    main()
