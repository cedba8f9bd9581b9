#!/usr/bin/env python3
"""Throughput of matmul against GGUF block-quantized weights on one MI355X.

One step is the decode GEMV workload: y = x . W^T for Q4_K and Q6_K weights
of N=14336 rows by K=4096, each at M=1 and at M=8 tokens, f32 activations,
f32 outputs -- four GEMV launches through the C ABI.  The reported value is
the quantized-weight bytes those launches read per second (each weight byte
counted once per launch), over exactly --steps steps after --warmup steps.

By default the weights are held in the load-time repacked layout
(qmm_repack, run once before timing: the same bytes, permuted into 16-row
records in the order the GEMV lanes load them) and the step calls
qmm_gemv_packed; --layout native times qmm_gemv_ex on the GGUF rows as
stored.  The step in the other layout is reported among the secondary lines.

Weights are resident in HBM before timing starts.  To measure HBM rather
than the 256 MiB Infinity Cache, every launch reads a different copy of its
weight set; a copy is read again only after more than 1 GiB of other weights
has been streamed.  Steps are replayed from captured HIP graphs so host
launch overhead does not enter the timing.

Also printed in the same JSON line:
  roofline      the dominant kernel's algorithmic bytes per launch over its
                average launch duration (HIP events on its stream), against
                the 8 TB/s HBM peak, with measured HBM traffic when a
                counter summary for the current kernel sources exists, and
                the practical ceiling: a plain streaming-read kernel
                (libqmm_probe.so) timed over the same bytes with the same
                copy rotation (ceiling_GBps, frac_of_ceiling);
  roofline_gemm the same for the prefill GEMM half of the metric: the slower
                of the two 512 x 4096 x 4096 GEMMs (Q8_0, Q5_0) in the step's
                weight layout (repacked records by default), TFLOP/s against
                the 2.5 PFLOP/s dense f16 matrix-core peak, with both layouts
                of both kinds under "all";
  cpu_baseline  the oracle (binary64 CPU reference) timed on the host cores
                on full steps of the same workload, and on one core over a
                sample of rows (single_core);
  cases         each of the four GEMVs alone (best and median of 5 rounds);
  secondary     the decode step's GEMVs in the other weight layout, and the
                other workloads (Q4_0 GEMV, prefill GEMMs, codebook kinds,
                in both layouts where they are GEMVs, the Q4_0 and MXFP4
                GEMVs with int8 activations, routed experts, the scaled
                MXFP4 GEMM, the routed expert FFN), each timed the same way.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense FP8 (and FP8 x FP4) matrix-core peak
MALL_DEFEAT_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")


def source_digest() -> str:
    """Hash of the HIP sources, to tell whether a stored counter summary
    still describes the kernels being timed."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gguf_block_quantized_kind_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not os.path.isfile(os.path.join(csrc, name)):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class Case:
    """One matmul (GEMV, GEMM or routed experts) on rotating weight copies."""

    def __init__(self, name, kind, launch, copies, weight_bytes, flops):
        self.name, self.kind, self.launch = name, kind, launch
        self.copies, self.weight_bytes, self.flops = copies, weight_bytes, flops


def make_copies(torch, W: np.ndarray, min_copies: int = 2):
    base = torch.from_numpy(W).cuda()
    n = max(min_copies, math.ceil(MALL_DEFEAT_BYTES / base.numel()) + 1)
    return [base] + [base.clone() for _ in range(n - 1)]


def capture(torch, fn, count: int):
    """A HIP graph of `count` consecutive calls fn(i)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    return g


ROUNDS = 5


def time_graph(torch, fn, launches: int) -> tuple[float, float]:
    """(best, median) over ROUNDS replays of the average duration of one of
    `launches` back-to-back calls fn(i) captured in one graph, from HIP
    events on the stream the graph replays on (seconds)."""
    g = capture(torch, fn, launches)
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(ROUNDS):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        end.synchronize()
        per.append(start.elapsed_time(end) / 1e3 / launches)
    del g
    per.sort()
    return per[0], per[len(per) // 2]


def time_launches(torch, case: Case, launches: int) -> tuple[float, float]:
    return time_graph(torch, lambda i: case.launch(i), launches)


def stream_ceiling(torch, nbytes: int) -> dict:
    """The practical HBM read ceiling for nbytes per launch: the streaming
    probe over rotating copies (a copy is read again only after more than
    1 GiB of others), best over a few grid sizes."""
    import ctypes

    from gguf_block_quantized_kind_amd import _build

    if not os.path.exists(_build.PROBE_LIBRARY):
        raise RuntimeError(f"{_build.PROBE_LIBRARY} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(_build.PROBE_LIBRARY)
    lib.qmm_probe_stream_read.restype = ctypes.c_int
    lib.qmm_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                                          ctypes.c_void_p, ctypes.c_void_p]
    nbytes = nbytes // 16 * 16
    n = math.ceil(MALL_DEFEAT_BYTES / nbytes) + 1
    copies = [torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda") for _ in range(n)]
    best = None
    for grid in (1024, 2048, 4096, 8192):
        out = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")

        def launch(i, grid=grid, out=out):
            st = lib.qmm_probe_stream_read(copies[i % n].data_ptr(), nbytes, grid, 0x5EED1234, out.data_ptr(),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError(f"stream probe failed: {st}")

        launch(0)
        torch.cuda.synchronize()
        b, med = time_graph(torch, launch, 32)
        if best is None or b < best[0]:
            best = (b, med, grid)
    del copies
    torch.cuda.empty_cache()
    return {"GBps": round(nbytes / best[0] / 1e9, 1), "GBps_median": round(nbytes / best[1] / 1e9, 1),
            "bytes_per_launch": nbytes, "grid": best[2]}


def packed_copies(torch, qmm, w, min_copies: int = 2):
    """Rotating copies of w's weights in the load-time repacked layout: the
    repack runs once, here, before anything is timed."""
    base = qmm.repack(w.kind, torch.from_numpy(w.weights()).cuda(), w.N, w.K)
    torch.cuda.synchronize()
    n = max(min_copies, math.ceil(MALL_DEFEAT_BYTES / base.numel()) + 1)
    return [base] + [base.clone() for _ in range(n - 1)]


def gemv_cases(torch, qmm, wl, layout: str = "packed"):
    """The decode step: Q4_K and Q6_K at M = 1 and 8, their weights in the
    repacked layout (qmm_gemv_packed) or as native GGUF rows (qmm_gemv_ex)."""
    cases = []
    for kind in ("Q4_K", "Q6_K"):
        w1 = next(w for w in wl.C2 if w.kind == kind and w.M == 1)
        copies = packed_copies(torch, qmm, w1) if layout == "packed" else make_copies(torch, w1.weights())
        for M in (1, 8):
            w = next(w for w in wl.C2 if w.kind == kind and w.M == M)
            x = torch.from_numpy(w.x()).cuda()
            y = torch.empty((M, w.N), dtype=torch.float32, device="cuda")
            # M=1 reads even copies, M=8 odd ones, so one step never re-reads a copy.
            par = 0 if M == 1 else 1

            def launch(i, kind=kind, x=x, y=y, M=M, w=w, copies=copies, par=par):
                c = copies[(2 * i + par) % len(copies)]
                if layout == "packed":
                    qmm.qmm_gemv_packed(kind, c, x, y, M, w.N, w.K)
                else:
                    qmm.qmm_gemv_ex(kind, c, x, y, M, w.N, w.K)

            name = w.name + ("_packed" if layout == "packed" else "")
            cases.append(Case(name, kind, launch, copies, w.weight_bytes, w.flops))
    return cases


def gemm_cases(torch, qmm, wl):
    """(case, layout) for the 512 x 4096 x 4096 prefill GEMMs, Q8_0 and Q5_0,
    on native GGUF rows (qmm_matmul) and on repacked records
    (qmm_matmul_packed).  Weight copies are made as each case is built."""
    for w in wl.C3:
        for lay in ("native", "packed"):
            copies = packed_copies(torch, qmm, w) if lay == "packed" else make_copies(torch, w.weights())
            x = torch.from_numpy(w.x()).cuda()
            y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

            def launch(i, w=w, x=x, y=y, copies=copies, lay=lay):
                if lay == "packed":
                    qmm.qmm_matmul_packed(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K)
                else:
                    qmm.qmm_matmul(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K)

            yield Case(w.name + ("_packed" if lay == "packed" else ""), w.kind, launch, copies, w.weight_bytes,
                       w.flops), lay


def secondary_cases(torch, qmm, wl, layout: str = "packed"):
    cases = []
    # The decode step in the other weight layout.
    cases += gemv_cases(torch, qmm, wl, "native" if layout == "packed" else "packed")
    # The other decode workloads over repacked weights (their native-layout
    # lines follow below).
    for w in [w for w in wl.C1 + wl.C4 if w.M <= 8]:
        copies = packed_copies(torch, qmm, w)
        x = torch.from_numpy(w.x()).cuda()
        y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

        def launch(i, w=w, x=x, y=y, copies=copies):
            qmm.qmm_gemv_packed(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K)

        cases.append(Case(w.name + "_packed", w.kind, launch, copies, w.weight_bytes, w.flops))
    # The Q4_0 and MXFP4 decode workloads on the int8-activation path (its
    # own tolerance; the call quantizes x, then multiplies on the int8
    # matrix cores, over repacked weights), at one token and at eight.
    eight = [wl.Matmul(w.name.replace("_m1", "_m8"), w.kind, 8, w.N, w.K, w.x_dtype)
             for w in wl.C1 + [w for w in wl.C4 if w.kind == "MXFP4" and w.M == 1]]
    for w in eight:
        copies = packed_copies(torch, qmm, w)
        x = torch.from_numpy(w.x()).cuda()
        y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

        def launch(i, w=w, x=x, y=y, copies=copies):
            qmm.qmm_gemv_packed(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K)

        cases.append(Case(w.name + "_packed", w.kind, launch, copies, w.weight_bytes, w.flops))
    for w in wl.C1 + [w for w in wl.C4 if w.kind == "MXFP4" and w.M == 1] + eight:
        copies = packed_copies(torch, qmm, w)
        x = torch.from_numpy(w.x()).cuda()
        y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        ws = torch.empty(qmm.qmm_gemv_i8_workspace_bytes(w.M, w.K), dtype=torch.uint8, device="cuda")

        def launch(i, w=w, x=x, y=y, ws=ws, copies=copies):
            qmm.qmm_gemv_i8(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K, ws)

        cases.append(Case(w.name + "_i8", w.kind, launch, copies, w.weight_bytes, w.flops))
    for w in wl.C1 + wl.C4:
        copies = make_copies(torch, w.weights())
        x = torch.from_numpy(w.x()).cuda()
        y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

        def launch(i, w=w, x=x, y=y, copies=copies):
            qmm.qmm_matmul(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K)

        cases.append(Case(w.name, w.kind, launch, copies, w.weight_bytes, w.flops))
    # The other super-block kinds at the decode step's shape (N=14336,
    # K=4096, f32 x, M = 1 and 8; weights drawn as the step's): repacked,
    # then native rows.
    for kind in ("Q2_K", "Q3_K", "Q5_K"):
        for M in (1, 8):
            w = wl.Matmul(f"c2_{kind.lower()}_m{M}", kind, M, 14336, 4096, "f32")
            x = torch.from_numpy(w.x()).cuda()
            y = torch.empty((M, w.N), dtype=torch.float32, device="cuda")
            for layout in ("packed", "native"):
                copies = packed_copies(torch, qmm, w) if layout == "packed" else make_copies(torch, w.weights())

                def launch(i, w=w, x=x, y=y, copies=copies, layout=layout):
                    c = copies[i % len(copies)]
                    if layout == "packed":
                        qmm.qmm_gemv_packed(w.kind, c, x, y, w.M, w.N, w.K)
                    else:
                        qmm.qmm_gemv_ex(w.kind, c, x, y, w.M, w.N, w.K)

                cases.append(Case(w.name + ("_packed" if layout == "packed" else ""), w.kind, launch, copies,
                                  w.weight_bytes, w.flops))
    # The codebook prefill workloads over repacked records.
    for w in [w for w in wl.C4 if w.M > 8 and w.kind in ("IQ4_NL", "IQ4_XS", "MXFP4")]:
        copies = packed_copies(torch, qmm, w)
        x = torch.from_numpy(w.x()).cuda()
        y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")

        def launch(i, w=w, x=x, y=y, copies=copies):
            qmm.qmm_matmul_packed(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K)

        cases.append(Case(w.name + "_packed", w.kind, launch, copies, w.weight_bytes, w.flops))
    # The MXFP4 prefill workload again on the scaled FP8 x FP4 matrix cores
    # (its own, looser tolerance; activations quantized to MX FP8 in the call).
    for w in [w for w in wl.C4 if w.kind == "MXFP4" and w.M > 8]:
        copies = make_copies(torch, w.weights())
        x = torch.from_numpy(w.x()).cuda()
        y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        ws = torch.empty(qmm.qmm_gemm_mx_workspace_bytes(w.M, w.K), dtype=torch.uint8, device="cuda")

        def launch(i, w=w, x=x, y=y, ws=ws, copies=copies):
            qmm.qmm_gemm_mx(w.kind, copies[i % len(copies)], x, y, w.M, w.N, w.K, ws)

        cases.append(Case(w.name + "_mx", w.kind, launch, copies, w.weight_bytes, w.flops))
    for e in wl.C5:
        ids_np = e.ids()
        ids = torch.from_numpy(ids_np).cuda()
        touched = e.touched_bytes(ids_np)
        for mat, N, K, X, per_slot in (("gate_up", e.N_gu, e.K_gu, e.x(), 0),
                                       ("down", e.N_d, e.K_d, e.h(), 1)):
            W = e.w_gu() if mat == "gate_up" else e.w_d()
            copies = make_copies(torch, W)
            Xd = torch.from_numpy(X).cuda()
            Y = torch.empty((e.M, e.topk, N), dtype=torch.float32, device="cuda")
            ws = torch.empty((qmm.qmm_moe_workspace_bytes(e.E, e.M, e.topk) + 3) // 4,
                             dtype=torch.int32, device="cuda")
            row_b = wl.row_bytes(e.kind, K)
            distinct = np.unique(ids_np).size

            def launch(i, e=e, N=N, K=K, Xd=Xd, Y=Y, ws=ws, per_slot=per_slot, copies=copies, ids=ids):
                qmm.qmm_moe(e.kind, copies[i % len(copies)], e.E, ids, e.topk, Xd, per_slot, Y,
                            e.M, N, K, ws)

            cases.append(Case(f"{e.name}_{mat}", e.kind, launch, copies, distinct * N * row_b,
                              2 * e.M * e.topk * N * K))
            # The same products over the experts repacked once at load.
            base = qmm.repack_experts(e.kind, copies[0], e.E, N, K)
            torch.cuda.synchronize()
            pcopies = [base] + [base.clone() for _ in range(len(copies) - 1)]

            def launch_p(i, e=e, N=N, K=K, Xd=Xd, Y=Y, ws=ws, per_slot=per_slot, pcopies=pcopies, ids=ids):
                qmm.qmm_moe_packed(e.kind, pcopies[i % len(pcopies)], e.E, ids, e.topk, Xd, per_slot, Y,
                                   e.M, N, K, ws)

            cases.append(Case(f"{e.name}_{mat}_packed", e.kind, launch_p, pcopies, distinct * N * row_b,
                              2 * e.M * e.topk * N * K))
        del touched
    # The whole routed expert FFN (gate/up, SiLU-product, down, weighted
    # combine) on the same experts and routing; bytes are the touched
    # experts' gate/up and down weights, each read once.
    for e in wl.C5:
        ids_np = e.ids()
        ids = torch.from_numpy(ids_np).cuda()
        gu = make_copies(torch, e.w_gu())
        dn = make_copies(torch, e.w_d())
        n = min(len(gu), len(dn))
        g = wl.rng(e.name, "ffn")
        w = g.uniform(0.05, 1.0, size=(e.M, e.topk))
        w = torch.from_numpy((w / w.sum(axis=1, keepdims=True)).astype(np.float32)).cuda()
        Xd = torch.from_numpy(e.x()).cuda()
        N_ff = e.N_gu // 2
        Y = torch.empty((e.M, e.K_gu), dtype=torch.float32, device="cuda")
        ws = torch.empty(qmm.qmm_moe_ffn_workspace_bytes(e.E, e.M, e.topk, N_ff, e.K_gu), dtype=torch.uint8,
                         device="cuda")

        def launch(i, e=e, ids=ids, w=w, Xd=Xd, Y=Y, ws=ws, gu=gu, dn=dn, n=n, N_ff=N_ff):
            qmm.qmm_moe_ffn(e.kind, gu[i % n], dn[i % n], e.E, ids, w, e.topk, Xd, Y, e.M, N_ff, e.K_gu, ws)

        cases.append(Case(f"{e.name}_ffn", e.kind, launch, gu + dn, e.touched_bytes(ids_np),
                          2 * e.M * e.topk * (e.N_gu * e.K_gu + e.N_d * e.K_d)))
        # The same FFN over the experts repacked once at load.
        pgu0 = qmm.repack_experts(e.kind, gu[0], e.E, e.N_gu, e.K_gu)
        pdn0 = qmm.repack_experts(e.kind, dn[0], e.E, e.N_d, e.K_d)
        torch.cuda.synchronize()
        pgu = [pgu0] + [pgu0.clone() for _ in range(n - 1)]
        pdn = [pdn0] + [pdn0.clone() for _ in range(n - 1)]

        def launch_p(i, e=e, ids=ids, w=w, Xd=Xd, Y=Y, ws=ws, pgu=pgu, pdn=pdn, n=n, N_ff=N_ff):
            qmm.qmm_moe_ffn_packed(e.kind, pgu[i % n], pdn[i % n], e.E, ids, w, e.topk, Xd, Y, e.M, N_ff,
                                   e.K_gu, ws)

        cases.append(Case(f"{e.name}_ffn_packed", e.kind, launch_p, pgu + pdn, e.touched_bytes(ids_np),
                          2 * e.M * e.topk * (e.N_gu * e.K_gu + e.N_d * e.K_d)))
    return cases


def describe(case: Case, timing: tuple[float, float]) -> dict:
    seconds, median = timing
    gbs = case.weight_bytes / seconds / 1e9
    tflops = case.flops / seconds / 1e12
    out = {"us_per_launch": round(seconds * 1e6, 3), "us_median": round(median * 1e6, 3),
           "weight_bytes": case.weight_bytes,
           "weight_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "TFLOPs": round(tflops, 2)}
    if case.name.endswith("_mx"):
        out["mfma_fp8_frac"] = round(tflops / FP8_MFMA_PEAK_TFLOPS, 4)
    elif "_m512" in case.name or "_m256" in case.name:
        out["mfma_f16_frac"] = round(tflops / F16_MFMA_PEAK_TFLOPS, 4)
    return out


def measured_traffic(kernel_case: str):
    """HBM bytes per launch from a stored rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_digest") != source_digest():
        return None
    entry = data.get("cases", {}).get(kernel_case)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def _pmc_average(directory: str, counter: str, kernel_substr: str) -> tuple[float, int]:
    """Average per-dispatch value of `counter` over the dispatches of kernels
    whose name contains kernel_substr, from rocprofv3's counter_collection
    CSV files under `directory`."""
    import csv
    import glob

    vals = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter and kernel_substr in row["Kernel_Name"]:
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples for '{kernel_substr}' under {directory}")
    return sum(vals) / len(vals), len(vals)


def write_traffic(case, case_fetch, case_write, copy_fetch, copy_write, copy_bytes):
    """HBM bytes per launch of one decode GEMV case from FETCH_SIZE /
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a plain device copy of copy_bytes (it reads and writes copy_bytes)."""
    cf, _ = _pmc_average(copy_fetch, "FETCH_SIZE", "copyBuffer")
    cw, _ = _pmc_average(copy_write, "WRITE_SIZE", "copyBuffer")
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    out = {"source_digest": source_digest(), "copy_bytes": copy_bytes,
           "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": fetch_scale, "write_scale": write_scale, "cases": {}}
    # The decode GEMV kernels (gemv_t1_kernel, gemv_xs_kernel, gemv_mfma_kernel).
    f, nf = _pmc_average(case_fetch, "FETCH_SIZE", "qmm::gv::gemv_")
    w, nw = _pmc_average(case_write, "WRITE_SIZE", "qmm::gv::gemv_")
    out["cases"][case] = {"fetch_kib": f, "write_kib": w, "dispatches": [nf, nw],
                          "hbm_bytes_per_launch": round(f * 1024.0 * fetch_scale + w * 1024.0 * write_scale)}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, "traffic.json")
    old = {}
    if os.path.exists(path):
        with open(path) as fh:
            old = json.load(fh)
    if old.get("source_digest") == out["source_digest"]:
        old["cases"].update(out["cases"])
        out["cases"] = old["cases"]
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def cpu_baseline(wl, target_seconds: float) -> dict:
    """The oracle on full steps with all host threads, then on one thread
    over the first rows of each weight set (weight bytes of the rows it
    decodes per second)."""
    import oracle

    orc = oracle.default()
    data = []
    for w in wl.C2:
        data.append((w, w.weights(), w.x()))
    total_bytes, steps = 0, 0
    t0 = time.perf_counter()
    while True:
        for w, W, X in data:
            orc.matmul(w.kind, W, w.K, X)
            total_bytes += w.weight_bytes
        steps += 1
        if time.perf_counter() - t0 >= target_seconds:
            break
    dt = time.perf_counter() - t0
    rows = np.arange(1024)
    one_bytes, one_steps = 0, 0
    t1 = time.perf_counter()
    while True:
        for w, W, X in data:
            orc.matmul(w.kind, W, w.K, X, rows=rows, threads=1)
            one_bytes += w.weight_bytes * len(rows) // w.N
        one_steps += 1
        if time.perf_counter() - t1 >= target_seconds / 2:
            break
    dt1 = time.perf_counter() - t1
    return {"value": round(total_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": orc.max_threads(),
            "kind": "oracle",
            "sample": (f"{steps} full step(s): Q4_K and Q6_K, M=1 and M=8, N=14336, K=4096, "
                       f"binary64 decode + matmul + bound, no cache rotation, {dt:.1f} s"),
            "single_core": {"value": round(one_bytes / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "sample": (f"{one_steps} pass(es) over rows 0..1023 of each of the step's four "
                                       f"GEMVs, {dt1:.1f} s")}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--layout", choices=("packed", "native"), default="packed",
                    help="weight layout of the timed decode step: repacked once at load (default) or "
                         "native GGUF rows")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle timing budget (0: skip)")
    ap.add_argument("--profile-case", metavar="NAME",
                    help="counter-collection mode: launch only this case (a decode GEMV, prefill GEMM or "
                         "secondary workload), eagerly, --steps times")
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="counter-calibration mode: --steps device copies of MIB MiB each")
    ap.add_argument("--write-traffic", nargs=5, metavar=("CASE", "CASE_FETCH", "CASE_WRITE", "COPY_FETCH",
                                                          "COPY_WRITE"),
                    help="turn four rocprofv3 --pmc output directories (FETCH_SIZE and WRITE_SIZE of a "
                         "--profile-case CASE run and of --copy-probe runs) into an entry of "
                         "profiles/traffic.json")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of the --copy-probe copies (for --write-traffic)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, copy_bytes=args.copy_mib << 20)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    import torch

    import gguf_block_quantized_kind_amd as qmm
    import workloads as wl

    torch.cuda.set_device(0)
    qmm.load_library()
    props = torch.cuda.get_device_properties(0)

    if args.copy_probe:
        src = torch.ones(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel(), "copies": args.steps}))
        return

    cases = gemv_cases(torch, qmm, wl, args.layout)
    if args.profile_case:
        case = next((c for c in cases if c.name == args.profile_case), None)
        if case is None:  # a prefill GEMM or a secondary workload
            cases.clear()
            torch.cuda.empty_cache()
            case = next((c for c, _ in gemm_cases(torch, qmm, wl) if c.name == args.profile_case), None)
        if case is None:
            case = next((c for c in secondary_cases(torch, qmm, wl, args.layout) if c.name == args.profile_case),
                        None)
        if case is None:
            sys.exit(f"no case named {args.profile_case}")
        for i in range(args.steps):
            case.launch(i)
        torch.cuda.synchronize()
        print(json.dumps({"profile_case": case.name, "launches": args.steps}))
        return
    for c in cases:  # eager once: loads the code objects before capture
        c.launch(0)
    torch.cuda.synchronize()

    def step(t):
        for c in cases:
            c.launch(t)

    per_graph = 8  # copies are >= 2 * 8 deep, so no copy repeats inside a graph
    main_graph = capture(torch, step, per_graph)

    def run(n):
        for _ in range(n // per_graph):
            main_graph.replay()
        rem = n % per_graph
        if rem:
            g = capture(torch, step, rem)
            g.replay()
            torch.cuda.synchronize()
            del g

    run(args.warmup)
    torch.cuda.synchronize()
    rem_graph = capture(torch, step, args.steps % per_graph) if args.steps % per_graph else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps // per_graph):
        main_graph.replay()
    if rem_graph is not None:
        rem_graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    bytes_per_step = sum(c.weight_bytes for c in cases)
    value = bytes_per_step * args.steps / elapsed / 1e9

    per_case = {c.name: describe(c, time_launches(torch, c, 64)) for c in cases}
    dominant = max(cases, key=lambda c: per_case[c.name]["us_per_launch"])
    dom = per_case[dominant.name]
    achieved = dominant.weight_bytes / (dom["us_per_launch"] * 1e-6) / 1e9
    del main_graph, rem_graph
    for c in cases:
        c.copies.clear()
    torch.cuda.empty_cache()
    ceiling = stream_ceiling(torch, dominant.weight_bytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dominant.name),
                "kernel": f"qmm GEMV {dominant.name}", "algorithmic_bytes_per_launch": dominant.weight_bytes,
                "us_median": dom["us_median"],
                "ceiling_GBps": ceiling["GBps"], "frac_of_ceiling": round(achieved / ceiling["GBps"], 4),
                "ceiling": ceiling}

    # The prefill GEMM half of the metric: 512 x 4096 x 4096, Q8_0 and Q5_0,
    # on native GGUF rows (qmm_matmul) and on the load-time repacked records
    # (qmm_matmul_packed, the layout the decode step reads).  The roofline
    # block reports the slower kind in the step's layout.
    gemm = {}
    for c, lay in gemm_cases(torch, qmm, wl):
        c.launch(0)
        torch.cuda.synchronize()
        gemm[c.name] = (c, describe(c, time_launches(torch, c, 32)), lay)
        c.copies.clear()
        torch.cuda.empty_cache()
    in_layout = {k: v for k, v in gemm.items() if v[2] == ("packed" if args.layout == "packed" else "native")}
    gname = max(in_layout, key=lambda k: in_layout[k][1]["us_per_launch"])
    gcase, gd, _ = gemm[gname]
    gach = gcase.flops / (gd["us_per_launch"] * 1e-6) / 1e12
    roofline_gemm = {"bound": "mfma", "achieved": round(gach, 2), "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gach / F16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": f"qmm GEMM {gname}", "algorithmic_flops_per_launch": gcase.flops,
                     "us_per_launch": gd["us_per_launch"], "us_median": gd["us_median"],
                     "all": {k: v[1] for k, v in gemm.items()}}
    secondary = {}
    if not args.no_secondary:
        sec = secondary_cases(torch, qmm, wl, args.layout)
        # Cases of one weight set share its copies: free them after the last.
        last = {id(c.copies): i for i, c in enumerate(sec)}
        for i, c in enumerate(sec):
            c.launch(0)
            torch.cuda.synchronize()
            secondary[c.name] = describe(c, time_launches(torch, c, 32))
            if last[id(c.copies)] == i:
                c.copies.clear()
                torch.cuda.empty_cache()

    cpu = cpu_baseline(wl, args.cpu_seconds) if args.cpu_seconds > 0 else None

    line = {
        "metric": "quantized GEMV weight GB/s (% of HBM peak); prefill GEMM TFLOP/s (% MFMA peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 x f16 matrix cores, f32 accumulate (f32 x rounded once to f16; weight codes times "
                 "sub-block scales as exact f16 integers; super-block scales and mins applied in f32)",
        "data": "synthetic",
        "config": {"workload": "decode GEMV, Q4_K and Q6_K weights, M=1 and M=8, N=14336, K=4096, "
                               "f32 activations, one launch per (kind, M) per step",
                   "weight_layout": ("load-time repacked (same bytes, permuted; repacked once before "
                                     "timing)" if args.layout == "packed" else "native GGUF rows"),
                   "weight_bytes_per_step": bytes_per_step, "hbm_frac": round(value / HBM_PEAK_GBS, 4),
                   "device": props.name, "cus": props.multi_processor_count},
        "roofline": roofline,
        "roofline_gemm": roofline_gemm,
        "cpu_baseline": cpu,
        "cases": per_case,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
