#!/usr/bin/env python3
"""Throughput of one GPU's share of the expert-parallel MoE FFN on MI355X.

One step = the whole hot path on one batch: moe_plan (route scan), then
moe_forward (grouped SwiGLU GEMM up gathering the received rows through the
route table; for bf16, GEMM down writing the rows of received rows with one
local slot straight to the output and the weighted top-k reduce of the others,
or the whole reduce inside GEMM down for a decode batch; for fp32, GEMM down
and the reduce), captured once in a HIP graph and replayed, on synthetic
inputs already resident in HBM. The same kernels also run stage by stage
through their entry points, with events between the stages, for the
per-stage figures. Default workload: the prefill shape (16384 received
tokens, H=7168, I=2048, 32 local experts of 256, top-8, Zipf s=1.0
popularity), bf16.

Prints ONE JSON line: tokens/s over the timed steps, the roofline of the
dominant kernels (the forward's GEMM launches, HIP events around moe_forward
on the stream the kernels run on), per-stage rates, the low-batch combine
latencies, a sampled parity check and the CPU oracle's rate on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config c5] [--gpus 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 GPU; grouped-GEMM % MFMA peak; expand/reduce % HBM BW"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

WORKLOAD_NAMES = {
    "c1": "tiny fp32: T=64, H=256, I=128, 8 experts, top-2",
    "c2": "EP16 rank share: T=4096, H=7168, I=2048, 16 local of 256 experts, top-8 uniform",
    "c3": "low-batch decode: H=3584, I=2048, 28 local of 896 experts, top-16 stride, 1 real row in 8",
    "c4": "DP-padded skew: 960-row buffer (127 real), H=7168, I=2048, 32 local of 256, Zipf s=1.2",
    "c5": "prefill: T=16384, H=7168, I=2048, 32 local of 256 experts, top-8, Zipf s=1.0",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c5", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--T", type=int, default=None, help="row count override (c3: 1, 2, 4, 8, 64)")
    ap.add_argument("--cpu-seconds", type=float, default=18.0,
                    help="target length of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled parity check")
    ap.add_argument("--loop-only", action="store_true",
                    help="only warmup + timed steps (for profiler runs)")
    ap.add_argument("--forward-only", action="store_true",
                    help="only warmup + timed plan + moe_forward steps, as the library runs them "
                         "(for profiler runs of the forward's own launches)")
    ap.add_argument("--dense-expert-only", action="store_true",
                    help="time only the tiled GEMM on one dense expert of the config's H and I "
                         "(8192 rows) beside hipBLASLt on the same operands (for counter runs)")
    ap.add_argument("--lowbatch-only", action="store_true",
                    help="only the low-batch combine and cross-rank epilogue measurements "
                         "(for profiler runs of those launches)")
    ap.add_argument("--no-lowbatch", action="store_true",
                    help="skip the low-batch combine-reduce measurement")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain elementwise copy of this many MiB first (counter calibration)")
    return ap.parse_args()


def kernel_source_hash(name: str) -> str:
    """First 16 hex digits of the sha256 of a kernel source's code, with
    comments removed and whitespace runs collapsed (comment edits keep it)."""
    path = os.path.join(ROOT, "top_reduce_amd", "csrc", name)
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def stored_traffic(kernel: str, config: str, src: str):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/), or None
    when absent or taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{config}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_h and m_b) or m_h.group(1) != kernel_source_hash(src):
        return None
    return float(m_b.group(1))


def forward_gemm_launches(bf16: bool, T: int, K: int, E: int, H: int, I: int, cus: int):
    """The grouped-GEMM launches of moe_forward on a plan of this shape in the
    automatic GEMM mode, by the library's host-side rules (tiles of 256 rows
    and 256 columns, at most 32 expanded rows for the decode kernels, at most
    128 for streaming every expert). Returns (GEMM1 gathers x through the
    route table, GEMM2 writes single-slot rows to y and a reduce of the other
    rows follows, GEMM2 does the whole reduce, kernel names in launch order)."""
    cdiv = lambda a, b: -(-a // b)
    if not bf16:
        return True, False, False, ["gemm_f32<true> (GEMM1 gathering x)", "gemm_f32<false>"]
    if T * H * 2 > 0x7FFFFFFF:   # 32-bit offsets: expand first, no fused writes to y
        return False, False, False, ["gemm_tiled<true, false>", "gemm_stream<true>",
                                     "gemm_tiled<false, false>", "gemm_stream<false>"]
    if H % 256 or I % 128:
        return True, True, False, ["gemm_any<true>", "gemm_any<false>"]
    R_cap = T * K
    if R_cap <= 32:
        up = 8 if cdiv(cdiv(H, 32), 8) <= 8 else 16
        down = 8 if cdiv(cdiv(I, 32), 8) <= 8 else 16
        return True, True, True, [f"gemm_decode<true, {up}>",
                                  f"gemm_decode_y<{down}> (GEMM2 with the reduce folded in)"]
    if R_cap <= 128:
        return True, True, False, ["gemm_stream<true>", "gemm_stream<false>"]
    t1 = (cdiv(R_cap, 256) + E) * cdiv(I, 128)
    if t1 > 2 * cus:
        return True, True, False, ["gemm_tiled<true, true> (GEMM1 whole rounds)",
                                   "gemm_stream<true> (experts with <= 32 rows)",
                                   "gemm_hybrid<true> (GEMM1 last round beside early GEMM2 tiles)",
                                   "gemm_tiled<false, false> (rest of GEMM2)",
                                   "gemm_stream<false> (experts with <= 32 rows)"]
    return True, True, False, ["gemm_tiled<true, true>", "gemm_stream<true> (experts with <= 32 rows)",
                               "gemm_tiled<false, false>", "gemm_stream<false> (experts with <= 32 rows)"]


def lowbatch_combine(reps: int):
    """Device time of moe_combine_reduce on the low-batch decode rows (H=3584,
    top-16, 28 local experts, one real row in 8) at T = 1, 2, 4, 8 against
    T = 64, for the stride routing (one local slot per real row) and the dense
    stress variant (16 local slots per real row). Expert outputs are seeded
    synthetic rows.

    A Python call costs more than the kernel, so timing eager launches would
    measure the host. The `reps` launches are captured once in a HIP graph
    and the graph is replayed between two events on the replay stream: each
    time is the mean over the launches of the replays, kernel execution plus
    the graph's per-node dispatch gap. Every replay's output is compared
    bit-for-bit with the eager launch."""
    import numpy as np
    import torch

    import gen
    import top_reduce_amd as tr

    dev = torch.device("cuda:0")
    reps = max(reps, 50)
    replays = 5
    out = {"unit": "us", "launches_per_graph": reps, "replays": replays,
           "method": "HIP graph of back-to-back launches, events around the replays"}
    for variant in ("", "dense"):
        times = {}
        for T in (1, 2, 4, 8, 64):
            wl = gen.make_workload("c3", T=T, variant=variant)
            idx = torch.from_numpy(wl.idx).to(dev)
            w = torch.from_numpy(wl.weights).to(dev)
            side = torch.cuda.Stream(dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                p = tr.plan(idx, E=wl.E, H=wl.H, I=wl.I, stream=side)
                O = gen.make_expert_outputs(T * wl.K, wl.H, "bf16", seed=5)
                Od = torch.from_numpy(O.view(np.int16)).view(torch.bfloat16).to(dev)
                y_ref = torch.empty((T, wl.H), dtype=torch.bfloat16, device=dev)
                tr.combine_reduce(p, w, y=y_ref, expert_out=Od, stream=side)
                y = torch.zeros_like(y_ref)
            side.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for _ in range(reps):
                    tr.combine_reduce(p, w, y=y, expert_out=Od, stream=side)
            torch.cuda.synchronize()
            same = True
            for _ in range(3):
                y.zero_()
                g.replay()
                torch.cuda.synchronize()
                same &= bool(torch.equal(y.view(torch.int16), y_ref.view(torch.int16)))
            if not same:
                raise RuntimeError(f"low-batch combine: graph replay differs from eager (T={T})")
            st = torch.cuda.current_stream(dev)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            for _ in range(replays):
                g.replay()
            b.record(st)
            torch.cuda.synchronize()
            times[T] = a.elapsed_time(b) / (reps * replays) * 1e3
            del g
        key = "stride" if variant == "" else "dense16"
        out[key] = {str(T): round(t, 3) for T, t in times.items()}
        out[key + "_us_per_row"] = {str(T): round(t / T, 4) for T, t in times.items()}
        # per-call latency reading (T = 1..8 no slower than T = 64), and the
        # literal per-row throughput reading, which a microsecond launch floor
        # cannot meet
        out[key + "_ok"] = all(times[T] <= times[64] for T in (1, 2, 4, 8))
        out[key + "_ok_per_row"] = all(times[T] / T <= times[64] / 64 for T in (1, 2, 4, 8))
    out["criterion"] = ("met under the per-call latency reading (device time at T = 1..8 <= at "
                        "T = 64) when *_ok; *_ok_per_row is the per-row throughput reading "
                        "(t(T)/T <= t(64)/64)")
    log(f"[bench] low-batch combine (us): {out}")
    return out


def _graph_time(launch, check, reps: int, replays: int = 5) -> float:
    """Mean device time per launch (us) of `launch` captured `reps` times in a
    HIP graph and replayed; `check()` must hold after the eager launch and
    after every checked replay."""
    import torch

    dev = torch.device("cuda:0")
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        launch(side)
    side.synchronize()
    if not check():
        raise RuntimeError("eager launch failed its check")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(reps):
            launch(side)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        if not check():
            raise RuntimeError("graph replay differs from the eager launch")
    st = torch.cuda.current_stream(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(replays):
        g.replay()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * replays) * 1e3


def lowbatch_epilogue(reps: int):
    """Device time of moe_combine_epilogue on the DeepEP issue #760 combine
    shape: H=3584, 32 source ranks, one real output row in 8 with 16 rank
    contributions (the ranks holding its 16 experts), padding rows with none;
    and a dense variant where every output row is real. T = 1, 2, 4, 8 against
    T = 64; graph-replayed launches (kernel plus dispatch gap)."""
    import numpy as np
    import torch

    import top_reduce_amd as tr

    dev = torch.device("cuda:0")
    reps = max(reps, 50)
    H, P, J = 3584, 32, 16
    out = {"unit": "us", "launches_per_graph": reps, "hidden": H, "ranks": P,
           "contributions_per_real_row": J}
    rng = np.random.default_rng(760)
    for variant in ("stride", "dense"):
        times = {}
        for T in (1, 2, 4, 8, 64):
            real = np.ones(T, bool) if variant == "dense" else (np.arange(T) % 8 == 0)
            src = -np.ones((T, P), np.int32)
            for t in np.nonzero(real)[0]:
                src[t, :J] = np.arange(J) * T + t          # rank j's row for token t
            recv = torch.from_numpy(rng.standard_normal((P * T, H)).astype(np.float32)).to(
                dev).to(torch.bfloat16)
            src_d = torch.from_numpy(src).to(dev)
            y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            ref = torch.zeros((T, H), dtype=torch.float32, device=dev)
            for t in range(T):
                for j in range(P):
                    if src[t, j] >= 0:
                        ref[t] += recv[src[t, j]].float()
            ref_bf = ref.to(torch.bfloat16)

            def launch(stream, src_d=src_d, recv=recv, y=y):
                tr.combine_epilogue(src_d, recv, y=y, stream=stream)

            def check(y=y, ref_bf=ref_bf):
                return bool(torch.equal(y.view(torch.int16), ref_bf.view(torch.int16)))

            times[T] = _graph_time(launch, check, reps)
        out[variant] = {str(T): round(t, 3) for T, t in times.items()}
        out[variant + "_us_per_row"] = {str(T): round(t / T, 4) for T, t in times.items()}
        out[variant + "_ok"] = all(times[T] <= times[64] for T in (1, 2, 4, 8))
        out[variant + "_ok_per_row"] = all(times[T] / T <= times[64] / 64 for T in (1, 2, 4, 8))
    log(f"[bench] low-batch epilogue (us): {out}")
    return out


def padded_buffers(w1, w2, stream, reps: int = 20):
    """DP-padded inputs (SGLang PR #6092 review thread): the 960-row buffer of
    8 workers with batches [120, 1, ..., 1] (c4 routing) whose padding rows
    hold stale local expert ids, as a router run on zero rows would leave
    them. Forward time on a plain plan (which routes the stale ids: the
    padded GEMM input the thread warns about) against moe_plan_padded (padding
    rows cost nothing); then moe_compact_rows on the same buffer and on a
    16384-row buffer of 8 workers with halving batch sizes, in GB/s of
    effective rows read and written. The expert weights are the caller's
    (same shapes as c4's)."""
    import numpy as np
    import torch

    import gen
    import top_reduce_amd as tr

    dev = torch.device("cuda:0")
    wl = gen.make_workload("c4")
    B, counts = gen.C4_WORKER_ROWS, gen.C4_WORKER_COUNTS
    rng = np.random.default_rng(6092)
    stale = wl.idx.copy()
    pads = np.nonzero(~wl.real)[0]
    stale[pads] = rng.integers(0, wl.E, size=(pads.size, wl.K))
    idx = torch.from_numpy(stale).to(dev)
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(wl.weights).to(dev)
    bc = torch.tensor(counts, dtype=torch.int32, device=dev)
    y = torch.empty_like(x)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    out = {"workload": "c4 routing, 8 workers x 120 rows, batches [120, 1, 1, 1, 1, 1, 1, 1], "
                       "padding rows with stale local ids", "unit": "us", "launches": reps}
    ws = torch.empty(tr.workspace_size(tr.make_desc(wl.T, wl.K, wl.E, wl.H, wl.I)),
                     dtype=torch.uint8, device=dev)

    def fwd(padded):
        def run():
            if padded:
                q = tr.plan(idx, E=wl.E, H=wl.H, I=wl.I, ws=ws, stream=stream, block_rows=B,
                            block_counts=bc)
            else:
                q = tr.plan(idx, E=wl.E, H=wl.H, I=wl.I, ws=ws, stream=stream)
            tr.forward(q, x, w, w1, w2, y=y, stream=stream)
            return q
        return run

    for name, padded in (("plain_plan", False), ("padded_plan", True)):
        q = fwd(padded)()
        R = tr.plan_stats(q)[0]
        out[name] = {"us": timed(fwd(padded)), "R": R}
    out["speedup"] = out["plain_plan"]["us"] / out["padded_plan"]["us"]

    def compact_case(src, blocks, cnts):
        n_eff = int(sum(min(max(c, 0), blocks) for c in cnts))
        dst = torch.empty_like(src)
        cb = torch.tensor(cnts, dtype=torch.int32, device=dev)
        t_us = timed(lambda: tr.compact_rows(src, blocks, cb, dst=dst, stream=stream))
        amount = 2 * n_eff * src[0].numel() * src.element_size()
        ach = amount / t_us / 1e3
        return {"us": t_us, "rows": n_eff, "of_rows": src.shape[0], "bound": "hbm",
                "achieved": ach, "unit": "GB/s", "peak": PEAK_HBM_GBS, "frac": ach / PEAK_HBM_GBS,
                "algorithmic_bytes": amount}

    out["compact_c4_x"] = compact_case(x, B, counts)
    big = torch.ones((16384, wl.H), dtype=torch.bfloat16, device=dev)
    out["compact_16384"] = compact_case(big, 2048, [2048, 1024, 512, 256, 128, 64, 32, 16])
    del big
    log(f"[bench] padded buffers: {out}")
    return out


def dense_calibration(M: int, H: int, I: int, stream, reps: int = 10):
    """Dense bf16 GEMMs of the same shapes and flop as the two grouped GEMMs
    (M rows: [M, H] x [H, 2I] and [M, I] x [I, H]) through torch.matmul
    (hipBLASLt), N(0, 1) operands: what a vendor dense GEMM reaches on this
    GPU, at its power-limited clock, for the same work. A calibration, not a
    target."""
    import torch

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    a1 = torch.randn((M, H), generator=g, device=dev).to(torch.bfloat16)
    b1 = torch.randn((2 * I, H), generator=g, device=dev).to(torch.bfloat16)
    a2 = torch.randn((M, I), generator=g, device=dev).to(torch.bfloat16)
    b2 = torch.randn((H, I), generator=g, device=dev).to(torch.bfloat16)
    c1 = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    c2 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        torch.matmul(a1, b1.t(), out=c1)
        torch.matmul(a2, b2.t(), out=c2)
    torch.cuda.synchronize()
    t = [0.0, 0.0]
    for _ in range(reps):
        for i, (a, b, c) in enumerate(((a1, b1, c1), (a2, b2, c2))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.matmul(a, b.t(), out=c)
            e1.record(stream)
            torch.cuda.synchronize()
            t[i] += e0.elapsed_time(e1) * 1e3 / reps
    flops = 6.0 * M * H * I
    tf = flops / ((t[0] + t[1]) * 1e-6) / 1e12
    out = {"kernel": "torch.matmul bf16 (hipBLASLt), dense, N(0,1) operands",
           "shapes_mnk": [[M, 2 * I, H], [M, H, I]], "us": [t[0], t[1]], "TFLOP/s": tf,
           "frac": tf / PEAK_BF16_TFLOPS,
           "note": "same flop as the grouped GEMMs, as one dense GEMM per projection; calibration only"}
    log(f"[bench] dense bf16 calibration: {tf:.1f} TFLOP/s ({t[0]:.1f} + {t[1]:.1f} us)")
    del a1, b1, a2, b2, c1, c2
    return out


def dense_expert(M: int, H: int, I: int, stream, reps: int = 10):
    """The tiled grouped GEMM on one dense expert of M rows (every row routed
    to expert 0, tiled mode) beside torch.matmul (hipBLASLt) on the same
    operands: [M, H] x [H, 2I] with SwiGLU, and [M, I] x [I, H]. Separates the
    kernel's own efficiency from what ragged experts cost it. A calibration,
    not a target."""
    import torch

    import top_reduce_amd as tr

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(6)
    x = torch.randn((M, H), generator=g, device=dev).to(torch.bfloat16)
    w1 = (torch.randn((1, 2 * I, H), generator=g, device=dev) / H ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn((1, H, I), generator=g, device=dev) / I ** 0.5).to(torch.bfloat16)
    idx = torch.zeros((M, 1), dtype=torch.int64, device=dev)
    p = tr.plan(idx, E=1, H=H, I=I, flags=tr.FLAG_GEMM_FORCE_TILED, stream=stream)
    hcur = p.views()["h"][:M]
    b1, b2 = w1[0], w2[0]
    c1 = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    c2 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    runs = (lambda: tr.grouped_gemm_up_x(p, x, w1, stream=stream),
            lambda: tr.grouped_gemm_down(p, w2, stream=stream),
            lambda: torch.matmul(x, b1.t(), out=c1),
            lambda: torch.matmul(hcur, b2.t(), out=c2))
    for _ in range(2):
        for r in runs:
            r()
    torch.cuda.synchronize()
    t = [0.0] * 4
    for _ in range(reps):
        for i, r in enumerate(runs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            r()
            e1.record(stream)
            torch.cuda.synchronize()
            t[i] += e0.elapsed_time(e1) * 1e3 / reps
    f = (4.0 * M * I * H, 2.0 * M * H * I)
    frac = [f[i % 2] / (t[i] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS for i in range(4)]
    out = {"shapes_mnk": [[M, 2 * I, H], [M, H, I]], "unit": "us",
           "tiled_kernel_us": [t[0], t[1]], "tiled_kernel_frac": [frac[0], frac[1]],
           "hipblaslt_us": [t[2], t[3]], "hipblaslt_frac": [frac[2], frac[3]],
           "note": "one dense expert, N(0,1) activations; calibration only"}
    log(f"[bench] dense expert M={M}: tiled kernel {t[0]:.1f} + {t[1]:.1f} us "
        f"({frac[0]:.3f}, {frac[1]:.3f} of peak), hipBLASLt {t[2]:.1f} + {t[3]:.1f} us "
        f"({frac[2]:.3f}, {frac[3]:.3f})")
    del x, w1, w2, p, c1, c2
    return out


def copy_reference(stream, nbytes: int = 1 << 30, reps: int = 20):
    """Bandwidth of a plain device copy (torch's elementwise negation, read
    nbytes + write nbytes) on the same GPU in the same run: the practical
    ceiling for the HBM-bound kernels, next to the published 8 TB/s."""
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        torch.neg(src, out=dst)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    log(f"[bench] copy reference: {gbs:.1f} GB/s ({us:.1f} us for {2 * nbytes} bytes)")
    return {"GB/s": gbs, "bytes": 2 * nbytes, "us": us, "kernel": "torch.neg bf16 (read + write)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); this "
              "build has no multi-GPU path: sharding is by expert range, one process per GPU, "
              "each running this same single-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import top_reduce_amd as tr

    if not os.path.exists(tr.lib_path()):   # a fresh checkout: build it first
        from top_reduce_amd import build as hip_build
        hip_build.build()
    tr.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.lowbatch_only:
        out = {"lowbatch_combine": lowbatch_combine(args.steps),
               "lowbatch_epilogue": lowbatch_epilogue(args.steps)}
        print(json.dumps({"metric": METRIC, "lowbatch_only": True, **out}), flush=True)
        return
    if args.dense_expert_only:
        spec = gen.CONFIGS[args.config]
        H, I = spec.H, spec.I
        out = dense_expert(8192, H, I, torch.cuda.current_stream(dev), reps=args.steps)
        print(json.dumps({"metric": METRIC, "dense_expert_only": True, "dense_expert": out}), flush=True)
        return
    t0 = time.time()
    wl = gen.make_workload(args.config, T=args.T, with_weights=True)
    log(f"[bench] generated {args.config} T={wl.T} in {time.time() - t0:.1f}s")
    bf16 = wl.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    idx = torch.from_numpy(wl.idx).to(dev)
    x, w = up(wl.x), torch.from_numpy(wl.weights).to(dev)
    w1, w2 = up(wl.w1), up(wl.w2)
    y = torch.empty((wl.T, wl.H), dtype=tdt, device=dev)
    desc = tr.make_desc(wl.T, wl.K, wl.E, wl.H, wl.I, tdt, torch.int64)
    ws = torch.empty(tr.workspace_size(desc), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        p = tr.plan(idx, E=wl.E, H=wl.H, I=wl.I, dtype=tdt, ws=ws, stream=stream)
        tr.forward(p, x, w, w1, w2, y=y, stream=stream)
        return p

    p = step()
    R, T_loc, _, n_empty = tr.plan_stats(p)
    real_rows = int(wl.real.sum())
    # received rows with exactly one local slot (GEMM2 writes them to y)
    n_single = int((p.views()["row_dst"][:R] >= 0).sum()) if R else 0
    log(f"[bench] R={R} T_loc={T_loc} real_rows={real_rows} empty_experts={n_empty} "
        f"single_slot_rows={n_single}")

    if args.copy_calibration_mib:
        # A plain elementwise kernel over a known number of bytes: its HBM
        # counters calibrate the counters of the path's kernels.
        n = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: torch.neg over {n * 2} bytes read + {n * 2} written, x3")
        del src, dst

    if args.forward_only:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(args.steps):
            step()
        f1.record(stream)
        torch.cuda.synchronize()
        ms = f0.elapsed_time(f1) / args.steps
        log(f"[bench] {args.steps} forward steps: {ms:.4f} ms/step")
        print(json.dumps({"metric": METRIC, "value": int(wl.real.sum()) / (ms / 1e3), "unit": "tokens/s",
                          "ms_per_step": ms, "forward_only": True}), flush=True)
        return

    # One step = plan (route scan) + forward: the same kernels moe_forward
    # launches (GEMM up gathering x through the route table; bf16: GEMM down
    # writing single-slot rows to y, the reduce of the other rows; fp32: GEMM
    # down writing every expert row, the full reduce), called stage by stage
    # so that events between the stages, on the launch stream, give each
    # kernel's device time inside the timed region.
    gather, fused, reduce_in_gemm2, launches = forward_gemm_launches(
        bf16, wl.T, wl.K, wl.E, wl.H, wl.I, torch.cuda.get_device_properties(dev).multi_processor_count)
    stage_names = (("route_scan", "gemm_up", "gemm_down", "combine_reduce") if gather else
                   ("route_scan", "expand", "gemm_up", "gemm_down", "combine_reduce"))

    def staged_step(evs):
        i = 0
        evs[i].record(stream)
        q = tr.plan(idx, E=wl.E, H=wl.H, I=wl.I, dtype=tdt, ws=ws, stream=stream)
        i += 1
        evs[i].record(stream)
        if gather:
            tr.grouped_gemm_up_x(q, x, w1, stream=stream)
        else:
            tr.expand(q, x, stream=stream)
            i += 1
            evs[i].record(stream)
            tr.grouped_gemm_up(q, w1, stream=stream)
        i += 1
        evs[i].record(stream)
        if fused:
            tr.grouped_gemm_down_y(q, w2, w, y, stream=stream)
        else:
            tr.grouped_gemm_down(q, w2, stream=stream)
        i += 1
        evs[i].record(stream)
        if fused:
            tr.combine_reduce_multi(q, w, y, stream=stream)
        else:
            tr.combine_reduce(q, w, y=y, stream=stream)
        evs[i + 1].record(stream)

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(stage_names) + 1)]

    for _ in range(args.warmup):
        staged_step(new_events())
    torch.cuda.synchronize()
    step_events = [new_events() for _ in range(args.steps)]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for evs in step_events:
        staged_step(evs)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    tokens_per_s = real_rows * args.steps / (ms_total / 1e3)
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step (wall {wall / args.steps * 1e3:.4f}), "
        f"{tokens_per_s:.4e} tokens/s")

    # The forward as the library runs it (bf16 with enough tiles: GEMM1's
    # whole rounds, its last round beside early GEMM2 tiles, the rest of
    # GEMM2, the few-row experts' streaming launches, then the reduce), eager,
    # with events around moe_forward on the launch stream. Its GEMM launches
    # take the forward's time minus the reduce (and, for fp32, the expand) of
    # the staged steps: the same kernels over the same rows.
    def forward_step(e0, e1):
        q = tr.plan(idx, E=wl.E, H=wl.H, I=wl.I, dtype=tdt, ws=ws, stream=stream)
        e0.record(stream)
        tr.forward(q, x, w, w1, w2, y=y, stream=stream)
        e1.record(stream)

    for _ in range(args.warmup):
        forward_step(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    fwd_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
    for e0, e1 in fwd_events:
        forward_step(e0, e1)
    torch.cuda.synchronize()
    fwd_us = sum(e0.elapsed_time(e1) for e0, e1 in fwd_events) / args.steps * 1e3
    b = 2 if bf16 else 4
    H, I, T, K = wl.H, wl.I, wl.T, wl.K

    def expand_alone(reps: int = 20):
        """moe_expand on the step's plan, outside the step: the bf16 forward
        gathers x inside GEMM1 instead, but the entry point stays (fp32
        forwards, callers that keep the expanded rows)."""
        tr.expand(p, x, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            tr.expand(p, x, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t_us = e0.elapsed_time(e1) / reps * 1e3
        amount = (T_loc + R) * H * b + 4 * T * K
        ach = amount / t_us / 1e3
        log(f"[bench] expand (alone)   {t_us:10.2f} us  {ach:9.1f} GB/s  "
            f"{100 * ach / PEAK_HBM_GBS:5.1f}% of peak")
        return {"us": t_us, "bound": "hbm", "achieved": ach, "unit": "GB/s", "peak": PEAK_HBM_GBS,
                "frac": ach / PEAK_HBM_GBS, "algorithmic_bytes": amount, "launches": reps}

    if args.loop_only:
        print(json.dumps({"metric": METRIC, "value": tokens_per_s, "unit": "tokens/s",
                          "ms_per_step": ms_step, "loop_only": True,
                          "expand_alone": expand_alone(args.steps)}), flush=True)
        return
    eager = {"ms_per_step": ms_step, "tokens_per_s": tokens_per_s,
             "launch": "plan + the stage entry points from Python, events between stages"}

    # The same step (moe_plan + moe_forward) captured once in a HIP graph and
    # replayed: the host launch cost, which dominates the small decode shapes,
    # leaves the timed region. Every replay must reproduce the eager output
    # bit for bit (the path is deterministic and allocates nothing).
    y_ref = y.clone()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        qg = tr.plan(idx, E=wl.E, H=wl.H, I=wl.I, dtype=tdt, ws=ws, stream=side)
        tr.forward(qg, x, w, w1, w2, y=y, stream=side)
    torch.cuda.synchronize()
    for _ in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y.view(torch.int16 if bf16 else torch.int32),
                           y_ref.view(torch.int16 if bf16 else torch.int32)):
            raise RuntimeError("graph replay differs from the eager step")
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    ms_step = g0.elapsed_time(g1) / args.steps
    tokens_per_s = real_rows / (ms_step / 1e3)
    log(f"[bench] {args.steps} graph steps: {ms_step:.4f} ms/step, {tokens_per_s:.4e} tokens/s "
        f"(eager {eager['ms_per_step']:.4f} ms/step)")
    del graph
    # mean device time of each stage over the timed steps, us per launch
    us = {name: sum(evs[i].elapsed_time(evs[i + 1]) for evs in step_events) / args.steps * 1e3
          for i, name in enumerate(stage_names)}
    peak_mm = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    work = {
        # algorithmic bytes / flops per launch
        "expand": ("hbm", (T_loc + R) * H * b + 4 * T * K),
        "gemm_up": ("mfma" if bf16 else "alu", 4.0 * R * H * I),
        "gemm_down": ("mfma" if bf16 else "alu", 2.0 * R * H * I),
        "combine_reduce": ("hbm", R * H * b + T * H * b + 8 * T * K),
    }
    if gather:
        del work["expand"]
    if fused:
        # the reduce reads the rows of received rows with several local slots
        # and writes those and the rows without a local slot
        work["combine_reduce"] = ("hbm", (R - n_single) * H * b + (T - n_single) * H * b + 8 * T * K)
    # A GEMM whose arithmetic intensity (flops per algorithmic byte: the
    # weights of the non-empty experts plus the activations read and written)
    # is below the ridge of MFMA peak / HBM peak is bound by streaming its
    # weights, and is reported in GB/s (decode and DP-padded shapes).
    n_active = wl.E - n_empty
    gemm_bytes = {
        "gemm_up": n_active * 2 * I * H * b + T_loc * H * b + R * I * b,
        "gemm_down": n_active * H * I * b + R * I * b + R * H * b,
    }
    ridge = peak_mm * 1e12 / (PEAK_HBM_GBS * 1e9)
    stages = {"route_scan": {"us": us["route_scan"]}}
    for k, (bound, amount) in work.items():
        t_s = us[k] / 1e6
        extra = {}
        if k in gemm_bytes:
            ai = amount / gemm_bytes[k]
            extra = {"algorithmic_flops": amount, "algorithmic_bytes": gemm_bytes[k],
                     "arith_intensity": ai, "ridge": ridge}
            if ai < ridge:
                bound, amount = "hbm", gemm_bytes[k]
        if bound == "hbm":
            ach = amount / t_s / 1e9
            stages[k] = {"us": us[k], "bound": "hbm", "achieved": ach, "unit": "GB/s",
                         "peak": PEAK_HBM_GBS, "frac": ach / PEAK_HBM_GBS, "algorithmic_bytes": amount}
        else:
            ach = amount / t_s / 1e12
            stages[k] = {"us": us[k], "bound": bound, "achieved": ach, "unit": "TFLOP/s",
                         "peak": peak_mm, "frac": ach / peak_mm, "algorithmic_flops": amount}
        stages[k].update(extra)
    # The dominant kernels: the forward's GEMM launches (both projections,
    # 95% of a prefill step), timed inside the forward as the library runs it:
    # the forward's time minus its reduce launch, if it makes one.
    gemm_fwd_us = (fwd_us - (0.0 if reduce_in_gemm2 else us["combine_reduce"])
                   - (0.0 if gather else us["expand"]))
    both_flops = 6.0 * R * H * I
    both_bytes = gemm_bytes["gemm_up"] + gemm_bytes["gemm_down"]
    t_gemm = gemm_fwd_us / 1e6
    if bf16 and both_flops / both_bytes >= ridge:
        ach = both_flops / t_gemm / 1e12
        roofline = {"bound": "mfma", "achieved": ach, "peak": peak_mm, "unit": "TFLOP/s",
                    "frac": ach / peak_mm}
    elif bf16:
        ach = both_bytes / t_gemm / 1e9
        roofline = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": ach / PEAK_HBM_GBS}
    else:
        ach = both_flops / t_gemm / 1e12
        roofline = {"bound": "mfma", "achieved": ach, "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                    "frac": ach / PEAK_F32_TFLOPS}
    roofline = {"kernel": "grouped GEMM, both projections, as moe_forward launches them",
                **roofline,
                "traffic": stored_traffic("gemm_forward",
                                          args.config + (f"_T{args.T}" if args.T else ""),
                                          "grouped_gemm.hip"),
                "us_per_step": gemm_fwd_us, "algorithmic_flops": both_flops,
                "algorithmic_bytes": both_bytes, "launches": launches,
                "method": "HIP events around moe_forward in eager steps"
                          + ("" if reduce_in_gemm2 else ", minus the reduce")
                          + ("" if gather else " and the expand")
                          + ("" if reduce_in_gemm2 and gather else " of the staged steps")}
    log(f"[bench] forward GEMM launches {gemm_fwd_us:10.2f} us  {roofline['achieved']:9.1f} "
        f"{roofline['unit']}  {100 * roofline['frac']:5.1f}% of peak (forward {fwd_us:.2f} us)")
    for k, v in stages.items():
        log(f"[bench] {k:15s} {v['us']:10.2f} us" +
            (f"  {v['achieved']:9.1f} {v['unit']}  {100 * v['frac']:5.1f}% of peak" if "frac" in v else ""))

    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": f"{args.config} {WORKLOAD_NAMES[args.config]}", "T": T,
                   "real_rows": real_rows, "K": K, "E_local": wl.E, "E_global": wl.G, "H": H,
                   "I": I, "R": R, "T_loc": T_loc, "single_slot_rows": n_single,
                   "empty_experts": n_empty, "seed": wl.seed,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "stages": stages,
        "stages_launch": "stage entry points, one launch per GEMM (eager steps, events between stages)",
        "launch": "one step captured in a HIP graph, replayed; stage times from the eager steps",
        "eager": eager,
        "eager_forward_us": fwd_us,
    }
    if bf16 and both_flops / both_bytes >= ridge:
        result["dense_bf16_calibration"] = dense_calibration(R, H, I, stream)
        if H % 256 == 0 and I % 128 == 0:
            result["dense_expert"] = dense_expert(8192, H, I, stream)
    if gather:
        result["expand_alone"] = expand_alone()

    if not args.no_lowbatch:
        result["lowbatch_combine"] = lowbatch_combine(args.steps)
        result["lowbatch_epilogue"] = lowbatch_epilogue(args.steps)
    if not args.no_lowbatch and (wl.E, wl.H, wl.I) == (32, 7168, 2048) and bf16:
        result["padded_buffers"] = padded_buffers(w1, w2, stream)
    result["hbm_copy_reference"] = copy_reference(stream)
    result["buffer_rows_per_s"] = T / (ms_step / 1e3)

    # The HBM-bound stages once more with cold caches: before each launch a
    # 1 GiB read (a sum, so no dirty lines are left to write back during the
    # timed launch) evicts L2 and the 256 MB MALL, so the operands come from
    # HBM.
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def cold_us(launch, reps: int = 10) -> float:
        times = []
        for _ in range(reps):
            scratch.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        return sorted(times)[len(times) // 2]

    cold = {}
    y2 = torch.empty_like(y)
    if fused:
        cold["combine_reduce"] = cold_us(lambda: tr.combine_reduce_multi(p, w, y2, stream=stream))
        cold["expand_alone"] = cold_us(lambda: tr.expand(p, x, stream=stream))
        # the full reduce over every received row (moe_combine_reduce after the
        # unfused GEMM2 has written every expert row to O)
        tr.grouped_gemm_down(p, w2, stream=stream)
        cold["combine_reduce_full"] = cold_us(lambda: tr.combine_reduce(p, w, y=y2, stream=stream))
        cold_bytes = {"combine_reduce": work["combine_reduce"][1],
                      "expand_alone": (T_loc + R) * H * b + 4 * T * K,
                      "combine_reduce_full": R * H * b + T * H * b + 8 * T * K}
    else:
        # fp32 forwards gather x in GEMM1 too: moe_expand is timed alone
        ek = "expand_alone" if gather else "expand"
        cold["combine_reduce"] = cold_us(lambda: tr.combine_reduce(p, w, y=y, stream=stream))
        cold[ek] = cold_us(lambda: tr.expand(p, x, stream=stream))
        cold_bytes = {"combine_reduce": work["combine_reduce"][1],
                      ek: (T_loc + R) * H * b + 4 * T * K}
    # the GEMM stages cold: weight-streaming shapes (arithmetic intensity
    # below the ridge) are claimed against HBM on these numbers
    if fused:
        cold["gemm_up"] = cold_us(lambda: tr.grouped_gemm_up_x(p, x, w1, stream=stream))
        cold["gemm_down"] = cold_us(lambda: tr.grouped_gemm_down_y(p, w2, w, y2, stream=stream))
        cold_bytes["gemm_up"] = gemm_bytes["gemm_up"]
        cold_bytes["gemm_down"] = gemm_bytes["gemm_down"]
        if 0 < n_active <= 4:
            # The vendor library on the same decode shape: one row against each
            # active expert's W1 and W2 (torch.nn.functional.linear, a GEMV in
            # rocBLAS / hipBLASLt), cold, timed like the GEMMs. Calibration
            # only; nothing of the path runs here.
            act = [int(e) for e in np.nonzero(p.views()["counts"].cpu().numpy())[0]]
            xr = x[:1].contiguous()
            hr = torch.ones((1, I), dtype=x.dtype, device=dev)
            F = torch.nn.functional
            cold["library_gemv_up"] = cold_us(lambda: [F.linear(xr, w1[e]) for e in act])
            cold["library_gemv_down"] = cold_us(lambda: [F.linear(hr, w2[e]) for e in act])
            cold_bytes["library_gemv_up"] = len(act) * 2 * I * H * b
            cold_bytes["library_gemv_down"] = len(act) * H * I * b
    result["cold"] = {k: {"us": v, "achieved": cold_bytes[k] / v / 1e3, "unit": "GB/s",
                          "peak": PEAK_HBM_GBS, "frac": cold_bytes[k] / v / 1e3 / PEAK_HBM_GBS,
                          "method": "median of 10 launches, each after reading 1 GiB"}
                      for k, v in cold.items()}
    for k in ("library_gemv_up", "library_gemv_down"):
        if k in result["cold"]:
            result["cold"][k]["kernel"] = ("torch.nn.functional.linear of one row against each "
                                           "active expert's " + ("W1" if k.endswith("up") else "W2") +
                                           " (vendor GEMV on the same weights; calibration)")
    for k in ("gemm_up", "gemm_down"):
        if k in result["cold"]:
            flops = work[k][1]
            result["cold"][k]["TFLOP/s"] = flops / result["cold"][k]["us"] / 1e6
            result["cold"][k]["arith_intensity"] = flops / cold_bytes[k]
    for k, v in result["cold"].items():
        log(f"[bench] cold {k:15s} {v['us']:10.2f} us  {v['achieved']:9.1f} GB/s  "
            f"{100 * v['frac']:5.1f}% of peak")
    del scratch, y2

    # Sampled parity and the CPU oracle baseline on a bounded sample.
    if not (args.no_check and args.no_cpu_baseline):
        import oracle
        nthreads = oracle.threads()
        routes_per_row = max(R / max(real_rows, 1), 1e-9)
        probe = np.arange(min(16, T))
        t1 = time.perf_counter()
        oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E, tokens=probe)
        per_route = (time.perf_counter() - t1) / max(int((wl.idx[probe] >= 0).sum()), 1)
        n = int(args.cpu_seconds / max(per_route * routes_per_row, 1e-9))
        n = min(T, max(16, n))
        toks = np.arange(n)
        t1 = time.perf_counter()
        ref = oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E, tokens=toks)
        cpu_s = time.perf_counter() - t1
        n_real = int(wl.real[toks].sum())
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {
                "value": n_real / cpu_s, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
                "seconds": cpu_s,
                "sample": f"first {n} of {T} rows of the same workload ({n_real} real rows, "
                          f"{int((wl.idx[toks] >= 0).sum())} local routes), fp64 oracle, "
                          f"{nthreads} OpenMP threads"}
            log(f"[bench] cpu oracle: {n_real / cpu_s:.2f} tokens/s on {nthreads} threads ({cpu_s:.1f}s)")
        if not args.no_check:
            yh = y[:n].float().cpu().numpy().astype(np.float64)
            err = float(np.abs(yh - ref).max())
            tol = (1e-2 * float(np.abs(ref).max()) + 1e-3) if bf16 else 1e-5 * float(np.abs(ref).max())
            result["parity"] = {"rows": n, "max_abs_err": err, "tol": tol, "ratio": err / tol if tol else 0.0,
                                "ok": err <= tol}
            log(f"[bench] parity on {n} rows: max|d|={err:.3e} tol={tol:.3e}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
