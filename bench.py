"""Throughput of speculative-sampling verification on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload c2]
                    [--no-cpu-baseline] [--cpu-seconds 12] [--cpu-procs 16]

Default workload (the headline line): one step = one sv_verify_chain call over
one batch of B=64 sequences, K=5 drafted tokens, V=128256, bf16 logits,
temperature 0.7 (synthetic, seeded: target N(0, 2.5^2) plus a Zipf(1.1)
log-prior, draft = target + N(0, 0.8^2)). Three independent input sets
(3 x 180.6 MB) are rotated so that the 256 MB last-level cache cannot serve a
step from the previous one; every input is resident in HBM before the timed
region starts. Other workloads (--workload c1, c3_s0.3, c3_s1.0, c3_s3.0, c5,
c4, c4s) print a line of the same form; c5 rotates its ten iterations (one
set of logits, fresh uniforms each), c4 is the greedy tree call, c4s the
sampling tree call (B=32, N=64, V=128256 bf16, target and draft rows at every
position: 2 x 534 MB per input set). The s1, s2 and s3
workloads time draft-side sampling (sv_sample_rows) over the draft rows of c1,
c2 and c3_s1.0 (B*K rows each, one token drawn per row).

Prints one JSON line: rows x vocab elements verified per second over the
whole call, the roofline of the dominant kernel (the streaming pass, timed
with HIP events the library records around that one kernel) against MI355X's
8 TB/s HBM peak, its HBM traffic from committed rocprofv3 counter runs (when
the kernel sources still match the ones counted), and the CPU oracle timed on
a bounded sample of the same workload: on one core (cpu_baseline), and for the
chain workloads also in --cpu-procs worker processes at once (child processes
of this script with the GPU hidden, each running the unchanged oracle on its
own share of the sequences: cpu_baseline_multicore).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify throughput: rows·vocab/s + HBM GB/s vs peak, B=64 K=5 V=128256 bf16"
HBM_PEAK_GBS = 8000.0
N_SETS = 3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "rejection_sampling_verification_sv_amd", "csrc")
KERNEL_SOURCES = {
    "chain": ["sv_chain.hip", "sv_stream.h", "sv_device.h", "sv_internal.h", "sv_api.hip"],
    "sample": ["sv_sample.hip", "sv_device.h", "sv_internal.h", "sv_api.hip"],
    "tree": ["sv_tree.hip", "sv_device.h", "sv_internal.h", "sv_api.hip"],
    # the counted kernel is the statistics stream of sv_tree_sample.hip (the walk shares the file)
    "treesample": ["sv_tree_sample.hip", "sv_stream.h", "sv_device.h", "sv_internal.h", "sv_api.hip"],
    "lmhead": ["sv_lm_head.hip", "sv_device.h", "sv_internal.h", "sv_api.hip"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2",
                    help="c1, c2, c3_s0.3, c3_s1.0, c3_s3.0, c5 (chain), c4 (greedy tree), c4s (sampling tree), "
                         "s1, s2, s3 (draft-side sampling) or c2h (chain with the target's LM head in the call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of each call captured in a HIP graph (the call's launches without the "
                         "host-side launch path)")
    ap.add_argument("--entropy", action="store_true",
                    help="chain workloads: also request every position's entropy (the stream's entropy variant)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="bound on the oracle sample's wall time")
    ap.add_argument("--cpu-procs", type=int, default=16,
                    help="chain workloads: worker processes for the multi-core oracle figure (0: none)")
    # a worker of the multi-core oracle figure (started by this script itself)
    ap.add_argument("--oracle-worker", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--worker-index", type=int, default=0, help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run three plain device-to-device copies of MIB MiB (untimed), the known-size "
                         "kernel that scales hardware traffic counters")
    return ap.parse_args()


def sources_sha256(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def counted_traffic(workload: str, kind: str):
    """HBM bytes per launch of the streaming kernel from the committed counter
    runs (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or
    None when there are none or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != sources_sha256(kind):
        return None
    return rec["traffic_bytes_per_launch"]


def _timed_oracle(jobs, budget_s: float):
    """Run oracle jobs (each a (prepare, run, count) triple) in order, wrapping
    around, until about `budget_s` seconds have been spent inside `run`; the
    input conversion in `prepare` is not timed. Returns (items, wall, cpu)."""
    import torch

    threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        done = wall = cpu = 0.0
        i = 0
        while wall < budget_s:
            prepare, run, count = jobs[i % len(jobs)]
            args = prepare()
            t0, c0 = time.perf_counter(), os.times()
            run(*args)
            t1, c1 = time.perf_counter(), os.times()
            wall += t1 - t0
            cpu += (c1.user - c0.user) + (c1.system - c0.system)
            done += count
            i += 1
    finally:
        torch.set_num_threads(threads)
    return int(done), wall, cpu


def _chain_oracle_jobs(inp, cfg, first: int = 0):
    """Oracle jobs over the batch, four sequences each, starting at group `first`."""
    import oracle

    jobs = []
    for s0 in range(0, cfg.B, 4):
        s = slice(s0, min(cfg.B, s0 + 4))
        jobs.append((lambda s=s: (inp["target"][s].double().numpy(), inp["draft"][s].double().numpy(),
                                  inp["draft_tokens"][s].numpy().astype("int64"),
                                  inp["temperature"][s].double().numpy(), inp["uniforms"][s].double().numpy()),
                     oracle.verify_chain, s.stop - s.start))
    first %= len(jobs)
    return jobs[first:] + jobs[:first]


def cpu_baseline_chain(inp, cfg, budget_s: float) -> dict:
    """The float64 numpy oracle on the same workload: sequences four at a time,
    in order, wrapping around the batch, for about `budget_s` seconds."""
    done, wall, cpu = _timed_oracle(_chain_oracle_jobs(inp, cfg), budget_s)
    return {
        "value": done * (2 * cfg.K + 1) * cfg.V / wall,
        "unit": "rows·vocab/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{done} sequences ({done / cfg.B:.2f} passes over the {cfg.B}-sequence batch) of the same "
                  f"workload, float64 numpy, {wall:.1f} s in the oracle, {cpu:.1f} s CPU",
    }


def oracle_worker(args) -> None:
    """One process of the multi-core oracle figure: the workload's first input
    set generated on the CPU, the oracle timed as in cpu_baseline_chain from
    its own starting group of sequences; prints (sequences, wall, cpu)."""
    from workloads import CHAIN_CONFIGS, chain_inputs

    cfg = CHAIN_CONFIGS[args.workload]
    inp = chain_inputs(cfg, device="cpu")
    done, wall, cpu = _timed_oracle(_chain_oracle_jobs(inp, cfg, first=args.worker_index), args.cpu_seconds)
    print(json.dumps({"done": done, "wall": wall, "cpu": cpu}), flush=True)


def cpu_baseline_chain_procs(wl: str, cfg, budget_s: float, procs: int) -> dict:
    """The oracle in `procs` worker processes at once (this script with
    --oracle-worker, the GPU hidden from them), each for about `budget_s`
    seconds of oracle time: the sum of their rates."""
    import subprocess

    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="",
               OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    cmd = [sys.executable, os.path.abspath(__file__), "--oracle-worker", "--workload", wl,
           "--cpu-seconds", str(budget_s)]
    ps = [subprocess.Popen(cmd + ["--worker-index", str(i)], stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                           env=env, text=True) for i in range(procs)]
    recs = []
    for p in ps:
        out, err = p.communicate(timeout=budget_s + 600)
        if p.returncode != 0:
            raise RuntimeError(f"oracle worker failed ({p.returncode}): {err[-2000:]}")
        recs.append(json.loads(out.strip().splitlines()[-1]))
    per_seq = (2 * cfg.K + 1) * cfg.V
    done = sum(r["done"] for r in recs)
    return {
        "value": sum(r["done"] * per_seq / r["wall"] for r in recs),
        "unit": "rows·vocab/s",
        "cores": procs,
        "kind": "oracle",
        "sample": f"{procs} processes at once, each running the oracle on its own share of the same workload's "
                  f"sequences for about {budget_s:.0f} s ({done} sequences in all, float64 numpy, one thread each)",
    }


def cpu_baseline_tree(inp, cfg, budget_s: float) -> dict:
    """The oracle's greedy tree verification, one sequence at a time."""
    import oracle

    parents = inp["parents"].numpy()
    jobs = [(lambda b=b: (inp["target"][b:b + 1].float().numpy(), inp["node_tokens"][b:b + 1].numpy(), parents),
             oracle.verify_tree_greedy, 1) for b in range(cfg.B)]
    done, wall, cpu = _timed_oracle(jobs, budget_s)
    return {
        "value": done * (cfg.N + 1) * cfg.V / wall,
        "unit": "rows·vocab/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{done} sequences ({done / cfg.B:.2f} passes over the {cfg.B}-sequence batch) of the same "
                  f"workload, numpy argmax, {wall:.1f} s in the oracle, {cpu:.1f} s CPU",
    }


def cpu_baseline_tree_sampling(inp, cfg, budget_s: float) -> dict:
    """The oracle's sampling tree verification, one sequence at a time."""
    import oracle

    parents = inp["parents"].numpy().astype("int64")
    jobs = [(lambda b=b: (inp["target"][b:b + 1].double().numpy(), inp["draft"][b:b + 1].double().numpy(),
                          inp["node_tokens"][b:b + 1].numpy().astype("int64"), parents,
                          inp["temperature"][b:b + 1].double().numpy(), inp["uniforms"][b:b + 1].double().numpy()),
             oracle.verify_tree_stochastic, 1) for b in range(cfg.B)]
    done, wall, cpu = _timed_oracle(jobs, budget_s)
    return {
        "value": done * 2 * (cfg.N + 1) * cfg.V / wall,
        "unit": "rows·vocab/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{done} sequences ({done / cfg.B:.2f} passes over the {cfg.B}-sequence batch) of the same "
                  f"workload, float64 numpy, {wall:.1f} s in the oracle, {cpu:.1f} s CPU",
    }


# draft-side sampling workloads: the draft rows of a chain configuration
SAMPLE_WORKLOADS = {"s1": "c1", "s2": "c2", "s3": "c3_s1.0"}


def cpu_baseline_sample(inp, cfg, budget_s: float) -> dict:
    """The oracle's draft-side sampling, 16 rows at a time."""
    import oracle

    R = inp["logits"].shape[0]
    jobs = []
    for r0 in range(0, R, 16):
        s = slice(r0, min(R, r0 + 16))
        jobs.append((lambda s=s: (inp["logits"][s].double().numpy(), inp["temperature"][s].double().numpy(),
                                  inp["uniforms"][s].double().numpy()),
                     oracle.sample_rows, s.stop - s.start))
    done, wall, cpu = _timed_oracle(jobs, budget_s)
    return {
        "value": done * cfg.V / wall,
        "unit": "rows·vocab/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{done} rows ({done / R:.2f} passes over the {R} rows) of the same workload, float64 numpy, "
                  f"{wall:.1f} s in the oracle, {cpu:.1f} s CPU",
    }


def cpu_baseline_lm_head(inp, cfg, budget_s: float) -> dict:
    """The oracle's LM-head chain verification (fp64 matmul of each sequence's
    hidden states with the whole head, bf16 rounding, verify_chain), one
    sequence at a time; the head's conversion to fp64 is not timed."""
    import numpy as np

    import oracle

    w64 = inp["weight"].double().numpy()
    jobs = [(lambda b=b: (inp["hidden"][b:b + 1].double().numpy(), w64, inp["draft"][b:b + 1].double().numpy(),
                          inp["draft_tokens"][b:b + 1].numpy().astype(np.int64),
                          inp["temperature"][b:b + 1].double().numpy(), inp["uniforms"][b:b + 1].double().numpy()),
             oracle.verify_chain_lm_head, 1) for b in range(cfg.B)]
    threads_before = os.environ.get("OMP_NUM_THREADS")
    done, wall, cpu = _timed_oracle(jobs, budget_s)
    return {
        "value": done * (2 * cfg.K + 1) * cfg.V / wall,
        "unit": "rows·vocab/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{done} sequences of the same workload (fp64 LM head through numpy's multithreaded matmul, "
                  f"OMP_NUM_THREADS={threads_before}), {wall:.1f} s in the oracle, {cpu:.1f} s CPU",
    }


def bench_lm_head(args, sv, torch, cfg, dev, stream) -> dict:
    """Chain verification with the target's LM head in the call, against the
    LM head alone followed by sv_verify_chain on its logits."""
    from workloads import lm_head_chain_inputs

    B, K, V, H = cfg.B, cfg.K, cfg.V, cfg.H
    M = B * (K + 1)
    sets = [lm_head_chain_inputs(cfg.with_(variant=cfg.variant + 10 * i) if i else cfg, device=dev)
            for i in range(N_SETS)]
    fused = [sv.PreparedLMHeadChainCall(x["hidden"], x["weight"], x["draft"], x["draft_tokens"], x["temperature"],
                                        x["uniforms"], stream=stream) for x in sets]
    heads = [sv.PreparedLMHeadLogitsCall(x["hidden"], x["weight"], stream=stream) for x in sets]
    verifies = [sv.PreparedChainCall(h.logits, x["draft"], x["draft_tokens"], x["temperature"], x["uniforms"],
                                     stream=stream) for h, x in zip(heads, sets)]
    torch.cuda.synchronize()

    def timed(step, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                step(i)
            ev[0].record(stream)
            for i in range(n):
                step(i)
            ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n

    def armed(call, n):
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in kev:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for i in range(n):
            sv.sv_time_next_stream_pass(*kev[i])
            call(i)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in kev) / n

    nsets = len(sets)
    t0 = time.perf_counter()
    fused_ms = timed(lambda i: fused[i % nsets](), args.steps)
    t_wall = time.perf_counter() - t0
    unfused_ms = timed(lambda i: (heads[i % nsets](), verifies[i % nsets]()), args.steps)
    verify_ms = timed(lambda i: verifies[i % nsets](), args.steps)
    gemm_stats_ms = armed(lambda i: fused[i % nsets](), args.steps)
    gemm_plain_ms = armed(lambda i: heads[i % nsets](), args.steps)
    # the library GEMM beside it: torch's bf16 linear layer (hipBLASLt) on the same operands
    lib_ms = timed(lambda i: torch.nn.functional.linear(sets[i % nsets]["hidden"].reshape(M, H),
                                                        sets[i % nsets]["weight"]), args.steps)
    flags = sum(int(c.out["err_flags"].item()) for c in fused + verifies)
    assert flags == 0, f"device error flags {flags}"

    flops = 2.0 * M * H * V
    gemm_bytes = V * H * 2 + M * H * 2 + M * V * 2  # weights and hidden states once, logits written
    tflops = flops / (gemm_stats_ms * 1e-3) / 1e12
    elems = B * (2 * K + 1) * V
    return {
        "metric": f"lm-head verify throughput: rows·vocab/s, B={B} K={K} V={V} H={H} bf16",
        "value": elems / (fused_ms * 1e-3),
        "unit": "rows·vocab/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fused_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x bf16 -> f32 (GEMM), f32 (verification)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "K": K, "V": V, "H": H, "logits": "bf16",
                   "temperature": cfg.temperature, "input_sets_rotated": nsets},
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": 2500.0,
            "unit": "TFLOP/s",
            "frac": tflops / 2500.0,
            "traffic": counted_traffic(args.workload, "lmhead"),
            "kernel": "lm_head_gemm_kernel<true> (the LM head with the statistics epilogue)",
            "algorithmic_flops_per_launch": flops,
            "duration_us_avg": gemm_stats_ms * 1e3,
            "hbm": {"algorithmic_bytes_per_launch": gemm_bytes,
                    "achieved_gbs": gemm_bytes / (gemm_stats_ms * 1e-3) / 1e9, "peak_gbs": HBM_PEAK_GBS,
                    "frac": gemm_bytes / (gemm_stats_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "timing": "launch start/stop events of the GEMM over a separate pass of the same steps",
        },
        "fused_call_us": fused_ms * 1e3,
        "unfused_call_us": unfused_ms * 1e3,
        "lm_head_alone_us": gemm_plain_ms * 1e3,
        "lm_head_with_statistics_us": gemm_stats_ms * 1e3,
        "torch_linear_bf16_us": lib_ms * 1e3,
        "verify_after_fused_gemm_us": (fused_ms - gemm_stats_ms) * 1e3,
        "sv_verify_chain_on_the_logits_us": verify_ms * 1e3,
        "wall_s_timed": t_wall,
        "_cpu_inp": sets[0],
    }


def small_batch_latencies(sv, torch, cfg, dev, stream, batches=(1, 4, 16), n=200) -> dict:
    """Per-call time of the same chain recipe at the pages' batch sizes (one
    to sixteen sequences), three rotating input sets, n calls back to back
    between two events; with the form each call takes (sv_chain_form)."""
    from workloads import chain_inputs
    out = {}
    for B in batches:
        c = cfg.with_(B=B, variant=cfg.variant + 300 + B)
        sets = [chain_inputs(c.with_(variant=c.variant + 10 * i), device=dev) for i in range(N_SETS)]
        calls = [sv.PreparedChainCall(s["target"], s["draft"], s["draft_tokens"], s["temperature"], s["uniforms"],
                                      stream=stream) for s in sets]
        for i in range(20):
            calls[i % N_SETS]()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            calls[i % N_SETS]()
        b.record(stream)
        torch.cuda.synchronize()
        assert sum(int(x.out["err_flags"].item()) for x in calls) == 0
        out[f"B={B}"] = {"call_us": a.elapsed_time(b) / n * 1e3,
                         "form": {1: "small", 2: "one launch", 3: "two launches"}[
                             sv.sv_chain_form(B, c.K, c.V, sets[0]["target"].dtype)],
                         "K": c.K, "V": c.V, "logits": c.dtype}
    return out


def main():
    args = parse()
    if args.oracle_worker:  # a child of the multi-core oracle figure: CPU only
        oracle_worker(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); specverify runs on one GPU and has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import rejection_sampling_verification_sv_amd as sv
    from workloads import (CHAIN_CONFIGS, SAMPLE_TREE_CONFIGS, TREE_CONFIGS, chain_inputs, chain_uniforms,
                           sample_inputs, sample_tree_inputs, tree_inputs)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sv.library()
    dev = torch.device("cuda:0")
    # a captured graph needs a capture stream other than the default one
    stream = torch.cuda.Stream(dev) if args.graph else torch.cuda.current_stream(dev)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = args.workload
    from workloads import LM_HEAD_CONFIGS
    if wl in LM_HEAD_CONFIGS:
        cfg = LM_HEAD_CONFIGS[wl]
        result = bench_lm_head(args, sv, torch, cfg, dev, stream)
        cpu_inp = result.pop("_cpu_inp")
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline_lm_head({k: v.cpu() for k, v in cpu_inp.items()}, cfg,
                                                          args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return
    kind = ("tree" if wl in TREE_CONFIGS else "treesample" if wl in SAMPLE_TREE_CONFIGS
            else "sample" if wl in SAMPLE_WORKLOADS else "chain")
    if kind == "treesample":
        cfg = SAMPLE_TREE_CONFIGS[wl]
        B, N, V = cfg.B, cfg.N, cfg.V
        rows = cfg.rows  # target and draft rows
        eb = 2 if cfg.dtype == "bf16" else 4
        sets = [sample_tree_inputs(cfg.with_(variant=cfg.variant + 10 * i) if i else cfg, device=dev)
                for i in range(N_SETS)]
        calls = [sv.PreparedTreeSamplingCall(s["target"], s["draft"], s["node_tokens"], s["parents"],
                                             s["temperature"], s["uniforms"], stream=stream) for s in sets]
        stream_bytes = rows * V * eb
        # plus tokens, parents, uniforms and temperatures (the walk's re-reads of
        # the rows it visits are not counted)
        call_bytes = stream_bytes + B * N * 4 + N * 4 + B * (N + 1) * 4 + B * 4
        config = {"workload": cfg.name + ("_graph" if args.graph else ""), "B": B, "N": N, "V": V,
                  "logits": cfg.dtype, "temperature": cfg.temperature, "branching": list(cfg.branching),
                  "input_sets_rotated": len(sets)}
        kernel_name = "tree_stats_kernel (one pass over every target and draft row: a record per row chunk)"
    elif kind == "sample":
        cfg = CHAIN_CONFIGS[SAMPLE_WORKLOADS[wl]]
        R, V = cfg.B * cfg.K, cfg.V
        rows = R
        eb = 2 if cfg.dtype == "bf16" else 4
        sets = [sample_inputs(cfg.with_(variant=cfg.variant + 10 * i) if i else cfg, device=dev)
                for i in range(N_SETS)]
        calls = [sv.PreparedSampleCall(s["logits"], s["temperature"], s["uniforms"], stream=stream) for s in sets]
        stream_bytes = R * V * eb
        call_bytes = stream_bytes + R * 4 * 4  # plus temperature, uniform, token and probability per row
        config = {"workload": f"sample_r{R}_v{V}_{cfg.dtype}" + ("_graph" if args.graph else ""), "rows": R, "V": V,
                  "logits": cfg.dtype,
                  "from": cfg.name, "input_sets_rotated": len(sets)}
        kernel_name = ("sample_stream_kernel (one pass over the rows: a record per 256-vector segment; the draw "
                       "is a second launch)")
    elif kind == "chain":
        cfg = CHAIN_CONFIGS[wl]
        B, K, V = cfg.B, cfg.K, cfg.V
        rows = B * (2 * K + 1)
        eb = 2 if cfg.dtype == "bf16" else 4
        sets = []
        if cfg.iterations > 1:  # one set of logits, fresh uniforms per iteration
            base = chain_inputs(cfg, device=dev)
            for it in range(cfg.iterations):
                s = dict(base)
                s["uniforms"] = chain_uniforms(cfg, iteration=it, device=dev)
                sets.append(s)
        else:
            for i in range(N_SETS):
                sets.append(chain_inputs(cfg.with_(variant=cfg.variant + 10 * i) if i else cfg, device=dev))
        calls = [sv.PreparedChainCall(s["target"], s["draft"], s["draft_tokens"], s["temperature"], s["uniforms"],
                                      stream=stream, want_entropy=args.entropy) for s in sets]
        # every logit once, plus tokens (gathered by the stream), uniforms and temperatures
        stream_bytes = rows * V * eb + B * K * 4
        call_bytes = stream_bytes + B * (K + 1) * 4 + B * 4
        config = {"workload": cfg.name + ("_entropy" if args.entropy else "") + ("_graph" if args.graph else ""),
                  "B": B, "K": K, "V": V,
                  "logits": cfg.dtype,
                  "temperature": cfg.temperature if cfg.temperature is not None else list(cfg.temperature_range),
                  "input_sets_rotated": len(sets)}
        if args.entropy:
            config["entropy"] = "every position, [B, 2K+1]"
        form = sv.sv_chain_form(B, K, V, sets[0]["target"].dtype, True, args.entropy)
        config["launches_per_call"] = 2 if form == 3 else 1
        kernel_name = ("chain_small_kernel (the whole call in one launch, the statistics workgroups deciding and "
                       "drawing: every logit row once, then the row pair at each sequence's first rejection)"
                       if form == 1 else
                       ("chain_one_launch_entropy_kernel" if args.entropy else "chain_one_launch_kernel") +
                       " (the whole call in one launch: every logit row once, then the "
                       "row pair at each sequence's first rejection)" if form == 2 else
                       "chain_stats_chunk_entropy_kernel (statistics pass with the entropy: every logit row once)"
                       if args.entropy else "chain_stats_chunk_kernel (statistics pass: every logit row once)")
    else:
        cfg = TREE_CONFIGS[wl]
        B, N, V = cfg.B, cfg.N, cfg.V
        rows = B * (N + 1)
        eb = 2 if cfg.dtype == "bf16" else 4
        sets = [tree_inputs(cfg.with_(variant=cfg.variant + 10 * i) if i else cfg, device=dev)
                for i in range(N_SETS)]
        calls = [sv.PreparedTreeCall(s["target"], s["node_tokens"], s["parents"], stream=stream) for s in sets]
        stream_bytes = rows * V * eb
        call_bytes = stream_bytes + B * N * 4 + N * 4
        config = {"workload": cfg.name + ("_graph" if args.graph else ""), "B": B, "N": N, "V": V, "logits": cfg.dtype,
                  "branching": list(cfg.branching), "input_sets_rotated": len(sets)}
        kernel_name = "tree_argmax_kernel (argmax pass with the path decision of the last workgroup)"
    elems = rows * V
    torch.cuda.synchronize()
    nsets = len(calls)
    steps = calls
    if args.graph:
        graphs = []
        for c in calls:
            c()  # one call on the capture stream before capturing
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                c()
            graphs.append(g)
        steps = [g.replay for g in graphs]
        torch.cuda.synchronize()

    with torch.cuda.stream(stream):  # graph replays go to the current stream
        for i in range(args.warmup):
            steps[i % nsets]()
    torch.cuda.synchronize()

    # Timed region: K steps back to back on the library's stream, between one
    # start and one stop event.
    e_start, e_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e_start.record(stream)
        for i in range(args.steps):
            steps[i % nsets]()
        e_stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    total_ms = e_start.elapsed_time(e_stop)
    ms_per_step = total_ms / args.steps

    # Per-call times: the same K steps again with an event after every call
    # (the events add a little to each call, so they are kept out of the
    # timed region).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for i in range(args.steps):
            steps[i % nsets]()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_call_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))

    # Kernel region: the same K steps again, each call's streaming kernel
    # launched with a start / stop event pair (its own dispatch timestamps).
    # Kept apart from the timed region: an armed launch delays the next kernel
    # by a few microseconds.
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in kev:  # create the events on the device before arming them
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        sv.sv_time_next_stream_pass(*kev[i])
        calls[i % nsets]()
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in kev]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    kern_sorted = sorted(kern_ms)

    # warm reference: the same input set every call (the last-level cache may serve it)
    for _ in range(5):
        calls[0]()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    nw = 50
    for _ in range(nw):
        calls[0]()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / nw
    flags = sum(int(c.out["err_flags"].item()) for c in calls)
    assert flags == 0, f"device error flags {flags}"

    achieved = stream_bytes / (kern_avg_ms * 1e-3) / 1e9
    traffic = counted_traffic(wl + ("_entropy" if args.entropy else ""), kind)
    result = {
        "metric": (METRIC if wl == "c2" and not args.entropy and not args.graph else
                   f"sampling throughput: rows·vocab/s + HBM GB/s vs peak, {config['workload']}" if kind == "sample"
                   else f"tree sampling verify throughput: rows·vocab/s + HBM GB/s vs peak, {config['workload']}"
                   if kind == "treesample"
                   else f"verify throughput: rows·vocab/s + HBM GB/s vs peak, {config['workload']}"),
        "value": elems / (ms_per_step * 1e-3),
        "unit": "rows·vocab/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": kernel_name,
            "algorithmic_bytes_per_launch": stream_bytes,
            "duration_us_avg": kern_avg_ms * 1e3,
            "duration_us_median": kern_sorted[len(kern_sorted) // 2] * 1e3,
            "timing": "launch start/stop events of the streaming kernel over a second pass of the same steps",
        },
        "call_us_median": per_call_ms[len(per_call_ms) // 2] * 1e3,
        "call_hbm_gbs": call_bytes / (ms_per_step * 1e-3) / 1e9,
        "call_frac_of_peak": call_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "warm_same_inputs_us": warm_ms * 1e3,
        "wall_s_timed": t_wall,
    }
    if kind == "chain" and wl == "c2" and not args.entropy and not args.graph:
        result["small_batch"] = small_batch_latencies(sv, torch, cfg, dev, stream)
    if not args.no_cpu_baseline:
        cpu_inp = {k: v.cpu() for k, v in sets[0].items()}
        if kind == "chain":
            result["cpu_baseline"] = cpu_baseline_chain(cpu_inp, cfg, args.cpu_seconds)
            if args.cpu_procs > 0:
                result["cpu_baseline_multicore"] = cpu_baseline_chain_procs(wl, cfg, args.cpu_seconds,
                                                                            args.cpu_procs)
        elif kind == "sample":
            result["cpu_baseline"] = cpu_baseline_sample(cpu_inp, cfg, args.cpu_seconds)
        elif kind == "treesample":
            result["cpu_baseline"] = cpu_baseline_tree_sampling(cpu_inp, cfg, args.cpu_seconds)
        else:
            result["cpu_baseline"] = cpu_baseline_tree(cpu_inp, cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
