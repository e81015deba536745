#!/usr/bin/env python3
"""Benchmark of the MXFP4 routed-expert MoE layer on one MI355X.

One step is the whole layer -- moe_route, moe_dispatch, the three launches of
moe_expert_ffn and moe_combine -- over one batch of the workload's seeded
synthetic inputs, already resident in HBM.  The expert blob is held in four
copies at different addresses and the steps rotate through them, so the
256 MB last-level cache cannot serve one step's expert bytes to the next.

The default workload is the largest single-GPU configuration, the
16384-token prefill with Zipf-skewed routing (MFMA bound); the 64-token decode
batch (HBM bound) is timed in the same run and reported in a "decode"
sub-object, so both halves of the metric come from one invocation.

Prints ONE JSON line: tokens/s (whole job), the roofline of the dominant
kernel (the expert gate/up launch: MFMA for prefill, HBM for decode), timed
with HIP events on the library's stream, per-stage times, and the CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload prefill_t16384_zipf] [--decode-workload decode_t64]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published (the fp8 x fp4 scaled MFMA runs at this rate)
METRIC = "MoE-layer tokens/s at 1 GPU + achieved HBM GB/s (decode) / MFMA % (prefill)"
CSRC = os.path.join(ROOT, "mxfp4_routed_expert_moe_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="prefill_t16384_zipf")
    p.add_argument("--decode-workload", default="decode_t64",
                   help="second workload timed in the same run and reported as the decode sub-object ('none': skip)")
    p.add_argument("--copies", type=int, default=4, help="expert blob copies rotated across steps")
    p.add_argument("--cpu-sample-tokens", type=int, default=40,
                   help="tokens of the workload the CPU oracle runs on (about 10-15 s of work)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="skip timing the step replayed from a captured HIP graph (reported beside the plain step)")
    p.add_argument("--ffn-split-fp8", action="store_true",
                   help="prefill expert FFN on the scaled FP4 matrix cores (MOE_FFN_SPLIT_FP8)")
    p.add_argument("--shared-mxfp8", action="store_true", help="the shared expert in MXFP8 (MOE_SHARED_MXFP8)")
    p.add_argument("--routed-affine2", action="store_true",
                   help="the routed experts in the 2-bit affine codec (MOE_ROUTED_AFFINE2)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run one device copy of this size first (to scale HBM counters)")
    return p.parse_args()


KERNEL_HEADERS = ("ffn_internal.h", "moe_internal.h")  # included by every FFN kernel source


def _code_text(path: str) -> bytes:
    """A C++ source with its comments and whitespace removed (string literals
    in these files hold no comment markers)."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text).encode()


def source_hash(name: str) -> str:
    """Short hash of the code of a kernel source file (ffn_decode.hip,
    ffn_prefill.hip or ffn_prefill_f8.hip) followed by the headers it
    includes: a change to the code or to a shared device helper retires the
    counters taken before it, an edit of comments does not."""
    h = hashlib.sha256()
    for n in (name,) + KERNEL_HEADERS:
        h.update(_code_text(os.path.join(CSRC, n)))
    return h.hexdigest()[:16]


def read_traffic(workload: str, source: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when none exists or the kernel source changed since."""
    path = os.path.join(PROFILES, f"ffn_gateup_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source") != source or kv.get("source_sha256_16") != source_hash(source):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, n_tokens: int, shared_fmt: str = "mxfp4", routed_fmt: str = "mxfp4"):
    """The oracle as it stands, on the first n_tokens of the workload."""
    import numpy as np
    from oracle import moe_oracle as O
    from mxfp4_routed_expert_moe_amd import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        cores = 1
    host_cpus = os.cpu_count()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = host_cpus
    S = min(n_tokens, inp.x.shape[0])
    t0 = time.perf_counter()
    r = O.moe_layer(inp.x[:S], inp.experts, n_experts=inp.n_experts, hidden=inp.hidden, inter=inp.inter,
                    top_k=inp.top_k, route_scale=WL.ROUTE_SCALE, limit=WL.CLAMP_LIMIT, w_router=inp.router,
                    bias=inp.bias, token_ids=None if inp.tok is None else inp.tok[:S], table=inp.table,
                    shared_fmt=shared_fmt, routed_fmt=routed_fmt)
    dt = time.perf_counter() - t0
    n_exp = int(np.count_nonzero(np.diff(r["offsets"])))
    return dict(value=S / dt, unit="tokens/s", cores=int(cores), kind="oracle", host_cpus=host_cpus,
                affinity_cpus=affinity,
                sample=f"first {S} of {inp.x.shape[0]} tokens of {inp.workload.name}: full layer, "
                       f"{n_exp} experts decoded, {dt:.1f} s wall; float64 numpy on {cores} BLAS threads "
                       f"(host: {host_cpus} CPUs, {affinity} in this process's affinity mask)")


STAGES = ("route", "dispatch", "ffn_plan", "ffn_gateup", "ffn_down", "combine")


def measure(wl, args, B, WL, np, torch):
    """Time K steps of the whole layer on workload wl (after W warm-up steps)
    and return the figures of one JSON record (without the CPU baseline)."""
    print(f"[bench] workload {wl.name} T={wl.T}: generating inputs", file=sys.stderr, flush=True)
    shared_fmt = "mxfp8" if args.shared_mxfp8 else "mxfp4"
    if args.routed_affine2:
        canon = WL.make_experts_affine2(wl.seed, WL.N_EXPERTS, shared=shared_fmt)
    elif args.shared_mxfp8:
        canon = WL.make_experts_shared_mxfp8(wl.seed, WL.N_EXPERTS)
    else:
        canon = None
    inp = WL.make_layer_inputs(wl, experts=canon)
    del canon
    H, I, E, k, T = inp.hidden, inp.inter, inp.n_experts, inp.top_k, wl.T

    dev = torch.device("cuda", 0)
    if args.calib_copy_mib > 0:
        # an elementwise kernel that reads n bytes and writes n bytes
        n = (args.calib_copy_mib << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty(n, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b

    nb = E * (WL.affine2_expert_bytes(H, I) if args.routed_affine2 else WL.expert_bytes(H, I))
    routed = (B.pack_affine2(inp.experts[:nb], E, H, I) if args.routed_affine2
              else B.pack_mxfp4(inp.experts[:nb], E, H, I))
    shared = B.pack_mxfp8(inp.experts[nb:], H, I) if args.shared_mxfp8 else B.pack_mxfp4(inp.experts[nb:], 1, H, I)
    packed = np.concatenate([routed, shared])
    del routed, shared
    blob0 = torch.from_numpy(packed).to(dev)
    del packed
    blobs = [blob0] + [blob0.clone() for _ in range(args.copies - 1)]
    experts = [B.Experts(b, E, H, I, split_fp8=args.ffn_split_fp8, shared_mxfp8=args.shared_mxfp8,
                         routed_affine2=args.routed_affine2) for b in blobs]
    to_dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    layer = B.MoeLayer(experts[0], T, k, WL.ROUTE_SCALE, WL.CLAMP_LIMIT, w_router=to_dev(inp.router),
                       sel_bias=to_dev(inp.bias), hash_table=to_dev(inp.table))
    x = to_dev(inp.x.view(np.int16))
    tok = to_dev(inp.tok)
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    # events on the library's stream (torch's current stream, which the
    # binding passes to every call) between the launches of each stage
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(K)]

    def step(i, timed):
        e = ev[i] if timed else None
        layer.set_experts(experts[i % len(experts)])
        calls = (lambda: layer.route(x, tok), layer.dispatch, lambda: layer.expert_ffn_phase(x, 0),
                 lambda: layer.expert_ffn_phase(x, 1), lambda: layer.expert_ffn_phase(x, 2), layer.combine)
        if timed:
            e[0].record()
        for j, c in enumerate(calls):
            c()
            if timed:
                e[j + 1].record()

    print(f"[bench] {wl.name}: warmup {W} steps", file=sys.stderr, flush=True)
    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: timing {K} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(K):
        step(i, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / K
    value = T * K / elapsed
    stage_ms = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)]))
                for j, name in enumerate(STAGES)}
    gateup_ms = stage_ms["ffn_gateup"]

    # The same step captured once per blob copy into a HIP graph (the library
    # allocates nothing and issues no memsets, so the four calls capture as
    # they are) and replayed in rotation: the step without host launch cost.
    graph = None
    if not args.no_graph:
        graphs = []
        for c in range(len(experts)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c, False)
            graphs.append(g)
        for i in range(W):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for i in range(K):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - tg0) * 1e3 / K
        graph = dict(ms_per_step=round(gms, 4), value=round(T / (gms * 1e-3), 1))
        del graphs

    # algorithmic work of the gate/up launch, from this run's own ids
    ids = layer.ids.cpu().numpy()
    used = int(len(np.unique(ids[(ids >= 0) & (ids < E)]))) + 1   # + the shared expert
    rows = int(layer.offsets[-1].item())
    # expert bytes per projection: routed gate / up and down, and the shared expert's
    mx4_proj = H * I * 17 // 32
    if args.routed_affine2:
        gate_proj, down_proj = H * I * 5 // 16, H * I * 3 // 8    # 2 bits + bf16 (s, b) per 64 / per 32
    else:
        gate_proj = down_proj = mx4_proj
    shared_proj = H * I * 33 // 32 if args.shared_mxfp8 else mx4_proj
    gateup_bytes = (used - 1) * 2 * gate_proj + 2 * shared_proj + rows * H * 2 + rows * I * 2
    gateup_flops = rows * 2 * 2 * H * I
    layer_flops = rows * 2 * 3 * H * I
    decode = rows <= 16 * (E + 1)
    if decode:
        achieved = gateup_bytes / (gateup_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
        traffic = read_traffic(wl.name, "ffn_decode.hip")
    elif not args.ffn_split_fp8:
        achieved = gateup_flops / (gateup_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4))
        traffic = read_traffic(wl.name, "ffn_prefill.hip")
    else:
        # fp8 x fp4 scaled MFMA at its own (fp8) peak; each product is issued
        # twice (the hi and lo activation terms), and the timed launch pair
        # includes splitting x.
        achieved = gateup_flops / (gateup_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / FP8_MFMA_PEAK_TFLOPS, 4), issued_tflops=round(2 * achieved, 1))
        traffic = read_traffic(wl.name, "ffn_prefill_f8.hip")
    # the counter summaries were taken on the MXFP4 experts with an MXFP4 shared expert
    roof["traffic"] = None if (args.routed_affine2 or args.shared_mxfp8) else traffic
    roof["kernel"] = "ffn gate/up (moe_expert_ffn phase 1)"
    roof["avg_launch_us"] = round(gateup_ms * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = gateup_bytes
    roof["algorithmic_flops_per_launch"] = gateup_flops

    layer_bytes = (used - 1) * (2 * gate_proj + down_proj) + 3 * shared_proj
    rec = dict(value=round(value, 1), ms_per_step=round(ms_per_step, 4), T=T, H=H, I=I, E=E, k=k,
               used=used, rows=rows, layer_bytes=layer_bytes, roofline=roof, decode=decode,
               layer_hbm_gbs=round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1),
               layer_mfma_tflops=round(layer_flops / (ms_per_step * 1e-3) / 1e12, 1),
               stages_us={n: round(v * 1e3, 2) for n, v in stage_ms.items()}, graph=graph, inp=inp)
    del layer, experts, blobs, blob0, x, tok
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mxfp4_routed_expert_moe_amd import binding as B
    from mxfp4_routed_expert_moe_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fail loudly if the library is missing
    if args.ffn_split_fp8 and (args.shared_mxfp8 or args.routed_affine2):
        print("--ffn-split-fp8 combines with neither --shared-mxfp8 nor --routed-affine2", file=sys.stderr)
        sys.exit(2)
    shared_fmt = "mxfp8" if args.shared_mxfp8 else "mxfp4"
    routed_fmt = "affine2" if args.routed_affine2 else "mxfp4"
    by_name = {w.name: w for w in WL.WORKLOADS}
    wl = by_name[args.workload]
    r = measure(wl, args, B, WL, np, torch)
    inp = r.pop("inp")
    out = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8x2-fp4" if (args.ffn_split_fp8 and not r["decode"]) else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": r["T"], "hidden": r["H"], "inter": r["I"], "experts": r["E"],
                   "top_k": r["k"], "routing": wl.routing, "bias": wl.bias,
                   "weights": ("affine 2-bit, bf16 (s, b) per 64/64/32" if args.routed_affine2
                               else "mxfp4 e2m1+e8m0/32"),
                   "experts_read_per_step": r["used"], "expert_bytes_per_step": r["layer_bytes"],
                   "rows_per_step": r["rows"], "blob_copies_rotated": args.copies,
                   "ffn_prefill_arith": "split-fp8 scaled mfma" if args.ffn_split_fp8 else "bf16 mfma",
                   "shared_expert": shared_fmt},
        "roofline": r["roofline"],
        "layer_hbm_gbs": r["layer_hbm_gbs"],
        "layer_mfma_tflops": r["layer_mfma_tflops"],
        "layer_mfma_frac": round(r["layer_mfma_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
        "stages_us": r["stages_us"],
        "graph": r["graph"],
        "decode": None,
        "cpu_baseline": None,
    }
    if args.decode_workload != "none" and args.decode_workload != wl.name:
        d = measure(by_name[args.decode_workload], args, B, WL, np, torch)
        d.pop("inp")
        out["decode"] = {"workload": args.decode_workload, "tokens": d["T"], "value": d["value"],
                         "unit": "tokens/s", "ms_per_step": d["ms_per_step"], "roofline": d["roofline"],
                         "layer_hbm_gbs": d["layer_hbm_gbs"],
                         "layer_hbm_frac": round(d["layer_hbm_gbs"] / HBM_PEAK_GBS, 4),
                         "experts_read_per_step": d["used"], "expert_bytes_per_step": d["layer_bytes"],
                         "stages_us": d["stages_us"], "graph": d["graph"]}
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on {args.cpu_sample_tokens} tokens", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens, shared_fmt, routed_fmt)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
