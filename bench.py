"""Throughput of the MI355X ALBERT phoneme encoder (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one albert_encode call: the whole encoder forward pass (embedding,
projection, 12 shared-layer executions, output projection) over one batch
of synthetic phoneme IDs already resident in HBM.  Prints one JSON line.

Besides the headline tokens/s the line carries
  roofline      the dominant kernel's algorithmic FLOP per launch divided by
                its average launch time, measured with HIP events on the
                library's stream during the timed steps, against MI355X's
                dense bf16 MFMA peak;
  cpu_baseline  the float64 oracle timed on this host's cores over a
                bounded sample of the same sequences (also a parity check of
                those sequences).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "encoded phoneme tokens/sec at B=256,T=128 bf16; % of MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (vendor figure)
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (vendor figure)
PEAKS = {"bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_TFLOPS, "fp8": PEAK_FP8_TFLOPS}
H, E, F, O, NITER = 768, 128, 2048, 512, 12


def seq_flops(L: np.ndarray) -> float:
    """Algorithmic FLOP of one encoder pass over sequences of lengths L."""
    L = np.asarray(L, np.float64)
    return float(np.sum(133_103_616.0 * L + 36_864.0 * L * L))


def kernel_flops(kind: str, lengths: np.ndarray) -> float:
    """Algorithmic FLOP of ONE launch of a kernel kind (valid tokens only)."""
    M = float(np.sum(lengths))
    L = np.asarray(lengths, np.float64)
    return {
        "embed": 0.0,
        "proj": 2 * M * E * H,
        "qkv": 2 * M * H * 3 * H,
        "attn": float(np.sum(4.0 * H * L * L)),
        "attn_out_ln": 2 * M * H * H,
        "ffn1_gelu": 2 * M * H * F,
        "ffn2_ln": 2 * M * F * H,
        "out": 2 * M * H * O,
        "qkv_attn": 2 * M * H * 3 * H + float(np.sum(4.0 * H * L * L)),
    }[kind]


def source_hash() -> str:
    d = os.path.join(ROOT, "albert_transformer_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_for(kind: str, config: int):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernels changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    rec = t.get("kernels", {}).get(kind)
    if not rec or t.get("source_sha") != source_hash() or t.get("config") != config:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def host_cpu() -> dict:
    """The host the oracle runs on: CPU model and logical CPU count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count()}


def cpu_baseline(wl, got, budget_s: float, cfg=synth.KOKORO, weights=None, dtype=None):
    """Time the float64 oracle on this host over whole sequences of the same
    workload until `budget_s` seconds have passed; compare the GPU rows."""
    import oracle
    from threadpoolctl import threadpool_info
    dtype = wl.dtype if dtype is None else dtype
    W = oracle.prepare_weights(synth.make_weights() if weights is None else weights, dtype)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    order = np.random.default_rng(7).permutation(wl.n_seq)
    tokens, done, max_abs, min_cos = 0, 0, 0.0, 1.0
    t0 = time.perf_counter()
    for s in order:
        L = int(wl.lengths[s])
        if wl.packed:
            a = int(wl.cu_seqlens[s])
            ids, rows = wl.ids[a:a + L], got[a:a + L]
        else:
            ids, rows = wl.ids[s, :L], got[s, :L]
        if dtype == "fp8":  # the variant's own definition (its storage roundings)
            ref = oracle.encode_fp8_features(oracle.embed_ln(ids, W, cfg), W, cfg)
        else:
            ref = oracle.encode_sequence(ids, W, cfg)
        tokens += L
        done += 1
        d = rows.astype(np.float64) - ref
        max_abs = max(max_abs, float(np.abs(d).max()))
        cos = (rows * ref).sum(-1) / (np.linalg.norm(rows, axis=-1) * np.linalg.norm(ref, axis=-1))
        min_cos = min(min_cos, float(cos.min()))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    base = {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {wl.n_seq} sequences ({tokens} tokens), float64 NumPy/BLAS, "
                      f"{dt:.1f} s", **host_cpu()}
    parity = {"sequences": done, "max_abs": max_abs, "min_token_cosine": min_cos}
    return base, parity


def measure_length_regulation(steps: int = 20) -> dict:
    """Duration rule + frame expansion on the packed-workload shape (63k
    tokens x 512 fp32, durations from 8 synthetic logit channels).  HBM
    bound: bytes = token rows read once + frame rows written."""
    import torch
    import albert_transformer_amd as A
    wl = synth.make_workload(5)
    rng = np.random.default_rng(55)
    feat = torch.from_numpy(rng.normal(0, 0.5, (wl.tokens, O)).astype(np.float32)).cuda()
    logits = torch.from_numpy(rng.normal(0.4, 1.0, (wl.tokens, 8)).astype(np.float32)).cuda()
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    dur = A.durations(logits, 1.0)
    frames = int(dur.sum().item())
    out = torch.empty((frames, O), dtype=torch.float32, device="cuda")
    cuf = torch.empty(wl.n_seq + 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(A.expand_workspace_bytes(wl.tokens), dtype=torch.uint8, device="cuda")
    assert A.expand_raw(feat, dur, cu, frames, out, cuf, ws) == A.OK
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        A.expand_raw(feat, dur, cu, frames, out, cuf, ws, flags=A.ASYNC)
    e1.record()
    torch.cuda.synchronize()
    assert A.read_status(ws) == A.OK
    ms = e0.elapsed_time(e1) / steps
    nbytes = wl.tokens * O * 4 + frames * O * 4 + wl.tokens * 4 * 3
    return {"workload": f"{wl.n_seq} packed sequences, {wl.tokens} tokens x {O} fp32 -> "
                        f"{frames} frames", "ms_per_call": round(ms, 4),
            "frames_per_s": round(frames / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "peak": 8000.0, "unit": "GB/s",
                         "frac": round(nbytes / (ms * 1e-3) / 1e9 / 8000.0, 4)}}


def hailo_fidelity(enc, cfg, weights, n: int = 16) -> dict:
    """The Hailo card's fidelity method: n N(0,1) inputs [128,128] at the
    LayerNorm output, per-sample cosine and MSE of the flattened [128,512]
    output against full precision (the float64 oracle, unrounded weights)."""
    import torch
    import oracle
    W64 = oracle.prepare_weights(weights, "f32")
    x = np.random.default_rng(2024).normal(0, 1, (n * 128, 128))
    cu = torch.from_numpy(np.arange(0, (n + 1) * 128, 128, dtype=np.int32)).cuda()
    got = enc.encode_features(torch.from_numpy(x.astype(np.float32)).cuda(), cu, 128)
    got = got.cpu().numpy().astype(np.float64)
    cos, mse, lo, hi = [], [], [], []
    for s in range(n):
        sl = slice(128 * s, 128 * (s + 1))
        ref = oracle.encode_features(x[sl], W64, cfg)
        g = got[sl]
        cos.append(float((g * ref).sum() / np.linalg.norm(g) / np.linalg.norm(ref)))
        mse.append(float(np.mean((g - ref) ** 2)))
        lo.append(float(g.min()))
        hi.append(float(g.max()))
    return {"method": "16 N(0,1) [128,128] inputs at the LayerNorm output, per-sample cosine "
                      "of [128,512] vs float64", "cos_mean": round(float(np.mean(cos)), 5),
            "cos_min": round(min(cos), 5), "cos_max": round(max(cos), 5),
            "mse_mean": float(np.mean(mse)), "range": [round(min(lo), 3), round(max(hi), 3)]}


TEXT_METRIC = ("text-encoder tokens/sec at B=256,T=128 bf16 (Kokoro's parallel text path); "
               "% of MFMA roofline")


def text_kernel_flops(kind: str, tokens: int, tc) -> float:
    """Algorithmic FLOP of one launch of a text-path kernel kind."""
    C, K, H = tc.channels, tc.kernel, tc.hidden
    return {"conv": 2.0 * tokens * C * K * C, "lstm_in": 2.0 * tokens * C * 8 * H,
            "lstm": 2.0 * 2 * tokens * 4 * H * H}.get(kind, 0.0)


def bench_text(args) -> int:
    """The parallel text encoder on a workload's batch (one JSON line)."""
    import torch
    import albert_transformer_amd as A
    import oracle.text_encoder as te
    tc = synth.TEXT
    wl = synth.make_workload(args.config)
    weights = synth.make_text_weights(tc)
    enc = A.TextEncoder(weights)
    if wl.packed:
        raise SystemExit("the text bench takes a padded workload")
    ids = torch.from_numpy(wl.ids).cuda()
    lens = torch.from_numpy(wl.lengths).cuda()
    out = torch.empty((wl.n_seq, wl.T, 2 * tc.hidden), dtype=torch.float32, device="cuda")
    ws = enc.new_workspace(wl.n_seq, wl.n_seq * wl.T)

    def step():
        return enc.encode_raw(ids, lens, out, ws, flags=A.ASYNC)

    for _ in range(args.warmup):
        assert step() == A.OK
    torch.cuda.synchronize()
    if A.read_status(ws) != A.OK:
        raise SystemExit("text encoder rejected the workload")
    per_kind = {}
    for kind in A.TEXT_KERNEL_KINDS:
        enc.time_kernel(kind)
        for _ in range(3):
            step()
        n, ms = enc.kernel_time()
        per_kind[kind] = {"launches_per_step": n // 3, "ms_per_step": ms / 3,
                          "ms_per_launch": ms / max(n, 1)}
    enc.time_kernel(None)
    dominant = max(per_kind, key=lambda k: per_kind[k]["ms_per_step"])
    enc.time_kernel(dominant, max_launches=max(
        per_kind[dominant]["launches_per_step"] * args.steps * args.batches, 1))
    batch_s = []
    for _ in range(args.batches):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        batch_s.append(time.perf_counter() - t0)
    elapsed = float(np.median(batch_s))
    n_dom, ms_dom = enc.kernel_time()
    enc.time_kernel(None)
    if A.read_status(ws) != A.OK:
        raise SystemExit("text encoder failed during timing")
    tokens = wl.tokens
    launch_ms = ms_dom / max(n_dom, 1)
    achieved = text_kernel_flops(dominant, tokens, tc) / (launch_ms * 1e-3) / 1e12
    ms_step = 1e3 * elapsed / args.steps
    flops_step = sum(text_kernel_flops(k, tokens, tc) * v["launches_per_step"]
                     for k, v in per_kind.items())

    base = None
    if args.cpu_seconds > 0:
        from threadpoolctl import threadpool_info
        TW = te.prepare_text_weights(weights, tc, "bf16")
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
        got = out.cpu().numpy()
        done = tok = 0
        worst = 0.0
        t0 = time.perf_counter()
        for b in np.random.default_rng(7).permutation(wl.n_seq):
            L = int(wl.lengths[b])
            ref = te.text_encode_sequence(wl.ids[b, :L], TW, tc)
            worst = max(worst, float(np.abs(got[b, :L] - ref).max()))
            done += 1
            tok += L
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        base = {"value": tok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{done} of {wl.n_seq} sequences ({tok} tokens), float64 NumPy, "
                          f"{dt:.1f} s", "parity_max_abs": worst, **host_cpu()}
    line = {
        "metric": TEXT_METRIC, "value": round(tokens * args.steps / elapsed, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "batches": args.batches,
        "ms_per_step_batches": [round(1e3 * t / args.steps, 4) for t in batch_s],
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded text-encoder weights, uniform phoneme ids)",
        "config": {"workload": f"text encoder, {wl.name}", "sequences": wl.n_seq, "T": wl.T,
                   "tokens_per_step": tokens, "conv_blocks": tc.n_conv, "kernel": tc.kernel,
                   "lstm_units": tc.hidden},
        "tflops_end_to_end": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "ms_per_launch": round(launch_ms, 5), "launches_timed": n_dom},
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in per_kind.items()},
        "cpu_baseline": base, "source_sha": source_hash(),
    }
    print(json.dumps(line), flush=True)
    enc.close()
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = headline)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall budget of the oracle CPU baseline (0 = skip)")
    ap.add_argument("--dtype", choices=("bf16", "fp8", "f32"), default=None,
                    help="override the workload's compute type (fp8: E4M3 operands)")
    ap.add_argument("--model", choices=("albert", "text"), default="albert",
                    help="albert: the phoneme encoder (default); text: the parallel text path")
    ap.add_argument("--groups", type=int, default=1,
                    help="distinct layer weight sets (1 = Kokoro's full sharing)")
    ap.add_argument("--batches", type=int, default=5,
                    help="timed batches of --steps steps each; the median is reported")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step from a captured HIP graph (launch-bound small batches)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the encoder shards as independent data-parallel copies; nothing here "
              "uses a second GPU).", file=sys.stderr)
        return 2

    import torch
    import albert_transformer_amd as A

    torch.cuda.set_device(0)
    if args.model == "text":
        return bench_text(args)
    wl = synth.make_workload(args.config)
    dtype = wl.dtype if args.dtype is None else args.dtype
    cfg = synth.Config(n_groups=args.groups)
    weights = synth.make_weights(cfg)
    enc = A.Encoder(weights, dtype, n_groups=args.groups)
    ids = torch.from_numpy(wl.ids).cuda()
    if wl.packed:
        cu = torch.from_numpy(wl.cu_seqlens).cuda()
        out = torch.empty((wl.tokens, O), dtype=torch.float32, device="cuda")
        ws = enc.new_workspace(wl.n_seq, wl.tokens)

        def step():
            return enc.encode_varlen_raw(ids, cu, wl.T, out, ws, flags=A.ASYNC)
    else:
        lens = torch.from_numpy(wl.lengths).cuda()
        out = torch.empty((wl.n_seq, wl.T, O), dtype=torch.float32, device="cuda")
        ws = enc.new_workspace(wl.n_seq, wl.n_seq * wl.T)

        def step():
            return enc.encode_raw(ids, lens, out, ws, flags=A.ASYNC)

    if args.copy_probe_mib > 0:
        a = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        assert step() == A.OK
    torch.cuda.synchronize()
    st = A.read_status(ws)
    if st != A.OK:
        raise SystemExit(f"encoder rejected the workload: {A.STATUS_NAMES.get(st, st)}")

    # per-kind breakdown (3 steps each) to find the dominant kernel
    per_kind = {}
    for kind in A.KERNEL_KINDS:
        enc.time_kernel(kind)
        for _ in range(3):
            step()
        n, ms = enc.kernel_time()
        per_kind[kind] = {"launches_per_step": n // 3, "ms_per_step": ms / 3,
                          "ms_per_launch": ms / max(n, 1)}
    enc.time_kernel(None)
    dominant = max(per_kind, key=lambda k: per_kind[k]["ms_per_step"])

    # With --graph the step's whole launch sequence is captured once into a
    # HIP graph and replayed (small batches are bound by launch overhead).
    graph = None
    if args.graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                step()
        torch.cuda.synchronize()
        run_step = graph.replay
    else:
        run_step = step

    # timed region: `batches` batches of exactly K steps, each bracketed by a
    # synchronisation on both sides; the median batch is reported.  The
    # dominant kernel is bracketed by events in every batch (not in graph
    # mode, where the per-kind breakdown above stands).
    batch_s = []
    n_dom = ms_dom = 0
    if graph is None:
        launches = per_kind[dominant]["launches_per_step"] * args.steps * args.batches
        enc.time_kernel(dominant, max_launches=max(launches, 1))
    for _ in range(args.batches):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run_step()
        torch.cuda.synchronize()
        batch_s.append(time.perf_counter() - t0)
    if graph is None:
        n_dom, ms_dom = enc.kernel_time()
        enc.time_kernel(None)
    else:
        n_dom = per_kind[dominant]["launches_per_step"]
        ms_dom = per_kind[dominant]["ms_per_step"]
    st = A.read_status(ws)
    if st != A.OK:
        raise SystemExit(f"encoder failed during timing: {A.STATUS_NAMES.get(st, st)}")

    elapsed = float(np.median(batch_s))
    ms_step = 1e3 * elapsed / args.steps
    tokens = wl.tokens
    value = tokens * args.steps / elapsed
    flops_step = seq_flops(wl.lengths)
    peak = PEAKS[dtype]
    launch_ms = ms_dom / max(n_dom, 1)
    achieved = kernel_flops(dominant, wl.lengths) / (launch_ms * 1e-3) / 1e12

    got = out.cpu().numpy()
    base, parity = (cpu_baseline(wl, got, args.cpu_seconds, cfg, weights, dtype) if args.cpu_seconds > 0
                    else (None, None))
    length_reg = (measure_length_regulation() if args.config == 3 and args.groups == 1
                  and dtype == "bf16" else None)
    fidelity = hailo_fidelity(enc, cfg, weights) if dtype == "fp8" else None

    line = {
        "metric": METRIC if dtype == "bf16" else METRIC.replace(" bf16;", f" {dtype};"),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "batches": args.batches,
        "ms_per_step_batches": [round(1e3 * t / args.steps, 4) for t in batch_s],
        "graph": bool(args.graph),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,0.02) weights, uniform phoneme ids)",
        "config": {
            "workload": wl.name,
            "sequences": wl.n_seq,
            "T": wl.T,
            "packed": wl.packed,
            "tokens_per_step": tokens,
            "padded_slots_per_step": wl.rows,
            "shared_layer_executions": NITER,
            "layer_weight_sets": args.groups,
        },
        "tflops_end_to_end": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "mfma_frac_end_to_end": round(flops_step / (ms_step * 1e-3) / 1e12 / peak, 4),
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic_for(dominant, args.config) if args.groups == 1 else None,
            "ms_per_launch": round(launch_ms, 5),
            "launches_timed": n_dom,
        },
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4) for k, v in per_kind.items()},
        "cpu_baseline": base,
        "parity_sample": parity,
        "length_regulation": length_reg,
        "fp8_fidelity": fidelity,
        "source_sha": source_hash(),
    }
    print(json.dumps(line), flush=True)
    enc.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
