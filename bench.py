"""Benchmark of the DSA layer (lightning indexer + Top-K + sparse MLA) on one GPU.

A step is one pass of the layer over one batch of synthetic input resident in
HBM: one dsa_layer call (fused indexer/Top-K/merge, which plans a call of up
to 64 queries itself, else after a planning kernel; sparse MLA split +
combine) for decode, one per chunk for chunked prefill.  The default workload
is 64 decoding sequences with cached lengths uniform in [65536, 131072], an FP8
e4m3 index-K cache (per-token fp32 scale, 64 heads x 128), Top-2048, and a bf16
576-wide latent cache read by 128-head sparse MLA.

Prints one JSON line.  `value` is query tokens per second of the whole layer;
`roofline` reports the dominant kernel, the indexer (planning + indexer
kernels), timed with HIP events on its launch stream inside a layer-shaped
sequence (indexer, then attention, per step): its algorithmic HBM bytes per
launch over that duration (or, where the indexer's algorithmic flops per byte
exceed the MFMA ridge, as in chunked prefill, its FP8 / bf16 MFMA flops
against the dense MFMA peak), plus `layer_frac_hbm`, the whole step's
algorithmic bytes (indexer + Top-K + sparse MLA) over its time against 8 TB/s;
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload.  Before the W warm-up steps, untimed steps run for at least
--settle-ms of wall time (`settle_steps` in the line), so the K timed steps
start from the GPU's steady state under the layer's load, not from idle.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# dense MFMA peaks of the chip (TFLOP/s): FP8 for an FP8 / MXFP8 index, bf16 otherwise
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "mxfp8": 5000.0, "bf16": 2500.0}
METRIC = "DSA decode tokens/s + % HBM roofline (indexer+top-k+sparse MLA, 128K ctx)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps for at least this long before the warm-up steps, so the timed steps "
                         "start from the GPU's steady state under this load rather than from idle")
    ap.add_argument("--workload", default="decode_b64_128k_fp8")
    ap.add_argument("--op", choices=("layer", "quantize"), default="layer",
                    help="layer: the DSA layer step (default); quantize: the index-query quantization that "
                         "prepares the workload's q_idx from its bf16 projection")
    ap.add_argument("--epilogue", action="store_true",
                    help="layer: fuse residual + RMSNorm (synthetic bf16 residual and norm weight) into the "
                         "attention's tail; the step then also writes the new residual stream")
    ap.add_argument("--quant-dtype", choices=("fp8", "mxfp8"), default=None,
                    help="--op quantize: the code format (default: the workload's index dtype)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-bandwidth", action="store_true",
                    help="skip the plain device copy whose rate is reported as context")
    ap.add_argument("--cpu-sample", type=int, default=48, help="queries the CPU oracle is timed on")
    ap.add_argument("--copies", type=int, default=2,
                    help="input copies the steps rotate through, so no step re-reads the previous step's "
                         "data from the 256 MB last-level cache")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the benchmark, run a plain 1 GiB device copy three times (the reference kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


# sources each measured call depends on: a stored counter measurement is
# reported only while these are unchanged
KERNEL_SOURCES = {
    "indexer": ["api.hip", "indexer.hip", "dsa_device.h", "dsa_params.h"],
    "quantize": ["api.hip", "quant.hip"],
}


def source_digest(kind="indexer"):
    """sha256 over the kernel and ABI sources of one measured call."""
    import hashlib
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "sparse_attention_07_amd", "csrc", f) for f in KERNEL_SOURCES[kind]]
    files.append(os.path.join(ROOT, "include", "dsa.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(name, kind="indexer"):
    """HBM bytes per call from the counter runs recorded under profiles/
    (profiles/<name>.json), or None when absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_sha256") != source_digest(kind):
        return None
    return rec.get("traffic_bytes_per_call")


def copy_calibration(dev):
    """A plain 1 GiB device copy, three times: the reference kernel that scales
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 3}), flush=True)


def algorithmic_bytes(case, indices, epilogue=False):
    """Bytes the method itself must move per step: the index-K cache once per
    sequence (codes + scales), the tables, each query's indexer query, weights
    and index row, the gathered latent rows (the union over a sequence's
    queries), each query's MLA q and output."""
    import torch
    s = case.spec
    lens = case.seq_lens.tolist()
    # bytes per key: codes + scale (fp32 per token, or one E8M0 byte per 32 elements)
    scale_b = {"fp8": 4, "mxfp8": s.D_idx // 32}.get(s.idx_dtype, 0)
    per_key = s.D_idx + scale_b if scale_b else 2 * s.D_idx
    idx_bytes = sum(per_key * L for L in lens)
    idx_bytes += 4 * sum((L + 63) // 64 for L in lens) + 4 * len(lens)
    T = case.T
    qi = s.H_idx * per_key
    idx_bytes += T * (qi + 4 * s.H_idx + 4 * s.K)
    rows = 0
    seqs = case.q_seq.tolist()
    for b in sorted(set(seqs)):
        sel = indices[torch.tensor([t for t in range(T) if seqs[t] == b])]
        rows += int(torch.unique(sel[sel >= 0]).numel())
    row_b = 656 if s.kv_dtype == "fp8" else 1152  # FP8 latent: 512 codes + 4 fp32 scales + 64 bf16 rope
    mla_bytes = rows * row_b + T * (s.H * 576 * 2 + s.H * 512 * 2 + 4 * s.K)
    if epilogue:  # residual read, new residual written, norm weight read
        mla_bytes += T * s.H * 512 * 2 * 2 + s.H * 512 * 2
    return idx_bytes, idx_bytes + mla_bytes


def algorithmic_flops(case, indices):
    """Multiply-adds (x2) the method itself must do per step: the indexer's
    H_i x D_i dot product for every visible key of every query, and the sparse
    MLA's logits (576 dims) and PV (512 dims) over every selected row and head."""
    s = case.spec
    lens = case.seq_lens.tolist()
    seqs = case.q_seq.tolist()
    maxlen = case.block_table.shape[1] * 64
    if case.q_visible is not None:
        vis = [min(max(v, 0), min(lens[b], maxlen)) for v, b in zip(case.q_visible.tolist(), seqs)]
    else:
        vis = [min(lens[b], maxlen) for b in seqs]
    idx_flops = 2 * s.H_idx * s.D_idx * sum(vis)
    rows = int((indices >= 0).sum().item())
    mla_flops = 2 * s.H * (576 + 512) * rows
    return idx_flops, mla_flops


def cpu_baseline(case, n_sample):
    """Time the oracle (numpy fp64, full sort, dense softmax) on the first
    n_sample queries of the workload, on this host's cores."""
    import numpy as np
    import torch
    from oracle import dsa_oracle as O
    from sparse_attention_07_amd import synth

    def bits16(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    s = case.spec
    secs, keys = 0.0, 0
    qs = list(range(min(n_sample, case.T)))
    for t in qs:
        b = int(case.q_seq[t])
        L = int(case.seq_lens[b])
        nblk = (L + 63) // 64
        pages = case.block_table[b, :nblk].long()
        kp = case.k_idx_pool[pages]
        d = dict(T=1, B=1, H_idx=s.H_idx, D_idx=s.D_idx, idx_dtype=s.idx_dtype, K=s.K, H=s.H, scale=s.scale,
                 num_blocks=nblk, seq_lens=np.array([L], np.int32),
                 block_table=np.arange(nblk, dtype=np.int32)[None], q_seq=np.array([0], np.int32),
                 q_visible=np.array([int(case.q_visible[t])], np.int32), w=case.w[t:t + 1].cpu().numpy(),
                 q=bits16(case.q[t:t + 1]),
                 kv_pool=(case.kv_pool.view(-1, 64, synth.KV_FP8_ROW)[pages].reshape(-1, synth.KV_FP8_ROW).cpu().numpy()
                          if s.kv_dtype == "fp8" else bits16(case.kv_pool.view(-1, 64, 576)[pages].reshape(-1, 576))),
                 kv_dtype=s.kv_dtype,
                 k_idx_pool=kp.cpu().numpy() if s.idx_dtype != "bf16" else bits16(kp))
        if s.idx_dtype != "bf16":
            d["q_idx"], d["q_idx_scale"] = case.q_idx[t:t + 1].cpu().numpy(), case.q_idx_scale[t:t + 1].cpu().numpy()
        else:
            d["q_idx"], d["q_idx_scale"] = bits16(case.q_idx[t:t + 1]), None
        t0 = time.perf_counter()
        O.layer_query(d, 0)
        secs += time.perf_counter() - t0
        keys += int(case.q_visible[t])
    return dict(value=len(qs) / secs, unit="tokens/s", cores=len(os.sched_getaffinity(0)), kind="oracle",
                sample=f"{len(qs)} of {case.T} queries of {s.name} ({keys} visible keys in total), "
                       f"numpy fp64, {secs:.1f} s",
                omp_num_threads=os.environ.get("OMP_NUM_THREADS"))


def quant_cpu_baseline(src, kind, label):
    """Time the oracle's quantizer (numpy) on the whole query of the workload."""
    from oracle import dsa_oracle as O
    x = src.cpu().float().numpy()
    rows = x.size // x.shape[-1]
    t0 = time.perf_counter()
    if kind == "fp8":
        O.quantize_fp8_per_row(x)
    else:
        O.quantize_mxfp8(x)
    secs = time.perf_counter() - t0
    return dict(value=round(rows / secs, 1), unit="rows/s", cores=len(os.sched_getaffinity(0)), kind="oracle",
                sample=f"all {rows} rows of {label}'s index query ({x.shape[-1]} wide), numpy, {secs:.2f} s")


def bench_quantize(args, spec, case):
    """Index-query quantization: bf16 q_idx [T, H_idx, D_idx] -> e4m3fn codes +
    scales, rotating through enough input/output copies that no launch reads
    the previous launch's data from the last-level cache."""
    import torch
    from sparse_attention_07_amd import dsa
    kind = args.quant_dtype or (spec.idx_dtype if spec.idx_dtype != "bf16" else "fp8")
    dt = dsa.IDX_FP8_E4M3FN if kind == "fp8" else dsa.IDX_MXFP8_E4M3
    src = case.q_idx_src
    D = src.shape[-1]
    rows = src.numel() // D
    scale_b = 4 if kind == "fp8" else D // 32
    per_call = rows * (D * 2 + D + scale_b)
    ncopy = max(2, min(16, -(-(512 << 20) // per_call)))
    ins = [src.clone() for _ in range(ncopy)]
    outs = [dsa.quantize_index_q(x, dt) for x in ins]
    stream = torch.cuda.current_stream()
    n_settle = settle(lambda i: dsa.quantize_index_q(ins[i % ncopy], dt, codes=outs[i % ncopy][0],
                                                     scales=outs[i % ncopy][1]), args.settle_ms)
    for i in range(args.warmup):
        dsa.quantize_index_q(ins[i % ncopy], dt, codes=outs[i % ncopy][0], scales=outs[i % ncopy][1])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        dsa.quantize_index_q(ins[i % ncopy], dt, codes=outs[i % ncopy][0], scales=outs[i % ncopy][1])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = e0.elapsed_time(e1) / args.steps
    achieved = per_call / (launch_ms * 1e-3) / 1e9
    line = {
        "metric": "index-Q quantization rows/s + % HBM roofline",
        "value": round(rows * args.steps / wall, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"bf16->{kind}",
        "data": "synthetic",
        "config": {"workload": f"{spec.name} index query", "rows": rows, "row_width": D,
                   "codes": kind, "input_copies_rotated": ncopy, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": stored_traffic(f"quantize_traffic_{spec.name}_{kind}", "quantize"),
            "kernel": "quantize_q_kernel", "launch_ms": round(launch_ms, 5), "algorithmic_bytes": per_call,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = quant_cpu_baseline(src, kind, spec.name)
    print(json.dumps(line), flush=True)


def settle(run, ms):
    """Run ``run(i)`` untimed, four calls per synchronisation, for at least
    ``ms`` milliseconds of wall time; returns the number of calls.  From idle,
    the first few milliseconds of steps run slower (the 128K decode step: 0.270
    ms per step over 20 steps after 5 warm-up steps, 0.254 ms after 100), so
    the timed steps start from the steady state a serving loop runs in."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            run(n)
            n += 1
        torch.cuda.synchronize()
    return n


def copy_bandwidth(dev, nbytes=2 << 30, reps=5):
    """Context, not a denominator: a plain device-to-device copy's rate (GB/s,
    read + write bytes over time)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbps, 1)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the layer has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_attention_07_amd import dsa, synth

    spec = synth.PRESETS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    # A step is one pass of the whole layer over one batch: one dsa_layer call
    # for decode; for chunked prefill, one call per chunk (all chunks of the
    # sequence, in order).
    if spec.prefill is not None:
        n_chunks = -(-spec.prefill[0] // spec.prefill[1])
        step_cases = [[synth.build_case(spec, device=dev, prefill_chunk=c) for c in range(n_chunks)]]
    else:
        step_cases = [[synth.build_case(spec, device=dev)]]
    case = step_cases[0][-1]
    ep_kw = {}
    if args.epilogue:
        g = torch.Generator(device=dev).manual_seed(spec.seed + 7)
        T_max = max(c.T for c in step_cases[0])
        res = torch.randn(T_max, spec.H, 512, generator=g, device=dev).to(torch.bfloat16)
        gam = (1.0 + 0.1 * torch.randn(spec.H * 512, generator=g, device=dev)).to(torch.bfloat16)
        ep_kw = dict(residual=res, norm_weight=gam, residual_out=torch.empty_like(res), eps=1e-6)
    if args.op == "quantize":
        bench_quantize(args, spec, case)
        if args.copy_calibration:
            copy_calibration(dev)
        return
    if spec.prefill is None:
        # copies of the caches the steps rotate through
        for _ in range(max(0, args.copies - 1)):
            c2 = synth.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
            c2.k_idx_pool = case.k_idx_pool.clone()
            c2.kv_pool = case.kv_pool.clone()
            step_cases.append([c2])

    def ep_for(c):
        if not ep_kw:
            return {}
        return dict(residual=ep_kw["residual"][: c.T], norm_weight=ep_kw["norm_weight"],
                    residual_out=ep_kw["residual_out"][: c.T], eps=ep_kw["eps"])

    layers = [[dsa.layer_from_case(c, **ep_for(c)) for c in cs] for cs in step_cases]
    torch.cuda.synchronize()

    def step(i):
        for lay in layers[i % len(layers)]:
            lay()

    n_settle = settle(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall / args.steps * 1e3
    tokens_per_step = sum(c.T for c in step_cases[0])
    value = tokens_per_step * args.steps / wall

    # The same kernels in the same order, one C call per step part, with HIP
    # events on the launch stream around each: the indexer (planning +
    # indexer/Top-K/merge kernels) and the sparse MLA (split + combine) as they
    # run inside the layer step.
    stream = torch.cuda.current_stream()
    splits = []
    for cs, lays in zip(step_cases, layers):
        parts = []
        for c, lay in zip(cs, lays):
            idx_out = torch.empty(c.T, spec.K, dtype=torch.int32, device=dev)
            ws = dsa.workspace_init(torch.empty(max(256, dsa.workspace_bytes(lay.idx, None, spec.K)),
                                                dtype=torch.uint8, device=dev))
            mws = dsa.workspace_init(torch.empty(max(256, dsa.workspace_bytes(None, lay.mla, spec.K)),
                                                 dtype=torch.uint8, device=dev))
            out = torch.empty_like(lay.out)
            parts.append((c, idx_out, ws, mws, out))
        splits.append(parts)

    def run_split(i, ev=None):
        for j, (c, idx_out, ws, mws, out) in enumerate(splits[i % len(splits)]):
            if ev is not None:
                ev[j][0].record(stream)
            dsa.indexer_topk(c.q_idx, c.w, c.k_idx_pool, c.block_table, c.seq_lens, spec.K,
                             q_idx_scale=c.q_idx_scale, q_seq=c.q_seq, q_visible=c.q_visible,
                             max_q_per_seq=c.max_q_per_seq, out=idx_out, workspace=ws)
            if ev is not None:
                ev[j][1].record(stream)
            dsa.sparse_mla_attn(c.q, c.kv_pool, idx_out, spec.scale, out=out, workspace=mws, **ep_for(c))
            if ev is not None:
                ev[j][2].record(stream)

    for i in range(args.warmup):
        run_split(i)
    n_split = max(20, args.steps)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in step_cases[0]] for _ in range(n_split)]
    for i in range(n_split):
        run_split(i, evs[i])
    torch.cuda.synchronize()
    idx_ms = sum(e[0].elapsed_time(e[1]) for ev in evs for e in ev) / n_split
    mla_ms = sum(e[1].elapsed_time(e[2]) for ev in evs for e in ev) / n_split

    # the indexer alone, back to back (context: no attention kernels between)
    def run_indexer(i):
        for c, idx_out, ws, _, _ in splits[i % len(splits)]:
            dsa.indexer_topk(c.q_idx, c.w, c.k_idx_pool, c.block_table, c.seq_lens, spec.K,
                             q_idx_scale=c.q_idx_scale, q_seq=c.q_seq, q_visible=c.q_visible,
                             max_q_per_seq=c.max_q_per_seq, out=idx_out, workspace=ws)

    for i in range(args.warmup):
        run_indexer(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n_split):
        run_indexer(i)
    e1.record(stream)
    torch.cuda.synchronize()
    idx_b2b_ms = e0.elapsed_time(e1) / n_split

    idx_bytes = layer_bytes = idx_flops = mla_flops = 0
    for c, lay in zip(step_cases[0], layers[0]):
        ib, lb = algorithmic_bytes(c, lay.indices, args.epilogue)
        fi, fm = algorithmic_flops(c, lay.indices)
        idx_bytes, layer_bytes, idx_flops, mla_flops = idx_bytes + ib, layer_bytes + lb, idx_flops + fi, mla_flops + fm
    achieved = idx_bytes / (idx_ms * 1e-3) / 1e9
    layer_frac = layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS
    planning = "in-kernel planning" if step_cases[0][0].T <= 64 else "planning kernel"
    kernel = (f"dsa_indexer_topk: {planning} + dsa_indexer_kernel (Top-K and list merge), timed inside the layer "
              "step" + (f" (all {len(step_cases[0])} chunk calls of a step)" if len(step_cases[0]) > 1 else ""))
    # the indexer's bound: MFMA when its flops per algorithmic byte exceed the
    # chip's ridge (prefill: each key serves thousands of queries), else HBM
    mfma_peak = MFMA_PEAK_TFLOPS[spec.idx_dtype]
    if idx_flops / idx_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBPS * 1e9):
        tflops = idx_flops / (idx_ms * 1e-3) / 1e12
        roofline = {
            "bound": "mfma", "achieved": round(tflops, 1), "peak": mfma_peak, "unit": "TFLOP/s",
            "frac": round(tflops / mfma_peak, 4), "traffic": stored_traffic(f"indexer_traffic_{spec.name}"),
            "kernel": kernel, "launch_ms": round(idx_ms, 5), "algorithmic_flops": idx_flops,
            "algorithmic_bytes": idx_bytes, "dtype": "fp8" if spec.idx_dtype != "bf16" else "bf16",
            "back_to_back_ms": round(idx_b2b_ms, 5),
        }
    else:
        roofline = {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(f"indexer_traffic_{spec.name}"),
            "kernel": kernel, "launch_ms": round(idx_ms, 5), "algorithmic_bytes": idx_bytes,
            "back_to_back_ms": round(idx_b2b_ms, 5),
            "back_to_back_frac": round(idx_bytes / (idx_b2b_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        }
    # the metric's own scope (indexer + Top-K + sparse MLA): the whole step
    roofline["layer_frac_hbm"] = round(layer_frac, 4)
    cfg = {
        "workload": spec.name, "queries": tokens_per_step, "sequences": case.B,
        "context_tokens_total": int(case.seq_lens.sum()), "index": f"{spec.idx_dtype} {spec.H_idx}x{spec.D_idx}",
        "top_k": spec.K, "mla_heads": spec.H, "latent_dim": 576, "latent_cache": spec.kv_dtype,
        "page_tokens": 64, "calls_per_step": len(step_cases[0]),
        "input_copies_rotated": len(step_cases), "parallelism": "single GPU",
        "epilogue": "residual + RMSNorm" if args.epilogue else None,
    }
    if spec.prefill is None and case.B > 1:
        lens = case.seq_lens.tolist()
        cfg["longest_over_mean_context"] = round(max(lens) / (sum(lens) / len(lens)), 3)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": n_settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if spec.idx_dtype == "bf16" else f"{spec.idx_dtype}+bf16")
                 + ("+fp8kv" if spec.kv_dtype == "fp8" else ""),
        "data": "synthetic",
        "config": cfg,
        "roofline": roofline,
        "layer": {
            "algorithmic_bytes": layer_bytes, "GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(layer_frac, 4),
            "algorithmic_flops": idx_flops + mla_flops,
            "TFLOPs": round((idx_flops + mla_flops) / (ms * 1e-3) / 1e12, 1),
            "mla_flops_bf16": mla_flops,
            "indexer_ms_in_step": round(idx_ms, 5), "mla_ms_in_step": round(mla_ms, 5),
        },
    }
    if not args.no_copy_bandwidth:
        line["context"] = {"device_copy_GBps": copy_bandwidth(dev)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_sample)
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        copy_calibration(dev)


if __name__ == "__main__":
    main()
