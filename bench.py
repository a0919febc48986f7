"""Benchmark: one MLA decode step (query absorption, split-KV latent attention,
combine + W_UV projection) at H=64, B=32, L=4096 on one MI355X.

Prints one JSON line.  `value` is the step's algorithmic HBM traffic divided
by its time (TB/s); `ms_per_step` gives the step time.  Inputs are synthetic
(seeded, shapes and distributions of the workload) and resident in HBM; the
timed steps rotate over several independently drawn input sets whose total
size exceeds the 256 MB Infinity Cache, so repeats are served from HBM.

Timing: the step's kernels are captured in a HIP graph whose one replay
launches --passes rotations (every input set several times, as a model's
layers follow one another in one graph), and HIP events on the launching
stream bracket the replays; the launch gap between replays is then spread
over many steps, as in a multi-layer graph.  The split-KV attention kernel
is timed the same way on its own for the roofline entry.  The oracle is timed on the host cores on a bounded
sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "MLA latent decode: µs/step, HBM TB/s, MFMA TFLOP/s at H=64 B=32 L=4096"
ATTN_SRC = os.path.join(ROOT, "mla_latent_kv_26_amd", "csrc", "attention_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attention_traffic.json")


def algorithmic(cfg, lens):
    """Bytes and FLOPs a decode step must move/do (cache rows once, weights
    once, queries in, outputs out) and the attention kernel's share."""
    H, R, Dr, Dn, Dv = (cfg[k] for k in ("num_heads", "kv_lora_rank", "rope_dim",
                                         "qk_nope_dim", "v_dim"))
    B = len(lens)
    tokens = int(np.sum(lens))
    # bf16 rows, or FP8 rows: R codes, Dr bf16 rope values, scale and padding
    row_bytes = R + 2 * Dr + 16 if cfg.get("cache_dtype") == "fp8" else (R + Dr) * 2
    cache = tokens * row_bytes
    weights = 2 * (cfg.get("kv_groups") or H) * R * (Dn + Dv)   # W_UK, W_UV (shared or per head)
    io = 2 * B * H * (Dn + Dr + Dv)
    flops_attn = 2 * H * (R + Dr + R) * tokens
    flops_proj = 2 * B * H * R * (Dn + Dv)
    return dict(step_bytes=cache + weights + io, attn_bytes=cache, tokens=tokens,
                step_flops=flops_attn + flops_proj, attn_flops=flops_attn)


def prefill_algorithmic(cfg):
    """FLOPs and bytes of one prefill call (T new tokens per sequence, causal,
    absorbed path): projections, cache append, attention on the latent rows,
    W_UV."""
    B, T, M, H = cfg["batch"], cfg["q_len"], cfg["d_model"], cfg["num_heads"]
    R, Dr, Dn, Dv = (cfg[k] for k in ("kv_lora_rank", "rope_dim", "qk_nope_dim", "v_dim"))
    Rq = cfg.get("q_lora_rank", 0)
    n = B * T
    qw = H * (Dn + Dr)
    proj = 2 * n * M * (R + Dr) + (2 * n * M * Rq + 2 * n * Rq * qw if Rq else 2 * n * M * qw)
    absorb = 2 * n * H * Dn * R
    pairs = B * T * (T + 1) // 2                        # causal (query, key) pairs
    attn = 2 * H * (R + Dr + R) * pairs
    out = 2 * n * H * R * Dv
    weights = 2 * (M * (R + Dr) + (M * Rq + Rq * qw if Rq else M * qw) + H * R * (Dn + Dv))
    bytes_ = 2 * n * M + weights + 2 * n * (R + Dr) + 2 * n * H * Dv
    # the same result through per-head keys and values (rebuilt for the
    # context, T tokens per sequence here): what the library executes for
    # long spans
    recon = 2 * n * H * R * (Dn + Dv)
    attn_heads = 2 * H * (Dn + Dr + Dv) * pairs
    return dict(flops=proj + absorb + attn + out, attn_flops=attn, bytes=bytes_,
                per_head_flops=proj + recon + attn_heads, per_head_attn_flops=attn_heads)


def prefill_main(args, torch, m):
    """Time mla_prefill on the prefill workload (MFMA-bound)."""
    dev = torch.device("cuda", 0)
    cfg = workloads.WORKLOADS[args.workload]
    mc = m.MLAConfig.from_dict(cfg)
    inp = workloads.prefill_inputs_torch(cfg, cfg["seed"], dev)
    B, T = cfg["batch"], cfg["q_len"]
    rope = m.mla_rope_table(mc, T).to(dev)
    ws = torch.zeros(m.mla_prefill_workspace_size(mc, B, T, T), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, cfg["num_heads"], cfg["v_dim"]), dtype=torch.bfloat16, device=dev)

    def call():
        m.mla_prefill(mc, inp["x"], inp["weights"], inp["pool"], inp["block_table"],
                      inp["start_pos"], 0, rope_table=rope, out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ms = graph_time(torch, call, args.steps, side)
    alg = prefill_algorithmic(cfg)
    tflops = alg["flops"] / (ms * 1e-3) / 1e12
    executed = alg["per_head_flops"] / (ms * 1e-3) / 1e12
    line = {
        "metric": "MLA prefill with cache append: ms per call; effective TFLOP/s over the "
                  "latent-path FLOP count",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_len": T, "d_model": cfg["d_model"],
                   "q_lora_rank": cfg.get("q_lora_rank", 0), "heads": cfg["num_heads"],
                   "algorithmic_flops": alg["flops"], "attention_flops": alg["attn_flops"],
                   "executed_flops_per_head_path": alg["per_head_flops"],
                   "cache": "fp8 e4m3 rows, 656 B/token" if cfg.get("cache_dtype") == "fp8"
                            else "bf16 rows, 1152 B/token",
                   "timing": "hip graph replay, events on the launching stream"},
        "roofline": {"kernel": "mla_prefill (whole call, per-head key/value path)",
                     "bound": "mfma", "achieved": round(executed, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(executed / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_call": alg["per_head_flops"]},
    }
    print(json.dumps(line), flush=True)


def output_gate_main(args, torch, m):
    """Time mla_output_gate_projection (gate GEMM with the sigmoid and the
    head outputs fused into its epilogue, then W_O; MFMA-bound)."""
    dev = torch.device("cuda", 0)
    cfg = workloads.WORKLOADS[args.workload]
    mc = m.MLAConfig.from_dict(cfg)
    inp = workloads.output_gate_inputs_torch(cfg, cfg["seed"], dev)
    n, M, HV = cfg["rows"], cfg["d_model"], cfg["num_heads"] * cfg["v_dim"]
    ws = torch.zeros(m.mla_output_gate_workspace_size(mc, n), dtype=torch.uint8, device=dev)
    out = torch.empty((n, M), dtype=torch.bfloat16, device=dev)

    def call():
        m.mla_output_gate_projection(mc, inp["x"], inp["head_out"], inp["w_o"],
                                     w_g=inp["w_g"] if cfg["gated"] else None, out=out,
                                     workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms = graph_time(torch, call, args.steps, torch.cuda.Stream())
    flops = 2 * n * M * HV * (2 if cfg["gated"] else 1)
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "MLA output gate + W_O: TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": n, "d_model": M, "heads": cfg["num_heads"],
                   "v_dim": cfg["v_dim"], "gated": cfg["gated"], "flops": flops,
                   "timing": "hip graph replay, events on the launching stream"},
        "roofline": {"kernel": "mla_output_gate_projection (gate GEMM + W_O GEMM)",
                     "bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_call": flops},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, seconds):
    """Time the oracle's decode (float64 numpy, as it stands) on whole steps of
    the same workload until about `seconds` of work; report TB/s of
    algorithmic bytes like the GPU line."""
    import oracle
    from threadpoolctl import threadpool_info
    inp = workloads.decode_inputs(cfg)
    args = [workloads.to_f64(a) for a in (inp.q_nope, inp.q_rope, inp.w_uk, inp.w_uv, inp.pool)]
    alg = algorithmic(cfg, inp.seq_lens)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.decode(*args, inp.block_table, inp.seq_lens, cfg)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > seconds:
            break
    t = float(np.median(times))
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])
    blas = ",".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools
                            if p.get("user_api") == "blas"})) or "unknown"
    return {"value": alg["step_bytes"] / t / 1e12, "unit": "TB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(times)} full decode steps of {cfg['batch']}x{cfg['context']} tokens, "
                      f"absorbed path in float64 numpy, median {t * 1e3:.1f} ms/step; "
                      f"CPU {cpu_model()}, BLAS {blas}",
            "ms_per_step": t * 1e3}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traffic_entry(workload):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on this workload and on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


VALU_PEAK_TFLOPS = 157.3      # fp32 vector ALU, 256 CUs at 2.4 GHz


def narrow_roofline(alg, attn_ms):
    """Narrow latents run on vector-ALU kernels: 2 H (2R + Dr) flops per
    token against (R + Dr) 2 bytes, beyond what the ALUs can do at the HBM
    rate, so the bound is the ALU peak."""
    tf = alg["attn_flops"] / (attn_ms * 1e-3) / 1e12
    return {"kernel": "attention_generic_kernel + merge_generic_kernel", "bound": "alu",
            "achieved": round(tf, 2), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / VALU_PEAK_TFLOPS, 4), "traffic": None,
            "kernel_us": round(attn_ms * 1e3, 3),
            "hbm_gbs": round(alg["attn_bytes"] / (attn_ms * 1e-3) / 1e9, 1),
            "algorithmic_flops_per_launch": alg["attn_flops"],
            "algorithmic_bytes_per_launch": alg["attn_bytes"]}


def graph_time(torch, fn, reps, stream):
    """Capture fn() once in a graph, replay `reps` times between two events."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    a.record(cur)
    for _ in range(reps):
        g.replay()
    b.record(cur)
    b.synchronize()
    return a.elapsed_time(b) / reps  # ms per replay


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=workloads.HEADLINE,
                    choices=[k for k, v in workloads.WORKLOADS.items() if v["dtype"] == "bf16"])
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--passes", type=int, default=10,
                    help="rotations over the input sets captured in one graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MB (10 times), as the "
                         "known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 10}))
        return
    import mla_latent_kv_26_amd as m
    if "q_len" in workloads.WORKLOADS[args.workload]:
        return prefill_main(args, torch, m)
    if "rows" in workloads.WORKLOADS[args.workload]:
        return output_gate_main(args, torch, m)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = workloads.WORKLOADS[args.workload]
    mc = m.MLAConfig.from_dict(cfg)
    lens0 = workloads.decode_lengths(cfg, np.random.Generator(np.random.PCG64(cfg["seed"])))
    sets = [workloads.decode_inputs_torch(cfg, cfg["seed"] + 1000 * i, dev, lengths=lens0)
            for i in range(args.rotate)]
    B, H = len(lens0), cfg["num_heads"]
    max_len = int(lens0.max())
    alg = algorithmic(cfg, lens0)
    ws = [torch.zeros(m.mla_decode_workspace_size(mc, B, max_len), dtype=torch.uint8, device=dev)
          for _ in sets]
    out = torch.empty((B, H, cfg["v_dim"]), dtype=torch.bfloat16, device=dev)
    qf = [m.mla_absorb_query(mc, s["q_nope"], s["q_rope"], s["w_uk"]) for s in sets]
    torch.cuda.synchronize()

    def step(i):
        s = sets[i]
        m.mla_decode(mc, s["q_nope"], s["q_rope"], s["w_uk"], s["w_uv"], s["pool"],
                     s["block_table"], s["seq_lens"], max_len, out=out, workspace=ws[i])

    narrow = cfg["kv_lora_rank"] != 512   # the narrow-latent kernels (attention + merge)

    def attn(i):
        s = sets[i]
        if narrow:
            m.mla_latent_attention(mc, qf[i], s["pool"], s["block_table"], s["seq_lens"], max_len,
                                   workspace=ws[i])
            return
        m.mla_attention_partials(mc, qf[i], s["pool"], s["block_table"], s["seq_lens"], max_len,
                                 ws[i])

    R = len(sets)
    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()

    # eager: python issues every call
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.steps):
        step(i % R)
    b.record()
    b.synchronize()
    eager_ms = a.elapsed_time(b) / args.steps

    # graph: one replay = `passes` rotations over the input sets
    side = torch.cuda.Stream()
    per = R * max(1, args.passes)
    reps = max(1, args.steps // per)
    step_ms = graph_time(torch, lambda: [step(i % R) for i in range(per)], reps, side) / per
    attn_ms = graph_time(torch, lambda: [attn(i % R) for i in range(per)], reps, side) / per
    steps_timed = reps * per

    peak_bytes = torch.cuda.max_memory_allocated(dev)
    value = alg["step_bytes"] / (step_ms * 1e-3) / 1e12
    achieved = alg["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "us_per_step": round(step_ms * 1e3, 3),
        "tflops": round(alg["step_flops"] / (step_ms * 1e-3) / 1e12, 2),
        "cached_tokens_per_s": round(alg["tokens"] / (step_ms * 1e-3), 1),
        "eager_us_per_step": round(eager_ms * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "context": max_len,
                   "cached_tokens": alg["tokens"], "heads": H,
                   "kv_lora_rank": cfg["kv_lora_rank"], "rope_dim": cfg["rope_dim"],
                   "qk_nope_dim": cfg["qk_nope_dim"], "v_dim": cfg["v_dim"],
                   "block_size": cfg["block_size"], "input_sets_rotated": R,
                   "kv_groups": cfg.get("kv_groups", 0),
                   # the tutorial's state ledger (5.4): cached bytes per token against
                   # multi-head K and V at the same head width
                   "state_bytes_per_token": alg["attn_bytes"] // max(1, alg["tokens"]),
                   "mha_state_bytes_per_token": 2 * H * cfg["qk_nope_dim"] * 2,
                   "peak_allocated_bytes": peak_bytes,
                   "cache": "fp8 e4m3 rows, 656 B/token" if cfg.get("cache_dtype") == "fp8"
                   else f"bf16 rows, {2 * (cfg['kv_lora_rank'] + cfg['rope_dim'])} B/token",
                   "timing": f"hip graph replay ({per} steps per replay), events on the launching stream"},
        "roofline": narrow_roofline(alg, attn_ms) if narrow else {
            "kernel": "attn_decode_partials_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_entry(args.workload),
            "kernel_us": round(attn_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": alg["attn_bytes"],
            "mfma_tflops": round(alg["attn_flops"] / (attn_ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(alg["attn_flops"] / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        },
    }
    if not args.no_cpu_baseline and args.workload == workloads.HEADLINE:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
