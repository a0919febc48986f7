"""Benchmark: one MLA decode step (query absorption, split-KV latent attention,
combine + W_UV projection) at H=64, B=32, L=4096 on one MI355X.

Prints one JSON line.  `value` is the step's algorithmic HBM traffic divided
by its time (TB/s); `ms_per_step` gives the step time.  Inputs are synthetic
(seeded, shapes and distributions of the workload) and resident in HBM; the
timed steps rotate over several independently drawn input sets whose total
size exceeds the 256 MB Infinity Cache, so repeats are served from HBM.

Timing: after --warmup untimed steps, exactly --steps steps (rotating over
the input sets) are captured in one HIP graph; the graph is replayed
--repeats times, each replay bracketed by HIP events on the launching
stream, and the median replay (with p10 and p90) divided by --steps is the
step time.  Unless --repeats is given, the replay count is chosen so that
about 6000 steps are timed (at least 20 replays).  The same steps issued
eagerly from Python are timed the same way and reported beside it.  The
split-KV attention kernel alone is timed the same way for the roofline
entry.  The oracle is timed on the host cores on a bounded sample of the
same workload.
"""
import argparse
import hashlib
import json
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
    """FLOPs of one prefill call (T new tokens per sequence, causal) in both
    attention forms: on the latent rows (absorbed) and through per-head keys
    and values rebuilt for the context (T tokens per sequence here)."""
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
    recon = 2 * n * H * R * (Dn + Dv)
    attn_heads = 2 * H * (Dn + Dr + Dv) * pairs
    return dict(latent_flops=proj + absorb + attn + out, latent_attn_flops=attn,
                per_head_flops=proj + recon + attn_heads, per_head_attn_flops=attn_heads)


def stats(per_step_ms):
    a = np.asarray(per_step_ms, np.float64)
    return dict(median=float(np.median(a)), p10=float(np.percentile(a, 10)),
                p90=float(np.percentile(a, 90)), mean=float(a.mean()))


def capture(torch, fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    g.replay()                   # first replay uploads the graph
    torch.cuda.synchronize()
    return g


def time_replays(torch, run, repeats):
    """ms of each of `repeats` calls of run(), each bracketed by HIP events on
    the current stream (the one graph replays and library calls launch on)."""
    cur = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(repeats)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(cur)
        run()
        b.record(cur)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


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
    form = m.mla_prefill_attention_form(mc, T, 0)

    def call():
        m.mla_prefill(mc, inp["x"], inp["weights"], inp["pool"], inp["block_table"],
                      inp["start_pos"], 0, rope_table=rope, out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    g = capture(torch, call, torch.cuda.Stream())
    st = stats(time_replays(torch, g.replay, args.steps))
    ms = st["median"]
    alg = prefill_algorithmic(cfg)
    executed = alg["per_head_flops"] if form == "per_head" else alg["latent_flops"]
    tflops = executed / (ms * 1e-3) / 1e12
    line = {
        "metric": "MLA prefill with cache append: ms per call; TFLOP/s of the FLOPs the "
                  "call executes",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_p10": round(st["p10"], 4), "ms_p90": round(st["p90"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_len": T, "d_model": cfg["d_model"],
                   "q_lora_rank": cfg.get("q_lora_rank", 0), "heads": cfg["num_heads"],
                   "attention_form": form, "executed_flops": executed,
                   "latent_form_flops": alg["latent_flops"],
                   "per_head_form_flops": alg["per_head_flops"],
                   "cache": "fp8 e4m3 rows, 656 B/token" if cfg.get("cache_dtype") == "fp8"
                            else "bf16 rows, 1152 B/token",
                   "timing": f"one call per graph replay, {args.steps} replays, median "
                             "(events on the launching stream)"},
        "roofline": {"kernel": f"mla_prefill (whole call, {form} attention)",
                     "bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_call": executed},
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
    g = capture(torch, call, torch.cuda.Stream())
    st = stats(time_replays(torch, g.replay, args.steps))
    ms = st["median"]
    flops = 2 * n * M * HV * (2 if cfg["gated"] else 1)
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "MLA output gate + W_O: TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_p10": round(st["p10"], 4), "ms_p90": round(st["p90"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": n, "d_model": M, "heads": cfg["num_heads"],
                   "v_dim": cfg["v_dim"], "gated": cfg["gated"], "flops": flops,
                   "timing": f"one call per graph replay, {args.steps} replays, median "
                             "(events on the launching stream)"},
        "roofline": {"kernel": "mla_output_gate_projection (gate GEMM + W_O GEMM)",
                     "bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_call": flops},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, seconds):
    """Time the oracle's decode as it stands on whole steps of the same
    workload: the absorbed path in float32 (the fastest faithful CPU form),
    the absorbed path in float64 (the parity reference) and the naive
    reconstruction path in float32 on a few sequences (scaled to a step).
    BLAS threads = the cores this process may run on.  `value` is the float32
    absorbed rate in the metric's unit (TB/s of algorithmic step bytes)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    inp = workloads.decode_inputs(cfg)
    alg = algorithmic(cfg, inp.seq_lens)
    B = len(inp.seq_lens)

    def timed(fn, budget, max_reps=50):
        times = []
        t_start = time.perf_counter()
        while len(times) < max_reps:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget:
                break
        return float(np.median(times)), len(times)

    def inputs(wd):
        return [workloads.to_f64(a).astype(wd)
                for a in (inp.q_nope, inp.q_rope, inp.w_uk, inp.w_uv, inp.pool)]

    paths = {}
    with threadpool_limits(limits=cores):
        for wd, name in ((np.float32, "absorbed_f32"), (np.float64, "absorbed_f64")):
            args = inputs(wd)
            t, n = timed(lambda: oracle.decode(*args, inp.block_table, inp.seq_lens, cfg,
                                               wd=wd), seconds * 0.4)
            paths[name] = {"ms_per_step": round(t * 1e3, 2), "steps_timed": n}
            del args
        args = inputs(np.float32)
        ids = [0, B // 2, B - 1]
        per_seq = [timed(lambda: oracle.decode(*args, inp.block_table, inp.seq_lens, cfg,
                                               path="naive", wd=np.float32, batch_ids=[b]),
                         0.0, max_reps=1)[0] for b in ids]
        paths["naive_f32"] = {"ms_per_step": round(float(np.mean(per_seq)) * B * 1e3, 2),
                              "sequences_timed": ids}
        pools = threadpool_info()
    blas = ",".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools
                            if p.get("user_api") == "blas"})) or "unknown"
    t = paths["absorbed_f32"]["ms_per_step"] * 1e-3
    return {"value": alg["step_bytes"] / t / 1e12, "unit": "TB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"decode steps of {B}x{cfg['context']} tokens: absorbed path in "
                      f"float32 numpy ({paths['absorbed_f32']['steps_timed']} whole steps, "
                      f"median; this is value), in float64 "
                      f"({paths['absorbed_f64']['steps_timed']} steps), naive "
                      f"reconstruction path in float32 on sequences {ids} scaled to the "
                      f"batch; CPU {cpu_model()}, BLAS {blas}, {cores} threads",
            "ms_per_step": paths["absorbed_f32"]["ms_per_step"], "paths": paths}


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


def narrow_roofline(alg, attn_ms):
    """Narrow latents (kv_lora_rank 128 / 256): the attention and merge
    kernels move (R + Dr) 2 bytes and do 2 H (2R + Dr) flops per token; both
    rooflines are given, `bound` names the nearer one."""
    tf = alg["attn_flops"] / (attn_ms * 1e-3) / 1e12
    gbs = alg["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    hbm_frac, mfma_frac = gbs / HBM_PEAK_GBS, tf / BF16_PEAK_TFLOPS
    if hbm_frac >= mfma_frac:
        entry = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(hbm_frac, 4)}
    else:
        entry = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(mfma_frac, 4)}
    return {"kernel": "narrow-latent attention + merge", **entry, "traffic": None,
            "kernel_us": round(attn_ms * 1e3, 3), "hbm_frac": round(hbm_frac, 4),
            "mfma_frac": round(mfma_frac, 4),
            "algorithmic_flops_per_launch": alg["attn_flops"],
            "algorithmic_bytes_per_launch": alg["attn_bytes"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--repeats", type=int, default=0,
                    help="graph replays of --steps steps each; the median is reported "
                         "(default: enough replays for about 6000 timed steps, at least 20)")
    ap.add_argument("--workload", default=workloads.HEADLINE,
                    choices=[k for k, v in workloads.WORKLOADS.items() if v["dtype"] == "bf16"])
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the device's HBM read, bf16 MFMA and LDS read ceilings with the "
                         "library's probes (include/mla.h) and print them")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MB (10 times), as the "
                         "known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.repeats < 0:
        print("--steps must be positive and --repeats not negative", file=sys.stderr)
        sys.exit(2)
    if args.repeats == 0:
        # Replays of a few steps last about a millisecond each, where clock and
        # power management move single replays by 10 % and more: time enough of
        # them that the median rests on several thousand steps.
        args.repeats = max(20, -(-6000 // args.steps))

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
    if args.ceilings:
        return ceilings_main(args, torch, m)
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
    R = len(sets)
    K = args.steps

    def step(i):
        s = sets[i % R]
        m.mla_decode(mc, s["q_nope"], s["q_rope"], s["w_uk"], s["w_uv"], s["pool"],
                     s["block_table"], s["seq_lens"], max_len, out=out, workspace=ws[i % R])

    narrow = cfg["kv_lora_rank"] != 512   # the narrow-latent kernels (attention + merge)

    def attn(i):
        s = sets[i % R]
        if narrow:
            m.mla_latent_attention(mc, qf[i % R], s["pool"], s["block_table"], s["seq_lens"],
                                   max_len, workspace=ws[i % R])
            return
        m.mla_attention_partials(mc, qf[i % R], s["pool"], s["block_table"], s["seq_lens"],
                                 max_len, ws[i % R])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def steps_eager():
        for i in range(K):
            step(i)

    eager = stats([t / K for t in time_replays(torch, steps_eager, args.repeats)])
    side = torch.cuda.Stream()
    g_step = capture(torch, steps_eager, side)
    graph = stats([t / K for t in time_replays(torch, g_step.replay, args.repeats)])
    g_attn = capture(torch, lambda: [attn(i) for i in range(K)], side)
    attn_st = stats([t / K for t in time_replays(torch, g_attn.replay, args.repeats)])
    step_ms, attn_ms = graph["median"], attn_st["median"]

    peak_bytes = torch.cuda.max_memory_allocated(dev)
    value = alg["step_bytes"] / (step_ms * 1e-3) / 1e12
    achieved = alg["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "us_per_step": round(step_ms * 1e3, 3),
        "us_per_step_p10": round(graph["p10"] * 1e3, 3),
        "us_per_step_p90": round(graph["p90"] * 1e3, 3),
        "tflops": round(alg["step_flops"] / (step_ms * 1e-3) / 1e12, 2),
        "cached_tokens_per_s": round(alg["tokens"] / (step_ms * 1e-3), 1),
        "eager_us_per_step": round(eager["median"] * 1e3, 3),
        "eager_us_per_step_p10": round(eager["p10"] * 1e3, 3),
        "eager_us_per_step_p90": round(eager["p90"] * 1e3, 3),
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
                   "timing": f"{K} steps per hip graph replay, {args.repeats} replays, median "
                             "per step (events on the launching stream)"},
        "roofline": narrow_roofline(alg, attn_ms) if narrow else {
            "kernel": "attn_decode_partials_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_entry(args.workload),
            "kernel_us": round(attn_ms * 1e3, 3),
            "kernel_us_p10": round(attn_st["p10"] * 1e3, 3),
            "kernel_us_p90": round(attn_st["p90"] * 1e3, 3),
            "algorithmic_bytes_per_launch": alg["attn_bytes"],
            "mfma_tflops": round(alg["attn_flops"] / (attn_ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(alg["attn_flops"] / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        },
    }
    if cfg.get("kv_groups"):
        line["forms"] = mechanism_forms(args, torch, m, cfg, mc, sets, max_len, step_ms, alg)
    if not args.no_cpu_baseline and args.workload == workloads.HEADLINE:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def ceilings_main(args, torch, m):
    """The ceilings the kernels are measured against, on this device: HBM
    reads of a 2 GiB buffer (8x the 256 MB Infinity Cache) through 16-byte
    vector loads and through direct-to-LDS loads of 36 KB pieces (the decode
    attention's way), back-to-back bf16 32x32x16 MFMAs, and conflict-free
    LDS reads of 16 and 8 bytes per lane on every CU.  Median of
    --repeats launches each, HIP events on the launching stream."""
    dev = torch.device("cuda", 0)
    buf = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    sink = m.mla_probe_sink(dev)
    st = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.repeats):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            fn()
            b.record(st)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return stats(ts)

    nbytes = buf.numel()
    dma_bytes = (nbytes // 36864) * 36864
    vec = timed(lambda: m.mla_probe_hbm_read(buf, 0, sink))
    dma = timed(lambda: m.mla_probe_hbm_read(buf, 1, sink))
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs, iters = 4 * cus, 4000
    flops = wgs * 4 * iters * 4 * 32768
    mf = timed(lambda: m.mla_probe_mfma(wgs, iters, sink))
    lds_iters = 20000
    lds_bytes = {w: cus * 8 * lds_iters * 8 * 64 * w for w in (16, 8)}
    lds = {w: timed(lambda w=w: m.mla_probe_lds_read(w, lds_iters, sink)) for w in (16, 8)}
    gbs = lambda b, t: b / (t * 1e-3) / 1e9
    line = {
        "metric": "device ceilings: HBM read GB/s, bf16 MFMA TFLOP/s, LDS read GB/s per CU",
        "hbm_read_vector_GBs": round(gbs(nbytes, vec["median"]), 1),
        "hbm_read_direct_to_lds_GBs": round(gbs(dma_bytes, dma["median"]), 1),
        "hbm_peak_GBs": HBM_PEAK_GBS,
        "mfma_bf16_TFLOPs": round(flops / (mf["median"] * 1e-3) / 1e12, 1),
        "mfma_bf16_peak_TFLOPs": BF16_PEAK_TFLOPS,
        "buffer_bytes": nbytes, "repeats": args.repeats,
        "lds_read_b128_GBs_per_cu": round(gbs(lds_bytes[16], lds[16]["median"]) / cus, 1),
        "lds_read_b64_GBs_per_cu": round(gbs(lds_bytes[8], lds[8]["median"]) / cus, 1),
        "mfma_workgroups": wgs, "mfma_iterations": iters, "compute_units": cus,
        "lds_iterations": lds_iters,
        "ms": {"vector": round(vec["median"], 4), "direct_to_lds": round(dma["median"], 4),
               "mfma": round(mf["median"], 4), "lds_b128": round(lds[16]["median"], 4),
               "lds_b64": round(lds[8]["median"], 4)},
    }
    print(json.dumps(line), flush=True)


def mechanism_forms(args, torch, m, cfg, mc, sets, max_len, latent_ms, alg):
    """The tutorial's mechanism comparison (5.1, 5.4) between the two forms
    of the same decode step: attention on the latent rows (absorbed) and
    through per-head keys and values rebuilt from them for the step
    (reconstruction).  Per form: time per step (graph replay, median), the
    bytes of rebuilt keys and values, the workspace the form needs (the
    library allocates nothing else) and the peak memory torch saw while one
    step ran; the outputs' cosine against each other (the cosine of each
    against the oracle is printed by the parity tests)."""
    import dataclasses
    dev = torch.device("cuda", 0)
    B, H = len(sets[0]["seq_lens"]), cfg["num_heads"]
    G = cfg.get("kv_groups") or H
    tokens = alg["tokens"]
    rec = {}
    outs = {}
    for form in ("latent", "per_head"):
        fc = dataclasses.replace(mc, decode_attention=form)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        wsb = m.mla_decode_workspace_size(fc, B, max_len)
        ws = [torch.zeros(wsb, dtype=torch.uint8, device=dev)]
        out = torch.empty((B, H, cfg["v_dim"]), dtype=torch.bfloat16, device=dev)

        def step(i, fc=fc, ws=ws, out=out):
            s = sets[i % len(sets)]
            m.mla_decode(fc, s["q_nope"], s["q_rope"], s["w_uk"], s["w_uv"], s["pool"],
                         s["block_table"], s["seq_lens"], max_len, out=out,
                         workspace=ws[i % len(sets)])

        step(0)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base   # one step: workspace + output
        outs[form] = out.float().clone()
        ws += [torch.zeros(wsb, dtype=torch.uint8, device=dev) for _ in sets[1:]]
        if form == "latent":
            ms = latent_ms
        else:
            for i in range(args.warmup):
                step(i)
            g = capture(torch, lambda: [step(i) for i in range(args.steps)], torch.cuda.Stream())
            ms = stats([t / args.steps for t in time_replays(torch, g.replay, args.repeats)])["median"]
        rebuilt = 0 if form == "latent" else \
            tokens * G * (cfg["qk_nope_dim"] + cfg["rope_dim"] + cfg["v_dim"]) * 2
        rec[form] = {"us_per_step": round(ms * 1e3, 3), "rebuilt_kv_bytes": rebuilt,
                     "workspace_bytes": wsb, "peak_extra_bytes": int(peak),
                     "cache_bytes": alg["attn_bytes"]}
        del ws
    a, b = outs["latent"].flatten(), outs["per_head"].flatten()
    rec["cosine_between_forms"] = round(float(torch.dot(a, b) / (a.norm() * b.norm())), 7)
    rec["max_abs_between_forms"] = round(float((a - b).abs().max()), 6)
    return rec


if __name__ == "__main__":
    main()
