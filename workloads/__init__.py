"""Seeded synthetic inputs for the MLA latent-KV workloads.

This module only draws random numbers, rounds them to the storage dtype and
builds index structures (sequence lengths, page tables).  It holds none of the
attention arithmetic, so both the CPU oracle and the HIP library can be fed
from it without sharing any method code.

Storage convention: float32 tensors are numpy float32 arrays; bf16 tensors are
numpy uint16 arrays holding the bf16 bit patterns (round-to-nearest-even from
the float32 draw).  ``to_f64`` turns either into exact float64 values.

Distributions follow the workload descriptions: hidden states, queries and
cache rows are N(0, 1); a weight matrix is N(0, 1/fan_in), with fan_in the
matrix's input width (d_model for the down projections and W_Q, q_lora_rank
for W_UQ, kv_lora_rank for W_UK and W_UV).  RMSNorm gains are 1 unless a test
asks for perturbed gains (so that a kernel ignoring the gain cannot pass).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# --------------------------------------------------------------------------
# Workload shapes.  Each entry is named for what it is.
# --------------------------------------------------------------------------
WORKLOADS: Dict[str, dict] = {
    # Tiny single layer, fp32 end to end, CPU-checkable in seconds.
    "tiny_fp32": dict(
        d_model=64, num_heads=4, kv_lora_rank=32, rope_dim=8, qk_nope_dim=16,
        v_dim=16, q_lora_rank=0, batch=1, context=64, block_size=64,
        dtype="f32", rope_theta=10000.0, seed=1),
    # Kimi-scale decode, contiguous cache (identity page table).
    "decode_h64_b32_l4096": dict(
        num_heads=64, kv_lora_rank=512, rope_dim=64, qk_nope_dim=128, v_dim=128,
        batch=32, lengths="fixed", context=4096, block_size=64, paged=False,
        dtype="bf16", seed=2),
    # Ragged batch over a shared pool with permuted pages.
    "paged_ragged_h128_b64": dict(
        num_heads=128, kv_lora_rank=512, rope_dim=64, qk_nope_dim=128, v_dim=128,
        batch=64, lengths="uniform", min_len=512, max_len=16384, block_size=64,
        paged=True, dtype="bf16", seed=3),
    # Long context, few sequences: needs many KV splits per sequence.
    "longctx_h64_b4_l131072": dict(
        num_heads=64, kv_lora_rank=512, rope_dim=64, qk_nope_dim=128, v_dim=128,
        batch=4, lengths="fixed", context=131072, block_size=64, paged=True,
        dtype="bf16", seed=4),
    # Prefill with cache append through the absorbed path.
    "prefill_d7168_b2_t4096": dict(
        d_model=7168, q_lora_rank=1536, kv_lora_rank=512, rope_dim=64,
        num_heads=64, qk_nope_dim=128, v_dim=128, batch=2, q_len=4096,
        block_size=64, dtype="bf16", rope_theta=10000.0, seed=5),
    # The output gate and W_O after the heads, at the prefill workload's widths
    # and token count (2 x 4096 rows).
    "output_gate_d7168_t8192": dict(
        d_model=7168, q_lora_rank=0, kv_lora_rank=512, rope_dim=64, num_heads=64,
        qk_nope_dim=128, v_dim=128, rows=8192, gated=True, block_size=64, dtype="bf16",
        seed=6),
}
# The same decode shapes over an FP8 latent cache (E4M3 codes with a per-row
# power-of-two scale, bf16 rope key: 656 bytes per token instead of 1152).
WORKLOADS["decode_h64_b32_l4096_fp8"] = dict(WORKLOADS["decode_h64_b32_l4096"],
                                             cache_dtype="fp8")
WORKLOADS["longctx_h64_b4_l131072_fp8"] = dict(WORKLOADS["longctx_h64_b4_l131072"],
                                               cache_dtype="fp8")
WORKLOADS["prefill_d7168_b2_t4096_fp8"] = dict(WORKLOADS["prefill_d7168_b2_t4096"],
                                               cache_dtype="fp8")
# The prefill workload with its attention forced onto the latent rows (the
# absorbed form; the default takes whichever form needs fewer FLOPs, at this
# size the per-head keys and values).
WORKLOADS["prefill_d7168_b2_t4096_absorbed"] = dict(WORKLOADS["prefill_d7168_b2_t4096"],
                                                    prefill_attention="latent")
# The tutorial's mechanism experiment widths ("ARCH-MLA. Multihead Latent
# Attention", 5.1): 16 query heads sharing 4 W_UK / W_UV matrices, head
# width 64, latent 256, rope 64, bf16; one sequence per history length
# 512, 2048, 8192 (the batch is not stated: one sequence is the reading).
for _L in (512, 2048, 8192):
    WORKLOADS[f"mechanism_h16_g4_r256_l{_L}"] = dict(
        num_heads=16, kv_groups=4, kv_lora_rank=256, rope_dim=64, qk_nope_dim=64, v_dim=64,
        batch=1, lengths="fixed", context=_L, block_size=64, paged=False, dtype="bf16",
        seed=60 + _L % 97)


HEADLINE = "decode_h64_b32_l4096"


# --------------------------------------------------------------------------
# dtype helpers (input rounding only)
# --------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (no NaNs drawn)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of a stored tensor (float32 or bf16 bits)."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(dtype)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, std=1.0) -> np.ndarray:
    out = rng.standard_normal(size=int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def normal_tensor(shape, seed: int, dtype: str = "bf16", std: float = 1.0) -> np.ndarray:
    """A seeded N(0, std^2) draw of the given shape in the storage dtype."""
    return _store(_normal(_rng(seed), tuple(shape), std), dtype)


def _gain(rng, n, gain_jitter):
    if gain_jitter == 0.0:
        return np.ones(n, dtype=np.float32)
    return (1.0 + gain_jitter * _normal(rng, (n,))).astype(np.float32)


# --------------------------------------------------------------------------
# Page tables
# --------------------------------------------------------------------------
def page_table(rng, lengths, block_size, permute: bool, spare_blocks: int = 0):
    """Map each sequence's logical pages to physical pages of one shared pool.

    Returns (block_table int32 [B, max_blocks], num_blocks).  Unused table
    entries hold 0, a valid page, so that a stray read stays in bounds.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    nblk = (lengths + block_size - 1) // block_size
    total = int(nblk.sum()) + spare_blocks
    phys = rng.permutation(total) if permute else np.arange(total)
    max_blocks = int(nblk.max()) if len(nblk) else 0
    table = np.zeros((len(lengths), max(max_blocks, 1)), dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = phys[off:off + n]
        off += n
    return table, total


@dataclasses.dataclass
class DecodeInputs:
    cfg: dict
    seq_lens: np.ndarray      # int32 [B], counts the current token
    block_table: np.ndarray   # int32 [B, max_blocks]
    pool: np.ndarray          # [num_blocks, block_size, R + Dr] storage dtype
    q_nope: np.ndarray        # [B, H, Dn]
    q_rope: np.ndarray        # [B, H, Dr] (already rotated)
    w_uk: np.ndarray          # [H or kv_groups, Dn, R]
    w_uv: np.ndarray          # [H or kv_groups, R, Dv]


def decode_lengths(cfg: dict, rng) -> np.ndarray:
    B = cfg["batch"]
    if cfg.get("lengths", "fixed") == "uniform":
        return rng.integers(cfg["min_len"], cfg["max_len"], size=B,
                            endpoint=True).astype(np.int32)
    return np.full(B, cfg["context"], dtype=np.int32)


def decode_inputs(cfg: dict, seed: Optional[int] = None,
                  lengths: Optional[np.ndarray] = None) -> DecodeInputs:
    """Decode-step inputs: a filled latent cache plus queries and weights.

    The cache is filled directly with N(0,1) values (both the latent part and
    the rope key), as for a cache that already went through the append step.
    Draw order: lengths, page permutation, pool, q_nope, q_rope, W_UK, W_UV.
    """
    rng = _rng(cfg["seed"] if seed is None else seed)
    H, R, Dr = cfg["num_heads"], cfg["kv_lora_rank"], cfg["rope_dim"]
    Dn, Dv, bs = cfg["qk_nope_dim"], cfg["v_dim"], cfg["block_size"]
    dt = cfg["dtype"]
    lens = decode_lengths(cfg, rng) if lengths is None else np.asarray(lengths, np.int32)
    table, nblocks = page_table(rng, lens, bs, cfg.get("paged", False))
    row = R + Dr
    pool = np.empty((nblocks, bs, row), dtype=np.uint16 if dt == "bf16" else np.float32)
    step = max(1, (1 << 22) // (bs * row))   # ~4M values per chunk
    for s in range(0, nblocks, step):
        e = min(nblocks, s + step)
        pool[s:e] = _store(_normal(rng, (e - s, bs, row)), dt)
    B = len(lens)
    q_nope = _store(_normal(rng, (B, H, Dn)), dt)
    q_rope = _store(_normal(rng, (B, H, Dr)), dt)
    G = cfg.get("kv_groups") or H          # matrices shared by H / G consecutive heads
    w_uk = _store(_normal(rng, (G, Dn, R), 1.0 / math.sqrt(R)), dt)
    w_uv = _store(_normal(rng, (G, R, Dv), 1.0 / math.sqrt(R)), dt)
    return DecodeInputs(cfg, lens, table, pool, q_nope, q_rope, w_uk, w_uv)


@dataclasses.dataclass
class LayerWeights:
    w_q: Optional[np.ndarray]       # [M, H*(Dn+Dr)] when q_lora_rank == 0
    w_dq: Optional[np.ndarray]      # [M, Rq]
    q_norm_w: Optional[np.ndarray]  # [Rq] float32
    w_uq: Optional[np.ndarray]      # [Rq, H*(Dn+Dr)]
    w_dkv: np.ndarray               # [M, R + Dr]
    kv_norm_w: np.ndarray           # [R] float32
    w_uk: np.ndarray                # [H, Dn, R]
    w_uv: np.ndarray                # [H, R, Dv]


@dataclasses.dataclass
class PrefillInputs:
    cfg: dict
    x: np.ndarray             # [B, T, M] storage dtype
    weights: LayerWeights
    start_pos: np.ndarray     # int32 [B]
    block_table: np.ndarray   # int32 [B, max_blocks]
    num_blocks: int


def layer_weights(cfg: dict, rng, gain_jitter: float = 0.0) -> LayerWeights:
    M, H = cfg["d_model"], cfg["num_heads"]
    R, Dr, Dn, Dv = cfg["kv_lora_rank"], cfg["rope_dim"], cfg["qk_nope_dim"], cfg["v_dim"]
    Rq, dt = cfg.get("q_lora_rank", 0), cfg["dtype"]
    qw = H * (Dn + Dr)
    w_q = w_dq = q_norm_w = w_uq = None
    if Rq:
        w_dq = _store(_normal(rng, (M, Rq), 1.0 / math.sqrt(M)), dt)
        q_norm_w = _gain(rng, Rq, gain_jitter)
        w_uq = _store(_normal(rng, (Rq, qw), 1.0 / math.sqrt(Rq)), dt)
    else:
        w_q = _store(_normal(rng, (M, qw), 1.0 / math.sqrt(M)), dt)
    w_dkv = _store(_normal(rng, (M, R + Dr), 1.0 / math.sqrt(M)), dt)
    kv_norm_w = _gain(rng, R, gain_jitter)
    w_uk = _store(_normal(rng, (H, Dn, R), 1.0 / math.sqrt(R)), dt)
    w_uv = _store(_normal(rng, (H, R, Dv), 1.0 / math.sqrt(R)), dt)
    return LayerWeights(w_q, w_dq, q_norm_w, w_uq, w_dkv, kv_norm_w, w_uk, w_uv)


def prefill_inputs(cfg: dict, seed: Optional[int] = None, q_len: Optional[int] = None,
                   batch: Optional[int] = None, start_pos=None, gain_jitter: float = 0.0,
                   paged: bool = True, extra_ctx: int = 0) -> PrefillInputs:
    """Hidden states for T fresh tokens per sequence plus one layer's weights.

    ``start_pos`` gives each sequence's first new position (default 0);
    the page table covers start_pos + T + extra_ctx tokens per sequence.
    Draw order: weights, x, page permutation.
    """
    rng = _rng(cfg["seed"] if seed is None else seed)
    B = cfg["batch"] if batch is None else batch
    T = cfg.get("q_len", cfg.get("context", 1)) if q_len is None else q_len
    w = layer_weights(cfg, rng, gain_jitter)
    x = _store(_normal(rng, (B, T, cfg["d_model"])), cfg["dtype"])
    sp = np.zeros(B, np.int32) if start_pos is None else np.asarray(start_pos, np.int32)
    table, nblocks = page_table(rng, sp + T + extra_ctx, cfg["block_size"], paged)
    return PrefillInputs(cfg, x, w, sp, table, nblocks)


def tiny_sequence(seed: Optional[int] = None, gain_jitter: float = 0.0) -> PrefillInputs:
    """The tiny fp32 layer: 65 tokens (positions 0..64) of one sequence."""
    cfg = WORKLOADS["tiny_fp32"]
    return prefill_inputs(cfg, seed=seed, q_len=cfg["context"] + 1, batch=1,
                          gain_jitter=gain_jitter, paged=False)


# --------------------------------------------------------------------------
# Device-side generation for the benchmark (same distributions, torch RNG).
# --------------------------------------------------------------------------
def decode_inputs_torch(cfg: dict, seed: int, device, lengths=None):
    """Same shapes and distributions as ``decode_inputs``, drawn on the device.

    Used where host generation plus upload would dominate (benchmark input
    rotation).  Values differ from the numpy draw; parity tests use the numpy
    path.  Returns a dict of torch tensors.
    """
    import torch
    rng = _rng(seed)
    lens = decode_lengths(cfg, rng) if lengths is None else np.asarray(lengths, np.int32)
    table, nblocks = page_table(rng, lens, cfg["block_size"], cfg.get("paged", False))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    H, R, Dr = cfg["num_heads"], cfg["kv_lora_rank"], cfg["rope_dim"]
    Dn, Dv, bs = cfg["qk_nope_dim"], cfg["v_dim"], cfg["block_size"]
    G = cfg.get("kv_groups") or H
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    B = len(lens)

    def n(shape, std=1.0):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dt)

    if cfg.get("cache_dtype") == "fp8":
        # FP8 rows drawn directly (no values are quantized here): codes
        # uniform over the finite non-negative E4M3 codes with a random sign,
        # one power-of-two scale per row (2^-9 .. 2^-7), a N(0,1) bf16 rope
        # key, zero padding: R codes | Dr bf16 | float32 scale | 12 bytes
        pool = torch.zeros((nblocks, bs, R + 2 * Dr + 16), dtype=torch.uint8, device=device)
        codes = torch.randint(0, 0x7F, (nblocks, bs, R), generator=g, device=device,
                              dtype=torch.uint8)
        sign = torch.randint(0, 2, (nblocks, bs, R), generator=g, device=device,
                             dtype=torch.uint8)
        pool[..., :R] = codes | (sign << 7)
        pool[..., R:R + 2 * Dr] = torch.randn((nblocks, bs, Dr), generator=g, device=device,
                                              dtype=torch.float32).to(torch.bfloat16).view(
                                                  torch.uint8)
        expo = torch.randint(-9, -6, (nblocks, bs, 1), generator=g, device=device)
        pool[..., R + 2 * Dr:R + 2 * Dr + 4] = torch.exp2(expo.float()).view(torch.uint8)
    else:
        pool = n((nblocks, bs, R + Dr))
    return dict(
        seq_lens=torch.from_numpy(lens).to(device),
        block_table=torch.from_numpy(table).to(device),
        max_seq_len=int(lens.max()),
        pool=pool,
        q_nope=n((B, H, Dn)), q_rope=n((B, H, Dr)),
        w_uk=n((G, Dn, R), 1.0 / math.sqrt(R)), w_uv=n((G, R, Dv), 1.0 / math.sqrt(R)),
    )


def prefill_inputs_torch(cfg: dict, seed: int, device):
    """Same shapes and distributions as ``prefill_inputs`` (fresh tokens at
    positions 0..T-1, gains 1, block-64 pool with permuted pages), drawn on
    the device for the benchmark.  Returns a dict of torch tensors."""
    import torch
    rng = _rng(seed)
    B, T = cfg["batch"], cfg["q_len"]
    M, H = cfg["d_model"], cfg["num_heads"]
    R, Dr, Dn, Dv = cfg["kv_lora_rank"], cfg["rope_dim"], cfg["qk_nope_dim"], cfg["v_dim"]
    Rq, bs = cfg.get("q_lora_rank", 0), cfg["block_size"]
    table, nblocks = page_table(rng, np.full(B, T), bs, True)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32

    def n(shape, std=1.0):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dt)

    qw = H * (Dn + Dr)
    w = dict(w_dkv=n((M, R + Dr), 1.0 / math.sqrt(M)),
             kv_norm_w=torch.ones(R, dtype=torch.float32, device=device),
             w_uk=n((H, Dn, R), 1.0 / math.sqrt(R)), w_uv=n((H, R, Dv), 1.0 / math.sqrt(R)))
    if Rq:
        w.update(w_dq=n((M, Rq), 1.0 / math.sqrt(M)),
                 q_norm_w=torch.ones(Rq, dtype=torch.float32, device=device),
                 w_uq=n((Rq, qw), 1.0 / math.sqrt(Rq)))
    else:
        w.update(w_q=n((M, qw), 1.0 / math.sqrt(M)))
    if cfg.get("cache_dtype") == "fp8":   # rows of R + 2 Dr + 16 bytes
        pool = torch.zeros((nblocks, bs, R + 2 * Dr + 16), dtype=torch.uint8, device=device)
    else:
        pool = torch.zeros((nblocks, bs, R + Dr), dtype=dt, device=device)
    return dict(x=n((B, T, M)), weights=w, pool=pool,
                block_table=torch.from_numpy(table).to(device),
                start_pos=torch.zeros(B, dtype=torch.int32, device=device))


def output_gate_inputs_torch(cfg: dict, seed: int, device):
    """x [rows, M], head outputs [rows, H, Dv] ~ N(0,1); W_G [M, H Dv] ~
    N(0, 1/M), W_O [H Dv, M] ~ N(0, 1/(H Dv)); drawn on the device."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    n, M, H, Dv = cfg["rows"], cfg["d_model"], cfg["num_heads"], cfg["v_dim"]

    def draw(shape, std=1.0):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(torch.bfloat16)

    return dict(x=draw((n, M)), head_out=draw((n, H, Dv)),
                w_g=draw((M, H * Dv), 1.0 / math.sqrt(M)),
                w_o=draw((H * Dv, M), 1.0 / math.sqrt(H * Dv)))
