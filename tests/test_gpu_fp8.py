"""FP8 latent cache on the GPU, through the C ABI, against the oracle.

Rows are quantized by the oracle (oracle/fp8_cache.py: E4M3 latent with a
per-row power-of-two scale, bf16 rope key, 656-byte rows) from the seeded
N(0,1) pools of ``workloads``; the GPU decodes those bytes and the oracle
attends over their dequantized values in float64.  The append test checks
the rows the GPU quantizes itself against the oracle's quantization of the
same layer.  Tolerances: those of the bf16 paths (rel-L2 <= 5e-3, max abs
<= 2e-2 on outputs); quantized rows within one E4M3 step.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import to_dev, to_host_f64, assert_bf16, compact_sequences

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch  # noqa: F401
    import mla_latent_kv_26_amd as m
    return m


def sync():
    import torch
    torch.cuda.synchronize()


def fp8_pool(inp, R):
    """The inputs' pool rows quantized to FP8 rows: (bytes, dequantized f64)."""
    codes, s, rope = oracle.quantize_rows_fp8(workloads.to_f64(inp.pool), R)
    return oracle.pack_rows_fp8(codes, s, rope), oracle.dequantize_rows_fp8(codes, s, rope)


def check_fp8_decode(m, cfg, lengths=None, sample=None, seed=None):
    import torch
    cfg = dict(cfg, cache_dtype="fp8")
    mc = m.MLAConfig.from_dict(cfg)
    lens = None if lengths is None else np.asarray(lengths, np.int32)
    inp = workloads.decode_inputs(cfg, seed=seed, lengths=lens)
    raw, deq = fp8_pool(inp, cfg["kv_lora_rank"])
    B, L = len(inp.seq_lens), int(inp.seq_lens.max())
    ws = torch.zeros(m.mla_decode_workspace_size(mc, B, L), dtype=torch.uint8, device="cuda")
    out = m.mla_decode(mc, to_dev(inp.q_nope), to_dev(inp.q_rope), to_dev(inp.w_uk),
                       to_dev(inp.w_uv), to_dev(raw), to_dev(inp.block_table),
                       to_dev(inp.seq_lens), L, workspace=ws)
    sync()
    got = to_host_f64(out)
    ids = list(range(B)) if sample is None else list(sample)
    inp_q = dataclasses.replace(inp, pool=deq)
    ref = []
    for b, (pages, table, ln) in zip(ids, compact_sequences(inp_q, ids)):
        o, _ = oracle.decode(workloads.to_f64(inp.q_nope[b:b + 1]),
                             workloads.to_f64(inp.q_rope[b:b + 1]), workloads.to_f64(inp.w_uk),
                             workloads.to_f64(inp.w_uv), pages, table, ln, cfg)
        ref.append(o[0])
    return assert_bf16(got[ids], np.stack(ref), f"fp8 {str(list(inp.seq_lens[:6]))}",
                       per_row_axis=0)


def test_fp8_decode_h64_b32_l4096_full(m):
    """The headline shape over an FP8 cache, every sequence checked."""
    e = check_fp8_decode(m, workloads.WORKLOADS["decode_h64_b32_l4096"])
    print("fp8 decode_h64_b32_l4096", e)


def test_fp8_decode_paged_edge_lengths(m):
    """Permuted pages, partial tiles and pages, one-token sequences."""
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=64, lengths="explicit",
               seed=31)
    check_fp8_decode(m, cfg, [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 1000, 4097])


def test_fp8_decode_h128_ragged_sample(m):
    """128 heads (two head groups read the same staged tiles), ragged batch."""
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], batch=16, max_len=6000, seed=32)
    check_fp8_decode(m, cfg, sample=[0, 5, 15])


def test_fp8_decode_larger_pages(m):
    """FP8 rows in 256-token pages (8 tiles per page), ragged lengths."""
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=64, lengths="explicit",
               paged=True, block_size=256, seed=41)
    check_fp8_decode(m, cfg, [1, 255, 256, 257, 799, 4096, 3000])


@pytest.mark.parametrize("heads", [32, 96])
def test_fp8_decode_heads_not_a_multiple_of_64(m, heads):
    """The 32-heads-per-workgroup FP8 kernels (H = 32, and 96 in three head
    groups), ragged lengths over permuted pages."""
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=heads, lengths="explicit",
               paged=True, seed=33 + heads)
    check_fp8_decode(m, cfg, [1, 31, 32, 33, 700, 4096, 2049, 65])


def test_fp8_decode_single_long_sequence(m):
    """One 20,000-token sequence: 625 tiles over all workgroups."""
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=64, lengths="explicit",
               seed=33)
    check_fp8_decode(m, cfg, [20000])


def bf16(a):
    """(bf16 bit patterns, their float64 values) of a float array."""
    bits = workloads.bf16_bits(np.asarray(a, np.float32))
    return bits, workloads.to_f64(bits)


def check_fp8_rows(got_raw, rows, R, Dr):
    """Stored FP8 rows against the oracle's unrounded rows (float64): scales
    equal unless max|c| sits on a power-of-two boundary, codes within one
    E4M3 step (the two sides round different float32/float64 sums), the rope
    key within a bf16 step, pad bytes zero."""
    codes, s, rope = oracle.unpack_rows_fp8(got_raw, R, Dr)
    q_codes, q_s, _ = oracle.quantize_rows_fp8(rows, R)
    same = s == q_s
    assert same.mean() >= 0.98, same.mean()
    assert np.all((s == 2 * q_s) | (2 * s == q_s) | same)
    got_c = oracle.e4m3_value(codes) * s[:, None]
    ref_c = rows[:, :R]
    # one E4M3 step of |c| / s (3 mantissa bits), at least a subnormal step
    step = np.maximum(np.abs(ref_c) / 8.0, 2.0 ** -9 * q_s[:, None])
    assert np.all(np.abs(got_c - ref_c) <= step + 1e-12)
    assert np.mean(codes[same] == q_codes[same]) >= 0.999
    assert np.all(np.abs(rope - rows[:, R:]) <= 2.0 ** -7 * np.abs(rows[:, R:]) + 1e-6)
    assert np.all(got_raw[:, R + 2 * Dr + 4:] == 0)


def _append_case(n=300, seed=41):
    rng = np.random.default_rng(seed)
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=640, q_lora_rank=0,
               cache_dtype="fp8", seed=seed)
    M, R, Dr = cfg["d_model"], cfg["kv_lora_rank"], cfg["rope_dim"]
    w_dkv = bf16(rng.standard_normal((M, R + Dr)) / np.sqrt(M))
    gain = (1.0 + 0.1 * rng.standard_normal(R)).astype(np.float32)
    x = bf16(rng.standard_normal((n, M)))
    pos = rng.permutation(4 * n)[:n].astype(np.int32)
    return cfg, x, w_dkv, gain, pos


def test_fp8_cache_append_rows(m):
    """mla_cache_append into an FP8 pool: every written row against the
    oracle's quantization of the same layer (codes within one E4M3 step,
    scales equal unless max|c| sits on a power-of-two boundary, rope key
    within a bf16 step, pad bytes zero, skipped slots untouched)."""
    import torch
    cfg, (x_bits, x), (w_bits, w_dkv), gain, pos = _append_case()
    mc = m.MLAConfig.from_dict(cfg)
    R, Dr, bs = cfg["kv_lora_rank"], cfg["rope_dim"], cfg["block_size"]
    n = x.shape[0]
    nb = -(-2 * n // bs)
    slots = np.random.default_rng(42).permutation(nb * bs)[:n].astype(np.int32)
    slots[::7] = -1                                        # skipped tokens
    pool = torch.full((nb, bs, mc.pool_row), 0xAB, dtype=torch.uint8, device="cuda")
    m.mla_cache_append(mc, to_dev(x_bits), to_dev(w_bits), to_dev(gain), to_dev(pos),
                       to_dev(slots), pool)
    sync()
    raw = pool.cpu().numpy().reshape(nb * bs, -1)
    keep = slots >= 0
    w64 = {"w_dkv": w_dkv, "kv_norm_w": gain.astype(np.float64)}
    rows = oracle.append_rows(x[keep], pos[keep], w64, cfg, storage="f64")
    check_fp8_rows(raw[slots[keep]], rows, R, Dr)
    untouched = np.setdiff1d(np.arange(nb * bs), slots[keep])
    assert np.all(raw[untouched] == 0xAB)


def test_fp8_append_then_decode(m):
    """Rows the GPU appends, then decoded by the GPU, against the oracle's own
    append (FP8 storage) and decode of the same layer."""
    import torch
    cfg, (x_bits, x), (w_bits, w_dkv), gain, _ = _append_case(n=777, seed=43)
    mc = m.MLAConfig.from_dict(cfg)
    R, Dr, bs, H = cfg["kv_lora_rank"], cfg["rope_dim"], cfg["block_size"], cfg["num_heads"]
    n = x.shape[0]
    nb = -(-n // bs)
    table = np.random.default_rng(44).permutation(nb).astype(np.int32)[None]
    pos = np.arange(n, dtype=np.int32)
    slots = (table[0][pos // bs] * bs + pos % bs).astype(np.int32)
    pool = torch.zeros((nb, bs, mc.pool_row), dtype=torch.uint8, device="cuda")
    m.mla_cache_append(mc, to_dev(x_bits), to_dev(w_bits), to_dev(gain), to_dev(pos),
                       to_dev(slots), pool)
    rng = np.random.default_rng(45)
    Dn, Dv = cfg["qk_nope_dim"], cfg["v_dim"]
    q_nope = bf16(rng.standard_normal((1, H, Dn)))
    q_rope = bf16(rng.standard_normal((1, H, Dr)))
    w_uk = bf16(rng.standard_normal((H, Dn, R)) / np.sqrt(R))
    w_uv = bf16(rng.standard_normal((H, R, Dv)) / np.sqrt(R))
    out = m.mla_decode(mc, to_dev(q_nope[0]), to_dev(q_rope[0]), to_dev(w_uk[0]),
                       to_dev(w_uv[0]), pool, to_dev(table),
                       torch.tensor([n], dtype=torch.int32, device="cuda"), n)
    sync()
    w64 = {"w_dkv": w_dkv, "kv_norm_w": gain.astype(np.float64)}
    rows = oracle.append_rows(x, pos, w64, cfg, storage="fp8")
    ref, _ = oracle.decode(q_nope[1], q_rope[1], w_uk[1], w_uv[1], rows[None],
                           np.arange(1)[None], np.array([n]), dict(cfg, block_size=n))
    assert_bf16(to_host_f64(out), ref, "fp8 append then decode", per_row_axis=0)


def _pool_raw(pool, table, L):
    raw = pool.cpu().numpy()
    j = np.arange(L)
    return raw[table[j // raw.shape[1]], j % raw.shape[1]]


def test_fp8_prefill_with_continuation(m):
    """Prefill into an FP8 cache (600 new tokens, then 300 more at position
    600, permuted pages, jittered gains): the stored rows against the
    oracle's quantization, the outputs against the oracle's forward over an
    FP8 cache (new rows stored first, every key and value read back from
    the stored rows)."""
    import torch
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=640, q_lora_rank=128,
               cache_dtype="fp8", seed=47)
    mc = m.MLAConfig.from_dict(cfg)
    R, Dr = cfg["kv_lora_rank"], cfg["rope_dim"]
    inp = workloads.prefill_inputs(cfg, q_len=900, batch=2, gain_jitter=0.1)
    w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
    w64 = {k: (None if v is None else workloads.to_f64(v)) for k, v in vars(inp.weights).items()}
    pool = torch.zeros((inp.num_blocks, 64, mc.pool_row), dtype=torch.uint8, device="cuda")
    table = to_dev(inp.block_table)
    x = to_dev(inp.x)
    out1 = m.mla_prefill(mc, x[:, :600].contiguous(), w, pool, table,
                         torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
    out2 = m.mla_prefill(mc, x[:, 600:].contiguous(), w, pool, table,
                         torch.full((2,), 600, dtype=torch.int32, device="cuda"), 600)
    sync()
    got = np.concatenate([to_host_f64(out1), to_host_f64(out2)], axis=1)
    for b in range(2):
        x64 = workloads.to_f64(inp.x[b])
        rows = oracle.append_rows(x64, np.arange(900), w64, cfg, storage="f64")
        check_fp8_rows(_pool_raw(pool, inp.block_table[b], 900), rows, R, Dr)
        ref, _ = oracle.layer_forward(x64, w64, cfg, storage="fp8")
        assert_bf16(got[b], ref, f"fp8 prefill b={b}", per_row_axis=0)


def test_fp8_prefill_d7168_b2_t4096_sample(m):
    """The full-size prefill over an FP8 cache: every stored row checked,
    outputs on a sample of query rows of both sequences."""
    import torch
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], cache_dtype="fp8")
    mc = m.MLAConfig.from_dict(cfg)
    R, Dr, T = cfg["kv_lora_rank"], cfg["rope_dim"], cfg["q_len"]
    inp = workloads.prefill_inputs(cfg)
    w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
    pool = torch.zeros((inp.num_blocks, 64, mc.pool_row), dtype=torch.uint8, device="cuda")
    out = m.mla_prefill(mc, to_dev(inp.x), w, pool, to_dev(inp.block_table),
                        torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
    sync()
    w64 = {k: (None if v is None else workloads.to_f64(v)) for k, v in vars(inp.weights).items()}
    sample = [0, 1, 63, 64, 65, 1000, 2047, 4095]
    for b in range(2):
        x64 = workloads.to_f64(inp.x[b])
        rows = oracle.append_rows(x64, np.arange(T), w64, cfg, storage="f64")
        check_fp8_rows(_pool_raw(pool, inp.block_table[b], T), rows, R, Dr)
        stored = oracle.fp8_store_rows(rows, R)
        ref = oracle.attend_tokens(x64[sample], np.array(sample), w64, cfg, stored, q_block=1)
        e = assert_bf16(to_host_f64(out[b, sample]), ref, f"fp8 prefill b={b}", per_row_axis=0)
        print("fp8 prefill_d7168_b2_t4096", b, e)


def test_fp8_prefill_other_widths_rejected(m):
    """FP8 prefill runs on the per-head key/value kernels only (Dn = Dv =
    128); other head widths get MLA_ERR_UNSUPPORTED before any launch."""
    import torch
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=640, q_lora_rank=128,
               qk_nope_dim=64, v_dim=64, cache_dtype="fp8", seed=46)
    mc = m.MLAConfig.from_dict(cfg)
    inp = workloads.prefill_inputs(cfg, q_len=8, batch=1)
    w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
    pool = torch.zeros((inp.num_blocks, 64, mc.pool_row), dtype=torch.uint8, device="cuda")
    with pytest.raises(m.MLAError) as e:
        m.mla_prefill(mc, to_dev(inp.x), w, pool, to_dev(inp.block_table),
                      torch.zeros(1, dtype=torch.int32, device="cuda"), 0)
    assert e.value.status == 2 and "FP8" in str(e.value)
