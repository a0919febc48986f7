"""Parity of the HIP library with the CPU oracle, on seeded inputs.

Every workload runs at its full size through the C ABI; where the oracle
would take too long on everything it checks a stated sample of sequences or
query rows, computed one by one.  Tolerances: float32 max abs <= 1e-5;
bf16 storage relative L2 <= 5e-3 and max abs <= 2e-2 (plus the cosine floor
printed by the tutorial's bf16 run).
"""
import dataclasses
import os

import numpy as np
import pytest

import oracle
import workloads
from workloads import to_f64
from gpu_util import (to_dev, to_host_f64, assert_f32, assert_bf16, compact_sequences,
                      errors, BF16_REL_L2)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch  # noqa: F401
    import mla_latent_kv_26_amd as m
    return m


def sync():
    import torch
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def gpu_decode(m, cfg, inp, workspace=None):
    """mla_decode through the C ABI (workspace: reuse a buffer across calls)."""
    import torch
    mc = m.MLAConfig.from_dict(cfg)
    B, L = len(inp.seq_lens), int(inp.seq_lens.max())
    if workspace is None:
        workspace = torch.zeros(m.mla_decode_workspace_size(mc, B, L), dtype=torch.uint8,
                                device="cuda")
    out = m.mla_decode(mc, to_dev(inp.q_nope), to_dev(inp.q_rope), to_dev(inp.w_uk),
                       to_dev(inp.w_uv), to_dev(inp.pool), to_dev(inp.block_table),
                       to_dev(inp.seq_lens), L, workspace=workspace)
    sync()
    return to_host_f64(out)


def oracle_decode(cfg, inp, ids):
    outs = []
    for b, (pages, table, lens) in zip(ids, compact_sequences(inp, ids)):
        o, _ = oracle.decode(to_f64(inp.q_nope[b:b + 1]), to_f64(inp.q_rope[b:b + 1]),
                             to_f64(inp.w_uk), to_f64(inp.w_uv), pages, table, lens, cfg)
        outs.append(o[0])
    return np.stack(outs)


def bf16_decode_cfg(**over):
    base = dict(workloads.WORKLOADS["paged_ragged_h128_b64"])
    base.update(dict(num_heads=64, lengths="explicit", paged=True, seed=11))
    base.update(over)
    return base


def check_decode(m, cfg, lengths, sample=None, seed=None):
    inp = workloads.decode_inputs(cfg, seed=seed, lengths=np.asarray(lengths, np.int32))
    got = gpu_decode(m, cfg, inp)
    ids = list(range(len(lengths))) if sample is None else list(sample)
    ref = oracle_decode(cfg, inp, ids)
    if cfg["dtype"] == "f32":
        return assert_f32(got[ids], ref, str(lengths[:8]))
    return assert_bf16(got[ids], ref, str(lengths[:8]), per_row_axis=0)


# ---------------------------------------------------------------------------
# tiny float32 layer: full forward, incremental decode, append
# ---------------------------------------------------------------------------
def tiny_setup(m, gain_jitter=0.1):
    seq = workloads.tiny_sequence(gain_jitter=gain_jitter)
    cfg = seq.cfg
    mc = m.MLAConfig.from_dict(cfg)
    w = {k: to_dev(v) for k, v in vars(seq.weights).items() if v is not None}
    w64 = {k: (None if v is None else to_f64(v)) for k, v in vars(seq.weights).items()}
    return seq, cfg, mc, w, w64


def test_tiny_fp32_full_forward(m):
    import torch
    seq, cfg, mc, w, w64 = tiny_setup(m)
    pool = torch.zeros((2, 64, mc.row), dtype=torch.float32, device="cuda")
    table = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    out = m.mla_prefill(mc, to_dev(seq.x), w, pool, table,
                        torch.zeros(1, dtype=torch.int32, device="cuda"), 0)
    sync()
    ref, rows = oracle.layer_forward(to_f64(seq.x[0]), w64, cfg, storage="f32")
    assert_f32(to_host_f64(out)[0], ref, "tiny full forward")
    got_rows = to_host_f64(pool).reshape(-1, mc.row)[:65]
    assert_f32(got_rows, rows, "tiny cache rows")


def test_tiny_fp32_incremental_equals_full(m):
    """Ticket acceptance criterion on the GPU: decode of token 64 after a
    64-token prefill equals row 64 of the 65-token forward within 1e-5."""
    import torch
    seq, cfg, mc, w, w64 = tiny_setup(m)
    table = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    pool_a = torch.zeros((2, 64, mc.row), dtype=torch.float32, device="cuda")
    full = m.mla_prefill(mc, to_dev(seq.x), w, pool_a, table,
                         torch.zeros(1, dtype=torch.int32, device="cuda"), 0)
    pool_b = torch.zeros_like(pool_a)
    x = to_dev(seq.x)
    m.mla_prefill(mc, x[:, :64].contiguous(), w, pool_b, table,
                  torch.zeros(1, dtype=torch.int32, device="cuda"), 0)
    step = m.mla_prefill(mc, x[:, 64:].contiguous(), w, pool_b, table,
                         torch.full((1,), 64, dtype=torch.int32, device="cuda"), 64)
    sync()
    assert_f32(to_host_f64(step)[0, 0], to_host_f64(full)[0, 64], "incremental vs full (gpu)")
    ref, _ = oracle.layer_forward(to_f64(seq.x[0]), w64, cfg, storage="f32")
    assert_f32(to_host_f64(step)[0, 0], ref[64], "incremental vs oracle")
    np.testing.assert_array_equal(to_host_f64(pool_a), to_host_f64(pool_b))


def test_tiny_fp32_decode_ragged(m):
    cfg = dict(workloads.WORKLOADS["tiny_fp32"], batch=5, lengths="explicit", paged=True,
               block_size=16, seed=21)
    check_decode(m, cfg, [1, 5, 64, 65, 200])


def test_tiny_fp32_cache_append_with_skip(m):
    import torch
    seq, cfg, mc, w, w64 = tiny_setup(m)
    mc16 = dataclasses.replace(mc, block_size=16)
    pool = torch.full((8, 16, mc.row), 7.0, dtype=torch.float32, device="cuda")
    pos = np.array([3, 0, 50, 64, 9], np.int32)
    slots = np.array([5, 17, -1, 127, 40], np.int32)
    x = to_dev(seq.x[0, :5].copy())
    m.mla_cache_append(mc16, x, w["w_dkv"], w["kv_norm_w"], to_dev(pos), to_dev(slots), pool,
                       rope_table=m.mla_rope_table(mc16, 65).cuda())
    sync()
    ref = oracle.append_rows(to_f64(seq.x[0, :5]), pos, w64, cfg, storage="f32")
    flat = to_host_f64(pool).reshape(-1, mc.row)
    for i, s in enumerate(slots):
        if s >= 0:
            assert_f32(flat[s], ref[i], f"append slot {s}")
    untouched = np.setdiff1d(np.arange(flat.shape[0]), slots[slots >= 0])
    assert np.all(flat[untouched] == 7.0)


# ---------------------------------------------------------------------------
# bf16 decode
# ---------------------------------------------------------------------------
def test_decode_h64_b32_l4096_full(m):
    """Kimi-scale decode, contiguous cache, every sequence checked."""
    cfg = workloads.WORKLOADS["decode_h64_b32_l4096"]
    inp = workloads.decode_inputs(cfg)
    got = gpu_decode(m, cfg, inp)
    ref = oracle_decode(cfg, inp, range(cfg["batch"]))
    e = assert_bf16(got, ref, "decode_h64_b32_l4096", per_row_axis=0)
    print("decode_h64_b32_l4096", e)


def test_decode_workspace_reused_across_calls(m):
    """One workspace, several consecutive decode calls with different inputs:
    each call must merge only the partials it wrote itself (with fewer tiles
    than workgroups, some workgroups write none), so every result matches
    the oracle although the workspace holds the previous call's values."""
    import torch
    cfg = bf16_decode_cfg()
    lens = np.array([700, 64, 3000, 1, 129, 2048, 511, 900], np.int32)
    mc = m.MLAConfig.from_dict(cfg)
    ws = torch.zeros(m.mla_decode_workspace_size(mc, len(lens), int(lens.max())),
                     dtype=torch.uint8, device="cuda")
    for seed in (21, 22, 23):
        inp = workloads.decode_inputs(cfg, seed=seed, lengths=lens)
        got = gpu_decode(m, cfg, inp, workspace=ws)
        ref = oracle_decode(cfg, inp, range(len(lens)))
        assert_bf16(got, ref, f"reused workspace, seed {seed}", per_row_axis=0)


def test_decode_edge_lengths(m):
    check_decode(m, bf16_decode_cfg(), [1, 2, 63, 64, 65, 127, 128, 129, 1000, 4097])


def test_decode_more_sequences_than_workgroups(m):
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 300, size=300)
    check_decode(m, bf16_decode_cfg(), lens, sample=[0, 1, 2, 150, 298, 299])


def test_decode_max_batch_1024(m):
    lens = (np.arange(1024) % 97) + 1
    check_decode(m, bf16_decode_cfg(seed=12), lens, sample=[0, 96, 500, 1023])


def test_decode_single_long_sequence(m):
    check_decode(m, bf16_decode_cfg(), [20000])


def test_decode_h128_ragged(m):
    check_decode(m, bf16_decode_cfg(num_heads=128, seed=13), [1, 100, 4096, 5000, 16384])


@pytest.mark.parametrize("block_size", [128, 1024])
def test_decode_larger_pages(m, block_size):
    """Pages of 128 and 1024 tokens (4 and 32 tiles per page: the page-id
    cursor and the guessed first tiles index pages by shifts), ragged lengths
    at page and tile edges over a permuted pool."""
    check_decode(m, bf16_decode_cfg(block_size=block_size, seed=37 + block_size),
                 [1, block_size - 1, block_size, block_size + 1, 3 * block_size + 31, 4096, 5000])


@pytest.mark.parametrize("heads", [32, 96])
def test_decode_heads_not_a_multiple_of_64(m, heads):
    """H = 32 and 96 run the 32-heads-per-workgroup kernels (two active score
    waves, two that only load; 96 heads are three head groups sharing every
    tile): ragged lengths over permuted pages against the oracle."""
    check_decode(m, bf16_decode_cfg(num_heads=heads, seed=29 + heads),
                 [1, 31, 32, 33, 700, 4096, 2049, 65])


def test_paged_ragged_h128_b64_full(m):
    """H=128, 64 ragged sequences (512..16384 tokens) over a permuted pool:
    every sequence against the oracle."""
    cfg = workloads.WORKLOADS["paged_ragged_h128_b64"]
    inp = workloads.decode_inputs(cfg)
    got = gpu_decode(m, cfg, inp)
    ids = list(range(cfg["batch"]))
    ref = oracle_decode(cfg, inp, ids)
    e = assert_bf16(got, ref, "paged_ragged_h128_b64", per_row_axis=0)
    print("paged_ragged_h128_b64 all sequences", e)


def test_longctx_h64_b4_l131072_full(m):
    """4 sequences of 131072 tokens (64 split pieces each): every sequence
    against the oracle."""
    cfg = workloads.WORKLOADS["longctx_h64_b4_l131072"]
    inp = workloads.decode_inputs(cfg)
    got = gpu_decode(m, cfg, inp)
    ids = list(range(cfg["batch"]))
    ref = oracle_decode(cfg, inp, ids)
    e = assert_bf16(got, ref, "longctx_h64_b4_l131072", per_row_axis=0)
    print("longctx_h64_b4_l131072 all sequences", e)


@pytest.mark.parametrize("lens", [[4096] * 8, [1, 31, 32, 33, 700, 5000, 64, 20000]])
def test_split_count_invariance(m, lens):
    """The split-KV partition is free: the same call with 8, 40, 256 and 1024
    workgroups (one to hundreds of pieces per sequence, empty workgroups when
    there are fewer tiles than workgroups) matches the oracle each time, and
    the results agree with each other to within bf16 output rounding."""
    cfg = bf16_decode_cfg(seed=18)
    inp = workloads.decode_inputs(cfg, lengths=np.asarray(lens, np.int32))
    ref = oracle_decode(cfg, inp, range(len(lens)))
    outs = {}
    for n in (8, 40, 256, 1024):
        got = gpu_decode(m, dict(cfg, split_workgroups=n), inp)
        assert_bf16(got, ref, f"split_workgroups={n}", per_row_axis=0)
        outs[n] = got
    for n, o in outs.items():
        e = errors(o, outs[256])
        assert e["rel_l2"] <= BF16_REL_L2, f"split_workgroups {n} vs 256: {e}"


def test_decode_zero_query_is_mean_of_latents(m):
    cfg = bf16_decode_cfg(seed=14)
    lens = np.array([1, 77, 3000], np.int32)
    inp = workloads.decode_inputs(cfg, lengths=lens)
    inp.q_nope[:] = 0
    inp.q_rope[:] = 0
    mc = m.MLAConfig.from_dict(cfg)
    o_lat = m.mla_latent_attention(
        mc, m.mla_absorb_query(mc, to_dev(inp.q_nope), to_dev(inp.q_rope), to_dev(inp.w_uk)),
        to_dev(inp.pool), to_dev(inp.block_table), to_dev(inp.seq_lens), int(lens.max()))
    sync()
    got = to_host_f64(o_lat)
    for b, (pages, table, L) in enumerate(compact_sequences(inp, range(3))):
        rows = oracle.gather_sequence(pages, table[0], int(L[0]))
        mean = rows[:, :cfg["kv_lora_rank"]].mean(axis=0)
        assert_bf16(got[b], np.broadcast_to(mean, got[b].shape), f"uniform mean b={b}")


def test_staged_calls_match_decode_and_oracle_latent(m):
    cfg = bf16_decode_cfg(seed=15)
    lens = np.array([5, 64, 700, 2500], np.int32)
    inp = workloads.decode_inputs(cfg, lengths=lens)
    mc = m.MLAConfig.from_dict(cfg)
    qf = m.mla_absorb_query(mc, to_dev(inp.q_nope), to_dev(inp.q_rope), to_dev(inp.w_uk))
    o_lat = m.mla_latent_attention(mc, qf, to_dev(inp.pool), to_dev(inp.block_table),
                                   to_dev(inp.seq_lens), int(lens.max()))
    out = m.mla_output_projection(mc, o_lat, to_dev(inp.w_uv))
    sync()
    full = gpu_decode(m, cfg, inp)
    assert_bf16(to_host_f64(out), full, "staged vs fused")
    # o_lat against the oracle's absorbed latent output
    for b, (pages, table, L) in enumerate(compact_sequences(inp, range(len(lens)))):
        _, ol = oracle.decode(to_f64(inp.q_nope[b:b + 1]), to_f64(inp.q_rope[b:b + 1]),
                              to_f64(inp.w_uk), to_f64(inp.w_uv), pages, table, L, cfg)
        assert_bf16(to_host_f64(o_lat)[b], ol[0], f"o_lat b={b}")
    # absorbed query: scale * log2(e) * [q_nope W_UK | q_rope]
    alpha = oracle.softmax_scale(cfg) / np.log(2.0)
    ql = oracle.absorb_query(to_f64(inp.q_nope), to_f64(inp.w_uk))
    want = alpha * np.concatenate([ql, to_f64(inp.q_rope)], axis=-1)
    assert_bf16(to_host_f64(qf), want, "q_full")


def test_output_projection_many_rows(m):
    """From 256 rows on, the projection takes the 256-row tile GEMM
    (direct-to-LDS stages, transposed accumulators): 700 and 300 rows (a
    ragged last row tile), 64 heads of 512 x 128, against the oracle."""
    cfg = bf16_decode_cfg()
    mc = m.MLAConfig.from_dict(cfg)
    H, R, Dv = cfg["num_heads"], cfg["kv_lora_rank"], cfg["v_dim"]
    w_uv = workloads.normal_tensor((H, R, Dv), seed=53, std=1.0 / np.sqrt(R))
    for n, seed in ((700, 51), (300, 52)):
        o_lat = workloads.normal_tensor((n, H, R), seed=seed)
        got = m.mla_output_projection(mc, to_dev(o_lat), to_dev(w_uv))
        sync()
        ref = oracle.project_output(to_f64(o_lat), to_f64(w_uv))
        assert_bf16(to_host_f64(got), ref, f"projection n={n}", per_row_axis=0)


def test_page_permutation_invariance_and_determinism(m):
    """Same logical rows in two physical page orders give bitwise-equal
    outputs, and a repeated call is bitwise identical."""
    cfg = bf16_decode_cfg(seed=16)
    lens = np.array([130, 3000, 64, 1], np.int32)
    inp = workloads.decode_inputs(cfg, lengths=lens)
    a = gpu_decode(m, cfg, inp)
    a2 = gpu_decode(m, cfg, inp)
    np.testing.assert_array_equal(a, a2)
    rng = np.random.default_rng(0)
    perm = rng.permutation(inp.pool.shape[0])       # new physical index of each page
    pool2 = np.empty_like(inp.pool)
    pool2[perm] = inp.pool
    table2 = inp.block_table.copy()
    for b, L in enumerate(lens):
        n = -(-int(L) // 64)
        table2[b, :n] = perm[inp.block_table[b, :n]]
    inp2 = dataclasses.replace(inp, pool=pool2, block_table=table2)
    b_ = gpu_decode(m, cfg, inp2)
    np.testing.assert_array_equal(a, b_)


def test_garbage_beyond_sequence_end_is_ignored(m):
    """Unused slots of a sequence's last page hold NaN; they must not leak."""
    cfg = bf16_decode_cfg(seed=17)
    lens = np.array([65, 1, 200], np.int32)
    inp = workloads.decode_inputs(cfg, lengths=lens)
    ref = oracle_decode(cfg, inp, range(3))
    nan_bits = np.uint16(0x7FC0)
    for b, L in enumerate(lens):
        last = inp.block_table[b, (int(L) - 1) // 64]
        inp.pool[last, (int(L) - 1) % 64 + 1:] = nan_bits
    got = gpu_decode(m, cfg, inp)
    assert_bf16(got, ref, "NaN padding")


@pytest.mark.parametrize("filler", [-1, 1 << 30, "pool_size"])
def test_unused_block_table_entries_outside_the_pool(m, filler):
    """Block-table entries past each sequence's pages point outside the pool
    (negative, huge, or exactly the pool size).  The equal-length guess of the
    decode prologue (every sequence 4096 tokens long) lands on such entries
    for the short sequences: the guessed tiles must be skipped and the queries
    staged for the guess replaced, with no effect on the output."""
    cfg = bf16_decode_cfg(seed=19)
    lens = np.array([4096, 64, 2000, 4096, 33, 4096, 1, 700], np.int32)
    inp = workloads.decode_inputs(cfg, lengths=lens)
    bs = inp.pool.shape[1]
    fill = inp.pool.shape[0] if filler == "pool_size" else filler
    for b, L in enumerate(lens):
        inp.block_table[b, -(-int(L) // bs):] = fill
    got = gpu_decode(m, cfg, inp)
    ref = oracle_decode(cfg, inp, range(len(lens)))
    assert_bf16(got, ref, f"unused entries = {filler}", per_row_axis=0)


# ---------------------------------------------------------------------------
# bf16 prefill
# ---------------------------------------------------------------------------
def _pool_rows(pool_np, table, L):
    bs = pool_np.shape[1]
    j = np.arange(L)
    return pool_np[table[j // bs], j % bs]


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits): 2^(e - 7) for
    |v| in [2^e, 2^(e+1))."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_rows(got, ref, what):
    """Stored bf16 rows: each element within one bf16 step of the oracle's
    stored value (the two sides round different float32/float64 sums, so a
    value next to a rounding boundary can land one step apart; the step is
    taken at the larger of the two magnitudes), or within 1e-4 absolute where
    the value is near zero (the float32 sum over d_model products carries
    ~1e-5 absolute error before the store); plus the bf16 relative-L2 bar."""
    bound = np.maximum(bf16_ulp(np.maximum(np.abs(got), np.abs(ref))), 1e-4)
    worst = np.max(np.abs(got - ref) / bound)
    assert worst <= 1.0, f"{what}: worst element at {worst:.2f} of its bound"
    e = assert_bf16(got, ref, what)
    print(what, "exact fraction", float(np.mean(got == ref)), e)


@pytest.mark.parametrize("d_model,n", [(7168, 300), (640, 129)])
def test_cache_append_bf16_rows(m, d_model, n):
    """mla_cache_append in bf16 (the down-projection with RMSNorm, RoPE and
    the store fused in one launch): panels of 128 tokens with a ragged last
    one, permuted slots, every 7th token skipped, jittered gains, positions
    out of order; every written row within one bf16 step of the oracle,
    skipped and unused slots untouched."""
    import torch
    rng = np.random.default_rng(d_model + n)
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=d_model, q_lora_rank=0)
    mc = m.MLAConfig.from_dict(cfg)
    R, Dr, bs = cfg["kv_lora_rank"], cfg["rope_dim"], cfg["block_size"]
    x = workloads.normal_tensor((n, d_model), seed=d_model + 1)
    w_dkv = workloads.normal_tensor((d_model, R + Dr), seed=d_model + 2, std=1.0 / np.sqrt(d_model))
    gain = (1.0 + 0.1 * rng.standard_normal(R)).astype(np.float32)
    pos = rng.permutation(4 * n)[:n].astype(np.int32)
    nb = -(-2 * n // bs)
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    slots[::7] = -1
    pool = torch.full((nb, bs, R + Dr), 7.0, dtype=torch.bfloat16, device="cuda")
    m.mla_cache_append(mc, to_dev(x), to_dev(w_dkv), to_dev(gain), to_dev(pos), to_dev(slots),
                       pool)
    sync()
    flat = to_host_f64(pool).reshape(nb * bs, R + Dr)
    keep = slots >= 0
    w64 = {"w_dkv": to_f64(w_dkv), "kv_norm_w": gain.astype(np.float64)}
    ref = oracle.append_rows(to_f64(x)[keep], pos[keep], w64, cfg, storage="bf16")
    check_rows(flat[slots[keep]], ref, f"append d_model {d_model}")
    untouched = np.setdiff1d(np.arange(nb * bs), slots[keep])
    assert np.all(flat[untouched] == 7.0)


def test_prefill_small_bf16_with_query_rank_and_continuation(m):
    import torch
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=640, q_lora_rank=128,
               seed=31)
    mc = m.MLAConfig.from_dict(cfg)
    inp = workloads.prefill_inputs(cfg, q_len=150, batch=2, gain_jitter=0.1)
    w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
    w64 = {k: (None if v is None else to_f64(v)) for k, v in vars(inp.weights).items()}
    pool = torch.zeros((inp.num_blocks, 64, mc.row), dtype=torch.bfloat16, device="cuda")
    table = to_dev(inp.block_table)
    x = to_dev(inp.x)
    # first 100 tokens, then 50 more continuing at position 100
    out1 = m.mla_prefill(mc, x[:, :100].contiguous(), w, pool, table,
                         torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
    out2 = m.mla_prefill(mc, x[:, 100:].contiguous(), w, pool, table,
                         torch.full((2,), 100, dtype=torch.int32, device="cuda"), 100)
    sync()
    got = np.concatenate([to_host_f64(out1), to_host_f64(out2)], axis=1)
    pool_np = to_host_f64(pool)
    for b in range(2):
        ref, rows = oracle.layer_forward(to_f64(inp.x[b]), w64, cfg, storage="bf16")
        g_rows = _pool_rows(pool_np, inp.block_table[b], 150)
        check_rows(g_rows, rows, f"small prefill rows b={b}")
        assert_bf16(got[b], ref, f"small prefill b={b}", per_row_axis=0)


def test_prefill_per_head_path_with_continuation(m):
    """Spans long enough for the per-head key/value path (600 new tokens,
    then 300 more at position 600): partial query blocks, keys from earlier
    calls through permuted pages, jittered gains; outputs and cache rows
    against the oracle."""
    import torch
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=640, q_lora_rank=128,
               seed=41)
    mc = m.MLAConfig.from_dict(cfg)
    inp = workloads.prefill_inputs(cfg, q_len=900, batch=2, gain_jitter=0.1)
    w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
    w64 = {k: (None if v is None else to_f64(v)) for k, v in vars(inp.weights).items()}
    pool = torch.zeros((inp.num_blocks, 64, mc.row), dtype=torch.bfloat16, device="cuda")
    table = to_dev(inp.block_table)
    x = to_dev(inp.x)
    out1 = m.mla_prefill(mc, x[:, :600].contiguous(), w, pool, table,
                         torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
    out2 = m.mla_prefill(mc, x[:, 600:].contiguous(), w, pool, table,
                         torch.full((2,), 600, dtype=torch.int32, device="cuda"), 600)
    sync()
    got = np.concatenate([to_host_f64(out1), to_host_f64(out2)], axis=1)
    pool_np = to_host_f64(pool)
    for b in range(2):
        ref, rows = oracle.layer_forward(to_f64(inp.x[b]), w64, cfg, storage="bf16")
        check_rows(_pool_rows(pool_np, inp.block_table[b], 900), rows, f"rows b={b}")
        assert_bf16(got[b], ref, f"per-head path b={b}", per_row_axis=0)


@pytest.mark.parametrize("heads,t1,t2,bs", [(64, 77, 51, 64), (32, 93, 30, 128), (64, 1, 1, 64)])
def test_prefill_latent_form_edges(m, heads, t1, t2, bs):
    """Attention on the latent rows forced: token counts that leave a partial
    block of query tokens (2 per workgroup at 64 heads, 4 at 32), a
    continuation whose first position is not on a 32-key tile boundary, and
    128-row pages; outputs and cache rows of both calls against the oracle."""
    import torch
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=640, q_lora_rank=128,
               num_heads=heads, block_size=bs, prefill_attention="latent", seed=51 + heads)
    mc = m.MLAConfig.from_dict(cfg)
    T = t1 + t2
    inp = workloads.prefill_inputs(cfg, q_len=T, batch=2, gain_jitter=0.1)
    w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
    w64 = {k: (None if v is None else to_f64(v)) for k, v in vars(inp.weights).items()}
    pool = torch.zeros((inp.num_blocks, bs, mc.row), dtype=torch.bfloat16, device="cuda")
    table = to_dev(inp.block_table)
    x = to_dev(inp.x)
    out1 = m.mla_prefill(mc, x[:, :t1].contiguous(), w, pool, table,
                         torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
    out2 = m.mla_prefill(mc, x[:, t1:].contiguous(), w, pool, table,
                         torch.full((2,), t1, dtype=torch.int32, device="cuda"), t1)
    sync()
    got = np.concatenate([to_host_f64(out1), to_host_f64(out2)], axis=1)
    pool_np = to_host_f64(pool)
    for b in range(2):
        ref, rows = oracle.layer_forward(to_f64(inp.x[b]), w64, cfg, storage="bf16")
        check_rows(_pool_rows(pool_np, inp.block_table[b], T), rows, f"rows b={b}")
        assert_bf16(got[b], ref, f"latent form H={heads} b={b}", per_row_axis=0)


def test_prefill_latent_form_large_late_score(m):
    """Token 80's hidden state scaled by 50: its rope key (not normalised)
    gives later queries scores up to about 150 (log2 units) above the maximum
    of their first key tile, so weights taken relative to that maximum would
    overflow; the latent-form kernel then takes those workgroups' key range a
    second time with the row maxima as references.  Both attention forms run.
    Scores this large carry absolute errors of about |s| 2^-8 from the bf16
    queries and rows, so the bound here is rel-L2 <= 1e-2, max abs <= 0.25,
    cosine >= 0.9999, and the latent form within 25 % of the per-head form's
    rel-L2 (the per-head kernel rescales its output lazily instead)."""
    import torch
    T = 150
    errs = {}
    for form in ("latent", "per_head"):
        cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=640, q_lora_rank=128,
                   prefill_attention=form, seed=61)
        mc = m.MLAConfig.from_dict(cfg)
        inp = workloads.prefill_inputs(cfg, q_len=T, batch=2)
        xs = to_f64(inp.x)
        xs[:, 80] *= 50.0
        x_big = workloads.bf16_bits(xs.astype(np.float32))
        w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
        w64 = {k: (None if v is None else to_f64(v)) for k, v in vars(inp.weights).items()}
        pool = torch.zeros((inp.num_blocks, 64, mc.row), dtype=torch.bfloat16, device="cuda")
        out = m.mla_prefill(mc, to_dev(x_big), w, pool, to_dev(inp.block_table),
                            torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
        sync()
        got = to_host_f64(out)
        assert np.all(np.isfinite(got)), f"{form}: non-finite output"
        ref = np.stack([oracle.layer_forward(to_f64(x_big[b]), w64, cfg, storage="bf16")[0]
                        for b in range(2)])
        e = errors(got, ref)
        print("large late score", form, e)
        assert e["rel_l2"] <= 1e-2 and e["max_abs"] <= 0.25 and e["cosine"] >= 0.9999, (form, e)
        errs[form] = e["rel_l2"]
    assert errs["latent"] <= 1.25 * errs["per_head"] + 1e-4, errs


@pytest.mark.parametrize("form", ["auto", "latent"])
def test_prefill_d7168_b2_t4096_full(m, form):
    """Full-size prefill (d_model 7168, q rank 1536, 2 x 4096 new tokens):
    every appended cache row checked, outputs on the first and last page of
    query rows and three middle rows of both sequences.  "auto" takes the
    form with fewer FLOPs (per-head keys and values at this size), "latent"
    forces attention on the latent rows (the absorbed form)."""
    import torch
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], prefill_attention=form)
    mc = m.MLAConfig.from_dict(cfg)
    assert m.mla_prefill_attention_form(mc, cfg["q_len"], 0) == (
        "per_head" if form == "auto" else "latent")
    inp = workloads.prefill_inputs(cfg)
    w = {k: to_dev(v) for k, v in vars(inp.weights).items() if v is not None}
    pool = torch.zeros((inp.num_blocks, 64, mc.row), dtype=torch.bfloat16, device="cuda")
    out = m.mla_prefill(mc, to_dev(inp.x), w, pool, to_dev(inp.block_table),
                        torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
    sync()
    w64 = {k: (None if v is None else to_f64(v)) for k, v in vars(inp.weights).items()}
    pool_np = to_host_f64(pool)
    T = cfg["q_len"]
    # the first and last page of each sequence in full, plus the middle
    sample = list(range(64)) + [1000, 2047, 2048] + list(range(T - 64, T))
    for b in range(2):
        x64 = to_f64(inp.x[b])
        rows = oracle.append_rows(x64, np.arange(T), w64, cfg, storage="bf16")
        g_rows = _pool_rows(pool_np, inp.block_table[b], T)
        check_rows(g_rows, rows, f"cache rows b={b}")
        ref = oracle.attend_tokens(x64[sample], np.array(sample), w64, cfg, rows, q_block=64)
        got = to_host_f64(out[b, sample])
        e = assert_bf16(got, ref, f"prefill {form} b={b}", per_row_axis=0)
        print("prefill_d7168_b2_t4096", form, b, e)


# ---------------------------------------------------------------------------
# output gate and W_O ("GatedMLA" docs, "Output projection and optional gate")
# ---------------------------------------------------------------------------
def gate_inputs(cfg, n, seed):
    M, HV = cfg["d_model"], cfg["num_heads"] * cfg["v_dim"]
    dt = cfg["dtype"]
    return (workloads.normal_tensor((n, M), seed, dt),
            workloads.normal_tensor((n, cfg["num_heads"], cfg["v_dim"]), seed + 1, dt),
            workloads.normal_tensor((M, HV), seed + 2, dt, std=1.0 / np.sqrt(M)),
            workloads.normal_tensor((HV, M), seed + 3, dt, std=1.0 / np.sqrt(HV)))


def run_gate(m, cfg, n, seed, gated):
    mc = m.MLAConfig.from_dict(cfg)
    x, h, w_g, w_o = gate_inputs(cfg, n, seed)
    got = m.mla_output_gate_projection(mc, to_dev(x), to_dev(h), to_dev(w_o),
                                       w_g=to_dev(w_g) if gated else None)
    sync()
    ref = oracle.output_gate_projection(to_f64(h), to_f64(x), to_f64(w_o),
                                        to_f64(w_g) if gated else None)
    return to_host_f64(got), ref


def test_output_gate_tiny_fp32(m):
    """float32, d_model 64, 4 heads of 16: with and without the gate."""
    cfg = workloads.WORKLOADS["tiny_fp32"]
    for gated in (True, False):
        got, ref = run_gate(m, cfg, 65, 71, gated)
        assert_f32(got, ref, f"gate={gated}")


def test_output_gate_bf16_decode_rows(m):
    """bf16, d_model 7168, 64 heads of 128 (the prefill workload's widths), 32
    rows as in a decode step: the small-row GEMM with the gate fused into its
    epilogue, then W_O."""
    cfg = workloads.WORKLOADS["prefill_d7168_b2_t4096"]
    for gated in (True, False):
        got, ref = run_gate(m, cfg, 32, 81, gated)
        assert_bf16(got, ref, f"gate={gated}", per_row_axis=0)


def test_output_gate_bf16_short_k(m):
    """bf16, 300 rows, d_model 352, 4 heads of 128: both products have
    K <= 512, so they take the two-workgroups-per-CU tile launch (256 x 128
    tiles) with a ragged last row tile; x W_G carries the gate in its
    epilogue, and W_O's 352 columns leave a partial column tile."""
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=352, q_lora_rank=0,
               kv_lora_rank=256, num_heads=4)
    for gated in (True, False):
        got, ref = run_gate(m, cfg, 300, 97, gated)
        assert_bf16(got, ref, f"gate={gated}", per_row_axis=0)


def test_output_gate_bf16_many_rows(m):
    """bf16, 600 rows (the 256-row tile GEMM, ragged last row tile), d_model
    1024, 16 heads of 128."""
    cfg = dict(workloads.WORKLOADS["prefill_d7168_b2_t4096"], d_model=1024, q_lora_rank=0,
               num_heads=16)
    for gated in (True, False):
        got, ref = run_gate(m, cfg, 600, 91, gated)
        assert_bf16(got, ref, f"gate={gated}", per_row_axis=0)
