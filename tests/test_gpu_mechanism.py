"""Narrow latents and shared W_UK / W_UV on the GPU, through the C ABI,
against the oracle.

The tutorial's mechanism experiment ("ARCH-MLA. Multihead Latent Attention",
5.1) runs 16 query heads over 4 rebuilt key/value heads, head width 64,
latent 256, rope 64, bf16, at history lengths 512, 2048 and 8192.  Here the
same widths go through mla_decode (kv_groups = 4: heads 4g..4g+3 share
W_UK[g] and W_UV[g]); the oracle expands the 4 matrices to 16 heads
(``oracle.head_matrices``, pinned against torch's grouped-query SDPA).
Tolerances: the bf16 bars (rel-L2 <= 5e-3, max abs <= 2e-2).
"""
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


def run_decode(m, cfg, inp):
    import torch
    mc = m.MLAConfig.from_dict(cfg)
    B, L = len(inp.seq_lens), int(inp.seq_lens.max())
    ws = torch.zeros(m.mla_decode_workspace_size(mc, B, L), dtype=torch.uint8, device="cuda")
    out = m.mla_decode(mc, to_dev(inp.q_nope), to_dev(inp.q_rope), to_dev(inp.w_uk),
                       to_dev(inp.w_uv), to_dev(inp.pool), to_dev(inp.block_table),
                       to_dev(inp.seq_lens), L, workspace=ws)
    sync()
    return to_host_f64(out)


def oracle_decode(cfg, inp, ids, latent=False):
    outs = []
    for b, (pages, table, lens) in zip(ids, compact_sequences(inp, ids)):
        o, ol = oracle.decode(workloads.to_f64(inp.q_nope[b:b + 1]),
                              workloads.to_f64(inp.q_rope[b:b + 1]), workloads.to_f64(inp.w_uk),
                              workloads.to_f64(inp.w_uv), pages, table, lens, cfg)
        outs.append(ol[0] if latent else o[0])
    return np.stack(outs)


def check(m, cfg, lengths=None, sample=None, seed=None):
    lens = None if lengths is None else np.asarray(lengths, np.int32)
    inp = workloads.decode_inputs(cfg, seed=seed, lengths=lens)
    got = run_decode(m, cfg, inp)
    ids = list(range(len(inp.seq_lens))) if sample is None else list(sample)
    return assert_bf16(got[ids], oracle_decode(cfg, inp, ids),
                       f"{cfg.get('num_heads')} heads {list(inp.seq_lens[:8])}", per_row_axis=0)


@pytest.mark.parametrize("L", [512, 2048, 8192])
def test_mechanism_widths_decode(m, L):
    """16 heads sharing 4 W_UK / W_UV, latent 256, rope 64, head width 64."""
    e = check(m, workloads.WORKLOADS[f"mechanism_h16_g4_r256_l{L}"])
    print(f"mechanism_h16_g4_r256_l{L}", e)


def test_narrow_latent_paged_ragged_two_head_blocks(m):
    """32 heads (two blocks of 16) sharing 8 matrices, 16-token pages in a
    permuted pool, lengths at tile and page edges, one-token sequences."""
    cfg = dict(workloads.WORKLOADS["mechanism_h16_g4_r256_l512"], num_heads=32, kv_groups=8,
               block_size=16, paged=True, lengths="explicit", seed=71)
    check(m, cfg, [1, 2, 15, 16, 17, 63, 64, 65, 127, 129, 1000, 3001])


def test_narrow_latent_r128_per_head_weights(m):
    """kv_lora_rank 128, a W_UK / W_UV per head (kv_groups 0), 48-token pages."""
    cfg = dict(workloads.WORKLOADS["mechanism_h16_g4_r256_l512"], kv_lora_rank=128, kv_groups=0,
               qk_nope_dim=128, v_dim=128, block_size=48, paged=True, lengths="explicit",
               seed=72)
    check(m, cfg, [1, 47, 48, 49, 300, 2500])


def test_narrow_latent_attention_o_lat(m):
    """mla_latent_attention on the narrow-latent kernels: o_lat against the
    oracle's softmax-weighted latent rows (absorbed query from
    mla_absorb_query with shared W_UK)."""
    import torch
    cfg = dict(workloads.WORKLOADS["mechanism_h16_g4_r256_l2048"], lengths="explicit",
               paged=True, seed=73)
    inp = workloads.decode_inputs(cfg, lengths=np.array([2048, 700, 65], np.int32))
    mc = m.MLAConfig.from_dict(cfg)
    qf = m.mla_absorb_query(mc, to_dev(inp.q_nope), to_dev(inp.q_rope), to_dev(inp.w_uk))
    ws = torch.zeros(m.mla_decode_workspace_size(mc, 3, 2048), dtype=torch.uint8, device="cuda")
    o_lat = m.mla_latent_attention(mc, qf, to_dev(inp.pool), to_dev(inp.block_table),
                                   to_dev(inp.seq_lens), 2048, workspace=ws)
    sync()
    ref = oracle_decode(cfg, inp, [0, 1, 2], latent=True)
    assert_bf16(to_host_f64(o_lat), ref, "narrow o_lat", per_row_axis=0)


def test_shared_weights_on_the_tuned_kernels(m):
    """kv_groups on the kv_lora_rank 512 kernels: 64 heads sharing 8 W_UK /
    W_UV (grouped absorb, merge to o_lat, grouped W_UV)."""
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=64, kv_groups=8,
               lengths="explicit", seed=74)
    check(m, cfg, [1, 64, 65, 1000, 4097])


def test_shared_weights_many_rows_r512(m):
    """kv_groups with more than 32 rows: 64 heads sharing 8 matrices at
    kv_lora_rank 512 over 72 sequences, so the absorption and the W_UV product
    run as per-group batched GEMMs (batch stride 0 on the shared matrix) with
    the scaled q_rope copy as its own pass."""
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=64, kv_groups=8,
               lengths="explicit", seed=75)
    rng = np.random.default_rng(75)
    check(m, cfg, rng.integers(1, 1500, size=72), sample=[0, 1, 35, 70, 71])


def test_shared_weights_many_rows_narrow(m):
    """The mechanism widths (16 heads, 4 shared matrices, latent 256) over 64
    sequences: per-group GEMMs instead of the small-row kernels."""
    cfg = dict(workloads.WORKLOADS["mechanism_h16_g4_r256_l512"], lengths="explicit",
               paged=True, seed=76)
    rng = np.random.default_rng(76)
    check(m, cfg, rng.integers(1, 1200, size=64))


def test_staged_calls_refuse_what_they_lack(m):
    """Split partials exist for the 512-wide kernels only, and their merge
    applies per-head W_UV only: both refuse before any launch."""
    import torch
    cfg = workloads.WORKLOADS["mechanism_h16_g4_r256_l512"]
    mc = m.MLAConfig.from_dict(cfg)
    inp = workloads.decode_inputs(cfg)
    ws = torch.zeros(m.mla_decode_workspace_size(mc, 1, 512), dtype=torch.uint8, device="cuda")
    qf = torch.zeros((1, 16, 320), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MLAError) as e:
        m.mla_attention_partials(mc, qf, to_dev(inp.pool), to_dev(inp.block_table),
                                 to_dev(inp.seq_lens), 512, ws)
    assert e.value.status == 2
    big = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=64, kv_groups=8)
    mb = m.MLAConfig.from_dict(big)
    wsb = torch.zeros(m.mla_decode_workspace_size(mb, 1, 64), dtype=torch.uint8, device="cuda")
    w_uv = torch.zeros((8, 512, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MLAError) as e:
        m.mla_combine_output(mb, 1, 64, wsb, w_uv=w_uv)
    assert e.value.status == 2


# ---------------------------------------------------------------------------
# The reconstruction form (decode_attention "per_head"): per-head keys and
# values rebuilt from the latent rows for the step, then grouped attention,
# against the oracle's naive path (keys and values rebuilt in float64).
# ---------------------------------------------------------------------------
def check_per_head(m, cfg, lengths=None, seed=None):
    cfg = dict(cfg, decode_attention="per_head")
    lens = None if lengths is None else np.asarray(lengths, np.int32)
    inp = workloads.decode_inputs(cfg, seed=seed, lengths=lens)
    got = run_decode(m, cfg, inp)
    ids = list(range(len(inp.seq_lens)))
    refs = []
    for b, (pages, table, ln) in zip(ids, compact_sequences(inp, ids)):
        o, _ = oracle.decode(workloads.to_f64(inp.q_nope[b:b + 1]),
                             workloads.to_f64(inp.q_rope[b:b + 1]), workloads.to_f64(inp.w_uk),
                             workloads.to_f64(inp.w_uv), pages, table, ln, cfg, path="naive")
        refs.append(o[0])
    e = assert_bf16(got, np.stack(refs), f"per-head {list(inp.seq_lens[:8])}", per_row_axis=0)
    # the latent form of the same step agrees with it to the same bar
    lat = run_decode(m, dict(cfg, decode_attention="latent"), inp)
    assert_bf16(got, lat, "per-head vs latent form", per_row_axis=0)
    return e


@pytest.mark.parametrize("L", [512, 2048, 8192])
def test_mechanism_widths_per_head_form(m, L):
    """The tutorial's reconstruction leg at its widths: 16 query heads over 4
    rebuilt key/value heads of width 64 (rope 64), latent 256."""
    e = check_per_head(m, workloads.WORKLOADS[f"mechanism_h16_g4_r256_l{L}"])
    print(f"per-head form mechanism_h16_g4_r256_l{L}", e)


def test_per_head_form_paged_ragged(m):
    """Several sequences of ragged lengths (1 token up to past a tile) over
    16-token pages of a permuted pool; 32 heads in 8 groups; latent 128."""
    cfg = dict(workloads.WORKLOADS["mechanism_h16_g4_r256_l512"], num_heads=32, kv_groups=8,
               kv_lora_rank=128, block_size=16, paged=True, lengths="explicit", seed=81)
    check_per_head(m, cfg, [1, 2, 15, 16, 17, 63, 64, 65, 129, 700])


def test_per_head_form_one_head_per_group_and_rank_512(m):
    """32 heads with their own matrices (no sharing) over latent-512 rows."""
    cfg = dict(workloads.WORKLOADS["mechanism_h16_g4_r256_l512"], num_heads=32, kv_groups=32,
               kv_lora_rank=512, lengths="explicit", paged=True, seed=83)
    check_per_head(m, cfg, [300, 1, 1024, 77])
