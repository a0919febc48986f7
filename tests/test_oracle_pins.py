"""Pins for the CPU oracle: it is checked against things other than itself.

Each check ties an oracle function to a fixed fact: a value the pages print
(tests/golden), a closed form, an invariant, a library routine (torch CPU
SDPA, torch's bf16 cast) or brute-force loops written independently here.
The last section plants plausible mistakes in copies of oracle functions
and shows that these pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import ledger
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


TINY = dict(num_heads=3, kv_lora_rank=6, rope_dim=4, qk_nope_dim=5, v_dim=2, d_model=8,
            rms_eps=1e-6, rope_theta=10000.0)


def tiny_weights(seed=0, with_q_rank=False, cfg=TINY):
    r = rng(seed)
    M, H, R, Dr, Dn, Dv = (cfg[k] for k in ("d_model", "num_heads", "kv_lora_rank",
                                            "rope_dim", "qk_nope_dim", "v_dim"))
    w = dict(w_dkv=r.standard_normal((M, R + Dr)) / math.sqrt(M),
             kv_norm_w=1.0 + 0.2 * r.standard_normal(R),
             w_uk=r.standard_normal((H, Dn, R)) / math.sqrt(R),
             w_uv=r.standard_normal((H, R, Dv)) / math.sqrt(R))
    if with_q_rank:
        Rq = 5
        w.update(w_dq=r.standard_normal((M, Rq)) / math.sqrt(M),
                 q_norm_w=1.0 + 0.2 * r.standard_normal(Rq),
                 w_uq=r.standard_normal((Rq, H * (Dn + Dr))) / math.sqrt(Rq))
    else:
        w.update(w_q=r.standard_normal((M, H * (Dn + Dr))) / math.sqrt(M))
    return w


# ===========================================================================
# 1. Ledger: values printed on the pages
# ===========================================================================
def test_ledger_tutorial_step4_values():
    g = golden("ledger_tutorial_step4.json")
    rep = ledger.compare_states(g["config"])
    assert rep["bytes_per_token"] == g["bytes_per_token"]
    assert rep["ratio_vs_mha"] == g["ratio_vs_mha"]
    assert rep["most_compact"] == g["most_compact"]
    bad = dict(g["config"], **g["rejected_config_override"])
    with pytest.raises(ValueError):
        ledger.check_state_config(bad)
    with pytest.raises(ValueError):
        ledger.state_bytes("mqa-typo", g["config"])
    for field in ledger.FIELDS:
        with pytest.raises(ValueError):
            ledger.check_state_config(dict(g["config"], **{field: 0}))


def test_ledger_kimi_scale_table():
    g = golden("ledger_kimi_scale.json")
    cfg = g["config"]
    for mode, n in g["elements_per_token"].items():
        assert ledger.state_elements(mode if mode != "gqa8" else "gqa", cfg) == n
    assert ledger.state_bytes("mla", cfg) == g["mla_bf16_bytes_per_token"]
    assert round(ledger.state_elements("mha", cfg) / ledger.state_elements("mla", cfg)) == g["mha_over_mla_approx"]
    assert ledger.state_elements("mha", cfg) / ledger.state_elements("gqa", cfg) == g["gqa_over_mha_approx"]


def test_ledger_tutorial_experiment_reductions():
    g = golden("ledger_tutorial_experiment.json")
    rep = ledger.compare_states(g["config"])
    for mode, red in g["reduction_vs_mha"].items():
        assert 1.0 - rep["ratio_vs_mha"][mode] == pytest.approx(red, abs=0)


# ===========================================================================
# 2. RoPE, RMSNorm and storage rounding: closed forms and library routines
# ===========================================================================
def test_rope_position_zero_is_identity():
    x = rng(1).standard_normal((1, 3, 8))
    np.testing.assert_array_equal(oracle.apply_rope(x, [0]), x)


def test_rope_two_dims_is_rotation_by_position_radians():
    for p in (1, 2, 7, 100):
        y = oracle.apply_rope(np.array([[1.0, 0.0], [0.0, 1.0]]), [p, p])
        np.testing.assert_allclose(y[0], [math.cos(p), math.sin(p)], rtol=0, atol=1e-15)
        np.testing.assert_allclose(y[1], [-math.sin(p), math.cos(p)], rtol=0, atol=1e-15)


def test_rope_half_split_pairing_closed_form():
    # Dr = 4, theta 10000: pair (0, 2) turns at 1 rad/position, pair (1, 3) at 0.01.
    p = 3
    e = np.eye(4)
    y = oracle.apply_rope(e, [p] * 4)
    np.testing.assert_allclose(y[0], [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    np.testing.assert_allclose(y[1], [0, math.cos(0.01 * p), 0, math.sin(0.01 * p)], atol=1e-15)
    np.testing.assert_allclose(y[2], [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)


def test_rope_norm_and_relative_position():
    r = rng(2)
    q, k = r.standard_normal(64), r.standard_normal(64)
    for m, n, d in ((5, 2, 11), (100, 37, 1000), (4095, 0, 7)):
        qm = oracle.apply_rope(q[None], [m])[0]
        assert np.linalg.norm(qm) == pytest.approx(np.linalg.norm(q), rel=1e-14)
        a = qm @ oracle.apply_rope(k[None], [n])[0]
        b = oracle.apply_rope(q[None], [m + d])[0] @ oracle.apply_rope(k[None], [n + d])[0]
        assert a == pytest.approx(b, rel=1e-9, abs=1e-9)


def test_rms_norm_closed_forms():
    r = rng(3)
    x = r.standard_normal((5, 512))
    y = oracle.rms_norm(x, np.ones(512), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rms_norm(7.5 * x, np.ones(512), eps=0.0), y, rtol=1e-13)
    g = r.standard_normal(512)
    np.testing.assert_allclose(oracle.rms_norm(x, g, eps=0.0), y * g, rtol=1e-13)
    # eps enters under the root: a constant row c gives c / sqrt(c^2 + eps)
    c = 1e-3
    np.testing.assert_allclose(oracle.rms_norm(np.full((1, 4), c), np.ones(4), eps=1e-6),
                               c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_store_round_against_torch_and_ties():
    torch = pytest.importorskip("torch")
    x = rng(4).standard_normal(20000) * np.exp(rng(5).uniform(-20, 20, 20000))
    ours = oracle.store_round(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])
    np.testing.assert_array_equal(oracle.store_round(ties, "bf16"), [1.0, 1 + 2 ** -6, -1.0])
    np.testing.assert_array_equal(oracle.store_round(x, "f32"), x.astype(np.float32).astype(np.float64))


# ===========================================================================
# 3. Attention: library routine, identities, closed forms
# ===========================================================================
def _sdpa_vs_naive(naive_fn, cfg=TINY, T=7, seed=6):
    torch = pytest.importorskip("torch")
    r = rng(seed)
    H, R, Dr, Dn, Dv = (cfg[k] for k in ("num_heads", "kv_lora_rank", "rope_dim", "qk_nope_dim", "v_dim"))
    w = tiny_weights(seed)
    c, kr = r.standard_normal((T, R)), r.standard_normal((T, Dr))
    qn, qr = r.standard_normal((T, H, Dn)), r.standard_normal((T, H, Dr))
    k, v = oracle.reconstruct_kv(c, kr, w["w_uk"], w["w_uv"])
    q = np.concatenate([qn, qr], axis=-1)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    ref = ref[0].numpy().transpose(1, 0, 2)
    ours = naive_fn(qn, qr, c, kr, w["w_uk"], w["w_uv"], oracle.softmax_scale(cfg), np.arange(T))
    return np.max(np.abs(ours - ref))


def test_naive_matches_torch_cpu_sdpa():
    assert _sdpa_vs_naive(oracle.naive_attention) < 1e-13


def test_shared_rope_key_identical_across_heads():
    r = rng(7)
    w = tiny_weights(7)
    c, kr = r.standard_normal((5, 6)), r.standard_normal((5, 4))
    k, _ = oracle.reconstruct_kv(c, kr, w["w_uk"], w["w_uv"])
    for h in range(1, k.shape[1]):
        np.testing.assert_array_equal(k[:, h, -4:], k[:, 0, -4:])
    np.testing.assert_array_equal(k[:, 0, -4:], kr)


def test_reconstruct_kv_brute_force():
    r = rng(8)
    w = tiny_weights(8)
    c, kr = r.standard_normal((4, 6)), r.standard_normal((4, 4))
    k, v = oracle.reconstruct_kv(c, kr, w["w_uk"], w["w_uv"])
    H, Dn, R = w["w_uk"].shape
    Dv = w["w_uv"].shape[2]
    for j in range(4):
        for h in range(H):
            for d in range(Dn):
                assert k[j, h, d] == pytest.approx(sum(w["w_uk"][h, d, q] * c[j, q] for q in range(R)), abs=1e-14)
            for e in range(Dv):
                assert v[j, h, e] == pytest.approx(sum(c[j, q] * w["w_uv"][h, q, e] for q in range(R)), abs=1e-14)


def _naive_vs_absorbed(absorbed_fn, wd=np.float64, seed=9, cfg=TINY, Tq=4, Tk=9):
    r = rng(seed)
    H, R, Dr, Dn = (cfg[k] for k in ("num_heads", "kv_lora_rank", "rope_dim", "qk_nope_dim"))
    w = tiny_weights(seed, cfg=cfg)
    c, kr = r.standard_normal((Tk, R)), r.standard_normal((Tk, Dr))
    qn, qr = r.standard_normal((Tq, H, Dn)), r.standard_normal((Tq, H, Dr))
    qpos = np.arange(Tk - Tq, Tk)
    s = oracle.softmax_scale(cfg)
    a = oracle.naive_attention(qn, qr, c, kr, w["w_uk"], w["w_uv"], s, qpos, wd=wd)
    b, _ = absorbed_fn(qn, qr, c, kr, w["w_uk"], w["w_uv"], s, qpos, wd=wd)
    return np.max(np.abs(a - b))


def test_naive_equals_absorbed_fp64_and_fp32():
    assert _naive_vs_absorbed(oracle.absorbed_attention) < 1e-13
    assert _naive_vs_absorbed(oracle.absorbed_attention, wd=np.float32) < 1e-5


def test_naive_equals_absorbed_kimi_width():
    cfg = dict(num_heads=4, kv_lora_rank=512, rope_dim=64, qk_nope_dim=128, v_dim=128, d_model=8)
    assert _naive_vs_absorbed(oracle.absorbed_attention, cfg=cfg, Tq=2, Tk=300) < 1e-12
    assert _naive_vs_absorbed(oracle.absorbed_attention, wd=np.float32, cfg=cfg, Tq=2, Tk=300) < 1e-5


def test_length_one_returns_the_single_row():
    r = rng(10)
    c, kr = r.standard_normal((1, 6)), r.standard_normal((1, 4))
    ql, qr = 50 * r.standard_normal((1, 3, 6)), r.standard_normal((1, 3, 4))
    o_lat = oracle.latent_attention(ql, qr, c, kr, 0.3, [0])
    for h in range(3):
        np.testing.assert_array_equal(o_lat[0, h], c[0])
    w = tiny_weights(10)
    out = oracle.project_output(o_lat, w["w_uv"])
    for h in range(3):
        np.testing.assert_allclose(out[0, h], c[0] @ w["w_uv"][h], rtol=1e-15)


def test_zero_query_gives_uniform_mean():
    r = rng(11)
    c, kr = r.standard_normal((37, 6)), r.standard_normal((37, 4))
    o = oracle.latent_attention(np.zeros((1, 3, 6)), np.zeros((1, 3, 4)), c, kr, 1.0, [36])
    np.testing.assert_allclose(o[0], np.broadcast_to(c.mean(axis=0), (3, 6)), rtol=1e-13)


def test_identical_rows_give_that_row():
    r = rng(12)
    row = r.standard_normal(6)
    c = np.broadcast_to(row, (50, 6)).copy()
    kr = r.standard_normal((50, 4))
    o = oracle.latent_attention(r.standard_normal((2, 3, 6)), r.standard_normal((2, 3, 4)),
                                c, kr, 2.0, [10, 49])
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-13)


def test_split_partials_merge_equals_single_softmax():
    r = rng(13)
    L, H, R, Dr = 333, 4, 16, 8
    c, kr = r.standard_normal((L, R)), r.standard_normal((L, Dr))
    ql, qr = 3 * r.standard_normal((H, R)), r.standard_normal((H, Dr))
    ref = oracle.latent_attention(ql[None], qr[None], c, kr, 0.4, [L - 1])[0]
    for chunk in (1, 64, 100, 333, 1000):
        m, l, O = oracle.chunk_partials(ql, qr, c, kr, 0.4, chunk)
        assert m.shape[0] == -(-L // chunk)
        np.testing.assert_allclose(oracle.merge_partials(m, l, O), ref, rtol=1e-12, atol=1e-14)


def test_paged_gather_and_decode_match_contiguous_rows():
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=4, batch=3,
               min_len=1, max_len=200, seed=14)
    inp = workloads.decode_inputs(cfg)
    pool = workloads.to_f64(inp.pool)
    # rebuild each sequence's rows by walking its pages one token at a time
    R = cfg["kv_lora_rank"]
    for b, L in enumerate(inp.seq_lens):
        rows = oracle.gather_sequence(pool, inp.block_table[b], int(L))
        for j in (0, int(L) // 2, int(L) - 1):
            np.testing.assert_array_equal(rows[j], pool[inp.block_table[b, j // 64], j % 64])
    out, o_lat = oracle.decode(workloads.to_f64(inp.q_nope), workloads.to_f64(inp.q_rope),
                               workloads.to_f64(inp.w_uk), workloads.to_f64(inp.w_uv), pool,
                               inp.block_table, inp.seq_lens, cfg)
    # the same sequences laid out contiguously (identity page table)
    for b, L in enumerate(inp.seq_lens):
        rows = oracle.gather_sequence(pool, inp.block_table[b], int(L)).copy()
        ident = np.arange(-(-int(L) // 64))
        cpool = np.zeros((len(ident), 64, rows.shape[1]))
        cpool.reshape(-1, rows.shape[1])[:L] = rows
        o2, ol2 = oracle.decode(workloads.to_f64(inp.q_nope[b:b + 1]), workloads.to_f64(inp.q_rope[b:b + 1]),
                                workloads.to_f64(inp.w_uk), workloads.to_f64(inp.w_uv), cpool,
                                ident[None], np.array([L]), cfg)
        np.testing.assert_array_equal(o2[0], out[b])
    naive, _ = oracle.decode(workloads.to_f64(inp.q_nope), workloads.to_f64(inp.q_rope),
                             workloads.to_f64(inp.w_uk), workloads.to_f64(inp.w_uv), pool,
                             inp.block_table, inp.seq_lens, cfg, path="naive")
    np.testing.assert_allclose(naive, out, rtol=1e-10, atol=1e-12)
    assert o_lat.shape == (3, 4, R)


# ===========================================================================
# 4. Whole layer: brute force, causality, incremental == full
# ===========================================================================
def brute_layer(x, w, cfg, start_pos, prior_rows, q_rank):
    """Independent loop implementation of one layer (tiny sizes only)."""
    H, R, Dr, Dn, Dv, M = (cfg[k] for k in ("num_heads", "kv_lora_rank", "rope_dim",
                                            "qk_nope_dim", "v_dim", "d_model"))
    eps, theta = cfg["rms_eps"], cfg["rope_theta"]
    half = Dr // 2

    def matvec(v, W):
        return [sum(v[i] * W[i][j] for i in range(len(v))) for j in range(len(W[0]))]

    def rot(v, p):
        out = list(v)
        for i in range(half):
            a = p * theta ** (-2.0 * i / Dr)
            out[i] = v[i] * math.cos(a) - v[i + half] * math.sin(a)
            out[i + half] = v[i + half] * math.cos(a) + v[i] * math.sin(a)
        return out

    def norm(v, g):
        ms = sum(t * t for t in v) / len(v)
        return [v[i] / math.sqrt(ms + eps) * g[i] for i in range(len(v))]

    rows = [list(r) for r in prior_rows]
    T = len(x)
    for t in range(T):
        z = matvec(x[t], w["w_dkv"])
        rows.append(norm(z[:R], w["kv_norm_w"]) + rot(z[R:], start_pos + t))
    out = []
    for t in range(T):
        p = start_pos + t
        if q_rank:
            q = matvec(norm(matvec(x[t], w["w_dq"]), w["q_norm_w"]), w["w_uq"])
        else:
            q = matvec(x[t], w["w_q"])
        o_t = []
        for h in range(H):
            qh = q[h * (Dn + Dr):(h + 1) * (Dn + Dr)]
            qn, qr = qh[:Dn], rot(qh[Dn:], p)
            scores = []
            for j in range(p + 1):
                c, kr = rows[j][:R], rows[j][R:]
                kn = [sum(w["w_uk"][h][d][q_] * c[q_] for q_ in range(R)) for d in range(Dn)]
                s = sum(qn[d] * kn[d] for d in range(Dn)) + sum(qr[d] * kr[d] for d in range(Dr))
                scores.append(s / math.sqrt(Dn + Dr))
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = sum(e)
            o_h = [0.0] * Dv
            for j in range(p + 1):
                c = rows[j][:R]
                vj = [sum(c[q_] * w["w_uv"][h][q_][k] for q_ in range(R)) for k in range(Dv)]
                for k in range(Dv):
                    o_h[k] += e[j] / z * vj[k]
            o_t.append(o_h)
        out.append(o_t)
    return np.array(out), np.array(rows[len(prior_rows):])


@pytest.mark.parametrize("q_rank", [False, True])
@pytest.mark.parametrize("path", ["absorbed", "naive"])
def test_layer_forward_brute_force(q_rank, path):
    cfg = dict(TINY)
    w = tiny_weights(15, with_q_rank=q_rank)
    r = rng(16)
    x = r.standard_normal((6, cfg["d_model"]))
    o, rows = oracle.layer_forward(x[:3], w, cfg, path=path)
    bo, brows = brute_layer(x[:3].tolist(), w, cfg, 0, [], q_rank)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rows, brows, rtol=0, atol=1e-12)
    o2, rows2 = oracle.layer_forward(x[3:], w, cfg, path=path, start_pos=3, prior_rows=rows)
    bo2, brows2 = brute_layer(x[3:].tolist(), w, cfg, 3, rows.tolist(), q_rank)
    np.testing.assert_allclose(o2, bo2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rows2, brows2, rtol=0, atol=1e-12)


def test_tiny_layer_brute_force_fp64_all_65_tokens():
    seq = workloads.tiny_sequence(gain_jitter=0.1)
    cfg = dict(seq.cfg, rms_eps=1e-6)
    w = {k: (None if v is None else workloads.to_f64(v)) for k, v in vars(seq.weights).items()}
    x = workloads.to_f64(seq.x[0])
    o, _ = oracle.layer_forward(x, w, cfg)
    idx = [0, 1, 31, 64]
    bo, _ = brute_layer(x.tolist(), w, cfg, 0, [], False)
    np.testing.assert_allclose(o[idx], bo[idx], rtol=0, atol=1e-12)


def test_causality_future_tokens_do_not_matter():
    seq = workloads.tiny_sequence()
    w = {k: (None if v is None else workloads.to_f64(v)) for k, v in vars(seq.weights).items()}
    x = workloads.to_f64(seq.x[0])
    o, _ = oracle.layer_forward(x, w, seq.cfg)
    x2 = x.copy()
    x2[40:] += 5.0 * rng(17).standard_normal(x2[40:].shape)
    o2, _ = oracle.layer_forward(x2, w, seq.cfg)
    np.testing.assert_array_equal(o2[:40], o[:40])
    assert np.max(np.abs(o2[40:] - o[40:])) > 1e-3


@pytest.mark.parametrize("storage", ["f32", "f64"])
def test_incremental_decode_equals_full_forward_fp32(storage):
    """Acceptance criterion of the ticket: cached decode equals the full forward
    within atol 1e-5, here with every definition evaluated in float32."""
    seq = workloads.tiny_sequence()
    w = {k: v for k, v in vars(seq.weights).items()}
    x = seq.x[0]
    full, _ = oracle.layer_forward(x, w, seq.cfg, storage=storage, wd=np.float32)
    inc = oracle.incremental_decode(x, w, seq.cfg, storage=storage, wd=np.float32, n_prefill=64)
    assert np.max(np.abs(full - inc)) <= 1e-5
    inc_all = oracle.incremental_decode(x, w, seq.cfg, storage=storage, wd=np.float32)
    assert np.max(np.abs(full - inc_all)) <= 1e-5
    assert full.dtype == np.float32


def test_decode_of_token_64_uses_stored_rows():
    """Decode at position 64 through the paged-decode function equals row 64
    of the full forward (fp64, rows rounded to bf16 at the store)."""
    seq = workloads.tiny_sequence()
    cfg = seq.cfg
    w = {k: (None if v is None else workloads.to_f64(v)) for k, v in vars(seq.weights).items()}
    x = workloads.to_f64(seq.x[0])
    full, rows = oracle.layer_forward(x, w, cfg, storage="bf16")
    qn, qr = oracle.query_heads(x[64:65], [64], w, cfg)
    pool = np.zeros((2, 64, rows.shape[1]))
    pool.reshape(-1, rows.shape[1])[:65] = rows
    out, _ = oracle.decode(qn, qr, w["w_uk"], w["w_uv"], pool, np.array([[0, 1]]), np.array([65]), cfg)
    np.testing.assert_allclose(out[0], full[64], rtol=1e-13, atol=1e-15)


# ===========================================================================
# 4b. Output gate and W_O ("GatedMLA" docs, "Output projection and optional
#     gate"): sigmoid closed forms, brute-force loops, invariants
# ===========================================================================
def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(oracle.sigmoid(math.log(3.0)) - 0.75) < 1e-15          # 1 / (1 + 1/3)
    z = rng(60).standard_normal(50) * 4
    assert np.max(np.abs(oracle.sigmoid(z) + oracle.sigmoid(-z) - 1.0)) < 1e-15


def brute_gate_projection(h, x, w_o, w_g):
    """out[i][m] = sum_j h[i][j] * gate[i][j] * w_o[j][m], gate = 1 / (1 + e^-(x w_g)),
    with plain loops (gate 1 without w_g)."""
    n, HV, M = len(h), len(w_o), len(w_o[0])
    out = [[0.0] * M for _ in range(n)]
    for i in range(n):
        for j in range(HV):
            g = 1.0
            if w_g is not None:
                z = sum(x[i][k] * w_g[k][j] for k in range(len(x[i])))
                g = 1.0 / (1.0 + math.exp(-z))
            for m in range(M):
                out[i][m] += h[i][j] * g * w_o[j][m]
    return np.array(out)


def gate_case(seed, n=3, H=2, Dv=3, M=5):
    r = rng(seed)
    return (r.standard_normal((n, H, Dv)), r.standard_normal((n, M)),
            r.standard_normal((H * Dv, M)), r.standard_normal((M, H * Dv)))


def test_output_gate_projection_brute_force():
    h, x, w_o, w_g = gate_case(61)
    hf = h.reshape(h.shape[0], -1)
    for g in (w_g, None):
        got = oracle.output_gate_projection(h, x, w_o, g)
        ref = brute_gate_projection(hf.tolist(), x.tolist(), w_o.tolist(),
                                    None if g is None else g.tolist())
        assert np.max(np.abs(got - ref)) < 1e-12


def test_output_gate_invariants():
    h, x, w_o, w_g = gate_case(62)
    plain = oracle.output_gate_projection(h, x, w_o)
    # W_G = 0: sigmoid(0) = 1/2 on every value
    half = oracle.output_gate_projection(h, x, w_o, np.zeros_like(w_g))
    assert np.max(np.abs(half - 0.5 * plain)) < 1e-12
    # the gate reads x only: linear in the head outputs for a fixed x
    a = oracle.output_gate_projection(h, x, w_o, w_g)
    b = oracle.output_gate_projection(2.0 * h, x, w_o, w_g)
    assert np.max(np.abs(b - 2.0 * a)) < 1e-12
    # ... and it does depend on x
    c = oracle.output_gate_projection(h, x + 1.0, w_o, w_g)
    assert np.max(np.abs(c - a)) > 1e-3


# ===========================================================================
# 5. Planted mistakes: a wrong oracle fails the pins above
# ===========================================================================
def test_planted_wrong_scale_is_caught():
    def wrong(qn, qr, c, kr, wuk, wuv, scale, qpos, **kw):
        return oracle.naive_attention(qn, qr, c, kr, wuk, wuv, 1.0 / math.sqrt(qn.shape[-1]), qpos, **kw)
    assert _sdpa_vs_naive(wrong) > 1e-3


def test_planted_off_by_one_mask_is_caught():
    def wrong(qn, qr, c, kr, wuk, wuv, scale, qpos, **kw):
        return oracle.naive_attention(qn, qr, c, kr, wuk, wuv, scale, np.asarray(qpos) + 1, **kw)
    assert _sdpa_vs_naive(wrong) > 1e-3


def test_planted_missing_rope_term_is_caught():
    def wrong(qn, qr, c, kr, wuk, wuv, scale, qpos, wd=np.float64):
        ql = oracle.absorb_query(qn, wuk, wd)
        o = oracle.latent_attention(ql, 0 * qr, c, kr, scale, qpos, wd=wd)
        return oracle.project_output(o, wuv, wd), o
    assert _naive_vs_absorbed(wrong) > 1e-3


def test_planted_transposed_uk_is_caught():
    cfg = dict(TINY, qk_nope_dim=6)   # square W_UK[h] so the transpose type-checks

    def wrong(qn, qr, c, kr, wuk, wuv, scale, qpos, wd=np.float64):
        return oracle.absorbed_attention(qn, qr, c, kr, wuk.transpose(0, 2, 1), wuv, scale, qpos, wd=wd)
    assert _naive_vs_absorbed(wrong, cfg=cfg) > 1e-3


def test_planted_interleaved_rope_is_caught(monkeypatch):
    def interleaved(x, positions, theta=10000.0, wd=np.float64):
        x = np.asarray(x, dtype=wd)
        ang = oracle.rope_angles(positions, x.shape[-1], theta)
        shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (ang.shape[1],)
        cs, sn = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
        a, b = x[..., 0::2], x[..., 1::2]
        y = np.empty_like(x)
        y[..., 0::2], y[..., 1::2] = a * cs - b * sn, b * cs + a * sn
        return y
    e = np.eye(4)
    y = interleaved(e, [3] * 4)
    assert np.max(np.abs(y[0] - [math.cos(3), 0, math.sin(3), 0])) > 1e-3
    monkeypatch.setattr(oracle.mla_oracle, "apply_rope", interleaved)
    cfg = dict(TINY)
    w = tiny_weights(15)
    x = rng(16).standard_normal((3, cfg["d_model"]))
    o, _ = oracle.layer_forward(x, w, cfg)
    bo, _ = brute_layer(x.tolist(), w, cfg, 0, [], False)
    assert np.max(np.abs(o - bo)) > 1e-6


def test_planted_norm_over_whole_row_is_caught(monkeypatch):
    real = oracle.mla_oracle.kv_latent_rows

    def wrong(x, w_dkv, g, positions, R, eps=1e-6, theta=10000.0, wd=np.float64):
        z = np.asarray(x, dtype=wd) @ np.asarray(w_dkv, dtype=wd)
        full = z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)
        return full[:, :R] * g, oracle.apply_rope(full[:, R:], positions, theta, wd)
    monkeypatch.setattr(oracle.mla_oracle, "kv_latent_rows", wrong)
    cfg = dict(TINY)
    w = tiny_weights(15)
    x = rng(16).standard_normal((3, cfg["d_model"]))
    _, rows = oracle.layer_forward(x, w, cfg)
    _, brows = brute_layer(x.tolist(), w, cfg, 0, [], False)
    assert np.max(np.abs(rows - brows)) > 1e-3
    monkeypatch.setattr(oracle.mla_oracle, "kv_latent_rows", real)


def test_planted_gate_from_attention_result_is_caught():
    h, x, w_o, w_g = gate_case(63, M=6)   # M = H*Dv so h W_G type-checks

    def wrong(h, x, w_o, w_g):
        hf = h.reshape(h.shape[0], -1)
        return (hf * oracle.sigmoid(hf @ w_g)) @ w_o
    ref = brute_gate_projection(h.reshape(3, -1).tolist(), x.tolist(), w_o.tolist(), w_g.tolist())
    assert np.max(np.abs(wrong(h, x, w_o, w_g) - ref)) > 1e-3
    a, b = wrong(h, x, w_o, w_g), wrong(2.0 * h, x, w_o, w_g)
    assert np.max(np.abs(b - 2.0 * a)) > 1e-3           # breaks the linearity pin


def test_planted_gate_after_projection_is_caught():
    h, x, w_o, w_g = gate_case(64, M=6)

    def wrong(h, x, w_o, w_g):
        return (h.reshape(h.shape[0], -1) @ w_o) * oracle.sigmoid(x @ w_g)
    ref = brute_gate_projection(h.reshape(3, -1).tolist(), x.tolist(), w_o.tolist(), w_g.tolist())
    assert np.max(np.abs(wrong(h, x, w_o, w_g) - ref)) > 1e-3


def test_planted_missing_sigmoid_is_caught():
    h, x, w_o, w_g = gate_case(65)

    def wrong(h, x, w_o, w_g):
        return (h.reshape(h.shape[0], -1) * (x @ w_g)) @ w_o
    plain = oracle.output_gate_projection(h, x, w_o)
    half = wrong(h, x, w_o, np.zeros_like(w_g))
    assert np.max(np.abs(half - 0.5 * plain)) > 1e-3    # the W_G = 0 pin fails


# ---------------------------------------------------------------------------
# FP8 latent cache rows (softved article, "Practical Implementation Tips for
# MLA in LLM Serving": quantize the cache; the E4M3 format, the per-row
# power-of-two scale and the row layout are readings, pinned here against the
# format's definition and against torch's float8_e4m3fn)
# ---------------------------------------------------------------------------
def _torch_e4m3(values):
    import torch
    return torch.from_numpy(np.asarray(values, np.float64)).to(torch.float8_e4m3fn)


def test_e4m3_decode_matches_torch_on_every_code():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_value(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    assert np.isnan(got).sum() == 2                      # S.1111.111 only: no infinities


def test_e4m3_closed_forms():
    v = oracle.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0        # largest finite
    assert v(0x01) == 2.0 ** -9                          # smallest subnormal
    assert v(0x08) == 2.0 ** -6 and v(0x07) == 7 * 2.0 ** -9   # normal / subnormal edge
    assert v(0x38) == 1.0 and v(0x39) == 1.125
    r = oracle.e4m3_round
    assert r(1.0625) == 0x38 and r(1.1875) == 0x3A      # ties go to the even code
    assert r(448.0) == 0x7E and r(1e9) == 0x7E and r(-1e9) == 0xFE   # saturation
    assert r(0.75 * 2.0 ** -9) == 0x01 and r(0.25 * 2.0 ** -9) == 0x00


def test_e4m3_rounding_matches_torch_in_range():
    rng = np.random.default_rng(71)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(5000) * 1e-3,
                        oracle.e4m3_value(np.arange(126)) * 1.0625])   # many exact ties
    x = np.clip(x, -448, 448)
    got = oracle.e4m3_value(oracle.e4m3_round(x))
    want = _torch_e4m3(x).to(dtype=__import__("torch").float64).numpy()
    assert np.array_equal(got, want)


def test_e4m3_round_is_nearest():
    rng = np.random.default_rng(72)
    x = rng.uniform(-448, 448, 5000)
    got = oracle.e4m3_value(oracle.e4m3_round(x))
    grid = oracle.e4m3_value(np.arange(256))
    grid = grid[~np.isnan(grid)]
    best = np.min(np.abs(x[:, None] - grid[None, :]), axis=1)   # brute force
    assert np.array_equal(np.abs(x - got), best)


def test_fp8_row_scale_rule():
    rng = np.random.default_rng(73)
    c = rng.standard_normal((200, 512)) * np.exp2(rng.integers(-12, 12, (200, 1)))
    s = oracle.fp8_row_scale(c)
    assert np.all(np.exp2(np.round(np.log2(s))) == s)          # powers of two
    ratio = np.max(np.abs(c), axis=1) / s
    assert np.all(ratio <= 448.0) and np.all(ratio > 224.0)
    assert oracle.fp8_row_scale(np.zeros((1, 8)))[0] == 1.0


def test_fp8_rows_error_bound_and_layout():
    rng = np.random.default_rng(74)
    rows = rng.standard_normal((64, 576))
    codes, s, rope = oracle.quantize_rows_fp8(rows, 512)
    deq = oracle.dequantize_rows_fp8(codes, s, rope)
    c, cq = rows[:, :512], deq[:, :512]
    normal = np.abs(c) / s[:, None] >= 2.0 ** -6
    # half a step of a 3-bit mantissa (relative), half a subnormal step below
    assert np.all(np.abs(cq - c)[normal] <= 2.0 ** -4 * np.abs(c)[normal])
    assert np.all(np.abs(cq - c)[~normal] <= (2.0 ** -10 * s[:, None] * np.ones_like(c))[~normal])
    assert np.all(np.abs(deq[:, 512:] - rows[:, 512:]) <= 2.0 ** -8 * np.abs(rows[:, 512:]))
    raw = oracle.pack_rows_fp8(codes, s, rope)
    assert raw.shape == (64, 656) and oracle.fp8_row_bytes(512, 64) == 656
    assert np.array_equal(raw[:, :512], codes) and np.all(raw[:, 644:] == 0)
    assert np.array_equal(raw[:, 640:644].copy().view("<f4")[:, 0], s.astype(np.float32))
    back = oracle.unpack_rows_fp8(raw, 512, 64)
    assert all(np.array_equal(a, b) for a, b in zip(back, (codes, s, rope)))


def test_fp8_append_rows_store_the_quantized_values():
    cfg = dict(workloads.WORKLOADS["tiny_fp32"], kv_lora_rank=16, rope_dim=8)
    rng = np.random.default_rng(75)
    M = cfg["d_model"]
    w = {"w_dkv": rng.standard_normal((M, 24)) / 8, "kv_norm_w": 1 + 0.1 * rng.standard_normal(16)}
    x = rng.standard_normal((5, M))
    f64 = oracle.append_rows(x, np.arange(5), w, cfg, storage="f64")
    q = oracle.append_rows(x, np.arange(5), w, cfg, storage="fp8")
    assert np.array_equal(q, oracle.fp8_store_rows(f64, 16))
    assert not np.array_equal(q[:, :16], f64[:, :16])


def test_planted_fnuz_bias_is_caught():
    """The other common 8-bit E4M3 (exponent bias 8, as on earlier AMD
    matrix cores) halves every value: the torch pin fails."""
    import torch
    codes = np.arange(0x7F, dtype=np.uint8)
    wrong = oracle.e4m3_value(codes) / 2
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert not np.array_equal(wrong, want)


# ===========================================================================
# Shared W_UK / W_UV: G matrices for H heads ("ARCH-MLA. Multihead Latent
# Attention", 5.1: 4 key/value heads for 16 query heads)
# ===========================================================================
def _grouped_case(seed=61, H=8, G=2, L=37):
    r = rng(seed)
    R, Dr, Dn, Dv, bs = 24, 8, 12, 10, 16
    cfg = dict(num_heads=H, kv_lora_rank=R, rope_dim=Dr, qk_nope_dim=Dn, v_dim=Dv,
               block_size=bs)
    nblk = -(-L // bs)
    pool = r.standard_normal((nblk, bs, R + Dr))
    qn, qr = r.standard_normal((1, H, Dn)), r.standard_normal((1, H, Dr))
    w_uk, w_uv = r.standard_normal((G, Dn, R)), r.standard_normal((G, R, Dv))
    return cfg, pool, qn, qr, w_uk, w_uv, L


@pytest.mark.parametrize("path", ["absorbed", "naive"])
def test_grouped_decode_matches_torch_gqa_sdpa(path):
    """Library check of the grouping convention: keys and values rebuilt for
    the G groups only, then torch's SDPA with grouped-query heads (query
    head h reads key/value head h // (H / G)); the oracle expands the G
    matrices to H heads and attends per head."""
    torch = pytest.importorskip("torch")
    cfg, pool, qn, qr, w_uk, w_uv, L = _grouped_case()
    R = cfg["kv_lora_rank"]
    rows = pool.reshape(-1, pool.shape[-1])[:L]
    k, v = oracle.reconstruct_kv(rows[:, :R], rows[:, R:], w_uk, w_uv)     # [L, G, .]
    q = np.concatenate([qn, qr], axis=-1)                                  # [1, H, Dn + Dr]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), scale=oracle.softmax_scale(cfg), enable_gqa=True)[0].numpy()
    ref = ref.transpose(1, 0, 2)[0]                                        # [H, Dv]
    table = np.arange(pool.shape[0])[None]
    got, _ = oracle.decode(qn, qr, w_uk, w_uv, pool, table, np.array([L]), cfg, path=path)
    assert np.max(np.abs(got[0] - ref)) < 1e-12


def test_head_matrices_special_cases():
    """G = H returns the per-head matrices unchanged; G = 1 gives every head
    the one matrix; consecutive heads share (not round-robin); a G that does
    not divide H is refused."""
    w = rng(62).standard_normal((4, 3, 5))
    assert np.array_equal(oracle.head_matrices(w, 4), w)
    one = oracle.head_matrices(w[:1], 6)
    assert all(np.array_equal(one[h], w[0]) for h in range(6))
    two = oracle.head_matrices(w[:2], 4)
    assert np.array_equal(two[1], w[0]) and np.array_equal(two[2], w[1])
    with pytest.raises(ValueError):
        oracle.head_matrices(w[:3], 4)


def test_grouped_decode_planted_round_robin_is_caught():
    """A round-robin grouping (head h reads matrix h % G) differs from the
    consecutive grouping the torch check fixes."""
    cfg, pool, qn, qr, w_uk, w_uv, L = _grouped_case(seed=63)
    table = np.arange(pool.shape[0])[None]
    got, _ = oracle.decode(qn, qr, w_uk, w_uv, pool, table, np.array([L]), cfg)
    H, G = qn.shape[1], w_uk.shape[0]
    rr = np.stack([w_uk[h % G] for h in range(H)]), np.stack([w_uv[h % G] for h in range(H)])
    bad, _ = oracle.decode(qn, qr, rr[0], rr[1], pool, table, np.array([L]), cfg)
    assert np.max(np.abs(got - bad)) > 1e-3
