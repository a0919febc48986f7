"""Host-side checks of the C ABI library: it loads, exports every symbol the
header declares, and rejects invalid calls before anything is enqueued.  No
GPU needed: only host functions are called, and invalid calls return before
touching any pointer."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from oracle import ledger

m = pytest.importorskip("mla_latent_kv_26_amd")
from mla_latent_kv_26_amd import _lib  # noqa: E402
from mla_latent_kv_26_amd._lib import lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KIMI = m.MLAConfig(num_heads=64, kv_lora_rank=512, rope_dim=64, qk_nope_dim=128, v_dim=128)
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def header_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_header_symbol_is_exported_and_bound():
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_abi_version_and_status_strings():
    assert lib.mla_abi_version() == 5
    for s, name in _lib.STATUS_NAMES.items():
        assert lib.mla_status_string(s).decode() == name


def test_bytes_per_token_matches_ledger():
    g = dict(num_heads=64, num_kv_heads=8, head_dim=128, latent_dim=512, rope_dim=64, dtype_bytes=2)
    assert m.mla_cache_bytes_per_token(KIMI) == ledger.state_bytes("mla", g) == 1152
    assert m.mla_cache_row_elems(KIMI) == ledger.state_elements("mla", g) == 576
    f32 = m.MLAConfig(4, 32, 8, 16, 16, dtype="f32")
    assert m.mla_cache_bytes_per_token(f32) == 40 * 4


def test_rope_table_matches_oracle_angles():
    for cfg, n in ((KIMI, 5000), (m.MLAConfig(4, 32, 8, 16, 16, dtype="f32"), 70)):
        tab = m.mla_rope_table(cfg, n).numpy().astype(np.float64)
        ang = oracle.rope_angles(np.arange(n), cfg.rope_dim, cfg.rope_theta)
        half = cfg.rope_dim // 2
        np.testing.assert_allclose(tab[:, :half], np.cos(ang), rtol=0, atol=6e-8)
        np.testing.assert_allclose(tab[:, half:], np.sin(ang), rtol=0, atol=6e-8)


@pytest.mark.parametrize("field,value", [
    ("num_heads", 0), ("kv_lora_rank", -1), ("rope_dim", 63), ("qk_nope_dim", 0), ("v_dim", 0),
    ("block_size", 0), ("softmax_scale", -1.0), ("rms_eps", -1e-6), ("rope_theta", 0.0),
    ("d_model", -5), ("split_workgroups", -8), ("split_workgroups", 12),
    ("split_workgroups", 8200)])
def test_invalid_config_rejected(field, value):
    import dataclasses
    bad = dataclasses.replace(KIMI, **{field: value})
    with pytest.raises(m.MLAError) as e:
        m.mla_validate_config(bad)
    assert e.value.status == _lib.MLA_ERR_INVALID_ARG
    assert _lib.last_error()


def test_split_workgroups_sizes_the_workspace():
    """The decode workspace holds one partial per (workgroup, sequence) slot:
    more split workgroups need more of it; 0 is the library's own choice."""
    import dataclasses
    sizes = [m.mla_decode_workspace_size(dataclasses.replace(KIMI, split_workgroups=n), 32, 4096)
             for n in (8, 64, 512)]
    assert sizes[0] < sizes[1] < sizes[2]
    m.mla_validate_config(dataclasses.replace(KIMI, split_workgroups=8192))


def test_latent_ranks_must_be_below_model_width():
    import dataclasses
    for over in (dict(d_model=512), dict(d_model=1024, q_lora_rank=1024)):
        with pytest.raises(m.MLAError):
            m.mla_validate_config(dataclasses.replace(KIMI, **over))
    m.mla_validate_config(dataclasses.replace(KIMI, d_model=7168, q_lora_rank=1536))


def _decode(cfg, **over):
    a = dict(q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE, pool=FAKE, nb=100, table=FAKE,
             mb=64, lens=FAKE, batch=32, max_len=4096, out=FAKE, ws=FAKE, ws_bytes=1 << 40,
             stream=None)
    a.update(over)
    return lib.mla_decode(ctypes.byref(cfg.c()), a["q_nope"], a["q_rope"], a["w_uk"], a["w_uv"],
                          a["pool"], a["nb"], a["table"], a["mb"], a["lens"], a["batch"],
                          a["max_len"], a["out"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(batch=0), _lib.MLA_ERR_INVALID_ARG),
    (dict(max_len=0), _lib.MLA_ERR_INVALID_ARG),
    (dict(max_len=4097), _lib.MLA_ERR_INVALID_ARG),       # beyond 64 blocks x 64 tokens
    (dict(nb=0), _lib.MLA_ERR_INVALID_ARG),
    (dict(mb=0), _lib.MLA_ERR_INVALID_ARG),
    (dict(table=None), _lib.MLA_ERR_INVALID_ARG),
    (dict(lens=None), _lib.MLA_ERR_INVALID_ARG),
    (dict(q_nope=None), _lib.MLA_ERR_INVALID_ARG),
    (dict(out=FAKE + 2), _lib.MLA_ERR_INVALID_ARG),       # misaligned
    (dict(ws=None), _lib.MLA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _lib.MLA_ERR_WORKSPACE),
    (dict(batch=1025), _lib.MLA_ERR_UNSUPPORTED),
])
def test_decode_rejects_invalid_calls(over, status):
    assert _decode(KIMI, **over) == status
    assert _lib.last_error()


def test_decode_rejects_unsupported_shapes():
    import dataclasses
    for over in (dict(kv_lora_rank=384), dict(rope_dim=32), dict(num_heads=48),
                 dict(block_size=16), dict(block_size=96), dict(v_dim=136),
                 dict(kv_lora_rank=256, num_heads=24), dict(kv_lora_rank=256, rope_dim=32),
                 dict(kv_lora_rank=256, cache_dtype="fp8")):
        cfg = dataclasses.replace(KIMI, **over)
        assert _decode(cfg, max_len=64) == _lib.MLA_ERR_UNSUPPORTED, over


MECH = m.MLAConfig(num_heads=16, kv_lora_rank=256, rope_dim=64, qk_nope_dim=64, v_dim=64,
                   kv_groups=4)


def test_decode_attention_field():
    """decode_attention: 0..2 accepted, others rejected; the per-head form
    takes its own workspace, refuses shapes outside Dn = Dv = Dr = 64 or more
    than 16 heads per group, and the staged (latent-form) calls refuse it."""
    import dataclasses
    for v, st in ((0, _lib.MLA_OK), (1, _lib.MLA_OK), (2, _lib.MLA_OK),
                  (3, _lib.MLA_ERR_INVALID_ARG), (-1, _lib.MLA_ERR_INVALID_ARG)):
        c = MECH.c()
        c.decode_attention = v
        assert lib.mla_validate_config(ctypes.byref(c)) == st, v
    ph = dataclasses.replace(MECH, decode_attention="per_head")
    lat = m.mla_decode_workspace_size(MECH, 1, 8192)
    per = m.mla_decode_workspace_size(ph, 1, 8192)
    # the rebuilt rows alone: 4 groups x 8192 tokens x 192 values x 2 bytes
    assert per > 4 * 8192 * 192 * 2 > lat
    assert _decode(dataclasses.replace(KIMI, decode_attention="per_head"), max_len=64) == \
        _lib.MLA_ERR_UNSUPPORTED                                   # Dn = Dv = 128
    assert _decode(dataclasses.replace(ph, num_heads=32, kv_groups=1), max_len=64) == \
        _lib.MLA_ERR_UNSUPPORTED                                   # 32 heads in one group
    assert _decode(dataclasses.replace(ph, cache_dtype="fp8"), max_len=64) == \
        _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_latent_attention(ctypes.byref(ph.c()), FAKE, FAKE, 100, FAKE, 64, FAKE, 1, 64,
                                    FAKE, FAKE, 1 << 40, None) == _lib.MLA_ERR_UNSUPPORTED
    assert "mla_decode only" in _lib.last_error()


def test_workspace_size_of_unsupported_shape_is_an_error():
    """A shape no decode kernel takes (16 heads on the latent-512 kernels)
    gets MLA_ERR_UNSUPPORTED from the workspace query too."""
    import dataclasses
    with pytest.raises(m.MLAError) as e:
        m.mla_decode_workspace_size(dataclasses.replace(KIMI, num_heads=16), 1, 64)
    assert e.value.status == _lib.MLA_ERR_UNSUPPORTED


def test_kv_groups_must_divide_heads():
    import dataclasses
    for g, st in ((0, _lib.MLA_OK), (1, _lib.MLA_OK), (8, _lib.MLA_OK), (64, _lib.MLA_OK),
                  (3, _lib.MLA_ERR_INVALID_ARG), (-1, _lib.MLA_ERR_INVALID_ARG)):
        cfg = dataclasses.replace(KIMI, kv_groups=g)
        assert lib.mla_validate_config(ctypes.byref(cfg.c())) == st, g


def test_prefill_and_append_reject_invalid_calls():
    cfg = m.MLAConfig(64, 512, 64, 128, 128, d_model=7168, q_lora_rank=1536)
    c = ctypes.byref(cfg.c())
    args = [c, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 128, FAKE,
            64, FAKE, 0, 2, 4096, FAKE, FAKE, 1 << 40, None]
    # every case below breaks exactly one rule, so the call returns before any launch:
    # q_len 0, rope table too short, page table too small, workspace too small
    for idx, val, st in ((19, 0, _lib.MLA_ERR_INVALID_ARG), (11, 100, _lib.MLA_ERR_INVALID_ARG),
                         (15, 10, _lib.MLA_ERR_INVALID_ARG), (22, 16, _lib.MLA_ERR_WORKSPACE)):
        a = list(args)
        a[idx] = val
        assert lib.mla_prefill(*a) == st, (idx, val)
    no_model = m.MLAConfig(64, 512, 64, 128, 128)
    assert lib.mla_cache_append(ctypes.byref(no_model.c()), FAKE, FAKE, FAKE, FAKE, 16, FAKE,
                                FAKE, 4, FAKE, 10, FAKE, 1 << 30, None) == _lib.MLA_ERR_INVALID_ARG


def test_empty_calls_are_rejected():
    """A zero count is MLA_ERR_INVALID_ARG on every entry point (checked on the
    host before anything is enqueued), never a silent no-op."""
    bad = _lib.MLA_ERR_INVALID_ARG
    cfg = m.MLAConfig(64, 512, 64, 128, 128, d_model=7168, q_lora_rank=1536)
    c = ctypes.byref(cfg.c())
    assert _decode(KIMI, batch=0) == bad
    args = [c, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 128, FAKE,
            64, FAKE, 0, 2, 4096, FAKE, FAKE, 1 << 40, None]
    for idx in (18, 19):  # batch, q_len
        a = list(args)
        a[idx] = 0
        assert lib.mla_prefill(*a) == bad, idx
    assert lib.mla_cache_append(c, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 0, FAKE, 10, FAKE,
                                1 << 30, None) == bad
    assert lib.mla_output_projection(c, FAKE, FAKE, 0, FAKE, None) == bad
    assert lib.mla_output_gate_projection(c, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1 << 30,
                                          None) == bad
    assert "positive" in _lib.last_error()


def test_probes_reject_invalid_calls():
    """The measurement probes validate before any launch."""
    bad = _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_lds_read(4, 10, FAKE, None) == bad      # width 16 or 8 only
    assert lib.mla_probe_lds_read(16, 0, FAKE, None) == bad
    assert lib.mla_probe_lds_read(8, 10, None, None) == bad
    assert lib.mla_probe_mfma(0, 10, FAKE, None) == bad
    assert lib.mla_probe_hbm_read(FAKE, 1024, 0, FAKE, None) == bad   # below one 36864-byte piece
    assert lib.mla_probe_hbm_read(FAKE, 1 << 20, 2, FAKE, None) == bad


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m.mla_absorb_query(KIMI, q, torch.zeros(2, 64, 64, dtype=torch.bfloat16),
                           torch.zeros(64, 128, 512, dtype=torch.bfloat16))


def test_pool_allocator_bookkeeping():
    cfg = m.MLAConfig(4, 32, 8, 16, 16, dtype="f32", block_size=16)
    pool = m.LatentKVPool(cfg, 10, device="cpu")
    assert pool.reserve(7, 20) and len(pool.blocks(7)) == 2
    pool.reserve(9, 16)
    pool.reserve(7, 33)
    assert len(pool.blocks(7)) == 3 and pool.free_blocks == 6
    t = pool.block_table([7, 9], device="cpu")
    assert t.shape == (2, 3) and t[0].tolist() == pool.blocks(7)
    s = pool.slot_mapping(7, [0, 15, 16, 32], device="cpu").tolist()
    b = pool.blocks(7)
    assert s == [b[0] * 16, b[0] * 16 + 15, b[1] * 16, b[2] * 16]
    assert pool.seq_lens([7, 9], device="cpu").tolist() == [33, 16]
    pool.release(7)
    assert pool.free_blocks == 9
    with pytest.raises(MemoryError):
        pool.reserve(1, 16 * 11)
