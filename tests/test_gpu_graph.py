"""The decode step captured in a HIP graph (as the benchmark times it) and
replayed: every replay, with other eager decodes and device work run between
the replays, gives bitwise the output of the same call issued eagerly (the
kernels are deterministic), for mla_decode with a caller workspace and for
mla_decode_noalloc, on bf16 and FP8 cache rows.  The eager outputs are
checked against the oracle on a few sequences as well."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import to_dev, to_host_f64, assert_bf16, compact_sequences

pytestmark = pytest.mark.gpu

LENS = np.array([4096, 100, 2049, 1, 700, 4096, 33, 1500], np.int32)


@pytest.fixture(scope="module")
def m():
    import torch  # noqa: F401
    import mla_latent_kv_26_amd as m
    return m


def _inputs(cfg, seed):
    inp = workloads.decode_inputs(cfg, seed=seed, lengths=LENS)
    pool = inp.pool
    deq = None
    if cfg.get("cache_dtype") == "fp8":
        codes, s, rope = oracle.quantize_rows_fp8(workloads.to_f64(inp.pool), cfg["kv_lora_rank"])
        pool = oracle.pack_rows_fp8(codes, s, rope)
        deq = oracle.dequantize_rows_fp8(codes, s, rope)
    args = [to_dev(a) for a in (inp.q_nope, inp.q_rope, inp.w_uk, inp.w_uv, pool,
                                inp.block_table, inp.seq_lens)]
    return inp, deq, args


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_graph_replays_equal_eager(m, cache, entry):
    import torch
    cfg = dict(workloads.WORKLOADS["paged_ragged_h128_b64"], num_heads=64, lengths="explicit",
               paged=True, seed=23)
    if cache == "fp8":
        cfg["cache_dtype"] = "fp8"
    mc = m.MLAConfig.from_dict(cfg)
    L = int(LENS.max())
    inp_a, deq_a, a = _inputs(cfg, 23)
    _, _, b = _inputs(cfg, 24)
    ws_size = m.mla_decode_workspace_size(mc, len(LENS), L)
    ws_eager = torch.zeros(ws_size, dtype=torch.uint8, device="cuda")
    eager_a = m.mla_decode(mc, *a, L, workspace=ws_eager).clone()
    eager_b = m.mla_decode(mc, *b, L, workspace=ws_eager).clone()
    torch.cuda.synchronize()
    # the eager result of set a against the oracle on a few sequences
    inp_q = inp_a if deq_a is None else __import__("dataclasses").replace(inp_a, pool=deq_a)
    ids = [0, 3, 6]
    ref = []
    for bi, (pages, table, ln) in zip(ids, compact_sequences(inp_q, ids)):
        o, _ = oracle.decode(workloads.to_f64(inp_a.q_nope[bi:bi + 1]),
                             workloads.to_f64(inp_a.q_rope[bi:bi + 1]),
                             workloads.to_f64(inp_a.w_uk), workloads.to_f64(inp_a.w_uv), pages,
                             table, ln, cfg)
        ref.append(o[0])
    assert_bf16(to_host_f64(eager_a)[ids], np.stack(ref), f"eager {cache}", per_row_axis=0)

    out = torch.full_like(eager_a, float("nan"))
    ws_graph = torch.zeros(ws_size, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()

    def call():
        if entry == "noalloc":
            m.mla_decode_noalloc(mc, *a, L, out=out)
        else:
            m.mla_decode(mc, *a, L, out=out, workspace=ws_graph)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm the path (and, for noalloc, the device scratch) outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    other = torch.empty_like(eager_b)
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_a), f"replay {r}: {cache} {entry}"
        # eager work between the replays: a decode of other inputs (through
        # the same entry point, so the noalloc scratch is overwritten) and a
        # device op
        if entry == "noalloc":
            m.mla_decode_noalloc(mc, *b, L, out=other)
        else:
            m.mla_decode(mc, *b, L, out=other, workspace=ws_eager)
        other.mul_(1.0)
        torch.cuda.synchronize()
        assert torch.equal(other, eager_b), f"eager between replays {r}: {cache} {entry}"
