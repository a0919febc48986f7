"""Helpers shared by the GPU tests: uploading seeded inputs and comparing the
HIP results with the oracle to the stated tolerances."""
import json
import os

import numpy as np

import workloads

# float32 storage: max abs <= 1e-5.  bf16 storage with float32 accumulation:
# relative L2 <= 5e-3 and max abs <= 2e-2.
F32_MAX_ABS = 1e-5
BF16_REL_L2 = 5e-3
BF16_MAX_ABS = 2e-2

_GOLD = os.path.join(os.path.dirname(__file__), "golden")
COSINE_FLOOR = json.load(open(os.path.join(_GOLD, "cosine_tutorial_5_4.json")))["cosine_min"]


def to_dev(arr, device="cuda"):
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_host_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def errors(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    d = gpu - ref
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    cos = float(np.dot(gpu.ravel(), ref.ravel()) /
                max(np.linalg.norm(gpu) * np.linalg.norm(ref), 1e-300))
    return dict(max_abs=float(np.max(np.abs(d))) if d.size else 0.0, rel_l2=float(rel), cosine=cos)


def assert_f32(gpu, ref, what=""):
    e = errors(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert e["max_abs"] <= F32_MAX_ABS, f"{what}: {e}"
    return e


def assert_bf16(gpu, ref, what="", per_row_axis=None):
    e = errors(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert e["rel_l2"] <= BF16_REL_L2 and e["max_abs"] <= BF16_MAX_ABS, f"{what}: {e}"
    assert e["cosine"] >= COSINE_FLOOR, f"{what}: {e}"
    if per_row_axis is not None:
        g = np.moveaxis(np.asarray(gpu, np.float64), per_row_axis, 0)
        r = np.moveaxis(np.asarray(ref, np.float64), per_row_axis, 0)
        for i in range(g.shape[0]):
            ei = errors(g[i], r[i])
            assert ei["rel_l2"] <= BF16_REL_L2, f"{what} row {i}: {ei}"
    return e


def compact_sequences(inp, ids):
    """float64 pools holding only the given sequences (identity page tables),
    for the oracle: pages are copied, nothing is computed."""
    bs = inp.pool.shape[1]
    out = []
    for b in ids:
        L = int(inp.seq_lens[b])
        nblk = -(-L // bs)
        pages = workloads.to_f64(inp.pool[inp.block_table[b, :nblk]])
        out.append((pages, np.arange(nblk)[None], np.array([L])))
    return out


def decode_config(cfg_dict):
    from mla_latent_kv_26_amd import MLAConfig
    return MLAConfig.from_dict(cfg_dict)
