"""KV-state ledger: cached elements and bytes per token per layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Three ways to keep the history of one token in one layer:
  * MHA keeps a key and a value vector for every query head,
  * GQA/MQA keeps them only for the (fewer) shared KV heads,
  * MLA keeps one latent of width latent_dim plus one rope key of width
    rope_dim, independent of the head count.
(ARCH-MLA tutorial, Step 1 and Step 2; modeldna MLA module, cache-size
table.)  Configuration fields use the tutorial's names (Step 4): num_heads,
num_kv_heads, head_dim, latent_dim, rope_dim, dtype_bytes; all must be
positive integers and num_heads must be a multiple of num_kv_heads, else
ValueError.
"""
from __future__ import annotations

from typing import Dict, Mapping

FIELDS = ("num_heads", "num_kv_heads", "head_dim", "latent_dim", "rope_dim", "dtype_bytes")
MODES = ("mha", "gqa", "mla")


def check_state_config(cfg: Mapping[str, int]) -> None:
    absent = [f for f in FIELDS if f not in cfg]
    if absent:
        raise ValueError(f"state config lacks {absent}")
    for f in FIELDS:
        v = cfg[f]
        if isinstance(v, bool) or not isinstance(v, int) or v <= 0:
            raise ValueError(f"{f} must be a positive integer, got {v!r}")
    if cfg["num_heads"] % cfg["num_kv_heads"]:
        raise ValueError("num_heads must be a multiple of num_kv_heads")


def state_elements(mode: str, cfg: Mapping[str, int]) -> int:
    """Cached values per token per layer for one representation."""
    check_state_config(cfg)
    if mode == "mha":
        return 2 * cfg["num_heads"] * cfg["head_dim"]      # K and V, every head
    if mode == "gqa":
        return 2 * cfg["num_kv_heads"] * cfg["head_dim"]   # K and V, shared heads
    if mode == "mla":
        return cfg["latent_dim"] + cfg["rope_dim"]         # latent + rope key
    raise ValueError(f"unknown representation {mode!r}")


def state_bytes(mode: str, cfg: Mapping[str, int]) -> int:
    return state_elements(mode, cfg) * cfg["dtype_bytes"]


def compare_states(cfg: Mapping[str, int]) -> Dict[str, object]:
    """Bytes per token for each representation, each as a fraction of MHA,
    and the most compact one."""
    nbytes = {m: state_bytes(m, cfg) for m in MODES}
    ratio = {m: nbytes[m] / nbytes["mha"] for m in MODES}
    smallest = sorted(MODES, key=lambda m: (nbytes[m], MODES.index(m)))[0]
    return {"bytes_per_token": nbytes, "ratio_vs_mha": ratio, "most_compact": smallest}
