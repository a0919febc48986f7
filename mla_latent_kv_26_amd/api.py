"""Python binding of the C ABI (include/mla.h), same names, torch tensors in.

Argument marshalling only: shapes and dtypes are checked, missing outputs and
workspaces are allocated with torch, and every computation runs in the HIP
library.  PyTorch provides device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import lib, check, MLAConfigC

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_C_DTYPE = {"f32": _lib.DTYPE_F32, "bf16": _lib.DTYPE_BF16}
_C_CACHE = {"same": _lib.CACHE_SAME, "fp8": _lib.CACHE_FP8_E4M3}
_C_PREFILL = {"auto": 0, "latent": 1, "per_head": 2}
_C_DECODE = {"auto": 0, "latent": 1, "per_head": 2}


@dataclasses.dataclass(frozen=True)
class MLAConfig:
    """Geometry of one MLA layer (mirrors struct mla_config)."""
    num_heads: int
    kv_lora_rank: int
    rope_dim: int
    qk_nope_dim: int
    v_dim: int
    d_model: int = 0
    q_lora_rank: int = 0
    block_size: int = 64
    softmax_scale: float = 0.0
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    dtype: str = "bf16"
    cache_dtype: str = "same"   # "same" (rows in dtype) or "fp8" (E4M3 latent, see mla.h)
    kv_groups: int = 0          # 0: W_UK, W_UV per head; G: heads share G matrices in order
    split_workgroups: int = 0   # decode attention workgroups per head group (0: one per CU)
    prefill_attention: str = "auto"   # "auto" (fewer FLOPs), "latent" (absorbed), "per_head"
    decode_attention: str = "latent"  # "latent" (absorbed) or "per_head" (keys, values rebuilt)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    @property
    def row(self) -> int:
        return self.kv_lora_rank + self.rope_dim

    @property
    def pool_dtype(self) -> torch.dtype:
        """Element type of a cache pool tensor (bytes for FP8 rows)."""
        return torch.uint8 if self.cache_dtype == "fp8" else self.torch_dtype

    @property
    def pool_row(self) -> int:
        """Elements per cached row in a pool tensor: R + Dr values, or the
        R + 2 Dr + 16 bytes of an FP8 row."""
        if self.cache_dtype == "fp8":
            return self.kv_lora_rank + 2 * self.rope_dim + 16
        return self.row

    @property
    def uk_heads(self) -> int:
        """Leading dimension of w_uk and w_uv: H, or kv_groups when set."""
        return self.kv_groups or self.num_heads

    @property
    def scale(self) -> float:
        return self.softmax_scale or 1.0 / math.sqrt(self.qk_nope_dim + self.rope_dim)

    def c(self) -> MLAConfigC:
        return MLAConfigC(self.num_heads, self.kv_lora_rank, self.rope_dim, self.qk_nope_dim,
                          self.v_dim, self.d_model, self.q_lora_rank, self.block_size,
                          self.softmax_scale, self.rms_eps, self.rope_theta,
                          _C_DTYPE[self.dtype], _C_CACHE[self.cache_dtype], self.kv_groups,
                          self.split_workgroups, _C_PREFILL[self.prefill_attention],
                          _C_DECODE[self.decode_attention])

    @classmethod
    def from_dict(cls, d: dict, **over) -> "MLAConfig":
        keys = {f.name for f in dataclasses.fields(cls)}
        kw = {k: v for k, v in d.items() if k in keys}
        kw.update(over)
        return cls(**kw)


def _ref(cfg: MLAConfig):
    return ctypes.byref(cfg.c())


def _dev(t: torch.Tensor, name: str, dtype: Optional[torch.dtype] = None,
         shape: Optional[Sequence[int]] = None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    if ws is None:
        return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or ws.numel() < nbytes:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nbytes} bytes")
    return ws


# ---------------------------------------------------------------------------
# host-only queries
# ---------------------------------------------------------------------------
def mla_abi_version() -> int:
    return lib.mla_abi_version()


def mla_validate_config(cfg: MLAConfig) -> None:
    check(lib.mla_validate_config(_ref(cfg)), "mla_validate_config")


def mla_cache_row_elems(cfg: MLAConfig) -> int:
    n = lib.mla_cache_row_elems(_ref(cfg))
    if n < 0:
        raise _lib.MLAError(_lib.MLA_ERR_INVALID_ARG, "mla_cache_row_elems", _lib.last_error())
    return n


def mla_cache_bytes_per_token(cfg: MLAConfig) -> int:
    n = lib.mla_cache_bytes_per_token(_ref(cfg))
    if n < 0:
        raise _lib.MLAError(_lib.MLA_ERR_INVALID_ARG, "mla_cache_bytes_per_token", _lib.last_error())
    return n


def mla_rope_table(cfg: MLAConfig, num_positions: int) -> torch.Tensor:
    """Host float32 tensor [num_positions, rope_dim]: cos half | sin half."""
    out = torch.empty((num_positions, cfg.rope_dim), dtype=torch.float32)
    ptr = ctypes.cast(out.data_ptr(), ctypes.POINTER(ctypes.c_float))
    check(lib.mla_rope_table(_ref(cfg), num_positions, ptr), "mla_rope_table")
    return out


def mla_decode_workspace_size(cfg: MLAConfig, batch: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    check(lib.mla_decode_workspace_size(_ref(cfg), batch, max_seq_len, ctypes.byref(n)),
          "mla_decode_workspace_size")
    return n.value


def mla_cache_append_workspace_size(cfg: MLAConfig, n_tokens: int) -> int:
    n = ctypes.c_size_t()
    check(lib.mla_cache_append_workspace_size(_ref(cfg), n_tokens, ctypes.byref(n)),
          "mla_cache_append_workspace_size")
    return n.value


def mla_output_gate_workspace_size(cfg: MLAConfig, n_rows: int) -> int:
    n = ctypes.c_size_t()
    check(lib.mla_output_gate_workspace_size(_ref(cfg), n_rows, ctypes.byref(n)),
          "mla_output_gate_workspace_size")
    return n.value


def mla_prefill_workspace_size(cfg: MLAConfig, batch: int, q_len: int, max_context: int = 0) -> int:
    n = ctypes.c_size_t()
    check(lib.mla_prefill_workspace_size(_ref(cfg), batch, q_len, max_context, ctypes.byref(n)),
          "mla_prefill_workspace_size")
    return n.value


def mla_prefill_attention_form(cfg: MLAConfig, q_len: int, max_start_pos: int = 0) -> str:
    """"latent" or "per_head": the attention form mla_prefill takes."""
    f = ctypes.c_int32()
    check(lib.mla_prefill_attention_form(_ref(cfg), q_len, max_start_pos, ctypes.byref(f)),
          "mla_prefill_attention_form")
    return {1: "latent", 2: "per_head"}[f.value]


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def _pool_args(cfg, kv_pool, block_table, batch):
    nb = kv_pool.shape[0]
    _dev(kv_pool, "kv_pool", cfg.pool_dtype, (nb, cfg.block_size, cfg.pool_row))
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError(f"block_table must be [batch={batch}, max_blocks]")
    _dev(block_table, "block_table", torch.int32)
    return nb, block_table.shape[1]


def mla_decode(cfg: MLAConfig, q_nope, q_rope, w_uk, w_uv, kv_pool, block_table, seq_lens,
               max_seq_len: int, out=None, workspace=None, stream=None) -> torch.Tensor:
    """out [B, H, Dv] for one decode step (see mla_decode in include/mla.h)."""
    dt = cfg.torch_dtype
    B, H = q_nope.shape[0], cfg.num_heads
    _dev(q_nope, "q_nope", dt, (B, H, cfg.qk_nope_dim))
    _dev(q_rope, "q_rope", dt, (B, H, cfg.rope_dim))
    _dev(w_uk, "w_uk", dt, (cfg.uk_heads, cfg.qk_nope_dim, cfg.kv_lora_rank))
    _dev(w_uv, "w_uv", dt, (cfg.uk_heads, cfg.kv_lora_rank, cfg.v_dim))
    nb, mb = _pool_args(cfg, kv_pool, block_table, B)
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, H, cfg.v_dim), dtype=dt, device=q_nope.device)
    _dev(out, "out", dt, (B, H, cfg.v_dim))
    need = mla_decode_workspace_size(cfg, B, max_seq_len)
    ws = _workspace(workspace, need, q_nope.device)
    check(lib.mla_decode(_ref(cfg), q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(),
                         w_uv.data_ptr(), kv_pool.data_ptr(), nb, block_table.data_ptr(), mb,
                         seq_lens.data_ptr(), B, int(max_seq_len), out.data_ptr(),
                         ws.data_ptr(), ws.numel(), _stream(stream)), "mla_decode")
    return out


def mla_decode_noalloc(cfg: MLAConfig, q_nope, q_rope, w_uk, w_uv, kv_pool, block_table,
                       seq_lens, max_seq_len: int, out, stream=None) -> torch.Tensor:
    """mla_decode without a workspace (see mla_decode_noalloc in
    include/mla.h): out [B, H, Dv] must be given."""
    dt = cfg.torch_dtype
    B, H = q_nope.shape[0], cfg.num_heads
    _dev(q_nope, "q_nope", dt, (B, H, cfg.qk_nope_dim))
    _dev(q_rope, "q_rope", dt, (B, H, cfg.rope_dim))
    _dev(w_uk, "w_uk", dt, (cfg.uk_heads, cfg.qk_nope_dim, cfg.kv_lora_rank))
    _dev(w_uv, "w_uv", dt, (cfg.uk_heads, cfg.kv_lora_rank, cfg.v_dim))
    nb, mb = _pool_args(cfg, kv_pool, block_table, B)
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _dev(out, "out", dt, (B, H, cfg.v_dim))
    check(lib.mla_decode_noalloc(_ref(cfg), q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(),
                                 w_uv.data_ptr(), kv_pool.data_ptr(), nb, block_table.data_ptr(),
                                 mb, seq_lens.data_ptr(), B, int(max_seq_len), out.data_ptr(),
                                 _stream(stream)), "mla_decode_noalloc")
    return out


def mla_absorb_query(cfg: MLAConfig, q_nope, q_rope, w_uk, q_full=None, stream=None):
    """q_full [n, H, R + Dr] = scale*log2(e)*[q_nope W_UK | q_rope]."""
    dt = cfg.torch_dtype
    n, H = q_nope.shape[0], cfg.num_heads
    _dev(q_nope, "q_nope", dt, (n, H, cfg.qk_nope_dim))
    _dev(q_rope, "q_rope", dt, (n, H, cfg.rope_dim))
    _dev(w_uk, "w_uk", dt, (cfg.uk_heads, cfg.qk_nope_dim, cfg.kv_lora_rank))
    if q_full is None:
        q_full = torch.empty((n, H, cfg.row), dtype=dt, device=q_nope.device)
    _dev(q_full, "q_full", dt, (n, H, cfg.row))
    check(lib.mla_absorb_query(_ref(cfg), q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(),
                               n, q_full.data_ptr(), _stream(stream)), "mla_absorb_query")
    return q_full


def mla_latent_attention(cfg: MLAConfig, q_full, kv_pool, block_table, seq_lens,
                         max_seq_len: int, o_lat=None, workspace=None, stream=None):
    """o_lat [B, H, R]: softmax-weighted latent rows for absorbed queries."""
    dt = cfg.torch_dtype
    B, H = q_full.shape[0], cfg.num_heads
    _dev(q_full, "q_full", dt, (B, H, cfg.row))
    nb, mb = _pool_args(cfg, kv_pool, block_table, B)
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    if o_lat is None:
        o_lat = torch.empty((B, H, cfg.kv_lora_rank), dtype=dt, device=q_full.device)
    _dev(o_lat, "o_lat", dt, (B, H, cfg.kv_lora_rank))
    need = mla_decode_workspace_size(cfg, B, max_seq_len)
    ws = _workspace(workspace, need, q_full.device)
    check(lib.mla_latent_attention(_ref(cfg), q_full.data_ptr(), kv_pool.data_ptr(), nb,
                                   block_table.data_ptr(), mb, seq_lens.data_ptr(), B,
                                   int(max_seq_len), o_lat.data_ptr(), ws.data_ptr(), ws.numel(),
                                   _stream(stream)), "mla_latent_attention")
    return o_lat


def mla_attention_partials(cfg: MLAConfig, q_full, kv_pool, block_table, seq_lens,
                           max_seq_len: int, workspace, stream=None) -> None:
    """Split-KV attention partials into `workspace` (bf16 only)."""
    dt = cfg.torch_dtype
    B, H = q_full.shape[0], cfg.num_heads
    _dev(q_full, "q_full", dt, (B, H, cfg.row))
    nb, mb = _pool_args(cfg, kv_pool, block_table, B)
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _dev(workspace, "workspace", torch.uint8)
    check(lib.mla_attention_partials(_ref(cfg), q_full.data_ptr(), kv_pool.data_ptr(), nb,
                                     block_table.data_ptr(), mb, seq_lens.data_ptr(), B,
                                     int(max_seq_len), workspace.data_ptr(), workspace.numel(),
                                     _stream(stream)), "mla_attention_partials")


def mla_combine_output(cfg: MLAConfig, batch: int, max_seq_len: int, workspace, w_uv=None,
                       out=None, stream=None):
    """Merge the partials in `workspace`: o_lat [B, H, R] (w_uv None) or out [B, H, Dv]."""
    dt = cfg.torch_dtype
    H = cfg.num_heads
    _dev(workspace, "workspace", torch.uint8)
    width = cfg.kv_lora_rank if w_uv is None else cfg.v_dim
    if w_uv is not None:
        _dev(w_uv, "w_uv", dt, (cfg.uk_heads, cfg.kv_lora_rank, cfg.v_dim))
    if out is None:
        out = torch.empty((batch, H, width), dtype=dt, device=workspace.device)
    _dev(out, "out", dt, (batch, H, width))
    check(lib.mla_combine_output(_ref(cfg), None if w_uv is None else w_uv.data_ptr(), batch,
                                 int(max_seq_len), out.data_ptr(), workspace.data_ptr(),
                                 workspace.numel(), _stream(stream)), "mla_combine_output")
    return out


def mla_output_projection(cfg: MLAConfig, o_lat, w_uv, out=None, stream=None):
    """out [n, H, Dv] = o_lat[n, h] W_UV[h]."""
    dt = cfg.torch_dtype
    n, H = o_lat.shape[0], cfg.num_heads
    _dev(o_lat, "o_lat", dt, (n, H, cfg.kv_lora_rank))
    _dev(w_uv, "w_uv", dt, (cfg.uk_heads, cfg.kv_lora_rank, cfg.v_dim))
    if out is None:
        out = torch.empty((n, H, cfg.v_dim), dtype=dt, device=o_lat.device)
    _dev(out, "out", dt, (n, H, cfg.v_dim))
    check(lib.mla_output_projection(_ref(cfg), o_lat.data_ptr(), w_uv.data_ptr(), n,
                                    out.data_ptr(), _stream(stream)), "mla_output_projection")
    return out


# ---------------------------------------------------------------------------
# append and prefill
# ---------------------------------------------------------------------------
def _rope_dev(cfg, rope_table, n_pos, device):
    if rope_table is None:
        rope_table = mla_rope_table(cfg, n_pos).to(device)
    _dev(rope_table, "rope_table", torch.float32)
    if rope_table.dim() != 2 or rope_table.shape[1] != cfg.rope_dim:
        raise ValueError("rope_table must be [positions, rope_dim]")
    return rope_table


def mla_cache_append(cfg: MLAConfig, x, w_dkv, kv_norm_w, positions, slot_mapping, kv_pool,
                     rope_table=None, workspace=None, stream=None) -> None:
    """Write [RMSNorm(x W_DKV[:, :R]) g | RoPE(x W_DKV[:, R:])] rows into kv_pool."""
    dt = cfg.torch_dtype
    n = x.shape[0]
    _dev(x, "x", dt, (n, cfg.d_model))
    _dev(w_dkv, "w_dkv", dt, (cfg.d_model, cfg.row))
    _dev(kv_norm_w, "kv_norm_w", torch.float32, (cfg.kv_lora_rank,))
    _dev(positions, "positions", torch.int32, (n,))
    _dev(slot_mapping, "slot_mapping", torch.int32, (n,))
    nb = kv_pool.shape[0]
    _dev(kv_pool, "kv_pool", cfg.pool_dtype, (nb, cfg.block_size, cfg.pool_row))
    if rope_table is None:
        rope_table = _rope_dev(cfg, None, int(positions.max().item()) + 1, x.device)
    rope_table = _rope_dev(cfg, rope_table, 0, x.device)
    ws = _workspace(workspace, mla_cache_append_workspace_size(cfg, n), x.device)
    check(lib.mla_cache_append(_ref(cfg), x.data_ptr(), w_dkv.data_ptr(), kv_norm_w.data_ptr(),
                               rope_table.data_ptr(), rope_table.shape[0], positions.data_ptr(),
                               slot_mapping.data_ptr(), n, kv_pool.data_ptr(), nb, ws.data_ptr(),
                               ws.numel(), _stream(stream)), "mla_cache_append")


def mla_prefill(cfg: MLAConfig, x, weights: dict, kv_pool, block_table, start_pos,
                max_start_pos: int, rope_table=None, out=None, workspace=None, stream=None):
    """out [B, T, H, Dv]: append T tokens per sequence and attend causally.

    weights: dict with w_q (q_lora_rank == 0) or w_dq, q_norm_w, w_uq; and
    w_dkv, kv_norm_w, w_uk, w_uv.  Norm gains are float32.
    """
    dt = cfg.torch_dtype
    B, T = x.shape[0], x.shape[1]
    H = cfg.num_heads
    QW = H * (cfg.qk_nope_dim + cfg.rope_dim)
    _dev(x, "x", dt, (B, T, cfg.d_model))
    w = weights
    null = 0
    if cfg.q_lora_rank:
        p_wq = null
        p_wdq = _dev(w["w_dq"], "w_dq", dt, (cfg.d_model, cfg.q_lora_rank))
        p_qn = _dev(w["q_norm_w"], "q_norm_w", torch.float32, (cfg.q_lora_rank,))
        p_wuq = _dev(w["w_uq"], "w_uq", dt, (cfg.q_lora_rank, QW))
    else:
        p_wq = _dev(w["w_q"], "w_q", dt, (cfg.d_model, QW))
        p_wdq = p_qn = p_wuq = null
    p_wdkv = _dev(w["w_dkv"], "w_dkv", dt, (cfg.d_model, cfg.row))
    p_kvn = _dev(w["kv_norm_w"], "kv_norm_w", torch.float32, (cfg.kv_lora_rank,))
    p_wuk = _dev(w["w_uk"], "w_uk", dt, (cfg.uk_heads, cfg.qk_nope_dim, cfg.kv_lora_rank))
    p_wuv = _dev(w["w_uv"], "w_uv", dt, (cfg.uk_heads, cfg.kv_lora_rank, cfg.v_dim))
    nb, mb = _pool_args(cfg, kv_pool, block_table, B)
    _dev(start_pos, "start_pos", torch.int32, (B,))
    rope_table = _rope_dev(cfg, rope_table, int(max_start_pos) + T, x.device)
    if out is None:
        out = torch.empty((B, T, H, cfg.v_dim), dtype=dt, device=x.device)
    _dev(out, "out", dt, (B, T, H, cfg.v_dim))
    ws = _workspace(workspace, mla_prefill_workspace_size(cfg, B, T, int(max_start_pos) + T),
                    x.device)
    check(lib.mla_prefill(_ref(cfg), x.data_ptr(), p_wq, p_wdq, p_qn, p_wuq, p_wdkv, p_kvn, p_wuk,
                          p_wuv, rope_table.data_ptr(), rope_table.shape[0], kv_pool.data_ptr(),
                          nb, block_table.data_ptr(), mb, start_pos.data_ptr(),
                          int(max_start_pos), B, T, out.data_ptr(), ws.data_ptr(), ws.numel(),
                          _stream(stream)), "mla_prefill")
    return out


# ---------------------------------------------------------------------------
# after the heads
# ---------------------------------------------------------------------------
def mla_output_gate_projection(cfg: MLAConfig, x, head_out, w_o, w_g=None, out=None,
                               workspace=None, stream=None) -> torch.Tensor:
    """out [n, M] = (head_out * sigmoid(x W_G)) W_O, or head_out W_O without a
    gate (see mla_output_gate_projection in include/mla.h).  x [n, M];
    head_out [n, H, Dv] (or [n, H*Dv]); w_g [M, H*Dv] or None; w_o [H*Dv, M]."""
    dt = cfg.torch_dtype
    n, M, HV = x.shape[0], cfg.d_model, cfg.num_heads * cfg.v_dim
    _dev(x, "x", dt, (n, M))
    _dev(head_out, "head_out", dt)
    if head_out.numel() != n * HV:
        raise ValueError(f"head_out must hold {n} x {HV} values")
    _dev(w_o, "w_o", dt, (HV, M))
    if w_g is not None:
        _dev(w_g, "w_g", dt, (M, HV))
    if out is None:
        out = torch.empty((n, M), dtype=dt, device=x.device)
    _dev(out, "out", dt, (n, M))
    ws_ptr, ws_len = 0, 0
    if w_g is not None:
        need = mla_output_gate_workspace_size(cfg, n)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr, ws_len = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib.mla_output_gate_projection(_ref(cfg), x.data_ptr(), head_out.data_ptr(),
                                         0 if w_g is None else w_g.data_ptr(), w_o.data_ptr(), n,
                                         out.data_ptr(), ws_ptr, ws_len, _stream(stream)),
          "mla_output_gate_projection")
    return out


# ---------------------------------------------------------------------------
# Measurement probes (include/mla.h): the HBM read, bf16 MFMA and LDS read
# ceilings.
# ---------------------------------------------------------------------------
def mla_probe_sink(device=None) -> torch.Tensor:
    """A device buffer large enough for the probes' per-thread outputs."""
    return torch.empty(lib.mla_probe_sink_bytes(), dtype=torch.uint8,
                       device=device or torch.device("cuda"))


def mla_probe_hbm_read(buf: torch.Tensor, mode: int, sink: torch.Tensor, stream=None) -> None:
    """Read all of `buf` (device) once: mode 0 vector loads, mode 1
    direct-to-LDS loads of 36864-byte pieces."""
    _dev(buf, "buf", buf.dtype, tuple(buf.shape))
    _dev(sink, "sink", torch.uint8, (lib.mla_probe_sink_bytes(),))
    check(lib.mla_probe_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), mode,
                                 sink.data_ptr(), _stream(stream)), "mla_probe_hbm_read")


def mla_probe_mfma(workgroups: int, iterations: int, sink: torch.Tensor, stream=None) -> int:
    """Run the MFMA probe; returns the FLOPs it executes."""
    _dev(sink, "sink", torch.uint8, (lib.mla_probe_sink_bytes(),))
    check(lib.mla_probe_mfma(workgroups, iterations, sink.data_ptr(), _stream(stream)),
          "mla_probe_mfma")
    return workgroups * 4 * iterations * 4 * 32768


def mla_probe_lds_read(width: int, iterations: int, sink: torch.Tensor, stream=None) -> int:
    """Run the LDS read probe (16- or 8-byte reads per lane, one workgroup
    per compute unit); returns the bytes it reads."""
    _dev(sink, "sink", torch.uint8, (lib.mla_probe_sink_bytes(),))
    check(lib.mla_probe_lds_read(width, iterations, sink.data_ptr(), _stream(stream)),
          "mla_probe_lds_read")
    cus = torch.cuda.get_device_properties(sink.device).multi_processor_count
    return cus * 8 * iterations * 8 * 64 * width
