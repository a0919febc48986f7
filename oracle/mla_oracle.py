"""MLA latent-KV oracle: definitions written out in plain numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 by default;
``wd=np.float32`` runs the same definitions in float32.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "store_round", "rope_angles", "apply_rope", "rms_norm", "kv_latent_rows",
    "query_heads", "reconstruct_kv", "naive_attention", "absorb_query",
    "latent_attention", "project_output", "absorbed_attention",
    "chunk_partials", "merge_partials", "gather_sequence", "decode",
    "append_rows", "attend_tokens", "layer_forward", "incremental_decode",
    "softmax_scale", "DEFAULT_EPS", "DEFAULT_THETA", "sigmoid", "output_gate_projection",
    "head_matrices",
]

DEFAULT_EPS = 1e-6
DEFAULT_THETA = 10000.0


def _cfg(cfg, key, default=None):
    v = cfg.get(key, default) if isinstance(cfg, dict) else getattr(cfg, key, default)
    return default if v is None else v


def _w(weights, key):
    if isinstance(weights, dict):
        return weights.get(key)
    return getattr(weights, key, None)


def softmax_scale(cfg) -> float:
    """1/sqrt(Dn + Dr): the scale uses the entire per-head Q/K width, nope and
    rope parts together (GatedMLA docs, "Observe logits, then compute causal
    attention": SDPA scales by the full head dimension D + D_s)."""
    s = _cfg(cfg, "softmax_scale", 0.0)
    if s:
        return float(s)
    return 1.0 / math.sqrt(_cfg(cfg, "qk_nope_dim") + _cfg(cfg, "rope_dim"))


# --------------------------------------------------------------------------
# Storage rounding of cache rows
# --------------------------------------------------------------------------
def store_round(x: np.ndarray, storage: str) -> np.ndarray:
    """Value a tensor holds after being written in the storage dtype.

    'f64' keeps it, 'f32' rounds to float32, 'bf16' rounds once to the
    nearest bfloat16 (8 significant bits, ties to even), written out on the
    float64 bit pattern: keep the top 7 of the 52 stored mantissa bits.
    Reading: a cache row is rounded once, when stored, and every later read
    sees the stored value.  (Values here are normal and far from overflow.)
    """
    x = np.asarray(x, dtype=np.float64)
    if storage == "f64":
        return x.copy()
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)
    if storage == "bf16":
        bits = np.ascontiguousarray(x).view(np.uint64)
        drop = np.uint64(52 - 7)
        lsb = (bits >> drop) & np.uint64(1)
        half = np.uint64((1 << (52 - 7 - 1)) - 1)
        bits = ((bits + half + lsb) >> drop) << drop
        return bits.view(np.float64)
    raise ValueError(f"unknown storage dtype {storage!r}")


# --------------------------------------------------------------------------
# RoPE and RMSNorm
# --------------------------------------------------------------------------
def rope_angles(positions: Sequence[int], rope_dim: int, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Rotation angles [T, Dr/2]: position p times theta^(-2i/Dr).

    The pages only name the decoupled rope key (modeldna MLA module, "Under
    the hood") and give theta = 10000; the frequency ladder is the standard
    rotary one (reading).
    """
    if rope_dim % 2:
        raise ValueError("rope_dim must be even")
    i = np.arange(rope_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / rope_dim)
    p = np.asarray(positions, dtype=np.float64)
    return p[:, None] * inv_freq[None, :]


def apply_rope(x: np.ndarray, positions: Sequence[int], theta: float = DEFAULT_THETA,
               wd=np.float64) -> np.ndarray:
    """Rotate the last axis of x [T, ..., Dr] by each token's position.

    Half-split pairing (reading): element i pairs with i + Dr/2,
      y_i        = x_i cos a_i - x_{i+Dr/2} sin a_i
      y_{i+Dr/2} = x_{i+Dr/2} cos a_i + x_i sin a_i.
    cos/sin are evaluated in float64 and then cast to the working dtype.
    """
    x = np.asarray(x, dtype=wd)
    Dr = x.shape[-1]
    half = Dr // 2
    ang = rope_angles(positions, Dr, theta)
    shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    cos = np.cos(ang).astype(wd).reshape(shape)
    sin = np.sin(ang).astype(wd).reshape(shape)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float = DEFAULT_EPS, wd=np.float64) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis (GatedMLA docs,
    "Projection geometry and stored weights": q_rmsnorm and kv_rmsnorm
    normalise the compressed features; eps is a reading)."""
    x = np.asarray(x, dtype=wd)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + wd(eps)) * np.asarray(gain, dtype=wd)


# --------------------------------------------------------------------------
# Projections
# --------------------------------------------------------------------------
def kv_latent_rows(x, w_dkv, kv_norm_w, positions, kv_lora_rank: int,
                   eps: float = DEFAULT_EPS, theta: float = DEFAULT_THETA, wd=np.float64):
    """Down-project hidden states to the cached state of each token.

    z = x W_DKV is split into the compressed latent c_raw (first R values)
    and the shared rope key k_pe (the rest) (GatedMLA docs, "Build per-head
    Q, K and V"; modeldna MLA module, "Under the hood": R + rope_dim cached
    values per token).  c = RMSNorm(c_raw) * g_kv; k_rope = RoPE(k_pe, pos).
    Returns (c [T, R], k_rope [T, Dr]).
    """
    x = np.asarray(x, dtype=wd)
    z = x @ np.asarray(w_dkv, dtype=wd)
    c = rms_norm(z[:, :kv_lora_rank], kv_norm_w, eps, wd)
    k_rope = apply_rope(z[:, kv_lora_rank:], positions, theta, wd)
    return c, k_rope


def query_heads(x, positions, weights, cfg, wd=np.float64):
    """Per-head queries [T, H, Dn] and rotated rope queries [T, H, Dr].

    With a query rank: q = RMSNorm(x W_DQ) * g_q, then W_UQ (GatedMLA docs,
    "Projection geometry and stored weights"; modeldna MLA module, "Under the
    hood": q_lora_rank).  Without one: q = x W_Q (reading for the tiny
    layer).  Each head's slice is [nope | rope]; the rope part is rotated at
    the token's position.
    """
    H, Dn, Dr = _cfg(cfg, "num_heads"), _cfg(cfg, "qk_nope_dim"), _cfg(cfg, "rope_dim")
    eps, theta = _cfg(cfg, "rms_eps", DEFAULT_EPS), _cfg(cfg, "rope_theta", DEFAULT_THETA)
    x = np.asarray(x, dtype=wd)
    if _w(weights, "w_dq") is not None:
        cq = rms_norm(x @ np.asarray(_w(weights, "w_dq"), dtype=wd), _w(weights, "q_norm_w"), eps, wd)
        q = cq @ np.asarray(_w(weights, "w_uq"), dtype=wd)
    else:
        q = x @ np.asarray(_w(weights, "w_q"), dtype=wd)
    q = q.reshape(x.shape[0], H, Dn + Dr)
    return q[..., :Dn], apply_rope(q[..., Dn:], positions, theta, wd)


# --------------------------------------------------------------------------
# Attention: the naive (reconstruction) path
# --------------------------------------------------------------------------
def reconstruct_kv(c, k_rope, w_uk, w_uv, wd=np.float64):
    """Materialise per-head K and V from the latent (GatedMLA docs, "Build
    per-head Q, K and V").

    K_nope[j,h,d] = sum_r W_UK[h,d,r] c[j,r];  V[j,h,e] = sum_r c[j,r] W_UV[h,r,e].
    The shared rope key is broadcast to every head and placed after the
    content key: K[j,h] = [K_nope[j,h] | k_rope[j]].
    """
    c = np.asarray(c, dtype=wd)
    w_uk = np.asarray(w_uk, dtype=wd)
    w_uv = np.asarray(w_uv, dtype=wd)
    H = w_uk.shape[0]
    k_nope = np.matmul(w_uk[None], c[:, None, :, None])[..., 0]          # [Tk, H, Dn]
    v = np.matmul(c[:, None, None, :], w_uv[None])[:, :, 0, :]           # [Tk, H, Dv]
    shared = np.broadcast_to(np.asarray(k_rope, dtype=wd)[:, None, :],
                             (c.shape[0], H, k_rope.shape[-1]))
    return np.concatenate([k_nope, shared], axis=-1), v


def _causal_softmax(s, q_pos, k_pos):
    """Softmax over keys with j allowed iff k_pos[j] <= q_pos[i]; the maximum
    is subtracted first.  s: [H, Tq, Tk]."""
    allowed = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    if not np.all(allowed.any(axis=1)):
        raise ValueError("a query row has no visible key")
    s = np.where(allowed[None], s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / np.sum(p, axis=-1, keepdims=True)


def naive_attention(q_nope, q_rope, c, k_rope, w_uk, w_uv, scale, q_pos,
                    k_pos=None, wd=np.float64):
    """Reconstruction path: causal softmax attention over materialised K, V.

    s[h,i,j] = scale * ([q_nope | q_rope][i,h] . K[j,h]) for k_pos[j] <= q_pos[i]
    (GatedMLA docs, "Observe logits, then compute causal attention": causal,
    dropout 0, scale over the full Q/K width).  Returns o [Tq, H, Dv].
    """
    k, v = reconstruct_kv(c, k_rope, w_uk, w_uv, wd)
    q = np.concatenate([np.asarray(q_nope, dtype=wd), np.asarray(q_rope, dtype=wd)], axis=-1)
    if k_pos is None:
        k_pos = np.arange(k.shape[0])
    s = np.matmul(q.transpose(1, 0, 2), k.transpose(1, 2, 0)) * wd(scale)   # [H, Tq, Tk]
    p = _causal_softmax(s, q_pos, k_pos)
    return np.matmul(p, v.transpose(1, 0, 2)).transpose(1, 0, 2)            # [Tq, H, Dv]


# --------------------------------------------------------------------------
# Attention: the absorbed path
# --------------------------------------------------------------------------
def absorb_query(q_nope, w_uk, wd=np.float64):
    """q_lat[i,h,r] = sum_d q_nope[i,h,d] W_UK[h,d,r]: W_UK folded into the
    query (modeldna MLA module, "Under the hood": the up-projections can be
    absorbed into the query and output projections)."""
    q = np.asarray(q_nope, dtype=wd).transpose(1, 0, 2)                   # [H, Tq, Dn]
    return np.matmul(q, np.asarray(w_uk, dtype=wd)).transpose(1, 0, 2)    # [Tq, H, R]


def latent_attention(q_lat, q_rope, c, k_rope, scale, q_pos, k_pos=None, wd=np.float64):
    """Attention directly on the cached latent rows.

    s[h,i,j] = scale * (q_lat[i,h] . c[j] + q_rope[i,h] . k_rope[j]);
    P = causal softmax over j; o_lat[i,h] = sum_j P[h,i,j] c[j].
    Returns o_lat [Tq, H, R].
    """
    c = np.asarray(c, dtype=wd)
    kr = np.asarray(k_rope, dtype=wd)
    if k_pos is None:
        k_pos = np.arange(c.shape[0])
    ql = np.asarray(q_lat, dtype=wd).transpose(1, 0, 2)                   # [H, Tq, R]
    qr = np.asarray(q_rope, dtype=wd).transpose(1, 0, 2)                  # [H, Tq, Dr]
    s = (np.matmul(ql, c.T) + np.matmul(qr, kr.T)) * wd(scale)
    p = _causal_softmax(s, q_pos, k_pos)
    return np.matmul(p, c).transpose(1, 0, 2)


def project_output(o_lat, w_uv, wd=np.float64):
    """out[i,h,e] = sum_r o_lat[i,h,r] W_UV[h,r,e]: W_UV applied after P.c
    (modeldna MLA module, "Under the hood")."""
    o = np.asarray(o_lat, dtype=wd).transpose(1, 0, 2)
    return np.matmul(o, np.asarray(w_uv, dtype=wd)).transpose(1, 0, 2)


def absorbed_attention(q_nope, q_rope, c, k_rope, w_uk, w_uv, scale, q_pos,
                       k_pos=None, wd=np.float64):
    """Absorbed path end to end; returns (o [Tq, H, Dv], o_lat [Tq, H, R])."""
    q_lat = absorb_query(q_nope, w_uk, wd)
    o_lat = latent_attention(q_lat, q_rope, c, k_rope, scale, q_pos, k_pos, wd)
    return project_output(o_lat, w_uv, wd), o_lat


# --------------------------------------------------------------------------
# Split-KV partials for one query row
# --------------------------------------------------------------------------
def chunk_partials(q_lat, q_rope, c, k_rope, scale, chunk: int, wd=np.float64):
    """Per-chunk softmax statistics for one query row attending to all keys.

    q_lat [H, R], q_rope [H, Dr], c [L, R], k_rope [L, Dr].  For chunk s of
    keys: m_s = max_j s_j, l_s = sum_j exp(s_j - m_s), O_s = sum_j exp(s_j - m_s) c_j.
    The pages do not describe this split; it is the log-sum-exp
    decomposition of one softmax.  Returns (m [S, H], l [S, H], O [S, H, R]).
    """
    c = np.asarray(c, dtype=wd)
    kr = np.asarray(k_rope, dtype=wd)
    ql = np.asarray(q_lat, dtype=wd)
    qr = np.asarray(q_rope, dtype=wd)
    ms, ls, os_ = [], [], []
    for s0 in range(0, c.shape[0], chunk):
        cc, kk = c[s0:s0 + chunk], kr[s0:s0 + chunk]
        s = (ql @ cc.T + qr @ kk.T) * wd(scale)                          # [H, n]
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        ms.append(m)
        ls.append(p.sum(axis=1))
        os_.append(p @ cc)
    return np.stack(ms), np.stack(ls), np.stack(os_)


def merge_partials(m, l, O):
    """Combine chunk statistics: M = max_s m_s, w_s = exp(m_s - M),
    o_lat = sum_s w_s O_s / sum_s w_s l_s.  Returns o_lat [H, R]."""
    M = np.max(m, axis=0)
    w = np.exp(m - M[None])
    return np.sum(w[..., None] * O, axis=0) / np.sum(w * l, axis=0)[..., None]


# --------------------------------------------------------------------------
# Paged cache and decode
# --------------------------------------------------------------------------
def gather_sequence(pool, block_table_row, seq_len: int) -> np.ndarray:
    """Cached rows 0..seq_len-1 of one sequence from a paged pool.

    pool [num_blocks, block_size, row]; logical token j lives in physical
    page block_table_row[j // block_size] at offset j % block_size (the
    ticket's PagedKVCache pool with a block allocator, "Description").
    """
    bs = pool.shape[1]
    j = np.arange(seq_len)
    return np.asarray(pool)[np.asarray(block_table_row)[j // bs], j % bs]


def head_matrices(w, H: int) -> np.ndarray:
    """One matrix per query head from G shared ones ([G, ...] -> [H, ...]):
    head h uses matrix h // (H / G), i.e. consecutive heads share, the way the
    tutorial's experiment ("ARCH-MLA. Multihead Latent Attention", 5.1)
    rebuilds 4 key/value heads for 16 query heads (reading: the grouping of
    grouped-query attention).  G = H returns w unchanged."""
    w = np.asarray(w)
    G = w.shape[0]
    if H % G:
        raise ValueError(f"{G} matrices cannot be shared evenly by {H} heads")
    return np.repeat(w, H // G, axis=0)


def decode(q_nope, q_rope, w_uk, w_uv, pool, block_table, seq_lens, cfg,
           path: str = "absorbed", wd=np.float64, batch_ids=None):
    """One decode step for a batch of sequences over a paged latent cache.

    The current token's row is already in the cache, so sequence b attends
    to its rows 0..seq_lens[b]-1 (ticket, "Description": project the new
    token, concat with the cache, attend).  q_rope is already rotated.
    w_uk / w_uv hold H matrices, or G < H shared by consecutive heads
    (``head_matrices``).
    Returns (o [B, H, Dv], o_lat [B, H, R] or None for the naive path).
    """
    H = np.asarray(q_nope).shape[1]
    w_uk, w_uv = head_matrices(w_uk, H), head_matrices(w_uv, H)
    R = _cfg(cfg, "kv_lora_rank")
    scale = softmax_scale(cfg)
    ids = range(len(seq_lens)) if batch_ids is None else batch_ids
    outs, lats = [], []
    for b in ids:
        L = int(seq_lens[b])
        rows = np.asarray(gather_sequence(pool, block_table[b], L), dtype=wd)
        c, kr = rows[:, :R], rows[:, R:]
        qn = np.asarray(q_nope[b], dtype=wd)[None]
        qr = np.asarray(q_rope[b], dtype=wd)[None]
        if path == "naive":
            outs.append(naive_attention(qn, qr, c, kr, w_uk, w_uv, scale, [L - 1], wd=wd)[0])
        elif path == "absorbed":
            o, ol = absorbed_attention(qn, qr, c, kr, w_uk, w_uv, scale, [L - 1], wd=wd)
            outs.append(o[0])
            lats.append(ol[0])
        else:
            raise ValueError(path)
    return np.stack(outs), (np.stack(lats) if lats else None)


# --------------------------------------------------------------------------
# Whole layer: append + attend
# --------------------------------------------------------------------------
def append_rows(x, positions, weights, cfg, storage: str = "f64", wd=np.float64) -> np.ndarray:
    """Cache rows [T, R + Dr] = [c | k_rope] for new tokens, rounded to the
    storage dtype (the append step; modeldna MLA module, "Under the hood")."""
    c, kr = kv_latent_rows(x, _w(weights, "w_dkv"), _w(weights, "kv_norm_w"), positions,
                           _cfg(cfg, "kv_lora_rank"), _cfg(cfg, "rms_eps", DEFAULT_EPS),
                           _cfg(cfg, "rope_theta", DEFAULT_THETA), wd)
    rows = np.concatenate([c, kr], axis=-1)
    if storage == "fp8":  # FP8 latent, bf16 rope key (fp8_cache)
        from .fp8_cache import fp8_store_rows
        return fp8_store_rows(rows, _cfg(cfg, "kv_lora_rank")).astype(wd)
    return store_round(rows, storage).astype(wd)


def attend_tokens(x, positions, weights, cfg, rows, path: str = "absorbed",
                  wd=np.float64, q_block: int = 256):
    """Outputs [T, H, Dv] of new tokens at ``positions`` attending causally to
    cached rows [Tk, R + Dr] (key j at position j).  Query rows are handled
    in independent blocks of ``q_block`` only to bound memory."""
    R = _cfg(cfg, "kv_lora_rank")
    rows = np.asarray(rows, dtype=wd)
    c, kr = rows[:, :R], rows[:, R:]
    q_nope, q_rope = query_heads(x, positions, weights, cfg, wd)
    scale = softmax_scale(cfg)
    pos = np.asarray(positions)
    out = []
    for s in range(0, len(pos), q_block):
        sl = slice(s, s + q_block)
        if path == "naive":
            o = naive_attention(q_nope[sl], q_rope[sl], c, kr, _w(weights, "w_uk"),
                                _w(weights, "w_uv"), scale, pos[sl], wd=wd)
        else:
            o, _ = absorbed_attention(q_nope[sl], q_rope[sl], c, kr, _w(weights, "w_uk"),
                                      _w(weights, "w_uv"), scale, pos[sl], wd=wd)
        out.append(o)
    return np.concatenate(out, axis=0)


def layer_forward(x, weights, cfg, storage: str = "f64", path: str = "absorbed",
                  wd=np.float64, start_pos: int = 0, prior_rows: Optional[np.ndarray] = None):
    """Full causal forward of T new tokens of one sequence.

    Positions are start_pos .. start_pos + T - 1 (0-based absolute, reading);
    ``prior_rows`` holds the already cached rows 0..start_pos-1.  The new
    rows are appended (rounded at the store) and every new token attends to
    rows 0..its own position.  Returns (o [T, H, Dv], new rows [T, row]).
    """
    T = np.asarray(x).shape[0]
    positions = np.arange(start_pos, start_pos + T)
    new_rows = append_rows(x, positions, weights, cfg, storage, wd)
    rows = new_rows if prior_rows is None else np.concatenate(
        [np.asarray(prior_rows, dtype=wd), new_rows], axis=0)
    if rows.shape[0] != start_pos + T:
        raise ValueError("prior_rows must hold exactly start_pos rows")
    return attend_tokens(x, positions, weights, cfg, rows, path, wd), new_rows


def incremental_decode(x, weights, cfg, storage: str = "f64", path: str = "absorbed",
                       wd=np.float64, n_prefill: int = 0):
    """Token-by-token generation path: the first ``n_prefill`` tokens go
    through one full forward, then each later token is projected alone,
    appended to the cache and attends over it (ticket, "Description").
    Returns o [T, H, Dv] for all T tokens."""
    x = np.asarray(x)
    outs = []
    rows = np.zeros((0, _cfg(cfg, "kv_lora_rank") + _cfg(cfg, "rope_dim")), dtype=wd)
    if n_prefill:
        o, rows = layer_forward(x[:n_prefill], weights, cfg, storage, path, wd)
        outs.append(o)
    for t in range(n_prefill, x.shape[0]):
        o, new = layer_forward(x[t:t + 1], weights, cfg, storage, path, wd,
                               start_pos=t, prior_rows=rows)
        rows = np.concatenate([rows, new], axis=0)
        outs.append(o)
    return np.concatenate(outs, axis=0)


def sigmoid(z, wd=np.float64):
    """The logistic function 1 / (1 + e^-z), the output gate's squashing."""
    z = np.asarray(z, dtype=wd)
    return 1.0 / (1.0 + np.exp(-z))


def output_gate_projection(head_out, x, w_o, w_g=None, wd=np.float64):
    """The layer's attention contribution from its head outputs ("GatedMLA"
    docs, "Output projection and optional gate"): the head outputs are laid
    side by side as one row of H*Dv values per token; with a gate they are
    multiplied elementwise by sigmoid(x W_G), where x is the layer input (not
    the attention result); then W_O maps them back to the model width.  No
    residual is added.  head_out [n, H, Dv] or [n, H*Dv]; x [n, M];
    w_g [M, H*Dv] or None; w_o [H*Dv, M].  Returns [n, M]."""
    h = np.asarray(head_out, dtype=wd)
    h = h.reshape(h.shape[0], -1)
    if w_g is not None:
        h = h * sigmoid(np.asarray(x, dtype=wd) @ np.asarray(w_g, dtype=wd), wd)
    return h @ np.asarray(w_o, dtype=wd)
