/*
 * mla.h -- C ABI of an MI355X (gfx950) library for Multi-head Latent
 * Attention (MLA) over a paged, compressed latent KV cache.
 *
 * The method (modeldna "MLA" module, "Under the hood"; "GatedMLA" docs,
 * "Projection geometry and stored weights" and "Build per-head Q, K and V"):
 * each token of a layer caches one row [c (kv_lora_rank R) | k_rope (rope_dim Dr)],
 * where c = RMSNorm(x W_DKV[:, :R]) * g_kv is the compressed latent and k_rope
 * = RoPE(x W_DKV[:, R:], position) is a rope key shared by all heads.  W_UK
 * is absorbed into the query and W_UV applied after attention, so attention
 * runs on the latent rows directly:
 *   q_lat[h] = q_nope[h] W_UK[h]                          (R values per head)
 *   s[h, j]  = scale * (q_lat[h] . c_j + q_rope[h] . k_rope_j)
 *   P        = softmax_j(s)     (causal: keys up to the query's position)
 *   o_lat[h] = sum_j P[h, j] c_j;   out[h] = o_lat[h] W_UV[h]  (Dv values)
 * Per-head K and V are never materialised.  scale defaults to
 * 1/sqrt(qk_nope_dim + rope_dim), the full per-head Q/K width ("GatedMLA"
 * docs, "Observe logits, then compute causal attention").
 *
 * Conventions for every call below:
 *   - Tensor pointers are DEVICE pointers unless marked "host", dense
 *     row-major in the shapes given, 16-byte aligned, in the config's dtype
 *     (float32 or bfloat16) unless a type is named.  RMSNorm gains and the
 *     RoPE table are float32 in every dtype.  Accumulation is float32.
 *   - The caller owns every buffer.  The library allocates no memory and keeps
 *     no state between calls; it writes only the outputs and the workspace
 *     named in a call.  `stream` is a hipStream_t (NULL = default stream);
 *     every device call is asynchronous on it.  Calls that share a
 *     workspace or write the same pool rows must be ordered on one stream.
 *   - Validation runs on the host before anything is enqueued.  An invalid
 *     call returns MLA_ERR_INVALID_ARG (or MLA_ERR_UNSUPPORTED /
 *     MLA_ERR_WORKSPACE), enqueues nothing, writes nothing, and
 *     mla_last_error() says why.  Counts (batch, n_tokens, q_len, n_rows)
 *     must be positive: an empty call is MLA_ERR_INVALID_ARG, not a no-op.
 *     Device-resident integers (page tables, sequence lengths, positions,
 *     slots) are trusted: the caller keeps them within the sizes passed.  Page-table entries past the pages a sequence
 *     uses may hold any value: they are read (the decode prologue guesses
 *     pages from them) but never followed outside [0, num_blocks).  A failed
 *     launch returns MLA_ERR_HIP.
 *   - Cache pool: [num_blocks, block_size, R + Dr].  Logical token j of
 *     sequence b lives at page block_table[b * max_blocks_per_seq + j / block_size],
 *     offset j % block_size (the ticket "MLA + KV cache (Tier 3 #5)",
 *     "Description": a PagedKVCache pool with a block allocator).  A
 *     contiguous cache is the same pool with an identity page table.
 *   - FP8 cache (cache_dtype MLA_CACHE_FP8_E4M3, bf16 configs): the softved
 *     article "Multi-Head Latent Attention" advises quantizing the cache on
 *     top of MLA ("Practical Implementation Tips for MLA in LLM Serving")
 *     without naming a format; here a row is R + 2 Dr + 16 bytes (656 at
 *     R=512, Dr=64): R codes of c / s in OCP FP8 E4M3 (bias 7, largest
 *     finite 448, round to nearest even), the Dr rope values in bf16, the
 *     row's scale s as float32, 12 zero bytes.  s is the smallest power of
 *     two with max|c| <= 448 s (1 for an all-zero c), so s * code is exact
 *     in bf16.  The pool is then [num_blocks, block_size, R + 2 Dr + 16]
 *     bytes.  Decode reads and mla_cache_append writes such pools (R=512,
 *     Dr=64); mla_prefill takes them when Dn = Dv = 128 as well (else
 *     MLA_ERR_UNSUPPORTED).
 */
#ifndef MLA_LATENT_KV_H
#define MLA_LATENT_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 5

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* a size, pointer or config field is out of range */
  MLA_ERR_UNSUPPORTED = 2, /* valid, but no kernel for this shape/dtype      */
  MLA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required       */
  MLA_ERR_HIP = 4          /* a HIP runtime call or a kernel launch failed   */
} mla_status;

typedef enum mla_dtype { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

/* How cache rows are stored: in the config's dtype, or FP8 (see above). */
typedef enum mla_cache_dtype { MLA_CACHE_SAME = 0, MLA_CACHE_FP8_E4M3 = 1 } mla_cache_dtype;

/* One MLA layer's geometry ("GatedMLA" docs, "Projection geometry and stored
 * weights": W_DQ M->Rq, W_DKV M->R+Dr, W_UQ Rq->H(Dn+Dr), the KV
 * up-projection split into W_UK [H,Dn,R] and W_UV [H,R,Dv]). */
typedef struct mla_config {
  int32_t num_heads;    /* H > 0                                               */
  int32_t kv_lora_rank; /* R > 0: latent width                                 */
  int32_t rope_dim;     /* Dr > 0, even: shared rope key width                 */
  int32_t qk_nope_dim;  /* Dn > 0                                              */
  int32_t v_dim;        /* Dv > 0                                              */
  int32_t d_model;      /* M >= 0; 0 when only decode calls are made; else
                           R < M and q_lora_rank < M                           */
  int32_t q_lora_rank;  /* Rq >= 0; 0 = queries through one matrix W_Q          */
  int32_t block_size;   /* tokens per cache page, > 0                          */
  float softmax_scale;  /* >= 0; 0 = 1/sqrt(Dn + Dr)                           */
  float rms_eps;        /* >= 0, RMSNorm epsilon                               */
  float rope_theta;     /* > 0, RoPE base                                      */
  int32_t dtype;        /* mla_dtype of every tensor (storage); fp32 accumulate */
  int32_t cache_dtype;  /* mla_cache_dtype of the cache rows; FP8 needs bf16   */
  int32_t kv_groups;    /* G >= 0: 0 = one W_UK and W_UV per head; else H % G
                           == 0 and heads g H/G .. (g+1) H/G - 1 share
                           W_UK[g], W_UV[g] (w_uk [G, Dn, R], w_uv [G, R, Dv])  */
  int32_t split_workgroups; /* >= 0: workgroups per head group of the split-KV
                           decode attention (kv_lora_rank 512 kernels), each
                           taking an equal share of the batch's 32-token tiles;
                           0 = one per compute unit in total; else a multiple
                           of 8, at most 8192.  Results do not depend on it
                           beyond float32 rounding (the partition is free).  */
  int32_t prefill_attention; /* form of mla_prefill's attention: 0 = the one
                           needing fewer FLOPs, 1 = on the latent rows
                           (absorbed), 2 = through per-head keys and values
                           (bf16, R = 512, Dr = 64, Dn = Dv = 128 only; an FP8
                           cache takes 0 or 2).  Same result up to rounding. */
  int32_t decode_attention; /* form of mla_decode's attention: 0 or 1 = on the
                           latent rows (absorbed: W_UK folded into the query,
                           W_UV applied after), 2 = through per-head keys and
                           values rebuilt from the latent rows for the step
                           (K_nope = c W_UK^T, V = c W_UV per kv group, then
                           grouped attention over them; bf16, Dn = Dv = 64,
                           Dr = 64, at most 16 query heads per kv group).  The
                           reconstruction form of the tutorial's mechanism
                           experiment ("ARCH-MLA", 5.1); same result up to
                           rounding, more memory and bytes moved.            */
} mla_config;

/* ---- library information ------------------------------------------------ */
int32_t mla_abi_version(void);
const char* mla_status_string(int32_t status);
/* Message for the last failing call made on this thread ("" if none). */
const char* mla_last_error(void);

/* Checks every field of *cfg (rules in the struct comments).  MLA_OK or
 * MLA_ERR_INVALID_ARG.  Host only. */
mla_status mla_validate_config(const mla_config* cfg);

/* Values per cached token per layer, R + Dr (576 at R=512, Dr=64: modeldna
 * "MLA" module, cache-size table).  -1 if *cfg is invalid.  Host only. */
int64_t mla_cache_row_elems(const mla_config* cfg);
/* Bytes per cached token per layer, (R + Dr) * sizeof(dtype): 1152 for
 * bf16 at R=512, Dr=64 (same table); R + 2 Dr + 16 for an FP8 cache (656).
 * -1 if *cfg is invalid.  Host only. */
int64_t mla_cache_bytes_per_token(const mla_config* cfg);

/* RoPE table for positions 0..num_positions-1, written to HOST memory
 * host_table[num_positions][Dr] (float32): entries i < Dr/2 hold
 * cos(p * theta^(-2i/Dr)), entries Dr/2 + i hold the matching sin.  Computed
 * in double precision, rounded to float.  Rotation pairs element i with
 * element i + Dr/2 (the rope key is only named on the pages: modeldna "MLA"
 * module, "Under the hood"; the pairing is this library's convention). */
mla_status mla_rope_table(const mla_config* cfg, int32_t num_positions, float* host_table);

/* ---- decode (one new query token per sequence) -------------------------- */

/* Workspace bytes needed by the decode calls (mla_decode,
 * mla_latent_attention, mla_attention_partials, mla_combine_output) for this
 * batch and maximum length.  Scratch only: no initial contents required,
 * and a call reads only what it wrote itself.  Do not share one workspace
 * between calls that may run concurrently. */
mla_status mla_decode_workspace_size(const mla_config* cfg, int32_t batch, int32_t max_seq_len,
                                     size_t* bytes /* host out */);

/* One decode step for `batch` sequences (modeldna "MLA" module, "Under the
 * hood": absorbed up-projections; the ticket's "Description": the new token's
 * row is already in the cache and the token attends over the cache).
 *   q_nope [batch, H, Dn]; q_rope [batch, H, Dr], already rotated;
 *   w_uk [H, Dn, R]; w_uv [H, R, Dv] ([G, Dn, R], [G, R, Dv] with kv_groups
 *     G > 0: the tutorial "ARCH-MLA. Multihead Latent Attention", 5.1,
 *     rebuilds 4 key/value heads for 16 query heads);
 *   kv_pool [num_blocks, block_size, R + Dr];
 *   block_table int32 [batch, max_blocks_per_seq];
 *   seq_lens int32 [batch]: tokens in each sequence's cache including the
 *     current one, 1 <= seq_lens[b] <= max_seq_len (trusted);
 *   max_seq_len (host): bound on seq_lens, <= max_blocks_per_seq * block_size;
 *   out [batch, H, Dv] (written).
 * Runs mla_absorb_query, mla_latent_attention and mla_output_projection,
 * with q and o_lat staged in the workspace.  Shapes (bf16): the tuned
 * kernels take R = 512, Dr = 64, H a multiple of 32, block_size a power of
 * two >= 64, batch <= 1024; the narrow-latent kernels take R = 128 or 256,
 * Dr = 64, H a multiple of 16, any block_size (bf16 rows, no FP8);
 * anything else is MLA_ERR_UNSUPPORTED.  mla_attention_partials and
 * mla_combine_output exist for the tuned kernels only, and
 * mla_combine_output applies W_UV only without kv_groups. */
mla_status mla_decode(const mla_config* cfg, const void* q_nope, const void* q_rope,
                      const void* w_uk, const void* w_uv, const void* kv_pool, int32_t num_blocks,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* mla_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and arguments without the workspace, which
 * here is a device array inside the library's code object, one per GPU,
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB) large, held from the first call on that
 * GPU until the process ends.  The call allocates nothing.  A call whose
 * workspace (mla_decode_workspace_size) would exceed that size returns
 * MLA_ERR_WORKSPACE before anything is enqueued: at H = 64 up to about 250
 * sequences of any length fit, at H = 128 about 100.  Every call on one GPU
 * uses the same array and leaves its contents behind; no call needs it
 * cleared (a call reads only what it wrote).  Calls that may overlap on one
 * GPU (different streams, or host threads without ordering) race on it:
 * order them on one stream. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_noalloc(const mla_config* cfg, const void* q_nope, const void* q_rope,
                              const void* w_uk, const void* w_uv, const void* kv_pool,
                              int32_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                              int32_t max_seq_len, void* out, void* stream);

/* Stage 1 of decode: query absorption (modeldna "MLA" module, "Under the
 * hood": W_UK absorbed into the query).  For n_rows query rows:
 *   q_full[n, h, 0:R]    = scale * log2(e) * q_nope[n, h, :] W_UK[h]
 *   q_full[n, h, R:R+Dr] = scale * log2(e) * q_rope[n, h, :]
 * q_nope [n_rows, H, Dn], q_rope [n_rows, H, Dr], w_uk [H, Dn, R];
 * q_full [n_rows, H, R + Dr] (written).  The factor log2(e) lets the
 * attention take exponentials in base 2. */
mla_status mla_absorb_query(const mla_config* cfg, const void* q_nope, const void* q_rope,
                            const void* w_uk, int32_t n_rows, void* q_full, void* stream);

/* Stage 2 of decode: attention on the latent rows, split over KV chunks
 * and merged in the same call.  q_full as written by mla_absorb_query
 * ([batch, H, R + Dr]); o_lat [batch, H, R] (written) is
 * sum_j P[h, j] c_j with P the softmax over the sequence's seq_lens[b] rows.
 * Pool, table and lengths as in mla_decode.  Uses the workspace for split
 * partials (size from mla_decode_workspace_size). */
mla_status mla_latent_attention(const mla_config* cfg, const void* q_full, const void* kv_pool,
                                int32_t num_blocks, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, void* o_lat, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Stage 2 in two launches, for callers that overlap or time them apart.
 * mla_attention_partials runs the split-KV attention only: each workgroup
 * takes an equal share of the concatenated 64-token tiles of all sequences
 * and leaves, per (piece of a sequence, head), the piece's normalised latent
 * output with its running max and sum in the workspace (an internal format).
 * mla_combine_output then merges the pieces of each (sequence, head):
 *   o_lat = sum_s e_s O_s / sum_s e_s,  e_s = 2^(m_s - max_s m_s) l_s,
 * and writes o_lat [batch, H, R] when w_uv is NULL, else
 * out[b, h, :] = o_lat[b, h, :] W_UV[h] ([batch, H, Dv]).  Both calls take the
 * same config, batch, max_seq_len and workspace; bf16 only (the float32 path
 * has no split; use mla_latent_attention). */
mla_status mla_attention_partials(const mla_config* cfg, const void* q_full, const void* kv_pool,
                                  int32_t num_blocks, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t batch, int32_t max_seq_len, void* workspace,
                                  size_t workspace_bytes, void* stream);
mla_status mla_combine_output(const mla_config* cfg, const void* w_uv /* NULL: o_lat out */,
                              int32_t batch, int32_t max_seq_len, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Stage 3 of decode: output up-projection out[n, h, :] = o_lat[n, h, :] W_UV[h]
 * (modeldna "MLA" module, "Under the hood": W_UV applied after attention).
 * o_lat [n_rows, H, R]; w_uv [H, R, Dv]; out [n_rows, H, Dv] (written). */
mla_status mla_output_projection(const mla_config* cfg, const void* o_lat, const void* w_uv,
                                 int32_t n_rows, void* out, void* stream);

/* ---- cache append -------------------------------------------------------- */

mla_status mla_cache_append_workspace_size(const mla_config* cfg, int32_t n_tokens,
                                           size_t* bytes /* host out */);

/* Project new tokens into cache rows and store them ("GatedMLA" docs, "Build
 * per-head Q, K and V": W_DKV output split into the latent and the shared key;
 * "Projection geometry and stored weights": kv RMSNorm; modeldna "MLA" module,
 * "Under the hood": decoupled rope key):
 *   z = x[t] W_DKV;  c = z[:R] / sqrt(mean(z[:R]^2) + eps) * kv_norm_w;
 *   k_rope = RoPE(z[R:], positions[t]);  pool slot slot_mapping[t] <- [c | k_rope],
 * rounded to the storage dtype once, at the store.
 *   x [n_tokens, M]; w_dkv [M, R + Dr]; kv_norm_w float32 [R];
 *   rope_table float32 [rope_table_len, Dr] as made by mla_rope_table;
 *   positions int32 [n_tokens], each < rope_table_len (trusted);
 *   slot_mapping int32 [n_tokens]: page * block_size + offset, each
 *     < num_blocks * block_size; a negative slot skips that token (trusted). */
mla_status mla_cache_append(const mla_config* cfg, const void* x, const void* w_dkv,
                            const float* kv_norm_w, const float* rope_table, int32_t rope_table_len,
                            const int32_t* positions, const int32_t* slot_mapping, int32_t n_tokens,
                            void* kv_pool, int32_t num_blocks, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---- prefill (T new tokens per sequence, causal) ------------------------- */

/* Workspace bytes for mla_prefill with this batch and q_len; max_context is
 * the largest start_pos + q_len the call will see (values below q_len count
 * as q_len).  Scratch only: no initial contents required. */
mla_status mla_prefill_workspace_size(const mla_config* cfg, int32_t batch, int32_t q_len,
                                      int32_t max_context, size_t* bytes /* host out */);

/* The attention form mla_prefill takes for q_len new tokens after
 * max_start_pos cached ones under this config (prefill_attention, or with 0
 * the one needing fewer FLOPs): *form = 1 on the latent rows (absorbed), 2
 * through per-head keys and values.  Host only. */
mla_status mla_prefill_attention_form(const mla_config* cfg, int32_t q_len, int32_t max_start_pos,
                                      int32_t* form /* host out */);

/* Forward of q_len new tokens per sequence through one MLA layer, absorbed
 * path ("GatedMLA" docs, "Build per-head Q, K and V" and "Observe logits,
 * then compute causal attention"; modeldna "MLA" module, "Under the hood"):
 * token t of sequence b sits at position p = start_pos[b] + t; its cache row
 * is appended (as mla_cache_append, slot from the page table); its queries
 * are q = x W_Q, or q = RMSNorm(x W_DQ) * q_norm_w W_UQ when q_lora_rank > 0,
 * split per head into [nope (Dn) | rope (Dr)] with the rope part rotated at
 * p; it attends causally to the stored rows 0..p of its sequence.
 *   x [batch, q_len, M];
 *   w_q [M, H(Dn+Dr)] when q_lora_rank == 0 (else NULL);
 *   w_dq [M, Rq], q_norm_w float32 [Rq], w_uq [Rq, H(Dn+Dr)] when q_lora_rank > 0;
 *   w_dkv [M, R + Dr]; kv_norm_w float32 [R]; w_uk [H, Dn, R]; w_uv [H, R, Dv];
 *   rope_table as for mla_cache_append, rope_table_len > max_start_pos + q_len - 1;
 *   kv_pool, block_table [batch, max_blocks_per_seq]: pages covering
 *     positions 0 .. start_pos[b] + q_len - 1 of each sequence;
 *   start_pos int32 [batch] (device, trusted, each <= max_start_pos);
 *   max_start_pos (host); (max_start_pos + q_len) <= max_blocks_per_seq * block_size;
 *   out [batch, q_len, H, Dv] (written); workspace as sized by
 *   mla_prefill_workspace_size with max_context = max_start_pos + q_len.
 * Attention takes one of two equivalent forms (same result up to rounding):
 * on the latent rows (q_full = [q_nope W_UK | q_rope], P V on c, then W_UV),
 * or through per-head keys and values rebuilt for the context (K_h =
 * [c W_UK[h]^T | k_rope], V_h = c W_UV[h], "GatedMLA" docs, "Build per-head
 * Q, K and V").  bf16 with R = 512, Dr = 64, Dn = Dv = 128 takes the second
 * when it needs fewer FLOPs: 2H(Dn + Dr + Dv) per (query, key) pair plus
 * 2H R (Dn + Dv) per context token, against 2H(2R + Dr) per pair (long new
 * spans; continuations of a few tokens stay on the latent rows).  Over an
 * FP8 cache the second form is always taken: the new rows are stored in FP8
 * first, and every key and value, the new tokens' own included, comes from
 * the stored rows. */
mla_status mla_prefill(const mla_config* cfg, const void* x, const void* w_q, const void* w_dq,
                       const float* q_norm_w, const void* w_uq, const void* w_dkv,
                       const float* kv_norm_w, const void* w_uk, const void* w_uv,
                       const float* rope_table, int32_t rope_table_len, void* kv_pool,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* start_pos, int32_t max_start_pos, int32_t batch,
                       int32_t q_len, void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---- after the heads: optional output gate, then W_O ---------------------- */

/* Workspace bytes for mla_output_gate_projection with n_rows rows (the gated
 * head outputs, n_rows x H x Dv values of the storage dtype; 0 is enough
 * without a gate).  Scratch only. */
mla_status mla_output_gate_workspace_size(const mla_config* cfg, int32_t n_rows,
                                          size_t* bytes /* host out */);

/* The layer's attention contribution from its head outputs ("GatedMLA" docs,
 * "Output projection and optional gate"): the heads' outputs, one row of
 * H x Dv values per token, are multiplied elementwise by sigmoid(x W_G) when
 * a gate is given (the gate reads the layer input x, not the attention
 * result), then projected by W_O back to the model width.  No residual.
 *   x [n_rows, M] (M = d_model > 0); head_out [n_rows, H, Dv] (as written by
 *   mla_decode / mla_prefill); w_g [M, H Dv] or NULL (no gate);
 *   w_o [H Dv, M]; out [n_rows, M] (written).
 * bf16 needs M and H Dv multiples of 8.  The gated values are rounded to the
 * storage dtype before W_O (they are staged in the workspace). */
mla_status mla_output_gate_projection(const mla_config* cfg, const void* x, const void* head_out,
                                      const void* w_g, const void* w_o, int32_t n_rows, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- measurement probes (not part of the method) ------------------------
 * The ceilings this library's kernels are measured against, taken on the
 * device at hand: the caller times each launch on `stream`.
 * mla_probe_sink_bytes: bytes of device memory `sink` must hold.
 * mla_probe_hbm_read: reads bytes (>= 36864) of buf (device, 16-byte
 *   aligned) once and writes one value per thread to sink.  mode 0: 16-byte
 *   vector loads by 8 workgroups of 512 threads per compute unit; mode 1:
 *   whole 36864-byte pieces (bytes rounded down) through direct-to-LDS loads
 *   into four rotating LDS buffers by one 512-thread workgroup per compute
 *   unit, the way the decode attention moves its tiles.
 * mla_probe_mfma: workgroups x 4 waves each run iterations x 4 independent
 *   32x32x16 bf16 MFMAs on register operands (32768 FLOP each; workgroups of
 *   256 threads); one value per thread to sink.
 * mla_probe_lds_read: one workgroup of 8 waves per compute unit; every wave
 *   runs iterations x 8 bank-conflict-free LDS reads of width (16 or 8)
 *   bytes per lane, i.e. CUs x 8 x iterations x 8 x 64 x width bytes in all;
 *   one value per thread to sink.
 * Errors: MLA_ERR_INVALID_ARG for NULL or misaligned pointers, a too small
 * buffer, an unknown mode or width or non-positive counts; MLA_ERR_HIP if
 * the launch fails.  Nothing is allocated. */
size_t mla_probe_sink_bytes(void);
mla_status mla_probe_hbm_read(const void* buf, size_t bytes, int32_t mode, void* sink,
                              void* stream);
mla_status mla_probe_mfma(int32_t workgroups, int32_t iterations, void* sink, void* stream);
mla_status mla_probe_lds_read(int32_t width, int32_t iterations, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LATENT_KV_H */
