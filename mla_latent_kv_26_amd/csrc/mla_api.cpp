// Host side of the C ABI: validation, workspace layout and kernel dispatch.
// Every check runs before anything is enqueued; see include/mla.h.
#include "mla.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_err;

mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

struct Dims {
  int H, R, Dr, Dn, Dv, M, Rq, bs, dt, W, shift;
  float scale, eps, theta;
  size_t esz;
  bool fp8;          // FP8 cache rows
  size_t row_bytes;  // bytes per cache row
  int G, gs;         // W_UK / W_UV matrices, heads per matrix
  int split_wg;      // requested decode workgroups per head group (0: one per CU)
  int prefill_form;  // 0 fewer FLOPs, 1 latent rows, 2 per-head keys and values
  int decode_form;   // 0, 1 latent rows, 2 per-head keys and values rebuilt per step
};

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

mla_status check_cfg(const mla_config* c, Dims* d) {
  if (!c) return fail(MLA_ERR_INVALID_ARG, "config pointer is NULL");
  if (c->num_heads <= 0 || c->kv_lora_rank <= 0 || c->rope_dim <= 0 || c->qk_nope_dim <= 0 ||
      c->v_dim <= 0)
    return fail(MLA_ERR_INVALID_ARG,
                "num_heads, kv_lora_rank, rope_dim, qk_nope_dim and v_dim must be positive "
                "(got %d, %d, %d, %d, %d)",
                c->num_heads, c->kv_lora_rank, c->rope_dim, c->qk_nope_dim, c->v_dim);
  if (c->rope_dim % 2) return fail(MLA_ERR_INVALID_ARG, "rope_dim must be even (got %d)", c->rope_dim);
  if (c->d_model < 0 || c->q_lora_rank < 0)
    return fail(MLA_ERR_INVALID_ARG, "d_model and q_lora_rank must be >= 0");
  if (c->d_model > 0 && c->kv_lora_rank >= c->d_model)
    return fail(MLA_ERR_INVALID_ARG, "kv_lora_rank (%d) must be smaller than d_model (%d)",
                c->kv_lora_rank, c->d_model);
  if (c->d_model > 0 && c->q_lora_rank >= c->d_model)
    return fail(MLA_ERR_INVALID_ARG, "q_lora_rank (%d) must be smaller than d_model (%d)",
                c->q_lora_rank, c->d_model);
  if (c->block_size <= 0) return fail(MLA_ERR_INVALID_ARG, "block_size must be positive");
  if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(MLA_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta))
    return fail(MLA_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (c->dtype != MLA_DTYPE_F32 && c->dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (c->cache_dtype != MLA_CACHE_SAME && c->cache_dtype != MLA_CACHE_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARG, "unknown cache_dtype %d", c->cache_dtype);
  if (c->cache_dtype == MLA_CACHE_FP8_E4M3 && c->dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARG, "an FP8 cache needs dtype bf16");
  if (c->kv_groups < 0 || (c->kv_groups > 0 && c->num_heads % c->kv_groups))
    return fail(MLA_ERR_INVALID_ARG, "kv_groups (%d) must be 0 or divide num_heads (%d)",
                c->kv_groups, c->num_heads);
  if (c->split_workgroups < 0 || c->split_workgroups > 8192 || c->split_workgroups % 8)
    return fail(MLA_ERR_INVALID_ARG,
                "split_workgroups (%d) must be 0 or a multiple of 8 up to 8192",
                c->split_workgroups);
  if (c->prefill_attention < 0 || c->prefill_attention > 2)
    return fail(MLA_ERR_INVALID_ARG, "prefill_attention (%d) must be 0, 1 or 2",
                c->prefill_attention);
  if (c->decode_attention < 0 || c->decode_attention > 2)
    return fail(MLA_ERR_INVALID_ARG, "decode_attention (%d) must be 0, 1 or 2",
                c->decode_attention);
  if (d) {
    d->H = c->num_heads;
    d->R = c->kv_lora_rank;
    d->Dr = c->rope_dim;
    d->Dn = c->qk_nope_dim;
    d->Dv = c->v_dim;
    d->M = c->d_model;
    d->Rq = c->q_lora_rank;
    d->bs = c->block_size;
    d->dt = c->dtype;
    d->W = d->R + d->Dr;
    d->shift = pow2(d->bs) ? ilog2(d->bs) : -1;
    d->scale = c->softmax_scale > 0.f ? c->softmax_scale
                                      : (float)(1.0 / std::sqrt((double)(d->Dn + d->Dr)));
    d->eps = c->rms_eps;
    d->theta = c->rope_theta;
    d->esz = d->dt == MLA_DTYPE_BF16 ? 2 : 4;
    d->fp8 = c->cache_dtype == MLA_CACHE_FP8_E4M3;
    d->row_bytes = d->fp8 ? (size_t)d->R + 2 * (size_t)d->Dr + 16 : (size_t)d->W * d->esz;
    d->G = c->kv_groups > 0 ? c->kv_groups : d->H;
    d->gs = d->H / d->G;
    d->split_wg = c->split_workgroups;
    d->prefill_form = c->prefill_attention;
    d->decode_form = c->decode_attention;
  }
  return MLA_OK;
}

// Decode through per-head keys and values rebuilt for the step.
bool perhead_decode(const Dims& d) { return d.decode_form == 2; }

// Shape support of the kernels (after the config itself is valid).
mla_status check_decode_kernels(const Dims& d, int batch) {
  if (perhead_decode(d)) {
    if (d.dt != MLA_DTYPE_BF16 || d.fp8 || d.Dn != 64 || d.Dv != 64 || d.Dr != 64 ||
        d.gs > 16 || d.R % 8)
      return fail(MLA_ERR_UNSUPPORTED,
                  "decode_attention 2 (per-head keys and values) needs bf16 rows, qk_nope_dim = "
                  "v_dim = rope_dim = 64, at most 16 heads per kv group and kv_lora_rank %% 8 == 0 "
                  "(got %d, %d, %d, %d heads per group, rank %d)",
                  d.Dn, d.Dv, d.Dr, d.gs, d.R);
    return MLA_OK;
  }
  if (d.dt == MLA_DTYPE_F32) {
    if (d.R > 1024)
      return fail(MLA_ERR_UNSUPPORTED, "float32 path supports kv_lora_rank <= 1024 (got %d)", d.R);
    return MLA_OK;
  }
  if (d.Dn % 8 || d.Dv % 16 || d.Dv > 128)
    return fail(MLA_ERR_UNSUPPORTED,
                "bf16 projections need qk_nope_dim % 8 == 0 and v_dim % 16 == 0, v_dim <= 128");
  if (d.R != 512 && !d.fp8 && mla::attention_generic_fits(d.H, d.R, d.Dr)) return MLA_OK;
  if (d.R != 512 || d.Dr != 64)
    return fail(MLA_ERR_UNSUPPORTED,
                "bf16 attention kernels are built for kv_lora_rank 512 (or 128, 256 with heads in "
                "multiples of 16, bf16 rows) and rope_dim 64 (got %d, %d, %d heads)",
                d.R, d.Dr, d.H);
  if (d.H % 32)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 attention needs num_heads a multiple of 32 (got %d)", d.H);
  if (d.shift < 6)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 attention needs block_size a power of two >= 64 (got %d)",
                d.bs);
  if (batch > 1024)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 decode handles at most 1024 sequences per call (got %d)",
                batch);
  return MLA_OK;
}

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

mla_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MLA_OK;
}

// ---- decode workspace layout ----
struct DecodeWs {
  size_t prefix, part_ml, part_o, q_full, o_lat, total;
  int n_wg, hgc, heads;
  int chunk, n_split;  // narrow-latent kernels
  // per-head form: latent part, rebuilt rows, grouped queries, lengths, table
  size_t cg, rows, q2, seq2, tab2;
  int lpad;
};
// bf16 shapes that go to the narrow-latent kernels instead of the tuned ones
bool generic_decode(const Dims& d) { return d.dt == MLA_DTYPE_BF16 && d.R != 512; }

DecodeWs decode_ws(const Dims& d, int batch, int max_seq_len) {
  DecodeWs w{};
  size_t off = 256;  // reserved
  if (perhead_decode(d)) {
    const size_t nb2 = (size_t)d.G * batch;
    w.lpad = (max_seq_len + 15) / 16 * 16;
    mla::generic_split((int)nb2, 16, max_seq_len, num_cus(), &w.chunk, &w.n_split);
    w.cg = off;
    off = up256(off + (size_t)batch * w.lpad * d.R * 2);
    w.rows = off;
    off = up256(off + nb2 * w.lpad * 192 * 2);
    w.q2 = off;
    off = up256(off + nb2 * 16 * 128 * 2);
    w.seq2 = off;
    off = up256(off + nb2 * 4);
    w.tab2 = off;
    off = up256(off + nb2 * 4);
    w.part_ml = off;
    off = up256(off + nb2 * w.n_split * 16 * 2 * 4);
    w.part_o = off;
    off = up256(off + nb2 * w.n_split * 16 * 64 * 4);
    w.o_lat = off;
    off = up256(off + nb2 * 16 * 64 * 2);
    w.q_full = off;
    w.total = off;
    return w;
  }
  if (generic_decode(d)) {
    mla::generic_split(batch, d.H, max_seq_len, num_cus(), &w.chunk, &w.n_split);
    w.part_ml = off;
    off = up256(off + (size_t)batch * w.n_split * d.H * 2 * 4);
    w.part_o = off;
    off = up256(off + (size_t)batch * w.n_split * d.H * d.R * 4);
    w.o_lat = off;
    off = up256(off + (size_t)batch * d.H * d.R * 2);
  } else if (d.dt == MLA_DTYPE_BF16) {
    const int cus = num_cus();
    w.heads = mla::decode_heads_per_wg(d.H, batch, max_seq_len, cus);
    w.hgc = d.H / w.heads;
    w.n_wg = d.split_wg > 0 ? d.split_wg : mla::decode_num_wg(w.hgc, cus);
    const size_t slots = mla::decode_partial_slots(batch, w.n_wg);
    w.prefix = off;
    off = up256(off + (size_t)(batch + 1) * 4);
    w.part_ml = off;
    off = up256(off + (size_t)w.hgc * slots * w.heads * 2 * 4);
    w.part_o = off;
    off = up256(off + (size_t)w.hgc * slots * w.heads * 512 * 2);
    if (d.gs > 1) {  // o_lat for the grouped W_UV product
      w.o_lat = off;
      off = up256(off + (size_t)batch * d.H * d.R * 2);
    }
  }
  w.q_full = off;
  off = up256(off + (size_t)batch * d.H * d.W * d.esz);
  if (d.dt == MLA_DTYPE_F32) {
    w.o_lat = off;
    off = up256(off + (size_t)batch * d.H * d.R * 4);
  }
  w.total = off;
  return w;
}

// ---- prefill path choice and workspace layout ----
// Per-head keys and values (the naive path) when they cost fewer FLOPs than
// attending on the latent rows: per (query, key) pair 2H(Dn + Dr + Dv)
// against 2H(2R + Dr), plus 2H R (Dn + Dv) per context token to build K and V
// (context = max_start_pos + q_len).  bf16 with the shapes of its kernels.
bool prefill_naive_shapes(const Dims& d) {
  return d.dt == MLA_DTYPE_BF16 && d.R == 512 && d.Dr == 64 && d.Dn == 128 && d.Dv == 128;
}
// An FP8 cache always takes the naive path: its gather widens the stored
// rows to bf16, and everything after it is the bf16 path.
bool prefill_naive(const Dims& d, int q_len, int max_start_pos) {
  if (!prefill_naive_shapes(d) || d.prefill_form == 1) return false;
  if (d.fp8 || d.prefill_form == 2) return true;
  const double T = q_len, S = max_start_pos;
  const double pairs = T * (S + (T + 1) / 2);
  const double latent = (2.0 * d.R + d.Dr) * pairs;
  const double naive = (double)(d.Dn + d.Dr + d.Dv) * pairs + (double)d.R * (d.Dn + d.Dv) * (S + T);
  return naive < latent;
}

struct PrefillWs {
  size_t z, cq32, cq, q, q_full, o_lat, cg, kn, vv, total;
  int ctx_pad;
  bool naive;
};
PrefillWs prefill_ws(const Dims& d, int batch, int q_len, int max_start_pos) {
  const long n = (long)batch * q_len;
  PrefillWs w{};
  w.naive = prefill_naive(d, q_len, max_start_pos);
  w.ctx_pad = (int)(((long)max_start_pos + q_len + 63) / 64 * 64);
  size_t off = 256;
  w.z = off;
  off = up256(off + (size_t)n * d.W * 4);
  if (d.Rq > 0) {
    w.cq32 = off;
    off = up256(off + (size_t)n * d.Rq * 4);
    w.cq = off;
    off = up256(off + (size_t)n * d.Rq * d.esz);
  }
  w.q = off;
  off = up256(off + (size_t)n * d.H * (d.Dn + d.Dr) * d.esz);
  if (!w.naive) {
    w.q_full = off;
    off = up256(off + (size_t)n * d.H * d.W * d.esz);
  }
  if (w.naive) {
    const size_t rows = (size_t)batch * w.ctx_pad;
    w.cg = off;
    off = up256(off + rows * d.W * 2);
    w.kn = off;
    off = up256(off + rows * d.H * d.Dn * 2);
    w.vv = off;
    off = up256(off + rows * d.H * d.Dv * 2);
  } else {
    w.o_lat = off;
    off = up256(off + (size_t)n * d.H * d.R * (d.dt == MLA_DTYPE_BF16 ? 2 : 4));
  }
  w.total = off;
  return w;
}

char* at(void* base, size_t off) { return (char*)base + off; }

// dtype-dispatched GEMM: C = alpha * A B (batched, strided); out_f32 selects
// a float32 C for bf16 inputs (float32 inputs always give float32).
void gemm(const Dims& d, const void* A, const void* B, void* C, int M, int N, int K, long lda,
          long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha, bool out_f32,
          hipStream_t st) {
  if (d.dt == MLA_DTYPE_BF16)
    mla::launch_gemm_bf16(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, out_f32 ? 1 : 0,
                          st);
  else
    mla::launch_gemm_f32((const float*)A, (const float*)B, (float*)C, M, N, K, lda, ldb, ldc, sA, sB,
                         sC, batch, alpha, st);
}

// Stage 1 (shared by decode entry points).
// C[., h, :] = alpha A[., h, :] Wm[h / gs] for every head h: one batched
// GEMM over the heads when each has its own matrix (gs = 1), else one per
// group of heads sharing a matrix (batch stride 0 on Wm).  a_head, w_head,
// c_head: element strides between heads (A, C) and between matrices (Wm).
void head_gemm(const Dims& d, const void* A, long lda, long a_head, const void* Wm, long ldb,
               long w_head, void* C, long ldc, long c_head, int rows, int N, int K, float alpha,
               bool out_f32, hipStream_t st) {
  if (d.gs == 1) {
    gemm(d, A, Wm, C, rows, N, K, lda, ldb, ldc, a_head, w_head, c_head, d.H, alpha, out_f32, st);
    return;
  }
  const size_t ce = out_f32 ? 4 : d.esz;
  for (int g = 0; g < d.G; ++g)
    gemm(d, (const char*)A + (size_t)g * d.gs * a_head * d.esz,
         (const char*)Wm + (size_t)g * w_head * d.esz, (char*)C + (size_t)g * d.gs * c_head * ce,
         rows, N, K, lda, ldb, ldc, a_head, 0, c_head, d.gs, alpha, out_f32, st);
}

// out[., h, :] = o_lat[., h, :] W_UV[h / gs] for `rows` rows
void project_out(const Dims& d, const void* o_lat, const void* w_uv, void* out, int rows,
                 hipStream_t st) {
  if ((d.gs > 1 || generic_decode(d)) && mla::small_projection_fits(rows, d.Dn, d.R, d.Dv)) {
    mla::launch_project_small(o_lat, w_uv, rows, d.H, d.gs, d.R, d.Dv, d.dt, out, st);
    return;
  }
  head_gemm(d, o_lat, (long)d.H * d.R, d.R, w_uv, d.Dv, (long)d.R * d.Dv, out, (long)d.H * d.Dv,
            d.Dv, rows, d.Dv, d.R, 1.0f, false, st);
}

void enqueue_absorb(const Dims& d, const void* q_nope, const void* q_rope, const void* w_uk,
                    int n_rows, void* q_full, hipStream_t st) {
  const float alpha = d.scale * 1.4426950408889634f;
  if ((d.gs > 1 || generic_decode(d)) && mla::small_projection_fits(n_rows, d.Dn, d.R, d.Dv)) {
    mla::launch_absorb_small(q_nope, q_rope, w_uk, n_rows, d.H, d.gs, d.Dn, d.R, d.Dr, alpha, d.dt,
                             q_full, st);
    return;
  }
  if (d.gs > 1) {  // heads sharing W_UK: one GEMM per group, then the scaled q_rope copy
    head_gemm(d, q_nope, (long)d.H * d.Dn, d.Dn, w_uk, d.R, (long)d.Dn * d.R, q_full,
              (long)d.H * d.W, d.W, n_rows, d.R, d.Dn, alpha, false, st);
    mla::launch_q_rope(q_rope, (long)d.H * d.Dr, d.Dr, 0, nullptr, nullptr, 1, q_full, n_rows, d.H,
                       d.R, d.Dr, alpha, d.dt, st);
    return;
  }
  if (d.dt == MLA_DTYPE_BF16) {
    if (mla::launch_absorb_query_bf16(q_nope, q_rope, w_uk, q_full, n_rows, d.H, d.Dn, d.R, d.Dr,
                                      alpha, st))
      return;
    // one launch: q_lat = alpha * q_nope W_UK, plus the scaled copy of q_rope
    mla::launch_gemm_bf16(q_nope, w_uk, q_full, n_rows, d.R, d.Dn, (long)d.H * d.Dn, d.R,
                          (long)d.H * d.W, d.Dn, (long)d.Dn * d.R, d.W, d.H, alpha, 0, st, q_rope,
                          (long)d.H * d.Dr, d.Dr, (char*)q_full + (size_t)d.R * d.esz, d.Dr);
    return;
  }
  gemm(d, q_nope, w_uk, q_full, n_rows, d.R, d.Dn, (long)d.H * d.Dn, d.R, (long)d.H * d.W, d.Dn,
       (long)d.Dn * d.R, d.W, d.H, alpha, false, st);
  mla::launch_q_rope(q_rope, (long)d.H * d.Dr, d.Dr, 0, nullptr, nullptr, 1, q_full, n_rows, d.H,
                     d.R, d.Dr, alpha, d.dt, st);
}

mla_status check_pool(const Dims& d, const void* pool, int num_blocks, const int32_t* table,
                      int max_blocks) {
  if (!pool || !table) return fail(MLA_ERR_INVALID_ARG, "kv_pool and block_table must be non-NULL");
  if (num_blocks <= 0) return fail(MLA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (max_blocks <= 0) return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (d.dt == MLA_DTYPE_BF16 && !al16(pool))
    return fail(MLA_ERR_INVALID_ARG, "kv_pool must be 16-byte aligned");
  return MLA_OK;
}

mla_status check_ptrs16(const Dims& d, std::initializer_list<const void*> ps, const char* names) {
  for (const void* p : ps) {
    if (!p) return fail(MLA_ERR_INVALID_ARG, "NULL pointer among %s", names);
    if (d.dt == MLA_DTYPE_BF16 && !al16(p))
      return fail(MLA_ERR_INVALID_ARG, "%s must be 16-byte aligned", names);
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_err.c_str(); }

mla_status mla_validate_config(const mla_config* cfg) {
  g_err.clear();
  return check_cfg(cfg, nullptr);
}

int64_t mla_cache_row_elems(const mla_config* cfg) {
  Dims d;
  g_err.clear();
  if (check_cfg(cfg, &d) != MLA_OK) return -1;
  return d.W;
}

int64_t mla_cache_bytes_per_token(const mla_config* cfg) {
  Dims d;
  g_err.clear();
  if (check_cfg(cfg, &d) != MLA_OK) return -1;
  return (int64_t)d.row_bytes;
}

mla_status mla_rope_table(const mla_config* cfg, int32_t num_positions, float* host_table) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (num_positions <= 0) return fail(MLA_ERR_INVALID_ARG, "num_positions must be positive");
  if (!host_table) return fail(MLA_ERR_INVALID_ARG, "host_table is NULL");
  const int half = d.Dr / 2;
  for (int p = 0; p < num_positions; ++p) {
    for (int i = 0; i < half; ++i) {
      const double inv_freq = std::pow((double)d.theta, -2.0 * i / (double)d.Dr);
      const double a = (double)p * inv_freq;
      host_table[(size_t)p * d.Dr + i] = (float)std::cos(a);
      host_table[(size_t)p * d.Dr + half + i] = (float)std::sin(a);
    }
  }
  return MLA_OK;
}

// ---------------------------------------------------------------------------
mla_status mla_decode_workspace_size(const mla_config* cfg, int32_t batch, int32_t max_seq_len,
                                     size_t* bytes) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (batch <= 0) return fail(MLA_ERR_INVALID_ARG, "batch must be positive (got %d)", batch);
  if (max_seq_len <= 0) return fail(MLA_ERR_INVALID_ARG, "max_seq_len must be positive");
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  // the layout follows the kernels the call would take: none for a shape
  // they do not cover
  s = check_decode_kernels(d, batch);
  if (s != MLA_OK) return s;
  *bytes = decode_ws(d, batch, max_seq_len).total;
  return MLA_OK;
}

static mla_status check_decode_common(const Dims& d, const void* pool, int32_t num_blocks,
                                      const int32_t* table, int32_t max_blocks,
                                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len) {
  if (batch <= 0) return fail(MLA_ERR_INVALID_ARG, "batch must be positive (got %d)", batch);
  if (max_seq_len <= 0) return fail(MLA_ERR_INVALID_ARG, "max_seq_len must be positive (got %d)", max_seq_len);
  mla_status s = check_pool(d, pool, num_blocks, table, max_blocks);
  if (s != MLA_OK) return s;
  if (!seq_lens) return fail(MLA_ERR_INVALID_ARG, "seq_lens is NULL");
  if ((long)max_seq_len > (long)max_blocks * d.bs)
    return fail(MLA_ERR_INVALID_ARG,
                "max_seq_len %d exceeds the page table capacity %ld (max_blocks_per_seq %d x block_size %d)",
                max_seq_len, (long)max_blocks * d.bs, max_blocks, d.bs);
  // the split-KV partition counts 32-token tiles of the whole batch in 32 bits
  if ((long)batch * ((max_seq_len + 31) / 32) > 0x7fffffffL)
    return fail(MLA_ERR_UNSUPPORTED, "batch x max_seq_len / 32 must stay below 2^31 (got %d x %d)",
                batch, max_seq_len);
  return check_decode_kernels(d, batch);
}

static mla_status enqueue_latent(const Dims& d, const void* q_full, const void* pool,
                                 int32_t num_blocks, const int32_t* table, int32_t max_blocks, const int32_t* seq_lens,
                                 int32_t batch, int32_t max_seq_len, const void* w_uv, void* dst,
                                 void* ws, hipStream_t st) {
  const DecodeWs w = decode_ws(d, batch, max_seq_len);
  // o_lat in the workspace when W_UV follows as its own product
  void* o_lat = dst;
  if (generic_decode(d)) {
    if (w_uv) o_lat = at(ws, w.o_lat);
    mla::launch_attention_generic(q_full, pool, table, max_blocks, d.bs, seq_lens, batch, d.H,
                                  d.R, w.chunk, w.n_split, (float*)at(ws, w.part_ml),
                                  (float*)at(ws, w.part_o), o_lat, false, st);
  } else if (d.dt == MLA_DTYPE_BF16) {
    mla::launch_attention_partials_bf16(q_full, pool, num_blocks, table, max_blocks, d.shift,
                                        seq_lens, batch, max_seq_len, d.H, w.heads, w.n_wg,
                                        (int*)at(ws, w.prefix), (float*)at(ws, w.part_ml),
                                        at(ws, w.part_o), st, d.fp8);
    const bool fuse = w_uv && d.gs == 1;  // the merge applies per-head W_UV itself
    if (w_uv && !fuse) o_lat = at(ws, w.o_lat);
    mla::launch_combine((const int*)at(ws, w.prefix), (const float*)at(ws, w.part_ml),
                        at(ws, w.part_o), batch, d.H, w.heads, w.n_wg, max_seq_len,
                        fuse ? w_uv : nullptr, d.Dv, fuse ? dst : o_lat, num_cus(), st);
    if (fuse) return MLA_OK;
  } else {
    if (w_uv) o_lat = at(ws, w.o_lat);
    mla::launch_attention_f32((const float*)q_full, (const float*)pool, table, max_blocks, d.bs,
                              seq_lens, nullptr, 1, (float*)o_lat, batch, d.H, d.R, d.Dr, st);
  }
  if (w_uv) project_out(d, o_lat, w_uv, dst, batch, st);
  return MLA_OK;
}

// Validation shared by mla_decode and mla_decode_noalloc (everything but
// the workspace); fills *d.
static mla_status check_decode_call(const mla_config* cfg, Dims* d, const void* q_nope,
                                    const void* q_rope, const void* w_uk, const void* w_uv,
                                    const void* kv_pool, int32_t num_blocks,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                    void* out) {
  mla_status s = check_cfg(cfg, d);
  if (s != MLA_OK) return s;
  s = check_decode_common(*d, kv_pool, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                          max_seq_len);
  if (s != MLA_OK) return s;
  return check_ptrs16(*d, {q_nope, q_rope, w_uk, w_uv, out}, "q_nope, q_rope, w_uk, w_uv, out");
}

static void enqueue_decode(const Dims& d, const void* q_nope, const void* q_rope, const void* w_uk,
                           const void* w_uv, const void* kv_pool, int32_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, void* out,
                           void* workspace, hipStream_t st) {
  const DecodeWs w = decode_ws(d, batch, max_seq_len);
  if (perhead_decode(d)) {
    // keys and values of every kv group rebuilt from the latent rows
    // (K_nope = c W_UK[g]^T, V = c W_UV[g], rows [V | K_nope | k_rope]),
    // then grouped attention over them; nothing is applied after
    const int M = batch * w.lpad, G = d.G;
    void* cg = at(workspace, w.cg);
    uint16_t* rows = (uint16_t*)at(workspace, w.rows);
    const long sC = (long)M * 192;
    mla::launch_perhead_gather(kv_pool, block_table, max_blocks_per_seq, d.bs, seq_lens, batch, G,
                               d.R, w.lpad, cg, rows, (int*)at(workspace, w.seq2),
                               (int*)at(workspace, w.tab2), st);
    mla::launch_gemm_bf16_bt(cg, w_uk, rows + 64, M, 64, d.R, d.R, d.R, 192, 0, 64L * d.R, sC, G,
                             1.0f, 0, st);
    mla::launch_gemm_bf16(cg, w_uv, rows, M, 64, d.R, d.R, 64, 192, 0, 64L * d.R, sC, G, 1.0f, 0,
                          st);
    mla::launch_perhead_query(q_nope, q_rope, batch, d.H, G, d.scale * 1.4426950408889634f,
                              at(workspace, w.q2), st);
    mla::launch_attention_perhead(at(workspace, w.q2), rows, (const int*)at(workspace, w.tab2),
                                  w.lpad, (const int*)at(workspace, w.seq2), G * batch, w.chunk,
                                  w.n_split, (float*)at(workspace, w.part_ml),
                                  (float*)at(workspace, w.part_o), at(workspace, w.o_lat), st);
    mla::launch_perhead_out(at(workspace, w.o_lat), batch, d.H, G, out, st);
    return;
  }
  void* q_full = at(workspace, w.q_full);
  enqueue_absorb(d, q_nope, q_rope, w_uk, batch, q_full, st);
  enqueue_latent(d, q_full, kv_pool, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                 max_seq_len, w_uv, out, workspace, st);
}

mla_status mla_decode(const mla_config* cfg, const void* q_nope, const void* q_rope,
                      const void* w_uk, const void* w_uv, const void* kv_pool, int32_t num_blocks,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, void* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_decode_call(cfg, &d, q_nope, q_rope, w_uk, w_uv, kv_pool, num_blocks,
                                   block_table, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                                   out);
  if (s != MLA_OK) return s;
  const DecodeWs w = decode_ws(d, batch, max_seq_len);
  if (!workspace || workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", w.total, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!al16(workspace)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  enqueue_decode(d, q_nope, q_rope, w_uk, w_uv, kv_pool, num_blocks, block_table,
                 max_blocks_per_seq, seq_lens, batch, max_seq_len, out, workspace,
                 (hipStream_t)stream);
  return launched("mla_decode");
}

mla_status mla_absorb_query(const mla_config* cfg, const void* q_nope, const void* q_rope,
                            const void* w_uk, int32_t n_rows, void* q_full, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (n_rows <= 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be positive (got %d)", n_rows);
  s = check_ptrs16(d, {q_nope, q_rope, w_uk, q_full}, "q_nope, q_rope, w_uk, q_full");
  if (s != MLA_OK) return s;
  if (d.dt == MLA_DTYPE_BF16 && (d.Dn % 8 || d.Dr % 8 || d.W % 8))
    return fail(MLA_ERR_UNSUPPORTED,
                "bf16 absorption needs qk_nope_dim, rope_dim and kv_lora_rank + rope_dim multiples of 8");
  enqueue_absorb(d, q_nope, q_rope, w_uk, n_rows, q_full, (hipStream_t)stream);
  return launched("mla_absorb_query");
}

mla_status mla_latent_attention(const mla_config* cfg, const void* q_full, const void* kv_pool,
                                int32_t num_blocks, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, void* o_lat, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (perhead_decode(d))
    return fail(MLA_ERR_UNSUPPORTED,
                "the staged decode calls run on the latent rows; decode_attention 2 applies to "
                "mla_decode only");
  s = check_decode_common(d, kv_pool, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                          max_seq_len);
  if (s != MLA_OK) return s;
  s = check_ptrs16(d, {q_full, o_lat}, "q_full, o_lat");
  if (s != MLA_OK) return s;
  const DecodeWs w = decode_ws(d, batch, max_seq_len);
  if (!workspace || workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", w.total, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!al16(workspace)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  enqueue_latent(d, q_full, kv_pool, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                 nullptr, o_lat, workspace, (hipStream_t)stream);
  return launched("mla_latent_attention");
}

static mla_status check_ws(const DecodeWs& w, void* workspace, size_t workspace_bytes) {
  if (!workspace || workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", w.total, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!al16(workspace)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return MLA_OK;
}

mla_status mla_attention_partials(const mla_config* cfg, const void* q_full, const void* kv_pool,
                                  int32_t num_blocks, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t batch, int32_t max_seq_len, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (perhead_decode(d))
    return fail(MLA_ERR_UNSUPPORTED,
                "the staged decode calls run on the latent rows; decode_attention 2 applies to "
                "mla_decode only");
  if (d.dt != MLA_DTYPE_BF16 || generic_decode(d))
    return fail(MLA_ERR_UNSUPPORTED,
                "split partials exist for the bf16 kernels at kv_lora_rank 512 only; use "
                "mla_latent_attention");
  s = check_decode_common(d, kv_pool, num_blocks, block_table, max_blocks_per_seq, seq_lens, batch,
                          max_seq_len);
  if (s != MLA_OK) return s;
  s = check_ptrs16(d, {q_full}, "q_full");
  if (s != MLA_OK) return s;
  const DecodeWs w = decode_ws(d, batch, max_seq_len);
  s = check_ws(w, workspace, workspace_bytes);
  if (s != MLA_OK) return s;
  mla::launch_attention_partials_bf16(q_full, kv_pool, num_blocks, block_table, max_blocks_per_seq,
                                      d.shift, seq_lens, batch, max_seq_len, d.H, w.heads, w.n_wg,
                                      (int*)at(workspace, w.prefix),
                                      (float*)at(workspace, w.part_ml), at(workspace, w.part_o),
                                      (hipStream_t)stream, d.fp8);
  return launched("mla_attention_partials");
}

mla_status mla_combine_output(const mla_config* cfg, const void* w_uv, int32_t batch,
                              int32_t max_seq_len, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (perhead_decode(d))
    return fail(MLA_ERR_UNSUPPORTED,
                "the staged decode calls run on the latent rows; decode_attention 2 applies to "
                "mla_decode only");
  if (d.dt != MLA_DTYPE_BF16 || generic_decode(d))
    return fail(MLA_ERR_UNSUPPORTED,
                "split partials exist for the bf16 kernels at kv_lora_rank 512 only; use "
                "mla_latent_attention");
  if (w_uv && d.gs > 1)
    return fail(MLA_ERR_UNSUPPORTED,
                "the merge applies W_UV per head only; with kv_groups merge to o_lat and call "
                "mla_output_projection");
  if (batch <= 0) return fail(MLA_ERR_INVALID_ARG, "batch must be positive (got %d)", batch);
  if (max_seq_len <= 0) return fail(MLA_ERR_INVALID_ARG, "max_seq_len must be positive");
  s = check_decode_kernels(d, batch);
  if (s != MLA_OK) return s;
  if (!out || !al16(out)) return fail(MLA_ERR_INVALID_ARG, "out must be non-NULL and 16-byte aligned");
  if (w_uv && !al16(w_uv)) return fail(MLA_ERR_INVALID_ARG, "w_uv must be 16-byte aligned");
  const DecodeWs w = decode_ws(d, batch, max_seq_len);
  s = check_ws(w, workspace, workspace_bytes);
  if (s != MLA_OK) return s;
  mla::launch_combine((const int*)at(workspace, w.prefix), (const float*)at(workspace, w.part_ml),
                      at(workspace, w.part_o), batch, d.H, w.heads, w.n_wg, max_seq_len, w_uv, d.Dv,
                      out, num_cus(), (hipStream_t)stream);
  return launched("mla_combine_output");
}

mla_status mla_output_projection(const mla_config* cfg, const void* o_lat, const void* w_uv,
                                 int32_t n_rows, void* out, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (n_rows <= 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be positive (got %d)", n_rows);
  s = check_ptrs16(d, {o_lat, w_uv, out}, "o_lat, w_uv, out");
  if (s != MLA_OK) return s;
  if (d.dt == MLA_DTYPE_BF16 && (d.R % 8 || d.Dv % 8))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 projection needs kv_lora_rank and v_dim multiples of 8");
project_out(d, o_lat, w_uv, out, n_rows, (hipStream_t)stream);
  return launched("mla_output_projection");
}

// ---------------------------------------------------------------------------
mla_status mla_output_gate_workspace_size(const mla_config* cfg, int32_t n_rows, size_t* bytes) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (n_rows <= 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be positive (got %d)", n_rows);
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = up256((size_t)n_rows * d.H * d.Dv * d.esz);
  return MLA_OK;
}

mla_status mla_output_gate_projection(const mla_config* cfg, const void* x, const void* head_out,
                                      const void* w_g, const void* w_o, int32_t n_rows, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (d.M <= 0) return fail(MLA_ERR_INVALID_ARG, "the output projection needs d_model > 0");
  if (n_rows <= 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be positive (got %d)", n_rows);
  s = check_ptrs16(d, {x, head_out, w_o, out}, "x, head_out, w_o, out");
  if (s != MLA_OK) return s;
  const int HV = d.H * d.Dv;
  if (d.dt == MLA_DTYPE_BF16 && (d.M % 8 || HV % 8))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 output projection needs d_model and H*v_dim multiples of 8");
  hipStream_t st = (hipStream_t)stream;
  const void* src = head_out;
  if (w_g) {
    s = check_ptrs16(d, {w_g}, "w_g");
    if (s != MLA_OK) return s;
    const size_t need = up256((size_t)n_rows * HV * d.esz);
    if (!workspace || workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                  workspace ? "" : ", NULL");
    if (!al16(workspace)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (d.dt == MLA_DTYPE_BF16) {
      mla::launch_gemm_bf16_gated(x, w_g, workspace, n_rows, HV, d.M, d.M, HV, HV, 1.0f, head_out,
                                  st);
    } else {
      mla::launch_gemm_f32((const float*)x, (const float*)w_g, (float*)workspace, n_rows, HV, d.M,
                           d.M, HV, HV, 0, 0, 0, 1, 1.0f, st);
      mla::launch_gate_mul_f32((float*)workspace, (const float*)head_out, (long)n_rows * HV, st);
    }
    src = workspace;
  }
  gemm(d, src, w_o, out, n_rows, d.M, HV, HV, d.M, d.M, 0, 0, 0, 1, 1.0f, false, st);
  return launched("mla_output_gate_projection");
}

// ---------------------------------------------------------------------------
mla_status mla_cache_append_workspace_size(const mla_config* cfg, int32_t n_tokens, size_t* bytes) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (n_tokens <= 0) return fail(MLA_ERR_INVALID_ARG, "n_tokens must be positive");
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  // the fused down-projection keeps z on chip; the other shapes stage it
  const bool fused = d.dt == MLA_DTYPE_BF16 && mla::append_gemm_fits(d.R, d.Dr, d.M, d.M);
  *bytes = fused ? 256 : up256(256 + (size_t)n_tokens * d.W * 4);
  return MLA_OK;
}

mla_status mla_cache_append(const mla_config* cfg, const void* x, const void* w_dkv,
                            const float* kv_norm_w, const float* rope_table, int32_t rope_table_len,
                            const int32_t* positions, const int32_t* slot_mapping, int32_t n_tokens,
                            void* kv_pool, int32_t num_blocks, void* workspace,
                            size_t workspace_bytes, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (d.M <= 0) return fail(MLA_ERR_INVALID_ARG, "cache append needs d_model > 0");
  if (n_tokens <= 0) return fail(MLA_ERR_INVALID_ARG, "n_tokens must be positive (got %d)", n_tokens);
  if (rope_table_len <= 0) return fail(MLA_ERR_INVALID_ARG, "rope_table_len must be positive");
  if (!kv_norm_w || !rope_table || !positions || !slot_mapping)
    return fail(MLA_ERR_INVALID_ARG, "kv_norm_w, rope_table, positions and slot_mapping must be non-NULL");
  if (!kv_pool || num_blocks <= 0) return fail(MLA_ERR_INVALID_ARG, "kv_pool NULL or num_blocks <= 0");
  s = check_ptrs16(d, {x, w_dkv, kv_pool}, "x, w_dkv, kv_pool");
  if (s != MLA_OK) return s;
  if (d.dt == MLA_DTYPE_BF16 && (d.M % 8 || d.W % 8))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 append needs d_model and kv_lora_rank + rope_dim multiples of 8");
  if (d.fp8 && (d.R % 16 || d.Dr % 8))
    return fail(MLA_ERR_UNSUPPORTED, "FP8 cache rows need kv_lora_rank % 16 == 0 and rope_dim % 8 == 0");
  size_t need = 0;
  mla_cache_append_workspace_size(cfg, n_tokens, &need);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (!al16(workspace)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (d.dt == MLA_DTYPE_BF16 && mla::append_gemm_fits(d.R, d.Dr, d.M, d.M)) {
    // down-projection, RMSNorm, RoPE and the store in one launch
    mla::launch_append_gemm(x, d.M, n_tokens, d.M, w_dkv, kv_norm_w, rope_table, positions,
                            slot_mapping, kv_pool, d.fp8, d.eps, st);
    return launched("mla_cache_append");
  }
  float* z = (float*)at(workspace, 256);
  gemm(d, x, w_dkv, z, n_tokens, d.W, d.M, d.M, d.W, d.W, 0, 0, 0, 1, 1.0f, true, st);
  mla::launch_append_rows(z, d.W, kv_norm_w, rope_table, positions, slot_mapping, kv_pool, n_tokens,
                          d.R, d.Dr, d.eps, d.fp8 ? 2 : d.dt, st);
  return launched("mla_cache_append");
}

// ---------------------------------------------------------------------------
mla_status mla_prefill_workspace_size(const mla_config* cfg, int32_t batch, int32_t q_len,
                                      int32_t max_context, size_t* bytes) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (batch <= 0 || q_len <= 0) return fail(MLA_ERR_INVALID_ARG, "batch and q_len must be positive");
  if (max_context < 0) return fail(MLA_ERR_INVALID_ARG, "max_context must be >= 0");
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  const int max_start = max_context > q_len ? max_context - q_len : 0;
  *bytes = prefill_ws(d, batch, q_len, max_start).total;
  return MLA_OK;
}

mla_status mla_prefill_attention_form(const mla_config* cfg, int32_t q_len, int32_t max_start_pos,
                                      int32_t* form) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (q_len <= 0 || max_start_pos < 0)
    return fail(MLA_ERR_INVALID_ARG, "q_len must be positive and max_start_pos >= 0");
  if (!form) return fail(MLA_ERR_INVALID_ARG, "form is NULL");
  *form = prefill_naive(d, q_len, max_start_pos) ? 2 : 1;
  return MLA_OK;
}

mla_status mla_prefill(const mla_config* cfg, const void* x, const void* w_q, const void* w_dq,
                       const float* q_norm_w, const void* w_uq, const void* w_dkv,
                       const float* kv_norm_w, const void* w_uk, const void* w_uv,
                       const float* rope_table, int32_t rope_table_len, void* kv_pool,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* start_pos, int32_t max_start_pos, int32_t batch,
                       int32_t q_len, void* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_cfg(cfg, &d);
  if (s != MLA_OK) return s;
  if (d.M <= 0) return fail(MLA_ERR_INVALID_ARG, "prefill needs d_model > 0");
  if (d.gs > 1)
    return fail(MLA_ERR_UNSUPPORTED, "prefill takes one W_UK and W_UV per head (kv_groups 0)");
  if (d.dt == MLA_DTYPE_BF16 && d.R != 512)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 prefill kernels are built for kv_lora_rank 512");
  if (d.fp8 && !prefill_naive_shapes(d))
    return fail(MLA_ERR_UNSUPPORTED,
                "prefill over an FP8 cache needs bf16 with kv_lora_rank 512, rope_dim 64 and "
                "qk_nope_dim = v_dim = 128");
  if (d.fp8 && d.prefill_form == 1)
    return fail(MLA_ERR_UNSUPPORTED,
                "prefill over an FP8 cache runs through per-head keys and values (prefill_attention "
                "0 or 2)");
  if (d.prefill_form == 2 && !prefill_naive_shapes(d))
    return fail(MLA_ERR_UNSUPPORTED,
                "per-head prefill attention needs bf16 with kv_lora_rank 512, rope_dim 64 and "
                "qk_nope_dim = v_dim = 128");
  if (batch <= 0 || q_len <= 0)
    return fail(MLA_ERR_INVALID_ARG, "batch and q_len must be positive (got %d, %d)", batch, q_len);
  if (max_start_pos < 0) return fail(MLA_ERR_INVALID_ARG, "max_start_pos must be >= 0");
  if (!start_pos || !kv_norm_w || !rope_table)
    return fail(MLA_ERR_INVALID_ARG, "start_pos, kv_norm_w and rope_table must be non-NULL");
  if ((long)rope_table_len < (long)max_start_pos + q_len)
    return fail(MLA_ERR_INVALID_ARG, "rope_table_len %d must exceed the last position %ld",
                rope_table_len, (long)max_start_pos + q_len - 1);
  s = check_pool(d, kv_pool, num_blocks, block_table, max_blocks_per_seq);
  if (s != MLA_OK) return s;
  if ((long)max_start_pos + q_len > (long)max_blocks_per_seq * d.bs)
    return fail(MLA_ERR_INVALID_ARG, "max_start_pos + q_len (%ld) exceeds the page table capacity %ld",
                (long)max_start_pos + q_len, (long)max_blocks_per_seq * d.bs);
  if (d.Rq > 0) {
    s = check_ptrs16(d, {w_dq, w_uq, (const void*)q_norm_w}, "w_dq, w_uq, q_norm_w");
    if (s != MLA_OK) return s;
  } else {
    s = check_ptrs16(d, {w_q}, "w_q");
    if (s != MLA_OK) return s;
  }
  s = check_ptrs16(d, {x, w_dkv, w_uk, w_uv, out}, "x, w_dkv, w_uk, w_uv, out");
  if (s != MLA_OK) return s;
  if (d.dt == MLA_DTYPE_BF16) {
    s = check_decode_kernels(d, 1);
    if (s != MLA_OK) return s;
    if (d.M % 8 || d.Rq % 8)
      return fail(MLA_ERR_UNSUPPORTED, "bf16 prefill needs d_model and q_lora_rank multiples of 8");
  } else if (d.R > 1024) {
    return fail(MLA_ERR_UNSUPPORTED, "float32 path supports kv_lora_rank <= 1024");
  }
  const long n = (long)batch * q_len;
  if (n > (1L << 30)) return fail(MLA_ERR_INVALID_ARG, "batch * q_len too large");
  const PrefillWs w = prefill_ws(d, batch, q_len, max_start_pos);
  if (!workspace || workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", w.total, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!al16(workspace)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  const int QW = d.H * (d.Dn + d.Dr);
  const float alpha = d.scale * 1.4426950408889634f;
  // 1. cache rows: the down-projection with the RMSNorm, RoPE and store in
  //    its epilogue (bf16, R = 512, Dr = 64); with a q rank, x W_DQ goes in
  //    the same launch (both read x, and together they fill the CUs)
  float* cq32 = d.Rq > 0 ? (float*)at(workspace, w.cq32) : nullptr;
  void* cq = d.Rq > 0 ? at(workspace, w.cq) : nullptr;
  bool have_cq = false;
  if (d.dt == MLA_DTYPE_BF16 && mla::append_gemm_fits(d.R, d.Dr, d.M, d.M)) {
    have_cq = d.Rq > 0 && mla::gemm_tile256_fits((int)n, d.Rq, d.M, d.M, d.Rq, d.Rq);
    mla::launch_project_append(x, d.M, batch, q_len, d.M, w_dkv, kv_norm_w, rope_table, start_pos,
                               block_table, max_blocks_per_seq, d.bs, kv_pool, d.fp8, d.eps,
                               have_cq ? w_dq : nullptr, d.Rq, d.Rq, cq32, d.Rq, st);
  } else {
    float* z = (float*)at(workspace, w.z);
    gemm(d, x, w_dkv, z, (int)n, d.W, d.M, d.M, d.W, d.W, 0, 0, 0, 1, 1.0f, true, st);
    mla::launch_append_rows_paged(z, d.W, kv_norm_w, rope_table, start_pos, block_table,
                                  max_blocks_per_seq, d.bs, kv_pool, batch, q_len, d.R, d.Dr, d.eps,
                                  d.fp8 ? 2 : d.dt, st);
  }
  // 2. queries
  void* q = at(workspace, w.q);
  if (d.Rq > 0) {
    if (!have_cq)
      gemm(d, x, w_dq, cq32, (int)n, d.Rq, d.M, d.M, d.Rq, d.Rq, 0, 0, 0, 1, 1.0f, true, st);
    mla::launch_rms_norm_rows(cq32, d.Rq, q_norm_w, cq, d.Rq, (int)n, d.Rq, d.eps, d.dt, st);
    gemm(d, cq, w_uq, q, (int)n, QW, d.Rq, d.Rq, QW, QW, 0, 0, 0, 1, 1.0f, false, st);
  } else {
    gemm(d, x, w_q, q, (int)n, QW, d.M, d.M, QW, QW, 0, 0, 0, 1, 1.0f, false, st);
  }
  if (w.naive) {
    // 3'. per-head keys and values over each sequence's context, then causal
    //     attention straight to the output
    void* cg = at(workspace, w.cg);
    mla::launch_gather_rows(kv_pool, block_table, max_blocks_per_seq, d.shift, start_pos, batch,
                            q_len, w.ctx_pad, cg, d.fp8, st);
    // K_nope[t, h*Dn + d] = c_t . W_UK[h, d, :] (W_UK as one [H*Dn, R] matrix, given
    // transposed) and V[t, h*Dv + e] = c_t . W_UV[h, :, e] (W_UV as column blocks of Dv),
    // every sequence of the batch in one launch each
    const long sa = (long)w.ctx_pad * d.W;
    if (mla::gemm_tile256_fits(w.ctx_pad, d.H * d.Dn, d.R, d.W, d.R, (long)d.H * d.Dn) &&
        mla::gemm_tile256_fits(w.ctx_pad, d.H * d.Dv, d.R, d.W, d.Dv, (long)d.H * d.Dv) &&
        d.Dv % 8 == 0) {
      mla::launch_gemm_bf16_bt(cg, w_uk, at(workspace, w.kn), w.ctx_pad, d.H * d.Dn, d.R, d.W,
                               d.R, (long)d.H * d.Dn, sa, 0, (long)w.ctx_pad * d.H * d.Dn, batch,
                               1.0f, 0, st);
      mla::launch_gemm_tile256(cg, w_uv, at(workspace, w.vv), w.ctx_pad, d.H * d.Dv, d.R, d.W,
                               d.Dv, (long)d.H * d.Dv, sa, 0, (long)w.ctx_pad * d.H * d.Dv, batch,
                               1.0f, 0, false, st, d.Dv, (long)d.R * d.Dv);
    } else {
      for (int b = 0; b < batch; ++b) {
        const long r0 = (long)b * w.ctx_pad;
        const uint16_t* a = (const uint16_t*)cg + r0 * d.W;
        mla::launch_gemm_bf16_bt(a, w_uk, (uint16_t*)at(workspace, w.kn) + r0 * d.H * d.Dn,
                                 w.ctx_pad, d.H * d.Dn, d.R, d.W, d.R, (long)d.H * d.Dn, 0, 0, 0,
                                 1, 1.0f, 0, st);
        mla::launch_gemm_bf16(a, w_uv, (uint16_t*)at(workspace, w.vv) + r0 * d.H * d.Dv,
                              w.ctx_pad, d.Dv, d.R, d.W, d.Dv, (long)d.H * d.Dv, 0,
                              (long)d.R * d.Dv, d.Dv, d.H, 1.0f, 0, st);
      }
    }
    mla::launch_flash_prefill(q, rope_table, alpha, at(workspace, w.kn), cg, at(workspace, w.vv),
                              start_pos, batch, q_len, d.H, w.ctx_pad, out, st);
    return launched("mla_prefill");
  }
  // 3. absorbed query: q_full = alpha * [q_nope W_UK | RoPE(q_pe)]
  void* q_full = at(workspace, w.q_full);
  mla::launch_q_rope(q, QW, d.Dn + d.Dr, d.Dn, rope_table, start_pos, q_len, q_full, (int)n, d.H,
                     d.R, d.Dr, alpha, d.dt, st);
  gemm(d, q, w_uk, q_full, (int)n, d.R, d.Dn, QW, d.R, (long)d.H * d.W, d.Dn + d.Dr,
       (long)d.Dn * d.R, d.W, d.H, alpha, false, st);
  // 4. causal attention on the latent rows
  void* o_lat = at(workspace, w.o_lat);
  if (d.dt == MLA_DTYPE_BF16)
    mla::launch_attention_prefill_bf16(q_full, kv_pool, block_table, max_blocks_per_seq, d.shift,
                                       start_pos, q_len, batch, d.H, o_lat, st);
  else
    mla::launch_attention_f32((const float*)q_full, (const float*)kv_pool, block_table,
                              max_blocks_per_seq, d.bs, nullptr, start_pos, q_len, (float*)o_lat,
                              (int)n, d.H, d.R, d.Dr, st);
  // 5. output up-projection
  gemm(d, o_lat, w_uv, out, (int)n, d.Dv, d.R, (long)d.H * d.R, d.Dv, (long)d.H * d.Dv, d.R,
       (long)d.R * d.Dv, d.Dv, d.H, 1.0f, false, st);
  return launched("mla_prefill");
}

// ---------------------------------------------------------------------------
// Decode for callers that cannot allocate.  The workspace lives in `scratch`,
// one array per GPU in the code object's device memory (held until the
// process ends); host code reaches it only through the address
// hipGetSymbolAddress returns on that device.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// The current device's address of `scratch`, looked up on its first use on
// that device (with the device current) and kept.
mla_status scratch_on_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MLA_ERR_UNSUPPORTED, "device index %d above 63", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_decode_noalloc(const mla_config* cfg, const void* q_nope, const void* q_rope,
                              const void* w_uk, const void* w_uv, const void* kv_pool,
                              int32_t num_blocks, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                              int32_t max_seq_len, void* out, void* stream) {
  Dims d;
  g_err.clear();
  mla_status s = check_decode_call(cfg, &d, q_nope, q_rope, w_uk, w_uv, kv_pool, num_blocks,
                                   block_table, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                                   out);
  if (s != MLA_OK) return s;
  const DecodeWs w = decode_ws(d, batch, max_seq_len);
  if (w.total > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE,
                "this decode needs %zu bytes of scratch; mla_decode_noalloc has %zu (call "
                "mla_decode with a workspace instead)",
                w.total, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  s = scratch_on_device(&ws);
  if (s != MLA_OK) return s;
  enqueue_decode(d, q_nope, q_rope, w_uk, w_uv, kv_pool, num_blocks, block_table,
                 max_blocks_per_seq, seq_lens, batch, max_seq_len, out, ws, (hipStream_t)stream);
  return launched("mla_decode_noalloc");
}

}  // extern "C"
