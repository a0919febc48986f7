// Internal launch interface between the host dispatch and the kernels.
// Not part of the public ABI (see include/mla.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// ---- generic kernels (any dtype where templated; float32 VALU otherwise) ----

// C[b] = alpha * A[b] (M x K, row stride lda) * B[b] (K x N, row stride ldb),
// float32 everywhere.  Batch strides in elements.
void launch_gemm_f32(const float* A, const float* B, float* C, int M, int N, int K, long lda,
                     long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                     hipStream_t st);

// out[n, k] = in[n, k] / sqrt(mean_k(in[n, :]^2) + eps) * gain[k]; in float32.
// dtype selects out's type (0 f32, 1 bf16).
void launch_rms_norm_rows(const float* in, long ld_in, const float* gain, void* out, long ld_out,
                          int n, int K, float eps, int dtype, hipStream_t st);

// Cache rows from z = x W_DKV (float32 [n, R + Dr], row stride ld_z):
// pool[slot[t]] = [RMSNorm(z[t, :R]) * gain | RoPE(z[t, R:], pos[t])].
// Tokens with slot < 0 are skipped.  dtype: 0 f32, 1 bf16 pool, 2 FP8 rows
// (R E4M3 codes | Dr bf16 | float32 power-of-two scale | 12 zero bytes).
void launch_append_rows(const float* z, long ld_z, const float* gain, const float* rope,
                        const int* pos, const int* slot, void* pool, int n, int R, int Dr,
                        float eps, int dtype, hipStream_t st);

// Same, but positions and slots derived from a page table: token t of
// sequence b (n = b * T + t) sits at start_pos[b] + t.
void launch_append_rows_paged(const float* z, long ld_z, const float* gain, const float* rope,
                              const int* start_pos, const int* block_table, int max_blocks,
                              int block_size, void* pool, int batch, int T, int R, int Dr,
                              float eps, int dtype, hipStream_t st);

// q_full[n, h, R + i] = alpha * RoPE(q[n, h, Dn + :], pos)[i]   (i < Dr),
// q of dtype `dtype` with row stride ld_q (per token) and head stride
// Dn + Dr; q_full row stride H * (R + Dr).  pos = start_pos[n / T] + n % T
// when start_pos != NULL, else no rotation (decode: q_rope already rotated,
// then q points at q_rope with Dn = 0 and head stride Dr).
void launch_q_rope(const void* q, long ld_q, int head_stride, int rope_off, const float* rope,
                   const int* start_pos, int T, void* q_full, int n, int H, int R, int Dr,
                   float alpha, int dtype, hipStream_t st);

// float32 latent attention, one workgroup per (query row, head):
// o_lat[n, h] = softmax over keys 0..len-1 of 2^(q_full[n,h] . row_j) applied to c_j.
// len = seq_lens[n] (decode) or start_pos[n / T] + n % T + 1 (prefill,
// seq_lens == NULL); sequence = n (decode) or n / T.
void launch_attention_f32(const float* q_full, const float* pool, const int* block_table,
                          int max_blocks, int block_size, const int* seq_lens,
                          const int* start_pos, int T, float* o_lat, int n, int H, int R, int Dr,
                          hipStream_t st);

// g[i] = h[i] * sigmoid(g[i]) for i < n (float32 output gate).
void launch_gate_mul_f32(float* g, const float* h, long n, hipStream_t st);

// ---- bf16 MFMA kernels (gfx950) ----

// C[b] = alpha * A[b] * B[b]; A, B bf16 row-major; C bf16 (c_f32 == 0) or
// float32.  Requires K % 8 == 0, N % 8 == 0, lda/ldb % 8 == 0, 16-B aligned
// bases and batch strides.  When side_src is set (bf16 C only), also
// C_b[r, c] = alpha * side_src[b * side_sb + r * side_ld + c] into
// side_dst (same ldc / sC as C) for c < side_cols.
// 256 x (256|128) x 32 tiles, direct-to-LDS staging (gemm_tile256.hip): taken
// by launch_gemm_bf16(_bt) when the shape fits (M >= 256, N >= 128, K a
// multiple of 32, rows and leading dimensions in whole 16-byte chunks).
bool gemm_tile256_fits(int M, int N, int K, long lda, long ldb, long ldc);
// nb > 0 (row-major B only): B's columns come in blocks of nb, block j at
// B + j * sBn, i.e. element (k, n) at B[(n / nb) * sBn + k * ldb + n % nb]
// (nb a multiple of 8); nb <= 0 means one plain [K, N] matrix.
void launch_gemm_tile256(const void* A, const void* B, void* C, int M, int N, int K, long lda,
                         long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                         int c_f32, bool b_transposed, hipStream_t st, int nb = 0, long sBn = 0,
                         const void* gmul = nullptr);
// Cache append fused into the down-projection (append_gemm.hip), bf16 with
// R = 512, Dr = 64: rows of z = x W_DKV ([n, K] x [K, 576]) are normalised
// (RMSNorm on the latent with gain, eps), the rope key rotated by the table
// row of its position, and stored to the pool in bf16 or as FP8 rows,
// without z leaving the CU.  append_gemm: token t has position pos[t] and
// slot slot[t] (negative: skipped).  project_append: token t = b T + i of a
// prefill sits at start_pos[b] + i through the page table; when w_q is set,
// the same launch also computes c = x w_q (float32 [n, N], row stride ldc,
// w_q [K, N] row-major, ldb; n >= 256, N >= 128 and a multiple of 8).
bool append_gemm_fits(int R, int Dr, int K, long ldx);
void launch_append_gemm(const void* x, long ldx, int n, int K, const void* w_dkv,
                        const float* gain, const float* rope, const int* pos, const int* slot,
                        void* pool, bool fp8, float eps, hipStream_t st);
void launch_project_append(const void* x, long ldx, int batch, int T, int K, const void* w_dkv,
                           const float* gain, const float* rope, const int* start_pos,
                           const int* block_table, int max_blocks, int block_size, void* pool,
                           bool fp8, float eps, const void* w_q, int N, long ldb, float* c,
                           long ldc, hipStream_t st);
// Gated GEMM (bf16 out, batch 1): C = gmul * sigmoid(alpha A B), gmul [M, N]
// laid out as C (row stride ldc).
void launch_gemm_bf16_gated(const void* A, const void* B, void* C, int M, int N, int K, long lda,
                            long ldb, long ldc, float alpha, const void* gmul, hipStream_t st);

// As launch_gemm_bf16 with B given transposed: Bt[b] is [N, K] row-major
// (row stride ldb), C[b] = alpha * A[b] * Bt[b]^T.
void launch_gemm_bf16_bt(const void* A, const void* Bt, void* C, int M, int N, int K, long lda,
                         long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                         int c_f32, hipStream_t st);
void launch_gemm_bf16(const void* A, const void* B, void* C, int M, int N, int K, long lda,
                      long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                      int c_f32, hipStream_t st, const void* side_src = nullptr,
                      long side_ld = 0, long side_sb = 0, void* side_dst = nullptr,
                      int side_cols = 0);

// Query absorption for the bf16 decode: q_full[b, h] = alpha [q_nope[b, h]
// W_UK[h] | q_rope[b, h]] (absorb_bf16.hip).  Returns false, having launched
// nothing, unless Dn = 128, R = 512 and Dr = 64.
bool launch_absorb_query_bf16(const void* q_nope, const void* q_rope, const void* w_uk,
                              void* q_full, int B, int H, int Dn, int R, int Dr, float alpha,
                              hipStream_t st);

// Decode attention over a paged bf16 pool (or, with fp8, FP8 cache rows of
// 656 bytes), R = 512, Dr = 64, 32 or 64 heads per workgroup, block_size a
// power of two >= 64.  Writes split partials
// (bf16 O normalised by its own sum, float32 (m, l) in log2 units) and the
// tile prefix sums, for launch_combine.
size_t decode_partial_slots(int batch, int n_wg);
int decode_heads_per_wg(int H, int batch, int max_seq_len, int num_cus);
int decode_num_wg(int head_groups, int num_cus);

void launch_attention_partials_bf16(const void* q_full, const void* pool, int num_blocks,
                                    const int* block_table, int max_blocks, int block_shift,
                                    const int* seq_lens,
                                    int batch, int max_seq_len, int H, int heads_per_wg, int n_wg,
                                    int* prefix, float* part_ml, void* part_o, hipStream_t st,
                                    bool fp8 = false);

// Merge the partials of each (sequence, head) into o_lat (bf16 [batch, H, R])
// or, when w_uv != NULL, project directly: out[b, h] = o_lat[b, h] W_UV[h].
// max_seq_len only steers which partials are fetched before the prefix sums
// arrive (right when all sequences have that length; any value is correct).
// num_cus sets how many sequences share a workgroup (combine_rows_per_wg).
int combine_rows_per_wg(int H, int batch, int num_cus);
void launch_combine(const int* prefix, const float* part_ml, const void* part_o, int batch, int H,
                    int heads_per_wg, int n_wg, int max_seq_len, const void* w_uv, int Dv,
                    void* out, int num_cus, hipStream_t st);

// Decode attention for narrower latents (attention_generic.hip): R = 128 or
// 256, Dr = 64, H a multiple of 16, any block size.  q_full [batch, H, R +
// Dr] bf16 (scaled by softmax_scale * log2 e), pool bf16 rows; chunk /
// n_split from generic_split; part_ml float [batch, n_split, H, 2] and
// part_o float [batch, n_split, H, R] scratch; o_lat [batch, H, R] in bf16 or
// float32.
bool attention_generic_fits(int H, int R, int Dr);
void generic_split(int batch, int H, int max_seq_len, int num_cus, int* chunk, int* n_split);
void launch_attention_generic(const void* q_full, const void* pool, const int* block_table,
                              int max_blocks, int block_size, const int* seq_lens, int batch,
                              int H, int R, int chunk, int n_split, float* part_ml, float* part_o,
                              void* o_lat, bool o_f32, hipStream_t st);

// Decode through per-head keys and values rebuilt for the step, for Dn = Dv
// = Dr = 64 (kernels_generic.hip, attention_generic.hip).  Sequence b' =
// g B + b of the grouped attention is (kv group g, sequence b).
// gather: cg [B, lpad, R] = the latent part of each sequence's rows 0 ..
// len-1 (zero after), rows[g][b lpad + t][128 .. 191] = its rope key; also
// seq2[b'] = len(b), tab2[b'] = b'.  query: q2 [G B, 16, 128] = alpha
// [q_nope | q_rope] of the group's gs heads (zero rows after gs).  out:
// out[b, g gs + i] = o2[g B + b, i] (i < gs), 64 values.  attention: as
// launch_attention_generic over rows [G B lpad, 192] of one row_block-row
// page per sequence b', 16 heads, outputs o [G B, 16, 64] bf16.
void launch_perhead_gather(const void* pool, const int* block_table, int max_blocks,
                           int block_size, const int* seq_lens, int batch, int G, int R, int lpad,
                           void* cg, void* rows, int* seq2, int* tab2, hipStream_t st);
void launch_perhead_query(const void* q_nope, const void* q_rope, int batch, int H, int G,
                          float alpha, void* q2, hipStream_t st);
void launch_perhead_out(const void* o2, int batch, int H, int G, void* out, hipStream_t st);
void launch_attention_perhead(const void* q, const void* rows, const int* table, int row_block,
                              const int* seq_lens, int batch, int chunk, int n_split,
                              float* part_ml, float* part_o, void* o, hipStream_t st);

// Per-head projections of a few rows (rows <= 32, Dn, R, Dv <= 1024)
// with W_UK / W_UV shared by gs consecutive heads: q_full [n, H, R + Dr] =
// alpha [q_nope W_UK[h / gs] | q_rope]; out [n, H, Dv] = o_lat W_UV[h / gs].
bool small_projection_fits(int rows, int Dn, int R, int Dv);
void launch_absorb_small(const void* q_nope, const void* q_rope, const void* w_uk, int n, int H,
                         int gs, int Dn, int R, int Dr, float alpha, int dtype, void* q_full,
                         hipStream_t st);
void launch_project_small(const void* o_lat, const void* w_uv, int n, int H, int gs, int R, int Dv,
                          int dtype, void* out, hipStream_t st);

// Prefill attention: query row n = b * T + t at position start_pos[b] + t
// attends to its sequence's rows 0..position; writes o_lat bf16 [n, H, R].
// Prefill through per-head keys and values (bf16, R = 512, Dn = Dv = 128,
// Dr = 64).  gather: dst [batch, ctx_pad, R + Dr] = each sequence's cache
// rows 0 .. start_pos[b] + T - 1, zero after (fp8: from 656-byte FP8 rows,
// widened to bf16).  flash: out [batch, T, H, Dv] =
// causal softmax(Q K^T) V with Q = alpha [q_nope | RoPE(q_pe, position)] from
// q [batch * T, H (Dn + Dr)], K = [kn | rope part of cg] (kn, v: [batch,
// ctx_pad, H, 128]).
void launch_gather_rows(const void* pool, const int* block_table, int max_blocks, int shift,
                        const int* start_pos, int batch, int T, int ctx_pad, void* dst,
                        bool fp8, hipStream_t st);
void launch_flash_prefill(const void* q, const float* rope, float alpha, const void* kn,
                          const void* cg, const void* v, const int* start_pos, int batch, int T,
                          int H, int ctx_pad, void* out, hipStream_t st);

void launch_attention_prefill_bf16(const void* q_full, const void* pool, const int* block_table,
                                   int max_blocks, int block_shift, const int* start_pos, int T,
                                   int batch, int H, void* o_lat, hipStream_t st);

}  // namespace mla
