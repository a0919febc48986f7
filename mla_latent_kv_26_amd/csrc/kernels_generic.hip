// Generic kernels: the float32 VALU path and the dtype-templated epilogues
// (RMSNorm, RoPE, paged row store) used by both dtypes.
#include "device_common.h"
#include "launch.h"

namespace mla {

// ---------------------------------------------------------------------------
// float32 GEMM, 16x16 output tile per 256-thread block, K staged through LDS.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       float* __restrict__ C, int M, int N, int K,
                                                       long lda, long ldb, long ldc, long sA,
                                                       long sB, long sC, float alpha) {
  __shared__ float As[16][17];
  __shared__ float Bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = blockIdx.y * 16 + ty, col = blockIdx.x * 16 + tx;
  A += blockIdx.z * sA;
  B += blockIdx.z * sB;
  C += blockIdx.z * sC;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int ka = k0 + tx, kb = k0 + ty;
    As[ty][tx] = (row < M && ka < K) ? A[(long)row * lda + ka] : 0.f;
    Bs[ty][tx] = (kb < K && col < N) ? B[(long)kb * ldb + col] : 0.f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) acc = fmaf(As[ty][k], Bs[k][tx], acc);
    __syncthreads();
  }
  if (row < M && col < N) C[(long)row * ldc + col] = alpha * acc;
}

void launch_gemm_f32(const float* A, const float* B, float* C, int M, int N, int K, long lda,
                     long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                     hipStream_t st) {
  dim3 grid((N + 15) / 16, (M + 15) / 16, batch);
  gemm_f32_kernel<<<grid, 256, 0, st>>>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, alpha);
}

// g[i] = h[i] * sigmoid(g[i]) (the output gate, float32 storage).
__global__ void __launch_bounds__(256) gate_mul_f32_kernel(float* __restrict__ g,
                                                           const float* __restrict__ h, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) g[i] = h[i] * (1.0f / (1.0f + expf(-g[i])));
}

void launch_gate_mul_f32(float* g, const float* h, long n, hipStream_t st) {
  if (n <= 0) return;
  gate_mul_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(g, h, n);
}

// ---------------------------------------------------------------------------
// Block-wide sum over 256 threads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_sum_256(float v, float* red /* [4] */) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// Block-wide max over 256 threads.
__device__ __forceinline__ float block_max_256(float v, float* red /* [4] */) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return m;
}

// RMSNorm of float32 rows into dtype T.  One block per row.
template <typename T>
__global__ void __launch_bounds__(256) rms_norm_rows_kernel(const float* __restrict__ in, long ld_in,
                                                            const float* __restrict__ gain,
                                                            T* __restrict__ out, long ld_out, int K,
                                                            float eps) {
  __shared__ float red[4];
  const float* x = in + (long)blockIdx.x * ld_in;
  float ss = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) ss = fmaf(x[k], x[k], ss);
  ss = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)K + eps);
  T* y = out + (long)blockIdx.x * ld_out;
  for (int k = threadIdx.x; k < K; k += 256) y[k] = from_f32<T>(x[k] * inv * gain[k]);
}

void launch_rms_norm_rows(const float* in, long ld_in, const float* gain, void* out, long ld_out,
                          int n, int K, float eps, int dtype, hipStream_t st) {
  if (n <= 0) return;
  if (dtype == 1)
    rms_norm_rows_kernel<bf16><<<n, 256, 0, st>>>(in, ld_in, gain, (bf16*)out, ld_out, K, eps);
  else
    rms_norm_rows_kernel<float><<<n, 256, 0, st>>>(in, ld_in, gain, (float*)out, ld_out, K, eps);
}

// ---------------------------------------------------------------------------
// Cache rows: [RMSNorm(z[:R]) * g | RoPE(z[R:], pos)] -> pool slot.  One
// block per token.  The RoPE table row for position p holds cos in its first
// Dr/2 entries and sin in the rest; element i pairs with i + Dr/2.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void store_row(const float* z, const float* gain, const float* rope_row,
                                          T* dst, int R, int Dr, float eps, float* red) {
  float ss = 0.f;
  for (int k = threadIdx.x; k < R; k += 256) ss = fmaf(z[k], z[k], ss);
  ss = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)R + eps);
  for (int k = threadIdx.x; k < R; k += 256) dst[k] = from_f32<T>(z[k] * inv * gain[k]);
  const int half = Dr >> 1;
  for (int i = threadIdx.x; i < half; i += 256) {
    const float c = rope_row[i], s = rope_row[half + i];
    const float a = z[R + i], b = z[R + half + i];
    dst[R + i] = from_f32<T>(a * c - b * s);
    dst[R + half + i] = from_f32<T>(b * c + a * s);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) append_rows_kernel(const float* __restrict__ z, long ld_z,
                                                          const float* __restrict__ gain,
                                                          const float* __restrict__ rope,
                                                          const int* __restrict__ pos,
                                                          const int* __restrict__ slot,
                                                          T* __restrict__ pool, int R, int Dr,
                                                          float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int s = slot[t];
  if (s < 0) return;  // uniform across the block
  store_row<T>(z + (long)t * ld_z, gain, rope + (long)pos[t] * Dr, pool + (long)s * (R + Dr), R,
               Dr, eps, red);
}

template <typename T>
__global__ void __launch_bounds__(256) append_rows_paged_kernel(
    const float* __restrict__ z, long ld_z, const float* __restrict__ gain,
    const float* __restrict__ rope, const int* __restrict__ start_pos,
    const int* __restrict__ block_table, int max_blocks, int block_size, T* __restrict__ pool,
    int T_len, int R, int Dr, float eps) {
  __shared__ float red[4];
  const int n = blockIdx.x;
  const int b = n / T_len, t = n - b * T_len;
  const int p = start_pos[b] + t;
  const long s = (long)block_table[(long)b * max_blocks + p / block_size] * block_size + p % block_size;
  store_row<T>(z + (long)n * ld_z, gain, rope + (long)p * Dr, pool + s * (R + Dr), R, Dr, eps, red);
}

// FP8 cache rows (R + 2 Dr + 16 bytes): the latent c = RMSNorm(z[:R]) g in
// FP8 E4M3 with one power-of-two scale per row, s = 2^e for the smallest e
// with max|c| <= 448 2^e (1 for an all-zero c), code = RNE(c / s); then the
// rotated rope key in bf16, then s as float32 and 12 zero bytes.  The
// exponent comes from frexp (max|c| = m 2^E, m in [0.5, 1): e = E - 9 when
// m <= 0.875, else E - 8), so no rounding enters the choice of s, and c / s
// is exact before the hardware's round-to-nearest-even conversion.
__device__ __forceinline__ void store_row_fp8(const float* z, const float* gain,
                                              const float* rope_row, unsigned char* dst, int R,
                                              int Dr, float eps, float* red) {
  float ss = 0.f;
  for (int k = threadIdx.x; k < R; k += 256) ss = fmaf(z[k], z[k], ss);
  ss = block_sum_256(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)R + eps);
  float amax = 0.f;
  for (int k = threadIdx.x; k < R; k += 256) amax = fmaxf(amax, fabsf(z[k] * inv * gain[k]));
  amax = block_max_256(amax, red);
  float scale = 1.0f;
  if (amax > 0.f) {
    int E;
    const float m = frexpf(amax, &E);
    scale = ldexpf(1.0f, m <= 0.875f ? E - 9 : E - 8);
  }
  typedef short __attribute__((ext_vector_type(2))) short2v;
  for (int k2 = threadIdx.x; 2 * k2 < R; k2 += 256) {
    const float a = z[2 * k2] * inv * gain[2 * k2], b = z[2 * k2 + 1] * inv * gain[2 * k2 + 1];
    const short2v pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2v{0, 0}, a, b, scale, false);
    *(unsigned short*)(dst + 2 * k2) = (unsigned short)pk[0];
  }
  bf16* rope_dst = (bf16*)(dst + R);
  const int half = Dr >> 1;
  for (int i = threadIdx.x; i < half; i += 256) {
    const float c = rope_row[i], s = rope_row[half + i];
    const float a = z[R + i], b = z[R + half + i];
    rope_dst[i] = (bf16)(a * c - b * s);
    rope_dst[half + i] = (bf16)(b * c + a * s);
  }
  if (threadIdx.x < 4) {
    float* tail = (float*)(dst + R + 2 * Dr);
    tail[threadIdx.x] = threadIdx.x == 0 ? scale : 0.f;
  }
}

__global__ void __launch_bounds__(256) append_rows_fp8_kernel(
    const float* __restrict__ z, long ld_z, const float* __restrict__ gain,
    const float* __restrict__ rope, const int* __restrict__ pos, const int* __restrict__ slot,
    unsigned char* __restrict__ pool, int R, int Dr, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int s = slot[t];
  if (s < 0) return;  // uniform across the block
  store_row_fp8(z + (long)t * ld_z, gain, rope + (long)pos[t] * Dr,
                pool + (long)s * (R + 2 * Dr + 16), R, Dr, eps, red);
}

// FP8 rows of a prefill: token t of sequence b goes to position start_pos[b] + t
// through the page table, in the format of store_row_fp8.
__global__ void __launch_bounds__(256) append_rows_paged_fp8_kernel(
    const float* __restrict__ z, long ld_z, const float* __restrict__ gain,
    const float* __restrict__ rope, const int* __restrict__ start_pos,
    const int* __restrict__ block_table, int max_blocks, int block_size,
    unsigned char* __restrict__ pool, int T_len, int R, int Dr, float eps) {
  __shared__ float red[4];
  const int n = blockIdx.x;
  const int b = n / T_len, t = n - b * T_len;
  const int p = start_pos[b] + t;
  const long s = (long)block_table[(long)b * max_blocks + p / block_size] * block_size + p % block_size;
  store_row_fp8(z + (long)n * ld_z, gain, rope + (long)p * Dr, pool + s * (R + 2 * Dr + 16), R, Dr,
                eps, red);
}

void launch_append_rows(const float* z, long ld_z, const float* gain, const float* rope,
                        const int* pos, const int* slot, void* pool, int n, int R, int Dr,
                        float eps, int dtype, hipStream_t st) {
  if (n <= 0) return;
  if (dtype == 2)
    append_rows_fp8_kernel<<<n, 256, 0, st>>>(z, ld_z, gain, rope, pos, slot, (unsigned char*)pool,
                                              R, Dr, eps);
  else if (dtype == 1)
    append_rows_kernel<bf16><<<n, 256, 0, st>>>(z, ld_z, gain, rope, pos, slot, (bf16*)pool, R, Dr, eps);
  else
    append_rows_kernel<float><<<n, 256, 0, st>>>(z, ld_z, gain, rope, pos, slot, (float*)pool, R, Dr, eps);
}

void launch_append_rows_paged(const float* z, long ld_z, const float* gain, const float* rope,
                              const int* start_pos, const int* block_table, int max_blocks,
                              int block_size, void* pool, int batch, int T, int R, int Dr,
                              float eps, int dtype, hipStream_t st) {
  const int n = batch * T;
  if (n <= 0) return;
  if (dtype == 2)
    append_rows_paged_fp8_kernel<<<n, 256, 0, st>>>(z, ld_z, gain, rope, start_pos, block_table,
                                                    max_blocks, block_size, (unsigned char*)pool,
                                                    T, R, Dr, eps);
  else if (dtype == 1)
    append_rows_paged_kernel<bf16><<<n, 256, 0, st>>>(z, ld_z, gain, rope, start_pos, block_table,
                                                      max_blocks, block_size, (bf16*)pool, T, R,
                                                      Dr, eps);
  else
    append_rows_paged_kernel<float><<<n, 256, 0, st>>>(z, ld_z, gain, rope, start_pos,
                                                       block_table, max_blocks, block_size,
                                                       (float*)pool, T, R, Dr, eps);
}

// ---------------------------------------------------------------------------
// Rope part of the query into q_full[n, h, R:R+Dr], scaled by alpha.
// One block per token row; threads over (head, pair).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) q_rope_kernel(const T* __restrict__ q, long ld_q,
                                                     int head_stride, int rope_off,
                                                     const float* __restrict__ rope,
                                                     const int* __restrict__ start_pos, int T_len,
                                                     T* __restrict__ q_full, int H, int R, int Dr,
                                                     float alpha) {
  const int n = blockIdx.x;
  const int half = Dr >> 1;
  const T* src = q + (long)n * ld_q + rope_off;
  T* dst = q_full + (long)n * H * (R + Dr) + R;
  const float* rr = nullptr;
  if (start_pos) {
    const int b = n / T_len;
    rr = rope + (long)(start_pos[b] + (n - b * T_len)) * Dr;
  }
  for (int idx = threadIdx.x; idx < H * half; idx += 256) {
    const int h = idx / half, i = idx - h * half;
    const float a = to_f32(src[(long)h * head_stride + i]);
    const float b = to_f32(src[(long)h * head_stride + half + i]);
    float ya = a, yb = b;
    if (rr) {
      const float c = rr[i], s = rr[half + i];
      ya = a * c - b * s;
      yb = b * c + a * s;
    }
    dst[(long)h * (R + Dr) + i] = from_f32<T>(alpha * ya);
    dst[(long)h * (R + Dr) + half + i] = from_f32<T>(alpha * yb);
  }
}

void launch_q_rope(const void* q, long ld_q, int head_stride, int rope_off, const float* rope,
                   const int* start_pos, int T, void* q_full, int n, int H, int R, int Dr,
                   float alpha, int dtype, hipStream_t st) {
  if (n <= 0) return;
  if (dtype == 1)
    q_rope_kernel<bf16><<<n, 256, 0, st>>>((const bf16*)q, ld_q, head_stride, rope_off, rope,
                                           start_pos, T, (bf16*)q_full, H, R, Dr, alpha);
  else
    q_rope_kernel<float><<<n, 256, 0, st>>>((const float*)q, ld_q, head_stride, rope_off, rope,
                                            start_pos, T, (float*)q_full, H, R, Dr, alpha);
}

// ---------------------------------------------------------------------------
// float32 latent attention: one 64-lane workgroup per (query row, head).
// Scores are already in log2 units (q_full carries scale * log2 e).  Lane r
// owns latent entries r, r + 64, ... (at most kMaxPer of them).
// ---------------------------------------------------------------------------
constexpr int kMaxPer = 16;  // R <= 1024

__global__ void __launch_bounds__(64) attention_f32_kernel(
    const float* __restrict__ q_full, const float* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int block_size,
    const int* __restrict__ seq_lens, const int* __restrict__ start_pos, int T_len,
    float* __restrict__ o_lat, int H, int R, int Dr) {
  const int n = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  int seq, len;
  if (seq_lens) {
    seq = n;
    len = seq_lens[n];
  } else {
    seq = n / T_len;
    len = start_pos[seq] + (n - seq * T_len) + 1;
  }
  const int W = R + Dr;
  const float* q = q_full + ((long)n * H + h) * W;
  const int* table = block_table + (long)seq * max_blocks;
  float m = -INFINITY, l = 0.f;
  float o[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) o[i] = 0.f;
  for (int j = 0; j < len; ++j) {
    const float* row = pool + ((long)table[j / block_size] * block_size + j % block_size) * W;
    float part = 0.f;
    for (int d = lane; d < W; d += 64) part = fmaf(q[d], row[d], part);
    const float s = wave_sum(part);
    const float m_new = fmaxf(m, s);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int r = lane + 64 * i;
      if (r < R) o[i] = o[i] * alpha + p * row[r];
    }
    m = m_new;
  }
  float* dst = o_lat + ((long)n * H + h) * R;
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int r = lane + 64 * i;
    if (r < R) dst[r] = o[i] * inv;
  }
}

void launch_attention_f32(const float* q_full, const float* pool, const int* block_table,
                          int max_blocks, int block_size, const int* seq_lens,
                          const int* start_pos, int T, float* o_lat, int n, int H, int R, int Dr,
                          hipStream_t st) {
  if (n <= 0) return;
  attention_f32_kernel<<<dim3(n, H), 64, 0, st>>>(q_full, pool, block_table, max_blocks,
                                                  block_size, seq_lens, start_pos, T, o_lat, H, R,
                                                  Dr);
}

}  // namespace mla

// ---------------------------------------------------------------------------
// Per-head projections for a few rows (decode of small batches), with G
// matrices shared by H / G consecutive heads: one block per (row, head), the
// head's input vector in LDS, threads over the output columns.  Used where a
// tiled GEMM would run one row tile per launch.
// ---------------------------------------------------------------------------
namespace mla {
namespace {

// q_full[n, h] = alpha [q_nope[n, h] W_UK[h / gs] | q_rope[n, h]]; thread t
// sums part t / R of the Dn inputs for column t % R, the parts are added
// through LDS
template <typename T>
__global__ void __launch_bounds__(1024) absorb_small_kernel(const T* __restrict__ q_nope,
                                                            const T* __restrict__ q_rope,
                                                            const T* __restrict__ w_uk, int H,
                                                            int gs, int Dn, int R, int Dr,
                                                            float alpha, T* __restrict__ q_full) {
  __shared__ float qv[1024];
  __shared__ float part[1024];
  const int n = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const T* q = q_nope + ((long)n * H + h) * Dn;
  for (int d = t; d < Dn; d += 1024) qv[d] = to_f32(q[d]);
  __syncthreads();
  const int parts = 1024 / R, r = t % R, p = t / R;
  const T* w = w_uk + (long)(h / gs) * Dn * R;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (p < parts) {
    const int d0 = (int)((long)Dn * p / parts), d1 = (int)((long)Dn * (p + 1) / parts);
    int d = d0;
#pragma unroll 4
    for (; d + 4 <= d1; d += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = fmaf(qv[d + u], to_f32(w[(long)(d + u) * R + r]), acc[u]);
    for (; d < d1; ++d) acc[0] = fmaf(qv[d], to_f32(w[(long)d * R + r]), acc[0]);
  }
  part[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  T* dst = q_full + ((long)n * H + h) * (R + Dr);
  if (t < R) {
    float s = 0.f;
    for (int k = 0; k < parts; ++k) s += part[k * R + t];
    dst[t] = from_f32<T>(alpha * s);
  }
  const T* qr = q_rope + ((long)n * H + h) * Dr;
  for (int i = t; i < Dr; i += 1024) dst[R + i] = from_f32<T>(alpha * to_f32(qr[i]));
}

// out[n, h] = o_lat[n, h] W_UV[h / gs]; thread t sums part t / Dv of the R
// inputs for column t % Dv, the parts are added through LDS
template <typename T>
__global__ void __launch_bounds__(1024) project_small_kernel(const T* __restrict__ o_lat,
                                                             const T* __restrict__ w_uv, int H,
                                                             int gs, int R, int Dv,
                                                             T* __restrict__ out) {
  __shared__ float ov[1024];
  __shared__ float part[1024];
  const int n = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const T* o = o_lat + ((long)n * H + h) * R;
  for (int r = t; r < R; r += 1024) ov[r] = to_f32(o[r]);
  __syncthreads();
  const int parts = 1024 / Dv, e = t % Dv, p = t / Dv;
  const T* w = w_uv + (long)(h / gs) * R * Dv;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (p < parts) {
    const int r0 = (int)((long)R * p / parts), r1 = (int)((long)R * (p + 1) / parts);
    int r = r0;
#pragma unroll 4
    for (; r + 4 <= r1; r += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = fmaf(ov[r + u], to_f32(w[(long)(r + u) * Dv + e]), acc[u]);
    for (; r < r1; ++r) acc[0] = fmaf(ov[r], to_f32(w[(long)r * Dv + e]), acc[0]);
  }
  part[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (t < Dv) {
    float s = 0.f;
    for (int k = 0; k < parts; ++k) s += part[k * Dv + t];
    out[((long)n * H + h) * Dv + t] = from_f32<T>(s);
  }
}

}  // namespace

bool small_projection_fits(int rows, int Dn, int R, int Dv) {
  return rows <= 32 && Dn <= 1024 && R <= 1024 && Dv <= 1024;
}

void launch_absorb_small(const void* q_nope, const void* q_rope, const void* w_uk, int n, int H,
                         int gs, int Dn, int R, int Dr, float alpha, int dtype, void* q_full,
                         hipStream_t st) {
  const dim3 grid(n, H);
  if (dtype == 1)
    absorb_small_kernel<bf16><<<grid, 1024, 0, st>>>((const bf16*)q_nope, (const bf16*)q_rope,
                                                    (const bf16*)w_uk, H, gs, Dn, R, Dr, alpha,
                                                    (bf16*)q_full);
  else
    absorb_small_kernel<float><<<grid, 1024, 0, st>>>((const float*)q_nope, (const float*)q_rope,
                                                     (const float*)w_uk, H, gs, Dn, R, Dr, alpha,
                                                     (float*)q_full);
}

void launch_project_small(const void* o_lat, const void* w_uv, int n, int H, int gs, int R, int Dv,
                          int dtype, void* out, hipStream_t st) {
  const dim3 grid(n, H);
  if (dtype == 1)
    project_small_kernel<bf16><<<grid, 1024, 0, st>>>((const bf16*)o_lat, (const bf16*)w_uv, H, gs,
                                                     R, Dv, (bf16*)out);
  else
    project_small_kernel<float><<<grid, 1024, 0, st>>>((const float*)o_lat, (const float*)w_uv, H,
                                                      gs, R, Dv, (float*)out);
}

}  // namespace mla

// ---------------------------------------------------------------------------
// Decode through per-head keys and values rebuilt for the step (Dn = Dv = Dr
// = 64): the gather of the latent rows, the grouped queries and the output
// reordering around two batched GEMMs and the narrow attention kernel.
// ---------------------------------------------------------------------------
namespace mla {
namespace {

// One block of 64 threads per (sequence b, position t < lpad): the latent
// part of row t (R values) to cg[b lpad + t], its rope key (64 values) to
// value columns 128 .. 191 of rows[g][b lpad + t] for every group g; zeros
// past the sequence's length.  Block (b, 0) also writes seq2 and tab2.
__global__ void __launch_bounds__(64) perhead_gather_kernel(
    const bf16* __restrict__ pool, const int* __restrict__ block_table, int max_blocks,
    int block_size, const int* __restrict__ seq_lens, int batch, int G, int R, int lpad,
    bf16* __restrict__ cg, bf16* __restrict__ rows, int* __restrict__ seq2,
    int* __restrict__ tab2) {
  const int t = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int len = seq_lens[b];
  if (t == 0)
    for (int g = lane; g < G; g += 64) {
      seq2[g * batch + b] = len;
      tab2[g * batch + b] = g * batch + b;
    }
  const long row = (long)b * lpad + t;
  const int W = R + 64;
  const bf16* src = nullptr;
  if (t < len) {
    const long page = block_table[(long)b * max_blocks + t / block_size];
    src = pool + (page * block_size + t % block_size) * W;
  }
  const uint4 zero = {0u, 0u, 0u, 0u};
  for (int c = lane; c < R / 8; c += 64)
    *(uint4*)(cg + row * R + c * 8) = src ? *(const uint4*)(src + c * 8) : zero;
  for (int e = lane; e < 8 * G; e += 64) {
    const int g = e / 8, c = e % 8;
    *(uint4*)(rows + ((long)g * batch * lpad + row) * 192 + 128 + c * 8) =
        src ? *(const uint4*)(src + R + c * 8) : zero;
  }
}

// q2[g B + b, i] = alpha [q_nope[b, g gs + i] | q_rope[b, g gs + i]] (i <
// gs), zero for gs <= i < 16; one block of 256 threads per (b, g), 8 values
// per thread.
__global__ void __launch_bounds__(256) perhead_query_kernel(
    const bf16* __restrict__ q_nope, const bf16* __restrict__ q_rope, int batch, int H, int G,
    float alpha, bf16* __restrict__ q2) {
  const int b = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int gs = H / G, i = t / 16, c = (t % 16) * 8;
  bf16x8 v;
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (bf16)0.f;
  if (i < gs) {
    const long h = (long)b * H + g * gs + i;
    const bf16x8 s = c < 64 ? *(const bf16x8*)(q_nope + h * 64 + c)
                            : *(const bf16x8*)(q_rope + h * 64 + c - 64);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (bf16)(alpha * (float)s[k]);
  }
  *(bf16x8*)(q2 + (((long)g * batch + b) * 16 + i) * 128 + c) = v;
}

// out[b, g gs + i] = o2[g B + b, i] for i < gs (64 values); one block of 64
// threads per (b, g), 8 values per thread.
__global__ void __launch_bounds__(128) perhead_out_kernel(const bf16* __restrict__ o2, int batch,
                                                          int H, int G, bf16* __restrict__ out) {
  const int b = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int gs = H / G, i = t / 8, c = (t % 8) * 8;
  if (i < gs)
    *(bf16x8*)(out + ((long)b * H + g * gs + i) * 64 + c) =
        *(const bf16x8*)(o2 + (((long)g * batch + b) * 16 + i) * 64 + c);
}

}  // namespace

void launch_perhead_gather(const void* pool, const int* block_table, int max_blocks,
                           int block_size, const int* seq_lens, int batch, int G, int R, int lpad,
                           void* cg, void* rows, int* seq2, int* tab2, hipStream_t st) {
  perhead_gather_kernel<<<dim3(lpad, batch), 64, 0, st>>>(
      (const bf16*)pool, block_table, max_blocks, block_size, seq_lens, batch, G, R, lpad,
      (bf16*)cg, (bf16*)rows, seq2, tab2);
}

void launch_perhead_query(const void* q_nope, const void* q_rope, int batch, int H, int G,
                          float alpha, void* q2, hipStream_t st) {
  perhead_query_kernel<<<dim3(batch, G), 256, 0, st>>>((const bf16*)q_nope, (const bf16*)q_rope,
                                                       batch, H, G, alpha, (bf16*)q2);
}

void launch_perhead_out(const void* o2, int batch, int H, int G, void* out, hipStream_t st) {
  perhead_out_kernel<<<dim3(batch, G), 128, 0, st>>>((const bf16*)o2, batch, H, G, (bf16*)out);
}

}  // namespace mla
