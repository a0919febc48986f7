// Large bf16 GEMM on MFMA (gfx950): C[z] = alpha * A[z] * B[z] (or A Bt^T),
// float32 accumulate, bf16 or float32 output, in 256 x (256|128) tiles; the
// main loop, LDS layouts and epilogue are in tile_gemm.h.
//
// Two shapes of launch: one workgroup per CU with 256 x 256 (or 256 x 128)
// tiles and four stages, and for short K (at most kShortK) two workgroups
// per CU with 256 x 128 tiles and three stages (72 KB of LDS and at most
// 256 registers per lane each), so one workgroup's pipeline fill and
// stores run beside the other's MFMAs.  Measured on MI355X: the per-head
// key and value products of the prefill (M 4096 per sequence, N 8192,
// K 512) 124 -> 117 us; at K = 1536 (c_q W_UQ) the short-K shape is slower.
#include "launch.h"
#include "tile_gemm.h"

namespace mla {
namespace {

template <int BN, bool kBT, bool kOutF32, int NS, int OCC>
__global__ void __launch_bounds__(kTThreads, OCC) gemm_tile256_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B, void* __restrict__ Cv, int M, int N,
    int K, long lda, long ldb, long ldc, long sA, long sB, long sC, int batch, int m_per,
    float alpha, int nb, long sBn, const bf16* __restrict__ gmul) {
  using Cf = TileCfg<BN>;
  static_assert(OCC * NS * Cf::STAGE <= 160 * 1024, "LDS of the resident workgroups");
  __shared__ __attribute__((aligned(16))) char smem[NS * Cf::STAGE];
  const uint32_t lds = lds_addr(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // tile of this block
  const int n_mt = (M + kTM - 1) / kTM, n_nt = (N + BN - 1) / BN;
  const int rows_total = n_mt * batch;
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int r_first = x * m_per;
  if (r_first >= rows_total) return;
  const int rows_here = min(m_per, rows_total - r_first);
  if (j >= rows_here * n_nt) return;
  const int row_tile = r_first + j % rows_here, nt = j / rows_here;
  const int z = row_tile / n_mt, m0 = (row_tile % n_mt) * kTM, n0 = nt * BN;

  TileSrc<BN, kBT> src;
  tile_sources<BN, kBT>(src, A + z * sA, M, lda, m0, B + z * sB, N, ldb, n0, nb, sBn, wave,
                        lane);
  f32x16 acc[4][Cf::FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < Cf::FN; ++jb) acc[i][jb] = f32x16{};
  tile_mainloop<BN, kBT, NS>(lds, src, 0, K / kTK, acc);
  if constexpr (kOutF32)
    tile_epilogue<BN, true, false>(acc, (float*)Cv + z * sC, M, N, ldc, m0, n0, alpha, nullptr);
  else
    tile_epilogue<BN, false, false>(acc, (bf16*)Cv + z * sC, M, N, ldc, m0, n0, alpha,
                                    gmul ? gmul + z * sC : nullptr);
}

template <int BN, bool kBT, int NS = kTStages, int OCC = 1>
void launch_tile(const void* A, const void* B, void* C, int M, int N, int K, long lda, long ldb,
                 long ldc, long sA, long sB, long sC, int batch, float alpha, int c_f32, int nb,
                 long sBn, const void* gmul, hipStream_t st) {
  const int n_mt = (M + kTM - 1) / kTM, n_nt = (N + BN - 1) / BN;
  const int rows_total = n_mt * batch;
  const int m_per = (rows_total + 7) / 8;
  const int grid = 8 * m_per * n_nt;
  if (c_f32)
    gemm_tile256_kernel<BN, kBT, true, NS, OCC><<<grid, kTThreads, 0, st>>>(
        (const bf16*)A, (const bf16*)B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, m_per, alpha,
        nb, sBn, (const bf16*)gmul);
  else
    gemm_tile256_kernel<BN, kBT, false, NS, OCC><<<grid, kTThreads, 0, st>>>(
        (const bf16*)A, (const bf16*)B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, m_per, alpha,
        nb, sBn, (const bf16*)gmul);
}

}  // namespace

constexpr int kShortK = 512;  // longest K that takes the two-workgroup launch

bool gemm_tile256_fits(int M, int N, int K, long lda, long ldb, long ldc) {
  // 16-byte aligned rows and chunks, whole 32-wide k steps, vector stores of 4
  return M >= kTM && N >= 128 && K >= kTK && K % kTK == 0 && N % 8 == 0 && lda % 8 == 0 &&
         ldb % 8 == 0 && ldc % 4 == 0;
}

void launch_gemm_tile256(const void* A, const void* B, void* C, int M, int N, int K, long lda,
                         long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                         int c_f32, bool b_transposed, hipStream_t st, int nb, long sBn,
                         const void* gmul) {
  if (M <= 0 || N <= 0 || batch <= 0) return;
  if (nb <= 0) {
    nb = N;
    sBn = 0;
  }
  const bool wide = N >= 256;
  if (K <= kShortK) {
    if (b_transposed)
      launch_tile<128, true, 3, 2>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha,
                                   c_f32, nb, sBn, gmul, st);
    else
      launch_tile<128, false, 3, 2>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha,
                                    c_f32, nb, sBn, gmul, st);
    return;
  }
  if (b_transposed) {
    if (wide)
      launch_tile<256, true>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, nb,
                             sBn, gmul, st);
    else
      launch_tile<128, true>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, nb,
                             sBn, gmul, st);
  } else {
    if (wide)
      launch_tile<256, false>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, nb,
                              sBn, gmul, st);
    else
      launch_tile<128, false>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, nb,
                              sBn, gmul, st);
  }
}

}  // namespace mla
