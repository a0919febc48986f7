// bf16 GEMM on MFMA (gfx950): C[b] = alpha * A[b] * B[b], float32 accumulate.
//
// A is [M, K] row-major (K contiguous) and B is [K, N] row-major (N
// contiguous), the layout of every weight in this library (x W with W
// [in, out]).  The MFMA B operand wants 8 consecutive k per lane, so the B
// tile is kept in LDS in its natural [k][n] layout and read with the gfx950
// transposing LDS load, which hands each lane one column of a 4 x 16 block.
//
// Tile: BM x 128 x BK per 256-thread workgroup, 4 waves, 32x32x16 MFMAs.
// launch_gemm_bf16_bt takes B transposed ([N, K], K contiguous).
// Global loads for the next K-tile are in flight (in registers) while the
// current one is multiplied; BK = 128 covers short contractions in one pass.
//
// Optional side job (used by query absorption): the workgroups of the first
// column tile also copy side_cols values per row, scaled by alpha, from
// side_src (row stride side_ld, batch stride side_sb) to side_dst (row stride
// ldc, batch stride sC), i.e. next to their rows of C (side_cols % 8 == 0,
// 16-byte aligned rows).
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kBN = 128;
// bf16 per B row in LDS: 320 B (64 mod 256), so the 4 rows x 64 bytes that
// 32 lanes of a transposing read touch are 4 disjoint bank ranges
constexpr int kBStride = kBN + 32;

struct Side {
  const bf16* src;
  long ld, sb;
  bf16* dst;
  int cols;
  const bf16* gmul;  // bf16 C only: C = gmul * sigmoid(alpha A B), gmul laid out as C
};

template <int BM, int kBK>
struct Cfg {
  static constexpr int A_STRIDE = kBK + 8;   // bf16 per A row in LDS (conflict-free b128 reads)
  static constexpr int WAVES_M = BM >= 64 ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int FM = BM / (32 * WAVES_M);
  static constexpr int FN = kBN / (32 * WAVES_N);
  static constexpr int A_CHUNKS = BM * kBK / 8;    // 16-byte chunks per A tile
  static constexpr int B_CHUNKS = kBK * kBN / 8;
  static constexpr int A_PER_T = (A_CHUNKS + 255) / 256;
  static constexpr int B_PER_T = B_CHUNKS / 256;
};

// kBT: B is given transposed, [N, K] row-major (K contiguous, row stride
// ldb); its tile is then kept as [n][k] in LDS like A's and read with plain
// 16-byte reads.
template <int BM, int kBK, bool kOutF32, bool kBT>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(const bf16* __restrict__ A,
                                                        const bf16* __restrict__ B,
                                                        void* __restrict__ Cv, int M, int N, int K,
                                                        long lda, long ldb, long ldc, long sA,
                                                        long sB, long sC, float alpha, Side side) {
  using C_ = Cfg<BM, kBK>;
  constexpr int kAStride = C_::A_STRIDE;
  constexpr int kBRows = kBT ? kBN : kBK;
  constexpr int kBCols = kBT ? kBK + 8 : kBStride;
  __shared__ __attribute__((aligned(16))) bf16 As[BM * kAStride];
  __shared__ __attribute__((aligned(16))) bf16 Bs[kBRows * kBCols];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C_::WAVES_N, wn = wave % C_::WAVES_N;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * kBN;
  A += blockIdx.z * sA;
  B += blockIdx.z * sB;

  bf16x8 ra[C_::A_PER_T], rb[C_::B_PER_T];
  const bf16x8 zero8 = {};

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C_::A_PER_T; ++i) {
      const int c = tid + 256 * i;
      const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      const int gr = m0 + r, gk = k0 + kc;
      ra[i] = (c < C_::A_CHUNKS && gr < M && gk < K)
                  ? *(const bf16x8*)(A + (long)gr * lda + gk) : zero8;
    }
#pragma unroll
    for (int i = 0; i < C_::B_PER_T; ++i) {
      const int c = tid + 256 * i;
      if constexpr (kBT) {
        const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
        const int gn = n0 + r, gk = k0 + kc;
        rb[i] = (gn < N && gk < K) ? *(const bf16x8*)(B + (long)gn * ldb + gk) : zero8;
      } else {
        const int r = c / (kBN / 8), nc = (c % (kBN / 8)) * 8;
        const int gk = k0 + r, gn = n0 + nc;
        rb[i] = (gk < K && gn < N) ? *(const bf16x8*)(B + (long)gk * ldb + gn) : zero8;
      }
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < C_::A_PER_T; ++i) {
      const int c = tid + 256 * i;
      if (c < C_::A_CHUNKS) {
        const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
        *(bf16x8*)(As + r * kAStride + kc) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C_::B_PER_T; ++i) {
      const int c = tid + 256 * i;
      if constexpr (kBT) {
        const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
        *(bf16x8*)(Bs + r * kBCols + kc) = rb[i];
      } else {
        const int r = c / (kBN / 8), nc = (c % (kBN / 8)) * 8;
        *(bf16x8*)(Bs + r * kBStride + nc) = rb[i];
      }
    }
  };

  f32x16 acc[C_::FM][C_::FN];
#pragma unroll
  for (int i = 0; i < C_::FM; ++i)
#pragma unroll
    for (int j = 0; j < C_::FN; ++j) acc[i][j] = f32x16{};

  const uint32_t as_base = lds_addr(As), bs_base = lds_addr(Bs);
  // transposed-read coordinates of this lane inside a 32x32x16 B fragment
  const int g = lane >> 4, li = lane & 15;
  const int tr_row = 8 * (g >> 1) + (li >> 2);           // + 16 * ks (+ 4 for the high half)
  const int tr_col = 16 * (g & 1) + 4 * (li & 3);        // + fragment column base

  load_tiles(0);
  if (side.src && blockIdx.x == 0) {
    // side job: scaled copy of side_cols values for each of this tile's rows
    const bf16* ss = side.src + blockIdx.z * side.sb;
    bf16* sd = side.dst + blockIdx.z * sC;
    const int cc = side.cols / 8;  // 16-byte chunks per row
    for (int i = tid; i < BM * cc; i += 256) {
      const int r = i / cc, c = (i % cc) * 8;
      if (m0 + r < M) {
        bf16x8 v = *(const bf16x8*)(ss + (long)(m0 + r) * side.ld + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)(alpha * (float)v[e]);
        *(bf16x8*)(sd + (long)(m0 + r) * ldc + c) = v;
      }
    }
  }
  for (int k0 = 0; k0 < K; k0 += kBK) {
    store_tiles();
    __syncthreads();
    if (k0 + kBK < K) load_tiles(k0 + kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 af[C_::FM], bfr[C_::FN];
#pragma unroll
      for (int i = 0; i < C_::FM; ++i) {
        const int r = (wm * C_::FM + i) * 32 + (lane & 31);
        af[i] = lds_read_b128(as_base + (r * kAStride + 16 * ks + 8 * (lane >> 5)) * 2);
      }
#pragma unroll
      for (int j = 0; j < C_::FN; ++j) {
        if constexpr (kBT) {
          // lane l: column n = l%32 of the fragment, k = 16 ks + 8 (l/32) .. + 7
          const int n = (wn * C_::FN + j) * 32 + (lane & 31);
          bfr[j] = lds_read_b128(bs_base + (n * kBCols + 16 * ks + 8 * (lane >> 5)) * 2);
        } else {
          const int col = (wn * C_::FN + j) * 32 + tr_col;
          const int row = 16 * ks + tr_row;
          const bf16x4 lo = lds_read_tr(bs_base + (row * kBStride + col) * 2);
          const bf16x4 hi = lds_read_tr(bs_base + ((row + 4) * kBStride + col) * 2);
          bfr[j] = cat(lo, hi);
        }
      }
#pragma unroll
      for (int i = 0; i < C_::FM; ++i)
#pragma unroll
        for (int j = 0; j < C_::FN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    __syncthreads();
  }

  // epilogue: register v of lane l is row 8(v/4) + 4(l/32) + v%4, column l%32
#pragma unroll
  for (int i = 0; i < C_::FM; ++i)
#pragma unroll
    for (int j = 0; j < C_::FN; ++j) {
      const int col = n0 + (wn * C_::FN + j) * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + (wm * C_::FM + i) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < M) {
          const long ci = blockIdx.z * sC + (long)row * ldc + col;
          float x = alpha * acc[i][j][v];
          if constexpr (kOutF32) {
            ((float*)Cv)[ci] = x;
          } else {
            if (side.gmul) x = (float)side.gmul[ci] * sigmoid_f(x);
            ((bf16*)Cv)[ci] = (bf16)x;
          }
        }
      }
    }
}

template <int BM, int BK, bool BT>
void launch_bm(const void* A, const void* B, void* C, int M, int N, int K, long lda, long ldb,
               long ldc, long sA, long sB, long sC, int batch, float alpha, int c_f32, Side side,
               hipStream_t st) {
  dim3 grid((N + kBN - 1) / kBN, (M + BM - 1) / BM, batch);
  if (c_f32)
    gemm_bf16_kernel<BM, BK, true, BT><<<grid, 256, 0, st>>>((const bf16*)A, (const bf16*)B, C, M,
                                                             N, K, lda, ldb, ldc, sA, sB, sC, alpha,
                                                             side);
  else
    gemm_bf16_kernel<BM, BK, false, BT><<<grid, 256, 0, st>>>((const bf16*)A, (const bf16*)B, C,
                                                              M, N, K, lda, ldb, ldc, sA, sB, sC,
                                                              alpha, side);
}

template <int BK, bool BT>
void launch_bk(const void* A, const void* B, void* C, int M, int N, int K, long lda, long ldb,
               long ldc, long sA, long sB, long sC, int batch, float alpha, int c_f32, Side side,
               hipStream_t st) {
  if (M <= 32)
    launch_bm<32, BK, BT>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, side,
                          st);
  else if (M <= 64)
    launch_bm<64, BK, BT>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, side,
                          st);
  else
    launch_bm<128, BK, BT>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, side,
                           st);
}

}  // namespace

void launch_gemm_bf16(const void* A, const void* B, void* C, int M, int N, int K, long lda,
                      long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                      int c_f32, hipStream_t st, const void* side_src, long side_ld,
                      long side_sb, void* side_dst, int side_cols) {
  if (M <= 0 || N <= 0 || batch <= 0) return;
  if (!side_src && gemm_tile256_fits(M, N, K, lda, ldb, ldc)) {
    launch_gemm_tile256(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, false, st);
    return;
  }
  const Side side{(const bf16*)side_src, side_ld, side_sb, (bf16*)side_dst, side_cols, nullptr};
  if (K <= 128)
    launch_bk<128, false>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, side,
                          st);
  else
    launch_bk<32, false>(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, side,
                         st);
}

void launch_gemm_bf16_bt(const void* A, const void* Bt, void* C, int M, int N, int K, long lda,
                         long ldb, long ldc, long sA, long sB, long sC, int batch, float alpha,
                         int c_f32, hipStream_t st) {
  if (M <= 0 || N <= 0 || batch <= 0) return;
  if (gemm_tile256_fits(M, N, K, lda, ldb, ldc)) {
    launch_gemm_tile256(A, Bt, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, true, st);
    return;
  }
  const Side side{nullptr, 0, 0, nullptr, 0, nullptr};
  if (K <= 128)
    launch_bk<128, true>(A, Bt, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, side,
                         st);
  else
    launch_bk<32, true>(A, Bt, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, alpha, c_f32, side,
                        st);
}

void launch_gemm_bf16_gated(const void* A, const void* B, void* C, int M, int N, int K, long lda,
                            long ldb, long ldc, float alpha, const void* gmul, hipStream_t st) {
  if (M <= 0 || N <= 0) return;
  if (gemm_tile256_fits(M, N, K, lda, ldb, ldc)) {
    launch_gemm_tile256(A, B, C, M, N, K, lda, ldb, ldc, 0, 0, 0, 1, alpha, 0, false, st, 0, 0,
                        gmul);
    return;
  }
  const Side side{nullptr, 0, 0, nullptr, 0, (const bf16*)gmul};
  if (K <= 128)
    launch_bk<128, false>(A, B, C, M, N, K, lda, ldb, ldc, 0, 0, 0, 1, alpha, 0, side, st);
  else
    launch_bk<32, false>(A, B, C, M, N, K, lda, ldb, ldc, 0, 0, 0, 1, alpha, 0, side, st);
}

}  // namespace mla
