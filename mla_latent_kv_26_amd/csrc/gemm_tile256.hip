// Large bf16 GEMM on MFMA (gfx950): C[z] = alpha * A[z] * B[z] (or A Bt^T),
// float32 accumulate, bf16 or float32 output.  For the prefill projections
// and the per-head key/value reconstruction (M in the thousands, N >= 128,
// K a multiple of 32).
//
// Tile 256 x BN x 32 (BN = 256 or 128) per 512-thread workgroup, 8 waves as
// 2 (M) x 4 (N), each wave 128 x BN/4 with 32x32x16 MFMAs.  Tiles move
// HBM/L2 -> LDS with direct-to-LDS loads into four stages, three in flight
// while one is multiplied; one LDS-only barrier per stage.
//
// LDS layouts (16-byte chunks, chosen by which global chunk each lane
// loads, so the direct-to-LDS write pattern stays linear):
//   A stage  [256 m][32 k]: chunk c of row m at c ^ ((m >> 2) & 3); the 16
//            rows of a 16-lane fragment read then hit 16 distinct bank slots.
//   B stage  [32 k][BN n] (B row-major): chunk c of row k at c ^ 4 (k & 3);
//            the 4 rows x 64 bytes of a transposing read fall on 4 distinct
//            quarters of a bank window.
//   Bt stage [BN n][32 k] (B given transposed): as A.
// The accumulators hold C transposed (the MFMA takes the B fragment as its
// first operand): a lane owns one row of C and runs of 4 columns, so the
// epilogue writes 16-byte (float32) or 8-byte (bf16) vectors.
//
// Workgroup -> tile: blocks go round-robin over the 8 XCDs; XCD x owns a
// contiguous group of row tiles (of all batch entries together) and walks
// all column tiles with the row tile fastest, so the workgroups resident on
// one XCD share their B column tiles in its L2 and each A row tile stays in
// L2 while the columns pass.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kTM = 256, kTK = 32, kTStages = 4;
constexpr int kTWavesN = 4;                    // waves along N (2 along M)
constexpr int kTThreads = 128 * kTWavesN;
constexpr int kTABytes = kTM * kTK * 2;  // 16 KB

template <int BN>
struct TileCfg {
  static constexpr int WN = BN / kTWavesN;             // columns per wave
  static constexpr int FN = WN / 32;                   // 32-column blocks per wave
  static constexpr int B_BYTES = BN * kTK * 2;
  static constexpr int STAGE = kTABytes + B_BYTES;
  static constexpr int A_LOADS = kTM * kTK / 8 / kTThreads;  // 16-byte loads per thread
  static constexpr int B_LOADS = BN * kTK / 8 / kTThreads;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert(kTStages * STAGE <= 160 * 1024, "LDS budget");
};

template <int N>
__device__ __forceinline__ void wait_stages(int pending) {
  static_assert(kTStages <= 5, "up to three later stages in flight");
  if (pending >= 3)
    wait_vmcnt<3 * N>();
  else if (pending == 2)
    wait_vmcnt<2 * N>();
  else if (pending == 1)
    wait_vmcnt<N>();
  else
    wait_vmcnt<0>();
}

// Four transposing LDS reads, finished inside the asm block (see
// lds_read_tr_x8).
__device__ __forceinline__ void lds_read_tr_x4(const uint32_t (&a)[4], bf16x4 (&o)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

template <int BN, bool kBT, bool kOutF32>
__global__ void __launch_bounds__(kTThreads, 1) gemm_tile256_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B, void* __restrict__ Cv, int M, int N,
    int K, long lda, long ldb, long ldc, long sA, long sB, long sC, int batch, int m_per,
    float alpha, int nb, long sBn, const bf16* __restrict__ gmul) {
  using Cf = TileCfg<BN>;
  __shared__ __attribute__((aligned(16))) char smem[kTStages * Cf::STAGE];
  const uint32_t lds = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

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
  A += z * sA;
  B += z * sB;

  // this thread's direct-to-LDS sources (global chunk for each LDS slot)
  const bf16* a_src[Cf::A_LOADS];
#pragma unroll
  for (int i = 0; i < Cf::A_LOADS; ++i) {
    const int p = (wave * Cf::A_LOADS + i) * 64 + lane;  // LDS chunk slot
    const int m = p >> 2, c = (p & 3) ^ ((m >> 2) & 3);
    a_src[i] = A + (long)min(m0 + m, M - 1) * lda + 8 * c;
  }
  const bf16* b_src[Cf::B_LOADS];
#pragma unroll
  for (int i = 0; i < Cf::B_LOADS; ++i) {
    const int p = (wave * Cf::B_LOADS + i) * 64 + lane;
    if constexpr (kBT) {
      const int n = p >> 2, c = (p & 3) ^ ((n >> 2) & 3);
      b_src[i] = B + (long)min(n0 + n, N - 1) * ldb + 8 * c;
    } else {
      constexpr int CPR = BN / 8;  // chunks per k row
      const int k = p / CPR, c = (p % CPR) ^ (4 * (k & 3));
      const int n = min(n0 + 8 * c, N - 8);  // column blocks of nb (a chunk never straddles one)
      b_src[i] = B + (long)(n / nb) * sBn + (long)k * ldb + n % nb;
    }
  }
  auto issue = [&](int kt) {
    const uint32_t st = lds + (uint32_t)(kt % kTStages) * Cf::STAGE;
#pragma unroll
    for (int i = 0; i < Cf::A_LOADS; ++i)
      g2lds16(a_src[i] + (long)kt * kTK, st + (uint32_t)(wave * Cf::A_LOADS + i) * 1024u);
#pragma unroll
    for (int i = 0; i < Cf::B_LOADS; ++i) {
      const long off = kBT ? (long)kt * kTK : (long)kt * kTK * ldb;
      g2lds16(b_src[i] + off, st + kTABytes + (uint32_t)(wave * Cf::B_LOADS + i) * 1024u);
    }
  };

  const int wm = wave / kTWavesN, wn = wave % kTWavesN;
  const int l32 = lane & 31, hi = lane >> 5;
  // A fragment (m-block i, k-step s): row 128 wm + 32 i + l32, chunk 2 s + hi
  uint32_t a_off[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int m = 128 * wm + 32 * i + l32;
      a_off[i][s] = (uint32_t)(m * 64 + (((2 * s + hi) ^ ((m >> 2) & 3)) * 16));
    }
  // B fragment (n-block jb, k-step s): 32 columns at BN/4 wn + 32 jb
  uint32_t b_off[Cf::FN][2][2];  // [jb][s][lo/hi] (transposing reads) or [jb][s][0] (rows)
  {
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int jb = 0; jb < Cf::FN; ++jb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if constexpr (kBT) {
          const int n = Cf::WN * wn + 32 * jb + l32;
          b_off[jb][s][0] = (uint32_t)(n * 64 + (((2 * s + hi) ^ ((n >> 2) & 3)) * 16));
          b_off[jb][s][1] = 0;
        } else {
          constexpr int RB = BN * 2;  // bytes per k row
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int k = 16 * s + 8 * (g >> 1) + (li >> 2) + 4 * h2;
            const int col = Cf::WN * wn + 32 * jb + 16 * (g & 1) + 4 * (li & 3);
            b_off[jb][s][h2] =
                (uint32_t)(k * RB + (((col >> 3) ^ (4 * (k & 3))) * 16) + ((col >> 2) & 1) * 8);
          }
        }
      }
  }

  f32x16 acc[4][Cf::FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < Cf::FN; ++jb) acc[i][jb] = f32x16{};

  const int nk = K / kTK;
  for (int kt = 0; kt < min(nk, kTStages - 1); ++kt) issue(kt);
  if constexpr (kBT) {
    // Both operands are read as rows (plain 16-byte LDS reads), so the
    // fragments of each k-step are read during the previous k-step's MFMAs
    // (two half-stage fragment sets, H0 for k 0..15 and H1 for 16..31 of a
    // stage).  A fragment base is the same for every 32-row block (the row
    // swizzle only looks at bits 2..3), so blocks differ by a constant.
    struct Half {
      bf16x8 a[4];
      bf16x8 b[Cf::FN];
    };
    auto read_half = [&](int kt, int s, Half& h) {
      const uint32_t st = lds + (uint32_t)(kt % kTStages) * Cf::STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) h.a[i] = lds_read_b128(st + a_off[0][s] + 2048u * i);
#pragma unroll
      for (int jb = 0; jb < Cf::FN; ++jb)
        h.b[jb] = lds_read_b128(st + kTABytes + b_off[0][s][0] + 2048u * jb);
    };
    // hand fragments whose reads are known to be done on as plain values
    auto settle = [](Half& h) {
      asm volatile("" : "+v"(h.a[0]), "+v"(h.a[1]), "+v"(h.a[2]), "+v"(h.a[3]));
#pragma unroll
      for (int jb = 0; jb < Cf::FN; ++jb) asm volatile("" : "+v"(h.b[jb]));
    };
    auto mfma_half = [&](const Half& h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jb = 0; jb < Cf::FN; ++jb) acc[i][jb] = mfma32(h.b[jb], h.a[i], acc[i][jb]);
    };
    Half h0, h1;
    wait_stages<Cf::LOADS>(min(nk - 1, kTStages - 2));
    lds_barrier();
    if (kTStages - 1 < nk) issue(kTStages - 1);
    read_half(0, 0, h0);
    for (int kt = 0; kt < nk; ++kt) {
      settle(h0);
      read_half(kt, 1, h1);
      mfma_half(h0);
      if (kt + 1 < nk) {
        wait_stages<Cf::LOADS>(min(nk - 2 - kt, kTStages - 2));
        lds_barrier();  // also retires h1's reads
        settle(h1);
        if (kt + kTStages < nk) issue(kt + kTStages);
        read_half(kt + 1, 0, h0);
      } else {
        settle(h1);
      }
      mfma_half(h1);
    }
  } else
  for (int kt = 0; kt < nk; ++kt) {
    wait_stages<Cf::LOADS>(min(nk - 1 - kt, kTStages - 2));
    lds_barrier();
    if (kt + kTStages - 1 < nk) issue(kt + kTStages - 1);
    const uint32_t st = lds + (uint32_t)(kt % kTStages) * Cf::STAGE;
    // every fragment of the stage in flight at once (the transposing reads
    // end with a wait that also covers the A reads issued before them)
    bf16x8 af[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) af[s][i] = lds_read_b128(st + a_off[i][s]);
    bf16x8 bf[Cf::FN][2];
    if constexpr (Cf::FN % 2 == 0) {
      // reads q = 8 g + r: block 2 g + r / 4, k-step (r / 2) % 2, half r % 2
#pragma unroll
      for (int g8 = 0; g8 < Cf::FN / 2; ++g8) {
        uint32_t ta[8];
        bf16x4 t[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
          ta[r] = st + kTABytes + b_off[2 * g8 + (r >> 2)][(r >> 1) & 1][r & 1];
        lds_read_tr_x8<0>(ta, t);
#pragma unroll
        for (int r = 0; r < 4; ++r) bf[2 * g8 + (r >> 1)][r & 1] = cat(t[2 * r], t[2 * r + 1]);
      }
    } else {
      uint32_t ta[4];
      bf16x4 t[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) ta[q] = st + kTABytes + b_off[0][q >> 1][q & 1];
      lds_read_tr_x4(ta, t);
      bf[0][0] = cat(t[0], t[1]);
      bf[0][1] = cat(t[2], t[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jb = 0; jb < Cf::FN; ++jb) acc[i][jb] = mfma32(bf[jb][s], af[s][i], acc[i][jb]);
  }

  // register v of acc[i][jb]: column (BN/4) wn + 32 jb + 8 (v/4) + 4 (lane/32) + v%4,
  // row 128 wm + 32 i + lane%32
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 128 * wm + 32 * i + l32;
    if (m >= M) continue;
#pragma unroll
    for (int jb = 0; jb < Cf::FN; ++jb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + Cf::WN * wn + 32 * jb + 8 * q + 4 * hi;
        if (n >= N) continue;
        if constexpr (kOutF32) {
          const f32x4 v = {alpha * acc[i][jb][4 * q], alpha * acc[i][jb][4 * q + 1],
                           alpha * acc[i][jb][4 * q + 2], alpha * acc[i][jb][4 * q + 3]};
          *(f32x4*)((float*)Cv + z * sC + (long)m * ldc + n) = v;
        } else {
          const long ci = z * sC + (long)m * ldc + n;
          bf16x4 v;
          if (gmul) {  // gate: C = gmul * sigmoid(alpha A B)
            const bf16x4 gv = *(const bf16x4*)(gmul + ci);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v[r] = (bf16)((float)gv[r] * sigmoid_f(alpha * acc[i][jb][4 * q + r]));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (bf16)(alpha * acc[i][jb][4 * q + r]);
          }
          *(bf16x4*)((bf16*)Cv + ci) = v;
        }
      }
  }
}

template <int BN, bool kBT>
void launch_tile(const void* A, const void* B, void* C, int M, int N, int K, long lda, long ldb,
                 long ldc, long sA, long sB, long sC, int batch, float alpha, int c_f32, int nb,
                 long sBn, const void* gmul, hipStream_t st) {
  const int n_mt = (M + kTM - 1) / kTM, n_nt = (N + BN - 1) / BN;
  const int rows_total = n_mt * batch;
  const int m_per = (rows_total + 7) / 8;
  const int grid = 8 * m_per * n_nt;
  if (c_f32)
    gemm_tile256_kernel<BN, kBT, true><<<grid, kTThreads, 0, st>>>(
        (const bf16*)A, (const bf16*)B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, m_per, alpha,
        nb, sBn, (const bf16*)gmul);
  else
    gemm_tile256_kernel<BN, kBT, false><<<grid, kTThreads, 0, st>>>(
        (const bf16*)A, (const bf16*)B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, m_per, alpha,
        nb, sBn, (const bf16*)gmul);
}

}  // namespace

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
