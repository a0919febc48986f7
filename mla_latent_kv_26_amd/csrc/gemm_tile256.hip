// Large bf16 GEMM on MFMA (gfx950): C[z] = alpha * A[z] * B[z] (or A Bt^T),
// float32 accumulate, bf16 or float32 output.  For the prefill projections,
// the per-head key/value reconstruction and the output projections (M in the
// thousands, N >= 128, K a multiple of 32).
//
// Tile 256 x BN x 32 (BN = 256 or 128) per 256-thread workgroup: 4 waves as
// 2 (M) x 2 (N), one per SIMD, each wave 128 x BN/2 with 32x32x16 MFMAs
// (the accumulators, 128 or 256 registers, live in AGPRs).  Operand tiles
// move HBM/L2 -> LDS with direct-to-LDS loads into four stages.
//
// One wave per SIMD means nothing hides a stall of the MFMA pipe but the
// wave's own instruction order, so each half step (16 of the stage's 32 k,
// 16 or 8 MFMAs per wave) carries, between its MFMAs, the LDS fragment
// reads of the next half step and, after the stage barrier, the
// direct-to-LDS loads of the stage four ahead.  The reads sit in MFMA slots
// 4..9 (they end several MFMAs before the wait for them, and the first
// MFMAs of a half step never queue behind them), the loads in slots from a
// quarter of the way on.  Measured on MI355X at 8192 x 8192 x 7168: 0.37
// of the bf16 peak with each half step's reads issued as one block ahead
// of its MFMAs (8 waves, two per SIMD), 0.49 interleaved like this.
//
// Stage lifetime: stage s is read during iteration s - 1 (its first half
// step) and iteration s (its second); the barrier after the second read has
// completed in every wave frees its buffer, which then receives stage s + 4.
// So all four buffers hold loads in flight or landed data at once.
//
// LDS layouts (16-byte chunks, chosen by which global chunk each lane
// loads, so the direct-to-LDS write pattern stays linear):
//   A stage  [256 m][32 k]: chunk c of row m at c ^ ((m >> 2) & 3); the 16
//            rows of a 16-lane fragment read then hit 16 distinct bank slots.
//   B stage  [32 k][BN n] (B row-major): chunk c of row k at c ^ 4 (k & 3);
//            the 4 rows x 64 bytes of a transposing read fall on 4 distinct
//            quarters of a bank window.
//   Bt stage [BN n][32 k] (B given transposed): as A.
// Fragment reads are issued from inline assembly and completed by a
// separate wait that names their registers: reads the compiler issues
// itself make it wait for every direct-to-LDS load in flight first.
// The accumulators hold C transposed (the MFMA takes the B fragment as its
// first operand): a lane owns one row of C and runs of 4 columns, so the
// epilogue writes 16-byte (float32) or 8-byte (bf16) vectors.
//
// Workgroup -> tile: blocks go round-robin over the 8 XCDs; XCD x owns a
// contiguous group of row tiles (of all batch entries together) and walks
// all column tiles with the row tile fastest, so the workgroups resident on
// one XCD share their B column tiles in its L2 and each A row tile stays in
// L2 while the columns pass.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kTM = 256, kTK = 32, kTStages = 4, kTThreads = 256;
constexpr int kTABytes = kTM * kTK * 2;  // 16 KB

template <int BN>
struct TileCfg {
  static constexpr int WN = BN / 2;                    // columns per wave
  static constexpr int FN = WN / 32;                   // 32-column blocks per wave
  static constexpr int B_BYTES = BN * kTK * 2;
  static constexpr int STAGE = kTABytes + B_BYTES;
  static constexpr int A_LOADS = kTM * kTK / 8 / kTThreads;  // 16-byte loads per thread
  static constexpr int B_LOADS = BN * kTK / 8 / kTThreads;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int T = 4 * FN;                     // MFMAs per wave per half step
  // MFMA slots of a half step that carry the fragment reads: RO .. RO + RS - 1
  static constexpr int RO = T >= 16 ? 4 : 2, RS = 6;
  static_assert(kTStages * STAGE <= 160 * 1024, "LDS budget");
  static_assert(RO + RS <= T, "read slots inside the half step");
};

// waits until at most `pending` later stages of this thread's loads are in flight
template <int N>
__device__ __forceinline__ void wait_stages(int pending) {
  static_assert(kTStages <= 4 && 3 * N < 64, "vmcnt range");
  if (pending >= 3)
    wait_vmcnt<3 * N>();
  else if (pending == 2)
    wait_vmcnt<2 * N>();
  else if (pending == 1)
    wait_vmcnt<N>();
  else
    wait_vmcnt<0>();
}

// Fragment reads (ds_*_nowait) are valid after settle() below.
// r selects the 32-row block (2048 bytes apart); a constant after unrolling
__device__ __forceinline__ void read_blk(bf16x8& o, uint32_t a, int r) {
  switch (r) {
    case 0: ds_b128_nowait<0>(o, a); break;
    case 1: ds_b128_nowait<2048>(o, a); break;
    case 2: ds_b128_nowait<4096>(o, a); break;
    default: ds_b128_nowait<6144>(o, a); break;
  }
}
// sh = 2 s + h2: k moves by 16 s + 4 h2 rows of RB bytes
template <int RB>
__device__ __forceinline__ void read_tr(bf16x4& o, uint32_t a, int sh) {
  switch (sh) {
    case 0: ds_tr_nowait<0>(o, a); break;
    case 1: ds_tr_nowait<4 * RB>(o, a); break;
    case 2: ds_tr_nowait<16 * RB>(o, a); break;
    default: ds_tr_nowait<20 * RB>(o, a); break;
  }
}

// One half step's fragments: A blocks, and B blocks either as plain rows
// (transposed B) or as two transposing halves (row-major B).
template <int FN, bool BT>
struct Frag {
  bf16x8 a[4];
  bf16x8 b[FN];
  bf16x4 t[FN][2];
};

// Waits for this wave's LDS reads and hands their registers on as written
// here, so no use of them is scheduled before the wait.
template <int FN, bool BT>
__device__ __forceinline__ void settle(Frag<FN, BT>& f) {
  if constexpr (BT && FN == 4)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),
                   "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
  else if constexpr (BT)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),
                   "+v"(f.b[1]));
  else if constexpr (FN == 4)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.t[0][0]),
                   "+v"(f.t[0][1]), "+v"(f.t[1][0]), "+v"(f.t[1][1]), "+v"(f.t[2][0]),
                   "+v"(f.t[2][1]), "+v"(f.t[3][0]), "+v"(f.t[3][1]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.t[0][0]),
                   "+v"(f.t[0][1]), "+v"(f.t[1][0]), "+v"(f.t[1][1]));
}

// This thread's direct-to-LDS sources for one tile (the global chunk for
// each of its LDS slots) and B's row stride.
template <int BN, bool kBT>
struct TileSrc {
  const bf16* a[TileCfg<BN>::A_LOADS];
  const bf16* b[TileCfg<BN>::B_LOADS];
  long ldb;
};

// Sources of tile (m0, n0).  Row-major B may come as column blocks of nb
// (block j at B + j * sBn); nb = N for one plain matrix.
template <int BN, bool kBT>
__device__ __forceinline__ void tile_sources(TileSrc<BN, kBT>& t, const bf16* A, int M, long lda,
                                             int m0, const bf16* B, int N, long ldb, int n0,
                                             int nb, long sBn, int wave, int lane) {
  using Cf = TileCfg<BN>;
#pragma unroll
  for (int i = 0; i < Cf::A_LOADS; ++i) {
    const int p = (wave * Cf::A_LOADS + i) * 64 + lane;  // LDS chunk slot
    const int m = p >> 2, c = (p & 3) ^ ((m >> 2) & 3);
    t.a[i] = A + (long)min(m0 + m, M - 1) * lda + 8 * c;
  }
#pragma unroll
  for (int i = 0; i < Cf::B_LOADS; ++i) {
    const int p = (wave * Cf::B_LOADS + i) * 64 + lane;
    if constexpr (kBT) {
      const int n = p >> 2, c = (p & 3) ^ ((n >> 2) & 3);
      t.b[i] = B + (long)min(n0 + n, N - 1) * ldb + 8 * c;
    } else {
      constexpr int CPR = BN / 8;  // chunks per k row
      const int k = p / CPR, c = (p % CPR) ^ (4 * (k & 3));
      const int n = min(n0 + 8 * c, N - 8);  // column blocks of nb (a chunk never straddles one)
      t.b[i] = B + (long)(n / nb) * sBn + (long)k * ldb + n % nb;
    }
  }
  t.ldb = ldb;
}

// acc += the product over k stages [kt0, kt1) of the tile whose sources are
// `src` (kt1 > kt0).  The LDS buffers are free on entry and on return.
template <int BN, bool kBT>
__device__ __forceinline__ void tile_mainloop(uint32_t lds, const TileSrc<BN, kBT>& src, int kt0,
                                              int kt1, f32x16 (&acc)[4][TileCfg<BN>::FN]) {
  using Cf = TileCfg<BN>;
  constexpr int FN = Cf::FN, T = Cf::T, L = Cf::LOADS;
  constexpr int NR = kBT ? 4 + FN : 4 + 2 * FN;  // fragment reads per half step
  constexpr int RB = BN * 2;                     // bytes per k row of a row-major B stage
  constexpr int kDOff = T / 4;                   // first MFMA slot carrying loads
  constexpr int kROff = Cf::RO, kRSpan = Cf::RS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // load q (0 .. L-1) of stage kt
  auto issue_one = [&](int kt, int q) {
    const uint32_t st = lds + (uint32_t)(kt % kTStages) * Cf::STAGE;
    if (q < Cf::A_LOADS) {
      g2lds16(src.a[q] + (long)kt * kTK, st + (uint32_t)(wave * Cf::A_LOADS + q) * 1024u);
    } else {
      const int i = q - Cf::A_LOADS;
      const long off = kBT ? (long)kt * kTK : (long)kt * kTK * src.ldb;
      g2lds16(src.b[i] + off, st + kTABytes + (uint32_t)(wave * Cf::B_LOADS + i) * 1024u);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  // A fragment (block i, k step s): row 128 wm + 32 i + l32, chunk (2 s + hi)
  // swizzled; blocks are 2048 bytes apart (the swizzle sees row bits 2..3 only)
  uint32_t a_off[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int m = 128 * wm + l32;
    a_off[s] = (uint32_t)(m * 64 + (((2 * s + hi) ^ ((m >> 2) & 3)) * 16));
  }
  // B fragment offsets.  Transposed B: as A, per k step.  Row-major B: one
  // address per 32-column block jb (in a 16-lane group g, lane 4a + b reads
  // row k0 + a, columns c0 + 4b .. +3); the k step s and the half h2 move k
  // by 16 s + 4 h2, which keeps k & 3 and so the swizzle.
  uint32_t b_off[kBT ? 2 : FN];
  {
    const int g = lane >> 4, li = lane & 15;
    if constexpr (kBT) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int n = Cf::WN * wn + l32;
        b_off[s] = (uint32_t)(kTABytes + n * 64 + (((2 * s + hi) ^ ((n >> 2) & 3)) * 16));
      }
    } else {
#pragma unroll
      for (int jb = 0; jb < FN; ++jb) {
        const int k = 8 * (g >> 1) + (li >> 2);
        const int col = Cf::WN * wn + 32 * jb + 16 * (g & 1) + 4 * (li & 3);
        b_off[jb] = (uint32_t)(kTABytes + k * RB + (((col >> 3) ^ (4 * (k & 3))) * 16) +
                               ((col >> 2) & 1) * 8);
      }
    }
  }

  // read r (0 .. NR-1) of half step s of the stage at LDS address st
  auto read_one = [&](uint32_t st, int s, int r, Frag<FN, kBT>& f) {
    if (r < 4) {
      read_blk(f.a[r], st + a_off[s], r);
    } else if constexpr (kBT) {
      read_blk(f.b[r - 4], st + b_off[s], r - 4);
    } else {
      const int jb = (r - 4) >> 1, h2 = (r - 4) & 1;
      read_tr<RB>(f.t[jb][h2], st + b_off[jb], 2 * s + h2);
    }
  };
  auto mfma_one = [&](const Frag<FN, kBT>& f, int e) {
    const int i = e / FN, jb = e % FN;
    if constexpr (kBT)
      acc[i][jb] = mfma32(f.b[jb], f.a[i], acc[i][jb]);
    else
      acc[i][jb] = mfma32(cat(f.t[jb][0], f.t[jb][1]), f.a[i], acc[i][jb]);
  };

  Frag<FN, kBT> f0, f1;
  // Iteration kt: half step (kt, 0) on f0 while f1 = (kt, 1) is read; the
  // barrier that publishes stage kt + 1 (and frees stage kt's buffer); half
  // step (kt, 1) on f1 while f0 = (kt + 1, 0) is read and stage kt + 4 is
  // loaded into kt's buffer.
  auto body = [&](int kt, auto load_c, auto next_c) {
    constexpr bool LOAD = decltype(load_c)::value;  // stage kt + 4 exists
    constexpr bool NEXT = decltype(next_c)::value;  // stage kt + 1 exists
    const uint32_t st = lds + (uint32_t)(kt % kTStages) * Cf::STAGE;
#pragma unroll
    for (int e = 0; e < T; ++e) {
      mfma_one(f0, e);
      __builtin_amdgcn_sched_barrier(0);
      if (e >= kROff && e < kROff + kRSpan) {
#pragma unroll
        for (int r = (e - kROff) * NR / kRSpan; r < (e - kROff + 1) * NR / kRSpan; ++r)
          read_one(st, 1, r, f1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    settle(f1);
    if constexpr (NEXT) {
      wait_stages<L>(min(kt1 - 2 - kt, kTStages - 2));
      lds_barrier();
    }
    const uint32_t sn = lds + (uint32_t)((kt + 1) % kTStages) * Cf::STAGE;
#pragma unroll
    for (int e = 0; e < T; ++e) {
      mfma_one(f1, e);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NEXT) {
        if (e >= kROff && e < kROff + kRSpan) {
#pragma unroll
          for (int r = (e - kROff) * NR / kRSpan; r < (e - kROff + 1) * NR / kRSpan; ++r)
            read_one(sn, 0, r, f0);
        }
      }
      if constexpr (LOAD) {
        if (e >= kDOff) {
#pragma unroll
          for (int q = (e - kDOff) * L / (T - kDOff); q < (e - kDOff + 1) * L / (T - kDOff); ++q)
            issue_one(kt + kTStages, q);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) settle(f0);
  };

  for (int kt = kt0; kt < min(kt1, kt0 + kTStages); ++kt)
#pragma unroll
    for (int q = 0; q < L; ++q) issue_one(kt, q);
  wait_stages<L>(min(kt1 - kt0 - 1, kTStages - 1));
  lds_barrier();
  {
    const uint32_t st = lds + (uint32_t)(kt0 % kTStages) * Cf::STAGE;
#pragma unroll
    for (int r = 0; r < NR; ++r) read_one(st, 0, r, f0);
  }
  settle(f0);
  int kt = kt0;
  for (; kt + kTStages < kt1; ++kt) body(kt, std::true_type{}, std::true_type{});
  for (; kt + 1 < kt1; ++kt) body(kt, std::false_type{}, std::true_type{});
  body(kt, std::false_type{}, std::false_type{});
  lds_barrier();  // every wave is done with the buffers
}

// C[m0.., n0..] = alpha * acc (kAdd: += by float32 atomics), optionally gated.
// Register v of acc[i][jb]: column (BN/2) wn + 32 jb + 8 (v/4) + 4 (lane/32)
// + v%4, row 128 wm + 32 i + lane%32.
template <int BN, bool kOutF32, bool kAdd>
__device__ __forceinline__ void tile_epilogue(const f32x16 (&acc)[4][TileCfg<BN>::FN], void* Cv,
                                              int M, int N, long ldc, int m0, int n0,
                                              float alpha, const bf16* gmul) {
  using Cf = TileCfg<BN>;
  static_assert(!kAdd || kOutF32, "accumulating epilogue is float32");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
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
        const long ci = (long)m * ldc + n;
        if constexpr (kAdd) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            unsafeAtomicAdd((float*)Cv + ci + r, alpha * acc[i][jb][4 * q + r]);
        } else if constexpr (kOutF32) {
          const f32x4 v = {alpha * acc[i][jb][4 * q], alpha * acc[i][jb][4 * q + 1],
                           alpha * acc[i][jb][4 * q + 2], alpha * acc[i][jb][4 * q + 3]};
          *(f32x4*)((float*)Cv + ci) = v;
        } else {
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

template <int BN, bool kBT, bool kOutF32>
__global__ void __launch_bounds__(kTThreads, 1) gemm_tile256_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B, void* __restrict__ Cv, int M, int N,
    int K, long lda, long ldb, long ldc, long sA, long sB, long sC, int batch, int m_per,
    float alpha, int nb, long sBn, const bf16* __restrict__ gmul) {
  using Cf = TileCfg<BN>;
  __shared__ __attribute__((aligned(16))) char smem[kTStages * Cf::STAGE];
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
  tile_mainloop<BN, kBT>(lds, src, 0, K / kTK, acc);
  if constexpr (kOutF32)
    tile_epilogue<BN, true, false>(acc, (float*)Cv + z * sC, M, N, ldc, m0, n0, alpha, nullptr);
  else
    tile_epilogue<BN, false, false>(acc, (bf16*)Cv + z * sC, M, N, ldc, m0, n0, alpha,
                                    gmul ? gmul + z * sC : nullptr);
}

// ---------------------------------------------------------------------------
// Two float32 GEMMs that share A as one launch: C1 = alpha A B1 ([M, N1],
// N1 a multiple of 256) and C2 = alpha A B2 ([M, N2]), B row-major.  Their
// column tiles side by side (C1's first) give n_nt tiles per 256-row tile.
// All but the last column are whole tiles, one per workgroup, with the
// row-group-per-XCD mapping above; the last column tile of each row tile is
// split along k into S parts, one per workgroup, whose float32 partial
// tiles a second kernel adds in a fixed order (deterministic).  S is chosen
// so that the split parts of all row tiles take exactly one round of the
// CUs (S = CUs / row tiles), and the launch is used only when the whole
// tiles take a whole number of rounds too: then no round of the CUs is left
// partly idle.  (The prefill's x [W_DQ | W_DKV] at 8192 rows: 32 row tiles,
// 8 whole column tiles = one round of 256 CUs; 32 last-column tiles split
// 8 ways = one more, short round.)  Other shapes take two tile launches.
// ---------------------------------------------------------------------------
struct PairGemm {
  const bf16* A;
  const bf16* B1;
  const bf16* B2;
  float* C1;
  float* C2;
  float* part;  // S x n_mt partial tiles of 256 x 256 floats
  int M, N1, N2, K;
  long lda, ldb1, ldb2, ldc1, ldc2;
  float alpha;
  int n_nt1, n_nt, n_mt, m_per, S, nk;
};

// column tile ct of the pair: its matrix and column offset
struct PairCol {
  const bf16* B;
  float* C;
  long ldb, ldc;
  int N, n0;
};
__device__ __forceinline__ PairCol pair_col(const PairGemm& g, int ct) {
  if (ct < g.n_nt1) return PairCol{g.B1, g.C1, g.ldb1, g.ldc1, g.N1, ct * 256};
  return PairCol{g.B2, g.C2, g.ldb2, g.ldc2, g.N2, (ct - g.n_nt1) * 256};
}

__global__ void __launch_bounds__(kTThreads, 1) gemm_pair_kernel(PairGemm g) {
  using Cf = TileCfg<256>;
  __shared__ __attribute__((aligned(16))) char smem[kTStages * Cf::STAGE];
  const uint32_t lds = lds_addr(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int r_first = x * g.m_per;
  const int n_whole = g.m_per * (g.n_nt - 1);
  int rt, ct, kt0, kt1, s = -1;
  if (j < n_whole) {
    rt = r_first + j % g.m_per;
    ct = j / g.m_per;
    kt0 = 0;
    kt1 = g.nk;
  } else {
    const int jj = j - n_whole;
    s = jj / g.m_per;
    rt = r_first + jj % g.m_per;
    ct = g.n_nt - 1;
    kt0 = s * g.nk / g.S;
    kt1 = (s + 1) * g.nk / g.S;
  }
  const PairCol c = pair_col(g, ct);
  const int m0 = rt * kTM;
  TileSrc<256, false> src;
  tile_sources<256, false>(src, g.A, g.M, g.lda, m0, c.B, c.N, c.ldb, c.n0, c.N, 0, wave, lane);
  f32x16 acc[4][Cf::FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < Cf::FN; ++jb) acc[i][jb] = f32x16{};
  tile_mainloop<256, false>(lds, src, kt0, kt1, acc);
  // a split part writes its whole 256 x 256 partial tile, unscaled
  const bool whole = s < 0;
  float* C = whole ? c.C : g.part + ((long)s * g.n_mt + rt) * kTM * 256;
  tile_epilogue<256, true, false>(acc, C, whole ? g.M : kTM, whole ? c.N : 256,
                                  whole ? c.ldc : 256, whole ? m0 : 0, whole ? c.n0 : 0,
                                  whole ? g.alpha : 1.0f, nullptr);
}

// last column tiles: C = alpha * sum over s of the partial tiles, s in order
__global__ void __launch_bounds__(256) gemm_pair_reduce_kernel(PairGemm g) {
  const PairCol c = pair_col(g, g.n_nt - 1);
  const long per_tile = (long)kTM * 64;  // 16-byte chunks of a 256 x 256 float tile
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_tile * g.n_mt) return;
  const int rt = (int)(i / per_tile);
  const int e = (int)(i % per_tile), r = e >> 6, col = (e & 63) * 4;
  const int m = rt * kTM + r, n = c.n0 + col;
  if (m >= g.M || n >= c.N) return;
  f32x4 sum = f32x4{};
  for (int s = 0; s < g.S; ++s)
    sum += *(const f32x4*)(g.part + ((long)s * g.n_mt + rt) * kTM * 256 + (long)r * 256 + col);
  *(f32x4*)(c.C + (long)m * c.ldc + n) = g.alpha * sum;
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

size_t gemm_pair_scratch_bytes(int M, int N1, int N2, int num_cus) {
  (void)N1;
  (void)N2;
  const int n_mt = (M + kTM - 1) / kTM;
  const int S = num_cus / n_mt;
  return (size_t)S * n_mt * kTM * 256 * sizeof(float);
}

bool launch_gemm_pair_f32(const void* A, int M, int K, long lda, const void* B1, int N1,
                          long ldb1, float* C1, long ldc1, const void* B2, int N2, long ldb2,
                          float* C2, long ldc2, float alpha, int num_cus, void* scratch,
                          size_t scratch_bytes, hipStream_t st) {
  if (M < kTM || K % kTK != 0 || N1 % 256 != 0 || N1 <= 0 || N2 < 8 || N2 % 8 != 0 ||
      lda % 8 != 0 || ldb1 % 8 != 0 || ldb2 % 8 != 0 || ldc1 % 4 != 0 || ldc2 % 4 != 0)
    return false;
  PairGemm g;
  g.A = (const bf16*)A;
  g.B1 = (const bf16*)B1;
  g.B2 = (const bf16*)B2;
  g.C1 = C1;
  g.C2 = C2;
  g.part = (float*)scratch;
  g.M = M;
  g.N1 = N1;
  g.N2 = N2;
  g.K = K;
  g.lda = lda;
  g.ldb1 = ldb1;
  g.ldb2 = ldb2;
  g.ldc1 = ldc1;
  g.ldc2 = ldc2;
  g.alpha = alpha;
  g.n_nt1 = N1 / 256;
  g.n_nt = g.n_nt1 + (N2 + 255) / 256;
  g.n_mt = (M + kTM - 1) / kTM;
  g.m_per = g.n_mt / 8;
  g.nk = K / kTK;
  // the split parts fill the CUs once (8 row groups of m_per row tiles, one
  // per XCD, S parts each), the whole tiles a whole number of times, and
  // every part gets at least two k stages
  if (g.n_mt % 8 != 0 || num_cus % g.n_mt != 0) return false;
  g.S = num_cus / g.n_mt;
  const long whole = (long)g.n_mt * (g.n_nt - 1);
  if (g.S < 2 || g.n_nt < 2 || whole % num_cus != 0 || g.nk < 2 * g.S ||
      scratch_bytes < gemm_pair_scratch_bytes(M, N1, N2, num_cus))
    return false;
  gemm_pair_kernel<<<8 * g.m_per * (g.n_nt - 1 + g.S), kTThreads, 0, st>>>(g);
  const long chunks = (long)g.n_mt * kTM * 64;
  gemm_pair_reduce_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>(g);
  return true;
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
