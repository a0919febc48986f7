// The 256-row tile GEMM main loop on MFMA (gfx950), shared by the plain tile
// kernel (gemm_tile256.hip) and the projection + cache append launch
// (append_gemm.hip): C[z] = alpha * A[z] * B[z] (or A Bt^T),
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
#pragma once
#include <type_traits>

#include "device_common.h"

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
// `src` (kt1 > kt0), through NS stage buffers (the loads of stage kt + NS go
// into stage kt's buffer; the description above is for NS = 4).  The LDS
// buffers are free on entry and on return.
template <int BN, bool kBT, int NS = kTStages>
__device__ __forceinline__ void tile_mainloop(uint32_t lds, const TileSrc<BN, kBT>& src, int kt0,
                                              int kt1, f32x16 (&acc)[4][TileCfg<BN>::FN]) {
  static_assert(NS >= 2 && NS <= kTStages, "stage count");
  using Cf = TileCfg<BN>;
  constexpr int FN = Cf::FN, T = Cf::T, L = Cf::LOADS;
  constexpr int NR = kBT ? 4 + FN : 4 + 2 * FN;  // fragment reads per half step
  constexpr int RB = BN * 2;                     // bytes per k row of a row-major B stage
  constexpr int kDOff = T / 4;                   // first MFMA slot carrying loads
  constexpr int kROff = Cf::RO, kRSpan = Cf::RS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // load q (0 .. L-1) of stage kt
  auto issue_one = [&](int kt, int q) {
    const uint32_t st = lds + (uint32_t)(kt % NS) * Cf::STAGE;
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
  // step (kt, 1) on f1 while f0 = (kt + 1, 0) is read and stage kt + NS is
  // loaded into kt's buffer.
  auto body = [&](int kt, auto load_c, auto next_c) {
    constexpr bool LOAD = decltype(load_c)::value;  // stage kt + NS exists
    constexpr bool NEXT = decltype(next_c)::value;  // stage kt + 1 exists
    const uint32_t st = lds + (uint32_t)(kt % NS) * Cf::STAGE;
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
      wait_stages<L>(min(kt1 - 2 - kt, NS - 2));
      lds_barrier();
    }
    const uint32_t sn = lds + (uint32_t)((kt + 1) % NS) * Cf::STAGE;
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
            issue_one(kt + NS, q);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) settle(f0);
  };

  for (int kt = kt0; kt < min(kt1, kt0 + NS); ++kt)
#pragma unroll
    for (int q = 0; q < L; ++q) issue_one(kt, q);
  wait_stages<L>(min(kt1 - kt0 - 1, NS - 1));
  lds_barrier();
  {
    const uint32_t st = lds + (uint32_t)(kt0 % NS) * Cf::STAGE;
#pragma unroll
    for (int r = 0; r < NR; ++r) read_one(st, 0, r, f0);
  }
  settle(f0);
  int kt = kt0;
  for (; kt + NS < kt1; ++kt) body(kt, std::true_type{}, std::true_type{});
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

}  // namespace
}  // namespace mla
