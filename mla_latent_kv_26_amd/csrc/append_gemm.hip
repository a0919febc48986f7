// Cache append fused into its down-projection ("GatedMLA" docs, "Build
// per-head Q, K and V": the W_DKV output split into the compressed latent and
// the shared key; "Projection geometry and stored weights": RMSNorm on the
// latent; modeldna "MLA" module, "Under the hood": the rope key rotated and
// cached beside the latent), bf16 with kv_lora_rank 512 and rope_dim 64:
//
//   z = x W_DKV (576 columns);  row = [RMSNorm(z[:512]) g | RoPE(z[512:], p)]
//
// One workgroup (4 waves, one per SIMD) computes a 64-row panel of z with
// all 576 columns in registers (16x16x32 MFMAs, 144 float32 accumulators per
// lane, which stay in the accumulation registers), so the row-wise RMSNorm
// and the rotation run on the accumulators and z never leaves the CU; the
// rows go straight to their cache slots in bf16, or as FP8 rows (E4M3 codes
// with a power-of-two row scale, bf16 rope key).
//
// Panel layout: wave w owns columns 144 w .. +143 (nine 16-column blocks)
// of all 64 rows (four 16-row blocks).  The product is taken transposed
// (C^T = W^T x^T: the W fragment is the MFMA's first operand), so a lane
// owns one row per row block and runs of 4 columns; the row sums of squares
// and maxima need two lane swaps (l ^ 16, l ^ 32) and one LDS exchange
// between the four waves.
//
// Operands stream HBM/L2 -> LDS with direct-to-LDS loads, four stages of
// 32 k: x rows [64][32] (4 KB; chunk c of row m at c ^ ((m >> 2) & 3)) and
// W rows [32][576] (36 KB; chunk c of row k at c ^ (2 bit1(k) + 4 bit3(k)),
// so the 8 rows x 32 bytes a transposing read of 32 lanes touches fall on
// distinct bank groups).  Each thread issues 10 of a stage's 40 one-KB loads.
// Fragment reads come from inline assembly and are completed by one wait
// that names their registers: the compiler's own LDS reads would first wait
// for every direct-to-LDS load in flight.
//
// In the prefill with a query rank, x W_DQ (256 x 256 tiles of the tile GEMM)
// runs in the same launch: at 8192 rows, 128 panel workgroups and 192 tiles.
#include "launch.h"
#include "tile_gemm.h"

namespace mla {
namespace {

constexpr int kPM = 64, kPN = 576, kPK = 32, kPStages = 4, kPThreads = 256;
constexpr int kPR = 512, kPDr = 64;
constexpr int kPABytes = kPM * kPK * 2;              // 4 KB
constexpr int kPBRow = kPN * 2;                      // 1152 bytes per k row
constexpr int kPBBytes = kPK * kPBRow;               // 36 KB
constexpr int kPStage = kPABytes + kPBBytes;         // 40 KB
constexpr int kPLoads = kPStage / 1024 / 4;          // 10 per thread and stage
constexpr int kPXLoads = kPABytes / 1024;            // the first 4 of 40 load x
constexpr int kPRB = kPM / 16;                       // 4 row blocks
constexpr int kPCB = kPN / 4 / 16;                   // 9 column blocks per wave
static_assert(kPStages * kPStage <= 160 * 1024, "LDS budget");
static_assert(kPLoads * 4 * 1024 == kPStage, "every stage slot loaded once");

// Where a panel's rows go.
struct AppendDst {
  void* pool;
  int fp8;                 // FP8 rows (R + 2 Dr + 16 bytes) instead of bf16
  const float* gain;       // [512]
  const float* rope;       // [positions, 64]: cos | sin halves
  float eps;
  // slot mode (mla_cache_append): position and slot per token
  const int* pos;
  const int* slot;
  // paged mode (prefill): token t = b T + i at position start_pos[b] + i
  const int* start_pos;
  const int* block_table;
  int T, max_blocks, block_size;
};

// Element offset (from x or from W) of this thread's load j (0 .. 39) of a
// stage: slot j of 40, 4 x rows then 36 W rows.
__device__ __forceinline__ uint32_t panel_src(long ldx, int rows, int row0, int j, int lane) {
  const int p = j * 64 + lane;
  if (j < kPXLoads) {
    const int m = p >> 2, c = (p & 3) ^ ((m >> 2) & 3);
    return (uint32_t)(min(row0 + m, rows - 1) * ldx + 8 * c);
  }
  const int q = p - kPXLoads * 64, k = q / 72;
  const int c = (q % 72) ^ (2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1));
  return (uint32_t)(k * kPN + 8 * c);
}

// One stage's fragments: four x row blocks (16-byte row reads) and nine W
// column blocks (two transposing reads each), completed by panel_settle.
struct PanelFrag {
  bf16x8 a[kPRB];
  bf16x4 t[kPCB][2];
};
constexpr int kPCBA = 5;  // W blocks read with the x fragments
__device__ __forceinline__ void panel_issue_a(PanelFrag& f, uint32_t st,
                                              const uint32_t (&a_off)[kPRB],
                                              const uint32_t (&b_off)[kPCB]) {
#pragma unroll
  for (int rb = 0; rb < kPRB; ++rb) ds_b128_nowait<0>(f.a[rb], st + a_off[rb]);
#pragma unroll
  for (int cb = 0; cb < kPCBA; ++cb) {
    ds_tr_nowait<0>(f.t[cb][0], st + b_off[cb]);
    ds_tr_nowait<4 * kPBRow>(f.t[cb][1], st + b_off[cb]);
  }
}
__device__ __forceinline__ void panel_issue_b(PanelFrag& f, uint32_t st,
                                              const uint32_t (&b_off)[kPCB]) {
#pragma unroll
  for (int cb = kPCBA; cb < kPCB; ++cb) {
    ds_tr_nowait<0>(f.t[cb][0], st + b_off[cb]);
    ds_tr_nowait<4 * kPBRow>(f.t[cb][1], st + b_off[cb]);
  }
}
// each waits for the reads in flight (one part at a time) and hands that
// part's registers on
__device__ __forceinline__ void panel_settle_a(PanelFrag& f) {
  static_assert(kPRB == 4 && kPCBA == 5 && 2 * (kPCB - kPCBA) == 8, "operand list below");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.t[0][0]),
                 "+v"(f.t[0][1]), "+v"(f.t[1][0]), "+v"(f.t[1][1]), "+v"(f.t[2][0]),
                 "+v"(f.t[2][1]), "+v"(f.t[3][0]), "+v"(f.t[3][1]), "+v"(f.t[4][0]),
                 "+v"(f.t[4][1]));
}
__device__ __forceinline__ void panel_settle_b(PanelFrag& f) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(f.t[5][0]), "+v"(f.t[5][1]), "+v"(f.t[6][0]), "+v"(f.t[6][1]),
                 "+v"(f.t[7][0]), "+v"(f.t[7][1]), "+v"(f.t[8][0]), "+v"(f.t[8][1]));
}

// z panel (rows row0 .. row0 + 63 of x [rows, K] row-major, ldx) times W
// [K, 576] into acc; acc[rb][cb] holds C^T blocks: register v of lane l is
// row 16 rb + l % 16, column 144 wave + 16 cb + 4 (l / 16) + v.
__device__ __forceinline__ void panel_mainloop(uint32_t lds, const bf16* x, long ldx, int rows,
                                               int row0, const bf16* w, int K,
                                               f32x4 (&acc)[kPRB][kPCB]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nk = K / kPK;
  // element offsets of this thread's loads (x rows first, then W rows)
  uint32_t src[kPLoads];
#pragma unroll
  for (int q = 0; q < kPLoads; ++q) src[q] = panel_src(ldx, rows, row0, wave * kPLoads + q, lane);
  auto issue = [&](int kt) {
    const uint32_t st = lds + (uint32_t)(kt % kPStages) * kPStage;
    // stage bases made opaque, so the per-load 64-bit addresses are formed
    // here rather than kept (and spilled) across the loop
    const bf16* xk = x + (long)kt * kPK;
    const bf16* wk = w + (long)kt * kPK * kPN;
    asm volatile("" : "+s"(xk), "+s"(wk));
#pragma unroll
    for (int q = 0; q < kPLoads; ++q) {
      const int j = wave * kPLoads + q;  // x loads step 32 columns, W loads 32 rows
      g2lds16((j < kPXLoads ? xk : wk) + src[q], st + (uint32_t)j * 1024u);
    }
  };
  // fragment offsets inside a stage: x rows (b128) and W columns (transposing)
  const int g = lane >> 4, li = lane & 15;
  uint32_t a_off[kPRB];
#pragma unroll
  for (int rb = 0; rb < kPRB; ++rb) {
    const int m = 16 * rb + li;
    a_off[rb] = (uint32_t)(m * 64 + ((g ^ ((m >> 2) & 3)) * 16));
  }
  // W fragment of column block cb: rows k = 8 g + li / 4 (+ 4 for the second
  // read, which keeps bits 1 and 3), columns 144 wave + 16 cb + 4 (li % 4)
  const int kb = 8 * g + (li >> 2);
  const uint32_t sw = 2u * ((kb >> 1) & 1) + 4u * ((kb >> 3) & 1);
  uint32_t b_off[kPCB];
#pragma unroll
  for (int cb = 0; cb < kPCB; ++cb) {
    const int col = 144 * wave + 16 * cb + 4 * (li & 3);
    b_off[cb] = (uint32_t)(kPABytes + kb * kPBRow + (((uint32_t)(col >> 3) ^ sw) * 16) +
                           ((col >> 2) & 1) * 8);
  }

#pragma unroll
  for (int rb = 0; rb < kPRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kPCB; ++cb) acc[rb][cb] = f32x4{};

  for (int kt = 0; kt < min(nk, kPStages - 1); ++kt) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's loads of stage kt have landed (later ones may be in flight)
    const int later = min(nk - 1 - kt, kPStages - 2);
    if (later >= 2)
      wait_vmcnt<2 * kPLoads>();
    else if (later == 1)
      wait_vmcnt<kPLoads>();
    else
      wait_vmcnt<0>();
    lds_barrier();  // every thread's stage kt landed; stage kt - 1's buffer is free
    if (kt + kPStages - 1 < nk) issue(kt + kPStages - 1);
    const uint32_t st = lds + (uint32_t)(kt % kPStages) * kPStage;
    // the x fragments and W blocks 0 .. 4 first; blocks 5 .. 8 are read
    // while the first blocks' MFMAs run
    PanelFrag f;
    panel_issue_a(f, st, a_off, b_off);
    panel_settle_a(f);
    __builtin_amdgcn_sched_barrier(0);
    panel_issue_b(f, st, b_off);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cb = 0; cb < kPCBA; ++cb) {
      const bf16x8 bw = cat(f.t[cb][0], f.t[cb][1]);
#pragma unroll
      for (int rb = 0; rb < kPRB; ++rb) acc[rb][cb] = mfma16(bw, f.a[rb], acc[rb][cb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    panel_settle_b(f);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cb = kPCBA; cb < kPCB; ++cb) {
      const bf16x8 bw = cat(f.t[cb][0], f.t[cb][1]);
#pragma unroll
      for (int rb = 0; rb < kPRB; ++rb) acc[rb][cb] = mfma16(bw, f.a[rb], acc[rb][cb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  lds_barrier();  // every wave is done with the stages
}

// Cache slot and position of token t, or slot -1.
__device__ __forceinline__ long row_slot(const AppendDst& d, int t, int n, int& pos) {
  if (t >= n) return -1;
  if (d.slot) {
    pos = d.pos[t];
    return d.slot[t];
  }
  const int b = t / d.T, i = t - b * d.T;
  pos = d.start_pos[b] + i;
  return (long)d.block_table[(long)b * d.max_blocks + pos / d.block_size] * d.block_size +
         pos % d.block_size;
}

// RMSNorm, RoPE and the store of the panel's rows.  A lane owns one row per
// row block (its columns split with lanes l ^ 16, l ^ 32 and the other three
// waves).  LDS: per (row, wave) the sum of squares and the latent max, float
// [64][4][2]; the gain vector float [512].
__device__ __forceinline__ void panel_epilogue(uint32_t lds, const f32x4 (&acc)[kPRB][kPCB],
                                               const AppendDst& d, int row0, int n) {
  typedef __attribute__((address_space(3))) float lds_f;
  typedef __attribute__((address_space(3))) f32x4 lds_f4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const uint32_t xch = lds, gl = lds + kPM * 8 * 4;
  for (int k = threadIdx.x; k < kPR; k += kPThreads) *(lds_f*)(uintptr_t)(gl + 4 * k) = d.gain[k];
  // latent blocks of this wave: all 9, except columns 512 .. 575 of wave 3
  const int nlat = wave == 3 ? 5 : kPCB;
  float inv[kPRB];
#pragma unroll
  for (int rb = 0; rb < kPRB; ++rb) {
    float s = 0.f;
#pragma unroll
    for (int cb = 0; cb < kPCB; ++cb)
      if (cb < nlat)
#pragma unroll
        for (int v = 0; v < 4; ++v) s = fmaf(acc[rb][cb][v], acc[rb][cb][v], s);
    s = sum_xor32(sum_xor16(s));
    if (g == 0) *(lds_f*)(uintptr_t)(xch + ((16 * rb + li) * 8 + 2 * wave) * 4) = s;
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < kPRB; ++rb) {
    const uint32_t r = xch + (16 * rb + li) * 32;
    const float ss = (*(lds_f*)(uintptr_t)r + *(lds_f*)(uintptr_t)(r + 8)) +
                     (*(lds_f*)(uintptr_t)(r + 16) + *(lds_f*)(uintptr_t)(r + 24));
    inv[rb] = 1.0f / sqrtf(ss / (float)kPR + d.eps);
  }
  // FP8: the row's largest |c| sets its power-of-two scale
  float scale[kPRB];
#pragma unroll
  for (int rb = 0; rb < kPRB; ++rb) scale[rb] = 1.0f;
  if (d.fp8) {
#pragma unroll
    for (int rb = 0; rb < kPRB; ++rb) {
      float mx = 0.f;
#pragma unroll
      for (int cb = 0; cb < kPCB; ++cb)
        if (cb < nlat) {
          const f32x4 gv = *(lds_f4*)(uintptr_t)(gl + 4 * (144 * wave + 16 * cb + 4 * g));
#pragma unroll
          for (int v = 0; v < 4; ++v) mx = fmaxf(mx, fabsf(acc[rb][cb][v] * inv[rb] * gv[v]));
        }
      mx = max_xor32(max_xor16(mx));
      if (g == 0) *(lds_f*)(uintptr_t)(xch + ((16 * rb + li) * 8 + 2 * wave + 1) * 4) = mx;
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kPRB; ++rb) {
      const uint32_t r = xch + (16 * rb + li) * 32 + 4;
      const float amax = fmaxf(fmaxf(*(lds_f*)(uintptr_t)r, *(lds_f*)(uintptr_t)(r + 8)),
                               fmaxf(*(lds_f*)(uintptr_t)(r + 16), *(lds_f*)(uintptr_t)(r + 24)));
      if (amax > 0.f) {
        int E;
        const float m = frexpf(amax, &E);
        scale[rb] = ldexpf(1.0f, m <= 0.875f ? E - 9 : E - 8);
      }
    }
  }
  typedef short __attribute__((ext_vector_type(2))) short2v;
  const long row_bytes = d.fp8 ? kPR + 2 * kPDr + 16 : (kPR + kPDr) * 2;
#pragma unroll
  for (int rb = 0; rb < kPRB; ++rb) {
    int pos = 0;
    const long s = row_slot(d, row0 + 16 * rb + li, n, pos);
    if (s < 0) continue;
    unsigned char* dst = (unsigned char*)d.pool + s * row_bytes;
#pragma unroll
    for (int cb = 0; cb < kPCB; ++cb) {
      if (cb < nlat) {
        const int c0 = 144 * wave + 16 * cb + 4 * g;
        const f32x4 gv = *(lds_f4*)(uintptr_t)(gl + 4 * c0);
        float c[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) c[v] = acc[rb][cb][v] * inv[rb] * gv[v];
        if (d.fp8) {
          const short2v lo =
              __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2v{0, 0}, c[0], c[1], scale[rb], false);
          const short2v pk =
              __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c[2], c[3], scale[rb], true);
          *(unsigned*)(dst + c0) = __builtin_bit_cast(unsigned, pk);
        } else {
          bf16x4 o;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = (bf16)c[v];
          *(bf16x4*)(dst + 2 * c0) = o;
        }
      } else if (cb == 5 || cb == 6) {
        // rope key (wave 3): element e = 16 (cb - 5) + 4 g + v of block cb
        // pairs with the same element of block cb + 2 (e + 32)
        const int e0 = 16 * (cb - 5) + 4 * g;
        const float* rr = d.rope + (long)pos * kPDr;
        const f32x4 cs = *(const f32x4*)(rr + e0);
        const f32x4 sn = *(const f32x4*)(rr + kPDr / 2 + e0);
        bf16* kd = (bf16*)(dst + (d.fp8 ? kPR : 2 * kPR));
        bf16x4 o1, o2;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float a = acc[rb][cb][v], b = acc[rb][cb + 2][v];
          o1[v] = (bf16)(a * cs[v] - b * sn[v]);
          o2[v] = (bf16)(b * cs[v] + a * sn[v]);
        }
        *(bf16x4*)(kd + e0) = o1;
        *(bf16x4*)(kd + kPDr / 2 + e0) = o2;
      }
    }
    if (d.fp8 && wave == 3 && g == 0) {
      // the row's scale and 12 zero bytes after the rope key
      const f32x4 tail = {scale[rb], 0.f, 0.f, 0.f};
      *(f32x4*)(dst + kPR + 2 * kPDr) = tail;
    }
  }
  __syncthreads();  // the exchange area is free before the next panel's loads
}

// Panels (blocks 0 .. np8 - 1, np8 a multiple of 8; block p takes panels p,
// p + np8, ...) and the 256 x 256 tiles of C = x B (float32, the q-rank
// projection) with the tile GEMM's XCD-grouped mapping.
__global__ void __launch_bounds__(kTThreads, 1) project_append_kernel(
    const bf16* __restrict__ x, long ldx, int n, int K, const bf16* __restrict__ w, AppendDst d,
    int np8, const bf16* __restrict__ B, int N, long ldb, float* __restrict__ C, long ldc,
    int m_per) {
  constexpr int kLds = kPStages * kPStage > kTStages * TileCfg<256>::STAGE
                           ? kPStages * kPStage
                           : kTStages * TileCfg<256>::STAGE;
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  const uint32_t lds = lds_addr(smem);
  const int blk = blockIdx.x;
  if (blk < np8) {
    for (int row0 = blk * kPM; row0 < n; row0 += np8 * kPM) {
      f32x4 acc[kPRB][kPCB];
      panel_mainloop(lds, x, ldx, n, row0, w, K, acc);
      panel_epilogue(lds, acc, d, row0, n);
    }
    return;
  }
  using Cf = TileCfg<256>;
  const int tb = blk - np8;
  const int n_mt = (n + kTM - 1) / kTM, n_nt = (N + 255) / 256;
  const int xx = tb & 7, j = tb >> 3;
  const int r_first = xx * m_per;
  if (r_first >= n_mt) return;
  const int rows_here = min(m_per, n_mt - r_first);
  if (j >= rows_here * n_nt) return;
  const int m0 = (r_first + j % rows_here) * kTM, n0 = (j / rows_here) * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  TileSrc<256, false> src;
  tile_sources<256, false>(src, x, n, ldx, m0, B, N, ldb, n0, N, 0, wave, lane);
  f32x16 acc[4][Cf::FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < Cf::FN; ++jb) acc[i][jb] = f32x16{};
  tile_mainloop<256, false>(lds, src, 0, K / kTK, acc);
  tile_epilogue<256, true, false>(acc, C, n, N, ldc, m0, n0, 1.0f, nullptr);
}

AppendDst make_dst(void* pool, bool fp8, const float* gain, const float* rope, float eps) {
  AppendDst d{};
  d.pool = pool;
  d.fp8 = fp8 ? 1 : 0;
  d.gain = gain;
  d.rope = rope;
  d.eps = eps;
  return d;
}

}  // namespace

bool append_gemm_fits(int R, int Dr, int K, long ldx) {
  return R == kPR && Dr == kPDr && K >= kPK && K % kPK == 0 && ldx % 8 == 0;
}

void launch_append_gemm(const void* x, long ldx, int n, int K, const void* w_dkv,
                        const float* gain, const float* rope, const int* pos, const int* slot,
                        void* pool, bool fp8, float eps, hipStream_t st) {
  if (n <= 0) return;
  AppendDst d = make_dst(pool, fp8, gain, rope, eps);
  d.pos = pos;
  d.slot = slot;
  const int np8 = ((n + kPM - 1) / kPM + 7) / 8 * 8;  // one panel per workgroup
  project_append_kernel<<<np8, kPThreads, 0, st>>>((const bf16*)x, ldx, n, K, (const bf16*)w_dkv,
                                                   d, np8, nullptr, 0, 0, nullptr, 0, 0);
}

void launch_project_append(const void* x, long ldx, int batch, int T, int K, const void* w_dkv,
                           const float* gain, const float* rope, const int* start_pos,
                           const int* block_table, int max_blocks, int block_size, void* pool,
                           bool fp8, float eps, const void* w_q, int N, long ldb, float* c,
                           long ldc, hipStream_t st) {
  const int n = batch * T;
  if (n <= 0) return;
  AppendDst d = make_dst(pool, fp8, gain, rope, eps);
  d.start_pos = start_pos;
  d.block_table = block_table;
  d.T = T;
  d.max_blocks = max_blocks;
  d.block_size = block_size;
  // one panel per workgroup, also beside the q-rank tiles: a panel streams
  // all of W_DKV, so two panels per workgroup (one round of the CUs with the
  // tiles) measured 4 % slower than a partial second round
  const int np = (n + kPM - 1) / kPM;
  const int np8 = (np + 7) / 8 * 8;
  int tiles = 0, m_per = 0;
  if (w_q) {
    const int n_mt = (n + kTM - 1) / kTM, n_nt = (N + 255) / 256;
    m_per = (n_mt + 7) / 8;
    tiles = 8 * m_per * n_nt;
  }
  project_append_kernel<<<np8 + tiles, kPThreads, 0, st>>>(
      (const bf16*)x, ldx, n, K, (const bf16*)w_dkv, d, np8, (const bf16*)w_q, N, ldb, c, ldc,
      m_per);
}

}  // namespace mla
