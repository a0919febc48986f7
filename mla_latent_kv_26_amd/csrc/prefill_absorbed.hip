// Causal prefill attention in the absorbed form, on MFMA (gfx950), over a
// paged bf16 pool of latent rows [c (512) | k_rope (64)].
//
// Query row r = (token t of sequence b, head h) sits at position
// p = start_pos[b] + t and attends to its sequence's rows 0 .. p (GatedMLA
// docs, "Observe logits, then compute causal attention"); with W_UK folded
// into the query (modeldna "MLA" module, "Under the hood"):
//   s[r, j]  = q_full[r] . row_j            (q_full scaled by scale * log2 e)
//   o_lat[r] = sum_j 2^(s[r,j] - m_r) c_j / sum_j 2^(s[r,j] - m_r).
// Every head of every new token reads the same rows, so a workgroup takes
// 128 query rows at once (2 consecutive tokens x 64 heads, or 4 x 32) and
// streams their common key range 0 .. p_max through LDS once, in 32-row
// tiles, instead of once per query row.
//
// Workgroup: 256 threads, 4 waves (one per SIMD, up to 512 registers each).
// Wave w owns
//   * the scores of query rows 32w .. 32w+31 (one token, 32 heads), their
//     queries in registers:  S^T[32 keys x 32 rows] = T[32 x 576] Q^T, 36
//     32x32x16 MFMAs per tile, A from 16-byte LDS reads of the tile;
//     a lane owns one query row (and 16 of the 32 keys), so row maxima and
//     sums need one permlane32 swap;
//   * columns 128w .. 128w+127 of O for all 128 rows, O^T accumulated in
//     256 registers: O^T[128 x 128] += T[:, cols]^T P^T, 32 MFMAs per tile,
//     A from transposing LDS reads of the tile, B = P from LDS.
// Per tile step k: the scores of tile k, then P*C of tile k-1 (whose P every
// wave published before the step's barrier), then the softmax of tile k
// (base-2, reference max moved only when a tile exceeds it by more than 8,
// so P < 2^8 and O is rescaled rarely), publishing P, the rescale factors
// and a per-wave "rescaled" flag.  One LDS barrier per step.  Tiles go
// HBM/L2 -> LDS by direct-to-LDS loads (9 per wave and tile) into three
// buffers: tile k+1 loads while tiles k (scores) and k-1 (P*C) are read.
//
// Tile layout as in the decode kernel: row t (72 chunks of 16 B) at
// t * 1152, chunk k at position k ^ swz(t) within its group of 8, which
// keeps both the row-wise and the transposing fragment reads free of bank
// conflicts.  P: [128 rows][32 keys] bf16, chunk c of row r at
// c ^ ((r >> 2) & 3) (16 rows of one chunk hit 16 distinct bank slots).
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace mla {
namespace {

constexpr int kR = 512, kDr = 64, kW = kR + kDr;  // row width 576
constexpr int kTok = 32;                          // keys per tile
constexpr int kCh = kW * 2 / 16;                  // 72 chunks per row
constexpr int kTileBytes = kTok * kW * 2;         // 36864
constexpr int kNBuf = 3;
constexpr int kRows = 128;                        // query rows per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoads = kTileBytes / 1024 / kWaves;  // 9 load instructions per wave and tile
constexpr int kNK = kW / 16;                        // 36 k-steps of the scores
constexpr int kSAhead = 4;                          // score fragments read ahead
constexpr int kPBytes = kRows * kTok * 2;           // 8192
constexpr int kOffP = kNBuf * kTileBytes;           // bf16 [2][128][32]
constexpr int kOffOver = kOffP + 2 * kPBytes;       // float [4]: a wave saw a weight overflow
constexpr int kOffInv = kOffOver + 16;              // float [32][4]: 1 / row sum
// Query columns from kQL * 16 on (the last 128 of 576) live in LDS, not in
// registers: bf16 [128 rows][128], chunk c of row r at c ^ (r % 16).
constexpr int kQL = 28;                             // score k-steps with queries in registers
constexpr int kOffQ = kOffInv + kRows * 4;
constexpr int kQRow = (kNK - kQL) * 32;             // 256 bytes per row
constexpr int kLdsBytes = kOffQ + kRows * kQRow;
static_assert(kLdsBytes <= 163840, "LDS budget");
static_assert(kLoads * kWaves * 1024 == kTileBytes, "every tile slot loaded once");
// Weights are 2^(s - m_ref) with m_ref fixed per row (the first tile's
// maximum): no rescaling of O.  A score more than this above m_ref (a weight
// above 2^64) sends the workgroup through its key range once more with the
// row maxima as references.
constexpr float kHeadroom = 64.0f;

__device__ __forceinline__ uint32_t swz(uint32_t t) {
  return (((t >> 1) & 1u) << 2) | ((t >> 2) & 3u);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// O lives in accumulation registers named in the code: block i = 4 rb + cb
// of O^T is a[16 i .. 16 i + 15].  Every statement that touches a block lists
// its registers as clobbered; nothing else in the kernel uses accumulation
// registers (the score MFMAs write ordinary registers), so no value of the
// compiler's own is ever kept there.  The MFMAs start with s_nop 1: the two
// wait states a VALU write of a source needs (the compiler inserts none for
// assembly); they issue while the previous MFMA occupies the pipe.
template <int I>
struct OBlk;
#define MLA_OBLK(I, LO, HI, r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11, r12, r13, r14, r15) \
  template <> \
  struct OBlk<I> { \
    static __device__ __forceinline__ void zero() { \
      asm volatile("v_accvgpr_write_b32 a" #r0 ", 0\n\t" "v_accvgpr_write_b32 a" #r1 ", 0\n\t" \
          "v_accvgpr_write_b32 a" #r2 ", 0\n\t" "v_accvgpr_write_b32 a" #r3 ", 0\n\t" \
          "v_accvgpr_write_b32 a" #r4 ", 0\n\t" "v_accvgpr_write_b32 a" #r5 ", 0\n\t" \
          "v_accvgpr_write_b32 a" #r6 ", 0\n\t" "v_accvgpr_write_b32 a" #r7 ", 0\n\t" \
          "v_accvgpr_write_b32 a" #r8 ", 0\n\t" "v_accvgpr_write_b32 a" #r9 ", 0\n\t" \
          "v_accvgpr_write_b32 a" #r10 ", 0\n\t" "v_accvgpr_write_b32 a" #r11 ", 0\n\t" \
          "v_accvgpr_write_b32 a" #r12 ", 0\n\t" "v_accvgpr_write_b32 a" #r13 ", 0\n\t" \
          "v_accvgpr_write_b32 a" #r14 ", 0\n\t" "v_accvgpr_write_b32 a" #r15 ", 0\n\t" : : : \
          "a" #r0, "a" #r1, "a" #r2, "a" #r3, "a" #r4, "a" #r5, "a" #r6, "a" #r7, "a" #r8, "a" \
          #r9, "a" #r10, "a" #r11, "a" #r12, "a" #r13, "a" #r14, "a" #r15); \
    } \
    static __device__ __forceinline__ void mfma(const bf16x8& a, const bf16x8& b) { \
      asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[" #LO ":" #HI "], %0, %1, a[" #LO \
          ":" #HI "]" : : "v"(a), "v"(b) : "a" #r0, "a" #r1, "a" #r2, "a" #r3, "a" #r4, "a" \
          #r5, "a" #r6, "a" #r7, "a" #r8, "a" #r9, "a" #r10, "a" #r11, "a" #r12, "a" #r13, "a" \
          #r14, "a" #r15); \
    } \
    static __device__ __forceinline__ void read(float (&e)[16]) { \
      asm volatile("v_accvgpr_read_b32 %0, a" #r0 "\n\t" "v_accvgpr_read_b32 %1, a" #r1 "\n\t" \
          "v_accvgpr_read_b32 %2, a" #r2 "\n\t" "v_accvgpr_read_b32 %3, a" #r3 "\n\t" \
          "v_accvgpr_read_b32 %4, a" #r4 "\n\t" "v_accvgpr_read_b32 %5, a" #r5 "\n\t" \
          "v_accvgpr_read_b32 %6, a" #r6 "\n\t" "v_accvgpr_read_b32 %7, a" #r7 "\n\t" \
          "v_accvgpr_read_b32 %8, a" #r8 "\n\t" "v_accvgpr_read_b32 %9, a" #r9 "\n\t" \
          "v_accvgpr_read_b32 %10, a" #r10 "\n\t" "v_accvgpr_read_b32 %11, a" #r11 "\n\t" \
          "v_accvgpr_read_b32 %12, a" #r12 "\n\t" "v_accvgpr_read_b32 %13, a" #r13 "\n\t" \
          "v_accvgpr_read_b32 %14, a" #r14 "\n\t" "v_accvgpr_read_b32 %15, a" #r15 "\n\t" : \
          "=v"(e[0]), "=v"(e[1]), "=v"(e[2]), "=v"(e[3]), "=v"(e[4]), "=v"(e[5]), "=v"(e[6]), \
          "=v"(e[7]), "=v"(e[8]), "=v"(e[9]), "=v"(e[10]), "=v"(e[11]), "=v"(e[12]), \
          "=v"(e[13]), "=v"(e[14]), "=v"(e[15])); \
    } \
  };
MLA_OBLK(0, 0, 15, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15)
MLA_OBLK(1, 16, 31, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31)
MLA_OBLK(2, 32, 47, 32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43, 44, 45, 46, 47)
MLA_OBLK(3, 48, 63, 48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63)
MLA_OBLK(4, 64, 79, 64, 65, 66, 67, 68, 69, 70, 71, 72, 73, 74, 75, 76, 77, 78, 79)
MLA_OBLK(5, 80, 95, 80, 81, 82, 83, 84, 85, 86, 87, 88, 89, 90, 91, 92, 93, 94, 95)
MLA_OBLK(6, 96, 111, 96, 97, 98, 99, 100, 101, 102, 103, 104, 105, 106, 107, 108, 109, 110, 111)
MLA_OBLK(7, 112, 127, 112, 113, 114, 115, 116, 117, 118, 119, 120, 121, 122, 123, 124, 125, 126, 127)
MLA_OBLK(8, 128, 143, 128, 129, 130, 131, 132, 133, 134, 135, 136, 137, 138, 139, 140, 141, 142, 143)
MLA_OBLK(9, 144, 159, 144, 145, 146, 147, 148, 149, 150, 151, 152, 153, 154, 155, 156, 157, 158, 159)
MLA_OBLK(10, 160, 175, 160, 161, 162, 163, 164, 165, 166, 167, 168, 169, 170, 171, 172, 173, 174, 175)
MLA_OBLK(11, 176, 191, 176, 177, 178, 179, 180, 181, 182, 183, 184, 185, 186, 187, 188, 189, 190, 191)
MLA_OBLK(12, 192, 207, 192, 193, 194, 195, 196, 197, 198, 199, 200, 201, 202, 203, 204, 205, 206, 207)
MLA_OBLK(13, 208, 223, 208, 209, 210, 211, 212, 213, 214, 215, 216, 217, 218, 219, 220, 221, 222, 223)
MLA_OBLK(14, 224, 239, 224, 225, 226, 227, 228, 229, 230, 231, 232, 233, 234, 235, 236, 237, 238, 239)
MLA_OBLK(15, 240, 255, 240, 241, 242, 243, 244, 245, 246, 247, 248, 249, 250, 251, 252, 253, 254, 255)
#undef MLA_OBLK

// Score accumulation S += A B in ordinary registers.  The last of a chain
// ends with 19 wait states, what a VALU read of its result needs.
template <bool kLast>
__device__ __forceinline__ void mfma32_v(f32x16& o, const bf16x8& a, const bf16x8& b) {
  if constexpr (kLast)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 2"
                 : "+v"(o) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(o) : "v"(a), "v"(b));
}

// Waits until at most N LDS operations of this wave are outstanding and
// hands a quarter step's P*C fragments on as written here.
template <int N>
__device__ __forceinline__ void settle_q(bf16x8 (&pa)[4], bf16x4 (&t)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(pa[0]), "+v"(pa[1]), "+v"(pa[2]), "+v"(pa[3]), "+v"(t[0]), "+v"(t[1]),
                 "+v"(t[2]), "+v"(t[3])
               : "i"(N));
}

template <int OFF>
__device__ __forceinline__ void ds_f32x4_nowait(f32x4& o, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(o) : "v"(a), "i"(OFF));
}

// Page ids of one sequence, 64 at a time: lane i holds the id of page index
// base + i (clamped to the table row).  Pages are visited in order; a new
// chunk is loaded and waited for at once (every 64 pages).
struct Pages {
  const int* row;
  int max_blocks, base, ids;
  __device__ __forceinline__ void start(const int* r, int mb, int lane) {
    row = r;
    max_blocks = mb;
    base = 0;
    ids = row[min(lane, mb - 1)];
    wait_vmcnt<0>();
    asm volatile("" : "+v"(ids));
  }
  __device__ __forceinline__ int page(int p, int lane) {
    if (p - base >= 64) {
      base = p;
      ids = row[min(base + lane, max_blocks - 1)];
      wait_vmcnt<0>();
      asm volatile("" : "+v"(ids));
    }
    return __builtin_amdgcn_readlane(ids, p - base);
  }
};

// This wave's 9 of the 36 direct-to-LDS loads of tile `tile` (keys 32 tile
// .. 32 tile + 31; keys past last_key repeat the last valid row, so the tile
// holds finite data; they are masked).
__device__ __forceinline__ void issue_tile(const bf16* pool, Pages& pg, int shift, int tile,
                                           int last_key, uint32_t buf, int wave, int lane) {
  const int tok = tile * kTok;
  const int page = pg.page(tok >> shift, lane);
  const int mask = (1 << shift) - 1;
  const bf16* rows = pool + ((long)page * (mask + 1) + (tok & mask)) * kW;
  const uint32_t valid = (uint32_t)min(kTok, last_key + 1 - tok);
  // The lane's source offsets are recomputed at each tile (a few VALU
  // operations) rather than kept in registers across the tile loop.
  uint32_t ln = (uint32_t)lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const uint32_t j = (uint32_t)(kLoads * wave + i);
    const uint32_t s = 64u * j + ln;
    const uint32_t t = s / kCh;
    const uint32_t k = (s - t * kCh) ^ swz(t);
    const uint32_t tt = min(t, valid - 1);
    g2lds16(rows + (tt * kW + k * 8), buf + j * 1024u);
  }
}

template <int HEADS>
__global__ void __launch_bounds__(kThreads, 1) prefill_absorbed_kernel(
    const bf16* __restrict__ q_full, const bf16* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int shift,
    const int* __restrict__ start_pos, int T, int batch, int H, bf16* __restrict__ o_lat) {
  static_assert(HEADS == 32 || HEADS == 64, "32 or 64 heads per workgroup");
  constexpr int QT = kRows / HEADS;  // tokens per workgroup
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const uint32_t lds = lds_addr(smem);
  const int lane = (int)threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const uint32_t lr = (uint32_t)lane & 31u, lh = (uint32_t)lane >> 5;

  // Work item: head group, sequence and token block; the blocks with the
  // longest key ranges (the last tokens) first, sequences interleaved.
  const int hgc = H / HEADS;
  const int nblk = (T + QT - 1) / QT;
  const int hg = (int)blockIdx.x % hgc;
  const int r = (int)blockIdx.x / hgc;
  const int b = r % batch;
  const int t0 = (nblk - 1 - r / batch) * QT;
  const int sp = start_pos[b];
  const int last_key = sp + min(t0 + QT - 1, T - 1);  // keys 0 .. last_key
  const int n = last_key / kTok + 1;                   // tiles
  // this wave's score rows: one token (rows past T repeat the last token)
  const int tw = min(t0 + (32 * wave) / HEADS, T - 1);
  const int pw = sp + tw;  // its keys: 0 .. pw

  Pages pg;
  pg.start(block_table + (long)b * max_blocks, max_blocks, lane);
  issue_tile(pool, pg, shift, 0, last_key, lds, wave, lane);
  bf16x8 qf[kNK];
  {
    const int head = hg * HEADS + (32 * wave) % HEADS + (int)lr;
    const bf16* q = q_full + ((long)(b * T + tw) * H + head) * kW + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < kNK; ++ks) qf[ks] = *(const bf16x8*)(q + 16 * ks);
  }
  if (n > 1) issue_tile(pool, pg, shift, 1, last_key, lds + kTileBytes, wave, lane);
  // tile 0 and the queries land (tile 1 may stay in flight); the queries are
  // handed on as plain register values, so no wait in the loop is tied to
  // their loads
  if (n > 1) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < kQL; ++ks) asm volatile("" : "+v"(qf[ks]));
  // the query tail to LDS (each wave reads back only its own rows, after
  // its own writes, so no barrier is needed)
  const uint32_t q_lds = lds + kOffQ + (32u * wave + lr) * kQRow;
#pragma unroll
  for (int ks = kQL; ks < kNK; ++ks)
    *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(
        q_lds + (((2u * (ks - kQL) + lh) ^ (lr & 15u)) * 16u)) = qf[ks];

  // score fragment (ks): key lr, chunk 2 ks + lh, at 128 (ks / 4) +
  // 16 ((2 (ks % 4) + lh) ^ swz(lr)) within row lr
  uint32_t soff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) soff[m] = lr * (kCh * 16) + (((2u * m + lh) ^ swz(lr)) * 16u);
  // P*C transposing reads: lane (16 g + li) reads row x + 4 hi (+ 16 ks) of
  // chunk 16 w + 4 cb + 2 (g % 2) + b1 (+ 8 bytes for odd li); with both
  // halves, lane l holds column 128 w + 32 cb + l % 32, keys 8 (l / 32) + 0..7.
  // Offsets for cb = 0, 1; cb + 2 is 8 chunks (128 bytes) further.
  uint32_t tr_off[4];
  {
    const uint32_t g = (uint32_t)lane >> 4, li = (uint32_t)lane & 15;
    const uint32_t x = 8u * (g >> 1) + (li >> 2), b1 = (li >> 1) & 1u;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const uint32_t cc = 4u * (cb & 1) + 2u * (g & 1) + b1;
        const uint32_t row = x + 4u * hi;
        tr_off[2 * cb + hi] = (row * kCh + 16u * wave + (cc ^ swz(row))) * 16u + 8u * (li & 1);
      }
  }
  // P fragment (B operand, rows 32 rb + lr, keys 16 ks + 8 lh .. + 7):
  // chunk 2 ks + lh of row lr + 32 rb
  const uint32_t p_rd0 = lr * 64u + (((0u + lh) ^ ((lr >> 2) & 3u)) * 16u);
  const uint32_t p_rd1 = lr * 64u + (((2u + lh) ^ ((lr >> 2) & 3u)) * 16u);
  // P written by this lane: row 32 w + lr, keys 8 j + 4 lh .. + 3
  const uint32_t p_row = (32u * wave + lr) * 64u + 8u * lh;
  const uint32_t p_sw = ((32u * wave + lr) >> 2) & 3u;
  // Source offsets (elements) of this wave's 9 loads of a full tile, two
  // 16-bit offsets per register: slot s = 64 j + lane holds chunk
  // (s % 72) ^ swz(t) of row t = s / 72.
  uint32_t dma_off[(kLoads + 1) / 2];
  {
    uint32_t o[kLoads + 1];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const uint32_t s = 64u * (uint32_t)(kLoads * wave + i) + (uint32_t)lane;
      const uint32_t t = s / kCh;
      o[i] = t * kW + ((s - t * kCh) ^ swz(t)) * 8u;
    }
    o[kLoads] = 0;
#pragma unroll
    for (int i = 0; i < (kLoads + 1) / 2; ++i) dma_off[i] = o[2 * i] | (o[2 * i + 1] << 16);
  }

  // m_ref: this lane's row reference for the weights, fixed within a pass;
  // m_hi: the largest score of the row so far
  float m_ref = -INFINITY, m_hi = -INFINITY, l = 0.f;
  for (int pass = 0;; ++pass) {
    static_for<0, 16>([&](auto c) { OBlk<decltype(c)::value>::zero(); });
    l = 0.f;
    bool over = false;
    if (pass > 0) {
      pg.start(block_table + (long)b * max_blocks, max_blocks, lane);
      issue_tile(pool, pg, shift, 0, last_key, lds, wave, lane);
      if (n > 1) issue_tile(pool, pg, shift, 1, last_key, lds + kTileBytes, wave, lane);
    }
    for (int k = 0; k <= n; ++k) {
      // tile k landed: in flight at the top of step k are {tile 0, tile 1}
      // (k = 0; waited for before the loop in the first pass), {tile 1,
      // tile 2} (k = 1), {tile k} (k >= 2)
      if (k == 0) {
        if (pass > 0) {
          if (n > 1) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
        }
      } else if (k == 1) {
        if (n > 2) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      asm volatile("" : "+v"(pg.ids));
      lds_barrier();
      // The tile this step loads, into the buffer of tile k-2 (last read by
      // P*C of tile k-2, in step k-1): tile 2 at step 0, none at step 1,
      // tile k+1 after.  A full tile's loads go out one by one among the
      // score MFMAs; a partial last tile (rows clamped) goes out here.
      const int ld = k == 0 ? 2 : (k >= 2 ? k + 1 : n);
      bool ld_full = false;
      const bf16* ld_rows = pool;
      uint32_t ld_buf = lds;
      if (ld < n) {
        ld_buf = lds + (uint32_t)(ld % kNBuf) * kTileBytes;
        if ((ld + 1) * kTok <= last_key + 1) {
          const int tok = ld * kTok;
          const int page = pg.page(tok >> shift, lane);
          const int mask = (1 << shift) - 1;
          ld_rows = pool + ((long)page * (mask + 1) + (tok & mask)) * kW;
          ld_full = true;
        } else {
          issue_tile(pool, pg, shift, ld, last_key, ld_buf, wave, lane);
        }
      }
      auto dma_one = [&](auto ci) {
        constexpr int i = decltype(ci)::value;
        // unpacked here, not once before the loop (nine live registers)
        uint32_t pk2 = dma_off[i / 2];
        asm volatile("" : "+v"(pk2));
        const uint32_t off = (i & 1) ? (pk2 >> 16) : (pk2 & 0xffffu);
        g2lds16(ld_rows + off, ld_buf + (uint32_t)(kLoads * wave + i) * 1024u);
      };

      // P*C of tile k-1 in quarters q = (16-key half ks = q / 2, column
      // blocks 2 (q % 2) .. + 1): the P fragments of half ks (4 rows blocks)
      // come with its first quarter, each quarter's two transposed column
      // fragments with it; a quarter's reads are in flight during the
      // previous quarter's MFMAs.
      const int kp = k - 1;
      const uint32_t pc_buf = lds + (uint32_t)((kp + kNBuf) % kNBuf) * kTileBytes;
      const uint32_t pb = lds + kOffP + (uint32_t)(kp & 1) * kPBytes;
      bf16x8 pa[2][4];
      bf16x4 tf[4][4];
      auto pc_reads = [&](auto cq) {
        constexpr int q = decltype(cq)::value, ks = q / 2, ch = q % 2;
        if constexpr (ch == 0) {
          const uint32_t pr = pb + (ks == 0 ? p_rd0 : p_rd1);
          ds_b128_nowait<0 * 2048>(pa[ks][0], pr);
          ds_b128_nowait<1 * 2048>(pa[ks][1], pr);
          ds_b128_nowait<2 * 2048>(pa[ks][2], pr);
          ds_b128_nowait<3 * 2048>(pa[ks][3], pr);
        }
        // column blocks 2 ch and 2 ch + 1; block cb + 2 sits 8 chunks after cb
        ds_tr_nowait<ks * 16 * kCh * 16 + ch * 128>(tf[q][0], pc_buf + tr_off[0]);
        ds_tr_nowait<ks * 16 * kCh * 16 + ch * 128>(tf[q][1], pc_buf + tr_off[1]);
        ds_tr_nowait<ks * 16 * kCh * 16 + ch * 128>(tf[q][2], pc_buf + tr_off[2]);
        ds_tr_nowait<ks * 16 * kCh * 16 + ch * 128>(tf[q][3], pc_buf + tr_off[3]);
      };

      // ---- scores of tile k, with this step's tile loads among them ----
      f32x16 sacc = f32x16{};
      auto scores = [&]() {
        const uint32_t buf = lds + (uint32_t)(k % kNBuf) * kTileBytes;
        bf16x8 kf[kSAhead + 1], qt[kSAhead + 1];
        // fragment reads of k-step j: the tile row chunk, and from kQL on the
        // query tail chunk (2 (j - kQL) + lh) ^ (lr % 16) of this lane's row
        auto rd = [&](auto cj) {
          constexpr int j = decltype(cj)::value;
          ds_b128_nowait<128 * (j / 4)>(kf[j % (kSAhead + 1)], buf + soff[j % 4]);
          if constexpr (j >= kQL)
            ds_b128_nowait<0>(qt[j % (kSAhead + 1)],
                              q_lds + (((2u * (j - kQL) + lh) ^ (lr & 15u)) * 16u));
        };
        static_for<0, kSAhead>([&](auto c) { rd(c); });
        static_for<0, kNK>([&](auto c) {
          constexpr int ks = decltype(c)::value;
          constexpr int nx = ks + kSAhead;
          if constexpr (nx < kNK) rd(std::integral_constant<int, nx>{});
          // LDS reads issued after this k-step's: one or two per later k-step
          constexpr int last = (ks + kSAhead < kNK - 1) ? ks + kSAhead : kNK - 1;
          constexpr int later = (last - ks) + (last >= kQL ? last - (ks >= kQL ? ks : kQL - 1) : 0);
          if constexpr (ks < kQL) {
            lds_settle<later>(kf[ks % (kSAhead + 1)]);
            mfma32_v<false>(sacc, kf[ks % (kSAhead + 1)], qf[ks]);
          } else {
            lds_settle<later>(kf[ks % (kSAhead + 1)], qt[ks % (kSAhead + 1)]);
            mfma32_v<ks == kNK - 1>(sacc, kf[ks % (kSAhead + 1)], qt[ks % (kSAhead + 1)]);
          }
          if constexpr (ks % 4 == 1) {
            if (ld_full) dma_one(std::integral_constant<int, ks / 4>{});
          }
        });
      };

      // ---- P*C of tile k-1, with the weights of tile k among its MFMAs ----
      // register v of sacc <-> key 32 k + 8 (v/4) + 4 lh + v%4 of row 32 w + lr
      float tmax = 0.f;
      bf16x4 pk[4];
      float ps[4];
      auto w_max = [&]() {
        asm volatile("" : "+v"(sacc));
        if (k * kTok + kTok - 1 > pw) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k * kTok + 8 * (v / 4) + 4 * (int)lh + (v % 4);
            if (key > pw) sacc[v] = -INFINITY;
          }
        }
        tmax = fmaxf(fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3])),
                     fmaxf(fmaxf(sacc[4], sacc[5]), fmaxf(sacc[6], sacc[7])));
        tmax = fmaxf(tmax, fmaxf(fmaxf(fmaxf(sacc[8], sacc[9]), fmaxf(sacc[10], sacc[11])),
                                 fmaxf(fmaxf(sacc[12], sacc[13]), fmaxf(sacc[14], sacc[15]))));
        tmax = max_xor32(tmax);
        // tile 0 holds key 0, so the first pass's reference is finite
        if (pass == 0 && k == 0) m_ref = tmax;
        m_hi = fmaxf(m_hi, tmax);
        over |= tmax > m_ref + kHeadroom;
        asm volatile("" : "+v"(m_ref), "+v"(sacc));
      };
      auto w_exp = [&](auto cj) {
        constexpr int j = decltype(cj)::value;
        float mr = m_ref;
        asm volatile("" : "+v"(mr));
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bf16 p = (bf16)fast_exp2(sacc[4 * j + v] - mr);
          pk[j][v] = p;
          sum += (float)p;
        }
        ps[j] = sum;
        asm volatile("" : "+v"(pk[j]), "+v"(ps[j]));
      };
      auto w_store = [&]() {
        const uint32_t pw_addr = lds + kOffP + (uint32_t)(k & 1) * kPBytes + p_row;
#pragma unroll
        for (int j = 0; j < 4; ++j) lds_st(pw_addr + (((uint32_t)j ^ p_sw) * 16u), pk[j]);
        l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      };
      // One quarter of P*C: its reads done (the next quarter's may stay in
      // flight), 8 MFMAs, the next-but-one quarter's reads issued after them.
      // W(i) places the weight computations among the MFMAs.
      auto pc_quarter = [&](auto cq, auto W) {
        constexpr int q = decltype(cq)::value, ks = q / 2, ch = q % 2;
        if constexpr (q == 0) settle_q<4>(pa[0], tf[0]);
        if constexpr (q == 1) settle_q<8>(pa[0], tf[1]);
        if constexpr (q == 2) settle_q<4>(pa[1], tf[2]);
        if constexpr (q == 3) settle_q<0>(pa[1], tf[3]);
        static_for<0, 8>([&](auto c) {
          constexpr int i = decltype(c)::value, cbl = i / 4, rb = i % 4, cb = 2 * ch + cbl;
          OBlk<4 * rb + cb>::mfma(cat(tf[q][2 * cbl], tf[q][2 * cbl + 1]), pa[ks][rb]);
          W(std::integral_constant<int, 8 * q + i>{});
        });
        if constexpr (q == 0) pc_reads(std::integral_constant<int, 2>{});
        if constexpr (q == 1) pc_reads(std::integral_constant<int, 3>{});
      };
      if (k < n && k > 0) {
        // Even waves compute the scores first, odd waves after half of P*C,
        // so at any time only two waves stream score fragments from LDS.
        // The weights go among the last 16 MFMAs (after the scores).
        auto W = [&](auto ci) {
          constexpr int i = decltype(ci)::value;
          if constexpr (i == 16) w_max();
          if constexpr (i == 19) w_exp(std::integral_constant<int, 0>{});
          if constexpr (i == 22) w_exp(std::integral_constant<int, 1>{});
          if constexpr (i == 24) w_exp(std::integral_constant<int, 2>{});
          if constexpr (i == 27) w_exp(std::integral_constant<int, 3>{});
          if constexpr (i == 29) w_store();
        };
        if ((wave & 1) == 0) scores();
        pc_reads(std::integral_constant<int, 0>{});
        pc_reads(std::integral_constant<int, 1>{});
        pc_quarter(std::integral_constant<int, 0>{}, W);
        pc_quarter(std::integral_constant<int, 1>{}, W);
        if ((wave & 1) != 0) scores();
        pc_quarter(std::integral_constant<int, 2>{}, W);
        pc_quarter(std::integral_constant<int, 3>{}, W);
      } else if (k > 0) {
        auto W = [&](auto) {};
        pc_reads(std::integral_constant<int, 0>{});
        pc_reads(std::integral_constant<int, 1>{});
        static_for<0, 4>([&](auto cq) { pc_quarter(cq, W); });
      } else {
        scores();
        w_max();
        static_for<0, 4>([&](auto cj) { w_exp(cj); });
        w_store();
      }
    }
    // Done unless some row of the workgroup scored more than kHeadroom above
    // its reference (its weights could have overflowed): then every wave
    // runs the key range again with each row's true maximum as reference.
    const bool wave_over = __ballot(over) != 0ull;  // every lane votes (outside the branch)
    if (lane == 0) lds_st(lds + kOffOver + wave * 4u, wave_over ? 1.0f : 0.0f);
    lds_barrier();
    f32x4 ov;
    ds_f32x4_nowait<0>(ov, lds + kOffOver);
    lds_settle<0>(ov);
    const float any_over = ov[0] + ov[1] + ov[2] + ov[3];
    if (pass > 0 || __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, any_over)) == 0) break;
    m_ref = m_hi;
  }

  // ---- epilogue: 1 / row sum to the owners of the columns, O / l out ----
  l = sum_xor32(l);
  if (lh == 0) lds_st(lds + kOffInv + (lr * 4u + wave) * 4u, 1.0f / l);
  lds_barrier();
  f32x4 inv;
  ds_f32x4_nowait<0>(inv, lds + kOffInv + lr * 16u);
  lds_settle<0>(inv);
  static_for<0, 4>([&](auto cr) {
    constexpr int rb = decltype(cr)::value;
    const int row = 32 * rb + (int)lr;
    const int t = t0 + row / HEADS;
    bf16* dst = o_lat + ((long)(b * T + min(t, T - 1)) * H + hg * HEADS + row % HEADS) * kR +
                128 * wave + 4 * lh;
    static_for<0, 4>([&](auto cc) {
      constexpr int cb = decltype(cc)::value;
      float e[16];
      OBlk<4 * rb + cb>::read(e);
      if (t < T) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 o;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = (bf16)(e[4 * q + v] * inv[rb]);
          *(bf16x4*)(dst + 32 * cb + 8 * q) = o;
        }
      }
    });
  });
}

}  // namespace

void launch_attention_prefill_bf16(const void* q_full, const void* pool, const int* block_table,
                                   int max_blocks, int block_shift, const int* start_pos, int T,
                                   int batch, int H, void* o_lat, hipStream_t st) {
  if (T <= 0 || batch <= 0) return;
  if (H % 64 == 0) {
    const int blocks = batch * ((T + 1) / 2) * (H / 64);
    prefill_absorbed_kernel<64><<<blocks, kThreads, 0, st>>>(
        (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_shift, start_pos, T,
        batch, H, (bf16*)o_lat);
  } else {
    const int blocks = batch * ((T + 3) / 4) * (H / 32);
    prefill_absorbed_kernel<32><<<blocks, kThreads, 0, st>>>(
        (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_shift, start_pos, T,
        batch, H, (bf16*)o_lat);
  }
}

}  // namespace mla
