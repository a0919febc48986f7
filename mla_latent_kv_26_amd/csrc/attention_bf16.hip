// Latent attention on MFMA (gfx950), bf16 cache rows, float32 accumulate.
//
// For one query row and up to 64 heads (modeldna "MLA" module, "Under the
// hood": W_UK absorbed into the query, attention run on the cached latent):
//   s[h, j]  = q_full[h] . row_j          (q_full = scale*log2e*[q_lat | q_rope])
//   o_lat[h] = sum_j 2^(s[h,j] - m[h]) c_j / sum_j 2^(s[h,j] - m[h]).
// The rows are dense bf16 [c (512) | k_rope (64)], 1152 B each, shared by
// every head, so both contractions are matrix products:
//   S^T [32 tok x 16 h] = T [32 tok x 576] * Q^T [576 x 16 h]   (per score wave)
//   O   [H x 128]      += P [H x 32 tok] * T[:, 128 w .. +128]   (per P*C wave)
// and one LDS copy of each 32-token tile serves both: T is read row-wise for
// S (16-byte LDS reads) and column-wise for P*C (transposing LDS reads), so
// every cached byte leaves HBM once.
//
// Workgroup: 512 threads = 8 waves, one "score" wave and one "P*C" wave per
// SIMD, working on consecutive tiles at once.  In step k the score waves
// compute S, the softmax and P for tile k (each owns 16 heads and all 32
// tokens, so row maxima need no exchange between waves) while the P*C waves
// fold P of tile k-1 into O (each owns 128 columns of O for all heads, fp32
// in registers).  One barrier per step hands P from one group to the other.
// Tiles stream HBM -> LDS with asynchronous direct-to-LDS loads into four
// buffers: tiles k-1 and k are being read, k+1 and k+2 are in flight.
//
// Tile layout in LDS: row-major, row t (1152 B = 72 chunks of 16 B) at
// t*1152, with its chunk k stored at position k ^ swz(t) (a permutation
// inside each aligned group of 8 chunks).  A direct-to-LDS load instruction
// fills 64 consecutive slots; its lanes read the matching 1 KB of global
// memory in that permuted order, so every instruction stays fully coalesced.
// The LDS serves a 16-byte read 16 lanes (256 bytes) at a time and an
// 8-byte read 32 lanes at a time; rows are 1152 B (128 mod 256).  swz(t) =
// 4 ((t/2) % 2) + (t/4) % 4 gives the 16 consecutive rows of a row-wise
// fragment read 16 distinct 16-byte bank slots, and the 4 rows x 4 chunks
// of a transposing read (rows 4-aligned, chunks 4-aligned) 16 distinct
// slots too: neither access pattern has bank conflicts.
#include <algorithm>
#include <climits>
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kR = 512, kDr = 64, kW = kR + kDr;       // row width 576
constexpr int kTok = 32;                                // tokens per tile
constexpr int kCh = kW * 2 / 16;                        // 72 chunks per row
constexpr int kTileBytes = kTok * kW * 2;               // 36864
constexpr int kNBuf = 4;                                // tile buffers
constexpr int kTileLoads = kTileBytes / 1024;           // 36 1-KB load instructions
constexpr int kSLoads = 4, kPLoads = 5;                 // per score wave / per P*C wave
constexpr int kSAhead = 4;  // score fragment pairs read ahead of their MFMAs
static_assert(4 * kSLoads + 4 * kPLoads == kTileLoads, "every slot loaded once");
// The tile loads can also all go to the P*C waves (SL = 0 score-wave loads,
// 9 per P*C wave): that takes the load issue off the score waves' chain,
// which sets the tile step where HBM does not (two head groups of 64 heads,
// each tile read by two workgroups: 3-4 % off the attention at H=128), and
// costs where the stream binds (4 x 131,072 tokens 1-2 % slower).
template <int SL>
__device__ __forceinline__ constexpr int p_loads() {
  static_assert(SL >= 0 && 4 * SL <= kTileLoads && (kTileLoads - 4 * SL) % 4 == 0, "load split");
  return (kTileLoads - 4 * SL) / 4;
}
constexpr int kMaxHG = 64;                              // heads per workgroup, at most
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPStride = kTok + 8;                      // bf16 per P row (80 B)
constexpr int kOStride = kR + 8;                        // bf16 per staged output row
constexpr int kMaxBatch = 1024;

constexpr int kOffP = kNBuf * kTileBytes;               // bf16 [2][64][40]
constexpr int kOffAlpha = kOffP + 2 * kMaxHG * kPStride * 2;  // float [2][64]
constexpr int kOffFlag = kOffAlpha + 2 * kMaxHG * 4;    // float [2][4] rescale flags
constexpr int kOffInv = kOffFlag + 2 * 4 * 4;           // float [64] 1 / row sum
constexpr int kOffScan = kOffInv + kMaxHG * 4;          // int [8] scan scratch
constexpr int kOffPrefix = kOffScan + 32;               // int [kMaxBatch + 1]
constexpr int kOffLenLo = kOffPrefix + (kMaxBatch + 1) * 4;  // uint8 [kMaxBatch]
constexpr int kLdsBytes = kOffLenLo + kMaxBatch;
static_assert(kLdsBytes <= 163840, "LDS budget");
static_assert(kMaxHG * kOStride * 2 <= kNBuf * kTileBytes, "output staging fits the tile buffers");

// Per-HEADS geometry: SW score waves of 16 heads; HB 32-head row blocks of O
// per P*C wave.
template <int HEADS>
struct Geo {
  static_assert(HEADS == 32 || HEADS == 64, "32 or 64 heads per workgroup");
  static constexpr int SW = HEADS / 16;
  static constexpr int HB = HEADS / 32;
};
// A head's reference max only moves when a tile exceeds it by more than this
// (log2 units): probabilities stay below 2^8 and O is rescaled rarely.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ uint32_t swz(uint32_t t) { return (((t >> 1) & 1u) << 2) | ((t >> 2) & 3u); }

// Page ids of one sequence, 64 at a time in a register (lane i holds the id
// of page index base + i), the following 64 loaded ahead.  Loads are plain
// vector loads issued before the tile loads of the same step, so waiting for
// a tile also retires them.  Indices are clamped to the table row.
struct PageCursor {
  const int* row;
  int max_blocks, base, cur, nxt;

  __device__ __forceinline__ int fetch(int first, int lane) const {
    return row[min(first + lane, max_blocks - 1)];
  }
  __device__ __forceinline__ void start(const int* r, int mb, int page0, int lane) {
    row = r;
    max_blocks = mb;
    base = page0;
    cur = fetch(base, lane);
    nxt = fetch(base + 64, lane);
  }
  // page id of page index p (p >= base, p < base + 128, non-decreasing).
  // A new chunk (once per 64 pages) is waited for at once and handed on as
  // a plain value: a load still in flight in a register carried around the
  // tile loop makes the compiler wait for every load, tile loads included,
  // wherever the register is copied.
  __device__ __forceinline__ int page(int p, int lane) {
    if (p - base >= 64) {
      cur = nxt;
      base += 64;
      nxt = fetch(base + 64, lane);
      wait_vmcnt<0>();
      asm volatile("" : "+v"(nxt));
    }
    return __builtin_amdgcn_readlane(cur, p - base);
  }
};

// Issue this wave's share of the asynchronous loads of one tile: NL
// instructions j = j0 .. j0+NL-1, each filling LDS slots [64 j, 64 j + 64)
// of the buffer.  `valid` rows (1..32) start at row pointer `rows`
// (consecutive rows of one page); rows past `valid` repeat the last valid
// row so the tile holds finite data (their probabilities are zero).
template <int NL>
__device__ __forceinline__ void issue_part(const bf16* rows, int valid, uint32_t buf, uint32_t j0,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const uint32_t j = j0 + i;
    const uint32_t s = 64u * j + (uint32_t)lane;
    const uint32_t t = s / kCh;
    const uint32_t k = (s - t * kCh) ^ swz(t);
    const uint32_t tt = min(t, (uint32_t)(valid - 1));
    g2lds16(rows + tt * kW + k * 8, buf + j * 1024u);
  }
}

// FP8 cache rows (R E4M3 codes | Dr bf16 rope values | float32 scale | 12
// zero bytes, 656 bytes = 41 chunks; the softved article's advice to
// quantize the cache, in a format it leaves open).  Tiles stay FP8 in LDS:
// the score waves widen the codes of their fragments in registers (scale 1)
// and apply each row's power-of-two scale to its score, s = scale (q_lat .
// code) + q_rope . k_rope; the P*C waves read the codes transposed and take
// P scaled by the row's scale (exact in bf16), so O = sum P scale code.  HBM
// and LDS move 656 instead of 1152 bytes per token, and six 24 KB staging
// slots keep four tiles in flight.
// A staged tile comes by 24 direct-to-LDS instructions of 1 KB, 3 per wave:
// slot s < 1280 is position s % 40 of row s / 40 (rows of 640 bytes: 32
// code chunks, then 8 rope chunks), slots 1280 .. 1535 hold the scale chunk
// of row (s - 1280) % 32 (eight copies).  Chunk c of row t sits at position
// 8 (c / 8) + ((c % 8) ^ s8(t)): the 16 rows x 16 bytes of a score fragment
// read and the 8 rows x 2 chunks of a transposing read (32 lanes each) then
// fall on distinct bank slots.  Rows past `valid` repeat the last valid row.
constexpr int kF8Row = kR + 2 * kDr + 16;               // 656 bytes
constexpr int kF8Data = (kR + 2 * kDr) / 16;            // 40 data chunks per row
constexpr int kF8RowBytes = kF8Data * 16;               // 640 bytes per staged row
constexpr int kF8ScaleOff = kTok * kF8RowBytes;         // scale chunks of the slot
constexpr int kF8Loads = 3;                             // per wave and tile
constexpr int kF8StageBytes = 8 * kF8Loads * 1024;      // 24 KB
constexpr int kF8Slots = 6;                             // tiles k-1, k and four in flight
static_assert(kTok * kF8Data + kTok <= kF8StageBytes / 16, "staging slots");
static_assert(kF8Slots * kF8StageBytes <= kOffP, "FP8 LDS layout");

__device__ __forceinline__ uint32_t s8(uint32_t t) { return (((t >> 1) & 3u) << 1) | ((t >> 3) & 1u); }

__device__ __forceinline__ void issue_part_fp8(const unsigned char* rows, int valid, uint32_t stg,
                                               uint32_t j0, int lane) {
#pragma unroll
  for (int i = 0; i < kF8Loads; ++i) {
    const uint32_t j = j0 + i;
    const uint32_t s = 64u * j + (uint32_t)lane;
    uint32_t t, c;
    if (s < (uint32_t)(kTok * kF8Data)) {
      t = s / kF8Data;
      const uint32_t p = s - t * kF8Data;
      c = (p & ~7u) | ((p & 7u) ^ s8(t));
    } else {
      t = (s - kTok * kF8Data) & (kTok - 1);
      c = kF8Data;
    }
    const uint32_t tt = min(t, (uint32_t)(valid - 1));
    g2lds16(rows + tt * kF8Row + c * 16, stg + j * 1024u);
  }
}

// One segment: a query row (HEADS heads at q_rows, row stride kW) against
// tiles [tile0, tile1) of one sequence of `len` rows (page table `table`).
struct SegArgs {
  const bf16* q_rows;
  const bf16* pool;
  const int* table;
  int max_blocks, shift, len, tile0, tile1;
  const PageCursor* pre;  // page ids already loaded for tile0's page, or null
  bool tile0_issued;      // tile0's loads already in flight into buffer 0
  bool tile1_issued;      // and tile0 + 1's into buffer 1
};

// Where the loads of local tile x go and the waves read it: four bf16 tile
// buffers or six FP8 staging slots, round robin.
template <bool kFp8>
__device__ __forceinline__ uint32_t load_slot(uint32_t lds, int x) {
  if constexpr (kFp8)
    return lds + (uint32_t)(x % kF8Slots) * kF8StageBytes;
  else
    return lds + (uint32_t)(x % kNBuf) * kTileBytes;
}
// Loads per wave and tile, and the first load index of wave `wave`.
template <bool kFp8, int SL = kSLoads>
__device__ __forceinline__ constexpr int tile_loads(bool score) {
  return kFp8 ? kF8Loads : score ? SL : p_loads<SL>();
}
template <bool kFp8, int SL = kSLoads>
__device__ __forceinline__ uint32_t first_load(int wave) {
  if constexpr (kFp8) return (uint32_t)wave * kF8Loads;
  return wave < 4 ? (uint32_t)wave * SL : 4u * SL + (uint32_t)(wave - 4) * p_loads<SL>();
}

// This wave's share of the loads of segment tile `tile` into `dst`.
template <bool kFp8, int NL>
__device__ __forceinline__ void issue_tile(const SegArgs& a, PageCursor& pc, int tile,
                                           uint32_t dst, uint32_t j0, int lane) {
  const int tok = tile * kTok;
  const int page = pc.page(tok >> a.shift, lane);
  const int mask = (1 << a.shift) - 1;
  const long row = (long)page * (mask + 1) + (tok & mask);
  const int valid = min(kTok, a.len - tok);
  if constexpr (kFp8)
    issue_part_fp8((const unsigned char*)a.pool + row * kF8Row, valid, dst, j0, lane);
  else
    issue_part<NL>(a.pool + row * kW, valid, dst, j0, lane);
}

// Segment prologue shared by both wave roles: the page ids, then this
// wave's share of tile 0 (the caller issues its queries, then tile 1).
template <bool kFp8, int NL>
__device__ __forceinline__ void seg_start(const SegArgs& a, PageCursor& pc, uint32_t lds,
                                          uint32_t j0, int lane) {
  if (a.pre) {
    pc = *a.pre;
  } else {
    pc.start(a.table, a.max_blocks, (a.tile0 * kTok) >> a.shift, lane);
    // Tile 0's address needs the page ids at once; waited for here, before
    // any tile load, they become plain values.  (Registers loaded before
    // direct-to-LDS loads are otherwise completed by the compiler with a
    // drain of every load in flight, placed where the tile loop starts and
    // so paid on every step.)
    wait_vmcnt<0>();
    asm volatile("" : "+v"(pc.cur), "+v"(pc.nxt));
  }
  if (!a.tile0_issued) issue_tile<kFp8, NL>(a, pc, a.tile0, load_slot<kFp8>(lds, 0), j0, lane);
}

// Step-top synchronisation shared by both wave roles (bf16 rows): wait for
// this wave's loads of tile k (tile k+1 may stay in flight), barrier.  The
// caller then issues tile k+2 into the buffer tile k-2 used (step_issue):
// the P*C waves at once, the score waves after their first MFMA pair, so
// that the 36 load instructions of a tile do not all queue behind the
// barrier together (measured: 2 % off the attention at H=128).
template <int NL>
__device__ __forceinline__ void step_sync(const SegArgs& a, PageCursor& pc, uint32_t lds,
                                          uint32_t j0, int k, int n, int lane) {
  if (k < n) {
    if (k + 1 < n)
      wait_vmcnt<NL>();
    else
      wait_vmcnt<0>();
  }
  // The page-id loads went out before the tile loads just waited for, so
  // they have landed: hand their registers on as plain values (the compiler
  // would otherwise wait for every load in flight, tile k+1 included, before
  // it reads a page id).
  asm volatile("" : "+v"(pc.cur), "+v"(pc.nxt));
  lds_barrier();
}
template <int NL>
__device__ __forceinline__ void step_issue(const SegArgs& a, PageCursor& pc, uint32_t lds,
                                           uint32_t j0, int k, int n, int lane) {
  if (k + 2 < n) issue_tile<false, NL>(a, pc, a.tile0 + k + 2, load_slot<false>(lds, k + 2), j0, lane);
}

// Queries of head 16 sw + lane%16, chunks 4 ks + lane/16 (the B operand of
// the score MFMAs), from the segment's query rows.  FP8 rows: loaded into
// registers (the split into e4m3 terms follows).
__device__ __forceinline__ void load_queries(const bf16* q_rows, int sw, int lane,
                                             bf16x8 (&qf)[kW / 32]) {
  const bf16* q = q_rows + (16 * sw + (lane & 15)) * kW + 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < kW / 32; ++ks) qf[ks] = *(const bf16x8*)(q + 32 * ks);
}
// bf16 rows: staged through LDS.  Score wave sw's 18 KB go by direct-to-LDS
// loads into tile buffers 2 and 3, load ks filling 1 KB at q_stage(sw) +
// 1024 ks with lane l's 16 bytes, and come back into registers by 16-byte
// LDS reads before the segment's first barrier (tile 2 is issued into
// buffer 2 only after it, tile 3 into buffer 3 a step later).  Loaded into
// registers by vector loads instead, the queries make the compiler complete
// them by draining every load in flight, so the first step waits for tile 1
// as well as tile 0 (measured 0.4 us per step at 32 x 4096 tokens; for FP8
// rows staging measured no faster).
constexpr uint32_t kQStage = (kW / 32) * 1024;  // 18 KB per score wave
static_assert(4 * kQStage <= 2 * kTileBytes, "staged queries fit tile buffers 2 and 3");
__device__ __forceinline__ uint32_t q_stage(uint32_t lds, int sw) {
  return lds + 2u * kTileBytes + (uint32_t)sw * kQStage;
}
__device__ __forceinline__ void stage_queries(const bf16* q_rows, int sw, int lane, uint32_t lds) {
  const bf16* q = q_rows + (16 * sw + (lane & 15)) * kW + 8 * (lane >> 4);
  const uint32_t dst = q_stage(lds, sw);
#pragma unroll
  for (int ks = 0; ks < kW / 32; ++ks) g2lds16(q + 32 * ks, dst + (uint32_t)ks * 1024u);
}
// The staged queries into registers (after the wave's wait for them).
__device__ __forceinline__ void read_staged_queries(uint32_t lds, int sw, int lane,
                                                    bf16x8 (&qf)[kW / 32]) {
  static_assert(kW / 32 == 18, "eighteen query fragments");
  const uint32_t a = q_stage(lds, sw) + 16u * (uint32_t)lane;
  ds_b128_nowait<0 * 1024>(qf[0], a);
  ds_b128_nowait<1 * 1024>(qf[1], a);
  ds_b128_nowait<2 * 1024>(qf[2], a);
  ds_b128_nowait<3 * 1024>(qf[3], a);
  ds_b128_nowait<4 * 1024>(qf[4], a);
  ds_b128_nowait<5 * 1024>(qf[5], a);
  ds_b128_nowait<6 * 1024>(qf[6], a);
  ds_b128_nowait<7 * 1024>(qf[7], a);
  ds_b128_nowait<8 * 1024>(qf[8], a);
  ds_b128_nowait<9 * 1024>(qf[9], a);
  ds_b128_nowait<10 * 1024>(qf[10], a);
  ds_b128_nowait<11 * 1024>(qf[11], a);
  ds_b128_nowait<12 * 1024>(qf[12], a);
  ds_b128_nowait<13 * 1024>(qf[13], a);
  ds_b128_nowait<14 * 1024>(qf[14], a);
  ds_b128_nowait<15 * 1024>(qf[15], a);
  ds_b128_nowait<16 * 1024>(qf[16], a);
  ds_b128_nowait<17 * 1024>(qf[17], a);
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]), "+v"(qf[4]), "+v"(qf[5]),
                 "+v"(qf[6]), "+v"(qf[7]), "+v"(qf[8]), "+v"(qf[9]), "+v"(qf[10]), "+v"(qf[11]),
                 "+v"(qf[12]), "+v"(qf[13]), "+v"(qf[14]), "+v"(qf[15]), "+v"(qf[16]),
                 "+v"(qf[17]));
}

// Score wave `sw` (heads 16 sw .. 16 sw + 15): runs the segment's steps and
// returns (in lanes 0..15) the reference max and full row sum of head
// 16 sw + lane.  Inactive score waves (sw >= SW) only take part in loads and
// barriers.  qf receives the segment's queries from their LDS staging:
// staged with the guessed tiles when q_ready, else staged here (after tile 0,
// before tile 1).
template <int HEADS, int SL>
__device__ __forceinline__ void score_role(const SegArgs& a, uint32_t lds, int sw, int lane,
                                           bf16x8 (&qf)[kW / 32], bool q_ready, float& m_out,
                                           float& l_out) {
  using G = Geo<HEADS>;
  const bool active = sw < G::SW;
  const int n = a.tile1 - a.tile0;
  constexpr int NL = tile_loads<false, SL>(true);
  const uint32_t j0 = first_load<false, SL>(sw);
  PageCursor pc;
  seg_start<false, NL>(a, pc, lds, j0, lane);

  const int h = 16 * sw + (lane & 15);
  const uint32_t kq = lane >> 4;
  if (active && !q_ready) stage_queries(a.q_rows, sw, lane, lds);
  // tile 0 and the queries (issued before tile 1) land; tile 1 may stay in flight
  if (n > 1) {
    if (!a.tile1_issued) issue_tile<false, NL>(a, pc, a.tile0 + 1, load_slot<false>(lds, 1), j0, lane);
    wait_vmcnt<NL>();
  } else {
    wait_vmcnt<0>();
  }
  // the staged queries into registers, before the first barrier frees
  // their buffers for tiles 2 and 3
  if (active) read_staged_queries(lds, sw, lane, qf);

  // S fragment (ks, tb): row tr0 + 16 tb, chunk 4 ks + kq at position
  // 8 (ks/2) + ((4 (ks%2) + kq) ^ swz(tr0)); swz depends on lane%16 only.
  const uint32_t tr0 = lane & 15;
  const uint32_t s_even = (tr0 * kCh + (kq ^ swz(tr0))) * 16u;
  const uint32_t s_odd = (tr0 * kCh + ((4u + kq) ^ swz(tr0))) * 16u;
  const uint32_t pw_base = lds + kOffP + (h * kPStride + 4 * kq) * 2;

  float m = -INFINITY, l = 0.f;
  for (int k = 0; k <= n; ++k) {
    step_sync<NL>(a, pc, lds, j0, k, n, lane);
    if (k == n || !active) {
      step_issue<NL>(a, pc, lds, j0, k, n, lane);
      continue;
    }
    const uint32_t buf = load_slot<false>(lds, k);
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
    {
      // Fragments (ks, tb = 0 and 1) are read kSAhead steps ahead of their
      // MFMAs, from inline assembly without a wait, and each pair is
      // completed by a wait that allows the later pairs to stay in flight
      // (LDS reads complete in order) and names its registers.  Reads the
      // compiler issues itself are completed by full drains of the LDS
      // queue, which expose the whole read latency several times a tile.
      // The scheduling barriers keep each step's reads, wait and MFMAs in
      // this order.
      constexpr int NK = kW / 32;
      const uint32_t be = buf + s_even, bo = buf + s_odd;
      auto issue = [&](int ks, bf16x8(&f)[2]) {
        const uint32_t ad = ((ks & 1) ? bo : be) + (uint32_t)((ks >> 1) * 128);
        ds_b128_nowait<0>(f[0], ad);
        ds_b128_nowait<16 * kCh * 16>(f[1], ad);
      };
      // waits until at most 2 * later LDS reads of this wave are pending
      auto settle = [&](bf16x8(&f)[2], int later) {
        switch (later) {
          case 0: lds_settle<0>(f[0], f[1]); break;
          case 1: lds_settle<2>(f[0], f[1]); break;
          case 2: lds_settle<4>(f[0], f[1]); break;
          case 3: lds_settle<6>(f[0], f[1]); break;
          default: lds_settle<8>(f[0], f[1]); break;
        }
      };
      static_assert(kSAhead <= 4, "lgkmcnt range of the settle switch");
      bf16x8 fr[kSAhead + 1][2];
#pragma unroll
      for (int i = 0; i < kSAhead; ++i) issue(i, fr[i]);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        if (ks + kSAhead < NK) issue(ks + kSAhead, fr[(ks + kSAhead) % (kSAhead + 1)]);
        settle(fr[ks % (kSAhead + 1)], min(kSAhead, NK - 1 - ks));
        __builtin_amdgcn_sched_barrier(0);
        sacc[0] = mfma16(fr[ks % (kSAhead + 1)][0], qf[ks], sacc[0]);
        sacc[1] = mfma16(fr[ks % (kSAhead + 1)][1], qf[ks], sacc[1]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) {  // this wave's loads of tile k + 2
          step_issue<NL>(a, pc, lds, j0, k, n, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // register v of block tb <-> token 16 tb + 4 kq + v, head h
    const int valid = a.len - (a.tile0 + k) * kTok;
    float hmax = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (16 * tb + 4 * (int)kq + v >= valid) sacc[tb][v] = -INFINITY;
        hmax = fmaxf(hmax, sacc[tb][v]);
      }
    hmax = max_xor32(max_xor16(hmax));
    const bool grow = hmax > m + kRescaleSlack;
    const float m_new = grow ? hmax : m;
    const float alpha = grow ? fast_exp2(m - m_new) : 1.0f;
    const bool any = __ballot(grow) != 0ull;
    const uint32_t pb = pw_base + (uint32_t)(k & 1) * (kMaxHG * kPStride * 2);
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      bf16x4 pk;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bf16 p = (bf16)fast_exp2(sacc[tb][v] - m_new);
        pk[v] = p;
        psum += (float)p;
      }
      lds_st(pb + tb * 32, pk);
    }
    l = l * alpha + psum;
    m = m_new;
    if (lane < 16) lds_st(lds + kOffAlpha + ((k & 1) * kMaxHG + h) * 4, alpha);
    if (lane == 0) lds_st(lds + kOffFlag + ((k & 1) * 4 + sw) * 4, any ? 1.0f : 0.0f);
  }
  l = sum_xor32(sum_xor16(l));
  m_out = m;
  l_out = l;
}

// P*C wave `pw` (columns 128 pw .. 128 pw + 127 of O, all HEADS heads),
// accumulated transposed: register v of o[hb][cb] holds column
// 128 pw + 32 cb + 8 (v/4) + 4 (lane/32) + v%4 of head 32 hb + lane%32, so a
// lane owns one head per hb (one rescale factor) and runs of 4 columns.
template <int HEADS>
struct OAcc {
  f32x16 o[Geo<HEADS>::HB][4];
};

template <int HEADS, int SL>
__device__ __forceinline__ void pv_role(const SegArgs& a, uint32_t lds, int pw, int lane,
                                        OAcc<HEADS>& acc) {
  using G = Geo<HEADS>;
  const int n = a.tile1 - a.tile0;
  constexpr int NL = tile_loads<false, SL>(false);
  const uint32_t j0 = first_load<false, SL>(4 + pw);
  PageCursor pc;
  seg_start<false, NL>(a, pc, lds, j0, lane);
  if (n > 1 && !a.tile1_issued)
    issue_tile<false, NL>(a, pc, a.tile0 + 1, load_slot<false>(lds, 1), j0, lane);
#pragma unroll
  for (int hb = 0; hb < G::HB; ++hb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc.o[hb][cb] = f32x16{};

  // Transposing reads: lane (16 g + li) of the fragment for token block ks
  // and column block cb reads row 16 ks + x + 4 hi, chunk 16 pw + 4 cb +
  // 2 (g%2) + b1, stored at 8 (2 pw + cb/2) + ((4 (cb%2) + 2 (g%2) + b1) ^ swz(row)),
  // plus 8 bytes for odd li (16 ks does not change swz).
  const uint32_t g = lane >> 4, li = lane & 15;
  const uint32_t x = 8u * (g >> 1) + (li >> 2), b1 = (li >> 1) & 1u;
  uint32_t tr_off[4][2];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const uint32_t cc = 4u * (cb & 1) + 2u * (g & 1) + b1;
      const uint32_t row = x + 4u * hi;
      tr_off[cb][hi] = (row * kCh + 8u * (2u * pw + (cb >> 1)) + (cc ^ swz(row))) * 16u +
                       8u * (li & 1);
    }
  // P fragments (B operand of 32x32x16): head 32 hb + lane%32, tokens 16 ks + 8 (lane/32)
  const uint32_t pa_base = lds + kOffP + ((lane & 31) * kPStride + 8 * (lane >> 5)) * 2;
  const uint32_t al_base = lds + kOffAlpha + (lane & 31) * 4;

  for (int k = 0; k <= n; ++k) {
    step_sync<NL>(a, pc, lds, j0, k, n, lane);
    step_issue<NL>(a, pc, lds, j0, k, n, lane);
    if (k == 0) continue;
    const int kp = k - 1;  // tile whose P is ready
    const uint32_t buf = load_slot<false>(lds, kp);
    const uint32_t par = (uint32_t)(kp & 1);
    const f32x4 f = lds_ld4(lds + kOffFlag + par * 16);
    float fs = f[0] + f[1];
    if (G::SW > 2) fs += f[2] + f[3];
    if (fs != 0.0f) {
#pragma unroll
      for (int hb = 0; hb < G::HB; ++hb) {
        const float al = lds_ld(al_base + (par * kMaxHG + 32 * hb) * 4);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc.o[hb][cb][v] *= al;
      }
    }
    const uint32_t pbase = pa_base + par * (kMaxHG * kPStride * 2);
    uint32_t ta[8];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) ta[2 * cb + hi] = buf + tr_off[cb][hi];
#pragma unroll
    for (int ks = 0; ks < kTok / 16; ++ks) {
      bf16x8 pa[G::HB];
#pragma unroll
      for (int hb = 0; hb < G::HB; ++hb)
        pa[hb] = lds_read_b128(pbase + hb * 32 * kPStride * 2 + ks * 32);
      bf16x4 t[8];
      if (ks == 0)
        lds_read_tr_x8<0>(ta, t);
      else
        lds_read_tr_x8<16 * kCh * 16>(ta, t);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const bf16x8 bv = cat(t[2 * cb], t[2 * cb + 1]);
#pragma unroll
        for (int hb = 0; hb < G::HB; ++hb) acc.o[hb][cb] = mfma32(bv, pa[hb], acc.o[hb][cb]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 rows: the tile loop on the staged codes (see the FP8 section above).
// ---------------------------------------------------------------------------
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// LDS reads without a wait (completed by an lds_settle naming the registers).
template <int OFF>
__device__ __forceinline__ void ds_b64_nowait(u32x2& o, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(o) : "v"(a), "i"(OFF));
}
// Transposing 8-bit read: within each group of 16 lanes, output lane i byte j
// is byte i % 8 of the 8 bytes addressed by lane 2 j + i / 8 of the group.
template <int OFF>
__device__ __forceinline__ void ds_tr8_nowait(u32x2& o, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(o) : "v"(a), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_b32_nowait(float& o, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(o) : "v"(a), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_b128f_nowait(f32x4& o, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(o) : "v"(a), "i"(OFF));
}
// Eight E4M3 codes (byte j is element j) as bf16, without a scale (exact).
__device__ __forceinline__ bf16x8 widen8(const u32x2& c) {
  bf16x8 r;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[d], 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[d], 1.0f, true);
    r[4 * d + 0] = lo[0];
    r[4 * d + 1] = lo[1];
    r[4 * d + 2] = hi[0];
    r[4 * d + 3] = hi[1];
  }
  return r;
}

// Step-top synchronisation for FP8 rows.  A segment starts with tiles 0 and
// 1 in flight (seg_start, then the caller); step 0 waits for tile 0 and
// issues tiles 2 .. 4; step k > 0 waits for tile k (tiles k+1 .. k+3 may
// stay in flight) and issues tile k+4 into the slot tile k-2 left.
template <int NL>
__device__ __forceinline__ void step_sync_f8(const SegArgs& a, PageCursor& pc, uint32_t lds,
                                             uint32_t j0, int k, int n, int lane) {
  if (k < n) {
    const int ahead = min(n - 1 - k, k == 0 ? 1 : 3);  // tiles issued after tile k
    if (ahead >= 3)
      wait_vmcnt<3 * NL>();
    else if (ahead == 2)
      wait_vmcnt<2 * NL>();
    else if (ahead == 1)
      wait_vmcnt<NL>();
    else
      wait_vmcnt<0>();
  }
  asm volatile("" : "+v"(pc.cur), "+v"(pc.nxt));  // landed before the tile loads
  lds_barrier();
  auto tile = [&](int x) {
    if (x < n) issue_tile<true, NL>(a, pc, a.tile0 + x, load_slot<true>(lds, x), j0, lane);
  };
  if (k == 0) {
    tile(2);
    tile(3);
  }
  tile(k + 4);
}

// Query split for the FP8 score MFMAs: a bf16 value has 8 significant
// bits and an e4m3 code 4, so two e4m3 terms hold it (hi = e4m3(q / 2^e1),
// lo = e4m3((q - 2^e1 hi) / 2^e2), one power-of-two scale per head and
// term); what is left is below 2^-20 of the head's largest value.
typedef int v8i __attribute__((ext_vector_type(8)));
// smallest e with amax / 2^e <= 448 (exact: amax = m 2^E, m in [0.5, 1))
__device__ __forceinline__ int e4m3_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = frexpf(amax, &E);
  return max(-127, min(127, m <= 0.875f ? E - 9 : E - 8));
}
// e4m3 codes of a / s .. d / s (round to nearest even) in one dword
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d, float s) {
  typedef short __attribute__((ext_vector_type(2))) short2v;
  const short2v lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2v{0, 0}, a, b, s, false);
  const short2v pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c, d, s, true);
  return __builtin_bit_cast(int, pk);
}
// A score wave's queries in the form its FP8 MFMAs take: the latent part as
// hi and lo terms in the byte order of the code fragments (step kc, byte
// 8 i + j holds qf[4 kc + i][j]) with their E8M0 scale bytes eb1, eb2 (127 +
// e), the rope part as bf16.
struct QSplit {
  v8i qh[4], ql[4];
  bf16x8 qr[2];
  int eb1, eb2;
};
__device__ __forceinline__ void split_queries(bf16x8 (&qf)[kW / 32], QSplit& qs) {
  v8i(&qh)[4] = qs.qh;
  v8i(&ql)[4] = qs.ql;
  // Three passes over the 128 values; between them the inputs are handed on
  // through empty asm statements, so each pass converts its values again
  // instead of keeping all of them live in registers.
  auto launder = [&]() {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+v"(qf[ks]));
  };
  float amax = 0.f;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)qf[ks][j]));
  amax = max_xor32(max_xor16(amax));  // the head's four lanes
  const int e1 = e4m3_exp(amax);
  const float s1 = ldexpf(1.0f, e1);
  launder();
  float rmax = 0.f;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const bf16x8& q = qf[4 * kc + (d >> 1)];
      const int j = 4 * (d & 1);
      const float v0 = (float)q[j], v1 = (float)q[j + 1], v2 = (float)q[j + 2], v3 = (float)q[j + 3];
      qh[kc][d] = pack4_e4m3(v0, v1, v2, v3, s1);
      const auto f01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((unsigned)qh[kc][d], s1, false);
      const auto f23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((unsigned)qh[kc][d], s1, true);
      rmax = fmaxf(rmax, fmaxf(fmaxf(fabsf(v0 - f01[0]), fabsf(v1 - f01[1])),
                               fmaxf(fabsf(v2 - f23[0]), fabsf(v3 - f23[1]))));
    }
  rmax = max_xor32(max_xor16(rmax));
  const int e2 = e4m3_exp(rmax);
  const float s2 = ldexpf(1.0f, e2);
  launder();
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) asm volatile("" : "+v"(qh[kc]));
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const bf16x8& q = qf[4 * kc + (d >> 1)];
      const int j = 4 * (d & 1);
      const auto f01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((unsigned)qh[kc][d], s1, false);
      const auto f23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((unsigned)qh[kc][d], s1, true);
      ql[kc][d] = pack4_e4m3((float)q[j] - f01[0], (float)q[j + 1] - f01[1],
                             (float)q[j + 2] - f23[0], (float)q[j + 3] - f23[1], s2);
    }
  qs.eb1 = 127 + e1;
  qs.eb2 = 127 + e2;
  qs.qr[0] = qf[16];
  qs.qr[1] = qf[17];
}
// Waits until at most N LDS operations of this wave are outstanding and
// hands the four named registers on as written here.
template <int N>
__device__ __forceinline__ void lds_settle4(u32x2& a, u32x2& b, u32x2& c, u32x2& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}
__device__ __forceinline__ v8i cat4(const u32x2& a, const u32x2& b, const u32x2& c,
                                    const u32x2& d) {
  return v8i{(int)a[0], (int)a[1], (int)b[0], (int)b[1], (int)c[0], (int)c[1], (int)d[0], (int)d[1]};
}
// 16x16x128 e4m3 MFMA with E8M0 scales (the A scale of row r is taken from
// the lanes holding row r, the B scale of column n from the lanes holding
// column n; each is the same in all four of them here, so how the blocks of
// 32 map to lanes does not matter).  Same accumulator layout as mfma16.
__device__ __forceinline__ f32x4 mfma_f8(const v8i& a, const v8i& b, const f32x4& c, int sa,
                                         int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Score wave `sw` on FP8 rows: the codes of the 512 latent columns go into
// e4m3 MFMAs as they are, with the row's scale as the A scale and the
// split queries (hi and lo terms) as B: s = scale (q_lat . code) + q_rope .
// k_rope in one accumulator (the rope steps are bf16 MFMAs).  A fragment
// (step kc, tb): row t = lane%16 + 16 tb, codes 128 kc + 32 i + 8 kq .. +7
// for i = 0 .. 3 (four 8-byte reads, the byte order of the split queries).
template <int HEADS>
__device__ __forceinline__ void score_role_f8(const SegArgs& a, uint32_t lds, int sw, int lane,
                                              float& m_out, float& l_out) {
  using G = Geo<HEADS>;
  const bool active = sw < G::SW;
  const int n = a.tile1 - a.tile0;
  constexpr int NL = kF8Loads;
  const uint32_t j0 = first_load<true>(sw);
  PageCursor pc;
  seg_start<true, NL>(a, pc, lds, j0, lane);
  const int h = 16 * sw + (lane & 15);
  const uint32_t kq = lane >> 4;
  // this segment's queries (bf16), split once they land
  bf16x8 qt[kW / 32];
  if (active) load_queries(a.q_rows, sw, lane, qt);
  // tile 0 and the queries land; tile 1 may stay in flight
  if (n > 1) {
    if (!a.tile1_issued) issue_tile<true, NL>(a, pc, a.tile0 + 1, load_slot<true>(lds, 1), j0, lane);
    wait_vmcnt<NL>();
  } else {
    wait_vmcnt<0>();
  }
  QSplit qs;
  if (active) {
#pragma unroll
    for (int ks = 0; ks < kW / 32; ++ks) asm volatile("" : "+v"(qt[ks]));
    split_queries(qt, qs);
  }

  // Code reads of step ks (i = ks % 4 of group kc = ks / 4): chunk 2 ks +
  // kq/2 of row t (position by s8(t); s8(t + 16) = s8(t)), half kq%2.  Rope
  // steps r = 0, 1: bf16 chunk 32 + 4 r + kq.
  const uint32_t t0 = lane & 15, sx = s8(t0);
  uint32_t lat_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    lat_off[i] = t0 * kF8RowBytes + (((2u * i + (kq >> 1)) ^ sx) * 16u) + 8u * (kq & 1u);
  uint32_t rope_off[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) rope_off[r] = t0 * kF8RowBytes + (32u + ((4u * r + kq) ^ sx)) * 16u;
  const uint32_t sc_off = kF8ScaleOff + 64u * kq;   // scale chunk of token 4 kq
  const uint32_t rs_off = kF8ScaleOff + 16u * t0;   // scale chunk of row t0
  const uint32_t pw_base = lds + kOffP + (h * kPStride + 4 * kq) * 2;
  constexpr uint32_t kTb = 16 * kF8RowBytes;        // rows 16 .. 31

  float m = -INFINITY, l = 0.f;
  for (int k = 0; k <= n; ++k) {
    step_sync_f8<NL>(a, pc, lds, j0, k, n, lane);
    if (k == n || !active) continue;
    const uint32_t stg = load_slot<true>(lds, k);
    // the hi terms (with the rope steps) and the lo terms accumulate apart:
    // four independent MFMA chains instead of two
    f32x4 sacc[2] = {f32x4{}, f32x4{}}, slo[2] = {f32x4{}, f32x4{}};
    // scales of tokens 16 tb + 4 kq + v (for P), of rows t0 and t0 + 16
    // (the A scales) and the rope fragments, read first (LDS reads complete
    // in order)
    float sc[2][4], rs[2];
    bf16x8 rope[2][2];
    {
      const uint32_t sa = stg + sc_off;
      ds_b32_nowait<0>(sc[0][0], sa);
      ds_b32_nowait<16>(sc[0][1], sa);
      ds_b32_nowait<32>(sc[0][2], sa);
      ds_b32_nowait<48>(sc[0][3], sa);
      ds_b32_nowait<256>(sc[1][0], sa);
      ds_b32_nowait<272>(sc[1][1], sa);
      ds_b32_nowait<288>(sc[1][2], sa);
      ds_b32_nowait<304>(sc[1][3], sa);
      ds_b32_nowait<0>(rs[0], stg + rs_off);
      ds_b32_nowait<256>(rs[1], stg + rs_off);
      ds_b128_nowait<0>(rope[0][0], stg + rope_off[0]);
      ds_b128_nowait<kTb>(rope[0][1], stg + rope_off[0]);
      ds_b128_nowait<0>(rope[1][0], stg + rope_off[1]);
      ds_b128_nowait<kTb>(rope[1][1], stg + rope_off[1]);
    }
    {
      // groups g = 0 .. 7 (kc = g / 2, tb = g % 2) of four 8-byte reads,
      // one group ahead of its MFMAs
      constexpr int NG = 8, A = 1;
      u32x2 grp[A + 1][4];
      auto issue = [&](int g) {
        const uint32_t ad = stg + 128u * (uint32_t)(g >> 1);
        u32x2(&f)[4] = grp[g % (A + 1)];
        if (g & 1) {
          ds_b64_nowait<kTb>(f[0], ad + lat_off[0]);
          ds_b64_nowait<kTb>(f[1], ad + lat_off[1]);
          ds_b64_nowait<kTb>(f[2], ad + lat_off[2]);
          ds_b64_nowait<kTb>(f[3], ad + lat_off[3]);
        } else {
          ds_b64_nowait<0>(f[0], ad + lat_off[0]);
          ds_b64_nowait<0>(f[1], ad + lat_off[1]);
          ds_b64_nowait<0>(f[2], ad + lat_off[2]);
          ds_b64_nowait<0>(f[3], ad + lat_off[3]);
        }
      };
#pragma unroll
      for (int g = 0; g < A; ++g) issue(g);
      // the scales and rope fragments (issued first) have landed once at
      // most 4 A reads remain
      asm volatile("s_waitcnt lgkmcnt(%14)"
                   : "+v"(sc[0][0]), "+v"(sc[0][1]), "+v"(sc[0][2]), "+v"(sc[0][3]),
                     "+v"(sc[1][0]), "+v"(sc[1][1]), "+v"(sc[1][2]), "+v"(sc[1][3]), "+v"(rs[0]),
                     "+v"(rs[1]), "+v"(rope[0][0]), "+v"(rope[0][1]), "+v"(rope[1][0]),
                     "+v"(rope[1][1])
                   : "i"(4 * A));
      // E8M0 bytes of the row scales (a power of two: its exponent field)
      const int rb0 = (int)((__builtin_bit_cast(unsigned, rs[0]) >> 23) & 255u);
      const int rb1 = (int)((__builtin_bit_cast(unsigned, rs[1]) >> 23) & 255u);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        sacc[0] = mfma16(rope[r][0], qs.qr[r], sacc[0]);
        sacc[1] = mfma16(rope[r][1], qs.qr[r], sacc[1]);
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + A < NG) issue(g + A);
        u32x2(&f)[4] = grp[g % (A + 1)];
        if (g + 1 < NG)
          lds_settle4<4 * A>(f[0], f[1], f[2], f[3]);
        else
          lds_settle4<0>(f[0], f[1], f[2], f[3]);
        const v8i av = cat4(f[0], f[1], f[2], f[3]);
        const int tb = g & 1, kc = g >> 1;
        sacc[tb] = mfma_f8(av, qs.qh[kc], sacc[tb], tb ? rb1 : rb0, qs.eb1);
        slo[tb] = mfma_f8(av, qs.ql[kc], slo[tb], tb ? rb1 : rb0, qs.eb2);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) sacc[tb] += slo[tb];
    // register v of block tb <-> token 16 tb + 4 kq + v, head h
    const int valid = a.len - (a.tile0 + k) * kTok;
    float hmax = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (16 * tb + 4 * (int)kq + v >= valid) sacc[tb][v] = -INFINITY;
        hmax = fmaxf(hmax, sacc[tb][v]);
      }
    hmax = max_xor32(max_xor16(hmax));
    const bool grow = hmax > m + kRescaleSlack;
    const float m_new = grow ? hmax : m;
    const float alpha = grow ? fast_exp2(m - m_new) : 1.0f;
    const bool any = __ballot(grow) != 0ull;
    const uint32_t pb = pw_base + (uint32_t)(k & 1) * (kMaxHG * kPStride * 2);
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      bf16x4 pk;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bf16 p = (bf16)fast_exp2(sacc[tb][v] - m_new);
        psum += (float)p;
        pk[v] = (bf16)((float)p * sc[tb][v]);  // exact: a power-of-two scale
      }
      lds_st(pb + tb * 32, pk);
    }
    l = l * alpha + psum;
    m = m_new;
    if (lane < 16) lds_st(lds + kOffAlpha + ((k & 1) * kMaxHG + h) * 4, alpha);
    if (lane == 0) lds_st(lds + kOffFlag + ((k & 1) * 4 + sw) * 4, any ? 1.0f : 0.0f);
  }
  l = sum_xor32(sum_xor16(l));
  m_out = m;
  l_out = l;
}

// P*C wave `pw` on FP8 rows: as pv_role, with the A fragments (32 columns x
// 16 tokens) read from the codes by one transposing 8-bit read each and
// widened in registers; P carries the row scales.
template <int HEADS>
__device__ __forceinline__ void pv_role_f8(const SegArgs& a, uint32_t lds, int pw, int lane,
                                           OAcc<HEADS>& acc) {
  using G = Geo<HEADS>;
  const int n = a.tile1 - a.tile0;
  constexpr int NL = kF8Loads;
  const uint32_t j0 = first_load<true>(4 + pw);
  PageCursor pc;
  seg_start<true, NL>(a, pc, lds, j0, lane);
  if (n > 1 && !a.tile1_issued)
    issue_tile<true, NL>(a, pc, a.tile0 + 1, load_slot<true>(lds, 1), j0, lane);
#pragma unroll
  for (int hb = 0; hb < G::HB; ++hb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc.o[hb][cb] = f32x16{};

  // Group g4 = lane/16 of the fragment for (ks, cb) holds columns 128 pw +
  // 32 cb + 16 (g4 % 2) + 0..15 of tokens 16 ks + 8 (g4 / 2) + 0..7; lane li
  // of the group addresses row 16 ks + 8 (g4 / 2) + li / 2, chunk 8 pw + 2 cb
  // + g4 % 2, half li % 2 (s8 of the row does not depend on ks).
  const uint32_t g4 = lane >> 4, li = lane & 15;
  const uint32_t row = 8u * (g4 >> 1) + (li >> 1), sx = s8(row);
  uint32_t tr_off[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    tr_off[cb] = row * kF8RowBytes + (8u * pw + ((2u * cb + (g4 & 1u)) ^ sx)) * 16u + 8u * (li & 1u);
  constexpr uint32_t kKs = 16 * kF8RowBytes;  // tokens 16 .. 31
  // P fragments (B operand of 32x32x16): head 32 hb + lane%32, tokens 16 ks + 8 (lane/32)
  const uint32_t pa_base = lds + kOffP + ((lane & 31) * kPStride + 8 * (lane >> 5)) * 2;
  const uint32_t al_base = lds + kOffAlpha + (lane & 31) * 4;
  constexpr uint32_t kPHb = 32 * kPStride * 2;  // next 32 heads of P

  for (int k = 0; k <= n; ++k) {
    step_sync_f8<NL>(a, pc, lds, j0, k, n, lane);
    if (k == 0) continue;
    const int kp = k - 1;  // tile whose P is ready
    const uint32_t stg = load_slot<true>(lds, kp);
    const uint32_t par = (uint32_t)(kp & 1);
    const uint32_t pbase = pa_base + par * (kMaxHG * kPStride * 2);
    f32x4 f;
    ds_b128f_nowait<0>(f, lds + kOffFlag + par * 16);
    float al[G::HB];
#pragma unroll
    for (int hb = 0; hb < G::HB; ++hb) ds_b32_nowait<0>(al[hb], al_base + (par * kMaxHG + 32 * hb) * 4);
    // both token blocks' reads: P (HB) and codes (4) of ks 0, then of ks 1
    bf16x8 pa[2][G::HB];
    u32x2 cr[2][4];
#pragma unroll
    for (int hb = 0; hb < G::HB; ++hb) ds_b128_nowait<0>(pa[0][hb], pbase + hb * kPHb);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) ds_tr8_nowait<0>(cr[0][cb], stg + tr_off[cb]);
#pragma unroll
    for (int hb = 0; hb < G::HB; ++hb) ds_b128_nowait<32>(pa[1][hb], pbase + hb * kPHb);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) ds_tr8_nowait<kKs>(cr[1][cb], stg + tr_off[cb]);
    // flags and factors (issued first) have landed once the 2 (HB + 4) reads remain
    constexpr int kLater = 2 * (G::HB + 4);
    if constexpr (G::HB == 2)
      asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(f), "+v"(al[0]), "+v"(al[1]) : "i"(kLater));
    else
      asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(f), "+v"(al[0]) : "i"(kLater));
    float fs = f[0] + f[1];
    if (G::SW > 2) fs += f[2] + f[3];
    if (fs != 0.0f) {
#pragma unroll
      for (int hb = 0; hb < G::HB; ++hb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc.o[hb][cb][v] *= al[hb];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks == 0) {
        if constexpr (G::HB == 2)
          asm volatile("s_waitcnt lgkmcnt(%6)"
                       : "+v"(pa[0][0]), "+v"(pa[0][1]), "+v"(cr[0][0]), "+v"(cr[0][1]),
                         "+v"(cr[0][2]), "+v"(cr[0][3])
                       : "i"(G::HB + 4));
        else
          asm volatile("s_waitcnt lgkmcnt(%5)"
                       : "+v"(pa[0][0]), "+v"(cr[0][0]), "+v"(cr[0][1]), "+v"(cr[0][2]),
                         "+v"(cr[0][3])
                       : "i"(G::HB + 4));
      } else {
        if constexpr (G::HB == 2)
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(pa[1][0]), "+v"(pa[1][1]), "+v"(cr[1][0]), "+v"(cr[1][1]),
                         "+v"(cr[1][2]), "+v"(cr[1][3]));
        else
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(pa[1][0]), "+v"(cr[1][0]), "+v"(cr[1][1]), "+v"(cr[1][2]),
                         "+v"(cr[1][3]));
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const bf16x8 bv = widen8(cr[ks][cb]);
#pragma unroll
        for (int hb = 0; hb < G::HB; ++hb) acc.o[hb][cb] = mfma32(bv, pa[ks][hb], acc.o[hb][cb]);
      }
    }
  }
}

// A whole segment plus its normalised output, in two halves by wave role
// (with the same barriers): score waves publish 1/l per head, P*C waves
// stage O/l in LDS (the tile buffers, idle by then), then all waves copy it
// out with 16-byte stores (copy_out).  m and the sum come back in lanes
// 0..15 of the active score waves (for the split statistics).  Ends with a
// barrier, so the next segment may refill the buffers.
template <int HEADS>
__device__ __forceinline__ void copy_out(uint32_t lds, bf16* dst) {
#pragma unroll
  for (int i0 = 0; i0 < HEADS * kR / 8; i0 += kThreads) {
    const int i = i0 + (int)threadIdx.x;
    const int hh = i / (kR / 8), c8 = (i % (kR / 8)) * 8;
    __builtin_nontemporal_store(lds_read_b128(lds + (hh * kOStride + c8) * 2),
                                (bf16x8*)(dst + hh * kR + c8));
  }
  lds_barrier();
}

template <int HEADS, bool kFp8, int SL>
__device__ __forceinline__ void score_segment(const SegArgs& a, uint32_t lds, bf16* dst, int wave,
                                              int lane, bf16x8 (&qf)[kW / 32], bool q_ready,
                                              float& m_out, float& l_out) {
  using G = Geo<HEADS>;
  if constexpr (kFp8)
    score_role_f8<HEADS>(a, lds, wave, lane, m_out, l_out);
  else
    score_role<HEADS, SL>(a, lds, wave, lane, qf, q_ready, m_out, l_out);
  if (wave < G::SW && lane < 16) lds_st(lds + kOffInv + (16 * wave + lane) * 4, 1.0f / l_out);
  lds_barrier();
  lds_barrier();
  copy_out<HEADS>(lds, dst);
}

template <int HEADS, bool kFp8, int SL>
__device__ __forceinline__ void pv_segment(const SegArgs& a, uint32_t lds, bf16* dst, int wave,
                                           int lane) {
  using G = Geo<HEADS>;
  const int pw = wave - 4;
  OAcc<HEADS> acc;
  if constexpr (kFp8)
    pv_role_f8<HEADS>(a, lds, pw, lane, acc);
  else
    pv_role<HEADS, SL>(a, lds, pw, lane, acc);
  lds_barrier();
  // lane: head 32 hb + lane%32; register v of o[hb][cb]: column
  // 128 pw + 32 cb + 8 (v/4) + 4 (lane/32) + v%4 (runs of 4 -> 8-byte stores)
#pragma unroll
  for (int hb = 0; hb < G::HB; ++hb) {
    const int head = 32 * hb + (lane & 31);
    const float inv = lds_ld(lds + kOffInv + head * 4);
    const uint32_t row = lds + (head * kOStride + 128 * pw + 4 * (lane >> 5)) * 2;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 w4;
#pragma unroll
        for (int r = 0; r < 4; ++r) w4[r] = (bf16)(acc.o[hb][cb][4 * q + r] * inv);
        lds_st(row + (32 * cb + 8 * q) * 2, w4);
      }
  }
  lds_barrier();
  copy_out<HEADS>(lds, dst);
}

// Workgroup -> (head group, stream index).  Blocks go round-robin over the
// 8 XCDs, so block b runs on XCD b % 8; each XCD gets a contiguous run of
// stream indices (consecutive pieces of the same sequences share its
// queries in that XCD's L2), and the head groups of one stream index sit 8
// blocks apart on the same XCD (the second group reads each tile from L2).
// n_wg is a multiple of 8.
__device__ __forceinline__ void map_block(int b, int hgc, int n_wg, int& hg, int& w) {
  const int x = b & 7, j = b >> 3;
  hg = j % hgc;
  w = x * (n_wg >> 3) + j / hgc;
}

// Equal shares of a stream of T tiles over n workgroups: workgroup w owns
// [start(w), start(w + 1)), start(w) = floor(w T / n).  With T = q n + r
// that is w q + floor(w r / n), which stays in 32 bits (T < 2^31, and
// w r < n^2); a 64-bit division would cost hundreds of instructions.
struct StreamSplit {
  int n, q, r;
  __device__ __forceinline__ StreamSplit(int T, int n_) : n(n_), q(T / n_), r(T % n_) {}
  __device__ __forceinline__ int start(int w) const { return w * q + (w * r) / n; }
  // Whether workgroup w's range holds a tile (all do once T >= n).
  __device__ __forceinline__ bool nonempty(int w) const {
    return q > 0 || ((w + 1) * r) / n > (w * r) / n;
  }
  // The workgroup whose range holds tile x (0 <= x < T): a float estimate
  // of x n / T, then exact corrections.
  __device__ __forceinline__ int owner(int x) const {
    const float T = (float)q * (float)n + (float)r;
    int w = min(n - 1, (int)((float)x * (float)n / T));
    while (w + 1 < n && start(w + 1) <= x) ++w;
    while (w > 0 && start(w) > x) --w;
    return w;
  }
};

// Prefix sums of tiles per sequence into LDS prefix[0..batch] (2 sequences
// per thread, then a scan); optionally (len - 1) % kTok per sequence into
// lenlo, so a length needs no further global read.  All kThreads threads
// call it; ends with a barrier.  `issued` runs once the length loads are in
// flight and before they are waited for.  `early` runs once the lengths have
// landed and before the scan: loads it issues overlap the rest (the barriers
// here are LDS-only, so they do not wait for them).
template <typename Issued, typename Early>
__device__ __forceinline__ void tile_prefix(const int* __restrict__ seq_lens, int batch,
                                            int* prefix, int* scan, unsigned char* lenlo,
                                            Issued&& issued, Early&& early) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int lens[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) lens[i] = tid * 2 + i < batch ? seq_lens[tid * 2 + i] : 0;
  issued();
  // the lengths are plain values from here on: no wait below is tied to them
  asm volatile("" : "+v"(lens[0]), "+v"(lens[1]));
  early();
  int cnt[2], tot = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = tid * 2 + i;
    const int len = lens[i];
    cnt[i] = len > 0 ? (len + kTok - 1) / kTok : 0;
    if (lenlo && b < batch) lenlo[b] = (unsigned char)((len - 1) & (kTok - 1));
    tot += cnt[i];
  }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) scan[wave] = incl;
  lds_barrier();
  int base = 0;
  for (int i = 0; i < wave; ++i) base += scan[i];
  int run = base + incl - tot;
  if (tid == 0) prefix[0] = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = tid * 2 + i;
    if (b < batch) {
      run += cnt[i];
      prefix[b + 1] = run;
    }
  }
  lds_barrier();
}

// One decode workgroup of the tile stream (block `blk`): every (workgroup,
// sequence) piece writes one partial into slot w + b (unique: w + b grows
// along the stream).  Returns whether this workgroup wrote any piece.
template <int HEADS, bool kFp8, int SL>
__device__ __forceinline__ bool decode_attention_wg(
    char* smem, int blk, const int* __restrict__ seq_lens, const int* __restrict__ block_table,
    const bf16* __restrict__ pool, int H, int n_wg, int batch, int guess_tiles, int max_blocks,
    int shift, int num_blocks, const bf16* __restrict__ q_full, int* __restrict__ prefix_out,
    float* __restrict__ part_ml, bf16* __restrict__ part_o) {
  const uint32_t lds = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hgc = H / HEADS;
  int hg, w;
  map_block(blk, hgc, n_wg, hg, w);
  int* prefix = (int*)(smem + kOffPrefix);
  unsigned char* lenlo = (unsigned char*)(smem + kOffLenLo);

  // Where this workgroup's range would start if every sequence had
  // guess_tiles tiles (the common equal-length batch): load that page-id
  // chunk now, in parallel with the lengths, and keep it if the guess holds.
  // As soon as the ids land, the guessed first tile (as a full tile) goes in
  // flight into buffer 0, then the guessed sequence's queries (score waves,
  // staged in LDS), then the guessed second tile into buffer 1, overlapping
  // the prefix sums and the range search; a page id outside the pool is never
  // dereferenced.  (Issuing a third tile here measured slower: the opening
  // burst delays every workgroup's first tiles.)
  const StreamSplit gsplit(batch * guess_tiles, n_wg);
  const int xg = gsplit.start(w);
  const int bg = min(xg / guess_tiles, batch - 1);
  const int tg0 = xg - bg * guess_tiles;
  const int pg0 = (tg0 * kTok) >> shift;
  PageCursor spec;
  spec.start(block_table + (long)bg * max_blocks, max_blocks, pg0, lane);
  bf16x8 qf[kW / 32];  // score waves: the queries of sequence qb
  int qb = -1;
  bool spec_issued = false, spec2 = false;
  bool q_spec = false;  // queries of sequence qb staged in LDS before the range was known
  // guessed tile tg0 + t (as a full tile) into buffer t; false if its page
  // id is outside the pool (then nothing is issued)
  auto spec_tile = [&](int t) {
    const int tok = (tg0 + t) * kTok;
    const int page = spec.page(tok >> shift, lane);  // page index pg0 or pg0 + 1
    if (page < 0 || page >= num_blocks) return false;
    const long row = (long)page * (1 << shift) + (tok & ((1 << shift) - 1));
    if constexpr (kFp8)
      issue_part_fp8((const unsigned char*)pool + row * kF8Row, kTok, load_slot<true>(lds, t),
                     first_load<true>(wave), lane);
    else if (wave < 4)
      issue_part<SL>(pool + row * kW, kTok, load_slot<false>(lds, t), first_load<false, SL>(wave),
                          lane);
    else
      issue_part<p_loads<SL>()>(pool + row * kW, kTok, load_slot<false>(lds, t),
                                first_load<false, SL>(wave),
                          lane);
    return true;
  };
  auto early = [&]() {
    spec_issued = spec_tile(0);
    if (!kFp8 && wave < Geo<HEADS>::SW) {  // FP8: each segment loads and splits its own
      stage_queries(q_full + ((long)bg * H + hg * HEADS) * kW, wave, lane, lds);
      qb = bg;
      q_spec = true;
    }
    if (spec_issued && tg0 + 1 < guess_tiles) spec2 = spec_tile(1);
  };

  // The arguments past the ones the hardware preloads into scalar registers
  // are scalar loads from the argument segment, which the compiler would
  // issue and wait for where first used (the queries, the epilogue): fetched
  // here, their round trip overlaps that of the lengths and page ids.
  auto issued = [&]() {
    fetch_arg(q_full);
    fetch_arg(prefix_out);
    fetch_arg(part_ml);
    fetch_arg(part_o);
  };
  tile_prefix(seq_lens, batch, prefix, (int*)(smem + kOffScan), lenlo, issued, early);
  const int T = prefix[batch];
  if (blk == 0)
    for (int b = tid; b <= batch; b += kThreads) prefix_out[b] = prefix[b];

  const StreamSplit split(T, n_wg);
  const int x0 = split.start(w);
  const int x1 = split.start(w + 1);
  if (x0 >= x1) {
    wait_vmcnt<0>();  // no load may land in LDS after the exit
    return false;
  }
  // first sequence touching x0
  int b0 = 0;
  {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= x0) lo = mid; else hi = mid - 1;
    }
    b0 = lo;
  }
  const long n_slots = (long)n_wg + batch;
  // The segments of [x0, x1), one per sequence, in order; both wave roles
  // walk them with the same barriers (the roles are split at the top, so
  // the score waves' queries and the P*C waves' accumulators never share
  // registers).
  auto walk = [&](auto&& segment) {
    int x = x0, b = b0;
    while (x < x1) {
      const int p0 = prefix[b], p1 = prefix[b + 1];
      const int seg_end = min(x1, p1);
      const int tile0 = x - p0, tile1 = seg_end - p0;
      if (tile1 <= tile0) {  // a sequence without rows (invalid input): nothing to attend
        ++b;
        continue;
      }
      const int len = (p1 - p0 - 1) * kTok + lenlo[b] + 1;
      const long slot = (long)hg * n_slots + w + b;
      const bool guessed = b == bg && ((tile0 * kTok) >> shift) == pg0;
      // the speculative tile is this segment's tile 0 only if it is the same
      // tile and a full one (a partial tile repeats its last row instead)
      const bool reuse = spec_issued && guessed && tile0 == tg0 && (tile0 + 1) * kTok <= len;
      const bool reuse2 = reuse && spec2 && tile1 - tile0 >= 2 && (tile0 + 2) * kTok <= len;
      // speculative loads (tiles, staged queries) not taken over land before
      // their buffers are refilled
      if ((spec_issued || q_spec) && !(reuse && (reuse2 || !spec2))) wait_vmcnt<0>();
      const SegArgs a{q_full + ((long)b * H + hg * HEADS) * kW, pool,
                      block_table + (long)b * max_blocks, max_blocks, shift, len, tile0, tile1,
                      guessed ? &spec : nullptr, reuse, reuse2};
      spec_issued = spec2 = q_spec = false;
      segment(a, b, slot);
      x = seg_end;
      ++b;
    }
  };
  if (wave < 4) {
    walk([&](const SegArgs& a, int b, long slot) {
      float m, tot;
      score_segment<HEADS, kFp8, SL>(a, lds, part_o + slot * HEADS * kR, wave, lane, qf, qb == b, m,
                                 tot);
      qb = b;
      if (wave < Geo<HEADS>::SW && lane < 16) {
        const int h = 16 * wave + lane;
        const f32x2 ml = {m, tot};
        __builtin_nontemporal_store(ml, (f32x2*)(part_ml + (slot * HEADS + h) * 2));
      }
    });
  } else {
    walk([&](const SegArgs& a, int, long slot) {
      pv_segment<HEADS, kFp8, SL>(a, lds, part_o + slot * HEADS * kR, wave, lane);
    });
  }
  if (spec_issued || q_spec) wait_vmcnt<0>();
  return true;
}

// ---------------------------------------------------------------------------
// Combine (+ optional W_UV projection): one workgroup per (head, S
// consecutive sequences), 8 waves; lane l holds columns 8 l .. 8 l + 7 of a
// row of o_lat.
//   o_lat[b, h] = sum_s e_s O_s / sum_s e_s,  e_s = 2^(m_s - M) l_s.
// S is picked on the host so that the grid fills the CUs once (8 at 32
// sequences x 64 heads, 1 at 4 long sequences, 32 at 64 sequences x 128
// heads): with S < 8, 8/S waves share a sequence, each taking every
// (8/S)-th piece, and their partial sums meet in LDS; with S > 8 a wave
// merges S/8 sequences in turn.  Every wave computes all of its sequence's
// weights (one statistics load per 64 pieces), so partial sums share one
// reference max and add without rescaling, in a fixed order.
// The first pieces of a wave's first sequence are fetched at the slots they
// have in the equal-length layout (guessed from max_seq_len) before the
// prefix sums (scalar loads) arrive, and reloaded only when the real layout
// differs.  W_UV[h] (128 KB) streams into LDS with direct-to-LDS loads
// issued between the statistics and the piece values (it takes no
// registers): the step is bound by the bytes it moves, so the values land
// last whatever the order, and W_UV issued first is in LDS when the merged
// rows are, instead of trailing them.  A piece is read only if its workgroup's range is non-empty
// (with fewer tiles than workgroups some write nothing), so stale workspace
// contents never enter the merge.
// ---------------------------------------------------------------------------
constexpr int kCWaves = 8;
constexpr int kCThreads = 64 * kCWaves;
constexpr int kCMaxRows = 32;                  // sequences per workgroup, at most
constexpr int kCOBytes = kCMaxRows * kR * 2;   // o_lat rows (partial sums at +16 KB when S < 8)
constexpr int kCWBytes = kR * 128 * 2;         // W_UV[h] (Dv <= 128)
constexpr int kCWLoads = kCWBytes / (kCThreads * 16);
static_assert(kCWBytes + kCOBytes <= 163840, "LDS budget");

// W_UV[h] in LDS: rows of 16 chunks (256 B, Dv <= 128), chunk c of row r at
// position c ^ 2((r % 4) + 4 ((r / 8) % 2)), so the 8 rows (r0 .. r0+3 and
// r0+8 .. r0+11) x 2 chunks that 32 lanes of a transposing read touch fall
// on 16 distinct bank slots.
__device__ __forceinline__ uint32_t w_swz(uint32_t r) { return ((r & 3u) | ((r >> 1) & 4u)) << 1; }
__device__ __forceinline__ uint32_t w_off(uint32_t r, uint32_t c) {
  return (r * 16u + (c ^ w_swz(r))) * 16u;
}
// o_lat rows in LDS: 1 KB each, 16-byte chunk c of row r at position
// c ^ (r % 16), so the 16 rows of a fragment read hit distinct bank groups.
__device__ __forceinline__ uint32_t o_off(uint32_t r, uint32_t c) {
  return (r * (kR / 8) + (c ^ (r & 15u))) * 16u;
}

// Direct-to-LDS loads of W_UV[h]: instruction j of the workgroup fills slots
// 64 j .. 64 j + 63, slot s holding row s/16, the chunk w_off puts at s%16;
// chunks past Dv/8 load the row's chunk 0 (never read).
__device__ __forceinline__ void issue_w_uv(const bf16* W, int Dv, uint32_t wb, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kCWLoads; ++i) {
    const uint32_t j = (uint32_t)wave * kCWLoads + i;
    const uint32_t s = 64u * j + (uint32_t)lane, r = s >> 4;
    uint32_t c = (s & 15u) ^ w_swz(r);
    if ((int)c >= Dv / 8) c = 0;
    g2lds16(W + (long)r * Dv + c * 8, wb + j * 1024u);
  }
}

// The pieces of one sequence: workgroups f .. f+n-1 of the stream, slot
// slot0 + s for piece s.
struct SeqPieces {
  long slot0;
  int f, n;
};

// kChunk (8 or 16): piece values a wave has in flight at once; 16 also
// brings the statistics of pieces 64..127 with the first chunk.
template <bool kProject, int kChunk>
__device__ __forceinline__ void combine_wg(const int* prefix, const float* __restrict__ part_ml,
                                           const bf16* __restrict__ part_o, int batch, int H,
                                           int hg_heads, int n_wg, int guess_tiles, int S,
                                           const bf16* __restrict__ w_uv, int Dv,
                                           bf16* __restrict__ out, int h, int b0, uint32_t wb,
                                           uint32_t ob) {
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4v;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index as a wave-uniform value: the prefix sums then come
  // through scalar loads, whose waits do not hold up the vector loads
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = h / hg_heads, hl = h % hg_heads;
  const long n_slots = (long)n_wg + batch;
  const int wps = S < kCWaves ? kCWaves / S : 1;  // waves per sequence
  const int spw = S > kCWaves ? S / kCWaves : 1;  // sequences per wave
  const int part = wave % wps;                    // this wave's pieces: part + wps i
  const int row0 = S < kCWaves ? wave / wps : wave;

  auto ld_ml = [&](long slot0, int s) {
    return *(const f32x2*)(part_ml + ((slot0 + s) * hg_heads + hl) * 2);
  };
  auto ld_o = [&](long slot0, int s) {
    return *(const bf16x8*)(part_o + ((slot0 + s) * hg_heads + hl) * kR + 8 * lane);
  };
  // this wave's first chunk of a sequence: the statistics of pieces 0 ..
  // 64 kStats - 1 (kStats per lane) and the values of pieces part + wps u,
  // u < kChunk (below 64 kStats, as wps <= 8), indices clamped to the last
  // piece (what is not a piece is masked afterwards)
  constexpr int kStats = kChunk > 8 ? 2 : 1;
  constexpr int kStatPieces = 64 * kStats;
  bf16x8 v[kChunk];
  f32x2 ml_raw[kStats];
  auto first_stats = [&](const SeqPieces& q) {
    const int last = max(q.n, 1) - 1;
#pragma unroll
    for (int i = 0; i < kStats; ++i) ml_raw[i] = ld_ml(q.slot0, min(64 * i + lane, last));
  };
  auto first_values = [&](const SeqPieces& q) {
    const int last = max(q.n, 1) - 1;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) v[u] = ld_o(q.slot0, min(part + wps * u, last));
  };
  auto first_chunk = [&](const SeqPieces& q) {
    first_stats(q);
    first_values(q);
  };
  auto settle_first_chunk = [&]() {
    wait_vmcnt<0>();
#pragma unroll
    for (int i = 0; i < kStats; ++i) asm volatile("" : "+v"(ml_raw[i]));
#pragma unroll
    for (int u = 0; u < kChunk; ++u) asm volatile("" : "+v"(v[u]));
  };

  const int bw0 = b0 + row0;  // the wave's first sequence
  SeqPieces g{0, 0, 1};
  if (bw0 < batch) {
    const StreamSplit gsplit(batch * guess_tiles, n_wg);
    g.f = gsplit.owner(bw0 * guess_tiles);
    g.n = gsplit.owner((bw0 + 1) * guess_tiles - 1) - g.f + 1;
  }
  g.slot0 = (long)hg * n_slots + g.f + min(bw0, batch - 1);
  // statistics, then W_UV, then the piece values: the values arrive last in
  // any order (the bytes are bound by HBM), and W_UV is then in LDS by the
  // time the merged rows are
  first_stats(g);
  if constexpr (kProject) issue_w_uv(w_uv + (long)h * kR * Dv, Dv, wb, wave, lane);
  first_values(g);
  // The prefix sums are scalar loads, and a scalar load is waited for with
  // lgkmcnt(0) at its first use: hoisted above the loads just issued, they
  // would hold their issue back by a whole round trip.  The output pointer
  // (an argument past the preloaded ones) is fetched here too, not in the
  // epilogue.
  fetch_arg(out);
  asm volatile("" ::: "memory");

  // the first sequence's prefix sums load with the total (one round trip)
  const int T = prefix[batch];
  const int first_p0 = bw0 < batch ? prefix[bw0] : 0, first_p1 = bw0 < batch ? prefix[bw0 + 1] : 0;
  const StreamSplit split(T, n_wg);
  auto pieces = [&](int b) {
    SeqPieces q{0, 0, 0};
    const bool first = b == bw0;
    const int p0 = first ? first_p0 : b < batch ? prefix[b] : 0;
    const int p1 = first ? first_p1 : b < batch ? prefix[b + 1] : 0;
    if (p1 > p0) {
      q.f = split.owner(p0);
      q.n = split.owner(p1 - 1) - q.f + 1;
    }
    q.slot0 = (long)hg * n_slots + q.f + min(b, batch - 1);
    return q;
  };
  auto stat = [&](const SeqPieces& q, int s, f32x2 raw) {
    return s < q.n && split.nonempty(q.f + s) ? raw : f32x2{-INFINITY, 0.f};
  };

  for (int j = 0; j < spw; ++j) {
    const int row = row0 + kCWaves * j;
    const int b = b0 + row;
    const SeqPieces q = pieces(b);
    // A wrong guess (first sequence) or a later sequence: the first chunk
    // from the real slots, waited for here, so that on the common path the
    // compiler waits for each piece in turn, not for W_UV behind them.
    if (j > 0 || q.f != g.f || max(q.n, 1) != g.n) {
      first_chunk(q);
      settle_first_chunk();
    }
    const int n = q.n;
    f32x2 st[kStats];
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kStats; ++i) {
      st[i] = stat(q, 64 * i + lane, ml_raw[i]);
      M = fmaxf(M, st[i][0]);
    }
    for (int s = kStatPieces + lane; s < n; s += 64)  // long sequences only
      M = fmaxf(M, stat(q, s, ld_ml(q.slot0, s))[0]);
    M = wave_max(M);
    auto weight = [&](f32x2 t) { return t[1] > 0.f ? exp2f(t[0] - M) * t[1] : 0.f; };
    float e[kStats], den = 0.f;
#pragma unroll
    for (int i = 0; i < kStats; ++i) den += (e[i] = weight(st[i]));
    for (int s = kStatPieces + lane; s < n; s += 64) den += weight(stat(q, s, ld_ml(q.slot0, s)));
    // weight of piece p (wave-uniform p < n)
    auto weight_of = [&](int p) {
      if (p < 64) return lane_value(e[0], p);
      if (kStats > 1 && p < 128) return lane_value(e[kStats - 1], p - 64);
      return weight(stat(q, p, ld_ml(q.slot0, p)));
    };
    float acc[8];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) acc[e8] = 0.f;
    // A piece with zero weight (missing, or a clamped duplicate) is
    // skipped, so its values never meet the sum.
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int p = part + wps * u;
      const float eu = p < n ? lane_value(e[p < 64 ? 0 : kStats - 1], p & 63) : 0.f;
      if (eu != 0.f) {
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) acc[e8] += eu * (float)v[u][e8];
      }
    }
    // the rest of this wave's pieces (more than kChunk per wave)
    for (int u0 = kChunk; part + wps * u0 < n; u0 += kChunk) {
      const int cnt = min(kChunk, (n - 1 - part) / wps + 1 - u0);
#pragma unroll
      for (int u = 0; u < kChunk; ++u) v[u] = ld_o(q.slot0, part + wps * (u0 + min(u, cnt - 1)));
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const float eu = u < cnt ? weight_of(part + wps * (u0 + u)) : 0.f;
        if (eu != 0.f) {
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) acc[e8] += eu * (float)v[u][e8];
        }
      }
    }
    den = wave_sum(den);
    if (wps > 1) {
      // the sequence's waves add their partial sums in LDS, in wave order
      const uint32_t ps = ob + 16 * 1024 + ((uint32_t)wave * 64 + lane) * 32;
      *(lds_f32x4v*)(uintptr_t)ps = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(lds_f32x4v*)(uintptr_t)(ps + 16) = f32x4{acc[4], acc[5], acc[6], acc[7]};
      __syncthreads();
      if (part == 0) {
        for (int w2 = 1; w2 < wps; ++w2) {
          const uint32_t p2 = ps + (uint32_t)w2 * 64 * 32;
          const f32x4 x0 = *(lds_f32x4v*)(uintptr_t)p2, x1 = *(lds_f32x4v*)(uintptr_t)(p2 + 16);
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            acc[e4] += x0[e4];
            acc[4 + e4] += x1[e4];
          }
        }
      }
    }
    if (part == 0) {
      const float inv = den > 0.f ? 1.0f / den : 0.f;
      bf16x8 o;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) o[e8] = (bf16)(acc[e8] * inv);
      if constexpr (kProject)
        *(lds_bf16x8*)(uintptr_t)(ob + o_off(row, lane)) = o;
      else if (b < batch)
        *(bf16x8*)(out + ((long)b * H + h) * kR + 8 * lane) = o;
    }
  }
  if constexpr (!kProject) return;

  // out[b, h, :] = o_lat[b, h, :] W_UV[h]: rows in blocks of 16 x Dv, K =
  // 512, 16x16x32 MFMAs; wave w owns the 16-column block w (Dv <= 128).
  // Rows past S in a block hold stale LDS; they only reach output rows that
  // are not stored.
  __syncthreads();
  if (16 * wave >= Dv) return;
  const int g4 = lane >> 4, li = lane & 15;
  for (int rb = 0; 16 * rb < S; ++rb) {
    // eight k-steps at a time: their LDS reads first, then the MFMAs over
    // two accumulators (shorter dependency chains)
    f32x4 pacc[2] = {};
#pragma unroll
    for (int k8 = 0; k8 < kR / 32; k8 += 8) {
      bf16x8 a[8], bwf[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        a[u] = lds_read_b128(ob + o_off(16 * rb + li, 4 * (k8 + u) + g4));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // 16x16x32 B operand: lane (16 g + li) needs column li of rows 8 g .. 8 g + 7
        const uint32_t r = 32 * (k8 + u) + 8 * g4 + (li >> 2);
        const uint32_t c = 2 * wave + ((li & 3) >> 1), sub = 8 * (li & 1);
        bwf[u] = cat(lds_read_tr(wb + w_off(r, c) + sub), lds_read_tr(wb + w_off(r + 4, c) + sub));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) pacc[u & 1] = mfma16(a[u], bwf[u], pacc[u & 1]);
      __builtin_amdgcn_sched_group_barrier(0x100, 24, 0);  // the 24 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // then the 8 MFMAs
    }
    // register v of lane l: row 4 (l/16) + v of the block, column l%16
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int r = 16 * rb + 4 * g4 + v4;
      if (r < S && b0 + r < batch)
        out[((long)(b0 + r) * H + h) * Dv + 16 * wave + li] = (bf16)(pacc[0][v4] + pacc[1][v4]);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Split-KV attention partials only (the staged call).
// ---------------------------------------------------------------------------
// The arguments are ordered by when the workgroup needs them: the first 14
// dwords (up to num_blocks) are the ones the prologue uses before its first
// loads land, which the hardware preloads into scalar registers.
template <int HEADS, bool kFp8, int SL>
__global__ void __launch_bounds__(kThreads, 1) attn_decode_partials_kernel(
    const int* __restrict__ seq_lens, const int* __restrict__ block_table,
    const bf16* __restrict__ pool, int H, int n_wg, int batch, int guess_tiles, int max_blocks,
    int shift, int num_blocks, const bf16* __restrict__ q_full, int* __restrict__ prefix_out,
    float* __restrict__ part_ml, bf16* __restrict__ part_o) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  decode_attention_wg<HEADS, kFp8, SL>(smem, blockIdx.x, seq_lens, block_table, pool, H, n_wg,
                                       batch, guess_tiles, max_blocks, shift, num_blocks, q_full,
                                       prefix_out, part_ml, part_o);
}

// Combine of the partials (the staged call): grid (H, ceil(batch / S)).
// Arguments in the order the workgroup needs them (the first 14 dwords are
// preloaded into scalar registers).
template <bool kProject, int kChunk>
__global__ void __launch_bounds__(kCThreads) combine_kernel(
    const float* __restrict__ part_ml, const bf16* __restrict__ part_o,
    const bf16* __restrict__ w_uv, int batch, int H, int hg_heads, int n_wg, int guess_tiles,
    int S, int Dv, const int* __restrict__ prefix, bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char smem[kCWBytes + kCOBytes];
  const uint32_t wb = lds_addr(smem), ob = wb + kCWBytes;
  combine_wg<kProject, kChunk>(prefix, part_ml, part_o, batch, H, hg_heads, n_wg, guess_tiles, S,
                               w_uv, Dv, out, blockIdx.x, blockIdx.y * S, wb, ob);
}

// ---------------------------------------------------------------------------
size_t decode_partial_slots(int batch, int n_wg) { return (size_t)n_wg + (size_t)batch; }

int decode_heads_per_wg(int H, int batch, int max_seq_len, int num_cus) {
  // 64 heads per workgroup reads each tile once.  32 halves the split
  // partials and doubles the tiles per workgroup, but measured slower at
  // 32 x 4096 tokens (two workgroups then fetch every tile); it serves head
  // counts that are not a multiple of 64.
  (void)batch;
  (void)max_seq_len;
  (void)num_cus;
  return H % 64 == 0 ? 64 : 32;
}

int decode_num_wg(int head_groups, int num_cus) {
  // one workgroup per CU in total; a multiple of 8 per head group (XCD pairing)
  int n = num_cus / (head_groups > 0 ? head_groups : 1);
  n = (n / 8) * 8;
  return n < 8 ? 8 : n;
}

void launch_attention_partials_bf16(const void* q_full, const void* pool, int num_blocks,
                                    const int* block_table, int max_blocks, int block_shift,
                                    const int* seq_lens,
                                    int batch, int max_seq_len, int H, int heads_per_wg, int n_wg,
                                    int* prefix, float* part_ml, void* part_o, hipStream_t st,
                                    bool fp8) {
  const int hgc = H / heads_per_wg;
  const int guess_tiles = (max_seq_len + kTok - 1) / kTok;
  auto go = [&](auto kernel) {
    kernel<<<n_wg * hgc, kThreads, 0, st>>>(seq_lens, block_table, (const bf16*)pool, H, n_wg,
                                            batch, guess_tiles, max_blocks, block_shift,
                                            num_blocks, (const bf16*)q_full, prefix, part_ml,
                                            (bf16*)part_o);
  };
  // bf16 rows over several 64-head groups: every tile load on the P*C waves
  if (heads_per_wg == 64 && fp8)
    go(attn_decode_partials_kernel<64, true, kSLoads>);
  else if (heads_per_wg == 64 && hgc > 1)
    go(attn_decode_partials_kernel<64, false, 0>);
  else if (heads_per_wg == 64)
    go(attn_decode_partials_kernel<64, false, kSLoads>);
  else
    fp8 ? go(attn_decode_partials_kernel<32, true, kSLoads>)
        : go(attn_decode_partials_kernel<32, false, kSLoads>);
}

int combine_rows_per_wg(int H, int batch, int num_cus) {
  // the largest power of two (at most 32) whose grid still fills the CUs once
  int S = kCMaxRows;
  while (S > 1 && (long)H * ((batch + S - 1) / S) < num_cus) S >>= 1;
  return S;
}

void launch_combine(const int* prefix, const float* part_ml, const void* part_o, int batch, int H,
                    int heads_per_wg, int n_wg, int max_seq_len, const void* w_uv, int Dv,
                    void* out, int num_cus, hipStream_t st) {
  const int S = combine_rows_per_wg(H, batch, num_cus);
  dim3 grid(H, (batch + S - 1) / S);
  const int guess_tiles =
      (int)std::clamp(((long)max_seq_len + kTok - 1) / kTok, 1L, (long)INT_MAX / max(batch, 1));
  // pieces of a sequence in the equal-length layout, at most: the first
  // chunk holds 8 of a wave's pieces, or 16 when a wave has more
  const long T = (long)batch * guess_tiles, q = T / n_wg, r = T % n_wg;
  auto start = [&](long w) { return w * q + (w * r) / n_wg; };
  auto owner = [&](long x) {  // the workgroup whose range holds tile x
    long lo = 0, hi = n_wg - 1;
    while (lo < hi) {
      const long mid = (lo + hi + 1) / 2;
      if (start(mid) <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  long n_max = 1;
  for (long b = 0; b < batch; ++b)
    n_max = std::max(n_max, owner((b + 1) * guess_tiles - 1) - owner(b * guess_tiles) + 1);
  const int wps = S < kCWaves ? kCWaves / S : 1;
  const bool wide = (n_max + wps - 1) / wps > 8;
  auto go = [&](auto kernel, const void* w) {
    kernel<<<grid, kCThreads, 0, st>>>(part_ml, (const bf16*)part_o, (const bf16*)w, batch, H,
                                       heads_per_wg, n_wg, guess_tiles, S, Dv, prefix,
                                       (bf16*)out);
  };
  if (w_uv)
    wide ? go(combine_kernel<true, 16>, w_uv) : go(combine_kernel<true, 8>, w_uv);
  else
    wide ? go(combine_kernel<false, 16>, nullptr) : go(combine_kernel<false, 8>, nullptr);
}

}  // namespace mla
