// Latent attention on MFMA (gfx950), bf16 cache rows, float32 accumulate.
//
// For one query row and 64 heads (modeldna "MLA" module, "Under the hood":
// W_UK absorbed into the query, attention run on the cached latent):
//   s[h, j]  = q_full[h] . row_j          (q_full = scale*log2e*[q_lat | q_rope])
//   o_lat[h] = sum_j 2^(s[h,j] - m[h]) c_j / sum_j 2^(s[h,j] - m[h]).
// The rows are dense bf16 [c (512) | k_rope (64)], 1152 B each, shared by
// every head, so both contractions are matrix products:
//   S^T [64 tok x 64 h] = T [64 tok x 576] * Q^T [576 x 64 h]
//   O   [64 h x 512]   += P [64 h x 64 tok] * T[:, :512]
// and one LDS copy of each 64-token tile serves both: T is read row-wise
// for S (16-byte LDS reads) and column-wise for P*C (transposing LDS reads),
// so every cached byte leaves HBM once.
//
// Workgroup: 512 threads = 8 waves (two per SIMD, so one wave's LDS waits
// overlap the other's MFMAs) and HEADS = 64 or 32 heads.  For S, each wave
// takes 16 heads and 32 (HEADS = 64) or 16 (HEADS = 32) tokens of the tile
// (its heads' queries stay in registers); for P*C, wave w owns columns
// 64 w .. +64 of O for all HEADS heads.  Tiles stream HBM -> LDS with
// asynchronous direct-to-LDS loads into two buffers: tile j+1 is in flight
// while tile j is multiplied.  With HEADS = 32, two workgroups share each
// tile; they are placed on the same XCD so the second read hits its L2.
//
// Tile layout in LDS: row-major, row t (1152 B = 72 chunks of 16 B) at
// t*1152, with its chunk k stored at position k ^ swz(t) (a permutation
// inside each aligned group of 8 chunks).  A direct-to-LDS load instruction
// fills 64 consecutive slots; its lanes read the matching 1 KB of global
// memory in that permuted order, so every instruction stays fully coalesced.
// swz(t) = 2(t%4) + (t/4)%2 puts 8 consecutive rows (row-wise fragment
// reads) and the 4 rows x 2 neighbouring chunks of a transposing read on 8
// distinct bank groups: neither access pattern has bank conflicts.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kR = 512, kDr = 64, kW = kR + kDr;       // row width 576
constexpr int kTok = 64;                                // tokens per tile
constexpr int kCh = kW * 2 / 16;                        // 72 chunks per row
constexpr int kTileBytes = kTok * kW * 2;               // 73728
constexpr int kMaxHG = 64;                              // heads per workgroup, at most
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoads = kCh / kWaves;                    // 9 chunk loads per wave per tile
constexpr int kPStride = 72;                            // bf16 per P row (64 + 8)
constexpr int kOStride = kR + 8;                        // bf16 per staged output row
constexpr int kMaxBatch = 1024;

constexpr int kOffP = 2 * kTileBytes;                   // bf16 [64][72]
constexpr int kOffRed = kOffP + kMaxHG * kPStride * 2;  // float [4][64] per-token-group maxima
constexpr int kOffAlpha = kOffRed + 4 * kMaxHG * 4;     // float [64] rescale factors
constexpr int kOffFlag = kOffAlpha + kMaxHG * 4;        // float [8] per-wave rescale flags
constexpr int kOffLsum = kOffFlag + 32;                 // float [4][64] row sums
constexpr int kOffInv = kOffLsum + 4 * kMaxHG * 4;      // float [64] 1 / row sum
constexpr int kOffScan = kOffInv + kMaxHG * 4;          // int [8] scan scratch
constexpr int kOffPrefix = kOffScan + 32;               // int [kMaxBatch + 1]
constexpr int kLdsBytes = kOffPrefix + (kMaxBatch + 1) * 4;
static_assert(kLdsBytes <= 163840, "LDS budget");
static_assert(kMaxHG * kOStride * 2 <= 2 * kTileBytes, "output staging fits the tile buffers");

// Per-HEADS geometry: HQ 16-head blocks x TQ token groups = 8 waves for S;
// HB 32-head row blocks of O per wave for P*C.
template <int HEADS>
struct Geo {
  static_assert(HEADS == 32 || HEADS == 64, "32 or 64 heads per workgroup");
  static constexpr int HQ = HEADS / 16;
  static constexpr int TQ = kWaves / HQ;
  static constexpr int TPW = kTok / TQ;   // tokens per wave in S
  static constexpr int TB = TPW / 16;     // 16-token blocks per wave in S
  static constexpr int HB = HEADS / 32;
};
// A head's reference max only moves when a tile exceeds it by more than this
// (log2 units): probabilities stay below 2^8 and O is rescaled rarely.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ uint32_t swz(uint32_t t) { return ((t & 3u) << 1) | ((t >> 2) & 1u); }

// Issue the asynchronous loads of one tile: `valid` rows (1..64) starting at
// row pointer `rows` (consecutive rows of one page).  Wave w fills slots
// [64 j, 64 j + 64) for j = w, w+8, ..., w+64.  Rows past `valid` repeat
// the last valid row so the tile holds finite data (their probabilities are
// zero).
__device__ __forceinline__ void issue_tile(const bf16* rows, int valid, uint32_t buf, int wave,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const uint32_t j = (uint32_t)wave + 8u * i;
    const uint32_t s = 64u * j + (uint32_t)lane;
    const uint32_t t = s / kCh;
    const uint32_t k = (s - t * kCh) ^ swz(t);
    const uint32_t tt = min(t, (uint32_t)(valid - 1));
    g2lds16(rows + tt * kW + k * 8, buf + j * 1024u);
  }
}

template <int HEADS>
struct SegState {
  f32x16 o[Geo<HEADS>::HB][2];  // O[32 hb + ..][64 wave + 32 cb + ..]
  float m;                      // reference max of this lane's S head, log2 units
  float l;                      // lane-partial running sum for that head
};

// Attend one query row (HEADS heads at q_rows, row stride kW) over tiles
// [tile0, tile1) of one sequence (len rows, page table `table`).
template <int HEADS>
__device__ __forceinline__ void run_segment(const bf16* __restrict__ q_rows,
                                            const bf16* __restrict__ pool,
                                            const int* __restrict__ table, int shift, int len,
                                            int tile0, int tile1, uint32_t lds,
                                            SegState<HEADS>& st, int wave, int lane) {
  using G = Geo<HEADS>;
  const uint32_t p_lds = lds + kOffP, alp = lds + kOffAlpha, red = lds + kOffRed;
  const int hq = wave % G::HQ, tq = wave / G::HQ;
  const int h = 16 * hq + (lane & 15);     // this lane's head in the S phase
  const uint32_t kq = lane >> 4;           // 0..3

  // Per-lane LDS bases; every other offset below is a compile-time constant.
  // S: row tr = TPW tq + 16 tb + lane%16, chunk k = 4 ks + kq at position
  // 8 (ks/2) + ((4 (ks%2) + kq) ^ swz(tr)); swz(tr) depends on lane%16 only.
  const uint32_t tr0 = (uint32_t)(G::TPW * tq) + (lane & 15);
  const uint32_t s_even = (tr0 * kCh + (kq ^ swz(tr0))) * 16u;
  const uint32_t s_odd = (tr0 * kCh + ((4u + kq) ^ swz(tr0))) * 16u;
  // P*C transposing reads: lane (16 g + li) of the fragment for token block
  // ks and column block cb reads row 16 ks + x + 4 hi, chunk 8 wave + cc,
  // cc = 4 cb + 2 (g%2) + b1, at position 8 wave + (cc ^ (2 a + hi)), a = li/4.
  const uint32_t g = lane >> 4, li = lane & 15;
  const uint32_t x = 8u * (g >> 1) + (li >> 2), b1 = (li >> 1) & 1u, a2 = 2u * (li >> 2);
  uint32_t tr_off[2][2];  // [cb][hi]
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const uint32_t cc = 4u * cb + 2u * (g & 1) + b1;
      tr_off[cb][hi] = ((x + 4u * hi) * kCh + 8u * wave + (cc ^ (a2 + hi))) * 16u + 8u * (li & 1);
    }
  // P fragments (A operand of 32x32x16): row 32 hb + lane%32, tokens 16 ks + 8 (lane/32)
  const uint32_t pa_base = p_lds + ((lane & 31) * kPStride + 8 * (lane >> 5)) * 2;
  const uint32_t pw_base = p_lds + (h * kPStride + G::TPW * tq + 4 * kq) * 2;
  const uint32_t al_base = alp + 16 * (lane >> 5);

  // queries of this wave's 16 heads: B operand of S^T = T Q^T (16x16x32)
  bf16x8 qf[kW / 32];
  {
    const bf16* q = q_rows + h * kW + 8 * kq;
#pragma unroll
    for (int ks = 0; ks < kW / 32; ++ks) qf[ks] = *(const bf16x8*)(q + 32 * ks);
  }
#pragma unroll
  for (int a = 0; a < G::HB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) st.o[a][b] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;

  const int mask = (1 << shift) - 1;
  auto rows_at = [&](int tile, int page) {
    return pool + ((long)page * (mask + 1) + ((tile * kTok) & mask)) * kW;
  };
  int page = table[(tile0 * kTok) >> shift];
  issue_tile(rows_at(tile0, page), min(kTok, len - tile0 * kTok), lds, wave, lane);
  int next_page = (tile0 + 1 < tile1) ? table[((tile0 + 1) * kTok) >> shift] : 0;

  for (int tile = tile0; tile < tile1; ++tile) {
    const uint32_t buf = lds + (uint32_t)((tile - tile0) & 1) * kTileBytes;
    wait_vmcnt<0>();
    lds_barrier();  // tile visible to all waves; previous tile fully consumed
    if (tile + 1 < tile1) {
      issue_tile(rows_at(tile + 1, next_page), min(kTok, len - (tile + 1) * kTok),
                 lds + (uint32_t)((tile + 1 - tile0) & 1) * kTileBytes, wave, lane);
      if (tile + 2 < tile1) next_page = table[((tile + 2) * kTok) >> shift];
    }

    // ---- S^T for tokens TPW tq + (0..TPW-1) x heads 16 hq + (0..15), K = 576
    f32x4 sacc[G::TB];
#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb) sacc[tb] = f32x4{};
    {
      // fragment (ks, tb): row tr0 + 16 tb -> + tb * 16 * 1152 bytes
      auto frag = [&](int ks, int tb) {
        return lds_read_b128(buf + ((ks & 1) ? s_odd : s_even) +
                             (uint32_t)((ks >> 1) * 128 + tb * 16 * kCh * 16));
      };
      constexpr int D = G::TB == 1 ? 3 : 1;  // k-steps read ahead
      bf16x8 fr[D + 1][G::TB];
#pragma unroll
      for (int d = 0; d < D; ++d)
#pragma unroll
        for (int tb = 0; tb < G::TB; ++tb) fr[d][tb] = frag(d, tb);
#pragma unroll
      for (int ks = 0; ks < kW / 32; ++ks) {
        if (ks + D < kW / 32) {
#pragma unroll
          for (int tb = 0; tb < G::TB; ++tb) fr[(ks + D) % (D + 1)][tb] = frag(ks + D, tb);
        }
#pragma unroll
        for (int tb = 0; tb < G::TB; ++tb)
          sacc[tb] = mfma16(fr[ks % (D + 1)][tb], qf[ks], sacc[tb]);
      }
    }
    // register v of block tb <-> token TPW tq + 16 tb + 4 kq + v, head h
    const int valid = len - tile * kTok;
    float hmax = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (G::TPW * tq + 16 * tb + 4 * (int)kq + v >= valid) sacc[tb][v] = -INFINITY;
        hmax = fmaxf(hmax, sacc[tb][v]);
      }
    hmax = fmaxf(hmax, __shfl_xor(hmax, 16, 64));
    hmax = fmaxf(hmax, __shfl_xor(hmax, 32, 64));
    if (lane < 16) lds_st(red + (tq * kMaxHG + h) * 4, hmax);
    lds_barrier();
    float tmax = lds_ld(red + h * 4);
#pragma unroll
    for (int t2 = 1; t2 < G::TQ; ++t2) tmax = fmaxf(tmax, lds_ld(red + (t2 * kMaxHG + h) * 4));
    const bool grow = tmax > st.m + kRescaleSlack;
    const float m_new = grow ? tmax : st.m;
    const float alpha = grow ? exp2f(st.m - m_new) : 1.0f;
    const bool any = __ballot(grow) != 0ull;
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb) {
      bf16x4 pk;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bf16 pb = (bf16)exp2f(sacc[tb][v] - m_new);
        pk[v] = pb;
        psum += (float)pb;
      }
      lds_st(pw_base + tb * 32, pk);
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
    if (tq == 0 && lane < 16) lds_st(alp + h * 4, alpha);
    if (lane == 0) lds_st(lds + kOffFlag + wave * 4, any ? 1.0f : 0.0f);
    lds_barrier();

    // ---- O[HEADS h, 64 wave + (0..63)] = O * alpha + P T
    const f32x4 f0 = lds_ld4(lds + kOffFlag), f1 = lds_ld4(lds + kOffFlag + 16);
    if (f0[0] + f0[1] + f0[2] + f0[3] + f1[0] + f1[1] + f1[2] + f1[3] != 0.0f) {
#pragma unroll
      for (int hb = 0; hb < G::HB; ++hb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 a4 = lds_ld4(al_base + hb * 128 + q * 32);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.o[hb][cb][4 * q + r] *= a4[r];
        }
    }
#pragma unroll
    for (int ks = 0; ks < kTok / 16; ++ks) {
      bf16x8 pa[G::HB];
#pragma unroll
      for (int hb = 0; hb < G::HB; ++hb)
        pa[hb] = lds_read_b128(pa_base + hb * 32 * kPStride * 2 + ks * 32);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const uint32_t off = buf + (uint32_t)(ks * 16 * kCh * 16);
        const bf16x8 bv = cat(lds_read_tr(off + tr_off[cb][0]), lds_read_tr(off + tr_off[cb][1]));
#pragma unroll
        for (int hb = 0; hb < G::HB; ++hb) st.o[hb][cb] = mfma32(pa[hb], bv, st.o[hb][cb]);
      }
    }
  }
}

// Row sums of the segment: per-wave partial sums into LDS, then the S-phase
// waves of the first token group combine them into 1/l per head.  Returns the
// head's full sum in lanes 0..15 of waves 0..HQ-1 (the lanes that hold its m).
// Ends with a barrier.
template <int HEADS>
__device__ __forceinline__ float finish_sums(const SegState<HEADS>& st, uint32_t lds, int wave,
                                             int lane) {
  using G = Geo<HEADS>;
  float lt = st.l + __shfl_xor(st.l, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  const int h = 16 * (wave % G::HQ) + (lane & 15);
  if (lane < 16) lds_st(lds + kOffLsum + ((wave / G::HQ) * kMaxHG + h) * 4, lt);
  lds_barrier();
  float tot = 0.f;
  if (wave < G::HQ && lane < 16) {
#pragma unroll
    for (int t2 = 0; t2 < G::TQ; ++t2) tot += lds_ld(lds + kOffLsum + (t2 * kMaxHG + h) * 4);
    lds_st(lds + kOffInv + h * 4, 1.0f / tot);
  }
  lds_barrier();
  return tot;
}

// Store O / l for the HEADS heads of this workgroup to dst[h * head_stride + c]
// (bf16): normalise into an LDS staging area (the tile buffers, free by
// now), then copy out with 16-byte coalesced stores.  Call after
// finish_sums; ends with a barrier.
template <int HEADS>
__device__ __forceinline__ void store_normalised(const SegState<HEADS>& st, uint32_t lds,
                                                 bf16* dst, long head_stride, int wave, int lane) {
  typedef __attribute__((address_space(3))) bf16 lds_bf16;
  // one per-lane base; (head, column-block) offsets are constants below 64 KiB
  const uint32_t st_base = lds + ((4 * (lane >> 5)) * kOStride + 64 * wave + (lane & 31)) * 2;
  const uint32_t inv_base = lds + kOffInv + 16 * (lane >> 5);
#pragma unroll
  for (int hb = 0; hb < Geo<HEADS>::HB; ++hb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 inv = lds_ld4(inv_base + (32 * hb + 8 * q) * 4);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *(lds_bf16*)(uintptr_t)(st_base + ((32 * hb + 8 * q + r) * kOStride + 32 * cb) * 2) =
              (bf16)(st.o[hb][cb][4 * q + r] * inv[r]);
    }
  lds_barrier();
#pragma unroll
  for (int i0 = 0; i0 < HEADS * kR / 8; i0 += kThreads) {
    const int i = i0 + threadIdx.x;
    const int hh = i / (kR / 8), c8 = (i % (kR / 8)) * 8;
    *(bf16x8*)(dst + hh * head_stride + c8) = lds_read_b128(lds + (hh * kOStride + c8) * 2);
  }
  lds_barrier();
}

// Workgroup -> (head group, stream index); the head groups of one stream
// index sit 8 workgroups apart, so round-robin dispatch puts them on the
// same XCD and the second group reads each tile from that XCD's L2.
__device__ __forceinline__ void map_block(int hgc, int& hg, int& w) {
  const int b = blockIdx.x;
  const int per = 8 * hgc;
  hg = (b % per) / 8;
  w = (b / per) * 8 + (b % 8);
}

}  // namespace

// Which workgroup of the stream owns tile x (ranges [w*T/n, (w+1)*T/n)).
__host__ __device__ inline int owner_of(long x, long T, int n) {
  int w = (int)((x * n) / T);
  while (w + 1 < n && ((long)(w + 1) * T) / n <= x) ++w;
  while (w > 0 && ((long)w * T) / n > x) --w;
  return w;
}

// ---------------------------------------------------------------------------
// Decode: each workgroup takes an equal share of the concatenated tile stream
// of all sequences; every (workgroup, sequence) piece writes one partial
// into slot w + b (unique: w + b grows along the stream).
// ---------------------------------------------------------------------------
template <int HEADS>
__global__ void __launch_bounds__(kThreads, 1) attn_decode_partials_kernel(
    const bf16* __restrict__ q_full, const bf16* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int shift,
    const int* __restrict__ seq_lens, int batch, int H, int n_wg, int* __restrict__ prefix_out,
    float* __restrict__ part_ml, bf16* __restrict__ part_o) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const uint32_t lds = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hgc = H / HEADS;
  int hg, w;
  map_block(hgc, hg, w);
  int* prefix = (int*)(smem + kOffPrefix);

  // prefix sums of tiles per sequence (2 sequences per thread, then a scan)
  {
    int cnt[2], tot = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = tid * 2 + i;
      cnt[i] = b < batch ? (seq_lens[b] + kTok - 1) / kTok : 0;
      tot += cnt[i];
    }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int* wsum = (int*)(smem + kOffScan);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wave; ++i) base += wsum[i];
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
    __syncthreads();
  }
  const long T = prefix[batch];
  if (blockIdx.x == 0)
    for (int b = tid; b <= batch; b += kThreads) prefix_out[b] = prefix[b];

  long x0 = ((long)w * T) / n_wg, x1 = ((long)(w + 1) * T) / n_wg;
  if (x0 >= x1) return;
  // first sequence touching x0
  int b = 0;
  {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= x0) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  const long n_slots = (long)n_wg + batch;
  SegState<HEADS> st;
  while (x0 < x1) {
    const long seg_end = min(x1, (long)prefix[b + 1]);
    const int len = seq_lens[b];
    const int tile0 = (int)(x0 - prefix[b]), tile1 = (int)(seg_end - prefix[b]);
    if (tile1 <= tile0) {  // a sequence without rows (invalid input): nothing to attend
      ++b;
      continue;
    }
    run_segment<HEADS>(q_full + ((long)b * H + hg * HEADS) * kW, pool,
                       block_table + (long)b * max_blocks, shift, len, tile0, tile1, lds, st,
                       wave, lane);
    const float tot = finish_sums<HEADS>(st, lds, wave, lane);
    const long slot = (long)hg * n_slots + w + b;
    if (wave < Geo<HEADS>::HQ && lane < 16) {
      const int h = 16 * wave + lane;
      part_ml[(slot * HEADS + h) * 2 + 0] = st.m;
      part_ml[(slot * HEADS + h) * 2 + 1] = tot;
    }
    store_normalised<HEADS>(st, lds, part_o + slot * HEADS * kR, kR, wave, lane);
    x0 = seg_end;
    ++b;
  }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup per (query row, head group); whole causal range.
// Rows are processed longest first.
// ---------------------------------------------------------------------------
template <int HEADS>
__global__ void __launch_bounds__(kThreads, 1) attn_prefill_kernel(
    const bf16* __restrict__ q_full, const bf16* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int shift,
    const int* __restrict__ start_pos, int T_len, int n_rows, int H, bf16* __restrict__ o_lat) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const uint32_t lds = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hgc = H / HEADS;
  const int hg = blockIdx.x % hgc;
  const int r = blockIdx.x / hgc;
  // longest rows first: t descending, sequences interleaved
  const int nb = n_rows / T_len;
  const int t = T_len - 1 - r / nb;
  const int b = r % nb;
  const int n = b * T_len + t;
  const int len = start_pos[b] + t + 1;
  (void)tid;
  SegState<HEADS> st;
  run_segment<HEADS>(q_full + ((long)n * H + hg * HEADS) * kW, pool,
                     block_table + (long)b * max_blocks, shift, len, 0, (len + kTok - 1) / kTok,
                     lds, st, wave, lane);
  finish_sums<HEADS>(st, lds, wave, lane);
  store_normalised<HEADS>(st, lds, o_lat + ((long)n * H + hg * HEADS) * kR, kR, wave, lane);
}

// ---------------------------------------------------------------------------
// Combine (+ optional W_UV projection).  Workgroup = (head, 16 sequences),
// 512 threads; thread (row tid/32, 16 columns).
// o_lat[b, h] = sum_s e_s O_s / sum_s e_s,  e_s = 2^(m_s - M) l_s.
// Dependent global round trips are kept to two: the prefix sums, then every
// piece's statistics and values at once.  W_UV[h] streams into LDS with
// direct-to-LDS loads issued first.
// ---------------------------------------------------------------------------
namespace {
constexpr int kCRows = 16;
constexpr int kCThreads = 512;
constexpr int kCOStride = kR + 8;       // bf16 per o_lat row in LDS
constexpr int kSegChunk = 8;            // pieces whose values are in flight together

// W_UV[h] in LDS: rows of 16 chunks (256 B, Dv <= 128), chunk c of row r at
// position c ^ 2(r&3), so the 4 rows x 2 chunks of a transposing read fall
// on 8 distinct bank groups.
__device__ __forceinline__ uint32_t w_off(uint32_t r, uint32_t c) {
  return (r * 16u + (c ^ ((r & 3u) << 1))) * 16u;
}
}  // namespace

__global__ void __launch_bounds__(kCThreads) combine_kernel(
    const int* __restrict__ prefix, const float* __restrict__ part_ml,
    const bf16* __restrict__ part_o, int batch, int H, int hg_heads, int n_wg,
    const bf16* __restrict__ w_uv, int Dv, bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16 olds[kCRows * kCOStride];
  __shared__ __attribute__((aligned(16))) bf16 wlds[kR * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b0 = blockIdx.y * kCRows;
  const int hg = h / hg_heads, hl = h % hg_heads;
  const long n_slots = (long)n_wg + batch;
  const bf16* W = w_uv ? w_uv + (long)h * kR * Dv : nullptr;
  const uint32_t wb = lds_addr(wlds);

  // W_UV[h] -> LDS (asynchronous): slot s = 64 j + lane holds row s/16,
  // chunk (s%16) ^ 2(row&3); chunks past Dv/8 load the row's chunk 0 (unused).
  if (W) {
#pragma unroll
    for (int i = 0; i < kR * 16 / 64 / 8; ++i) {
      const uint32_t j = (uint32_t)wave * (kR * 16 / 64 / 8) + i;
      const uint32_t s = 64u * j + lane, r = s >> 4;
      uint32_t c = (s & 15u) ^ ((r & 3u) << 1);
      if ((int)c >= Dv / 8) c = 0;
      g2lds16(W + (long)r * Dv + c * 8, wb + j * 1024u);
    }
  }

  const int rr = tid >> 5, sl = tid & 31, c0 = sl * 16;
  const int b = b0 + rr;
  const long T = prefix[batch];
  int f = 0, n = 0;
  if (b < batch) {
    const int p0 = prefix[b], p1 = prefix[b + 1];
    if (p1 > p0) {
      f = owner_of(p0, T, n_wg);
      n = owner_of(p1 - 1, T, n_wg) - f + 1;
    }
  }
  const long slot0 = (long)hg * n_slots + f + b;
  // statistics: thread sl holds pieces sl and sl + 32 (n <= 64 here; longer
  // merges loop over groups of 64)
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float M = -INFINITY;
  for (int s = sl; s < n; s += 32) M = fmaxf(M, part_ml[((slot0 + s) * hg_heads + hl) * 2]);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float den = 0.f;
  for (int s0 = 0; s0 < n; s0 += 32) {
    // weight of piece s0 + sl, then all of this group's values, kSegChunk at a time
    const int sw = s0 + sl;
    float e = 0.f;
    if (sw < n) {
      const float2 ml = *(const float2*)(part_ml + ((slot0 + sw) * hg_heads + hl) * 2);
      e = exp2f(ml.x - M) * ml.y;
    }
    den += e;
    const int m = min(32, n - s0);
    for (int u0 = 0; u0 < m; u0 += kSegChunk) {
      bf16x8 v[kSegChunk][2];
#pragma unroll
      for (int u = 0; u < kSegChunk; ++u)
        if (u0 + u < m) {
          const bf16* src = part_o + ((slot0 + s0 + u0 + u) * hg_heads + hl) * kR + c0;
          v[u][0] = *(const bf16x8*)src;
          v[u][1] = *(const bf16x8*)(src + 8);
        }
#pragma unroll
      for (int u = 0; u < kSegChunk; ++u) {
        const float eu = __shfl(e, (lane & 32) + u0 + u, 64);
        if (u0 + u < m) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            acc[i] += eu * (float)v[u][0][i];
            acc[8 + i] += eu * (float)v[u][1][i];
          }
        }
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) den += __shfl_xor(den, o, 64);
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  bf16x8 o0, o1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o0[i] = (bf16)(acc[i] * inv);
    o1[i] = (bf16)(acc[8 + i] * inv);
  }
  if (!W) {
    if (b < batch) {
      *(bf16x8*)(out + ((long)b * H + h) * kR + c0) = o0;
      *(bf16x8*)(out + ((long)b * H + h) * kR + c0 + 8) = o1;
    }
    return;
  }
  *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(lds_addr(olds) + (rr * kCOStride + c0) * 2) = o0;
  *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(lds_addr(olds) + (rr * kCOStride + c0 + 8) * 2) = o1;
  wait_vmcnt<0>();
  __syncthreads();

  // out[b, h, :] = o_lat[b, h, :] W_UV[h]: 16 rows x Dv, K = 512, 16x16x32 MFMAs;
  // wave w owns the 16-column block w (Dv <= 128).
  if (16 * wave >= Dv) return;
  f32x4 pacc = {};
  const uint32_t ob = lds_addr(olds);
  const int g = lane >> 4, li = lane & 15;
#pragma unroll 4
  for (int ks = 0; ks < kR / 32; ++ks) {
    const bf16x8 a = lds_read_b128(ob + ((lane & 15) * kCOStride + 32 * ks + 8 * (lane >> 4)) * 2);
    // 16x16x32 B operand: lane (16g + li) needs column li of rows 8g .. 8g+7
    const uint32_t row = 32 * ks + 8 * g + (li >> 2);
    const uint32_t c = 2 * wave + ((li & 3) >> 1), sub = 8 * (li & 1);
    const bf16x4 lo = lds_read_tr(wb + w_off(row, c) + sub);
    const bf16x4 hi = lds_read_tr(wb + w_off(row + 4, c) + sub);
    pacc = mfma16(a, cat(lo, hi), pacc);
  }
  // register v of lane l: row 4(l/16) + v, column l%16
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int bb = b0 + 4 * (lane >> 4) + v;
    if (bb < batch) out[((long)bb * H + h) * Dv + 16 * wave + (lane & 15)] = (bf16)pacc[v];
  }
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
  int n = num_cus / head_groups;
  n = (n / 8) * 8;
  return n < 8 ? 8 : n;
}

void launch_attention_partials_bf16(const void* q_full, const void* pool, const int* block_table,
                                    int max_blocks, int block_shift, const int* seq_lens,
                                    int batch, int H, int heads_per_wg, int n_wg, int* prefix,
                                    float* part_ml, void* part_o, hipStream_t st) {
  const int hgc = H / heads_per_wg;
  if (heads_per_wg == 64)
    attn_decode_partials_kernel<64><<<n_wg * hgc, kThreads, 0, st>>>(
        (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_shift, seq_lens,
        batch, H, n_wg, prefix, part_ml, (bf16*)part_o);
  else
    attn_decode_partials_kernel<32><<<n_wg * hgc, kThreads, 0, st>>>(
        (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_shift, seq_lens,
        batch, H, n_wg, prefix, part_ml, (bf16*)part_o);
}

void launch_combine(const int* prefix, const float* part_ml, const void* part_o, int batch, int H,
                    int heads_per_wg, int n_wg, const void* w_uv, int Dv, void* out,
                    hipStream_t st) {
  dim3 grid(H, (batch + kCRows - 1) / kCRows);
  combine_kernel<<<grid, kCThreads, 0, st>>>(prefix, part_ml, (const bf16*)part_o, batch, H,
                                       heads_per_wg, n_wg, (const bf16*)w_uv, Dv, (bf16*)out);
}

void launch_attention_prefill_bf16(const void* q_full, const void* pool, const int* block_table,
                                   int max_blocks, int block_shift, const int* start_pos, int T,
                                   int batch, int H, void* o_lat, hipStream_t st) {
  const int n_rows = batch * T;
  if (H % 64 == 0)
    attn_prefill_kernel<64><<<n_rows * (H / 64), kThreads, 0, st>>>(
        (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_shift, start_pos, T,
        n_rows, H, (bf16*)o_lat);
  else
    attn_prefill_kernel<32><<<n_rows * (H / 32), kThreads, 0, st>>>(
        (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_shift, start_pos, T,
        n_rows, H, (bf16*)o_lat);
}

}  // namespace mla
