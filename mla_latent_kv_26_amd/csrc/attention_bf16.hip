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
// overlap the other's MFMAs), 64 heads.  For S, wave w takes heads
// 16 (w%4) .. +16 and tokens 32 (w/4) .. +32 of the tile (its heads' queries
// stay in registers); for P*C, wave w owns columns 64 w .. +64 of O for all
// 64 heads.  Tiles stream HBM -> LDS with asynchronous direct-to-LDS loads
// into two buffers: tile j+1 is in flight while tile j is multiplied.
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
constexpr int kHG = 64;                                 // heads per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoads = kCh / kWaves;                    // 9 chunk loads per wave per tile
constexpr int kPStride = 72;                            // bf16 per P row (64 + 8)
constexpr int kOStride = kR + 8;                        // bf16 per staged output row
constexpr int kMaxBatch = 1024;

constexpr int kOffP = 2 * kTileBytes;                   // bf16 [64][72]
constexpr int kOffRed = kOffP + kHG * kPStride * 2;     // float [2][64] half-tile maxima
constexpr int kOffAlpha = kOffRed + 2 * kHG * 4;        // float [64] rescale factors
constexpr int kOffFlag = kOffAlpha + kHG * 4;           // float [8] per-wave rescale flags
constexpr int kOffLsum = kOffFlag + 32;                 // float [2][64] row sums
constexpr int kOffInv = kOffLsum + 2 * kHG * 4;         // float [64] 1 / row sum
constexpr int kOffScan = kOffInv + kHG * 4;             // int [8] scan scratch
constexpr int kOffPrefix = kOffScan + 32;               // int [kMaxBatch + 1]
constexpr int kLdsBytes = kOffPrefix + (kMaxBatch + 1) * 4;
static_assert(kLdsBytes <= 163840, "LDS budget");
static_assert(kHG * kOStride * 2 <= 2 * kTileBytes, "output staging fits the tile buffers");
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

struct SegState {
  f32x16 o[2][2];   // O[32 hb + ..][64 wave + 32 cb + ..]
  float m;          // reference max of this lane's S head, log2 units
  float l;          // lane-partial running sum for that head
};

// Attend one query row (64 heads at q_rows, row stride kW) over tiles
// [tile0, tile1) of one sequence (len rows, page table `table`).
__device__ __forceinline__ void run_segment(const bf16* __restrict__ q_rows,
                                            const bf16* __restrict__ pool,
                                            const int* __restrict__ table, int shift, int len,
                                            int tile0, int tile1, uint32_t lds, SegState& st,
                                            int wave, int lane) {
  const uint32_t p_lds = lds + kOffP, alp = lds + kOffAlpha, red = lds + kOffRed;
  const int hq = wave & 3, th = wave >> 2;
  const int h = 16 * hq + (lane & 15);     // this lane's head in the S phase
  const uint32_t kq = lane >> 4;           // 0..3

  // Per-lane LDS bases; every other offset below is a compile-time constant.
  // S: row tr = 32 th + 16 tb + lane%16, chunk k = 4 ks + kq at position
  // 8 (ks/2) + ((4 (ks%2) + kq) ^ swz(tr)); swz(tr) depends on lane%16 only.
  const uint32_t tr0 = 32u * th + (lane & 15);
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
  const uint32_t pw_base = p_lds + (h * kPStride + 32 * th + 4 * kq) * 2;
  const uint32_t al_base = alp + 16 * (lane >> 5);

  // queries of this wave's 16 heads: B operand of S^T = T Q^T (16x16x32)
  bf16x8 qf[kW / 32];
  {
    const bf16* q = q_rows + h * kW + 8 * kq;
#pragma unroll
    for (int ks = 0; ks < kW / 32; ++ks) qf[ks] = *(const bf16x8*)(q + 32 * ks);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
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

    // ---- S^T for tokens 32 th + (0..31) x heads 16 hq + (0..15), K = 576
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
    {
      // fragment (ks, tb): row tr0 + 16 tb -> + tb * 16 * 1152 bytes
      auto frag = [&](int ks, int tb) {
        return lds_read_b128(buf + ((ks & 1) ? s_odd : s_even) +
                             (uint32_t)((ks >> 1) * 128 + tb * 16 * kCh * 16));
      };
      bf16x8 a0 = frag(0, 0), a1 = frag(0, 1);
      bf16x8 b0 = frag(1, 0), b1v = frag(1, 1);
#pragma unroll
      for (int ks = 0; ks < kW / 32; ++ks) {
        bf16x8 n0 = a0, n1 = a1;
        if (ks + 2 < kW / 32) {
          n0 = frag(ks + 2, 0);
          n1 = frag(ks + 2, 1);
        }
        sacc[0] = mfma16(a0, qf[ks], sacc[0]);
        sacc[1] = mfma16(a1, qf[ks], sacc[1]);
        a0 = b0;
        a1 = b1v;
        b0 = n0;
        b1v = n1;
      }
    }
    // register v of block tb <-> token 32 th + 16 tb + 4 kq + v, head h
    const int valid = len - tile * kTok;
    float hmax = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (32 * th + 16 * tb + 4 * (int)kq + v >= valid) sacc[tb][v] = -INFINITY;
        hmax = fmaxf(hmax, sacc[tb][v]);
      }
    hmax = fmaxf(hmax, __shfl_xor(hmax, 16, 64));
    hmax = fmaxf(hmax, __shfl_xor(hmax, 32, 64));
    if (lane < 16) lds_st(red + (th * kHG + h) * 4, hmax);
    lds_barrier();
    const float tmax = fmaxf(lds_ld(red + h * 4), lds_ld(red + (kHG + h) * 4));
    const bool grow = tmax > st.m + kRescaleSlack;
    const float m_new = grow ? tmax : st.m;
    const float alpha = grow ? exp2f(st.m - m_new) : 1.0f;
    const bool any = __ballot(grow) != 0ull;
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
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
    if (th == 0 && lane < 16) lds_st(alp + h * 4, alpha);
    if (lane == 0) lds_st(lds + kOffFlag + wave * 4, any ? 1.0f : 0.0f);
    lds_barrier();

    // ---- O[64 h, 64 wave + (0..63)] = O * alpha + P T
    const f32x4 f0 = lds_ld4(lds + kOffFlag), f1 = lds_ld4(lds + kOffFlag + 16);
    if (f0[0] + f0[1] + f0[2] + f0[3] + f1[0] + f1[1] + f1[2] + f1[3] != 0.0f) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
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
      const bf16x8 pa0 = lds_read_b128(pa_base + ks * 32);
      const bf16x8 pa1 = lds_read_b128(pa_base + 32 * kPStride * 2 + ks * 32);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const uint32_t off = buf + (uint32_t)(ks * 16 * kCh * 16);
        const bf16x8 bv = cat(lds_read_tr(off + tr_off[cb][0]), lds_read_tr(off + tr_off[cb][1]));
        st.o[0][cb] = mfma32(pa0, bv, st.o[0][cb]);
        st.o[1][cb] = mfma32(pa1, bv, st.o[1][cb]);
      }
    }
  }
}

// Row sums of the segment: per-wave partial sums into LDS, then the S-phase
// waves of the first token half combine them into 1/l per head.  Returns the
// head's full sum in lanes 0..15 of waves 0..3 (the lanes that hold its m).
// Ends with a barrier.
__device__ __forceinline__ float finish_sums(const SegState& st, uint32_t lds, int wave, int lane) {
  float lt = st.l + __shfl_xor(st.l, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (lane < 16) lds_st(lds + kOffLsum + ((wave >> 2) * kHG + 16 * (wave & 3) + lane) * 4, lt);
  lds_barrier();
  float tot = 0.f;
  if (wave < 4 && lane < 16) {
    const int h = 16 * wave + lane;
    tot = lds_ld(lds + kOffLsum + h * 4) + lds_ld(lds + kOffLsum + (kHG + h) * 4);
    lds_st(lds + kOffInv + h * 4, 1.0f / tot);
  }
  lds_barrier();
  return tot;
}

// Store O / l for the 64 heads of this workgroup to dst[h * head_stride + c]
// (bf16): normalise into an LDS staging area (the tile buffers, free by
// now), then copy out with 16-byte coalesced stores.  Call after
// finish_sums; ends with a barrier.
__device__ __forceinline__ void store_normalised(const SegState& st, uint32_t lds, bf16* dst,
                                                 long head_stride, int wave, int lane) {
  typedef __attribute__((address_space(3))) bf16 lds_bf16;
  // one per-lane base; (head, column-block) offsets are constants below 64 KiB
  const uint32_t st_base = lds + ((4 * (lane >> 5)) * kOStride + 64 * wave + (lane & 31)) * 2;
  const uint32_t inv_base = lds + kOffInv + 16 * (lane >> 5);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
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
  for (int i = threadIdx.x; i < kHG * kR / 8; i += kThreads) {
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
__global__ void __launch_bounds__(kThreads, 1) attn_decode_partials_kernel(
    const bf16* __restrict__ q_full, const bf16* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int shift,
    const int* __restrict__ seq_lens, int batch, int H, int n_wg, int* __restrict__ prefix_out,
    float* __restrict__ part_ml, bf16* __restrict__ part_o) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const uint32_t lds = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hgc = H / kHG;
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
  SegState st;
  while (x0 < x1) {
    const long seg_end = min(x1, (long)prefix[b + 1]);
    const int len = seq_lens[b];
    const int tile0 = (int)(x0 - prefix[b]), tile1 = (int)(seg_end - prefix[b]);
    if (tile1 <= tile0) {  // a sequence without rows (invalid input): nothing to attend
      ++b;
      continue;
    }
    run_segment(q_full + ((long)b * H + hg * kHG) * kW, pool, block_table + (long)b * max_blocks,
                shift, len, tile0, tile1, lds, st, wave, lane);
    const float tot = finish_sums(st, lds, wave, lane);
    const long slot = (long)hg * n_slots + w + b;
    if (wave < 4 && lane < 16) {
      const int h = 16 * wave + lane;
      part_ml[(slot * kHG + h) * 2 + 0] = st.m;
      part_ml[(slot * kHG + h) * 2 + 1] = tot;
    }
    store_normalised(st, lds, part_o + slot * kHG * kR, kR, wave, lane);
    x0 = seg_end;
    ++b;
  }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup per (query row, head group); whole causal range.
// Rows are processed longest first.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads, 1) attn_prefill_kernel(
    const bf16* __restrict__ q_full, const bf16* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int shift,
    const int* __restrict__ start_pos, int T_len, int n_rows, int H, bf16* __restrict__ o_lat) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const uint32_t lds = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hgc = H / kHG;
  const int hg = blockIdx.x % hgc;
  const int r = blockIdx.x / hgc;
  // longest rows first: t descending, sequences interleaved
  const int nb = n_rows / T_len;
  const int t = T_len - 1 - r / nb;
  const int b = r % nb;
  const int n = b * T_len + t;
  const int len = start_pos[b] + t + 1;
  (void)tid;
  SegState st;
  run_segment(q_full + ((long)n * H + hg * kHG) * kW, pool, block_table + (long)b * max_blocks,
              shift, len, 0, (len + kTok - 1) / kTok, lds, st, wave, lane);
  finish_sums(st, lds, wave, lane);
  store_normalised(st, lds, o_lat + ((long)n * H + hg * kHG) * kR, kR, wave, lane);
}

// ---------------------------------------------------------------------------
// Combine (+ optional W_UV projection).  Workgroup = (head, 16 sequences).
// o_lat[b, h] = sum_s e_s O_s / sum_s e_s,  e_s = 2^(m_s - M) l_s.
// All global loads of a phase are issued before any is used.
// ---------------------------------------------------------------------------
namespace {
constexpr int kCRows = 16;
constexpr int kCOStride = kR + 8;       // bf16 per o_lat row in LDS
// W_UV[h] in LDS: rows of 16 chunks (256 B, Dv <= 128), chunk c of row r at
// position c ^ 2(r&3), so the 4 rows x 2 chunks of a transposing read fall
// on 8 distinct bank groups.
__device__ __forceinline__ uint32_t w_off(uint32_t r, uint32_t c) {
  return (r * 16u + (c ^ ((r & 3u) << 1))) * 16u;
}
constexpr int kMaxSeg = 64;             // pieces per (sequence, head) with weights kept in LDS
}

__global__ void __launch_bounds__(256) combine_kernel(
    const int* __restrict__ prefix, const float* __restrict__ part_ml,
    const bf16* __restrict__ part_o, int batch, int H, int n_wg, const bf16* __restrict__ w_uv,
    int Dv, bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16 olds[kCRows * kCOStride];
  __shared__ __attribute__((aligned(16))) bf16 wlds[kR * 128];
  __shared__ float wts[kCRows][kMaxSeg];
  __shared__ int seg0[kCRows], nseg[kCRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b0 = blockIdx.y * kCRows;
  const int hg = h / kHG, hl = h % kHG;
  const long T = prefix[batch];
  const long n_slots = (long)n_wg + batch;
  const bf16* W = w_uv ? w_uv + (long)h * kR * Dv : nullptr;

  // W_UV[h] -> LDS: every load of the matrix is issued up front
  if (W) {
    // at most 32 chunks per thread (Dv <= 128): all loads issued, then stored
    const int chunks = kR * Dv / 8;
    const uint32_t wb0 = lds_addr(wlds);
    bf16x8 wv[kR * 128 / 8 / 256];
#pragma unroll
    for (int i = 0; i < kR * 128 / 8 / 256; ++i) {
      const int c = tid + 256 * i;
      if (c < chunks) wv[i] = *(const bf16x8*)(W + (long)(c / (Dv / 8)) * Dv + (c % (Dv / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < kR * 128 / 8 / 256; ++i) {
      const int c = tid + 256 * i;
      if (c < chunks)
        *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(wb0 + w_off(c / (Dv / 8), c % (Dv / 8))) = wv[i];
    }
  }
  // segment ranges of the 16 sequences
  if (tid < kCRows) {
    const int b = b0 + tid;
    int f = 0, n = 0;
    if (b < batch && prefix[b + 1] > prefix[b]) {
      f = owner_of(prefix[b], T, n_wg);
      n = owner_of(prefix[b + 1] - 1, T, n_wg) - f + 1;
    }
    seg0[tid] = f;
    nseg[tid] = n;
  }
  __syncthreads();
  // merge weights e_s / sum e_s, 16 threads per row
  {
    const int rr = tid >> 4, sl = tid & 15;
    const int b = b0 + rr, f = seg0[rr], n = nseg[rr];
    float m_loc = -INFINITY;
    for (int s = sl; s < n; s += 16)
      m_loc = fmaxf(m_loc, part_ml[(((long)hg * n_slots + f + s + b) * kHG + hl) * 2]);
    for (int o = 1; o < 16; o <<= 1) m_loc = fmaxf(m_loc, __shfl_xor(m_loc, o, 64));
    float d_loc = 0.f;
    for (int s = sl; s < n; s += 16) {
      const long slot = (long)hg * n_slots + f + s + b;
      const float e = exp2f(part_ml[(slot * kHG + hl) * 2] - m_loc) * part_ml[(slot * kHG + hl) * 2 + 1];
      if (s < kMaxSeg) wts[rr][s] = e;
      d_loc += e;
    }
    for (int o = 1; o < 16; o <<= 1) d_loc += __shfl_xor(d_loc, o, 64);
    __syncthreads();
    for (int s = sl; s < min(n, kMaxSeg); s += 16) wts[rr][s] /= d_loc;
  }
  __syncthreads();
  // weighted sum: thread -> (row tid/16, 32 columns); four pieces in flight at a time
  {
    const int rr = tid >> 4, c0 = (tid & 15) * 32;
    const int b = b0 + rr, f = seg0[rr], n = nseg[rr];
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    if (n > kMaxSeg) {
      // long merges recompute their weights on the fly (more than 64 pieces)
      float M = -INFINITY, den = 0.f;
      for (int s = 0; s < n; ++s)
        M = fmaxf(M, part_ml[(((long)hg * n_slots + f + s + b) * kHG + hl) * 2]);
      for (int s = 0; s < n; ++s) {
        const long slot = (long)hg * n_slots + f + s + b;
        const float e = exp2f(part_ml[(slot * kHG + hl) * 2] - M) * part_ml[(slot * kHG + hl) * 2 + 1];
        den += e;
        const bf16* src = part_o + (slot * kHG + hl) * kR + c0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x8 v = *(const bf16x8*)(src + 8 * q);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[8 * q + i] += e * (float)v[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] /= den;
    } else {
      int s = 0;
      for (; s + 4 <= n; s += 4) {
        bf16x8 v[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16* src = part_o + (((long)hg * n_slots + f + s + u + b) * kHG + hl) * kR + c0;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[u][q] = *(const bf16x8*)(src + 8 * q);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float e = wts[rr][s + u];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[8 * q + i] += e * (float)v[u][q][i];
        }
      }
      for (; s < n; ++s) {
        const bf16* src = part_o + (((long)hg * n_slots + f + s + b) * kHG + hl) * kR + c0;
        const float e = wts[rr][s];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x8 v = *(const bf16x8*)(src + 8 * q);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[8 * q + i] += e * (float)v[i];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (bf16)acc[8 * q + i];
      if (!W) {
        if (b < batch) *(bf16x8*)(out + ((long)b * H + h) * kR + c0 + 8 * q) = v;
      } else {
        *(bf16x8*)(olds + rr * kCOStride + c0 + 8 * q) = v;
      }
    }
  }
  if (!W) return;
  __syncthreads();

  // out[b, h, :] = o_lat[b, h, :] W_UV[h]: 16 rows x Dv, K = 512, 16x16x32 MFMAs.
  // Wave w owns 16-column blocks w, w + 4 (Dv <= 128).
  const int nblk = Dv / 16;
  f32x4 acc[2] = {f32x4{}, f32x4{}};
  const uint32_t ob = lds_addr(olds), wb = lds_addr(wlds);
  const int g = lane >> 4, li = lane & 15;
#pragma unroll 4
  for (int ks = 0; ks < kR / 32; ++ks) {
    const bf16x8 a = lds_read_b128(ob + ((lane & 15) * kCOStride + 32 * ks + 8 * (lane >> 4)) * 2);
    // 16x16x32 B operand: lane (16g + li) needs column li of rows 8g .. 8g+7
    const uint32_t row = 32 * ks + 8 * g + (li >> 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nb = wave + 4 * j;
      if (nb < nblk) {
        const uint32_t c = 2 * nb + ((li & 3) >> 1), sub = 8 * (li & 1);
        const bf16x4 lo = lds_read_tr(wb + w_off(row, c) + sub);
        const bf16x4 hi = lds_read_tr(wb + w_off(row + 4, c) + sub);
        acc[j] = mfma16(a, cat(lo, hi), acc[j]);
      }
    }
  }
  // register v of lane l: row 4(l/16) + v, column l%16
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int nb = wave + 4 * j;
    if (nb >= nblk) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int b = b0 + 4 * (lane >> 4) + v;
      if (b < batch) out[((long)b * H + h) * Dv + 16 * nb + (lane & 15)] = (bf16)acc[j][v];
    }
  }
}

// ---------------------------------------------------------------------------
size_t decode_partial_slots(int batch, int n_wg) { return (size_t)n_wg + (size_t)batch; }

int decode_num_wg(int batch, int max_seq_len, int head_groups, int num_cus) {
  // one workgroup per CU in total; a multiple of 8 per head group (XCD pairing)
  (void)batch;
  (void)max_seq_len;
  int n = num_cus / head_groups;
  n = (n / 8) * 8;
  return n < 8 ? 8 : n;
}

void launch_attention_partials_bf16(const void* q_full, const void* pool, const int* block_table,
                                    int max_blocks, int block_shift, const int* seq_lens,
                                    int batch, int H, int n_wg, int* prefix, float* part_ml,
                                    void* part_o, hipStream_t st) {
  const int hgc = H / kHG;
  attn_decode_partials_kernel<<<n_wg * hgc, kThreads, 0, st>>>(
      (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_shift, seq_lens,
      batch, H, n_wg, prefix, part_ml, (bf16*)part_o);
}

void launch_combine(const int* prefix, const float* part_ml, const void* part_o, int batch, int H,
                    int n_wg, const void* w_uv, int Dv, void* out, hipStream_t st) {
  dim3 grid(H, (batch + kCRows - 1) / kCRows);
  combine_kernel<<<grid, 256, 0, st>>>(prefix, part_ml, (const bf16*)part_o, batch, H, n_wg,
                                       (const bf16*)w_uv, Dv, (bf16*)out);
}

void launch_attention_prefill_bf16(const void* q_full, const void* pool, const int* block_table,
                                   int max_blocks, int block_shift, const int* start_pos, int T,
                                   int batch, int H, void* o_lat, hipStream_t st) {
  const int hgc = H / kHG;
  const int n_rows = batch * T;
  attn_prefill_kernel<<<n_rows * hgc, kThreads, 0, st>>>((const bf16*)q_full, (const bf16*)pool,
                                                          block_table, max_blocks, block_shift,
                                                          start_pos, T, n_rows, H, (bf16*)o_lat);
}

}  // namespace mla
