// Decode attention on the latent rows for narrower latents than the tuned
// kernel takes: kv_lora_rank 128 or 256 with a 64-wide rope key, heads in
// blocks of 16, any page size.  These are the widths of the tutorial's
// mechanism experiment ("ARCH-MLA. Multihead Latent Attention", 5.1: 16
// query heads, latent 256, rope 64).  The math is the absorbed form of the
// modeldna "MLA" module ("Under the hood"): scores q_full . [c | k_rope] with
// q_full already scaled by softmax_scale * log2(e), softmax over each
// sequence's tokens, weights applied to c.
//
// One workgroup (4 waves) takes 16 heads of one sequence over one chunk of
// its tokens in 64-token steps; wave w owns tokens 16 w .. 16 w + 15 of each
// step and keeps its own running maximum, sum and output, so the waves never
// wait for one another until the chunk ends.  Per step a wave stages its 16
// rows in its own LDS buffer (rows padded to W + 8 values: 16 consecutive
// rows of one column, and the 4 x 4 pieces of a transposing read, hit
// distinct banks) and runs
//   S^T [16 tok x 16 h]  = T [16 x W] Q^T        16x16x32 MFMAs, W / 32 of them
//   O^T [R x 16 h]      += T[:, :R]^T P^T        16x16x16 MFMAs, R / 16 of them
// with the queries (B of the first product) in registers and P (B of the
// second) straight from the score accumulators: lane l holds tokens
// 4 (l/16) .. + 3 of head l % 16 in both layouts.  The column fragments of
// the second product come from transposing LDS reads.  At the chunk's end
// the four waves' partials are merged through LDS and written once
// (float32 (m, l, O), m in log2 units); merge_generic_kernel combines the
// chunks of a sequence.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kGT = 64;   // tokens per workgroup step (16 per wave)
constexpr int kGH = 16;   // heads per workgroup
constexpr float kNarrowSlack = 8.0f;  // lazy rescale threshold (log2 units)

__device__ __forceinline__ f32x4 mfma16k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// Rows of RW values; scores over values SOFF .. SOFF + SW - 1 of a row
// (queries of SW values), the weighted sum over values 0 .. VW - 1.  Latent
// rows: RW = SW = R + 64, SOFF = 0, VW = R.  Reconstructed per-head rows
// [V | K_nope | k_rope]: RW = Dv + Dn + Dr, SOFF = Dv, SW = Dn + Dr, VW = Dv.
template <int RW, int SOFF, int SW, int VW>
__global__ void __launch_bounds__(256) attention_generic_kernel(
    const bf16* __restrict__ q_full, const bf16* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int block_size,
    const int* __restrict__ seq_lens, int H, int chunk, int n_split, float* __restrict__ part_ml,
    float* __restrict__ part_o) {
  constexpr int W = RW;                // row width (values)
  constexpr int R = VW;                // output width
  constexpr int kRowE = W + 8;         // LDS row stride (values)
  constexpr int kChunks = W / 8;       // 16-byte pieces per row
  constexpr int kLoads = 16 * kChunks / 64;  // per lane and step
  constexpr int kKS = SW / 32;         // score k-steps
  constexpr int kCB = R / 16;          // column blocks of O^T
  static_assert(SW % 32 == 0 && R % 16 == 0 && SOFF + SW <= W && R <= W, "row layout");
  static_assert(16 * kChunks % 64 == 0, "a wave's rows split evenly over its lanes");
  constexpr int kBufE = 16 * kRowE;    // one wave's buffer (values)
  // per wave: one row buffer; at the end, O^T of the four waves (float)
  constexpr int kTileBytes = 4 * kBufE * 2;
  constexpr int kMergeBytes = 4 * kGH * R * 4;
  __shared__ __align__(16) unsigned char smem[kTileBytes > kMergeBytes ? kTileBytes : kMergeBytes];
  __shared__ float mls[4][2][kGH];

  const int split = blockIdx.x, hb = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int len = seq_lens[b];
  const int begin = split * chunk;
  const int end = min(len, begin + chunk);
  const long slot = ((long)b * n_split + split) * H + hb * kGH;
  if (begin >= end) {  // nothing in this chunk: an empty partial (uniform per block)
    if (tid < kGH) {
      part_ml[(slot + tid) * 2] = -INFINITY;
      part_ml[(slot + tid) * 2 + 1] = 0.f;
    }
    // zero O too, so the merge reads every chunk's O without a branch
    for (int i = tid; i < kGH * R; i += 256) part_o[slot * R + i] = 0.f;
    return;
  }

  // queries (B of the score product): head li, values 32 ks + 8 lg .. + 7
  bf16x8 qf[kKS];
  {
    const bf16* q = q_full + ((long)b * H + hb * kGH + li) * SW + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[ks] = *(const bf16x8*)(q + 32 * ks);
  }
  bf16* buf = (bf16*)smem + w * kBufE;

  // this wave's rows of the step at t0: tokens t0 + 16 w + r (r < 16), piece
  // c = lane + 64 i of the wave's 16 x kChunks pieces; zero past the chunk
  uint4 pre[kLoads];
  auto load = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = lane + 64 * i, r = c / kChunks, k = c - r * kChunks;
      const int j = t0 + 16 * w + r;
      uint4 v = {0u, 0u, 0u, 0u};
      if (j < end) {
        const long page = block_table[(long)b * max_blocks + j / block_size];
        v = *(const uint4*)(pool + (page * block_size + j % block_size) * W + k * 8);
      }
      pre[i] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = lane + 64 * i, r = c / kChunks, k = c - r * kChunks;
      *(uint4*)(buf + r * kRowE + k * 8) = pre[i];
    }
  };

  float m = -INFINITY, l = 0.f;  // for head li (identical in the four lane groups)
  f32x4 acc[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc[cb] = f32x4{};

  const int n_steps = (end - begin + kGT - 1) / kGT;
  load(begin);
  for (int t = 0; t < n_steps; ++t) {
    const int t0 = begin + t * kGT;
    // the previous step's reads of the buffer are done (this wave's own
    // program order), so it can take this step's rows
    store();
    if (t + 1 < n_steps) load(t0 + kGT);
    // S^T: A = rows li (16 tokens), values 32 ks + 8 lg .. + 7
    f32x4 s = f32x4{};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const bf16x8 a = *(const bf16x8*)(buf + li * kRowE + SOFF + 32 * ks + 8 * lg);
      s = mfma16(a, qf[ks], s);
    }
    // register v <-> token t0 + 16 w + 4 lg + v, head li
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (t0 + 16 * w + 4 * lg + v >= end) s[v] = -INFINITY;
      tmax = fmaxf(tmax, s[v]);
    }
    tmax = max_xor32(max_xor16(tmax));
    // lazy reference: moved only when a step exceeds it by more than the slack
    const bool grow = tmax > m + kNarrowSlack;
    const float m_new = grow ? tmax : m;
    if (__ballot(grow) != 0ull) {
      const float alpha = grow ? fast_exp2(m - m_new) : 1.0f;  // 0 on the first step
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) acc[cb] *= alpha;
      l *= alpha;
    }
    m = m_new;
    bf16x4 p;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      // a wave whose tokens are all past the chunk's end has m = -inf
      const bf16 pv = (bf16)(m == -INFINITY ? 0.f : fast_exp2(s[v] - m));
      p[v] = pv;
      psum += (float)pv;
    }
    l += psum;
    // O^T += T[:, cols]^T P^T: A = columns 16 cb + li, tokens 4 lg .. + 3 (a
    // transposing read: lane 4 a + c of the group reads row 4 lg + a, columns
    // 16 cb + 4 c .. + 3)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const bf16x4 a = lds_read_tr(lds_addr(buf) +
                                   ((4 * lg + (li >> 2)) * kRowE + 16 * cb + 4 * (li & 3)) * 2);
      acc[cb] = mfma16k16(a, p, acc[cb]);
    }
  }

  // ---- merge the four waves' partials of the chunk, then write it ----
  l = sum_xor32(sum_xor16(l));
  __syncthreads();  // every wave is done with its row buffer
  float* ob = (float*)smem;
  if (lg == 0) {
    mls[w][0][li] = m;
    mls[w][1][li] = l;
  }
  // O^T register v of block cb <-> column 16 cb + 4 lg + v, head li
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
    *(f32x4*)(ob + ((w * kGH + li) * R + 16 * cb + 4 * lg)) = acc[cb];
  __syncthreads();
  // thread (head hh, column block) combines the four waves with weights
  // 2^(m_w - M) (M: the largest m; waves that saw no token have m = -inf)
  for (int e = tid; e < kGH * (R / 4); e += 256) {
    const int hh = e / (R / 4), c4 = (e % (R / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, mls[v][0][hh]);
    f32x4 o = f32x4{};
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float mw = mls[v][0][hh];
      const float wt = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      o += wt * *(const f32x4*)(ob + (v * kGH + hh) * R + c4);
      L += wt * mls[v][1][hh];
    }
    *(f32x4*)(part_o + (slot + hh) * R + c4) = o;
    if (c4 == 0) {
      part_ml[(slot + hh) * 2] = M;
      part_ml[(slot + hh) * 2 + 1] = L;
    }
  }
}

// o_lat[b, h, :] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the
// chunks s (M = the largest m; empty chunks have m = -inf, weight 0 and a
// zero O); zero for an empty sequence.  One 256-thread block per (head,
// sequence): the chunk weights go to LDS, then wave w sums chunks w, w + 4,
// ... for all R columns (independent loads, several in flight), and the four
// wave sums are added.
constexpr int kMaxSplit = 1024;

template <int R, typename TO>
__global__ void __launch_bounds__(256) merge_generic_kernel(const float* __restrict__ part_ml,
                                                            const float* __restrict__ part_o,
                                                            int H, int n_split,
                                                            TO* __restrict__ o_lat) {
  constexpr int kC = R / 64;
  __shared__ float wts[kMaxSplit];
  __shared__ float red[4];
  __shared__ __align__(16) float sums[4][R];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const float* ml = part_ml + ((long)b * n_split * H + h) * 2;
  float mx = -INFINITY;
  for (int s = tid; s < n_split; s += 256) mx = fmaxf(mx, ml[(long)s * H * 2]);
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float ls = 0.f;
  for (int s = tid; s < n_split; s += 256) {
    const float ms = ml[(long)s * H * 2];
    const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
    wts[s] = wgt;
    ls = fmaf(wgt, ml[(long)s * H * 2 + 1], ls);
  }
  ls = wave_sum(ls);
  if (lane == 0) red[w] = ls;
  __syncthreads();
  const float L = (red[0] + red[1]) + (red[2] + red[3]);
  float acc[kC];
#pragma unroll
  for (int c = 0; c < kC; ++c) acc[c] = 0.f;
  const float* o = part_o + ((long)b * n_split * H + h) * R + kC * lane;
#pragma unroll 4
  for (int s = w; s < n_split; s += 4) {
    const float wgt = wts[s];
    const float* os = o + (long)s * H * R;
#pragma unroll
    for (int c = 0; c < kC; ++c) acc[c] = fmaf(wgt, os[c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < kC; ++c) sums[w][kC * lane + c] = acc[c];
  __syncthreads();
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  TO* dst = o_lat + ((long)b * H + h) * R;
  for (int r = tid; r < R; r += 256)
    dst[r] = from_f32<TO>(((sums[0][r] + sums[1][r]) + (sums[2][r] + sums[3][r])) * inv);
}

}  // namespace

bool attention_generic_fits(int H, int R, int Dr) {
  return (R == 256 || R == 128) && Dr == 64 && H % kGH == 0;
}

void generic_split(int batch, int H, int max_seq_len, int num_cus, int* chunk, int* n_split) {
  const int tiles = (max_seq_len + kGT - 1) / kGT;
  const long wgs_per_split = (long)batch * (H / kGH);
  const long want = (2L * num_cus + wgs_per_split - 1) / wgs_per_split;
  long splits = want < 1 ? 1 : want > tiles ? tiles : want;
  if (splits > kMaxSplit) splits = kMaxSplit;   // the merge keeps one weight per chunk in LDS
  const int per = (int)((tiles + splits - 1) / splits);
  *chunk = per * kGT;
  *n_split = (tiles + per - 1) / per;   // <= splits
}

template <int RW, int SOFF, int SW, int VW>
void launch_narrow(const void* q_full, const void* pool, const int* block_table, int max_blocks,
                   int block_size, const int* seq_lens, int batch, int H, int chunk, int n_split,
                   float* part_ml, float* part_o, void* o_lat, bool o_f32, hipStream_t st) {
  const dim3 grid(n_split, H / kGH, batch);
  attention_generic_kernel<RW, SOFF, SW, VW><<<grid, 256, 0, st>>>(
      (const bf16*)q_full, (const bf16*)pool, block_table, max_blocks, block_size, seq_lens, H,
      chunk, n_split, part_ml, part_o);
  const dim3 mg(H, batch);
  if (o_f32)
    merge_generic_kernel<VW, float><<<mg, 256, 0, st>>>(part_ml, part_o, H, n_split, (float*)o_lat);
  else
    merge_generic_kernel<VW, bf16><<<mg, 256, 0, st>>>(part_ml, part_o, H, n_split, (bf16*)o_lat);
}

void launch_attention_generic(const void* q_full, const void* pool, const int* block_table,
                              int max_blocks, int block_size, const int* seq_lens, int batch,
                              int H, int R, int chunk, int n_split, float* part_ml, float* part_o,
                              void* o_lat, bool o_f32, hipStream_t st) {
  if (R == 256)
    launch_narrow<320, 0, 320, 256>(q_full, pool, block_table, max_blocks, block_size, seq_lens,
                                    batch, H, chunk, n_split, part_ml, part_o, o_lat, o_f32, st);
  else
    launch_narrow<192, 0, 192, 128>(q_full, pool, block_table, max_blocks, block_size, seq_lens,
                                    batch, H, chunk, n_split, part_ml, part_o, o_lat, o_f32, st);
}

void launch_attention_perhead(const void* q, const void* rows, const int* table, int row_block,
                              const int* seq_lens, int batch, int chunk, int n_split,
                              float* part_ml, float* part_o, void* o, hipStream_t st) {
  // rows [V (64) | K_nope (64) | k_rope (64)]; scores over values 64 .. 191
  launch_narrow<192, 64, 128, 64>(q, rows, table, 1, row_block, seq_lens, batch, kGH, chunk,
                                  n_split, part_ml, part_o, o, false, st);
}

}  // namespace mla
