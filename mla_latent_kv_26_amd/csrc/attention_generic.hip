// Decode attention on the latent rows for narrower latents than the tuned
// kernel takes: kv_lora_rank 128 or 256 with a 64-wide rope key, heads in
// blocks of 16, any page size.  These are the widths of the tutorial's
// mechanism experiment ("ARCH-MLA. Multihead Latent Attention", 5.1: 16
// query heads, latent 256, rope 64).  The math is the absorbed form of the
// modeldna "MLA" module ("Under the hood"): scores q_full . [c | k_rope] with
// q_full already scaled by softmax_scale * log2(e), softmax over each
// sequence's tokens, weights applied to c.
//
// One workgroup (8 waves) takes 16 heads of one sequence over one chunk of
// its tokens, 64-token tiles staged in LDS (two buffers; the next tile's
// global loads are in flight while the current one is used).  Wave w owns
// heads 2w, 2w+1: lane n scores token n of the tile (bf16 dot2 products,
// float32 sums), the wave keeps the running max and sum of its heads, and for
// the weighted sum lane n owns R/64 latent columns of those heads.  Each
// chunk writes an unnormalised partial (m, l, O) in float32; a second kernel
// merges the chunks of a sequence.  Vector-ALU work: at these widths one
// token costs 2 * 16 * (2R + 64) flops against (R + 64) * 2 bytes.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kGT = 64;   // tokens per tile
constexpr int kGH = 16;   // heads per workgroup

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ float lo_bf16(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xffff0000u);
}

template <int R, int kWaves>
__global__ void __launch_bounds__(64 * kWaves) attention_generic_kernel(
    const bf16* __restrict__ q_full, const bf16* __restrict__ pool,
    const int* __restrict__ block_table, int max_blocks, int block_size,
    const int* __restrict__ seq_lens, int H, int chunk, int n_split, float* __restrict__ part_ml,
    float* __restrict__ part_o) {
  constexpr int W = R + 64;           // row width (values)
  constexpr int kRow = W * 2 + 16;    // LDS row stride (bytes), padded
  constexpr int kChunks = W / 8;      // 16-byte pieces per row
  constexpr int kThreads = 64 * kWaves;
  constexpr int kHW = kGH / kWaves;   // heads per wave
  constexpr int kLoads = kGT * kChunks / kThreads;
  constexpr int kC = R / 64;          // latent columns per lane
  static_assert(kGT * kChunks % kThreads == 0, "tile pieces must split evenly over the block");
  static_assert(kHW == 2 || kHW == 4, "two or four heads per wave");
  __shared__ __align__(16) unsigned char tile[2][kGT * kRow];
  __shared__ __align__(16) unsigned char qs[kGH * W * 2];
  __shared__ __align__(16) float ps[kGT * kGH];

  const int split = blockIdx.x, hb = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int len = seq_lens[b];
  const int begin = split * chunk;
  const int end = min(len, begin + chunk);
  const long slot = ((long)b * n_split + split) * H + hb * kGH + kHW * w;
  if (begin >= end) {  // nothing in this chunk: an empty partial (uniform per block)
    if (lane < kHW) {
      part_ml[(slot + lane) * 2] = -INFINITY;
      part_ml[(slot + lane) * 2 + 1] = 0.f;
    }
    // zero O too, so the merge reads every chunk's O without a branch
    for (int i = lane; i < kHW * R; i += 64) part_o[slot * R + i] = 0.f;
    return;
  }

  // queries of the 16 heads
  const bf16* qsrc = q_full + ((long)b * H + hb * kGH) * W;
  for (int i = tid; i < kGH * kChunks; i += kThreads)
    *(uint4*)(qs + i * 16) = *(const uint4*)(qsrc + i * 8);

  uint4 pre[kLoads];
  auto load = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i, r = c / kChunks, k = c - r * kChunks;
      const int j = t0 + r;
      uint4 v = {0u, 0u, 0u, 0u};
      if (j < end) {
        const long page = block_table[(long)b * max_blocks + j / block_size];
        v = *(const uint4*)(pool + (page * block_size + j % block_size) * W + k * 8);
      }
      pre[i] = v;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i, r = c / kChunks, k = c - r * kChunks;
      *(uint4*)(tile[buf] + r * kRow + k * 16) = pre[i];
    }
  };

  float m[kHW], l[kHW], acc[kHW][kC];
#pragma unroll
  for (int j = 0; j < kHW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) acc[j][c] = 0.f;
  }

  load(begin);
  store(0);
  __syncthreads();
  const int n_tiles = (end - begin + kGT - 1) / kGT;
  for (int t = 0; t < n_tiles; ++t) {
    const int t0 = begin + t * kGT;
    const bool more = t + 1 < n_tiles;
    if (more) load(t0 + kGT);
    const unsigned char* tb = tile[t & 1];

    // scores of token `lane` for heads kHW w .. kHW w + kHW - 1
    float s[kHW];
#pragma unroll
    for (int j = 0; j < kHW; ++j) s[j] = 0.f;
    const unsigned char* rowp = tb + lane * kRow;
    const unsigned char* qp = qs + (kHW * w) * W * 2;
#pragma unroll 4
    for (int k = 0; k < kChunks; ++k) {
      const uint4 rv = *(const uint4*)(rowp + k * 16);
#pragma unroll
      for (int j = 0; j < kHW; ++j) {
        const uint4 qv = *(const uint4*)(qp + j * W * 2 + k * 16);
        s[j] = dot2(rv.x, qv.x, s[j]);
        s[j] = dot2(rv.y, qv.y, s[j]);
        s[j] = dot2(rv.z, qv.z, s[j]);
        s[j] = dot2(rv.w, qv.w, s[j]);
      }
    }
    const bool valid = t0 + lane < end;
    float p[kHW];
#pragma unroll
    for (int j = 0; j < kHW; ++j) {
      const float sj = valid ? s[j] : -INFINITY;
      const float mn = fmaxf(m[j], wave_max(sj));   // finite: the tile has a valid token
      const float corr = exp2f(m[j] - mn);          // 0 on the first tile
      p[j] = valid ? exp2f(sj - mn) : 0.f;
      l[j] = l[j] * corr + wave_sum(p[j]);
      m[j] = mn;
#pragma unroll
      for (int c = 0; c < kC; ++c) acc[j][c] *= corr;
    }
    if constexpr (kHW == 4)
      *(f32x4*)(ps + lane * kGH + 4 * w) = f32x4{p[0], p[1], p[2], p[3]};
    else
      *(f32x2*)(ps + lane * kGH + 2 * w) = f32x2{p[0], p[1]};
    __syncthreads();

    // weighted sum: lane owns latent columns kC*lane .. kC*lane + kC - 1
#pragma unroll 4
    for (int n = 0; n < kGT; ++n) {
      float pn[kHW];
      if constexpr (kHW == 4) {
        const f32x4 v = *(const f32x4*)(ps + n * kGH + 4 * w);
        pn[0] = v[0], pn[1] = v[1], pn[2] = v[2], pn[3] = v[3];
      } else {
        const f32x2 v = *(const f32x2*)(ps + n * kGH + 2 * w);
        pn[0] = v[0], pn[1] = v[1];
      }
      float cv[kC];
      if constexpr (kC == 4) {
        const uint2 raw = *(const uint2*)(tb + n * kRow + lane * 8);
        cv[0] = lo_bf16(raw.x);
        cv[1] = hi_bf16(raw.x);
        cv[2] = lo_bf16(raw.y);
        cv[3] = hi_bf16(raw.y);
      } else {
        const uint32_t raw = *(const uint32_t*)(tb + n * kRow + lane * 4);
        cv[0] = lo_bf16(raw);
        cv[1] = hi_bf16(raw);
      }
#pragma unroll
      for (int j = 0; j < kHW; ++j)
#pragma unroll
        for (int c = 0; c < kC; ++c) acc[j][c] = fmaf(pn[j], cv[c], acc[j][c]);
    }
    if (more) store((t + 1) & 1);
    __syncthreads();
  }

  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < kHW; ++j) {
      part_ml[(slot + j) * 2] = m[j];
      part_ml[(slot + j) * 2 + 1] = l[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kHW; ++j) {
    float* dst = part_o + (slot + j) * R + kC * lane;
    if constexpr (kC == 4)
      *(f32x4*)dst = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
    else
      *(f32x2*)dst = f32x2{acc[j][0], acc[j][1]};
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

void launch_attention_generic(const void* q_full, const void* pool, const int* block_table,
                              int max_blocks, int block_size, const int* seq_lens, int batch,
                              int H, int R, int chunk, int n_split, float* part_ml, float* part_o,
                              void* o_lat, bool o_f32, hipStream_t st) {
  const dim3 grid(n_split, H / kGH, batch);
  if (R == 256)
    attention_generic_kernel<256, 8><<<grid, 512, 0, st>>>((const bf16*)q_full, (const bf16*)pool,
                                                       block_table, max_blocks, block_size,
                                                       seq_lens, H, chunk, n_split, part_ml, part_o);
  else
    attention_generic_kernel<128, 8><<<grid, 512, 0, st>>>((const bf16*)q_full, (const bf16*)pool,
                                                       block_table, max_blocks, block_size,
                                                       seq_lens, H, chunk, n_split, part_ml, part_o);
  const dim3 mg(H, batch);
  if (R == 256) {
    if (o_f32)
      merge_generic_kernel<256, float><<<mg, 256, 0, st>>>(part_ml, part_o, H, n_split, (float*)o_lat);
    else
      merge_generic_kernel<256, bf16><<<mg, 256, 0, st>>>(part_ml, part_o, H, n_split, (bf16*)o_lat);
  } else {
    if (o_f32)
      merge_generic_kernel<128, float><<<mg, 256, 0, st>>>(part_ml, part_o, H, n_split, (float*)o_lat);
    else
      merge_generic_kernel<128, bf16><<<mg, 256, 0, st>>>(part_ml, part_o, H, n_split, (bf16*)o_lat);
  }
}

}  // namespace mla
