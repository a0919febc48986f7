// Query absorption for the bf16 decode (modeldna "MLA" module, "Under the
// hood": W_UK folded into the query), at the widths of the latent kernels
// (qk_nope_dim 128, kv_lora_rank 512, rope_dim 64):
//   q_full[b, h] = alpha [q_nope[b, h] W_UK[h] | q_rope[b, h]]      (576 values)
// alpha = softmax scale * log2(e).  One workgroup per (128-column block of
// the latent, head, 32 query rows); 4 waves of 32 columns.
//
// The whole operand set of a workgroup (W_UK[h][:, 128 columns], 32 KB; 32
// query rows, 8 KB; the rope part for column block 0) goes in flight at once
// and through LDS in one step: with K = 128 there is a single k block, so
// the kernel is one round trip to HBM plus 8 MFMAs per wave.  The product is
// computed transposed (C^T = W_UK^T q_nope^T: the transposing LDS read of
// W_UK is the MFMA A operand, the query rows the B operand), so each lane
// holds runs of 4 consecutive columns of one query row and stores 8 bytes at
// a time.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kAbN = 128;        // latent columns per workgroup
constexpr int kAbK = 128;        // qk_nope_dim
constexpr int kAbRows = 32;      // query rows per workgroup
constexpr int kAbR = 512, kAbDr = 64, kAbW = kAbR + kAbDr;
// W rows in LDS: 320 B (64 mod 256), so the 4 rows x 64 bytes that 32 lanes
// of a transposing read touch are 4 disjoint bank ranges; query rows: 272 B,
// so 16-byte row-wise reads of 32 rows spread over all banks.
constexpr int kWStride = kAbN + 32;
constexpr int kQStride = kAbK + 8;

__global__ void __launch_bounds__(256) absorb_query_kernel(const bf16* __restrict__ q_nope,
                                                           const bf16* __restrict__ q_rope,
                                                           const bf16* __restrict__ w_uk,
                                                           bf16* __restrict__ q_full, int B, int H,
                                                           float alpha) {
  __shared__ __attribute__((aligned(16))) bf16 ws[kAbK * kWStride];
  __shared__ __attribute__((aligned(16))) bf16 qs[kAbRows * kQStride];
  const int cb = blockIdx.x, h = blockIdx.y, b0 = blockIdx.z * kAbRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = cb * kAbN;
  const bf16* W = w_uk + (long)h * kAbK * kAbR + n0;

  // every load first: W (8 chunks of 16 B per thread), query rows (2), rope (1)
  bf16x8 wr[8], qr[2], rr = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i, r = c >> 4, k = (c & 15) * 8;
    wr[i] = *(const bf16x8*)(W + (long)r * kAbR + k);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, r = c >> 4, k = (c & 15) * 8, b = b0 + r;
    qr[i] = b < B ? *(const bf16x8*)(q_nope + ((long)b * H + h) * kAbK + k) : bf16x8{};
  }
  const int rb = b0 + (tid >> 3), rk = (tid & 7) * 8;
  const bool rope = cb == 0 && rb < B;
  if (rope) rr = *(const bf16x8*)(q_rope + ((long)rb * H + h) * kAbDr + rk);

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i, r = c >> 4, k = (c & 15) * 8;
    *(bf16x8*)(ws + r * kWStride + k) = wr[i];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, r = c >> 4, k = (c & 15) * 8;
    *(bf16x8*)(qs + r * kQStride + k) = qr[i];
  }
  if (rope) {
#pragma unroll
    for (int e = 0; e < 8; ++e) rr[e] = (bf16)(alpha * (float)rr[e]);
    *(bf16x8*)(q_full + ((long)rb * H + h) * kAbW + kAbR + rk) = rr;
  }
  __syncthreads();

  // C^T [32 columns of wave, 32 rows] over K = 128 (8 steps of 16): A
  // fragment lane l = column l%32, k 8(l/32) .. +7 (transposing reads of W),
  // B fragment lane l = query row l%32, the same k (one 16-byte row read)
  const uint32_t wb = lds_addr(ws), qb = lds_addr(qs);
  const int g = lane >> 4, li = lane & 15;
  const int tr_row = 8 * (g >> 1) + (li >> 2), tr_col = 32 * wave + 16 * (g & 1) + 4 * (li & 3);
  bf16x8 af[kAbK / 16], bfr[kAbK / 16];
#pragma unroll
  for (int ks = 0; ks < kAbK / 16; ++ks) {
    const int row = 16 * ks + tr_row;
    af[ks] = cat(lds_read_tr(wb + (row * kWStride + tr_col) * 2),
                 lds_read_tr(wb + ((row + 4) * kWStride + tr_col) * 2));
    bfr[ks] = lds_read_b128(qb + ((lane & 31) * kQStride + 16 * ks + 8 * (lane >> 5)) * 2);
  }
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < kAbK / 16; ++ks) acc = mfma32(af[ks], bfr[ks], acc);

  // register v of lane l: column 32 wave + 8 (v/4) + 4 (l/32) + v%4, row l%32
  const int b = b0 + (lane & 31);
  if (b >= B) return;
  bf16* dst = q_full + ((long)b * H + h) * kAbW + n0 + 32 * wave + 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (bf16)(alpha * acc[4 * j + i]);
    *(bf16x4*)(dst + 8 * j) = o;
  }
}

}  // namespace

bool launch_absorb_query_bf16(const void* q_nope, const void* q_rope, const void* w_uk,
                              void* q_full, int B, int H, int Dn, int R, int Dr, float alpha,
                              hipStream_t st) {
  if (Dn != kAbK || R != kAbR || Dr != kAbDr || B <= 0 || H <= 0) return false;
  dim3 grid(kAbR / kAbN, H, (B + kAbRows - 1) / kAbRows);
  absorb_query_kernel<<<grid, 256, 0, st>>>((const bf16*)q_nope, (const bf16*)q_rope,
                                            (const bf16*)w_uk, (bf16*)q_full, B, H, alpha);
  return true;
}

}  // namespace mla
