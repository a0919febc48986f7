// Prefill through per-head keys and values ("GatedMLA" docs, "Build per-head
// Q, K and V": K_h = [c W_UK[h]^T | k_rope], the rope key shared by every
// head, V_h = c W_UV[h]; "Observe logits, then compute causal attention").
// For long new-token spans this costs far fewer FLOPs than attending on the
// latent rows (scores over 192 instead of 576 values, P V over 128 instead
// of 512), at the price of materialising K and V once per call (the
// memory-for-compute trade named in the modeldna "MLA" module).
//
// Pieces: gather the cache rows of each sequence into a dense buffer (zero
// past its length), two batched GEMMs for K_nope and V (in the GEMM file),
// and a causal flash-attention kernel that scales and rotates the queries
// as it loads them and whose output is the layer's per-head output.
//
// Attention kernel: workgroup = (sequence, head, 256 query rows), 8 waves of
// 32 queries.  Per 64-key tile in LDS (K 64 x 192, V 64 x 128; four
// buffers, three tiles in flight):
//   S^T [64 keys x 32 q] = K_tile [64 x 192] Q^T          (32x32x16 MFMAs)
//   O^T [128 x 32 q]    += V_tile^T [128 x 64] P^T [64 x 32 q]
// Computing the transposes puts one query in each lane, so row maxima,
// sums and rescales are per-lane values.  P stays in registers: in a 16-key
// step the S^T accumulator gives lane l (h = l/32) keys 4h .. 4h+3 and
// 8+4h .. 8+4h+3, which is the second product's k order once the V^T
// fragments are read from those same key rows (a permutation of the 16 keys
// of the step, applied to both operands).  Scores are in base 2 (the
// queries carry scale * log2 e).
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kQH = 1;                        // 32-query halves per wave
constexpr int kQW = 32 * kQH;                 // queries per wave
constexpr int kFW = 8 / kQH;                  // waves per workgroup
constexpr int kFThreads = 64 * kFW;
constexpr int kFQ = kQW * kFW;                // queries per workgroup
constexpr int kFK = 64;                       // keys per tile
constexpr int kNDn = 128, kNDr = 64, kNDk = kNDn + kNDr, kNDv = 128;
constexpr int kKS = kNDk / 16;                // 12 k steps of S^T
constexpr int kKCh = kNDk * 2 / 16;           // 24 chunks per K row (384 B)
constexpr int kVCh = kNDv * 2 / 16;           // 16 chunks per V row (256 B)
constexpr int kKBytes = kFK * kNDk * 2;       // 24576
constexpr int kVBytes = kFK * kNDv * 2;       // 16384
constexpr int kTBytes = kKBytes + kVBytes;    // 40960
constexpr int kFBuf = 4;                      // tile buffers
constexpr int kTLoads = kTBytes / 1024;       // 40 one-KB load instructions per tile
constexpr int kWLoads = kTLoads / kFW;        // 10 per wave
static_assert(kWLoads * kFW == kTLoads, "tile loads split evenly");
constexpr int kFLds = kFBuf * kTBytes;
static_assert(kFLds <= 163840, "LDS budget");
constexpr int kFSStride = kNDv + 8;           // bf16 per staged output row
static_assert(kFW * kQW * kFSStride * 2 <= kFLds, "output staging fits the tile buffers");
constexpr float kFSlack = 8.0f;               // lazy rescale threshold (log2 units)

// The LDS serves a 16-byte read 16 lanes (256 bytes) at a time and an
// 8-byte read 32 lanes at a time.  K row t (384 B, 128 mod 256): chunk k
// (24 per row) at position k ^ f(t) within its group of 8, f(t) = 4 ((t/2)
// % 2) + (t/4) % 4, so 16 consecutive rows of a fragment read hit 16
// distinct bank slots.  V row t (256 B): chunk k (16 per row) at position
// k ^ 4 (t % 4), so the 4 rows x 4 chunks of a transposing read do.
__device__ __forceinline__ uint32_t k_swz(uint32_t t) { return (((t >> 1) & 1u) << 2) | ((t >> 2) & 3u); }
__device__ __forceinline__ uint32_t k_pos(uint32_t t, uint32_t k) { return k ^ k_swz(t); }
__device__ __forceinline__ uint32_t v_pos(uint32_t t, uint32_t k) { return k ^ ((t & 3u) << 2); }

// This wave's share of one tile's loads: instruction j fills slots
// [64 j, 64 j + 64); slots [0, 1536) are K (row t = s / 24), the rest V.
// Each lane's source pointer for the first tile is set up once; issuing a
// tile advances it by 64 rows, of the latent rows (rope chunks, bit i of
// `rope`) or of the per-head rows.  Keys past a sequence's length are zero
// rows of the buffers, so every address is in bounds.
struct KvSource {
  const bf16* p[kWLoads];
  uint32_t rope;  // bit i: load i reads the rope key from the latent rows

  __device__ __forceinline__ void setup(const bf16* kn, const bf16* cg, const bf16* vv, long row0,
                                        int H, int h, int wave, int lane) {
    rope = 0;
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
      const uint32_t j = (uint32_t)(wave * kWLoads + i);
      const uint32_t s = 64u * j + (uint32_t)lane;
      if (s < (uint32_t)(kFK * kKCh)) {
        const uint32_t t = s / kKCh, k = k_pos(t, s % kKCh);
        const long r = row0 + t;
        if (k < 16) {
          p[i] = kn + (r * H + h) * kNDn + k * 8;
        } else {
          p[i] = cg + r * 576 + 512 + (k - 16) * 8;
          rope |= 1u << i;
        }
      } else {
        const uint32_t sv = s - kFK * kKCh;
        const uint32_t t = sv / kVCh, k = v_pos(t, sv % kVCh);
        p[i] = vv + ((row0 + t) * H + h) * kNDv + k * 8;
      }
    }
  }
  // issue the next tile into `buf` (per-head rows: H * 128 elements, the
  // same for K_nope and V)
  __device__ __forceinline__ void issue(uint32_t buf, int wave, int H) {
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
      g2lds16(p[i], buf + (uint32_t)(wave * kWLoads + i) * 1024u);
      p[i] += ((rope >> i) & 1u) ? (size_t)kFK * 576 : (size_t)kFK * H * kNDn;
    }
  }
};

// Wait for this wave's tile loads except those of its c most recent tiles.
__device__ __forceinline__ void wait_tiles(int c) {
  static_assert(kFBuf <= 4, "up to two later tiles in flight");
  if (c >= 2)
    wait_vmcnt<2 * kWLoads>();
  else if (c == 1)
    wait_vmcnt<kWLoads>();
  else
    wait_vmcnt<0>();
}

// K fragment (S^T A operand) of k step ks, 32-key block kb: the lane's base
// address for ks % 4 plus 128 bytes per 4 steps and 32 rows per block.
__device__ __forceinline__ void read_k(bf16x8& o, uint32_t a, int ks, int kb) {
  switch (2 * (ks >> 2) + kb) {
    case 0: ds_b128_nowait<0>(o, a); break;
    case 1: ds_b128_nowait<32 * kKCh * 16>(o, a); break;
    case 2: ds_b128_nowait<128>(o, a); break;
    case 3: ds_b128_nowait<128 + 32 * kKCh * 16>(o, a); break;
    case 4: ds_b128_nowait<256>(o, a); break;
    default: ds_b128_nowait<256 + 32 * kKCh * 16>(o, a); break;
  }
}
// V^T fragment half of 16-key step ks: 16 rows of V per step
__device__ __forceinline__ void read_v(bf16x4& o, uint32_t a, int ks) {
  switch (ks) {
    case 0: ds_tr_nowait<0>(o, a); break;
    case 1: ds_tr_nowait<16 * kVCh * 16>(o, a); break;
    case 2: ds_tr_nowait<32 * kVCh * 16>(o, a); break;
    default: ds_tr_nowait<48 * kVCh * 16>(o, a); break;
  }
}

// Workgroup = (sequence, head, 256 query rows), 8 waves of 32 queries (a
// lane owns query lane%32), two waves per SIMD.  Per 64-key tile:
//   S^T = K Q^T                 24 MFMAs per wave, K fragments read one step ahead
//   causal mask, row maxima, lazy rescale (VALU)
//   O^T += V^T P^T              4 steps of 16 keys, 4 MFMAs each
// The weights P of 16-key step ks + 1 (8 exponentials per lane) are
// computed while the MFMAs of step ks run, and the V^T fragments of step
// ks + 1 are read as soon as step ks's MFMAs have taken theirs.  LDS reads
// are issued without a wait and completed by waits that name their
// registers (the compiler's own reads would wait for the tile loads in
// flight).  Tiles go through four buffers, three in flight; the barrier at
// the top of tile k frees tile k - 1's buffer for tile k + 3.
// Measured on MI355X (the 2 x 4096 prefill at 64 heads): the LDS serves
// 16-byte reads at about 190 bytes per clock per CU and transposing 8-byte
// reads at about 100, so the K and V^T fragment reads of the 8 waves
// (192 + 128 KB per tile) occupy the LDS for about as long as the MFMAs
// take; 64 queries per wave would halve them, but then the registers of
// one wave (queries, O and S for 64 rows) no longer fit without spills.
__global__ void __launch_bounds__(kFThreads, 1) flash_prefill_kernel(
    const bf16* __restrict__ q, const float* __restrict__ rope, float alpha,
    const bf16* __restrict__ kn, const bf16* __restrict__ cg, const bf16* __restrict__ vv,
    const int* __restrict__ start_pos, int B, int T, int H, int ctx_pad,
    bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char smem[kFLds];
  const uint32_t lds = lds_addr(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // longest query blocks first; a (sequence, head) stays on one XCD
  const int nqb = (T + kFQ - 1) / kFQ;
  const int bh = blockIdx.x % (B * H);
  const int qb = nqb - 1 - blockIdx.x / (B * H);
  const int b = bh / H, h = bh % H;
  const int sp = start_pos[b];
  const int q0 = qb * kFQ;
  const int last = min(q0 + kFQ, T) - 1;                 // last query row of the block
  const int n = (sp + last) / kFK + 1;                  // key tiles the block needs
  const long row0 = (long)b * ctx_pad;

  // this wave's queries (rows past T repeat the last one; not stored)
  const int qw0 = q0 + kQW * wave;
  const bool wave_live = qw0 < T;
  const int wave_last = sp + min(qw0 + kQW - 1, T - 1);  // largest position in the wave
  const int kw = wave_live ? min(wave_last / kFK, n - 1) : -1;  // its last tile with a live key
  int pos[kQH];
  int tq[kQH];
#pragma unroll
  for (int qh = 0; qh < kQH; ++qh) {
    tq[qh] = min(qw0 + 32 * qh + (lane & 31), T - 1);
    pos[qh] = sp + tq[qh];
  }

  KvSource src;
  src.setup(kn, cg, vv, row0, H, h, wave, lane);
  src.issue(lds, wave, H);
  // This lane's query fragments (B operand of S^T): dims 16 ks + 8 (lane/32)
  // .. + 7 of head h, straight from the query projection; the rope dims
  // (ks >= 8) are rotated here (dim i of the rope part pairs with i + 32,
  // two steps further in the same lane) and all are scaled by alpha.
  bf16x8 qf[kQH][kKS];
  f32x4 cs[kQH][4], sn[kQH][4];  // cos, sin of the lane's 16 rope angles per half
#pragma unroll
  for (int qh = 0; qh < kQH; ++qh) {
    const bf16* qr = q + (((long)b * T + tq[qh]) * H + h) * kNDk + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[qh][ks] = *(const bf16x8*)(qr + 16 * ks);
    const float* rc = rope + (long)pos[qh] * kNDr + 8 * (lane >> 5);
    const float* rs = rc + kNDr / 2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {  // ks = 8 + e: angles 16 e + 8 (lane/32) + j
      cs[qh][2 * e] = *(const f32x4*)(rc + 16 * e);
      cs[qh][2 * e + 1] = *(const f32x4*)(rc + 16 * e + 4);
      sn[qh][2 * e] = *(const f32x4*)(rs + 16 * e);
      sn[qh][2 * e + 1] = *(const f32x4*)(rs + 16 * e + 4);
    }
  }
  for (int t = 1; t < min(n, kFBuf - 1); ++t) src.issue(lds + (uint32_t)t * kTBytes, wave, H);
  wait_tiles(min(n, kFBuf - 1) - 1);  // tile 0 and the queries have landed
#pragma unroll
  for (int qh = 0; qh < kQH; ++qh) {
    const float* c = (const float*)cs[qh];
    const float* sv = (const float*)sn[qh];
#pragma unroll
    for (int ks = 0; ks < kNDn / 16; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[qh][ks][j] = (bf16)(alpha * (float)qf[qh][ks][j]);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (float)qf[qh][8 + e][j], y = (float)qf[qh][10 + e][j];
        const float co = c[8 * e + j], si = sv[8 * e + j];
        qf[qh][8 + e][j] = (bf16)(alpha * (x * co - y * si));
        qf[qh][10 + e][j] = (bf16)(alpha * (y * co + x * si));
      }
  }

  // per-lane LDS offsets.  K fragment: row 32 kb + lane%32, chunk
  // 2 ks + lane/32 -> position 8 (ks/4) + ((2 (ks%4) + lane/32) ^ f(row)).
  const uint32_t hi = lane >> 5, fk = k_swz(lane & 31);
  uint32_t k_off[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) k_off[q4] = ((lane & 31) * kKCh + ((2u * q4 + hi) ^ fk)) * 16u;
  // V^T fragment (transposing reads): group g, lane li = 4a + bb reads key
  // row 4 (g/2) + 8 hh + a (+ 16 ks; hh: first or second 4 keys of the
  // lane's k order), dv chunk 4 db + 2 (g%2) + bb/2 at position chunk ^ 4a,
  // plus 8 bytes for odd bb.
  const uint32_t g = lane >> 4, li = lane & 15, a4 = li >> 2, bb = li & 3;
  uint32_t v_off[8];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t row = 4u * (g >> 1) + 8u * hh + a4;
      const uint32_t ch = 4u * db + 2u * (g & 1) + (bb >> 1);
      v_off[2 * db + hh] = kKBytes + (row * kVCh + (ch ^ (a4 << 2))) * 16u + 8u * (bb & 1);
    }

  f32x16 o[kQH][4];
#pragma unroll
  for (int qh = 0; qh < kQH; ++qh)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qh][db] = f32x16{};
  float m[kQH], l[kQH];
#pragma unroll
  for (int qh = 0; qh < kQH; ++qh) {
    m[qh] = -INFINITY;
    l[qh] = 0.f;
  }
  f32x16 sacc[kQH][2];

  // S^T = K Q^T for the tile in kbuf, the K fragments read two steps ahead
  auto scores = [&](uint32_t kbuf) {
    uint32_t ka[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) ka[q4] = kbuf + k_off[q4];
    bf16x8 fr[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) read_k(fr[0][kb], ka[0], 0, kb);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if (ks + 1 < kKS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) read_k(fr[(ks + 1) & 1][kb], ka[(ks + 1) & 3], ks + 1, kb);
        lds_settle<2>(fr[ks & 1][0], fr[ks & 1][1]);
      } else {
        lds_settle<0>(fr[ks & 1][0], fr[ks & 1][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qh = 0; qh < kQH; ++qh)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sacc[qh][kb] = mfma32(fr[ks & 1][kb], qf[qh][ks], ks == 0 ? f32x16{} : sacc[qh][kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int k = 0; k < n; ++k) {
    wait_tiles(min(n - 1 - k, kFBuf - 2));
    lds_barrier();  // tile k visible; tile k - 1 consumed by every wave
    if (k + kFBuf - 1 < n)
      src.issue(lds + (uint32_t)((k + kFBuf - 1) % kFBuf) * kTBytes, wave, H);
    if (k > kw) continue;  // every key of the tile is masked for the wave
    const uint32_t buf = lds + (uint32_t)(k % kFBuf) * kTBytes;
    scores(buf);

    // the first V^T fragments go out before the softmax needs the scores
    uint32_t va[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) va[i] = buf + v_off[i];
    bf16x4 vt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) read_v(vt[i], va[i], 0);

    // causal mask, only where the tile reaches past the wave's first query;
    // register v of block kb <-> key key0 + 32 kb + 8 (v/4) + 4 hi + v%4
    const int key0 = k * kFK;
    if (key0 + kFK - 1 > sp + qw0) {
#pragma unroll
      for (int qh = 0; qh < kQH; ++qh) {
        const int lim = pos[qh] - key0 - 4 * (int)hi;  // mask where 32 kb + 8 (v/4) + v%4 > lim
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * kb + 8 * (v >> 2) + (v & 3) > lim) sacc[qh][kb][v] = -INFINITY;
      }
    }
    // row maxima over the tile's 64 keys (32 in this lane, 32 in lane ^ 32)
    float m_new[kQH], al[kQH];
    bool grow_any = false;
#pragma unroll
    for (int qh = 0; qh < kQH; ++qh) {
      float hm = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) hm = fmaxf(hm, sacc[qh][kb][v]);
      hm = max_xor32(hm);
      const bool grow = hm > m[qh] + kFSlack;
      m_new[qh] = grow ? hm : m[qh];
      al[qh] = grow ? fast_exp2(m[qh] - m_new[qh]) : 1.0f;
      grow_any = grow_any || grow;
    }
    if (__ballot(grow_any) != 0ull) {
#pragma unroll
      for (int qh = 0; qh < kQH; ++qh)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[qh][db][v] *= al[qh];
    }
    // P^T of 16-key step ks for half qh: registers 8 (ks%2) .. + 7 of block ks/2
    float psum[kQH];
#pragma unroll
    for (int qh = 0; qh < kQH; ++qh) psum[qh] = 0.f;
    bf16x8 pr[2][kQH];  // [step parity][half]
    auto weights = [&](int ks, bf16x8 (&dst)[kQH]) {
#pragma unroll
      for (int qh = 0; qh < kQH; ++qh)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pv = fast_exp2(sacc[qh][ks >> 1][8 * (ks & 1) + j] - m_new[qh]);
          psum[qh] += pv;
          dst[qh][j] = (bf16)pv;
        }
    };
    weights(0, pr[0]);
#pragma unroll
    for (int ks = 0; ks < kFK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) lds_settle<0>(vt[i], vt[i + 1]);
      __builtin_amdgcn_sched_barrier(0);
      // step ks's MFMAs; the next step's fragments are read as soon as the
      // MFMAs have taken these (the reads land long after the MFMAs read
      // their operands), and its weights are computed beside them
#pragma unroll
      for (int qh = 0; qh < kQH; ++qh)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          o[qh][db] = mfma32(cat(vt[2 * db], vt[2 * db + 1]), pr[ks & 1][qh], o[qh][db]);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < kFK / 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) read_v(vt[i], va[i], ks + 1);
        __builtin_amdgcn_sched_barrier(0);
        weights(ks + 1, pr[(ks + 1) & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qh = 0; qh < kQH; ++qh) {
      l[qh] = l[qh] * al[qh] + psum[qh];
      m[qh] = m_new[qh];
    }
  }

  // ---- out[b, t, h, :] = O / l, staged per wave in the (idle) tile buffers
  float inv[kQH];
#pragma unroll
  for (int qh = 0; qh < kQH; ++qh) {
    const float lt = sum_xor32(l[qh]);
    inv[qh] = lt > 0.f ? 1.0f / lt : 0.f;
  }
  lds_barrier();  // every wave is done with the tile buffers
  typedef __attribute__((address_space(3))) bf16x4 lds_b4;
  const uint32_t st = lds + wave * kQW * kFSStride * 2;
#pragma unroll
  for (int qh = 0; qh < kQH; ++qh)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 w4;
#pragma unroll
        for (int r = 0; r < 4; ++r) w4[r] = (bf16)(o[qh][db][4 * q4 + r] * inv[qh]);
        const int row = 32 * qh + (lane & 31);
        *(lds_b4*)(uintptr_t)(st + (row * kFSStride + 32 * db + 8 * q4 + 4 * hi) * 2) = w4;
      }
  // each wave writes its 64 rows (256 B each) with 16-byte stores
#pragma unroll
  for (int i = 0; i < kQW * kVCh / 64; ++i) {
    const int c = i * 64 + lane;
    const int r = c / kVCh, ch = c % kVCh;
    const int t = qw0 + r;
    const bf16x8 v8 = lds_read_b128(st + (r * kFSStride + 8 * ch) * 2);
    if (t < T) *(bf16x8*)(out + (((long)b * T + t) * H + h) * kNDv + 8 * ch) = v8;
  }
}

// Dense copy of each sequence's cache rows 0 .. start_pos + T - 1 (zero past
// that, up to ctx_pad): one thread per 16-byte chunk.
__global__ void __launch_bounds__(256) gather_rows_kernel(
    const bf16* __restrict__ pool, const int* __restrict__ block_table, int max_blocks, int shift,
    const int* __restrict__ start_pos, int T, int ctx_pad, long total, bf16* __restrict__ dst) {
  constexpr int kChunks = 576 / 8;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long row = i / kChunks;
  const int c = (int)(i - row * kChunks);
  const int b = (int)(row / ctx_pad), j = (int)(row - (long)b * ctx_pad);
  bf16x8 v = {};
  if (j < start_pos[b] + T) {
    const int page = block_table[(long)b * max_blocks + (j >> shift)];
    const long r = ((long)page << shift) + (j & ((1 << shift) - 1));
    v = *(const bf16x8*)(pool + r * 576 + c * 8);
  }
  *(bf16x8*)(dst + row * 576 + c * 8) = v;
}

// The same rows from an FP8 cache (656-byte rows: 512 E4M3 codes, 64 bf16
// rope values, the float32 power-of-two scale), widened to bf16 rows.  scale
// times a code is exact in bf16 (3 mantissa bits, a power-of-two factor), so
// the rows match what the decode path reads.  One thread per 8 values.
__global__ void __launch_bounds__(256) gather_rows_fp8_kernel(
    const unsigned char* __restrict__ pool, const int* __restrict__ block_table, int max_blocks,
    int shift, const int* __restrict__ start_pos, int T, int ctx_pad, long total,
    bf16* __restrict__ dst) {
  constexpr int kChunks = 576 / 8, kRow = 656;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long row = i / kChunks;
  const int c = (int)(i - row * kChunks);
  const int b = (int)(row / ctx_pad), j = (int)(row - (long)b * ctx_pad);
  bf16x8 v = {};
  if (j < start_pos[b] + T) {
    const int page = block_table[(long)b * max_blocks + (j >> shift)];
    const unsigned char* src = pool + (((long)page << shift) + (j & ((1 << shift) - 1))) * kRow;
    if (c < 64) {
      const float sc = *(const float*)(src + 640);
      const uint2 raw = *(const uint2*)(src + c * 8);
      const uint32_t w[2] = {raw.x, raw.y};
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], sc, false);
        const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], sc, true);
        v[4 * d + 0] = lo[0];
        v[4 * d + 1] = lo[1];
        v[4 * d + 2] = hi[0];
        v[4 * d + 3] = hi[1];
      }
    } else {
      v = *(const bf16x8*)(src + 512 + (c - 64) * 16);
    }
  }
  *(bf16x8*)(dst + row * 576 + c * 8) = v;
}

}  // namespace

void launch_gather_rows(const void* pool, const int* block_table, int max_blocks, int shift,
                        const int* start_pos, int batch, int T, int ctx_pad, void* dst,
                        bool fp8, hipStream_t st) {
  const long chunks = (long)batch * ctx_pad * (576 / 8);
  if (fp8) {
    gather_rows_fp8_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>(
        (const unsigned char*)pool, block_table, max_blocks, shift, start_pos, T, ctx_pad, chunks,
        (bf16*)dst);
    return;
  }
  gather_rows_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>(
      (const bf16*)pool, block_table, max_blocks, shift, start_pos, T, ctx_pad, chunks,
      (bf16*)dst);
}

void launch_flash_prefill(const void* q, const float* rope, float alpha, const void* kn,
                          const void* cg, const void* v, const int* start_pos, int batch, int T,
                          int H, int ctx_pad, void* out, hipStream_t st) {
  const int nqb = (T + kFQ - 1) / kFQ;
  flash_prefill_kernel<<<batch * H * nqb, kFThreads, 0, st>>>(
      (const bf16*)q, rope, alpha, (const bf16*)kn, (const bf16*)cg, (const bf16*)v, start_pos,
      batch, T, H, ctx_pad, (bf16*)out);
}

}  // namespace mla
