// Measurement probes: the ceilings the kernels of this library are judged
// against, measured on the device at hand rather than taken from data
// sheets.  Not part of the method.
//   hbm_read_kernel:  every lane streams 16-byte loads over a buffer far
//                     larger than the caches (vector loads into registers);
//   dma_read_kernel:  the same bytes through direct-to-LDS loads into four
//                     rotating LDS buffers, as the decode attention moves its
//                     tiles (one workgroup per CU, 512 threads);
//   mfma_kernel:      back-to-back independent 32x32x16 bf16 MFMAs on
//                     register operands (one 256-thread workgroup per CU
//                     slot, four accumulators per wave);
//   lds_read_kernel:  LDS reads of 16 or 8 bytes per lane, eight in flight
//                     per wave, bank-conflict free, by one 512-thread
//                     workgroup per CU (the decode attention's shape).
#include "device_common.h"
#include "mla.h"

namespace mla {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(512) hbm_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                       uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t x = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^
         d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// Workgroup w streams chunks w, w + G, ... of 36 KB (the decode tile size)
// through four LDS buffers, two in flight while two are "read".
constexpr int kProbeTile = 36864;
__global__ void __launch_bounds__(512, 1) dma_read_kernel(const unsigned char* __restrict__ src,
                                                          size_t n_tiles,
                                                          uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kProbeTile];
  const uint32_t lds = lds_addr(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t G = gridDim.x;
  // each wave issues 36864 / (8 * 1024) = 4.5 loads per tile: waves 0..3
  // issue 5, waves 4..7 issue 4 (36 one-KB loads in all)
  const int j0 = wave < 4 ? 5 * wave : 20 + 4 * (wave - 4);
  const int nl = wave < 4 ? 5 : 4;
  auto issue = [&](size_t t, int slot) {
    const unsigned char* p = src + t * kProbeTile;
    for (int i = 0; i < nl; ++i)
      g2lds16(p + (size_t)(j0 + i) * 1024 + lane * 16, lds + slot * kProbeTile + (j0 + i) * 1024);
  };
  size_t k = 0;
  const size_t mine = blockIdx.x < n_tiles ? (n_tiles - blockIdx.x + G - 1) / G : 0;
  if (mine > 0) issue(blockIdx.x, 0);
  if (mine > 1) issue(blockIdx.x + G, 1);
  uint32_t x = 0;
  for (k = 0; k < mine; ++k) {
    // this wave's loads of tile k landed (tile k+1's may stay in flight)
    if (k + 1 < mine) {
      if (nl == 5) wait_vmcnt<5>(); else wait_vmcnt<4>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (k + 2 < mine) issue(blockIdx.x + (k + 2) * G, (int)((k + 2) & 3));
    // touch one value of the landed tile so the loads have a consumer (an
    // LDS read of the compiler's own would first wait for every load in
    // flight)
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v)
                 : "v"(lds + (uint32_t)(k & 3) * kProbeTile + threadIdx.x * 4u));
    x ^= v;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

__global__ void __launch_bounds__(256) mfma_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (bf16)(0.001f * (float)(threadIdx.x + k));
    b[k] = (bf16)(0.002f * (float)(threadIdx.x - k));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each wave reads rows of 64 x W bytes (W = 16 or 8) at consecutive
// addresses, eight per iteration, all below 64 KB of a 96 KB allocation
// (which keeps the workgroup alone on its CU); 64 consecutive lanes of one
// read touch every bank equally, so the reads are conflict free.
constexpr int kProbeLds = 96 * 1024;
template <int W>
__global__ void __launch_bounds__(512, 1) lds_read_kernel(int iters, uint32_t* __restrict__ sink) {
  typedef unsigned v4 __attribute__((ext_vector_type(4)));
  typedef unsigned v2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v4 lds_v4;
  typedef __attribute__((address_space(3))) v2 lds_v2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kProbeLds];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kProbeLds / 4; i += 512) ((uint32_t*)smem)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const uint32_t base = lds_addr(smem) + (uint32_t)wave * 8192u + (uint32_t)lane * W;
  uint32_t x = 0;
  for (int it = 0; it < iters; ++it) {
    if constexpr (W == 16) {
      v4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *(volatile lds_v4*)(uintptr_t)(base + j * 1024u);
#pragma unroll
      for (int j = 0; j < 8; ++j) x ^= v[j][0] + v[j][1] + v[j][2] + v[j][3];
    } else {
      v2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *(volatile lds_v2*)(uintptr_t)(base + j * 512u);
#pragma unroll
      for (int j = 0; j < 8; ++j) x ^= v[j][0] + v[j][1];
    }
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace
}  // namespace mla

extern "C" {

size_t mla_probe_sink_bytes(void) { return (size_t)8 * 1024 * 512 * 4; }

mla_status mla_probe_hbm_read(const void* buf, size_t bytes, int32_t mode, void* sink,
                              void* stream) {
  hipStream_t st = (hipStream_t)stream;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (cus <= 0 || cus > 1024) cus = 256;
  if (!buf || !sink || bytes < (size_t)mla::kProbeTile || ((uintptr_t)buf & 15) ||
      (mode != 0 && mode != 1))
    return MLA_ERR_INVALID_ARG;
  if (mode == 0)
    mla::hbm_read_kernel<<<8 * cus, 512, 0, st>>>((const mla::u32x4*)buf, bytes / 16,
                                                  (uint32_t*)sink);
  else
    mla::dma_read_kernel<<<cus, 512, 0, st>>>((const unsigned char*)buf,
                                              bytes / mla::kProbeTile, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_probe_lds_read(int32_t width, int32_t iterations, void* sink, void* stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (cus <= 0 || cus > 1024) cus = 256;
  if (!sink || iterations <= 0 || (width != 16 && width != 8) ||
      (size_t)cus * 512 * 4 > mla_probe_sink_bytes())
    return MLA_ERR_INVALID_ARG;
  if (width == 16)
    mla::lds_read_kernel<16><<<cus, 512, 0, (hipStream_t)stream>>>(iterations, (uint32_t*)sink);
  else
    mla::lds_read_kernel<8><<<cus, 512, 0, (hipStream_t)stream>>>(iterations, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_probe_mfma(int32_t workgroups, int32_t iterations, void* sink, void* stream) {
  if (workgroups <= 0 || iterations <= 0 || !sink ||
      (size_t)workgroups * 256 * 4 > mla_probe_sink_bytes())
    return MLA_ERR_INVALID_ARG;
  mla::mfma_kernel<<<workgroups, 256, 0, (hipStream_t)stream>>>(iterations, (float*)sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
