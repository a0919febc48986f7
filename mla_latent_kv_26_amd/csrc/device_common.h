// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;

// log2(e): scores are pre-multiplied by it so the softmax uses exp2.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 32x32x16 bf16 MFMA.  Lane l holds A[l%32][8(l/32)+j] and B[8(l/32)+j][l%32];
// accumulator register v of lane l is C[8(v/4) + 4(l/32) + v%4][l%32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 MFMA.  Lane l holds A[l%16][8(l/16)+j] and B[8(l/16)+j][l%16];
// accumulator register v of lane l is C[4(l/16) + v][l%16].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each group of 16 lanes, output lane i element j
// is element (i % 4) of the 8 bytes read by lane 4j + i/4 of that group.  If
// lane 4a + b of a group reads row (r0 + a), columns (c0 + 4b .. c0 + 4b + 3)
// of a row-major 16-bit matrix, lane i receives column c0 + i, rows r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 lds_read_tr(uint32_t byte_addr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(uintptr_t)byte_addr);
  return __builtin_bit_cast(bf16x4, v);
}
// Eight transposing LDS reads at a[i] + OFF, finished before the block ends
// (the wait is inside the asm block, so the outputs are valid when it
// returns).  Unlike the builtin, this does not make the compiler wait for
// in-flight direct-to-LDS loads into other buffers first.
template <int OFF>
__device__ __forceinline__ void lds_read_tr_x8(const uint32_t (&a)[8], bf16x4 (&o)[8]) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "i"(OFF));
}
// LDS reads without a wait, for reads kept in flight across other work: the
// result registers are valid only after an lds_settle that names them (the
// compiler treats an asm output as written when the asm ends, so nothing
// may read or copy them before that wait).  The compiler's own LDS reads
// would make it wait for every direct-to-LDS load in flight first.
template <int OFF>
__device__ __forceinline__ void ds_b128_nowait(bf16x8& o, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(o) : "v"(a), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_tr_nowait(bf16x4& o, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(o) : "v"(a), "i"(OFF));
}
// Waits until at most N LDS operations of this wave are outstanding (they
// complete in issue order) and hands the named registers on as written here.
template <int N, typename T>
__device__ __forceinline__ void lds_settle(T& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
template <int N, typename T>
__device__ __forceinline__ void lds_settle(T& x, T& y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N));
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)byte_addr;
}

typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ float lds_ld(uint32_t a) { return *(lds_f32*)(uintptr_t)a; }
__device__ __forceinline__ f32x4 lds_ld4(uint32_t a) { return *(lds_f32x4*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st(uint32_t a, float v) { *(lds_f32*)(uintptr_t)a = v; }
__device__ __forceinline__ void lds_st(uint32_t a, const bf16x4& v) { *(lds_bf16x4*)(uintptr_t)a = v; }

// Address of a __shared__ object in the LDS aperture.
template <typename T> __device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)p;
}

// A kernel argument past the ones preloaded into scalar registers is a
// scalar load from the argument segment, which the compiler issues and waits
// for where the argument is first used.  fetch_arg makes it a value at this
// point instead (placed where other loads are in flight, its round trip
// overlaps theirs).  The pointer stays a global one, so the accesses through
// it remain global (not flat) loads and stores.
template <typename P> __device__ __forceinline__ void fetch_arg(P& p) {
  typedef std::remove_reference_t<decltype(*p)> T;
  typedef __attribute__((address_space(1))) T gT;
  gT* g = (gT*)p;
  asm volatile("" : "+s"(g));
  p = (T*)g;
}

// Asynchronous 16-byte copy global -> LDS: lane l's 16 bytes land at
// lds_base + 16 * l (lds_base is wave-uniform).
__device__ __forceinline__ void g2lds16(const void* gptr, uint32_t lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void*)(uintptr_t)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4]; lgkmcnt [11:8]).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (a fenced __syncthreads
// would also wait for in-flight direct-to-LDS prefetches).  Callers wait for
// the direct-to-LDS loads they depend on themselves (wait_vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 2^x by the hardware instruction (no denormal range fix-up): results below
// 2^-126 come out as zero, which only drops softmax weights far below
// anything a bf16 probability or a float32 sum can register.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// 1 / (1 + e^-x), saturating to 0 and 1 (2^x is +inf or 0 at the ends)
__device__ __forceinline__ float sigmoid_f(float x) {
  return 1.0f / (1.0f + fast_exp2(-1.4426950408889634f * x));
}

// Lane permutations within rows of 16 lanes (DPP, no LDS traffic; an LDS
// permute would also make the compiler wait for in-flight direct-to-LDS
// loads).  Controls: quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror,
// row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// max / sum of v over lanes l and l ^ 16 (rows of 16 lanes swapped in pairs
// by one permlane16 swap; no LDS traffic).  Both lanes get the same bits.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// max / sum of v over lanes l and l ^ 32 (both lanes get the same bits):
// one permlane32 swap, no LDS traffic.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  // the two registers hold x[l] and x[l ^ 32] in either order; a sum of two
  // is the same bits in either order
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// Reductions over the 64 lanes; every lane gets the same value (each step
// combines a pair of lanes with a commutative operation, so both members of
// a pair hold identical bits).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

}  // namespace mla
