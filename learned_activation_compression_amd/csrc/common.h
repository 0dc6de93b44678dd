// Device-side helpers shared by the MAPL kernels (gfx950 only).
//
// Matrix-core conventions used throughout (wave64):
//   v_mfma_f32_32x32x16_bf16  A: lane l supplies row  (l & 31), 8 consecutive k (k = 8*(l>>5) + i)
//                             B: lane l supplies col  (l & 31), the same 8 k
//                             D: lane l, register v holds row 8*(v>>2) + 4*(l>>5) + (v&3), col (l & 31)
//   v_mfma_f32_32x32x2_f32    A: lane l supplies row (l & 31), k = (l >> 5)
//                             B: lane l supplies col (l & 31), k = (l >> 5)
//                             D: same layout as above.
// The pairing of k slots between A and B is symmetric, so any consistent
// assignment of contraction indices to k slots gives the same sum.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mapl {

typedef uint16_t bf16_t;  // bf16 storage (raw bits)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

// 16-byte global load of 8 bf16 as an MFMA operand.
__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Wave index within the block as a scalar (wave-uniform) value, so that
// control flow that depends on it compiles to scalar branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Keep an MFMA operand (mask = ~0u) or zero it (mask = 0) without a branch.
__device__ __forceinline__ bf16x8 mask_bf16x8(bf16x8 v, uint32_t m) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u &= u32x4{m, m, m, m};
  return __builtin_bit_cast(bf16x8, u);
}

// Row index (within a 32x32 tile) held by register v of a lane in the upper
// (hi = 1) or lower half-wave, for the 32x32 MFMA output layout.
__device__ __forceinline__ int mfma32_row(int v, int hi) { return 8 * (v >> 2) + 4 * hi + (v & 3); }

// Workgroups are dispatched to the 8 XCDs round-robin (id i to XCD i % 8).
// Renumber them so that each XCD receives a contiguous range of tiles (tiles
// that share operands then share an L2): XCD x holds the ids i = x + 8 j, and
// takes tiles start_x + j, where the first total % 8 XCDs hold one id more
// than the others.  A bijection of [0, total) for any total; only locality,
// never a result, depends on the dispatch order.
__device__ __forceinline__ int xcd_swizzle(int bid, int total) {
  const int x = bid & 7, j = bid >> 3, q = total >> 3, rem = total & 7;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + j;
}

// Lane l copies 16 bytes from g to LDS byte address (l_base + 16 l); l_base is
// uniform over the wave.  Written as inline assembly: the compiler would
// otherwise treat every such copy as a possible write to any LDS the later
// copies and reads touch and wait for all of them, and the ring's order is
// kept here by explicit vmcnt waits and barriers instead.  The "memory"
// clobber keeps every LDS access of the program on its side of the copy.
__device__ __forceinline__ void copy16_to_lds(const void* g, const void* l_base) {
  const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(l_base)));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(la) : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Host side: a kernel launch that, given both events, goes through
// hipExtLaunchKernelGGL so that the events take the kernel's own begin and end
// time stamps (no marker packets between them and the kernel).  Each argument
// is converted to the kernel's parameter type before it is packed.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool armed() const { return start != nullptr && stop != nullptr; }
};

template <typename... Formals, typename... Actuals>
inline void launch_k(KernelEvents ev, void (*k)(Formals...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                     Actuals... a) {
  static_assert(sizeof...(Formals) == sizeof...(Actuals), "argument count");
  if (ev.armed())
    hipExtLaunchKernelGGL(k, grid, block, lds, s, ev.start, ev.stop, 0u, Formals(a)...);
  else
    hipLaunchKernelGGL(k, grid, block, lds, s, Formals(a)...);
}

// LDS of one gfx950 workgroup (static plus dynamic).
constexpr int kMaxLdsBytes = 160 * 1024;

// Host side: kernels launched with more dynamic LDS than the default 64 KB
// limit.  LdsLimit<kernel, BYTES>::bytes() (used at the launch site) fails to
// compile for more than a workgroup can have, and registers the kernel at
// library load; lds_prepare_device() (abi.hip) raises the limit of every
// registered kernel on the current device once, before an entry point's first
// launch, so a refusal by the runtime is reported before anything is enqueued.
void lds_register(const void* kernel, int bytes);
hipError_t lds_prepare_device();

template <auto K, int BYTES>
struct LdsLimit {
  static_assert(BYTES > 0 && BYTES <= kMaxLdsBytes, "dynamic LDS above what a gfx950 workgroup has");
  struct Reg {
    Reg() { lds_register(reinterpret_cast<const void*>(K), BYTES); }
  };
  static inline Reg reg;
  static int bytes() {
    (void)&reg;
    return BYTES;
  }
};

}  // namespace mapl
