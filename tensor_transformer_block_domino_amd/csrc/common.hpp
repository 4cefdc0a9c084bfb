// Device-side helpers shared by the HIP kernels of the Domino shard library (gfx950).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace domino {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bf16 <-> fp32. A bf16 value is the top half of an fp32; conversion to bf16 rounds to
// nearest, ties to even (v_cvt_pk_bf16_f32, two values per instruction).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Element type traits for the generic (fp32 / bf16) paths.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = uint16_t(f32_to_bf16_bits(v)); }
};

// Activations, written from their definitions. σ(x) = 1 / (1 + e^(−x)), evaluated as
// rcp(1 + 2^(−x·log2 e)) (v_exp_f32, v_rcp_f32: about 1 ulp each). The tanh-form GeLU
// uses 0.5·(1 + tanh(u)) = σ(2u) with u = √(2/π)·(x + 0.044715·x³), so
// gelu(x) = x·σ(2u) and, with s = σ(2u) and 1 − tanh²(u) = 4·s·(1 − s),
// gelu'(x) = s + x·s·(1 − s)·2√(2/π)·(1 + 3·0.044715·x²).
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

constexpr float kGeluA = 2.0f * 0.7978845608028654f;  // 2·√(2/π): 2u = x·(A + B·x²)
constexpr float kGeluB = kGeluA * 0.044715f;
constexpr float kGeluC = kGeluA * 3.0f * 0.044715f;   // d(2u)/dx = A + C·x²

__device__ __forceinline__ float gelu_tanh_f(float x) { return x * sigmoidf_(x * fmaf(kGeluB, x * x, kGeluA)); }

__device__ __forceinline__ float gelu_tanh_grad_f(float x) {
  const float x2 = x * x;
  const float s = sigmoidf_(x * fmaf(kGeluB, x2, kGeluA));
  return fmaf(s, x * (1.0f - s) * fmaf(kGeluC, x2, kGeluA), s);
}

__device__ __forceinline__ float silu_f(float x) { return x * sigmoidf_(x); }

// Global → LDS copies are buffer loads that write LDS directly (no registers): lane l of
// one instruction writes 16 bytes at LDS address base + 16·l, so a wave instruction
// fills one contiguous 1 KB block, and each lane picks which 16-byte chunk of the tile it
// fetches. A lane outside the matrix uses byte offset kOOB; the buffer range check turns
// it into zeros written to LDS, without a branch.
constexpr int32_t kOOB = int32_t(0x80000000u);
constexpr int32_t kRangeBytes = 0x7fffffff;
constexpr int32_t kRsrcWord3 = 0x00020000;

// The descriptor must be wave-uniform (scalar registers); the compiler cannot always
// prove that of a pointer kept in a per-thread struct, and would then wrap every load in
// a loop over lanes. readfirstlane states the uniformity explicitly.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  void* b = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, kRangeBytes, kRsrcWord3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint16_t* lds, int32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// LDS byte address of a pointer into a __shared__ array (for inline-assembly LDS reads).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// LDS reads as inline assembly: the compiler neither reorders them against other inline
// assembly nor inserts waits for them, so every use must follow an explicit lgkmcnt wait
// that ties the destination (lgkm_wait_tied, or a wait plus empty "+v" asm statements).
__device__ __forceinline__ void lds_read_b128(u32x4_t& d, const void* p) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(d) : "v"(lds_addr(p)));
}
__device__ __forceinline__ void lds_read_tr16_b64(u32x2_t& d, const void* p) {
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(d) : "v"(lds_addr(p)));
}

// Waits until at most n (0..15) LDS operations of this wave are in flight, tying a and b
// (their consumers stay after the wait). n is a constant after unrolling, so the switch
// folds to one instruction.
__device__ __forceinline__ void lgkm_wait_tied(int n, u32x4_t& a, u32x4_t& b) {
  switch (n) {
    case 0: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b)); break;
    case 1: asm volatile("s_waitcnt lgkmcnt(1)" : "+v"(a), "+v"(b)); break;
    case 2: asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(a), "+v"(b)); break;
    case 3: asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(a), "+v"(b)); break;
    case 4: asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(a), "+v"(b)); break;
    case 5: asm volatile("s_waitcnt lgkmcnt(5)" : "+v"(a), "+v"(b)); break;
    case 6: asm volatile("s_waitcnt lgkmcnt(6)" : "+v"(a), "+v"(b)); break;
    case 7: asm volatile("s_waitcnt lgkmcnt(7)" : "+v"(a), "+v"(b)); break;
    case 8: asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(a), "+v"(b)); break;
    case 9: asm volatile("s_waitcnt lgkmcnt(9)" : "+v"(a), "+v"(b)); break;
    case 10: asm volatile("s_waitcnt lgkmcnt(10)" : "+v"(a), "+v"(b)); break;
    case 11: asm volatile("s_waitcnt lgkmcnt(11)" : "+v"(a), "+v"(b)); break;
    case 12: asm volatile("s_waitcnt lgkmcnt(12)" : "+v"(a), "+v"(b)); break;
    case 13: asm volatile("s_waitcnt lgkmcnt(13)" : "+v"(a), "+v"(b)); break;
    case 14: asm volatile("s_waitcnt lgkmcnt(14)" : "+v"(a), "+v"(b)); break;
    case 15: asm volatile("s_waitcnt lgkmcnt(15)" : "+v"(a), "+v"(b)); break;
    default: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b)); break;
  }
}

// The same wait tying one register group.
__device__ __forceinline__ void lgkm_wait_tied1(int n, u32x4_t& a) {
  switch (n) {
    case 0: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a)); break;
    case 1: asm volatile("s_waitcnt lgkmcnt(1)" : "+v"(a)); break;
    case 2: asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(a)); break;
    case 3: asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(a)); break;
    case 4: asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(a)); break;
    case 5: asm volatile("s_waitcnt lgkmcnt(5)" : "+v"(a)); break;
    case 6: asm volatile("s_waitcnt lgkmcnt(6)" : "+v"(a)); break;
    case 7: asm volatile("s_waitcnt lgkmcnt(7)" : "+v"(a)); break;
    case 8: asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(a)); break;
    case 9: asm volatile("s_waitcnt lgkmcnt(9)" : "+v"(a)); break;
    case 10: asm volatile("s_waitcnt lgkmcnt(10)" : "+v"(a)); break;
    case 11: asm volatile("s_waitcnt lgkmcnt(11)" : "+v"(a)); break;
    case 12: asm volatile("s_waitcnt lgkmcnt(12)" : "+v"(a)); break;
    case 13: asm volatile("s_waitcnt lgkmcnt(13)" : "+v"(a)); break;
    case 14: asm volatile("s_waitcnt lgkmcnt(14)" : "+v"(a)); break;
    case 15: asm volatile("s_waitcnt lgkmcnt(15)" : "+v"(a)); break;
    default: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a)); break;
  }
}

// Wait until at most N vector-memory operations of this wave are in flight and all its
// LDS operations are done, then barrier. A workgroup fence would wait for every LDS
// write in flight (vmcnt(0)), which serialises the stage ring, so the wait is explicit.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace domino

// Every kernel launch of the library: a plain launch, or while a call is timed the extended
// launch that records that call's events with the kernel's own start and end.
#define DOMINO_LAUNCH(kernel, grid, block, lds, stream, ...)                                        \
  do {                                                                                              \
    ::domino::LaunchEvents& ev_ = ::domino::launch_events();                                        \
    if (ev_.stop) {                                                                                 \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev_.start, ev_.stop, 0, __VA_ARGS__); \
      ev_.start = nullptr;                                                                          \
    } else {                                                                                        \
      hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                            \
    }                                                                                               \
  } while (0)
