// Shared device-side types and helpers of the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bfloat16, round to nearest even
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// Store 4 consecutive values of type T from fp32 (one 8- or 16-byte store).
__device__ __forceinline__ void store4(float* p, const float v[4]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void store4(bf16* p, const float v[4]) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{from_f32<bf16>(v[0]), from_f32<bf16>(v[1]),
                                           from_f32<bf16>(v[2]), from_f32<bf16>(v[3])};
}

// Load 8 consecutive elements as floats.
__device__ __forceinline__ void load8(const bf16* p, float out[8]) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = static_cast<float>(v[i]);
}
__device__ __forceinline__ void load8(const float* p, float out[8]) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
    out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
}

// 16-byte load of data read once per call (the KV cache in decode), marked nontemporal.  On
// MI355X a stream of such loads, each wave instruction one contiguous 1 KB run, measured
// 7.2 TB/s against 6.0 TB/s with plain loads; with 64-byte pieces per row there was no gain.
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4): lane i
// of the wave writes LDS bytes [lds + 16 i, lds + 16 i + 16).  Issued from inline asm so
// that the compiler does not serialise every later LDS read behind it; completion is
// tracked by hand with s_waitcnt vmcnt (the copy has no VGPR result).
__device__ __forceinline__ void lds_dma16(const void* gptr, unsigned lds_byte) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_byte)), "v"(gptr)
                 : "memory");
}

// The same copy addressed as a 64-bit base in scalar registers plus a 32-bit byte offset
// per lane (the base and the LDS address must be uniform across the wave).
__device__ __forceinline__ void lds_dma16_s(const void* sbase, unsigned voff, unsigned lds_byte) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_byte), "v"(voff), "s"(sbase)
                 : "memory");
}

// Wait until this wave's copies into LDS have landed and its own LDS reads have returned,
// then synchronise the workgroup: after it every wave's copies are visible and no wave still
// reads a buffer that a copy issued next may overwrite.  (A read's data being consumed later
// in program order is no guarantee: the compiler may move the consuming instructions past the
// barrier.)
__device__ __forceinline__ void wait_copies_and_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Wait for this wave's LDS operations, then synchronise the workgroup (outstanding global
// loads stay in flight).
__device__ __forceinline__ void wait_lgkm_and_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// LDS byte address of a __shared__ (address space 3) pointer, for the m0 of lds_dma16.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// Device error flags, OR-ed into a word of the workspace and read by llama_sync_status.
enum : uint32_t { DEVERR_TOKEN_RANGE = 1u, DEVERR_NAN_LOGIT = 2u, DEVERR_POSITION_RANGE = 4u };
