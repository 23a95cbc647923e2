// mhc_device.h -- device helpers shared by the kernel files: vector types, bf16 bit
// conversions, an explicit vector-memory wait, and raw buffer resources.
//
// Everything is in an unnamed namespace inside mhc: each translation unit that includes
// it gets its own internal copy (no device symbols cross translation units).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mhc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits by the hardware conversion (v_cvt_pk_bf16_f32 on gfx950): round to
// nearest, ties to even, in the default rounding mode; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats -> a packed bf16 pair (lo in bits 0-15), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ double bf16_bits_to_double(uint32_t b)
{
    return (double)__uint_as_float(b << 16);
}

// binary16 (fp16) storage of x and hIn: the same helpers for the other 16-bit format.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
// Two floats -> a packed fp16 pair (lo in bits 0-15), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
// Element access for a kernel compiled for either format (H: fp16).
template <bool H> __device__ __forceinline__ float x16_lo(uint32_t w) { return H ? f16_lo(w) : bf16_lo(w); }
template <bool H> __device__ __forceinline__ float x16_hi(uint32_t w) { return H ? f16_hi(w) : bf16_hi(w); }
template <bool H> __device__ __forceinline__ uint32_t pack_x16(float lo, float hi)
{
    return H ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// s_waitcnt vmcnt(n): at most n vector memory operations of this wave outstanding. Called
// from fully unrolled loops with n a constant after unrolling; each case is one instruction.
#define MHC_VM_CASE(n) \
    case n: __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00); break;
#define MHC_VM_CASE8(b) MHC_VM_CASE(b) MHC_VM_CASE(b + 1) MHC_VM_CASE(b + 2) MHC_VM_CASE(b + 3) \
    MHC_VM_CASE(b + 4) MHC_VM_CASE(b + 5) MHC_VM_CASE(b + 6) MHC_VM_CASE(b + 7)
__device__ __forceinline__ void wait_vm(int n)
{
    switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
        MHC_VM_CASE8(0) MHC_VM_CASE8(8) MHC_VM_CASE8(16) MHC_VM_CASE8(24)
        MHC_VM_CASE8(32) MHC_VM_CASE8(40) MHC_VM_CASE8(48) MHC_VM_CASE8(56)
        default: break;
    }
}
#undef MHC_VM_CASE8
#undef MHC_VM_CASE

// Each launch is checked with hipGetLastError, which reports the last error of any HIP call
// of this thread: an entry point first clears one left pending by an earlier, unrelated call,
// so that it is not taken for a failed launch.
inline void clear_pending_error() { (void)hipGetLastError(); }

// Buffer resources: a base address and a byte range in four scalar registers; vector
// accesses take a 32-bit byte offset, and loads outside the range return zero (stores
// outside it are dropped), which bounds every access of a ragged tile in hardware.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) buffer on gfx9-family targets
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ void st_buf(rsrc_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}

// DPP lane moves within a 16-lane row (one cycle, no LDS): quad permutes, row rotates,
// the half-row mirror. Each lane reads the value of the lane the control names.
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

}  // namespace
}  // namespace mhc
