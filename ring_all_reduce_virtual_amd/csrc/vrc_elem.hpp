// vrc_elem.hpp -- element types for the virtual-rank collective kernels.
//
// Every kernel moves data in 16-byte vectors (one global_load_dwordx4 /
// global_store_dwordx4 per lane) and computes in an accumulator type:
//   int32 -> uint32 (two's-complement wrap), fp32 -> float,
//   fp16  -> float (exact widening, round-to-nearest-even narrowing),
//   bf16  -> float (exact widening, round-to-nearest-even narrowing).
// A ring step adds two stored values and rounds once to the storage type;
// the fused kernels fold N values in the accumulator and round once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vrc {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// The same 16 bytes at any address.  The HSA ABI runs the GPU in unaligned
// access mode, so one global_load/store_dwordx4 serves an operand on any byte
// offset (for this target the compiler emits that single instruction even for
// a 16-byte memcpy from a char pointer).  The hardware reads and writes the
// cache lines such a vector straddles, so misalignment costs bandwidth only
// where a wave's 1 KiB run crosses a line or write block that another wave
// also touches (measured on MI355X, 8 x 512 MiB fused bf16 all-reduce: inputs
// on other offsets +8 %, outputs on other 64-byte offsets +22 %, which the
// realigned kernels bring down to +5-9 % for inputs and outputs together).
typedef u32x4 u32x4_any __attribute__((aligned(1)));

// Every buffer the library is given is device (global) memory.  Accessing it
// through global address-space pointers gives global_load/global_store
// instructions even where the compiler cannot trace a pointer back to a
// kernel argument (flat instructions would also count against the LDS
// counter).
template <class X>
using global_ptr = __attribute__((address_space(1))) X*;

// 16-byte load/store at any element alignment, optionally with the
// non-temporal hint (streaming data that is never re-read should not displace
// other lines from the caches).
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const char* p)
{
    const auto g = (global_ptr<const u32x4_any>)p;
    if constexpr (NT) return __builtin_nontemporal_load(g);
    else return *g;
}

template <bool NT>
__device__ __forceinline__ void st16(char* p, u32x4 v)
{
    const auto g = (global_ptr<u32x4_any>)p;
    if constexpr (NT) __builtin_nontemporal_store(v, g);
    else *g = v;
}

// Bytes 4Q + s .. 4Q + s + 15 (s < 4) of the eight dwords w, as one vector:
// dword i is funnelled from w[Q + i] and w[Q + i + 1] by v_alignbyte.
template <int Q>
__device__ __forceinline__ u32x4 funnel(const unsigned* w, uint32_t s)
{
    return u32x4{__builtin_amdgcn_alignbyte(w[Q + 1], w[Q], s), __builtin_amdgcn_alignbyte(w[Q + 2], w[Q + 1], s),
                 __builtin_amdgcn_alignbyte(w[Q + 3], w[Q + 2], s), __builtin_amdgcn_alignbyte(w[Q + 4], w[Q + 3], s)};
}

// Compiler barrier.  A load after it is issued even when this lane has just
// stored the value it reads (the compiler would otherwise reuse the stored
// register): the memory-faithful ring chains read every partial back from
// the buffer the previous step wrote it to.
__device__ __forceinline__ void reload_fence() { __asm__ __volatile__("" ::: "memory"); }

// Scheduling barrier: everything before it is issued before anything after
// it.  Placed between a kernel's loads and the fold that consumes them, it
// keeps all of a lane's loads in flight at once; without it the compiler may
// interleave the fold with the loads and wait on each pair (for fp32, fp16 and
// int32 it did, and the 8 x 512 MiB fused all-reduce ran at 3.8-4.3 TB/s
// instead of 5.4).
__device__ __forceinline__ void issue_loads_first() { __builtin_amdgcn_sched_barrier(0); }

// Wait until at most W vector memory operations of this wave are outstanding
// (the gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt 7 and
// lgkmcnt 15 wait on nothing).
template <int W>
__device__ __forceinline__ void wait_vmem_below()
{
    static_assert(W >= 0 && W < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (W & 15) | ((W >> 4) << 14));
}

struct I32 {
    using S = uint32_t;  // stored bits
    using A = uint32_t;  // accumulator
    static constexpr int ESZ = 4, VEC = 4;
    __device__ static A widen(S s) { return s; }
    __device__ static S narrow(A a) { return a; }
    __device__ static A add(A a, A b) { return a + b; }
    __device__ static void unpack(u32x4 v, A* a) { a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w; }
    __device__ static u32x4 pack(const A* a) { return u32x4{a[0], a[1], a[2], a[3]}; }
};

struct F32 {
    using S = uint32_t;
    using A = float;
    static constexpr int ESZ = 4, VEC = 4;
    __device__ static A widen(S s) { return __uint_as_float(s); }
    __device__ static S narrow(A a) { return __float_as_uint(a); }
    __device__ static A add(A a, A b) { return a + b; }
    __device__ static void unpack(u32x4 v, A* a)
    {
        a[0] = __uint_as_float(v.x); a[1] = __uint_as_float(v.y);
        a[2] = __uint_as_float(v.z); a[3] = __uint_as_float(v.w);
    }
    __device__ static u32x4 pack(const A* a)
    {
        return u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                     __float_as_uint(a[3])};
    }
};

struct F16 {
    using S = uint16_t;
    using A = float;
    static constexpr int ESZ = 2, VEC = 8;
    __device__ static A widen(S s) { return (float)__builtin_bit_cast(_Float16, s); }
    // The hardware conversion rounds to nearest even (the default mode),
    // keeps fp16 subnormals and overflows to infinity.
    __device__ static S narrow(A a) { return __builtin_bit_cast(uint16_t, (_Float16)a); }
    __device__ static A add(A a, A b) { return a + b; }
    __device__ static void unpack(u32x4 v, A* a)
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a[2 * i] = widen((S)(w[i] & 0xffffu));
            a[2 * i + 1] = widen((S)(w[i] >> 16));
        }
    }
    __device__ static u32x4 pack(const A* a)
    {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; i++) w[i] = (uint32_t)narrow(a[2 * i]) | ((uint32_t)narrow(a[2 * i + 1]) << 16);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
};

struct BF16 {
    using S = uint16_t;
    using A = float;
    static constexpr int ESZ = 2, VEC = 8;
    // bfloat16 is the upper half of an IEEE binary32.
    __device__ static A widen(S s) { return __uint_as_float((uint32_t)s << 16); }
    // Round to nearest even on the 16 discarded bits; a NaN keeps its sign
    // and upper payload bits and becomes quiet (bit 6 of the half set).  The
    // target's conversion (v_cvt_pk_bf16_f32, two values per instruction)
    // does exactly that in this library's floating-point mode (denormals
    // kept): tests/c/bf16_cvt_check.hip compares it with the bit-level
    // rounding on all 2^32 inputs.
    __device__ static S narrow(A a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }
    __device__ static uint32_t narrow2(A lo, A hi)
    {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
    }
    __device__ static A add(A a, A b) { return a + b; }
    __device__ static void unpack(u32x4 v, A* a)
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a[2 * i] = __uint_as_float(w[i] << 16);
            a[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static u32x4 pack(const A* a)
    {
        return u32x4{narrow2(a[0], a[1]), narrow2(a[2], a[3]), narrow2(a[4], a[5]), narrow2(a[6], a[7])};
    }
};

template <class T>
__device__ __forceinline__ typename T::S load_s(const char* p)
{
    return *(global_ptr<const typename T::S>)p;
}

template <class T>
__device__ __forceinline__ void store_s(char* p, typename T::S v)
{
    *(global_ptr<typename T::S>)p = v;
}

// One ring-step element: round(widen(a) + widen(b)) in the storage type.
template <class T>
__device__ __forceinline__ typename T::S add_s(typename T::S a, typename T::S b)
{
    return T::narrow(T::add(T::widen(a), T::widen(b)));
}

// The same on a 16-byte vector.
template <class T>
__device__ __forceinline__ u32x4 add_v(u32x4 a, u32x4 b)
{
    typename T::A x[T::VEC], y[T::VEC];
    T::unpack(a, x);
    T::unpack(b, y);
#pragma unroll
    for (int i = 0; i < T::VEC; i++) x[i] = T::add(x[i], y[i]);
    return T::pack(x);
}

}  // namespace vrc
