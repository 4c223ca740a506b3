// Helpers shared by the gfx950 (MI355X) kernels of this library: the two
// 16-bit element formats and their matrix-core products, buffer resources
// and buffer loads (to registers and straight into LDS), the transposing LDS
// read, integer division by an invariant divisor, and the XCD-aware
// renumbering of workgroups.  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace evo {
namespace gfx {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

// A buffer offset past every range: the load returns zeros.  Offsets past a
// range stay below 2^32 (kOOB plus less than 2^31).
constexpr uint32_t kOOB = 0x80000000u;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The two 16-bit element formats: bfloat16 and IEEE binary16.  Data moves as
// integers; the vector types appear only as MFMA operands and in the
// float -> 16-bit conversion.
struct Bf16Fmt {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    static constexpr bool kF16 = false;
    static constexpr uint32_t kOnes2 = 0x3f803f80u;  // two 1.0
    __device__ static float widen(u16 x) { return __builtin_bit_cast(float, (uint32_t)x << 16); }
    __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
};
struct F16Fmt {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    static constexpr bool kF16 = true;
    static constexpr uint32_t kOnes2 = 0x3c003c00u;  // two 1.0
    __device__ static float widen(u16 x) { return (float)__builtin_bit_cast(_Float16, x); }
    __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
};

// Two floats -> two 16-bit values (round to nearest even) in one dword, low half first.
template <class E>
__device__ inline uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, typename E::v2));
}

template <class E>
__device__ inline typename E::v8 as_v8(uint4 x) { return __builtin_bit_cast(typename E::v8, x); }

// The two 16-bit values of a dword, widened.
template <class E>
__device__ inline f32x2 unpack2(uint32_t w) { return f32x2{E::widen((u16)(w & 0xffffu)), E::widen((u16)(w >> 16))}; }

// ds_read_b64_tr_b16 of the 8 bytes at p: in each 16-lane group, lane i
// receives element e (e = 0..3) from column i % 4 of the 4-element row that
// lane 4e + i/4 addressed.  With lane a addressing row R0 + a/4, columns
// 4(a%4) .. +3 of a row-major matrix, lane i gets column i of rows R0 .. R0+3.
__device__ inline uint2 ds_read_tr(const void* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) char*)p));
    return __builtin_bit_cast(uint2, r);
}

__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Cross-lane max / sum over the four lanes (c, c+16, c+32, c+48) that share a
// column of a 16x16 MFMA result.  (LDS-routed shuffles; the v_permlane16/32
// swap builtins fold into one half when both operands are the same value.)
__device__ inline float max_over_groups(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ inline float sum_over_groups(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Buffer resources: base address + byte range in SGPRs, 32-bit per-lane
// offsets.  A load past the range returns zeros.  Every offset is passed in
// the per-lane part (the scalar offset stays 0), so the range check sees the
// whole offset.
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ inline Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint4 bload16(Rsrc r, uint32_t voff, uint32_t soff = 0) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at
// lds + 16*l (lds must be the same for the whole wave).
__device__ inline void dma16(Rsrc r, const void* lds, uint32_t voff, uint32_t soff = 0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff,
                                             (int)soff, 0, 0);
}

// The same copy written as assembly: the compiler then neither tracks it nor
// makes later LDS reads wait for it (with the builtin it orders every later
// LDS read, of any buffer, behind the copy's completion).  The caller waits
// for it itself (wait_all, or an s_waitcnt on the vector-memory count) before
// a barrier publishes the data.  M0 carries the LDS address, taken from the
// low 32 bits of the generic pointer (the LDS offset); one wait state
// separates its write from the load that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is named as clobbered on purpose
__device__ inline void dma16_untracked(Rsrc r, const void* lds, uint32_t voff) {
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(a), "v"(voff), "s"(r)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait for every outstanding memory operation of this wave.
__device__ inline void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// 16 bytes at byte offset `off` of a buffer of `range` bytes, any 2-byte
// alignment.  A chunk that starts inside the range and ends past it is read
// element by element, so that its elements inside the range keep their
// values (the range check of a wider load may drop more than the part
// outside); a chunk wholly past the range reads as zeros either way.
__device__ inline uint4 bload16_any(Rsrc r, uint32_t off, uint32_t range) {
    if (off >= range || off + 16u <= range) return bload16(r, off, 0);
    uint32_t w[4];
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, (int)(off + 4 * e), 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, (int)(off + 4 * e + 2), 0, 0);
        w[e] = lo | (hi << 16);
    }
    return uint4{w[0], w[1], w[2], w[3]};
}

// x / d for 0 <= x < 2^31 and 1 <= d < 2^31 as a multiply-high and a shift
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, section 4): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, x / d = (mulhi(x, m) + x) >> l; the sum
// cannot overflow because mulhi(x, m) <= x < 2^31.
struct FastDiv {
    uint32_t d, m, l;
};

__device__ inline uint32_t fdiv(uint32_t x, FastDiv f) { return (__umulhi(x, f.m) + x) >> f.l; }

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

// Workgroups are dealt round-robin over the 8 XCDs (workgroup w runs on XCD
// w mod 8).  This renumbering gives each XCD one contiguous range of the
// logical order, so that neighbouring work items, which share operand lines,
// meet in one XCD's L2.
__device__ inline int64_t logical_block(int64_t hw, int64_t total) {
    const int64_t xcd = hw % 8, j = hw / 8;
    const int64_t per = total / 8, extra = total % 8;  // the first `extra` XCDs get one more
    return xcd < extra ? xcd * (per + 1) + j : extra * (per + 1) + (xcd - extra) * per + j;
}

}  // namespace gfx
}  // namespace evo
