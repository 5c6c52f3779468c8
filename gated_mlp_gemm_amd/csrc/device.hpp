// Device primitives for gfx950 (CDNA4): MFMA wrappers, LDS access helpers,
// the SiLU activation and bf16 conversion.
//
// Lane layouts used throughout (wave64), as exercised by the parity tests:
//   v_mfma_f32_32x32x16_bf16, operands A (32 x 16) and B (16 x 32):
//     lane l holds A[l % 32][8*(l/32) + j] and B[8*(l/32) + j][l % 32], j < 8;
//     accumulator register i of lane l is D[8*(i/4) + 4*(l/32) + i%4][l % 32].
//   v_mfma_f32_16x16x32_bf16, operands A (16 x 32) and B (32 x 16):
//     lane l holds A[l % 16][8*(l/16) + j] and B[8*(l/16) + j][l % 16], j < 8;
//     accumulator register i of lane l is D[4*(l/16) + i][l % 16].
//   ds_read_b64_tr_b16: within each group of 16 lanes, element j of lane i is
//     element (i % 4) of the 8-byte chunk addressed by lane 4*j + i/4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swiglu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SWIGLU_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8 &a, const bf16x8 &b,
                                                const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// c += A . B on one 16x16 accumulator quad, in place.  Written as inline
// assembly with the accumulator tied to its own AGPRs: through the builtin the
// compiler assigns the result of a 16x16 MFMA other registers than its C
// operand and then rotates the accumulators back every loop iteration (about
// as many AGPR copies per K step as MFMAs).  The compiler does not see these
// as MFMAs, so their hazards are the pipeline's job: the result is read by
// other instructions only after Pipeline::drain(), which waits out the MFMA
// latency, and MFMAs follow the zeroing of their accumulators only after
// zero_acc()'s wait.
__device__ __forceinline__ void mfma_16x16x32_acc(f32x4 &c, const u32x4 &a, const u32x4 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// The same with a zero accumulator input: c = a b, the first MFMA of a
// contraction (no zeroing of c before it, which the compiler could move).
__device__ __forceinline__ void mfma_16x16x32_init(f32x4 &c, const u32x4 &a, const u32x4 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}
// At least 24 wait states: more than any MFMA result needs before another
// instruction may read it (the longest, 32x32 MFMAs, need 19).
__device__ __forceinline__ void wait_mfma_results() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
}

// The accumulators of one 32x32 output block, 16 registers a lane, numbered
// r = 0..15 in quads q = r / 4: either the 16 registers of one 32x32 MFMA
// (Acc32), or the 4 registers of each of four 16x16 MFMAs, quad q covering
// rows 16 (q / 2) + [0, 16) and columns 16 (q % 2) + [0, 16) of the block
// (Acc16).  Each 16x16 MFMA then works on a whole register quad, which the
// compiler keeps as one 4-register tuple.
struct Acc32 {
    f32x16 v;
    __device__ __forceinline__ float get(int r) const { return v[r]; }
    __device__ __forceinline__ void set(int r, float x) { v[r] = x; }
    __device__ __forceinline__ f32x4 quad(int q) const {
        return f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    }
    __device__ __forceinline__ void set_quad(int q, const f32x4 &x) {
        v[4 * q] = x[0];
        v[4 * q + 1] = x[1];
        v[4 * q + 2] = x[2];
        v[4 * q + 3] = x[3];
    }
};
struct Acc16 {
    f32x4 v[4];
    __device__ __forceinline__ float get(int r) const { return v[r >> 2][r & 3]; }
    __device__ __forceinline__ void set(int r, float x) { v[r >> 2][r & 3] = x; }
    __device__ __forceinline__ f32x4 quad(int q) const { return v[q]; }
    __device__ __forceinline__ void set_quad(int q, const f32x4 &x) { v[q] = x; }
};

// FP8 E4M3 x FP8 E4M3 -> fp32, 32x32 outputs, 64 k (v_mfma_f32_32x32x64_f8f6f4;
// format code 0 = E4M3 for both operands, no block scales).  Each operand is
// 32 bytes per lane, given as two 16-byte chunks (low chunk first).
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(const u32x4 &a0, const u32x4 &a1,
                                                    const u32x4 &b0, const u32x4 &b1,
                                                    const f32x16 &c) {
    const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                     (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16-byte LDS read (ds_read_b128).
__device__ __forceinline__ u32x4 lds_read16(const SWIGLU_LDS char *p) {
    return *reinterpret_cast<const SWIGLU_LDS u32x4 *>(p);
}

// 16-byte LDS write (ds_write_b128).
__device__ __forceinline__ void lds_write16(SWIGLU_LDS char *p, const u32x4 &v) {
    *reinterpret_cast<SWIGLU_LDS u32x4 *>(p) = v;
}

// 8-byte transposing LDS read (ds_read_b64_tr_b16), see the layout note above.
__device__ __forceinline__ u32x2 lds_read_tr8(const SWIGLU_LDS char *p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<SWIGLU_LDS i16x4 *>(const_cast<SWIGLU_LDS char *>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// 16-byte global load / store (global_load_dwordx4 / global_store_dwordx4).
__device__ __forceinline__ u32x4 gload16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void gstore16(uint16_t *p, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Value of lane (l ^ 1) (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ float swap_adjacent_lanes(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}

// Per-lane choice by lane parity: even lanes get `even_v`, odd lanes `odd_v`
// (v_cndmask against the constant odd-lane mask).  Written out so that the
// compiler cannot turn a parity choice between two elements of one vector
// into a variable-index extract, which it expands into a select chain over
// the whole vector.
__device__ __forceinline__ float by_lane_parity(float even_v, float odd_v) {
    float r;
    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3"
        : "=v"(r)
        : "v"(even_v), "v"(odd_v), "s"(0xAAAAAAAAAAAAAAAAull));
    return r;
}

// An accumulator value read out of its AGPR at this point of the program.
// Volatile asm keeps the reads in order with the other volatile statements,
// so the compiler cannot hoist all of a tile's accumulator reads above the
// epilogue (it would then hold the whole tile in VGPRs and spill).
__device__ __forceinline__ float read_acc(float a) {
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(a));
    return r;
}

template <bool kFromAcc>
__device__ __forceinline__ float acc_value(float a) {
    if constexpr (kFromAcc) return read_acc(a);
    else return a;
}

// SiLU(x) = x / (1 + e^{-x}) = x * rcp(1 + 2^{-x log2 e}) with the hardware
// exp2 and reciprocal (about 1 ulp each in fp32).  Very negative x: the exp2
// overflows to +inf, the reciprocal is 0 and the result is -0; large x:
// exp2 -> 0 and the result is x.
__device__ __forceinline__ float silu(float x) {
    const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Two floats -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed
// low = a, high = b.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
    return static_cast<uint16_t>(pack_bf16x2(a, 0.0f) & 0xFFFFu);
}

}  // namespace swiglu
