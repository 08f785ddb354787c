// gdn_device.hpp -- device helpers shared by the gfx950 GDN kernels.
//
// bf16 is carried as raw uint16_t bits: widening is exact (bits << 16) and
// narrowing rounds to nearest, ties to even, quieting NaNs.  Reductions inside
// a wavefront use DPP lane permutations in a fixed butterfly, so every lane of
// a group ends with the bitwise-same sum and the order never depends on the
// batch, the grid or the tile (the property the batch-invariance tests of
// RL-Kernel PR #469, "L1, and the bf16 recurrent state", ask of a golden).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (the hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats to two packed bf16 (element a in the low half), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    const f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Widen the low / high bf16 of a packed pair.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Typed load/store of one element as fp32.
template <typename T> struct elem;
template <> struct elem<float> {
    __device__ __forceinline__ static float ld(const float* p) { return *p; }
    __device__ __forceinline__ static void st(float* p, float v) { *p = v; }
};
template <> struct elem<bf16_t> {
    __device__ __forceinline__ static float ld(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// DPP controls (GCN/CDNA encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- lane 7-i within each 8
constexpr int DPP_ROW_MIRROR = 0x140;  // lane i <- lane 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group receives the
// bitwise-identical total (fp addition is commutative, and each step pairs
// lanes symmetrically).
__device__ __forceinline__ float sum8(float x) {
    x = x + dpp<DPP_QUAD_XOR1>(x);
    x = x + dpp<DPP_QUAD_XOR2>(x);
    x = x + dpp<DPP_HALF_MIRROR>(x);
    return x;
}

// Device-side validation result: nonzero means fail closed.
__device__ __forceinline__ bool call_rejected(const int32_t* err_flag) {
    return err_flag != nullptr && __builtin_nontemporal_load(err_flag) != 0;
}

// SiLU through the hardware base-2 exponential (__expf) and reciprocal
// (v_rcp_f32, 1 ulp): a few fp32 ulps from the correctly rounded value, the
// form a production conv provider uses (exp2 approximation and an approximate
// division), against the exp and IEEE division of the golden.  Every conv path
// calls this one function, so the paths stay bitwise equal to each other.
__device__ __forceinline__ float silu(float y) {
    return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

}  // namespace gdn
