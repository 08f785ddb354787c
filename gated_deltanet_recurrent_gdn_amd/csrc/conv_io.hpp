// conv_io.hpp -- vector access to groups of 4 conv channels and the decode-form
// conv of one group (shared by the conv kernels and the fused decode step).
//
// RL-Kernel PR #469, "Summary" and "The conv half: coverage and the two
// mismatch mechanisms": the conv state is [num_blocks, dim, W-1]; the window
// is the state followed by the new token; the fp32 accumulator starts from the
// bias and adds the taps in order; the state is rolled to the last W-1 raw
// inputs; SiLU is optional.
#pragma once

#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int CONV_W = 4;

// ---------------------------------------------------------------------------
// Vector access to 4 consecutive channels (16 taps / 12 cached taps) of any
// element type: 4 bf16 are one 8-byte access, 4 fp32 one 16-byte access.
// ---------------------------------------------------------------------------
template <typename T> struct V4;
template <> struct V4<bf16_t> {
    typedef uint2 raw;
    __device__ __forceinline__ static uint32_t bits(const raw& r, int j) {
        const uint32_t w = (j < 2) ? r.x : r.y;
        return (j & 1) ? (w >> 16) : (w & 0xffffu);
    }
    __device__ __forceinline__ static float get(const raw& r, int j) {
        return __uint_as_float(bits(r, j) << 16);
    }
    __device__ __forceinline__ static raw make(float a, float b, float c, float d) {
        return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
    }
    __device__ __forceinline__ static raw make_bits(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        return make_uint2(a | (b << 16), c | (d << 16));
    }
    __device__ __forceinline__ static uint32_t to_bits(float f) { return f32_to_bf16(f); }
};
template <> struct V4<float> {
    typedef float4 raw;
    __device__ __forceinline__ static float get(const raw& r, int j) {
        return (j == 0) ? r.x : (j == 1) ? r.y : (j == 2) ? r.z : r.w;
    }
    __device__ __forceinline__ static uint32_t bits(const raw& r, int j) { return __float_as_uint(get(r, j)); }
    __device__ __forceinline__ static raw make(float a, float b, float c, float d) {
        return make_float4(a, b, c, d);
    }
    __device__ __forceinline__ static raw make_bits(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        return make_float4(__uint_as_float(a), __uint_as_float(b), __uint_as_float(c), __uint_as_float(d));
    }
    __device__ __forceinline__ static uint32_t to_bits(float f) { return __float_as_uint(f); }
};
// element j of an array of raw words holding 4 elements each
template <typename T, int N>
__device__ __forceinline__ float vget(const typename V4<T>::raw (&r)[N], int j) {
    return V4<T>::get(r[j >> 2], j & 3);
}
template <typename T, int N>
__device__ __forceinline__ uint32_t vbits(const typename V4<T>::raw (&r)[N], int j) {
    return V4<T>::bits(r[j >> 2], j & 3);
}

typedef float v4f_c __attribute__((ext_vector_type(4)));
template <typename R> __device__ __forceinline__ R ld_nt(const R* p);
template <> __device__ __forceinline__ uint2 ld_nt<uint2>(const uint2* p) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
    return make_uint2(v.x, v.y);
}
template <> __device__ __forceinline__ float4 ld_nt<float4>(const float4* p) {
    const v4f_c v = __builtin_nontemporal_load(reinterpret_cast<const v4f_c*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
template <typename R> __device__ __forceinline__ void st_nt(R* p, const R& x);
template <> __device__ __forceinline__ void st_nt<uint2>(uint2* p, const uint2& x) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 v = {x.x, x.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u2*>(p));
}
template <> __device__ __forceinline__ void st_nt<float4>(float4* p, const float4& x) {
    const v4f_c v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<v4f_c*>(p));
}

// One token of the decode-form conv for channels c .. c+3 of one row, in two
// halves so that a caller can put other loads between them: conv4_load reads
// the 12 cached taps (cache row `st` = &cs[(slot * D + c) * 3]), the 4 inputs,
// 16 weights and the bias; conv4_finish returns the 4 fp32 outputs (SiLU
// applied when asked) and writes the rolled taps back.  Old taps move as raw
// bits; the token keeps its bits when the cache has its dtype and is rounded
// to the cache dtype otherwise.  The cache and token streams are nontemporal.
template <typename XT, typename CT, typename WT>
struct Conv4In {
    typename V4<CT>::raw raw[3];
    typename V4<XT>::raw xin;
    typename V4<WT>::raw wr[4];
    typename V4<WT>::raw br;
};

template <typename XT, typename CT, typename WT>
__device__ __forceinline__ void conv4_load(const XT* __restrict__ xp, const CT* __restrict__ stp,
                                           const WT* __restrict__ wp, const WT* __restrict__ bp,
                                           Conv4In<XT, CT, WT>& in) {
    typedef typename V4<CT>::raw CR;
    const CR* st = reinterpret_cast<const CR*>(stp);
#pragma unroll
    for (int j = 0; j < 3; ++j) in.raw[j] = ld_nt<CR>(st + j);
    in.xin = ld_nt<typename V4<XT>::raw>(reinterpret_cast<const typename V4<XT>::raw*>(xp));
#pragma unroll
    for (int j = 0; j < 4; ++j) in.wr[j] = reinterpret_cast<const typename V4<WT>::raw*>(wp)[j];
    // branch-free bias: without one, re-read the weights and select zeros (a
    // conditional load would make later waits drain every load before it)
    const typename V4<WT>::raw bl = *reinterpret_cast<const typename V4<WT>::raw*>(bp ? bp : wp);
    in.br = bp ? bl : V4<WT>::make(0.f, 0.f, 0.f, 0.f);
}

template <typename XT, typename CT, typename WT>
__device__ __forceinline__ void conv4_finish(const Conv4In<XT, CT, WT>& in, CT* __restrict__ stp,
                                             bool silu_on, float (&y)[4]) {
    static_assert(CONV_W == 4, "four taps");
    typedef typename V4<CT>::raw CR;
#pragma unroll
    for (int e = 0; e < 4; ++e) {                // channel c + e: taps 3e .. 3e+2, token e
        float acc = V4<WT>::get(in.br, e);
#pragma unroll
        for (int j = 0; j < CONV_W - 1; ++j)
            acc = fmaf(vget<WT, 4>(in.wr, 4 * e + j), vget<CT, 3>(in.raw, 3 * e + j), acc);
        acc = fmaf(vget<WT, 4>(in.wr, 4 * e + 3), V4<XT>::get(in.xin, e), acc);
        if (silu_on) acc = silu(acc);
        y[e] = acc;
    }
    uint32_t nb[12];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        nb[3 * e] = vbits<CT, 3>(in.raw, 3 * e + 1);
        nb[3 * e + 1] = vbits<CT, 3>(in.raw, 3 * e + 2);
        nb[3 * e + 2] = std::is_same<XT, CT>::value ? V4<XT>::bits(in.xin, e)
                                                    : V4<CT>::to_bits(V4<XT>::get(in.xin, e));
    }
    CR* st = reinterpret_cast<CR*>(stp);
#pragma unroll
    for (int j = 0; j < 3; ++j)
        st_nt<CR>(st + j, V4<CT>::make_bits(nb[4 * j], nb[4 * j + 1], nb[4 * j + 2], nb[4 * j + 3]));
}

template <typename XT, typename CT, typename WT>
__device__ __forceinline__ void conv4_token(const XT* __restrict__ xp, CT* __restrict__ stp,
                                            const WT* __restrict__ wp, const WT* __restrict__ bp,
                                            bool silu_on, float (&y)[4]) {
    Conv4In<XT, CT, WT> in;
    conv4_load<XT, CT, WT>(xp, stp, wp, bp, in);
    conv4_finish<XT, CT, WT>(in, stp, silu_on, y);
}

}  // namespace gdn
