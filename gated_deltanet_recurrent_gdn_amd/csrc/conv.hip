// conv.hip -- causal depthwise conv1d update over a slot-indexed conv cache.
//
// RL-Kernel PR #469, "Summary" and "The conv half: coverage and the two
// mismatch mechanisms": the conv state is [num_blocks, dim, W-1]; the window
// is the state followed by the new token(s); the fp32 accumulator starts from
// the bias and adds the taps in order; the state is rolled to the last W-1
// raw inputs (compared bitwise there); SiLU is optional.  This build keeps the
// exact bf16 x bf16 products (exact in fp32) instead of rounding each product
// to bf16, and computes SiLU with IEEE division and the device expf.
//
// Ownership: each (sequence, channel) is read and rolled by exactly one
// workgroup, and inside it by one thread, after every read of the old state
// by that workgroup -- no cross-workgroup race on the in-place roll.
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

// ---------------------------------------------------------------------------
// Decode: one token per row.  grid = (ceil(D / 1024), rows); a thread owns 4
// consecutive channels: it reads their 12 cached taps, the 4 new inputs and
// 16 weights with vector loads, writes 4 outputs and the 12 rolled taps.
// The cache and token streams are nontemporal (touched once per step); the
// output stays cacheable for the kernel that consumes it next.
// ---------------------------------------------------------------------------
template <typename XT, typename CT, typename WT, typename OT>
__global__ __launch_bounds__(256) void conv_decode_kernel(
    const XT* __restrict__ x, const int32_t* __restrict__ slot, CT* __restrict__ cs,
    const WT* __restrict__ w, const WT* __restrict__ bias, OT* __restrict__ out, int32_t D,
    int32_t flags, const int32_t* __restrict__ err_flag) {
    static_assert(CONV_W == 4, "four taps");
    if (call_rejected(err_flag)) return;
    const int b = blockIdx.y;
    const int c = 4 * (blockIdx.x * 256 + threadIdx.x);
    if (c >= D) return;
    const int32_t s = slot[b];
    typename V4<OT>::raw* o = reinterpret_cast<typename V4<OT>::raw*>(out + static_cast<size_t>(b) * D + c);
    if (s <= 0) {                       // inactive row: zeros, cache untouched
        *o = V4<OT>::make(0.f, 0.f, 0.f, 0.f);
        return;
    }
    typedef typename V4<CT>::raw CR;
    CR* st = reinterpret_cast<CR*>(cs + (static_cast<size_t>(s) * D + c) * (CONV_W - 1));
    CR raw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) raw[j] = ld_nt<CR>(st + j);
    const typename V4<XT>::raw xin =
        ld_nt<typename V4<XT>::raw>(reinterpret_cast<const typename V4<XT>::raw*>(x + static_cast<size_t>(b) * D + c));
    typename V4<WT>::raw wr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[j] = reinterpret_cast<const typename V4<WT>::raw*>(w + c * CONV_W)[j];
    typename V4<WT>::raw br = V4<WT>::make(0.f, 0.f, 0.f, 0.f);
    if (bias) br = *reinterpret_cast<const typename V4<WT>::raw*>(bias + c);

    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {                // channel c + e: taps 3e .. 3e+2, token e
        float acc = V4<WT>::get(br, e);
#pragma unroll
        for (int j = 0; j < CONV_W - 1; ++j)
            acc = fmaf(vget<WT, 4>(wr, 4 * e + j), vget<CT, 3>(raw, 3 * e + j), acc);
        acc = fmaf(vget<WT, 4>(wr, 4 * e + 3), V4<XT>::get(xin, e), acc);
        if (flags & GDN_FLAG_SILU) acc = silu(acc);
        y[e] = acc;
    }
    *o = V4<OT>::make(y[0], y[1], y[2], y[3]);

    // roll: per channel drop the oldest tap and append the token.  Old taps
    // move as raw bits; the token keeps its bits when the cache has its dtype
    // and is rounded to the cache dtype otherwise.
    uint32_t nb[12];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        nb[3 * e] = vbits<CT, 3>(raw, 3 * e + 1);
        nb[3 * e + 1] = vbits<CT, 3>(raw, 3 * e + 2);
        nb[3 * e + 2] = std::is_same<XT, CT>::value ? V4<XT>::bits(xin, e)
                                                    : V4<CT>::to_bits(V4<XT>::get(xin, e));
    }
#pragma unroll
    for (int j = 0; j < 3; ++j)
        st_nt<CR>(st + j, V4<CT>::make_bits(nb[4 * j], nb[4 * j + 1], nb[4 * j + 2], nb[4 * j + 3]));
}

// ---------------------------------------------------------------------------
// Varlen: grid = (ceil(D / 64), n_seqs), 256 threads = 64 channels x 4 token
// lanes; token lane tg handles tokens tg, tg+4, ...  The old state is read
// into registers by every thread before a barrier; after it, token lane 0
// alone writes the rolled state.
// ---------------------------------------------------------------------------
template <typename XT, typename CT, typename WT, typename OT>
__global__ __launch_bounds__(256) void conv_varlen_kernel(
    const XT* __restrict__ x, const int32_t* __restrict__ cu, const int32_t* __restrict__ slot,
    CT* __restrict__ cs, const WT* __restrict__ w, const WT* __restrict__ bias,
    OT* __restrict__ out, int32_t D, int32_t flags, const int32_t* __restrict__ err_flag) {
    if (call_rejected(err_flag)) return;
    const int n = blockIdx.y;
    const int cl = threadIdx.x & 63;
    const int tg = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + cl;
    const bool valid = c < D;
    const int32_t start = cu[n];
    const int32_t L = cu[n + 1] - start;
    const int32_t s = slot[n];
    if (s <= 0) {                       // block-uniform branch
        if (valid)
            for (int t = tg; t < L; t += 4)
                elem<OT>::st(out + static_cast<size_t>(start + t) * D + c, 0.0f);
        return;
    }
    CT* st = cs + (static_cast<size_t>(s) * D + (valid ? c : 0)) * (CONV_W - 1);
    CT raw[CONV_W - 1];
    float prev[CONV_W - 1];
    float wt[CONV_W];
#pragma unroll
    for (int j = 0; j < CONV_W - 1; ++j) {
        raw[j] = valid ? st[j] : CT(0);
        prev[j] = elem<CT>::ld(&raw[j]);
    }
#pragma unroll
    for (int j = 0; j < CONV_W; ++j) wt[j] = valid ? elem<WT>::ld(w + c * CONV_W + j) : 0.0f;
    const float b0 = (valid && bias) ? elem<WT>::ld(bias + c) : 0.0f;
    __syncthreads();                    // all reads of the old state precede the roll

    if (valid) {
        for (int t = tg; t < L; t += 4) {
            float acc = b0;
#pragma unroll
            for (int j = 0; j < CONV_W; ++j) {
                const int idx = t + j;          // position in [state | tokens]
                float v = 0.0f;
                if (idx < CONV_W - 1) {
#pragma unroll
                    for (int m = 0; m < CONV_W - 1; ++m)
                        if (idx == m) v = prev[m];
                } else {
                    v = elem<XT>::ld(x + static_cast<size_t>(start + idx - (CONV_W - 1)) * D + c);
                }
                acc = fmaf(wt[j], v, acc);
            }
            if (flags & GDN_FLAG_SILU) acc = silu(acc);
            elem<OT>::st(out + static_cast<size_t>(start + t) * D + c, acc);
        }
        if (tg == 0 && L > 0) {
#pragma unroll
            for (int j = 0; j < CONV_W - 1; ++j) {
                const int idx = L + j;          // new state = last W-1 of [state | tokens]
                CT nv = CT(0);
                if (idx < CONV_W - 1) {
#pragma unroll
                    for (int m = 0; m < CONV_W - 1; ++m)
                        if (idx == m) nv = raw[m];
                } else {
                    elem<CT>::st(&nv, elem<XT>::ld(x + static_cast<size_t>(start + idx - (CONV_W - 1)) * D + c));
                }
                st[j] = nv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dtype dispatch
// ---------------------------------------------------------------------------
namespace {
template <typename XT, typename CT, typename WT, typename OT>
struct DecodeK {
    static hipError_t run(const void* x, const int32_t* slot, int32_t rows, void* cs,
                          const void* w, const void* bias, void* out, int32_t D, int32_t flags,
                          const int32_t* err, hipStream_t st) {
        dim3 grid((D / 4 + 255) / 256, rows);
        return launch(conv_decode_kernel<XT, CT, WT, OT>, grid, dim3(256), 0, st,
                      static_cast<const XT*>(x), slot, static_cast<CT*>(cs),
                      static_cast<const WT*>(w), static_cast<const WT*>(bias),
                      static_cast<OT*>(out), D, flags, err);
    }
};
template <typename XT, typename CT, typename WT, typename OT>
struct VarlenK {
    static hipError_t run(const void* x, const int32_t* cu, int32_t n_seqs, const int32_t* slot,
                          void* cs, const void* w, const void* bias, void* out, int32_t D,
                          int32_t flags, const int32_t* err, hipStream_t st) {
        dim3 grid((D + 63) / 64, n_seqs);
        return launch(conv_varlen_kernel<XT, CT, WT, OT>, grid, dim3(256), 0, st,
                      static_cast<const XT*>(x), cu, slot, static_cast<CT*>(cs),
                      static_cast<const WT*>(w), static_cast<const WT*>(bias),
                      static_cast<OT*>(out), D, flags, err);
    }
};

template <template <typename, typename, typename, typename> class K, typename OT, typename WT,
          typename CT, typename... A>
hipError_t pick_x(gdn_dtype x, A&&... a) {
    return x == GDN_BF16 ? K<bf16_t, CT, WT, OT>::run(std::forward<A>(a)...)
                         : K<float, CT, WT, OT>::run(std::forward<A>(a)...);
}
template <template <typename, typename, typename, typename> class K, typename OT, typename WT,
          typename... A>
hipError_t pick_c(gdn_dtype x, gdn_dtype c, A&&... a) {
    return c == GDN_BF16 ? pick_x<K, OT, WT, bf16_t>(x, std::forward<A>(a)...)
                         : pick_x<K, OT, WT, float>(x, std::forward<A>(a)...);
}
template <template <typename, typename, typename, typename> class K, typename OT, typename... A>
hipError_t pick_w(gdn_dtype x, gdn_dtype c, gdn_dtype w, A&&... a) {
    return w == GDN_BF16 ? pick_c<K, OT, bf16_t>(x, c, std::forward<A>(a)...)
                         : pick_c<K, OT, float>(x, c, std::forward<A>(a)...);
}
template <template <typename, typename, typename, typename> class K, typename... A>
hipError_t pick_all(gdn_dtype x, gdn_dtype c, gdn_dtype w, gdn_dtype o, A&&... a) {
    return o == GDN_BF16 ? pick_w<K, bf16_t>(x, c, w, std::forward<A>(a)...)
                         : pick_w<K, float>(x, c, w, std::forward<A>(a)...);
}
}  // namespace

hipError_t launch_conv_decode(const void* x, gdn_dtype x_dt, const int32_t* slot_idx,
                              int32_t rows, void* conv_state, gdn_dtype cs_dt,
                              const void* weight, const void* bias, gdn_dtype w_dt,
                              void* out, gdn_dtype out_dt, int32_t dim, int32_t flags,
                              const int32_t* err_flag, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    return pick_all<DecodeK>(x_dt, cs_dt, w_dt, out_dt, x, slot_idx, rows, conv_state, weight,
                             bias, out, dim, flags, err_flag, stream);
}

hipError_t launch_conv_varlen(const void* x, gdn_dtype x_dt, const int32_t* cu_seqlens,
                              int32_t n_seqs, const int32_t* slot_idx, void* conv_state,
                              gdn_dtype cs_dt, const void* weight, const void* bias,
                              gdn_dtype w_dt, void* out, gdn_dtype out_dt, int32_t dim,
                              int32_t flags, const int32_t* err_flag, hipStream_t stream) {
    if (n_seqs == 0) return hipSuccess;
    return pick_all<VarlenK>(x_dt, cs_dt, w_dt, out_dt, x, cu_seqlens, n_seqs, slot_idx,
                             conv_state, weight, bias, out, dim, flags, err_flag, stream);
}

}  // namespace gdn
