// conv.hip -- causal depthwise conv1d update over a slot-indexed conv cache.
//
// RL-Kernel PR #469, "Summary" and "The conv half: coverage and the two
// mismatch mechanisms": the conv state is [num_blocks, dim, W-1]; the window
// is the state followed by the new token(s); the fp32 accumulator starts from
// the bias and adds the taps in order; the state is rolled to the last W-1
// raw inputs (compared bitwise there); SiLU is optional.  The products are
// kept exact (bf16 x bf16 is exact in fp32) rather than rounded to bf16 one by
// one.  SiLU is the hardware form x * rcp(1 + 2^(-x log2 e)) (the production
// provider's kind), a few fp32 ulps from the golden's exp with IEEE division.
//
// The in-place roll never races a read of the old state: in the decode form
// and the general varlen kernel one thread reads and then rolls each
// (sequence, channel) (the varlen one after a barrier that follows every read
// of its workgroup); the token-parallel varlen kernel only reads the cache,
// and a separate kernel, next on the stream, rolls it.
#include <type_traits>

#include "conv_io.hpp"

namespace gdn {

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
    float y[4];
    conv4_token<XT, CT, WT>(x + static_cast<size_t>(b) * D + c, cs + (static_cast<size_t>(s) * D + c) * (CONV_W - 1),
                            w + c * CONV_W, bias ? bias + c : nullptr, (flags & GDN_FLAG_SILU) != 0, y);
    *o = V4<OT>::make(y[0], y[1], y[2], y[3]);
}

// ---------------------------------------------------------------------------
// Varlen, token-parallel (the path for dim % 4 == 0 and 16-byte aligned
// tensors).  One-dimensional grid of ceil(T / (4 CONV_TT)) token tiles times
// ceil(D / 256) channel blocks, channel block fastest: consecutive workgroups
// read consecutive 512- or 1024-byte pieces of the same token rows (7-9% faster
// than token tiles fastest, whose neighbours read pieces a row apart), and with
// a multiple of 8 channel blocks a channel block stays on one XCD for every
// tile, so a tile's W-1 halo rows are in that XCD's L2.  A thread owns 4
// channels and CONV_TT consecutive tokens of the concatenated token rows (a
// wave: 256 channels of the same tokens, so each token row is read as one
// contiguous 512- or 1024-byte span).  All CONV_TT + 3 inputs of the thread's
// window are loaded before any arithmetic; the sequence of each token comes from a binary search
// of cu_seqlens (and a walk across the sequence starts inside the tile), and a
// token among the first W-1 of its sequence takes the missing taps from the
// cached state of its slot.  The cache is not written here: conv_roll_kernel,
// launched after this kernel on the same stream, rolls it, so no thread can
// read a rolled tap.  Arithmetic per channel: bias, then taps 0..W-1 with
// fmaf, then SiLU -- the order of every other conv path, bitwise.
// ---------------------------------------------------------------------------
// Tokens per thread.  Measured (eager, conv + roll, dim 8192, bf16, with the
// sequence search and window branches on the scalar unit): 24,674 tokens over
// 8 sequences 141-143 us at 4 against 146-148 at 8, 153 at 16 and 163-167 at
// 2; 200 x 17 tokens 35 us at 4 and 8, 37 at 2.  (Before the scalar control
// flow, when the VALU was the limit, 8 was the best.)
constexpr int CONV_TT = 4;

template <typename XT, typename CT, typename WT, typename OT>
__global__ __launch_bounds__(256) void conv_varlen_tok_kernel(
    const XT* __restrict__ x, const int32_t* __restrict__ cu, int32_t n_seqs, int32_t T,
    const int32_t* __restrict__ slot, const CT* __restrict__ cs, const WT* __restrict__ w,
    const WT* __restrict__ bias, OT* __restrict__ out, int32_t D, int32_t flags,
    const int32_t* __restrict__ err_flag) {
    static_assert(CONV_W == 4, "four taps");
    typedef typename V4<XT>::raw XR;
    typedef typename V4<WT>::raw WR;
    if (call_rejected(err_flag)) return;
    const int ncb = (D / 4 + 63) / 64;            // 256-channel blocks per token tile
    const int cbk = static_cast<int>(blockIdx.x % static_cast<unsigned>(ncb));
    const int tile = static_cast<int>(blockIdx.x / static_cast<unsigned>(ncb));
    const int c = 4 * (cbk * 64 + static_cast<int>(threadIdx.x & 63));
    // t0 is the same for the whole wave; saying so puts the sequence search,
    // the cu_seqlens / slot reads and every per-token branch below on the scalar
    // unit (as vector compares with exec masking they cost 16% of the call:
    // 24,674 tokens 167-174 -> 146-148 us at 8 tokens per thread)
    const int t0 = __builtin_amdgcn_readfirstlane(tile * (4 * CONV_TT) + static_cast<int>(threadIdx.x >> 6) * CONV_TT);
    if (c >= D || t0 >= T || n_seqs <= 0) return;

    // the window's inputs first (rows clamped into [0, T); unused ones are
    // ignored).  Cacheable loads: the first W-1 rows of a tile are the last rows
    // of the tile before it, read again from L2 (2-7% faster than nontemporal).
    XR xv[CONV_TT + CONV_W - 1];
#pragma unroll
    for (int i = 0; i < CONV_TT + CONV_W - 1; ++i) {
        const int p = min(max(t0 - (CONV_W - 1) + i, 0), T - 1);
        xv[i] = *reinterpret_cast<const XR*>(x + static_cast<size_t>(p) * D + c);
    }
    WR wr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[j] = reinterpret_cast<const WR*>(w + static_cast<size_t>(c) * CONV_W)[j];
    const WR br = bias ? *reinterpret_cast<const WR*>(bias + c) : V4<WT>::make(0.f, 0.f, 0.f, 0.f);
    // widened once: each input feeds up to W tokens, each weight every token
    float wf[4][CONV_W], bf[4], xf[CONV_TT + CONV_W - 1][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf[e] = V4<WT>::get(br, e);
#pragma unroll
        for (int j = 0; j < CONV_W; ++j) wf[e][j] = vget<WT, 4>(wr, 4 * e + j);
    }
#pragma unroll
    for (int i = 0; i < CONV_TT + CONV_W - 1; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) xf[i][e] = V4<XT>::get(xv[i], e);

    // the sequence n with cu[n] <= t0 < cu[n + 1]
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t0) lo = mid; else hi = mid;
    }
    int n = lo;
    int st = cu[n], en = cu[n + 1];
    int32_t s = slot[n];
    const bool silu_on = (flags & GDN_FLAG_SILU) != 0;

#pragma unroll
    for (int i = 0; i < CONV_TT; ++i) {
        const int t = t0 + i;
        if (t >= T) break;
        while (t >= en && n + 1 < n_seqs) {       // sequence starts inside the tile
            ++n;
            st = en;
            en = cu[n + 1];
            s = slot[n];
        }
        if (t < st || t >= en) continue;          // outside every sequence: nothing to write
        typename V4<OT>::raw* o = reinterpret_cast<typename V4<OT>::raw*>(out + static_cast<size_t>(t) * D + c);
        if (s <= 0) {                             // inactive sequence: zeros, cache untouched
            *o = V4<OT>::make(0.f, 0.f, 0.f, 0.f);
            continue;
        }
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = bf[e];
        if (t - (CONV_W - 1) >= st) {             // the whole window is in the sequence
#pragma unroll
            for (int j = 0; j < CONV_W; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = fmaf(wf[e][j], xf[i + j][e], y[e]);
        } else {
#pragma unroll
            for (int j = 0; j < CONV_W; ++j) {
                const int p = t - (CONV_W - 1) + j;
                if (p >= st) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = fmaf(wf[e][j], xf[i + j][e], y[e]);
                } else {                          // tap m of the cached state
                    const CT* sp = cs + (static_cast<size_t>(s) * D + c) * (CONV_W - 1) + (p - st + CONV_W - 1);
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = fmaf(wf[e][j], elem<CT>::ld(sp + (CONV_W - 1) * e), y[e]);
                }
            }
        }
        if (silu_on) {
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = silu(y[e]);
        }
        {   // streaming (nontemporal) output store: 2-7% faster than a cached one
            const typename V4<OT>::raw v = V4<OT>::make(y[0], y[1], y[2], y[3]);
            if constexpr (sizeof(v) == 8) {
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                __builtin_nontemporal_store(*reinterpret_cast<const u2v*>(&v), reinterpret_cast<u2v*>(o));
            } else {
                typedef uint32_t u4v __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(*reinterpret_cast<const u4v*>(&v), reinterpret_cast<u4v*>(o));
            }
        }
    }
}

// Roll of the conv cache after conv_varlen_tok_kernel: the new state of an
// active sequence of length L > 0 is the last W-1 entries of [state | tokens],
// copied as raw bits (a token is rounded to the cache dtype when the dtypes
// differ).  grid = (ceil(D / 1024), n_seqs); a thread owns 4 channels.
template <typename XT, typename CT>
__global__ __launch_bounds__(256) void conv_roll_kernel(
    const XT* __restrict__ x, const int32_t* __restrict__ cu, const int32_t* __restrict__ slot,
    CT* __restrict__ cs, int32_t D, const int32_t* __restrict__ err_flag) {
    typedef typename V4<XT>::raw XR;
    typedef typename V4<CT>::raw CR;
    if (call_rejected(err_flag)) return;
    const int c = 4 * (static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x));
    const int n = blockIdx.y;
    if (c >= D) return;
    const int st = cu[n];
    const int L = cu[n + 1] - st;
    const int32_t s = slot[n];
    if (s <= 0 || L <= 0) return;
    CR* sp = reinterpret_cast<CR*>(cs + (static_cast<size_t>(s) * D + c) * (CONV_W - 1));
    CR raw[CONV_W - 1];
    if (L < CONV_W - 1) {
#pragma unroll
        for (int j = 0; j < CONV_W - 1; ++j) raw[j] = sp[j];
    }
    uint32_t nb[4 * (CONV_W - 1)];
#pragma unroll
    for (int m = 0; m < CONV_W - 1; ++m) {
        const int q = L - (CONV_W - 1) + m;       // position of new tap m within the tokens
        if (q >= 0) {
            const XR xin = *reinterpret_cast<const XR*>(x + static_cast<size_t>(st + q) * D + c);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                nb[(CONV_W - 1) * e + m] = std::is_same<XT, CT>::value ? V4<XT>::bits(xin, e)
                                                                       : V4<CT>::to_bits(V4<XT>::get(xin, e));
        } else {                                  // old tap q + W-1 (constant indices)
#pragma unroll
            for (int k = 0; k < CONV_W - 1; ++k) {
                if (q + (CONV_W - 1) == k) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        nb[(CONV_W - 1) * e + m] = vbits<CT, CONV_W - 1>(raw, (CONV_W - 1) * e + k);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CONV_W - 1; ++j)
        st_nt<CR>(sp + j, V4<CT>::make_bits(nb[4 * j], nb[4 * j + 1], nb[4 * j + 2], nb[4 * j + 3]));
}

// ---------------------------------------------------------------------------
// Varlen, general (any dim, any alignment): grid = (ceil(D / 64), n_seqs), 256
// threads = 64 channels x 4 token lanes; token lane tg handles tokens tg,
// tg+4, ...  The old state is read into registers by every thread before a
// barrier; after it, token lane 0 alone writes the rolled state.
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
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename XT, typename CT, typename WT, typename OT>
struct VarlenK {
    static hipError_t run(const void* x, const int32_t* cu, int32_t n_seqs, int32_t T,
                          const int32_t* slot, void* cs, const void* w, const void* bias,
                          void* out, int32_t D, int32_t flags, const int32_t* err, hipStream_t st) {
        const bool vec = D % 4 == 0 && a16(x) && a16(out) && a16(cs) && a16(w) && (!bias || a16(bias)) &&
                         (static_cast<size_t>(D) * sizeof(XT)) % 8 == 0;
        if (vec) {
            if (T > 0) {
                const size_t nblk = static_cast<size_t>((T + 4 * CONV_TT - 1) / (4 * CONV_TT)) *
                                    static_cast<size_t>((D / 4 + 63) / 64);
                if (nblk > 0x7fffffffu) return hipErrorInvalidValue;
                dim3 grid(static_cast<unsigned>(nblk));
                const hipError_t e = launch(conv_varlen_tok_kernel<XT, CT, WT, OT>, grid, dim3(256), 0, st,
                                            static_cast<const XT*>(x), cu, n_seqs, T, slot,
                                            static_cast<const CT*>(cs), static_cast<const WT*>(w),
                                            static_cast<const WT*>(bias), static_cast<OT*>(out), D,
                                            flags, err);
                if (e != hipSuccess) return e;
            }
            dim3 rgrid((D / 4 + 255) / 256, n_seqs);
            return launch(conv_roll_kernel<XT, CT>, rgrid, dim3(256), 0, st,
                          static_cast<const XT*>(x), cu, slot, static_cast<CT*>(cs), D, err);
        }
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
                              int32_t n_seqs, int32_t total_tokens, const int32_t* slot_idx,
                              void* conv_state, gdn_dtype cs_dt, const void* weight,
                              const void* bias, gdn_dtype w_dt, void* out, gdn_dtype out_dt,
                              int32_t dim, int32_t flags, const int32_t* err_flag,
                              hipStream_t stream) {
    if (n_seqs == 0) return hipSuccess;
    return pick_all<VarlenK>(x_dt, cs_dt, w_dt, out_dt, x, cu_seqlens, n_seqs, total_tokens,
                             slot_idx, conv_state, weight, bias, out, dim, flags, err_flag, stream);
}

}  // namespace gdn
