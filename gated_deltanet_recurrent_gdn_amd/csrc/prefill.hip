// prefill.hip -- varlen chunked gated delta-rule prefill on bf16 MFMA (gfx950).
//
// Method.  For one value head, a chunk of L <= 64 tokens and the state S0 at
// its start (o = S q, S[v, k]), with gamma_r = sum_{i<=r} g_i:
//   A[r,i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)  (i < r),  T = (I + A)^-1
//   W  = T diag(beta e^gamma) K          Ut = T diag(beta) V
//   U  = Ut - W S0^T                     (row r: beta_r times the delta of token r)
//   O  = diag(e^gamma) Q S0^T + (M o P) U, P = Q K^T, M[r,i] = exp(gamma_r - gamma_i), i <= r
//   S1 = e^{gamma_L} S0 + U^T diag(exp(gamma_L - gamma)) K
// which equals the token-by-token recurrence S_t = exp(g_t) S (I - b k k^T) +
// b v k^T exactly in exact arithmetic.  The 64-token chunk and the inverse of
// the lower-triangular KK^T matrix through its 16x16 diagonal blocks follow
// vLLM PR #53864 ("Numerical root cause and fix"); the diagonal blocks are
// inverted by exact fp32 forward substitution (not Newton-Schulz) and merged
// 16 -> 32 -> 64 with T21 = -T22 A21 T11.
//
// Design.  One workgroup per (sequence, value head) walks the sequence's
// chunks in order with the state resident on chip: wave w owns 32 value
// columns of S0^T (DK x DV) in MFMA accumulator registers.  Every contraction
// is v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Raw bf16 inputs (K, Q,
// V) are exact MFMA operands; fp32-derived operands that the error budget
// cannot afford to round once (T-derived coefficients, U, the masked decayed
// Q K^T block, S0) are split into bf16 hi + lo parts and contracted as
// hi*x + lo*x (and hi*hi + hi*lo + lo*hi when both sides are split), which
// keeps ~16 mantissa bits; W is used rounded to bf16 once.
//
// Operand layouts.  For 16x16x32, lane l supplies A[l%16][k] and B[k][l%16]
// for 8 k-slots selected by q = l/16, and holds D[4q + r][l%16], r < 4.  A
// contraction only needs A and B to agree on which k each (q, slot) means:
// "standard" slots are k = 8q + s; "permuted" slots are k = 4q + s (s < 4) and
// 16 + 4q + s - 4 (s >= 4), which is exactly what two vertically adjacent
// accumulator tiles hold in one lane.  With permuted slots the state, U and
// (cK . U) feed MFMA B operands straight from accumulator registers.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int CH = 64;          // chunk length (tokens)
constexpr int PADB = 8;         // bf16 row padding (16 bytes) against LDS bank conflicts
constexpr int PADF = 4;         // fp32 row padding

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack2(bf16_t lo, bf16_t hi) {
    return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// Split four floats into packed bf16 hi parts and packed bf16 lo parts.
__device__ __forceinline__ void split4(const f32x4& x, uint2& hi, uint2& lo) {
    bf16_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = f32_to_bf16(x[j]);
        l[j] = f32_to_bf16(x[j] - bf16_to_f32(h[j]));
    }
    hi = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
    lo = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
}

__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }

// Standard-slot fragment: 8 consecutive bf16 at row `row`, column c0 + 8q.
__device__ __forceinline__ bf16x8 frag_std(const bf16_t* base, int stride, int row, int c0, int q) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(base + row * stride + c0 + 8 * q));
}
// Permuted-slot fragment: 4 bf16 at c0 + 4q and 4 bf16 at c0 + 16 + 4q.
__device__ __forceinline__ bf16x8 frag_perm(const bf16_t* base, int stride, int row, int c0, int q) {
    const uint2 a = *reinterpret_cast<const uint2*>(base + row * stride + c0 + 4 * q);
    const uint2 b = *reinterpret_cast<const uint2*>(base + row * stride + c0 + 16 + 4 * q);
    return as_bf16x8(cat(a, b));
}

template <int DK, int DV, typename IT, typename OT>
struct PrefillSmem {
    static constexpr int SK = DK + PADB;        // row stride of K, Q, W (bf16)
    static constexpr int ST = CH + PADB;        // row stride of K^T, V^T, coefficient arrays
    static constexpr int SF = CH + PADF;        // row stride of fp32 64x64 arrays
    bf16_t k[CH * SK];                          // K   [t][k]
    bf16_t q[CH * SK];                          // Q   [t][k]
    bf16_t kt[DK * ST];                         // K^T [k][t]
    bf16_t vt_w[(DV * ST > CH * SK) ? DV * ST : CH * SK];   // V^T [v][t], later -W [t][k]
    float g[CH * SF];                           // K K^T -> A -> T (and merge scratch)
    union {
        float p[CH * SF];                       // Q K^T
        bf16_t c[4 * CH * ST];                  // cW hi, cW lo, cU hi, cU lo   [t][t']
    } pc;
    bf16_t mp[2 * CH * ST];                     // (M o P) hi, lo   [t][t']
    float gam[CH], beta[CH], rk[CH], rq[CH], eg[CH], ck[CH], cwc[CH];
    float egl;
};

template <int DK, int DV, typename IT, typename OT>
__global__ __launch_bounds__(256) void prefill_kernel(
    const IT* __restrict__ qg, const IT* __restrict__ kg, const IT* __restrict__ vg,
    const float* __restrict__ gg, const float* __restrict__ bg, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slot, float* __restrict__ rec, OT* __restrict__ out, int32_t H,
    int32_t HV, float scale, int32_t flags, const int32_t* __restrict__ err_flag) {
    static_assert(DK == DV, "square heads");
    static_assert(DV == 128 || DV == 64, "value head dim");
    constexpr int NW = 4;                        // waves
    constexpr int VB = DV / 16 / NW;             // value blocks (16 wide) per wave
    constexpr int KB = DK / 16;                  // key blocks (16 tall)
    constexpr int KS = DK / 32;                  // k-steps over DK
    using Sm = PrefillSmem<DK, DV, IT, OT>;
    constexpr int SK = Sm::SK, ST = Sm::ST, SF = Sm::SF;
    __shared__ Sm sm;

    if (call_rejected(err_flag)) return;
    const int hv = blockIdx.x;
    const int n = blockIdx.y;
    const int h = hv / (HV / H);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int q4 = lane >> 4;                    // lane / 16
    const int l16 = lane & 15;
    const int32_t t0 = cu[n];
    const int32_t t1 = cu[n + 1];
    const int32_t s = slot[n];

    if (s <= 0) {                                // inactive: zero outputs, state untouched
        for (int64_t i = tid; i < static_cast<int64_t>(t1 - t0) * DV; i += 256) {
            const int64_t t = t0 + i / DV;
            elem<OT>::st(out + (t * HV + hv) * DV + i % DV, 0.0f);
        }
        return;
    }
    if (t1 <= t0) return;                        // empty sequence: state untouched

    float* S = rec + (static_cast<size_t>(s) * HV + hv) * static_cast<size_t>(DV) * DK;

    // ---- state S0^T [k][v] in accumulator layout: tile (kb, vb) lane holds
    //      S0^T[16 kb + 4 q4 + r][16 (wave VB + vb) + l16] = S[v][k..k+3]
    f32x4 st[KB][VB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
            const int v = 16 * (wave * VB + vb) + l16;
            const float4 x = *reinterpret_cast<const float4*>(S + static_cast<size_t>(v) * DK + 16 * kb + 4 * q4);
            st[kb][vb] = f32x4{x.x, x.y, x.z, x.w};
        }

    for (int32_t c0 = t0; c0 < t1; c0 += CH) {
        const int L = min(CH, t1 - c0);

        // ---------------- load the chunk: K, Q (row-major), K^T, V^T, g, beta
        for (int i = tid; i < CH * DK / 8; i += 256) {
            const int t = i / (DK / 8);
            const int k0 = (i % (DK / 8)) * 8;
            uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
            if (t < L) {
                const size_t off = (static_cast<size_t>(c0 + t) * H + h) * DK + k0;
                kv = *reinterpret_cast<const uint4*>(kg + off);
                qv = *reinterpret_cast<const uint4*>(qg + off);
            }
            *reinterpret_cast<uint4*>(&sm.k[t * SK + k0]) = kv;
            *reinterpret_cast<uint4*>(&sm.q[t * SK + k0]) = qv;
            const bf16_t* kb16 = reinterpret_cast<const bf16_t*>(&kv);
#pragma unroll
            for (int j = 0; j < 8; ++j) sm.kt[(k0 + j) * ST + t] = kb16[j];
        }
        for (int i = tid; i < CH * DV / 8; i += 256) {
            const int t = i / (DV / 8);
            const int v0 = (i % (DV / 8)) * 8;
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (t < L) vv = *reinterpret_cast<const uint4*>(vg + (static_cast<size_t>(c0 + t) * HV + hv) * DV + v0);
            const bf16_t* vb16 = reinterpret_cast<const bf16_t*>(&vv);
#pragma unroll
            for (int j = 0; j < 8; ++j) sm.vt_w[(v0 + j) * ST + t] = vb16[j];
        }
        if (tid < CH) {
            const bool ok = tid < L;
            sm.beta[tid] = ok ? bg[static_cast<size_t>(c0 + tid) * HV + hv] : 0.0f;
            sm.gam[tid] = ok ? gg[static_cast<size_t>(c0 + tid) * HV + hv] : 0.0f;
        }
        __syncthreads();

        // ---------------- G = K K^T and P = Q K^T (raw bf16, exact products)
        {
            const int tb = wave;                 // wave computes row block tb of G and P
            f32x4 accg[4], accp[4];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) { accg[jb] = f32x4{0, 0, 0, 0}; accp[jb] = f32x4{0, 0, 0, 0}; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ak = frag_std(sm.k, SK, 16 * tb + l16, 32 * ks, q4);
                const bf16x8 aq = frag_std(sm.q, SK, 16 * tb + l16, 32 * ks, q4);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    const bf16x8 bk = frag_std(sm.k, SK, 16 * jb + l16, 32 * ks, q4);
                    accg[jb] = mfma(ak, bk, accg[jb]);
                    accp[jb] = mfma(aq, bk, accp[jb]);
                }
            }
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sm.g[(16 * tb + 4 * q4 + r) * SF + 16 * jb + l16] = accg[jb][r];
                    sm.pc.p[(16 * tb + 4 * q4 + r) * SF + 16 * jb + l16] = accp[jb][r];
                }
        }
        // ---------------- row norms (8 lanes per row, the decode kernel's order) + gamma
        {
            // 64 K rows then 64 Q rows; 256 threads = 32 rows per pass
            for (int pass = 0; pass < 4; ++pass) {
                const int rowid = pass * 32 + (tid >> 3);
                const int sub = tid & 7;
                const bf16_t* rowp = (rowid < CH) ? &sm.k[rowid * SK] : &sm.q[(rowid - CH) * SK];
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < DK / 32; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = bf16_to_f32(rowp[32 * i + 4 * sub + e]);
                        acc = fmaf(x, x, acc);
                    }
                acc = sum8(acc);
                if (sub == 0) {
                    if (rowid < CH)
                        sm.rk[rowid] = (flags & GDN_FLAG_QK_L2NORM) ? 1.0f / sqrtf(acc + 1e-6f) : 1.0f;
                    else
                        sm.rq[rowid - CH] = (flags & GDN_FLAG_QK_L2NORM) ? scale / sqrtf(acc + 1e-6f) : scale;
                }
            }
            if (tid == 0) {                      // cumulative log-decay, sequential order
                float a = 0.f;
                for (int t = 0; t < CH; ++t) { a += sm.gam[t]; sm.gam[t] = a; }
            }
        }
        __syncthreads();

        // ---------------- per-token coefficient vectors
        if (tid < CH) {
            const float gl = sm.gam[L - 1];
            const float gt = sm.gam[tid];
            const float et = expf(gt);
            sm.eg[tid] = et * sm.rq[tid];
            sm.ck[tid] = (tid < L) ? expf(gl - gt) * sm.rk[tid] : 0.0f;
            sm.cwc[tid] = sm.beta[tid] * et * sm.rk[tid];
            if (tid == 0) sm.egl = expf(gl);
        }
        // ---------------- A (in sm.g) and M o P (split into sm.mp)
        for (int i = tid; i < CH * CH; i += 256) {
            const int r = i / CH, c = i % CH;
            const float dec = (c <= r) ? expf(sm.gam[r] - sm.gam[c]) : 0.0f;
            const float a = (c < r) ? sm.beta[r] * dec * (sm.g[r * SF + c] * (sm.rk[r] * sm.rk[c])) : 0.0f;
            sm.g[r * SF + c] = a;
            const float mp = dec * (sm.pc.p[r * SF + c] * (sm.rq[r] * sm.rk[c]));
            const bf16_t hi = f32_to_bf16(mp);
            sm.mp[r * ST + c] = hi;
            sm.mp[CH * ST + r * ST + c] = f32_to_bf16(mp - bf16_to_f32(hi));
        }
        __syncthreads();

        // ---------------- T = (I + A)^-1: diagonal 16x16 blocks by forward substitution
        if (wave == 0) {
            const int b = lane >> 4;             // block
            const int c = lane & 15;             // column within the block
            float tc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) tc[r] = (r == c) ? 1.0f : 0.0f;
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j)
                    acc = fmaf(sm.g[(16 * b + r) * SF + 16 * b + j], tc[j], acc);
                tc[r] = (r > c) ? -acc : tc[r];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.g[(16 * b + r) * SF + 16 * b + c] = tc[r];
        }
        __syncthreads();
        // merge 16 -> 32 for block pairs (0,1) and (2,3):  T21 = -T22 (A21 T11).
        // X = A21 T11 goes to the (unused) upper block T[16p .. 16p+15][16p+16 ..].
        for (int i = tid; i < 2 * 256; i += 256) {
            const int p = i >> 8, e = i & 255, r = e >> 4, c = e & 15;
            const int b0 = 32 * p, b1 = b0 + 16;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc = fmaf(sm.g[(b1 + r) * SF + b0 + j], sm.g[(b0 + j) * SF + b0 + c], acc);
            sm.g[(b0 + r) * SF + b1 + c] = acc;
        }
        __syncthreads();
        for (int i = tid; i < 2 * 256; i += 256) {
            const int p = i >> 8, e = i & 255, r = e >> 4, c = e & 15;
            const int b0 = 32 * p, b1 = b0 + 16;
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc = fmaf(sm.g[(b1 + r) * SF + b1 + j], sm.g[(b0 + j) * SF + b1 + c], acc);
            sm.g[(b1 + r) * SF + b0 + c] = -acc;
        }
        __syncthreads();
        // merge 32 -> 64: X = A[32:64][0:32] T[0:32][0:32] -> T[0:32][32:64]
        for (int i = tid; i < 1024; i += 256) {
            const int r = i >> 5, c = i & 31;
            float acc = 0.f;
#pragma unroll 8
            for (int j = 0; j < 32; ++j) {
                const float tv = (j >= c) ? sm.g[j * SF + c] : 0.0f;   // T11 lower part only
                acc = fmaf(sm.g[(32 + r) * SF + j], tv, acc);
            }
            sm.g[r * SF + 32 + c] = acc;
        }
        __syncthreads();
        for (int i = tid; i < 1024; i += 256) {
            const int r = i >> 5, c = i & 31;
            float acc = 0.f;
#pragma unroll 8
            for (int j = 0; j < 32; ++j) {
                const float tv = (r >= j) ? sm.g[(32 + r) * SF + 32 + j] : 0.0f;   // T22 lower
                acc = fmaf(tv, sm.g[j * SF + 32 + c], acc);
            }
            sm.g[(32 + r) * SF + c] = -acc;
        }
        __syncthreads();

        // ---------------- coefficients cW = T diag(cwc), cU = T diag(beta), split
        for (int i = tid; i < CH * CH; i += 256) {
            const int r = i / CH, c = i % CH;
            // T is lower triangular with unit diagonal; the upper part of sm.g
            // holds merge scratch and is masked here.
            const float tv = (c < r) ? sm.g[r * SF + c] : ((c == r) ? 1.0f : 0.0f);
            const float w = tv * sm.cwc[c];
            const float u = tv * sm.beta[c];
            const bf16_t wh = f32_to_bf16(w), uh = f32_to_bf16(u);
            sm.pc.c[0 * CH * ST + r * ST + c] = wh;
            sm.pc.c[1 * CH * ST + r * ST + c] = f32_to_bf16(w - bf16_to_f32(wh));
            sm.pc.c[2 * CH * ST + r * ST + c] = uh;
            sm.pc.c[3 * CH * ST + r * ST + c] = f32_to_bf16(u - bf16_to_f32(uh));
        }
        __syncthreads();

        // ---------------- Ut = cU V (wave's value columns) and W = cW K
        f32x4 u[4][VB];                          // U tiles (t-block, v-block): rows t, cols v
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) u[tb][vb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 ah = frag_std(sm.pc.c + 2 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
                const bf16x8 al = frag_std(sm.pc.c + 3 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    const bf16x8 bv = frag_std(sm.vt_w, ST, 16 * (wave * VB + vb) + l16, 32 * ks, q4);
                    u[tb][vb] = mfma(ah, bv, u[tb][vb]);
                    u[tb][vb] = mfma(al, bv, u[tb][vb]);
                }
            }
        constexpr int WB = KB / NW;              // key blocks of W per wave
        f32x4 w[4][WB];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int kb = 0; kb < WB; ++kb) w[tb][kb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 ah = frag_std(sm.pc.c + 0 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
                const bf16x8 al = frag_std(sm.pc.c + 1 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
#pragma unroll
                for (int kb = 0; kb < WB; ++kb) {
                    const bf16x8 bk = frag_std(sm.kt, ST, 16 * (wave * WB + kb) + l16, 32 * ks, q4);
                    w[tb][kb] = mfma(ah, bk, w[tb][kb]);
                    w[tb][kb] = mfma(al, bk, w[tb][kb]);
                }
            }
        __syncthreads();                         // V^T is dead: its space takes -W
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int kb = 0; kb < WB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.vt_w[(16 * tb + 4 * q4 + r) * SK + 16 * (wave * WB + kb) + l16] = f32_to_bf16(-w[tb][kb][r]);

        // ---------------- split the state into hi/lo B fragments (permuted k-slots)
        bf16x8 sh[KS][VB], sl[KS][VB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
                uint2 h0, l0, h1, l1;
                split4(st[2 * ks][vb], h0, l0);
                split4(st[2 * ks + 1][vb], h1, l1);
                sh[ks][vb] = as_bf16x8(cat(h0, h1));
                sl[ks][vb] = as_bf16x8(cat(l0, l1));
            }
        __syncthreads();                         // -W visible to all waves

        // ---------------- U = Ut - W S0^T ;  O1 = Q S0^T
        f32x4 o[4][VB];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) o[tb][vb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 aw = frag_perm(sm.vt_w, SK, 16 * tb + l16, 32 * ks, q4);
                const bf16x8 aq = frag_perm(sm.q, SK, 16 * tb + l16, 32 * ks, q4);
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    u[tb][vb] = mfma(aw, sh[ks][vb], u[tb][vb]);
                    u[tb][vb] = mfma(aw, sl[ks][vb], u[tb][vb]);
                    o[tb][vb] = mfma(aq, sh[ks][vb], o[tb][vb]);
                    o[tb][vb] = mfma(aq, sl[ks][vb], o[tb][vb]);
                }
            }
        // O1 rows scaled by e^gamma_t rq_t
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = sm.eg[16 * tb + 4 * q4 + r];
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) o[tb][vb][r] *= e;
            }

        // ---------------- O += (M o P) U   (U split, permuted t-slots)
        bf16x8 uh[2][VB], ul[2][VB];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
                uint2 h0, l0, h1, l1;
                split4(u[2 * ks][vb], h0, l0);
                split4(u[2 * ks + 1][vb], h1, l1);
                uh[ks][vb] = as_bf16x8(cat(h0, h1));
                ul[ks][vb] = as_bf16x8(cat(l0, l1));
            }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (32 * ks > 16 * tb + 15) continue;          // strictly above the diagonal
                const bf16x8 mh = frag_perm(sm.mp, ST, 16 * tb + l16, 32 * ks, q4);
                const bf16x8 ml = frag_perm(sm.mp + CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    o[tb][vb] = mfma(mh, uh[ks][vb], o[tb][vb]);
                    o[tb][vb] = mfma(mh, ul[ks][vb], o[tb][vb]);
                    o[tb][vb] = mfma(ml, uh[ks][vb], o[tb][vb]);
                }
            }
        // store O rows t < L
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tb + 4 * q4 + r;
                if (t < L) {
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb)
                        elem<OT>::st(out + (static_cast<size_t>(c0 + t) * HV + hv) * DV + 16 * (wave * VB + vb) + l16,
                                     o[tb][vb][r]);
                }
            }

        // ---------------- S0^T <- e^{gamma_L} S0^T + K^T (cK . U)
        bf16x8 ch[2][VB], cl[2][VB];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
                f32x4 a = u[2 * ks][vb], b = u[2 * ks + 1][vb];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a[r] *= sm.ck[32 * ks + 4 * q4 + r];
                    b[r] *= sm.ck[32 * ks + 16 + 4 * q4 + r];
                }
                uint2 h0, l0, h1, l1;
                split4(a, h0, l0);
                split4(b, h1, l1);
                ch[ks][vb] = as_bf16x8(cat(h0, h1));
                cl[ks][vb] = as_bf16x8(cat(l0, l1));
            }
        const float egl = sm.egl;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
                f32x4 acc = st[kb][vb];
                acc[0] *= egl; acc[1] *= egl; acc[2] *= egl; acc[3] *= egl;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 ak = frag_perm(sm.kt, ST, 16 * kb + l16, 32 * ks, q4);
                    acc = mfma(ak, ch[ks][vb], acc);
                    acc = mfma(ak, cl[ks][vb], acc);
                }
                st[kb][vb] = acc;
            }
        __syncthreads();                         // LDS is rewritten by the next chunk
    }

    // ---- final state back to the slot
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
            const int v = 16 * (wave * VB + vb) + l16;
            *reinterpret_cast<float4*>(S + static_cast<size_t>(v) * DK + 16 * kb + 4 * q4) =
                make_float4(st[kb][vb][0], st[kb][vb][1], st[kb][vb][2], st[kb][vb][3]);
        }
}

namespace {
template <int D, typename OT>
hipError_t run_prefill(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const int32_t* cu, int32_t n_seqs, const int32_t* slot,
                       float* rec, void* out, const gdn_dims& d, float scale, int32_t flags,
                       const int32_t* err, hipStream_t st) {
    dim3 grid(d.num_v_heads, n_seqs);
    return launch(prefill_kernel<D, D, bf16_t, OT>, grid, dim3(256), 0, st,
                  static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                  static_cast<const bf16_t*>(v), g, beta, cu, slot, rec, static_cast<OT*>(out),
                  d.num_k_heads, d.num_v_heads, scale, flags, err);
}
}  // namespace

bool prefill_supported(const gdn_dims& d, gdn_dtype in_dt) {
    return in_dt == GDN_BF16 && d.head_k_dim == d.head_v_dim &&
           (d.head_k_dim == 128 || d.head_k_dim == 64);
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                          const float* g, const float* beta, const int32_t* cu, int32_t n_seqs,
                          const int32_t* slot, float* rec, void* out, gdn_dtype out_dt,
                          const gdn_dims& d, float scale, int32_t flags, const int32_t* err,
                          hipStream_t st) {
    if (n_seqs == 0) return hipSuccess;
    if (!prefill_supported(d, in_dt)) return hipErrorInvalidValue;
    if (d.head_k_dim == 128)
        return out_dt == GDN_BF16
            ? run_prefill<128, bf16_t>(q, k, v, g, beta, cu, n_seqs, slot, rec, out, d, scale, flags, err, st)
            : run_prefill<128, float>(q, k, v, g, beta, cu, n_seqs, slot, rec, out, d, scale, flags, err, st);
    return out_dt == GDN_BF16
        ? run_prefill<64, bf16_t>(q, k, v, g, beta, cu, n_seqs, slot, rec, out, d, scale, flags, err, st)
        : run_prefill<64, float>(q, k, v, g, beta, cu, n_seqs, slot, rec, out, d, scale, flags, err, st);
}

}  // namespace gdn
