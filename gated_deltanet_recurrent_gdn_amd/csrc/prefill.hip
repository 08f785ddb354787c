// prefill.hip -- varlen chunked gated delta-rule prefill on bf16 MFMA (gfx950).
//
// Method.  For one value head, a chunk of L <= 64 tokens and the state S0 at
// its start (o = S q, S[v, k]), with gamma_r = sum_{i<=r} g_i:
//   A[r,i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)  (i < r),  T = (I + A)^-1
//   W  = T diag(beta e^gamma) K          Ut = T diag(beta) V
//   U  = Ut - W S0^T                     (row r: beta_r times the delta of token r)
//   O  = diag(e^gamma) Q S0^T + (M o P) U, P = Q K^T, M[r,i] = exp(gamma_r - gamma_i), i <= r
//   S1 = e^{gamma_L} S0 + U^T diag(exp(gamma_L - gamma)) K
// The kernel forms U as cU (V - diag(e^gamma) K S0^T) with cU = T diag(beta):
// W and Ut share the factor T diag(beta), so one coefficient matrix serves.
// which equals the token-by-token recurrence S_t = exp(g_t) S (I - b k k^T) +
// b v k^T exactly in exact arithmetic.  The 64-token chunk and the inverse of
// the lower-triangular KK^T matrix through its 16x16 diagonal blocks follow
// vLLM PR #53864 ("Numerical root cause and fix"); the diagonal blocks are
// inverted by exact fp32 forward substitution (not Newton-Schulz) and merged
// 16 -> 32 -> 64 with T21 = -T22 A21 T11.
//
// Design.  One workgroup of eight waves per (sequence, value head) walks the
// sequence's chunks in order with the state resident on chip: wave w owns 16
// value columns of S0^T (DK x DV) in MFMA accumulator registers (two waves per
// SIMD, so one wave's LDS and MFMA latency hides behind the other's work).  Every contraction
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
#include <type_traits>

#include "gate.hpp"
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int CH = 64;          // chunk length (tokens)
// bf16 row padding.  The MFMA fragment reads are 16-byte ds_read_b128 with lane l
// on row l % 16 and 16-byte column block l / 16; the LDS serves them 16 lanes a
// cycle over 64 banks, and a one-wave probe found them conflict-free when the
// row stride in 4-byte words is 8 mod 16 (2-way at 4 mod 16).  Every bf16
// operand array takes such a stride.  K and Q are also swizzled (kq_swz).
constexpr int PADK = 16;
constexpr int PADT = 16;

// K and Q swizzle: row r's 16-byte units are XOR-permuted within each 64-byte
// group by (r / 4) % 4.  A lane's 8-byte row stores of token pairs 2tp, 2tp+1
// then spread over 8 bank pairs instead of 2 (2-way instead of 8-way at the
// 8 mod 16 stride), and the fragment reads stay conflict-free: for a read
// group (lanes 0-3, 12-15, 20-27 or the rest of a half-wave) the 16 (row,
// block) pairs still land on 16 distinct 16-byte bank slots.  Element index e
// of row r sits at e ^ kq_swz(r).
__host__ __device__ constexpr int kq_swz(int r) { return ((r >> 2) & 3) << 3; }
constexpr int PADF = 4;         // fp32 row padding

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16].
__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }

// Split four floats into packed bf16 hi parts and packed bf16 lo parts
// (x = hi + lo to ~16 significant bits; x - hi is exact in fp32).
__device__ __forceinline__ void split4(const f32x4& x, uint2& hi, uint2& lo) {
    const uint32_t h01 = pack_bf16x2(x[0], x[1]), h23 = pack_bf16x2(x[2], x[3]);
    hi = make_uint2(h01, h23);
    lo = make_uint2(pack_bf16x2(x[0] - bf16lo_to_f32(h01), x[1] - bf16hi_to_f32(h01)),
                    pack_bf16x2(x[2] - bf16lo_to_f32(h23), x[3] - bf16hi_to_f32(h23)));
}

// Raw buffer access.  The descriptor holds a workgroup-uniform base and a byte
// range; each lane adds a 32-bit offset.  Loads past the range return zero and
// stores past it are dropped, which masks a partial chunk's missing rows.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_WORD3 = 0x00020000;          // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), RSRC_WORD3);
}
__device__ __forceinline__ uint4 buf_ld16(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float buf_ld4f(rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ bf16_t buf_ld2(rsrc_t r, uint32_t off) {
    return static_cast<bf16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st16(rsrc_t r, uint32_t off, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{a, b, c, d}, r, off, 0, 0);
}
// The same with the nontemporal hint (cache policy bit NT)
__device__ __forceinline__ void buf_st16_nt(rsrc_t r, uint32_t off, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{a, b, c, d}, r, off, 0, 2);
}
__device__ __forceinline__ void buf_st8(rsrc_t r, uint32_t off, uint32_t a, uint32_t b) {
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{a, b}, r, off, 0, 0);
}

// One step of an inclusive wave prefix sum: the DPP-moved value, or zero in
// lanes whose source lies outside the row or whose row is masked off.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_scan_step(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

// T = (I + A)^-1 for the four unit lower triangular 16x16 diagonal blocks
// of a chunk, one block per 16-lane row of the wave, by exact fp32 forward
// substitution in place (blk: the block's top-left element, row stride ld; the
// strictly lower part holds A, lane c of the row owns column c).
// Right-looking order: once T[j][c] is final every later row r adds
// A[r][j] T[j][c], so each row still accumulates its terms in ascending j.
// The accumulators start at -1 on the diagonal and hold -T, so the negated
// accumulator is the multiplier with no select per step (for j < c the term
// is A[r][j] * (-0), which leaves every accumulator's value as it was).
// Each term is one v_fmac_f32_dpp: the DPP row broadcast row_newbcast:j hands
// A[r][j] from lane j to the whole row inside the multiply-add (the compiler
// keeps a separate DPP move in front of each fma).  A VGPR a VALU instruction
// wrote may be read through DPP only two wait states later; A comes from LDS
// loads, and the s_nop at the top of every step covers any copy the compiler
// might place in front of the block.
#define GDN_FS_FMAC(R, J) "v_fmac_f32_dpp %[c" #R "], %[a" #R "], -%[c" #J "] row_newbcast:" #J \
                          " row_mask:0xf bank_mask:0xf\n\t"
#define GDN_FS_ROWS1(J) GDN_FS_FMAC(1, J) GDN_FS_ROWS2(J)
#define GDN_FS_ROWS2(J) GDN_FS_FMAC(2, J) GDN_FS_ROWS3(J)
#define GDN_FS_ROWS3(J) GDN_FS_FMAC(3, J) GDN_FS_ROWS4(J)
#define GDN_FS_ROWS4(J) GDN_FS_FMAC(4, J) GDN_FS_ROWS5(J)
#define GDN_FS_ROWS5(J) GDN_FS_FMAC(5, J) GDN_FS_ROWS6(J)
#define GDN_FS_ROWS6(J) GDN_FS_FMAC(6, J) GDN_FS_ROWS7(J)
#define GDN_FS_ROWS7(J) GDN_FS_FMAC(7, J) GDN_FS_ROWS8(J)
#define GDN_FS_ROWS8(J) GDN_FS_FMAC(8, J) GDN_FS_ROWS9(J)
#define GDN_FS_ROWS9(J) GDN_FS_FMAC(9, J) GDN_FS_ROWS10(J)
#define GDN_FS_ROWS10(J) GDN_FS_FMAC(10, J) GDN_FS_ROWS11(J)
#define GDN_FS_ROWS11(J) GDN_FS_FMAC(11, J) GDN_FS_ROWS12(J)
#define GDN_FS_ROWS12(J) GDN_FS_FMAC(12, J) GDN_FS_ROWS13(J)
#define GDN_FS_ROWS13(J) GDN_FS_FMAC(13, J) GDN_FS_ROWS14(J)
#define GDN_FS_ROWS14(J) GDN_FS_FMAC(14, J) GDN_FS_ROWS15(J)
#define GDN_FS_ROWS15(J) GDN_FS_FMAC(15, J)
#define GDN_FS_OUT [c0] "+v"(acc[0]), [c1] "+v"(acc[1]), [c2] "+v"(acc[2]), [c3] "+v"(acc[3]), \
                   [c4] "+v"(acc[4]), [c5] "+v"(acc[5]), [c6] "+v"(acc[6]), [c7] "+v"(acc[7]), \
                   [c8] "+v"(acc[8]), [c9] "+v"(acc[9]), [c10] "+v"(acc[10]), [c11] "+v"(acc[11]), \
                   [c12] "+v"(acc[12]), [c13] "+v"(acc[13]), [c14] "+v"(acc[14]), [c15] "+v"(acc[15])
#define GDN_FS_IN [a1] "v"(ar[1]), [a2] "v"(ar[2]), [a3] "v"(ar[3]), [a4] "v"(ar[4]), [a5] "v"(ar[5]), \
                  [a6] "v"(ar[6]), [a7] "v"(ar[7]), [a8] "v"(ar[8]), [a9] "v"(ar[9]), [a10] "v"(ar[10]), \
                  [a11] "v"(ar[11]), [a12] "v"(ar[12]), [a13] "v"(ar[13]), [a14] "v"(ar[14]), \
                  [a15] "v"(ar[15])
__device__ __forceinline__ void fwd_subst16(float* blk, int ld, int c) {
    float ar[16], acc[16];
#pragma unroll
    for (int r = 1; r < 16; ++r) ar[r] = blk[r * ld + c];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = (r == c) ? -1.0f : 0.0f;
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS1(0) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS2(1) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS3(2) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS4(3) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS5(4) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS6(5) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS7(6) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS8(7) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS9(8) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS10(9) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS11(10) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS12(11) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS13(12) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS14(13) : GDN_FS_OUT : GDN_FS_IN);
    asm volatile("s_nop 1\n\t" GDN_FS_ROWS15(14) : GDN_FS_OUT : GDN_FS_IN);
#pragma unroll
    for (int r = 0; r < 16; ++r) blk[r * ld + c] = (r < c) ? 0.0f : -acc[r];
}
#undef GDN_FS_FMAC
#undef GDN_FS_ROWS1
 #undef GDN_FS_ROWS2
 #undef GDN_FS_ROWS3
 #undef GDN_FS_ROWS4
 #undef GDN_FS_ROWS5
 #undef GDN_FS_ROWS6
 #undef GDN_FS_ROWS7
 #undef GDN_FS_ROWS8
 #undef GDN_FS_ROWS9
 #undef GDN_FS_ROWS10
 #undef GDN_FS_ROWS11
 #undef GDN_FS_ROWS12
 #undef GDN_FS_ROWS13
 #undef GDN_FS_ROWS14
 #undef GDN_FS_ROWS15
#undef GDN_FS_OUT
#undef GDN_FS_IN

// K/Q fragment (either slot order): the 8 bf16 at row `row`, columns
// (c0 + 8q) ^ kq_swz(row); row % 16 is the lane's l16, so the caller passes
// sw = kq_swz(l16) (c0 is a multiple of 32, so the XOR stays in the block).
__device__ __forceinline__ bf16x8 frag_kq(const bf16_t* base, int stride, int row, int c0, int q, int sw) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(base + row * stride + c0 + ((8 * q) ^ sw)));
}
// Standard-slot fragment: 8 consecutive bf16 at row `row`, column c0 + 8q.
__device__ __forceinline__ bf16x8 frag_std(const bf16_t* base, int stride, int row, int c0, int q) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(base + row * stride + c0 + 8 * q));
}
// Arrays read with permuted k-slots are stored with each 32-element block
// reordered: element 4b + s (b < 8, s < 4) of a block sits at position 8b + s
// for b < 4 and at 8(b - 4) + 4 + s otherwise, so the eight elements a lane's
// permuted slots name (c0 + 4q .. + 3 and c0 + 16 + 4q .. + 3) are contiguous
// at c0 + 8q: one 16-byte read with an immediate offset.  A product of two
// such arrays along their permuted dimension (K K^T, Q K^T) is unchanged.
__host__ __device__ constexpr int pperm(int e) {
    return (e & ~31) + (((e & 31) >> 2) < 4 ? 8 * ((e & 31) >> 2) : 8 * (((e & 31) >> 2) - 4) + 4) + (e & 3);
}
// Permuted-slot fragment (from an array in pperm order): the elements
// c0 + 4q .. + 3 and c0 + 16 + 4q .. + 3 of row `row`.
__device__ __forceinline__ bf16x8 frag_perm(const bf16_t* base, int stride, int row, int c0, int q) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(base + row * stride + c0 + 8 * q));
}

// Eight fp32 values (two uint4 of bits) into packed bf16 hi and lo words.
__device__ __forceinline__ void split8(const uint4& a, const uint4& b, uint4& hi, uint4& lo) {
    const float f[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                        __uint_as_float(a.w), __uint_as_float(b.x), __uint_as_float(b.y),
                        __uint_as_float(b.z), __uint_as_float(b.w)};
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
        l[j] = pack_bf16x2(f[2 * j] - bf16lo_to_f32(h[j]), f[2 * j + 1] - bf16hi_to_f32(h[j]));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// One 8-byte LDS store, kept whole (ds_write_b64).  A store through a uint2
// can reach the backend as two 32-bit halves (ds_write2_b32), which took more
// than twice the cycles of ds_write_b64 on the same strided addresses.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_st8(bf16_t* p, uint32_t a, uint32_t b) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{a, b};
}

// Store the 32-bit (t, t+1) pairs of two token rows' 8 columns into a
// transposed [col][t] array at column c0, token position ta (even; the pair
// stays adjacent under pperm).
__device__ __forceinline__ void store_pairs_t(bf16_t* arr, int stride, int c0, int ta, const uint4& ra,
                                              const uint4& rb) {
    const uint32_t* a32 = reinterpret_cast<const uint32_t*>(&ra);
    const uint32_t* b32 = reinterpret_cast<const uint32_t*>(&rb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<uint32_t*>(&arr[(c0 + 2 * j) * stride + ta]) = (a32[j] & 0xffffu) | (b32[j] << 16);
        *reinterpret_cast<uint32_t*>(&arr[(c0 + 2 * j + 1) * stride + ta]) = (a32[j] >> 16) | (b32[j] & 0xffff0000u);
    }
}

// Newton-Schulz inverse of one 16x16 unit-lower block L = I + A (A strictly
// lower, fp32 at blk with row stride sf), as the pages' CuteDSL prefill does
// it: X0 = I - A, then `rounds` times X <- X (2I - L X), with L, every product
// 2I - L X and every X rounded to bf16 (vLLM PR #53864, "Numerical root cause
// and fix": three rounds are exact in exact arithmetic for 16x16, since the
// error after round n is A^(2^(n+1)), but can fail with bf16 intermediates on
// correlated keys; four fixed it there).  The result (its bf16 values) goes
// back to blk in fp32.  One wave; scratch holds 512 bf16 (X^T, then the 2I - LX
// transpose, and X), wave-local.  Products run on v_mfma_f32_16x16x32_bf16 with
// the upper half of K zero: lane (q, i) supplies A[i][8q + s] and B[8q + s][i]
// for q < 2, zeros for q >= 2, and holds D[4q + r][i].
__device__ __forceinline__ void ns_block_inverse(float* blk, int sf, bf16_t* scratch, int rounds,
                                                 int i, int q) {
    bf16_t* Xt = scratch;          // X^T [j][k], then (2I - L X)^T
    bf16_t* Xr = scratch + 256;    // X [i][k]
    const bf16x8 zero8 = as_bf16x8(make_uint4(0, 0, 0, 0));
    // L (A operand, row i, columns 8q .. 8q+7), rounded to bf16
    bf16x8 aL = zero8;
    if (q < 2) {
        uint32_t w[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k0 = 8 * q + 2 * s;
            const float l0 = blk[i * sf + k0] + (i == k0 ? 1.0f : 0.0f);
            const float l1 = blk[i * sf + k0 + 1] + (i == k0 + 1 ? 1.0f : 0.0f);
            w[s] = pack_bf16x2(l0, l1);
        }
        aL = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
    // X0 = I - A in the accumulator layout: lane holds X0[4q + r][i]
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        x[r] = (row == i ? 1.0f : 0.0f) - blk[row * sf + i];
    }
    auto store_x = [&](const f32x4& v) {     // X^T rows (contiguous) and X rows (scattered)
        const uint32_t h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(&Xt[i * 16 + 4 * q]) = make_uint2(h01, h23);
        Xr[(4 * q + 0) * 16 + i] = static_cast<bf16_t>(h01 & 0xffffu);
        Xr[(4 * q + 1) * 16 + i] = static_cast<bf16_t>(h01 >> 16);
        Xr[(4 * q + 2) * 16 + i] = static_cast<bf16_t>(h23 & 0xffffu);
        Xr[(4 * q + 3) * 16 + i] = static_cast<bf16_t>(h23 >> 16);
    };
    store_x(x);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (int n = 0; n < rounds; ++n) {
        const bf16x8 bX = (q < 2) ? frag_std(Xt, 16, i, 0, q) : zero8;   // X[8q + s][i]
        const bf16x8 aX = (q < 2) ? frag_std(Xr, 16, i, 0, q) : zero8;   // X[i][8q + s]
        const f32x4 p = mfma(aL, bX, f32x4{0, 0, 0, 0});                   // (L X)[4q + r][i]
        f32x4 zz;
#pragma unroll
        for (int r = 0; r < 4; ++r) zz[r] = ((4 * q + r) == i ? 2.0f : 0.0f) - p[r];
        *reinterpret_cast<uint2*>(&Xt[i * 16 + 4 * q]) =
            make_uint2(pack_bf16x2(zz[0], zz[1]), pack_bf16x2(zz[2], zz[3]));   // (2I - LX)^T
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const bf16x8 bZ = (q < 2) ? frag_std(Xt, 16, i, 0, q) : zero8;   // (2I - LX)[8q + s][i]
        x = mfma(aX, bZ, f32x4{0, 0, 0, 0});                               // X (2I - L X)
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        store_x(x);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) blk[(4 * q + r) * sf + i] = bf16_to_f32(f32_to_bf16(x[r]));
}

// LDS of one workgroup.  NP planes hold a raw input as bf16 (NP = 1) or as
// bf16 hi + lo parts of fp32 values (NP = 2).
template <int D, bool SPL>
struct PrefillSmem {
    static constexpr int NP = SPL ? 2 : 1;
    static constexpr int SK = D + PADK;         // row stride of K, Q, W (bf16)
    // row stride of K^T, V^T, coefficient arrays (PADT, except where it would
    // not fit the 160 KB of LDS: hi/lo planes at D = 64)
    static constexpr int ST = CH + ((SPL && D == 64) ? 8 : PADT);
    static constexpr int SF = CH + PADF;        // row stride of fp32 64x64 arrays
    bf16_t k[NP][CH * SK];                      // K   [t][k]
    bf16_t q[NP][CH * SK];                      // Q   [t][k]
    bf16_t kt[NP][D * ST];                      // K^T [k][t]
    bf16_t vt[NP][D * ST];                      // V^T [v][t]
    float g[CH * SF];                           // A, then T in place (lower, unit diag, zero upper),
                                                // except T's block [32:64][0:32], which is in xs
    struct {
        bf16_t c[2 * CH * ST];                  // cU hi, cU lo [t][t'], pperm order along t'
    } pc;
    float xs[32 * 36];                          // merge scratch X; finally T[32:64][0:32]
    bf16_t mp[2 * CH * ST];                     // (M o P) hi, lo   [t][t']
    float gam[CH], beta[CH], rk[CH], rq[CH], eg[CH], ck[CH], cy[CH];
    float egl;
};

// D: head dim (d_k = d_v).  IT: input element type (bf16_t, or float read as
// hi/lo bf16 planes).  OT: output element type.
constexpr int PF_NW = 8;                 // waves per workgroup
constexpr int PF_NT = 64 * PF_NW;        // threads per workgroup

// Which part of each sequence a launch walks.  Pass 0: whole sequences.
// Segment passes (blockIdx.z picks the segment): segment 0 of a sequence is
// its first `head` tokens and segments 1.. are the following runs of seg_len
// tokens (head >= seg_len, both multiples of CH; a sequence of at most head
// tokens is one segment).  Pass 1 runs segment 0 from the slot's state (z = 0)
// and, for each middle segment j, its run from the zero state (its B) and its
// run from the identity with v = 0 (its P), both without outputs: paired in
// one workgroup (z = j; the P run's state is a second register array), or as
// two workgroups (z = 2j - 1 the B run, z = 2j the P run; one state, so the
// kernel keeps the registers of a whole-sequence run).  Pass 2 reruns segment
// j = z + 1 from its composed start state.  ws holds the D x D fp32 matrices
// [segment id][start, P, B][value head].
struct SegArgs {
    float* ws;
    int32_t seg_len;
    int32_t pass;
    int32_t head;
    int32_t pair;        // pass 1: P and B runs paired in one workgroup
    // Segment map (written by prefill_seg_map_kernel), so that the grid
    // carries a bound on the real workgroup count instead of every sequence
    // times the longest.  Pass 1: blockIdx.y < n_seqs is sequence blockIdx.y's
    // segment 0 (all of them dispatched first, so that no P/B run takes a CU
    // before every segment 0 has one); y = n_seqs + i indexes the P/B runs,
    // sequence n owning i in [map[n], map[n + 1]) with z = 1 + i - map[n].
    // Pass 2: sequence n owns y in [map[n], map[n + 1]), z = y - map[n].
    const int32_t* map;
    int32_t n_seqs;
};

// Segments of a sequence of L tokens (head >= seg >= 1).
__host__ __device__ inline int32_t seg_count(int32_t L, int32_t head, int32_t seg) {
    return L <= head ? 1 : 1 + (L - head + seg - 1) / seg;
}

template <int D, typename IT, typename OT, bool NSV, bool SEG, bool PAIR>
__global__ __launch_bounds__(PF_NT) void prefill_kernel(
    const IT* __restrict__ qg, const IT* __restrict__ kg, const IT* __restrict__ vg,
    const GateArgs ga, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slot, float* __restrict__ rec, OT* __restrict__ out, int32_t H,
    int32_t HV, int32_t sqk, int32_t sv, float scale, int32_t flags, int32_t ns_rounds,
    const SegArgs sg, const int32_t* __restrict__ err_flag) {
    constexpr bool SPL = sizeof(IT) == 4;        // fp32 inputs: hi/lo planes
    constexpr bool PAIRED = SEG && PAIR;         // P and B runs share a workgroup
    constexpr int NP = SPL ? 2 : 1;
    static_assert(D == 32 || D == 64 || D == 128, "head dim");
    constexpr int NW = PF_NW;                    // waves
    constexpr int KB = D / 16;                   // 16-row key blocks of the state
    constexpr int KS = D / 32;                   // 32-wide k-steps over the head dim
    constexpr int VB = (D / 16 / NW > 0) ? D / 16 / NW : 1;   // 16-wide value blocks per wave
    constexpr int CG = PF_NT / 32;               // 8-column groups per load pass
    constexpr int CP = (D / (8 * CG) > 0) ? D / (8 * CG) : 1; // load passes
    constexpr int WPE = SPL ? 2 : 1;             // uint4 words per 8 input elements
    using Sm = PrefillSmem<D, SPL>;
    constexpr int SK = Sm::SK, ST = Sm::ST, SF = Sm::SF;
    __shared__ Sm sm;

    if (call_rejected(err_flag)) return;
    // Value heads to workgroups so that the G = HV / H heads sharing a key head
    // get workgroup ids 8 apart (workgroups go to the 8 XCDs round-robin by
    // id, and each XCD has its own L2): they then read that key head's q and k
    // through one L2.  Needs HV % 8 == 0 and H % 8 == 0; identity otherwise.
    int hv = blockIdx.x;
    {
        const int G = HV / H;
        if (HV % 8 == 0 && H % 8 == 0) {
            const int a = hv >> 3, b = hv & 7;
            hv = G * (8 * (a / G) + b) + a % G;
        }
    }
    // the sequence and the segment index within its pass: from the grid, or,
    // for segment passes, from the segment map (binary search)
    int n = blockIdx.y;
    int zseg = blockIdx.z;
    if constexpr (SEG) {
        int g = blockIdx.y;
        if (sg.pass == 1 && g < sg.n_seqs) {
            zseg = 0;                            // segment 0 of sequence g
        } else {
            const int base = sg.pass == 1 ? 1 : 0;
            if (sg.pass == 1) g -= sg.n_seqs;
            if (g >= sg.map[sg.n_seqs]) return;
            int lo = 0, hi = sg.n_seqs;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (sg.map[mid] <= g) lo = mid; else hi = mid;
            }
            n = lo;
            zseg = base + g - sg.map[lo];
        }
    }
    const int h = hv / (HV / H);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int q4 = lane >> 4;                    // lane / 16
    const int l16 = lane & 15;
    const int32_t t0 = cu[n];
    const int32_t t1 = cu[n + 1];
    const int32_t s = slot[n];
    const bool norm = (flags & GDN_FLAG_QK_L2NORM) != 0;
    const bool vact = wave * VB * 16 < D;        // this wave owns value columns

    if (s <= 0) {                                // inactive: zero outputs, state untouched
        if (SEG && (sg.pass == 2 || zseg != 0)) return;
        for (int64_t i = tid; i < static_cast<int64_t>(t1 - t0) * D; i += PF_NT) {
            const int64_t t = t0 + i / D;
            elem<OT>::st(out + (t * HV + hv) * D + i % D, 0.0f);
        }
        return;
    }
    if (t1 <= t0) return;                        // empty sequence: state untouched

    float* S = rec + (static_cast<size_t>(s) * HV + hv) * static_cast<size_t>(D) * D;

    // The tokens [a0, a1) this workgroup walks, where its start state comes
    // from (`init`; nullptr: the zero state), whether it writes outputs, and
    // where its end state goes (nullptr: dropped).  A paired workgroup (pb)
    // also carries a second state from the identity with v = 0 (a middle
    // segment's P run beside its B run, sharing every intra-chunk step) and
    // writes it to fin2.  Whole-sequence launches (SEG false) compile none of
    // the segment logic.
    int32_t a0 = t0, a1 = t1;
    const float* init = S;
    float* fin = S;
    float* fin2 = nullptr;
    bool wo = true, pb = false, ident = false, use_v = true;
    if constexpr (SEG) {
        const int32_t seg = sg.seg_len;
        const int32_t nseg = seg_count(t1 - t0, sg.head, seg);
        const int64_t id0 = n + t0 / seg;        // segment id of the sequence's first segment
        auto seg_start = [&](int j) { return j == 0 ? t0 : t0 + sg.head + (j - 1) * seg; };
        auto wsm = [&](int64_t id, int kind) {
            return sg.ws + ((id * 3 + kind) * HV + hv) * static_cast<size_t>(D) * D;
        };
        const int z = zseg;
        if (sg.pass == 1) {
            const int j = z;
            if (nseg <= 1) {
                if (z != 0) return;              // one segment: the whole run, as pass 0
            } else if (j == 0) {
                a1 = t0 + sg.head;
                fin = wsm(id0 + 1, 0);           // start state of segment 1
            } else if constexpr (PAIR) {
                if (j > nseg - 2) return;
                a0 = seg_start(j);
                a1 = a0 + seg;
                wo = false;
                pb = true;
                init = nullptr;
                fin = wsm(id0 + j, 2);           // B: the run from zero
                fin2 = wsm(id0 + j, 1);          // P: the run from the identity, v = 0
            } else {
                const int jj = (z + 1) / 2;      // z = 2 jj - 1: B run, z = 2 jj: P run
                if (jj > nseg - 2) return;
                a0 = seg_start(jj);
                a1 = a0 + seg;
                wo = false;
                init = nullptr;
                if (z & 1) {
                    fin = wsm(id0 + jj, 2);      // B: the run from zero
                } else {
                    fin = wsm(id0 + jj, 1);      // P: the run from the identity, v = 0
                    ident = true;
                    use_v = false;
                }
            }
        } else {
            const int j = z + 1;
            if (nseg <= 1 || j > nseg - 1) return;
            a0 = seg_start(j);
            a1 = min(a0 + seg, t1);
            init = wsm(id0 + j, 0);
            fin = (j == nseg - 1) ? S : nullptr;
        }
    }

    // ---- state S0^T [k][v] in accumulator layout: tile (kb, vb) lane holds
    //      S0^T[16 kb + 4 q4 + r][16 (wave VB + vb) + l16] = S[v][k..k+3]
    f32x4 st[KB][VB], st2[KB][VB];           // st2: the paired P run's state
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
            st[kb][vb] = f32x4{0, 0, 0, 0};
            st2[kb][vb] = f32x4{0, 0, 0, 0};
            if (vact) {
                const int v = 16 * (wave * VB + vb) + l16;
                if (!SEG || init) {
                    const float4 x = *reinterpret_cast<const float4*>(init + static_cast<size_t>(v) * D + 16 * kb + 4 * q4);
                    st[kb][vb] = f32x4{x.x, x.y, x.z, x.w};
                }
                if constexpr (SEG && !PAIR) {
                    if (ident) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) st[kb][vb][r] = (16 * kb + 4 * q4 + r == v) ? 1.0f : 0.0f;
                    }
                }
                if constexpr (PAIRED) {
                    if (pb) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) st2[kb][vb][r] = (16 * kb + 4 * q4 + r == v) ? 1.0f : 0.0f;
                    }
                }
            }
        }

    // Chunk loads.  Thread (tp, cg) moves token rows 2tp, 2tp+1 at columns
    // 8 (cg + CG pass); K^T / V^T receive 32-bit (t, t+1) pairs, so the 32 lanes
    // of a half-wave (one cg) store 32 consecutive words: no bank conflict, as
    // the LDS takes 32-bit stores 32 lanes a cycle over 32 banks.  The next chunk's loads are issued
    // during the current chunk's state update and staged at the loop top.
    const int tp = tid & 31;
    const int cg = tid >> 5;                     // 0..CG-1
    const int ta = 2 * tp;
    uint4 pk[CP][2][WPE], pq[CP][2][WPE], pv[CP][2][WPE];
    uint32_t pbeta = 0, pg = 0;                  // raw bits of the chunk's gate inputs
    const GateHead gh = gate_head(ga, hv);       // per-head gating constants, loaded once
    // Loads go through buffer descriptors over the chunk's rows (the entry
    // point's dims bound a chunk's span, 64 HV D elements, below 2^28 bytes),
    // so rows past the chunk's length read as zero.
    // Token rows are sqk (q, k) and sv (v) elements apart: H D and HV D for
    // separate q, k, v tensors, the conv width for slices of one activation row.
    const uint32_t off_kq = static_cast<uint32_t>(h * D) * sizeof(IT);
    const uint32_t off_v = static_cast<uint32_t>(hv * D) * sizeof(IT);
    const uint32_t row_kq = static_cast<uint32_t>(sqk) * sizeof(IT);
    const uint32_t row_v = static_cast<uint32_t>(sv) * sizeof(IT);
    // gate sources, resolved once: g, beta fp32 or a, b (bf16 or fp32)
    const bool ghalf = ga.a != nullptr && ga.ab_bf16;
    const uint32_t ges = ghalf ? 2 : 4;
    const uint32_t grow = static_cast<uint32_t>(HV) * ges;
    const char* gsrc0 = static_cast<const char*>(ga.a ? ga.a : static_cast<const void*>(ga.g));
    const char* gsrc1 = static_cast<const char*>(ga.a ? ga.b : static_cast<const void*>(ga.beta));
    auto fetch = [&](int32_t c, int Lc) {
        const rsrc_t rk_ = make_rsrc(kg + static_cast<size_t>(c) * sqk, Lc * row_kq);
        const rsrc_t rq_ = make_rsrc(qg + static_cast<size_t>(c) * sqk, Lc * row_kq);
        const rsrc_t rv_ = make_rsrc(vg + static_cast<size_t>(c) * sv, Lc * row_v);
#pragma unroll
        for (int pass = 0; pass < CP; ++pass) {
            const int k0 = 8 * (cg + CG * pass);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t t = ta + e;
                const uint32_t kk = k0 * sizeof(IT);
#pragma unroll
                for (int w = 0; w < WPE; ++w) {
                    if (8 * CG * CP == D || k0 < D) {
                        pk[pass][e][w] = buf_ld16(rk_, t * row_kq + off_kq + kk + 16 * w);
                        pq[pass][e][w] = buf_ld16(rq_, t * row_kq + off_kq + kk + 16 * w);
                        pv[pass][e][w] = buf_ld16(rv_, t * row_v + off_v + kk + 16 * w);
                    }
                }
            }
        }
        // the chunk's raw gate values (g and beta, or a and b for fused gating);
        // used by wave 0 at the loop top
        const rsrc_t r0 = make_rsrc(gsrc0 + static_cast<size_t>(c) * grow, Lc * grow);
        const rsrc_t r1 = make_rsrc(gsrc1 + static_cast<size_t>(c) * grow, Lc * grow);
        const uint32_t ob = static_cast<uint32_t>(min(tid, CH) * HV + hv) * ges;
        // raw bits only: converting here would wait for every load issued above
        if (ghalf) {
            pg = buf_ld2(r0, ob);
            pbeta = buf_ld2(r1, ob);
        } else {
            pg = __builtin_amdgcn_raw_buffer_load_b32(r0, ob, 0, 0);
            pbeta = __builtin_amdgcn_raw_buffer_load_b32(r1, ob, 0, 0);
        }
    };
    fetch(a0, min(CH, a1 - a0));

    for (int32_t c0 = a0; c0 < a1; c0 += CH) {
        const int L = min(CH, a1 - c0);
        // Segment launches: the lane coordinates re-derived each chunk from an
        // opaque copy of the thread index, so the compiler recomputes the
        // chunk's LDS addresses inside the loop instead of holding them in
        // registers across it (the registers the paired P/B runs need).
        // Whole-sequence launches keep the hoisted addresses (faster there).
        int tid_o = static_cast<int>(threadIdx.x);
        if constexpr (PAIRED) asm volatile("" : "+v"(tid_o));
        const int tid = tid_o;
        const int lane = tid & 63;
        const int q4 = lane >> 4;
        const int l16 = lane & 15;
        const int swl = kq_swz(l16);             // K/Q swizzle of the lane's fragment rows
        // M o P-hat takes the same swizzle at the 8 mod 16 word stride (its 8-byte
        // row stores: 4-way -> 2-way; reads stay conflict-free), not at 4 mod 16
        const int swm = (ST % 32 == 16) ? swl : 0;
        const int tp = tid & 31;
        const int ta = 2 * tp;

        // ---------------- stage the fetched chunk into LDS (planes hi [, lo])
#pragma unroll
        for (int pass = 0; pass < CP; ++pass) {
            const int k0 = 8 * (cg + CG * pass);
            if (k0 < D) {
                uint4 kw[2][2], qw[2][2], vw[2][2];      // [row][plane]
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    if constexpr (SPL) {
                        split8(pk[pass][e][0], pk[pass][e][WPE - 1], kw[e][0], kw[e][1]);
                        split8(pq[pass][e][0], pq[pass][e][WPE - 1], qw[e][0], qw[e][1]);
                        split8(pv[pass][e][0], pv[pass][e][WPE - 1], vw[e][0], vw[e][1]);
                    } else {
                        kw[e][0] = pk[pass][e][0]; qw[e][0] = pq[pass][e][0]; vw[e][0] = pv[pass][e][0];
                        kw[e][1] = kw[e][0]; qw[e][1] = qw[e][0]; vw[e][1] = vw[e][0];
                    }
                }
#pragma unroll
                for (int pl = 0; pl < NP; ++pl) {
                    // K and Q rows in pperm order along k (swizzled: rows ta, ta + 1
                    // share kq_swz); K^T in pperm order along t
                    const int p0 = pperm(k0), p1 = pperm(k0 + 4), swt = kq_swz(ta);
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        lds_st8(&sm.k[pl][(ta + e) * SK + (p0 ^ swt)], kw[e][pl].x, kw[e][pl].y);
                        lds_st8(&sm.k[pl][(ta + e) * SK + (p1 ^ swt)], kw[e][pl].z, kw[e][pl].w);
                        lds_st8(&sm.q[pl][(ta + e) * SK + (p0 ^ swt)], qw[e][pl].x, qw[e][pl].y);
                        lds_st8(&sm.q[pl][(ta + e) * SK + (p1 ^ swt)], qw[e][pl].z, qw[e][pl].w);
                    }
                    store_pairs_t(sm.kt[pl], ST, k0, pperm(ta), kw[0][pl], kw[1][pl]);
                    store_pairs_t(sm.vt[pl], ST, k0, ta, vw[0][pl], vw[1][pl]);
                }
            }
        }
        if (wave == 0) {                         // gate, then the cumulative log-decay:
            float gt, bv;                        // fixed-order DPP wave scan
            const bool half = ghalf;
            gate_finish(ga, gh, half ? bf16_to_f32(static_cast<bf16_t>(pg)) : __uint_as_float(pg),
                        half ? bf16_to_f32(static_cast<bf16_t>(pbeta)) : __uint_as_float(pbeta), gt, bv);
            if (lane >= L) { gt = 0.0f; bv = 0.0f; }   // rows past the chunk (raw values read as 0)
            sm.beta[lane] = bv;
            gt += dpp_scan_step<0x111, 0xF>(gt);     // row_shr:1 .. row_shr:8 inside each 16-lane row
            gt += dpp_scan_step<0x112, 0xF>(gt);
            gt += dpp_scan_step<0x114, 0xF>(gt);
            gt += dpp_scan_step<0x118, 0xF>(gt);
            gt += dpp_scan_step<0x142, 0xA>(gt);     // row_bcast:15 -> rows 1, 3
            gt += dpp_scan_step<0x143, 0xC>(gt);     // row_bcast:31 -> rows 2, 3
            sm.gam[lane] = gt;
        }
        __syncthreads();

        // ---------------- G = K K^T, P = Q K^T and the diagonal block of Q Q^T on
        // MFMA (raw x raw: hh, plus hl + lh for split inputs), computed as
        // transposed tiles (key block as the A operand) so that a lane holds one
        // row i and four consecutive columns c.  The row norms come from the
        // diagonals of K K^T and Q Q^T (sums of squares in the MFMA's fixed
        // order); after a barrier the epilogue forms A (fp32 into sm.g) and
        // M o P (hi/lo bf16 into sm.mp) straight from the accumulators.
        {
            const int tb = wave & 3;             // 16-token row block
            const int jh = wave >> 2;            // column blocks 2 jh, 2 jh + 1
            const bool diag = (tb >> 1) == jh;   // this wave also owns block (tb, tb)
            f32x4 accg[2], accp[2], accq = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 2; ++j) { accg[j] = f32x4{0, 0, 0, 0}; accp[j] = f32x4{0, 0, 0, 0}; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int pa = 0; pa < NP; ++pa) {
                    const bf16x8 ak = frag_kq(sm.k[pa], SK, 16 * tb + l16, 32 * ks, q4, swl);
                    const bf16x8 aq = frag_kq(sm.q[pa], SK, 16 * tb + l16, 32 * ks, q4, swl);
#pragma unroll
                    for (int pb = 0; pb < NP - pa; ++pb) {
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const bf16x8 bk = frag_kq(sm.k[pb], SK, 16 * (2 * jh + j) + l16, 32 * ks, q4, swl);
                            accg[j] = mfma(bk, ak, accg[j]);
                            accp[j] = mfma(bk, aq, accp[j]);
                        }
                        if (diag)
                            accq = mfma(frag_kq(sm.q[pb], SK, 16 * tb + l16, 32 * ks, q4, swl), aq, accq);
                    }
                }
            }
            // lane holds G[i][c + r], P[i][c + r] for i = 16 tb + l16, c = 16 jc + 4 q4;
            // the diagonal element (i, i) sits at r = l16 - 4 q4 of column block tb
            const int i = 16 * tb + l16;
            const int r0 = l16 - 4 * q4;
            if (diag && r0 >= 0 && r0 < 4) {
                const f32x4 gd = accg[tb & 1];
                float dk = gd[0], dq = accq[0];
#pragma unroll
                for (int r = 1; r < 4; ++r)
                    if (r == r0) { dk = gd[r]; dq = accq[r]; }
                sm.rk[i] = norm ? 1.0f / sqrtf(dk + 1e-6f) : 1.0f;
                sm.rq[i] = norm ? scale / sqrtf(dq + 1e-6f) : scale;
            }
            __syncthreads();
            // Decays e^x (x <= 0 inside the chunk, x = gamma_t for e^gamma) use the
            // hardware base-2 exponential: a few fp32 ulps, far below the bf16
            // operand rounding they feed, and a third of the instructions of
            // the correctly rounded expf in this VALU-bound epilogue.
            if (tid < CH) {                      // per-token coefficients (wave 0)
                const float gl = sm.gam[L - 1];
                const float gv = sm.gam[tid];
                const float et = __expf(gv);
                sm.eg[tid] = et * sm.rq[tid];
                sm.ck[tid] = (tid < L) ? __expf(gl - gv) * sm.rk[tid] : 0.0f;
                sm.cy[tid] = et * sm.rk[tid];
                if (tid == 0) sm.egl = __expf(gl);
            }
            const float gi = sm.gam[i];
            const float brk = sm.beta[i] * sm.rk[i];
            const float rqi = sm.rq[i];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = 16 * (2 * jh + j) + 4 * q4;
                const float4 gc = *reinterpret_cast<const float4*>(&sm.gam[c]);
                const float4 rkc = *reinterpret_cast<const float4*>(&sm.rk[c]);
                const float gcs[4] = {gc.x, gc.y, gc.z, gc.w};
                const float rks[4] = {rkc.x, rkc.y, rkc.z, rkc.w};
                f32x4 a, mp;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dec = (c + r <= i) ? __expf(gi - gcs[r]) : 0.0f;
                    a[r] = (c + r < i) ? (brk * rks[r]) * (dec * accg[j][r]) : 0.0f;
                    mp[r] = (rqi * rks[r]) * (dec * accp[j][r]);
                }
                *reinterpret_cast<float4*>(&sm.g[i * SF + c]) = make_float4(a[0], a[1], a[2], a[3]);
                uint2 h2, l2;
                split4(mp, h2, l2);
                // pperm order, swizzled like K and Q where the stride suits it
                // (row i = 16 tb + l16: the lane's swl)
                lds_st8(&sm.mp[i * ST + (pperm(c) ^ swm)], h2.x, h2.y);
                lds_st8(&sm.mp[CH * ST + i * ST + (pperm(c) ^ swm)], l2.x, l2.y);
            }
        }
        __syncthreads();

        // ---------------- state products that need only S0 and the staged
        // chunk: Z = K S0^T (so that U = cU (V - diag(cy) Z), with no W formed) and,
        // transposed, O1^T = S0 Q^T, scaled by e^gamma_t rq_t.  The state's
        // hi/lo fragments (permuted k-slots) are the B operand of the first
        // and, holding the same values, the A operand of the second.  They run
        // on the waves the block inverse below leaves idle.
        f32x4 z[4][VB];                          // Z tiles (t-block, v-block)
        f32x4 o[VB][4];                          // O^T tiles (v-block, t-block)
        auto early = [&](auto DZ, auto DO) {
            constexpr bool dz = decltype(DZ)::value, doo = decltype(DO)::value;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    if (dz) z[tb][vb] = f32x4{0, 0, 0, 0};
                    if (doo) o[vb][tb] = f32x4{0, 0, 0, 0};
                }
            if (!vact) return;
            // per k-step: every fragment load first, then the state split (VALU
            // work that covers the loads' latency), then the MFMAs; the
            // scheduling barriers keep the compiler from sinking each load
            // next to its first use
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 ak[4], akl[4], bq[4], bql[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    if (dz || (PAIRED && doo && pb)) {
                        ak[tb] = frag_kq(sm.k[0], SK, 16 * tb + l16, 32 * ks, q4, swl);
                        if constexpr (SPL) akl[tb] = frag_kq(sm.k[NP - 1], SK, 16 * tb + l16, 32 * ks, q4, swl);
                    }
                    if (doo && (!SEG || wo)) {
                        bq[tb] = frag_kq(sm.q[0], SK, 16 * tb + l16, 32 * ks, q4, swl);
                        if constexpr (SPL) bql[tb] = frag_kq(sm.q[NP - 1], SK, 16 * tb + l16, 32 * ks, q4, swl);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 sh[VB], sl[VB];
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    uint2 h0, l0, h1, l1;
                    split4(st[2 * ks][vb], h0, l0);
                    split4(st[2 * ks + 1][vb], h1, l1);
                    sh[vb] = as_bf16x8(cat(h0, h1));
                    sl[vb] = as_bf16x8(cat(l0, l1));
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (PAIRED && doo) {
                    // paired P run: its Z (from st2) accumulates in the O tiles,
                    // which a run without outputs does not use
                    if (pb) {
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            uint2 h0, l0, h1, l1;
                            split4(st2[2 * ks][vb], h0, l0);
                            split4(st2[2 * ks + 1][vb], h1, l1);
                            const bf16x8 s2h = as_bf16x8(cat(h0, h1)), s2l = as_bf16x8(cat(l0, l1));
#pragma unroll
                            for (int tb = 0; tb < 4; ++tb) {
                                o[vb][tb] = mfma(ak[tb], s2h, o[vb][tb]);
                                o[vb][tb] = mfma(ak[tb], s2l, o[vb][tb]);
                                if constexpr (SPL) o[vb][tb] = mfma(akl[tb], s2h, o[vb][tb]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    if constexpr (dz) {
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            z[tb][vb] = mfma(ak[tb], sh[vb], z[tb][vb]);
                            z[tb][vb] = mfma(ak[tb], sl[vb], z[tb][vb]);
                        }
                        if constexpr (SPL) {
#pragma unroll
                            for (int vb = 0; vb < VB; ++vb) z[tb][vb] = mfma(akl[tb], sh[vb], z[tb][vb]);
                        }
                    }
                    if (doo && (!SEG || wo)) {
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            o[vb][tb] = mfma(sh[vb], bq[tb], o[vb][tb]);
                            o[vb][tb] = mfma(sl[vb], bq[tb], o[vb][tb]);
                        }
                        if constexpr (SPL) {
#pragma unroll
                            for (int vb = 0; vb < VB; ++vb) o[vb][tb] = mfma(sh[vb], bql[tb], o[vb][tb]);
                        }
                    }
                }
            }
            if (doo && (!SEG || wo)) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const float e = sm.eg[16 * tb + l16];
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        o[vb][tb][0] *= e; o[vb][tb][1] *= e; o[vb][tb][2] *= e; o[vb][tb][3] *= e;
                    }
                }
            }
        };
        using T_ = std::true_type;
        using F_ = std::false_type;

        // ---------------- T = (I + A)^-1.  Diagonal 16x16 blocks by forward
        // substitution (wave WF: lane = 16 block + column c).  Lane c holds column
        // c of each row of the block; row r's entry A[r][j] reaches every lane of
        // the block by a DPP row broadcast from lane j.  Right-looking order: once
        // T[j][c] is final, every later row r adds A[r][j] T[j][c], so each row
        // still accumulates its terms in ascending j.  The upper triangle of
        // sm.g is zero from the epilogue above and stays zero.  The other waves
        // run `early` meanwhile; WF runs its Z part during the 16 -> 32 merge and
        // its O1 part during the 32 -> 64 merge.
        // With ns_rounds > 0 the blocks are instead inverted by Newton-Schulz with
        // bf16 intermediates (an A/B variant reproducing vLLM PR #53864,
        // "Numerical root cause and fix"): waves 0-3, one block each, and then
        // every wave runs `early`.
        constexpr int WF = NW - 1;               // forward-substitution wave
        constexpr int WM = NW - 3;               // merge waves WM, WM + 1
        if constexpr (NSV) {
            if (wave < 4) ns_block_inverse(&sm.g[(16 * wave) * SF + 16 * wave], SF,
                                           reinterpret_cast<bf16_t*>(sm.xs) + 512 * wave, ns_rounds,
                                           l16, q4);
            __syncthreads();
            early(T_{}, T_{});
        } else if (wave == WF) {
            const int b = lane >> 4;
            fwd_subst16(&sm.g[(16 * b) * SF + 16 * b], SF, lane & 15);
        } else {
            early(T_{}, T_{});
        }
        __syncthreads();
        // merge 16 -> 32 for block pairs p = (0,1), (2,3) on fp32 MFMA (wave WM + p):
        // X = A21 T11 goes through the LDS scratch and straight back into the same
        // wave (LDS is in order within a wave; the fence keeps the compiler from
        // reordering), then T21 = -T22 X.  Operands are loaded before the MFMAs.
        if (wave == WM || wave == WM + 1) {
            const int pw = wave - WM;
            const int b0 = 32 * pw, b1 = b0 + 16;
            float a[4], bb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                a[kk] = sm.g[(b1 + l16) * SF + b0 + 4 * kk + q4];
                bb[kk] = sm.g[(b0 + 4 * kk + q4) * SF + b0 + l16];
            }
            f32x4 x = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) x = mfma4(a[kk], bb[kk], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.xs[(16 * pw + 4 * q4 + r) * 36 + l16] = x[r];
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                a[kk] = sm.g[(b1 + l16) * SF + b1 + 4 * kk + q4];
                bb[kk] = sm.xs[(16 * pw + 4 * kk + q4) * 36 + l16];
            }
            f32x4 t = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) t = mfma4(a[kk], bb[kk], t);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.g[(b1 + 4 * q4 + r) * SF + b0 + l16] = -t[r];
        } else if (!NSV && wave == WF) {
            early(T_{}, F_{});
        }
        __syncthreads();
        // merge 32 -> 64 (wave WM + tj, tj < 2: output column block tj of the
        // lower-left 32x32 block, both row blocks ti): X[:, tj] = A[32:64][0:32]
        // T11[:, tj], then T21[:, tj] = -T22 X[:, tj], the same wave-local LDS
        // round trip; T21 is left in xs.  T11's block (0, 1) and T22's block
        // (0, 1) are zero: skipped.
        if (wave == WM || wave == WM + 1) {
            const int tj = wave - WM;
            const int k0 = 4 * tj;                 // T11[:, tj] is zero above row 16 tj
            float a[2][8], bb[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (kk < k0) continue;
                bb[kk] = sm.g[(4 * kk + q4) * SF + 16 * tj + l16];
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) a[ti][kk] = sm.g[(32 + 16 * ti + l16) * SF + 4 * kk + q4];
            }
            f32x4 x[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (kk < k0) continue;
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) x[ti] = mfma4(a[ti][kk], bb[kk], x[ti]);
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.xs[(16 * ti + 4 * q4 + r) * 36 + 16 * tj + l16] = x[ti][r];
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                bb[kk] = sm.xs[(4 * kk + q4) * 36 + 16 * tj + l16];
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) a[ti][kk] = sm.g[(32 + 16 * ti + l16) * SF + 32 + 4 * kk + q4];
            }
            f32x4 t[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                t[1] = mfma4(a[1][kk], bb[kk], t[1]);
                if (kk < 4) t[0] = mfma4(a[0][kk], bb[kk], t[0]);   // T22 row block 0 is zero past col 16
            }
            // T21[:, tj] replaces this wave's own column of X (its reads of X are
            // done); sm.g's block [32:64][0:32] still holds A21, which the other
            // wave may be reading
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.xs[(16 * ti + 4 * q4 + r) * 36 + 16 * tj + l16] = -t[ti][r];
        } else if (!NSV && wave == WF) {
            early(F_{}, T_{});
        }
        __syncthreads();

        // ---------------- coefficients cU = T diag(beta), split into hi/lo and
        // stored in pperm order along t' (it meets Y in permuted t-slots)
        // (thread: row r, 8 columns; T's upper triangle is exactly zero)
        {
            const int r = tid >> 3, cb = 8 * (tid & 7);
            uint32_t uh[4], ul[4];
            const float* trow = (r >= 32 && cb < 32) ? &sm.xs[(r - 32) * 36 + cb] : &sm.g[r * SF + cb];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float4 t = *reinterpret_cast<const float4*>(trow + 4 * j);
                const float4 bt = *reinterpret_cast<const float4*>(&sm.beta[cb + 4 * j]);
                const f32x4 u = {t.x * bt.x, t.y * bt.y, t.z * bt.z, t.w * bt.w};
                uint2 h2, l2;
                split4(u, h2, l2); uh[2 * j] = h2.x; uh[2 * j + 1] = h2.y; ul[2 * j] = l2.x; ul[2 * j + 1] = l2.y;
            }
            bf16_t* ubase = sm.pc.c + r * ST;
            lds_st8(ubase + 0 * CH * ST + pperm(cb), uh[0], uh[1]);
            lds_st8(ubase + 0 * CH * ST + pperm(cb + 4), uh[2], uh[3]);
            lds_st8(ubase + 1 * CH * ST + pperm(cb), ul[0], ul[1]);
            lds_st8(ubase + 1 * CH * ST + pperm(cb + 4), ul[2], ul[3]);
        }
        __syncthreads();

        // ---------------- U = cU Y with Y = V - diag(cy) Z, cy = e^gamma rk: the
        // same U as Ut - W S0^T (W = cU diag(cy) K, so W S0^T = cU diag(cy) Z),
        // with one coefficient matrix.  Y is formed in fp32 from the Z
        // accumulators and V (read from V^T, four consecutive tokens of one
        // value column per lane: the accumulator layout), split into hi/lo and
        // fed as permuted t-slots; cU (split) is lower triangular, so blocks
        // above the diagonal are skipped (hh + hl + lh).
        f32x4 u[4][VB];                          // U tiles (t-block, v-block): rows t, cols v
        f32x4 u2[4][VB];                         // the paired P run's U (= cU Y2, Y2 = -diag(cy) Z2)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) { u[tb][vb] = f32x4{0, 0, 0, 0}; u2[tb][vb] = f32x4{0, 0, 0, 0}; }
        if (vact) {
            bf16x8 yh[2][VB], yl[2][VB];
            auto make_y = [&](const f32x4 (&zz)[4][VB], bool with_v) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        const int vr = 16 * (wave * VB + vb) + l16;
                        f32x4 n[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int tb = 2 * ks + e;
                            const int t0 = 16 * tb + 4 * q4;
                            const float4 cyv = *reinterpret_cast<const float4*>(&sm.cy[t0]);
                            float vv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                            if (with_v) {
#pragma unroll
                                for (int pl = 0; pl < NP; ++pl) {
                                    const uint2 w = *reinterpret_cast<const uint2*>(&sm.vt[pl][vr * ST + t0]);
                                    vv[0] += bf16lo_to_f32(w.x); vv[1] += bf16hi_to_f32(w.x);
                                    vv[2] += bf16lo_to_f32(w.y); vv[3] += bf16hi_to_f32(w.y);
                                }
                            }
                            n[e][0] = vv[0] - cyv.x * zz[tb][vb][0];
                            n[e][1] = vv[1] - cyv.y * zz[tb][vb][1];
                            n[e][2] = vv[2] - cyv.z * zz[tb][vb][2];
                            n[e][3] = vv[3] - cyv.w * zz[tb][vb][3];
                        }
                        uint2 h0, l0, h1, l1;
                        split4(n[0], h0, l0);
                        split4(n[1], h1, l1);
                        yh[ks][vb] = as_bf16x8(cat(h0, h1));
                        yl[ks][vb] = as_bf16x8(cat(l0, l1));
                    }
            };
            auto mul_cu = [&](f32x4 (&acc)[4][VB]) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (32 * ks > 16 * tb + 15) continue;          // strictly above the diagonal
                        const bf16x8 ch = frag_perm(sm.pc.c + 0 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
                        const bf16x8 cl = frag_perm(sm.pc.c + 1 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            acc[tb][vb] = mfma(ch, yh[ks][vb], acc[tb][vb]);
                            acc[tb][vb] = mfma(ch, yl[ks][vb], acc[tb][vb]);
                            acc[tb][vb] = mfma(cl, yh[ks][vb], acc[tb][vb]);
                        }
                    }
            };
            make_y(z, use_v);
            mul_cu(u);
            if constexpr (PAIRED) {
                if (pb) {                        // U2 = cU Y2, Z2 held in the O tiles
                    f32x4 z2[4][VB];
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) z2[tb][vb] = o[vb][tb];
                    make_y(z2, false);
                    mul_cu(u2);
                }
            }
        }

        if (vact && (!SEG || wo)) {
            // ------------ O^T += U^T (M o P)^T  (U split: A operand, permuted t-slots)
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
                    const bf16x8 mh = frag_kq(sm.mp, ST, 16 * tb + l16, 32 * ks, q4, swm);
                    const bf16x8 ml = frag_kq(sm.mp + CH * ST, ST, 16 * tb + l16, 32 * ks, q4, swm);
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        o[vb][tb] = mfma(uh[ks][vb], mh, o[vb][tb]);
                        o[vb][tb] = mfma(ul[ks][vb], mh, o[vb][tb]);
                        o[vb][tb] = mfma(uh[ks][vb], ml, o[vb][tb]);
                    }
                }
            // store O: lane holds O[t = 16 tb + l16][v = 16 (wave VB + vb) + 4 q4 .. + 3];
            // rows t >= L fall outside the descriptor's range and are dropped
            const uint32_t row_o = static_cast<uint32_t>(HV * D) * sizeof(OT);
            const rsrc_t ro = make_rsrc(out + static_cast<size_t>(c0) * HV * D, L * row_o);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    const uint32_t off = static_cast<uint32_t>(16 * tb + l16) * row_o +
                        static_cast<uint32_t>(hv * D + 16 * (wave * VB + vb) + 4 * q4) * sizeof(OT);
                    if constexpr (sizeof(OT) == 4) {
                        buf_st16(ro, off, __float_as_uint(o[vb][tb][0]), __float_as_uint(o[vb][tb][1]),
                                 __float_as_uint(o[vb][tb][2]), __float_as_uint(o[vb][tb][3]));
                    } else {
                        buf_st8(ro, off, pack_bf16x2(o[vb][tb][0], o[vb][tb][1]),
                                pack_bf16x2(o[vb][tb][2], o[vb][tb][3]));
                    }
                }
            }
        }

        if (vact) {
            // ------------ S0^T <- e^{gamma_L} S0^T + K^T (cK . U)
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
            bf16x8 c2h[2][VB], c2l[2][VB];       // the paired P run's cK . U2
            if constexpr (PAIRED) {
                if (pb) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            f32x4 a = u2[2 * ks][vb], b = u2[2 * ks + 1][vb];
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                a[r] *= sm.ck[32 * ks + 4 * q4 + r];
                                b[r] *= sm.ck[32 * ks + 16 + 4 * q4 + r];
                            }
                            uint2 h0, l0, h1, l1;
                            split4(a, h0, l0);
                            split4(b, h1, l1);
                            c2h[ks][vb] = as_bf16x8(cat(h0, h1));
                            c2l[ks][vb] = as_bf16x8(cat(l0, l1));
                        }
                }
            }
            if (c0 + CH < a1) fetch(c0 + CH, min(CH, a1 - c0 - CH));   // next chunk, in flight
            const float egl = sm.egl;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                bf16x8 ak[2], akl[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    ak[ks] = frag_perm(sm.kt[0], ST, 16 * kb + l16, 32 * ks, q4);
                    akl[ks] = frag_perm(sm.kt[NP - 1], ST, 16 * kb + l16, 32 * ks, q4);
                }
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    f32x4 acc = st[kb][vb];
                    acc[0] *= egl; acc[1] *= egl; acc[2] *= egl; acc[3] *= egl;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        acc = mfma(ak[ks], ch[ks][vb], acc);
                        acc = mfma(ak[ks], cl[ks][vb], acc);
                        if constexpr (SPL) acc = mfma(akl[ks], ch[ks][vb], acc);
                    }
                    st[kb][vb] = acc;
                    if constexpr (PAIRED) {
                        if (pb) {
                            f32x4 acc2 = st2[kb][vb];
                            acc2[0] *= egl; acc2[1] *= egl; acc2[2] *= egl; acc2[3] *= egl;
#pragma unroll
                            for (int ks = 0; ks < 2; ++ks) {
                                acc2 = mfma(ak[ks], c2h[ks][vb], acc2);
                                acc2 = mfma(ak[ks], c2l[ks][vb], acc2);
                                if constexpr (SPL) acc2 = mfma(akl[ks], c2h[ks][vb], acc2);
                            }
                            st2[kb][vb] = acc2;
                        }
                    }
                }
            }
        }
        if (!vact && c0 + CH < a1) fetch(c0 + CH, min(CH, a1 - c0 - CH));
        __syncthreads();                         // LDS is rewritten by the next chunk
    }

    // ---- the paired P run's end state, then the final state back to the slot
    //      (or to the segment workspace)
    if constexpr (PAIRED) {
        if (vact && pb) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    const int v = 16 * (wave * VB + vb) + l16;
                    *reinterpret_cast<float4*>(fin2 + static_cast<size_t>(v) * D + 16 * kb + 4 * q4) =
                        make_float4(st2[kb][vb][0], st2[kb][vb][1], st2[kb][vb][2], st2[kb][vb][3]);
                }
        }
    }
    if (vact && (!SEG || fin)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
                const int v = 16 * (wave * VB + vb) + l16;
                *reinterpret_cast<float4*>(fin + static_cast<size_t>(v) * D + 16 * kb + 4 * q4) =
                    make_float4(st[kb][vb][0], st[kb][vb][1], st[kb][vb][2], st[kb][vb][3]);
            }
    }
}

// ---------------------------------------------------------------------------
// Pipelined chunk step (d = 128, bf16 inputs; whole runs and unpaired segment
// runs).  The arithmetic of prefill_kernel term for term and in the same order
// (so the two kernels agree bit for bit), with the eight waves split by role,
// so that the state-independent work of one chunk runs beside the state
// products of another:
//   state waves 0-3 (one per SIMD) own 32 value columns each of S0^T and do
//     Z = K S0^T, O1^T = S0 Q^T, Y, U = cU Y, O and the state update of chunk c;
//   coefficient waves 4-7 invert chunk c's (I + A) (forward substitution on
//     wave 7, merges on waves 5 and 6), form its cU, and then build chunk
//     c + 1's gate scan, G = K K^T, P = Q K^T, norms, A and M o P-hat while the
//     state waves finish chunk c.
// One chunk step is six barrier-separated sub-steps.  The two roles run as
// two loops over the same chunks with the same six barriers per chunk, so
// every barrier is met by all eight waves:
//   A1  state: Z                        coef: forward substitution (wave 7);
//                                             eg/ck/cy(c) (wave 4); loads of chunk
//                                             c+1 (waves 4-6); M o P-hat(c) rows (5, 6)
//   A2  state: O1, scaled (its MFMAs    coef: stage K^T(c); loads (wave 7);
//       overlap Y's vector work);             merge 16 -> 32 (waves 5, 6)
//       Y = V - cy Z
//   A3  state: cU(c) of the diagonal    coef: merge 32 -> 64 and the cU(c) of
//       32x32 blocks                          that block (waves 5, 6);
//                                             M o P-hat(c) rows (waves 4, 7)
//   B1  state: U = cU Y                 coef: stage K, Q, V(c+1); gate scan(c+1)
//   B2  state: O (stored)               coef: G, P, norms(c+1)
//   B3  state: cK . U, the state update coef: A(c+1), and the masked decays
//                                             its M o P-hat reuses
// (O1 sits beside Y rather than beside the 32 -> 64 merge: the two waves of a
// SIMD then do not both issue MFMAs in the same sub-step.)
// Each coefficient wave keeps its G and P tiles of chunk c+1 and the decays in
// registers from B2/B3 to the next chunk's M o P-hat step, so that work lands
// where the wave has slack.  The waves on the critical path of their sub-step
// (substitution, merges) raise their issue priority over the state wave
// sharing their SIMD.  The chunk loads go out on waves with little else to do
// in that sub-step.
// LDS ownership follows from that order: K and Q (c) are read in A1-A2 and
// replaced in B1; V(c) is read in A2 and replaced in B1; K^T(c) is read in
// B3 and replaced in A2; A / T live in g (and the merge scratch xs) from B3 to
// A3; cU is written in A3 and read in B1; M o P-hat is written in A1 and A3
// and read in B2.  The per-token coefficients the state waves use
// (e^gamma r_q, c_K, e^gamma r_k, e^gamma_L) are double-buffered by chunk
// parity.
struct alignas(16) PipeSmem {
    static constexpr int D = 128;
    static constexpr int SK = D + PADK;         // row stride of K, Q (bf16)
    static constexpr int ST = CH + PADT;        // row stride of K^T, cU, M o P-hat
    // row stride of V (bf16): 16-byte rows for its staging stores, and rows
    // four apart 16 banks apart, so that the value-column reads (16 columns x
    // rows t, t + 4, t + 8, t + 12 per instruction) are conflict-free
    static constexpr int SV = D + 8;
    static constexpr int SF = CH + PADF;        // row stride of the fp32 64x64 array
    bf16_t k[CH * SK];                          // K   [t][k]
    bf16_t q[CH * SK];                          // Q   [t][k]
    bf16_t kt[D * ST];                          // K^T [k][t]
    bf16_t v[CH * SV];                          // V   [t][v]
    float g[CH * SF];                           // A, then T in place (block [32:64][0:32] in xs)
    bf16_t cu[2 * CH * ST];                     // cU hi, lo [t][t'], pperm order along t'
    float xs[32 * 36];                          // merge scratch X; finally T[32:64][0:32]
    bf16_t mp[2 * CH * ST];                     // (M o P) hi, lo [t][t']
    float gam[CH], beta[CH], rk[CH], rq[CH];
    float eg[2][CH], ck[2][CH], cy[2][CH];
    float egl[2];
    // bf16 output tile of the chunk [t][v] (row stride SO): written by the state
    // waves in B2 from their accumulators, stored as whole 256-byte rows in B3
    static constexpr int SO = D + 8;
    bf16_t ob[CH * SO];
};

template <typename OT, bool SEG>
__global__ __launch_bounds__(PF_NT) void prefill_pipe_kernel(
    const bf16_t* __restrict__ qg, const bf16_t* __restrict__ kg, const bf16_t* __restrict__ vg,
    const GateArgs ga, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slot, float* __restrict__ rec, OT* __restrict__ out, int32_t H,
    int32_t HV, int32_t sqk, int32_t sv, float scale, int32_t flags,
    const SegArgs sg, const int32_t* __restrict__ err_flag) {
    constexpr int D = 128;
    constexpr int KB = D / 16;                   // 16-row key blocks of the state
    constexpr int KS = D / 32;                   // 32-wide k-steps over the head dim
    constexpr int VB = 2;                        // 16-wide value blocks per state wave
    constexpr int SK = PipeSmem::SK, ST = PipeSmem::ST, SF = PipeSmem::SF;
    constexpr int WF = 7;                        // forward-substitution wave
    constexpr int WM = 5;                        // merge waves WM, WM + 1
    constexpr int GW = 4;                        // gate-scan wave
    __shared__ PipeSmem sm;

    if (call_rejected(err_flag)) return;
    int hv = blockIdx.x;
    {
        const int G = HV / H;
        if (HV % 8 == 0 && H % 8 == 0) {
            const int a = hv >> 3, b = hv & 7;
            hv = G * (8 * (a / G) + b) + a % G;
        }
    }
    int n = blockIdx.y;
    int zseg = blockIdx.z;
    if constexpr (SEG) {
        int gy = blockIdx.y;
        if (sg.pass == 1 && gy < sg.n_seqs) {
            zseg = 0;
        } else {
            const int base = sg.pass == 1 ? 1 : 0;
            if (sg.pass == 1) gy -= sg.n_seqs;
            if (gy >= sg.map[sg.n_seqs]) return;
            int lo = 0, hi = sg.n_seqs;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (sg.map[mid] <= gy) lo = mid; else hi = mid;
            }
            n = lo;
            zseg = base + gy - sg.map[lo];
        }
    }
    const int h = hv / (HV / H);
    const int tid = threadIdx.x;
    // the wave index read from the first lane: the role branches below are
    // then scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool state_w = wave < 4;
    // Lane coordinates, re-derived at every chunk from an opaque copy of the
    // thread index, so that the compiler recomputes the chunk's LDS addresses
    // inside the loop instead of holding them in registers across it.
    int lane, q4, l16, tp, cg, ta, swl, swm;
    auto set_lane = [&]() {
        int t = static_cast<int>(threadIdx.x);
        asm volatile("" : "+v"(t));
        lane = t & 63;
        q4 = lane >> 4;
        l16 = lane & 15;
        tp = t & 31;
        cg = (t >> 5) & 7;                       // staging: 8 column groups, two passes
        ta = 2 * tp;
        swl = kq_swz(l16);
        swm = (PipeSmem::ST % 32 == 16) ? swl : 0;
    };
    set_lane();
    const int32_t t0 = cu[n];
    const int32_t t1 = cu[n + 1];
    const int32_t s = slot[n];
    const bool norm = (flags & GDN_FLAG_QK_L2NORM) != 0;

    if (s <= 0) {                                // inactive: zero outputs, state untouched
        if (SEG && (sg.pass == 2 || zseg != 0)) return;
        for (int64_t i = tid; i < static_cast<int64_t>(t1 - t0) * D; i += PF_NT) {
            const int64_t t = t0 + i / D;
            elem<OT>::st(out + (t * HV + hv) * D + i % D, 0.0f);
        }
        return;
    }
    if (t1 <= t0) return;                        // empty sequence: state untouched

    float* S = rec + (static_cast<size_t>(s) * HV + hv) * static_cast<size_t>(D) * D;
    // the token range, start state (nullptr: zero), outputs, end state: as in
    // prefill_kernel's unpaired segment runs
    int32_t a0 = t0, a1 = t1;
    const float* init = S;
    float* fin = S;
    bool wo = true, ident = false, use_v = true;
    if constexpr (SEG) {
        const int32_t seg = sg.seg_len;
        const int32_t nseg = seg_count(t1 - t0, sg.head, seg);
        const int64_t id0 = n + t0 / seg;
        auto seg_start = [&](int j) { return j == 0 ? t0 : t0 + sg.head + (j - 1) * seg; };
        auto wsm = [&](int64_t id, int kind) {
            return sg.ws + ((id * 3 + kind) * HV + hv) * static_cast<size_t>(D) * D;
        };
        const int z = zseg;
        if (sg.pass == 1) {
            if (nseg <= 1) {
                if (z != 0) return;
            } else if (z == 0) {
                a1 = t0 + sg.head;
                fin = wsm(id0 + 1, 0);
            } else {
                const int jj = (z + 1) / 2;      // z = 2 jj - 1: B run, z = 2 jj: P run
                if (jj > nseg - 2) return;
                a0 = seg_start(jj);
                a1 = a0 + seg;
                wo = false;
                init = nullptr;
                if (z & 1) {
                    fin = wsm(id0 + jj, 2);
                } else {
                    fin = wsm(id0 + jj, 1);
                    ident = true;
                    use_v = false;
                }
            }
        } else {
            const int j = z + 1;
            if (nseg <= 1 || j > nseg - 1) return;
            a0 = seg_start(j);
            a1 = min(a0 + seg, t1);
            init = wsm(id0 + j, 0);
            fin = (j == nseg - 1) ? S : nullptr;
        }
    }

    // ---- state S0^T [k][v] (state waves): tile (kb, vb) lane holds
    //      S0^T[16 kb + 4 q4 + r][32 wave + 16 vb + l16]
    f32x4 st[KB][VB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
            st[kb][vb] = f32x4{0, 0, 0, 0};
            if (state_w) {
                const int v = 16 * (wave * VB + vb) + l16;
                if (!SEG || init) {
                    const float4 x = *reinterpret_cast<const float4*>(init + static_cast<size_t>(v) * D + 16 * kb + 4 * q4);
                    st[kb][vb] = f32x4{x.x, x.y, x.z, x.w};
                }
                if constexpr (SEG) {
                    if (ident) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) st[kb][vb][r] = (16 * kb + 4 * q4 + r == v) ? 1.0f : 0.0f;
                    }
                }
            }
        }

    // Chunk loads (coefficient waves), through buffer descriptors over the
    // chunk's rows (rows past its length read as zero), issued one or two
    // sub-steps before they are staged; the state waves hold no chunk
    // registers.  Load i of coefficient wave cw reads rows 16 cw + 4 i .. + 3
    // of K, Q and V, 16 bytes per lane, so that every load covers four whole
    // 256-byte rows (eight cache lines, each read once); all three are staged
    // row-major.  (A token-pair mapping, thread (tp, cg) on rows 2tp, 2tp+1 at
    // columns 8 (cg + 8 pass), touched 32 rows for 32 bytes each per load, and
    // issuing the loads stalled the coefficient waves for much of their
    // sub-step.)
    uint4 pk2[4], pq[4], pv[4];                  // K, Q, V of chunk c + 1 [load]
    uint32_t pbeta = 0, pg = 0;
    const GateHead gh = gate_head(ga, hv);
    const uint32_t off_kq = static_cast<uint32_t>(h * D) * sizeof(bf16_t);
    const uint32_t off_v = static_cast<uint32_t>(hv * D) * sizeof(bf16_t);
    const uint32_t row_kq = static_cast<uint32_t>(sqk) * sizeof(bf16_t);
    const uint32_t row_v = static_cast<uint32_t>(sv) * sizeof(bf16_t);
    const bool ghalf = ga.a != nullptr && ga.ab_bf16;
    const uint32_t ges = ghalf ? 2 : 4;
    const uint32_t grow = static_cast<uint32_t>(HV) * ges;
    const char* gsrc0 = static_cast<const char*>(ga.a ? ga.a : static_cast<const void*>(ga.g));
    const char* gsrc1 = static_cast<const char*>(ga.a ? ga.b : static_cast<const void*>(ga.beta));
    auto fetch = [&](int32_t c, int Lc) {
        const rsrc_t rk_ = make_rsrc(kg + static_cast<size_t>(c) * sqk, Lc * row_kq);
        const rsrc_t rq_ = make_rsrc(qg + static_cast<size_t>(c) * sqk, Lc * row_kq);
        // (runs that take no values, the segment transition runs, get an empty
        // range: V reads as zero)
        const rsrc_t rv_ = make_rsrc(vg + static_cast<size_t>(c) * sv, use_v ? Lc * row_v : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t tr = static_cast<uint32_t>(16 * (wave & 3) + 4 * i + (lane >> 4));
            const uint32_t kc = off_kq + static_cast<uint32_t>(16 * (lane & 15));
            pk2[i] = buf_ld16(rk_, tr * row_kq + kc);
            pq[i] = buf_ld16(rq_, tr * row_kq + kc);
            pv[i] = buf_ld16(rv_, tr * row_v + off_v + static_cast<uint32_t>(16 * (lane & 15)));
        }
        if (wave == GW) {                        // the gate-scan wave: token = lane
            const rsrc_t r0 = make_rsrc(gsrc0 + static_cast<size_t>(c) * grow, Lc * grow);
            const rsrc_t r1 = make_rsrc(gsrc1 + static_cast<size_t>(c) * grow, Lc * grow);
            const uint32_t ob = static_cast<uint32_t>(lane * HV + hv) * ges;
            if (ghalf) {
                pg = buf_ld2(r0, ob);
                pbeta = buf_ld2(r1, ob);
            } else {
                pg = __builtin_amdgcn_raw_buffer_load_b32(r0, ob, 0, 0);
                pbeta = __builtin_amdgcn_raw_buffer_load_b32(r1, ob, 0, 0);
            }
        }
    };
    // K, Q rows (pperm order along k, swizzled) and V rows from the fetched registers
    auto stage_kqv = [&]() {
        const int k0 = 8 * (lane & 15);
        const int p0 = pperm(k0), p1 = pperm(k0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * (wave & 3) + 4 * i + (lane >> 4);
            const int swt = kq_swz(row);
            lds_st8(&sm.k[row * SK + (p0 ^ swt)], pk2[i].x, pk2[i].y);
            lds_st8(&sm.k[row * SK + (p1 ^ swt)], pk2[i].z, pk2[i].w);
            lds_st8(&sm.q[row * SK + (p0 ^ swt)], pq[i].x, pq[i].y);
            lds_st8(&sm.q[row * SK + (p1 ^ swt)], pq[i].z, pq[i].w);
            *reinterpret_cast<uint4*>(&sm.v[row * PipeSmem::SV + 8 * (lane & 15)]) = pv[i];
        }
    };
    // K^T(c) from the K(c) rows in LDS: thread (tp, cg) reads rows 2tp, 2tp+1
    // at columns 8 (cg + 8 pass) and stores their 32-bit token pairs
    auto stage_kt = [&]() {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int k0 = 8 * (cg + 8 * pass);
            const int swt = kq_swz(ta);
            uint4 kw[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(&sm.k[(ta + e) * SK + (pperm(k0) ^ swt)]);
                const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(&sm.k[(ta + e) * SK + (pperm(k0 + 4) ^ swt)]);
                kw[e] = uint4{lo[0], lo[1], hi[0], hi[1]};
            }
            store_pairs_t(sm.kt, ST, k0, pperm(ta), kw[0], kw[1]);
        }
    };
    // cU = T diag(beta), hi/lo, pperm order along t', for the blocks of T in
    // g: rows 0-31 x columns 0-31 and rows 32-63 x columns 32-63 (state thread
    // t < 256: row r, eight columns from cb).  The block rows 32-63 x columns
    // 0-31 comes from the 32 -> 64 merge's registers, and rows 0-31 x columns
    // 32-63 (zero) is never read.
    auto cu_part = [&](int t) {
        const int r = (t < 128) ? (t >> 2) : 32 + ((t - 128) >> 2);
        const int cb = (t < 128) ? 8 * (t & 3) : 32 + 8 * (t & 3);
        uint32_t uh[4], ul[4];
        const float* trow = &sm.g[r * SF + cb];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float4 tv = *reinterpret_cast<const float4*>(trow + 4 * j);
            const float4 bt = *reinterpret_cast<const float4*>(&sm.beta[cb + 4 * j]);
            const f32x4 u = {tv.x * bt.x, tv.y * bt.y, tv.z * bt.z, tv.w * bt.w};
            uint2 h2, l2;
            split4(u, h2, l2);
            uh[2 * j] = h2.x; uh[2 * j + 1] = h2.y; ul[2 * j] = l2.x; ul[2 * j + 1] = l2.y;
        }
        bf16_t* ubase = sm.cu + r * ST;
        lds_st8(ubase + 0 * CH * ST + pperm(cb), uh[0], uh[1]);
        lds_st8(ubase + 0 * CH * ST + pperm(cb + 4), uh[2], uh[3]);
        lds_st8(ubase + 1 * CH * ST + pperm(cb), ul[0], ul[1]);
        lds_st8(ubase + 1 * CH * ST + pperm(cb + 4), ul[2], ul[3]);
    };
    // gate, then the cumulative log-decay: fixed-order DPP wave scan (wave GW)
    auto gate_scan = [&](int L) {
        float gt, bv;
        gate_finish(ga, gh, ghalf ? bf16_to_f32(static_cast<bf16_t>(pg)) : __uint_as_float(pg),
                    ghalf ? bf16_to_f32(static_cast<bf16_t>(pbeta)) : __uint_as_float(pbeta), gt, bv);
        if (lane >= L) { gt = 0.0f; bv = 0.0f; }
        sm.beta[lane] = bv;
        gt += dpp_scan_step<0x111, 0xF>(gt);
        gt += dpp_scan_step<0x112, 0xF>(gt);
        gt += dpp_scan_step<0x114, 0xF>(gt);
        gt += dpp_scan_step<0x118, 0xF>(gt);
        gt += dpp_scan_step<0x142, 0xA>(gt);
        gt += dpp_scan_step<0x143, 0xC>(gt);
        sm.gam[lane] = gt;
    };
    // coefficient waves: G = K K^T and P = Q K^T tiles of row block tb = wave - 4
    // (key block as the A operand, so a lane holds row i and four consecutive
    // columns), and the diagonal block of Q Q^T; the norms from the diagonals
    const int tb_c = wave & 3;
    f32x4 accg[4], accp[4], accq;
    float dmp[4][4];                             // masked decays of the row block, epi_a -> epi_mp
    auto gram = [&]() {
        accq = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) { accg[j] = f32x4{0, 0, 0, 0}; accp[j] = f32x4{0, 0, 0, 0}; }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ak = frag_kq(sm.k, SK, 16 * tb_c + l16, 32 * ks, q4, swl);
            const bf16x8 aq = frag_kq(sm.q, SK, 16 * tb_c + l16, 32 * ks, q4, swl);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 bk = frag_kq(sm.k, SK, 16 * j + l16, 32 * ks, q4, swl);
                accg[j] = mfma(bk, ak, accg[j]);
                accp[j] = mfma(bk, aq, accp[j]);
            }
            accq = mfma(frag_kq(sm.q, SK, 16 * tb_c + l16, 32 * ks, q4, swl), aq, accq);
        }
        const int i = 16 * tb_c + l16;
        const int r0 = l16 - 4 * q4;
        if (r0 >= 0 && r0 < 4) {
            const f32x4 gd = accg[tb_c];
            float dk = gd[0], dq = accq[0];
#pragma unroll
            for (int r = 1; r < 4; ++r)
                if (r == r0) { dk = gd[r]; dq = accq[r]; }
            sm.rk[i] = norm ? 1.0f / sqrtf(dk + 1e-6f) : 1.0f;
            sm.rq[i] = norm ? scale / sqrtf(dq + 1e-6f) : scale;
        }
    };
    // the chunk's per-token coefficients (one wave, token = lane; parity pc);
    // decays use the hardware base-2 exponential, as in prefill_kernel
    auto coefs = [&](int L, int pc) {
        const float gl = sm.gam[L - 1];
        const float gv = sm.gam[lane];
        const float rql = sm.rq[lane], rkl = sm.rk[lane];
        asm volatile("" :: "v"(rkl));            // (no read inside the masked select)
        const float et = __expf(gv);
        const float ck = __expf(gl - gv) * rkl;
        sm.eg[pc][lane] = et * rql;
        sm.ck[pc][lane] = (lane < L) ? ck : 0.0f;
        sm.cy[pc][lane] = et * rkl;
        if (lane == 0) sm.egl[pc] = __expf(gl);
    };
    // A (fp32 into g) and, separately, M o P-hat (hi/lo into mp) from this
    // wave's G and P tiles: row i = 16 tb + l16, columns c .. c + 3
    // epi_a reads every operand from LDS first and evaluates the decay
    // exponentials unconditionally (a masked one may overflow; the select drops
    // it), so the reads overlap and no lane mask splits the code; for A the
    // decay's own mask (c <= i) is implied by A's (c < i).  It keeps the masked
    // decays of its row block in registers for that block's M o P-hat (the same
    // chunk, one or two sub-steps later).
    auto epi_a = [&]() {
        const int i = 16 * tb_c + l16;
        float4 gc[4], rkc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gc[j] = *reinterpret_cast<const float4*>(&sm.gam[16 * j + 4 * q4]);
            rkc[j] = *reinterpret_cast<const float4*>(&sm.rk[16 * j + 4 * q4]);
        }
        // (keeps the compiler from sinking a read into a masked branch)
        asm volatile("" :: "v"(gc[0].x), "v"(rkc[0].x));
        const float gi = sm.gam[i];
        const float brk = sm.beta[i] * sm.rk[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 16 * j + 4 * q4;
            const float gcs[4] = {gc[j].x, gc[j].y, gc[j].z, gc[j].w};
            const float rks[4] = {rkc[j].x, rkc[j].y, rkc[j].z, rkc[j].w};
            f32x4 a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float dec = __expf(gi - gcs[r]);
                a[r] = (c + r < i) ? (brk * rks[r]) * (dec * accg[j][r]) : 0.0f;
                dmp[j][r] = (c + r <= i) ? dec : 0.0f;
            }
            *reinterpret_cast<float4*>(&sm.g[i * SF + c]) = make_float4(a[0], a[1], a[2], a[3]);
        }
    };
    auto epi_mp = [&]() {
        const int i = 16 * tb_c + l16;
        float4 rkc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) rkc[j] = *reinterpret_cast<const float4*>(&sm.rk[16 * j + 4 * q4]);
        const float rqi = sm.rq[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 16 * j + 4 * q4;
            const float rks[4] = {rkc[j].x, rkc[j].y, rkc[j].z, rkc[j].w};
            f32x4 mp;
#pragma unroll
            for (int r = 0; r < 4; ++r) mp[r] = (rqi * rks[r]) * (dmp[j][r] * accp[j][r]);
            uint2 h2, l2;
            split4(mp, h2, l2);
            lds_st8(&sm.mp[i * ST + (pperm(c) ^ swm)], h2.x, h2.y);
            lds_st8(&sm.mp[CH * ST + i * ST + (pperm(c) ^ swm)], l2.x, l2.y);
        }
    };

    // ---- the first chunk's staging and coefficient work
    {
        const int L0 = min(CH, a1 - a0);
        if (!state_w) {
            fetch(a0, L0);
            stage_kqv();
            if (wave == GW) gate_scan(L0);
        }
        __syncthreads();
        if (!state_w) gram();
        __syncthreads();
        if (!state_w) epi_a();
        __syncthreads();
    }

    // The two roles run as two loops over the same chunks, each with the same
    // seven barriers per chunk (so every barrier is met by all eight waves),
    // which keeps each role's registers out of the other's code.
    if (state_w) {
        int p = 0;                               // parity of chunk c
        for (int32_t c0 = a0; c0 < a1; c0 += CH) {
            const int L = min(CH, a1 - c0);
            const bool nxt = c0 + CH < a1;
            const int Ln = nxt ? min(CH, a1 - c0 - CH) : 0;
            set_lane();
            f32x4 z[4][VB];                      // Z tiles (t-block, v-block)
            f32x4 o[VB][4];                      // O^T tiles (v-block, t-block)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) { z[tb][vb] = f32x4{0, 0, 0, 0}; o[vb][tb] = f32x4{0, 0, 0, 0}; }
            // one k-step of Z = K S0^T (doz) or O1^T = S0 Q^T (doo): every
            // fragment load first, then the state split (VALU work that covers
            // the loads' latency), then the MFMAs
            auto early = [&](int ks, bool doz, bool doo) {
                bf16x8 ak[4], bq[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    if (doz) ak[tb] = frag_kq(sm.k, SK, 16 * tb + l16, 32 * ks, q4, swl);
                    if (doo) bq[tb] = frag_kq(sm.q, SK, 16 * tb + l16, 32 * ks, q4, swl);
                }
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 sh[VB], sl[VB];
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    uint2 h0, l0, h1, l1;
                    split4(st[2 * ks][vb], h0, l0);
                    split4(st[2 * ks + 1][vb], h1, l1);
                    sh[vb] = as_bf16x8(cat(h0, h1));
                    sl[vb] = as_bf16x8(cat(l0, l1));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    if (doz) {
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            z[tb][vb] = mfma(ak[tb], sh[vb], z[tb][vb]);
                            z[tb][vb] = mfma(ak[tb], sl[vb], z[tb][vb]);
                        }
                    }
                    if (doo) {
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            o[vb][tb] = mfma(sh[vb], bq[tb], o[vb][tb]);
                            o[vb][tb] = mfma(sl[vb], bq[tb], o[vb][tb]);
                        }
                    }
                }
            };

            // ---- A1: Z = K S0^T (O1 runs in A3, where the state waves have no
            // other work; beside Z here it measured the same)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) early(ks, true, false);
            __syncthreads();
            // ---- A2: O1^T = S0 Q^T, scaled by e^gamma_t r_q (also in runs
            // that store no outputs, so that it interleaves with Y)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) early(ks, false, true);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float e = sm.eg[p][16 * tb + l16];
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    o[vb][tb][0] *= e; o[vb][tb][1] *= e; o[vb][tb][2] *= e; o[vb][tb][3] *= e;
                }
            }
            // Y = V - diag(cy) Z in fp32 (four consecutive tokens of
            // one value column per lane, the accumulator layout), split hi/lo
            bf16x8 yh[2][VB], yl[2][VB];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    const int vr = 16 * (wave * VB + vb) + l16;
                    f32x4 nn[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int tb = 2 * ks + e;
                        const int tt = 16 * tb + 4 * q4;
                        const float4 cyv = *reinterpret_cast<const float4*>(&sm.cy[p][tt]);
                        float vv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int r = 0; r < 4; ++r) vv[r] += bf16_to_f32(sm.v[(tt + r) * PipeSmem::SV + vr]);
                        nn[e][0] = vv[0] - cyv.x * z[tb][vb][0];
                        nn[e][1] = vv[1] - cyv.y * z[tb][vb][1];
                        nn[e][2] = vv[2] - cyv.z * z[tb][vb][2];
                        nn[e][3] = vv[3] - cyv.w * z[tb][vb][3];
                    }
                    uint2 h0, l0, h1, l1;
                    split4(nn[0], h0, l0);
                    split4(nn[1], h1, l1);
                    yh[ks][vb] = as_bf16x8(cat(h0, h1));
                    yl[ks][vb] = as_bf16x8(cat(l0, l1));
                }
            __syncthreads();
            // ---- A3
            // cU(c) outside the 32 -> 64 merge's block
            cu_part(tid);
            __syncthreads();
            // ---- B1: U = cU Y (cU lower triangular: blocks above the diagonal
            // skipped)
            f32x4 u[4][VB];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) u[tb][vb] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (32 * ks > 16 * tb + 15) continue;
                    const bf16x8 ch = frag_perm(sm.cu + 0 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
                    const bf16x8 cl = frag_perm(sm.cu + 1 * CH * ST, ST, 16 * tb + l16, 32 * ks, q4);
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        u[tb][vb] = mfma(ch, yh[ks][vb], u[tb][vb]);
                        u[tb][vb] = mfma(ch, yl[ks][vb], u[tb][vb]);
                        u[tb][vb] = mfma(cl, yh[ks][vb], u[tb][vb]);
                    }
                }
            __syncthreads();
            // ---- B2: O^T += U^T (M o P)^T (U split: A operand, permuted
            // t-slots), stored; cK . U split; state rows 0-63
            if (wo) {
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
                        if (32 * ks > 16 * tb + 15) continue;
                        const bf16x8 mh = frag_kq(sm.mp, ST, 16 * tb + l16, 32 * ks, q4, swm);
                        const bf16x8 ml = frag_kq(sm.mp + CH * ST, ST, 16 * tb + l16, 32 * ks, q4, swm);
#pragma unroll
                        for (int vb = 0; vb < VB; ++vb) {
                            o[vb][tb] = mfma(uh[ks][vb], mh, o[vb][tb]);
                            o[vb][tb] = mfma(ul[ks][vb], mh, o[vb][tb]);
                            o[vb][tb] = mfma(uh[ks][vb], ml, o[vb][tb]);
                        }
                    }
                // lane holds O[t = 16 tb + l16][v = 16 (wave VB + vb) + 4 q4 .. + 3].
                // fp32 outputs go straight out (64 bytes of a row per lane group;
                // rows t >= L fall outside the descriptor's range and are
                // dropped); bf16 outputs go to the LDS tile, stored in B3 as
                // whole rows (a direct store wrote 32 bytes of each of 16 rows,
                // and at full load those partial lines cost ~1.3 us per chunk)
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        if constexpr (sizeof(OT) == 4) {
                            const uint32_t row_o = static_cast<uint32_t>(HV * D) * sizeof(OT);
                            const rsrc_t ro = make_rsrc(out + static_cast<size_t>(c0) * HV * D, L * row_o);
                            const uint32_t off = static_cast<uint32_t>(16 * tb + l16) * row_o +
                                static_cast<uint32_t>(hv * D + 16 * (wave * VB + vb) + 4 * q4) * sizeof(OT);
                            buf_st16(ro, off, __float_as_uint(o[vb][tb][0]), __float_as_uint(o[vb][tb][1]),
                                     __float_as_uint(o[vb][tb][2]), __float_as_uint(o[vb][tb][3]));
                        } else {
                            lds_st8(&sm.ob[(16 * tb + l16) * PipeSmem::SO + 16 * (wave * VB + vb) + 4 * q4],
                                    pack_bf16x2(o[vb][tb][0], o[vb][tb][1]),
                                    pack_bf16x2(o[vb][tb][2], o[vb][tb][3]));
                        }
                    }
                }
            }
            __syncthreads();
            // ---- B3: the bf16 output tile as whole rows (wave w: rows 16 w ..
            // 16 w + 15, four per store); cK . U split; the state update
            if constexpr (sizeof(OT) == 2) {
                if (wo) {
                    const uint32_t row_o = static_cast<uint32_t>(HV * D) * sizeof(OT);
                    const rsrc_t ro = make_rsrc(out + static_cast<size_t>(c0) * HV * D, L * row_o);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * wave + 4 * i + (lane >> 4);
                        const uint4 w = *reinterpret_cast<const uint4*>(&sm.ob[row * PipeSmem::SO + 8 * (lane & 15)]);
                        // (nontemporal: the outputs are not read again here)
                        buf_st16_nt(ro, static_cast<uint32_t>(row) * row_o +
                                            static_cast<uint32_t>(hv * D + 8 * (lane & 15)) * sizeof(OT),
                                    w.x, w.y, w.z, w.w);
                    }
                }
            }
            bf16x8 chk[2][VB], clk[2][VB];       // cK . U, split
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    f32x4 a = u[2 * ks][vb], b = u[2 * ks + 1][vb];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        a[r] *= sm.ck[p][32 * ks + 4 * q4 + r];
                        b[r] *= sm.ck[p][32 * ks + 16 + 4 * q4 + r];
                    }
                    uint2 h0, l0, h1, l1;
                    split4(a, h0, l0);
                    split4(b, h1, l1);
                    chk[ks][vb] = as_bf16x8(cat(h0, h1));
                    clk[ks][vb] = as_bf16x8(cat(l0, l1));
                }
            // S0^T <- e^{gamma_L} S0^T + K^T (cK . U), key blocks kb0 .. kb0 + 3
            auto update = [&](int kb0) {
                const float egl = sm.egl[p];
#pragma unroll
                for (int kb = kb0; kb < kb0 + 4; ++kb) {
                    bf16x8 ak[2];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) ak[ks] = frag_perm(sm.kt, ST, 16 * kb + l16, 32 * ks, q4);
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) {
                        f32x4 acc = st[kb][vb];
                        acc[0] *= egl; acc[1] *= egl; acc[2] *= egl; acc[3] *= egl;
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            acc = mfma(ak[ks], chk[ks][vb], acc);
                            acc = mfma(ak[ks], clk[ks][vb], acc);
                        }
                        st[kb][vb] = acc;
                    }
                }
            };
            update(0);
            update(4);
            __syncthreads();
            p ^= 1;
        }
    } else {
        for (int32_t c0 = a0; c0 < a1; c0 += CH) {
            const bool nxt = c0 + CH < a1;
            const int Ln = nxt ? min(CH, a1 - c0 - CH) : 0;
            const int L = min(CH, a1 - c0);
            const int pc = ((c0 - a0) / CH) & 1;         // parity of chunk c
            set_lane();
            // ---- A1: K^T(c); forward substitution of the four diagonal 16x16
            // blocks of chunk c (wave WF: lane = 16 block + column c).  Lane c
            // holds column c of each row of the block; row r's entry A[r][j]
            // reaches every lane of the block by a DPP row broadcast from lane
            // j.  Right-looking order: once T[j][c] is final, every later row r
            // adds A[r][j] T[j][c], so each row still accumulates its terms in
            // ascending j.
            if (wave == GW) coefs(L, pc);
            if (wave != WF && nxt) fetch(c0 + CH, Ln);
            if (wave == WF) {
                __builtin_amdgcn_s_setprio(2);
                const int b = lane >> 4;
                fwd_subst16(&sm.g[(16 * b) * SF + 16 * b], SF, lane & 15);
                __builtin_amdgcn_s_setprio(0);
            } else if (wave == WM || wave == WM + 1) {
                epi_mp();                        // M o P-hat(c), rows of this wave
            }
            __syncthreads();
            // ---- A2: K^T(c); merge 16 -> 32 for block pairs (0,1), (2,3) on
            // fp32 MFMA (wave WM + pair): X = A21 T11 through the LDS scratch and
            // straight back into the same wave, then T21 = -T22 X
            stage_kt();
            if (wave == WF && nxt) fetch(c0 + CH, Ln);
            if (wave == WM || wave == WM + 1) {
                __builtin_amdgcn_s_setprio(2);
                const int pw = wave - WM;
                const int b0 = 32 * pw, b1 = b0 + 16;
                float a[4], bb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    a[kk] = sm.g[(b1 + l16) * SF + b0 + 4 * kk + q4];
                    bb[kk] = sm.g[(b0 + 4 * kk + q4) * SF + b0 + l16];
                }
                f32x4 x = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) x = mfma4(a[kk], bb[kk], x);
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.xs[(16 * pw + 4 * q4 + r) * 36 + l16] = x[r];
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    a[kk] = sm.g[(b1 + l16) * SF + b1 + 4 * kk + q4];
                    bb[kk] = sm.xs[(16 * pw + 4 * kk + q4) * 36 + l16];
                }
                f32x4 t = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) t = mfma4(a[kk], bb[kk], t);
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.g[(b1 + 4 * q4 + r) * SF + b0 + l16] = -t[r];
            }
            __syncthreads();
            // ---- A3: merge 32 -> 64 (wave WM + tj: output column block tj of
            // the lower-left 32x32 block T21, whose cU block goes straight from
            // the accumulators to cU); M o P-hat(c) rows of waves 4 and 7
            // (the column block is a compile-time constant in each wave's copy,
            // so the triangular k-ranges unroll with every operand read issued
            // up front)
            auto merge2 = [&](auto tjc) {
                constexpr int tj = decltype(tjc)::value;
                constexpr int k0 = 4 * tj;
                float a[2][8], bb[8];
#pragma unroll
                for (int kk = k0; kk < 8; ++kk) {
                    bb[kk] = sm.g[(4 * kk + q4) * SF + 16 * tj + l16];
#pragma unroll
                    for (int ti = 0; ti < 2; ++ti) a[ti][kk] = sm.g[(32 + 16 * ti + l16) * SF + 4 * kk + q4];
                }
                f32x4 x[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
                for (int kk = k0; kk < 8; ++kk) {
#pragma unroll
                    for (int ti = 0; ti < 2; ++ti) x[ti] = mfma4(a[ti][kk], bb[kk], x[ti]);
                }
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sm.xs[(16 * ti + 4 * q4 + r) * 36 + 16 * tj + l16] = x[ti][r];
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    bb[kk] = sm.xs[(4 * kk + q4) * 36 + 16 * tj + l16];
#pragma unroll
                    for (int ti = 0; ti < 2; ++ti) a[ti][kk] = sm.g[(32 + 16 * ti + l16) * SF + 32 + 4 * kk + q4];
                }
                f32x4 t[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    t[1] = mfma4(a[1][kk], bb[kk], t[1]);
                    if (kk < 4) t[0] = mfma4(a[0][kk], bb[kk], t[0]);
                }
                // cU = T21 diag(beta) (lane: rows 32 + 16 ti + 4 q4 + r, column
                // 16 tj + l16), hi/lo, one bf16 per store
                const float bc = sm.beta[16 * tj + l16];
                const int pcol = pperm(16 * tj + l16);
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    f32x4 u;
#pragma unroll
                    for (int r = 0; r < 4; ++r) u[r] = -t[ti][r] * bc;
                    uint2 h2, l2;
                    split4(u, h2, l2);
                    const uint32_t hv[4] = {h2.x, h2.x >> 16, h2.y, h2.y >> 16};
                    const uint32_t lv[4] = {l2.x, l2.x >> 16, l2.y, l2.y >> 16};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        bf16_t* dst = sm.cu + (32 + 16 * ti + 4 * q4 + r) * ST + pcol;
                        dst[0] = static_cast<bf16_t>(hv[r]);
                        dst[CH * ST] = static_cast<bf16_t>(lv[r]);
                    }
                }
            };
            if (wave == WM) {
                merge2(std::integral_constant<int, 0>{});
                __builtin_amdgcn_s_setprio(0);
            } else if (wave == WM + 1) {
                merge2(std::integral_constant<int, 1>{});
                __builtin_amdgcn_s_setprio(0);
            } else {
                epi_mp();
            }
            __syncthreads();
            // ---- B1: K, Q, V^T(c + 1); gate scan(c + 1)
            if (nxt) {
                stage_kqv();
                if (wave == GW) gate_scan(Ln);
            }
            __syncthreads();
            // ---- B2: G, P, norms(c + 1)
            if (nxt) gram();
            __syncthreads();
            // ---- B3: A, M o P-hat, coefficients(c + 1)
            if (nxt) epi_a();
            __syncthreads();
        }
    }

    // ---- the final state back to the slot (or the segment's matrix)
    if (state_w && (!SEG || fin)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
                const int v = 16 * (wave * VB + vb) + l16;
                *reinterpret_cast<float4*>(fin + static_cast<size_t>(v) * D + 16 * kb + 4 * q4) =
                    make_float4(st[kb][vb][0], st[kb][vb][1], st[kb][vb][2], st[kb][vb][3]);
            }
    }
}

namespace {
template <int D, typename IT, typename OT>
hipError_t run_prefill(const void* q, const void* k, const void* v, const GateArgs& ga,
                       const int32_t* cu, int32_t n_seqs, const int32_t* slot,
                       float* rec, void* out, const gdn_dims& d, int32_t sqk, int32_t sv,
                       float scale, int32_t flags, const SegArgs& sg, int32_t nz,
                       const int32_t* err, hipStream_t st) {
    dim3 grid(d.num_v_heads, n_seqs, nz);
    const int32_t ns = (flags & GDN_FLAG_PREFILL_NS3) ? 3 : (flags & GDN_FLAG_PREFILL_NS4) ? 4 : 0;
    auto go = [&](auto kernel, int32_t nsr) {
        return launch(kernel, grid, dim3(PF_NT), 0, st, static_cast<const IT*>(q),
                      static_cast<const IT*>(k), static_cast<const IT*>(v), ga, cu, slot, rec,
                      static_cast<OT*>(out), d.num_k_heads, d.num_v_heads, sqk, sv, scale, flags,
                      nsr, sg, err);
    };
    // d = 128 with bf16 inputs: the pipelined chunk step, for whole runs and
    // unpaired segment runs (the Newton-Schulz variant and paired P/B runs keep
    // prefill_kernel, and so does a call that asks for the single-role step;
    // both compute the same values bit for bit)
    if constexpr (D == 128 && std::is_same<IT, bf16_t>::value) {
        if (ns == 0 && !(sg.pass == 1 && sg.pair) && !(flags & GDN_FLAG_PREFILL_SINGLE_ROLE)) {
            auto go2 = [&](auto kernel) {
                return launch(kernel, grid, dim3(PF_NT), 0, st, static_cast<const bf16_t*>(q),
                              static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), ga, cu,
                              slot, rec, static_cast<OT*>(out), d.num_k_heads, d.num_v_heads, sqk,
                              sv, scale, flags, sg, err);
            };
            return sg.pass != 0 ? go2(prefill_pipe_kernel<OT, true>) : go2(prefill_pipe_kernel<OT, false>);
        }
    }
    // pass 2 never pairs runs: it takes the unpaired kernel, whose registers
    // are those of a whole-sequence run
    if (sg.pass == 1 && sg.pair)
        return ns > 0 ? go(prefill_kernel<D, IT, OT, true, true, true>, ns)
                      : go(prefill_kernel<D, IT, OT, false, true, true>, 0);
    if (sg.pass != 0)
        return ns > 0 ? go(prefill_kernel<D, IT, OT, true, true, false>, ns)
                      : go(prefill_kernel<D, IT, OT, false, true, false>, 0);
    return ns > 0 ? go(prefill_kernel<D, IT, OT, true, false, false>, ns)
                  : go(prefill_kernel<D, IT, OT, false, false, false>, 0);
}

template <int D, typename IT>
hipError_t pick_out(gdn_dtype out_dt, const void* q, const void* k, const void* v, const GateArgs& ga,
                    const int32_t* cu, int32_t n_seqs, const int32_t* slot,
                    float* rec, void* out, const gdn_dims& d, int32_t sqk, int32_t sv, float scale,
                    int32_t flags, const SegArgs& sg, int32_t nz, const int32_t* err,
                    hipStream_t st) {
    return out_dt == GDN_BF16
        ? run_prefill<D, IT, bf16_t>(q, k, v, ga, cu, n_seqs, slot, rec, out, d, sqk, sv, scale, flags, sg, nz, err, st)
        : run_prefill<D, IT, float>(q, k, v, ga, cu, n_seqs, slot, rec, out, d, sqk, sv, scale, flags, sg, nz, err, st);
}

hipError_t prefill_pass(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                        const GateArgs& ga, const int32_t* cu, int32_t n_seqs,
                        const int32_t* slot, float* rec, void* out, gdn_dtype out_dt,
                        const gdn_dims& d, int32_t sqk, int32_t sv, float scale, int32_t flags,
                        const SegArgs& sg, int32_t nz, const int32_t* err, hipStream_t st) {
    const int D = d.head_k_dim;
    if (in_dt == GDN_F32) {
        if (D == 32) return pick_out<32, float>(out_dt, q, k, v, ga, cu, n_seqs, slot, rec, out, d, sqk, sv, scale, flags, sg, nz, err, st);
        return pick_out<64, float>(out_dt, q, k, v, ga, cu, n_seqs, slot, rec, out, d, sqk, sv, scale, flags, sg, nz, err, st);
    }
    if (D == 32) return pick_out<32, bf16_t>(out_dt, q, k, v, ga, cu, n_seqs, slot, rec, out, d, sqk, sv, scale, flags, sg, nz, err, st);
    if (D == 64) return pick_out<64, bf16_t>(out_dt, q, k, v, ga, cu, n_seqs, slot, rec, out, d, sqk, sv, scale, flags, sg, nz, err, st);
    return pick_out<128, bf16_t>(out_dt, q, k, v, ga, cu, n_seqs, slot, rec, out, d, sqk, sv, scale, flags, sg, nz, err, st);
}
}  // namespace

// Head dims 32, 64 and 128 with d_k == d_v; fp32 inputs (hi/lo planes in LDS)
// only up to 64, where the doubled input planes fit in LDS.
bool prefill_supported(const gdn_dims& d, gdn_dtype in_dt) {
    const int D = d.head_k_dim;
    if (d.head_v_dim != D || (D != 32 && D != 64 && D != 128)) return false;
    return in_dt == GDN_BF16 || (in_dt == GDN_F32 && D <= 64);
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                          const GateArgs& ga, const int32_t* cu, int32_t n_seqs,
                          const int32_t* slot, float* rec, void* out, gdn_dtype out_dt,
                          const gdn_dims& d, int32_t sqk, int32_t sv, float scale, int32_t flags,
                          const int32_t* err, hipStream_t st) {
    if (n_seqs == 0) return hipSuccess;
    if (!prefill_supported(d, in_dt)) return hipErrorInvalidValue;
    return prefill_pass(q, k, v, in_dt, ga, cu, n_seqs, slot, rec, out, out_dt, d, sqk, sv,
                        scale, flags, SegArgs{nullptr, 0, 0, 0, 0, nullptr, 0}, 1, err, st);
}

// ---------------------------------------------------------------------------
// Segment-parallel prefill

// Start states of segments 2.. of each sequence: start[j + 1] = start[j] P_j + B_j.
// Row v of a state depends only on row v of the previous one, so a workgroup
// owns 16 state rows of one (sequence, value head).  Each step is a 16 x D by
// D x D product on fp32 MFMA (v_mfma_f32_16x16x4f32: fp32 products and sums),
// accumulated onto B_j's rows: wave w computes the 16-column tiles
// w TPW .. w TPW + TPW - 1; lane group q of a wave takes the inner indices
// KT q + t (t = 0 .. KT - 1), so a lane's row fragment is one contiguous run of
// the LDS row buffer, and the wave's columns of P_j come from global memory
// straight into registers in the operand layout -- P_{j+1}'s (and B_{j+1}'s)
// during step j.
template <int D>
__global__ __launch_bounds__(256) void prefill_seg_scan_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slot, int32_t HV, int32_t seg_len,
    int32_t head, float* __restrict__ ws, const int32_t* __restrict__ err_flag) {
    constexpr int NTL = D / 16;                  // 16-column tiles
    constexpr int TPW = NTL >= 4 ? NTL / 4 : 1;  // tiles per wave
    constexpr int KT = D / 4;                    // inner steps per lane group
    constexpr int RS = D + 4;                    // LDS row stride (floats): 2-way at most
    __shared__ float rows[16 * RS];
    if (call_rejected(err_flag)) return;
    const int hv = blockIdx.x, n = blockIdx.y, rb = blockIdx.z;
    const int32_t t0 = cu[n], t1 = cu[n + 1];
    if (slot[n] <= 0 || t1 <= t0) return;
    const int32_t nseg = seg_count(t1 - t0, head, seg_len);
    if (nseg < 3) return;
    const int64_t id0 = n + t0 / seg_len;
    auto wsm = [&](int64_t id, int kind) {
        return ws + ((id * 3 + kind) * HV + hv) * static_cast<size_t>(D) * D;
    };
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int q = lane >> 4, l16 = lane & 15;
    const bool active = wave * TPW < NTL;        // D = 32: two waves hold the two tiles
    const int v0 = 16 * rb;                      // first state row of the block

    // start[1]'s rows into LDS
    {
        const float* s1 = wsm(id0 + 1, 0) + static_cast<size_t>(v0) * D;
        for (int i = tid; i < 16 * D; i += 256) rows[(i / D) * RS + i % D] = s1[i];
    }
    // P_j in the B-operand layout: pc[tt][t] = P_j[KT q + t][16 (wave TPW + tt) + l16];
    // B_j in the accumulator layout: bc[tt][r] = B_j[v0 + 4 q + r][16 (wave TPW + tt) + l16]
    float pc[TPW][KT], pn[TPW][KT];
    f32x4 bc[TPW], bn[TPW];
    auto load_pb = [&](int j, float (&pp)[TPW][KT], f32x4 (&bb)[TPW]) {
        const float* P = wsm(id0 + j, 1);
        const float* Bm = wsm(id0 + j, 2);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int col = 16 * (wave * TPW + tt) + l16;
#pragma unroll
            for (int t = 0; t < KT; ++t) pp[tt][t] = P[static_cast<size_t>(KT * q + t) * D + col];
#pragma unroll
            for (int r = 0; r < 4; ++r) bb[tt][r] = Bm[static_cast<size_t>(v0 + 4 * q + r) * D + col];
        }
    };
    if (active) load_pb(1, pc, bc);
    for (int j = 1; j <= nseg - 2; ++j) {
        __syncthreads();                         // rows holds start[j]
        if (active && j + 1 <= nseg - 2) load_pb(j + 1, pn, bn);
        f32x4 acc[TPW];
        if (active) {
            float a[KT];
#pragma unroll
            for (int t = 0; t < KT; t += 4) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(&rows[l16 * RS + KT * q + t]);
                a[t] = v[0]; a[t + 1] = v[1]; a[t + 2] = v[2]; a[t + 3] = v[3];
            }
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) acc[tt] = bc[tt];
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) acc[tt] = mfma4(a[t], pc[tt][t], acc[tt]);
        }
        __syncthreads();                         // every read of start[j] is done
        if (active) {
            float* dst = wsm(id0 + j + 1, 0);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int col = 16 * (wave * TPW + tt) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    rows[(4 * q + r) * RS + col] = acc[tt][r];
                    dst[static_cast<size_t>(v0 + 4 * q + r) * D + col] = acc[tt][r];
                }
            }
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                bc[tt] = bn[tt];
#pragma unroll
                for (int t = 0; t < KT; ++t) pc[tt][t] = pn[tt][t];
            }
        }
    }
}

int64_t prefill_segment_ids(int32_t n_seqs, int32_t total_tokens, int32_t seg_len) {
    return static_cast<int64_t>(n_seqs) + total_tokens / seg_len + 1;
}

// Bytes of the segment matrices; the two segment maps ([n_seqs + 1] int32
// each) follow them.
static size_t seg_matrix_bytes(const gdn_dims& d, int32_t n_seqs, int32_t total_tokens,
                               int32_t seg_len) {
    const size_t mat = static_cast<size_t>(d.head_k_dim) * d.head_v_dim * sizeof(float);
    return static_cast<size_t>(prefill_segment_ids(n_seqs, total_tokens, seg_len)) * 3 *
           static_cast<size_t>(d.num_v_heads) * mat;
}

size_t prefill_segmented_workspace(const gdn_dims& d, int32_t n_seqs, int32_t total_tokens,
                                   int32_t seg_len) {
    if (seg_len <= 0) return 0;
    return seg_matrix_bytes(d, n_seqs, total_tokens, seg_len) +
           ((2 * (static_cast<size_t>(n_seqs) + 1) * sizeof(int32_t) + 255) & ~static_cast<size_t>(255));
}

// Segment maps of the two passes: map1[n] / map2[n] = the workgroups of pass
// 1 (P/B runs only: segment 0 of every sequence has a grid row of its own) /
// pass 2 that sequences 0 .. n-1 own.  Pass 1: a sequence of nseg segments
// owns its nseg - 2 middle segments' runs (one workgroup each when paired, two
// otherwise); pass 2 its nseg - 1 reruns.  One workgroup: each thread counts a contiguous range of sequences,
// then the partial sums are scanned in LDS (fixed order).
__global__ __launch_bounds__(1024) void prefill_seg_map_kernel(
    const int32_t* __restrict__ cu, int32_t n_seqs, int32_t head, int32_t seg, int32_t pair,
    int32_t* __restrict__ map1, int32_t* __restrict__ map2, const int32_t* __restrict__ err_flag) {
    __shared__ int32_t s1[1024], s2[1024];
    if (call_rejected(err_flag)) return;
    const int t = threadIdx.x;
    const int per = (n_seqs + 1023) / 1024;
    const int b0 = min(t * per, n_seqs), b1 = min(b0 + per, n_seqs);
    auto counts = [&](int n, int32_t& c1, int32_t& c2) {
        const int32_t L = cu[n + 1] - cu[n];
        const int32_t m = L > 0 ? seg_count(L, head, seg) : 1;
        c1 = m > 2 ? (pair ? 1 : 2) * (m - 2) : 0;
        c2 = m - 1;
    };
    int32_t a1 = 0, a2 = 0;
    for (int n = b0; n < b1; ++n) {
        int32_t c1, c2;
        counts(n, c1, c2);
        a1 += c1;
        a2 += c2;
    }
    s1[t] = a1;
    s2[t] = a2;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {     // inclusive scan (Hillis-Steele)
        const int32_t v1 = t >= off ? s1[t - off] : 0;
        const int32_t v2 = t >= off ? s2[t - off] : 0;
        __syncthreads();
        s1[t] += v1;
        s2[t] += v2;
        __syncthreads();
    }
    int32_t r1 = t > 0 ? s1[t - 1] : 0, r2 = t > 0 ? s2[t - 1] : 0;
    for (int n = b0; n < b1; ++n) {
        map1[n] = r1;
        map2[n] = r2;
        int32_t c1, c2;
        counts(n, c1, c2);
        r1 += c1;
        r2 += c2;
    }
    if (t == 1023) {
        map1[n_seqs] = s1[1023];
        map2[n_seqs] = s2[1023];
    }
}

// Bounds on the workgroups of each pass over all sequences: a sequence of
// L > head tokens has nseg - 1 = ceil((L - head) / seg_len) <= L / seg_len + 1
// segments past the first; pass 1 holds every segment 0 and the middle
// segments' P/B runs (one workgroup each when paired, two otherwise), pass 2
// the reruns.
static int64_t seg_rest(int32_t n_seqs, int32_t total_tokens, int32_t seg_len) {
    return static_cast<int64_t>(total_tokens) / seg_len + n_seqs;
}
static int64_t seg_grid1(int32_t n_seqs, int32_t total_tokens, const PrefillSchedule& sch) {
    return n_seqs + (sch.paired ? 1 : 2) * seg_rest(n_seqs, total_tokens, sch.seg_len);
}
bool prefill_seg_grid_fits(int32_t n_seqs, int32_t total_tokens, PrefillSchedule sch) {
    return sch.seg_len <= 0 || seg_grid1(n_seqs, total_tokens, sch) <= 65535;
}

// The schedule the plain prefill call takes for these sizes on the current
// device (seg_len 0: whole sequences).  Units of the model are chunk-times of
// one workgroup per CU; c = chunks per sequence (average), whole sequences
// take c.
//  * Few (sequence, value head) runs (G = n_seqs HV at most half the CUs), head
//    dim 128 (the pipelined step, whose P and B runs are separate workgroups):
//    a head of h chunks and m tails of s chunks.  Pass 1 runs segment 0 (G
//    workgroups, h chunks) and the P and B runs of the m - 1 middle tails
//    (2 G (m - 1) workgroups of s chunks) on the CUs segment 0 leaves free, in
//    r = ceil(2 G (m - 1) / (CUs - G)) rounds; pass 2 reruns the m tails in
//    ceil(G m / CUs) rounds.  With s = ceil(c / (r + m)) and h = c - m s the
//    head lasts about as long as the P/B rounds; the model charges
//    max(h, r s) + ceil(G m / CUs) s, plus about half a chunk per scan step and
//    two for the extra launches, and the call segments where that is at most
//    0.85 c.  (One 16,384-token sequence: head 48, tails 26 chunks.)
//  * Few runs at head dims 32 and 64 (prefill_kernel, P and B runs paired in
//    one workgroup, about 1.3 chunk-times per chunk): equal segments; with m
//    segments of c / m chunks, pass 1 runs G (m - 1) workgroups and pass 2
//    G (m - 1), each in ceil(count / CUs) rounds, plus the scan's m - 2 steps
//    at about a quarter chunk each; the call segments where that gains at
//    least 15%.
//  * A busy chip: a head of the chunks a CU carries when the work is spread
//    evenly (C = ceil(chunks x HV / CUs), chunks estimated as total / 64 plus
//    half a chunk per sequence) and tail segments of about C / 4 chunks.  A
//    sequence no longer than the head is one segment and runs whole in pass 1,
//    so equal lengths keep whole runs; the tails of longer sequences get their
//    P/B runs (as separate workgroups, which keep the registers of a whole run,
//    on the CUs that shorter sequences free during pass 1), and reruns about
//    C / 4 chunks long in pass 2.
static PrefillSchedule auto_schedule_model(const gdn_dims& d, int32_t n_seqs, int32_t total_tokens) {
    if (n_seqs <= 0 || total_tokens <= 0) return PrefillSchedule{0, 0, true};
    const int64_t groups = static_cast<int64_t>(n_seqs) * d.num_v_heads;
    const int64_t cus = cu_count();
    if (groups * 2 > cus) {
        const int64_t chunks = (static_cast<int64_t>(total_tokens) + 63) / 64 + (n_seqs + 1) / 2;
        const int64_t bal = (chunks * d.num_v_heads + cus - 1) / cus;
        if (bal < 8) return PrefillSchedule{0, 0, true};
        const int64_t tail = (bal + 3) / 4;
        return PrefillSchedule{static_cast<int32_t>(64 * tail), static_cast<int32_t>(64 * bal), false};
    }
    const int64_t chunks = (total_tokens / n_seqs + 63) / 64;
    if (chunks < 8) return PrefillSchedule{0, 0, true};
    if (d.head_k_dim == 128) {
        double best = static_cast<double>(chunks);
        int64_t best_s = 0, best_h = 0;
        for (int64_t m = 2; m <= 64; ++m) {                    // tails after the head
            const int64_t r = (2 * groups * (m - 1) + (cus - groups) - 1) / (cus - groups);
            const int64_t s = (chunks + r + m - 1) / (r + m);
            const int64_t h = std::max(s, chunks - m * s);
            const int64_t r2 = (groups * m + cus - 1) / cus;
            const double t = static_cast<double>(std::max(h, r * s) + r2 * s) + 0.55 * static_cast<double>(m - 1) + 2.0;
            if (t < best * 0.999) { best = t; best_s = s; best_h = h; }
        }
        return (best_s > 0 && best <= 0.85 * static_cast<double>(chunks))
            ? PrefillSchedule{static_cast<int32_t>(64 * best_s), static_cast<int32_t>(64 * best_h), false}
            : PrefillSchedule{0, 0, true};
    }
    double best = static_cast<double>(chunks);
    int32_t best_len = 0;
    for (int64_t m = 3; m <= 64; ++m) {
        const int64_t per = (chunks + m - 1) / m;          // chunks per segment
        const int64_t mm = (chunks + per - 1) / per;        // segments actually used
        if (mm < 3) continue;
        const int64_t r1 = (groups * (mm - 1) + cus - 1) / cus;
        const int64_t r2 = (groups * (mm - 1) + cus - 1) / cus;
        const double t = static_cast<double>(per) * (1.3 * r1 + r2) + 0.25 * (mm - 2);
        if (t < best * 0.999) { best = t; best_len = static_cast<int32_t>(per * 64); }
    }
    return (best <= 0.85 * chunks) ? PrefillSchedule{best_len, best_len, true} : PrefillSchedule{0, 0, true};
}

PrefillSchedule prefill_auto_schedule(const gdn_dims& d, int32_t n_seqs, int32_t total_tokens) {
    const PrefillSchedule sch = auto_schedule_model(d, n_seqs, total_tokens);
    // many thousands of sequences could overflow a segment pass's grid: whole runs then
    return prefill_seg_grid_fits(n_seqs, total_tokens, sch) ? sch : PrefillSchedule{0, 0, true};
}

hipError_t launch_prefill_segmented(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                    const GateArgs& ga, const int32_t* cu, int32_t n_seqs,
                                    int32_t total_tokens, const int32_t* slot, float* rec,
                                    void* out, gdn_dtype out_dt, const gdn_dims& d,
                                    int32_t sqk, int32_t sv, float scale, int32_t flags,
                                    PrefillSchedule sch, float* ws, const int32_t* err,
                                    hipStream_t st) {
    if (n_seqs == 0) return hipSuccess;
    const int32_t seg_len = sch.seg_len, head = sch.head, pair = sch.paired ? 1 : 0;
    if (!prefill_supported(d, in_dt) || seg_len <= 0 || seg_len % CH != 0 || head < seg_len ||
        head % CH != 0)
        return hipErrorInvalidValue;
    const int64_t g1 = seg_grid1(n_seqs, total_tokens, sch);
    const int64_t g2 = seg_rest(n_seqs, total_tokens, seg_len);
    if (g1 > 65535) return hipErrorInvalidValue;
    int32_t* map1 = reinterpret_cast<int32_t*>(
        reinterpret_cast<char*>(ws) + seg_matrix_bytes(d, n_seqs, total_tokens, seg_len));
    int32_t* map2 = map1 + (n_seqs + 1);
    hipError_t e = launch(prefill_seg_map_kernel, dim3(1), dim3(1024), 0, st, cu, n_seqs, head,
                          seg_len, pair, map1, map2, err);
    if (e != hipSuccess) return e;
    // the pass kernels take the sequence count as the grid's y extent for
    // whole runs; segment passes index the map with blockIdx.y instead
    e = prefill_pass(q, k, v, in_dt, ga, cu, static_cast<int32_t>(g1), slot, rec, out, out_dt, d,
                     sqk, sv, scale, flags, SegArgs{ws, seg_len, 1, head, pair, map1, n_seqs}, 1,
                     err, st);
    if (e != hipSuccess) return e;
    {
        const int D = d.head_k_dim;
        const dim3 grid(d.num_v_heads, n_seqs, D / 16);
        if (D == 32) e = launch(prefill_seg_scan_kernel<32>, grid, dim3(256), 0, st, cu, slot, d.num_v_heads, seg_len, head, ws, err);
        else if (D == 64) e = launch(prefill_seg_scan_kernel<64>, grid, dim3(256), 0, st, cu, slot, d.num_v_heads, seg_len, head, ws, err);
        else e = launch(prefill_seg_scan_kernel<128>, grid, dim3(256), 0, st, cu, slot, d.num_v_heads, seg_len, head, ws, err);
        if (e != hipSuccess) return e;
    }
    if (g2 <= 0) return hipSuccess;
    return prefill_pass(q, k, v, in_dt, ga, cu, static_cast<int32_t>(g2), slot, rec, out, out_dt,
                        d, sqk, sv, scale, flags, SegArgs{ws, seg_len, 2, head, 0, map2, n_seqs},
                        1, err, st);
}

}  // namespace gdn
