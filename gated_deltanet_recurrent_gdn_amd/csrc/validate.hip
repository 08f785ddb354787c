// validate.hip -- device-side index validation (fail-closed contract).
//
// RL-Kernel PR #469, "State ABI: index validation and the two NULL_BLOCK_ID
// contracts": an active index (> 0) must be < num_slots and must not repeat;
// indices <= 0 are inactive and may repeat freely.  cu_seqlens must start at
// 0, never decrease, and end at the token count.
//
// One workgroup of 1024 threads writes *err_flag unconditionally (0 when
// clean), so the flag never needs clearing beforehand.  Repeats are found by
// comparing each row against every earlier row through LDS tiles:
// O(n^2 / 1024) compares per thread, which is microseconds for decode batches.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

constexpr int VAL_THREADS = 1024;

// n slot indices; cu (when non-null) describes n_cu sequences (n_cu + 1 offsets)
// over `total` tokens -- n_cu == n except in a mixed step, whose slot list also
// holds the decode rows before the prefill sequences.
__global__ __launch_bounds__(VAL_THREADS) void validate_kernel(
    const int32_t* __restrict__ slot, int32_t n, int32_t num_slots,
    const int32_t* __restrict__ cu, int32_t n_cu, int32_t total, int32_t* __restrict__ err_flag) {
    __shared__ int32_t tile[VAL_THREADS];
    __shared__ int32_t bits_sh;
    const int tid = threadIdx.x;
    if (tid == 0) bits_sh = 0;
    int bits = 0;
    for (int i = tid; i < n; i += VAL_THREADS) {
        const int32_t s = slot[i];
        if (s > 0 && s >= num_slots) bits |= GDN_EFLAG_SLOT_RANGE;
    }
    if (cu != nullptr) {
        for (int i = tid; i < n_cu; i += VAL_THREADS)
            if (cu[i + 1] < cu[i]) bits |= GDN_EFLAG_SEQLENS;
        if (tid == 0 && (cu[0] != 0 || cu[n_cu] != total)) bits |= GDN_EFLAG_SEQLENS;
    }

    for (int i0 = 0; i0 < n; i0 += VAL_THREADS) {          // uniform loop
        const int i = i0 + tid;
        const int32_t s = (i < n) ? slot[i] : 0;
        for (int j0 = 0; j0 <= i0; j0 += VAL_THREADS) {    // uniform loop
            __syncthreads();
            tile[tid] = (j0 + tid < n) ? slot[j0 + tid] : 0;
            __syncthreads();
            if (s > 0) {
                const int jmax = min(VAL_THREADS, i - j0);   // rows j < i only
                for (int j = 0; j < jmax; ++j)
                    if (tile[j] == s) bits |= GDN_EFLAG_SLOT_REPEAT;
            }
        }
    }
    __syncthreads();
    if (bits) atomicOr(&bits_sh, bits);
    __syncthreads();
    if (tid == 0) *err_flag = bits_sh;
}

hipError_t launch_validate(const int32_t* slot_idx, int32_t n, int32_t num_slots,
                           const int32_t* cu_seqlens, int32_t n_cu, int32_t total,
                           int32_t* err_flag, hipStream_t stream) {
    return launch(validate_kernel, dim3(1), dim3(VAL_THREADS), 0, stream, slot_idx, n,
                  num_slots, cu_seqlens, n_cu, total, err_flag);
}

}  // namespace gdn
