// gate.hpp -- where the kernels get the per-(token, value head) log-decay g
// and write strength beta: given directly, or by fused gating from the raw
// projections ([P1] RL-Kernel PR #469, "How the golden relates to the kernel",
// item 1): beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias), all in
// fp32, softplus(x) = x above the threshold 20 and log(1 + e^x) at or below it.
// The switch is a workgroup-uniform pointer test, so both forms share one
// kernel instantiation.
#pragma once

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// Raw values at flat index idx = token * HV + hv: (g, beta) when given
// directly, (a, b) for fused gating.
__device__ __forceinline__ void gate_raw(const GateArgs& ga, size_t idx, float& x0, float& x1) {
    if (ga.a) {
        if (ga.ab_bf16) {
            x0 = bf16_to_f32(static_cast<const bf16_t*>(ga.a)[idx]);
            x1 = bf16_to_f32(static_cast<const bf16_t*>(ga.b)[idx]);
        } else {
            x0 = static_cast<const float*>(ga.a)[idx];
            x1 = static_cast<const float*>(ga.b)[idx];
        }
    } else {
        x0 = ga.g[idx];
        x1 = ga.beta[idx];
    }
}

// Per-value-head constants of the fused gating: -exp(A_log[hv]) and
// dt_bias[hv] (zeros when g and beta are given directly).  Loaded once where
// the head is fixed, so the per-token work is only the finish below.
struct GateHead {
    float nexp;
    float dtb;
};

__device__ __forceinline__ GateHead gate_head(const GateArgs& ga, int hv) {
    if (ga.a) return GateHead{-expf(ga.A_log[hv]), ga.dt_bias[hv]};
    return GateHead{0.0f, 0.0f};
}

// (g, beta) from the raw values.  (-e^A) * sp equals -(e^A * sp) bit for bit;
// log1pf keeps softplus accurate where e^x is small (the threshold branch is
// the pages').
__device__ __forceinline__ void gate_finish(const GateArgs& ga, const GateHead& gh, float x0, float x1,
                                            float& g, float& beta) {
    if (ga.a) {
        const float x = x0 + gh.dtb;
        const float sp = (x <= 20.0f) ? log1pf(expf(x)) : x;
        g = gh.nexp * sp;
        beta = 1.0f / (1.0f + expf(-x1));
    } else {
        g = x0;
        beta = x1;
    }
}

}  // namespace gdn
