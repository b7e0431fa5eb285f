// geglu_bwd.h -- the GeGLU backward's per-element arithmetic, applied in the
// epilogue of the NT GEMM that computes dh_raw = dy W_down^T (gemm_bw.hip).
#pragma once

#include "common.h"

namespace moe {

// Phi(v) and phi(v) (standard normal CDF and density) in fp32: Phi through
// the complementary error function of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7), whose
// exp(-z^2) = exp(-v^2 / 2) also gives the density.
__device__ __forceinline__ void normal_cdf_pdf(float v, float& Phi, float& phi) {
    const float z = fabsf(v) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float p = fmaf(t, 1.061405429f, -1.453152027f);
    p = fmaf(t, p, 1.421413741f);
    p = fmaf(t, p, -0.284496736f);
    p = fmaf(t, p, 0.254829592f);
    const float ez = __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);
    const float half_erfc = 0.5f * t * p * ez;
    Phi = v >= 0.0f ? 1.0f - half_erfc : half_erfc;
    phi = ez * 0.39894228040143267794f;   // 1 / sqrt(2 pi)
}

// GeGLU backward of one element: g, u the pre-activations, dh_raw = dy W_down^T
// (before the gate), gt the gate.  h = GELU(g) u; outputs dg, du, gate h and
// the term h dh_raw of dgate.
__device__ __forceinline__ void geglu_bwd_elem(float g, float u, float dh_raw, float gt, float& dg,
                                               float& du, float& gh, float& dot_term) {
    float Phi, phi;
    normal_cdf_pdf(g, Phi, phi);
    const float a = g * Phi;
    const float h = a * u;
    dot_term = h * dh_raw;
    const float dh = gt * dh_raw;
    du = dh * a;
    dg = dh * u * fmaf(g, phi, Phi);
    gh = gt * h;
}

}  // namespace moe
