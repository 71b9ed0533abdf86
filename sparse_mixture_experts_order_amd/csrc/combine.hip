// Gate-scaled combine with residual passthrough:
//   out_t = residual_t + sum_i keep_ti * gate_ti * y[e_ti, slot_ti]   (fp32, one bf16 rounding)
// (k = 1 for the Switch layer).  Tokens with every choice dropped copy
// residual_t bit for bit (or write zeros without a residual).
//
// Sources: "042 Switch Transformer" (wq-win.github.io) sec. 1: y = p_e* f_e*(x),
// overflow tokens skip the expert branch and continue on the residual; sec. 2:
// the selected probability stays on the output (no renormalisation to 1);
// sec. 3: multiply by the routing probability and put the result back at the
// token's original position, then add the residual.
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

// One thread per 8 consecutive elements of a row: one 16-byte bf16 load of the
// residual, 2 x 16-byte fp32 loads of y per kept choice, one 16-byte store.
// The k choices of a token are added in rank order into the fp32 residual,
// then rounded once.  `slot` indexes the expert's buffer rows (the position
// itself when there is one routing group).  KC = k at compile time (1, the
// Switch layer), or 0 for a run-time k.
template <int KC>
__global__ __launch_bounds__(256) void combine(const float* __restrict__ y, const int32_t* __restrict__ expert,
                                               const int32_t* __restrict__ slot,
                                               const uint8_t* __restrict__ keep, const float* __restrict__ gate,
                                               const bf16_t* __restrict__ residual, int64_t T, int d, int E, int kr,
                                               int C, bf16_t* __restrict__ out) {
    const int k = KC > 0 ? KC : kr;
    const int vpr = d >> 3;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T * vpr) return;
    const int64_t t = i / vpr;
    const int v = (int)(i - t * vpr);
    uint4 res = make_uint4(0, 0, 0, 0);
    if (residual) res = ((const uint4*)(residual + t * d))[v];
    const uint32_t r[4] = {res.x, res.y, res.z, res.w};
    float acc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[2 * j] = bf16_to_f32(r[j] & 0xffffu);
        acc[2 * j + 1] = bf16_to_f32(r[j] >> 16);
    }
    bool any = false;
    for (int c = 0; c < k; ++c) {
        const int64_t o = t * k + c;
        const int e = expert[o];
        const int pos = slot[o];
        if (!keep[o] || e < 0 || e >= E || pos < 0 || pos >= C) continue;
        const float g = gate[o];
        const float* yr = y + ((size_t)e * C + pos) * d + v * 8;
        const f32x4 y0 = *(const f32x4*)yr, y1 = *(const f32x4*)(yr + 4);
        const float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(g, yv[j], acc[j]);
        any = true;
    }
    if (!any) {   // every choice dropped: the residual passes through bit for bit
        ((uint4*)(out + t * d))[v] = res;
        return;
    }
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
    ((uint4*)(out + t * d))[v] = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_combine(const float* y, const int32_t* expert, const int32_t* slot, const uint8_t* keep,
                          const float* gate, const bf16_t* residual, int64_t T, int d, int E, int k, int C,
                          bf16_t* out, hipStream_t s) {
    const int64_t n = T * (d >> 3);
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (k == 1)
        hipLaunchKernelGGL(combine<1>, grid, dim3(256), 0, s, y, expert, slot, keep, gate, residual, T, d, E, k, C,
                           out);
    else
        hipLaunchKernelGGL(combine<0>, grid, dim3(256), 0, s, y, expert, slot, keep, gate, residual, T, d, E, k, C,
                           out);
    return hipGetLastError();
}

}  // namespace swmoe
