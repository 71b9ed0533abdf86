// Gate-scaled combine with residual passthrough:
//   out_t = residual_t + keep_t * gate_t * y[e*_t, pos_t]     (fp32, one bf16 rounding)
// Dropped tokens copy residual_t bit for bit (or write zeros without a residual).
//
// Sources: "042 Switch Transformer" (wq-win.github.io) sec. 1: y = p_e* f_e*(x),
// overflow tokens skip the expert branch and continue on the residual; sec. 2:
// the selected probability stays on the output (no renormalisation to 1);
// sec. 3: multiply by the routing probability and put the result back at the
// token's original position, then add the residual.
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

// One thread per 8 consecutive elements of a row: 2 x 16-byte fp32 loads of y,
// one 16-byte bf16 load of the residual, one 16-byte store.
__global__ __launch_bounds__(256) void combine(const float* __restrict__ y, const int32_t* __restrict__ expert,
                                               const int32_t* __restrict__ position,
                                               const uint8_t* __restrict__ keep, const float* __restrict__ gate,
                                               const bf16_t* __restrict__ residual, int64_t T, int d, int E, int C,
                                               bf16_t* __restrict__ out) {
    const int vpr = d >> 3;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T * vpr) return;
    const int64_t t = i / vpr;
    const int v = (int)(i - t * vpr);
    uint4 res = make_uint4(0, 0, 0, 0);
    if (residual) res = ((const uint4*)(residual + t * d))[v];
    const int e = expert[t];
    const int pos = position[t];
    if (!keep[t] || e < 0 || e >= E || pos < 0 || pos >= C) {
        ((uint4*)(out + t * d))[v] = res;
        return;
    }
    const float g = gate[t];
    const float* yr = y + ((size_t)e * C + pos) * d + v * 8;
    const f32x4 y0 = *(const f32x4*)yr, y1 = *(const f32x4*)(yr + 4);
    const uint32_t r[4] = {res.x, res.y, res.z, res.w};
    const float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = fmaf(g, yv[2 * j], bf16_to_f32(r[j] & 0xffffu));
        const float hi = fmaf(g, yv[2 * j + 1], bf16_to_f32(r[j] >> 16));
        o[j] = bf16_rne(lo) | (bf16_rne(hi) << 16);
    }
    ((uint4*)(out + t * d))[v] = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_combine(const float* y, const int32_t* expert, const int32_t* position, const uint8_t* keep,
                          const float* gate, const bf16_t* residual, int64_t T, int d, int E, int C, bf16_t* out,
                          hipStream_t s) {
    const int64_t n = T * (d >> 3);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, expert, position, keep, gate,
                       residual, T, d, E, C, out);
    return hipGetLastError();
}

}  // namespace swmoe
