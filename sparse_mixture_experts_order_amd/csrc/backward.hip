// Backward of the Switch layer: gradients of  sum_t <dout_t, out_t> + L_aux
// (+ L_z)  with respect to x, W1, W2, W_r and b_r, the choices and capacity
// masks held fixed (argmax has no gradient; the router learns through the
// selected gate).
//
// Sources: "042 Switch Transformer" (wq-win.github.io) sec. 2: the router stays
// differentiable through the selected gate p_e*, and the balance loss is added
// to the training loss; "MoE routing load collapse" (zffjzz.top),
// "troubleshooting": the gradient is checked by central finite differences that
// leave the discrete choices and masks unchanged.
//
// Kernels here (the expert GEMMs reuse expert_gemm):
//   combine_bwd     dy[e, s] = bf16(gate_t dout_t) for kept tokens and
//                   dgate_t = <dout_t, y[e, s]> (fp32), one wave per token
//   transpose_rows  [E][R][S] -> [E][S][Rp] bf16 through 64x64 LDS tiles,
//                   zero for rows >= valid[e] (the token axis of activations)
//   router_wgrad    dW_r partial sums over token slices (fp32), then
//   router_wgrad_reduce  the slices added in order in fp64
//   dx_assemble     dx_t = bf16(dout_t + dbuf[e, s] + sum_e dz_te W_r[:, e])
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

__global__ __launch_bounds__(256) void combine_bwd(const bf16_t* __restrict__ dout, const float* __restrict__ y,
                                                   const int32_t* __restrict__ expert,
                                                   const int32_t* __restrict__ position,
                                                   const uint8_t* __restrict__ keep, const float* __restrict__ gate,
                                                   int64_t T, int d, int E, int C, bf16_t* __restrict__ dy,
                                                   float* __restrict__ dgate) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int e = expert[t], pos = position[t];
    if (!keep[t] || e < 0 || e >= E || pos < 0 || pos >= C) {
        if (lane == 0) dgate[t] = 0.f;
        return;
    }
    const float g = gate[t];
    const bf16_t* drow = dout + t * d;
    const float* yrow = y + ((size_t)e * C + pos) * d;
    bf16_t* dyrow = dy + ((size_t)e * C + pos) * d;
    float acc = 0.f;
    for (int c = lane * 8; c < d; c += 64 * 8) {
        const uint4 dv = *(const uint4*)(drow + c);
        const f32x4 y0 = *(const f32x4*)(yrow + c), y1 = *(const f32x4*)(yrow + c + 4);
        const uint32_t w[4] = {dv.x, dv.y, dv.z, dv.w};
        const float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = bf16_to_f32(w[j] & 0xffffu), hi = bf16_to_f32(w[j] >> 16);
            acc = fmaf(lo, yv[2 * j], acc);
            acc = fmaf(hi, yv[2 * j + 1], acc);
            o[j] = bf16_rne(g * lo) | (bf16_rne(g * hi) << 16);
        }
        *(uint4*)(dyrow + c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    acc = wave_sum(acc);
    if (lane == 0) dgate[t] = acc;
}

// dst[e][c][r] = src[e][r][c] for r < valid (valid[e], or R), else 0; r < Rp.
__global__ __launch_bounds__(256) void transpose_rows(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int R,
                                                     int S, int Rp, const int32_t* __restrict__ valid) {
    __shared__ uint16_t tile[64][66];
    const int e = blockIdx.z;
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int nv = min(valid ? min(max(valid[e], 0), R) : R, R);
    const bf16_t* s = src + (size_t)e * R * S;
    bf16_t* o = dst + (size_t)e * S * Rp;
    // load: 64 rows x 8 vectors of 8 elements
    for (int i = threadIdx.x; i < 512; i += 256) {
        const int r = i >> 3, v = i & 7;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r0 + r < nv) val = *(const uint4*)(s + (size_t)(r0 + r) * S + c0 + v * 8);
        const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tile[r][v * 8 + 2 * j] = (uint16_t)(w[j] & 0xffffu);
            tile[r][v * 8 + 2 * j + 1] = (uint16_t)(w[j] >> 16);
        }
    }
    __syncthreads();
    // store: 64 output rows (columns of src) x 8 vectors of 8 source rows
    for (int i = threadIdx.x; i < 512; i += 256) {
        const int c = i >> 3, v = i & 7;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)tile[v * 8 + 2 * j][c] | ((uint32_t)tile[v * 8 + 2 * j + 1][c] << 16);
        if (r0 + v * 8 < Rp) *(uint4*)(o + (size_t)(c0 + c) * Rp + r0 + v * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// dW_r partial sums: workgroup (i block, e block, slice) adds
// x[t, i] dz[t, e] over the slice's tokens, 64 x 64 outputs, 16 per thread.
constexpr int RW_CHUNK = 32;
__global__ __launch_bounds__(256) void router_wgrad(const bf16_t* __restrict__ x, const float* __restrict__ dz,
                                                    int64_t T, int d, int E, int tps, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) float xs[RW_CHUNK][64];
    __shared__ __attribute__((aligned(16))) float zs[RW_CHUNK][64];
    const int i0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    const int64_t t0 = (int64_t)blockIdx.z * tps;
    const int64_t t1 = min(T, t0 + tps);
    const int ti = threadIdx.x >> 4, te = threadIdx.x & 15;   // 4 i x 4 e per thread
    float acc[4][4] = {};
    for (int64_t tc = t0; tc < t1; tc += RW_CHUNK) {
        __syncthreads();
        for (int q = threadIdx.x; q < RW_CHUNK * 64; q += 256) {
            const int r = q >> 6, c = q & 63;
            const int64_t t = tc + r;
            xs[r][c] = (t < t1 && i0 + c < d) ? bf16_to_f32(x[t * d + i0 + c]) : 0.f;
            zs[r][c] = (t < t1 && e0 + c < E) ? dz[t * E + e0 + c] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int r = 0; r < RW_CHUNK; ++r) {
            const f32x4 xv = *(const f32x4*)&xs[r][ti * 4];
            const f32x4 zv = *(const f32x4*)&zs[r][te * 4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(xv[a], zv[b], acc[a][b]);
        }
    }
    float* p = part + (size_t)blockIdx.z * d * E;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = i0 + ti * 4 + a, e = e0 + te * 4 + b;
            if (i < d && e < E) p[(size_t)i * E + e] = acc[a][b];
        }
}

__global__ __launch_bounds__(256) void router_wgrad_reduce(const float* __restrict__ part, int slices, int64_t n,
                                                           float* __restrict__ dw_r) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    double s = 0.0;
    for (int k = 0; k < slices; ++k) s += (double)part[(size_t)k * n + i];
    dw_r[i] = (float)s;
}

// dx: workgroup = 64 tokens x 64 columns of x, 4 x 4 per thread; K = E in
// chunks of 32.
__global__ __launch_bounds__(256) void dx_assemble(const bf16_t* __restrict__ dout, const float* __restrict__ dbuf,
                                                   const int32_t* __restrict__ expert,
                                                   const int32_t* __restrict__ position,
                                                   const uint8_t* __restrict__ keep, const float* __restrict__ dz,
                                                   const float* __restrict__ w_r, int64_t T, int d, int E, int C,
                                                   bf16_t* __restrict__ dx) {
    __shared__ __attribute__((aligned(16))) float zs[32][68];   // [e][token] (rows padded against bank conflicts)
    __shared__ __attribute__((aligned(16))) float ws[32][68];   // [e][i]
    const int64_t t0 = (int64_t)blockIdx.y * 64;
    const int i0 = blockIdx.x * 64;
    const int tq = threadIdx.x >> 4, iq = threadIdx.x & 15;     // tokens 4 tq.., columns 4 iq..
    float acc[4][4] = {};
    for (int e0 = 0; e0 < E; e0 += 32) {
        __syncthreads();
        for (int q = threadIdx.x; q < 32 * 64; q += 256) {
            const int r = q >> 5, c = q & 31;    // token r, expert c: consecutive threads read consecutive e
            zs[c][r] = (t0 + r < T && e0 + c < E) ? dz[(t0 + r) * E + e0 + c] : 0.f;
            const int ii = q >> 5;               // column ii of x, expert c
            ws[c][ii] = (e0 + c < E) ? w_r[(size_t)(i0 + ii) * E + e0 + c] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int ee = 0; ee < 32; ++ee) {
            const f32x4 zv = *(const f32x4*)&zs[ee][tq * 4];
            const f32x4 wv = *(const f32x4*)&ws[ee][iq * 4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(zv[a], wv[b], acc[a][b]);
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t t = t0 + tq * 4 + a;
        if (t >= T) break;
        const int i = i0 + iq * 4;
        const uint2 dv = *(const uint2*)(dout + t * d + i);
        float v[4] = {bf16_to_f32(dv.x & 0xffffu) + acc[a][0], bf16_to_f32(dv.x >> 16) + acc[a][1],
                      bf16_to_f32(dv.y & 0xffffu) + acc[a][2], bf16_to_f32(dv.y >> 16) + acc[a][3]};
        const int e = expert[t], pos = position[t];
        if (keep[t] && e >= 0 && e < E && pos >= 0 && pos < C) {
            const f32x4 b = *(const f32x4*)(dbuf + ((size_t)e * C + pos) * d + i);
            v[0] += b[0]; v[1] += b[1]; v[2] += b[2]; v[3] += b[3];
        }
        *(uint2*)(dx + t * d + i) = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                               bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
    }
}

__global__ __launch_bounds__(256) void fill_zero(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_combine_bwd(const bf16_t* dout, const float* y, const int32_t* expert, const int32_t* position,
                              const uint8_t* keep, const float* gate, int64_t T, int d, int E, int C, bf16_t* dy,
                              float* dgate, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_bwd, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, dout, y, expert, position, keep,
                       gate, T, d, E, C, dy, dgate);
    return hipGetLastError();
}

hipError_t launch_transpose_rows(const bf16_t* src, bf16_t* dst, int E, int R, int S, int Rp, const int32_t* valid,
                                 hipStream_t s) {
    if (E == 0 || Rp == 0 || S == 0) return hipSuccess;
    const dim3 grid(S / 64, (Rp + 63) / 64, E);
    hipLaunchKernelGGL(transpose_rows, grid, dim3(256), 0, s, src, dst, R, S, Rp, valid);
    return hipGetLastError();
}

int router_wgrad_slices(int64_t T, int d, int E) {
    if (T <= 0) return 0;
    const int64_t by_mem = std::max<int64_t>(1, (int64_t(1) << 24) / ((int64_t)d * E));   // <= 64 MiB of partials
    const int64_t by_tok = (T + 255) / 256;
    return (int)std::min<int64_t>(std::min(by_mem, by_tok), 1024);
}

hipError_t launch_router_wgrad(const bf16_t* x, const float* dz, int64_t T, int d, int E, float* part, float* dw_r,
                               hipStream_t s) {
    const int slices = router_wgrad_slices(T, d, E);
    const int64_t n = (int64_t)d * E;
    if (slices == 0) {   // no tokens: the gradient is zero
        hipLaunchKernelGGL(router_wgrad_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, 0, n, dw_r);
        return hipGetLastError();
    }
    int tps = (int)((T + slices - 1) / slices);
    tps = (tps + RW_CHUNK - 1) / RW_CHUNK * RW_CHUNK;
    const int used = (int)((T + tps - 1) / tps);
    hipLaunchKernelGGL(router_wgrad, dim3((d + 63) / 64, (E + 63) / 64, used), dim3(256), 0, s, x, dz, T, d, E, tps,
                       part);
    hipLaunchKernelGGL(router_wgrad_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, used, n, dw_r);
    return hipGetLastError();
}

hipError_t launch_dx_assemble(const bf16_t* dout, const float* dbuf, const int32_t* expert, const int32_t* position,
                              const uint8_t* keep, const float* dz, const float* w_r, int64_t T, int d, int E, int C,
                              bf16_t* dx, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(dx_assemble, dim3(d / 64, (unsigned)((T + 63) / 64)), dim3(256), 0, s, dout, dbuf, expert,
                       position, keep, dz, w_r, T, d, E, C, dx);
    return hipGetLastError();
}

}  // namespace swmoe
