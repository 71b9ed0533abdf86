// Router: logits z = x W_r + b_r (fp32-accurate on bf16 MFMA), then
// softmax / top-1 / log-sum-exp per token and the per-expert probability sums.
//
// Sources: "042 Switch Transformer" (wq-win.github.io) sec. 1, p = softmax(W_r x)
// and e* = argmax p; sec. 2, the router alone runs in float32; "MoE routing
// load collapse" (zffjzz.top), "core idea and formulas": Z = XW, ties go to the
// first index.
//
// fp32 accuracy on bf16 MFMA: every fp32 router weight w is split into three
// bf16 terms w = hi + mid + lo (hi = bf16(w), mid = bf16(w - hi),
// lo = bf16(w - hi - mid); each subtraction is exact in fp32 and the three
// terms hold all 24 significand bits).  x is bf16, so each product x*term is
// exact in fp32 and the MFMA accumulates the three partial GEMMs in fp32
// (the three-term bf16 split of Henry, Tang and Heinecke, ARITH 2019).
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

// w_r [d, E] fp32 -> wr3 [3][E][d] bf16 (expert-major so that an MFMA operand
// row -- one expert, 8 consecutive k -- is 16 contiguous bytes).
__global__ __launch_bounds__(256) void split_router_weights(const float* __restrict__ w_r,
                                                            bf16_t* __restrict__ wr3, int d, int E) {
    __shared__ float tile[32][33];
    const int e0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int r = ty; r < 32; r += 8) {
        int k = k0 + r, e = e0 + tx;
        tile[r][tx] = (k < d && e < E) ? w_r[(size_t)k * E + e] : 0.f;
    }
    __syncthreads();
    const size_t plane = (size_t)E * d;
    for (int r = ty; r < 32; r += 8) {
        int e = e0 + r, k = k0 + tx;
        if (e < E && k < d) {
            float w = tile[tx][r];
            uint32_t hi = bf16_rne(w);
            float r1 = w - bf16_to_f32(hi);
            uint32_t mid = bf16_rne(r1);
            float r2 = r1 - bf16_to_f32(mid);
            uint32_t lo = bf16_rne(r2);
            size_t o = (size_t)e * d + k;
            wr3[o] = (bf16_t)hi;
            wr3[plane + o] = (bf16_t)mid;
            wr3[2 * plane + o] = (bf16_t)lo;
        }
    }
}

// logits[t, e] = sum_k x[t, k] (hi + mid + lo)[e, k] + b[e].
// v_mfma_f32_16x16x32_bf16 with rows = experts (A operand, from wr3) and
// columns = tokens (B operand, from x).  A wave owns RT_TB token blocks x
// RT_EB expert blocks of 16; a workgroup of 4 waves covers 4*16*RT_TB tokens
// and 16*RT_EB experts.  Operands are loaded straight from global memory
// (x once per wave; the split weights are shared through L2).
constexpr int RT_TB = 2, RT_EB = 4;

__global__ __launch_bounds__(256) void router_gemm(const bf16_t* __restrict__ x,
                                                   const bf16_t* __restrict__ wr3,
                                                   const float* __restrict__ b_r,
                                                   float* __restrict__ logits, int T, int d, int E) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t_base = (blockIdx.x * 4 + wave) * (16 * RT_TB);
    const int e_base = blockIdx.y * (16 * RT_EB);
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    const size_t plane = (size_t)E * d;

    const bf16_t* xrow[RT_TB];
#pragma unroll
    for (int tb = 0; tb < RT_TB; ++tb) {
        int t = min(t_base + tb * 16 + r16, T - 1);
        xrow[tb] = x + (size_t)t * d + kq;
    }
    const bf16_t* wrow[RT_EB];
#pragma unroll
    for (int eb = 0; eb < RT_EB; ++eb) {
        int e = min(e_base + eb * 16 + r16, E - 1);
        wrow[eb] = wr3 + (size_t)e * d + kq;
    }
    f32x4 acc[RT_TB][RT_EB];
#pragma unroll
    for (int tb = 0; tb < RT_TB; ++tb)
#pragma unroll
        for (int eb = 0; eb < RT_EB; ++eb) acc[tb][eb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < d; k0 += 32) {
        bf16x8 xb[RT_TB];
#pragma unroll
        for (int tb = 0; tb < RT_TB; ++tb) xb[tb] = as_bf16x8(*(const uint4*)(xrow[tb] + k0));
        bf16x8 wa[3][RT_EB];
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int eb = 0; eb < RT_EB; ++eb)
                wa[j][eb] = as_bf16x8(*(const uint4*)(wrow[eb] + (2 - j) * plane + k0));
        // small terms first: lo, mid, hi
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int tb = 0; tb < RT_TB; ++tb)
#pragma unroll
                for (int eb = 0; eb < RT_EB; ++eb)
                    acc[tb][eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[j][eb], xb[tb], acc[tb][eb], 0, 0, 0);
    }
    // lane holds token column (lane & 15) and expert rows 4*(lane>>4) + 0..3
#pragma unroll
    for (int tb = 0; tb < RT_TB; ++tb) {
        int t = t_base + tb * 16 + r16;
        if (t >= T) continue;
#pragma unroll
        for (int eb = 0; eb < RT_EB; ++eb) {
            int e = e_base + eb * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (e + i < E) logits[(size_t)t * E + e + i] = acc[tb][eb][i] + (b_r ? b_r[e + i] : 0.f);
        }
    }
}

// Softmax statistics per token.  A workgroup (4 waves) owns `tpb` consecutive
// tokens; a wave handles one token at a time with lane j holding experts
// j, j+64, ...  Writes expert, gate, lse and the workgroup's partial sums of
// p_te over its tokens (fixed order: lanes in registers, waves in turn).
template <int NCH>
__global__ __launch_bounds__(256) void router_softmax(const float* __restrict__ logits, int T, int E,
                                                      int tpb, int32_t* __restrict__ expert,
                                                      float* __restrict__ gate, float* __restrict__ lse,
                                                      float* __restrict__ part) {
    extern __shared__ float red[];  // [E]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * tpb, t1 = min(T, t0 + tpb);
    float acc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) acc[i] = 0.f;

    for (int t = t0 + wave; t < t1; t += 4) {
        const float* row = logits + (size_t)t * E;
        float v[NCH];
        float m = -INFINITY;
        int mi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            int e = lane + 64 * i;
            v[i] = e < E ? row[e] : -INFINITY;
            if (v[i] > m) { m = v[i]; mi = e; }   // strict: first (lowest) index per lane
        }
        wave_argmax(m, mi);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            v[i] = (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
            s += v[i];
        }
        s = wave_sum(s);
        const float inv = 1.0f / s;
#pragma unroll
        for (int i = 0; i < NCH; ++i) acc[i] += v[i] * inv;
        if (lane == 0) {
            expert[t] = mi;
            gate[t] = inv;           // p_{e*} = exp(z_e* - m) / s = 1 / s
            lse[t] = m + logf(s);
        }
    }
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                int e = lane + 64 * i;
                if (e < E) red[e] = (w == 0) ? acc[i] : red[e] + acc[i];
            }
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < E; e += 256) part[(size_t)blockIdx.x * E + e] = red[e];
}

// prob_sum[e] = sum over workgroups of the partial sums, in fp64, in a fixed
// order: a workgroup owns 64 experts; its 16 row groups take every 16th
// partial row, then the row groups are added in order.
__global__ __launch_bounds__(1024) void router_reduce(const float* __restrict__ part, int nblk, int E,
                                                      float* __restrict__ prob_sum) {
    __shared__ double red[16][64];
    const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + c;
    double s = 0.0;
    if (e < E) {
        int b = rg;
        for (; b + 48 < nblk; b += 64) {
            const float v0 = part[(size_t)b * E + e], v1 = part[(size_t)(b + 16) * E + e];
            const float v2 = part[(size_t)(b + 32) * E + e], v3 = part[(size_t)(b + 48) * E + e];
            s += (double)v0;
            s += (double)v1;
            s += (double)v2;
            s += (double)v3;
        }
        for (; b < nblk; b += 16) s += (double)part[(size_t)b * E + e];
    }
    red[rg][c] = s;
    __syncthreads();
    if (rg == 0 && e < E) {
        double t = 0.0;
        for (int r = 0; r < 16; ++r) t += red[r][c];
        prob_sum[e] = (float)t;
    }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_split_router_weights(const float* w_r, bf16_t* wr3, int d, int E, hipStream_t s) {
    dim3 grid((E + 31) / 32, (d + 31) / 32);
    hipLaunchKernelGGL(split_router_weights, grid, dim3(256), 0, s, w_r, wr3, d, E);
    return hipGetLastError();
}

hipError_t launch_router_gemm(const bf16_t* x, const bf16_t* wr3, const float* b_r, float* logits,
                              int T, int d, int E, hipStream_t s) {
    dim3 grid((T + 64 * RT_TB - 1) / (64 * RT_TB), (E + 16 * RT_EB - 1) / (16 * RT_EB));
    hipLaunchKernelGGL(router_gemm, grid, dim3(256), 0, s, x, wr3, b_r, logits, T, d, E);
    return hipGetLastError();
}

int router_softmax_blocks(int64_t T, int E) {
    if (T <= 0) return 0;
    // about 64 tokens per workgroup, at most 4 MiB of partial sums
    int64_t nblk = std::min<int64_t>((T + 63) / 64, std::max<int64_t>(1, (int64_t(1) << 20) / E));
    int64_t tpb = (T + nblk - 1) / nblk;
    return (int)((T + tpb - 1) / tpb);
}

hipError_t launch_router_softmax(const float* logits, int T, int E, int32_t* expert, float* gate,
                                 float* lse, float* part, hipStream_t s) {
    int nblk = router_softmax_blocks(T, E);
    int tpb = (T + nblk - 1) / nblk;
    size_t shm = (size_t)E * sizeof(float);
    int nch = (E + 63) / 64;
#define SWMOE_SOFTMAX(N)                                                                          \
    hipLaunchKernelGGL(router_softmax<N>, dim3(nblk), dim3(256), shm, s, logits, T, E, tpb, expert, \
                       gate, lse, part)
    if (nch <= 1) SWMOE_SOFTMAX(1);
    else if (nch <= 2) SWMOE_SOFTMAX(2);
    else if (nch <= 4) SWMOE_SOFTMAX(4);
    else if (nch <= 8) SWMOE_SOFTMAX(8);
    else if (nch <= 16) SWMOE_SOFTMAX(16);
    else if (nch <= 32) SWMOE_SOFTMAX(32);
    else SWMOE_SOFTMAX(64);
#undef SWMOE_SOFTMAX
    return hipGetLastError();
}

hipError_t launch_router_reduce(const float* part, int nblk, int E, float* prob_sum, hipStream_t s) {
    hipLaunchKernelGGL(router_reduce, dim3((E + 63) / 64), dim3(1024), 0, s, part, nblk, E, prob_sum);
    return hipGetLastError();
}

}  // namespace swmoe
