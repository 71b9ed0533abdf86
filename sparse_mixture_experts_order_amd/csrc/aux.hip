// Load-balancing statistics, aux loss and its gradient with respect to the logits.
//   f_e = counts_e / T,  P_e = prob_sum_e / T,  L = alpha E sum_e f_e P_e
//   dL/dz_tj = (alpha E / T) p_tj (f_j - sum_e f_e p_te),  p_tj = exp(z_tj - lse_t)
//
// Sources: "042 Switch Transformer" (wq-win.github.io) sec. 2: the aux loss,
// f from the hard choice (no gradient), P the differentiable mean probability;
// "MoE routing load collapse" (zffjzz.top), "core idea and formulas": f counts
// the choices before the capacity limit, the gradient flows through P only.
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

// The load-balancing statistics (aux_stats_block) as a kernel of its own.
__global__ __launch_bounds__(1024) void aux_stats(const int32_t* __restrict__ counts,
                                                  const float* __restrict__ prob_sum, int64_t G, int ngroups, int E,
                                                  int k, float alpha, float* __restrict__ f, float* __restrict__ P,
                                                  float* __restrict__ loss) {
    aux_stats_block<1024>(AuxStatsArgs{counts, prob_sum, G, ngroups, E, k, alpha, f, P, loss});
}

// Router z-loss (ST-MoE, as restated in "MoE routing load collapse",
// zffjzz.top, "core idea and formulas"): L_z = beta (1/T) sum_t lse_t^2.
// One workgroup, fp64, fixed tree order.
__global__ __launch_bounds__(1024) void z_loss_reduce(const float* __restrict__ lse, int64_t T, float beta,
                                                      float* __restrict__ z_loss) {
    __shared__ double red[1024];
    double acc = 0.0;
    for (int64_t t = threadIdx.x; t < T; t += 1024) {
        const double l = (double)lse[t];
        acc += l * l;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) z_loss[0] = T > 0 ? (float)((double)beta * red[0] / (double)T) : 0.f;
}

// Gradient with respect to the logits of  c_aux-weighted aux loss and
// c_z-weighted z-loss, with p_tj = exp(z_tj - lse_t):
//   G_tj = p_tj * (c_aux (f_j - sum_e f_e p_te) + c_z lse_t)
// c_aux = alpha E / T (aux, f held constant; f is the row of the token's
// routing group of G tokens), c_z = 2 beta / T (z-loss).
// With dgate (the layer backward) the task gradient through the selected
// gates is added:  + sum_i dgate_ti gate_ti (delta_{j e_ti} - p_tj) over the
// token's k choices  (d p_te / d z_tj = p_te (delta_ej - p_tj)); expert, gate
// and dgate are [T, k].
// One wave per token row; lane j holds experts j, j+64, ...  With
// `accumulate` the result is added to dlogits instead of stored.
template <int NCH>
__global__ __launch_bounds__(256) void aux_grad(const float* __restrict__ logits, const float* __restrict__ lse,
                                                const float* __restrict__ f, int64_t T, int64_t G, int E, float c_aux,
                                                float c_z, const int32_t* __restrict__ expert,
                                                const float* __restrict__ gate, const float* __restrict__ dgate,
                                                int k, int accumulate, float* __restrict__ dlogits) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    if (f) f += (t / G) * E;
    const float* row = logits + t * E;
    const float l = lse[t];
    float p[NCH], fr[NCH];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int e = lane + 64 * i;
        p[i] = e < E ? expf(row[e] - l) : 0.f;
        fr[i] = (e < E && f) ? f[e] : 0.f;
        s = fmaf(fr[i], p[i], s);
    }
    s = wave_sum(s);
    const float zt = c_z * l;
    // the gate terms: dg_i = dgate_ti gate_ti of choice i, and their sum
    float dgi[kMaxTopK];
    int es[kMaxTopK];
    float dg = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxTopK; ++c) {
        const bool on = dgate && c < k;
        dgi[c] = on ? dgate[t * k + c] * gate[t * k + c] : 0.f;
        es[c] = on ? expert[t * k + c] : -1;
        dg += dgi[c];
    }
    float* g = dlogits + t * E;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            float sel = 0.f;
#pragma unroll
            for (int c = 0; c < kMaxTopK; ++c) sel += e == es[c] ? dgi[c] : 0.f;
            const float v = p[i] * (c_aux * (fr[i] - s) + zt - dg) + sel;
            g[e] = accumulate ? g[e] + v : v;
        }
    }
}

// The same gradient for E a multiple of 4 with 16-byte aligned rows: L lanes
// per token (E / 4 rounded up to a power of two, at most 64), so a wave
// finishes 64 / L tokens; lane s of a token holds experts 4 (s + L i) .. + 3,
// i < NV, and moves them with 16-byte loads and stores.  All of a token's
// loads are issued before the first is used.
template <int L, int NV>
__global__ __launch_bounds__(256) void aux_grad4(const float* __restrict__ logits, const float* __restrict__ lse,
                                                 const float* __restrict__ f, int64_t T, int64_t G, int E,
                                                 float c_aux, float c_z, const int32_t* __restrict__ expert,
                                                 const float* __restrict__ gate, const float* __restrict__ dgate,
                                                 int k, int accumulate, float* __restrict__ dlogits) {
    constexpr int TPW = 64 / L;
    const int lane = threadIdx.x & 63, sub = lane % L;
    const int64_t t = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW + lane / L;
    if (t >= T) return;   // whole groups of L lanes (one token) leave together
    const float* row = logits + t * E;
    const float* fr = f ? f + (t / G) * E : nullptr;
    float* g = dlogits + t * E;
    f32x4 z[NV], fv[NV], acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e0 = 4 * (sub + L * i);
        const bool in = e0 < E;
        z[i] = in ? *(const f32x4*)(row + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
        fv[i] = (in && fr) ? *(const f32x4*)(fr + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
        acc[i] = (in && accumulate) ? *(const f32x4*)(g + e0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float l = lse[t];
    float dgi[kMaxTopK];
    int es[kMaxTopK];
    float dg = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxTopK; ++c) {
        const bool on = dgate && c < k;
        dgi[c] = on ? dgate[t * k + c] * gate[t * k + c] : 0.f;
        es[c] = on ? expert[t * k + c] : -1;
        dg += dgi[c];
    }
    float p[NV][4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * (sub + L * i) + j;
            p[i][j] = e < E ? expf(z[i][j] - l) : 0.f;
            s = fmaf(fv[i][j], p[i][j], s);
        }
#pragma unroll
    for (int m = L / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    const float zt = c_z * l;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e0 = 4 * (sub + L * i);
        if (e0 < E) {
            f32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float sel = 0.f;
#pragma unroll
                for (int c = 0; c < kMaxTopK; ++c) sel += e0 + j == es[c] ? dgi[c] : 0.f;
                o[j] = p[i][j] * (c_aux * (fv[i][j] - s) + zt - dg) + sel;
            }
            *(f32x4*)(g + e0) = accumulate ? acc[i] + o : o;
        }
    }
}

hipError_t launch_aux_stats(const int32_t* counts, const float* prob_sum, int64_t G, int ngroups, int E, int k,
                            float alpha, float* f, float* P, float* loss, hipStream_t s) {
    hipLaunchKernelGGL(aux_stats, dim3(1), dim3(1024), 0, s, counts, prob_sum, G, ngroups, E, k, alpha, f, P, loss);
    return hipGetLastError();
}

hipError_t launch_z_loss(const float* lse, int64_t T, float beta, float* z_loss, hipStream_t s) {
    hipLaunchKernelGGL(z_loss_reduce, dim3(1), dim3(1024), 0, s, lse, T, beta, z_loss);
    return hipGetLastError();
}

hipError_t launch_aux_grad(const float* logits, const float* lse, const float* f, int64_t T, int64_t G, int E,
                           float alpha, float beta, const int32_t* expert, const float* gate, const float* dgate,
                           int k, int accumulate, float* dlogits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const float c_aux = f ? (float)((double)alpha * (double)E / (double)T) : 0.f;
    const float c_z = (float)(2.0 * (double)beta / (double)T);
    const int64_t Gc = std::max<int64_t>(G, 1);
    if (E % 4 == 0 && ((uintptr_t)logits | (uintptr_t)dlogits | (uintptr_t)f) % 16 == 0) {
        int lanes = 1;
        while (lanes < 64 && 4 * lanes < E) lanes <<= 1;
        const int64_t waves = (T + 64 / lanes - 1) / (64 / lanes);
        const dim3 g4((unsigned)((waves + 3) / 4));
#define SWMOE_GRAD4(L, NV)                                                                                     \
    hipLaunchKernelGGL((aux_grad4<L, NV>), g4, dim3(256), 0, s, logits, lse, f, T, Gc, E, c_aux, c_z, expert, gate, \
                       dgate, k, accumulate, dlogits)
        if (lanes < 64) {
            switch (lanes) {
                case 1: SWMOE_GRAD4(1, 1); break;
                case 2: SWMOE_GRAD4(2, 1); break;
                case 4: SWMOE_GRAD4(4, 1); break;
                case 8: SWMOE_GRAD4(8, 1); break;
                case 16: SWMOE_GRAD4(16, 1); break;
                default: SWMOE_GRAD4(32, 1); break;
            }
        } else {
            const int nv = (E + 255) / 256;
            if (nv <= 1) SWMOE_GRAD4(64, 1);
            else if (nv <= 2) SWMOE_GRAD4(64, 2);
            else if (nv <= 4) SWMOE_GRAD4(64, 4);
            else if (nv <= 8) SWMOE_GRAD4(64, 8);
            else SWMOE_GRAD4(64, 16);
        }
#undef SWMOE_GRAD4
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)((T + 3) / 4);
    const int nch = (E + 63) / 64;
#define SWMOE_GRAD(N)                                                                                          \
    hipLaunchKernelGGL(aux_grad<N>, dim3(grid), dim3(256), 0, s, logits, lse, f, T, std::max<int64_t>(G, 1), E, \
                       c_aux, c_z, expert, gate, dgate, k, accumulate, dlogits)
    if (nch <= 1) SWMOE_GRAD(1);
    else if (nch <= 2) SWMOE_GRAD(2);
    else if (nch <= 4) SWMOE_GRAD(4);
    else if (nch <= 8) SWMOE_GRAD(8);
    else if (nch <= 16) SWMOE_GRAD(16);
    else if (nch <= 32) SWMOE_GRAD(32);
    else SWMOE_GRAD(64);
#undef SWMOE_GRAD
    return hipGetLastError();
}

}  // namespace swmoe
