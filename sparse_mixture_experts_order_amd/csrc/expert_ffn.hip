// Grouped expert GEMM on bf16 MFMA (v_mfma_f32_32x32x16_bf16), used twice:
//   H[e, s, :] = bf16(ReLU(buf[e, s, :] W1_e^T))     (N = d_ff, K = d)
//   Y[e, s, :] = H[e, s, :] W2_e^T                   (N = d,    K = d_ff), fp32
// for rows s < accepted[e]; the row counts are read on the device, so the
// grid covers every possible tile and tiles past accepted[e] return at once.
//
// Sources: "Switch Transformers ..." essay (dmxsf.com), "core structure":
// experts replace the FFN sublayer; "Mixture of experts" (world.lapla.si),
// "what is inside an expert": d -> d_ff with negatives set to zero -> d.
//
// Design for one MI355X.  At Switch-Base shapes an expert sees ~120 rows, so
// the layer is bound by streaming every expert's weights from HBM once, not
// by MFMA.  The kernel is organised around that stream:
//   - a workgroup (4 waves) owns TOK = 32*TOKB rows of one expert and
//     NWG = 4*32*NBW weight rows; each wave owns 32*NBW weight rows and
//     computes them against all TOK rows (weights = MFMA A operand, tokens =
//     MFMA B operand, so a lane's results are 4 consecutive outputs of one row);
//   - weights never touch LDS: each lane loads 64 contiguous bytes of its
//     weight row per 64-wide K chunk straight into registers, one chunk ahead
//     of the MFMAs.  The K order inside a chunk is permuted identically for
//     both operands (a reduction is order free), so the 32 lanes of a half
//     wave read whole 64-byte runs;
//   - the token tile is shared by the 4 waves through LDS, double buffered,
//     rows padded to 144 bytes so the MFMA-layout reads are conflict free;
//   - tile ids are dealt XCD-major so the tiles of one expert share an L2.
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

constexpr int FFN_LDS_STRIDE = 72;  // bf16 elements per LDS row (64 + 8 pad)

template <int TOKB, int NBW, bool GEMM1>
__global__ __launch_bounds__(256) void expert_gemm(const bf16_t* __restrict__ A,   // [E, C, K]
                                                   const bf16_t* __restrict__ W,   // [E, N, K]
                                                   const int32_t* __restrict__ accepted,
                                                   void* __restrict__ out,         // [E, C, N]
                                                   int C, int K, int N, int n_tiles, int tok_tiles,
                                                   int ntiles, int grid_padded) {
    constexpr int TOK = 32 * TOKB;
    constexpr int NWG = 4 * 32 * NBW;
    __shared__ __attribute__((aligned(16))) bf16_t lds[2][TOK * FFN_LDS_STRIDE];

    const int tile = xcd_swizzle(blockIdx.x, grid_padded);
    if (tile >= ntiles) return;
    const int tt = tile % tok_tiles;
    const int rest = tile / tok_tiles;
    const int nt = rest % n_tiles;
    const int e = rest / n_tiles;
    const int tok_base = tt * TOK;
    const int acc_e = min(max(accepted[e], 0), C);  // rows in use, never past the capacity
    if (tok_base >= acc_e) return;
    const int nv = min(TOK, acc_e - tok_base);  // valid rows in this tile
    const int nvb = (nv + 31) >> 5;             // valid 32-row blocks

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int wrow0 = nt * NWG + wave * 32 * NBW;
    const bool wave_active = wrow0 < N;

    const bf16_t* Ae = A + ((size_t)e * C + tok_base) * K;
    const bf16_t* wptr[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        const int r = wave_active ? wrow0 + nb * 32 + l32 : 0;
        wptr[nb] = W + ((size_t)e * N + r) * K + half * 32;
    }

    // token tile staging: thread -> (row = tid/8 + 32*j, 16-byte column tid%8)
    const int srow = threadIdx.x >> 3, scol = (threadIdx.x & 7) * 8;
    uint4 areg[TOKB];
    auto load_a = [&](int kc) {
#pragma unroll
        for (int j = 0; j < TOKB; ++j) {
            const int r = srow + 32 * j;
            if (r < nv) areg[j] = *(const uint4*)(Ae + (size_t)r * K + kc * 64 + scol);
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < TOKB; ++j) {
            const int r = srow + 32 * j;
            if (r < nv) *(uint4*)(&lds[buf][r * FFN_LDS_STRIDE + scol]) = areg[j];
        }
    };

    uint4 wreg[2][NBW][4];
    auto load_w = [&](int kc, int buf) {
        if (!wave_active) return;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) wreg[buf][nb][j] = *(const uint4*)(wptr[nb] + kc * 64 + j * 8);
    };

    f32x16 acc[NBW][TOKB];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;

    auto compute = [&](int buf) {
        if (!wave_active) return;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 bt[TOKB];
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb)
                if (tb < nvb)
                    bt[tb] = as_bf16x8(*(const uint4*)(&lds[buf][(tb * 32 + l32) * FFN_LDS_STRIDE + half * 32 + s * 8]));
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const bf16x8 wa = as_bf16x8(wreg[buf][nb][s]);
#pragma unroll
                for (int tb = 0; tb < TOKB; ++tb)
                    if (tb < nvb) acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt[tb], acc[nb][tb], 0, 0, 0);
            }
        }
    };

    const int nk = K >> 6;
    load_a(0);
    load_w(0, 0);
    store_a(0);
    for (int kc = 0; kc < nk; kc += 2) {
        // even step: compute chunk kc from buffers 0
        if (kc + 1 < nk) { load_a(kc + 1); load_w(kc + 1, 1); }
        __syncthreads();
        compute(0);
        if (kc + 1 < nk) store_a(1);
        if (kc + 1 >= nk) break;
        // odd step: compute chunk kc+1 from buffers 1
        if (kc + 2 < nk) { load_a(kc + 2); load_w(kc + 2, 0); }
        __syncthreads();
        compute(1);
        if (kc + 2 < nk) store_a(0);
    }

    if (!wave_active) return;
    // lane holds token column l32 of block tb and weight rows 8*(i/4) + 4*half + i%4
#pragma unroll
    for (int tb = 0; tb < TOKB; ++tb) {
        const int r = tb * 32 + l32;
        if (r >= nv) continue;
        const size_t orow = ((size_t)e * C + tok_base + r) * N;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = wrow0 + nb * 32 + q * 8 + half * 4;
                const f32x16& a = acc[nb][tb];
                if constexpr (GEMM1) {
                    const uint32_t b0 = bf16_rne(fmaxf(a[4 * q + 0], 0.f)), b1 = bf16_rne(fmaxf(a[4 * q + 1], 0.f));
                    const uint32_t b2 = bf16_rne(fmaxf(a[4 * q + 2], 0.f)), b3 = bf16_rne(fmaxf(a[4 * q + 3], 0.f));
                    *(uint2*)((bf16_t*)out + orow + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                } else {
                    *(f32x4*)((float*)out + orow + n) = f32x4{a[4 * q + 0], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                }
            }
    }
}

// ------------------------------------------------------------------ launchers
template <int TOKB, int NBW, bool GEMM1>
static hipError_t launch_expert_gemm_t(const bf16_t* A, const bf16_t* W, const int32_t* accepted, void* out,
                                       int E, int C, int K, int N, hipStream_t s) {
    constexpr int TOK = 32 * TOKB, NWG = 128 * NBW;
    const int n_tiles = (N + NWG - 1) / NWG;
    const int tok_tiles = (C + TOK - 1) / TOK;
    const int64_t ntiles = (int64_t)E * n_tiles * tok_tiles;
    if (ntiles == 0) return hipSuccess;
    const int64_t grid = (ntiles + 7) / 8 * 8;
    hipLaunchKernelGGL((expert_gemm<TOKB, NBW, GEMM1>), dim3((unsigned)grid), dim3(256), 0, s, A, W, accepted,
                       out, C, K, N, n_tiles, tok_tiles, (int)ntiles, (int)grid);
    return hipGetLastError();
}

template <bool GEMM1>
static hipError_t launch_expert_gemm(const bf16_t* A, const bf16_t* W, const int32_t* accepted, void* out, int E,
                                     int C, int K, int N, hipStream_t s) {
    // rows per tile: enough 32-row blocks for the capacity, at most 8
    if (C > 128) return launch_expert_gemm_t<8, 1, GEMM1>(A, W, accepted, out, E, C, K, N, s);
    if (C > 64) return launch_expert_gemm_t<4, 1, GEMM1>(A, W, accepted, out, E, C, K, N, s);
    if (C > 32) return launch_expert_gemm_t<2, 2, GEMM1>(A, W, accepted, out, E, C, K, N, s);
    return launch_expert_gemm_t<1, 2, GEMM1>(A, W, accepted, out, E, C, K, N, s);
}

hipError_t launch_expert_gemm1(const bf16_t* buf, const bf16_t* w1, const int32_t* accepted, bf16_t* h, int E,
                               int C, int d, int d_ff, hipStream_t s) {
    return launch_expert_gemm<true>(buf, w1, accepted, h, E, C, d, d_ff, s);
}

hipError_t launch_expert_gemm2(const bf16_t* h, const bf16_t* w2, const int32_t* accepted, float* y, int E, int C,
                               int d, int d_ff, hipStream_t s) {
    return launch_expert_gemm<false>(h, w2, accepted, y, E, C, d_ff, d, s);
}

}  // namespace swmoe
