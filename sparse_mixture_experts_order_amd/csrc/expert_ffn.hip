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

#include <type_traits>

namespace swmoe {

constexpr int FFN_LDS_STRIDE = 72;  // bf16 elements per LDS row (64 + 8 pad)

// TOKB: 32-row token blocks per tile; NBW: 32-row weight blocks per wave;
// WAVES: waves per workgroup; R: depth of the register rings (R-1 chunks of
// 64 K-elements in flight ahead of the MFMAs).
template <int TOKB, int NBW, int WAVES, int R, bool GEMM1>
__global__ __launch_bounds__(64 * WAVES) void expert_gemm(const bf16_t* __restrict__ A,   // [E, C, K]
                                                          const bf16_t* __restrict__ W,   // [E, N, K]
                                                          const int32_t* __restrict__ accepted,
                                                          void* __restrict__ out,         // [E, C, N]
                                                          int C, int K, int N, int n_tiles, int tok_tiles,
                                                          int ntiles, int grid_padded) {
    constexpr int TOK = 32 * TOKB;
    constexpr int NWG = WAVES * 32 * NBW;
    constexpr int NTHR = 64 * WAVES;
    constexpr int PIECES = TOK * 8;                       // 16-byte pieces of one token chunk
    constexpr int APT = (PIECES + NTHR - 1) / NTHR;       // pieces per thread
    // output staging after the K loop reuses the same LDS: TOK rows of NWG
    // values (bf16 for GEMM1, fp32 for GEMM2), rows padded by 16 bytes
    constexpr int OUT_BYTES = GEMM1 ? 2 : 4;
    constexpr int OSTRIDE = NWG * OUT_BYTES + 16;                     // bytes per staged row
    constexpr int A_BYTES = 2 * TOK * FFN_LDS_STRIDE * 2;
    constexpr int LDS_BYTES = A_BYTES > TOK * OSTRIDE ? A_BYTES : TOK * OSTRIDE;
    __shared__ __attribute__((aligned(16))) char lds_raw[LDS_BYTES];
    bf16_t (*lds)[TOK * FFN_LDS_STRIDE] = reinterpret_cast<bf16_t (*)[TOK * FFN_LDS_STRIDE]>(lds_raw);

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

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int half = lane >> 5, l32 = lane & 31;
    const int wrow0 = nt * NWG + wave * 32 * NBW;
    const bool wave_active = wrow0 < N;

    // Weight rows: lane l reads row wrow0 + 32*nb + l%32, 64 contiguous bytes
    // per chunk (its half of the 128-byte chunk).  Waves past the last row
    // read row 0 and store nothing.
    const bf16_t* wptr[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        const int r = wave_active ? wrow0 + nb * 32 + l32 : 0;
        wptr[nb] = W + ((size_t)e * N + r) * K + half * 32;
    }

    // Token-tile staging: piece q = tid + j*NTHR -> (row q/8, 16-byte column q%8).
    // Pieces past the tile repeat the last piece and rows past the valid count
    // re-load the last valid row, so every load is unconditional.
    const bf16_t* Ae = A + ((size_t)e * C + tok_base) * K;
    const bf16_t* aptr[APT];
    int aoff[APT];
#pragma unroll
    for (int j = 0; j < APT; ++j) {
        const int q = min((int)threadIdx.x + j * NTHR, PIECES - 1);
        const int row = q >> 3, c16 = (q & 7) * 8;
        aptr[j] = Ae + (size_t)min(row, nv - 1) * K + c16;
        aoff[j] = row * FFN_LDS_STRIDE + c16;
    }

    // Register rings.  At step k a wave issues the token chunk k+R-1 first
    // and then the weight chunk k+R-1: vector-memory counters complete in
    // issue order, so waiting for the token chunk k+1 never waits for a
    // weight chunk that is still ahead of the MFMAs.
    u32x4 areg[R][APT];
    u32x4 wreg[R][NBW][4];

    f32x16 acc[NBW][TOKB];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;

    const int nk = K >> 6;
#pragma unroll
    for (int p = 0; p < R - 1; ++p) {
        const int kc = min(p, nk - 1);
#pragma unroll
        for (int j = 0; j < APT; ++j) areg[p][j] = *(const u32x4*)(aptr[j] + kc * 64);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) wreg[p][nb][j] = *(const u32x4*)(wptr[nb] + kc * 64 + j * 8);
    }
#pragma unroll
    for (int j = 0; j < APT; ++j) *(u32x4*)(&lds[0][aoff[j]]) = areg[0][j];

    for (int k0 = 0; k0 < nk; k0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int k = k0 + u;
            if (k < nk) {
                const int kn = min(k + R - 1, nk - 1);   // chunk entering the rings (clamped)
                const int slot_n = (u + R - 1) % R;      // a constant once the u loop is unrolled
#pragma unroll
                for (int j = 0; j < APT; ++j) areg[slot_n][j] = *(const u32x4*)(aptr[j] + kn * 64);
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        wreg[slot_n][nb][j] = *(const u32x4*)(wptr[nb] + kn * 64 + j * 8);
                __syncthreads();
                const bf16_t* lb = &lds[k & 1][0];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 bt[TOKB];
#pragma unroll
                    for (int tb = 0; tb < TOKB; ++tb)
                        bt[tb] = as_bf16x8(*(const u32x4*)(lb + (tb * 32 + l32) * FFN_LDS_STRIDE + half * 32 + s * 8));
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        const bf16x8 wa = as_bf16x8(wreg[u][nb][s]);
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb)
                            acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt[tb], acc[nb][tb], 0, 0, 0);
                    }
                }
                // token chunk k+1 (ring slot u+1) into the other LDS buffer
                const int slot_a = (u + 1) % R;
                bf16_t* sb = &lds[(k + 1) & 1][0];
#pragma unroll
                for (int j = 0; j < APT; ++j) *(u32x4*)(sb + aoff[j]) = areg[slot_a][j];
            }
        }
    }

    // Epilogue: each wave parks its tile in LDS (lane: token column l32 of
    // block tb, weight rows 8*(i/4) + 4*half + i%4, so 4 consecutive outputs
    // per store), then the workgroup writes whole rows of NWG outputs per
    // token with 16-byte stores, so every token row gets NWG*OUT_BYTES
    // contiguous bytes instead of scattered 8/16-byte pieces.
    __syncthreads();   // all waves are done reading the token tile
#pragma unroll
    for (int tb = 0; tb < TOKB; ++tb) {
        const int r = tb * 32 + l32;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = wave * 32 * NBW + nb * 32 + q * 8 + half * 4;   // column within the tile
                const f32x16& a = acc[nb][tb];
                char* dst = lds_raw + r * OSTRIDE + c * OUT_BYTES;
                if constexpr (GEMM1) {
                    const uint32_t b0 = bf16_rne(fmaxf(a[4 * q + 0], 0.f)), b1 = bf16_rne(fmaxf(a[4 * q + 1], 0.f));
                    const uint32_t b2 = bf16_rne(fmaxf(a[4 * q + 2], 0.f)), b3 = bf16_rne(fmaxf(a[4 * q + 3], 0.f));
                    *(uint2*)dst = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
                } else {
                    *(f32x4*)dst = f32x4{a[4 * q + 0], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                }
            }
    }
    __syncthreads();
    constexpr int VPR = NWG * OUT_BYTES / 16;        // 16-byte vectors per staged row
    const int ncols = min(NWG, N - nt * NWG);        // valid columns (a multiple of 32)
    const int vpr_valid = ncols * OUT_BYTES / 16;
    char* gout = (char*)out + (((size_t)e * C + tok_base) * N + (size_t)nt * NWG) * OUT_BYTES;
    for (int i = threadIdx.x; i < TOK * VPR; i += NTHR) {
        const int r = i / VPR, v = i - r * VPR;
        if (r < nv && v < vpr_valid)
            *(u32x4*)(gout + (size_t)r * N * OUT_BYTES + v * 16) = *(const u32x4*)(lds_raw + r * OSTRIDE + v * 16);
    }
}

// ------------------------------------------------------------------ launchers
template <int TOKB, int NBW, int WAVES, int R, bool GEMM1>
hipError_t launch_expert_gemm_t(const bf16_t* A, const bf16_t* W, const int32_t* accepted, void* out, int E, int C,
                                int K, int N, hipStream_t s) {
    constexpr int TOK = 32 * TOKB, NWG = WAVES * 32 * NBW;
    const int n_tiles = (N + NWG - 1) / NWG;
    const int tok_tiles = (C + TOK - 1) / TOK;
    const int64_t ntiles = (int64_t)E * n_tiles * tok_tiles;
    if (ntiles == 0) return hipSuccess;
    const int64_t grid = (ntiles + 7) / 8 * 8;
    hipLaunchKernelGGL((expert_gemm<TOKB, NBW, WAVES, R, GEMM1>), dim3((unsigned)grid), dim3(64 * WAVES), 0, s, A, W,
                       accepted, out, C, K, N, n_tiles, tok_tiles, (int)ntiles, (int)grid);
    return hipGetLastError();
}

#ifndef SWMOE_FFN_CUSTOM_DISPATCH
template <bool GEMM1>
static hipError_t launch_expert_gemm(const bf16_t* A, const bf16_t* W, const int32_t* accepted, void* out, int E,
                                     int C, int K, int N, hipStream_t s) {
    // rows per tile: enough 32-row blocks for the capacity, at most 8
    if (C > 128) return launch_expert_gemm_t<8, 1, 4, 3, GEMM1>(A, W, accepted, out, E, C, K, N, s);
    if (C > 64) return launch_expert_gemm_t<4, 1, 8, 5, GEMM1>(A, W, accepted, out, E, C, K, N, s);
    if (C > 32) return launch_expert_gemm_t<2, 2, 4, 3, GEMM1>(A, W, accepted, out, E, C, K, N, s);
    return launch_expert_gemm_t<1, 2, 4, 3, GEMM1>(A, W, accepted, out, E, C, K, N, s);
}

hipError_t launch_expert_gemm1(const bf16_t* buf, const bf16_t* w1, const int32_t* accepted, bf16_t* h, int E,
                               int C, int d, int d_ff, hipStream_t s) {
    return launch_expert_gemm<true>(buf, w1, accepted, h, E, C, d, d_ff, s);
}

hipError_t launch_expert_gemm2(const bf16_t* h, const bf16_t* w2, const int32_t* accepted, float* y, int E, int C,
                               int d, int d_ff, hipStream_t s) {
    return launch_expert_gemm<false>(h, w2, accepted, y, E, C, d_ff, d, s);
}
#endif

}  // namespace swmoe
