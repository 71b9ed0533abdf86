// Backward of the Switch layer: gradients of  sum_t <dout_t, out_t> + L_aux
// (+ L_z)  with respect to x, W1, W2, W_r and b_r, the choices and capacity
// masks held fixed (argmax has no gradient; the router learns through the
// selected gate).  With routing groups and top-k choices every kept (token,
// choice) is one buffer row of its expert and gets the single-choice chain
// rule with its own gate; a token's input gradient adds all its choices.
//
// Sources: "042 Switch Transformer" (wq-win.github.io) sec. 2: the router stays
// differentiable through the selected gate p_e*, and the balance loss is added
// to the training loss; "MoE routing load collapse" (zffjzz.top),
// "troubleshooting": the gradient is checked by central finite differences that
// leave the discrete choices and masks unchanged.
//
// Kernels here (the expert GEMMs reuse expert_gemm):
//   combine_bwd     dy[e, s] = bf16(gate_ti dout_t) for kept choices (buffer
//                   row s of expert e) and dgate_ti = <dout_t, y[e, s]> (fp32),
//                   one wave per (token, choice)
//   transpose_rows  [E][R][S] -> [E][S][Rp] bf16 through 64x64 LDS tiles,
//                   zero for rows >= valid[e] (the token axis of activations)
//   router_wgrad    dW_r partial sums over token slices (fp32 MFMA), then
//   router_wgrad_reduce  the slices added in order in fp64
//   dx_assemble     dx_t = bf16(dout_t + sum_e dz_te W_r[:, e] + sum_i dbuf[e_ti, s_ti])
//                   over the token's kept choices (dx_assemble_mfma on the bf16
//                   MFMA when E is a multiple of 32); dout == NULL leaves the
//                   identity term out (the branch of dx alone)
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

__global__ __launch_bounds__(256) void combine_bwd(const bf16_t* __restrict__ dout, const float* __restrict__ y,
                                                   const int32_t* __restrict__ expert,
                                                   const int32_t* __restrict__ slot,
                                                   const uint8_t* __restrict__ keep, const float* __restrict__ gate,
                                                   int N, int k, int d, int E, int R, bf16_t* __restrict__ dy,
                                                   float* __restrict__ dgate) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);   // assignment (token n / k, choice n % k)
    if (n >= N) return;
    const int64_t t = k == 1 ? n : n / k;
    const int e = expert[n], pos = slot[n];
    if (!keep[n] || e < 0 || e >= E || pos < 0 || pos >= R) {
        if (lane == 0) dgate[n] = 0.f;
        return;
    }
    const float g = gate[n];
    const bf16_t* drow = dout + t * d;
    const float* yrow = y + ((size_t)e * R + pos) * d;
    bf16_t* dyrow = dy + ((size_t)e * R + pos) * d;
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
            o[j] = pack_bf16x2(g * lo, g * hi);
        }
        *(uint4*)(dyrow + c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    acc = wave_sum(acc);
    if (lane == 0) dgate[n] = acc;
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

// dW_r partial sums on the bf16 MFMA: dz = hi + mid + lo exactly (three bf16
// terms, as W_r in the router) and x is bf16, so every product is exact in
// fp32 and v_mfma_f32_32x32x16_bf16 sums the three partial products in fp32.
// Workgroup (128 rows i of W_r, 128 experts e, one token slice); wave w takes
// rows 64 (w >> 1) and experts 64 (w & 1) as 2 x 2 blocks of 32 (A = x
// columns, B = dz columns, K = tokens).  Per chunk of 64 tokens, x and the
// three terms of dz are staged in LDS as K-major rows (token k: 128 bf16, the
// 16-byte slot c at c ^ kmajor_swz(256, k)) and the fragments (8 consecutive tokens
// of one column) come from transposed reads.  The next chunk is loaded into
// registers while the MFMAs run, through descriptors that end with the
// chunk's last token of the slice (rows past it read as zero; the byte count,
// not the scalar offset, decides).
constexpr int RW_CHUNK = 64;
constexpr int RW_TILE = 128;
constexpr int RW_ROW = RW_TILE * 2;             // bytes per staged token row
constexpr int RW_PLANE = RW_CHUNK * RW_ROW;     // one staged operand (16 KiB)
constexpr int RW_PER = RW_CHUNK * 16 / 256;     // 16-byte x slots per thread per chunk

__global__ __launch_bounds__(256) void router_wgrad(const bf16_t* __restrict__ x, const float* __restrict__ dz,
                                                    int64_t T, int d, int E, int tps, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) char lds[4 * RW_PLANE];   // x, then dz's hi, mid, lo
    const int i0 = blockIdx.x * RW_TILE, e0 = blockIdx.y * RW_TILE;
    const int64_t t0 = (int64_t)blockIdx.z * tps;
    const int64_t t1 = min(T, t0 + tps);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, m = lane & 15, g1 = (lane >> 4) & 1;
    const int wi = (wave >> 1) * 64, we = (wave & 1) * 64;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
    // thread q (of RW_PER x 256) loads row q >> 4, 16-byte slot q & 15 of x (8
    // bf16) and the matching 8 floats of dz (two 16-byte loads)
    u32x4 xr[RW_PER], zr[RW_PER][2];
    auto load_chunk = [&](int64_t tc) {
        const uint32_t rows = (uint32_t)min<int64_t>(RW_CHUNK, t1 - tc);
        const __amdgpu_buffer_rsrc_t rx = buffer_rsrc_uniform(x + tc * d, rows * d * 2);
        const __amdgpu_buffer_rsrc_t rz = buffer_rsrc_uniform(dz + tc * E, rows * E * 4);
#pragma unroll
        for (int jj = 0; jj < RW_PER; ++jj) {
            const int q = threadIdx.x + 256 * jj;
            const int r = q >> 4, c = q & 15;
            xr[jj] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)((r * d + i0 + 8 * c) * 2), 0, 0);
            zr[jj][0] = __builtin_amdgcn_raw_buffer_load_b128(rz, (uint32_t)((r * E + e0 + 8 * c) * 4), 0, 0);
            zr[jj][1] = __builtin_amdgcn_raw_buffer_load_b128(rz, (uint32_t)((r * E + e0 + 8 * c) * 4 + 16), 0, 0);
        }
    };
    if (t0 < t1) load_chunk(t0);
    for (int64_t tc = t0; tc < t1; tc += RW_CHUNK) {
        lds_barrier();   // the previous chunk's fragment reads are done
#pragma unroll
        for (int jj = 0; jj < RW_PER; ++jj) {
            const int q = threadIdx.x + 256 * jj;
            const int r = q >> 4, c = q & 15;
            const int at = r * RW_ROW + ((c ^ kmajor_swz(RW_ROW, r)) << 4);
            *(u32x4*)(lds + at) = xr[jj];
            u32x4 hi, mid, lo;
#pragma unroll
            for (int p2 = 0; p2 < 4; ++p2) {   // the three terms of floats 2 p2, 2 p2 + 1
                uint32_t th, tm, tl;
                split3_bf16x2(__uint_as_float(zr[jj][p2 >> 1][2 * (p2 & 1)]),
                              __uint_as_float(zr[jj][p2 >> 1][2 * (p2 & 1) + 1]), th, tm, tl);
                hi[p2] = th;
                mid[p2] = tm;
                lo[p2] = tl;
            }
            *(u32x4*)(lds + RW_PLANE + at) = hi;
            *(u32x4*)(lds + 2 * RW_PLANE + at) = mid;
            *(u32x4*)(lds + 3 * RW_PLANE + at) = lo;
        }
        if (tc + RW_CHUNK < t1) load_chunk(tc + RW_CHUNK);
        lds_barrier();
#pragma unroll
        for (int s = 0; s < RW_CHUNK / 16; ++s) {   // tokens 16 s .. 16 s + 15; this half wave's 8 are 8 (2 s + h) ..
            const int k = 8 * (2 * s + h) + (m >> 2);
            bf16x8 a[2], b[3][2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                a[blk] = kmajor_fragment(lds, RW_ROW, k, wi + 32 * blk + 16 * g1 + 4 * (m & 3));
#pragma unroll
                for (int term = 0; term < 3; ++term)
                    b[term][blk] = kmajor_fragment(lds + (1 + term) * RW_PLANE, RW_ROW, k,
                                                   we + 32 * blk + 16 * g1 + 4 * (m & 3));
            }
#pragma unroll
            for (int jj = 0; jj < 3; ++jj)   // lo, mid, hi
#pragma unroll
                for (int x0 = 0; x0 < 2; ++x0)
#pragma unroll
                    for (int y0 = 0; y0 < 2; ++y0)
                        acc[x0][y0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x0], b[2 - jj][y0], acc[x0][y0], 0, 0, 0);
        }
    }
    // lane: expert column e0 + we + 32 b + (l & 31), rows 8 (i / 4) + 4 h + i % 4 of block a
    float* p = part + (size_t)blockIdx.z * d * E;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int e = e0 + we + 32 * b + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = i0 + wi + 32 * a + 8 * (i >> 2) + 4 * h + (i & 3);
                if (row < d && e < E) p[(size_t)row * E + e] = acc[a][b][i];
            }
        }
}

// dW_r = the slices' partial sums added in slice order in fp64.  A thread
// takes 4 consecutive outputs (one 16-byte load per slice) and issues the
// loads of 8 slices before adding them, in order.
__global__ __launch_bounds__(256) void router_wgrad_reduce(const float* __restrict__ part, int slices, int64_t n,
                                                           float* __restrict__ dw_r) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    if (i + 4 <= n && (n & 3) == 0 && ((uintptr_t)dw_r & 15) == 0) {   // part is 16-byte aligned (workspace)
        int k = 0;
        for (; k + 8 <= slices; k += 8) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *(const f32x4*)(part + (size_t)(k + u) * n + i);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) s[j] += (double)v[u][j];
        }
        for (; k < slices; ++k) {
            const f32x4 v = *(const f32x4*)(part + (size_t)k * n + i);
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] += (double)v[j];
        }
        *(f32x4*)(dw_r + i) = f32x4{(float)s[0], (float)s[1], (float)s[2], (float)s[3]};
    } else {
        for (int j = 0; j < 4 && i + j < n; ++j) {
            double a = 0.0;
            for (int k = 0; k < slices; ++k) a += (double)part[(size_t)k * n + i + j];
            dw_r[i + j] = (float)a;
        }
    }
}

// dx: workgroup = 64 tokens x 64 columns of x, 4 x 4 per thread; K = E in
// chunks of 32.
__global__ __launch_bounds__(256) void dx_assemble(const bf16_t* __restrict__ dout, const float* __restrict__ dbuf,
                                                   const int32_t* __restrict__ expert,
                                                   const int32_t* __restrict__ slot,
                                                   const uint8_t* __restrict__ keep, const float* __restrict__ dz,
                                                   const float* __restrict__ w_r, int64_t T, int d, int E, int k,
                                                   int R, bf16_t* __restrict__ dx) {
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
        const uint2 dv = dout ? *(const uint2*)(dout + t * d + i) : make_uint2(0, 0);
        float v[4] = {bf16_to_f32(dv.x & 0xffffu) + acc[a][0], bf16_to_f32(dv.x >> 16) + acc[a][1],
                      bf16_to_f32(dv.y & 0xffffu) + acc[a][2], bf16_to_f32(dv.y >> 16) + acc[a][3]};
        for (int c = 0; c < k; ++c) {   // the kept choices in rank order
            const int64_t n = t * k + c;
            const int e = expert[n], pos = slot[n];
            if (keep[n] && e >= 0 && e < E && pos >= 0 && pos < R) {
                const f32x4 b = *(const f32x4*)(dbuf + ((size_t)e * R + pos) * d + i);
                v[0] += b[0]; v[1] += b[1]; v[2] += b[2]; v[3] += b[3];
            }
        }
        *(uint2*)(dx + t * d + i) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
}

// dx on the bf16 MFMA (E a multiple of 32, d a multiple of 128, w_r and dz
// 16-byte aligned): workgroup = 128 columns i x 128 tokens, wave w = columns
// 64 (w >> 1) x tokens 64 (w & 1) as 2 x 2 blocks of 32.  A = W_r rows (i,
// K = e), B = dz^T (K = e, column = token).  Both are fp32; each goes into
// the MFMA as the first two terms of its bf16 split (hi + mid, a remainder
// below 2^-16 of the value), and the products mid x hi, hi x mid and hi x hi
// are accumulated in fp32, so the router term dz W_r^T carries a relative
// error of about 2^-15 of sum_e |dz_te W_r[i, e]|, far below the bf16
// rounding of dx.  Per chunk of 32 experts the
// workgroup's 128 W_r rows and 128 dz rows (128 bytes each) go from memory
// straight into LDS, eight 1 KiB copies per wave with the lanes along the
// expert axis (16-byte column c of row r at c ^ ((r >> 1) & 7): any 16
// consecutive rows of a fragment read on all 64 LDS banks); two stages, one barrier per
// chunk; dz rows past T read as zero.  A chunk is two 16-expert MFMA steps
// (v_mfma_f32_32x32x16_bf16): in step kq half wave h takes experts 16 kq +
// 8 h .. + 7, two 16-byte columns of each of its rows, split in registers.
// In a result block lane l holds token l & 31 and columns
// {0-3, 8-11, 16-19, 24-27} (+4 for h = 1); one v_permlane32_swap per register
// pair turns these into two runs of 8 consecutive columns, so dout, dbuf and
// dx move 16 or 32 bytes at a time.  dx = bf16(dout + sum_e dz W_r +
// the kept choices' dbuf rows) as in dx_assemble.
constexpr int DX_STAGE = 2 * 128 * 128;   // bytes: the W_r tile, then the dz tile

// v = hi + mid + (a remainder below 2^-16 |v|): the first two terms of the
// exact three-term bf16 split, eight values at a time
// (the hardware's round-to-nearest-even conversion, two values per instruction)
__device__ __forceinline__ void split2_bf16x8(const f32x4& v0, const f32x4& v1, bf16x8& hi, bf16x8& mid) {
    const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    u32x4 ph, pm;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t h = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        ph[j] = h;
        pm[j] = pack_bf16x2(v[2 * j] - bf16_lo_f32(h), v[2 * j + 1] - bf16_hi_f32(h));
    }
    hi = as_bf16x8(ph);
    mid = as_bf16x8(pm);
}

template <int K>
__global__ __launch_bounds__(256) void dx_assemble_mfma(const bf16_t* __restrict__ dout,
                                                        const float* __restrict__ dbuf,
                                                        const int32_t* __restrict__ expert,
                                                        const int32_t* __restrict__ slot,
                                                        const uint8_t* __restrict__ keep,
                                                        const float* __restrict__ dz, const float* __restrict__ w_r,
                                                        int64_t T, int d, int E, int R, bf16_t* __restrict__ dx) {
    __shared__ __attribute__((aligned(16))) char lds[2 * DX_STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int ib = blockIdx.x * 128;
    const int64_t tb = (int64_t)blockIdx.y * 128;
    const int i0 = ib + (wave >> 1) * 64;
    const int64_t t0 = tb + (wave & 1) * 64;
    const int nk = E / 32;

    // copy q = 8 wave + i lands at stage + 1 KiB q: W_r rows for q < 16, dz rows
    // after; lane -> row 8 (q % 16) + lane / 8, LDS column lane % 8
    const bool wrows = wave < 2;
    const char* base = wrows ? (const char*)(w_r + (size_t)ib * E) : (const char*)(dz + tb * E);
    const uint32_t nbytes = wrows ? (uint32_t)128 * E * 4 : (uint32_t)min<int64_t>(128, T - tb) * E * 4;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, nbytes);
    uint32_t vo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * ((8 * wave + i) & 15) + (lane >> 3);
        vo[i] = (uint32_t)row * E * 4 + (((lane & 7) ^ ((row >> 1) & 7)) << 4);
    }
    auto issue = [&](int kc, int stg) {
        char* dst = lds + stg * DX_STAGE + wave * 8 * 1024;
        const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane(kc * 128);
#pragma unroll
        for (int i = 0; i < 8; ++i) copy_to_lds(rs, dst + i * 1024, vo[i], so);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    // the routing of this lane's two tokens, fetched now (the first chunk's
    // wait covers it): the dbuf row e * R + slot of each kept choice, else -1
    int te[2][K], tp[2][K], tk[2][K];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t tc = min<int64_t>(t0 + 32 * b + l32, T - 1);
#pragma unroll
        for (int c = 0; c < K; ++c) {
            te[b][c] = expert[tc * K + c];
            tp[b][c] = slot[tc * K + c];
            tk[b][c] = keep[tc * K + c];
        }
    }
    issue(0, 0);
    int kc = 0;
    do {   // E >= 32: at least one chunk
        wait_copies<0>();   // this wave's copies of chunk kc
        lds_barrier();      // every wave's, and chunk kc - 1 is read out
        issue(min(kc + 1, nk - 1), (kc + 1) & 1);   // the last chunk is fetched twice, never read
        const char* st = lds + (kc & 1) * DX_STAGE;
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {   // experts 16 kq + 8 h .. + 7 of the chunk: 16-byte columns 4 kq + 2 h + {0, 1}
            bf16x8 ah[2], am[2], bh[2], bm[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int ra = (wave >> 1) * 64 + 32 * q + l32;   // W_r row in the tile
                const int rb = (wave & 1) * 64 + 32 * q + l32;    // dz row in the tile
                const int c0 = 4 * kq + 2 * h;
                const f32x4 a0 = *(const f32x4*)(st + ra * 128 + ((c0 ^ ((ra >> 1) & 7)) << 4));
                const f32x4 a1 = *(const f32x4*)(st + ra * 128 + (((c0 + 1) ^ ((ra >> 1) & 7)) << 4));
                const f32x4 b0 = *(const f32x4*)(st + 128 * 128 + rb * 128 + ((c0 ^ ((rb >> 1) & 7)) << 4));
                const f32x4 b1 = *(const f32x4*)(st + 128 * 128 + rb * 128 + (((c0 + 1) ^ ((rb >> 1) & 7)) << 4));
                split2_bf16x8(a0, a1, ah[q], am[q]);
                split2_bf16x8(b0, b1, bh[q], bm[q]);
            }
            // small products first: mid x hi, hi x mid, then hi x hi
#pragma unroll
            for (int x0 = 0; x0 < 2; ++x0)
#pragma unroll
                for (int y0 = 0; y0 < 2; ++y0) {
                    acc[x0][y0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[x0], bh[y0], acc[x0][y0], 0, 0, 0);
                    acc[x0][y0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[x0], bm[y0], acc[x0][y0], 0, 0, 0);
                    acc[x0][y0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[x0], bh[y0], acc[x0][y0], 0, 0, 0);
                }
        }
    } while (++kc < nk);
    wait_copies<0>();   // the spare copy of the last chunk
    // runs of 8 columns: swap rows 8-11 of half 0 with rows 4-7 of half 1 (and 24-27 with 20-23)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(
                        __float_as_uint(acc[a][b][8 * pr + i]), __float_as_uint(acc[a][b][8 * pr + 4 + i]), false,
                        false);
                    acc[a][b][8 * pr + i] = __uint_as_float(sw[0]);
                    acc[a][b][8 * pr + 4 + i] = __uint_as_float(sw[1]);
                }
    // every load of the epilogue before its first store (a load issued after a
    // store waits for that store too); rows past T read row T - 1 and are not stored
    uint4 dv[2][2][2];
    f32x4 bq[2][2][2][2];   // the sum of the kept choices' dbuf rows
#pragma unroll
    for (int c = 0; c < K; ++c) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t tc = min<int64_t>(t0 + 32 * b + l32, T - 1);
            const bool kept = tk[b][c] && te[b][c] >= 0 && te[b][c] < E && tp[b][c] >= 0 && tp[b][c] < R;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    const int i = i0 + 32 * a + 16 * run + 8 * h;
                    if (c == 0) {
                        dv[b][a][run] = dout ? *(const uint4*)(dout + tc * d + i) : make_uint4(0, 0, 0, 0);
                        bq[b][a][run][0] = bq[b][a][run][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                    if (kept) {
                        const float* br = dbuf + ((size_t)te[b][c] * R + tp[b][c]) * d + i;
                        const f32x4 l0 = *(const f32x4*)br, l1 = *(const f32x4*)(br + 4);
                        if (c == 0) {
                            bq[b][a][run][0] = l0;
                            bq[b][a][run][1] = l1;
                        } else {
                            bq[b][a][run][0] += l0;
                            bq[b][a][run][1] += l1;
                        }
                    }
                }
        }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const uint4 v = dv[b][a][run];
                const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4& bb = bq[b][a][run][j >> 1];
                    const float v0 = (bf16_to_f32(dw[j] & 0xffffu) + acc[a][b][8 * run + 2 * j]) + bb[2 * (j & 1)];
                    const float v1 = (bf16_to_f32(dw[j] >> 16) + acc[a][b][8 * run + 2 * j + 1]) + bb[2 * (j & 1) + 1];
                    o[j] = pack_bf16x2(v0, v1);
                }
                dv[b][a][run] = make_uint4(o[0], o[1], o[2], o[3]);
            }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t t = t0 + 32 * b + l32;
        if (t >= T) continue;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int run = 0; run < 2; ++run)
                *(uint4*)(dx + t * d + i0 + 32 * a + 16 * run + 8 * h) = dv[b][a][run];
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

hipError_t launch_combine_bwd(const bf16_t* dout, const float* y, const int32_t* expert, const int32_t* slot,
                              const uint8_t* keep, const float* gate, int64_t T, int k, int d, int E, int R,
                              bf16_t* dy, float* dgate, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int N = (int)(T * k);
    hipLaunchKernelGGL(combine_bwd, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, dout, y, expert, slot, keep, gate,
                       N, k, d, E, R, dy, dgate);
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
    const unsigned rblocks = (unsigned)((n + 1023) / 1024);   // 4 outputs per thread
    if (slices == 0) {   // no tokens: the gradient is zero
        hipLaunchKernelGGL(router_wgrad_reduce, dim3(rblocks), dim3(256), 0, s, part, 0, n, dw_r);
        return hipGetLastError();
    }
    int tps = (int)((T + slices - 1) / slices);
    tps = (tps + RW_CHUNK - 1) / RW_CHUNK * RW_CHUNK;
    const int used = (int)((T + tps - 1) / tps);
    hipLaunchKernelGGL(router_wgrad, dim3((d + RW_TILE - 1) / RW_TILE, (E + RW_TILE - 1) / RW_TILE, used), dim3(256), 0,
                       s, x, dz, T, d, E, tps, part);
    hipLaunchKernelGGL(router_wgrad_reduce, dim3(rblocks), dim3(256), 0, s, part, used, n, dw_r);
    return hipGetLastError();
}

hipError_t launch_dx_assemble(const bf16_t* dout, const float* dbuf, const int32_t* expert, const int32_t* slot,
                              const uint8_t* keep, const float* dz, const float* w_r, int64_t T, int d, int E, int k,
                              int R, bf16_t* dx, hipStream_t s) {
    if (T == 0) return hipSuccess;
    // the MFMA kernel copies 32-expert chunks of w_r and dz rows 16 bytes at a time
    if (E % 32 == 0 && d % 128 == 0 && ((uintptr_t)w_r | (uintptr_t)dz) % 16 == 0) {
        const dim3 grid(d / 128, (unsigned)((T + 127) / 128));
#define SWMOE_DX(K)                                                                                            \
    hipLaunchKernelGGL(dx_assemble_mfma<K>, grid, dim3(256), 0, s, dout, dbuf, expert, slot, keep, dz, w_r, T, d, \
                       E, R, dx)
        switch (k) {
            case 1: SWMOE_DX(1); break;
            case 2: SWMOE_DX(2); break;
            case 3: SWMOE_DX(3); break;
            default: SWMOE_DX(4); break;
        }
#undef SWMOE_DX
    } else {
        hipLaunchKernelGGL(dx_assemble, dim3(d / 64, (unsigned)((T + 63) / 64)), dim3(256), 0, s, dout, dbuf, expert,
                           slot, keep, dz, w_r, T, d, E, k, R, dx);
    }
    return hipGetLastError();
}

}  // namespace swmoe
