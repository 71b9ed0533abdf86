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

// w_r [d, E] fp32 -> the three bf16 terms, one K stage of 32 per block,
// [d / 32][3][E][32], so that an MFMA operand row (one expert, 8 consecutive
// k) is 16 contiguous bytes and the weight rows of one stage are one block
// (d is a multiple of 32).
__global__ __launch_bounds__(256) void split_router_weights(const float* __restrict__ w_r,
                                                            bf16_t* __restrict__ wr3, int d, int E) {
    // thread i: expert e = i % E and the 8 consecutive rows k = 8 (i / E) ..;
    // a wave's eight loads (one per k) are each 64 consecutive experts, and
    // each term's 8 values of one expert are one 16-byte store
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= (d / 8) * E) return;
    const int kc = i / E, e = i - kc * E;
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = w_r[(size_t)(8 * kc + j) * E + e];
    uint32_t t3[3][4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) split3_bf16x2(w[j], w[j + 1], t3[0][j / 2], t3[1][j / 2], t3[2][j / 2]);
    bf16_t* o = wr3 + (size_t)(kc / 4) * 3 * E * 32 + (size_t)e * 32 + 8 * (kc % 4);
#pragma unroll
    for (int q = 0; q < 3; ++q)
        *(uint4*)(o + (size_t)q * E * 32) = make_uint4(t3[q][0], t3[q][1], t3[q][2], t3[q][3]);
}

// logits[t, e] = sum_k x[t, k] (hi + mid + lo)[e, k] + b[e] for E > 256.
// A workgroup of 8 waves computes a tile of RG_T = 256 tokens x RG_E = 256
// experts; wave (wt, we) = (w / 4, w % 4) owns tokens 128 wt .. + 127 and
// experts 64 we .. + 63 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (A =
// token rows, B = expert rows), each block taking the lo, mid and hi terms
// in that order.  Per 32-wide K stage, the 256 token rows and the 3 x 256
// weight rows (64 bytes each; in the chunked split layout each term's rows of
// one stage are one contiguous block) go from memory straight into LDS, eight
// 1 KiB copies per wave (waves 0-1 the token rows, 2-7 the weight terms), the
// four 16-byte columns of row r at column ^ ((r >> 2) & 3), which puts any
// 16 consecutive rows of a fragment read on all 64 LDS banks.  Two stages, one barrier per
// stage.  Token rows past T read as zero; expert rows past E repeat row E - 1
// and only reach logits that are never stored.  Tiles are numbered expert-tile-major and dealt XCD-major, so the
// workgroups of an XCD share one expert tile's weight rows in its L2.
constexpr int RG_T = 256, RG_E = 256;
constexpr int RG_STAGE = (RG_T + 3 * RG_E) * 64;   // bytes of one K stage

__global__ __launch_bounds__(512) void router_gemm(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr3,
                                                   const float* __restrict__ b_r, float* __restrict__ logits,
                                                   int T, int d, int E, int n_tt, int n_tiles) {
    __shared__ __attribute__((aligned(16))) char lds[2 * RG_STAGE];
    const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
    if (tile >= n_tiles) return;
    // (the division runs on the vector unit: readfirstlane keeps the tile, and
    // so the copies' descriptors, scalar)
    const int et = __builtin_amdgcn_readfirstlane(tile / n_tt), tt = tile - et * n_tt;
    const int t0 = tt * RG_T, e0 = et * RG_E;
    const int lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wt = wave >> 2, we = wave & 3;
    const int nk = d / 32;

    // this wave's eight copies: q = 8 wave + i lands at stage + 1 KiB q; lane ->
    // row 16 (q % 16) + lane / 4 of its 256-row block, LDS column lane % 4
    const bool tok_rows = wave < 2;
    const char* base = tok_rows ? (const char*)(x + (size_t)t0 * d) : (const char*)wr3;
    const uint32_t nbytes = tok_rows ? (uint32_t)min(RG_T, T - t0) * d * 2 : (uint32_t)3 * E * d * 2;
    const uint32_t kstep = tok_rows ? 64u : (uint32_t)3 * E * 64;   // source bytes per K stage
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, nbytes);
    uint32_t vo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = 8 * wave + i;
        const int row = 16 * (q & 15) + (lane >> 2);
        const uint32_t col = (uint32_t)(((lane & 3) ^ ((row >> 2) & 3)) << 4);
        const int term = (q >> 4) - 1;   // weight copies: q = 16 (1 + term) + row block
        vo[i] = tok_rows ? (uint32_t)row * d * 2 + col : (uint32_t)(term * E + min(e0 + row, E - 1)) * 64 + col;
    }
    auto issue = [&](int kk, int stg) {
        char* dst = lds + stg * RG_STAGE + wave * 8 * 1024;
        const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)kk * kstep);
#pragma unroll
        for (int i = 0; i < 8; ++i) copy_to_lds(rs, dst + i * 1024, vo[i], so);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int eb = 0; eb < 2; ++eb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[tb][eb][i] = 0.f;

    issue(0, 0);
    int kk = 0;
    do {   // d >= 32: at least one stage
        wait_copies<0>();   // this wave's copies of stage kk
        lds_barrier();      // every wave's, and stage kk - 1 is read out
        issue(min(kk + 1, nk - 1), (kk + 1) & 1);   // the last stage is fetched twice, never read
        const char* st = lds + (kk & 1) * RG_STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = 2 * ks + hl;   // this lane's 16-byte column of the 64-byte rows
            bf16x8 a[4], b[3][2];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int r = wt * 128 + tb * 32 + l32;
                a[tb] = as_bf16x8(*(const u32x4*)(st + r * 64 + ((c ^ ((r >> 2) & 3)) << 4)));
            }
#pragma unroll
            for (int term = 0; term < 3; ++term)
#pragma unroll
                for (int eb = 0; eb < 2; ++eb) {
                    const int r = we * 64 + eb * 32 + l32;
                    b[term][eb] = as_bf16x8(
                        *(const u32x4*)(st + (1 + term) * RG_E * 64 + r * 64 + ((c ^ ((r >> 2) & 3)) << 4)));
                }
#pragma unroll
            for (int jj = 0; jj < 3; ++jj)   // lo, mid, hi
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                    for (int eb = 0; eb < 2; ++eb)
                        acc[tb][eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tb], b[2 - jj][eb], acc[tb][eb], 0, 0, 0);
        }
    } while (++kk < nk);
    wait_copies<0>();   // the spare copy of the last stage

    // lane: expert column e0 + 64 we + 32 eb + l32, token rows 8 (i / 4) + 4 hl + i % 4 of
    // block tb; stores past T (the descriptor's count) or past E (offset past it) are dropped
    // The descriptor comes from readfirstlane'd words and the offset from a
    // bitwise select, so the compiler sees no divergence to guard the stores
    // with.  readfirstlane returns a signed int: each word goes through
    // uint32_t, or the low word would be sign-extended into the high one.
    const uint32_t out_bytes = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)min(RG_T, T - t0) * E * 4);
    const uint64_t ob = (uint64_t)(uintptr_t)(logits + (size_t)t0 * E);
    const uint32_t ob_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ob);
    const uint32_t ob_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ob >> 32));
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(uintptr_t)(((uint64_t)ob_hi << 32) | (uint64_t)ob_lo), (short)0, (int)out_bytes, kBufferWord3);
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
        const int e = e0 + we * 64 + eb * 32 + l32;
        const uint32_t in_e = 0u - (uint32_t)(e < E);
        const float bias = b_r ? b_r[min(e, E - 1)] : 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = wt * 128 + tb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
                const uint32_t off = ((((uint32_t)row * E + e) * 4) & in_e) | (out_bytes & ~in_e);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[tb][eb][i] + bias), ro, off, 0, 0);
            }
    }
}

// e^x for the softmax as 2^(x log2 e) on the hardware exp2 (v_exp_f32): the
// rounding of the product adds a relative error of about |x| 2^-24 ln 2 to a
// term, so the terms that matter (x near 0) stay within a few ulp.
__device__ __forceinline__ float rf_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Softmax statistics per token.  A workgroup (4 waves) owns `tpb` consecutive
// tokens; a wave handles one token at a time with lane j holding experts
// j, j+64, ...  Writes the k choices and their gates ([T, k], choices in
// decreasing logit order, ties to the lower index), lse and the workgroup's
// partial sums of p_te over its tokens (fixed order: lanes in registers,
// waves in turn).  KMAX bounds k at compile time.
template <int NCH, int KMAX>
__global__ __launch_bounds__(256) void router_softmax(const float* __restrict__ logits, int T, int E, int k,
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
        float zc[KMAX > 1 ? NCH : 1];
        float m = -INFINITY;
        int mi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            int e = lane + 64 * i;
            v[i] = e < E ? row[e] : -INFINITY;
            if constexpr (KMAX > 1) zc[i] = v[i];
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
            expert[(size_t)t * k] = mi;
            gate[(size_t)t * k] = inv;    // p_{e*} = exp(z_e* - m) / s = 1 / s
            lse[t] = m + logf(s);
        }
        if constexpr (KMAX > 1) {
            // choice r: the largest logit among the experts not yet chosen
            int ch[KMAX];
            ch[0] = mi;
#pragma unroll
            for (int r = 1; r < KMAX; ++r) {
                if (r >= k) break;
                float mr = -INFINITY;
                int ir = 0x7fffffff;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const int e = lane + 64 * i;
                    bool taken = e >= E;
#pragma unroll
                    for (int q = 0; q < r; ++q) taken |= e == ch[q];
                    if (!taken && zc[i] > mr) { mr = zc[i]; ir = e; }
                }
                wave_argmax(mr, ir);
                ch[r] = ir;
                if (lane == 0) {
                    expert[(size_t)t * k + r] = ir;
                    gate[(size_t)t * k + r] = expf(mr - m) * inv;
                }
            }
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

// The same for E a multiple of 4 (and 16-byte aligned logits): lane j holds
// experts 4 j + 256 i .. + 3 (one 16-byte load each), and a wave loads the
// row of its next token while it works on the current one.  e^x is rf_exp,
// as in the fused router.
template <int NC4, int KMAX, int R = 2>
__global__ __launch_bounds__(256) void router_softmax4(const float* __restrict__ logits, int T, int E, int k,
                                                       int tpb, int32_t* __restrict__ expert,
                                                       float* __restrict__ gate, float* __restrict__ lse,
                                                       float* __restrict__ part) {
    extern __shared__ float red[];  // [E]
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = blockIdx.x * tpb, t1 = min(T, t0 + tpb);
    float acc[NC4][4];
#pragma unroll
    for (int i = 0; i < NC4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    // every load unconditional (a load under a lane or token condition makes
    // the compiler wait for all loads in flight, the prefetch included): the
    // row's descriptor ends at E, and lanes past it read zero, taken as -inf
    auto load = [&](int t, f32x4 (&v)[NC4]) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc_uniform(logits + (size_t)t * E, (uint32_t)E * 4);
#pragma unroll
        for (int i = 0; i < NC4; ++i)
            v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(4 * lane + 256 * i) * 4, 0, 0));
        // issued here: the scheduler may not sink them below the waits for the other buffer
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // two row buffers: the row after next is always in flight while a row is
    // processed (rows past the slice repeat its last row, unused)
    auto process = [&](int t, f32x4 (&cur)[NC4]) {
#pragma unroll
        for (int i = 0; i < NC4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * lane + 256 * i + j >= E) cur[i][j] = -INFINITY;
        float m = -INFINITY;
        int mi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NC4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (cur[i][j] > m) { m = cur[i][j]; mi = 4 * lane + 256 * i + j; }   // strict: lowest index per lane
        wave_argmax_valu(m, mi);
        float p[NC4][4];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < NC4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[i][j] = (4 * lane + 256 * i + j < E) ? rf_exp(cur[i][j] - m) : 0.f;
                sum += p[i][j];
            }
        sum = wave_sum_valu(sum);
        const float inv = 1.0f / sum;
#pragma unroll
        for (int i = 0; i < NC4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += p[i][j] * inv;
        if (lane == 0) {
            expert[(size_t)t * k] = mi;
            gate[(size_t)t * k] = inv;    // p_{e*} = exp(z_e* - m) / s = 1 / s
            lse[t] = m + logf(sum);
        }
        if constexpr (KMAX > 1) {
            // choice r: the largest logit among the experts not yet chosen
            int ch[KMAX];
            ch[0] = mi;
#pragma unroll
            for (int r = 1; r < KMAX; ++r) {
                if (r >= k) break;
                float mr = -INFINITY;
                int ir = 0x7fffffff;
#pragma unroll
                for (int i = 0; i < NC4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int e = 4 * lane + 256 * i + j;
                        bool taken = e >= E;
#pragma unroll
                        for (int q = 0; q < r; ++q) taken |= e == ch[q];
                        if (!taken && cur[i][j] > mr) { mr = cur[i][j]; ir = e; }
                    }
                wave_argmax_valu(mr, ir);
                ch[r] = ir;
                if (lane == 0) {
                    expert[(size_t)t * k + r] = ir;
                    gate[(size_t)t * k + r] = rf_exp(mr - m) * inv;
                }
            }
        }
    };
    // a ring of R row buffers: while a row is processed the next R - 1 rows of
    // the wave are in flight (rows past the slice repeat its last row, unused);
    // the loop is unrolled by R so every buffer index is a constant
    f32x4 ring[R][NC4];
    const int tw = t0 + wave;
    if (tw < t1) {
#pragma unroll
        for (int i = 0; i < R - 1; ++i) load(min(tw + 4 * i, t1 - 1), ring[i]);
        for (int t = tw; t < t1; t += 4 * R) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                load(min(t + 4 * (u + R - 1), t1 - 1), ring[(u + R - 1) % R]);
                if (t + 4 * u < t1) process(t + 4 * u, ring[u]);
            }
        }
    }
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int i = 0; i < NC4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 4 * lane + 256 * i + j;
                    if (e < E) red[e] = (w == 0) ? acc[i][j] : red[e] + acc[i][j];
                }
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < E; e += 256) part[(size_t)blockIdx.x * E + e] = red[e];
}

// prob_sum[g][e] = sum over the partial rows of routing group g (rows
// g*nblk .. g*nblk+nblk-1), in fp64, in a fixed order: a workgroup owns 64
// experts of one group; its 16 row groups take every 16th partial row, then
// the row groups are added in order.  One group: prob_sum[e] over all rows.
__global__ __launch_bounds__(1024) void router_reduce(const float* __restrict__ part, int nblk, int total, int E,
                                                      float* __restrict__ prob_sum) {
    __shared__ double red[16][64];
    const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + c;
    part += (size_t)blockIdx.y * nblk * E;
    prob_sum += (size_t)blockIdx.y * E;
    nblk = min(nblk, total - (int)blockIdx.y * nblk);   // the last group may be short
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
    const int64_t n = (int64_t)(d / 8) * E;   // d is a multiple of 32
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(split_router_weights, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, w_r, wr3, d, E);
    return hipGetLastError();
}

hipError_t launch_router_gemm(const bf16_t* x, const bf16_t* wr3, const float* b_r, float* logits,
                              int T, int d, int E, hipStream_t s) {
    const int n_tt = (T + RG_T - 1) / RG_T, n_et = (E + RG_E - 1) / RG_E;
    const int n_tiles = n_tt * n_et;
    const int grid = (n_tiles + 7) / 8 * 8;
    hipLaunchKernelGGL(router_gemm, dim3(grid), dim3(512), 0, s, x, wr3, b_r, logits, T, d, E, n_tt, n_tiles);
    return hipGetLastError();
}

int router_softmax_blocks(int64_t T, int E) {
    if (T <= 0) return 0;
    // about 64 tokens per workgroup, at most 4 MiB of partial sums
    int64_t nblk = std::min<int64_t>((T + 63) / 64, std::max<int64_t>(1, (int64_t(1) << 20) / E));
    int64_t tpb = (T + nblk - 1) / nblk;
    return (int)((T + tpb - 1) / tpb);
}

int router_softmax_blocks_grouped(int64_t T) { return (int)((T + 63) / 64); }

// row buffers per wave of router_softmax4
constexpr int kSoftmaxRing = 2;

template <int KMAX>
static void softmax_by_width(int nblk, int tpb, const float* logits, int T, int E, int k, int32_t* expert,
                             float* gate, float* lse, float* part, hipStream_t s) {
    const size_t shm = (size_t)E * sizeof(float);
    if (E % 4 == 0 && (uintptr_t)logits % 16 == 0) {   // 16-byte rows
        const int nc4 = (E + 255) / 256;
#define SWMOE_SOFTMAX4(N)                                                                                  \
    hipLaunchKernelGGL((router_softmax4<N, KMAX, kSoftmaxRing>), dim3(nblk), dim3(256), shm, s, logits, T, E, k, \
                       tpb, expert, gate, lse, part)
        if (nc4 <= 1) SWMOE_SOFTMAX4(1);
        else if (nc4 <= 2) SWMOE_SOFTMAX4(2);
        else if (nc4 <= 4) SWMOE_SOFTMAX4(4);
        else if (nc4 <= 8) SWMOE_SOFTMAX4(8);
        else SWMOE_SOFTMAX4(16);
#undef SWMOE_SOFTMAX4
        return;
    }
    const int nch = (E + 63) / 64;
#define SWMOE_SOFTMAX(N)                                                                                  \
    hipLaunchKernelGGL((router_softmax<N, KMAX>), dim3(nblk), dim3(256), shm, s, logits, T, E, k, tpb, expert, \
                       gate, lse, part)
    if (nch <= 1) SWMOE_SOFTMAX(1);
    else if (nch <= 2) SWMOE_SOFTMAX(2);
    else if (nch <= 4) SWMOE_SOFTMAX(4);
    else if (nch <= 8) SWMOE_SOFTMAX(8);
    else if (nch <= 16) SWMOE_SOFTMAX(16);
    else if (nch <= 32) SWMOE_SOFTMAX(32);
    else SWMOE_SOFTMAX(64);
#undef SWMOE_SOFTMAX
}

hipError_t launch_router_softmax(const float* logits, int T, int E, int k, bool rows_of_64, int32_t* expert,
                                 float* gate, float* lse, float* part, hipStream_t s) {
    const int nblk = rows_of_64 ? router_softmax_blocks_grouped(T) : router_softmax_blocks(T, E);
    const int tpb = rows_of_64 ? 64 : (T + nblk - 1) / nblk;
    if (k <= 1) softmax_by_width<1>(nblk, tpb, logits, T, E, k, expert, gate, lse, part, s);
    else if (k <= 2) softmax_by_width<2>(nblk, tpb, logits, T, E, k, expert, gate, lse, part, s);
    else softmax_by_width<kMaxTopK>(nblk, tpb, logits, T, E, k, expert, gate, lse, part, s);
    return hipGetLastError();
}

hipError_t launch_router_reduce(const float* part, int nblk, int ngroups, int E, float* prob_sum, hipStream_t s) {
    if (ngroups == 0) return hipSuccess;
    hipLaunchKernelGGL(router_reduce, dim3((E + 63) / 64, ngroups), dim3(1024), 0, s, part, nblk, nblk * ngroups, E,
                       prob_sum);
    return hipGetLastError();
}

// rows per slice of the column sum: 16 per thread of router_reduce, so each
// thread's loads are few and the slices many
constexpr int kColumnSlice = 256;
int column_sum_slices(int64_t rows) { return (int)std::max<int64_t>(1, (rows + kColumnSlice - 1) / kColumnSlice); }

// out[e] = sum over the rows of a [rows, E] array: slices of kColumnSlice rows
// summed in parallel (each in the fixed order above), then the slices in order.
hipError_t launch_column_sum(const float* a, int rows, int E, float* slices, float* out, hipStream_t s) {
    const int ns = column_sum_slices(rows);
    if (ns == 1) {
        hipLaunchKernelGGL(router_reduce, dim3((E + 63) / 64, 1), dim3(1024), 0, s, a, rows, rows, E, out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(router_reduce, dim3((E + 63) / 64, ns), dim3(1024), 0, s, a, kColumnSlice, rows, E, slices);
    hipLaunchKernelGGL(router_reduce, dim3((E + 63) / 64, 1), dim3(1024), 0, s, slices, ns, ns, E, out);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Fused router for E <= 256: logits, softmax statistics and top-k in one pass.
// A workgroup (4 waves) owns RF_TOK = 64 tokens and all experts.  The waves
// split the expert blocks of 16 (up to 4 ways) and, with fewer than 4 expert
// blocks, the four 16-token blocks.  Per 32-wide K stage:
//  - the 64 token rows (64 bytes each) are copied from memory straight into
//    an LDS stage shared by the waves (one 1 KiB copy per wave), the four
//    16-byte columns of a row XOR-swizzled by (row >> 2) & 3 so that the
//    16 rows of a fragment read fall on all 64 LDS banks; token rows past T read as
//    zero through the descriptor's byte count;
//  - each wave loads the fp32 router weights of its own fragments from W_r
//    as stored ([d, E]: for lane (r16, g) of an expert block, the 8 values
//    k = 8 g .. 8 g + 7 of expert r16, 8 dword loads whose lanes read 64
//    contiguous bytes per k row) from memory straight into a register ring,
//    and splits them into their hi, mid and lo bf16 terms right before the
//    MFMAs (the hardware's round-to-nearest-even conversion, two values per
//    instruction; the same exact split as split_router_weights, so no split
//    pass runs and each weight crosses the caches as 4 bytes, not 6);
//    experts past E repeat expert E - 1 (they only feed outputs that are
//    never used).
// Both run S - 1 stages ahead of the MFMAs, with one workgroup barrier per
// stage.  After the last stage the logits go through an LDS tile, and wave w
// finishes tokens 16 w .. 16 w + 15: bias, row max with the lowest index on
// ties, sum of exp, lse, gate = 1/sum, optional logits store, the top-k
// choices, and the workgroup's partial sums of p_te over its tokens (DPP sums
// over the 16 tokens of a wave, then the waves in turn through LDS: a fixed
// order).
constexpr int RF_TOK = 64;     // tokens per workgroup (one partial row)
constexpr int RF_KC = 32;      // K per stage (one 16x16x32 MFMA step)

// routing groups reduce whole 64-token partial rows (router_reduce)
static_assert(RF_TOK == 64, "the fused router writes one partial row per 64 tokens");
int router_fused_blocks(int64_t T) { return (int)((T + RF_TOK - 1) / RF_TOK); }


template <int EB, int S, int KMAX, bool FULL>
__global__ __launch_bounds__(256) void router_fused(const bf16_t* __restrict__ x, const float* __restrict__ w_r,
                                                    const float* __restrict__ b_r, int T, int d, int E, int k,
                                                    float* __restrict__ logits_out, int32_t* __restrict__ expert,
                                                    float* __restrict__ gate, float* __restrict__ lse,
                                                    float* __restrict__ part) {
    constexpr int EP = EB * 16;
    // E a whole number of expert blocks: each K stage of W_r (32 rows of E
    // floats, one contiguous block) is copied into LDS next to the token rows;
    // otherwise each wave loads its fragments' weights into a register ring
    constexpr bool LDSW = FULL;
    constexpr int WSTAGE = LDSW ? RF_KC * EP * 4 : 0;   // W_r bytes of one stage
    constexpr int NWC = WSTAGE / 1024;                  // its 1 KiB copies
    constexpr int WCP = (NWC + 3) / 4;                  // per wave (past NWC: repeats)
    constexpr int XSTAGE = RF_TOK * 64;                 // token rows of one stage
    constexpr int STAGE = XSTAGE + WSTAGE;
    constexpr int WE = EB < 4 ? EB : 4;         // waves across expert blocks
    constexpr int WT = 4 / WE;                  // waves across the four token blocks
    constexpr int EBW = EB / WE, TBW = 4 / WT;  // blocks per wave
    constexpr int NWL = LDSW ? 0 : 8 * EBW;     // fp32 weight loads per wave per stage (8 k per fragment)
    constexpr int PER_STAGE = 1 + (LDSW ? WCP : NWL);   // loads per wave per stage
    constexpr int LROW = EP + 4;                // floats per token row of the logit tile
    constexpr int TILE = RF_TOK * LROW * 4;
    constexpr int LDS_BYTES = S * STAGE > TILE ? S * STAGE : TILE;
    static_assert(EB == 1 || EB == 2 || EB % 4 == 0, "expert blocks split evenly over the waves");
    static_assert(S >= 2 && PER_STAGE * (S - 1) < 64, "outstanding loads fit the counter");
    // one LDS object: stages (later the logit tile), then the bias and the
    // expert sums (with a second object the compiler could no longer tell that
    // the fragment reads need only the waited-for copies, and would wait for
    // all of them)
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES + 2 * EP * 4];
    float* bias = (float*)(lds + LDS_BYTES);
    float* red = bias + EP;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int we = wave / WT, wt = wave - we * WT;
    const int tbase = blockIdx.x * RF_TOK;
    const int nk = d / RF_KC;
    // the bias is fetched now and parked in LDS after the last stage
    const float b_mine = (b_r && (int)threadIdx.x < E) ? b_r[threadIdx.x] : 0.f;

    // token copy: wave w covers rows 16 w .. 16 w + 15; lane -> row 16 w + lane / 4,
    // LDS slot lane % 4, which holds 16-byte column slot ^ ((row >> 2) & 3)
    const int ntok = min(RF_TOK, T - tbase);
    const bf16_t* xw = x + (size_t)tbase * d;
    const uint32_t x_bytes = (uint32_t)ntok * d * 2;
    const int xr = wave * 16 + (lane >> 2);
    const uint32_t xvo = (uint32_t)(xr * d * 2 + (((lane & 3) ^ ((xr >> 2) & 3)) << 4));
    // weight fragment eb: expert (we * EBW + eb) * 16 + r16, rows k = 32 kk + 8 g + j of W_r
    const uint32_t w_bytes = (uint32_t)d * E * 4;
    const uint32_t w_stage = (uint32_t)RF_KC * E * 4;     // bytes of one K stage of W_r
    // LDS stage of W_r: 32 rows of EP floats; the 16-byte chunk c of row k sits at
    // c ^ wswz(k), so a fragment read (16 experts x rows 8 g + j, g = 0..3, one j)
    // falls on all 64 banks
    auto wswz = [](int k) { return (4 * ((k >> 3) & 3)) & (EP / 4 - 1); };
    uint32_t wvo[LDSW ? WCP : EBW], wdst[LDSW ? WCP : 1];
    if constexpr (LDSW) {
#pragma unroll
        for (int i = 0; i < WCP; ++i) {
            const int q = (wave * WCP + i) % NWC;   // copies past NWC repeat one (same bytes, same place)
            const int lin = q * 1024 + lane * 16;
            const int k = lin / (EP * 4), c = (lin - k * EP * 4) >> 4;
            wvo[i] = (uint32_t)(k * EP * 4 + ((c ^ wswz(k)) << 4));
            wdst[i] = (uint32_t)(XSTAGE + q * 1024);
        }
    } else {
#pragma unroll
        for (int eb = 0; eb < EBW; ++eb) {
            const int e = min((we * EBW + eb) * 16 + r16, E - 1);
            wvo[eb] = (uint32_t)((8 * g * E + e) * 4);
        }
    }
    float wreg[LDSW ? 1 : S][LDSW ? 1 : NWL];
    auto issue = [&](int kk, int stg, float (&wr)[LDSW ? 1 : NWL]) {
        kk = min(kk, nk - 1);
        copy_to_lds(buffer_rsrc(xw, x_bytes), lds + stg * STAGE + wave * 1024, xvo, kk * 64);
        if constexpr (LDSW) {
#pragma unroll
            for (int i = 0; i < WCP; ++i)
                copy_to_lds(buffer_rsrc(w_r, w_bytes), lds + stg * STAGE + wdst[i], wvo[i], kk * w_stage);
        } else {
#pragma unroll
            for (int eb = 0; eb < EBW; ++eb)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    wr[eb * 8 + j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        buffer_rsrc(w_r, w_bytes), wvo[eb] + (uint32_t)j * E * 4, kk * w_stage, 0));
        }
        // loads stay in step order (the waits count whole steps): neither the
        // optimizer nor the scheduler may move them past this point
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x4 acc[TBW][EBW];
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb)
#pragma unroll
        for (int eb = 0; eb < EBW; ++eb) acc[tb][eb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < S - 1; ++p) issue(p, p, wreg[LDSW ? 0 : p]);
    // whole rounds of S steps keep every load and the register ring
    // unconditional (steps past nk re-read the last stage and skip the MFMAs)
    // (d >= 32, so there is at least one round: no guard for the loads to sink past)
    const int nk_pad = (nk + S - 1) / S * S;
    int k0 = 0;
    do {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int kk = k0 + u;
            wait_copies<PER_STAGE * (S - 2)>();        // this wave's loads of step kk are done
            lds_barrier();                             // every wave's token copy too, and step kk - 1 is read out
            issue(kk + S - 1, (u + S - 1) % S, wreg[LDSW ? 0 : (u + S - 1) % S]);   // into the slots of step kk - 1
            if (kk < nk) {
                const char* sb = lds + u * STAGE;
                bf16x8 xb[TBW];
#pragma unroll
                for (int tb = 0; tb < TBW; ++tb) {
                    const int r = (wt * TBW + tb) * 16 + r16;
                    xb[tb] = as_bf16x8(*(const u32x4*)(sb + r * 64 + ((g ^ ((r >> 2) & 3)) << 4)));
                }
                // the three bf16 terms of each fragment, then the MFMAs with the
                // small terms first: lo, mid, hi
                float wv[EBW][8];
                if constexpr (LDSW) {   // rows 8 g + j of expert (we EBW + eb) 16 + r16, from the stage
                    const char* sw = sb + XSTAGE;
#pragma unroll
                    for (int eb = 0; eb < EBW; ++eb) {
                        const int e = (we * EBW + eb) * 16 + r16;
                        const char* base = sw + 8 * g * EP * 4 + ((((e >> 2) ^ wswz(8 * g)) << 2) + (e & 3)) * 4;
#pragma unroll
                        for (int j = 0; j < 8; ++j) wv[eb][j] = *(const float*)(base + j * EP * 4);
                    }
                } else {
#pragma unroll
                    for (int eb = 0; eb < EBW; ++eb)
#pragma unroll
                        for (int j = 0; j < 8; ++j) wv[eb][j] = wreg[LDSW ? 0 : u][eb * 8 + j];
                }
                uint32_t t3[3][EBW][4];
#pragma unroll
                for (int eb = 0; eb < EBW; ++eb)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        split3_bf16x2(wv[eb][2 * j], wv[eb][2 * j + 1], t3[0][eb][j], t3[1][eb][j], t3[2][eb][j]);
#pragma unroll
                for (int jj = 0; jj < 3; ++jj) {
                    const int term = 2 - jj;
#pragma unroll
                    for (int eb = 0; eb < EBW; ++eb) {
                        const bf16x8 a = as_bf16x8(
                            u32x4{t3[term][eb][0], t3[term][eb][1], t3[term][eb][2], t3[term][eb][3]});
#pragma unroll
                        for (int tb = 0; tb < TBW; ++tb)
                            acc[tb][eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[tb], acc[tb][eb], 0, 0, 0);
                    }
                }
            }
        }
        k0 += S;
    } while (k0 < nk_pad);
    wait_copies<0>();                                  // the clamped spare loads have landed
    lds_barrier();

    // logit tile: lane holds token 16 tb' + r16 and experts 16 eb' + 4 g + i
    float* tile = (float*)lds;
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb)
#pragma unroll
        for (int eb = 0; eb < EBW; ++eb)
            *(f32x4*)&tile[((wt * TBW + tb) * 16 + r16) * LROW + (we * EBW + eb) * 16 + 4 * g] = acc[tb][eb];
    if ((int)threadIdx.x < EP) bias[threadIdx.x] = b_mine;
    lds_barrier();

    // ------------------------------------------------------------ epilogue
    // wave w, lane (r16, g): token 16 w + r16, experts 16 eb + 4 g + i
    const int t = tbase + wave * 16 + r16;
    const float* trow = tile + (wave * 16 + r16) * LROW;
    float v[EB][4];
    float zc[KMAX > 1 ? EB : 1][4];
    float m = -INFINITY;
    int mi = 0x7fffffff;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
        const f32x4 z4 = *(const f32x4*)&trow[eb * 16 + 4 * g];
        const f32x4 b4 = *(const f32x4*)&bias[eb * 16 + 4 * g];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = eb * 16 + 4 * g + i;
            v[eb][i] = (FULL || e < E) ? z4[i] + b4[i] : -INFINITY;
            if constexpr (KMAX > 1) zc[eb][i] = v[eb][i];
            if (v[eb][i] > m) { m = v[eb][i]; mi = e; }
        }
    }
    // the 4 lane groups (g) hold the other experts of the same token
    {
        float om = lane_xor16(m);
        int oi = lane_xor16(mi);
        if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
        om = lane_xor32(m);
        oi = lane_xor32(mi);
        if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
    }
    if (logits_out && t < T) {
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = eb * 16 + 4 * g + i;
                if (FULL || e < E) logits_out[(size_t)t * E + e] = v[eb][i];
            }
    }
    float ssum = 0.f;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = eb * 16 + 4 * g + i;
            v[eb][i] = (FULL || e < E) ? rf_exp(v[eb][i] - m) : 0.f;
            ssum += v[eb][i];
        }
    ssum += lane_xor16(ssum);
    ssum += lane_xor32(ssum);
    const float inv = 1.0f / ssum;
    if (t < T && lane < 16) {
        expert[(size_t)t * k] = mi;
        gate[(size_t)t * k] = inv;
        lse[t] = m + logf(ssum);
    }
    if constexpr (KMAX > 1) {
        // choice r: the largest logit among the experts not yet chosen
        // (zc keeps the logits; v now holds the exponentials)
        int ch[KMAX];
        ch[0] = mi;
#pragma unroll
        for (int r = 1; r < KMAX; ++r) {
            if (r >= k) break;
            float mr = -INFINITY;
            int ir = 0x7fffffff;
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = eb * 16 + 4 * g + i;
                    bool taken = e >= E;
#pragma unroll
                    for (int q = 0; q < r; ++q) taken |= e == ch[q];
                    if (!taken && zc[eb][i] > mr) { mr = zc[eb][i]; ir = e; }
                }
            {
                float om = lane_xor16(mr);
                int oi = lane_xor16(ir);
                if (om > mr || (om == mr && oi < ir)) { mr = om; ir = oi; }
                om = lane_xor32(mr);
                oi = lane_xor32(ir);
                if (om > mr || (om == mr && oi < ir)) { mr = om; ir = oi; }
            }
            ch[r] = ir;
            if (t < T && lane < 16) {
                expert[(size_t)t * k + r] = ir;
                gate[(size_t)t * k + r] = rf_exp(mr - m) * inv;
            }
        }
    }
    // p_te summed over the 16 tokens of a lane group, then the waves in order
    const float w = t < T ? inv : 0.f;
    float psum[EB * 4];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) psum[eb * 4 + i] = v[eb][i] * w;
    row16_sum_all(psum);
    for (int ww = 0; ww < 4; ++ww) {
        if (wave == ww && r16 == 0) {
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = eb * 16 + 4 * g + i;
                    red[e] = (ww == 0) ? psum[eb * 4 + i] : red[e] + psum[eb * 4 + i];
                }
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < E; e += 256) part[(size_t)blockIdx.x * E + e] = red[e];
}

template <int KMAX>
static void fused_by_width(const bf16_t* x, const float* w_r, const float* b_r, int T, int d, int E, int k,
                           float* logits_out, int32_t* expert, float* gate, float* lse, float* part, hipStream_t s) {
// SL: stages with W_r through LDS (E a multiple of 16), SR: with the register ring
#define SWMOE_RF(EB, SL, SR)                                                                                    \
    do {                                                                                                        \
        if (E == 16 * (EB))                                                                                     \
            hipLaunchKernelGGL((router_fused<EB, SL, KMAX, true>), dim3(router_fused_blocks(T)), dim3(256), 0, s, \
                               x, w_r, b_r, T, d, E, k, logits_out, expert, gate, lse, part);                   \
        else                                                                                                    \
            hipLaunchKernelGGL((router_fused<EB, SR, KMAX, false>), dim3(router_fused_blocks(T)), dim3(256), 0, s, \
                               x, w_r, b_r, T, d, E, k, logits_out, expert, gate, lse, part);                   \
    } while (0)
    // (LDS stages sized so that two workgroups fit a CU)
    if (E <= 16) SWMOE_RF(1, 6, 4);
    else if (E <= 32) SWMOE_RF(2, 6, 4);
    else if (E <= 64) SWMOE_RF(4, 5, 4);
    else if (E <= 128) SWMOE_RF(8, 3, 3);
    else SWMOE_RF(16, 2, 2);   // register ring: 32 weight loads per wave per stage, one stage ahead
#undef SWMOE_RF
}

hipError_t launch_router_fused(const bf16_t* x, const float* w_r, const float* b_r, int T, int d, int E, int k,
                               float* logits_out, int32_t* expert, float* gate, float* lse, float* part,
                               hipStream_t s) {
    if (k <= 1) fused_by_width<1>(x, w_r, b_r, T, d, E, k, logits_out, expert, gate, lse, part, s);
    else if (k <= 2) fused_by_width<2>(x, w_r, b_r, T, d, E, k, logits_out, expert, gate, lse, part, s);
    else fused_by_width<kMaxTopK>(x, w_r, b_r, T, d, E, k, logits_out, expert, gate, lse, part, s);
    return hipGetLastError();
}

}  // namespace swmoe
