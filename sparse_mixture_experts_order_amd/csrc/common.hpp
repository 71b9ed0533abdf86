// Device-side helpers shared by the Switch FFN layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swmoe {

typedef uint16_t bf16_t;                                        // raw bf16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));      // MFMA A/B operand (8 x bf16)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte load/store unit (a native vector, kept in VGPRs)
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bf16 bits (low half) -> float, exactly
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 values rounded to bf16 (nearest, ties to even; NaN stays NaN) by
// one hardware conversion (v_cvt_pk_bf16_f32); a in the low half.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float bf16_lo_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// The exact three-term bf16 split of two fp32 values (a = hi + mid + lo
// exactly; Henry, Tang and Heinecke, ARITH 2019), each term a packed pair.
__device__ __forceinline__ void split3_bf16x2(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = pack_bf16x2(a, b);
    const float ra = a - bf16_lo_f32(hi), rb = b - bf16_hi_f32(hi);
    mid = pack_bf16x2(ra, rb);
    lo = pack_bf16x2(ra - bf16_lo_f32(mid), rb - bf16_hi_f32(mid));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// Largest value, lowest index among equal values.  (The test is bitwise, not
// short-circuit: no branch per step, the values move by selects.)
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(v, m);
        const int oi = __shfl_xor(i, m);
        const bool take = (ov > v) | ((ov == v) & (oi < i));
        v = take ? ov : v;
        i = take ? oi : i;
    }
}

// Map a linear block id to a logical tile id so that consecutive logical tiles
// run on the same XCD (the hardware deals workgroups round-robin over the 8
// XCDs, each with its own L2).  The grid is padded to a multiple of 8; the
// caller exits when the returned id is >= the real tile count.
__device__ __forceinline__ int xcd_swizzle(int bid, int grid_padded) {
    const int per_xcd = grid_padded >> 3;
    return (bid & 7) * per_xcd + (bid >> 3);
}

// Cross-lane moves that stay in the VALU (no LDS round trip).
// lane ^ 16 and lane ^ 32: the gfx950 row swaps, applied to two copies of v,
// return {v's even rows, v's odd rows} (or lower, upper halves) laid out so
// that each lane picks its partner's value.
__device__ __forceinline__ uint32_t lane_xor16(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ float lane_xor16(float v) { return __uint_as_float(lane_xor16(__float_as_uint(v))); }
__device__ __forceinline__ float lane_xor32(float v) { return __uint_as_float(lane_xor32(__float_as_uint(v))); }
__device__ __forceinline__ int lane_xor16(int v) { return (int)lane_xor16((uint32_t)v); }
__device__ __forceinline__ int lane_xor32(int v) { return (int)lane_xor32((uint32_t)v); }

// Sum over each row of 16 lanes, every lane of the row getting the sum: the
// partners lane ^ 1, ^ 2 (quad permutations), then the mirrored quad and the
// mirrored half row (DPP row_half_mirror, row_mirror), so the additions pair
// the same values in the same order as a butterfly over lane ^ 1, 2, 4, 8.
__device__ __forceinline__ float row16_sum(float v) {
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x141, 0xF, 0xF, false));  // half mirror
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x140, 0xF, 0xF, false));  // mirror
    return v;
}

// Largest value with the lowest index on ties over each row of 16 lanes, every
// lane of the row getting the result: the same four DPP partners as
// row16_sum.  The selection is a total order on (value desc, index asc), so
// any pairing gives the same result.
__device__ __forceinline__ void row16_argmax(float& v, int& i) {
#define SWMOE_ARGMAX_DPP(ctrl)                                                                                   \
    {                                                                                                           \
        const float ov = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), ctrl, 0xF, 0xF, false)); \
        const int oi = __builtin_amdgcn_update_dpp(0, i, ctrl, 0xF, 0xF, false);                                 \
        const bool take = (ov > v) | ((ov == v) & (oi < i));                                                    \
        v = take ? ov : v;                                                                                      \
        i = take ? oi : i;                                                                                      \
    }
    SWMOE_ARGMAX_DPP(0xB1)
    SWMOE_ARGMAX_DPP(0x4E)
    SWMOE_ARGMAX_DPP(0x141)
    SWMOE_ARGMAX_DPP(0x140)
#undef SWMOE_ARGMAX_DPP
}

// wave_sum and wave_argmax without the LDS path: rows of 16 by DPP, then the
// row swaps (lane ^ 16, lane ^ 32).  Every lane gets the result.
__device__ __forceinline__ float wave_sum_valu(float v) {
    v = row16_sum(v);
    v += lane_xor16(v);
    v += lane_xor32(v);
    return v;
}

__device__ __forceinline__ void wave_argmax_valu(float& v, int& i) {
    row16_argmax(v, i);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float ov = h ? lane_xor32(v) : lane_xor16(v);
        const int oi = h ? lane_xor32(i) : lane_xor16(i);
        const bool take = (ov > v) | ((ov == v) & (oi < i));
        v = take ? ov : v;
        i = take ? oi : i;
    }
}

// row16_sum on each element of an array, one step over all elements before
// the next (the same additions; independent instructions between dependent
// DPP moves instead of wait states)
template <int N>
__device__ __forceinline__ void row16_sum_all(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v[i]), 0xB1, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v[i]), 0x4E, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v[i]), 0x141, 0xF, 0xF, false));
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v[i]), 0x140, 0xF, 0xF, false));
}

// Token-tile list of the expert GEMMs, built by one workgroup of NT threads:
// pre[e] = number of valid TOK-row token tiles of experts < e (pre[E] = total
// V), and ttab[v] = {expert, first row, valid rows, w[e]} for v = pre[e] + tt,
// the token tiles of each expert in row order; without w the fourth word is
// the expert's number of token tiles.  accepted == NULL means every expert
// has all C rows.  The exclusive scan runs over the waves' prefix sums in wave
// order.
template <int NT>
__device__ void ffn_tile_list(const int32_t* __restrict__ accepted, int E, int C, int TOK, int32_t* __restrict__ pre,
                              int4* __restrict__ ttab, const int32_t* __restrict__ w = nullptr) {
    __shared__ int wsum[NT / 64];
    const int per = (E + NT - 1) / NT;
    const int e0 = threadIdx.x * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) local += (min(max(accepted ? accepted[e] : C, 0), C) + TOK - 1) / TOK;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    int run = base + incl - local;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            pre[e] = run;
            const int a = min(max(accepted ? accepted[e] : C, 0), C);
            const int we = w ? w[e] : (a + TOK - 1) / TOK;
            for (int tt = 0; tt * TOK < a; ++tt) ttab[run + tt] = make_int4(e, tt * TOK, min(TOK, a - tt * TOK), we);
            run += (a + TOK - 1) / TOK;
        }
    }
    if ((int)threadIdx.x == NT - 1) pre[E] = base + incl;
}

// Load-balancing statistics, one workgroup of NT threads, fp64 in a fixed
// order.  Routing groups: counts and prob_sum are [ngroups, E]; group g has G
// tokens and k choices per token, f_ge = counts_ge / (k G), P_ge = prob_sum_ge
// / G and the loss is alpha E times the mean over groups of sum_e f_ge P_ge
// (each thread adds the terms of columns i, i + NT, ... in order, then a fixed
// tree).  One group of T tokens with k = 1 is the Switch layer's loss.
struct AuxStatsArgs {
    const int32_t* counts; const float* prob_sum; int64_t G; int ngroups, E, k; float alpha;
    float* f; float* P; float* loss;
};

template <int NT>
__device__ void aux_stats_block(const AuxStatsArgs a) {
    __shared__ double red[NT];
    double acc = 0.0;
    const int64_t n = (int64_t)a.ngroups * a.E;
    for (int64_t i = threadIdx.x; i < n; i += NT) {
        const double fe = a.G > 0 ? (double)a.counts[i] / ((double)a.k * (double)a.G) : 0.0;
        const double pe = a.G > 0 ? (double)a.prob_sum[i] / (double)a.G : 0.0;
        a.f[i] = (float)fe;
        a.P[i] = (float)pe;
        acc += fe * pe;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = NT / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        a.loss[0] = a.ngroups > 0 ? (float)((double)a.alpha * (double)a.E * red[0] / (double)a.ngroups) : 0.f;
}

// Raw buffer descriptors.  The fourth word selects the 32-bit data format
// (unused by 16-byte loads, but a zero format is invalid); reads at or past
// the descriptor's byte count return zero.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, kBufferWord3);
}

// The same from values the compiler may have computed on the vector unit but
// that are uniform: each word goes through readfirstlane (as uint32_t: the
// builtin returns a signed int), so the descriptor stays scalar and the loads
// need no per-lane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc_uniform(const void* base, uint32_t nbytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane(nbytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                             kBufferWord3);
}

// Copies from memory straight into LDS.  A wave's copy instruction moves
// 64 x 16 bytes (lane i's 16 bytes land at dst + 16 i) and counts in vmcnt
// like any other load, so a wave waits for its own copies with wait_copies
// and then meets the other waves at an LDS-only barrier (the full barrier's
// memory fence would also wait for every copy still in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N_OUTSTANDING>
__device__ __forceinline__ void wait_copies() {
    static_assert(N_OUTSTANDING >= 0 && N_OUTSTANDING < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N_OUTSTANDING & 15) | ((N_OUTSTANDING >> 4) << 14) | 0x0F70);
}

// The XOR applied to the 16-byte slots of row k of a K-major LDS stage with
// rows of rbw bytes (a multiple of 128).  A half wave's transposed reads take
// 4 consecutive rows x 4 consecutive slots (the first a multiple of 4); the
// swizzle spreads those 16 pieces over all 64 four-byte banks: rows of a
// multiple of 256 bytes take XOR 4 (k & 3) (within 16-slot groups); rows of
// 256 m + 128 bytes already alternate between the two bank halves and take
// XOR 4 ((k >> 1) & 1) (within 8-slot groups).
__device__ __forceinline__ int kmajor_swz(int rbw, int k) {
    return (rbw & 255) ? 4 * ((k >> 1) & 1) : 4 * (k & 3);
}

// An MFMA operand fragment (8 consecutive k of one column) from a K-major
// LDS stage (rows k of rbw bytes, bf16), by two transposed reads
// (ds_read_b64_tr_b16): this lane's piece is row k (the group's rows k0 +
// lane / 4 of 16) and 4 elements from column col; the group's lanes get rows
// k0 .. k0 + 3 (first read) and k0 + 4 .. k0 + 7 (second) of their own
// column.  The 16-byte slot c of row k sits at c ^ kmajor_swz(rbw, k).
__device__ __forceinline__ bf16x8 kmajor_fragment(const char* st, int rbw, int k, int col) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const int slot = col >> 3, half = (col >> 2) & 1;
    const int k2 = k + 4;
    const char* p1 = st + k * rbw + ((slot ^ kmajor_swz(rbw, k)) << 4) + half * 8;
    const char* p2 = st + k2 * rbw + ((slot ^ kmajor_swz(rbw, k2)) << 4) + half * 8;
    v4s lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p1);
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p2);
#endif
    const u32x4 w = u32x4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                          (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                          (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                          (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
    return as_bf16x8(w);
}

// Cache policy of a load (the buffer instructions' auxiliary operand): kStream
// marks data read once (the non-temporal hint, `nt`), so that streaming it
// does not push out what is read again soon (L2 and the memory-side cache).
constexpr int kCached = 0, kStream = 2;

// One 1 KiB copy: lane i's 16 bytes land at dst + 16 i.  (The LDS address
// space exists only in the device pass.)
// The two LDS byte addresses of a kmajor_fragment (rows k and k + 4).
__device__ __forceinline__ void kmajor_addr(const char* st, int rbw, int k, int col, uint32_t& a1, uint32_t& a2) {
    const int slot = col >> 3, half = (col >> 2) & 1;
    const int k2 = k + 4;
    const char* p1 = st + k * rbw + ((slot ^ kmajor_swz(rbw, k)) << 4) + half * 8;
    const char* p2 = st + k2 * rbw + ((slot ^ kmajor_swz(rbw, k2)) << 4) + half * 8;
    a1 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p1;
    a2 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p2;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// N transposed 64-bit LDS reads (N = 2, 4 or 8: one, two or four K-major
// fragments) written out in asm, and their wait in the same block, so every
// output is complete when the block ends.  The compiler's wait insertion
// cannot tell a ds_read_b64_tr_b16 of the stage being read from the direct
// copies still in flight into the other stages, and so waits for all of them
// before the first such read; reads it does not see cost no such wait (the
// pipeline's own wait and barrier already order them after their copies).
// Outputs are early-clobber: a read's data may land before a later read of
// the block has taken its address.
template <int N>
__device__ __forceinline__ void lds_read_tr_batch(const uint32_t (&a)[N], u32x2 (&r)[N]) {
    static_assert(N == 2 || N == 4 || N == 8, "two, four or eight reads");
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (N == 2) {
        asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    } else if constexpr (N == 4) {
        asm volatile("ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %5\n\t"
                     "ds_read_b64_tr_b16 %2, %6\n\tds_read_b64_tr_b16 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    } else {
        asm volatile("ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
                     "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
                     "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
                     "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
                       "=&v"(r[7])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
                     : "memory");
    }
#else
    for (int i = 0; i < N; ++i) r[i] = u32x2{a[i], 0u};
#endif
}

// Fragment f of a batch: its rows k (read 2 f) and k + 4 (read 2 f + 1).
template <int N>
__device__ __forceinline__ bf16x8 batch_fragment(const u32x2 (&r)[N], int f) {
    return as_bf16x8(u32x4{r[2 * f].x, r[2 * f].y, r[2 * f + 1].x, r[2 * f + 1].y});
}

template <int AUX = kCached>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, AUX);
#endif
}

}  // namespace swmoe
