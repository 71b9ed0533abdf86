// Grouped expert GEMM on bf16 MFMA (v_mfma_f32_32x32x16_bf16), used twice:
//   H[e, s, :] = bf16(ReLU(buf[e, s, :] W1_e^T))     (N = d_ff, K = d)
//   Y[e, s, :] = H[e, s, :] W2_e^T                   (N = d,    K = d_ff), fp32
// for rows s < accepted[e].  The row counts stay on the device: a one-block
// kernel turns them into a prefix over experts of valid token tiles, and the
// GEMMs walk that list without any host synchronisation.
//
// Sources: "Switch Transformers ..." essay (dmxsf.com), "core structure":
// experts replace the FFN sublayer; "Mixture of experts" (world.lapla.si),
// "what is inside an expert": d -> d_ff with negatives set to zero -> d.
//
// Design for one MI355X.  At Switch-Base shapes an expert sees ~120 rows, so
// the layer is bound by streaming every expert's weights from HBM once, not
// by MFMA.  Both kernels here are organised around that stream: persistent
// workgroups (as many as fit on the chip) walk the tile list; a tile is (token
// block of TOK rows of one expert, weight-row block of NWG rows), ordered so
// the token tiles that read one weight block are neighbours, and dealt
// XCD-major so neighbours share an L2.
//   - expert_gemm_dma (every forward product, the first one on 320-row
//     "tall" token tiles where experts fill several 128-row tiles, and the
//     backward's products with 128-row token tiles): both operands of a
//     64-wide K chunk go from
//     memory straight into LDS stages by buffer loads with an LDS
//     destination, S - 1 chunks ahead of the MFMAs, one barrier per chunk;
//     no register holds data in flight.  Its notes are at the kernel.
//   - expert_gemm (the register kernel: the backward's products with 32- and
//     64-row token tiles): each wave owns 32*NBW weight rows of the tile and
//     computes them against all TOK token rows.  Weights never touch LDS:
//     each lane loads 64 contiguous bytes of its weight row per 64-wide K
//     chunk straight into registers.  The K order inside a chunk is permuted
//     identically for both operands (a reduction is order free), so a half
//     wave reads whole 64-byte runs.  Weights and token tiles flow through
//     rings of R register chunks, R-1 of them in flight, and the ring runs
//     across tile boundaries.  The token tile is shared by the waves through
//     LDS, double buffered, rows padded to 144 bytes so the MFMA-layout reads
//     are conflict free.  Token loads are issued before weight loads of the
//     same step: vector memory counters complete in issue order, so waiting
//     for a token chunk never waits for a weight chunk still ahead of the
//     MFMAs.
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

constexpr int FFN_LDS_STRIDE = 72;  // bf16 elements per token row in LDS (64 + 8 pad)

// Token-tile lists (ffn_tile_list) as a kernel of their own: block b builds list b.
__global__ __launch_bounds__(1024) void ffn_tile_prefix(const FfnTileLists L) {
    const FfnTileListSpec& t = L.list[blockIdx.x];
    ffn_tile_list<1024>(t.accepted, L.E, t.C, t.tok, t.pre, t.ttab, t.w);
}

struct FfnTile {
    int e, nt, tok_base, nv, w;
};

// Tile i of a GEMM over the list: token tile v, weight block nt.  The n_tiles
// * cnt tiles of an expert with cnt token tiles are consecutive, and inside
// them the order is weight block major (EM, the fourth word of the list's
// entries holding cnt): the token tiles that read one weight block are
// neighbours, so they run together on one XCD and read it once from memory
// (weight block minor, the tiles of one token tile share its token rows).
// With one token tile per expert the two orders are the same.  The table
// reads are uniform, so they go through the scalar cache and use no vector
// registers.
template <bool EM = false>
__device__ __forceinline__ FfnTile decode_tile(int i, const int4* __restrict__ ttab, int n_tiles, int TOK = 1) {
    const int v1 = __builtin_amdgcn_readfirstlane(i / n_tiles);
    int4 m = ttab[v1];
    int nt = i - v1 * n_tiles;
    if constexpr (EM) {
        const int cnt = __builtin_amdgcn_readfirstlane(m.w);
        if (cnt > 1) {
            const int p0 = v1 - __builtin_amdgcn_readfirstlane(m.y) / TOK;   // the expert's first token tile
            const int local = i - p0 * n_tiles;
            nt = __builtin_amdgcn_readfirstlane(local / cnt);
            m = ttab[p0 + local - nt * cnt];
        }
    }
    FfnTile t;
    t.e = __builtin_amdgcn_readfirstlane(m.x);
    t.tok_base = __builtin_amdgcn_readfirstlane(m.y);
    t.nv = __builtin_amdgcn_readfirstlane(m.z);
    t.w = __builtin_amdgcn_readfirstlane(m.w);
    t.nt = nt;
    return t;
}

// Output modes: bf16(ReLU(.)) (the first expert GEMM), fp32 (the second one,
// and the gradients that reuse this kernel), bf16 masked by a second array
// (the backward of the ReLU: zero wherever the saved activation is 0), and the
// second GEMM with the gate-scaled combine into the token rows (FfnCombine).
enum FfnOut { OUT_RELU_BF16 = 0, OUT_F32 = 1, OUT_MASK_BF16 = 2, OUT_COMBINE = 3 };

// Tile epilogue shared by the GEMM kernels.  Output rows go out through LDS in
// passes of CPP columns: the waves owning a pass park their results (lane:
// token column l32 of block tb, weight rows 8*(i/4) + 4*half + i%4), then the
// workgroup writes whole row segments with 16-byte stores.  `bar` is the
// workgroup barrier between the passes.
template <int TOKB, int NBW, int WAVES, int MODE, int PB>
struct FfnOutShape {
    static constexpr int TOK = 32 * TOKB;
    static constexpr int NWG = WAVES * 32 * NBW;
    static constexpr int OUT_BYTES = MODE != OUT_F32 ? 2 : 4;
    static constexpr int ROW_BYTES = NWG * OUT_BYTES;
    static constexpr int PASS_BYTES = ROW_BYTES <= PB ? ROW_BYTES
                                      : (ROW_BYTES % PB == 0 ? PB : (ROW_BYTES % (PB / 2) == 0 ? PB / 2 : PB / 4));
    static_assert(ROW_BYTES % PASS_BYTES == 0 && PASS_BYTES % 16 == 0, "whole 16-byte passes");
    static constexpr int NPASS = ROW_BYTES / PASS_BYTES;
    static constexpr int CPP = PASS_BYTES / OUT_BYTES;    // columns per pass
    static constexpr int OSTRIDE = PASS_BYTES + 16;       // bytes per staged row
    static constexpr int O_BYTES = TOK * OSTRIDE;
};

// What the combine epilogue reads besides the accumulators: the token of each
// of the lane's rows (-1 past the tile), its gate, and the residual runs of
// the lane's columns (two runs of 8 per 32-column block).
template <int TOKB, int NBW>
struct CombineInputs {
    int tok[TOKB];
    float g[TOKB];
    u32x4 rr[TOKB][NBW][2];
};

// Both loaders load unconditionally from clamped addresses and select after:
// a load under a branch makes the next wait a full one (every memory operation
// before it, the previous loads and stores included).
template <int TOKB, int NBW>
__device__ __forceinline__ void combine_load_tokens(CombineInputs<TOKB, NBW>& in, const FfnTile& t,
                                                    const FfnCombine& cb, int C, int l32) {
#pragma unroll
    for (int tb = 0; tb < TOKB; ++tb) {
        const int r = tb * 32 + l32;
        const int v = cb.slot_token[(size_t)t.e * C + min(t.tok_base + r, C - 1)];
        in.tok[tb] = r < t.nv ? v : -1;
    }
}

// (without a residual the runs are read from `out`, which has the same shape,
// and replaced by zeros)
template <int TOKB, int NBW>
__device__ __forceinline__ void combine_load_rows(CombineInputs<TOKB, NBW>& in, const FfnCombine& cb, int N, int n0,
                                                  int half) {
    const bf16_t* res = cb.residual ? cb.residual : cb.out;
#pragma unroll
    for (int tb = 0; tb < TOKB; ++tb) {
        const int tk = max(in.tok[tb], 0);
        in.g[tb] = cb.gate[tk];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const int n = n0 + nb * 32 + run * 16 + half * 8;
                in.rr[tb][nb][run] = *(const u32x4*)(res + (size_t)tk * N + min(n, N - 8));
            }
    }
    // every load is issued before the selects below use one (one wait for all)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < TOKB; ++tb) {
        const bool on = in.tok[tb] >= 0;
        in.g[tb] = on ? in.g[tb] : 0.f;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const int n = n0 + nb * 32 + run * 16 + half * 8;
                in.rr[tb][nb][run] = (on && cb.residual && n < N) ? in.rr[tb][nb][run] : u32x4{0u, 0u, 0u, 0u};
            }
    }
}

// Tile epilogue without LDS: each lane stores its accumulator values straight
// to memory; L2 merges the pieces into whole lines.  In the MFMA layout a lane
// holds, for one token, weight rows {0-3, 8-11, 16-19, 24-27} of a 32-row block
// (half wave 0) or {4-7, 12-15, 20-23, 28-31} (half wave 1).
//  - fp32 output: 4 consecutive columns (16 bytes) per store.
//  - bf16 outputs: swapping rows 8-11 of half 0 with rows 4-7 of half 1 (and
//    24-27 with 20-23; v_permlane32_swap) gives every lane two runs of 8
//    consecutive columns, so each store (and each residual load of the
//    combine mode) moves 16 bytes.  In the combine mode the row goes to its
//    token's output row (and y, if kept, gets the fp32 values).
template <int TOKB, int NBW, int WAVES, int MODE>
__device__ __forceinline__ void ffn_store_tile_direct(f32x16 (&acc)[NBW][TOKB], const FfnTile& t, void* out,
                                                      const bf16_t* mask, const FfnCombine& cb,
                                                      CombineInputs<TOKB, NBW>& in, int C, int N, int wave, int l32,
                                                      int half) {
    constexpr int NWG = WAVES * 32 * NBW;
    constexpr bool RUNS = MODE == OUT_RELU_BF16 || MODE == OUT_COMBINE || MODE == OUT_MASK_BF16;
    if constexpr (RUNS) {
        // lanes l and l ^ 32 hold the same token, so the swap is done by whole pairs
#pragma unroll
        for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(
                            __float_as_uint(acc[nb][tb][8 * pr + i]), __float_as_uint(acc[nb][tb][8 * pr + 4 + i]),
                            false, false);
                        acc[nb][tb][8 * pr + i] = __uint_as_float(sw[0]);
                        acc[nb][tb][8 * pr + 4 + i] = __uint_as_float(sw[1]);
                    }
    }
    const int n0 = t.nt * NWG + wave * 32 * NBW;   // first column of this wave
    if constexpr (MODE == OUT_COMBINE) {
        // the token rows, gates and residual runs are in `in` (every load
        // issued before the first store: a load issued after a store waits
        // for that store too); each output run replaces its residual run
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    const f32x16& a = acc[nb][tb];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t res = in.rr[tb][nb][run][j];
                        const float o0 = fmaf(in.g[tb], a[8 * run + 2 * j], bf16_to_f32(res & 0xffffu));
                        const float o1 = fmaf(in.g[tb], a[8 * run + 2 * j + 1], bf16_to_f32(res >> 16));
                        in.rr[tb][nb][run][j] = pack_bf16x2(o0, o1);
                    }
                    // the results are made here, in straight-line code: sunk into the
                    // stores' branches, each branch would wait for every memory operation
                    // before it, the previous stores included
                    asm volatile("" : "+v"(in.rr[tb][nb][run]));
                }
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb) {
                if (in.tok[tb] < 0) continue;
                const size_t orow = (size_t)in.tok[tb] * N;
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    const int n = n0 + nb * 32 + run * 16 + half * 8;
                    if (n < N) *(u32x4*)(cb.out + orow + n) = in.rr[tb][nb][run];
                }
            }
            if (cb.y) {
#pragma unroll
                for (int tb = 0; tb < TOKB; ++tb) {
                    if (in.tok[tb] < 0) continue;
                    const size_t row = ((size_t)t.e * C + t.tok_base + tb * 32 + l32) * N;
#pragma unroll
                    for (int run = 0; run < 2; ++run) {
                        const int n = n0 + nb * 32 + run * 16 + half * 8;
                        if (n >= N) continue;
                        const f32x16& a = acc[nb][tb];
                        *(f32x4*)(cb.y + row + n) = f32x4{a[8 * run + 0], a[8 * run + 1], a[8 * run + 2], a[8 * run + 3]};
                        *(f32x4*)(cb.y + row + n + 4) =
                            f32x4{a[8 * run + 4], a[8 * run + 5], a[8 * run + 6], a[8 * run + 7]};
                    }
                }
            }
        }
        return;
    }
    if constexpr (MODE == OUT_MASK_BF16) {
        // keep the elements whose saved activation is non-zero.  Every mask
        // run is loaded before the first store (a load issued after a store
        // waits for that store too), without branches: rows and columns past
        // the tile read the last valid run, whose result is never stored.
        u32x4 mk[NBW][TOKB][2];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    const int r = min(tb * 32 + l32, t.nv - 1);
                    const int n = min(n0 + nb * 32 + run * 16 + half * 8, N - 8);
                    mk[nb][tb][run] = *(const u32x4*)(mask + ((size_t)t.e * C + t.tok_base + r) * N + n);
                }
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    const f32x16& a = acc[nb][tb];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t m = mk[nb][tb][run][j];
                        const uint32_t keep = ((m & 0x7fffu) ? 0xffffu : 0u) | ((m & 0x7fff0000u) ? 0xffff0000u : 0u);
                        mk[nb][tb][run][j] =
                            pack_bf16x2(a[8 * run + 2 * j], a[8 * run + 2 * j + 1]) & keep;
                    }
                    // computed here, not inside each store's branch (one wait for the loads)
                    asm volatile("" : "+v"(mk[nb][tb][run]));
                }
#pragma unroll
        for (int tb = 0; tb < TOKB; ++tb) {
            const int r = tb * 32 + l32;
            if (r >= t.nv) continue;
            const size_t row = ((size_t)t.e * C + t.tok_base + r) * N;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    const int n = n0 + nb * 32 + run * 16 + half * 8;
                    if (n < N) *(u32x4*)((bf16_t*)out + row + n) = mk[nb][tb][run];
                }
        }
        return;
    }
#pragma unroll
    for (int tb = 0; tb < TOKB; ++tb) {
        const int r = tb * 32 + l32;
        if (r >= t.nv) continue;
        const size_t row = ((size_t)t.e * C + t.tok_base + r) * N;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const f32x16& a = acc[nb][tb];
            if constexpr (MODE == OUT_RELU_BF16) {
#pragma unroll
                for (int run = 0; run < 2; ++run) {
                    const int n = n0 + nb * 32 + run * 16 + half * 8;
                    if (n >= N) continue;
                    float v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = fmaxf(a[8 * run + j], 0.f);
                    *(u32x4*)((bf16_t*)out + row + n) =
                        u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                              pack_bf16x2(v[6], v[7])};
                }
            }
        }
    }
}

// v_permlane32_swap of rows 8-11 of half 0 with rows 4-7 of half 1 (and 24-27
// with 20-23) in one 32 x 32 accumulator block: each lane then holds two runs
// of 8 consecutive columns of its token.  The block is first copied into
// vector registers (the asm operand), so the accumulators themselves can stay
// in the accumulation registers through the K loop.
__device__ __forceinline__ f32x16 ffn_swapped_runs(const f32x16& acc) {
    f32x16 a = acc;
    asm volatile("" : "+v"(a));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[8 * pr + i]),
                                                             __float_as_uint(a[8 * pr + 4 + i]), false, false);
            a[8 * pr + i] = __uint_as_float(sw[0]);
            a[8 * pr + 4 + i] = __uint_as_float(sw[1]);
        }
    return a;
}

// Tall token tiles (the forward's first GEMM where experts fill more than one
// 128-row tile): the waves split the tile two ways, wave w taking the token
// blocks 2 i + (w & 1) (interleaved, so both halves have about as many valid
// blocks) against weight rows 32 NBW (w >> 1) .. + 32 NBW - 1; a tile is
// 16 NBW WAVES weight rows wide.  Its epilogue below takes the wave's TBW
// token blocks, acc[nb][i] holding block 2 i + tg.
template <int TOKB, int NBW, int WAVES>
constexpr int dma_tile_cols() {
    return TOKB > 4 ? WAVES * 32 * NBW / 2 : WAVES * 32 * NBW;
}

// bf16(ReLU) output of tall token tiles, one accumulator block at a time (the
// swap needs the block in vector registers, and all blocks do not fit there).
template <int TBW, int NBW>
__device__ __forceinline__ void ffn_store_tile_relu_tall(f32x16 (&acc)[NBW][TBW], const FfnTile& t, bf16_t* out,
                                                         int C, int N, int n0, int tg, int l32, int half) {
#pragma unroll
    for (int i = 0; i < TBW; ++i) {
        const int r = (2 * i + tg) * 32 + l32;
        const size_t row = ((size_t)t.e * C + t.tok_base + r) * N;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const f32x16 a = ffn_swapped_runs(acc[nb][i]);
#pragma unroll
            for (int run = 0; run < 2; ++run) {
                const int n = n0 + nb * 32 + run * 16 + half * 8;
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = fmaxf(a[8 * run + j], 0.f);
                const u32x4 o = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                      pack_bf16x2(v[6], v[7])};
                if (r < t.nv && n < N) *(u32x4*)(out + row + n) = o;
            }
        }
    }
}

// fp32 output as buffer stores: the descriptor ends with the tile's valid rows
// and columns past N get an offset past it, so every lane issues every store
// and a wave always issues exactly ffn_f32_stores<TOKB, NBW> of them (the next
// wait of the caller counts on that); out-of-range stores are dropped.
template <int TOKB, int NBW>
constexpr int ffn_f32_stores = TOKB * NBW * 4;

template <int TOKB, int NBW, int WAVES>
__device__ __forceinline__ void ffn_store_tile_f32(const f32x16 (&acc)[NBW][TOKB], const FfnTile& t, float* out,
                                                   int C, int N, int wave, int l32, int half) {
    constexpr int NWG = WAVES * 32 * NBW;
    const int n0 = t.nt * NWG + wave * 32 * NBW;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc_uniform(out + ((size_t)t.e * C + t.tok_base) * N, (uint32_t)max(t.nv, 0) * (uint32_t)N * 4u);
#pragma unroll
    for (int tb = 0; tb < TOKB; ++tb) {
        const int r = tb * 32 + l32;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const f32x16& a = acc[nb][tb];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + nb * 32 + q * 8 + half * 4;
                const uint32_t off = (r < t.nv && n < N) ? (uint32_t)(r * N + n) * 4u : 0x80000000u;
                const u32x4 v = u32x4{__float_as_uint(a[4 * q + 0]), __float_as_uint(a[4 * q + 1]),
                                      __float_as_uint(a[4 * q + 2]), __float_as_uint(a[4 * q + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
            }
        }
    }
}

template <int TOKB, int NBW, int WAVES, int MODE, int PB, class Bar>
__device__ __forceinline__ void ffn_store_tile(f32x16 (&acc)[NBW][TOKB], char* lds_o, const FfnTile& t, void* out,
                                               const bf16_t* mask, int C, int N, int wave, int l32, int half,
                                               Bar bar) {
    using Sh = FfnOutShape<TOKB, NBW, WAVES, MODE, PB>;
    constexpr int TOK = Sh::TOK, NWG = Sh::NWG, OUT_BYTES = Sh::OUT_BYTES, PASS_BYTES = Sh::PASS_BYTES;
    constexpr int NPASS = Sh::NPASS, CPP = Sh::CPP, OSTRIDE = Sh::OSTRIDE, NTHR = 64 * WAVES;
    const int ncols = min(NWG, N - t.nt * NWG);
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        if (pass > 0) bar();
        const int c0 = wave * 32 * NBW - pass * CPP;
        if (c0 >= 0 && c0 < CPP) {
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int c = c0 + nb * 32 + q * 8 + half * 4;
                        const f32x16& a = acc[nb][tb];
                        char* dst = lds_o + (tb * 32 + l32) * OSTRIDE + c * OUT_BYTES;
                        if constexpr (MODE == OUT_RELU_BF16) {
                            *(uint2*)dst = make_uint2(pack_bf16x2(fmaxf(a[4 * q + 0], 0.f), fmaxf(a[4 * q + 1], 0.f)),
                                                      pack_bf16x2(fmaxf(a[4 * q + 2], 0.f), fmaxf(a[4 * q + 3], 0.f)));
                        } else if constexpr (MODE == OUT_MASK_BF16) {
                            *(uint2*)dst = make_uint2(pack_bf16x2(a[4 * q + 0], a[4 * q + 1]),
                                                      pack_bf16x2(a[4 * q + 2], a[4 * q + 3]));
                        } else {
                            *(f32x4*)dst = f32x4{a[4 * q + 0], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                        }
                    }
        }
        bar();
        constexpr int VPR = PASS_BYTES / 16;           // 16-byte vectors per staged row
        const int vpr_valid = max(0, min(CPP, ncols - pass * CPP)) * OUT_BYTES / 16;
        char* gout = (char*)out + (((size_t)t.e * C + t.tok_base) * N + (size_t)t.nt * NWG + pass * CPP) * OUT_BYTES;
#pragma unroll
        for (int it = 0; it < (TOK * VPR + NTHR - 1) / NTHR; ++it) {
            const int i = threadIdx.x + it * NTHR;
            const int r = i / VPR, v = i - r * VPR;
            if (i < TOK * VPR && r < t.nv && v < vpr_valid) {
                u32x4 val = *(const u32x4*)(lds_o + r * OSTRIDE + v * 16);
                if constexpr (MODE == OUT_MASK_BF16) {
                    // keep the elements whose saved activation is non-zero
                    const size_t off = (size_t)(gout - (char*)out) + (size_t)r * N * OUT_BYTES + v * 16;
                    const u32x4 m = *(const u32x4*)((const char*)mask + off);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t keep_lo = (m[w] & 0x7fffu) ? 0xffffu : 0u;
                        const uint32_t keep_hi = (m[w] & 0x7fff0000u) ? 0xffff0000u : 0u;
                        val[w] &= keep_lo | keep_hi;
                    }
                }
                *(u32x4*)(gout + (size_t)r * N * OUT_BYTES + v * 16) = val;
            }
        }
    }
}

// TOKB: 32-row token blocks per tile; NBW: 32-row weight blocks per wave;
// WAVES: waves per workgroup; R: depth of the register rings; PB: bytes of an
// output row staged through LDS per pass; MODE: an FfnOut; WKM: the weights
// are stored K-major, W[e][k][n] (the backward's products with W1 and W2 as
// stored), instead of W[e][n][k].  K-major weight chunks are read as 64 k-rows
// of NWG contiguous columns, transposed 4 x 8 in registers and staged through
// LDS like the token tile.
template <int TOKB, int NBW, int WAVES, int R, int MODE, int PB, bool WKM = false>
__global__ __launch_bounds__(64 * WAVES) void expert_gemm(const bf16_t* __restrict__ A,   // [E, C, K]
                                                          const bf16_t* __restrict__ W,   // [E, N, K] or [E, K, N]
                                                          const int32_t* __restrict__ pre,
                                                          const int4* __restrict__ ttab,
                                                          void* __restrict__ out,         // [E, C, N]
                                                          const bf16_t* __restrict__ mask, // [E, C, N] (OUT_MASK_BF16)
                                                          int E, int C, int K, int N, int n_tiles) {
    constexpr int TOK = 32 * TOKB;
    constexpr int NWG = WAVES * 32 * NBW;
    constexpr int NTHR = 64 * WAVES;
    constexpr int PIECES = TOK * 8;                       // 16-byte pieces of one token chunk
    constexpr int APT = (PIECES + NTHR - 1) / NTHR;       // pieces per thread
    constexpr int A_BYTES = 2 * TOK * FFN_LDS_STRIDE * 2;
    constexpr int O_BYTES = FfnOutShape<TOKB, NBW, WAVES, MODE, PB>::O_BYTES;
    constexpr int W_BYTES = WKM ? 2 * NWG * FFN_LDS_STRIDE * 2 : 0;
    __shared__ __attribute__((aligned(16))) char lds_raw[A_BYTES + O_BYTES + W_BYTES];
    bf16_t* const lds_a = reinterpret_cast<bf16_t*>(lds_raw);
    char* const lds_o = lds_raw + A_BYTES;
    bf16_t* const lds_w = reinterpret_cast<bf16_t*>(lds_raw + A_BYTES + O_BYTES);   // [2][NWG][72] (WKM)
    static_assert(!WKM || 2 * NWG == NBW * NTHR, "K-major weights: NBW groups of 4 k x 8 n per thread");

    const int total = pre[E] * n_tiles;
    const int G = gridDim.x;                                          // a multiple of 8
    const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3); // XCD-major
    if (slot >= total) return;
    const int ntl = (total - slot + G - 1) / G;                       // tiles of this workgroup
    const int nk = K >> 6;
    const int P = ntl * nk;                                           // chunk positions

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, l32 = lane & 31;

    // Frontier tile (the one whose chunks are being loaded).  Loads go through
    // buffer descriptors (scalar registers) set once per tile: the per-lane
    // offsets never change, the chunk step is the scalar offset, and the
    // descriptor's byte count is the bound, so token rows past the tile's
    // valid rows (and weight rows past N) read as zero with no per-lane
    // clamping.  The loop therefore computes no per-lane addresses at all.
    int f_tile = -1;
    // descriptor fields, kept as scalars (a descriptor carried across the loop
    // would be taken for a per-lane value); the descriptors are rebuilt at use
    uint32_t a_lo = 0, a_hi = 0, a_n = 0, w_lo = 0, w_hi = 0, w_n = 0;
    // Every field comes from scalar arithmetic on uniform values, with no
    // min/max pairs or 64-bit compares: those become vector instructions, and
    // a vector temporary here would make the loop wait for the ring's loads.
    auto set_rsrc = [](const char* base, uint32_t nbytes, uint32_t& lo, uint32_t& hi, uint32_t& n) {
        const uint64_t b = (uint64_t)(uintptr_t)base;
        lo = (uint32_t)b;
        hi = (uint32_t)(b >> 32);
        n = nbytes;
    };
    auto rsrc = [](uint32_t lo, uint32_t hi, uint32_t n) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                                 kBufferWord3);
    };
    uint32_t woff[NBW];            // per lane: weight row nb*32 + l32, half-chunk `half`
                                   // (K-major: group nb's k-row 4 kq and columns 8 nq ..)
    uint32_t aoffg[APT];           // per lane: token row and 16-byte column of piece j
    int wcol[NBW];                 // K-major: first column 8 nq of group nb inside the tile
    int wlds[NBW];                 // K-major: LDS element offset of group nb's (column 8 nq, k 4 kq)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        if constexpr (WKM) {
            const int g = (int)threadIdx.x + nb * NTHR;
            const int kq = g / (NWG / 8), nq = g - kq * (NWG / 8);
            wcol[nb] = nq * 8;
            wlds[nb] = nq * 8 * FFN_LDS_STRIDE + kq * 4;
            woff[nb] = 0;
        } else {
            woff[nb] = ((uint32_t)(nb * 32 + l32) * K + half * 32) * 2;
        }
    }
#pragma unroll
    for (int j2 = 0; j2 < APT; ++j2) {
        const int q = min((int)threadIdx.x + j2 * NTHR, PIECES - 1);
        aoffg[j2] = ((uint32_t)(q >> 3) * K + (q & 7) * 8) * 2;
    }
    auto set_frontier = [&](int j) {
        f_tile = j;
        const FfnTile t = decode_tile(j * G + slot, ttab, n_tiles);
        const char* ab = (const char*)A + ((size_t)t.e * C + t.tok_base) * K * 2;
        set_rsrc(ab, (uint32_t)(t.nv * K * 2), a_lo, a_hi, a_n);
        if constexpr (WKM) {
            // columns past N read column group 0 and store nothing
            const int c0 = t.nt * NWG;
            set_rsrc((const char*)W + (size_t)t.e * K * N * 2, (uint32_t)(K * N * 2), w_lo, w_hi, w_n);
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int g = (int)threadIdx.x + nb * NTHR;
                const int kq = g / (NWG / 8);
                int col = c0 + wcol[nb];
                if (col >= N) col = 0;
                woff[nb] = ((uint32_t)(kq * 4) * N + col) * 2;
            }
        } else {
            // rows past N read zeros (the byte count ends at the expert's last
            // row); a wave whose first row is past N reads from row 0 and stores
            // nothing
            int wr0 = t.nt * NWG + wave * 32 * NBW;
            wr0 = wr0 < N ? wr0 : 0;
            set_rsrc((const char*)W + ((size_t)t.e * N + wr0) * K * 2, (uint32_t)((N - wr0) * K * 2), w_lo, w_hi,
                     w_n);
        }
    };
    int aoff[APT];
#pragma unroll
    for (int j2 = 0; j2 < APT; ++j2) {
        const int q = min((int)threadIdx.x + j2 * NTHR, PIECES - 1);
        aoff[j2] = (q >> 3) * FFN_LDS_STRIDE + (q & 7) * 8;
    }

    u32x4 areg[R][APT];
    u32x4 wreg[R][NBW][4];
    f32x16 acc[NBW][TOKB];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;

    // loads of position f (clamped to the last position) into one ring slot
    auto load_pos = [&](int f, u32x4 (&ar)[APT], u32x4 (&wr)[NBW][4]) {
        f = min(f, P - 1);
        const int jf = f / nk, kf = f - jf * nk;
        if (jf != f_tile) set_frontier(jf);
        const __amdgpu_buffer_rsrc_t rs_a = rsrc(a_lo, a_hi, a_n), rs_w = rsrc(w_lo, w_hi, w_n);
#pragma unroll
        for (int j2 = 0; j2 < APT; ++j2) ar[j2] = __builtin_amdgcn_raw_buffer_load_b128(rs_a, aoffg[j2], kf * 128, 0);
        if constexpr (WKM) {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int j2 = 0; j2 < 4; ++j2)   // k-rows 64 kf + 4 kq + j2
                    wr[nb][j2] = __builtin_amdgcn_raw_buffer_load_b128(rs_w, woff[nb], (kf * 64 + j2) * N * 2, 0);
        } else {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int j2 = 0; j2 < 4; ++j2)
                    wr[nb][j2] = __builtin_amdgcn_raw_buffer_load_b128(rs_w, woff[nb] + j2 * 16, kf * 128, 0);
        }
    };

    // K-major weights: group nb holds k-rows 4 kq .. 4 kq + 3 of columns 8 nq ..;
    // column n of it goes to LDS row n as 4 consecutive k values
    auto stage_w = [&](bf16_t* dstb, const u32x4 (&wr)[NBW][4]) {
        if constexpr (WKM) {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t r0 = wr[nb][0][w], r1 = wr[nb][1][w], r2 = wr[nb][2][w], r3 = wr[nb][3][w];
                    // columns 2w (low halves) and 2w + 1 (high halves)
                    const uint2 lo = make_uint2((r0 & 0xffffu) | (r1 << 16), (r2 & 0xffffu) | (r3 << 16));
                    const uint2 hi = make_uint2((r0 >> 16) | (r1 & 0xffff0000u), (r2 >> 16) | (r3 & 0xffff0000u));
                    *(uint2*)(dstb + wlds[nb] + (2 * w) * FFN_LDS_STRIDE) = lo;
                    *(uint2*)(dstb + wlds[nb] + (2 * w + 1) * FFN_LDS_STRIDE) = hi;
                }
        }
    };

#pragma unroll
    for (int p = 0; p < R - 1; ++p) load_pos(p, areg[p], wreg[p]);
#pragma unroll
    for (int j2 = 0; j2 < APT; ++j2) *(u32x4*)(lds_a + aoff[j2]) = areg[0][j2];
    stage_w(lds_w, wreg[0]);

    for (int p0 = 0; p0 < P; p0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int p = p0 + u;
            if (p < P) {
                const int slot_n = (u + R - 1) % R;   // constant once the u loop is unrolled
                load_pos(p + R - 1, areg[slot_n], wreg[slot_n]);
                __syncthreads();
                const bf16_t* lb = lds_a + (p & 1) * (TOK * FFN_LDS_STRIDE);
                const bf16_t* lw = lds_w + (p & 1) * (NWG * FFN_LDS_STRIDE) + (wave * 32 * NBW + l32) * FFN_LDS_STRIDE;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 bt[TOKB];
#pragma unroll
                    for (int tb = 0; tb < TOKB; ++tb)
                        bt[tb] = as_bf16x8(*(const u32x4*)(lb + (tb * 32 + l32) * FFN_LDS_STRIDE + half * 32 + s * 8));
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        bf16x8 wa;
                        if constexpr (WKM)
                            wa = as_bf16x8(*(const u32x4*)(lw + nb * 32 * FFN_LDS_STRIDE + half * 32 + s * 8));
                        else
                            wa = as_bf16x8(wreg[u][nb][s]);
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb)
                            acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt[tb], acc[nb][tb], 0, 0, 0);
                    }
                }
                // token chunk (and K-major weight chunk) of position p+1 into the other LDS buffer
                const int slot_a = (u + 1) % R;
                bf16_t* sb = lds_a + ((p + 1) & 1) * (TOK * FFN_LDS_STRIDE);
#pragma unroll
                for (int j2 = 0; j2 < APT; ++j2) *(u32x4*)(sb + aoff[j2]) = areg[slot_a][j2];
                stage_w(lds_w + ((p + 1) & 1) * (NWG * FFN_LDS_STRIDE), wreg[slot_a]);

                const int j = p / nk;
                if (p - j * nk == nk - 1) {
                    // ------------------------------------------------ tile epilogue
                    const FfnTile t = decode_tile(j * G + slot, ttab, n_tiles);
                    ffn_store_tile<TOKB, NBW, WAVES, MODE, PB>(acc, lds_o, t, out, mask, C, N, wave, l32, half,
                                                               [] { __syncthreads(); });
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                            for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Direct-to-LDS variant for 32-, 64-, 128- or 320-row token tiles with
// weights stored [N][K] (or [K][N], WKM).
// Both operands of a KC-wide K chunk (KC = 64 or 32) are copied from memory
// straight into an LDS stage by buffer loads with an LDS destination, so no
// registers hold data in flight and the copies run S - 1 chunks ahead of the
// MFMAs (the register rings above are limited by the register file to about
// three chunks); the narrower chunk fits more stages, i.e. more bytes in
// flight per CU, in the same LDS.  A copy instruction moves 1 KiB: 8 rows of
// 128 bytes or 16 rows of 64 bytes.  Its lanes fetch 16-byte columns
// XOR-swizzled by the row (column c of row r lands in slot c ^ ((r >> 1) & 7)
// of a 128-byte row, c ^ ((r >> 2) & 3) of a 64-byte row): a fragment read
// (32 consecutive rows at one column) serves 16 lanes at a time, and the
// swizzle puts any 16 consecutive rows on 16 different 16-byte bank groups,
// all 64 four-byte banks of gfx950's LDS (the row-only swizzles c ^ (r & 7)
// and c ^ ((r >> 1) & 3) cover 32 banks and halve the read rate).
// Rows past a tile's valid tokens, or past N, read as zero through the
// descriptors' byte counts.  One workgroup barrier per chunk: each wave waits
// for its own copies of chunk p (vmcnt), the LDS-only barrier then publishes
// every wave's copies and also certifies that all waves are done with chunk
// p - 1, whose stage the copies of chunk p + S - 1 refill right after.  (The
// standard barrier's memory fence would wait for every copy in flight.)  The
// tile's output goes straight from the accumulators to memory.
template <int KC>
__device__ __forceinline__ int dma_slot(int r, int c) {
    return KC == 64 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
}

// With a_rows the token rows are gathered straight from A = x [T, K]: row s of
// expert e is x[a_rows[e * C + s]] (a_bytes = T K 2, the descriptor's byte
// count; a_rows has kRowMapPad entries of padding past E C).  The row map is read with uniform (scalar) loads when a tile starts,
// so waiting for it never waits for the copies in flight; rows past the tile's
// valid count point past the descriptor and read as zero.
// With WKM the weights are stored K-major, [E, K, N] (the backward reads W1
// and W2 as stored): a chunk's stage holds KC rows k of NWG weights each, the
// 16-byte slot c of row k at c ^ kmajor_swz(row bytes, k), and an MFMA
// fragment (8 consecutive k of one weight row n per lane) is two
// ds_read_b64_tr_b16: in each 16-lane group, lane 4 j + a reads 4 weights of
// row k0 + j at columns n0 + 4 a .. + 3, and lane i gets the 4 rows k0 .. k0 +
// 3 of column n0 + i.
template <int TOKB, int NBW, int WAVES, int MODE, int S, int KC, bool WKM = false, bool AKM = false,
          int STREAM = 0>
__global__ __launch_bounds__(64 * WAVES) void expert_gemm_dma(const bf16_t* __restrict__ A,   // [E, C, K], x or [E, K, C]
                                                              const bf16_t* __restrict__ W,   // [E, N, K] or [E, K, N]
                                                              const int32_t* __restrict__ pre,
                                                              const int4* __restrict__ ttab,
                                                              void* __restrict__ out,
                                                              const bf16_t* __restrict__ mask,
                                                              const FfnCombine cb,
                                                              const int32_t* __restrict__ a_rows, uint32_t a_bytes,
                                                              int E, int C, int K, int N, int n_tiles,
                                                              int k_in_table, int kst) {
    static_assert(KC == 64 || KC == 32, "64- or 32-wide K chunks");
    static_assert(!AKM || WKM, "K-major token rows come with K-major weights");
    constexpr int TOK = 32 * TOKB;
    constexpr int NWG = dma_tile_cols<TOKB, NBW, WAVES>();
    constexpr int RB = KC * 2;                              // bytes per staged row
    constexpr int RPC = 1024 / RB;                          // rows per 1 KiB copy
    constexpr int NCOL = RB / 16;                           // 16-byte columns per row
    constexpr int W_COPIES = NWG / RPC;                     // copies per chunk
    constexpr int A_COPIES = TOK / RPC;
    static_assert(W_COPIES % WAVES == 0, "whole weight copies per wave");
    constexpr int WPW = W_COPIES / WAVES;
    constexpr int APW = (A_COPIES + WAVES - 1) / WAVES;     // the last copies of some waves are spares
    constexpr int W_STAGE = NWG * RB;
    constexpr int A_STAGE = APW * WAVES * 1024;             // token rows, then the spares' landing area
    constexpr int STAGE = W_STAGE + A_STAGE;
    constexpr int PER_CHUNK = WPW + APW;                    // copies per wave per chunk
    static_assert(S >= 2 && PER_CHUNK * (S - 1) < 64, "outstanding copies fit the counter");
    // tall token tiles (more than four 32-row blocks): the forward's products
    // where experts fill several 128-row tiles, one tile of up to 32 TOKB rows
    // per expert instead
    constexpr bool TALL = TOKB > 4;
    static_assert(!TALL || (!WKM && !AKM && TOKB % 2 == 0 && WAVES % 2 == 0 && MODE == OUT_RELU_BF16),
                  "tall token tiles: the first GEMM (row-major operands, bf16 ReLU output)");
    constexpr int TBW = TALL ? TOKB / 2 : TOKB;   // token blocks per wave
    __shared__ __attribute__((aligned(16))) char lds[S * STAGE];

    const int total = pre[E] * n_tiles;
    const int G = gridDim.x;                                          // a multiple of 8
    const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3); // XCD-major
    if (slot >= total) return;
    const int ntl = (total - slot + G - 1) / G;
    const int nk = K / KC;
    const int P = ntl * nk;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    const int tg = wave & 1, wn = wave >> 1;   // tall tiles: token half and weight slice of this wave

    // lane offsets of the copies (row RPC q + lane / NCOL, swizzled 16-byte column)
    uint32_t wvo[WPW], avo[APW];
    constexpr int RBW = NWG * 2;                            // bytes per K-major stage row
    constexpr int RBA = TOK * 2;
    static_assert(!WKM || (KC == 64 && RBW % 128 == 0), "K-major stages: 64-wide chunks, whole swizzle groups");
    static_assert(!AKM || RBA % 128 == 0, "K-major token stages: whole swizzle groups");
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        if constexpr (WKM) {
            const int lin = (wave * WPW + i) * 1024 + lane * 16;   // this lane's 16 bytes of the stage
            const int k = lin / RBW, slot = (lin - k * RBW) >> 4;
            wvo[i] = (uint32_t)k * N * 2 + ((slot ^ kmajor_swz(RBW, k)) << 4);
        } else {
            const int r = RPC * (wave * WPW + i) + lane / NCOL;
            wvo[i] = (uint32_t)r * K * 2 + (dma_slot<KC>(r, lane % NCOL) << 4);
        }
    }
#pragma unroll
    for (int i = 0; i < APW; ++i) {
        const int q = wave * APW + i;
        if constexpr (AKM) {
            const int lin = (q < A_COPIES ? q : 0) * 1024 + lane * 16;   // spares copy the first bytes again
            const int k = lin / RBA, sl = (lin - k * RBA) >> 4;
            avo[i] = (uint32_t)k * C * 2 + ((sl ^ kmajor_swz(RBA, k)) << 4);
        } else {
            const int r = RPC * (q < A_COPIES ? q : 0) + lane / NCOL;   // spares copy the first rows again
            avo[i] = (uint32_t)r * K * 2 + (dma_slot<KC>(r, lane % NCOL) << 4);
        }
    }

    int f_tile = -1;
    bool w_once = false;             // STREAM == 2: the frontier tile's expert has one token tile
    int c_tile = -1, c_nvb = TOKB;   // tall tiles: the computed tile and its valid token blocks
    uint32_t a_lo = 0, a_hi = 0, a_n = 0, w_lo = 0, w_hi = 0, w_n = 0;
    // K-major operands: the tile's valid K rows and the byte offset of its first column in a K row
    int kv = kst;
    uint32_t a_col = 0, w_col = 0;
    auto rsrc = [](uint32_t lo, uint32_t hi, uint32_t n) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                                 kBufferWord3);
    };
    // the descriptor of one 64-row K chunk of a K-major operand (rows of `row_bytes`,
    // tile base lo/hi): rows at or past kv, and the columns past the row's end in
    // the last valid row, read as zero
    // (the clamp and the byte count come out of vector instructions: readfirstlane
    // keeps the descriptor scalar, each word through uint32_t)
    auto kmajor_chunk = [&](uint32_t lo, uint32_t hi, int kf, uint32_t row_bytes, uint32_t col) {
        const uint64_t b = ((((uint64_t)hi << 32) | lo) + (uint64_t)kf * KC * row_bytes);
        const int vr = min(max(kv - kf * KC, 0), KC);
        const int n = vr * (int)row_bytes - (int)col;
        return rsrc((uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
                    (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)),
                    (uint32_t)__builtin_amdgcn_readfirstlane(n > 0 ? n : 0));
    };
    auto set_frontier = [&](int j) {
        f_tile = j;
        const FfnTile t = decode_tile<!AKM>(j * G + slot, ttab, n_tiles, TOK);
        if constexpr (STREAM == 2) w_once = t.w == 1;
        if (a_rows) {
            const uint64_t ab = (uint64_t)(uintptr_t)A;
            a_lo = (uint32_t)ab;
            a_hi = (uint32_t)(ab >> 32);
            a_n = a_bytes;
            const int32_t* rowp = a_rows + (size_t)t.e * C + t.tok_base;
            const int rl = lane / NCOL;
            // each copy's RPC row entries in one uniform load, all issued before any
            // is used (the map is padded by kRowMapPad entries, so a short last tile
            // reads past its rows harmlessly); readfirstlane keeps them scalar,
            // or the per-lane pick below becomes a vector load, whose wait would
            // also wait for the copies in flight
            int tk[APW][RPC];
#pragma unroll
            for (int i = 0; i < APW; ++i) {
                const int q = wave * APW + i;
                const int r0 = RPC * (q < A_COPIES ? q : 0);
#pragma unroll
                for (int u = 0; u < RPC; ++u) tk[i][u] = __builtin_amdgcn_readfirstlane(rowp[r0 + u]);
            }
#pragma unroll
            for (int i = 0; i < APW; ++i) {
                const int q = wave * APW + i;
                const int r0 = RPC * (q < A_COPIES ? q : 0);
                int mine = tk[i][0];
#pragma unroll
                for (int u = 1; u < RPC; ++u) mine = rl == u ? tk[i][u] : mine;
                // rows past the tile: past the end, zeros (a bitwise select, so no branch
                // sinks the uniform loads into lane-dependent code)
                const uint32_t valid = 0u - (uint32_t)(r0 + rl < t.nv);
                const uint32_t off = (((uint32_t)mine * K * 2) & valid) | (a_bytes & ~valid);
                avo[i] = off + (dma_slot<KC>(r0 + rl, lane % NCOL) << 4);
            }
        } else if constexpr (AKM) {   // columns past the tile only reach rows past C, never stored
            const uint64_t ab = (uint64_t)(uintptr_t)((const char*)A + ((size_t)t.e * kst * C + t.tok_base) * 2);
            a_lo = (uint32_t)ab;
            a_hi = (uint32_t)(ab >> 32);
            a_col = (uint32_t)t.tok_base * 2;
        } else {
            const uint64_t ab = (uint64_t)(uintptr_t)((const char*)A + ((size_t)t.e * C + t.tok_base) * K * 2);
            a_lo = (uint32_t)ab;
            a_hi = (uint32_t)(ab >> 32);
            a_n = (uint32_t)(t.nv * K * 2);
        }
        const int r0 = t.nt * NWG;                                   // rows past N read zeros
        if constexpr (WKM) {   // columns past N only reach outputs past N, never stored
            const uint64_t wb = (uint64_t)(uintptr_t)((const char*)W + ((size_t)t.e * kst * N + r0) * 2);
            w_lo = (uint32_t)wb;
            w_hi = (uint32_t)(wb >> 32);
            w_col = (uint32_t)r0 * 2;
            kv = k_in_table ? min(max(t.w, 0), kst) : kst;
        } else {
            const uint64_t wb = (uint64_t)(uintptr_t)((const char*)W + ((size_t)t.e * N + r0) * K * 2);
            w_lo = (uint32_t)wb;
            w_hi = (uint32_t)(wb >> 32);
            w_n = (uint32_t)((N - r0) * K * 2);
        }
    };
    // copies of chunk position f (clamped to the last one) into stage `stg`
    auto issue = [&](int f, int stg) {
        f = min(f, P - 1);
        // (the division runs on the vector unit: readfirstlane keeps the chunk, and
        // the descriptors built from it, scalar)
        const int jf = __builtin_amdgcn_readfirstlane(f / nk), kf = f - jf * nk;
        if (jf != f_tile) set_frontier(jf);
        const __amdgpu_buffer_rsrc_t rs_a = AKM ? kmajor_chunk(a_lo, a_hi, kf, (uint32_t)C * 2, a_col)
                                                : rsrc(a_lo, a_hi, a_n);
        const __amdgpu_buffer_rsrc_t rs_w = WKM ? kmajor_chunk(w_lo, w_hi, kf, (uint32_t)N * 2, w_col)
                                                : rsrc(w_lo, w_hi, w_n);
        char* sb = lds + stg * STAGE;
#pragma unroll
        for (int i = 0; i < WPW; ++i)
            if (STREAM == 1 || (STREAM == 2 && w_once))
                copy_to_lds<kStream>(rs_w, sb + (wave * WPW + i) * 1024, wvo[i], WKM ? 0u : kf * RB);
            else
                copy_to_lds<kCached>(rs_w, sb + (wave * WPW + i) * 1024, wvo[i], WKM ? 0u : kf * RB);
#pragma unroll
        for (int i = 0; i < APW; ++i)
            copy_to_lds(rs_a, sb + W_STAGE + (wave * APW + i) * 1024, avo[i], AKM ? 0u : kf * RB);
    };

    f32x16 acc[NBW][TBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int tb = 0; tb < TBW; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;

#pragma unroll
    for (int p = 0; p < S - 1; ++p) issue(p, p);

    CombineInputs<TOKB, NBW> cin;   // the combine epilogue's loads
    // fp32 output: right after a tile's stores, the wait for the next copies
    // lets those stores (a fixed number, issued after the copies) stay in flight
    constexpr int NST = MODE == OUT_F32 ? ffn_f32_stores<TBW, NBW> : 0;
    static_assert(PER_CHUNK * (S - 2) + NST < 64, "vmcnt range");
    bool stored = false;
    for (int p0 = 0; p0 < P; p0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int p = p0 + u;
            if (p < P) {
                if (MODE == OUT_F32 && stored) wait_copies<PER_CHUNK * (S - 2) + NST>();
                else wait_copies<PER_CHUNK * (S - 2)>();   // this wave's copies of position p are in LDS
                stored = false;
                lds_barrier();                           // every wave's too, and position p - 1 is read out
                issue(p + S - 1, (u + S - 1) % S);      // into the stage of position p - 1
                const char* sw = lds + u * STAGE;
                const char* sa = sw + W_STAGE;
                // K permuted identically for both operands: MFMA step s takes 16-byte
                // columns s (half 0) and KC / 32 + s (half 1) of the chunk
                if constexpr (TALL) {
                    // the valid 32-row token blocks of the tile this chunk belongs to
                    const int jc = __builtin_amdgcn_readfirstlane(p / nk);
                    if (jc != c_tile) {
                        c_tile = jc;
                        const FfnTile tc = decode_tile<true>(jc * G + slot, ttab, n_tiles, TOK);
                        c_nvb = __builtin_amdgcn_readfirstlane((tc.nv + 31) >> 5);
                    }
                    // one register set of token fragments, refilled as it is
                    // consumed: block i's fragment for step s + 1 is read right
                    // after the MFMAs of step s that use it (the weight fragments,
                    // used by all of the wave's blocks, take two sets); blocks past
                    // the valid rows hold zeros and get no MFMAs
                    auto tok_frag = [&](int s, int i) {
                        const int c = half * (KC / 16) + s;
                        const int r = (2 * i + tg) * 32 + l32;
                        return as_bf16x8(*(const u32x4*)(sa + r * RB + (dma_slot<KC>(r, c) << 4)));
                    };
                    auto w_frag = [&](int s, int nb) {
                        const int c = half * (KC / 16) + s;
                        const int r = wn * 32 * NBW + nb * 32 + l32;
                        return as_bf16x8(*(const u32x4*)(sw + r * RB + (dma_slot<KC>(r, c) << 4)));
                    };
                    bf16x8 fb[TBW], fw[2][NBW];
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) fw[0][nb] = w_frag(0, nb);
#pragma unroll
                    for (int i = 0; i < TBW; ++i) fb[i] = tok_frag(0, i);
#pragma unroll
                    for (int s = 0; s < KC / 16; ++s) {
                        if (s + 1 < KC / 16) {
#pragma unroll
                            for (int nb = 0; nb < NBW; ++nb) fw[(s + 1) & 1][nb] = w_frag(s + 1, nb);
                        }
#pragma unroll
                        for (int i = 0; i < TBW; ++i) {
                            if (2 * i + tg < c_nvb) {
#pragma unroll
                                for (int nb = 0; nb < NBW; ++nb)
                                    acc[nb][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s & 1][nb], fb[i],
                                                                                         acc[nb][i], 0, 0, 0);
                            }
                            if (s + 1 < KC / 16) fb[i] = tok_frag(s + 1, i);
                        }
                    }
                } else if constexpr (!AKM && !WKM) {
                    // row-major stages: the fragments of step s + 1 are read while
                    // the MFMAs of step s run (two register sets), so only the first
                    // step of a chunk waits for the LDS latency
                    bf16x8 fb[2][TOKB], fw[2][NBW];
                    auto read_step = [&](int s, bf16x8 (&bt)[TOKB], bf16x8 (&wv)[NBW]) {
                        const int c = half * (KC / 16) + s;
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb) {
                            const int r = tb * 32 + l32;
                            bt[tb] = as_bf16x8(*(const u32x4*)(sa + r * RB + (dma_slot<KC>(r, c) << 4)));
                        }
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb) {
                            const int r = wave * 32 * NBW + nb * 32 + l32;
                            wv[nb] = as_bf16x8(*(const u32x4*)(sw + r * RB + (dma_slot<KC>(r, c) << 4)));
                        }
                    };
                    read_step(0, fb[0], fw[0]);
#pragma unroll
                    for (int s = 0; s < KC / 16; ++s) {
                        if (s + 1 < KC / 16) read_step(s + 1, fb[(s + 1) & 1], fw[(s + 1) & 1]);
                        // the reads above are issued before these MFMAs
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                            for (int tb = 0; tb < TOKB; ++tb)
                                acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s & 1][nb], fb[s & 1][tb],
                                                                                      acc[nb][tb], 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
#pragma unroll
                for (int s = 0; s < KC / 16; ++s) {
                    const int c = half * (KC / 16) + s;
                    const int m = lane & 15;
                    bf16x8 bt[TOKB];
                    if constexpr (AKM) {   // rows k = 8 c .. 8 c + 7 of token column tb * 32 + (l & 31)
                        // two fragments per asm batch (fewer addresses live at once)
                        static_assert(TOKB % 2 == 0, "token fragments in pairs");
#pragma unroll
                        for (int tp = 0; tp < TOKB; tp += 2) {
                            uint32_t ta[4];
                            u32x2 tr[4];
#pragma unroll
                            for (int q = 0; q < 2; ++q)
                                kmajor_addr(sa, RBA, 8 * c + (m >> 2),
                                            (tp + q) * 32 + 16 * ((lane >> 4) & 1) + 4 * (m & 3), ta[2 * q],
                                            ta[2 * q + 1]);
                            lds_read_tr_batch(ta, tr);
                            bt[tp] = batch_fragment(tr, 0);
                            bt[tp + 1] = batch_fragment(tr, 1);
                        }
                    } else {
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb) {
                            const int r = tb * 32 + l32;
                            bt[tb] = as_bf16x8(*(const u32x4*)(sa + r * RB + (dma_slot<KC>(r, c) << 4)));
                        }
                    }
                    // K-major weights: rows k = 8 c .. 8 c + 7 of columns wave * 32 NBW + 32 nb + (l & 31)
                    u32x2 wtr[WKM ? 2 * NBW : 2];
                    if constexpr (WKM) {
                        static_assert(NBW == 1 || NBW == 2, "one or two K-major weight fragments per asm batch");
                        uint32_t wad[2 * NBW];
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
                            kmajor_addr(sw, RBW, 8 * c + (m >> 2),
                                        wave * 32 * NBW + nb * 32 + 16 * ((lane >> 4) & 1) + 4 * (m & 3), wad[2 * nb],
                                        wad[2 * nb + 1]);
                        lds_read_tr_batch(wad, wtr);
                    }
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        bf16x8 wa;
                        if constexpr (WKM) {
                            wa = batch_fragment(wtr, nb);
                        } else {
                            const int r = wave * 32 * NBW + nb * 32 + l32;
                            wa = as_bf16x8(*(const u32x4*)(sw + r * RB + (dma_slot<KC>(r, c) << 4)));
                        }
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb)
                            acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt[tb], acc[nb][tb], 0, 0, 0);
                    }
                }
                }

                const int j = p / nk;
                if (p - j * nk == nk - 1) {
                    const FfnTile t = decode_tile<!AKM>(j * G + slot, ttab, n_tiles, TOK);
                    if constexpr (MODE == OUT_COMBINE && !TALL) {
                        combine_load_tokens(cin, t, cb, C, l32);
                        combine_load_rows(cin, cb, N, t.nt * NWG + wave * 32 * NBW, half);
                    }
                    if constexpr (TALL) {
                        ffn_store_tile_relu_tall<TBW, NBW>(acc, t, (bf16_t*)out, C, N,
                                                           t.nt * NWG + wn * 32 * NBW, tg, l32, half);
                    } else if constexpr (MODE == OUT_F32) {
                        ffn_store_tile_f32<TOKB, NBW, WAVES>(acc, t, (float*)out, C, N, wave, l32, half);
                        stored = true;
                    } else {
                        ffn_store_tile_direct<TOKB, NBW, WAVES, MODE>(acc, t, out, mask, cb, cin, C, N, wave, l32,
                                                                      half);
                    }
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                        for (int tb = 0; tb < TBW; ++tb)
#pragma unroll
                            for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;
                }
            }
        }
    }
    wait_copies<0>();   // the clamped copies past the last chunk land before the workgroup ends
}

// ------------------------------------------------------------------ fused FFN, small capacity
// Both expert products in one kernel for experts of at most 64 buffer rows
// (one token tile of 32 or 64 rows; d a multiple of 256 up to 1024, d_ff a
// multiple of 256): the hidden activation H never goes to memory.  (Stores
// inside the weight stream cost far more than their bytes on this chip, and
// at these shapes H is as large as the layer output or larger.)  One
// workgroup of 8 waves per expert, persistent over the tile list, each
// expert's weights streamed once.  d_ff is taken in pieces of HB blocks of
// 256 columns; per piece:
//   phase 1, for each block of the piece: K = d in KC-wide chunks, a chunk
//     holding 256 W1 rows and the tile's TOK token rows (gathered from x
//     through the slot table; rows past the tile read as zero); after the
//     block's last chunk each wave writes bf16(ReLU(acc)) into the LDS piece
//     of H (TOK x 256 HB);
//   phase 2, for each block db of 256 output columns: K = the piece's
//     columns of d_ff, a chunk holding 256 W2 rows; the token operand comes
//     from H, and each wave adds into its accumulators of block db (the ND =
//     d / 256 accumulators stay in registers over the pieces, so H is never
//     needed whole).
// After the last piece the combine epilogue writes the kept tokens' output
// rows.  The copies run one pipeline over all chunks of all tiles, S LDS
// stages, one barrier per chunk.  Wave w owns weight rows 32 w .. 32 w + 31
// of each 256-row block against all TOK tokens.  In the H piece, within each
// 256-byte window of a row, the 16-byte slot s of row r sits at s ^ (r & 15),
// so the 16 rows of a fragment read cover all 64 banks.
constexpr int FS_NWG = 256, FS_WAVES = 8, FS_MAXND = 4;

// byte offset in an H piece of rows of `rb` bytes of the 16-byte slot s
// (columns 8 s .. 8 s + 7) of token row r
__device__ __forceinline__ int fs_h_slot(int r, int s, int rb) {
    return r * rb + (((s & ~15) | ((s & 15) ^ (r & 15))) << 4);
}

// wait_copies<BASE + n> for a uniform n in 0 .. MAXN
template <int BASE, int MAXN>
__device__ __forceinline__ void wait_copies_upto(int n) {
    if constexpr (MAXN == 0) {
        wait_copies<BASE>();
    } else {
        if (n >= MAXN) wait_copies<BASE + MAXN>();
        else wait_copies_upto<BASE, MAXN - 1>(n);
    }
}

template <int KC, int S, int HB, int ND, int TOKB>
__global__ __launch_bounds__(64 * FS_WAVES) void expert_ffn_fused(const bf16_t* __restrict__ x, uint32_t x_bytes,
                                                                  const int32_t* __restrict__ a_rows,
                                                                  const bf16_t* __restrict__ W1,
                                                                  const bf16_t* __restrict__ W2,
                                                                  const int32_t* __restrict__ pre,
                                                                  const int4* __restrict__ ttab, const FfnCombine cb,
                                                                  int E, int C, int F) {
    static_assert(KC == 64 || KC == 32, "64- or 32-wide K chunks");
    static_assert(ND >= 1 && ND <= FS_MAXND, "d = 256 ND");
    static_assert(TOKB == 1 || TOKB == 2, "32- or 64-row token tiles");
    constexpr int TOK = 32 * TOKB;
    constexpr int d = ND * FS_NWG;
    constexpr int RB = KC * 2;                     // bytes per staged row
    constexpr int RPC = 1024 / RB;                 // rows per 1 KiB copy
    constexpr int NCOL = RB / 16;                  // 16-byte slots per row
    constexpr int KS = KC / 16;                    // MFMA steps per chunk
    constexpr int WPW = FS_NWG / RPC / FS_WAVES;   // weight copies per wave per chunk
    constexpr int XCP = TOK / RPC;                 // token copies per chunk, one each by waves 0 .. XCP - 1
    static_assert(XCP <= FS_WAVES, "one token copy per wave at most");
    constexpr int W_STAGE = FS_NWG * RB;
    constexpr int STAGE = W_STAGE + TOK * RB;
    constexpr int HRB = HB * FS_NWG * 2;           // bytes per row of the H piece
    constexpr int NKD = d / KC;                    // chunks of a phase-1 block
    constexpr int NKH = HB * FS_NWG / KC;          // chunks of a phase-2 block (one piece)
    constexpr int PH1 = HB * NKD;                  // phase-1 chunks of a piece
    constexpr int PP = PH1 + ND * NKH;             // chunks of a piece
    static_assert(S >= 2 && (WPW + 1) * (S - 1) < 64, "outstanding copies fit the counter");
    __shared__ __attribute__((aligned(16))) char lds[S * STAGE + TOK * HRB];
    char* const hl = lds + S * STAGE;

    const int total = pre[E];
    const int G = gridDim.x;                                          // a multiple of 8
    const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3); // XCD-major
    if (slot >= total) return;
    const int ntl = (total - slot + G - 1) / G;
    const int npc = F / (HB * FS_NWG);   // pieces of a tile
    const int PE = npc * PP;             // chunks of a tile
    const int P = ntl * PE;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, l32 = lane & 31;

    // weight copy i of this wave: rows RPC (WPW wave + i) + lane / NCOL of the block
    uint32_t wvo1[WPW], wvo2[WPW];
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        const int r = RPC * (wave * WPW + i) + lane / NCOL;
        const uint32_t col = (uint32_t)(dma_slot<KC>(r, lane % NCOL) << 4);
        wvo1[i] = (uint32_t)r * d * 2 + col;
        wvo2[i] = (uint32_t)r * F * 2 + col;
    }
    // token copy (waves below XCP): tile rows RPC wave + lane / NCOL
    const bool has_x = wave < XCP;
    const int qt = has_x ? wave : 0;
    const int xr = RPC * qt + lane / NCOL;
    const uint32_t xcol = (uint32_t)(dma_slot<KC>(xr, lane % NCOL) << 4);
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc_uniform(x, x_bytes);

    // the copies' tile (ahead of the compute's by up to S - 1 chunks)
    int c_tile = -1, c_e = 0;
    uint32_t xo = 0;
    auto issue = [&](int f) {
        f = min(f, P - 1);   // past the end: the last chunk again (never read)
        const int j = __builtin_amdgcn_readfirstlane(f / PE);
        const int q = f - j * PE;
        if (j != c_tile) {
            c_tile = j;
            const FfnTile t = decode_tile(j * G + slot, ttab, 1, TOK);
            c_e = t.e;
            // this wave's RPC row-map entries, all issued as uniform loads before
            // any is used (the map is padded past its end), then the lane's own;
            // a per-lane load would be a vector load, whose wait would also wait
            // for the copies in flight
            const int32_t* rowp = a_rows + (size_t)t.e * C + t.tok_base + RPC * qt;
            int tk[RPC];
#pragma unroll
            for (int u = 0; u < RPC; ++u) tk[u] = __builtin_amdgcn_readfirstlane(rowp[u]);
            int mine = tk[0];
#pragma unroll
            for (int u = 1; u < RPC; ++u) mine = (lane / NCOL) == u ? tk[u] : mine;
            const uint32_t valid = 0u - (uint32_t)(xr < t.nv);
            xo = (((uint32_t)mine * (uint32_t)d * 2u) & valid) | (x_bytes & ~valid);   // past the end: reads zero
            xo += xcol;
        }
        const int pc = __builtin_amdgcn_readfirstlane(q / PP), qq = q - pc * PP;
        char* sb = lds + (f % S) * STAGE;
        if (qq < PH1) {
            const int fl = __builtin_amdgcn_readfirstlane(qq / NKD), kf = qq - fl * NKD;
            const __amdgpu_buffer_rsrc_t rw = buffer_rsrc_uniform(
                W1 + ((size_t)c_e * F + (size_t)(pc * HB + fl) * FS_NWG) * d, (uint32_t)FS_NWG * d * 2);
#pragma unroll
            for (int i = 0; i < WPW; ++i) copy_to_lds<kStream>(rw, sb + (wave * WPW + i) * 1024, wvo1[i], kf * RB);
            if (has_x) copy_to_lds(rx, sb + W_STAGE + qt * 1024, xo, kf * RB);
        } else {
            const int q2 = qq - PH1;
            const int db = __builtin_amdgcn_readfirstlane(q2 / NKH), kf = q2 - db * NKH;
            const __amdgpu_buffer_rsrc_t rw =
                buffer_rsrc_uniform(W2 + ((size_t)c_e * d + (size_t)db * FS_NWG) * F, (uint32_t)FS_NWG * F * 2);
#pragma unroll
            for (int i = 0; i < WPW; ++i)
                copy_to_lds<kStream>(rw, sb + (wave * WPW + i) * 1024, wvo2[i], (pc * NKH + kf) * RB);
        }
    };

    f32x16 acc1[TOKB];       // phase 1: this wave's 32 H columns of the block, per 32 tokens
    f32x16 acc2[ND][TOKB];   // phase 2: per output block, per 32 tokens
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc2[b][tb][i] = 0.f;
    const int r = wave * 32 + l32;   // this lane's weight row in a stage

    // chunk f is a phase-1 one
    auto phase1 = [&](int f) {
        const int qf = f % PE;
        return f < P && qf % PP < PH1;
    };
    // the next chunk p: wait for it, meet the other waves, send the copies
    // S - 1 chunks ahead; returns its stage
    int p = 0;
    auto next_chunk = [&]() -> const char* {
        // this wave's copies of chunk p are in: the copies issued after them,
        // those of chunks p + 1 .. p + S - 2, may still be in flight (WPW per
        // chunk, one more for a phase-1 chunk in waves with a token copy; the
        // clamped ones past the end repeat the last chunk, a phase-2 one)
        int n1 = 0;
#pragma unroll
        for (int i = 1; i <= S - 2; ++i) n1 += phase1(p + i) ? 1 : 0;
        wait_copies_upto<WPW * (S - 2), S - 2>(has_x ? __builtin_amdgcn_readfirstlane(n1) : 0);
        lds_barrier();   // every wave's; chunk p - 1 is read out, and the H writes before it are in
        issue(p + S - 1);
        const char* sw = lds + (p % S) * STAGE;
        ++p;
        return sw;
    };

#pragma unroll
    for (int f = 0; f < S - 1; ++f) issue(f);
    for (int jt = 0; jt < ntl; ++jt) {
        for (int pc = 0; pc < npc; ++pc) {
            // phase 1: the piece's H blocks
            for (int fl = 0; fl < HB; ++fl) {
#pragma unroll
                for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc1[tb][i] = 0.f;
                for (int kf = 0; kf < NKD; ++kf) {
                    const char* sw = next_chunk();
                    const char* sx = sw + W_STAGE;
#pragma unroll
                    for (int st = 0; st < KS; ++st) {
                        const int c = half * KS + st;
                        const bf16x8 wa = as_bf16x8(*(const u32x4*)(sw + r * RB + (dma_slot<KC>(r, c) << 4)));
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb) {
                            const int xrow = tb * 32 + l32;
                            const bf16x8 bt =
                                as_bf16x8(*(const u32x4*)(sx + xrow * RB + (dma_slot<KC>(xrow, c) << 4)));
                            acc1[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt, acc1[tb], 0, 0, 0);
                        }
                    }
                }
                // lane: token 32 tb + l32, piece columns 256 fl + 32 wave + 8 g + 4 half + (0..3)
                // from acc1[tb][4 g + (0..3)]
#pragma unroll
                for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int f0 = fl * FS_NWG + wave * 32 + 8 * g + 4 * half;
                        const f32x16& a = acc1[tb];
                        *(uint2*)(hl + fs_h_slot(tb * 32 + l32, f0 >> 3, HRB) + (f0 & 7) * 2) =
                            make_uint2(pack_bf16x2(fmaxf(a[4 * g + 0], 0.f), fmaxf(a[4 * g + 1], 0.f)),
                                       pack_bf16x2(fmaxf(a[4 * g + 2], 0.f), fmaxf(a[4 * g + 3], 0.f)));
                    }
            }
            // phase 2: every output block takes the piece's part of its sum
#pragma unroll
            for (int b = 0; b < ND; ++b) {
                for (int kf = 0; kf < NKH; ++kf) {
                    const char* sw = next_chunk();
#pragma unroll
                    for (int st = 0; st < KS; ++st) {
                        const int c = half * KS + st;
                        const bf16x8 wa = as_bf16x8(*(const u32x4*)(sw + r * RB + (dma_slot<KC>(r, c) << 4)));
#pragma unroll
                        for (int tb = 0; tb < TOKB; ++tb) {
                            const bf16x8 bt =
                                as_bf16x8(*(const u32x4*)(hl + fs_h_slot(tb * 32 + l32, kf * NCOL + c, HRB)));
                            acc2[b][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bt, acc2[b][tb], 0, 0, 0);
                        }
                    }
                }
            }
        }
        // the combine of every block
        FfnTile t = decode_tile(jt * G + slot, ttab, 1, TOK);
        CombineInputs<TOKB, 1> cin;
        combine_load_tokens(cin, t, cb, C, l32);
#pragma unroll
        for (int b = 0; b < ND; ++b) {
            t.nt = b;
            combine_load_rows(cin, cb, d, b * FS_NWG + wave * 32, half);
            f32x16 ab[1][TOKB];
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb) ab[0][tb] = acc2[b][tb];
            ffn_store_tile_direct<TOKB, 1, FS_WAVES, OUT_COMBINE>(ab, t, nullptr, nullptr, cb, cin, C, d, wave, l32,
                                                                  half);
#pragma unroll
            for (int tb = 0; tb < TOKB; ++tb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc2[b][tb][i] = 0.f;
        }
    }
    wait_copies<0>();   // the clamped copies past the last chunk land before the workgroup ends
}

// ------------------------------------------------------------------ launchers
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int TOKB, int NBW, int WAVES, int R, int MODE, int PB, bool WKM = false>
hipError_t launch_expert_gemm_t(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab, void* out,
                                const bf16_t* mask, int E, int C, int K, int N, hipStream_t s) {
    constexpr int NWG = WAVES * 32 * NBW;
    const int n_tiles = (N + NWG - 1) / NWG;
    static int per_cu = 0;   // resident workgroups per CU for this kernel
    if (!per_cu) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, expert_gemm<TOKB, NBW, WAVES, R, MODE, PB, WKM>, 64 * WAVES, 0) !=
                hipSuccess || b <= 0)
            b = 1;
        per_cu = b;
    }
    const int tok_tiles = (C + 32 * TOKB - 1) / (32 * TOKB);
    const int64_t max_tiles = (int64_t)E * n_tiles * tok_tiles;
    int64_t grid = std::min<int64_t>((int64_t)device_cus() * per_cu, (max_tiles + 7) / 8 * 8);
    grid = std::max<int64_t>(8, grid / 8 * 8);
    hipLaunchKernelGGL((expert_gemm<TOKB, NBW, WAVES, R, MODE, PB, WKM>), dim3((unsigned)grid), dim3(64 * WAVES), 0, s, A, W,
                       pre, ttab, out, mask, E, C, K, N, n_tiles);
    return hipGetLastError();
}

template <int TOKB, int NBW, int WAVES, int MODE, int S, int KC, bool WKM = false, bool AKM = false>
hipError_t launch_expert_gemm_dma_t(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab, void* out,
                                    const bf16_t* mask, const FfnCombine& cb, int E, int C, int K, int N,
                                    hipStream_t s, const int32_t* a_rows = nullptr, uint32_t a_bytes = 0,
                                    bool k_in_table = false, int kst = -1) {
    constexpr int NWG = dma_tile_cols<TOKB, NBW, WAVES>();
    const int n_tiles = (N + NWG - 1) / NWG;
    const int tok_tiles = (C + 32 * TOKB - 1) / (32 * TOKB);
    const int64_t max_tiles = (int64_t)E * n_tiles * tok_tiles;
    int64_t grid = std::min<int64_t>((int64_t)device_cus(), (max_tiles + 7) / 8 * 8);   // one workgroup per CU
    grid = std::max<int64_t>(8, grid / 8 * 8);
    // expert weights read by a single token tile per expert are streamed (read
    // once); with several token tiles they are read again and stay cached, so
    // where some experts may hold several, the policy follows each tile's
    // expert (the list entry's tile count); the K-major token-axis products' W
    // operand is an activation, read again too
    if constexpr (!AKM) {
        if (tok_tiles == 1) {
            hipLaunchKernelGGL((expert_gemm_dma<TOKB, NBW, WAVES, MODE, S, KC, WKM, AKM, 1>), dim3((unsigned)grid),
                               dim3(64 * WAVES), 0, s, A, W, pre, ttab, out, mask, cb, a_rows, a_bytes, E, C, K, N,
                               n_tiles, k_in_table ? 1 : 0, kst < 0 ? K : kst);
            return hipGetLastError();
        }
        if (!k_in_table) {
            hipLaunchKernelGGL((expert_gemm_dma<TOKB, NBW, WAVES, MODE, S, KC, WKM, AKM, 2>), dim3((unsigned)grid),
                               dim3(64 * WAVES), 0, s, A, W, pre, ttab, out, mask, cb, a_rows, a_bytes, E, C, K, N,
                               n_tiles, 0, kst < 0 ? K : kst);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((expert_gemm_dma<TOKB, NBW, WAVES, MODE, S, KC, WKM, AKM>), dim3((unsigned)grid), dim3(64 * WAVES),
                       0, s, A, W, pre, ttab, out, mask, cb, a_rows, a_bytes, E, C, K, N, n_tiles, k_in_table ? 1 : 0,
                       kst < 0 ? K : kst);
    return hipGetLastError();
}

int ffn_token_tile(int C) { return C > 64 ? 128 : (C > 32 ? 64 : 32); }

// Tall token tiles for the forward's first expert GEMM: when experts are
// expected to fill more than one 128-row tile, a tile holds up to 32 kTallTokB
// = 320 rows, so each (expert, weight block) is usually one tile.  Its
// weights are then staged once for all of the expert's rows instead of once
// per 128-row tile (whose copies of one weight block waited on a single HBM
// stream), and a staged byte feeds M N / (M + N) flop, 142 at 320 x 256
// against 102 at 128 x 512.  MFMAs of blocks past the valid rows are skipped.
// A 320 x 256 tile's 72 KiB chunk leaves room for one chunk in flight, so the
// copies bound it: where the token rows come from HBM (the second GEMM's H),
// or where there are too few tiles to fill the chip a few times over, the
// 128-row tiles stay (measured: Switch-Large shape, first GEMM 371 -> 307 us,
// second 384 -> 420 us tall; congested 64-expert shape, both slower tall).
int ffn_expected_fill(int64_t assignments, int E, int rows) {
    if (assignments <= 0 || E <= 0) return 0;
    return (int)std::min<int64_t>((assignments + E - 1) / E, rows);
}

int ffn_gemm1_token_tile(int E, int C, int fill, int d_ff) {
    const int rows = fill > 0 ? std::min(fill, C) : C;
    const int64_t tiles = (int64_t)E * ((d_ff + 255) / 256);
    if (C > 128 && rows > 128 && tiles >= 4 * (int64_t)device_cus()) return 32 * kTallTokB;
    return ffn_token_tile(C);
}

bool ffn_fused_ok(int C, int d, int d_ff) {
    return C >= 1 && C <= 64 && d % FS_NWG == 0 && d <= FS_MAXND * FS_NWG && d_ff % FS_NWG == 0;
}

template <int ND, int TOKB>
static hipError_t launch_expert_ffn_fused_t(const bf16_t* x, uint32_t x_bytes, const int32_t* slot_token,
                                            const bf16_t* w1, const bf16_t* w2, const int32_t* pre, const int4* ttab,
                                            const FfnCombine& cb, int E, int C, int d_ff, hipStream_t s) {
    int64_t grid = std::min<int64_t>((int64_t)device_cus(), ((int64_t)E + 7) / 8 * 8);   // one workgroup per CU
    grid = std::max<int64_t>(8, grid / 8 * 8);
    // 32-row tiles: pieces of two 256-column blocks of d_ff where they divide
    // it (fewer token-row reads), else one with a stage more; 64-row tiles:
    // pieces of one block, three stages
    if constexpr (TOKB == 1) {
        if ((d_ff / FS_NWG) % 2 == 0) {
            hipLaunchKernelGGL((expert_ffn_fused<64, 3, 2, ND, TOKB>), dim3((unsigned)grid), dim3(64 * FS_WAVES), 0, s,
                               x, x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d_ff);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((expert_ffn_fused<64, TOKB == 1 ? 4 : 3, 1, ND, TOKB>), dim3((unsigned)grid),
                       dim3(64 * FS_WAVES), 0, s, x, x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d_ff);
    return hipGetLastError();
}

template <int TOKB>
static hipError_t launch_expert_ffn_fused_nd(const bf16_t* x, uint32_t x_bytes, const int32_t* slot_token,
                                             const bf16_t* w1, const bf16_t* w2, const int32_t* pre, const int4* ttab,
                                             const FfnCombine& cb, int E, int C, int d, int d_ff, hipStream_t s) {
    switch (d / FS_NWG) {
        case 1: return launch_expert_ffn_fused_t<1, TOKB>(x, x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d_ff, s);
        case 2: return launch_expert_ffn_fused_t<2, TOKB>(x, x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d_ff, s);
        case 3: return launch_expert_ffn_fused_t<3, TOKB>(x, x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d_ff, s);
        default: return launch_expert_ffn_fused_t<4, TOKB>(x, x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d_ff, s);
    }
}

hipError_t launch_expert_ffn_fused(const bf16_t* x, int64_t T, const int32_t* slot_token, const bf16_t* w1,
                                   const bf16_t* w2, const int32_t* pre, const int4* ttab, const FfnCombine& cb,
                                   int E, int C, int d, int d_ff, hipStream_t s) {
    if (!ffn_fused_ok(C, d, d_ff) || T < 1) return hipErrorInvalidValue;
    const int64_t x_bytes = T * d * 2;
    if (x_bytes + 2 * (int64_t)d + 256 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    // the tile list holds one ffn_token_tile(C)-row tile per non-empty expert
    if (ffn_token_tile(C) == 32)
        return launch_expert_ffn_fused_nd<1>(x, (uint32_t)x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d, d_ff, s);
    return launch_expert_ffn_fused_nd<2>(x, (uint32_t)x_bytes, slot_token, w1, w2, pre, ttab, cb, E, C, d, d_ff, s);
}

size_t ffn_tile_table_entries(int E, int C) {
    const int tok = ffn_token_tile(C);
    return (size_t)E * ((C + tok - 1) / tok);
}

hipError_t launch_ffn_tile_lists(const FfnTileLists& L, int n, hipStream_t s) {
    if (n < 1 || n > kMaxTileLists) return hipErrorInvalidValue;
    FfnTileLists Lt = L;
    for (int i = 0; i < n; ++i)
        if (Lt.list[i].tok <= 0) Lt.list[i].tok = ffn_token_tile(Lt.list[i].C);
    hipLaunchKernelGGL(ffn_tile_prefix, dim3(n), dim3(1024), 0, s, Lt);
    return hipGetLastError();
}

#ifndef SWMOE_FFN_CUSTOM_DISPATCH
// Tile width for 128-row token tiles (the direct-to-LDS kernel).  Every
// workgroup streams NWG weight rows per tile, so a round of tiles over the
// persistent grid (one workgroup per CU) costs about NWG, and the kernel takes
// ceil(tiles / grid) rounds.  The width with the smallest rounds * NWG wins,
// the wider one on a tie (fewer, longer weight streams per workgroup); every
// expert's token tiles count as full.  E.g. at 128 experts, N = 768 takes 384
// columns (two tiles per expert, one round); N = 3072 and N = 4096 take 512.
// `narrow` restricts the choice to one 32-row block per wave: 256 or 192
// columns (8 or 6 waves), or 384 (12 waves) where `wide12`.
static int dma_tile_width(int E, int C, int N, bool narrow = false, bool wide12 = false) {
    const int64_t tok_tiles = (int64_t)E * ((C + 127) / 128);
    const int64_t grid = device_cus();
    int best = 0;
    int64_t best_cost = 0;
    for (const int nwg : {512, 384, 256, 192}) {
        if (narrow && nwg > 256 && !(wide12 && nwg == 384)) continue;
        const int64_t tiles = tok_tiles * ((N + nwg - 1) / nwg);
        const int64_t cost = (tiles + grid - 1) / grid * nwg;
        if (best == 0 || cost < best_cost) { best = nwg; best_cost = cost; }
    }
    return best;
}

// The direct-to-LDS kernel with 32- or 64-row token tiles (C <= 64: the
// forward's expert GEMMs, whose weight stream bounds them at these sizes), the
// column width chosen as for 128-row tiles.
template <int TOKB, int MODE>
static hipError_t launch_expert_gemm_dma_small(const bf16_t* A, const bf16_t* W, const int32_t* pre,
                                               const int4* ttab, void* out, const bf16_t* mask, int E, int C, int K,
                                               int N, hipStream_t s, const FfnCombine& cb, const int32_t* a_rows,
                                               uint32_t a_bytes) {
    if constexpr (MODE == OUT_COMBINE) {   // one 32-row block per wave, as with 128-row tiles
        if (dma_tile_width(E, C, N, true) == 256)
            return launch_expert_gemm_dma_t<TOKB, 1, 8, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s,
                                                                     a_rows, a_bytes);
        return launch_expert_gemm_dma_t<TOKB, 1, 6, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s, a_rows,
                                                                 a_bytes);
    } else {
        switch (dma_tile_width(E, C, N)) {
            case 512:
                return launch_expert_gemm_dma_t<TOKB, 2, 8, MODE, 2, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s,
                                                                         a_rows, a_bytes);
            case 384:
                return launch_expert_gemm_dma_t<TOKB, 2, 6, MODE, 2, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s,
                                                                         a_rows, a_bytes);
            case 256:
                return launch_expert_gemm_dma_t<TOKB, 1, 8, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s,
                                                                         a_rows, a_bytes);
            default:
                return launch_expert_gemm_dma_t<TOKB, 1, 6, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s,
                                                                         a_rows, a_bytes);
        }
    }
}

// forward: the forward's expert GEMMs, which take the direct-to-LDS kernel at
// every C (gathered token rows and the fused combine need it); otherwise
// C <= 64 keeps the register kernel (the backward's small products).
template <int MODE>
static hipError_t launch_expert_gemm(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab, void* out,
                                     const bf16_t* mask, int E, int C, int K, int N, hipStream_t s,
                                     const FfnCombine& cb = FfnCombine{}, const int32_t* a_rows = nullptr,
                                     uint32_t a_bytes = 0, bool forward = false, int fill = 0, int tok = 0) {
    // rows an expert is expected to fill (the tile shapes below depend on how
    // many 128-row token tiles it holds; the capacity alone overstates that
    // when most slots stay empty)
    const int rows = fill > 0 ? std::min(fill, C) : C;
    // the token tile must be the list's: tok rows (the forward's first GEMM
    // may take tall tiles), else ffn_token_tile(C)
    if constexpr (MODE == OUT_RELU_BF16) {
        if (forward && tok == 32 * kTallTokB)
            return launch_expert_gemm_dma_t<kTallTokB, 2, 8, MODE, 2, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N,
                                                                          s, a_rows, a_bytes);
    }
    if (tok == 32 * kTallTokB) return hipErrorInvalidValue;   // tall tiles: the first GEMM only
    if (C <= 64 && forward) {
        if (C <= 32)
            return launch_expert_gemm_dma_small<1, MODE>(A, W, pre, ttab, out, mask, E, C, K, N, s, cb, a_rows,
                                                         a_bytes);
        return launch_expert_gemm_dma_small<2, MODE>(A, W, pre, ttab, out, mask, E, C, K, N, s, cb, a_rows, a_bytes);
    }
    // a_rows (token rows gathered from x) needs the direct-to-LDS kernel
    if (a_rows && C <= 64) return hipErrorInvalidValue;
    if constexpr (MODE == OUT_COMBINE) {
        // one 32-row block per wave: the epilogue's residual runs fit in registers
        if (C <= 64) return hipErrorInvalidValue;   // the fused combine needs the direct-to-LDS kernel
        // 384 columns on 12 waves (three per SIMD, two stages) where experts
        // hold several token tiles: each tile's H rows are read by half as
        // many column tiles (measured faster there, slower with one token
        // tile per expert)
        if (dma_tile_width(E, C, N, true, rows > 128) == 384)
            return launch_expert_gemm_dma_t<4, 1, 12, MODE, 2, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s, a_rows,
                                                                   a_bytes);
        if (dma_tile_width(E, C, N, true) == 256)
            return launch_expert_gemm_dma_t<4, 1, 8, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s, a_rows, a_bytes);
        return launch_expert_gemm_dma_t<4, 1, 6, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s, a_rows, a_bytes);
    } else {
        if (C > 64) {
            // the first GEMM with one 128-row token tile per expert: 256
            // columns and three stages where the cost model allows them
            // (measured faster there than 512 columns and two stages; slower
            // with several token tiles per expert)
            if (MODE == OUT_RELU_BF16 && rows <= 128 && dma_tile_width(E, C, N, true) == 256)
                return launch_expert_gemm_dma_t<4, 1, 8, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N, s,
                                                                      a_rows, a_bytes);
            switch (dma_tile_width(E, C, N)) {
                case 512:
                    return launch_expert_gemm_dma_t<4, 2, 8, MODE, 2, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N,
                                                                          s, a_rows, a_bytes);
                case 384:
                    return launch_expert_gemm_dma_t<4, 2, 6, MODE, 2, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N,
                                                                          s, a_rows, a_bytes);
                case 256:
                    return launch_expert_gemm_dma_t<4, 1, 8, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N,
                                                                          s, a_rows, a_bytes);
                default:
                    return launch_expert_gemm_dma_t<4, 1, 6, MODE, 3, 64>(A, W, pre, ttab, out, mask, cb, E, C, K, N,
                                                                          s, a_rows, a_bytes);
            }
        }
        if (C > 32) return launch_expert_gemm_t<2, 2, 4, 3, MODE, 512>(A, W, pre, ttab, out, mask, E, C, K, N, s);
        return launch_expert_gemm_t<1, 2, 4, 4, MODE, 512>(A, W, pre, ttab, out, mask, E, C, K, N, s);
    }
}

// Register kernel with 128-row token tiles: 192 columns (6 waves) when that
// takes fewer rounds x columns over the grid than 256 (8 waves).
static bool narrow_tiles(int E, int C, int N) {
    const int64_t tok_tiles = (int64_t)E * ((C + 127) / 128);
    const int64_t grid = device_cus();
    auto cost = [&](int nwg) {
        const int64_t tiles = tok_tiles * ((N + nwg - 1) / nwg);
        return (tiles + grid - 1) / grid * nwg;
    };
    return cost(192) < cost(256);
}

// K-major weights (the register kernel): one configuration per token-tile
// size; the staged weight tile needs a 256-byte output pass to fit LDS next to it.
template <int MODE>
static hipError_t launch_expert_gemm_kmajor(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab,
                                            void* out, const bf16_t* mask, int E, int C, int K, int N, hipStream_t s) {
    if (C > 64) {   // the direct-to-LDS kernel with transposed fragment reads
        const FfnCombine none{};
        switch (dma_tile_width(E, C, N)) {
            case 512:
                return launch_expert_gemm_dma_t<4, 2, 8, MODE, 2, 64, true>(A, W, pre, ttab, out, mask, none, E, C, K, N,
                                                                            s);
            case 384:
                return launch_expert_gemm_dma_t<4, 2, 6, MODE, 2, 64, true>(A, W, pre, ttab, out, mask, none, E, C, K, N,
                                                                            s);
            case 256:
                return launch_expert_gemm_dma_t<4, 1, 8, MODE, 3, 64, true>(A, W, pre, ttab, out, mask, none, E, C, K, N,
                                                                            s);
            default:
                return launch_expert_gemm_dma_t<4, 1, 6, MODE, 3, 64, true>(A, W, pre, ttab, out, mask, none, E, C, K, N,
                                                                            s);
        }
    }
    if (C > 32) return launch_expert_gemm_t<2, 2, 4, 3, MODE, 512, true>(A, W, pre, ttab, out, mask, E, C, K, N, s);
    return launch_expert_gemm_t<1, 2, 4, 4, MODE, 512, true>(A, W, pre, ttab, out, mask, E, C, K, N, s);
}

hipError_t launch_expert_gemm1(const bf16_t* buf, const bf16_t* w1, const int32_t* pre, const int4* ttab, bf16_t* h,
                               int E, int C, int d, int d_ff, hipStream_t s, int fill) {
    return launch_expert_gemm<OUT_RELU_BF16>(buf, w1, pre, ttab, h, nullptr, E, C, d, d_ff, s, FfnCombine{}, nullptr,
                                             0, true, fill, ffn_gemm1_token_tile(E, C, fill, d_ff));
}

hipError_t launch_expert_gemm1_gather(const bf16_t* x, int64_t T, const int32_t* slot_token, const bf16_t* w1,
                                      const int32_t* pre, const int4* ttab, bf16_t* h, int E, int C, int d, int d_ff,
                                      hipStream_t s, int fill) {
    if (!ffn_rows_fused(C) || T * d * 2 + 2 * (int64_t)d + 256 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    return launch_expert_gemm<OUT_RELU_BF16>(x, w1, pre, ttab, h, nullptr, E, C, d, d_ff, s, FfnCombine{}, slot_token,
                                             (uint32_t)(T * d * 2), true, fill, ffn_gemm1_token_tile(E, C, fill, d_ff));
}

hipError_t launch_expert_gemm2(const bf16_t* h, const bf16_t* w2, const int32_t* pre, const int4* ttab, float* y,
                               int E, int C, int d, int d_ff, hipStream_t s, int fill) {
    return launch_expert_gemm<OUT_F32>(h, w2, pre, ttab, y, nullptr, E, C, d_ff, d, s, FfnCombine{}, nullptr, 0, true,
                                       fill);
}

bool ffn_wide_tiles(int C) { return C > 64; }
bool ffn_rows_fused(int C) { return C >= 1; }

hipError_t launch_expert_gemm2_combine(const bf16_t* h, const bf16_t* w2, const int32_t* pre, const int4* ttab,
                                       const FfnCombine& cb, int E, int C, int d, int d_ff, hipStream_t s, int fill) {
    if (!ffn_rows_fused(C)) return hipErrorInvalidValue;
    return launch_expert_gemm<OUT_COMBINE>(h, w2, pre, ttab, nullptr, nullptr, E, C, d_ff, d, s, cb, nullptr, 0, true,
                                           fill);
}

hipError_t launch_grouped_gemm_kmajor_f32(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab,
                                          float* out, int E, int rows, int K, int N, hipStream_t s) {
    return launch_expert_gemm_kmajor<OUT_F32>(A, W, pre, ttab, out, nullptr, E, rows, K, N, s);
}

hipError_t launch_grouped_gemm_kmajor_masked(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab,
                                             bf16_t* out, const bf16_t* mask, int E, int rows, int K, int N,
                                             hipStream_t s) {
    return launch_expert_gemm_kmajor<OUT_MASK_BF16>(A, W, pre, ttab, out, mask, E, rows, K, N, s);
}

// out[e] = A[e]^T W[e] with the token axis as K, both operands as stored:
// A [E, kst, M] and W [E, kst, N] bf16, out [E, M, N] fp32; rows k of expert
// e at or past the valid count in the fourth word of its tile entries read as
// zero.  The direct-to-LDS kernel with K-major stages for both operands
// (128-row tiles over M, so M > 64).
hipError_t launch_grouped_gemm_tn_f32(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab,
                                      float* out, int E, int M, int kst, int N, hipStream_t s) {
    if (!ffn_wide_tiles(M) || kst <= 0) return hipErrorInvalidValue;
    const int K = (kst + 63) / 64 * 64;
    const FfnCombine none{};
    switch (dma_tile_width(E, M, N)) {
        case 512:
            return launch_expert_gemm_dma_t<4, 2, 8, OUT_F32, 2, 64, true, true>(A, W, pre, ttab, out, nullptr, none, E,
                                                                              M, K, N, s, nullptr, 0, true, kst);
        case 384:
            return launch_expert_gemm_dma_t<4, 2, 6, OUT_F32, 2, 64, true, true>(A, W, pre, ttab, out, nullptr, none, E,
                                                                              M, K, N, s, nullptr, 0, true, kst);
        case 256:
            return launch_expert_gemm_dma_t<4, 1, 8, OUT_F32, 3, 64, true, true>(A, W, pre, ttab, out, nullptr, none, E,
                                                                              M, K, N, s, nullptr, 0, true, kst);
        default:
            return launch_expert_gemm_dma_t<4, 1, 6, OUT_F32, 3, 64, true, true>(A, W, pre, ttab, out, nullptr, none, E,
                                                                              M, K, N, s, nullptr, 0, true, kst);
    }
}

// Products whose output outweighs the weight stream (a short K, such as the
// token axis of the weight gradients) keep the register kernel, whose tile
// output leaves through LDS as whole 16-byte row segments.
hipError_t launch_grouped_gemm_f32(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab, float* out,
                                   int E, int rows, int K, int N, hipStream_t s) {
    if (rows > 64) {
        if (narrow_tiles(E, rows, N))
            return launch_expert_gemm_t<4, 1, 6, 3, OUT_F32, 256>(A, W, pre, ttab, out, nullptr, E, rows, K, N, s);
        return launch_expert_gemm_t<4, 1, 8, 4, OUT_F32, 512>(A, W, pre, ttab, out, nullptr, E, rows, K, N, s);
    }
    return launch_expert_gemm<OUT_F32>(A, W, pre, ttab, out, nullptr, E, rows, K, N, s);
}
#endif

}  // namespace swmoe
