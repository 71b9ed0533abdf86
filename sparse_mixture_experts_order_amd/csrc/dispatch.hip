// Token-order slot scan and dispatch gather, with routing groups and top-k.
//
// Sources: "MoE routing load collapse" (zffjzz.top), "official code reading
// route": a token's slot is the running count of earlier tokens that chose the
// same expert (a cumulative sum along the sequence, not an ordering by
// probability), and the raw choice is kept apart from the capacity mask;
// "evaluation protocol": the capacity limit applies to each 64-row batch on
// its own.  "042 Switch Transformer" (wq-win.github.io) sec. 3: truncate the
// assignment by expert capacity, build the dispatch tensor, cast to bf16 and
// send tokens to their expert.  "Mixture of experts" (world.lapla.si), "full
// means turned back": with k choices per token the capacity scales with k.
//
// The scan runs over the T*k assignments (token t, choice i) in scan order:
// inside each routing group of G tokens either (t, i) lexicographic ("token"
// priority, the same as the [T, k] output layout) or (i, t) ("rank" priority:
// all first choices of the group before any second choice).  With k = 1 and
// one group this is the plain token order of the Switch layer.
//
// Three launches, no host synchronisation:
//   scan_local   per tile of 64*W assignments in scan order: each one's rank
//                among the earlier assignments of its tile with the same
//                expert (wave ballots for the match, then the tile's waves in
//                order through an LDS histogram), and the tile's per-expert
//                counts.  Tiles never straddle a group.
//   scan_offsets per expert: exclusive prefix of the tile counts over the
//                tiles of each group (a segmented scan); per group the raw
//                counts, accepted = min(counts, C), and the first buffer row
//                of the group (accepted rows of the earlier groups).
//   gather       per assignment: in-group position, keep flag, buffer row,
//                slot_token and the row copy x[t] -> buf[e, row]; extra
//                workgroups zero the empty rows.
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

// scan index j -> [T, k] output index, and back.  G: tokens per group, k:
// choices per token, rank: 1 for (i, t) order inside a group.
__device__ __forceinline__ int out_of_scan(int j, int k, int G, int rank) {
    if (!rank || k == 1) return j;
    const int Gk = G * k;
    const int g = j / Gk, r = j - g * Gk;
    const int i = r / G, u = r - i * G;
    return (g * G + u) * k + i;
}
__device__ __forceinline__ int scan_of_out(int o, int k, int G, int rank) {
    if (!rank || k == 1) return o;
    const int t = o / k, i = o - t * k;
    const int g = t / G, u = t - g * G;
    return g * G * k + i * G + u;
}

template <int W>
__global__ __launch_bounds__(64 * W) void scan_local(const int32_t* __restrict__ expert, int N, int E, int nbits,
                                                     int k, int G, int rank, int32_t* __restrict__ local_rank,
                                                     int32_t* __restrict__ tile_counts) {
    extern __shared__ int32_t hist[];  // [E]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = blockIdx.x * (64 * W) + threadIdx.x;
    for (int e = threadIdx.x; e < E; e += 64 * W) hist[e] = 0;

    // ids outside [0, E) are outside the contract: such assignments are not
    // counted and never dispatched (gather marks them dropped with position -1)
    const int o = j < N ? out_of_scan(j, k, G, rank) : 0;
    const int eid = j < N ? expert[o] : -1;
    const bool valid = eid >= 0 && eid < E;
    const int e = valid ? eid : 0;
    // lanes of this wave holding the same expert id ("match any")
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t set = __ballot(bit);
        peers &= bit ? set : ~set;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank_in_wave = __popcll(peers & lt);
    const int group = __popcll(peers);
    const bool leader = valid && rank_in_wave == 0;
    __syncthreads();
    // waves in scan order: read the running count, then the group leader adds the group size
    for (int w = 0; w < W; ++w) {
        if (wave == w && valid) local_rank[o] = hist[e] + rank_in_wave;
        if constexpr (W > 1) __syncthreads();
        if (wave == w && leader) hist[e] += group;
        if constexpr (W > 1) __syncthreads();
    }
    if constexpr (W == 1) __syncthreads();
    for (int i = threadIdx.x; i < E; i += 64 * W) tile_counts[(size_t)blockIdx.x * E + i] = hist[i];
}

// tile_counts[b][e] becomes the exclusive prefix over the earlier tiles of
// b's group (tpg tiles per group).  One wave per expert: lanes take 64 tiles
// at a time (the counts of 4 such chunks are loaded together); a segmented wave scan (shuffles, restarting at each group's
// first tile) ranks them and the open group's total carries into the next 64.
// At each group's last tile: counts, accepted = min(counts, C) and, with
// group_base, the group's first buffer row (a plain wave scan over the
// accepted counts of the groups that end in these 64 tiles).  rows_total[e]
// (optional) gets the accepted rows over all groups.
// With parts (the layer forward) the wave also sums its expert's column of the
// router's partial probability rows, prows rows per group, into prob_sum[g][e]
// (fp64): with one group the lanes take every 64th row in row order and the
// wave adds the lanes' sums in a fixed butterfly; with several groups lane l
// takes a group and adds its rows in order.
__device__ __forceinline__ void sum_prob_column(const float* __restrict__ parts, int prows, int ngroups, int E, int e,
                                                int lane, float* __restrict__ prob_sum) {
    if (ngroups == 1) {
        double s = 0.0;
        int r = lane;
        for (; r + 192 < prows; r += 256) {   // four loads in flight, added in row order
            const float v0 = parts[(size_t)r * E + e], v1 = parts[(size_t)(r + 64) * E + e];
            const float v2 = parts[(size_t)(r + 128) * E + e], v3 = parts[(size_t)(r + 192) * E + e];
            s += (double)v0;
            s += (double)v1;
            s += (double)v2;
            s += (double)v3;
        }
        for (; r < prows; r += 64) s += (double)parts[(size_t)r * E + e];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
        if (lane == 0) prob_sum[e] = (float)s;
        return;
    }
    for (int g0 = 0; g0 < ngroups; g0 += 64) {
        const int g = g0 + lane;
        if (g >= ngroups) break;
        const float* col = parts + (size_t)g * prows * E + e;
        double s = 0.0;
        int r = 0;
        for (; r + 3 < prows; r += 4) {
            const float v0 = col[(size_t)r * E], v1 = col[(size_t)(r + 1) * E];
            const float v2 = col[(size_t)(r + 2) * E], v3 = col[(size_t)(r + 3) * E];
            s += (double)v0;
            s += (double)v1;
            s += (double)v2;
            s += (double)v3;
        }
        for (; r < prows; ++r) s += (double)col[(size_t)r * E];
        prob_sum[(size_t)g * E + e] = (float)s;
    }
}

__global__ __launch_bounds__(256) void scan_offsets(int32_t* __restrict__ tile_counts, int ntiles, int tpg,
                                                    int ngroups, int E, int C, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ accepted, int32_t* __restrict__ group_base,
                                                    int32_t* __restrict__ rows_total, const float* __restrict__ parts,
                                                    int prows, float* __restrict__ prob_sum) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    if (parts) sum_prob_column(parts, prows, ngroups, E, e, lane, prob_sum);
    int run = 0;    // count of the open group over the earlier chunks
    int rows = 0;   // accepted rows of the finished groups
    constexpr int NB = 4;   // chunks of 64 tiles whose counts are loaded together
    int cb[NB];
    for (int b0 = 0; b0 < ntiles; b0 += 64) {
        const int q = (b0 >> 6) % NB;
        if (q == 0) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int bi = b0 + 64 * i + lane;
                cb[i] = bi < ntiles ? tile_counts[(size_t)bi * E + e] : 0;
            }
        }
        const int b = b0 + lane;
        const bool in = b < ntiles;
        const size_t o = (size_t)b * E + e;
        int c = cb[0];
#pragma unroll
        for (int i = 1; i < NB; ++i) c = q == i ? cb[i] : c;
        const int gi = b / tpg;
        const int head = (b - gi * tpg) == 0;
        const bool tail = in && ((b - gi * tpg) == tpg - 1 || b == ntiles - 1);
        int v = c, f = head;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int vu = __shfl_up(v, off);
            const int fu = __shfl_up(f, off);
            if (lane >= off && !f) { v += vu; f |= fu; }
        }
        const int incl = v + (f ? 0 : run);
        if (in) tile_counts[o] = incl - c;
        const int acc = tail ? min(incl, C) : 0;
        int a = acc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int au = __shfl_up(a, off);
            if (lane >= off) a += au;
        }
        if (tail) {
            counts[(size_t)gi * E + e] = incl;
            accepted[(size_t)gi * E + e] = acc;
            if (group_base) group_base[(size_t)gi * E + e] = rows + a - acc;
        }
        rows += __shfl(a, 63);
        run = __shfl((int)tail, 63) ? 0 : __shfl(incl, 63);
    }
    if (ntiles == 0 && lane == 0 && ngroups == 1) {   // no tokens, one group
        counts[e] = 0;
        accepted[e] = 0;
        if (group_base) group_base[e] = 0;
    }
    if (rows_total && lane == 0) rows_total[e] = rows;
}

// Workgroups [0, ntok_blocks) handle GATHER_TOK assignments each (in [T, k]
// order); the rest zero the empty rows, GATHER_ROWS rows each.  Buffer row of a
// kept assignment: group_base[g][e] + position (position alone with one group).
// With out_pass (k = 1, the combine done by the second expert GEMM) a dropped
// token's output row is written here: its residual x row bit for bit, or zeros
// without a residual.  With buf == NULL (the first expert GEMM gathers the
// token rows from x itself) no rows are copied or zeroed.  Each token-tile
// list asked for (tl0, tl1: the expert GEMMs' lists, built from the filled
// rows per expert by ffn_tile_list) takes one extra workgroup at the end of
// the grid, and with aux.prob_sum one more computes the load-balancing
// statistics (aux_stats_block; counts and prob_sum are final once the scan
// has run).
constexpr int GATHER_TOK = 16, GATHER_ROWS = 16;

__global__ __launch_bounds__(256) void gather(const bf16_t* __restrict__ x, const int32_t* __restrict__ expert,
                                              const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ group_base,
                                              const int32_t* __restrict__ rows_filled, int N, int d, int E, int k,
                                              int G, int rank, int tile, int C, int rows, int ntok_blocks,
                                              int32_t* __restrict__ position, uint8_t* __restrict__ keep,
                                              int32_t* __restrict__ slot, int32_t* __restrict__ slot_token,
                                              bf16_t* __restrict__ buf, bf16_t* __restrict__ out_pass,
                                              int pass_residual, const TileListOut tl0, const TileListOut tl1,
                                              const AuxStatsArgs aux) {
    const int nl = (tl0.pre ? 1 : 0) + (tl1.pre ? 1 : 0);
    if ((int)blockIdx.x >= (int)gridDim.x - nl) {   // the expert GEMMs' token-tile lists
        const TileListOut& t = ((int)blockIdx.x == (int)gridDim.x - 1 && tl0.pre) ? tl0 : tl1;
        ffn_tile_list<256>(rows_filled, E, rows, t.tok, t.pre, t.tab);
        return;
    }
    if (aux.prob_sum && (int)blockIdx.x == (int)gridDim.x - 1 - nl) {   // the load-balancing statistics
        aux_stats_block<256>(aux);
        return;
    }
    __shared__ int s_dst[GATHER_TOK];
    __shared__ int s_tok[GATHER_TOK];
    const int vpr = d >> 3;  // 16-byte vectors per row
    if ((int)blockIdx.x < ntok_blocks) {
        const int o0 = blockIdx.x * GATHER_TOK;
        if (threadIdx.x < GATHER_TOK) {
            const int o = o0 + threadIdx.x;
            int dst = -1, tok = 0;
            if (o < N) {
                const int e = expert[o];
                tok = o / k;
                if (e < 0 || e >= E) {
                    position[o] = -1;
                    keep[o] = 0;
                    if (slot) slot[o] = -1;
                } else {
                    const int j = scan_of_out(o, k, G, rank);
                    const int pos = offsets[(size_t)(j / tile) * E + e] + position[o];
                    const bool kp = pos < C;
                    int row = -1;
                    position[o] = pos;
                    keep[o] = kp;
                    if (kp) {
                        row = group_base ? group_base[(size_t)(tok / G) * E + e] + pos : pos;
                        dst = e * rows + row;
                        if (slot_token) slot_token[dst] = tok;
                    }
                    if (slot) slot[o] = row;
                }
            }
            // -1: nothing to copy; -2: a dropped token whose output row is written here
            s_dst[threadIdx.x] = (dst < 0 && o < N && out_pass) ? -2 : dst;
            s_tok[threadIdx.x] = tok;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < GATHER_TOK * vpr; i += 256) {
            const int r = i / vpr, v = i - r * vpr;
            const int dst = s_dst[r];
            if (dst == -1) continue;
            if (dst >= 0 && !buf) continue;
            if (dst == -2) {
                const uint4 val = pass_residual ? ((const uint4*)(x + (size_t)s_tok[r] * d))[v] : make_uint4(0, 0, 0, 0);
                ((uint4*)(out_pass + (size_t)s_tok[r] * d))[v] = val;
                continue;
            }
            const uint4 val = ((const uint4*)(x + (size_t)s_tok[r] * d))[v];
            ((uint4*)(buf + (size_t)dst * d))[v] = val;
        }
    } else {
        const int row0 = (blockIdx.x - ntok_blocks) * GATHER_ROWS;
        for (int i = threadIdx.x; i < GATHER_ROWS * vpr; i += 256) {
            const int r = i / vpr, v = i - r * vpr;
            const int row = row0 + r;
            if (row >= E * rows) break;
            const int e = row / rows, s = row - e * rows;
            if (s < rows_filled[e]) continue;
            ((uint4*)(buf + (size_t)row * d))[v] = make_uint4(0, 0, 0, 0);
            if (v == 0 && slot_token) slot_token[row] = -1;
        }
    }
}

// ------------------------------------------------------------------ launchers
int scan_tile(int64_t group_assignments, bool one_group) {
    if (one_group || group_assignments % 256 == 0) return 256;
    return group_assignments % 128 == 0 ? 128 : 64;
}
int scan_tiles(int64_t N, int tile) { return (int)((N + tile - 1) / tile); }

hipError_t launch_scan_local(const int32_t* expert, int N, int E, int k, int G, int rank, int tile,
                             int32_t* local_rank, int32_t* tile_counts, hipStream_t s) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const dim3 grid(scan_tiles(N, tile));
    const size_t shm = (size_t)E * sizeof(int32_t);
    if (tile == 256)
        hipLaunchKernelGGL(scan_local<4>, grid, dim3(256), shm, s, expert, N, E, nbits, k, G, rank, local_rank,
                           tile_counts);
    else if (tile == 128)
        hipLaunchKernelGGL(scan_local<2>, grid, dim3(128), shm, s, expert, N, E, nbits, k, G, rank, local_rank,
                           tile_counts);
    else
        hipLaunchKernelGGL(scan_local<1>, grid, dim3(64), shm, s, expert, N, E, nbits, k, G, rank, local_rank,
                           tile_counts);
    return hipGetLastError();
}

hipError_t launch_scan_offsets(int32_t* tile_counts, int ntiles, int tiles_per_group, int ngroups, int E, int C,
                               int32_t* counts, int32_t* accepted, int32_t* group_base, int32_t* rows_total,
                               const float* parts, int prows, float* prob_sum, hipStream_t s) {
    hipLaunchKernelGGL(scan_offsets, dim3((E + 3) / 4), dim3(256), 0, s, tile_counts, ntiles,
                       std::max(tiles_per_group, 1), ngroups, E, C, counts, accepted, group_base, rows_total, parts,
                       prows, prob_sum);
    return hipGetLastError();
}

hipError_t launch_gather(const bf16_t* x, const int32_t* expert, const int32_t* offsets, const int32_t* group_base,
                         const int32_t* rows_filled, int N, int d, int E, int k, int G, int rank, int tile, int C,
                         int rows, int32_t* position, uint8_t* keep, int32_t* slot, int32_t* slot_token, bf16_t* buf,
                         bf16_t* out_pass, bool pass_residual, const TileListOut& tl0, const TileListOut& tl1,
                         const AuxStatsArgs* aux, hipStream_t s) {
    const int ntok = (N + GATHER_TOK - 1) / GATHER_TOK;
    const int64_t nrows = buf ? (int64_t)E * rows : 0;
    const int nzero = (int)((nrows + GATHER_ROWS - 1) / GATHER_ROWS);
    const int nlist = (tl0.pre ? 1 : 0) + (tl1.pre ? 1 : 0) + (aux ? 1 : 0);
    if (ntok + nzero + nlist == 0) return hipSuccess;
    const AuxStatsArgs no_aux{};
    hipLaunchKernelGGL(gather, dim3(ntok + nzero + nlist), dim3(256), 0, s, x, expert, offsets, group_base, rows_filled, N, d,
                       E, k, std::max(G, 1), rank, tile, C, rows, ntok, position, keep, slot, slot_token, buf,
                       k == 1 ? out_pass : nullptr, pass_residual ? 1 : 0, tl0, tl1, aux ? *aux : no_aux);
    return hipGetLastError();
}

}  // namespace swmoe
