// Token-order slot scan and dispatch gather.
//
// Sources: "MoE routing load collapse" (zffjzz.top), "official code reading
// route": a token's slot is the running count of earlier tokens that chose the
// same expert (a cumulative sum along the sequence, not an ordering by
// probability), and the raw choice is kept apart from the capacity mask;
// "042 Switch Transformer" (wq-win.github.io) sec. 3: truncate the assignment
// by expert capacity, build the dispatch tensor, cast to bf16 and send tokens
// to their expert.
//
// Three launches, no host synchronisation:
//   scan_local   per tile of 256 tokens: each token's rank among the earlier
//                tokens of its tile with the same expert (wave ballots for
//                the match, then the tile's waves in order through an LDS
//                histogram), and the tile's per-expert counts.
//   scan_offsets per expert: exclusive prefix of the tile counts over tiles;
//                raw counts and accepted = min(counts, C).
//   gather       per token: final position and keep flag, slot_token, and the
//                row copy x[t] -> buf[e, pos]; extra workgroups zero the empty
//                slots.
#include "common.hpp"
#include "kernels.hpp"

namespace swmoe {

constexpr int SCAN_TILE = 256;

__global__ __launch_bounds__(256) void scan_local(const int32_t* __restrict__ expert, int T, int E,
                                                  int nbits, int32_t* __restrict__ local_rank,
                                                  int32_t* __restrict__ tile_counts) {
    extern __shared__ int32_t hist[];  // [E]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * SCAN_TILE + threadIdx.x;
    for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;

    // ids outside [0, E) are outside the contract: such tokens are not counted
    // and never dispatched (gather marks them dropped with position -1)
    const int eid = t < T ? expert[t] : -1;
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
    // waves in token order: read the running count, then the group leader adds the group size
    for (int w = 0; w < 4; ++w) {
        if (wave == w && valid) {
            const int base = hist[e];
            local_rank[t] = base + rank_in_wave;
        }
        __syncthreads();
        if (wave == w && leader) hist[e] += group;
        __syncthreads();
    }
    for (int i = threadIdx.x; i < E; i += 256) tile_counts[(size_t)blockIdx.x * E + i] = hist[i];
}

// tile_counts[b][e] becomes the exclusive prefix over tiles b' < b.  One wave
// per expert: lanes take 64 tiles at a time, a wave prefix sum (shuffles)
// ranks them and the running total carries into the next 64.
__global__ __launch_bounds__(256) void scan_offsets(int32_t* __restrict__ tile_counts, int ntiles, int E,
                                                    int C, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ accepted) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    int run = 0;
    for (int b0 = 0; b0 < ntiles; b0 += 64) {
        const int b = b0 + lane;
        const size_t o = (size_t)b * E + e;
        const int c = b < ntiles ? tile_counts[o] : 0;
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        if (b < ntiles) tile_counts[o] = run + incl - c;
        run += __shfl(incl, 63);
    }
    if (lane == 0) {
        counts[e] = run;
        accepted[e] = min(run, C);
    }
}

// Workgroups [0, ntok_blocks) handle GATHER_TOK tokens each; the rest zero the
// empty slots, GATHER_ROWS slot rows each.
constexpr int GATHER_TOK = 16, GATHER_ROWS = 16;

__global__ __launch_bounds__(256) void gather(const bf16_t* __restrict__ x, const int32_t* __restrict__ expert,
                                              const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ accepted, int T, int d, int E, int C,
                                              int ntok_blocks, int32_t* __restrict__ position,
                                              uint8_t* __restrict__ keep, int32_t* __restrict__ slot_token,
                                              bf16_t* __restrict__ buf) {
    __shared__ int s_dst[GATHER_TOK];
    const int vpr = d >> 3;  // 16-byte vectors per row
    if ((int)blockIdx.x < ntok_blocks) {
        const int t0 = blockIdx.x * GATHER_TOK;
        if (threadIdx.x < GATHER_TOK) {
            const int t = t0 + threadIdx.x;
            int dst = -1;
            if (t < T && (expert[t] < 0 || expert[t] >= E)) {
                position[t] = -1;
                keep[t] = 0;
            } else if (t < T) {
                const int e = expert[t];
                const int pos = offsets[(size_t)(t / SCAN_TILE) * E + e] + position[t];
                const bool k = pos < C;
                position[t] = pos;
                keep[t] = k;
                if (k) {
                    dst = e * C + pos;
                    if (slot_token) slot_token[dst] = t;
                }
            }
            s_dst[threadIdx.x] = dst;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < GATHER_TOK * vpr; i += 256) {
            const int r = i / vpr, v = i - r * vpr;
            const int dst = s_dst[r];
            if (dst < 0) continue;
            const uint4 val = ((const uint4*)(x + (size_t)(t0 + r) * d))[v];
            ((uint4*)(buf + (size_t)dst * d))[v] = val;
        }
    } else {
        const int row0 = (blockIdx.x - ntok_blocks) * GATHER_ROWS;
        for (int i = threadIdx.x; i < GATHER_ROWS * vpr; i += 256) {
            const int r = i / vpr, v = i - r * vpr;
            const int row = row0 + r;
            if (row >= E * C) break;
            const int e = row / C, s = row - e * C;
            if (s < accepted[e]) continue;
            ((uint4*)(buf + (size_t)row * d))[v] = make_uint4(0, 0, 0, 0);
            if (v == 0 && slot_token) slot_token[row] = -1;
        }
    }
}

// ------------------------------------------------------------------ launchers
int scan_tiles(int64_t T) { return (int)((T + SCAN_TILE - 1) / SCAN_TILE); }

hipError_t launch_scan_local(const int32_t* expert, int T, int E, int32_t* local_rank, int32_t* tile_counts,
                             hipStream_t s) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipLaunchKernelGGL(scan_local, dim3(scan_tiles(T)), dim3(256), (size_t)E * sizeof(int32_t), s, expert, T,
                       E, nbits, local_rank, tile_counts);
    return hipGetLastError();
}

hipError_t launch_scan_offsets(int32_t* tile_counts, int ntiles, int E, int C, int32_t* counts,
                               int32_t* accepted, hipStream_t s) {
    hipLaunchKernelGGL(scan_offsets, dim3((E + 3) / 4), dim3(256), 0, s, tile_counts, ntiles, E, C, counts,
                       accepted);
    return hipGetLastError();
}

hipError_t launch_gather(const bf16_t* x, const int32_t* expert, const int32_t* offsets, const int32_t* accepted,
                         int T, int d, int E, int C, int32_t* position, uint8_t* keep, int32_t* slot_token,
                         bf16_t* buf, hipStream_t s) {
    const int ntok = (T + GATHER_TOK - 1) / GATHER_TOK;
    const int64_t rows = (int64_t)E * C;
    const int nzero = (int)((rows + GATHER_ROWS - 1) / GATHER_ROWS);
    if (ntok + nzero == 0) return hipSuccess;
    hipLaunchKernelGGL(gather, dim3(ntok + nzero), dim3(256), 0, s, x, expert, offsets, accepted, T, d, E, C,
                       ntok, position, keep, slot_token, buf);
    return hipGetLastError();
}

}  // namespace swmoe
