// Host-side launchers of the device kernels (one per kernel; each enqueues on
// the given stream and returns hipGetLastError()).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace swmoe {
typedef uint16_t bf16_t;
struct AuxStatsArgs;   // common.hpp

// route.hip
hipError_t launch_split_router_weights(const float* w_r, bf16_t* wr3, int d, int E, hipStream_t s);
hipError_t launch_router_gemm(const bf16_t* x, const bf16_t* wr3, const float* b_r, float* logits, int T, int d,
                              int E, hipStream_t s);
constexpr int kMaxTopK = 4;             // largest k the routers support
int router_softmax_blocks(int64_t T, int E);
int router_softmax_blocks_grouped(int64_t T);   // one partial row per 64 tokens
hipError_t launch_router_softmax(const float* logits, int T, int E, int k, bool rows_of_64, int32_t* expert,
                                 float* gate, float* lse, float* part, hipStream_t s);
hipError_t launch_router_reduce(const float* part, int nblk, int ngroups, int E, float* prob_sum, hipStream_t s);
int column_sum_slices(int64_t rows);
hipError_t launch_column_sum(const float* a, int rows, int E, float* slices, float* out, hipStream_t s);
constexpr int kRouterFusedMaxE = 256;
int router_fused_blocks(int64_t T);     // one partial row per 64 tokens
// E <= kRouterFusedMaxE; w_r as stored, [d, E] fp32 (split into bf16 terms inside)
hipError_t launch_router_fused(const bf16_t* x, const float* w_r, const float* b_r, int T, int d, int E, int k,
                               float* logits_out, int32_t* expert, float* gate, float* lse, float* part,
                               hipStream_t s);

// dispatch.hip
int scan_tile(int64_t group_assignments, bool one_group);   // 256, 128 or 64 assignments
int scan_tiles(int64_t N, int tile);
hipError_t launch_scan_local(const int32_t* expert, int N, int E, int k, int G, int rank, int tile,
                             int32_t* local_rank, int32_t* tile_counts, hipStream_t s);
// parts (NULL: none): the router's partial probability rows, prows per group,
// summed per expert into prob_sum [ngroups, E]
hipError_t launch_scan_offsets(int32_t* tile_counts, int ntiles, int tiles_per_group, int ngroups, int E, int C,
                               int32_t* counts, int32_t* accepted, int32_t* group_base, int32_t* rows_total,
                               const float* parts, int prows, float* prob_sum, hipStream_t s);
// a token-tile list for the expert GEMMs (ffn_tile_list): built when pre is not NULL
struct TileListOut {
    int32_t* pre = nullptr; int4* tab = nullptr; int tok = 0;
};
hipError_t launch_gather(const bf16_t* x, const int32_t* expert, const int32_t* offsets, const int32_t* group_base,
                         const int32_t* rows_filled, int N, int d, int E, int k, int G, int rank, int tile, int C,
                         int rows, int32_t* position, uint8_t* keep, int32_t* slot, int32_t* slot_token, bf16_t* buf,
                         bf16_t* out_pass, bool pass_residual, const TileListOut& tl0, const TileListOut& tl1,
                         const AuxStatsArgs* aux, hipStream_t s);

// expert_ffn.hip
int ffn_token_tile(int C);
// the forward's expert GEMMs: rows an expert is expected to fill (T k / E,
// at most the buffer rows; 0 when unknown), and the token-tile height of the
// first GEMM's list (ffn_token_tile(C), or taller; the second GEMM's list is
// always ffn_token_tile(C), so ffn_tile_table_entries bounds both)
int ffn_expected_fill(int64_t assignments, int E, int rows);
int ffn_gemm1_token_tile(int E, int C, int fill, int d_ff);
size_t ffn_tile_table_entries(int E, int C);
// several token-tile lists over the same experts in one launch (block b builds list b);
// w, if not NULL, goes into the fourth word of each tile entry of its expert
constexpr int kMaxTileLists = 3;
struct FfnTileListSpec {
    const int32_t* accepted; const int32_t* w; int C; int32_t* pre; int4* ttab;
    int tok;   // rows per tile (0: ffn_token_tile(C), set by launch_ffn_tile_lists)
};
struct FfnTileLists {
    FfnTileListSpec list[kMaxTileLists]; int E;
};
hipError_t launch_ffn_tile_lists(const FfnTileLists& L, int n, hipStream_t s);
// fill (the forward's products): the rows each expert is expected to fill,
// e.g. T k / E, which picks the tile shapes; 0: C
hipError_t launch_expert_gemm1(const bf16_t* buf, const bf16_t* w1, const int32_t* pre, const int4* ttab, bf16_t* h,
                               int E, int C, int d, int d_ff, hipStream_t s, int fill = 0);
hipError_t launch_expert_gemm2(const bf16_t* h, const bf16_t* w2, const int32_t* pre, const int4* ttab, float* y,
                               int E, int C, int d, int d_ff, hipStream_t s, int fill = 0);
// The second expert GEMM with the combine (k = 1) in its epilogue: buffer row
// s of expert e holds token slot_token[e * C + s], and
//   out[token] = bf16(residual[token] + gate[token] * y[e, s])
// (fp32, one rounding; no residual when it is NULL), plus y itself when y is
// not NULL.  Any C >= 1 (ffn_rows_fused).
struct FfnCombine {
    const int32_t* slot_token;
    const float* gate;
    const bf16_t* residual;
    bf16_t* out;
    float* y;
};
// 128-row token tiles (C > 64), the direct-to-LDS kernel for every product
// over them, the backward's included
bool ffn_wide_tiles(int C);
// the forward's expert GEMMs run the direct-to-LDS kernel at every C >= 1 (32-,
// 64- or 128-row token tiles, 320 for the first GEMM where ffn_gemm1_token_tile
// picks them), so they can gather token rows and fuse the combine
bool ffn_rows_fused(int C);
// the tallest token tile of the forward's expert GEMMs, in 32-row blocks
constexpr int kTallTokB = 10;
constexpr int kRowMapPad = 32 * kTallTokB;   // a whole token tile past the last expert's rows
// The first expert GEMM reading its token rows straight from x [T, d]: buffer
// row s of expert e is x[slot_token[e * C + s]] (no buf array).  Needs
// ffn_rows_fused(C), T * d * 2 well below 2^32, and kRowMapPad readable
// entries past slot_token[E * C - 1].
hipError_t launch_expert_gemm1_gather(const bf16_t* x, int64_t T, const int32_t* slot_token, const bf16_t* w1,
                                      const int32_t* pre, const int4* ttab, bf16_t* h, int E, int C, int d, int d_ff,
                                      hipStream_t s, int fill = 0);
// Both expert products and the combine (k = 1) in one kernel, the hidden
// activation kept on chip: token rows gathered from x as in
// launch_expert_gemm1_gather, output as in launch_expert_gemm2_combine, no H.
// Needs ffn_fused_ok(C, d, d_ff): C <= 64 (one token tile per expert), d a
// multiple of 256 up to 1024, d_ff a multiple of 256.
bool ffn_fused_ok(int C, int d, int d_ff);
hipError_t launch_expert_ffn_fused(const bf16_t* x, int64_t T, const int32_t* slot_token, const bf16_t* w1,
                                   const bf16_t* w2, const int32_t* pre, const int4* ttab, const FfnCombine& cb,
                                   int E, int C, int d, int d_ff, hipStream_t s);
hipError_t launch_expert_gemm2_combine(const bf16_t* h, const bf16_t* w2, const int32_t* pre, const int4* ttab,
                                       const FfnCombine& cb, int E, int C, int d, int d_ff, hipStream_t s, int fill = 0);
// the same kernel on other operands: out[e, r, n] = sum_k A[e, r, k] W[e, n, k]
// for the rows listed in (pre, ttab), fp32 out
hipError_t launch_grouped_gemm_f32(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab, float* out,
                                   int E, int rows, int K, int N, hipStream_t s);
// the same with W stored K-major, W[e][k][n]
hipError_t launch_grouped_gemm_kmajor_f32(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab,
                                          float* out, int E, int rows, int K, int N, hipStream_t s);
hipError_t launch_grouped_gemm_kmajor_masked(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab,
                                             bf16_t* out, const bf16_t* mask, int E, int rows, int K, int N,
                                             hipStream_t s);
// out[e, m, n] = sum_k A[e, k, m] W[e, k, n], both operands as stored (the token
// axis k, kst rows per expert), for the M-row tiles listed in (pre, ttab), whose
// fourth word holds the expert's valid k rows (the rest count as zero); M > 64
hipError_t launch_grouped_gemm_tn_f32(const bf16_t* A, const bf16_t* W, const int32_t* pre, const int4* ttab,
                                      float* out, int E, int M, int kst, int N, hipStream_t s);

// combine.hip
hipError_t launch_combine(const float* y, const int32_t* expert, const int32_t* slot, const uint8_t* keep,
                          const float* gate, const bf16_t* residual, int64_t T, int d, int E, int k, int C,
                          bf16_t* out, hipStream_t s);

// aux.hip
hipError_t launch_aux_stats(const int32_t* counts, const float* prob_sum, int64_t G, int ngroups, int E, int k,
                            float alpha, float* f, float* P, float* loss, hipStream_t s);
// the layer forward hands the router's partial rows to the dispatch step's
// scan (one wave per expert sums its column) when there are at most this
// many values
constexpr int64_t kAuxPartsMax = 262144;
hipError_t launch_z_loss(const float* lse, int64_t T, float beta, float* z_loss, hipStream_t s);
hipError_t launch_aux_grad(const float* logits, const float* lse, const float* f, int64_t T, int64_t G, int E,
                           float alpha, float beta, const int32_t* expert, const float* gate, const float* dgate,
                           int k, int accumulate, float* dlogits, hipStream_t s);

// backward.hip
// expert, slot, keep, gate, dgate [T, k]; R buffer rows per expert
hipError_t launch_combine_bwd(const bf16_t* dout, const float* y, const int32_t* expert, const int32_t* slot,
                              const uint8_t* keep, const float* gate, int64_t T, int k, int d, int E, int R,
                              bf16_t* dy, float* dgate, hipStream_t s);
hipError_t launch_transpose_rows(const bf16_t* src, bf16_t* dst, int E, int R, int S, int Rp, const int32_t* valid,
                                 hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
int router_wgrad_slices(int64_t T, int d, int E);
hipError_t launch_router_wgrad(const bf16_t* x, const float* dz, int64_t T, int d, int E, float* part, float* dw_r,
                               hipStream_t s);
hipError_t launch_dx_assemble(const bf16_t* dout, const float* dbuf, const int32_t* expert, const int32_t* slot,
                              const uint8_t* keep, const float* dz, const float* w_r, int64_t T, int d, int E, int k,
                              int R, bf16_t* dx, hipStream_t s);

// api.hip
hipError_t launch_stream_copy(void* dst, const void* src, size_t nbytes, hipStream_t s);
}  // namespace swmoe
