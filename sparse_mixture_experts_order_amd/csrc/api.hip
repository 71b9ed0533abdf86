// C ABI of the Switch FFN layer: argument validation (before any HIP call),
// workspace layout, kernel launches on the caller's stream, error text and
// the optional per-launch event timing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/switch_moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace swmoe;

namespace {

thread_local std::string g_err;

switch_status fail(switch_status s, const char* fmt, ...) {
    char b[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(b, sizeof b, fmt, ap);
    va_end(ap);
    g_err = b;
    return s;
}

switch_status hip_fail(hipError_t e, const char* where) {
    return fail(SWITCH_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ----------------------------------------------------------- launch timing
enum KernelId {
    K_SPLIT = 0, K_RGEMM, K_RSOFTMAX, K_RREDUCE, K_SCAN_LOCAL, K_SCAN_OFFSETS, K_GATHER,
    K_GEMM1, K_GEMM2, K_COMBINE, K_AUX_STATS, K_AUX_GRAD, K_COPY, K_FFN_TILES, K_Z_LOSS, K_RFUSED,
    K_COMBINE_BWD, K_ROUTER_DZ, K_ROUTER_DB, K_ROUTER_WGRAD, K_TRANSPOSE, K_GEMM_DA, K_GEMM_DBUF, K_GEMM_DW2,
    K_GEMM_DW1, K_DX, K_FFN_FUSED, K_COUNT
};
const char* kKernelNames[K_COUNT] = {
    "split_router_weights", "router_gemm", "router_softmax", "router_reduce", "scan_local", "scan_offsets",
    "gather", "expert_gemm1", "expert_gemm2", "combine", "aux_stats", "aux_grad", "stream_copy", "ffn_tile_prefix", "z_loss", "router_fused",
    "combine_bwd", "router_dz", "router_db", "router_wgrad", "transpose_rows", "gemm_dA", "gemm_dbuf", "gemm_dW2",
    "gemm_dW1", "dx_assemble", "expert_ffn_fused"};

struct ProfRec { int id; hipEvent_t a, b; };
bool g_prof = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_get() {
    if (!g_pool.empty()) { hipEvent_t e = g_pool.back(); g_pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <class F>
hipError_t timed(int id, hipStream_t s, F&& launch) {
    if (!g_prof) return launch();
    ProfRec r{id, pool_get(), pool_get()};
    if (r.a) (void)hipEventRecord(r.a, s);
    hipError_t err = launch();
    if (r.b) (void)hipEventRecord(r.b, s);
    if (r.a && r.b) g_recs.push_back(r);
    return err;
}

#define LAUNCH(id, where, stream, call)                                     \
    do {                                                                    \
        hipError_t _e = timed(id, stream, [&]() { return (call); });       \
        if (_e != hipSuccess) return hip_fail(_e, where);                   \
    } while (0)

// ----------------------------------------------------------- workspace
constexpr size_t kAlign = 256;
size_t up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct Carver {
    char* base;
    size_t off = 0;
    template <class T> T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base + off);
        off += up(count * sizeof(T));
        return p;
    }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// GEMM mode with E <= kRouterFusedMaxE runs the fused router (no logits
// round trip); wider routers write the logits and run the softmax pass.
bool route_fused(int32_t E) { return E <= kRouterFusedMaxE; }
size_t route_parts(int64_t T, int32_t E) {
    return (size_t)std::max(router_softmax_blocks(T, E), router_fused_blocks(T)) * E;
}
size_t route_ws(int64_t T, int32_t d, int32_t E, bool logits_out_given) {
    size_t n = up((size_t)3 * d * E * sizeof(bf16_t)) + up(route_parts(T, E) * sizeof(float));
    if (!logits_out_given && !route_fused(E)) n += up((size_t)T * E * sizeof(float));
    return n;
}
// Routing groups: group == 0 (or == T) is one group of all T tokens.
bool one_group(int64_t T, int64_t G) { return G == 0 || G == T; }
int64_t group_count(int64_t T, int64_t G) { return one_group(T, G) ? 1 : T / G; }
int64_t group_tokens(int64_t T, int64_t G) { return one_group(T, G) ? T : G; }
// buffer rows per expert: C per group, groups packed one after the other
int64_t buffer_rows(int64_t T, int64_t G, int32_t C) { return group_count(T, G) * C; }

size_t dispatch_ws(int64_t T, int32_t E, int32_t k, int64_t G) {
    const bool one = one_group(T, G);
    const int tile = scan_tile(group_tokens(T, G) * k, one);
    size_t n = up((size_t)scan_tiles(T * k, tile) * E * sizeof(int32_t));
    if (!one) n += up((size_t)group_count(T, G) * E * sizeof(int32_t)) + up((size_t)E * sizeof(int32_t));
    return n;
}
// the expert FFN's workspace: H, the second GEMM's token-tile list
// (ffn_token_tile(C) rows per tile), and room for the first GEMM's own list
// when it takes taller tiles (ffn_gemm1_token_tile; never more entries)
size_t ffn_ws(int32_t E, int32_t C, int32_t d_ff) {
    return up((size_t)E * C * d_ff * sizeof(bf16_t)) +
           2 * (up((size_t)(E + 1) * sizeof(int32_t)) + up(ffn_tile_table_entries(E, C) * sizeof(int4)));
}
struct FfnSpace {
    bf16_t* h; TileListOut l2, l1;   // l1.pre NULL: the first GEMM reads l2 too
};
FfnSpace carve_ffn(void* ws, int32_t E, int32_t C, int32_t d_ff, int fill) {
    Carver c{(char*)ws};
    FfnSpace f{};
    f.h = c.take<bf16_t>((size_t)E * C * d_ff);
    f.l2.pre = c.take<int32_t>((size_t)E + 1);
    f.l2.tab = c.take<int4>(ffn_tile_table_entries(E, C));
    f.l2.tok = ffn_token_tile(C);
    const int tok1 = ffn_gemm1_token_tile(E, C, fill, d_ff);
    if (tok1 != f.l2.tok) {
        f.l1.pre = c.take<int32_t>((size_t)E + 1);
        f.l1.tab = c.take<int4>(ffn_tile_table_entries(E, C));
        f.l1.tok = tok1;
    }
    return f;
}

// ----------------------------------------------------------- validation
#define REQUIRE(cond, ...) \
    do { if (!(cond)) return fail(SWITCH_E_INVALID, __VA_ARGS__); } while (0)
#define SUPPORT(cond, ...) \
    do { if (!(cond)) return fail(SWITCH_E_UNSUPPORTED, __VA_ARGS__); } while (0)

switch_status check_TE(int64_t T, int32_t E) {
    REQUIRE(T >= 0, "T must be >= 0 (got %lld)", (long long)T);
    REQUIRE(E >= 1, "E must be >= 1 (got %d)", E);
    SUPPORT(T < (int64_t(1) << 31), "T must be < 2^31 (got %lld)", (long long)T);
    SUPPORT(E <= 4096, "E must be <= 4096 (got %d)", E);
    SUPPORT((int64_t)T * E < (int64_t(1) << 40), "T*E too large");
    return SWITCH_OK;
}

switch_status check_C(int32_t E, int32_t C) {
    REQUIRE(C >= 0, "C must be >= 0 (got %d)", C);
    SUPPORT((int64_t)E * C < (int64_t(1) << 31), "E*C must be < 2^31");
    return SWITCH_OK;
}

// k choices per token and routing groups of G tokens
switch_status check_kG(int64_t T, int32_t E, int32_t k, int64_t G) {
    REQUIRE(k >= 1 && k <= E, "k must be in [1, E] (got %d)", k);
    SUPPORT(k <= kMaxTopK, "k must be <= %d (got %d)", kMaxTopK, k);
    SUPPORT(T * k < (int64_t(1) << 31), "T*k must be < 2^31");
    REQUIRE(G >= 0, "group must be >= 0 (got %lld)", (long long)G);
    if (!one_group(T, G)) {
        REQUIRE(T % G == 0, "T (%lld) must be a multiple of the group size (%lld)", (long long)T, (long long)G);
        SUPPORT(G % 64 == 0, "the group size must be a multiple of 64 (got %lld)", (long long)G);
    }
    return SWITCH_OK;
}

#define CHECK(x) do { switch_status _s = (x); if (_s != SWITCH_OK) return _s; } while (0)
#define NONNULL(p) REQUIRE((p) != nullptr, "%s must not be NULL", #p)
// arrays with zero elements may be NULL (torch gives empty tensors a NULL data pointer)
#define NONNULL_IF(cond, p) do { if (cond) NONNULL(p); } while (0)
#define ALIGNED16(p) REQUIRE((p) == nullptr || aligned((p), 16), "%s must be 16-byte aligned", #p)
#define ALIGNED4(p) REQUIRE((p) == nullptr || aligned((p), 4), "%s must be 4-byte aligned", #p)

// ----------------------------------------------------------- the steps
struct RouteArgs {
    const bf16_t* x; const float* w_r; const float* b_r; const float* logits_in;
    int64_t T; int32_t d, E;
    float* logits_out; int32_t* expert; float* gate; float* lse; float* prob_sum;
    int32_t k = 1; int64_t G = 0;   // choices per token; tokens per routing group (0: one group)
    // the layer forward: when the partial probability rows are few, leave their
    // sum to the aux kernel (part_out / part_rows_out receive them; prob_sum unset)
    bool defer_reduce = false; const float** part_out = nullptr; int* part_rows_out = nullptr;
};

switch_status validate_route(const RouteArgs& a, const void* ws, size_t ws_bytes) {
    CHECK(check_TE(a.T, a.E));
    CHECK(check_kG(a.T, a.E, a.k, a.G));
    const bool tok = a.T > 0;
    NONNULL_IF(tok, a.expert); NONNULL_IF(tok, a.gate); NONNULL_IF(tok, a.lse);
    NONNULL_IF(group_count(a.T, a.G) > 0, a.prob_sum);
    ALIGNED4(a.expert); ALIGNED4(a.gate); ALIGNED4(a.lse); ALIGNED4(a.prob_sum); ALIGNED4(a.logits_out);
    ALIGNED4(a.logits_in);
    if (!a.logits_in) {
        NONNULL_IF(tok, a.x); NONNULL(a.w_r);
        ALIGNED16(a.x); ALIGNED4(a.w_r); ALIGNED4(a.b_r);
        REQUIRE(a.d >= 1, "d must be >= 1 (got %d)", a.d);
        SUPPORT(a.d % 32 == 0, "d must be a multiple of 32 for the router GEMM (got %d)", a.d);
        SUPPORT((int64_t)6 * a.E * a.d < (int64_t(1) << 31), "the split router weights (3*E*d bf16) must be < 2 GiB");
    }
    REQUIRE(a.logits_in != nullptr || !tok || a.x != nullptr, "x must not be NULL");
    const size_t need = a.logits_in ? route_ws(a.T, 0, a.E, true) : route_ws(a.T, a.d, a.E, a.logits_out != nullptr);
    if (ws_bytes < need) return fail(SWITCH_E_WORKSPACE, "route needs %zu workspace bytes, got %zu", need, ws_bytes);
    REQUIRE(need == 0 || ws != nullptr, "ws must not be NULL");
    REQUIRE(aligned(ws, kAlign), "ws must be %zu-byte aligned", kAlign);
    return SWITCH_OK;
}

// Sum the partial rows into prob_sum, or hand them to the aux step.
switch_status finish_route(const RouteArgs& a, const float* part, int rows, int ng, hipStream_t s) {
    if (a.defer_reduce && (int64_t)rows * ng * a.E <= kAuxPartsMax) {
        *a.part_out = part;
        *a.part_rows_out = rows;
        return SWITCH_OK;
    }
    LAUNCH(K_RREDUCE, "router_reduce", s, launch_router_reduce(part, rows, ng, a.E, a.prob_sum, s));
    return SWITCH_OK;
}

switch_status run_route(const RouteArgs& a, void* ws, hipStream_t s) {
    const int T = (int)a.T, E = a.E;
    // with routing groups the partial rows cover 64 tokens each and are summed per group
    const bool one = one_group(a.T, a.G);
    const int ng = (int)group_count(a.T, a.G);
    const int rows_per_group = one ? 0 : (int)(a.G / 64);
    Carver c{(char*)ws};
    const float* logits = a.logits_in;
    if (!logits) {
        bf16_t* wr3 = c.take<bf16_t>((size_t)3 * a.d * E);
        if (route_fused(E)) {   // splits W_r into its bf16 terms itself
            float* part = c.take<float>(route_parts(T, E));
            const int nblk = T > 0 ? router_fused_blocks(T) : 0;
            if (T > 0)
                LAUNCH(K_RFUSED, "router_fused", s,
                       launch_router_fused(a.x, a.w_r, a.b_r, T, a.d, E, a.k, a.logits_out, a.expert, a.gate, a.lse,
                                           part, s));
            return finish_route(a, part, one ? nblk : rows_per_group, ng, s);
        }
        LAUNCH(K_SPLIT, "split_router_weights", s, launch_split_router_weights(a.w_r, wr3, a.d, E, s));
        float* z = a.logits_out ? a.logits_out : c.take<float>((size_t)T * E);
        if (T > 0) LAUNCH(K_RGEMM, "router_gemm", s, launch_router_gemm(a.x, wr3, a.b_r, z, T, a.d, E, s));
        logits = z;
    }
    const int nblk = one ? router_softmax_blocks(T, E) : router_softmax_blocks_grouped(T);
    float* part = c.take<float>(route_parts(T, E));
    if (T > 0)
        LAUNCH(K_RSOFTMAX, "router_softmax", s,
               launch_router_softmax(logits, T, E, a.k, !one, a.expert, a.gate, a.lse, part, s));
    return finish_route(a, part, one ? nblk : rows_per_group, ng, s);
}

struct DispatchArgs {
    const bf16_t* x; const int32_t* expert; int64_t T; int32_t d, E, C;
    int32_t* position; uint8_t* keep; int32_t* counts; int32_t* accepted; int32_t* slot_token; bf16_t* buf;
    int32_t k = 1; int64_t G = 0; int32_t priority = 0;   // C is the capacity of one group
    int32_t* slot = nullptr; int32_t* rows_total = nullptr;
    bf16_t* out_pass = nullptr; bool pass_residual = false;   // k = 1: dropped tokens' output rows (fused combine)
    bool no_buf = false;   // the first expert GEMM gathers the token rows itself: buf is not written
    TileListOut tl0, tl1;   // also build the expert GEMMs' token-tile lists (those with pre set)
    const AuxStatsArgs* aux = nullptr;                   // and the load-balancing statistics
    // the router's partial probability rows (prows per group), summed into prob_sum by the scan
    const float* parts = nullptr; int prows = 0; float* prob_sum = nullptr;
};

switch_status validate_dispatch(const DispatchArgs& a, const void* ws, size_t ws_bytes) {
    CHECK(check_TE(a.T, a.E));
    CHECK(check_C(a.E, a.C));
    CHECK(check_kG(a.T, a.E, a.k, a.G));
    REQUIRE(a.priority == 0 || a.priority == 1, "priority must be 0 (token) or 1 (rank)");
    const int64_t rows = buffer_rows(a.T, a.G, a.C);
    SUPPORT((int64_t)a.E * rows < (int64_t(1) << 31), "E * groups * C must be < 2^31");
    const bool grouped = group_count(a.T, a.G) > 0;
    REQUIRE(a.d >= 1, "d must be >= 1 (got %d)", a.d);
    SUPPORT(a.d % 8 == 0, "d must be a multiple of 8 (got %d)", a.d);
    const bool tok = a.T > 0;
    NONNULL_IF(tok, a.x); NONNULL_IF(tok, a.expert); NONNULL_IF(tok, a.position); NONNULL_IF(tok, a.keep);
    NONNULL_IF(grouped, a.counts); NONNULL_IF(grouped, a.accepted);
    NONNULL_IF(rows > 0 && !a.no_buf, a.buf);
    ALIGNED16(a.x); ALIGNED16(a.buf); ALIGNED4(a.expert); ALIGNED4(a.position); ALIGNED4(a.counts);
    ALIGNED4(a.accepted); ALIGNED4(a.slot_token); ALIGNED4(a.slot); ALIGNED4(a.rows_total);
    const size_t need = dispatch_ws(a.T, a.E, a.k, a.G);
    if (ws_bytes < need) return fail(SWITCH_E_WORKSPACE, "dispatch needs %zu workspace bytes, got %zu", need, ws_bytes);
    REQUIRE(need == 0 || ws != nullptr, "ws must not be NULL");
    REQUIRE(aligned(ws, kAlign), "ws must be %zu-byte aligned", kAlign);
    return SWITCH_OK;
}

switch_status run_dispatch(const DispatchArgs& a, void* ws, hipStream_t s) {
    const bool one = one_group(a.T, a.G);
    const int N = (int)(a.T * a.k);
    const int G = (int)std::max<int64_t>(group_tokens(a.T, a.G), 1);
    const int ng = (int)group_count(a.T, a.G);
    const int tile = scan_tile((int64_t)G * a.k, one);
    const int ntiles = scan_tiles(N, tile);
    const int tpg = one ? ntiles : G * a.k / tile;
    const int rows = (int)buffer_rows(a.T, a.G, a.C);
    Carver c{(char*)ws};
    int32_t* tile_counts = c.take<int32_t>((size_t)ntiles * a.E);
    int32_t* group_base = one ? nullptr : c.take<int32_t>((size_t)ng * a.E);
    int32_t* rows_total = a.rows_total;
    if (!one) {
        int32_t* own = c.take<int32_t>((size_t)a.E);
        if (!rows_total) rows_total = own;
    }
    if (N > 0)
        LAUNCH(K_SCAN_LOCAL, "scan_local", s,
               launch_scan_local(a.expert, N, a.E, a.k, G, a.priority, tile, a.position, tile_counts, s));
    LAUNCH(K_SCAN_OFFSETS, "scan_offsets", s,
           launch_scan_offsets(tile_counts, ntiles, tpg, ng, a.E, a.C, a.counts, a.accepted, group_base, rows_total,
                               a.parts, a.prows, a.prob_sum, s));
    LAUNCH(K_GATHER, "gather", s,
           launch_gather(a.x, a.expert, tile_counts, group_base, one ? a.accepted : rows_total, N, a.d, a.E, a.k, G,
                         a.priority, tile, a.C, rows, a.position, a.keep, a.slot, a.slot_token,
                         a.no_buf ? nullptr : a.buf, a.out_pass, a.pass_residual, a.tl0, a.tl1, a.aux, s));
    return SWITCH_OK;
}

struct FfnArgs {
    const bf16_t* buf; const int32_t* accepted; const bf16_t* w1; const bf16_t* w2;
    int32_t E, C, d, d_ff; float* y;
    bf16_t* h = nullptr;   // [E, C, d_ff] hidden activations; NULL: workspace only
    const FfnCombine* cb = nullptr;   // the combine in the second GEMM's epilogue (y optional then)
    // token rows gathered by the first GEMM from x [x_tokens, d] through a_rows (= slot_token); buf unused
    const bf16_t* x_src = nullptr; int64_t x_tokens = 0; const int32_t* a_rows = nullptr;
    bool tiles_ready = false;   // the token-tile list in the workspace was built by the dispatch step
    int64_t assignments = 0;    // T k of the layer (0: unknown): T k / E rows per expert expected
};

switch_status validate_ffn(const FfnArgs& a, const void* ws, size_t ws_bytes) {
    REQUIRE(a.E >= 1, "E must be >= 1 (got %d)", a.E);
    SUPPORT(a.E <= 4096, "E must be <= 4096 (got %d)", a.E);
    CHECK(check_C(a.E, a.C));
    REQUIRE(a.d >= 1 && a.d_ff >= 1, "d and d_ff must be >= 1");
    SUPPORT(a.d % 64 == 0 && a.d_ff % 64 == 0, "d and d_ff must be multiples of 64 (got %d, %d)", a.d, a.d_ff);
    SUPPORT((int64_t)a.E * a.C * std::max(a.d, a.d_ff) < (int64_t(1) << 40), "E*C*max(d,d_ff) too large");
    SUPPORT((int64_t)a.d * a.d_ff * 2 < (int64_t(1) << 31), "one expert's weights must be < 2 GiB (d*d_ff*2)");
    SUPPORT((int64_t)a.C * std::max(a.d, a.d_ff) * 2 < (int64_t(1) << 31), "C*max(d,d_ff)*2 must be < 2 GiB");
    NONNULL(a.accepted); NONNULL(a.w1); NONNULL(a.w2);
    if (a.C > 0) {
        if (a.a_rows) NONNULL(a.x_src); else NONNULL(a.buf);
        if (!a.cb) NONNULL(a.y);
    }
    REQUIRE(!a.a_rows || ffn_rows_fused(a.C), "gathered token rows need at least one buffer row per expert");
    REQUIRE(!a.cb || ffn_rows_fused(a.C), "the fused combine needs at least one buffer row per expert");
    ALIGNED16(a.buf); ALIGNED16(a.w1); ALIGNED16(a.w2); ALIGNED16(a.y); ALIGNED4(a.accepted); ALIGNED16(a.h);
    const size_t need = ffn_ws(a.E, a.C, a.d_ff);
    if (ws_bytes < need) return fail(SWITCH_E_WORKSPACE, "expert_ffn needs %zu workspace bytes, got %zu", need, ws_bytes);
    REQUIRE(need == 0 || ws != nullptr, "ws must not be NULL");
    REQUIRE(aligned(ws, kAlign), "ws must be %zu-byte aligned", kAlign);
    return SWITCH_OK;
}

switch_status run_ffn(const FfnArgs& a, void* ws, hipStream_t s) {
    if (a.C == 0) return SWITCH_OK;
    const int fill = ffn_expected_fill(a.assignments, a.E, a.C);
    const FfnSpace f = carve_ffn(ws, a.E, a.C, a.d_ff, fill);
    bf16_t* h = a.h ? a.h : f.h;
    int32_t* pre = f.l2.pre;
    int4* ttab = f.l2.tab;
    // the first GEMM's list: its own when it takes taller token tiles
    const int32_t* pre1 = f.l1.pre ? f.l1.pre : pre;
    const int4* ttab1 = f.l1.pre ? f.l1.tab : ttab;
    if (!a.tiles_ready) {
        FfnTileLists tl{};
        tl.E = a.E;
        tl.list[0] = FfnTileListSpec{a.accepted, nullptr, a.C, pre, ttab, f.l2.tok};
        if (f.l1.pre) tl.list[1] = FfnTileListSpec{a.accepted, nullptr, a.C, f.l1.pre, f.l1.tab, f.l1.tok};
        LAUNCH(K_FFN_TILES, "ffn_tile_prefix", s, launch_ffn_tile_lists(tl, f.l1.pre ? 2 : 1, s));
    }
    // gathered token rows, the fused combine and no H asked for: at small
    // capacity both products run in one kernel with H on chip
    if (a.a_rows && a.cb && !a.h && ffn_fused_ok(a.C, a.d, a.d_ff)) {
        LAUNCH(K_FFN_FUSED, "expert_ffn_fused", s,
               launch_expert_ffn_fused(a.x_src, a.x_tokens, a.a_rows, a.w1, a.w2, pre, ttab, *a.cb, a.E, a.C, a.d,
                                       a.d_ff, s));
        return SWITCH_OK;
    }
    if (a.a_rows)
        LAUNCH(K_GEMM1, "expert_gemm1", s,
               launch_expert_gemm1_gather(a.x_src, a.x_tokens, a.a_rows, a.w1, pre1, ttab1, h, a.E, a.C, a.d, a.d_ff,
                                          s, fill));
    else
        LAUNCH(K_GEMM1, "expert_gemm1", s,
               launch_expert_gemm1(a.buf, a.w1, pre1, ttab1, h, a.E, a.C, a.d, a.d_ff, s, fill));
    if (a.cb)
        LAUNCH(K_GEMM2, "expert_gemm2", s,
               launch_expert_gemm2_combine(h, a.w2, pre, ttab, *a.cb, a.E, a.C, a.d, a.d_ff, s, fill));
    else
        LAUNCH(K_GEMM2, "expert_gemm2", s,
               launch_expert_gemm2(h, a.w2, pre, ttab, a.y, a.E, a.C, a.d, a.d_ff, s, fill));
    return SWITCH_OK;
}

struct CombineArgs {
    const float* y; const int32_t* expert; const int32_t* position; const uint8_t* keep; const float* gate;
    const bf16_t* residual; int64_t T; int32_t d, E, C; bf16_t* out;
    int32_t k = 1;   // choices per token; `position` holds buffer rows, C the rows per expert
};

switch_status validate_combine(const CombineArgs& a) {
    CHECK(check_TE(a.T, a.E));
    CHECK(check_C(a.E, a.C));
    CHECK(check_kG(a.T, a.E, a.k, 0));
    REQUIRE(a.d >= 1, "d must be >= 1 (got %d)", a.d);
    SUPPORT(a.d % 8 == 0, "d must be a multiple of 8 (got %d)", a.d);
    const bool tok = a.T > 0;
    NONNULL_IF(tok, a.expert); NONNULL_IF(tok, a.position); NONNULL_IF(tok, a.keep); NONNULL_IF(tok, a.gate);
    NONNULL_IF(tok, a.out);
    NONNULL_IF(tok && a.C > 0, a.y);
    ALIGNED16(a.y); ALIGNED16(a.residual); ALIGNED16(a.out); ALIGNED4(a.expert); ALIGNED4(a.position);
    ALIGNED4(a.gate);
    REQUIRE(!tok || a.residual == nullptr || (const void*)a.residual != (const void*)a.out,
            "out must not alias residual");
    return SWITCH_OK;
}

switch_status run_combine(const CombineArgs& a, hipStream_t s) {
    LAUNCH(K_COMBINE, "combine", s,
           launch_combine(a.y, a.expert, a.position, a.keep, a.gate, a.residual, a.T, a.d, a.E, a.k, a.C, a.out, s));
    return SWITCH_OK;
}

struct AuxArgs {
    const int32_t* counts; const float* prob_sum; const float* logits; const float* lse;
    int64_t T; int32_t E; float alpha; float* f; float* P; float* loss; float* dlogits;
    float beta; float* z_loss;   // router z-loss (optional, z_loss == NULL: not computed)
    int32_t k = 1; int64_t G = 0;   // counts, prob_sum, f, P are [groups, E]
    bool stats_done = false;   // prob_sum, f, P and the loss already computed by the dispatch step
};

switch_status validate_aux(const AuxArgs& a) {
    CHECK(check_TE(a.T, a.E));
    CHECK(check_kG(a.T, a.E, a.k, a.G));
    REQUIRE(std::isfinite(a.alpha), "alpha must be finite");
    const bool grouped = group_count(a.T, a.G) > 0;
    NONNULL_IF(grouped, a.counts); NONNULL_IF(grouped, a.prob_sum); NONNULL_IF(grouped, a.f);
    NONNULL_IF(grouped, a.P); NONNULL(a.loss);
    if (a.dlogits && a.T > 0) { NONNULL(a.logits); NONNULL(a.lse); }
    if (a.z_loss && a.T > 0) NONNULL(a.lse);
    REQUIRE(std::isfinite(a.beta), "beta must be finite");
    ALIGNED4(a.z_loss);
    ALIGNED4(a.counts); ALIGNED4(a.prob_sum); ALIGNED4(a.logits); ALIGNED4(a.lse); ALIGNED4(a.f); ALIGNED4(a.P);
    ALIGNED4(a.loss); ALIGNED4(a.dlogits);
    return SWITCH_OK;
}

switch_status run_aux(const AuxArgs& a, hipStream_t s) {
    const int64_t Gt = group_tokens(a.T, a.G);
    if (!a.stats_done)
        LAUNCH(K_AUX_STATS, "aux_stats", s,
               launch_aux_stats(a.counts, a.prob_sum, Gt, (int)group_count(a.T, a.G), a.E, a.k, a.alpha, a.f, a.P,
                                a.loss, s));
    if (a.z_loss) LAUNCH(K_Z_LOSS, "z_loss", s, launch_z_loss(a.lse, a.T, a.beta, a.z_loss, s));
    if (a.dlogits && a.T > 0)
        LAUNCH(K_AUX_GRAD, "aux_grad", s,
               launch_aux_grad(a.logits, a.lse, a.f, a.T, Gt, a.E, a.alpha, a.z_loss ? a.beta : 0.f, nullptr, nullptr,
                               nullptr, 1, 0, a.dlogits,
                               s));
    return SWITCH_OK;
}

}  // namespace

namespace swmoe {
__global__ __launch_bounds__(256) void stream_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          size_t n) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    for (; i < n; i += stride) dst[i] = src[i];
}
hipError_t launch_stream_copy(void* dst, const void* src, size_t nbytes, hipStream_t s) {
    const size_t n = nbytes / 16;
    if (n == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 256 * 64);
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint4*)src, (uint4*)dst, n);
    return hipGetLastError();
}
}  // namespace swmoe

// ------------------------------------------------ allocation-free dispatch
// The scratch of switch_dispatch_noalloc: the per-tile expert counts of the
// slot scan (ceil(T / 256) * E int32).  A file-scope device array, so a call
// allocates nothing; each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch (looked up on the device's first call).
switch_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SWITCH_E_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, kAlign)) return fail(SWITCH_E_HIP, "scratch has no aligned device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SWITCH_OK;
}
}  // namespace

// =================================================================== C ABI
extern "C" {

switch_status switch_capacity(int64_t T, int32_t E, double c, int32_t* C_out) {
    if (!C_out) return fail(SWITCH_E_INVALID, "C_out must not be NULL");
    if (T < 0) return fail(SWITCH_E_INVALID, "T must be >= 0");
    if (E <= 0) return fail(SWITCH_E_INVALID, "E must be > 0");
    if (!std::isfinite(c) || c < 0) return fail(SWITCH_E_INVALID, "c must be finite and >= 0");
    if (c == 0 || T == 0) { *C_out = 0; return SWITCH_OK; }
    // c = m * 2^ex exactly, with m a 53-bit integer
    int ex = 0;
    const double fr = std::frexp(c, &ex);
    const uint64_t m = (uint64_t)std::ldexp(fr, 53);
    ex -= 53;
    typedef unsigned __int128 u128;
    const u128 num = (u128)m * (u128)(uint64_t)T;  // < 2^84
    u128 q;
    if (ex >= 0) {
        if (ex > 40) return fail(SWITCH_E_INVALID, "capacity does not fit in int32");
        const u128 n2 = num << ex;
        q = (n2 + (u128)(uint32_t)E - 1) / (u128)(uint32_t)E;
    } else {
        const int sh = -ex;
        if (sh >= 96) {
            q = num > 0 ? 1 : 0;  // 0 < c T / E < 1
        } else {
            const u128 den = (u128)(uint32_t)E << sh;
            q = (num + den - 1) / den;
        }
    }
    if (q > (u128)INT32_MAX) return fail(SWITCH_E_INVALID, "capacity does not fit in int32");
    *C_out = (int32_t)q;
    return SWITCH_OK;
}

size_t switch_route_workspace_bytes(int64_t T, int32_t d, int32_t E) {
    if (T < 0 || d < 0 || E < 1 || E > 4096 || T >= (int64_t(1) << 31)) return 0;
    return route_ws(T, d, E, false);
}
size_t switch_dispatch_workspace_bytes(int64_t T, int32_t E) {
    if (T < 0 || E < 1 || E > 4096 || T >= (int64_t(1) << 31)) return 0;
    return dispatch_ws(T, E, 1, 0);
}
size_t switch_dispatch_workspace_bytes_ex(int64_t T, int32_t E, int32_t k, int64_t group) {
    if (T < 0 || E < 1 || E > 4096 || k < 1 || k > kMaxTopK || group < 0 || T * k >= (int64_t(1) << 31)) return 0;
    if (!one_group(T, group) && (T % group != 0)) return 0;
    return dispatch_ws(T, E, k, group);
}
size_t switch_expert_ffn_workspace_bytes(int32_t E, int32_t C, int32_t d_ff) {
    if (E < 1 || C < 0 || d_ff < 0) return 0;
    return ffn_ws(E, C, d_ff);
}
size_t switch_aux_loss_workspace_bytes(int64_t, int32_t) { return 0; }

static size_t layer_ws(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C, int32_t k, int64_t G) {
    const int64_t rows = buffer_rows(T, G, C);
    const int64_t ng = group_count(T, G);
    size_t n = route_ws(T, d, E, true) + dispatch_ws(T, E, k, G) + ffn_ws(E, (int32_t)rows, d_ff);
    n += up((size_t)T * E * sizeof(float));          // logits
    n += up((size_t)T * sizeof(float));              // lse
    n += up((size_t)ng * E * sizeof(float));         // prob_sum
    n += up((size_t)E * rows * d * sizeof(bf16_t));  // buf
    n += up((size_t)E * rows * d * sizeof(float));   // y
    n += up(((size_t)E * rows + kRowMapPad) * sizeof(int32_t));   // slot_token (padded for the gathering GEMM)
    if (!one_group(T, G)) {
        n += up((size_t)T * k * sizeof(int32_t));    // slot
        n += up((size_t)E * sizeof(int32_t));        // accepted rows per expert
    }
    return n;
}

// ----------------------------------------------------------- layer backward
static int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

// C: the buffer rows per expert (groups x the capacity of one group)
static size_t layer_bwd_ws(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C, int32_t k) {
    const size_t Cp = (size_t)pad64(C), e = (size_t)E;
    size_t n = 0;
    n += up(e * C * d * sizeof(bf16_t));          // dy
    n += up(e * d * Cp * sizeof(bf16_t));         // dy^T
    n += up(e * d_ff * Cp * sizeof(bf16_t));      // H^T
    n += up(e * C * d_ff * sizeof(bf16_t));       // dA
    n += up(e * d_ff * Cp * sizeof(bf16_t));      // dA^T
    n += up(e * d * Cp * sizeof(bf16_t));         // buf^T
    n += up(e * C * d * sizeof(float));           // dbuf
    n += up((size_t)T * E * sizeof(float));       // dz
    n += up((size_t)T * k * sizeof(float));       // dgate
    n += up((size_t)std::max(router_wgrad_slices(T, d, E), 1) * d * E * sizeof(float));   // dW_r slices
    n += up((size_t)column_sum_slices(T) * E * sizeof(float));                              // db_r slices
    n += 3 * up((e + 1) * sizeof(int32_t));       // tile prefixes: token rows, d rows, d_ff rows
    n += up(ffn_tile_table_entries(E, C) * sizeof(int4)) + up(ffn_tile_table_entries(E, d) * sizeof(int4)) +
         up(ffn_tile_table_entries(E, d_ff) * sizeof(int4));
    return n;
}

size_t switch_layer_bwd_workspace_bytes(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C) {
    if (T < 0 || d < 1 || d_ff < 1 || E < 1 || E > 4096 || C < 0 || T >= (int64_t(1) << 31)) return 0;
    return layer_bwd_ws(T, d, d_ff, E, C, 1);
}

size_t switch_layer_bwd_workspace_bytes_ex(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C, int32_t k,
                                           int64_t group) {
    if (T < 0 || d < 1 || d_ff < 1 || E < 1 || E > 4096 || C < 0 || T >= (int64_t(1) << 31)) return 0;
    if (k < 1 || k > kMaxTopK || group < 0 || T * k >= (int64_t(1) << 31)) return 0;
    if (!one_group(T, group) && T % group != 0) return 0;
    const int64_t rows = buffer_rows(T, group, C);
    if ((int64_t)E * rows >= (int64_t(1) << 31)) return 0;
    return layer_bwd_ws(T, d, d_ff, E, (int32_t)rows, k);
}

switch_status switch_layer_bwd(const switch_layer_bwd_args* ba, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (!ba) return fail(SWITCH_E_INVALID, "args must not be NULL");
    const switch_layer_bwd_args& B = *ba;
    hipStream_t s = (hipStream_t)stream;
    const int64_t T = B.T;
    const int32_t d = B.d, F = B.d_ff, E = B.E, Cg = B.C;
    const int32_t k = B.k == 0 ? 1 : B.k;
    const int64_t G = B.group;
    CHECK(check_TE(T, E));
    CHECK(check_C(E, Cg));
    CHECK(check_kG(T, E, k, G));
    const bool one = one_group(T, G);
    const int64_t rows64 = buffer_rows(T, G, Cg);
    SUPPORT((int64_t)E * rows64 < (int64_t(1) << 31), "E * groups * C must be < 2^31");
    // from here on C is the buffer rows per expert (groups x the capacity of one group)
    const int32_t C = (int32_t)rows64;
    REQUIRE(d >= 1 && F >= 1, "d and d_ff must be >= 1");
    SUPPORT(d % 64 == 0 && F % 64 == 0, "d and d_ff must be multiples of 64 (got %d, %d)", d, F);
    SUPPORT((int64_t)E * std::max<int64_t>(pad64(C), std::max(d, F)) * std::max(d, F) < (int64_t(1) << 40),
            "E*C*max(d,d_ff) too large");
    REQUIRE(std::isfinite(B.alpha) && std::isfinite(B.z_beta), "alpha and z_beta must be finite");
    REQUIRE(B.dx_branch_only == 0 || B.dx_branch_only == 1, "dx_branch_only must be 0 or 1");
    SUPPORT((int64_t)d * F * 2 < (int64_t(1) << 31), "one expert's weights must be < 2 GiB (d*d_ff*2)");
    SUPPORT((int64_t)pad64(C) * std::max(d, F) * 2 < (int64_t(1) << 31), "C*max(d,d_ff)*2 must be < 2 GiB");
    // one group: the buffer row is the position and accepted counts the filled rows
    const int32_t* slot = one ? B.position : B.slot;
    const int32_t* filled = one ? B.accepted : B.accepted_total;
    const bool tok = T > 0;
    NONNULL_IF(tok, B.x); NONNULL(B.w_r); NONNULL(B.w1); NONNULL(B.w2);
    NONNULL_IF(tok, B.expert); NONNULL_IF(tok, B.gate); NONNULL_IF(tok, B.keep);
    if (one) { NONNULL_IF(tok, B.position); NONNULL(B.accepted); }
    else { NONNULL_IF(tok, B.slot); NONNULL(B.accepted_total); }
    NONNULL(B.f); NONNULL_IF(tok, B.logits); NONNULL_IF(tok, B.lse);
    NONNULL_IF(C > 0, B.buf); NONNULL_IF(C > 0, B.h); NONNULL_IF(C > 0, B.y); NONNULL_IF(tok, B.dout);
    NONNULL_IF(tok, B.dx); NONNULL(B.dw_r); NONNULL(B.db_r); NONNULL(B.dw1); NONNULL(B.dw2);
    ALIGNED16(B.x); ALIGNED16(B.w1); ALIGNED16(B.w2); ALIGNED16(B.buf); ALIGNED16(B.h); ALIGNED16(B.y);
    ALIGNED16(B.dout); ALIGNED16(B.dx); ALIGNED16(B.dw1); ALIGNED16(B.dw2);
    ALIGNED4(B.w_r); ALIGNED4(B.expert); ALIGNED4(B.gate); ALIGNED4(B.position); ALIGNED4(B.accepted);
    ALIGNED4(B.f); ALIGNED4(B.logits); ALIGNED4(B.lse); ALIGNED4(B.dw_r); ALIGNED4(B.db_r); ALIGNED4(B.dz);
    ALIGNED4(B.dgate); ALIGNED4(B.slot); ALIGNED4(B.accepted_total);
    const size_t need = layer_bwd_ws(T, d, F, E, C, k);
    if (ws_bytes < need) return fail(SWITCH_E_WORKSPACE, "layer backward needs %zu workspace bytes, got %zu", need, ws_bytes);
    REQUIRE(ws != nullptr, "ws must not be NULL");
    REQUIRE(aligned(ws, kAlign), "ws must be %zu-byte aligned", kAlign);

    const int Cp = (int)pad64(C);
    Carver c{(char*)ws};
    bf16_t* dy = c.take<bf16_t>((size_t)E * C * d);
    bf16_t* dyT = c.take<bf16_t>((size_t)E * d * Cp);
    bf16_t* hT = c.take<bf16_t>((size_t)E * F * Cp);
    bf16_t* dA = c.take<bf16_t>((size_t)E * C * F);
    bf16_t* dAT = c.take<bf16_t>((size_t)E * F * Cp);
    bf16_t* bufT = c.take<bf16_t>((size_t)E * d * Cp);
    float* dbuf = c.take<float>((size_t)E * C * d);
    float* dz = c.take<float>((size_t)T * E);
    float* dgate = c.take<float>((size_t)T * k);
    float* part = c.take<float>((size_t)std::max(router_wgrad_slices(T, d, E), 1) * d * E);
    float* dbs = c.take<float>((size_t)column_sum_slices(T) * E);
    int32_t* pre_c = c.take<int32_t>((size_t)E + 1);
    int32_t* pre_d = c.take<int32_t>((size_t)E + 1);
    int32_t* pre_f = c.take<int32_t>((size_t)E + 1);
    int4* tt_c = c.take<int4>(ffn_tile_table_entries(E, C));
    int4* tt_d = c.take<int4>(ffn_tile_table_entries(E, d));
    int4* tt_f = c.take<int4>(ffn_tile_table_entries(E, F));
    if (B.dz) dz = B.dz;
    if (B.dgate) dgate = B.dgate;
    const bf16_t* x = B.x;

    // gate and router: dgate, then dz = task + aux (+ z) gradient, db_r, dW_r
    LAUNCH(K_COMBINE_BWD, "combine_bwd", s,
           launch_combine_bwd(B.dout, B.y, B.expert, slot, B.keep, B.gate, T, k, d, E, C, dy, dgate, s));
    if (tok)
        LAUNCH(K_ROUTER_DZ, "router_dz", s,
               launch_aux_grad(B.logits, B.lse, B.f, T, group_tokens(T, G), E, B.alpha, B.z_beta, B.expert, B.gate,
                               dgate, k, 0, dz, s));
    LAUNCH(K_ROUTER_DB, "router_db", s, launch_column_sum(dz, (int)T, E, dbs, B.db_r, s));
    LAUNCH(K_ROUTER_WGRAD, "router_wgrad", s, launch_router_wgrad(x, dz, T, d, E, part, B.dw_r, s));
    // experts: the two products with the weights read W1 and W2 as stored
    // (K-major).  The weight gradients take the token axis as K: with d, d_ff
    // > 64 they read dy, H, dA and buf as stored (K-major operands, rows past
    // the filled ones read as zero), else transposed copies of them
    const bool tn = ffn_wide_tiles(d) && ffn_wide_tiles(F);
    if (C > 0) {
        if (!tn) {
            LAUNCH(K_TRANSPOSE, "transpose_rows", s, launch_transpose_rows(dy, dyT, E, C, d, Cp, filled, s));
            LAUNCH(K_TRANSPOSE, "transpose_rows", s, launch_transpose_rows(B.h, hT, E, C, F, Cp, filled, s));
            LAUNCH(K_TRANSPOSE, "transpose_rows", s, launch_transpose_rows(B.buf, bufT, E, C, d, Cp, filled, s));
        }
        // the token tiles of the data products, and the d- and d_ff-row tiles of the
        // weight gradients (carrying each expert's filled row count), in one launch
        FfnTileLists tl{};
        tl.E = E;
        tl.list[0] = FfnTileListSpec{filled, nullptr, C, pre_c, tt_c};
        // (the fourth word is the filled row count only for the K-major products;
        // the transposed path's GEMM reads it as the tile count of the expert)
        tl.list[1] = FfnTileListSpec{nullptr, tn ? filled : nullptr, d, pre_d, tt_d};
        tl.list[2] = FfnTileListSpec{nullptr, tn ? filled : nullptr, F, pre_f, tt_f};
        LAUNCH(K_FFN_TILES, "ffn_tile_prefix", s, launch_ffn_tile_lists(tl, 3, s));
        // dA = (dy W2) * [H > 0]          rows: tokens, K = d, N = d_ff; W2[e] is [d][d_ff]
        LAUNCH(K_GEMM_DA, "gemm_dA", s,
               launch_grouped_gemm_kmajor_masked(dy, B.w2, pre_c, tt_c, dA, B.h, E, C, d, F, s));
        // dbuf = dA W1                    rows: tokens, K = d_ff, N = d; W1[e] is [d_ff][d]
        LAUNCH(K_GEMM_DBUF, "gemm_dbuf", s,
               launch_grouped_gemm_kmajor_f32(dA, B.w1, pre_c, tt_c, dbuf, E, C, F, d, s));
        if (!tn) LAUNCH(K_TRANSPOSE, "transpose_rows", s, launch_transpose_rows(dA, dAT, E, C, F, Cp, filled, s));
    }
    // weight gradients: K = the (zero-padded) token axis
    if (C > 0) {
        // dW2[e] = dy^T H                 rows: d, K = tokens, N = d_ff
        // dW1[e] = dA^T buf               rows: d_ff, K = tokens, N = d
        if (tn) {
            LAUNCH(K_GEMM_DW2, "gemm_dW2", s,
                   launch_grouped_gemm_tn_f32(dy, B.h, pre_d, tt_d, B.dw2, E, d, C, F, s));
            LAUNCH(K_GEMM_DW1, "gemm_dW1", s,
                   launch_grouped_gemm_tn_f32(dA, B.buf, pre_f, tt_f, B.dw1, E, F, C, d, s));
        } else {
            LAUNCH(K_GEMM_DW2, "gemm_dW2", s, launch_grouped_gemm_f32(dyT, hT, pre_d, tt_d, B.dw2, E, d, Cp, F, s));
            LAUNCH(K_GEMM_DW1, "gemm_dW1", s, launch_grouped_gemm_f32(dAT, bufT, pre_f, tt_f, B.dw1, E, F, Cp, d, s));
        }
    } else {
        LAUNCH(K_GEMM_DW2, "zero", s, launch_fill_zero(B.dw2, (int64_t)E * d * F, s));
        LAUNCH(K_GEMM_DW1, "zero", s, launch_fill_zero(B.dw1, (int64_t)E * d * F, s));
    }
    // dx = dout + sum of the kept choices' dbuf rows + dz W_r^T
    LAUNCH(K_DX, "dx_assemble", s,
           launch_dx_assemble(B.dx_branch_only ? nullptr : B.dout, dbuf, B.expert, slot, B.keep, dz, B.w_r, T, d,
                              E, k, C, B.dx, s));
    return SWITCH_OK;
}

size_t switch_workspace_bytes(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C) {
    if (T < 0 || d < 0 || d_ff < 0 || E < 1 || E > 4096 || C < 0 || T >= (int64_t(1) << 31)) return 0;
    return layer_ws(T, d, d_ff, E, C, 1, 0);
}

size_t switch_workspace_bytes_ex(int64_t T, int32_t d, int32_t d_ff, int32_t E, int32_t C, int32_t k,
                                 int64_t group) {
    if (T < 0 || d < 0 || d_ff < 0 || E < 1 || E > 4096 || C < 0 || T >= (int64_t(1) << 31)) return 0;
    if (k < 1 || k > kMaxTopK || group < 0 || T * k >= (int64_t(1) << 31)) return 0;
    if (!one_group(T, group) && T % group != 0) return 0;
    if ((int64_t)E * buffer_rows(T, group, C) >= (int64_t(1) << 31)) return 0;
    return layer_ws(T, d, d_ff, E, C, k, group);
}

const char* switch_status_string(switch_status s) {
    switch (s) {
        case SWITCH_OK: return "ok";
        case SWITCH_E_INVALID: return "invalid argument";
        case SWITCH_E_UNSUPPORTED: return "unsupported size";
        case SWITCH_E_WORKSPACE: return "workspace too small";
        case SWITCH_E_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* switch_last_error(void) { return g_err.c_str(); }

#ifndef SWITCH_SOURCE_HASH
#define SWITCH_SOURCE_HASH "unknown"
#endif
// the marker lets a reader find the hash in the file without loading it
static const char kSourceHashTag[] = "switch-source-hash:" SWITCH_SOURCE_HASH;
const char* switch_build_source_hash(void) { return kSourceHashTag + sizeof("switch-source-hash:") - 1; }

switch_status switch_route(const switch_bf16* x, const float* w_r, const float* b_r, const float* logits_in,
                           int64_t T, int32_t d, int32_t E, float* logits_out, int32_t* expert, float* gate,
                           float* lse, float* prob_sum, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    RouteArgs a{x, w_r, b_r, logits_in, T, d, E, logits_out, expert, gate, lse, prob_sum};
    CHECK(validate_route(a, ws, ws_bytes));
    return run_route(a, ws, (hipStream_t)stream);
}

switch_status switch_route_ex(const switch_bf16* x, const float* w_r, const float* b_r, const float* logits_in,
                              int64_t T, int32_t d, int32_t E, int32_t k, int64_t group, float* logits_out,
                              int32_t* expert, float* gate, float* lse, float* prob_sum, void* ws, size_t ws_bytes,
                              void* stream) {
    g_err.clear();
    RouteArgs a{x, w_r, b_r, logits_in, T, d, E, logits_out, expert, gate, lse, prob_sum, k, group};
    CHECK(validate_route(a, ws, ws_bytes));
    return run_route(a, ws, (hipStream_t)stream);
}

switch_status switch_dispatch_ex(const switch_bf16* x, const int32_t* expert, int64_t T, int32_t d, int32_t E,
                                 int32_t k, int64_t group, int32_t C, int32_t priority, int32_t* position,
                                 uint8_t* keep, int32_t* slot, int32_t* counts, int32_t* accepted,
                                 int32_t* accepted_total, int32_t* slot_token, switch_bf16* buf, void* ws,
                                 size_t ws_bytes, void* stream) {
    g_err.clear();
    DispatchArgs a{x, expert, T, d, E, C, position, keep, counts, accepted, slot_token, buf,
                   k, group, priority, slot, accepted_total};
    CHECK(validate_dispatch(a, ws, ws_bytes));
    REQUIRE(one_group(T, group) || accepted_total != nullptr || group_count(T, group) == 0,
            "accepted_total must not be NULL with several routing groups");
    NONNULL_IF(T > 0 && !one_group(T, group), slot);
    return run_dispatch(a, ws, (hipStream_t)stream);
}

switch_status switch_combine_ex(const float* y, const int32_t* expert, const int32_t* slot, const uint8_t* keep,
                                const float* gate, const switch_bf16* residual, int64_t T, int32_t d, int32_t E,
                                int32_t k, int32_t rows, switch_bf16* out, void* stream) {
    g_err.clear();
    CombineArgs a{y, expert, slot, keep, gate, residual, T, d, E, rows, out, k};
    CHECK(validate_combine(a));
    return run_combine(a, (hipStream_t)stream);
}

switch_status switch_aux_loss_ex(const int32_t* counts, const float* prob_sum, const float* logits, const float* lse,
                                 int64_t T, int32_t E, int32_t k, int64_t group, float alpha, float* f, float* P,
                                 float* loss, float* dlogits, void* stream) {
    g_err.clear();
    AuxArgs a{counts, prob_sum, logits, lse, T, E, alpha, f, P, loss, dlogits, 0.f, nullptr, k, group};
    CHECK(validate_aux(a));
    return run_aux(a, (hipStream_t)stream);
}

switch_status switch_dispatch(const switch_bf16* x, const int32_t* expert, int64_t T, int32_t d, int32_t E,
                              int32_t C, int32_t* position, uint8_t* keep, int32_t* counts, int32_t* accepted,
                              int32_t* slot_token, switch_bf16* buf, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    DispatchArgs a{x, expert, T, d, E, C, position, keep, counts, accepted, slot_token, buf};
    CHECK(validate_dispatch(a, ws, ws_bytes));
    return run_dispatch(a, ws, (hipStream_t)stream);
}

size_t switch_dispatch_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

switch_status switch_dispatch_noalloc(const switch_bf16* x, const int32_t* expert, int64_t T, int32_t d, int32_t E,
                                      int32_t C, int32_t* position, uint8_t* keep, int32_t* counts,
                                      int32_t* accepted, int32_t* slot_token, switch_bf16* buf, void* stream) {
    g_err.clear();
    DispatchArgs a{x, expert, T, d, E, C, position, keep, counts, accepted, slot_token, buf};
    CHECK(check_TE(T, E));
    const size_t need = dispatch_ws(T, E, 1, 0);
    if (need > kNoAllocScratchBytes)
        return fail(SWITCH_E_UNSUPPORTED,
                    "switch_dispatch_noalloc: T = %lld, E = %d need %zu scratch bytes, above its fixed %zu "
                    "(ceil(T / 256) * E * 4 must be <= %zu); use switch_dispatch with a workspace",
                    (long long)T, E, need, kNoAllocScratchBytes, kNoAllocScratchBytes);
    // the same checks as switch_dispatch, with the scratch as the workspace (an
    // aligned stand-in address: only its size and alignment are looked at)
    CHECK(validate_dispatch(a, reinterpret_cast<void*>(kAlign), kNoAllocScratchBytes));
    void* ws = nullptr;
    CHECK(scratch_address(&ws));
    return run_dispatch(a, ws, (hipStream_t)stream);
}

switch_status switch_expert_ffn(const switch_bf16* buf, const int32_t* accepted, const switch_bf16* w1,
                                const switch_bf16* w2, int32_t E, int32_t C, int32_t d, int32_t d_ff, float* y,
                                void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    FfnArgs a{buf, accepted, w1, w2, E, C, d, d_ff, y};
    CHECK(validate_ffn(a, ws, ws_bytes));
    return run_ffn(a, ws, (hipStream_t)stream);
}

switch_status switch_combine(const float* y, const int32_t* expert, const int32_t* position, const uint8_t* keep,
                             const float* gate, const switch_bf16* residual, int64_t T, int32_t d, int32_t E,
                             int32_t C, switch_bf16* out, void* stream) {
    g_err.clear();
    CombineArgs a{y, expert, position, keep, gate, residual, T, d, E, C, out};
    CHECK(validate_combine(a));
    return run_combine(a, (hipStream_t)stream);
}

switch_status switch_aux_loss(const int32_t* counts, const float* prob_sum, const float* logits, const float* lse,
                              int64_t T, int32_t E, float alpha, float* f, float* P, float* loss, float* dlogits,
                              void* ws, size_t ws_bytes, void* stream) {
    (void)ws; (void)ws_bytes;
    g_err.clear();
    AuxArgs a{counts, prob_sum, logits, lse, T, E, alpha, f, P, loss, dlogits, 0.f, nullptr};
    CHECK(validate_aux(a));
    return run_aux(a, (hipStream_t)stream);
}

switch_status switch_router_z_loss(const float* lse, const float* logits, int64_t T, int32_t E, float beta,
                                   float* z_loss, float* dlogits, int32_t accumulate, void* stream) {
    g_err.clear();
    CHECK(check_TE(T, E));
    REQUIRE(std::isfinite(beta), "beta must be finite");
    NONNULL(z_loss);
    NONNULL_IF(T > 0, lse);
    if (dlogits && T > 0) NONNULL(logits);
    REQUIRE(accumulate == 0 || accumulate == 1, "accumulate must be 0 or 1");
    ALIGNED4(lse); ALIGNED4(logits); ALIGNED4(z_loss); ALIGNED4(dlogits);
    hipStream_t s = (hipStream_t)stream;
    LAUNCH(K_Z_LOSS, "z_loss", s, launch_z_loss(lse, T, beta, z_loss, s));
    if (dlogits && T > 0)
        LAUNCH(K_AUX_GRAD, "aux_grad", s,
               launch_aux_grad(logits, lse, nullptr, T, T, E, 0.f, beta, nullptr, nullptr, nullptr, 1, accumulate,
                               dlogits, s));
    return SWITCH_OK;
}

switch_status switch_layer_fwd(const switch_layer_args* la, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (!la) return fail(SWITCH_E_INVALID, "args must not be NULL");
    const switch_layer_args& L = *la;
    hipStream_t s = (hipStream_t)stream;
    const int32_t k = L.k == 0 ? 1 : L.k;
    const int64_t G = L.group;
    CHECK(check_TE(L.T, L.E));
    CHECK(check_C(L.E, L.C));
    CHECK(check_kG(L.T, L.E, k, G));
    REQUIRE(L.d >= 1 && L.d_ff >= 1, "d and d_ff must be >= 1");
    SUPPORT(L.d % 64 == 0 && L.d_ff % 64 == 0, "d and d_ff must be multiples of 64 (got %d, %d)", L.d, L.d_ff);
    REQUIRE(L.residual == 0 || L.residual == 1, "residual must be 0 or 1");
    const int64_t rows64 = buffer_rows(L.T, G, L.C);
    SUPPORT((int64_t)L.E * rows64 < (int64_t(1) << 31), "E * groups * C must be < 2^31");
    const int32_t rows = (int32_t)rows64;
    const bool one = one_group(L.T, G);
    const size_t need = layer_ws(L.T, L.d, L.d_ff, L.E, L.C, k, G);
    if (ws_bytes < need) return fail(SWITCH_E_WORKSPACE, "layer needs %zu workspace bytes, got %zu", need, ws_bytes);
    REQUIRE(ws != nullptr, "ws must not be NULL");
    REQUIRE(aligned(ws, kAlign), "ws must be %zu-byte aligned", kAlign);
    Carver c{(char*)ws};
    char* route_space = c.take<char>(route_ws(L.T, L.d, L.E, true));
    char* dispatch_space = c.take<char>(dispatch_ws(L.T, L.E, k, G));
    char* ffn_space = c.take<char>(ffn_ws(L.E, rows, L.d_ff));
    float* logits = c.take<float>((size_t)L.T * L.E);
    float* lse = c.take<float>((size_t)L.T);
    float* prob_sum = c.take<float>((size_t)group_count(L.T, G) * L.E);
    bf16_t* buf = c.take<bf16_t>((size_t)L.E * rows * L.d);
    float* y = c.take<float>((size_t)L.E * rows * L.d);
    int32_t* slot_token = c.take<int32_t>((size_t)L.E * rows + kRowMapPad);
    int32_t* slot = nullptr;
    int32_t* acc_total = nullptr;
    if (!one) {
        slot = c.take<int32_t>((size_t)L.T * k);
        acc_total = c.take<int32_t>((size_t)L.E);
    }
    if (L.logits) logits = L.logits;
    else if (!L.dlogits && route_fused(L.E)) logits = nullptr;   // the fused router needs no logits array
    if (L.lse) lse = L.lse;
    if (L.prob_sum) prob_sum = L.prob_sum;
    if (L.buf) buf = L.buf;
    if (L.y) y = L.y;
    if (L.slot_token) slot_token = L.slot_token;
    if (L.slot) slot = L.slot;
    if (L.accepted_total) acc_total = L.accepted_total;
    // one group: the buffer row is the position, and accepted is per expert
    const int32_t* rows_of = one ? L.position : slot;
    const int32_t* filled = one ? L.accepted : acc_total;

    RouteArgs ra{L.x, L.w_r, L.b_r, nullptr, L.T, L.d, L.E, logits, L.expert, L.gate, lse, prob_sum, k, G};
    const float* parts = nullptr;   // partial probability rows left to the aux step
    int parts_rows = 0;
    ra.defer_reduce = true;
    ra.part_out = &parts;
    ra.part_rows_out = &parts_rows;
    DispatchArgs da{L.x, L.expert, L.T, L.d, L.E, L.C, L.position, L.keep, L.counts, L.accepted, slot_token, buf,
                    k, G, L.priority, slot, acc_total};
    FfnArgs fa{buf, filled, L.w1, L.w2, L.E, rows, L.d, L.d_ff, y, L.h};
    fa.assignments = L.T * k;
    // k = 1 with 128-row token tiles: the second GEMM writes the kept tokens'
    // output rows (and y only when asked for), gather the dropped ones, and
    // there is no combine pass
    const bool fused = k == 1 && L.T > 0 && ffn_rows_fused(rows);
    const FfnCombine cb{slot_token, L.gate, L.residual ? L.x : nullptr, L.out, L.y};
    if (fused) {
        da.out_pass = L.out;
        da.pass_residual = L.residual != 0;
        fa.cb = &cb;
    }
    // the dispatch step's extra workgroups build the expert GEMMs' token-tile
    // lists (same workspace carve as run_ffn), so no tile-prefix launch
    if (rows > 0) {
        const FfnSpace f = carve_ffn(ffn_space, L.E, rows, L.d_ff, ffn_expected_fill(fa.assignments, L.E, rows));
        da.tl0 = f.l2;
        da.tl1 = f.l1;
        fa.tiles_ready = true;
    }
    // buf and slot_token not kept: the first GEMM reads the token rows from x
    // through the (padded) workspace slot_token
    if (!L.buf && !L.slot_token && L.T > 0 && ffn_rows_fused(rows) && L.T * L.d * 2 + 2 * (int64_t)L.d + 256 < (int64_t(1) << 32)) {
        da.no_buf = true;
        fa.x_src = L.x;
        fa.x_tokens = L.T;
        fa.a_rows = slot_token;
    }
    CombineArgs ca{y, L.expert, rows_of, L.keep, L.gate, L.residual ? L.x : nullptr, L.T, L.d, L.E, rows, L.out, k};
    AuxArgs xa{L.counts, prob_sum, logits, lse, L.T, L.E, L.alpha, L.f, L.P, L.loss, L.dlogits, L.z_beta, L.z_loss,
               k, G};
    // validate everything before the first launch
    CHECK(validate_route(ra, route_space, route_ws(L.T, L.d, L.E, logits != nullptr)));
    CHECK(validate_dispatch(da, dispatch_space, dispatch_ws(L.T, L.E, k, G)));
    if (L.T > 0 && group_count(L.T, G) > 0) NONNULL(filled);
    CHECK(validate_ffn(fa, ffn_space, ffn_ws(L.E, rows, L.d_ff)));
    CHECK(validate_combine(ca));
    CHECK(validate_aux(xa));
    CHECK(run_route(ra, route_space, s));
    AuxStatsArgs aux_in_gather{};
    if (parts) {   // the scan sums the partial rows into prob_sum; gather's extra workgroup does f, P, loss
        da.parts = parts;
        da.prows = parts_rows;
        da.prob_sum = prob_sum;
        aux_in_gather = AuxStatsArgs{L.counts, prob_sum, group_tokens(L.T, G), (int)group_count(L.T, G), L.E, k,
                                     L.alpha, L.f, L.P, L.loss};
        da.aux = &aux_in_gather;
        xa.stats_done = true;
    }
    CHECK(run_dispatch(da, dispatch_space, s));
    CHECK(run_ffn(fa, ffn_space, s));
    if (!fused) CHECK(run_combine(ca, s));
    CHECK(run_aux(xa, s));
    return SWITCH_OK;
}

switch_status switch_stream_copy(void* dst, const void* src, size_t nbytes, void* stream) {
    g_err.clear();
    REQUIRE(dst && src, "dst and src must not be NULL");
    REQUIRE(nbytes % 16 == 0, "nbytes must be a multiple of 16");
    REQUIRE(aligned(dst, 16) && aligned(src, 16), "pointers must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    LAUNCH(K_COPY, "stream_copy", s, launch_stream_copy(dst, src, nbytes, s));
    return SWITCH_OK;
}

void switch_profile_enable(int on) { g_prof = on != 0; }

int switch_profile_collect(int max, int32_t* kernel_ids, float* ms) {
    int n = 0;
    int status = 0;
    for (const ProfRec& r : g_recs) {
        if (hipEventSynchronize(r.b) != hipSuccess) status = -1;
        if (n < max && status == 0) {
            float t = 0.f;
            if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) status = -1;
            if (kernel_ids) kernel_ids[n] = r.id;
            if (ms) ms[n] = t;
            ++n;
        }
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    return status ? status : n;
}

const char* switch_kernel_name(int32_t id) { return (id >= 0 && id < K_COUNT) ? kKernelNames[id] : "?"; }

int32_t switch_ffn_gemm1_token_tile(int32_t E, int32_t rows, int64_t assignments, int32_t d_ff) {
    if (E <= 0 || rows <= 0 || d_ff <= 0) return 0;
    return ffn_gemm1_token_tile(E, rows, ffn_expected_fill(assignments, E, rows), d_ff);
}

}  // extern "C"
