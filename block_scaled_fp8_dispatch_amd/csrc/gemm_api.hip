// C ABI of the plain FP8 x FP4 GEMMs and the FP8 cast (include/fp8_fp4_gemm.h): argument
// checks, workspace layout, and the launches. Host code only; the kernels are the grouped
// GEMM of gemm.hip in its plain mode (dense: rows and tiles derived in the kernel, K split
// over several workgroups when the output has few tiles), the routing kernels of route.hip
// (contiguous layout: rows grouped by their group id, stable in row order, each group padded
// to the row-tile size), the layout kernel of route.hip (masked layout), and cast.hip.
#include "fp8_fp4_gemm.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGemmMaxBlockM = 256;
constexpr int kGemmMinBlockM = 64;
// FP32 partials of the split-K dense GEMM (a fixed part of every GEMM workspace)
constexpr size_t kSplitPartialBytes = size_t(16) << 20;
// Split K only when the output tiles would fill fewer than this many workgroups
constexpr int kSplitBelowTiles = 128;
// Workgroups split-K aims for (the CUs of one MI355X)
constexpr int kSplitTargetWorkgroups = 256;

bool gemm_shape_ok(int G, int N, int K) {
    if (G < 1 || G > MOE_MAX_EXPERTS) return false;
    if (N < 16 || N % 16 != 0) return false;
    if (K < 128 || K % 128 != 0) return false;
    return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct GemmWs {
    size_t meta, blk, counts, offsets, perm, inv, tile_expert, tile_row0, partial, total;
    int max_tiles, pad_rows;
};

GemmWs gemm_ws(int max_rows, int G) {
    GemmWs w{};
    const size_t rows = (size_t)max_rows;
    const size_t nblk = (rows + kRouteChunk - 1) / kRouteChunk;
    const size_t ppad = rows + (size_t)G * (kGemmMaxBlockM - 1);
    const size_t tiles = (rows + kGemmMinBlockM - 1) / kGemmMinBlockM + G;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    w.meta = take(8 * sizeof(int32_t));
    w.blk = take((nblk * G + nblk) * sizeof(int32_t));
    w.counts = take(G * sizeof(int32_t));
    w.offsets = take((G + 1) * sizeof(int32_t));
    w.perm = take(ppad * sizeof(int32_t));
    w.inv = take(rows * sizeof(int32_t));
    w.tile_expert = take(tiles * sizeof(int32_t));
    w.tile_row0 = take(tiles * sizeof(int32_t));
    w.partial = take(kSplitPartialBytes);
    w.total = off;
    w.max_tiles = (int)tiles;
    w.pad_rows = (int)ppad;
    return w;
}

bool rows_ok(long long max_rows, int G, int K) {
    if (max_rows < 0) return false;
    if (max_rows + (long long)G * kGemmMaxBlockM >= (1ll << 31)) return false;
    if (max_rows * (long long)K >= (1ll << 32)) return false;   // 32-bit A offsets
    return true;
}

// Row-tile size from the expected rows per group (the same classes as the MoE forward)
int gemm_block_m(long long rows_per_group) {
    if (rows_per_group >= 512) return 256;
    if (rows_per_group >= 128) return 128;
    return 64;
}

GemmArgs plain_args(const uint8_t* a, const uint8_t* a_sf, int N, int K, const void* packed_b,
                    const PackedBLayout& L, uint8_t* ws, const GemmWs& W, uint16_t* d, int BM,
                    int tiles_bound) {
    GemmArgs g{};
    g.a = a;
    g.a_blocked = 0;
    g.a_sf = a_sf;
    g.a_stride = K;
    g.a_sf_stride = 4 * cdiv(K, 512);
    g.K = K;
    g.topk = 1;
    g.perm = reinterpret_cast<const int32_t*>(ws + W.perm);
    g.meta = reinterpret_cast<const int32_t*>(ws + W.meta);
    g.tile_expert = reinterpret_cast<const int32_t*>(ws + W.tile_expert);
    g.tile_row0 = reinterpret_cast<const int32_t*>(ws + W.tile_row0);
    g.n_tiles = L.n_tiles;
    g.max_tiles = tiles_bound < W.max_tiles ? tiles_bound : W.max_tiles;
    const uint8_t* pk = static_cast<const uint8_t*>(packed_b);
    g.b = pk + L.data;
    g.b_sf = reinterpret_cast<const uint32_t*>(pk + L.scales);
    g.b_expert = L.d_group;
    g.b_ntile = L.d_ntile;
    g.bs_expert = L.s_group / 4;
    g.bs_ntile = L.s_ntile / 4;
    g.hblk = BM;
    g.stage = d;
    g.topk_weights = nullptr;
    g.out_cols = N;
    g.host_tiles = -1;
    g.max_half = 0;
    g.dense_rows = 0;
    g.splits = 1;
    g.ks_split = K / kBK;
    g.partial = reinterpret_cast<float*>(ws + W.partial);
    return g;
}

// Split-K plan of a dense GEMM with `tiles` output tiles of BM rows: how many splits of
// how many K steps (a multiple of 4, so every split starts on a scale word), or 1 split.
// Every split has at least 4 steps, and the FP32 partials fit the workspace.
void split_plan(int tiles, int BM, int K, int& splits, int& ks_split) {
    const int nks = K / kBK;
    splits = 1;
    ks_split = nks;
    if (tiles >= kSplitBelowTiles || nks % 4 != 0 || nks < 8) return;
    int want = kSplitTargetWorkgroups / tiles;
    const size_t per_split = (size_t)tiles * BM * kBN * sizeof(float);
    const int fit = (int)(kSplitPartialBytes / per_split);
    want = want < fit ? want : fit;
    want = want < nks / 4 ? want : nks / 4;
    if (want < 2) return;
    ks_split = (nks + want - 1) / want;
    ks_split = (ks_split + 3) / 4 * 4;
    splits = (nks + ks_split - 1) / ks_split;
    if (splits < 2) {
        splits = 1;
        ks_split = nks;
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_gemm_packed_b_bytes(int32_t groups, int32_t n, int32_t k) {
    if (!gemm_shape_ok(groups, n, k)) return 0;
    return packed_b_layout(groups, n, k).total;
}

int moe_gemm_prepare_b(int32_t groups, int32_t n, int32_t k, const uint8_t* b,
                       const uint8_t* b_sf, void* packed, size_t packed_bytes,
                       hipStream_t stream) {
    if (!b || !b_sf || !packed) return MOE_ERR_NULL;
    if (!gemm_shape_ok(groups, n, k)) return MOE_ERR_SHAPE;
    if (!aligned16(b) || !aligned16(b_sf) || !aligned16(packed)) return MOE_ERR_ALIGN;
    const PackedBLayout L = packed_b_layout(groups, n, k);
    if (packed_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (launch_pack_b(groups, n, k, L, b, b_sf, static_cast<uint8_t*>(packed), stream) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

size_t moe_gemm_workspace_bytes(int32_t max_rows, int32_t groups) {
    if (groups < 1 || groups > MOE_MAX_EXPERTS || max_rows < 0) return 0;
    if ((long long)max_rows + (long long)groups * kGemmMaxBlockM >= (1ll << 31)) return 0;
    return gemm_ws(max_rows, groups).total;
}

int moe_fp8_fp4_gemm(uint16_t* d, const uint8_t* a, const uint8_t* a_sf, int32_t m, int32_t n,
                     int32_t k, const void* packed_b, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    if (!d || !a || !a_sf || !packed_b || !workspace) return MOE_ERR_NULL;
    if (!gemm_shape_ok(1, n, k)) return MOE_ERR_SHAPE;
    if (!aligned16(d) || !aligned16(a) || !aligned16(a_sf) || !aligned16(packed_b) ||
        !aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (!rows_ok(m, 1, k)) return MOE_ERR_TOKENS;
    const GemmWs W = gemm_ws(m, 1);
    if (workspace_bytes < W.total) return MOE_ERR_WORKSPACE;
    if (m == 0) return MOE_OK;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const int BM = gemm_block_m(m);
    // rows are 0 .. m-1 of one group: the kernels derive tiles and rows arithmetically
    const PackedBLayout L = packed_b_layout(1, n, k);
    GemmArgs g = plain_args(a, a_sf, n, k, packed_b, L, ws, W, d, BM, cdiv(m, BM));
    g.host_tiles = cdiv(m, BM);
    g.dense_rows = m;
    if (BM <= 128) {
        split_plan(cdiv(m, BM) * L.n_tiles, BM, k, g.splits, g.ks_split);
        if (g.splits > 1)
            return launch_gemm_splitk(BM, g, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    }
    if (launch_gemm_plain(BM, g, stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_m_grouped_fp8_fp4_gemm_contiguous(uint16_t* d, const uint8_t* a, const uint8_t* a_sf,
                                          const int32_t* group_of_row, int32_t m,
                                          int32_t groups, int32_t n, int32_t k,
                                          const void* packed_b, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    if (!d || !a || !a_sf || !group_of_row || !packed_b || !workspace) return MOE_ERR_NULL;
    if (!gemm_shape_ok(groups, n, k)) return MOE_ERR_SHAPE;
    if (!aligned16(d) || !aligned16(a) || !aligned16(a_sf) || !aligned16(group_of_row) ||
        !aligned16(packed_b) || !aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (!rows_ok(m, groups, k)) return MOE_ERR_TOKENS;
    const GemmWs W = gemm_ws(m, groups);
    if (workspace_bytes < W.total) return MOE_ERR_WORKSPACE;
    if (m == 0) return MOE_OK;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const int BM = gemm_block_m(m / groups);
    auto i32 = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
    // each row is one slot of a top-1 routing over `groups` experts
    if (launch_route(group_of_row, m, groups, BM, i32(W.blk), i32(W.meta), i32(W.counts),
                     i32(W.offsets), i32(W.perm), i32(W.inv), i32(W.tile_expert),
                     i32(W.tile_row0), W.max_tiles, stream) != hipSuccess)
        return MOE_ERR_HIP;
    const PackedBLayout L = packed_b_layout(groups, n, k);
    GemmArgs g = plain_args(a, a_sf, n, k, packed_b, L, ws, W, d, BM, cdiv(m, BM) + groups);
    g.max_half = groups;   // the routing may list one half tile per group
    if (launch_gemm_plain(BM, g, stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_m_grouped_fp8_fp4_gemm_masked(uint16_t* d, const uint8_t* a, const uint8_t* a_sf,
                                      const int32_t* masked_m, int32_t groups, int32_t max_m,
                                      int32_t expected_m, int32_t n, int32_t k,
                                      const void* packed_b, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    if (!d || !a || !a_sf || !masked_m || !packed_b || !workspace) return MOE_ERR_NULL;
    if (!gemm_shape_ok(groups, n, k)) return MOE_ERR_SHAPE;
    if (!aligned16(d) || !aligned16(a) || !aligned16(a_sf) || !aligned16(masked_m) ||
        !aligned16(packed_b) || !aligned16(workspace))
        return MOE_ERR_ALIGN;
    if (max_m < 0) return MOE_ERR_TOKENS;
    const long long rows = (long long)groups * max_m;
    if (!rows_ok(rows, groups, k)) return MOE_ERR_TOKENS;
    const GemmWs W = gemm_ws((int)rows, groups);
    if (workspace_bytes < W.total) return MOE_ERR_WORKSPACE;
    if (max_m == 0) return MOE_OK;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const int BM = gemm_block_m(expected_m);
    if (launch_gemm_layout(groups, max_m, masked_m, BM, W.pad_rows,
                           reinterpret_cast<int32_t*>(ws + W.perm),
                           reinterpret_cast<int32_t*>(ws + W.tile_expert),
                           reinterpret_cast<int32_t*>(ws + W.tile_row0),
                           reinterpret_cast<int32_t*>(ws + W.meta), stream) != hipSuccess)
        return MOE_ERR_HIP;
    const PackedBLayout L = packed_b_layout(groups, n, k);
    const GemmArgs g = plain_args(a, a_sf, n, k, packed_b, L, ws, W, d, BM,
                                  groups * cdiv(max_m, BM));
    if (launch_gemm_plain(BM, g, stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_cast_to_fp8(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* x_fp8,
                    uint8_t* x_sf, hipStream_t stream) {
    if (!x || !x_fp8 || !x_sf) return MOE_ERR_NULL;
    if (cols < 128 || cols % 128 != 0) return MOE_ERR_SHAPE;
    if (rows < 0) return MOE_ERR_TOKENS;
    if (!aligned16(x) || !aligned16(x_fp8) || !aligned16(x_sf)) return MOE_ERR_ALIGN;
    if (rows == 0) return MOE_OK;
    if (launch_cast_fp8(x, rows, cols, x_fp8, x_sf, stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"
