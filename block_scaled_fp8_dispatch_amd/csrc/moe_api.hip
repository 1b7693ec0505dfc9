// C ABI of the MoE library: argument checks, workspace layout, tile-class choice and the
// launch sequence route -> Linear1(+SwiGLU+requant) -> Linear2(+weights) -> combine.
// Everything is enqueued on the caller's stream; nothing here synchronises except
// moe_read_diagnostics, and nothing allocates device memory.
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxBlockM = 256;
constexpr int kMinBlockM = 64;
// Largest top-k for which dispatch copies x into the blocked layout Linear1 reads. The copy
// pays off when each token is copied at most twice: at T=8192, k=2 it makes Linear1 4-5 %
// faster for 1 % of the forward; at k=8 it costs more than it saves.
constexpr int kDispatchCopyMaxTopk = 2;

bool shape_ok(const moe_shape_t* s) {
    if (!s) return false;
    if (s->num_experts < 1 || s->num_experts > MOE_MAX_EXPERTS) return false;
    if (s->hidden < 128 || s->hidden % 128 != 0) return false;
    if (s->intermediate < 128 || s->intermediate % 128 != 0) return false;
    if (s->num_topk < 1 || s->num_topk > MOE_MAX_TOPK || s->num_topk > s->num_experts) return false;
    if (s->max_tokens < 0) return false;
    const uint64_t slots = (uint64_t)s->max_tokens * (uint64_t)s->num_topk;
    if (slots >= (1ull << 31)) return false;
    const uint64_t ppad = slots + (uint64_t)s->num_experts * (kMaxBlockM - 1);
    // 32-bit row offsets inside the GEMM kernels
    if ((uint64_t)s->max_tokens * (uint64_t)s->hidden >= (1ull << 32)) return false;
    if (ppad * (uint64_t)s->intermediate >= (1ull << 32)) return false;
    if (s->num_topk <= kDispatchCopyMaxTopk && ppad * (uint64_t)s->hidden >= (1ull << 32))
        return false;
    return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Row-tile class from the mean rows per expert; MOE_BLOCK_M (64, 128 or 256) overrides it
// for tuning.
int choose_block_m(const moe_shape_t& s, int T) {
    static const int forced = [] {
        const char* v = std::getenv("MOE_BLOCK_M");
        const int b = v ? std::atoi(v) : 0;
        return (b == 64 || b == 128 || b == 256) ? b : 0;
    }();
    if (forced) return forced;
    const long avg = (long)T * s.num_topk / s.num_experts;
    if (avg >= 512) return 256;
    if (avg >= 128) return 128;
    return 64;
}

struct WsLayout {
    moe_layout_t pub;
    size_t blk;        // i32 [nblk * E] chunk histograms, then i32 [nblk] invalid counts
    int max_pad_rows;
};

WsLayout ws_layout(const moe_shape_t& s) {
    WsLayout w{};
    const size_t E = s.num_experts, H = s.hidden, I = s.intermediate;
    const size_t slots = (size_t)s.max_tokens * s.num_topk;
    const size_t nblk = (slots + kRouteChunk - 1) / kRouteChunk;
    const size_t ppad = slots + E * (kMaxBlockM - 1);
    const size_t max_tiles = (slots + kMinBlockM - 1) / kMinBlockM + E;
    const size_t sfs = 4 * ((I + 511) / 512);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    w.pub.meta = take(8 * sizeof(int32_t));
    w.pub.counts = take(E * sizeof(int32_t));
    w.pub.offsets = take((E + 1) * sizeof(int32_t));
    w.blk = take((nblk * E + nblk) * sizeof(int32_t));
    w.pub.perm = take(ppad * sizeof(int32_t));
    w.pub.inv = take(slots * sizeof(int32_t));
    w.pub.tile_expert = take(max_tiles * sizeof(int32_t));
    w.pub.tile_row0 = take(max_tiles * sizeof(int32_t));
    w.pub.h8 = take(ppad * I);
    w.pub.h_sf = take(ppad * sfs);
    w.pub.h_sf_stride = sfs;
    w.pub.stage = take(slots * H * sizeof(uint16_t));
    const bool copy = s.num_topk <= kDispatchCopyMaxTopk;
    w.pub.xg = take(copy ? ppad * H : 0);
    w.pub.xg_sf = take(ppad * 4 * ((H + 511) / 512));
    w.pub.total = off;
    w.pub.max_tiles = (int32_t)max_tiles;
    w.max_pad_rows = (int)ppad;
    return w;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_version(void) { return 10000; }

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "null pointer";
        case MOE_ERR_SHAPE: return "unsupported shape";
        case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "buffer too small";
        case MOE_ERR_TOKENS: return "num_tokens out of range";
        case MOE_ERR_HIP: return "HIP error";
        case MOE_ERR_SCRATCH: return "problem exceeds the library's fixed scratch buffer";
        default: return "unknown status";
    }
}

size_t moe_packed_weights_bytes(const moe_shape_t* shape) {
    if (!shape_ok(shape)) return 0;
    return packed_layout(*shape).total;
}

size_t moe_workspace_bytes(const moe_shape_t* shape) {
    if (!shape_ok(shape)) return 0;
    return ws_layout(*shape).pub.total;
}

int moe_workspace_layout(const moe_shape_t* shape, int32_t num_tokens, moe_layout_t* out) {
    if (!out || !shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    if (num_tokens < 0 || num_tokens > shape->max_tokens) return MOE_ERR_TOKENS;
    WsLayout w = ws_layout(*shape);
    w.pub.block_m = choose_block_m(*shape, num_tokens);
    *out = w.pub;
    return MOE_OK;
}

int moe_prepare_weights(const moe_shape_t* shape, const uint8_t* w1, const uint8_t* w1_sf,
                        const uint8_t* w2, const uint8_t* w2_sf, void* packed,
                        size_t packed_bytes, hipStream_t stream) {
    if (!shape || !w1 || !w1_sf || !w2 || !w2_sf || !packed) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    if (!aligned16(w1) || !aligned16(w1_sf) || !aligned16(w2) || !aligned16(w2_sf) ||
        !aligned16(packed))
        return MOE_ERR_ALIGN;
    const PackedLayout L = packed_layout(*shape);
    if (packed_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (launch_pack(*shape, L, w1, w1_sf, w2, w2_sf, static_cast<uint8_t*>(packed), stream) !=
        hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

static int forward_impl(uint16_t* y_bf16, const uint8_t* x_fp8, const uint8_t* x_sf,
                        const int32_t* topk_idx, const float* topk_weights, int32_t num_tokens,
                        const moe_shape_t* shape, const void* packed, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
    if (!shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    if (num_tokens < 0 || num_tokens > shape->max_tokens) return MOE_ERR_TOKENS;
    if (!y_bf16 || !x_fp8 || !x_sf || !topk_idx || !topk_weights || !packed || !workspace)
        return MOE_ERR_NULL;
    if (!aligned16(y_bf16) || !aligned16(x_fp8) || !aligned16(x_sf) || !aligned16(topk_idx) ||
        !aligned16(topk_weights) || !aligned16(packed) || !aligned16(workspace))
        return MOE_ERR_ALIGN;
    const WsLayout W = ws_layout(*shape);
    if (workspace_bytes < W.pub.total) return MOE_ERR_WORKSPACE;
    if (num_tokens == 0) return MOE_OK;
    auto mark = [&](int i) { return events ? hipEventRecord(events[i], stream) : hipSuccess; };

    const moe_shape_t& s = *shape;
    const int T = num_tokens, E = s.num_experts, H = s.hidden, I = s.intermediate, k = s.num_topk;
    const int BM = choose_block_m(s, T);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    auto i32 = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
    int32_t* meta = i32(W.pub.meta);
    int32_t* perm = i32(W.pub.perm);
    int32_t* tile_e = i32(W.pub.tile_expert);
    int32_t* tile_r = i32(W.pub.tile_row0);

    // The gather copies the x rows of the dispatched tokens into expert order (xg) for
    // top-k <= 2, and their scale rows into the blocked scale copy (xg_sf) for top-k <= 2
    // and for 128- and 256-row tiles. With 64-row tiles and top-k > 2 Linear1 reads x and
    // x_sf through the row list and there is no gather.
    const int xsfs = 4 * ((H + 511) / 512);
    const bool dispatch_copy = k <= kDispatchCopyMaxTopk;
    const bool scale_copy = dispatch_copy || BM > 64;
    if (mark(0) != hipSuccess) return MOE_ERR_HIP;
    if (launch_route(topk_idx, T * k, E, BM, i32(W.blk), meta, i32(W.pub.counts),
                     i32(W.pub.offsets), perm, i32(W.pub.inv), tile_e, tile_r, W.pub.max_tiles,
                     stream) != hipSuccess)
        return MOE_ERR_HIP;
    if (scale_copy && launch_gather(x_fp8, x_sf, perm, meta, k, H, xsfs, BM, W.max_pad_rows,
                                    dispatch_copy ? ws + W.pub.xg : nullptr, ws + W.pub.xg_sf,
                                    stream) != hipSuccess)
        return MOE_ERR_HIP;
    if (mark(1) != hipSuccess) return MOE_ERR_HIP;

    const PackedLayout L = packed_layout(s);
    const uint8_t* pk = static_cast<const uint8_t*>(packed);
    // The grid covers every tile the routing of T tokens can produce.
    const int tiles_bound = (T * k + BM - 1) / BM + E;
    const int max_tiles = tiles_bound < W.pub.max_tiles ? tiles_bound : W.pub.max_tiles;

    GemmArgs a1{};
    a1.host_tiles = -1;   // the tile count is known only on the device
    a1.max_half = E;      // the routing may list one half tile per expert
    a1.dense_rows = 0;
    a1.a = dispatch_copy ? ws + W.pub.xg : x_fp8;
    a1.a_sf = scale_copy ? ws + W.pub.xg_sf : x_sf;
    a1.a_blocked = dispatch_copy ? 1 : 0;
    a1.a_stride = H;
    a1.a_sf_stride = xsfs;
    a1.K = H;
    a1.topk = k;
    a1.perm = perm;
    a1.meta = meta;
    a1.tile_expert = tile_e;
    a1.tile_row0 = tile_r;
    a1.n_tiles = I / 128;
    a1.max_tiles = max_tiles;
    a1.b = pk + L.w1d;
    a1.b_sf = reinterpret_cast<const uint32_t*>(pk + L.w1s);
    a1.b_expert = L.w1d_expert;
    a1.b_ntile = L.w1d_ntile;
    a1.bs_expert = L.w1s_expert / 4;
    a1.bs_ntile = L.w1s_ntile / 4;
    a1.h8 = ws + W.pub.h8;
    a1.h_sf = ws + W.pub.h_sf;
    a1.h_stride = I;
    a1.hblk = BM;
    a1.h_sf_stride = (int)W.pub.h_sf_stride;
    if (launch_linear1(BM, a1, stream) != hipSuccess) return MOE_ERR_HIP;
    if (mark(2) != hipSuccess) return MOE_ERR_HIP;

    GemmArgs a2 = a1;
    a2.a = ws + W.pub.h8;
    a2.a_sf = ws + W.pub.h_sf;
    a2.a_blocked = 1;
    a2.a_stride = I;
    a2.a_sf_stride = (int)W.pub.h_sf_stride;
    a2.K = I;
    a2.n_tiles = cdiv(H, 256);   // a last tile of 128 columns when H is an odd multiple of 128
    a2.b = pk + L.w2d;
    a2.b_sf = reinterpret_cast<const uint32_t*>(pk + L.w2s);
    a2.b_expert = L.w2d_expert;
    a2.b_ntile = L.w2d_ntile;
    a2.bs_expert = L.w2s_expert / 4;
    a2.bs_ntile = L.w2s_ntile / 4;
    a2.stage = reinterpret_cast<uint16_t*>(ws + W.pub.stage);
    a2.topk_weights = topk_weights;
    a2.out_cols = H;
    // Below 4 GiB of staging rows Linear2 addresses them by 32-bit byte offsets
    const uint64_t stage_bytes = (uint64_t)T * k * H * sizeof(uint16_t);
    a2.out_bytes = stage_bytes < (1ull << 32) ? (uint32_t)stage_bytes : 0u;
    if (launch_linear2(BM, a2, stream) != hipSuccess) return MOE_ERR_HIP;
    if (mark(3) != hipSuccess) return MOE_ERR_HIP;

    if (launch_combine(reinterpret_cast<const uint16_t*>(ws + W.pub.stage), topk_idx, topk_weights,
                       T, k, E, H, y_bf16, stream) != hipSuccess)
        return MOE_ERR_HIP;
    if (mark(4) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_forward(uint16_t* y_bf16, const uint8_t* x_fp8, const uint8_t* x_sf,
                const int32_t* topk_idx, const float* topk_weights, int32_t num_tokens,
                const moe_shape_t* shape, const void* packed, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
    return forward_impl(y_bf16, x_fp8, x_sf, topk_idx, topk_weights, num_tokens, shape, packed,
                        workspace, workspace_bytes, stream, nullptr);
}

int moe_forward_events(uint16_t* y_bf16, const uint8_t* x_fp8, const uint8_t* x_sf,
                       const int32_t* topk_idx, const float* topk_weights, int32_t num_tokens,
                       const moe_shape_t* shape, const void* packed, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
    if (!events) return MOE_ERR_NULL;
    for (int i = 0; i < 5; ++i)
        if (!events[i]) return MOE_ERR_NULL;
    return forward_impl(y_bf16, x_fp8, x_sf, topk_idx, topk_weights, num_tokens, shape, packed,
                        workspace, workspace_bytes, stream, events);
}

// Scratch of moe_forward_noalloc: a fixed device array in this library's code object, one
// copy per GPU, held until the process ends. Host code never passes `scratch` itself to a
// kernel or a copy (on the host it only names the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on a HIP error).
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

int moe_forward_noalloc(uint16_t* y_bf16, const uint8_t* x_fp8, const uint8_t* x_sf,
                        const int32_t* topk_idx, const float* topk_weights, int32_t num_tokens,
                        const moe_shape_t* shape, const void* packed, hipStream_t stream) {
    if (!shape) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    if (num_tokens < 0 || num_tokens > shape->max_tokens) return MOE_ERR_TOKENS;
    if (!y_bf16 || !x_fp8 || !x_sf || !topk_idx || !topk_weights || !packed) return MOE_ERR_NULL;
    if (!aligned16(y_bf16) || !aligned16(x_fp8) || !aligned16(x_sf) || !aligned16(topk_idx) ||
        !aligned16(topk_weights) || !aligned16(packed))
        return MOE_ERR_ALIGN;
    // the workspace regions sized for this call's tokens, all inside the scratch array
    moe_shape_t s = *shape;
    s.max_tokens = num_tokens;
    if (ws_layout(s).pub.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    if (num_tokens == 0) return MOE_OK;
    void* ws = scratch_address();
    if (!ws) return MOE_ERR_HIP;
    return forward_impl(y_bf16, x_fp8, x_sf, topk_idx, topk_weights, num_tokens, &s, packed, ws,
                        (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_read_diagnostics(const moe_shape_t* shape, const void* workspace, int32_t* invalid_ids,
                         int32_t* counts_out, hipStream_t stream) {
    if (!shape || !workspace || !invalid_ids) return MOE_ERR_NULL;
    if (!shape_ok(shape)) return MOE_ERR_SHAPE;
    const WsLayout W = ws_layout(*shape);
    const uint8_t* ws = static_cast<const uint8_t*>(workspace);
    if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
    int32_t meta[8];
    if (hipMemcpy(meta, ws + W.pub.meta, sizeof(meta), hipMemcpyDeviceToHost) != hipSuccess)
        return MOE_ERR_HIP;
    *invalid_ids = meta[1];
    if (counts_out &&
        hipMemcpy(counts_out, ws + W.pub.counts, sizeof(int32_t) * shape->num_experts,
                  hipMemcpyDeviceToHost) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"
