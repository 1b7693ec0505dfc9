/*
 * moe.h -- C ABI of the one-GPU Mega MoE forward for MI355X (gfx950).
 *
 * The operation (chenxutan.com/d/1930 sections 3.1-3.3; zevenfang.github.io DeepGEMM
 * review section 5): for T tokens with FP8 activations and their top-k expert choices,
 * run, over the E experts held by this GPU,
 *   dispatch  -> group each (token, slot) by expert, stable in (token, slot) order,
 *                each expert's group padded to a multiple of the row-tile size
 *                (juejin.cn/post/7631516744872673307, contiguous-layout grouped GEMM)
 *   Linear1   -> FP8 e4m3 activations (one UE8M0 scale per 1x128) x FP4 E2M1 weights
 *                (one UE8M0 scale per 1x32 along K), FP32 accumulation, 2I outputs
 *                (gate rows 0..I-1, up rows I..2I-1)
 *   SwiGLU    -> h = silu(gate) * up, requantised to FP8 e4m3 with one UE8M0 scale per
 *                1x128 (the smallest power of two that brings the block amax to <= 448,
 *                elements rounded to nearest even)
 *   Linear2   -> FP8 h x FP4 W2 [H, I], FP32 accumulation
 *   combine   -> y[t] = bf16( sum over slots j = 0..k-1 of topk_weights[t,j] * o[t,j] )
 *
 * Formats (chenxutan.com/d/1930 sections 4.1-4.2; zevenfang.github.io section 4):
 *   FP8   OCP e4m3fn, one byte per element (max 448; 0x7F/0xFF NaN).
 *   FP4   E2M1, two per byte, element 2i in the low nibble.
 *   UE8M0 one byte, value 2^(b-127). Activation scale rows hold 4*ceil(K/512) bytes so
 *         that four consecutive 128-blocks share one little-endian 32-bit word (byte j
 *         of word w = block 4w+j), the "four UE8M0 per int" packing; bytes past K/128
 *         are ignored.
 *   bf16  output, round to nearest even.
 *
 * Memory: every pointer argument is a device pointer, 16-byte aligned, owned by the
 * caller. The library allocates no device memory and holds no global state, so calls
 * on different streams with different workspaces are independent; the one exception is
 * moe_forward_noalloc, whose workspace is a fixed array inside the library. Every call is
 * asynchronous on `stream`; outputs are valid once the stream has reached it.
 *
 * Errors: host-detectable problems return a negative status before anything is
 * launched; a failed launch returns MOE_ERR_HIP. Bad expert ids found on the device
 * (outside [-1, E)) do not abort: the slot is skipped and counted (see
 * moe_read_diagnostics). No C++ exception crosses this interface.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem shape. num_experts = E local experts (1..1024); hidden = H and intermediate = I,
 * each a positive multiple of 128 (one 1x128 activation scale block; the pages' block
 * granularity, chenxutan.com/d/1930 section 11.1); num_topk = k (1..min(64, E));
 * max_tokens = the largest num_tokens a workspace must serve (the capacity of the pages'
 * per-rank buffer, section 3.3). Shapes whose byte offsets would not fit the kernels' 32-bit
 * offsets are refused (MOE_ERR_SHAPE). */
typedef struct {
    int32_t num_experts;
    int32_t hidden;
    int32_t intermediate;
    int32_t num_topk;
    int32_t max_tokens;
} moe_shape_t;

enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,      /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,     /* shape outside the supported set */
    MOE_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = -4, /* workspace or packed buffer too small */
    MOE_ERR_TOKENS = -5,    /* num_tokens < 0 or > max_tokens */
    MOE_ERR_HIP = -6,       /* a HIP call or kernel launch failed */
    MOE_ERR_SCRATCH = -7    /* moe_forward_noalloc: the call needs more than its fixed scratch */
};

/* Limits of the shapes this library accepts. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64

/* Bytes of the packed weight buffer for `shape` (W1 and W2 with their scales, in the
 * kernels' fragment order): the destination of the one-time weight transform that the
 * pages' call sequence runs before any forward (chenxutan.com/d/1930 section 3.3,
 * transform_weights_for_mega_moe). The input's byte count, plus W2's last 256-row column
 * tile completed with zero rows when H is an odd multiple of 128. Returns 0 if the shape
 * is unsupported. */
size_t moe_packed_weights_bytes(const moe_shape_t* shape);

/* Weight transform (the pages' transform_weights_for_mega_moe, chenxutan.com/d/1930
 * section 3.3): reorders FP4 nibbles and UE8M0 scale bytes into the layout the
 * grouped-GEMM kernels read with one 16-byte load per lane.
 *   w1     u8 [E, 2I, H/2]   FP4 E2M1 pairs; rows 0..I-1 gate, I..2I-1 up
 *   w1_sf  u8 [E, 2I, H/32]  UE8M0, one per 32 consecutive K
 *   w2     u8 [E, H, I/2]
 *   w2_sf  u8 [E, H, I/32]
 *   packed device buffer of moe_packed_weights_bytes(shape) bytes (caller-owned)
 * Asynchronous; inputs may be freed once the stream has passed the call. */
int moe_prepare_weights(const moe_shape_t* shape,
                        const uint8_t* w1, const uint8_t* w1_sf,
                        const uint8_t* w2, const uint8_t* w2_sf,
                        void* packed, size_t packed_bytes, hipStream_t stream);

/* Bytes of the workspace `moe_forward` needs for up to shape->max_tokens tokens
 * (routing tables, FP8 intermediate with its scales, per-slot bf16 staging): the analogue
 * of the per-rank buffer the pages size from (E, max tokens, k, H, I) before the first
 * forward (chenxutan.com/d/1930 section 3.3, get_symm_buffer_for_mega_moe), without the
 * symmetric-memory part, since one GPU exchanges nothing. Returns 0 if the shape is
 * unsupported. */
size_t moe_workspace_bytes(const moe_shape_t* shape);

/* The forward (the pages' fp8_fp4_mega_moe, chenxutan.com/d/1930 section 3.3).
 *   y_bf16        u16 [T, H] output, fully overwritten (bf16 bit patterns)
 *   x_fp8         u8  [T, H] e4m3fn codes
 *   x_sf          u8  [T, 4*ceil(H/512)] UE8M0 per 1x128 block (see Formats)
 *   topk_idx      i32 [T, k] expert id per slot; -1 = unused slot
 *   topk_weights  f32 [T, k] routing weights, applied as given
 *   num_tokens    T, 0 <= T <= shape->max_tokens (T = 0 returns MOE_OK, no launch)
 *   packed        buffer filled by moe_prepare_weights for the same shape
 *   workspace     >= moe_workspace_bytes(shape) bytes; contents need no initialisation
 * Calls sharing one workspace must be ordered (same stream or synchronised). */
int moe_forward(uint16_t* y_bf16,
                const uint8_t* x_fp8, const uint8_t* x_sf,
                const int32_t* topk_idx, const float* topk_weights,
                int32_t num_tokens, const moe_shape_t* shape, const void* packed,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_forward, also recording five caller-created events on `stream` at the stage
 * boundaries: events[0] before dispatch, [1] after dispatch, [2] after Linear1 (with its
 * SwiGLU/requant epilogue), [3] after Linear2, [4] after
 * the combine. For per-stage timing with hipEventElapsedTime; nothing synchronises.
 * events must point to 5 valid hipEvent_t; other arguments as for moe_forward. */
int moe_forward_events(uint16_t* y_bf16,
                       const uint8_t* x_fp8, const uint8_t* x_sf,
                       const int32_t* topk_idx, const float* topk_weights,
                       int32_t num_tokens, const moe_shape_t* shape, const void* packed,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       hipEvent_t* events);

/* Largest workspace, in bytes, that moe_forward_noalloc can serve from its fixed scratch
 * array: 64 MiB, which covers decode-sized calls (for instance 256 tokens, 32 experts,
 * top-8, H = 7168, I = 2048 needs 49 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory or size a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments and results as moe_forward, without workspace and workspace_bytes: the routing
 * tables, the FP8 intermediate and the staging rows live in a device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes inside the library (one per GPU, held until the process
 * ends), laid out as moe_workspace_layout gives for a shape with max_tokens = num_tokens.
 * A call whose layout would need more returns MOE_ERR_SCRATCH before anything is launched.
 * The call allocates nothing; its first call on a device looks up that device's copy of
 * the array (hipGetSymbolAddress). Every call on one GPU shares its array, which keeps the
 * last call's contents (no call needs it cleared): calls that overlap on one GPU (on
 * different streams without ordering, or from several host threads) race and give wrong
 * results; order them on one stream or synchronise between them. */
int moe_forward_noalloc(uint16_t* y_bf16,
                        const uint8_t* x_fp8, const uint8_t* x_sf,
                        const int32_t* topk_idx, const float* topk_weights,
                        int32_t num_tokens, const moe_shape_t* shape, const void* packed,
                        hipStream_t stream);

/* Where the last moe_forward on `workspace` left its routing tables and
 * intermediates (byte offsets from the workspace base; for tests and tools). */
typedef struct {
    int32_t block_m;        /* rows per tile (the padding granularity) used for T */
    int32_t max_tiles;      /* capacity of the tile list */
    size_t meta;            /* i32[8]: [0] tiles used, [1] invalid ids, [2] block_m, [3] full
                               tiles: with block_m 256, an expert's last tile holding at most
                               128 rows is listed after all full tiles (run as a 128-row tile) */
    size_t counts;          /* i32[E]      rows per expert */
    size_t offsets;         /* i32[E+1]    padded group starts */
    size_t perm;            /* i32[P_pad]  slot t*k+j per row, -1 on padding */
    size_t inv;             /* i32[T*k]    row of each slot, -1 if skipped */
    size_t tile_expert;     /* i32[max_tiles] */
    size_t tile_row0;       /* i32[max_tiles] */
    size_t h8;              /* u8 FP8 intermediate in blocks of block_m rows x 128 columns,
                               [P_pad/block_m][I/128][block_m][128]: padded row p, column c
                               at ((p/block_m)*(I/128) + c/128)*block_m*128 + (p%block_m)*128
                               + c%128 */
    size_t h_sf;            /* u8 its UE8M0 scales, one byte per (padded row, 128-column
                               block), in the blocked scale layout: with W = h_sf_stride/4
                               32-bit words per row (word w = bytes of blocks 4w..4w+3) and
                               r = p % block_m, word w of row p is word
                               ((p/block_m)*W + w)*block_m + (r/64)*64 + (r%16)*4 + (r/16)%4
                               (within 64 rows, row 16f+i at 4i+f) */
    size_t h_sf_stride;     /* scale bytes per row (4*ceil(I/512)) */
    size_t stage;           /* u16[T*k, H]  weighted bf16 Linear2 rows, by slot */
    size_t xg;              /* u8 the dispatched activations, only when num_topk <= 2 (zero
                               bytes otherwise: xg == xg_sf): the x row of each padded row's
                               token (zero on padding rows), blocked like h8 with H columns:
                               [P_pad/block_m][H/128][block_m][128] */
    size_t xg_sf;           /* u8 the scale rows of the dispatched tokens, 4*ceil(H/512)
                               bytes per padded row in the blocked scale layout of h_sf, zero
                               on padding rows; written for num_topk <= 2 and for 128- and
                               256-row tiles (with 64-row tiles and num_topk > 2 Linear1 reads
                               x_sf through perm and the region is left untouched) */
    size_t total;           /* bytes used */
} moe_layout_t;

int moe_workspace_layout(const moe_shape_t* shape, int32_t num_tokens, moe_layout_t* out);

/* Synchronous: waits for `stream`, then copies the number of skipped invalid expert
 * ids of the last forward on `workspace` into *invalid_ids and, if counts_out is not
 * NULL, the E per-expert row counts. */
int moe_read_diagnostics(const moe_shape_t* shape, const void* workspace,
                         int32_t* invalid_ids, int32_t* counts_out, hipStream_t stream);

/* Human-readable name of a status code. */
const char* moe_status_string(int status);

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
