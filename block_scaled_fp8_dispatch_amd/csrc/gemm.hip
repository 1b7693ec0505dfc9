// Grouped FP8 x FP4 block-scaled GEMMs of the MoE forward, on gfx950's scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4: A e4m3, B E2M1, one UE8M0 scale per lane per
// instruction, FP32 accumulation).
//
//   Linear1 (chenxutan.com/d/1930 section 3.1 step 2): the dispatched rows of x (copied
//     into expert order by the dispatch when k <= 2, else read from x through the row list)
//     x packed W1 of the row tile's expert; the epilogue applies SwiGLU (step 3) and
//     requantises h to e4m3 with one UE8M0 scale per 1x128 block (section 11.1's per-block
//     amax scaling, rounded up to a power of two).
//   Linear2 (step 4): rows of h8 x packed W2; the epilogue writes each row, as bf16, to the
//     staging row of its (token, slot) (the combine of step 5 then weights a token's slots
//     by their top-k weights and sums them in slot order, without atomics).
//   Plain GEMM (section 4.3's FP8 x FP4 GEMM, and its M-grouped contiguous and masked
//     forms): rows of A named by the row list x packed B of the tile's group; the epilogue
//     writes each row, as bf16, to the same row of D, skipping columns past N. With few
//     output tiles (a decode-sized dense GEMM) the K steps are split over several
//     workgroups: each stores its FP32 sums, and a reduction adds the splits in order and
//     rounds once to bf16.
//
// Tiling. A workgroup of 4 waves owns a BM x 256 output tile of one expert's rows (row
// tiles come from the dispatch tile list; an expert's group is padded to BM rows). When
// the last round of 256-row tiles would be at most half full, a second launch runs its
// tiles as 128-row halves.
//
// Pipeline. The A tile of a K step (BM x 128 bytes, XOR-swizzled 16-byte chunks) and the
// B tile (16 packed fragments, 16 KB) are fetched straight into LDS rings with gfx950's
// global_load_lds_dwordx4 (no staging registers): A into 3 slots, loaded two steps ahead;
// B into 4 slots, loaded three steps ahead (3 slots and two steps for 64-row tiles, whose
// LDS must leave room for two workgroups per CU). 256-row tiles fill the CU's 160 KB. There
// is one barrier per K step, half way through its MFMAs: it waits for this wave's loads of
// the next step (only the B loads issued after them may stay in flight). B loads go out in
// the first half of a step and A loads in the second, so each has between half a step and
// a step and a half to arrive. 128-row tiles load A three steps ahead into a fourth slot,
// which gives every load a step more; they run the launches that stream weights with
// little reuse, where loads wait longest. After the barrier the next step's B fragments and first A
// fragment are read into registers, so MFMAs never wait on LDS at a step boundary. The
// steps are branch-free and carry scheduling-group hints, so the compiler places one load
// between consecutive MFMAs instead of issuing the loads as a burst. Scales are read
// straight from global memory: one 32-bit word per lane covers four K steps, and the
// instruction's byte select picks the step. B words come one per fragment; the forward's A
// words come four fragments at a time, one 16-byte load from the blocked scale layout.
//
// Operand layout of the 16x16x128 instruction with A = FP8, B = FP4 (measured on gfx950):
//   A lane 16g+i : row i, bytes 0..15 = K[16g, 16g+16), bytes 16..31 = K[64+16g, 64+16g+16)
//   B lane 16g+j : column j, 32 nibbles (low first) = K[32g, 32g+32)
//   scale lane 16b+i (A) / 16b+j (B): the 32-block b of row i / column j
//   C lane l     : C[4*(l/16) + r][l%16], r = 0..3
//
// Launch mapping. Workgroups go round-robin to the 8 XCDs (id mod 8). Each XCD owns a
// range of tile ids and its workgroups take consecutive ids in each round; tile ids walk
// groups of 4 row tiles across all column tiles, so the tiles resident on one XCD at any
// time share A rows and B columns in its L2. Where the groups divide evenly, XCD x takes
// groups x, x+8, ..., so that neighbouring XCDs share B tiles through the last-level cache.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroupM = 4;
// Shortest K (in elements) for which half tiles run in the second launch
constexpr int kHalfTileMinK = 32 * kBK;
constexpr int kThreads = 256;
// Word 3 of a raw buffer descriptor on gfx950 (32-bit data format, no swizzle); with a zero
// stride, offsets are plain byte offsets, range-checked against the record count.
constexpr int kRsrcWord3 = 0x00020000;
// Record count of a raw buffer descriptor spanning the whole 32-bit offset range (every
// A, h8 and weight offset stays below 2^32 under the accepted shapes).
constexpr int kAllRecords = -1;   // 0xFFFFFFFF

template <int N>
struct IntC {
    static constexpr int value = N;
};

#define MOE_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

// Wait for this wave's outstanding vector-memory operations (the direct-to-LDS tile loads
// included), then meet the other waves. The asm statement (with a memory clobber, so no
// LDS access moves across it) does the wait; the builtin wait before it tells the
// compiler's own wait tracking that every earlier load has landed, so it adds no waits of
// its own further on (it would otherwise wait on the tile loads issued after this point).
__device__ inline void wait_vmem_barrier() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt left at their maximum
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait for this wave's LDS accesses, then meet the other waves.
__device__ inline void wait_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// UE8M0 byte for a block whose largest magnitude is `amax` (fp32): the smallest s with
// amax <= 448 * 2^s, stored as s + 127 and clamped at 0; amax == 0 gives 127. Branch-free.
__device__ inline int requant_scale_byte(float amax) {
    const uint32_t bits = __float_as_uint(amax);
    const int ex = (int)((bits >> 23) & 0xffu);
    const uint32_t mant = bits & 0x7fffffu;
    int b = ex - 8 + (mant > 0x600000u ? 1 : 0);   // 448 = 1.75 * 2^8
    b = b < 0 ? 0 : b;                              // also covers subnormal amax (ex == 0)
    return amax == 0.f ? 127 : b;
}

// Largest of four non-negative floats over the 16 lanes of a DPP row (lanes 16r .. 16r+15),
// in every lane, for four rows at once: swap neighbours, swap pairs, mirror each half row,
// mirror the row. The values are compared as their bit patterns (non-negative floats order
// like their bits), which needs no NaN canonicalisation and lets each step be one DPP max;
// the four independent chains fill each other's DPP wait states.
__device__ inline void row16_max4(uint32_t (&m)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = max(m[r], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m[r], 0xB1, 0xF, 0xF, false));
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = max(m[r], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m[r], 0x4E, 0xF, 0xF, false));
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = max(m[r], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m[r], 0x141, 0xF, 0xF, false));
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = max(m[r], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m[r], 0x140, 0xF, 0xF, false));
}

// silu(g) * u = g * u / (1 + e^-g), with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ inline float swiglu(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// acc += A x B with one UE8M0 scale byte per lane and operand, the byte chosen by OPS
// (scale word byte OPS): v_mfma_scale_f32_16x16x128_f8f6f4 with A e4m3 (format 0), B E2M1
// (format 4, 4 registers), FP32 accumulators held in AGPRs and updated in place. Written
// as asm so that the accumulators stay tied to their registers (the builtin lets the
// register allocator rotate 256 accumulators through spare registers every K step). The
// compiler does not pad asm for MFMA hazards, so the kernel keeps them by construction:
// the A, B and scale operands are only ever written by LDS or buffer loads (never by a
// VALU instruction), and explicit s_nop padding separates the accumulators' VALU
// initialisation from the first MFMA and the last MFMA from the epilogue's reads.
template <int OPS>
__device__ inline void mfma_scaled(v4f& acc, const v8i& a, const v4i& b, uint32_t sa, uint32_t sb) {
    if constexpr (OPS == 0)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] blgp:4"
                     : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else if constexpr (OPS == 1)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,1,0] op_sel_hi:[0,0,0] blgp:4"
                     : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else if constexpr (OPS == 2)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[1,1,0] blgp:4"
                     : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,1,0] op_sel_hi:[1,1,0] blgp:4"
                     : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

template <int BM, int WAVES_M, int WAVES_N, int MODE>
struct Cfg {
    static constexpr int WM = BM / WAVES_M;
    static constexpr int WN = kBN / WAVES_N;
    static constexpr int FM = WM / 16;
    static constexpr int FN = WN / 16;
    static constexpr int A_BYTES = BM * kBK;
    // B ring depth: 4 slots (B loads 3 steps ahead) where the LDS allows it; 64-row tiles
    // keep 3 (72 KB, two workgroups per CU)
    static constexpr int KB = BM == 64 ? 3 : 4;
    static constexpr int DB = KB - 1;
    // A ring: A loads DA steps ahead into AS = DA + 1 slots. 128-row tiles have the LDS for a
    // fourth slot (128 KB), which doubles the loads a wave may keep in flight at a barrier
    // (see the step below); 256-row tiles (160 KB with three) and 64-row tiles keep three.
    static constexpr int DA = BM == 128 ? 3 : 2;
    static constexpr int AS = DA + 1;
    static constexpr int LDS_BYTES = AS * A_BYTES + KB * kBTileBytes;
    static constexpr int A_DMA = A_BYTES / 1024 / 4;   // 1 KB direct-to-LDS loads per wave
    static constexpr int B_DMA = kBTileBytes / 1024 / 4;
    static constexpr int DMA = A_DMA + B_DMA;
    static_assert(WAVES_M * WAVES_N == 4, "4 waves");
    static_assert(FM >= 2 && FM % 2 == 0, "mid-step split");
    static_assert(MODE != 1 || WAVES_N * (FN / 2) == 8, "gate/up pairing");
    static_assert(MODE != 1 || 4 * WAVES_N * BM <= A_BYTES, "epilogue fits a slot");
    static_assert(MODE == 1 || FN == 8 || FN == 4, "one 16- or 8-byte store per row");
    static_assert(MODE != 4 || BM <= 128, "split-K runs without the tail split");
    static_assert(DA == 2 || (DA == 3 && DB == 3), "issue orders written for these");
};

// STREAM: B through non-temporal loads (the second launch of the 256-row class: one row tile
// or one pair of halves per B tile, see kBAux below).
// ABLK: A in the blocked layout (Linear2's h8, Linear1's dispatch copy); otherwise A rows are
// read through the row list. A's scales: Linear2 and Linear1 read the blocked scale copy
// (h_sf, xg_sf), four fragments' words per 16-byte load, except Linear1's 64-row tiles
// without a dispatch copy, which read one word per fragment from x_sf through the row list
// (so a decode needs no gather launch: c1 -1.6 %; with 256-row tiles the per-fragment words
// cost c3 and c4 3 %). The plain GEMMs read the caller's scale rows likewise.
template <int BM, int WAVES_M, int WAVES_N, int MODE, bool ABLK, bool OUT32, bool STREAM = false>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs args) {
    // The body uses gfx950 buffer descriptors, a device-only type: the host pass of the
    // split compilation sees an empty kernel and emits only its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Cfg<BM, WAVES_M, WAVES_N, MODE>;
    constexpr int WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
    constexpr int A_BYTES = C::A_BYTES;
    constexpr int A_DMA = C::A_DMA, B_DMA = C::B_DMA, DMA = C::DMA;
    constexpr int KB = C::KB, DB = C::DB, DA = C::DA, AS = C::AS;

    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
    uint8_t* const bring = smem + AS * A_BYTES;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int g = lane >> 4;

    // ---- tile id -> (row tile, column tile), XCD-aware ----------------------------------
    // Tile ids walk groups of kGroupM row tiles across all column tiles. Workgroups go
    // round-robin to the 8 XCDs (id mod 8); each XCD owns a contiguous range of tile ids and
    // its workgroups take consecutive ids in each round, so the tiles resident on one XCD at
    // any time share A rows and B columns in its L2. The first launch runs the full row
    // tiles (the tile list's first meta[3]; all tiles where half tiles are not deferred,
    // below). With the tail split, the tiles of a last round that would be at most half full
    // are left to the second (128-row) launch, which runs each of them as two 128-row halves
    // (workgroup u: tile main_total + u/2, half u%2), and then each half tile (an expert's
    // last tile holding at most 128 rows, listed after the full tiles) as one 128-row tile.
    // A dense plain GEMM (dense_rows > 0) needs no row or tile list: tile mt is rows
    // mt*hblk .. mt*hblk+hblk-1 of group 0 (hblk = the launch's tile rows, which the tail
    // launch runs as two halves), and rows at or past dense_rows are padding
    const bool dense = MODE >= 3 && args.dense_rows > 0;
    // Tile metadata read from memory is uniform across the workgroup; readfirstlane says so,
    // so that every address and buffer descriptor derived from it stays in scalar registers
    // (where the compiler cannot prove it, a descriptor in vector registers turns each tile
    // load into a loop over lanes).
    int num_mt = dense ? (args.dense_rows + args.hblk - 1) / args.hblk : __builtin_amdgcn_readfirstlane(args.meta[0]);
    if (num_mt > args.max_tiles) num_mt = args.max_tiles;
    // Half tiles go to the second launch only where K is long: there a 128-row tile takes
    // about 0.6 of a 256-row tile's time; with short K the fixed costs of a tile dominate and
    // they stay in the first launch as ordinary 256-row tiles (both launches decide alike).
    const bool defer_half = !dense && args.K >= kHalfTileMinK;
    const int n_full = defer_half ? min(__builtin_amdgcn_readfirstlane(args.meta[3]), num_mt) : num_mt;
    const int NT = args.n_tiles;
    const int S = MODE == 4 ? args.splits : 1;   // split-K: S workgroups per output tile
    const int total = n_full * NT * S;
    int main_total = total;
    if (args.split_round > 0) {
        const int rem = total % args.split_round;
        if (rem > 0 && 2 * rem <= args.split_round) main_total = total - rem;
    }
    int v = -1, half = 0, mt, nt;
    if (!args.tail) {
        const int xcd = blockIdx.x & 7;
        const int li = blockIdx.x >> 3;
        const int per = main_total >> 3, rem = main_total & 7;
        if (li >= per + (xcd < rem ? 1 : 0)) return;
        v = xcd * per + (xcd < rem ? xcd : rem) + li;
        // Row groups interleaved over the XCDs (XCD x: groups x, x+8, ...) where that keeps
        // the split exact (every group full, a multiple of 8 groups): neighbouring groups,
        // usually rows of one expert, then run on neighbouring XCDs at the same time and
        // sweep the same column tiles together, so each B tile comes from HBM once and the
        // second XCD finds it in the last-level cache (with contiguous ranges, one XCD swept
        // an expert's B once per group, the second time from HBM)
        const int ng = n_full / kGroupM;
        if (MODE <= 2 && main_total == total && n_full % kGroupM == 0 && ng % 8 == 0 && ng > 0) {
            const int gsz = kGroupM * NT;
            const int j = li / gsz;
            v = (xcd + 8 * j) * gsz + (li - j * gsz);
        }
    } else {
        const int u = blockIdx.x;
        const int halves = 2 * (total - main_total);
        if (u < halves) {
            v = main_total + (u >> 1);
            half = u & 1;
        } else {
            const int q = u - halves;                  // half tile n_full + q / NT
            mt = n_full + q / NT;
            nt = q % NT;
            if (mt >= num_mt) return;
        }
    }
    const int split = MODE == 4 && v >= 0 ? v % S : 0;
    if (v >= 0) {
        if (MODE == 4) v /= S;
        const int grp = v / (kGroupM * NT);
        const int mt0 = grp * kGroupM;
        const int gm = min(kGroupM, n_full - mt0);
        const int vin = v - grp * kGroupM * NT;
        mt = mt0 + vin % gm;
        nt = vin / gm;
    }
    const int expert = dense ? 0 : __builtin_amdgcn_readfirstlane(args.tile_expert[mt]);
    const int row0 = (dense ? mt * args.hblk : __builtin_amdgcn_readfirstlane(args.tile_row0[mt])) + half * BM;
    // K steps of this workgroup: all of them, or (split-K) the split's range, which starts at
    // a multiple of 4 so that scale words and byte selects line up
    const int k_begin = MODE == 4 ? split * args.ks_split : 0;
    const int nks = MODE == 4 ? min(args.ks_split, args.K / kBK - k_begin) : args.K / kBK;   // >= 1

    // ---- A rows this lane fetches and reads scales for ----------------------------------
    // Every tile load and scale load is a buffer load: 32-bit per-lane offset in a VGPR,
    // per-step offset in an SGPR, base in a descriptor. DMA j of wave w fills LDS rows
    // 8*(w*A_DMA + j) .. +7 of the A tile; lane l lands at row + l/8, physical 16-byte chunk
    // l%8, which holds logical chunk (l%8) ^ (row%8).
    const int a_chunk = (lane & 7) ^ (lane >> 3);
    // A blocked (h8 for Linear2, the dispatched x for Linear1): row r of the tile at K step
    // ks sits at (tile block + ks) * hblk * 128 + (row in block) * 128, the per-step part in
    // the uniform offset. Otherwise (Linear1 without a dispatch copy) A is x itself,
    // row-major, its rows the tokens perm names (padding rows read token 0 and are never
    // stored); in the plain GEMM perm names A rows directly.
    constexpr bool blocked = ABLK;
    static_assert(!ABLK || MODE <= 2, "blocked A: the forward's GEMMs only");
    static_assert(!OUT32 || MODE == 2, "32-bit output offsets: Linear2 only");
    constexpr bool sblk = MODE == 2 || (MODE == 1 && (ABLK || BM > 64));   // A scales blocked
    static_assert(!sblk || (FM % 4 == 0 && WM % 64 == 0), "scale words of 4 fragments per load");
    const int NKB = args.K / kBK;
    const uint32_t a_kstep = blocked ? (uint32_t)args.hblk * kBK : (uint32_t)kBK;
    auto src_row = [&](int r) __attribute__((always_inline)) -> uint32_t {
        if (dense) return row0 + r < args.dense_rows ? (uint32_t)(row0 + r) : 0u;
        const int slot = args.perm[row0 + r];
        if (slot < 0) return 0u;
        return MODE == 3 ? (uint32_t)slot : (uint32_t)(slot / args.topk);
    };
    uint32_t a_off[A_DMA];
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int r = 8 * (wave * A_DMA + j) + (lane >> 3);
        if constexpr (blocked) {
            const uint32_t blk_row = (uint32_t)(row0 / args.hblk) * (uint32_t)NKB * (uint32_t)args.hblk +
                                     (uint32_t)(row0 % args.hblk + r);
            a_off[j] = blk_row * kBK + a_chunk * 16;
        } else {
            a_off[j] = src_row(r) * (uint32_t)args.a_stride + a_chunk * 16 + (uint32_t)(k_begin * kBK);
        }
    }
    // A scale words: blocked, one 16-byte load per 4 fragments (rows i, 16+i, 32+i, 48+i of
    // a 64-row group, stored together; word w of the block is w * hblk words further on);
    // otherwise one word per fragment from the A row's scale row
    constexpr int NSA = sblk ? FM / 4 : FM;
    uint32_t sa_off[NSA];
#pragma unroll
    for (int i = 0; i < NSA; ++i) {
        if constexpr (sblk) {
            const int r = wm * WM + i * 64 + (lane & 15);
            sa_off[i] = 4u * blocked_scale_word((uint32_t)(row0 + r), 0u, (uint32_t)args.a_sf_stride / 4u,
                                                (uint32_t)args.hblk);
        } else {
            const int r = wm * WM + i * 16 + (lane & 15);
            sa_off[i] = src_row(r) * (uint32_t)args.a_sf_stride +
                        (uint32_t)k_begin;   // byte of scale block k_begin (k_begin % 4 == 0)
        }
    }
    const uint32_t sa_kstep = sblk ? 4u * (uint32_t)args.hblk : 4u;   // per scale word (4 K steps)
    // B fragment index of the wave's n-th fragment
    auto bfrag = [&](int fn) __attribute__((always_inline)) -> int {
        if (MODE == 1) return fn < FN / 2 ? wn * (FN / 2) + fn : 8 + wn * (FN / 2) + (fn - FN / 2);
        return wn * FN + fn;
    };
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)args.a, 0, kAllRecords, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_asf = __builtin_amdgcn_make_buffer_rsrc((void*)args.a_sf, 0, kAllRecords, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(args.b + (size_t)expert * args.b_expert + (size_t)nt * args.b_ntile + (size_t)k_begin * kBTileBytes),
        0, kAllRecords, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs_bsf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(args.b_sf + (size_t)expert * args.bs_expert + (size_t)nt * args.bs_ntile +
                (size_t)(k_begin / 4) * (kBScaleBlockBytes / 4)),
        0, kAllRecords, kRsrcWord3);
    // 64-row tiles (a few rows per expert, so one row tile reads each weight tile) and the
    // second launch of the 256-row class (its half tiles are one row tile per expert; its
    // leftover halves run together): B data and scales through non-temporal loads, which
    // stream past the caches (c1: 157 -> 148 us; second launches: c2 -0.4 %, c3 -0.3 %). The
    // main launches of the larger classes read each B tile from several row tiles and keep
    // the default policy, which lets the later reads hit in L2 (non-temporal there: c4
    // +3.6 %, c2 +0.7 %).
    constexpr int kBAux = (BM == 64 || STREAM) ? 2 : 0;   // cache-policy bits: nt
    const uint32_t b_voff = (uint32_t)(wave * B_DMA * 1024 + lane * 16);
    const uint32_t bs_voff = (uint32_t)(lane * 4);

    // one direct-to-LDS load (j < A_DMA: A rows, else B fragments) of K step ks into ring
    // slot `slot` (ks is clamped by the caller)
    auto dma_one = [&](int ks, int slot, int j) __attribute__((always_inline)) {
        if (j < A_DMA) {
            uint8_t* As = smem + slot * A_BYTES;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, MOE_LPTR(As + (wave * A_DMA + j) * 1024), 16,
                                                     a_off[j], ks * a_kstep, 0, 0);
        } else {
            const int jj = j - A_DMA;
            uint8_t* Bs = bring + slot * kBTileBytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, MOE_LPTR(Bs + (wave * B_DMA + jj) * 1024),
                                                     16, b_voff, ks * kBTileBytes + jj * 1024, 0, kBAux);
        }
    };
    // scale load i of the 4-step block holding ks: i < NSA the A words (4 fragments' or one
    // fragment's), else the word of B fragment i - NSA
    auto scale_one = [&](int ks, int i, uint32_t* sa, uint32_t* sb) __attribute__((always_inline)) {
        const int kb = ks >> 2;
        if (i < NSA) {
            if constexpr (sblk) {
                const v4i w = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_asf, sa_off[i], kb * sa_kstep, 0));
                sa[4 * i] = w.x;
                sa[4 * i + 1] = w.y;
                sa[4 * i + 2] = w.z;
                sa[4 * i + 3] = w.w;
            } else {
                sa[i] = __builtin_amdgcn_raw_buffer_load_b32(rs_asf, sa_off[i], kb * sa_kstep, 0);
            }
        } else {
            sb[i - NSA] = __builtin_amdgcn_raw_buffer_load_b32(rs_bsf, bs_voff + bfrag(i - NSA) * 256,
                                                               kb * kBScaleBlockBytes, kBAux);
        }
    };
    // LDS fragment reads: per-lane base addresses; fragment and slot offsets are uniform
    const uint32_t a_lo = (uint32_t)((wm * WM + (lane & 15)) * kBK + ((g ^ (lane & 7)) << 4));
    const uint32_t a_hi = (uint32_t)((wm * WM + (lane & 15)) * kBK + (((g + 4) ^ (lane & 7)) << 4));
    const uint32_t b_rd = (uint32_t)(lane * 16);
    auto read_a = [&](int slot, int fm) __attribute__((always_inline)) -> v8i {
        const uint8_t* As = smem + slot * A_BYTES + fm * 16 * kBK;
        const v4i lo4 = *reinterpret_cast<const v4i*>(As + a_lo);
        const v4i hi4 = *reinterpret_cast<const v4i*>(As + a_hi);
        return (v8i){lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
    };
    auto read_b = [&](int slot, int fn) __attribute__((always_inline)) -> v4i {
        const uint8_t* Bs = bring + slot * kBTileBytes + bfrag(fn) * kFragBytes;
        return *reinterpret_cast<const v4i*>(Bs + b_rd);
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            acc[fm][fn] = (v4f){0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+a"(acc[fm][fn]));
        }
    asm volatile("s_nop 7" ::: "memory");   // accumulator writes -> first MFMA
    v4i bq[FN];
    v8i a_cur, a_nx;
    // scale words of two consecutive 4-step blocks: set (ks / 4) % 2 serves step ks
    uint32_t sa[2][FM], sb[2][FN];

    // Linear2 / plain GEMM output rows: their slots (D rows) from the row list, loaded before
    // the prologue's tile loads and first used after its wait, so that the epilogue does not
    // start with a round trip to memory (c4 -0.3 %, c3 -0.2 %); a load between the K steps
    // would make the compiler wait for every tile load in flight
    int slot[FM][4];
    if constexpr (MODE == 2 || MODE == 3) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row0 + wm * WM + fm * 16 + 4 * g + r;
                slot[fm][r] = dense ? (row < args.dense_rows ? row : -1) : args.perm[row];
            }
        asm volatile("" ::: "memory");
    }
    // prologue, in the order the steps keep (B, then scales and A): scales of block 0, A
    // and B of step 0, then the loads of the steps before step 0 as the steps would have
    // issued them. DA = 2: B of steps 1 .. DB-1, A of step 1. DA = 3: B(1), A(1), B(2), A(2).
    // So that at every barrier the loads allowed in flight are exactly those issued after
    // the A loads of the next step.
#pragma unroll
    for (int i = 0; i < NSA + FN; ++i) scale_one(0, i, sa[0], sb[0]);
#pragma unroll
    for (int j = 0; j < DMA; ++j) dma_one(0, 0, j);
    if constexpr (DA == 2) {
#pragma unroll
        for (int s2 = 1; s2 < DB; ++s2)
#pragma unroll
            for (int j = A_DMA; j < DMA; ++j) dma_one(min(s2, nks - 1), s2, j);
#pragma unroll
        for (int j = 0; j < A_DMA; ++j) dma_one(min(1, nks - 1), 1, j);
    } else {
#pragma unroll
        for (int s2 = 1; s2 < DA; ++s2) {
#pragma unroll
            for (int j = A_DMA; j < DMA; ++j) dma_one(min(s2, nks - 1), s2, j);
#pragma unroll
            for (int j = 0; j < A_DMA; ++j) dma_one(min(s2, nks - 1), s2, j);
        }
    }
    // everything after A(0) and B(0)
    constexpr int WAIT0 = DA == 2 ? (DB - 1) * B_DMA + A_DMA : (DA - 1) * DMA;
    __builtin_amdgcn_s_waitcnt(0x0F70 | (WAIT0 & 15) | (((WAIT0 >> 4) & 3) << 14));
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(WAIT0) : "memory");
    if constexpr (MODE == 2 || MODE == 3) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(slot[fm][r]));
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) bq[fn] = read_b(0, fn);
    a_nx = read_a(0, 0);

    // One K step, free of branches and scheduled by hand: every MFMA is followed by at most
    // a few memory operations, in a fixed order the compiler may not change (scheduling
    // barriers that only let ALU work move). Each A fragment is read right after the first
    // MFMA of the fragment before it. In the first half go the B loads of step ks+DB, one
    // per MFMA, into the slot of step ks-1 (every wave holds that step's B fragments in
    // registers since before the previous barrier). Half way: barrier (this wave's A and
    // B of step ks+1 have landed, every wave is past step ks-1; the B loads just issued
    // stay in flight). In the second half go, one or a few per MFMA: in the third step of
    // each 4-step block the scale words of the next block into the other scale set (needed
    // only after the next barrier, which waits for them), then the A loads of step ks+2
    // into the slot of step ks-1. Steps past the last are clamped to it: a harmless reload
    // into a free slot. Splitting the loads over both halves measured faster than issuing
    // them all in the second half; vector-memory counts retire in issue order, so a B load
    // issued before the A loads of a step waits with them.
    // The last A fragment's MFMAs reload each B fragment register with the next step's
    // fragment right after its last use, and the next step's first A fragment is read with
    // them: no double buffers.
    auto step = [&](int ks, auto ops_c, auto set_c) __attribute__((always_inline)) {
        constexpr int OPS = decltype(ops_c)::value;
        constexpr int SET = decltype(set_c)::value;
        constexpr int HALF = FM / 2 * FN;
        // the scales of the next 4-step block go out with the A loads of its first step
        constexpr int SOPS = 4 - DA;
        constexpr int NS = OPS == SOPS ? NSA + FN : 0;      // scale loads of this step
        constexpr int NOPS = NS + A_DMA;                     // second-half loads
        constexpr int PER = (NOPS + HALF - 1) / HALF;
        constexpr int PERB = (B_DMA + HALF - 1) / HALF;      // first-half loads
        const int slot = ks % AS;
        const int slot1 = (ks + 1) % AS;
        const int slota = (ks + DA) % AS;
        const int bslot1 = (ks + 1) % KB;
        const int bslotn = (ks + DB) % KB;
        const int ksa = min(ks + DA, nks - 1);
        const int ksb = min(ks + DB, nks - 1);
        auto issue = [&](int op) __attribute__((always_inline)) {
            if (op < NS) scale_one(ksa, op, sa[SET ^ 1], sb[SET ^ 1]);
            else if (op < NOPS) dma_one(ksa, slota, op - NS);
        };
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            a_cur = a_nx;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                mfma_scaled<OPS>(acc[fm][fn], a_cur, bq[fn], sa[SET][fm], sb[SET][fn]);
                if (fn == 0) a_nx = fm + 1 < FM ? read_a(slot, fm + 1) : read_a(slot1, 0);
                if (fm == FM - 1) bq[fn] = read_b(bslot1, fn);
                if (fm >= FM / 2) {
                    const int t = (fm - FM / 2) * FN + fn;
#pragma unroll
                    for (int q = 0; q < PER; ++q) issue(t * PER + q);
                } else {
                    const int t = fm * FN + fn;
#pragma unroll
                    for (int q = 0; q < PERB; ++q)
                        if (t * PERB + q < B_DMA) dma_one(ksb, bslotn, A_DMA + t * PERB + q);
                }
                __builtin_amdgcn_sched_barrier(0x7);
            }
            if (fm == FM / 2 - 1) {
                // this wave's A and B of step ks+1 (and the scales of its block) have landed;
                // still in flight may be only what was issued after A of step ks+1. DA = 2:
                // the B loads of step ks+DB. DA = 3: those of steps ks+DB-1 and ks+DB, and
                // the scales and A loads of step ks-1.
                constexpr int WN = DA == 2 ? B_DMA
                                           : 2 * B_DMA + A_DMA + ((OPS + 3) % 4 == SOPS ? NSA + FN : 0);
                static_assert(WN < 64, "vmcnt range");
                __builtin_amdgcn_s_waitcnt(0x0F70 | (WN & 15) | (((WN >> 4) & 3) << 14));
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(WN) : "memory");
            }
        }
    };

    // 8 steps per iteration: two 4-step scale blocks, one per scale set
    int ks0 = 0;
    for (; ks0 + 8 <= nks; ks0 += 8) {
        step(ks0, IntC<0>{}, IntC<0>{});
        step(ks0 + 1, IntC<1>{}, IntC<0>{});
        step(ks0 + 2, IntC<2>{}, IntC<0>{});
        step(ks0 + 3, IntC<3>{}, IntC<0>{});
        step(ks0 + 4, IntC<0>{}, IntC<1>{});
        step(ks0 + 5, IntC<1>{}, IntC<1>{});
        step(ks0 + 6, IntC<2>{}, IntC<1>{});
        step(ks0 + 7, IntC<3>{}, IntC<1>{});
    }
    if (ks0 < nks) step(ks0, IntC<0>{}, IntC<0>{});
    if (ks0 + 1 < nks) step(ks0 + 1, IntC<1>{}, IntC<0>{});
    if (ks0 + 2 < nks) step(ks0 + 2, IntC<2>{}, IntC<0>{});
    if (ks0 + 3 < nks) step(ks0 + 3, IntC<3>{}, IntC<0>{});
    if (ks0 + 4 < nks) step(ks0 + 4, IntC<0>{}, IntC<1>{});
    if (ks0 + 5 < nks) step(ks0 + 5, IntC<1>{}, IntC<1>{});
    if (ks0 + 6 < nks) step(ks0 + 6, IntC<2>{}, IntC<1>{});
    // the last steps' clamped reloads must land before the slot is reused or the wave ends
    wait_vmem_barrier();
    // Reads of the accumulators after the last MFMA need wait states, which the s_nop block
    // gives. The reads are plain register moves that the compiler may hoist above that asm
    // statement (it did: up to 32 reads, so far only of accumulators a dozen MFMAs old, which
    // is safe by distance alone); passing every accumulator through an empty asm statement
    // after it (asm statements keep their order) pins all reads below.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // last MFMA -> reads of acc
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) asm volatile("" : "+a"(acc[fm][fn]));
        // ---- epilogue, in the first A slot (every load has landed) -----------------------
        uint8_t* ep = smem;
        if constexpr (MODE == 1) {
            // Lane column l of the wave's gate fragment wn*FQ + q holds h column
            // col0 + q (the packed W1 interleaves its rows so), up fragment FQ + q the matching
            // up sum. Per row: h = silu(gate) * up, the largest |h| over the 128-block (lane,
            // DPP row, then the WAVES_N waves through LDS), the UE8M0 byte and the e4m3 codes,
            // stored as one word per lane and row.
            constexpr int FQ = FN / 2;
            const int l = lane & 15;
            uint32_t* red = reinterpret_cast<uint32_t*>(ep);              // [WAVES_N][BM] max |h| bits
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                uint32_t m[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float h[FQ];
#pragma unroll
                    for (int q = 0; q < FQ; ++q) {
                        h[q] = swiglu(acc[fm][q][r], acc[fm][q + FQ][r]);
                        acc[fm][q][r] = h[q];              // h replaces the gate sum
                    }
                    // the lane's largest |h| (abs is a free input modifier), then as bits
                    if constexpr (FQ == 4)
                        m[r] = __float_as_uint(fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3]))));
                    else
                        m[r] = __float_as_uint(fmaxf(fabsf(h[0]), fabsf(h[1])));
                }
                row16_max4(m);
                if (l == 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[wn * BM + wm * WM + fm * 16 + 4 * g + r] = m[r];
                }
            }
            wait_lds_barrier();
            // codes and scale bytes go out through buffer stores: a per-lane offset of the
            // lane's first row and columns, plus a uniform offset of the row (row0 + fm*16 + r)
            const int fw = wn * FQ;                                      // first gate fragment
            const int col0 = 64 * (fw >> 2) + 4 * l + (fw & 3);
            const __amdgpu_buffer_rsrc_t rs_h8 = __builtin_amdgcn_make_buffer_rsrc(args.h8, 0, kAllRecords, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rs_hsf = __builtin_amdgcn_make_buffer_rsrc(args.h_sf, 0, kAllRecords, kRsrcWord3);
            // h8 block (row tile, K block nt of Linear2): hblk rows of 128 bytes
            const uint32_t h_blk = ((uint32_t)(row0 / args.hblk) * (uint32_t)(args.h_stride / 128) + nt) *
                                   (uint32_t)args.hblk * 128u + (uint32_t)(row0 % args.hblk) * 128u;
            const uint32_t h_lane = (uint32_t)((wm * WM + 4 * g) * 128 + col0);
            // h_sf bytes (blocked scale layout): the tile's rows lie in one block of hblk rows,
            // and tile row wm*WM + 16*fm + 4g + r is at position base + 64*(fm/4) + 16g + 4r +
            // fm%4 of it (base = the row of the wave's first 64-row group in the block)
            const uint32_t hsf_words = (uint32_t)args.h_sf_stride / 4u;   // scale words per h row
            const uint32_t hsf_base = (uint32_t)(row0 % args.hblk) + (uint32_t)(wm * WM);
            const uint32_t hsf_u = 4u * (((uint32_t)(row0 / args.hblk) * hsf_words + ((uint32_t)nt >> 2)) *
                                         (uint32_t)args.hblk + hsf_base) + (uint32_t)(nt & 3);
            const uint32_t hsf_lane = 64u * (uint32_t)g;
            // the block maxima of all the lane's rows first (one batch of LDS reads), then the
            // scale bytes, then codes and stores; the scale bytes go out in one masked pass
            uint32_t mbv[FM][4];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rt = wm * WM + fm * 16 + 4 * g + r;
                    mbv[fm][r] = red[rt];
#pragma unroll
                    for (int w = 1; w < WAVES_N; ++w) mbv[fm][r] = max(mbv[fm][r], red[w * BM + rt]);
                }
            int bytes[FM][4];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int byte = requant_scale_byte(__uint_as_float(mbv[fm][r]));
                    bytes[fm][r] = byte;
                    const float mul = __uint_as_float((uint32_t)(254 - byte) << 23);  // 2^-(byte-127)
                    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(acc[fm][0][r] * mul, acc[fm][1][r] * mul, 0, false);
                    if constexpr (FQ == 4) {
                        pk = __builtin_amdgcn_cvt_pk_fp8_f32(acc[fm][2][r] * mul, acc[fm][3][r] * mul, pk, true);
                        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)pk, rs_h8, h_lane,
                                                              h_blk + (uint32_t)(fm * 16 + r) * 128u, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pk, rs_h8, h_lane,
                                                              h_blk + (uint32_t)(fm * 16 + r) * 128u, 0);
                    }
                }
            }
            if (wn == 0 && l == 0) {   // the scale bytes of (row, block nt)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_amdgcn_raw_buffer_store_b8(
                            (uint8_t)bytes[fm][r], rs_hsf, hsf_lane + 4u * (64u * (fm / 4) + 4u * r + fm % 4), hsf_u, 0);
            }
        } else if constexpr (MODE == 4) {
            // Split-K: the FP32 sums of this K range, row-major [BM][256] per (tile, split),
            // every row of the tile (the reduction skips padding rows and columns past N).
            // Lane column l of the wave's fragments holds columns col0 .. col0+FN-1, as below.
            const int l = lane & 15;
            const int fw = wn * FN;
            const int col0 = 128 * (fw >> 3) + 8 * l + (fw & 7);
            float* pbase = args.partial + ((size_t)((mt * NT + nt) * S + split) * BM) * kBN + col0;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float* dst = pbase + (size_t)(wm * WM + fm * 16 + 4 * g + r) * kBN;
#pragma unroll
                    for (int q = 0; q < FN / 4; ++q)
                        *reinterpret_cast<v4f*>(dst + 4 * q) = (v4f){acc[fm][4 * q][r], acc[fm][4 * q + 1][r],
                                                                     acc[fm][4 * q + 2][r], acc[fm][4 * q + 3][r]};
                }
            }
        } else {
            // Lane column l of the wave's fragments wn*FN .. wn*FN+FN-1 holds output columns
            // col0 .. col0+FN-1 (the packed W2 interleaves its rows so). Each row is rounded to
            // bf16 (round to nearest even) and stored as one FN*2-byte chunk per lane into the
            // stage row of its slot (the plain GEMM: row of D); the combine applies the top-k
            // weights. Padding rows are skipped, and so are columns past H or N (the last
            // column tile may be partly past them; H is a multiple of 128 and N of 16, so a
            // lane's chunk is wholly in or out). The rows' slots were loaded before the K loop.
            typedef float v2f __attribute__((ext_vector_type(2)));
            typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
            const int l = lane & 15;
            const int fw = wn * FN;
            const int col0 = 128 * (fw >> 3) + 8 * l + (fw & 7);
            const bool col_ok = nt * kBN + col0 < args.out_cols;
            uint16_t* sbase = args.stage + nt * kBN + col0;
            // OUT32 (Linear2 with a staging buffer of less than 4 GiB): buffer stores at 32-bit
            // byte offsets, a padding row or a column past the end sent to an offset past the
            // descriptor's range, where the store is dropped; no 64-bit address arithmetic and
            // no branch per row (c4: about -1 %). Otherwise 64-bit addresses, padding rows
            // branched around.
            const uint32_t out_limit = args.out_bytes;
            const uint32_t row_bytes = 2u * (uint32_t)args.out_cols;
            const uint32_t col_byte = 2u * (uint32_t)(nt * kBN + col0);
            const __amdgpu_buffer_rsrc_t rs_out = __builtin_amdgcn_make_buffer_rsrc(args.stage, 0, (int)out_limit, kRsrcWord3);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t pk[FN / 2];
#pragma unroll
                    for (int p = 0; p < FN / 2; ++p) {
                        const v2f x = {acc[fm][2 * p][r], acc[fm][2 * p + 1][r]};
                        pk[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf));
                    }
                    if constexpr (OUT32) {
                        const uint32_t off = slot[fm][r] >= 0 && col_ok
                                                 ? (uint32_t)slot[fm][r] * row_bytes + col_byte
                                                 : out_limit;
                        if constexpr (FN == 8)
                            __builtin_amdgcn_raw_buffer_store_b128((v4i){(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]},
                                                                   rs_out, off, 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b64((v2u){pk[0], pk[1]}, rs_out, off, 0, 0);
                    } else if (slot[fm][r] >= 0 && col_ok) {
                        uint16_t* dst = sbase + (size_t)slot[fm][r] * args.out_cols;
                        if constexpr (FN == 8)
                            *reinterpret_cast<v4i*>(dst) = (v4i){(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
                        else
                            *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
                    }
                }
            }
        }
#endif
}

// Split-K reduction of the plain GEMM: thread (tile, row, 4-column chunk) adds the S FP32
// partials of its 4 columns in split order, rounds once to bf16 (nearest even) and stores
// them into the row of D the row list names; padding rows and columns past N are skipped.
// The partial loads of 4 splits at a time are issued before their sums.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            const int32_t* __restrict__ perm,
                                                            const int32_t* __restrict__ meta,
                                                            const int32_t* __restrict__ tile_row0,
                                                            int max_tiles, int NT, int S, int BM, int N,
                                                            int dense_rows, uint16_t* __restrict__ d) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    int num_mt = dense_rows > 0 ? (dense_rows + BM - 1) / BM : meta[0];
    if (num_mt > max_tiles) num_mt = max_tiles;
    const size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t per_tile = (size_t)BM * (kBN / 4);
    const size_t tile = idx / per_tile;
    if (tile >= (size_t)num_mt * NT) return;
    const int rem = (int)(idx - tile * per_tile);
    const int row = rem / (kBN / 4), c4 = rem % (kBN / 4);
    const int mt = (int)(tile / NT), nt = (int)(tile % NT);
    const int col = nt * kBN + c4 * 4;
    if (col >= N) return;
    int out_row;
    if (dense_rows > 0) {
        out_row = mt * BM + row;
        if (out_row >= dense_rows) return;
    } else {
        out_row = perm[tile_row0[mt] + row];
        if (out_row < 0) return;
    }
    const float* p = partial + ((tile * S) * BM + row) * kBN + c4 * 4;
    const size_t stride = (size_t)BM * kBN;
    v4f sum = *reinterpret_cast<const v4f*>(p);
    int sp = 1;
    for (; sp + 4 <= S; sp += 4) {
        const v4f a0 = *reinterpret_cast<const v4f*>(p + sp * stride);
        const v4f a1 = *reinterpret_cast<const v4f*>(p + (sp + 1) * stride);
        const v4f a2 = *reinterpret_cast<const v4f*>(p + (sp + 2) * stride);
        const v4f a3 = *reinterpret_cast<const v4f*>(p + (sp + 3) * stride);
        sum += a0;
        sum += a1;
        sum += a2;
        sum += a3;
    }
    for (; sp < S; ++sp) sum += *reinterpret_cast<const v4f*>(p + sp * stride);
    const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(((v2f){sum.x, sum.y}), v2bf));
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(((v2f){sum.z, sum.w}), v2bf));
    *reinterpret_cast<uint2*>(d + (size_t)out_row * N + col) = make_uint2(lo, hi);
}

template <int BM, int WAVES_M, int WAVES_N, int MODE, bool ABLK, bool OUT32>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
    // one workgroup per possible tile; those past the tiles in use return at once
    const unsigned grid = (unsigned)a.max_tiles * (unsigned)a.n_tiles;
    grouped_gemm_kernel<BM, WAVES_M, WAVES_N, MODE, ABLK, OUT32><<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

// Workgroups of a kernel the current device runs at once (CUs x workgroups per CU),
// computed once per device; 0 if unknown.
template <int BM, int WAVES_M, int WAVES_N, int MODE, bool ABLK, bool OUT32>
int resident_workgroups() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, grouped_gemm_kernel<BM, WAVES_M, WAVES_N, MODE, ABLK, OUT32>, kThreads, 0) != hipSuccess)
            return 0;
        cached[dev] = cus * (per_cu > 0 ? per_cu : 1);
    }
    return cached[dev];
}

// Row-tile classes (4 waves each): 256 rows as 2x2 waves of 128x128, 128 rows as 2x2
// waves of 64x128, 64 rows as 1x4 waves of 64x64. The 256-row class leaves a last round
// that would be at most half full to a 128-row launch over tile halves (the tile count
// is known only on the device, so that launch always goes out and finds its share).
template <int MODE, bool ABLK, bool OUT32>
hipError_t launch_mode(int block_m, const GemmArgs& a, hipStream_t stream) {
    if (a.max_tiles == 0 || a.n_tiles == 0) return hipSuccess;
    switch (block_m) {
        case 256: {
            GemmArgs m = a;
            m.split_round = resident_workgroups<256, 2, 2, MODE, ABLK, OUT32>();
            m.tail = 0;
            hipError_t e = launch_cfg<256, 2, 2, MODE, ABLK, OUT32>(m, stream);
            if (e != hipSuccess || (m.split_round == 0 && m.max_half == 0)) return e;
            if (m.host_tiles >= 0 && m.max_half == 0) {   // tiles known on the host: launch the tail only if it has work
                const long long rem = (long long)m.host_tiles * m.n_tiles % m.split_round;
                if (rem == 0 || 2 * rem > m.split_round) return e;
            }
            GemmArgs t = m;
            t.tail = 1;
            // leftover halves (at most split_round) and the half tiles (at most one per group),
            // which the kernel defers to this launch only where K is long (with short K their
            // workgroups would all return at once: 896 of them at c3, 3 us)
            const bool defer_half = !(MODE >= 3 && m.dense_rows > 0) && m.K >= kHalfTileMinK;
            const unsigned grid = (unsigned)m.split_round + (defer_half ? (unsigned)m.max_half * (unsigned)m.n_tiles : 0u);
            if (grid == 0) return e;
            grouped_gemm_kernel<128, 2, 2, MODE, ABLK, OUT32, true><<<grid, kThreads, 0, stream>>>(t);
            return hipGetLastError();
        }
        case 128: {
            GemmArgs m = a;
            m.split_round = 0;
            m.tail = 0;
            return launch_cfg<128, 2, 2, MODE, ABLK, OUT32>(m, stream);
        }
        case 64: {
            GemmArgs m = a;
            m.split_round = 0;
            m.tail = 0;
            return launch_cfg<64, 1, 4, MODE, ABLK, OUT32>(m, stream);
        }
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_linear1(int block_m, const GemmArgs& a, hipStream_t stream) {
    return a.a_blocked ? launch_mode<1, true, false>(block_m, a, stream) : launch_mode<1, false, false>(block_m, a, stream);
}
hipError_t launch_linear2(int block_m, const GemmArgs& a, hipStream_t stream) {
    return a.out_bytes > 0 ? launch_mode<2, true, true>(block_m, a, stream)
                           : launch_mode<2, true, false>(block_m, a, stream);
}
hipError_t launch_gemm_plain(int block_m, const GemmArgs& a, hipStream_t stream) {
    return launch_mode<3, false, false>(block_m, a, stream);
}
hipError_t launch_gemm_splitk(int block_m, const GemmArgs& a, hipStream_t stream) {
    if (a.max_tiles == 0 || a.n_tiles == 0) return hipSuccess;
    GemmArgs m = a;
    m.split_round = 0;
    m.tail = 0;
    const unsigned grid = (unsigned)m.max_tiles * (unsigned)m.n_tiles * (unsigned)m.splits;
    if (block_m == 128)
        grouped_gemm_kernel<128, 2, 2, 4, false, false><<<grid, kThreads, 0, stream>>>(m);
    else if (block_m == 64)
        grouped_gemm_kernel<64, 1, 4, 4, false, false><<<grid, kThreads, 0, stream>>>(m);
    else
        return hipErrorInvalidValue;
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const size_t n = (size_t)m.max_tiles * m.n_tiles * block_m * (kBN / 4);
    splitk_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
        m.partial, m.perm, m.meta, m.tile_row0, m.max_tiles, m.n_tiles, m.splits, block_m, m.out_cols,
        m.dense_rows, m.stage);
    return hipGetLastError();
}

}  // namespace moe
