// Dispatch for the one-GPU MoE forward: per-expert histogram, block-aligned exclusive
// scan, stable permutation of the (token, slot) assignments, inverse map and tile list.
//
// The explainer (chenxutan.com/d/1930 section 3.1, step 1) describes dispatch as moving
// each token to its experts' regions; the contiguous-layout grouped GEMM
// (juejin.cn/post/7631516744872673307, "MoE模型专属优化") keeps every expert's rows
// together with each group block-aligned. After the routing, a copy moves each padded
// row's scale row into expert order, in the blocked scale layout the GEMM reads, and,
// when each token has at most two slots, its activation row too, in the blocked layout
// the GEMM reads (one contiguous 1 KB piece per load); with more slots per token the GEMM
// reads x rows through the row list instead.
//
// The same kernels group the rows of the standalone contiguous-layout GEMM (a top-1
// routing of rows to groups), and a small layout kernel builds the row and tile lists of
// the masked-layout GEMM.
//
// Up to kFusedMaxSlots slots, one launch of one workgroup does all of it (histogram,
// scan, then the stable scatter in rounds of 1024 slots): small batches are bound by
// launch latency, not work. Larger inputs take three launches, all deterministic:
//   count   one workgroup per chunk of kRouteChunk slots: per-expert histogram of the
//           chunk (LDS integer atomics; the count does not depend on their order) and
//           the chunk's number of invalid ids
//   scan    one workgroup: expert totals, per-chunk bases, padded offsets, tile list,
//           padding rows of perm set to -1, invalid-id total
//   scatter one workgroup per chunk: the stable rank of each slot among the chunk's
//           slots of the same expert (wave ballots), then perm / inv
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxE = MOE_MAX_EXPERTS;
constexpr int kSlotsPerThread = kRouteChunk / kRouteThreads;
constexpr int kFusedThreads = 1024;
constexpr int kFusedMaxSlots = 4096;   // measured: one workgroup beats three launches up to here

// Exclusive scan of `v` over the 1024 threads of a workgroup (thread order); the total
// goes to *total. warp_sums: 16 ints of LDS.
__device__ inline int block_exclusive_scan_1024(int v, int* warp_sums, int* total) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int incl = v;
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
    }
    if (lane == 63) warp_sums[wave] = incl;
    __syncthreads();
    int wave_base = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) wave_base += warp_sums[w];
        all += warp_sums[w];
    }
    *total = all;
    return wave_base + incl - v;
}

// Stable rank of slot s among the slots of this round with the same expert id, for one
// wave: lanes holding the same id match on every bit of it (ballots).
__device__ inline void wave_match(int e, bool ok, int nbits, int lane, int& rank_w, int& cnt) {
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
    }
    rank_w = __popcll(peers & lt_mask);
    cnt = __popcll(peers);
}

// Tile list of expert e (one thread per expert, all 1024 threads of the workgroup calling):
// its padded rows [excl, excl + pad) in tiles of block_m rows. With 256-row tiles, an
// expert's last tile that holds at most 128 rows is a half tile: the GEMM runs it as one
// 128-row tile in its second (128-row) launch. Half tiles go after all full tiles: full
// tiles keep their order at index (row tile - half tiles of earlier experts), and the half
// tile of expert e takes index n_full + (half tiles of earlier experts). meta[3] = n_full.
// Uses warp_sums (16 ints of LDS) for its scan.
__device__ inline void write_tile_list(int e, int E, int c, int excl, int pad, int total_rows,
                                       int block_m, int max_tiles, int* warp_sums,
                                       int32_t* __restrict__ tile_expert,
                                       int32_t* __restrict__ tile_row0, int32_t* __restrict__ meta) {
    const bool has_half = block_m == kHalfTileRows * 2 && e < E && c > 0 &&
                          c - (pad - block_m) <= kHalfTileRows;
    int n_half = 0;
    __syncthreads();                                     // warp_sums may still be read
    const int half_before = block_exclusive_scan_1024(has_half ? 1 : 0, warp_sums, &n_half);
    const int n_full = total_rows / block_m - n_half;
    if (e < E) {
        const int last = has_half ? excl + pad - block_m : excl + pad;
        for (int r = excl; r < last; r += block_m) {
            const int t = r / block_m - half_before;
            if (t < max_tiles) {
                tile_expert[t] = e;
                tile_row0[t] = r;
            }
        }
        if (has_half && n_full + half_before < max_tiles) {
            tile_expert[n_full + half_before] = e;
            tile_row0[n_full + half_before] = last;
        }
    }
    if (threadIdx.x == 0) meta[3] = n_full;
}

__global__ __launch_bounds__(kFusedThreads) void route_fused_kernel(
    const int32_t* __restrict__ idx, int num_slots, int E, int nbits, int block_m,
    int32_t* __restrict__ meta, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ tile_row0, int max_tiles) {
    __shared__ int hist[kMaxE];                          // then: next row of each expert
    __shared__ int pad_lo[kMaxE], pad_hi[kMaxE];         // padding rows [lo, hi) of each expert
    __shared__ int wave_cnt[kFusedThreads / 64][kMaxE];
    __shared__ int warp_sums[16];
    __shared__ int invalid;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += kFusedThreads) {
        hist[e] = 0;
        for (int w = 0; w < kFusedThreads / 64; ++w) wave_cnt[w][e] = 0;
    }
    if (tid == 0) invalid = 0;
    // the thread's slots tid, tid + 1024, ..., read once: the scatter below reuses them
    constexpr int kPer = kFusedMaxSlots / kFusedThreads;
    int ev[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s = i * kFusedThreads + tid;
        ev[i] = s < num_slots ? idx[s] : -1;
    }
    __syncthreads();
    // histogram and invalid ids
    int my_invalid = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = ev[i];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
        else if (e != -1) ++my_invalid;
    }
    if (my_invalid) atomicAdd(&invalid, my_invalid);
    __syncthreads();
    // padded exclusive scan over experts (thread e owns expert e), tile list, padding rows
    const int c = tid < E ? hist[tid] : 0;
    const int pad = (c + block_m - 1) / block_m * block_m;
    int total = 0;
    const int excl = block_exclusive_scan_1024(pad, warp_sums, &total);
    write_tile_list(tid, E, c, excl, pad, total, block_m, max_tiles, warp_sums, tile_expert, tile_row0, meta);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = excl;
        if (tid == E - 1) offsets[E] = excl + pad;
        pad_lo[tid] = excl + c;
        pad_hi[tid] = excl + pad;
        hist[tid] = excl;                                // next row of expert tid
    }
    if (tid == 0) {
        meta[0] = total / block_m;
        meta[1] = invalid;
        meta[2] = block_m;
    }
    __syncthreads();
    // padding rows of perm set to -1: 1024 / E threads per expert, each taking every
    // (1024 / E)-th of the expert's padding rows
    {
        const int tpe = kFusedThreads / E;
        const int e = tid / tpe, j = tid % tpe;
        if (e < E)
            for (int r = pad_lo[e] + j; r < pad_hi[e]; r += tpe) perm[r] = -1;
    }
    // stable scatter, 1024 slots per round in slot order
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int s0 = i * kFusedThreads;
        if (s0 >= num_slots) break;   // uniform
        const int s = s0 + tid;
        const bool in_range = s < num_slots;
        const int e = ev[i];
        const bool ok = e >= 0 && e < E;
        int rank_w, cnt;
        wave_match(e, ok, nbits, lane, rank_w, cnt);
        if (ok && rank_w == cnt - 1) wave_cnt[wave][e] = cnt;
        __syncthreads();
        if (ok) {
            int pos = hist[e] + rank_w;
            for (int w = 0; w < wave; ++w) pos += wave_cnt[w][e];
            perm[pos] = s;
            inv[s] = pos;
        } else if (in_range) {
            inv[s] = -1;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kFusedThreads) {
            int add = 0;
            for (int w = 0; w < kFusedThreads / 64; ++w) {
                add += wave_cnt[w][x];
                wave_cnt[w][x] = 0;
            }
            hist[x] += add;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(
    const int32_t* __restrict__ idx, int num_slots, int E, int32_t* __restrict__ blk_counts,
    int32_t* __restrict__ blk_invalid) {
    __shared__ int hist[kMaxE];
    __shared__ int invalid;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kRouteThreads) hist[e] = 0;
    if (tid == 0) invalid = 0;
    __syncthreads();
    const int base = blockIdx.x * kRouteChunk;
    int my_invalid = 0;
    for (int i = 0; i < kSlotsPerThread; ++i) {
        const int s = base + i * kRouteThreads + tid;
        if (s < num_slots) {
            const int e = idx[s];
            if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
            else if (e != -1) ++my_invalid;
        }
    }
    if (my_invalid) atomicAdd(&invalid, my_invalid);
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) blk_counts[(size_t)blockIdx.x * E + e] = hist[e];
    if (tid == 0) blk_invalid[blockIdx.x] = invalid;
}

// One workgroup of up to 1024 threads; thread e owns expert e.
__global__ __launch_bounds__(1024) void route_scan_kernel(
    int32_t* __restrict__ blk_counts, const int32_t* __restrict__ blk_invalid, int nblk, int E,
    int block_m, int32_t* __restrict__ meta, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ tile_row0, int max_tiles) {
    __shared__ int warp_sums[16];
    __shared__ int pad_lo[kMaxE], pad_hi[kMaxE];   // padding rows [lo, hi) of each expert
    __shared__ int inv_total;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // invalid ids over all chunks: a strided sum per thread, then atomics in LDS (integer,
    // so their order does not matter)
    if (tid == 0) inv_total = 0;
    int my_inv = 0;
    for (int b = tid; b < nblk; b += 1024) my_inv += blk_invalid[b];
    int c = 0;
    if (tid < E) {
        // per-chunk bases within the expert, in chunk order (exclusive prefix). The counts of
        // 16 chunks are all loaded before any is replaced, so that their loads overlap (one
        // load, then its store, per chunk waited out a memory latency per chunk).
        for (int b0 = 0; b0 < nblk; b0 += 16) {
            int v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = b0 + j < nblk ? blk_counts[(size_t)(b0 + j) * E + tid] : 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (b0 + j < nblk) blk_counts[(size_t)(b0 + j) * E + tid] = c;
                c += v[j];
            }
        }
    }
    const int pad = (c + block_m - 1) / block_m * block_m;
    // exclusive scan of `pad` over threads 0..1023 (experts in order)
    int incl = pad;
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
    }
    if (lane == 63) warp_sums[wave] = incl;
    __syncthreads();
    int wave_base = 0;
    for (int w = 0; w < wave; ++w) wave_base += warp_sums[w];
    const int excl = wave_base + incl - pad;
    int total = 0;
    for (int w = 0; w < 16; ++w) total += warp_sums[w];
    write_tile_list(tid, E, c, excl, pad, total, block_m, max_tiles, warp_sums, tile_expert, tile_row0, meta);
    if (my_inv) atomicAdd(&inv_total, my_inv);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = excl;
        if (tid == E - 1) offsets[E] = excl + pad;
        pad_lo[tid] = excl + c;
        pad_hi[tid] = excl + pad;
    }
    __syncthreads();
    // padding rows of perm set to -1: 1024 / E threads per expert (E <= 1024), each taking
    // every (1024 / E)-th of the expert's padding rows
    {
        const int tpe = 1024 / E;
        const int e = tid / tpe, j = tid % tpe;
        if (e < E)
            for (int r = pad_lo[e] + j; r < pad_hi[e]; r += tpe) perm[r] = -1;
    }
    if (tid == 0) {
        meta[0] = total / block_m;
        meta[1] = inv_total;
        meta[2] = block_m;
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t* __restrict__ idx, int num_slots, int E, int nbits,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int base[kMaxE];      // offsets[e] + rows of e in earlier chunks
    __shared__ int running[kMaxE];   // rows of e in earlier rounds of this chunk
    __shared__ int wave_cnt[kRouteThreads / 64][kMaxE];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += kRouteThreads) {
        base[e] = offsets[e] + blk_base[(size_t)blockIdx.x * E + e];
        running[e] = 0;
        for (int w = 0; w < kRouteThreads / 64; ++w) wave_cnt[w][e] = 0;
    }
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int chunk0 = blockIdx.x * kRouteChunk;
    // the thread's ids of every round, loaded before the first round (one memory latency,
    // not one per round)
    int ev[kSlotsPerThread];
#pragma unroll
    for (int round = 0; round < kSlotsPerThread; ++round) {
        const int s = chunk0 + round * kRouteThreads + tid;
        ev[round] = s < num_slots ? idx[s] : -1;
    }
#pragma unroll
    for (int round = 0; round < kSlotsPerThread; ++round) {
        const int s = chunk0 + round * kRouteThreads + tid;
        const bool in_range = s < num_slots;
        const int e = ev[round];
        const bool ok = e >= 0 && e < E;
        // lanes of this wave holding the same expert id
        uint64_t peers = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank_w = __popcll(peers & lt_mask);
        const int cnt = __popcll(peers);
        if (ok && rank_w == cnt - 1) wave_cnt[wave][e] = cnt;
        __syncthreads();
        if (ok) {
            int before = running[e];
            for (int w = 0; w < wave; ++w) before += wave_cnt[w][e];
            const int pos = base[e] + before + rank_w;
            perm[pos] = s;
            inv[s] = pos;
        } else if (in_range) {
            inv[s] = -1;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kRouteThreads) {
            int add = 0;
            for (int w = 0; w < kRouteThreads / 64; ++w) {
                add += wave_cnt[w][x];
                wave_cnt[w][x] = 0;
            }
            running[x] += add;
        }
        __syncthreads();
    }
}

// Dispatch copy: thread d writes bytes [16d, 16d+16) of the blocked buffer
// [P_pad/hblk][H/128][hblk][128] (consecutive threads, consecutive bytes): padded row
// p = blk*hblk + r, columns kb*128 + 16*c8 .. +15, from the x row of token perm[p]/k (zero
// on padding rows). With xg null only the scales are copied. The first rows*sfs/4 threads
// write word d of the blocked scale copy (consecutive threads, consecutive words): its
// padded row and word index come from inverting blocked_scale_word, its value from the
// token's scale row (zero on padding rows).
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ x,
                                                     const uint8_t* __restrict__ x_sf,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ meta, int k, int H,
                                                     int sfs, int hblk, int max_rows,
                                                     uint8_t* __restrict__ xg,
                                                     uint8_t* __restrict__ xg_sf) {
    int rows = meta[0] * hblk;
    if (rows > max_rows) rows = max_rows;
    const size_t d = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const int nkb = H / 128;
    if (xg != nullptr && d < (size_t)rows * (H / 16)) {
        const int c8 = (int)(d & 7);
        const size_t q = d >> 3;
        const int r = (int)(q % hblk);
        const size_t q2 = q / hblk;
        const int kb = (int)(q2 % nkb);
        const int blk = (int)(q2 / nkb);
        const int p = blk * hblk + r;
        const int slot = p < rows ? perm[p] : -1;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (slot >= 0) v = *reinterpret_cast<const uint4*>(x + (size_t)(slot / k) * H + kb * 128 + c8 * 16);
        *reinterpret_cast<uint4*>(xg + d * 16) = v;
    }
    const int words = sfs / 4;
    if (d < (size_t)rows * words) {
        const uint32_t per_blk = (uint32_t)words * (uint32_t)hblk;
        const uint32_t blk = (uint32_t)(d / per_blk), rem = (uint32_t)(d % per_blk);
        const uint32_t w = rem / (uint32_t)hblk, pos = rem % (uint32_t)hblk;
        const uint32_t r = (pos & ~63u) | ((pos & 3u) << 4) | ((pos >> 2) & 15u);   // 4i + f -> 16f + i
        const int p = (int)(blk * hblk + r);
        const int slot = p < rows ? perm[p] : -1;
        const uint32_t v = slot >= 0 ? reinterpret_cast<const uint32_t*>(x_sf + (size_t)(slot / k) * sfs)[w] : 0u;
        reinterpret_cast<uint32_t*>(xg_sf)[d] = v;
    }
}

// Row and tile lists of the masked plain GEMM (no routing pass: the groups' rows are known
// by position). Every workgroup scans the groups' padded sizes (group g: c_g =
// clamp(masked_m[g], 0, max_m) rows, ceil(c_g / BM) tiles), then writes perm for its share
// of padded rows: A row g * max_m + i, or -1 on padding. Workgroup 0 also writes the tile
// list and meta[0].
constexpr int kLayoutRows = 16384;

__device__ inline int upper_group(const int* off, int G, int v) {
    // largest g in [0, G) with off[g] <= v
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(1024) void gemm_layout_kernel(int G, int max_m,
                                                          const int32_t* __restrict__ masked_m,
                                                          int block_m, int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ tile_expert,
                                                          int32_t* __restrict__ tile_row0,
                                                          int32_t* __restrict__ meta) {
    __shared__ int warp_sums[16];
    __shared__ int toff[MOE_MAX_EXPERTS + 1];     // first tile of each group
    __shared__ int cnt[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    int c = 0;
    if (tid < G) {
        c = masked_m[tid];
        c = c < 0 ? 0 : (c > max_m ? max_m : c);
    }
    const int nt = (c + block_m - 1) / block_m;
    int total = 0;
    const int excl = block_exclusive_scan_1024(nt, warp_sums, &total);
    if (tid < G) {
        toff[tid] = excl;
        cnt[tid] = c;
    }
    if (tid == 0) toff[G] = total;
    __syncthreads();
    const int rows = total * block_m;
    const int r0 = blockIdx.x * kLayoutRows;
    for (int p = r0 + tid; p < rows && p < r0 + kLayoutRows; p += 1024) {
        const int t = p / block_m;
        const int g = upper_group(toff, G, t);
        const int i = p - toff[g] * block_m;
        perm[p] = i < cnt[g] ? g * max_m + i : -1;
    }
    if (blockIdx.x == 0) {
        for (int t = tid; t < total; t += 1024) {
            const int g = upper_group(toff, G, t);
            tile_expert[t] = g;
            tile_row0[t] = t * block_m;
        }
        if (tid == 0) {
            meta[0] = total;
            meta[3] = total;                             // no half tiles
        }
    }
}

}  // namespace

hipError_t launch_gemm_layout(int G, int max_m, const int32_t* masked_m, int block_m,
                              int pad_rows_cap, int32_t* perm, int32_t* tile_expert,
                              int32_t* tile_row0, int32_t* meta, hipStream_t stream) {
    if (G < 1 || G > MOE_MAX_EXPERTS) return hipErrorInvalidValue;
    const int grid = pad_rows_cap > 0 ? cdiv(pad_rows_cap, kLayoutRows) : 1;
    gemm_layout_kernel<<<grid, 1024, 0, stream>>>(G, max_m, masked_m, block_m, perm, tile_expert,
                                                  tile_row0, meta);
    return hipGetLastError();
}

hipError_t launch_gather(const uint8_t* x, const uint8_t* x_sf, const int32_t* perm,
                         const int32_t* meta, int k, int H, int sfs, int hblk, int max_rows,
                         uint8_t* xg, uint8_t* xg_sf, hipStream_t stream) {
    // one thread per 16 bytes of x copy, or per scale word when only the scales are copied
    const size_t n = (size_t)max_rows * (xg != nullptr ? H / 16 : sfs / 4);
    if (n == 0) return hipSuccess;
    gather_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(x, x_sf, perm, meta, k, H, sfs, hblk,
                                                                  max_rows, xg, xg_sf);
    return hipGetLastError();
}

hipError_t launch_route(const int32_t* topk_idx, int num_slots, int E, int block_m,
                        int32_t* blk_counts, int32_t* meta, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* inv, int32_t* tile_expert, int32_t* tile_row0,
                        int max_tiles, hipStream_t stream) {
    const int nblk = cdiv(num_slots, kRouteChunk);
    int32_t* blk_invalid = blk_counts + (size_t)nblk * E;
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    if (num_slots <= kFusedMaxSlots) {
        route_fused_kernel<<<1, kFusedThreads, 0, stream>>>(topk_idx, num_slots, E, nbits, block_m, meta,
                                                           counts, offsets, perm, inv, tile_expert,
                                                           tile_row0, max_tiles);
        return hipGetLastError();
    }
    route_count_kernel<<<nblk, kRouteThreads, 0, stream>>>(topk_idx, num_slots, E, blk_counts,
                                                            blk_invalid);
    route_scan_kernel<<<1, 1024, 0, stream>>>(blk_counts, blk_invalid, nblk, E, block_m, meta,
                                              counts, offsets, perm, tile_expert, tile_row0,
                                              max_tiles);
    route_scatter_kernel<<<nblk, kRouteThreads, 0, stream>>>(topk_idx, num_slots, E, nbits,
                                                              blk_counts, offsets, perm, inv);
    return hipGetLastError();
}

}  // namespace moe
