// Grouped FP8 x FP4 block-scaled GEMMs of the MoE forward, on gfx950's scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4: A e4m3, B E2M1, one UE8M0 scale per lane per
// instruction, FP32 accumulation).
//
//   Linear1 (chenxutan.com/d/1930 section 3.1 step 2): rows of x gathered through the
//     dispatch permutation x packed W1 of the row tile's expert; the epilogue applies
//     SwiGLU (step 3) and requantises h to e4m3 with one UE8M0 scale per 1x128 block
//     (section 11.1's per-block amax scaling, rounded up to a power of two).
//   Linear2 (step 4): rows of h8 x packed W2; the epilogue multiplies each row by its
//     top-k weight and writes it, as bf16, to the staging row of its (token, slot) (the
//     combine of step 5 then sums a token's slots in slot order, without atomics).
//
// Tiling. A workgroup of 4 waves owns one BM x 256 output tile of one expert's rows
// (row tiles come from the dispatch tile list; an expert's group is padded to BM rows).
// Each K step (128) stages the A tile (BM x 128 bytes, XOR-swizzled 16-byte chunks) and
// the B tile (16 packed fragments, 16 KB) in LDS, double-buffered with one barrier per
// step; the next step's global loads are in flight while the MFMAs of this step run.
// Scales are read straight from global memory: one 32-bit word per lane covers four K
// steps, and the instruction's byte select picks the step.
//
// Operand layout of the 16x16x128 instruction with A = FP8, B = FP4 (measured on gfx950):
//   A lane 16g+i : row i, bytes 0..15 = K[16g, 16g+16), bytes 16..31 = K[64+16g, 64+16g+16)
//   B lane 16g+j : column j, 32 nibbles (low first) = K[32g, 32g+32)
//   scale lane 16b+i (A) / 16b+j (B): the 32-block b of row i / column j
//   C lane l     : C[4*(l/16) + r][l%16], r = 0..3
//
// Launch mapping. Workgroups go round-robin to the 8 XCDs (id mod 8). Each XCD gets a
// contiguous range of tile ids, and tile ids walk groups of 4 row tiles across all column
// tiles, so the workgroups resident on one XCD share A rows and B columns in its L2.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kGroupM = 4;

template <int N>
struct IntC {
    static constexpr int value = N;
};

__device__ inline uint16_t f32_to_bf16_rne(float v) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// UE8M0 byte for a block whose largest magnitude is `amax` (fp32): the smallest s with
// amax <= 448 * 2^s, stored as s + 127 and clamped at 0; amax == 0 gives 127.
__device__ inline int requant_scale_byte(float amax) {
    const uint32_t bits = __float_as_uint(amax);
    const int ex = (int)((bits >> 23) & 0xffu);
    const uint32_t mant = bits & 0x7fffffu;
    if (amax == 0.f) return 127;
    if (ex == 0) return 0;
    const int b = ex - 8 + (mant > 0x600000u ? 1 : 0);  // 448 = 1.75 * 2^8
    return b < 0 ? 0 : b;
}

template <int BM, int WAVES_M, int WAVES_N, int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs args) {
    constexpr int WM = BM / WAVES_M;
    constexpr int WN = kBN / WAVES_N;
    constexpr int FM = WM / 16;
    constexpr int FN = WN / 16;
    constexpr int A_BYTES = BM * kBK;                 // fp8: one byte per element
    constexpr int STAGE_BYTES = A_BYTES + kBTileBytes;
    constexpr int A_ROWS_PER_THREAD = BM / 32;        // 8 threads x 16 B per 128-byte row
    static_assert(WAVES_M * WAVES_N == 4, "4 waves");
    static_assert(MODE != 1 || WAVES_N * (FN / 2) == 8, "gate/up pairing");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;

    // ---- tile id -> (row tile, column tile), XCD-aware --------------------------------
    int num_mt = args.meta[0];
    if (num_mt > args.max_tiles) num_mt = args.max_tiles;
    const int NT = args.n_tiles;
    const int total = num_mt * NT;
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int li = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    if (li >= per + (xcd < rem ? 1 : 0)) return;
    const int v = xcd * per + (xcd < rem ? xcd : rem) + li;
    const int grp = v / (kGroupM * NT);
    const int mt0 = grp * kGroupM;
    const int gm = min(kGroupM, num_mt - mt0);
    const int vin = v - grp * kGroupM * NT;
    const int mt = mt0 + vin % gm;
    const int nt = vin / gm;
    const int expert = args.tile_expert[mt];
    const int row0 = args.tile_row0[mt];

    const int K = args.K;
    const int nks = K / kBK;
    const int nkb = (nks + 3) / 4;

    // ---- A row sources (staging) and A scale sources (per lane) ------------------------
    const int chunk = tid & 7;
    uint32_t a_off[A_ROWS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < A_ROWS_PER_THREAD; ++i) {
        const int r = (tid >> 3) + 32 * i;
        if (MODE == 1) {
            const int slot = args.perm[row0 + r];
            const int tok = slot >= 0 ? slot / args.topk : 0;
            a_off[i] = (uint32_t)tok * (uint32_t)args.a_stride;
        } else {
            a_off[i] = (uint32_t)(row0 + r) * (uint32_t)args.a_stride;
        }
    }
    uint32_t sa_off[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * WM + fm * 16 + (lane & 15);
        if (MODE == 1) {
            const int slot = args.perm[row0 + r];
            const int tok = slot >= 0 ? slot / args.topk : 0;
            sa_off[fm] = (uint32_t)tok * (uint32_t)args.a_sf_stride;
        } else {
            sa_off[fm] = (uint32_t)(row0 + r) * (uint32_t)args.a_sf_stride;
        }
    }
    // B fragment index of the wave's n-th fragment
    auto bfrag = [&](int fn) __attribute__((always_inline)) -> int {
        if (MODE == 1) return fn < FN / 2 ? wn * (FN / 2) + fn : 8 + wn * (FN / 2) + (fn - FN / 2);
        return wn * FN + fn;
    };
    const uint8_t* bdata = args.b + (size_t)expert * args.b_expert + (size_t)nt * args.b_ntile;
    const uint32_t* bscale = args.b_sf + (size_t)expert * args.bs_expert + (size_t)nt * args.bs_ntile;

    v4f acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = (v4f){0.f, 0.f, 0.f, 0.f};

    v4i a_st[A_ROWS_PER_THREAD];
    v4i b_st[4];
    auto load_stage = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < A_ROWS_PER_THREAD; ++i)
            a_st[i] = *reinterpret_cast<const v4i*>(args.a + a_off[i] + (size_t)ks * kBK + chunk * 16);
        const uint8_t* bsrc = bdata + (size_t)ks * kBTileBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            b_st[i] = *reinterpret_cast<const v4i*>(bsrc + (tid + kThreads * i) * 16);
    };
    auto store_stage = [&](int buf) __attribute__((always_inline)) {
        uint8_t* As = smem + buf * STAGE_BYTES;
        uint8_t* Bs = As + A_BYTES;
#pragma unroll
        for (int i = 0; i < A_ROWS_PER_THREAD; ++i) {
            const int r = (tid >> 3) + 32 * i;
            *reinterpret_cast<v4i*>(As + r * kBK + ((chunk ^ (r & 7)) << 4)) = a_st[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<v4i*>(Bs + (tid + kThreads * i) * 16) = b_st[i];
    };

    uint32_t sa_cur[FM], sb_cur[FN], sa_nxt[FM], sb_nxt[FN];
    auto load_scales = [&](int kb, uint32_t* sa, uint32_t* sb) __attribute__((always_inline)) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            sa[fm] = *reinterpret_cast<const uint32_t*>(args.a_sf + sa_off[fm] + 4 * kb);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            sb[fn] = bscale[(size_t)kb * (16 * 64) + bfrag(fn) * 64 + lane];
    };

    const int g = lane >> 4;
    const int sw = lane & 7;   // row & 7 for every row this lane reads
    auto compute = [&](int buf, auto ops_c) __attribute__((always_inline)) {
        constexpr int OPS = decltype(ops_c)::value;
        const uint8_t* As = smem + buf * STAGE_BYTES;
        const uint8_t* Bs = As + A_BYTES;
        v4i bq[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            bq[fn] = *reinterpret_cast<const v4i*>(Bs + bfrag(fn) * kFragBytes + lane * 16);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = wm * WM + fm * 16 + (lane & 15);
            const v4i lo = *reinterpret_cast<const v4i*>(As + r * kBK + ((g ^ sw) << 4));
            const v4i hi = *reinterpret_cast<const v4i*>(As + r * kBK + (((g + 4) ^ sw) << 4));
            const v8i a = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const v8i b = {bq[fn].x, bq[fn].y, bq[fn].z, bq[fn].w, 0, 0, 0, 0};
                acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a, b, acc[fm][fn], 0, 4, OPS, (int)sa_cur[fm], OPS, (int)sb_cur[fn]);
            }
        }
    };
    auto step = [&](int ks, auto ops_c) __attribute__((always_inline)) {
        const bool more = ks + 1 < nks;
        if (more) load_stage(ks + 1);
        compute(ks & 1, ops_c);
        if (more) store_stage((ks + 1) & 1);
        __syncthreads();
    };

    load_stage(0);
    store_stage(0);
    load_scales(0, sa_cur, sb_cur);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        if (kb + 1 < nkb) load_scales(kb + 1, sa_nxt, sb_nxt);
        const int ks0 = kb * 4;
        step(ks0, IntC<0>{});
        if (ks0 + 1 < nks) step(ks0 + 1, IntC<1>{});
        if (ks0 + 2 < nks) step(ks0 + 2, IntC<2>{});
        if (ks0 + 3 < nks) step(ks0 + 3, IntC<3>{});
        if (kb + 1 < nkb) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) sa_cur[fm] = sa_nxt[fm];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) sb_cur[fn] = sb_nxt[fn];
        }
    }

    // ---- epilogues (LDS is free: the last step ended with a barrier) ------------------
    if constexpr (MODE == 1) {
        // SwiGLU, then per-row amax over the tile's 128 intermediate columns
        constexpr int FQ = FN / 2;
        float* red = reinterpret_cast<float*>(smem + A_BYTES * 2);   // [WAVES_N][BM]
        uint8_t* hq = smem;                                          // [BM][128] codes
        float hv[FM][FQ][4];
        float rmax[FM][4];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rmax[fm][r] = 0.f;
#pragma unroll
            for (int q = 0; q < FQ; ++q) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float gt = acc[fm][q][r];
                    const float up = acc[fm][q + FQ][r];
                    const float h = gt / (1.0f + expf(-gt)) * up;
                    hv[fm][q][r] = h;
                    rmax[fm][r] = fmaxf(rmax[fm][r], fabsf(h));
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m = rmax[fm][r];
                m = fmaxf(m, __shfl_xor(m, 1, 64));
                m = fmaxf(m, __shfl_xor(m, 2, 64));
                m = fmaxf(m, __shfl_xor(m, 4, 64));
                m = fmaxf(m, __shfl_xor(m, 8, 64));
                rmax[fm][r] = m;
                if ((lane & 15) == 0) red[wn * BM + wm * WM + fm * 16 + 4 * g + r] = m;
            }
        }
        __syncthreads();
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rt = wm * WM + fm * 16 + 4 * g + r;
                float m = red[rt];
#pragma unroll
                for (int w = 1; w < WAVES_N; ++w) m = fmaxf(m, red[w * BM + rt]);
                const int byte = requant_scale_byte(m);
                const float mul = __uint_as_float((uint32_t)(254 - byte) << 23);  // 2^-(byte-127)
#pragma unroll
                for (int q = 0; q < FQ; q += 2) {
                    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(hv[fm][q][r] * mul,
                                                                   hv[fm][q + 1][r] * mul, 0, false);
                    const int col = 16 * (wn * FQ + q) + (lane & 15);
                    hq[rt * 128 + col] = (uint8_t)(pk & 0xff);
                    hq[rt * 128 + col + 16] = (uint8_t)((pk >> 8) & 0xff);
                }
                if (wn == 0 && (lane & 15) == 0)
                    args.h_sf[(size_t)(row0 + rt) * args.h_sf_stride + nt] = (uint8_t)byte;
            }
        }
        __syncthreads();
        // coalesced copy of the BM x 128 code tile
        constexpr int CHUNKS = BM * 128 / 16;
#pragma unroll
        for (int c = tid; c < CHUNKS; c += kThreads) {
            const int r = c >> 3, cc = c & 7;
            *reinterpret_cast<v4i*>(args.h8 + (size_t)(row0 + r) * args.h_stride + nt * 128 + cc * 16) =
                *reinterpret_cast<const v4i*>(hq + r * 128 + cc * 16);
        }
    } else {
        // weight by the row's top-k weight, bf16, write the slot's staging row
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rt = wm * WM + fm * 16 + 4 * g + r;
                const int slot = args.perm[row0 + rt];
                if (slot < 0) continue;
                const float w = args.topk_weights[slot];
                uint16_t* dst = args.stage + (size_t)slot * args.out_cols + nt * kBN + wn * WN + (lane & 15);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) dst[fn * 16] = f32_to_bf16_rne(acc[fm][fn][r] * w);
            }
        }
    }
}

template <int MODE>
hipError_t launch_mode(int block_m, const GemmArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)a.max_tiles * (unsigned)a.n_tiles;
    if (grid == 0) return hipSuccess;
    switch (block_m) {
        case 256: grouped_gemm_kernel<256, 2, 2, MODE><<<grid, kThreads, 0, stream>>>(a); break;
        case 128: grouped_gemm_kernel<128, 2, 2, MODE><<<grid, kThreads, 0, stream>>>(a); break;
        case 64: grouped_gemm_kernel<64, 1, 4, MODE><<<grid, kThreads, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear1(int block_m, const GemmArgs& a, hipStream_t stream) {
    return launch_mode<1>(block_m, a, stream);
}
hipError_t launch_linear2(int block_m, const GemmArgs& a, hipStream_t stream) {
    return launch_mode<2>(block_m, a, stream);
}

}  // namespace moe
