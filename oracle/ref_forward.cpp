// Plain, slow fp64 CPU oracle of the one-GPU Mega MoE forward, in C++17.
//
// TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline
// leg may build, load or call this file's library. It shares no code with the HIP path
// (it includes nothing of it and the HIP path includes nothing of it). It is the second,
// independently written form of the oracle in oracle/moe_oracle.py; the tests check the
// two against each other and against the hand-derived worked example.
//
// What it computes (chenxutan.com/d/1930, "DeepSeek DeepGEMM 2026年4月重磅更新", section 3.1:
// dispatch, Linear1, SwiGLU, Linear2, combine; section 4.1: the E4M3 and E2M1 formats;
// section 11.1: one scale per block, block amax over the format maximum; zevenfang.github.io
// DeepGEMM review, section 4: UE8M0 scales), with the readings of the design notes
// (FP8 activations x FP4 weights; W1 rows 0..I-1 gate, I..2I-1 up; element 2i in the low
// nibble; UE8M0 byte b = 2^(b-127); scale rounded up to a power of two; ties to even):
//
//   x[t, c]   = e4m3(x_fp8[t, c]) * 2^(x_sf[t, c/128] - 127)
//   W[e, n, c] = e2m1(nibble c of row n) * 2^(sf[e, n, c/32] - 127)
//   for every slot (t, j) with e = topk_idx[t, j] in [0, E):
//     g[n] = sum_c x[t, c] W1[e, n, c],  u[n] = sum_c x[t, c] W1[e, I + n, c]   (fp64, c ascending)
//     h[n] = g[n] / (1 + exp(-g[n])) * u[n]                                      (fp64)
//     per block of 128 n, decided on float(h): byte = max(s + 127, 0), s the least integer
//       with amax <= 448 * 2^s (s = 0 for an all-zero block); q = e4m3 RNE of
//       float(h) * 2^(127 - byte); h'[n] = e4m3(q) * 2^(byte - 127)
//     o[m] = sum_n h'[n] W2[e, m, n]                                             (fp64, n ascending)
//   y[t, m] = bf16 RNE of sum over j = 0..k-1 (valid slots only) of w[t, j] * o_j[m]  (fp64)
//
// Every product of an e4m3 and an E2M1 value with power-of-two scales is exact in fp64, so
// the only roundings are those of the fp64 sums, the exponential, and the stated roundings.
// Threads split the output rows n (and m) of each expert; each dot product is one ascending
// fp64 sum, so the thread count changes nothing in the result.
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <exception>
#include <thread>
#include <vector>

namespace {

constexpr double kNaN = __builtin_nan("");

// OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; 0x7F/0xFF NaN.
double e4m3_value(uint8_t code) {
    const int sign = code >> 7, ex = (code >> 3) & 15, man = code & 7;
    if (ex == 15 && man == 7) return kNaN;
    const double mag = ex == 0 ? std::ldexp(man / 8.0, -6) : std::ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

// E2M1: 1 sign, 2 exponent, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
double e2m1_value(uint8_t nib) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    return (nib & 8) ? -mag[nib & 7] : mag[nib & 7];
}

// UE8M0: 2^(b-127); 255 is NaN.
double ue8m0_value(uint8_t b) { return b == 255 ? kNaN : std::ldexp(1.0, (int)b - 127); }

// Nearest e4m3fn code of v (|v| <= 448), ties to the even code.
uint8_t e4m3_encode(double v) {
    const uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
    const double a = std::fabs(v);
    if (a < std::ldexp(1.0, -6)) {                       // subnormals: quantum 2^-9
        const double q = std::nearbyint(a * 512.0);      // 8 is the first normal, 2^-6
        return sign | (uint8_t)q;
    }
    int e2 = 0;
    const double m = std::frexp(a, &e2);                 // a = m 2^e2, m in [0.5, 1)
    int ex = e2 - 1;                                     // a = (2m) 2^ex, 2m in [1, 2)
    double q = std::nearbyint((2.0 * m - 1.0) * 8.0);    // 3 mantissa bits
    if (q == 8.0) {
        q = 0.0;
        ++ex;
    }
    return sign | (uint8_t)(((ex + 7) << 3) | (int)q);
}

// fp64 -> bf16 bits, one rounding to 8 significant bits (subnormal quantum 2^-133), ties to even.
uint16_t bf16_bits(double v) {
    if (v == 0.0) return std::signbit(v) ? 0x8000 : 0x0000;
    int e2 = 0;
    std::frexp(v, &e2);                                  // |v| in [2^(e2-1), 2^e2)
    const int q = e2 - 8 > -133 ? e2 - 8 : -133;
    const double r = std::ldexp(std::nearbyint(std::ldexp(v, -q)), q);
    const float f = (float)r;                            // exact (or infinity past bf16's range)
    uint32_t bits;
    std::memcpy(&bits, &f, 4);
    return (uint16_t)(bits >> 16);
}

// Least s with amax <= 448 * 2^s (448 = 1.75 * 2^8), 0 for amax == 0.
int block_scale_exponent(double amax) {
    if (amax == 0.0) return 0;
    int e2 = 0;
    const double m = std::frexp(amax, &e2);              // amax = (2m) 2^(e2-1)
    return (e2 - 1) - 8 + (2.0 * m > 1.75 ? 1 : 0);
}

template <class F>
void parallel_for(int n, int threads, F&& body) {
    std::vector<std::thread> pool;
    const int per = (n + threads - 1) / threads;
    for (int t = 0; t < threads; ++t) {
        const int lo = t * per, hi = lo + per < n ? lo + per : n;
        if (lo >= hi) break;
        pool.emplace_back([&body, lo, hi] { for (int i = lo; i < hi; ++i) body(i); });
    }
    for (auto& th : pool) th.join();
}

// Row n of a packed FP4 matrix [rows][K/2] with UE8M0 scales [rows][K/32], decoded to fp64.
// Returns false on a NaN scale byte.
bool decode_fp4_row(const uint8_t* w, const uint8_t* sf, int K, double* out) {
    for (int c = 0; c < K; ++c) {
        const uint8_t byte = w[c / 2];
        const uint8_t nib = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
        const double s = ue8m0_value(sf[c / 32]);
        if (std::isnan(s)) return false;
        out[c] = e2m1_value(nib) * s;
    }
    return true;
}

double dot(const double* a, const double* b, int n) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += a[i] * b[i];
    return acc;
}

}  // namespace

extern "C" {

// Status codes: 0 ok, -1 bad arguments or shape, -2 a NaN code or scale byte in the input,
// -3 an internal error.
int ref_moe_forward(const uint8_t* x_fp8, const uint8_t* x_sf, int x_sf_stride,
                    const int32_t* topk_idx, const float* topk_w, int T, int k,
                    const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf,
                    int E, int H, int I, const int32_t* tokens, int n_tokens, int threads,
                    uint16_t* y_bits, double* y_out, uint8_t* h8_out, uint8_t* hsf_out,
                    double* seconds, int* threads_used) {
    try {
        const auto t0 = std::chrono::steady_clock::now();
        if (!x_fp8 || !x_sf || !topk_idx || !topk_w || !w1 || !w1_sf || !w2 || !w2_sf || !y_bits)
            return -1;
        if (T < 0 || k < 1 || E < 1 || H < 128 || H % 128 || I < 128 || I % 128) return -1;
        if (x_sf_stride < H / 128) return -1;
        if (threads <= 0) threads = (int)std::thread::hardware_concurrency();
        if (threads <= 0) threads = 1;
        std::vector<int> toks;
        if (tokens) {
            for (int i = 0; i < n_tokens; ++i) {
                if (tokens[i] < 0 || tokens[i] >= T) return -1;
                toks.push_back(tokens[i]);
            }
        } else {
            for (int t = 0; t < T; ++t) toks.push_back(t);
        }
        const int nt = (int)toks.size();

        // x rows of the tokens, decoded
        std::vector<double> xd((size_t)nt * H);
        bool bad = false;
        for (int i = 0; i < nt && !bad; ++i) {
            const int t = toks[i];
            for (int c = 0; c < H; ++c) {
                const double v = e4m3_value(x_fp8[(size_t)t * H + c]);
                const double s = ue8m0_value(x_sf[(size_t)t * x_sf_stride + c / 128]);
                if (std::isnan(v) || std::isnan(s)) bad = true;
                xd[(size_t)i * H + c] = v * s;
            }
        }
        if (bad) return -2;

        std::vector<double> contrib((size_t)nt * k * H, 0.0);   // w[t,j] * o[t,j,:]
        std::vector<double> G, U, Hq;
        for (int e = 0; e < E; ++e) {
            // the expert's slots, ascending (token, slot) within the given token order
            std::vector<int> rows;   // i * k + j
            for (int i = 0; i < nt; ++i)
                for (int j = 0; j < k; ++j)
                    if (topk_idx[(size_t)toks[i] * k + j] == e) rows.push_back(i * k + j);
            const int R = (int)rows.size();
            if (R == 0) continue;
            G.assign((size_t)R * I, 0.0);
            U.assign((size_t)R * I, 0.0);
            // Linear1: thread over n; rows n (gate) and I + n (up) of W1[e]
            std::vector<char> fail(I, 0);
            parallel_for(I, threads, [&](int n) {
                std::vector<double> wg(H), wu(H);
                const size_t base = (size_t)e * 2 * I;
                if (!decode_fp4_row(w1 + (base + n) * (H / 2), w1_sf + (base + n) * (H / 32), H, wg.data()) ||
                    !decode_fp4_row(w1 + (base + I + n) * (H / 2), w1_sf + (base + I + n) * (H / 32), H, wu.data())) {
                    fail[n] = 1;
                    return;
                }
                for (int r = 0; r < R; ++r) {
                    const double* xr = &xd[(size_t)(rows[r] / k) * H];
                    G[(size_t)r * I + n] = dot(xr, wg.data(), H);
                    U[(size_t)r * I + n] = dot(xr, wu.data(), H);
                }
            });
            for (char f : fail)
                if (f) return -2;
            // SwiGLU and the requantisation of each slot's h
            Hq.assign((size_t)R * I, 0.0);
            for (int r = 0; r < R; ++r) {
                for (int b = 0; b < I / 128; ++b) {
                    double h32[128];
                    double amax = 0.0;
                    for (int q = 0; q < 128; ++q) {
                        const size_t n = (size_t)r * I + b * 128 + q;
                        const double h = G[n] / (1.0 + std::exp(-G[n])) * U[n];
                        h32[q] = (double)(float)h;                  // the decision is taken on fp32
                        amax = std::fabs(h32[q]) > amax ? std::fabs(h32[q]) : amax;
                    }
                    int byte = block_scale_exponent(amax) + 127;
                    if (byte < 0) byte = 0;
                    const double inv = std::ldexp(1.0, 127 - byte), scale = std::ldexp(1.0, byte - 127);
                    const int slot = rows[r];
                    if (hsf_out) hsf_out[(size_t)slot * (I / 128) + b] = (uint8_t)byte;
                    for (int q = 0; q < 128; ++q) {
                        const uint8_t code = e4m3_encode(h32[q] * inv);
                        if (h8_out) h8_out[(size_t)slot * I + b * 128 + q] = code;
                        Hq[(size_t)r * I + b * 128 + q] = e4m3_value(code) * scale;
                    }
                }
            }
            // Linear2: thread over m; row m of W2[e]; weighted per slot
            std::vector<char> fail2(H, 0);
            parallel_for(H, threads, [&](int m) {
                std::vector<double> w(I);
                const size_t row = (size_t)e * H + m;
                if (!decode_fp4_row(w2 + row * (I / 2), w2_sf + row * (I / 32), I, w.data())) {
                    fail2[m] = 1;
                    return;
                }
                for (int r = 0; r < R; ++r) {
                    const int i = rows[r] / k, j = rows[r] % k;
                    const double o = dot(&Hq[(size_t)r * I], w.data(), I);
                    contrib[((size_t)i * k + j) * H + m] = (double)topk_w[(size_t)toks[i] * k + j] * o;
                }
            });
            for (char f : fail2)
                if (f) return -2;
        }
        // combine: slots in order j = 0..k-1; skipped slots add nothing
        for (int i = 0; i < nt; ++i) {
            for (int m = 0; m < H; ++m) {
                double acc = 0.0;
                for (int j = 0; j < k; ++j) acc += contrib[((size_t)i * k + j) * H + m];
                y_bits[(size_t)i * H + m] = bf16_bits(acc);
                if (y_out) y_out[(size_t)i * H + m] = acc;
            }
        }
        const auto t1 = std::chrono::steady_clock::now();
        if (seconds) *seconds = std::chrono::duration<double>(t1 - t0).count();
        if (threads_used) *threads_used = threads;
        return 0;
    } catch (...) {
        return -3;
    }
}

}  // extern "C"
