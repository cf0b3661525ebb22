// search.hip -- gfx950 encoder: the exhaustive seed search of SeedLM over a whole matrix.
//
// For one block of 8 weights w (and optional importances d), every seed 1..65535 gives
// a basis U (8 x P, U_ij = s_{iP+j+1} - 32768, the same states the decode kernels
// regenerate).  The weighted least-squares coefficients alpha solve
//     A alpha = r,   A_jk = sum_i (d_i U_ij) U_ik,   r_j = sum_i (d_i U_ij) w_i,
// by Gaussian elimination with partial pivoting (a pivot below 1e-300 in magnitude
// skips the seed).  Every code 0..15 then rounds alpha / 2^(code + exp_bias - 15) half
// to even, clamps it to [-8, 7] and measures err = sum_i d_i (w_i - 2^(...) v_i)^2 with
// v_i = sum_j U_ij c_j.  The block keeps the smallest (err, seed, code) in that order.
// (Qwen3.8-Flash-Next-NanoSeedLM-P4 card, "How it works": the search tries all 65,535
// seeds per block; barnson.org post, "GPU search == CPU search": no contracted
// multiply-adds, so the GPU search returns exactly what a CPU search returns.)
//
// Every floating-point step is a separately rounded IEEE double operation in the order
// written above (sums in increasing i, contraction off), so the result is the same, bit
// for bit, as any CPU evaluation of that definition.  Three exact shortcuts:
//   - alpha / 2^e is computed as alpha * 2^-e (exact for the normal values involved);
//   - v_i is an integer below 2^21 in magnitude, summed in int32 and converted exactly
//     (a NaN coefficient, which only a degenerate system could produce, takes the
//     integer -2^31 and the sum is formed in double instead);
//   - once every coefficient of a seed rounds to zero, all larger codes do too and all
//     have the same error (that of zero coefficients), so only the first is compared.
//
// Mapping: one wave per block; lane l tries seeds 1 + l + 64 k in increasing order and
// keeps its best candidate with a strict comparison (so ties keep its lower seed, then
// its lower code); a wave reduction takes the lexicographic minimum.  A 256-thread
// workgroup owns 4 consecutive blocks, whose coefficient nibbles fill whole words for
// P = 3 and 4 and whose codes fill whole bytes, so it writes its streams without races.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/seedmm.h"
#include "seed_decode.hpp"

namespace seedmm {

// Gaussian elimination with partial pivoting on a P x P system (first row with the
// largest magnitude, strictly), rows exchanged with selects so no array is indexed at
// run time.  Returns false for a pivot below 1e-300 in magnitude.
template <int P>
__device__ __forceinline__ bool solve_small(double (&a)[4][4], double (&r)[4], double (&x)[4]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int col = 0; col < P; ++col) {
        int piv = col;
        double pv = fabs(a[col][col]);
#pragma unroll
        for (int row = col + 1; row < P; ++row) {
            const double v = fabs(a[row][col]);
            if (v > pv) { pv = v; piv = row; }
        }
        if (pv < 1e-300) return false;
#pragma unroll
        for (int row = col + 1; row < P; ++row) {
            const bool sw = piv == row;
#pragma unroll
            for (int k = 0; k < P; ++k) {
                const double t = a[col][k];
                a[col][k] = sw ? a[row][k] : a[col][k];
                a[row][k] = sw ? t : a[row][k];
            }
            const double t = r[col];
            r[col] = sw ? r[row] : r[col];
            r[row] = sw ? t : r[row];
        }
#pragma unroll
        for (int row = col + 1; row < P; ++row) {
            const double f = a[row][col] / a[col][col];
#pragma unroll
            for (int k = col; k < P; ++k) a[row][k] -= f * a[col][k];
            r[row] -= f * r[col];
        }
    }
#pragma unroll
    for (int row = P - 1; row >= 0; --row) {
        double s = r[row];
#pragma unroll
        for (int k = row + 1; k < P; ++k) s -= a[row][k] * x[k];
        x[row] = s / a[row][row];
    }
    return true;
}

template <int P, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_search(const float* __restrict__ W, int64_t ldw,
                                                const float* __restrict__ colw, int K,
                                                int exp_bias, int64_t nblk,
                                                uint16_t* __restrict__ seeds,
                                                uint16_t* __restrict__ coefs,
                                                uint8_t* __restrict__ codes,
                                                double* __restrict__ errs) {
#pragma clang fp contract(off)
    __shared__ uint32_t res[4][2];   // per block: seed | code << 16, coefficient nibbles
    __shared__ int qseed[4][128];    // per wave: queued seeds and their solutions
    __shared__ double qalpha[4][128][P];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t b = (int64_t)blockIdx.x * 4 + wave;
    if (b < nblk) {
        const int nbpr = K / 8;
        const int64_t m = b / nbpr;
        const int kb = (int)(b % nbpr);
        double w[8], d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = (double)W[m * ldw + 8 * kb + i];
            d[i] = WEIGHTED ? (double)colw[8 * kb + i] : 1.0;
        }
        // error of the all-zero coefficients, summed exactly as the code loop sums it
        double e0 = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double dd = w[i] - 0.0;
            e0 += WEIGHTED ? d[i] * (dd * dd) : dd * dd;
        }
        double best = __builtin_inf();
        int bkey = 0x7FFFFFFF;            // seed * 16 + code
        uint32_t bnib = 0;

        // Every code of one seed, from its solution alpha (the definition's arithmetic).
        // Lanes see seeds in no particular order, so candidates compare on the whole key
        // (err, seed * 16 + code).
        auto try_codes = [&](int seed, const double (&alpha)[4]) {
            const Window win = lfsr_window((uint32_t)seed);
            int Ui[8][P];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < P; ++j) Ui[i][j] = (int)state(win, i * P + j + 1) - 32768;
            // A NaN coefficient comes only from a NaN alpha (alpha * 2^-e is otherwise a
            // number, and rint and the clamps keep it one), so the path is chosen once.
            bool anynan = false;
#pragma unroll
            for (int j = 0; j < P; ++j) anynan |= alpha[j] != alpha[j];
            auto codes_loop = [&](auto nanpath) {
                constexpr bool NANP = decltype(nanpath)::value;
#pragma unroll 1
                for (int code = 0; code < 16; ++code) {
                    const int e = code + exp_bias - 15;
                    const double sc = __builtin_ldexp(1.0, e), inv = __builtin_ldexp(1.0, -e);
                    const int key = seed * 16 + code;
                    int c[P];
                    bool zero = true;
#pragma unroll
                    for (int j = 0; j < P; ++j) {
                        double q = __builtin_rint(alpha[j] * inv);   // half to even
                        if (q < -8.0) q = -8.0;
                        if (q > 7.0) q = 7.0;
                        c[j] = q != q ? (int)0x80000000 : (int)q;
                        zero &= c[j] == 0;
                    }
                    if (zero) {
                        // |alpha_j| / 2^e only shrinks as the code grows, so every larger
                        // code rounds to zero as well, with error e0 and a larger key
                        if (e0 < best || (e0 == best && key < bkey)) {
                            best = e0;
                            bkey = key;
                            bnib = 0;
                        }
                        break;
                    }
                    double err = 0.0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        double v;
                        if constexpr (!NANP) {
                            int vi = 0;
#pragma unroll
                            for (int j = 0; j < P; ++j) vi += Ui[i][j] * c[j];
                            v = (double)vi;
                        } else {
                            v = 0.0;
#pragma unroll
                            for (int j = 0; j < P; ++j) v += (double)Ui[i][j] * (double)c[j];
                        }
                        const double dd = w[i] - sc * v;
                        err += WEIGHTED ? d[i] * (dd * dd) : dd * dd;
                    }
                    if (err < best || (err == best && key < bkey)) {
                        best = err;
                        bkey = key;
                        uint32_t nib = 0;
#pragma unroll
                        for (int j = 0; j < P; ++j) nib |= ((uint32_t)c[j] & 0xFu) << (4 * j);
                        bnib = nib;
                    }
                }
            };
            if (anynan) codes_loop(std::true_type{});
            else codes_loop(std::false_type{});
        };

        // Seeds whose systems survive the bound below queue up in LDS; each time 64 are
        // queued, every lane runs the code loop of one of them.
        int qn = 0;                       // queued entries (wave-uniform)
        double thr = __builtin_inf();     // best error found so far by this wave
        auto run_batch = [&](int base, int n) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            if (lane < n) {
                double al[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int j = 0; j < P; ++j) al[j] = qalpha[wave][base + lane][j];
                try_codes(qseed[wave][base + lane], al);
            }
            double m = best;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) m = fmin(m, __shfl_xor(m, off));
            thr = m;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        };

        for (int k = 0; k < 1024; ++k) {
            const int seed = 1 + lane + 64 * k;
            const bool valid = seed <= 65535;
            const Window win = lfsr_window((uint32_t)(valid ? seed : 1));
            double U[8][P];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < P; ++j) U[i][j] = (double)((int)state(win, i * P + j + 1) - 32768);
            double a[4][4], r[4], r0[4], alpha[4];
#pragma unroll
            for (int j = 0; j < P; ++j) {
                r[j] = 0.0;
#pragma unroll
                for (int i = 0; i < 8; ++i) r[j] += (WEIGHTED ? d[i] * U[i][j] : U[i][j]) * w[i];
                r0[j] = r[j];
                if constexpr (WEIGHTED) {
#pragma unroll
                    for (int kk = 0; kk < P; ++kk) {
                        a[j][kk] = 0.0;
#pragma unroll
                        for (int i = 0; i < 8; ++i) a[j][kk] += (d[i] * U[i][j]) * U[i][kk];
                    }
                } else {
                    // products of 16-bit integers and their partial sums (below 2^34) are
                    // exact in double, so A_jk and A_kj are the same double
#pragma unroll
                    for (int kk = j; kk < P; ++kk) {
                        a[j][kk] = 0.0;
#pragma unroll
                        for (int i = 0; i < 8; ++i) a[j][kk] += U[i][j] * U[i][kk];
                    }
                }
            }
            if constexpr (!WEIGHTED) {
#pragma unroll
                for (int j = 0; j < P; ++j)
#pragma unroll
                    for (int kk = 0; kk < j; ++kk) a[j][kk] = a[kk][j];
            }
            double trace = 0.0;
#pragma unroll
            for (int j = 0; j < P; ++j) trace += a[j][j];
            const bool ok = valid && solve_small<P>(a, r, alpha);

            // Bound: every code's error is at least the least-squares residual
            // R = e0 - r . alpha.  Elimination with partial pivoting on this system
            // misses R by at most ~4 n eps kappa(A) e0, and kappa(A) <= trace^P / |det|
            // (det = product of the pivots).  With that bound at most 1e7 the margin
            // 1e-6 e0 covers it many times over, so a seed with
            // (R - 1e-6 e0)(1 - 1e-12) > thr cannot reach an error <= thr, which some
            // candidate already has: it cannot win, and skipping it changes nothing.
            bool keep = ok;
            if (ok && e0 > 0.0 && thr < __builtin_inf()) {
                double det = 1.0, ra = 0.0, tp = 1.0;
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    det *= a[j][j];
                    ra += r0[j] * alpha[j];
                    tp *= trace;
                }
                const double lb = ((e0 - ra) - 1e-6 * e0) * (1.0 - 1e-12);
                if (tp <= 1e7 * fabs(det) && lb > thr) keep = false;
            }
            const uint64_t bal = __ballot(keep);
            const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
            if (keep) {
                const int pos = qn + __popcll(below);
                qseed[wave][pos] = seed;
#pragma unroll
                for (int j = 0; j < P; ++j) qalpha[wave][pos][j] = alpha[j];
            }
            qn += __popcll(bal);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            if (qn >= 64) {
                run_batch(qn - 64, 64);
                qn -= 64;
            }
        }
        if (qn > 0) run_batch(0, qn);
        // lexicographic minimum of (err, seed, code) over the wave
        const int own = bkey;
        double gb = best;
        int gk = bkey;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const double ob = __shfl_xor(gb, off);
            const int ok = __shfl_xor(gk, off);
            if (ob < gb || (ob == gb && ok < gk)) { gb = ob; gk = ok; }
        }
        if (own == gk && gk != 0x7FFFFFFF) {
            res[wave][0] = (uint32_t)(gk >> 4) | ((uint32_t)(gk & 15) << 16);
            res[wave][1] = bnib;
            if (errs) errs[b] = gb;
        }
        if (lane == 0 && gk == 0x7FFFFFFF) {   // no seed had a solvable system
            res[wave][0] = 0u;
            res[wave][1] = 0u;
            if (errs) errs[b] = __builtin_inf();
        }
    }
    __syncthreads();
    // the group's streams: 4 seeds, 4*P nibbles (P whole words), 4 codes (2 whole bytes)
    const int64_t b0 = (int64_t)blockIdx.x * 4;
    const int nb = (int)(nblk - b0 < 4 ? nblk - b0 : 4);
    const int tid = threadIdx.x;
    if (tid < nb) seeds[b0 + tid] = (uint16_t)(res[tid][0] & 0xFFFFu);
    if (tid < (nb * P + 3) / 4) {           // coefficient word tid of the group
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = 4 * tid + q;          // nibble within the group
            const int blk = n / P, j = n % P;
            if (blk < nb) word |= ((res[blk][1] >> (4 * j)) & 0xFu) << (4 * q);
        }
        coefs[b0 * P / 4 + tid] = (uint16_t)word;
    }
    if (tid >= 64 && tid < 64 + (nb + 1) / 2) {   // code byte of blocks 2t, 2t+1
        const int t = tid - 64;
        uint32_t byte = (res[2 * t][0] >> 16) & 0xFu;
        if (2 * t + 1 < nb) byte |= ((res[2 * t + 1][0] >> 16) & 0xFu) << 4;
        codes[b0 / 2 + t] = (uint8_t)byte;
    }
}

}  // namespace seedmm

using namespace seedmm;

extern "C" int seedmm_search(const float* W, int ldw, const float* colw, int M, int K, int P,
                             int32_t exp_bias, uint16_t* seeds, uint16_t* coefs,
                             uint8_t* codes, double* err, void* hip_stream) {
    if (M < 0 || K < 0 || K % 8 != 0 || (P != 3 && P != 4)) return SEEDMM_EINVAL;
    if (exp_bias < -100 || exp_bias > 100) return SEEDMM_EINVAL;
    if (ldw < K) return SEEDMM_EINVAL;
    const int64_t nblk = (int64_t)M * (K / 8);
    if (nblk == 0) return SEEDMM_OK;
    if (!W || !seeds || !coefs || !codes) return SEEDMM_EINVAL;
    hipStream_t st = (hipStream_t)hip_stream;
    const dim3 grid((unsigned)((nblk + 3) / 4));
    if (P == 4) {
        if (colw) hipLaunchKernelGGL((k_search<4, true>), grid, dim3(256), 0, st, W, (int64_t)ldw, colw, K, exp_bias, nblk, seeds, coefs, codes, err);
        else hipLaunchKernelGGL((k_search<4, false>), grid, dim3(256), 0, st, W, (int64_t)ldw, colw, K, exp_bias, nblk, seeds, coefs, codes, err);
    } else {
        if (colw) hipLaunchKernelGGL((k_search<3, true>), grid, dim3(256), 0, st, W, (int64_t)ldw, colw, K, exp_bias, nblk, seeds, coefs, codes, err);
        else hipLaunchKernelGGL((k_search<3, false>), grid, dim3(256), 0, st, W, (int64_t)ldw, colw, K, exp_bias, nblk, seeds, coefs, codes, err);
    }
    return hipGetLastError() == hipSuccess ? SEEDMM_OK : SEEDMM_EHIP;
}
