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
// Every candidate that can win is evaluated with separately rounded IEEE double
// operations in the order written above (sums in increasing i, contraction off), and
// candidates compare on the whole key (err, seed * 16 + code), so the result is the same,
// bit for bit, as any CPU evaluation of that definition.  Fused multiply-adds appear only
// in the bounds and filters that decide, with safe margins, which pairs and codes cannot
// win.  Three exact shortcuts:
//   - alpha / 2^e is computed as alpha * 2^-e (exact for the normal values involved);
//   - v_i is an integer below 2^21 in magnitude, summed in int32 and converted exactly
//     (a NaN coefficient, which only a degenerate system could produce, takes the
//     integer -2^31 and the sum is formed in double instead);
//   - once every coefficient of a seed rounds to zero, all larger codes do too and all
//     have the same error (that of zero coefficients), so only the first is compared.
//
// Two kernels:
//   - k_search (with importances): one wave per block; lane l tries seeds 1 + l + 64 k,
//     each building and solving its own system, and a wave reduction takes the
//     lexicographic minimum.  A 256-thread workgroup owns 4 consecutive blocks, whose
//     coefficient nibbles fill whole words for P = 3 and 4 and whose codes fill whole
//     bytes, so it writes its streams without races.
//   - k_search_lanes (without importances): one block per lane, a per-seed table and a
//     walk along the register's cycle (see there); a workgroup owns 512 blocks.  The
//     table lives in caller-owned device memory, filled by seedmm_search_prepare.
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

// The candidates of one seed: every code 0..15 from its solution alpha, in the
// definition's arithmetic, each compared with the best so far on the whole key
// (err, seed * 16 + code).
template <int P, bool WEIGHTED>
__device__ __forceinline__ void try_codes_of(int seed, const double (&alpha)[4], const double (&w)[8],
                                             const double (&d)[8], double e0, int exp_bias,
                                             double& best, int& bkey, uint32_t& bnib) {
#pragma clang fp contract(off)
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
        auto try_codes = [&](int seed, const double (&alpha)[4]) {
            try_codes_of<P, WEIGHTED>(seed, alpha, w, d, e0, exp_bias, best, bkey, bnib);
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

// ----------------------------------------------------------------------------------
// Unweighted search, one block per lane.  Without importances A = U^T U depends on the
// seed alone, so its Cholesky factor is computed once per seed into a table, and the
// least-squares residual R = e0 - r^T A^-1 r of a (block, seed) pair costs one forward
// substitution instead of a full elimination.  The seeds are visited along the
// register's cycle, x_0 = 1, x_{t+1} = the state after x_t: the seed x_t has states
// s_k = x_{t+k}, so with c_u = sum_i (x_{u+iP} - 32768) w_i its right-hand side is
// r_j = c_{t+j+1}, and each step along the cycle needs one new c (8 multiply-adds).
// All lanes of a wave (64 consecutive blocks) walk the cycle together, so each step's
// table records are uniform (scalar) loads; a workgroup is 8 waves (512 blocks).  A pair
// whose bound does not already exceed its block's best error joins the wave's queue in
// LDS; each time 64 pairs are queued, every lane runs the exact definition (elimination
// with partial pivoting, then every code) on one of them, whatever its block, and the
// candidates merge into their blocks.
// Once a block's best error is exactly 0, a seed can only win with a smaller key
// (errors are never negative), so seeds with seed * 16 above the best key are skipped.
//
// Bound: the table's factor L of A gives R~ = e0 - |y|^2, L y = r.  The factorisation and
// the substitution are backward stable, so R~ misses R by at most ~c P eps kappa(A) e0
// (c ~ 10); the table flags a seed usable when A is positive definite with
// trace(A)^P <= 1e7 det(A), which bounds kappa(A) by 1e7.  The margin 1e-6 e0 covers that
// error more than 20 times over, so a pair with (R~ - 1e-6 e0)(1 - 1e-12) > best cannot
// reach an error <= best and skipping it changes nothing.  Unflagged seeds always go to
// the exact path.
// ----------------------------------------------------------------------------------

constexpr int kCycle = 65535;                 // the register's period
constexpr int kXLen = kCycle + 64;            // cycle positions stepped (past one period)

// Factor record of the seed at cycle position t, in doubles: the strictly lower entries
// of L row by row, 1 / L_jj, an upper bound of 1 / lambda_min(A) (0 unless the seed is
// usable), and the seed (its bits in the low word, the usable flag in bit 32).
template <int P> struct SeedRecord {
    static constexpr int kL = 0, kD = P * (P - 1) / 2, kLam = kD + P, kSeed = kLam + 1;
    static constexpr int kSize = P == 4 ? 12 : 8;
    static_assert(kSeed < kSize, "record layout");
};
__device__ __forceinline__ int rec_seed(double v) { return (int)(uint32_t)__double_as_longlong(v); }
__device__ __forceinline__ bool rec_usable(double v) { return (__double_as_longlong(v) >> 32) & 1; }
// X record at cycle position u: x_{u+iP} - 32768, i = 0..7 (one 64-byte line).
constexpr int kXRecs = kCycle + 8;
constexpr int kSteps = kCycle + 1;           // steps walked: the cycle, then seed 1 again

// Layout of the caller's table memory for one P: the cycle positions (uint32[kXLen]),
// the X records (double[kXRecs][8]) and the factor records (double[kSteps][kSize]),
// each part starting on a 256-byte boundary.
struct TableLayout {
    size_t cycle, xrec, chol, amat, total;
};
// A = U^T U of the seed at cycle position t, upper triangle row by row (exact integers),
// then sqrt(trace A) rounded up.
constexpr int amat_size(int P) { return P * (P + 1) / 2 + 1; }
inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }
inline TableLayout table_layout(int P) {
    TableLayout L;
    L.cycle = 0;
    L.xrec = al256(sizeof(uint32_t) * kXLen);
    L.chol = L.xrec + al256(sizeof(double) * 8 * (size_t)kXRecs);
    const int ks = P == 4 ? SeedRecord<4>::kSize : SeedRecord<3>::kSize;
    L.amat = L.chol + al256(sizeof(double) * (size_t)ks * kSteps);
    L.total = L.amat + al256(sizeof(double) * (size_t)amat_size(P) * kSteps);
    return L;
}

// The cycle positions, one thread (32 states per window).
__global__ void k_cycle(uint32_t* __restrict__ x) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    uint32_t s = 1;
    for (int t = 0; t < kXLen; t += 32) {
        const Window win = lfsr_window(s);
        x[t] = s;
        for (int k = 1; k < 32 && t + k < kXLen; ++k) x[t + k] = state(win, k);
        s = state(win, 32);
    }
}

template <int P>
__global__ __launch_bounds__(256) void k_seed_tables(const uint32_t* __restrict__ x,
                                                     double* __restrict__ xrec,
                                                     double* __restrict__ chol,
                                                     double* __restrict__ amat) {
    using Rec = SeedRecord<P>;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < kXRecs) {
#pragma unroll
        for (int i = 0; i < 8; ++i) xrec[(int64_t)t * 8 + i] = (double)((int)x[t + i * P] - 32768);
    }
    if (t >= kSteps) return;
    double* rec = chol + (int64_t)t * Rec::kSize;
    double U[8][P];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < P; ++j) U[i][j] = (double)((int)x[t + i * P + j + 1] - 32768);
    // products of 16-bit integers and their sums (below 2^34) are exact in double
    double A[P][P];
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
        for (int k = 0; k < P; ++k) {
            double a = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) a += U[i][j] * U[i][k];
            A[j][k] = a;
        }
    {
        double* ar = amat + (int64_t)t * amat_size(P);
        int o = 0;
#pragma unroll
        for (int j = 0; j < P; ++j)
#pragma unroll
            for (int k = j; k < P; ++k) ar[o++] = A[j][k];
        double tr = 0.0;
#pragma unroll
        for (int j = 0; j < P; ++j) tr += A[j][j];
        ar[o] = sqrt(tr) * (1.0 + 1e-12);
    }
    double L[P][P];
    bool pd = true;
    double det = 1.0, trace = 0.0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        double dj = A[j][j];
#pragma unroll
        for (int k = 0; k < j; ++k) dj -= L[j][k] * L[j][k];
        if (!(dj > 0.0)) {
            pd = false;
            dj = 1.0;
        }
        L[j][j] = sqrt(dj);
        det *= dj;
        trace += A[j][j];
#pragma unroll
        for (int i = j + 1; i < P; ++i) {
            double v = A[i][j];
#pragma unroll
            for (int k = 0; k < j; ++k) v -= L[i][k] * L[j][k];
            L[i][j] = v / L[j][j];
        }
    }
    int o = Rec::kL;
#pragma unroll
    for (int i = 1; i < P; ++i)
#pragma unroll
        for (int j = 0; j < i; ++j) rec[o++] = L[i][j];
#pragma unroll
    for (int j = 0; j < P; ++j) rec[Rec::kD + j] = 1.0 / L[j][j];
    double tp = 1.0;
#pragma unroll
    for (int j = 0; j < P; ++j) tp *= trace;
    const bool usable = pd && tp <= 1e7 * det;
    // A lower bound of lambda_min(A): bisection on mu with an LDL^T factorisation of
    // A - mu I (all pivots positive: positive definite), then less 1e-12 trace(A), which
    // covers the factorisation's backward error (~P^2 eps |A|) many times over.
    double lam = 0.0;
    if (usable) {
        double lo = 0.0, hi = A[0][0];
#pragma unroll
        for (int j = 1; j < P; ++j) hi = fmin(hi, A[j][j]);
#pragma unroll 1
        for (int it = 0; it < 48; ++it) {
            const double mu = 0.5 * (lo + hi);
            double l[P][P], d[P];
            bool ok = true;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                double dj = A[j][j] - mu;
#pragma unroll
                for (int k = 0; k < j; ++k) dj -= l[j][k] * l[j][k] * d[k];
                ok = ok && dj > 0.0;
                d[j] = dj > 0.0 ? dj : 1.0;
#pragma unroll
                for (int i = j + 1; i < P; ++i) {
                    double v = A[i][j];
#pragma unroll
                    for (int k = 0; k < j; ++k) v -= l[i][k] * l[j][k] * d[k];
                    l[i][j] = v / d[j];
                }
            }
            if (ok) lo = mu;
            else hi = mu;
        }
        lam = fmax(0.0, lo - 1e-12 * trace);
    }
    rec[Rec::kLam] = lam > 0.0 ? (1.0 / lam) * (1.0 + 1e-12) : 0.0;
    rec[Rec::kSeed] = __longlong_as_double((long long)x[t] | ((long long)usable << 32));
#pragma unroll
    for (int k = Rec::kSeed + 1; k < Rec::kSize; ++k) rec[k] = 0.0;
}

template <int P>
__global__ __launch_bounds__(512) void k_search_lanes(const float* __restrict__ W, int64_t ldw,
                                                      int K, int exp_bias, int64_t nblk,
                                                      const double* __restrict__ xtab,
                                                      const double* __restrict__ ctab,
                                                      const double* __restrict__ atab,
                                                      uint16_t* __restrict__ seeds,
                                                      uint16_t* __restrict__ coefs,
                                                      uint8_t* __restrict__ codes,
                                                      double* __restrict__ errs) {
#pragma clang fp contract(off)
    using Rec = SeedRecord<P>;
    // P = 4: the pairs past the residual bound go through the code bound first (it cut the
    // exact evaluations from 12% to 2.4% of the pairs and the search time by 8%); at P = 3
    // only 6% of the pairs pass the residual bound and the exact systems are smaller, so
    // they go straight to the exact definition (the code bound measured 3% slower there).
    constexpr bool kCodeBound = P == 4;
    constexpr int QCAP = kCodeBound ? 256 : 1;    // wave ring of pairs past the residual bound
    constexpr int QCAP2 = kCodeBound ? 128 : 256; // wave ring of pairs for the exact definition
    __shared__ double wv[8][8][64];           // per wave: the weights of its 64 blocks
    __shared__ double e0v[8][64], bestv[8][64];
    __shared__ unsigned long long mbits[8][64];   // merge: per block, best error bits,
    __shared__ int mkey[8][64];                   // its key and its nibbles
    __shared__ uint32_t mnib[8][64];
    __shared__ uint32_t qe[8][QCAP];          // pairs past the residual bound: t | lane << 16
    __shared__ double qy[8][QCAP][P];         // ... and their substitution vectors y
    __shared__ uint32_t qe2[8][QCAP2];        // pairs past the code bound: seed | lane << 16
    __shared__ double wl1[8][64];             // sum of |w_i| of each block
    __shared__ unsigned long long ubits[8][64];   // per block: an upper bound of its final best
                                                  // error (bits), from candidates still queued
    __shared__ uint32_t res[512][2];          // per block: seed | code << 16, coefficient nibbles
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * 512;
    const int64_t b = b0 + threadIdx.x;
    const bool active = b < nblk;

    double w[8];
    {
        const int nbpr = K / 8;
        const int64_t m = active ? b / nbpr : 0;
        const int kb = active ? (int)(b % nbpr) : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = active ? (double)W[m * ldw + 8 * kb + i] : 0.0;
            wv[wave][i][lane] = w[i];
        }
    }
    // error of the all-zero coefficients, summed exactly as the code loop sums it
    double e0 = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double dd = w[i] - 0.0;
        e0 += dd * dd;
    }
    e0v[wave][lane] = e0;
    {
        double l1 = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) l1 += fabs(w[i]);
        wl1[wave][lane] = l1;
    }
    double best = __builtin_inf();            // this lane's block: best candidate so far
    int bkey = 0x7FFFFFFF;                    // seed * 16 + code
    uint32_t bnib = 0;
    bestv[wave][lane] = best;

    // The definition for the pair (block blk of this wave, seed): system, elimination,
    // then every code.  A code whose error provably exceeds thr (see below) is not
    // evaluated; the others are, in the definition's arithmetic, and the best of them
    // (whole key) is returned in (cb, ck, cn).
    auto exact = [&](int blk, int seed, double thr, double& cb, int& ck, uint32_t& cn) {
        double wl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wl[i] = wv[wave][i][blk];
        const double e0l = e0v[wave][blk];
        const Window win = lfsr_window((uint32_t)seed);
        int Ui[8][P];
        double U[8][P];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < P; ++j) {
                Ui[i][j] = (int)state(win, i * P + j + 1) - 32768;
                U[i][j] = (double)Ui[i][j];
            }
        double a[4][4], a0[4][4], r[4], r0[4], alpha[4];   // a0: diagonal of A
#pragma unroll
        for (int j = 0; j < P; ++j) {
            r[j] = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) r[j] += U[i][j] * wl[i];
            r0[j] = r[j];
            // products of 16-bit integers and their partial sums (below 2^34) are exact
            // in double, so A_jk and A_kj are the same double, and a fused multiply-add
            // gives the same bits as the separate operations
#pragma unroll
            for (int kk = j; kk < P; ++kk) {
                a[j][kk] = 0.0;
#pragma unroll
                for (int i = 0; i < 8; ++i) a[j][kk] = __builtin_fma(U[i][j], U[i][kk], a[j][kk]);
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j)
#pragma unroll
            for (int kk = 0; kk < j; ++kk) a[j][kk] = a[kk][j];
        double a2[4][4];                      // 2 A_jk above the diagonal (exact)
#pragma unroll
        for (int j = 0; j < P; ++j) {
            a0[j][j] = a[j][j];
#pragma unroll
            for (int kk = j + 1; kk < P; ++kk) a2[j][kk] = 2.0 * a[j][kk];
        }
        double trace = 0.0;
#pragma unroll
        for (int j = 0; j < P; ++j) trace += a[j][j];
        if (!solve_small<P>(a, r, alpha)) return;
        // Code filter.  For any coefficients c, err(c) = R + d^T A d exactly, with R the
        // least-squares residual and d = alpha - 2^e c.  From the computed alpha,
        // Rt = e0 - r . alpha and the computed d^T A d miss R and d^T A d by at most
        // ~c P eps kappa(A) (e0 + d^T A d) (c ~ 10; elimination with partial pivoting is
        // backward stable and A is positive definite).  With kappa(A) <= trace^P / |det|
        // <= 1e7 the margin 1e-6 (e0 + d^T A d) covers that many times over, so a code
        // whose filtered value exceeds thr has an error above thr and cannot win.
        double det = 1.0, ra = 0.0, tp = 1.0;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            det *= a[j][j];
            ra += r0[j] * alpha[j];
            tp *= trace;
        }
        const bool filt = tp <= 1e7 * fabs(det);
        const double Rt = e0l - ra;
        bool anynan = false;
#pragma unroll
        for (int j = 0; j < P; ++j) anynan |= alpha[j] != alpha[j];
        if (anynan) {
            // only a degenerate system gives a NaN; evaluate it plainly
            double dd[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) dd[i] = 1.0;
            try_codes_of<P, false>(seed, alpha, wl, dd, e0l, exp_bias, cb, ck, cn);
            return;
        }
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
                c[j] = (int)q;
                zero &= c[j] == 0;
            }
            if (zero) {
                // |alpha_j| / 2^e only shrinks as the code grows, so every larger code
                // rounds to zero as well, with error e0 and a larger key
                if (e0l < cb || (e0l == cb && key < ck)) {
                    cb = e0l;
                    ck = key;
                    cn = 0;
                }
                break;
            }
            if (filt) {
                // d^T A d = sum_j d_j (A_jj d_j + 2 sum_{k>j} A_jk d_k), fused (the
                // margin covers the rounding)
                double d[P];
#pragma unroll
                for (int j = 0; j < P; ++j) d[j] = __builtin_fma(-sc, (double)c[j], alpha[j]);
                double qf = 0.0;
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    double t = a0[j][j] * d[j];
#pragma unroll
                    for (int kk = j + 1; kk < P; ++kk) t = __builtin_fma(a2[j][kk], d[kk], t);
                    qf = __builtin_fma(d[j], t, qf);
                }
                const double lim = thr < cb ? thr : cb;
                if (((Rt + qf) - 1e-6 * (e0l + qf)) * (1.0 - 1e-12) > lim) continue;
            }
            double err = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int vi = 0;
#pragma unroll
                for (int j = 0; j < P; ++j) vi += Ui[i][j] * c[j];
                const double dd = wl[i] - sc * (double)vi;
                err += dd * dd;
            }
            if (err < cb || (err == cb && key < ck)) {
                cb = err;
                ck = key;
                uint32_t nib = 0;
#pragma unroll
                for (int j = 0; j < P; ++j) nib |= ((uint32_t)c[j] & 0xFu) << (4 * j);
                cn = nib;
            }
        }
    };

    // The queued pairs, n <= 64 of them from the ring head: lane t evaluates pair t; the
    // candidates then merge into their blocks' bests through LDS, on whole keys.  Errors
    // are never negative (nor NaN), so their bit patterns order like the values: a
    // 64-bit minimum over the bits finds each block's smallest error, a 32-bit minimum
    // the smallest key among the candidates with that error (the owner first clears the
    // key when the error went down), and that candidate writes its nibbles.  One wave's
    // LDS operations take effect in program order.
    int qh = 0, qn = 0;                       // ring head and length (wave-uniform)
    int qh2 = 0, qn2 = 0;                     // the same for the code-bound ring
    mbits[wave][lane] = (unsigned long long)__double_as_longlong(best);
    ubits[wave][lane] = (unsigned long long)__double_as_longlong(best);
    mkey[wave][lane] = bkey;
    mnib[wave][lane] = bnib;
    auto run_batch = [&](int n) {
        double cb = __builtin_inf();
        int ck = 0x7FFFFFFF;
        uint32_t cn = 0;
        int blk = 0;
        if (lane < n) {
            const uint32_t ent = qe2[wave][(qh2 + lane) & (QCAP2 - 1)];
            blk = (int)(ent >> 16);
            exact(blk, (int)(ent & 0xFFFFu), bestv[wave][blk], cb, ck, cn);
        }
        const unsigned long long cbits = (unsigned long long)__double_as_longlong(cb);
        const bool has = lane < n && ck != 0x7FFFFFFF;
        if (has) __hip_atomic_fetch_min(&mbits[wave][blk], cbits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        const unsigned long long mine = mbits[wave][lane];
        if (mine != (unsigned long long)__double_as_longlong(best)) mkey[wave][lane] = 0x7FFFFFFF;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        const bool tie = has && mbits[wave][blk] == cbits;
        if (tie) __hip_atomic_fetch_min(&mkey[wave][blk], ck, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        if (tie && mkey[wave][blk] == ck) mnib[wave][blk] = cn;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        best = __longlong_as_double((long long)mine);
        bkey = mkey[wave][lane];
        bnib = mnib[wave][lane];
        bestv[wave][lane] = best;
        qh2 = (qh2 + n) & (QCAP2 - 1);
        qn2 -= n;
    };

    // Code bound of the queued pairs, n <= 64 of them from the ring head, lane t on pair
    // t; those it cannot rule out go on to the exact definition (run_batch).  In exact
    // arithmetic every code's error is R + d^T A d with d = alpha - 2^e c, for any c.
    // Computed from the tables: Rlb <= R <= Rub as in the step's bound; 1 / ilam <=
    // lambda_min(A) (the table's certified bound); alpha~ = L^-T y misses alpha, and the
    // definition's own solution alpha_o, by at most del = 1e-6 |alpha~|_1 (backward-stable
    // solves, kappa(A) <= 1e7 for usable seeds) plus the correlation's rounding times ilam.
    // A code is ruled out when its bound times (1 - 1e-12) exceeds thr, the block's best
    // or a queued candidate's upper bound; gap = thr (1 + 4e-12) - Rlb covers that factor.
    // With amax = max_j |alpha~_j| in [2^g, 2^(g+1)):
    //   - codes e_lo .. e_lo + 5 (2^e from 2^(g-3) to 2^(g+2)): out if
    //     sum_j (dist(alpha~_j, 2^e {-8..7}) - del)_+^2 > gap ilam (R + lambda_min |d|^2,
    //     valid for every c), or, when no alpha~_j / 2^e lies within 2 del / 2^e of a
    //     rounding boundary (then the definition's candidate is c~ = clamp(rint(alpha~ /
    //     2^e))), if d~^T A d~ (1 - 1e-6) > (eta + sqrt(gap))^2 with d~ = alpha~ - 2^e c~,
    //     the exact integer A, and eta = sqrt(trace A) sqrt(P) del >= |d - d~|_A;
    //   - codes below (2^e <= amax / 16): the largest coefficient misses by at least
    //     amax / 2 - del;
    //   - codes above (2^e > 4 amax): the candidate is 0, with error e0 exactly (ties stay).
    // Pairs with a code left go on to the exact ring, and give their block an upper bound
    // of their best clear candidate's error at once, (Rub + (|d~|_A + eta)^2) (1 + 1e-12),
    // or e0: the block's final best cannot exceed it (the candidate is evaluated).
    auto run_bound = [&](int n) {
        bool surv = false;
        uint32_t out = 0;
        double ub = __builtin_inf();
        int ublk = 0;
        if (lane < n) {
            const int slot = (qh + lane) & (QCAP - 1);
            const uint32_t ent = qe[wave][slot];
            const int t = (int)(ent & 0xFFFFu), blk = (int)(ent >> 16);
            ublk = blk;
            const double* rec = ctab + (int64_t)t * Rec::kSize;
            double rr[Rec::kSize];
#pragma unroll
            for (int k = 0; k < Rec::kSize; ++k) rr[k] = rec[k];
            out = (uint32_t)rec_seed(rr[Rec::kSeed]) | ((uint32_t)blk << 16);
            const double e0l = e0v[wave][blk];
            const double thr = fmin(bestv[wave][blk], __longlong_as_double((long long)ubits[wave][blk]));
            const double ilam = rr[Rec::kLam];
            surv = true;
            if (rec_usable(rr[Rec::kSeed]) && e0l > 0.0 && thr < __builtin_inf() && ilam > 0.0) {
                double y[P], al[P], q = 0.0;
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    y[j] = qy[wave][slot][j];
                    q = __builtin_fma(y[j], y[j], q);
                }
                const double Rlb = ((e0l - q) - 1e-6 * e0l) * (1.0 - 1e-12);
                const double gap = thr * (1.0 + 4e-12) - Rlb;
                surv = gap >= 0.0;   // else every code's error is at least R > thr
                if (surv) {
#pragma unroll
                    for (int j = P - 1; j >= 0; --j) {
                        double v = y[j];
#pragma unroll
                        for (int k = j + 1; k < P; ++k)
                            v = __builtin_fma(-rr[Rec::kL + k * (k - 1) / 2 + j], al[k], v);
                        al[j] = v * rr[Rec::kD + j];
                    }
                    constexpr int NA = amat_size(P);
                    double am[NA];
                    const double* arec = atab + (int64_t)t * NA;
#pragma unroll
                    for (int k = 0; k < NA; ++k) am[k] = arec[k];
                    auto aidx = [](int j, int k) { return j * P - j * (j - 1) / 2 + (k - j); };   // j <= k
                    double l1a = 0.0, amax = 0.0;
#pragma unroll
                    for (int j = 0; j < P; ++j) {
                        l1a += fabs(al[j]);
                        amax = fmax(amax, fabs(al[j]));
                    }
                    // the correlation c = U^T w was summed in double: |error| <= 8 eps 2^15
                    // |w|_1 per component, which moves alpha by sqrt(P) that / lambda_min
                    const double del = 1e-6 * l1a + 4.0 * (8.0 * 1.2e-16 * 32768.0) * wl1[wave][blk] * ilam;
                    const double eta = am[NA - 1] * 2.0 * del;
                    const double glam = gap * ilam * (1.0 + 1e-12);
                    const double sg = sqrt(gap) * (1.0 + 1e-12) + eta;
                    const double ath = sg * sg * (1.0 + 2e-6);
                    // d~^T A d~ of one code's candidate
                    auto qform = [&](const double* dd) {
                        double qa = 0.0;
#pragma unroll
                        for (int j = 0; j < P; ++j) {
                            double v = am[aidx(j, j)] * dd[j];
#pragma unroll
                            for (int k = j + 1; k < P; ++k) v = __builtin_fma(2.0 * am[aidx(j, k)], dd[k], v);
                            qa = __builtin_fma(dd[j], v, qa);
                        }
                        return fmax(qa, 0.0);
                    };
                    bool open = amax == 0.0;   // alpha~ = 0: the bound is Rlb <= thr
                    int elo = 0;
                    if (!open) {
                        elo = min(max(ilogb(amax) - 3 - exp_bias + 15, 0), 16);
                        if (elo > 0) {
                            const double d = fmax(0.5 * amax - del, 0.0);
                            open = open || !(d * d > glam);
                        }
                        if (elo + 6 <= 15) open = open || !(e0l > thr);
                        double sc = __builtin_ldexp(1.0, elo + exp_bias - 15);
                        double inv = __builtin_ldexp(1.0, -(elo + exp_bias - 15));
#pragma unroll
                        for (int c = 0; c < 6; ++c) {
                            if (elo + c <= 15) {
                                const double tol = 2.0 * del * inv;
                                double dd[P], s2 = 0.0;
                                bool clear = true;
#pragma unroll
                                for (int j = 0; j < P; ++j) {
                                    const double tj = al[j] * inv;
                                    const double rj = __builtin_rint(tj);
                                    clear = clear && (0.5 - fabs(tj - rj)) > tol;
                                    dd[j] = __builtin_fma(-sc, fmin(fmax(rj, -8.0), 7.0), al[j]);
                                    const double dj = fmax(fabs(dd[j]) - del, 0.0);
                                    s2 = __builtin_fma(dj, dj, s2);
                                }
                                bool gone = s2 > glam;
                                if (!gone && clear) gone = qform(dd) > ath;
                                open = open || !gone;
                            }
                            sc *= 2.0;
                            inv *= 0.5;
                        }
                    }
                    surv = open;
                    if (surv && amax > 0.0) {
                        // the upper bound of this pair's best clear candidate (rare)
                        const double Rub = ((e0l - q) + 1e-6 * e0l) * (1.0 + 1e-12);
                        if (elo + 6 <= 15) ub = e0l;
                        double sc = __builtin_ldexp(1.0, elo + exp_bias - 15);
                        double inv = __builtin_ldexp(1.0, -(elo + exp_bias - 15));
                        for (int c = 0; c < 6 && elo + c <= 15; ++c) {
                            const double tol = 2.0 * del * inv;
                            double dd[P];
                            bool clear = true;
#pragma unroll
                            for (int j = 0; j < P; ++j) {
                                const double tj = al[j] * inv;
                                const double rj = __builtin_rint(tj);
                                clear = clear && (0.5 - fabs(tj - rj)) > tol;
                                dd[j] = __builtin_fma(-sc, fmin(fmax(rj, -8.0), 7.0), al[j]);
                            }
                            if (clear) {
                                const double nup = sqrt(qform(dd) * (1.0 + 1e-6)) + eta;
                                ub = fmin(ub, __builtin_fma(nup, nup, Rub) * (1.0 + 1e-12));
                            }
                            sc *= 2.0;
                            inv *= 0.5;
                        }
                    }
                }
            }
        }
        const bool go = surv && lane < n;
        // survivors lower their block's bound at once (non-negative doubles order like
        // their bits); the exact ring still evaluates them against the true best
        if (go && ub < __builtin_inf())
            __hip_atomic_fetch_min(&ubits[wave][ublk], (unsigned long long)__double_as_longlong(ub),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint64_t bal = __ballot(go);
        if (go) {
            const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
            qe2[wave][(qh2 + qn2 + __popcll(below)) & (QCAP2 - 1)] = out;
        }
        qn2 += __popcll(bal);
        qh = (qh + n) & (QCAP - 1);
        qn -= n;
    };
    // drain the residual-bound ring, keeping the exact ring below 64 + 64 entries
    auto drain = [&]() {
        if constexpr (kCodeBound) {
            while (qn >= 64) {
                run_bound(64);
                while (qn2 >= 64) run_batch(64);
            }
        } else {
            while (qn2 >= 64) run_batch(64);
        }
    };

    // c_{t+1} .. c_{t+P} of the current cycle position t
    double cw[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fma(xtab[(1 + j) * 8 + i], w[i], acc);
        cw[j] = acc;
    }
    // One step along the cycle from its records: bound, queue, slide the window.
    auto step = [&](const double* rec, const double* xn, int t) {
        // bound (fused multiply-adds are fine here: the margin covers any rounding)
        double y[P], q = 0.0;
        int o = Rec::kL;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            double v = cw[j];
#pragma unroll
            for (int k = 0; k < j; ++k) v = __builtin_fma(-rec[o + k], y[k], v);
            o += j;
            y[j] = v * rec[Rec::kD + j];
            q = __builtin_fma(y[j], y[j], q);
        }
        const int s = rec_seed(rec[Rec::kSeed]);
        const double lb = ((e0 - q) - 1e-6 * e0) * (1.0 - 1e-12);
        // the block's best so far, or the upper bound that a queued candidate already gives
        const double thr = kCodeBound ? fmin(best, __longlong_as_double((long long)ubits[wave][lane])) : best;
        const bool prune = (rec_usable(rec[Rec::kSeed]) & (e0 > 0.0) & (thr < __builtin_inf()) & (lb > thr)) |
                           ((best == 0.0) & (s * 16 > bkey));
        const bool keep = active & !prune;
        const uint64_t bal = __ballot(keep);
        if constexpr (kCodeBound) {
            if (keep) {
                const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
                const int slot = (qh + qn + __popcll(below)) & (QCAP - 1);
                qe[wave][slot] = (uint32_t)t | ((uint32_t)lane << 16);
#pragma unroll
                for (int j = 0; j < P; ++j) qy[wave][slot][j] = y[j];
            }
            qn += __popcll(bal);
        } else {   // straight to the exact definition
            if (keep) {
                const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
                qe2[wave][(qh2 + qn2 + __popcll(below)) & (QCAP2 - 1)] = (uint32_t)s | ((uint32_t)lane << 16);
            }
            qn2 += __popcll(bal);
        }
        // slide the window: c_{t+P+1} in, c_{t+1} out
        double cn = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) cn = __builtin_fma(xn[i], w[i], cn);
#pragma unroll
        for (int j = 0; j + 1 < P; ++j) cw[j] = cw[j + 1];
        cw[P - 1] = cn;
    };
    // Two steps per round, their four records read together (one wait per round).  The
    // last step revisits seed 1; its pairs merge like any other (same candidates).
#pragma unroll 1
    for (int t = 0; t < kSteps; t += 2) {
        double ra[Rec::kSize], rb[Rec::kSize], xa[8], xb[8];
        const double* pa = ctab + (int64_t)t * Rec::kSize;
        const double* pxa = xtab + (int64_t)(t + P + 1) * 8;
#pragma unroll
        for (int k = 0; k < Rec::kSize; ++k) {
            ra[k] = pa[k];
            rb[k] = pa[Rec::kSize + k];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xa[i] = pxa[i];
            xb[i] = pxa[8 + i];
        }
        step(ra, xa, t);
        step(rb, xb, t + 1);
        drain();
        // every 64 steps the group's waves meet, so they read the same table records
        // at about the same time and one wave's cache misses are the others' hits
        if ((t & 63) == 0) __syncthreads();
    }
    // the rest of both rings, one batch at a time
#pragma unroll 1
    while (qn > 0 || qn2 > 0) {
        if constexpr (kCodeBound) {
            if (qn > 0) {
                run_bound(qn < 64 ? qn : 64);
                continue;
            }
        }
        run_batch(qn2 < 64 ? qn2 : 64);
    }

    if (bkey != 0x7FFFFFFF) {
        res[threadIdx.x][0] = (uint32_t)(bkey >> 4) | ((uint32_t)(bkey & 15) << 16);
        res[threadIdx.x][1] = bnib;
        if (errs && active) errs[b] = best;
    } else {                                  // no seed had a solvable system
        res[threadIdx.x][0] = 0u;
        res[threadIdx.x][1] = 0u;
        if (errs && active) errs[b] = __builtin_inf();
    }
    __syncthreads();
    // the group's streams: its seeds, nb * P nibbles and nb codes (whole words and bytes:
    // the group starts at a multiple of 512 blocks)
    const int nb = (int)(nblk - b0 < 512 ? nblk - b0 : 512);
    const int tid = threadIdx.x;
    if (tid < nb) seeds[b0 + tid] = (uint16_t)(res[tid][0] & 0xFFFFu);
    if (tid < (nb * P + 3) / 4) {             // coefficient word tid of the group
        uint32_t word = 0;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int n = 4 * tid + qq;       // nibble within the group
            const int blk = n / P, j = n % P;
            if (blk < nb) word |= ((res[blk][1] >> (4 * j)) & 0xFu) << (4 * qq);
        }
        coefs[b0 * P / 4 + tid] = (uint16_t)word;
    }
    if (tid < (nb + 1) / 2) {                 // code byte of blocks 2t, 2t+1
        uint32_t byte = (res[2 * tid][0] >> 16) & 0xFu;
        if (2 * tid + 1 < nb) byte |= ((res[2 * tid + 1][0] >> 16) & 0xFu) << 4;
        codes[b0 / 2 + tid] = (uint8_t)byte;
    }
}

}  // namespace seedmm

using namespace seedmm;

extern "C" size_t seedmm_search_table_bytes(int P) {
    if (P != 3 && P != 4) return 0;
    return table_layout(P).total;
}

extern "C" int seedmm_search_prepare(int P, void* table, size_t table_bytes, void* hip_stream) {
    if ((P != 3 && P != 4) || !table) return SEEDMM_EINVAL;
    const TableLayout L = table_layout(P);
    if (table_bytes < L.total) return SEEDMM_EINVAL;
    if (((uintptr_t)table & 255u) != 0) return SEEDMM_EALIGN;
    hipStream_t st = (hipStream_t)hip_stream;
    char* base = (char*)table;
    uint32_t* x = (uint32_t*)(base + L.cycle);
    hipLaunchKernelGGL(k_cycle, dim3(1), dim3(64), 0, st, x);
    const dim3 grid((kXRecs + 255) / 256);   // kXRecs >= kSteps
    if (P == 4) hipLaunchKernelGGL(k_seed_tables<4>, grid, dim3(256), 0, st, (const uint32_t*)x, (double*)(base + L.xrec), (double*)(base + L.chol), (double*)(base + L.amat));
    else hipLaunchKernelGGL(k_seed_tables<3>, grid, dim3(256), 0, st, (const uint32_t*)x, (double*)(base + L.xrec), (double*)(base + L.chol), (double*)(base + L.amat));
    return hipGetLastError() == hipSuccess ? SEEDMM_OK : SEEDMM_EHIP;
}

extern "C" int seedmm_search(const float* W, int ldw, const float* colw, int M, int K, int P,
                             int32_t exp_bias, uint16_t* seeds, uint16_t* coefs,
                             uint8_t* codes, double* err, const void* table,
                             void* hip_stream) {
    if (M < 0 || K < 0 || K % 8 != 0 || (P != 3 && P != 4)) return SEEDMM_EINVAL;
    if (exp_bias < -100 || exp_bias > 100) return SEEDMM_EINVAL;
    if (ldw < K) return SEEDMM_EINVAL;
    const int64_t nblk = (int64_t)M * (K / 8);
    if (nblk == 0) return SEEDMM_OK;
    if (!W || !seeds || !coefs || !codes) return SEEDMM_EINVAL;
    hipStream_t st = (hipStream_t)hip_stream;
    if (!colw) {
        // without importances: one block per lane with the per-seed table
        if (!table) return SEEDMM_EINVAL;
        if (((uintptr_t)table & 255u) != 0) return SEEDMM_EALIGN;
        const TableLayout L = table_layout(P);
        const double* xt = (const double*)((const char*)table + L.xrec);
        const double* ct = (const double*)((const char*)table + L.chol);
        const double* at = (const double*)((const char*)table + L.amat);
        const dim3 grid((unsigned)((nblk + 511) / 512));
        if (P == 4) hipLaunchKernelGGL((k_search_lanes<4>), grid, dim3(512), 0, st, W, (int64_t)ldw, K, exp_bias, nblk, xt, ct, at, seeds, coefs, codes, err);
        else hipLaunchKernelGGL((k_search_lanes<3>), grid, dim3(512), 0, st, W, (int64_t)ldw, K, exp_bias, nblk, xt, ct, at, seeds, coefs, codes, err);
    } else {
        const dim3 grid((unsigned)((nblk + 3) / 4));
        if (P == 4) hipLaunchKernelGGL((k_search<4, true>), grid, dim3(256), 0, st, W, (int64_t)ldw, colw, K, exp_bias, nblk, seeds, coefs, codes, err);
        else hipLaunchKernelGGL((k_search<3, true>), grid, dim3(256), 0, st, W, (int64_t)ldw, colw, K, exp_bias, nblk, seeds, coefs, codes, err);
    }
    return hipGetLastError() == hipSuccess ? SEEDMM_OK : SEEDMM_EHIP;
}
