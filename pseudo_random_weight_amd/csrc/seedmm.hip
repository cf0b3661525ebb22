// seedmm.hip -- gfx950 kernels and the C ABI of the SeedLM seed-decoding products.
//
// Every kernel regenerates the weight blocks it needs from (seed, coefficients,
// exponent code) in registers and consumes them at once; no kernel but
// seedmm_reconstruct writes a weight to memory (NanoSeedLM README, "Highlights";
// barnson.org post, "What I changed: September 2026", never decompress).
//
// Work mapping shared by the product kernels.  A wave owns 16 rows of one matrix.
// Lane l = r + 16 q (r = l % 16, q = l / 16) decodes blocks of row r in runs of 8
// consecutive blocks ("segments"), so one lane's 8 seeds, 8 coefficient words and 8
// codes arrive in three vector loads.  Segments are dealt round-robin to the 4 lane
// quarters and to the waves that split K.  At each step a lane holds one block = 8
// consecutive k of its row, which is exactly the A operand of one
// v_mfma_f32_16x16x32_bf16 lane (16 rows x 32 k per wave); the matching B lane holds the
// same 8 k of one token.  The k order inside the MFMA is a permutation of the true k
// order, applied identically to A and B.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/seedmm.h"
#include "moe_layer.hpp"
#include "seed_decode.hpp"

namespace seedmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte register value.  HIP's uint4 is a struct whose copies lower to memcpy, which
// keeps staging registers in scratch memory; the native vector type stays in VGPRs.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { MODE_GEMM = 0, MODE_GATEUP = 1, MODE_DOWN = 2 };

// ----------------------------------------------------------------------------------
// Stream access for a run of 8 blocks starting at block b0 of one matrix.
// VEC: b0 % 8 == 0 and the stream bases are 16-byte aligned -> three vector loads.
// Otherwise each block is read on its own (any K % 8 == 0, any alignment).
// ----------------------------------------------------------------------------------
template <int P, bool VEC>
struct Seg {
    uint32_t sd[4];                   // VEC: seeds, two per word
    uint32_t cf[P == 4 ? 4 : 3];      // VEC: 8 blocks of P nibbles
    uint32_t cd;                      // VEC: 8 codes
    uint32_t s1[8], c1[8], d1[8];     // per-block path

    __device__ __forceinline__ void load(const uint16_t* __restrict__ seeds,
                                         const uint16_t* __restrict__ coefs,
                                         const uint8_t* __restrict__ codes, int64_t b0,
                                         int nvalid) {
        if constexpr (VEC) {
            const uint4 s = *reinterpret_cast<const uint4*>(seeds + b0);
            sd[0] = s.x; sd[1] = s.y; sd[2] = s.z; sd[3] = s.w;
            if constexpr (P == 4) {
                const uint4 c = *reinterpret_cast<const uint4*>(coefs + b0);
                cf[0] = c.x; cf[1] = c.y; cf[2] = c.z; cf[3] = c.w;
            } else {
                const uint32_t* c = reinterpret_cast<const uint32_t*>(coefs) + (b0 * 3) / 8;
                cf[0] = c[0]; cf[1] = c[1]; cf[2] = c[2];
            }
            cd = *reinterpret_cast<const uint32_t*>(codes + b0 / 2);
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                s1[s] = 0; c1[s] = 0; d1[s] = 0;
                if (s < nvalid) {
                    const int64_t b = b0 + s;
                    s1[s] = seeds[b];
                    if constexpr (P == 4) {
                        c1[s] = coefs[b];
                    } else {
                        const int64_t n = b * 3;
                        const int sh = 4 * (int)(n & 3);
                        uint32_t v = (uint32_t)coefs[n >> 2] >> sh;
                        if (sh > 4) v |= (uint32_t)coefs[(n >> 2) + 1] << (16 - sh);
                        c1[s] = v;
                    }
                    d1[s] = ((uint32_t)codes[b >> 1] >> (4 * (int)(b & 1))) & 0xFu;
                }
            }
        }
    }
    // VEC: the loaded words are needed here (an empty asm reads them), so the loads
    // complete before this point and cannot be moved past it into a later iteration
    __device__ __forceinline__ void hold() const {
        static_assert(VEC, "vector-load segments only");
        if constexpr (P == 4)
            asm volatile("" ::"v"(sd[0]), "v"(sd[1]), "v"(sd[2]), "v"(sd[3]), "v"(cf[0]),
                         "v"(cf[1]), "v"(cf[2]), "v"(cf[3]), "v"(cd));
        else
            asm volatile("" ::"v"(sd[0]), "v"(sd[1]), "v"(sd[2]), "v"(sd[3]), "v"(cf[0]),
                         "v"(cf[1]), "v"(cf[2]), "v"(cd));
    }
    __device__ __forceinline__ uint32_t seed(int s) const {
        if constexpr (VEC) return __builtin_amdgcn_ubfe(sd[s >> 1], 16 * (s & 1), 16);
        else return s1[s];
    }
    __device__ __forceinline__ uint32_t coef(int s) const {
        if constexpr (VEC) {
            if constexpr (P == 4) {
                return __builtin_amdgcn_ubfe(cf[s >> 1], 16 * (s & 1), 16);
            } else {
                const int bit = 12 * s, w = bit >> 5, sh = bit & 31;
                return sh <= 20 ? (cf[w] >> sh)
                                : __builtin_amdgcn_alignbit(cf[w + 1], cf[w], sh);
            }
        } else {
            return c1[s];
        }
    }
    __device__ __forceinline__ uint32_t code(int s) const {
        if constexpr (VEC) return __builtin_amdgcn_ubfe(cd, 4 * s, 4);
        else return d1[s];
    }
    // VEC: all-zero coefficients for a segment outside the matrix (zero weights); the
    // per-block path loads zeros for missing blocks already
    __device__ __forceinline__ void clear_coefs_unless(bool keep) {
        if constexpr (VEC) {
#pragma unroll
            for (int k = 0; k < (P == 4 ? 4 : 3); ++k) cf[k] = keep ? cf[k] : 0u;
        }
    }
};

// Base pointers of matrix `e` of E stacked [M][K] matrices.
struct Mat {
    const uint16_t* seeds;
    const uint16_t* coefs;
    const uint8_t* codes;
    int exp_bias;
};

// Mixed packs (P chosen per expert): bit e of p4mask is set when expert e has P = 4.
__device__ __forceinline__ bool p4_of(const uint32_t* p4mask, int e) {
    return (p4mask[e >> 5] >> (e & 31)) & 1u;
}

// Coefficient words of experts 0..e-1: e * nblk * P / 4 for one P; with a mask, experts
// of P = 3 take 3 nblk / 4 words and experts of P = 4 take nblk words (nblk % 4 == 0).
__device__ __forceinline__ int64_t coef_words_before(const uint32_t* p4mask, int e,
                                                     int64_t nblk, int P) {
    if (!p4mask) return (int64_t)e * (nblk * P / 4);
    int n4 = 0;
    for (int w = 0; w < (e >> 5); ++w) n4 += __popc(p4mask[w]);
    n4 += __popc(p4mask[e >> 5] & ((1u << (e & 31)) - 1u));
    return (nblk / 4) * (3 * (int64_t)e + n4);
}

// slot (device int32[E], or null): an expert cache, where expert e's streams sit in slot
// slot[e] and slot s starts slot_stride bytes after slot s - 1 (m's pointers are slot 0's
// streams); its exp_bias stays at index e.  Slots are used with one P only.
__device__ __forceinline__ Mat mat_of(const seedmm_mat& m, int e, int64_t nblk, int P,
                                      int eb_scalar, bool eb_from_ptr,
                                      const uint32_t* p4mask = nullptr,
                                      const int32_t* slot = nullptr, int64_t slot_stride = 0) {
    Mat r;
    if (slot) {
        const int64_t off = (int64_t)slot[e] * slot_stride;
        r.seeds = (const uint16_t*)((const char*)m.seeds + off);
        r.coefs = (const uint16_t*)((const char*)m.coefs + off);
        r.codes = m.codes + off;
    } else {
        r.seeds = m.seeds + (int64_t)e * nblk;
        r.coefs = m.coefs + coef_words_before(p4mask, e, nblk, P);
        r.codes = m.codes + (int64_t)e * (nblk / 2);
    }
    r.exp_bias = eb_from_ptr ? m.exp_bias[e] : eb_scalar;
    return r;
}

__device__ __forceinline__ bf16x8 pack_bf16(const float w[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)w[i];
    return v;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
    return v;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8, u);
}

// ----------------------------------------------------------------------------------
// seedmm_reconstruct: one thread per block, writes the block's 8 weights.
// ----------------------------------------------------------------------------------
template <int P, bool BF16>
__global__ __launch_bounds__(256) void k_reconstruct(const uint16_t* __restrict__ seeds,
                                                     const uint16_t* __restrict__ coefs,
                                                     const uint8_t* __restrict__ codes,
                                                     int exp_bias, void* __restrict__ W,
                                                     int K, int64_t nblk) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    Seg<P, false> sg;
    sg.load(seeds, coefs, codes, b, 1);
    const Window win = lfsr_window(sg.seed(0));
    float w[8];
    decode_block<P>(win, sg.coef(0), sg.code(0), exp_bias, w);
    const int nbpr = K / 8;
    const int64_t m = b / nbpr, kb = b % nbpr;
    if constexpr (BF16) {
        bf16x8 v = pack_bf16(w);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(W) + m * K + 8 * kb) =
            __builtin_bit_cast(uint4, v);
    } else {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(W) + m * K + 8 * kb);
        o[0] = make_float4(w[0], w[1], w[2], w[3]);
        o[1] = make_float4(w[4], w[5], w[6], w[7]);
    }
}

// ----------------------------------------------------------------------------------
// fp32 activations: products on the vector ALUs with exact fp32 weights.
// 4 waves split K; NTOK activation rows per pass.
// ----------------------------------------------------------------------------------
template <int P, bool VEC, int NTOK>
__global__ __launch_bounds__(256) void k_gemv_f32(const uint16_t* __restrict__ seeds,
                                                  const uint16_t* __restrict__ coefs,
                                                  const uint8_t* __restrict__ codes,
                                                  int exp_bias, const float* __restrict__ x,
                                                  int ldx, float* __restrict__ y, int ldy,
                                                  int M, int K, int N) {
    __shared__ float red[4][NTOK][16];
    __shared__ uint32_t tab[512];
    fill_lfsr_tables(tab);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int row = blockIdx.x * 16 + r;
    const bool rv = row < M;
    const int nbpr = K / 8;
    const int nseg = (nbpr + 7) / 8;
    const int n_it = (nseg + 15) / 16;
    const int n0 = blockIdx.y * NTOK;
    const int64_t rowb = (int64_t)(rv ? row : 0) * nbpr;

    float acc[NTOK];
#pragma unroll
    for (int n = 0; n < NTOK; ++n) acc[n] = 0.0f;

    for (int it = 0; it < n_it; ++it) {
        const int g = it * 16 + wave * 4 + q;
        if (!(g < nseg && rv)) continue;
        const int nvalid = min(8, nbpr - g * 8);
        Seg<P, VEC> sg;
        sg.load(seeds, coefs, codes, rowb + g * 8, nvalid);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if (!VEC && s >= nvalid) break;
            const int kb = g * 8 + s;
            const Window win = window_from_tables(sg.seed(s), tab);
            int f[8];
            block_sums<P>(win, sg.coef(s), f);
            const float sc = block_scale(sg.code(s), exp_bias);
#pragma unroll
            for (int n = 0; n < NTOK; ++n) {
                if (n0 + n < N) {
                    const float4* xp =
                        reinterpret_cast<const float4*>(x + (int64_t)(n0 + n) * ldx + 8 * kb);
                    const float4 xa = xp[0], xb = xp[1];
                    const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
                    float blk = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        blk = __builtin_fmaf(xv[i], __int_as_float(f[i]) - kMagic, blk);
                    acc[n] = __builtin_fmaf(blk, sc, acc[n]);
                }
            }
        }
    }
    // reduce the four lane quarters of each row, then the four waves
#pragma unroll
    for (int n = 0; n < NTOK; ++n) {
        float v = acc[n];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (q == 0) red[wave][n][r] = v;
    }
    __syncthreads();
    if (wave == 0 && q == 0 && rv) {
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
            if (n0 + n < N)
                y[(int64_t)(n0 + n) * ldy + row] =
                    ((red[0][n][r] + red[1][n][r]) + red[2][n][r]) + red[3][n][r];
        }
    }
}

// ----------------------------------------------------------------------------------
// bf16 activations: weights regenerated per lane, rounded to bf16, multiplied on the
// matrix cores (16x16x32 bf16 -> fp32).
//   MODE_GEMM   : y[n][m] = sum_k W[m][k] x[n][k]                       (one matrix)
//   MODE_GATEUP : h[p][m] = bf16( silu(G_e x_t)[m] * (U_e x_t)[m] ),  t = p / top_k
//   MODE_DOWN   : o[p][m] = w[p] * (D_e h_p)[m]
// Grid: x = tiles of 16 weight rows, y = active experts (expert y = the y-th expert with
// a nonzero count).  The 4 waves of a workgroup split K (and, for GATEUP, the two
// matrices).  Tokens are processed in passes of NT*16.
// ----------------------------------------------------------------------------------
struct MfmaArgs {
    seedmm_mat A;           // gate (GATEUP) or the matrix
    seedmm_mat A2;          // up (GATEUP)
    int exp_bias;           // GEMM: scalar exp_bias
    int M, K;               // rows and columns of one matrix
    const uint16_t* x;      // GEMM/GATEUP: activations bf16 [.][ldx]; DOWN: h [.][ldx]
    int ldx;
    int N;                  // GEMM: number of rows of x
    const int32_t* counts;  // experts: int32[E]
    const int32_t* lists;   // experts: int32[E][T]
    int E, T, top_k;
    const float* topk_w;    // DOWN
    float* y;               // GEMM: fp32 [N][ldy]; DOWN: fp32 [T*top_k][ldy]
    uint16_t* h;            // GATEUP: bf16 [T*top_k][ldy]
    int ldy;
    const int32_t* ids;     // one token (T = 1): topk_ids, workgroup y serves slot y
    const uint32_t* p4mask; // mixed packs: bit e set = expert e has P = 4; this launch
                            // serves the experts of its own P only (null: one P)
    const int32_t* slot;    // expert cache: int32[E], slot of expert e's streams (null:
                            // stacked experts, expert e at position e)
    int64_t slot_stride;    // expert cache: bytes from one slot to the next
    int e_lo, e_hi;         // routed kernels: serve experts e_lo <= e < e_hi only (e_hi = 0:
                            // all E; the one-token path ignores them)
};

// Pair lists of the one-token path: slot y's list is the single pair index y.
__device__ const int32_t kSlotIota[64] = {
    0,  1,  2,  3,  4,  5,  6,  7,  8,  9,  10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20, 21,
    22, 23, 24, 25, 26, 27, 28, 29, 30, 31, 32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43,
    44, 45, 46, 47, 48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63};

// Per-lane state of one pass over K.
struct Lane {
    const uint32_t* tab;  // LDS continuation tables (TAB kernels), else null
    Mat W;               // the matrix this wave regenerates
    int64_t rowb;        // first block of this lane's row (row clamped into range)
    bool rv;             // the row exists
    int nbpr, nseg, n_it, ks, q;
};

template <bool TAB>
__device__ __forceinline__ Window window_of(uint32_t seed16, const uint32_t* tab) {
    if constexpr (TAB) return window_from_tables(seed16, tab);
    else return lfsr_window(seed16);
}

// One pass over this wave's share of K for NTA token tiles.  Branch-free: addresses are
// clamped into range and padding blocks get all-zero coefficients, which decode to exact
// zero weights.  The stream words of the next segment are loaded while the current one
// is regenerated.  XL: the single token's activation row sits in LDS (xs, K bf16), so
// the stream words are the loop's only global loads.

// Segment of iteration `it` of a lane (KS waves share one K range): its first block
// gc * 8 (clamped into the row) and how many of its blocks exist.
template <int KS>
__device__ __forceinline__ void seg_of(const Lane& L, int it, int& gc, int& nvalid) {
    const int g = it * (KS * 4) + L.ks * 4 + L.q;
    gc = g < L.nseg ? g : L.nseg - 1;
    nvalid = (g < L.nseg && L.rv) ? min(8, L.nbpr - gc * 8) : 0;
}

// The stream words of a lane's first segment.
template <int P, bool VEC, int KS>
__device__ __forceinline__ Seg<P, VEC> first_seg(const Lane& L) {
    int gc, nvalid;
    seg_of<KS>(L, 0, gc, nvalid);
    Seg<P, VEC> s;
    s.load(L.W.seeds, L.W.coefs, L.W.codes, L.rowb + gc * 8, VEC ? 8 : nvalid);
    return s;
}

// PRE: the first segment's words were loaded by the caller (`pre`, from first_seg), so
// their latency overlaps the caller's set-up.
template <int P, bool VEC, int NTA, int KS, bool TAB, bool XL = false, bool PRE = false>
__device__ __forceinline__ void mfma_k_loop(const Lane& L, const uint16_t* const* brow,
                                            f32x4* acc, const uint16_t* xs = nullptr,
                                            const Seg<P, VEC>* pre = nullptr) {
    static_assert(!XL || NTA == 1, "the LDS activation row serves one token");
    auto seg = [&](int it, int& gc, int& nvalid) { seg_of<KS>(L, it, gc, nvalid); };
    int gc, nvalid;
    seg(0, gc, nvalid);
    Seg<P, VEC> cur;
    if constexpr (PRE) cur = *pre;
    else cur = first_seg<P, VEC, KS>(L);
    for (int it = 0; it < L.n_it; ++it) {
        int gn, nvn;
        seg(it + 1 < L.n_it ? it + 1 : it, gn, nvn);
        Seg<P, VEC> nxt;
        nxt.load(L.W.seeds, L.W.coefs, L.W.codes, L.rowb + gn * 8, VEC ? 8 : nvn);
        // one-token kernel: issue those loads here, ahead of this segment's work
        if constexpr (XL && VEC) __builtin_amdgcn_sched_barrier(0);
        cur.clear_coefs_unless(nvalid > 0);   // VEC segments are whole or absent
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            float w[8];
            decode_block<P>(window_of<TAB>(cur.seed(s), L.tab), cur.coef(s), cur.code(s),
                            L.W.exp_bias, w);
            const bf16x8 A = pack_bf16(w);
            // VEC rows hold whole segments, so block gc*8+s exists; the per-block path
            // clamps the padding blocks of a row's last segment
            const int kb = VEC ? gc * 8 + s : min(gc * 8 + s, L.nbpr - 1);
#pragma unroll
            for (int t = 0; t < NTA; ++t) {
                const bf16x8 B = XL ? *(const bf16x8*)(xs + 8 * kb)
                                    : load_bf16x8(brow[t] + 8 * kb);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[t], 0, 0, 0);
            }
        }
        // one-token kernel: the next segment's words arrive during this iteration (the
        // barrier keeps their wait after this segment's work)
        if constexpr (XL && VEC) {
            __builtin_amdgcn_sched_barrier(0);
            nxt.hold();
        }
        cur = nxt;
        gc = gn;
        nvalid = nvn;
    }
}

// One pass: NTA tiles of 16 tokens starting at token slot `pass`.
template <int P, bool VEC, int NTA, int MODE, int NT, bool TAB, int RT, bool XL = false,
          bool PRE = false>
__device__ __forceinline__ void mfma_pass(const MfmaArgs& a, const Lane& L, const int32_t* list,
                                          int n_e, int pass, int m0, int wave, int lane, int r,
                                          f32x4 (*red)[NT][64], const uint16_t* xs = nullptr,
                                          const Seg<P, VEC>* pre = nullptr) {
    constexpr int KS = MODE == MODE_GATEUP ? 2 : 4 / RT;   // waves sharing one K range
    // B rows of this lane (token column r of every tile); slots past n_e repeat the last
    // token so every load stays in range -- their outputs are never stored.
    const uint16_t* brow[NTA];
#pragma unroll
    for (int t = 0; t < NTA; ++t) {
        const int i = min(pass + 16 * t + r, n_e - 1);
        int64_t src;
        if constexpr (MODE == MODE_GEMM) src = i;
        else if constexpr (MODE == MODE_GATEUP) src = list[i] / a.top_k;
        else src = list[i];
        brow[t] = a.x + src * a.ldx;
    }
    f32x4 acc[NTA];
#pragma unroll
    for (int t = 0; t < NTA; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_k_loop<P, VEC, NTA, KS, TAB, XL, PRE>(L, brow, acc, xs, pre);

    // partial sums of the four waves meet in LDS (fixed order); wave c % 4 finishes the
    // (row tile, token tile) pair c
#pragma unroll
    for (int t = 0; t < NTA; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < RT * NTA; ++c) {
        if ((c & 3) != wave) continue;
        const int rt = c % RT, t = c / RT;
        f32x4 v, v2;
        if constexpr (MODE == MODE_GATEUP) {
            v = red[0][t][lane] + red[1][t][lane];      // gate
            v2 = red[2][t][lane] + red[3][t][lane];     // up
        } else if constexpr (KS == 4) {
            v = ((red[0][t][lane] + red[1][t][lane]) + red[2][t][lane]) + red[3][t][lane];
        } else if constexpr (KS == 2) {
            v = red[2 * rt][t][lane] + red[2 * rt + 1][t][lane];
        } else {
            v = red[rt][t][lane];
        }
        const int i = pass + 16 * t + r;     // D column = token slot
        if (i >= n_e) continue;
        int64_t dst;
        float scale = 1.0f;
        if constexpr (MODE == MODE_GEMM) {
            dst = i;
        } else {
            dst = list[i];
            if constexpr (MODE == MODE_DOWN) scale = a.topk_w[dst];
        }
        const int mq = m0 + 16 * rt + 4 * (lane >> 4);   // D rows mq .. mq+3
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = mq + j;
            if (m >= a.M) continue;
            if constexpr (MODE == MODE_GATEUP) {
                const float gt = v[j], up = v2[j];
                const float hv = gt / (1.0f + expf(-gt)) * up;
                const __bf16 hb = (__bf16)hv;
                a.h[dst * a.ldy + m] = __builtin_bit_cast(uint16_t, hb);
            } else {
                a.y[dst * a.ldy + m] = scale * v[j];
            }
        }
    }
    __syncthreads();
}

// 4 waves on 16 weight rows.  GATEUP: waves 0-1 regenerate gate, waves 2-3 up, each
// over half of K; otherwise the 4 waves take a quarter of K each.
// The products of one workgroup once its expert (e, n_e pairs in `list`) is known.
// The lane state of wave `wave` of a workgroup serving expert e (row tile blockIdx.x).
template <int P, int MODE, bool TAB, int RT>
__device__ __forceinline__ Lane make_lane(const MfmaArgs& a, int e, const uint32_t* tab,
                                          int wave, int lane, int& m0) {
    constexpr int KS = MODE == MODE_GATEUP ? 2 : 4 / RT;
    const int r = lane & 15;
    Lane L;
    L.tab = TAB ? tab : nullptr;
    L.ks = wave % KS;
    L.q = lane >> 4;
    L.nbpr = a.K / 8;
    const int64_t nblk = (int64_t)a.M * L.nbpr;
    // gate/up: waves KS.. regenerate up (field-wise selects keep the pointers scalar)
    const bool second = MODE == MODE_GATEUP && wave >= KS;
    seedmm_mat src;
    src.seeds = second ? a.A2.seeds : a.A.seeds;
    src.coefs = second ? a.A2.coefs : a.A.coefs;
    src.codes = second ? a.A2.codes : a.A.codes;
    src.exp_bias = second ? a.A2.exp_bias : a.A.exp_bias;
    L.W = mat_of(src, e, nblk, P, a.exp_bias, MODE != MODE_GEMM, a.p4mask, a.slot, a.slot_stride);
    m0 = blockIdx.x * 16 * RT;
    const int row = m0 + 16 * (wave / KS % RT) + r;
    L.rv = row < a.M;
    L.rowb = (int64_t)(L.rv ? row : a.M - 1) * L.nbpr;
    L.nseg = (L.nbpr + 7) / 8;
    L.n_it = (L.nseg + KS * 4 - 1) / (KS * 4);
    return L;
}

template <int P, bool VEC, int NT, int MODE, bool TAB, int RT, bool XL = false>
__device__ __forceinline__ void mfma_run(const MfmaArgs& a, int e, int n_e, const int32_t* list,
                                         const uint32_t* tab, f32x4 (*red)[NT][64],
                                         const uint16_t* xs = nullptr) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r = lane & 15;
    int m0;
    const Lane L = make_lane<P, MODE, TAB, RT>(a, e, tab, wave, lane, m0);

    if constexpr (NT == 1) {   // one token (n_e == 1)
        mfma_pass<P, VEC, 1, MODE, NT, TAB, RT, XL>(a, L, list, n_e, 0, m0, wave, lane, r, red, xs);
    } else {
        static_assert(NT == 4, "the decode kernel holds 1 or at most 4 token tiles");
        for (int pass = 0; pass < n_e; pass += NT * 16) {
            const int ntiles = min(NT, (n_e - pass + 15) / 16);   // uniform
            switch (ntiles) {
                case 1: mfma_pass<P, VEC, 1, MODE, NT, TAB, RT>(a, L, list, n_e, pass, m0, wave, lane, r, red); break;
                case 2: mfma_pass<P, VEC, 2, MODE, NT, TAB, RT>(a, L, list, n_e, pass, m0, wave, lane, r, red); break;
                case 3: mfma_pass<P, VEC, 3, MODE, NT, TAB, RT>(a, L, list, n_e, pass, m0, wave, lane, r, red); break;
                default: mfma_pass<P, VEC, 4, MODE, NT, TAB, RT>(a, L, list, n_e, pass, m0, wave, lane, r, red); break;
            }
        }
    }
}

// Mixed packs (a.p4mask set) run one launch per P; each launch serves only the experts
// of its own P.  (One launch holding both bodies was slower: the two bodies shared one
// register allocation and the P = 3 loop came out scheduled worse than in its own kernel.)
// Register budget: 5 waves per SIMD for P = 4 and 6 for P = 3, the fastest of 4, 5 and 6
// measured (6 makes P = 4 gate/up spill; 4 leaves fewer waves to hide load latency).
template <int P, bool VEC, int NT, int MODE, bool TAB, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(VEC ? (P == 4 ? 5 : 6) : 2))) void k_mfma(const MfmaArgs a) {
    static_assert(MODE != MODE_GATEUP || RT == 1, "gate/up pairs its waves by matrix");
    __shared__ f32x4 red[4][NT][64];
    __shared__ uint32_t tab[TAB ? 512 : 1];

    const int lane = threadIdx.x & 63;

    // ---- which expert this workgroup serves --------------------------------------
    int e = 0, n_e = a.N;
    const int32_t* list = nullptr;
    if (MODE != MODE_GEMM && a.ids) {
        // one token: its top_k slots are top_k distinct experts, one workgroup row each
        const int y = blockIdx.y;   // slot
        e = a.ids[y];
        if (e < 0 || e >= a.E) return;   // uniform; invalid ids are the caller's error
        if (a.p4mask && p4_of(a.p4mask, e) != (P == 4)) return;   // the other launch's
        n_e = 1;
        list = kSlotIota + y;
    } else if constexpr (MODE != MODE_GEMM) {
        // the target-th active expert (of this launch's P when the pack is mixed)
        const int target = blockIdx.y;
        const int ehi = a.e_hi > 0 ? a.e_hi : a.E;
        int found = -1, cum = 0;
        for (int base = a.e_lo; base < ehi && found < 0; base += 64) {
            const int idx = base + lane;
            const bool act = idx < ehi && a.counts[idx] > 0 &&
                             (!a.p4mask || p4_of(a.p4mask, idx) == (P == 4));
            const uint64_t bal = __ballot(act);
            const int c = __popcll(bal);
            if (target < cum + c) {
                const int k = target - cum;
                const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
                const bool mine = act && __popcll(below) == k;
                found = base + __ffsll((long long)__ballot(mine)) - 1;
            }
            cum += c;
        }
        if (found < 0) return;   // uniform across the workgroup
        e = found;
        n_e = a.counts[e];
        list = a.lists + (int64_t)e * a.T;
    }
    if (n_e <= 0) return;
    if constexpr (TAB) fill_lfsr_tables(tab);
    mfma_run<P, VEC, NT, MODE, TAB, RT>(a, e, n_e, list, tab, red);
}

// One token (T = 1): workgroup row y serves slot y of the token.  The same products as
// k_mfma's one-token path (bit for bit), with the activation row (x for gate/up, the
// slot's h row for down) staged once in LDS and a register budget of 2 waves per SIMD
// (one wave round fills the chip at T = 1), so each segment's stream loads can be in
// flight while the previous segment is regenerated.  Dynamic LDS: K bf16.
template <int P, bool VEC, int MODE, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_mfma_one(const MfmaArgs a) {
    static_assert(MODE != MODE_GEMM, "one-token kernel of the routed layer");
    constexpr int KS = MODE == MODE_GATEUP ? 2 : 4 / RT;
    __shared__ f32x4 red[4][1][64];
    __shared__ uint32_t tab[512];
    extern __shared__ uint4 xs[];
    // Start-up: the activation row's first piece and the first segment's stream words
    // are requested together, before the tables are computed and the barrier, so the
    // two memory latencies overlap each other and the table fill.
    const int y = blockIdx.y;   // slot
    const int e = a.ids[y];
    const int tid = threadIdx.x;
    const int64_t row = MODE == MODE_GATEUP ? 0 : (int64_t)y;
    const uint4* src = (const uint4*)(a.x + row * a.ldx);
    const int nx = a.K / 8;
    uint4 x0 = {0u, 0u, 0u, 0u};
    if (tid < nx) x0 = src[tid];
    // uniform; invalid ids are the caller's error, other-P experts the other launch's
    const bool serve = e >= 0 && e < a.E && !(a.p4mask && p4_of(a.p4mask, e) != (P == 4));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    int m0 = 0;
    Lane L;
    Seg<P, VEC> first;
    if (serve) {
        L = make_lane<P, MODE, true, RT>(a, e, tab, wave, lane, m0);
        first = first_seg<P, VEC, KS>(L);
    }
    for (int i = tid; i < 512; i += 256)
        tab[i] = lfsr_next32(i < 256 ? (uint32_t)i : (uint32_t)(i - 256) << 8);
    if (tid < nx) xs[tid] = x0;
    for (int i = tid + 256; i < nx; i += 256) xs[i] = src[i];
    __syncthreads();   // publishes the tables and xs
    if (!serve) return;
    mfma_pass<P, VEC, 1, MODE, 1, true, RT, true, true>(a, L, kSlotIota + y, 1, 0, m0, wave,
                                                        lane, lane & 15, red,
                                                        (const uint16_t*)xs, &first);
}

// One token, down with the combine folded in: a workgroup owns 8 rows of y for all top_k
// (<= 8) slots, so the slot outputs meet in its LDS and no other launch adds them.
// Wave w regenerates rows m0..m0+7 of the down matrices of slots 2(w/2) and 2(w/2)+1
// (A rows 0-7 and 8-15) over K half w % 2, which is the K split, segment order and MFMA
// sequence of k_mfma_one's down for every row.  The activation rows (the slots' h rows)
// sit in LDS; B column n is slot n's row, so D[(slot s, row), s] is that row's product.
// The epilogue forms each slot's output as k_mfma_one does (the two K halves, then the
// router weight) and adds them in slot order from slot 0, as k_combine does, so y is bit
// for bit the three-launch result.  Lanes of a missing slot (s >= top_k) or an invalid
// id regenerate zero weights and their slots are not added.  Dynamic LDS: top_k K bf16.
template <int P, bool VEC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_down_one(const MfmaArgs a) {
    constexpr int KS = 2;
    __shared__ f32x4 red[8][64];
    __shared__ uint32_t tab[512];
    extern __shared__ uint4 xs[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int r = lane & 15;
    const int kk = a.top_k;
    const int slot = 2 * (wave >> 1) + (r >> 3);   // this lane's A row: slot, row m0 + (r & 7)
    const int m0 = blockIdx.x * 8;
    const int nk = a.K / 8;                        // 16-byte pieces of one h row
    const int np = kk * nk;                        // h rows of the slots are consecutive
    const uint4* src = (const uint4*)a.x;
    uint4 x0 = {0u, 0u, 0u, 0u};
    if (tid < np) x0 = src[tid];
    const int e = slot < kk ? a.ids[slot] : -1;
    const bool serve = e >= 0 && e < a.E;
    Lane L;
    L.tab = tab;
    L.ks = wave % KS;
    L.q = lane >> 4;
    L.nbpr = nk;
    const int64_t nblk = (int64_t)a.M * L.nbpr;
    // a lane without an expert reads expert 0's stacked streams (or cache slot 0's, which
    // is where the stream pointers point): in range, and its weights are zeroed anyway
    L.W = serve ? mat_of(a.A, e, nblk, P, 0, true, nullptr, a.slot, a.slot_stride)
                : mat_of(a.A, 0, nblk, P, 0, true);
    const int row = m0 + (r & 7);
    L.rv = serve && row < a.M;
    L.rowb = (int64_t)(row < a.M ? row : a.M - 1) * L.nbpr;
    L.nseg = (L.nbpr + 7) / 8;
    L.n_it = (L.nseg + KS * 4 - 1) / (KS * 4);
    const Seg<P, VEC> first = first_seg<P, VEC, KS>(L);
    tab[tid] = lfsr_next32(tid < 256 ? (uint32_t)tid : (uint32_t)(tid - 256) << 8);   // 512 threads
    if (tid < np) xs[tid] = x0;
    for (int i = tid + 512; i < np; i += 512) xs[i] = src[i];
    __syncthreads();   // publishes the tables and the h rows

    const uint16_t* xrow = (const uint16_t*)xs + (int64_t)min(r, kk - 1) * a.K;   // B column r
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_k_loop<P, VEC, 1, KS, true, true, true>(L, nullptr, &acc, xrow, &first);
    red[wave][lane] = acc;
    __syncthreads();
    if (tid < 8 && m0 + tid < a.M) {
#pragma clang fp contract(off)
        float yv = 0.f;
        for (int s2 = 0; s2 < kk; ++s2) {
            const int ar = 8 * (s2 & 1) + tid;          // A row of (slot s2, row m0 + tid)
            const int dl = s2 + 16 * (ar >> 2);          // lane holding D[ar][s2]
            const int w0 = 2 * (s2 >> 1);
            // no contraction into an fma here: the three-launch path stores each slot
            // output (rounded product) before the combine adds it
            const float v = red[w0][dl][ar & 3] + red[w0 + 1][dl][ar & 3];
            const float o = a.topk_w[s2] * v;
            yv = s2 == 0 ? o : yv + o;
        }
        a.y[m0 + tid] = yv;
    }
}

// ----------------------------------------------------------------------------------
// Wide-token products (prefill and long token lists), vector-load layouts only
// (K % 256 == 0, 16-byte aligned streams).  A workgroup of 16 waves owns AR = 128 weight
// rows (64 rows of gate and of up, or 128 rows of one matrix) for up to NC = 384 tokens,
// so each weight block is regenerated once per pass over its expert's tokens.  It walks
// K in 64-k steps, one barrier per step.  The waves split by role, two of each role on
// every SIMD, so that each SIMD always has regeneration work and matrix work queued (on
// gfx950 its vector ALU and matrix core measured no overlap in time, so a step costs
// about the sum of the two; the split keeps either unit from waiting on the other's
// latencies):
//   - producers (waves 0-7) regenerate the next step's A tile (two blocks per lane) and
//     stage its B tile (the step's 128-byte slice of every token row), both in LDS;
//   - consumers (waves 8-15), wave (row half rh, token quarter tq), multiply their two
//     32-row A tiles (gate and up rows of one half, or two row tiles) with three
//     32-token B tiles on v_mfma_f32_32x32x16_bf16 (four k16 slices per step),
//     accumulators in registers, and write the results.
// LDS tiles are stored per k16 slice ([slice][row or token][2 blocks][8 bf16]) so every
// MFMA fragment is one contiguous 1 KB read.  A and B are double-buffered: the producers
// fill step s+1 while the consumers multiply step s.  A producer stores step s+1's B
// slice (loaded during step s-1) first, then issues step s+2's B loads, regenerates step
// s+1's blocks and reads its stream values for step s+2.  Each B load instruction covers
// whole 128-byte lines: 8 tokens x 8 pieces.
// The seed / coefficient / code streams of each 32-block group (four steps) are staged
// in LDS with 16-byte loads, one buffer: a row's chunks are written and read by four
// lanes of one wave, so same-wave LDS order puts the group's stores after the previous
// group's last reads and before its own first (no barrier needed).
// Lane l of producer wave w takes row 16 w + (l & 15) and blocks l >> 4 and 4 + (l >> 4)
// of each step, so each 16-lane group of an A store writes 256 contiguous bytes.
// Workgroups are numbered so that every row group of one expert lands on the same XCD
// (workgroups are dealt to the 8 XCDs round-robin), keeping that expert's token rows in
// one L2.
// ----------------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int P, int MODE>
__global__ __launch_bounds__(1024, 1) void k_wide(const MfmaArgs a) {
    constexpr int NMAT = MODE == MODE_GATEUP ? 2 : 1;
    constexpr int AR = 128;                   // A rows per workgroup
    constexpr int RM = AR / NMAT;             // rows per matrix
    constexpr int NTW = 3;                    // 32-token tiles per consumer wave
    constexpr int NC = 4 * NTW * 32;          // token slots per pass (384)
    constexpr int NQ = 4;                     // k16 slices per 64-k step
    constexpr int NBU = NC * 8 / 512;         // B pieces per producer lane and step (6)
    constexpr int SROW = 40;                  // staged stream row stride in u16 (80 B: the
                                              // 16 rows a lane group reads start in distinct banks)
    __shared__ u32x4 As[2][NQ * AR * 2];
    __shared__ u32x4 Bs[2][NQ * NC * 2];
    __shared__ uint16_t Ss[AR * SROW];
    __shared__ uint16_t Cs[AR * SROW + 8];
    __shared__ uint8_t Ds[AR * 16];
    __shared__ uint32_t tab[512];
    fill_lfsr_tables(tab);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const bool producer = wave < 8;           // wave-uniform

    // ---- XCD-aware numbering: consecutive work items share an XCD ------------------
    const int total = gridDim.x * gridDim.y;
    const int L = blockIdx.y * gridDim.x + blockIdx.x;
    const int xcd = L & 7, slot = L >> 3, q8 = total >> 3, r8 = total & 7;
    const int work = xcd * q8 + min(xcd, r8) + slot;
    const int rg = work % gridDim.x;          // row group
    const int target = work / gridDim.x;      // active-expert index

    // ---- expert ------------------------------------------------------------------
    int e = 0, n_e = a.N;
    const int32_t* list = nullptr;
    if constexpr (MODE != MODE_GEMM) {
        const int ehi = a.e_hi > 0 ? a.e_hi : a.E;
        int found = -1, cum = 0;
        for (int base = a.e_lo; base < ehi && found < 0; base += 64) {
            const int idx = base + lane;
            const bool act = idx < ehi && a.counts[idx] > 0 &&
                             (!a.p4mask || p4_of(a.p4mask, idx) == (P == 4));
            const uint64_t bal = __ballot(act);
            const int c = __popcll(bal);
            if (target < cum + c) {
                const int k = target - cum;
                const uint64_t below = lane ? (bal & ((~0ull) >> (64 - lane))) : 0ull;
                const bool mine = act && __popcll(below) == k;
                found = base + __ffsll((long long)__ballot(mine)) - 1;
            }
            cum += c;
        }
        if (found < 0) return;
        e = found;
        n_e = a.counts[e];
        list = a.lists + (int64_t)e * a.T;
    }
    if (n_e <= 0) return;

    const int M = a.M, K = a.K, nbpr = K / 8;
    const int64_t nblk = (int64_t)M * nbpr;
    const int m0 = rg * RM;
    const int ngroups = nbpr / 32;            // K % 256 == 0
    const int NS = ngroups * 4;               // 64-k steps

    if (producer) {
        // ---- producer: A row r (matrix dmat, row drow), blocks dj and 4 + dj ----------
        const int dj = lane >> 4;
        const int r = 16 * wave + (lane & 15);
        const int dmat = r / RM, drow = r % RM;
        Mat W = mat_of(a.A, e, nblk, P, a.exp_bias, MODE != MODE_GEMM, a.p4mask, a.slot, a.slot_stride);
        if constexpr (NMAT == 2) {
            if (dmat == 1) W = mat_of(a.A2, e, nblk, P, 0, true, a.p4mask, a.slot, a.slot_stride);
        }
        const bool drv = m0 + drow < M;
        const int64_t drowb = (int64_t)(drv ? m0 + drow : M - 1) * nbpr;
        // LDS tile layout [k16 slice][32-row group][block in slice][32 rows]: a half-wave's
        // fragment read is 512 contiguous bytes (no bank conflicts).  Block dj of a step
        // lies in slice dj >> 1, block 4 + dj in slice 2 + (dj >> 1).
        const int a_slot = ((dj >> 1) * AR + (r & ~31)) * 2 + (dj & 1) * 32 + (r & 31);
        constexpr int A_HI = 2 * AR * 2;      // offset of slices 2, 3

        u32x4 sreg_s, sreg_c, sreg_d;
        auto stream_load = [&](int g) {
            const int64_t b0 = drowb + 32 * g;    // first block of the group in this row
            sreg_s = *reinterpret_cast<const u32x4*>(W.seeds + b0 + 8 * dj);
            if (dj < P) sreg_c = *reinterpret_cast<const u32x4*>(W.coefs + (b0 * P) / 4 + 8 * dj);
            if (dj == 0) sreg_d = *reinterpret_cast<const u32x4*>(W.codes + b0 / 2);
        };
        auto stream_store = [&]() {
            *reinterpret_cast<u32x4*>(&Ss[r * SROW + 8 * dj]) = sreg_s;
            // missing rows get zero coefficients (zero weights); applied here, not at the
            // load, so the load is not waited for early
            if (dj < P)
                *reinterpret_cast<u32x4*>(&Cs[r * SROW + 8 * dj]) =
                    drv ? sreg_c : u32x4{0u, 0u, 0u, 0u};
            if (dj == 0) *reinterpret_cast<u32x4*>(&Ds[r * 16]) = sreg_d;
        };
        struct Blk { uint32_t seed, cw, code; };
        auto fetch1 = [&](int bl) {           // block bl (0..31) of the staged group
            Blk k;
            k.seed = Ss[r * SROW + bl];
            if constexpr (P == 4) {
                k.cw = Cs[r * SROW + bl];
            } else {
                const int n = 3 * bl, sh = 4 * (n & 3);
                const uint16_t* c = &Cs[r * SROW + (n >> 2)];
                k.cw = ((uint32_t)c[0] | ((uint32_t)c[1] << 16)) >> sh;
            }
            k.code = ((uint32_t)Ds[r * 16 + (bl >> 1)] >> (4 * (bl & 1))) & 0xFu;
            return k;
        };
        auto regen = [&](const Blk& k, u32x4* dst) {
            float w[8];
            decode_block<P>(window_from_tables(k.seed, tab), k.cw, k.code, W.exp_bias, w);
            *dst = __builtin_bit_cast(u32x4, pack_bf16(w));
        };

        for (int pass = 0; pass < n_e; pass += NC) {
            // B staging: instruction u covers token slots 8 (wave + 8 u) .. +7 (lane & 7),
            // 16-byte piece p = lane >> 3 of each token's 128-byte slice
            const int p = lane >> 3;
            const uint16_t* brow[NBU];
#pragma unroll
            for (int u = 0; u < NBU; ++u) {
                const int ts = 8 * (wave + 8 * u) + (lane & 7);
                const int i = min(pass + ts, n_e - 1);
                int64_t src;
                if constexpr (MODE == MODE_GEMM) src = i;
                else if constexpr (MODE == MODE_GATEUP) src = list[i] / a.top_k;
                else src = list[i];
                brow[u] = a.x + src * a.ldx + 8 * p;
            }
            // slot of piece p of token ts: slice p >> 1, block p & 1
            auto bslot = [&](int u) {
                const int ts = 8 * (wave + 8 * u) + (lane & 7);
                return ((p >> 1) * NC + (ts & ~31)) * 2 + (p & 1) * 32 + (ts & 31);
            };

            // prologue: group 0 staged and group 1 in registers; step 0's weights and B
            // slice in buffer 0; step 1's B slice in registers; step 1's stream values read
            stream_load(0);
            stream_store();
            if (ngroups > 1) stream_load(1);
            u32x4 breg[NBU];
#pragma unroll
            for (int u = 0; u < NBU; ++u) breg[u] = *reinterpret_cast<const u32x4*>(brow[u]);
            Blk c0 = fetch1(dj), c1 = fetch1(4 + dj);
            regen(c0, &As[0][a_slot]);
            regen(c1, &As[0][A_HI + a_slot]);
#pragma unroll
            for (int u = 0; u < NBU; ++u) Bs[0][bslot(u)] = breg[u];
#pragma unroll
            for (int u = 0; u < NBU; ++u) breg[u] = *reinterpret_cast<const u32x4*>(brow[u] + 64);
            Blk n0 = fetch1(8 + dj), n1 = fetch1(12 + dj);
            __syncthreads();

            // step s: step s+1's B slice and weights into buffer s&1^1, step s+2's B loads,
            // and step s+2's stream values (staging its group first when it opens one).
            // Indices past the last step are clamped; those writes land in buffers nobody
            // reads.
            // The producers leave each barrier together; their B loads are spread over
            // the step (half before each block) so the vector-memory queue drains while
            // the vector ALU decodes, instead of stalling every producer at once.
            for (int s = 0; s < NS; ++s) {
                const int nb = (s & 1) ^ 1;
                const int sn = min(s + 2, NS - 1);
#pragma unroll
                for (int u = 0; u < NBU / 2; ++u) {
                    Bs[nb][bslot(u)] = breg[u];
                    breg[u] = *reinterpret_cast<const u32x4*>(brow[u] + 64 * sn);
                }
                __builtin_amdgcn_sched_barrier(0);
                regen(n0, &As[nb][a_slot]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = NBU / 2; u < NBU; ++u) {
                    Bs[nb][bslot(u)] = breg[u];
                    breg[u] = *reinterpret_cast<const u32x4*>(brow[u] + 64 * sn);
                }
                __builtin_amdgcn_sched_barrier(0);
                regen(n1, &As[nb][A_HI + a_slot]);
                if (((s + 2) & 3) == 0 && s + 2 < NS) {
                    const int g2 = (s + 2) >> 2;
                    stream_store();           // after the last reads of group g2 - 1
                    if (g2 + 1 < ngroups) stream_load(g2 + 1);
                }
                const int bl = 8 * (sn & 3) + dj;
                n0 = fetch1(bl);
                n1 = fetch1(bl + 4);
                __syncthreads();
            }
            __syncthreads();   // LDS buffers are reused by the next pass
        }
    } else {
        // ---- consumer: wave (rh, tq) --------------------------------------------------
        const int rh = (wave - 8) >> 2, tq = (wave - 8) & 3;
        // its two A tiles (32 A-rows each): gate and up rows of half rh, or 2rh, 2rh+1
        const int ta0 = NMAT == 2 ? rh : 2 * rh;
        const int ta1 = NMAT == 2 ? 2 + rh : 2 * rh + 1;

        for (int pass = 0; pass < n_e; pass += NC) {
            f32x16 acc[2][NTW];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int t = 0; t < NTW; ++t)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[x][t][v] = 0.f;
            __syncthreads();   // the producers' prologue

            for (int s = 0; s < NS; ++s) {
                const int buf = s & 1;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const bf16x8 A0 = __builtin_bit_cast(bf16x8, As[buf][(q * AR + 32 * ta0) * 2 + lane]);
                    const bf16x8 A1 = __builtin_bit_cast(bf16x8, As[buf][(q * AR + 32 * ta1) * 2 + lane]);
#pragma unroll
                    for (int t = 0; t < NTW; ++t) {
                        const bf16x8 Bf =
                            __builtin_bit_cast(bf16x8, Bs[buf][(q * NC + 32 * (tq * NTW + t)) * 2 + lane]);
                        acc[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, Bf, acc[0][t], 0, 0, 0);
                        acc[1][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, Bf, acc[1][t], 0, 0, 0);
                    }
                }
                // per slice: read A0, A1, B0, B1; two MFMAs on B0 while B2 is read; then
                // the MFMAs on B1 and B2 (one fragment read in flight behind each pair)
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                }
                __syncthreads();
            }

            // ---- epilogue: lane holds, for token slot 96 tq + 32 t + l32, rows
            //      8 g + 4 lh + c (g, c = 0..3) of each of its two 32-row tiles ------------
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
                const int i = pass + 32 * (tq * NTW + t) + l32;
                if (i >= n_e) continue;
                int64_t dst;
                float scale = 1.0f;
                if constexpr (MODE == MODE_GEMM) {
                    dst = i;
                } else {
                    dst = list[i];
                    if constexpr (MODE == MODE_DOWN) scale = a.topk_w[dst];
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if constexpr (MODE == MODE_GATEUP) {
                        const int m = m0 + 32 * rh + 8 * g + 4 * lh;
                        uint16_t hb[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const float gt = acc[0][t][4 * g + c], up = acc[1][t][4 * g + c];
                            hb[c] = __builtin_bit_cast(uint16_t, (__bf16)(gt / (1.0f + expf(-gt)) * up));
                        }
                        uint16_t* dp = a.h + dst * a.ldy + m;
                        if (m + 3 < M && ((uintptr_t)dp & 7) == 0) {
                            *reinterpret_cast<uint2*>(dp) =
                                make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
                        } else {
                            for (int c = 0; c < 4; ++c)
                                if (m + c < M) dp[c] = hb[c];
                        }
                    } else {
#pragma unroll
                        for (int x = 0; x < 2; ++x) {
                            const int m = m0 + 32 * (x == 0 ? ta0 : ta1) + 8 * g + 4 * lh;
                            float* dp = a.y + dst * a.ldy + m;
                            const f32x4 v = {scale * acc[x][t][4 * g + 0], scale * acc[x][t][4 * g + 1],
                                             scale * acc[x][t][4 * g + 2], scale * acc[x][t][4 * g + 3]};
                            if (m + 3 < M && ((uintptr_t)dp & 15) == 0) {
                                *reinterpret_cast<f32x4*>(dp) = v;
                            } else {
                                for (int c = 0; c < 4; ++c)
                                    if (m + c < M) dp[c] = v[c];
                            }
                        }
                    }
                }
            }
            __syncthreads();   // LDS buffers are reused by the next pass
        }
    }
}

// ----------------------------------------------------------------------------------
// MoE dispatch: workgroup e compacts the pairs routed to expert e, in pair order.
// The ids are staged through LDS in tiles of 8192 with coalesced loads; within a tile
// thread t owns the contiguous run [t*R, (t+1)*R): it counts its matches, a workgroup
// prefix sum of the counts (plus the matches of earlier tiles) gives its first output
// slot, and a second pass over the run writes the pair indices.  No atomics: the lists
// are deterministic.  The tile is stored with one padding word per 32 so that the 64
// runs a wave reads at once fall in different banks.
// ----------------------------------------------------------------------------------
// Exclusive prefix of per-thread counts over a 256-thread workgroup (wave shuffles, then
// the four wave totals through LDS); `total` receives the sum.  Contains a barrier.
__device__ __forceinline__ int wg_exclusive_scan(int c, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int excl = incl - c;
    for (int w = 0; w < wave; ++w) excl += wsum[w];
    total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    return excl;
}

constexpr int kDispTile = 8192;

__device__ __forceinline__ int disp_slot(int i) { return i + (i >> 5); }

// One tile of pairs [t0, t0 + n): the pairs routed to expert e, written in pair order from
// list slot `done` on (slots at or past T are dropped: ids repeated within a token).
// Returns the number of matches in the tile.  Uses s_ids and wsum; ends with a barrier.
__device__ __forceinline__ int dispatch_tile(const int32_t* __restrict__ ids, int t0, int n, int e,
                                             int T, int done, int32_t* __restrict__ out,
                                             int32_t* s_ids, int* wsum) {
    const int tid = threadIdx.x;
    {   // all of a thread's loads in flight at once, then the LDS stores
        int32_t v[kDispTile / 256];
#pragma unroll
        for (int k = 0; k < kDispTile / 256; ++k) {
            const int i = tid + 256 * k;
            v[k] = i < n ? ids[t0 + i] : 0;
        }
#pragma unroll
        for (int k = 0; k < kDispTile / 256; ++k) {
            const int i = tid + 256 * k;
            if (i < n) s_ids[disp_slot(i)] = v[k];
        }
    }
    __syncthreads();
    const int R = (n + 255) / 256;
    const int p0 = min(tid * R, n), p1 = min(p0 + R, n);
    int c = 0;
    for (int p = p0; p < p1; ++p) c += s_ids[disp_slot(p)] == e;
    int tile_total;
    int slot = done + wg_exclusive_scan(c, wsum, tile_total);
    if (c > 0) {
        for (int p = p0; p < p1; ++p) {
            if (s_ids[disp_slot(p)] == e) {
                if (slot < T) out[slot] = t0 + p;   // ids repeated within a token: dropped
                ++slot;
            }
        }
    }
    __syncthreads();   // the tile and wsum are reused
    return tile_total;
}

__global__ __launch_bounds__(256) void k_dispatch(const int32_t* __restrict__ ids, int total,
                                                  int T, int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ lists) {
    __shared__ int32_t s_ids[kDispTile + kDispTile / 32];
    __shared__ int wsum[4];
    const int e = blockIdx.x;
    int32_t* out = lists + (int64_t)e * T;
    int done = 0;   // matches in earlier tiles
    for (int t0 = 0; t0 < total; t0 += kDispTile)
        done += dispatch_tile(ids, t0, min(kDispTile, total - t0), e, T, done, out, s_ids, wsum);
    if (threadIdx.x == 0) counts[e] = done < T ? done : T;
}

// Many pairs: the same lists from two launches over (expert, tile) workgroups, so the
// tiles of one expert run side by side.  First each workgroup counts its expert's pairs
// in its tile (cc[tile][e]); then each writes them from the slot that the earlier tiles'
// counts give, and the last tile writes the expert's count.
__global__ __launch_bounds__(256) void k_dispatch_count(const int32_t* __restrict__ ids, int total,
                                                        int E, int32_t* __restrict__ cc) {
    __shared__ int wsum[4];
    const int e = blockIdx.x, tile = blockIdx.y, tid = threadIdx.x;
    const int t0 = tile * kDispTile, n = min(kDispTile, total - t0);
    int c = 0;
#pragma unroll 4
    for (int i = tid; i < n; i += 256) c += ids[t0 + i] == e;
    int tile_total;
    (void)wg_exclusive_scan(c, wsum, tile_total);
    if (tid == 0) cc[(int64_t)tile * E + e] = tile_total;
}

__global__ __launch_bounds__(256) void k_dispatch_scatter(const int32_t* __restrict__ ids, int total,
                                                          int T, int E,
                                                          const int32_t* __restrict__ cc,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ lists) {
    __shared__ int32_t s_ids[kDispTile + kDispTile / 32];
    __shared__ int wsum[4];
    const int e = blockIdx.x, tile = blockIdx.y;
    int done = 0;
    for (int t = 0; t < tile; ++t) done += cc[(int64_t)t * E + e];
    const int t0 = tile * kDispTile;
    const int got = dispatch_tile(ids, t0, min(kDispTile, total - t0), e, T, done,
                                  lists + (int64_t)e * T, s_ids, wsum);
    if (tile == (int)gridDim.y - 1 && threadIdx.x == 0) {
        const int all = done + got;
        counts[e] = all < T ? all : T;
    }
}

// y[n][0..M) = 0 for the N rows of a strided fp32 matrix (nm = N * M elements).
__global__ __launch_bounds__(256) void k_zero_rows(float* __restrict__ y, int ldy, int M,
                                                   int64_t nm) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nm) return;
    y[(i / M) * ldy + i % M] = 0.0f;
}

// y[t][:] = sum_s o[t*top_k + s][:], slot order fixed.  KMAX > 0: top_k <= KMAX, and all
// of a thread's slot loads are issued before the first add (the adds keep slot order).
template <int KMAX>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ o, int top_k,
                                                 float* __restrict__ y, int H, int T) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index
    const int h4 = H / 4;
    if (idx >= (int64_t)T * h4) return;
    const int64_t t = idx / h4, c = idx % h4;
    const float4* src = reinterpret_cast<const float4*>(o) + (t * top_k) * h4 + c;
    float4 s;
    if constexpr (KMAX > 0) {
        float4 v[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < top_k) v[k] = src[(int64_t)k * h4];
        s = v[0];
#pragma unroll
        for (int k = 1; k < KMAX; ++k) {
            if (k < top_k) {
                s.x += v[k].x; s.y += v[k].y; s.z += v[k].z; s.w += v[k].w;
            }
        }
    } else {
        s = src[0];
        for (int k = 1; k < top_k; ++k) {
            const float4 v = src[(int64_t)k * h4];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
    }
    reinterpret_cast<float4*>(y)[idx] = s;
}

}  // namespace seedmm

// ==================================================================================
// Host side: validation, path selection, launches.
// ==================================================================================
using namespace seedmm;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_shape(int M, int K, int P) {
    return M >= 0 && K >= 0 && K % 8 == 0 && (P == 3 || P == 4);
}

bool valid_bias(int32_t eb) { return eb >= -100 && eb <= 100; }

// Vector-load path: every row starts a whole segment and every base is 16-byte aligned.
bool use_vec(const void* seeds, const void* coefs, const void* codes, int K) {
    return K % 64 == 0 && aligned16(seeds) && aligned16(coefs) && aligned16(codes);
}

int launch_status() {
    return hipGetLastError() == hipSuccess ? SEEDMM_OK : SEEDMM_EHIP;
}

template <int P, bool VEC, int NTOK>
void launch_gemv_f32(const uint16_t* s, const uint16_t* c, const uint8_t* d, int eb,
                     const float* x, int ldx, float* y, int ldy, int M, int K, int N,
                     hipStream_t st) {
    dim3 grid((M + 15) / 16, (N + NTOK - 1) / NTOK);
    hipLaunchKernelGGL((k_gemv_f32<P, VEC, NTOK>), grid, dim3(256), 0, st, s, c, d, eb, x, ldx,
                       y, ldy, M, K, N);
}

constexpr int kGridYMax = 65535;   // workgroup rows of one launch along y

template <int P>
void gemv_f32(const uint16_t* s, const uint16_t* c, const uint8_t* d, int eb, const float* x,
              int ldx, float* y, int ldy, int M, int K, int N, hipStream_t st) {
    const bool vec = use_vec(s, c, d, K);
    if (N <= 1) {
        if (vec) launch_gemv_f32<P, true, 1>(s, c, d, eb, x, ldx, y, ldy, M, K, N, st);
        else launch_gemv_f32<P, false, 1>(s, c, d, eb, x, ldx, y, ldy, M, K, N, st);
        return;
    }
    // 4 rows of X per workgroup row: larger N runs as several launches of whole chunks
    constexpr int kChunk = kGridYMax * 4;
    for (int n0 = 0; n0 < N; n0 += kChunk) {
        const int n = N - n0 < kChunk ? N - n0 : kChunk;
        const float* xc = x + (int64_t)n0 * ldx;
        float* yc = y + (int64_t)n0 * ldy;
        if (vec) launch_gemv_f32<P, true, 4>(s, c, d, eb, xc, ldx, yc, ldy, M, K, n, st);
        else launch_gemv_f32<P, false, 4>(s, c, d, eb, xc, ldx, yc, ldy, M, K, n, st);
    }
}

// Decode shape: 4 waves split K, up to 64 tokens per pass.  Prefill shape: 4 waves on
// 4 row tiles, up to 256 tokens per pass.
constexpr int kOneMaxK = 16384;   // one-token kernel: activation row of at most 32 KB in LDS

template <int P, bool VEC, int MODE>
void launch_mfma(const MfmaArgs& a, bool prefill, int gridy, hipStream_t st) {
    if (prefill && VEC && a.K % 256 == 0) {
        constexpr int RM = MODE == MODE_GATEUP ? 64 : 128;
        dim3 grid((a.M + RM - 1) / RM, gridy);
        hipLaunchKernelGGL((k_wide<P, MODE>), grid, dim3(1024), 0, st, a);
    } else {
        // down and the plain product: two 16-row tiles per workgroup, K in halves
        constexpr int RT = MODE == MODE_GATEUP ? 1 : 2;
        dim3 grid((a.M + 16 * RT - 1) / (16 * RT), gridy);
        if constexpr (MODE != MODE_GEMM) {
            if (a.ids && a.K <= kOneMaxK) {
                hipLaunchKernelGGL((k_mfma_one<P, VEC, MODE, RT>), grid, dim3(256),
                                   (size_t)a.K * 2, st, a);
                return;
            }
        }
        hipLaunchKernelGGL((k_mfma<P, VEC, 4, MODE, true, RT>), grid, dim3(256), 0, st, a);
    }
}

// One token, uniform P: down and the combine in one launch (k_down_one) when the slots'
// h rows fit its LDS budget.
constexpr int kDownOneMaxLds = 65536;

bool down_one_fits(int top_k, int K) {
    return top_k >= 2 && top_k <= 8 && (int64_t)top_k * K * 2 <= kDownOneMaxLds;
}

template <int P>
void launch_down_one(const MfmaArgs& b, hipStream_t st) {
    const dim3 grid((unsigned)((b.M + 7) / 8));
    hipLaunchKernelGGL((k_down_one<P, true>), grid, dim3(512), (size_t)b.top_k * b.K * 2, st, b);
}

// The caller's second stream and its fork / join events (seedmm_side), or all null.
struct Side {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool on() const { return s != nullptr; }
    // hip_stream's work so far becomes a dependency of the side stream's next launches
    bool fork_from(hipStream_t st) const {
        return hipEventRecord(fork, st) == hipSuccess && hipStreamWaitEvent(s, fork, 0) == hipSuccess;
    }
    // hip_stream's later work waits for everything launched on the side stream
    bool join_into(hipStream_t st) const {
        return hipEventRecord(join, s) == hipSuccess && hipStreamWaitEvent(st, join, 0) == hipSuccess;
    }
};

// P = 3 or 4, or P = 0 for mixed packs (a.p4mask): then one launch per P, each serving
// only the experts of its own P.  The two write disjoint rows (an expert's pairs belong
// to one P), so with a side stream the P = 3 launch runs there, forked from and joined
// back into `st` with the caller's events (which graph capture records as dependencies):
// the two grids share the chip instead of each leaving it part empty at its tail.
// Returns false only when the join back into `st` could not be recorded (the caller's
// later work would not wait for the side stream's launch).
template <int MODE>
bool mfma_dispatch(int P, bool vec, const MfmaArgs& a, bool prefill, int gridy, hipStream_t st,
                   const Side& side = Side()) {
    auto run = [&](int p, hipStream_t s) {
        if (p == 4) {
            if (vec) launch_mfma<4, true, MODE>(a, prefill, gridy, s);
            else launch_mfma<4, false, MODE>(a, prefill, gridy, s);
        } else {
            if (vec) launch_mfma<3, true, MODE>(a, prefill, gridy, s);
            else launch_mfma<3, false, MODE>(a, prefill, gridy, s);
        }
    };
    if (P != 0) {
        run(P, st);
        return true;
    }
    if (!side.on() || !side.fork_from(st)) {
        run(4, st);
        run(3, st);
        return true;
    }
    run(3, side.s);
    run(4, st);
    return side.join_into(st);
}

// Split point of a multi-token call: experts e < E * kSplitNum / kSplitDen on the caller's
// stream (an even split measured best, decode and prefill).
constexpr int kSplitNum = 1, kSplitDen = 2;

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct MoeLayout {
    size_t counts, lists, h, o, cc, total;
};

int dispatch_tiles(int64_t pairs) { return (int)((pairs + kDispTile - 1) / kDispTile); }

// Pair indices t * top_k + slot are int32 in the lists and the kernels.
constexpr int64_t kMaxPairs = 0x7FFFFFFF;

bool moe_layout(int T, int top_k, int E, int H, int I, MoeLayout* L) {
    if (T < 0 || top_k < 1 || E < 1 || H < 0 || I < 0) return false;
    if ((int64_t)T * top_k > kMaxPairs) return false;
    const size_t pairs = (size_t)T * top_k;
    L->counts = 0;
    L->lists = L->counts + align_up(sizeof(int32_t) * (size_t)E);
    L->h = L->lists + align_up(sizeof(int32_t) * (size_t)E * (size_t)T);
    L->o = L->h + align_up(sizeof(uint16_t) * pairs * (size_t)I);
    L->cc = L->o + align_up(sizeof(float) * pairs * (size_t)H);
    const int tiles = dispatch_tiles((int64_t)pairs);
    L->total = L->cc + (tiles > 1 ? align_up(sizeof(int32_t) * (size_t)tiles * (size_t)E) : 0);
    return true;
}

}  // namespace

extern "C" {

int seedmm_version(void) { return 200; }

const char* seedmm_strerror(int status) {
    switch (status) {
        case SEEDMM_OK: return "ok";
        case SEEDMM_EINVAL: return "invalid argument";
        case SEEDMM_EALIGN: return "misaligned pointer or leading dimension";
        case SEEDMM_EWORKSPACE: return "workspace missing or too small";
        case SEEDMM_EHIP: return "HIP launch failure";
        case SEEDMM_ECAPACITY: return "more distinct experts in one call than cache slots";
        case SEEDMM_ESCRATCH: return "batch needs more scratch than the static buffer of seedmm_moe_noalloc";
        default: return "unknown status";
    }
}

int seedmm_gemv_ex(const uint16_t* seeds, const uint16_t* coefs, const uint8_t* codes,
                   int32_t exp_bias, const void* x, int x_dtype, int ldx, float* y, int ldy,
                   int M, int K, int P, int N, void* hip_stream) {
    if (!valid_shape(M, K, P) || !valid_bias(exp_bias) || N < 0 || ldx < K || ldy < M)
        return SEEDMM_EINVAL;
    if (x_dtype != SEEDMM_F32 && x_dtype != SEEDMM_BF16) return SEEDMM_EINVAL;
    if (M == 0 || N == 0) return SEEDMM_OK;
    if (!seeds || !coefs || !codes || !x || !y) return SEEDMM_EINVAL;
    if (!aligned16(x)) return SEEDMM_EALIGN;
    hipStream_t st = (hipStream_t)hip_stream;
    if (K == 0) {   // empty product: y = 0 (a kernel, not a memset node, under capture)
        const int64_t n = (int64_t)N * M;
        hipLaunchKernelGGL(k_zero_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, y,
                           ldy, M, n);
        return launch_status();
    }
    if (x_dtype == SEEDMM_F32) {
        if (ldx % 4 != 0) return SEEDMM_EALIGN;
        if (P == 4) gemv_f32<4>(seeds, coefs, codes, exp_bias, (const float*)x, ldx, y, ldy, M, K, N, st);
        else gemv_f32<3>(seeds, coefs, codes, exp_bias, (const float*)x, ldx, y, ldy, M, K, N, st);
        return launch_status();
    }
    if (ldx % 8 != 0) return SEEDMM_EALIGN;
    MfmaArgs a = {};
    a.A.seeds = seeds; a.A.coefs = coefs; a.A.codes = codes; a.A.exp_bias = nullptr;
    a.exp_bias = exp_bias;
    a.M = M; a.K = K;
    a.x = (const uint16_t*)x; a.ldx = ldx; a.N = N;
    a.y = y; a.ldy = ldy;
    const bool vec = use_vec(seeds, coefs, codes, K);
    mfma_dispatch<MODE_GEMM>(P, vec, a, N > 64, 1, st);
    return launch_status();
}

int seedmm_gemv(const uint16_t* seeds, const uint16_t* coefs, const uint8_t* codes,
                int32_t exp_bias, const float* x, float* y, int M, int K, int P) {
    return seedmm_gemv_ex(seeds, coefs, codes, exp_bias, x, SEEDMM_F32, K < 4 ? 4 : K, y,
                          M, M, K, P, 1, nullptr);
}

int seedmm_reconstruct(const uint16_t* seeds, const uint16_t* coefs, const uint8_t* codes,
                       int32_t exp_bias, void* W, int w_dtype, int M, int K, int P,
                       void* hip_stream) {
    if (!valid_shape(M, K, P) || !valid_bias(exp_bias)) return SEEDMM_EINVAL;
    if (w_dtype != SEEDMM_F32 && w_dtype != SEEDMM_BF16) return SEEDMM_EINVAL;
    const int64_t nblk = (int64_t)M * (K / 8);
    if (nblk == 0) return SEEDMM_OK;
    if (!seeds || !coefs || !codes || !W) return SEEDMM_EINVAL;
    if (!aligned16(W)) return SEEDMM_EALIGN;
    hipStream_t st = (hipStream_t)hip_stream;
    dim3 grid((unsigned)((nblk + 255) / 256));
    if (P == 4) {
        if (w_dtype == SEEDMM_BF16)
            hipLaunchKernelGGL((k_reconstruct<4, true>), grid, dim3(256), 0, st, seeds, coefs, codes, exp_bias, W, K, nblk);
        else
            hipLaunchKernelGGL((k_reconstruct<4, false>), grid, dim3(256), 0, st, seeds, coefs, codes, exp_bias, W, K, nblk);
    } else {
        if (w_dtype == SEEDMM_BF16)
            hipLaunchKernelGGL((k_reconstruct<3, true>), grid, dim3(256), 0, st, seeds, coefs, codes, exp_bias, W, K, nblk);
        else
            hipLaunchKernelGGL((k_reconstruct<3, false>), grid, dim3(256), 0, st, seeds, coefs, codes, exp_bias, W, K, nblk);
    }
    return launch_status();
}

int seedmm_moe_dispatch(const int32_t* topk_ids, int T, int top_k, int E, int32_t* counts,
                        int32_t* lists, void* hip_stream) {
    if (T < 0 || top_k < 1 || E < 1 || (int64_t)T * top_k > kMaxPairs) return SEEDMM_EINVAL;
    if (!counts || !lists || (T > 0 && !topk_ids)) return SEEDMM_EINVAL;
    hipLaunchKernelGGL(k_dispatch, dim3(E), dim3(256), 0, (hipStream_t)hip_stream, topk_ids,
                       T * top_k, T, counts, lists);
    return launch_status();
}

size_t seedmm_moe_workspace_bytes(int T, int top_k, int E, int H, int I) {
    MoeLayout L;
    if (!moe_layout(T, top_k, E, H, I, &L)) return 0;
    return L.total;
}

}  // extern "C"

namespace seedmm_layer {

int moe_run(const int32_t* topk_ids, const float* topk_w, int T, int top_k, const void* x,
            float* y, int E, int H, int I, int P, const uint32_t* p4mask, seedmm_mat gate,
            seedmm_mat up, seedmm_mat down, void* workspace, size_t workspace_bytes,
            void* hip_stream, void* const* events, const int32_t* slot, int64_t slot_stride,
            const seedmm_side* side) {
    if (T < 0 || E < 1 || E > 4096 || top_k < 1 || top_k > E || top_k > 64) return SEEDMM_EINVAL;
    if ((int64_t)T * top_k > kMaxPairs) return SEEDMM_EINVAL;
    if (H <= 0 || I <= 0 || H % 8 != 0 || I % 8 != 0) return SEEDMM_EINVAL;
    if (P == 0 ? !p4mask : (P != 3 && P != 4)) return SEEDMM_EINVAL;
    const int64_t nblk = (int64_t)I * (H / 8);   // blocks of one gate/up/down matrix
    if (P == 0 ? nblk % 4 != 0 : ((nblk * P) % 4 != 0 || nblk % 2 != 0)) return SEEDMM_EINVAL;
    if (T == 0) return SEEDMM_OK;
    const seedmm_mat* mats[3] = {&gate, &up, &down};
    for (const seedmm_mat* m : mats)
        if (!m->seeds || !m->coefs || !m->codes || !m->exp_bias) return SEEDMM_EINVAL;
    if (!topk_ids || !topk_w || !x || !y) return SEEDMM_EINVAL;
    if (!aligned16(x) || !aligned16(y)) return SEEDMM_EALIGN;
    MoeLayout L;
    if (!moe_layout(T, top_k, E, H, I, &L)) return SEEDMM_EINVAL;
    if (!workspace || workspace_bytes < L.total) return SEEDMM_EWORKSPACE;
    if (!aligned16(workspace)) return SEEDMM_EALIGN;
    hipStream_t st = (hipStream_t)hip_stream;
    Side sd;
    if (side && side->stream) {
        if (!side->fork || !side->join || side->stream == hip_stream) return SEEDMM_EINVAL;
        sd.s = (hipStream_t)side->stream;
        sd.fork = (hipEvent_t)side->fork;
        sd.join = (hipEvent_t)side->join;
    }
    char* ws = (char*)workspace;
    int32_t* counts = (int32_t*)(ws + L.counts);
    int32_t* lists = (int32_t*)(ws + L.lists);
    uint16_t* hbuf = (uint16_t*)(ws + L.h);
    float* obuf = (float*)(ws + L.o);

    auto mark = [&](int i) {
        if (events && events[i]) (void)hipEventRecord((hipEvent_t)events[i], st);
    };
    // one token: the expert kernels read its top_k ids directly (no dispatch)
    const bool one = T == 1;
    mark(0);
    if (!one) {
        const int tiles = dispatch_tiles((int64_t)T * top_k);
        if (tiles > 1) {
            int32_t* cc = (int32_t*)(ws + L.cc);
            hipLaunchKernelGGL(k_dispatch_count, dim3(E, tiles), dim3(256), 0, st, topk_ids,
                               T * top_k, E, cc);
            hipLaunchKernelGGL(k_dispatch_scatter, dim3(E, tiles), dim3(256), 0, st, topk_ids,
                               T * top_k, T, E, (const int32_t*)cc, counts, lists);
        } else {
            hipLaunchKernelGGL(k_dispatch, dim3(E), dim3(256), 0, st, topk_ids, T * top_k, T,
                               counts, lists);
        }
    }
    mark(1);

    const int pairs = T * top_k;
    const int gridy = one ? top_k : (pairs < E ? pairs : E);   // workgroup rows
    const bool prefill = (int64_t)pairs >= 64LL * E;  // >= 64 tokens per expert on average
    bool vec = true;
    for (const seedmm_mat* m : mats) vec = vec && use_vec(m->seeds, m->coefs, m->codes, 64);
    vec = vec && H % 64 == 0 && I % 64 == 0 && (nblk % 32 == 0);

    MfmaArgs a = {};
    a.A = gate; a.A2 = up;
    a.M = I; a.K = H;
    a.x = (const uint16_t*)x; a.ldx = H;
    a.counts = counts; a.lists = lists; a.E = E; a.T = T; a.top_k = top_k;
    a.h = hbuf; a.ldy = I;
    a.ids = one ? topk_ids : nullptr;
    a.p4mask = p4mask;
    a.slot = slot;
    a.slot_stride = slot_stride;

    MfmaArgs b = {};
    b.A = down;
    b.M = H; b.K = I;
    b.x = hbuf; b.ldx = I;
    b.counts = counts; b.lists = lists; b.E = E; b.T = T; b.top_k = top_k;
    // top-1 routing: the per-slot outputs are y itself (the combine of one slot copies it).
    // One token with one P and vector layouts: down adds the slots itself (k_down_one).
    const bool down_one = one && P != 0 && vec && down_one_fits(top_k, I);
    const bool direct = top_k == 1 || down_one;
    b.topk_w = topk_w; b.y = direct ? y : obuf; b.ldy = H;
    b.ids = a.ids;
    b.p4mask = p4mask;
    b.slot = slot;
    b.slot_stride = slot_stride;

    // Several tokens, one P, and a side stream from the caller: the experts below `cut`
    // run their gate/up and down launches on hip_stream, the others on the side stream
    // (forked and joined with the caller's events, which graph capture records as
    // dependencies).  Each launch ends in a partly empty last round of workgroups (for
    // the prefill kernel, one workgroup per CU and ~16 per expert, most of the chip), and
    // down cannot start before gate/up has drained; with two streams the other half's
    // workgroups fill those gaps.  Timed calls (events) keep the single-stream order.
    bool split = false, joined = true;
    if (!one && P != 0 && !events && E >= 2 && sd.on() && sd.fork_from(st)) {
        const int cut = (int)((int64_t)E * kSplitNum / kSplitDen);
        MfmaArgs pa[2] = {a, a}, pb[2] = {b, b};
        int gy[2];
        for (int part = 0; part < 2; ++part) {
            pa[part].e_lo = pb[part].e_lo = part ? cut : 0;
            pa[part].e_hi = pb[part].e_hi = part ? E : cut;
            const int ne = pa[part].e_hi - pa[part].e_lo;
            gy[part] = pairs < ne ? pairs : ne;
        }
        mfma_dispatch<MODE_GATEUP>(P, vec, pa[0], prefill, gy[0], st);
        mfma_dispatch<MODE_GATEUP>(P, vec, pa[1], prefill, gy[1], sd.s);
        mfma_dispatch<MODE_DOWN>(P, vec, pb[0], prefill, gy[0], st);
        mfma_dispatch<MODE_DOWN>(P, vec, pb[1], prefill, gy[1], sd.s);
        joined = sd.join_into(st);
        split = true;
    } else if (!one && P == 0 && !events && sd.on() && sd.fork_from(st)) {
        // mixed packs: each P's gate/up and down on a stream of its own (the P = 4 and
        // P = 3 launches touch disjoint pairs' rows of h and of the slot outputs), with
        // one fork and one join, so neither down launch waits for the other P's gate/up
        mfma_dispatch<MODE_GATEUP>(4, vec, a, prefill, gridy, st);
        mfma_dispatch<MODE_GATEUP>(3, vec, a, prefill, gridy, sd.s);
        mfma_dispatch<MODE_DOWN>(4, vec, b, prefill, gridy, st);
        mfma_dispatch<MODE_DOWN>(3, vec, b, prefill, gridy, sd.s);
        joined = sd.join_into(st);
        split = true;
    }
    if (!split) {
        joined = mfma_dispatch<MODE_GATEUP>(P, vec, a, prefill, gridy, st, events ? Side() : sd);
        mark(2);
        if (down_one) {
            if (P == 4) launch_down_one<4>(b, st);
            else launch_down_one<3>(b, st);
        } else {
            joined = mfma_dispatch<MODE_DOWN>(P, vec, b, prefill, gridy, st, events ? Side() : sd) && joined;
        }
        mark(3);
    }
    // without the join the combine could read outputs still being written: report it
    if (!joined) return SEEDMM_EHIP;

    if (!direct) {
        const int64_t n4 = (int64_t)T * (H / 4);
        const dim3 cg((unsigned)((n4 + 255) / 256));
        if (top_k <= 8)
            hipLaunchKernelGGL(k_combine<8>, cg, dim3(256), 0, st, obuf, top_k, y, H, T);
        else
            hipLaunchKernelGGL(k_combine<0>, cg, dim3(256), 0, st, obuf, top_k, y, H, T);
    }
    mark(4);
    return launch_status();
}

}  // namespace seedmm_layer

using seedmm_layer::moe_run;

extern "C" {

int seedmm_moe_timed(const int32_t* topk_ids, const float* topk_w, int T, int top_k,
                     const void* x, float* y, int E, int H, int I, int P, seedmm_mat gate,
                     seedmm_mat up, seedmm_mat down, void* workspace, size_t workspace_bytes,
                     void* hip_stream, void* const* events) {
    if (P != 3 && P != 4) return SEEDMM_EINVAL;
    return moe_run(topk_ids, topk_w, T, top_k, x, y, E, H, I, P, nullptr, gate, up, down,
                   workspace, workspace_bytes, hip_stream, events, nullptr, 0, nullptr);
}

int seedmm_moe_ex(const int32_t* topk_ids, const float* topk_w, int T, int top_k, const void* x,
                  float* y, int E, int H, int I, int P, const uint32_t* p4mask, seedmm_mat gate,
                  seedmm_mat up, seedmm_mat down, void* workspace, size_t workspace_bytes,
                  void* hip_stream, const seedmm_side* side) {
    if (P == 0 ? !p4mask : ((P != 3 && P != 4) || p4mask)) return SEEDMM_EINVAL;
    return moe_run(topk_ids, topk_w, T, top_k, x, y, E, H, I, P, p4mask, gate, up, down,
                   workspace, workspace_bytes, hip_stream, nullptr, nullptr, 0, side);
}

int seedmm_moe_mixed(const int32_t* topk_ids, const float* topk_w, int T, int top_k,
                     const void* x, float* y, int E, int H, int I, const uint32_t* p4mask,
                     seedmm_mat gate, seedmm_mat up, seedmm_mat down, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
    if (!p4mask) return SEEDMM_EINVAL;
    return moe_run(topk_ids, topk_w, T, top_k, x, y, E, H, I, 0, p4mask, gate, up, down,
                   workspace, workspace_bytes, hip_stream, nullptr, nullptr, 0, nullptr);
}

int seedmm_moe(const int32_t* topk_ids, const float* topk_w, int T, int top_k, const void* x,
               float* y, int E, int H, int I, int P, seedmm_mat gate, seedmm_mat up,
               seedmm_mat down, void* workspace, size_t workspace_bytes, void* hip_stream) {
    return seedmm_moe_timed(topk_ids, topk_w, T, top_k, x, y, E, H, I, P, gate, up, down,
                            workspace, workspace_bytes, hip_stream, nullptr);
}

}  // extern "C"

// ----------------------------------------------------------------------------------
// seedmm_moe_noalloc: seedmm_moe with its workspace in a static device array.  Every
// device the library runs on holds its own copy of `scratch` until the process ends.
// In host code the array's name is only a stand-in: the device address of the current
// device's copy comes from hipGetSymbolAddress, looked up once per device and kept.
// ----------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = 8u << 20;   // SEEDMM_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == SEEDMM_NOALLOC_SCRATCH_BYTES, "header and library agree");
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once known

// Device `dev`'s copy of `scratch` (dev current; nullptr if the lookup fails).
void* scratch_of_device(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int seedmm_moe_noalloc(const int32_t* topk_ids, const float* topk_w, int T,
                                  int top_k, const void* x, float* y, int E, int H, int I,
                                  int P, seedmm_mat gate, seedmm_mat up, seedmm_mat down,
                                  void* hip_stream) {
    if (P != 3 && P != 4) return SEEDMM_EINVAL;
    const size_t need = seedmm_moe_workspace_bytes(T, top_k, E, H, I);
    if (need == 0) return SEEDMM_EINVAL;
    if (need > kScratchBytes) return SEEDMM_ESCRATCH;
    if (T == 0) return SEEDMM_OK;
    // the array used is the current device's, so the stream must run on that device
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SEEDMM_EHIP;
    if (hip_stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice((hipStream_t)hip_stream, &sdev) != hipSuccess || sdev != dev)
            return SEEDMM_EINVAL;
    }
    void* ws = scratch_of_device(dev);
    if (!ws) return SEEDMM_EHIP;
    // Every scratch word the kernels read is written earlier in the same call (the
    // dispatch writes all E counts and the lists up to them; the expert kernels write
    // every SwiGLU row and per-slot output they later read), so nothing is cleared.
    return moe_run(topk_ids, topk_w, T, top_k, x, y, E, H, I, P, nullptr, gate, up, down, ws,
                   kScratchBytes, hip_stream, nullptr, nullptr, 0, nullptr);
}
