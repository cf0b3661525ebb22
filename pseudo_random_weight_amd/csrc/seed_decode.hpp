// seed_decode.hpp -- in-register regeneration of SeedLM weight blocks on gfx950.
//
// A block of 8 weights is a 16-bit seed, P int4 coefficients and a 4-bit exponent
// code (Qwen3.8-Flash-Next-NanoSeedLM-P4 card, "How it works"):
//     w_i = 2^(code + exp_bias - 15) * sum_j c_j * (s_{iP+j+1} - 32768)
// with s_t the register state after t steps from the seed (barnson.org post, "LFSR is
// free" and "What I changed": the seed is the initial state).
//
// Register: 16-bit Fibonacci LFSR shifting left, feedback x^16 + x^14 + x^13 + x^11 + 1.
// Viewed as a bit stream x_0, x_1, ... (x_0..x_15 = seed, most significant bit first,
// x_n = x_{n-16} ^ x_{n-14} ^ x_{n-13} ^ x_{n-11}), state s_t is the 16-bit window
// x_t .. x_{t+15}, so every state of a block sits inside the 48-bit word x_0..x_47
// (barnson.org post, "LFSR is free": states become shifts of one word).
//
// The kernels never step the register one bit at a time.  Because the nearest tap is
// 11 positions back, 11 new stream bits come out of one shift/xor group; the bits
// x_32..x_47 follow from x_0..x_25 through the squared polynomial (distances 32, 28,
// 26, 22).  Alternatively the 32 bits after a seed come from two 256-entry tables, the
// 32-bit continuation being GF(2)-linear in the seed (same section: stream tables).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seedmm {

// 1.5 * 2^23: adding an integer |T| < 2^22 to this float's bit pattern gives the float
// 1.5*2^23 + T exactly, so the block sums need no integer-to-float convert.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

struct Window {
    uint32_t hi;  // x_0 .. x_31  (bit 31 = x_0):  s_t = bits [16-t, 32-t) for t <= 16
    uint32_t lo;  // x_16 .. x_47 (bit 31 = x_16): s_t = bits [32-t, 48-t) for t >= 16
};

// Stream bits x_0..x_47 of a seed with three shift/xor groups (17 VALU ops).
__device__ __forceinline__ Window lfsr_window(uint32_t seed16) {
    uint32_t R = seed16 << 16;                // x_0..x_15 at bits 31..16
    uint32_t a = R ^ (R >> 3);
    uint32_t b = a ^ (a >> 2);                // b>>11 = R>>11 ^ R>>13 ^ R>>14 ^ R>>16
    R |= (b >> 11) & 0xFFE0u;                 // x_16..x_26 at bits 15..5
    a = R ^ (R >> 3);
    b = a ^ (a >> 2);
    R |= (b >> 11) & 0x1Fu;                   // x_27..x_31 at bits 4..0
    uint32_t c = R ^ (R << 4);
    uint32_t L = c ^ (c << 6);                // bits 31..16 = x_32..x_47 (squared taps)
    Window w;
    w.hi = R;
    w.lo = __builtin_amdgcn_alignbit(R, L, 16);
    return w;
}

// Same window from the 32-bit continuation of the seed (table lookup result).
__device__ __forceinline__ Window window_from_next32(uint32_t seed16, uint32_t next32) {
    Window w;
    w.hi = __builtin_amdgcn_alignbit(seed16, next32, 16);
    w.lo = next32;
    return w;
}

// Window from two 256-entry tables of 32-bit continuations: the continuation is
// GF(2)-linear in the seed, so next32(seed) = lo[seed & 0xFF] ^ hi[seed >> 8] with
// lo[b] = next32(b) and hi[b] = next32(b << 8).  `tab` holds lo in [0, 256) and hi in
// [256, 512) (LDS).
__device__ __forceinline__ Window window_from_tables(uint32_t seed16, const uint32_t* tab) {
    const uint32_t n32 = tab[seed16 & 0xFFu] ^ tab[256 + (seed16 >> 8)];
    return window_from_next32(seed16, n32);
}

// 32-bit continuation x_16..x_47 of a seed (used to fill the lookup tables).
__device__ __forceinline__ uint32_t lfsr_next32(uint32_t seed16) {
    return lfsr_window(seed16).lo;
}

// Fills the two continuation tables (512 words of LDS) with the workgroup's threads and
// waits for them; call before any thread of the workgroup can leave.
__device__ __forceinline__ void fill_lfsr_tables(uint32_t* tab) {
    for (int i = threadIdx.x; i < 512; i += blockDim.x)
        tab[i] = lfsr_next32(i < 256 ? (uint32_t)i : (uint32_t)(i - 256) << 8);
    __syncthreads();
}

// State s_t (1 <= t <= 32) of a window.  Callers unroll their loops, so t folds to a
// constant and each state costs one bit-field extract.
__device__ __forceinline__ uint32_t state(const Window& w, int t) {
    return t <= 16 ? __builtin_amdgcn_ubfe(w.hi, 16 - t, 16)
                   : __builtin_amdgcn_ubfe(w.lo, 32 - t, 16);
}

// Power-of-two block scale 2^(code + exp_bias - 15) as an exact float.
__device__ __forceinline__ float block_scale(uint32_t code, int exp_bias) {
    return __int_as_float((int)(code + (uint32_t)(exp_bias - 15 + 127)) << 23);
}

// d = a * b + c on the 24-bit integer multiplier (one v_mad_i32_i24).  Written out
// because the compiler otherwise splits the chain into multiplies plus 3-input adds,
// which costs half again as many instructions per basis value.
__device__ __forceinline__ int mad24(int a, int b, int c) {
    int d;
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// Integer block sums T_i = sum_j c_j (s_{iP+j+1} - 32768), i = 0..7, returned as the bit
// patterns of the floats 1.5*2^23 + T_i (|T_i| <= 2^20).  `cw` holds the block's P
// coefficient nibbles in its low 4P bits; nibble q decodes as (q ^ 8) - 8 (barnson.org
// post, "LFSR is free": convert-free coefficients), which the signed bit-field extract
// does in one step.
template <int P>
__device__ __forceinline__ void block_sums(const Window& w, uint32_t cw, int f[8]) {
    int c[P];
    int csum = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        c[j] = __builtin_amdgcn_sbfe((int)cw, 4 * j, 4);
        csum += c[j];
    }
    const int k0 = kMagicBits - 32768 * csum;   // folds the -32768 offset of every state
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int acc = k0;
#pragma unroll
        for (int j = 0; j < P; ++j)
            acc = mad24(c[j], (int)state(w, i * P + j + 1), acc);   // row-major basis
        f[i] = acc;
    }
}

// Exact fp32 weights of one block: (1.5*2^23 + T) * s - 1.5*2^23 * s = T * s in one
// rounding-free fused multiply-add (s is a power of two, T * s is representable).
template <int P>
__device__ __forceinline__ void decode_block(const Window& w, uint32_t cw, uint32_t code,
                                             int exp_bias, float out[8]) {
    int f[8];
    block_sums<P>(w, cw, f);
    const float s = block_scale(code, exp_bias);
    const float off = -kMagic * s;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        out[i] = __builtin_fmaf(__int_as_float(f[i]), s, off);
}

}  // namespace seedmm
