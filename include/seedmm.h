/*
 * seedmm.h -- C ABI of the SeedLM seed-decoding matrix products for AMD MI355X (gfx950).
 *
 * What the library computes.  A weight matrix W[M][K] is stored as blocks of 8
 * consecutive weights along K (block b = m*(K/8) + k/8).  Each block holds a 16-bit
 * LFSR seed, P (3 or 4) signed int4 coefficients and a 4-bit exponent code; each
 * matrix holds one int32 exp_bias (model card "K2-Horizon-MoVA-36B-A4B - NanoSeedLM
 * p4mx-q4v", section "This upload": NAME.seeds U16, NAME.coefs U16, NAME.codes U8,
 * NAME.exp_bias I32).  The kernels regenerate each block inside the product and never
 * write W back (NanoSeedLM README, "Highlights"; barnson.org post, "What I changed:
 * September 2026", never decompress):
 *
 *     w_i = 2^(code + exp_bias - 15) * sum_{j<P} c_j * (s_{iP+j+1} - 32768),  i = 0..7
 *
 * where s_1, s_2, ... are the states after steps 1, 2, ... of a 16-bit Fibonacci
 * register started at the seed (shift left, new bit = parity(state & 0xB400)), the
 * basis is filled row-major, c_j = (q ^ 8) - 8 for nibble q (barnson.org post, "LFSR is
 * free"), and the power of two multiplies (barnson.org post, "Attempt one").
 *
 * Stream layout of one matrix (all little-endian):
 *   seeds  uint16[M*K/8]              one seed per block;
 *   coefs  uint16[ceil(M*K/8*P/4)]    one nibble stream, P nibbles per block, nibble
 *                                     n = b*P + j at word n>>2, bits 4*(n&3);
 *   codes  uint8 [ceil(M*K/16)]       two 4-bit codes per byte, even block in the low nibble.
 * Stacked experts ([E] matrices of equal shape) are the E single-matrix streams
 * concatenated; this requires (M*K/8)*P % 4 == 0 and (M*K/8) % 2 == 0.  The weights
 * are exact in fp32: |sum| <= 2^20 and the scale is a power of two.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller (e.g. PyTorch tensors).
 *     The library allocates no memory and keeps no mutable global state: no streams,
 *     events or tables of its own.  Scratch memory (the layer's workspace, the encoder's
 *     table, a second stream and its events) comes from the caller, so calls are
 *     reentrant and calls from several host threads are independent as long as they do
 *     not share a workspace, a table being prepared or a seedmm_side.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL = the
 *     default stream).  Results are valid after the stream is synchronised.
 *   - Arguments are validated before anything is launched; an error returns a negative
 *     status and launches nothing.  SEEDMM_EHIP reports a failed kernel launch
 *     (hipGetLastError); faults during execution surface at the next synchronisation.
 *   - Limits: K % 8 == 0; P in {3, 4}; exp_bias in [-100, 100] (keeps every weight a
 *     normal fp32); activation rows 16-byte aligned (x pointer 16-byte aligned, ldx a
 *     multiple of 8 elements for bf16 and of 4 for fp32).  Seed streams that are 16-byte
 *     aligned with K % 64 == 0 take the vector-load path; other layouts take a per-block
 *     path with the same results.
 */
#ifndef SEEDMM_H
#define SEEDMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SEEDMM_OK = 0,
    SEEDMM_EINVAL = -1,     /* null pointer, bad size, bad P / dtype / exp_bias / ld   */
    SEEDMM_EALIGN = -2,     /* activation or output pointer / leading dim misaligned  */
    SEEDMM_EWORKSPACE = -3, /* workspace missing or smaller than seedmm_moe_workspace_bytes */
    SEEDMM_EHIP = -4,       /* the HIP runtime reported a launch failure              */
    SEEDMM_ECAPACITY = -5,  /* an expert cache call routes to more distinct experts
                               than the cache has slots                               */
    SEEDMM_ESCRATCH = -6    /* seedmm_moe_noalloc: the batch needs more scratch than
                               SEEDMM_NOALLOC_SCRATCH_BYTES                           */
};

enum { SEEDMM_F32 = 0, SEEDMM_BF16 = 1 };

/* One seed-coded matrix, or E stacked matrices of one shape (streams concatenated). */
typedef struct seedmm_mat {
    const uint16_t *seeds;    /* NAME.seeds                                     */
    const uint16_t *coefs;    /* NAME.coefs (nibble stream)                     */
    const uint8_t *codes;     /* NAME.codes (two codes per byte)                */
    const int32_t *exp_bias;  /* NAME.exp_bias, int32[E] in device memory      */
} seedmm_mat;

/*
 * seedmm_gemv -- y = W x for one fp32 activation vector (the decode matrix-vector
 * product of the SeedLM pages: NanoSeedLM README "How it works").
 *   seeds/coefs/codes: one [M][K] matrix;  exp_bias: its bias (by value);
 *   x: fp32[K];  y: fp32[M] (overwritten).  Runs on the default stream.
 *   Accumulates in fp32 with exact fp32 weights.
 * Errors: SEEDMM_EINVAL (null pointer, M < 0, K < 0, K % 8 != 0, P not 3/4, exp_bias
 * out of range), SEEDMM_EALIGN (x not 16-byte aligned), SEEDMM_EHIP.
 */
int seedmm_gemv(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                int32_t exp_bias, const float *x, float *y, int M, int K, int P);

/*
 * seedmm_gemv_ex -- Y[n] = W X[n] for N activation rows: the product of seedmm_gemv for a
 * batch of rows that share each regenerated block (barnson.org post, "What I changed:
 * September 2026": the weights are rebuilt inside the product, never stored).
 *   x: row-major [N][ldx] of dtype x_dtype (SEEDMM_F32 or SEEDMM_BF16 raw bits);
 *   y: fp32 row-major [N][ldy], overwritten (ldy >= M).
 *   fp32 x: fp32 products and sums with exact weights.  bf16 x: the block weights are
 *   rounded to bf16 (nearest even) and multiplied on the matrix cores with fp32
 *   accumulation.
 * Errors: as seedmm_gemv, plus SEEDMM_EINVAL for N < 0, ldx < K, ldy < M, bad dtype;
 * SEEDMM_EALIGN for a misaligned x or ldx.
 */
int seedmm_gemv_ex(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                   int32_t exp_bias, const void *x, int x_dtype, int ldx, float *y, int ldy,
                   int M, int K, int P, int N, void *hip_stream);

/*
 * seedmm_reconstruct -- write W[M][K] row-major: fp32 (exact) or bf16 (round to nearest
 * even of the exact fp32).  The reference point for bit-exact checks against a scalar C
 * reference (barnson.org post, "What I changed: September 2026": every GPU path is held
 * to a plain C function); the products above never materialise W.  A seed of 0 is
 * decoded like any other (every state is 0, every basis value -32768).
 * Errors: SEEDMM_EINVAL (null pointer, bad size, P, dtype or exp_bias), SEEDMM_EHIP.
 */
int seedmm_reconstruct(const uint16_t *seeds, const uint16_t *coefs, const uint8_t *codes,
                       int32_t exp_bias, void *W, int w_dtype, int M, int K, int P,
                       void *hip_stream);

/*
 * seedmm_moe_dispatch -- group the (token, slot) pairs of a routed batch by expert (the
 * routed experts of a layer, K2-Horizon card "This upload": 100 routed experts per
 * layer, top-8; each expert's matrices are then read once for all its tokens).
 *   topk_ids: int32[T][top_k], each in [0, E) and distinct within a token.
 *   counts: int32[E] (out) -- number of pairs routed to each expert;
 *   lists:  int32[E][T] (out) -- expert e's pair indices p = t*top_k + slot, in
 *           increasing order, in lists[e*T .. e*T + counts[e]).  Entries past counts[e]
 *           are not written.
 * Deterministic.  Ids outside [0, E) are counted nowhere (the caller validates ids).
 * Errors: SEEDMM_EINVAL (null pointer, T < 0, top_k < 1, E < 1, T*top_k >= 2^31),
 * SEEDMM_EHIP.
 */
int seedmm_moe_dispatch(const int32_t *topk_ids, int T, int top_k, int E, int32_t *counts,
                        int32_t *lists, void *hip_stream);

/* Bytes of scratch memory seedmm_moe (and _ex, _timed, _mixed, seedmm_cache_moe) needs
 * for a batch of T tokens routed to top_k of E experts of hidden size H and intermediate
 * size I (0 on bad args, T*top_k >= 2^31 among them): expert counts int32[E], pair lists int32[E][T], the SwiGLU rows
 * bf16 [T*top_k][I] and the per-slot outputs fp32 [T*top_k][H], each 256-byte aligned,
 * plus per-tile counts int32[ceil(T*top_k/8192)][E] above 8,192 pairs.  H and I enter
 * because the SwiGLU rows and the per-slot outputs dominate the size.  (Routed layer of
 * the K2-Horizon card, "This upload".) */
size_t seedmm_moe_workspace_bytes(int T, int top_k, int E, int H, int I);

/*
 * seedmm_moe -- one routed mixture-of-experts layer of SwiGLU experts whose weights
 * are seeds (K2-Horizon card "This upload": routed FFN experts are SeedLM P=4):
 *     y[t] = sum_{s < top_k} topk_w[t][s] * down_e( silu(gate_e x[t]) * (up_e x[t]) ),
 *     e = topk_ids[t][s],  silu(z) = z / (1 + exp(-z)).
 *   (The pages do not spell out the expert FFN; SwiGLU experts with softmax-weighted
 *   top-k slots are this library's reading.)
 *   x: bf16 [T][H] (raw bits), y: fp32 [T][H] (overwritten);
 *   gate, up: E stacked [I][H] matrices; down: E stacked [H][I] matrices;
 *   topk_ids: int32[T][top_k], each in [0, E) and distinct within a token (the caller
 *   validates them; a token that breaks this gets undefined y);
 *   workspace: device scratch of at least seedmm_moe_workspace_bytes(T, top_k, E, H, I)
 *   bytes, 16-byte aligned; its contents need not be initialised.  Calls that overlap
 *   in time must use different workspaces.
 *   Expert products run on the matrix cores with bf16 weights and fp32 accumulation;
 *   the SwiGLU output h is rounded to bf16 (nearest even) before the down product, in
 *   the decode and the prefill kernels alike; the slots of a token are summed in slot
 *   order, so results are bit-reproducible and a token's output does not depend on the
 *   other tokens of the batch.  All work runs on hip_stream (seedmm_moe_ex splits it
 *   over a second stream of the caller's).
 * Errors: SEEDMM_EINVAL (null pointer, T < 0, top_k outside [1, min(E, 64)], T*top_k
 * >= 2^31 (pair indices are int32), E < 1 or > 4096, H or I not a multiple of 8, P not 3/4, stacked streams not whole words),
 * SEEDMM_EALIGN (x not 16-byte aligned or H % 8 != 0), SEEDMM_EWORKSPACE, SEEDMM_EHIP.
 */
int seedmm_moe(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
               const void *x, float *y, int E, int H, int I, int P,
               seedmm_mat gate, seedmm_mat up, seedmm_mat down,
               void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * seedmm_moe_ex -- the routed layer of seedmm_moe (one P) or seedmm_moe_mixed (P = 0 and
 * p4mask), with a second stream from the caller.  The layer runs as two independent
 * halves: for one P, the experts e < E/2 on hip_stream and the others on side->stream;
 * for mixed packs, the P = 4 launches on hip_stream and the P = 3 launches on
 * side->stream.  side->fork is recorded on hip_stream after the dispatch and waited for
 * by side->stream; side->join is recorded on side->stream after its launches and waited
 * for by hip_stream before the combine.  So all the work still completes in hip_stream's
 * order, and graph capture on hip_stream records the fork and the join as dependencies.
 * The two halves' workgroups fill each other's partly empty last rounds (each expert
 * kernel leaves part of the chip idle at its tail).  The output bits equal seedmm_moe's.
 *   side: NULL or side->stream NULL = everything on hip_stream.  Otherwise side->stream
 *   is a stream of hip_stream's device other than hip_stream, and side->fork and
 *   side->join are events (hipEventDisableTiming is enough), all created and owned by
 *   the caller.  Calls that may overlap in time must not share a seedmm_side.  One-token
 *   batches run on hip_stream alone (splitting their slots over two streams measured
 *   slower: the cross-stream edges cost more than the overlap gains).
 * Errors: as seedmm_moe; SEEDMM_EINVAL also for P = 0 without p4mask, a p4mask with
 * P = 3 or 4, or a side stream given without both events or equal to hip_stream.  If the
 * fork cannot be recorded the call runs on hip_stream alone; if the join cannot be
 * recorded it returns SEEDMM_EHIP without launching the combine (y is then not valid).
 */
typedef struct seedmm_side {
    void *stream;   /* hipStream_t */
    void *fork;     /* hipEvent_t  */
    void *join;     /* hipEvent_t  */
} seedmm_side;

int seedmm_moe_ex(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                  const void *x, float *y, int E, int H, int I, int P, const uint32_t *p4mask,
                  seedmm_mat gate, seedmm_mat up, seedmm_mat down,
                  void *workspace, size_t workspace_bytes, void *hip_stream,
                  const seedmm_side *side);

/*
 * seedmm_moe_noalloc -- seedmm_moe without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Its scratch memory is a static device array of the library,
 * SEEDMM_NOALLOC_SCRATCH_BYTES (8 MiB) on every device it runs on, held until the process
 * ends; the call allocates nothing (no hipMalloc, no hipFree, no allocating library
 * routine).  The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress) with the device current; make it outside graph capture.
 *   Arguments, results and errors as seedmm_moe (one stream), plus SEEDMM_ESCRATCH when
 *   seedmm_moe_workspace_bytes(T, top_k, E, H, I) exceeds SEEDMM_NOALLOC_SCRATCH_BYTES
 *   (for 100 experts 2048 -> 1024 -> 2048, top-8: up to 96 tokens), checked before
 *   anything runs, and SEEDMM_EINVAL when hip_stream belongs to another device than the
 *   current one (the array used is the current device's).
 *   Every call on one device shares that device's array: calls that overlap in time on
 *   one device race (serialise them on one stream), and the array keeps the last call's
 *   contents, which no call reads before writing them.
 */
#define SEEDMM_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int seedmm_moe_noalloc(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                       const void *x, float *y, int E, int H, int I, int P,
                       seedmm_mat gate, seedmm_mat up, seedmm_mat down, void *hip_stream);

/*
 * seedmm_moe_timed -- seedmm_moe that also records caller-created hipEvent_t handles on
 * hip_stream between its kernels, for measuring each stage in place (the pages time
 * their engines stage by stage: NanoSeedLM documentation index, "Results"):
 *   events[0] before the dispatch, events[1] after it, events[2] after the gate/up
 *   kernel, events[3] after the down kernel, events[4] after the combine.  A one-token
 *   batch (T = 1) runs no dispatch kernel (its top_k ids name the experts directly), so
 *   events[0] and events[1] are recorded back to back; with one P, vector layouts and
 *   2 <= top_k <= 8 it runs no combine kernel either (its down kernel adds the slots,
 *   same bits), so events[3] and events[4] are back to back too.
 * `events` may be NULL and any entry may be NULL.  Same arguments, results and errors
 * as seedmm_moe; no event is recorded when the arguments are rejected.  When `events`
 * is not NULL every kernel runs on hip_stream (no side stream), so the recorded stage
 * times are those of single launches over all experts.
 */
int seedmm_moe_timed(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                     const void *x, float *y, int E, int H, int I, int P,
                     seedmm_mat gate, seedmm_mat up, seedmm_mat down,
                     void *workspace, size_t workspace_bytes, void *hip_stream,
                     void *const *events);

/*
 * seedmm_moe_mixed -- seedmm_moe for mixed packs: P chosen per expert (NanoSeedLM
 * documentation index: "Results", hybrid P3 / P4 seed packs with a third of the experts
 * in P4; "Plans", a P4 tier for the hot experts and P3 for the rest).
 *   p4mask: device uint32[ceil(E/32)], bit e (word e/32, bit e%32) set when expert e has
 *   P = 4, clear when it has P = 3.
 *   Stacked streams: seeds and codes at the same per-expert strides as seedmm_moe;
 *   expert e's coefficient stream starts at word (I*H/8/4) * (3e + number of P = 4
 *   experts before e), i.e. the experts' own streams concatenated in expert order.
 *   Requires (I*H/8) % 4 == 0.  Other arguments, results and errors as seedmm_moe
 *   (SEEDMM_EINVAL also for a NULL p4mask).  Each expert kernel runs once per P; a
 *   launch serves only the experts of its P.  All work runs on hip_stream
 *   (seedmm_moe_ex with P = 0 runs the P = 3 launches on a second stream).
 */
int seedmm_moe_mixed(const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                     const void *x, float *y, int E, int H, int I, const uint32_t *p4mask,
                     seedmm_mat gate, seedmm_mat up, seedmm_mat down,
                     void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * seedmm_search -- encode W [M][K] into a seed-coded matrix by the exhaustive seed search
 * (Qwen3.8-Flash-Next-NanoSeedLM-P4 card, "How it works": every one of the 65,535 seeds
 * is tried for every block; barnson.org post, "GPU search == CPU search").  For each
 * block of 8 weights w (with importances d, all ones when colw is NULL) and every seed:
 *   U_ij = s_{iP+j+1} - 32768 (the states the products regenerate);
 *   alpha solves A alpha = r, A_jk = sum_i (d_i U_ij) U_ik, r_j = sum_i (d_i U_ij) w_i, by
 *   Gaussian elimination with partial pivoting (a pivot below 1e-300 skips the seed);
 *   for every code 0..15: c_j = clamp(round_half_even(alpha_j / 2^(code+exp_bias-15)),
 *   -8, 7), err = sum_i d_i (w_i - 2^(code+exp_bias-15) sum_j U_ij c_j)^2;
 * and keeps the smallest (err, seed, code).  Every step is an IEEE double operation in
 * that order (sums in increasing i, no contraction), so the result equals a CPU
 * evaluation of the same definition bit for bit.
 *   W: fp32 row-major [M][ldw] (ldw >= K), K % 8 == 0;  colw: fp32 [K] importances of
 *   the columns (activation weighting) or NULL;  outputs in the layout the products
 *   read: seeds uint16[M*K/8], coefs uint16[ceil(M*K/8*P/4)], codes uint8[ceil(M*K/16)],
 *   err: float64[M*K/8] squared error of each block (may be NULL).  A block for which
 *   no seed gives a solvable system gets seed 0, zero coefficients and err = +inf.
 *   Pairs (block, seed) that provably cannot win are skipped (a least-squares bound and,
 *   at P = 4, a bound of every code's error, each with a safe margin); the result is the
 *   same as evaluating them all.
 *   table: without importances (colw NULL), device memory of at least
 *   seedmm_search_table_bytes(P) bytes, 256-byte aligned, filled for this P by
 *   seedmm_search_prepare on hip_stream or before it in stream order (a table filled for
 *   the other P, or not filled, gives undefined results); with importances it is not
 *   read and may be NULL.  The call only launches kernels (no host wait), so it can be
 *   captured into a graph.  Calls may share a prepared table and overlap on different
 *   streams.
 * Errors: SEEDMM_EINVAL (null pointer, a NULL table without importances, bad size, P not
 * 3/4, exp_bias outside [-100, 100], ldw < K), SEEDMM_EALIGN (table not 256-byte
 * aligned), SEEDMM_EHIP.
 */
int seedmm_search(const float *W, int ldw, const float *colw, int M, int K, int P,
                  int32_t exp_bias, uint16_t *seeds, uint16_t *coefs, uint8_t *codes,
                  double *err, const void *table, void *hip_stream);

/*
 * The encoder's per-seed table for one P (barnson.org post, "LFSR is free": the pages'
 * encoder and decoder precompute per-seed streams; here the search precomputes, once per
 * P, each seed's basis rows along the register's cycle, its normal matrix, the matrix's
 * Cholesky factor and a certified bound of its smallest eigenvalue): about 16.5 MB
 * (P = 4) or 12.3 MB (P = 3) of caller-owned device memory.
 * seedmm_search_table_bytes returns the size (0 for P not 3/4).  seedmm_search_prepare
 * fills `table` on hip_stream with kernels only (no host wait; capturable).
 * Errors: SEEDMM_EINVAL (P not 3/4, NULL table, table_bytes too small), SEEDMM_EALIGN
 * (table not 256-byte aligned), SEEDMM_EHIP.
 */
size_t seedmm_search_table_bytes(int P);
int seedmm_search_prepare(int P, void *table, size_t table_bytes, void *hip_stream);

/*
 * Expert cache: routed experts resident in host memory, the recently used ones in device
 * memory (NanoSeedLM README, "Highlights": the engine can keep the routed experts in
 * RAM with a VRAM cache of the recently used ones, and "With the engine": a cache sized
 * with --expert-cache-gb; documentation index, "Results": LRU beats LFU and a fixed hot
 * set as the eviction policy).
 *
 * One cache serves one layer of E experts (gate/up [I][H], down [H][I], one P) with S
 * device slots.  An expert is one RECORD of its nine streams, in the order gate.seeds,
 * gate.coefs, gate.codes, up.seeds, ..., down.codes, each stream (the expert's own
 * streams as in seedmm_moe: n*2, ceil(n*P/4)*2 and ceil(n/2) bytes, n = I*H/8) starting
 * at a multiple of 256 bytes from the record start; seedmm_cache_record_layout gives the
 * offsets and the record size (a multiple of 256).  Loading an expert copies its record.
 * All memory is the caller's:
 *   state      host memory of seedmm_cache_state_bytes(E, S) bytes, 8-byte aligned: the
 *              bookkeeping (which expert sits in which slot, last use of each slot,
 *              counters); it is the cache handle, used only by the calls below;
 *   device     device memory of seedmm_cache_device_bytes(E, H, I, P, S) bytes,
 *              256-byte aligned: S records and the device expert -> slot map;
 *   host_pack  PINNED host memory (hipHostMalloc) of E records, expert e at byte
 *              e * record; read by host-to-device copies only;
 *   exp_bias   device int32[3][E]: the exp_bias of gate, up and down of every expert
 *              (stays resident).
 * Calls on one cache must not overlap (one host thread at a time), and their device work
 * must run in call order: a call's record copies can overwrite slots that the previous
 * call's kernels still read, so pass one stream to every call on a cache, or make the
 * new call's stream wait for the previous call's.  The host pack must stay unchanged
 * while the cache is in use (seedmm_cache_reset after changing it).
 */
typedef struct seedmm_cache seedmm_cache;

/* Record size in bytes, and the nine stream offsets into `offsets` (may be NULL); 0 for
 * an invalid shape. */
size_t seedmm_cache_record_layout(int H, int I, int P, size_t offsets[9]);
size_t seedmm_cache_state_bytes(int E, int S);
size_t seedmm_cache_device_bytes(int E, int H, int I, int P, int S);

/* Initialise `state` as an empty cache.  Host only (no HIP call).  Requires E in
 * [1, 4096], S in [1, E], P in {3, 4} and the layer shapes of seedmm_moe (H, I > 0,
 * multiples of 8, with the stacking conditions on n = I*H/8: n*P % 4 == 0, n % 2 == 0).
 * Errors: SEEDMM_EINVAL (null pointer, bad size, state_bytes or device_bytes too small),
 * SEEDMM_EALIGN (state not 8-byte or device not 256-byte aligned). */
int seedmm_cache_init(void *state, size_t state_bytes, int E, int H, int I, int P, int S,
                      const void *host_pack, const int32_t *exp_bias, void *device,
                      size_t device_bytes);

/* Empty the cache and zero its counters (every expert is loaded again on its next use).
 * Host only. */
int seedmm_cache_reset(seedmm_cache *cache);

/* The host half of one call, on its own: marks the distinct experts of topk_ids_host
 * [T][top_k] used and assigns a slot to each that is not resident.  Resident experts are
 * hits; each miss takes, in increasing expert order, the lowest free slot, else the slot
 * whose expert was used longest ago (ties: lowest slot) among those this call does not
 * use.  loads: host int32[2*S] receiving (expert, slot) pairs in that order (may be
 * NULL); *n_loads their count.  Host only; the state changes only on success.
 * Errors: SEEDMM_EINVAL (id outside [0, E), bad T / top_k), SEEDMM_ECAPACITY (more
 * distinct experts than slots). */
int seedmm_cache_plan(seedmm_cache *cache, const int32_t *topk_ids_host, int T, int top_k,
                      int32_t *loads, int *n_loads);

/* One routed layer call through the cache: seedmm_cache_plan on topk_ids_host, then on
 * hip_stream one host-to-device copy of every loaded expert's record into its slot, the
 * update of the device slot map, and the layer of seedmm_moe reading the experts from
 * their slots.  topk_ids (device) must hold the same ids as topk_ids_host; the other
 * arguments, results and errors are seedmm_moe's, plus SEEDMM_ECAPACITY; argument errors
 * leave the state unchanged.  The output equals seedmm_moe's on the resident layer bit
 * for bit.  If a copy or launch fails the cache is emptied and SEEDMM_EHIP returned. */
int seedmm_cache_moe(seedmm_cache *cache, const int32_t *topk_ids_host,
                     const int32_t *topk_ids, const float *topk_w, int T, int top_k,
                     const void *x, float *y, void *workspace, size_t workspace_bytes,
                     void *hip_stream);

/* Counters since init or reset: out[0] calls, out[1] expert uses (distinct experts per
 * call, summed), out[2] hits, out[3] misses (= records copied), out[4] bytes copied
 * host-to-device. */
int seedmm_cache_stats(const seedmm_cache *cache, uint64_t out[5]);

/* Static description of a status code (the C engine's error convention: a plain C99
 * interface, NanoSeedLM README "How it works"). */
const char *seedmm_strerror(int status);

/* Library ABI version (major * 100 + minor); 200 = caller-owned side streams and
 * encoder tables. */
int seedmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEEDMM_H */
