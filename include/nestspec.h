/*
 * nestspec.h -- C ABI of the nested-weight self-speculative decoding round.
 *
 * The method is BitNest ("BitNest: Bit-Nested Speculative Decoding for
 * Memory-Efficient LLM Inference Acceleration"). Per its Figure 2, one
 * quantized weight copy holds a b-bit base and an r-bit refinement of the
 * base's remaining error. Per its Figure 3, the two codes sit in two
 * independent 4-bit planes of N/2 bytes each for N weights. The draft reads
 * only the base plane; verification reads both planes to recover the 8-bit
 * target. Per its Figure 4, a nested KV cache gives the draft a low-bit
 * base view and verification the full view of the same cache.
 *
 * The round is the one in "How Speculative Decoding Speeds Up Inference",
 * section "Drafting and checking tokens" (three numbered steps, Table 1).
 * The draft proposes k tokens and the target checks all positions in one
 * pass. The matching prefix is kept and the first mismatch is replaced by
 * the target's token, so a round yields 1..k+1 tokens. With greedy decoding
 * every kept token is the target's own choice (section "The same output as
 * the large model alone").
 *
 * The pages fix no group size, scale rule, rounding, nibble order or data
 * layout. This library fixes them as below, and the oracle follows the same
 * definitions.
 *
 * ---------------------------------------------------------------------------
 * Conventions for every entry point
 * ---------------------------------------------------------------------------
 *  - Every buffer pointer is a DEVICE pointer unless the argument says
 *    "host". The caller allocates and owns every buffer it passes,
 *    workspaces included; the library allocates, frees and keeps no device
 *    memory of its own and never synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call enqueues its kernels on that stream and returns without
 *    synchronising.
 *  - Workspaces: sizes come from the *_workspace_size functions. The GEMV
 *    workspaces (draft_gemv, draft_gemv_x, verify_gemm, verify_gemm_x,
 *    verify_accept, verify_accept_x) are 256-byte aligned and must be all
 *    zero before their first use. Their first 4352 bytes are a counter zone
 *    (block counters, laid out alike for all six entry points and every
 *    shape) that every call leaves at zero and no call stores data in, so
 *    one workspace, sized for the largest call, serves any number of calls
 *    of these entry points and shapes. Calls that share a workspace must
 *    not overlap in time (same stream, or ordered by events).
 *  - Lengths that change from round to round can live on the device: the
 *    calls that take a position or a context length also take an optional
 *    device int32 pointer whose value is added to the host value, so a
 *    loop of rounds can advance them (verify_accept does) without the host
 *    reading anything back.
 *  - Arguments are checked on the host before anything is launched. On an
 *    error nothing is launched, the return value is a nest_status code, and
 *    nest_last_error() holds a message for the calling thread. A launch
 *    failure returns NEST_EHIP. A device fault surfaces at the caller's
 *    next synchronisation.
 *  - Input floats must be finite.
 *
 * ---------------------------------------------------------------------------
 * Nested weight format (BitNest, Figures 2 and 3)
 * ---------------------------------------------------------------------------
 *  W is fp32 [rows][cols], row-major. `rows` are output features; `cols` is
 *  the reduction dimension K. A group is `group` consecutive elements of one
 *  row along cols, so a row has G = cols/group groups. Per (row, group):
 *      m   = max |w| over the group
 *      s   = fl32(m / 7)                        base scale (0 when m == 0)
 *      q_b = clamp(rint(w / s), -7, 7)          base code, ties to even
 *      e   = fma(-s, q_b, w)                    remaining error, one rounding
 *      s16 = s * 2^-4                           refinement scale
 *      q_r = clamp(rint(e / s16), -8, 7)        refinement code (0 when s16 == 0)
 *  Every division is IEEE fp32, correctly rounded. When s == 0 both codes
 *  are 0.
 *  Base view of a weight: s * q_b. Full (8-bit) view: s16 * (16*q_b + q_r).
 *  Planes: base and refine are each uint8 [rows][cols/2]. Byte j of a row
 *  holds element 2j in bits 0..3 and element 2j+1 in bits 4..7, as 4-bit
 *  two's complement. Each plane is exactly rows*cols/2 bytes.
 *  Scales: fp32 [rows][G]. Only s is stored; s16 is derived from it.
 *  This row-major form is the storage format nest_pack writes.
 *
 *  Tile layout (what draft_gemv, verify_gemm and verify_accept read; made
 *  from the storage format by nest_tile; group == 128). Rows go in tiles of
 *  16, T = ceil(rows/16); the last tile is padded with zero rows.
 *    plane: byte ((t*G + g)*4 + q)*256 + r*16 + j holds storage byte
 *           (row 16t + r, byte 64g + 16q + j), i.e. per (tile, group) one
 *           kilobyte of [k-quarter q][row r][16 bytes]. T*16*cols/2 bytes.
 *    scales: float ((t*Gq + u)*16 + r)*4 + i, Gq = ceil(G/4), holds the
 *           scale of (row 16t + r, group 4u + i); padding holds 0.
 *           T*64*Gq floats.
 *  Each 16-byte piece a GEMV lane needs, and the four scales of its quad,
 *  are then contiguous across a wave, so the weight stream reads whole
 *  kilobytes instead of 64-byte pieces of 16 rows.
 *
 * ---------------------------------------------------------------------------
 * Activations (the "A8" of W4A8 / W8A8 in BitNest's Table 1)
 * ---------------------------------------------------------------------------
 *  x is fp32 [M][K]. Per row:
 *      sa = fl32(max|x| / 127),  qa = clamp(rint(x / sa), -127, 127).
 *  An all-zero row gives sa = 0 and qa = 0.
 *
 * ---------------------------------------------------------------------------
 * Products and their fp32 fold
 * ---------------------------------------------------------------------------
 *  For output row n, activation row m and group g, the group sums are exact
 *  int32:
 *      Ab[m][n][g] = sum_{k in g} qa[m][k] * q_b[n][k]
 *      Av[m][n][g] = sum_{k in g} qa[m][k] * (16*q_b[n][k] + q_r[n][k])
 *  Reference fold, groups in ascending order, starting from +0:
 *      draft:  run = fmaf(s[n][g],          (float)Ab[m][n][g], run)
 *      verify: run = fmaf(s[n][g] * 2^-4,   (float)Av[m][n][g], run)
 *      y[m][n] = run * sa[m]
 *  Entry points that return an argmax (draft_gemv with `argmax`, and
 *  verify_accept) use exactly this fold, so their y and indices are
 *  bit-identical to it. draft_gemv and verify_gemm without an argmax may
 *  split a row's groups into contiguous segments. Each segment is folded
 *  as above, and the segments are then added in ascending order. In that
 *  case |y - y_ref| <= (G+2) * 2^-24 * sa * sum_g |scale_g * A_g|.
 *  The debug accumulators (`acc_dbg`) are always exact.
 *  argmax: the lowest index among the maximal y (-0 counts as +0).
 *
 * ---------------------------------------------------------------------------
 * Nested KV cache (BitNest, Figure 4)
 * ---------------------------------------------------------------------------
 *  Each (kv head, block of `block` tokens) of K is one quantization group,
 *  and likewise for V. It uses the same rule as the weights, over its
 *  block*d values. Layouts, in elements:
 *      K planes: [Hkv][capacity][d]                 token-major
 *      V planes: [Hkv][capacity/block][d][block]    each block dim-major
 *      scales:   [Hkv][capacity/block] fp32 (one for K, one for V)
 *  Planes pack element pairs into bytes exactly as for weights.
 *  Base view (draft): value = s * q_b. Full view (verify): value =
 *  s16 * (16*q_b + q_r).
 *  Attention: query i of nq sits at position p_i = ctx_len - nq + i and
 *  sees tokens 0..p_i. Query head hq reads kv head hq / (Hq/Hkv).
 *  score = (q . k) / sqrt(d), softmax over the visible tokens, and out is
 *  the probability-weighted sum of v, in fp32 [nq][Hq][d].
 *  Truncation after a round is the caller's length update. A round that
 *  verified k drafts and accepted a of them keeps ctx_len - k + a entries.
 *  Entries past ctx_len are never read. New entries go in through
 *  kv_nest_append, which quantizes each touched block again over its valid
 *  tokens (the open block's scale covers the tokens written so far).
 */
#ifndef NESTSPEC_H
#define NESTSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NEST_OK = 0,
  NEST_EINVAL = 1,       /* null pointer, negative or inconsistent size   */
  NEST_EALIGN = 2,       /* a pointer is not 16- (or 256-) byte aligned   */
  NEST_ESHAPE = 3,       /* a size breaks a divisibility rule             */
  NEST_EWORKSPACE = 4,   /* workspace missing or smaller than required    */
  NEST_EUNSUPPORTED = 5, /* valid, but not a shape these kernels handle   */
  NEST_EHIP = 6          /* a HIP call or kernel launch failed            */
} nest_status;

/* Message describing the last error on the calling thread ("" if none).
   The pointer stays valid until the thread's next call into the library. */
const char* nest_last_error(void);

/* nest_pack -- nested quantization of a weight matrix (BitNest, Figures 2
 * and 3; rule above).
 *   w       fp32 [rows][cols]
 *   base    uint8 [rows][cols/2]   (out)
 *   refine  uint8 [rows][cols/2]   (out)
 *   scales  fp32 [rows][cols/group] (out)
 * Requires rows >= 1, cols >= 2, even group >= 2 and cols % group == 0.
 * Errors: NEST_EINVAL, NEST_ESHAPE, NEST_EHIP. */
int nest_pack(const float* w, int64_t rows, int64_t cols, int64_t group,
              uint8_t* base, uint8_t* refine, float* scales, void* stream);

/* nest_tile -- storage format (nest_pack) -> tile layout (above), for the
 * planes and the scales of one weight matrix. Pure data movement.
 *   base, refine  uint8 [rows][cols/2] (refine may be NULL, with refine_t)
 *   scales        fp32 [rows][cols/128]
 *   base_t, refine_t  uint8, nest_tile_plane_bytes(rows, cols) each (out)
 *   scales_t      fp32, nest_tile_scale_count(rows, cols, group) (out)
 * Requires group == 128, cols % 128 == 0, 16-byte aligned planes. The
 * outputs must not overlap the inputs.
 * Errors: NEST_EINVAL, NEST_EALIGN, NEST_ESHAPE, NEST_EUNSUPPORTED, NEST_EHIP. */
int nest_tile(const uint8_t* base, const uint8_t* refine, const float* scales,
              int64_t rows, int64_t cols, int64_t group, uint8_t* base_t,
              uint8_t* refine_t, float* scales_t, void* stream);
size_t nest_tile_plane_bytes(int64_t rows, int64_t cols);            /* 0 if invalid */
size_t nest_tile_scale_count(int64_t rows, int64_t cols, int64_t group); /* 0 if invalid */

/* nest_act_quant -- per-row symmetric int8 quantization of activations.
 *   x   fp32 [M][K];  qa int8 [M][K] (out);  sa fp32 [M] (out).
 * Requires M >= 1 and K >= 1. Errors: NEST_EINVAL, NEST_EHIP. */
int nest_act_quant(const float* x, int64_t M, int64_t K, int8_t* qa, float* sa,
                   void* stream);

/* draft_gemv -- the draft's W4A8 product over the base plane only (BitNest,
 * Figure 3: the draft touches the base plane alone).
 *   qa       int8 [M][K], 16-byte aligned;  sa fp32 [M]
 *   base     base plane in the tile layout (nest_tile), 16-byte aligned
 *   scales   scales in the tile layout, 16-byte aligned
 *   y        fp32 [M][N] (out, may be NULL when argmax is given)
 *   argmax   int32 [M] (out, nullable). When given, the fold is exact and
 *            argmax[m] is the index of the largest y[m][.].
 *   acc_dbg  int32 [M][N][K/group] (out, nullable): the exact Ab.
 *   ws       workspace of draft_gemv_workspace_size(M, N) bytes (zeroed
 *            before first use, see the conventions), needed only when
 *            argmax is given (else it may be NULL). It holds the per-block
 *            partial maxima and the counter that finds the last block.
 * Up to 16 rows: one GEMV launch, the argmax fused in it (its fold then
 * bit-identical to the sequential one). More rows (the drafts of more than
 * 16 sequences): the batched MFMA kernel over the base plane alone writes
 * y (required then), and one block per row takes the argmax of those
 * values with the same tie rule; the fold adds the group sums in that
 * kernel's order, within the same rounding bound.
 * Requires 1 <= M <= 65535, group == 128, K % 128 == 0, N >= 1.
 * Errors: NEST_EINVAL, NEST_EALIGN, NEST_ESHAPE, NEST_EUNSUPPORTED,
 * NEST_EWORKSPACE, NEST_EHIP. */
int draft_gemv(const int8_t* qa, const float* sa, int64_t M, int64_t K,
               const uint8_t* base, const float* scales, int64_t N, int64_t group,
               float* y, int32_t* argmax, int32_t* acc_dbg,
               void* ws, size_t ws_bytes, void* stream);
size_t draft_gemv_workspace_size(int64_t M, int64_t N);

/* Workspace of the fp32-activation GEMV calls: draft_gemv_x, verify_gemm_x
 * (M rows) and verify_accept_x (M = B*(k+1)) over N output rows (V for the
 * LM head) and reduction length K. 0 if the sizes are invalid. */
size_t nest_gemv_x_workspace_size(int64_t M, int64_t K, int64_t N);

/* draft_gemv_x -- draft_gemv on fp32 activations. Each block quantizes x
 * itself while staging it (the nest_act_quant rule above), so the result is
 * bit-identical to nest_act_quant followed by draft_gemv, with one launch
 * fewer.
 *   x        fp32 [M][K], 16-byte aligned
 *   the rest as for draft_gemv (no debug accumulators)
 *   ws       nest_gemv_x_workspace_size(M, K, N) bytes, zeroed before first
 *            use (always required)
 * Requires 1 <= M <= 65535 (more than 16 rows as for draft_gemv).
 * Activations with M*K > 131072 (beyond the LDS budget for codes), more
 * than 16 rows, and several rows that many blocks would each quantize
 * again (N*M*K >= 1.2e8, M >= 2), are quantized once by a nest_act_quant
 * launch into the workspace; the codes are the same either way.
 * Errors: as draft_gemv. */
int draft_gemv_x(const float* x, int64_t M, int64_t K, const uint8_t* base,
                 const float* scales, int64_t N, int64_t group, float* y,
                 int32_t* argmax, void* ws, size_t ws_bytes, void* stream);

/* verify_gemm -- the target's W8A8 product over both planes (BitNest,
 * Figure 3: the target reads the refinement plane as well and so works with
 * the whole 8-bit code), for the k+1 rows of a round or a batch of rounds.
 *   qa int8 [M][K] (16-byte aligned); sa fp32 [M]
 *   base, refine, scales: the tile layout (nest_tile), 16-byte aligned
 *   y fp32 [M][N] (out); acc_dbg int32 [M][N][K/group] (out, nullable): Av
 *   ws       verify_gemm_workspace_size(M, K, N) bytes (256-byte aligned),
 *            zeroed before first use; may be NULL (ws_bytes 0) when that
 *            size is 0
 * Requires M >= 1, group == 128, K % 128 == 0, N >= 1. M <= 16 runs the
 * one-tile kernel. Larger M runs the batched MFMA kernel in launches of up
 * to 144 rows; with few weight rows over long rows (e.g. 4096 x 14336) it
 * splits the groups over several blocks per row block, whose sums meet in
 * the workspace.
 * Errors: NEST_EINVAL, NEST_EALIGN, NEST_ESHAPE, NEST_EUNSUPPORTED,
 * NEST_EWORKSPACE, NEST_EHIP. */
int verify_gemm(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                const uint8_t* base, const uint8_t* refine, const float* scales,
                int64_t N, int64_t group, float* y, int32_t* acc_dbg, void* ws,
                size_t ws_bytes, void* stream);

/* Workspace of verify_gemm over M rows, reduction length K and N output
 * rows: 0 when the call needs none (M <= 16, or no group split) or the
 * sizes are invalid. It depends on the current device's CU count. */
size_t verify_gemm_workspace_size(int64_t M, int64_t K, int64_t N);

/* verify_gemm_x -- verify_gemm on fp32 activations, quantized in the kernel
 * as for draft_gemv_x (bit-identical to nest_act_quant + verify_gemm), or
 * first quantized into the workspace under the same rule (always when
 * M > 16, which then runs the batched kernel).
 *   ws  nest_gemv_x_workspace_size(M, K, N) bytes, zeroed before first use
 * Requires M >= 1. Errors: as verify_gemm, and NEST_EWORKSPACE. */
int verify_gemm_x(const float* x, int64_t M, int64_t K, const uint8_t* base,
                  const uint8_t* refine, const float* scales, int64_t N,
                  int64_t group, float* y, void* ws, size_t ws_bytes,
                  void* stream);

/* verify_accept -- the verify pass through the nested LM head, with the
 * greedy accept step ("How Speculative Decoding Speeds Up Inference",
 * numbered round steps and Table 1).
 *   qa int8 [B*(k+1)][K]; sa fp32 [B*(k+1)]. Row b*(k+1)+i is sequence b's
 *        input at slot i. Slot 0 is the last committed token and slot
 *        i >= 1 is draft token i.
 *   base, refine, scales: the LM head in the tile layout (nest_tile)
 *   draft     int32 [B][k]: draft tokens d_1..d_k, each in [0, V)
 *   target    int32 [B][k+1] (out): t_i = argmax of the exact verify fold
 *             of row i
 *   n_emitted int32 [B] (out): a+1, where a is the largest j <= k with
 *             d_i == t_{i-1} for all 1 <= i <= j
 *   emitted   int32 [B][k+1] (out): t_0..t_a, then -1 in the unused slots
 *   y         fp32 [B*(k+1)][V] (out; nullable up to 16 rows): the verify
 *             logits
 *   len       int32 [B] (in/out, nullable): each sequence's committed
 *             length, advanced by n_emitted (BitNest, Figure 4: the
 *             accepted entries stay; the blog's round step 3: the next pass
 *             starts after the kept tokens). A loop that keeps its cache
 *             length here passes the same pointer to kv_nest_append,
 *             kv_nest_attend and nest_rope_split.
 *   next      int32 [B] (out, nullable): t_a, the last emitted token, which
 *             is the next round's slot-0 input
 *   ws        verify_accept_workspace_size(B, k, V) bytes, zeroed before
 *             first use (per-block partial maxima and the last-block
 *             counter).
 * Up to 16 rows, one launch: the argmax is fused into the GEMV and its
 * last block applies the rule. More rows (several sequences, or k >= 16):
 * the batched verify kernel writes y (required then), one block per row
 * takes its argmax with the same tie rule (the lowest index), and one
 * thread per sequence applies the rule; the fp32 fold then adds the group
 * sums in the batched kernel's order, so a target can differ from the
 * fused path's only where a row's two largest logits are within the
 * fold's rounding of each other.
 * Requires B >= 1, k >= 0, B*(k+1) <= 65535, group == 128, K % 128 == 0.
 * Draft ids are not read on the host, so an id outside [0, V) simply
 * never matches. Errors: NEST_EINVAL, NEST_EALIGN, NEST_ESHAPE,
 * NEST_EUNSUPPORTED, NEST_EWORKSPACE, NEST_EHIP. */
int verify_accept(const int8_t* qa, const float* sa, int64_t B, int64_t k,
                  int64_t K, const uint8_t* base, const uint8_t* refine,
                  const float* scales, int64_t V, int64_t group,
                  const int32_t* draft, int32_t* target, int32_t* n_emitted,
                  int32_t* emitted, float* y, int32_t* len, int32_t* next,
                  void* ws, size_t ws_bytes, void* stream);
size_t verify_accept_workspace_size(int64_t B, int64_t k, int64_t V);

/* verify_accept_x -- verify_accept on fp32 activations x [B*(k+1)][K]
 * (16-byte aligned), quantized in the kernel as for draft_gemv_x
 * (bit-identical to nest_act_quant + verify_accept); when
 * B*(k+1)*K > 131072 the activations are first quantized into the
 * workspace, of nest_gemv_x_workspace_size(B*(k+1), K, V) bytes (zeroed
 * before first use). Errors: as verify_accept. */
int verify_accept_x(const float* x, int64_t B, int64_t k, int64_t K,
                    const uint8_t* base, const uint8_t* refine,
                    const float* scales, int64_t V, int64_t group,
                    const int32_t* draft, int32_t* target, int32_t* n_emitted,
                    int32_t* emitted, float* y, int32_t* len, int32_t* next,
                    void* ws, size_t ws_bytes, void* stream);

/* verify_accept_x_static -- verify_accept_x with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). The workspace is a
 * device array inside the library, 1 MiB per device, held from the first
 * call on a device until the process ends. It allocates and frees nothing. The call needs
 * nest_gemv_x_workspace_size(B*(k+1), K, V) <= 1 MiB (the 152064-row LM
 * head with up to 16 rows of K = 3584 needs 362 KB); a larger one returns
 * NEST_EUNSUPPORTED before anything runs. All calls on one device share the array, so calls
 * that overlap in time on one device (different streams, or threads
 * without ordering) race; calls on one stream are ordered and safe.
 * Arguments and errors otherwise as verify_accept_x. */
int verify_accept_x_static(const float* x, int64_t B, int64_t k, int64_t K,
                           const uint8_t* base, const uint8_t* refine,
                           const float* scales, int64_t V, int64_t group,
                           const int32_t* draft, int32_t* target,
                           int32_t* n_emitted, int32_t* emitted, float* y,
                           int32_t* len, int32_t* next, void* stream);

/* Nested KV cache: a host struct holding device pointers (layouts above). */
typedef struct nest_kv {
  const uint8_t* k_base;   /* [Hkv][capacity][d/2] bytes             */
  const uint8_t* k_refine; /* same shape; may be NULL for view 0     */
  const float* k_scale;    /* [Hkv][capacity/block]                  */
  const uint8_t* v_base;   /* [Hkv][capacity/block][d][block/2] bytes */
  const uint8_t* v_refine; /* same shape; may be NULL for view 0     */
  const float* v_scale;    /* [Hkv][capacity/block]                  */
  int64_t n_kv_heads;      /* Hkv                                    */
  int64_t head_dim;        /* d                                      */
  int64_t capacity;        /* tokens the planes hold                 */
  int64_t block;           /* tokens per quantization group          */
} nest_kv;

/* kv_nest_pack -- build a nested KV cache from fp32 K and V (BitNest,
 * Figure 4), with the same quantization rule as nest_pack. One group is a
 * (head, block).
 *   k, v     fp32 [Hkv][capacity][d], token-major
 *   k_base, k_refine, v_base, v_refine  (out) planes in the layouts above
 *   k_scale, v_scale  fp32 [Hkv][capacity/block] (out)
 * Requires capacity % block == 0, even block, even d.
 * Errors: NEST_EINVAL, NEST_ESHAPE, NEST_EHIP. */
int kv_nest_pack(const float* k, const float* v, int64_t n_kv_heads,
                 int64_t capacity, int64_t head_dim, int64_t block,
                 uint8_t* k_base, uint8_t* k_refine, float* k_scale,
                 uint8_t* v_base, uint8_t* v_refine, float* v_scale,
                 void* stream);

/* kv_nest_append -- write n new tokens' fp32 K and V at positions
 * pos .. pos+n-1 of the nested cache and quantize again every block they
 * touch (BitNest, Figure 4: accepted entries are retained; the rejected
 * suffix is discarded by the caller's length update and overwritten by the
 * next append at the same positions).
 *   kv        the cache; the planes and scales of the touched blocks are
 *             written (through the pointers in *kv)
 *   shadow_k, shadow_v  fp32 [Hkv][2][block][d] each: the values of the two
 *             most recent blocks, block b in slot b % 2. On entry, slot
 *             (pos/block) % 2 must hold tokens block*floor(pos/block) .. pos-1
 *             (kv_nest_shadow_fill sets this up after a prefill); the call
 *             keeps it so for the next append at any pos' in
 *             (floor(pos/block)*block, pos+n].
 *   k_new, v_new  fp32 [Hkv][n][d]
 *   pos_dev   int32 (device, nullable): when given, the first position is
 *             *pos_dev + pos, read by the kernel; an append that would then
 *             start below 0 or end past capacity writes nothing
 *   pos, n    host values: the first position (or its offset from
 *             *pos_dev) and the token count; 1 <= n <= block, and without
 *             pos_dev pos >= 0, pos + n <= capacity
 * A touched block with L valid tokens (those before pos + n) is quantized as
 * kv_nest_pack quantizes a block whose tokens from L on are 0: its scale
 * covers the valid tokens only and the padding codes are 0; a block that
 * fills equals kv_nest_pack of its tokens. Blocks outside the touched range
 * are not written.
 * Errors: NEST_EINVAL, NEST_ESHAPE, NEST_EUNSUPPORTED, NEST_EHIP. */
int kv_nest_append(const nest_kv* kv, float* shadow_k, float* shadow_v,
                   const float* k_new, const float* v_new, const int32_t* pos_dev,
                   int64_t pos, int64_t n, void* stream);
size_t kv_nest_shadow_floats(int64_t n_kv_heads, int64_t head_dim,
                             int64_t block); /* per shadow (K or V); 0 if invalid */

/* kv_nest_shadow_fill -- after a prefill: copy the open block's tokens
 * block*floor(ctx_len/block) .. ctx_len-1 of each head from fp32 K and V
 * [Hkv][src_len][d] into their shadow slot (nothing when ctx_len is a
 * multiple of block). Errors: NEST_EINVAL, NEST_ESHAPE, NEST_EHIP. */
int kv_nest_shadow_fill(const nest_kv* kv, const float* k, const float* v,
                        int64_t src_len, int64_t ctx_len, float* shadow_k,
                        float* shadow_v, void* stream);

/* kv_nest_attend -- decode attention over the nested cache (BitNest,
 * Figure 4). view 0 is the base view, which the draft uses and which reads
 * only the base planes. view 1 is the full view, which verification uses
 * and which reads both planes.
 *   q        bf16 bit patterns [nq][Hq][d]
 *   kv       host pointer to a nest_kv
 *   ctx_dev  int32 (device, nullable): when given, the visible length is
 *            *ctx_dev + ctx_len, read by the kernels and clamped into
 *            [nq, capacity]; the grid then covers the whole capacity
 *   ctx_len  host value: the visible cache length, nq <= ctx_len <=
 *            capacity (or, with ctx_dev, the offset added to it,
 *            0 <= ctx_len <= capacity)
 *   out      fp32 [nq][Hq][d] (out)
 *   ws       kv_nest_attend_workspace_size(nq, Hq, Hkv, d, L) bytes with
 *            L = ctx_len, or L = capacity when ctx_dev is given (no
 *            zero-fill needed)
 * Requires head_dim == 128, block == 128, Hq % Hkv == 0,
 * 1 <= Hq/Hkv <= 64, and 16-byte aligned planes and q. Up to 64 query
 * rows per kv head (nq*(Hq/Hkv)) run in one launch of the attention and
 * one of the merge; more are taken in chunks of 64/(Hq/Hkv) queries, each
 * chunk launched as the call of those queries alone (the same positions,
 * hence the same results), the chunks sharing the workspace in turn.
 * Errors: NEST_EINVAL, NEST_EALIGN, NEST_ESHAPE, NEST_EUNSUPPORTED,
 * NEST_EWORKSPACE, NEST_EHIP. */
int kv_nest_attend(const uint16_t* q, int64_t nq, int64_t n_q_heads,
                   const nest_kv* kv, const int32_t* ctx_dev, int64_t ctx_len,
                   int view, float* out, void* ws, size_t ws_bytes,
                   void* stream);
/* kv_nest_attend_exact -- the k+1 queries of one verify pass, each seeing
 * the cache exactly as a one-token pass at its own position would ("How
 * Speculative Decoding Speeds Up Inference", section "Drafting and checking
 * tokens", step 2: one pass checks every position; section "The same
 * output as the large model alone"), in one call.
 * Query i (position p_i = L - nq + i, L the visible length) sees tokens
 * 0..p_i. The block holding p_i is taken as kv_nest_append would have
 * quantized it after a one-token append at p_i: from its fp32 values in
 * the shadows, over its tokens up to p_i only; every earlier block comes
 * from the planes. Each query's output is bit-identical to kv_nest_attend
 * with that one query at length p_i + 1 (same view, same ctx_dev use) when
 * both split the context alike, which they always do when the length is on
 * the device. Call it after kv_nest_append of the nq new tokens: the
 * append leaves every token of the (at most two) blocks they touch in the
 * shadows and seals a block they fill.
 *   shadow_k, shadow_v  the kv_nest_append shadows of this cache
 *   ws       kv_nest_attend_exact_workspace_size(nq, Hq, Hkv, d, L) bytes
 *            (L as for kv_nest_attend): the chunk partials, then one
 *            rebuilt open block (both planes of K and V, 32 KB) and its two
 *            scales per (query, kv head); no zero-fill needed
 *   the rest as for kv_nest_attend.
 * Three launches: the open blocks are rebuilt into the workspace, then
 * one attention kernel serves all queries (as many queries per workgroup
 * as their GQA groups fit in 16 rows), then the chunk partials are merged.
 * With nq == 1 the call is kv_nest_attend's (the append already quantized
 * the block over the tokens up to the query).
 * Requires Hq/Hkv <= 16 and nq <= block; all nq queries go through one
 * attention launch, whatever nq*(Hq/Hkv). Errors: as kv_nest_attend. */
int kv_nest_attend_exact(const uint16_t* q, int64_t nq, int64_t n_q_heads,
                         const nest_kv* kv, const float* shadow_k,
                         const float* shadow_v, const int32_t* ctx_dev,
                         int64_t ctx_len, int view, float* out, void* ws,
                         size_t ws_bytes, void* stream);

/* kv_nest_append_attend_exact -- a verify pass's append and exact attention
 * in one call (the same two steps of "How Speculative Decoding Speeds Up
 * Inference", "Drafting and checking tokens", step 2): the result, the
 * planes, scales and shadows afterwards are bit-identical to
 *   kv_nest_append(kv, shadow_k, shadow_v, k_new, v_new, pos_dev, pos, n)
 *   kv_nest_attend_exact(q, n, Hq, kv, shadow_k, shadow_v, pos_dev, pos + n, ...)
 * on the same stream, with one launch fewer: the append's codes, scales and
 * shadow rows are written by the kernel that rebuilds the queries' open
 * blocks, which reads the new tokens from k_new / v_new.
 *   k_new, v_new  fp32 [Hkv][n][d], 16-byte aligned: the n new tokens at
 *                 positions pos .. pos + n - 1 (plus *pos_dev when given)
 *   q             bf16 bits [n][Hq][d]: query i at position pos + i
 *   the rest as for kv_nest_attend_exact with nq = n and ctx_len = pos + n;
 *   ws is kv_nest_attend_exact_workspace_size(n, Hq, Hkv, d, L).
 * With a device position whose append would not fit in the capacity,
 * nothing is appended (as kv_nest_append) and the queries attend as
 * kv_nest_attend_exact would after it. With n == 1: the append, then
 * kv_nest_attend's one-query launch (no launch is saved).
 * Requires 1 <= n <= block, pos + n <= capacity without pos_dev and
 * -capacity <= pos <= capacity, pos + n >= 0 with it; both refinement
 * planes. Errors: as kv_nest_attend_exact. */
int kv_nest_append_attend_exact(const uint16_t* q, int64_t n, int64_t n_q_heads,
                                const nest_kv* kv, float* shadow_k,
                                float* shadow_v, const float* k_new,
                                const float* v_new, const int32_t* pos_dev,
                                int64_t pos, int view, float* out, void* ws,
                                size_t ws_bytes, void* stream);

size_t kv_nest_attend_workspace_size(int64_t nq, int64_t n_q_heads,
                                     int64_t n_kv_heads, int64_t head_dim,
                                     int64_t ctx_len);
/* Bytes of kv_nest_attend_exact's workspace; 0 for an unsupported shape. */
size_t kv_nest_attend_exact_workspace_size(int64_t nq, int64_t n_q_heads,
                                           int64_t n_kv_heads,
                                           int64_t head_dim, int64_t ctx_len);

/* ---------------------------------------------------------------------------
 * Speculative sampling ("How Speculative Decoding Speeds Up Inference",
 * section "The same output as the large model alone", and the method of
 * Leviathan et al. and Chen et al. it names). Scores are softmax(y / T) of
 * fp32 logits y; a draw with uniform u takes the smallest id whose running
 * weight exceeds u times the total weight (inverse CDF). The uniforms are
 * inputs, so a caller owns the random stream. Arithmetic is fp32; a draw
 * whose target lies within rounding of an id boundary may take either id.
 * Logits must be finite or -inf (a masked id), with at least one finite
 * value per row. Device pointers unless stated; the calls are asynchronous
 * on `stream`, and the workspace needs no zero-fill.
 * --------------------------------------------------------------------------- */

/* nest_sample -- one id per row from softmax(y / T).
 *   y            fp32 [M][V] logits
 *   M, V         host values: rows (1..65535) and vocabulary (<= 8388608)
 *   temperature  host value, > 0
 *   u            fp32 [M] uniforms in [0, 1)
 *   tokens       int32 [M] (out)
 *   ws           nest_sample_workspace_size(M, V) bytes, 16-byte aligned
 * Errors: NEST_EINVAL, NEST_EUNSUPPORTED, NEST_EWORKSPACE, NEST_EALIGN,
 * NEST_EHIP. */
int nest_sample(const float* y, int64_t M, int64_t V, float temperature,
                const float* u, int32_t* tokens, void* ws, size_t ws_bytes,
                void* stream);
size_t nest_sample_workspace_size(int64_t M, int64_t V);

/* verify_sample -- the accept test and last draw of B speculative rounds.
 * Slot i (1..k) of sequence b keeps its draft d_i while
 * u_acc * q_i(d_i) < p_i(d_i), i.e. with probability min(1, p/q); at the
 * first slot that fails, the last id is drawn with u_fin from
 * max(0, p_i - q_i) normalized (from p_i itself if rounding leaves that
 * without mass); when all k are kept, from p_{k+1} (the bonus).
 *   yt       fp32 [B][k+1][V]: the target's logits; row i-1 scores slot i,
 *            row k the bonus position
 *   yd       fp32 [B][k][V]: the draft logits each d_i was drawn from
 *            (may be NULL when k == 0)
 *   B, k, V  host values: 1 <= B, 0 <= k <= 32, B*(2k+1) <= 65535,
 *            V <= 8388608
 *   temperature  host value, > 0: the same T for both models
 *   draft    int32 [B][k]; an id outside [0, V) is never kept
 *   u_acc    fp32 [B][k] uniforms of the accept tests
 *   u_fin    fp32 [B] uniforms of the last draws
 *   n_emitted  int32 [B] (out): kept drafts + 1
 *   emitted    int32 [B][k+1] (out): the kept drafts, the drawn id, then -1
 *   ws       verify_sample_workspace_size(B, k, V) bytes, 16-byte aligned
 * Errors: NEST_EINVAL, NEST_EUNSUPPORTED, NEST_EWORKSPACE, NEST_EALIGN,
 * NEST_EHIP. */
int verify_sample(const float* yt, const float* yd, int64_t B, int64_t k,
                  int64_t V, float temperature, const int32_t* draft,
                  const float* u_acc, const float* u_fin, int32_t* n_emitted,
                  int32_t* emitted, void* ws, size_t ws_bytes, void* stream);
size_t verify_sample_workspace_size(int64_t B, int64_t k, int64_t V);

/* ---------------------------------------------------------------------------
 * Decoder glue for running rounds end to end through a small synthetic
 * pre-norm decoder ("How Speculative Decoding Speeds Up Inference", section
 * "The same output as the large model alone": greedy speculation keeps only
 * the target's own top choices). The pages define none of these layers;
 * they are the plain Llama/Qwen-style ones. Every output row depends only
 * on its own input row and is computed in a fixed order, so a position is
 * bit-identical whether it runs alone or inside a batch. fp32, device
 * pointers, asynchronous on `stream`.
 * --------------------------------------------------------------------------- */

/* out [M][H] = table [V][H] rows at tokens [M] (int32); an id outside
 * [0, V) gives a zero row. Errors: NEST_EINVAL, NEST_EUNSUPPORTED, NEST_EHIP. */
int nest_embed(const float* table, int64_t V, int64_t H, const int32_t* tokens,
               int64_t M, float* out, void* stream);

/* Residual add and RMSNorm: when y is non-NULL, x += y (x is written);
 * then out = x / sqrt(mean(x^2) + eps) * gamma, per row of x [M][H].
 * out may not alias x. Errors: NEST_EINVAL, NEST_EUNSUPPORTED, NEST_EHIP. */
int nest_add_rmsnorm(float* x, const float* y, const float* gamma, int64_t M,
                     int64_t H, float eps, float* out, void* stream);

/* Rotary embedding and q/k/v split of a QKV projection qkv
 * [M][(Hq + 2 Hkv) * d] (q heads, then k heads, then v heads). Row m is at
 * position p_m = pos0 + m, plus *pos_dev when pos_dev (device int32,
 * nullable) is given; pair (i, i + d/2) of a q or k head is rotated by
 * p_m * theta^(-2i/d) (rotate-half convention). Outputs: q as bf16
 * bit patterns [M][Hq][d] (nearest, ties to even), ready for
 * kv_nest_attend; k and v fp32, laid out [Hkv][M][d] (token_major = 0, the
 * kv_nest_append layout for M tokens) or [M][Hkv][d] (token_major = 1, so
 * that each token's slice is a [Hkv][1][d] append). d even, theta > 1.
 * Errors: NEST_EINVAL, NEST_EUNSUPPORTED, NEST_EHIP. */
int nest_rope_split(const float* qkv, int64_t M, const int32_t* pos_dev, int64_t pos0,
                    int64_t n_q_heads, int64_t n_kv_heads, int64_t head_dim,
                    float theta, int token_major, uint16_t* q, float* k,
                    float* v, void* stream);

/* SwiGLU: out [M][I] = silu(g) * u with gate_up [M][2I] = [g | u] per row
 * and silu(g) = g / (1 + exp(-g)). Errors: NEST_EINVAL, NEST_EUNSUPPORTED,
 * NEST_EHIP. */
int nest_swiglu(const float* gate_up, int64_t M, int64_t I, float* out,
                void* stream);

/* ---------------------------------------------------------------------------
 * Choosing the draft length ("How Speculative Decoding Speeds Up Inference",
 * section "Tokens per pass and time per token"). Host functions: every
 * pointer is a host pointer and nothing runs on the GPU.
 * --------------------------------------------------------------------------- */

/* Eq. (1): expected tokens per pass, E = (1 - alpha^(k+1)) / (1 - alpha)
 * (k + 1 at alpha = 1). NaN for alpha outside [0, 1] or k < 0. */
double nest_expected_tokens(double alpha, int64_t k);

/* Eq. (2): time per token, (t_pass + k * t_draft) / E(alpha, k). */
double nest_token_time(double alpha, int64_t k, double t_draft, double t_pass);

/* The k in [0, kmax] with the least time per token, given the time of one
 * draft step t_draft and the pass times t_pass[0..kmax] (host array; the
 * pass with k draft tokens checks k+1 positions). Ties keep the smaller k.
 * Writes that time to *t_token when non-NULL. Returns -1 on bad arguments
 * (message in nest_last_error). */
int64_t nest_choose_k(double alpha, double t_draft, const double* t_pass,
                      int64_t kmax, double* t_token);

/* Running acceptance rate. A round that kept a of k drafts judged a + 1
 * slots when a < k (a accepted, one rejected) and k slots when a == k (all
 * accepted), independently per slot as Eq. (1) assumes; the estimate is
 * accepted over judged slots, older rounds weighted by decay^(age) and the
 * prior counting as judged slots before the first round. */
typedef struct nest_alpha {
  double accepted; /* weighted accepted slots */
  double rejected; /* weighted rejected slots */
  double decay;    /* weight kept per round, in [0, 1] */
} nest_alpha;
void nest_alpha_init(nest_alpha* st, double decay, double prior_accepted,
                     double prior_rejected);
void nest_alpha_update(nest_alpha* st, int64_t accepted, int64_t k);
double nest_alpha_value(const nest_alpha* st);

/* ---------------------------------------------------------------------------
 * Calibration
 * --------------------------------------------------------------------------- */

/* nest_read_stream -- read `bytes` of device memory once as a plain stream
 * (16-byte nontemporal loads, as the weight and cache streams use; each
 * wave reads whole 16 KB chunks, the fastest pattern measured). *sink
 * is written only if a thread's folded word equals a fixed constant, which
 * keeps the loads live without contended writes. Its rate is what a kernel
 * that reads each byte once can reach on the device: the "achievable"
 * bandwidth the kernels' roofline fractions are also quoted against.
 *   src   device, 16-byte aligned;  bytes  a positive multiple of 16
 *   sink  uint32 (device)
 * Errors: NEST_EINVAL, NEST_ESHAPE, NEST_EALIGN, NEST_EHIP. */
int nest_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NESTSPEC_H */
