/*
 * bd.h - C ABI of the block-diffusion denoise-step library (libbd.so, gfx950).
 *
 * One denoising step of a block-diffusion VLM decoder, plus the companion
 * calls of linear self-speculative decoding.  The operations follow:
 *
 *  [FD]  "Fast-dVLM" write-up (itsolotime.com): section 4.1 (causal-context
 *        attention: a noisy block attends to itself bidirectionally and to
 *        every earlier clean position, vision included), section 5.1 (each
 *        block opens with an AR step), section 5.3 (linear self-speculative
 *        decoding: bidirectional draft, causal verify, accept the longest
 *        prefix that matches the AR prediction, crop the KV cache).
 *  [FD2] Fast-dVLM summary page, Fig. 3 caption (M_N2N block-diagonal mask).
 *  [DV]  "DiffusionVL" notes (papernotes.org): cached block decoding and
 *        Algorithm 1 as restated there (confidence = probability of the
 *        chosen token; commit the k = min(ceil(D/S), |M|) most confident
 *        masked positions plus, under the dynamic rule, every masked
 *        position whose confidence is greater than tau; committed tokens stay
 *        as context; a finished block joins the KV cache).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `stream` and the descriptors is a DEVICE
 *    pointer, 16-byte aligned, owned by the caller.  The library allocates no
 *    memory and keeps no state beyond a thread-local last HIP error.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and performs no host synchronisation.  Lengths that change on
 *    the device (prefix lengths, accepted lengths) stay on the device.
 *  - Host-side validation happens before anything is launched: on a bad
 *    argument the call returns a non-zero bd_status and touches nothing.
 *    BD_E_LAUNCH means the HIP runtime rejected a launch (bd_last_hip_error()).
 *  - Workspaces: size them with the matching *_workspace_bytes() call and
 *    zero-fill them once before first use.  Each call leaves the counter area
 *    it uses (for the confidence and verify calls: the whole workspace)
 *    zeroed again, so later calls with the same descriptor on the same
 *    stream can reuse the workspace.  The counter area's place depends on the
 *    descriptor: a workspace used with another descriptor, or for anything
 *    else, must be zero-filled again before such a call.  Calls that overlap
 *    in time must not share a workspace.
 *  - bf16 data is raw 16-bit storage (round-to-nearest-even when produced).
 *    Accumulation is fp32.  Results do not depend on scheduling: every
 *    reduction runs in a fixed order.  bd_attn_step may split a long
 *    context into key ranges; each range's normalised partial output is
 *    exchanged through the workspace rounded to bf16 (its max and sum stay
 *    fp32) and merged by a second kernel on the same stream.
 *
 * Layouts (row-major, innermost index last):
 *    q, out     [n][D][Hq][d]        queries / outputs of every block slot
 *    k_blk,v_blk[n][D][Hkv][d]       this step's block keys / values
 *    k_cache    [n][Hkv][cap][d]     frozen keys of prompt and finished blocks
 *    v_cache    [n][Hkv][cap][d]     frozen values of the same positions
 *    prefix_len int32[n]             valid cache length of each item (device)
 *    logits     f32[n_req][D][V]
 *    masked     u8[n_req][D]         1 = still [MASK]
 *    tokens     i32[n_req][D]        committed token ids
 */
#ifndef BD_H
#define BD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bd_status;
#define BD_OK 0
#define BD_E_NULL 1      /* a required pointer is NULL */
#define BD_E_SHAPE 2     /* a size is out of range or inconsistent */
#define BD_E_DTYPE 3     /* unknown or unsupported dtype */
#define BD_E_PARAM 4     /* unknown mode, S < 1, NaN tau or scale, ... */
#define BD_E_WORKSPACE 5 /* workspace missing or too small */
#define BD_E_LAUNCH 6    /* the HIP runtime rejected a launch */
#define BD_E_SCRATCH 7   /* bd_attn_step_noalloc: the call needs more than its fixed scratch */

enum { BD_F32 = 0, BD_BF16 = 1, BD_FP8KV = 2 };
enum { BD_BLOCK_BIDIR = 0, BD_BLOCK_CAUSAL = 1, BD_BLOCK_QUAD = 2 };
/* Plan flag, or-ed into bd_attn_desc.mode: the batch is ragged (items with
 * different prefix lengths).  With at most 64 items, bd_attn_step then sizes
 * each item's key splits from the device-side prefix lengths, so that every
 * split of the call carries about the same number of keys; otherwise the
 * split plan follows max_prefix alone (a short item then gets few splits and
 * part of the GPU idles while the long ones finish).  Same results within the
 * bf16 bar (the splits, hence the rounding of the exchange, differ); results
 * still do not depend on scheduling.  Ignored beyond 64 items, by the vector
 * (BD_F32) path and by bd_kv_append. */
#define BD_PLAN_BALANCED 0x100

/* Shape of one block-attention call.
 *  n_items    independent (request, layer) items, >= 1
 *  D          block length, 1..64 (BD_BLOCK_QUAD: the draft block size B, 1..32)
 *  Hq, Hkv    query / KV heads, Hq % Hkv == 0; head h uses KV head h / (Hq/Hkv)
 *  d          head dim, 64 or 128
 *  cap        cache capacity in tokens, >= 1
 *  dtype      BD_BF16 (MFMA path), BD_F32 (vector path) or BD_FP8KV (bf16
 *             queries and outputs, E4M3 keys and values: bd_attn_step_fp8kv)
 *  mode       BD_BLOCK_BIDIR, BD_BLOCK_CAUSAL or BD_BLOCK_QUAD, optionally | BD_PLAN_BALANCED
 *  max_prefix host-side upper bound of every prefix_len[i], 0..cap; sizes the grid
 *             (and, for bf16 caches, the first tile copies a workgroup issues
 *             before the device-side lengths arrive)
 *  scale      softmax scale (normally 1/sqrt(d)); finite and > 0
 * Size limits (BD_E_SHAPE otherwise), with S = block slots per item (D, or
 * B (B + 3) / 2 for BD_BLOCK_QUAD): S * Hq <= 2^20, cap * d <= 2^30, and the
 * launch fits 32-bit grids: n_items * Hkv * ceil(S * (Hq/Hkv) / 128) <
 * 2^31 / 64 and n_items * S * Hq / 4 < 2^31. */
typedef struct {
    int32_t n_items, D, Hq, Hkv, d, cap, dtype, mode, max_prefix;
    float scale;
} bd_attn_desc;

/* Shape of one confidence + commit call.
 *  n_req >= 1, D 1..64, V >= 2, S >= 1 denoising steps per block,
 *  tau threshold (not NaN; tau >= 1 disables the threshold rule). */
typedef struct {
    int32_t n_req, D, V, S;
    float tau;
} bd_commit_desc;

/* Workspace bytes bd_attn_step needs for `desc` (0 if none); SIZE_MAX if desc is invalid. */
size_t bd_attn_workspace_bytes(const bd_attn_desc *desc);

/* Block attention of one denoising step ([FD] 4.1, 5.1, 5.3; [FD2] Fig. 3).
 * For item i with P = prefix_len[i], slot s < D and head h (KV head g):
 *   keys/values are cache positions 0..P-1 followed by block slots 0..D-1;
 *   BD_BLOCK_BIDIR  : slot s sees all P + D of them (denoise step);
 *   BD_BLOCK_CAUSAL : slot s sees cache 0..P-1 and block slots 0..s (verify / AR step);
 *   BD_BLOCK_QUAD   : quadratic self-speculative step ([FD] 5.3, the quadratic variant:
 *                     verify fused with the next block's draft).  With B = desc->D the
 *                     block holds S = B (B + 3) / 2 slots: slots 0..B-1 are the B draft
 *                     tokens, then for g = 0..B-1 the B - g mask tokens of group g (the
 *                     next-block proposal under the hypothesis that drafts 0..g-1 are
 *                     accepted).  Every slot sees cache 0..P-1; draft t sees drafts
 *                     0..t; a mask token of group g sees drafts 0..g-1 and every mask
 *                     token of group g.  (The B x B expansion of the pages, with each
 *                     draft token's K/V held once since it is the same in every group.)
 *                     q, out, k_blk, v_blk then have S slots per item instead of D.
 *   out = softmax(scale * q k^T) v over the visible keys.
 * Cache positions >= P are never read.  `out` has the input dtype.
 * Preconditions (device): 0 <= prefix_len[i] <= max_prefix.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_PARAM, BD_E_WORKSPACE, BD_E_LAUNCH. */
bd_status bd_attn_step(const bd_attn_desc *desc, const void *q, const void *k_blk,
                       const void *v_blk, const void *k_cache, const void *v_cache,
                       const int32_t *prefix_len, void *out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* bd_attn_step for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments, results and errors as bd_attn_step (BD_F32 / BD_BF16,
 * every mode), with no workspace argument.  The split-K exchange goes through
 * a fixed device array of BD_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * nothing and calls no allocating routine.
 *  - A call whose workspace (bd_attn_workspace_bytes) exceeds that size
 *    returns BD_E_SCRATCH before anything is launched.
 *  - The array's address on a device is looked up on the first call on that
 *    device (hipGetSymbolAddress); `stream` must belong to the current device
 *    (BD_E_LAUNCH otherwise).  Nothing in the array needs to start at zero.
 *  - Every call on one GPU shares that GPU's array: calls that overlap in time
 *    on one GPU (on different streams, or from different threads) race and
 *    give wrong results.  Calls in order on one stream are safe. */
#define BD_NOALLOC_SCRATCH_BYTES (64u << 20)
bd_status bd_attn_step_noalloc(const bd_attn_desc *desc, const void *q, const void *k_blk,
                               const void *v_blk, const void *k_cache, const void *v_cache,
                               const int32_t *prefix_len, void *out, void *stream);

/* BD_NOALLOC_SCRATCH_BYTES, as the library was built. */
size_t bd_attn_noalloc_max_scratch_bytes(void);

/* Block attention over an FP8 KV cache (desc->dtype == BD_FP8KV).  The same
 * operation, masks and layouts as bd_attn_step (for BD_FP8KV,
 * bd_attn_workspace_bytes sizes its workspace), with keys and values stored
 * as one byte each in OCP FP8 E4M3 (bias 7, no infinities, 0x7F / 0xFF NaN;
 * the FP8 rung of [FD] 5.4 and Table 4, applied here to the cache):
 *   key   = e4m3(k_cache or k_blk byte) * k_scale[i][g]
 *   value = e4m3(v_cache or v_blk byte) * v_scale[i][g]
 * for item i and KV head g.  q and out are bf16 [n][D][Hq][d].
 *   k_blk, v_blk   u8 [n][D][Hkv][d]      k_cache, v_cache u8 [n][Hkv][cap][d]
 *   k_scale, v_scale f32 [n][Hkv] (device)
 * E4M3 values are widened to bf16 exactly; products and sums are fp32, the
 * attention weights bf16, as in bd_attn_step.  Every k_scale and v_scale
 * entry must be finite and > 0 (device values, not checked).
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE (dtype != BD_FP8KV), BD_E_PARAM,
 * BD_E_WORKSPACE, BD_E_LAUNCH.  bd_attn_step rejects BD_FP8KV with BD_E_DTYPE. */
bd_status bd_attn_step_fp8kv(const bd_attn_desc *desc, const void *q, const void *k_blk,
                             const void *v_blk, const void *k_cache, const void *v_cache,
                             const float *k_scale, const float *v_scale, const int32_t *prefix_len,
                             void *out, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes bd_confidence_commit needs; SIZE_MAX if desc is invalid. */
size_t bd_commit_workspace_bytes(const bd_commit_desc *desc);

/* Confidence + commit of one denoising step ([DV] cached block decoding, Algorithm 1).
 * For each request r and masked slot i (masked[r][i] == 1):
 *   a_i = argmax_v logits[r][i][v] (lowest index on ties), conf_i = softmax(logits[r][i])[a_i];
 *   k = min(ceil(D/S), |M|); T = the k masked slots first in (conf desc, index asc);
 *   commit C = T u { i in M : conf_i > tau }: tokens[r][i] = a_i, masked[r][i] = 0.
 * Rows of unmasked slots are not read; their tokens and masked flags do not change.
 * masked and tokens are updated in place.  Optional outputs (NULL to skip):
 *   conf f32[n_req][D] (NaN at unmasked slots), argmax i32[n_req][D] (-1 at unmasked),
 *   committed u8[n_req][D] (1 where committed now), n_committed i32[n_req].
 * NaN logits are not supported (results unspecified).
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_PARAM, BD_E_WORKSPACE, BD_E_LAUNCH. */
bd_status bd_confidence_commit(const bd_commit_desc *desc, const float *logits, uint8_t *masked,
                               int32_t *tokens, float *conf, int32_t *argmax, uint8_t *committed,
                               int32_t *n_committed, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Workspace bytes bd_spec_verify needs; SIZE_MAX if the sizes are invalid. */
size_t bd_verify_workspace_bytes(int32_t n_req, int32_t D, int32_t V);

/* Speculative verify ([FD] 5.3, linear variant).  Row i of request r holds the
 * causal pass's logits for draft slot i (the caller aligns rows and slots).
 *   a_i = argmax_v logits[r][i][v] (lowest index on ties);
 *   accepted_len[r] = first i with a_i != draft[r][i], or D if none.
 * argmax (optional, i32[n_req][D]) receives every a_i, so a caller can take
 * a_L as the next token.  All D rows are read.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_WORKSPACE, BD_E_LAUNCH. */
bd_status bd_spec_verify(int32_t n_req, int32_t D, int32_t V, const float *logits,
                         const int32_t *draft, int32_t *accepted_len, int32_t *argmax,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Append accepted block K/V to the cache ([FD] 5.3: crop the cache to the accepted
 * prefix; [DV] a finished block joins the history cache).  Uses n_items, D, Hkv, d,
 * cap, dtype and mode of `desc`.  For item i with P = prefix_len[i] and
 * L = n_accept ? n_accept[i] : D (device values): cache slots P..P+L-1 receive block
 * slots 0..L-1 bit for bit (one d-element row per slot and KV head, keys and
 * values alike) and prefix_len[i] becomes P + L.  Nothing else is written.
 *  - BD_FP8KV: the E4M3 bytes are copied; they share the cache's per-(item, KV head)
 *    scales.
 *  - BD_BLOCK_QUAD: k_blk / v_blk hold B (B + 3) / 2 slots per item (the layout of
 *    that mode) and L <= B accepted drafts, slots 0..L-1, are appended.
 * If L is outside 0..D or P + L > cap, item i is left untouched and *dev_err
 * (optional device int32) is set to 1.
 * Size limits (BD_E_SHAPE otherwise): cap * d <= 2^30 and, with S block slots
 * per item, S * Hkv * d <= 2^30.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_PARAM (a pointer not 16-byte
 * aligned), BD_E_LAUNCH. */
bd_status bd_kv_append(const bd_attn_desc *desc, void *k_cache, void *v_cache,
                       int32_t *prefix_len, const void *k_blk, const void *v_blk,
                       const int32_t *n_accept, int32_t *dev_err, void *stream);

/* Shape of one LM-head + confidence + commit call.
 *  R = n_req * D block slots (1..16 in total, D 1..64), vocabulary V >= 2,
 *  hidden size H (a multiple of 256, at most 4096), S >= 1, tau not NaN. */
typedef struct {
    int32_t n_req, D, V, H, S;
    float tau;
} bd_lmhead_desc;

/* Workspace bytes bd_lmhead_confidence_commit needs; SIZE_MAX if desc is invalid. */
size_t bd_lmhead_workspace_bytes(const bd_lmhead_desc *desc);

/* The vocabulary projection that produces a denoising step's logits, fused with
 * that step's confidence + commit ([DV] cached block decoding: the confidence is
 * the model's probability of the chosen token, then Algorithm 1's commit rule).
 *   logits[r][i][v] = sum_h hidden[r][i][h] * weight[v][h]  (bf16 inputs, fp32 sums),
 * followed by exactly the confidence + commit of bd_confidence_commit on those
 * logits (same outputs, same rules).  The logits themselves never reach memory.
 *   hidden  bf16 [n_req][D][H]   final hidden state of every block slot
 *   weight  bf16 [V][H]          the vocabulary projection (a linear layer's weight)
 * Every slot's logits are formed (the weight is read once for all of them);
 * only masked slots take part in the confidence and the commit.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_PARAM, BD_E_WORKSPACE, BD_E_LAUNCH. */
bd_status bd_lmhead_confidence_commit(const bd_lmhead_desc *desc, const void *hidden, const void *weight,
                                      uint8_t *masked, int32_t *tokens, float *conf, int32_t *argmax,
                                      uint8_t *committed, int32_t *n_committed, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* Shape of one two-stream training-attention call ([FD] 4.1, 4.3, 4.4; [FD2] Fig. 3).
 *  n_seq      sequences, >= 1
 *  Lc         clean-stream length (vision, prompts and responses), >= 1
 *  Ln         noisy-stream length (the responses' corrupted tokens), >= 0
 *  cap        positions held by k and v, a multiple of 32, >= Lc + Ln
 *  D          block size of the noisy stream, 1..4096
 *  Hq, Hkv    query / KV heads, Hq % Hkv == 0 (head h uses KV head h / (Hq/Hkv))
 *  d          head dim, 64 or 128
 *  max_spans  response spans per sequence (rows of `spans`), 0..256 (0 only if Ln == 0)
 *  scale      softmax scale, finite and > 0
 * Size limits (BD_E_SHAPE otherwise), with L = Lc + Ln: L * Hq <= 2^20,
 * cap * d <= 2^30, n_seq * Hkv * ceil(L * (Hq/Hkv) / 128) < 2^31 / 64 and
 * n_seq * L * Hq / 4 < 2^31. */
typedef struct {
    int32_t n_seq, Lc, Ln, cap, D, Hq, Hkv, d, max_spans;
    float scale;
} bd_two_stream_desc;

/* Workspace bytes bd_two_stream_attn needs (0 if none); SIZE_MAX if desc is invalid. */
size_t bd_two_stream_workspace_bytes(const bd_two_stream_desc *desc);

/* Two-stream training attention over [clean stream x ; noisy stream w] ([FD] 4.1:
 * causal-context attention with the masks M_N2N, M_N2C, M_C2C; [FD] 4.3: blocks cut at
 * response ends; [FD] 4.4: vision tokens only in the clean stream).  Sequence s has
 * L = Lc + Ln positions, clean positions 0..Lc-1 then noisy positions Lc..L-1.  Its
 * responses are spans[s][r] = (clean start c_r, length len_r), r < n_spans[s], in
 * order; w holds their tokens in the same order, response r at noisy offset
 * o_r = len_0 + ... + len_{r-1}.  Each response is cut into blocks of D tokens from
 * its start, the last block ending at the response end.
 *   clean position p         sees clean positions 0..p                       (M_C2C)
 *   noisy token of response r, block k, covering clean positions [b0, b1):
 *                            sees clean positions 0..b0-1                   (M_N2C)
 *                            and the noisy tokens of its own block            (M_N2N)
 *   noisy positions past the last response see nothing and get 0;
 *   out = softmax(scale * q k^T) v over the visible keys.
 * Layouts (bf16, row-major): q, out [n_seq][L][Hq][d]; k, v [n_seq][Hkv][cap][d]
 * (as the decode cache); spans int32
 * [n_seq][max_spans][2], n_spans int32 [n_seq] (device).  k and v positions
 * L..cap-1 are read (as parts of 32-key tiles) but never weighted; they must hold
 * finite values (zeros, say).  Span values out of range are clamped into the
 * sequence, never read outside it.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_PARAM, BD_E_WORKSPACE, BD_E_LAUNCH. */
bd_status bd_two_stream_attn(const bd_two_stream_desc *desc, const void *q, const void *k, const void *v,
                             const int32_t *spans, const int32_t *n_spans, void *out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *bd_status_string(bd_status status);

/* hipError_t value of the last failed launch on the calling thread (0 if none). */
int32_t bd_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BD_H */
