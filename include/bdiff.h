/*
 * bdiff.h - C ABI of libbdiff, the block-diffusion decode step and the
 * dual-stream training attention of Fast-dVLM, for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources (web pages on the method, cited by page and section):
 *   [OV]   Fast-dVLM engineering overview (ocdem.com/news/1032714)
 *   [TH]   Fast-dVLM article, Thai translation (itsolotime.com/th/archives/34466)
 *   [LOWN] LOWN article (paper.rainbus.top/paper/2610.36671)
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless the argument says "host".
 *   - Every compute call is asynchronous on `stream` (0 = the null stream)
 *     and returns as soon as its kernels are enqueued.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no global mutable state; scratch space comes in as a
 *     caller-provided workspace sized by the matching *_ws_bytes query.  The
 *     one exception is bd_lmhead_conf_noalloc, whose scratch is a static
 *     device array of the library (one per GPU).
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is launched and the outputs are untouched.  A failed
 *     launch returns BD_E_LAUNCH.  No call aborts or throws.
 *   - Tensors are dense, row-major, in the layouts given below.  bf16 means
 *     IEEE bfloat16 storage with float32 accumulation inside the kernels.
 *   - Vector-loaded tensors (q, k, v, caches, h, W, outputs, workspaces)
 *     must be 16-byte aligned (BD_E_ALIGN otherwise).
 *   - Two calls that share a workspace must be ordered on one stream.
 */
#ifndef BDIFF_H
#define BDIFF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Each enum below carries two bound enumerators that are never used as
 * values: they make its range every int32, so that any int a C caller passes
 * is a valid value of the type in the C++ implementation, which then
 * rejects it (BD_E_DTYPE, BD_E_SHAPE) or describes it ("unknown status"). */
typedef enum {
    BD_STATUS_INT32_MIN_ = -2147483647 - 1,
    BD_OK = 0,
    BD_E_NULL = 1,       /* a required pointer is NULL                        */
    BD_E_SHAPE = 2,      /* a size is out of range or sizes are inconsistent  */
    BD_E_DTYPE = 3,      /* unknown dtype, or dtype not supported for the call */
    BD_E_ALIGN = 4,      /* a vector-loaded pointer is not 16-byte aligned    */
    BD_E_WORKSPACE = 5,  /* workspace missing or smaller than *_ws_bytes      */
    BD_E_DEVICE = 6,     /* current device is not gfx950                      */
    BD_E_LAUNCH = 7,     /* the HIP runtime rejected a kernel launch          */
    BD_STATUS_INT32_MAX_ = 2147483647
} bd_status;

typedef enum {
    BD_DTYPE_INT32_MIN_ = -2147483647 - 1,
    BD_F32 = 0,
    BD_BF16 = 1,
    BD_DTYPE_INT32_MAX_ = 2147483647
} bd_dtype;

/* Visibility among the Bq block queries (block key j for block query i). */
typedef enum {
    BD_MASK_INT32_MIN_ = -2147483647 - 1,
    BD_MASK_BIDIR = 0,      /* all ones: parallel denoising inside a block [OV §1.2] */
    BD_MASK_CAUSAL = 1,     /* j <= i: the AR verify pass [OV §2.3.1]               */
    BD_MASK_SPEC_FUSED = 2, /* draft+verify in one forward [OV §2.3.1], Bq = 2B:
                               rows 0..B-1 causal among themselves; rows B..2B-1
                               see row j < B iff j <= i-B, and all of B..2B-1 */
    BD_MASK_INT32_MAX_ = 2147483647
} bd_mask_kind;

/* Static description of a status code; never NULL. */
const char* bd_status_str(bd_status s);

/* BD_OK iff `device` exists and is a gfx950 GPU; BD_E_DEVICE otherwise
 * (including when no GPU is present).  There is no fallback path. */
bd_status bd_device_check(int device);

/* Host helper: fills host_rows[i] (i < Bq) with the intra-block bitmask of
 * block query i (bit j set = block key j visible) for `kind`.
 * Bq in [1, 64]; BD_MASK_SPEC_FUSED needs an even Bq.  host_rows: host array
 * of Bq words.  Errors: BD_E_NULL, BD_E_SHAPE. */
bd_status bd_make_intra_mask(bd_mask_kind kind, int32_t Bq, uint64_t* host_rows);

/*
 * bd_block_attn - attention of a block of Bq queries over a KV-cached prefix
 * plus the block itself.  [OV §1.2: blocks decoded in order, each block's
 * tokens denoised in parallel with bidirectional attention, the prefix
 * (visual + prompt + earlier blocks) kept in the KV cache; TH §1]
 *
 *   o[i][h] = sum_j softmax_j(scale * q[i][h] . k[g][j]) v[g][j]
 *   over j in [0, P) (always visible) and j = P + jb for block key jb with
 *   bit jb of intra_mask[i] set; g = h / (Hq / Hkv) (grouped-query heads).
 *   A query row with no visible key gets a zero output row.
 *
 *   q           [Bq][Hq][dh]   dtype dt
 *   k_cache,
 *   v_cache     [Hkv][cap][dh] dtype dt; rows P..P+Bq-1 hold the block's keys
 *                              and values (written by the caller)
 *   intra_mask  [Bq] uint64 (device), e.g. from bd_make_intra_mask
 *   out         [Bq][Hq][dh]   dtype dt
 *   scale       softmax scale, > 0; 0 selects 1/sqrt(dh)
 *   ws          workspace of at least bd_block_attn_ws_bytes(...) bytes; the
 *               size never decreases as P grows (other arguments fixed), so
 *               a workspace sized for the longest prefix serves every call
 *               with a shorter one
 * Limits: 1 <= Bq <= 64, 0 <= P, P + Bq <= cap, Hkv >= 1, Hq % Hkv == 0,
 *   BD_BF16: dh == 128 and P + Bq <= 65536;  BD_F32: dh % 4 == 0 and
 *   4 <= dh <= 128.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_ALIGN, BD_E_WORKSPACE,
 *   BD_E_LAUNCH.
 */
size_t bd_block_attn_ws_bytes(int32_t P, int32_t Bq, int32_t Hq, int32_t Hkv, int32_t dh);
bd_status bd_block_attn(bd_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                        int32_t P, int32_t cap, const uint64_t* intra_mask,
                        int32_t Bq, int32_t Hq, int32_t Hkv, int32_t dh, float scale,
                        void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bd_block_attn_paged - bd_block_attn (bf16) over a paged KV cache, visiting
 * the keys from key_lo on.  [OV §2.3.2: the serving system keeps the KV
 * cache in pages; LOWN 'method step details': the TEXT-ONLY forward leaves
 * the visual tokens out - key_lo = the number of visual tokens]
 *   Logical key position j (prefix 0..P-1, then the block's own keys
 *   P..P+Bq-1) of KV head g is row j % page_size of page
 *   page_table[j / page_size]:  k_pool[page][g][j % page_size][dh].
 *   Query i sees prefix keys key_lo <= j < P and block key P + jb iff bit jb
 *   of intra_mask[i] is set; otherwise as bd_block_attn.
 *   k_pool, v_pool [n_pages][Hkv][page_size][dh] bf16
 *   page_table     [ceil((P + Bq) / page_size)] int32 (device); entries are
 *                  physical page indices in [0, n_pages) (the kernel clamps
 *                  others into that range)
 *   ws             at least bd_block_attn_ws_bytes(P - key_lo, Bq, Hq, Hkv, dh)
 * Limits: dh == 128, page_size >= 1, 0 <= key_lo <= P,
 *   P + Bq - key_lo <= 65536, n_pages * page_size >= P + Bq, the pools
 *   smaller than 4 GiB each; otherwise those of bd_block_attn.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_ALIGN, BD_E_WORKSPACE, BD_E_LAUNCH.
 */
bd_status bd_block_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* page_table, int32_t page_size, int32_t n_pages,
                              int32_t P, int32_t key_lo, const uint64_t* intra_mask, int32_t Bq,
                              int32_t Hq, int32_t Hkv, int32_t dh, float scale, void* out,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bd_lmhead_conf - LM-head contraction fused with the softmax maximum:
 * per position b, logits l[v] = h[b] . W[v] (never written to memory),
 *   argmax[b] = smallest v with l[v] = max l,
 *   conf[b]   = 1 / sum_v exp(l[v] - max l) = the largest softmax probability.
 * [LOWN 'method step details' (1): confidence = max_w p(y_i = w | .);
 *  OV §1.1: batch-1 decode is bound by reloading the weights every step]
 *
 *   h       [B][d]  dtype dt
 *   W       [V][d]  dtype dt (row-major: one row per vocabulary entry)
 *   conf    [B] float32 out;  argmax [B] int32 out
 *   ws      workspace of at least bd_lmhead_conf_ws_bytes(B, d, V) bytes
 *           (per-workgroup partial maxima, sums and indices; no initial
 *           contents required).  Two kernels run: the streaming contraction
 *           and a small merge of the partials.
 * Limits: 1 <= B <= 64, 1 <= V <= 2^30, d >= 1;  BD_BF16 needs d % 128 == 0 and
 *   d <= 16384.  The result is deterministic (fixed reduction order).
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_ALIGN, BD_E_WORKSPACE,
 *   BD_E_LAUNCH.
 */
size_t bd_lmhead_conf_ws_bytes(int32_t B, int32_t d, int32_t V);
bd_status bd_lmhead_conf(bd_dtype dt, const void* h, const void* W,
                         int32_t B, int32_t d, int32_t V,
                         float* conf, int32_t* argmax,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bd_lmhead_conf_commit - bd_lmhead_conf followed by bd_commit on its
 * outputs, as one call: the merge of the LM-head partials and the threshold
 * commit run in the same small kernel, saving a launch per decode step.
 * [OV §1.2 parallel denoising inside a block; OV §4.1 threshold 0.9;
 *  LOWN 'method step details' (1) for the confidence]
 * Arguments as in bd_lmhead_conf and bd_commit; conf and argmax are written
 * exactly as bd_lmhead_conf writes them (bit-identical), then positions are
 * committed exactly as bd_commit would commit them.  The workspace size is
 * bd_lmhead_conf_ws_bytes(B, d, V).
 * Errors: those of bd_lmhead_conf, plus BD_E_NULL for masked, tokens or
 *   n_committed and BD_E_SHAPE for a NaN tau.
 */
bd_status bd_lmhead_conf_commit(bd_dtype dt, const void* h, const void* W,
                                int32_t B, int32_t d, int32_t V, float tau,
                                float* conf, int32_t* argmax,
                                uint8_t* masked, int32_t* tokens, int32_t* n_committed,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bd_lmhead_conf_noalloc - bd_lmhead_conf without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The partial
 * states live in a static device array of the library, 196608 bytes (3 x 256
 * partials x 64 positions x 4 bytes), of which each GPU that the library runs
 * on holds its own copy until the process ends.  Results are bit-identical to
 * bd_lmhead_conf's for the same inputs.
 *   Arguments, layouts and limits as in bd_lmhead_conf.  Every bf16 shape
 *   within those limits fits; a float32 shape needs V <= 65536 (its partials
 *   are one per 256 vocabulary rows).  A shape whose partials exceed the
 *   array returns BD_E_WORKSPACE.
 *   The array needs no initial contents and is not cleared between calls.
 *   All calls on one GPU share it: calls that may overlap on the same GPU
 *   (different streams, or several host threads, without ordering between
 *   them) race and give undefined results.  The first call on a device looks
 *   the array's device address up (hipGetSymbolAddress; BD_E_DEVICE if that
 *   fails); no call allocates memory.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_ALIGN, BD_E_WORKSPACE,
 *   BD_E_DEVICE, BD_E_LAUNCH.
 */
bd_status bd_lmhead_conf_noalloc(bd_dtype dt, const void* h, const void* W,
                                 int32_t B, int32_t d, int32_t V,
                                 float* conf, int32_t* argmax, hipStream_t stream);

/*
 * bd_lmhead_conf_fp8 - bd_lmhead_conf with FP8 weights and activations
 * (W8A8, the quantization of the fastest configuration: OV §2.3.2 FP8
 * SmoothQuant W8A8; OV §4.1 quant_mode fp8).  The number format is OCP E4M3
 * (OFP8 specification: sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * largest finite value 448; S.1111.111 is NaN).
 *   W8A8 rule.  W is given as E4M3 codes with one float32 dequantization
 *   scale per vocabulary row.  Each hidden row is quantized when the call
 *   runs, exactly as bd_quant_fp8_rows quantizes a row (qh[b], s_h[b]); then
 *     l[v] = s_h[b] * w_scale[v] * sum_k dec(qh[b][k]) dec(Wq[v][k])
 *   with float32 accumulation, and conf/argmax as in bd_lmhead_conf.
 *
 *   h        [B][d] bf16 (finite)
 *   Wq       [V][d] E4M3 codes (uint8); NaN codes are not allowed
 *   w_scale  [V] float32
 *   conf     [B] float32 out;  argmax [B] int32 out
 *   ws       workspace of at least bd_lmhead_conf_fp8_ws_bytes(B, d, V) bytes
 *            (no initial contents required)
 * Limits: 1 <= B <= 64, 1 <= V <= 2^30, d % 128 == 0, 128 <= d <= 16384.  h, Wq,
 *   w_scale and ws must be 16-byte aligned.  Deterministic (fixed reduction
 *   order).  bd_lmhead_conf_fp8_ws_bytes returns 0 for shapes out of range.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_ALIGN, BD_E_WORKSPACE, BD_E_LAUNCH.
 */
size_t bd_lmhead_conf_fp8_ws_bytes(int32_t B, int32_t d, int32_t V);
bd_status bd_lmhead_conf_fp8(const void* h, const uint8_t* Wq, const float* w_scale,
                             int32_t B, int32_t d, int32_t V,
                             float* conf, int32_t* argmax,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bd_lmhead_conf_commit_fp8 - bd_lmhead_conf_fp8 followed by bd_commit, as
 * one call (the same relation as bd_lmhead_conf_commit to bd_lmhead_conf).
 * [OV §1.2, §2.3.2, §4.1]  Workspace: bd_lmhead_conf_fp8_ws_bytes(B, d, V).
 * Errors: those of bd_lmhead_conf_fp8, plus BD_E_NULL for masked, tokens or
 *   n_committed and BD_E_SHAPE for a NaN tau.
 */
bd_status bd_lmhead_conf_commit_fp8(const void* h, const uint8_t* Wq, const float* w_scale,
                                    int32_t B, int32_t d, int32_t V, float tau,
                                    float* conf, int32_t* argmax,
                                    uint8_t* masked, int32_t* tokens, int32_t* n_committed,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bd_quant_fp8_rows - per-row dynamic quantization to E4M3, the rule that
 * bd_lmhead_conf_fp8 applies to its hidden rows (and a way to store weights
 * with per-row scales).  [OV §2.3.2 W8A8]  Per row, in float32:
 *   amax = max_k |x[k]|;  r = 448 / amax and scale = amax / 448, each
 *   correctly rounded (r = scale = 1 for an all-zero row);
 *   q[k] = E4M3(clamp(x[k] * r, -448, 448)), rounded to nearest, ties to the
 *   even code; a negative value that rounds to zero gives 0x80.
 *   x [R][d] bf16 (finite);  q [R][d] uint8 out;  scale [R] float32 out
 * Limits: R >= 0 (R = 0 launches nothing), d % 8 == 0, d >= 8.  x and q must
 *   be 16-byte aligned.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_ALIGN, BD_E_LAUNCH.
 */
bd_status bd_quant_fp8_rows(const void* x, int32_t R, int32_t d, uint8_t* q, float* scale,
                            hipStream_t stream);

/*
 * bd_block_loop - the device-resident block loop: decode steps on one block
 * until every position is committed, with no host round trip.  [OV §1.2:
 * each block is denoised in parallel over several steps before the next
 * block starts; OV §2.2.2: the block's first position is the AR seed; OV
 * §4.1: threshold 0.9]
 * Step s (s < max_steps) runs only while some position is still masked:
 *   bd_block_attn(q_steps[s]) -> attn_out[s];
 *   the LM head on h_steps[s] (bd_lmhead_conf, or bd_lmhead_conf_fp8 when
 *   w_scale is given) -> conf[s], argmax[s]; then bd_commit on the block.
 * A step that finds the block complete is skipped entirely on the device:
 * its outputs are left untouched and n_committed[s] stays 0.  Every kernel
 * of every step is enqueued up front, so the call can be captured in a HIP
 * graph; the steps that run are decided on the device.  The per-step inputs
 * stand for the hidden states and queries that the model's other layers
 * produce at each step.
 *   q_steps    [max_steps][B][Hq][dh] dtype dt (block queries per step)
 *   k_cache, v_cache, P, cap, intra_mask, Hq, Hkv, dh, scale: as in
 *              bd_block_attn with Bq = B (the block's K/V rows stay fixed)
 *   h_steps    [max_steps][B][d] dtype dt (bf16 when w_scale is given)
 *   W          [V][d] dtype dt, or E4M3 codes when w_scale ([V] float32) is
 *              given (then dt must be BD_BF16)
 *   tau        threshold (not NaN);  max_steps in [1, 1024]
 *   masked [B] uint8, tokens [B] int32: block state, in/out
 *   attn_out   [max_steps][B][Hq][dh] dtype dt out
 *   conf, argmax [max_steps][B] out
 *   n_committed [max_steps] int32 out (commits per step, 0 for skipped steps)
 *   n_steps    [1] int32 out (steps executed)
 *   ws         workspace of at least bd_block_loop_ws_bytes(P, B, Hq, Hkv, dh,
 *              d, V, w_scale != NULL) bytes (holds the gate word between
 *              steps; no initial contents required)
 * Limits: those of bd_block_attn and of the LM-head call used.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_ALIGN, BD_E_WORKSPACE,
 *   BD_E_LAUNCH.
 */
size_t bd_block_loop_ws_bytes(int32_t P, int32_t B, int32_t Hq, int32_t Hkv, int32_t dh,
                              int32_t d, int32_t V, int32_t w_fp8);
bd_status bd_block_loop(bd_dtype dt, const void* q_steps, const void* k_cache,
                        const void* v_cache, int32_t P, int32_t cap, const uint64_t* intra_mask,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t dh, float scale,
                        const void* h_steps, const void* W, const float* w_scale, int32_t d,
                        int32_t V, float tau, int32_t max_steps, uint8_t* masked,
                        int32_t* tokens, void* attn_out, float* conf, int32_t* argmax,
                        int32_t* n_committed, int32_t* n_steps, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * bd_decode_blocks - the device-resident decode loop over n_blocks blocks of
 * B positions, generated one after another with the KV cache growing by each
 * block, and no host round trip.  [OV §1.2: blocks are generated in order,
 * each denoised in parallel over several steps, the KV cache of the earlier
 * blocks reused; OV §2.2.2: causal-context decoding, the block's first token
 * comes from the AR (causal) prediction; OV §4.1: threshold 0.9]
 * The prefix length lives on the device: *kv_len (the prompt's P0 on entry).
 * For block b = 0 .. n_blocks-1, in order:
 *   1. kv_len += B if b > 0 (the previous block joins the prefix); the
 *      block's own K/V rows k_blk[b], v_blk[b] are written into cache rows
 *      kv_len .. kv_len + B - 1;
 *   2. AR seed: q_seed[b] attends the prefix [0, kv_len) (bd_block_attn with
 *      one query and no block key visible) -> seed_attn[b]; the LM head on
 *      h_seed[b] gives seed_conf[b] and the seed token tokens[b][0];
 *      tokens[b][1..B-1] = 0 and masked[b] = [0, 1, ..., 1];
 *   3. up to max_steps denoising steps while a position of the block is
 *      masked, exactly as bd_block_loop runs them (bd_block_attn over the
 *      prefix kv_len and the block's rows under intra_mask, the LM head, the
 *      threshold commit on tokens[b], masked[b]); a block with max_steps >=
 *      B - 1 always completes (every step commits at least one position).
 * Finally kv_len += B for the last block, so *kv_len = P0 + n_blocks B on
 * exit.  A block that has not completed after max_steps is appended anyway,
 * with its masked flags left set.  Every kernel is enqueued up front, so the
 * call can be captured in a HIP graph.  The per-step queries, hidden rows and
 * block K/V rows stand for what the model's other layers produce.
 *   q_seed   [n_blocks][Hq][dh] bf16;    h_seed  [n_blocks][d] bf16
 *   q_steps  [n_blocks][max_steps][B][Hq][dh] bf16
 *   h_steps  [n_blocks][max_steps][B][d] bf16
 *   k_blk, v_blk  [n_blocks][B][Hkv][dh] bf16
 *   k_cache, v_cache [Hkv][cap][dh] bf16, in/out (rows from kv_len on are
 *            overwritten by the blocks)
 *   kv_len   [1] int32 (device), in/out; P_max (host) bounds its value on
 *            entry (larger values are clamped to it)
 *   intra_mask [B] uint64 (device), as for bd_block_attn
 *   W        [V][d] bf16, or E4M3 codes when w_scale ([V] float32) is given
 *   tokens [n_blocks][B] int32 out, masked [n_blocks][B] uint8 out (final state)
 *   n_steps [n_blocks] int32 out; n_committed [n_blocks][max_steps] int32 out
 *            (0 for steps not run)
 *   seed_attn [n_blocks][Hq][dh] bf16 out; seed_conf [n_blocks] float32 out
 *   attn_out [n_blocks][max_steps][B][Hq][dh] bf16 out; conf, argmax
 *            [n_blocks][max_steps][B] out (steps not run: left untouched)
 *   ws       at least bd_decode_blocks_ws_bytes(P_max, n_blocks, B, Hq, Hkv,
 *            dh, d, V, w_scale != NULL) bytes (no initial contents required)
 * Limits: dh == 128, 1 <= B <= 64, Hq % Hkv == 0, P_max >= 0,
 *   P_max + n_blocks B <= min(cap, 65536), 1 <= max_steps <= 1024, LM-head
 *   limits of bd_lmhead_conf (bf16) or bd_lmhead_conf_fp8.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_ALIGN, BD_E_WORKSPACE, BD_E_LAUNCH.
 */
size_t bd_decode_blocks_ws_bytes(int32_t P_max, int32_t n_blocks, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t dh, int32_t d, int32_t V, int32_t w_fp8);
bd_status bd_decode_blocks(const void* q_seed, const void* h_seed, const void* q_steps,
                           const void* h_steps, const void* k_blk, const void* v_blk,
                           void* k_cache, void* v_cache, int32_t cap, int32_t* kv_len,
                           int32_t P_max, const uint64_t* intra_mask, int32_t n_blocks, int32_t B,
                           int32_t max_steps, int32_t Hq, int32_t Hkv, int32_t dh, float scale,
                           const void* W, const float* w_scale, int32_t d, int32_t V, float tau,
                           int32_t* tokens, uint8_t* masked, int32_t* n_steps,
                           int32_t* n_committed, void* seed_attn, float* seed_conf,
                           void* attn_out, float* conf, int32_t* argmax, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * bd_commit - threshold unmasking with the always-one rule.
 * [OV §4.1: denoising confidence threshold 0.9; OV §1.2 parallel unmasking]
 * Every position i with masked[i] != 0 and conf[i] > tau is committed.  If
 * none qualifies and some position is masked, the masked position with the
 * largest conf (lowest index on ties) is committed alone.  Committing i sets
 * tokens[i] = argmax[i] and masked[i] = 0; other positions are untouched.
 *
 *   conf [B] float32, argmax [B] int32   (e.g. from bd_lmhead_conf)
 *   masked [B] uint8 in/out, tokens [B] int32 in/out
 *   n_committed [1] int32 out
 * Limits: 0 <= B <= 64; conf values must not be NaN.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_LAUNCH.
 */
bd_status bd_commit(const float* conf, const int32_t* argmax, int32_t B, float tau,
                    uint8_t* masked, int32_t* tokens, int32_t* n_committed,
                    hipStream_t stream);

/*
 * bd_spec_accept - self-speculative verification: keep the longest prefix
 * of the diffusion draft that the causal (AR) pass reproduces, truncate the
 * KV cache to it and append the accepted tokens.  [OV §2.3.1; TH §5.3]
 *   L = max { l <= B : draft[0..l) == verify[0..l) }   (index-aligned)
 *   accepted[0] = L;  kv_len[0] = P + L;  out_tokens[0..L) = draft[0..L)
 * The KV truncation is the length update: cache rows below P + L stay valid,
 * rows from P + L on are free to be overwritten.  out_tokens[L..B) are left
 * untouched.  Used by both the linear (two forwards) and the fused quadratic
 * (one forward, rows 0..B-1 of the fused block give `verify`) variants.
 *   draft, verify [B] int32;  accepted [1], kv_len [1], out_tokens [B] int32 out
 * Limits: 0 <= B <= 64, P >= 0, P + B must fit in int32.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_LAUNCH.
 */
bd_status bd_spec_accept(const int32_t* draft, const int32_t* verify, int32_t B, int32_t P,
                         int32_t* accepted, int32_t* kv_len, int32_t* out_tokens,
                         hipStream_t stream);

/*
 * bd_spec_accept_bonus - bd_spec_accept that also takes the verify pass's
 * own token at the first disagreement.  The pages state no such token [OV
 * §2.3.1]; it is the correction token of greedy speculative decoding
 * (Leviathan et al. 2023; Chen et al. 2023), with which the tokens appended
 * over the steps are exactly those of greedy decoding with the verifier.
 *   L as in bd_spec_accept.  If L < B:  accepted[0] = L + 1,
 *   out_tokens[0..L) = draft[0..L), out_tokens[L] = verify[L];
 *   otherwise as bd_spec_accept.  kv_len[0] = P + L in both cases: the K/V
 *   row of position L was computed from the rejected draft token, so the
 *   caller's next step computes the appended token's row.
 *   out_tokens[accepted..B) are left untouched.
 *   Arguments, limits and errors as bd_spec_accept.
 */
bd_status bd_spec_accept_bonus(const int32_t* draft, const int32_t* verify, int32_t B, int32_t P,
                               int32_t* accepted, int32_t* kv_len, int32_t* out_tokens,
                               hipStream_t stream);

/*
 * bd_lmhead_conf_accept - the verify pass's LM head followed by the
 * speculative accept, as one call: bd_lmhead_conf on h, then
 * bd_spec_accept (bd_spec_accept_bonus when bonus != 0) with verify = this
 * call's argmax[0..B_acc) against draft[0..B_acc).  The merge of the LM-head
 * partials and the accept run in the same small kernel, saving the accept's
 * launch per speculative step.  [OV §2.3.1 the linear (two forwards) and
 * quadratic (one forward; rows 0..B_acc-1 of the fused block are the verify
 * half) self-speculative steps; LOWN 'method step details' (1) for conf]
 *   h, W, B, d, V, conf, argmax, ws, ws_bytes  as in bd_lmhead_conf
 *   draft     [B_acc] int32 (device; read only)
 *   B_acc     positions verified, 1 <= B_acc <= B
 *   P, accepted, kv_len, out_tokens  as in bd_spec_accept
 * argmax is bit-identical to bd_lmhead_conf's; conf is too for B <= 16 and
 * otherwise within float32 rounding of it (the merge sums the partials of
 * several positions side by side, in another fixed order).  accepted, kv_len
 * and out_tokens are exactly those of the two separate calls.
 * Errors: those of bd_lmhead_conf, plus BD_E_NULL for draft, accepted, kv_len
 *   or out_tokens, and BD_E_SHAPE unless 1 <= B_acc <= B, P >= 0 and
 *   P + B_acc fits in int32.
 */
bd_status bd_lmhead_conf_accept(bd_dtype dt, const void* h, const void* W,
                                int32_t B, int32_t d, int32_t V,
                                float* conf, int32_t* argmax,
                                const int32_t* draft, int32_t B_acc, int32_t P, int32_t bonus,
                                int32_t* accepted, int32_t* kv_len, int32_t* out_tokens,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bd_cert_scan - LOWN certificate over n masked positions.
 * [LOWN 'method step details' (2)-(3)]  order = the positions sorted by
 * anchor_conf descending (stable: lower index first on ties);
 * L = the longest prefix of `order` on which text_tok == anchor_tok;
 * skip_full = (L >= k): the image forward can be skipped this step.
 *   anchor_conf [n] float32 (finite), anchor_tok [n] int32, text_tok [n] int32
 *   order [n] int32 out, accepted [1] int32 out (= L), skip_full [1] int32 out
 * Limits: 0 <= n <= 1024.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_LAUNCH.
 */
bd_status bd_cert_scan(const float* anchor_conf, const int32_t* anchor_tok,
                       const int32_t* text_tok, int32_t n, int32_t k,
                       int32_t* order, int32_t* accepted, int32_t* skip_full,
                       hipStream_t stream);

/*
 * bd_block_attn_fp8kv - bd_block_attn (bf16 queries and output) over an FP8
 * KV cache.  [OV §2.3.2: the fastest configuration runs FP8; OCP OFP8 E4M3]
 * The cache holds OCP E4M3 codes, and a cached entry stands for
 *   decode(code) * k_scale[g]   (K of KV head g),  decode(code) * v_scale[g]
 * (V), so scores are scale * k_scale[g] * (q . decode(k)) and the output is
 * v_scale[g] * (softmax-weighted decoded V).  Masks, heads, prefix and the
 * block's own rows as in bd_block_attn.
 *   q            [Bq][Hq][dh] bfloat16;  out the same
 *   k_cache, v_cache  [Hkv][cap][dh] uint8 E4M3 codes (NaN codes not allowed)
 *   k_scale, v_scale  [Hkv] float32 (device)
 *   ws           at least bd_block_attn_ws_bytes(P, Bq, Hq, Hkv, dh) bytes
 * Limits: dh == 128, Bq <= 64, P + Bq <= min(cap, 65536), Hq % Hkv == 0.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_ALIGN (16 bytes; scales 4),
 *   BD_E_WORKSPACE, BD_E_LAUNCH.
 */
bd_status bd_block_attn_fp8kv(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                              const float* k_scale, const float* v_scale, int32_t P, int32_t cap,
                              const uint64_t* intra_mask, int32_t Bq, int32_t Hq, int32_t Hkv,
                              int32_t dh, float scale, void* out, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * bd_kv_quant_fp8 - writes n new K (or V) rows into an FP8 cache, e.g. the
 * block's own rows at pos = P.  [OV §2.3.2; OCP OFP8 E4M3]
 *   cache[g][pos + i][d] = E4M3 rounding (nearest, ties to even) of
 *                          clamp(fl32(x[i][g][d] * fl32(1 / scale[g])), -448, 448)
 *   x      [n][Hkv][dh] bfloat16 (finite), 8-byte aligned
 *   scale  [Hkv] float32 (device), > 0
 *   cache  [Hkv][cap][dh] uint8, 4-byte aligned; rows outside pos .. pos+n-1
 *          are left untouched
 * Limits: dh % 4 == 0, 0 <= pos, pos + n <= cap; n = 0 is a no-op.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_ALIGN, BD_E_LAUNCH.
 */
bd_status bd_kv_quant_fp8(const void* x, int32_t n, int32_t Hkv, int32_t dh, const float* scale,
                          uint8_t* cache, int32_t cap, int32_t pos, hipStream_t stream);

/*
 * bd_dualstream_attn - training-time attention over the vision-efficient
 * dual-stream sequence [visual (n_vis) | clean text (n_txt) | noisy text
 * (n_txt)], N = n_vis + 2 n_txt.  [OV §2.2.1-§2.2.2; TH §4.1, §4.4]
 * Query row i sees key j iff
 *   C2C: i, j < n_vis + n_txt and j <= i             (clean stream, causal)
 *   N2C: i noisy (r = i - n_vis - n_txt), j visual, or j clean text with
 *        j - n_vis <= r                               (printed N2C matrix)
 *   N2N: i, j noisy with (r / block) == (r_j / block) (bidirectional block)
 * and no clean query sees a noisy key.  Softmax scaled dot-product per head.
 *   q, k, v, out [N][H][dh] dtype dt;  scale > 0, or 0 for 1/sqrt(dh)
 * Limits: n_vis >= 0, n_txt >= 0, N >= 1, block >= 1, H >= 1,
 *   BD_BF16: dh == 128;  BD_F32: dh % 4 == 0 and 4 <= dh <= 128.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_ALIGN, BD_E_LAUNCH.
 */
bd_status bd_dualstream_attn(bd_dtype dt, const void* q, const void* k, const void* v,
                             int32_t n_vis, int32_t n_txt, int32_t block, int32_t H,
                             int32_t dh, float scale, void* out, hipStream_t stream);

/*
 * bd_dualstream_attn_seg - bd_dualstream_attn with the auto-truncation mask
 * for multi-turn text [OV §2.2.2: the mask keeps the last block of a
 * response from spilling into the next turn's prompt; TH §4.3].  The text
 * positions 0..n_txt-1 are split into n_seg segments (the turns' prompts and
 * responses) starting at seg_starts[s].  N2N blocks tile every segment from
 * its own start and end at the segment's end:
 *   N2N: noisy r, r' (text positions) see each other iff they lie in the
 *        same segment S = [s0, s1) and floor((r - s0) / block) ==
 *        floor((r' - s0) / block).
 * C2C and N2C are those of bd_dualstream_attn.  n_seg = 1 gives exactly
 * bd_dualstream_attn.
 *   seg_starts  HOST array of n_seg int32: seg_starts[0] = 0, strictly
 *               increasing, every entry < n_txt (copied at the call)
 * Limits: those of bd_dualstream_attn; 1 <= n_seg <= 64.
 * Errors: those of bd_dualstream_attn, plus BD_E_NULL for seg_starts and
 *   BD_E_SHAPE for an invalid segmentation.
 */
bd_status bd_dualstream_attn_seg(bd_dtype dt, const void* q, const void* k, const void* v,
                                 int32_t n_vis, int32_t n_txt, int32_t block,
                                 const int32_t* seg_starts, int32_t n_seg, int32_t H,
                                 int32_t dh, float scale, void* out, hipStream_t stream);

/*
 * bd_dualstream_attn_fwd - the training forward: bd_dualstream_attn (or, with
 * seg_starts, bd_dualstream_attn_seg) that also keeps the row log-sum-exp
 * the backward needs.  [OV §2.2.1-§2.2.2; TH §4.1]
 *   lse[i][h] = log sum_{j visible from i} exp(scale q_i . k_j)  (natural log)
 *   seg_starts  HOST array of n_seg segment starts, or NULL for one segment
 *   lse         [N][H] float32 out, or NULL (then this is the plain forward)
 * For bf16, lse is formed from the same rounded probabilities that the output
 * uses (about 1e-3 from the exact value).
 * Errors: those of bd_dualstream_attn_seg; BD_E_ALIGN for a misaligned lse.
 */
bd_status bd_dualstream_attn_fwd(bd_dtype dt, const void* q, const void* k, const void* v,
                                 int32_t n_vis, int32_t n_txt, int32_t block,
                                 const int32_t* seg_starts, int32_t n_seg, int32_t H,
                                 int32_t dh, float scale, void* out, float* lse,
                                 hipStream_t stream);

/*
 * bd_dualstream_attn_bwd - the training backward of the dual-stream
 * attention: given the forward's q, k, v, out and lse and the output
 * gradient d_out, the gradients
 *   dV = P^T dO,  dS = P * (dO V^T - D),  D = rowsum(dO * O),
 *   dQ = scale dS K,  dK = scale dS^T Q,   P = exp(scale Q K^T - lse),
 * per head under the same masks (and segments) as the forward.  Nothing is
 * accumulated with atomics; the result is deterministic.
 * [OV §2.2.1: the dual-stream training objective; TH §4.1]
 *   q, k, v, out, d_out  [N][H][dh] dtype dt (out from bd_dualstream_attn_fwd)
 *   lse          [N][H] float32 from bd_dualstream_attn_fwd
 *   dq, dk, dv   [N][H][dh] dtype dt out (float32 accumulation inside)
 *   ws           workspace of at least bd_dualstream_attn_bwd_ws_bytes(n_vis,
 *                n_txt, H) bytes (holds D and lse in log2 units; no initial
 *                contents required)
 * Limits: those of bd_dualstream_attn; seg_starts as in bd_dualstream_attn_fwd.
 * Errors: BD_E_NULL, BD_E_SHAPE, BD_E_DTYPE, BD_E_ALIGN, BD_E_WORKSPACE,
 *   BD_E_LAUNCH.
 */
size_t bd_dualstream_attn_bwd_ws_bytes(int32_t n_vis, int32_t n_txt, int32_t H);
bd_status bd_dualstream_attn_bwd(bd_dtype dt, const void* q, const void* k, const void* v,
                                 const void* out, const void* d_out, const float* lse,
                                 int32_t n_vis, int32_t n_txt, int32_t block,
                                 const int32_t* seg_starts, int32_t n_seg, int32_t H, int32_t dh,
                                 float scale, void* dq, void* dk, void* dv, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BDIFF_H */
