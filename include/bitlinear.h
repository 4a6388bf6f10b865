/*
 * bitlinear.h -- C ABI of the Sparse-BitNet BitLinear hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * A BitLinear layer replaces a linear layer and has no bias (BitNet b1.58
 * 2B4T article, §一).  Its weight path, per Sparse-BitNet (explainer
 * article §三-§六; paper abstract), recomputes an N:M mask from the latent
 * full-precision weights every step, quantises to absmean ternary codes
 * (quantise first, then sparsify), multiplies with per-token int8
 * activations, and trains through both non-differentiable steps with a
 * straight-through estimator that still sends gradient to masked weights.
 *
 * Conventions shared by every call
 *   - Pointers named as device pointers must be device memory of the
 *     current HIP device, 16-byte aligned (gamma: 8-byte; x_scale: 4-byte).
 *     The caller allocates and frees every buffer; the library keeps no
 *     device memory and no global state between calls, except the static
 *     scratch of bitlinear_fwd_noalloc.
 *   - bf16 tensors are passed as uint16_t bit patterns.  W is [n_out x k],
 *     X is [tokens x k], dY is [tokens x n_out]; all row-major, contiguous.
 *   - Supported patterns (n, m): 8:8 (dense), 6:8, 4:8, 3:8, 2:8 (the
 *     sweep of the Sparse-BitNet article, §四) and 2:4.  k must be a
 *     positive multiple of 128; n_out >= 1; n_out*k, tokens*k and
 *     tokens*n_out below 2^31.
 *   - Outputs must not alias inputs or each other.
 *   - Every compute call only enqueues work on `stream` (a hipStream_t; NULL
 *     = the default stream) and returns without synchronising.  Arguments
 *     are validated on the host before anything is enqueued; on a non-zero
 *     status nothing was enqueued, except BL_EHIP, which reports a failed
 *     launch (work enqueued earlier in the same call may have run).  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - NaN or infinite inputs are outside the contract (not checked).
 *   - Calls are reentrant; the last-error text is per host thread.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BL_OK            0
#define BL_EINVAL        1  /* null or misaligned pointer, bad enum value  */
#define BL_ESHAPE        2  /* sizes outside the supported range           */
#define BL_EUNSUPPORTED  3  /* N:M pattern not supported                    */
#define BL_EWORKSPACE    4  /* workspace missing or smaller than required   */
#define BL_EHIP          5  /* a HIP runtime call or kernel launch failed   */

/* Which entries the absmean scale averages over (gamma_over). */
#define BL_GAMMA_DENSE   0  /* all n_out*k latent entries: quantise first
                               (Sparse-BitNet article §六, the order the
                               pages report as better)                    */
#define BL_GAMMA_MASKED  1  /* ablation: sum over kept entries only, still
                               divided by n_out*k (sparsify first)        */

/* Bytes of the packed ternary weights for an [n_out x k] layer under
 * pattern n:m, or 0 if the shape or pattern is unsupported.  The packed
 * layout stores each row's codes per 8-group as a nonzero bitmap plus one
 * sign bit per nonzero (S = 8, 6, 4, 4, 4, 2 sign slots for 8:8, 6:8, 4:8,
 * 3:8, 2:4, 2:8: the nonzeros an 8-group can hold, rounded up to even),
 * 16 groups per 128-wide k block, rows in strips of 64 (the last strip
 * padded with zero fields):
 *   ceil(n_out/64) * 64 * (k/128) * 2*(8+S) bytes.
 * A field is 8+S bits: bitmap of positions 0..3, the S sign bits (the
 * i-th nonzero of positions 0..3 at sign bit i, of positions 4..7 at sign
 * bit S-1-i), bitmap of positions 4..7.  The (strip p, k block kb)
 * superblock, at index p*(k/128)+kb, holds 64 chunks of 16 fields; chunk
 * c = r + 16q holds, as its field f = 4i + 2h + e (at bit f*(8+S)), the
 * 8-group 8h + 2q + e of row 64p + 16i + r. 
 * The 2-bit-per-weight storage of BitNet b1.58 (2B4T article §四) is the
 * 8:8 size of this format. */
size_t bitlinear_packed_bytes(int64_t n_out, int64_t k, int n, int m);

/* Workspace bytes bitlinear_quantize_mask needs: one exact partial |W| sum
 * per workgroup of the mask kernel plus its exponent bins (at most about
 * 2 MiB).  Host function; 0 for invalid shapes. */
size_t bitlinear_workspace_bytes(int64_t n_out, int64_t k);

/* Workspace bytes bitlinear_bwd needs: the bf16 operands of its two
 * products, bf16(dY * s_t) and x_q transposed to [n_out x tp] and [k x tp]
 * (tp = tokens rounded up to 64) and the decoded codes transposed to
 * [k x n_out rounded up to 64]; about 113 MB for a 6912 x 2560 layer at
 * 4096 tokens.  A product with few output tiles and a deep contraction
 * (e.g. dW of a 640 x 2560 layer at 4096 tokens) is split along it, and
 * the workspace then also holds its binary32 partial results (up to 8
 * planes of the product's output; 33 MB there).  0 for invalid shapes. */
size_t bitlinear_bwd_workspace_bytes(int64_t tokens, int64_t k, int64_t n_out);

/* Workspace bytes bitlinear_fwd / bitlinear_contract need for `tokens`
 * tokens: split-k partial sums and counters of the decode kernel (tokens
 * <= 16), or, for the prefill kernel, counters and exact int32 partial
 * tiles when the layer has too few 256 x 64 output tiles to fill the GPU
 * and the k range is split (e.g. a 1536-row layer with k >= 1024 at 1024
 * tokens: 12 MiB).  0 means ws may be NULL. */
size_t bitlinear_fwd_workspace_bytes(int64_t tokens, int64_t k, int64_t n_out);

/* Steps 1-2 (and optionally 3): mask and absmean scale.
 * Sparse-BitNet article §三 (mask recomputed every step), §五 (keep N of
 * every M by a per-group threshold), §六 (rank by the latent
 * full-precision weights); BitNet b1.58 2B4T article §一 (absmean).
 *   W      device, bf16 [n_out x k], read only.
 *   mask   device, uint8 [n_out x k/8], written: bit (c % 8) of byte
 *          (r, c/8) is 1 where W[r, c] is kept.  In each group of m
 *          consecutive entries along k the n largest |W| are kept; equal
 *          magnitudes keep the lower index (+0 and -0 are equal).
 *   wq     device, int8 [n_out x k] or NULL; if given, the masked ternary
 *          codes are also written (see bitlinear_pack).
 *   gamma  device, one double, written: the exact sum of |W| (over all
 *          entries, or kept entries for BL_GAMMA_MASKED) rounded once to
 *          binary64, divided by n_out*k in binary64.  Bit-reproducible.
 *   ws     device workspace of at least bitlinear_workspace_bytes(); its
 *          contents need not be initialised and are clobbered.
 */
int bitlinear_quantize_mask(const uint16_t *W, int64_t n_out, int64_t k,
                            int n, int m, int gamma_over, uint8_t *mask,
                            int8_t *wq, double *gamma, void *ws,
                            size_t ws_bytes, void *stream);

/* Step 3-4: masked ternary codes, packed.  BitNet b1.58 2B4T article §一
 * (ternary codes) and §四 (packed low-bit storage streamed from HBM).
 * The code of W[r, c] is sign(W) where the mask keeps it and 2|W| > gamma
 * (the exact form of clip(round_half_even(W/gamma), -1, 1) != 0), else 0.
 *   W, mask, gamma  device inputs as produced above.
 *   packed          device output of packed_bytes bytes (must equal
 *                   bitlinear_packed_bytes(n_out, k, n, m)).
 */
int bitlinear_pack(const uint16_t *W, const uint8_t *mask,
                   const double *gamma, int64_t n_out, int64_t k, int n,
                   int m, void *packed, size_t packed_bytes, void *stream);

/* Steps 5-7: per-token int8 activations, int32 contraction, epilogue.
 * BitNet b1.58 2B4T article §一 (8-bit activations, no bias) and §四
 * (ternary times int8 kernel).  For each token t:
 *   a_t = max_c |X[t, c]|,  x_q = clip(round_half_even(127 X / a_t),
 *   -128, 127) (exact quotient),  s_t = a_t / 127 (binary32, correctly
 *   rounded); a_t = 0 gives x_q = 0, s_t = 0.
 *   acc[t, r] = sum_c x_q[t, c] * code[r, c]  (int32, exact)
 *   Y[t, r]   = acc[t, r] * gamma * s_t      (binary32)
 *   X        device bf16 [tokens x k].
 *   packed   device, from bitlinear_pack with the same n_out, k, n, m.
 *   gamma    device double from bitlinear_quantize_mask.
 *   Y        device float [tokens x n_out], written.
 *   xq       device int8 [tokens x k], written (kept for the backward).
 *   x_scale  device float [tokens], written (s_t).
 *   acc      device int32 [tokens x n_out] or NULL (debug output).
 *   ws       device workspace of bitlinear_fwd_workspace_bytes(), or NULL
 *            when that is 0; clobbered.
 * tokens <= 16 runs the decode kernel, larger counts the prefill kernel;
 * both give identical results.  tokens == 0 is a no-op.
 */
int bitlinear_fwd(const uint16_t *X, int64_t tokens, int64_t k,
                  const void *packed, int64_t n_out, int n, int m,
                  const double *gamma, float *Y, int8_t *xq, float *x_scale,
                  int32_t *acc, void *ws, size_t ws_bytes, void *stream);

/* bitlinear_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without ws/ws_bytes.  The forward's
 * workspace lives in a static device array of 8 MiB that the library
 * holds on each device it runs on until the process ends; a call whose
 * bitlinear_fwd_workspace_bytes() exceeds 8 MiB (a prefill split along k
 * over more than 63 output tiles, or a decode with n_out * tokens above
 * about 2 million) returns BL_EWORKSPACE before anything is enqueued.  The
 * call allocates nothing and records no memset: the counters that must
 * start at zero are cleared inside its activation kernel.  The first call
 * on a device resolves the array's address there (hipGetSymbolAddress;
 * make it outside graph capture).  Every call on a device shares that
 * device's array, so calls that overlap in time on one device (several
 * streams, several host threads) race; serialise them. */
int bitlinear_fwd_noalloc(const uint16_t *X, int64_t tokens, int64_t k,
                          const void *packed, int64_t n_out, int n, int m,
                          const double *gamma, float *Y, int8_t *xq,
                          float *x_scale, int32_t *acc, void *stream);

/* The two halves of bitlinear_fwd, for callers that quantise activations
 * once and contract them against several weights, or that time the steps
 * separately.  Same arguments and results as bitlinear_fwd.
 * bitlinear_contract's ws (bitlinear_fwd_workspace_bytes, may be NULL when
 * that is 0) must be all zeros before its first use; every call returns
 * the counters in it to zero, so a workspace is zero-filled once and then
 * reused by one call at a time (calls that overlap on one workspace race).
 * bitlinear_fwd zero-fills what it needs itself. */
int bitlinear_act_quant(const uint16_t *X, int64_t tokens, int64_t k, int8_t *xq,
                        float *x_scale, void *stream);
int bitlinear_contract(const int8_t *xq, const float *x_scale, int64_t tokens,
                       int64_t k, const void *packed, int64_t n_out, int n,
                       int m, const double *gamma, float *Y, int32_t *acc,
                       void *ws, size_t ws_bytes, void *stream);

/* bitlinear_fwd and bitlinear_contract with bf16 outputs: the optional bf16
 * Y epilogue of the block glue, for a BitNet block whose next operation
 * takes bf16 (the 2B4T article §二 describes a bf16 model around the
 * BitLinears); it halves the bytes written at prefill sizes, where the
 * binary32 Y is the largest stream.  Y is the binary32 Y of bitlinear_fwd,
 * rounded once more to the nearest bf16 (ties to even), written as bf16 bit
 * patterns: device uint16 [tokens x n_out], 16-byte aligned.  Every other
 * argument, output, workspace rule and error is that of bitlinear_fwd /
 * bitlinear_contract. */
int bitlinear_fwd_bf16(const uint16_t *X, int64_t tokens, int64_t k,
                       const void *packed, int64_t n_out, int n, int m,
                       const double *gamma, uint16_t *Y, int8_t *xq,
                       float *x_scale, int32_t *acc, void *ws, size_t ws_bytes,
                       void *stream);
int bitlinear_contract_bf16(const int8_t *xq, const float *x_scale,
                            int64_t tokens, int64_t k, const void *packed,
                            int64_t n_out, int n, int m, const double *gamma,
                            uint16_t *Y, int32_t *acc, void *ws,
                            size_t ws_bytes, void *stream);

/* Steps 6-7 for several layers that read the same activations (a block's
 * q, k and v, or gate and up): the contraction and epilogue of
 * bitlinear_contract (BitNet b1.58 2B4T article §四) for every item, with
 * the layers' tiles sharing launches at prefill sizes, so the short layers
 * fill the partial rounds the others leave.  Per item the results (Y, or
 * bf16 Y) are those of bitlinear_contract / bitlinear_contract_bf16 on the
 * same arguments, bit for bit (the int32 sums are exact in any order).
 *   items    host array of `count` (>= 1) descriptors: packed and gamma as
 *            for bitlinear_contract, exactly one of Y (binary32) and Y_bf16
 *            (bf16 bit patterns) non-NULL, both [tokens x n_out] device
 *            arrays, 16-byte aligned; the outputs must not overlap each
 *            other or the inputs.
 *   xq, x_scale, tokens, k, n, m: as for bitlinear_contract, shared.
 *   ws       bitlinear_contract_group_workspace_bytes() bytes (0 above 16
 *            tokens; at most 16 tokens each item runs the decode-shaped
 *            call in turn on this one workspace), zero-filled before the
 *            first use, as for bitlinear_contract.
 * Every item is validated before anything is enqueued; `bitlinear_last_error`
 * names an invalid item's index. */
typedef struct bitlinear_contract_item {
    const void *packed;     /* packed codes [n_out x k]          */
    const double *gamma;    /* absmean scale                     */
    float *Y;               /* binary32 [tokens x n_out] or NULL */
    uint16_t *Y_bf16;       /* bf16 [tokens x n_out] or NULL     */
    int64_t n_out;
} bitlinear_contract_item;

size_t bitlinear_contract_group_workspace_bytes(const bitlinear_contract_item *items, int count,
                                                int64_t tokens, int64_t k);
int bitlinear_contract_group(const bitlinear_contract_item *items, int count, const int8_t *xq,
                             const float *x_scale, int64_t tokens, int64_t k, int n, int m,
                             void *ws, size_t ws_bytes, void *stream);

/* 2:4 on structured-sparse matrix hardware.  The Sparse-BitNet article
 * (§七) ties N:M sparsity's speed-up to matrix units that skip the pruned
 * half (2:4 sparse tensor cores); gfx950's counterpart is
 * v_smfmac_i32_16x16x128_i8, whose sparse operand holds two values per four
 * k plus a 2-bit position per value.  These calls store the 2:4 codes in
 * that operand form and contract them at the sparse instruction's rate;
 * the results are those of bitlinear_contract on the same codes.
 *
 * The sparse-operand + index layout (2 bits per weight): rows in strips of
 * 64 (the last padded with zero codes), k in blocks of 128; superblock
 * (strip p, block kb) at index p*(k/128) + kb holds 64 chunks of 32
 * bytes; chunk c = r + 16q covers rows 64p + 16i + r (i = 0..3) over
 * k = 128kb + 32q .. +31.  For row tile i, element e = 2u + s is slot s of
 * quad u (k = 128kb + 32q + 4u .. +3): 32-bit word 2i of the chunk holds
 * the slot's position in its quad at bits 2e..2e+1, word 2i+1 its code at
 * bits 8(e%4) + 2(e/4) .. +1 (0 = 0, 1 = +1, 3 = -1).  A quad's two
 * nonzero codes take the slots in position order; a single nonzero at
 * position a takes slot 0 if a = 0 (slot 1: position 1, code 0), else
 * slot 1 (slot 0: position 0, code 0); an all-zero quad has positions
 * 0 and 1. */
size_t bitlinear_sp24_packed_bytes(int64_t n_out, int64_t k);

/* Workspace of bitlinear_contract_sp24 (split-k counters and int32 partial
 * tiles for layers with few output tiles, as for the prefill kernel of
 * bitlinear_contract); 0 means ws may be NULL. */
size_t bitlinear_sp24_workspace_bytes(int64_t tokens, int64_t k, int64_t n_out);

/* Codes of a 2:4-masked layer in the sparse-operand layout.  W, mask and
 * gamma as for bitlinear_pack with n:m = 2:4 (the codes are identical:
 * kept by the mask and 2|W| > gamma); mask must be a 2:4 mask (a quad with
 * more than two kept nonzero codes keeps only its first two).  packed_bytes
 * must equal bitlinear_sp24_packed_bytes(n_out, k). */
int bitlinear_pack_sp24(const uint16_t *W, const uint8_t *mask,
                        const double *gamma, int64_t n_out, int64_t k,
                        void *packed, size_t packed_bytes, void *stream);

/* acc = x_q codes^T and Y = acc * gamma * s_t, as bitlinear_contract, for
 * codes in the sparse-operand layout (any token count; one workgroup tile
 * is 256 rows x 64 tokens).  ws: bitlinear_sp24_workspace_bytes() bytes,
 * all zeros before its first use and returned to zero by every call (calls
 * that overlap on one workspace race), or NULL when that is 0. */
int bitlinear_contract_sp24(const int8_t *xq, const float *x_scale,
                            int64_t tokens, int64_t k, const void *packed,
                            int64_t n_out, const double *gamma, float *Y,
                            int32_t *acc, void *ws, size_t ws_bytes,
                            void *stream);

/* Grouped decode: many BitLinear forwards with the same token count (1..16)
 * and N:M pattern in two launches (all activations, then all contractions),
 * e.g. the projections of several layers or of independent streams.  The
 * per-item results are those of bitlinear_fwd.
 *   items  host array of `count` (<= 65535) item descriptors; every
 *          pointer is a device pointer as in bitlinear_fwd.
 *   plan   device buffer of bitlinear_fwd_group_plan_bytes() bytes, written
 *          by bitlinear_fwd_group_plan (which synchronises `stream` once);
 *          it must stay allocated and unchanged while the plan is used.
 *   stages 1 = activation quantisation only, 2 = contraction only (x_q and
 *          x_scale already written), 3 = both (two launches), 4 = both in
 *          one launch: each workgroup quantises the activation rows of the
 *          items it contracts into its LDS (x_q and x_scale are still
 *          written, once per item); results identical to 3.  Stage 4 needs
 *          a plan whose workgroups' activation rows fit their LDS and
 *          split into at most 64 segments of up to 1024 values (rows of
 *          k values take ceil(k / 1024)) per workgroup
 *          (bitlinear_fwd_group_plan_fuses() == 1, e.g. decode plans of
 *          one token); run on any other plan it sets every Y to a quiet NaN
 *          (status BL_OK: the host does not read the plan back).
 * n, m passed to bitlinear_fwd_group must be those the plan was made with;
 * the plan records its sign-slot count, and a contraction run whose n:m
 * has another count (4:8, 3:8 and 2:4 share one) reads no packed byte and
 * sets every Y of every item to a quiet NaN instead (the status is still
 * BL_OK: the host does not read the plan back). */
typedef struct bitlinear_fwd_item {
    const uint16_t *X;      /* bf16 [tokens x k]      */
    const void *packed;     /* packed codes           */
    const double *gamma;    /* absmean scale          */
    float *Y;               /* float [tokens x n_out] */
    int8_t *xq;             /* int8 [tokens x k]      */
    float *x_scale;         /* float [tokens]         */
    int64_t k, n_out;
} bitlinear_fwd_item;

size_t bitlinear_fwd_group_plan_bytes(const bitlinear_fwd_item *items, int count,
                                      int64_t tokens);
int bitlinear_fwd_group_plan(const bitlinear_fwd_item *items, int count,
                             int64_t tokens, int n, int m, void *plan,
                             size_t plan_bytes, void *stream);
int bitlinear_fwd_group(const void *plan, int n, int m, int stages, void *stream);

/* 1 when the plan bitlinear_fwd_group_plan would build for these items can
 * run stage 4 (every workgroup's activation rows fit its LDS and its 64
 * segment slots), 0 when not,
 * minus the status (BL_EINVAL, BL_ESHAPE) for invalid items.  Host only: the plan is built in
 * host memory and discarded. */
int bitlinear_fwd_group_plan_fuses(const bitlinear_fwd_item *items, int count,
                                   int64_t tokens, int n, int m);

/* The bytes bitlinear_fwd_group_plan uploads, written to host memory
 * instead (image: image_bytes >= bitlinear_fwd_group_plan_bytes(), any
 * alignment of 16).  For callers that place the plan themselves (a copy of
 * their own, pinned staging memory) and for host-side checks of a plan; no
 * device call is made, and the item pointers are only stored.  Same
 * validation and errors as bitlinear_fwd_group_plan. */
int bitlinear_fwd_group_plan_host(const bitlinear_fwd_item *items, int count,
                                  int64_t tokens, int n, int m, void *image,
                                  size_t image_bytes);

/* Grouped weight quantisation: steps 1-3 (mask, absmean scale, packing) of
 * many layers with the same N:M pattern in three launches (every mask and
 * partial sum, every gamma, every packed block), e.g. the per-step mask
 * recompute of all BitLinears of a block.  Sparse-BitNet article §三 and
 * §五, BitNet b1.58 2B4T article §一, as for bitlinear_quantize_mask and
 * bitlinear_pack; each item's mask, gamma and packed bytes are bit-identical
 * to what those two calls give.
 *   items  host array of `count` (1..65535) descriptors; W, mask, gamma and
 *          packed are device pointers with the shapes and alignments of
 *          bitlinear_quantize_mask / bitlinear_pack (packed holds
 *          bitlinear_packed_bytes(n_out, k, n, m) bytes).
 *   ws     device workspace of bitlinear_quant_group_workspace_bytes()
 *          bytes, 16-byte aligned; contents need not be initialised.  The
 *          plan records it: runs of one plan share it, so they must not
 *          overlap in time.
 *   plan   device buffer of bitlinear_quant_group_plan_bytes() bytes,
 *          written by bitlinear_quant_group_plan (which synchronises
 *          `stream` once); the host array is not used afterwards.
 * n, m and gamma_over passed to bitlinear_quant_group must be those the plan
 * was made with (a dense-to-sparse schedule builds one plan per pattern).
 * The plan records them; a run with other values writes no mask or packed
 * byte (the packed buffers are sized for the planned pattern) and sets
 * every item's gamma to a quiet NaN, so every forward or backward output
 * formed from those stale codes is NaN (the status is still BL_OK, as the
 * host does not read the plan back).  Errors as for the single-layer
 * calls, plus BL_EWORKSPACE for a short plan or workspace. */
typedef struct bitlinear_quant_item {
    const uint16_t *W;      /* bf16 [n_out x k], read            */
    uint8_t *mask;          /* [n_out x k/8], written            */
    double *gamma;          /* one double, written               */
    void *packed;           /* packed codes, written             */
    int64_t n_out, k;
} bitlinear_quant_item;

size_t bitlinear_quant_group_workspace_bytes(const bitlinear_quant_item *items, int count);
size_t bitlinear_quant_group_plan_bytes(const bitlinear_quant_item *items, int count);
int bitlinear_quant_group_plan(const bitlinear_quant_item *items, int count, int n, int m,
                               int gamma_over, void *ws, size_t ws_bytes, void *plan,
                               size_t plan_bytes, void *stream);
int bitlinear_quant_group(const void *plan, int n, int m, int gamma_over, void *stream);

/* Squared-ReLU gating of a block's feed-forward, fused with the down
 * projection's activation quantisation.  BitNet b1.58 2B4T article §一
 * (squared ReLU in place of SwiGLU; 8-bit activations into every
 * BitLinear).  With G and U the fp32 outputs of the gate and up
 * BitLinears ([tokens x n], row-major), per element, in binary32:
 *   r = max(g, 0),  h = bf16 nearest to RN32(RN32(r * r) * u) (ties even)
 * and then, per token, x_q and x_scale of h exactly as bitlinear_act_quant
 * forms them from a bf16 tensor (so they are the down BitLinear's inputs).
 *   H        device bf16 [tokens x n], written, or NULL.
 *   xq       device int8 [tokens x n]; x_scale device float [tokens].
 * n a positive multiple of 128, tokens*n below 2^31; tokens == 0 is a
 * no-op. */
int bitlinear_relu2_gate(const float *G, const float *U, int64_t tokens, int64_t n,
                         uint16_t *H, int8_t *xq, float *x_scale, void *stream);

/* Its backward (the derivative of h = relu(g)^2 u, with relu'(0) = 0),
 * given dH = dL/dh (fp32, e.g. the down BitLinear's dX), per element, in
 * binary32 with each product rounded:
 *   dU = bf16(RN32(dh * RN32(r * r))),  dG = bf16(RN32(RN32(dh * u) * 2r))
 * (bf16 nearest, ties to even): the dY inputs of the gate and up
 * BitLinears' bitlinear_bwd.  count a multiple of 8 below 2^31. */
int bitlinear_relu2_gate_bwd(const float *dH, const float *G, const float *U, int64_t count,
                             uint16_t *dG, uint16_t *dU, void *stream);

/* Latent-weight update, closing a training step.  Sparse-BitNet article
 * §三 and §六: the latent full-precision weights receive the dense gradient
 * (both straight-through estimators pass it through the mask and the
 * ternary rounding) and the next step recomputes mask, gamma and codes
 * from the updated latent weights.  The pages name no optimiser; this is
 * the plain gradient step, with the latent weights held in binary32:
 *   W_master[i] = RN32(W_master[i] - lr * dW[i])   (one fused rounding)
 *   W[i]        = bf16 nearest to W_master[i] (ties to even), the W the
 *                 next bitlinear_quantize_mask / bitlinear_pack read.
 * A dense-to-sparse schedule (the paper abstract) is the caller passing
 * n:m = 8:8 to the weight-path calls before its switch step and the sparse
 * pattern after it; nothing else changes.
 *   W_master  device float [count], updated in place.
 *   dW        device float [count] (e.g. bitlinear_bwd's dW), read.
 *   W         device bf16 [count], written.
 *   count     a multiple of 8 below 2^31 (n_out*k of a layer); 0 is a
 *             no-op.  BL_ESHAPE otherwise, BL_EINVAL for a null or
 *             misaligned pointer. */
int bitlinear_latent_update(float *W_master, const float *dW, int64_t count, float lr,
                            uint16_t *W, void *stream);

/* Step 8-9: dual straight-through backward.  Sparse-BitNet article §三 and
 * §六: gradients pass straight through the ternary rounding and the
 * sparsification, and masked weights still receive their gradient.
 *   dX[t, c] = gamma * sum_r dY[t, r] * code[r, c]          (binary32)
 *   dW[r, c] = sum_t dY[t, r] * s_t * x_q[t, c]   for all (r, c), masked
 *              entries included                               (binary32)
 * computed on bf16 matrix cores with binary32 accumulation (dY*s_t is
 * rounded to bf16; codes and x_q are exact in bf16).
 *   dY       device bf16 [tokens x n_out].
 *   xq, x_scale  device, as written by bitlinear_fwd.
 *   packed, gamma  device, as for bitlinear_fwd.
 *   dX       device float [tokens x k] or NULL (skip).
 *   dW       device float [n_out x k] or NULL (skip).
 *   ws       device workspace of at least bitlinear_bwd_workspace_bytes()
 *            bytes, 256-byte aligned; its contents need not be initialised
 *            and are clobbered (may be NULL when tokens == 0).
 * n_out must be a multiple of 16.  Calls that overlap on one workspace race.
 */
int bitlinear_bwd(const uint16_t *dY, const int8_t *xq, const float *x_scale,
                  const void *packed, const double *gamma, int64_t tokens,
                  int64_t k, int64_t n_out, int n, int m, float *dX,
                  float *dW, void *ws, size_t ws_bytes, void *stream);

/* Step 8-9 for several layers at once: the same dual straight-through
 * backward (Sparse-BitNet article §三 and §六; formulas as for bitlinear_bwd)
 * of independent layers, in shared launches.  Every item's operands are
 * prepared first, then all their dX and dW products run in launches of up
 * to 16 products (8 layers with both outputs), their tiles dealt over the
 * CUs longest contraction first, so small layers fill what large ones
 * leave instead of each leaving part of the chip idle.  Per item the
 * results are those of bitlinear_bwd on the same arguments, bit for bit
 * (every product contracts k in the same order through the same matrix
 * instruction), except for products bitlinear_bwd splits along k (at most
 * 128 tiles of 128 x 128 and k of 2048 or more): the grouped call sums
 * those in one pass, so they agree to binary32 rounding.  Items whose
 * xq pointers and k are equal (layers fed the same input) share one
 * prepared copy of x_q.
 *   items   host array of `count` (>= 1) descriptors; every pointer is a
 *           device pointer with bitlinear_bwd's meaning, alignment and
 *           rules; a NULL dX or dW skips that output; all items share
 *           tokens and n:m.
 *   ws      device workspace of at least bitlinear_bwd_group_workspace_bytes()
 *           bytes, 256-byte aligned, clobbered (may be NULL when tokens is
 *           0: every dW is then zeroed and nothing else runs).
 * The layers must be independent: no item's dX or dW may overlap any
 * item's inputs or another output (all conversions run before all
 * products).  Every item is validated before anything is enqueued; an
 * invalid one returns its bitlinear_bwd status and `bitlinear_last_error`
 * names its index.  Calls that overlap on one workspace race. */
typedef struct bitlinear_bwd_item {
    const uint16_t *dY;     /* bf16 [tokens x n_out]          */
    const int8_t *xq;       /* int8 [tokens x k] (for dW)     */
    const float *x_scale;   /* float [tokens] (for dW)        */
    const void *packed;     /* packed codes (for dX)          */
    const double *gamma;    /* absmean scale (for dX)         */
    float *dX;              /* float [tokens x k] or NULL     */
    float *dW;              /* float [n_out x k] or NULL      */
    int64_t k, n_out;
} bitlinear_bwd_item;

size_t bitlinear_bwd_group_workspace_bytes(const bitlinear_bwd_item *items, int count,
                                           int64_t tokens);
int bitlinear_bwd_group(const bitlinear_bwd_item *items, int count, int64_t tokens,
                        int n, int m, void *ws, size_t ws_bytes, void *stream);

/* bitlinear_bwd_group in two halves, so that the half that does not wait
 * for dY can run on another stream while earlier work runs (the same
 * method and sections as bitlinear_bwd_group):
 *   BL_BWD_PREPARE  converts what reads only packed codes and x_q (the
 *                   codes for dX, x_q^T for dW) into ws; no product runs
 *                   and nothing but ws is written.
 *   BL_BWD_FINISH   converts dY, then runs every product, reading what a
 *                   BL_BWD_PREPARE call with the same items, tokens, n:m
 *                   and ws left in ws.
 *   both            exactly bitlinear_bwd_group.
 * PREPARE then FINISH gives bitlinear_bwd_group's results bit for bit,
 * provided packed, x_q and ws are not changed in between and FINISH is
 * ordered after PREPARE (same stream, or an event).  With tokens == 0
 * PREPARE does nothing and FINISH zeroes every dW.  Other arguments and
 * errors as for bitlinear_bwd_group; any other phase is BL_EINVAL. */
#define BL_BWD_PREPARE 1
#define BL_BWD_FINISH 2
int bitlinear_bwd_group_phase(const bitlinear_bwd_item *items, int count, int64_t tokens,
                              int n, int m, int phase, void *ws, size_t ws_bytes,
                              void *stream);

/* Steps 8-9 of the down projection of the BitNet b1.58 2B4T feed-forward
 * with the squared-ReLU gating backward (2B4T article §一) fused into its dX
 * product: the dual straight-through backward of bitlinear_bwd (Sparse-BitNet
 * article §三 and §六) whose dX, h's gradient dH, never reaches memory;
 * the product's epilogue forms dG and dU as bitlinear_relu2_gate_bwd forms
 * them from dH.  Results are those of bitlinear_bwd (with the same dW)
 * followed by bitlinear_relu2_gate_bwd, bit for bit.
 *   dY, xq, x_scale, packed, gamma, tokens, k, n_out, n, m, dW, ws:
 *            as for bitlinear_bwd (k is the gate and up layers' n_out).
 *   G, U     device float [tokens x k]: the gate and up outputs, read.
 *   dG, dU   device bf16 [tokens x k]: their output gradients, written.
 * All 16-byte aligned; outputs must not overlap the inputs.  Errors as for
 * bitlinear_bwd.  The products always run on 256-row tiles: a fixed
 * 128 x 128 choice of bitlinear_bwd_tiles falls back to the per-launch
 * choice here, which changes no bit. */
int bitlinear_bwd_relu2_gate(const uint16_t *dY, const int8_t *xq, const float *x_scale,
                             const void *packed, const double *gamma, int64_t tokens,
                             int64_t k, int64_t n_out, int n, int m, const float *G,
                             const float *U, uint16_t *dG, uint16_t *dU, float *dW,
                             void *ws, size_t ws_bytes, void *stream);

/* Output tiles of bitlinear_bwd's products, process-wide: 0 (the default)
 * chooses per launch from the tile counts; 1, 2 or 3 fixes 128 x 128,
 * 256 x 128 or 256 x 256.  Every choice contracts k in the same order
 * through the same matrix instruction, so the results are identical bit
 * for bit.  For tests and tuning; returns BL_EINVAL for any other value. */
int bitlinear_bwd_tiles(int tiles);

/* Static text for a status code. */
const char *bitlinear_status_string(int status);

/* Detail of the last non-zero status returned on this host thread ("" if
 * none).  The pointer stays valid until the next call on this thread. */
const char *bitlinear_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
