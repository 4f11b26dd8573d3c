/*
 * fa.h — C ABI of exact_attention_30_amd: fused exact attention (forward and
 * backward) for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch b and query head h, with kv head
 * hk = h / (Hq / Hkv) (grouped-query attention, consecutive grouping: see
 * "FlashAttention" note, «Grouped-Query Attention» paragraph, and the cuTile
 * page's QUERY_GROUP_SIZE, "Optimización de Flash Attention ... NVIDIA CUDA
 * Tile", «Parte 1 ... interfaz del kernel»):
 *
 *     O = softmax(Q K^T * scale + mask) V
 *
 * where the causal mask lets query i see key j iff j <= i + q_offset
 * ("Optimización de Flash Attention ...", «Atención causal»; the offset is the
 * position of query row 0 among the keys, the input_pos argument of the
 * cuTile kernel in «Parte 1»; it is 0 when queries and keys are one
 * sequence).  The Tq x Tk score and weight matrices are never written to
 * memory: the forward walks key tiles with the
 * online softmax (running max m, sum l, rescale by exp(m - m')), as in
 * "L'attention fusionnée", «Le softmax en ligne», and stores per query row the
 * log-sum-exp L = m + ln(l).  The backward recomputes P = exp(S - L) tile by
 * tile and uses the row reduction Delta_i = sum_d dO_id O_id in place of the
 * softmax Jacobian term ("L'attention fusionnée", «La passe arrière»):
 *
 *     dV = P^T dO,  dS = P * (dO V^T - Delta),  dQ = dS K * scale,
 *     dK = dS^T Q * scale.
 *
 * Head dimensions.  D = 64 and 128 in both element types; D = 96 in bf16 (the
 * 96-component queries and keys that "L'attention fusionnée", «Ce qui reste»,
 * names as the case its kernels could not reach): the forward on 96-column
 * tiles; the backward's products over the 96 columns, on 128-column LDS tiles
 * whose last 32 columns are zeros.
 *
 * Layouts.  All tensors are contiguous, row-major, element type `dt`:
 *     q, o, dout, dq : [B][Hq][Tq][D]
 *     k, v, dk, dv   : [B][Hkv][Tk][D]
 *     lse            : [B][Hq][Tq] float32, natural log, in units of the scaled
 *                      scores (lse_i = log sum_j exp(scale * q_i . k_j)).
 * The calls without a _kv suffix take one length T = Tq = Tk and offset 0.
 *
 * Ownership and execution.  The caller owns every buffer; the library never
 * allocates device memory and keeps no pointer after a call returns.  Each call
 * enqueues kernels on `stream` (a hipStream_t; NULL is the default stream) and
 * returns without waiting for them.  Outputs are overwritten, never
 * accumulated.  Inputs and outputs must not overlap.  Two calls on one stream
 * run in order; calls on different streams that share an output race.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued, in
 * this order, and the first failure is returned:
 *     FA_ERR_SHAPE        B < 0, Tq < 0, Tk < 0, Hq < 1, Hkv < 1,
 *                         Hq % Hkv != 0, query rows without keys (B*Tq > 0
 *                         and Tk == 0), causal with q_offset < 0 or
 *                         q_offset + Tq > 2^31 - 4097, a grid too large to
 *                         index, or one head of a tensor (T * D elements)
 *                         larger than 2^31 - 1 bytes;
 *     FA_ERR_UNSUPPORTED  unknown dtype, D not in {64, 128} (bf16: also 96),
 *                         or scale not a finite positive number;
 *     FA_ERR_NULL         a required pointer is NULL (pointers are not needed
 *                         when there is nothing to compute: B * Tq == 0 for
 *                         the forward, B * Tk == 0 for the backward; with
 *                         Tq == 0 the backward only needs k, v, dk, dv, and
 *                         sets dk = dv = 0);
 *     FA_ERR_ALIGN        a tensor pointer is not 16-byte aligned (lse and the
 *                         workspace: 4-byte and 16-byte);
 *     FA_ERR_HIP          the HIP runtime reported an error while launching.
 * NaN or Inf inside the inputs is not checked and propagates.
 * No exception or abort crosses this interface.
 */
#ifndef EXACT_ATTENTION_30_AMD_FA_H
#define EXACT_ATTENTION_30_AMD_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_BF16 = 0, /* bfloat16 inputs/outputs; bf16 MFMA with fp32 accumulation */
    FA_FP32 = 1, /* float32 inputs/outputs; fp32 MFMA with fp32 accumulation */
    /* bfloat16 q, k, v, dout; float32 o, dq, dk, dv.  The FA_BF16 kernels
     * and arithmetic, with each result stored as the float32 it was before
     * the rounding to bf16 (so bf16(result) is the FA_BF16 result bit for
     * bit).  The backward reads this float32 o; its Delta comes from the
     * preprocess kernel, whose bits equal the FA_BF16 backward's own Delta
     * when o holds bf16 values.  Accepted wherever FA_BF16 is, except
     * fa_bwd_atomic (FA_ERR_UNSUPPORTED); the fp8 calls take no dtype. */
    FA_BF16_F32OUT = 2
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,
    FA_ERR_SHAPE = 2,
    FA_ERR_UNSUPPORTED = 3,
    FA_ERR_ALIGN = 4,
    FA_ERR_HIP = 5,
    FA_ERR_SCRATCH = 6 /* fa_bwd_noalloc: the shapes need more than its static scratch */
} fa_status;

/*
 * Forward pass: o = softmax(q k^T * scale [+ causal mask]) v and lse.
 * Source: "L'attention fusionnée", «Le softmax en ligne» (tiled online softmax,
 * division by l at the end) and «La passe arrière» (L = m + ln l saved for the
 * backward); "FlashAttention: l'attenzione che non spreca memoria",
 * «L'idea: lavorare a tessere» (a query block stays on chip while key/value
 * blocks stream past it).
 *   q [B,Hq,T,D], k/v [B,Hkv,T,D]  (device, read)
 *   o [B,Hq,T,D]                   (device, written)
 *   lse [B,Hq,T] float32           (device, written)
 *   causal: nonzero applies the causal mask.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int T, int D, float scale, int causal, fa_dtype dt, void* stream);

/*
 * Forward pass of Tq query rows against Tk key rows: as fa_fwd, with
 *   q, o [B,Hq,Tq,D], k/v [B,Hkv,Tk,D], lse [B,Hq,Tq];
 *   q_offset (causal only, >= 0): query row i sees keys j <= i + q_offset.
 *   Tk - Tq aligns the last query with the last key (a block of new queries
 *   against cached keys; a single query against Tk keys sees all of them, as
 *   in "L'attention fusionnée", «Un premier kernel plus lent»).
 */
fa_status fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                    int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                    fa_dtype dt, void* stream);

/*
 * The forward with each query block's key range split into up to 8 chunks,
 * for shapes whose query blocks alone give the GPU too few workgroups (few
 * query heads, short query sequences; bf16 only).  Each chunk runs the online
 * softmax over its key tiles and writes its unnormalised numerator, reference
 * max and sum (fp32) to `partial`; a second kernel merges the chunks with the
 * rule by which block results combine ("FlashAttention" note,
 * «Blockergebnisse…»; "L'attention fusionnée", «Le softmax en ligne»):
 * M = max m_s, O = sum 2^(m_s-M) o_s / sum 2^(m_s-M) l_s.
 *   fa_fwd_split_bytes: bytes of `partial` (0: these shapes do not split).
 *   fa_fwd_split: as fa_fwd_kv plus `partial` (device scratch, 16-byte
 *       aligned, contents on return unspecified); NULL or no split: it is
 *       fa_fwd_kv.  O and lse agree with the unsplit forward to rounding.
 */
size_t fa_fwd_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt);

/*
 * The single-kernel backward of the FA2 formulation ("L'attention fusionnée",
 * «La passe arrière»: a workgroup keeps dK and dV of its keys in registers and
 * adds its share of dQ to the rows' accumulators with atomic adds), built as an
 * alternative to fa_bwd for comparison; fa_bwd is faster on this GPU (its dQ
 * kernel recomputes S and dP instead of moving dQ through atomics).  bf16,
 * D = 64 and Tq = Tk (offset 0) only.
 *   fa_bwd_atomic_workspace_bytes: bytes of `workspace` (0: unsupported
 *       shapes): Delta [B][Hq][T], then an fp32 dQ accumulator [B][Hq][T][D].
 *   fa_bwd_atomic: the preprocess (Delta), a zero fill of the accumulator, the
 *       dK/dV kernel accumulating dQ per 32-row query tile (the workgroup's
 *       eight waves summed in LDS, then one fp32 atomic add per element), and
 *       a kernel writing dq = bf16(scale * accumulator).  dK and dV are bitwise
 *       those of fa_bwd_dkdv; dQ agrees with fa_bwd to rounding but is not
 *       bitwise reproducible (the order of the atomic adds varies).
 *       FA_ERR_UNSUPPORTED for other dtypes or head sizes.
 */
size_t fa_bwd_atomic_workspace_bytes(int B, int Hq, int T, int D, fa_dtype dt);
fa_status fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, int B, int Hq, int Hkv, int T, int D, float scale,
                        int causal, fa_dtype dt, void* stream);

/*
 * The static tile table of the bf16 kernels (the blocked loops of
 * "FlashAttention: l'attenzione che non spreca memoria", «L'idea: lavorare a
 * tessere»; the tile sizes of "Optimización de Flash Attention ...", «La pila
 * de optimización»): the rows of one workgroup's block for these shapes.
 *   FA_STAGE_FWD: query rows of the forward; 256 (eight waves), or 128 (four
 *       waves, two workgroups per compute unit) at D = 64 when the 256-row
 *       blocks number fewer than 512.
 *   FA_STAGE_DQ: query rows of the dQ stage; 128 at D = 64 when the 256-row
 *       blocks number fewer than 256, else 256.
 *   FA_STAGE_DKDV: keys of the dK/dV stage (H = Hkv, T = Tk); 128 at D = 64
 *       when the 256-key blocks number fewer than 256, else 256.
 * fp32: 128 always (four waves of 32).  The split rules count these
 * blocks; unsplit, no result depends on the choice.  Host only; returns 0 for
 * shapes, types or stages the kernels reject.
 */
typedef enum { FA_STAGE_FWD = 0, FA_STAGE_DQ = 1, FA_STAGE_DKDV = 2 } fa_stage;
int fa_block_rows(fa_stage stage, int B, int H, int T, int D, fa_dtype dt);
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* partial, int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale,
                       int causal, int q_offset, fa_dtype dt, void* stream);

/*
 * FP8 forward ("FlashAttention: l'attenzione che non spreca memoria",
 * «La frontiera», names narrower formats as the next lever for the matrix
 * units; the pages give no scaling convention).  q, k, v hold e4m3 codes
 * (OCP e4m3fn: 1 sign, 4 exponent, 3 mantissa bits, largest 448, no
 * infinities), one byte per element, layouts as above; the real value of an
 * element is its code times the tensor's descale (q_descale, k_descale,
 * v_descale: finite, > 0).  The result is the forward of those real values:
 * o (bf16) and lse (float32, natural log of the sum over visible keys of
 * exp(scale * q_i . k_j) with the real q, k), as fa_fwd_kv computes them.
 * Both products run on the e4m3 matrix instructions: the scores are exact
 * products summed in fp32; the weights P (at most 2^8 relative to a row's
 * reference, see fa_fwd) are rounded to e4m3 for P V, which bounds the error
 * of O_id by about 2^-4 sum_j P_ij |v_jd| (relative rounding of each weight)
 * plus 2^-10 sum_j |v_jd| / l_i (weights in e4m3's subnormal range), l_i the
 * row sum of the weights relative to the row max.
 *   fa_fwd_fp8_workspace_bytes: bytes of `workspace`, B * Hkv *
 *       ceil(Tk / 64) * 64 * D (V transposed, tile by tile; 0 for invalid
 *       shapes).
 *   fa_fwd_fp8: D must be 64 or 128 (FA_ERR_UNSUPPORTED otherwise, also for
 *       a descale that is not finite and positive); workspace: device,
 *       16-byte aligned, contents on return unspecified; other arguments and
 *       errors as fa_fwd_kv.  It is fa_fp8_transpose_v into `workspace`
 *       followed by fa_fwd_fp8_vt.
 *   fa_fp8_transpose_v: writes V (e4m3 codes, [B][Hkv][Tk][D]) transposed
 *       into vt (fa_fwd_fp8_workspace_bytes bytes, 16-byte aligned): per kv
 *       head and 64-key tile t, D rows of 64 bytes, byte q of row d holding
 *       V[64t + 32(q/32) + 8((q%16)/4) + 4((q/16)%2) + q%4][d] (0 past Tk),
 *       the key order the product of weights and values reads.  Errors:
 *       FA_ERR_SHAPE (B < 0, Hkv < 1, Tk < 0, sizes past 2^31),
 *       FA_ERR_UNSUPPORTED (D), FA_ERR_NULL, FA_ERR_ALIGN, FA_ERR_HIP.
 *   fa_fwd_fp8_vt: the forward with V given as fa_fp8_transpose_v wrote it
 *       (a caller that keeps V fixed across calls transposes it once).
 */
size_t fa_fwd_fp8_workspace_bytes(int B, int Hkv, int Tk, int D);
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float q_descale, float k_descale,
                     float v_descale, void* o, float* lse, void* workspace, int B, int Hq, int Hkv,
                     int Tq, int Tk, int D, float scale, int causal, int q_offset, void* stream);
fa_status fa_fp8_transpose_v(const void* v, void* vt, int B, int Hkv, int Tk, int D, void* stream);
fa_status fa_fwd_fp8_vt(const void* q, const void* k, const void* vt, float q_descale,
                        float k_descale, float v_descale, void* o, float* lse, int B, int Hq,
                        int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                        void* stream);

/*
 * Bytes of device workspace fa_bwd (fa_bwd_kv) needs: one float32 Delta per
 * query row, B * Hq * Tq * 4 rounded up to 256, followed by one region for the
 * partial sums of the split stages, of the larger of fa_bwd_dkdv_split_bytes
 * and fa_bwd_dq_split_bytes (0 when neither stage splits).  Returns 0 for
 * invalid or empty shapes.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int T, int D, fa_dtype dt);
size_t fa_bwd_kv_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt);

/*
 * Backward pass of fa_fwd for the upstream gradient dout: writes dq, dk, dv.
 * Source: "L'attention fusionnée", «La passe arrière»: P is recomputed from
 * lse, Delta = rowsum(dout * o) replaces the Jacobian term, and two kernels
 * (one for dK/dV per key tile, one for dQ per query tile walking keys in the
 * forward's order) avoid atomic additions, so results are bitwise
 * reproducible run to run.  The results are bitwise those of
 * fa_bwd_preprocess, fa_bwd_dkdv and fa_bwd_dq; for bf16 the dQ kernel forms
 * Delta itself (in the preprocess kernel's order) and runs first, writing
 * Delta into the workspace for the dK/dV kernel.
 *   q, k, v, o, lse: as produced for/by fa_fwd with the same scale and causal;
 *   dout [B,Hq,T,D] (device, read); dq [B,Hq,T,D], dk/dv [B,Hkv,T,D]
 *   (device, written); workspace: fa_bwd_workspace_bytes(...) bytes of device
 *   memory (scratch, contents on return unspecified).
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int Hq,
                 int Hkv, int T, int D, float scale, int causal, fa_dtype dt, void* stream);

/*
 * Backward pass of fa_fwd_kv: as fa_bwd, with dq [B,Hq,Tq,D], dk/dv
 * [B,Hkv,Tk,D] and the same q_offset as the forward.  Keys that no query row
 * sees get dk = dv = 0.
 */
fa_status fa_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace, int B, int Hq,
                    int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                    fa_dtype dt, void* stream);

/*
 * The three stages of fa_bwd, for callers that schedule or time them
 * separately.  `delta` is a [B,Hq,T] float32 device buffer (for instance the
 * start of the fa_bwd workspace).  The _kv forms take Tq, Tk and q_offset as
 * fa_bwd_kv does (delta [B,Hq,Tq]: fa_bwd_preprocess with T = Tq).
 *   fa_bwd_preprocess: delta_i = sum_d dout_id * o_id ("L'attention
 *       fusionnée", «La passe arrière», the row reduction run before the rest).
 *   fa_bwd_dkdv: dk, dv for every key row (per key tile, summed over the query
 *       heads of the kv group).
 *   fa_bwd_dq: dq for every query row.
 */
fa_status fa_bwd_preprocess(const void* o, const void* dout, float* delta, int B, int Hq, int T,
                            int D, fa_dtype dt, void* stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, const float* delta, void* dk, void* dv, int B, int Hq,
                      int Hkv, int T, int D, float scale, int causal, fa_dtype dt, void* stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, const float* delta, void* dq, int B, int Hq, int Hkv, int T,
                    int D, float scale, int causal, fa_dtype dt, void* stream);
fa_status fa_bwd_dkdv_kv(const void* q, const void* k, const void* v, const void* dout,
                         const float* lse, const float* delta, void* dk, void* dv, int B, int Hq,
                         int Hkv, int Tq, int Tk, int D, float scale, int causal, int q_offset,
                         fa_dtype dt, void* stream);
fa_status fa_bwd_dq_kv(const void* q, const void* k, const void* v, const void* dout,
                       const float* lse, const float* delta, void* dq, int B, int Hq, int Hkv,
                       int Tq, int Tk, int D, float scale, int causal, int q_offset, fa_dtype dt,
                       void* stream);

/*
 * The dK/dV stage with its query side split, for shapes whose key blocks
 * alone give the GPU too few workgroups (few kv heads, short key sequences;
 * bf16 only).  Each key block's (query head, query tile) pairs are cut into
 * up to 8 contiguous chunks; every chunk writes fp32 partial sums of dK and dV
 * into `partial`, and a second kernel adds the chunks in chunk order, scales
 * dK and rounds both to bf16, so the result is the same on every run.  This is
 * the split of the dK/dV work of "L'attention fusionnée", «La passe arrière»,
 * over more workgroups; the terms themselves are those of fa_bwd_dkdv.
 *   fa_bwd_dkdv_split_bytes: bytes of `partial` for these shapes (0: the
 *       shapes do not split; the 256-byte rounded size of
 *       2 * chunks * B * Hkv * Tk * D float32 otherwise).
 *   fa_bwd_dkdv_split: as fa_bwd_dkdv_kv, plus `partial` (device scratch of
 *       fa_bwd_dkdv_split_bytes bytes, 16-byte aligned, contents on return
 *       unspecified).  With partial == NULL, or when the shapes do not split,
 *       it is fa_bwd_dkdv_kv.  fa_bwd and fa_bwd_kv use it with the part of
 *       their workspace after Delta.
 */
size_t fa_bwd_dkdv_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt);
fa_status fa_bwd_dkdv_split(const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, const float* delta, void* dk, void* dv, void* partial,
                            int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                            int q_offset, fa_dtype dt, void* stream);

/*
 * The dQ stage with its key range split the same way, for shapes whose query
 * blocks alone give the GPU too few workgroups: up to 8 contiguous chunks of
 * each query block's key tiles, fp32 partial sums of dQ in `partial`, added in
 * chunk order, scaled and rounded to bf16 by a second kernel (bf16 only).
 *   fa_bwd_dq_split_bytes: bytes of `partial` (0: no split; the 256-byte
 *       rounded size of chunks * B * Hq * Tq * D float32 otherwise).
 *   fa_bwd_dq_split: as fa_bwd_dq_kv, plus `partial` (NULL or no split: it is
 *       fa_bwd_dq_kv).  fa_bwd and fa_bwd_kv give both split stages the part
 *       of their workspace after Delta, one after the other.
 */
size_t fa_bwd_dq_split_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, fa_dtype dt);
fa_status fa_bwd_dq_split(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, const float* delta, void* dq, void* partial, int B,
                          int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                          int q_offset, fa_dtype dt, void* stream);

/*
 * The dQ stage forming Delta itself, as fa_bwd and fa_bwd_kv run it in bf16
 * (Delta = rowsum(dout * o), "L'attention fusionnée", «La passe arrière»):
 * the dQ kernel already holds dout of its query rows, also reads o, and
 * writes Delta in the summation order of the preprocess kernel (bitwise the
 * output of fa_bwd_preprocess) before using it; run it before the dK/dV
 * stage, which reads that Delta.  Saves the preprocess launch.
 *   o [B,Hq,Tq,D] (device, read); delta [B,Hq,Tq] float32 (device,
 *   written); q, k, v, dout, lse, dq, partial and the sizes as
 *   fa_bwd_dq_split.  bf16 inputs only: FA_ERR_UNSUPPORTED for fp32; with
 *   FA_BF16_F32OUT (float32 o) it runs fa_bwd_preprocess, then
 *   fa_bwd_dq_split, with the same results.  The other errors as
 *   fa_bwd_dq_split, FA_ERR_NULL / FA_ERR_ALIGN also for o.
 */
fa_status fa_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, float* delta, void* dq, void* partial,
                          int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                          int q_offset, fa_dtype dt, void* stream);

/*
 * Size of the static scratch of fa_bwd_noalloc, per GPU: 64 MiB.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fa_bwd_kv for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels, with the workspace taken from a static device array of the
 * library (FA_NOALLOC_SCRATCH_BYTES, one copy on every GPU the library runs
 * on, held until the process ends) instead of a caller buffer.  The call
 * allocates nothing and calls no allocating routine.
 *   Arguments, layouts, results and errors: as fa_bwd_kv without `workspace`
 *   (the results are bitwise those of fa_bwd_kv), plus FA_ERR_SCRATCH when
 *   fa_bwd_kv_workspace_bytes(...) of these shapes exceeds
 *   FA_NOALLOC_SCRATCH_BYTES (checked after the shape and dtype checks,
 *   before anything is enqueued).  `stream` must belong to the current
 *   device: the scratch used is the current device's, whose address the
 *   first call on each device looks up (FA_ERR_HIP if that fails).
 *   Every call on one GPU shares that GPU's scratch and leaves its own
 *   contents there; nothing in it needs clearing between calls (Delta and
 *   every partial sum are written before they are read).  Calls that overlap
 *   on one GPU (different streams, or host threads) race on the scratch: run
 *   them on one stream, one after the other.
 */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
                         int q_offset, fa_dtype dt, void* stream);

/* Static, human-readable name of a status code. */
const char* fa_status_string(fa_status s);

/* Library version string, e.g. "0.2.0". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_30_AMD_FA_H */
