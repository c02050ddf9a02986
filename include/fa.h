/*
 * fa.h — C ABI of libfa.so: exact attention forward (FlashAttention) on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (unite.ai page "Atención Flash: Revolucionando la Eficiencia
 * de los Modelos de Transformador": the standard-attention code block defines
 * it; section "La Matemática detrás de la Atención Flash", formulas 1 and 2,
 * and section "Detalles de Implementación" give the blocked evaluation with a
 * running row maximum and running sum; nisoo.com page "Un'immersione
 * approfondita nell'algoritmo FlashAttention – parte 3", sections "Softmax
 * Sicura" and "SafeSoftmax con Calcolo Normalizzatore Online"):
 *
 *     for every (b, h) and query row i:
 *       S_ij  = scale * <Q[b,h,i,:], K[b,h,j,:]>           j = 0 .. N-1
 *       O[b,h,i,:] = sum_j exp(S_ij) V[b,h,j,:] / sum_j exp(S_ij)
 *       LSE[b,h,i] = ln sum_j exp(S_ij)
 *
 * No causal or padding mask, no dropout.  The N x N matrix S is never
 * written to memory: it is produced tile by tile on chip and folded into a
 * running (max, sum, output) state per query row.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum {
    FA_DTYPE_FP32 = 0,
    FA_DTYPE_FP16 = 1,
    FA_DTYPE_BF16 = 2
} fa_dtype_t;

/* Return codes of fa_forward. */
typedef enum {
    FA_OK = 0,
    FA_ERR_NULL_POINTER = 1,          /* a tensor pointer is NULL while B*H*N > 0      */
    FA_ERR_BAD_SHAPE = 2,             /* a size negative, sizes overflow, H_kv !| H      */
    FA_ERR_UNSUPPORTED_HEAD_DIM = 3,  /* d is not 64 or 128                             */
    FA_ERR_UNSUPPORTED_DTYPE = 4,     /* dtype is not one of fa_dtype_t                 */
    FA_ERR_MISALIGNED = 5,            /* Q/K/V/O not 16-byte or LSE not 4-byte aligned  */
    FA_ERR_ALIAS = 6,                 /* O or LSE overlaps an input or each other       */
    FA_ERR_BAD_SCALE = 7,             /* scale not finite, or |scale|*log2(e) overflows */
    FA_ERR_LAUNCH = 8,                /* the HIP kernel launch itself failed            */
    FA_ERR_WORKSPACE = 9,             /* workspace NULL or smaller than required        */
    FA_ERR_SCRATCH_LIMIT = 10         /* sizes need more than FA_SCRATCH_BYTES          */
} fa_status_t;

/* Bytes of the fixed device scratch of fa_forward_split_noalloc (64 MiB). */
#define FA_SCRATCH_BYTES ((int64_t)64 << 20)

/*
 * fa_forward — attention forward for a batch of heads.
 *
 * Q, K, V  device pointers, read only.  Dense row-major (B, H, N, d) tensors
 *          of `dtype` (no strides; element [b,h,n,e] sits at
 *          ((b*H + h)*N + n)*d + e).  They may alias each other.
 * O        device pointer, written: (B, H, N, d), same dtype and layout.
 * LSE      device pointer, written: (B, H, N) float32, the natural-log
 *          log-sum-exp of row i of the *scaled* scores, ln sum_j exp(S_ij).
 * B, H, N  batch, heads, sequence length (queries = keys = N).  N may be any
 *          value >= 0; a partial last tile is masked, not padded by the caller.
 * d        head dimension: 64 or 128.
 * scale    multiplies Q.K^T before the softmax (usually 1/sqrt(d)); any finite
 *          value.  It is applied to the float32 scores, never to the inputs.
 * dtype    fa_dtype_t.  fp16/bf16: both products run on MFMA with float32
 *          accumulation, and the softmax weights are rounded to `dtype` for the
 *          second product.  fp32: both products use float32 MFMA.
 * stream   HIP stream to launch on (0 = the null stream).  The call is
 *          asynchronous: it returns after the launch; results are ready when
 *          the stream reaches that point.
 *
 * Ownership: the caller owns every buffer.  The library allocates, frees,
 * copies and synchronises nothing and keeps no state between calls
 * (reentrant, thread safe).  Every element of O and LSE is written.
 * Pointers must belong to the current HIP device.
 *
 * Errors: arguments are checked on the host before anything is launched;
 * a failed check returns its code and touches no memory.  B*H*N == 0 returns
 * FA_OK without a launch (pointers may then be NULL).  FA_ERR_LAUNCH reports a
 * launch failure.  Faults during execution surface at the caller's next
 * synchronisation, not here.
 */
int fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int64_t B, int64_t H, int64_t N, int64_t d,
               float scale, int dtype, hipStream_t stream);

/*
 * fa_forward_gqa — the same forward pass with grouped K/V heads (grouped-query
 * attention; H_kv = 1 is multi-query attention).  unite.ai page, section
 * "Atención Flash-2", item 3, names both variants; this is the reading:
 *
 *     query head h of batch b attends to K/V head h / (H / H_kv) of batch b:
 *       S_ij  = scale * <Q[b,h,i,:], K[b,h/g,j,:]>,   g = H / H_kv
 *       O[b,h,i,:] = sum_j exp(S_ij) V[b,h/g,j,:] / sum_j exp(S_ij)
 *       LSE[b,h,i] = ln sum_j exp(S_ij)
 *
 * Q, O     (B, H, N, d) as for fa_forward.
 * K, V     (B, H_kv, N, d), same dtype and layout rules.
 * H_kv     >= 1 and divides H (else FA_ERR_BAD_SHAPE, unless B*H*N == 0).
 * Everything else (LSE, scale, dtype, stream, ownership, errors) is as for
 * fa_forward, which is fa_forward_gqa with H_kv = H.
 */
int fa_forward_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                   float scale, int dtype, hipStream_t stream);

/*
 * fa_backward — gradients of fa_forward_gqa with respect to Q, K and V.
 *
 * The unite.ai page names recomputation in the backward pass (section
 * "Introducción a la Atención Flash", item 2) and a faster backward pass
 * (section "Atención Flash-2", item 2); the nisoo.com page (part 3) explains
 * the recomputation.  This is the gradient of the forward definition, per
 * query head h (K/V head g = h / (H / H_kv)), with P recomputed from Q, K
 * and the forward's LSE instead of being stored:
 *
 *     P_ij  = exp(scale <Q_i, K_j> - LSE_i)
 *     D_i   = sum_e dO_ie O_ie
 *     dV_g += P^T dO
 *     dS_ij = P_ij (sum_e dO_ie V_je - D_i)
 *     dQ    = scale dS K,    dK_g += scale dS^T Q
 *
 * Q, O, dO  device, read only, (B, H, N, d) of `dtype`.
 * K, V      device, read only, (B, H_kv, N, d).
 * LSE       device, read only, (B, H, N) float32: the LSE that fa_forward /
 *           fa_forward_gqa wrote for these Q, K, V and scale.
 * Dws       device, written, (B, H, N) float32 workspace: receives D_i (the
 *           caller allocates it; its contents on return are D).
 * dQ        device, written, (B, H, N, d) of `dtype`.
 * dK, dV    device, written, (B, H_kv, N, d) of `dtype`.
 * dtype     FA_DTYPE_FP16 or FA_DTYPE_BF16 (fp32 inputs: FA_ERR_UNSUPPORTED_DTYPE).
 *           Products run on MFMA with float32 accumulation; P and dS are
 *           rounded to `dtype` before their second products; outputs are
 *           rounded to `dtype`.
 * d, scale, stream, H_kv: as for fa_forward_gqa.
 *
 * Ownership and errors as for fa_forward; the outputs and Dws must not
 * overlap each other or any input (FA_ERR_ALIAS).  The call launches three
 * kernels in stream order and returns after queueing them.
 */
int fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* LSE, float* Dws, void* dQ, void* dK, void* dV,
                int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                float scale, int dtype, hipStream_t stream);

/*
 * fa_forward_fp8 — the forward pass with FP8 inputs.  The unite.ai page,
 * section "Atención Flash-3", names low-precision FP8 for the attention
 * products without fixing a format or scaling; this is the reading:
 *
 * Q, K, V  device, read only: OCP FP8 E4M3 codes (1 byte each: sign, 4
 *          exponent bits with bias 7, 3 mantissa bits; no infinities, S.1111.111
 *          is NaN), layouts as for fa_forward_gqa ((B, H, N, d) and
 *          (B, H_kv, N, d)).  The values they stand for are
 *          q_descale * Q, k_descale * K, v_descale * V (float32 factors,
 *          one per tensor, any finite value).
 * O        device, written: (B, H, N, d) of out_dtype (FA_DTYPE_BF16,
 *          FA_DTYPE_FP16 or FA_DTYPE_FP32), the attention output of the
 *          dequantised values, rounded to nearest even.
 * LSE      device, written: (B, H, N) float32,
 *          ln sum_j exp(scale * q_descale * k_descale * <Q_i, K_j>).
 * Both products run on the e4m3 matrix instructions (float32 accumulation);
 * the softmax is float32; the weights P are rounded to e4m3 before the
 * product with V.  Everything else (shapes, d, H_kv, ownership, errors) as
 * for fa_forward_gqa; a non-finite descale factor is FA_ERR_BAD_SCALE.
 */
int fa_forward_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                   float scale, float q_descale, float k_descale, float v_descale,
                   int out_dtype, hipStream_t stream);

/*
 * fa_forward_split — fa_forward_gqa with the keys of every head cut into
 * ranges processed by separate workgroups, then merged.  For few heads and
 * long sequences (B*H*ceil(N/256) below the number of compute units) this
 * fills the GPU that one query tile per workgroup leaves idle.
 *
 * Each range r yields the normalised partial result of the rows against its
 * keys alone, (O_r, LSE_r); the ranges merge by the softmax merge of the
 * unite.ai page (section "La Matemática detrás de la Atención Flash",
 * formula 2, normalisers restored), in log-sum-exp form:
 *
 *     m = max_r LSE_r,   w_r = exp(LSE_r - m)
 *     O = sum_r w_r O_r / sum_r w_r,   LSE = m + ln sum_r w_r
 *
 * which is exactly the unsplit result up to rounding.  The partials are kept
 * in float32 in the caller's workspace.
 *
 * splits    requested number of ranges, >= 1.  Ranges hold a whole number
 *           of 64-key tiles and none is empty, so the count used is
 *           ceil(N / kchunk) with kchunk = 64 * ceil(ceil(N/64) / splits),
 *           at most `splits`.  One range runs fa_forward_gqa (no workspace
 *           needed).
 * workspace device, 16-byte aligned, at least fa_split_workspace_bytes(...)
 *           bytes, overlapping no other argument; its contents on return are
 *           the partial results (O parts (B*H, ranges, N, d) float32, then
 *           LSE parts (B*H, ranges, N) float32).
 * Everything else as for fa_forward_gqa.  FA_ERR_WORKSPACE: workspace NULL
 * or too small.  Two kernels are launched in stream order.
 */
int fa_forward_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                     float scale, int dtype, int64_t splits, void* workspace,
                     int64_t workspace_bytes, hipStream_t stream);

/*
 * fa_forward_split_noalloc — fa_forward_split with no workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It calls
 * no allocating routine: the partial results go to a fixed device array of
 * FA_SCRATCH_BYTES inside the library, one per GPU, held until the process
 * ends (its address is looked up on the first call on each device).
 *
 * Arguments, split plan, result, ownership and errors are those of
 * fa_forward_split, minus workspace / workspace_bytes.  The partials need
 * fa_split_workspace_bytes(B, H, N, d, splits) bytes; more than
 * FA_SCRATCH_BYTES returns FA_ERR_SCRATCH_LIMIT before anything is launched
 * (one range needs none: it runs fa_forward_gqa).  Every call on a GPU shares
 * that GPU's scratch, so calls that may overlap in time on one GPU (other
 * streams, other host threads) race and give wrong results: order them on
 * one stream or use fa_forward_split with a workspace of their own.
 */
int fa_forward_split_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                             float scale, int dtype, int64_t splits, hipStream_t stream);

/* Workspace bytes fa_forward_split needs for these sizes and requested
 * splits (0 when one range results or B*H*N == 0; -1 for invalid sizes). */
int64_t fa_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t splits);

/* A split count for fa_forward_split on the MI355X's 256 compute units:
 * the count with the fewest estimated workgroup-tile steps (waves of
 * workgroups times tiles per range, plus the merge's memory traffic), at
 * most 64 and keeping at least 512 keys per range; 1 when no split pays off
 * or the sizes are invalid. */
int64_t fa_split_suggest(int64_t B, int64_t H, int64_t N, int64_t d, int dtype);

/*
 * fa_merge — merge S normalised partial attention results per row (the
 * merge of fa_forward_split on its own; also the combine step for keys
 * sharded over devices, each shard having produced (O_s, LSE_s)).
 *
 * O_parts   device, read only, (G, S, M, d) float32: part s of row i of
 *           group g at ((g*S + s)*M + i)*d.
 * LSE_parts device, read only, (G, S, M) float32, natural log.  A part with
 *           LSE = -inf has no keys and weighs 0; a row whose parts are all
 *           -inf gets O = 0 and LSE = -inf.
 * O         device, written, (G, M, d) of `dtype` (rounded to nearest even).
 * LSE       device, written, (G, M) float32.
 * S >= 1; d 64 or 128; outputs must not overlap each other or the inputs.
 * Ownership and errors as for fa_forward; G*M == 0 returns FA_OK.
 */
int fa_merge(const float* O_parts, const float* LSE_parts, int64_t G, int64_t S, int64_t M,
             int64_t d, void* O, float* LSE, int dtype, hipStream_t stream);

/* Static, human-readable name of a return code ("unknown status" otherwise). */
const char* fa_status_string(int status);

/* Static string naming the library build and its kernel tile configuration. */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
