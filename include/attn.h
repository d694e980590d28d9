/*
 * attn.h -- C ABI of the MI355X (gfx950) exact attention forward library.
 *
 * The library computes, without ever writing the Nq x Nkv score matrix to
 * memory, the exact attention forward pass
 *
 *     O = softmax(scale * Q K^T + mask) V,    LSE = log-sum-exp of each row,
 *
 * by tiling Q into row blocks and streaming K/V tiles through on-chip memory
 * with the online softmax (running row max m, running row sum l, rescaled
 * output accumulator).  Sources: FlashAttention summary page (method
 * paragraph: tiles in SRAM, running (m, l) and output kept on chip, exact);
 * FlashAttention v1/v2/v3/v4 blog post, section "El truco que hizo posible
 * todo: online softmax" (the recurrence); FFPA README, section "Split-D and
 * TiledMMA" (head dims 320..1024 by chunking D).
 *
 * Semantics shared by every entry point
 * -------------------------------------
 *  Layout (FFPA README, "Quick Start": layout follows SDPA, (B, H, N, D)):
 *    q   : (B, Hq,  Nq,  D) contiguous, row-major
 *    k, v: (B, Hkv, Nkv, D) contiguous, row-major
 *    o   : (B, Hq,  Nq,  D) contiguous, row-major
 *    lse : (B, Hq,  Nq)     contiguous float32, natural log; may be NULL
 *  GQA/MQA (FFPA README feature table; ZYFA article, "Who should actually run
 *    it"): Hq must be a multiple of Hkv; query head hq reads KV head
 *    hq / (Hq / Hkv) (contiguous groups).  Cross attention: Nq != Nkv.
 *  Causal (causal != 0): key j is visible to query i iff j <= i + (Nkv - Nq)
 *    (bottom-right alignment; equal to top-left when Nq == Nkv).  A row that
 *    sees no key gets O = 0 and LSE = -inf.
 *  scale multiplies Q K^T before the mask and softmax; any finite value.
 *  LSE_i = ln(sum over visible j of exp(s_ij)) in float32.
 *  Every element of o and lse is written; no other memory is written.
 *  Results are bitwise identical from launch to launch (no atomics, fixed
 *  reduction order) -- ZYFA article, "The details that make it
 *  production-grade" (determinism; LSE lets key-range results merge).
 *
 *  Supported sizes: B, Hq, Hkv, Nq, Nkv >= 1.  Head dim D: ATTN_BF16 any
 *    multiple of 32 in [32, 1024] (above 256 on the split-D kernels, an odd
 *    multiple of 32 at the layout of D + 32); ATTN_F32 a multiple of 32 in
 *    [32, 128]; fp8 a multiple of 64 in [64, 256].  Each (batch, head) slab of q, k, v and o must be
 *    smaller than 2^31 bytes; B*Hq*ceil(Nq/32) < 2^31.
 *
 * Ownership, synchronisation and errors
 * -------------------------------------
 *  All tensor pointers are DEVICE pointers owned by the caller; they must stay
 *  valid until the enqueued work on `stream` completes.  Pointers must be
 *  16-byte aligned.  The calls are asynchronous: they validate, enqueue one
 *  kernel on `stream` (NULL = the default stream) and return without
 *  synchronising the host.  The library allocates no memory and keeps no
 *  per-shape state, so calls may be captured into a HIP graph.
 *  Return value: ATTN_OK, or an attn_status code.  On a validation failure
 *  nothing is enqueued.  ATTN_ERR_HIP reports a launch failure returned by
 *  the HIP runtime (for example: no device).  Faults inside the kernel
 *  surface at the caller's next synchronisation, as usual in HIP.  A
 *  human-readable description of the last failure on the calling thread is
 *  returned by attn_last_error().  No C++ exception crosses this boundary.
 */
#ifndef EXACT_IO_AWARE_ATTN_AMD_ATTN_H
#define EXACT_IO_AWARE_ATTN_AMD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t is an opaque pointer; the ABI takes it as void* so that this
 * header needs no HIP include. */
typedef void* attn_stream_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* NULL pointer, size < 1, Hq % Hkv != 0, non-finite
                               scale, unknown dtype, misaligned pointer,
                               non-positive or non-finite descale value */
  ATTN_ERR_UNSUPPORTED = 2, /* valid but outside the supported D / size range */
  ATTN_ERR_HIP = 3          /* the HIP runtime refused the launch */
} attn_status;

typedef enum {
  ATTN_F32 = 0,      /* q, k, v, o float32; products and softmax in float32  */
  ATTN_BF16 = 1,     /* q, k, v, o bfloat16; float32 accumulation and softmax */
  ATTN_FP8_E4M3 = 2  /* q, k, v OCP e4m3fn codes; o bfloat16 (see attn_fwd_fp8) */
} attn_dtype;

/*
 * attn_fwd -- exact attention forward (see the semantics above).
 *   q, k, v : device inputs of element type `dtype`
 *   o       : device output; float32 for ATTN_F32, bfloat16 otherwise
 *   lse     : device float32 output (B, Hq, Nq), or NULL to skip it
 *   B, Hq, Hkv, Nq, Nkv, D : sizes (see "Supported sizes")
 *   causal  : 0 = no mask, nonzero = bottom-right causal mask
 *   scale   : multiplier of Q K^T (the caller passes 1/sqrt(D) for SDPA's
 *             default)
 *   dtype   : attn_dtype; ATTN_FP8_E4M3 here means all descales equal 1
 *   stream  : hipStream_t to enqueue on (NULL = default stream)
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
             int causal, float scale, int dtype, attn_stream_t stream);

/*
 * attn_fwd_fp8 -- exact attention forward on per-tensor-scaled e4m3 inputs.
 * ZYFA article, sections "Getting started with ZYFA" and "Who should actually
 * run it": FP8 calls take one descale per tensor and the kernel reads the
 * descales from GPU memory, so a call never waits on the host.
 *   q, k, v    : OCP e4m3fn codes (1 byte each), layouts as above
 *   descale_q, descale_k, descale_v : DEVICE pointers to one float32 each
 *                (the value each code is multiplied by); NULL means 1.0.
 *                The values must be positive and finite; they are read by the
 *                kernel, so the host never checks them.
 *   o          : bfloat16 output; lse as above
 * Computed: s_ij = scale * dq * dk * (q8_i . k8_j), O = dv * softmax(s) v8.
 * Q K^T runs on the fp8 matrix cores; P V runs with P rounded to bfloat16
 * and the e4m3 values of V widened exactly to bfloat16.  Supported D:
 * multiples of 64 in [64, 256].
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                 int causal, float scale,
                 const float* descale_q, const float* descale_k, const float* descale_v,
                 attn_stream_t stream);

/*
 * Key ranges and their merge (split-KV, chunked prefill, ring attention).
 * ZYFA article, section "The details that make it production-grade": results
 * computed over different key ranges merge consistently through the LSE,
 * which is what chunked prefill requires.  For partial results (O_p, LSE_p)
 * over disjoint key ranges, each normalised over its own range:
 *     LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p.
 */

/* Probability precision of attn_fwd_fp8_p (the P of P V). */
typedef enum {
  ATTN_P_E4M3 = 1,      /* e4m3 codes of 2^(x - E), nearest, ties to even */
  ATTN_P_E4M3_LEAN = 2  /* Lean P codes rne(8 (x - E) + 56): no exponential */
} attn_p_mode;

/*
 * attn_fwd_fp8_p -- attn_fwd_fp8 with e4m3 probabilities, so that both
 * products run on the fp8 matrix instruction (ZYFA article, section "The
 * three techniques, in plain terms": per-block scaling with a rounded row
 * sum, and Lean P).  Not exact attention: each probability is rounded to
 * e4m3.  With base-2 scores x_ij = scale dq dk log2(e) (q8_i . k8_j), for
 * each row and each 64-key block b (keys [64 b, 64 b + 64)):
 *   E = ceil(max over the block's visible keys of x_ij) - 8,
 *   p_ij = decode(code_ij) 2^E with code_ij as `p_mode` says,
 *   O_i = dv sum_j p_ij v8_j / sum_j p_ij,  LSE_i = ln sum_j p_ij
 * (the row sum is taken from the same rounded p_ij, on the matrix unit).
 *   p_mode : ATTN_P_E4M3 or ATTN_P_E4M3_LEAN
 * D = 64 or 128, scale > 0; other arguments, outputs and errors as
 * attn_fwd_fp8.
 */
int attn_fwd_fp8_p(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                   int causal, float scale,
                   const float* descale_q, const float* descale_k, const float* descale_v,
                   int p_mode, attn_stream_t stream);

/*
 * attn_fwd_exp_poly -- attn_fwd (bf16) with each probability's exponential
 * computed by a polynomial on the FMA pipe instead of the transcendental
 * instruction (blog post "FlashAttention v1/v2/v3/v4", table of ideas: FA4's
 * polynomial exponential): 2^y = 2^floor(y) p(y - floor(y)) with the cubic
 * p(f) = 1 + 0.69511634 f + 0.22764705 f^2 + 0.07706515 f^3, relative error
 * at most 8.6e-5 on [0, 1).  Inexact only by that error, below bf16
 * rounding.  bf16 q, k, v, o; D = 64 or 128; scale > 0; outputs and errors as
 * attn_fwd.
 */
int attn_fwd_exp_poly(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                      int causal, float scale, attn_stream_t stream);

/*
 * attn_fwd_partial -- attention over the keys kv_begin <= j < kv_end only.
 *   q, k, v, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype: as attn_fwd; k and
 *            v hold the whole Nkv-key sequence and the causal mask keeps the
 *            whole problem's alignment (j <= i + Nkv - Nq, j the absolute key
 *            index), so the partial results of a partition of [0, Nkv) merge
 *            to attn_fwd's result.
 *   descale_q, descale_k, descale_v: as attn_fwd_fp8 for ATTN_FP8_E4M3 (NULL
 *            means 1.0); must be NULL for the other dtypes.
 *   o_part : DEVICE float32 (B, Hq, Nq, D): O normalised over the range
 *   lse_part: DEVICE float32 (B, Hq, Nq), required (not NULL)
 *   kv_begin, kv_end: 0 <= kv_begin <= kv_end <= Nkv.  A row that sees no
 *            key of the range gets O = 0 and LSE = -inf.
 * Errors as attn_fwd; ATTN_ERR_INVALID_ARG also for a bad range or a NULL
 * lse_part.
 */
int attn_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                     int causal, float scale, int dtype, int64_t kv_begin, int64_t kv_end,
                     const float* descale_q, const float* descale_k, const float* descale_v,
                     attn_stream_t stream);

/*
 * attn_merge -- merge n_parts partial results by their LSE (formula above).
 *   o_parts  : DEVICE float32 (n_parts, B, Hq, Nq, D), 16-byte aligned
 *   lse_parts: DEVICE float32 (n_parts, B, Hq, Nq); -inf marks a row that saw
 *              no key in that part
 *   o        : DEVICE output (B, Hq, Nq, D), float32 (out_dtype ATTN_F32) or
 *              bfloat16 (ATTN_BF16), 16-byte aligned
 *   lse      : DEVICE float32 (B, Hq, Nq), or NULL
 *   D        : multiple of 32 in [32, 1024]
 * Rows empty in every part get O = 0, LSE = -inf.  One kernel, enqueued on
 * `stream`; nothing is allocated.
 */
int attn_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse,
               int64_t B, int64_t Hq, int64_t Nq, int64_t D, int out_dtype, attn_stream_t stream);

/* Bytes of device workspace attn_fwd_splitkv needs (0 for invalid sizes). */
size_t attn_splitkv_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t D, int64_t n_splits);

/*
 * attn_fwd_splitkv -- attn_fwd computed as n_splits key ranges in ONE launch
 * (n_splits times the work-groups, for problems whose B * Hq * query tiles
 * leave compute units idle: few heads, long keys) followed by attn_merge.
 *   Arguments as attn_fwd, plus:
 *   descale_q, descale_k, descale_v: as attn_fwd_partial
 *   n_splits : 1..4096; the keys are cut into ranges of
 *              ceil(ceil(Nkv / n_splits) / 64) * 64 keys (the last ones may
 *              be short or empty)
 *   workspace, workspace_bytes: caller-owned DEVICE buffer, 256-byte aligned,
 *              of at least attn_splitkv_workspace_bytes(...) bytes; it holds
 *              the partial results, is overwritten, and must not be used by
 *              other work until the merge on `stream` completes.
 * The result equals attn_fwd's up to float32 rounding order.  Two kernels are
 * enqueued on `stream`; nothing is allocated.
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                     int causal, float scale, int dtype,
                     const float* descale_q, const float* descale_k, const float* descale_v,
                     int64_t n_splits, void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* Size of the scratch area of attn_fwd_splitkv_noalloc, per GPU: 64 MiB. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The same two launches on `stream`, with the
 * partial results in a scratch area the library holds at file scope
 * (ATTN_NOALLOC_SCRATCH_BYTES of device memory on each GPU it runs on, from
 * the loading of the library's code until the process ends) instead of a
 * caller workspace.  The call allocates nothing: no hipMalloc, no library
 * allocator.
 *   Arguments, outputs and results as attn_fwd_splitkv without workspace
 *   and workspace_bytes.
 *   ATTN_ERR_UNSUPPORTED when attn_splitkv_workspace_bytes(B, Hq, Nq, D,
 *   n_splits) exceeds ATTN_NOALLOC_SCRATCH_BYTES (use attn_fwd_splitkv, or
 *   fewer splits).
 * All calls on one GPU share its scratch area, which keeps the last call's
 * partial results (nothing in it needs clearing: each call writes every
 * partial element before reading it).  Calls that overlap on one GPU --
 * concurrent streams, or host threads enqueueing on different streams --
 * race on it and must be serialised by the caller.  The first call on each
 * GPU resolves the scratch area's device address (hipGetSymbolAddress):
 * make it once before any graph capture that records this call.
 */
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                             int causal, float scale, int dtype,
                             const float* descale_q, const float* descale_k, const float* descale_v,
                             int64_t n_splits, attn_stream_t stream);

/*
 * The fp8 input pipeline (FA blog, section "FA3 — el momento Hopper": FP8
 * with one scale per 64 x d tile and a random orthogonal Hadamard-based
 * pre-multiplication that spreads outliers; ZYFA article, section "The ZYFA
 * accuracy work is the sleeper contribution": a Hadamard rotation of Q and K
 * before quantisation roughly halves the input error).
 */

/*
 * attn_quantize_fp8 -- e4m3fn codes of a bf16 (B, H, N, D) tensor with one
 * descale per block of 64 rows of each (batch, head) slab, optionally after
 * rotating every row by R = diag(signs) H_D / sqrt(D) (H_D the Sylvester
 * Hadamard matrix).  R is orthogonal, so rotating Q and K with the same
 * signs leaves Q K^T unchanged; V is quantised without rotation.
 *   x        : DEVICE bfloat16 (B, H, N, D), 16-byte aligned
 *   codes    : DEVICE uint8 (B, H, N, D), 16-byte aligned
 *   descales : DEVICE float32 (B, H, ceil(N / 64)): descale = amax / 448 of
 *              the block (after rotation), 1 for an all-zero block
 *   D        : 64, 128 or 256
 *   signs    : DEVICE int8 (D) of +1 / -1, or NULL for no rotation
 * code = nearest e4m3fn value of x * (448 / amax), ties to even, computed in
 * float32.  One kernel on `stream`; nothing is allocated.
 */
int attn_quantize_fp8(const void* x, void* codes, float* descales, int64_t B, int64_t H, int64_t N, int64_t D,
                      const int8_t* signs, attn_stream_t stream);

/*
 * attn_fwd_fp8_blocks -- attn_fwd_fp8 with one descale per 64-row block
 * (the layout attn_quantize_fp8 writes): element i of q stands for
 * decode(code) * dq_blocks[b, hq, i / 64], and likewise for k (dk_blocks)
 * and v (dv_blocks), (B, Hkv, ceil(Nkv / 64)) each.  D = 64, 128 or 256;
 * scale > 0.  Other arguments, outputs and errors as attn_fwd_fp8.
 */
int attn_fwd_fp8_blocks(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                        int causal, float scale,
                        const float* dq_blocks, const float* dk_blocks, const float* dv_blocks,
                        attn_stream_t stream);

/*
 * The backward pass (FlashAttention summary page, method paragraph: the
 * backward pass recomputes S = Q K^T rather than storing it; blog post
 * "FlashAttention v1/v2/v3/v4", section "FA1 — el cambio de orden de las
 * operaciones": only the softmax statistics are kept; FFPA README feature
 * table: forward and backward).
 */

/* Bytes of workspace attn_bwd needs: two float32 (B, Hq, Nq) arrays, each
 * rounded up to 256 bytes.  0 for invalid sizes. */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq);

/*
 * attn_bwd -- gradients of O = softmax(scale Q K^T + mask) V with respect to
 * Q, K and V, given the upstream gradient dO:
 *   P = exp(scale Q K^T - LSE) (masked),  dV = P^T dO,  dP = dO V^T,
 *   delta_i = dO_i . O_i,  dS = P * (dP - delta),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * dK and dV of a KV head summed over the query heads of its group.
 *   q, o, dout, dq : DEVICE bf16 (B, Hq, Nq, D)
 *   k, v, dk, dv   : DEVICE bf16 (B, Hkv, Nkv, D)
 *   lse            : DEVICE float32 (B, Hq, Nq), natural log, as attn_fwd
 *                    writes it (-inf for a row that sees no key)
 *   o, lse         : the forward outputs for the same q, k, v, causal, scale
 *   workspace      : DEVICE, 16-byte aligned, >= attn_bwd_workspace_bytes;
 *                    overwritten (the library allocates nothing)
 *   dtype          : ATTN_BF16 only; D a multiple of 64 up to 512; causal and scale as
 *                    attn_fwd (any finite scale).
 * Outputs are overwritten (not accumulated into).  float32 accumulation;
 * every output element is accumulated by one wave, without atomics, so
 * results are deterministic.  Three kernels on `stream`.
 * Errors: ATTN_ERR_INVALID_ARG (NULL, sizes, alignment, workspace size),
 * ATTN_ERR_UNSUPPORTED (dtype, D, sizes past 2^31), ATTN_ERR_HIP.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv,
             int64_t D, int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
             attn_stream_t stream);

/* Static English name of a status code ("ATTN_OK", ...); never NULL. */
const char* attn_status_string(int status);

/* Description of the last failure on the calling thread ("" if none).  The
 * pointer stays valid until the next call of this library on this thread. */
const char* attn_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_ATTN_AMD_ATTN_H */
