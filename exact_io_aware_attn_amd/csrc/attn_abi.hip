// attn_abi.hip -- the extern "C" boundary: argument validation, kernel
// selection by (dtype, D) and error reporting.  Host code only.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "attn.h"
#include "attn_common.h"
#include "attn_bwd.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Key ranges of one forward launch: n_splits ranges of split_len keys from
// kv_begin (the last one ends at kv_end); outputs of split s at o + s *
// o_split_stride, lse + s * lse_split_stride; o in float32 when o_f32.
struct Ranges {
  int64_t kv_begin, kv_end, split_len, n_splits;
  bool o_f32;
  int64_t o_split_stride, lse_split_stride;
};

int run_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale, int dtype,
                const float* dq, const float* dk, const float* dv, const Ranges* ranges, attn_stream_t stream,
                bool blk_scaled = false, int p_mode = 0, bool poly = false) {
  g_last_error[0] = '\0';
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL device pointers");
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 1 (B=%lld Hq=%lld Hkv=%lld Nq=%lld Nkv=%lld D=%lld)",
                (long long)B, (long long)Hq, (long long)Hkv, (long long)Nq, (long long)Nkv, (long long)D);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if ((dq && (reinterpret_cast<uintptr_t>(dq) & 3u)) || (dk && (reinterpret_cast<uintptr_t>(dk) & 3u)) ||
      (dv && (reinterpret_cast<uintptr_t>(dv) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "descale pointers must be 4-byte aligned");

  const int elt = dtype == ATTN_F32 ? attn::ELT_F32 : dtype == ATTN_BF16 ? attn::ELT_BF16 : attn::ELT_FP8;
  const int64_t in_bytes = dtype == ATTN_F32 ? 4 : dtype == ATTN_BF16 ? 2 : 1;
  const int64_t out_bytes = (dtype == ATTN_F32 || (ranges && ranges->o_f32)) ? 4 : 2;
  const int64_t lim = (int64_t)1 << 31;
  if (D > 1024 || D % 32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "D=%lld unsupported: D must be a multiple of 32 in [32, 1024]", (long long)D);
  if (Nq * D * in_bytes >= lim || Nkv * D * in_bytes >= lim || Nq * D * out_bytes >= lim)
    return fail(ATTN_ERR_UNSUPPORTED, "a (batch, head) slab of q, k, v or o reaches 2^31 bytes");
  if (B * Hq > (int64_t)INT32_MAX || Nq > INT32_MAX || Nkv > INT32_MAX)
    return fail(ATTN_ERR_UNSUPPORTED, "B*Hq and sequence lengths must fit in 31 bits");
  const int64_t n_splits = ranges ? ranges->n_splits : 1;
  if (B * Hq * ((Nq + 31) / 32) * n_splits >= lim)
    return fail(ATTN_ERR_UNSUPPORTED, "grid too large: splits*B*Hq*ceil(Nq/32) must be < 2^31");

  // bf16 D = 1024 runs on the eight-wave split-D kernel (any scale).
  // The wide-head kernel (bf16, D a multiple of 64 in [192, 512]) and the
  // direct-to-LDS kernel (bf16, D = 64 or 128; e4m3, D = 64, 128 or 256) fold
  // the scale into one FMA before exp2 and take row maxima of the unscaled
  // scores, which needs scale > 0.  Every other D <= 256 case runs on the
  // generic tiled kernel and every other D > 256 case on the four-wave
  // split-D kernel; both scale before masking.
  attn::LaunchFn fn = nullptr;
  if (p_mode != 0) {
    // e4m3 probabilities: the fp8 P V kernel only
    if (p_mode != ATTN_P_E4M3 && p_mode != ATTN_P_E4M3_LEAN)
      return fail(ATTN_ERR_INVALID_ARG, "unknown p_mode %d", p_mode);
    if (dtype == ATTN_FP8_E4M3 && scale > 0.0f && !blk_scaled) fn = attn::p8_launcher((int)D, p_mode == ATTN_P_E4M3_LEAN);
    if (!fn)
      return fail(ATTN_ERR_UNSUPPORTED, "e4m3 probabilities need e4m3 inputs, D in {64, 128} and scale > 0 (D=%lld)",
                  (long long)D);
  }
  if (poly) {
    if (dtype == ATTN_BF16 && scale > 0.0f) fn = attn::pipe_poly_launcher((int)D);
    if (!fn)
      return fail(ATTN_ERR_UNSUPPORTED, "the polynomial exponential needs bf16, D in {64, 128} and scale > 0 (D=%lld)",
                  (long long)D);
  }
  if (!fn && blk_scaled) {
    // block descales: the e4m3 direct-to-LDS kernel only
    if (scale > 0.0f) fn = attn::pipe_launcher(elt, (int)D);
    if (!fn)
      return fail(ATTN_ERR_UNSUPPORTED, "block-scaled e4m3 needs D in {64, 128, 256} and scale > 0 (D=%lld)",
                  (long long)D);
  }
  if (!fn) fn = attn::splitd8_launcher(elt, (int)D);
  if (!fn && scale > 0.0f) fn = attn::wide_launcher(elt, (int)D);
  if (!fn && scale > 0.0f) fn = attn::pipe_launcher(elt, (int)D);
  if (!fn) fn = D <= 256 ? attn::tiled_launcher(elt, (int)D) : attn::splitd_launcher(elt, (int)D);
  if (!fn)
    return fail(ATTN_ERR_UNSUPPORTED, "no kernel for dtype=%d D=%lld (fp32: D%%32==0, D<=128; fp8: D%%64==0, "
                "D<=256; bf16: D%%32==0, D<=1024)", dtype, (long long)D);

  attn::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nkv = (int)Nkv;
  p.D = (int)D;
  p.group = (int)(Hq / Hkv);
  p.causal = causal ? 1 : 0;
  p.kv_off = (int)(Nkv - Nq);
  p.scale = scale;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  if (ranges) {
    p.kv_begin = (int)ranges->kv_begin;
    p.kv_end = (int)ranges->kv_end;
    p.split_len = (int)ranges->split_len;
    p.n_splits = (int)ranges->n_splits;
    p.o_f32 = ranges->o_f32 ? 1 : 0;
    p.o_split_stride = ranges->o_split_stride;
    p.lse_split_stride = ranges->lse_split_stride;
  } else {
    p.kv_begin = 0;
    p.kv_end = (int)Nkv;
    p.split_len = (int)Nkv;
    p.n_splits = 1;
    p.o_f32 = dtype == ATTN_F32 ? 1 : 0;
    p.o_split_stride = 0;
    p.lse_split_stride = 0;
  }
  p.blk_scaled = blk_scaled ? 1 : 0;
  hipError_t err = fn(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

// Checks of attn_fwd_splitkv's arguments that do not involve the workspace
// (the rest are run_forward's).
int splitkv_check(const void* q, const void* k, const void* v, const void* o, int64_t B, int64_t Hq, int64_t Hkv,
                  int64_t Nq, int64_t Nkv, int64_t D, float scale, int dtype, const float* descale_q,
                  const float* descale_k, const float* descale_v, int64_t n_splits) {
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL device pointers");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (Hkv < 1 || (Hq >= 1 && Hq % Hkv != 0))
    return fail(ATTN_ERR_INVALID_ARG, "Hkv must be >= 1 and divide Hq");
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (dtype != ATTN_FP8_E4M3 && (descale_q || descale_k || descale_v))
    return fail(ATTN_ERR_INVALID_ARG, "descales apply to ATTN_FP8_E4M3 only");
  if (n_splits < 1 || n_splits > 4096) return fail(ATTN_ERR_INVALID_ARG, "n_splits must be in [1, 4096]");
  if (B < 1 || Hq < 1 || Nq < 1 || Nkv < 1 || D < 1)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 1");
  return ATTN_OK;
}

// The partial-attention launch over n_splits key ranges into `workspace`
// (attn_splitkv_workspace_bytes of it: float32 partial O of every split, then
// float32 partial LSE of every split, each part 256-byte aligned), then the
// merge into o and lse.  Every element of the partial results is written by
// the first launch before the second reads it (a range without keys for a
// row writes O = 0, LSE = -inf), so the workspace needs no clearing.
int splitkv_run(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale, int dtype,
                const float* descale_q, const float* descale_k, const float* descale_v, int64_t n_splits,
                void* workspace, attn_stream_t stream) {
  const int64_t rows = B * Hq * Nq;
  const int64_t o_bytes = (rows * D * 4 + 255) / 256 * 256;
  const int64_t l_bytes = (rows * 4 + 255) / 256 * 256;
  float* o_parts = static_cast<float*>(workspace);
  float* lse_parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + n_splits * o_bytes);
  // ranges of a multiple of 64 keys (whole tiles of every kernel); trailing
  // ranges may be short or empty
  const int64_t split_len = ((Nkv + n_splits - 1) / n_splits + 63) / 64 * 64;
  const Ranges r{0, Nkv, split_len, n_splits, true, o_bytes / 4, l_bytes / 4};
  int st = run_forward(q, k, v, o_parts, lse_parts, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, descale_q,
                       descale_k, descale_v, &r, stream);
  if (st != ATTN_OK) return st;
  attn::MergeParams mp{};
  mp.o_parts = o_parts;
  mp.lse_parts = lse_parts;
  mp.o = o;
  mp.lse = lse;
  mp.n_parts = (int)n_splits;
  mp.D = (int)D;
  mp.o_f32 = dtype == ATTN_F32 ? 1 : 0;
  mp.rows = rows;
  mp.o_part_stride = o_bytes / 4;
  mp.lse_part_stride = l_bytes / 4;
  hipError_t err = attn::launch_merge(mp, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "merge launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

// Scratch of attn_fwd_splitkv_noalloc: device memory of fixed size at file
// scope, so the entry point allocates nothing.  Each GPU the library runs on
// holds its own copy, from the loading of this code object until the
// process ends; calls on one GPU share it (the last call's partial results
// stay in it).  In host code `scratch` names a host-side stand-in, not the
// device array: its device address is taken once per device, with that
// device current, by hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || ptr == nullptr)
      return fail(ATTN_ERR_HIP, "hipGetSymbolAddress of the scratch area failed: %s", hipGetErrorString(err));
    if (reinterpret_cast<uintptr_t>(ptr) & 255u)
      return fail(ATTN_ERR_HIP, "the scratch area is not 256-byte aligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
             int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale, int dtype,
             attn_stream_t stream) {
  return run_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, nullptr, nullptr, nullptr,
                     nullptr, stream);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale,
                 const float* descale_q, const float* descale_k, const float* descale_v, attn_stream_t stream) {
  return run_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, ATTN_FP8_E4M3, descale_q, descale_k,
                     descale_v, nullptr, stream);
}

int attn_fwd_fp8_p(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale,
                   const float* descale_q, const float* descale_k, const float* descale_v, int p_mode,
                   attn_stream_t stream) {
  g_last_error[0] = '\0';
  if (p_mode != ATTN_P_E4M3 && p_mode != ATTN_P_E4M3_LEAN)
    return fail(ATTN_ERR_INVALID_ARG, "unknown p_mode %d", p_mode);
  return run_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, ATTN_FP8_E4M3, descale_q, descale_k,
                     descale_v, nullptr, stream, false, p_mode);
}

int attn_fwd_exp_poly(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale,
                      attn_stream_t stream) {
  g_last_error[0] = '\0';
  return run_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, ATTN_BF16, nullptr, nullptr, nullptr,
                     nullptr, stream, false, 0, true);
}

int attn_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int64_t B,
                     int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale, int dtype,
                     int64_t kv_begin, int64_t kv_end, const float* descale_q, const float* descale_k,
                     const float* descale_v, attn_stream_t stream) {
  g_last_error[0] = '\0';
  if (!lse_part) return fail(ATTN_ERR_INVALID_ARG, "lse_part must be a non-NULL device pointer");
  if (kv_begin < 0 || kv_begin > kv_end || kv_end > Nkv)
    return fail(ATTN_ERR_INVALID_ARG, "key range [%lld, %lld) must lie within [0, Nkv=%lld]", (long long)kv_begin,
                (long long)kv_end, (long long)Nkv);
  if (dtype != ATTN_FP8_E4M3 && (descale_q || descale_k || descale_v))
    return fail(ATTN_ERR_INVALID_ARG, "descales apply to ATTN_FP8_E4M3 only");
  const Ranges r{kv_begin, kv_end, kv_end - kv_begin, 1, true, 0, 0};
  return run_forward(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, descale_q, descale_k,
                     descale_v, &r, stream);
}

int attn_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse, int64_t B,
               int64_t Hq, int64_t Nq, int64_t D, int out_dtype, attn_stream_t stream) {
  g_last_error[0] = '\0';
  if (!o_parts || !lse_parts || !o)
    return fail(ATTN_ERR_INVALID_ARG, "o_parts, lse_parts and o must be non-NULL device pointers");
  if (n_parts < 1 || B < 1 || Hq < 1 || Nq < 1 || D < 1)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 1 (n_parts=%lld B=%lld Hq=%lld Nq=%lld D=%lld)",
                (long long)n_parts, (long long)B, (long long)Hq, (long long)Nq, (long long)D);
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "out_dtype must be ATTN_F32 or ATTN_BF16");
  if (!aligned16(o_parts) || !aligned16(o) || (reinterpret_cast<uintptr_t>(lse_parts) & 3u) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "o_parts and o must be 16-byte aligned, lse_parts and lse 4-byte aligned");
  if (D > 1024 || D % 32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "D=%lld unsupported: D must be a multiple of 32 in [32, 1024]", (long long)D);
  if (n_parts > INT32_MAX || B * Hq * Nq >= ((int64_t)1 << 40))
    return fail(ATTN_ERR_UNSUPPORTED, "too many parts or rows");
  attn::MergeParams mp{};
  mp.o_parts = o_parts;
  mp.lse_parts = lse_parts;
  mp.o = o;
  mp.lse = lse;
  mp.n_parts = (int)n_parts;
  mp.D = (int)D;
  mp.o_f32 = out_dtype == ATTN_F32 ? 1 : 0;
  mp.rows = B * Hq * Nq;
  mp.o_part_stride = mp.rows * D;
  mp.lse_part_stride = mp.rows;
  hipError_t err = attn::launch_merge(mp, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "merge launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

int attn_quantize_fp8(const void* x, void* codes, float* descales, int64_t B, int64_t H, int64_t N, int64_t D,
                      const int8_t* signs, attn_stream_t stream) {
  g_last_error[0] = '\0';
  if (!x || !codes || !descales) return fail(ATTN_ERR_INVALID_ARG, "x, codes and descales must be non-NULL device pointers");
  if (B < 1 || H < 1 || N < 1 || D < 1) return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!aligned16(x) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(descales) & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "x and codes must be 16-byte aligned, descales 4-byte aligned");
  if (D != 64 && D != 128 && D != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "D=%lld unsupported: the quantiser takes D = 64, 128 or 256", (long long)D);
  if (B * H > INT32_MAX || N * D * 2 >= ((int64_t)1 << 31) || B * H * ((N + 63) / 64) >= ((int64_t)1 << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
  attn::QuantParams qp{};
  qp.x = static_cast<const __bf16*>(x);
  qp.codes = static_cast<uint8_t*>(codes);
  qp.descales = descales;
  qp.signs = signs;
  qp.S = (int)(B * H);
  qp.N = (int)N;
  qp.D = (int)D;
  hipError_t err = attn::launch_quant_fp8(qp, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "quantiser launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

int attn_fwd_fp8_blocks(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale,
                        const float* dq_blocks, const float* dk_blocks, const float* dv_blocks,
                        attn_stream_t stream) {
  g_last_error[0] = '\0';
  if (!dq_blocks || !dk_blocks || !dv_blocks)
    return fail(ATTN_ERR_INVALID_ARG, "dq_blocks, dk_blocks and dv_blocks must be non-NULL device pointers");
  return run_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, ATTN_FP8_E4M3, dq_blocks, dk_blocks,
                     dv_blocks, nullptr, stream, true);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq) {
  if (B < 1 || Hq < 1 || Nq < 1) return 0;
  const int64_t one = (B * Hq * Nq * 4 + 255) / 256 * 256;
  return (size_t)(2 * one);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
             int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  g_last_error[0] = '\0';
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o, lse, dout, dq, dk and dv must be non-NULL device pointers");
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 1");
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  for (const void* t : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(t)) return fail(ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Nq);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(ATTN_ERR_INVALID_ARG, "workspace must be a 16-byte aligned device buffer of at least %zu bytes",
                need);
  if (dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "the backward pass takes bf16 only (dtype=%d)", dtype);
  if (D % 64 != 0 || D < 64 || D > 512)
    return fail(ATTN_ERR_UNSUPPORTED, "D=%lld unsupported: the backward pass takes D a multiple of 64 up to 512",
                (long long)D);
  const int64_t lim = (int64_t)1 << 31;
  if (Nq * D * 2 >= lim || Nkv * D * 2 >= lim)
    return fail(ATTN_ERR_UNSUPPORTED, "a (batch, head) slab reaches 2^31 bytes");
  if (B * Hq * Nq >= lim || B * Hq > (int64_t)INT32_MAX)
    return fail(ATTN_ERR_UNSUPPORTED, "B*Hq*Nq must be < 2^31");
  attn::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  const size_t one = need / 2;
  p.delta = static_cast<float*>(workspace);
  p.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + one);
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nkv = (int)Nkv;
  p.D = (int)D;
  p.group = (int)(Hq / Hkv);
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  hipError_t err = attn::launch_bwd(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

size_t attn_splitkv_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t D, int64_t n_splits) {
  if (B < 1 || Hq < 1 || Nq < 1 || D < 1 || n_splits < 1) return 0;
  const int64_t rows = B * Hq * Nq;
  // float32 partial O, then float32 partial LSE, each part 256-byte aligned
  const int64_t o_bytes = (rows * D * 4 + 255) / 256 * 256;
  const int64_t l_bytes = (rows * 4 + 255) / 256 * 256;
  return (size_t)(n_splits * (o_bytes + l_bytes));
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale, int dtype,
                     const float* descale_q, const float* descale_k, const float* descale_v, int64_t n_splits,
                     void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  g_last_error[0] = '\0';
  const int st = splitkv_check(q, k, v, o, B, Hq, Hkv, Nq, Nkv, D, scale, dtype, descale_q, descale_k, descale_v,
                               n_splits);
  if (st != ATTN_OK) return st;
  const size_t need = attn_splitkv_workspace_bytes(B, Hq, Nq, D, n_splits);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_INVALID_ARG, "workspace must be a device buffer of at least %zu bytes", need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return splitkv_run(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, descale_q, descale_k, descale_v,
                     n_splits, workspace, stream);
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                             int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale,
                             int dtype, const float* descale_q, const float* descale_k, const float* descale_v,
                             int64_t n_splits, attn_stream_t stream) {
  g_last_error[0] = '\0';
  const int st = splitkv_check(q, k, v, o, B, Hq, Hkv, Nq, Nkv, D, scale, dtype, descale_q, descale_k, descale_v,
                               n_splits);
  if (st != ATTN_OK) return st;
  const size_t need = attn_splitkv_workspace_bytes(B, Hq, Nq, D, n_splits);
  if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return fail(ATTN_ERR_UNSUPPORTED,
                "the partial results need %zu bytes, more than the %zu-byte scratch of attn_fwd_splitkv_noalloc "
                "(use attn_fwd_splitkv with a caller workspace, or fewer splits)",
                need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != ATTN_OK) return sst;
  return splitkv_run(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, descale_q, descale_k, descale_v,
                     n_splits, ws, stream);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_UNKNOWN_STATUS";
  }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_version(void) { return 100; }

}  // extern "C"
