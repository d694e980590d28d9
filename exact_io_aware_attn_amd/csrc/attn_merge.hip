// attn_merge.hip -- log-sum-exp merge of partial attention results on gfx950.
//
// ZYFA article, section "The details that make it production-grade": results
// computed over different key ranges have to merge consistently, which is
// what chunked prefill needs.  For partial results (O_p, LSE_p), p = 0..P-1,
// each normalised over its own key range,
//
//     LSE = ln sum_p exp(LSE_p),    O = sum_p exp(LSE_p - LSE) O_p,
//
// because the range sums l_p = exp(LSE_p) (in the scores' common scale) add
// up to the full row sum and O = sum_p l_p O_p / l.  The weights are formed
// against the largest LSE_p, so no exp overflows; a row empty in every part
// (all LSE_p = -inf) gets O = 0, LSE = -inf.
//
// The work is a streaming reduction (P D float32 reads and D writes per row),
// bound by HBM bandwidth: one thread owns four consecutive elements of a row
// (16-byte loads, coalesced across the D/4 threads of the row), a 256-thread
// work-group covers 1024/D rows, and each thread walks the parts in order.
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  const int tpr = p.D / 4;                          // threads per row
  const int rows_per_wg = 256 / tpr;
  if ((int)threadIdx.x >= rows_per_wg * tpr) return;  // D/4 need not divide 256
  const int64_t row = (int64_t)blockIdx.x * rows_per_wg + threadIdx.x / tpr;
  const int d = (threadIdx.x % tpr) * 4;
  if (row >= p.rows) return;
  const float* lse_p = p.lse_parts + row;
  float m = -INFINITY;
  for (int i = 0; i < p.n_parts; ++i) m = fmaxf(m, lse_p[i * p.lse_part_stride]);
  const float m_safe = m == -INFINITY ? 0.0f : m;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float tot = 0.0f;
  const float* o_p = p.o_parts + row * p.D + d;
  // four parts per step so that their loads are in flight together; an empty
  // part (weight 0) contributes nothing even if its O is not finite
#pragma unroll 4
  for (int i = 0; i < p.n_parts; ++i) {
    const float w = exp2_fast((lse_p[i * p.lse_part_stride] - m_safe) * kLog2e);  // 0 for an empty part
    const f32x4 x = *reinterpret_cast<const f32x4*>(o_p + i * p.o_part_stride);
    tot += w;
    acc += w != 0.0f ? w * x : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  store_o4(p.o, p.o_f32, row * p.D + d, acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (p.lse != nullptr && d == 0) p.lse[row] = tot > 0.0f ? m_safe + __builtin_log2f(tot) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int rows_per_wg = 256 / (p.D / 4);
  const int64_t wgs = (p.rows + rows_per_wg - 1) / rows_per_wg;
  if (wgs <= 0 || wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
