// attn_quant.hip -- the fp8 input pipeline on gfx950: e4m3 quantisation of a
// (B, H, N, D) bf16 tensor with one descale per 64-row block of each (batch,
// head) slab, optionally after rotating every row by a signed Hadamard matrix.
//
// FA blog, section "FA3 — el momento Hopper": FP8 with block quantisation (a
// scale per 64 x d tile rather than per tensor) and incoherent processing (a
// random orthogonal Hadamard-based matrix spreads outliers before
// quantising).  ZYFA article, section "The ZYFA accuracy work is the sleeper
// contribution": rotating Q and K by a Hadamard matrix before quantisation
// roughly halves the input error.  q' = q R with R = diag(signs) H_D / sqrt(D)
// is orthogonal, so Q'K'^T = QK^T: Q and K are rotated with the same signs,
// V is not.
//
// One work-group per 64-row block, 4 waves of 16 rows.  A lane holds 8
// consecutive elements of a row (one 16-byte load), D/8 lanes a row, so one
// load instruction of a wave covers 512/D rows; every load of a wave is
// issued before the first use (rows past N load row N-1 and are zeroed, so
// no branch splits them).  The rotation is the fast Walsh-Hadamard
// transform: the three butterfly stages of stride 1, 2, 4 inside a lane,
// then one stage per lane bit (stride 8, 16, ...) with the partner lane's
// value from a DPP quad permutation (lane ^ 1, lane ^ 2) or a swizzle
// (lane ^ 4 and up), then one multiply by 1/sqrt(D).  The block's amax is
// reduced over the wave and then the work-group; descale = amax / 448 and
// inv = 448 / amax (float32, correctly rounded), and each value becomes the
// nearest e4m3fn code of x * inv (ties to even; x * inv is clamped to +-448
// first, which only removes the float32 rounding of amax * inv), eight codes
// per 8-byte store.  An all-zero block gets descale 1 and codes 0.
// Memory-bound: 2 D bytes read and D + 4/64 bytes written per row.
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {

namespace {

// value of lane ^ M (M a power of two below 32)
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
  } else {
    r = __builtin_amdgcn_ds_swizzle(v, 0x1F | (M << 10));   // bitmask mode: lane ^ M within 32
  }
  return __builtin_bit_cast(float, r);
}

template <int D>
__global__ __launch_bounds__(256) void attn_quant_fp8_kernel(QuantParams p) {
  constexpr int LPR = D / 8;        // lanes per row
  constexpr int RPI = 64 / LPR;     // rows per load instruction of a wave
  constexpr int NI = 16 / RPI;      // load instructions per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nblk = (p.N + 63) / 64;
  const int slab = blockIdx.x / nblk;
  const int blk = blockIdx.x - slab * nblk;
  const int sub = lane / LPR;       // row of this lane within one instruction
  const int col = (lane % LPR) * 8;
  const int row0 = blk * 64 + wave * 16 + sub;
  const int64_t base = (int64_t)slab * p.N * D;

  float x[NI][8];
  {
    u32x4 raw[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = min(row0 + i * RPI, p.N - 1);
      raw[i] = *reinterpret_cast<const u32x4*>(p.x + base + (int64_t)row * D + col);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool live = row0 + i * RPI < p.N;
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // bf16 -> float32 is exact: the 16 bits become the high half
        x[i][2 * j] = live ? __builtin_bit_cast(float, w[j] << 16) : 0.0f;
        x[i][2 * j + 1] = live ? __builtin_bit_cast(float, w[j] & 0xFFFF0000u) : 0.0f;
      }
    }
  }

  if (p.signs != nullptr) {
    float sg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = (float)p.signs[col + e];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] *= sg[e];
      // strides 1, 2, 4: both partners in this lane
#pragma unroll
      for (int s = 1; s < 8; s *= 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if ((e & s) == 0) {
            const float a = x[i][e], c = x[i][e + s];
            x[i][e] = a + c;
            x[i][e + s] = a - c;
          }
        }
      }
    }
    // strides 8 .. D/2: the partner is lane ^ (stride / 8); the lower lane
    // keeps a + c, the upper c - (its own) = a - c
    static_for<0, 5>([&](auto st) {
      constexpr int M = 1 << decltype(st)::value;
      if constexpr (M < LPR) {
        const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[i][e] = __builtin_fmaf(sgn, x[i][e], xor_lane<M>(x[i][e]));
      }
    });
    constexpr float kNorm = D == 64 ? 0.125f : D == 256 ? 0.0625f : 0.088388347648318440550f;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] *= kNorm;
  }

  // block amax: lane, wave, work-group
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
#pragma unroll
  for (int m = 1; m < 64; m *= 2) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  __shared__ float wmax[4];
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool zero = amax == 0.0f;
  const float inv = zero ? 0.0f : 448.0f / amax;
  if (threadIdx.x == 0) p.descales[(int64_t)slab * nblk + blk] = zero ? 1.0f : amax / 448.0f;

#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = row0 + i * RPI;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(x[i][e] * inv, -448.0f), 448.0f);
    // four codes per register: low word then high word
    const int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false), true);
    const int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false), true);
    if (row < p.N) {
      uint2 st;
      st.x = (uint32_t)w0;
      st.y = (uint32_t)w1;
      *reinterpret_cast<uint2*>(p.codes + base + (int64_t)row * D + col) = st;
    }
  }
}

template <int D>
hipError_t launch_quant(const QuantParams& p, hipStream_t stream) {
  const int64_t wgs = (int64_t)p.S * ((p.N + 63) / 64);
  if (wgs <= 0 || wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_quant_fp8_kernel<D>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(const QuantParams& p, hipStream_t stream) {
  switch (p.D) {
    case 64: return launch_quant<64>(p, stream);
    case 128: return launch_quant<128>(p, stream);
    case 256: return launch_quant<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
