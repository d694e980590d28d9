// attn_fwd_tiled.hip -- exact tiled attention forward for head dims D <= 256
// on gfx950: Q block resident in registers, K/V tiles streamed through LDS,
// online softmax with the output accumulator kept in MFMA registers.
//
// The algorithm (FlashAttention summary page, method paragraph; blog post
// "FlashAttention v1/v2/v3/v4", sections "El truco que hizo posible todo:
// online softmax" and "FA2 — paralelizar en serie"):
//   for each block of query rows (one work-group, rows split over waves):
//     m = -inf, l = 0, O = 0
//     for each tile of keys: S = Q K^T; m' = max(m, rowmax S);
//       P = exp(S - m'); l = e^{m-m'} l + rowsum P; O = e^{m-m'} O + P V
//     O /= l,  LSE = m + ln l
// S never leaves the chip.  The work is split over (batch, head, query
// tile) work-groups (FA2's sequence parallelism) and each wave owns 32 query
// rows (FA2's split-Q), so no cross-wave reduction exists.
//
// gfx950 mapping
//   * Transposed products: the kernel computes S^T = K Q^T and O^T = V^T P^T
//     on 32x32 MFMA tiles.  In that orientation a lane owns one query
//     (column l % 32) in both accumulators, so the softmax row max and row
//     sum are in-lane reductions over the lane's 16 registers per 32 keys plus
//     one exchange with the other half-wave, and the rescale factor
//     e^{m-m'} is a per-lane scalar for the O accumulator.  The S accumulator
//     registers, rounded to bf16, are directly the B operand of the P V
//     product (no data movement); only the key order inside each 16-key
//     block is permuted, which the V^T layout in LDS absorbs.
//   * Q is loaded once into registers in B-operand layout.  K tiles are
//     stored row-major in LDS (row pitch padded by 16 bytes so that the 8
//     lanes of each LDS phase hit distinct banks).  V tiles are transposed in
//     registers while staging and stored as V^T (bf16, even for fp8 inputs)
//     with the key order of each 16-key block permuted to match the S
//     registers and an XOR swizzle on 8-byte slots against bank conflicts.
//   * Global -> register prefetch of tile t+1 overlaps the MFMA work of tile
//     t; the LDS copy is single-buffered between two barriers.
//   * Ragged tails need no padding: loads go through buffer resources whose
//     range check returns zeros past the end of each (batch, head) slab, and
//     the scores of keys >= Nkv are masked to -inf (ZYFA article, "Getting
//     started with ZYFA", pads inputs instead; this kernel does not copy).
//   * Causal: key tiles entirely above the diagonal are never visited and the
//     mask is applied only on tiles that cross it; query tiles are issued
//     heaviest first.  Work-group ids are remapped so that each XCD processes
//     a contiguous range of (head, query tile) work (ZYFA article, "The
//     details that make it production-grade": eight chiplets, neighbouring
//     tiles of one head share K/V in that chiplet's L2).
//   * exp is computed as exp2 on pre-scaled scores (v_exp_f32 is base 2): the
//     scale * log2(e) factor is applied to S and the final LSE is converted
//     back to natural log.
#include "attn_common.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int E, int D, int NW, int BC>
struct TiledCfg {
  static constexpr int ES = EltInfo<E>::bytes;       // input element bytes
  static constexpr int NT = NW * 64;                 // threads per work-group
  static constexpr int BR = NW * 32;                 // query rows per work-group
  static constexpr int KS = D * ES + 16;             // K row pitch in LDS (bytes)
  static constexpr int K_BYTES = BC * KS;
  // V: fp32 kept row-major [key][d]; bf16/fp8 stored transposed V^T [d][key]
  // as bf16.
  static constexpr bool VT = (E != ELT_F32);
  static constexpr int VS = VT ? (BC * 2 + 16) : (D * 4 + 16);
  static constexpr int V_BYTES = VT ? D * VS : BC * VS;
  static constexpr int LDS_BYTES = K_BYTES + V_BYTES;
  // K staging: 16-byte chunks per tile
  static constexpr int K_CHUNKS_ROW = D * ES / 16;
  static constexpr int K_CHUNKS = BC * K_CHUNKS_ROW;
  static constexpr int K_PER_THREAD = (K_CHUNKS + NT - 1) / NT;
  // V staging: fp32 copies 16-byte chunks; bf16/fp8 transpose (4 keys x one
  // 16-byte chunk of a row) pairs.
  static constexpr int V_DCHUNK = 16 / ES;                       // d values per 16 bytes
  static constexpr int V_UNITS = VT ? (BC / 4) * (D / V_DCHUNK) : BC * (D * 4 / 16);
  static constexpr int V_PER_THREAD = (V_UNITS + NT - 1) / NT;
  static constexpr int V_LOADS = VT ? 4 : 1;                     // 16-byte loads per unit
  static constexpr int SLOTS = BC / 4;                           // 8-byte slots per V^T row
  static_assert(D % 32 == 0, "D must be a multiple of 32");
  static_assert(BC % 32 == 0, "BC must be a multiple of 32");
  static_assert(!VT || SLOTS >= 8, "V^T swizzle needs >= 8 slots");
  static_assert(E != ELT_FP8 || D % 64 == 0, "fp8 needs D % 64 == 0");
};

// Position (8-byte slot) of key group g (keys 4g..4g+3) inside a V^T row: the
// two middle bits of the key index within its 16-key block are swapped so
// that the 8 keys a lane contributes to one P V instruction are contiguous.
__device__ __forceinline__ int vt_slot(int g) {
  const int q4 = g & 3;
  return (g & ~3) | ((q4 & 1) << 1) | ((q4 >> 1) & 1);
}

// XOR applied to the slot index of V^T row d (even, so 16-byte pairs of
// slots stay adjacent); spreads the rows a wave writes at once over banks.
template <int SLOTS>
__device__ __forceinline__ int vt_xor(int d) {
  return (2 * (d >> 3)) & (SLOTS - 1) & ~1;
}

template <int E, int D, int NW, int BC>
__global__ __launch_bounds__(NW * 64) void attn_fwd_tiled_kernel(FwdParams p) {
  using C = TiledCfg<E, D, NW, BC>;
  __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
  char* const ldsK = lds;
  char* const ldsV = lds + C::K_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work decomposition: (b, hq, query tile) ----------------------------
  const int wg_all = xcd_remap(blockIdx.x, p.total_wg);
  const int per_split = p.total_wg / p.n_splits;
  const int split = wg_all / per_split;  // key range (split-KV); 0 for a plain call
  const int wg = wg_all - split * per_split;
  const KeyRange kr = key_range(p, split);
  const int qt_raw = wg % p.n_qtiles;
  const int bh = wg / p.n_qtiles;
  const int hq = bh % p.Hq;
  const int b = bh / p.Hq;
  const int qt = p.causal ? (p.n_qtiles - 1 - qt_raw) : qt_raw;  // heaviest first
  const int hk = hq / p.group;
  const int q0 = qt * C::BR;
  const int q0w = q0 + wave * 32;     // first query row of this wave
  const int qrow = q0w + l32;         // query row owned by this lane

  const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq * D;
  const int64_t kv_slab = (((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv + kr.k0) * D;
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc((const char*)p.q + q_slab * C::ES, (uint32_t)((int64_t)p.Nq * D * C::ES));
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc((const char*)p.k + kv_slab * C::ES, (uint32_t)((int64_t)kr.nkv * D * C::ES));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc((const char*)p.v + kv_slab * C::ES, (uint32_t)((int64_t)kr.nkv * D * C::ES));

  // ---- scale: exp(x) = exp2(x * log2 e); fp8 folds the Q and K descales ---
  float qk_scale = p.scale * kLog2e;
  float out_scale = 1.0f;
  if constexpr (E == ELT_FP8) {
    const float dq = p.dq ? p.dq[0] : 1.0f;
    const float dk = p.dk ? p.dk[0] : 1.0f;
    out_scale = p.dv ? p.dv[0] : 1.0f;
    qk_scale *= dq * dk;
  }

  // ---- Q block -> registers (B operand of S^T = K Q^T) ---------------------
  // bf16: 16 d per instruction, lane half h holds d = 16c + 8h .. +7
  // fp8 : 64 d per instruction, lane half h holds d = 64c + 32h .. +31
  // fp32:  2 d per instruction, lane half h holds d = 2c + h
  constexpr int QF = (E == ELT_BF16) ? D / 16 : (E == ELT_FP8) ? D / 64 : D / 2;
  u32x4 qb[E == ELT_BF16 ? QF : 1];
  i32x8 q8[E == ELT_FP8 ? QF : 1];
  float qf[E == ELT_F32 ? QF : 1];
  {
    const uint32_t row_off = (uint32_t)qrow * (uint32_t)(D * C::ES);
    if constexpr (E == ELT_BF16) {
#pragma unroll
      for (int c = 0; c < QF; ++c) qb[c] = buf_load16(rq, row_off + (uint32_t)(c * 32 + h * 16));
    } else if constexpr (E == ELT_FP8) {
#pragma unroll
      for (int c = 0; c < QF; ++c) {
        const u32x4 lo = buf_load16(rq, row_off + (uint32_t)(c * 64 + h * 32));
        const u32x4 hi = buf_load16(rq, row_off + (uint32_t)(c * 64 + h * 32 + 16));
        q8[c] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    } else {
#pragma unroll
      for (int c = 0; c < QF; ++c)
        qf[c] = __builtin_bit_cast(float, buf_load4(rq, row_off + (uint32_t)((2 * c + h) * 4)));
    }
  }

  // ---- key range ------------------------------------------------------------
  int kv_end = kr.nkv;
  if (p.causal) {
    const int last_row = min(q0 + C::BR, p.Nq) - 1;
    kv_end = min(kr.nkv, last_row + kr.kv_off + 1);
  }
  const int n_kt = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // ---- accumulators -----------------------------------------------------------
  constexpr int NDB = D / 32;   // 32-row blocks of O^T
  constexpr int NKB = BC / 32;  // 32-key blocks of S^T per tile
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of the scaled (base-2) scores
  float l_run = 0.0f;       // this lane's partial running sum

  // ---- staging registers ------------------------------------------------------
  u32x4 kst[C::K_PER_THREAD];
  u32x4 vst[C::V_PER_THREAD][C::V_LOADS];

  auto gload = [&](int kt) {
    const uint32_t tile_off = (uint32_t)(kt * BC) * (uint32_t)(D * C::ES);
#pragma unroll
    for (int i = 0; i < C::K_PER_THREAD; ++i) {
      const int u = tid + i * C::NT;
      if (C::K_CHUNKS % C::NT == 0 || u < C::K_CHUNKS) {
        const int key = u / C::K_CHUNKS_ROW, c = u % C::K_CHUNKS_ROW;
        kst[i] = buf_load16(rk, tile_off + (uint32_t)(key * D * C::ES + c * 16));
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_THREAD; ++i) {
      const int u = tid + i * C::NT;
      if (C::V_UNITS % C::NT == 0 || u < C::V_UNITS) {
        if constexpr (C::VT) {
          constexpr int NDC = D / C::V_DCHUNK;   // 16-byte chunks per row
          const int g = u / NDC, c = u % NDC;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            vst[i][r] = buf_load16(rv, tile_off + (uint32_t)((4 * g + r) * D * C::ES + c * 16));
        } else {
          constexpr int NDC = D * 4 / 16;
          const int key = u / NDC, c = u % NDC;
          vst[i][0] = buf_load16(rv, tile_off + (uint32_t)(key * D * 4 + c * 16));
        }
      }
    }
  };

  auto lds_put = [&]() {
#pragma unroll
    for (int i = 0; i < C::K_PER_THREAD; ++i) {
      const int u = tid + i * C::NT;
      if (C::K_CHUNKS % C::NT == 0 || u < C::K_CHUNKS) {
        const int key = u / C::K_CHUNKS_ROW, c = u % C::K_CHUNKS_ROW;
        lds_store16(ldsK, (uint32_t)(key * C::KS + c * 16), kst[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_THREAD; ++i) {
      const int u = tid + i * C::NT;
      if (C::V_UNITS % C::NT == 0 || u < C::V_UNITS) {
        if constexpr (C::VT) {
          constexpr int NDC = D / C::V_DCHUNK;
          const int g = u / NDC, c = u % NDC;
          const int slot = vt_slot(g);
          if constexpr (E == ELT_BF16) {
            // rows r = 0..3 hold d = 8c .. 8c+7 (dword w: d = 2w lo, 2w+1 hi)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t a0 = vst[i][0][w], a1 = vst[i][1][w], a2 = vst[i][2][w], a3 = vst[i][3][w];
              const int d_even = 8 * c + 2 * w;
              u32x2 ev, od;
              ev.x = (a0 & 0xffffu) | (a1 << 16);
              ev.y = (a2 & 0xffffu) | (a3 << 16);
              od.x = (a0 >> 16) | (a1 & 0xffff0000u);
              od.y = (a2 >> 16) | (a3 & 0xffff0000u);
              lds_store8(ldsV, (uint32_t)(d_even * C::VS + ((slot ^ vt_xor<C::SLOTS>(d_even)) * 8)), ev);
              lds_store8(ldsV, (uint32_t)((d_even + 1) * C::VS + ((slot ^ vt_xor<C::SLOTS>(d_even + 1)) * 8)), od);
            }
          } else {
            // fp8: rows r = 0..3 hold d = 16c .. 16c+15 as bytes; widen to bf16
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              u32x2 b4[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) b4[r] = e4m3x4_to_bf16x4(vst[i][r][w]);
              // b4[r].x = (d0 | d1<<16), b4[r].y = (d2 | d3<<16) for d = 16c + 4w + ...
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t s0 = (j < 2) ? b4[0].x : b4[0].y;
                const uint32_t s1 = (j < 2) ? b4[1].x : b4[1].y;
                const uint32_t s2 = (j < 2) ? b4[2].x : b4[2].y;
                const uint32_t s3 = (j < 2) ? b4[3].x : b4[3].y;
                u32x2 o;
                if ((j & 1) == 0) {
                  o.x = (s0 & 0xffffu) | (s1 << 16);
                  o.y = (s2 & 0xffffu) | (s3 << 16);
                } else {
                  o.x = (s0 >> 16) | (s1 & 0xffff0000u);
                  o.y = (s2 >> 16) | (s3 & 0xffff0000u);
                }
                const int d = 16 * c + 4 * w + j;
                lds_store8(ldsV, (uint32_t)(d * C::VS + ((slot ^ vt_xor<C::SLOTS>(d)) * 8)), o);
              }
            }
          }
        } else {
          constexpr int NDC = D * 4 / 16;
          const int key = u / NDC, c = u % NDC;
          lds_store16(ldsV, (uint32_t)(key * C::VS + c * 16), vst[i][0]);
        }
      }
    }
  };

  if (n_kt > 0) gload(0);

  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt > 0) __syncthreads();  // every wave is done reading the previous tile
    lds_put();
    __syncthreads();
    if (kt + 1 < n_kt) gload(kt + 1);

    const int key0 = kt * BC;
    // ---- S^T = K Q^T for this wave's 32 queries ------------------------------
    f32x16 s[NKB];
#pragma unroll
    for (int nb = 0; nb < NKB; ++nb) {
      s[nb] = f32x16{};
      const uint32_t krow = (uint32_t)((nb * 32 + l32) * C::KS);
      if constexpr (E == ELT_BF16) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          s[nb] = mfma_bf16(lds_load16(ldsK, krow + c * 32 + h * 16), qb[c], s[nb]);
      } else if constexpr (E == ELT_FP8) {
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
          const u32x4 lo = lds_load16(ldsK, krow + c * 64 + h * 32);
          const u32x4 hi = lds_load16(ldsK, krow + c * 64 + h * 32 + 16);
          const i32x8 kf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          s[nb] = mfma_fp8(kf, q8[c], s[nb]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < D / 2; ++c)
          s[nb] = mfma_f32(lds_loadf(ldsK, krow + (2 * c + h) * 4), qf[c], s[nb]);
      }
    }

    // ---- scale, mask, online softmax ------------------------------------------
    const bool need_mask = (key0 + BC > kr.nkv) || (p.causal && key0 + BC - 1 > q0w + kr.kv_off);
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NKB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[nb][r] * qk_scale;
        if (need_mask) {
          const int key = key0 + nb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool vis = key < kr.nkv && (!p.causal || key <= qrow + kr.kv_off);
          x = vis ? x : -INFINITY;
        }
        s[nb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float lsum = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NKB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(s[nb][r] - m_use);
        s[nb][r] = pr;
        lsum += pr;
      }
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] *= alpha;

    // ---- O^T += V^T P^T -----------------------------------------------------------
    if constexpr (E == ELT_F32) {
#pragma unroll
      for (int nb = 0; nb < NKB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = nb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma_f32(lds_loadf(ldsV, (uint32_t)(key * C::VS + (db * 32 + l32) * 4)), s[nb][r], acc[db]);
        }
      }
    } else {
#pragma unroll
      for (int s16 = 0; s16 < BC / 16; ++s16) {
        const int nb = s16 >> 1, r0 = (s16 & 1) * 8;
        u32x4 pf;
        pf.x = pack_bf16x2(s[nb][r0 + 0], s[nb][r0 + 1]);
        pf.y = pack_bf16x2(s[nb][r0 + 2], s[nb][r0 + 3]);
        pf.z = pack_bf16x2(s[nb][r0 + 4], s[nb][r0 + 5]);
        pf.w = pack_bf16x2(s[nb][r0 + 6], s[nb][r0 + 7]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = db * 32 + l32;
          const int slot = (4 * s16 + 2 * h) ^ vt_xor<C::SLOTS>(d);
          acc[db] = mfma_bf16(lds_load16(ldsV, (uint32_t)(d * C::VS + slot * 8)), pf, acc[db]);
        }
      }
    }
  }

  // ---- epilogue: O = O / l (x dv for fp8), LSE = ln2 * (m + log2 l) ------------
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.0f ? out_scale / l_tot : 0.0f;
  if (qrow < p.Nq) {
    const int64_t orow = split * p.o_split_stride + q_slab + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * h;
        const float o0 = acc[db][4 * g + 0] * inv, o1 = acc[db][4 * g + 1] * inv;
        const float o2 = acc[db][4 * g + 2] * inv, o3 = acc[db][4 * g + 3] * inv;
        store_o4(p.o, E == ELT_F32 || p.o_f32, orow + d, o0, o1, o2, o3);
      }
    }
    if (p.lse != nullptr && h == 0) {
      const float lse = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
      p.lse[split * p.lse_split_stride + ((int64_t)b * p.Hq + hq) * p.Nq + qrow] = lse;
    }
  }
}

template <int E, int D, int NW, int BC>
hipError_t launch_tiled(const FwdParams& p0, hipStream_t stream) {
  using C = TiledCfg<E, D, NW, BC>;
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + C::BR - 1) / C::BR;
  const int64_t total = (int64_t)p.n_splits * p.B * p.Hq * p.n_qtiles;
  if (total <= 0 || total >= (int64_t)1 << 31) return hipErrorInvalidValue;
  p.total_wg = (int)total;
  hipLaunchKernelGGL((attn_fwd_tiled_kernel<E, D, NW, BC>), dim3(p.total_wg), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Dispatch: one instantiation per (element type, D).  fp32 is kept to
// D <= 128 (its Q and O registers grow as D/2 per lane each).
LaunchFn tiled_launcher(int elt, int D) {
#define ATTN_CASE(E_, D_, NW_, BC_) \
  if (elt == E_ && D == D_) return &launch_tiled<E_, D_, NW_, BC_>;
  ATTN_CASE(ELT_BF16, 32, 4, 64)
  ATTN_CASE(ELT_BF16, 64, 4, 64)
  ATTN_CASE(ELT_BF16, 96, 4, 64)
  ATTN_CASE(ELT_BF16, 128, 4, 64)
  ATTN_CASE(ELT_BF16, 160, 4, 64)
  ATTN_CASE(ELT_BF16, 192, 4, 64)
  ATTN_CASE(ELT_BF16, 224, 4, 32)
  ATTN_CASE(ELT_BF16, 256, 4, 32)
  ATTN_CASE(ELT_F32, 32, 4, 32)
  ATTN_CASE(ELT_F32, 64, 4, 32)
  ATTN_CASE(ELT_F32, 96, 4, 32)
  ATTN_CASE(ELT_F32, 128, 4, 32)
  ATTN_CASE(ELT_FP8, 64, 4, 64)
  ATTN_CASE(ELT_FP8, 128, 4, 64)
  ATTN_CASE(ELT_FP8, 192, 4, 64)
  ATTN_CASE(ELT_FP8, 256, 4, 32)
#undef ATTN_CASE
  return nullptr;
}

}  // namespace attn
