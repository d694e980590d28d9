// attn_fwd_wide.hip -- bf16 attention forward for gfx950, head dims 192..512
// (multiples of 64), positive scale, with the softmax of each key tile run
// between the MFMAs of the previous tile's P V product.
//
// Same arithmetic as the direct-to-LDS kernel (FlashAttention summary page,
// method paragraph; blog post "FlashAttention v1/v2/v3/v4", section "El truco
// que hizo posible todo: online softmax"): S^T = K Q^T and O^T += V^T P^T on
// the bf16 matrix instruction, base-2 online softmax with a lazy rescale,
// K/V tiles streamed into LDS by direct-to-LDS buffer loads.
//
// At these head dims a wave holds Q in D/4 VGPRs and O in D/2 accumulation
// registers, so a SIMD runs one wave (two at D = 192) and no other wave can
// fill the matrix pipe while it computes exponentials.  The wave overlaps the
// two itself:
//
//  * Iteration t computes S_t = K_t Q^T, then the product P_{t-1} V_{t-1} of
//    the PREVIOUS tile, and between those MFMAs the exponentials, packing and
//    row sums that make P_t from S_t.  P_t is used one iteration later.
//  * The recurrence is unchanged: with alpha_t = 2^(m_{t-1} - m_t), iteration t
//    turns the accumulator O' into alpha_t (O' + P_{t-1} V_{t-1}), computed as
//    alpha_t O' + (alpha_t P_{t-1}) V_{t-1}: when the lazy rescale fires, O
//    and the not yet used bf16 P_{t-1} are scaled before the MFMAs.  The
//    stale max then moves up by a whole number of base-2 units, so alpha_t is
//    a power of two and scaling P_{t-1} is exact.  l follows the usual
//    recurrence, updated with P_t.
//  * K_{t+1} streams into LDS during the S_t MFMAs and V_t during the
//    P_{t-1} V_{t-1} MFMAs (V_0 with K_0 before the loop), one load block
//    after each of the phase's first MFMAs so the tile has the rest of the
//    phase to land.  Two slots per operand suffice: iteration t reads K_t
//    and V_{t-1} and writes K_{t+1} and V_t.
//  * A tile is 32 keys, or 64 (NKB = 2 blocks of 32) where four such tiles
//    fit in LDS (D = 256, 320): twice the work per barrier and per max
//    reduction, measured faster there.
//  * The ZYFA article ("The three techniques, in plain terms") describes the
//    same goal -- exponentials off the matrix pipe's critical path -- reached
//    there with two waves per SIMD; with one wave per SIMD the overlap has to
//    come from the wave's own instruction order.
#include "attn_common.h"
#include "attn_dma.h"
#include "attn_launch.h"

#include <type_traits>

namespace attn {

namespace {

// An empty asm that takes x and gives it back in the same vector register:
// computed values cannot be moved past it.  Without it the exponentials of
// P_t, which are only used after the loop over the P V MFMAs, are sunk
// below all of them and no longer overlap the matrix work.
__device__ __forceinline__ void pin_f(float& x) { asm volatile("" : "+v"(x)); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, base-2 units

// Eight bf16 values (packed pairs) times alpha, rounded back to bf16.
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float alpha) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_bit_cast(float, v[i] << 16) * alpha;
    const float hi = __builtin_bit_cast(float, v[i] & 0xffff0000u) * alpha;
    r[i] = pack_bf16x2(lo, hi);
  }
  return r;
}

template <int D_, int NKB_>
struct WideCfg {
  static constexpr int D = D_;
  static constexpr int NKB = NKB_;              // 32-key blocks per tile
  static constexpr int NW = 4;                  // waves per work-group, one per SIMD
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * 32;            // query rows per work-group
  static constexpr int BC = 32 * NKB_;          // keys per tile
  static constexpr int RP = D_ * 2;             // LDS row pitch (bytes)
  static constexpr int TILE = BC * RP;          // one K or V tile
  static constexpr int DMA_WAVE = TILE / 1024 / NW;
  static constexpr int NDB = D_ / 32;           // 32-row blocks of O^T
  static constexpr int NQC = D_ / 16;           // 16-wide d chunks of QK^T (MFMAs per 32-key block of S)
  static constexpr int NFQ = NKB_ * NQC;        // MFMAs per S tile
  static constexpr int NFV = 2 * NKB_ * NDB;    // MFMAs per P V tile
  static constexpr int NE = 16 * NKB_;          // scores per lane per tile
  static constexpr int SW = (D_ % 128 == 0) ? 16 : 8;
  static constexpr int LK = 8;                  // K fragments in flight
  static constexpr int LV = 4;                  // V fragments in flight (8 reads)
  static constexpr int LDS = 4 * TILE;          // K slots 0, 1; V slots 0, 1
  static_assert(D_ % 64 == 0 && D_ >= 192 && D_ <= 512, "head dims 192..512");
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(DMA_WAVE <= NFQ && DMA_WAVE <= NFV, "one load block per MFMA at most");
};

template <int D, int NKB>
__global__ __launch_bounds__(256, 1) void attn_fwd_wide_kernel(FwdParams p) {
  using C = WideCfg<D, NKB>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);
  char* const ldsV = lds + 2 * C::TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work decomposition (heaviest causal tiles first, XCD-local heads) ----
  const int wg_all = xcd_remap(blockIdx.x, p.total_wg);
  const int per_split = p.total_wg / p.n_splits;
  const int split = wg_all / per_split;  // key range (split-KV); 0 for a plain call
  const int wg = wg_all - split * per_split;
  const KeyRange kr = key_range(p, split);
  const int qt_raw = wg % p.n_qtiles;
  const int bh = wg / p.n_qtiles;
  const int hq = bh % p.Hq;
  const int b = bh / p.Hq;
  const int qt = p.causal ? (p.n_qtiles - 1 - qt_raw) : qt_raw;
  const int hk = hq / p.group;
  const int q0 = qt * C::BR;
  const int q0w = q0 + wave * 32;

  const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq * D;
  const int64_t kv_slab = (((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv + kr.k0) * D;
  const uint32_t kv_bytes = (uint32_t)((int64_t)kr.nkv * D * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)p.q + q_slab, (uint32_t)((int64_t)p.Nq * D * 2));
  const i32x4 rk = sgpr_rsrc((const __bf16*)p.k + kv_slab, kv_bytes);
  const i32x4 rv = sgpr_rsrc((const __bf16*)p.v + kv_slab, kv_bytes);

  const float c = p.scale * kLog2e;  // > 0 (the launcher routes other scales elsewhere)

  int kv_end = kr.nkv;
  if (p.causal) kv_end = min(kr.nkv, min(q0 + C::BR, p.Nq) + kr.kv_off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;

  // ---- K/V loads: tile t in slot t & 1 of each operand ------------------------
  uint32_t dk[C::DMA_WAVE], dv[C::DMA_WAVE];
  dma_offsets<C, false>(dk, wave, lane);
  dma_offsets<C, true>(dv, wave, lane);
  auto dma_off = [&](bool is_v, int j) -> uint32_t {
    if constexpr (C::RP % 1024 == 0)
      return is_v ? dma_offset_1k<C, true>(wave, lane, j) : dma_offset_1k<C, false>(wave, lane, j);
    else
      return is_v ? dv[j] : dk[j];
  };
  auto k_slot = [&](int t) { return lds_base + (uint32_t)((t & 1) * C::TILE); };
  auto v_slot = [&](int t) { return lds_base + (uint32_t)((2 + (t & 1)) * C::TILE); };
  if (n_kt > 0) {
    dma_tile<C>(rk, k_slot(0), dk, wave);
    dma_tile<C>(rv, v_slot(0), dv, wave);
  }

  // ---- Q fragments (B operand of S^T = K Q^T): d = 16cc + 8h .. +7 ----------
  u32x4 qf[C::NQC];
  {
    const uint32_t row_off = (uint32_t)(q0w + l32) * (uint32_t)(D * 2);
#pragma unroll
    for (int cc = 0; cc < C::NQC; ++cc) qf[cc] = buf_load16(rq, row_off + (uint32_t)(cc * 32 + h * 16));
  }

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  // per-lane LDS offsets (the layouts of the direct-to-LDS kernel)
  constexpr int KG = C::SW / 2, VG = C::SW / 4;
  uint32_t kbase[KG];
#pragma unroll
  for (int i = 0; i < KG; ++i) kbase[i] = (uint32_t)(l32 * C::RP + (((2 * i + h) ^ k_swz<D>(l32)) << 4));
  auto koff = [&](int cc) { return kbase[cc % KG] + (uint32_t)((cc / KG) * C::SW * 16); };
  const int g16 = lane >> 4, r16 = lane & 15;
  uint32_t vbase[VG];
#pragma unroll
  for (int i = 0; i < VG; ++i) {
    const int chunk = i * 4 + 2 * (g16 & 1) + ((r16 & 3) >> 1);
    const int row = 4 * h + (r16 >> 2);
    vbase[i] = (uint32_t)(row * C::RP + ((chunk ^ v_swz<D>(row)) << 4) + ((r16 & 1) << 3));
  }
  auto voff = [&](int db) { return vbase[db % VG] + (uint32_t)((db / VG) * C::SW * 16); };
  const int qrow = q0w + l32;
  const int klim = p.causal ? min(kr.nkv - 1, qrow + kr.kv_off) : kr.nkv - 1;

  u32x4 pprev[2 * NKB];  // P_{t-1} (bf16), the B operand of this iteration's P V
#pragma unroll
  for (int g = 0; g < 2 * NKB; ++g) pprev[g] = u32x4{};

  // ---- one iteration; HAS_QK: tile t exists, HAS_PV: tile t-1 exists ----------
  auto step = [&](int t, auto has_qk, auto has_pv) {
    constexpr bool QK = decltype(has_qk)::value, PV = decltype(has_pv)::value;
    // K_t and V_{t-1} resident; slots of K_{t-1} and V_{t-2} free
    wait_vmem_all();
    __syncthreads();
    const char* const kb_cur = lds + (t & 1) * C::TILE;
    const char* const vb_prev = ldsV + ((t - 1) & 1) * C::TILE;

    // V_{t-1} fragment f (two transposing reads)
    auto vfrag = [&](int f) {
      const int s16 = f / C::NDB, db = f % C::NDB;
      const uint32_t a0 = voff(db) + (uint32_t)(s16 * 16 * C::RP);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb_prev + a0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb_prev + a0 + 8 * C::RP));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2.x, l2.y, h2.x, h2.y};
    };
    u32x4 vf[C::LV];

    // ---- S_t^T = K_t Q^T, K_{t+1} streaming in between the MFMAs --------------
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    float mneg = 0.0f;
    if constexpr (QK) {
      const bool k_next = t + 1 < n_kt;
      const i32x4 rk_n = rsrc_at(rk, (uint32_t)((t + 1) * C::TILE));
      // fragment f: key block f / NQC, d chunk f % NQC
      auto kfrag = [&](int f) { return lds_load16(kb_cur, koff(f % C::NQC) + (uint32_t)((f / C::NQC) * 32 * C::RP)); };
      u32x4 kf[C::LK];
#pragma unroll
      for (int i = 0; i < C::LK; ++i) kf[i] = kfrag(i);
#pragma unroll
      for (int f = 0; f < C::NFQ; ++f) {
        const u32x4 cur = kf[f % C::LK];
        if (f + C::LK < C::NFQ) kf[f % C::LK] = kfrag(f + C::LK);
        __builtin_amdgcn_sched_barrier(0);
        s[f / C::NQC] = mfma_bf16(cur, qf[f % C::NQC], s[f / C::NQC]);
        // one load block after each of the first MFMAs: the tile lands well
        // before the barrier that needs it
        if (k_next && f < C::DMA_WAVE) dma_block_at<C::DMA_WAVE>(rk_n, k_slot(t + 1), dma_off(false, f), wave, f);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the first V fragments of the P V product below, read while the
      // MFMAs drain and the row maximum is formed
      if constexpr (PV) {
#pragma unroll
        for (int i = 0; i < C::LV; ++i) vf[i] = vfrag(i);
        __builtin_amdgcn_sched_barrier(0);
      }
      // mask (tiles crossing the diagonal or the key tail only)
      const int key0 = t * C::BC;
      if ((key0 + C::BC > kr.nkv) || (p.causal && key0 + C::BC - 1 > q0w + kr.kv_off)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            s[kb][r] = key <= klim ? s[kb][r] : -INFINITY;
          }
      }
      // running max.  O' + P_{t-1} V_{t-1} is due to be scaled by alpha;
      // alpha O' + (alpha P_{t-1}) V_{t-1} is the same, so O is scaled now
      // (before its MFMAs) and P_{t-1} with it.  The max moves up by a whole
      // number of base-2 units, which makes alpha a power of two and the
      // scaling of the bf16 P_{t-1} exact.
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int i = 2; i < C::NE; i += 2) mx = fmaxf(fmaxf(mx, s[i / 16][i % 16]), s[i / 16][i % 16 + 1]);
      const float mrow = max_halves(mx) * c;
      if (__builtin_amdgcn_ballot_w64(mrow > m_run + kTau) != 0) {
        float m_new = m_run;
        if (mrow > m_run) m_new = m_run == -INFINITY ? mrow : m_run + __builtin_ceilf(mrow - m_run);
        const float alpha = exp2_fast(m_run - (m_new == -INFINITY ? 0.0f : m_new));
        if constexpr (PV) {
          // (the first tile has no O and no P_{t-1} yet, both still zero)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) scale_acc(acc[db], alpha);
#pragma unroll
          for (int g = 0; g < 2 * NKB; ++g) pprev[g] = scale_bf16x8(pprev[g], alpha);
        }
        l_run *= alpha;
        m_run = m_new;
      }
      mneg = m_run == -INFINITY ? 0.0f : -m_run;
    }

    // ---- O^T += V_{t-1}^T P_{t-1}^T, with P_t computed between the MFMAs ------
    float e[C::NE];
    auto exps = [&](int lo, int hi) {
#pragma unroll
      for (int i = lo; i < hi; ++i) {
        e[i] = exp2_fast(__builtin_fmaf(s[i / 16][i % 16], c, mneg));
        pin_f(e[i]);
      }
    };
    if constexpr (PV) {
      const bool v_now = t < n_kt;  // V_t streams in meanwhile
      const i32x4 rv_t = rsrc_at(rv, (uint32_t)(t * C::TILE));
      if constexpr (!QK) {
#pragma unroll
        for (int i = 0; i < C::LV; ++i) vf[i] = vfrag(i);
      }
#pragma unroll
      for (int f = 0; f < C::NFV; ++f) {
        const u32x4 cur = vf[f % C::LV];
        if (f + C::LV < C::NFV) vf[f % C::LV] = vfrag(f + C::LV);
        __builtin_amdgcn_sched_barrier(0);
        acc[f % C::NDB] = mfma_bf16(cur, pprev[f / C::NDB], acc[f % C::NDB]);
        if constexpr (QK) exps((f * C::NE + C::NFV - 1) / C::NFV, ((f + 1) * C::NE + C::NFV - 1) / C::NFV);
        if (v_now && f < C::DMA_WAVE) dma_block_at<C::DMA_WAVE>(rv_t, v_slot(t), dma_off(true, f), wave, f);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if constexpr (QK) exps(0, C::NE);
    }
    if constexpr (QK) {
      float ls = l_run;
#pragma unroll
      for (int g = 0; g < 2 * NKB; ++g) {
        pprev[g].x = pack_bf16x2(e[8 * g + 0], e[8 * g + 1]);
        pprev[g].y = pack_bf16x2(e[8 * g + 2], e[8 * g + 3]);
        pprev[g].z = pack_bf16x2(e[8 * g + 4], e[8 * g + 5]);
        pprev[g].w = pack_bf16x2(e[8 * g + 6], e[8 * g + 7]);
        ls += ((e[8 * g + 0] + e[8 * g + 1]) + (e[8 * g + 2] + e[8 * g + 3])) +
              ((e[8 * g + 4] + e[8 * g + 5]) + (e[8 * g + 6] + e[8 * g + 7]));
      }
      l_run = ls;
    }
  };

  // ---- iterations t = 0 .. n_kt ------------------------------------------------
  if (n_kt > 0) {
    step(0, std::true_type{}, std::false_type{});
    for (int t = 1; t < n_kt; ++t) step(t, std::true_type{}, std::true_type{});
    step(n_kt, std::false_type{}, std::true_type{});
  }

  // ---- epilogue ---------------------------------------------------------------------
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < p.Nq) {
    const int64_t orow = split * p.o_split_stride + q_slab + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * h;
        store_o4(p.o, p.o_f32, orow + d, acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                 acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
      }
    }
    if (p.lse != nullptr && h == 0)
      p.lse[split * p.lse_split_stride + ((int64_t)b * p.Hq + hq) * p.Nq + qrow] =
          l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int NKB>
hipError_t launch_wide(const FwdParams& p0, hipStream_t stream) {
  using C = WideCfg<D, NKB>;
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + C::BR - 1) / C::BR;
  const int64_t total = (int64_t)p.n_splits * p.B * p.Hq * p.n_qtiles;
  if (total <= 0 || total >= (int64_t)1 << 31) return hipErrorInvalidValue;
  p.total_wg = (int)total;
  hipLaunchKernelGGL((attn_fwd_wide_kernel<D, NKB>), dim3(p.total_wg), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

LaunchFn wide_launcher(int elt, int D) {
  if (elt != ELT_BF16) return nullptr;
  switch (D) {
    // 64-key tiles where two K and two V tiles fit in LDS and pay off
    case 192: return &launch_wide<192, 1>;
    case 256: return &launch_wide<256, 2>;
    case 320: return &launch_wide<320, 2>;
    case 384: return &launch_wide<384, 1>;
    case 448: return &launch_wide<448, 1>;
    case 512: return &launch_wide<512, 1>;
    default: return nullptr;
  }
}

}  // namespace attn
