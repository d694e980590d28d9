// attn_fwd_bf16.hip -- bf16 attention forward for head dims 64 and 128 on
// gfx950, positive scale: the hot path of the prefill workloads.
//
// Algorithm: the tiled online softmax (FlashAttention summary page, method
// paragraph; blog post "FlashAttention v1/v2/v3/v4", section "El truco que
// hizo posible todo: online softmax"): per query row a running maximum m,
// a running sum l and an output accumulator, updated one key tile at a
// time; S is never written out.
//
// Layout (the direct-to-LDS kernel's, attn_fwd_pipe.hip, which keeps the
// e4m3 paths):
//  * A work-group is 4 waves x 32 query rows of one head; on large grids 8
//    waves, either 256 rows of one head (no causal mask) or the same 64
//    rows of 4 query heads that share a KV head (128 rows of 2), so that
//    every wave sees the same causal key range (GQA).  A wave owns its rows
//    through every key tile.  Transposed products on the 32x32x16 bf16 matrix
//    instruction: S^T = K Q^T (A = K from LDS, B = Q held in registers) and
//    O^T += V^T P^T (A = V^T from the transposing LDS read, B = P).  Lane l
//    holds query l % 32 in both accumulators, so the S^T registers rounded
//    to bf16 are the P operand as they stand.
//  * K and V tiles stream HBM/L2 -> LDS through buffer loads that write LDS
//    directly, two slots per operand, one barrier per tile.  The key loop
//    is unrolled by two tiles, so each tile's slot is a compile-time
//    constant and every LDS fragment address is a per-lane base register
//    plus an immediate offset (no address arithmetic per tile).
//  * Lazy rescale without a per-tile maximum.  The ZYFA article ("The
//    details that make it production-grade") rescales O only when the
//    running maximum grows past a threshold; here the tile's probabilities
//    are formed directly with the running maximum as it stands,
//    p = 2^(s c - m), and are kept unless some lane's sum of them over its
//    keys of the tile exceeds 2^16, or the row has seen no key yet (m =
//    -inf).  Only then is the tile's maximum taken, O and l rescaled and
//    the probabilities formed again.  Every kept probability is at most
//    2^16, far inside bf16 and the fp32 accumulators; m only ever takes
//    values that are row maxima, so probabilities never underflow more than
//    with the exact maximum; O / l and m + log2(l) do not depend on which m
//    was used, so the result is exact.  The common tile costs one compare
//    instead of the maximum's 14 vector instructions.
//  * Row sums add the fp32 probabilities before rounding (a sum of the
//    bf16-rounded values moves the LSE of short rows by up to ~2^-9).
#include "attn_common.h"
#include "attn_dma.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSumMax = 65536.0f;  // per-lane tile sum that forces a rescale

template <int D_, int BC_, int NW_ = 4>
struct Bf16Cfg {
  static constexpr int D = D_;
  static constexpr int NW = NW_;                // waves per work-group (4 or 8)
  static constexpr int NT = NW * 64;
  static constexpr int QW = 32;                 // query rows per wave
  static constexpr int BR = NW * QW;            // query rows per work-group
  static constexpr int BC = BC_;                // keys per tile
  static constexpr int RP = D_ * 2;             // row pitch (bytes), HBM and LDS
  static constexpr int TILE = BC * RP;          // one K or V tile
  static constexpr int DMA_WAVE = TILE / 1024 / NW;  // direct-to-LDS loads per wave per operand
  static constexpr int NDB = D_ / 32;           // 32-row blocks of O^T
  static constexpr int NQC = D_ / 16;           // 16-wide d chunks of the QK^T contraction
  static constexpr int NKB = BC / 32;           // 32-key blocks of S^T per tile
  static constexpr int NS16 = BC / 16;          // 16-key chunks of P per tile
  static constexpr int LDS = 4 * TILE;          // K slots 0, 1; V slots 0, 1
  static constexpr int SW = (D_ % 128 == 0) ? 16 : 8;  // swizzle width (16-byte chunks)
  static_assert(D_ == 64 || D_ == 128, "head dims 64 and 128");
  static_assert(BC % 32 == 0, "BC must be a multiple of 32");
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(LDS <= 64 * 1024, "two work-groups per CU at least");
};

template <int D, int BC, int NW = 4, int HP = 1>
__global__ __launch_bounds__(NW * 64, NW == 8 ? 1 : ((D == 128 && BC == 32) ? 3 : 2)) void attn_fwd_bf16_kernel(
    FwdParams p) {
  using C = Bf16Cfg<D, BC, NW>;
  // HP query heads of one KV head per work-group (GQA), WPH waves each; a
  // query tile is TR rows of every one of those heads
  static_assert(NW % HP == 0, "waves must split evenly over the heads");
  constexpr int WPH = NW / HP;
  constexpr int TR = WPH * C::QW;
  // LDS: K slot 0, K slot 1, V slot 0, V slot 1
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work decomposition --------------------------------------------------
  // One query tile per work-group, or a causal pair n-1-i, i (largest
  // first), over XCD-contiguous work-group ranges.
  const int wg_all = xcd_remap(blockIdx.x, p.total_wg);
  const int per_split = p.total_wg / p.n_splits;
  const int split = wg_all / per_split;  // key range (split-KV); 0 for a plain call
  const int wg = wg_all - split * per_split;
  const int nslot = qtile_slots(p);
  const int slot_q = wg % nslot;
  const int bh = wg / nslot;
  const int njobs = (p.pair_causal && 2 * slot_q + 1 != p.n_qtiles) ? 2 : 1;
  const KeyRange kr = key_range(p, split);

  // per-lane LDS byte offsets that do not change across tiles.  The swizzles
  // XOR the low log2(SW) bits of a 16-byte chunk index, so fragment cc of K
  // (chunk 2cc + h) sits at kbase[cc % KG] + (cc / KG) * SW * 16 and fragment
  // db of V (chunk 4db + ...) at vbase[db % VG] + (db / VG) * SW * 16.
  constexpr int KG = C::SW / 2, VG = C::SW / 4;
  uint32_t kbase[KG];
#pragma unroll
  for (int i = 0; i < KG; ++i) kbase[i] = (uint32_t)(l32 * C::RP + (((2 * i + h) ^ k_swz<D>(l32)) << 4));
  // V fragment via the transposing read: lane r of each 16-lane group
  // addresses row 4h + r/4 (+16 s16, +8), columns dbase + 4(r%4)..+3
  const int g16 = lane >> 4, r16 = lane & 15;
  uint32_t vbase[VG];
#pragma unroll
  for (int i = 0; i < VG; ++i) {
    const int chunk = i * 4 + 2 * (g16 & 1) + ((r16 & 3) >> 1);
    const int row = 4 * h + (r16 >> 2);  // + 16 s16 (+ 8): multiples of 4 keep row & 3
    vbase[i] = (uint32_t)(2 * C::TILE + row * C::RP + ((chunk ^ v_swz<D>(row)) << 4) + ((r16 & 1) << 3));
  }
  uint32_t dk[C::DMA_WAVE], dv[C::DMA_WAVE];
  dma_offsets<C, false>(dk, wave, lane);
  dma_offsets<C, true>(dv, wave, lane);

  for (int job = 0; job < njobs; ++job) {
    // (batch, head) re-derived per job: kept live across the key loop they
    // would take the last registers at three waves per SIMD
    const int hgroups = p.Hq / HP;
    const int hq = (bh % hgroups) * HP + wave / WPH;
    const int b = bh / hgroups;
    const int qt = (p.causal && job == 0) ? (p.n_qtiles - 1 - slot_q) : slot_q;
    if (job > 0) __syncthreads();  // every wave is done with the LDS of the previous tile
    const int hk = hq / p.group;
    const int q0 = qt * TR;
    const int q0w = q0 + (wave % WPH) * C::QW;

    const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq * D;
    const int64_t kv_slab = (((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv + kr.k0) * D;
    const uint32_t kv_bytes = (uint32_t)((int64_t)kr.nkv * D * 2);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)p.q + q_slab, (uint32_t)((int64_t)p.Nq * D * 2));
    const i32x4 rk = sgpr_rsrc((const __bf16*)p.k + kv_slab, kv_bytes);
    const i32x4 rv = sgpr_rsrc((const __bf16*)p.v + kv_slab, kv_bytes);
    const float c = p.scale * kLog2e;  // > 0: the launcher routes other scales elsewhere

    int kv_end = kr.nkv;
    if (p.causal) kv_end = min(kr.nkv, min(q0 + TR, p.Nq) + kr.kv_off);
    const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;

    auto issue_tile = [&](int t, int slot) {
      dma_blocks<C::DMA_WAVE>(rsrc_at(rk, (uint32_t)(t * C::TILE)), lds_base + (uint32_t)(slot * C::TILE), dk, wave);
      dma_blocks<C::DMA_WAVE>(rsrc_at(rv, (uint32_t)(t * C::TILE)), lds_base + (uint32_t)((2 + slot) * C::TILE), dv,
                              wave);
    };
    if (n_kt > 0) issue_tile(0, 0);

    // Q fragments (B operand of S^T = K Q^T): 16 d per instruction, lane
    // half h holds d = 16cc + 8h .. +7
    u32x4 qf[C::NQC];
    {
      const uint32_t row_off = (uint32_t)(q0w + l32) * (uint32_t)C::RP;
#pragma unroll
      for (int cc = 0; cc < C::NQC; ++cc) qf[cc] = buf_load16(rq, row_off + (uint32_t)(cc * 32 + h * 16));
    }
    f32x16 acc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    const int qrow = q0w + l32;
    const int klim = p.causal ? min(kr.nkv - 1, qrow + kr.kv_off) : kr.nkv - 1;

    auto tile = [&](int kt, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      // Tile kt's loads (issued one iteration earlier) are complete once
      // none is outstanding; the barrier makes every wave's loads visible
      // and frees the other slot (tile kt-1), which tile kt+1 then fills.
      wait_vmem_all();
      __syncthreads();
      if (kt + 1 < n_kt) issue_tile(kt + 1, 1 - SLOT);
      // a causal tile entirely above this wave's rows (loaded for the
      // work-group's later waves) adds nothing to them
      if (p.causal && kt * C::BC > q0w + C::QW - 1 + kr.kv_off) return;
      const char* const kb_cur = lds + SLOT * C::TILE;
      const char* const vb_cur = lds + SLOT * C::TILE;  // vbase already holds the V area's offset

      // ---- S^T = K Q^T: the K fragments of a 32-key block are read before
      // its MFMAs, the next block's while they run
      f32x16 s[C::NKB];
      auto kfrag = [&](int kb, int cc) {
        return lds_load16(kb_cur, kbase[cc % KG] + (uint32_t)((cc / KG) * C::SW * 16 + kb * 32 * C::RP));
      };
      u32x4 kfa[C::NQC], kfb[C::NQC];
#pragma unroll
      for (int cc = 0; cc < C::NQC; ++cc) kfa[cc] = kfrag(0, cc);
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        u32x4(&cur)[C::NQC] = (kb & 1) ? kfb : kfa;
        u32x4(&nxt)[C::NQC] = (kb & 1) ? kfa : kfb;
        if (kb + 1 < C::NKB) {
#pragma unroll
          for (int cc = 0; cc < C::NQC; ++cc) nxt[cc] = kfrag(kb + 1, cc);
        }
        s[kb] = f32x16{};
#pragma unroll
        for (int cc = 0; cc < C::NQC; ++cc) s[kb] = mfma_bf16(cur[cc], qf[cc], s[kb]);
      }

      // ---- mask (tiles crossing the diagonal or the key tail only) -------
      const int key0 = kt * C::BC;
      if ((key0 + C::BC > kr.nkv) || (p.causal && key0 + C::BC - 1 > q0w + kr.kv_off)) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            s[kb][r] = key <= klim ? s[kb][r] : -INFINITY;
          }
      }

      // ---- probabilities with the running maximum as it stands ------------
      float e[C::NKB][16];
      auto form = [&](float mneg) {
        float part[2 * C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) e[kb][r] = exp2_fast(__builtin_fmaf(s[kb][r], c, mneg));
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const float* x = &e[kb][8 * g];
            part[2 * kb + g] = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
          }
        }
        float ls = part[0];
#pragma unroll
        for (int i = 1; i < 2 * C::NKB; ++i) ls += part[i];
        return ls;
      };
      // A row that has seen no key yet (m = -inf) always takes the rescale
      // path; its first attempt's probabilities are discarded.  (NaN inputs
      // are outside the contract and compiled as absent, so the test is on
      // m itself, not on the sum.)
      float ls = form(-m_run);
      if (__builtin_amdgcn_ballot_w64(ls > kSumMax || m_run == -INFINITY) != 0) {
        // the tile's row maximum (both halves of the wave hold one query's
        // keys: the same maximum in both), then rescale and form again
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[kb][r]), s[kb][r + 1]);
        const float m_new = fmaxf(m_run, max_halves(mx) * c);
        // rows that have seen no visible key keep m = -inf; exp2 of
        // (-inf) - 0 is 0 there, never (-inf) - (-inf)
        const float alpha = exp2_fast(m_run - (m_new == -INFINITY ? 0.0f : m_new));
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) acc[db] *= alpha;
        l_run *= alpha;
        m_run = m_new;
        ls = form(m_run == -INFINITY ? 0.0f : -m_run);
      }
      l_run += ls;
      u32x4 pf[C::NS16];
#pragma unroll
      for (int s16 = 0; s16 < C::NS16; ++s16) {
        const int kb = s16 >> 1, r0 = (s16 & 1) * 8;
        pf[s16].x = pack_bf16x2(e[kb][r0 + 0], e[kb][r0 + 1]);
        pf[s16].y = pack_bf16x2(e[kb][r0 + 2], e[kb][r0 + 3]);
        pf[s16].z = pack_bf16x2(e[kb][r0 + 4], e[kb][r0 + 5]);
        pf[s16].w = pack_bf16x2(e[kb][r0 + 6], e[kb][r0 + 7]);
      }

      // ---- O^T += V^T P^T: the V reads of 16-key chunk s16+1 are issued
      // before the MFMAs of chunk s16
      auto vfrag = [&](int s16, int db) {
        const uint32_t a0 = vbase[db % VG] + (uint32_t)((db / VG) * C::SW * 16 + s16 * 16 * C::RP);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb_cur + a0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb_cur + a0 + 8 * C::RP));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2.x, l2.y, h2.x, h2.y};
      };
      u32x4 vfa[C::NDB], vfb[C::NDB];
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) vfa[db] = vfrag(0, db);
#pragma unroll
      for (int s16 = 0; s16 < C::NS16; ++s16) {
        u32x4(&cur)[C::NDB] = (s16 & 1) ? vfb : vfa;
        u32x4(&nxt)[C::NDB] = (s16 & 1) ? vfa : vfb;
        if (s16 + 1 < C::NS16) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) nxt[db] = vfrag(s16 + 1, db);
        }
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) acc[db] = mfma_bf16(cur[db], pf[s16], acc[db]);
      }
    };

    int kt = 0;
    for (; kt + 1 < n_kt; kt += 2) {
      tile(kt, std::integral_constant<int, 0>{});
      tile(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < n_kt) tile(kt, std::integral_constant<int, 0>{});

    // ---- epilogue -----------------------------------------------------------------
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
  }  // job
}

// Work-groups of a launch with NW waves per work-group over HP query heads
// (query tiles of 32 NW / HP rows), after the causal pairing; fills
// n_qtiles and pair_causal.
template <int NW, int HP>
int64_t bf16_grid(FwdParams& p) {
  constexpr int TR = NW * 32 / HP;
  const int64_t heads = (int64_t)p.n_splits * p.B * (p.Hq / HP);
  p.n_qtiles = (p.Nq + TR - 1) / TR;
  p.pair_causal = pair_causal_grid(p.causal, heads, p.n_qtiles, p.Nq, p.Nkv);
  return heads * qtile_slots(p);
}

template <int D, int BC, int NW = 4, int HP = 1>
hipError_t launch_bf16(const FwdParams& p0, hipStream_t stream) {
  using C = Bf16Cfg<D, BC, NW>;
  FwdParams p = p0;
  if (p.group % HP != 0) return hipErrorInvalidValue;
  const int64_t total = bf16_grid<NW, HP>(p);
  if (total <= 0 || total >= (int64_t)1 << 31) return hipErrorInvalidValue;
  p.total_wg = (int)total;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, BC, NW, HP>), dim3(p.total_wg), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

// D = 128: 32-key tiles at three waves per SIMD where the grid gives every
// CU at least three work-groups, otherwise 64-key tiles at two (a grid too
// small for the third slot gains nothing from the smaller tiles' extra
// barriers).  Where eight-wave work-groups still give every CU one, eight
// waves share each 64-key K/V tile instead: half the direct-to-LDS loads and
// L2-to-LDS bytes per product at two waves per SIMD.  Without the causal
// mask the eight waves take 256 rows of one query head.  With it, a 256-row
// work-group would load diagonal tiles that its first waves skip, so under
// GQA the eight waves take the same 64 rows of four query heads of one KV
// head (128 rows of two for a group of two), which see the same keys;
// causal MHA keeps the four-wave layouts.
hipError_t launch_bf16_d128(const FwdParams& p0, hipStream_t stream) {
  FwdParams p = p0;
  const int64_t cus = cu_count();
  if (!p.causal) {
    if (bf16_grid<8, 1>(p) >= cus) return launch_bf16<128, 64, 8>(p0, stream);
  } else if (p.group % 4 == 0) {
    if (bf16_grid<8, 4>(p) >= cus) return launch_bf16<128, 64, 8, 4>(p0, stream);
  } else if (p.group % 2 == 0) {
    if (bf16_grid<8, 2>(p) >= cus) return launch_bf16<128, 64, 8, 2>(p0, stream);
  }
  return bf16_grid<4, 1>(p) >= 3 * cus ? launch_bf16<128, 32>(p0, stream) : launch_bf16<128, 64>(p0, stream);
}

}  // namespace

LaunchFn bf16_launcher(int D) {
  switch (D) {
    case 64: return &launch_bf16<64, 64>;
    case 128: return &launch_bf16_d128;
    default: return nullptr;
  }
}

}  // namespace attn
