// attn_fwd_splitd.hip -- exact attention forward for large head dims
// (bf16, D a multiple of 32 in [288, 992]; D = 1024 has its own eight-wave
// kernel, attn_fwd_splitd8.hip) on gfx950.
//
// FFPA README, section "Split-D and TiledMMA": two things grow with D -- the
// on-chip footprint of the Q/K/V tiles and the registers of the output
// accumulator.  FFPA breaks the first by chunking D and the second by
// splitting the P V product's N = D dimension across warps ("M4N2").  The
// same two ideas, recast for wave64 MFMA and the MI355X register file:
//
//  * A work-group has 4 waves = 2 query halves (32 rows each) x 2 head-dim
//    halves (D/2 columns each).  Wave (qh, dh) keeps Q[32 rows, D/2 cols] in
//    registers and accumulates O^T[D/2 rows, 32 queries] -- D/8 + D/4
//    registers per lane, so D = 960 fits (120 VGPRs of Q, 240 accumulator
//    registers) where a wave owning all of D would need twice that.  The two
//    halves are interleaved: for S, wave dh owns the 16-column chunks
//    2cc + dh; for O, the 32-column blocks 2db + dh.  With the XOR swizzle
//    acting on the low three bits of the 16-byte chunk index, every fragment
//    address is then one per-lane base plus a compile-time offset.
//  * S^T = K Q^T is contracted over D in two halves: each wave of a
//    (qh, 0)/(qh, 1) pair computes the partial sum over its own D/2 columns,
//    the pair swaps partials through LDS (4 KiB per wave per tile), and both
//    add them (fp32 addition is commutative, so both hold bit-identical S).
//    Both then run the same online softmax (running max m, running sum l;
//    FA blog "El truco que hizo posible todo: online softmax") and each
//    multiplies P by its own D/2 columns of V.
//  * K and V tiles of 32 keys stream into LDS with direct-to-LDS buffer
//    loads (zero past Nkv) using the same XOR swizzles as the D <= 128
//    kernel.  At D = 960 one K tile and one V tile already take 120 KiB of
//    the 160 KiB LDS, so each is single-buffered and the two loads are
//    staggered: K(t+1) streams in while the softmax and P V of tile t run, and
//    V(t+1) streams in while the scores of tile t+1 are computed.  Two
//    barriers per tile.
//  * Causal masking, tails, lazy rescale (tau = 8, exact), XCD-contiguous
//    work-group ranges and heaviest-first causal order as in the other
//    kernels.
//  * A head dim that is an odd multiple of 32 runs at the layout of the next
//    multiple of 64, DP = D + 32: the 32 extra columns of each K/V row in LDS
//    hold whatever the loads bring (the start of the next row, or zeros past
//    the slab), the matching Q columns are zero, so the scores are exact,
//    and the extra 32 output columns are not stored.  HBM addressing uses the
//    real row pitch 2D throughout.
#include "attn_common.h"
#include "attn_dma.h"
#include "attn_launch.h"

namespace attn {

namespace {

// An empty asm that takes x and gives it back in the same vector register:
// the computation of x cannot be moved past it.
__device__ __forceinline__ void pin_f(float& x) { asm volatile("" : "+v"(x)); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;

typedef float f32x8 __attribute__((ext_vector_type(8)));

template <int D_>
struct SplitCfg {
  static constexpr int D = D_;
  static constexpr int NW = 4;                     // (query half) x (head-dim half)
  static constexpr int NT = NW * 64;
  static constexpr int BR = 64;                    // query rows per work-group
  static constexpr int BC = 32;                    // keys per tile
  static constexpr int DH = D_ / 2;                // head-dim columns per wave
  static constexpr int RP = D_ * 2;                // LDS row pitch (bytes)
  static constexpr int TILE = BC * RP;             // one K or V tile
  static constexpr int DMA_WAVE = TILE / 1024 / NW;
  static constexpr int NQC = DH / 16;              // QK^T k-steps per wave (16-col chunks 2cc + dh)
  static constexpr int NDB = DH / 32;              // 32-row blocks of O^T per wave (blocks 2db + dh)
  // fragments in flight (K: one read each, V: two); smaller windows for the
  // largest D, where Q alone takes D/8 VGPRs
  static constexpr int LK = D_ >= 896 ? 4 : 8;
  static constexpr int LV = D_ >= 896 ? 4 : 6;
  static constexpr bool TWO_ACC = D_ < 960;        // second S accumulator (16 VGPRs)
  static constexpr int KS = DMA_WAVE / 4;          // K(kt+1) blocks issued before the softmax
  static constexpr int XCH = NW * 64 * 16 * 4;     // partial-S exchange area
  static constexpr int LDS = 2 * TILE + XCH;
  static_assert(D_ % 64 == 0, "D must be a multiple of 64");
  static_assert((TILE / 1024) % NW == 0, "tile must split evenly over the waves");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  // one load block per two MFMAs in both the QK and the PV loop
  static_assert(NQC == 2 * DMA_WAVE && 2 * NDB == 2 * DMA_WAVE, "load interleave");
};

// DP: the layout's head dim (a multiple of 64); the real one is p.D, DP or
// DP - 32.
template <int DP>
__global__ __launch_bounds__(256, 1) void attn_fwd_splitd_kernel(FwdParams p) {
  using C = SplitCfg<DP>;
  const int D = p.D;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  char* const kbuf = lds;
  char* const vbuf = lds + C::TILE;
  char* const xch = lds + 2 * C::TILE;
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);
  const uint32_t lk = lds_base, lv = lds_base + C::TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave >> 1, dh = wave & 1;
  const int l32 = lane & 31;
  const int h = lane >> 5;

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
  const int q0w = q0 + qh * 32;
  const int qrow = q0w + l32;

  const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq * D;
  const int64_t kv_slab = (((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv + kr.k0) * D;
  const uint32_t kv_bytes = (uint32_t)((int64_t)kr.nkv * D * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)p.q + q_slab, (uint32_t)((int64_t)p.Nq * D * 2));
  const i32x4 rk = sgpr_rsrc((const __bf16*)p.k + kv_slab, kv_bytes);
  const i32x4 rv = sgpr_rsrc((const __bf16*)p.v + kv_slab, kv_bytes);
  const float c = p.scale * kLog2e;

  int kv_end = kr.nkv;
  if (p.causal) kv_end = min(kr.nkv, min(q0 + C::BR, p.Nq) + kr.kv_off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;

  // Per-lane HBM offsets of this wave's direct-to-LDS loads: block j covers
  // LDS tile bytes [(wave DMA_WAVE + j) KiB, +1 KiB) of RP-byte rows; lane l
  // writes 16 of them and fetches the 16-byte chunk the swizzle places there,
  // from the HBM row of pitch 2D.
  const uint32_t gpitch = (uint32_t)(2 * D);
  const uint32_t gtile = (uint32_t)C::BC * gpitch;  // one key tile in HBM
  auto dma_at = [&](bool is_v, int j) -> uint32_t {
    const int o = (wave * C::DMA_WAVE + j) * 1024 + lane * 16;
    const int row = o / C::RP;
    const int pc = (o - row * C::RP) >> 4;
    const int gc = pc ^ (is_v ? v_swz<DP>(row) : k_swz<DP>(row));
    return (uint32_t)row * gpitch + (uint32_t)(gc << 4);
  };
  uint32_t dk[C::DMA_WAVE], dv[C::DMA_WAVE];
#pragma unroll
  for (int j = 0; j < C::DMA_WAVE; ++j) {
    dk[j] = dma_at(false, j);
    dv[j] = dma_at(true, j);
  }
  // offset of load block j inside the loop: recomputed when the row pitch
  // makes a block one LDS row (DP = 512, 1024: the row, and so its swizzle
  // key, is uniform), which frees the 2 DMA_WAVE offset registers
  auto dma_off = [&](bool is_v, int j) -> uint32_t {
    if constexpr (C::RP % 1024 == 0) {
      constexpr int BPR = C::RP / 1024;  // blocks per row
      const int blk = wave * C::DMA_WAVE + j;
      const int row = blk / BPR;
      const int gc = ((blk % BPR) * 64 + lane) ^ (is_v ? v_swz<DP>(row) : k_swz<DP>(row));
      return (uint32_t)row * gpitch + (uint32_t)(gc << 4);
    } else {
      return is_v ? dv[j] : dk[j];
    }
  };
  if (n_kt > 0) {
    dma_tile<C>(rk, lk, dk, wave);
    dma_tile<C>(rv, lv, dv, wave);
  }
  // Q[qrow, 32 cc + 16 dh + 8 h .. + 7] (B operand of S^T = K Q^T)
  u32x4 qf[C::NQC];
  {
    const uint32_t row_off = (uint32_t)qrow * (uint32_t)(D * 2) + (uint32_t)(dh * 32 + h * 16);
#pragma unroll
    for (int cc = 0; cc < C::NQC; ++cc)
      qf[cc] = 32 * cc < D ? buf_load16(rq, row_off + (uint32_t)(cc * 64)) : u32x4{};  // zero past D
  }

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const int klim = p.causal ? min(kr.nkv - 1, qrow + kr.kv_off) : kr.nkv - 1;

  // K fragment: row l32, 16-byte chunk 4 cc + 2 dh + h.  The swizzle XORs
  // the low KB bits (KB = 3 or 4), so with G = 2^KB / 4 the address is
  // kbase[cc % G] + (cc / G) * 2^KB * 16.
  constexpr int KG = (DP % 128 == 0) ? 4 : 2;
  const int kx = k_swz<DP>(l32);
  uint32_t kbase[KG];
#pragma unroll
  for (int i = 0; i < KG; ++i) kbase[i] = (uint32_t)(l32 * C::RP + (((4 * i + 2 * dh + h) ^ kx) << 4));
  // V fragment (transposing read): row 16 s16 + 4 h + r16/4 (+ 8), columns
  // 64 db + 32 dh + 16 (g16 & 1) + 4 (r16 & 3) .. + 3, i.e. 16-byte chunk
  // 8 db + vlow with vlow = 4 dh + 2 (g16 & 1) + (r16 & 3) / 2; with
  // VG = 2^VB / 8 (VB = swizzle width in bits) the address is
  // vbase[db % VG] + (db / VG) * 2^VB * 16.
  constexpr int VG = (DP % 128 == 0) ? 2 : 1;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int vrow0 = 4 * h + (r16 >> 2);
  const int vlow = 4 * dh + 2 * (g16 & 1) + ((r16 & 3) >> 1);
  uint32_t vbase[VG];
#pragma unroll
  for (int i = 0; i < VG; ++i)
    vbase[i] = (uint32_t)(vrow0 * C::RP + (((8 * i + vlow) ^ v_swz<DP>(vrow0)) << 4) + ((r16 & 1) << 3));
  // partial-S exchange slots: wave w writes [w][j][lane] (16 B per lane, j = 0..3)
  char* const xmine = xch + wave * 4096 + lane * 16;
  const char* const xpeer = xch + (wave ^ 1) * 4096 + lane * 16;

  if (n_kt > 0) {
    wait_vmem_all();
    __syncthreads();
  }

  for (int kt = 0; kt < n_kt; ++kt) {
    // ---- partial S^T over this wave's D/2 columns (chunks 2cc + dh) -------------
    // K fragments through a rolling window of LK reads; two accumulators
    // (even and odd chunks, where registers allow) so that consecutive MFMAs
    // do not depend on each other.  V(kt) streams into its (free) buffer meanwhile, one block per
    // two MFMAs (the first tile's V came with the prologue).
    const i32x4 rv_t = rsrc_at(rv, (uint32_t)kt * gtile);
    f32x16 s;
    {
      auto kaddr = [&](int cc) { return kbase[cc % KG] + (uint32_t)((cc / KG) * KG * 64); };
      u32x4 kf[C::LK];
#pragma unroll
      for (int i = 0; i < C::LK; ++i) kf[i] = lds_load16(kbuf, kaddr(i));
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int cc = 0; cc < C::NQC; ++cc) {
        const u32x4 cur = kf[cc % C::LK];
        if (cc + C::LK < C::NQC) kf[cc % C::LK] = lds_load16(kbuf, kaddr(cc + C::LK));
        __builtin_amdgcn_sched_barrier(0);
        if ((cc & 1) && C::TWO_ACC)
          s1 = mfma_bf16(cur, qf[cc], s1);
        else
          s0 = mfma_bf16(cur, qf[cc], s0);
        if (cc < C::DMA_WAVE && kt > 0) dma_block_at<C::DMA_WAVE>(rv_t, lv, dma_off(true, cc), wave, cc);
        __builtin_amdgcn_sched_barrier(0);
      }
      s = C::TWO_ACC ? s0 + s1 : s0;
    }
    // (float sub-vectors, not per-element bit casts: this compiler collapses
    // bit-cast elements of an MFMA result vector onto element 0)
    *reinterpret_cast<f32x4*>(xmine) = __builtin_shufflevector(s, s, 0, 1, 2, 3);
    *reinterpret_cast<f32x4*>(xmine + 1024) = __builtin_shufflevector(s, s, 4, 5, 6, 7);
    *reinterpret_cast<f32x4*>(xmine + 2048) = __builtin_shufflevector(s, s, 8, 9, 10, 11);
    *reinterpret_cast<f32x4*>(xmine + 3072) = __builtin_shufflevector(s, s, 12, 13, 14, 15);
    wait_vmem_all();   // V(kt) resident
    __syncthreads();   // K buffer free, partials written, V(kt) visible
    // K(kt+1): the first KS blocks now (their issue overlaps the exchange
    // read and the softmax), the rest between the PV MFMAs below
    const bool k_next = kt + 1 < n_kt;
    const i32x4 rk_n = rsrc_at(rk, (uint32_t)(kt + 1) * gtile);
    if (k_next) {
#pragma unroll
      for (int j = 0; j < C::KS; ++j) dma_block_at<C::DMA_WAVE>(rk_n, lk, dma_off(false, j), wave, j);
    }

    // ---- S^T = own partial + peer partial --------------------------------------
    {
      const f32x4 o0 = *reinterpret_cast<const f32x4*>(xpeer);
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(xpeer + 1024);
      const f32x4 o2 = *reinterpret_cast<const f32x4*>(xpeer + 2048);
      const f32x4 o3 = *reinterpret_cast<const f32x4*>(xpeer + 3072);
      const f32x8 lo = __builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7);
      const f32x8 hi = __builtin_shufflevector(o2, o3, 0, 1, 2, 3, 4, 5, 6, 7);
      s += __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }

    // scale first (any sign of scale is allowed), then mask
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] *= c;
    const int key0 = kt * C::BC;
    if ((key0 + C::BC > kr.nkv) || (p.causal && key0 + C::BC - 1 > q0w + kr.kv_off)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * h + (r & 3);
        s[r] = key <= klim ? s[r] : -INFINITY;
      }
    }

    // ---- online softmax (identical in both waves of a pair) -------------------------
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
    const float mrow = max_halves(mx);  // base-2 units
    if (__builtin_amdgcn_ballot_w64(mrow > m_run + kTau) != 0) {
      const float m_new = fmaxf(m_run, mrow);
      const float alpha = exp2_fast(m_run - (m_new == -INFINITY ? 0.0f : m_new));
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) scale_acc(acc[db], alpha);
      l_run *= alpha;
      m_run = m_new;
    }
    const float mneg = m_run == -INFINITY ? 0.0f : -m_run;
    // P of keys 0..15 now; that of keys 16..31 between the first half of the
    // P V MFMAs below, which use only the first (spread evenly over them and
    // pinned there: left to the compiler they are moved past every MFMA to
    // their first use)
    u32x4 pf[2];
    float e[16];
    auto expo = [&](int i) {
      e[i] = exp2_fast(s[i] + mneg);
      pin_f(e[i]);
    };
    auto pack = [&](int s16) {
      pf[s16].x = pack_bf16x2(e[8 * s16 + 0], e[8 * s16 + 1]);
      pf[s16].y = pack_bf16x2(e[8 * s16 + 2], e[8 * s16 + 3]);
      pf[s16].z = pack_bf16x2(e[8 * s16 + 4], e[8 * s16 + 5]);
      pf[s16].w = pack_bf16x2(e[8 * s16 + 6], e[8 * s16 + 7]);
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) expo(i);
    pack(0);

    // ---- O^T[D/2 rows] += V^T P^T ------------------------------------------------------
    // V fragments (two transposing reads each) through a rolling window of
    // LV; the remaining blocks of K(kt+1) go out evenly between the MFMAs.
    {
      auto vfrag = [&](int f) {
        const int s16 = f / C::NDB, db = f % C::NDB;
        const uint32_t a0 = vbase[db % VG] + (uint32_t)(s16 * 16 * C::RP + (db / VG) * VG * 128);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vbuf + a0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vbuf + a0 + 8 * C::RP));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2.x, l2.y, h2.x, h2.y};
      };
      constexpr int NF = 2 * C::NDB;
      u32x4 vf[C::LV];
#pragma unroll
      for (int i = 0; i < C::LV; ++i) vf[i] = vfrag(i);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const u32x4 cur = vf[f % C::LV];
        if (f + C::LV < NF) vf[f % C::LV] = vfrag(f + C::LV);
        if (f == C::NDB) pack(1);
        __builtin_amdgcn_sched_barrier(0);
        acc[f % C::NDB] = mfma_bf16(cur, pf[f / C::NDB], acc[f % C::NDB]);
        if (f < C::NDB) {
#pragma unroll
          for (int i = (8 * f + C::NDB - 1) / C::NDB; i < (8 * (f + 1) + C::NDB - 1) / C::NDB; ++i) expo(8 + i);
        }
        if (k_next) {
          // blocks KS .. DMA_WAVE - 1, one after each of the first MFMAs
          if (C::KS + f < C::DMA_WAVE) dma_block_at<C::DMA_WAVE>(rk_n, lk, dma_off(false, C::KS + f), wave, C::KS + f);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {
      float ls = l_run;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        ls += ((e[4 * g + 0] + e[4 * g + 1]) + (e[4 * g + 2] + e[4 * g + 3]));
      l_run = ls;
    }
    wait_vmem_all();   // K(kt+1) resident
    __syncthreads();   // V buffer free, exchange area read, K(kt+1) visible
  }

  // ---- epilogue: this wave's 32-column blocks 2db + dh; LSE from the dh = 0 wave --
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < p.Nq) {
    const int64_t orow = split * p.o_split_stride + q_slab + (int64_t)qrow * D + dh * 32;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      if (db * 64 + dh * 32 >= D) continue;  // padding columns
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 64 + 8 * g + 4 * h;
        store_o4(p.o, p.o_f32, orow + d, acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                 acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
      }
    }
    if (p.lse != nullptr && dh == 0 && h == 0)
      p.lse[split * p.lse_split_stride + ((int64_t)b * p.Hq + hq) * p.Nq + qrow] =
          l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int DP>
hipError_t launch_splitd(const FwdParams& p0, hipStream_t stream) {
  using C = SplitCfg<DP>;
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + C::BR - 1) / C::BR;
  const int64_t total = (int64_t)p.n_splits * p.B * p.Hq * p.n_qtiles;
  if (total <= 0 || total >= (int64_t)1 << 31) return hipErrorInvalidValue;
  p.total_wg = (int)total;
  hipLaunchKernelGGL((attn_fwd_splitd_kernel<DP>), dim3(p.total_wg), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// D a multiple of 32 in [288, 992]; an odd multiple of 32 runs at the
// layout of D + 32.
LaunchFn splitd_launcher(int elt, int D) {
  if (elt != ELT_BF16 || D % 32 != 0 || D < 288 || D > 992) return nullptr;
  switch (D % 64 == 0 ? D : D + 32) {
    case 320: return &launch_splitd<320>;
    case 384: return &launch_splitd<384>;
    case 448: return &launch_splitd<448>;
    case 512: return &launch_splitd<512>;
    case 576: return &launch_splitd<576>;
    case 640: return &launch_splitd<640>;
    case 704: return &launch_splitd<704>;
    case 768: return &launch_splitd<768>;
    case 832: return &launch_splitd<832>;
    case 896: return &launch_splitd<896>;
    case 960: return &launch_splitd<960>;
    case 1024: return &launch_splitd<1024>;
    default: return nullptr;
  }
}

}  // namespace attn
