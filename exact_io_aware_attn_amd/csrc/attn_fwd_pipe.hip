// attn_fwd_pipe.hip -- attention forward for gfx950 with direct-to-LDS K/V
// streaming: e4m3 (fp8) for head dims 64, 128 and 256, and the bf16 variant
// with a polynomial exponential (D = 64, 128), positive scale.  (Plain bf16
// runs attn_fwd_bf16.hip at D = 64 and 128 and the wide-head kernel at
// larger head dims.)
//
// Same algorithm as the generic tiled kernel (FlashAttention summary page,
// method paragraph; blog post "FlashAttention v1/v2/v3/v4", section "El truco
// que hizo posible todo: online softmax"), laid out for the MI355X pipes:
//
//  * Each wave owns 32 query rows; a work-group of 4 waves owns 128 rows and
//    two work-groups share a CU, so every SIMD runs two waves from two
//    independent work-groups (e4m3 D = 128 without the causal mask, on
//    large grids: one work-group of 8 waves, 256 rows, per CU).  Their barriers are independent, so while one
//    wave runs its exp/sum/convert work on the vector ALU the other keeps the
//    matrix pipe busy (the ZYFA article, sections "Why FP8 attention is
//    softmax-bound on MI355X" and "The three techniques, in plain terms",
//    explains why this overlap decides the speed on this GPU).
//  * K and V tiles move HBM/L2 -> LDS with buffer loads that write LDS
//    directly (no staging registers, no LDS store instructions); the range
//    check of the buffer resource zero-fills keys past Nkv.  Two buffers per
//    operand: the loads of tile t+1 are issued at the top of iteration t and
//    waited for at its end, one barrier per iteration.  The loads are issued
//    from inline assembly so that the compiler's own wait insertion, which
//    cannot tell the two buffers apart, does not stall every LDS read on
//    them; the kernel waits for them explicitly before its barrier.
//  * LDS layouts are unpadded with XOR swizzles on 16-byte chunks (see
//    k_swz / v_swz): every LDS read phase touches distinct banks.
//  * V is never transposed in registers: ds_read_b64_tr_b16 returns, for
//    each lane, four consecutive keys of one head-dim column, which is
//    exactly the A operand of O^T += V^T P^T.
//  * Row sums add the fp32 probabilities before rounding: a sum of the
//    bf16-rounded values would move the LSE of short (early causal) rows by
//    up to ~2^-9 relative.
//  * e4m3 inputs (ZYFA article, "Why FP8 attention is softmax-bound on
//    MI355X": only the two products change precision): K tiles stream into
//    LDS as codes and feed the fp8 matrix instruction (64-wide contraction)
//    against Q codes held in registers.  V is staged through registers one
//    tile ahead, widened exactly to bf16 and written to LDS in the bf16
//    layout, so P V runs on the bf16 matrix instruction with P rounded to
//    bf16 as in the bf16 kernel.  The Q and K descales fold into the exp2
//    multiplier and the V descale into the final 1/l.
//  * Lazy rescale (ZYFA article, "The details that make it
//    production-grade"): the running max moves, and O and l are rescaled,
//    only when a row's new max exceeds it by more than 8 (base-2 units).
//    With a stale max the probabilities are at most 2^8, which bf16 and the
//    fp32 accumulators hold as well as values <= 1; O/l and m + log2(l) are
//    unchanged, so the result is still exact.
#include "attn_common.h"
#include "attn_dma.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, base-2 units

template <int E_, int D_, int NW_, int NBUF_, int BC_>
struct PipeCfg {
  static constexpr bool FP8 = E_ == ELT_FP8;    // e4m3 Q/K/V, otherwise bf16
  static constexpr int D = D_;
  static constexpr int NW = NW_;                // waves per work-group
  static constexpr int NBUF = NBUF_;            // K/V tiles resident (ring)
  static constexpr int QB = 1;                  // 32-row query blocks per wave
  static constexpr int BC = BC_;                // keys per tile
  static constexpr bool LARGE = D_ > 128;       // Q/O too large for 2 waves per SIMD (e4m3 D = 256)
  static constexpr int NT = NW * 64;            // threads per work-group
  static constexpr int QW = QB * 32;            // query rows per wave
  static constexpr int BR = NW * QW;            // query rows per work-group
  static constexpr int ES = FP8 ? 1 : 2;        // bytes per input element
  static constexpr int RPK = D_ * ES;           // K row pitch (bytes, HBM and LDS)
  static constexpr int RP = D_ * 2;             // V row pitch in LDS (bf16)
  static constexpr int TILE_K = BC * RPK;       // bytes of one K tile in LDS
  static constexpr int TILE = BC * RP;          // bytes of one V tile in LDS
  static constexpr int DMA_K = TILE_K / 1024 / NW;       // direct-to-LDS loads per wave, K tile
  static constexpr int DMA_WAVE = FP8 ? 1 : TILE / 1024 / NW;  // same, V tile (bf16 only)
  static constexpr int VST = FP8 ? BC * D_ / (16 * NT) : 1;    // e4m3 V: 16-byte loads per thread
  static constexpr int NDB = D_ / 32;           // 32-row blocks of O^T
  static constexpr int NQC = D_ / 16;           // 16-wide d chunks of the bf16 QK^T contraction
  static constexpr int NQ8 = D_ / 64;           // 64-wide d chunks of the e4m3 QK^T contraction
  static constexpr int NKB = BC / 32;           // 32-key blocks of S^T per tile
  static constexpr int LDS = NBUF * (TILE_K + TILE);  // K ring, V ring
  static constexpr int SW = (D_ % 128 == 0) ? 16 : 8;  // swizzle width (16-byte chunks)
  static constexpr int LK = NQC < 8 ? NQC : 8;  // K fragments in flight (large D)
  static constexpr int LV = NDB < 4 ? NDB : 4;  // V fragments in flight (large D)
  // s_waitcnt immediate for vmcnt(n): the loads of the NBUF-2 tiles issued
  // after a given tile may stay in flight (expcnt, lgkmcnt at their maxima)
  static constexpr int LATER = (NBUF - 2) * (DMA_K + DMA_WAVE);
  static constexpr int WAIT_LATER = 0x0F70 | (LATER & 15) | ((LATER >> 4) << 14);
  static_assert(NBUF >= 2 && LATER < 64, "ring depth");
  static_assert(!FP8 || NBUF == 2, "the e4m3 V staging assumes two buffers");
  static_assert(D_ % 64 == 0, "D must be a multiple of 64");
  static_assert(BC % 32 == 0, "BC must be a multiple of 32");
  static_assert(TILE_K % (1024 * NW) == 0 && TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(!FP8 || (BC * D_) % (16 * NT) == 0, "e4m3 V tile must split evenly over the threads");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(!LARGE || FP8, "bf16 beyond D = 128 runs the wide-head kernel");
};

// 2^y by a polynomial on the FMA pipe instead of v_exp_f32 (blog post
// "FlashAttention v1/v2/v3/v4", table of ideas: FA4 computes part of the
// exponentials with a polynomial): y = j + f with j = floor(y), 2^f from a
// cubic fitted to minimise the relative error on [0, 1) (at most 8.6e-5,
// below bf16's 2^-9), then scaled by 2^j (v_ldexp; y below -200, -inf
// included, gives 0).
__device__ __forceinline__ float poly_exp2(float y) {
  y = fmaxf(y, -200.0f);
  const float j = __builtin_floorf(y);
  const float f = y - j;
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(0.07706515f, f, 0.22764705f), f, 0.69511634f), f, 1.0f);
  return __builtin_ldexpf(p, (int)j);
}

template <int E, int D, int NW, int NBUF, int BC, bool POLY = false>
__global__ __launch_bounds__(NW * 64, (NW == 4 && D <= 128) ? ((E == ELT_BF16 && D == 128 && BC == 32) ? 3 : 2) : 1) void attn_fwd_pipe_kernel(FwdParams p) {
  using C = PipeCfg<E, D, NW, NBUF, BC>;
  constexpr bool FP8 = C::FP8;
  constexpr int QB = C::QB;
  // LDS: K ring (NBUF tiles) then V ring (NBUF tiles)
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  // LDS byte address of the buffer (the M0 operand of the loads)
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);
  char* const ldsV = lds + NBUF * C::TILE_K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work decomposition --------------------------------------------------
  const int wg_all = xcd_remap(blockIdx.x, p.total_wg);
  const int per_split = p.total_wg / p.n_splits;
  const int split = wg_all / per_split;  // key range (split-KV); 0 for a plain call
  const int wg = wg_all - split * per_split;
  const KeyRange kr = key_range(p, split);
  // one query tile per work-group, or a causal pair n-1-i, i (largest first)
  const int nslot = qtile_slots(p);
  const int slot_q = wg % nslot;
  const int bh = wg / nslot;
  const int hq = bh % p.Hq;
  const int b = bh / p.Hq;
  const int njobs = (p.pair_causal && 2 * slot_q + 1 != p.n_qtiles) ? 2 : 1;
  for (int job = 0; job < njobs; ++job) {
  if (job > 0) __syncthreads();  // every wave is done with the LDS of the first tile
  const int qt = (p.causal && job == 0) ? (p.n_qtiles - 1 - slot_q) : slot_q;
  const int hk = hq / p.group;
  const int q0 = qt * C::BR;
  const int q0w = q0 + wave * C::QW;

  const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq * D;
  const int64_t kv_slab = (((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv + kr.k0) * D;
  const uint32_t kv_bytes = (uint32_t)((int64_t)kr.nkv * D * C::ES);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc((const char*)p.q + q_slab * C::ES, (uint32_t)((int64_t)p.Nq * D * C::ES));
  const i32x4 rk = sgpr_rsrc((const char*)p.k + kv_slab * C::ES, kv_bytes);
  const i32x4 rv = sgpr_rsrc((const char*)p.v + kv_slab * C::ES, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv8 = make_rsrc((const char*)p.v + kv_slab * C::ES, kv_bytes);

  // exp(x) = exp2(x log2 e); e4m3 folds the Q and K descales in here and the
  // V descale into 1/l.  Positive (the launcher routes other scales elsewhere).
  // With one descale per 64-row block (FA blog, "FA3 — el momento Hopper":
  // a scale per 64 x d tile), this wave's 32 query rows lie in one Q block
  // and each key tile in one K/V block: the Q and K block descales fold into
  // the tile's exp2 multiplier and the V block descale into the exponent
  // (P is formed already multiplied by it) and into the tile's row sum.
  float c = p.scale * kLog2e;
  float out_scale = 1.0f;
  int64_t kv_blk0 = 0;   // first K/V block descale of this (batch, KV head)
  if constexpr (FP8) {
    if (p.blk_scaled) {
      const int nqb = (p.Nq + 63) / 64;
      c *= p.dq[((int64_t)b * p.Hq + hq) * nqb + min(q0w, p.Nq - 1) / 64];
      kv_blk0 = ((int64_t)b * p.Hkv + hk) * ((p.Nkv + 63) / 64);
    } else {
      c *= (p.dq ? p.dq[0] : 1.0f) * (p.dk ? p.dk[0] : 1.0f);
      out_scale = p.dv ? p.dv[0] : 1.0f;
    }
  }

  // ---- key range ------------------------------------------------------------------
  int kv_end = kr.nkv;
  if (p.causal) kv_end = min(kr.nkv, min(q0 + C::BR, p.Nq) + kr.kv_off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;

  // ---- K/V staging ------------------------------------------------------------------
  // K (either type) and bf16 V: direct-to-LDS loads.  e4m3 V: thread t loads
  // 16-byte runs (16 codes of one key) u = t + i NT of the tile, widens them
  // to two bf16 chunks and stores those where the bf16 layout puts them.
  uint32_t dk[C::DMA_K], dv[C::DMA_WAVE];
  if constexpr (FP8)
    dma_offsets_rows<C::DMA_K, C::RPK>(dk, wave, lane, [](int row) { return k8_swz<C::RPK>(row); });
  else
    dma_offsets<C, false>(dk, wave, lane);
  if constexpr (!FP8) dma_offsets<C, true>(dv, wave, lane);
  auto issue_k = [&](int t, int slot) {
    dma_blocks<C::DMA_K>(rsrc_at(rk, (uint32_t)(t * C::TILE_K)), lds_base + (uint32_t)(slot * C::TILE_K), dk,
                         wave);
  };
  auto issue_tile = [&](int t, int slot) {
    issue_k(t, slot);
    dma_tile<C>(rsrc_at(rv, (uint32_t)(t * C::TILE)), lds_base + (uint32_t)(NBUF * C::TILE_K + slot * C::TILE),
                dv, wave);
  };
  constexpr int V8_CH = D / 16;  // 16-byte code runs per key row
  u32x4 vst[C::VST];
  auto v8_load = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::VST; ++i) {
      const int u = tid + i * C::NT;
      vst[i] = buf_load16(rv8, (uint32_t)((t * C::BC + u / V8_CH) * D + (u % V8_CH) * 16));
    }
  };
  auto v8_store = [&](int slot) {
#pragma unroll
    for (int i = 0; i < C::VST; ++i) {
      const int u = tid + i * C::NT;
      const int row = u / V8_CH, ch = u % V8_CH;
      const u32x2 w0 = e4m3x4_to_bf16x4(vst[i].x), w1 = e4m3x4_to_bf16x4(vst[i].y);
      const u32x2 w2 = e4m3x4_to_bf16x4(vst[i].z), w3 = e4m3x4_to_bf16x4(vst[i].w);
      char* const vrow = ldsV + slot * C::TILE + row * C::RP;
      lds_store16(vrow, (uint32_t)(((2 * ch) ^ v_swz<D>(row)) << 4), u32x4{w0.x, w0.y, w1.x, w1.y});
      lds_store16(vrow, (uint32_t)(((2 * ch + 1) ^ v_swz<D>(row)) << 4), u32x4{w2.x, w2.y, w3.x, w3.y});
    }
  };

  // ---- prologue loads: tiles 0 .. NBUF-2 (LDS), Q (registers) --------------------
  if constexpr (FP8) {
    // K tile 0 to LDS, V tile 0 widened into its slot, V tile 1 to registers
    if (n_kt > 0) {
      v8_load(0);
      issue_k(0, 0);
      v8_store(0);
      if (n_kt > 1) v8_load(1);
    }
  } else {
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
      if (t < n_kt) issue_tile(t, t);
  }
  // Q fragments (B operand of S^T = K Q^T).  bf16: 16 d per instruction,
  // lane half h holds d = 16cc + 8h .. +7.  e4m3: 64 d per instruction, lane
  // half h holds d = 64cc + 32h .. +31.
  u32x4 qf[QB][FP8 ? 1 : C::NQC];
  i32x8 q8[QB][FP8 ? C::NQ8 : 1];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint32_t row_off = (uint32_t)(q0w + qb * 32 + l32) * (uint32_t)C::RPK;
    if constexpr (FP8) {
#pragma unroll
      for (int cc = 0; cc < C::NQ8; ++cc) {
        const u32x4 lo = buf_load16(rq, row_off + (uint32_t)(cc * 64 + h * 32));
        const u32x4 hi = buf_load16(rq, row_off + (uint32_t)(cc * 64 + h * 32 + 16));
        q8[qb][cc] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < C::NQC; ++cc) qf[qb][cc] = buf_load16(rq, row_off + (uint32_t)(cc * 32 + h * 16));
    }
  }

  f32x16 acc[QB][C::NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[qb][db] = f32x16{};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }

  // per-lane LDS byte offsets that do not change across tiles.  The swizzles
  // XOR the low log2(SW) bits of a 16-byte chunk index, so fragment cc of K
  // (chunk 2cc + h) sits at kbase[cc % KG] + (cc / KG) * SW * 16 and fragment
  // db of V (chunk 4db + ...) at vbase[db % VG] + (db / VG) * SW * 16.
  // K fragment (A operand of S^T = K Q^T): row l32 (+32 kb), chunk 2cc + h
  constexpr int KG = C::SW / 2, VG = C::SW / 4;
  uint32_t kbase[KG];
#pragma unroll
  for (int i = 0; i < KG; ++i) kbase[i] = (uint32_t)(l32 * C::RP + (((2 * i + h) ^ k_swz<D>(l32)) << 4));
  auto koff = [&](int cc) { return kbase[cc % KG] + (uint32_t)((cc / KG) * C::SW * 16); };
  // e4m3 K fragment cc: row l32 (+32 kb), code chunks 4cc + 2h and 4cc + 2h + 1
  uint32_t k8base[FP8 ? 2 * C::NQ8 : 1];
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < 2 * C::NQ8; ++i)
      k8base[i] = (uint32_t)(l32 * C::RPK + (((4 * (i >> 1) + 2 * h + (i & 1)) ^ k8_swz<C::RPK>(l32)) << 4));
  }
  // V fragment (A operand of O^T += V^T P^T) via the transposing read: lane r
  // of each 16-lane group addresses row kbase + r/4, columns dbase + 4(r%4)..+3
  const int g16 = lane >> 4, r16 = lane & 15;
  uint32_t vbase[VG];
#pragma unroll
  for (int i = 0; i < VG; ++i) {
    const int chunk = i * 4 + 2 * (g16 & 1) + ((r16 & 3) >> 1);
    const int row = 4 * h + (r16 >> 2);  // + 16 s16 (+ 8): multiples of 4 keep row & 3
    vbase[i] = (uint32_t)(row * C::RP + ((chunk ^ v_swz<D>(row)) << 4) + ((r16 & 1) << 3));
  }
  auto voff = [&](int db) { return vbase[db % VG] + (uint32_t)((db / VG) * C::SW * 16); };
  // last visible key of this lane's query row in each block
  int klim[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = q0w + qb * 32 + l32;
    klim[qb] = p.causal ? min(kr.nkv - 1, qrow + kr.kv_off) : kr.nkv - 1;
  }

  // Block descales of the K/V tiles: scalar loads one tile ahead, taken up
  // right after the loop-top barrier, whose wait already covers them (a
  // vector load would be waited for behind the in-flight tile loads).
  float dk_nx = 1.0f, dv_nx = 1.0f;
  if constexpr (FP8) {
    if (p.blk_scaled && n_kt > 0) {
      dk_nx = load_scalar(p.dk, kv_blk0 + kr.k0 / 64);
      dv_nx = load_scalar(p.dv, kv_blk0 + kr.k0 / 64);
    }
  }

  int slot = 0;  // ring slot of tile kt
  for (int kt = 0; kt < n_kt; ++kt) {
    // Tile kt is resident once at most the loads of the NBUF-2 later tiles
    // are outstanding (loads complete in order); the barrier makes every
    // wave's loads and LDS stores visible and frees the slot of tile kt-1.
    if (kt + NBUF - 2 < n_kt)
      __builtin_amdgcn_s_waitcnt(C::WAIT_LATER);
    else
      wait_vmem_all();
    __syncthreads();
    // this tile's exp2 multiplier, log2 of the V factor in P, 1 / that factor
    float ct = c, lg_v = 0.0f, inv_v = 1.0f;
    if constexpr (FP8) {
      if (p.blk_scaled) {
        ct = c * dk_nx;
        lg_v = __builtin_amdgcn_logf(dv_nx);
        inv_v = __builtin_amdgcn_rcpf(dv_nx);
        asm volatile("" ::"v"(ct), "v"(lg_v), "v"(inv_v));
        if (kt + 1 < n_kt) {
          const int64_t kblk = kv_blk0 + (kr.k0 + (kt + 1) * C::BC) / 64;
          dk_nx = load_scalar(p.dk, kblk);
          dv_nx = load_scalar(p.dv, kblk);
        }
      }
    }
    const int nslot = slot == 0 ? NBUF - 1 : slot - 1;  // slot of tile kt-1, free now
    if constexpr (FP8) {
      // V tile kt+1 (in registers since the last iteration) into its slot,
      // V tile kt+2 into the registers, then K tile kt+1.  The K loads go
      // last so that the wait the compiler places before the widening (it
      // does not see them) never covers them.
      if (kt + 1 < n_kt) {
        v8_store(nslot);
        if (kt + 2 < n_kt) v8_load(kt + 2);
        issue_k(kt + 1, nslot);
      }
    } else if constexpr (!C::LARGE) {
      if (kt + NBUF - 1 < n_kt) issue_tile(kt + NBUF - 1, nslot);
    }
    const char* const kb_cur = lds + slot * C::TILE_K;
    const char* const vb_cur = ldsV + slot * C::TILE;
    slot = slot == NBUF - 1 ? 0 : slot + 1;
    // a causal tile entirely above this wave's rows (loaded for the
    // work-group's later waves) adds nothing to them
    if (p.causal && kt * C::BC > q0w + C::QW - 1 + kr.kv_off) continue;

  // ---- S^T = K Q^T ------------------------------------------------------------
    f32x16 s[QB][C::NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) s[qb][kb] = f32x16{};
    if constexpr (FP8) {
      // e4m3: K fragments of one 32-key block (D/64 x 32 bytes per lane) are
      // read before its MFMAs, the next block's while they run
      auto kfrag8 = [&](int kb, int cc) {
        const uint32_t kbo = (uint32_t)(kb * 32 * C::RPK);
        const u32x4 lo = lds_load16(kb_cur, k8base[2 * cc] + kbo);
        const u32x4 hi = lds_load16(kb_cur, k8base[2 * cc + 1] + kbo);
        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      i32x8 kfa[C::NQ8], kfb[C::NQ8];
#pragma unroll
      for (int cc = 0; cc < C::NQ8; ++cc) kfa[cc] = kfrag8(0, cc);
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        i32x8(&cur)[C::NQ8] = (kb & 1) ? kfb : kfa;
        i32x8(&nxt)[C::NQ8] = (kb & 1) ? kfa : kfb;
        if (kb + 1 < C::NKB) {
#pragma unroll
          for (int cc = 0; cc < C::NQ8; ++cc) nxt[cc] = kfrag8(kb + 1, cc);
        }
#pragma unroll
        for (int cc = 0; cc < C::NQ8; ++cc) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma_fp8(cur[cc], q8[qb][cc], s[qb][kb]);
        }
      }
    } else if constexpr (!C::LARGE) {
      // K fragments of a whole 32-key block are read before its MFMAs, and the
      // next block's reads are issued before the current block's MFMAs, so LDS
      // latency overlaps the matrix work instead of stalling each instruction.
      u32x4 kfa[C::NQC], kfb[C::NQC];
#pragma unroll
      for (int cc = 0; cc < C::NQC; ++cc) kfa[cc] = lds_load16(kb_cur, koff(cc));
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        u32x4(&cur)[C::NQC] = (kb & 1) ? kfb : kfa;
        u32x4(&nxt)[C::NQC] = (kb & 1) ? kfa : kfb;
        if (kb + 1 < C::NKB) {
#pragma unroll
          for (int cc = 0; cc < C::NQC; ++cc) nxt[cc] = lds_load16(kb_cur, koff(cc) + (uint32_t)((kb + 1) * 32 * C::RP));
        }
#pragma unroll
        for (int cc = 0; cc < C::NQC; ++cc) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma_bf16(cur[cc], qf[qb][cc], s[qb][kb]);
        }
      }
    } else {
      // large D: a rolling window of LK K fragments over the whole tile
      // (fragment f = (kb, cc)); the fences keep each read LK MFMAs ahead
      constexpr int NF = C::NKB * C::NQC;
      auto kaddr = [&](int f) { return koff(f % C::NQC) + (uint32_t)((f / C::NQC) * 32 * C::RP); };
      u32x4 kf[C::LK];
#pragma unroll
      for (int i = 0; i < C::LK; ++i) kf[i] = lds_load16(kb_cur, kaddr(i));
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const u32x4 cur = kf[f % C::LK];
        if (f + C::LK < NF) kf[f % C::LK] = lds_load16(kb_cur, kaddr(f + C::LK));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][f / C::NQC] = mfma_bf16(cur, qf[qb][f % C::NQC], s[qb][f / C::NQC]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- mask (tiles crossing the diagonal or the key tail only) ------------------
    const int key0 = kt * C::BC;
    if ((key0 + C::BC > kr.nkv) || (p.causal && key0 + C::BC - 1 > q0w + kr.kv_off)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            s[qb][kb][r] = key <= klim[qb] ? s[qb][kb][r] : -INFINITY;
          }
    }

    // ---- online softmax with lazy rescale -----------------------------------------
    u32x4 pf[QB][2 * C::NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // one running chain, so the compiler forms v_max3 (two scores each)
      float mx = fmaxf(s[qb][0][0], s[qb][0][1]);
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[qb][kb][r]), s[qb][kb][r + 1]);
      const float mrow = max_halves(mx) * ct;  // scaled (base-2) units
      if (__builtin_amdgcn_ballot_w64(mrow > m_run[qb] + kTau) != 0) {
        // rows that have seen no visible key yet keep m = -inf; exp2 of
        // (-inf) - 0 is 0 there, never (-inf) - (-inf)
        const float m_new = fmaxf(m_run[qb], mrow);
        const float alpha = exp2_fast(m_run[qb] - (m_new == -INFINITY ? 0.0f : m_new));
        if constexpr (C::LARGE) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) scale_acc(acc[qb][db], alpha);
        } else {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) acc[qb][db] *= alpha;
        }
        l_run[qb] *= alpha;
        m_run[qb] = m_new;
      }
      const float mneg = (m_run[qb] == -INFINITY ? 0.0f : -m_run[qb]) + lg_v;
      float ls = FP8 ? 0.0f : l_run[qb];
#pragma unroll
      for (int s16 = 0; s16 < 2 * C::NKB; ++s16) {
        const int kb = s16 >> 1, r0 = (s16 & 1) * 8;
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float y = __builtin_fmaf(s[qb][kb][r0 + i], ct, mneg);
          e[i] = POLY ? poly_exp2(y) : exp2_fast(y);
        }
        pf[qb][s16].x = pack_bf16x2(e[0], e[1]);
        pf[qb][s16].y = pack_bf16x2(e[2], e[3]);
        pf[qb][s16].z = pack_bf16x2(e[4], e[5]);
        pf[qb][s16].w = pack_bf16x2(e[6], e[7]);
        ls += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      }
      l_run[qb] = FP8 ? __builtin_fmaf(ls, inv_v, l_run[qb]) : ls;
    }

    // ---- O^T += V^T P^T ---------------------------------------------------------------
    // V fragments: the reads of 16-key sub-block s16+1 are issued before the
    // MFMAs of sub-block s16.
    auto vfrag = [&](int s16, int db) {
      const uint32_t a0 = voff(db) + (uint32_t)(s16 * 16 * C::RP);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb_cur + a0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb_cur + a0 + 8 * C::RP));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2.x, l2.y, h2.x, h2.y};
    };
    if constexpr (!C::LARGE) {
      u32x4 vfa[C::NDB], vfb[C::NDB];
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) vfa[db] = vfrag(0, db);
#pragma unroll
      for (int s16 = 0; s16 < 2 * C::NKB; ++s16) {
        u32x4(&cur)[C::NDB] = (s16 & 1) ? vfb : vfa;
        u32x4(&nxt)[C::NDB] = (s16 & 1) ? vfa : vfb;
        if (s16 + 1 < 2 * C::NKB) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) nxt[db] = vfrag(s16 + 1, db);
        }
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma_bf16(cur[db], pf[qb][s16], acc[qb][db]);
        }
      }
    } else {
      // large D: a rolling window of LV V fragments over the whole tile
      // (fragment f = (s16, db))
      constexpr int NF = 2 * C::NKB * C::NDB;
      u32x4 vf[C::LV];
#pragma unroll
      for (int i = 0; i < C::LV; ++i) vf[i] = vfrag(i / C::NDB, i % C::NDB);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const u32x4 cur = vf[f % C::LV];
        if (f + C::LV < NF) vf[f % C::LV] = vfrag((f + C::LV) / C::NDB, (f + C::LV) % C::NDB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][f % C::NDB] = mfma_bf16(cur, pf[qb][f / C::NDB], acc[qb][f % C::NDB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

  }

  // ---- epilogue ---------------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_halves(l_run[qb]);
    const float inv = l_tot > 0.0f ? out_scale / l_tot : 0.0f;
    const int qrow = q0w + qb * 32 + l32;
    if (qrow < p.Nq) {
      const int64_t orow = split * p.o_split_stride + q_slab + (int64_t)qrow * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * h;
          store_o4(p.o, p.o_f32, orow + d, acc[qb][db][4 * g + 0] * inv, acc[qb][db][4 * g + 1] * inv,
                   acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv);
        }
      }
      if (p.lse != nullptr && h == 0)
        p.lse[split * p.lse_split_stride + ((int64_t)b * p.Hq + hq) * p.Nq + qrow] =
            l_tot > 0.0f ? (m_run[qb] + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}  // job
}

template <int E, int D, int NW, int NBUF, int BC, bool POLY = false>
hipError_t launch_pipe(const FwdParams& p0, hipStream_t stream) {
  using C = PipeCfg<E, D, NW, NBUF, BC>;
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + C::BR - 1) / C::BR;
  p.pair_causal = pair_causal_tiles(p);
  const int64_t total = (int64_t)p.n_splits * p.B * p.Hq * qtile_slots(p);
  if (total <= 0 || total >= (int64_t)1 << 31) return hipErrorInvalidValue;
  p.total_wg = (int)total;
  hipLaunchKernelGGL((attn_fwd_pipe_kernel<E, D, NW, NBUF, BC, POLY>), dim3(p.total_wg), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

// e4m3 D = 128: without the causal mask, and where 256-row work-groups
// still give every CU one, eight waves share each 64-key tile (half the K
// loads and V staging per product at the same two waves per SIMD), as in
// the bf16 kernel of attn_fwd_bf16.hip.
hipError_t launch_pipe_fp8_d128(const FwdParams& p, hipStream_t stream) {
  if (!p.causal) {
    using C8 = PipeCfg<ELT_FP8, 128, 8, 2, 64>;
    const int64_t wide = (int64_t)p.n_splits * p.B * p.Hq * ((p.Nq + C8::BR - 1) / C8::BR);
    if (wide >= (int64_t)cu_count()) return launch_pipe<ELT_FP8, 128, 8, 2, 64>(p, stream);
  }
  return launch_pipe<ELT_FP8, 128, 4, 2, 64>(p, stream);
}

}  // namespace

LaunchFn pipe_launcher(int elt, int D) {
  if (elt == ELT_FP8) {
    switch (D) {
      // e4m3 K rows of D bytes; V widened to bf16 in LDS
      case 64: return &launch_pipe<ELT_FP8, 64, 4, 2, 64>;
      case 128: return &launch_pipe_fp8_d128;
      case 256: return &launch_pipe<ELT_FP8, 256, 4, 2, 32>;
      default: return nullptr;
    }
  }
  if (elt != ELT_BF16) return nullptr;
  return bf16_launcher(D);  // attn_fwd_bf16.hip
}

LaunchFn pipe_poly_launcher(int D) {
  switch (D) {
    case 64: return &launch_pipe<ELT_BF16, 64, 4, 2, 64, true>;
    case 128: return &launch_pipe<ELT_BF16, 128, 4, 2, 64, true>;
    default: return nullptr;
  }
}

}  // namespace attn
