// attn_fwd_splitd8.hip -- exact attention forward for the largest head dim
// (bf16, D = 1024; the layout holds for D a multiple of 256 from 512) on
// gfx950: eight waves per work-group, the head dim split four ways, K/V
// staged in half-width column panels.
//
// FFPA README, section "Split-D and TiledMMA": with a large head dim the
// on-chip copies of Q/K/V and the output accumulator both grow with D; FFPA
// stages the D axis in chunks and splits the P V product's output columns
// across warps.  The same two ideas, sized for the MI355X register file and
// its 160 KiB LDS:
//
//  * A work-group owns 64 query rows and has 8 waves: 2 query halves (32
//    rows each) x 4 head-dim quarters.  Wave (qh, dq) keeps Q[32 rows, D/4
//    cols] in registers (16-column chunks 4cc + dq) and accumulates O^T[D/4
//    rows, 32 queries] (32-row blocks 4db + dq): D/16 + D/8 registers per
//    lane, 192 at D = 1024, so two waves fit on each SIMD and one wave's
//    matrix work covers the other's loads, waits and vector work.
//  * S^T = K Q^T is contracted over D in quarters.  Each wave writes the
//    three key quarters of its partial S^T that other waves own to LDS, and
//    sums its own key quarter (8 keys) over the four head-dim quarters in a
//    fixed order (a reduce-scatter: 3 KiB out and 3 KiB in per wave per
//    tile).  The online softmax (running max m, running sum l; FA blog "El
//    truco que hizo posible todo: online softmax") then runs on 8 keys per
//    wave instead of 32, and the waves exchange the bf16 probabilities (2
//    KiB in per wave) that every wave needs as the B operand of its P V.
//  * Every probability is formed with the running maximum as it stands,
//    p = 2^(s c - m), and kept unless some score of the tile exceeds m by
//    more than 8 (or the row has seen no key yet).  Such a tile is rare; the
//    four waves of a query half then agree on the tile's maximum through
//    LDS, rescale O and l by 2^(m_old - m_new) and form the probabilities
//    again.  Kept probabilities are at most 2^8, and O / l, m + log2 l do
//    not depend on which m was used, so the result is exact.  The decision
//    is taken by all eight waves together (a flag word per wave), so every
//    wave meets the same barriers.
//  * The key loop is skewed by one tile: iteration t forms the softmax of
//    tile t between the QK^T MFMAs of tile t+1, then runs tile t's P V, so
//    the vector work sits under matrix work of the same wave.
//  * K and V tiles (32 keys) are stored in LDS as two panels of D/2
//    columns each (panel row pitch D bytes, XOR-swizzled 16-byte chunks as
//    in the other kernels) and streamed by direct-to-LDS buffer loads issued
//    by all eight waves, one load after every other MFMA.  A panel is
//    refilled as soon as every wave has finished reading it (four barriers
//    per tile, one before each half of QK^T and of P V), so each load has
//    about one and a half MFMA phases to land instead of one; with a whole
//    K and a whole V tile in flight at once the L2-to-LDS path stays busy
//    for the whole tile.  At D = 1024 the two tiles take 128 KiB; the
//    exchange areas take the rest of the 160 KiB.
//  * Loads run up to two tiles ahead and are issued unconditionally (past
//    the last tile they re-read it; nothing reads that copy), so every wait
//    is the same vmcnt(2 x loads per panel) and the loop has no tail cases.
//  * Causal masking on diagonal and tail tiles, XCD-contiguous work-group
//    ranges, heaviest-first causal order, key ranges for split-KV: as in the
//    other kernels.  Scale of any sign.
#include "attn_common.h"
#include "attn_dma.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // log2 of the largest kept probability

template <int D_>
struct Sd8Cfg {
  static constexpr int D = D_;
  static constexpr int NW = 8;                     // (query half) x (head-dim quarter)
  static constexpr int NT = NW * 64;
  static constexpr int BR = 64;                    // query rows per work-group
  static constexpr int BC = 32;                    // keys per tile
  static constexpr int PP = D_;                    // panel row pitch (bytes): D/2 bf16 columns
  static constexpr int PANEL = BC * PP;
  static constexpr int TILE = 2 * PANEL;           // = one 32-key tile of K or V in HBM
  static constexpr int GP = PANEL / 1024 / NW;     // direct-to-LDS loads per wave per panel
  static constexpr int NQC = D_ / 64;              // QK^T MFMAs per wave per tile
  static constexpr int NDB = D_ / 128;             // 32-row blocks of O^T per wave
  static constexpr int HQ = NQC / 2;               // QK^T MFMAs per panel
  static constexpr int HD = NDB / 2;               // O^T blocks per panel
  // fragments in flight per wave (two waves per SIMD hide the rest; at D =
  // 1024 a second V fragment would not fit in the registers)
  static constexpr int LK = 2;
  static constexpr int LV = D_ == 1024 ? 1 : 2;
  // LDS map
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = TILE;
  static constexpr int OFF_RS = 2 * TILE;          // [qh][dest quarter][3 sources] x 1 KiB
  static constexpr int OFF_P = OFF_RS + 24 * 1024; // [qh][quarter] x 512 B of bf16 probabilities
  static constexpr int OFF_MX = OFF_P + 4 * 1024;  // [qh][quarter][32 rows] floats
  static constexpr int OFF_FL = OFF_MX + 1024;     // one flag word per wave
  static constexpr int LDS = OFF_FL + 64;
  static_assert(D_ % 256 == 0 && D_ >= 512 && D_ <= 1024, "D = 512, 768 or 1024");
  static_assert(PANEL % (1024 * NW) == 0, "a panel must split evenly over the waves");
  static_assert(HQ == 2 * GP && 2 * HD == 2 * GP, "one load after every other MFMA");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// s_waitcnt vmcnt(N), expcnt and lgkmcnt left at their maxima (gfx9 encoding:
// vmcnt bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// A copy of x the optimiser cannot see through (so what is computed from it
// is neither folded nor hoisted out of the loop).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// An empty use of x, held in vector registers, at this point of the program:
// keeps the MFMAs that produce it where they are written (the optimiser
// otherwise sinks them towards their first use, past the barriers that
// follow).  Accumulators stay in ordinary VGPRs in this kernel (two waves
// per SIMD share 512 registers; Q and O alone take 192 per wave at D = 1024).
__device__ __forceinline__ void pin_v(const f32x16& x) { asm volatile("" : : "v"(x)); }

template <int D>
__global__ __launch_bounds__(512, 1) void attn_fwd_splitd8_kernel(FwdParams p) {
  using C = Sd8Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave >> 2, dq = wave & 3;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- work decomposition ----------------------------------------------------
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
  // (uniform: kept in a scalar register)
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, p.scale * kLog2e)));

  int kv_end = kr.nkv;
  if (p.causal) kv_end = min(kr.nkv, min(q0 + C::BR, p.Nq) + kr.kv_off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;
  const int klim = p.causal ? min(kr.nkv - 1, qrow + kr.kv_off) : kr.nkv - 1;

  // ---- direct-to-LDS loads -----------------------------------------------------
  // Block j of this wave's share of a panel covers panel bytes
  // [(wave GP + j) KiB, +1 KiB); lane l writes 16 of them, so it fetches the
  // global 16-byte chunk that the swizzle places there.  Everything uniform
  // (the tile, the panel's D/2-column displacement and, where a block is one
  // row, the row) goes into the descriptor's base by scalar arithmetic; the
  // per-lane part is either one XOR of a lane base with a constant (D =
  // 1024: a block is one row, the K key is 4 (wave & 3) + j and the V key
  // 4 j) or one of GP offsets computed once (blocks spanning rows).
  constexpr bool kRowBlocks = C::PP == 1024;
  static_assert(!kRowBlocks || C::GP == 4, "one-row blocks: four per wave");
  uint32_t dko[kRowBlocks ? 1 : C::GP], dvo[kRowBlocks ? 1 : C::GP];
  if constexpr (kRowBlocks) {
    dko[0] = (uint32_t)((lane ^ ((wave * C::GP) & 15)) << 4);
    dvo[0] = (uint32_t)(lane << 4);
  } else {
#pragma unroll
    for (int j = 0; j < C::GP; ++j) {
      const int o = (wave * C::GP + j) * 1024 + lane * 16;
      const int row = o / C::PP;
      const int pc = (o - row * C::PP) >> 4;
      dko[j] = (uint32_t)(row * 2 * D + ((pc ^ k_swz<D>(row)) << 4));
      dvo[j] = (uint32_t)(row * 2 * D + ((pc ^ v_swz<D>(row)) << 4));
    }
  }
  // The descriptor of panel pn of K (is_v false) or V tile t, computed once
  // per group of loads: based `disp` bytes into the slab, record count cut by
  // as much (0 past the end), so the hardware range check still zero-fills
  // rows past the last key.  The loads run two tiles ahead of their use;
  // those past the last tile re-read the last one (their data is never used).
  auto desc = [&](bool is_v, int t, int pn) -> i32x4 {
    const i32x4 r = is_v ? rv : rk;
    const uint32_t disp = (uint32_t)min(t, n_kt - 1) * (uint32_t)C::TILE + (uint32_t)(pn * C::PP);
    const uint64_t a = ((uint64_t)(uint32_t)r.y << 32 | (uint32_t)r.x) + disp;
    const uint32_t n = (uint32_t)r.z;
    i32x4 rt;
    rt.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    rt.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    rt.z = __builtin_amdgcn_readfirstlane((int)(disp < n ? n - disp : 0u));
    rt.w = r.w;
    return rt;
  };
  // load j of a panel through descriptor rt
  const uint32_t row_base = (uint32_t)(wave * C::GP * 2 * D);  // one-row blocks: this wave's first row
  auto dma = [&](const i32x4& rt, bool is_v, int pn, int j) {
    uint32_t voff;
    if constexpr (kRowBlocks) {
      // (through opaque(): hoisted out of the loop, the eight XORs would
      // take eight registers the kernel does not have at D = 1024)
      voff = (is_v ? (opaque(dvo[0]) ^ (uint32_t)((j & 3) << 6)) : (opaque(dko[0]) ^ (uint32_t)(j << 4))) +
             (row_base + (uint32_t)(j * 2 * D));
    } else {
      voff = is_v ? dvo[j] : dko[j];
    }
    const uint32_t lds_panel = lds_base + (uint32_t)((is_v ? C::OFF_V : C::OFF_K) + pn * C::PANEL);
    dma_block_at<C::GP>(rt, lds_panel, voff, wave, j);
  };
  // all GP loads of one panel, back to back
  auto dma_panel = [&](bool is_v, int t, int pn) {
    const i32x4 rt = desc(is_v, t, pn);
    static_for<0, C::GP>([&](auto j) { dma(rt, is_v, pn, j); });
  };

  // ---- per-lane LDS fragment addresses --------------------------------------
  // K fragment cc (chunk 4cc + dq, lane half h: 16-byte chunk 8cc + 2dq + h
  // of the row) lies in panel cc / HQ; the swizzle XORs the low four bits of
  // the chunk index, so two bases (cc even, odd) plus immediates cover all.
  const int kx = k_swz<D>(l32);
  const uint32_t kb0 = (uint32_t)(l32 * C::PP + (((2 * dq + h) ^ kx) << 4));
  // (the odd base, chunk 8 + 2dq + h, is kb0 ^ 128: formed at each use, one
  // register fewer at D = 1024)
  auto kfrag = [&](int cc) -> u32x4 {
    const int pn = cc / C::HQ, c2 = cc - pn * C::HQ;
    const uint32_t base = (c2 & 1) ? (opaque(kb0) ^ 128u) : kb0;
    return lds_load16(lds, base + (uint32_t)(C::OFF_K + pn * C::PANEL + (c2 >> 1) * 256));
  };
  // V fragment (transposing read) of O^T block 4db + dq: rows 16 s16 + 4h +
  // r16/4 (+ 8), columns 128 db + 32 dq + 16 (g16 & 1) + 4 (r16 & 3) .. + 3,
  // i.e. 16-byte chunk 16 db + vlow of the row.
  const int g16 = lane >> 4, r16 = lane & 15;
  const int vrow0 = 4 * h + (r16 >> 2);
  const int vlow = 4 * dq + 2 * (g16 & 1) + ((r16 & 3) >> 1);
  // (opaque: the optimiser would otherwise fold the V area's offset into each
  // fragment's constant, overflow the 16-bit LDS immediate and hold one
  // address register per fragment)
  const uint32_t vb =
      opaque((uint32_t)(C::OFF_V + vrow0 * C::PP + ((vlow ^ v_swz<D>(vrow0)) << 4) + ((r16 & 1) << 3)));
  auto vfrag = [&](int f) -> u32x4 {  // f = s16 * NDB + db
    const int s16 = f / C::NDB, db = f % C::NDB;
    const int pn = db / C::HD, d2 = db - pn * C::HD;
    const uint32_t a0 = vb + (uint32_t)(pn * C::PANEL + d2 * 256 + s16 * 16 * C::PP);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + a0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + a0 + 8 * C::PP));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };
  // exchange slots: partial S^T quarter j of source wave (qh, src) goes to
  // slot (qh, j, src - [src > j]); wave (qh, j) reads its three.
  char* const rs_in = lds + C::OFF_RS + (qh * 4 + dq) * 3 * 1024 + lane * 16;
  // (the write addresses and the row-maximum area's are formed at each use)
  const char* const p_half = lds + C::OFF_P + qh * 4 * 512 + lane * 8;
  auto p_mine = [&]() { return lds + opaque((uint32_t)(C::OFF_P + qh * 4 * 512 + lane * 8)) + dq * 512; };
  auto mx_at = [&](int quarter) {
    return (float*)(lds + C::OFF_MX + (qh * 4 + quarter) * 128) + (opaque((uint32_t)lane) & 31u);
  };

  if (n_kt > 0) {
    dma_panel(false, 0, 0);
    dma_panel(false, 0, 1);
  }
  // Q[qrow, 16 (4cc + dq) + 8h .. + 7] (B operand of S^T = K Q^T)
  u32x4 qf[C::NQC];
  {
    const uint32_t row_off = (uint32_t)qrow * (uint32_t)(D * 2) + (uint32_t)(dq * 32 + h * 16);
#pragma unroll
    for (int cc = 0; cc < C::NQC; ++cc) qf[cc] = buf_load16(rq, row_off + (uint32_t)(cc * 128));
  }
  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_q = 0.0f;

  // S^T += K Q^T over the MFMAs [C0, C0 + HQ) (one panel), with load j of
  // `load` after MFMA 2j + 1 and `step(i)` (vector work) after MFMA i.
  auto qk_panel = [&](f32x16& s, auto c0c, auto&& load, auto&& step) {
    constexpr int C0 = decltype(c0c)::value;
    u32x4 kf[C::LK];
#pragma unroll
    for (int i = 0; i < C::LK; ++i) kf[i] = kfrag(C0 + i);
    static_for<0, C::HQ>([&](auto ic) {
      constexpr int i = ic;
      const u32x4 cur = kf[i % C::LK];
      if constexpr (i + C::LK < C::HQ) kf[i % C::LK] = kfrag(C0 + i + C::LK);
      __builtin_amdgcn_sched_barrier(0);
      s = mfma_bf16(cur, qf[C0 + i], s);
      if constexpr (i & 1) load(std::integral_constant<int, i / 2>{});
      step(ic);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // O^T += V^T P^T over the blocks of panel PN, with load j of `load` after
  // MFMA 2j + 1 and `step(i)` after MFMA i.
  u32x4 pf[2];
  auto pv_panel = [&](auto pnc, auto&& load, auto&& step) {
    constexpr int PN = decltype(pnc)::value;
    constexpr int NF = 2 * C::HD;
    auto fidx = [](int i) { return (i / C::HD) * C::NDB + PN * C::HD + i % C::HD; };
    u32x4 vf[C::LV];
#pragma unroll
    for (int i = 0; i < C::LV; ++i) vf[i] = vfrag(fidx(i));
    static_for<0, NF>([&](auto ic) {
      constexpr int i = ic;
      constexpr int s16 = i / C::HD, db = PN * C::HD + i % C::HD;
      const u32x4 cur = vf[i % C::LV];
      if constexpr (i + C::LV < NF) vf[i % C::LV] = vfrag(fidx(i + C::LV));
      __builtin_amdgcn_sched_barrier(0);
      acc[db] = mfma_bf16(cur, pf[s16], acc[db]);
      if constexpr (i & 1) load(std::integral_constant<int, i / 2>{});
      step(ic);
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int db = PN * C::HD; db < (PN + 1) * C::HD; ++db) pin_v(acc[db]);
  };
  auto no_step = [](auto) {};

  // partial S^T of the tile being contracted, and this wave's own key
  // quarter of it (kept in registers, the other three go through LDS);
  // gather() sums the quarter once every wave's partials are visible
  f32x16 s = f32x16{};
  f32x4 own = f32x4{};
  f32x4 xq = f32x4{};  // the summed scores of this wave's key quarter
  auto scatter = [&]() {
    static_for<0, 4>([&](auto jc) {
      constexpr int j = jc;
      const f32x4 q4 = __builtin_shufflevector(s, s, 4 * j, 4 * j + 1, 4 * j + 2, 4 * j + 3);
      if (j == dq) {
        own = q4;
      } else {
        const int k = dq - (dq > j ? 1 : 0);
        *reinterpret_cast<f32x4*>(lds + C::OFF_RS + ((qh * 4 + j) * 3 + k) * 1024 + lane * 16) = q4;
      }
    });
  };
  auto gather = [&]() {
    const f32x4 a = *reinterpret_cast<const f32x4*>(rs_in);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(rs_in + 1024);
    const f32x4 b2 = *reinterpret_cast<const f32x4*>(rs_in + 2048);
    xq = ((own + a) + b1) + b2;
  };

  if (n_kt > 0) {
    wait_vmem_all();  // Q and K(0)
    __syncthreads();
    // the contraction of tile 0 (no softmax yet to overlap)
    qk_panel(s, std::integral_constant<int, 0>{}, [](auto) {}, no_step);
    __syncthreads();  // K(0) panel 0 read by every wave
    const i32x4 rk1 = desc(false, 1, 0);
    qk_panel(s, std::integral_constant<int, C::HQ>{}, [&](auto j) { dma(rk1, false, 0, j); }, no_step);
    scatter();
    __syncthreads();  // K(0) panel 1 read by every wave, partial sums visible
    gather();
    dma_panel(false, 1, 1);
    dma_panel(true, 0, 0);
  }

  for (int kt = 0; kt < n_kt; ++kt) {
    const bool has_next = kt + 1 < n_kt;
    // ==== phase A: QK^T of tile kt+1, panel 0; softmax of tile kt ==========
    // (K(kt+1) panel 0 resident and the partial sums of tile kt written)
    wait_vmem<2 * C::GP>();
    __syncthreads();
    float t[4], e[4];
    float lsum = 0.0f;
    bool big = false;
    const float mneg0 = m_run == -INFINITY ? 0.0f : -m_run;
    const int key0 = kt * C::BC + 8 * dq + 4 * h;
    const bool edge = (kt * C::BC + C::BC > kr.nkv) || (p.causal && kt * C::BC + C::BC - 1 > q0w + kr.kv_off);
    auto softmax_step = [&](auto ic) {
      constexpr int i = ic;
      if constexpr (i == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = xq[r] * c;
        if (edge) {
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] = key0 + r <= klim ? t[r] : -INFINITY;
        }
      } else if constexpr (i == 2) {
        const float thr = m_run + kTau;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          big |= t[r] > thr;
          e[r] = exp2_fast(t[r] + mneg0);
        }
      } else if constexpr (i == 3) {
        *reinterpret_cast<u32x2*>(p_mine()) = u32x2{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
        const int flag = __builtin_amdgcn_ballot_w64(big) != 0 ? 1 : 0;
        if (lane == 0) *reinterpret_cast<int*>(lds + C::OFF_FL + wave * 4) = flag;
        lsum = (e[0] + e[1]) + (e[2] + e[3]);
      }
    };
    s = f32x16{};
    const i32x4 rA = desc(true, kt, 1);
    if (has_next) {
      qk_panel(s, std::integral_constant<int, 0>{}, [&](auto j) { dma(rA, true, 1, j); }, softmax_step);
      pin_v(s);
    } else {
      static_for<0, C::GP>([&](auto j) { dma(rA, true, 1, j); });
      static_for<0, C::HQ>(softmax_step);
    }

    // ==== phase B: QK^T of tile kt+1, panel 1; agree on the rescale ==========
    wait_vmem<2 * C::GP>();
    __syncthreads();
    {
      const u32x4 f0 = *reinterpret_cast<const u32x4*>(lds + C::OFF_FL);
      const u32x4 f1 = *reinterpret_cast<const u32x4*>(lds + C::OFF_FL + 16);
      const uint32_t any = (f0.x | f0.y | f0.z | f0.w) | (f1.x | f1.y | f1.z | f1.w);
      if (__builtin_amdgcn_readfirstlane(any) != 0) {
        // some score of some row exceeds its running maximum by more than
        // 2^kTau: the tile's maximum of each row, from the four quarters
        float mx = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
        mx = max_halves(mx);
        if (h == 0) *mx_at(dq) = mx;
        __syncthreads();
        const float* const mx_half = mx_at(0);
        const float mt = fmaxf(fmaxf(mx_half[0], mx_half[32]), fmaxf(mx_half[64], mx_half[96]));
        const float m_new = fmaxf(m_run, mt);
        // rows that have seen no visible key keep m = -inf; exp2 of
        // (-inf) - 0 is 0 there, never (-inf) - (-inf)
        const float alpha = exp2_fast(m_run - (m_new == -INFINITY ? 0.0f : m_new));
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) acc[db] *= alpha;
        l_q *= alpha;
        m_run = m_new;
        const float mneg = m_run == -INFINITY ? 0.0f : -m_run;
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = exp2_fast(t[r] + mneg);
        *reinterpret_cast<u32x2*>(p_mine()) = u32x2{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
        lsum = (e[0] + e[1]) + (e[2] + e[3]);
        __syncthreads();
      }
    }
    l_q += lsum;
    const i32x4 rB = desc(false, kt + 2, 0);
    if (has_next) {
      qk_panel(s, std::integral_constant<int, C::HQ>{}, [&](auto j) { dma(rB, false, 0, j); }, no_step);
      pin_v(s);
    } else {
      static_for<0, C::GP>([&](auto j) { dma(rB, false, 0, j); });
    }

    // ==== phase C: P V of tile kt, panel 0; scatter tile kt+1's partial sums ==
    wait_vmem<2 * C::GP>();
    __syncthreads();
    {
      // P^T of tile kt, 16 keys per MFMA: quarters (0, 1) and (2, 3)
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(p_half);
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(p_half + 512);
      const u32x2 a2 = *reinterpret_cast<const u32x2*>(p_half + 1024);
      const u32x2 a3 = *reinterpret_cast<const u32x2*>(p_half + 1536);
      pf[0] = u32x4{a0.x, a0.y, a1.x, a1.y};
      pf[1] = u32x4{a2.x, a2.y, a3.x, a3.y};
    }
    const i32x4 rC = desc(false, kt + 2, 1);
    pv_panel(std::integral_constant<int, 0>{}, [&](auto j) { dma(rC, false, 1, j); }, [&](auto ic) {
      if constexpr (decltype(ic)::value == 0) {
        if (has_next) scatter();
      }
    });

    // ==== phase D: P V of tile kt, panel 1 ======================================
    wait_vmem<2 * C::GP>();
    __syncthreads();
    const i32x4 rD = desc(true, kt + 1, 0);
    pv_panel(std::integral_constant<int, 1>{}, [&](auto j) { dma(rD, true, 0, j); }, [&](auto ic) {
      // tile kt+1's partial sums (scattered in phase C) are visible now
      if constexpr (decltype(ic)::value == 0) {
        if (has_next) gather();
      }
    });
  }
  // the loads issued past the last tile must land before the work-group's
  // LDS is released
  wait_vmem_all();

  // ---- epilogue: l summed over the four key quarters, then O / l and LSE --
  const float lh = sum_halves(l_q);
  if (h == 0) *mx_at(dq) = lh;
  __syncthreads();
  const float* const mx_half = mx_at(0);
  const float l_tot = ((mx_half[0] + mx_half[32]) + mx_half[64]) + mx_half[96];
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < p.Nq) {
    const int64_t orow = split * p.o_split_stride + q_slab + (int64_t)qrow * D + dq * 32;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 128 + 8 * g + 4 * h;
        store_o4(p.o, p.o_f32, orow + d, acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv,
                 acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
      }
    }
    if (p.lse != nullptr && dq == 0 && h == 0)
      p.lse[split * p.lse_split_stride + ((int64_t)b * p.Hq + hq) * p.Nq + qrow] =
          l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_splitd8(const FwdParams& p0, hipStream_t stream) {
  using C = Sd8Cfg<D>;
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + C::BR - 1) / C::BR;
  const int64_t total = (int64_t)p.n_splits * p.B * p.Hq * p.n_qtiles;
  if (total <= 0 || total >= (int64_t)1 << 31) return hipErrorInvalidValue;
  p.total_wg = (int)total;
  hipLaunchKernelGGL((attn_fwd_splitd8_kernel<D>), dim3(p.total_wg), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// D = 1024 only: at D = 768 the four-wave kernel is as fast or faster (827
// against 812 TFLOP/s on B=1, H=8, N=4096), at D = 512 the wide-head kernel
// (1132 against 658).
LaunchFn splitd8_launcher(int elt, int D) {
  if (elt != ELT_BF16) return nullptr;
  return D == 1024 ? &launch_splitd8<1024> : nullptr;
}

}  // namespace attn
