// attn_bwd.hip -- exact attention backward on gfx950 (bf16, D = 64 and 128,
// and every multiple of 64 from 192 to 512).
//
// FlashAttention summary page, method paragraph: the backward pass recomputes
// S = Q K^T instead of storing it; FlashAttention v1/v2/v3/v4 blog post,
// section "FA1 — el cambio de orden de las operaciones": only the softmax
// statistics are kept, and S is recomputed block by block from Q, K and
// them.  With the natural-log LSE of the forward pass, P = exp(scale S - LSE)
// needs no running max, and the gradients of the forward definition are
//   dV = P^T dO,  dP = dO V^T,  delta_i = dO_i . O_i (= sum_j P_ij dP_ij),
//   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,
// with dK and dV of a KV head summed over the query heads of its group.
//
// Three launches on one stream:
//   * prep: delta_i = dO_i . O_i in float32 and lse2_i = LSE_i log2(e)
//     (+inf for a row that saw no key, so that its P is 0), into a
//     caller-owned workspace;
//   * dK/dV: the keys of a (batch, KV head) in blocks of 32 per wave, held in
//     registers with the wave's dK^T and dV^T accumulators; Q and dO tiles of
//     every query head of the group stream through LDS.  S = Q K^T and dP =
//     dO V^T put one key per lane (column) and 16 query rows per lane in the
//     accumulator registers, which rounded to bf16 are the B operands of
//     dV^T += dO^T P and dK^T += Q^T dS as they stand; the A operands dO^T
//     and Q^T come from the transposing LDS read.  No atomics: each key's
//     gradients are owned by one wave.
//   * dQ: the forward pass's layout, query rows in registers (one query per
//     lane), K and V tiles in LDS; S^T = K Q^T, dP^T = V dO^T, then
//     dQ^T += K^T dS^T with K^T from the transposing read.
// S and dP are recomputed in both the dK/dV and the dQ launch (seven matrix
// products where five would do with atomic dQ accumulation): the results
// are deterministic.
//
// D = 64 and 128: one wave holds both K and V of its keys (dK/dV, 128 keys
// and one wave per SIMD per work-group, 64-row Q/dO tiles) or both Q and dO
// of its rows (dQ, 128 rows, two waves per SIMD, 64-key K/V tiles).  D = 192
// to 512: those registers no longer fit, and the work of each block is
// split between the two waves of a pair (the split kernels below).
//
// Q/dO and K/V tiles stream into LDS with direct-to-LDS buffer loads, two
// slots, one barrier per tile (the next tile's loads are issued right after
// it).  Their rows are read both as row fragments (16 rows of one 16-byte
// chunk per LDS phase) and through ds_read_b64_tr_b16 (4 rows x 4 chunks per
// phase); the XOR swizzle rt_swz keeps both conflict-free.
#include "attn_common.h"
#include "attn_dma.h"
#include "attn_bwd.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Chunk swizzle for rows read both ways.  D = 128 (16 chunks): row reads
// put rows 0..15 in a phase, and 4 (row & 3) + ((row >> 2) & 3) is a
// permutation of 0..15 over them; transposing reads put rows 4g..4g+3 and
// chunks 4c..4c+3 in a phase, where the term 4 (row & 3) sends each row to
// its own group of four chunks.  D = 64 (8 chunks, two rows per 256 bytes):
// m = (row >> 1) & 7 separates the rows of one parity; m ^ 4 (m & 1) gives
// rows 4g and 4g + 2 different halves of the 8 chunks.
template <int D>
__device__ __forceinline__ int rt_swz(int row) {
  if constexpr (D % 128 == 0) {
    return 4 * (row & 3) + ((row >> 2) & 3);
  } else {
    const int m = (row >> 1) & 7;
    return m ^ ((m & 1) << 2);
  }
}

// Keep an MFMA accumulator in accumulation registers at this point (an
// empty asm that may modify it there): with both dK^T/dV^T and the S/dP
// accumulators live, the allocator otherwise parks values in AGPRs and
// shuttles them back and forth every tile.
__device__ __forceinline__ void hold_acc(f32x16& x) { asm volatile("" : "+a"(x)); }
// The same for an operand fragment that stays live for the whole kernel
// (the MFMA reads its A/B operands from accumulation registers as well).
__device__ __forceinline__ void hold_frag(u32x4& x) { asm volatile("" : "+a"(x)); }

// An empty asm that takes x and gives it back in the same vector register:
// the computation of x cannot be moved past it.
__device__ __forceinline__ void pin_u(uint32_t& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// ---- prep: delta = rowsum(dO * O), lse2 = LSE log2(e) ---------------------------------

// lanes per row of the prep kernel: 16 bytes each, rounded up to a power of
// two so that the shuffle reduction stays within a row
template <int D>
constexpr int prep_lanes() {
  int n = 1;
  while (n < D / 8) n *= 2;
  return n;
}

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdParams p) {
  constexpr int LPR = prep_lanes<D>();
  constexpr int RPB = 256 / LPR;   // rows per work-group
  const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows && sub < D / 8) {
    const u32x4 a = *reinterpret_cast<const u32x4*>((const __bf16*)p.o + row * D + sub * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>((const __bf16*)p.dout + row * D + sub * 8);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += bf_lo(aw[j]) * bf_lo(gw[j]) + bf_hi(aw[j]) * bf_hi(gw[j]);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 64);
  if (sub == 0 && row < rows) {
    p.delta[row] = acc;
    const float l = p.lse[row];
    p.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ---- dK, dV ---------------------------------------------------------------------------

template <int D>
struct KVCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32 * NW;             // keys per work-group
  static constexpr int BQ = 64;                  // query rows per LDS tile
  static constexpr int RP = 2 * D;               // bf16 row pitch (bytes)
  static constexpr int NC = D / 16;              // 16-wide d chunks (S, dP contraction)
  static constexpr int NDB = D / 32;             // 32-row blocks of dK^T, dV^T
  static constexpr int TILE = BQ * RP;           // bytes of one Q or dO tile
  static constexpr int DMA = TILE / 1024 / NW;   // direct-to-LDS loads per wave per tile
  static constexpr int SLOT = 2 * TILE + 2 * BQ * 4;  // Q, dO, lse2, delta
  static constexpr int LDS = 2 * SLOT;           // two slots
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(2 * BQ <= NT, "one thread per lse2 / delta value");
};

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  using C = KVCfg<D>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int g16 = lane >> 4, r16 = lane & 15;

  // work decomposition: the key tiles of one (batch, KV head) are
  // neighbours, so they run together on one XCD and share its Q/dO in L2
  // (causal, paired: key tiles i and n-1-i, the heavier first)
  const int n_kt = (p.Nkv + C::BK - 1) / C::BK;
  const int nslot = p.pair_kv ? (n_kt + 1) / 2 : n_kt;
  const int wg = xcd_remap(blockIdx.x, nslot * p.B * p.Hkv);
  const int slot_k = wg % nslot;
  const int bh = wg / nslot;
  const int hk = bh % p.Hkv;
  const int b = bh / p.Hkv;
  const int njobs = (p.pair_kv && 2 * slot_k + 1 != n_kt) ? 2 : 1;
  for (int job = 0; job < njobs; ++job) {
  if (job > 0) __syncthreads();  // every wave is done with the LDS of the first tile
  const int kt = job == 0 ? slot_k : n_kt - 1 - slot_k;
  const int k0 = kt * C::BK;
  const int k0w = k0 + 32 * wave;
  const int key = k0w + l32;

  // this wave's K and V rows in B-operand layout (d chunk 2c + h)
  const int64_t kv_slab = ((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const __bf16*)p.k + kv_slab, (uint32_t)(p.Nkv * C::RP));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const __bf16*)p.v + kv_slab, (uint32_t)(p.Nkv * C::RP));
  u32x4 kreg[C::NC], vreg[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    kreg[c] = buf_load16(rk, (uint32_t)(key * C::RP + (2 * c + h) * 16));
    vreg[c] = buf_load16(rv, (uint32_t)(key * C::RP + (2 * c + h) * 16));
    hold_frag(kreg[c]);
    hold_frag(vreg[c]);
  }

  f32x16 adv[C::NDB], adk[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    adv[db] = f32x16{};
    adk[db] = f32x16{};
  }

  // per-lane LDS offsets: row fragments (row l32, chunk 2c + h) and
  // transposing reads (rows 4h + r16/4 and +8, chunk 4db + ...); a block or
  // row offset that is a multiple of 16 rows leaves the swizzle unchanged
  uint32_t rf[C::NC], tl[C::NDB], th[C::NDB];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) rf[c] = (uint32_t)(l32 * C::RP + (((2 * c + h) ^ rt_swz<D>(l32)) << 4));
  {
    const int rlo = 4 * h + (r16 >> 2), rhi = rlo + 8;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int chunk = db * 4 + 2 * (g16 & 1) + ((r16 & 3) >> 1);
      tl[db] = (uint32_t)(rlo * C::RP + ((chunk ^ rt_swz<D>(rlo)) << 4) + ((r16 & 1) << 3));
      th[db] = (uint32_t)(rhi * C::RP + ((chunk ^ rt_swz<D>(rhi)) << 4) + ((r16 & 1) << 3));
    }
  }
  auto trf = [&](const char* tile, int r0, int db) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + r0 * C::RP + tl[db]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + r0 * C::RP + th[db]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };

  // query tiles: every head of the group, from the first tile with a row
  // that sees key k0
  const int kv_off = p.Nkv - p.Nq;
  const int n_qt = (p.Nq + C::BQ - 1) / C::BQ;
  const int qt0 = p.causal ? min(max(0, k0 - kv_off) / C::BQ, n_qt) : 0;
  const int nq = n_qt - qt0;
  const int T = p.group * nq;
  const float c = p.scale * kLog2e;

  // tile t: Q and dO rows by direct-to-LDS loads, lse2 / delta through
  // registers (loaded at the top of the iteration before, stored at its end)
  uint32_t voff[C::DMA];
  dma_offsets_rows<C::DMA, C::RP>(voff, wave, lane, [](int row) { return rt_swz<D>(row); });
  auto q_row0 = [&](int t) { return (int64_t)b * p.Hq + hk * p.group + t / nq; };
  auto issue = [&](int t, int slot) {
    const int q0 = (qt0 + t % nq) * C::BQ;
    const int64_t slab = q_row0(t) * (int64_t)p.Nq * D;
    const uint32_t dst = lds_base + (uint32_t)(slot * C::SLOT);
    const i32x4 rq = sgpr_rsrc((const __bf16*)p.q + slab, (uint32_t)(p.Nq * C::RP));
    const i32x4 ro = sgpr_rsrc((const __bf16*)p.dout + slab, (uint32_t)(p.Nq * C::RP));
    dma_blocks<C::DMA>(rsrc_at(rq, (uint32_t)(q0 * C::RP)), dst, voff, wave);
    dma_blocks<C::DMA>(rsrc_at(ro, (uint32_t)(q0 * C::RP)), dst + C::TILE, voff, wave);
  };
  float st_l = 0.0f;
  auto load_ld = [&](int t) {
    if (tid < 2 * C::BQ) {
      const int r = (qt0 + t % nq) * C::BQ + (tid % C::BQ);
      const int64_t row = q_row0(t) * (int64_t)p.Nq + r;
      const bool live = r < p.Nq;
      st_l = tid < C::BQ ? (live ? p.lse2[row] : INFINITY) : (live ? p.delta[row] : 0.0f);
    }
  };
  auto store_ld = [&](int slot) {
    if (tid < 2 * C::BQ) reinterpret_cast<float*>(lds + slot * C::SLOT + 2 * C::TILE)[tid] = st_l;
  };

  if (T > 0) {
    issue(0, 0);
    load_ld(0);
    store_ld(0);
  }
  for (int t = 0; t < T; ++t) {
    const int slot = t & 1;
    const int q0 = (qt0 + t % nq) * C::BQ;
    wait_vmem_all();
    __syncthreads();  // tile t resident; the other slot (tile t-1) is free
    if (t + 1 < T) {
      issue(t + 1, slot ^ 1);
      load_ld(t + 1);
    }
    const char* const tQ = lds + slot * C::SLOT;
    const char* const tO = tQ + C::TILE;
    const float* const tL = reinterpret_cast<const float*>(tQ + 2 * C::TILE);
    const float* const tD = tL + C::BQ;

    // A software pipeline over the tile's two 32-row blocks, in steps of
    // two MFMAs, so that one wave keeps the matrix pipe fed by itself:
    //   A: S(0), dP(0)                      B: S(1), dP(1) + softmax of block 0
    //   C: dV^T, dK^T += ... (0) + softmax of block 1      D: dV^T, dK^T += ... (1)
    // LDS fragments are read W steps (row reads) or W2 steps (transposing
    // reads) ahead, fragment g of a phase pair's sequence in slot g % W; scheduling fences keep the steps in order (otherwise
    // the compiler sinks every read to just before its MFMA and the wave
    // waits out each read's latency).  Both blocks are computed even when
    // one is entirely masked (only on a causal tile crossing the diagonal):
    // branches around the products cost accumulator copies.
    constexpr int W = 3, W2 = 2, NS = 2 * C::NDB;  // NS: steps of phase C or D
    constexpr int EB = 16 / C::NC, EC = 16 / NS;   // softmax elements per step in B, C
    f32x16 s0 = f32x16{}, dp0 = f32x16{}, s1 = f32x16{}, dp1 = f32x16{};
    u32x4 fq[W], fo[W];
    u32x4 tq[W2], to[W2];
    u32x4 pf[2][2], df[2][2];
    float L[16], Dl[16];  // lse2 and delta of the block whose softmax runs next
    auto rowA = [&](const char* tile, int qb, int cc) { return lds_load16(tile, rf[cc] + qb * 32 * C::RP); };
    // step j of phase C/D: (kc, db) = (j / NDB, j % NDB)
    auto tr_load = [&](int qb, int j, int w) {
      const int r0 = 32 * qb + 16 * (j / C::NDB);
      to[w] = trf(tO, r0, j % C::NDB);
      tq[w] = trf(tQ, r0, j % C::NDB);
    };
    // lse2 and delta of block qb's 16 rows per lane.  The causal mask goes
    // into lse2: a row that must not see this lane's key gets +inf, so its P
    // is exp2(-inf) = 0; only blocks that cross the wave's keys pay for it.
    auto load_ld_block = [&](int qb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(tL + 32 * qb + 8 * j + 4 * h);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(tD + 32 * qb + 8 * j + 4 * h);
        L[4 * j + 0] = l4.x; L[4 * j + 1] = l4.y; L[4 * j + 2] = l4.z; L[4 * j + 3] = l4.w;
        Dl[4 * j + 0] = d4.x; Dl[4 * j + 1] = d4.y; Dl[4 * j + 2] = d4.z; Dl[4 * j + 3] = d4.w;
      }
      const int r0 = q0 + 32 * qb;
      if (p.causal && r0 + kv_off < k0w + 31) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (key > r0 + 8 * (rr / 4) + 4 * h + (rr % 4) + kv_off) L[rr] = INFINITY;
      }
    };
    // softmax and dS of elements r .. r+1 (a packed pair) of block qb
    auto soft2 = [&](int qb, int r, const f32x16& sv, const f32x16& dv) {
      float e[2], d[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rr = r + i;
        e[i] = exp2_fast(__builtin_fmaf(sv[rr], c, -L[rr]));
        d[i] = e[i] * (dv[rr] - Dl[rr]);
      }
      uint32_t pe = pack_bf16x2(e[0], e[1]), pd = pack_bf16x2(d[0], d[1]);
      // kept in this step: used only by the next phase's MFMAs, they would
      // otherwise be moved past all of this phase's
      pin_u(pe);
      pin_u(pd);
      const int kc = r / 8, comp = (r % 8) / 2;
      if (comp == 0) { pf[qb][kc].x = pe; df[qb][kc].x = pd; }
      else if (comp == 1) { pf[qb][kc].y = pe; df[qb][kc].y = pd; }
      else if (comp == 2) { pf[qb][kc].z = pe; df[qb][kc].z = pd; }
      else { pf[qb][kc].w = pe; df[qb][kc].w = pd; }
    };

    load_ld_block(0);
    static_for<0, W>([&](auto iI) {
      constexpr int i = decltype(iI)::value;
      fq[i] = rowA(tQ, 0, i);
      fo[i] = rowA(tO, 0, i);
    });
    // phase A
    static_for<0, C::NC>([&](auto cI) {
      constexpr int cc = decltype(cI)::value;
      __builtin_amdgcn_sched_barrier(0);
      s0 = mfma_bf16(fq[cc % W], kreg[cc], s0);
      dp0 = mfma_bf16(fo[cc % W], vreg[cc], dp0);
      hold_acc(s0);
      hold_acc(dp0);
      constexpr int n = cc + W;
      if constexpr (n < C::NC) {
        fq[cc % W] = rowA(tQ, 0, n);
        fo[cc % W] = rowA(tO, 0, n);
      } else {
        fq[cc % W] = rowA(tQ, 1, n - C::NC);
        fo[cc % W] = rowA(tO, 1, n - C::NC);
      }
    });
    // phase B
    static_for<0, C::NC>([&](auto cI) {
      constexpr int cc = decltype(cI)::value;
      __builtin_amdgcn_sched_barrier(0);
      // fragment g = NC + cc of the two blocks' sequence sits in slot g % W
      s1 = mfma_bf16(fq[(C::NC + cc) % W], kreg[cc], s1);
      dp1 = mfma_bf16(fo[(C::NC + cc) % W], vreg[cc], dp1);
      hold_acc(s1);
      hold_acc(dp1);
      constexpr int n = cc + W;
      if constexpr (n < C::NC) {
        fq[(C::NC + cc) % W] = rowA(tQ, 1, n);
        fo[(C::NC + cc) % W] = rowA(tO, 1, n);
      }
      if constexpr (cc >= C::NC - W2) tr_load(0, cc - (C::NC - W2), cc - (C::NC - W2));
#pragma unroll
      for (int e = 0; e < EB; e += 2) soft2(0, cc * EB + e, s0, dp0);
      if constexpr (cc == C::NC - 1) load_ld_block(1);  // block 0's values are used up
    });
    // phase C
    static_for<0, NS>([&](auto jI) {
      constexpr int j = decltype(jI)::value;
      __builtin_amdgcn_sched_barrier(0);
      constexpr int db = j % C::NDB, kc = j / C::NDB;
      adv[db] = mfma_bf16(to[j % W2], pf[0][kc], adv[db]);
      adk[db] = mfma_bf16(tq[j % W2], df[0][kc], adk[db]);
      hold_acc(adv[db]);
      hold_acc(adk[db]);
      constexpr int n = j + W2;
      if constexpr (n < NS) tr_load(0, n, j % W2);
      else tr_load(1, n - NS, j % W2);
#pragma unroll
      for (int e = 0; e < EC; e += 2) soft2(1, j * EC + e, s1, dp1);
    });
    // phase D
    static_for<0, NS>([&](auto jI) {
      constexpr int j = decltype(jI)::value;
      __builtin_amdgcn_sched_barrier(0);
      constexpr int db = j % C::NDB, kc = j / C::NDB;
      adv[db] = mfma_bf16(to[(NS + j) % W2], pf[1][kc], adv[db]);
      adk[db] = mfma_bf16(tq[(NS + j) % W2], df[1][kc], adk[db]);
      hold_acc(adv[db]);
      hold_acc(adk[db]);
      constexpr int n = j + W2;
      if constexpr (n < NS) tr_load(1, n, (NS + j) % W2);
    });
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < T) store_ld(slot ^ 1);
  }

  // ---- epilogue: lane = key, registers = d ----------------------------------------
  if (key < p.Nkv) {
    const int64_t row = kv_slab + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * h;
        store_o4(p.dv, false, row + d, adv[db][4 * g + 0], adv[db][4 * g + 1], adv[db][4 * g + 2],
                 adv[db][4 * g + 3]);
        store_o4(p.dk, false, row + d, adk[db][4 * g + 0] * p.scale, adk[db][4 * g + 1] * p.scale,
                 adk[db][4 * g + 2] * p.scale, adk[db][4 * g + 3] * p.scale);
      }
    }
  }
}  // job
}

// ---- dQ -------------------------------------------------------------------------------

template <int D>
struct QCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BR = 32 * NW;             // query rows per work-group
  static constexpr int BC = 64;                  // keys per LDS tile
  static constexpr int RP = 2 * D;
  static constexpr int NC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int TILE = BC * RP;
  static constexpr int DMA = TILE / 1024 / NW;
  static constexpr int SLOT = 2 * TILE;          // K, V
  static constexpr int LDS = 2 * SLOT;
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdParams p) {
  using C = QCfg<D>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int g16 = lane >> 4, r16 = lane & 15;

  const int n_qt = (p.Nq + C::BR - 1) / C::BR;
  const int wg = xcd_remap(blockIdx.x, n_qt * p.B * p.Hq);
  const int qt_raw = wg % n_qt;
  const int bh = wg / n_qt;
  const int hq = bh % p.Hq;
  const int b = bh / p.Hq;
  const int qt = p.causal ? n_qt - 1 - qt_raw : qt_raw;
  const int hk = hq / p.group;
  const int q0 = qt * C::BR;
  const int q0w = q0 + 32 * wave;
  const int qrow = q0w + l32;

  const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const __bf16*)p.q + q_slab * D, (uint32_t)(p.Nq * C::RP));
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((const __bf16*)p.dout + q_slab * D, (uint32_t)(p.Nq * C::RP));
  u32x4 qreg[C::NC], oreg[C::NC];
#pragma unroll
  for (int cc = 0; cc < C::NC; ++cc) {
    qreg[cc] = buf_load16(rq, (uint32_t)(qrow * C::RP + (2 * cc + h) * 16));
    oreg[cc] = buf_load16(ro, (uint32_t)(qrow * C::RP + (2 * cc + h) * 16));

  }
  const bool live = qrow < p.Nq;
  const float lq = live ? p.lse2[q_slab + qrow] : INFINITY;
  const float dq_row = live ? p.delta[q_slab + qrow] : 0.0f;

  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

  const int kv_off = p.Nkv - p.Nq;
  int kv_end = p.Nkv;
  if (p.causal) kv_end = min(p.Nkv, min(q0 + C::BR, p.Nq) + kv_off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;
  const int klim = p.causal ? min(p.Nkv - 1, qrow + kv_off) : p.Nkv - 1;  // last visible key
  const float c = p.scale * kLog2e;

  uint32_t rf[C::NC], tl[C::NDB], th[C::NDB];
#pragma unroll
  for (int cc = 0; cc < C::NC; ++cc) rf[cc] = (uint32_t)(l32 * C::RP + (((2 * cc + h) ^ rt_swz<D>(l32)) << 4));
  {
    const int rlo = 4 * h + (r16 >> 2), rhi = rlo + 8;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int chunk = db * 4 + 2 * (g16 & 1) + ((r16 & 3) >> 1);
      tl[db] = (uint32_t)(rlo * C::RP + ((chunk ^ rt_swz<D>(rlo)) << 4) + ((r16 & 1) << 3));
      th[db] = (uint32_t)(rhi * C::RP + ((chunk ^ rt_swz<D>(rhi)) << 4) + ((r16 & 1) << 3));
    }
  }

  const int64_t kv_slab = ((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv * D;
  const i32x4 rk = sgpr_rsrc((const __bf16*)p.k + kv_slab, (uint32_t)(p.Nkv * C::RP));
  const i32x4 rv = sgpr_rsrc((const __bf16*)p.v + kv_slab, (uint32_t)(p.Nkv * C::RP));
  uint32_t voff[C::DMA];
  dma_offsets_rows<C::DMA, C::RP>(voff, wave, lane, [](int row) { return rt_swz<D>(row); });
  auto issue = [&](int kt, int slot) {
    const uint32_t dst = lds_base + (uint32_t)(slot * C::SLOT);
    dma_blocks<C::DMA>(rsrc_at(rk, (uint32_t)(kt * C::TILE)), dst, voff, wave);
    dma_blocks<C::DMA>(rsrc_at(rv, (uint32_t)(kt * C::TILE)), dst + C::TILE, voff, wave);
  };

  if (n_kt > 0) issue(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int slot = kt & 1;
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < n_kt) issue(kt + 1, slot ^ 1);
    const int key0 = kt * C::BC;
    // wave-uniform: this wave's rows see none of the tile
    if (p.causal && key0 > q0w + 31 + kv_off) continue;
    const char* const tK = lds + slot * C::SLOT;
    const char* const tV = tK + C::TILE;
    const bool mask = key0 + C::BC > p.Nkv || (p.causal && key0 + C::BC - 1 > q0w + kv_off);

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int cc = 0; cc < C::NC; ++cc) {
        s = mfma_bf16(lds_load16(tK, rf[cc] + kb * 32 * C::RP), qreg[cc], s);
        dp = mfma_bf16(lds_load16(tV, rf[cc] + kb * 32 * C::RP), oreg[cc], dp);
      }
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) dsv[r] = exp2_fast(__builtin_fmaf(s[r], c, -lq)) * (dp[r] - dq_row);
      // keys past the end or after the row (tail and causal-diagonal tiles
      // only: the compare and select are skipped elsewhere)
      if (mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + 32 * kb + 8 * (r / 4) + 4 * h + (r % 4) > klim) dsv[r] = 0.0f;
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const u32x4 df = u32x4{pack_bf16x2(dsv[8 * kc + 0], dsv[8 * kc + 1]), pack_bf16x2(dsv[8 * kc + 2], dsv[8 * kc + 3]),
                               pack_bf16x2(dsv[8 * kc + 4], dsv[8 * kc + 5]), pack_bf16x2(dsv[8 * kc + 6], dsv[8 * kc + 7])};
        const int r0 = 32 * kb + 16 * kc;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tK + r0 * C::RP + tl[db]));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tK + r0 * C::RP + th[db]));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          acc[db] = mfma_bf16(u32x4{l2.x, l2.y, h2.x, h2.y}, df, acc[db]);
        }
      }
    }
  }

  if (live) {
    const int64_t row = (q_slab + qrow) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * h;
        store_o4(p.dq, false, row + d, acc[db][4 * g + 0] * p.scale, acc[db][4 * g + 1] * p.scale,
                 acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
      }
    }
  }
}

// ---- D = 192 .. 512: the work of one key (or query) block split between two waves ---
// At D = 512 one wave's registers hold either the K rows or the V rows of its
// 32 keys (128 registers each), and a dK^T or dV^T accumulator for the whole
// head dim takes all 256 accumulation registers; at D = 256 half of each,
// which leaves room to read LDS fragments well ahead of the products.  A
// work-group's four waves therefore form two pairs over the same 32 keys.
// The first wave of a pair holds K, computes S = Q K^T, P = exp2(c S - lse2)
// (masked) and dV^T += dO^T P; the second holds V, computes dP = dO V^T,
// takes P from its partner through LDS (float32, one barrier later), forms
// dS = P (dP - delta) and dK^T += Q^T dS.  Each wave does the same number of
// products per tile (two D-long contractions of a 32 x 32 block), and P is
// computed once.  Query tiles are 32 rows (Q and dO of one tile take 128 D
// bytes), two slots.

template <int D>
struct KVSplitCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32 * NW / 2;         // keys per work-group, 32 per pair
  static constexpr int BQ = 32;                  // query rows per LDS tile
  static constexpr int RP = 2 * D;
  static constexpr int NC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int TILE = BQ * RP;
  static constexpr int DMA = TILE / 1024 / NW;
  static constexpr int SLOT = 2 * TILE + 2 * BQ * 4;   // Q, dO, lse2, delta
  static constexpr int XCH = (NW / 2) * 64 * 16 * 4;   // P of each pair: 16 floats per lane
  static constexpr int LDS = 2 * SLOT + XCH;
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(2 * DMA <= NC, "a tile's loads fit between the first phase's products");
  static_assert(2 * BQ <= NT, "one thread per lse2 / delta value");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_split_kernel(BwdParams p) {
  using C = KVSplitCfg<D>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave & 1;   // 0: K, S, P, dV;  1: V, dP, dS, dK
  const int pair = wave >> 1;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int g16 = lane >> 4, r16 = lane & 15;

  const int n_kt = (p.Nkv + C::BK - 1) / C::BK;
  const int nslot = p.pair_kv ? (n_kt + 1) / 2 : n_kt;
  const int wg = xcd_remap(blockIdx.x, nslot * p.B * p.Hkv);
  const int slot_k = wg % nslot;
  const int bh = wg / nslot;
  const int hk = bh % p.Hkv;
  const int b = bh / p.Hkv;
  const int njobs = (p.pair_kv && 2 * slot_k + 1 != n_kt) ? 2 : 1;
  for (int job = 0; job < njobs; ++job) {
  if (job > 0) __syncthreads();
  const int kt = job == 0 ? slot_k : n_kt - 1 - slot_k;
  const int k0 = kt * C::BK;
  const int k0w = k0 + 32 * pair;
  const int key = k0w + l32;

  // this wave's K (role 0) or V (role 1) rows in B-operand layout
  const int64_t kv_slab = ((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv * D;
  const __amdgpu_buffer_rsrc_t rr =
      make_rsrc((const __bf16*)(role ? p.v : p.k) + kv_slab, (uint32_t)(p.Nkv * C::RP));
  u32x4 reg[C::NC];
#pragma unroll
  for (int cc = 0; cc < C::NC; ++cc) reg[cc] = buf_load16(rr, (uint32_t)(key * C::RP + (2 * cc + h) * 16));
  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    acc[db] = f32x16{};
    hold_acc(acc[db]);
  }

  // Per-lane LDS offsets.  The swizzle keys are below 16, so they change only
  // the low four bits of a chunk index: row fragment cc (chunk 2 cc + h) is
  // one of eight per-lane offsets plus 256 (cc / 8) bytes, and a transposed
  // read of block db (chunk 4 db + cpart) one of four plus 256 (db / 4), the
  // constants going into the instructions' offset fields.
  const int xr = rt_swz<D>(l32);
  const int rlo = 4 * h + (r16 >> 2), rhi = rlo + 8;
  const int xlo = rt_swz<D>(rlo), xhi = rt_swz<D>(rhi);
  const int cpart = 2 * (g16 & 1) + ((r16 & 3) >> 1);
  uint32_t ro[8], tlo[4], thi[4];
#pragma unroll
  for (int m = 0; m < 8; ++m) ro[m] = (uint32_t)(l32 * C::RP + (((2 * m + h) ^ xr) << 4));
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    tlo[m] = (uint32_t)(rlo * C::RP + ((r16 & 1) << 3) + (((4 * m + cpart) ^ xlo) << 4));
    thi[m] = (uint32_t)(rhi * C::RP + ((r16 & 1) << 3) + (((4 * m + cpart) ^ xhi) << 4));
  }
  auto rowfrag = [&](const char* tile, int cc) { return lds_load16(tile, ro[cc % 8] + 256 * (cc / 8)); };
  auto trfrag = [&](const char* tile, int r0, int db) {
    const uint32_t k = (uint32_t)(256 * (db / 4) + r0 * C::RP);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + tlo[db % 4] + k));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + thi[db % 4] + k));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };

  const int kv_off = p.Nkv - p.Nq;
  const int n_qt = (p.Nq + C::BQ - 1) / C::BQ;
  const int qt0 = p.causal ? min(max(0, k0 - kv_off) / C::BQ, n_qt) : 0;
  const int nq = n_qt - qt0;
  const int T = p.group * nq;
  const float c = p.scale * kLog2e;

  uint32_t voff[C::DMA];
  dma_offsets_rows<C::DMA, C::RP>(voff, wave, lane, [](int row) { return rt_swz<D>(row); });
  auto q_row0 = [&](int t) { return (int64_t)b * p.Hq + hk * p.group + t / nq; };
  // descriptor of tile t of Q (or dO)
  auto tile_rsrc = [&](int t, const void* base) {
    const int q0 = (qt0 + t % nq) * C::BQ;
    const int64_t slab = q_row0(t) * (int64_t)p.Nq * D;
    return rsrc_at(sgpr_rsrc((const __bf16*)base + slab, (uint32_t)(p.Nq * C::RP)), (uint32_t)(q0 * C::RP));
  };
  auto issue = [&](int t, int slot) {
    const uint32_t dst = lds_base + (uint32_t)(slot * C::SLOT);
    dma_blocks<C::DMA>(tile_rsrc(t, p.q), dst, voff, wave);
    dma_blocks<C::DMA>(tile_rsrc(t, p.dout), dst + C::TILE, voff, wave);
  };
  float st_l = 0.0f;
  auto load_ld = [&](int t) {
    if (tid < 2 * C::BQ) {
      const int r = (qt0 + t % nq) * C::BQ + (tid % C::BQ);
      const int64_t row = q_row0(t) * (int64_t)p.Nq + r;
      const bool live = r < p.Nq;
      st_l = tid < C::BQ ? (live ? p.lse2[row] : INFINITY) : (live ? p.delta[row] : 0.0f);
    }
  };
  auto store_ld = [&](int slot) {
    if (tid < 2 * C::BQ) reinterpret_cast<float*>(lds + slot * C::SLOT + 2 * C::TILE)[tid] = st_l;
  };
  // the pair's P: register r of lane l at float 4 (64 (r / 4) + l) + r % 4
  float* const xch = reinterpret_cast<float*>(lds + 2 * C::SLOT) + pair * (64 * 16);

  if (T > 0) {
    issue(0, 0);
    load_ld(0);
    store_ld(0);
  }
  for (int t = 0; t < T; ++t) {
    const int slot = t & 1;
    const int q0 = (qt0 + t % nq) * C::BQ;
    wait_vmem_all();
    __syncthreads();  // tile t resident; the other slot (tile t-1) and xch are free
    // tile t+1's loads go out one per product of the first phase below
    const bool more = t + 1 < T;
    const uint32_t ndst = lds_base + (uint32_t)((slot ^ 1) * C::SLOT);
    i32x4 nrq = {}, nro = {};
    if (more) {
      nrq = tile_rsrc(t + 1, p.q);
      nro = tile_rsrc(t + 1, p.dout);
      load_ld(t + 1);
    }
    const char* const tQ = lds + slot * C::SLOT;
    const char* const tO = tQ + C::TILE;
    const float* const tL = reinterpret_cast<const float*>(tQ + 2 * C::TILE);
    const float* const tD = tL + C::BQ;
    const char* const tR = role ? tO : tQ;   // row operand of S or dP
    const char* const tT = role ? tQ : tO;   // transposed operand of dK^T or dV^T

    // S (role 0) or dP (role 1): 32 query rows x the pair's 32 keys.  One
    // wave per SIMD has no other wave to hide LDS latency behind, so the
    // row fragments are read W products ahead and the transposed fragments
    // of the dV^T / dK^T products W2 ahead (fragment j in slot j % W);
    // scheduling fences keep the compiler from sinking each read to just
    // before its product.
    constexpr int W = 4, W2 = 4, NS = 2 * C::NDB;
    f32x16 x = f32x16{};
    u32x4 f[W], tf[W2];
    static_for<0, W>([&](auto iI) {
      constexpr int i = decltype(iI)::value;
      f[i] = rowfrag(tR, i);
    });
    static_for<0, C::NC>([&](auto cI) {
      constexpr int cc = decltype(cI)::value;
      __builtin_amdgcn_sched_barrier(0);
      x = mfma_bf16(f[cc % W], reg[cc], x);
      if constexpr (cc < 2 * C::DMA) {
        if (more) {
          if constexpr (cc % 2 == 0) dma_block_one<C::DMA>(nrq, ndst, voff, wave, cc / 2);
          else dma_block_one<C::DMA>(nro, ndst + C::TILE, voff, wave, cc / 2);
        }
      }
      if constexpr (cc + W < C::NC) f[cc % W] = rowfrag(tR, cc + W);
    });
    __builtin_amdgcn_sched_barrier(0);
    // step j of the second products: (kc, db) = (j / NDB, j % NDB); their
    // operands do not depend on P
    static_for<0, W2>([&](auto jI) {
      constexpr int j = decltype(jI)::value;
      tf[j] = trfrag(tT, 16 * (j / C::NDB), j % C::NDB);
    });
    float pv[16];  // P (role 0)
    if (role == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(tL + 8 * g + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[4 * g + i] = exp2_fast(__builtin_fmaf(x[4 * g + i], c, -l4[i]));
      }
      // rows before this lane's key (only tiles that cross the pair's keys)
      if (p.causal && q0 + kv_off < k0w + 31) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key > q0 + 8 * (r / 4) + 4 * h + (r % 4) + kv_off) pv[r] = 0.0f;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(xch + 4 * (64 * g + lane)) =
            f32x4{pv[4 * g], pv[4 * g + 1], pv[4 * g + 2], pv[4 * g + 3]};
    }
    __syncthreads();  // P of the pair visible to its second wave
    u32x4 fr[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v[4];
      if (role == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pv[4 * g + i];
      } else {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(xch + 4 * (64 * g + lane));
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(tD + 8 * g + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = p4[i] * (x[4 * g + i] - d4[i]);
      }
      const uint32_t w0 = pack_bf16x2(v[0], v[1]), w1 = pack_bf16x2(v[2], v[3]);
      if (g & 1) {
        fr[g >> 1].z = w0;
        fr[g >> 1].w = w1;
      } else {
        fr[g >> 1].x = w0;
        fr[g >> 1].y = w1;
      }
    }
    // dV^T += dO^T P (role 0), dK^T += Q^T dS (role 1)
    static_for<0, NS>([&](auto jI) {
      constexpr int j = decltype(jI)::value;
      constexpr int kc = j / C::NDB, db = j % C::NDB;
      __builtin_amdgcn_sched_barrier(0);
      acc[db] = mfma_bf16(tf[j % W2], fr[kc], acc[db]);
      hold_acc(acc[db]);
      if constexpr (j + W2 < NS) tf[j % W2] = trfrag(tT, 16 * ((j + W2) / C::NDB), (j + W2) % C::NDB);
    });
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < T) store_ld(slot ^ 1);
  }

  if (key < p.Nkv) {
    const int64_t row = kv_slab + (int64_t)key * D;
    void* const out = role ? p.dk : p.dv;
    const float f = role ? p.scale : 1.0f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * h;
        store_o4(out, false, row + d, acc[db][4 * g + 0] * f, acc[db][4 * g + 1] * f, acc[db][4 * g + 2] * f,
                 acc[db][4 * g + 3] * f);
      }
    }
  }
}  // job
}

// dQ at D = 192 .. 512: pairs of waves over the same 32 query rows.  The
// first wave holds the Q rows and computes S^T = K Q^T and P^T, the second
// holds the dO rows and computes dP^T = V dO^T; they swap the two through LDS
// (float32), both form dS^T = P^T (dP^T - delta) from the same values, and
// each accumulates one half of dQ^T += K^T dS^T (d below or above D / 2).
// Key tiles are 32 keys (K and V of one tile take 128 D bytes), two slots.

template <int D>
struct QSplitCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BR = 32 * NW / 2;         // query rows per work-group, 32 per pair
  static constexpr int BC = 32;                  // keys per LDS tile
  static constexpr int RP = 2 * D;
  static constexpr int NC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int HDB = NDB / 2;            // dQ^T blocks per wave
  static constexpr int TILE = BC * RP;
  static constexpr int DMA = TILE / 1024 / NW;
  static constexpr int SLOT = 2 * TILE;          // K, V
  static constexpr int XCH = NW * 64 * 16 * 4;   // each wave's S or dP block
  static constexpr int LDS = 2 * SLOT + XCH;
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(2 * DMA <= NC, "a tile's loads fit between the first phase's products");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_split_kernel(BwdParams p) {
  using C = QSplitCfg<D>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave & 1;   // 0: Q, S, P;  1: dO, dP
  const int pair = wave >> 1;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int g16 = lane >> 4, r16 = lane & 15;

  const int n_qt = (p.Nq + C::BR - 1) / C::BR;
  const int wg = xcd_remap(blockIdx.x, n_qt * p.B * p.Hq);
  const int qt_raw = wg % n_qt;
  const int bh = wg / n_qt;
  const int hq = bh % p.Hq;
  const int b = bh / p.Hq;
  const int qt = p.causal ? n_qt - 1 - qt_raw : qt_raw;
  const int hk = hq / p.group;
  const int q0 = qt * C::BR;
  const int q0w = q0 + 32 * pair;
  const int qrow = q0w + l32;

  const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq;
  const __amdgpu_buffer_rsrc_t rr =
      make_rsrc((const __bf16*)(role ? p.dout : p.q) + q_slab * D, (uint32_t)(p.Nq * C::RP));
  u32x4 reg[C::NC];
#pragma unroll
  for (int cc = 0; cc < C::NC; ++cc) reg[cc] = buf_load16(rr, (uint32_t)(qrow * C::RP + (2 * cc + h) * 16));
  const bool live = qrow < p.Nq;
  const float lq = live ? p.lse2[q_slab + qrow] : INFINITY;
  const float dq_row = live ? p.delta[q_slab + qrow] : 0.0f;

  f32x16 acc[C::HDB];
#pragma unroll
  for (int db = 0; db < C::HDB; ++db) {
    acc[db] = f32x16{};
    hold_acc(acc[db]);
  }

  const int kv_off = p.Nkv - p.Nq;
  int kv_end = p.Nkv;
  if (p.causal) kv_end = min(p.Nkv, min(q0 + C::BR, p.Nq) + kv_off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;
  const int klim = p.causal ? min(p.Nkv - 1, qrow + kv_off) : p.Nkv - 1;  // last visible key
  const float c = p.scale * kLog2e;

  // Per-lane LDS offsets.  The swizzle keys are below 16, so they change only
  // the low four bits of a chunk index: row fragment cc (chunk 2 cc + h) is
  // one of eight per-lane offsets plus 256 (cc / 8) bytes, and a transposed
  // read of block db (chunk 4 db + cpart) one of four plus 256 (db / 4), the
  // constants going into the instructions' offset fields.
  const int xr = rt_swz<D>(l32);
  const int rlo = 4 * h + (r16 >> 2), rhi = rlo + 8;
  const int xlo = rt_swz<D>(rlo), xhi = rt_swz<D>(rhi);
  const int cpart = 2 * (g16 & 1) + ((r16 & 3) >> 1);
  uint32_t ro[8], tlo[4], thi[4];
#pragma unroll
  for (int m = 0; m < 8; ++m) ro[m] = (uint32_t)(l32 * C::RP + (((2 * m + h) ^ xr) << 4));
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    tlo[m] = (uint32_t)(rlo * C::RP + ((r16 & 1) << 3) + (((4 * m + cpart) ^ xlo) << 4));
    thi[m] = (uint32_t)(rhi * C::RP + ((r16 & 1) << 3) + (((4 * m + cpart) ^ xhi) << 4));
  }
  auto rowfrag = [&](const char* tile, int cc) { return lds_load16(tile, ro[cc % 8] + 256 * (cc / 8)); };
  auto trfrag = [&](const char* tile, int r0, int db) {
    const uint32_t k = (uint32_t)(256 * (db / 4) + r0 * C::RP);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + tlo[db % 4] + k));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + thi[db % 4] + k));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
  };

  const int64_t kv_slab = ((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv * D;
  const i32x4 rk = sgpr_rsrc((const __bf16*)p.k + kv_slab, (uint32_t)(p.Nkv * C::RP));
  const i32x4 rv = sgpr_rsrc((const __bf16*)p.v + kv_slab, (uint32_t)(p.Nkv * C::RP));
  uint32_t voff[C::DMA];
  dma_offsets_rows<C::DMA, C::RP>(voff, wave, lane, [](int row) { return rt_swz<D>(row); });
  auto issue = [&](int kt, int slot) {
    const uint32_t dst = lds_base + (uint32_t)(slot * C::SLOT);
    dma_blocks<C::DMA>(rsrc_at(rk, (uint32_t)(kt * C::TILE)), dst, voff, wave);
    dma_blocks<C::DMA>(rsrc_at(rv, (uint32_t)(kt * C::TILE)), dst + C::TILE, voff, wave);
  };
  // each wave's block: register r of lane l at float 4 (64 (r / 4) + l) + r % 4
  float* const mine = reinterpret_cast<float*>(lds + 2 * C::SLOT) + wave * (64 * 16);
  const float* const other = reinterpret_cast<const float*>(lds + 2 * C::SLOT) + (wave ^ 1) * (64 * 16);

  if (n_kt > 0) issue(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int slot = kt & 1;
    wait_vmem_all();
    __syncthreads();  // tile kt resident; the other slot and the exchange are free
    const int key0 = kt * C::BC;
    // uniform over the pair: its rows see none of the tile (the barriers
    // below are still taken)
    const bool skip = p.causal && key0 > q0w + 31 + kv_off;
    // tile kt+1's loads: one per product of the first phase below (all at
    // once here when this wave skips the tile)
    const bool more = kt + 1 < n_kt;
    const uint32_t ndst = lds_base + (uint32_t)((slot ^ 1) * C::SLOT);
    const i32x4 nrk = rsrc_at(rk, (uint32_t)((kt + 1) * C::TILE));
    const i32x4 nrv = rsrc_at(rv, (uint32_t)((kt + 1) * C::TILE));
    if (more && skip) issue(kt + 1, slot ^ 1);
    const char* const tK = lds + slot * C::SLOT;
    const char* const tV = tK + C::TILE;
    const bool mask = key0 + C::BC > p.Nkv || (p.causal && key0 + C::BC - 1 > q0w + kv_off);

    // fragment reads run ahead of the products as in the dK/dV kernel
    constexpr int W = 4, W2 = 4, NS = 2 * C::HDB;
    f32x16 x = f32x16{};
    float xv[16];
    u32x4 tf[W2];
    if (!skip) {
      const char* const tR = role ? tV : tK;
      u32x4 f[W];
      static_for<0, W>([&](auto iI) {
        constexpr int i = decltype(iI)::value;
        f[i] = rowfrag(tR, i);
      });
      static_for<0, C::NC>([&](auto cI) {
        constexpr int cc = decltype(cI)::value;
        __builtin_amdgcn_sched_barrier(0);
        x = mfma_bf16(f[cc % W], reg[cc], x);
        if constexpr (cc < 2 * C::DMA) {
          if (more) {
            if constexpr (cc % 2 == 0) dma_block_one<C::DMA>(nrk, ndst, voff, wave, cc / 2);
            else dma_block_one<C::DMA>(nrv, ndst + C::TILE, voff, wave, cc / 2);
          }
        }
        if constexpr (cc + W < C::NC) f[cc % W] = rowfrag(tR, cc + W);
      });
      __builtin_amdgcn_sched_barrier(0);
      // step j of dQ^T += K^T dS^T: (kc, db) = (j / HDB, role HDB + j % HDB)
      static_for<0, W2>([&](auto jI) {
        constexpr int j = decltype(jI)::value;
        tf[j] = trfrag(tK, 16 * (j / C::HDB), role * C::HDB + j % C::HDB);
      });
      // role 0: P; role 1: dP as it stands
      if (role == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xv[r] = exp2_fast(__builtin_fmaf(x[r], c, -lq));
        // keys past the end or after the row (tail and diagonal tiles only)
        if (mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + 8 * (r / 4) + 4 * h + (r % 4) > klim) xv[r] = 0.0f;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) xv[r] = x[r];
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(mine + 4 * (64 * g + lane)) =
            f32x4{xv[4 * g], xv[4 * g + 1], xv[4 * g + 2], xv[4 * g + 3]};
    }
    __syncthreads();  // both blocks of each pair visible
    if (!skip) {
      u32x4 fr[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 y = *reinterpret_cast<const f32x4*>(other + 4 * (64 * g + lane));
        float v[4];
        if (role == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = xv[4 * g + i] * (y[i] - dq_row);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = y[i] * (xv[4 * g + i] - dq_row);
        }
        const uint32_t w0 = pack_bf16x2(v[0], v[1]), w1 = pack_bf16x2(v[2], v[3]);
        if (g & 1) {
          fr[g >> 1].z = w0;
          fr[g >> 1].w = w1;
        } else {
          fr[g >> 1].x = w0;
          fr[g >> 1].y = w1;
        }
      }
      static_for<0, NS>([&](auto jI) {
        constexpr int j = decltype(jI)::value;
        constexpr int kc = j / C::HDB, db = j % C::HDB;
        __builtin_amdgcn_sched_barrier(0);
        acc[db] = mfma_bf16(tf[j % W2], fr[kc], acc[db]);
        hold_acc(acc[db]);
        if constexpr (j + W2 < NS)
          tf[j % W2] = trfrag(tK, 16 * ((j + W2) / C::HDB), role * C::HDB + (j + W2) % C::HDB);
      });
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (live) {
    const int64_t row = (q_slab + qrow) * D;
#pragma unroll
    for (int db = 0; db < C::HDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = (role * C::HDB + db) * 32 + 8 * g + 4 * h;
        store_o4(p.dq, false, row + d, acc[db][4 * g + 0] * p.scale, acc[db][4 * g + 1] * p.scale,
                 acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
      }
    }
  }
}

template <int D>
hipError_t launch(const BwdParams& p0, hipStream_t stream) {
  // D from 192 run the kernels that split each block between two waves
  constexpr bool split = D > 128;
  constexpr int BK = split ? KVSplitCfg<D>::BK : KVCfg<D>::BK;
  constexpr int BR = split ? QSplitCfg<D>::BR : QCfg<D>::BR;
  BwdParams p = p0;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
  constexpr int RPB = 256 / prep_lanes<D>();
  const int64_t prep_wg = (rows + RPB - 1) / RPB;
  const int n_kt = (p.Nkv + BK - 1) / BK;
  const int n_qt = (p.Nq + BR - 1) / BR;
  p.pair_kv = pair_causal_grid(p.causal, (int64_t)p.B * p.Hkv, n_kt, p.Nq, p.Nkv);
  const int64_t kv_wg = (int64_t)(p.pair_kv ? (n_kt + 1) / 2 : n_kt) * p.B * p.Hkv;
  const int64_t q_wg = (int64_t)n_qt * p.B * p.Hq;
  if (prep_wg >= ((int64_t)1 << 31) || kv_wg >= ((int64_t)1 << 31) || q_wg >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_bwd_prep_kernel<D>), dim3((unsigned)prep_wg), dim3(256), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if constexpr (split)
    hipLaunchKernelGGL((attn_bwd_dkdv_split_kernel<D>), dim3((unsigned)kv_wg), dim3(KVSplitCfg<D>::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D>), dim3((unsigned)kv_wg), dim3(KVCfg<D>::NT), 0, stream, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if constexpr (split)
    hipLaunchKernelGGL((attn_bwd_dq_split_kernel<D>), dim3((unsigned)q_wg), dim3(QSplitCfg<D>::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), dim3((unsigned)q_wg), dim3(QCfg<D>::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  switch (p.D) {
    case 64: return launch<64>(p, stream);
    case 128: return launch<128>(p, stream);
    case 192: return launch<192>(p, stream);
    case 256: return launch<256>(p, stream);
    case 320: return launch<320>(p, stream);
    case 384: return launch<384>(p, stream);
    case 448: return launch<448>(p, stream);
    case 512: return launch<512>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
