// attn_fwd_p8.hip -- e4m3 attention forward on gfx950 with e4m3 probabilities:
// both products run on the fp8 matrix instruction (D = 64 and 128, scale > 0).
//
// ZYFA article, section "The three techniques, in plain terms":
//  * per-block scaling with a rounded row sum: each 64-key block of a row's
//    probabilities is multiplied by a power of two before rounding to e4m3,
//    the scaled matrix instruction divides it back out in P V, and the row
//    sum is taken on the matrix unit from the same rounded values (one more
//    instruction per block), so the output is a true weighted average;
//  * Lean P (optional): the e4m3 code of 2^y is about 8 y + 56, so a
//    probability's code comes from one multiply-add and one conversion to an
//    unsigned byte, with no exponential.
//
// Layout (the direct-to-LDS e4m3 kernel's, with P V changed):
//  * 4 waves x 32 query rows per work-group, two work-groups per CU, 64-key
//    tiles streamed into LDS by direct-to-LDS loads, two slots.
//  * S^T = K Q^T on the fp8 instruction as in that kernel: one query per lane,
//    keys 32 kb + 8 (r / 4) + 4 h + r % 4 in accumulator register r of key
//    block kb (h = lane / 32).
//  * Base-2 scores x = s c (c = scale log2(e) dq dk).  The running maximum m
//    is an integer (raised to ceil of the tile maximum when the tile maximum
//    passes it by more than 8), so the rescale factor and every block scale
//    are powers of two.  The tile's block exponent is E = ceil(tile max) - 8:
//    the codes are those of 2^(x - E) (largest in (2^7, 2^8]), and the
//    matrix instruction's scale for P is 2^(E - m), an E8M0 byte per lane.
//  * P codes: lane (query, h) holds the 32 probabilities of its query whose
//    keys have lane half h, byte t = 16 kb + r of its B operand.  V tiles are
//    stored in LDS with rows permuted to that order (LDS row 32 h + t holds
//    key 32 (t / 16) + 8 ((t % 16) / 4) + 4 h + t % 4), so that the
//    transposing byte read ds_read_b64_tr_b8 returns, for each lane, 8 of the
//    32 keys of one head-dim column: four reads make the A operand V^T.
//  * Row sum: one more scaled instruction per tile with an A operand of
//    e4m3 ones; every row of its 32 x 32 result holds the column sums.
#include "attn_common.h"
#include "attn_dma.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;   // lazy-rescale threshold, base-2 units
constexpr int kTop = 8;        // block maximum scaled into (2^(kTop-1), 2^kTop]
constexpr int kOnes = 0x38383838;  // four e4m3 ones

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

template <int D_, bool LEAN_>
struct P8Cfg {
  static constexpr int D = D_;
  static constexpr bool LEAN = LEAN_;
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * 32;            // query rows per work-group
  static constexpr int BC = 64;                 // keys per tile (= one scale block)
  static constexpr int RPK = D;                 // e4m3 row pitch (bytes), K and V
  static constexpr int TILE = BC * RPK;         // bytes of one K or V tile
  static constexpr int DMA = TILE / 1024 / NW;  // direct-to-LDS loads per wave, one tile
  static constexpr int NDB = D / 32;            // 32-row blocks of O^T
  static constexpr int NQ8 = D / 64;            // 64-wide d chunks of the Q K^T contraction
  static constexpr int SLOT = 2 * TILE;         // K tile, V tile
  static constexpr int LDS = 2 * SLOT;
  static_assert(TILE % (1024 * NW) == 0, "tile must split evenly over the waves");
};

// V tile LDS row rho holds key vperm(rho) of the tile (see the file comment).
__device__ __forceinline__ int vperm(int rho) {
  const int h = rho >> 5, t = rho & 31;
  return 32 * (t >> 4) + 8 * ((t & 15) >> 2) + 4 * h + (t & 3);
}

// XOR swizzle of the 16-byte chunks of V rows: a transposing byte read puts
// 8 consecutive LDS rows x 2 chunks in one phase; rows of one bank window
// (two 128-byte rows, or four 64-byte rows) get different chunk pairs.
template <int D>
__device__ __forceinline__ int v8_swz(int rho) {
  if constexpr (D == 128) {
    return 2 * ((rho >> 1) & 3);
  } else {
    return 2 * ((rho >> 2) & 1);
  }
}

template <int D, bool LEAN>
__global__ __launch_bounds__(256, 2) void attn_fwd_p8_kernel(FwdParams p) {
  using C = P8Cfg<D, LEAN>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];
  const uint32_t lds_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int g16 = lane >> 4, r16 = lane & 15;

  // ---- work decomposition (as the direct-to-LDS kernel, one key range) ----
  const int wg_all = xcd_remap(blockIdx.x, p.total_wg);
  const int per_split = p.total_wg / p.n_splits;
  const int split = wg_all / per_split;
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
  const int q0w = q0 + wave * 32;

  const int64_t q_slab = ((int64_t)b * p.Hq + hq) * (int64_t)p.Nq * D;
  const int64_t kv_slab = (((int64_t)b * p.Hkv + hk) * (int64_t)p.Nkv + kr.k0) * D;
  const uint32_t kv_bytes = (uint32_t)((int64_t)kr.nkv * D);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + q_slab, (uint32_t)((int64_t)p.Nq * D));
  const i32x4 rk = sgpr_rsrc((const char*)p.k + kv_slab, kv_bytes);
  const i32x4 rv = sgpr_rsrc((const char*)p.v + kv_slab, kv_bytes);

  float c = p.scale * kLog2e * (p.dq ? p.dq[0] : 1.0f) * (p.dk ? p.dk[0] : 1.0f);
  const float out_scale = p.dv ? p.dv[0] : 1.0f;

  int kv_end = kr.nkv;
  if (p.causal) kv_end = min(kr.nkv, min(q0 + C::BR, p.Nq) + kr.kv_off);
  const int n_kt = kv_end > 0 ? (kv_end + C::BC - 1) / C::BC : 0;

  // ---- tile loads: K rows as stored (e4m3 K swizzle), V rows permuted ------
  uint32_t koff[C::DMA], voff[C::DMA];
  dma_offsets_rows<C::DMA, C::RPK>(koff, wave, lane, [](int row) { return k8_swz<C::RPK>(row); });
#pragma unroll
  for (int j = 0; j < C::DMA; ++j) {
    const int o = (wave * C::DMA + j) * 1024 + lane * 16;
    const int rho = o / C::RPK;
    const int pc = (o % C::RPK) >> 4;
    voff[j] = (uint32_t)(vperm(rho) * C::RPK + ((pc ^ v8_swz<D>(rho)) << 4));
  }
  auto issue = [&](int t, int slot) {
    const uint32_t dst = lds_base + (uint32_t)(slot * C::SLOT);
    dma_blocks<C::DMA>(rsrc_at(rk, (uint32_t)(t * C::TILE)), dst, koff, wave);
    dma_blocks<C::DMA>(rsrc_at(rv, (uint32_t)(t * C::TILE)), dst + C::TILE, voff, wave);
  };
  if (n_kt > 0) issue(0, 0);

  // Q codes (B operand of S^T = K Q^T): lane half h holds d = 64 cc + 32 h .. +31
  i32x8 q8[C::NQ8];
  {
    const uint32_t row_off = (uint32_t)(q0w + l32) * (uint32_t)D;
#pragma unroll
    for (int cc = 0; cc < C::NQ8; ++cc) {
      const u32x4 lo = buf_load16(rq, row_off + (uint32_t)(cc * 64 + h * 32));
      const u32x4 hi = buf_load16(rq, row_off + (uint32_t)(cc * 64 + h * 32 + 16));
      q8[cc] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }

  // LDS offsets: K fragment cc of key block kb (row l32 + 32 kb, code chunks
  // 4 cc + 2 h and +1); V^T read j of d-block db (rows 32 h + 8 j + r16 / 2,
  // chunk 2 db + (g16 & 1), byte 8 (r16 & 1))
  uint32_t k8base[2 * C::NQ8];
#pragma unroll
  for (int i = 0; i < 2 * C::NQ8; ++i)
    k8base[i] = (uint32_t)(l32 * C::RPK + (((4 * (i >> 1) + 2 * h + (i & 1)) ^ k8_swz<C::RPK>(l32)) << 4));
  uint32_t vtr[4 * C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rho = 32 * h + 8 * j + (r16 >> 1);
      const int chunk = 2 * db + (g16 & 1);
      vtr[4 * db + j] = (uint32_t)(rho * C::RPK + ((chunk ^ v8_swz<D>(rho)) << 4) + ((r16 & 1) << 3));
    }

  f32x16 acc[C::NDB], lacc = f32x16{};
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // an integer, or -inf before the first visible key
  const int qrow = q0w + l32;
  const int klim = p.causal ? min(kr.nkv - 1, qrow + kr.kv_off) : kr.nkv - 1;
  const i32x8 ones = i32x8{kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes};

  for (int kt = 0; kt < n_kt; ++kt) {
    const int slot = kt & 1;
    wait_vmem_all();
    __syncthreads();  // tile kt resident; the other slot (tile kt-1) is free
    if (kt + 1 < n_kt) issue(kt + 1, slot ^ 1);
    const char* const kb_cur = lds + slot * C::SLOT;
    const char* const vb_cur = kb_cur + C::TILE;
    // a causal tile entirely above this wave's rows (loaded for the
    // work-group's later waves) adds nothing to them
    if (p.causal && kt * C::BC > q0w + 31 + kr.kv_off) continue;

    // ---- S^T = K Q^T ------------------------------------------------------
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < C::NQ8; ++cc) {
        const uint32_t kbo = (uint32_t)(kb * 32 * C::RPK);
        const u32x4 lo = lds_load16(kb_cur, k8base[2 * cc] + kbo);
        const u32x4 hi = lds_load16(kb_cur, k8base[2 * cc + 1] + kbo);
        const i32x8 kf = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        s[kb] = mfma_fp8(kf, q8[cc], s[kb]);
      }
    }

    // ---- mask (tiles crossing the diagonal or the key tail) -------------------
    const int key0 = kt * C::BC;
    if ((key0 + C::BC > kr.nkv) || (p.causal && key0 + C::BC - 1 > q0w + kr.kv_off)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          s[kb][r] = key <= klim ? s[kb][r] : -INFINITY;
        }
    }

    // ---- tile maximum, lazy rescale with an integer running maximum ---------
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[kb][r]), s[kb][r + 1]);
    const float mrow = max_halves(mx) * c;  // base-2 units; -inf: no visible key here
    if (__builtin_amdgcn_ballot_w64(mrow > m_run + kTau) != 0) {
      const float m_new = mrow > m_run + kTau ? __builtin_ceilf(mrow) : m_run;
      const float alpha = m_run == -INFINITY ? 0.0f : exp2_fast(m_run - m_new);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) acc[db] *= alpha;
      lacc *= alpha;
      m_run = m_new;
    }
    // block exponent E = ceil(tile max) - 8 and the P scale 2^(E - m)
    const bool any = mrow != -INFINITY;
    const float E = any ? __builtin_ceilf(mrow) - (float)kTop : 0.0f;
    const int sc_code = any ? min(max(127 + (int)(E - m_run), 0), 254) : 0;

    // ---- e4m3 codes of 2^(x - E), byte t = 16 kb + r -----------------------------
    int pw[8];
    if constexpr (LEAN) {
      // code = rne(8 (x - E) + 56), one FMA and one conversion to a byte
      // (round to nearest even; negative values, -inf included, convert to 0)
      const float c8 = 8.0f * c, k8 = 56.0f - 8.0f * E;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = (w & 3) * 4;
        uint32_t u = 0;
        u = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[kb][r0 + 0], c8, k8), 0, u);
        u = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[kb][r0 + 1], c8, k8), 1, u);
        u = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[kb][r0 + 2], c8, k8), 2, u);
        u = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s[kb][r0 + 3], c8, k8), 3, u);
        pw[w] = (int)u;
      }
    } else {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = (w & 3) * 4;
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = exp2_fast(__builtin_fmaf(s[kb][r0 + i], c, -E));
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        pw[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], lo, true);
      }
    }
    const i32x8 pf = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};

    // ---- O^T += V^T P^T and the row sum, scale 2^(E - m) on P ------------------
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      int vw[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vb_cur + vtr[4 * db + j]));
        vw[2 * j] = v2.x;
        vw[2 * j + 1] = v2.y;
      }
      const i32x8 vf = i32x8{vw[0], vw[1], vw[2], vw[3], vw[4], vw[5], vw[6], vw[7]};
      acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, acc[db], 0, 0, 0, 127, 0, sc_code);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 127, 0, sc_code);
  }

  // ---- epilogue ---------------------------------------------------------------------
  const float l_tot = lacc[0];  // every row of the row-sum tile holds the column sums
  const float inv = l_tot > 0.0f ? out_scale / l_tot : 0.0f;
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

template <int D, bool LEAN>
hipError_t launch_p8(const FwdParams& p0, hipStream_t stream) {
  using C = P8Cfg<D, LEAN>;
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + C::BR - 1) / C::BR;
  p.pair_causal = pair_causal_tiles(p);
  const int64_t total = (int64_t)p.n_splits * p.B * p.Hq * qtile_slots(p);
  if (total <= 0 || total >= (int64_t)1 << 31) return hipErrorInvalidValue;
  p.total_wg = (int)total;
  hipLaunchKernelGGL((attn_fwd_p8_kernel<D, LEAN>), dim3(p.total_wg), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

LaunchFn p8_launcher(int D, bool lean) {
  switch (D) {
    case 64: return lean ? &launch_p8<64, true> : &launch_p8<64, false>;
    case 128: return lean ? &launch_p8<128, true> : &launch_p8<128, false>;
    default: return nullptr;
  }
}

}  // namespace attn
