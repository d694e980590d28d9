// attn_launch.h -- internal interface between the C-ABI layer and the kernel
// launchers (not part of the public ABI; see include/attn.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace attn {

// Arguments of one forward call after validation.  Sizes are int: the ABI
// layer has already checked that every per-(batch, head) slab and the grid
// fit in 31 bits.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  int B, Hq, Hkv, Nq, Nkv;
  int D;               // head dim (a kernel may run at a padded size of its own)
  int group;           // Hq / Hkv
  int causal;          // 0 or 1
  int kv_off;          // Nkv - Nq: key j visible to query i iff j <= i + kv_off
  int n_qtiles;        // filled by the launcher
  int total_wg;        // filled by the launcher: n_splits * B * Hq * (query tiles or pairs)
  float scale;         // multiplier of Q K^T
  const float* dq;     // fp8 descales (device pointers) or null
  const float* dk;
  const float* dv;
  // Key ranges (split-KV).  Split s of n_splits attends to the keys
  // [kv_begin + s * split_len, min(kv_begin + (s + 1) * split_len, kv_end))
  // of the Nkv-key sequence, with the causal alignment of the whole problem,
  // and writes its own O (normalised over its range) and LSE at o +
  // s * o_split_stride and lse + s * lse_split_stride (elements).  A plain
  // call is one split over [0, Nkv).
  int kv_begin;
  int kv_end;
  int split_len;
  int n_splits;
  int o_f32;                // O stored as float32 (partial results) instead of the dtype's output
  int64_t o_split_stride;
  int64_t lse_split_stride;
  // e4m3 with one descale per 64-row block (a plain key range only): dq
  // points at (B, Hq, ceil(Nq/64)) floats, dk and dv at (B, Hkv, ceil(Nkv/64))
  int blk_scaled;
  // causal query tiles paired first with last in one work-group (set by the
  // direct-to-LDS kernel's launcher)
  int pair_causal;
};

// The keys one work-group attends to: nkv keys starting at row k0 of its
// (batch, KV head) slab; local key j is visible to query row i iff
// j <= i + kv_off when causal.
struct KeyRange {
  int k0;
  int nkv;
  int kv_off;
};

__device__ __forceinline__ KeyRange key_range(const FwdParams& p, int split) {
  const int k0 = p.kv_begin + split * p.split_len;
  const int k1 = min(k0 + p.split_len, p.kv_end);
  return KeyRange{k0, k1 > k0 ? k1 - k0 : 0, p.kv_off - k0};
}

typedef hipError_t (*LaunchFn)(const FwdParams&, hipStream_t);

// Compute units of the current device, queried once per device (256 on
// MI355X; that value if the query fails).
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Causal tiles paired first with last (the ZYFA article, "The details that
// make it production-grade"): work-group i of a head runs tiles i and n-1-i
// back to back, the heavier first, so every work-group does about the same
// work (a query tile with key tiles, or a key tile with query tiles) and the
// last wave of work-groups is not a tail of short ones.  It halves the
// work-groups, so it is taken only where the queries' own triangle dominates
// (at most as many earlier keys as queries) and the paired grid still covers
// every compute unit four times over.  `heads` (batch, head) pairs of
// `n_tiles` tiles each, where `nq` queries see `nkv` keys.
inline int pair_causal_grid(int causal, int64_t heads, int n_tiles, int nq, int nkv) {
  const int64_t paired = heads * ((n_tiles + 1) / 2);
  return (causal && n_tiles > 1 && nkv - nq <= nq && paired >= 4 * (int64_t)cu_count()) ? 1 : 0;
}

// The rule for a forward launch (needs p.n_qtiles).
inline int pair_causal_tiles(const FwdParams& p) {
  return pair_causal_grid(p.causal, (int64_t)p.n_splits * p.B * p.Hq, p.n_qtiles, p.Nq, p.Nkv);
}

// Work-group slots per (split, batch, query head): query tiles or pairs.
__host__ __device__ inline int qtile_slots(const FwdParams& p) {
  return p.pair_causal ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
}

// Launcher for the tiled kernel (D <= 256) of element type `elt`
// (attn::Elt) and head dim D, or nullptr if that pair is not instantiated.
LaunchFn tiled_launcher(int elt, int D);

// Launcher for the direct-to-LDS kernel (bf16: D = 64 or 128, through
// bf16_launcher; e4m3: D = 64, 128 or 256; scale > 0), or nullptr.
LaunchFn pipe_launcher(int elt, int D);

// Launcher for the bf16 kernel of head dims 64 and 128 (scale > 0), or
// nullptr.
LaunchFn bf16_launcher(int D);

// Launcher for the software-pipelined wide-head kernel (bf16, D a multiple
// of 64 in [192, 512], scale > 0), or nullptr.
LaunchFn wide_launcher(int elt, int D);

// Launcher for the four-wave split-D kernel (bf16, D a multiple of 64 in
// [320, 960]), or nullptr.
LaunchFn splitd_launcher(int elt, int D);

// Launcher for the eight-wave split-D kernel (bf16, D = 1024; any scale), or
// nullptr.
LaunchFn splitd8_launcher(int elt, int D);

// Log-sum-exp merge of partial results: part i of o_parts (rows, D) starts
// at o_parts + i * o_part_stride and part i of lse_parts (rows) at
// lse_parts + i * lse_part_stride, all float32 -> o (rows, D; float32 if
// o_f32, else bf16) and lse (rows, or null).  D a multiple of 32 in
// [32, 1024]; o_part_stride a multiple of 4.
struct MergeParams {
  const float* o_parts;
  const float* lse_parts;
  void* o;
  float* lse;
  int n_parts;
  int D;
  int o_f32;
  int64_t rows;
  int64_t o_part_stride;
  int64_t lse_part_stride;
};

hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

// e4m3 Q/K/V with e4m3 probabilities: P V and the row sum on the fp8 matrix
// instruction, one power-of-two P scale per 64-key tile of each row; exact
// codes or Lean P codes.  D = 64 or 128, scale > 0, per-tensor descales.
LaunchFn p8_launcher(int D, bool lean);

// bf16 direct-to-LDS kernel with the probabilities' exponentials from a cubic
// polynomial on the FMA pipe (D = 64 or 128, scale > 0).
LaunchFn pipe_poly_launcher(int D);

// e4m3 block quantisation of S = B * H slabs of N x D bf16 rows (D = 64,
// 128 or 256): codes (S, N, D), descales (S, ceil(N/64)); rows rotated by
// diag(signs) H_D / sqrt(D) first when signs (D values of +-1) is not null.
struct QuantParams {
  const __bf16* x;
  uint8_t* codes;
  float* descales;
  const int8_t* signs;
  int S, N, D;
};

hipError_t launch_quant_fp8(const QuantParams& p, hipStream_t stream);

}  // namespace attn
