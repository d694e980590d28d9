// attn_dma.h -- direct-to-LDS K/V tile streaming shared by the kernels
// on gfx950: buffer descriptors in scalar registers, XOR swizzles matched to
// the 64-bank LDS, per-lane load offsets and the loads themselves.
#pragma once

#include "attn_common.h"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// XOR swizzles on the 16-byte chunk index of a row.  gfx950's LDS serves
// 256 bytes (64 banks) per clock, i.e. 16 lanes of a 16-byte read or 32
// lanes of an 8-byte read per phase, so a phase is conflict-free when its
// lanes touch 16 distinct chunks modulo 16.  K fragment reads put rows
// 0..15 in one phase: chunk ^ (row & 15).  Transposing V reads put 4 rows x
// 4 chunks (two 16-lane groups) in one phase: chunk ^ 4 (row & 3).  Both
// need 16 chunks per row (D a multiple of 128); D = 64 rows have 8 chunks and
// use the 8-wide forms (2-way conflicts remain there).
template <int D>
__device__ __forceinline__ int k_swz(int row) { return row & (D % 128 == 0 ? 15 : 7); }
template <int D>
__device__ __forceinline__ int v_swz(int row) { return (row & 3) * (D % 128 == 0 ? 4 : 2); }

// Swizzle of rows that are RP bytes long (RP a power of two times 16) read
// as K fragments, rows 0..15 of a 16-lane phase at one logical chunk: the
// RP/16 chunks of a row cover 16/(RP/16) rows' worth of one bank window, so
// the XOR key steps once every 16/(RP/16) rows.  Used for e4m3 K rows (D
// bytes each).
template <int RP>
__device__ __forceinline__ int k8_swz(int row) {
  constexpr int NCH = RP / 16;
  static_assert(NCH >= 4 && (NCH & (NCH - 1)) == 0, "row pitch");
  return NCH >= 16 ? (row & 15) : ((row / (16 / NCH)) & (NCH - 1));
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (base, stride 0, num_records = nbytes, gfx9 raw
// format) in scalar registers, for the inline-assembly loads below.
__device__ __forceinline__ i32x4 sgpr_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane((int)nbytes);
  r.w = 0x00020000;
  return r;
}

// The descriptor of one tile: base advanced by `off` bytes and the record
// count reduced to what is left of the slab (0 past its end, so every load of
// such a tile reads zeros).  Scalar arithmetic only.
__device__ __forceinline__ i32x4 rsrc_at(i32x4 r, uint32_t off) {
  const uint64_t a = ((uint64_t)(uint32_t)r.y << 32 | (uint32_t)r.x) + off;
  const uint32_t n = (uint32_t)r.z;
  const int left = max((int)n - (int)off, 0);  // slabs are < 2^31 bytes
  i32x4 t;
  t.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  t.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  t.z = __builtin_amdgcn_readfirstlane(left);
  t.w = r.w;
  return t;
}

// Per-lane byte offsets (within one tile of RP-byte rows) of N direct-to-LDS
// loads.  Wave `wave` fills N consecutive 1 KiB blocks of the LDS tile; lane
// l writes bytes [16 l, 16 l + 16) of a block, so the global chunk it
// fetches is the one that swizzle `swz` (row -> XOR key) places there.
template <int N, int RP, typename Swz>
__device__ __forceinline__ void dma_offsets_rows(uint32_t (&voff)[N], int wave, int lane, Swz swz) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int o = (wave * N + j) * 1024 + lane * 16;
    const int row = o / RP;
    const int pc = (o % RP) >> 4;
    const int gc = pc ^ swz(row);
    voff[j] = (uint32_t)(row * RP + (gc << 4));
  }
}

// The same for a bf16 K (IS_V = false) or V tile of config C (row pitch
// C::RP, C::DMA_WAVE loads per wave).
template <typename C, bool IS_V>
__device__ __forceinline__ void dma_offsets(uint32_t (&voff)[C::DMA_WAVE], int wave, int lane) {
  dma_offsets_rows<C::DMA_WAVE, C::RP>(voff, wave, lane,
                                       [](int row) { return IS_V ? v_swz<C::D>(row) : k_swz<C::D>(row); });
}

// Issue N direct-to-LDS loads of one tile (descriptor `rsrc`, positioned at
// the tile) into LDS byte address `lds_tile`.  M0 holds each 1 KiB block's
// LDS address.  Offsets at or past num_records read as zero.
template <int N>
__device__ __forceinline__ void dma_blocks(i32x4 rsrc, uint32_t lds_tile, const uint32_t (&voff)[N], int wave) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    // uniform by construction; readfirstlane keeps it in a scalar register
    // when the compiler has placed the slot arithmetic in vector registers
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(lds_tile + (uint32_t)((wave * N + j) * 1024));
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff[j]), "s"(rsrc), "s"(lds_addr)
        : "memory", "m0");
  }
}

// Block j (a compile-time index once unrolled) of the N that wave `wave`
// loads for one tile: lets a kernel spread a tile's loads between its MFMAs.
// A wave stalls on a load until the address path accepts it; issued back to
// back, a large tile's loads hold the wave for about the time the whole tile
// takes to stream, while between MFMAs the matrix pipe keeps working meanwhile.
template <int N>
__device__ __forceinline__ void dma_block_at(i32x4 rsrc, uint32_t lds_tile, uint32_t voff, int wave, int j) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(lds_tile + (uint32_t)((wave * N + j) * 1024));
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void dma_block_one(i32x4 rsrc, uint32_t lds_tile, const uint32_t (&voff)[N], int wave,
                                              int j) {
  dma_block_at<N>(rsrc, lds_tile, voff[j], wave, j);
}

// The offset dma_offsets computes for block j, computed on the spot for row
// pitches that are a multiple of 1 KiB: then a block lies within one row, so
// the row and its XOR key are uniform and only the chunk depends on the lane
// (a few VALU instructions instead of one register per block held for the
// whole kernel).
template <typename C, bool IS_V>
__device__ __forceinline__ uint32_t dma_offset_1k(int wave, int lane, int j) {
  static_assert(C::RP % 1024 == 0, "row pitch must be a multiple of 1 KiB");
  constexpr int BPR = C::RP / 1024;  // blocks per row
  const int blk = wave * C::DMA_WAVE + j;
  const int row = blk / BPR;
  const int pc = (blk % BPR) * 64 + lane;
  const int gc = pc ^ (IS_V ? v_swz<C::D>(row) : k_swz<C::D>(row));
  return (uint32_t)(row * C::RP + (gc << 4));
}

template <typename C>
__device__ __forceinline__ void dma_tile(i32x4 rsrc, uint32_t lds_tile, const uint32_t (&voff)[C::DMA_WAVE],
                                         int wave) {
  dma_blocks<C::DMA_WAVE>(rsrc, lds_tile, voff, wave);
}

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// acc *= alpha with every element kept in an accumulation register (AGPR).
// Written as C++, the multiply would make the register allocator hold the
// loop-carried accumulators in VGPRs and copy all of them to and from AGPRs
// on every tile (D/4 registers each way); the "a" constraint pins them.
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = acc[r], t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(v), "=&v"(t)
        : "v"(alpha));
    acc[r] = v;
  }
}

}  // namespace attn
