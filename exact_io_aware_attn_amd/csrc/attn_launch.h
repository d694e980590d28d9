// attn_launch.h -- internal interface between the C-ABI layer and the kernel
// launchers (not part of the public ABI; see include/attn.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  int group;           // Hq / Hkv
  int causal;          // 0 or 1
  int kv_off;          // Nkv - Nq: key j visible to query i iff j <= i + kv_off
  int n_qtiles;        // filled by the launcher
  int total_wg;        // filled by the launcher
  float scale;         // multiplier of Q K^T
  const float* dq;     // fp8 descales (device pointers) or null
  const float* dk;
  const float* dv;
};

typedef hipError_t (*LaunchFn)(const FwdParams&, hipStream_t);

// Launcher for the tiled kernel (D <= 256) of element type `elt`
// (attn::Elt) and head dim D, or nullptr if that pair is not instantiated.
LaunchFn tiled_launcher(int elt, int D);

// Launcher for the direct-to-LDS kernel (bf16: D = 64 or 128; e4m3: D = 64,
// 128 or 256; scale > 0), or nullptr.
LaunchFn pipe_launcher(int elt, int D);

// Launcher for the software-pipelined wide-head kernel (bf16, D a multiple
// of 64 in [192, 512], scale > 0), or nullptr.
LaunchFn wide_launcher(int elt, int D);

// Launcher for the split-D kernels (bf16, 256 < D <= 1024), or nullptr.
LaunchFn splitd_launcher(int elt, int D);

}  // namespace attn
