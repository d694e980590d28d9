// attn_bwd.h -- internal interface of the backward launches (not part of
// the public ABI; see include/attn.h for that).
#pragma once

#include "attn_launch.h"

namespace attn {

// Backward pass (bf16, D a multiple of 64 up to 512): dQ, dK, dV from Q, K, V, the forward
// O and LSE and the upstream dO.  delta and lse2 are (B, Hq, Nq) float32
// workspace arrays the first launch fills.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  float* lse2;
  int B, Hq, Hkv, Nq, Nkv, D;
  int group;
  int causal;
  float scale;
  // causal key tiles of the dK/dV kernel paired first with last in one
  // work-group (set by the launcher)
  int pair_kv;
};

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

}  // namespace attn
