"""Seeded synthetic inputs, shared by the GPU tests, the bench and the oracle.

This module holds no attention arithmetic: it only draws random numbers,
casts them to the storage dtype the library consumes, and (for the fp8 path)
quantises them with a per-tensor descale.  Both sides of every parity check
read their inputs from here; the oracle then decodes the exact stored values
to float64 on its own.

Recipe (every workload):
  * generator ``numpy.random.default_rng(seed)`` (PCG64), seed 0 unless told
    otherwise; ``standard_normal`` in float64, drawn in the order Q, K, V,
    each as one full C-ordered tensor of shape (B, H, N, D);
  * an optional multiplier (0.5 for the large-head-dim workloads), applied in
    float64 before the cast;
  * cast to the storage dtype with round-to-nearest-even (torch's cast).

The fp8 recipe draws Q, K, V the same way, then for each tensor in the order
Q, K, V multiplies round(0.01 * H * D) distinct (head, channel) columns by 8
(the "1% outlier channels" of the diffusion-style fp8 workload; a channel is
read as one of the H*D hidden features), then quantises each tensor with
descale = absmax / 448 (float32) and code = e4m3fn(clamp(x / descale)).
The fp8 input-pipeline recipe ("fp8blk") draws Q, K, V the same way but
plants the outlier channels of Q and K in the same (head, channel) columns
(one draw for Q, reused for K; then one for V), the aligned large channels of
real query and key activations that a rotation before quantising is meant to
spread; it then casts Q, K, V to bf16 and draws the D rotation signs (+-1,
int8) with ``rng.integers(0, 2, D) * 2 - 1``.  The device quantises.

These Gaussian tensors stand in for the captured model activations that the
ZYFA article measures on (section "What the numbers establish, and where they
overstate"); the article notes that Gaussian inputs overstate speed-ups.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3FN_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype and input recipe."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    causal: bool
    dtype: str  # "f32", "bf16", "fp8" or "fp8blk" (bf16 inputs of the fp8 pipeline)
    value_scale: float = 1.0
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_mult: float = 8.0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def scale(self):
        """Softmax scale 1/sqrt(D) (every workload states or implies it)."""
        return 1.0 / float(np.sqrt(self.D))

    @property
    def visible_pairs(self):
        """Number of visible (query, key) pairs per head."""
        if not self.causal:
            return self.Nq * self.Nkv
        off = self.Nkv - self.Nq
        total = 0
        # rows i see keys j <= i + off, clipped to [0, Nkv)
        lo = max(0, -off)
        for_rows = np.arange(lo, self.Nq, dtype=np.int64)
        total = int(np.minimum(for_rows + off + 1, self.Nkv).sum())
        return total

    @property
    def flops(self):
        """Matmul flops: 4 * B * Hq * D * visible pairs (QK^T and PV)."""
        return 4 * self.B * self.Hq * self.D * self.visible_pairs

    def replace(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # tiny fp32 self-attention; the oracle finishes it in well under a second
    "tiny_f32": Workload("tiny_f32", 1, 2, 2, 256, 256, 64, False, "f32"),
    # LLM prefill, causal self-attention, bf16
    "prefill_causal_bf16": Workload("prefill_causal_bf16", 4, 32, 32, 4096, 4096, 128, True, "bf16"),
    # GQA causal prefill (group size 4) and its cross-attention variant
    "gqa_causal_bf16": Workload("gqa_causal_bf16", 2, 32, 8, 8192, 8192, 128, True, "bf16"),
    "gqa_cross_bf16": Workload("gqa_cross_bf16", 2, 32, 8, 2048, 8192, 128, False, "bf16"),
    # large head dims (split-D), inputs scaled by 0.5
    **{
        f"splitd_bf16_d{d}": Workload(f"splitd_bf16_d{d}", 1, 8, 8, 4096, 4096, d, False, "bf16", value_scale=0.5)
        for d in (320, 512, 768, 1024)
    },
    # fp8 e4m3 diffusion-style attention with 1% outlier channels
    "fp8_outlier": Workload("fp8_outlier", 1, 24, 24, 16384, 16384, 128, False, "fp8", outlier_frac=0.01),
    # the causal prefill with the probabilities' exponentials from a cubic
    # polynomial instead of the transcendental unit (extra["exp"])
    "prefill_causal_bf16_poly": Workload("prefill_causal_bf16_poly", 4, 32, 32, 4096, 4096, 128, True, "bf16",
                                         extra={"exp": "poly"}),
    # the backward pass of the causal prefill problem (extra["pass"]): dQ, dK,
    # dV from Q, K, V, the forward O and LSE and an upstream dO
    "bwd_causal_bf16": Workload("bwd_causal_bf16", 4, 32, 32, 4096, 4096, 128, True, "bf16",
                                extra={"pass": "bwd"}),
    # the backward at D = 256 and 512, causal self-attention over 4096
    # tokens, with the flops of the D = 128 problem
    "bwd_causal_bf16_d256": Workload("bwd_causal_bf16_d256", 2, 32, 32, 4096, 4096, 256, True, "bf16",
                                     extra={"pass": "bwd"}),
    "bwd_causal_bf16_d512": Workload("bwd_causal_bf16_d512", 1, 32, 32, 4096, 4096, 512, True, "bf16",
                                     extra={"pass": "bwd"}),
    # chunked prefill: a 256-token chunk against a 32K-token context, GQA,
    # causal (bottom-right: the chunk sees the whole context and itself
    # causally).  B * Hq * query tiles = 64 work-groups for 256 CUs, the case
    # key-range splitting is for; the same problem run plainly and split into
    # 8 key ranges (extra["n_splits"]; 512 work-groups, two per CU, the best
    # of 1..64 measured) merged by LSE.
    # the same problem with e4m3 probabilities (both products on the fp8
    # matrix instruction), exact or Lean P codes (extra["p"])
    "fp8_p8_outlier": Workload("fp8_p8_outlier", 1, 24, 24, 16384, 16384, 128, False, "fp8", outlier_frac=0.01,
                               extra={"p": "e4m3"}),
    "fp8_lean_outlier": Workload("fp8_lean_outlier", 1, 24, 24, 16384, 16384, 128, False, "fp8", outlier_frac=0.01,
                                 extra={"p": "lean"}),
    # the configuration the ZYFA article quotes its fp8 figure on: causal
    # prefill, 32K tokens, D = 128, Gaussian inputs (the article gives no head
    # count; 32 heads of 128, a 4096-wide model); e4m3 P, exact or Lean codes
    "fp8_p8_causal_32k": Workload("fp8_p8_causal_32k", 1, 32, 32, 32768, 32768, 128, True, "fp8",
                                  extra={"p": "e4m3"}),
    "fp8_lean_causal_32k": Workload("fp8_lean_causal_32k", 1, 32, 32, 32768, 32768, 128, True, "fp8",
                                    extra={"p": "lean"}),
    # the fp8 input pipeline on the same problem: bf16 Q, K, V with the same
    # outlier channels, quantised on the device with one descale per 64-row
    # block, Q and K rotated by a signed Hadamard matrix first
    "fp8_blocks_outlier": Workload("fp8_blocks_outlier", 1, 24, 24, 16384, 16384, 128, False, "fp8blk",
                                   outlier_frac=0.01),
    "chunk_prefill_bf16": Workload("chunk_prefill_bf16", 1, 32, 8, 256, 32768, 128, True, "bf16"),
    "chunk_prefill_splitkv_bf16": Workload("chunk_prefill_splitkv_bf16", 1, 32, 8, 256, 32768, 128, True, "bf16",
                                           extra={"n_splits": 8}),
}


_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def draw_gaussian_qkv(w: Workload):
    """float64 numpy Q, K, V drawn in that order from the workload's seed."""
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((w.B, w.Hq, w.Nq, w.D))
    k = rng.standard_normal((w.B, w.Hkv, w.Nkv, w.D))
    v = rng.standard_normal((w.B, w.Hkv, w.Nkv, w.D))
    if w.value_scale != 1.0:
        q *= w.value_scale
        k *= w.value_scale
        v *= w.value_scale
    return rng, q, k, v


def make_inputs(w: Workload):
    """CPU torch tensors (q, k, v) in the workload's storage dtype.

    For fp8 workloads returns (q8, k8, v8, descales) where the codes are
    ``torch.float8_e4m3fn`` tensors and ``descales`` is a float32 numpy array
    [dq, dk, dv].
    """
    rng, q, k, v = draw_gaussian_qkv(w)
    if w.dtype in _TORCH_DTYPE:
        dt = _TORCH_DTYPE[w.dtype]
        return tuple(torch.from_numpy(x).to(dt) for x in (q, k, v))
    if w.dtype == "fp8blk":
        cols = _outlier_channels(rng, q, w)
        _outlier_channels(rng, k, w, cols, group=w.Hq // w.Hkv)
        _outlier_channels(rng, v, w)
        signs = (rng.integers(0, 2, size=w.D) * 2 - 1).astype(np.int8)
        return (*(torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v)), torch.from_numpy(signs))
    if w.dtype != "fp8":
        raise ValueError(f"unknown dtype {w.dtype}")
    out, desc = [], []
    for x in (q, k, v):
        _outlier_channels(rng, x, w)
        code, d = quantize_e4m3(x)
        out.append(code)
        desc.append(d)
    if w.extra.get("qk_codes") == "narrow":
        # Q and K codes of magnitude in [1/2, 4) with random signs (descale
        # 1/4 each): every product is a multiple of 2^-8 below 16, so q . k
        # is exact in float32 whatever the summation order
        for i, x in enumerate((q, k)):
            mag = rng.integers(6 * 8, 9 * 8, size=x.shape)          # exponent field 6..8, any mantissa
            sign = rng.integers(0, 2, size=x.shape) << 7
            out[i] = torch.from_numpy((mag | sign).astype(np.uint8)).view(torch.float8_e4m3fn)
            desc[i] = np.float32(0.25)
    return out[0], out[1], out[2], np.array(desc, dtype=np.float32)


def _outlier_channels(rng, x, w, cols=None, group=1):
    """Multiply round(outlier_frac * H * D) distinct (head, channel) columns of
    x (B, H, N, D) by outlier_mult, in place, and return them.  Given columns
    (drawn over the query heads) are reused, query head h mapping to head
    h // group of x (the KV head of a GQA group); a column hit twice that way
    is multiplied once."""
    H, D = x.shape[1], x.shape[3]
    if cols is None:
        n_out = int(round(w.outlier_frac * H * D))
        if not n_out:
            return None
        cols = rng.choice(H * D, size=n_out, replace=False)
    if cols is not None and len(cols):
        hh, dd = np.divmod(cols, D)
        mine = np.unique((hh // group) * D + dd)
        hh, dd = np.divmod(mine, D)
        x[:, hh, :, dd] *= w.outlier_mult
    return cols


def block_descales(w, seed=1):
    """Per-64-row-block descales for the e4m3 codes of an fp8 workload (a
    kernel input of the block-scaled path): each tensor's per-tensor descale
    times factors drawn uniformly from [1/2, 2] (float32), one per (batch,
    head, block), from ``default_rng(seed)`` in the order Q, K, V.  Returns
    three float32 numpy arrays of shape (B, H, ceil(N / 64))."""
    _, _, _, desc = make_inputs(w)
    rng = np.random.default_rng(seed)
    out = []
    for d, H, N in zip(desc, (w.Hq, w.Hkv, w.Hkv), (w.Nq, w.Nkv, w.Nkv)):
        f = rng.uniform(0.5, 2.0, size=(w.B, H, (N + 63) // 64))
        out.append((f * np.float64(d)).astype(np.float32))
    return out


def quantize_e4m3(x):
    """Per-tensor absmax quantisation to e4m3fn: (codes, float32 descale)."""
    amax = float(np.abs(x).max())
    descale = np.float32(amax / E4M3FN_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(x / np.float64(descale), -E4M3FN_MAX, E4M3FN_MAX)
    return torch.from_numpy(y).to(torch.float8_e4m3fn), descale


def make_grad(w: Workload, seed_offset=1000):
    """Upstream gradient dO of the backward pass: standard normal, shape
    (B, Hq, Nq, D), from ``default_rng(w.seed + seed_offset)``, cast to bf16."""
    rng = np.random.default_rng(w.seed + seed_offset)
    g = rng.standard_normal((w.B, w.Hq, w.Nq, w.D))
    return torch.from_numpy(g).to(torch.bfloat16)


def random_problem(B, Hq, Hkv, Nq, Nkv, D, dtype="bf16", seed=0, value_scale=1.0, causal=False):
    """Inputs for an ad-hoc shape (tests): same recipe as the named workloads."""
    w = Workload("adhoc", B, Hq, Hkv, Nq, Nkv, D, causal, dtype, value_scale=value_scale, seed=seed)
    return w, make_inputs(w)
