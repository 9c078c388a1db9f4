"""Workload definitions and seeded generators.

Every draw uses numpy's PCG64 through ``SeedSequence(seed).spawn(4)``: child 0
draws the hidden states x, child 1 the router logits, child 2 the expert
permutation behind the Zipf bias, child 3 the expert weights.  Inputs are drawn
in float32 and stored as:

* ``f32``  -- float32 [N, D];
* ``bf16`` -- uint16 bit patterns [N, D], rounded to nearest-even by torch's
  CPU cast;
* ``f8``   -- uint8 E4M3FN bit patterns [N, D] plus float32 block scales
  [N, D/128]: s = amax(|x block|) / 448 (1 for an all-zero block), q =
  round-to-nearest-even of clamp(x / s, -448, 448) by torch's CPU cast.

Router logits are float32 N(0, 1).  The prefill workload adds a per-expert
bias b_e = -s * ln(1 + pi(e)) with pi a seeded permutation of the experts,
which makes expert popularity Zipf-like with exponent s = 1.1.  The bias is
part of the input: the router sees plain logits.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    seed: int
    n_tokens: int
    hidden: int
    dtype: str            # 'f32' | 'bf16' | 'f8'
    n_experts: int
    top_k: int
    n_segments: int = 1
    sort: object = -1     # -1 auto, 0 unsorted, 1 sorted, 'alternate'
    sort_cutoff: int = 0  # 0: 24 rows per expert, 24 * E // k (the measured crossover)
    renormalize: bool = True
    zipf_s: float = 0.0
    ffn: int = 0          # > 0: grouped SwiGLU experts, else identity experts
    weight_std: float = 0.02
    note: str = field(default="", compare=False)

    def __post_init__(self):
        if self.sort_cutoff <= 0:
            object.__setattr__(self, "sort_cutoff", max(1, 24 * self.n_experts // self.top_k))

    def with_tokens(self, n: int) -> "WorkloadConfig":
        return replace(self, n_tokens=n)

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "f8": 1}[self.dtype]


CONFIGS = {
    "tiny": WorkloadConfig(
        "tiny", 0, 16, 64, "f32", 8, 2, 1, sort=-1,
        note="N=16, D=64 fp32, E=8, softmax top-2 renormalised, identity experts"),
    "decode": WorkloadConfig(
        "decode", 1, 128, 7168, "bf16", 256, 8, 1, sort=0,
        note="N=128, D=7168 bf16, E=256, top-8, unsorted dispatch, identity experts"),
    "prefill": WorkloadConfig(
        "prefill", 2, 4096, 7168, "bf16", 256, 8, 1, sort=1, zipf_s=1.1,
        note="N=4096, D=7168 bf16, E=256, top-8, Zipf(1.1) popularity, sorted dispatch"),
    "mixtral": WorkloadConfig(
        "mixtral", 3, 8192, 4096, "bf16", 8, 2, 1, sort=-1, ffn=14336,
        note="N=8192, D=4096 bf16, E=8, top-2, grouped SwiGLU F=14336 read in place"),
    "segment": WorkloadConfig(
        "segment", 4, 1024, 7168, "f8", 256, 8, 8, sort="alternate",
        note="N=1024, D=7168 fp8-e4m3 + fp32/128 scales, E=256 in 8 groups, top-8"),
}


# The decode workload with real experts behind it: the same tokens, logits and
# unsorted layout, each of the 256 experts a SwiGLU FFN of a DeepSeek-V3-sized
# routed expert (F = 2048; 88 MB of bf16 weights per expert, 22.5 GB in all).
DECODE_FFN = replace(CONFIGS["decode"], name="decode_ffn", ffn=2048,
                     note="N=128, D=7168 bf16, E=256, top-8, unsorted dispatch, "
                          "SwiGLU experts F=2048 picked per row")


def _children(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(4)]


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_fp8_blocks(a: np.ndarray, block: int = 128):
    n, d = a.shape
    if d % block:
        raise ValueError("fp8 payload needs hidden % 128 == 0")
    xb = a.reshape(n, d // block, block).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    scaled = np.clip(xb / scales[:, :, None], -448.0, 448.0).astype(np.float32)
    q = torch.from_numpy(scaled.reshape(n, d)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), scales


def make_inputs(cfg: WorkloadConfig) -> dict:
    """-> dict(x, x_scales (f8 only, else None), logits) as numpy arrays."""
    gx, gl, gp, _ = _children(cfg.seed)
    n, d, e = cfg.n_tokens, cfg.hidden, cfg.n_experts
    xf = gx.standard_normal((n, d), dtype=np.float32)
    logits = gl.standard_normal((n, e), dtype=np.float32)
    if cfg.zipf_s:
        perm = gp.permutation(e)
        bias = (-cfg.zipf_s * np.log1p(perm.astype(np.float64))).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
    x_scales = None
    if cfg.dtype == "f32":
        x = xf
    elif cfg.dtype == "bf16":
        x = _to_bf16_bits(xf)
    elif cfg.dtype == "f8":
        x, x_scales = _to_fp8_blocks(xf)
    else:
        raise ValueError(cfg.dtype)
    return dict(x=x, x_scales=x_scales, logits=logits)


def make_swiglu_weights(cfg: WorkloadConfig, experts=None) -> dict:
    """bf16 bit patterns: w_gate, w_up [E, F, D] and w_down [E, D, F], drawn
    N(0, weight_std) expert by expert (so a subset can be regenerated
    identically).  ``experts`` restricts which experts are materialised (the
    others are left as zeros)."""
    if cfg.ffn <= 0:
        raise ValueError("workload has identity experts")
    e, f, d = cfg.n_experts, cfg.ffn, cfg.hidden
    _, _, _, gw = _children(cfg.seed)
    seqs = np.random.SeedSequence(int(gw.integers(0, 2**63 - 1))).spawn(3 * e)
    want = range(e) if experts is None else experts
    out = {name: np.zeros(shape, dtype=np.uint16) for name, shape in
           (("w_gate", (e, f, d)), ("w_up", (e, f, d)), ("w_down", (e, d, f)))}
    for i in want:
        for m, name in enumerate(("w_gate", "w_up", "w_down")):
            g = np.random.Generator(np.random.PCG64(seqs[3 * i + m]))
            shape = out[name].shape[1:]
            w = g.standard_normal(shape, dtype=np.float32) * np.float32(cfg.weight_std)
            out[name][i] = _to_bf16_bits(w)
    return out


def make_swiglu_weights_device(cfg: WorkloadConfig, device="cuda:0") -> dict:
    """The expert weights of a full-size workload drawn directly in device
    memory (2.8 GB of bf16 for the Mixtral-like layer would take minutes to
    draw on the host): torch's seeded Philox generator draws N(0, 1) in
    float32, scaled by weight_std and rounded to bfloat16 by torch's cast.
    Returns bfloat16 tensors w_gate, w_up [E, F, D] and w_down [E, D, F]."""
    if cfg.ffn <= 0:
        raise ValueError("workload has identity experts")
    e, f, d = cfg.n_experts, cfg.ffn, cfg.hidden
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed * 1000003 + 17)
    out = {}
    for name, shape in (("w_gate", (e, f, d)), ("w_up", (e, f, d)), ("w_down", (e, d, f))):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for i in range(e):                       # one expert at a time bounds the fp32 temporary
            t[i] = (torch.randn(shape[1:], generator=gen, device=device, dtype=torch.float32)
                    * cfg.weight_std).to(torch.bfloat16)
        out[name] = t
    return out


# fp8 expert projection consuming the segment-major rows: a DeepSeek-V3-sized
# expert's gate and up projections (F = 2048 each) stacked, N = 4096, K = 7168.
FP8_GEMM_N = 4096


def make_fp8_expert_weights_device(cfg: WorkloadConfig, n_out: int = FP8_GEMM_N,
                                   device="cuda:0", weight_std: float = 0.02) -> dict:
    """fp8 expert weights for a workload, drawn in device memory (256 experts
    x 4096 x 7168 is 7.5 GB): torch's seeded Philox draws N(0, weight_std) in
    float32 per expert; each 128 x 128 block gets the scale amax / 448 (1 for
    an all-zero block) and its codes are torch's round-to-nearest-even cast of
    w / scale to float8 E4M3FN.  Returns w [E, N, K] uint8 codes and w_scales
    [E, N/128, K/128] float32."""
    e, k = cfg.n_experts, cfg.hidden
    if k % 128 or n_out % 128:
        raise ValueError("N and K must be multiples of 128")
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed * 1000003 + 29)
    w = torch.empty((e, n_out, k), dtype=torch.uint8, device=device)
    ws = torch.empty((e, n_out // 128, k // 128), dtype=torch.float32, device=device)
    for i in range(e):
        f = torch.randn((n_out, k), generator=gen, device=device, dtype=torch.float32) * weight_std
        blocks = f.view(n_out // 128, 128, k // 128, 128)
        amax = blocks.abs().amax(dim=(1, 3))
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (blocks / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        w[i] = q.view(torch.uint8).view(n_out, k)
        ws[i] = s
    return {"w": w, "w_scales": ws}


def alternating_sort(call_index: int) -> int:
    """The segment-major workload toggles the runtime sort flag per call:
    even calls unsorted, odd calls sorted."""
    return call_index & 1
