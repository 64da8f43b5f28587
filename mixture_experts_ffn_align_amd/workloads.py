"""Seeded synthetic inputs for the fused MoE expert-FFN forward.

This module is shared by the GPU path, the CPU oracle, the tests and the
benchmark. It holds no arithmetic of the method: it only draws random
tensors and lays them out (packed weight views, strided id slices,
transposed activations). Routing, sorting, quantisation and the FFN all live
elsewhere, once in the HIP library and once, independently, in the oracle.

Shapes and distributions follow the workloads the pages measure:

* Liger-Kernel PR "Support strided Liger MoE input weights", section
  Problems: Qwen-style packed ``w13 [E, 2I, H]`` with gate = rows ``[0, I)``
  and up = rows ``[I, 2I)``; the Qwen3-235B shape H=4096, I=1536 (EP8 gives
  16 experts per GPU, the full layer has 128 experts, top-8).
* prime-rl PR "contiguous routed_experts slice for glm4_moe", section
  Problem: ``routed_experts [batch, seq, num_layers, top_k]`` sliced per
  layer, token stride num_layers * top_k = 46 * 8 = 368.
* LightLLM issue "_rms_norm_fwd_fused drops x_stride1", section
  Reproduction: an activation built as ``randn(N, M).t()`` whose last-dim
  stride is not 1.
* ROCm/aiter PR "add TP2 MXFP4 fused-MoE configs for Qwen3.5-397B",
  sections Summary and Details: model_dim 4096, inter_dim 512 (the TP2
  shard), 512 routed experts with top-10, or 513 with top-11 where the
  513th is a shared expert; token buckets 1 ... 32768.

Everything is drawn with ``torch.Generator(device).manual_seed(seed)`` in
float32 and cast to bfloat16 with round-to-nearest-even (torch's cast). Draw
order is fixed: logits, x, w13 (expert by expert), w2 (expert by expert),
then any extra routing layers. The same seed on another device gives other
values; parity always feeds both sides the same bytes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """Static sizes of one MoE layer."""

    name: str
    hidden: int          # H (model_dim)
    inter: int           # I (inter_dim, per expert)
    experts: int         # E rows in the weight tensors
    top_k: int           # k slots per token (includes a shared slot if any)
    mode: str            # "bf16" or "mxfp4"
    routed_experts: int  # experts the router chooses among
    routed_k: int        # slots the router fills
    shared_expert: int = -1   # id appended with weight 1.0, or -1
    w13_std: float = 0.02
    w2_std: float = 0.02


# Tiny case the oracle finishes in well under a second.
TINY_BF16 = MoEShape("tiny_bf16_h256_i128_e8_k2", 256, 128, 8, 2, "bf16", 8, 2,
                     w13_std=1.0 / 16.0, w2_std=1.0 / math.sqrt(128.0))
# Qwen3-235B-shaped layer, all 128 experts on one GPU.
QWEN3_235B_BF16 = MoEShape("qwen3_235b_bf16_h4096_i1536_e128_k8", 4096, 1536, 128, 8,
                           "bf16", 128, 8)
# Qwen3.5-397B TP2 shard, unfused routing (512 experts, top-10).
QWEN35_397B_TP2_FP4_512 = MoEShape("qwen35_397b_tp2_mxfp4_h4096_i512_e512_k10", 4096, 512,
                                   512, 10, "mxfp4", 512, 10, w13_std=1.0, w2_std=1.0)
# Same shard with the shared expert fused in as expert 512 (513 experts, top-11).
QWEN35_397B_TP2_FP4_513 = MoEShape("qwen35_397b_tp2_mxfp4_h4096_i512_e513_k11", 4096, 512,
                                   513, 11, "mxfp4", 512, 10, shared_expert=512,
                                   w13_std=1.0, w2_std=1.0)

SHAPES = {s.name: s for s in (TINY_BF16, QWEN3_235B_BF16, QWEN35_397B_TP2_FP4_512,
                               QWEN35_397B_TP2_FP4_513)}

REPLAY_LAYERS = 46   # GLM-4.5-Air layer count in the prime-rl report
REPLAY_LAYER = 7     # layer whose slice is fed to the MoE


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device, std=1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def draw_weights(shape: MoEShape, g: torch.Generator, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Packed ``w13 [E, 2I, H]`` and ``w2 [E, H, I]`` in bf16, expert by expert."""
    E, H, I = shape.experts, shape.hidden, shape.inter
    w13 = torch.empty((E, 2 * I, H), dtype=torch.bfloat16, device=device)
    for e in range(E):
        w13[e].copy_(_randn((2 * I, H), g, device, shape.w13_std))
    w2 = torch.empty((E, H, I), dtype=torch.bfloat16, device=device)
    for e in range(E):
        w2[e].copy_(_randn((H, I), g, device, shape.w2_std))
    return w13, w2


def uniform_logits(T: int, n: int, g, device) -> torch.Tensor:
    """Router logits ``[T, n]`` iid N(0, 1) in fp32."""
    return _randn((T, n), g, device)


def zipf_logits(T: int, n: int, g, device, s: float = 1.2, empty: int = 4) -> torch.Tensor:
    """Router logits whose top-k choice follows a Zipf(s) popularity.

    Expert popularity p_r is proportional to r**-s over ranks r = 1..n, the
    ``empty`` least popular ranks get p = 0 so some experts receive no
    tokens, and a seeded permutation assigns ranks to experts. The logits are
    ln p_e plus standard Gumbel noise (-inf where p = 0), so that picking the
    k largest is a draw without replacement proportional to p.
    """
    ranks = torch.arange(1, n + 1, dtype=torch.float64)
    p = ranks.pow(-s)
    p[n - empty:] = 0.0
    perm = torch.randperm(n, generator=g, device=device).cpu()
    pe = torch.empty(n, dtype=torch.float64)
    pe[perm] = p
    logp = torch.where(pe > 0, pe.log(), torch.full_like(pe, -math.inf)).to(torch.float32)
    u = torch.rand((T, n), generator=g, device=device, dtype=torch.float32)
    u = u.clamp_(min=1e-12, max=1.0 - 1e-7)
    gumbel = -torch.log(-torch.log(u))
    return gumbel + logp.to(device)[None, :]


def random_routing(T: int, n_experts: int, k: int, g, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Distinct random expert ids ``[T, k]`` int32 and positive weights summing to 1.

    Used where the routing is an *input* (router replay): the ids are the
    first k entries of a random permutation per token.
    """
    keys = torch.rand((T, n_experts), generator=g, device=device)
    ids = keys.argsort(dim=1)[:, :k].to(torch.int32)
    w = torch.rand((T, k), generator=g, device=device, dtype=torch.float32) + 0.05
    w = w / w.sum(dim=1, keepdim=True)
    return ids.contiguous(), w.contiguous()


def make_inputs(shape: MoEShape, T: int, *, seed: int = 0, device="cpu",
                routing: str = "logits", x_layout: str = "contiguous",
                weights: Optional[tuple] = None, logits_kind: str = "uniform") -> dict:
    """One seeded input set.

    routing:   "logits" -> router logits [T, routed_experts] are returned and
               routing is part of the call;
               "replay" -> ids/weights are slices [:, :, 7, :] of
               [1, T, 46, k] int32/fp32 tensors (token stride 46*k).
    x_layout:  "contiguous" or "transposed" (x = randn(H, T).t(), last-dim
               stride T).
    weights:   an existing (w13, w2) pair to reuse instead of drawing.
    """
    dev = torch.device(device)
    g = _gen(dev, seed)
    out = {"shape": shape, "T": T, "seed": seed}
    if routing == "logits":
        if logits_kind == "zipf":
            out["logits"] = zipf_logits(T, shape.routed_experts, g, dev)
        else:
            out["logits"] = uniform_logits(T, shape.routed_experts, g, dev)
    if x_layout == "transposed":
        buf = _randn((shape.hidden, T), g, dev).to(torch.bfloat16)
        out["x"] = buf.t()
    else:
        out["x"] = _randn((T, shape.hidden), g, dev).to(torch.bfloat16)
    if weights is None:
        w13, w2 = draw_weights(shape, g, dev)
    else:
        w13, w2 = weights
    out["w13"], out["w2"] = w13, w2
    if routing == "replay":
        k = shape.top_k
        ids_all = torch.empty((1, T, REPLAY_LAYERS, k), dtype=torch.int32, device=dev)
        w_all = torch.empty((1, T, REPLAY_LAYERS, k), dtype=torch.float32, device=dev)
        for layer in range(REPLAY_LAYERS):
            gl = _gen(dev, seed * 1000 + layer + 1)
            i_l, w_l = random_routing(T, shape.experts, k, gl, dev)
            ids_all[0, :, layer, :] = i_l
            w_all[0, :, layer, :] = w_l
        out["ids_all"], out["w_all"] = ids_all, w_all
        out["topk_ids"] = ids_all[0, :, REPLAY_LAYER, :]
        out["topk_weights"] = w_all[0, :, REPLAY_LAYER, :]
    return out


def packed_views(w13: torch.Tensor, inter: int) -> tuple[torch.Tensor, torch.Tensor]:
    """gate = w13[:, :I], up = w13[:, I:] — views with expert stride 2*I*H."""
    return w13[:, :inter, :], w13[:, inter:, :]


def bucket_tokens() -> list[int]:
    """Token buckets 1, 2, 4, ..., 32768."""
    return [1 << i for i in range(16)]
