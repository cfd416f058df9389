"""Workload shapes and seeded input generators.

The shapes follow the DeepSeek-V3 expert-parallel setting the MORI-EP User
Guide uses throughout (section 2 "Configuration", DeepSeek V3 example:
hidden 7168, 256 experts, top-8, 4096 tokens per rank) and the two benchmark
tables of the MORI README (4096 tokens for bandwidth, 128 tokens for
latency, FP8 dispatch + BF16 combine).  The pages benchmark on synthetic
random routing (section 7 "Complete Example": randn token rows, randperm
top-k), not on a dataset, so nothing here stands in for a public suite.

Draw order for a given seed (one ``numpy.random.default_rng(seed)``):

1. token rows ``x``: standard normal float32, rounded to bfloat16 by torch;
2. expert ids (uniform distinct, or Zipf-skewed distinct, see below);
3. gate logits ``standard_normal((T, k))``; weights are their softmax taken
   in float64 and stored as float32.

The routing draws (which experts each token picks) and gate weights are
inputs of the method; they are produced here and handed to both sides.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int            # T, tokens of this call
    hidden: int            # H, hidden_dim
    ranks: int             # R, world_size (virtual ranks on one GPU)
    experts_per_rank: int  # num_experts_per_rank
    topk: int              # num_experts_per_token
    cap: int               # max_num_inp_token_per_rank
    quant: str             # "none", "fp8" (OCP E4M3, per-128-column fp32 scales) or
                           # "mxfp4" (OCP MX FP4, per-32-column E8M0 scales)
    routing: str           # "uniform" or "zipf"
    expert: str            # expert stand-in: "identity", "dequant_half", "dequant"
    layout: str            # "rank_major" or "expert_major"
    zipf_s: float = 1.2
    combine: str = "bf16"  # combine payload: "bf16", or "fp8_direct" (E4M3 cast, no scale)

    @property
    def experts(self) -> int:
        return self.ranks * self.experts_per_rank

    @property
    def scale_dim(self) -> int:
        return self.hidden // 128 if self.quant in ("fp8", "mxfp4") else 0

    @property
    def cap_em(self) -> int:
        """Upper bound on expert-major rows: every token-expert pair plus the
        worst-case padding of each expert segment to a multiple of 128."""
        return self.tokens * self.topk + 127 * self.experts

    def with_tokens(self, tokens: int, cap: int | None = None) -> "Workload":
        return dataclasses.replace(self, tokens=tokens,
                                   cap=max(cap if cap is not None else self.cap, tokens))


WORKLOADS = {
    # plumbing case: everything small enough to check by hand
    "tiny": Workload("tiny", 16, 256, 4, 2, 2, 16, "none", "uniform", "identity", "rank_major"),
    # latency shape of the README latency table (128 tokens), bf16 both ways
    "decode": Workload("decode", 128, 7168, 8, 32, 8, 4096, "none", "uniform", "identity", "rank_major"),
    # bandwidth shape of the README bandwidth table: FP8 dispatch + BF16 combine
    "prefill": Workload("prefill", 4096, 7168, 8, 32, 8, 4096, "fp8", "uniform", "dequant_half", "rank_major"),
    # skewed routing: Zipf(1.2) expert popularity, 16 ranks x 16 experts
    "skew": Workload("skew", 4096, 7168, 16, 16, 8, 4096, "none", "zipf", "identity", "rank_major"),
    # standard-MoE layout: FP8 dispatch, expert-major conversion, combine from it
    "stdmoe": Workload("stdmoe", 4096, 7168, 32, 8, 8, 4096, "fp8", "uniform", "dequant", "expert_major"),
    # the prefill shape with the tuning matrix's low-precision pairings: FP4
    # dispatch with a bf16 combine, and an FP8 direct-cast combine payload
    "prefill_mxfp4": Workload("prefill_mxfp4", 4096, 7168, 8, 32, 8, 4096, "mxfp4", "uniform",
                              "dequant_half", "rank_major"),
    "prefill_fp8direct": Workload("prefill_fp8direct", 4096, 7168, 8, 32, 8, 4096, "fp8",
                                  "uniform", "dequant_half", "rank_major", combine="fp8_direct"),
}


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _uniform_topk(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    # k distinct experts per token, every k-subset equally likely
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def _zipf_topk(rng: np.random.Generator, T: int, E: int, k: int, s: float) -> np.ndarray:
    # expert popularity p ~ 1/i^s over a seeded permutation of the experts;
    # k distinct draws by successive renormalised sampling, done in one go
    # as Gumbel-top-k on log p
    perm = rng.permutation(E)
    p = np.empty(E, dtype=np.float64)
    p[perm] = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    p /= p.sum()
    g = rng.gumbel(size=(T, E))
    keys = np.log(p)[None, :] + g
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def make_inputs(wl: Workload, seed: int) -> dict:
    """Return host arrays: x (uint16 bf16 bits, [T,H]), indices (int32 [T,k]),
    weights (float32 [T,k])."""
    rng = np.random.default_rng(seed)
    T, H, k, E = wl.tokens, wl.hidden, wl.topk, wl.experts
    x32 = rng.standard_normal((T, H), dtype=np.float32)
    x = _bf16_bits(x32)
    if wl.routing == "uniform":
        idx = _uniform_topk(rng, T, E, k)
    elif wl.routing == "zipf":
        idx = _zipf_topk(rng, T, E, k, wl.zipf_s)
    else:
        raise ValueError(wl.routing)
    logits = rng.standard_normal((T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return {"x": x, "indices": np.ascontiguousarray(idx), "weights": np.ascontiguousarray(w)}


def make_fp8_payload(T: int, H: int, scale_dim: int, seed: int) -> dict:
    """An already-quantized payload for the carry mode: E4M3 bytes drawn
    uniformly over the 254 non-NaN codes ([T,H] uint8) and fp32 scales drawn
    uniformly from [2^-8, 1) ([T,scale_dim]).  Own generator, seeded apart
    from make_inputs."""
    rng = np.random.default_rng(10_000 + seed)
    codes = rng.integers(0, 254, (T, H), dtype=np.int32)
    codes += codes >= 0x7F   # skip 0x7F (NaN)
    codes += codes >= 0xFF   # skip 0xFF (NaN)
    scales = (2.0 ** -8 + rng.random((T, scale_dim)) * (1 - 2.0 ** -8)).astype(np.float32)
    return {"q": codes.astype(np.uint8), "scales": scales}
