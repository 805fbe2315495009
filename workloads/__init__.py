"""Seeded synthetic inputs for the expert load-balancing path.

This module only draws inputs: gate top-k expert IDs, the native expert
placement with its spare-slot budget, and bf16 expert weights.  It holds none
of the balancing arithmetic (no histogram, planner, reroute or statistics), so
both the HIP path and the CPU oracle can be fed from it without sharing code.

Workload shapes follow the model families the UltraEP article evaluates
(Qwen3-235B, GLM-4.5, DeepSeek-V3 at EP64 / EP40; m.youleyou.com article,
section on the key designs, evaluation paragraph) and the EPLB tutorial's
12 logical + 4 redundant example on 8 GPUs (t6page EPLB page, "12 logical + 4
redundant" example).  No routing trace or trained weight is available, so the
distributions below are synthetic stand-ins:

* top-k without replacement is drawn with the Gumbel-top-k trick (Kool, van
  Hoof and Welling, ICML 2019): adding i.i.d. Gumbel noise to log-probabilities
  and keeping the k largest keys is the same as sampling k experts one after
  another proportionally to p without replacement.  Each token's k IDs are
  stored in descending key order.
* per-plan parameters (Dirichlet probabilities, permutations, biases) come from
  numpy's PCG64 seeded by ``SeedSequence([20260101, workload index, microbatch,
  layer])``; the per-token noise comes from a torch generator seeded from the
  same sequence, on whatever device the caller asks for.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

SEED_ROOT = 20260101


@dataclass(frozen=True)
class Workload:
    """One routing workload: the EP group, its slot budget and its routing law.

    Native placement is a contiguous split of the logical experts over the
    ranks (rank r hosts ``native_count[r]`` consecutive expert IDs) and every
    rank owns ``spare_count[r]`` reserved replica slots.
    """

    name: str
    index: int                      # seed-tree branch for this workload
    num_experts: int                # E, logical experts
    top_k: int                      # k
    num_ranks: int                  # R, EP size
    tokens_per_rank: int            # T
    microbatches: int
    layers: int                     # MoE layers planned per microbatch
    native_count: Tuple[int, ...]   # [R]
    spare_count: Tuple[int, ...]    # [R]
    expert_shape: Tuple[int, ...]   # bf16 elements of one expert's weights
    law: str                        # routing distribution, see _plan_probs
    params: Tuple[Tuple[str, float], ...] = field(default_factory=tuple)

    # ---- derived sizes -------------------------------------------------
    @property
    def num_plans(self) -> int:
        return self.microbatches * self.layers

    @property
    def pairs_per_plan(self) -> int:
        return self.num_ranks * self.tokens_per_rank * self.top_k

    @property
    def num_spare(self) -> int:
        return int(sum(self.spare_count))

    @property
    def num_phys(self) -> int:
        return self.num_experts + self.num_spare

    @property
    def bytes_per_expert(self) -> int:
        return int(np.prod(self.expert_shape)) * 2

    def param(self, key: str) -> float:
        return dict(self.params)[key]

    def native_experts(self) -> np.ndarray:
        """Rank-major list of native expert IDs (rank r's block is consecutive)."""
        return np.arange(self.num_experts, dtype=np.int32)

    def scaled(self, tokens_per_rank: Optional[int] = None,
               layers: Optional[int] = None,
               microbatches: Optional[int] = None) -> "Workload":
        """The same routing law and placement at fewer tokens / plans."""
        return replace(
            self,
            tokens_per_rank=self.tokens_per_rank if tokens_per_rank is None else tokens_per_rank,
            layers=self.layers if layers is None else layers,
            microbatches=self.microbatches if microbatches is None else microbatches,
        )


def contiguous_native_counts(num_experts: int, num_ranks: int) -> Tuple[int, ...]:
    """Experts per rank for a contiguous split: the first E mod R ranks get one more."""
    q, m = divmod(num_experts, num_ranks)
    return tuple(q + (1 if r < m else 0) for r in range(num_ranks))


def spread_spares(num_spare: int, num_ranks: int) -> Tuple[int, ...]:
    """Spare slots per rank when only the total is fixed: the first S mod R ranks get one more."""
    q, m = divmod(num_spare, num_ranks)
    return tuple(q + (1 if r < m else 0) for r in range(num_ranks))


def _tiny() -> Workload:
    E, R, per_rank = 12, 8, 2
    nat = contiguous_native_counts(E, R)
    spare = tuple(per_rank - n for n in nat)
    return Workload("tiny", 0, E, 2, R, 32, 1, 2, nat, spare, (64, 32),
                    "zipf_perm_layer", (("s", 1.2),))


def _qwen3() -> Workload:
    E, R = 128, 64
    return Workload("qwen3_235b", 1, E, 8, R, 8192, 1, 94,
                    contiguous_native_counts(E, R), (1,) * R, (3, 4096, 1536),
                    "dirichlet", (("alpha", 0.3),))


def _dsv3() -> Workload:
    E, R = 256, 64
    return Workload("deepseek_v3", 2, E, 8, R, 4096, 1, 58,
                    contiguous_native_counts(E, R), spread_spares(32, R), (3, 7168, 2048),
                    "grouped_lognormal", (("groups", 8), ("topk_groups", 4), ("sigma", 1.5)))


def _glm() -> Workload:
    E, R = 160, 40
    return Workload("glm_4_5", 3, E, 8, R, 16384, 1, 92,
                    contiguous_native_counts(E, R), (1,) * R, (3, 5120, 1536),
                    "dirichlet_hot", (("alpha", 0.1), ("hot_frac", 0.02), ("boost", 10.0)))


def _stress() -> Workload:
    E, R = 384, 64
    return Workload("stress", 4, E, 8, R, 8192, 64, 4,
                    contiguous_native_counts(E, R), (2,) * R, (3, 4096, 2048),
                    "zipf_perm_microbatch", (("s", 1.5),))


WORKLOADS = {w.name: w for w in (_tiny(), _qwen3(), _dsv3(), _glm(), _stress())}
WORKLOAD_ORDER = ("tiny", "qwen3_235b", "deepseek_v3", "glm_4_5", "stress")


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------------------
# seeding
# ---------------------------------------------------------------------------
def _seed_seq(*path: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([SEED_ROOT, *[int(p) for p in path]])


def _torch_gen(ss: np.random.SeedSequence, device: torch.device) -> torch.Generator:
    seed = int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _zipf_over_perm(rng: np.random.Generator, E: int, s: float) -> np.ndarray:
    perm = rng.permutation(E)
    p = np.empty(E, dtype=np.float64)
    p[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def _plan_probs(wl: Workload, mb: int, layer: int) -> np.ndarray:
    """Per-plan expert probabilities (or biases for the grouped law)."""
    E = wl.num_experts
    if wl.law == "zipf_perm_microbatch":
        # the hot set is reshuffled per microbatch and shared by its layers
        return _zipf_over_perm(np.random.default_rng(_seed_seq(wl.index, mb)), E, wl.param("s"))
    rng = np.random.default_rng(_seed_seq(wl.index, mb, layer))
    if wl.law == "zipf_perm_layer":
        return _zipf_over_perm(rng, E, wl.param("s"))
    if wl.law == "dirichlet":
        return rng.dirichlet(np.full(E, wl.param("alpha")))
    if wl.law == "dirichlet_hot":
        p = rng.dirichlet(np.full(E, wl.param("alpha")))
        hot = rng.choice(E, size=int(round(wl.param("hot_frac") * E)), replace=False)
        p[hot] *= wl.param("boost")
        return p / p.sum()
    if wl.law == "grouped_lognormal":
        return rng.lognormal(0.0, wl.param("sigma"), size=E)   # additive expert bias
    raise ValueError(f"unknown routing law {wl.law}")


def _gumbel(shape, gen, device) -> torch.Tensor:
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    u.clamp_(min=1e-20, max=1.0 - 1e-7)
    return -torch.log(-torch.log(u))


def _plan_ids(wl: Workload, mb: int, layer: int, tokens: int, device: torch.device) -> torch.Tensor:
    """Top-k IDs of one plan as int32 [tokens * k] (token-major, k-minor)."""
    E, k = wl.num_experts, wl.top_k
    gen = _torch_gen(_seed_seq(wl.index, mb, layer, 1), device)
    probs = _plan_probs(wl, mb, layer)
    if wl.law == "grouped_lognormal":
        G, TG = int(wl.param("groups")), int(wl.param("topk_groups"))
        bias = torch.tensor(probs, dtype=torch.float32, device=device)
        gscore = torch.randn((tokens, G), generator=gen, device=device)
        top_groups = torch.topk(gscore, TG, dim=1).indices                     # [t, TG]
        allowed = torch.zeros((tokens, G), dtype=torch.bool, device=device)
        allowed.scatter_(1, top_groups, True)
        escore = torch.randn((tokens, E), generator=gen, device=device) + bias
        allowed_e = allowed.repeat_interleave(E // G, dim=1)
        escore.masked_fill_(~allowed_e, float("-inf"))
        ids = torch.topk(escore, k, dim=1).indices
    else:
        logp = torch.tensor(np.log(np.maximum(probs, 1e-30)), dtype=torch.float32, device=device)
        keys = _gumbel((tokens, E), gen, device) + logp
        ids = torch.topk(keys, k, dim=1).indices
    return ids.to(torch.int32).reshape(-1)


def make_ids(wl: Workload, device="cpu", plans: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Gate output for the workload: int32 tensor [P][R*T*k] in (rank, token, k) order.

    ``plans`` selects plan indices (plan = microbatch * layers + layer); the
    default is every plan of the workload.  The global token order is rank-major,
    so the flat index of a (rank, token, k) pair is ``(rank*T + token)*k + k_index``.
    """
    device = torch.device(device)
    if plans is None:
        plans = range(wl.num_plans)
    plans = list(plans)
    out = torch.empty((len(plans), wl.pairs_per_plan), dtype=torch.int32, device=device)
    tokens = wl.num_ranks * wl.tokens_per_rank
    for i, p in enumerate(plans):
        mb, layer = divmod(p, wl.layers)
        out[i] = _plan_ids(wl, mb, layer, tokens, device)
    return out


def inject_invalid(ids: torch.Tensor, num_experts: int, frac_pad: float, frac_bad: float,
                   seed: int = 7) -> torch.Tensor:
    """Return a copy with a seeded fraction of padding (-1) and out-of-range (>= E) IDs."""
    rng = np.random.default_rng(_seed_seq(99, seed))
    flat = ids.detach().to("cpu").clone().reshape(-1)
    n = flat.numel()
    if n:
        npad, nbad = int(frac_pad * n), int(frac_bad * n)
        pos = rng.permutation(n)[: npad + nbad]
        vals = np.concatenate([
            -rng.integers(1, 4, size=npad),
            num_experts + rng.integers(0, 5, size=nbad),
        ]).astype(np.int32)
        flat[torch.from_numpy(pos.astype(np.int64))] = torch.from_numpy(vals)
    return flat.reshape(ids.shape).to(ids.device)


def make_weights(wl: Workload, device="cpu", num_experts: Optional[int] = None,
                 elems_per_expert: Optional[int] = None) -> torch.Tensor:
    """bf16 N(0,1) weights of one MoE layer: [E][elements of one expert].

    One layer's weights stand in for every layer (each layer's slot fill reads
    the same source), which keeps device memory at one layer's footprint.
    """
    device = torch.device(device)
    E = wl.num_experts if num_experts is None else num_experts
    n = int(np.prod(wl.expert_shape)) if elems_per_expert is None else elems_per_expert
    gen = _torch_gen(_seed_seq(wl.index, 0xBEEF), device)
    return torch.randn((E, n), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16) \
        if E * n <= (1 << 26) else _randn_bf16_chunked(E, n, gen, device)


def _randn_bf16_chunked(E: int, n: int, gen, device) -> torch.Tensor:
    out = torch.empty((E, n), dtype=torch.bfloat16, device=device)
    for e in range(E):
        out[e] = torch.randn((n,), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def random_layout(rng: np.random.Generator, max_experts: int = 12, max_ranks: int = 8,
                  max_spare_per_rank: int = 3) -> Tuple[int, int, np.ndarray, np.ndarray, np.ndarray]:
    """A small random placement: (E, R, native_count[R], native_experts[E], spare_count[R]).

    Every rank hosts at least one native expert; native experts are a random
    permutation split into per-rank blocks, each block listed in ascending order.
    """
    R = int(rng.integers(1, max_ranks + 1))
    E = int(rng.integers(R, max(R, max_experts) + 1))
    cuts = np.sort(rng.choice(np.arange(1, E), size=R - 1, replace=False)) if R > 1 else np.array([], int)
    counts = np.diff(np.concatenate([[0], cuts, [E]])).astype(np.int32)
    perm = rng.permutation(E).astype(np.int32)
    blocks, off = [], 0
    for c in counts:
        blocks.append(np.sort(perm[off:off + c]))
        off += c
    spare = rng.integers(0, max_spare_per_rank + 1, size=R).astype(np.int32)
    return E, R, counts, np.concatenate(blocks).astype(np.int32), spare
