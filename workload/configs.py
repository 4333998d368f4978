"""Synthetic H2O workloads: shapes, budgets and the anchor-bias recipe.

This module holds workload *descriptions* only.  It does no attention, scoring
or eviction arithmetic; both the GPU path and the CPU oracle read it.

The shapes follow the model shapes the H2O pages evaluate (OPT-6.7B: 32 heads of
dimension 128; OPT-30B: 56 heads of dimension 128; a LLaMA-7B-shaped streaming run)
and the throughput settings they quote (prompt 512 + 1024 generated, 2048 + 2048
at batch 64, 4 M-token streaming), see the report "H2O: Heavy-Hitter Oracle for
Efficient Generative Inference of Large Language Models — 深度解读报告", §4.3 and
§4.4 (Q1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

#: Root seed of every draw (the arXiv number of the H2O paper).
ROOT_SEED = 230614048


def budget_from_percent(percent: int, prompt_len: int) -> int:
    """Heavy and recent budgets for a total budget of ``percent`` % of the prompt.

    The total is split evenly between the heavy-hitter set and the recent window,
    and each half is rounded *up* so the cache never falls under the requested
    share: ``ceil(percent/200 * prompt_len)``, in exact integer arithmetic.
    This is the reading that gives 26 + 26 = 52 for a 256-token prompt at 20 %
    and 205 per half for a 2048-token prompt at 20 %, the integers the workload
    descriptions print.
    """
    if percent <= 0 or prompt_len < 0:
        raise ValueError("percent must be > 0 and prompt_len >= 0")
    return (percent * prompt_len + 199) // 200


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    A *unit* is one (layer, batch element, head); units are independent.
    ``anchor`` selects how the heavy-hitter-inducing bias is laid out:

    * ``"fixed"``: ``n_anchors`` positions per (layer, sequence), drawn without
      replacement from all ``prompt_len + decode_steps`` positions, get
      ``+alpha * u_h`` on their keys; every query gets ``+u_h``.
    * ``"zipf"``: every position j gets ``+alpha * rho_j**(-zipf_s) * u_h`` on
      its key, with ``rho`` a seeded random permutation of 1..N per sequence.
    * ``"drift"``: ``n_anchors`` prompt anchors with direction ``u^(0)``; then a
      new anchor every ``drift_every`` positions after the prompt, each with a
      fresh direction; queries at position p get the direction of the latest
      anchor epoch at or before p.
    """

    name: str
    cid: int
    layers: int
    batch: int
    heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16": storage type of Q/K/V and of the cached K/V
    prompt_len: int
    decode_steps: int
    heavy_budget: int
    recent_budget: int
    anchor: str = "fixed"
    n_anchors: int = 0
    alpha: float = 3.0
    zipf_s: float = 1.1
    drift_every: int = 10_000
    budget_percent: int | None = None
    notes: str = field(default="", compare=False)

    @property
    def n_positions(self) -> int:
        return self.prompt_len + self.decode_steps

    @property
    def k(self) -> int:
        return self.heavy_budget + self.recent_budget

    @property
    def units_per_layer(self) -> int:
        return self.batch * self.heads

    @property
    def units(self) -> int:
        return self.layers * self.batch * self.heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _ceil_percent(p: int, n: int) -> int:
    return (p * n + 99) // 100


def _make() -> dict[str, Workload]:
    w: dict[str, Workload] = {}
    w["tiny-fp32"] = Workload(
        name="tiny-fp32", cid=0, layers=1, batch=1, heads=1, head_dim=64, dtype="f32",
        prompt_len=256, decode_steps=64,
        heavy_budget=budget_from_percent(20, 256), recent_budget=budget_from_percent(20, 256),
        anchor="fixed", n_anchors=8, budget_percent=20,
        notes="single attention layer, batch 1, one head, d=64, fp32, 8 anchors")
    w["opt6.7b-layer-b16"] = Workload(
        name="opt6.7b-layer-b16", cid=1, layers=1, batch=16, heads=32, head_dim=128, dtype="bf16",
        prompt_len=512, decode_steps=512,
        heavy_budget=budget_from_percent(20, 512), recent_budget=budget_from_percent(20, 512),
        anchor="fixed", n_anchors=_ceil_percent(1, 1024), budget_percent=20,
        notes="OPT-6.7B attention layer, batch 16, 512+512, 20% budget")
    w["opt6.7b-32L-b64"] = Workload(
        name="opt6.7b-32L-b64", cid=2, layers=32, batch=64, heads=32, head_dim=128, dtype="bf16",
        prompt_len=2048, decode_steps=1024,
        heavy_budget=budget_from_percent(20, 2048), recent_budget=budget_from_percent(20, 2048),
        anchor="fixed", n_anchors=_ceil_percent(1, 3072), budget_percent=20,
        notes="OPT-6.7B 32-layer stack of independent attention layers, batch 64, 2048+1024")
    for pct in (4, 10, 20, 100):
        kh = budget_from_percent(pct, 1024) if pct < 100 else 1024
        w[f"opt30b-b128-{pct}pct"] = Workload(
            name=f"opt30b-b128-{pct}pct", cid=3, layers=1, batch=128, heads=56, head_dim=128,
            dtype="bf16", prompt_len=1024, decode_steps=1024,
            heavy_budget=kh, recent_budget=kh, anchor="zipf", budget_percent=pct,
            notes="OPT-30B attention, batch 128, 1024+1024, Zipf(1.1) anchor strength; "
                  "100% keeps N/2 + N/2 so nothing is ever evicted")
    w["llama7b-stream-4m"] = Workload(
        name="llama7b-stream-4m", cid=4, layers=1, batch=1, heads=32, head_dim=128, dtype="bf16",
        prompt_len=512, decode_steps=4_000_000, heavy_budget=1024, recent_budget=1024,
        anchor="drift", n_anchors=_ceil_percent(1, 512), drift_every=10_000,
        notes="LLaMA-7B-shaped streaming, batch 1, 512-token prompt then 4M decode steps, "
              "k = 1024 + 1024, a new anchor every 10k tokens")
    return w


WORKLOADS: dict[str, Workload] = _make()

#: Configuration index -> workload names (index 3 has one entry per budget).
BY_INDEX: dict[int, list[str]] = {}
for _n, _w in WORKLOADS.items():
    BY_INDEX.setdefault(_w.cid, []).append(_n)


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (used for reduced test sizes)."""
    from dataclasses import replace
    return replace(w, **changes)
