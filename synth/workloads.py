"""The five synthetic workloads: shapes, value recipes and seed streams.

Shapes borrow the LLaMA models the ReSpinQuant pages evaluate (technical
summary, "Results" section: LLaMA-2 7B/13B, LLaMA-3 8B, LLaMA-3.2 1B/3B); the
outlier channels stand in for the large activation outliers described in
each page's "Problem" section. No dataset or trained weight is used.

Seed streams (``numpy.random.SeedSequence([seed_id, stream])``):
  0 residual h, 3 outlier channel indices,
  1/2 site-A skew generators (in/out), 13/14 site-B skew generators (in/out),
  4..10 weights q, k, v, o, gate, up, down,
  11 o_proj input stand-in, 12 down_proj input stand-in,
  15/16 site-A and 17/18 site-B low-rank skew factors (in/out; the rank sweep's
  low-rank mismatch only).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str                # model, phase and bit widths
    seed_id: int             # seed family (the decode workload reuses the prefill one)
    D: int                   # hidden size (residual width)
    F: Optional[int]         # FFN width (None: single-linear block)
    r: int                   # headline subspace rank
    n: int                   # tokens in the batch
    bits: int                # weight and activation bit width (4 or 3)
    h_dtype: str             # residual storage dtype: "bf16" or "f32"
    y_dtype: str             # linear output dtype: "bf16" or "f32"
    eps_rot: float           # Cayley step size of the synthetic rotations
    n_outliers: int          # outlier channel count
    outlier_scale: float
    sigma_w: float           # weight standard deviation
    kv: Optional[int] = None         # k/v projection width (GQA); None = same as D (MHA)
    ranks: Tuple[int, ...] = ()      # ranks swept for the accuracy/throughput curve
    decode_batches: Tuple[int, ...] = ()
    single_linear: Optional[Tuple[int, int]] = None  # (N, K) of the one linear of a tiny block


TINY = "tiny-d256-r8"                       # one 256 x 256 linear, 16 tokens
LLAMA2_7B_PREFILL = "llama2-7b-prefill-w4a4"  # D 4096, FFN 11008, 2048 tokens
LLAMA2_7B_DECODE = "llama2-7b-decode-w4a4"    # D 4096, FFN 11008, 1 to 64 tokens
LLAMA3_8B_W3A3 = "llama3-8b-prefill-w3a3"     # D 4096, FFN 14336, k/v 1024, 4096 tokens
LLAMA2_70B_PREFILL = "llama2-70b-prefill-w4a4"  # D 8192, FFN 28672, k/v 1024, 4096 tokens

WORKLOADS = {w.name: w for w in (
    Workload(TINY, 1, D=256, F=None, r=8, n=16, bits=4, h_dtype="f32",
             y_dtype="f32", eps_rot=0.02, n_outliers=4, outlier_scale=40.0, sigma_w=0.02,
             single_linear=(256, 256)),
    Workload(LLAMA2_7B_PREFILL, 2, D=4096, F=11008, r=32, n=2048, bits=4,
             h_dtype="bf16", y_dtype="bf16", eps_rot=0.01, n_outliers=20,  # 0.5% of 4096
             outlier_scale=50.0, sigma_w=0.02, kv=None),
    Workload(LLAMA2_7B_DECODE, 2, D=4096, F=11008, r=32, n=64, bits=4,
             h_dtype="bf16", y_dtype="bf16", eps_rot=0.01, n_outliers=20,
             outlier_scale=50.0, sigma_w=0.02, kv=None, decode_batches=(1, 8, 64)),
    Workload(LLAMA3_8B_W3A3, 4, D=4096, F=14336, r=32, n=4096, bits=3,
             h_dtype="bf16", y_dtype="bf16", eps_rot=0.01, n_outliers=41,  # 1% of 4096
             outlier_scale=30.0, sigma_w=0.02, kv=1024, ranks=(8, 16, 32, 64)),
    Workload(LLAMA2_70B_PREFILL, 5, D=8192, F=28672, r=32, n=4096, bits=4,
             h_dtype="bf16", y_dtype="bf16", eps_rot=0.01, n_outliers=25,  # 0.3% of 8192
             outlier_scale=60.0, sigma_w=0.01, kv=1024),
)}


def workload(key) -> Workload:
    """A workload by name, or by its 1-based position in WORKLOADS."""
    if isinstance(key, Workload):
        return key
    if isinstance(key, int) or (isinstance(key, str) and key.isdigit()):
        names = list(WORKLOADS)
        i = int(key)
        if not 1 <= i <= len(names):
            raise KeyError(f"no workload at position {i}; positions 1..{len(names)}")
        return WORKLOADS[names[i - 1]]
    if key not in WORKLOADS:
        raise KeyError(f"unknown workload {key!r}; known: {', '.join(WORKLOADS)}")
    return WORKLOADS[key]


# weight name -> seed stream
WEIGHT_STREAMS = {"q": 4, "k": 5, "v": 6, "o": 7, "gate": 8, "up": 9, "down": 10, "proj": 4}
SKEW_STREAMS = {("A", "in"): 1, ("A", "out"): 2, ("B", "in"): 13, ("B", "out"): 14}
LOW_RANK_STREAMS = {("A", "in"): 15, ("A", "out"): 16, ("B", "in"): 17, ("B", "out"): 18}
INPUT_STREAMS = {"o_in": 11, "down_in": 12}


@dataclass(frozen=True)
class Linear:
    name: str                # "qkv", "o", "gate_up", "down" or "proj"
    N: int                   # output channels
    K: int                   # reduction width
    source: str              # what feeds it: "siteA", "siteB", "o_in", "down_in"
    parts: Tuple[Tuple[str, int], ...] = field(default=())  # stacked weights (name, rows)


def layer_linears(cfg: Workload, gqa: bool = True):
    """The linears of one decoder layer in execution order.

    Site A (attention input) feeds the fused q|k|v projection, the o_proj
    input is a stand-in, site B (FFN input) feeds the fused gate|up
    projection and the down_proj input is a stand-in.
    """
    if cfg.single_linear is not None:
        N, K = cfg.single_linear
        return [Linear("proj", N, K, "siteA", (("proj", N),))]
    D, F = cfg.D, cfg.F
    kv = cfg.kv if (gqa and cfg.kv is not None) else D
    return [
        Linear("qkv", D + 2 * kv, D, "siteA", (("q", D), ("k", kv), ("v", kv))),
        Linear("o", D, D, "o_in", (("o", D),)),
        Linear("gate_up", 2 * F, D, "siteB", (("gate", F), ("up", F))),
        Linear("down", D, F, "down_in", (("down", D),)),
    ]
