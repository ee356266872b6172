"""The five synthetic workloads the fused norm + FC step is checked and timed on.

Shapes follow the serving situations the pages describe:

* decode: a handful of live sequences times a few draft tokens per verify
  round (concurrency 1..16 in the vLLM EAGLE 3.1 release post,
  devlery.com/blog/vllm-eagle31-attention-drift, first section);
* long-context prefill: the >=32K contexts where the EAGLE 3.1 explainer
  (llm-wiki.hwlabs.dev/study/dist/ai-frontier/76.html, section on long-context
  performance) places the acceptance-length gain;
* the hidden-state magnitude growth with depth (low < mid < high) that the
  explainer's section on EAGLE-3's multi-layer fusion gives as the reason for
  normalising each state.

No dataset is involved: the real hidden states would need trained target
weights, which are not available; seeded Gaussian draws with per-state scales,
per-channel offsets and outlier channels stand in for them.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

NORM_NONE = 0
NORM_LN = 1
NORM_RMS = 2

NORM_NAMES = {NORM_NONE: "none", NORM_LN: "layernorm", NORM_RMS: "rmsnorm"}


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    d: int
    Ms: Tuple[int, ...]
    # (norm_kind, eps) pairs this workload is run with
    norms: Tuple[Tuple[int, float], ...]
    # per-state scale of the N(0,1) part: low, mid, high
    scales: Tuple[float, float, float]
    # std of the per-channel offset shared by all tokens: low, mid, high
    offset_std: Tuple[float, float, float] = (0.5, 0.5, 0.5)
    # number of outlier channels per state and their multiplier
    n_outliers: int = 0
    outlier_mult: float = 1.0
    has_beta: bool = True
    has_bias: bool = True
    gamma_mean: float = 1.0
    gamma_std: float = 0.1
    beta_std: float = 0.05
    bias_std: float = 0.01

    @property
    def seed(self) -> int:
        return 20260526 + self.cfg_id

    @property
    def max_M(self) -> int:
        return max(self.Ms)

    @property
    def w_std(self) -> float:
        return (3 * self.d) ** -0.5


CONFIGS = {
    1: Workload(1, "tiny_ln", 512, (64,), ((NORM_LN, 1e-5),), (1.0, 4.0, 16.0)),
    2: Workload(2, "decode_ln_d4096", 4096, (1, 4, 8, 16, 64), ((NORM_LN, 1e-5),), (1.0, 4.0, 16.0)),
    3: Workload(3, "tree_rms_d5120", 5120, (64, 128, 256), ((NORM_RMS, 1e-6),), (1.0, 6.0, 24.0),
                has_beta=False, has_bias=False),
    4: Workload(4, "prefill_ln_d7168_M32768", 7168, (32768,), ((NORM_LN, 1e-5),), (1.0, 4.0, 16.0),
                n_outliers=8, outlier_mult=20.0),
    5: Workload(5, "chunked_prefill_d8192", 8192, (512, 2048, 4093, 4096),
                ((NORM_LN, 1e-5), (NORM_RMS, 1e-6)), (1.0, 8.0, 32.0), offset_std=(0.5, 0.5, 2.0)),
}


def workload(cfg_id: int) -> Workload:
    return CONFIGS[cfg_id]


def algorithmic_bytes(d: int, M: int, has_bias: bool = True, n_param_vecs: int = 6) -> int:
    """Bytes the step must move at least once: W, the three hidden states,
    the output, and the bf16 parameter vectors (gamma/beta per state, bias)."""
    w = 3 * d * d * 2
    h = 3 * M * d * 2
    out = M * d * 2
    params = (n_param_vecs + (1 if has_bias else 0)) * d * 2
    return w + h + out + params


def algorithmic_flops(d: int, M: int) -> int:
    """Dense contraction flops of the FC: 2 * M * 3d * d."""
    return 2 * M * 3 * d * d


def param_vec_count(norm_kind: int, has_beta: bool) -> int:
    if norm_kind == NORM_LN:
        return 3 + (3 if has_beta else 0)
    if norm_kind == NORM_RMS:
        return 3
    return 0


def describe(w: Workload, M: Optional[int] = None) -> str:
    Mtxt = M if M is not None else "/".join(str(m) for m in w.Ms)
    norms = "+".join(f"{NORM_NAMES[k]}(eps={e:g})" for k, e in w.norms)
    return f"cfg{w.cfg_id} {w.name}: d={w.d} M={Mtxt} {norms}"
