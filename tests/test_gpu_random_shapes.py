"""GPU parity on seeded random draws of the forward pass's configuration space:
kind (KDA / GDN), head dimensions, fixed or packed lengths (empty, one-token,
ragged and multi-chunk sequences), head counts, decay regime (fast, default,
slow, clamp-active for KDA), initial state or none, and segment length
(automatic, whole sequences, or an explicit number of chunks, so that warm-up
attempts, retries and restarts all occur).  Each draw is checked against the
fp64 oracle within the acceptance bounds.  The draws are fixed by their seeds,
so a failure names a reproducible case."""
import numpy as np
import pytest

from chunked_gated_delta_kda_amd import inputs
from parity_util import check_parity, say

pytestmark = pytest.mark.gpu

N_DRAWS = 96


def draw(i):
    """Configuration i (a pure function of i)."""
    rng = np.random.default_rng(91000 + i)
    kind = "kda" if i % 3 else "gdn"
    K = int(rng.choice([64, 128]))
    V = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 7))
    packed = bool(rng.integers(0, 2))
    init = float(rng.choice([0.0, 0.05]))
    seg = int(rng.choice([0, -1, 1, 3, 8]))
    regime = str(rng.choice(["default", "slow", "fast", "clamp"] if kind == "kda"
                            else ["default", "slow", "fast"]))
    if packed:
        n = int(rng.integers(1, 7))
        lengths = [int(x) for x in rng.integers(0, 700, size=n)]
        lengths[int(rng.integers(0, n))] = int(rng.choice([0, 1, 31, 32, 33]))
        B, T = 1, 0
    else:
        lengths = None
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 900))
    seed = 92000 + i
    name = f"rand{i}_{kind}_K{K}_V{V}_H{H}_{regime}_seg{seg}"
    common = dict(init_std=init if init > 0 else None, lengths=lengths, name=name)
    if kind == "kda":
        extra = {"default": {}, "slow": {"dt_bias_value": -6.0},
                 "fast": {"dt_bias_value": 2.0}, "clamp": {"g_mean": 8.0, "g_std": 1.0}}[regime]
        w = inputs.kda_workload(B, T, H, K, V, seed, **common, **extra)
    else:
        shift = {"default": 0.0, "slow": -6.0, "fast": 2.0}[regime]
        w = inputs.gdn_workload(B, T, H, K, V, seed, decay_shift=shift, **common)
    return w, (None if seg == 0 else seg)


@pytest.mark.parametrize("i", range(N_DRAWS))
def test_random_configuration(i):
    w, seg = draw(i)
    say(f"[random] draw {i}: segment_chunks={seg} lengths="
        f"{None if w.cu_seqlens is None else (w.cu_seqlens[1:] - w.cu_seqlens[:-1]).tolist()}")
    kw = {} if seg is None else {"segment_chunks": seg}
    check_parity(w, first_tokens=32, **kw)
