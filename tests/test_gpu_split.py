"""GPU parity of sequence splitting (kda_fwd_split / gdn_fwd_split and the
automatic choice of kda_fwd) against the fp64 oracle, in the regimes of the
transition bound: a segment that forgets its entering state within a few
chunks (the transition is skipped and the first pass runs only the decay
window), one that forgets it within part of the segment, one that keeps it
(the transition is computed and applied by the scan) and no decay at all."""
import pytest
import torch

from chunked_gated_delta_kda_amd import inputs
from parity_util import assert_close, check_parity, gpu_run, say, to64

pytestmark = pytest.mark.gpu

CASES = [
    # name, workload, segment_chunks
    ("slow decay: transitions applied",
     lambda: inputs.kda_workload(1, 4000, 2, 128, 128, seed=6000, dt_bias_value=-6.0,
                                 init_std=0.05, name="split_slow"), 16),
    ("default decay: transitions negligible",
     lambda: inputs.kda_workload(2, 3000, 2, 128, 128, seed=6100, init_std=0.05,
                                 name="split_fast"), 16),
    ("medium decay: decay window shorter than the segment",
     lambda: inputs.kda_workload(1, 3000, 2, 128, 128, seed=6150, dt_bias_value=-2.0,
                                 init_std=0.05, name="split_medium"), 16),
    ("no decay",
     lambda: inputs.kda_workload(1, 1500, 2, 128, 128, seed=6200, g_mean=-20.0, g_std=1.0,
                                 init_std=0.05, name="split_nodecay"), 8),
    ("K=V=64, segments of one chunk",
     lambda: inputs.kda_workload(1, 700, 3, 64, 64, seed=6300, dt_bias_value=-6.0,
                                 init_std=0.05, name="split_k64"), 1),
    ("K=128 V=64",
     lambda: inputs.kda_workload(1, 1200, 2, 128, 64, seed=6350, dt_bias_value=-6.0,
                                 init_std=0.05, name="split_v64"), 4),
    ("varlen with empty and short sequences",
     lambda: inputs.kda_workload(1, 0, 2, 128, 128, seed=6400, dt_bias_value=-6.0,
                                 init_std=0.05, lengths=[0, 1000, 5, 3000, 33],
                                 name="split_varlen"), 8),
    ("GDN slow decay",
     lambda: inputs.gdn_workload(1, 3000, 2, 128, 128, seed=6500, init_std=0.05,
                                 decay_shift=-6.0, name="split_gdn"), 16),
]


@pytest.mark.parametrize("name,make,seg", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle(name, make, seg):
    w = make()
    say(f"[split] {name}: segment_chunks={seg}")
    check_parity(w, first_tokens=32, segment_chunks=seg)


def test_split_equals_unsplit():
    """Split and unsplit runs agree to rounding (every segment boundary inside
    the sequence, slow decay so every boundary carries state)."""
    w = inputs.kda_workload(1, 2500, 2, 128, 128, seed=6600, dt_bias_value=-6.0, init_std=0.05)
    o1, S1 = gpu_run(w, segment_chunks=-1)
    o2, S2 = gpu_run(w, segment_chunks=8)
    assert_close("o split vs unsplit", to64(o2), to64(o1))
    assert_close("state split vs unsplit", to64(S2), to64(S1))


def test_automatic_split_long_sequence():
    """kda_fwd splits on its own for one long sequence with few heads."""
    w = inputs.kda_workload(1, 16384, 2, 128, 128, seed=6700, dt_bias_value=-6.0,
                            init_std=0.05, name="auto_split_T16384_H2")
    check_parity(w, first_tokens=32)


def test_split_deterministic():
    w = inputs.kda_workload(1, 2000, 2, 128, 128, seed=6800, dt_bias_value=-6.0, init_std=0.05)
    o1, S1 = gpu_run(w, segment_chunks=4)
    o2, S2 = gpu_run(w, segment_chunks=4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
