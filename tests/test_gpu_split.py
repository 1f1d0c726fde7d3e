"""GPU parity of sequence splitting against the fp64 oracle, for both forward
paths:

  staged (kda_fwd_split / gdn_fwd_split): segments run from a zero state, a
    scan over the segment transitions carries the state across them; a
    transition whose bound shows it negligible is skipped and the first pass
    then runs only the decay window;
  fused (kda_fwd_segmented / gdn_fwd_segmented and the automatic choice of
    kda_fwd): a segment starts one chunk early from a zero state and keeps
    that start only if the bound of that chunk's transitions is below 2^-24;
    else it tries four chunks early, and else it restarts from the sequence
    start.

The cases cover the regimes of both bounds: state forgotten within one chunk
(default decay), within four (the fused segments' second attempt holds),
within part of a segment, kept across segments (slow decay: the staged scan
applies transitions, the fused segments restart) and no decay at all."""
import numpy as np
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
    ("faster decay: one warm-up chunk too short, four enough",
     lambda: inputs.kda_workload(1, 3000, 2, 128, 128, seed=6160, dt_bias_value=-1.0,
                                 init_std=0.05, name="split_retry"), 16),
    ("GDN: one warm-up chunk too short, four enough",
     lambda: inputs.gdn_workload(1, 3000, 2, 128, 128, seed=6510, init_std=0.05,
                                 decay_shift=-1.5, name="split_gdn_retry"), 16),
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


PATHS = ["fused", "staged"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name,make,seg", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle(name, make, seg, path):
    w = make()
    say(f"[split] {name}: path={path} segment_chunks={seg}")
    check_parity(w, first_tokens=32, segment_chunks=seg, path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dt_bias", [-6.0, 0.0])
def test_split_equals_unsplit(path, dt_bias):
    """Split and unsplit runs agree to rounding (every segment boundary inside
    the sequence; slow decay: every boundary carries state, default decay: the
    fused segments keep their zero start)."""
    w = inputs.kda_workload(1, 2500, 2, 128, 128, seed=6600, dt_bias_value=dt_bias,
                            init_std=0.05)
    o1, S1 = gpu_run(w, path=path, segment_chunks=-1)
    o2, S2 = gpu_run(w, path=path, segment_chunks=8)
    assert_close("o split vs unsplit", to64(o2), to64(o1))
    assert_close("state split vs unsplit", to64(S2), to64(S1))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dt_bias", [-6.0, 0.0])
def test_automatic_split_long_sequence(path, dt_bias):
    """The automatic choice splits one long sequence with few heads on its own."""
    w = inputs.kda_workload(1, 16384, 2, 128, 128, seed=6700, dt_bias_value=dt_bias,
                            init_std=0.05, name=f"auto_split_T16384_H2_dt{dt_bias:g}")
    check_parity(w, first_tokens=32, path=path)


@pytest.mark.parametrize("path", PATHS)
def test_split_deterministic(path):
    w = inputs.kda_workload(1, 2000, 2, 128, 128, seed=6800, dt_bias_value=-6.0, init_std=0.05)
    o1, S1 = gpu_run(w, path=path, segment_chunks=4)
    o2, S2 = gpu_run(w, path=path, segment_chunks=4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("seg", [1, 2, 3, 4, 5])
def test_fused_segments_short_and_warm_up(seg):
    """Fused segments shorter than, equal to and longer than the warm-up
    chunks of either attempt, on a ragged packed batch, default decay (the zero start is kept)
    and GDN; every segment's outputs and the final states checked."""
    lengths = [0, 31, 32, 33, 200, 7, 513, 96]
    w = inputs.kda_workload(1, 0, 3, 128, 128, seed=6900 + seg, init_std=0.05,
                            lengths=lengths, name=f"fused_seg{seg}_packed")
    check_parity(w, first_tokens=32, segment_chunks=seg)
    w = inputs.gdn_workload(2, 300, 2, 64, 128, seed=6950 + seg, init_std=0.05,
                            name=f"fused_seg{seg}_gdn")
    check_parity(w, first_tokens=32, segment_chunks=seg)


@pytest.mark.parametrize("seg", [None, 1])
def test_fused_many_packed_sequences(seg):
    """Three hundred packed sequences of 0..70 tokens (zeros included): many
    more segments than compute units, most of them one or two chunks, so the
    segment table, its longest-first order and the per-sequence final states
    are exercised at scale; KDA and GDN."""
    rng = np.random.default_rng(7100)
    lengths = rng.integers(0, 71, size=300).tolist()
    lengths[:3] = [0, 0, 1]
    w = inputs.kda_workload(1, 0, 2, 64, 64, seed=7101, init_std=0.05, lengths=lengths,
                            name="fused_many_packed_kda")
    kw = {} if seg is None else {"segment_chunks": seg}
    check_parity(w, first_tokens=32, **kw)
    w = inputs.gdn_workload(1, 0, 2, 64, 64, seed=7102, init_std=0.05, lengths=lengths,
                            name="fused_many_packed_gdn")
    check_parity(w, first_tokens=32, **kw)


def test_fused_segments_beyond_sort_buckets():
    """Segments of 1100 chunks: more than the 1024 length buckets of the
    longest-first sort (the longest share its last bucket), on two sequences
    of over 33,000 tokens around a short one."""
    lengths = [33000, 5, 34000]
    w = inputs.kda_workload(1, 0, 1, 64, 64, seed=7200, init_std=0.05, lengths=lengths,
                            name="fused_long_segments")
    check_parity(w, first_tokens=32, segment_chunks=1100)
