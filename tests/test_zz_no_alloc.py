"""kda_fwd_noalloc (the entry point that allocates nothing: packed-batch
tables in the library's per-GPU scratch array) against kda_fwd on the same
inputs, through the C ABI.  Two calls in a row share the array, the second
with a smaller batch, so a table left by the first call must not leak into
the second.  Same kernels and plan as kda_fwd: outputs and final states must
be bitwise equal (a fortiori within the forward pass's parity bounds)."""
import pytest
import torch

import chunked_gated_delta_kda_amd as kda
from chunked_gated_delta_kda_amd import inputs
from parity_util import assert_close, say, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def both(w):
    d = w.to(DEV)
    o_ref, s_ref = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                               d["dt_bias"], w.lower_bound, w.scale, d["initial_state"], True,
                               d["cu_seqlens"])
    out = torch.full_like(o_ref, float("nan"))
    fin = torch.full_like(s_ref, float("nan"))
    kda.kda_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], out,
                        fin, w.lower_bound, w.scale, d["initial_state"], d["cu_seqlens"])
    torch.cuda.synchronize()
    say(f"[noalloc] {w.name}: B={w.B} T={w.T} H={w.H} N={w.n_seqs}")
    assert_close("o noalloc vs kda_fwd", to64(out), to64(o_ref))
    assert_close("state noalloc vs kda_fwd", to64(fin), to64(s_ref))
    assert torch.equal(out, o_ref) and torch.equal(fin, s_ref)


def test_noalloc_equals_kda_fwd_two_calls_second_smaller():
    # packed: 9 sequences (one empty, several ragged), then 3 shorter ones
    both(inputs.kda_workload(1, 0, 4, 128, 128, seed=8100, init_std=0.05,
                             lengths=[700, 0, 33, 1500, 64, 5, 900, 257, 1200],
                             name="noalloc_packed_9"))
    both(inputs.kda_workload(1, 0, 2, 128, 128, seed=8101, init_std=0.05, lengths=[40, 300, 1],
                             name="noalloc_packed_3"))


def test_noalloc_fixed_length_and_k64():
    both(inputs.kda_workload(2, 333, 3, 128, 128, seed=8200, init_std=0.05, name="noalloc_fixed"))
    both(inputs.kda_workload(1, 0, 2, 64, 64, seed=8201, lengths=[100, 7, 64],
                             name="noalloc_packed_k64"))
