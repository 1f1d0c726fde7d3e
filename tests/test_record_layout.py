"""CPU check of the record decoder used by the GPU record test: encoding the
chunkwise oracle's matrices in the documented layout (csrc/kda_common.h) and
decoding them again returns them (to bf16 truncation), and every byte of a
record is covered by exactly one matrix entry."""
import numpy as np

from chunked_gated_delta_kda_amd import inputs
from test_gpu_record import C, decode, encode, expected_records, record_size


def test_tok_and_rho_are_permutations():
    from test_gpu_record import rho, tok
    assert sorted(tok(g, e) for g in range(4) for e in range(8)) == list(range(C))
    for K in (64, 128):
        assert sorted(rho(t, r) for t in range(K // 16) for r in range(16)) == list(range(K))


def test_record_roundtrip():
    for K, kind in ((128, "kda"), (64, "kda"), (128, "gdn")):
        if kind == "kda":
            w = inputs.kda_workload(1, 45, 1, K, K, seed=11, dt_bias_value=-2.0)
        else:
            w = inputs.gdn_workload(1, 45, 1, K, K, seed=11)
        recs = expected_records(w, kind)
        assert len(recs) == 2  # one whole and one ragged chunk
        for mats in recs.values():
            raw = encode(mats, K)
            assert raw.size == record_size(K)
            got = decode(raw, K)
            for name in ("nKG", "QG", "Kd", "Aqk", "Tb"):
                ref = mats[name]
                assert np.all(np.abs(got[name] - ref) <= 2 ** -7 * np.abs(ref) + 1e-30), name
            assert np.array_equal(got["GamC"], mats["GamC"].astype(np.float32).astype(np.float64))
