"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins
from oracle.chunked import chunked_forward


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__[4:])
def test_pin(orc, pin):
    pin(orc)


def test_pin_list_is_complete():
    assert len(oracle_pins.ALL_PINS) >= 15


def test_rejects_bad_arguments(orc):
    q = np.zeros((2, 4, 1, 3))
    with pytest.raises(ValueError):  # cu_seqlens needs B == 1
        orc.kda(q, q, q, q, np.zeros((2, 4, 1)), np.zeros(1), np.zeros((1, 3)),
                cu_seqlens=np.array([0, 2, 4]))


def test_chunk_intermediates_are_exact_inverse():
    """The recorded chunk factors satisfy (I + A) T = I with A strictly lower
    triangular, and T is unit lower triangular (nilpotent A)."""
    rng = np.random.default_rng(3)
    B, T, H, K, V = 1, 40, 1, 8, 4
    rec = []
    chunked_forward(rng.standard_normal((B, T, H, K)), rng.standard_normal((B, T, H, K)),
                    rng.standard_normal((B, T, H, V)), rng.normal(0, 1, (B, T, H, K)),
                    rng.standard_normal((B, T, H)), rng.normal(0, .3, H),
                    np.zeros((H, K)), -5.0, None, chunk=16, record=rec)
    assert len(rec) == 3
    for r in rec:
        m = r["A"].shape[0]
        assert np.allclose(np.triu(r["A"]), 0)
        assert np.allclose((np.eye(m) + r["A"]) @ r["T"], np.eye(m), atol=1e-12)
        assert np.allclose(np.diag(r["T"]), 1) and np.allclose(np.triu(r["T"], 1), 0)


def test_page_shapes(orc):
    """Output and state shapes of the pages' usage example (B2 T2048 H32 K=V=128),
    computed on one head to keep the CPU time short."""
    gold = oracle_pins.load_golden("page_shapes.json")
    B, T, H, K, V = (gold[x] for x in "BTHKV")
    rng = np.random.default_rng(0)
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    o, S = orc.kda(q, q, q, q * 0.1, q[..., 0], np.zeros(H), np.zeros((H, K)), heads=[5])
    assert list(o.shape[:2]) + [H] + list(o.shape[3:]) == gold["o_shape"]
    assert [S.shape[0], H] + list(S.shape[2:]) == gold["final_state_shape"]
