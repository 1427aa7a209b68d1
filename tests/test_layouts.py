"""The page layouts the tests gather codes by: each maps the 16 tokens x 128
channels of a page-head block one-to-one onto its bytes (or 16-bit words)."""
import numpy as np

from tests import helpers as H


def _covers(fn, shape):
    idx = np.arange(int(np.prod(shape))).reshape((1, 1, 1) + shape)
    got = fn(idx, 0, np.zeros(1, dtype=np.int64), 16, 0)
    assert got.shape == (16, 128)
    assert np.array_equal(np.sort(got.ravel()), np.arange(16 * 128))


def test_code_layouts_are_bijections():
    _covers(H.gather_k_codes, (2, 4, 16, 16))
    _covers(H.gather_v_codes, (2, 4, 16, 4, 4))
    _covers(H.gather_k_bf16, (4, 4, 16, 8))
    _covers(H.gather_v_bf16, (4, 4, 16, 2, 4))


def test_value_word_holds_four_tokens_of_one_channel():
    # the decode reads one 32-bit word per (channel, 4 tokens): bytes t % 4 of
    # a word are consecutive tokens of the same channel
    idx = np.arange(2048).reshape(1, 1, 1, 2, 4, 16, 4, 4)
    got = H.gather_v_codes(idx, 0, np.zeros(1, dtype=np.int64), 16, 0)
    for t0 in range(0, 16, 4):
        w = got[t0:t0 + 4]                     # [4 tokens, 128 channels]
        assert np.all(w[1:] - w[:-1] == 1) and np.all(w[0] % 4 == 0)
