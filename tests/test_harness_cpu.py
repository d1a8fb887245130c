"""CPU checks of the GPU tests' comparison helpers: the per-(sequence, head)
and per-chunk maxima catch a localised error that the whole-tensor relative
Frobenius norm lets through."""
import numpy as np
import pytest

from kda_harness import LOCAL_CHUNK, assert_close, local_errors, state_pair_errors


def _pair(T, H=4, cols=8, noise=1e-3, seed=0):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal((T, H, cols))
    x = ref * (1.0 + noise * rng.standard_normal(ref.shape))
    return x, ref


def test_one_corrupted_row_in_a_long_sequence_fails_the_chunk_maximum():
    T = 131072
    x, ref = _pair(T)
    x[77777, 2] = -ref[77777, 2]        # one token row of one head with the sign flipped
    whole = np.linalg.norm(x - ref) / np.linalg.norm(ref)
    assert whole < 5e-3                 # the whole-tensor norm alone would pass
    pair, chunk = local_errors(x, ref, [0, T])
    assert pair.shape == (1, 4) and chunk.shape == (T // LOCAL_CHUNK, 4)
    assert chunk.max() > 0.1 and np.argmax(chunk[:, 2]) == 77777 // LOCAL_CHUNK
    with pytest.raises(AssertionError):
        assert_close(x, ref, None, None, [0, T], 5e-3)


def test_chunks_start_at_each_sequence_and_skip_empty_ones():
    cu = [0, 100, 100, 165, 166]        # lengths 100, 0, 65, 1
    x, ref = _pair(166, H=2)
    pair, chunk = local_errors(x, ref, cu)
    assert pair.shape == (3, 2)         # the empty sequence has no rows
    assert chunk.shape == (2 + 0 + 2 + 1, 2)
    x[164, 1] += 10.0                   # second chunk of the third sequence (its token 64)
    pair, chunk = local_errors(x, ref, cu)
    # pair rows are the non-empty sequences 0, 2, 3: sequence 2 is row 1
    assert np.argmax(chunk[:, 1]) == 3 and np.argmax(pair[:, 1]) == 1


def test_state_pairs_are_compared_one_by_one():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((3, 5, 16, 16))
    fs = ref.copy()
    fs[2, 4, 0, 0] += 3.0
    err = state_pair_errors(fs, ref)
    assert err.shape == (3, 5) and np.argmax(err) == 2 * 5 + 4
    assert np.count_nonzero(err) == 1


def test_exact_zero_reference_reports_the_absolute_error():
    ref = np.zeros((64, 1, 4))
    x = np.full_like(ref, 1e-9)
    pair, chunk = local_errors(x, ref, [0, 64])
    assert np.allclose(pair, np.sqrt(64 * 4) * 1e-9)
