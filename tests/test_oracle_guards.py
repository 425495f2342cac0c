"""The oracle's wrapper rejects inputs that would read outside its arrays
(a GPU selection that names an incomplete block, a row past the queries, a
position past the keys) with ValueError instead of passing them to C."""
import numpy as np
import pytest


def _inputs(synth_lib, T=40):
    Q = synth_lib.normal_bf16(1, (T, 24, 256), 2)
    K = synth_lib.normal_bf16(2, (T, 2, 256), 2)
    V = synth_lib.normal_bf16(3, (T, 2, 256), 2)
    return Q, K, V


def test_selection_naming_an_incomplete_block(oracle_lib, synth_lib):
    Q, K, V = _inputs(synth_lib)
    rows = np.array([9])                    # position 9: complete blocks 0 and 1
    sel = np.array([[0, 2]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle_lib.sparse_attn_rows(Q, K, V, rows, sel, np.array([2], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle_lib.sparse_attn_rows(Q, K, V, rows, np.array([[0, -1]], dtype=np.int32),
                                    np.array([3], dtype=np.int32))
    O, _ = oracle_lib.sparse_attn_rows(Q, K, V, rows, np.array([[1, -1]], dtype=np.int32),
                                       np.array([1], dtype=np.int32))
    assert np.isfinite(O).all()


def test_rows_and_positions_out_of_range(oracle_lib, synth_lib):
    Q, K, V = _inputs(synth_lib)
    qi = synth_lib.normal_bf16(4, (40, 4, 128), 2)
    kb = oracle_lib.compress(synth_lib.normal_bf16(5, (40, 128), 2))
    with pytest.raises(ValueError):
        oracle_lib.dense_rows(Q, K, V, np.array([40]))
    with pytest.raises(ValueError):
        oracle_lib.dense_rows(Q[:5], K, V, np.array([3]), pos0=37)
    with pytest.raises(ValueError):
        oracle_lib.qsa_rows(Q, K, V, qi, kb, np.array([-1]))
    with pytest.raises(ValueError):
        oracle_lib.qsa_rows_at(Q[:2], K, V, qi[:2], kb, np.array([3, 40]))
    with pytest.raises(ValueError):
        oracle_lib.select_rows(qi, kb, np.array([41]))
    with pytest.raises(ValueError):
        oracle_lib.attend_row(Q[0], K, V, np.array([0, 40]))
