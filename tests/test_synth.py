"""The seeded input generator: determinism, distribution, slicing, needles."""
import numpy as np


def test_deterministic_and_sliceable(synth_lib):
    s = synth_lib
    a = s.normal_bf16(2, (64, 2, 256), seed=0)
    b = s.normal_bf16(2, (64, 2, 256), seed=0)
    assert np.array_equal(a, b)
    # any element range regenerates the same values
    part = s.normal_bf16(2, (10, 2, 256), seed=0, first=17 * 512)
    assert np.array_equal(part, a[17:27])
    rows = s.normal_bf16_rows(2, first=3 * 512, nrows=5, row_len=256, src_stride=512)
    assert np.array_equal(rows, a.reshape(-1, 256)[[6, 8, 10, 12, 14]])
    # streams and seeds differ
    assert not np.array_equal(a, s.normal_bf16(3, (64, 2, 256), seed=0))
    assert not np.array_equal(a, s.normal_bf16(2, (64, 2, 256), seed=1))


def test_standard_normal_moments(synth_lib):
    x = synth_lib.bf16_to_f32(synth_lib.normal_bf16(1, (1 << 20,))).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    assert abs((x ** 4).mean() - 3.0) < 5e-2           # normal kurtosis
    assert abs((np.abs(x) < 1).mean() - 0.6827) < 3e-3


def test_decode_sequence_slices_batched_cache(synth_lib):
    s = synth_lib
    L, Lmax = 64, 96
    seq = s.decode_seq(2, L, Lmax)
    full = s.normal_bf16(2, (3, Lmax, 2, 256))
    assert np.array_equal(seq.K, full[2, :L])


def test_needles(synth_lib):
    nd = synth_lib.needle_blocks(1000, 2, 64, seed=0)
    assert nd.shape == (2, 64)
    for row in nd:
        assert len(set(row.tolist())) == 64 and np.all(np.diff(row) > 0)
        assert row.min() >= 0 and row.max() < 1000
    pi = synth_lib.prefill_inputs(256, needles_per_head=4)
    base = synth_lib.prefill_inputs(256)
    K1, K0 = synth_lib.bf16_to_f32(pi.K), synth_lib.bf16_to_f32(base.K)
    for g in range(2):
        for b in pi.needles[g]:
            assert np.array_equal(K1[4 * b:4 * b + 4, g], 4 * K0[4 * b:4 * b + 4, g])
    changed = np.unique(np.nonzero(np.any(K1 != K0, axis=2))[0])
    want = np.unique((pi.needles[:, :, None] * 4 + np.arange(4)).reshape(-1))
    assert np.array_equal(changed, want)
