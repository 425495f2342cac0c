"""Pins of the fp64 oracle against closed forms, brute force and invariants.

Each test fixes a value the pages or the mathematics determine independently
of the oracle's own code, chosen so that a plausible slip (a dropped term, a
wrong sign, index or pairing, a transposed operand, an off-by-one in the
block rule) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    """float array -> bf16 bits (values used here are exactly representable)."""
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "test value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def f32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Page parameters (golden fixture of values the pages print).
# ----------------------------------------------------------------------------

def test_page_parameters_fixture(synth_lib):
    vals = {}
    with open(os.path.join(GOLDEN, "qsa_parameters.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                vals[k] = int(v)
    s = synth_lib
    assert (s.H, s.HKV, s.D, s.HI, s.DI, s.R) == (
        vals["query_heads"], vals["kv_heads"], vals["head_dim"], vals["indexer_query_heads"],
        vals["indexer_head_dim"], vals["block_size"])
    assert vals["indexer_key_heads"] == 1
    assert vals["budget_blocks"] * vals["block_size"] == vals["budget_tokens"]
    assert vals["rope_dim"] == 64


# ----------------------------------------------------------------------------
# bf16 narrowing: nearest, ties to even.
# ----------------------------------------------------------------------------

def test_bf16_rounding_rule(oracle_lib):
    o = oracle_lib
    one = 1.0
    q = 2.0 ** -7   # bf16 spacing just above 1
    assert f32(o.f64_to_bf16(one + 0.5 * q)) == one              # tie -> even (1.0)
    assert f32(o.f64_to_bf16(one + 1.5 * q)) == one + 2 * q      # tie -> even (k=2)
    assert f32(o.f64_to_bf16(one + 0.5 * q + 1e-12)) == one + q  # above tie -> up
    assert f32(o.f64_to_bf16(-(one + 0.49 * q))) == -one
    assert f32(o.f64_to_bf16(255.5)) == 256.0                    # carries into next binade
    assert f32(o.f64_to_bf16(3.0)) == 3.0


# ----------------------------------------------------------------------------
# RoPE: NeoX pairs (j, j+32) on dims [0,64), angle p * theta^(-2j/64).
# ----------------------------------------------------------------------------

def _unit_head(j, val=1.0, D=256):
    x = np.zeros((1, 1, D), dtype=np.float32)
    x[0, 0, j] = val
    return bf(x)


def test_rope_identity_at_position_zero(oracle_lib, synth_lib):
    x = synth_lib.normal_bf16(1, (3, 24, 256))
    y = oracle_lib.rope(x, pos0=0, pos=np.zeros(3, dtype=np.int64))
    assert np.array_equal(x, y)


def test_rope_leaves_dims_64_and_up(oracle_lib, synth_lib):
    x = synth_lib.normal_bf16(1, (5, 3, 256))
    y = oracle_lib.rope(x, pos0=12345)
    assert np.array_equal(x[..., 64:], y[..., 64:])
    assert not np.array_equal(x[..., :64], y[..., :64])


@pytest.mark.parametrize("j,p,omega", [
    (0, 1, 1.0),                         # theta^0
    (16, 2000, 1.0 / math.sqrt(1e7)),    # theta^(-1/2)
    (8, 300, 1e7 ** -0.25),              # theta^(-1/4)
])
def test_rope_pair_and_angle(oracle_lib, j, p, omega):
    """A unit vector on dim j turns inside the plane (j, j+32), counter-clockwise,
    by p*omega_j; nothing else moves."""
    y = f32(oracle_lib.rope(_unit_head(j), pos0=p))[0, 0]
    others = np.delete(y, [j, j + 32])
    assert np.all(others == 0)
    ang = math.atan2(y[j + 32], y[j])
    want = math.remainder(p * omega, 2 * math.pi)
    assert abs(math.remainder(ang - want, 2 * math.pi)) < 2e-2
    # second member of the pair: e_{j+32} -> (-sin, cos)
    y2 = f32(oracle_lib.rope(_unit_head(j + 32), pos0=p))[0, 0]
    ang2 = math.atan2(-y2[j], y2[j + 32])
    assert abs(math.remainder(ang2 - want, 2 * math.pi)) < 2e-2


def test_rope_large_position(oracle_lib):
    """Pair 0 has unit frequency, so at p = 1,048,575 it must show cos/sin of p."""
    p = 1048575
    y = f32(oracle_lib.rope(_unit_head(0), pos0=p))[0, 0]
    assert abs(y[0] - math.cos(p)) < 4e-3 and abs(y[32] - math.sin(p)) < 4e-3


def test_rope_relative_position(oracle_lib, synth_lib):
    """q'(p1).k'(p2) depends only on p1 - p2 (up to the bf16 output rounding)."""
    q = synth_lib.normal_bf16(7, (1, 1, 256))
    k = synth_lib.normal_bf16(8, (1, 1, 256))

    def dot(p1, p2):
        a = f32(oracle_lib.rope(q, pos0=p1)).astype(np.float64)
        b = f32(oracle_lib.rope(k, pos0=p2)).astype(np.float64)
        return float((a * b).sum())

    base = dot(100, 37)
    for shift in (1, 1000, 500000):
        assert abs(dot(100 + shift, 37 + shift) - base) < 0.15
    # and it does change with the distance
    assert abs(dot(100, 38) - base) > 1e-3 or abs(dot(100, 90) - base) > 1e-3


def test_rope_pair_norms_preserved(oracle_lib, synth_lib):
    x = synth_lib.normal_bf16(1, (4, 2, 256))
    y = oracle_lib.rope(x, pos0=777)
    a, b = f32(x).astype(np.float64), f32(y).astype(np.float64)
    na = a[..., :32] ** 2 + a[..., 32:64] ** 2
    nb = b[..., :32] ** 2 + b[..., 32:64] ** 2
    assert np.allclose(na, nb, rtol=2e-2, atol=1e-6)


# ----------------------------------------------------------------------------
# Key compression.
# ----------------------------------------------------------------------------

def test_compress_block_membership(oracle_lib):
    """Block b pools tokens 4b..4b+3: with k[t] = t the mean is 4b + 1.5;
    the trailing incomplete block is not pooled."""
    Tk = 4 * 12 + 3
    k = np.repeat(np.arange(Tk, dtype=np.float32)[:, None], 128, axis=1)
    kb = f32(oracle_lib.compress(bf(k)))
    assert kb.shape == (12, 128)
    assert np.array_equal(kb[:, 0], 4 * np.arange(12) + 1.5)


def test_compress_constant_and_exact(oracle_lib):
    k = np.zeros((8, 128), dtype=np.float32)
    k[0:4] = 0.375
    k[4:8, 0] = [1.0, 2.0, 3.0, 6.0]
    k[4:8, 1] = [1.0, 1.0, 1.0, 1.0 + 2 ** -6]   # mean 1 + 2^-8: tie -> 1.0
    k[4:8, 2] = [1.0, 1.0, 1.0, 1.0 + 3 * 2 ** -6]  # mean 1 + 1.5*2^-7: tie -> 1 + 2^-6
    kb = f32(oracle_lib.compress(bf(k)))
    assert np.all(kb[0] == 0.375)
    assert kb[1, 0] == 3.0
    assert kb[1, 1] == 1.0
    assert kb[1, 2] == 1.0 + 2 ** -6
    assert np.all(kb[1, 3:] == 0.0)


def test_compress_rmsnorm_mode(oracle_lib):
    k = np.zeros((4, 128), dtype=np.float32)
    k[:, :64] = 3.0
    k[:, 64:] = -3.0
    kb = f32(oracle_lib.compress(bf(k), mode=1))[0]
    assert np.all(kb[:64] == 1.0) and np.all(kb[64:] == -1.0)
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((16, 128)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(
        np.float32)
    kb2 = f32(oracle_lib.compress(bf(x), mode=1)).astype(np.float64)
    rms = np.sqrt((kb2 ** 2).mean(axis=1))
    assert np.allclose(rms, 1.0, atol=1e-2)
    mean = x.reshape(4, 4, 128).mean(axis=1)
    assert np.all(np.sign(kb2) == np.sign(mean))


def test_compress_gain_scales_rmsnorm(oracle_lib, synth_lib):
    """A power-of-two gain scales the normalised key exactly, dim by dim."""
    k = synth_lib.normal_bf16(5, (64, 128), seed=3)
    g = np.ones(128, dtype=np.float32)
    g[::3] = 2.0
    g[1::3] = 0.25
    plain = f32(oracle_lib.compress(k, mode=1))
    gained = f32(oracle_lib.compress(k, mode=1, gain=bf(g)))
    assert np.array_equal(gained, plain * g)
    # MEAN mode ignores the gain
    assert np.array_equal(oracle_lib.compress(k, gain=bf(g)), oracle_lib.compress(k))


def test_compress_rope_is_o1_at_block_start(oracle_lib, synth_lib):
    """Blocks of four equal keys pool exactly, so pooling-then-RoPE must equal
    O1 applied to the key at the block's first token r*(block0 + b)."""
    rows = synth_lib.normal_bf16(5, (40, 128), seed=4)
    k = np.repeat(rows, 4, axis=0)
    for rd, block0 in [(64, 0), (64, 1000), (32, 7), (128, 262143)]:
        got = oracle_lib.compress(k, rope_dim=rd, block0=block0)
        want = oracle_lib.rope(rows[:, None, :], rope_dim=rd,
                               pos=4 * (block0 + np.arange(40)))[:, 0, :]
        assert np.array_equal(got, want), (rd, block0)
    assert np.array_equal(oracle_lib.compress(k, rope_dim=64, block0=0)[0], rows[0])


def test_compress_rope_relative_scores(oracle_lib, synth_lib):
    """Indexer scores with rotated queries and pooled keys depend on the
    query-block distance only: shifting every position by 4m keeps them (up
    to the bf16 roundings of the rotated vectors)."""
    ki = synth_lib.normal_bf16(5, (256, 128), seed=5)
    qi = synth_lib.normal_bf16(4, (1, 4, 128), seed=5)
    p = 255
    s = []
    for m in (0, 5000):
        kb = oracle_lib.compress(ki, rope_dim=64, block0=m)
        q = oracle_lib.rope(qi, rope_dim=64, pos0=p + 4 * m)
        s.append(oracle_lib.scores_row(q[0], kb, 255))
    assert np.abs(s[0] - s[1]).max() < 0.02 * np.abs(s[0]).max()
    kb0 = oracle_lib.compress(ki)
    s_none = oracle_lib.scores_row(qi[0], kb0, 255)
    assert np.abs(s[0] - s_none).max() > 0.05   # the rotation does act


# ----------------------------------------------------------------------------
# Indexer scores.
# ----------------------------------------------------------------------------

def test_candidate_count_is_complete_blocks(oracle_lib):
    """Only fully formed micro-blocks are scored: p=0..2 none, p=3 one, ..."""
    assert [oracle_lib.num_complete(p) for p in range(10)] == [0, 0, 0, 1, 1, 1, 1, 2, 2, 2]
    kb = np.zeros((100, 128), dtype=np.uint16)
    qi = np.zeros((4, 128), dtype=np.uint16)
    for p, n in [(0, 0), (2, 0), (3, 1), (6, 1), (7, 2), (398, 99), (399, 100), (1000, 100)]:
        assert oracle_lib.scores_row(qi, kb, p).size == n


def test_scores_heads_scale_and_modes(oracle_lib):
    """Head h carries a_h on dim h only; block b carries 1 on dim b%4 only, so
    <q_h, kbar_b> = a_h if h == b%4 else 0."""
    a = [2.0, -3.0, 0.5, 1.0]
    qi = np.zeros((4, 128), dtype=np.float32)
    for h in range(4):
        qi[h, h] = a[h]
    kb = np.zeros((8, 128), dtype=np.float32)
    for b in range(8):
        kb[b, b % 4] = 1.0
    p = 31
    s_max = oracle_lib.scores_row(bf(qi), bf(kb), p, mode=0)
    s_sum = oracle_lib.scores_row(bf(qi), bf(kb), p, mode=1)
    want = np.array([2.0, 0.0, 0.5, 1.0] * 2)
    assert np.allclose(s_max, want / math.sqrt(128), rtol=0, atol=1e-15)
    assert np.allclose(s_sum, want, rtol=0, atol=1e-15)
    # max over heads, not sum: two positive heads on one block
    kb2 = np.zeros((1, 128), dtype=np.float32)
    kb2[0, 0] = 1.0
    kb2[0, 3] = 1.0
    s2 = oracle_lib.scores_row(bf(qi), bf(kb2), 3, mode=0)
    s3 = oracle_lib.scores_row(bf(qi), bf(kb2), 3, mode=1)
    assert abs(s2[0] - 2.0 / math.sqrt(128)) < 1e-15
    assert abs(s3[0] - 3.0) < 1e-15


# ----------------------------------------------------------------------------
# Top-K: brute force over all K-subsets.
# ----------------------------------------------------------------------------

def _brute_topk(s, K):
    n = len(s)
    if n <= K:
        return list(range(n))
    best = None
    for comb in itertools.combinations(range(n), K):
        key = (sum(s[i] for i in comb), tuple(-i for i in comb))
        # maximise the score sum; among equal sums prefer the lexicographically
        # smallest ascending index tuple
        cand = (key[0], [-x for x in comb])
        if best is None or cand[0] > best[0] or (cand[0] == best[0] and list(comb) < best[1]):
            best = (cand[0], list(comb))
    return best[1]


@pytest.mark.parametrize("seed", range(40))
def test_topk_brute_force(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    K = int(rng.integers(1, 4))
    if seed % 2:
        s = rng.integers(-2, 3, size=n).astype(np.float64)   # many ties
    else:
        s = rng.standard_normal(n)
    got, sK, sK1 = oracle_lib.topk_row(s, K)
    want = _brute_topk(list(s), K)
    assert list(got) == want
    if n > K:
        order = sorted(range(n), key=lambda i: (-s[i], i))
        assert sK == s[order[K - 1]] and sK1 == s[order[K]]
        assert sorted(s, reverse=True)[K - 1] == sK


def test_topk_within_budget_takes_all(oracle_lib):
    s = np.random.default_rng(1).standard_normal(37)
    got, _, sK1 = oracle_lib.topk_row(s, 512)
    assert list(got) == list(range(37)) and math.isnan(sK1)


# ----------------------------------------------------------------------------
# Token set: selected blocks expanded + the incomplete trailing block.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("p", [0, 1, 2, 3, 4, 5, 6, 7, 8, 41, 42, 43])
def test_token_set(oracle_lib, p):
    nc = (p + 1) // 4
    blk = np.arange(0, nc, 2, dtype=np.int32)
    tok = oracle_lib.token_set(blk, p)
    assert tok.size == 4 * blk.size + (p + 1) % 4
    assert tok.max() <= p
    want = sorted([4 * b + t for b in blk for t in range(4)] + list(range(4 * nc, p + 1)))
    assert list(tok) == want


# Index reuse by later speculative queries: the selection made for p_sel
# expanded, then every token from r*nc(p_sel) through the query's position.
@pytest.mark.parametrize("p_sel", [0, 1, 2, 3, 4, 6, 30, 33, 34])
def test_token_set_reuse(oracle_lib, p_sel):
    nc = (p_sel + 1) // 4
    blk = np.arange(0, nc, 3, dtype=np.int32)
    assert np.array_equal(oracle_lib.token_set_reuse(blk, p_sel, p_sel),
                          oracle_lib.token_set(blk, p_sel))
    for p in range(p_sel, p_sel + 7):
        tok = oracle_lib.token_set_reuse(blk, p_sel, p)
        want = {4 * b + t for b in blk for t in range(4)} | set(range(4 * nc, p + 1))
        assert tok.size == len(want) and set(tok.tolist()) == want
        assert tok.size == 4 * blk.size + p - 4 * nc + 1 and tok.max() <= p


# ----------------------------------------------------------------------------
# Attention: closed forms.
# ----------------------------------------------------------------------------

def test_attend_zero_query_is_mean(oracle_lib, synth_lib):
    """q = 0 gives uniform weights: O = mean of V over the set, lse = ln |S|."""
    Kc = synth_lib.normal_bf16(2, (40, 2, 256))
    Vc = synth_lib.normal_bf16(3, (40, 2, 256))
    q = np.zeros((24, 256), dtype=np.uint16)
    tok = np.array([0, 3, 4, 5, 17, 39])
    O, lse, err = oracle_lib.attend_row(q, Kc, Vc, tok)
    Vf = f32(Vc).astype(np.float64)
    for h in range(24):
        g = h // 12
        assert np.allclose(O[h], Vf[tok, g].mean(axis=0), atol=1e-12)
    assert np.allclose(lse, math.log(tok.size), atol=1e-12)
    assert err < 1e-12


def test_attend_two_tokens_scale(oracle_lib):
    """Logit gap a*b/sqrt(256) -> weights sigma(gap), 1 - sigma(gap)."""
    a, b = 6.0, 5.0
    q = np.zeros((24, 256), dtype=np.float32)
    q[:, 7] = a
    Kc = np.zeros((2, 2, 256), dtype=np.float32)
    Kc[0, :, 7] = b
    Vc = np.zeros((2, 2, 256), dtype=np.float32)
    Vc[0, :, 0] = 1.0
    Vc[1, :, 1] = 1.0
    O, lse, _ = oracle_lib.attend_row(bf(q), bf(Kc), bf(Vc), np.array([0, 1]))
    w0 = 1.0 / (1.0 + math.exp(-a * b / 16.0))
    assert np.allclose(O[:, 0], w0, atol=1e-14) and np.allclose(O[:, 1], 1 - w0, atol=1e-14)
    assert np.allclose(lse, math.log(math.exp(a * b / 16.0) + 1.0), atol=1e-12)


def test_attend_gqa_mapping(oracle_lib):
    """Query heads 0..11 read KV head 0, heads 12..23 read KV head 1."""
    Kc = np.zeros((3, 2, 256), dtype=np.float32)
    Vc = np.zeros((3, 2, 256), dtype=np.float32)
    Vc[:, 0, :] = 1.0
    Vc[:, 1, :] = 2.0
    # key 1 of KV head 1 is the only one aligned with the queries
    Kc[1, 1, 5] = 8.0
    q = np.zeros((24, 256), dtype=np.float32)
    q[:, 5] = 8.0
    Vc[1, 1, 3] = 5.0
    O, _, _ = oracle_lib.attend_row(bf(q), bf(Kc), bf(Vc), np.array([0, 1, 2]))
    assert np.allclose(O[:12], 1.0, atol=1e-14)
    assert np.allclose(np.delete(O[12:], 3, axis=1), 2.0, atol=1e-14)
    w = math.exp(4.0) / (math.exp(4.0) + 2)
    assert np.allclose(O[12:, 3], 2 + 3 * w, atol=1e-12)


def test_attend_single_token_and_permutation(oracle_lib, synth_lib):
    q = synth_lib.normal_bf16(1, (24, 256))
    Kc = synth_lib.normal_bf16(2, (9, 2, 256))
    Vc = synth_lib.normal_bf16(3, (9, 2, 256))
    O, _, _ = oracle_lib.attend_row(q, Kc, Vc, np.array([4]))
    Vf = f32(Vc).astype(np.float64)
    assert np.array_equal(O[:12], np.broadcast_to(Vf[4, 0], (12, 256)))
    O1, l1, _ = oracle_lib.attend_row(q, Kc, Vc, np.array([0, 2, 5, 8]))
    O2, l2, _ = oracle_lib.attend_row(q, Kc, Vc, np.array([8, 5, 0, 2]))
    assert np.allclose(O1, O2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


# ----------------------------------------------------------------------------
# End-to-end QSA rows.
# ----------------------------------------------------------------------------

def _small_inputs(synth_lib, T, seed=0):
    Q = synth_lib.normal_bf16(1, (T, 24, 256), seed)
    K = synth_lib.normal_bf16(2, (T, 2, 256), seed)
    V = synth_lib.normal_bf16(3, (T, 2, 256), seed)
    qi = synth_lib.normal_bf16(4, (T, 4, 128), seed)
    ki = synth_lib.normal_bf16(5, (T, 128), seed)
    return Q, K, V, qi, ki


@pytest.mark.parametrize("mode", [0, 1])
def test_qsa_equals_dense_within_budget(oracle_lib, synth_lib, mode):
    """While a query sees at most K complete blocks, QSA is dense causal attention."""
    T, Kb = 70, 8
    Q, K, V, qi, ki = _small_inputs(synth_lib, T)
    kb = oracle_lib.compress(ki)
    rows = np.arange(0, 35)          # nc(p) = floor((p+1)/4) <= 8 for p <= 34
    res = oracle_lib.qsa_rows(Q, K, V, qi, kb, rows, Kbudget=Kb, mode=mode)
    Od, lsed = oracle_lib.dense_rows(Q, K, V, rows)
    assert np.allclose(res["O"], Od, atol=1e-12) and np.allclose(res["lse"], lsed, atol=1e-12)
    # beyond the budget it differs
    rows2 = np.arange(40, 70)
    res2 = oracle_lib.qsa_rows(Q, K, V, qi, kb, rows2, Kbudget=Kb, mode=mode)
    Od2, _ = oracle_lib.dense_rows(Q, K, V, rows2)
    assert np.abs(res2["O"] - Od2).max() > 1e-3
    assert np.all(res2["nsel"] == Kb)
    assert np.all(res["wsum_err"] < 1e-12)


@pytest.mark.parametrize("seq_len", [2, 5, 31, 34, 35, 36])
def test_decode_reuse_equals_dense_within_budget(oracle_lib, synth_lib, seq_len):
    """Four speculative queries sharing one selection: while the selecting
    query sees at most K complete blocks, every query is dense causal
    attention at its own position (queries before position 0 see nothing)."""
    T, n = 40, 4
    Q, K, V, qi, ki = _small_inputs(synth_lib, T)
    kb = oracle_lib.compress(ki[:seq_len])
    p0 = seq_len - n
    res = oracle_lib.decode_reuse_rows(_window(Q, p0, n), K, V, qi[max(p0, 0)], kb, seq_len,
                                       Kbudget=10)
    for i in range(n):
        p = p0 + i
        if p < 0:
            assert np.all(res["O"][i] == 0) and np.all(np.isneginf(res["lse"][i]))
            continue
        Od, lsed = oracle_lib.dense_rows(Q, K, V, np.array([p]))
        assert np.allclose(res["O"][i], Od[0], atol=1e-12)
        assert np.allclose(res["lse"][i], lsed[0], atol=1e-12)
    assert np.all(res["wsum_err"] < 1e-12)


def _window(Q, p0, n):
    """Rows p0 .. p0+n-1 of Q; rows before position 0 are zero."""
    out = np.zeros((n,) + Q.shape[1:], dtype=Q.dtype)
    for i in range(n):
        if p0 + i >= 0:
            out[i] = Q[p0 + i]
    return out


def test_decode_reuse_token_sets_from_outputs(oracle_lib):
    """Planted indexer scores and uniform attention (Q = 0) with one-hot V:
    every speculative query attends the first query's K best blocks plus all
    tokens from that query's incomplete block through its own position, also
    when a block completes inside the window."""
    T, Kb, n = 64, 3, 4
    c = np.array([0.5, 3.0, -1.0, 2.0, 0.25, 4.0, 1.0, -2.0, 3.5, 0.125, 1.5, 2.5,
                  -0.5, 0.75, 6.0, 1.25], dtype=np.float32)
    kb = np.zeros((T // 4, 128), dtype=np.float32)
    kb[:, 0] = c
    qi = np.zeros((4, 128), dtype=np.float32)
    qi[1, 0] = 1.0
    Q = np.zeros((n, 24, 256), dtype=np.uint16)
    Kc = np.zeros((T, 2, 256), dtype=np.uint16)
    V = np.zeros((T, 2, 256), dtype=np.float32)
    for j in range(T):
        V[j, :, j] = 1.0
    for seq_len in (31, 33, 34, 35, 36, 50, 64):
        p0 = seq_len - n
        nc0 = (p0 + 1) // 4
        res = oracle_lib.decode_reuse_rows(Q, Kc, bf(V), bf(qi), bf(kb[:seq_len // 4]), seq_len,
                                           Kbudget=Kb)
        sel = sorted(sorted(range(nc0), key=lambda b: (-c[b], b))[:Kb])
        assert list(res["sel"][:res["nsel"]]) == sel
        for i in range(n):
            p = p0 + i
            S = sorted([4 * b + t for b in sel for t in range(4)] + list(range(4 * nc0, p + 1)))
            O = res["O"][i, 5, :T]
            assert np.allclose(O[S], 1.0 / len(S), atol=1e-14), (seq_len, i)
            assert np.allclose(np.delete(O, S), 0.0, atol=1e-14), (seq_len, i)


def test_qsa_selection_and_token_set_from_outputs(oracle_lib):
    """Indexer scores planted as c_b = b-dependent values; uniform attention
    (Q = 0) with one-hot V reveals the attended token set exactly."""
    T = 64
    Kb = 3
    # indexer: one head aligned with dim 0; block b gets kbar[b,0] = c_b
    c = np.array([0.5, 3.0, -1.0, 2.0, 0.25, 4.0, 1.0, -2.0, 3.5, 0.125, 1.5, 2.5,
                  -0.5, 0.75, 6.0, 1.25], dtype=np.float32)
    nb = T // 4
    kb = np.zeros((nb, 128), dtype=np.float32)
    kb[:, 0] = c
    qi = np.zeros((T, 4, 128), dtype=np.float32)
    qi[:, 2, 0] = 1.0
    Q = np.zeros((T, 24, 256), dtype=np.uint16)
    Kc = np.zeros((T, 2, 256), dtype=np.uint16)
    V = np.zeros((T, 2, 256), dtype=np.float32)
    for j in range(T):
        V[j, :, j] = 1.0
    rows = np.arange(T)
    res = oracle_lib.qsa_rows(Q, Kc, bf(V), bf(qi), bf(kb), rows, Kbudget=Kb)
    for t in range(T):
        nc = (t + 1) // 4
        order = sorted(range(nc), key=lambda b: (-c[b], b))
        want_blocks = sorted(order[:Kb])
        assert list(res["sel"][t, :res["nsel"][t]]) == want_blocks
        S = sorted([4 * b + i for b in want_blocks for i in range(4)] + list(range(4 * nc, t + 1)))
        O = res["O"][t, 0, :T]
        assert np.allclose(O[S], 1.0 / len(S), atol=1e-14)
        assert np.allclose(np.delete(O, S), 0.0, atol=1e-14)
        assert np.allclose(res["lse"][t], math.log(len(S)), atol=1e-12)


def test_needle_blocks_always_selected(oracle_lib, synth_lib):
    T = 1024
    Q, K, V, qi, ki = _small_inputs(synth_lib, T, seed=3)
    nd = synth_lib.needle_blocks(T // 4, 2, 4, seed=3)
    # a stronger plant than the workloads' x4 so that selection is certain
    for _ in range(3):
        synth_lib.apply_needles(K, ki, nd)
    kb = oracle_lib.compress(ki)
    rows = np.arange(T - 8, T)
    sel = oracle_lib.select_rows(qi, kb, rows, Kbudget=64)
    for i in range(rows.size):
        chosen = set(sel["sel"][i, :sel["nsel"][i]])
        # every needle whose indexer key aligns positively with some head of
        # this query ranks above the N(0,1) background
        s = oracle_lib.scores_row(qi[rows[i]], kb, int(rows[i]))
        pos_needles = [b for b in np.unique(nd) if s[b] > 1.5]
        assert pos_needles, "plant too weak for this check"
        assert set(pos_needles) <= chosen


def test_r1_full_budget_is_dense(oracle_lib, synth_lib):
    """With micro-blocks of one token and a budget covering the context, the
    selection is every past token and QSA is dense attention."""
    T = 24
    Q, K, V, qi, ki = _small_inputs(synth_lib, T, seed=5)
    kb = oracle_lib.compress(ki, r=1)
    rows = np.arange(T)
    res = oracle_lib.qsa_rows(Q, K, V, qi, kb, rows, Kbudget=T, r=1)
    Od, _ = oracle_lib.dense_rows(Q, K, V, rows)
    assert np.allclose(res["O"], Od, atol=1e-12)


def test_indexer_pairs_count(oracle_lib):
    """The indexer compares each query with its complete blocks: sum over p of
    floor((p+1)/4) pairs, about n^2/(2r) (the n^2/r cost statement of section 6)."""
    m = 1024
    n = 4 * m
    tot = sum(oracle_lib.num_complete(p) for p in range(n))
    assert tot == 2 * m * m - m          # sum_{q=1..4m} floor(q/4), closed form
    assert abs(tot / (n * n / 8) - 1) < 2e-3


# ----------------------------------------------------------------------------
# Stage-1 indexer distillation (forward): teacher = dense attention max-pooled
# per block, heads summed, L1-normalised; KL against softmax of the scores.
# ----------------------------------------------------------------------------

def _distill_inputs(p, planted):
    """q_row [24, 256] and K [p+1, 2, 256] with logits q_h.k_j / 16 equal to
    planted[(group, j)] (0 elsewhere): dim g*2 carries group g's keys."""
    q = np.zeros((24, 256), dtype=np.float32)
    q[:12, 0] = 4.0
    q[12:, 1] = 4.0
    K = np.zeros((p + 1, 2, 256), dtype=np.float32)
    for (g, j), c in planted.items():
        K[j, g, g] = c * 16.0 / 4.0   # (4 * x) / 16 = c
    return bf(q), bf(K)


def test_distill_uniform_attention_closed_form(oracle_lib):
    """K = 0: attention is uniform, so the teacher is uniform over the nc
    complete blocks and KL = -ln nc - mean(s) + logsumexp(s)."""
    p = 41
    nc = (p + 1) // 4
    q, K = _distill_inputs(p, {})
    s0 = np.zeros(nc)
    kl, T, _ = oracle_lib.distill_row(q, K, p, s0)
    assert abs(kl) < 1e-14 and np.allclose(T, 1.0 / nc, atol=1e-15)
    s = np.linspace(-1.0, 2.0, nc)
    kl, T, lS = oracle_lib.distill_row(q, K, p, s)
    lse = np.log(np.exp(s).sum())
    assert abs(kl - (-np.log(nc) - s.mean() + lse)) < 1e-12
    assert np.allclose(lS, s - lse, atol=1e-14)
    assert oracle_lib.distill_row(q, K, 2, np.zeros(0))[0] == 0.0   # no complete block


def test_distill_max_pool_and_head_sum(oracle_lib):
    """Planted logits: group 1 heads see logit c1 on token 1 (block 0) and c2
    on token 2 (same block); group 0 heads see c0 on token 9, inside the
    query's incomplete block (p = 10: blocks 0, 1 complete).  The teacher is
    the max inside each block, summed over all 24 heads, normalised; the
    incomplete block counts in each head's softmax but not in the teacher."""
    p, c0, c1, c2 = 10, 3.0, 2.0, 1.0
    q, K = _distill_inputs(p, {(0, 9): c0, (1, 1): c1, (1, 2): c2})
    kl, T, _ = oracle_lib.distill_row(q, K, p, np.zeros(2))
    z0 = np.exp(c0) + 10.0                        # group 0 softmax denominator
    z1 = np.exp(c1) + np.exp(c2) + 9.0            # group 1
    m0 = 12 * (1.0 / z0) + 12 * (np.exp(c1) / z1)   # block 0: max = token 1
    m1 = 12 * (1.0 / z0) + 12 * (1.0 / z1)          # block 1: all logits 0
    want = np.array([m0, m1]) / (m0 + m1)
    assert np.allclose(T, want, atol=1e-14)
    assert abs(kl - np.sum(want * (np.log(want) - np.log(0.5)))) < 1e-13


def test_distill_rows_nonnegative_and_zero_at_teacher(oracle_lib, synth_lib):
    """KL >= 0 on random inputs, and KL = 0 when the indexer scores are the
    log of the teacher (up to a constant)."""
    T_len = 80
    Q, K, V, qi, ki = _small_inputs(synth_lib, T_len)
    kb = oracle_lib.compress(ki)
    rows = np.arange(0, T_len, 7)
    kl = oracle_lib.distill_rows(Q, K, qi, kb, rows)
    assert np.all(kl >= -1e-12) and kl[rows >= 7].min() > 1e-6
    kl_t, T, _ = oracle_lib.distill_row(Q[70], K, 70, np.zeros(17))
    kl2, _, _ = oracle_lib.distill_row(Q[70], K, 70, np.log(T) + 3.0)
    assert abs(kl2) < 1e-12 and kl_t > 0


# ----------------------------------------------------------------------------
# Distillation KL under the sparse pattern: teacher = the sparse attention
# (softmax over the selected blocks and the incomplete block) max-pooled per
# selected block, heads summed, L1-normalised; student = softmax of the
# selected blocks' scores.
# ----------------------------------------------------------------------------

def test_sparse_kl_planted_closed_form(oracle_lib):
    """p = 30: complete blocks 0..6, incomplete block 28..30; blocks 1, 4, 6
    selected.  Group 0 heads see c0 on token 17 (block 4) and c2 on token 29
    (incomplete block); group 1 heads see c1 on token 5 (block 1) and c3 on
    token 9 (block 2, not selected, so outside every softmax).  Each head's
    softmax runs over the 15 tokens of the set."""
    p, c0, c1, c2, c3 = 30, 2.5, 1.75, 3.0, 5.0
    q, K = _distill_inputs(p, {(0, 17): c0, (0, 29): c2, (1, 5): c1, (1, 9): c3})
    blk = np.array([1, 4, 6], dtype=np.int32)
    s = np.array([0.3, -0.2, 1.1])
    kl, T, lS = oracle_lib.sparse_kl_row(q, K, p, blk, s)
    z0 = np.exp(c0) + np.exp(c2) + 13.0
    z1 = np.exp(c1) + 14.0
    m = 12 * np.array([1.0 / z0 + np.exp(c1) / z1,
                       np.exp(c0) / z0 + 1.0 / z1,
                       1.0 / z0 + 1.0 / z1])
    want = m / m.sum()
    ls = s - np.log(np.exp(s).sum())
    assert np.allclose(T, want, atol=1e-14)
    assert np.allclose(lS, ls, atol=1e-14)
    assert abs(kl - np.sum(want * (np.log(want) - ls))) < 1e-13
    # nothing selected: no distribution, KL 0
    assert oracle_lib.sparse_kl_row(q, K, p, np.zeros(0, np.int32), np.zeros(0))[0] == 0.0


def test_sparse_kl_with_every_block_selected_is_stage1(oracle_lib, synth_lib):
    """A budget above nc(p) selects every complete block: the token set is
    0..p, the sparse softmax is the dense one, and the KL equals the dense
    distillation's (computed by its own code)."""
    T_len = 90
    Q, K, V, qi, ki = _small_inputs(synth_lib, T_len, seed=7)
    kb = oracle_lib.compress(ki)
    rows = np.arange(0, T_len, 5)
    for mode in (oracle_lib.MODE_MAXHEAD, oracle_lib.MODE_RELUSUM):
        sel = oracle_lib.select_rows(qi, kb, rows, Kbudget=32, mode=mode)
        assert np.all(sel["nsel"] == np.array([oracle_lib.num_complete(t) for t in rows]))
        got = oracle_lib.sparse_kl_rows(Q, K, qi, kb, rows, sel["sel"], sel["nsel"], mode=mode)
        ref = oracle_lib.distill_rows(Q, K, qi, kb, rows, mode=mode)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-13), mode


def test_sparse_kl_subset_rows_scores_and_bounds(oracle_lib, synth_lib):
    """A budget of 5 below nc(p): the rows form takes each selected block's
    own score (checked against the single-row form fed the selected entries of
    the full score row); KL >= 0, = 0 when the scores are ln T + const, and the
    subset KL differs from the dense one."""
    T_len = 90
    Q, K, V, qi, ki = _small_inputs(synth_lib, T_len, seed=8)
    kb = oracle_lib.compress(ki)
    rows = np.arange(30, T_len, 6)
    sel = oracle_lib.select_rows(qi, kb, rows, Kbudget=5, want_scores=True)
    got = oracle_lib.sparse_kl_rows(Q, K, qi, kb, rows, sel["sel"], sel["nsel"])
    dense = oracle_lib.distill_rows(Q, K, qi, kb, rows)
    for i, t in enumerate(rows):
        ns = sel["nsel"][i]
        assert ns == 5
        blk = sel["sel"][i, :ns]
        s = sel["s"][i, blk]
        kl, T, _ = oracle_lib.sparse_kl_row(Q[t], K, int(t), blk, s)
        assert abs(kl - got[i]) < 1e-13
        assert kl >= -1e-12 and abs(kl - dense[i]) > 1e-6
        kl0, _, _ = oracle_lib.sparse_kl_row(Q[t], K, int(t), blk, np.log(T) - 2.0)
        assert abs(kl0) < 1e-12


# ----------------------------------------------------------------------------
# Row drivers (the functions every full-size GPU comparison calls): rows that
# are not 0..n-1, a chunk that does not start at position 0, a compact form.
# Planted inputs make each row's selection, token set and query row visible
# in its output, so a row or position taken from the wrong index fails.
# ----------------------------------------------------------------------------

_DRV_POS0, _DRV_TQ, _DRV_K = 100, 100, 3
# (p + 1) mod 4 of the rows' positions p = 100 + t is 2, 1, 0, 3, 2: every
# trailing-block length, and never the value of position 100 + i for row i
_DRV_ROWS = np.array([5, 40, 63, 2, 97])


def _driver_inputs(mode):
    """Positions 0..199; queries t = 0..99 at positions 100 + t.  Indexer:
    pooled key b carries c_b in dim 0 (distinct multiples of 1/8), every head
    of query t carries +1 (t even) or -1 (t odd) there, so the score order is
    c ascending or descending by row.  Returns inputs, scores per row, the
    selection by brute force and the planted target token per row."""
    Tk, nb = _DRV_POS0 + _DRV_TQ, (_DRV_POS0 + _DRV_TQ) // 4
    c = (np.random.default_rng(17).permutation(nb) - 20.0) / 8.0
    kb = np.zeros((nb, 128), dtype=np.float32)
    kb[:, 0] = c
    qi = np.zeros((_DRV_TQ, 4, 128), dtype=np.float32)
    qi[:, :, 0] = np.where(np.arange(_DRV_TQ) % 2 == 0, 1.0, -1.0)[:, None]
    sel, targets = {}, {}
    for t in _DRV_ROWS:
        p = _DRV_POS0 + int(t)
        nc = (p + 1) // 4
        sgn = 1.0 if t % 2 == 0 else -1.0
        sc = [sgn * c[b] / math.sqrt(128) if mode == 0 else 4 * max(0.0, sgn * c[b])
              for b in range(nc)]
        blocks = sorted(sorted(range(nc), key=lambda b: (-sc[b], b))[:_DRV_K])
        sel[int(t)] = blocks
        targets[int(t)] = 4 * blocks[1] + int(t) % 4
    assert len(set(targets.values())) == len(_DRV_ROWS)
    # one-hot keys and values: K[j, g, j] = 64, V[j, g, j] = 1 (j < 200 < 256)
    K = np.zeros((Tk, 2, 256), dtype=np.float32)
    V = np.zeros((Tk, 2, 256), dtype=np.float32)
    for j in range(Tk):
        K[j, :, j] = 64.0
        V[j, :, j] = 1.0
    # Q row t points at its target token: logit 64 * 64 / 16 = 256 there, 0
    # elsewhere, so the softmax is one-hot at the target to e^-256
    Qt = np.zeros((_DRV_TQ, 24, 256), dtype=np.float32)
    for t, j in targets.items():
        Qt[t, :, j] = 64.0
    return dict(kb=bf(kb), qi=bf(qi), K=bf(K), V=bf(V), Qt=bf(Qt),
                Q0=np.zeros((_DRV_TQ, 24, 256), dtype=np.uint16), sel=sel, targets=targets)


def _token_set_expected(blocks, p):
    nc = (p + 1) // 4
    return sorted([4 * b + u for b in blocks for u in range(4)] + list(range(4 * nc, p + 1)))


def _check_uniform(O, lse, S, what):
    """Q = 0: O of every head is 1/|S| on the tokens of S, 0 elsewhere."""
    want = np.zeros(256)
    want[S] = 1.0 / len(S)
    assert np.allclose(O, want[None, :], atol=1e-14), what
    assert np.allclose(lse, math.log(len(S)), atol=1e-12), what


def _check_target(O, lse, target, what):
    want = np.zeros(256)
    want[target] = 1.0
    assert np.allclose(O, want[None, :], atol=1e-12), what
    assert np.allclose(lse, 256.0, atol=1e-12), what


@pytest.mark.parametrize("mode", [0, 1])
def test_row_drivers_select_planted(oracle_lib, mode):
    x = _driver_inputs(mode)
    res = oracle_lib.select_rows(x["qi"], x["kb"], _DRV_ROWS, pos0=_DRV_POS0, Kbudget=_DRV_K,
                                 mode=mode)
    for i, t in enumerate(_DRV_ROWS):
        assert list(res["sel"][i, :res["nsel"][i]]) == x["sel"][int(t)], (mode, t)
        assert np.all(res["sel"][i, res["nsel"][i]:] == -1)


@pytest.mark.parametrize("mode", [0, 1])
def test_row_drivers_qsa_rows_planted(oracle_lib, mode):
    """qsa_rows (full chunk arrays, row t = query at pos0 + t) and
    qsa_rows_at (compact arrays, row i = query at positions[i]) give each row
    its own selection, trailing block and query row."""
    x = _driver_inputs(mode)
    rows = _DRV_ROWS
    pos = _DRV_POS0 + rows
    for qkey in ("Q0", "Qt"):
        Q = x[qkey]
        full = oracle_lib.qsa_rows(Q, x["K"], x["V"], x["qi"], x["kb"], rows, pos0=_DRV_POS0,
                                   Kbudget=_DRV_K, mode=mode)
        at = oracle_lib.qsa_rows_at(Q[rows], x["K"], x["V"], x["qi"][rows], x["kb"], pos,
                                    Kbudget=_DRV_K, mode=mode)
        for res, name in ((full, "qsa_rows"), (at, "qsa_rows_at")):
            for i, t in enumerate(rows):
                t = int(t)
                what = (name, qkey, mode, t)
                assert list(res["sel"][i, :res["nsel"][i]]) == x["sel"][t], what
                S = _token_set_expected(x["sel"][t], _DRV_POS0 + t)
                if qkey == "Q0":
                    _check_uniform(res["O"][i], res["lse"][i], S, what)
                else:
                    _check_target(res["O"][i], res["lse"][i], x["targets"][t], what)
            assert np.all(res["wsum_err"] < 1e-12)


def test_row_drivers_sparse_attn_rows_planted(oracle_lib):
    """Attention over a given selection: row i uses Q row rows[i], the
    selection row i and the trailing block of position pos0 + rows[i]."""
    x = _driver_inputs(0)
    rows = _DRV_ROWS
    sel = np.full((rows.size, 8), -1, dtype=np.int32)   # a wider budget than used
    nsel = np.zeros(rows.size, dtype=np.int32)
    for i, t in enumerate(rows):
        sel[i, :_DRV_K] = x["sel"][int(t)]
        nsel[i] = _DRV_K
    for qkey in ("Q0", "Qt"):
        O, lse = oracle_lib.sparse_attn_rows(x[qkey], x["K"], x["V"], rows, sel, nsel,
                                             pos0=_DRV_POS0)
        for i, t in enumerate(rows):
            t = int(t)
            S = _token_set_expected(x["sel"][t], _DRV_POS0 + t)
            if qkey == "Q0":
                _check_uniform(O[i], lse[i], S, (qkey, t))
            else:
                _check_target(O[i], lse[i], x["targets"][t], (qkey, t))
        # the compact form: row i is the query at position pos0 + rows[i]
        Oc, lc = oracle_lib.sparse_attn_rows_at(x[qkey][rows], x["K"], x["V"], _DRV_POS0 + rows,
                                                sel, nsel)
        for i, t in enumerate(rows):
            t = int(t)
            S = _token_set_expected(x["sel"][t], _DRV_POS0 + t)
            if qkey == "Q0":
                _check_uniform(Oc[i], lc[i], S, ("at", qkey, t))
            else:
                _check_target(Oc[i], lc[i], x["targets"][t], ("at", qkey, t))
    # an empty selection leaves the trailing block alone
    O, lse = oracle_lib.sparse_attn_rows(x["Q0"], x["K"], x["V"], rows, sel,
                                         np.zeros(rows.size, dtype=np.int32), pos0=_DRV_POS0)
    for i, t in enumerate(rows):
        p = _DRV_POS0 + int(t)
        tail = list(range(4 * ((p + 1) // 4), p + 1))
        if tail:
            _check_uniform(O[i], lse[i], tail, ("empty", int(t)))


def test_row_drivers_dense_rows_planted(oracle_lib):
    x = _driver_inputs(0)
    rows = _DRV_ROWS
    for qkey in ("Q0", "Qt"):
        O, lse = oracle_lib.dense_rows(x[qkey], x["K"], x["V"], rows, pos0=_DRV_POS0)
        for i, t in enumerate(rows):
            t = int(t)
            if qkey == "Q0":
                _check_uniform(O[i], lse[i], list(range(_DRV_POS0 + t + 1)), (qkey, t))
            else:
                _check_target(O[i], lse[i], x["targets"][t], (qkey, t))


@pytest.mark.parametrize("mode", [0, 1])
def test_row_drivers_compact_within_budget_is_dense(oracle_lib, synth_lib, mode):
    """Compact rows at positions whose context fits the budget: QSA is dense
    causal attention there (N(0,1) inputs, rows out of order, positions
    spread over every trailing-block length)."""
    T, Kb = 60, 9
    Q, K, V, qi, ki = _small_inputs(synth_lib, T, seed=21)
    kb = oracle_lib.compress(ki)
    pos = np.array([33, 2, 17, 36, 0, 24, 11])          # nc(p) <= 9
    at = oracle_lib.qsa_rows_at(Q[pos], K, V, qi[pos], kb, pos, Kbudget=Kb, mode=mode)
    Od, lsed = oracle_lib.dense_rows(Q, K, V, pos)
    assert np.allclose(at["O"], Od, atol=1e-12) and np.allclose(at["lse"], lsed, atol=1e-12)
    assert list(at["nsel"]) == [(p + 1) // 4 for p in pos]
    # beyond the budget it is not dense, and it equals the full-array driver
    pos2 = np.array([59, 41, 50])
    at2 = oracle_lib.qsa_rows_at(Q[pos2], K, V, qi[pos2], kb, pos2, Kbudget=Kb, mode=mode)
    full2 = oracle_lib.qsa_rows(Q, K, V, qi, kb, pos2, Kbudget=Kb, mode=mode)
    Od2, _ = oracle_lib.dense_rows(Q, K, V, pos2)
    assert np.abs(at2["O"] - Od2).max() > 1e-3
    assert np.array_equal(at2["sel"], full2["sel"]) and np.array_equal(at2["O"], full2["O"])


# ----------------------------------------------------------------------------
# bf16 narrowing below the normal range: a fixed quantum of 2^-133, ties to
# even, the sign kept.
# ----------------------------------------------------------------------------

def test_bf16_rounding_subnormals(oracle_lib):
    o = oracle_lib
    u = 2.0 ** -133                      # the smallest bf16 subnormal (bits 0x0001)
    assert o.f64_to_bf16(u) == 0x0001
    assert o.f64_to_bf16(0.5 * u) == 0x0000            # tie -> even (0)
    assert o.f64_to_bf16(0.5 * u * (1 + 2 ** -20)) == 0x0001
    assert o.f64_to_bf16(1.5 * u) == 0x0002            # tie -> even (2)
    assert o.f64_to_bf16(2.5 * u) == 0x0002            # tie -> even (2)
    assert o.f64_to_bf16(2.4 * u) == 0x0002
    assert o.f64_to_bf16(-5 * u) == 0x8005
    assert o.f64_to_bf16(-0.25 * u) == 0x8000          # rounds to -0
    assert o.f64_to_bf16(0.25 * u) == 0x0000
    assert o.f64_to_bf16(127 * u) == 0x007F            # largest subnormal
    assert o.f64_to_bf16(127.5 * u) == 0x0080          # tie -> even: the smallest normal 2^-126
    assert o.f64_to_bf16(2.0 ** -126) == 0x0080
    # the normal quantum starts at 2^-126: 2^-126 + 2^-133 is exact
    assert o.f64_to_bf16(2.0 ** -126 + u) == 0x0081
    for k in (1, 2, 3, 64, 100, 127):
        assert f32(o.f64_to_bf16(k * u)) == np.float32(k * u)
