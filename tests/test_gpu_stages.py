"""Stage-wise parity of the HIP path against the fp64 oracle (small sizes that
span several tiles and a ragged tail)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_close, check_selection, dev, host_u16, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import torch
    import block_sparse_long_08_amd as q
    assert torch.cuda.is_available()
    q.qsa_check_device()
    return q


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------ A1 RoPE
@pytest.mark.parametrize("T,pos0", [(1029, 0), (257, 1040384)])
def test_rope_parity(qsa, T, pos0):
    torch = _torch()
    log(f"rope T={T} pos0={pos0}")
    x = synth.normal_bf16(1, (T, 24, 256), seed=3)
    y = torch.empty((T, 24, 256), dtype=torch.int16, device="cuda")
    qsa.qsa_rope_bf16(dev(x), y, T, 24, 256, 64, 1e7, pos0)
    torch.cuda.synchronize()
    got = host_u16(y)
    ref = oracle.rope(x, pos0=pos0)
    mism = int((got != ref).sum())
    log(f"  bf16 mismatches {mism} of {got.size}")
    # both sides round the fp64 rotation to bf16 once: allow a 1-ulp flip
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and mism <= got.size * 1e-6


def test_rope_in_place_and_decode_form(qsa):
    torch = _torch()
    B = 5
    x = synth.normal_bf16(1, (B, 24, 256), seed=4)
    lens = np.array([1, 2, 4099, 262144, 1048576], dtype=np.int64)
    t = dev(x)
    qsa.qsa_rope_bf16(t, t, B, 24, 256, 64, 1e7, 0, dev(lens))
    torch.cuda.synchronize()
    got = host_u16(t)
    ref = oracle.rope(x, pos=lens - 1)
    assert np.abs(got.astype(np.int32) - ref.astype(np.int32)).max() <= 1


# -------------------------------------------------------------- A2 compress
@pytest.mark.parametrize("mode", [0, 1])
def test_compress_parity(qsa, mode):
    torch = _torch()
    B, Tk = 3, 4 * 1000 + 3
    k = synth.normal_bf16(5, (B, Tk, 128), seed=6)
    nb = Tk // 4
    out = torch.zeros((B, nb + 5, 128), dtype=torch.int16, device="cuda")
    qsa.qsa_compress_keys(dev(k), B, Tk, Tk * 128, 128, 4, mode, out, (nb + 5) * 128)
    torch.cuda.synchronize()
    got = host_u16(out)[:, :nb]
    for b in range(B):
        ref = oracle.compress(k[b], mode=mode)
        if mode == 0:
            assert np.array_equal(got[b], ref), "MEAN pooling must be bit-exact"
        else:
            assert np.abs(got[b].astype(np.int32) - ref.astype(np.int32)).max() <= 1
    assert np.all(host_u16(out)[:, nb:] == 0), "wrote past the complete blocks"


# ---------------------------------------------------------- A3 index scores
def _score_tol(qi_rows, kb, mode):
    """|fp32 - fp64| bound: 1e-5 * sum of |terms| (per row, max over blocks)."""
    q = synth.bf16_to_f32(qi_rows).astype(np.float64)   # [n, 4, 128]
    k = synth.bf16_to_f32(kb).astype(np.float64)        # [nb, 128]
    mag = np.abs(q) @ np.abs(k).T                        # [n, 4, nb]
    if mode == 0:
        return 1e-5 * mag.max(axis=1) / np.sqrt(128) + 1e-30
    return 1e-5 * mag.sum(axis=1) + 1e-30


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("Tq,pos0", [(2048, 0), (333, 4101)])
def test_index_scores_parity(qsa, mode, Tq, pos0):
    torch = _torch()
    log(f"index scores Tq={Tq} pos0={pos0} mode={mode}")
    Tk = pos0 + Tq
    qi = synth.normal_bf16(4, (Tq, 4, 128), seed=7)
    ki = synth.normal_bf16(5, (Tk, 128), seed=7)
    kb = oracle.compress(ki)
    nb = kb.shape[0]
    ld = (nb + 3) // 4 * 4
    sc = torch.full((Tq, ld), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_index_scores(dev(qi), dev(kb), 1, Tq, pos0, None, nb, 4, 128, 4, mode, sc, ld)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, Tq, 7), [Tq - 1]]))
    ref = oracle.select_rows(qi, kb, rows, pos0=pos0, Kbudget=64, mode=mode, want_scores=True)
    tol = _score_tol(qi[rows], kb, mode)
    worst = 0.0
    for i, t in enumerate(rows):
        nc = min((pos0 + t + 1) // 4, nb)
        d = np.abs(got[t, :nc] - ref["s"][i, :nc])
        assert np.all(d <= tol[i, :nc]), (t, float(d.max()))
        worst = max(worst, float((d / tol[i, :nc]).max()) if nc else 0.0)
    log(f"  worst |err|/bound = {worst:.3f}")


@pytest.mark.parametrize("mode", [0, 1])
def test_index_scores_decode_form(qsa, mode):
    """Decode form: one query per sequence at seq_len - 1 over a per-sequence
    pooled-key cache; ragged lengths (no block, a partial 64-block tile, a
    cache longer than the sequence)."""
    torch = _torch()
    B, nb_max = 5, 17501
    lens = np.array([1, 5, 259, 4 * 4097 + 2, 4 * nb_max], dtype=np.int64)
    qi = synth.normal_bf16(4, (B, 4, 128), seed=17)
    kb = np.stack([oracle.compress(synth.normal_bf16(5, (4 * nb_max, 128), seed=17 + b))
                   for b in range(B)])
    ld = (nb_max + 3) // 4 * 4
    sc = torch.full((B, ld), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_index_scores(dev(qi), dev(kb), B, 1, 0, dev(lens), nb_max, 4, 128, 4, mode, sc, ld)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    for b in range(B):
        p = int(lens[b]) - 1
        ref = oracle.scores_row(qi[b], kb[b], p, mode=mode)
        nc = ref.size
        tol = _score_tol(qi[b:b + 1], kb[b], mode)[0, :nc]
        d = np.abs(got[b, :nc] - ref)
        assert np.all(d <= tol), (b, float(d.max()))


# ------------------------------------------------------------------ A4 top-K
def run_topk(qsa, scores, B, Tq, ld, pos0, lens, nb_max, K):
    """qsa_topk_blocks with the workspace it asks for; returns (blk, n_sel)."""
    torch = _torch()
    blk = torch.empty((B * Tq, K), dtype=torch.int32, device="cuda")
    ns = torch.empty((B * Tq,), dtype=torch.int32, device="cuda")
    wsb = qsa.qsa_topk_workspace_bytes(B, Tq, nb_max, K)
    ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device="cuda")
    qsa.qsa_topk_blocks(scores, B, Tq, ld, pos0, lens, nb_max, 4, K, blk, ns, ws, wsb)
    torch.cuda.synchronize()
    return blk.cpu().numpy(), ns.cpu().numpy()


@pytest.mark.parametrize("K", [1, 3, 64, 512])
def test_topk_exact_on_shared_scores(qsa, K):
    """Given the same fp32 scores, the GPU selection equals the oracle's
    (score desc, index asc) top-K exactly, ties included."""
    torch = _torch()
    Tq, pos0 = 300, 3000
    nb = (pos0 + Tq) // 4
    rng = np.random.default_rng(K)
    s = rng.standard_normal((Tq, nb)).astype(np.float32)
    s[::3] = np.round(s[::3] * 4) / 4           # heavy ties on every third row
    s[5] = 0.0                                   # an all-tie row
    s[7, ::2] = -0.0                             # signed zeros compare equal
    s[7, 1::2] = 0.0
    ld = (nb + 3) // 4 * 4
    sp = np.zeros((Tq, ld), dtype=np.float32)
    sp[:, :nb] = s
    g, n = run_topk(qsa, dev(sp), 1, Tq, ld, pos0, None, nb, K)
    for t in range(Tq):
        nc = (pos0 + t + 1) // 4
        row = s[t, :nc].astype(np.float64)
        row[row == 0] = 0.0
        want, _, _ = oracle.topk_row(row, K)
        assert n[t] == want.size
        assert np.array_equal(g[t, :n[t]], want), t
        assert np.all(g[t, n[t]:] == -1)


def test_topk_decode_form_and_small_contexts(qsa):
    torch = _torch()
    B, nb_max, K = 6, 5000, 512
    lens = np.array([1, 3, 4, 2049, 2052, 20000], dtype=np.int64)
    s = np.random.default_rng(9).standard_normal((B, nb_max)).astype(np.float32)
    g, n = run_topk(qsa, dev(s), B, 1, nb_max, 0, dev(lens), nb_max, K)
    for b in range(B):
        nc = min(int(lens[b]) // 4, nb_max)
        want, _, _ = oracle.topk_row(s[b, :nc].astype(np.float64), K)
        assert n[b] == want.size and np.array_equal(g[b, :n[b]], want)


def test_topk_long_rows_and_heavy_ties(qsa):
    """Rows longer than one segment (reduced over per-segment top-K lists),
    threshold bins too crowded for the per-wave lists (block-wide resolve),
    and all-equal rows where the lowest indices must win, K = 512."""
    K, nb_max = 512, 100000
    lens = np.array([4 * 100000, 4 * 50000, 4 * 30000, 4 * 32768, 4 * 32769, 4 * 7000],
                    dtype=np.int64)
    B = lens.size
    rng = np.random.default_rng(21)
    s = rng.standard_normal((B, nb_max)).astype(np.float32)
    s[1] = 0.75                                        # one value: every key ties
    s[2] = rng.choice([0.0, 0.25, 0.5], size=nb_max)   # three values, bins of ~10,000
    s[5, :3000] = 1.0                                  # 3000 ties above the rest
    g, n = run_topk(qsa, dev(s), B, 1, nb_max, 0, dev(lens), nb_max, K)
    for b in range(B):
        nc = min(int(lens[b]) // 4, nb_max)
        want, _, _ = oracle.topk_row(s[b, :nc].astype(np.float64), K)
        assert n[b] == want.size and np.array_equal(g[b, :n[b]], want), b


@pytest.mark.parametrize("Tq,pos0,K", [(300, 4 * 40000, 512), (200, 4 * 70000, 2048),
                                       (130, 4 * 40000, 1024)])
def test_topk_prefill_rows_longer_than_a_segment(qsa, Tq, pos0, K):
    """Prefill-form rows past 32,768 candidates: one reduction pass over
    32,768-key segments (or 4,096-key ones when rows are few), then the final
    pass; rows cut at every 4th query position."""
    nb = (pos0 + Tq) // 4
    ld = (nb + 3) // 4 * 4
    rng = np.random.default_rng(K + Tq)
    s = np.zeros((Tq, ld), dtype=np.float32)
    s[:, :nb] = rng.standard_normal((Tq, nb)).astype(np.float32)
    s[1::7, :nb] = np.round(s[1::7, :nb] * 2) / 2     # crowded rows
    g, n = run_topk(qsa, dev(s), 1, Tq, ld, pos0, None, nb, K)
    for t in range(0, Tq, 3):
        nc = (pos0 + t + 1) // 4
        want, _, _ = oracle.topk_row(s[t, :nc].astype(np.float64), K)
        assert n[t] == want.size and np.array_equal(g[t, :n[t]], want), t


@pytest.mark.parametrize("pos0", [4 * 50000, 4 * 20000])
def test_topk_streaming_rows(qsa, pos0):
    """Many long prefill rows take the streaming kernel (1024 threads past
    32,768 blocks, 256 threads below): exact selections on random rows,
    coarse ties, an all-equal row (the crowded-floor fallback) and a row
    whose top-K sits in one block range."""
    Tq, K = 300, 512
    nb = (pos0 + Tq) // 4
    ld = (nb + 3) // 4 * 4
    rng = np.random.default_rng(77)
    s = np.zeros((Tq, ld), dtype=np.float32)
    s[:, :nb] = rng.standard_normal((Tq, nb)).astype(np.float32)
    s[1::5, :nb] = np.round(s[1::5, :nb] * 4) / 4
    s[2, :nb] = 0.5                                  # every key ties
    s[3, 1000:3000] = 9.0                            # 2000 equal top keys
    g, n = run_topk(qsa, dev(s), 1, Tq, ld, pos0, None, nb, K)
    for t in list(range(0, 12)) + list(range(12, Tq, 23)):
        nc = (pos0 + t + 1) // 4
        want, _, _ = oracle.topk_row(s[t, :nc].astype(np.float64), K)
        assert n[t] == want.size and np.array_equal(g[t, :n[t]], want), t


def test_topk_million_token_decode_rows(qsa):
    """Decode form at 1,048,576 tokens (262,144 blocks): two reduction passes
    and the final pass; one row of random scores, one of coarse ties."""
    K, nb_max, B = 512, 262144, 2
    lens = np.array([4 * nb_max, 4 * nb_max - 5], dtype=np.int64)
    rng = np.random.default_rng(5)
    s = rng.standard_normal((B, nb_max)).astype(np.float32)
    s[1] = np.round(s[1] * 8) / 8
    g, n = run_topk(qsa, dev(s), B, 1, nb_max, 0, dev(lens), nb_max, K)
    for b in range(B):
        nc = min(int(lens[b]) // 4, nb_max)
        want, _, _ = oracle.topk_row(s[b, :nc].astype(np.float64), K)
        assert n[b] == want.size and np.array_equal(g[b, :n[b]], want), b


# --------------------------------------------------- A3+A4 vs fp64 scores
@pytest.mark.parametrize("mode", [0, 1])
def test_selection_tie_band(qsa, mode):
    torch = _torch()
    Tq, pos0, K = 512, 8192, 512
    Tk = pos0 + Tq
    qi = synth.normal_bf16(4, (Tq, 4, 128), seed=8)
    ki = synth.normal_bf16(5, (Tk, 128), seed=8)
    kb = oracle.compress(ki)
    nb = kb.shape[0]
    ws_bytes = qsa.qsa_select_workspace_bytes(1, Tq, nb, K)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")
    blk = torch.empty((Tq, K), dtype=torch.int32, device="cuda")
    ns = torch.empty((Tq,), dtype=torch.int32, device="cuda")
    qsa.qsa_select_blocks(dev(qi), dev(kb), 1, Tq, pos0, None, nb, 4, 128, 4, mode, K, blk, ns,
                          ws, ws_bytes)
    torch.cuda.synchronize()
    g, n = blk.cpu().numpy(), ns.cpu().numpy()
    rows = np.arange(0, Tq, 3)
    ref = oracle.select_rows(qi, kb, rows, pos0=pos0, Kbudget=K, mode=mode, want_scores=True)
    exempt = 0
    for i, t in enumerate(rows):
        nc = (pos0 + t + 1) // 4
        exempt += check_selection(ref["s"][i, :nc], K, ref["sK"][i], ref["sK1"][i], g[t], n[t])
    log(f"  mode {mode}: {exempt} of {rows.size} rows differ inside the tie band")


@pytest.mark.parametrize("mode,Tq,pos0,K", [(0, 1500, 0, 64), (1, 1500, 0, 64),
                                            (0, 700, 140000, 512), (1, 300, 1900, 512),
                                            (0, 37, 5, 3), (0, 300, 2000, 100),
                                            (1, 400, 12000, 1024), (0, 1300, 60000, 512),
                                            (1, 700, 140000, 512), (0, 300, 1048000, 512),
                                            (1, 260, 1048000, 2048), (0, 600, 100000, 512),
                                            (0, 2000, 64000, 512), (0, 2000, 64000, 100),
                                            (0, 60000, 0, 512), (1, 20000, 32000, 512),
                                            (1, 300, 300000, 512), (0, 512, 262144, 64),
                                            (1, 260, 600000, 300)])
def test_select_matches_scores_plus_topk(qsa, mode, Tq, pos0, K):
    """qsa_select_blocks returns exactly what qsa_index_scores followed by
    qsa_topk_blocks returns (same scores bit for bit, same tie order);
    RELUSUM rows near nc = K put the K-th score on a run of exact zeros.
    Chunks of >= 256 rows longer than 12,288 blocks take the one-wave top-K
    when K <= 512: rows of at least 3K/2 groups of 16 blocks take the floor
    from the indexer's group maxima and read only the groups that reach it,
    rows of K .. 3K/2 groups from a histogram of their keys, and rows of
    fewer groups (or crowded lists) go to the streaming kernel (the 60,000
    and 20,000-row cases hold all of these, and rows of nc <= K); larger
    budgets take the streaming kernel, with its floor from the group maxima
    for rows of at least 4 groups per thread (the 300,000, 262,144 and
    600,000 cases add long rows in both modes and budgets of 64 and 300);
    qsa_topk_blocks alone reads the scores only, so the paths must agree
    exactly, RELUSUM zero runs included."""
    torch = _torch()
    Tk = pos0 + Tq
    qi = synth.normal_bf16(4, (Tq, 4, 128), seed=13)
    ki = synth.normal_bf16(5, (Tk, 128), seed=13)
    kb = oracle.compress(ki)
    nb = kb.shape[0]
    ld = (nb + 3) // 4 * 4
    sc = torch.empty((Tq, ld), dtype=torch.float32, device="cuda")
    b2 = torch.full((Tq, K), 7, dtype=torch.int32, device="cuda")
    n2 = torch.full((Tq,), 7, dtype=torch.int32, device="cuda")
    qd, kd = dev(qi), dev(kb)
    qsa.qsa_index_scores(qd, kd, 1, Tq, pos0, None, nb, 4, 128, 4, mode, sc, ld)
    b1, n1 = run_topk(qsa, sc, 1, Tq, ld, pos0, None, nb, K)
    wsb = qsa.qsa_select_workspace_bytes(1, Tq, nb, K)
    ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device="cuda")
    qsa.qsa_select_blocks(qd, kd, 1, Tq, pos0, None, nb, 4, 128, 4, mode, K, b2, n2, ws, wsb)
    torch.cuda.synchronize()
    assert np.array_equal(n1, n2.cpu().numpy())
    assert np.array_equal(b1, b2.cpu().numpy())


@pytest.mark.parametrize("case", ["tie_classes", "all_equal"])
def test_select_planted_ties(qsa, case):
    """Tie handling of the one-wave top-K (300 rows at 140,000, K = 512).
    tie_classes: only indexer head 0 sees dim 0 of the pooled keys; 300
    blocks score 2/sqrt(128), 400 score 1/sqrt(128), the rest 0 (the other
    heads' zero dot products win the max): the list holds the 700 and the
    K-th key falls inside the 400-way tie, taken lowest index first.
    all_equal: zero queries, every score 0, so every group survives, the list
    overflows and the streaming kernel finishes every row: the K lowest
    blocks.  Both against qsa_topk_blocks on the scores and against the
    selection written out from the planted classes."""
    torch = _torch()
    Tq, pos0, K = 300, 140000, 512
    nb = (pos0 + Tq) // 4
    rng = np.random.default_rng(5)
    kb = np.zeros((nb, 128), dtype=np.uint16)
    qi = np.zeros((Tq, 4, 128), dtype=np.uint16)
    two = one = np.zeros(0, dtype=np.int64)
    if case == "tie_classes":
        perm = rng.permutation(pos0 // 4)  # blocks every row sees
        two, one = np.sort(perm[:300]), np.sort(perm[300:700])
        kb[:, 0] = 0xBF80  # -1: negative dot products for head 0
        kb[two, 0] = 0x4000  # 2.0
        kb[one, 0] = 0x3F80  # 1.0
        qi[:, 0, 0] = 0x3F80
    ld = (nb + 3) // 4 * 4
    qd, kd = dev(qi), dev(kb)
    sc = torch.empty((Tq, ld), dtype=torch.float32, device="cuda")
    qsa.qsa_index_scores(qd, kd, 1, Tq, pos0, None, nb, 4, 128, 4, 0, sc, ld)
    b1, n1 = run_topk(qsa, sc, 1, Tq, ld, pos0, None, nb, K)
    wsb = qsa.qsa_select_workspace_bytes(1, Tq, nb, K)
    ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device="cuda")
    b2 = torch.full((Tq, K), 7, dtype=torch.int32, device="cuda")
    n2 = torch.full((Tq,), 7, dtype=torch.int32, device="cuda")
    qsa.qsa_select_blocks(qd, kd, 1, Tq, pos0, None, nb, 4, 128, 4, 0, K, b2, n2, ws, wsb)
    torch.cuda.synchronize()
    b2, n2 = b2.cpu().numpy(), n2.cpu().numpy()
    if case == "tie_classes":
        want = np.sort(np.concatenate([two, one[:K - two.size]]))
    else:
        want = np.arange(K)
    assert np.all(n2 == K)
    for t in range(Tq):
        assert np.array_equal(b2[t], want), t
    assert np.array_equal(n1, n2) and np.array_equal(b1, b2)


def _decode_select(qsa, qi, kb, lens, K, mode=0):
    """qsa_select_blocks in the decode form; also returns the GPU scores."""
    torch = _torch()
    B, nb_max = kb.shape[0], kb.shape[1]
    ld = (nb_max + 3) // 4 * 4
    qd, kd, ln = dev(qi), dev(kb), dev(lens)
    sc = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    qsa.qsa_index_scores(qd, kd, B, 1, 0, ln, nb_max, 4, 128, 4, mode, sc, ld)
    blk = torch.full((B, K), 7, dtype=torch.int32, device="cuda")
    ns = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    wsb = qsa.qsa_select_workspace_bytes(B, 1, nb_max, K)
    ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device="cuda")
    qsa.qsa_select_blocks(qd, kd, B, 1, 0, ln, nb_max, 4, 128, 4, mode, K, blk, ns, ws, wsb)
    torch.cuda.synchronize()
    return sc.cpu().numpy(), blk.cpu().numpy(), ns.cpu().numpy()


def _check_decode_rows(scores, blk, ns, lens, nb_max, K):
    """Each row's selection is the exact (score desc, index asc) top-K of the
    row's GPU scores."""
    for b in range(lens.size):
        nc = min(int(lens[b]) // 4, nb_max)
        row = scores[b, :nc].astype(np.float64)
        row[row == 0] = 0.0
        want, _, _ = oracle.topk_row(row, K)
        assert ns[b] == want.size, (b, int(ns[b]), want.size)
        assert np.array_equal(blk[b, :ns[b]], want), b
        assert np.all(blk[b, ns[b]:] == -1), b


@pytest.mark.parametrize("K,mode", [(512, 0), (512, 1), (2048, 0), (64, 0)])
def test_select_decode_form_long_rows(qsa, K, mode):
    """Decode-form selection over long pooled-key caches (the filter pass on
    a floor from the scan's group maxima, then one exact pass per row), with
    ragged lengths: rows at or under K, rows too short for the floor (all
    keys kept, packed or streamed), a ragged last segment, needle blocks,
    rows of 16 and 300 distinct pooled keys (ties at the threshold) and an
    all-equal row (lists beyond the LDS capacity: streamed)."""
    nb_max = 65536 + 7
    lens = np.array([4 * nb_max, 4 * nb_max - 1, 4 * 40000 + 3, 4 * 20000, 4 * 6000, 4 * K + 3,
                     1, 4 * 33000, 4 * nb_max, 4 * nb_max, 4 * nb_max], dtype=np.int64)
    B = lens.size
    qi = synth.normal_bf16(4, (B, 4, 128), seed=21)
    kb = synth.normal_bf16(5, (B, nb_max, 128), seed=21)
    rng = np.random.default_rng(21)
    # needles: 40 blocks of row 2 scaled by 4 (bf16 exponent + 2)
    nd = rng.choice(40000, 40, replace=False)
    kb[2, nd] = (kb[2, nd].astype(np.uint32) + (2 << 7)).astype(np.uint16)
    kb[8] = kb[8, rng.integers(0, 16, nb_max)]          # 16 distinct keys
    kb[9] = kb[9, rng.integers(0, 300, nb_max)]         # 300 distinct keys
    kb[10] = kb[10, 0]                                  # all equal
    scores, blk, ns = _decode_select(qsa, qi, kb, lens, K, mode)
    _check_decode_rows(scores, blk, ns, lens, nb_max, K)


def test_select_decode_form_million_tokens(qsa):
    """Decode-form selection at 1,048,576 tokens (4,096 groups per row) with
    needle blocks, and a row whose scores agree with the old path's."""
    nb_max, K = 262144, 512
    lens = np.array([4 * nb_max, 4 * nb_max - 2, 4 * 200000 + 1], dtype=np.int64)
    B = lens.size
    qi = synth.normal_bf16(4, (B, 4, 128), seed=22)
    kb = synth.normal_bf16(5, (B, nb_max, 128), seed=22)
    nd = np.random.default_rng(22).choice(nb_max, 64, replace=False)
    kb[0, nd] = (kb[0, nd].astype(np.uint32) + (2 << 7)).astype(np.uint16)
    scores, blk, ns = _decode_select(qsa, qi, kb, lens, K)
    _check_decode_rows(scores, blk, ns, lens, nb_max, K)
    g, n = run_topk(qsa, dev(scores), B, 1, nb_max, 0, dev(lens), nb_max, K)
    assert np.array_equal(g, blk) and np.array_equal(n, ns)


# ---------------------------------------------------------- A6 attention
def test_sparse_prefill_attention_parity(qsa):
    torch = _torch()
    T, K = 1029, 64
    x = synth.prefill_inputs(T, seed=10)
    Qr, Kr = oracle.rope(x.Q), oracle.rope(x.K)
    kb = oracle.compress(x.ki)
    rows = np.arange(T)
    sel = oracle.select_rows(x.qi, kb, rows, Kbudget=K)
    O = torch.empty((T, 24, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, 24), dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_prefill(dev(Qr), dev(Kr), dev(x.V), dev(sel["sel"]), dev(sel["nsel"]), T,
                                T, 0, 24, 2, 256, 4, K, O, lse)
    torch.cuda.synchronize()
    Oref, lref = oracle.sparse_attn_rows(Qr, Kr, x.V, rows, sel["sel"], sel["nsel"])
    assert_close(O.cpu().numpy(), Oref, "sparse prefill O")
    assert_close(lse.cpu().numpy(), lref, "sparse prefill lse")


def _random_selection(T, pos0, K, seed):
    """Valid selections: row t takes min(K, nc) distinct complete blocks
    (nc = (pos0 + t + 1) // 4) in ascending order, padded with -1."""
    rng = np.random.default_rng(seed)
    blk = np.full((T, K), -1, dtype=np.int32)
    nsel = np.empty(T, dtype=np.int32)
    for t in range(T):
        nc = (pos0 + t + 1) // 4
        n = min(K, nc)
        if n:
            blk[t, :n] = np.sort(rng.choice(nc, size=n, replace=False))
        nsel[t] = n
    return blk, nsel


@pytest.mark.parametrize("T,pos0,H,Hkv,rope_dim,theta,K", [
    (1029, 0, 24, 2, 64, 1e7, 64),          # the model's heads, ragged tail
    (333, 70001, 24, 2, 64, 1e7, 512),      # full budget, positions past 2^16
    (517, 4093, 16, 1, 128, 1e4, 128),      # rope over 128 dims, one KV head
    (260, 1000, 32, 4, 64, 5e5, 256),       # four KV heads
])
def test_sparse_prefill_rope_on_load(qsa, T, pos0, H, Hkv, rope_dim, theta, K):
    """The queries rotated as the attention loads them: O and lse equal, bit
    for bit, the RoPE kernel followed by the plain sparse attention, and
    sampled rows match the oracle (its RoPE, then its attention)."""
    torch = _torch()
    log(f"rope on load T={T} pos0={pos0} H={H} Hkv={Hkv} rope_dim={rope_dim} theta={theta} K={K}")
    Tk = pos0 + T
    Q = synth.normal_bf16(1, (T, H, 256), seed=70 + T)
    Kc = synth.normal_bf16(2, (Tk, Hkv, 256), seed=70 + T)
    V = synth.normal_bf16(3, (Tk, Hkv, 256), seed=70 + T)
    blk, nsel = _random_selection(T, pos0, K, seed=T)
    Qd, Kd, Vd, bd, nd = dev(Q), dev(Kc), dev(V), dev(blk), dev(nsel)
    Qr = torch.empty_like(Qd)
    qsa.qsa_rope_bf16(Qd, Qr, T, H, 256, rope_dim, theta, pos0)
    outs = []
    for fused in (False, True):
        O = torch.full((T, H, 256), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            qsa.qsa_sparse_attn_prefill_rope(Qd, Kd, Vd, bd, nd, T, Tk, pos0, H, Hkv, 256, 4, K,
                                             rope_dim, theta, O, lse)
        else:
            qsa.qsa_sparse_attn_prefill(Qr, Kd, Vd, bd, nd, T, Tk, pos0, H, Hkv, 256, 4, K, O, lse)
        torch.cuda.synchronize()
        outs.append((O.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32)), "O"
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32)), "lse"
    rows = np.unique(np.array([0, 1, 2, 3, 4, T // 2, T - 2, T - 1]))
    Qo = oracle.rope(Q, rope_dim=rope_dim, theta=theta, pos0=pos0)
    Oref, lref = oracle.sparse_attn_rows(Qo, Kc, V, rows, blk[rows], nsel[rows], pos0=pos0)
    assert_close(outs[1][0][rows], Oref, "rope-on-load O vs oracle")
    assert_close(outs[1][1][rows], lref, "rope-on-load lse vs oracle")


def test_decode_attention_parity(qsa):
    torch = _torch()
    B, Lmax, K = 5, 5000, 64
    lens = np.array([1, 2, 7, 4096, 4999], dtype=np.int64)
    Kc = synth.normal_bf16(2, (B, Lmax, 2, 256), seed=11)
    Vc = synth.normal_bf16(3, (B, Lmax, 2, 256), seed=11)
    q = synth.normal_bf16(1, (B, 24, 256), seed=11)
    rng = np.random.default_rng(0)
    sel = np.full((B, K), -1, dtype=np.int32)
    nsel = np.zeros(B, dtype=np.int32)
    for b in range(B):
        nc = int(lens[b]) // 4
        m = min(K, nc)
        sel[b, :m] = np.sort(rng.choice(nc, size=m, replace=False)) if m else []
        nsel[b] = m
    wsb = qsa.qsa_decode_workspace_bytes(B, 1, 24, 2, 256, K)
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    O = torch.empty((B, 24, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, 24), dtype=torch.float32, device="cuda")
    qsa.qsa_sparse_attn_decode(dev(q), dev(Kc), dev(Vc), dev(lens), dev(sel), dev(nsel), B, 1,
                               Lmax, 24, 2, 256, 4, K, O, lse, ws, wsb)
    torch.cuda.synchronize()
    Og, lg = O.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        L = int(lens[b])
        Oref, lref = oracle.sparse_attn_rows(q[b:b + 1], Kc[b, :L], Vc[b, :L], np.array([0]),
                                             sel[b:b + 1], nsel[b:b + 1], pos0=L - 1)
        assert_close(Og[b], Oref[0], f"decode seq {b} (L={L}) O")
        assert_close(lg[b], lref[0], f"decode seq {b} lse")


@pytest.mark.parametrize("lens,n,H,Hkv,rope_dim,theta,K,P", [
    ((1, 2, 7, 4096, 4999), 1, 24, 2, 64, 1e7, 64, 0),   # the model's heads, short lengths
    ((3001, 2, 20003), 4, 24, 2, 64, 1e7, 512, 0),       # speculative queries: tiles of 2 positions
    ((5000, 3), 16, 4, 4, 128, 1e4, 128, 0),             # one head per KV head: 16 positions a tile
    ((4097, 1030, 70001), 5, 32, 4, 64, 5e5, 256, 64),   # paged caches, 8 heads per KV head
    ((3000, 65), 16, 32, 2, 64, 1e7, 256, 0),            # 16 column tiles in 4 workgroup groups
])
def test_decode_rope_on_load(qsa, lens, n, H, Hkv, rope_dim, theta, K, P):
    """The decode attention rotating its queries as it loads them: O and lse
    equal, bit for bit, the RoPE kernel's decode form followed by the plain
    decode attention (contiguous or paged), and every query matches the
    oracle (its RoPE at the query's position, then its attention over the
    shared selection and the query's own tail)."""
    torch = _torch()
    from test_gpu_paged import page_layout, to_pool
    lens = np.array(lens, dtype=np.int64)
    B, Lmax = lens.size, int(lens.max())
    log(f"decode rope on load lens={lens.tolist()} next_n={n} H={H} Hkv={Hkv} "
        f"rope_dim={rope_dim} K={K} pages={P}")
    Kc = synth.normal_bf16(2, (B, Lmax, Hkv, 256), seed=80 + n)
    Vc = synth.normal_bf16(3, (B, Lmax, Hkv, 256), seed=80 + n)
    q = synth.normal_bf16(1, (B, n, H, 256), seed=80 + n)
    rng = np.random.default_rng(n)
    sel = np.full((B, K), -1, dtype=np.int32)
    nsel = np.zeros(B, dtype=np.int32)
    for b in range(B):
        p0 = int(lens[b]) - n
        nc = oracle.num_complete(p0) if p0 >= 0 else 0
        m = min(K, nc)
        if m:
            sel[b, :m] = np.sort(rng.choice(nc, size=m, replace=False))
        nsel[b] = m
    pg = None
    if P:
        table, total = page_layout(lens, Lmax, P, seed=P)
        pg = qsa.Pages(dev(table), P)
        kc = dev(to_pool(Kc, table, total, P, valid=lens))
        vc = dev(to_pool(Vc, table, total, P, valid=lens))
    else:
        kc, vc = dev(Kc), dev(Vc)
    qd, ln, sd, nd = dev(q), dev(lens), dev(sel), dev(nsel)
    qr = torch.empty_like(qd)
    qsa.qsa_rope_bf16(qd, qr, B * n, H, 256, rope_dim, theta, 0, ln, n)
    wsb = qsa.qsa_decode_workspace_bytes(B, n, H, Hkv, 256, K)
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    outs = []
    for fused in (False, True):
        O = torch.full((B, n, H, 256), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, n, H), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            qsa.qsa_sparse_attn_decode_rope(qd, kc, vc, ln, sd, nd, B, n, Lmax, H, Hkv, 256, 4, K,
                                            rope_dim, theta, O, lse, ws, wsb, pages=pg)
        else:
            qsa.qsa_sparse_attn_decode(qr, kc, vc, ln, sd, nd, B, n, Lmax, H, Hkv, 256, 4, K, O,
                                       lse, ws, wsb, pages=pg)
        torch.cuda.synchronize()
        outs.append((O.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32)), "O"
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32)), "lse"
    Og, lg = outs[1]
    got, ref, gl, rl = [], [], [], []
    for b in range(B):
        L = int(lens[b])
        p0 = L - n
        for i in range(n):
            p = p0 + i
            if p < 0:
                assert np.all(Og[b, i] == 0) and np.all(np.isneginf(lg[b, i])), f"seq {b} q {i}"
                continue
            if p0 < 0:
                tok = np.arange(p + 1)   # no complete block before the first query: every token
            else:
                tok = oracle.token_set_reuse(sel[b, :nsel[b]], p0, p)
            qo = oracle.rope(q[b, i:i + 1], rope_dim=rope_dim, theta=theta, pos=np.array([p]))
            o, l, _ = oracle.attend_row(qo[0], Kc[b], Vc[b], tok)
            got.append(Og[b, i])
            gl.append(lg[b, i])
            ref.append(o)
            rl.append(l)
    assert_close(np.stack(got), np.stack(ref), "decode rope-on-load O vs oracle")
    assert_close(np.stack(gl), np.stack(rl), "decode rope-on-load lse vs oracle")


# ------------------------------------------------------------- A8 dense
@pytest.mark.parametrize("B,Tq,pos0", [(1, 517, 0), (1, 200, 777), (1, 1, 1000), (1, 129, 64),
                                       (2, 100, 50)])
def test_dense_prefill_flash_parity(qsa, B, Tq, pos0):
    """Flash prefill over several 128-query blocks and 64-token tiles, ragged
    tails, a chunk after pos0 cached tokens, one query, two sequences."""
    torch = _torch()
    Tk = pos0 + Tq
    xs = [synth.prefill_inputs(Tq, pos0=pos0, seed=40 + 7 * b + Tq) for b in range(B)]
    Q = np.stack([x.Q for x in xs])
    K = np.stack([x.K for x in xs])
    V = np.stack([x.V for x in xs])
    O = torch.empty((B, Tq, 24, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Tq, 24), dtype=torch.float32, device="cuda")
    qsa.dense_attn(dev(Q), dev(K), dev(V), B, Tq, Tk, pos0, None, 24, 2, 256, O, lse)
    torch.cuda.synchronize()
    Og, lg = O.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        Oref, lref = oracle.dense_rows(Q[b], K[b], V[b], np.arange(Tq), pos0=pos0)
        assert_close(Og[b], Oref, f"flash prefill O (seq {b})")
        assert_close(lg[b], lref, f"flash prefill lse (seq {b})")


def test_dense_prefill_and_decode_parity(qsa):
    torch = _torch()
    T = 300
    x = synth.prefill_inputs(T, seed=12)
    O = torch.empty((T, 24, 256), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, 24), dtype=torch.float32, device="cuda")
    qsa.dense_attn(dev(x.Q), dev(x.K), dev(x.V), 1, T, T, 0, None, 24, 2, 256, O, lse)
    torch.cuda.synchronize()
    rows = np.arange(T)
    Oref, lref = oracle.dense_rows(x.Q, x.K, x.V, rows)
    assert_close(O.cpu().numpy(), Oref, "dense prefill O")
    assert_close(lse.cpu().numpy(), lref, "dense prefill lse")
    # decode form over the same keys, query at L-1
    B, Lmax = 2, T
    lens = np.array([T, 77], dtype=np.int64)
    Kc = np.stack([x.K, x.K])
    Vc = np.stack([x.V, x.V])
    q = np.stack([x.Q[T - 1], x.Q[76]])
    wsb = qsa.dense_attn_workspace_bytes(B, 1, Lmax, 24, 2, 256)
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    Od = torch.empty((B, 24, 256), dtype=torch.float32, device="cuda")
    qsa.dense_attn(dev(q), dev(Kc), dev(Vc), B, 1, Lmax, 0, dev(lens), 24, 2, 256, Od, None, ws,
                   wsb)
    torch.cuda.synchronize()
    assert_close(Od.cpu().numpy()[0], Oref[T - 1], "dense decode O (L=300)")
    assert_close(Od.cpu().numpy()[1], Oref[76], "dense decode O (L=77)")
