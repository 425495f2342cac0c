"""Stage-1 indexer distillation, forward (chlience section 6: the indexer is
first trained alone against the full attention distribution max-pooled
within each micro-block, by minimising KL).  qsa_distill_kl through the C
ABI, with the log-sum-exp of the library's dense attention, against the
fp64 oracle's per-row KL (oracle.distill_rows)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu

# the KL bar (derivation beside its definition)
from gpu_helpers import KL_ABS, KL_REL  # noqa: E402


@pytest.fixture(scope="module")
def qsa():
    import torch
    import block_sparse_long_08_amd as q
    assert torch.cuda.is_available()
    q.qsa_check_device()
    return q


def run_distill(qsa, Qr, K, qi, kbar, Tq, pos0, mode=0):
    """Dense attention for lse, then the distillation KL of the Tq rows."""
    import torch
    Tk = K.shape[0]
    dQ, dK = dev(Qr), dev(K)
    lse = torch.empty((1, Tq, 24), dtype=torch.float32, device="cuda")
    O = torch.empty((1, Tq, 24, 256), dtype=torch.float32, device="cuda")
    # lse does not depend on the values: the keys stand in for them
    qsa.dense_attn(dQ, dK, dK, 1, Tq, Tk, pos0, None, 24, 2, 256, O, lse)
    del O
    wsb = qsa.qsa_distill_workspace_bytes(Tq, Tk)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device="cuda") if wsb else None
    kl = torch.full((Tq,), float("nan"), dtype=torch.float32, device="cuda")
    if kbar.shape[0] == 0:  # no complete block: a placeholder row nobody reads
        kbar = np.zeros((1, 128), dtype=np.uint16)
    qsa.qsa_distill_kl(dQ, dK, lse, dev(qi), dev(kbar), Tq, Tk, pos0, 24, 2, 256, 4, 128, 4, mode,
                       kl, ws, wsb)
    torch.cuda.synchronize()
    return kl.cpu().numpy().astype(np.float64)


def check_kl(got, ref, what):
    err = np.abs(got - ref)
    w = int(np.argmax(err))
    rel = err / np.maximum(np.abs(ref), 1e-3)
    log(f"  {what}: max |dKL| {err.max():.3e} (KL there {ref[w]:.4f}), max |dKL|/|KL| "
        f"{rel.max():.3e}, KL range {ref.min():.3f} .. {ref.max():.3f}")
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= KL_ABS + KL_REL * np.abs(ref)), (what, float(err.max()))


@pytest.mark.parametrize("mode,needles", [(0, 0), (0, 8), (1, 0)])
def test_distill_all_rows(qsa, mode, needles):
    """T = 1000 from position 0 (rows 0..2 see no complete block: KL 0);
    every row against the oracle; two runs give the same bits."""
    T = 1000
    x = synth.prefill_inputs(T, seed=80 + needles, needles_per_head=needles)
    Qr, Kr = oracle.rope(x.Q), oracle.rope(x.K)
    kb = oracle.compress(x.ki)
    got = run_distill(qsa, Qr, Kr, x.qi, kb, T, 0, mode)
    ref = oracle.distill_rows(Qr, Kr, x.qi, kb, np.arange(T), 0, mode=mode)
    assert np.all(got[:3] == 0.0)
    check_kl(got, ref, f"mode {mode}, {needles} needles per head")
    again = run_distill(qsa, Qr, Kr, x.qi, kb, T, 0, mode)
    assert np.array_equal(got, again)


def test_distill_chunk_with_later_keys(qsa):
    """A chunk of 333 queries at pos0 = 5003 over a cache that also holds
    37 later tokens, which no row may see; sampled rows."""
    Tq, pos0, extra = 333, 5003, 37
    x = synth.prefill_inputs(Tq + extra, pos0=pos0, seed=84)
    Qr = oracle.rope(x.Q[:Tq], pos0=pos0)
    kb = oracle.compress(x.ki)
    got = run_distill(qsa, Qr, x.K, x.qi[:Tq], kb, Tq, pos0)
    rows = np.unique(np.r_[0, 1, 2, 3, np.arange(4, Tq, 11), Tq - 1])
    ref = oracle.distill_rows(Qr, x.K, x.qi[:Tq], kb, rows, pos0)
    check_kl(got[rows], ref, "pos0 5003 sampled rows")


def test_distill_tiny_contexts(qsa):
    """Contexts of 2 and 5 tokens: no block, then one complete block (the
    teacher and the student both put all mass on it: KL 0)."""
    for Tq in (2, 5):
        x = synth.prefill_inputs(Tq, seed=85)
        Qr, Kr = oracle.rope(x.Q), oracle.rope(x.K)
        kb = oracle.compress(x.ki)
        got = run_distill(qsa, Qr, Kr, x.qi, kb, Tq, 0)
        ref = oracle.distill_rows(Qr, Kr, x.qi, kb, np.arange(Tq), 0)
        assert np.all(np.abs(got) <= 1e-5) and np.all(np.abs(ref) <= 1e-12), (got, ref)


def test_distill_million_token_context_several_chunks(qsa):
    """8,500 queries ending a 1,048,576-token context: the row chunks of the
    workspace (8,192 rows at this length) split them 8192 + 308; rows at and
    next to the chunk edge and to an indexer workgroup edge (4,096) against
    the oracle."""
    Tk, Tq = 1 << 20, 8500
    pos0 = Tk - Tq
    K = synth.normal_bf16(synth.STREAM_K, (Tk, 2, 256), seed=86)
    ki = synth.normal_bf16(synth.STREAM_KIDX, (Tk, 128), seed=86)
    Q = synth.normal_bf16(synth.STREAM_Q, (Tq, 24, 256), seed=86)
    qi = synth.normal_bf16(synth.STREAM_QIDX, (Tq, 4, 128), seed=86)
    Qr = oracle.rope(Q, pos0=pos0)
    kb = oracle.compress(ki)
    got = run_distill(qsa, Qr, K, qi, kb, Tq, pos0)
    rows = np.array([0, 4095, 4096, 4097, 8191, 8192, 8499])
    ref = oracle.distill_rows(Qr, K, qi, kb, rows, pos0)
    check_kl(got[rows], ref, "1M context, chunk edges")
    assert np.all(np.isfinite(got)) and np.all(got >= -1e-6)
