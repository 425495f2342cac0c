"""The no-allocation decode entry point (qsa_sparse_attn_decode_noalloc,
for callers that cannot allocate): through the C ABI, its outputs equal the
workspace form qsa_sparse_attn_decode's bit for bit on the same inputs, on
two calls in a row of which the second is smaller (fewer sequences, a
shorter budget and context, next_n 4 then 1), so the second call cannot
lean on records the first one left in the shared scratch."""
import numpy as np
import pytest

import synth
from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    import torch
    import block_sparse_long_08_amd as q
    assert torch.cuda.is_available()
    q.qsa_check_device()
    return q


def _case(qsa, B, Lmax, lens, n, budget, seed):
    import torch
    log(f"no-alloc decode: B={B} Lmax={Lmax} next_n={n} budget={budget}")
    Kc = dev(synth.normal_bf16(2, (B, Lmax, 2, 256), seed=seed))
    Vc = dev(synth.normal_bf16(3, (B, Lmax, 2, 256), seed=seed))
    q = dev(synth.normal_bf16(1, (B, n, 24, 256), seed=seed))
    ln = dev(np.asarray(lens, dtype=np.int64))
    # a valid selection per sequence: seeded distinct ascending blocks
    rng = np.random.default_rng(seed)
    blk = np.full((B, budget), -1, dtype=np.int32)
    nsel = np.zeros(B, dtype=np.int32)
    for b in range(B):
        nc = max(0, (int(lens[b]) - n + 1) // 4)
        k = min(budget, nc)
        blk[b, :k] = np.sort(rng.choice(nc, size=k, replace=False))
        nsel[b] = k
    blk_d, ns_d = dev(blk), dev(nsel)
    outs = []
    for noalloc in (False, True):
        O = torch.full((B, n, 24, 256), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, n, 24), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            qsa.qsa_sparse_attn_decode_noalloc(q, Kc, Vc, ln, blk_d, ns_d, B, n, Lmax, 24, 2, 256,
                                               4, budget, O, lse)
        else:
            wsb = qsa.qsa_decode_workspace_bytes(B, n, 24, 2, 256, budget)
            ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
            qsa.qsa_sparse_attn_decode(q, Kc, Vc, ln, blk_d, ns_d, B, n, Lmax, 24, 2, 256, 4,
                                       budget, O, lse, ws, wsb)
        torch.cuda.synchronize()
        outs.append((O.cpu().numpy(), lse.cpu().numpy()))
    (O0, l0), (O1, l1) = outs
    assert np.all(np.isfinite(O0)) and np.all(np.isfinite(O1))
    assert np.array_equal(O0, O1) and np.array_equal(l0, l1)
    return O1


def test_noalloc_decode_equals_workspace_form_twice(qsa):
    _case(qsa, 6, 40000, [40000, 12345, 39999, 2050, 777, 30001], 4, 512, seed=301)
    _case(qsa, 3, 9000, [9000, 4097, 6], 1, 64, seed=302)
