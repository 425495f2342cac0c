"""The Python binding checks each tensor argument before a call (on the CPU,
no GPU needed): it must be a GPU tensor with the element size the call reads
and hold the bytes the call's size arguments imply, else ValueError, so a
short or mistyped tensor never reaches a kernel.  Every case here fails in
the checks, before the C library is called."""
import pytest
import torch

import block_sparse_long_08_amd as qsa


@pytest.fixture
def host_ok(monkeypatch):
    """Let host tensors through the device check so that the size and
    element checks can be exercised without a GPU."""
    monkeypatch.setattr(qsa, "_REQUIRE_GPU", False)


def test_host_tensors_are_rejected():
    x = torch.zeros((4, 24, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="not a GPU tensor"):
        qsa.qsa_rope_bf16(x, x, 4, 24, 256)


def test_short_and_mistyped_tensors(host_ok):
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)  # noqa: E731
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)  # noqa: E731
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
    with pytest.raises(ValueError, match="needs"):
        qsa.qsa_rope_bf16(bf(4, 24, 256), bf(3, 24, 256), 4, 24, 256)
    with pytest.raises(ValueError, match="byte elements"):
        qsa.qsa_rope_bf16(f32(4, 24, 256), bf(4, 24, 256), 4, 24, 256)
    T, K = 64, 8
    Q, Kc, V = bf(T, 24, 256), bf(T, 2, 256), bf(T, 2, 256)
    blk, ns = i32(T, K), i32(T)
    with pytest.raises(ValueError, match="O holds"):
        qsa.qsa_sparse_attn_prefill(Q, Kc, V, blk, ns, T, T, 0, 24, 2, 256, 4, K, f32(T - 1, 24, 256))
    with pytest.raises(ValueError, match="blk_idx holds"):
        qsa.qsa_sparse_attn_prefill(Q, Kc, V, i32(T, K - 1), ns, T, T, 0, 24, 2, 256, 4, K,
                                    f32(T, 24, 256))
    with pytest.raises(ValueError, match="K holds"):
        qsa.qsa_sparse_attn_prefill(Q, bf(T - 1, 2, 256), V, blk, ns, T, T, 0, 24, 2, 256, 4, K,
                                    f32(T, 24, 256))
    with pytest.raises(ValueError, match="byte elements"):
        qsa.qsa_sparse_attn_prefill(Q, Kc, V, blk.to(torch.int64), ns, T, T, 0, 24, 2, 256, 4, K,
                                    f32(T, 24, 256))
    # decode: the caches of B sequences, the selection rows, the workspace
    B, L = 3, 400
    q, kc, vc = bf(B, 24, 256), bf(B, L, 2, 256), bf(B, L, 2, 256)
    sl = torch.full((B,), L, dtype=torch.int64)
    with pytest.raises(ValueError, match="Kc holds"):
        qsa.qsa_sparse_attn_decode(q, bf(2, L, 2, 256), vc, sl, i32(B, K), i32(B), B, 1, L, 24, 2, 256, 4,
                                   K, f32(B, 24, 256), None, torch.zeros(10, dtype=torch.uint8), 10)
    with pytest.raises(ValueError, match="ws holds"):
        qsa.qsa_sparse_attn_decode(q, kc, vc, sl, i32(B, K), i32(B), B, 1, L, 24, 2, 256, 4, K,
                                   f32(B, 24, 256), None, torch.zeros(10, dtype=torch.uint8), 11)
    with pytest.raises(ValueError, match="seq_len holds"):
        qsa.qsa_sparse_attn_decode_noalloc(q, kc, vc, sl[:2].clone(), i32(B, K), i32(B), B, 1, L, 24, 2,
                                           256, 4, K, f32(B, 24, 256))
    # a strided view that reaches the end of its storage is accepted by the
    # checks: pooling into the cache rows of block 10 onwards of 3 sequences
    # fails only on a cache too short for the last sequence's append
    kb = bf(B, L // 4, 128)
    ki = bf(B, 40, 128)
    with pytest.raises(ValueError, match="kbar holds"):
        qsa.qsa_compress_keys(ki, B, 40, 40 * 128, 128, 4, 0, kb[:, 95], (L // 4) * 128,
                              block0=95)
    with pytest.raises(ValueError, match="needs"):
        qsa.qsa_select_blocks(bf(T, 4, 128), bf(T // 4 - 1, 128), 1, T, 0, None, T // 4, 4, 128,
                              4, 0, K, i32(T, K), i32(T), torch.zeros(16, dtype=torch.uint8), 16)


def test_page_table_checks(host_ok):
    with pytest.raises(ValueError, match="byte elements"):
        qsa.Pages(torch.zeros((2, 8), dtype=torch.int64), 64)
    with pytest.raises(ValueError, match="contiguous"):
        qsa.Pages(torch.zeros((2, 8), dtype=torch.int32).t(), 64)
