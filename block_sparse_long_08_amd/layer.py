"""The QSA layer's two hot paths as chains of C-ABI calls.

Each class owns its outputs and workspaces (torch device memory, allocated
once) and enqueues the steps of the method on the current stream:

prefill (chlience section 6): A1 RoPE on Q (by default inside the attention
kernel, as it loads the queries) and on K for a fresh context,
A2 pooling of the indexer keys, A3+A4 block scores and top-K selection,
A5+A6 sparse attention over the selected blocks plus the trailing block;
decode: A1 on the new query, optional A2 of a block the new token completes,
A3+A4 over the pooled-key cache, A7 split-K sparse attention.
"""
from __future__ import annotations

import torch

from . import (DI, HI, R, SCORE_MAXHEAD, KBAR_MEAN, qsa_compress_keys, qsa_decode_workspace_bytes,
               qsa_rope_bf16, qsa_select_blocks, qsa_select_workspace_bytes,
               qsa_sparse_attn_decode, qsa_sparse_attn_decode_rope, qsa_sparse_attn_prefill,
               qsa_sparse_attn_prefill_concurrency, qsa_sparse_attn_prefill_kl,
               qsa_sparse_attn_prefill_kl_staged, qsa_sparse_attn_prefill_kl_staged_workspace_bytes,
               qsa_sparse_attn_prefill_rope)


# rows per sparse-attention launch of the prefill when the device does not
# report how many of its workgroups it holds at once, or when one round of
# them would select each cached block fewer than SWEEP_REUSE times
ATTN_ROWS = 4096
SWEEP_REUSE = 8


class QSAPrefill:
    """Prefill of Tq queries at positions pos0 .. pos0+Tq-1 of one sequence.

    fresh=True: K is raw and rotated here, and the whole indexer-key input
    is pooled.  fresh=False: K is a post-RoPE cache and only the chunk's own
    indexer keys (positions pos0 ..) are pooled into the caller's kbar cache
    (pos0 must then be a multiple of r).

    rope_on_load (rope_dim 64 or 128): the sparse attention rotates the
    queries as it loads them (bit for bit the rotated queries), so the
    rotated copy is neither written nor read back; Q must then stay unchanged
    until attend() has run.  The Qr attribute still gives the rotated
    queries: it is computed on first use after rope_and_pool (the fused KL,
    dense references).  Otherwise Q is rotated into Qr by rope_and_pool.

    idx_rope_dim > 0: partial RoPE on the indexer (pooled keys rotated at their
    block's first token, indexer queries at their own positions); kbar_gain:
    the RMSNorm gain of the pooled keys (kbar_mode RMSNORM), bf16 [DI].

    The selection of all rows runs first (one call; the library scores the
    rows in chunks of at most 8 GiB of scores), then the sparse attention in
    launches of attn_rows rows.  The attention runs one one-wave workgroup
    per query and KV head, and the device deals workgroups to its XCDs in
    turn, so each XCD gathers the rows of one KV head.  By default a launch
    holds as many queries as the device runs workgroups of the kernel at
    once (1,536 on MI355X at Hkv = 2, budget 512): every query costs about
    the same, so workgroups run in rounds of that size, and each query walks
    its block list in ascending block order: within one round the
    concurrent gathers sweep the cache as a narrow band, which L2 and the
    Infinity Cache hold.  Launches that span several rounds let the
    workgroups drift apart and the band widen.  The 128K prefill's attention
    takes 41.0 ms in 1,536-row launches, 42.1 ms in 3,072-row launches,
    42.6 ms in 4,096-row launches and 58.4 ms as one launch of 131,072 rows
    (attn_rows <= 0 asks for that one launch); half-round launches leave CUs
    idle (768 rows: 60.8 ms).  The sweep pays only when a round's
    selections repeat each cached block: 1,536 x 512 selections over 32,768
    blocks come to 24 per block at 128K, but 3 at a 1M-token context, where
    4,096-row launches are faster (3.98 against 4.11-4.24 ms per 8,192
    queries); the default takes one-round launches at 8 or more per block.
    The KL form (attend_with_kl) launches kl_rows rows, by default the
    plain kernel's round.
    pipeline_rows > 0 (and < Tq) instead selects the queries in chunks of
    that many rows and runs each chunk's attention on a second stream while
    the next chunk is selected; the results are those of the stages run one
    after the other.  It is off by default: the selection's score traffic
    slows the attention more than the overlap saves (128K: 60.8 ms
    overlapped in 4,096-row chunks against 0.7 + 6.5 + 48.7 ms in turn; a
    1M-context chunk of 8,192 rows 8.40 against 7.9 ms).
    """

    def __init__(self, Tq: int, pos0: int = 0, H: int = 24, Hkv: int = 2, D: int = 256,
                 budget: int = 512, score_mode: int = SCORE_MAXHEAD, kbar_mode: int = KBAR_MEAN,
                 theta: float = 1e7, rope_dim: int = 64, fresh: bool = True,
                 idx_rope_dim: int = 0, kbar_gain=None, pages=None, pipeline_rows: int = 0,
                 attn_rows: int | None = None, kl_rows: int | None = None,
                 rope_on_load: bool = True, kl_staged: bool = True, device="cuda"):
        self.Tq, self.pos0, self.H, self.Hkv, self.D = Tq, pos0, H, Hkv, D
        self.pages = pages  # paged caches (fresh=False): K, V and kbar are page pools
        self.Tk = pos0 + Tq
        self.budget, self.score_mode, self.kbar_mode = budget, score_mode, kbar_mode
        self.theta, self.rope_dim, self.fresh = theta, rope_dim, fresh
        self.idx_rope_dim, self.kbar_gain = idx_rope_dim, kbar_gain
        self.nb = self.Tk // R
        dev = torch.device(device)
        self.dev = dev
        self.rope_on_load = bool(rope_on_load) and rope_dim in (64, 128)
        self._Qr = None          # rotated queries, allocated on first use
        self._q = None           # the queries of the last rope_and_pool
        self._qr_current = False  # _Qr holds the rotation of _q
        self.Kr = torch.empty((self.Tk, Hkv, D), dtype=torch.bfloat16, device=dev) if fresh else None
        self.kbar = (torch.empty((max(self.nb, 1), DI), dtype=torch.bfloat16, device=dev)
                     if fresh else None)
        if pages is not None and fresh:
            raise ValueError("paged caches hold earlier context: use fresh=False")
        self.blk_idx = torch.empty((Tq, budget), dtype=torch.int32, device=dev)
        self.n_sel = torch.empty((Tq,), dtype=torch.int32, device=dev)
        self.O = torch.empty((Tq, H, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
        self.pipeline_rows = pipeline_rows if 0 < pipeline_rows < Tq else 0
        if attn_rows is None:
            conc = qsa_sparse_attn_prefill_concurrency(Hkv, budget, paged=pages is not None)
            # one round per launch when a round's selections hit each cached
            # block several times over (the in-step sweep pays), else
            # larger launches (fewer launch tails)
            attn_rows = (conc if conc > 0 and conc * budget >= SWEEP_REUSE * max(self.nb, 1)
                         else max(conc, ATTN_ROWS))
        self.attn_rows = self.pipeline_rows or (attn_rows if attn_rows > 0 else Tq)
        if kl_rows is None:
            kl_rows = qsa_sparse_attn_prefill_concurrency(Hkv, budget) or ATTN_ROWS
        self.kl_rows = kl_rows if kl_rows > 0 else Tq
        self.kl_staged = kl_staged
        self._kl_ws = None  # workspace of the staged KL form, allocated on first use
        self.ws_bytes = qsa_select_workspace_bytes(1, self.pipeline_rows or Tq, self.nb, budget)
        self.ws = torch.empty((max(self.ws_bytes, 16),), dtype=torch.uint8, device=dev)
        # the attention stream of the pipeline (default priority)
        self.side = torch.cuda.Stream(device=dev) if self.pipeline_rows else None
        self.qir = (torch.empty((Tq, HI, DI), dtype=torch.bfloat16, device=dev)
                    if idx_rope_dim else None)

    @property
    def Qr(self):
        """The rotated queries [Tq, H, D] of the last rope_and_pool."""
        if self._Qr is None:
            self._Qr = torch.empty((self.Tq, self.H, self.D), dtype=torch.bfloat16,
                                   device=self.dev)
        if not self._qr_current:
            if self._q is None:
                raise RuntimeError("QSAPrefill.Qr: rope_and_pool has not run")
            qsa_rope_bf16(self._q, self._Qr, self.Tq, self.H, self.D, self.rope_dim, self.theta,
                          self.pos0)
            self._qr_current = True
        return self._Qr

    def rope_and_pool(self, Q, K, ki, kbar=None):
        self._q, self._qr_current = Q, False
        if not self.rope_on_load:
            _ = self.Qr  # rotates Q now
        pool = dict(gain=self.kbar_gain, rope_dim=self.idx_rope_dim, theta=self.theta)
        if self.fresh:
            qsa_rope_bf16(K, self.Kr, self.Tk, self.Hkv, self.D, self.rope_dim, self.theta, 0)
            qsa_compress_keys(ki, 1, self.Tk, self.Tk * DI, DI, R, self.kbar_mode, self.kbar,
                              self.nb * DI, **pool)
            return self.Kr, self.kbar
        # pool the chunk's own keys into the cache (blocks pos0/r ..)
        b0 = self.pos0 // R
        dst = kbar if self.pages is not None else kbar[b0:]
        qsa_compress_keys(ki[self.pos0:], 1, self.Tq, self.Tq * DI, DI, R, self.kbar_mode,
                          dst, self.Tq // R * DI, block0=b0, pages=self.pages, **pool)
        return K, kbar

    def rope_indexer(self, qi):
        """The indexer queries the scores use: qi, or qi rotated at positions
        pos0 + t when the indexer has partial RoPE."""
        if not self.idx_rope_dim:
            return qi
        qsa_rope_bf16(qi, self.qir, self.Tq, HI, DI, self.idx_rope_dim, self.theta, self.pos0)
        return self.qir

    def _chunks(self, rows=None):
        c = rows or self.pipeline_rows or self.Tq
        return [(r0, min(c, self.Tq - r0)) for r0 in range(0, self.Tq, c)]

    def attn_chunks(self):
        """(first row, rows) of each sparse-attention launch."""
        return self._chunks(self.attn_rows)

    def _select_rows(self, qi, kbar, r0, n):
        qsa_select_blocks(qi[r0:r0 + n], kbar, 1, n, self.pos0 + r0, None, self.nb, HI, DI, R,
                          self.score_mode, self.budget, self.blk_idx[r0:r0 + n],
                          self.n_sel[r0:r0 + n], self.ws, self.ws_bytes, pages=self.pages)

    def _attend_rows(self, Kr, V, r0, n):
        p0 = self.pos0 + r0
        rows = (self.blk_idx[r0:r0 + n], self.n_sel[r0:r0 + n], n, p0 + n, p0, self.H, self.Hkv,
                self.D, R, self.budget)
        if self.rope_on_load:
            if self._q is None:
                raise RuntimeError("QSAPrefill.attend: rope_and_pool has not run")
            qsa_sparse_attn_prefill_rope(self._q[r0:r0 + n], Kr, V, *rows, self.rope_dim,
                                         self.theta, self.O[r0:r0 + n], self.lse[r0:r0 + n],
                                         pages=self.pages)
        else:
            qsa_sparse_attn_prefill(self.Qr[r0:r0 + n], Kr, V, *rows, self.O[r0:r0 + n],
                                    self.lse[r0:r0 + n], pages=self.pages)

    def attend_with_kl(self, Kr, V, qi, kbar, kl):
        """Training form of attend(), after select(): the sparse attention of
        every row fused with the distillation KL under the sparse pattern
        (kl: fp32 [Tq]); qi and kbar as given to the selection (qi after
        rope_indexer).  Contiguous caches; launches of kl_rows rows.  By
        default the staged form (the plain attention writing each selected
        block's max logits, then the KL: the attention's head placement and
        occupancy; a workspace of about 48 KB per row of a launch); with
        kl_staged=False the one-kernel form (everything on chip).  Both give
        the same bits."""
        if self.pages is not None:
            raise ValueError("attend_with_kl: the fused KL runs on contiguous caches only")
        rows = min(self.kl_rows, self.Tq)
        if self.kl_staged and self._kl_ws is None:
            wsb = qsa_sparse_attn_prefill_kl_staged_workspace_bytes(rows, self.budget)
            self._kl_ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=self.dev)
        for r0, n in self._chunks(rows):
            p0 = self.pos0 + r0
            sel = (self.blk_idx[r0:r0 + n], self.n_sel[r0:r0 + n], n, p0 + n, p0, self.H,
                   self.Hkv, self.D, HI, DI, R, self.budget, self.score_mode,
                   self.O[r0:r0 + n], self.lse[r0:r0 + n], kl[r0:r0 + n])
            if not self.kl_staged:
                qsa_sparse_attn_prefill_kl(self.Qr[r0:r0 + n], Kr, V, qi[r0:r0 + n], kbar, *sel)
                continue
            on_load = self.rope_on_load and self._q is not None
            q = self._q if on_load else self.Qr
            qsa_sparse_attn_prefill_kl_staged(q[r0:r0 + n], Kr, V, qi[r0:r0 + n], kbar, *sel,
                                              self._kl_ws, self._kl_ws.numel(),
                                              rope_dim=self.rope_dim if on_load else 0,
                                              theta=self.theta)

    def select(self, qi, kbar):
        for r0, n in self._chunks():
            self._select_rows(qi, kbar, r0, n)

    def attend_chunks(self, Kr, V):
        """The sparse attention of every row, in its launches one after the
        other on the current stream."""
        for r0, n in self.attn_chunks():
            self._attend_rows(Kr, V, r0, n)

    def attend(self, Kr, V):
        self.attend_chunks(Kr, V)

    def select_and_attend(self, qi, kbar, Kr, V, attn_events=None, select_events=None):
        """Selection and sparse attention of every row; with pipeline_rows,
        the attention of each chunk on the second stream (after that chunk's
        selection) overlaps the selection of the next.  attn_events /
        select_events: lists that receive a timing event pair around each
        attention launch / each chunk's selection."""
        if not self.pipeline_rows:
            self.select(qi, kbar)
            self.attend(Kr, V)
            return
        main = torch.cuda.current_stream()
        for r0, n in self._chunks():
            if select_events is not None:
                s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s0.record()
            self._select_rows(qi, kbar, r0, n)
            if select_events is not None:
                s1.record()
                select_events.append((s0, s1))
            ready = torch.cuda.Event()
            ready.record(main)
            self.side.wait_event(ready)
            with torch.cuda.stream(self.side):
                if attn_events is not None:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                self._attend_rows(Kr, V, r0, n)
                if attn_events is not None:
                    e1.record()
                    attn_events.append((e0, e1))
        main.wait_stream(self.side)  # later work on the caller's stream sees O and lse

    def __call__(self, Q, K, V, qi, ki, kbar=None):
        Kr, kb = self.rope_and_pool(Q, K, ki, kbar)
        self.select_and_attend(self.rope_indexer(qi), kb, Kr, V)
        return self.O, self.lse


class QSADecode:
    """One decode step for B sequences over caches Kc/Vc [B, Lmax, Hkv, D]
    (post-RoPE) and kbar [B, Lmax/r, DI]: the next_n newest queries of
    sequence b sit at seq_len[b] - next_n .. seq_len[b] - 1.  With next_n > 1
    (speculative steps) the block selection is made once, for the first of
    them, and reused by all (each adds its own causal tail)."""

    def __init__(self, B: int, Lmax: int, H: int = 24, Hkv: int = 2, D: int = 256,
                 budget: int = 512, score_mode: int = SCORE_MAXHEAD, kbar_mode: int = KBAR_MEAN,
                 theta: float = 1e7, rope_dim: int = 64, next_n: int = 1,
                 idx_rope_dim: int = 0, kbar_gain=None, pages=None, rope_on_load: bool = True,
                 device="cuda"):
        self.B, self.Lmax, self.H, self.Hkv, self.D = B, Lmax, H, Hkv, D
        # rope_on_load (rope_dim 64 or 128): the attention rotates the queries
        # as it loads them (no RoPE launch, the rotated rows are not stored);
        # the qr property still gives them, computed on first use
        self.rope_on_load = bool(rope_on_load) and rope_dim in (64, 128)
        self.pages = pages  # paged caches: Kc, Vc and kbar are page pools
        self.budget, self.score_mode, self.kbar_mode = budget, score_mode, kbar_mode
        self.theta, self.rope_dim, self.next_n = theta, rope_dim, next_n
        self.idx_rope_dim, self.kbar_gain = idx_rope_dim, kbar_gain
        self.nb_max = Lmax // R
        dev = torch.device(device)
        n = next_n
        self.dev = dev
        self._qr = None
        self._q = self._seq_len = None
        self._qr_current = False
        self.blk_idx = torch.empty((B, budget), dtype=torch.int32, device=dev)
        self.n_sel = torch.empty((B,), dtype=torch.int32, device=dev)
        self.O = torch.empty((B, n, H, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, n, H), dtype=torch.float32, device=dev)
        self.sel_ws_bytes = qsa_select_workspace_bytes(B, n, self.nb_max, budget)
        self.sel_ws = torch.empty((max(self.sel_ws_bytes, 16),), dtype=torch.uint8, device=dev)
        self.dec_ws_bytes = qsa_decode_workspace_bytes(B, n, H, Hkv, D, budget)
        self.dec_ws = torch.empty((max(self.dec_ws_bytes, 16),), dtype=torch.uint8, device=dev)
        self.qir = (torch.empty((B, n, HI, DI), dtype=torch.bfloat16, device=dev)
                    if idx_rope_dim else None)

    @property
    def qr(self):
        """The rotated queries [B, next_n, H, D] of the last step."""
        if self._qr is None:
            self._qr = torch.empty((self.B, self.next_n, self.H, self.D), dtype=torch.bfloat16,
                                   device=self.dev)
        if not self._qr_current:
            if self._q is None:
                raise RuntimeError("QSADecode.qr: no step has run")
            qsa_rope_bf16(self._q, self._qr, self.B * self.next_n, self.H, self.D, self.rope_dim,
                          self.theta, 0, self._seq_len, self.next_n)
            self._qr_current = True
        return self._qr

    def pool_keys(self, ki, kbar, block0: int = 0):
        """Pool indexer keys ki [B, T, DI] (T a multiple of r) into kbar[:, block0 ..]."""
        T = ki.shape[1]
        dst = kbar if self.pages is not None else kbar[:, block0]
        qsa_compress_keys(ki, self.B, T, T * DI, DI, R, self.kbar_mode, dst,
                          self.nb_max * DI, gain=self.kbar_gain, rope_dim=self.idx_rope_dim,
                          theta=self.theta, block0=block0, pages=self.pages)

    def append_block(self, ki_tail, kbar, block: int):
        """Pool the r indexer keys ki_tail [B, r, DI] into kbar[:, block]."""
        self.pool_keys(ki_tail, kbar, block)

    def __call__(self, q, qi, Kc, Vc, kbar, seq_len):
        """q [B, next_n, H, D] and qi [B, next_n, HI, DI] (or [B, H, D] and
        [B, HI, DI] when next_n == 1); returns O [B, next_n, H, D] and lse
        [B, next_n, H] (O [B, H, D] and lse [B, H] when next_n == 1)."""
        n = self.next_n
        self._q, self._seq_len, self._qr_current = q, seq_len, False
        if not self.rope_on_load:
            q = self.qr
        if self.idx_rope_dim:  # indexer queries at their own positions
            qsa_rope_bf16(qi, self.qir, self.B * n, HI, DI, self.idx_rope_dim, self.theta, 0,
                          seq_len, n)
            qi = self.qir
        qsa_select_blocks(qi, kbar, self.B, n, 0, seq_len, self.nb_max, HI, DI, R,
                          self.score_mode, self.budget, self.blk_idx, self.n_sel, self.sel_ws,
                          self.sel_ws_bytes, pages=self.pages)
        if self.rope_on_load:
            qsa_sparse_attn_decode_rope(q, Kc, Vc, seq_len, self.blk_idx, self.n_sel, self.B, n,
                                        self.Lmax, self.H, self.Hkv, self.D, R, self.budget,
                                        self.rope_dim, self.theta, self.O, self.lse, self.dec_ws,
                                        self.dec_ws_bytes, pages=self.pages)
        else:
            qsa_sparse_attn_decode(q, Kc, Vc, seq_len, self.blk_idx, self.n_sel, self.B, n,
                                   self.Lmax, self.H, self.Hkv, self.D, R, self.budget, self.O,
                                   self.lse, self.dec_ws, self.dec_ws_bytes, pages=self.pages)
        if n == 1:
            return self.O[:, 0], self.lse[:, 0]
        return self.O, self.lse
