"""Sliding-window evaluation of a token stream, with optional score-first test-time training of the
tied embedding, driven through the library's C ABI (include/pg_lmhead.h).

Windows of ``window`` tokens advance by ``stride`` over the stream; each scores only the predictions
no earlier window scored (parameter-golf README leaderboard, "Sliding Window Eval" row, stride 64).
Batches of ``windows_per_batch`` windows are scored one after another, and the bits per byte
accumulate over all of them on the device. With ``ttt_lr > 0`` each batch, once scored, also yields
the gradient of its mean loss with respect to the tied embedding (the hidden states' gradient only
with ``keep_dhidden``), and the embedding takes one SGD step on it before the next batch is
scored: score-first test-time training, every chunk adapted on only after it has been
scored (README leaderboard, "Legal Score-First TTT" rows, and the row that trains in phases on
validation chunks already scored).

This module only sequences calls: the schedule's arithmetic, the rows of each batch, the forward,
the backward, the sums and the update all run in the library. The hidden states of each batch
come from the caller (the model run on each window).
"""
from __future__ import annotations

from typing import Iterator, Optional, Tuple

import torch

from . import abi


class SlidingWindowEval:
    def __init__(self, tokens: torch.Tensor, byte_len: torch.Tensor, V: int, D: int, window: int = 2048,
                 stride: int = 64, windows_per_batch: int = 32, softcap: float = 30.0, ttt_lr: float = 0.0,
                 embed_master: Optional[torch.Tensor] = None, keep_dhidden: bool = False,
                 int8_head: bool = False):
        """keep_dhidden: with ttt_lr > 0, also compute the gradient of the hidden states of each
        batch (into self.dH). The embedding step needs only dE, so by default dH is left out and
        its product is not run.
        int8_head: score the per-row int8 form of the tied embedding (pg_quantize_q8) with
        step_int8, as a model evaluated after quantisation is (README leaderboard, "Mixed Quant +
        Sliding Window Eval": int8 embeddings); evaluation only, no test-time training."""
        if ttt_lr and embed_master is None:
            raise ValueError("score-first TTT needs float32 master weights of the embedding (embed_master)")
        if ttt_lr and int8_head:
            raise ValueError("test-time training updates a bf16 embedding; the int8 head is evaluation only")
        self.int8_head = bool(int8_head)
        self.tokens, self.byte_len, self.V, self.D = tokens, byte_len, int(V), int(D)
        self.window, self.stride, self.per_batch = int(window), int(stride), int(windows_per_batch)
        self.softcap, self.ttt_lr, self.embed_master = float(softcap), float(ttt_lr), embed_master
        self.keep_dhidden = bool(keep_dhidden)
        self.n_windows = abi.pg_window_count(tokens.numel(), self.window, self.stride)
        dev = tokens.device
        rows = self.per_batch * self.window
        self.target = torch.empty(rows, dtype=torch.int32, device=dev)
        self.mask = torch.empty(rows, dtype=torch.uint8, device=dev)
        self.nats = torch.empty(rows, dtype=torch.float32, device=dev)
        self.lse = torch.empty(rows, dtype=torch.float32, device=dev)
        # running sums (nats, bytes, predictions) and their bits per byte: NaN (0 / 0) until a batch
        # with predictions has been scored, as for a stream too short to predict anything
        self.out = torch.tensor([0.0, 0.0, 0.0, float("nan")], dtype=torch.float64, device=dev)
        op = abi.PG_OP_FWD_BWD if self.ttt_lr else (abi.PG_OP_FWD_Q8 if self.int8_head else abi.PG_OP_FWD)
        self.ws = torch.empty(max(abi.workspace_bytes(op, rows, self.D, self.V), 256), dtype=torch.uint8, device=dev)
        self.ws_bpb = torch.empty(max(abi.workspace_bytes(abi.PG_OP_BPB, rows, 1, self.V), 256), dtype=torch.uint8,
                                  device=dev)
        self.dH = None
        if self.ttt_lr:
            if self.keep_dhidden:
                self.dH = torch.empty((rows, self.D), dtype=torch.float32, device=dev)
            self.dE = torch.empty((self.V, self.D), dtype=torch.float32, device=dev)

    def batches(self) -> Iterator[Tuple[int, int]]:
        """(first window, number of windows) of each batch, in order."""
        for w0 in range(0, self.n_windows, self.per_batch):
            yield w0, min(self.per_batch, self.n_windows - w0)

    def scored(self, first_window: int, n_windows: int) -> int:
        return abi.pg_window_scored(self.tokens.numel(), self.window, self.stride, first_window, n_windows)

    def step(self, hidden: torch.Tensor, embed: torch.Tensor, first_window: int, n_windows: int) -> int:
        """Score one batch. hidden: [n_windows * window, D] bf16, row (b, r) the hidden state of
        input position (first_window + b) stride + r in its window (only scored rows are read).
        embed: the bf16 tied embedding [V, D], updated in place by the SGD step when ttt_lr > 0.
        Returns the number of predictions the batch scored."""
        rows = n_windows * self.window
        tgt, msk, nats, lse = self.target[:rows], self.mask[:rows], self.nats[:rows], self.lse[:rows]
        abi.pg_window_rows(self.tokens, self.window, self.stride, first_window, n_windows, tgt, msk)
        n = self.scored(first_window, n_windows)
        if self.ttt_lr and n > 0:
            # the batch's scores and the gradients of its mean loss come from the same embedding;
            # the update reaches only later batches
            dH = self.dH[:rows] if self.dH is not None else None
            abi.pg_lmhead_ce_fwd_bwd(hidden, embed, tgt, msk, self.softcap, 1.0 / n, nats, lse, dH, self.dE, self.ws)
            abi.pg_bpb_accumulate(nats, tgt, msk, self.byte_len, None, self.V, self.out, self.ws_bpb)
            abi.pg_sgd_step_bf16(self.embed_master, self.dE, self.ttt_lr, embed)
        else:
            abi.pg_lmhead_ce_fwd(hidden, embed, tgt, msk, self.softcap, nats, lse, self.ws)
            abi.pg_bpb_accumulate(nats, tgt, msk, self.byte_len, None, self.V, self.out, self.ws_bpb)
        return n

    def step_int8(self, hidden: torch.Tensor, embed_q8: torch.Tensor, embed_scale: torch.Tensor,
                  first_window: int, n_windows: int) -> int:
        """Score one batch on the int8 head (embed_q8 [V, D] int8, embed_scale [V] float32, from
        pg_quantize_q8); hidden as for step. Returns the number of predictions the batch scored."""
        if not self.int8_head:
            raise ValueError("step_int8 needs a driver built with int8_head=True (its workspace)")
        rows = n_windows * self.window
        tgt, msk, nats, lse = self.target[:rows], self.mask[:rows], self.nats[:rows], self.lse[:rows]
        abi.pg_window_rows(self.tokens, self.window, self.stride, first_window, n_windows, tgt, msk)
        n = self.scored(first_window, n_windows)
        abi.pg_lmhead_ce_fwd_q8(hidden, embed_q8, embed_scale, tgt, msk, self.softcap, nats, lse, self.ws)
        abi.pg_bpb_accumulate(nats, tgt, msk, self.byte_len, None, self.V, self.out, self.ws_bpb)
        return n

    def result(self):
        """(sum of nats, sum of bytes, predictions scored, bits per byte) over the batches so far."""
        return self.out.cpu().tolist()
