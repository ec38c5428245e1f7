"""Plain float64 CPU oracle for the tied LM head + logit softcap + cross-entropy -> bits-per-byte path.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module. The GPU library never calls it, and it shares no code with the GPU library.

What it computes, and where the pages state it:

* Tied LM head: the input embedding E[V, D] is reused as the output projection, so the logits are
  z = H . E^T (trios issue #19, table of approaches, "Tied embeddings"; parameter-golf README
  leaderboard, "Naive Baseline" row: "TiedEmbeddings"; repo-explainer page, "The Baseline Is a Map":
  the model maps the input tokens to logits).
* Logit softcap: the pages only say the logits are "softcapped" (HYDRA Golf site, stack list,
  a fused softcapped cross-entropy kernel; README leaderboard, PR #1787 row). Reading taken: s = c * tanh(z / c)
  with c = 30; c = 0 means no cap (s = z).
* Asymmetric softcap: the pages name an "AsymLogit" head change (HYDRA Golf site, leaderboard
  table, entries #1 and #4; README leaderboard, PR #2135 and PR #1945 rows) without defining it.
  Reading taken: separate caps for positive and negative logits, s = c_pos tanh(z / c_pos) for
  z >= 0 and c_neg tanh(z / c_neg) for z < 0; every function taking a cap c accepts the pair
  (c_pos, c_neg) in its place.
* Quantised tied head: the model is quantised to fit the artifact (trios issue #19, approach table,
  "Квантование": INT4/INT8; README leaderboard, GPTQ and LQER rows); no format is given, so per-row
  symmetric int8 with float32
  scales is the reading taken, and the head computes on the bfloat16 rounding of q * scale
  (quantize_rows_q8, dequantize_rows_q8, forward_q8).
* Cross-entropy against the next token, in nats: lse(s) - s[target] (trios issue, "Контекст":
  cross-entropy loss and bits per byte; repo-explainer, baseline listing: the loss of the logits against
  the next tokens).
* Bits per byte: total -log2 p(target) over scored rows divided by the total UTF-8 bytes of those
  targets, a ratio of sums (README introduction: the score is compression in bits per byte,
  independent of the tokenizer; tproger article, "Правила и метрика": compression counted in bytes).
  A per-position byte count may replace the per-vocabulary table (README leaderboard, PR #1736 row:
  byte counts carried per position beside the tokens).
* Scored rows: a mask selects the rows that count (README leaderboard, "Sliding Window Eval" row,
  stride 64). Unscored rows get nats = 0 and lse = 0 and enter no sum.
* Sliding-window evaluation of a token stream (same row: windows advance by the stride, so that each
  scored token sees a long context): each window scores the predictions no earlier window scored
  (window_schedule); with score-first test-time training (README leaderboard, "Legal Score-First
  TTT" rows, and the row that trains in phases on validation chunks already scored) each batch of
  windows, once scored,
  gives one SGD step on the tied embedding for the batches after it (sliding_window_eval). The
  reading taken for the step: float32 master weights, w <- w - lr g with each operation rounded to
  float32, and the head reads their bfloat16 rounding.
* Backward of L = g * sum_scored nats (repo-explainer, baseline listing: the backward pass of the loss):
  dS = g (softmax(s) - onehot(target)), dZ = dS * ds/dz with ds/dz = 1 - tanh(z/c)^2,
  dH = dZ . E, dE = dZ^T . H (the LM-head part of the tied embedding's gradient).
  A scored row whose target lies outside [0, V) has NaN nats, so its loss term, and with it its
  row of dZ, is NaN: that dH row and all of dE are NaN (the reading of such a target as poison).

Every function works on float64 arrays (bf16 inputs are widened exactly before they get here).
Nothing is blocked, fused or reordered beyond the formulas above; numpy's matmul is the only
library primitive used for a step.
"""
from __future__ import annotations

import numpy as np

LN2 = float(np.log(2.0))

__all__ = ["LN2", "logits", "softcap", "softcap_derivative", "log_sum_exp", "forward", "bpb",
           "backward", "embed_grad_rows", "loss", "quantize_rows_q8", "dequantize_rows_q8", "forward_q8",
           "window_schedule", "sliding_window_eval"]


def logits(H: np.ndarray, E: np.ndarray) -> np.ndarray:
    """z[t, v] = sum_d H[t, d] * E[v, d]: the tied head, the embedding used as output projection."""
    return np.asarray(H, dtype=np.float64) @ np.asarray(E, dtype=np.float64).T


def _caps(c):
    """(cap of z >= 0, cap of z < 0). A single number caps both sides alike; a pair (c_pos, c_neg)
    is the asymmetric softcap."""
    if isinstance(c, (tuple, list)):
        return float(c[0]), float(c[1])
    return float(c), float(c)


def _cap_side(z: np.ndarray, c: float) -> np.ndarray:
    if c > 0:
        return c * np.tanh(z / c)
    return np.array(z, dtype=np.float64, copy=True)


def _cap_side_derivative(z: np.ndarray, c: float) -> np.ndarray:
    if c > 0:
        return 1.0 - np.tanh(z / c) ** 2
    return np.ones_like(z, dtype=np.float64)


def softcap(z: np.ndarray, c) -> np.ndarray:
    """s = c * tanh(z / c) for c > 0; s = z when c == 0 (no cap).

    With c = (c_pos, c_neg): s = c_pos tanh(z / c_pos) for z >= 0 and c_neg tanh(z / c_neg) for
    z < 0 (each side uncapped when its cap is 0).
    """
    cp, cn = _caps(c)
    z = np.asarray(z, dtype=np.float64)
    if cp == cn:
        return _cap_side(z, cp)
    return np.where(z >= 0, _cap_side(z, cp), _cap_side(z, cn))


def softcap_derivative(z: np.ndarray, c) -> np.ndarray:
    """ds/dz = 1 - tanh(z / c)^2 for c > 0, else 1; per side for c = (c_pos, c_neg)."""
    cp, cn = _caps(c)
    z = np.asarray(z, dtype=np.float64)
    if cp == cn:
        return _cap_side_derivative(z, cp)
    return np.where(z >= 0, _cap_side_derivative(z, cp), _cap_side_derivative(z, cn))


def log_sum_exp(s: np.ndarray) -> np.ndarray:
    """lse[t] = log sum_v exp(s[t, v]), shifted by the row maximum to stay finite."""
    m = np.max(s, axis=1)
    return m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))


def _scored(T: int, mask) -> np.ndarray:
    if mask is None:
        return np.ones(T, dtype=bool)
    return np.asarray(mask).astype(bool)


def forward(H, E, target, c: float, mask=None):
    """Per-row (nats, lse) of the softcapped cross-entropy.

    nats[t] = lse[t] - s[t, target[t]] on scored rows; 0 (and lse 0) on unscored rows.
    A scored row whose target lies outside [0, V) gets nats = NaN.
    """
    H = np.asarray(H, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    target = np.asarray(target, dtype=np.int64)
    T, V = H.shape[0], E.shape[0]
    s = softcap(logits(H, E), c)
    lse = log_sum_exp(s)
    valid = (target >= 0) & (target < V)
    s_target = np.full(T, np.nan)
    rows = np.nonzero(valid)[0]
    s_target[rows] = s[rows, target[rows]]
    nats = lse - s_target
    scored = _scored(T, mask)
    nats = np.where(scored, nats, 0.0)
    lse = np.where(scored, lse, 0.0)
    return nats, lse


def bpb(nats, target, byte_len, mask=None, byte_per_pos=None, V=None):
    """(sum_nats, sum_bytes, n_scored, bits_per_byte) over the scored rows.

    bytes[t] = byte_len[target[t]], or byte_per_pos[t] when given. A scored row whose target is
    outside [0, V) adds no bytes (its nats are NaN already). bits_per_byte = sum_nats /
    (ln 2 * sum_bytes), with IEEE results for empty sums (0/0 = NaN, x/0 = inf).
    """
    nats = np.asarray(nats, dtype=np.float64)
    target = np.asarray(target, dtype=np.int64)
    byte_len = np.asarray(byte_len, dtype=np.int64)
    V = byte_len.shape[0] if V is None else int(V)
    T = nats.shape[0]
    scored = _scored(T, mask)
    if byte_per_pos is not None:
        bytes_t = np.asarray(byte_per_pos, dtype=np.int64)
    else:
        valid = (target >= 0) & (target < V)
        bytes_t = np.where(valid, byte_len[np.clip(target, 0, V - 1)], 0)
    sum_nats = float(np.sum(nats[scored]))
    sum_bytes = int(np.sum(bytes_t[scored]))
    n_scored = int(np.count_nonzero(scored))
    with np.errstate(divide="ignore", invalid="ignore"):
        bits = np.float64(sum_nats) / (np.float64(LN2) * np.float64(sum_bytes))
    return sum_nats, sum_bytes, n_scored, float(bits)


def _bf16_round(x32: np.ndarray) -> np.ndarray:
    """float32 values -> nearest bfloat16 (ties to even), returned as float64."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def quantize_rows_q8(E):
    """Per-row symmetric int8 form of the tied embedding, (q [V, D] int8, scale [V] float32).

    The pages quantise the model to fit the artifact (trios issue #19, approach table,
    "Квантование": INT4/INT8; tproger article on int6/int5/ternary weights; README leaderboard,
    GPTQ and LQER rows) but define no format; the reading taken here, in float32 arithmetic:
    scale[v] = max_d |E[v, d]| / 127, q[v, d] = round_half_even(E[v, d] / scale[v]) clipped to
    [-127, 127], and q = 0 on a row whose scale is 0.
    """
    E32 = np.asarray(E, dtype=np.float32)
    scale = (np.max(np.abs(E32), axis=1) / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    r = np.rint(E32 / safe[:, None])
    r = np.where(scale[:, None] > 0, r, 0.0)
    return np.clip(r, -127, 127).astype(np.int8), scale


def dequantize_rows_q8(q, scale) -> np.ndarray:
    """E'[v, d] = bfloat16(float32(q[v, d]) * scale[v]), the embedding the quantised head uses."""
    prod = np.asarray(q, dtype=np.float32) * np.asarray(scale, dtype=np.float32)[:, None]
    return _bf16_round(prod)


def forward_q8(H, q, scale, target, c, mask=None):
    """Forward of the quantised tied head: :func:`forward` on the dequantised embedding."""
    return forward(H, dequantize_rows_q8(q, scale), target, c, mask)


def loss(H, E, target, c: float, g: float, mask=None) -> float:
    """L = g * sum over scored rows of nats."""
    nats, _ = forward(H, E, target, c, mask)
    return float(g * np.sum(nats))


def backward(H, E, target, c: float, g: float, mask=None):
    """(dH, dE) of L = g * sum_scored nats, from the definition.

    p = softmax(s) per row, dS = g * (p - onehot(target)), dZ = dS * ds/dz (zero on unscored
    rows), dH = dZ . E, dE = dZ^T . H. dE is only the LM-head part of the tied embedding's
    gradient; the caller adds the gradient of the input lookup.
    """
    H = np.asarray(H, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    target = np.asarray(target, dtype=np.int64)
    T, V = H.shape[0], E.shape[0]
    z = logits(H, E)
    s = softcap(z, c)
    p = np.exp(s - log_sum_exp(s)[:, None])
    valid = (target >= 0) & (target < V)
    onehot = np.zeros((T, V))
    rows = np.nonzero(valid)[0]
    onehot[rows, target[rows]] = 1.0
    dS = g * (p - onehot)
    dZ = dS * softcap_derivative(z, c)
    dZ[~valid] = np.nan                  # the row's nats are NaN: so is its gradient
    dZ[~_scored(T, mask)] = 0.0          # unscored rows enter nothing, whatever their target
    dH = dZ @ E
    dE = dZ.T @ H
    return dH, dE


def embed_grad_rows(H, E, target, c: float, g: float, lse, vocab_rows, mask=None):
    """dE[vocab_rows, :] from the same definition, given the per-row lse of the forward.

    Only the logits of the requested vocabulary entries are formed, so this works at full size;
    ``lse`` must come from :func:`forward` on the same inputs.
    """
    H = np.asarray(H, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    target = np.asarray(target, dtype=np.int64)
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    T = H.shape[0]
    z = H @ E[vocab_rows].T                                  # [T, n]
    s = softcap(z, c)
    p = np.exp(s - np.asarray(lse, dtype=np.float64)[:, None])
    onehot = (target[:, None] == vocab_rows[None, :]).astype(np.float64)
    dZ = g * (p - onehot) * softcap_derivative(z, c)
    dZ[~((target >= 0) & (target < E.shape[0]))] = np.nan   # poisoned rows, as in :func:`backward`
    dZ[~_scored(T, mask)] = 0.0
    return dZ.T @ H


def window_schedule(n_tokens: int, window: int, stride: int):
    """The scored predictions of each window of a sliding-window evaluation, as lists of input
    positions (position p predicts token p + 1; the predictions are p = 0 .. n_tokens - 2).

    Window w covers input positions w * stride .. w * stride + window - 1 and scores every prediction
    there that no earlier window has scored; windows are added until every prediction is scored.
    """
    n_pred = n_tokens - 1
    windows = []
    frontier = 0                       # predictions 0 .. frontier - 1 are scored
    w = 0
    while frontier < n_pred:
        start = w * stride
        stop = min(start + window, n_pred)
        windows.append(list(range(max(frontier, start), stop)))
        frontier = max(frontier, stop)
        w += 1
    return windows


def sliding_window_eval(tokens, byte_len, hidden_of_window, E, c, window: int, stride: int,
                        windows_per_batch: int, lr: float = 0.0):
    """Bits per byte of a token stream under the sliding-window schedule, batch by batch.

    hidden_of_window(w, n) returns the hidden states [n, D] of the n predictions window w scores, in
    position order (the model run on window w). Batches hold windows_per_batch consecutive windows.
    With lr > 0, after a batch is scored the gradient of its mean loss (backward with g = 1 / its
    scored count) gives one SGD step on the embedding: float32 master weights w <- w - lr g, each
    operation rounded to float32, and the next batch is scored with their bfloat16 rounding.
    Returns a dict with the sums, the bits per byte, and per batch the positions, the nats and, with
    lr > 0, the gradients (dH of the scored rows, dE) and the embedding the batch was scored with.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    byte_len = np.asarray(byte_len, dtype=np.int64)
    E_used = np.asarray(E, dtype=np.float64)
    master = E_used.astype(np.float32)
    sched = window_schedule(len(tokens), window, stride)
    res = {"sum_nats": 0.0, "sum_bytes": 0, "n_scored": 0, "batches": []}
    for b0 in range(0, len(sched), windows_per_batch):
        ws = range(b0, min(b0 + windows_per_batch, len(sched)))
        pos = np.array([p for w in ws for p in sched[w]], dtype=np.int64)
        H = np.vstack([np.asarray(hidden_of_window(w, len(sched[w])), dtype=np.float64) for w in ws])
        y = tokens[pos + 1]
        nats, _ = forward(H, E_used, y, c)
        sn, sb, n, _ = bpb(nats, y, byte_len)
        res["sum_nats"] += sn
        res["sum_bytes"] += sb
        res["n_scored"] += n
        batch = {"first_window": b0, "positions": pos, "nats": nats, "embed": E_used}
        if lr:
            dH, dE = backward(H, E_used, y, c, 1.0 / len(pos))
            batch["dH"], batch["dE"] = dH, dE
            master = master - np.float32(lr) * dE.astype(np.float32)
            E_used = _bf16_round(master)
        res["batches"].append(batch)
    with np.errstate(divide="ignore", invalid="ignore"):
        res["bpb"] = float(np.float64(res["sum_nats"]) / (np.float64(LN2) * np.float64(res["sum_bytes"])))
    return res
