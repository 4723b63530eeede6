"""CPU oracle for the IndexCache / DSA hot path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never
calls it and shares no code with it.

Everything here is the plain definition, evaluated in float64 on values that
were decoded exactly from the stored bytes: one query at a time, no tiling,
no radix tricks.  Sources, by page title and section:

  [Abstract]  "IndexCache: Accelerating Sparse Attention via Cross-Layer Index
              Reuse", arXiv abstract (fugumt.com listing): a lightning indexer
              picks the top-k tokens per query so core attention costs O(Lk);
              F layers run their indexer, S layers reuse the nearest F layer's
              top-k indices.
  [Skill]     "Indexcache Sparse Attention Acceleration" (skillmd.com), Core
              Concept; Step 1 (indices shaped (batch, seq_len, k)); Step 3
              (IndexCacheManager: F computes and caches, S reuses, an S layer
              with nothing cached is an error); Practical Guidance, Common
              Pitfalls (clear the cache between sequences).
  [Gist]      gist.science technical summary, "Methodologie" (binary pattern c,
              nearest preceding F layer) and "Probleemstelling" (the indexer
              scores all preceding tokens at every layer).
  [Blog]      "When the Optimizer Becomes the Bottleneck: A Close Look at
              IndexCache" (kualia.ai), Introduction (the indexer scores all
              preceding tokens; core attention over k tokens) and "The
              Redundancy That Was Sitting There" (one conditional branch; the
              cache is one index tensor overwritten at each F layer).
  [Note]      "Cross-Layer Index Reuse" knowledge note, How It Works (an F
              layer scores the visible positions and stores the top-k set).

The pages never write out the indexer formula; the score used is the DSA
lightning indexer's head-weighted ReLU dot product,
    I[t, s] = sum_j w[t, j] * max(0, q_I[t, j, :] . k_I[s, :]),
over H_I indexer heads that share one key vector per token.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * causal visibility is inclusive: query at absolute position p sees keys
    0..p;
  * ties in the top-k go to the lower key index; the row is emitted in
    ascending key order and padded with -1 when fewer than k keys are
    visible;
  * the top-k decision is taken on the score rounded to float32, the
    precision the GPU kernel decides in (the pages fix none);
  * sparse attention is softmax(q . K / sqrt(d)) V over the selected rows,
    one shared KV head, K and V stored as one [K | V] row per token;
  * decode appends the new token first, so its query sees itself;
  * the distillation loss of an F layer is KL(target || softmax of its
    indexer scores) per query, in nats, taken over the query's selected
    entries (the dense loss is the case where every visible key is
    selected); the target averages the attention distributions of every
    served layer (the F layer and its S layers) and head with equal weight;
  * dynamic refresh: an S layer that keeps its indexer probes every
    stride-th query (ending at the last), measures the pooled recall of its
    own top-k within the cached rows, sum |cached & own| / sum |own|, and
    re-indexes every query when that recall is below tau.

Parity of every function here is pinned by tests that do not reuse this code
(hand-worked examples, closed forms, brute force, library special cases);
the pages print no worked example, so no value here is pinned by the pages
themselves.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# Storage decoding (published format definitions)
# ---------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64.  bf16 is the upper half of an IEEE binary32."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": no infinities) codes -> float64.

    Layout s.eeee.mmm, exponent bias 7.  e == 0 is subnormal: m/8 * 2^-6.
    Otherwise (1 + m/8) * 2^(e-7).  The two codes with e == 15 and m == 7
    (0x7F, 0xFF) are NaN; every other code with e == 15 is a finite number
    (the largest, 0x7E, is 448).
    """
    c = codes.astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val).astype(np.float64)


# ---------------------------------------------------------------------------
# O1: lightning-indexer scores      [Abstract; Blog, Introduction; Note, How It Works]
# ---------------------------------------------------------------------------

def indexer_scores_row(q_I_t: np.ndarray, w_t: np.ndarray, k_I: np.ndarray, p: int) -> np.ndarray:
    """Scores of one query (absolute position p) against its visible keys 0..p.

    q_I_t [H_I, d_I], w_t [H_I], k_I [>= p+1, d_I], all float64.
    Returns I[s] for s = 0..p (length p+1), float64:
        I[s] = sum_j w_t[j] * max(0, q_I_t[j] . k_I[s]).
    """
    keys = k_I[: p + 1]                      # visible keys only: future keys are excluded
    y = q_I_t @ keys.T                       # [H_I, p+1] per-head dot products
    return w_t @ np.maximum(y, 0.0)          # ReLU, then the head-weighted sum


def indexer_scores(q_I: np.ndarray, w: np.ndarray, k_I: np.ndarray, pos0: int = 0) -> List[np.ndarray]:
    """O1 for every query of one sequence: query t sits at absolute position pos0 + t.

    q_I [Lq, H_I, d_I], w [Lq, H_I], k_I [Lk, d_I] (float64).  Returns a list
    of Lq rows, row t of length pos0 + t + 1.
    """
    return [indexer_scores_row(q_I[t], w[t], k_I, pos0 + t) for t in range(q_I.shape[0])]


# ---------------------------------------------------------------------------
# O2 + O3: top-k selection and emission          [Abstract; Skill, Step 1]
# ---------------------------------------------------------------------------

def to_decision_precision(row: np.ndarray) -> np.ndarray:
    """Round scores to float32, the precision the selection is decided in."""
    return np.asarray(row, dtype=np.float64).astype(np.float32)


def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """The k highest of one row of visible scores; ties go to the lower index.

    Brute force: a full stable sort of the keys by descending score (a stable
    sort keeps equal scores in index order, so the lower index comes first;
    -0.0 and +0.0 compare equal).  The chosen positions are returned in
    ascending order, padded with -1 up to k entries.
    """
    n = scores.shape[0]
    order = np.argsort(-scores, kind="stable")
    chosen = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: chosen.shape[0]] = chosen
    return out


def indexer_topk(q_I: np.ndarray, w: np.ndarray, k_I: np.ndarray, k: int, pos0: int = 0) -> np.ndarray:
    """O1 -> O2 -> O3 for one sequence: idx [Lq, k] int32."""
    rows = indexer_scores(q_I, w, k_I, pos0)
    return np.stack([topk_row(to_decision_precision(r), k) for r in rows]).astype(np.int32)


# ---------------------------------------------------------------------------
# O4: sparse attention over the selected rows     [Abstract; Blog, Introduction]
# ---------------------------------------------------------------------------

def sparse_attn_row(q_t: np.ndarray, kv: np.ndarray, idx_t: np.ndarray, scale: float) -> np.ndarray:
    """One query: q_t [H, d], kv [Lk, 2, d] (K = kv[:,0], V = kv[:,1]), idx_t [k] (-1 = unused).

    For every head h: softmax over the selected keys of scale * q_t[h] . K[s],
    weights applied to V[s].  Returns [H, d] float64.
    """
    sel = idx_t[idx_t >= 0]
    K = kv[sel, 0, :]                        # [m, d]
    V = kv[sel, 1, :]                        # [m, d]
    logits = scale * (q_t @ K.T)             # [H, m]
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V


def sparse_attn(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, scale: float = None) -> np.ndarray:
    """O4 for one sequence: q [Lq, H, d], kv [Lk, 2, d], idx [Lq, k] -> out [Lq, H, d] float64."""
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return np.stack([sparse_attn_row(q[t], kv, idx[t], scale) for t in range(q.shape[0])])


# ---------------------------------------------------------------------------
# O5: the F/S stack with its index cache   [Skill, Step 3; Gist, Methodologie; Blog]
# ---------------------------------------------------------------------------

class NoCachedIndices(ValueError):
    """An S layer came before any F layer: there are no cached indices to reuse."""


def is_full(c: str) -> bool:
    """Pattern character -> True for an F layer ('F' or '1'), False for S ('S' or '0')."""
    if c in "F1":
        return True
    if c in "S0":
        return False
    raise ValueError(f"bad pattern character {c!r}")


def run_stack(pattern: str, layers: Sequence[Dict[str, np.ndarray]], k: int, pos0: int = 0):
    """Prefill through a layer stack for one sequence.

    layers[l] holds float64 arrays: q [Lq,H,d], kv [Lk,2,d] and, on F
    layers, q_I [Lq,H_I,d_I], w [Lq,H_I], k_I [Lk,d_I].

    The cache starts empty on every call.  An F layer runs the indexer and
    top-k and overwrites the cache; an S layer reuses the cache unchanged,
    or raises NoCachedIndices when nothing has been cached yet.  Every layer
    then runs sparse attention with the cached indices.

    Returns (outs, idx_per_layer, indexer_calls).
    """
    if len(pattern) != len(layers):
        raise ValueError("pattern length must equal the number of layers")
    cache = None
    calls = 0
    outs, used = [], []
    for c, lay in zip(pattern, layers):
        if is_full(c):
            cache = indexer_topk(lay["q_I"], lay["w"], lay["k_I"], k, pos0)
            calls += 1
        elif cache is None:
            raise NoCachedIndices("no cached indices: an S layer came before any F layer")
        outs.append(sparse_attn(lay["q"], lay["kv"], cache))
        used.append(cache)
    return outs, used, calls


# ---------------------------------------------------------------------------
# O6: one decode step over a batch of sequences
# ---------------------------------------------------------------------------

def decode_step(pattern: str, layers: Sequence[Dict[str, np.ndarray]], seq_len: Sequence[int], k: int):
    """One decode step for a batch.

    layers[l]: q [B,H,d], kv [B,cap,2,d]; F layers also q_I [B,H_I,d_I],
    w [B,H_I], k_I [B,cap,d_I].  The new token of sequence b is already
    appended at row seq_len[b]-1 of k_I and kv; its query sits at that
    position and sees keys 0..seq_len[b]-1.  Returns (outs [layer][B,H,d],
    idx [layer][B,k], indexer_calls).
    """
    B = len(seq_len)
    outs = [np.zeros(l["q"].shape) for l in layers]
    idxs = [np.zeros((B, k), dtype=np.int32) for _ in layers]
    calls = 0
    for b in range(B):
        p = int(seq_len[b]) - 1
        per_seq = []
        for lay in layers:
            one = {"q": lay["q"][b][None], "kv": lay["kv"][b]}
            if "q_I" in lay:
                one.update(q_I=lay["q_I"][b][None], w=lay["w"][b][None], k_I=lay["k_I"][b])
            per_seq.append(one)
        o, used, calls = run_stack(pattern, per_seq, k, pos0=p)
        for l in range(len(layers)):
            outs[l][b] = o[l][0]
            idxs[l][b] = used[l][0]
    return outs, idxs, calls


# ---------------------------------------------------------------------------
# Cross-layer overlap diagnostic            [Skill, Step 1]
# ---------------------------------------------------------------------------

def jaccard_rows(idx_a: np.ndarray, idx_b: np.ndarray) -> np.ndarray:
    """Per-row Jaccard similarity |A & B| / (|A | B| + 1e-8) of two index tensors [..., k] (-1 ignored)."""
    a = idx_a.reshape(-1, idx_a.shape[-1])
    b = idx_b.reshape(-1, idx_b.shape[-1])
    out = np.zeros(a.shape[0])
    for r in range(a.shape[0]):
        sa = set(int(x) for x in a[r] if x >= 0)
        sb = set(int(x) for x in b[r] if x >= 0)
        out[r] = len(sa & sb) / (len(sa | sb) + 1e-8)
    return out.reshape(idx_a.shape[:-1])


# ---------------------------------------------------------------------------
# Multi-layer distillation loss, forward only
#   [Abstract: each retained indexer is trained against the averaged attention
#    distributions of all the layers it serves; Blog, "training-aware" variant;
#    Gist, Methodologie (an F layer predicts its own and its S layers'
#    attention, with a KL divergence to their average)]
# ---------------------------------------------------------------------------

def served_attention_row(qs_t: Sequence[np.ndarray], kvs: Sequence[np.ndarray], idx_t: np.ndarray,
                         scale: float) -> np.ndarray:
    """Target distribution of one query over its selected entries.

    qs_t: per served layer, q_t [H, d]; kvs: per served layer, kv [Lk, 2, d];
    idx_t [k] (-1 = unused).  For every served layer and head, the attention
    probabilities softmax(scale * q_t[h] . K[s]) over the selected keys; the
    target is their plain average over layers and heads.  Returns one value
    per entry idx_t >= 0, in entry order (float64, summing to 1).
    """
    sel = idx_t[idx_t >= 0]
    total = np.zeros(sel.shape[0])
    count = 0
    for q_t, kv in zip(qs_t, kvs):
        logits = scale * (q_t @ kv[sel, 0, :].T)          # [H, m]
        logits = logits - logits.max(axis=1, keepdims=True)
        a = np.exp(logits)
        a = a / a.sum(axis=1, keepdims=True)              # each head's distribution
        total += a.sum(axis=0)
        count += a.shape[0]
    return total / count


def distill_kl_row(I_t: np.ndarray, qs_t: Sequence[np.ndarray], kvs: Sequence[np.ndarray],
                   idx_t: np.ndarray, scale: float) -> float:
    """KL(target || softmax of the indexer scores) for one query, in nats.

    I_t: the F layer's indexer scores of this query over its visible keys
    (I_t[s] for key s); the indexer's distribution is the softmax of those
    scores over the selected entries.  Entries with zero target mass add 0.
    """
    sel = idx_t[idx_t >= 0]
    p = served_attention_row(qs_t, kvs, idx_t, scale)
    z = np.asarray(I_t, dtype=np.float64)[sel]
    log_r = z - z.max()
    log_r = log_r - math.log(np.exp(log_r).sum())
    nz = p > 0
    return float(np.sum(p[nz] * (np.log(p[nz]) - log_r[nz])))


def distill_kl(q_I: np.ndarray, w: np.ndarray, k_I: np.ndarray, idx: np.ndarray,
               qs: Sequence[np.ndarray], kvs: Sequence[np.ndarray], pos0: int = 0, scale: float = None,
               rows: Sequence[int] = None) -> np.ndarray:
    """Per-query loss of one F layer and the layers it serves (itself first).

    q_I [Lq, H_I, d_I], w [Lq, H_I], k_I [Lk, d_I]: the F layer's indexer
    inputs; idx [Lq, k]: the entries the loss is taken over (the F layer's
    top-k; the dense loss is the case of every visible key); qs[j] [Lq, H, d]
    and kvs[j] [Lk, 2, d]: the served layers.  Query t sits at position
    pos0 + t.  Returns [len(rows)] float64 (all queries when rows is None).
    """
    d = qs[0].shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    rows = range(q_I.shape[0]) if rows is None else rows
    out = []
    for t in rows:
        I_t = indexer_scores_row(q_I[t], w[t], k_I, pos0 + t)
        out.append(distill_kl_row(I_t, [q[t] for q in qs], kvs, idx[t], scale))
    return np.array(out)


# ---------------------------------------------------------------------------
# Drift-triggered dynamic refresh
#   [Blog, Conclusion: decide at runtime whether a layer's neighbour is still a
#    good proxy and refresh only when the drift exceeds a threshold; Skill,
#    Step 1: set overlap of the top-k selections as the similarity measure]
# ---------------------------------------------------------------------------

def probe_rows(Lq: int, stride: int) -> np.ndarray:
    """Queries the drift probe looks at: every stride-th query, ending at the last one."""
    return np.arange((Lq - 1) % stride, Lq, stride)


def run_stack_dynamic(pattern: str, layers: Sequence[Dict[str, np.ndarray]], k: int, stride: int, tau: float,
                      pos0: int = 0):
    """Prefill through a stack whose S layers may refresh the index cache.

    Layers as in run_stack.  An S layer that still holds its own indexer
    inputs (q_I, w, k_I) first probes the cache: for the probe queries it
    takes its own top-k and measures the pooled recall of that top-k within
    the cached rows, sum |cached & own| / sum |own|.  When the recall is below
    tau it runs its indexer and top-k for every query and overwrites the cache
    (acting as an F layer); otherwise it reuses the cache.  S layers without
    indexer inputs always reuse it.

    Returns (outs, idx_per_layer, refreshed [n_layers] bool, recall [n_layers]
    float64, nan where no probe ran).
    """
    if len(pattern) != len(layers):
        raise ValueError("pattern length must equal the number of layers")
    cache = None
    outs, used = [], []
    refreshed = np.zeros(len(layers), dtype=bool)
    recall = np.full(len(layers), np.nan)
    for l, (c, lay) in enumerate(zip(pattern, layers)):
        if is_full(c):
            cache = indexer_topk(lay["q_I"], lay["w"], lay["k_I"], k, pos0)
        elif cache is None:
            raise NoCachedIndices("no cached indices: an S layer came before any F layer")
        elif "q_I" in lay:
            hit = own = 0
            for t in probe_rows(lay["q_I"].shape[0], stride):
                row = indexer_scores_row(lay["q_I"][t], lay["w"][t], lay["k_I"], pos0 + int(t))
                mine = set(int(x) for x in topk_row(to_decision_precision(row), k) if x >= 0)
                cached = set(int(x) for x in cache[t] if x >= 0)
                hit += len(mine & cached)
                own += len(mine)
            recall[l] = hit / own
            if hit < tau * own:
                cache = indexer_topk(lay["q_I"], lay["w"], lay["k_I"], k, pos0)
                refreshed[l] = True
        outs.append(sparse_attn(lay["q"], lay["kv"], cache))
        used.append(cache)
    return outs, used, refreshed, recall
