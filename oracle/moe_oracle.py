"""Plain CPU oracle for MoE token layout, dispatch, combine and their backward passes.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The HIP
library never calls it and shares no code with it.

It is numpy, written to be read against the pages:

* "Add an opt-in DeepEP transport for the AutoEP expert all-to-all"
  (DeepSpeed PR), sections "Why" and "Scope and safety": the input is the
  tokens before their top-k expansion with their expert ids and weights;
  every rank hosting one of a token's experts receives that token, arrivals
  are grouped by expert, and the combine forms the weighted top-k sum in
  token order again.  Each backward pass is the opposite row movement on the
  forward's handle (spreading the output gradient for the combine, summing
  receive-row gradients for the dispatch).  The page's review-fix commit
  makes dispatch hand back the received weights and both backward passes
  return the router-weight gradient.
* "[MoE] Apply router scores before W2 projection" (torchtitan), sections
  "Motivation" and "Implementation": with scores absorbed, the per-row
  scores are gathered expert-major with the same permutation as the rows,
  the input of W2 is scaled in float32 and cast back, and the combine becomes
  a plain sum.  The routed-expert buffer holds T * top_k rows.
* "Avoid collective token preparation for AutoEP DeepEP" (DeepSpeed PR),
  section "Summary": the standard preparation orders the (token, k) pairs by
  a stable argsort on the expert id.
* "perf(dllm): use the DeepEP dispatcher in the DiffusionGemma recipes"
  (Automodel PR), section "Why hybridep + activation checkpointing fails":
  the dispatch must give the same rows when activation checkpointing replays
  it with the same routing.

Where the pages leave a step open, the reading taken is stated on the
function.  Conventions for every function here:

* ``dtype`` is ``"f32"`` (arrays are ``float32``) or ``"bf16"`` (arrays are
  the raw ``uint16`` bit patterns of bfloat16).
* All floating-point arithmetic is IEEE binary32: every product and every sum
  is rounded to float32 on its own (numpy never fuses a multiply into an add).
  The pages fix the accumulation precision (float32) but not the order; the
  order used is given per function.
* bfloat16 results are rounded from float32 to nearest, ties to even.

Parity pins: every function here is pinned in ``tests/`` against something
other than itself (brute force, dense fp64 algebra, exact-arithmetic
identities, the library's own bf16 conversion, printed page values).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "bf16_to_f32",
    "f32_to_bf16",
    "to_f32",
    "from_f32",
    "recv_rows",
    "recv_capacity",
    "padded_count",
    "Layout",
    "layout",
    "dispatch",
    "combine",
    "combine_bwd",
    "dispatch_bwd",
    "canonical_dot",
    "send",
    "expand",
    "reduce_partitions",
    "combine_partitions",
    "CHUNK_BYTES",
    "LANES",
]

# Canonical reduction geometry for the router-weight gradients (see
# ``canonical_dot``): 16-byte chunks, grouped into segments of 64 chunks.
CHUNK_BYTES = 16
LANES = 64


# --------------------------------------------------------------------------
# bfloat16 <-> float32
# --------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact: bf16 is the top half of binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even.

    Drop the low 16 bits after adding 0x7FFF plus the lowest kept bit, so that
    a discarded half rounds up only when the kept part is odd.  NaNs keep sign
    and top payload bits and are made quiet (bit 6 of the bf16 set).

    The map is elementwise; it runs over slices of a bounded number of
    elements only so that the 64-bit temporaries of a large array stay small.
    """
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 22
    for i in range(0, flat.size, step):
        b = flat[i:i + step].astype(np.uint64)
        is_nan = (b & 0x7FFFFFFF) > 0x7F800000
        keep_lsb = (b >> 16) & 1
        rounded = (b + 0x7FFF + keep_lsb) >> 16
        quiet_nan = (b >> 16) | 0x40
        out[i:i + step] = np.where(is_nan, quiet_nan, rounded)
    return out.reshape(np.shape(x))


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f32(a)
    raise ValueError(dtype)


def from_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16(a)
    raise ValueError(dtype)


def _elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


# --------------------------------------------------------------------------
# Layout (per-expert / per-partition counts, offsets, stable positions)
# --------------------------------------------------------------------------

def recv_rows(T: int, K: int) -> int:
    """Receive rows that hold a pair: one per (token, k) pair.

    The torchtitan issue's "Motivation" sizes the routed-expert (W2) output
    as (T * top_k) x D, which is one row per routed pair.
    """
    return T * K


def padded_count(n, m: int):
    """Rows of an expert segment of n pairs padded to a multiple of m: the
    least multiple of m that holds n (0 for an empty expert)."""
    return (np.asarray(n, np.int64) + m - 1) // m * m


def recv_capacity(T: int, K: int, E: int, pad_multiple: int = 1) -> int:
    """Rows a receive buffer needs for any routing: T*K pairs, plus at most
    m-1 padding rows per expert (each of the E segments is padded to a
    multiple of m).  Known on the host before the layout runs."""
    return T * K + E * (pad_multiple - 1)


@dataclass
class Layout:
    T: int
    K: int
    E: int
    P: int
    num_tokens_per_expert: np.ndarray  # [E]   int32
    num_tokens_per_rank: np.ndarray    # [P]   int32, distinct tokens per partition
    is_token_in_rank: np.ndarray       # [T,P] uint8
    expert_offset: np.ndarray          # [E+1] int32
    rank_offset: np.ndarray            # [P+1] int32, first receive row of each partition
    send_offset: np.ndarray            # [P+1] int32, prefix of num_tokens_per_rank
    token_slot: np.ndarray             # [T,P] int32, slot in the partition's send list or -1
    recv_pos: np.ndarray               # [T,K] int32, receive row of pair (t,k)
    recv_token: np.ndarray             # [R]   int32, inverse map: token of a receive row
    recv_k: np.ndarray                 # [R]   int32, inverse map: k of a receive row
    part: np.ndarray                   # [T,K] int32, partition of pair (t,k)'s expert
    send_token: np.ndarray             # [N_send] int32, token of each send row
    pad_multiple: int = 1              # expert segments padded to a multiple of this

    @property
    def n_send(self) -> int:
        """Rows of the deduplicated send buffer: one per (token, partition) pair."""
        return int(self.send_offset[-1])

    @property
    def R(self) -> int:
        """Rows of a receive buffer (T*K when unpadded)."""
        return recv_capacity(self.T, self.K, self.E, self.pad_multiple)

    def padding_rows(self) -> np.ndarray:
        """Receive rows inside an expert's padded segment that hold no pair."""
        n = self.num_tokens_per_expert.astype(np.int64)
        lo = self.expert_offset[:-1].astype(np.int64) + n
        hi = self.expert_offset[1:].astype(np.int64)
        return np.concatenate([np.arange(a, b) for a, b in zip(lo, hi)] + [np.zeros(0, np.int64)])


def layout(topk_idx: np.ndarray, E: int, P: int, pad_multiple: int = 1) -> Layout:
    """Dispatch layout of one routing decision.

    * Expert ``e`` lives on virtual partition ``e // (E/P)``: experts are split
      into P contiguous blocks (E must be a multiple of P).  The pages only
      say experts are spread over EP ranks; contiguous blocks is the reading.
    * ``num_tokens_per_expert[e]`` counts (t,k) pairs routed to e.
    * ``is_token_in_rank[t,r]`` is 1 when any of t's experts lives on r; a
      token is sent once per such partition, not once per expert (the DeepEP
      transport PR's "Why" section credits this deduplication with about
      1.29x on its own).  ``num_tokens_per_rank[r]`` sums it over t.
    * Offsets are exclusive prefix sums.  ``rank_offset[r]`` is the first
      receive row of partition r, i.e. ``expert_offset[r * E/P]``.
    * ``token_slot[t,r]`` is t's index in partition r's send list, which holds
      the tokens with ``is_token_in_rank[t,r]`` in increasing t; -1 if absent.
      The send row in a buffer of all partitions' lists is
      ``send_offset[r] + token_slot[t,r]``.
    * ``send_token[s]`` is the token of send row s (the inverse of
      ``send_offset[r] + token_slot[t,r]``).
    * ``recv_pos`` orders the pairs by expert, and within one expert by t then
      k: a stable sort of the flattened (t,k) stream by expert id.  This is
      the order the standard path's stable argsort gives, and it is a
      function of the routing alone, so a replay with the same routing
      reproduces every position.
    * ``pad_multiple`` m (a handle constant; the DiffusionGemma dispatcher
      page lists it as set once at construction): each expert's segment is
      padded to ``padded_count(n_e, m)`` rows, so every ``expert_offset`` is
      a multiple of m, as grouped-GEMM tiles want.  Pairs keep their order
      and fill the front of their segment; the rest are padding rows, with
      ``recv_token = recv_k = -1``.  m = 1 is the unpadded layout.
    """
    idx = np.asarray(topk_idx)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [T,K]")
    T, K = idx.shape
    if K < 1:
        raise ValueError("K must be >= 1")
    if E < 1 or P < 1 or E % P != 0:
        raise ValueError("E must be a positive multiple of P")
    if T and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("expert id out of range")
    if pad_multiple < 1:
        raise ValueError("pad_multiple must be >= 1")
    epr = E // P
    flat = idx.reshape(-1).astype(np.int64)
    R = recv_rows(T, K)

    num_tokens_per_expert = np.bincount(flat, minlength=E).astype(np.int32)

    part = idx.astype(np.int64) // epr                       # [T,K]
    is_token_in_rank = np.zeros((T, P), dtype=np.uint8)
    is_token_in_rank[np.repeat(np.arange(T), K), part.reshape(-1)] = 1
    num_tokens_per_rank = is_token_in_rank.sum(axis=0, dtype=np.int64).astype(np.int32)

    expert_offset = np.zeros(E + 1, dtype=np.int64)
    expert_offset[1:] = np.cumsum(padded_count(num_tokens_per_expert, pad_multiple))
    rank_offset = expert_offset[np.arange(P + 1) * epr]
    send_offset = np.zeros(P + 1, dtype=np.int64)
    send_offset[1:] = np.cumsum(num_tokens_per_rank)

    running = np.cumsum(is_token_in_rank, axis=0, dtype=np.int64) - 1
    token_slot = np.where(is_token_in_rank == 1, running, -1)
    # send rows partition by partition, tokens ascending inside each
    send_token = np.concatenate([np.nonzero(is_token_in_rank[:, r])[0] for r in range(P)]
                                + [np.zeros(0, np.int64)])

    order = np.argsort(flat, kind="stable")                  # pair ids, expert-major
    # rank of each pair among its expert's pairs, then its expert's first row
    first_pair = np.zeros(E + 1, dtype=np.int64)
    first_pair[1:] = np.cumsum(num_tokens_per_expert)
    e_sorted = flat[order]
    pos_sorted = expert_offset[e_sorted] + (np.arange(R) - first_pair[e_sorted])
    recv_pos = np.empty(R, dtype=np.int64)
    recv_pos[order] = pos_sorted
    cap = recv_capacity(T, K, E, pad_multiple)
    recv_token = np.full(cap, -1, dtype=np.int64)
    recv_k = np.full(cap, -1, dtype=np.int64)
    recv_token[pos_sorted] = order // K
    recv_k[pos_sorted] = order % K

    i32 = lambda a: np.ascontiguousarray(a, dtype=np.int32)
    return Layout(
        T=T, K=K, E=E, P=P,
        num_tokens_per_expert=num_tokens_per_expert,
        num_tokens_per_rank=num_tokens_per_rank,
        is_token_in_rank=is_token_in_rank,
        expert_offset=i32(expert_offset),
        rank_offset=i32(rank_offset),
        send_offset=i32(send_offset),
        token_slot=i32(token_slot),
        recv_pos=i32(recv_pos.reshape(T, K)),
        recv_token=i32(recv_token),
        recv_k=i32(recv_k),
        part=i32(part),
        send_token=i32(send_token),
        pad_multiple=int(pad_multiple),
    )


# --------------------------------------------------------------------------
# Row operations
# --------------------------------------------------------------------------

def dispatch(lay: Layout, x: np.ndarray, dtype: str, topk_weights=None,
             scale_rows: bool = False):
    """Forward dispatch: ``recv[recv_pos[t,k]] = x[t]``.

    Returns ``(recv[R,H], recv_scores[R] or None)``.

    * ``recv_scores[recv_pos[t,k]] = topk_weights[t,k]`` when weights are
      given: the per-row scores, gathered expert-major with the rows'
      permutation (torchtitan issue, "Implementation").
    * ``scale_rows``: the scores are absorbed before W2.  The row is scaled in
      float32 and cast back, ``recv = bf16(f32(x[t]) * w[t,k])``.  On one GPU,
      with no expert GEMM, the dispatch output is where that scaling lands.
    * Padded layouts: the padding rows of every expert segment are zero rows
      with a zero score (the zero-sentinel scores of the DiffusionGemma
      dispatcher page's padded permute).  Rows past ``expert_offset[E]`` are
      left unwritten.
    """
    x = np.asarray(x)
    T, K = lay.T, lay.K
    H = x.shape[1]
    recv = np.empty((lay.R, H), dtype=x.dtype)
    recv[lay.padding_rows()] = 0
    recv_scores = None
    if scale_rows:
        if topk_weights is None:
            raise ValueError("scale_rows needs topk_weights")
        xf = to_f32(x, dtype)
        for k in range(K):
            prod = topk_weights[:, k:k + 1].astype(np.float32) * xf   # one rounding
            recv[lay.recv_pos[:, k]] = from_f32(prod, dtype)
    else:
        for k in range(K):
            recv[lay.recv_pos[:, k]] = x
    if topk_weights is not None:
        recv_scores = np.empty(lay.R, dtype=np.float32)
        recv_scores[lay.padding_rows()] = 0.0
        recv_scores[lay.recv_pos.reshape(-1)] = np.asarray(topk_weights, np.float32).reshape(-1)
    return recv, recv_scores


def combine(lay: Layout, y: np.ndarray, dtype: str, topk_weights=None):
    """Forward combine: token rows from receive rows.

    ``out[t] = sum_k w[t,k] * y[recv_pos[t,k]]`` (weighted) or
    ``sum_k y[recv_pos[t,k]]`` (plain, scores already absorbed).

    Accumulation: float32, starting from +0.0, k = 0..K-1 in order, product
    and sum each rounded on its own.  The output is rounded once at the end.
    """
    yf = to_f32(y, dtype)
    acc = np.zeros((lay.T, yf.shape[1]), dtype=np.float32)
    for k in range(lay.K):
        rows = yf[lay.recv_pos[:, k]]
        if topk_weights is not None:
            rows = np.asarray(topk_weights, np.float32)[:, k:k + 1] * rows
        acc = acc + rows
    return from_f32(acc, dtype)


def combine_bwd(lay: Layout, grad_out: np.ndarray, dtype: str, topk_weights=None,
                y=None):
    """Backward of ``combine``: a dispatch of the output gradient.

    Returns ``(grad_y[R,H], grad_w[T,K] or None)``.

    * ``grad_y[recv_pos[t,k]] = w[t,k] * grad_out[t]`` (one float32 product,
      then rounded), or a copy of ``grad_out[t]`` in plain mode.
    * ``grad_w[t,k] = <grad_out[t], y[recv_pos[t,k]]>`` when weights and ``y``
      are given, as ``canonical_dot``.
    """
    g = np.asarray(grad_out)
    T, K = lay.T, lay.K
    grad_y = np.empty((lay.R, g.shape[1]), dtype=g.dtype)
    grad_y[lay.padding_rows()] = 0      # padding rows get no gradient
    if topk_weights is None:
        for k in range(K):
            grad_y[lay.recv_pos[:, k]] = g
    else:
        gf = to_f32(g, dtype)
        for k in range(K):
            prod = np.asarray(topk_weights, np.float32)[:, k:k + 1] * gf
            grad_y[lay.recv_pos[:, k]] = from_f32(prod, dtype)
    grad_w = None
    if topk_weights is not None and y is not None:
        rows = np.asarray(y)[lay.recv_pos.reshape(-1)]
        grad_w = canonical_dot(np.repeat(g, K, axis=0), rows, dtype).reshape(T, K)
    return grad_y, grad_w


def dispatch_bwd(lay: Layout, grad_recv: np.ndarray, dtype: str, topk_weights=None,
                 x=None):
    """Backward of ``dispatch``: a combine of the receive-row gradient.

    Returns ``(grad_x[T,H], grad_s[T,K] or None)``.

    * unscaled dispatch: ``grad_x[t] = sum_k grad_recv[recv_pos[t,k]]``;
    * scaled dispatch (scores absorbed): the scaling is differentiated straight
      through its rounding, ``grad_x[t] = sum_k w[t,k] * grad_recv[...]`` and
      ``grad_s[t,k] = <grad_recv[recv_pos[t,k]], x[t]>`` (``canonical_dot``).

    Sums as in ``combine``: float32, k order, from +0.0, no fused multiply-add.
    """
    gr = np.asarray(grad_recv)
    T, K = lay.T, lay.K
    grad_x = combine(lay, gr, dtype, topk_weights)
    grad_s = None
    if topk_weights is not None and x is not None:
        rows = gr[lay.recv_pos.reshape(-1)]
        grad_s = canonical_dot(rows, np.repeat(np.asarray(x), K, axis=0), dtype).reshape(T, K)
    return grad_x, grad_s


def canonical_dot(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """Row-wise dot products ``<a[n], b[n]>`` in a fixed float32 order.

    The pages fix float32 accumulation but not the order of a length-H sum,
    and at these magnitudes (|dot| ~ sqrt(H)) a different order moves the
    result by whole float32 ulps.  The order is therefore part of the
    contract (segment-major, so that one row can be spread over several
    64-lane wavefronts that each own one segment):

    1. Cut each row into 16-byte chunks of V elements (V = 4 for f32, 8 for
       bf16), NV = H / V chunks, and the chunks into segments of 64
       consecutive chunks (the last segment is padded with +0.0 chunks).
    2. Each chunk's partial starts at +0.0 and adds its V float32 products
       a*b in element order (product rounded, then sum rounded).
    3. Each segment folds its 64 chunk partials pairwise: for s = 32, 16, 8,
       4, 2, 1 partial l becomes L[l] + L[l xor s]; the segment's value is
       partial 0.
    4. The result starts at +0.0 and adds the segment values in segment
       order.
    """
    a = np.asarray(a)
    b = np.asarray(b)
    n, H = a.shape
    V = CHUNK_BYTES // _elem_bytes(dtype)
    if H % V:
        raise ValueError("H must be a whole number of 16-byte chunks")
    NV = H // V
    NS = -(-NV // LANES)                                   # segments
    prod = (to_f32(a, dtype) * to_f32(b, dtype)).reshape(n, NV, V)   # float32 products
    c = np.zeros((n, NS * LANES), dtype=np.float32)        # chunk partials, padded
    for i in range(V):
        c[:, :NV] = c[:, :NV] + prod[:, :, i]
    c = c.reshape(n, NS, LANES)
    lane = np.arange(LANES)
    for s in (32, 16, 8, 4, 2, 1):
        c = c + c[:, :, lane ^ s]
    seg = c[:, :, 0]
    out = np.zeros(n, dtype=np.float32)
    for k in range(NS):
        out = out + seg[:, k]
    return out


# --------------------------------------------------------------------------
# Staged exchange: a deduplicated send buffer per destination partition
# --------------------------------------------------------------------------
#
# The DeepSpeed transport PR's "Why" section: the exchange sends a token once
# per destination rank, not once per selected expert, and the receiver groups
# what arrives by expert; its combine reduces back to token order.  Staged on
# one GPU, the payload that would cross the link is a physical buffer
# S[N_send, H] with one row per (token, partition) pair, at row
# send_offset[r] + token_slot[t, r].  The combine then has two levels: each
# partition reduces its own experts' rows of a token (what the receiver sends
# back), and the source adds the partitions' partial rows.  Readings, since
# the pages give the order of neither sum: the partition-level sum runs over
# the token's k with an expert on that partition, in k order; its partial is
# rounded to the row type (the type a transport would send); the source adds
# the partials in ascending partition order.  Every sum is float32 from +0.0,
# product and sum rounded separately.

def _send_row(lay: Layout, t, r):
    return lay.send_offset[r] + lay.token_slot[t, r]


def send(lay: Layout, x: np.ndarray) -> np.ndarray:
    """Source side of a staged dispatch: ``S[send_offset[r] + token_slot[t,r]] = x[t]``
    for every partition r that hosts one of t's experts.  Returns ``S[N_send, H]``."""
    x = np.asarray(x)
    S = np.empty((lay.n_send, x.shape[1]), dtype=x.dtype)
    t_idx, r_idx = np.nonzero(lay.is_token_in_rank)
    S[_send_row(lay, t_idx, r_idx)] = x[t_idx]
    return S


def expand(lay: Layout, S: np.ndarray, dtype: str, topk_weights=None, scale_rows: bool = False):
    """Receiver side of a staged dispatch: each send row goes to the receive
    rows of its token's experts on that partition,
    ``recv[recv_pos[t,k]] = S[send_offset[part] + token_slot[t,part]]`` with
    ``part`` the partition of ``topk_idx[t,k]``; scaled as ``dispatch`` when
    ``scale_rows``.  Returns ``(recv[R,H], recv_scores[R] or None)``."""
    S = np.asarray(S)
    T, K = lay.T, lay.K
    recv = np.empty((lay.R, S.shape[1]), dtype=S.dtype)
    recv[lay.padding_rows()] = 0
    rows = _send_row(lay, np.repeat(np.arange(T), K), lay.part.reshape(-1)).reshape(T, K)
    if scale_rows:
        if topk_weights is None:
            raise ValueError("scale_rows needs topk_weights")
        for k in range(K):
            prod = np.asarray(topk_weights, np.float32)[:, k:k + 1] * to_f32(S[rows[:, k]], dtype)
            recv[lay.recv_pos[:, k]] = from_f32(prod, dtype)
    else:
        for k in range(K):
            recv[lay.recv_pos[:, k]] = S[rows[:, k]]
    recv_scores = None
    if topk_weights is not None:
        recv_scores = np.empty(lay.R, dtype=np.float32)
        recv_scores[lay.padding_rows()] = 0.0
        recv_scores[lay.recv_pos.reshape(-1)] = np.asarray(topk_weights, np.float32).reshape(-1)
    return recv, recv_scores


def reduce_partitions(lay: Layout, y: np.ndarray, dtype: str, topk_weights=None) -> np.ndarray:
    """Receiver side of a two-level combine: for every (token, partition) pair
    the partial ``sum_k [w[t,k] *] y[recv_pos[t,k]]`` over the k whose expert
    is on that partition, in k order, float32 from +0.0, rounded to the row
    type.  Returns ``Q[N_send, H]`` in send-row order."""
    yf = to_f32(y, dtype)
    T, K = lay.T, lay.K
    acc = np.zeros((lay.n_send, yf.shape[1]), dtype=np.float32)
    t_all = np.arange(T)
    for k in range(K):
        rows = _send_row(lay, t_all, lay.part[:, k])      # each token's row for this k's partition
        term = yf[lay.recv_pos[:, k]]
        if topk_weights is not None:
            term = np.asarray(topk_weights, np.float32)[:, k:k + 1] * term
        # tokens are distinct within one k, so this is one add per send row
        acc[rows] = acc[rows] + term
    return from_f32(acc, dtype)


def combine_partitions(lay: Layout, Q: np.ndarray, dtype: str) -> np.ndarray:
    """Source side of a two-level combine: ``out[t] = round(sum_r f32(Q[send row
    of (t,r)]))`` over t's partitions in ascending r, float32 from +0.0."""
    Qf = to_f32(Q, dtype)
    acc = np.zeros((lay.T, Qf.shape[1]), dtype=np.float32)
    for r in range(lay.P):
        ts = np.nonzero(lay.is_token_in_rank[:, r])[0]
        acc[ts] = acc[ts] + Qf[_send_row(lay, ts, r)]
    return from_f32(acc, dtype)
