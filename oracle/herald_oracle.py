"""CPU oracle for once-per-block sparse KV selection and block attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library never routes through it, and it shares no code with the HIP path.

Plain numpy in float64: every input is widened exactly to fp64 before use, each
step is the plain definition, matmul and a stable lexicographic sort are the only
library primitives, and nothing is blocked, fused or reordered. One sequence at a
time: arrays are per sequence, shapes are stated on every function.

Sources (titles of the pages the method is taken from):
  [HERALD-v3] "HERALD: High-Throughput Block Diffusion LLM Inference via CPU-GPU
              Cooperative KV Cache Retrieval", arXiv 2606.21633 v3, abstract.
  [HERALD-v1] HERALD abstract on the mlsift "KV cache offloading" listing.
  [HERALD-v2] "HERALD: High-Throughput Block Diffusion LLM Serving via CPU-GPU
              Cooperative KV Cache Retrieval", abstract (catalyzex author page).
  [SparDA]    hyper.ai summary of arXiv 2606.04511 (SparDA), Method section,
              target-score equation S_tgt = sum over the G heads of a KV group of
              softmax(Q_h K^T / tau); keys mean-pooled into overlapping compressed
              representations for block-level relevance.

Readings taken where the pages leave a step open (each is listed, with its
reason, in the design notes of the repository):
  * merged query = mean of the block's B queries, per query head, kept in fp64;
  * tau = sqrt(head_dim), i.e. logits scaled by 1/sqrt(d) unless a scale is given;
  * query head h belongs to KV head h // G (contiguous groups, G = Hq / Hkv);
  * the selection softmax normalises over the whole cache of the sequence;
  * the refine score of a candidate is the sum, over the B queries and the G
    heads of its group, of a softmax taken over the C candidates only;
  * top-k ties go to the lower cache index; index sets are returned ascending;
  * block attention attends to the selected keys plus the B in-block keys of the
    step, with no mask;
  * compressed keys: block m of a sequence owns tokens [m*stride, (m+1)*stride)
    (the last block may be short); its compressed key is the mean of the keys in
    the window [m*stride, m*stride + ksize) cut at the sequence end (windows
    overlap when ksize > stride); the block score is the group-summed softmax over
    the blocks; the candidates are the top-C tokens of the score each token takes
    from its block (whole blocks in score order, the boundary block from its lowest
    token up).

Every function here is pinned by ``tests/test_oracle_pins.py`` (closed forms,
invariants, special cases reduced to library routines, brute force on tiny
inputs, and a hand-worked example in ``tests/golden/``).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "default_scale",
    "kv_head_of",
    "softmax",
    "merge_queries",
    "scan_logits",
    "group_scores",
    "top_k_ascending",
    "select_merged",
    "select_query",
    "compress_keys",
    "select_compressed",
    "refine_scores",
    "refine_topk",
    "gather_kv",
    "block_attention",
    "herald_block",
]


def default_scale(head_dim: int) -> float:
    """Softmax temperature: logits are q.k / sqrt(d) ([SparDA] tau, read as sqrt(d))."""
    return 1.0 / math.sqrt(head_dim)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head used by query head h: contiguous groups of G = Hq/Hkv query heads share one KV head."""
    return h // (Hq // Hkv)


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(x - max) / sum(exp(x - max)) along ``axis``, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=axis, keepdims=True))
    return e / e.sum(axis=axis, keepdims=True)


def _row_dots(rows: np.ndarray, vec: np.ndarray) -> np.ndarray:
    """<rows[i], vec> for every row, as an elementwise product summed along d.

    Every row goes through the same summation, so identical rows give bitwise
    identical results; exact ties between identical keys stay exact.
    """
    return (rows * vec[None, :]).sum(axis=1)


def merge_queries(q_block: np.ndarray) -> np.ndarray:
    """One query per query head merged from the block's B queries ([HERALD-v3]).

    q_block: [B][Hq][d]. Returns [Hq][d], the mean over the B queries.
    """
    return np.asarray(q_block, dtype=np.float64).mean(axis=0)


def scan_logits(q_merged: np.ndarray, k_cache: np.ndarray, scale: float) -> np.ndarray:
    """Merged-query logits over the full cache of one sequence ([HERALD-v3] full-cache search).

    q_merged: [Hq][d]; k_cache: [L][Hkv][d]. Returns [Hq][L] with
    logits[h][j] = scale * <q_merged[h], k_cache[j][h // G]>.
    """
    q = np.asarray(q_merged, dtype=np.float64)
    k = np.asarray(k_cache, dtype=np.float64)
    Hq, L, Hkv = q.shape[0], k.shape[0], k.shape[1]
    out = np.empty((Hq, L), dtype=np.float64)
    for h in range(Hq):
        out[h] = scale * _row_dots(k[:, kv_head_of(h, Hq, Hkv), :], q[h])
    return out


def group_scores(logits: np.ndarray, Hkv: int) -> np.ndarray:
    """Per-KV-head selection score ([SparDA] S_tgt form).

    logits: [Hq][L]. Each query head's logits are turned into a softmax over all L
    keys of the sequence; a KV head's score is the sum of the softmaxes of its G
    query heads. Returns [Hkv][L]; each row sums to G.
    """
    Hq, L = logits.shape
    p = softmax(logits, axis=1)
    S = np.zeros((Hkv, L), dtype=np.float64)
    for h in range(Hq):
        S[kv_head_of(h, Hq, Hkv)] += p[h]
    return S


def top_k_ascending(score: np.ndarray, k: int, tiebreak: np.ndarray | None = None) -> np.ndarray:
    """Positions of the k largest scores, ties broken towards the lower ``tiebreak`` value.

    ``tiebreak`` defaults to the position itself. The order used is (score
    descending, tiebreak ascending); the first k positions of that order are
    returned sorted ascending.
    """
    score = np.asarray(score, dtype=np.float64)
    n = score.shape[0]
    if not 1 <= k <= n:
        raise ValueError(f"top-k needs 1 <= k <= n, got k={k}, n={n}")
    tb = np.arange(n) if tiebreak is None else np.asarray(tiebreak)
    order = np.lexsort((tb, -score))
    return np.sort(order[:k])


def select_merged(q_merge: np.ndarray, k_cache: np.ndarray, C: int, scale: float):
    """Stage one of the two-stage selection ([HERALD-v3]) for one sequence.

    q_merge: [B][Hq][d] (the queries merged into one per head); k_cache: [L][Hkv][d].
    Returns (cand [Hkv][C] int64 ascending sequence-local indices, S [Hkv][L] scores).
    """
    Hkv = k_cache.shape[1]
    S = group_scores(scan_logits(merge_queries(q_merge), k_cache, scale), Hkv)
    cand = np.stack([top_k_ascending(S[g], C) for g in range(Hkv)])
    return cand, S


def select_query(q_sel: np.ndarray, k_cache: np.ndarray, C: int, scale: float):
    """Stage one searched with one given query per head ([HERALD-v1]: a single [MASK]
    query cuts the selection cost) instead of the block mean.

    q_sel: [Hq][d]; k_cache: [L][Hkv][d]. The scan, scores and top-C are those of
    select_merged with q_sel as the merged query. Returns (cand [Hkv][C], S [Hkv][L]).
    """
    Hkv = k_cache.shape[1]
    S = group_scores(scan_logits(np.asarray(q_sel, dtype=np.float64), k_cache, scale), Hkv)
    cand = np.stack([top_k_ascending(S[g], C) for g in range(Hkv)])
    return cand, S


def compress_keys(k_cache: np.ndarray, ksize: int, stride: int) -> np.ndarray:
    """Mean-pooled, overlapping compressed keys ([SparDA] Method: keys mean-pooled into
    overlapping compressed representations), one per block of `stride` tokens.

    k_cache: [L][Hkv][d]. Returns [ceil(L / stride)][Hkv][d]: row m is the mean of
    k_cache[j] over j in [m*stride, min(m*stride + ksize, L)).
    """
    k = np.asarray(k_cache, dtype=np.float64)
    L = k.shape[0]
    M = -(-L // stride)
    out = np.empty((M,) + k.shape[1:], dtype=np.float64)
    for m in range(M):
        a = m * stride
        out[m] = k[a:min(a + ksize, L)].mean(axis=0)
    return out


def select_compressed(q_merge: np.ndarray, k_cache: np.ndarray, C: int, scale: float, ksize: int, stride: int):
    """Block-granular stage one over compressed keys for one sequence.

    q_merge: [B][Hq][d]; k_cache: [L][Hkv][d]. Block scores S_blk [Hkv][M] are the
    group-summed softmax of the merged query over the M compressed keys; token j takes
    the score of its block j // stride; the candidates are the top-C tokens of that
    score, ties to the lower token. Returns (cand [Hkv][C], S_tok [Hkv][L], S_blk [Hkv][M]).
    """
    L, Hkv = k_cache.shape[0], k_cache.shape[1]
    kc = compress_keys(k_cache, ksize, stride)
    S_blk = group_scores(scan_logits(merge_queries(q_merge), kc, scale), Hkv)
    S_tok = S_blk[:, np.arange(L) // stride]
    cand = np.stack([top_k_ascending(S_tok[g], C) for g in range(Hkv)])
    return cand, S_tok, S_blk


def refine_scores(q_refine: np.ndarray, k_cache: np.ndarray, cand: np.ndarray, scale: float) -> np.ndarray:
    """Refine score of every candidate with the block's real queries ([HERALD-v3] GPU refine).

    q_refine: [B][Hq][d]; k_cache: [L][Hkv][d]; cand: [Hkv][C].
    R[g][c] = sum over b and over the query heads h of group g of
    softmax_c(scale * <q_refine[b][h], k_cache[cand[g][c]][g]>), the softmax taken
    over the C candidates of group g. Returns [Hkv][C]; each row sums to B*G.
    """
    q = np.asarray(q_refine, dtype=np.float64)
    k = np.asarray(k_cache, dtype=np.float64)
    B, Hq, _ = q.shape
    Hkv, C = cand.shape
    R = np.zeros((Hkv, C), dtype=np.float64)
    for g in range(Hkv):
        keys = k[cand[g], g, :]                       # [C][d]
        for h in range(Hq):
            if kv_head_of(h, Hq, Hkv) != g:
                continue
            r = np.stack([scale * _row_dots(keys, q[b, h, :]) for b in range(B)])  # [B][C]
            R[g] += softmax(r, axis=1).sum(axis=0)
    return R


def refine_topk(q_refine: np.ndarray, k_cache: np.ndarray, cand: np.ndarray, topk: int, scale: float):
    """Stage two: the final top-K subset of the candidates ([HERALD-v3], K=1024 there).

    Ties go to the lower cache index. Returns (sel [Hkv][topk] ascending
    sequence-local cache indices, R [Hkv][C]).
    """
    R = refine_scores(q_refine, k_cache, cand, scale)
    sel = np.stack([cand[g][top_k_ascending(R[g], topk, tiebreak=cand[g])] for g in range(cand.shape[0])])
    return np.sort(sel, axis=1), R


def gather_kv(k_cache: np.ndarray, v_cache: np.ndarray, sel: np.ndarray):
    """Fetch the selected subset once per block ([HERALD-v1]: only a small critical subset).

    Returns (k_sel, v_sel), each [Hkv][topk][d], row i of KV head g being cache row sel[g][i].
    """
    Hkv = sel.shape[0]
    k_sel = np.stack([np.asarray(k_cache)[sel[g], g, :] for g in range(Hkv)])
    v_sel = np.stack([np.asarray(v_cache)[sel[g], g, :] for g in range(Hkv)])
    return k_sel, v_sel


def block_attention(q: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray,
                    k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """One denoising step of B-query attention over the selected subset plus the in-block keys.

    q: [B][Hq][d]; k_blk, v_blk: [B][Hkv][d]; k_sel, v_sel: [Hkv][topk][d].
    For every b and h: keys = k_sel[g] followed by k_blk[:, g], g = h // G; output
    = softmax(scale * q.keys^T) . values, no mask ([HERALD-v1]: the denoising phase
    reuses the selected subset for all T steps). Returns [B][Hq][d].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_sel.shape[0]
    out = np.empty((B, Hq, d), dtype=np.float64)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        keys = np.concatenate([np.asarray(k_sel[g], np.float64), np.asarray(k_blk[:, g, :], np.float64)])
        vals = np.concatenate([np.asarray(v_sel[g], np.float64), np.asarray(v_blk[:, g, :], np.float64)])
        w = softmax(scale * (q[:, h, :] @ keys.T), axis=1)
        out[:, h, :] = w @ vals
    return out


def herald_block(q0, k_cache, v_cache, q_steps, kb_steps, vb_steps, C: int, topk: int, scale: float) -> dict:
    """The whole per-block path for one sequence: select, refine, gather, then T attention steps.

    q0: [B][Hq][d] (merged for the scan and used by refine); k_cache, v_cache:
    [L][Hkv][d]; q_steps: [T][B][Hq][d]; kb_steps, vb_steps: [T][B][Hkv][d].
    """
    cand, S = select_merged(q0, k_cache, C, scale)
    sel, R = refine_topk(q0, k_cache, cand, topk, scale)
    k_sel, v_sel = gather_kv(k_cache, v_cache, sel)
    outs = [block_attention(q_steps[t], kb_steps[t], vb_steps[t], k_sel, v_sel, scale)
            for t in range(len(q_steps))]
    return {"cand": cand, "S": S, "sel": sel, "R": R, "k_sel": k_sel, "v_sel": v_sel, "out": outs}
