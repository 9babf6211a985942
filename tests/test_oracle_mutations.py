"""Plant plausible mistakes in the CPU oracle and check that some pin catches each one.

Each mutation patches one oracle function (on the CPU, restored afterwards) with a
copy that carries a single mistake: a dropped term, a wrong sign or index, a
swapped operand, a wrong axis, a wrong tie rule. The pins of oracle_pins.py must
reject every mutant; a mutant that passes all pins would mean that part of the
oracle is not pinned.
"""

import numpy as np
import pytest

import oracle.herald_oracle as orc
from oracle_pins import ALL_PINS


def _refine_softmax_over_queries(q_refine, k_cache, cand, scale):
    q = np.asarray(q_refine, np.float64)
    k = np.asarray(k_cache, np.float64)
    B, Hq, _ = q.shape
    Hkv, C = cand.shape
    R = np.zeros((Hkv, C))
    for g in range(Hkv):
        keys = k[cand[g], g, :]
        for h in range(Hq):
            if orc.kv_head_of(h, Hq, Hkv) == g:
                R[g] += orc.softmax(scale * (q[:, h, :] @ keys.T), axis=0).sum(axis=0)
    return R


def _refine_with_merged_query(q_refine, k_cache, cand, scale):
    qm = np.repeat(orc.merge_queries(q_refine)[None], q_refine.shape[0], axis=0)
    return _ORIG["refine_scores"](qm, k_cache, cand, scale)


def _attention_without_block_keys(q, k_blk, v_blk, k_sel, v_sel, scale):
    return _ORIG["block_attention"](q, k_blk[:0], v_blk[:0], k_sel, v_sel, scale)


def _attention_without_selected(q, k_blk, v_blk, k_sel, v_sel, scale):
    return _ORIG["block_attention"](q, k_blk, v_blk, k_sel[:, :0], v_sel[:, :0], scale)


def _scores_unnormalised(logits, Hkv):
    Hq, L = logits.shape
    S = np.zeros((Hkv, L))
    for h in range(Hq):
        S[orc.kv_head_of(h, Hq, Hkv)] += np.exp(logits[h] - logits[h].max())
    return S


def _scores_max_over_heads(logits, Hkv):
    Hq, L = logits.shape
    p = orc.softmax(logits, axis=1)
    S = np.zeros((Hkv, L))
    for h in range(Hq):
        g = orc.kv_head_of(h, Hq, Hkv)
        S[g] = np.maximum(S[g], p[h])
    return S


def _topk_ties_high(score, k, tiebreak=None):
    n = len(score)
    tb = np.arange(n) if tiebreak is None else np.asarray(tiebreak)
    return np.sort(np.lexsort((-tb, -np.asarray(score, np.float64)))[:k])


def _topk_smallest(score, k, tiebreak=None):
    n = len(score)
    tb = np.arange(n) if tiebreak is None else np.asarray(tiebreak)
    return np.sort(np.lexsort((tb, np.asarray(score, np.float64)))[:k])


def _gather_head0(k_cache, v_cache, sel):
    return (np.stack([np.asarray(k_cache)[sel[g], 0, :] for g in range(sel.shape[0])]),
            np.stack([np.asarray(v_cache)[sel[g], 0, :] for g in range(sel.shape[0])]))


def _gather_k_for_v(k_cache, v_cache, sel):
    ks, _ = _ORIG["gather_kv"](k_cache, v_cache, sel)
    return ks, ks


def _softmax_no_normalise(x, axis=-1):
    x = np.asarray(x, np.float64)
    return np.exp(x - x.max(axis=axis, keepdims=True))


def _scan_negated(q_merged, k_cache, scale):
    return -_ORIG["scan_logits"](q_merged, k_cache, scale)


def _scan_transposed_group(q_merged, k_cache, scale):
    q = np.asarray(q_merged, np.float64)
    k = np.asarray(k_cache, np.float64)
    Hq, Hkv = q.shape[0], k.shape[1]
    return np.stack([scale * (k[:, h % Hkv, :] @ q[h]) for h in range(Hq)])


def _compress_window_not_cut(k_cache, ksize, stride):
    # divides by ksize even where the window runs past the end of the sequence
    k = np.asarray(k_cache, np.float64)
    L = k.shape[0]
    M = -(-L // stride)
    return np.stack([k[m * stride:min(m * stride + ksize, L)].sum(axis=0) / ksize for m in range(M)])


def _compress_disjoint(k_cache, ksize, stride):
    # ignores the overlap: windows of `stride` tokens
    return _ORIG["compress_keys"](k_cache, stride, stride)


def _select_compressed_block_index(q_merge, k_cache, C, scale, ksize, stride):
    # maps token j to block j // ksize instead of j // stride
    L, Hkv = k_cache.shape[0], k_cache.shape[1]
    kc = orc.compress_keys(k_cache, ksize, stride)
    S_blk = orc.group_scores(orc.scan_logits(orc.merge_queries(q_merge), kc, scale), Hkv)
    S_tok = S_blk[:, np.minimum(np.arange(L) // ksize, S_blk.shape[1] - 1)]
    cand = np.stack([orc.top_k_ascending(S_tok[g], C) for g in range(Hkv)])
    return cand, S_tok, S_blk


_ORIG = {n: getattr(orc, n) for n in ["refine_scores", "block_attention", "gather_kv", "scan_logits",
                                       "compress_keys"]}

MUTANTS = {
    "merge_sum_not_mean": ("merge_queries", lambda q: np.asarray(q, np.float64).sum(axis=0)),
    "merge_first_query": ("merge_queries", lambda q: np.asarray(q, np.float64)[0]),
    "scale_one": ("default_scale", lambda d: 1.0),
    "scale_over_d": ("default_scale", lambda d: 1.0 / d),
    "interleaved_groups": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "scan_negated": ("scan_logits", _scan_negated),
    "scan_interleaved_groups": ("scan_logits", _scan_transposed_group),
    "scores_unnormalised": ("group_scores", _scores_unnormalised),
    "scores_max_over_heads": ("group_scores", _scores_max_over_heads),
    "softmax_not_normalised": ("softmax", _softmax_no_normalise),
    "topk_ties_to_high_index": ("top_k_ascending", _topk_ties_high),
    "topk_smallest": ("top_k_ascending", _topk_smallest),
    "refine_softmax_over_queries": ("refine_scores", _refine_softmax_over_queries),
    "refine_with_merged_query": ("refine_scores", _refine_with_merged_query),
    "attention_drops_block_keys": ("block_attention", _attention_without_block_keys),
    "attention_drops_selected": ("block_attention", _attention_without_selected),
    "gather_wrong_head": ("gather_kv", _gather_head0),
    "gather_k_as_v": ("gather_kv", _gather_k_for_v),
    "compress_window_not_cut": ("compress_keys", _compress_window_not_cut),
    "compress_disjoint": ("compress_keys", _compress_disjoint),
    "select_compressed_block_index": ("select_compressed", _select_compressed_block_index),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
