"""Plant plausible mistakes in the oracle (CPU only) and check a pin fails.

Each mutation replaces one oracle step with a subtly wrong version; the pin
suite in test_oracle_pins.py must reject every one of them.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.decode as od
import oracle.prefill as op
from tests import test_oracle_pins as pins

F32 = np.float32


def _swa_off_by_one(rows, w):
    lo = max(0, int(rows[0]) - w)
    union = np.arange(lo, int(rows[-1]) + 1, dtype=np.int64)
    i, j = rows[:, None], union[None, :]
    return union, (j <= i) & (j >= i - w)          # keeps w+1 keys


def _select_smallest(sc, qb, k):
    cand = np.arange(1, max(qb, 1), dtype=np.int64)
    order = np.lexsort((cand, sc))                  # sign flipped
    top = cand[order[:k]]
    s_k = float(sc[order[k - 1]]) if 1 <= k <= len(cand) else math.nan
    s_k1 = float(sc[order[k]]) if k + 1 <= len(cand) else math.nan
    return np.unique(np.concatenate([[0], top, [qb]])), s_k, s_k1


def _select_high_index_ties(sc, qb, k):
    cand = np.arange(1, max(qb, 1), dtype=np.int64)
    order = np.lexsort((-cand, -sc))                # ties: higher index
    top = cand[order[:k]]
    s_k = float(sc[order[k - 1]]) if 1 <= k <= len(cand) else math.nan
    s_k1 = float(sc[order[k]]) if k + 1 <= len(cand) else math.nan
    return np.unique(np.concatenate([[0], top, [qb]])), s_k, s_k1


def _score_drop_last_candidate(qbar_row, khat, qb, B):
    # the block just before the diagonal is wrongly left out
    sc = _orig_score(qbar_row, khat, qb, B).copy()
    if len(sc):
        sc[-1] = -np.inf
    return sc


def _select_diagonal_uses_slot(sc, qb, k):
    # the diagonal block wrongly counts against the top-k budget
    return _orig_select(sc, qb, max(k - 1, 0) if qb >= 1 else k)


def _score_mean_pool(qbar_row, khat, qb, B):
    if qb < 2:
        return np.zeros(0, dtype=F32)
    dots = khat[B:qb * B] @ qbar_row
    return dots.reshape(qb - 1, B).mean(axis=1).astype(F32)


def _score_shifted_block(qbar_row, khat, qb, B):
    if qb < 2:
        return np.zeros(0, dtype=F32)
    dots = khat[B - 1:qb * B - 1] @ qbar_row        # block edge off by one
    return dots.reshape(qb - 1, B).max(axis=1)


def _project_keys_with_pq_transposed(k_g, p_k):
    return (k_g @ p_k.T[::-1, ::-1].T).astype(F32)  # reversed coordinates


def _qmeans_last_row_only(q_h, p_q, B):
    S = q_h.shape[0]
    n_b = -(-S // B)
    qt = q_h @ p_q.T
    return np.stack([qt[min(S, (b + 1) * B) - 1] for b in range(n_b)]) \
        .astype(F32)


def _attend_no_scale(q_rows, k_keys, v_keys, member, scale):
    return _orig_attend(q_rows, k_keys, v_keys, member, 1.0)


def _attend_drop_max_row(q_rows, k_keys, v_keys, member, scale):
    member = member.copy()
    for r in range(member.shape[0]):            # drops the last key of a row
        idx = np.nonzero(member[r])[0]
        if len(idx) > 1:
            member[r, idx[-1]] = False
    return _orig_attend(q_rows, k_keys, v_keys, member, scale)


def _retrieval_keys_no_causal(rows, sel, B, S):
    union, _ = _orig_ret_keys(rows, sel, B, S)
    return union, np.ones((len(rows), len(union)), dtype=bool)


def _head_window_of_neighbour(window, h):
    if np.ndim(window) == 0:
        return int(window)
    w = np.asarray(window)
    return int(w[(h + 1) % len(w)])             # the next head's window


def _causal_keys_without_self(rows):
    union, member = _orig_causal_keys(rows)
    return union, member & (union[None, :] < rows[:, None])


def _decode_select_no_recent(q_tilde, cents, n_b, k, n_recent):
    sel, a, b = _orig_dec_select(q_tilde, cents, n_b, k, n_recent)
    return sel[sel < n_b - 1] if n_b > 1 else sel, a, b


def _dec_centroids_max_pool(k_seq, p_k, B, n_full):
    proj = k_seq[:n_full * B].astype(F32) @ p_k.astype(F32).T
    return proj.reshape(n_full, B, -1).max(axis=1).astype(F32)


def _dec_centroids_first_key(k_seq, p_k, B, n_full):
    proj = k_seq[:n_full * B].astype(F32) @ p_k.astype(F32).T
    return proj.reshape(n_full, B, -1)[:, 0].astype(F32)


def _decode_query_projected_with_pk(*args, **kw):
    # the decode query is wrongly projected with P_k instead of P_q
    args = list(args)
    if "p_k" in kw:
        pk = kw["p_k"]
    else:
        pk = args[7]
    if "p_q" in kw:
        kw["p_q"] = pk
    else:
        args[6] = pk
    return _orig_hybrid_decode(*args, **kw)


_orig_hybrid_decode = od.hybrid_decode
_orig_attend = op.attend
_orig_score = op.block_score_row
_orig_select = op.select_row
_orig_ret_keys = op.retrieval_block_keys
_orig_dec_select = od.decode_select
_orig_causal_keys = op.causal_block_keys

MUTATIONS = [
    (op, "swa_block_keys", _swa_off_by_one),
    (op, "select_row", _select_smallest),
    (op, "select_row", _select_high_index_ties),
    (op, "block_score_row", _score_drop_last_candidate),
    (op, "select_row", _select_diagonal_uses_slot),
    (op, "block_score_row", _score_mean_pool),
    (op, "block_score_row", _score_shifted_block),
    (op, "project_keys", _project_keys_with_pq_transposed),
    (op, "query_block_means", _qmeans_last_row_only),
    (op, "attend", _attend_no_scale),
    (op, "attend", _attend_drop_max_row),
    (op, "retrieval_block_keys", _retrieval_keys_no_causal),
    (od, "decode_select", _decode_select_no_recent),
    (op, "head_window", _head_window_of_neighbour),
    (op, "causal_block_keys", _causal_keys_without_self),
    (od, "decode_centroids", _dec_centroids_max_pool),
    (od, "decode_centroids", _dec_centroids_first_key),
    (oracle, "hybrid_decode", _decode_query_projected_with_pk),
]

PIN_TESTS = [
    lambda: pins.test_full_coverage_equals_dense_causal(300),
    pins.test_window_one_returns_v_exactly,
    pins.test_swa_band_matches_masked_sdpa,
    pins.test_block_sparse_matches_masked_sdpa,
    pins.test_identity_projection_picks_true_top_blocks,
    pins.test_random_projection_selection_brute_force,
    pins.test_planted_selection_known_by_construction,
    pins.test_indexer_linearity_and_centroids,
    pins.test_decode_full_coverage_equals_last_row_of_dense,
    pins.test_decode_window_is_last_w_tokens,
    pins.test_decode_planted_selection,
    pins.test_per_head_windows_match_masked_sdpa,
    pins.test_full_retrieval_heads_are_dense_causal_with_centroids,
    pins.test_decode_centroids_are_projected_block_means,
    pins.test_decode_selection_matches_fp64_brute_force,
    pins.test_decode_selection_override_attends_the_given_blocks,
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # a mutant may leave a row empty
@pytest.mark.parametrize("mod,name,fn", MUTATIONS,
                         ids=[m[2].__name__ for m in MUTATIONS])
def test_pins_reject_mutation(monkeypatch, mod, name, fn):
    monkeypatch.setattr(mod, name, fn)
    if mod is op and name == "attend":
        monkeypatch.setattr(od, "attend", fn)
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError, KeyError):
            caught += 1
            break
    assert caught, f"no pin rejects mutation {fn.__name__}"


# ------------------------------------------------------------- clustering
import oracle.cluster as oc  # noqa: E402
from tests import test_oracle_cluster_pins as cpins  # noqa: E402

_orig_nearest = oc.nearest_centroid
_orig_cselect = oc.clustered_select


def _nearest_by_dot(x, cents):
    # largest dot product instead of smallest distance (drops -|c|^2 / 2)
    return np.argmax(x @ cents.T, axis=1)


def _nearest_ties_high(x, cents):
    d2 = ((x[:, None, :] - cents[None, :, :]) ** 2).sum(axis=2)
    return d2.shape[1] - 1 - np.argmin(d2[:, ::-1], axis=1)


def _lloyd_empty_to_zero(x, cents):
    m = cents.shape[0]
    assign = oc.nearest_centroid(x, cents[1:]) + 1
    counts = np.bincount(assign, minlength=m)
    new = np.zeros_like(cents)
    for c in range(1, m):
        if counts[c]:
            new[c] = x[assign == c].mean(axis=0)
    return assign, new, counts


def _lloyd_sum_not_mean(x, cents):
    m = cents.shape[0]
    assign = oc.nearest_centroid(x, cents[1:]) + 1
    counts = np.bincount(assign, minlength=m)
    new = cents.copy()
    for c in range(1, m):
        if counts[c]:
            new[c] = x[assign == c].sum(axis=0)
    return assign, new, counts


def _count_off_by_one(L, block, n_recent):
    return max(-(-L // block) - n_recent + 1, 1)


def _group_members_descending(assign, m, first_token):
    off, mem = _orig_group(assign, m, first_token)
    mem = mem.copy()
    for c in range(1, m):
        mem[off[c]:off[c + 1]] = mem[off[c]:off[c + 1]][::-1]
    return off, mem


def _seeds_first_key(x, m, block):
    out = np.full((m, x.shape[1]), np.nan)
    for c in range(1, m):
        out[c] = x[(c - 1) * block]
    return out


def _select_ignores_empty(q_tilde, cent_of, valid_of, n_b, k, n_recent):
    return _orig_cselect(q_tilde, cent_of, lambda c: True, n_b, k, n_recent)


def _select_ties_high(q_tilde, cent_of, valid_of, n_b, k, n_recent):
    n_c = max(n_b - n_recent - 1, 0)
    cand = np.array([c for c in range(1, 1 + n_c) if valid_of(c)], np.int64)
    if len(cand) > k:
        sc = (np.stack([cent_of(c) for c in cand]).astype(F32) @
              q_tilde.astype(F32)).astype(F32)
        top = cand[np.lexsort((-cand, -sc))[:k]]
    else:
        top = cand
    recent = np.arange(n_b - n_recent, n_b, dtype=np.int64)
    sel = np.concatenate([[0], top, recent]).astype(np.int64)
    return np.unique(sel[sel >= 0])


def _kept_tokens_blocks_only(sel, m, offsets, members, L, block):
    parts = [np.arange(int(c) * block, min(L, (int(c) + 1) * block))
             for c in sel]
    return np.sort(np.concatenate(parts).astype(np.int64))


_orig_group = oc.group_members

CLUSTER_MUTATIONS = [
    (oc, "nearest_centroid", _nearest_by_dot),
    (oc, "nearest_centroid", _nearest_ties_high),
    (oc, "lloyd_step", _lloyd_empty_to_zero),
    (oc, "lloyd_step", _lloyd_sum_not_mean),
    (oc, "cluster_count", _count_off_by_one),
    (oc, "group_members", _group_members_descending),
    (oc, "block_means", _seeds_first_key),
    (oc, "clustered_select", _select_ignores_empty),
    (oc, "clustered_select", _select_ties_high),
    (oc, "kept_tokens", _kept_tokens_blocks_only),
]

CLUSTER_PIN_TESTS = [
    lambda: cpins.test_lloyd_matches_sklearn_kmeans(2),
    cpins.test_lloyd_brute_force_ties_and_empty_clusters,
    cpins.test_kmeans_objective_never_increases,
    cpins.test_planted_topics_are_recovered,
    cpins.test_cluster_range_and_tables,
    cpins.test_cluster_seeds_equal_decode_centroids,
    cpins.test_clustered_decode_with_block_clusters_equals_block_decode,
    cpins.test_clustered_decode_fp64_brute_force,
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("mod,name,fn", CLUSTER_MUTATIONS,
                         ids=[m[2].__name__ for m in CLUSTER_MUTATIONS])
def test_cluster_pins_reject_mutation(monkeypatch, mod, name, fn):
    monkeypatch.setattr(mod, name, fn)
    caught = 0
    for t in CLUSTER_PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError, KeyError):
            caught += 1
            break
    assert caught, f"no pin rejects mutation {fn.__name__}"
