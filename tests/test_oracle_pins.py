"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one oracle step to a closed form, a library routine in fp64
(torch on the CPU), brute force on tiny inputs, or a constructed input whose
answer is known by construction. The set is chosen so that a dropped term, a
wrong sign, an off-by-one in a window or block boundary, a transposed operand
or a swapped projection fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import numerics
from workloads import PrefillWorkload, DecodeWorkload, make_prefill, \
    make_decode, bf16_bits

torch.set_num_threads(min(8, torch.get_num_threads()))


def _prefill(S, Hq, Hkv, d, ret, window, top_k, r=16, block=64, seed=0,
             needles=0):
    w = PrefillWorkload("t", S=S, Hq=Hq, Hkv=Hkv, d=d, n_ret=len(ret),
                        window=window, r=r, block=block, top_k=top_k,
                        seed=seed, retrieval_heads=tuple(ret),
                        needles=needles)
    x = make_prefill(w)
    x["qb"], x["kb"], x["vb"] = (bf16_bits(x["q"]), bf16_bits(x["k"]),
                                 bf16_bits(x["v"]))
    return x


def _run(x, **kw):
    args = dict(window=x["window"], p_q=x["p_q"], p_k=x["p_k"],
                block=x["block"], top_k=x["top_k"])
    args.update(kw)
    return oracle.hybrid_prefill(x["qb"], x["kb"], x["vb"], x["is_retrieval"],
                                 **args)


def _sdpa64(q, k, v, mask):
    """torch fp64 reference: softmax(q k^T / sqrt(d) + mask) v, and lse."""
    q, k, v = (torch.from_numpy(np.asarray(t, np.float64)) for t in (q, k, v))
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None], v[None], attn_mask=m[None])[0]
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    lse = torch.logsumexp(s.masked_fill(~m, -math.inf), dim=-1)
    return o.numpy(), lse.numpy()


def _f32(bits):
    return numerics.bf16_to_f32(bits)


# ---------------------------------------------------------------- numerics
def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.normal(size=100000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40,
                  np.inf, -np.inf, 1.00390625, 1.01171875, 65504.0],
                 dtype=np.float32),
        # exact halfway cases between neighbouring bf16 values
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ours = numerics.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)
    assert np.array_equal(ours, ref)
    back = numerics.bf16_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16)
                          .float().numpy())


# ------------------------------------------------ attention given key sets
@pytest.mark.parametrize("S", [320, 300])
def test_full_coverage_equals_dense_causal(S):
    # window >= S and k >= n_b - 2: every head sees every earlier token.
    x = _prefill(S, Hq=4, Hkv=2, d=64, ret=(1, 2), window=S, top_k=8)
    res = _run(x)
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    causal = np.tril(np.ones((S, S), dtype=bool))
    for h in range(4):
        o, lse = _sdpa64(q[h], k[h // 2], v[h // 2], causal)
        assert np.abs(res["out"][h] - o).max() < 2e-5
        assert np.abs(res["lse"][h] - lse).max() < 2e-5


def test_window_one_returns_v_exactly():
    x = _prefill(256, Hq=2, Hkv=1, d=32, ret=(), window=1, top_k=4)
    res = _run(x)
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    for h in range(2):
        assert np.array_equal(res["out"][h], v[0])
        s = (q[h].astype(np.float64) * k[0]).sum(-1) / math.sqrt(32)
        assert np.abs(res["lse"][h] - s).max() < 1e-5


def test_v_all_ones_gives_ones():
    x = _prefill(384, Hq=4, Hkv=1, d=32, ret=(0, 3), window=70, top_k=2)
    x["vb"] = np.full_like(x["vb"], 0x3F80)  # bf16 1.0
    res = _run(x)
    assert np.abs(res["out"] - 1.0).max() < 1e-6


def test_swa_band_matches_masked_sdpa():
    S, w = 333, 37
    x = _prefill(S, Hq=2, Hkv=1, d=48, ret=(), window=w, top_k=1)
    res = _run(x)
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    t = torch.ones(S, S, dtype=torch.bool)
    band = (torch.tril(t) & torch.triu(t, diagonal=-(w - 1))).numpy()
    for h in range(2):
        o, lse = _sdpa64(q[h], k[0], v[0], band)
        assert np.abs(res["out"][h] - o).max() < 2e-5
        assert np.abs(res["lse"][h] - lse).max() < 2e-5


def test_per_head_windows_match_masked_sdpa():
    # a window per streaming head: each head is the textbook band of its own
    # width (1: the value itself; >= S: causal), whatever its neighbours use
    S = 300
    windows = [1, 37, 300 + 5, 64, 2, 150]
    x = _prefill(S, Hq=6, Hkv=2, d=48, ret=(), window=8, top_k=1)
    res = _run(x, window=windows)
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    t = torch.ones(S, S, dtype=torch.bool)
    for h, w in enumerate(windows):
        band = (torch.tril(t) & torch.triu(t, diagonal=-(w - 1))).numpy()
        o, lse = _sdpa64(q[h], k[h // 3], v[h // 3], band)
        assert np.abs(res["out"][h] - o).max() < 2e-5, h
        assert np.abs(res["lse"][h] - lse).max() < 2e-5, h
    assert np.array_equal(res["out"][0], v[0])


def test_full_retrieval_heads_are_dense_causal_with_centroids():
    # retrieval heads in full mode attend every earlier token (dense causal,
    # textbook), streaming heads keep their windows, and the key clustering
    # is still produced: centroid = P_k mean(k) per block (linearity)
    S = 330
    x = _prefill(S, Hq=4, Hkv=2, d=64, ret=(1, 2), window=40, top_k=2)
    res = _run(x, retrieval_full=True)
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    t = torch.ones(S, S, dtype=torch.bool)
    causal = torch.tril(t).numpy()
    band = (torch.tril(t) & torch.triu(t, diagonal=-39)).numpy()
    for h in range(4):
        o, lse = _sdpa64(q[h], k[h // 2], v[h // 2],
                         causal if h in (1, 2) else band)
        assert np.abs(res["out"][h] - o).max() < 2e-5, h
        assert np.abs(res["lse"][h] - lse).max() < 2e-5, h
    n_b = -(-S // 64)
    for rho, h in enumerate((1, 2)):
        kg = k[h // 2].astype(np.float64)
        means = np.stack([kg[b * 64:(b + 1) * 64].mean(0) for b in range(n_b)])
        alt = means @ x["p_k"][rho].T.astype(np.float64)
        assert np.abs(res["centroids"][rho] - alt).max() < \
            1e-5 * np.abs(alt).max()
    assert (res["sel_count"] == 0).all()  # no selection in full mode


def test_block_sparse_matches_masked_sdpa():
    S, B = 640, 64
    x = _prefill(S, Hq=2, Hkv=1, d=64, ret=(0,), window=64, top_k=3)
    res = _run(x)
    n_b = S // B
    sel = res["sel"][0]
    blk = np.zeros((n_b, n_b), dtype=bool)
    for qb in range(n_b):
        blk[qb, sel[qb][sel[qb] >= 0]] = True
    tok = np.kron(blk, np.ones((B, B), dtype=bool)).astype(bool)
    tok &= np.tril(np.ones((S, S), dtype=bool))
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    o, lse = _sdpa64(q[0], k[0], v[0], tok)
    assert np.abs(res["out"][0] - o).max() < 2e-5
    assert np.abs(res["lse"][0] - lse).max() < 2e-5


def test_block_membership_equals_per_query_sets():
    rows = np.arange(128, 192)
    union, mem = oracle.swa_block_keys(rows, 50)
    for r, i in enumerate(rows):
        assert np.array_equal(union[mem[r]], oracle.swa_keys(int(i), 50))
    sel = np.array([0, 1, 2])
    union, mem = oracle.retrieval_block_keys(rows, sel, 64, 170)
    for r, i in enumerate(rows):
        assert np.array_equal(union[mem[r]],
                              oracle.selected_keys(sel, int(i), 64, 170))
    assert oracle.swa_keys(0, 8).tolist() == [0]
    assert oracle.swa_keys(10, 3).tolist() == [8, 9, 10]


def test_poisoned_keys_outside_sets_do_not_change_output():
    S = 512
    x = _prefill(S, Hq=2, Hkv=1, d=32, ret=(0,), window=40, top_k=2)
    ref = _run(x)
    # poison every key neither head can see for the last query block
    qb = S // 64 - 1
    rows = np.arange(qb * 64, S)
    seen = set(oracle.swa_block_keys(rows, 40)[0].tolist())
    seen |= set(oracle.retrieval_block_keys(rows, ref["sel"][0, qb][
        ref["sel"][0, qb] >= 0], 64, S)[0].tolist())
    bad = np.array(sorted(set(range(S)) - seen))
    x2 = dict(x)
    x2["kb"], x2["vb"] = x["kb"].copy(), x["vb"].copy()
    x2["kb"][0, bad] = 0x7FC0  # NaN
    x2["vb"][0, bad] = 0x7FC0
    res = _run(x2, sel_override={0: {qb: ref["sel"][0, qb][
        ref["sel"][0, qb] >= 0]}}, query_blocks=[qb])
    assert np.array_equal(res["out"][:, rows], ref["out"][:, rows])


def test_future_blocks_do_not_change_earlier_outputs():
    S = 512
    x = _prefill(S, Hq=2, Hkv=1, d=32, ret=(1,), window=100, top_k=2)
    ref = _run(x)
    x2 = dict(x)
    for key in ("qb", "kb", "vb"):
        x2[key] = x[key].copy()
        x2[key][:, 256:] ^= 0x1234   # scramble blocks 4..7
    res = _run(x2)
    assert np.array_equal(res["out"][:, :256], ref["out"][:, :256])
    assert np.array_equal(res["sel"][:, :4], ref["sel"][:, :4])


# ----------------------------------------------------------------- selection
def test_k0_keeps_only_sink_and_diagonal():
    x = _prefill(512, Hq=1, Hkv=1, d=32, ret=(0,), window=8, top_k=0)
    res = _run(x)
    for qb in range(8):
        s = res["sel"][0, qb]
        assert s[s >= 0].tolist() == sorted({0, qb})
        assert res["sel_count"][0, qb] == len({0, qb})


def _true_block_scores64(q, k, B, pq=None, pk=None):
    """fp64 brute force: every (qb, kb) score from the full product."""
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))
    S = q.shape[0]
    n_b = S // B
    qmean = qt.reshape(n_b, B, -1).mean(1)            # mean first ...
    if pq is not None:                                 # ... then project
        qmean = qmean @ torch.from_numpy(pq.astype(np.float64)).T
        kt = kt @ torch.from_numpy(pk.astype(np.float64)).T
    full = qmean @ kt.T                                # [n_b, S]
    return full.reshape(n_b, n_b, B).amax(-1).numpy()  # [qb, kb]


def _check_sets_against_scores(sel_row, scores_row, qb, k, log):
    cand = np.arange(1, qb)
    if len(cand) == 0:
        assert sel_row.tolist() == sorted({0, qb})
        return
    sc = scores_row[1:qb]
    order = np.lexsort((cand, -sc))
    want = set(cand[order[:k]].tolist()) | {0, qb}
    got = set(sel_row.tolist())
    if got != want:
        # allowed only inside the tie band of the k-th / (k+1)-th score
        s_k, s_k1 = sc[order[k - 1]], sc[order[k]]
        assert abs(s_k - s_k1) < 1e-4 * abs(s_k), (qb, got ^ want)
        for b in got ^ want:
            assert abs(scores_row[b] - s_k) < 1e-4 * abs(s_k)
        log.append((qb, s_k, s_k1))


def test_identity_projection_picks_true_top_blocks():
    # r = d and P = I: the indexer score is max_j mean_i q_i . k_j, the
    # block-averaged true logit; selection must be its exact top-k.
    S, d, B, k = 1024, 32, 64, 5
    x = _prefill(S, Hq=1, Hkv=1, d=d, ret=(0,), window=8, top_k=k, r=d)
    eye = np.eye(d, dtype=np.float32)[None]
    res = _run(x, p_q=eye, p_k=eye)
    q, kk = _f32(x["qb"])[0], _f32(x["kb"])[0]
    true = _true_block_scores64(q, kk, B)
    log = []
    for qb in range(S // B):
        s = res["sel"][0, qb]
        _check_sets_against_scores(s[s >= 0], true[qb], qb, k, log)
    assert len(log) == 0


def test_random_projection_selection_brute_force():
    S, d, B, k = 2048, 64, 64, 6
    x = _prefill(S, Hq=2, Hkv=1, d=d, ret=(0, 1), window=8, top_k=k)
    res = _run(x)
    q, kk = _f32(x["qb"]), _f32(x["kb"])[0]
    log = []
    for rho, h in enumerate((0, 1)):
        true = _true_block_scores64(q[h], kk, B, x["p_q"][rho], x["p_k"][rho])
        for qb in range(S // B):
            s = res["sel"][rho, qb]
            _check_sets_against_scores(s[s >= 0], true[qb], qb, k, log)
            if qb >= k + 2:
                srt = np.sort(true[qb][1:qb])[::-1]
                assert abs(res["kth"][rho, qb, 0] - srt[k - 1]) < \
                    1e-4 * abs(srt[k - 1]) + 1e-6
                assert abs(res["kth"][rho, qb, 1] - srt[k]) < \
                    1e-4 * abs(srt[k]) + 1e-6
    assert len(log) <= 2


def test_planted_selection_known_by_construction():
    # Projection = first r coordinates; every query is e_0; key j carries a
    # planted value in coordinate 0, so sc(qb, kb) = max of the planted
    # values of block kb, known exactly.
    S, d, r, B, k = 64 * 10, 32, 16, 64, 3
    qbits = numerics.f32_to_bf16(np.tile(np.eye(d, dtype=np.float32)[0],
                                         (1, S, 1)))
    vals = np.zeros((S,), dtype=np.float32)
    # block maxima: block 9 (diagonal of the last row) and block 0 (sink)
    # get the largest values and must not use up the top-k budget
    block_max = {0: 100.0, 1: 5.0, 2: 7.0, 3: -1.0, 4: 7.0, 5: 2.0,
                 6: 9.0, 7: 3.0, 8: 8.0, 9: 50.0}
    rng = np.random.default_rng(3)
    for b, m in block_max.items():
        vals[b * B:(b + 1) * B] = m - rng.uniform(1, 2, size=B)
        vals[b * B + rng.integers(B)] = m
    kf = np.zeros((1, S, d), dtype=np.float32)
    kf[0, :, 0] = vals
    p = np.zeros((1, r, d), dtype=np.float32)
    p[0, np.arange(r), np.arange(r)] = 1.0
    res = oracle.hybrid_prefill(qbits, numerics.f32_to_bf16(kf),
                                numerics.f32_to_bf16(kf), np.array([1]),
                                window=8, p_q=p, p_k=p, block=B, top_k=k)
    sel = lambda qb: res["sel"][0, qb][res["sel"][0, qb] >= 0].tolist()
    # row 9: candidates 1..8 with maxima 5,7,-1,7,2,9,3,8 -> 6, 8, then the
    # tie 2 vs 4 at 7.0 goes to the lower index 2.
    assert sel(9) == [0, 2, 6, 8, 9]
    assert res["kth"][0, 9].tolist() == [7.0, 7.0]
    # row 4: candidates 1..3 (maxima 5, 7, -1) -> all three kept
    assert sel(4) == [0, 1, 2, 3, 4]
    assert res["kth"][0, 4, 0] == -1.0 and math.isnan(res["kth"][0, 4, 1])
    # row 5: candidates 1..4 -> 4, 2 (tie, lower first), then 1
    assert sel(5) == [0, 1, 2, 4, 5]
    # rows 0, 1: nothing to choose
    assert sel(0) == [0] and sel(1) == [0, 1]
    # row 2: one candidate
    assert sel(2) == [0, 1, 2]


def test_power_of_two_scaling_leaves_selection_unchanged():
    x = _prefill(1024, Hq=1, Hkv=1, d=64, ret=(0,), window=8, top_k=4)
    a = _run(x)
    b = _run(x, p_q=x["p_q"] * 4, p_k=x["p_k"] * 0.5)
    assert np.array_equal(a["sel"], b["sel"])
    assert np.array_equal(a["kth"] * 2, b["kth"], equal_nan=True)


def test_indexer_linearity_and_centroids():
    x = _prefill(640, Hq=1, Hkv=1, d=128, ret=(0,), window=8, top_k=4)
    q, k = _f32(x["qb"])[0], _f32(x["kb"])[0]
    pq, pk = x["p_q"][0], x["p_k"][0]
    qbar = oracle.query_block_means(q, pq, 64)
    alt = q.astype(np.float64).reshape(10, 64, -1).mean(1) @ pq.T
    assert np.abs(qbar - alt).max() < 1e-5 * np.abs(alt).max()
    khat = oracle.project_keys(k, pk)
    cent = oracle.block_centroids(khat, 64)
    alt = k.astype(np.float64).reshape(10, 64, -1).mean(1) @ pk.T
    assert np.abs(cent - alt).max() < 1e-5 * np.abs(alt).max()
    res = _run(x)
    assert np.array_equal(res["centroids"][0], cent)


# -------------------------------------------------------------------- decode
def _decode(batch, L, Hq, Hkv, d, ret, window, top_k, lens=None, seed=0):
    w = DecodeWorkload("t", batch=batch, L=L, Hq=Hq, Hkv=Hkv, d=d,
                       n_ret=len(ret), window=window, r=16, block=64,
                       top_k=top_k, seed=seed, retrieval_heads=tuple(ret))
    x = make_decode(w, cache_len=lens)
    x["qb"], x["kb"], x["vb"] = (bf16_bits(x["q"]), bf16_bits(x["k_cache"]),
                                 bf16_bits(x["v_cache"]))
    return x


def _run_dec(x, **kw):
    args = dict(window=x["window"], p_q=x["p_q"], p_k=x["p_k"],
                block=x["block"], top_k=x["top_k"], n_recent=x["n_recent"])
    args.update(kw)
    return oracle.hybrid_decode(x["qb"], x["kb"], x["vb"], x["cache_len"],
                                x["is_retrieval"], **args)


def test_decode_full_coverage_equals_last_row_of_dense():
    lens = [700, 640, 65, 1]
    x = _decode(4, 700, Hq=4, Hkv=2, d=64, ret=(0, 3), window=10 ** 6,
                top_k=64, lens=lens)
    res = _run_dec(x)
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    for b, L in enumerate(lens):
        for h in range(4):
            o, lse = _sdpa64(q[b, h][None], k[b, h // 2, :L], v[b, h // 2, :L],
                             np.ones((1, L), dtype=bool))
            assert np.abs(res["out"][b, h] - o[0]).max() < 2e-5
            assert abs(res["lse"][b, h] - lse[0]) < 2e-5


def test_decode_window_is_last_w_tokens():
    x = _decode(2, 300, Hq=2, Hkv=1, d=32, ret=(), window=5, top_k=1,
                lens=[300, 3])
    res = _run_dec(x)
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    for b, L in enumerate([300, 3]):
        js = np.arange(max(0, L - 5), L)
        for h in range(2):
            s = (k[b, 0, js].astype(np.float64) @ q[b, h]) / math.sqrt(32)
            p = np.exp(s - s.max())
            p /= p.sum()
            assert np.abs(res["out"][b, h] - p @ v[b, 0, js]).max() < 1e-5


def test_decode_planted_selection():
    # 12 full blocks + 1 partial; centroid of block b along coordinate 0 is
    # planted, the query is e_0 and the projection is the first 16 coords.
    d, B, L = 32, 64, 64 * 12 + 5
    kf = np.zeros((1, 1, L, d), dtype=np.float32)
    planted = [3.0, 1.0, 4.0, 1.5, 9.0, 2.5, 6.0, 5.0, 3.5, 5.0, 0.5, 7.0]
    for b, m in enumerate(planted):
        kf[0, 0, b * B:(b + 1) * B, 0] = m
    qf = np.zeros((1, 1, d), dtype=np.float32)
    qf[0, 0, 0] = 1.0
    p = np.zeros((1, 16, d), dtype=np.float32)
    p[0, np.arange(16), np.arange(16)] = 1.0
    res = oracle.hybrid_decode(numerics.f32_to_bf16(qf),
                               numerics.f32_to_bf16(kf),
                               numerics.f32_to_bf16(kf), np.array([L]),
                               np.array([1]), window=8, p_q=p, p_k=p, block=B,
                               top_k=3, n_recent=2)
    # n_b = 13, recent = {11, 12}, candidates 1..10 with centroids
    # 1.0 4.0 1.5 9.0 2.5 6.0 5.0 3.5 5.0 0.5 -> 4, 6, then 7 (tie with 9)
    got = res["sel"][0, 0][res["sel"][0, 0] >= 0].tolist()
    assert got == [0, 4, 6, 7, 11, 12]
    assert res["kth"][0, 0].tolist() == [5.0, 5.0]


def test_decode_short_cache_keeps_everything():
    x = _decode(1, 64 * 5 + 3, Hq=1, Hkv=1, d=32, ret=(0,), window=4,
                top_k=3)
    res = _run_dec(x)
    assert res["sel"][0, 0][res["sel"][0, 0] >= 0].tolist() == list(range(6))


def _fp64_decode_centroids(k_seq, p_k, n_full, B=64):
    """fp64: P_k applied to the mean key of each full block (linearity)."""
    if n_full == 0:
        return np.zeros((0, p_k.shape[0]))
    kg = k_seq[:n_full * B].astype(np.float64)
    return kg.reshape(n_full, B, -1).mean(1) @ p_k.T.astype(np.float64)


def test_decode_centroids_are_projected_block_means():
    # Random, non-constant keys and ragged caches: only the full blocks get
    # a centroid (the partial block holding the newest tokens has none), and
    # each is P_k applied to the block's mean key, computed in fp64. A
    # max-pooled, first-key or mis-projected centroid fails.
    lens = [64 * 9 + 23, 64 * 4, 63, 64 * 6 + 1]
    x = _decode(4, max(lens), Hq=4, Hkv=2, d=64, ret=(1, 2), window=16,
                top_k=2, lens=lens, seed=7)
    res = _run_dec(x)
    k = _f32(x["kb"])
    for b, L in enumerate(lens):
        n_full = L // 64
        for rho, h in enumerate((1, 2)):
            c = res["centroids"][(b, rho)]
            assert c.shape == (n_full, 16), (b, rho, c.shape)
            alt = _fp64_decode_centroids(k[b, h // 2], x["p_k"][rho], n_full)
            if n_full:
                assert np.abs(c - alt).max() <= 1e-5 * np.abs(alt).max(), \
                    (b, rho)
                direct = oracle.decode_centroids(k[b, h // 2, :L],
                                                 x["p_k"][rho], 64, n_full)
                assert np.array_equal(direct, c)


def test_decode_selection_matches_fp64_brute_force():
    # Independent random P_q and P_k (so that using one for the other, or
    # scoring with anything but the block mean, changes the choice). The
    # kept set is {0} u top-k u {last n_recent blocks}, with the top-k taken
    # by fp64 scores (P_q q).(P_k mean k) over the candidates 1 .. n_b-3,
    # fully sorted, ties to the lower block; s_k / s_{k+1} are the k-th and
    # (k+1)-th of the same sort.
    lens = [64 * 150 + 17, 64 * 90, 64 * 40 + 1, 64 * 13 + 5]
    top_k = 12
    x = _decode(4, max(lens), Hq=4, Hkv=2, d=64, ret=(0, 3), window=16,
                top_k=top_k, lens=lens, seed=4)
    assert np.abs(x["p_q"] - x["p_k"]).max() > 0.1
    res = _run_dec(x)
    q, k = _f32(x["qb"]), _f32(x["kb"])
    log = []
    for b, L in enumerate(lens):
        n_b, n_full = -(-L // 64), L // 64
        n_c = n_b - x["n_recent"] - 1
        for rho, h in enumerate((0, 3)):
            qt = x["p_q"][rho].astype(np.float64) @ q[b, h].astype(np.float64)
            cents = _fp64_decode_centroids(k[b, h // 2], x["p_k"][rho],
                                           n_full)
            sc = cents[1:1 + n_c] @ qt
            cand = np.arange(1, 1 + n_c)
            order = np.lexsort((cand, -sc))
            want = set(cand[order[:top_k]].tolist()) | {0} | set(
                range(n_b - x["n_recent"], n_b))
            got_row = res["sel"][b, rho]
            got = set(got_row[got_row >= 0].tolist())
            assert res["sel_count"][b, rho] == len(got)
            if got != want and n_c > top_k:
                s_k, s_k1 = sc[order[top_k - 1]], sc[order[top_k]]
                assert abs(s_k - s_k1) < 1e-4 * abs(s_k), (b, rho)
                for blk in got ^ want:
                    assert 1 <= blk <= n_c
                    assert abs(sc[blk - 1] - s_k) < 1e-4 * abs(s_k)
                log.append((b, rho))
            if n_c <= top_k:  # short cache: every block, no k-th score
                assert got == set(range(n_b)), (b, rho)
                continue
            srt = np.sort(sc)[::-1]
            assert abs(res["kth"][b, rho, 0] - srt[top_k - 1]) <= \
                1e-5 * abs(srt[top_k - 1]) + 1e-6, (b, rho)
            assert abs(res["kth"][b, rho, 1] - srt[top_k]) <= \
                1e-5 * abs(srt[top_k]) + 1e-6, (b, rho)
    assert len(log) <= 1


def test_decode_selection_override_attends_the_given_blocks():
    # sel_override replaces the block choice of one (sequence, head): the
    # output is then exact attention over the tokens of the given blocks
    # (fp64 textbook softmax), whatever the scores say
    lens = [64 * 20 + 9]
    x = _decode(1, lens[0], Hq=2, Hkv=1, d=32, ret=(1,), window=8, top_k=3,
                lens=lens)
    blocks = [0, 5, 6, 13, 19, 20]
    res = _run_dec(x, sel_override={(0, 0): blocks})
    q, k, v = _f32(x["qb"]), _f32(x["kb"]), _f32(x["vb"])
    L = lens[0]
    js = np.concatenate([np.arange(b * 64, min(L, b * 64 + 64))
                         for b in blocks])
    s = (k[0, 0, js].astype(np.float64) @ q[0, 1]) / math.sqrt(32)
    p = np.exp(s - s.max())
    p /= p.sum()
    assert np.abs(res["out"][0, 1] - p @ v[0, 0, js]).max() < 1e-5
    got = res["sel"][0, 0]
    assert got[got >= 0].tolist() == blocks
