"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to something other than its own code:
a library routine on a special case, a closed form, the explainer's chain
example (tests/golden/chain_example.json), brute force on tiny inputs, or
an invariant the pages state.  Chosen so that a plausible slip (a dropped
term, a wrong sign, a swapped tie rule, an off-by-one slot) fails one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, gen

HERE = os.path.dirname(os.path.abspath(__file__))
TINY = WORKLOADS["tiny"]


def _small(**kw):
    base = dict(batch=1, vocab=64, topk=2, depth=3, budget_n=6, threshold=0.0,
                logits_dtype="f32", sharpness=(1.5,), n_q_heads=1,
                n_kv_heads=1, head_dim=64, prefix_cap=16,
                prefix_range=(16, 16), qkv_dtype="f32", seed=0)
    base.update(kw)
    if "sharpness" not in kw:
        base["sharpness"] = tuple([1.5] * base["batch"])
    return TINY.with_(**base)


def _np_softmax64(row):
    x = row.astype(np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _rows_of(logits, dtype):
    return gen.bf16_bits_to_f32(logits) if dtype == "bf16" else logits


# ---------------------------------------------------------------- draft step
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_softmax_match_numpy(dtype):
    """Children and conf of step 1 == numpy fp64 softmax + lexsort top-k
    (library routine), including rows with many exactly equal logits."""
    V, k, B = 300, 7, 6
    w = _small(batch=B, vocab=V, topk=k, depth=1, budget_n=7,
               logits_dtype=dtype)
    g = np.random.default_rng(11)
    x = (g.standard_normal((B, 1, V)) * 2).astype(np.float32)
    x[0:3] = np.round(x[0:3])            # heavy ties: integer logits
    x[5, 0, :] = 0.0                      # all equal: ids 0..k-1 win
    x[4, 0, 17] = -np.inf                 # -inf is allowed (conf 0)
    logits = gen.f32_to_bf16_bits(x) if dtype == "bf16" else x
    roots = np.arange(B, dtype=np.int32)
    st = oracle.TreeState(w)
    oracle.draft_step(w, st, 1, roots, logits)
    xf = _rows_of(logits, dtype)
    for b in range(B):
        row = xf[b, 0]
        order = np.lexsort((np.arange(V), -row.astype(np.float64)))[:k]
        assert list(st.token[b, :k]) == list(order)
        p = _np_softmax64(row)[order].astype(np.float32)
        np.testing.assert_allclose(st.conf[b, :k], p, rtol=2e-7, atol=0)
        np.testing.assert_array_equal(st.value[b, :k], st.conf[b, :k])
        assert (st.parent[b, :k] == -1).all() and (st.depth[b, :k] == 1).all()
    assert list(st.token[5, :k]) == list(range(k))


def test_closed_form_single_peak():
    """One logit a, V-1 zeros: conf(peak) = e^a / (e^a + V - 1), the other
    children are the lowest ids with conf 1 / (e^a + V - 1)."""
    V, k, a, peak = 1000, 4, 5.0, 500
    w = _small(vocab=V, topk=k, depth=1, budget_n=4)
    x = np.zeros((1, 1, V), np.float32)
    x[0, 0, peak] = a
    st = oracle.TreeState(w)
    oracle.draft_step(w, st, 1, np.array([7], np.int32), x)
    den = math.exp(a) + V - 1
    assert list(st.token[0, :k]) == [peak, 0, 1, 2]
    assert st.conf[0, 0] == pytest.approx(math.exp(a) / den, rel=1e-7)
    for r in range(1, k):
        assert st.conf[0, r] == pytest.approx(1.0 / den, rel=1e-7)


def _peak_logit(c, V):
    """Logit a that gives the peak conf c in a row of V-1 zeros."""
    return math.log(c * (V - 1) / (1.0 - c))


def _chain_draft(conf_steps, V=512):
    D = len(conf_steps)
    draft = np.zeros((1, D, 1, V), np.float64)
    for l, c in enumerate(conf_steps):
        draft[0, l, 0, 10 + l] = _peak_logit(c, V)
    return draft.astype(np.float32)


def test_chain_example_values():
    """Explainer, 'Common misconception': path products 0.9, 0.72, 0.55,
    0.40 sum to 2.57 expected accepted tokens."""
    gold = json.load(open(os.path.join(HERE, "golden", "chain_example.json")))
    vals = gold["path_products"]
    steps = [vals[0]] + [vals[i] / vals[i - 1] for i in range(1, len(vals))]
    w = _small(vocab=512, topk=1, depth=4, budget_n=4)
    st = oracle.build_tree(w, np.array([3], np.int32), _chain_draft(steps))
    rr = oracle.rerank(w, st)
    np.testing.assert_allclose(rr["value"][0, 1:5], vals, rtol=2e-6)
    assert abs(float(rr["value"][0, 1:5].astype(np.float64).sum())
               - gold["expected_accepted"]) < 1e-5
    assert list(rr["parent_slot"][0]) == [-1, 0, 1, 2, 3]
    assert list(rr["tokens"][0, 1:]) == [10, 11, 12, 13]


def _calibrated_chain_targets(w, rr, steps, trials, rng):
    """Target rows whose argmax at slot s is the chain child with
    probability steps[s] (the child's conf), else another token."""
    T, V = w.T, w.vocab
    planted = np.empty((trials, T), np.int64)
    for s in range(T):
        child = rr["tokens"][0, s + 1] if s + 1 < T else 0
        hit = rng.random(trials) < (steps[s] if s < len(steps) else 0.0)
        other = rng.integers(0, V - 1, trials)
        other = np.where(other >= child, other + 1, other)
        planted[:, s] = np.where(hit, child, other)
    return planted


def test_chain_example_accept_statistics():
    """Greedy walk on calibrated targets: mean accept length -> 2.57 and
    full-sweep rate -> 0.40 (explainer chain example), each within a 99%
    interval of its Monte Carlo error."""
    gold = json.load(open(os.path.join(HERE, "golden", "chain_example.json")))
    vals = gold["path_products"]
    steps = [vals[0]] + [vals[i] / vals[i - 1] for i in range(1, len(vals))]
    w1 = _small(vocab=512, topk=1, depth=4, budget_n=4)
    st = oracle.build_tree(w1, np.array([3], np.int32), _chain_draft(steps))
    rr = oracle.rerank(w1, st)
    trials = 20000
    rng = np.random.default_rng(5)
    planted = _calibrated_chain_targets(w1, rr, steps, trials, rng)
    target = np.zeros((trials, w1.T, w1.vocab), np.float32)
    target[np.arange(trials)[:, None], np.arange(w1.T)[None, :], planted] = 1.0
    wt = w1.with_(batch=trials)
    rep = {k: np.repeat(rr[k], trials, axis=0) for k in ("tokens",
                                                         "parent_slot",
                                                         "n_kept")}
    acc = oracle.accept(wt, target, rep["tokens"], rep["parent_slot"],
                        rep["n_kept"])
    L = acc["accept_len"].astype(np.float64)
    z = 2.576
    assert abs(L.mean() - gold["expected_accepted"]) < z * L.std() / math.sqrt(trials)
    p = gold["full_sweep_probability"]
    sweep = (L == 4).mean()
    assert abs(sweep - p) < z * math.sqrt(p * (1 - p) / trials)


# ---------------------------------------------------------------- rerank
def _random_tree(w, seed, sharp=None):
    sharp = sharp if sharp is not None else w.sharpness
    ww = w.with_(sharpness=tuple(sharp), seed=seed)
    draft = gen.draft_logits(ww)
    roots = gen.root_tokens(ww)
    return ww, oracle.build_tree(ww, roots, draft), draft, roots


def _closed(subset, parent):
    s = set(subset)
    return all(parent[i] < 0 or parent[i] in s for i in subset)


@pytest.mark.parametrize("seed", range(40))
def test_rerank_brute_force_optimal(seed):
    """Greedy rerank maximises the sum of values over all connected
    (ancestor-closed) n-subsets of the pool, and is that subset when the
    maximum is unique (explainer: the objective is additive over nodes)."""
    sharp = [0.6, 1.0, 1.5, 2.5][seed % 4]
    w = _small(vocab=48, topk=2, depth=4, budget_n=5, sharpness=(sharp,))
    w, st, _, _ = _random_tree(w, seed)
    P = int(st.count[0])
    assert P <= 20
    n = min(w.budget_n, P)
    val = st.value[0, :P].astype(np.float64)
    par = st.parent[0, :P]
    sums = []
    for sub in itertools.combinations(range(P), n):
        if _closed(sub, par):
            sums.append((val[list(sub)].sum(), sub))
    sums.sort(key=lambda t: -t[0])
    rr = oracle.rerank(w, st)
    got = rr["value"][0, 1:n + 1].astype(np.float64).sum()
    assert abs(got - sums[0][0]) <= 1e-6
    if len(sums) == 1 or sums[0][0] - sums[1][0] > 1e-5:
        kept = set()
        for s in range(1, n + 1):
            # identify pool nodes by (token, depth-consistent parent chain)
            kept.add((int(rr["tokens"][0, s]), float(rr["value"][0, s])))
        best = {(int(st.token[0, i]), float(st.value[0, i])) for i in sums[0][1]}
        assert kept == best


@pytest.mark.parametrize("seed", range(60))
def test_rerank_invariants(seed):
    """Kept set connected, parent before child, values non-increasing along
    paths, conf in [0, 1] ([P2]: ancestors always outscore a node)."""
    w = _small(vocab=200, topk=3, depth=4, budget_n=12,
               sharpness=([0.8, 2.5, 1.5][seed % 3],))
    w, st, _, _ = _random_tree(w, seed)
    rr = oracle.rerank(w, st)
    n = int(rr["n_kept"][0])
    assert n == min(w.budget_n, int(st.count[0]))
    ps, v, c = rr["parent_slot"][0], rr["value"][0], rr["conf"][0]
    for s in range(1, n + 1):
        assert 0 <= ps[s] < s
        assert v[s] <= v[ps[s]]
        assert 0.0 <= c[s] <= 1.0
    for s in range(n + 1, w.T):
        assert rr["tokens"][0, s] == -1 and ps[s] == -1
    # kept values are the n largest of the pool
    pool_sorted = np.sort(st.value[0, :st.count[0]])[::-1]
    np.testing.assert_array_equal(np.sort(v[1:n + 1])[::-1], pool_sorted[:n])


def test_tie_goes_to_shallower_node():
    """[P3] ReRank: on equal values the shallower node ranks first.  A row
    with one logit 200 above the rest has conf == 1.0f exactly, so a chain
    of such rows gives parent and child the same value."""
    V = 64
    w = _small(vocab=V, topk=2, depth=4, budget_n=6)
    draft = np.full((1, 4, 2, V), -200.0, np.float32)
    for l in range(4):
        draft[0, l, :, 40 - l] = 0.0      # peak token 40, 39, 38, 37
    st = oracle.build_tree(w, np.array([1], np.int32), draft)
    rr = oracle.rerank(w, st)
    assert (rr["value"][0, 1:5] == 1.0).all()
    assert list(rr["tokens"][0, 1:5]) == [40, 39, 38, 37]
    assert list(rr["parent_slot"][0, 1:5]) == [0, 1, 2, 3]


def test_value_tie_then_lower_token():
    """Equal value and depth: lower token id first (exact logit ties inside
    one row give bit-identical conf)."""
    V = 32
    w = _small(vocab=V, topk=3, depth=1, budget_n=3)
    x = np.zeros((1, 1, V), np.float32)
    x[0, 0, [9, 4, 20]] = 3.0
    st = oracle.build_tree(w, np.array([0], np.int32), x[:, None])
    rr = oracle.rerank(w, st)
    assert list(rr["tokens"][0, 1:4]) == [4, 9, 20]


# ---------------------------------------------------------------- frontier
@pytest.mark.parametrize("seed", range(40))
def test_frontier_and_threshold_rule(seed):
    """Expansion ([P1] s4.1, [P3] Expand): each layer's expanded nodes are
    its top-k by value; no expanded node is below the threshold; every
    unexpanded node above depth D is below the threshold or ranked >= k."""
    w = _small(vocab=128, topk=2, depth=3, budget_n=8, threshold=0.1,
               sharpness=([1.5, 2.5, 3.5][seed % 3],))
    w, st, _, _ = _random_tree(w, seed)
    P = int(st.count[0])
    par = st.parent[0, :P]
    expanded = set(int(p) for p in par if p >= 0)
    for layer in range(1, w.depth):
        idx = [i for i in range(P) if st.depth[0, i] == layer]
        ranked = sorted(idx, key=lambda i: (-float(st.value[0, i]),
                                            int(st.token[0, i]), i))
        for r, i in enumerate(ranked):
            if i in expanded:
                assert st.value[0, i] >= w.threshold and r < w.topk
            else:
                assert st.value[0, i] < w.threshold or r >= w.topk
    for i in range(P):
        if st.depth[0, i] == w.depth:
            assert i not in expanded
    # children of one parent are that parent's row top-k (k per parent)
    for p in expanded:
        assert (par == p).sum() == w.topk


def _boundary_draft(w, ids=(5, 40)):
    """Every draft row: logit 0 at two ids, -inf elsewhere, so each row's
    softmax gives exactly 1/2 to both ids (a closed form)."""
    row = np.full(w.vocab, -np.inf, np.float32)
    row[list(ids)] = 0.0
    draft = np.ascontiguousarray(
        np.broadcast_to(row, (w.batch, w.depth, w.topk, w.vocab)))
    return gen.f32_to_bf16_bits(draft) if w.logits_dtype == "bf16" else draft


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_value_equal_to_threshold_is_expanded(dtype):
    """[P3] Expand stage: a node stays unexpanded only when its value is
    below the threshold.  With conf = 1/2 exactly (two equal finite
    logits), threshold 0.5 puts both children of the root exactly on it:
    they are expanded; their children (value 1/4) are not.  A '<=' slip
    in the stop rule leaves the root's children unexpanded."""
    w = _small(vocab=64, topk=2, depth=3, budget_n=8, threshold=0.5,
               logits_dtype=dtype)
    st = oracle.TreeState(w)
    roots = np.array([7], np.int32)
    draft = _boundary_draft(w)
    nt, nc = oracle.draft_step(w, st, 1, roots, draft[:, 0])
    assert st.conf[0, 0] == 0.5 and st.value[0, 0] == 0.5
    assert int(nc[0]) == 2 and sorted(nt[0].tolist()) == [5, 40]
    nt, nc = oracle.draft_step(w, st, 2, roots, draft[:, 1])
    assert (st.value[0, 2:6] == 0.25).all()
    assert int(nc[0]) == 0 and (nt[0] == -1).all()
    assert int(st.count[0]) == 6
    # just above the threshold: the root's children stop as well
    w2 = w.with_(threshold=float(np.nextafter(np.float32(0.5), np.float32(1))))
    st2 = oracle.TreeState(w2)
    _, nc2 = oracle.draft_step(w2, st2, 1, roots, draft[:, 0])
    assert int(nc2[0]) == 0


def test_stop_when_frontier_empty():
    """All values below the threshold after layer 1: nothing is expanded
    again and the pool keeps only the root's children."""
    w = _small(vocab=1000, topk=2, depth=3, budget_n=8, threshold=0.5,
               sharpness=(0.5,))
    w, st, _, _ = _random_tree(w, 3)
    assert st.count[0] == 2 and st.frontier_count[0] == 0


# ---------------------------------------------------------------- mask
@pytest.mark.parametrize("N", [6, 63, 64, 130, 255])
def test_mask_matches_parent_walk(N):
    """Mask bits == the slots met walking parent pointers to the root;
    popcount == depth + 1; pos = prefix + depth; pads are empty."""
    g = np.random.default_rng(N)
    B = 3
    w = _small(batch=B, budget_n=N)
    T = N + 1
    parent = np.full((B, T), -1, np.int32)
    n_kept = np.array([N, N // 2, 0], np.int32)
    for b in range(B):
        for s in range(1, n_kept[b] + 1):
            parent[b, s] = g.integers(0, s)
    prefix = np.array([5, 0, 17], np.int32)
    mk = oracle.tree_mask(w, parent, n_kept, prefix)
    for b in range(B):
        for s in range(T):
            bits = {t for t in range(T)
                    if (int(mk["mask"][b, s, t // 64]) >> (t % 64)) & 1}
            if s > n_kept[b]:
                assert not bits and mk["depth"][b, s] == -1
                assert mk["pos_ids"][b, s] == -1
                continue
            walk, cur = set(), s
            while cur >= 0:
                walk.add(cur)
                cur = parent[b, cur] if cur > 0 else -1
            assert bits == walk
            assert mk["depth"][b, s] == len(walk) - 1
            assert mk["pos_ids"][b, s] == prefix[b] + len(walk) - 1


# ---------------------------------------------------------------- attention
def _attn_case(seed, B=2, N=9, Hq=4, Hkv=2, d=64, Pcap=24, dtype="f32"):
    w = _small(batch=B, budget_n=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
               prefix_cap=Pcap, prefix_range=(3, Pcap), qkv_dtype=dtype,
               seed=seed)
    inp = gen.attention_inputs(w)
    prefix = gen.prefix_lens(w)
    g = np.random.default_rng(seed)
    parent = np.full((B, w.T), -1, np.int32)
    n_kept = g.integers(1, N + 1, B).astype(np.int32)
    for b in range(B):
        for s in range(1, n_kept[b] + 1):
            parent[b, s] = g.integers(0, s)
    mk = oracle.tree_mask(w, parent, n_kept, prefix)
    return w, inp, prefix, parent, n_kept, mk


def _f64(a, dtype):
    return (gen.bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_equals_per_path_causal(dtype):
    """Verify ([P2] one tree-attention pass, exactly as in the static-tree
    scheme): row s equals dense causal attention over prefix ++ the path
    root->s at its last position (torch fp64 SDPA)."""
    w, inp, prefix, parent, n_kept, mk = _attn_case(1, dtype=dtype)
    out = oracle.tree_attention(w, inp, prefix, mk["mask"], n_kept)
    q, kc, vc, kt, vt = (_f64(inp[n], dtype) for n in
                         ("q", "k_cache", "v_cache", "k_tree", "v_tree"))
    for b in range(w.batch):
        for s in range(w.T):
            if s > n_kept[b]:
                assert (out[b, s] == 0).all()
                continue
            path, cur = [], s
            while cur >= 0:
                path.append(cur)
                cur = parent[b, cur] if cur > 0 else -1
            path = path[::-1]
            for h in range(w.n_q_heads):
                kv = h // w.G
                K = np.concatenate([kc[b, kv, :prefix[b]], kt[b, kv, path]])
                Vv = np.concatenate([vc[b, kv, :prefix[b]], vt[b, kv, path]])
                L = K.shape[0]
                qs = np.zeros((L, w.head_dim))
                qs[-1] = q[b, s, h]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(qs)[None], torch.from_numpy(K)[None],
                    torch.from_numpy(Vv)[None], is_causal=True,
                    scale=w.scale)[0, -1].numpy()
                np.testing.assert_allclose(out[b, s, h], ref, rtol=0,
                                           atol=1e-12)


@pytest.mark.parametrize("dtype,seed,Pcap", [("f32", 3, 40), ("bf16", 4, 40),
                                              ("f32", 5, 12), ("bf16", 6, 12)])
def test_kv_commit_is_the_path_in_depth_order(dtype, seed, Pcap):
    """KV commit ([P1] s2.1: accepted tokens extend the sequence in path
    order): the appended rows are the K/V rows of the root->leaf path, one
    per depth (depth and ancestry from the independent mask walk, rows
    matched bit for bit); nothing else in the cache changes; P advances by
    L + 1 unless prefix_cap stops it; and when nothing is dropped the leaf's
    tree attention equals dense causal attention over the committed cache
    (torch fp64 SDPA)."""
    w, inp, prefix, parent, n_kept, mk = _attn_case(seed, Pcap=Pcap, dtype=dtype)
    g = np.random.default_rng(seed)
    path_slots = np.full((w.batch, w.depth + 1), -1, np.int32)
    accept_len = np.zeros(w.batch, np.int32)
    leaf = np.zeros(w.batch, np.int64)
    for b in range(w.batch):
        # the deepest kept slot that a depth-w.depth walk can reach
        cands = [s for s in range(n_kept[b] + 1) if mk["depth"][b, s] <= w.depth]
        leaf[b] = int(g.choice(cands))
        path, cur = [], int(leaf[b])
        while cur > 0:
            path.append(cur)
            cur = int(parent[b, cur])
        path = [0] + path[::-1]
        path_slots[b, :len(path)] = path
        accept_len[b] = len(path) - 1
    kc2, vc2, p2 = oracle.kv_commit(w, inp, prefix, path_slots, accept_len)
    kc, vc, kt, vt = (inp[n] for n in ("k_cache", "v_cache", "k_tree", "v_tree"))
    q64, kc64, vc64 = (_f64(a, dtype) for a in (inp["q"], kc2, vc2))
    for b in range(w.batch):
        P, L = int(prefix[b]), int(accept_len[b])
        assert p2[b] == min(P + L + 1, w.prefix_cap)
        new = int(p2[b])
        for h in range(w.n_kv_heads):
            assert np.array_equal(kc2[b, h, :P], kc[b, h, :P])
            assert np.array_equal(kc2[b, h, new:], kc[b, h, new:])
            assert np.array_equal(vc2[b, h, :P], vc[b, h, :P])
            assert np.array_equal(vc2[b, h, new:], vc[b, h, new:])
            for i in range(new - P):
                hits = [s for s in range(n_kept[b] + 1)
                        if np.array_equal(kt[b, h, s], kc2[b, h, P + i])]
                assert len(hits) == 1
                s = hits[0]
                assert mk["depth"][b, s] == i
                word = int(mk["mask"][b, leaf[b], s // 64])
                assert (word >> (s % 64)) & 1
                assert np.array_equal(vt[b, h, s], vc2[b, h, P + i])
        if P + L + 1 > w.prefix_cap:
            continue
        out = oracle.tree_attention(w, inp, prefix, mk["mask"], n_kept)
        for hq in range(w.n_q_heads):
            kv = hq // w.G
            qs = np.zeros((new, w.head_dim))
            qs[-1] = q64[b, leaf[b], hq]
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qs)[None], torch.from_numpy(kc64[b, kv, :new])[None],
                torch.from_numpy(vc64[b, kv, :new])[None], is_causal=True,
                scale=w.scale)[0, -1].numpy()
            np.testing.assert_allclose(out[b, leaf[b], hq], ref, rtol=0, atol=1e-12)


def test_attention_equal_keys_is_mean_of_visible_values():
    """Closed form: with every key equal the softmax is uniform, so the
    output is the mean of the visible values (prefix + ancestors + self)."""
    w, inp, prefix, parent, n_kept, mk = _attn_case(2)
    inp = dict(inp)
    inp["k_cache"] = np.ones_like(inp["k_cache"])
    inp["k_tree"] = np.ones_like(inp["k_tree"])
    out = oracle.tree_attention(w, inp, prefix, mk["mask"], n_kept)
    for b in range(w.batch):
        for s in range(n_kept[b] + 1):
            vis = [t for t in range(w.T)
                   if (int(mk["mask"][b, s, 0]) >> t) & 1]
            for h in range(w.n_q_heads):
                kv = h // w.G
                vals = np.concatenate([inp["v_cache"][b, kv, :prefix[b]],
                                       inp["v_tree"][b, kv, vis]]).astype(np.float64)
                np.testing.assert_allclose(out[b, s, h], vals.mean(0),
                                           atol=1e-12)


def test_attention_rows_match_full():
    w, inp, prefix, parent, n_kept, mk = _attn_case(3, dtype="bf16")
    full = oracle.tree_attention(w, inp, prefix, mk["mask"], n_kept)
    rows = [(0, 0, 0), (1, int(n_kept[1]), 3), (0, 1, 2), (1, w.T - 1, 1)]
    part = oracle.attention_rows(w, inp, prefix, mk["mask"], n_kept, rows)
    for i, (b, s, h) in enumerate(rows):
        np.testing.assert_array_equal(part[i], full[b, s, h])


# ---------------------------------------------------------------- accept
@pytest.mark.parametrize("seed", range(30))
def test_accept_brute_force(seed):
    """[P1] s2.1 greedy: the walk ends at the deepest slot all of whose
    path edges match the target argmax at the parent (numpy argmax, first
    maximum = lowest id); the bonus is that slot's argmax."""
    w = _small(vocab=40, topk=3, depth=4, budget_n=12, sharpness=(2.0,))
    w, st, _, _ = _random_tree(w, seed)
    rr = oracle.rerank(w, st)
    g = np.random.default_rng(seed)
    n = int(rr["n_kept"][0])
    # integer-valued targets (ties common), with a random kept path planted
    target = np.round(g.standard_normal((1, w.T, w.vocab)) * 2).astype(np.float32)
    leaf = int(g.integers(0, n + 1))
    path, cur = [], leaf
    while cur > 0:
        path.append(cur)
        cur = rr["parent_slot"][0, cur]
    for c in path:
        if g.random() < 0.85:
            target[0, rr["parent_slot"][0, c], rr["tokens"][0, c]] = 50.0
    acc = oracle.accept(w, target, rr["tokens"], rr["parent_slot"],
                        rr["n_kept"])
    am = np.argmax(target[0], axis=1)
    best, best_depth = 0, 0
    for s in range(1, n + 1):
        ok, cur, dep = True, s, 0
        while cur > 0:
            p = rr["parent_slot"][0, cur]
            ok &= rr["tokens"][0, cur] == am[p]
            cur, dep = p, dep + 1
        if ok and dep > best_depth:
            best, best_depth = s, dep
    L = int(acc["accept_len"][0])
    assert L == best_depth
    assert acc["path_slots"][0, L] == best
    assert acc["out_tokens"][0, L] == am[best]
    assert (acc["path_slots"][0, L + 1:] == -1).all()
    for i in range(1, L + 1):
        assert acc["out_tokens"][0, i - 1] == rr["tokens"][0, acc["path_slots"][0, i]]


def test_expected_accept_equals_sum_of_values():
    """Explainer value equation: E[#accepted] = sum of kept values when the
    target's choice at each slot is drawn from that slot's draft softmax
    (calibrated drafter).  Monte Carlo over 20000 targets, 99% interval."""
    w = _small(vocab=24, topk=2, depth=3, budget_n=5, sharpness=(1.0,))
    w, st, draft, roots = _random_tree(w, 7)
    rr = oracle.rerank(w, st)
    n = int(rr["n_kept"][0])
    # which draft row produced each slot's children: slot -> (layer, row)
    row_of = {}
    T = w.T
    P = int(st.count[0])
    order = sorted(range(P), key=lambda i: (-float(st.value[0, i]),
                                            int(st.depth[0, i]),
                                            int(st.token[0, i]), i))
    slot_of_pool = {order[s - 1]: s for s in range(1, n + 1)}
    assert [int(st.token[0, order[s - 1]]) for s in range(1, n + 1)] == \
        list(rr["tokens"][0, 1:n + 1])
    row_of[0] = (0, 0)
    # frontier order of layer l is the order of parents among layer-l+1 nodes
    for l in range(1, w.depth):
        parents = []
        for i in range(P):
            if st.depth[0, i] == l + 1 and st.parent[0, i] not in parents:
                parents.append(int(st.parent[0, i]))
        for j, p in enumerate(parents):
            if p in slot_of_pool:
                row_of[slot_of_pool[p]] = (l, j)
    trials = 20000
    rng = np.random.default_rng(1)
    planted = rng.integers(0, w.vocab, (trials, T))
    for s, (l, j) in row_of.items():
        p = _np_softmax64(draft[0, l, j])
        planted[:, s] = rng.choice(w.vocab, size=trials, p=p)
    target = np.zeros((trials, T, w.vocab), np.float32)
    target[np.arange(trials)[:, None], np.arange(T)[None, :], planted] = 1000.0
    wt = w.with_(batch=trials)
    rep = {k: np.repeat(rr[k], trials, axis=0) for k in ("tokens",
                                                         "parent_slot",
                                                         "n_kept")}
    acc = oracle.accept(wt, target, rep["tokens"], rep["parent_slot"],
                        rep["n_kept"])
    L = acc["accept_len"].astype(np.float64)
    expect = rr["value"][0, 1:n + 1].astype(np.float64).sum()
    assert abs(L.mean() - expect) < 2.576 * L.std() / math.sqrt(trials) + 1e-3


# ------------------------------------------------- sampled accept (T > 0)
def _tree_targets(w, rr, g, planted_boost, gap=0.0):
    """Target rows [1][T][V] ~ 1.5 N(0,1); every kept slot's token gets
    planted_boost at its parent's row (so children carry real mass); with
    gap > 0 each row's maximum is raised by gap above the runner-up."""
    target = g.standard_normal((1, w.T, w.vocab)) * 1.5
    n = int(rr["n_kept"][0])
    for c in range(1, n + 1):
        if g.random() < 0.8:
            target[0, rr["parent_slot"][0, c], rr["tokens"][0, c]] += planted_boost
    if gap > 0:
        for s in range(w.T):
            r = target[0, s]
            i = int(np.argmax(r))
            r[i] += gap
    return target.astype(np.float32)


@pytest.mark.parametrize("seed", range(20))
def test_sampled_accept_low_temperature_is_greedy(seed):
    """As the temperature goes to 0 the target softmax becomes the argmax
    point mass, so the ratio tests accept exactly the greedy path ([P1]
    s2.1 and [P4] s五: greedy decoding) and the bonus is the argmax: equal
    to the greedy walk, itself pinned by brute force."""
    w = _small(vocab=40, topk=3, depth=4, budget_n=12, sharpness=(2.0,))
    w, st, _, _ = _random_tree(w, 100 + seed)
    rr = oracle.rerank(w, st)
    g = np.random.default_rng(seed)
    target = _tree_targets(w, rr, g, planted_boost=6.0, gap=0.5)
    u = g.uniform(1e-3, 1.0, (1, w.T)).astype(np.float32)
    greedy = oracle.accept(w, target, rr["tokens"], rr["parent_slot"],
                           rr["n_kept"])
    samp = oracle.accept_sample(w, target, rr["tokens"], rr["parent_slot"],
                                rr["n_kept"], 1e-3, u)
    for k in ("accept_len", "path_slots", "out_tokens"):
        np.testing.assert_array_equal(samp[k], greedy[k])
    assert samp["margin"][0] > 1e-6


def _chi2_ok(counts, probs, alpha=1e-4):
    """Pearson chi-square of counts against probs, bins with expected
    count < 5 pooled into one."""
    from scipy.stats import chisquare
    n = counts.sum()
    exp = probs * n
    big = exp >= 5
    obs = np.append(counts[big], counts[~big].sum())
    ex = np.append(exp[big], exp[~big].sum())
    if ex[-1] < 5:
        obs[-2] += obs[-1]
        ex[-2] += ex[-1]
        obs, ex = obs[:-1], ex[:-1]
    return chisquare(obs, ex * (obs.sum() / ex.sum())).pvalue > alpha


@pytest.mark.parametrize("tau", [0.7, 1.3])
def test_sampled_accept_preserves_the_target_distribution(tau):
    """Losslessness ([P1] s1: the generated text keeps the target model's
    distribution).  Over many uniform draws on one tree, the first output
    token follows softmax(target[root] / tau) exactly, and given that it
    is the token of root child c, the second output token follows
    softmax(target[c] / tau), and so on one level deeper (chi-square)."""
    w = _small(vocab=10, topk=3, depth=3, budget_n=8, sharpness=(1.0,))
    w, st, _, _ = _random_tree(w, 3)
    rr = oracle.rerank(w, st)
    g = np.random.default_rng(11)
    target = _tree_targets(w, rr, g, planted_boost=1.5)
    trials = 60000
    wt = w.with_(batch=trials)
    rep = {k: np.repeat(rr[k], trials, axis=0)
           for k in ("tokens", "parent_slot", "n_kept")}
    tb = np.broadcast_to(target, (trials, w.T, w.vocab))
    u = g.random((trials, w.T), dtype=np.float32)
    acc = oracle.accept_sample(wt, tb, rep["tokens"], rep["parent_slot"],
                               rep["n_kept"], tau, u)
    out = acc["out_tokens"]
    tok, par = rr["tokens"][0], rr["parent_slot"][0]
    n = int(rr["n_kept"][0])

    def sm(s):
        x = target[0, s].astype(np.float64) / tau
        e = np.exp(x - x.max())
        return e / e.sum()

    assert _chi2_ok(np.bincount(out[:, 0], minlength=w.vocab), sm(0))
    checked = 0
    for c in range(1, n + 1):
        if par[c] != 0:
            continue
        sel = out[:, 0] == tok[c]
        assert (acc["accept_len"][sel] >= 1).all()
        if sel.sum() < 500:
            continue
        assert _chi2_ok(np.bincount(out[sel, 1], minlength=w.vocab), sm(c))
        checked += 1
        for c2 in range(1, n + 1):
            if par[c2] != c:
                continue
            sel2 = sel & (out[:, 1] == tok[c2])
            if sel2.sum() < 500:
                continue
            assert _chi2_ok(np.bincount(out[sel2, 2], minlength=w.vocab), sm(c2))
            checked += 1
    assert checked >= 2
    # the bonus is never a rejected sibling: when the walk stops at slot
    # s, out_tokens[L] is not the token of any child of s
    L = acc["accept_len"]
    last = acc["path_slots"][np.arange(trials), L]
    bonus = out[np.arange(trials), L]
    for s in range(n + 1):
        kids = {int(tok[c]) for c in range(1, n + 1) if par[c] == s}
        at = last == s
        assert not np.isin(bonus[at], list(kids)).any()


def test_sampled_accept_zero_uniforms_take_first_child():
    """u = 0: every ratio test passes for a child of positive mass, so the
    walk follows the first (highest-value) child of each slot to a leaf,
    and the bonus is id 0 (the residual's first id of positive mass)."""
    w = _small(vocab=30, topk=3, depth=4, budget_n=12, sharpness=(2.0,))
    for seed in range(10):
        w, st, _, _ = _random_tree(w, 200 + seed)
        rr = oracle.rerank(w, st)
        g = np.random.default_rng(seed)
        target = _tree_targets(w, rr, g, planted_boost=0.0)
        u = np.zeros((1, w.T), np.float32)
        acc = oracle.accept_sample(w, target, rr["tokens"], rr["parent_slot"],
                                   rr["n_kept"], 1.0, u)
        n = int(rr["n_kept"][0])
        par = rr["parent_slot"][0]
        cur, path = 0, [0]
        while True:
            kids = [c for c in range(1, n + 1) if par[c] == cur]
            if not kids:
                break
            cur = min(kids)
            path.append(cur)
        L = len(path) - 1
        assert acc["accept_len"][0] == L
        np.testing.assert_array_equal(acc["path_slots"][0, :L + 1], path)
        assert acc["out_tokens"][0, L] == 0


# ------------------------------------------------------------ LM head
def test_lm_head_logits_are_the_plain_sums():
    """Logits from hidden states equal the sums written out term by term
    (exact on bf16 inputs in fp64), for a tiny head in vocab blocks that
    do not divide the vocabulary."""
    g = np.random.default_rng(2)
    hb = gen.f32_to_bf16_bits(g.standard_normal((2, 3, 8)).astype(np.float32))
    wb = gen.f32_to_bf16_bits(g.standard_normal((7, 8)).astype(np.float32))
    got = oracle.lm_head_logits(hb, wb, block=3)
    h, W = gen.bf16_bits_to_f32(hb), gen.bf16_bits_to_f32(wb)
    for b in range(2):
        for j in range(3):
            for v in range(7):
                want = 0.0
                for k in range(8):
                    want += float(h[b, j, k]) * float(W[v, k])
                assert got[b, j, v] == want


# ------------------------------------------------------------ static tree
def _dynamic_shape(w, st, rr, b=0):
    """(parent, rank) of the kept dynamic tree in slot order; a node's rank
    among its parent's children comes from its pool index (children are
    appended per frontier row in rank order)."""
    n = int(rr["n_kept"][b])
    P = int(st.count[b])
    start = {}
    for i in range(P):
        start.setdefault(int(st.depth[b, i]), i)
    slot_of = {}
    order = sorted(range(P), key=lambda i: (-float(st.value[b, i]),
                                            int(st.depth[b, i]),
                                            int(st.token[b, i]), i))
    for s_, i in enumerate(order[:n], start=1):
        slot_of[i] = s_
    parent, rank = [-1], [-1]
    for s_, i in enumerate(order[:n], start=1):
        par = int(st.parent[b, i])
        parent.append(0 if par < 0 else slot_of[par])
        rank.append((i - start[int(st.depth[b, i])]) % w.topk)
    return np.array(parent, np.int32), np.array(rank, np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_static_tree_with_the_full_dynamic_shape_is_the_dynamic_tree(seed):
    """With a budget that keeps the whole pool, the dynamic tree's own
    shape, run as a static shape on the same logits, reads the same rows
    (its expanded nodes are the dynamic frontiers, in the same order) and
    must give the dynamic tree bit for bit: tokens, parents, conf, value."""
    w = _small(vocab=300, topk=3, depth=3, threshold=0.0, sharpness=(1.5,))
    w = w.with_(budget_n=w.pool_cap)
    w, st, draft, roots = _random_tree(w, 300 + seed)
    rr = oracle.rerank(w, st)
    assert int(rr["n_kept"][0]) == w.pool_cap
    p, r = _dynamic_shape(w, st, rr)
    sr = oracle.static_tree(w, roots, draft, p, r)
    for key in ("tokens", "parent_slot", "conf", "value", "n_kept"):
        np.testing.assert_array_equal(sr[key], rr[key])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_static_chain_is_the_product_of_top1_confidences(dtype):
    """A chain of rank-0 children reads row 0 of every layer: slot d holds
    that row's argmax (lowest id on ties) with conf = its numpy fp64
    softmax probability and value = the running fp32 product."""
    w = _small(batch=2, vocab=500, topk=4, depth=5, budget_n=5,
               logits_dtype=dtype, sharpness=(2.0, 0.9))
    draft = gen.draft_logits(w)
    roots = gen.root_tokens(w)
    p = np.arange(-1, w.depth, dtype=np.int32)
    r = np.zeros(w.depth + 1, np.int32)
    sr = oracle.static_tree(w, roots, draft, p, r)
    for b in range(w.batch):
        val = np.float32(1.0)
        for d in range(1, w.depth + 1):
            row = _rows_of(draft[b, d - 1, 0], dtype).astype(np.float64)
            tok = int(np.argmax(row))
            conf = np.float32(_np_softmax64(row)[tok])
            val = np.float32(val * conf)
            assert sr["tokens"][b, d] == tok and sr["parent_slot"][b, d] == d - 1
            assert abs(float(sr["conf"][b, d]) - float(conf)) <= 1e-6 * float(conf)
            assert abs(float(sr["value"][b, d]) - float(val)) <= 1e-5 * float(val)


def test_static_shape_rules_are_enforced():
    """Rank out of range, a repeated sibling rank, a forward parent, depth
    past D and more than k rows in one layer are all rejected."""
    w = _small(vocab=64, topk=2, depth=2, budget_n=6)
    draft, roots = gen.draft_logits(w), gen.root_tokens(w)
    bad = [([-1, 0], [-1, 2]),                    # rank >= k
           ([-1, 0, 0], [-1, 1, 1]),              # repeated sibling rank
           ([-1, 2, 0], [-1, 0, 0]),              # parent after the node
           ([-1, 0, 1, 2], [-1, 0, 0, 0])]        # depth 3 > D
    for p, r in bad:
        with pytest.raises(ValueError):
            oracle.static_tree(w, roots, draft, np.array(p), np.array(r))
    w3 = _small(vocab=64, topk=2, depth=3, budget_n=10)
    d3, r3 = gen.draft_logits(w3), gen.root_tokens(w3)
    # three depth-2 nodes with children: more than k = 2 rows in layer 2
    p = [-1, 0, 0, 1, 1, 2, 3, 4, 5]
    r = [-1, 0, 1, 0, 1, 0, 0, 0, 0]
    with pytest.raises(ValueError):
        oracle.static_tree(w3, r3, d3, np.array(p), np.array(r))
    sr = oracle.static_tree(w3, r3, d3, np.array(p[:8]), np.array(r[:8]))
    assert int(sr["n_kept"][0]) == 7


# ---------------------------------------------------------------- generator
def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.0e38],
                 np.float32)
    h = gen.f32_to_bf16_bits(x)
    back = gen.bf16_bits_to_f32(h)
    np.testing.assert_array_equal(back[:4], [1.0, 1.0, 1.0 + 2**-6, -2.5])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(back, ref)


def test_generator_is_seeded_and_shaped():
    w = WORKLOADS["tiny"]
    a, b = gen.draft_logits(w), gen.draft_logits(w)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (1, w.depth, w.topk, w.vocab)
    inp = gen.attention_inputs(w)
    assert inp["q"].shape == (1, w.T, 1, 64)
    w64 = WORKLOADS["llama8b_b64"]
    p = gen.prefix_lens(w64)
    assert p.min() >= 512 and p.max() <= 4096 and len(set(p)) > 10
