"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Every check below ties the oracle to something other than itself: the
worked example's printed result, brute force with Python floats, torch's
scaled-dot-product attention on an unpaged copy of the cache, closed forms
and invariants. The mutation tests at the end plant plausible mistakes in the
oracle (on the CPU) and show that a pin catches each one.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mla_oracle as orc
from mla_inputs import make_decode_case, random_tiny_mla, tiny_mla_weights
from conftest import load_golden


def _np(t):
    return t.detach().to(torch.float64).numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def _case_arrays(case):
    return (_np(case.q_lat), _np(case.cache), case.block_table.numpy(),
            case.seqlens.numpy())


# ---------------------------------------------------------------------------
# Independent references used by the pins
# ---------------------------------------------------------------------------

def brute_decode(q_lat, cache, table, seqlens, scale, causal, dv):
    """Python-float loops: one score at a time, math.exp, no numpy reductions."""
    B, s_q, H, D = q_lat.shape
    page = cache.shape[1]
    o = np.zeros((B, s_q, H, dv))
    lse = np.zeros((B, s_q, H))
    for b in range(B):
        L = int(seqlens[b])
        rows = [cache[int(table[b][j // page])][j % page] for j in range(L)]
        for i in range(s_q):
            last = (L - s_q + i) if causal else (L - 1)
            for h in range(H):
                q = [float(x) for x in q_lat[b, i, h]]
                scores = []
                for j in range(last + 1):
                    acc = 0.0
                    for k in range(D):
                        acc += q[k] * float(rows[j][k])
                    scores.append(acc * scale)
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                Z = sum(w)
                for c in range(dv):
                    acc = 0.0
                    for j in range(last + 1):
                        acc += w[j] * float(rows[j][c])
                    o[b, i, h, c] = acc / Z
                lse[b, i, h] = mx + math.log(Z)
    return o, lse


def sdpa_decode(q_lat, cache, table, seqlens, scale, causal, dv):
    """torch SDPA (fp64, CPU) on an unpaged copy: the absorbed decode is an MQA
    with one shared wide key/value head."""
    B, s_q, H, D = q_lat.shape
    page = cache.shape[1]
    o = np.zeros((B, s_q, H, dv))
    for b in range(B):
        L = int(seqlens[b])
        npg = (L + page - 1) // page
        flat = torch.from_numpy(cache[table[b, :npg]].reshape(npg * page, D)[:L])
        q = torch.from_numpy(q_lat[b]).transpose(0, 1)  # [H, s_q, D]
        k = flat.expand(H, L, D)
        v = flat[:, :dv].expand(H, L, dv)
        j = torch.arange(L)[None, :]
        i = torch.arange(s_q)[:, None]
        mask = (j <= L - s_q + i) if causal else torch.ones(s_q, L, dtype=torch.bool)
        out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        o[b] = out.transpose(0, 1).numpy()
    return o


# ---------------------------------------------------------------------------
# Worked example: the page prints that both paths agree (allclose, atol 1e-5).
# ---------------------------------------------------------------------------

def test_worked_example_matches_printed_output():
    g = load_golden("worked_example.txt")
    w = tiny_mla_weights(0)
    args = (w["h"], w["W_q"], w["W_dkv"], w["W_kr"], w["W_uk"], w["W_uv"], w["W_o"],
            w["H"], w["NOPE"], w["ROPE"])
    y1 = orc.mla_forward_expanded(*args)
    y2 = orc.mla_forward_absorbed(*args)
    assert bool(np.allclose(y1, y2, atol=g["paths_allclose_atol"], rtol=0)) == g["paths_allclose"]
    # In fp64 the two paths agree to rounding, far inside the printed bound.
    assert np.max(np.abs(y1 - y2)) <= 1e-12
    assert np.all(np.isfinite(y1)) and np.abs(y1).max() > 1e-3
    H, NOPE, ROPE, DV, DC = (int(w[k]) for k in ("H", "NOPE", "ROPE", "DV", "DC"))
    assert H * (NOPE + ROPE) + H * DV == g["cache_numbers_per_token_mha"]
    assert DC + ROPE == g["cache_numbers_per_token_mla"]


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("causal", [True, False])
def test_paths_agree_random_tiny(seed, causal):
    w = random_tiny_mla(seed, T=4 + seed, H=2 + seed, DC=7 + 3 * seed)
    args = (w["h"], w["W_q"], w["W_dkv"], w["W_kr"], w["W_uk"], w["W_uv"], w["W_o"],
            w["H"], w["NOPE"], w["ROPE"])
    y1 = orc.mla_forward_expanded(*args, causal=causal)
    y2 = orc.mla_forward_absorbed(*args, causal=causal)
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * max(1.0, np.abs(y1).max())


def test_expanded_attention_matches_sdpa():
    """Path one checked against torch SDPA with the per-head K, V it builds."""
    w = random_tiny_mla(7, T=7, H=3)
    q_n, q_r, c, k_r = orc.project(w["h"], w["W_q"], w["W_dkv"], w["W_kr"], w["H"], w["NOPE"], w["ROPE"])
    out = orc.expanded_attention(q_n, q_r, c, k_r, w["W_uk"], w["W_uv"], causal=True)
    T, H = q_n.shape[:2]
    kn = torch.einsum("tc,hcd->htd", torch.from_numpy(c), torch.from_numpy(w["W_uk"]))
    k = torch.cat([kn, torch.from_numpy(k_r).expand(H, T, -1)], -1)
    v = torch.einsum("tc,hcd->htd", torch.from_numpy(c), torch.from_numpy(w["W_uv"]))
    q = torch.cat([torch.from_numpy(q_n), torch.from_numpy(q_r)], -1).transpose(0, 1)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True,
                                         scale=1 / math.sqrt(w["NOPE"] + w["ROPE"]))
    assert np.max(np.abs(out - ref.transpose(0, 1).numpy())) <= 1e-13


# ---------------------------------------------------------------------------
# Projections of the worked example ("两条等价的路径"): q = h W_q viewed per
# head as [nope | rope], the nope block kept, the rope block rotated along the
# token axis; c = h W_dkv; k_r = RoPE(h W_kr); y = out flattened head-major
# (token t, head h, element d at column h*DV + d) times W_o. The checks take
# the projection (or forward) function as an argument so that the mutation
# tests below can run the same checks on planted mistakes.
# ---------------------------------------------------------------------------

def _project_dims():
    return dict(T=7, D=10, H=3, NOPE=4, ROPE=6, DC=5)


def check_project(project):
    """Raise AssertionError unless ``project`` places and rotates each block
    as the worked example defines. Expected values come from Python's
    math.cos / math.sin and from reading weight entries, not from the oracle."""
    d = _project_dims()
    T, D, H, NOPE, ROPE, DC = (d[k] for k in ("T", "D", "H", "NOPE", "ROPE", "DC"))
    W = NOPE + ROPE
    rng = np.random.default_rng(123)
    W_q = rng.standard_normal((D, H * W))
    W_dkv = rng.standard_normal((D, DC))
    W_kr = rng.standard_normal((D, ROPE))

    # (1) One-hot hidden rows h[t] = e_t: h W = the first T rows of W, so every
    # projected element is one weight entry. The nope block of head h, token
    # t, element d is W_q[t, h*W + d]; the latent is W_dkv[t]; at position 0
    # the rotation is the identity, so q_r[0] and k_r[0] are raw entries.
    h = np.eye(T, D)
    q_n, q_r, c, k_r = project(h, W_q, W_dkv, W_kr, H, NOPE, ROPE)
    assert q_n.shape == (T, H, NOPE) and q_r.shape == (T, H, ROPE)
    assert c.shape == (T, DC) and k_r.shape == (T, ROPE)
    for t in range(T):
        for hh in range(H):
            for e in range(NOPE):
                assert q_n[t, hh, e] == W_q[t, hh * W + e]
    assert np.array_equal(c, W_dkv[:T])
    for hh in range(H):
        for e in range(ROPE):
            assert abs(q_r[0, hh, e] - W_q[0, hh * W + NOPE + e]) <= 1e-15
    assert np.allclose(k_r[0], W_kr[0], rtol=0, atol=1e-15)

    # (2) Every token row equal to e_0 and one weight column of ones routed
    # into element 2i of head hh's rope block: along the tokens that pair is
    # (cos t*th_i, sin t*th_i), th_i = 10000^(-2i/R), and everything else is 0.
    h = np.zeros((T, D))
    h[:, 0] = 1.0
    for hh, i in ((0, 0), (2, 1), (1, 2)):
        Wq1 = np.zeros((D, H * W))
        Wq1[0, hh * W + NOPE + 2 * i] = 1.0
        Wkr1 = np.zeros((D, ROPE))
        Wkr1[0, 2 * i] = 1.0
        q_n, q_r, _, k_r = project(h, Wq1, W_dkv, Wkr1, H, NOPE, ROPE)
        exp_q = np.zeros((T, H, ROPE))
        exp_k = np.zeros((T, ROPE))
        for t in range(T):
            th = t / 10000.0 ** (2 * i / ROPE)
            exp_q[t, hh, 2 * i] = exp_k[t, 2 * i] = math.cos(th)
            exp_q[t, hh, 2 * i + 1] = exp_k[t, 2 * i + 1] = math.sin(th)
        assert not np.any(q_n)
        assert np.allclose(q_r, exp_q, rtol=0, atol=1e-14)
        assert np.allclose(k_r, exp_k, rtol=0, atol=1e-14)

    # (3) Random weights, every token row the same random vector: the rope
    # score <q_r[t,h], k_r[s]> depends on t - s only, and differs between
    # offsets (the rotation is not the identity).
    h = np.tile(rng.standard_normal(D), (T, 1))
    _, q_r, _, k_r = project(h, W_q, W_dkv, W_kr, H, NOPE, ROPE)
    for hh in range(H):
        dots = q_r[:, hh, :] @ k_r.T  # [t, s]
        for off in range(-(T - 1), T):
            diag = np.diagonal(dots, offset=-off)  # entries with t - s = off
            assert np.max(np.abs(diag - diag[0])) <= 1e-12
        assert abs(dots[3, 0] - dots[0, 0]) > 1e-6


def check_output_flatten(forward):
    """Raise AssertionError unless ``forward`` (a full tiny MLA path) applies
    W_o to the per-head outputs flattened head-major. With W_o a selector of
    column h*DV + d, output column j must equal head h's element d from
    expanded_attention (pinned against torch SDPA above)."""
    w = random_tiny_mla(9, T=5, D=12, H=3, NOPE=4, ROPE=4, DV=5, DC=6)
    H, DV, D = w["H"], w["DV"], w["D"]
    q_n, q_r, c, k_r = orc.project(w["h"], w["W_q"], w["W_dkv"], w["W_kr"], H, w["NOPE"], w["ROPE"])
    out = orc.expanded_attention(q_n, q_r, c, k_r, w["W_uk"], w["W_uv"], causal=True)
    picks = [(0, 1), (1, 0), (2, 4), (1, 3)]
    W_o = np.zeros((H * DV, D))
    for j, (hh, e) in enumerate(picks):
        W_o[hh * DV + e, j] = 1.0
    y = forward(w["h"], w["W_q"], w["W_dkv"], w["W_kr"], w["W_uk"], w["W_uv"], W_o,
                H, w["NOPE"], w["ROPE"])
    for j, (hh, e) in enumerate(picks):
        assert np.max(np.abs(y[:, j] - out[:, hh, e])) <= 1e-12
    assert not np.any(y[:, len(picks):])


def test_project_places_and_rotates_blocks():
    check_project(orc.project)


@pytest.mark.parametrize("path", ["expanded", "absorbed"])
def test_output_projection_is_head_major(path):
    check_output_flatten(orc.mla_forward_expanded if path == "expanded" else orc.mla_forward_absorbed)


def _project_rope_over_heads(h, W_q, W_dkv, W_kr, H, nope, rope_dim):
    """Planted mistake: the query's rotation runs over the head axis."""
    h = np.asarray(h, np.float64)
    T = h.shape[0]
    q = (h @ W_q).reshape(T, H, nope + rope_dim)
    return q[..., :nope], orc.rope_adjacent(q[..., nope:]), h @ W_dkv, orc.rope_adjacent(h @ W_kr)


def _project_swapped_halves(h, W_q, W_dkv, W_kr, H, nope, rope_dim):
    """Planted mistake: the rope block taken from the front of each head."""
    h = np.asarray(h, np.float64)
    T = h.shape[0]
    q = (h @ W_q).reshape(T, H, nope + rope_dim)
    q_r = orc.rope_adjacent(np.transpose(q[..., :rope_dim], (1, 0, 2))).transpose(1, 0, 2)
    return q[..., rope_dim:], q_r, h @ W_dkv, orc.rope_adjacent(h @ W_kr)


def _project_token_head_transposed(h, W_q, W_dkv, W_kr, H, nope, rope_dim):
    """Planted mistake: q viewed as [H, T, width] straight from h W_q."""
    h = np.asarray(h, np.float64)
    T = h.shape[0]
    q = (h @ W_q).reshape(H, T, nope + rope_dim).transpose(1, 0, 2)
    q_r = orc.rope_adjacent(np.transpose(q[..., nope:], (1, 0, 2))).transpose(1, 0, 2)
    return q[..., :nope], q_r, h @ W_dkv, orc.rope_adjacent(h @ W_kr)


def _project_unrotated_key(h, W_q, W_dkv, W_kr, H, nope, rope_dim):
    """Planted mistake: the shared RoPE key left unrotated."""
    q_n, q_r, c, _ = orc.project(h, W_q, W_dkv, W_kr, H, nope, rope_dim)
    return q_n, q_r, c, np.asarray(h, np.float64) @ W_kr


@pytest.mark.parametrize("mutant", [_project_rope_over_heads, _project_swapped_halves,
                                    _project_token_head_transposed, _project_unrotated_key])
def test_mutation_projection_mistakes_are_caught(mutant):
    with pytest.raises(AssertionError):
        check_project(mutant)


def test_mutation_transposed_output_flatten_is_caught():
    """Planted mistake: the per-head outputs flattened element-major."""
    def forward_transposed(h, W_q, W_dkv, W_kr, W_uk, W_uv, W_o, H, nope, rope_dim):
        q_n, q_r, c, k_r = orc.project(h, W_q, W_dkv, W_kr, H, nope, rope_dim)
        out = orc.expanded_attention(q_n, q_r, c, k_r, W_uk, W_uv, True)
        return out.transpose(0, 2, 1).reshape(out.shape[0], -1) @ W_o
    with pytest.raises(AssertionError):
        check_output_flatten(forward_transposed)


# ---------------------------------------------------------------------------
# RoPE: closed forms of the adjacent-pair rotation.
# ---------------------------------------------------------------------------

def test_rope_closed_forms():
    T, R = 9, 4
    x = np.zeros((T, R))
    x[:, 2] = 1.0  # unit vector on pair 1
    y = orc.rope_adjacent(x)
    t = np.arange(T)
    ang = t / 10000 ** (2 / R)  # pair 1 angle = t / 100
    assert np.allclose(y[:, 2], np.cos(ang), atol=1e-15)
    assert np.allclose(y[:, 3], np.sin(ang), atol=1e-15)
    assert np.allclose(y[:, :2], 0)
    x = np.zeros((T, R))
    x[:, 1] = 1.0  # second slot of pair 0, angle t
    y = orc.rope_adjacent(x)
    assert np.allclose(y[:, 0], -np.sin(t), atol=1e-15)
    assert np.allclose(y[:, 1], np.cos(t), atol=1e-15)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((T, 6))
    y = orc.rope_adjacent(x)
    assert np.allclose(y[0], x[0])  # position 0 is the identity
    assert np.allclose(x[:, 0::2] ** 2 + x[:, 1::2] ** 2, y[:, 0::2] ** 2 + y[:, 1::2] ** 2)
    # Relative position: <rope(a)_t, rope(b)_s> depends on t - s only.
    a = np.tile(rng.standard_normal(6), (T, 1))
    b = np.tile(rng.standard_normal(6), (T, 1))
    ra, rb = orc.rope_adjacent(a), orc.rope_adjacent(b)
    d1 = ra[5] @ rb[2]
    d2 = ra[7] @ rb[4]
    assert abs(d1 - d2) < 1e-12


# ---------------------------------------------------------------------------
# Absorbed decode against brute force and against SDPA.
# ---------------------------------------------------------------------------

def _tiny_case(seed, s_q, lens, H=3, d_qk=20):
    return make_decode_case(lens, s_q=s_q, H=H, seed=seed, dtype=torch.float32,
                            q_scale=0.4, d_qk=d_qk, scale=0.37)


@pytest.mark.parametrize("s_q,lens", [(1, [1, 13]), (2, [2, 70]), (3, [150, 65, 5])])
def test_decode_matches_brute_force(s_q, lens):
    case = _tiny_case(11 + s_q, s_q, lens)
    q, cache, table, L = _case_arrays(case)
    o, lse = orc.decode_absorbed(q, cache, table, L, case.scale, case.causal, dv=12)
    ob, lb = brute_decode(q, cache, table, L, case.scale, case.causal, 12)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(lse - lb)) <= 1e-12


@pytest.mark.parametrize("s_q,causal", [(1, False), (2, True), (4, True), (2, False)])
def test_decode_matches_sdpa_full_width(s_q, causal):
    case = make_decode_case([300, 64, 129, 7 + s_q], s_q=s_q, H=16, seed=5 + s_q,
                            dtype=torch.bfloat16, q_scale=1.0, causal=causal)
    q, cache, table, L = _case_arrays(case)
    o, _ = orc.decode_absorbed(q, cache, table, L, case.scale, case.causal, dv=512)
    ref = sdpa_decode(q, cache, table, L, case.scale, case.causal, 512)
    assert np.max(np.abs(o - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_single_key_returns_its_value_and_score():
    case = make_decode_case([1, 1], s_q=1, H=8, seed=21, dtype=torch.float32, q_scale=1.0)
    q, cache, table, L = _case_arrays(case)
    o, lse = orc.decode_absorbed(q, cache, table, L, case.scale, False, dv=512)
    for b in range(2):
        row = cache[table[b, 0], 0]
        assert np.allclose(o[b, 0], np.broadcast_to(row[:512], (8, 512)), atol=0, rtol=0)
        s = case.scale * (q[b, 0] @ row)
        assert np.allclose(lse[b, 0], s, atol=1e-12)


def test_zero_query_averages_values_and_lse_is_log_count():
    case = make_decode_case([200, 77], s_q=2, H=4, seed=22, dtype=torch.float32)
    q, cache, table, L = _case_arrays(case)
    q = np.zeros_like(q)
    o, lse = orc.decode_absorbed(q, cache, table, L, case.scale, True, dv=512)
    for b in range(2):
        for i in range(2):
            n = L[b] - 2 + i + 1
            rows = np.stack([cache[table[b, j // 64], j % 64, :512] for j in range(n)])
            assert np.allclose(o[b, i], rows.mean(0)[None], atol=1e-13)
            assert np.allclose(lse[b, i], math.log(n), atol=1e-13)


def test_identical_keys_give_that_value():
    case = make_decode_case([90], s_q=1, H=4, seed=23, dtype=torch.float32, q_scale=1.0)
    q, cache, table, L = _case_arrays(case)
    row = cache[table[0, 0], 0].copy()
    cache = cache.copy()
    for j in range(90):
        cache[table[0, j // 64], j % 64] = row
    o, lse = orc.decode_absorbed(q, cache, table, L, case.scale, False, dv=512)
    assert np.allclose(o[0, 0], row[None, :512], atol=1e-13)
    assert np.allclose(lse[0, 0], case.scale * (q[0, 0] @ row) + math.log(90), atol=1e-12)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def _random_chunks(rng, L, n):
    cuts = sorted(set(int(x) for x in rng.integers(1, L, size=n - 1))) if L > 1 else []
    bounds = [0] + cuts + [L]
    return [(bounds[k], bounds[k + 1]) for k in range(len(bounds) - 1)]


def check_split_merge(decode, partials, merge, case, seed):
    q, cache, table, L = _case_arrays(case)
    o, lse = decode(q, cache, table, L, case.scale, case.causal, dv=512)
    rng = np.random.default_rng(seed)
    chunks = [_random_chunks(rng, int(x), 5) for x in L]
    parts = partials(q, cache, table, L, case.scale, case.causal, chunks, dv=512)
    err = 0.0
    for b, (op, lp) in enumerate(parts):
        om, lm = merge(op, lp)
        err = max(err, np.max(np.abs(om - o[b])), np.max(np.abs(lm - lse[b])))
    return err


def test_split_merge_equals_unsplit():
    case = make_decode_case([500, 130, 3], s_q=3, H=8, seed=31, dtype=torch.bfloat16, q_scale=1.0)
    err = check_split_merge(orc.decode_absorbed, orc.decode_partials, orc.lse_merge, case, 0)
    assert err <= 1e-13


def test_merge_of_empty_chunk_contributes_nothing():
    o = np.random.default_rng(1).standard_normal((3, 2, 5))
    lse = np.array([[0.3, -np.inf], [-np.inf, -np.inf], [1.2, 0.5]])
    om, lm = orc.lse_merge(o, lse)
    om2, lm2 = orc.lse_merge(o[[0, 2]], lse[[0, 2]])
    assert np.allclose(om, om2) and np.allclose(lm, lm2)
    assert np.all(np.isfinite(om))


def test_page_permutation_is_bitwise_invariant():
    case = make_decode_case([300, 200], s_q=2, H=8, seed=41, dtype=torch.bfloat16, q_scale=1.0)
    q, cache, table, L = _case_arrays(case)
    perm = np.random.default_rng(3).permutation(cache.shape[0])
    cache2 = np.empty_like(cache)
    cache2[perm] = cache
    table2 = perm[table]
    o1, l1 = orc.decode_absorbed(q, cache, table, L, case.scale, True)
    o2, l2 = orc.decode_absorbed(q, cache2, table2, L, case.scale, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_head_permutation_and_sequence_independence():
    case = make_decode_case([260, 100], s_q=1, H=16, seed=42, dtype=torch.bfloat16, q_scale=1.0)
    q, cache, table, L = _case_arrays(case)
    o1, l1 = orc.decode_absorbed(q, cache, table, L, case.scale, False)
    hp = np.random.default_rng(4).permutation(16)
    o2, l2 = orc.decode_absorbed(q[:, :, hp], cache, table, L, case.scale, False)
    assert np.allclose(o2, o1[:, :, hp], atol=1e-14) and np.allclose(l2, l1[:, :, hp], atol=1e-14)
    q3, cache3 = q.copy(), cache.copy()
    q3[1] = -q3[1]
    cache3[table[1, :2]] *= 3.0
    o3, l3 = orc.decode_absorbed(q3, cache3, table, L, case.scale, False)
    assert np.array_equal(o3[0], o1[0]) and np.array_equal(l3[0], l1[0])
    assert not np.allclose(o3[1], o1[1])


def test_absorb_and_out_uv_agree_with_expansion():
    """q_lat . [c; k_r] equals the expanded per-head score, and o_lat W_UV the
    expanded per-head value mix (the two associativity steps of path two)."""
    rng = np.random.default_rng(9)
    H, NOPE, ROPE, DC, DV, N, T = 3, 5, 4, 11, 6, 4, 7
    q_n, q_r = rng.standard_normal((N, H, NOPE)), rng.standard_normal((N, H, ROPE))
    c, k_r = rng.standard_normal((T, DC)), rng.standard_normal((T, ROPE))
    W_uk, W_uv = rng.standard_normal((H, DC, NOPE)), rng.standard_normal((H, DC, DV))
    ql = orc.absorb_q(q_n, q_r, W_uk)
    s_abs = np.einsum("nhc,tc->nht", ql, np.concatenate([c, k_r], 1))
    kn = np.einsum("tc,hcd->htd", c, W_uk)
    s_exp = np.einsum("nhd,htd->nht", q_n, kn) + np.einsum("nhr,tr->nht", q_r, k_r)
    assert np.max(np.abs(s_abs - s_exp)) <= 1e-12
    p = rng.random((N, H, T))
    o_lat = np.einsum("nht,tc->nhc", p, c)
    v = np.einsum("tc,hcd->htd", c, W_uv)
    assert np.max(np.abs(orc.out_uv(o_lat, W_uv) - np.einsum("nht,htd->nhd", p, v))) <= 1e-12


# ---------------------------------------------------------------------------
# Mutation tests: plausible mistakes planted in the oracle must fail a pin.
# ---------------------------------------------------------------------------

def test_mutation_causal_off_by_one_is_caught(monkeypatch):
    case = _tiny_case(12, 2, [2, 70])
    q, cache, table, L = _case_arrays(case)
    ob, _ = brute_decode(q, cache, table, L, case.scale, True, 12)
    monkeypatch.setattr(orc, "_allowed_count", lambda L, s_q, i, c: L - s_q + i if c else L)
    with np.errstate(all="ignore"):
        try:
            o, _ = orc.decode_absorbed(q, cache, table, L, case.scale, True, dv=12)
        except ValueError:  # an empty row is also a detection
            return
    assert not np.allclose(o, ob, atol=1e-6, equal_nan=False)


def test_mutation_dropped_rope_term_is_caught(monkeypatch):
    w = tiny_mla_weights(0)
    args = (w["h"], w["W_q"], w["W_dkv"], w["W_kr"], w["W_uk"], w["W_uv"], w["W_o"],
            w["H"], w["NOPE"], w["ROPE"])
    real = orc.absorb_q
    monkeypatch.setattr(orc, "absorb_q", lambda qn, qr, W: real(qn, np.zeros_like(qr), W))
    y1 = orc.mla_forward_expanded(*args)
    y2 = orc.mla_forward_absorbed(*args)
    assert np.max(np.abs(y1 - y2)) > 1e-6


def test_mutation_log2_lse_is_caught(monkeypatch):
    class _NpLog2:
        def __getattr__(self, k):
            return getattr(np, k)
        log = staticmethod(np.log2)
    monkeypatch.setattr(orc, "np", _NpLog2())
    case = make_decode_case([200], s_q=1, H=4, seed=22, dtype=torch.float32)
    q, cache, table, L = _case_arrays(case)
    _, lse = orc.decode_absorbed(np.zeros_like(q), cache, table, L, case.scale, False)
    assert not np.allclose(lse, math.log(200), atol=1e-6)


def test_mutation_wrong_value_columns_is_caught():
    """V taken from the last 512 columns instead of the first 512."""
    def decode_wrong_v(q, cache, table, L, scale, causal, dv=512):
        return orc.decode_absorbed(q, cache[..., ::-1].copy(), table, L, scale, causal, dv)
    case = _tiny_case(13, 1, [1, 13])
    q, cache, table, L = _case_arrays(case)
    o, _ = decode_wrong_v(q[..., ::-1].copy(), cache, table, L, case.scale, False, dv=12)
    ob, _ = brute_decode(q, cache, table, L, case.scale, False, 12)
    assert np.max(np.abs(o - ob)) > 1e-3


def test_mutation_unnormalised_merge_is_caught():
    def merge_wrong(o_parts, lse_parts):
        M = lse_parts.max(axis=0)
        w = np.exp(lse_parts - M)
        return np.einsum("k...,k...d->...d", w, o_parts), M + np.log(w.sum(0))
    case = make_decode_case([500, 130], s_q=1, H=4, seed=31, dtype=torch.bfloat16, q_scale=1.0)
    err = check_split_merge(orc.decode_absorbed, orc.decode_partials, merge_wrong, case, 0)
    assert err > 1e-3


# ---------------------------------------------------------------------------
# Sparse (top-k) decode: [AI-MTP] section 6.
# ---------------------------------------------------------------------------

def brute_sparse(q_lat, cache, table, seqlens, indices, scale, dv):
    """Python-float loops over each row's list, skipping entries outside [0, L)."""
    B, s_q, H, D = q_lat.shape
    page = cache.shape[1]
    o = np.zeros((B, s_q, H, dv))
    lse = np.full((B, s_q, H), -math.inf)
    for b in range(B):
        L = int(seqlens[b])
        for i in range(s_q):
            sel = [int(j) for j in indices[b, i] if 0 <= int(j) < L]
            if not sel:
                continue
            rows = [cache[int(table[b][j // page])][j % page] for j in sel]
            for h in range(H):
                scores = [scale * sum(float(q_lat[b, i, h, k]) * float(r[k]) for k in range(D)) for r in rows]
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                Z = sum(w)
                for c in range(dv):
                    o[b, i, h, c] = sum(w[t] * float(rows[t][c]) for t in range(len(rows))) / Z
                lse[b, i, h] = mx + math.log(Z)
    return o, lse


@pytest.mark.parametrize("s_q", [1, 2])
def test_sparse_full_list_equals_dense(s_q):
    # Listing every visible position (any order, -1 padding) gives the dense decode.
    from mla_inputs import topk_indices
    lens = [300, 64, 129, 7 + s_q]
    case = make_decode_case(lens, s_q=s_q, H=16, seed=40 + s_q, dtype=torch.bfloat16, q_scale=1.0)
    q, cache, table, L = _case_arrays(case)
    idx = topk_indices(lens, s_q, 320, seed=3, causal=True).numpy()
    o, lse = orc.decode_sparse(q, cache, table, L, idx, case.scale, dv=512)
    od, ld = orc.decode_absorbed(q, cache, table, L, case.scale, s_q > 1, dv=512)
    assert np.max(np.abs(o - od)) <= 1e-12 and np.max(np.abs(lse - ld)) <= 1e-12


def test_sparse_matches_brute_force():
    from mla_inputs import topk_indices
    lens = [40, 70, 3]
    case = _tiny_case(31, 2, lens)
    q, cache, table, L = _case_arrays(case)
    idx = topk_indices(lens, 2, 9, seed=5, causal=True, repeat_frac=0.2).numpy()
    idx[0, 1, 2] = 500   # out of range: padding
    idx[2, 0, :] = -1    # a row with nothing selected
    o, lse = orc.decode_sparse(q, cache, table, L, idx, case.scale, dv=12)
    ob, lb = brute_sparse(q, cache, table, L, idx, case.scale, 12)
    assert np.max(np.abs(o - ob)) <= 1e-12
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - lb[fin])) <= 1e-12
    assert np.all(o[2, 0] == 0) and np.all(lse[2, 0] == -np.inf)


def test_sparse_duplicate_and_order():
    # A position listed twice: o = its value, lse = its score + ln 2. The list
    # order never matters.
    case = make_decode_case([100], s_q=1, H=4, seed=32, dtype=torch.float32, q_scale=1.0)
    q, cache, table, L = _case_arrays(case)
    idx = np.array([[[37, 37, -1, -1]]])
    o, lse = orc.decode_sparse(q, cache, table, L, idx, case.scale, dv=512)
    row = cache[table[0, 0], 37]
    assert np.allclose(o[0, 0], row[None, :512], atol=1e-13)
    assert np.allclose(lse[0, 0], case.scale * (q[0, 0] @ row) + math.log(2), atol=1e-12)
    idx2 = np.array([[[5, 80, 37, 12, 99]]])
    a = orc.decode_sparse(q, cache, table, L, idx2, case.scale, dv=512)
    b = orc.decode_sparse(q, cache, table, L, idx2[..., ::-1].copy(), case.scale, dv=512)
    assert np.max(np.abs(a[0] - b[0])) <= 1e-13 and np.max(np.abs(a[1] - b[1])) <= 1e-13


def test_mutation_sparse_padding_as_token_zero_is_caught(monkeypatch):
    # Treating the -1 padding as position 0 must fail a pin.
    real = orc.decode_sparse

    def pad_as_zero(q, cache, table, L, idx, scale, dv=512):
        return real(q, cache, table, L, np.where(np.asarray(idx) < 0, 0, idx), scale, dv)
    monkeypatch.setattr(orc, "decode_sparse", pad_as_zero)
    with pytest.raises(AssertionError):
        test_sparse_matches_brute_force()


# ---------------------------------------------------------------------------
# FP8 (e4m3) latent cache.
# ---------------------------------------------------------------------------

def test_e4m3_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_hand_values():
    v = orc.e4m3_decode([0x38, 0xB8, 0x7E, 0x01, 0x08, 0x00, 0x80, 0x3C])
    assert list(v[:5]) == [1.0, -1.0, 448.0, 2.0 ** -9, 2.0 ** -6]
    assert v[5] == 0.0 and np.signbit(v[6]) and v[7] == 1.5


def test_fp8_decode_closed_forms():
    # One key per sequence: o = its dequantised value, lse = its score. All
    # rows' codes equal with scales s_j: a softmax over s_j-scaled copies.
    from mla_inputs import fp8_case
    case = fp8_case([1, 1], s_q=1, H=8, seed=101, q_scale=1.0)
    q = _np(case.q_lat)
    codes = case.meta["cache_fp8"].numpy()
    sc = case.meta["row_scales"].numpy()
    table = case.block_table.numpy()
    o, lse = orc.decode_absorbed_fp8(q, codes, sc, table, case.seqlens.numpy(), case.scale, False)
    for b in range(2):
        p = table[b, 0]
        row = orc.e4m3_decode(codes[p, 0]) * float(sc[p, 0])
        assert np.allclose(o[b, 0], np.broadcast_to(row[:512], (8, 512)), rtol=0, atol=0)
        assert np.allclose(lse[b, 0], case.scale * (q[b, 0] @ row), atol=1e-12)
    # Same codes in every row, scales 1 and 2: o = sum_j w_j s_j r with
    # w = softmax(s_j * score(r)), lse closed form.
    case2 = fp8_case([2], s_q=1, H=4, seed=102, q_scale=1.0)
    q2 = _np(case2.q_lat)
    codes2 = case2.meta["cache_fp8"].numpy().copy()
    sc2 = case2.meta["row_scales"].numpy().copy()
    t2 = case2.block_table.numpy()
    p = t2[0, 0]
    codes2[p, 1] = codes2[p, 0]
    sc2[p, 0], sc2[p, 1] = 1.0, 2.0
    o2, l2 = orc.decode_absorbed_fp8(q2, codes2, sc2, t2, case2.seqlens.numpy(), case2.scale, False)
    r = orc.e4m3_decode(codes2[p, 0])
    s1 = case2.scale * (q2[0, 0] @ r)  # [H]
    w1, w2 = np.exp(s1), np.exp(2 * s1)
    assert np.allclose(l2[0, 0], np.log(w1 + w2), atol=1e-12)
    assert np.allclose(o2[0, 0], ((w1 + 2 * w2) / (w1 + w2))[:, None] * r[None, :512], atol=1e-12)


def test_mutation_e4m3_wrong_bias_is_caught(monkeypatch):
    real = orc.e4m3_decode
    monkeypatch.setattr(orc, "e4m3_decode", lambda c: real(c) * 2.0)  # bias 6 instead of 7
    with pytest.raises(AssertionError):
        test_e4m3_hand_values()


# ---------------------------------------------------------------------------
# Path one on a paged cache (prefill / extend) and the path choice.
# ---------------------------------------------------------------------------

def _prefill_case(seed, lens, s_q, H=4, nope=8, rope=4, dv=6, dc=16):
    rng = np.random.default_rng(seed)
    case = make_decode_case(lens, s_q=s_q, H=H, seed=seed, dtype=torch.float32, d_qk=dc + rope, q_scale=1.0,
                            scale=1.0 / math.sqrt(nope + rope))
    q_n = rng.standard_normal((len(lens), s_q, H, nope))
    q_r = rng.standard_normal((len(lens), s_q, H, rope))
    W_uk = rng.standard_normal((H, dc, nope)) / 4
    W_uv = rng.standard_normal((H, dc, dv)) / 4
    return case, q_n, q_r, W_uk, W_uv


@pytest.mark.parametrize("s_q,lens", [(1, [1, 40]), (3, [3, 70, 129]), (17, [17, 100])])
def test_prefill_expanded_equals_absorbed_path(s_q, lens):
    # Path one (expand, then MHA) and path two (absorb q, latent attention,
    # W_UV after) are the same computation: outputs and LSEs agree to rounding.
    case, q_n, q_r, W_uk, W_uv = _prefill_case(50 + s_q, lens, s_q)
    _, cache, table, L = _case_arrays(case)
    o1, l1 = orc.prefill_expanded(q_n, q_r, cache, table, L, W_uk, W_uv, case.scale)
    q_lat = orc.absorb_q(q_n.reshape(-1, *q_n.shape[2:]), q_r.reshape(-1, *q_r.shape[2:]), W_uk)
    q_lat = q_lat.reshape(len(lens), s_q, *q_lat.shape[1:])
    ol, l2 = orc.decode_absorbed(q_lat, cache, table, L, case.scale, True, dv=W_uk.shape[1])
    o2 = orc.out_uv(ol.reshape(-1, *ol.shape[2:]), W_uv).reshape(o1.shape)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12


@pytest.mark.parametrize("chunk", [1, 16, 64, 1000])
def test_prefill_chunked_equals_unchunked(chunk):
    case, q_n, q_r, W_uk, W_uv = _prefill_case(61, [130, 64, 7], 5)
    _, cache, table, L = _case_arrays(case)
    o1, l1 = orc.prefill_expanded(q_n, q_r, cache, table, L, W_uk, W_uv, case.scale)
    o2, l2 = orc.prefill_chunked(q_n, q_r, cache, table, L, W_uk, W_uv, case.scale, chunk)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12


def test_prefill_expanded_matches_worked_example():
    # The page's tiny model (T = 6 prompt tokens, no prefix): path one on a
    # one-page cache built from its c and k^R equals its expanded attention.
    w = tiny_mla_weights()
    q_n, q_r, c, k_r = orc.project(w["h"], w["W_q"], w["W_dkv"], w["W_kr"], w["H"], w["NOPE"], w["ROPE"])
    T = c.shape[0]
    cache = np.concatenate([c, k_r], axis=1)[None]  # [1 page, T rows, dc + rope]
    o, _ = orc.prefill_expanded(q_n[None], q_r[None], cache, np.zeros((1, 1), dtype=np.int64), [T],
                                w["W_uk"], w["W_uv"], 1.0 / math.sqrt(w["NOPE"] + w["ROPE"]))
    ref = orc.expanded_attention(q_n, q_r, c, k_r, w["W_uk"], w["W_uv"], causal=True)
    assert np.max(np.abs(o[0] - ref)) <= 1e-12


def test_crossover_matches_printed_171():
    g = load_golden("flop_accounting.txt")
    assert round(orc.crossover_tokens(10 ** 9)) == g["crossover_new_tokens"]
    # The cost comparison it stands for: at L = 32768 + 64 the absorbed path
    # wins for 64 new tokens, at 32768 + 512 the expanded one for 512.
    assert 64 < orc.crossover_tokens(32768 + 64) < 512
    g2 = load_golden("crossover.txt")
    assert round(orc.crossover_tokens(512)) == g2["crossover_L512"]
    # At L = 128K the formula gives 170.4; the text rounds the range's upper
    # end to the large-L limit 171 (170.7), so allow one unit there.
    assert abs(orc.crossover_tokens(131072) - g2["crossover_L131072"]) < 1.0


# ---------------------------------------------------------------------------
# FP8 bmm for the absorption: encoder, per-tensor quantiser, fp8 absorb/out_uv
# ---------------------------------------------------------------------------

def _e4m3_finite_values():
    v = orc.e4m3_decode(np.arange(256))
    return v[np.isfinite(v)]


def test_e4m3_encoder_matches_torch_on_every_tie_and_a_sweep():
    # torch's float8_e4m3fn conversion rounds to nearest, ties to even; every
    # midpoint between neighbouring values is a tie, exact in fp32.
    v = np.unique(np.abs(_e4m3_finite_values()))
    mids = (v[1:] + v[:-1]) / 2
    x = np.concatenate([np.linspace(-448.0, 448.0, 100001), mids, -mids, v, -v,
                        np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(x), ref)


def test_e4m3_encoder_round_trip_saturation_and_signed_zero():
    codes = np.arange(256)
    vals = orc.e4m3_decode(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(orc.e4m3_encode(vals[fin]), codes[fin].astype(np.uint8))
    # 2^-10 is half way from 0 to the smallest step 2^-9 (ties to code 0);
    # 3 * 2^-10 half way from 2^-9 to 2^-8 (ties to code 2).
    assert list(orc.e4m3_encode([448.0, 463.9, 1e9, -1e9, -0.0, 0.0, 2.0 ** -10, 3 * 2.0 ** -10])) == \
        [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x02]


def test_quantize_e4m3_scale_and_extremes():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 3, 64)).astype(np.float32)
    x[2, 1, 7] = -9.5  # the largest magnitude
    codes, s = orc.quantize_e4m3(x)
    assert s == np.float32(1.0) / (np.float32(448.0) / np.float32(9.5))
    assert codes[2, 1, 7] == 0xFE and np.max(np.abs(orc.e4m3_decode(codes))) == 448.0
    deq = orc.e4m3_decode(codes) * np.float64(s)
    assert np.max(np.abs(deq - x) / np.maximum(np.abs(x), 2.0 ** -6 * s)) <= 2.0 ** -4  # half an ulp of 3 bits
    zc, zs = orc.quantize_e4m3(np.zeros((4, 4), np.float32))
    assert zs == 1.0 and not zc.any()


def _representable_operands(rng, shape, step):
    # Values on the e4m3 grid times a power of two, with the grid maximum 448
    # present, so that the per-tensor scale is the power of two itself and
    # quantisation is exact.
    vals = _e4m3_finite_values()
    x = rng.choice(vals, size=shape) * step
    x.reshape(-1)[0] = 448.0 * step
    return x.astype(np.float32)


def test_absorb_q_fp8_equals_absorb_q_on_representable_inputs():
    rng = np.random.default_rng(11)
    q_n = _representable_operands(rng, (6, 4, 16), 2.0 ** -9)
    q_r = rng.standard_normal((6, 4, 8))
    w_codes = rng.integers(0, 256, size=(4, 32, 16)).astype(np.uint8)
    w_codes[(w_codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    got = orc.absorb_q_fp8(q_n, q_r, w_codes, 0.125)
    want = orc.absorb_q(q_n.astype(np.float64), q_r, orc.e4m3_decode(w_codes) * 0.125)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert np.array_equal(got[..., 32:], q_r)


def test_out_uv_fp8_equals_out_uv_on_representable_inputs():
    rng = np.random.default_rng(12)
    o = _representable_operands(rng, (5, 3, 32), 2.0 ** -8)
    w_t = rng.integers(0, 256, size=(3, 24, 32)).astype(np.uint8)  # [H, DV, DC]
    w_t[(w_t & 0x7F) == 0x7F] = 0x44
    got = orc.out_uv_fp8(o, w_t, 0.5)
    want = orc.out_uv(o.astype(np.float64), np.swapaxes(orc.e4m3_decode(w_t) * 0.5, 1, 2))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_mutation_e4m3_ties_away_from_zero_is_caught(monkeypatch):
    # A plausible encoder mistake, ties rounded away from zero, fails the torch pin.
    v = np.unique(np.abs(_e4m3_finite_values()))
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    real = orc.e4m3_encode
    monkeypatch.setattr(orc, "e4m3_encode", lambda x: real(np.nextafter(np.asarray(x, np.float64), np.inf)))
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(orc.e4m3_encode(mids), ref)
