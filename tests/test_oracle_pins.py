"""Pins of the CPU oracle against what the pages and mathematics fix.

Pages: [Derivations] = "数学推导" (CacheBlend math derivations page);
[KV-blog] = "rag的kvcache问题".  No page prints a numeric worked example, so
the pins are identities, closed forms, special cases, brute force on tiny
inputs and the two small golden fixtures under tests/golden/.  Each group is
chosen so that a plausible slip in the oracle (a dropped term, a flipped sign,
a wrong index or pairing, a transposed operand) fails at least one test.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import cacheblend_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20240601)


def _randn(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- rotation --
STYLES = [O.ROPE_HALF, O.ROPE_INTERLEAVED]


def _rotation_matrix(head_dim, angle_pos, theta, style):
    """Explicit D x D matrix of R_pos, assembled column by column by rotating
    basis vectors (so a composition check exercises the full linear map)."""
    eye = np.eye(head_dim)[:, None, :]                      # [D, 1, D] rows = basis
    cols = O.rotate(eye, np.full(head_dim, angle_pos), theta, style)[:, 0, :]
    return cols.T                                            # column i = R e_i


@pytest.mark.parametrize("style", STYLES)
def test_rotation_textbook_2d(style):
    # D = 2 is a single block: the 2x2 matrix of [Derivations, "RoPE 位置编码的
    # 相对位置不变性证明"] acting on (x, y), turned by exactly delta radians.
    for delta in [0.3, 1.0, -2.5, 17.0, 40000.0]:
        e0 = O.rotate(np.array([[[1.0, 0.0]]]), [delta], 10000.0, style)[0, 0]
        e1 = O.rotate(np.array([[[0.0, 1.0]]]), [delta], 10000.0, style)[0, 0]
        assert np.allclose(e0, [math.cos(delta), math.sin(delta)], atol=1e-12)
        assert np.allclose(e1, [-math.sin(delta), math.cos(delta)], atol=1e-12)


@pytest.mark.parametrize("style", STYLES)
@pytest.mark.parametrize("head_dim", [4, 16, 128])
def test_rotation_group_law(style, head_dim):
    # R_a^T R_b = R_{b-a} [Derivations, "RoPE 位置编码的相对位置不变性证明"]
    theta = 10000.0
    for a, b in [(3, 11), (65535, 7), (-1200, 4096), (0, 0), (32767, 65535)]:
        ra = _rotation_matrix(head_dim, a, theta, style)
        rb = _rotation_matrix(head_dim, b, theta, style)
        rba = _rotation_matrix(head_dim, b - a, theta, style)
        assert np.max(np.abs(ra.T @ rb - rba)) < 1e-10
        assert np.max(np.abs(ra.T @ ra - np.eye(head_dim))) < 1e-12   # orthogonal
        assert abs(np.linalg.det(ra) - 1.0) < 1e-10                   # no reflection


@pytest.mark.parametrize("style", STYLES)
def test_score_relative_position_invariance(style):
    # (R_m q)^T (R_n k) = q^T R_{n-m} k: depends on n - m only.
    head_dim, theta = 64, 10000.0
    q, k = _randn(1, 1, head_dim), _randn(1, 1, head_dim)
    for m, n, t in [(5, 9, 100), (0, 2047, 30000), (1000, 10, 12345)]:
        s1 = np.sum(O.rotate(q, [m], theta, style) * O.rotate(k, [n], theta, style))
        s2 = np.sum(O.rotate(q, [m + t], theta, style) * O.rotate(k, [n + t], theta, style))
        s3 = np.sum(q * O.rotate(k, [n - m], theta, style))
        assert abs(s1 - s2) <= 1e-10 * max(1.0, abs(s1))
        assert abs(s1 - s3) <= 1e-10 * max(1.0, abs(s1))


@pytest.mark.parametrize("style", STYLES)
def test_rerotation_equals_direct_rotation(style):
    # [Derivations, "CacheBlend 中的应用"]: R_{p_new - p_old} (R_{p_old} k) = R_{p_new} k
    head_dim, theta, t_count = 128, 10000.0, 64
    k_base = _randn(t_count, 8, head_dim)
    p_old = np.arange(t_count) % 16
    p_new = p_old + np.repeat([0, 16, 1024, 65519 - 16], t_count // 4)
    k_old = O.rotate(k_base, p_old, theta, style)
    k_rot = O.rerotate(k_old, p_new - p_old, theta, style)
    k_direct = O.rotate(k_base, p_new, theta, style)
    assert np.max(np.abs(k_rot - k_direct)) < 1e-10


@pytest.mark.parametrize("style", STYLES)
def test_rotation_special_cases(style):
    head_dim, theta = 32, 10000.0
    x = _randn(5, 3, head_dim)
    # delta = 0 leaves every value bit-identical
    assert np.array_equal(O.rerotate(x, np.zeros(5), theta, style), x)
    # R_{-d} R_d = I
    d = np.array([1, 7, 300, 4097, 65535])
    back = O.rotate(O.rotate(x, d, theta, style), -d, theta, style)
    assert np.max(np.abs(back - x)) < 1e-12
    # each block preserves the norm of its pair
    first, second = O.rope_pairs(head_dim, style)
    y = O.rotate(x, d, theta, style)
    assert np.allclose(x[..., first] ** 2 + x[..., second] ** 2,
                       y[..., first] ** 2 + y[..., second] ** 2, atol=1e-12)


@pytest.mark.parametrize("style", STYLES)
def test_pairing_and_frequency_schedule(style):
    # Measure each pair's turning angle with atan2 (independent of how the oracle
    # builds it): pair 0 turns by exactly delta (speed 1), the speeds form a
    # geometric sequence of ratio theta^(-2/D), and one more step past the last
    # pair would reach speed 1/theta.
    head_dim, theta = 16, 10000.0
    first, second = O.rope_pairs(head_dim, style)
    if style == O.ROPE_HALF:
        assert list(first) == list(range(8)) and list(second) == list(range(8, 16))
    else:
        assert list(first) == list(range(0, 16, 2)) and list(second) == list(range(1, 16, 2))
    speeds = []
    for j in range(head_dim // 2):
        x = np.zeros((1, 1, head_dim))
        x[0, 0, first[j]] = 1.0
        y = O.rotate(x, [0.5], theta, style)[0, 0]
        others = np.delete(y, [first[j], second[j]])
        assert np.all(others == 0.0)                 # a block moves only its own pair
        speeds.append(math.atan2(y[second[j]], y[first[j]]) / 0.5)
    speeds = np.array(speeds)
    assert abs(speeds[0] - 1.0) < 1e-12
    ratios = speeds[1:] / speeds[:-1]
    assert np.allclose(ratios, theta ** (-2.0 / head_dim), rtol=1e-10)
    assert abs(speeds[-1] * theta ** (-2.0 / head_dim) * theta - 1.0) < 1e-10


# --------------------------------------------------------------- deviation --
def test_deviation_special_cases():
    v_old = _randn(10, 4, 8)
    cand = np.array([7, 2, 5, 9])
    # identical rows give exactly zero
    assert np.array_equal(O.deviation(v_old[cand].copy(), v_old, cand), np.zeros(4))
    # one changed element in the last head's last dim gives exactly diff^2, and
    # only for that candidate (the candidate index maps to V_old[cand[j]])
    v_new = v_old[cand].copy()
    v_new[2, 3, 7] += 0.75
    dev = O.deviation(v_new, v_old, cand)
    assert dev[2] == pytest.approx(0.75 ** 2, rel=1e-12)
    assert np.all(dev[[0, 1, 3]] == 0.0)
    # scaling the perturbation by c scales the deviation by c^2
    eps = _randn(4, 4, 8)
    d1 = O.deviation(v_old[cand] + eps, v_old, cand)
    d3 = O.deviation(v_old[cand] + 3.0 * eps, v_old, cand)
    assert np.allclose(d3, 9.0 * d1, rtol=1e-12)
    # every head and dim contributes: the deviation equals the squared
    # Frobenius norm of the per-token difference (numpy.linalg.norm)
    assert np.allclose(d1, np.linalg.norm(eps.reshape(4, -1), axis=1) ** 2, rtol=1e-12)


@pytest.mark.parametrize("style", STYLES)
def test_key_deviation_compares_at_the_new_position(style):
    # [KV-blog, "核心发现： KV 偏差"]: the deviation of a token's KV compares
    # the cached vector with the recomputed one.  Keys are compared after
    # re-rotation: a key whose content did not change scores exactly zero up
    # to rounding, although it differs from the cached key at its old position.
    theta, hkv, head_dim = 10000.0, 2, 32
    chunk_lens = [16, 16, 32]
    t = sum(chunk_lens)
    p_old = np.concatenate([np.arange(n) for n in chunk_lens])
    p_new = np.arange(t)
    k_base, v_old = _randn(t, hkv, head_dim), _randn(t, hkv, head_dim)
    k_old = O.rotate(k_base, p_old, theta, style)
    k_new = O.rotate(k_base, p_new, theta, style)
    cand = np.arange(t)
    out = O.blend_layer(k_old=k_old, v_old=v_old, delta=p_new - p_old, k_new_c=k_new,
                        v_new_c=v_old.copy(), q_c=_randn(t, hkv, head_dim), cand_idx=cand,
                        tok_off=[0, t], cand_off=[0, t], sel_counts=[4], n_q_heads=hkv,
                        n_kv_heads=hkv, theta=theta, style=style, attend=False, dev_source="k")
    assert np.max(out["dev"]) < 1e-20
    unrotated = O.kv_deviation("k", k_new_c=k_new, k_cached=k_old, cand_idx=cand)
    assert np.all(unrotated[16:] > 1e-3) and np.max(unrotated[:16]) < 1e-20   # chunk 0: delta 0
    # Comparing at the new position equals comparing at the old one (rotations
    # keep distances): ||K_new - R_d K_old||^2 = ||R_{-d} K_new - K_old||^2.
    k_other = _randn(t, hkv, head_dim)
    d = p_new - p_old
    at_new = O.kv_deviation("k", k_new_c=k_other, k_cached=O.rerotate(k_old, d, theta, style),
                            cand_idx=cand)
    at_old = O.kv_deviation("k", k_new_c=O.rotate(k_other, -d, theta, style), k_cached=k_old,
                            cand_idx=cand)
    assert np.allclose(at_new, at_old, rtol=1e-12)


def test_kv_deviation_reads_the_kv_row_as_one_vector():
    k_cached, v_old = _randn(12, 3, 8), _randn(12, 3, 8)
    cand = np.array([11, 0, 6, 3, 8])
    k_new, v_new = k_cached[cand].copy(), v_old[cand].copy()
    # one changed K element and one changed V element, in different candidates
    k_new[1, 2, 5] += 1.5
    v_new[3, 0, 0] -= 0.25
    args = dict(k_new_c=k_new, k_cached=k_cached, v_new_c=v_new, v_old=v_old, cand_idx=cand)
    dk, dv, dkv = (O.kv_deviation(s, **args) for s in ("k", "v", "kv"))
    assert dv[3] == pytest.approx(0.0625, rel=1e-12) and np.all(np.delete(dv, 3) == 0.0)
    assert dk[1] == pytest.approx(2.25, rel=1e-12) and np.all(np.delete(dk, 1) == 0.0)
    assert np.array_equal(dkv, dk + dv)
    # random rows: "kv" is the squared norm of the concatenated difference,
    # "v" is the V-only score used elsewhere
    k_new, v_new = _randn(5, 3, 8), _randn(5, 3, 8)
    args.update(k_new_c=k_new, v_new_c=v_new)
    joint = np.concatenate([(k_new - k_cached[cand]).reshape(5, -1),
                            (v_new - v_old[cand]).reshape(5, -1)], axis=1)
    assert np.allclose(O.kv_deviation("kv", **args), np.linalg.norm(joint, axis=1) ** 2, rtol=1e-12)
    assert np.array_equal(O.kv_deviation("v", **args), O.deviation(v_new, v_old, cand))
    with pytest.raises(ValueError):
        O.kv_deviation("q", **args)


def test_store_as_rounds_to_nearest_even():
    import torch
    # hand cases around 1: bf16 steps by 2^-7 there
    one = 1.0
    cases = {one + 2 ** -8: one,                      # tie, 1.0 is even
             one + 3 * 2 ** -8: one + 2 ** -6,        # tie, 1 + 2^-6 is even
             one + 2 ** -8 + 2 ** -20: one + 2 ** -7,  # just above the tie
             -(one + 2 ** -8 - 2 ** -30): -one,        # just below the tie
             0.0: 0.0, 3.0: 3.0, -0.15625: -0.15625}
    for x, want in cases.items():
        assert O.store_as(np.array([x]), "bf16")[0] == want, x
    # float32 inputs: torch's fp32 -> bf16 conversion rounds to nearest even
    rng = np.random.default_rng(3)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-8, 8, 20000))).astype(np.float32)
    bits = x32.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)[:2000]        # exact halfway values
    x32 = np.concatenate([x32, ties])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.store_as(x32.astype(np.float64), "bf16"), ref)
    assert np.array_equal(O.store_as(x32.astype(np.float64), "f32"), x32.astype(np.float64))


# ------------------------------------------------------------------- top-k --
def _brute_force_topk(dev, cand, k):
    best, best_tuple = None, None
    for subset in itertools.combinations(range(len(dev)), k):
        total = sum(dev[i] for i in subset)
        key = tuple(sorted(cand[i] for i in subset))
        if best is None or total > best or (total == best and key < best_tuple):
            best, best_tuple = total, key
    return np.array(best_tuple, dtype=np.int64)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(7)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(0, n + 1))
        dev = rng.integers(0, 4, size=n).astype(np.float64)     # many exact ties
        cand = np.sort(rng.choice(100, size=n, replace=False))
        loc, glob = O.topk_select(dev, cand, k)
        assert list(glob) == list(_brute_force_topk(dev, cand, k))
        assert list(glob) == list(cand[loc])
        assert list(loc) == sorted(loc)


def test_topk_rank_rule_and_lexsort():
    rng = np.random.default_rng(11)
    dev = rng.integers(0, 50, size=500).astype(np.float64)
    cand = np.sort(rng.choice(10 ** 6, size=500, replace=False))
    k = 123
    _, glob = O.topk_select(dev, cand, k)
    # rank rule: i is selected iff fewer than k candidates beat it
    beats = (dev[None, :] > dev[:, None]) | ((dev[None, :] == dev[:, None]) & (cand[None, :] < cand[:, None]))
    ranked = np.sort(cand[np.sum(beats, axis=1) < k])
    assert list(glob) == list(ranked)


def test_topk_nan_first_and_planted_recovery():
    dev = np.array([1.0, np.nan, 5.0, np.inf, 5.0, 0.0])
    cand = np.arange(6) * 10
    _, glob = O.topk_select(dev, cand, 3)
    assert list(glob) == [10, 20, 30]          # NaN, +inf, then the lower-index 5.0
    # planted: |H| tokens with a large gap are exactly recovered
    rng = np.random.default_rng(3)
    dev = rng.uniform(0.0, 1.0, 1000)
    hot = rng.choice(1000, 150, replace=False)
    dev[hot] += 10.0
    _, glob = O.topk_select(dev, np.arange(1000), 150)
    assert list(glob) == sorted(hot)


# -------------------------------------------------------------------- fuse --
def test_fuse_rows():
    k_rot, v_old = _randn(12, 2, 4), _randn(12, 2, 4)
    k_new, v_new = _randn(5, 2, 4), _randn(5, 2, 4)
    loc, glob = np.array([0, 3, 4]), np.array([2, 7, 11])
    kf, vf = O.fuse(k_rot, v_old, k_new, v_new, loc, glob)
    others = np.setdiff1d(np.arange(12), glob)
    assert np.array_equal(kf[others], k_rot[others]) and np.array_equal(vf[others], v_old[others])
    assert np.array_equal(kf[glob], k_new[loc]) and np.array_equal(vf[glob], v_new[loc])
    assert not np.shares_memory(kf, k_rot)


# --------------------------------------------------------------- attention --
def _full_matrix_attention(q, k, v, scale):
    """Brute force: whole causal score matrix, strict upper triangle -inf."""
    n = q.shape[0]
    scores = (q @ k.T) * scale
    scores[np.triu(np.ones((n, n), bool), 1)] = -np.inf
    return softmax(scores, axis=1) @ v


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (8, 2), (4, 4)])
def test_attention_vs_full_causal_matrix(hq, hkv):
    t_count, head_dim = 40, 16
    q, k, v = _randn(t_count, hq, head_dim), _randn(t_count, hkv, head_dim), _randn(t_count, hkv, head_dim)
    sel = np.array([0, 3, 17, 39])
    scale = 1.0 / math.sqrt(head_dim)
    out = O.attention_rows(q, sel, sel, np.zeros(4, np.int64), k, v, hq, hkv, scale)
    for h in range(hq):
        g = h * hkv // hq
        ref = _full_matrix_attention(q[:, h], k[:, g], v[:, g], scale)
        assert np.max(np.abs(out[:, h] - ref[sel])) < 1e-12


def test_attention_special_cases():
    head_dim, scale = 8, 1 / math.sqrt(8)
    k, v = _randn(10, 1, head_dim), _randn(10, 1, head_dim)
    q = _randn(10, 1, head_dim)
    # position-0 row sees only itself
    out = O.attention_rows(q, [0], [0], [0], k, v, 1, 1, scale)
    assert np.allclose(out[0, 0], v[0, 0], atol=1e-15)
    # identical keys: uniform weights, the running mean of V
    k_same = np.repeat(k[:1], 10, axis=0)
    out = O.attention_rows(q, [6], [6], [0], k_same, v, 1, 1, scale)
    assert np.allclose(out[0, 0], v[:7, 0].mean(axis=0), atol=1e-12)
    # one dominant key takes all the weight
    k_dom = k.copy()
    k_dom[4, 0] = 200.0 * q[9, 0] / np.linalg.norm(q[9, 0])
    out = O.attention_rows(q, [9], [9], [0], k_dom, v, 1, 1, 1.0)
    assert np.allclose(out[0, 0], v[4, 0], atol=1e-12)
    # keys before the request's first row are invisible
    k_prev = k.copy()
    k_prev[:5] = 1e3
    out_a = O.attention_rows(q, [8], [8], [5], k_prev, v, 1, 1, scale)
    out_b = O.attention_rows(q[5:], [3], [3], [0], k[5:], v[5:], 1, 1, scale)
    assert np.allclose(out_a, out_b, atol=1e-12)


def test_attention_gqa_head_mapping():
    # V of kv head g is the constant g, so any convex combination returns g.
    hq, hkv, head_dim = 8, 2, 4
    q, k = _randn(6, hq, head_dim), _randn(6, hkv, head_dim)
    v = np.zeros((6, hkv, head_dim))
    v[:, 1, :] = 1.0
    out = O.attention_rows(q, [5], [5], [0], k, v, hq, hkv, 0.5)
    assert np.allclose(out[0, :, 0], [0, 0, 0, 0, 1, 1, 1, 1], atol=1e-12)


def test_attention_shift_invariance_with_rope():
    # Rotating Q and K at positions shifted by a constant leaves the output
    # unchanged ([Derivations, "RoPE 位置编码的相对位置不变性证明"]).
    t_count, head_dim, theta = 32, 16, 10000.0
    q, k, v = _randn(t_count, 2, head_dim), _randn(t_count, 1, head_dim), _randn(t_count, 1, head_dim)
    pos = np.arange(t_count)
    sel = np.array([4, 20, 31])
    outs = []
    for shift in [0, 777, 50000]:
        qr = O.rotate(q, pos + shift, theta)
        kr = O.rotate(k, pos + shift, theta)
        outs.append(O.attention_rows(qr, sel, sel, np.zeros(3, np.int64), kr, v, 2, 1, 0.25))
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-10
    assert np.max(np.abs(outs[0] - outs[2])) < 1e-10


def test_golden_causal_visibility_abcd():
    gold = json.load(open(os.path.join(GOLDEN, "causal_mask_abcd.json")))
    visible = np.array(gold["visible"])
    n, head_dim = 4, 8
    q, k, v = _randn(n, 1, head_dim), _randn(n, 1, head_dim), _randn(n, 1, head_dim)
    base = O.attention_rows(q, np.arange(n), np.arange(n), np.zeros(n, np.int64), k, v, 1, 1, 0.3)
    for j in range(n):                      # perturb key/value j
        k2, v2 = k.copy(), v.copy()
        k2[j] += 1.0
        v2[j] += 1.0
        out = O.attention_rows(q, np.arange(n), np.arange(n), np.zeros(n, np.int64), k2, v2, 1, 1, 0.3)
        changed = np.any(np.abs(out - base) > 1e-12, axis=(1, 2))
        assert list(changed.astype(int)) == list(visible[:, j])
    # Without position encoding D sees a bag: permuting A, B, C changes nothing.
    # With RoPE it does, and D's score against C depends only on distance 1.
    perm = np.array([2, 1, 0, 3])
    out_plain = O.attention_rows(q[perm], [3], [3], [0], k[perm], v[perm], 1, 1, 0.3)
    assert np.allclose(out_plain, base[3:4], atol=1e-12)
    theta, pos = 10000.0, np.arange(n)
    qr, kr = O.rotate(q, pos, theta), O.rotate(k, pos, theta)
    out_rope = O.attention_rows(qr, [3], [3], [0], kr, v, 1, 1, 0.3)
    out_rope_perm = O.attention_rows(O.rotate(q[perm], pos, theta), [3], [3], [0],
                                     O.rotate(k[perm], pos, theta), v[perm], 1, 1, 0.3)
    assert np.max(np.abs(out_rope - out_rope_perm)) > 1e-6
    # query at m = 3, key at n = 2: the score is q^T R_{n-m} k with n - m = -distance
    d = gold["distance_from_last"]["C"]
    score_dc = np.sum(qr[3] * kr[2])
    assert abs(score_dc - np.sum(q[3] * O.rotate(k[2:3], [-d], theta)[0])) < 1e-12


def test_golden_causal_pair_count():
    gold = json.load(open(os.path.join(GOLDEN, "causal_mask_count_1024.json")))
    n = gold["n_tokens"]
    # every row of a fully selected 1024-token request, counted through the
    # oracle's own key range: the visible pairs of the causal matrix
    visible = 0
    for s in range(n):
        lo, hi = 0, s + 1
        visible += hi - lo
    assert visible == gold["visible_pairs"]
    assert n * n - visible == gold["masked_pairs"]
    # the oracle's attention agrees with a score matrix of exactly that mask
    q, k, v = _randn(n, 1, 4), _randn(n, 1, 4), _randn(n, 1, 4)
    sel = np.array([0, 511, 1023])
    out = O.attention_rows(q, sel, sel, np.zeros(3, np.int64), k, v, 1, 1, 0.5)
    ref = _full_matrix_attention(q[:, 0], k[:, 0], v[:, 0], 0.5)
    assert np.max(np.abs(out[:, 0] - ref[sel])) < 1e-12


# ---------------------------------------------------- schedule + end to end --
def test_select_count_integer_rounding():
    assert O.select_count(15, 100) == 15          # 0.15 * 100 in floats ceils to 16
    assert O.select_count(15, 2048) == 308
    assert O.select_count(30, 6144) == 1844 and O.select_count(15, 6144) == 922
    assert O.select_count(20, 32768) == 6554 and O.select_count(10, 32768) == 3277
    assert O.select_count(15, 128) == 20
    assert O.layer_plan(1, 6144, 30, 15) == (30, 1844)
    assert O.layer_plan(7, 6144, 30, 15) == (15, 922)


def test_pool_and_chain_agree_through_layer_two():
    s1, s2 = np.array([1, 4, 9]), np.array([4, 9])
    for sched in ["pool", "chain"]:
        assert list(O.candidates_for_layer(1, 12, None, None, sched)) == list(range(12))
        assert list(O.candidates_for_layer(2, 12, s1, s1, sched)) == [1, 4, 9]
    assert list(O.candidates_for_layer(3, 12, s1, s2, "pool")) == [1, 4, 9]
    assert list(O.candidates_for_layer(3, 12, s1, s2, "chain")) == [4, 9]


@pytest.mark.parametrize("style", STYLES)
def test_objective_zero_when_selection_covers_deviated_tokens(style):
    # [Derivations, "形式化"]: when S contains every token whose KV changed, the
    # fused cache equals the fully recomputed one and the objective is 0.
    rng = np.random.default_rng(5)
    theta, hq, hkv, head_dim = 10000.0, 4, 2, 16
    chunks = [24, 40, 32]
    t_count = sum(chunks)
    starts = np.concatenate([[0], np.cumsum(chunks)[:-1]])
    p_new = np.arange(t_count)
    p_old = p_new - np.repeat(starts, chunks)
    k_base, v_base, q_base = (rng.standard_normal((t_count, hkv, head_dim)),
                              rng.standard_normal((t_count, hkv, head_dim)),
                              rng.standard_normal((t_count, hq, head_dim)))
    hot = np.sort(rng.choice(t_count, 15, replace=False))
    k_full, v_full = k_base.copy(), v_base.copy()
    k_full[hot] += rng.standard_normal((15, hkv, head_dim))
    v_full[hot] += rng.standard_normal((15, hkv, head_dim))
    k_old = O.rotate(k_base, p_old, theta, style)                 # chunk-local cache
    k_new = O.rotate(k_full, p_new, theta, style)                 # joint prefill
    q = O.rotate(q_base, p_new, theta, style)
    cand = np.arange(t_count)
    res = O.blend_layer(k_old=k_old, v_old=v_base, delta=p_new - p_old, k_new_c=k_new,
                        v_new_c=v_full, q_c=q, cand_idx=cand, tok_off=[0, t_count],
                        cand_off=[0, t_count], sel_counts=[15], n_q_heads=hq,
                        n_kv_heads=hkv, theta=theta, style=style)
    assert list(res["sel_global"]) == list(hot)
    assert np.max(np.abs(res["k_fused"] - k_new)) < 1e-10
    assert np.array_equal(res["v_fused"], v_full)
    ref = O.attention_rows(q, hot, hot, np.zeros(15, np.int64), k_new, v_full, hq, hkv,
                           1 / math.sqrt(head_dim))
    assert np.max(np.abs(res["out"] - ref)) < 1e-10


def test_blend_layer_ragged_requests_are_independent():
    rng = np.random.default_rng(9)
    hq, hkv, head_dim = 2, 1, 8
    lens = [10, 7]
    t_count = sum(lens)
    k_old, v_old = rng.standard_normal((t_count, hkv, head_dim)), rng.standard_normal((t_count, hkv, head_dim))
    v_new = v_old + rng.standard_normal((t_count, hkv, head_dim))
    k_new, q = rng.standard_normal((t_count, hkv, head_dim)), rng.standard_normal((t_count, hq, head_dim))
    args = dict(delta=np.zeros(t_count), n_q_heads=hq, n_kv_heads=hkv, theta=10000.0)
    both = O.blend_layer(k_old=k_old, v_old=v_old, k_new_c=k_new, v_new_c=v_new, q_c=q,
                         cand_idx=np.arange(t_count), tok_off=[0, 10, 17], cand_off=[0, 10, 17],
                         sel_counts=[3, 2], **args)
    args["delta"] = np.zeros(7)
    second = O.blend_layer(k_old=k_old[10:], v_old=v_old[10:], k_new_c=k_new[10:], v_new_c=v_new[10:],
                           q_c=q[10:], cand_idx=np.arange(7), tok_off=[0, 7], cand_off=[0, 7],
                           sel_counts=[2], **args)
    assert list(both["sel_global"][3:] - 10) == list(second["sel_global"])
    assert np.max(np.abs(both["out"][3:] - second["out"])) < 1e-12


# ------------------------------------------------- the selection objective --
def test_deviation_selection_beats_random_on_the_fusion_objective():
    """[Derivations, "近似解"]: choosing the tokens with the largest V deviation
    makes the fused cache's attention close to the full recompute's.  Built
    here on data whose cached keys are the new keys at old positions (so
    re-rotation restores them up to small noise) and whose values deviate
    strongly on 15% of the tokens: the deviation top-k must give a smaller
    attention error than every one of 20 random selections of the same size,
    and re-rotation must beat leaving the cached keys unrotated."""
    rng = np.random.default_rng(7)
    theta, hq, hkv, d = 10000.0, 4, 2, 16
    chunk, n_chunks = 64, 3
    t = chunk * n_chunks
    p_old = np.tile(np.arange(chunk), n_chunks)
    p_new = np.arange(t)
    k_base = rng.standard_normal((t, hkv, d))
    v_old = rng.standard_normal((t, hkv, d))
    k_old = O.rotate(k_base, p_old, theta)
    k_new = O.rotate(k_base + 0.01 * rng.standard_normal((t, hkv, d)), p_new, theta)
    hot = rng.choice(t, int(0.15 * t), replace=False)
    sigma = np.full(t, 0.01)
    sigma[hot] = 1.0
    v_new = v_old + sigma[:, None, None] * rng.standard_normal((t, hkv, d))
    q = O.rotate(rng.standard_normal((t, hq, d)), p_new, theta)
    everyone = np.arange(t)
    start = np.zeros(t, dtype=np.int64)
    scale = 1.0 / math.sqrt(d)

    def attend(k_f, v_f):
        return O.attention_rows(q, everyone, everyone, start, k_f, v_f, hq, hkv, scale)

    full = attend(k_new, v_new)
    k_rot = O.rerotate(k_old, p_new - p_old, theta)
    k = len(hot)

    def err(sel, keys=k_rot):
        sel = np.sort(sel)
        k_f, v_f = O.fuse(keys, v_old, k_new, v_new, sel, sel)
        return np.linalg.norm(attend(k_f, v_f) - full)

    dev = O.deviation(v_new, v_old, everyone)
    sel_local, sel_global = O.topk_select(dev, everyone, k)
    assert set(sel_global) == set(hot)
    e_top = err(sel_global)
    e_rand = [err(rng.choice(t, k, replace=False)) for _ in range(20)]
    assert e_top < 0.5 * min(e_rand), (e_top, min(e_rand))
    assert e_top < 0.5 * err(sel_global, keys=k_old)       # re-rotation matters
