"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against what the pages or the mathematics fix:
a 50-digit decimal brute force, closed forms, a hand-worked example, invariants,
and the byte counts the pages print.  A plausible slip in the oracle (a dropped
scale, a wrong index or stride, a transposed operand, a sign, a missing
normalisation) fails at least one of them; tests/test_oracle_mutants.py shows it.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture
def api():
    return oracle.api()


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, err


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("case", [
    # B, Nq, Nkv, H, D, value scale, seed
    (1, 1, 1, 1, 1, 1.0, 11),
    (1, 3, 5, 2, 4, 1.0, 12),
    (2, 4, 7, 2, 8, 1.0, 13),
    (1, 16, 16, 1, 8, 2.0, 14),
    (1, 5, 16, 2, 3, 0.5, 15),
    (2, 2, 9, 1, 6, 8.0, 16),      # large logits: naive exp of the raw score overflows fp64
])
def test_attention_matches_decimal_brute_force(api, case):
    B, Nq, Nkv, H, D, sc, seed = case
    g = _rng(seed)
    q = g.standard_normal((B, Nq, H, D)) * sc
    k = g.standard_normal((B, Nkv, H, D)) * sc
    v = g.standard_normal((B, Nkv, H, D))
    o, lse = api.attn(q, k, v)
    bo, bl = brute.attn(q.tolist(), k.tolist(), v.tolist())
    bo = np.array([[[[float(x) for x in bo[b][i][h]] for h in range(H)] for i in range(Nq)] for b in range(B)])
    bl = np.array([[[float(bl[b][h][i]) for i in range(Nq)] for h in range(H)] for b in range(B)])
    _close(o, bo, 1e-13)
    _close(lse, bl, 1e-13)


def test_attention_hand_picked_values_vs_brute(api):
    # keys with huge and tiny logits, ties, and a negative scale-free direction
    q = np.array([[[[3.0, -1.0]], [[0.0, 0.0]], [[-40.0, 25.0]]]])           # [1,3,1,2]
    k = np.array([[[[1.0, 2.0]], [[1.0, 2.0]], [[-30.0, 7.5]], [[0.5, -0.25]]]])  # [1,4,1,2]
    v = np.array([[[[1.0, -2.0]], [[3.0, 5.0]], [[-7.0, 0.125]], [[1e3, -1e-3]]]])
    o, lse = api.attn(q, k, v)
    bo, bl = brute.attn(q.tolist(), k.tolist(), v.tolist())
    for i in range(3):
        _close(o[0, i, 0], [float(x) for x in bo[0][i][0]], 1e-13)
        _close(lse[0, 0, i], float(bl[0][0][i]), 1e-13)


def test_worked_two_key_example(api):
    with open(os.path.join(GOLDEN, "two_key_worked_example.json")) as f:
        ex = json.load(f)
    ln3 = math.log(3.0)
    q = np.array(ex["q"]).reshape(1, 1, 1, 4)
    k = np.array([[ln3 if x == "ln3" else x for x in row] for row in ex["k"]]).reshape(1, 2, 1, 4)
    v = np.array(ex["v"]).reshape(1, 2, 1, 4)
    o, lse = api.attn(q, k, v)
    assert np.max(np.abs(o[0, 0, 0] - np.array(ex["expect_o"]))) <= ex["tol"] * 10
    assert abs(lse[0, 0, 0] - math.log(4.0)) <= ex["tol"]


# ---------------------------------------------------------------- closed forms

def test_single_key_gives_v_exactly(api):
    g = _rng(21)
    B, Nq, H, D = 2, 7, 3, 16
    q = g.standard_normal((B, Nq, H, D))
    k = g.standard_normal((B, 1, H, D))
    v = g.standard_normal((B, 1, H, D))
    o, lse = api.attn(q, k, v)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                exact = math.fsum(q[b, i, h] * k[b, 0, h]) / math.sqrt(D)
                assert abs(lse[b, h, i] - exact) <= 1e-13 * max(1.0, abs(exact))


def test_identical_keys_give_mean_v(api):
    g = _rng(22)
    B, Nq, Nkv, H, D = 1, 5, 37, 2, 8
    q = g.standard_normal((B, Nq, H, D))
    k1 = g.standard_normal((B, 1, H, D))
    k = np.repeat(k1, Nkv, axis=1)
    v = g.standard_normal((B, Nkv, H, D))
    o, lse = api.attn(q, k, v)
    mean_v = v.mean(axis=1, keepdims=True)
    _close(o, np.broadcast_to(mean_v, o.shape), 1e-14)
    for h in range(H):
        for i in range(Nq):
            exact = math.fsum(q[0, i, h] * k1[0, 0, h]) / math.sqrt(D) + math.log(Nkv)
            assert abs(lse[0, h, i] - exact) <= 1e-13


def test_zero_query_gives_mean_v_and_ln_n(api):
    g = _rng(23)
    B, Nq, Nkv, H, D = 2, 3, 50, 2, 4
    q = np.zeros((B, Nq, H, D))
    k = g.standard_normal((B, Nkv, H, D)) * 5
    v = g.standard_normal((B, Nkv, H, D))
    o, lse = api.attn(q, k, v)
    _close(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), 1e-14)
    assert np.max(np.abs(lse - math.log(Nkv))) <= 1e-14


def test_one_dominant_key_gives_its_v_exactly(api):
    """Hard-attention limit: a key whose logit exceeds every other one by more than 745
    (below which exp underflows to zero in fp64) takes the whole softmax weight, so
    O is that key's V exactly and LSE its logit; a naive exp of the raw logits (about 1000)
    would overflow.  The dominant key sits first, inside, and last along the keys."""
    g = _rng(25)
    B, Nq, Nkv, H, D = 2, 4, 9, 3, 8
    q = g.standard_normal((B, Nq, H, D))
    k = g.standard_normal((B, Nkv, H, D))
    v = g.standard_normal((B, Nkv, H, D))
    q[..., 0] = 40.0
    k[..., 0] = 0.0
    jstar = np.array([[0, 4, 8], [8, 1, 0]])
    for b in range(B):
        for h in range(H):
            k[b, jstar[b, h], h, 0] = 80.0   # logit gap >= (3200 - 20) / sqrt(8) > 1100
    o, lse = api.attn(q, k, v)
    for b in range(B):
        for h in range(H):
            j = jstar[b, h]
            assert np.array_equal(o[b, :, h], np.broadcast_to(v[b, j, h], (Nq, D)))
            for i in range(Nq):
                exact = math.fsum(q[b, i, h] * k[b, j, h]) / math.sqrt(D)
                assert abs(lse[b, h, i] - exact) <= 1e-13 * abs(exact)


def test_explicit_scale_argument(api):
    g = _rng(24)
    q = g.standard_normal((1, 4, 1, 8))
    k = g.standard_normal((1, 6, 1, 8))
    v = g.standard_normal((1, 6, 1, 8))
    o1, l1 = api.attn(q, k, v, scale=0.3)
    o2, l2 = api.attn(q * 0.3 * math.sqrt(8), k, v)
    _close(o1, o2, 1e-13)
    _close(l1, l2, 1e-13)


# ---------------------------------------------------------------- invariants

def test_ring_equivalence_merge_of_chunks_equals_full(api):
    """Ring rounds: attention over disjoint key chunks, merged by LSE, is full attention."""
    g = _rng(31)
    B, Nq, Nkv, H, D = 2, 9, 40, 3, 8
    q = g.standard_normal((B, Nq, H, D)) * 2
    k = g.standard_normal((B, Nkv, H, D)) * 2
    v = g.standard_normal((B, Nkv, H, D))
    o_ref, l_ref = api.attn(q, k, v)
    for bounds in ([0, 10, 20, 30, 40], [0, 1, 17, 40], [0, 39, 40]):
        parts = [api.attn(q, k[:, a:b], v[:, a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        o_p = np.stack([p[0] for p in parts])
        l_p = np.stack([p[1] for p in parts])
        o, l = api.merge(o_p, l_p)
        assert np.max(np.abs(o - o_ref)) <= 1e-12
        assert np.max(np.abs(l - l_ref)) <= 1e-12


def test_v_shift_and_kv_row_permutation(api):
    g = _rng(32)
    B, Nq, Nkv, H, D = 1, 6, 20, 2, 8
    q = g.standard_normal((B, Nq, H, D))
    k = g.standard_normal((B, Nkv, H, D))
    v = g.standard_normal((B, Nkv, H, D))
    o, l = api.attn(q, k, v)
    c = g.standard_normal(D)
    o2, l2 = api.attn(q, k, v + c)
    _close(o2, o + c, 1e-13)
    _close(l2, l, 1e-15)
    perm = g.permutation(Nkv)
    o3, l3 = api.attn(q, k[:, perm], v[:, perm])
    _close(o3, o, 1e-13)
    _close(l3, l, 1e-13)
    qp = g.permutation(Nq)
    o4, l4 = api.attn(q[:, qp], k, v)
    _close(o4, o[:, qp], 0.0)
    _close(l4, l[:, :, qp], 0.0)


def test_head_and_batch_independence(api):
    g = _rng(33)
    B, Nq, Nkv, H, D = 2, 5, 11, 3, 4
    q = g.standard_normal((B, Nq, H, D))
    k = g.standard_normal((B, Nkv, H, D))
    v = g.standard_normal((B, Nkv, H, D))
    o, l = api.attn(q, k, v)
    for b in range(B):
        for h in range(H):
            oh, lh = api.attn(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1])
            assert np.array_equal(oh[0, :, 0], o[b, :, h])
            assert np.array_equal(lh[0, 0], l[b, h])


def test_attn_rows_equals_full_rows(api):
    g = _rng(34)
    B, Nq, Nkv, H, D = 2, 13, 21, 3, 8
    q = g.standard_normal((B, Nq, H, D))
    k = g.standard_normal((B, Nkv, H, D))
    v = g.standard_normal((B, Nkv, H, D))
    o, l = api.attn(q, k, v)
    rows = np.array([[0, 0, 0], [1, 2, 12], [1, 0, 5], [0, 1, 7]], np.int64)
    orr, lr = api.attn_rows(q, k, v, rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(orr[r], o[b, i, h])
        assert lr[r] == l[b, h, i]
    with pytest.raises(ValueError):
        api.attn_rows(q, k, v, np.array([[0, 3, 0]], np.int64))


# ---------------------------------------------------------------- merge

def test_merge_matches_decimal_brute_force(api):
    g = _rng(41)
    P, B, N, H, D = 3, 1, 4, 2, 5
    o_p = g.standard_normal((P, B, N, H, D))
    l_p = g.standard_normal((P, B, H, N)) * 30
    o, l = api.merge(o_p, l_p)
    for n in range(N):
        for h in range(H):
            bo, bl = brute.merge_row([o_p[t, 0, n, h].tolist() for t in range(P)],
                                     [float(l_p[t, 0, h, n]) for t in range(P)])
            _close(o[0, n, h], [float(x) for x in bo], 1e-14)
            _close(l[0, h, n], float(bl), 1e-14)


def test_merge_single_part_is_identity_and_order_free(api):
    g = _rng(42)
    P, B, N, H, D = 4, 2, 6, 2, 8
    o_p = g.standard_normal((P, B, N, H, D))
    l_p = g.standard_normal((P, B, H, N)) * 4
    o1, l1 = api.merge(o_p[:1], l_p[:1])
    _close(o1, o_p[0], 1e-15)
    _close(l1, l_p[0], 0.0)
    o, l = api.merge(o_p, l_p)
    perm = [2, 0, 3, 1]
    o2, l2 = api.merge(o_p[perm], l_p[perm])
    _close(o2, o, 1e-14)
    _close(l2, l, 1e-14)


def test_merge_neg_inf_parts(api):
    g = _rng(43)
    P, B, N, H, D = 3, 1, 5, 2, 4
    o_p = g.standard_normal((P, B, N, H, D))
    l_p = g.standard_normal((P, B, H, N))
    o_ref, l_ref = api.merge(o_p[[0, 2]], l_p[[0, 2]])
    l_p2 = l_p.copy()
    l_p2[1] = -np.inf
    o_p2 = o_p.copy()
    o_p2[1] = 1e300  # an empty part's o is never used
    o, l = api.merge(o_p2, l_p2)
    _close(o, o_ref, 1e-15)
    _close(l, l_ref, 1e-15)
    l_all = np.full_like(l_p, -np.inf)
    o, l = api.merge(o_p, l_all)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


# ---------------------------------------------------------------- permute

def _permute_by_exchange(x, p):
    """The page's sequence, emulated with numpy: on each sequence shard split the heads
    into p groups, send group j to rank j, and on rank j concatenate what arrives
    along the token axis in source-rank order (MindIE SD page, Ulysses usage example)."""
    shards = [x[s] for s in range(p)]                   # each [B, N/p, H, D]
    send = [np.split(sh, p, axis=2) for sh in shards]  # send[s][j]: [B, N/p, H/p, D]
    return np.stack([np.concatenate([send[s][j] for s in range(p)], axis=1) for j in range(p)])


@pytest.mark.parametrize("p,B,N,H,D,dt", [
    (1, 1, 3, 2, 4, np.uint16), (2, 1, 8, 4, 3, np.uint16), (4, 2, 12, 8, 5, np.float32),
    (4, 1, 16, 24, 2, np.uint16), (3, 1, 9, 6, 7, np.uint8),
])
def test_permute_index_map(api, p, B, N, H, D, dt):
    g = _rng(51)
    x = g.integers(0, 2 ** 16 if dt != np.uint8 else 256, size=(p, B, N // p, H, D)).astype(dt)
    if dt == np.float32:
        x = g.standard_normal((p, B, N // p, H, D)).astype(np.float32)
    out = api.permute(x, p)
    ref1 = x.reshape(p, B, N // p, p, H // p, D).transpose(3, 1, 0, 2, 4, 5).reshape(p, B, N, H // p, D)
    ref2 = _permute_by_exchange(x, p)
    assert out.tobytes() == ref1.tobytes()
    assert out.tobytes() == ref2.tobytes()
    # inverse: head shards back to sequence shards
    back = out.reshape(p, B, p, N // p, H // p, D).transpose(2, 1, 3, 0, 4, 5).reshape(x.shape)
    assert back.tobytes() == x.tobytes()


def test_permute_rejects_nondivisible(api):
    x = np.zeros((4, 1, 3, 6, 2), np.uint16)  # 6 heads not divisible by 4
    with pytest.raises(ValueError):
        api.permute(x, 4)


def _head_to_seq_by_exchange(y, p):
    """The page's sequence after attention, emulated with numpy: on each head shard split
    the tokens into p ranges, send range s to rank s, and on rank s concatenate what
    arrives along the head axis in source-rank order (MindIE SD page, Ulysses usage
    example, the second all-to-all)."""
    shards = [y[j] for j in range(p)]                   # each [B, N, H/p, D]
    send = [np.split(sh, p, axis=1) for sh in shards]  # send[j][s]: [B, N/p, H/p, D]
    return np.stack([np.concatenate([send[j][s] for j in range(p)], axis=2) for s in range(p)])


def _random_bits(g, shape, dt):
    if dt == np.float32:
        return g.standard_normal(shape).astype(np.float32)
    return g.integers(0, 2 ** 16 if dt != np.uint8 else 256, size=shape).astype(dt)


@pytest.mark.parametrize("p,B,N,H,D,dt", [
    (1, 1, 3, 2, 4, np.uint16), (2, 1, 8, 4, 3, np.uint16), (4, 2, 12, 8, 5, np.float32),
    (4, 1, 16, 24, 2, np.uint16), (3, 1, 9, 6, 7, np.uint8),
])
def test_head_to_seq_index_map_and_round_trips(api, p, B, N, H, D, dt):
    g = _rng(52)
    y = _random_bits(g, (p, B, N, H // p, D), dt)
    out = api.head_to_seq(y, p)
    assert out.shape == (p, B, N // p, H, D)
    ref1 = y.reshape(p, B, p, N // p, H // p, D).transpose(2, 1, 3, 0, 4, 5).reshape(out.shape)
    assert out.tobytes() == ref1.tobytes()
    assert out.tobytes() == _head_to_seq_by_exchange(y, p).tobytes()
    # the two all-to-alls undo each other, in either order
    assert api.permute(out, p).tobytes() == y.tobytes()
    x = _random_bits(g, (p, B, N // p, H, D), dt)
    assert api.head_to_seq(api.permute(x, p), p).tobytes() == x.tobytes()


def test_head_to_seq_rejects_nondivisible(api):
    y = np.zeros((4, 1, 6, 2, 2), np.uint16)  # 6 tokens not divisible by 4
    with pytest.raises(ValueError):
        api.head_to_seq(y, 4)


@pytest.mark.parametrize("p,B,N,H,D,dt", [
    (1, 1, 3, 2, 4, np.uint16), (2, 1, 8, 4, 3, np.uint16), (4, 2, 12, 8, 5, np.float32),
    (3, 1, 9, 6, 7, np.uint8),
])
def test_qkv_permute_index_map(api, p, B, N, H, D, dt):
    g = _rng(53)
    x = _random_bits(g, (p, B, N // p, 3, H, D), dt)
    out = api.qkv_permute(x, p)
    assert out.shape == (p, 3, B, N, H // p, D)
    # one exchange of the packed rows: split each shard's heads into p groups, send group
    # j to rank j, concatenate along tokens in source order, then unpack q, k, v
    send = [np.split(x[s], p, axis=3) for s in range(p)]   # send[s][j]: [B, N/p, 3, H/p, D]
    recv = [np.concatenate([send[s][j] for s in range(p)], axis=1) for j in range(p)]
    ref = np.stack([r.transpose(2, 0, 1, 3, 4) for r in recv])
    assert out.tobytes() == ref.tobytes()
    # equal to three separate permutes of the q, k and v tensors
    for c in range(3):
        per = api.permute(np.ascontiguousarray(x[:, :, :, c]), p)
        assert out[:, c].tobytes() == per.tobytes()


# ---------------------------------------------------------------- page numbers

def test_page_byte_counts_and_cross_rank_traffic(api):
    with open(os.path.join(GOLDEN, "page_byte_counts.json")) as f:
        gold = json.load(f)
    for e in gold["entries"]:
        if "shape" in e:
            nbytes = int(np.prod(e["shape"])) * e["elem_bytes"]
            if "bytes_printed" in e:
                assert abs(nbytes / e["bytes_printed"] - 1) <= e["rel_tol"], e["id"]
            else:
                assert abs(nbytes / 2 ** 20 - e["mib_printed"]) <= e["abs_tol_mib"], e["id"]
        else:
            # Bytes one GPU sends to other ranks in one Ulysses all-to-all = the part of its
            # shard the permute's index map sends to a head group j != its own rank s.
            N, H, D, p = e["N"], e["H"], e["D"], e["p"]
            tag = np.zeros((p, 1, N // p, H, 1), np.int32)
            for s in range(p):
                tag[s] = s
            out = api.permute(tag, p)                           # [p,1,N,H/p,1]
            dest = np.arange(p).reshape(p, 1, 1, 1, 1)
            foreign = int(np.sum(out != dest)) // p               # elements per sending GPU
            nbytes = foreign * D * e["elem_bytes"]
            assert nbytes == (p - 1) * N * H * D * e["elem_bytes"] // (p * p)
            assert abs(nbytes / e["bytes_printed"] - 1) <= e["rel_tol"], (e["id"], nbytes)
    for own in gold["ownership"]:
        N, H, p = own["N"], own["H"], own["p"]
        x = np.zeros((p, 1, N // p, H, 1), np.uint8)
        assert list(x.shape[2:4]) == own["before"]
        assert list(api.permute(x, p).shape[2:4]) == own["after"]


# ---------------------------------------------------------------- QK-RMSNorm + RoPE

def _nr_inputs(g, p, B, N, H, D):
    x = g.standard_normal((p, B, N // p, 3, H, D))
    gq = 0.5 + g.random(H * D)
    gk = 0.5 + g.random(H * D)
    ang = g.uniform(-4, 4, size=(N, D // 2))
    return x, gq, gk, np.cos(ang), np.sin(ang)


@pytest.mark.parametrize("p,B,N,H,D,eps", [(1, 1, 3, 2, 4, 1e-6), (2, 2, 4, 4, 6, 0.5), (3, 1, 6, 3, 2, 0.0)])
def test_norm_rope_matches_decimal_brute_force(api, p, B, N, H, D, eps):
    g = _rng(61)
    x, gq, gk, cs, sn = _nr_inputs(g, p, B, N, H, D)
    out = api.qkv_norm_rope(x, gq, gk, cs, sn, p, eps)
    Ns, Hs = N // p, H // p
    worst = 0.0
    for s in range(p):
        for b in range(B):
            for n in range(Ns):
                t = s * Ns + n
                for c, gam in ((0, gq), (1, gk)):
                    ref = brute.norm_rope_token(x[s, b, n, c].reshape(-1), gam, cs[t], sn[t], D, eps)
                    for h in range(H):
                        for d in range(D):
                            got = out[h // Hs, c, b, t, h % Hs, d]
                            worst = max(worst, abs(float(ref[h * D + d]) - got))
                for h in range(H):   # v: copied unchanged
                    assert np.array_equal(out[h // Hs, 2, b, t, h % Hs], x[s, b, n, 2, h])
    assert worst <= 1e-12, worst


def test_norm_rope_closed_forms(api):
    g = _rng(62)
    p, B, N, H, D = 2, 1, 4, 2, 8
    zero = np.zeros((N, D // 2))
    one = np.ones((N, D // 2))
    ones = np.ones(H * D)
    # a constant row a: y = sign(a) / sqrt(1 + eps / a^2); with gamma the factor applies per element
    x = np.full((p, B, N // p, 3, H, D), -2.0)
    out = api.qkv_norm_rope(x, ones, 3 * ones, one, zero, p, eps=0.0)
    assert np.allclose(out[:, 0], -1.0, rtol=0, atol=1e-15) and np.allclose(out[:, 1], -3.0, atol=1e-15)
    out = api.qkv_norm_rope(x, ones, ones, one, zero, p, eps=4.0)
    assert np.allclose(out[:, 0], -1.0 / np.sqrt(2.0), atol=1e-15)
    # zero angles, eps = 0: scale invariance, and every token's q has mean square gamma^2 = 1
    x = g.standard_normal((p, B, N // p, 3, H, D))
    a = api.qkv_norm_rope(x, ones, ones, one, zero, p, eps=0.0)
    b_ = api.qkv_norm_rope(7.5 * x, ones, ones, one, zero, p, eps=0.0)
    assert np.allclose(a[:, :2], b_[:, :2], atol=1e-13)
    tok = a[:, 0, 0].transpose(1, 0, 2, 3).reshape(N, H * D)      # [N, H*D] per token
    assert np.allclose(np.mean(tok ** 2, axis=1), 1.0, atol=1e-13)
    # quarter turn on every pair: (y_2i, y_2i+1) -> (-y_2i+1, y_2i)
    q = api.qkv_norm_rope(x, ones, ones, zero, one, p, eps=0.0)
    assert np.allclose(q[:, :2, ..., 0::2], -a[:, :2, ..., 1::2], atol=1e-14)
    assert np.allclose(q[:, :2, ..., 1::2], a[:, :2, ..., 0::2], atol=1e-14)
    # random angles keep each pair's length
    ang = g.uniform(-3, 3, size=(N, D // 2))
    r = api.qkv_norm_rope(x, ones, ones, np.cos(ang), np.sin(ang), p, eps=0.0)
    assert np.allclose(r[..., 0::2] ** 2 + r[..., 1::2] ** 2, a[..., 0::2] ** 2 + a[..., 1::2] ** 2, atol=1e-12)
    # the head mixing of the norm: doubling head 0 changes head 1's output
    x2 = x.copy()
    x2[..., 0, :] *= 2.0
    c = api.qkv_norm_rope(x2, ones, ones, one, zero, p, eps=0.0)
    assert not np.allclose(c[1, :2], a[1, :2])       # head 1 (head group 1 at p = H = 2)
    # v is the fused QKV permute's v
    assert r[:, 2].tobytes() == api.qkv_permute(x, p)[:, 2].tobytes()


def test_rope_3d_angles_structure(api):
    F, R, C, D = 3, 4, 5, 128
    A = oracle.rope_3d_angles(F, R, C, D)
    assert A.shape == (F * R * C, D // 2)
    idx = lambda f, r, c: (f * R + r) * C + c
    assert np.all(A[idx(0, 0, 0)] == 0)
    ef, er, ec = A[idx(1, 0, 0)], A[idx(0, 1, 0)], A[idx(0, 0, 1)]
    dt, dh = 22, 21   # the default division of 64 pairs: 22 frames, 21 rows, 21 cols
    assert np.all(ef[dt:] == 0) and np.all(er[:dt] == 0) and np.all(er[dt + dh:] == 0)
    assert np.all(ec[:dt + dh] == 0)
    for part in (ef[:dt], er[dt:dt + dh], ec[dt + dh:]):
        # pair 0 turns by the position itself; each next pair base^(-1/d) slower
        assert part[0] == 1.0
        ratio = part[1:] / part[:-1]
        assert np.allclose(ratio, 10000.0 ** (-1.0 / len(part)), rtol=1e-13)
        assert part[-1] > 1e-4
    for f in range(F):           # angles are linear in each position
        for r in range(R):
            for c in range(C):
                assert np.allclose(A[idx(f, r, c)], f * ef + r * er + c * ec, rtol=0, atol=1e-12)


def test_rope_relative_position_property(api):
    """q.k after the embedding depends only on the position difference of the two
    tokens (the property rotary embeddings are built for), on the 3D grid tables."""
    g = _rng(63)
    F, R, C, H, D = 2, 3, 4, 1, 12
    N = F * R * C
    A = oracle.rope_3d_angles(F, R, C, D)
    qv = g.standard_normal(H * D)
    kv = g.standard_normal(H * D)
    x = np.zeros((1, 1, N, 3, H, D))
    x[0, 0, :, 0] = qv.reshape(H, D)
    x[0, 0, :, 1] = kv.reshape(H, D)
    ones = np.ones(H * D)
    out = api.qkv_norm_rope(x, ones, ones, np.cos(A), np.sin(A), 1, eps=0.0)
    qo, ko = out[0, 0, 0, :, 0], out[0, 1, 0, :, 0]   # [N, D]
    idx = lambda f, r, c: (f * R + r) * C + c
    d1 = qo[idx(1, 2, 3)] @ ko[idx(0, 1, 1)]
    d2 = qo[idx(1, 1, 2)] @ ko[idx(0, 0, 0)]          # the same difference (1, 1, 2)
    d3 = qo[idx(1, 1, 3)] @ ko[idx(0, 0, 0)]          # another difference
    assert abs(d1 - d2) <= 1e-12 * max(1.0, abs(d1))
    assert abs(d1 - d3) > 1e-3
