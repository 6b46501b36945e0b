"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` takes the oracle module and raises AssertionError on a
mismatch. test_oracle_pins.py runs them against the real oracle;
test_oracle_mutants.py plants mistakes in the oracle and requires that some
check fails for each planted mistake.

Pins come from: hand-worked golden values (tests/golden/, each citing the
page passage it follows), brute force written independently with math.fsum,
torch's fp64 CPU scaled_dot_product_attention on padded per-sequence
inputs, closed forms and invariants of softmax attention and of the merge.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f(x):
    if isinstance(x, str):
        return float(x)          # "-inf" / "inf"
    if isinstance(x, list):
        return [_f(e) for e in x]
    return x


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def _same(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    assert np.array_equal(inf_a, inf_b), "infinite entries differ"
    assert np.array_equal(a[inf_a], b[inf_b]), "signs of infinite entries differ"
    fin = ~inf_a
    assert not np.isnan(a).any() and not np.isnan(b).any(), "NaN"
    if fin.any():
        err = np.abs(a[fin] - b[fin])
        bound = tol + tol * np.abs(b[fin])
        assert (err <= bound).all(), f"max err {err.max():.3e}"


# ---------------------------------------------------------------- random cases

def _rand_case(rng, batch, max_len, hq, hkv, d, allow_unequal=True, allow_empty=False):
    lo = 0 if allow_empty else 1
    lq = rng.integers(lo, max_len + 1, batch)
    lk = rng.integers(lo, max_len + 1, batch) if allow_unequal else lq.copy()
    tq, tk = int(lq.sum()), int(lk.sum())
    q = rng.standard_normal((tq, hq, d))
    k = rng.standard_normal((tk, hkv, d))
    v = rng.standard_normal((tk, hkv, d))
    return lq, lk, q, k, v


def brute_force(q, k, v, lengths_q, lengths_k, hq, hkv, scale, causal, d, dv, offsets=None):
    """Pure-Python softmax attention from the definition, with math.fsum sums.

    offsets[b] (optional): query i of sequence b sees key j iff j <= i + offsets[b]."""
    cu_q = [0]
    for x in lengths_q:
        cu_q.append(cu_q[-1] + int(x))
    cu_k = [0]
    for x in lengths_k:
        cu_k.append(cu_k[-1] + int(x))
    grp = hq // hkv
    out = [[[0.0] * dv for _ in range(hq)] for _ in range(cu_q[-1])]
    lse = [[-math.inf] * hq for _ in range(cu_q[-1])]
    for b in range(len(lengths_q)):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for h in range(hq):
            kvh = h // grp
            for i in range(lq):
                t = cu_q[b] + i
                lim = i + (lk - lq if offsets is None else offsets[b])
                keys = [j for j in range(lk) if (not causal) or j <= lim]
                if not keys:
                    continue
                s = {j: scale * math.fsum(q[t][h][x] * k[cu_k[b] + j][kvh][x] for x in range(d))
                     for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                tot = math.fsum(w.values())
                for x in range(dv):
                    out[t][h][x] = math.fsum(w[j] * v[cu_k[b] + j][kvh][x] for j in keys) / tot
                lse[t][h] = mx + math.log(tot)
    return np.array(out, dtype=np.float64).reshape(cu_q[-1], hq, dv), \
        np.array(lse, dtype=np.float64).reshape(cu_q[-1], hq)


def check_golden_attention(orc):
    for case in _load("attention_handworked.json")["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        v = np.array(case["v"], dtype=np.float64)
        o, lse = orc.varlen_attention(q, k, v, _cu(case["lengths_q"]), _cu(case["lengths_k"]),
                                      case["num_heads_kv"], case["scale"], case["causal"])
        _same(o, np.array(_f(case["out"])), 1e-12)
        _same(lse, np.array(_f(case["lse"])), 1e-12)


def check_golden_merge(orc):
    g = _load("merge_handworked.json")
    lse = np.array(_f(g["lse"]), dtype=np.float64)
    go = np.array(g["go"], dtype=np.float64)
    out, lse_out = orc.attn_update(lse, go, 1)
    _same(out, np.array(g["out"]), 1e-12)
    _same(lse_out, np.array(_f(g["lse_out"])), 1e-12)
    out0, none = orc.attn_update(lse, go, 0)
    assert none is None
    _same(out0, np.array(g["out"]), 1e-12)


def check_golden_gather(orc):
    g = _load("gather_tiny.json")
    assert _cu(g["lengths"]).tolist() == g["cu_seqlens"]
    x = np.arange(g["cu_seqlens"][-1] * 3, dtype=np.float64).reshape(-1, 3)
    got = orc.last_token_gather(x, np.array(g["cu_seqlens"], dtype=np.int32))
    assert np.array_equal(got[:, 0] / 3, np.array(g["last_token_indices"], dtype=np.float64))


def check_brute_force(orc, n_cases=40, seed=11):
    rng = np.random.default_rng(seed)
    for _ in range(n_cases):
        batch = int(rng.integers(1, 4))
        hkv = int(rng.integers(1, 3))
        hq = hkv * int(rng.integers(1, 3))
        d = int(rng.integers(1, 5))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.uniform(0.2, 1.5))
        lq, lk, q, k, v = _rand_case(rng, batch, 5, hq, hkv, d, allow_unequal=True, allow_empty=True)
        o_b, lse_b = brute_force(q.tolist(), k.tolist(), v.tolist(), lq, lk, hq, hkv, scale, causal, d, d)
        o, lse = orc.varlen_attention(q, k, v, _cu(lq), _cu(lk), hkv, scale, causal)
        _same(o, o_b, 1e-12)
        _same(lse, lse_b, 1e-12)


def check_torch_sdpa(orc, seed=5):
    """torch CPU fp64 SDPA on padded per-sequence BNSD with repeat-interleaved K/V."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    for causal, (hq, hkv) in itertools.product([True, False], [(4, 2), (6, 3), (2, 2)]):
        d = 8
        lq = rng.integers(1, 12, 3)
        lk = lq + rng.integers(0, 4, 3)      # Lk >= Lq so no row is fully masked
        q = rng.standard_normal((int(lq.sum()), hq, d))
        k = rng.standard_normal((int(lk.sum()), hkv, d))
        v = rng.standard_normal((int(lk.sum()), hkv, d))
        scale = 0.37
        o, lse = orc.varlen_attention(q, k, v, _cu(lq), _cu(lk), hkv, scale, causal)
        cq, ck = _cu(lq), _cu(lk)
        for b in range(3):
            qb = torch.from_numpy(q[cq[b]:cq[b + 1]]).transpose(0, 1).unsqueeze(0)      # [1,Hq,Lq,D]
            kb = torch.from_numpy(k[ck[b]:ck[b + 1]]).repeat_interleave(hq // hkv, dim=1)
            vb = torch.from_numpy(v[ck[b]:ck[b + 1]]).repeat_interleave(hq // hkv, dim=1)
            kb = kb.transpose(0, 1).unsqueeze(0).contiguous()
            vb = vb.transpose(0, 1).unsqueeze(0).contiguous()
            lqb, lkb = int(lq[b]), int(lk[b])
            ii = torch.arange(lqb)[:, None]
            jj = torch.arange(lkb)[None, :]
            allow = (jj <= ii + (lkb - lqb)) if causal else torch.ones(lqb, lkb, dtype=torch.bool)
            ref = F.scaled_dot_product_attention(qb, kb, vb, attn_mask=allow, scale=scale)
            sc = scale * (qb @ kb.transpose(-1, -2))
            sc = sc.masked_fill(~allow, float("-inf"))
            ref_lse = torch.logsumexp(sc, dim=-1)                                           # [1,Hq,Lq]
            _same(o[cq[b]:cq[b + 1]], ref[0].transpose(0, 1).numpy(), 1e-10)
            _same(lse[cq[b]:cq[b + 1]], ref_lse[0].transpose(0, 1).numpy(), 1e-10)


def check_closed_forms(orc, seed=7):
    rng = np.random.default_rng(seed)
    hq, hkv, d = 4, 2, 6
    grp = hq // hkv
    lq = np.array([5, 9, 1]); lk = np.array([7, 9, 3])
    cq, ck = _cu(lq), _cu(lk)
    k = rng.standard_normal((int(lk.sum()), hkv, d))
    v = rng.standard_normal((int(lk.sum()), hkv, d))
    # (1) Q = 0: uniform weights over visible keys -> mean of visible V, lse = ln(#visible)
    q0 = np.zeros((int(lq.sum()), hq, d))
    o, lse = orc.varlen_attention(q0, k, v, cq, ck, hkv, 0.5, True)
    for b in range(3):
        for i in range(int(lq[b])):
            nvis = min(int(lk[b]), max(0, i + 1 + int(lk[b]) - int(lq[b])))
            for h in range(hq):
                t = cq[b] + i
                if nvis == 0:
                    assert lse[t, h] == -np.inf and not o[t, h].any()
                    continue
                exp_o = v[ck[b]:ck[b] + nvis, h // grp].mean(axis=0)
                _same(o[t, h], exp_o, 1e-12)
                _same(lse[t, h], math.log(nvis), 1e-12)
    # (2) causal, Lq = Lk: row 0 sees only key 0 -> O = V[0], lse = scale q0.k0
    q = rng.standard_normal((int(lq.sum()), hq, d))
    sq = np.array([4, 6]); cs = _cu(sq)
    qs = rng.standard_normal((10, hq, d)); ks = rng.standard_normal((10, hkv, d)); vs = rng.standard_normal((10, hkv, d))
    o, lse = orc.varlen_attention(qs, ks, vs, cs, cs, hkv, 0.3, True)
    for b in range(2):
        t = cs[b]
        for h in range(hq):
            _same(o[t, h], vs[t, h // grp], 1e-12)
            _same(lse[t, h], 0.3 * float(qs[t, h] @ ks[t, h // grp]), 1e-12)
    # (3) V constant per kv head -> O equals that constant on every row with a visible key
    vc = np.broadcast_to(np.array([1.5, -2.0])[None, :, None], v.shape).copy()
    o, lse = orc.varlen_attention(q, k, vc, cq, ck, hkv, 0.9, False)
    for h in range(hq):
        _same(o[:, h, :], np.full((int(lq.sum()), d), [1.5, -2.0][h // grp]), 1e-12)
    # (4) one key: O = V0, lse = s0
    q1 = rng.standard_normal((3, hq, d)); k1 = rng.standard_normal((1, hkv, d)); v1 = rng.standard_normal((1, hkv, d))
    o, lse = orc.varlen_attention(q1, k1, v1, np.array([0, 3]), np.array([0, 1]), hkv, 0.7, False)
    for h in range(hq):
        _same(o[:, h], np.repeat(v1[0:1, h // grp], 3, axis=0), 1e-12)
        _same(lse[:, h], 0.7 * (q1[:, h] @ k1[0, h // grp]), 1e-12)


def check_merge_invariants(orc, seed=3):
    rng = np.random.default_rng(seed)
    for causal, sp in itertools.product([True, False], [1, 2, 3, 8]):
        hq, hkv, d = 4, 2, 5
        lq = np.array([6, 13, 1, 9]); lk = lq.copy()
        if not causal:
            lk = np.array([7, 13, 11, 2])
        q = rng.standard_normal((int(lq.sum()), hq, d))
        k = rng.standard_normal((int(lk.sum()), hkv, d))
        v = rng.standard_normal((int(lk.sum()), hkv, d))
        o, lse = orc.varlen_attention(q, k, v, _cu(lq), _cu(lk), hkv, 0.4, causal)
        lse_c, go_c = orc.chunked_partials(q, k, v, _cu(lq), _cu(lk), hkv, 0.4, causal, sp)
        # (5) chunked + merged = unchunked
        out_m, lse_m = orc.attn_update(lse_c, go_c, 1)
        _same(out_m, o.reshape(-1, d), 1e-11)
        _same(lse_m, lse.reshape(-1), 1e-11)
        # (9) chunk order does not matter
        perm = rng.permutation(sp)
        out_p, lse_p = orc.attn_update(lse_c[perm], go_c[perm], 1)
        _same(out_p, out_m, 1e-12)
        _same(lse_p, lse_m, 1e-12)
    # (8) sp = 1 is the identity
    lse1 = rng.standard_normal((1, 10)); go1 = rng.standard_normal((1, 10, 3))
    out1, l1 = orc.attn_update(lse1, go1, 1)
    _same(out1, go1[0], 1e-13)
    _same(l1, lse1[0], 1e-13)
    # (10) a chunk with lse = -inf contributes nothing, whatever its O
    lse2 = np.concatenate([lse1, np.full((1, 10), -np.inf)], axis=0)
    go2 = np.concatenate([go1, 1e6 * rng.standard_normal((1, 10, 3))], axis=0)
    out2, l2 = orc.attn_update(lse2, go2, 1)
    _same(out2, go1[0], 1e-13)
    _same(l2, lse1[0], 1e-13)
    # merging two equal partials adds ln 2 to lse and keeps O
    out3, l3 = orc.attn_update(np.concatenate([lse1, lse1]), np.concatenate([go1, go1]), 1)
    _same(out3, go1[0], 1e-12)
    _same(l3, lse1[0] + math.log(2.0), 1e-12)


def check_attention_invariants(orc, seed=9):
    rng = np.random.default_rng(seed)
    hq, hkv, d = 6, 2, 7
    grp = hq // hkv
    lq = np.array([3, 10, 1, 6]); lk = np.array([5, 10, 4, 6])
    cq, ck = _cu(lq), _cu(lk)
    q = rng.standard_normal((int(lq.sum()), hq, d))
    k = rng.standard_normal((int(lk.sum()), hkv, d))
    v = rng.standard_normal((int(lk.sum()), hkv, d))
    for causal in (True, False):
        o, lse = orc.varlen_attention(q, k, v, cq, ck, hkv, 0.45, causal)
        # (6) packed TND = each sequence alone
        for b in range(4):
            ob, lb = orc.varlen_attention(q[cq[b]:cq[b + 1]], k[ck[b]:ck[b + 1]], v[ck[b]:ck[b + 1]],
                                          np.array([0, lq[b]]), np.array([0, lk[b]]), hkv, 0.45, causal)
            _same(o[cq[b]:cq[b + 1]], ob, 1e-13)
            _same(lse[cq[b]:cq[b + 1]], lb, 1e-13)
        # (7) GQA = MHA on K/V repeated along the head axis (repeat_interleave(G, dim=1))
        om, lm = orc.varlen_attention(q, np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1),
                                      cq, ck, hq, 0.45, causal)
        _same(o, om, 1e-13)
        _same(lse, lm, 1e-13)
        # (11) K -> K + u per kv head: O unchanged, lse shifts by scale * q.u
        u = rng.standard_normal((hkv, d))
        ou, lu = orc.varlen_attention(q, k + u[None], v, cq, ck, hkv, 0.45, causal)
        shift = 0.45 * np.einsum("thd,hd->th", q, np.repeat(u, grp, axis=0))
        fin = np.isfinite(lse)
        _same(ou, o, 1e-11)
        _same(lu[fin], (lse + shift)[fin], 1e-11)
        # (12) scale folded into Q
        os_, ls_ = orc.varlen_attention(0.45 * q, k, v, cq, ck, hkv, 1.0, causal)
        _same(os_, o, 1e-12)
        _same(ls_, lse, 1e-12)
        # (13) max_j s_j <= lse <= max_j s_j + ln(#visible)
        for b in range(4):
            for i in range(int(lq[b])):
                vis = [j for j in range(int(lk[b])) if (not causal) or j <= i + lk[b] - lq[b]]
                for h in range(hq):
                    t = cq[b] + i
                    if not vis:
                        assert lse[t, h] == -np.inf
                        continue
                    s = [0.45 * float(q[t, h] @ k[ck[b] + j, h // grp]) for j in vis]
                    assert max(s) - 1e-12 <= lse[t, h] <= max(s) + math.log(len(vis)) + 1e-12
        # (14) sequence order in the pack does not matter
        perm = np.array([2, 0, 3, 1])
        qp = np.concatenate([q[cq[b]:cq[b + 1]] for b in perm])
        kp = np.concatenate([k[ck[b]:ck[b + 1]] for b in perm])
        vp = np.concatenate([v[ck[b]:ck[b + 1]] for b in perm])
        op, lp = orc.varlen_attention(qp, kp, vp, _cu(lq[perm]), _cu(lk[perm]), hkv, 0.45, causal)
        _same(op, np.concatenate([o[cq[b]:cq[b + 1]] for b in perm]), 1e-13)
        _same(lp, np.concatenate([lse[cq[b]:cq[b + 1]] for b in perm]), 1e-13)


def check_rows_subset(orc, seed=13):
    """Selected-token evaluation equals the same rows of the whole-batch result."""
    rng = np.random.default_rng(seed)
    lq = np.array([4, 9, 2]); lk = np.array([4, 12, 2])
    q = rng.standard_normal((15, 4, 3)); k = rng.standard_normal((18, 2, 3)); v = rng.standard_normal((18, 2, 3))
    o, lse = orc.varlen_attention(q, k, v, _cu(lq), _cu(lk), 2, 0.8, True)
    tok = np.array([14, 0, 7, 4, 13])
    os_, ls_ = orc.varlen_attention_rows(q, k, v, _cu(lq), _cu(lk), 2, 0.8, True, tokens=tok)
    _same(os_, o[tok], 1e-14)
    _same(ls_, lse[tok], 1e-14)


def _num(x):
    """Golden numbers: plain floats, "a/b" fractions or "lnN"."""
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(x[2:]))
        sign = -1.0 if x.startswith("-") else 1.0
        a, b = x.lstrip("-").split("/")
        return sign * float(a) / float(b)
    return float(x)


def check_golden_paged(orc):
    g = _load("paged_handworked.json")
    ps, npg = g["page_size"], g["num_pages"]
    v_cache = np.full((npg, ps, 1, 2), np.nan)
    k_cache = np.full((npg, ps, 1, 2), np.nan)
    table = np.asarray(g["block_table"])
    for b, used in enumerate(g["seqused_k"]):          # fill only the slots a key names
        for j in range(used):
            p, s = table[b][j // ps], j % ps
            v_cache[p, s, 0] = [10 * p + s, -(10 * p + s)]
            k_cache[p, s, 0] = 0.0
    cu_q = np.asarray(g["cu_seqlens_q"])
    q = np.zeros((int(cu_q[-1]), 1, 2))
    out, lse = orc.paged_attention_rows(q, k_cache, v_cache, table, g["seqused_k"], cu_q, 1, 1.0, g["causal"])
    want_o = np.array([[_num(e) for e in row] for row in g["out"]])
    want_l = np.array([_num(e) for e in g["lse"]])
    assert np.allclose(out[:, 0, :], want_o, rtol=1e-14, atol=1e-12), (out[:, 0, :], want_o)
    assert np.allclose(lse[:, 0], want_l, rtol=1e-14, atol=1e-14), (lse[:, 0], want_l)


def check_paged_scatter(orc, seed=17):
    """Contiguous K/V scattered into shuffled pages, read back through the table, gives the
    contiguous oracle's result exactly; every slot no key names holds NaN."""
    rng = np.random.default_rng(seed)
    for ps in (1, 2, 3, 4, 16):
        for causal in (True, False):
            batch = int(rng.integers(1, 5))
            lk = rng.integers(0, 40, batch)
            lq = np.minimum(rng.integers(1, 4, batch), np.maximum(lk, 1))
            hq, hkv, d = 4, 2, 8
            q = rng.standard_normal((int(lq.sum()), hq, d))
            k = rng.standard_normal((int(lk.sum()), hkv, d))
            v = rng.standard_normal((int(lk.sum()), hkv, d))
            cu_q, cu_k = _cu(lq), _cu(lk)
            need = [-(-int(n) // ps) for n in lk]
            max_pages = max(need) + 1
            num_pages = sum(need) + 5                      # spare pages stay NaN
            perm = rng.permutation(num_pages)
            k_cache = np.full((num_pages, ps, hkv, d), np.nan)
            v_cache = np.full((num_pages, ps, hkv, d), np.nan)
            table = np.full((batch, max_pages), -1, dtype=np.int64)
            nxt = 0
            for b in range(batch):
                for p in range(need[b]):                   # logical page p of b -> a shuffled physical page
                    table[b, p] = perm[nxt]
                    nxt += 1
                for t in range(int(lk[b])):                # write each key row to its page and slot
                    phys, slot = table[b, t // ps], t % ps
                    k_cache[phys, slot] = k[cu_k[b] + t]
                    v_cache[phys, slot] = v[cu_k[b] + t]
            o_p, l_p = orc.paged_attention_rows(q, k_cache, v_cache, table, lk, cu_q, hkv, 0.3, causal)
            o_c, l_c = orc.varlen_attention(q, k, v, cu_q, cu_k, hkv, 0.3, causal)
            assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c), (ps, causal)
            assert np.all(np.isfinite(o_p))


def check_causal_offset_brute_force(orc, n_cases=24, seed=19):
    """Per-sequence causal offsets against the brute force, including offsets that hide every key
    from some rows and offsets past the last key."""
    rng = np.random.default_rng(seed)
    for _ in range(n_cases):
        batch = int(rng.integers(1, 4))
        lq = rng.integers(0, 6, batch)
        lk = rng.integers(0, 6, batch)
        hq, hkv, d = 2, 1, 3
        off = [int(rng.integers(-int(b) - 2, int(a) + int(b) + 3)) for a, b in zip(lq, lk)]
        q = rng.standard_normal((int(lq.sum()), hq, d))
        k = rng.standard_normal((int(lk.sum()), hkv, d))
        v = rng.standard_normal((int(lk.sum()), hkv, d))
        o, l = orc.varlen_attention(q, k, v, _cu(lq), _cu(lk), hkv, 0.7, True, causal_offset=off)
        ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), lq, lk, hq, hkv, 0.7, True, d, d, offsets=off)
        _same(o, ob, 1e-12)
        _same(l, lb, 1e-12)


def check_causal_offset_chunks(orc, seed=23):
    """A key chunk [a, c) of square causal sequences, packed alone and computed with offset -a, equals
    the chunk partial that keeps absolute positions through key_range (chunked_partials)."""
    rng = np.random.default_rng(seed)
    lens = np.array([9, 1, 14, 6])
    hq, hkv, d, sp = 4, 2, 5, 3
    q = rng.standard_normal((int(lens.sum()), hq, d))
    k = rng.standard_normal((int(lens.sum()), hkv, d))
    v = rng.standard_normal((int(lens.sum()), hkv, d))
    cu = _cu(lens)
    lse_c, go_c = orc.chunked_partials(q, k, v, cu, cu, hkv, 0.5, True, sp)
    for c in range(sp):
        bounds = [((c * int(n)) // sp, ((c + 1) * int(n)) // sp) for n in lens]
        kc = np.concatenate([k[cu[b] + lo:cu[b] + hi] for b, (lo, hi) in enumerate(bounds)])
        vc = np.concatenate([v[cu[b] + lo:cu[b] + hi] for b, (lo, hi) in enumerate(bounds)])
        o, l = orc.varlen_attention(q, kc, vc, cu, _cu([hi - lo for lo, hi in bounds]), hkv, 0.5, True,
                                    causal_offset=[-lo for lo, _ in bounds])
        assert np.allclose(o.reshape(-1, d), go_c[c], rtol=1e-13, atol=1e-13)
        assert np.array_equal(np.isneginf(l.reshape(-1)), np.isneginf(lse_c[c]))
        live = ~np.isneginf(lse_c[c])
        assert np.allclose(l.reshape(-1)[live], lse_c[c][live], rtol=1e-13, atol=1e-13)


ALL_CHECKS = [
    check_golden_attention,
    check_golden_merge,
    check_golden_gather,
    check_brute_force,
    check_torch_sdpa,
    check_closed_forms,
    check_merge_invariants,
    check_attention_invariants,
    check_rows_subset,
    check_golden_paged,
    check_paged_scatter,
    check_causal_offset_brute_force,
    check_causal_offset_chunks,
]


# ------------------------------------------------------------------ attention prologue (oracle/prologue.py)

def check_golden_qk_norm_rope(pro):
    g = _load("qk_norm_rope_handworked.json")
    x = np.array(g["x"], dtype=np.float64).reshape(1, 1, -1)
    cos = np.array(g["cos"], dtype=np.float64).reshape(1, -1)
    sin = np.array(g["sin"], dtype=np.float64).reshape(1, -1)
    q_out, k_out = pro.qk_norm_rope(x, x, g["weight"], g["k_weight"], cos, sin, g["eps"])
    want = np.array(g["out_times_sqrt_7_5"], dtype=np.float64) / math.sqrt(7.5)
    want_k = np.array(g["k_out_times_sqrt_7_5"], dtype=np.float64) / math.sqrt(7.5)
    assert np.allclose(q_out.reshape(-1), want, rtol=1e-15, atol=1e-15), (q_out, want)
    assert np.allclose(k_out.reshape(-1), want_k, rtol=1e-15, atol=1e-15), (k_out, want_k)


def check_rms_norm_torch(pro, seed=29):
    """torch's fp64 CPU rms_norm over the last dimension (a library routine) with a weight and eps."""
    import torch
    rng = np.random.default_rng(seed)
    for d, eps in ((128, 1e-6), (64, 0.1), (8, 2.0)):
        x = rng.standard_normal((5, 3, d)) * 3.0
        w = 1.0 + 0.2 * rng.standard_normal(d)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(w), eps).numpy()
        assert np.allclose(pro.rms_norm(x, w, eps), ref, rtol=1e-13, atol=1e-13)


def _angle_tables(rng, t, d):
    theta = rng.uniform(-math.pi, math.pi, (t, d // 2))
    emb = np.concatenate([theta, theta], axis=-1)
    return theta, np.cos(emb), np.sin(emb)


def check_rotary_complex(pro, seed=31):
    """With cos / sin built from angles (the same angle for d and d + D/2), the rotation is the complex
    product (y[:D/2] + i y[D/2:]) * exp(i theta): an independent way to write it."""
    rng = np.random.default_rng(seed)
    t, n, d = 6, 3, 16
    y = rng.standard_normal((t, n, d))
    theta, cos, sin = _angle_tables(rng, t, d)
    z = (y[..., :d // 2] + 1j * y[..., d // 2:]) * np.exp(1j * theta)[:, None, :]
    want = np.concatenate([z.real, z.imag], axis=-1)
    assert np.allclose(pro.rotary(y, cos, sin), want, rtol=1e-13, atol=1e-13)


def check_rotary_identity_and_pair_norms(pro, seed=37):
    rng = np.random.default_rng(seed)
    t, n, d = 4, 2, 8
    y = rng.standard_normal((t, n, d))
    assert np.array_equal(pro.rotary(y, np.ones((t, d)), np.zeros((t, d))), y)        # position 0
    _, cos, sin = _angle_tables(rng, t, d)
    out = pro.rotary(y, cos, sin)
    h = d // 2
    assert np.allclose(out[..., :h] ** 2 + out[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2, rtol=1e-13)


def check_rms_norm_invariants(pro, seed=41):
    """eps = 0: the output is unchanged by a positive scale, negated by a negative one, and its
    mean square is 1 with a unit weight."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((7, 2, 32))
    one = np.ones(32)
    base = pro.rms_norm(x, one, 0.0)
    assert np.allclose(pro.rms_norm(5.0 * x, one, 0.0), base, rtol=1e-14, atol=1e-14)
    assert np.allclose(pro.rms_norm(-0.25 * x, one, 0.0), -base, rtol=1e-14, atol=1e-14)
    assert np.allclose(np.mean(base ** 2, axis=-1), 1.0, rtol=1e-14)


PROLOGUE_CHECKS = [
    check_golden_qk_norm_rope,
    check_rms_norm_torch,
    check_rotary_complex,
    check_rotary_identity_and_pair_norms,
    check_rms_norm_invariants,
]


# ------------------------------------------------------------------ gated delta rule (oracle/linear_attention.py)

def _gdn_inputs(rng, lengths, hqk, hv, dk, dv, decay=(0.8, 1.0)):
    t = int(sum(lengths))
    q = rng.standard_normal((t, hqk, dk))
    k = rng.standard_normal((t, hqk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((t, hv, dv))
    g = np.log(rng.uniform(decay[0], decay[1], (t, hv)))
    beta = rng.uniform(0.0, 1.0, (t, hv))
    return q, k, v, g, beta


def check_golden_gated_delta(lin):
    gd = _load("gated_delta_handworked.json")
    q = np.array(gd["q"], dtype=np.float64)[:, None, :]
    k = np.array(gd["k"], dtype=np.float64)[:, None, :]
    v = np.array(gd["v"], dtype=np.float64)[:, None, :]
    g = np.log(np.array(gd["decay"], dtype=np.float64))[:, None]
    beta = np.array(gd["beta"], dtype=np.float64)[:, None]
    o, fin = lin.gated_delta_rule(q, k, v, g, beta, [0, 3], 1.0)
    assert np.allclose(o[:, 0, :], np.array(gd["out"], dtype=np.float64), rtol=1e-14, atol=1e-14), o
    assert np.allclose(fin[0, 0], np.array(gd["final_state"], dtype=np.float64), rtol=1e-14, atol=1e-14), fin


def check_gated_delta_beta_zero(lin, seed=43):
    """beta = 0: nothing is written, so the state is the decayed initial state and
    o_t = scale * (prod_{s<=t} a_s) * S0^T q_t."""
    rng = np.random.default_rng(seed)
    q, k, v, g, _ = _gdn_inputs(rng, [5, 3], 2, 4, 6, 5)
    s0 = rng.standard_normal((2, 4, 6, 5))
    o, fin = lin.gated_delta_rule(q, k, v, g, np.zeros_like(g), [0, 5, 8], 0.7, initial_state=s0)
    for b, (lo, hi) in enumerate(((0, 5), (5, 8))):
        for h in range(4):
            cum = np.exp(np.cumsum(g[lo:hi, h]))
            want = 0.7 * cum[:, None] * (q[lo:hi, h // 2] @ s0[b, h])
            assert np.allclose(o[lo:hi, h], want, rtol=1e-12, atol=1e-12)
            assert np.allclose(fin[b, h], cum[-1] * s0[b, h], rtol=1e-12, atol=1e-12)


def check_gated_delta_associative_recall(lin, seed=47):
    """No decay, beta = 1, keys the standard basis vectors e_0, e_1, ...: each write lands in an empty
    slot, so querying with e_r after token r returns scale * v_r exactly."""
    rng = np.random.default_rng(seed)
    dk, dv, t = 8, 3, 6
    k = np.eye(dk)[:t][:, None, :]
    v = rng.standard_normal((t, 1, dv))
    r = [0, 1, 0, 3, 2, 4]                               # query slot <= token index
    q = np.eye(dk)[r][:, None, :]
    o, _ = lin.gated_delta_rule(q, k, v, np.zeros((t, 1)), np.ones((t, 1)), [0, t], 1.5)
    assert np.allclose(o[:, 0, :], 1.5 * v[r, 0, :], rtol=1e-14, atol=1e-14)


def check_gated_delta_continuation_and_packing(lin, seed=53):
    """Running a sequence in two pieces, the second started from the first's final state, equals running
    it whole; a packed batch equals its sequences run one by one."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _gdn_inputs(rng, [9, 4, 7], 1, 2, 4, 3)
    o_all, fin_all = lin.gated_delta_rule(q, k, v, g, beta, [0, 9, 13, 20], 0.5)
    for b, (lo, hi) in enumerate(((0, 9), (9, 13), (13, 20))):
        o_b, fin_b = lin.gated_delta_rule(q[lo:hi], k[lo:hi], v[lo:hi], g[lo:hi], beta[lo:hi], [0, hi - lo], 0.5)
        assert np.allclose(o_b, o_all[lo:hi], rtol=1e-13, atol=1e-13)
        assert np.allclose(fin_b[0], fin_all[b], rtol=1e-13, atol=1e-13)
    lo, mid, hi = 0, 5, 9
    o1, f1 = lin.gated_delta_rule(q[lo:mid], k[lo:mid], v[lo:mid], g[lo:mid], beta[lo:mid], [0, mid], 0.5)
    o2, f2 = lin.gated_delta_rule(q[mid:hi], k[mid:hi], v[mid:hi], g[mid:hi], beta[mid:hi], [0, hi - mid], 0.5,
                                  initial_state=f1)
    assert np.allclose(np.concatenate([o1, o2]), o_all[lo:hi], rtol=1e-13, atol=1e-13)
    assert np.allclose(f2[0], fin_all[0], rtol=1e-13, atol=1e-13)


def check_gated_delta_linear_in_v(lin, seed=59):
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _gdn_inputs(rng, [6, 5], 2, 2, 5, 4)
    v2 = rng.standard_normal(v.shape)
    cu = [0, 6, 11]
    a, fa = lin.gated_delta_rule(q, k, v, g, beta, cu, 1.0)
    b, fb = lin.gated_delta_rule(q, k, v2, g, beta, cu, 1.0)
    c, fc = lin.gated_delta_rule(q, k, 2.0 * v - v2, g, beta, cu, 1.0)
    assert np.allclose(c, 2.0 * a - b, rtol=1e-12, atol=1e-12)
    assert np.allclose(fc, 2.0 * fa - fb, rtol=1e-12, atol=1e-12)


def _gdn_chunked(q, k, v, g, beta, cu, scale, chunk):
    """The same operator written the chunked (WY) way: per chunk, the corrections of all its tokens come
    from one lower-triangular solve, outputs and the state update from matrix products."""
    t_all, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    rep = hv // hqk
    out = np.zeros((t_all, hv, dv))
    fin = np.zeros((len(cu) - 1, hv, dk, dv))
    for b in range(len(cu) - 1):
        for h in range(hv):
            st = np.zeros((dk, dv))
            for c0 in range(cu[b], cu[b + 1], chunk):
                c1 = min(c0 + chunk, cu[b + 1])
                kc, qc, vc = k[c0:c1, h // rep], q[c0:c1, h // rep], v[c0:c1, h]
                gcum = np.cumsum(g[c0:c1, h])
                bc = beta[c0:c1, h]
                decay = np.exp(gcum[:, None] - gcum[None, :])
                n = c1 - c0
                strict = np.tril(np.ones((n, n)), -1)
                incl = np.tril(np.ones((n, n)))
                lmat = strict * decay * (kc @ kc.T)
                rhs = bc[:, None] * (vc - np.exp(gcum)[:, None] * (kc @ st))
                u = np.linalg.solve(np.eye(n) + bc[:, None] * lmat, rhs)
                out[c0:c1, h] = scale * (np.exp(gcum)[:, None] * (qc @ st) + (incl * decay * (qc @ kc.T)) @ u)
                st = np.exp(gcum[-1]) * st + kc.T @ (np.exp(gcum[-1] - gcum)[:, None] * u)
            fin[b, h] = st
    return out, fin


def check_gated_delta_chunked_form(lin, seed=61):
    rng = np.random.default_rng(seed)
    lens = [13, 1, 20, 8]
    q, k, v, g, beta = _gdn_inputs(rng, lens, 2, 4, 6, 5, decay=(0.5, 1.0))
    cu = [0, 13, 14, 34, 42]
    o, fin = lin.gated_delta_rule(q, k, v, g, beta, cu, 0.4)
    for chunk in (1, 4, 7, 64):
        oc, fc = _gdn_chunked(q, k, v, g, beta, cu, 0.4, chunk)
        assert np.allclose(oc, o, rtol=1e-11, atol=1e-11), chunk
        assert np.allclose(fc, fin, rtol=1e-11, atol=1e-11), chunk


GDN_CHECKS = [
    check_golden_gated_delta,
    check_gated_delta_beta_zero,
    check_gated_delta_associative_recall,
    check_gated_delta_continuation_and_packing,
    check_gated_delta_linear_in_v,
    check_gated_delta_chunked_form,
]
