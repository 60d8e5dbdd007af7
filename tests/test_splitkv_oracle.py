"""Pins for the split-KV oracle (oracle/splitkv.py).

* the decomposition identity: partials over any partition of the key axis
  into contiguous ranges merge to the full oracle's O and LSE (the full
  oracle is pinned on its own in test_oracle.py), causal and not, GQA, rope,
  ragged with an empty sequence;
* brute force: pure-Python loops (math.exp / math.fsum) for a partial over a
  key range on a tiny input;
* special cases: the full range is the full attention; an empty range gives
  O = 0 and LSE = -inf; merging one non-empty partial with empty ones
  returns it; two equal partials merge to the same O and LSE + ln 2; the
  merge does not depend on the order of the partials; partials with LSE in
  the thousands merge without overflow;
* planted mistakes (merge weights without the max shift, unnormalised
  weights) fail these pins.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import splitkv as osk


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _case(rng, lens, hq, hkv, dn, dr, dv):
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q, k, v = _rand(rng, T, hq, dn), _rand(rng, T, hkv, dn), _rand(rng, T, hkv, dv)
    qr = _rand(rng, T, hq, dr) if dr else None
    kr = _rand(rng, T, hkv, dr) if dr else None
    return q, k, v, cu, qr, kr


def _ranges_for_cuts(cu, cuts_per_seq, T):
    """Per token [lo, hi) of each partition piece: piece p of sequence b spans
    keys [cuts[p], cuts[p+1])."""
    n = len(next(iter(cuts_per_seq.values()))) - 1
    lo = np.zeros((n, T), np.int64)
    hi = np.zeros((n, T), np.int64)
    for b in range(len(cu) - 1):
        c = cuts_per_seq[b]
        for p in range(n):
            lo[p, cu[b]:cu[b + 1]] = c[p]
            hi[p, cu[b]:cu[b + 1]] = c[p + 1]
    return lo, hi


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens,hq,hkv,dn,dr", [([37], 2, 2, 16, 0), ([20, 0, 45, 1], 4, 2, 8, 4),
                                               ([64], 4, 1, 8, 0)])
def test_partials_merge_to_full_attention(causal, lens, hq, hkv, dn, dr):
    rng = np.random.default_rng(len(lens) * 10 + hq)
    q, k, v, cu, qr, kr = _case(rng, lens, hq, hkv, dn, dr, 8)
    T = int(cu[-1])
    full_o, full_l = oracle.mha_forward(q, k, v, cu, causal, q_rope=qr, k_rope=kr)
    for n in (1, 2, 3, 5):
        cuts = {}
        for b, L in enumerate(lens):
            inner = np.sort(rng.integers(0, L + 1, n - 1)) if L else np.zeros(n - 1, np.int64)
            cuts[b] = np.concatenate([[0], inner, [L]])
        lo, hi = _ranges_for_cuts(cu, cuts, T)
        parts = [osk.mha_forward_key_range(q, k, v, cu, causal, lo[p], hi[p], q_rope=qr, k_rope=kr)
                 for p in range(n)]
        o, l = osk.merge_partials([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(o, full_o, atol=1e-12, rtol=0)
        assert np.allclose(l, full_l, atol=1e-12, rtol=0)


def test_partial_matches_brute_force():
    rng = np.random.default_rng(7)
    L, h, d = 6, 1, 3
    q, k, v = _rand(rng, L, h, d), _rand(rng, L, h, d), _rand(rng, L, h, d)
    cu = np.array([0, L])
    lo = np.array([1, 1, 2, 0, 3, 2])
    hi = np.array([4, 6, 3, 2, 6, 5])
    sigma = 1 / math.sqrt(d)
    for causal in (False, True):
        o, lse = osk.mha_forward_key_range(q, k, v, cu, causal, lo, hi)
        for i in range(L):
            js = [j for j in range(lo[i], hi[i]) if not causal or j <= i]
            if not js:
                assert lse[0, i] == -math.inf and np.all(o[i, 0] == 0)
                continue
            sc = [sigma * sum(q[i, 0, a] * k[j, 0, a] for a in range(d)) for j in js]
            z = math.fsum(math.exp(x) for x in sc)
            assert abs(lse[0, i] - math.log(z)) < 1e-12
            for a in range(d):
                ref = math.fsum(math.exp(x) * v[j, 0, a] for x, j in zip(sc, js)) / z
                assert abs(o[i, 0, a] - ref) < 1e-12


def test_special_cases():
    rng = np.random.default_rng(8)
    q, k, v, cu, _, _ = _case(rng, [30, 9], 2, 2, 8, 0, 8)
    T = int(cu[-1])
    full = oracle.mha_forward(q, k, v, cu, True)
    whole = osk.mha_forward_key_range(q, k, v, cu, True, np.zeros(T, int), np.full(T, 10 ** 6))
    assert np.allclose(whole[0], full[0], atol=1e-13) and np.allclose(whole[1], full[1], atol=1e-13)
    empty = osk.mha_forward_key_range(q, k, v, cu, False, np.full(T, 5), np.full(T, 5))
    assert np.all(empty[0] == 0) and np.all(empty[1] == -np.inf)
    o, l = osk.merge_partials([empty[0], whole[0], empty[0]], [empty[1], whole[1], empty[1]])
    assert np.allclose(o, whole[0], atol=1e-15) and np.array_equal(l, whole[1])
    o2, l2 = osk.merge_partials([whole[0], whole[0]], [whole[1], whole[1]])
    assert np.allclose(o2, whole[0], atol=1e-14) and np.allclose(l2, whole[1] + math.log(2), atol=1e-14)
    oe, le = osk.merge_partials([empty[0]], [empty[1]])
    assert np.all(oe == 0) and np.all(le == -np.inf)


def test_merge_order_and_large_lse():
    rng = np.random.default_rng(9)
    n, T, H, D = 4, 5, 3, 6
    op = rng.standard_normal((n, T, H, D))
    lp = rng.standard_normal((n, H, T)) * 3 + 1000.0
    o, l = osk.merge_partials(op, lp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    perm = rng.permutation(n)
    o2, l2 = osk.merge_partials(op[perm], lp[perm])
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(l, l2, atol=1e-12)
    # against the definition written with a shift by hand
    for h in range(H):
        for t in range(T):
            m = lp[:, h, t].max()
            z = math.fsum(math.exp(x - m) for x in lp[:, h, t])
            assert abs(l[h, t] - (m + math.log(z))) < 1e-9
            ref = sum(math.exp(lp[s, h, t] - m) / z * op[s, t, h] for s in range(n))
            assert np.allclose(o[t, h], ref, atol=1e-12)


@pytest.mark.parametrize("mutant", ["no_shift", "unnormalised"])
def test_planted_mistakes_fail_pins(mutant, monkeypatch):
    def bad(o_parts, lse_parts):
        o_parts, lse_parts = np.asarray(o_parts, float), np.asarray(lse_parts, float)
        with np.errstate(all="ignore"):
            w = np.exp(lse_parts)
            total = w.sum(axis=0)
            lse = np.log(total)
            wn = w if mutant == "unnormalised" else w / total[None]
            return np.einsum("nht,nthd->thd", wn, o_parts), lse
    monkeypatch.setattr(osk, "merge_partials", bad)
    with pytest.raises(AssertionError):
        if mutant == "no_shift":
            test_merge_order_and_large_lse()
        else:
            test_partials_merge_to_full_attention(True, [37], 2, 2, 16, 0)
