"""Pins for the CPU oracle: facts the definition of the gated delta rule fixes
independently of the oracle's own code.

Each ``pin_*`` function takes ``upd`` (``oracle.update`` or the same call on
another build of the oracle source) and raises AssertionError when the oracle
disagrees.  The expected values come from hand-derived worked examples, closed
forms of the gates (written differently from the definition: a power instead
of exp-of-softplus, symmetric exponentials for the logistic), algebraic invariants of one
update, an independent numpy matrix form, and structural properties (GQA,
chaining, varlen, padding).

The pages name the fused gating + delta-rule update and its inputs (vLLM PR
#35777, implementation section: A_log, a, b, dt_bias; rsqrt normalisation;
speculative decoding with per-token states) but print neither its equations
nor any worked example, so every value here is derived from the definition.
"""
from __future__ import annotations

import numpy as np

f32 = np.float32


def _one_seq(upd, q, k, v, a, b, A_log, dt_bias, S0, **kw):
    """Single sequence of T tokens in slot 0.  q, k: [T, Hk, K]; v: [T, Hv, V];
    a, b: [T, Hv]; S0: [Hv, K, V].  Returns (out [T,Hv,V] f64, S [Hv,K,V] f32,
    inter or None)."""
    T = q.shape[0]
    pool = np.ascontiguousarray(S0[None], dtype=f32).copy()
    out, inter = upd(q, k, v, a, b, A_log, dt_bias, pool,
                     np.array([0], np.int32), None, tokens_per_seq=T, **kw)
    return out, pool[0], inter


def _close(x, ref, rtol, what):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(float(np.max(np.abs(ref))), 1e-300)
    err = float(np.max(np.abs(x - ref))) / scale
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    assert err <= rtol, f"{what}: relative error {err:.3e} > {rtol:.1e}"


def gamma_closed_form(A_log, x):
    """exp(-e^A_log * log(1 + e^x)) written as (1 + e^x)^(-e^A_log)."""
    return np.power(1.0 + np.exp(np.float64(x)), -np.exp(np.float64(A_log)))


def beta_closed_form(b):
    """The logistic function as a ratio of symmetric exponentials,
    e^(b/2) / (e^(b/2) + e^(-b/2)) (accurate in both tails for |b| < 1400)."""
    h = 0.5 * np.float64(b)
    return np.exp(h) / (np.exp(h) + np.exp(-h))


# ---------------------------------------------------------------------------
def pin_worked_example(upd):
    """K = V = 2, two tokens, hand-derived.  A_log = 0 and a + dt_bias = 0
    give gamma = (1+1)^-1 = 1/2; b = 0 gives beta = 1/2; scale = 1, eps = 0.
    3-4-5 and axis-aligned vectors make every norm exact.

    token 0: k = (3,4) -> khat = (.6,.8); q = (0,5) -> qhat = (0,1); v = (1,-1)
      gamma*S0 = [[.5,1],[1.5,2]];  S^T khat = (1.5, 2.2)
      u = .5*((1,-1) - (1.5,2.2)) = (-.25,-1.6)
      S1 = [[.5-.15, 1-.96],[1.5-.2, 2-1.28]] = [[.35,.04],[1.3,.72]]
      o0 = S1^T qhat = (1.3, .72)
    token 1: k = (0,2) -> khat = (0,1); q = (1,0) -> qhat = (1,0); v = (2,2)
      gamma*S1 = [[.175,.02],[.65,.36]];  S^T khat = (.65,.36)
      u = .5*((2,2) - (.65,.36)) = (.675,.82)
      S2 = [[.175,.02],[1.325,1.18]];  o1 = S2^T qhat = (.175,.02)
    """
    q = np.array([[[0.0, 5.0]], [[1.0, 0.0]]])
    k = np.array([[[3.0, 4.0]], [[0.0, 2.0]]])
    v = np.array([[[1.0, -1.0]], [[2.0, 2.0]]])
    z = np.zeros((2, 1))
    S0 = np.array([[[1.0, 2.0], [3.0, 4.0]]])
    out, S, inter = _one_seq(upd, q, k, v, z, z, np.zeros(1), np.zeros(1), S0,
                             scale=1.0, eps=0.0, intermediates=True)
    _close(out[0, 0], [1.3, 0.72], 1e-14, "worked example o0")
    _close(out[1, 0], [0.175, 0.02], 1e-13, "worked example o1")
    _close(inter[0, 0], [[0.35, 0.04], [1.3, 0.72]], 1e-7, "worked example S1")
    _close(S[0], [[0.175, 0.02], [1.325, 1.18]], 1e-7, "worked example S2")


def pin_gamma_closed_form(upd):
    """With beta = 0 (b = -1000) the update is a pure decay, so o = gamma *
    S0^T qhat exactly; gamma must equal (1 + e^x)^(-e^A_log) for every x,
    including the far tails of softplus, and 1/4 exactly at x = 0,
    A_log = log 2."""
    rng = np.random.default_rng(11)
    xs = np.array([-30.0, -5.0, -1.0, 0.0, 0.0, 0.5, 3.0, 25.0])
    A_log = np.array([0.3, 1.2, -0.7, np.log(2.0), 0.0, 2.5, np.log(16.0), -2.0])
    Hv, K, V = len(xs), 4, 3
    dt_bias = np.linspace(-0.4, 0.6, Hv)
    a = (xs - dt_bias)[None, :]
    b = np.full((1, Hv), -1000.0)
    q = rng.standard_normal((1, 1, K))
    k = rng.standard_normal((1, 1, K))
    v = rng.standard_normal((1, Hv, V))
    S0 = rng.standard_normal((Hv, K, V)).astype(f32)
    out, S, _ = _one_seq(upd, q, k, v, a, b, A_log, dt_bias, S0, eps=0.0)
    qhat = q[0, 0] / np.linalg.norm(q[0, 0]) / np.sqrt(K)
    a_plus = a[0] + dt_bias
    for h in range(Hv):
        base = S0[h].astype(np.float64).T @ qhat
        g_ref = gamma_closed_form(A_log[h], a_plus[h])
        _close(out[0, h], g_ref * base, 1e-12, f"pure decay output, head {h}")
        _close(S[h], (g_ref * S0[h].astype(np.float64)), 1e-7, f"pure decay state, head {h}")
    g4 = out[0, 3] / (S0[3].astype(np.float64).T @ qhat)
    _close(g4, np.full(V, 0.25), 1e-13, "gamma(x=0, A=2) = 1/4")


def pin_beta_closed_form(upd):
    """From a zero state with q = k (so qhat.khat = scale when eps = 0):
    o = beta * scale * v.  beta must be the logistic function of b, 1/2 at
    b = 0 and 3/4 at b = log 3."""
    Hv, K, V = 7, 8, 4
    bs = np.array([-40.0, -2.0, 0.0, np.log(3.0), 1.5, 30.0, 700.0])
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 1, K))
    v = rng.uniform(0.5, 2.0, (1, Hv, V))
    a = rng.standard_normal((1, Hv))
    S0 = np.zeros((Hv, K, V), f32)
    out, S, _ = _one_seq(upd, q, q.copy(), v, a, bs[None, :], np.zeros(Hv),
                         np.zeros(Hv), S0, eps=0.0)
    scale = 1.0 / np.sqrt(K)
    for h in range(Hv):
        _close(out[0, h], beta_closed_form(bs[h]) * scale * v[0, h], 1e-13,
               f"beta closed form, b={bs[h]}")
    _close(out[0, 2], 0.5 * scale * v[0, 2], 1e-15, "beta(0) = 1/2")
    _close(out[0, 3], 0.75 * scale * v[0, 3], 1e-14, "beta(log 3) = 3/4")


def pin_unit_write(upd):
    """gamma = 1 (A_log = -1000 makes e^A_log = 0), beta = 1 (b = 1000),
    eps = 0: one update writes v exactly along khat, S'^T khat = v.  With
    q = k the output is scale * S'^T khat = scale * v."""
    rng = np.random.default_rng(13)
    Hv, K, V = 2, 6, 5
    q = rng.standard_normal((1, 1, K))
    v = rng.standard_normal((1, Hv, V))
    a = rng.standard_normal((1, Hv))
    S0 = rng.standard_normal((Hv, K, V)).astype(f32)
    out, S, _ = _one_seq(upd, q, q.copy(), v, a, np.full((1, Hv), 1000.0),
                         np.full(Hv, -1000.0), np.zeros(Hv), S0, eps=0.0)
    khat = q[0, 0] / np.linalg.norm(q[0, 0])
    _close(out[0], v[0] / np.sqrt(K), 1e-12, "unit write output")
    for h in range(Hv):
        _close(S[h].astype(np.float64).T @ khat, v[0, h], 1e-6, "unit write state")


def pin_write_and_orthogonal_complement(upd):
    """Any gate, eps = 0: S'^T khat = (1-beta) gamma S0^T khat + beta v, and
    for w orthogonal to khat, S'^T w = gamma S0^T w.  Probed through the
    fp64 output with q = k and q = w."""
    rng = np.random.default_rng(14)
    Hv, K, V = 3, 8, 6
    k = rng.standard_normal((1, 1, K))
    w = rng.standard_normal(K)
    khat = k[0, 0] / np.linalg.norm(k[0, 0])
    w = w - (w @ khat) * khat
    what = w / np.linalg.norm(w)
    v = rng.standard_normal((1, Hv, V))
    a = rng.standard_normal((1, Hv))
    b = rng.standard_normal((1, Hv))
    A_log = rng.uniform(-1.0, 1.0, Hv)
    dt = rng.standard_normal(Hv) * 0.5
    S0 = rng.standard_normal((Hv, K, V)).astype(f32)
    scale = 1.0 / np.sqrt(K)
    outk, _, _ = _one_seq(upd, k, k.copy(), v, a, b, A_log, dt, S0, eps=0.0)
    outw, _, _ = _one_seq(upd, w[None, None, :], k, v, a, b, A_log, dt, S0, eps=0.0)
    for h in range(Hv):
        g = gamma_closed_form(A_log[h], a[0, h] + dt[h])
        be = beta_closed_form(b[0, h])
        S0h = S0[h].astype(np.float64)
        _close(outk[0, h], scale * ((1 - be) * g * (S0h.T @ khat) + be * v[0, h]),
               1e-12, "write along khat")
        _close(outw[0, h], scale * g * (S0h.T @ what), 1e-12, "orthogonal complement")


def pin_zero_state_output(upd):
    """From S0 = 0 the first output is beta (qhat . khat) v, with qhat carrying
    the default K^-1/2 scale."""
    rng = np.random.default_rng(15)
    Hk, Hv, K, V = 2, 4, 16, 8
    q = rng.standard_normal((1, Hk, K))
    k = rng.standard_normal((1, Hk, K))
    v = rng.standard_normal((1, Hv, V))
    a = rng.standard_normal((1, Hv))
    b = rng.standard_normal((1, Hv))
    out, _, _ = _one_seq(upd, q, k, v, a, b, rng.uniform(0, 2, Hv),
                         rng.standard_normal(Hv), np.zeros((Hv, K, V), f32), eps=0.0)
    G = Hv // Hk
    for h in range(Hv):
        j = h // G
        cos = (q[0, j] @ k[0, j]) / (np.linalg.norm(q[0, j]) * np.linalg.norm(k[0, j]))
        _close(out[0, h], beta_closed_form(b[0, h]) * cos / np.sqrt(K) * v[0, h],
               1e-12, f"zero-state output head {h}")


def pin_eps_inside_root(upd):
    """eps sits inside the root: with |k|^2 = eps and q = k from a zero state,
    qhat.khat = scale * |k|^2/(|k|^2+eps) = scale/2."""
    K, V = 4, 3
    eps = 1e-6
    k = np.full((1, 1, K), np.sqrt(eps / K))
    v = np.array([[[1.0, -2.0, 0.5]]])
    out, _, _ = _one_seq(upd, k, k.copy(), v, np.zeros((1, 1)), np.zeros((1, 1)),
                         np.zeros(1), np.zeros(1), np.zeros((1, K, V), f32), eps=eps)
    _close(out[0, 0], 0.5 * 0.5 / np.sqrt(K) * v[0, 0], 1e-12, "eps inside the root")


def _matrix_form(q, k, v, a, b, A_log, dt, S0, G, scale, eps):
    """Independent numpy form: S' = gamma (I - beta khat khat^T) S + beta khat v^T,
    o = S'^T qhat, over the tokens of one sequence."""
    T, Hv = a.shape
    K = q.shape[2]
    S = S0.astype(np.float64).copy()
    outs = np.zeros((T, Hv, v.shape[2]))
    for t in range(T):
        for h in range(Hv):
            j = h // G
            kh = k[t, j] / np.sqrt(np.sum(k[t, j] ** 2) + eps)
            qh = scale * q[t, j] / np.sqrt(np.sum(q[t, j] ** 2) + eps)
            g = gamma_closed_form(A_log[h], a[t, h] + dt[h])
            be = beta_closed_form(b[t, h])
            P = np.eye(K) - be * np.einsum("i,j->ij", kh, kh)
            S[h] = g * np.einsum("ij,jv->iv", P, S[h]) + be * np.einsum("i,v->iv", kh, v[t, h])
            outs[t, h] = np.einsum("iv,i->v", S[h], qh)
    return outs, S


def pin_matrix_form(upd):
    """Varlen batch with GQA (G = 3) and K != V against the numpy matrix form
    of the update, token by token."""
    rng = np.random.default_rng(16)
    Hk, Hv, K, V = 2, 6, 5, 3
    lens = [3, 1, 4]
    N = sum(lens)
    q = rng.standard_normal((N, Hk, K))
    k = rng.standard_normal((N, Hk, K))
    v = rng.standard_normal((N, Hv, V))
    a = rng.standard_normal((N, Hv))
    b = rng.standard_normal((N, Hv))
    A_log = rng.uniform(-2, 1, Hv)
    dt = rng.standard_normal(Hv) * 0.5
    slots = np.array([4, 0, 2], np.int32)
    pool = rng.standard_normal((5, Hv, K, V)).astype(f32)
    pool0 = pool.copy()
    cu = np.array([0, 3, 4, 8], np.int32)
    eps = 1e-6
    out, _ = upd(q, k, v, a, b, A_log, dt, pool, slots, cu, eps=eps)
    for i, L in enumerate(lens):
        t0 = cu[i]
        ref_o, ref_S = _matrix_form(q[t0:t0 + L], k[t0:t0 + L], v[t0:t0 + L],
                                    a[t0:t0 + L], b[t0:t0 + L], A_log, dt,
                                    pool0[slots[i]], Hv // Hk, 1 / np.sqrt(K), eps)
        _close(out[t0:t0 + L], ref_o, 1e-12, f"matrix form output, seq {i}")
        _close(pool[slots[i]], ref_S, 1e-7, f"matrix form state, seq {i}")
    for s in (1, 3):
        assert np.array_equal(pool[s], pool0[s]), "unreferenced slot changed"


def pin_chain(upd):
    """A T-token call equals T chained one-token calls (state rounded to fp32
    between calls, hence a 1e-6 bound)."""
    rng = np.random.default_rng(17)
    for (Hk, Hv, K, V, T) in [(1, 1, 4, 4, 5), (1, 2, 8, 3, 4), (2, 2, 3, 8, 2)]:
        q = rng.standard_normal((T, Hk, K))
        k = rng.standard_normal((T, Hk, K))
        v = rng.standard_normal((T, Hv, V))
        a = rng.standard_normal((T, Hv))
        b = rng.standard_normal((T, Hv))
        A_log = rng.uniform(-3, 0, Hv)
        dt = rng.standard_normal(Hv) * 0.5
        S0 = rng.standard_normal((Hv, K, V)).astype(f32)
        out_all, S_all, inter = _one_seq(upd, q, k, v, a, b, A_log, dt, S0,
                                         intermediates=True)
        S = S0.copy()
        for t in range(T):
            o_t, S, _ = _one_seq(upd, q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1],
                                 b[t:t + 1], A_log, dt, S)
            _close(o_t[0], out_all[t], 1e-6, f"chained output t={t}")
            _close(S, inter[t], 1e-6, f"chained state vs intermediate t={t}")
        _close(S, S_all, 1e-6, "chained final state")
        assert np.array_equal(inter[T - 1], S_all), "last intermediate != final state"


def _batch(rng, B, Hk, Hv, K, V, lens, slots_total):
    N = int(sum(lens))
    d = dict(q=rng.standard_normal((N, Hk, K)), k=rng.standard_normal((N, Hk, K)),
             v=rng.standard_normal((N, Hv, V)), a=rng.standard_normal((N, Hv)),
             b=rng.standard_normal((N, Hv)), A_log=rng.uniform(-2, 1, Hv),
             dt_bias=rng.standard_normal(Hv) * 0.5)
    pool = rng.standard_normal((slots_total, Hv, K, V)).astype(f32)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    return d, pool, cu


def pin_gqa_is_mha(upd):
    """GQA equals MHA with each k-head's q/k repeated for its G v-heads."""
    rng = np.random.default_rng(18)
    Hk, Hv, K, V = 2, 8, 6, 5
    G = Hv // Hk
    d, pool, cu = _batch(rng, 2, Hk, Hv, K, V, [2, 3], 3)
    idx = np.array([2, 0], np.int32)
    p1, p2 = pool.copy(), pool.copy()
    o1, _ = upd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                p1, idx, cu)
    qm = np.repeat(d["q"], G, axis=1)
    km = np.repeat(d["k"], G, axis=1)
    o2, _ = upd(qm, km, d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], p2, idx, cu)
    assert np.array_equal(o1, o2), "GQA output differs from repeated-head MHA"
    assert np.array_equal(p1, p2), "GQA state differs from repeated-head MHA"


def pin_scale_invariance(upd):
    """With eps = 0 the output does not depend on the lengths of q and k."""
    rng = np.random.default_rng(19)
    d, pool, cu = _batch(rng, 2, 1, 2, 8, 4, [3, 2], 2)
    idx = np.array([1, 0], np.int32)
    p1, p2 = pool.copy(), pool.copy()
    o1, _ = upd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                p1, idx, cu, eps=0.0)
    o2, _ = upd(3.7 * d["q"], 0.21 * d["k"], d["v"], d["a"], d["b"], d["A_log"],
                d["dt_bias"], p2, idx, cu, eps=0.0)
    _close(o2, o1, 1e-12, "q/k scale invariance")
    _close(p2, p1, 1e-7, "q/k scale invariance (state)")


def pin_structure(upd):
    """Permuting sequences with their slots permutes the results; a varlen
    batch equals each sequence alone; padded (-1) and zero-length sequences
    touch nothing and leave the rest bit-identical; the last intermediate is
    the final state; NO_FINAL_WRITEBACK leaves the pool as it was."""
    rng = np.random.default_rng(20)
    Hk, Hv, K, V = 2, 4, 4, 6
    lens = [2, 3, 1, 4]
    d, pool, cu = _batch(rng, 4, Hk, Hv, K, V, lens, 7)
    idx = np.array([5, 1, 6, 3], np.int32)
    args = lambda dd: (dd["q"], dd["k"], dd["v"], dd["a"], dd["b"], dd["A_log"], dd["dt_bias"])
    p_ref = pool.copy()
    o_ref, i_ref = upd(*args(d), p_ref, idx, cu, intermediates=True)
    # each sequence alone
    for i, L in enumerate(lens):
        t0, t1 = cu[i], cu[i + 1]
        di = {n: (x[t0:t1] if x.ndim >= 2 else x) for n, x in d.items()}
        pi = pool.copy()
        oi, _ = upd(*args(di), pi, idx[i:i + 1], np.array([0, L], np.int32))
        assert np.array_equal(oi, o_ref[t0:t1]), f"varlen seq {i} differs when run alone"
        assert np.array_equal(pi[idx[i]], p_ref[idx[i]]), f"varlen seq {i} state differs"
    # permutation of sequences (with their tokens and slots)
    perm = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in perm])
    dp = {n: (x[rows] if x.ndim >= 2 else x) for n, x in d.items()}
    cup = np.zeros(5, np.int32)
    cup[1:] = np.cumsum([lens[i] for i in perm])
    pp = pool.copy()
    op, _ = upd(*args(dp), pp, idx[perm], cup)
    assert np.array_equal(op, o_ref[rows]), "permuted batch output"
    assert np.array_equal(pp, p_ref), "permuted batch state"
    # padding and a zero-length sequence
    idx_pad = np.array([5, -1, 1, 6, 0, 3], np.int32)
    lens_pad = [2, 2, 3, 1, 0, 4]
    rows_pad = np.concatenate([np.arange(cu[0], cu[1]), np.arange(cu[1], cu[1] + 2),
                               np.arange(cu[1], cu[4])])
    dpad = {n: (x[rows_pad] if x.ndim >= 2 else x) for n, x in d.items()}
    cupad = np.zeros(7, np.int32)
    cupad[1:] = np.cumsum(lens_pad)
    ppad = pool.copy()
    opad, ipad = upd(*args(dpad), ppad, idx_pad, cupad, intermediates=True)
    live_rows = np.r_[0:2, 4:12]
    assert np.array_equal(opad[live_rows], o_ref), "padding changed live outputs"
    assert np.all(np.isnan(opad[2:4])), "padded sequence wrote outputs"
    assert np.all(np.isnan(ipad[2:4])), "padded sequence wrote intermediates"
    assert np.array_equal(ppad, p_ref), "padding or a zero-length sequence changed the pool"
    # last intermediate equals the final state, bitwise
    for i in range(4):
        assert np.array_equal(i_ref[cu[i + 1] - 1], p_ref[idx[i]]), "last intermediate"
    # no final write-back
    pn = pool.copy()
    on, inn = upd(*args(d), pn, idx, cu, intermediates=True, no_final_writeback=True)
    assert np.array_equal(pn, pool), "NO_FINAL_WRITEBACK changed the pool"
    assert np.array_equal(on, o_ref) and np.array_equal(inn, i_ref, equal_nan=True)
    # empty batch
    pe = pool.copy()
    oe, _ = upd(d["q"][:0], d["k"][:0], d["v"][:0], d["a"][:0], d["b"][:0], d["A_log"],
                d["dt_bias"], pe, np.zeros(0, np.int32), np.zeros(1, np.int32))
    assert oe.shape[0] == 0 and np.array_equal(pe, pool), "empty batch"


def pin_state_layouts(upd):
    """The transposed storage order ("VK": K fastest) holds the same state:
    running on the transposed pool gives the same outputs bit for bit and the
    transposed final states and intermediates."""
    rng = np.random.default_rng(21)
    Hk, Hv, K, V = 2, 4, 6, 5
    lens = [3, 1, 2]
    d, pool, cu = _batch(rng, 3, Hk, Hv, K, V, lens, 4)
    idx = np.array([3, -1, 0], np.int32)
    args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"])
    p_kv = pool.copy()
    o_kv, i_kv = upd(*args, p_kv, idx, cu, intermediates=True)
    p_vk = np.ascontiguousarray(pool.transpose(0, 1, 3, 2))
    o_vk, i_vk = upd(*args, p_vk, idx, cu, intermediates=True, state_layout="VK")
    assert np.array_equal(o_kv, o_vk, equal_nan=True), "layouts give different outputs"
    assert np.array_equal(p_vk, p_kv.transpose(0, 1, 3, 2)), "layouts give different states"
    assert np.array_equal(i_vk, i_kv.transpose(0, 1, 3, 2), equal_nan=True)


def pin_gating_step(upd):
    """The standalone gating step: exp(g) = (1 + e^x)^(-e^A_log) and beta is the
    logistic of b, per (token, head), over both tails of softplus."""
    import functools
    import oracle
    lib = getattr(upd, "keywords", {}).get("lib_path")
    gate = functools.partial(oracle.gating, lib_path=lib) if lib else oracle.gating
    xs = np.array([[-30.0, -1.0, 0.0, 0.5], [3.0, 25.0, -5.0, 0.0]])
    A_log = np.array([0.3, np.log(2.0), -0.7, 2.5])
    dt = np.array([0.1, -0.2, 0.3, 0.0])
    bs = np.array([[-40.0, 0.0, np.log(3.0), 2.0], [30.0, -2.0, 1.5, -0.5]])
    g, beta = gate(xs - dt, bs, A_log, dt)
    _close(np.exp(g), gamma_closed_form(A_log[None, :], xs), 1e-13, "gating step: exp(g)")
    _close(beta, beta_closed_form(bs), 1e-14, "gating step: beta")
    assert abs(np.exp(g[0, 2]) - 0.5 ** np.exp(-0.7)) < 1e-15  # x = 0: (1+1)^(-A)


def _bf16_bits(x):
    """bf16 bit patterns of values that are exactly bf16 (no rounding here)."""
    u = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _from_bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def pin_bf16_state_storage(upd):
    """bf16 state storage on the worked example: the state stays in double
    between tokens and every stored element is the exact value rounded once to
    the nearest bf16 (8 significant bits), hand-derived:
      S1 = [[.35, .04], [1.3, .72]]   -> [[179/512, 41/1024], [83/64, 23/32]]
      S2 = [[.175, .02], [1.325, 1.18]] -> [[179/1024, 41/2048], [85/64, 151/128]]
    (1.325*64 = 84.8 rounds up to 85; 0.175*1024 = 179.2 rounds down)."""
    q = np.array([[[0.0, 5.0]], [[1.0, 0.0]]])
    k = np.array([[[3.0, 4.0]], [[0.0, 2.0]]])
    v = np.array([[[1.0, -1.0]], [[2.0, 2.0]]])
    z = np.zeros((2, 1))
    pool = _bf16_bits([[[[1.0, 2.0], [3.0, 4.0]]]])
    out, inter = upd(q, k, v, z, z, np.zeros(1), np.zeros(1), pool, np.array([0], np.int32),
                     None, tokens_per_seq=2, scale=1.0, eps=0.0, intermediates=True)
    assert inter.dtype == np.uint16
    s1 = np.array([[179 / 512, 41 / 1024], [83 / 64, 23 / 32]])
    s2 = np.array([[179 / 1024, 41 / 2048], [85 / 64, 151 / 128]])
    assert np.array_equal(_from_bf16(inter[0, 0]), s1.astype(np.float32)), "bf16 S1"
    assert np.array_equal(_from_bf16(pool[0, 0]), s2.astype(np.float32)), "bf16 final state"
    assert np.array_equal(inter[1], pool[0]), "last intermediate != final state (bf16)"
    _close(out[1, 0], [0.175, 0.02], 1e-13, "bf16 storage leaves the outputs in double")


# (value written to the state, bf16 bit pattern it must be stored as), derived
# by hand from round-to-nearest-even with 8 significant bits, the subnormal
# quantum 2^-133 below 2^-126 and overflow to infinity from the midpoint
# between the largest finite bf16 (2 - 2^-7) 2^127 and 2^128 on.
BF16_ROUNDING_EDGES = [
    (3 * 2.0 ** -135, 0x0001),                  # 0.75 quantum rounds up to the smallest subnormal
    (2.0 ** -134, 0x0000),                      # half a quantum: tie to even (zero)
    (3 * 2.0 ** -134, 0x0002),                  # 1.5 quanta: tie to even (2)
    (-5 * 2.0 ** -134, 0x8002),                 # -2.5 quanta: tie to even, sign kept
    (2.0 ** -126 - 2.0 ** -133, 0x007F),        # largest subnormal, exact
    (2.0 ** -126 - 2.0 ** -134, 0x0080),        # 127.5 quanta: tie to even = smallest normal
    (-2.0 ** -150, 0x8000),                     # rounds to zero and keeps the sign
    (1.0 + 2.0 ** -8, 0x3F80),                  # tie between 1 and 1 + 2^-7: even is 1
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # tie between 1 + 2^-7 and 1 + 2^-6: even is the latter
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),     # just above the tie (a float detour would lose it)
    ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),   # largest finite bf16, exact
    (2.0 ** 128 - 2.0 ** 119 - 2.0 ** 90, 0x7F7F),  # just below the overflow midpoint
    (2.0 ** 128 - 2.0 ** 119, 0x7F80),          # the midpoint: tie to even overflows to +inf
    (-1e300, 0xFF80),                           # far beyond the range: -inf
]


def pin_bf16_rounding_edges(upd):
    """bf16 storage rounds the double-precision state once, to nearest even,
    through the subnormal range and into overflow.  K = 1, a unit key, eps = 0,
    beta = 1 (b = +1000) and gamma = 1 (A_log = -1000, so e^A_log is 0) from a
    zero state make the stored state exactly v: S' = 0 + khat (1 (v - 0)) = v.
    Each v is then stored as the hand-derived bit pattern above, in the pool
    and in the intermediate state alike."""
    vals = np.array([x for x, _ in BF16_ROUNDING_EDGES], np.float64)
    want = np.array([b for _, b in BF16_ROUNDING_EDGES], np.uint16)
    n = vals.size
    one = np.ones((1, 1, 1))
    pool = np.zeros((1, 1, 1, n), np.uint16)   # bf16 zeros
    out, inter = upd(one, one, vals.reshape(1, 1, n), np.zeros((1, 1)), np.full((1, 1), 1000.0),
                     np.full(1, -1000.0), np.zeros(1), pool, np.array([0], np.int32), None,
                     tokens_per_seq=1, scale=1.0, eps=0.0, intermediates=True)
    got = pool[0, 0, 0]
    bad = [f"{vals[i]!r} -> {got[i]:#06x}, want {want[i]:#06x}" for i in range(n) if got[i] != want[i]]
    assert not bad, "bf16 rounding: " + "; ".join(bad)
    assert np.array_equal(inter[0, 0, 0], want), "bf16 rounding of the intermediate state"
    assert np.array_equal(out[0, 0], vals), "the output stays in double (q = k, o = S^T qhat = v)"


ALL_PINS = [pin_worked_example, pin_gamma_closed_form, pin_beta_closed_form,
            pin_unit_write, pin_write_and_orthogonal_complement,
            pin_zero_state_output, pin_eps_inside_root, pin_matrix_form,
            pin_chain, pin_gqa_is_mha, pin_scale_invariance, pin_structure,
            pin_state_layouts, pin_gating_step, pin_bf16_state_storage,
            pin_bf16_rounding_edges]
