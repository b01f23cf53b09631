"""Pins for the FP64 oracle: checks against facts fixed by the mathematics, not by the oracle.

Each pin takes an oracle library handle (the real one, or a deliberately broken copy in the
mutation test) and raises AssertionError when the handle disagrees with the fact.

The facts used:
  * finite differences of the oracle's own forward (pins the hand-derived reverse mode,
    given that the forward is pinned by the rest);
  * an overwrite identity of the delta rule with decay before the correction: with
    beta = 1 and a unit key, S_t^T k_t = v_t whatever S_{t-1} and the decay are;
  * closed forms: beta = 0 (pure decay), one token (the transition matrix
    a (I - b k k^T) S + b k v^T), orthonormal keys with beta = 1 (exact store and decayed
    recall), and the transfer matrix of the state map for dh0;
  * structure: linearity in (v, h0), packed documents equal separate runs, a document split
    into fragments chained through ht/h0, grouped heads equal repeated heads, chunked form
    equal to the token recurrence.
"""
from __future__ import annotations

import numpy as np

import oracle


def rand_problem(rng, lengths, H, HV, dk, dv, h0=True, dht=True, scale_g=1.0):
    T = int(sum(lengths))
    N = len(lengths)
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    f = np.float32
    p = dict(
        cu=cu,
        q=rng.standard_normal((T, H, dk)).astype(f),
        k=rng.standard_normal((T, H, dk)).astype(f),
        v=rng.standard_normal((T, HV, dv)).astype(f),
        beta=(1.0 / (1.0 + np.exp(-rng.standard_normal((T, HV))))).astype(f),
        g=(-np.log1p(np.exp(-(rng.standard_normal((T, HV)) + 3.0))) * scale_g).astype(f),
        h0=(0.5 * rng.standard_normal((N, HV, dk, dv))).astype(f) if h0 else None,
        dO=rng.standard_normal((T, HV, dv)).astype(f),
        dht=(0.5 * rng.standard_normal((N, HV, dk, dv))).astype(f) if dht else None,
    )
    return p


def _fwd(lib, p, l2norm, **kw):
    return oracle.fwd(p["cu"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"], l2norm=l2norm, lib=lib,
                      threads=1, **kw)


def _bwd(lib, p, l2norm):
    return oracle.bwd(p["cu"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["dO"], p["h0"], p["dht"],
                      l2norm=l2norm, lib=lib, threads=1)


def _loss(lib, p, l2norm):
    o, ht = _fwd(lib, p, l2norm)
    val = float(np.sum(o * p["dO"].astype(np.float64)))
    if p["dht"] is not None:
        val += float(np.sum(ht * p["dht"].astype(np.float64)))
    return val


def _unit_rows(x, eps=1e-6):
    """x / sqrt(x.x + eps) row by row: the L2 norm with the same eps the kernel and oracle use."""
    x = x.astype(np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


# --------------------------------------------------------------------------------------------
# reverse mode


def pin_finite_differences(lib, l2norm=True, seed=0, tol=2e-5):
    """Every gradient entry equals a central difference of the FP64 forward.

    Two documents (5 + 7 tokens, so the check crosses a document boundary), grouped heads
    (H = 2, HV = 4), dk != dv so a transposed state is caught, nonzero h0 and dht.
    """
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [5, 7], H=2, HV=4, dk=4, dv=3)
    grads = _bwd(lib, p, l2norm)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("h0", "dh0")]
    for name, gname in names:
        x = p[name]
        flat = x.reshape(-1)
        fd = np.zeros(flat.shape, np.float64)
        for i in range(flat.size):
            x0 = flat[i]
            h = np.float32(2.0 ** -9) * max(np.float32(1.0), abs(x0))
            flat[i] = x0 + h
            xp = float(flat[i])
            lp = _loss(lib, p, l2norm)
            flat[i] = x0 - h
            xm = float(flat[i])
            lm = _loss(lib, p, l2norm)
            flat[i] = x0
            fd[i] = (lp - lm) / (xp - xm)
        an = grads[gname].reshape(-1)
        err = np.max(np.abs(fd - an)) / max(1e-12, np.max(np.abs(an)))
        assert err < tol, "%s: finite-difference mismatch %.3e" % (gname, err)


def pin_directional_derivative(lib, seed=1, tol=1e-6):
    """<grad, dx> equals the directional derivative (f(x + e dx) - f(x - e dx)) / 2e on a larger case."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [37, 64, 29], H=2, HV=6, dk=8, dv=16)
    grads = _bwd(lib, p, True)
    dirs = {n: rng.standard_normal(p[n].shape) for n in ("q", "k", "v", "g", "beta", "h0")}
    an = sum(float(np.sum(grads["d" + n if n != "beta" else "dbeta"] * dirs[n])) for n in dirs)
    # perturb in float64 through the float32 interface: use a step large enough to be exact-ish
    eps = 2.0 ** -12
    base = {n: p[n].copy() for n in dirs}
    vals = []
    for s in (+1, -1):
        actual = {}
        for n in dirs:
            p[n] = (base[n].astype(np.float64) + s * eps * dirs[n]).astype(np.float32)
            actual[n] = p[n].astype(np.float64) - base[n].astype(np.float64)
        vals.append((_loss(lib, p, True), actual))
    for n in dirs:
        p[n] = base[n]
    # the realised perturbation differs from eps*dir by float32 rounding: use it exactly
    num = vals[0][0] - vals[1][0]
    den_dot = sum(float(np.sum(grads["d" + n if n != "beta" else "dbeta"] * (vals[0][1][n] - vals[1][1][n])))
                  for n in dirs)
    rel = abs(num - den_dot) / max(1e-12, abs(den_dot))
    assert rel < tol, "directional derivative mismatch %.3e (an %.6e)" % (rel, an)


def pin_dh0_transfer(lib, seed=2, tol=1e-11):
    """With dO = 0, dh0 = M^T dht for the state map S_L = M S_0 + B, M = prod a_t (I - b_t k_t k_t^T)."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [9], H=1, HV=1, dk=5, dv=4)
    p["dO"][:] = 0
    grads = _bwd(lib, p, True)
    k = _unit_rows(p["k"][:, 0])
    M = np.eye(5)
    for t in range(9):
        a = np.exp(float(p["g"][t, 0]))
        b = float(p["beta"][t, 0])
        M = a * (np.eye(5) - b * np.outer(k[t], k[t])) @ M
    want = M.T @ p["dht"][0, 0].astype(np.float64)
    err = np.max(np.abs(grads["dh0"][0, 0] - want))
    assert err < tol * max(1.0, np.max(np.abs(want))), "dh0 transfer mismatch %.3e" % err


def pin_bwd_grouped_equals_repeated(lib, seed=3, tol=1e-12):
    """Gradients of q/k with H q/k heads equal the group sums of the HV-head run with repeated q/k."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [11, 6], H=2, HV=6, dk=4, dv=5)
    g1 = _bwd(lib, p, True)
    rep = dict(p)
    rep["q"] = np.repeat(p["q"], 3, axis=1)
    rep["k"] = np.repeat(p["k"], 3, axis=1)
    g2 = _bwd(lib, rep, True)
    for n in ("dq", "dk"):
        summed = g2[n].reshape(g2[n].shape[0], 2, 3, -1).sum(axis=2)
        assert np.max(np.abs(summed - g1[n])) < tol * max(1.0, np.max(np.abs(g1[n]))), n
    for n in ("dv", "dg", "dbeta", "dh0"):
        assert np.max(np.abs(g2[n] - g1[n])) < tol * max(1.0, np.max(np.abs(g1[n]))), n


def pin_bwd_packed_equals_separate(lib, seed=4, tol=1e-12):
    """Gradients of a packed run equal those of each document run alone."""
    rng = np.random.default_rng(seed)
    lens = [7, 1, 12]
    p = rand_problem(rng, lens, H=1, HV=2, dk=4, dv=4)
    g = _bwd(lib, p, True)
    cu = p["cu"]
    for n, L in enumerate(lens):
        s = slice(int(cu[n]), int(cu[n + 1]))
        one = dict(cu=np.array([0, L], np.int32), q=p["q"][s], k=p["k"][s], v=p["v"][s], g=p["g"][s],
                   beta=p["beta"][s], dO=p["dO"][s], h0=p["h0"][n:n + 1], dht=p["dht"][n:n + 1])
        g1 = _bwd(lib, one, True)
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.max(np.abs(g1[name] - g[name][s])) <= tol * max(1.0, np.max(np.abs(g[name]))), name
        assert np.max(np.abs(g1["dh0"][0] - g["dh0"][n])) <= tol * max(1.0, np.max(np.abs(g["dh0"])))


# --------------------------------------------------------------------------------------------
# forward


def pin_overwrite_identity(lib, seed=5, tol=1e-5):
    """beta = 1 and q_t = k_t (unit after the L2 norm): o_t = S_t^T k_t = v_t exactly, for any decay
    and any incoming state. Fails if the correction uses the undecayed state, if the output is read
    before the write, or if the write has the wrong sign."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [10, 7], H=1, HV=2, dk=6, dv=5)
    p["q"] = p["k"].copy()
    p["beta"][:] = 1.0
    o, _ = _fwd(lib, p, True)
    err = np.max(np.abs(o - p["v"].astype(np.float64)))
    # the norm's eps leaves |k|^2 = 1 - O(1e-7): allow that, far below any real mistake's O(1) error
    assert err < tol, "overwrite identity violated by %.3e" % err


def pin_beta_zero(lib, seed=6, tol=1e-12):
    """beta = 0: S_t = exp(G_t) S_0 with G_t the running sum of g, so o_t = exp(G_t) S_0^T qh_t."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [9, 4], H=2, HV=2, dk=4, dv=3)
    p["beta"][:] = 0.0
    o, ht = _fwd(lib, p, True)
    cu = p["cu"]
    qh = _unit_rows(p["q"])
    for n in range(2):
        for h in range(2):
            G = 0.0
            for t in range(int(cu[n]), int(cu[n + 1])):
                G += float(p["g"][t, h])
                want = np.exp(G) * p["h0"][n, h].astype(np.float64).T @ qh[t, h]
                assert np.max(np.abs(o[t, h] - want)) < tol * 10
            assert np.max(np.abs(ht[n, h] - np.exp(G) * p["h0"][n, h])) < tol * 10


def pin_single_token_transition(lib, seed=7, tol=1e-12):
    """One token: S_1 = a (I - b kh kh^T) S_0 + b kh v^T and o = S_1^T qh."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [1], H=1, HV=1, dk=5, dv=3)
    o, ht = _fwd(lib, p, True)
    kh = _unit_rows(p["k"][0, 0])
    qh = _unit_rows(p["q"][0, 0])
    a = np.exp(float(p["g"][0, 0]))
    b = float(p["beta"][0, 0])
    S0 = p["h0"][0, 0].astype(np.float64)
    S1 = a * (np.eye(5) - b * np.outer(kh, kh)) @ S0 + b * np.outer(kh, p["v"][0, 0].astype(np.float64))
    assert np.max(np.abs(ht[0, 0] - S1)) < tol
    assert np.max(np.abs(o[0, 0] - S1.T @ qh)) < tol


def pin_orthonormal_store_recall(lib, seed=8, tol=1e-12):
    """beta = 1, orthonormal keys, S_0 = 0: ht^T k_j = exp(sum_{s>j} g_s) v_j (store, then pure decay)."""
    rng = np.random.default_rng(seed)
    d, L = 8, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    p = rand_problem(rng, [L], H=1, HV=1, dk=d, dv=4, h0=False, dht=False)
    p["k"][:, 0, :] = Qm[:L].astype(np.float32)
    p["beta"][:] = 1.0
    _, ht = _fwd(lib, p, True)
    kk = _unit_rows(p["k"][:, 0])
    g = p["g"][:, 0].astype(np.float64)
    for j in range(L):
        got = ht[0, 0].T @ kk[j]
        want = np.exp(g[j + 1:].sum()) * p["v"][j, 0].astype(np.float64)
        # keys are orthonormal only up to float32 rounding and the norm's eps: allow that much crosstalk
        assert np.max(np.abs(got - want)) < 1e-5, (j, np.max(np.abs(got - want)))


def pin_linear_in_v_and_h0(lib, seed=9, tol=1e-12):
    """o(v, h0) = o(v, 0) + o(0, h0): the recurrence is linear in (state, values)."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [13], H=1, HV=2, dk=4, dv=4)
    o_full, _ = _fwd(lib, p, True)
    a = dict(p, h0=None)
    b = dict(p, v=np.zeros_like(p["v"]))
    oa, _ = _fwd(lib, a, True)
    ob, _ = _fwd(lib, b, True)
    assert np.max(np.abs(o_full - oa - ob)) < tol * 100


def pin_packed_equals_separate(lib, seed=10, tol=1e-13):
    """A packed run equals the per-document runs (the state restarts at every document)."""
    rng = np.random.default_rng(seed)
    lens = [5, 0, 9, 3]
    p = rand_problem(rng, lens, H=1, HV=2, dk=4, dv=3)
    o, ht = _fwd(lib, p, True)
    cu = p["cu"]
    for n, L in enumerate(lens):
        s = slice(int(cu[n]), int(cu[n + 1]))
        one = dict(cu=np.array([0, L], np.int32), q=p["q"][s], k=p["k"][s], v=p["v"][s], g=p["g"][s],
                   beta=p["beta"][s], h0=p["h0"][n:n + 1])
        o1, ht1 = _fwd(lib, one, True)
        assert np.max(np.abs(o1 - o[s]), initial=0.0) <= tol
        assert np.max(np.abs(ht1[0] - ht[n])) <= tol


def pin_fragment_chain(lib, seed=11, tol=1e-12):
    """run(document) == run(second fragment, h0 = ht(first fragment))."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [20], H=1, HV=1, dk=4, dv=4)
    o, ht = _fwd(lib, p, True)
    s1, s2 = slice(0, 8), slice(8, 20)
    f1 = dict(cu=np.array([0, 8], np.int32), q=p["q"][s1], k=p["k"][s1], v=p["v"][s1], g=p["g"][s1],
              beta=p["beta"][s1], h0=p["h0"])
    o1, ht1 = _fwd(lib, f1, True)
    f2 = dict(cu=np.array([0, 12], np.int32), q=p["q"][s2], k=p["k"][s2], v=p["v"][s2], g=p["g"][s2],
              beta=p["beta"][s2], h0=ht1.astype(np.float32))
    o2, ht2 = _fwd(lib, f2, True)
    # h0 of the second run went through float32: compare with a float32-sized tolerance
    assert np.max(np.abs(o1 - o[s1])) <= tol
    assert np.max(np.abs(o2 - o[s2])) <= 1e-6
    assert np.max(np.abs(ht2 - ht)) <= 1e-6


def pin_grouped_equals_repeated(lib, seed=12, tol=1e-13):
    """(H, HV) grouped heads equal (HV, HV) with every q/k head repeated HV/H times (v head h reads
    q/k head h // (HV/H))."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [15], H=2, HV=6, dk=4, dv=3)
    o, ht = _fwd(lib, p, True)
    rep = dict(p, q=np.repeat(p["q"], 3, axis=1), k=np.repeat(p["k"], 3, axis=1))
    o2, ht2 = _fwd(lib, rep, True)
    assert np.max(np.abs(o - o2)) <= tol and np.max(np.abs(ht - ht2)) <= tol


def pin_l2norm_scale_invariance(lib, seed=13, tol=1e-12):
    """With the L2 norm on, scaling q and k rows changes nothing; with it off, pre-normalised
    inputs give the same result as the norm on."""
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, [12], H=1, HV=1, dk=6, dv=3)
    o, _ = _fwd(lib, p, True)
    s = dict(p, q=(p["q"] * 4.0).astype(np.float32), k=(p["k"] * 0.25).astype(np.float32))
    o2, _ = _fwd(lib, s, True)
    assert np.max(np.abs(o - o2)) < 1e-5  # exact up to the norm's eps (relative 1e-7)
    pre = dict(p, q=_unit_rows(p["q"]).astype(np.float32), k=_unit_rows(p["k"]).astype(np.float32))
    o3, _ = _fwd(lib, pre, False)
    assert np.max(np.abs(o - o3)) < 1e-5  # pre-normalised inputs were rounded to float32


def pin_chunked_equals_recurrent(lib, seed=14, tol=1e-11):
    """The chunked form (any chunk size, partial last chunks) equals the token recurrence, and its
    Akk output inverts I + L: A (I + L) = I on every chunk."""
    rng = np.random.default_rng(seed)
    lens = [70, 64, 5, 130]
    p = rand_problem(rng, lens, H=2, HV=4, dk=8, dv=6)
    o, ht = _fwd(lib, p, True)
    for C in (64, 16):
        ch = oracle.chunked_fwd(p["cu"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"], l2norm=True,
                                chunk=C, lib=lib, threads=1)
        scale = max(1.0, np.max(np.abs(o)))
        assert np.max(np.abs(ch["o"] - o)) < tol * scale, C
        assert np.max(np.abs(ch["ht"] - ht)) < tol * scale, C
    # A check for C = 64: rebuild L from the definition on one chunk and multiply
    ch = oracle.chunked_fwd(p["cu"], p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"], l2norm=True, chunk=64,
                            lib=lib, threads=1)
    kh = _unit_rows(p["k"])
    t0, L = 70, 64  # the second document, one full chunk
    for h in range(4):
        j = h // 2
        G = np.cumsum(p["g"][t0:t0 + L, h].astype(np.float64))
        b = p["beta"][t0:t0 + L, h].astype(np.float64)
        Kc = kh[t0:t0 + L, j]
        Lm = np.tril(b[:, None] * np.exp(G[:, None] - G[None, :]) * (Kc @ Kc.T), -1)
        A = ch["A"][t0:t0 + L, h, :L]
        assert np.max(np.abs(A @ (np.eye(L) + Lm) - np.eye(L))) < 1e-10
        assert np.max(np.abs(ch["gcum"][t0:t0 + L, h] - G)) < 1e-12
    # gamma = exp(G_last) of each chunk: chunk 1 is the first chunk of the first document
    G = np.cumsum(p["g"][0:64, 0].astype(np.float64))
    assert abs(ch["gamma"][0, 0] - np.exp(G[-1])) < 1e-12


def pin_chunked_full_set(lib, seed=15, tol=1e-11):
    """What the full saved set adds, against the token recurrence:
    - the state at the start of every chunk is h0 for a document's first chunk and, for chunk m,
      the final state of the recurrence run over the document's first m C tokens;
    - v_new = R, row t: beta_t (v_t - a_t S_{t-1}^T kh_t), the correction the delta rule adds at
      token t (S_t = a_t S_{t-1} + kh_t r_t^T), with S_{t-1} from the recurrence over the tokens
      before t;
    - U = R wherever the chunk starts from a zero state, and U does not depend on the start state;
    - W maps the start state to the change of R: U - R = W S_c on every chunk (dv >= dk here, so
      the start states determine W);
    - P: with g = 0 and q = k, P_ij = kh_i . kh_j for i >= j (1 on the diagonal), 0 above it and
      past the chunk's valid length."""
    rng = np.random.default_rng(seed)
    lens, C = [21, 9], 8
    dk, dv = 4, 6
    p = rand_problem(rng, lens, H=1, HV=2, dk=dk, dv=dv)
    kh = _unit_rows(p["k"])

    def chunked(pp):
        return oracle.chunked_fwd(pp["cu"], pp["q"], pp["k"], pp["v"], pp["g"], pp["beta"], pp["h0"], l2norm=True,
                                  chunk=C, lib=lib, threads=1, full=True)

    def state_after(n, m):  # recurrent state of document n after its first m tokens
        t0 = int(p["cu"][n])
        sub = dict(cu=np.array([0, m], np.int32), h0=p["h0"][n:n + 1],
                   **{x: p[x][t0:t0 + m] for x in ("q", "k", "v", "g", "beta")})
        return _fwd(lib, sub, True)[1][0]

    ch = chunked(p)
    z = dict(p, h0=None)
    ch0 = chunked(z)
    cidx = 0
    for n, L in enumerate(lens):
        t0 = int(p["cu"][n])
        for cs in range(0, L, C):
            S_c = state_after(n, cs) if cs > 0 else p["h0"][n].astype(np.float64)
            if cs == 0:
                assert np.array_equal(ch["H"][cidx], S_c)
            assert np.max(np.abs(ch["H"][cidx] - S_c)) < tol
            if cs == 0:
                assert np.max(np.abs(ch0["U"][t0:t0 + C] - ch0["R"][t0:t0 + C])) < tol
            rows = slice(t0 + cs, t0 + min(cs + C, L))
            assert np.max(np.abs(ch["U"][rows] - ch0["U"][rows])) < tol
            for h in range(2):
                lhs = ch["U"][rows, h] - ch["R"][rows, h]
                assert np.max(np.abs(lhs - ch["W"][rows, h] @ ch["H"][cidx, h])) < tol
            cidx += 1
        for m in range(L):
            S_prev = state_after(n, m) if m > 0 else p["h0"][n].astype(np.float64)
            t = t0 + m
            for h in range(2):
                a = np.exp(np.float64(p["g"][t, h]))
                r = np.float64(p["beta"][t, h]) * (p["v"][t, h] - a * S_prev[h].T @ kh[t, 0])
                assert np.max(np.abs(ch["R"][t, h] - r)) < tol
    # P at g = 0 with q = k
    pq = dict(p, q=p["k"].copy(), g=np.zeros_like(p["g"]))
    P = chunked(pq)["P"]
    for n, L in enumerate(lens):
        t0 = int(p["cu"][n])
        for cs in range(0, L, C):
            Ce = min(C, L - cs)
            Kc = kh[t0 + cs:t0 + cs + Ce, 0]
            ref = np.zeros((Ce, C))
            ref[:, :Ce] = np.tril(Kc @ Kc.T)
            for h in range(2):
                assert np.max(np.abs(P[t0 + cs:t0 + cs + Ce, h] - ref)) < tol
                assert np.max(np.abs(np.diag(P[t0 + cs:t0 + cs + Ce, h, :Ce]) - 1.0)) < 1e-5


ALL_PINS = [
    pin_finite_differences,
    pin_directional_derivative,
    pin_dh0_transfer,
    pin_bwd_grouped_equals_repeated,
    pin_bwd_packed_equals_separate,
    pin_overwrite_identity,
    pin_beta_zero,
    pin_single_token_transition,
    pin_orthonormal_store_recall,
    pin_linear_in_v_and_h0,
    pin_packed_equals_separate,
    pin_fragment_chain,
    pin_grouped_equals_repeated,
    pin_l2norm_scale_invariance,
    pin_chunked_equals_recurrent,
    pin_chunked_full_set,
]
