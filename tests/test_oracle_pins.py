"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Each test reduces the oracle to a case with an independent definition:
closed-form rules printed on the pages, brute force on tiny inputs, finite
differences of an independently written loss, invariants.  None of them calls
the GPU library.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import erf

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(cfg, q, k, v, alpha, eta, theta, gamma, mem0=None, state=None, delta=None):
    """Single-sequence convenience wrapper: arrays without the sequence axis."""
    cfg.n_seq = 1
    st = state if state is not None else O.empty_state(cfg)
    if mem0 is not None:
        st["mem"][0] = np.asarray(mem0, dtype=np.float64).ravel()
    add = lambda a: np.asarray(a, dtype=np.float64)[None]
    out, _ = O.forward(cfg, add(q), add(k), add(v), add(alpha), add(eta), add(theta), add(gamma), st,
                       delta=None if delta is None else add(delta))
    return out[0], st


def rand_unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def gelu(z):
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


# --------------------------------------------------------------------------- phi
def test_phi_poly2_is_the_monomial_list():
    """ATLAS review sec. 3.1 'Polynomial Feature Mapping': phi_p(x) lists the
    monomials x^beta with |beta| <= p; degree 1 and 2 here, no constant."""
    rng = np.random.default_rng(1)
    d = 5
    x = rng.standard_normal(d)
    cfg = O.make_config(d_k=d, d_v=1, feature_map="poly2")
    got = O.phi(cfg, x)
    want = [x[i] for i in range(d)] + [x[a] * x[b] for a, b in
                                       itertools.combinations_with_replacement(range(d), 2)]
    assert len(got) == d + d * (d + 1) // 2 == O.feature_dim(cfg)
    np.testing.assert_array_equal(got, np.array(want))


def test_phi_raw_poly2_dimensions_and_layout():
    """[k, poly2(k[:p])]: the full raw key followed by the degree-2 map of its
    first p entries (688 wide for d_k = 128, p = 32)."""
    rng = np.random.default_rng(2)
    cfg = O.make_config(d_k=128, d_v=128, feature_map="raw_poly2", poly_dims=32)
    assert O.feature_dim(cfg) == 688
    x = rng.standard_normal(128)
    got = O.phi(cfg, x)
    np.testing.assert_array_equal(got[:128], x)
    np.testing.assert_array_equal(got[128:160], x[:32])
    pairs = list(itertools.combinations_with_replacement(range(32), 2))
    np.testing.assert_array_equal(got[160:], [x[a] * x[b] for a, b in pairs])


# --------------------------------------------------------------------------- delta rule
def test_deltanet_golden_two_tokens():
    g = json.load(open(os.path.join(GOLDEN, "deltanet_2token.json")))
    d = g["d"]
    cfg = O.make_config(d_k=d, d_v=d, window=1, chunk=1)
    beta = np.array(g["beta"])
    out, st = run(cfg, g["q"], g["k"], g["v"], np.zeros(2), np.zeros(2), beta, np.ones(2), g["M0"])
    np.testing.assert_array_equal(out, np.array(g["y"], dtype=float))
    np.testing.assert_array_equal(st["mem"][0].reshape(d, d), np.array(g["M"][-1], dtype=float))


@pytest.mark.parametrize("gated", [False, True])
def test_delta_rule_closed_form(gated):
    """b = c = 1, linear memory, no momentum: the update is the DeltaNet rule
    M_t = M_{t-1} + beta_t (v_t - M_{t-1} k_t) k_t^T with beta = theta*gamma
    (ATLAS review intro; Miras review Background); with decay it is the
    scalar-gated delta rule M_t = (1-alpha_t) M_{t-1} + beta_t (v_t - M_{t-1} k_t) k_t^T
    (Miras review, 'Miras: four design choices', gated DeltaNet)."""
    rng = np.random.default_rng(3)
    N, dk, dv = 40, 6, 4
    q, k, v = rand_unit(rng, N, dk), rand_unit(rng, N, dk), rng.standard_normal((N, dv))
    theta, gamma = rng.uniform(0.1, 0.9, N), rng.uniform(0.2, 1.0, N)
    alpha = rng.uniform(0, 0.3, N) if gated else np.zeros(N)
    M0 = rng.standard_normal((dv, dk)) * 0.3
    cfg = O.make_config(d_k=dk, d_v=dv, window=1, chunk=1)
    out, st = run(cfg, q, k, v, alpha, rng.uniform(size=N), theta, gamma, M0)
    M = M0.copy()
    for t in range(N):
        beta = theta[t] * gamma[t]
        M = (1 - alpha[t]) * M + beta * np.outer(v[t] - M @ k[t], k[t])
        np.testing.assert_allclose(out[t], M @ q[t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st["mem"][0].reshape(dv, dk), M, rtol=1e-12, atol=1e-13)


def test_delta_rule_as_gd_on_l2_with_phi():
    """ATLAS review sec. 3.1: GD on ||M phi(k) - v||^2 gives
    M_t = M_{t-1}(I - eta phi phi^T) + eta v phi^T (written there with M on the
    other side); poly2 map, b = c = 1."""
    rng = np.random.default_rng(4)
    N, dk, dv = 30, 3, 2
    cfg = O.make_config(d_k=dk, d_v=dv, feature_map="poly2", window=1, chunk=1)
    D = O.feature_dim(cfg)
    q, k, v = rand_unit(rng, N, dk), rand_unit(rng, N, dk), rng.standard_normal((N, dv))
    lr = rng.uniform(0.05, 0.4, N)
    out, st = run(cfg, q, k, v, np.zeros(N), np.zeros(N), lr, np.ones(N))
    M = np.zeros((dv, D))
    for t in range(N):
        f = O.phi(cfg, k[t])
        M = M @ (np.eye(D) - lr[t] * np.outer(f, f)) + lr[t] * np.outer(v[t], f)
        np.testing.assert_allclose(out[t], M @ O.phi(cfg, q[t]), rtol=1e-11, atol=1e-13)


def test_omeganet_linear_closed_form():
    """b = 1, window c > 1, no momentum: ATLAS review sec. 3.2 (OmegaNet, linear
    memory) M_t = M_{t-1}(a_t I - theta_t sum_i gamma_i phi_i phi_i^T)
    + theta_t sum_i gamma_i v_i phi_i^T, the sum over the last c tokens, with the
    keep factor a_t = 1 - alpha_t and the descent sign on the last term."""
    rng = np.random.default_rng(5)
    N, dk, dv, c = 50, 3, 3, 4
    cfg = O.make_config(d_k=dk, d_v=dv, feature_map="poly2", window=c, chunk=1)
    D = O.feature_dim(cfg)
    q, k, v = rand_unit(rng, N, dk), rand_unit(rng, N, dk), rng.standard_normal((N, dv))
    alpha, theta, gamma = rng.uniform(0, 0.2, N), rng.uniform(0.02, 0.15, N), rng.uniform(0.3, 1, N)
    out, st = run(cfg, q, k, v, alpha, np.zeros(N), theta, gamma)
    M = np.zeros((dv, D))
    X = np.array([O.phi(cfg, kk) for kk in k])
    for t in range(N):
        idx = range(max(0, t - c + 1), t + 1)
        H = sum(gamma[i] * np.outer(X[i], X[i]) for i in idx)
        R = sum(gamma[i] * np.outer(v[i], X[i]) for i in idx)
        M = M @ ((1 - alpha[t]) * np.eye(D) - theta[t] * H) + theta[t] * R
        np.testing.assert_allclose(out[t], M @ O.phi(cfg, q[t]), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("b,c", [(4, 1), (5, 3), (8, 8), (7, 10)])
def test_chunked_closed_form(b, c):
    """b > 1, no momentum: ATLAS review sec. 3.3 'Parallelizing Omega Rule'
    M_t = (prod_{u=t'}^{t} a_u) M_{t'-1}
          - sum_{n=t'}^{t} (prod_{u=n+1}^{t} a_u) theta_n sum_{i=n-c+1}^{n} grad_i(M_{t'-1})
    with t' the first token of the chunk (0-indexed chunks [jb, jb+b)), every
    gradient taken at the state the previous chunk left."""
    rng = np.random.default_rng(6)
    N, dk, dv = 37, 4, 3
    cfg = O.make_config(d_k=dk, d_v=dv, window=c, chunk=b)
    q, k, v = rand_unit(rng, N, dk), rand_unit(rng, N, dk), rng.standard_normal((N, dv))
    alpha, theta, gamma = rng.uniform(0, 0.3, N), rng.uniform(0.01, 0.1, N), rng.uniform(0.3, 1, N)
    out, st = run(cfg, q, k, v, alpha, np.zeros(N), theta, gamma)
    a = 1.0 - alpha
    Mprev = np.zeros((dv, dk))
    for t0 in range(0, N, b):
        grads = {i: gamma[i] * np.outer(Mprev @ k[i] - v[i], k[i]) for i in range(max(0, t0 - c + 1), min(N, t0 + b))}
        for t in range(t0, min(N, t0 + b)):
            M = np.prod(a[t0:t + 1]) * Mprev
            for n in range(t0, t + 1):
                gsum = sum(grads[i] for i in range(max(0, n - c + 1), n + 1))
                M = M - np.prod(a[n + 1:t + 1]) * theta[n] * gsum
            np.testing.assert_allclose(out[t], M @ q[t], rtol=1e-11, atol=1e-13)
        Mprev = M
    np.testing.assert_allclose(st["mem"][0].reshape(dv, dk), Mprev, rtol=1e-11, atol=1e-13)


def test_momentum_recurrence():
    """Titans review sec. 3.1 ('Forgetting Mechanism'):
    M_t = (1 - alpha_t) M_{t-1} + S_t,  S_t = eta_t S_{t-1} - theta_t grad l(M_{t-1}; x_t);
    b = c = 1 so the gradient is at M_{t-1}."""
    rng = np.random.default_rng(7)
    N, dk, dv = 60, 5, 3
    cfg = O.make_config(d_k=dk, d_v=dv, window=1, chunk=1, momentum=True)
    q, k, v = rand_unit(rng, N, dk), rand_unit(rng, N, dk), rng.standard_normal((N, dv))
    alpha, eta, theta = rng.uniform(0, 0.2, N), rng.uniform(0.5, 0.95, N), rng.uniform(0.05, 0.3, N)
    out, st = run(cfg, q, k, v, alpha, eta, theta, np.ones(N))
    M, S = np.zeros((dv, dk)), np.zeros((dv, dk))
    for t in range(N):
        grad = np.outer(M @ k[t] - v[t], k[t])
        S = eta[t] * S - theta[t] * grad
        M = (1 - alpha[t]) * M + S
        np.testing.assert_allclose(out[t], M @ q[t], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(st["mom"][0].reshape(dv, dk), S, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------- dot-product bias
@pytest.mark.parametrize("b", [1, 7, 16])
@pytest.mark.parametrize("fmap", ["identity", "poly2"])
def test_dot_bias_is_unnormalised_linear_attention(b, fmap):
    """Dot-product bias, no decay, theta = gamma = 1: the additive (Hebbian)
    rule M_t = M_{t-1} + v_t phi(k_t)^T (ATLAS review intro and sec. 3.1), whose
    read-out is unnormalised causal linear attention
    y_t = sum_{j<=t} (phi(q_t) . phi(k_j)) v_j (Miras review, Background)."""
    rng = np.random.default_rng(8)
    N, dk, dv = 33, 3, 4
    cfg = O.make_config(d_k=dk, d_v=dv, feature_map=fmap, window=1, chunk=b, bias="dot")
    q, k, v = rng.standard_normal((N, dk)), rng.standard_normal((N, dk)), rng.standard_normal((N, dv))
    out, st = run(cfg, q, k, v, np.zeros(N), np.zeros(N), np.ones(N), np.ones(N))
    X = np.array([O.phi(cfg, x) for x in k])
    Xq = np.array([O.phi(cfg, x) for x in q])
    for t in range(N):
        want = sum((Xq[t] @ X[j]) * v[j] for j in range(t + 1))
        np.testing.assert_allclose(out[t], want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st["mem"][0].reshape(dv, -1), v.T @ X, rtol=1e-11, atol=1e-12)


def test_dot_bias_chunk_size_invariance_and_scalar_weights():
    """With the dot-product bias every gradient -gamma_i v_i phi_i^T is
    independent of M, so the chunk size cannot matter, and
    M_n = sum_i mu_{n,i} v_i phi_i^T with the scalar recurrences
    sigma_{n,i} = eta_n sigma_{n-1,i} + theta_n gamma_i [i in window(n)],
    mu_{n,i} = (1 - alpha_n) mu_{n-1,i} + sigma_{n,i}."""
    rng = np.random.default_rng(9)
    N, dk, dv, c = 45, 3, 2, 5
    q, k, v = rand_unit(rng, N, dk), rand_unit(rng, N, dk), rng.standard_normal((N, dv))
    alpha, eta, theta, gamma = (rng.uniform(0, 0.3, N), rng.uniform(0.3, 0.9, N),
                                rng.uniform(0.05, 0.5, N), rng.uniform(0.2, 1, N))
    outs = []
    for b in (1, 4, 16, 64):
        cfg = O.make_config(d_k=dk, d_v=dv, feature_map="poly2", window=c, chunk=b,
                            momentum=True, bias="dot")
        out, _ = run(cfg, q, k, v, alpha, eta, theta, gamma)
        outs.append(out)
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-12, atol=1e-13)
    X = np.array([O.phi(cfg, x) for x in k])
    Xq = np.array([O.phi(cfg, x) for x in q])
    sig, mu = np.zeros(N), np.zeros(N)
    for n in range(N):
        inwin = (np.arange(N) >= n - c + 1) & (np.arange(N) <= n)
        sig = eta[n] * sig + theta[n] * gamma * inwin
        mu = (1 - alpha[n]) * mu + sig
        want = sum(mu[i] * (Xq[n] @ X[i]) * v[i] for i in range(N))
        np.testing.assert_allclose(outs[0][n], want, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- gates
def mlp_cfg(d=4, h=6, c=3, b=5, momentum=True, residual=True, bias="l2"):
    return O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=residual,
                         window=c, chunk=b, momentum=momentum, bias=bias)


def test_alpha_one_erases_memory():
    """Titans review sec. 3.1 'Forgetting Mechanism': alpha = 1 clears the memory;
    with theta = 0 nothing is written back, so the read-out is the residual
    path alone (MLP) or zero (linear)."""
    rng = np.random.default_rng(10)
    N, d = 23, 4
    q, k, v = rand_unit(rng, N, d), rand_unit(rng, N, d), rng.standard_normal((N, d))
    cfg = mlp_cfg()
    P = O.param_count(cfg)
    out, st = run(cfg, q, k, v, np.ones(N), rng.uniform(size=N), np.zeros(N), np.ones(N),
                  rng.standard_normal(P))
    np.testing.assert_array_equal(out, q)
    assert not st["mem"].any()
    lin = O.make_config(d_k=d, d_v=d, window=2, chunk=4, momentum=True)
    out, st = run(lin, q, k, v, np.ones(N), rng.uniform(size=N), np.zeros(N), np.ones(N),
                  rng.standard_normal(d * d))
    assert not out.any() and not st["mem"].any()


def test_theta_zero_keeps_memory_and_reads_plain_forward():
    """Titans review sec. 3.1: M_t = M_{t-1} - theta_t grad, so theta = 0 (and
    alpha = 0) leaves M unchanged; retrieval is a plain forward pass
    y = r + W2 gelu(W1 phi(q)) ('Retrieving a Memory')."""
    rng = np.random.default_rng(11)
    N, d, h = 19, 4, 6
    q, k, v = rand_unit(rng, N, d), rand_unit(rng, N, d), rng.standard_normal((N, d))
    cfg = mlp_cfg(d=d, h=h)
    W1, W2 = rng.standard_normal((h, d)), rng.standard_normal((d, h))
    out, st = run(cfg, q, k, v, np.zeros(N), rng.uniform(size=N), np.zeros(N), np.ones(N),
                  np.concatenate([W1.ravel(), W2.ravel()]))
    want = q + gelu(q @ W1.T) @ W2.T
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(st["mem"][0], np.concatenate([W1.ravel(), W2.ravel()]))


# --------------------------------------------------------------------------- MLP gradient
@pytest.mark.parametrize("bias", ["l2", "dot"])
@pytest.mark.parametrize("residual", [True, False])
def test_mlp_gradient_matches_finite_differences(bias, residual):
    """Central differences of an independently written loss:
    L2 : gamma*s/2 * |[r +] W2 gelu(W1 x) - v|^2,  DOT: -gamma*s*<[r +] W2 gelu(W1 x), v>."""
    rng = np.random.default_rng(12)
    d, h, gamma, s = 3, 5, 0.7, 1.0
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=residual, bias=bias,
                        grad_scale=s)
    theta = rng.standard_normal(h * d + d * h)
    x, v = rng.standard_normal(d), rng.standard_normal(d)

    def loss(th):
        W1, W2 = th[:h * d].reshape(h, d), th[h * d:].reshape(d, h)
        f = (x if residual else 0) + W2 @ gelu(W1 @ x)
        return gamma * s / 2 * np.sum((f - v) ** 2) if bias == "l2" else -gamma * s * f @ v

    g = O.token_grad(cfg, theta, x, x, v, gamma)
    eps = 1e-6
    fd = np.array([(loss(theta + eps * e) - loss(theta - eps * e)) / (2 * eps)
                   for e in np.eye(theta.size)])
    np.testing.assert_allclose(g, fd, rtol=1e-7, atol=1e-8)


def test_grad_scale_is_linear():
    """grad_scale s multiplies the gradient (s = 2 is the literal derivative of
    the squared norm; s = 1 matches the printed update rules)."""
    rng = np.random.default_rng(13)
    cfg1 = O.make_config(d_k=3, d_v=3, memory="mlp", hidden=4, residual=True, grad_scale=1.0)
    cfg2 = O.make_config(d_k=3, d_v=3, memory="mlp", hidden=4, residual=True, grad_scale=2.0)
    th, x, v = rng.standard_normal(24), rng.standard_normal(3), rng.standard_normal(3)
    np.testing.assert_allclose(O.token_grad(cfg2, th, x, x, v, 0.5),
                               2 * O.token_grad(cfg1, th, x, x, v, 0.5), rtol=1e-14)


# --------------------------------------------------------------------------- invariants
def test_min_norm_interpolation_of_independent_keys():
    """ATLAS summary, App. C: full-batch GD converges to the minimum-norm
    interpolating solution; with p <= d_k independent keys a matrix memory
    stores all p pairs (sec. 3.1, capacity).  A window c = p over a cyclic
    repetition of the p pairs makes every step the full-batch gradient."""
    rng = np.random.default_rng(14)
    d, p, dv, reps = 6, 4, 3, 400
    K, V = rng.standard_normal((p, d)), rng.standard_normal((p, dv))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    N = p * reps
    k = np.tile(K, (reps, 1))
    v = np.tile(V, (reps, 1))
    cfg = O.make_config(d_k=d, d_v=dv, window=p, chunk=1)
    out, st = run(cfg, k, k, v, np.zeros(N), np.zeros(N), np.full(N, 0.2), np.ones(N))
    M = st["mem"][0].reshape(dv, d)
    np.testing.assert_allclose(M, V.T @ np.linalg.pinv(K.T), rtol=1e-6, atol=1e-8)


def test_streaming_split_equals_single_call():
    """The state (weights, momentum, the last c-1 tokens, the token count)
    carries everything: M_t = f(M_{t-1}, x_t) (Titans review sec. 2.1).  Two
    calls with a chunk-aligned split equal one call."""
    rng = np.random.default_rng(15)
    N, d, b = 40, 4, 5
    q, k, v = rand_unit(rng, N, d), rand_unit(rng, N, d), rng.standard_normal((N, d))
    g = [rng.uniform(0, 0.3, N), rng.uniform(0.3, 0.9, N), rng.uniform(0.05, 0.3, N), rng.uniform(0.2, 1, N)]
    cfg = mlp_cfg(d=d, c=7, b=b)
    W0 = rng.standard_normal(O.param_count(cfg)) * 0.3
    full, st_full = run(cfg, q, k, v, *g, W0)
    st = O.empty_state(cfg)
    st["mem"][0] = W0
    s1 = 15
    o1, st = run(cfg, q[:s1], k[:s1], v[:s1], *[a[:s1] for a in g], state=st)
    o2, st = run(cfg, q[s1:], k[s1:], v[s1:], *[a[s1:] for a in g], state=st)
    np.testing.assert_allclose(np.concatenate([o1, o2]), full, rtol=1e-12, atol=1e-14)
    for key in ("mem", "mom", "halo_k", "halo_v", "halo_g", "count"):
        np.testing.assert_allclose(st[key], st_full[key], rtol=1e-12, atol=1e-14)


def test_window_truncates_at_sequence_start():
    """Before the first token there is nothing: a window reaching past it
    holds only the tokens that exist, so a huge c with one chunk equals the
    global objective over the prefix (ATLAS review sec. 3.2, global context)."""
    rng = np.random.default_rng(16)
    N, d = 12, 3
    q, k, v = rand_unit(rng, N, d), rand_unit(rng, N, d), rng.standard_normal((N, d))
    theta = rng.uniform(0.05, 0.2, N)
    big = O.make_config(d_k=d, d_v=d, window=100, chunk=1)
    exact = O.make_config(d_k=d, d_v=d, window=N, chunk=1)
    o1, _ = run(big, q, k, v, np.zeros(N), np.zeros(N), theta, np.ones(N))
    o2, _ = run(exact, q, k, v, np.zeros(N), np.zeros(N), theta, np.ones(N))
    np.testing.assert_array_equal(o1, o2)
    M = np.zeros((d, d))
    for t in range(N):
        M = M - theta[t] * sum(np.outer(M @ k[i] - v[i], k[i]) for i in range(t + 1))
        np.testing.assert_allclose(o1[t], M @ q[t], rtol=1e-12, atol=1e-14)


def test_bad_configs_are_rejected():
    cfg = O.make_config(d_k=3, d_v=4, memory="mlp", hidden=5, residual=True)
    st = O.empty_state(cfg)
    z = np.zeros((1, 2, 3))
    with pytest.raises(ValueError):
        O.forward(cfg, z, z, np.zeros((1, 2, 4)), *[np.zeros((1, 2))] * 4, st)


# --------------------------------------------------------------------------- other attentional biases
# Miras review, "Alternative Attentional Biases": the l_p loss |M(k) - v|_p^p
# and the Huber loss (squared error below a per-token threshold delta_t, the
# absolute error above it).  Readings: the l_p loss carries the 1/p that the
# squared error's 1/2 convention generalises to, so p = 2 is the squared
# error; the Huber choice is made per token on |e|_2, its large-error branch
# is delta_t * |e|_1.

def huber_loss(e, delta):
    n = np.linalg.norm(e)
    return 0.5 * n * n if n <= delta else delta * (np.sum(np.abs(e)) - 0.5 * delta)


@pytest.mark.parametrize("p", [3.0, 1.5])
@pytest.mark.parametrize("residual", [True, False])
def test_lp_gradient_matches_finite_differences(p, residual):
    """Central differences of gamma*s * sum_o |f_o - v_o|^p / p."""
    rng = np.random.default_rng(40)
    d, h, gamma, s = 3, 5, 0.7, 1.3
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=residual, bias="lp",
                        bias_p=p, grad_scale=s)
    theta = rng.standard_normal(h * d + d * h)
    x, v = rng.standard_normal(d), rng.standard_normal(d)

    def loss(th):
        W1, W2 = th[:h * d].reshape(h, d), th[h * d:].reshape(d, h)
        f = (x if residual else 0) + W2 @ gelu(W1 @ x)
        return gamma * s * np.sum(np.abs(f - v) ** p) / p

    g = O.token_grad(cfg, theta, x, x, v, gamma)
    eps = 1e-6
    fd = np.array([(loss(theta + eps * e) - loss(theta - eps * e)) / (2 * eps)
                   for e in np.eye(theta.size)])
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("alpha", [0.0, 3.0])
@pytest.mark.parametrize("regime", ["squared", "absolute", "between_norms"])
def test_huber_gradient_matches_finite_differences(regime, alpha):
    """Central differences of gamma*s * huber(f - v; delta), on both branches
    and with delta between |e|_2 and |e|_1 (the test uses the l2 norm).  With
    the smooth sign tanh(alpha e) the large-error branch is
    delta * sum_o log(cosh(alpha e_o)) / alpha."""
    rng = np.random.default_rng(41)
    d, h, gamma, s = 3, 5, 0.8, 1.0
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=True, bias="huber", grad_scale=s,
                        sign_alpha=alpha)
    theta = rng.standard_normal(h * d + d * h)
    x, v = rng.standard_normal(d), rng.standard_normal(d)
    W1, W2 = theta[:h * d].reshape(h, d), theta[h * d:].reshape(d, h)
    e = x + W2 @ gelu(W1 @ x) - v
    n2, n1 = np.linalg.norm(e), np.sum(np.abs(e))
    delta = {"squared": 2.0 * n1, "absolute": 0.3 * n2, "between_norms": 0.5 * (n1 + n2)}[regime]
    assert n2 < n1

    def loss(th):
        W1, W2 = th[:h * d].reshape(h, d), th[h * d:].reshape(d, h)
        e = x + W2 @ gelu(W1 @ x) - v
        if alpha > 0 and np.linalg.norm(e) > delta:
            return gamma * s * delta * np.sum(np.log(np.cosh(alpha * e))) / alpha
        return gamma * s * huber_loss(e, delta)

    g = O.token_grad(cfg, theta, x, x, v, gamma, delta)
    eps = 1e-6
    fd = np.array([(loss(theta + eps * e) - loss(theta - eps * e)) / (2 * eps)
                   for e in np.eye(theta.size)])
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def _mixed_run(bias, rng_seed=42, **kw):
    rng = np.random.default_rng(rng_seed)
    N, d = 37, 4
    q, k, v = rand_unit(rng, N, d), rand_unit(rng, N, d), rng.standard_normal((N, d))
    g = [rng.uniform(0, 0.3, N), rng.uniform(0.3, 0.9, N), rng.uniform(0.05, 0.4, N), rng.uniform(0.2, 1, N)]
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=6, residual=True, window=3, chunk=5,
                        momentum=True, bias=bias, **kw)
    W0 = np.random.default_rng(rng_seed + 1).standard_normal(O.param_count(cfg)) * 0.5
    return cfg, (q, k, v, *g), W0


def test_lp_with_p2_is_the_squared_error():
    """|e|_2^2 / 2 is the l_p loss at p = 2: the whole run (MLP, window,
    chunks, momentum) matches the squared-error bias."""
    cfg2, args, W0 = _mixed_run("l2")
    cfgp, _, _ = _mixed_run("lp", bias_p=2.0)
    want, st2 = run(cfg2, *args, W0)
    got, stp = run(cfgp, *args, W0)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(stp["mem"], st2["mem"], rtol=1e-12, atol=1e-14)


def test_huber_limits():
    """delta = +inf: always the squared error; delta = 0: the absolute branch
    times 0, so nothing is ever written and retrieval is the plain forward
    pass at the initial weights (as with theta = 0)."""
    cfg2, args, W0 = _mixed_run("l2")
    cfgh, _, _ = _mixed_run("huber")
    N = args[0].shape[0]
    want, st2 = run(cfg2, *args, W0)
    got, sth = run(cfgh, *args, W0, delta=np.full(N, 1e300))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    q, k, v, al, et, th, ga = args
    frozen, _ = run(cfg2, q, k, v, np.zeros(N), et, np.zeros(N), ga, W0)
    got0, st0 = run(cfgh, q, k, v, np.zeros(N), et, th, ga, W0, delta=np.zeros(N))
    np.testing.assert_allclose(got0, frozen, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(st0["mem"][0], W0)


@pytest.mark.parametrize("alpha", [0.0, 2.5])
@pytest.mark.parametrize("bias", ["lp1", "lp3", "huber"])
def test_scalar_memory_sign_rules(bias, alpha):
    """A 1x1 linear memory, b = c = 1, no decay or momentum: each token does
    m <- m - theta*gamma*g(m k - v) k, with g(e) = sign(e) (p = 1),
    e|e| (p = 3), or e if |e| <= delta else delta*sign(e) (Huber); y = m q.
    With alpha > 0, sign(e) is tanh(alpha e)."""
    rng = np.random.default_rng(43)
    N = 30
    q, k, v = rng.standard_normal((N, 1)), rng.standard_normal((N, 1)), rng.standard_normal((N, 1)) * 2
    th, ga, dl = rng.uniform(0.05, 0.5, N), rng.uniform(0.3, 1.0, N), rng.uniform(0.2, 2.0, N)
    kw = {"lp1": dict(bias="lp", bias_p=1.0), "lp3": dict(bias="lp", bias_p=3.0), "huber": dict(bias="huber")}[bias]
    cfg = O.make_config(d_k=1, d_v=1, window=1, chunk=1, sign_alpha=alpha, **kw)
    sg = (lambda e: np.tanh(alpha * e)) if alpha > 0 else np.sign
    m, want = 0.4, []
    for t in range(N):
        e = m * k[t, 0] - v[t, 0]
        gx = {"lp1": sg(e), "lp3": sg(e) * e * e, "huber": e if abs(e) <= dl[t] else dl[t] * sg(e)}[bias]
        m = m - th[t] * ga[t] * gx * k[t, 0]
        want.append(m * q[t, 0])
    out, st = run(cfg, q, k, v, np.zeros(N), np.zeros(N), th, ga, [0.4], delta=dl)
    np.testing.assert_allclose(out[:, 0], want, rtol=1e-12, atol=1e-14)


def test_huber_thresholds_of_the_halo_carry_over():
    """The last c-1 thresholds travel in the state like the keys, values and
    gammas: two chunk-aligned calls equal one."""
    cfg, args, W0 = _mixed_run("huber")
    N = args[0].shape[0]
    dl = np.random.default_rng(44).uniform(0.3, 3.0, N)
    full, st_full = run(cfg, *args, W0, delta=dl)
    st = O.empty_state(cfg)
    st["mem"][0] = W0
    s1 = 15
    o1, st = run(cfg, *[a[:s1] for a in args], state=st, delta=dl[:s1])
    o2, st = run(cfg, *[a[s1:] for a in args], state=st, delta=dl[s1:])
    np.testing.assert_allclose(np.concatenate([o1, o2]), full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st["halo_d"], st_full["halo_d"], rtol=0, atol=0)


def test_huber_needs_thresholds_and_lp_needs_p_at_least_one():
    cfg, args, W0 = _mixed_run("lp", bias_p=0.5)
    with pytest.raises(ValueError):
        run(cfg, *args, W0)


# --------------------------------------------------------------------------- layer-norm memory
# Miras review, the memory of its three models: M(x) = x + LN(W sigma(W' x)).
# Here f(x) = r + LN(W2 gelu(W1 x)), LN over the d_v outputs without gain or
# shift, (u - mean) / sqrt(var + eps) with the biased variance.

def ln_np(u, eps):
    return (u - u.mean()) / np.sqrt(u.var() + eps)


@pytest.mark.parametrize("bias", ["l2", "dot", "lp", "huber"])
def test_layernorm_gradient_matches_finite_differences(bias):
    rng = np.random.default_rng(50)
    d, h, gamma, s, eps = 4, 5, 0.7, 1.2, 0.05   # eps large enough that its placement matters
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=True, bias=bias, grad_scale=s,
                        bias_p=3.0, layernorm=True, ln_eps=eps)
    theta = rng.standard_normal(h * d + d * h)
    x, v = rng.standard_normal(d), rng.standard_normal(d) * 2
    delta = 1.5

    def loss(th):
        W1, W2 = th[:h * d].reshape(h, d), th[h * d:].reshape(d, h)
        f = x + ln_np(W2 @ gelu(W1 @ x), eps)
        e = f - v
        if bias == "l2":
            return gamma * s * 0.5 * e @ e
        if bias == "dot":
            return -gamma * s * f @ v
        if bias == "lp":
            return gamma * s * np.sum(np.abs(e) ** 3) / 3
        return gamma * s * huber_loss(e, delta)

    g = O.token_grad(cfg, theta, x, x, v, gamma, delta)
    eps_fd = 1e-6
    fd = np.array([(loss(theta + eps_fd * e) - loss(theta - eps_fd * e)) / (2 * eps_fd)
                   for e in np.eye(theta.size)])
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_layernorm_retrieval_is_the_plain_forward_and_scale_free():
    """theta = alpha = 0: y = q + LN(W2 gelu(W1 q)); LN removes any positive
    scale of W2 (eps small against the variance)."""
    rng = np.random.default_rng(51)
    N, d, h, eps = 13, 6, 7, 1e-12
    q, k, v = rand_unit(rng, N, d), rand_unit(rng, N, d), rng.standard_normal((N, d))
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=True, window=2, chunk=4,
                        momentum=True, layernorm=True, ln_eps=eps)
    W1, W2 = rng.standard_normal((h, d)), rng.standard_normal((d, h))
    out, _ = run(cfg, q, k, v, np.zeros(N), rng.uniform(size=N), np.zeros(N), np.ones(N),
                 np.concatenate([W1.ravel(), W2.ravel()]))
    want = np.array([q[t] + ln_np(W2 @ gelu(W1 @ q[t]), eps) for t in range(N)])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)
    out3, _ = run(cfg, q, k, v, np.zeros(N), rng.uniform(size=N), np.zeros(N), np.ones(N),
                  np.concatenate([W1.ravel(), 3.0 * W2.ravel()]))
    np.testing.assert_allclose(out3, out, rtol=1e-8, atol=1e-9)
    branch = out - q
    np.testing.assert_allclose(branch.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(branch.var(axis=1), 1.0, rtol=1e-7)


def test_layernorm_needs_an_mlp_and_a_positive_eps():
    for kw in (dict(memory="linear", layernorm=True), dict(memory="mlp", hidden=4, layernorm=True, ln_eps=0.0)):
        cfg = O.make_config(d_k=3, d_v=3, window=1, chunk=2, **kw)
        with pytest.raises(ValueError):
            run(cfg, np.zeros((2, 3)), np.zeros((2, 3)), np.zeros((2, 3)), *[np.zeros(2)] * 4)


# --------------------------------------------------------------------------- gated memory
# ATLAS summary, Atlas++: a gated MLP of three matrices.  Reading:
# f(x) = r + W2 (gelu(W1 x) .* (W3 x)), the GLU form with the memory's
# activation; weights W1 [h][D], W2 [d_v][h], W3 [h][D] in that order.

def gated_np(th, x, d, h, residual=True, ln_eps=None):
    W1 = th[:h * d].reshape(h, d)
    W2 = th[h * d:h * d + d * h].reshape(d, h)
    W3 = th[h * d + d * h:].reshape(h, d)
    u = W2 @ (gelu(W1 @ x) * (W3 @ x))
    if ln_eps is not None:
        u = ln_np(u, ln_eps)
    return (x if residual else 0) + u


@pytest.mark.parametrize("bias,residual,ln", [("l2", True, False), ("dot", True, False), ("l2", False, False),
                                              ("lp", True, False), ("l2", True, True)])
def test_gated_gradient_matches_finite_differences(bias, residual, ln):
    rng = np.random.default_rng(60)
    d, h, gamma, s = 3, 5, 0.6, 1.1
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=residual, bias=bias, grad_scale=s,
                        bias_p=3.0, gated=True, layernorm=ln, ln_eps=0.05)
    assert O.param_count(cfg) == 2 * h * d + d * h
    theta = rng.standard_normal(2 * h * d + d * h)
    x, v = rng.standard_normal(d), rng.standard_normal(d)

    def loss(th):
        f = gated_np(th, x, d, h, residual, 0.05 if ln else None)
        e = f - v
        if bias == "l2":
            return gamma * s * 0.5 * e @ e
        if bias == "dot":
            return -gamma * s * f @ v
        return gamma * s * np.sum(np.abs(e) ** 3) / 3

    g = O.token_grad(cfg, theta, x, x, v, gamma)
    eps = 1e-6
    fd = np.array([(loss(theta + eps * e) - loss(theta - eps * e)) / (2 * eps) for e in np.eye(theta.size)])
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_gated_retrieval_is_the_plain_forward_and_w3_zero_blocks_w1():
    rng = np.random.default_rng(61)
    N, d, h = 11, 4, 6
    q, k, v = rand_unit(rng, N, d), rand_unit(rng, N, d), rng.standard_normal((N, d))
    cfg = O.make_config(d_k=d, d_v=d, memory="mlp", hidden=h, residual=True, window=2, chunk=3,
                        momentum=True, gated=True)
    th = rng.standard_normal(2 * h * d + d * h)
    out, _ = run(cfg, q, k, v, np.zeros(N), rng.uniform(size=N), np.zeros(N), np.ones(N), th)
    want = np.array([gated_np(th, q[t], d, h) for t in range(N)])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)
    # W3 = 0: the branch is zero, so W1 and W2 get no gradient; W3 does
    th0 = th.copy()
    th0[h * d + d * h:] = 0.0
    g = O.token_grad(cfg, th0, k[0], k[0], v[0], 1.0)
    assert not g[:h * d + d * h].any() and g[h * d + d * h:].any()


# --------------------------------------------------------------------------- Muon
# ATLAS review, sec. 5 "Memory Optimization": Muon replaces gradient descent
# on the memory.  The oracle follows the published Muon optimizer (quintic
# Newton-Schulz, a, b, c = 3.4445, -4.7750, 2.0315, Frobenius normalisation).
NS_ABC = (3.4445, -4.7750, 2.0315)


def ns_by_svd(G, steps=5):
    """Newton-Schulz acts on the singular values alone: U f^steps(s/|G|_F) V^T
    with the scalar quintic f(x) = a x + b x^3 + c x^5."""
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    x = s / (np.linalg.norm(G) + 1e-7)
    a, b, c = NS_ABC
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return (U * x) @ Vt


@pytest.mark.parametrize("shape", [(4, 9), (9, 4), (6, 6), (1, 5), (32, 560)])
@pytest.mark.parametrize("steps", [1, 5])
def test_newton_schulz_is_the_singular_value_map(shape, steps):
    rng = np.random.default_rng(101)
    G = rng.standard_normal(shape) * 3.0
    np.testing.assert_allclose(O.newton_schulz(G, steps), ns_by_svd(G, steps), rtol=0, atol=1e-12)


def test_newton_schulz_of_a_rank_one_matrix():
    """u w^T has one singular value |u||w|, so NS gives f^5(1 - tiny) u^ w^^T."""
    rng = np.random.default_rng(102)
    u, w = rng.standard_normal(7), rng.standard_normal(11)
    G = np.outer(u, w)
    x = np.linalg.norm(G) / (np.linalg.norm(G) + 1e-7)
    a, b, c = NS_ABC
    for _ in range(5):
        x = a * x + b * x ** 3 + c * x ** 5
    want = x * np.outer(u / np.linalg.norm(u), w / np.linalg.norm(w))
    np.testing.assert_allclose(O.newton_schulz(G, 5), want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("b", [1, 4])
@pytest.mark.parametrize("bias", ["l2", "dot"])
def test_muon_without_momentum_is_a_normalised_delta_rule(b, bias):
    """Linear memory, c = 1, no momentum: each token's gradient is the rank-one
    (M0 k - v) k^T (l2; -v k^T for the dot bias) at the chunk-start memory M0,
    so Muon moves M by -theta f^5(~1) e^ k^^T."""
    rng = np.random.default_rng(103)
    N, dk, dv = 23, 6, 4
    cfg = O.make_config(d_k=dk, d_v=dv, window=1, chunk=b, bias=bias, optimizer="muon")
    q, k, v = rand_unit(rng, N, dk), rng.standard_normal((N, dk)) * 0.7, rng.standard_normal((N, dv))
    alpha, theta, gamma = rng.uniform(0, 0.2, N), rng.uniform(0.05, 0.3, N), rng.uniform(0.5, 1.5, N)
    M = rng.standard_normal((dv, dk)) * 0.3
    out, st = run(cfg, q, k, v, alpha, np.zeros(N), theta, gamma, M)
    a_, b_, c_ = NS_ABC
    for t0 in range(0, N, b):
        M0 = M.copy()
        for t in range(t0, min(N, t0 + b)):
            e = (M0 @ k[t] - v[t]) if bias == "l2" else -v[t]
            g = gamma[t] * np.outer(e, k[t])
            x = np.linalg.norm(g) / (np.linalg.norm(g) + 1e-7)
            for _ in range(5):
                x = a_ * x + b_ * x ** 3 + c_ * x ** 5
            M = (1 - alpha[t]) * M - theta[t] * x * np.outer(e / np.linalg.norm(e), k[t] / np.linalg.norm(k[t]))
            np.testing.assert_allclose(out[t], M @ q[t], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(st["mem"][0].reshape(dv, dk), M, rtol=1e-11, atol=1e-13)


def test_muon_scalar_memory():
    """A 1x1 memory with momentum, window c = 2 and chunk b = 3: NS of a
    scalar s is f^5(|s| / (|s| + 1e-7)) sign(s)."""
    rng = np.random.default_rng(104)
    N, c, b = 31, 2, 3
    q, k, v = rng.standard_normal((N, 1)), rng.standard_normal((N, 1)), rng.standard_normal((N, 1))
    al, et, th, ga = rng.uniform(0, 0.3, N), rng.uniform(0.2, 0.9, N), rng.uniform(0.05, 0.4, N), rng.uniform(0.3, 1.2, N)
    cfg = O.make_config(d_k=1, d_v=1, window=c, chunk=b, momentum=True, optimizer="muon")
    a_, b_, c_ = NS_ABC

    def ns(s):
        x = abs(s) / (abs(s) + 1e-7)
        for _ in range(5):
            x = a_ * x + b_ * x ** 3 + c_ * x ** 5
        return x * np.sign(s)

    m, S, want = 0.5, 0.0, []
    for t0 in range(0, N, b):
        m0 = m
        for t in range(t0, min(N, t0 + b)):
            g = sum(ga[i] * (m0 * k[i, 0] - v[i, 0]) * k[i, 0] for i in range(max(0, t - c + 1), t + 1))
            S = et[t] * S + g
            m = (1 - al[t]) * m - th[t] * ns(S)
            want.append(m * q[t, 0])
    out, st = run(cfg, q, k, v, al, et, th, ga, [0.5])
    np.testing.assert_allclose(out[:, 0], want, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(st["mom"][0, 0], S, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("memory", ["linear", "mlp"])
def test_muon_orthogonalises_each_weight_matrix(memory):
    """Window c = 2, chunk b = 3, momentum: the replay keeps S per weight
    matrix, takes each matrix's NS through its SVD, and uses the oracle's
    token gradient (itself pinned against finite differences)."""
    rng = np.random.default_rng(105)
    N, dk, dv, h, c, b = 17, 4, 4, 5, 2, 3
    kw = dict(memory="mlp", hidden=h, residual=True) if memory == "mlp" else {}
    cfg = O.make_config(d_k=dk, d_v=dv, window=c, chunk=b, momentum=True, optimizer="muon", **kw)
    P = O.param_count(cfg)
    q, k, v = rand_unit(rng, N, dk), rand_unit(rng, N, dk), rng.standard_normal((N, dv))
    al, et, th, ga = rng.uniform(0, 0.2, N), rng.uniform(0.3, 0.9, N), rng.uniform(0.05, 0.3, N), rng.uniform(0.5, 1.5, N)
    W = rng.standard_normal(P) * 0.4
    out, st = run(cfg, q, k, v, al, et, th, ga, W)
    shapes = [(dv, dk)] if memory == "linear" else [(h, dk), (dv, h)]
    S = np.zeros(P)
    for t0 in range(0, N, b):
        W0 = W.copy()
        for t in range(t0, min(N, t0 + b)):
            g = sum(O.token_grad(cfg, W0, k[i], k[i], v[i], ga[i]) for i in range(max(0, t - c + 1), t + 1))
            S = et[t] * S + g
            O_, off = np.zeros(P), 0
            for r_, c_ in shapes:
                O_[off:off + r_ * c_] = ns_by_svd(S[off:off + r_ * c_].reshape(r_, c_)).ravel()
                off += r_ * c_
            W = (1 - al[t]) * W - th[t] * O_
            np.testing.assert_allclose(out[t], O.memory_apply(cfg, W, q[t], q[t]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(st["mem"][0], W, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(st["mom"][0], S, rtol=1e-10, atol=1e-12)


def test_muon_config_checks():
    cfg = O.make_config(d_k=2, d_v=2, optimizer="muon", ns_steps=0)
    cfg.n_seq, cfg.seq_len = 1, 0
    st = O.empty_state(cfg)
    z = np.zeros((1, 0))
    with pytest.raises(Exception):
        O.forward(cfg, np.zeros((1, 0, 2)), np.zeros((1, 0, 2)), np.zeros((1, 0, 2)), z, z, z, z, st)
