"""Pins for the fp64 oracle, checked against facts that do not come from the
oracle itself: a hand-derived worked example, closed forms, special cases that
reduce to the pages' level-1 references and parallel form, exact invariants of
the delta rule, the chunk algebra, and agreement between the C oracle and its
numpy twin.  A mutation test shows that plausible mistakes fail at least one
pin.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(seed, T=21, H=2, dk=8, dv=6, h0=True, lengths=None, a_scale=1.0, A_hi=math.log(16)):
    r = RNG(seed)
    if lengths is not None:
        T = int(sum(lengths))
    d = dict(q=unit(r.standard_normal((T, H, dk))), k=unit(r.standard_normal((T, H, dk))),
             v=r.standard_normal((T, H, dv)), a=a_scale * r.standard_normal((T, H, dk)),
             b=r.standard_normal((T, H)), A_log=r.uniform(0, A_hi, H),
             dt_bias=r.uniform(-1, 1, (H, dk)))
    n_seq = 1 if lengths is None else len(lengths)
    d["h0"] = 0.3 * r.standard_normal((n_seq, H, dv, dk)) if h0 else None
    d["cu_seqlens"] = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)])
    d["scale"] = dk ** -0.5
    return d


def run_np(d):
    return ref.recurrent(**d)


def run_c(d):
    return oracle.fwd(**d, n_threads=2)


IMPLS = {"numpy": run_np, "c": run_c}


def close(x, y, tol):
    return np.max(np.abs(np.asarray(x) - np.asarray(y))) <= tol


# ----------------------------------------------------------------------------
# pins written as predicates over an implementation, so that the mutation
# test can reuse them
# ----------------------------------------------------------------------------
def pin_worked_example(impl):
    """I1: hand-derived two-token example (tests/golden/worked_example_i1.json)."""
    g = json.load(open(os.path.join(GOLD, "worked_example_i1.json")))
    x = g["inputs"]
    d = dict(q=np.array(x["q"]).reshape(2, 1, 1), k=np.array(x["k"]).reshape(2, 1, 1),
             v=np.array(x["v"]).reshape(2, 1, 1), a=np.array(x["a"]).reshape(2, 1, 1),
             b=np.array(x["b"]).reshape(2, 1), A_log=np.array([x["A_log"]]),
             dt_bias=np.array([[x["dt_bias"]]]), h0=None, cu_seqlens=None, scale=x["scale"])
    o, hT = impl(d)
    return close(o.ravel(), g["expected"]["o"], 1e-14) and close(hT.ravel(), [g["expected"]["S_T"]], 1e-14)


def pin_matrix_form(impl):
    """The literal product form S D (I - beta k k^T) + beta v k^T of the
    recurrence, evaluated with explicit matrices, on random inputs with
    gates, an initial state and two sequences (one of them ragged)."""
    ok = True
    for seed, kw in [(1, {}), (2, dict(lengths=[5, 9], dk=5, dv=7)), (3, dict(dk=6, dv=6, a_scale=3.0))]:
        d = rand_inputs(seed, **kw)
        o, hT = impl(d)
        o2, hT2 = ref.recurrent_matrix_form(**d)
        ok &= close(o, o2, 1e-12) and close(hT, hT2, 1e-12)
    return ok


def pin_gate_closed_form(impl):
    """I2 with exactly known gates: beta = 0 (b = -800), A_log = 0 and
    a = ln(2^m - 1), so softplus(a) = m ln 2 and e^{g} = 2^{-m}.  Then
    S_T = S0 * 2^{-sum_t m_t} column by column, and
    o_t = S0 (scale q_t * 2^{-sum_{j<=t} m_j})."""
    r = RNG(7)
    T, H, dk, dv = 9, 2, 5, 4
    m = r.integers(0, 4, (T, H, dk)).astype(float)
    a = np.where(m > 0, np.log(np.maximum(2.0 ** m - 1.0, 1e-300)), -800.0)
    # m = 0 -> softplus(-800) = e^{-800} ~ 0 -> e^g = 1
    d = dict(q=unit(r.standard_normal((T, H, dk))), k=unit(r.standard_normal((T, H, dk))),
             v=r.standard_normal((T, H, dv)), a=a, b=np.full((T, H), -800.0),
             A_log=np.zeros(H), dt_bias=np.zeros((H, dk)),
             h0=r.standard_normal((1, H, dv, dk)), cu_seqlens=None, scale=0.5)
    o, hT = impl(d)
    cum = np.cumsum(m, axis=0)                                      # [T,H,dk]
    S0 = d["h0"][0]
    o_exp = np.einsum("hvc,thc->thv", S0, 0.5 * d["q"] * 2.0 ** (-cum))
    hT_exp = S0 * 2.0 ** (-cum[-1])[:, None, :]
    return close(o, o_exp, 1e-13) and close(hT[0], hT_exp, 1e-13)


def pin_no_gate_no_beta(impl):
    """I3: g = 0 (A_log = -1000 -> exp = 0) and beta = 0 give o_t = S0 (scale q_t), S_T = S0."""
    r = RNG(8)
    d = rand_inputs(8)
    d["A_log"] = np.full(2, -1000.0)
    d["b"] = np.full_like(d["b"], -800.0)
    o, hT = impl(d)
    o_exp = d["scale"] * np.einsum("hvc,thc->thv", d["h0"][0], d["q"])
    return close(o, o_exp, 1e-13) and close(hT, d["h0"], 1e-13)


def _onehot_inputs(seed, gated, T=7, H=2, dk=8, dv=5):
    r = RNG(seed)
    perm = np.stack([r.permutation(dk)[:T] for _ in range(H)], axis=1)  # [T,H]
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            k[t, h, perm[t, h]] = 1.0
    d = dict(q=r.standard_normal((T, H, dk)), k=k, v=r.standard_normal((T, H, dv)),
             a=r.standard_normal((T, H, dk)) if gated else np.zeros((T, H, dk)),
             b=r.standard_normal((T, H)) if gated else np.full((T, H), 40.0),
             A_log=r.uniform(0, 1.5, H) if gated else np.full(H, -1000.0),
             dt_bias=r.uniform(-1, 1, (H, dk)), h0=None, cu_seqlens=None, scale=0.7)
    return d, perm


def pin_onehot_gated_parallel(impl):
    """I4: distinct one-hot keys and S0 = 0 make S'k_t = 0, so u_t = beta_t v_t
    and o_t = sum_{j<=t} beta_j v_j (scale q_t)[pi_j] e^{G_t[pi_j] - G_j[pi_j]}:
    a gated parallel form computed by an explicit double loop."""
    d, perm = _onehot_inputs(11, gated=True)
    o, _ = impl(d)
    g = -np.exp(d["A_log"])[:, None] * np.log1p(np.exp(d["a"] + d["dt_bias"]))   # direct softplus
    beta = 1.0 / (1.0 + np.exp(-d["b"]))
    G = np.cumsum(g, axis=0)
    T, H, dv = d["v"].shape
    o_exp = np.zeros_like(o)
    for h in range(H):
        for t in range(T):
            for j in range(t + 1):
                c = perm[j, h]
                o_exp[t, h] += beta[j, h] * d["v"][j, h] * d["scale"] * d["q"][t, h, c] * \
                    math.exp(G[t, h, c] - G[j, h, c])
    return close(o, o_exp, 1e-12)


def pin_onehot_level1(impl):
    """I4 with g = 0 and beta = 1: the output equals the parallel form
    tril((scale Q) K^T) V and the level-1 references A, B, D of the TileLang
    page (which all use the same one-hot keys)."""
    d, _ = _onehot_inputs(12, gated=False, T=8)
    o, _ = impl(d)
    ok = True
    for h in range(d["q"].shape[1]):
        par = ref.parallel_form(d["q"][:, h], d["k"][:, h], d["v"][:, h], scale=d["scale"])
        ok &= close(o[:, h], par, 1e-13)
    Q, K, V = (d[x][None] for x in ("q", "k", "v"))
    for l1 in (ref.level1_recurrent(d["scale"] * Q, K, V), ref.level1_chunked(d["scale"] * Q, K, V, 4),
               ref.level1_dv_slab(d["scale"] * Q, K, V, 4, 2)):
        ok &= close(o, l1[0], 1e-13)
    return ok


def pin_unit_key_readback(impl):
    """I5: beta = 1 and |k_t| = 1 give S_t k_t = v_t after every step, for any
    gates and any history, so q_t = k_t / scale reads o_t = v_t."""
    d = rand_inputs(13, T=17, dk=8, dv=5)
    d["b"] = np.full_like(d["b"], 40.0)          # sigmoid(40) == 1 in fp64
    d["q"] = d["k"] / d["scale"]
    o, _ = impl(d)
    return close(o, d["v"], 1e-12)


def pin_orthonormal_memory(impl):
    """I5 (spec invariant): orthonormal keys, g = 0, beta = 1, S0 = 0:
    h_T k_j = v_j for every written j."""
    r = RNG(14)
    dk, dv, T, H = 8, 6, 6, 2
    k = np.zeros((T, H, dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
        k[:, h] = Qm[:, :T].T
    d = dict(q=r.standard_normal((T, H, dk)), k=k, v=r.standard_normal((T, H, dv)),
             a=r.standard_normal((T, H, dk)), b=np.full((T, H), 40.0), A_log=np.full(H, -1000.0),
             dt_bias=np.zeros((H, dk)), h0=None, cu_seqlens=None, scale=1.0)
    _, hT = impl(d)
    read = np.einsum("hvc,thc->thv", hT[0], k)
    return close(read, d["v"], 1e-12)


def pin_varlen_is_separate(impl):
    """I8: packed sequences equal separate runs, bitwise."""
    lengths = [5, 1, 12]
    d = rand_inputs(15, lengths=lengths)
    o, hT = impl(d)
    ok = True
    cu = d["cu_seqlens"]
    for s in range(len(lengths)):
        sl = slice(cu[s], cu[s + 1])
        ds = dict(d, q=d["q"][sl], k=d["k"][sl], v=d["v"][sl], a=d["a"][sl], b=d["b"][sl],
                  h0=d["h0"][s:s + 1], cu_seqlens=None)
        os_, hs = impl(ds)
        ok &= np.array_equal(os_, o[sl]) and np.array_equal(hs[0], hT[s])
    return ok


def pin_continuation(impl):
    """I9: run(x[:n]) -> h_n, then run(x[n:], h0=h_n) equals run(x)."""
    d = rand_inputs(16, T=40)
    o, hT = impl(d)
    ok = True
    for n in (16, 23):
        d1 = dict(d, q=d["q"][:n], k=d["k"][:n], v=d["v"][:n], a=d["a"][:n], b=d["b"][:n])
        o1, h1 = impl(d1)
        d2 = dict(d, q=d["q"][n:], k=d["k"][n:], v=d["v"][n:], a=d["a"][n:], b=d["b"][n:], h0=h1)
        o2, h2 = impl(d2)
        ok &= close(np.concatenate([o1, o2]), o, 1e-13) and close(h2, hT, 1e-13)
    return ok


PINS = [pin_worked_example, pin_matrix_form, pin_gate_closed_form, pin_no_gate_no_beta,
        pin_onehot_gated_parallel, pin_onehot_level1, pin_unit_key_readback,
        pin_orthonormal_memory, pin_varlen_is_separate, pin_continuation]


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin, impl):
    with np.errstate(over="ignore"):
        assert pin(IMPLS[impl])


# ----------------------------------------------------------------------------
# C oracle vs numpy twin, at a larger shape
# ----------------------------------------------------------------------------
def test_c_matches_numpy():
    d = rand_inputs(21, lengths=[33, 7, 50], H=3, dk=16, dv=12)
    o1, h1 = run_np(d)
    o2, h2 = run_c(d)
    assert close(o1, o2, 1e-13) and close(h1, h2, 1e-13)


def test_c_chain_subset():
    d = rand_inputs(22, lengths=[9, 14], H=3)
    o_all, h_all = run_c(d)
    o_sub, h_sub = oracle.fwd(**d, chains=[4], n_threads=1)       # seq 1, head 1
    cu = d["cu_seqlens"]
    assert np.array_equal(o_sub[cu[1]:cu[2], 1], o_all[cu[1]:cu[2], 1])
    assert np.array_equal(h_sub[1, 1], h_all[1, 1])
    assert not o_sub[:, 0].any()


# ----------------------------------------------------------------------------
# chunk algebra (I6): the fp64 chunkwise form equals the token recurrence
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 2, 4, 8, 16])
def test_chunkwise_equals_recurrent(C):
    d = rand_inputs(31, lengths=[37, 16, 5], H=2, dk=8, dv=6)
    o1, h1 = ref.recurrent(**d)
    o2, h2 = ref.chunkwise(**d, C=C)
    assert close(o1, o2, 1e-12) and close(h1, h2, 1e-12)


def test_chunkwise_strong_decay():
    """Per-token decays of hundreds of nats: the pairwise-exponential chunk
    form still matches (no overflow anywhere)."""
    d = rand_inputs(32, T=48, a_scale=1.0)
    d["a"][5:9] = 30.0
    d["A_log"] = np.array([math.log(16), math.log(16)])
    o1, h1 = ref.recurrent(**d)
    o2, h2 = ref.chunkwise(**d, C=16)
    assert np.isfinite(o2).all() and close(o1, o2, 1e-12) and close(h1, h2, 1e-12)


def test_neumann_inverse_and_nilpotency():
    r = RNG(33)
    C, dk = 16, 32
    kc = unit(r.standard_normal((C, dk)))
    qc = unit(r.standard_normal((C, dk)))
    g = -np.exp(1.0) * ref.softplus(r.standard_normal((C, dk)))
    beta = ref.sigmoid(r.standard_normal(C))
    _, L, Mqk, INV = ref.chunk_matrices(qc, kc, g, beta, dk ** -0.5)
    assert np.array_equal(np.linalg.matrix_power(L, 16), np.zeros((C, C)))   # L^16 = 0 exactly
    assert np.max(np.abs(np.triu(L))) == 0.0 and np.max(np.abs(np.triu(Mqk, 1))) == 0.0
    assert close((np.eye(C) - L) @ INV, np.eye(C), 1e-14)
    assert close(INV, np.linalg.inv(np.eye(C) - L), 1e-13)


def test_worked_example_chunk_quantities():
    g = json.load(open(os.path.join(GOLD, "worked_example_i1.json")))
    kc = np.array([[1.0], [1.0]])
    G, L, Mqk, INV = ref.chunk_matrices(kc, kc, np.full((2, 1), -math.log(2)), np.array([0.5, 0.5]), 1.0)
    assert close(L, g["expected"]["L"], 1e-15) and close(Mqk, g["expected"]["Mqk"], 1e-15)
    u = np.array([1.0, 2.0])
    assert close(INV @ u, g["expected"]["U"], 1e-15)


# ----------------------------------------------------------------------------
# decode (I10): one step of the forward recurrence on L2-normalised q, k
# ----------------------------------------------------------------------------
def _decode_inputs(seed, B=6, H=2, HV=4, K=8, V=5, P=9):
    r = RNG(seed)
    d = dict(qkv=r.standard_normal((B, 2 * H * K + HV * V)), a=r.standard_normal((B, HV * K)),
             b=r.standard_normal((B, HV)), A_log=r.uniform(0, math.log(16), HV),
             dt_bias=r.uniform(-1, 1, HV * K))
    pool = 0.3 * r.standard_normal((P, HV, V, K))
    idx = r.permutation(P)[:B]
    idx[[1, 4]] = -1
    return d, pool, idx


@pytest.mark.parametrize("which", ["numpy", "c"])
def test_decode_is_one_forward_step(which):
    B, H, HV, K, V, P = 6, 2, 4, 8, 5, 9
    d, pool, idx = _decode_inputs(41)
    if which == "numpy":
        o, newpool = ref.decode_step(**d, pool=pool, state_idx=idx, H=H, HV=HV, K=K, V=V)
    else:
        o, newpool = oracle.decode(**d, pool=pool, state_idx=idx, H=H, HV=HV, K=K, V=V, n_threads=2)
    for n in range(B):
        if idx[n] < 0:
            assert not o[n].any()
            continue
        for hv in range(HV):
            hq = hv // (HV // H)
            x = d["qkv"][n]
            q = x[hq * K:(hq + 1) * K]
            k = x[H * K + hq * K:H * K + (hq + 1) * K]
            q = q / np.sqrt(q @ q + 1e-6)
            k = k / np.sqrt(k @ k + 1e-6)
            v = x[2 * H * K + hv * V:2 * H * K + (hv + 1) * V]
            one = dict(q=q[None, None], k=k[None, None], v=v[None, None],
                       a=d["a"][n, hv * K:(hv + 1) * K][None, None], b=d["b"][n, hv][None, None],
                       A_log=d["A_log"][hv:hv + 1], dt_bias=d["dt_bias"][hv * K:(hv + 1) * K][None],
                       h0=pool[idx[n], hv][None, None], cu_seqlens=None, scale=K ** -0.5)
            oo, hh = ref.recurrent_matrix_form(**one)
            assert close(o[n, hv], oo[0, 0], 1e-13)
            assert close(newpool[idx[n], hv], hh[0, 0], 1e-13)
    untouched = np.setdiff1d(np.arange(P), idx[idx >= 0])
    assert np.array_equal(newpool[untouched], pool[untouched])


def test_decode_c_matches_numpy():
    d, pool, idx = _decode_inputs(42, B=16, H=2, HV=6, K=16, V=12, P=20)
    o1, p1 = ref.decode_step(**d, pool=pool, state_idx=idx, H=2, HV=6, K=16, V=12)
    o2, p2 = oracle.decode(**d, pool=pool, state_idx=idx, H=2, HV=6, K=16, V=12, n_threads=2)
    assert close(o1, o2, 1e-13) and close(p1, p2, 1e-13)


# ----------------------------------------------------------------------------
# extend (I14): T decode steps per row in one call are the forward recurrence
# over those T tokens from the slot's state (matrix form, numpy), on
# L2-normalised q, k; pads give zero outputs and leave every slot alone.
# ----------------------------------------------------------------------------
def _extend_inputs(seed, B=5, T=7, H=2, HV=4, K=8, V=5, P=9):
    r = RNG(seed)
    d = dict(qkv=r.standard_normal((B, T, 2 * H * K + HV * V)), a=r.standard_normal((B, T, HV * K)),
             b=r.standard_normal((B, T, HV)), A_log=r.uniform(0, math.log(16), HV),
             dt_bias=r.uniform(-1, 1, HV * K))
    pool = 0.3 * r.standard_normal((P, HV, V, K))
    idx = r.permutation(P)[:B]
    idx[2] = -1
    return d, pool, idx


def test_extend_is_a_forward_chain():
    B, T, H, HV, K, V, P = 5, 7, 2, 4, 8, 5, 9
    d, pool, idx = _extend_inputs(61)
    o, newpool = oracle.extend(**d, pool=pool, state_idx=idx, H=H, HV=HV, K=K, V=V, n_threads=2)
    assert o.shape == (B, T, HV, V)
    for n in range(B):
        if idx[n] < 0:
            assert not o[n].any()
            continue
        for hv in range(HV):
            hq = hv // (HV // H)
            x = d["qkv"][n]
            q = x[:, hq * K:(hq + 1) * K]
            k = x[:, H * K + hq * K:H * K + (hq + 1) * K]
            q = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
            k = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
            v = x[:, 2 * H * K + hv * V:2 * H * K + (hv + 1) * V]
            chain = dict(q=q[:, None], k=k[:, None], v=v[:, None], a=d["a"][n][:, None, hv * K:(hv + 1) * K],
                         b=d["b"][n][:, hv:hv + 1], A_log=d["A_log"][hv:hv + 1],
                         dt_bias=d["dt_bias"][hv * K:(hv + 1) * K][None], h0=pool[idx[n], hv][None, None],
                         cu_seqlens=None, scale=K ** -0.5)
            oo, hh = ref.recurrent_matrix_form(**chain)
            assert close(o[n, :, hv], oo[:, 0], 1e-12)
            assert close(newpool[idx[n], hv], hh[0, 0], 1e-12)
    untouched = np.setdiff1d(np.arange(P), idx[idx >= 0])
    assert np.array_equal(newpool[untouched], pool[untouched])


def test_extend_equals_successive_decode_steps():
    B, T, H, HV, K, V = 5, 7, 2, 4, 8, 5
    d, pool, idx = _extend_inputs(62)
    o, newpool = oracle.extend(**d, pool=pool, state_idx=idx, H=H, HV=HV, K=K, V=V, n_threads=2)
    p = pool
    for t in range(T):
        ot, p = oracle.decode(d["qkv"][:, t], d["a"][:, t], d["b"][:, t], d["A_log"], d["dt_bias"], p, idx,
                              H=H, HV=HV, K=K, V=V, n_threads=2)
        assert np.array_equal(o[:, t], ot)
    assert np.array_equal(newpool, p)
    o0, p0 = oracle.extend(d["qkv"][:, :0], d["a"][:, :0], d["b"][:, :0], d["A_log"], d["dt_bias"], pool, idx,
                           H=H, HV=HV, K=K, V=V, n_threads=2)
    assert o0.shape == (B, 0, HV, V) and np.array_equal(p0, pool)


# ----------------------------------------------------------------------------
# chunk-boundary states (I16): the state entering chunk c of a sequence is the
# final state of the same recurrence run over the sequence's first C*c tokens
# (brute force over prefixes); row order follows the sequences.
# ----------------------------------------------------------------------------
def test_chunk_states_are_prefix_final_states():
    r = RNG(81)
    H, dk, dv, C = 2, 6, 5, 4
    lens = [9, 0, 4, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k = r.standard_normal((T, H, dk)), r.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v, a, b = r.standard_normal((T, H, dv)), r.standard_normal((T, H, dk)), r.standard_normal((T, H))
    A_log, dt_bias = r.uniform(0, 1, H), r.uniform(-1, 1, (H, dk))
    h0 = 0.1 * r.standard_normal((len(lens), H, dv, dk))
    o, hT, hc = oracle.fwd(q, k, v, a, b, A_log, dt_bias, h0=h0, cu_seqlens=cu, chunk_states=C, n_threads=2)
    o2, hT2 = oracle.fwd(q, k, v, a, b, A_log, dt_bias, h0=h0, cu_seqlens=cu, n_threads=2)
    assert np.array_equal(o, o2) and np.array_equal(hT, hT2)
    assert hc.shape == (sum((n + C - 1) // C for n in lens), H, dv, dk)
    row = 0
    for s, n in enumerate(lens):
        for c in range((n + C - 1) // C):
            t0 = int(cu[s])
            sl = slice(t0, t0 + C * c)
            _, want = ref.recurrent_matrix_form(q[sl], k[sl], v[sl], a[sl], b[sl], A_log, dt_bias,
                                                h0=h0[s:s + 1], cu_seqlens=None)
            assert close(hc[row], want[0], 1e-12), (s, c)
            row += 1
    assert row == hc.shape[0]


# ----------------------------------------------------------------------------
# gradients (I17): the fp64 autograd gradients of the PyTorch recurrence match
# central finite differences of the C oracle's loss sum(o * do) + sum(h_T * dh_T)
# for every input (two packed sequences, one with a ragged length, with h0).
# ----------------------------------------------------------------------------
def test_gradients_match_finite_differences():
    from oracle import grad
    r = RNG(91)
    H, dk, dv = 2, 4, 3
    cu = np.array([0, 5, 12])
    T = int(cu[-1])
    x = dict(q=r.standard_normal((T, H, dk)), k=r.standard_normal((T, H, dk)), v=r.standard_normal((T, H, dv)),
             a=r.standard_normal((T, H, dk)), b=r.standard_normal((T, H)), A_log=r.uniform(-1, 1, H),
             dt_bias=r.uniform(-1, 1, (H, dk)), h0=0.3 * r.standard_normal((2, H, dv, dk)))
    x["k"] /= np.linalg.norm(x["k"], axis=-1, keepdims=True)
    do, dhT = r.standard_normal((T, H, dv)), r.standard_normal((2, H, dv, dk))
    scale = 0.7

    def loss(xx):
        o, hT = oracle.fwd(xx["q"], xx["k"], xx["v"], xx["a"], xx["b"], xx["A_log"], xx["dt_bias"], h0=xx["h0"],
                           cu_seqlens=cu, scale=scale, n_threads=1)
        return float((o * do).sum() + (hT * dhT).sum())

    g = grad.backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["A_log"], x["dt_bias"], do, h0=x["h0"],
                      dh_T=dhT, cu_seqlens=cu, scale=scale)
    names = dict(q="dq", k="dk", v="dv", a="da", b="db", A_log="dA_log", dt_bias="ddt_bias", h0="dh0")
    eps = 1e-6
    for name, gname in names.items():
        flat = x[name].reshape(-1)
        for i in r.choice(flat.size, size=min(6, flat.size), replace=False):
            xp = {k_: np.array(v_, copy=True) for k_, v_ in x.items()}
            xm = {k_: np.array(v_, copy=True) for k_, v_ in x.items()}
            xp[name].reshape(-1)[i] += eps
            xm[name].reshape(-1)[i] -= eps
            fd = (loss(xp) - loss(xm)) / (2 * eps)
            got = g[gname].reshape(-1)[i]
            assert abs(fd - got) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, got)


# ----------------------------------------------------------------------------
# short convolution before decode (I15): width 1 is silu of an affine map;
# T updates from a zero state are the causal convolution of the whole input
# sequence (numpy's convolve), and the state ends holding the last W-1 inputs;
# pads give zero and leave their slots alone.
# ----------------------------------------------------------------------------
def test_conv_update_width1_is_silu():
    from scipy.special import expit
    r = RNG(71)
    B, D = 5, 12
    x, w, bias = r.standard_normal((B, D)), r.standard_normal((D, 1)), r.standard_normal(D)
    idx = np.arange(B)
    idx[3] = -1
    y, _ = oracle.conv_update(x, None, w, bias, idx)
    z = w[:, 0] * x + bias
    want = z * expit(z)
    want[3] = 0.0
    assert close(y, want, 1e-15)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv_updates_are_a_causal_convolution(W):
    r = RNG(72 + W)
    B, D, T, P = 4, 10, 9, 7
    xs = r.standard_normal((T, B, D))
    w, bias = r.standard_normal((D, W)), r.standard_normal(D)
    idx = np.array([5, -1, 0, 3])
    cs0 = r.standard_normal((P, W - 1, D))
    cs0[idx[idx >= 0]] = 0.0                      # live slots start empty
    cs = cs0
    ys = []
    for t in range(T):
        y, cs = oracle.conv_update(xs[t], cs, w, bias, idx)
        ys.append(y)
    ys = np.stack(ys)                             # [T, B, D]
    for n in range(B):
        if idx[n] < 0:
            assert not ys[:, n].any()
            continue
        for c in range(D):
            z = bias[c] + np.convolve(xs[:, n, c], w[c, ::-1])[:T]
            assert close(ys[:, n, c], z / (1 + np.exp(-z)), 1e-13)
        assert np.array_equal(cs[idx[n]], xs[T - W + 1:, n, :])
    others = np.setdiff1d(np.arange(P), idx[idx >= 0])
    assert np.array_equal(cs[others], cs0[others])


def test_conv_decode_composes():
    r = RNG(75)
    B, H, HV, K, V, P, W = 3, 1, 2, 8, 4, 5, 4
    D = 2 * H * K + HV * V
    x = r.standard_normal((B, D))
    cs = r.standard_normal((P, W - 1, D))
    w, bias = r.standard_normal((D, W)), r.standard_normal(D)
    d = dict(a=r.standard_normal((B, HV * K)), b=r.standard_normal((B, HV)),
             A_log=r.uniform(0, 1, HV), dt_bias=r.uniform(-1, 1, HV * K))
    pool = 0.3 * r.standard_normal((P, HV, V, K))
    idx = np.array([4, -1, 1])
    o, newpool, newcs = oracle.conv_decode(x, cs, w, bias, **d, pool=pool, state_idx=idx, H=H, HV=HV,
                                           K=K, V=V, n_threads=1)
    y, cs2 = oracle.conv_update(x, cs, w, bias, idx)
    o2, p2 = oracle.decode(y, **d, pool=pool, state_idx=idx, H=H, HV=HV, K=K, V=V, n_threads=1)
    assert np.array_equal(o, o2) and np.array_equal(newpool, p2) and np.array_equal(newcs, cs2)


# ----------------------------------------------------------------------------
# level-1 references of the TileLang page (I11): they agree to fp64 rounding
# (the page reports 1e-15-level max-abs and 1e-16-level rel-L2), and the two
# deliberate structural bugs give O(1) errors.
# ----------------------------------------------------------------------------
def rel_l2(x, y):
    return np.linalg.norm(x - y) / np.linalg.norm(y)


def test_level1_references_agree():
    r = RNG(51)
    Q, K, V = (r.standard_normal((2, 12, 2, 4)) for _ in range(3))
    A = ref.level1_recurrent(Q, K, V)
    B = ref.level1_chunked(Q, K, V, 4)
    assert np.max(np.abs(A - B)) < 1e-13 and rel_l2(B, A) < 1e-15
    assert rel_l2(ref.level1_chunked(Q, K, V, 4, right_shift=False), A) > 0.1
    Q, K = (r.standard_normal((2, 256, 3, 64)) for _ in range(2))
    V = r.standard_normal((2, 256, 3, 128))
    A = ref.level1_recurrent(Q, K, V)
    D = [ref.level1_dv_slab(Q, K, V, 64, bd) for bd in (32, 64, 128)]
    for x in D:
        assert rel_l2(x, A) < 1e-14
    assert np.array_equal(D[0], D[1]) and np.array_equal(D[1], D[2])   # DV slabs: bitwise
    assert rel_l2(ref.level1_dv_slab(Q, K, V, 64, 32, update_after_write=False), A) > 0.1


# ----------------------------------------------------------------------------
# mutation test: plausible mistakes in the recurrence fail at least one pin
# ----------------------------------------------------------------------------
def _mutant(kind):
    def impl(d):
        q, k, v, b = (np.asarray(d[x], float) for x in ("q", "k", "v", "b"))
        T, H, dk = q.shape
        dv = v.shape[-1]
        scale = d["scale"]
        A = np.exp(np.asarray(d["A_log"], float))
        sp = ref.softplus(np.asarray(d["a"], float) + d["dt_bias"])
        if kind == "relu_gate":
            sp = np.maximum(np.asarray(d["a"], float) + d["dt_bias"], 0.0)
        if kind == "no_A":
            A = np.ones_like(A)
        g = -A[:, None] * sp
        beta = ref.sigmoid(b)
        bounds = ref._seq_bounds(T, d["cu_seqlens"])
        o = np.zeros((T, H, dv))
        hT = np.zeros((len(bounds), H, dv, dk))
        for s, (t0, t1) in enumerate(bounds):
            S = np.zeros((H, dv, dk)) if d["h0"] is None else np.array(d["h0"][s], float)
            for t in range(t0, t1):
                Sprev = S
                if kind == "decay_value_axis":       # rows decayed instead of key columns
                    m = min(dv, dk)
                    rows = np.ones((H, dv))
                    rows[:, :m] = np.exp(g[t][:, :m])
                    S = S * rows[:, :, None]
                else:
                    S = S * np.exp(g[t])[:, None, :]
                base = Sprev if kind == "delta_before_decay" else S
                Sk = np.einsum("hvc,hc->hv", base, k[t])
                if kind == "delta_sign":
                    u = beta[t][:, None] * (v[t] + Sk)
                elif kind == "beta_on_v_only":
                    u = beta[t][:, None] * v[t] - Sk
                else:
                    u = beta[t][:, None] * (v[t] - Sk)
                if kind == "read_before_write":
                    o[t] = scale * np.einsum("hvc,hc->hv", S, q[t])
                S = S + u[:, :, None] * k[t][:, None, :]
                if kind != "read_before_write":
                    sc = 1.0 if kind == "no_scale" else scale
                    o[t] = sc * np.einsum("hvc,hc->hv", S, q[t])
            hT[s] = S
        return o, hT
    return impl


MUTANTS = ["relu_gate", "no_A", "decay_value_axis", "delta_before_decay", "delta_sign",
           "beta_on_v_only", "read_before_write", "no_scale"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_mutant_is_caught(kind):
    impl = _mutant(kind)
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                if not pin(impl):
                    failed.append(pin.__name__)
            except Exception:
                failed.append(pin.__name__ + " (raised)")
    assert failed, f"mutant {kind} passed every pin"


def test_unmutated_passes_all_pins():
    impl = _mutant("none")
    with np.errstate(over="ignore"):
        assert all(pin(impl) for pin in PINS)
