"""Pins of the CPU oracle against facts that do not come from the oracle:
hand-computed fixtures, closed forms, special cases that reduce to a
textbook identity or a library routine, invariants and exact brute force on
tiny inputs.  Each test names the mistake it is there to catch."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from audio_midi_transformer_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_int4_fixture():
    cases = []
    with open(os.path.join(GOLDEN, "int4_groups.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, k, w, scales, hexbytes = [x.strip() for x in line.split("|")]
            k = int(k)
            row = np.zeros((1, k), dtype=np.float32)
            vals = [float(x) for x in w.split()] if w else []
            row[0, :len(vals)] = vals
            cases.append((name, row, np.array([float(x) for x in scales.split()], np.float32),
                          bytes(int(x, 16) for x in hexbytes.split())))
    return cases


# ---------------------------------------------------------------- quantiser

@pytest.mark.parametrize("case", _read_int4_fixture(), ids=lambda c: c[0])
def test_quantize_hand_fixture(oracle_mod, case):
    """Hand-derived bytes and scales: catches nibble order, group axis,
    rounding mode (ties to even), /7 scale and zero point 8."""
    name, row, scales, expect = case
    q, s = oracle_mod.quantize_int4(row)
    assert s[0].tolist() == scales.tolist(), name
    assert bytes(q[0].tobytes()) == expect, name


def test_quantize_error_bound_and_range(oracle_mod):
    """|w - deq| <= s/2 (plus the few-ulp rounding of w/s and q*s); codes
    stay in [-7, 7]; the largest |w| of every group maps to +-7 exactly."""
    rng = np.random.default_rng(5)
    for scale in (0.02, 1.0, 3e-4):
        W = (rng.standard_normal((48, 256)) * scale).astype(np.float32)
        W[3, 32:64] = 0.0  # an all-zero group
        q, s = oracle_mod.quantize_int4(W)
        lo = (q & 0x0F).astype(np.int64)
        hi = (q >> 4).astype(np.int64)
        u = np.empty((48, 256), np.int64)
        u[:, 0::2], u[:, 1::2] = lo, hi
        code = u - 8
        assert code.min() >= -7 and code.max() <= 7
        wd = oracle_mod.dequantize_int4(q, s)
        sg = np.repeat(s.astype(np.float64), 32, axis=1)
        err = np.abs(W.astype(np.float64) - wd.astype(np.float64))
        assert np.all(err <= sg * (0.5 + 16 * 2.0 ** -24) + 1e-45)
        groups = np.abs(W).reshape(48, 8, 32)
        arg = groups.argmax(axis=2)
        cg = np.abs(code.reshape(48, 8, 32))
        picked = np.take_along_axis(cg, arg[..., None], axis=2)[..., 0]
        nonzero = groups.max(axis=2) > 0
        assert np.all(picked[nonzero] == 7)
        assert np.all(s[~nonzero] == 0) and np.all(code.reshape(48, 8, 32)[~nonzero] == 0)


def test_quantize_idempotent(oracle_mod):
    """Re-quantising the dequantised matrix returns the same codes and scales."""
    W = synth.random_matrix(7, 64, 512)
    q, s = oracle_mod.quantize_int4(W)
    q2, s2 = oracle_mod.quantize_int4(oracle_mod.dequantize_int4(q, s))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_dequantize_power_of_two_exact(oracle_mod):
    """With power-of-two scales every dequantised weight is exactly code * s;
    catches an off-by-one zero point or a swapped nibble in the reader."""
    rng = np.random.default_rng(3)
    u = rng.integers(0, 16, size=(8, 64))
    q = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    s = (2.0 ** rng.integers(-10, 4, size=(8, 2))).astype(np.float32)
    wd = oracle_mod.dequantize_int4(q, s)
    expect = (u - 8) * np.repeat(s.astype(np.float64), 32, axis=1)
    assert np.array_equal(wd.astype(np.float64), expect)


# ---------------------------------------------------------------- matmul

def test_matmul_exact_brute_force(oracle_mod):
    """Tiny non-square A . W^T against exact rational arithmetic; the result
    is the exact sum rounded once (catches a transposed operand or a dropped
    term)."""
    rng = np.random.default_rng(11)
    A = rng.standard_normal((3, 40)).astype(np.float32)
    W = rng.standard_normal((5, 40)).astype(np.float32)
    Y = oracle_mod.matmul(A, W)
    assert Y.shape == (3, 5)
    for m in range(3):
        for n in range(5):
            exact = sum(Fraction(float(A[m, k])) * Fraction(float(W[n, k])) for k in range(40))
            assert abs(Fraction(float(Y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 120)


def test_matmul_one_hot_column(oracle_mod):
    """e_k . W^T returns column k of W exactly."""
    W = synth.random_matrix(2, 24, 96)
    A = np.zeros((96, 96), np.float32)
    np.fill_diagonal(A, 1.0)
    Y = oracle_mod.matmul(A, W)
    assert np.array_equal(Y, W.T)


# ---------------------------------------------------------------- LayerNorm, GELU

def test_layernorm_closed_forms(oracle_mod):
    d = 64
    g = np.linspace(0.5, 1.5, d).astype(np.float32)
    b = np.linspace(-1, 1, d).astype(np.float32)
    # constant row -> x - mean == 0 -> output is the bias exactly
    y = oracle_mod.layernorm(np.full((1, d), 3.25, np.float32), g, b)
    assert np.array_equal(y[0], b)
    # unit gain, zero bias: mean 0, variance var/(var+eps)
    x = np.random.default_rng(1).standard_normal((4, d)).astype(np.float32) * 3
    y = oracle_mod.layernorm(x, np.ones(d, np.float32), np.zeros(d, np.float32)).astype(np.float64)
    var = x.astype(np.float64).var(axis=1)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-6)
    assert np.allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-6)
    # [1, 2, 3, 4] with gain 2 and bias 1: (x - 2.5) / sqrt(1.25 + 1e-5) * 2 + 1
    y = oracle_mod.layernorm(np.array([[1, 2, 3, 4]], np.float32), np.full(4, 2, np.float32),
                             np.ones(4, np.float32))
    want = [(v - 2.5) / math.sqrt(1.25 + 1e-5) * 2 + 1 for v in (1, 2, 3, 4)]
    assert np.allclose(y[0], want, rtol=0, atol=2e-7)


def test_gelu_closed_forms(oracle_mod):
    x = np.linspace(-6, 6, 241).astype(np.float32)
    y = oracle_mod.gelu(x).astype(np.float64)
    ym = oracle_mod.gelu(-x).astype(np.float64)
    assert oracle_mod.gelu(np.zeros(1, np.float32))[0] == 0.0
    assert np.allclose(y - ym, x, atol=4e-7)           # x*Phi(x) - (-x)*Phi(-x) = x
    # Phi(1) = 0.8413447460685429 (standard normal CDF); the tanh form is 1.5e-4 off
    assert abs(oracle_mod.gelu(np.ones(1, np.float32))[0] - 0.8413447460685429) < 1e-7
    # Phi(-2) = 0.022750131948179195
    assert abs(oracle_mod.gelu(np.full(1, -2, np.float32))[0] - (-2 * 0.022750131948179195)) < 1e-7


# ---------------------------------------------------------------- attention

def test_attention_single_key_returns_value(oracle_mod):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 64)).astype(np.float32)
    k = rng.standard_normal((1, 3, 64)).astype(np.float32)
    v = rng.standard_normal((1, 3, 64)).astype(np.float32)
    assert np.array_equal(oracle_mod.attention(q, k, v), v[0])


def test_attention_zero_query_is_mean(oracle_mod):
    rng = np.random.default_rng(6)
    k = rng.standard_normal((37, 2, 64)).astype(np.float32)
    v = rng.standard_normal((37, 2, 64)).astype(np.float32)
    out = oracle_mod.attention(np.zeros((2, 64), np.float32), k, v)
    assert np.allclose(out, v.astype(np.float64).mean(axis=0), rtol=0, atol=1e-7)


def test_attention_two_keys_logistic(oracle_mod):
    """q . K0 = 8 and q . K1 = 0: with the 1/8 scale the scores are 1 and 0,
    so the weights are e/(1+e) and 1/(1+e) (catches a missing scale or a sign);
    the second head is independent (catches a head-stride mistake)."""
    q = np.zeros((2, 64), np.float32)
    q[0, 5] = 8.0
    q[1, 9] = -16.0
    k = np.zeros((2, 2, 64), np.float32)
    k[0, 0, 5] = 1.0
    k[1, 1, 9] = 1.0
    v = np.zeros((2, 2, 64), np.float32)
    v[0, :, 0] = 1.0
    v[1, :, 1] = 1.0
    out = oracle_mod.attention(q, k, v)
    p0 = math.e / (1 + math.e)
    assert abs(out[0, 0] - p0) < 1e-7 and abs(out[0, 1] - (1 - p0)) < 1e-7
    # head 1: scores 0 and -2 -> weights 1/(1+e^-2), e^-2/(1+e^-2)
    p1 = 1 / (1 + math.exp(-2))
    assert abs(out[1, 0] - p1) < 1e-7 and abs(out[1, 1] - (1 - p1)) < 1e-7


def test_attention_softmax_sums_to_one(oracle_mod):
    """All values equal to 1 -> output 1 whatever the scores (weights sum to 1)."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 64)).astype(np.float32) * 3
    k = rng.standard_normal((300, 1, 64)).astype(np.float32)
    v = np.ones((300, 1, 64), np.float32)
    assert np.allclose(oracle_mod.attention(q, k, v), 1.0, atol=300 * 2.0 ** -24)


# ---------------------------------------------------------------- whole model

def _ln64(x, g, b, eps=1e-5):
    x = np.asarray(x, np.float64)
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def _tiny_weights(shape, seed=21):
    return synth.model_weights(shape, seed)


def test_model_zero_projections(oracle_mod):
    """All four projections zero: qkv = attn = o = 0 and f = GELU(0) W = 0, so
    the residual is the input row and logits = W_lm . LN_f(x_last)."""
    shape = synth.tiny_shape(n_layers=2, d_model=64, n_heads=1, d_ff=128, vocab=53)
    w = _tiny_weights(shape)
    for l in range(shape.n_layers):
        for lst in (w.w_qkv, w.w_o, w.w_up, w.w_down):
            lst[l] = np.zeros_like(lst[l])
    B, P, S = 2, 3, 2
    rng = np.random.default_rng(2)
    prefix = rng.standard_normal((B, P, 64)).astype(np.float32)
    tokens = rng.integers(0, 53, size=(B, S))
    m = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=16)
    logits, nxt = m.forward(tokens=tokens, prefix=prefix)
    for b in range(B):
        z = _ln64(w.tok_emb[tokens[b, -1]], w.lnf_g, w.lnf_b)
        want = w.lm_head.astype(np.float64) @ z
        assert np.allclose(logits[b], want, rtol=0, atol=2e-6)
        assert nxt[b] == int(np.argmax(logits[b]))
    # prefix only: last row is the last prefix row
    m.reset()
    logits, _ = m.forward(prefix=prefix)
    z = _ln64(prefix[1, -1], w.lnf_g, w.lnf_b)
    assert np.allclose(logits[1], w.lm_head.astype(np.float64) @ z, atol=2e-6)
    assert m.position == P


def test_model_argmax_tie_lowest_index(oracle_mod):
    """Greedy decoding takes the lowest index among bit-equal maxima.  LM-head
    rows 5 and 6 are identical and dominate (so their logits are exactly
    equal and largest): every call must pick 5, a tie rule that keeps the
    last maximum would pick 6.  A three-way tie (7, 20, 52) placed above
    them must pick 7; making row 6 alone the largest must pick 6."""
    shape = synth.tiny_shape(n_layers=2, d_model=64, n_heads=1, d_ff=128, vocab=53)
    B, P = 2, 5
    prefix = np.random.default_rng(3).standard_normal((B, P, 64)).astype(np.float32)
    cases = (({5, 6}, 4.0, 5), ({7, 20, 52}, 4.0, 7))
    for rows, gain, want in cases:
        w = synth.tie_head_rows(_tiny_weights(shape), sorted(rows), seed=1, gain=gain)
        if want == 7:  # rows 5 and 6 below the three-way tie
            w.lm_head[5] = w.lm_head[6] = np.float32(0.5) * w.lm_head[7]
        m = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=16)
        logits, nxt = m.forward(prefix=prefix)
        for step in range(4):
            r = sorted(rows)
            for b in range(B):
                assert all(logits[b, r[0]] == logits[b, j] for j in r[1:])
                assert logits[b, r[0]] > np.max(np.delete(logits[b], r))
            assert list(nxt) == [want] * B, (rows, step, nxt)
            logits, nxt = m.forward(tokens=nxt.reshape(B, 1))
        m.close()
    w = synth.tie_head_rows(_tiny_weights(shape), [5, 6], seed=1)
    w.lm_head[6] = w.lm_head[6] * np.float32(1.5)
    m = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=16)
    _, nxt = m.forward(prefix=prefix)
    assert list(nxt) == [6] * B
    m.close()


def _perm(n, seed):
    p = np.random.default_rng(seed).permutation(n)
    M = np.zeros((n, n), np.float32)
    M[np.arange(n), p] = 1.0
    return M


def _gelu64(x):
    from scipy.special import erf
    return 0.5 * x * (1 + erf(x / np.sqrt(2)))


def test_model_permutation_closed_form(oracle_mod):
    """Exactly representable 0/1 weights give a closed form the pages' steps
    reduce to: Q = 0 (uniform causal attention), K and V permutations (checks
    the Q|K|V split and the cache layout [L,B,T,H,64]), O, FFN-up and
    FFN-down permutations (checks operand orientation, GELU and both residual
    adds).  Two layers make layer 1's cache depend on layer 0's causal means."""
    d, F, V, L, H = 128, 256, 41, 2, 2
    shape = synth.tiny_shape(n_layers=L, d_model=d, n_heads=H, d_ff=F, vocab=V)
    w = _tiny_weights(shape, seed=5)
    Pk, Pv, Po, Pu, Pd = (_perm(d, s) for s in (1, 2, 3, 4, 5))
    for l in range(L):
        qkv = np.zeros((3 * d, d), np.float32)
        qkv[d:2 * d] = Pk
        qkv[2 * d:] = Pv
        up = np.zeros((F, d), np.float32)
        up[:d] = Pu
        down = np.zeros((d, F), np.float32)
        down[:, d:] = Pd          # reads the second half of the FFN width
        up[d:2 * d] = Pu.T        # ... which holds a different permutation
        w.w_qkv[l], w.w_o[l], w.w_up[l], w.w_down[l] = qkv, Po, up, down
    B, R = 1, 6
    x = np.random.default_rng(9).standard_normal((B, R, d)).astype(np.float32)
    m = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=8, quantize=False)
    logits, _ = m.forward(prefix=x)
    K, Vc = m.kv()
    r = x[0].astype(np.float64)
    for l in range(L):
        a = _ln64(r, w.ln1_g[l], w.ln1_b[l])
        k_rows, v_rows = a @ Pk.T, a @ Pv.T
        assert np.allclose(K[l, 0, :R].reshape(R, d), k_rows, atol=2e-6)
        assert np.allclose(Vc[l, 0, :R].reshape(R, d), v_rows, atol=2e-6)
        att = np.cumsum(v_rows, axis=0) / np.arange(1, R + 1)[:, None]   # causal mean
        r = r + att @ Po.T
        a2 = _ln64(r, w.ln2_g[l], w.ln2_b[l])
        h = np.zeros((R, F))
        h[:, :d] = a2 @ Pu.T
        h[:, d:2 * d] = a2 @ Pu
        r = r + _gelu64(h) @ down.astype(np.float64).T
    z = _ln64(r[-1], w.lnf_g, w.lnf_b)
    assert np.allclose(logits[0], w.lm_head.astype(np.float64) @ z, atol=1e-5)


def test_model_query_key_scores(oracle_mod):
    """One layer, Q and K permutations with V = O = identity and FFN zero:
    the output is x + softmax-weighted causal average of LN(x) rows with scores
    (P_q a_p) . (P_k a_t) / 8 per head."""
    d, F, V, H = 128, 128, 17, 2
    shape = synth.tiny_shape(n_layers=1, d_model=d, n_heads=H, d_ff=F, vocab=V)
    w = _tiny_weights(shape, seed=8)
    Pq, Pk = _perm(d, 11), _perm(d, 12)
    I = np.eye(d, dtype=np.float32)
    w.w_qkv[0] = np.concatenate([Pq, Pk, I]).astype(np.float32)
    w.w_o[0] = I
    w.w_up[0] = np.zeros((F, d), np.float32)
    w.w_down[0] = np.zeros((d, F), np.float32)
    R = 5
    x = np.random.default_rng(3).standard_normal((1, R, d)).astype(np.float32)
    m = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=R, quantize=False)
    logits, _ = m.forward(prefix=x)
    a = _ln64(x[0], w.ln1_g[0], w.ln1_b[0])
    q, k = a @ Pq.T, a @ Pk.T
    out = np.zeros(d)
    for h in range(H):
        sl = slice(64 * h, 64 * h + 64)
        s = k[:, sl] @ q[-1, sl] / 8.0
        p = np.exp(s - s.max())
        p /= p.sum()
        out[sl] = p @ a[:, sl]
    r = x[0, -1].astype(np.float64) + out
    z = _ln64(r, w.lnf_g, w.lnf_b)
    assert np.allclose(logits[0], w.lm_head.astype(np.float64) @ z, atol=1e-5)


def test_model_incremental_equals_one_shot(oracle_mod):
    """prefill(P + S) == prefill(P + S - 1) + decode(1), bit for bit, and the
    caches agree: causality and slot indexing (the rows are computed the same
    way whichever call appends them)."""
    shape = synth.tiny_shape()
    w = _tiny_weights(shape, seed=31)
    rng = np.random.default_rng(12)
    prefix = rng.standard_normal((2, 5, shape.d_model)).astype(np.float32)
    tokens = rng.integers(0, shape.vocab, size=(2, 4))
    a = oracle_mod.OracleModel.from_weights(w, batch=2, t_cap=12)
    la, na = a.forward(tokens=tokens, prefix=prefix)
    b = oracle_mod.OracleModel.from_weights(w, batch=2, t_cap=12)
    b.forward(prefix=prefix)
    b.forward(tokens=tokens[:, :2])
    b.forward(tokens=tokens[:, 2:3])
    lb, nb = b.forward(tokens=tokens[:, 3:])
    assert np.array_equal(la, lb) and np.array_equal(na, nb)
    Ka, Va = a.kv()
    Kb, Vb = b.kv()
    assert np.array_equal(Ka[:, :, :9], Kb[:, :, :9]) and np.array_equal(Va[:, :, :9], Vb[:, :, :9])
    assert a.position == b.position == 9


def test_model_batch_rows_independent(oracle_mod):
    """Sequence b's result does not depend on the other sequences."""
    shape = synth.tiny_shape()
    w = _tiny_weights(shape, seed=32)
    rng = np.random.default_rng(13)
    prefix = rng.standard_normal((3, 4, shape.d_model)).astype(np.float32)
    m3 = oracle_mod.OracleModel.from_weights(w, batch=3, t_cap=6)
    l3, _ = m3.forward(prefix=prefix)
    m1 = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=6)
    l1, _ = m1.forward(prefix=prefix[1:2])
    assert np.array_equal(l3[1], l1[0])


def test_model_cache_full_and_bad_token(oracle_mod):
    shape = synth.tiny_shape()
    w = _tiny_weights(shape, seed=33)
    m = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3)
    m.forward(tokens=np.array([[1, 2]]))
    with pytest.raises(OverflowError):
        m.forward(tokens=np.array([[1, 2]]))
    assert m.position == 2
    with pytest.raises(RuntimeError):
        m.forward(tokens=np.array([[shape.vocab]]))
    m.forward(tokens=np.array([[0]]))
    assert m.position == 3


def test_model_quantized_equals_dequantized_input(oracle_mod):
    """Quantising inside the model is the same as handing it the dequantised
    weights (ties the model's weight path to the pinned quantiser)."""
    shape = synth.tiny_shape(n_layers=1)
    w = _tiny_weights(shape, seed=34)
    x = np.random.default_rng(1).standard_normal((1, 3, shape.d_model)).astype(np.float32)
    mq = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3)
    lq, _ = mq.forward(prefix=x)
    for lst in (w.w_qkv, w.w_o, w.w_up, w.w_down):
        lst[0] = oracle_mod.dequantize_int4(*oracle_mod.quantize_int4(lst[0]))
    md = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3, quantize=False)
    ld, _ = md.forward(prefix=x)
    assert np.array_equal(lq, ld)


# ---------------------------------------------------------------- W4A8 variant

def _act_ref(x):
    """The activation-code definition in numpy binary32, element by element."""
    x = np.asarray(x, np.float32)
    m = np.float32(np.max(np.abs(x)))
    s = np.float32(m / np.float32(127.0))
    if s == 0:
        return np.zeros(x.shape, np.int8), s
    r = np.float32(np.float32(1.0) / s)
    q = np.clip(np.rint((x * r).astype(np.float32)), -127, 127).astype(np.int8)
    return q, s


def test_act_int8_hand_cases(oracle_mod):
    """Hand-computed groups: scale exactly 1, 0.5 and 2, ties to even, an
    all-zero group (catches a round-away-from-zero, a 128 divisor or a
    missing zero guard)."""
    g = np.zeros((4, 32), np.float32)
    g[0, :5] = [127.0, 2.5, 3.5, -2.5, 0.5]          # s = 1
    g[1, :5] = [63.5, 1.25, 0.75, -0.25, -63.5]       # s = 0.5
    g[2, :4] = [-254.0, 3.0, 1.0, -5.0]               # s = 2
    q, s = oracle_mod.quantize_act_int8(g.reshape(1, 128))
    assert np.array_equal(s[0], np.array([1.0, 0.5, 2.0, 0.0], np.float32))
    q = q.reshape(4, 32)
    assert list(q[0, :5]) == [127, 2, 4, -2, 0]
    assert list(q[1, :5]) == [127, 2, 2, 0, -127]
    assert list(q[2, :4]) == [-127, 2, 0, -2]
    assert not q[0, 5:].any() and not q[3].any()


def test_act_int8_matches_definition_and_bound(oracle_mod):
    """Random rows over a wide range: codes equal the binary32 definition,
    |x - s q| <= s / 2, the largest element maps to +-127, codes are odd in x."""
    rng = np.random.default_rng(40)
    X = (rng.standard_normal((6, 256)) * np.exp(rng.uniform(-8, 8, (6, 256)))).astype(np.float32)
    q, s = oracle_mod.quantize_act_int8(X)
    qn, sn = oracle_mod.quantize_act_int8(-X)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for m in range(6):
        for g in range(8):
            x = X[m, 32 * g:32 * g + 32]
            qr, sr = _act_ref(x)
            assert s[m, g] == sr
            assert np.array_equal(q[m, 32 * g:32 * g + 32], qr)
            err = np.abs(x.astype(np.float64) - np.float64(sr) * q[m, 32 * g:32 * g + 32])
            assert np.all(err <= 0.5 * np.float64(sr) * (1 + 2.0 ** -20))
            assert np.max(np.abs(q[m, 32 * g:32 * g + 32])) == 127


def test_matmul_w4a8_exact_brute_force(oracle_mod):
    """The W4A8 product against exact rational arithmetic from the codes
    (catches a dropped scale, a wrong nibble order or a group index slip)."""
    rng = np.random.default_rng(41)
    A = rng.standard_normal((3, 96)).astype(np.float32)
    W = (0.05 * rng.standard_normal((4, 96))).astype(np.float32)
    wq, ws = oracle_mod.quantize_int4(W)
    Y = oracle_mod.matmul_w4a8(A, wq, ws)
    assert Y.shape == (3, 4)
    u = np.zeros((4, 96), np.int64)
    u[:, 0::2] = wq & 15
    u[:, 1::2] = wq >> 4
    for m in range(3):
        qa, sa = zip(*[_act_ref(A[m, 32 * g:32 * g + 32]) for g in range(3)])
        for n in range(4):
            exact = Fraction(0)
            for g in range(3):
                I = int(np.sum((u[n, 32 * g:32 * g + 32] - 8) * qa[g].astype(np.int64)))
                exact += Fraction(float(ws[n, g])) * Fraction(float(sa[g])) * I
            assert abs(Fraction(float(Y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 120)


def test_matmul_w4a8_integer_activations_equal_w4a32(oracle_mod):
    """Activations that are integers with a group maximum of 127 have scale 1
    and codes equal to themselves; with power-of-two weight scales both
    products are the same exact sum, so the results are bit-equal."""
    rng = np.random.default_rng(42)
    A = rng.integers(-127, 128, (2, 64)).astype(np.float32)
    A[:, 0] = 127.0
    A[:, 32] = -127.0
    W = rng.integers(-7, 8, (5, 64)).astype(np.float32) * np.float32(0.25)
    W[:, 0] = 7 * 0.25
    W[:, 32] = -7 * 0.25
    wq, ws = oracle_mod.quantize_int4(W)
    assert np.all(ws == 0.25)
    y8 = oracle_mod.matmul_w4a8(A, wq, ws)
    y32 = oracle_mod.matmul(A, oracle_mod.dequantize_int4(wq, ws))
    assert np.array_equal(y8, y32)


def test_model_w4a8_projections_use_w4a8_product(oracle_mod):
    """In W4A8 mode the layer-0 K and V cache rows are the W4A8 product of
    LayerNorm(prefix) with the layer's QKV codes (ties the model to the pinned
    product), and they differ from the W4A32 rows."""
    shape = synth.tiny_shape(n_layers=1)
    w = _tiny_weights(shape, seed=43)
    d = shape.d_model
    x = np.random.default_rng(2).standard_normal((1, 3, d)).astype(np.float32)
    m8 = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3, w4a8=True)
    m8.forward(prefix=x)
    k8, v8 = m8.kv()
    a = oracle_mod.layernorm(x[0], w.ln1_g[0], w.ln1_b[0])
    qkv = oracle_mod.matmul_w4a8(a, *oracle_mod.quantize_int4(w.w_qkv[0]))
    assert np.array_equal(k8[0, 0].reshape(3, d), qkv[:, d:2 * d])
    assert np.array_equal(v8[0, 0].reshape(3, d), qkv[:, 2 * d:])
    m32 = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3)
    m32.forward(prefix=x)
    k32, _ = m32.kv()
    assert not np.array_equal(k8, k32)


# ---------------------------------------------------------------- ragged batch

def test_model_ragged_batch_equals_independent_sequences(oracle_mod):
    """Sequences of one batch with their own positions (single-sequence
    appends, a restart, lockstep decode at different positions) give
    bit-identical logits to independent one-sequence models fed the same
    rows (catches a shared position, a wrong cache slot or cross-sequence
    attention)."""
    shape = synth.tiny_shape(n_layers=2)
    w = _tiny_weights(shape, seed=50)
    d, V = shape.d_model, shape.vocab
    rng = np.random.default_rng(7)
    B = 3
    mb = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=40)
    ms = [oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=40) for _ in range(B)]
    # staggered single-sequence prefills
    for b, P in ((0, 5), (1, 9), (2, 2)):
        x = rng.standard_normal((P, d)).astype(np.float32)
        lb, nb = mb.forward_seq(b, prefix=x)
        ls, ns = ms[b].forward(prefix=x[None])
        assert np.array_equal(lb, ls[0]) and nb == int(ns[0])
    # sequence 1 appends two prompt tokens on its own
    t = rng.integers(0, V, 2)
    lb, _ = mb.forward_seq(1, tokens=t)
    ls, _ = ms[1].forward(tokens=t[None])
    assert np.array_equal(lb, ls[0])
    assert [mb.position_seq(b) for b in range(B)] == [5, 11, 2]
    for step in range(4):
        tok = rng.integers(0, V, B)
        lb, _ = mb.forward(tokens=tok[:, None])
        for b in range(B):
            ls, _ = ms[b].forward(tokens=tok[b:b + 1, None])
            assert np.array_equal(lb[b], ls[0]), f"step {step} sequence {b}"
        if step == 1:
            # sequence 2 restarts with a new chunk while the others continue
            mb.reset_seq(2)
            ms[2].reset()
            x = rng.standard_normal((3, d)).astype(np.float32)
            lb2, _ = mb.forward_seq(2, prefix=x)
            ls2, _ = ms[2].forward(prefix=x[None])
            assert np.array_equal(lb2, ls2[0])
    assert [mb.position_seq(b) for b in range(B)] == [9, 15, 5]
    for b in range(B):
        kb, vb = mb.kv()
        ks, vs = ms[b].kv()
        T = ms[b].position
        assert np.array_equal(kb[:, b, :T], ks[:, 0, :T]) and np.array_equal(vb[:, b, :T], vs[:, 0, :T])


# ---------------------------------------------------------------- dense FP16 / FP32 variants

@pytest.mark.parametrize("x,want", [
    (1.0, 1.0),
    (1.0 + 2.0 ** -11, 1.0),                    # tie between 1 and 1 + 2^-10: even mantissa
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),    # tie between odd and even: even wins, upward
    (1.0 + 2.0 ** -11 + 2.0 ** -20, 1.0 + 2.0 ** -10),  # just above the tie
    (-(2.0 - 2.0 ** -12), -2.0),                # rounds up into the next binade
    (65504.0, 65504.0),                         # largest finite half
    (65519.0, 65504.0),
    (65520.0, math.inf),                        # halfway to 2^16: overflow
    (-1e6, -math.inf),
    (2.0 ** -14, 2.0 ** -14),                   # smallest normal
    (2.0 ** -24, 2.0 ** -24),                   # smallest subnormal
    (2.0 ** -25, 0.0),                          # tie between 0 and 2^-24: even (0)
    (3 * 2.0 ** -26, 2.0 ** -24),
    (3 * 2.0 ** -25, 2 * 2.0 ** -24),           # tie between 1 and 2 quanta: 2
    (0.1, 1638.0 / 16384.0),                    # 0.1 = 1.6 * 2^-4: 1638.4 quanta of 2^-14
    (-0.0, -0.0),
])
def test_round_half_hand_cases(oracle_mod, x, want):
    """binary16 rounding from its definition: a wrong quantum (10 vs 11
    bits), truncation instead of ties-to-even, a wrong subnormal threshold or
    a wrong overflow threshold each fail one of these."""
    got = oracle_mod.round_half(np.array([x], np.float32))[0]
    assert got == np.float32(want) and math.copysign(1, got) == math.copysign(1, want), (x, got, want)


def test_round_half_matches_numpy_binary16(oracle_mod):
    """numpy's float16 conversion is an independent IEEE implementation."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-30, 18, 200000))).astype(np.float32)
    got = oracle_mod.round_half(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_model_dense_modes_are_unquantised_models(oracle_mod):
    """dense='f32' is the unquantised model and dense='f16' the unquantised
    model of binary16-rounded projections (rounded here with numpy)."""
    shape = synth.tiny_shape(n_layers=2)
    w = _tiny_weights(shape, seed=35)
    x = np.random.default_rng(2).standard_normal((1, 3, shape.d_model)).astype(np.float32)
    m32 = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3, dense="f32")
    mu = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3, quantize=False)
    m16 = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3, dense="f16")
    l32, _ = m32.forward(prefix=x)
    lu, _ = mu.forward(prefix=x)
    l16, _ = m16.forward(prefix=x)
    assert np.array_equal(l32, lu)
    for lst in (w.w_qkv, w.w_o, w.w_up, w.w_down):
        for l in range(shape.n_layers):
            lst[l] = lst[l].astype(np.float16).astype(np.float32)
    mr = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3, quantize=False)
    lr, _ = mr.forward(prefix=x)
    assert np.array_equal(l16, lr)
    assert not np.array_equal(l16, l32)
    with pytest.raises(ValueError):
        oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=3, dense="bf16")


# ---------------------------------------------------------------- classifier-free guidance

def _pairs(rows_c, rows_u):
    return np.asarray(list(rows_c) + list(rows_u), dtype=np.float32)


def test_cfg_hand_cases(oracle_mod):
    """Hand-computed guided rows of two pairs (rows 0, 1 conditional, rows
    2, 3 their partners): catches a sign error, conditional and
    unconditional swapped, row i paired with i + 1 instead of Np + i, and a
    tie not resolved to the lowest index."""
    lg = _pairs([[1, 3, 2], [1, 1, 0]], [[0, 4, 1], [0, 0, 5]])
    g, nx = oracle_mod.cfg_combine(lg, 2.0)
    # 2c - u
    assert np.array_equal(g, np.array([[2, 2, 3], [2, 2, -5]], np.float32))
    assert list(nx) == [2, 0]
    g, nx = oracle_mod.cfg_combine(lg, 3.0)
    # 3c - 2u
    assert np.array_equal(g, np.array([[3, 1, 4], [3, 3, -10]], np.float32))
    assert list(nx) == [2, 0]
    g, nx = oracle_mod.cfg_combine(lg, 0.5)
    # (c + u) / 2
    assert np.array_equal(g, np.array([[0.5, 3.5, 1.5], [0.5, 0.5, 2.5]], np.float32))
    assert list(nx) == [1, 2]


def test_cfg_coefficient_one_is_the_conditional_model(oracle_mod):
    """cfg = 1 returns the conditional logits bit for bit and numpy's first
    argmax: the released models' setting is the plain path."""
    rng = np.random.default_rng(90)
    lg = (rng.standard_normal((6, 1393)) * 3).astype(np.float32)
    g, nx = oracle_mod.cfg_combine(lg, 1.0)
    assert np.array_equal(g.view(np.uint32), lg[:3].view(np.uint32))
    assert list(nx) == [int(np.argmax(r)) for r in lg[:3]]


def test_cfg_coefficient_zero_is_the_unconditional_model(oracle_mod):
    """cfg = 0 returns the unconditional rows exactly (the differences of
    these binary32 values are exact in binary64)."""
    rng = np.random.default_rng(91)
    lg = (rng.standard_normal((8, 257)) * 5).astype(np.float32)
    g, nx = oracle_mod.cfg_combine(lg, 0.0)
    assert np.array_equal(g, lg[4:])
    assert list(nx) == [int(np.argmax(r)) for r in lg[4:]]


def test_cfg_equal_rows_are_fixed_points(oracle_mod):
    """Where both rows agree the coefficient does not matter."""
    rng = np.random.default_rng(92)
    c = rng.standard_normal((2, 100)).astype(np.float32)
    for cfg in (-3.0, 0.0, 2.0, 7.5, 1e6):
        g, nx = oracle_mod.cfg_combine(np.concatenate([c, c]), cfg)
        assert np.array_equal(g, c), cfg
        assert list(nx) == [int(np.argmax(r)) for r in c]


def _f32_ulp(x):
    x = np.float32(abs(x))
    return Fraction(float(np.nextafter(x, np.float32(np.inf)) - x))


@pytest.mark.parametrize("cfg", [2.0, 3.0, -0.75, 1.5, 10.0])
def test_cfg_exact_within_half_ulp(oracle_mod, cfg):
    """Each guided value is the exact rational u + cfg (c - u), computed
    with fractions, rounded to binary32: within half an ulp (catches a
    dropped term or a coefficient applied to the wrong operand for any
    coefficient, not only the special cases)."""
    rng = np.random.default_rng(93)
    lg = (rng.standard_normal((4, 64)) * 4).astype(np.float32)
    g, nx = oracle_mod.cfg_combine(lg, cfg)
    k = Fraction(cfg)
    for i in range(2):
        for v in range(64):
            c, u = Fraction(float(lg[i, v])), Fraction(float(lg[2 + i, v]))
            exact = u + k * (c - u)
            assert abs(Fraction(float(g[i, v])) - exact) <= _f32_ulp(g[i, v]) / 2, (i, v)
        assert nx[i] == int(np.argmax(g[i]))


def test_model_cfg_pairs_coefficient_one_equals_conditional_model(oracle_mod):
    """A batch of two conditional rows and their unconditional partners
    (different prefixes), decoded with the guided token fed to both rows of
    each pair, gives at cfg = 1 the logits and tokens of a model that holds
    the conditional rows alone; at cfg = 2 the unconditional rows change the
    result (catches guidance that ignores the partner, or partners fed their
    own tokens)."""
    shape = synth.tiny_shape(n_layers=2)
    w = _tiny_weights(shape, seed=51)
    d = shape.d_model
    rng = np.random.default_rng(8)
    Np, P = 2, 7
    cond = rng.standard_normal((Np, P, d)).astype(np.float32)
    uncond = cond.copy()
    uncond[:, -2:] = rng.standard_normal((Np, 2, d)).astype(np.float32)
    runs = {}
    for cfg in (1.0, 2.0):
        mp = oracle_mod.OracleModel.from_weights(w, batch=2 * Np, t_cap=24)
        lg, _ = mp.forward(prefix=np.concatenate([cond, uncond]))
        g, nx = oracle_mod.cfg_combine(lg, cfg)
        hist = [(g, nx)]
        for _ in range(5):
            lg, _ = mp.forward(tokens=np.concatenate([nx, nx])[:, None])
            g, nx = oracle_mod.cfg_combine(lg, cfg)
            hist.append((g, nx))
        runs[cfg] = hist
        mp.close()
    mc = oracle_mod.OracleModel.from_weights(w, batch=Np, t_cap=24)
    lc, nc = mc.forward(prefix=cond)
    for step, (g, nx) in enumerate(runs[1.0]):
        assert np.array_equal(g, lc) and np.array_equal(nx, nc), step
        lc, nc = mc.forward(tokens=nc[:, None])
    mc.close()
    assert not np.array_equal(runs[2.0][0][0], runs[1.0][0][0])
