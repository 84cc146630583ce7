"""GPU parity of the HIP path against the CPU oracle, through the C ABI:
dequantisation (bit-exact), the INT4 GEMV and GEMM kernels at every
projection shape, whole-model prefill + teacher-forced decode at small shapes
spanning several tiles with ragged tails, KV-slot indexing with a sentinel
cache, incremental-vs-one-shot and batch invariants, error paths."""
import numpy as np
import pytest

from audio_midi_transformer_amd import binding, synth
from parity import TOL, check_greedy, compare_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _t(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


# ------------------------------------------------------------------ one-layer models at real widths

@pytest.fixture(scope="module", params=["small", "medium", "large"])
def one_layer(request, oracle_mod):
    _dev()
    base = {"small": synth.SMALL, "medium": synth.MEDIUM, "large": synth.LARGE}[request.param]
    shape = synth.ModelShape(base.name, 1, base.d_model, base.n_heads, base.d_ff)
    w = synth.model_weights(shape, 77)
    dec = binding.Decoder(w, batch=1, t_cap=8)
    yield shape, w, dec
    dec.close()


def test_dequant_bit_exact(one_layer, oracle_mod):
    shape, w, dec = one_layer
    for p, W in enumerate((w.w_qkv[0], w.w_o[0], w.w_up[0], w.w_down[0])):
        want = oracle_mod.dequantize_int4(*oracle_mod.quantize_int4(W))
        got = dec.debug_dequant(0, p).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"projection {p}"


def _matmul_bound(x, q, s):
    """Rigorous FP32 bound for the kernels' evaluation: K * 2^-24 * sum |x| (|u| + 8) s."""
    u_lo = (q & 0x0F).astype(np.float64)
    u_hi = (q >> 4).astype(np.float64)
    u = np.empty((q.shape[0], q.shape[1] * 2))
    u[:, 0::2], u[:, 1::2] = u_lo, u_hi
    mag = (u + 8.0) * np.repeat(s.astype(np.float64), 32, axis=1)
    K = mag.shape[1]
    return K * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ mag.T) + 1e-30


@pytest.mark.parametrize("M,force_gemm", [(1, False), (3, False), (8, False), (13, False), (16, False),
                                          (32, False), (1, True), (13, True), (64, True), (130, True)])
def test_matmul_vs_oracle(one_layer, oracle_mod, M, force_gemm):
    shape, w, dec = one_layer
    rng = np.random.default_rng(M)
    for p, W in enumerate((w.w_qkv[0], w.w_o[0], w.w_up[0], w.w_down[0])):
        q, s = oracle_mod.quantize_int4(W)
        Wd = oracle_mod.dequantize_int4(q, s)
        x = rng.standard_normal((M, W.shape[1])).astype(np.float32)
        want = oracle_mod.matmul(x, Wd)
        got = dec.debug_matmul(0, p, _t(x), force_gemm=force_gemm).cpu().numpy()
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        assert np.all(err <= _matmul_bound(x, q, s) + 2.0 ** -24 * np.abs(want)), (
            f"projection {p}: max err {err.max():.3g}")


def test_matmul_one_hot_column_exact(one_layer, oracle_mod):
    """e_k through the GEMV returns column k of the dequantised matrix exactly."""
    shape, w, dec = one_layer
    W = w.w_o[0]
    Wd = oracle_mod.dequantize_int4(*oracle_mod.quantize_int4(W))
    for k in (0, 1, 31, 32, W.shape[1] - 1):
        x = np.zeros((1, W.shape[1]), np.float32)
        x[0, k] = 1.0
        got = dec.debug_matmul(0, 1, _t(x)).cpu().numpy()[0]
        assert np.array_equal(got, Wd[:, k])


# ------------------------------------------------------------------ whole model, tiny shapes

def _tiny(oracle_mod, B=2, t_cap=100, seed=3, n_layers=2, d=128, heads=2, ff=512, vocab=97):
    shape = synth.tiny_shape(n_layers=n_layers, d_model=d, n_heads=heads, d_ff=ff, vocab=vocab)
    w = synth.model_weights(shape, seed)
    return shape, w


def _run_pair(oracle_mod, shape, w, B, t_cap, prefix, tokens, steps, path=None):
    """Prefill + teacher-forced decode on both sides; returns max |delta| and ties."""
    om = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=t_cap)
    dec = binding.Decoder(w, batch=B, t_cap=t_cap)
    if path is not None:
        dec.set_decode_path(path)
    lo, no = om.forward(tokens=tokens, prefix=prefix)
    lg, ng = dec.prefill(_t(tokens) if tokens is not None else None,
                         _t(prefix) if prefix is not None else None)
    worst = compare_logits(lg.cpu().numpy(), lo, TOL["tiny"], "prefill")
    ties = check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, TOL["tiny"])
    for k in range(steps):
        tok = no.reshape(B, 1)
        lo, no = om.forward(tokens=tok)
        lg, ng = dec.decode_step(_t(tok.reshape(B)))
        worst = max(worst, compare_logits(lg.cpu().numpy(), lo, TOL["tiny"], f"step {k}"))
        ties += check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, TOL["tiny"])
    dec.check()
    K, V = dec.kv_cache()
    Ko, Vo = om.kv()
    T = om.position
    assert dec.position == T
    np.testing.assert_allclose(K[:, :, :T].cpu().numpy(), Ko[:, :, :T], rtol=0, atol=2e-5)
    np.testing.assert_allclose(V[:, :, :T].cpu().numpy(), Vo[:, :, :T], rtol=0, atol=2e-5)
    om.close()
    dec.close()
    return worst, ties


@pytest.mark.parametrize("path", [binding.MT_DECODE_KERNELS, binding.MT_DECODE_AUTO])
def test_model_prefix_and_tokens_then_decode(oracle_mod, path):
    _dev()
    shape, w = _tiny(oracle_mod)
    B, P, S = 2, 70, 5
    rng = np.random.default_rng(1)
    prefix = rng.standard_normal((B, P, shape.d_model)).astype(np.float32)
    tokens = rng.integers(0, shape.vocab, size=(B, S))
    _run_pair(oracle_mod, shape, w, B, 100, prefix, tokens, steps=20, path=path)


@pytest.mark.parametrize("B,P,S", [(16, 6, 3), (5, 0, 3), (13, 2, 0)])
def test_model_gemv_slices(oracle_mod, B, P, S):
    """Batches of 9 to 16 rows run the GEMV in launches of 8 whole
    sequences: B = 16 decodes in slices 8 + 8 (and prefills 9 rows per
    sequence on the GEMM); B = 5 with 3 prompt tokens prefills 15 rows in
    slices of two sequences (6 + 6 + 3 rows, so the K/V scatter starts
    mid-batch); B = 13 decodes with a 5-row tail slice."""
    _dev()
    shape, w = _tiny(oracle_mod)
    rng = np.random.default_rng(B)
    prefix = rng.standard_normal((B, P, shape.d_model)).astype(np.float32) if P else None
    tokens = rng.integers(0, shape.vocab, size=(B, S)) if S else None
    _run_pair(oracle_mod, shape, w, B, P + S + 12, prefix, tokens, steps=10)


@pytest.mark.parametrize("B,P,S", [(20, 6, 3), (33, 2, 0)])
def test_model_gemm_decode(oracle_mod, B, P, S):
    """Past 16 rows a decode step runs its projections on the GEMM (O and
    FFN-down with K split over several workgroups) and merges the split-K
    attention partials into rows with their own kernel."""
    _dev()
    shape, w = _tiny(oracle_mod)
    rng = np.random.default_rng(B + 100)
    prefix = rng.standard_normal((B, P, shape.d_model)).astype(np.float32) if P else None
    tokens = rng.integers(0, shape.vocab, size=(B, S)) if S else None
    _run_pair(oracle_mod, shape, w, B, P + S + 12, prefix, tokens, steps=10)


def test_model_tokens_only_small_width(oracle_mod):
    """Config-0 style: prompt tokens only, no prefix; the small model's width
    (768, 12 heads) with two layers."""
    _dev()
    shape, w = _tiny(oracle_mod, n_layers=2, d=768, heads=12, ff=3072, vocab=1393)
    tokens = np.random.default_rng(2).integers(0, 1393, size=(1, 8))
    _run_pair(oracle_mod, shape, w, 1, 40, None, tokens, steps=12)


@pytest.mark.parametrize("ff", [544, 96])
def test_ragged_group_counts(oracle_mod, ff):
    """FFN widths whose group count is not a multiple of 4 (17 and 3 groups):
    the GEMV waves take different numbers of groups (one takes none at 96)
    and load clamped dummy groups; every projection and the whole model
    still match the oracle."""
    _dev()
    shape, w = _tiny(oracle_mod, n_layers=2, d=128, heads=2, ff=ff, vocab=97, seed=21)
    dec = binding.Decoder(w, batch=1, t_cap=8)
    rng = np.random.default_rng(ff)
    for M, force in ((1, False), (5, False), (8, False), (11, True)):
        for p, W in enumerate((w.w_qkv[1], w.w_o[1], w.w_up[1], w.w_down[1])):
            q, s = oracle_mod.quantize_int4(W)
            x = rng.standard_normal((M, W.shape[1])).astype(np.float32)
            want = oracle_mod.matmul(x, oracle_mod.dequantize_int4(q, s))
            got = dec.debug_matmul(1, p, _t(x), force_gemm=force).cpu().numpy()
            err = np.abs(got.astype(np.float64) - want.astype(np.float64))
            assert np.all(err <= _matmul_bound(x, q, s) + 2.0 ** -24 * np.abs(want)), (M, p, float(err.max()))
    dec.close()
    prefix = rng.standard_normal((2, 9, shape.d_model)).astype(np.float32)
    _run_pair(oracle_mod, shape, w, 2, 30, prefix, None, steps=6)


def test_model_batch8_medium_width(oracle_mod):
    _dev()
    shape, w = _tiny(oracle_mod, n_layers=1, d=1024, heads=16, ff=4096, vocab=1393, seed=5)
    rng = np.random.default_rng(3)
    prefix = rng.standard_normal((8, 33, 1024)).astype(np.float32)
    _run_pair(oracle_mod, shape, w, 8, 48, prefix, None, steps=6)


def test_kv_sentinel_only_live_slots_written(oracle_mod):
    """Fill the cache with a NaN-payload sentinel; after prefill and decode
    steps exactly slots [0, T_past) differ from it, the rest are untouched."""
    _dev()
    shape, w = _tiny(oracle_mod)
    B, t_cap = 2, 50
    dec = binding.Decoder(w, batch=B, t_cap=t_cap)
    kp, vp = dec.kv_pointers()
    n = shape.n_layers * B * t_cap * shape.d_model
    sentinel = torch.full((n,), 0x7FC0DEAD, dtype=torch.int32, device=_dev())
    for p in (kp, vp):
        binding.hip_copy(p, sentinel.data_ptr(), n * 4)
    torch.cuda.synchronize()
    prefix = _t(np.random.default_rng(4).standard_normal((B, 11, shape.d_model)).astype(np.float32))
    _, nxt = dec.prefill(None, prefix)
    for _ in range(6):
        _, nxt = dec.decode_step(nxt)
    torch.cuda.synchronize()
    T = dec.position
    assert T == 17
    for cache in dec.kv_cache():
        bits = cache.view(torch.int32).cpu().numpy()
        live = bits[:, :, :T]
        dead = bits[:, :, T:]
        assert np.all(dead == 0x7FC0DEAD)
        assert not np.any(live == 0x7FC0DEAD)
    dec.close()


def test_incremental_equals_one_shot(oracle_mod):
    _dev()
    shape, w = _tiny(oracle_mod, seed=9)
    B = 2
    rng = np.random.default_rng(5)
    prefix = rng.standard_normal((B, 9, shape.d_model)).astype(np.float32)
    tokens = rng.integers(0, shape.vocab, size=(B, 4))
    a = binding.Decoder(w, batch=B, t_cap=20)
    la, _ = a.prefill(_t(tokens), _t(prefix))
    b = binding.Decoder(w, batch=B, t_cap=20)
    b.prefill(_t(tokens[:, :2]), _t(prefix))
    b.prefill(_t(tokens[:, 2:3]), None)
    lb, _ = b.decode_step(_t(tokens[:, 3].copy()))
    np.testing.assert_allclose(la.cpu().numpy(), lb.cpu().numpy(), rtol=0, atol=2e-5)
    a.close()
    b.close()


def test_identical_sequences_give_identical_rows(oracle_mod):
    _dev()
    shape, w = _tiny(oracle_mod, seed=10)
    B = 4
    one = np.random.default_rng(6).standard_normal((1, 13, shape.d_model)).astype(np.float32)
    dec = binding.Decoder(w, batch=B, t_cap=20)
    lg, nxt = dec.prefill(None, _t(np.repeat(one, B, axis=0)))
    for _ in range(3):
        lg, nxt = dec.decode_step(nxt)
    lg = lg.cpu().numpy()
    for b in range(1, B):
        np.testing.assert_allclose(lg[b], lg[0], rtol=0, atol=1e-6)
    dec.close()


def test_cache_full_leaves_state_untouched(oracle_mod):
    _dev()
    shape, w = _tiny(oracle_mod, seed=11)
    dec = binding.Decoder(w, batch=1, t_cap=6)
    _, nxt = dec.prefill(_t(np.array([[1, 2, 3, 4, 5]])), None)
    k0, v0 = dec.kv_cache()
    with pytest.raises(binding.MTError) as e:
        dec.prefill(_t(np.array([[1, 2]])), None)
    assert e.value.code == binding.MT_ERR_CACHE_FULL
    assert dec.position == 5
    _, nxt = dec.decode_step(nxt)
    assert dec.position == 6
    with pytest.raises(binding.MTError) as e:
        dec.decode_step(nxt)
    assert e.value.code == binding.MT_ERR_CACHE_FULL
    k1, _ = dec.kv_cache()
    assert torch.equal(k1[:, :, :5], k0[:, :, :5])
    dec.close()


def test_bad_token_reported_by_check(oracle_mod):
    _dev()
    shape, w = _tiny(oracle_mod, seed=12)
    dec = binding.Decoder(w, batch=1, t_cap=8)
    lg, _ = dec.prefill(_t(np.array([[shape.vocab + 5]])), None)
    with pytest.raises(binding.MTError) as e:
        dec.check()
    assert e.value.code == binding.MT_ERR_INVALID_ARG
    assert np.all(np.isnan(lg.cpu().numpy()))
    dec.check()  # flag was cleared
    dec.close()


def test_invalid_arguments_rejected(oracle_mod):
    _dev()
    shape, w = _tiny(oracle_mod, seed=13)
    dec = binding.Decoder(w, batch=1, t_cap=8)
    lib = binding.lib()
    out = torch.empty((1, shape.vocab), device=_dev())
    nxt = torch.empty((1,), dtype=torch.int64, device=_dev())
    assert lib.mt_prefill(dec.handle, None, 0, None, 0, out.data_ptr(), nxt.data_ptr(), None) == binding.MT_ERR_INVALID_ARG
    assert lib.mt_prefill(dec.handle, None, 2, None, 0, out.data_ptr(), nxt.data_ptr(), None) == binding.MT_ERR_INVALID_ARG
    assert lib.mt_decode_step(dec.handle, None, out.data_ptr(), nxt.data_ptr(), None) == binding.MT_ERR_INVALID_ARG
    assert lib.mt_set_decode_path(dec.handle, 7) == binding.MT_ERR_INVALID_ARG
    assert dec.position == 0
    dec.close()
