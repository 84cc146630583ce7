"""GPU parity at the configuration limits, against the CPU oracle through the
C ABI: the largest batch (64 sequences: projections on the GEMM, the decode
attention's partials merged into rows by their own kernel), the largest width (d_model 2048,
32 heads, FFN 8192: the LayerNorm GEMV with 16 groups per wave and a
multi-chunk FFN-down), and the largest cache (16384 positions: the decode
attention at its 64-split limit), filled to the last slot and then refused."""
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


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


def _run(oracle_mod, w, B, t_cap, prefix, tokens, steps, tol):
    om = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=t_cap)
    dec = binding.Decoder(w, batch=B, t_cap=t_cap)
    lo, no = om.forward(tokens=tokens, prefix=prefix)
    lg, ng = dec.prefill(_t(tokens) if tokens is not None else None, _t(prefix) if prefix is not None else None)
    worst = compare_logits(lg.cpu().numpy(), lo, tol, "prefill")
    check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, tol)
    for k in range(steps):
        tok = no.reshape(B, 1)
        lo, no = om.forward(tokens=tok)
        lg, ng = dec.decode_step(_t(tok.reshape(B)))
        worst = max(worst, compare_logits(lg.cpu().numpy(), lo, tol, f"step {k}"))
        check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, tol)
    dec.check()
    assert dec.position == om.position
    return om, dec, no, worst


def test_batch_64(oracle_mod):
    _dev()
    shape = synth.tiny_shape(n_layers=2, d_model=128, n_heads=2, d_ff=512, vocab=97)
    w = synth.model_weights(shape, 41)
    rng = np.random.default_rng(41)
    B = 64
    prefix = rng.standard_normal((B, 6, shape.d_model)).astype(np.float32)
    tokens = rng.integers(0, shape.vocab, size=(B, 3))
    om, dec, _, worst = _run(oracle_mod, w, B, 24, prefix, tokens, 5, TOL["tiny"])
    K, V = dec.kv_cache()
    Ko, Vo = om.kv()
    T = om.position
    np.testing.assert_allclose(K[:, :, :T].cpu().numpy(), Ko[:, :, :T], rtol=0, atol=2e-5)
    np.testing.assert_allclose(V[:, :, :T].cpu().numpy(), Vo[:, :, :T], rtol=0, atol=2e-5)
    om.close()
    dec.close()
    print(f"B=64: max |delta logits| {worst:.3g}")


def test_batch_40_medium_width(oracle_mod):
    """40 sequences at the medium width and vocabulary: the decode projections
    run on the GEMM with K split over several workgroups for the O and
    FFN-down products, the attention partials merged into rows first."""
    _dev()
    shape = synth.tiny_shape(n_layers=1, d_model=1024, n_heads=16, d_ff=4096, vocab=1393)
    w = synth.model_weights(shape, 44)
    rng = np.random.default_rng(44)
    B = 40
    prefix = rng.standard_normal((B, 12, shape.d_model)).astype(np.float32)
    om, dec, _, worst = _run(oracle_mod, w, B, 24, prefix, None, 4, TOL["medium"])
    om.close()
    dec.close()
    print(f"B=40 medium width: max |delta logits| {worst:.3g}")


@pytest.mark.parametrize("B", [1, 3])
def test_width_2048(oracle_mod, B):
    _dev()
    shape = synth.tiny_shape(n_layers=1, d_model=2048, n_heads=32, d_ff=8192, vocab=97)
    w = synth.model_weights(shape, 42)
    rng = np.random.default_rng(42 + B)
    prefix = rng.standard_normal((B, 20, shape.d_model)).astype(np.float32)
    om, dec, _, worst = _run(oracle_mod, w, B, 32, prefix, None, 4, TOL["medium"])
    om.close()
    dec.close()
    print(f"d=2048 B={B}: max |delta logits| {worst:.3g}")


def test_cache_16384_filled_then_refused(oracle_mod):
    """One head of 64, T_cap 16384 (64 splits of 256 positions): prefill
    16376 rows in four calls, decode to the last slot, then the next call is
    refused and changes nothing."""
    _dev()
    shape = synth.tiny_shape(n_layers=1, d_model=64, n_heads=1, d_ff=128, vocab=97)
    w = synth.model_weights(shape, 43)
    rng = np.random.default_rng(43)
    t_cap, P = 16384, 16376
    prefix = rng.standard_normal((1, P, 64)).astype(np.float32)
    om = oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=t_cap)
    dec = binding.Decoder(w, batch=1, t_cap=t_cap)
    worst = 0.0
    for c in range(4):
        part = prefix[:, c * P // 4:(c + 1) * P // 4]
        lo, no = om.forward(prefix=part)
        lg, ng = dec.prefill(None, _t(part))
        worst = max(worst, compare_logits(lg.cpu().numpy(), lo, TOL["tiny"], f"prefill chunk {c}"))
        check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, TOL["tiny"])
    for k in range(t_cap - P):
        tok = no.reshape(1, 1)
        lo, no = om.forward(tokens=tok)
        lg, ng = dec.decode_step(_t(tok.reshape(1)))
        worst = max(worst, compare_logits(lg.cpu().numpy(), lo, TOL["tiny"], f"step {k}"))
        check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, TOL["tiny"])
    dec.check()
    assert dec.position == t_cap == om.position
    K, _ = dec.kv_cache()
    before = K.clone()
    with pytest.raises(binding.MTError) as e:
        dec.decode_step(_t(no.reshape(1)))
    assert e.value.code == binding.MT_ERR_CACHE_FULL
    K2, _ = dec.kv_cache()
    assert torch.equal(K2, before)
    om.close()
    dec.close()
    print(f"T_cap 16384: max |delta logits| {worst:.3g}")
