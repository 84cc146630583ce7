"""GPU parity of classifier-free guidance over row pairs (mt_cfg_combine)
against the CPU oracle, through the C ABI.

The guided value is a binary64 difference, product and sum rounded once to
binary32 on both sides, so on identical logits the guided rows and the argmax
are compared bit for bit.  In whole-model pair runs the logits themselves
differ within the model tolerance tol, so the guided rows are held to
(|cfg| + |cfg - 1|) tol plus one binary32 rounding, and the argmax follows the
epsilon-tie rule with that bound."""
import numpy as np
import pytest

from audio_midi_transformer_amd import binding, synth
from parity import TOL, check_argmax, check_own_argmax, compare_logits, top2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


@pytest.mark.parametrize("pairs,V", [(1, 1393), (3, 1393), (8, 1393), (2, 1), (2, 255), (2, 256), (2, 257),
                                     (64, 1000)])
@pytest.mark.parametrize("cfg", [2.0, 1.0, 0.0, -0.5, 7.25])
def test_cfg_combine_bit_exact(oracle_mod, pairs, V, cfg):
    _dev()
    rng = np.random.default_rng(1000 * pairs + V)
    lg = (rng.standard_normal((2 * pairs, V)) * 3).astype(np.float32)
    if V > 4 and pairs > 1:
        # a pair whose guided row is constant (all ties: index 0) and one whose
        # maximum is repeated (the lower index wins)
        lg[1] = 2.0
        lg[pairs + 1] = 1.0
        lg[0, V // 2] = lg[0, V - 1] = 50.0
    want_g, want_n = oracle_mod.cfg_combine(lg, cfg)
    g, nx, tp = binding.cfg_combine(_t(lg), cfg)
    torch.cuda.synchronize()
    g, nx, tp = g.cpu().numpy(), nx.cpu().numpy(), tp.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), want_g.view(np.uint32))
    assert np.array_equal(nx, want_n)
    assert np.array_equal(tp, np.concatenate([want_n, want_n]))
    if cfg == 1.0:
        assert np.array_equal(g.view(np.uint32), lg[:pairs].view(np.uint32))
    # the argmax alone, without storing the guided rows
    _, nx2, _ = binding.cfg_combine(_t(lg), cfg, store_guided=False)
    assert np.array_equal(nx2.cpu().numpy(), want_n)


def _pair_run(oracle_mod, shape, seed, Np, P, steps, cfg, tol):
    w = synth.model_weights(shape, seed)
    rng = np.random.default_rng(seed)
    d = shape.d_model
    cond = rng.standard_normal((Np, P, d)).astype(np.float32)
    uncond = cond.copy()
    uncond[:, -2:] = rng.standard_normal((Np, 2, d)).astype(np.float32)  # the class rows differ
    prefix = np.concatenate([cond, uncond])
    B = 2 * Np
    t_cap = P + steps + 1
    om = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=t_cap)
    dec = binding.Decoder(w, batch=B, t_cap=t_cap)
    gtol = (abs(cfg) + abs(cfg - 1.0)) * tol * (1 + 2.0 ** -20) + 1e-6
    lo, _ = om.forward(prefix=prefix)
    lg, _ = dec.prefill(None, _t(prefix))
    worst = ties = 0
    for k in range(steps + 1):
        go, no = oracle_mod.cfg_combine(lo, cfg)
        gg, ng, tp = binding.cfg_combine(lg, cfg)
        gg, ng, tp = gg.cpu().numpy(), ng.cpu().numpy(), tp.cpu().numpy()
        worst = max(worst, compare_logits(gg, go, gtol, f"guided, call {k}"))
        check_own_argmax(ng, gg, f"guided, call {k}")
        ties += check_argmax(ng, *top2(go), go[np.arange(Np), ng], gtol)
        assert np.array_equal(tp, np.concatenate([ng, ng]))
        if k == steps:
            break
        tok = np.concatenate([no, no])  # the oracle's guided token for both rows of each pair
        lo, _ = om.forward(tokens=tok[:, None])
        lg, _ = dec.decode_step(_t(tok))
    dec.check()
    K, V = dec.kv_cache()
    Ko, Vo = om.kv()
    T = om.position
    np.testing.assert_allclose(K[:, :, :T].cpu().numpy(), Ko[:, :, :T], rtol=0, atol=2e-5)
    np.testing.assert_allclose(V[:, :, :T].cpu().numpy(), Vo[:, :, :T], rtol=0, atol=2e-5)
    om.close()
    dec.close()
    print(f"CFG {cfg} pairs {Np} width {d}: {steps + 1} calls, {ties} epsilon-ties, max |delta guided| {worst:.3g}")


@pytest.mark.parametrize("cfg", [2.0, 1.0, 3.5])
def test_cfg_pair_run_tiny(oracle_mod, cfg):
    _dev()
    shape = synth.tiny_shape(n_layers=2, d_model=128, n_heads=2, d_ff=512, vocab=97)
    _pair_run(oracle_mod, shape, 61, 3, 11, 12, cfg, TOL["tiny"])


def test_cfg_pair_run_medium_width(oracle_mod):
    """One pair (B = 2) at the medium width and vocabulary, CFG = 2 (the
    coefficient of the paper's scaling table)."""
    _dev()
    shape = synth.tiny_shape(n_layers=2, d_model=1024, n_heads=16, d_ff=4096, vocab=1393)
    _pair_run(oracle_mod, shape, 62, 1, 40, 8, 2.0, TOL["medium"])


def test_cfg_closed_loop_feeds_both_rows(oracle_mod):
    """Greedy guided decoding that never leaves the device: token_pair of one
    call is the token argument of the next, and at cfg = 1 the guided rows are
    the conditional rows of the same call bit for bit."""
    _dev()
    shape = synth.tiny_shape(n_layers=2, d_model=128, n_heads=2, d_ff=512, vocab=97)
    w = synth.model_weights(shape, 63)
    rng = np.random.default_rng(63)
    Np, P = 2, 6
    prefix = rng.standard_normal((2 * Np, P, shape.d_model)).astype(np.float32)
    dec = binding.Decoder(w, batch=2 * Np, t_cap=32)
    lg, _ = dec.prefill(None, _t(prefix))
    g, nx, tp = binding.cfg_combine(lg, 1.0)
    for k in range(10):
        assert torch.equal(g, lg[:Np]), k
        assert torch.equal(tp[:Np], nx) and torch.equal(tp[Np:], nx)
        lg, _ = dec.decode_step(tp)
        g, nx, tp = binding.cfg_combine(lg, 1.0, token_pair=torch.empty_like(tp))
    dec.check()
    assert dec.position == P + 10
    dec.close()
