"""GPU parity of the ragged batch (sequences of one batch at their own
positions: single-sequence prefills and restarts, lockstep decode at
different positions) against independent one-sequence oracle models fed
the same rows, through the C ABI."""
import numpy as np
import pytest

from audio_midi_transformer_amd import binding, synth
from parity import TOL, compare_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


class _Pair:
    """The GPU batch and one oracle model per sequence."""

    def __init__(self, oracle_mod, w, B, t_cap, path=None):
        self.dec = binding.Decoder(w, batch=B, t_cap=t_cap)
        if path is not None:
            self.dec.set_decode_path(path)
        self.om = [oracle_mod.OracleModel.from_weights(w, batch=1, t_cap=t_cap) for _ in range(B)]
        self.B = B

    def prefill_seq(self, b, tokens=None, prefix=None, what=""):
        lg, nx = self.dec.prefill_seq(b, _t(tokens) if tokens is not None else None,
                                      _t(prefix) if prefix is not None else None)
        lo, no = self.om[b].forward(tokens=None if tokens is None else tokens[None],
                                    prefix=None if prefix is None else prefix[None])
        compare_logits(lg.cpu().numpy()[None], lo, TOL["tiny"], f"prefill_seq {b} {what}")

    def decode(self, tok, what=""):
        lg, _ = self.dec.decode_step(_t(tok))
        lg = lg.cpu().numpy()
        for b in range(self.B):
            lo, _ = self.om[b].forward(tokens=tok[b:b + 1, None])
            compare_logits(lg[b:b + 1], lo, TOL["tiny"], f"decode {what} sequence {b}")

    def restart(self, b):
        self.dec.reset_seq(b)
        self.om[b].reset()

    def check_cache(self):
        self.dec.check()
        K, V = self.dec.kv_cache()
        for b in range(self.B):
            T = self.om[b].position
            assert self.dec.position_seq(b) == T
            Ko, Vo = self.om[b].kv()
            np.testing.assert_allclose(K[:, b, :T].cpu().numpy(), Ko[:, 0, :T], rtol=0, atol=2e-5)
            np.testing.assert_allclose(V[:, b, :T].cpu().numpy(), Vo[:, 0, :T], rtol=0, atol=2e-5)

    def close(self):
        self.dec.close()
        for m in self.om:
            m.close()


def test_ragged_tiny_staggered_joins_and_restart(oracle_mod):
    _dev()
    shape = synth.tiny_shape(n_layers=2)
    w = synth.model_weights(shape, 60)
    d, V = shape.d_model, shape.vocab
    rng = np.random.default_rng(8)
    p = _Pair(oracle_mod, w, 3, 48)
    for b, P in ((0, 5), (1, 19), (2, 2)):
        p.prefill_seq(b, prefix=rng.standard_normal((P, d)).astype(np.float32))
    p.prefill_seq(1, tokens=rng.integers(0, V, 3), what="prompt")
    for step in range(6):
        p.decode(rng.integers(0, V, 3), f"step {step}")
        if step == 2:
            p.restart(2)
            p.prefill_seq(2, prefix=rng.standard_normal((7, d)).astype(np.float32), what="restart")
    assert [p.dec.position_seq(b) for b in range(3)] == [11, 28, 10]
    p.check_cache()
    p.close()


@pytest.mark.parametrize("path", [binding.MT_DECODE_AUTO, binding.MT_DECODE_KERNELS])
def test_ragged_medium_width_long_and_short(oracle_mod, path):
    """Very different lengths in one batch: the decode attention's splits
    cover the longest sequence and are empty for the short ones."""
    _dev()
    shape = synth.tiny_shape(n_layers=1, d_model=1024, n_heads=16, d_ff=4096, vocab=1393)
    w = synth.model_weights(shape, 61)
    rng = np.random.default_rng(9)
    p = _Pair(oracle_mod, w, 4, 720, path)
    for b, P in ((0, 300), (1, 40), (2, 700), (3, 1)):
        p.prefill_seq(b, prefix=rng.standard_normal((P, 1024)).astype(np.float32))
    for step in range(4):
        p.decode(rng.integers(0, 1393, 4), f"step {step}")
    p.check_cache()
    p.close()


def test_ragged_one_sequence_batch_uses_own_position(oracle_mod):
    """B = 1: prefill_seq and reset_seq on the only sequence, the persistent
    step continuing from its position."""
    _dev()
    shape = synth.ModelShape("small", 2, 768, 12, 3072)
    w = synth.model_weights(shape, 62)
    rng = np.random.default_rng(10)
    p = _Pair(oracle_mod, w, 1, 64)
    p.prefill_seq(0, prefix=rng.standard_normal((20, 768)).astype(np.float32))
    for step in range(3):
        p.decode(rng.integers(0, 1393, 1), f"step {step}")
    p.restart(0)
    p.prefill_seq(0, tokens=rng.integers(0, 1393, 4), what="after restart")
    p.decode(rng.integers(0, 1393, 1), "after restart")
    p.check_cache()
    p.close()


def test_ragged_errors_leave_state_untouched(oracle_mod):
    _dev()
    shape = synth.tiny_shape(n_layers=1)
    w = synth.model_weights(shape, 63)
    dec = binding.Decoder(w, batch=2, t_cap=8)
    rng = np.random.default_rng(11)
    with pytest.raises(binding.MTError) as e:
        dec.prefill_seq(2, prefix=_t(rng.standard_normal((1, shape.d_model)).astype(np.float32)))
    assert e.value.code == binding.MT_ERR_INVALID_ARG
    dec.prefill_seq(1, prefix=_t(rng.standard_normal((8, shape.d_model)).astype(np.float32)))
    assert (dec.position_seq(0), dec.position_seq(1)) == (0, 8)
    # sequence 1 is full: a decode step of the batch is refused
    with pytest.raises(binding.MTError) as e:
        dec.decode_step(_t(np.array([1, 2])))
    assert e.value.code == binding.MT_ERR_CACHE_FULL
    assert (dec.position_seq(0), dec.position_seq(1)) == (0, 8)
    dec.reset_seq(1)
    dec.decode_step(_t(np.array([1, 2])))
    assert (dec.position_seq(0), dec.position_seq(1)) == (1, 1)
    dec.check()
    dec.close()
