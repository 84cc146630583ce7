"""GPU decode edge cases on every decode path (the persistent single-launch
step, one launch per sequence; the batched single-launch step, one XCD per
sequence; the per-operation kernels), at medium width:

  * exact greedy ties: LM-head rows made identical and dominant give
    bit-equal maximum logits, and the pick must be the lowest index (greedy
    decoding; the tie rule is this library's reading, the pages name none);
    the tied rows sit in different workgroups of the persistent step's LM
    head (6 rows per workgroup) and in different threads and iterations of
    the argmax kernel;
  * KV-cache indexing with a NaN-payload sentinel on the persistent step:
    after every call exactly slots [0, T_b) of sequence b hold data, every
    other slot of the cache (the sequence's own tail and the other
    sequence's slice) is bit-unchanged;
  * a decode step on an empty cache (T_past = 0: the new row is the only
    key), against the oracle.

Cache layout and in-place update: "MuScriptor Medium -- optimized W4A32
ONNX Runtime", "Model variant" (shared past/present buffers); decoder
inputs and outputs: "unifolia/muscriptor-small-onnx", "Files"."""
import numpy as np
import pytest

from audio_midi_transformer_amd import binding, synth
from parity import TOL, check_greedy, compare_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PATHS = {"persistent": binding.MT_DECODE_PERSISTENT, "kernels": binding.MT_DECODE_KERNELS,
         "batched": binding.MT_DECODE_BATCHED}
# (path, batch) pairs: the persistent step takes B <= 2 (one launch per
# sequence), the batched step 2 <= B <= 8 (one launch, one XCD per sequence)
CASES = [("persistent", 1), ("persistent", 2), ("kernels", 1), ("kernels", 2), ("batched", 2), ("batched", 8)]
MEDIUM2 = synth.ModelShape("medium", 2, 1024, 16, 4096)
SENTINEL = 0x7FC0DEAD


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


@pytest.mark.parametrize("path,B", CASES)
@pytest.mark.parametrize("rows,want", [((5, 6, 261, 700, 1392), 5), ((700, 701, 956, 1392), 700)])
def test_exact_tie_takes_lowest_index(oracle_mod, path, B, rows, want):
    _dev()
    w = synth.tie_head_rows(synth.model_weights(MEDIUM2, 50), list(rows), seed=2)
    P, steps = 40, 6
    prefix = np.random.default_rng(6).standard_normal((B, P, MEDIUM2.d_model)).astype(np.float32)
    om = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=P + steps + 1)
    dec = binding.Decoder(w, batch=B, t_cap=P + steps + 1)
    dec.set_decode_path(PATHS[path])
    lo, no = om.forward(prefix=prefix)
    lg, ng = dec.prefill(None, _t(prefix))
    for k in range(steps + 1):
        g, n = lg.cpu().numpy(), ng.cpu().numpy()
        compare_logits(g, lo, TOL["medium"], f"call {k}")
        for b in range(B):
            vals = g[b, list(rows)]
            assert np.all(vals == vals[0]), f"call {k}: tied rows differ on the GPU: {vals}"
            assert vals[0] > np.max(np.delete(g[b], list(rows)))
        assert list(n) == [want] * B, f"call {k}: picked {list(n)}, lowest tied index is {want}"
        assert list(no) == [want] * B
        check_greedy(n, g, lo, TOL["medium"], f"call {k}")
        if k == steps:
            break
        lo, no = om.forward(tokens=no.reshape(B, 1))
        lg, ng = dec.decode_step(ng)
    dec.check()
    dec.close()
    om.close()


def _fill_sentinel(dec, shape, B, t_cap):
    n = shape.n_layers * B * t_cap * shape.d_model
    sentinel = torch.full((n,), SENTINEL, dtype=torch.int32, device=_dev())
    for p in dec.kv_pointers():
        binding.hip_copy(p, sentinel.data_ptr(), n * 4)
    torch.cuda.synchronize()


def _check_slots(dec, om, T, what):
    K, V = dec.kv_cache()
    Ko, Vo = om.kv()
    for name, c, co in (("K", K, Ko), ("V", V, Vo)):
        bits = c.view(torch.int32).cpu().numpy()
        vals = c.cpu().numpy()
        for b, tb in enumerate(T):
            assert np.all(bits[:, b, tb:] == SENTINEL), f"{what}: {name} slots >= {tb} of sequence {b} were written"
            assert not np.any(bits[:, b, :tb] == SENTINEL), f"{what}: a live {name} slot of sequence {b} is unwritten"
            np.testing.assert_allclose(vals[:, b, :tb], co[:, b, :tb], rtol=0, atol=5e-5)


@pytest.mark.parametrize("B", [1, 2])
def test_persistent_kv_sentinel(oracle_mod, B):
    """Sequences at different positions (B = 2: 23 and 41 rows) decode on the
    persistent step; each launch writes only its own sequence's slot T_b of
    every layer."""
    _dev()
    w = synth.model_weights(MEDIUM2, 51)
    t_cap = 64
    lens = [23, 41][:B]
    dec = binding.Decoder(w, batch=B, t_cap=t_cap)
    dec.set_decode_path(binding.MT_DECODE_PERSISTENT)
    om = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=t_cap)
    _fill_sentinel(dec, MEDIUM2, B, t_cap)
    rng = np.random.default_rng(7)
    for b, P in enumerate(lens):
        x = rng.standard_normal((P, MEDIUM2.d_model)).astype(np.float32)
        om.forward_seq(b, prefix=x)
        dec.prefill_seq(b, None, _t(x))
    torch.cuda.synchronize()
    _check_slots(dec, om, lens, "after prefill")
    for k in range(5):
        tok = rng.integers(0, MEDIUM2.vocab, size=B)
        lo, _ = om.forward(tokens=tok[:, None])
        lg, ng = dec.decode_step(_t(tok))
        compare_logits(lg.cpu().numpy(), lo, TOL["medium"], f"step {k}")
        check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, TOL["medium"], f"step {k}")
        torch.cuda.synchronize()
        _check_slots(dec, om, [t + k + 1 for t in lens], f"after step {k}")
    dec.check()
    dec.close()
    om.close()


@pytest.mark.parametrize("path,B", CASES)
def test_decode_from_empty_cache(oracle_mod, path, B):
    """The first call is a decode step with T_past = 0: the new row is the only
    key, so attention returns its V row; then four more steps."""
    _dev()
    w = synth.model_weights(MEDIUM2, 52)
    t_cap = 16
    dec = binding.Decoder(w, batch=B, t_cap=t_cap)
    dec.set_decode_path(PATHS[path])
    om = oracle_mod.OracleModel.from_weights(w, batch=B, t_cap=t_cap)
    _fill_sentinel(dec, MEDIUM2, B, t_cap)
    tok = np.random.default_rng(8).integers(0, MEDIUM2.vocab, size=B)
    for k in range(5):
        lo, no = om.forward(tokens=tok[:, None])
        lg, ng = dec.decode_step(_t(tok))
        compare_logits(lg.cpu().numpy(), lo, TOL["medium"], f"step {k}")
        check_greedy(ng.cpu().numpy(), lg.cpu().numpy(), lo, TOL["medium"], f"step {k}")
        torch.cuda.synchronize()
        _check_slots(dec, om, [k + 1] * B, f"after step {k}")
        tok = no
    assert dec.position == 5
    dec.check()
    dec.close()
    om.close()
