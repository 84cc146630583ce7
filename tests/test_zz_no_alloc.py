"""mt_prefill_noalloc (the prefill entry point that allocates nothing)
against mt_prefill, through the C ABI.  Both run the same kernels; the
no-allocation variant keeps its row workspace in the library's fixed device
array instead of memory grown with hipMalloc.  Two calls in a row, the second
with a smaller input (the array keeps the first call's contents), then
decode steps from the state each call left; and a call larger than the fixed
workspace is refused before any launch."""
import numpy as np
import pytest

from audio_midi_transformer_amd import binding, synth
from parity import TOL, compare_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MEDIUM2 = synth.ModelShape("medium", 2, 1024, 16, 4096)


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(_dev())


def test_noalloc_prefill_matches_prefill():
    dev = _dev()
    w = synth.model_weights(MEDIUM2, 60)
    packed = binding.pack_weights(w)
    B, t_cap = 2, 600
    ref = binding.Decoder(w, batch=B, t_cap=t_cap, packed=packed)
    na = binding.Decoder(w, batch=B, t_cap=t_cap, packed=packed)
    rng = np.random.default_rng(61)
    for P, S in ((500, 4), (37, 0)):  # the second call is smaller
        ref.reset()
        na.reset()
        prefix = _t(rng.standard_normal((B, P, MEDIUM2.d_model)).astype(np.float32))
        tokens = _t(rng.integers(0, MEDIUM2.vocab, size=(B, S))) if S else None
        lr, nr = ref.prefill(tokens, prefix)
        lg = torch.empty_like(lr)
        ng = torch.empty_like(nr)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info(dev)[0]
        na.prefill_noalloc(tokens, prefix, lg, ng)
        torch.cuda.synchronize()
        free_after = torch.cuda.mem_get_info(dev)[0]
        assert free_after >= free_before - (4 << 20), f"device memory dropped by {free_before - free_after} bytes"
        compare_logits(lg.cpu().numpy(), lr.cpu().numpy(), TOL["medium"], f"prefill of {P} + {S} rows")
        assert np.array_equal(ng.cpu().numpy(), nr.cpu().numpy())
        assert na.position == ref.position == P + S
        T = P + S
        for c_na, c_ref in zip(na.kv_cache(), ref.kv_cache()):
            assert float((c_na[:, :, :T] - c_ref[:, :, :T]).abs().max()) <= 5e-5
        tok = nr.clone()
        for k in range(3):
            lr, nr = ref.decode_step(tok)
            lg, ng = na.decode_step(tok)
            compare_logits(lg.cpu().numpy(), lr.cpu().numpy(), TOL["medium"], f"decode step {k} after {P} + {S} rows")
            tok = nr.clone()
    ref.check()
    na.check()
    ref.close()
    na.close()


def test_noalloc_refuses_more_rows_than_the_workspace():
    """8 sequences x 504 rows at d = 1024 need 35.4 Mi floats; the fixed
    workspace holds 9 Mi: MT_ERR_UNSUPPORTED, nothing launched, position
    unchanged."""
    _dev()
    w = synth.model_weights(MEDIUM2, 62)
    dec = binding.Decoder(w, batch=8, t_cap=520)
    prefix = _t(np.zeros((8, 504, MEDIUM2.d_model), np.float32))
    with pytest.raises(binding.MTError) as e:
        dec.prefill_noalloc(None, prefix)
    assert e.value.code == binding.MT_ERR_UNSUPPORTED
    assert "fixed workspace" in str(e.value)
    assert dec.position == 0
    dec.close()
