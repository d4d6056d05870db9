"""Boundary behaviour that needs a device: a token id outside [0, vocab) is caught by the embedding
kernel and reported by lfm3_synchronize as LFM3_ERR_ARG (the flag clears once reported), and valid
calls around it are unaffected."""
import numpy as np
import pytest

from attention_decoder_amd import synth

pytestmark = pytest.mark.gpu


def test_bad_token_id_is_reported_at_synchronize():
    import torch
    from attention_decoder_amd.lfm3 import Engine, LFM3Error
    cfg = synth.make_config(layer_types=[0, 2, 1], max_slots=2, max_ctx=256, max_chunk=64)
    cfg["vocab"] = 1024
    eng = Engine(cfg, synth.cached_blob(cfg, seed=0))
    try:
        good = torch.from_numpy(np.array([1, 2, 1023], dtype=np.int32)).cuda()
        eng.prefill(0, tokens=good)
        eng.synchronize()                                   # nothing to report
        for bad in (1024, -1):
            toks = torch.from_numpy(np.array([5, bad, 7], dtype=np.int32)).cuda()
            eng.prefill(1, tokens=toks)                     # enqueued: returns OK
            with pytest.raises(LFM3Error) as ei:
                eng.synchronize()
            assert ei.value.status == 1 and "vocab" in ei.value.message
            eng.synchronize()                               # reported once, then cleared
            eng.reset(1)
        one = torch.from_numpy(np.array([3], dtype=np.int32)).cuda()
        eng.decode([0], tokens=one)
        eng.synchronize()
        eng.decode([0], tokens=torch.from_numpy(np.array([128000], dtype=np.int32)).cuda())
        with pytest.raises(LFM3Error):
            eng.synchronize()
    finally:
        eng.close()
