"""Boundary behaviour that needs a device:
- a token id outside [0, vocab) is caught by the embedding kernel and reported by lfm3_synchronize
  as LFM3_ERR_ARG (the flag clears once reported), and valid calls around it are unaffected;
- every host-side refusal of lfm3_prefill / lfm3_decode_batch (slot out of range, a slot twice in
  one step, no input or two, too many rows for max_ctx, the page pool exhausted, an empty or
  oversized batch) returns its named status before anything is enqueued: slot lengths and the
  free-page count are unchanged, and the slots then decode exactly as a context that never saw the
  bad calls ("TensorFold PR #1508": admission checks before any kernel; forward refuses rows past
  a slot's pages)."""
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


ERR_ARG, ERR_SLOT, ERR_CAPACITY = 1, 4, 5


def test_refused_calls_change_nothing():
    import torch
    from attention_decoder_amd.lfm3 import Engine, LFM3Error, lfm3_free_pages, lfm3_slot_length
    # 3 slots of up to 64 positions and a pool of 6 pages of 16: the two prompts (20 and 27
    # positions) hold 4 pages, so a 64-row prompt on the third slot finds the pool exhausted
    cfg = synth.make_config(layer_types=[0, 2, 1], max_slots=3, max_ctx=64, max_chunk=32, n_pages=6)
    blob = synth.cached_blob(cfg, seed=0)
    dev = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()
    prompt = [dev(synth.prompt_tokens(40 + i, 20 + 7 * i) % cfg["vocab"]) for i in range(2)]
    steps = [dev([(11 * t + 3) % cfg["vocab"], (13 * t + 5) % cfg["vocab"]]) for t in range(4)]

    def run(bad_calls):
        eng = Engine(cfg, blob)
        try:
            for i in range(2):
                eng.prefill(i, tokens=prompt[i], logits=False, argmax=False)
            state = lambda: ([lfm3_slot_length(eng.ctx, i) for i in range(3)], lfm3_free_pages(eng.ctx))
            before = state()
            for call, status in bad_calls(eng):
                with pytest.raises(LFM3Error) as ei:
                    call()
                assert ei.value.status == status, (ei.value.status, ei.value.message)
                assert state() == before, ei.value.message
            out = [eng.decode([0, 1], tokens=s)["logits"].clone() for s in steps]
            torch.cuda.synchronize()
            return torch.stack(out).cpu()
        finally:
            eng.close()

    def bad(eng):
        one = dev([7])
        fill = dev(synth.prompt_tokens(90, 64) % cfg["vocab"])
        hid = torch.zeros((1, cfg["hidden"]), dtype=torch.int16, device="cuda")
        return [
            (lambda: eng.prefill(3, tokens=one), ERR_SLOT),                            # slot past max_slots
            (lambda: eng.prefill(-1, tokens=one), ERR_SLOT),
            (lambda: eng.decode([0, 3], tokens=dev([1, 2])), ERR_SLOT),
            (lambda: eng.decode([1, 1], tokens=dev([1, 2])), ERR_ARG),                 # a slot twice
            (lambda: eng.decode([], tokens=dev([1])), ERR_ARG),                        # empty batch
            (lambda: eng.decode([0, 1, 2, 0], tokens=dev([1, 2, 3, 4])), ERR_ARG),    # more rows than slots
            (lambda: eng.prefill(0, tokens=one, hidden=hid), ERR_ARG),                 # two inputs
            (lambda: eng.prefill(0, tokens=fill[:64 - 19]), ERR_CAPACITY),             # 20 + 45 > max_ctx
            (lambda: eng.prefill(2, tokens=fill), ERR_CAPACITY),                       # needs 4 pages, 2 free
        ]

    ref = run(lambda eng: [])
    got = run(bad)
    assert torch.equal(ref, got)
