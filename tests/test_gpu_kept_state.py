"""Kept states: save a slot's state, load it into another slot (or the same one after it moved on),
and continue ("TensorFold PR #1508", Verification: resumed == fresh; "LFM3-1.7B port": a rewind
must restore the conv state as well).

Full geometry at 4-bit g64. A 700-token prompt (past the sliding window, so the rings hold a
wrapped window and the full layers several pages) is prefilled in slot 0 and its state saved;
slot 0 then decodes 6 teacher-forced steps. The same 6 steps are then decoded
- from the state loaded into another slot,
- from the state loaded back into slot 0 after it had moved on (a rewind),
- in a freshly reset slot that re-prefills the prompt,
- and from the state loaded into two slots decoded together (the same batch class),
and every logit must equal slot 0's bit for bit; slot 0's logits are held to the float64 oracle.
A state saved at the empty slot restores an empty slot. The pool's census closes.
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle

from gpu_full_common import compare_logits, dev_tokens, oracle_teacher_forced

pytestmark = pytest.mark.gpu


def test_resumed_equals_fresh():
    import torch
    from attention_decoder_amd.lfm3 import Engine, LFM3Error
    cfg = synth.full_config(bits=4, group=64, max_slots=8, max_ctx=2048, max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    try:
        free0 = eng.free_pages()
        prompt = synth.prompt_tokens(21, 700)
        forced = [int(t) for t in synth.prompt_tokens(22, 6)]

        def steps(slots):
            out = []
            for t in forced:
                o = eng.decode(slots, tokens=dev_tokens(torch, [t] * len(slots)), logits=True, argmax=True)
                out.append(o["logits"].clone())
            torch.cuda.synchronize()
            return [torch.stack([o[j] for o in out]) for j in range(len(slots))]

        eng.reset(0)
        eng.prefill(0, tokens=dev_tokens(torch, prompt), logits=False, argmax=False)
        state, n = eng.save_state(0)
        assert n == 700
        ref = steps([0])[0]
        print("slot 0 decoded", flush=True)

        eng.reset(3)
        eng.load_state(3, state, n)
        assert eng.length(3) == 700
        assert torch.equal(steps([3])[0], ref)
        eng.load_state(0, state, n)                      # rewind slot 0 to the saved point
        assert eng.length(0) == 700
        assert torch.equal(steps([0])[0], ref)
        eng.reset(5)
        eng.prefill(5, tokens=dev_tokens(torch, prompt), logits=False, argmax=False)
        assert torch.equal(steps([5])[0], ref)
        eng.load_state(6, state, n)
        eng.load_state(7, state, n)
        two = steps([6, 7])
        assert torch.equal(two[0], ref) and torch.equal(two[1], ref)
        print("resumed == fresh, bitwise", flush=True)

        # an empty state restores an empty slot
        eng.reset(2)
        empty, n0 = eng.save_state(2)
        assert n0 == 0
        eng.load_state(4, empty, 0)
        assert eng.length(4) == 0
        with pytest.raises(LFM3Error) as ei:
            eng.load_state(4, empty, 700)                # buffer too small for 700 positions
        assert ei.value.status == 1 and eng.length(4) == 0

        for s in range(8):
            eng.reset(s)
        assert eng.free_pages() == free0
    finally:
        eng.close()
    orc = Oracle(cfg, blob)
    orc.preload(16)
    try:
        want = oracle_teacher_forced(orc, prompt, forced)[1:]
        got = ref.cpu().numpy().astype(np.float64)
        compare_logits(got, list(np.argmax(got, axis=1)), want, "700-token prompt, state saved, 6 steps")
    finally:
        orc.drop_cache()
