"""GPU parity at the lengths the benchmark times, full LFM3-1.7B geometry, against the float64 oracle.

- 4-bit g64, the headline decode job's shape: a 2048-token prompt in one 2048-row pass, then greedy
  decode steps at T = 2049.. -- logits at every position within the bar and teacher-forced ids.
- 6-bit g64, an 8192-token prompt in four 2048-row passes (conv states, sliding rings and pages
  carried across passes): the last row's logits within the bar and its greedy id.
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle

from gpu_full_common import compare_logits, gpu_greedy, oracle_teacher_forced

pytestmark = pytest.mark.gpu


def _engine(bits):
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.full_config(bits=bits, group=64, max_slots=8, max_ctx=8704, max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    orc = Oracle(cfg, blob)
    orc.preload(16)
    print(f"{bits}-bit engine and oracle ready", flush=True)
    return cfg, eng, orc


def test_q4_2048_prompt_then_greedy():
    import torch
    cfg, eng, orc = _engine(4)
    try:
        prompt = synth.prompt_tokens(2, 2048)
        fed, ids, lg = gpu_greedy(eng, torch, 0, prompt, 8)
        print("GPU 2048 + 8 done", flush=True)
        ref = oracle_teacher_forced(orc, prompt, fed)
        compare_logits(lg, ids, ref, "q4 2048-token prompt (one pass) + 8 greedy steps")
    finally:
        eng.close()
        orc.drop_cache()


def test_q6_8192_prompt_last_row():
    import torch
    from gpu_full_common import dev_tokens
    cfg, eng, orc = _engine(6)
    try:
        prompt = synth.prompt_tokens(5, 8192)
        eng.reset(0)
        out = eng.prefill(0, tokens=dev_tokens(torch, prompt), logits=True, argmax=True)
        torch.cuda.synchronize()
        got = out["logits"].cpu().numpy().astype(np.float64)[None]
        gid = [int(out["argmax"].item())]
        print("GPU 8192-token prefill done", flush=True)
        st = orc.new_slot()
        for r0 in range(0, 8192, 2048):            # the oracle's prefill equals its chunked prefill
            out_o = orc.forward(st, tokens=prompt[r0:r0 + 2048], logits="last" if r0 == 6144 else None)
            print(f"oracle rows {r0}..{r0 + 2047} done", flush=True)
        want = out_o["logits"]
        compare_logits(got, gid, want, "q6 8192-token prompt (four 2048-row passes), last row")
    finally:
        eng.close()
        orc.drop_cache()
