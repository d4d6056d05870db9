"""GPU parity at the largest decode batch (64 rows, the boundary's limit), full geometry at q4 g64.

Decode batches fall into three classes, each batch-invariant inside itself: 1-2 rows run the exact
GEMV, 3-32 rows run every linear on the decode MFMA GEMM, 33-64 rows run the MFMA GEMM except
in_proj and qkvg, whose input pairs (value and fp16 remainder rows) would exceed the MFMA kernel's
64 operand rows and run on the GEMV instead. Here one 64-row step is checked against the float64
oracle on three streams and, bitwise, against the same rows decoded in two 40-row batches (one of
them in reverse order).
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle

from gpu_full_common import compare_logits, dev_tokens, oracle_teacher_forced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b64():
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.full_config(bits=4, group=64, max_slots=64, max_ctx=512, max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    orc = Oracle(cfg, blob)
    orc.preload(16)
    print("q4 engine (64 slots) and oracle ready", flush=True)
    yield torch, cfg, eng, orc
    eng.close()
    orc.drop_cache()


def _prefill_all(eng, torch, prompts):
    for i, p in enumerate(prompts):
        eng.reset(i)
        eng.prefill(i, tokens=dev_tokens(torch, p), logits=False, argmax=False)


def test_batch64_decode(b64):
    torch, cfg, eng, orc = b64
    lens = synth.stream_prompt_lengths(11, 64, lo=20, hi=120)
    prompts = synth.stream_prompts(11, lens)
    step_tok = [int(t) for t in synth.prompt_tokens(401, 64)]
    _prefill_all(eng, torch, prompts)
    full = eng.decode(list(range(64)), tokens=dev_tokens(torch, step_tok), logits=True, argmax=True)
    batched = full["logits"].clone()
    ids = full["argmax"].clone()
    torch.cuda.synchronize()
    for s in (0, 37, 63):
        want = oracle_teacher_forced(orc, np.concatenate([prompts[s], [step_tok[s]]]), [])
        got = batched[s].cpu().numpy().astype(np.float64)
        compare_logits(got[None], [int(ids[s].item())], want, f"batch-64 decode, stream {s}")
    for grp in (list(range(0, 40)), list(range(63, 23, -1))):
        _prefill_all(eng, torch, prompts)
        o = eng.decode(grp, tokens=dev_tokens(torch, [step_tok[i] for i in grp]), logits=True)["logits"]
        for j, i in enumerate(grp):
            assert torch.equal(batched[i], o[j]), i
