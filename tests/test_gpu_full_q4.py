"""GPU parity at the full LFM3-1.7B geometry, 4-bit g64 (the decode headline's weights), in the
launch configuration the benchmark times (2048-row prefill chunks, 8 slots)."""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle

from gpu_full_common import (REL_L2, compare_logits, dev_tokens, gpu_greedy, oracle_teacher_forced, rel_l2)

pytestmark = pytest.mark.gpu

PROMPT = 320     # crosses the 256-token window seam
STEPS = 12


@pytest.fixture(scope="module")
def q4():
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.full_config(bits=4, group=64, max_slots=8, max_ctx=8704, max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    orc = Oracle(cfg, blob)
    orc.preload(16)
    yield torch, cfg, eng, orc
    eng.close()
    orc.drop_cache()


@pytest.fixture(scope="module")
def run1(q4):
    torch, cfg, eng, orc = q4
    prompt = synth.prompt_tokens(2, PROMPT)
    fed, ids, lg = gpu_greedy(eng, torch, 0, prompt, STEPS)
    ref = oracle_teacher_forced(orc, prompt, fed)
    return prompt, fed, ids, lg, ref


def test_q4_prompt_then_greedy_decode(run1):
    prompt, fed, ids, lg, ref = run1
    compare_logits(lg, ids, ref, "q4 prompt 320 + 12 greedy")


def test_q4_caller_chunks_match(q4, run1):
    """The same prompt as three prefill calls (200 + 100 + 20): conv states, rings and pages carry."""
    torch, cfg, eng, orc = q4
    prompt, fed, ids, lg, ref = run1
    _, ids2, lg2 = gpu_greedy(eng, torch, 1, prompt, STEPS, chunks=[200, 100, 20], forced=fed)
    compare_logits(lg2, ids2, ref, "q4 chunked 200+100+20, teacher-forced")


def test_q4_per_layer_residuals(q4):
    torch, cfg, eng, orc = q4
    prompt = synth.prompt_tokens(3, 300)
    L, H = cfg["n_layers"], cfg["hidden"]
    cap = torch.zeros((L, len(prompt), H), dtype=torch.float32, device="cuda")
    eng.reset(2)
    eng.capture(cap, len(prompt))
    eng.prefill(2, tokens=dev_tokens(torch, prompt), logits=False, argmax=False)
    eng.capture(None, 0)
    torch.cuda.synchronize()
    got = cap.cpu().numpy().astype(np.float64)
    want = orc.forward(orc.new_slot(), tokens=prompt, logits=None, capture=True)["layers"]
    rels = [rel_l2(got[i], want[i]) for i in range(L)]
    print("per-layer rel-L2:", " ".join(f"{r:.2e}" for r in rels))
    assert max(rels) <= REL_L2, rels


def test_q4_batched_decode(q4):
    """Eight streams decoded together (the MFMA path of 3+ rows): equal, bitwise, to the same streams
    decoded as two batches of four (a row's result does not depend on the rows beside it); two of
    them against the float64 oracle."""
    torch, cfg, eng, orc = q4
    lens = [37, 300, 260, 5, 128, 257, 90, 400]
    prompts = [synth.prompt_tokens(100 + i, n) for i, n in enumerate(lens)]
    step_tok = [int(t) for t in synth.prompt_tokens(200, 8)]

    def run(groups):
        for i in range(8):
            eng.reset(i)
            eng.prefill(i, tokens=dev_tokens(torch, prompts[i]), logits=False, argmax=False)
        out = {}
        for grp in groups:
            o = eng.decode(list(grp), tokens=dev_tokens(torch, [step_tok[i] for i in grp]), logits=True, argmax=True)
            for j, i in enumerate(grp):
                out[i] = (o["logits"][j].clone(), int(o["argmax"][j].item()))
        torch.cuda.synchronize()
        return out

    eight = run([range(8)])
    halves = run([(4, 0, 6, 2), (1, 7, 3, 5)])
    for i in range(8):
        assert torch.equal(eight[i][0], halves[i][0]), i
    for i in (3, 0):
        want = oracle_teacher_forced(orc, np.concatenate([prompts[i], [step_tok[i]]]), [])
        got = eight[i][0].cpu().numpy().astype(np.float64)
        compare_logits(got[None], [eight[i][1]], want, f"q4 batch-8 decode, stream {i}")
