"""GPU parity for the long-context, many-stream layout: 4-bit linears in groups of 32 with an 8-bit
g64 embedding / tied head (the VL 4-bit export of "TensorFold issue #1491", "Checkpoint
handling"), decoded 32 streams at a time.

- A 300-token prompt and greedy steps against the float64 oracle, teacher-forced.
- 32 concurrent streams of different lengths: one batched decode step equals the same step decoded
  as two batches of 16, bitwise, and three of the streams match the oracle.
The full-size run (32768-token prefill, 32 streams at contexts uniform in [1k, 32k]) is timed by
bench.py; the whole-model oracle would take hours there. Its attention at that size is held to a
float64 bound at kernel level by test_gpu_attention.py: decode at T = 32768 alone and in batches of
8 and 32 mixed lengths, and the prompt's last 2048-row pass after 30,720 keys.
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle

from gpu_full_common import compare_logits, dev_tokens, gpu_greedy, oracle_teacher_forced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cfg5():
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.full_config(bits=4, group=32, embed_bits=8, embed_group=64, max_slots=32, max_ctx=2048,
                            max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    orc = Oracle(cfg, blob)
    orc.preload(16)
    print("g32 / 8-bit head engine and oracle ready", flush=True)
    yield torch, cfg, eng, orc
    eng.close()
    orc.drop_cache()


def test_cfg5_prompt_then_greedy(cfg5):
    torch, cfg, eng, orc = cfg5
    prompt = synth.prompt_tokens(8, 300)
    fed, ids, lg = gpu_greedy(eng, torch, 0, prompt, 4)
    ref = oracle_teacher_forced(orc, prompt, fed)
    compare_logits(lg, ids, ref, "q4 g32 + 8-bit head, prompt 300 + 4 greedy")


def test_cfg5_batch32_decode(cfg5):
    torch, cfg, eng, orc = cfg5
    lens = synth.stream_prompt_lengths(9, 32, lo=20, hi=80)
    prompts = synth.stream_prompts(9, lens)
    for i in range(32):
        eng.reset(i)
        eng.prefill(i, tokens=dev_tokens(torch, prompts[i]), logits=False, argmax=False)
    step_tok = [int(t) for t in synth.prompt_tokens(400, 32)]
    both = eng.decode(list(range(32)), tokens=dev_tokens(torch, step_tok), logits=True, argmax=True)
    batched = both["logits"].clone()
    torch.cuda.synchronize()
    for s in (0, 13, 31):
        want = oracle_teacher_forced(orc, np.concatenate([prompts[s], [step_tok[s]]]), [])
        got = batched[s].cpu().numpy().astype(np.float64)
        compare_logits(got[None], [int(both["argmax"][s].item())], want, f"batch-32 decode, stream {s}")
    for i in range(32):
        eng.reset(i)
        eng.prefill(i, tokens=dev_tokens(torch, prompts[i]), logits=False, argmax=False)
    for grp in (list(range(16, 32)), list(range(15, -1, -1))):
        o = eng.decode(grp, tokens=dev_tokens(torch, [step_tok[i] for i in grp]), logits=True)["logits"]
        for j, i in enumerate(grp):
            assert torch.equal(batched[i], o[j]), i
