"""GPU parity at the full LFM3-1.7B geometry for the 8-bit and 6-bit weight schemes.

- 8-bit g64, concurrent streams (the 8-stream structure): eight prompts of different lengths,
  each crossing the 256-token window seam, prefilled into their own slots, then greedy decode of
  all eight in one batch; every stream's logits against the float64 oracle run teacher-forced on
  that stream alone. At the full stream lengths (prompts uniform in [300, 2960]), where the oracle
  would take minutes, a batch of eight is checked against batches of three and five, bitwise.
- 6-bit g64, chunked prefill (the 8192-token structure): a prompt over several library chunks,
  whose last-position logits are checked against the oracle both when the library chunks it and
  when the caller does; at the full 8192 tokens in 2048-row chunks two different chunkings must
  agree.
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle, greedy_argmax, top2_margin

from gpu_full_common import LOGIT_TOL, MARGIN, compare_logits, dev_tokens, oracle_teacher_forced

pytestmark = pytest.mark.gpu


def _engine(bits, max_ctx):
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.full_config(bits=bits, group=64, max_slots=8, max_ctx=max_ctx, max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    return cfg, blob, Engine(cfg, blob)


@pytest.fixture(scope="module")
def q8():
    import torch
    cfg, blob, eng = _engine(8, 4096)
    orc = Oracle(cfg, blob)
    orc.preload(16)
    print("q8 engine and oracle ready", flush=True)
    yield torch, cfg, eng, orc
    eng.close()
    orc.drop_cache()


def test_q8_eight_streams_teacher_forced(q8):
    torch, cfg, eng, orc = q8
    steps = 5
    lens = synth.stream_prompt_lengths(5, 8, lo=260, hi=420)
    prompts = synth.stream_prompts(5, lens)
    first_ids, first_lg = [], []
    for i in range(8):
        eng.reset(i)
        out = eng.prefill(i, tokens=dev_tokens(torch, prompts[i]), logits=True, argmax=True)
        first_lg.append(out["logits"].clone())
        first_ids.append(int(out["argmax"].item()))
    ids = [first_ids]
    lgs = [torch.stack(first_lg)]
    for _ in range(steps):
        o = eng.decode(list(range(8)), tokens=dev_tokens(torch, ids[-1]), logits=True, argmax=True)
        lgs.append(o["logits"].clone())
        ids.append([int(v) for v in o["argmax"].cpu().numpy()])
    torch.cuda.synchronize()
    lg = torch.stack(lgs).cpu().numpy().astype(np.float64)   # [steps + 1, 8, vocab]
    for s in range(8):
        fed = [ids[t][s] for t in range(steps)]
        ref = oracle_teacher_forced(orc, prompts[s], fed)
        compare_logits(lg[:, s], [ids[t][s] for t in range(steps + 1)], ref, f"q8 stream {s} (prompt {lens[s]})")


def test_q8_full_length_streams_batch_composition(q8):
    """Prompts at the full stream lengths (uniform in [300, 2960]): one step of the 8 streams decoded
    together equals, bitwise, the same step decoded as batches of 3 and 5."""
    torch, cfg, eng, orc = q8
    lens = synth.stream_prompt_lengths(4, 8)
    prompts = synth.stream_prompts(4, lens)
    step_tok = [int(t) for t in synth.prompt_tokens(300, 8)]

    def run(groups):
        for i in range(8):
            eng.reset(i)
            eng.prefill(i, tokens=dev_tokens(torch, prompts[i]), logits=False, argmax=False)
        out = {}
        for grp in groups:
            o = eng.decode(list(grp), tokens=dev_tokens(torch, [step_tok[i] for i in grp]), logits=True)["logits"]
            for j, i in enumerate(grp):
                out[i] = o[j].clone()
        return out

    eight = run([range(8)])
    split = run([(5, 1, 7), (0, 6, 2, 4, 3)])
    for i in range(8):
        assert torch.equal(eight[i], split[i]), i


@pytest.fixture(scope="module")
def q6():
    import torch
    cfg, blob, eng = _engine(6, 8448)
    print("q6 engine ready", flush=True)
    yield torch, cfg, blob, eng
    eng.close()


def _last_logits(torch, eng, slot, toks, chunks):
    eng.reset(slot)
    pd = dev_tokens(torch, toks)
    r0 = 0
    for n in chunks:
        out = eng.prefill(slot, tokens=pd[r0:r0 + n], logits=True, argmax=True)
        r0 += n
    torch.cuda.synchronize()
    return out["logits"].cpu().numpy().astype(np.float64), int(out["argmax"].item())


def test_q6_chunked_prefill_last_logits(q6):
    """A 600-token prompt through 256-row library chunks (256 + 256 + 88) and through caller chunks
    (100 + 300 + 200): conv states, rings and pages carried across every boundary; the last
    position's logits against the oracle (the oracle takes ~0.05 s a token, so the prompt stays
    short; the 2048-row chunking at 8192 tokens is checked by the next test)."""
    from attention_decoder_amd.lfm3 import Engine
    torch, cfg, blob, _ = q6
    small = dict(cfg, max_slots=1, max_ctx=1024, max_chunk=256, n_pages=1024 // 16)
    eng = Engine(small, blob)
    toks = synth.prompt_tokens(6, 600)
    orc = Oracle(small, blob)
    orc.preload(16)
    print("q6 oracle preloaded", flush=True)
    want = orc.forward(orc.new_slot(), tokens=toks, logits="last")["logits"][0]
    orc.drop_cache()
    print("q6 oracle forward done", flush=True)
    for label, chunks in [("library chunks 256 + 256 + 88", [600]), ("caller chunks 100 + 300 + 200", [100, 300, 200])]:
        got, gid = _last_logits(torch, eng, 0, toks, chunks)
        compare_logits(got[None], [gid], want[None], f"q6 600-token prefill, {label}")
    eng.close()


def test_q6_8k_prefill_chunkings_agree(q6):
    """8192 tokens as four library chunks of 2048 and as caller chunks 3000 + 3000 + 2192."""
    torch, cfg, blob, eng = q6
    toks = synth.prompt_tokens(7, 8192)
    a, ia = _last_logits(torch, eng, 0, toks, [8192])
    b, ib = _last_logits(torch, eng, 1, toks, [3000, 3000, 2192])
    d = float(np.abs(a - b).max())
    print(f"q6 8k prefill, two chunkings: max|dlogit| {d:.3e}")
    assert np.isfinite(a).all() and d <= LOGIT_TOL, d
    if top2_margin(a[None])[0] >= MARGIN:
        assert ia == ib == int(greedy_argmax(a[None])[0])
