"""Drafted decoding with verify windows == plain greedy decoding ("TensorFold PR #1508",
Verification: drafted == plain; issue #1491, Validation: partial acceptance), full geometry at
4-bit g64.

A 300-token prompt; plain greedy decode gives the reference continuation. The drafted stream
proposes windows built from that continuation with planted wrong drafts (full acceptance, a miss
at the second and at the first draft, a six-row window), verifies each window in one pass and
commits the accepted rows (the conv states of the last accepted row, pages past it returned).
- The drafted ids equal the plain ones up to the first position whose float64 top-2 margin is
  below 4e-2 (after a near-tie the two may part legitimately).
- Every verify row's logits, accepted or not, are within 2e-2 of the float64 oracle run on the
  same window from the committed state, with teacher-forced ids.
- After the windows, plain decode steps on the drafted slot match the oracle (a commit that kept
  the wrong conv state moves the logits far past the bar).
- A slot with an open window refuses other calls; commits outside the window are refused.
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle, top2_margin

from gpu_full_common import MARGIN, compare_logits, dev_tokens, gpu_greedy, oracle_teacher_forced

pytestmark = pytest.mark.gpu


def test_drafted_equals_plain():
    import torch
    from attention_decoder_amd.lfm3 import Engine, LFM3Error
    cfg = synth.full_config(bits=4, group=64, max_slots=4, max_ctx=1024, max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    prompt = synth.prompt_tokens(31, 300)
    windows = []
    try:
        free0 = eng.free_pages()
        _, plain, _ = gpu_greedy(eng, torch, 0, prompt, 20)
        eng.reset(1)
        out = eng.prefill(1, tokens=dev_tokens(torch, prompt), logits=False, argmax=True)
        gen = [int(out["argmax"].item())]
        # (window rows, index of the first planted wrong draft or None)
        plan = [(4, None), (4, 2), (4, 1), (6, None), (3, 1), (4, 3)]
        for w, bad in plan:
            drafts = list(plain[len(gen):len(gen) + w - 1])
            drafts += [0] * (w - 1 - len(drafts))
            if bad is not None:
                drafts[bad - 1] = (drafts[bad - 1] + 7919) % 128000
            win = [gen[-1]] + drafts
            lg, am = eng.verify(1, dev_tokens(torch, win))
            am = [int(v) for v in am.cpu().numpy()]
            a = 1
            while a < w and win[a] == am[a - 1]:
                a += 1
            eng.commit(1, a)
            windows.append((win, a, lg.cpu().numpy().astype(np.float64), am))
            gen += am[:a]
            print(f"window {win} -> accepted {a}", flush=True)
        with pytest.raises(LFM3Error):
            eng.commit(1, 0)                              # no window open
        lg_v, _ = eng.verify(1, dev_tokens(torch, [gen[-1], 5]))
        with pytest.raises(LFM3Error):
            eng.decode([1], tokens=dev_tokens(torch, [1]))  # slot has an open window
        with pytest.raises(LFM3Error):
            eng.commit(1, 3)                              # more rows than the window holds
        eng.commit(1, 1)
        gen.append(int(np.argmax(lg_v[0].cpu().numpy())))
        tail_tok = [int(t) for t in synth.prompt_tokens(32, 3)]
        tail = []
        for t in tail_tok:
            o = eng.decode([1], tokens=dev_tokens(torch, [t]), logits=True, argmax=True)
            tail.append(o["logits"][0].cpu().numpy().astype(np.float64))
        torch.cuda.synchronize()
        for s in range(4):
            eng.reset(s)
        assert eng.free_pages() == free0
    finally:
        eng.close()

    orc = Oracle(cfg, blob)
    orc.preload(16)
    try:
        ref_plain = oracle_teacher_forced(orc, prompt, plain[:20])
        margins = top2_margin(ref_plain)
        n = min(len(gen), len(plain))
        for i in range(n):
            if margins[i] < MARGIN:
                print(f"near-tie at generated position {i}: ids compared up to it")
                break
            assert gen[i] == plain[i], (i, gen[:n], plain[:n])
        print(f"drafted ids {gen[:n]}\nplain ids   {plain[:n]}")
        st = orc.new_slot()
        orc.forward(st, tokens=prompt, logits=None)
        for win, a, lg, am in windows:
            tmp = st.copy()
            want = orc.forward(tmp, tokens=win, logits="all")["logits"]
            compare_logits(lg, am, want, f"verify window {win} (accepted {a})")
            orc.forward(st, tokens=win[:a], logits=None)
        orc.forward(st, tokens=[gen[-2]], logits=None)       # the last window: one accepted row
        want = np.stack([orc.forward(st, tokens=[t], logits="last")["logits"][0] for t in tail_tok])
        compare_logits(np.stack(tail), [int(np.argmax(x)) for x in tail], want, "plain steps after the windows")
    finally:
        orc.drop_cache()
