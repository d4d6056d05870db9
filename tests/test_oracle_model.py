"""Model-level pins of the float64 oracle on the seeded three-layer slice (CPU only).

- Prompt prefill equals one-row decode at every cut point ("TensorFold PR #1508", earlier head:
  prompt == one-row decode at 32/32 cut points; "LFM3-1.7B port", "Chunked prefill").
- Negative controls the pages ran must move the output ("LFM3-1.7B port": dropping the gate,
  rotating every dimension and removing the window turn the gate red; with the conv state not
  written back the logits move) and the window control must not move anything under 256 tokens.
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Oracle


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.fixture(scope="module")
def rows300(slice3):
    cfg, _ = slice3
    return synth.bf16_bits_to_f32(synth.hidden_rows(2, 300)).astype(np.float64)


@pytest.fixture(scope="module")
def whole300(slice3_oracle, rows300):
    st = slice3_oracle.new_slot()
    return slice3_oracle.forward(st, hidden=rows300, capture=True)


def test_prefill_equals_chunked_at_cut_points(slice3_oracle, rows300, whole300):
    orc = slice3_oracle
    x = rows300[:80]
    st = orc.new_slot()
    ref80 = orc.forward(st, hidden=x, capture=True)
    for cut in [1, 5, 6, 7, 31, 63, 64, 79]:
        st = orc.new_slot()
        a = orc.forward(st, hidden=x[:cut], capture=True)
        b = orc.forward(st, hidden=x[cut:], capture=True)
        for li in range(3):
            got = np.concatenate([a["layers"][li], b["layers"][li]])
            assert _rel(got, ref80["layers"][li]) < 1e-12
    # and the 80-row run is the prefix of the 300-row run
    assert _rel(ref80["final"], whole300["final"][:80]) < 1e-12


def test_prefill_equals_one_row_decode(slice3_oracle, rows300):
    """64 prompt rows then 16 one-row steps == one 80-row prefill."""
    orc = slice3_oracle
    x = rows300[:80]
    st = orc.new_slot()
    ref80 = orc.forward(st, hidden=x)
    st = orc.new_slot()
    orc.forward(st, hidden=x[:64])
    outs = [orc.forward(st, hidden=x[r:r + 1])["final"] for r in range(64, 80)]
    assert _rel(np.concatenate(outs), ref80["final"][64:]) < 1e-12
    assert st.length == 80


def test_cut_points_across_the_window(slice3_oracle, rows300, whole300):
    """Chunks that straddle the 256-token seam reproduce the single pass."""
    orc = slice3_oracle
    for cut in [250, 256, 257]:
        st = orc.new_slot()
        a = orc.forward(st, hidden=rows300[:cut])
        b = orc.forward(st, hidden=rows300[cut:])
        got = np.concatenate([a["final"], b["final"]])
        assert _rel(got, whole300["final"]) < 1e-12


@pytest.mark.parametrize("control", ["no_gate", "rotate_all", "no_window"])
def test_negative_controls_move_the_output(slice3, rows300, whole300, control):
    cfg, blob = slice3
    orc = Oracle(cfg, blob, controls=(control,))
    st = orc.new_slot()
    out = orc.forward(st, hidden=rows300)
    d = _rel(out["final"][-40:], whole300["final"][-40:])
    assert d > 1e-3, (control, d)
    if control == "no_window":
        # under 256 tokens the window never bites
        assert _rel(out["final"][:256], whole300["final"][:256]) < 1e-14


def test_conv_state_not_written_back_moves_the_output(slice3, rows300, whole300):
    cfg, blob = slice3
    orc = Oracle(cfg, blob, controls=("no_conv_state",))
    st = orc.new_slot()
    orc.forward(st, hidden=rows300[:100])
    out = orc.forward(st, hidden=rows300[100:110])
    assert _rel(out["final"], whole300["final"][100:110]) > 1e-3


def test_storage_points_stay_close(slice3, rows300, whole300):
    """The fp16-storage diagnostic mode stays well within the per-layer rel-L2 bar of float64."""
    cfg, blob = slice3
    orc = Oracle(cfg, blob, storage_points=True)
    st = orc.new_slot()
    out = orc.forward(st, hidden=rows300[:80], capture=True)
    for li in range(3):
        assert _rel(out["layers"][li], whole300["layers"][li][:80]) < 2e-3
