"""Validation readouts (perplexity, bits per byte) pinned to the numbers the
fairy-tale page prints for its full validation text and its eval log."""
import json
import math
import os

import pytest

from transformer_lm_pretraining_gpt2_amd import evaluation

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))["eval_readout"]


def test_perplexity_of_the_full_validation_loss():
    fv = GOLD["full_val"]
    assert round(evaluation.perplexity(fv["loss"]), 2) == fv["perplexity_rounded"]


def test_bytes_per_token_from_loss_and_bpb():
    # the worked answer: 1.1685 / 0.6931 / 0.4253 = 3.96
    fv = GOLD["full_val"]
    assert round(evaluation.bytes_per_token(fv["loss"], fv["bpb"]), 2) == fv["bytes_per_token_rounded"]


def test_bpb_from_the_text_counts():
    # bytes / tokens of the validation text (3.967) reproduces the printed bpb to
    # 0.1 %: the page's own figures (rounded loss, its byte count) agree to that
    fv = GOLD["full_val"]
    bpt = fv["bytes"] / fv["tokens"]
    assert round(bpt, 2) == pytest.approx(fv["bytes_per_token_rounded"], abs=0.011)
    assert evaluation.bits_per_byte(fv["loss"], bpt) == pytest.approx(fv["bpb"], rel=1e-3)


def test_eval_log_rows_share_one_tokenizer():
    # every eval line (same tokenizer, same validation text) implies the same
    # bytes per token within the 4-decimal rounding of the log
    vals = [evaluation.bytes_per_token(loss, bpb) for _, loss, bpb in GOLD["eval_log"]]
    assert max(vals) - min(vals) < 0.02
    assert all(3.95 < v < 3.98 for v in vals)


def test_readout_inverts():
    r = evaluation.readout(2.0, 4.0)
    assert r["val_bpb"] == pytest.approx(2.0 / math.log(2.0) / 4.0)
    assert evaluation.bytes_per_token(r["val_loss"], r["val_bpb"]) == pytest.approx(4.0)
    assert r["perplexity"] == pytest.approx(math.e ** 2)
    with pytest.raises(ValueError):
        evaluation.bits_per_byte(1.0, 0.0)
