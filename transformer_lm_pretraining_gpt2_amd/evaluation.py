"""Validation readouts of a language model's loss ("A small GPT that writes
fairy tales": the training log's val_loss / val_bpb columns and Problem 3).

The loss is the mean cross-entropy in nats per token.  Perplexity per token is
e^loss.  Bits per byte removes the tokenizer: loss / ln 2 gives bits per token,
divided by the average number of text bytes one token covers.
"""
import math


def perplexity(loss):
    return math.exp(loss)


def bits_per_byte(loss, bytes_per_token):
    if bytes_per_token <= 0:
        raise ValueError("bytes_per_token must be positive")
    return loss / math.log(2.0) / bytes_per_token


def bytes_per_token(loss, bpb):
    """The tokenizer's average bytes per token implied by a loss and its bits per byte."""
    if bpb <= 0:
        raise ValueError("bits per byte must be positive")
    return loss / math.log(2.0) / bpb


def val_loss(step, batches, loss_buf):
    """Mean loss over validation micro-batches [(ids, targets), ...] (equal sizes,
    device int32 tensors) with the forward-only path; loss_buf is a device fp32
    [1] scratch tensor.  Each batch's mean is read back and averaged on the host
    in float64, so every batch weighs the same."""
    total = 0.0
    for ids, tgt in batches:
        step.evaluate(ids, tgt, loss_buf)
        total += float(loss_buf.item())
    return total / max(len(batches), 1)


def readout(loss, bytes_per_token_):
    """The three numbers of an eval line: loss, bits per byte, perplexity."""
    return {"val_loss": loss, "val_bpb": bits_per_byte(loss, bytes_per_token_), "perplexity": perplexity(loss)}


__all__ = ["perplexity", "bits_per_byte", "bytes_per_token", "val_loss", "readout"]
