"""Helpers that turn the page fixtures under tests/golden into arrays."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def tok(fx, x):
    """Token id of a fixture symbol (ints pass through)."""
    if isinstance(x, int):
        return x
    return int(fx["tokens"][x])


def draft_lists(fx):
    """(scores [1, ncand] f32, tokens [1, ncand] i32, parents [1, npar] i32, bonus [1])."""
    scores = np.array([fx["scores"]], np.float32)
    tokens = np.array([[tok(fx, t) for t in fx["cand_tokens"]]], np.int32)
    parents = np.array([fx["parents"]], np.int32)
    bonus = np.array([tok(fx, fx["bonus"])], np.int32)
    return scores, tokens, parents, bonus


def vocab_size(fx):
    ids = [v for v in fx.get("tokens", {}).values()] + [0]
    return max(ids) + 1


def onehot_logits(fx, names, vocab):
    """f32 logits whose argmax per row is the named token."""
    x = np.zeros((len(names), vocab), np.float32)
    for r, t in enumerate(names):
        x[r, tok(fx, t)] = 1.0
    return x
