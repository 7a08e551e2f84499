"""Expected tokens per speculative decoding step with MTP drafts -- TEST
INFRASTRUCTURE ONLY.

Source: "Читаем техотчёт DeepSeek-V3 вместе" (ai.flicky.cc course lesson),
section 2.2 "Multi-Token Prediction" (second-token acceptance of 85-90%,
about 1.8x generation speed), the `tokens_per_step` exercise of its practice
part, quiz item 5 and the lesson summary (about 1.85 tokens per step at depth
1 and acceptance 0.85).

Model, as read here: a verify step always keeps the main model's token; the
drafts form a chain, and a drafted token is kept only while every draft
before it was kept, each draft being kept independently with probability
`acceptance`.

The function below is the expectation written out over every accept/reject
outcome of the drafts (2^depth of them), not a closed form.  Pins in the test
suite: the printed 1.85 (depth 1, acceptance 0.85) and 1.9 (0.90), the limits
acceptance 0 -> 1 and acceptance 1 -> 1 + depth, and the geometric series,
which a different derivation gives.
"""
import itertools


def tokens_per_step(acceptance, depth=1):
    """Mean number of tokens one verify step emits: 1 from the main model plus
    the drafts up to (not including) the first rejected one."""
    a = float(acceptance)
    if not (0.0 <= a <= 1.0) or depth < 0:
        raise ValueError("acceptance in [0, 1] and depth >= 0")
    mean = 0.0
    for outcome in itertools.product((True, False), repeat=depth):  # True: draft k accepted
        p = 1.0
        for ok in outcome:
            p *= a if ok else (1.0 - a)
        emitted = 1
        for ok in outcome:
            if not ok:
                break
            emitted += 1
        mean += p * emitted
    return mean
