"""The error-accumulation probe, run on the oracle (qualitative pins).

Pages: digest page (ai-feeds.com), title and "方法" (errors of a quantised
cache accumulate over long autoregressive decodes; KVarN is built to keep
them down); deep-dive page (vatt-ghern.pages.dev), the section on why naive
2-bit quantisation degrades long decodes.  The probe's GPU form is
kv_cache_bit_token_amd.error_probe; this is the same loop with the oracle's
quantiser and attention, on the same synthetic.FeedbackSource tokens.

Pins: before the first page fills, the KVarN cache is read as its fp16 tail,
so its output equals the fp16 cache's exactly; KVarN's per-step
(teacher-forced) error and its free-running divergence stay below naive
per-token RTN's on the outlier-structured stream.
"""
import numpy as np

from kv_cache_bit_token_amd.synthetic import FeedbackSource
from probe_oracle import D0, HQ, _Fp16, _Kvarn


def test_probe_on_oracle_kvarn_below_naive():
    steps = 320
    src = FeedbackSource(0, D0, HQ)
    ref = _Fp16(steps)
    runs = {"kvarn_forced": _Kvarn(), "naive_forced": _Fp16(steps, (4, 2)),
            "kvarn_free": _Kvarn(), "naive_free": _Fp16(steps, (4, 2))}
    err = {n: np.zeros(steps) for n in runs}
    prev = {"ref": None, "kvarn_free": None, "naive_free": None}
    for t in range(steps):
        q, k, v = src.token(t, prev["ref"])
        ref.append(k, v)
        o_ref = ref.attend(q)
        outs = {}
        for n in ("kvarn_forced", "naive_forced"):
            runs[n].append(k, v)
            outs[n] = runs[n].attend(q)
        for n in ("kvarn_free", "naive_free"):
            qf, kf, vf = src.token(t, prev[n])
            runs[n].append(kf, vf)
            outs[n] = prev[n] = runs[n].attend(qf)
        for n in runs:
            err[n][t] = np.linalg.norm(outs[n] - o_ref) / np.linalg.norm(o_ref)
        prev["ref"] = o_ref
    # the first 127 steps read only the fp16 tail: identical to the fp16 cache
    assert np.array_equal(err["kvarn_forced"][:127], np.zeros(127))
    assert np.array_equal(err["kvarn_free"][:127], np.zeros(127))
    assert err["kvarn_forced"].mean() < 0.5 * err["naive_forced"].mean()
    assert err["kvarn_free"][-64:].mean() < 0.5 * err["naive_free"][-64:].mean()


def test_feedback_source_steps_are_order_independent():
    a, b = FeedbackSource(3, 64, 2), FeedbackSource(3, 64, 2)
    for t in (0, 7, 3):
        a.token(t)
    o = np.ones((2, 64))
    for x, y in zip(a.token(5, o), b.token(5, o)):
        assert np.array_equal(x, y)
    # the previous output enters the next token
    assert not np.array_equal(a.token(5, o)[1], a.token(5, None)[1])
