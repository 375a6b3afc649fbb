"""The error-accumulation probe on the GPU (kv_cache_bit_token_amd.error_probe):
the paged KVarN cache (append by kvarn_quantize_tiles_to, attention by
kvarn_decode_attention_paged) against the fp16 cache
(kvarn_decode_attention_fp16) and naive per-token RTN, over 320 steps of the
feedback token stream.

Against the oracle: the teacher-forced stream the GPU run saw (the reference
trajectory's tokens) is replayed through the oracle's fp16 and paged KVarN
caches (tests/probe_oracle.py); the per-step KVarN errors must agree with the
GPU's, step by step and in window means.  The qualitative relations of the
oracle's own run (tests/test_oracle_error_probe.py) must hold too."""
import numpy as np
import pytest

from kv_cache_bit_token_amd import error_probe
from parity import record
from probe_oracle import _Fp16, _Kvarn

pytestmark = pytest.mark.gpu

STEPS = 320


def test_gpu_probe_kvarn_below_naive_and_matches_oracle():
    trace = []
    err = error_probe.run_probe(steps=STEPS, trace=trace)
    for e in err.values():
        assert np.isfinite(e).all()
    # the tail-only steps read fp16 through another kernel: equal up to fp32 rounding
    assert err["kvarn_forced"][:127].max() <= 1e-4
    assert err["kvarn_forced"].mean() < 0.5 * err["naive_forced"].mean()
    assert err["kvarn_free"][-64:].mean() < 0.5 * err["naive_free"][-64:].mean()

    # replay the teacher-forced stream on the oracle
    ref, kvc = _Fp16(STEPS), _Kvarn()
    e_or = np.zeros(STEPS)
    out_diff = 0.0
    for t, s in enumerate(trace):
        ref.append(s["k"], s["v"])
        kvc.append(s["k"], s["v"])
        o_ref = ref.attend(s["q"])
        o_kv = kvc.attend(s["q"])
        e_or[t] = np.linalg.norm(o_kv - o_ref) / np.linalg.norm(o_ref)
        out_diff = max(out_diff, float(np.abs(s["kvarn"] - o_kv).max()))
    e_gpu = err["kvarn_forced"]
    windows = {"first_64": slice(128, 192), "last_64": slice(STEPS - 64, STEPS),
               "all_paged": slice(128, STEPS)}
    rel = {n: abs(e_gpu[w].mean() - e_or[w].mean()) / e_or[w].mean() for n, w in windows.items()}
    stats = {"gpu_mean": float(e_gpu[128:].mean()), "oracle_mean": float(e_or[128:].mean()),
             "window_mean_rel_diff": max(rel.values()),
             "max_step_abs_diff": float(np.abs(e_gpu - e_or).max()),
             "max_output_abs_diff": out_diff}
    record("error probe, teacher-forced KVarN, GPU vs oracle (%d steps)" % STEPS, stats)
    assert np.all(e_or[:127] == 0.0)
    assert stats["window_mean_rel_diff"] <= 0.05, stats
    print(error_probe.summarise(err, 64), stats)
