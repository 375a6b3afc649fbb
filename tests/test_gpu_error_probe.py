"""The error-accumulation probe on the GPU (kv_cache_bit_token_amd.error_probe):
the paged KVarN cache (append by kvarn_quantize_tiles_to, attention by
kvarn_decode_attention_paged) against the fp16 cache
(kvarn_decode_attention_fp16) and naive per-token RTN, over 320 steps of the
feedback token stream.  The same qualitative relations as the oracle's run
(tests/test_oracle_error_probe.py) must hold."""
import numpy as np
import pytest

from kv_cache_bit_token_amd import error_probe

pytestmark = pytest.mark.gpu


def test_gpu_probe_kvarn_below_naive():
    err = error_probe.run_probe(steps=320)
    for e in err.values():
        assert np.isfinite(e).all()
    # the tail-only steps read fp16 through another kernel: equal up to fp32 rounding
    assert err["kvarn_forced"][:127].max() <= 1e-4
    assert err["kvarn_forced"].mean() < 0.5 * err["naive_forced"].mean()
    assert err["kvarn_free"][-64:].mean() < 0.5 * err["naive_free"][-64:].mean()
    print(error_probe.summarise(err, 64))
