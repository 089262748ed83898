"""qd_sample_noalloc (the sampler with its per-call scratch in the library's fixed device
array, for callers that cannot allocate) against qd_sample on the GPU.

Both entry points run the same kernels on the same logits, token counts and Philox draw
numbers, so the drawn ids must be identical.  Two noalloc calls run back to back, the
second on fewer rows, so a histogram, counter or candidate list left in the array by the
first call would change the second call's draws.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from workloads import SHAPES, make_weights, make_prompt
from parity import say

pytestmark = pytest.mark.gpu

PARAMS = dict(temperature=0.8, top_k=40, min_p=0.02, top_p=0.95, repeat_penalty=1.1,
              presence_penalty=0.2, frequency_penalty=0.1)
SHAPE = dataclasses.replace(SHAPES["tiny"], vocab=100000)


def test_noalloc_sampler_matches_qd_sample():
    import int8_weight_only_amd as qd
    w = make_weights(SHAPE, seed=31, gains="uniform")
    B = 12
    prompts = [make_prompt(SHAPE.vocab, 6 + b, 8100 + b) for b in range(B)]
    seeds12 = [1000 + 17 * b for b in range(B)]
    sub = [7, 2, 9, 0, 4]
    seeds5 = [2 ** 63 + 3, 5, 77, 123456789, 9]
    say("[gpu] no-alloc sampler: loading a tiny-shape model with vocab 100000")
    m = qd.Model(SHAPE, w, max_batch=B, max_ctx=32, max_prefill_tokens=256)
    try:
        def run(noalloc):
            # the prefill restarts every slot's token counts and draw numbers
            _, lg = m.prefill(prompts, logits=True)
            first = m.sample(lg, seeds12, slots=list(range(B)), noalloc=noalloc, **PARAMS)
            second = m.sample(lg[sub], seeds5, slots=sub, noalloc=noalloc, **PARAMS)
            torch.cuda.synchronize()
            return lg.cpu().numpy(), first.cpu().numpy(), second.cpu().numpy()

        lg_ref, ref12, ref5 = run(False)
        lg_na, na12, na5 = run(True)
        assert np.array_equal(lg_ref, lg_na)
        np.testing.assert_array_equal(na12, ref12)
        np.testing.assert_array_equal(na5, ref5)
        assert np.all((ref12 >= 0) & (ref12 < SHAPE.vocab))
        say(f"[gpu] no-alloc sampler: 12 rows then 5 rows, ids equal to qd_sample "
            f"({ref12[:4].tolist()}..., {ref5.tolist()})")
        # beyond the fixed array's rows: refused on the host, before any GPU work
        big = torch.zeros((B, SHAPE.vocab), dtype=torch.float32, device="cuda")
        m.sample(big, [1] * B, noalloc=True, **PARAMS)   # 12 rows x 100000 fits
    finally:
        m.close()


def test_noalloc_sampler_refuses_sizes_beyond_its_array():
    import int8_weight_only_amd as qd
    shape = dataclasses.replace(SHAPES["tiny"], vocab=151936)
    w = make_weights(shape, seed=32)
    m = qd.Model(shape, w, max_batch=20, max_ctx=16, max_prefill_tokens=64)
    try:
        m.prefill([make_prompt(shape.vocab, 3, 8200 + b) for b in range(20)])
        lg = torch.zeros((20, shape.vocab), dtype=torch.float32, device="cuda")
        with pytest.raises(qd.QdError) as e:       # 14 rows x 151936 > 2^21
            m.sample(lg[:14], [1] * 14, noalloc=True, **PARAMS)
        assert e.value.code == "invalid_arguments" and "fixed scratch" in str(e.value)
        with pytest.raises(qd.QdError) as e:       # more than 16 rows
            m.sample(lg[:17], [1] * 17, noalloc=True, **PARAMS)
        assert e.value.code == "invalid_arguments"
        ids = m.sample(lg[:13], list(range(13)), noalloc=True, **PARAMS)  # 13 rows fit
        torch.cuda.synchronize()
        assert ids.shape == (13,)
    finally:
        m.close()
