"""The oracle's E4M3FN encoder against torch's float8_e4m3fn cast on every finite fp32 bit pattern
with |v| <= 448 (2 x 1,138,753,537 values, in chunks over the host's cores).

Torch's cast is an independent implementation of the same round-to-nearest-even rule; above 448
the two differ by design (torch gives NaN past 464, the recipe saturates), so that region is
checked against the closed form in test_oracle_fp8.py. OCP E4M3FN format; "官方揭秘DeepSeek-V3
模型训练全流程" §4.3 (E4M3 with online max-abs scaling).
"""
import multiprocessing as mp
import os

import numpy as np
import pytest

import oracle

TOP = 0x43E00000            # bit pattern of 448.0; every pattern below it is a smaller finite value
CHUNK = 1 << 24


def _check(args):
    import torch
    torch.set_num_threads(1)
    start, sign = args
    stop = min(start + CHUNK, TOP + 1)
    bits = np.arange(start, stop, dtype=np.uint32) | np.uint32(sign)
    v = bits.view(np.float32)
    ours = oracle.e4m3fn_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    return int(bad.size), [(int(bits[i]), int(ours[i]), int(ref[i])) for i in bad[:4]]


@pytest.mark.slow
def test_encoder_exhaustive_against_torch_cast():
    jobs = [(s, sign) for sign in (0, 0x80000000) for s in range(0, TOP + 1, CHUNK)]
    workers = max(1, min(8, os.cpu_count() or 1))
    with mp.get_context("fork").Pool(workers) as pool:
        results = pool.map(_check, jobs, chunksize=1)
    n_bad = sum(r[0] for r in results)
    examples = [e for r in results for e in r[1]][:8]
    assert n_bad == 0, f"{n_bad} mismatches, e.g. (bits, oracle, torch) {examples}"
    assert sum(min(CHUNK, TOP + 1 - s) for s, _ in jobs) == 2 * (TOP + 1)
