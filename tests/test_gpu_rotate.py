"""GPU parity of the KV path's Haar rotation (gist.science explainer of
HyperQuant, Methodology section 4, "Bias Correction for KV Cache"): the
rotation kernel against the oracle's ascending fma chains, bit-exact, and the
rotated, dithered KV codec end to end (stream and reconstruction)."""
import numpy as np
import pytest
import torch

import oracle
from hq_testutil import rate_c
from kv_cache_tile_amd import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from kv_cache_tile_amd import hq
    hq.lib()                        # no fallback: a missing library fails every test


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def _bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy().view(np.uint32)


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("xdt,ydt", [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("d,rows", [(128, 1), (128, 127), (128, 300), (64, 255), (64, 513)])
def test_rotation_matches_the_oracle(d, rows, xdt, ydt, transpose):
    dev = _dev()
    Q = workloads.haar_orthogonal(d, rows)
    x = workloads.gaussian(rows, d, key=rows + d)
    xt = torch.from_numpy(x)
    if xdt == "bf16":
        xt = xt.to(torch.bfloat16)
        xo = workloads.bf16_bits(xt)
    else:
        xo = x
    print(f"[case] rotate d={d} rows={rows} {xdt}->{ydt} transpose={transpose}", flush=True)
    y = hq.rotate(torch.from_numpy(Q).to(dev), xt.to(dev), transpose=transpose,
                  out_dtype=torch.bfloat16 if ydt == "bf16" else torch.float32)
    ref = oracle.rotate(Q, xo, transpose=transpose, out_dtype=oracle.BF16 if ydt == "bf16" else oracle.F32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(y).reshape(-1), ref.reshape(-1).view(np.uint16 if ydt == "bf16" else np.uint32))


def test_rotation_many_blocks():
    # more row blocks than the grid holds workgroups: the persistent loop and
    # a ragged last block
    dev = _dev()
    Q = workloads.haar_orthogonal(128, 9)
    rows = 128 * 300 + 77
    x = workloads.gaussian(rows, 128, key=9)
    print(f"[case] rotate d=128 rows={rows}", flush=True)
    y = hq.rotate(torch.from_numpy(Q).to(dev), torch.from_numpy(x).to(dev))
    ref = oracle.rotate(Q, x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(y).reshape(-1), ref.reshape(-1).view(np.uint32))


@pytest.mark.parametrize("d,bps", [(128, 2.0), (64, 2.5)])
def test_haar_kv_end_to_end(d, bps):
    dev = _dev()
    tokens = 64 * 3 + 5
    Q = workloads.haar_orthogonal(d, 100 + d)
    k = workloads.kv_cache(1, 2, tokens // 2 + 1, d, key=4, which="K").reshape(-1, d)[:tokens]
    kt = torch.from_numpy(np.ascontiguousarray(k)).to(torch.bfloat16)
    ko = workloads.bf16_bits(kt)
    print(f"[case] haar kv d={d} bps={bps} tokens={tokens}", flush=True)
    h = hq.kv_encode_haar(kt.to(dev), torch.from_numpy(Q).to(dev), "E8", bps, seed=31)
    xh = hq.kv_decode_haar(h)
    torch.cuda.synchronize()
    # oracle: rotate (fp32), dithered KV codec, inverse rotation to bf16
    y = oracle.rotate(Q, ko)
    c = rate_c("E8", d, bps, 1)
    e = oracle.encode(y, d, "E8", c, 31, 1)
    np.testing.assert_array_equal(h.step.cpu().numpy().view(np.uint16), e.step)
    np.testing.assert_array_equal(h.meta.cpu().numpy().view(np.uint16), e.meta)
    np.testing.assert_array_equal(h.payload[:h.payload_words()].cpu().numpy().view(np.uint32), e.payload)
    yh, st = oracle.decode(e, tokens, d, d, "E8", c, 31, oracle.F32, 1)
    assert st == oracle.OK and h.flags() == 0
    ref = oracle.rotate(Q, yh, transpose=True, out_dtype=oracle.BF16)
    np.testing.assert_array_equal(_bits(xh).reshape(-1), ref.reshape(-1))
