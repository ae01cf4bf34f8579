"""Tensors past 2^31 elements: every offset the kernels form must be 64-bit.

A problem of three batch elements whose tensors hold more than 2^31 elements
each (12.9 GB per fp32 tensor, 6.4 GB per bf16 one) is run forward and
backward; its last batch element, whose elements all sit past index 2^31, is
then run alone as a problem of one batch element (a copy of the same data).
The kernels treat batch elements independently and the gather backward has
no atomics, so the two results must agree bit for bit. The one-element
problem has the shape of the parity workloads scaled up; its own arithmetic
is covered by the oracle comparisons at the parity sizes.
"""
import pytest
import torch

from fwd_bwd_amd import na

pytestmark = pytest.mark.gpu

# (shape [B, (T,) H, W, heads, D], kernel, dtype): 3 * 2048^2 * 8 * 32 and
# 3 * 16 * 512^2 * 8 * 32 elements, both above 2^31; fp32 on the register-
# resident kernels, bf16 on the 16-bit MFMA kernels (several planes per tile)
CASES = [
    ((3, 2048, 2048, 8, 32), (9, 9), torch.float32),
    ((3, 16, 512, 512, 8, 32), (5, 7, 7), torch.bfloat16),
]


def say(*a):
    print(*a, flush=True)


def _run(q, k, v, dout, kernel):
    out, lse = na.na_fwd(q, k, v, kernel)
    dq, dk, dv = na.na_bwd(q, k, v, out, dout, lse, kernel)
    torch.cuda.synchronize()
    return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("case", CASES, ids=["2d_2048sq_k9_f32", "3d_16x512sq_k5x7x7_bf16"])
def test_last_batch_element_past_2_31_equals_it_alone(case):
    shape, kernel, dtype = case
    n = 1
    for s in shape:
        n *= s
    assert n > 2 ** 31
    say("case", shape, kernel, dtype, f"{n / 2 ** 31:.2f} x 2^31 elements per tensor")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q, k, v, dout = (torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(dtype)
                     for _ in range(4))
    full = _run(q, k, v, dout, kernel)
    say("full problem done")
    last = shape[0] - 1
    one = _run(*(t[last:].clone() for t in (q, k, v, dout)), kernel)
    say("last batch element alone done")
    for name in full:
        a, b = full[name][last:], one[name]
        assert torch.isfinite(b.float()).all(), name
        assert torch.equal(a, b), (name, float((a.float() - b.float()).abs().max()))
    del q, k, v, dout, full, one
    torch.cuda.empty_cache()


def test_unfused_ops_past_2_31_attention_entries():
    """The unfused ops on head-major tensors [1, 8, 2048, 2048, 32] fp32: the
    attention array holds 8 * 2048^2 * 81 > 2^31 entries, so the last head's
    rows sit past entry 2^31. Scores, softmax, weighted sum and inverse
    weighted sum of the last head must equal those of that head alone."""
    shape, kernel = (1, 8, 2048, 2048, 32), (9, 9)
    assert shape[1] * shape[2] * shape[3] * 81 > 2 ** 31
    say("unfused", shape, kernel)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    q, k, v = (torch.randn(shape, generator=g, device=dev) for _ in range(3))

    def ops(q, k, v):
        attn = na.na_softmax(na.na_qk(q, k, kernel, alpha=32 ** -0.5), kernel)
        out = na.na_av(attn, v, kernel)
        vin = na.na_av_inverse(attn, q, kernel)
        torch.cuda.synchronize()
        return {"attn": attn, "out": out, "inverse": vin}

    full = ops(q, k, v)
    one = ops(*(t[:, -1:].clone() for t in (q, k, v)))
    for name in full:
        a, b = full[name][:, -1:], one[name]
        assert torch.isfinite(b).all(), name
        assert torch.equal(a, b), (name, float((a - b).abs().max()))
    del q, k, v, full, one
    torch.cuda.empty_cache()
