"""The library's fp64 exponential, pinned directly.

Every accept test and draw of the acceptance walk compares probabilities
P_u(x) = exp(p_u(x)/T - lse) (CSDN page "推理加速：推测解码与级联推理",
section 7.1) that the library evaluates with its own table-driven fp64
exponential.  Here it runs through spec_test_exp_f64 on a dense grid over
[-745, 709], on table boundaries k ln2/256 (every 7th k, which meets every
one of the 256 table entries) with their neighbours and midpoints, and on
values around the -708 guard, against exp in x86 extended precision (64-bit
mantissa, then rounded to double -- numpy's own float64 exp does not enter
the bound).

Stated bounds (measured on MI355X: at most 1.0 ulp, mean 0.27 ulp, over
4.2 million points):
* exp_f64 on [-708, 709]: within 2 ulp of the reference (the table entry
  and the final fused multiply-add each round once, the degree-4 Taylor
  term leaves below 4e-17 relative); exactly 0 below -708;
* exp_f64_clamped: bit-identical to exp_f64 at and above -708, and to
  exp_f64_stream(-708) below it;
* exp_f64_stream on [-745, -708): within 2 units of the smallest subnormal
  of the reference (the scaling into the subnormal range rounds once more).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from parity import log  # noqa: E402

ULP_BOUND = 2.0


@pytest.fixture(scope="module")
def lib():
    import tree_attention_verification_02_amd._lib as L
    return L


def _run(L, x, variant):
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to("cuda")
    yd = torch.empty_like(xd)
    L.spec_test_exp_f64(xd, yd, variant)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def _reference(x):
    assert np.finfo(np.longdouble).nmant >= 63, "needs x86 extended precision"
    return np.exp(np.asarray(x, dtype=np.longdouble)).astype(np.float64)


def _grid():
    rng = np.random.default_rng(11)
    dense = np.linspace(-745.0, 709.0, 3_000_001)
    ln2_256 = np.log(2.0) / 256
    k = np.arange(int(np.ceil(-708 / ln2_256)), int(np.floor(709 / ln2_256)) + 1, 7)
    edges = (k * ln2_256).astype(np.float64)
    near = np.concatenate([edges, np.nextafter(edges, np.inf), np.nextafter(edges, -np.inf),
                           edges + ln2_256 / 2])           # half-way between table points
    logits = rng.standard_normal(1_000_000) * 3.0 - 16.0  # like p/T - lse of the workloads
    special = np.array([0.0, -0.0, 5e-324, -5e-324, 1e-300, -1e-300, 1e-17, -1e-17, 1.0, -1.0,
                        -708.0, np.nextafter(-708.0, 0.0), 709.0, -707.5, -700.0])
    return np.concatenate([dense, near, logits, special])


def test_exp_f64_within_two_ulp_and_zero_below_guard(lib):
    x = _grid()
    y = _run(lib, x, 0)
    ref = _reference(x)
    inside = x >= -708.0
    err = np.abs(y[inside] - ref[inside]) / np.spacing(ref[inside])
    worst = float(err.max())
    log(f"[exp64] exp_f64 on {int(inside.sum())} points in [-708, 709]: max {worst:.3f} ulp, "
        f"mean {float(err.mean()):.3f} ulp, {int((err > 0.5).sum())} beyond half an ulp")
    assert worst <= ULP_BOUND, (worst, x[inside][np.argmax(err)])
    assert (y[~inside] == 0.0).all() and not np.signbit(y[~inside]).any()
    assert y[x == 0.0][0] == 1.0


def test_clamped_and_stream_variants(lib):
    x = _grid()
    y0 = _run(lib, x, 0)
    y1 = _run(lib, x, 1)
    y2 = _run(lib, x, 2)
    at_guard = _run(lib, np.array([-708.0]), 2)[0]
    inside = x >= -708.0
    assert np.array_equal(y1[inside].view(np.uint64), y0[inside].view(np.uint64))
    assert (y1[~inside] == at_guard).all() and at_guard > 0.0
    assert abs(at_guard - _reference([-708.0])[0]) <= ULP_BOUND * np.spacing(at_guard)
    assert np.array_equal(y2[inside].view(np.uint64), y0[inside].view(np.uint64))
    below = x < -708.0
    sub = np.abs(y2[below] - _reference(x[below]))
    tiny = 5e-324
    log(f"[exp64] exp_f64_stream on {int(below.sum())} points in [-745, -708): "
        f"max error {float(sub.max() / tiny):.1f} x the smallest subnormal")
    assert (sub <= ULP_BOUND * tiny + ULP_BOUND * np.spacing(_reference(x[below]))).all()


def test_paired_evaluation_is_bit_identical(lib):
    """The walk's and the statistics' sums evaluate their exponentials two at
    a time (both table reads issued first); that must not change a bit.  The
    grid is shuffled so pairs mix arguments from far apart, and has odd
    length so the last element is paired with itself."""
    x = _grid()
    x = np.random.default_rng(5).permutation(x)[: (len(x) // 2) * 2 - 1]
    y0 = _run(lib, x, 0)
    y1 = _run(lib, x, 1)
    y3 = _run(lib, x, 3)
    y4 = _run(lib, x, 4)
    assert np.array_equal(y3.view(np.uint64), y0.view(np.uint64))
    assert np.array_equal(y4.view(np.uint64), y1.view(np.uint64))
