"""GPU parity of the dense GEMV (sk_gemv) over every supported width, against its plain
definition in fp64: y[r] = W[r] . x' (+ residual[r]), x' = x or RMSNorm(x) * gamma, and
with the SwiGLU epilogue y[r] = SiLU(W[r] . x') * (W[rows + r] . x').

Row counts cover a ragged grid (fewer rows than one workgroup's waves), more rows than
the grid has waves (each wave then walks several rows, through the two-row register ring
or, for wide rows, one row at a time), the residual given, absent and aliasing y, and a
gate that skips the launch.

Tolerance (fp32 arithmetic, first order in u = 2^-24): each lane sums 8 J products in
sequence and the wave adds 64 lane sums in 6 levels, so the dot product is off by at most
(8 J + 6) u sum|w x'|; the RMSNorm scale comes from a sum of squares over J values per
thread, 6 wave levels and 8 waves in sequence, a square root and a reciprocal, which puts
x' within ((J + 14) / 2 + 5) u of exact. Together: (9 J + 20) u sum|w x'|, plus one
rounding of the result (and a few of SiLU's exponential) relative to |y|."""

import numpy as np
import pytest

from tests.helpers import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

U = 2.0 ** -24
WIDTHS = (1, 2, 3, 4, 6, 8, 12, 16)  # cols = 512 J


def _definition(W, x, rows, rmsnorm, gamma, eps, residual, swiglu):
    """fp64 value and error bound of every output row."""
    W = W.astype(np.float64)
    x = x.astype(np.float64)
    if rmsnorm:
        x = x / np.sqrt(np.mean(x * x) + eps) * gamma.astype(np.float64)
    a = W @ x
    mag = np.abs(W) @ np.abs(x)
    J = W.shape[1] // 512
    tol = (9 * J + 20) * U
    if swiglu:
        a0, a1 = a[:rows], a[rows:]
        d0, d1 = tol * mag[:rows], tol * mag[rows:]
        s = a0 / (1.0 + np.exp(-a0))
        y = s * a1
        return y, 1.1 * d0 * (np.abs(a1) + d1) + np.abs(s) * d1 + 8 * U * np.abs(y)
    y = a + (0.0 if residual is None else residual.astype(np.float64))
    return y, tol * mag + 2 * U * np.abs(y) + (0.0 if residual is None else U * np.abs(residual))


CASES = [  # (rows, rmsnorm, swiglu, residual: None | "vec" | "alias")
    (37, True, False, "vec"),
    (4100, False, False, "alias"),
    (4100, True, False, None),
    (29, False, True, None),
    (4099, True, True, None),
]


@pytest.mark.parametrize("J", WIDTHS)
def test_gemv_every_width(J):
    import torch
    from sparse_kv_recall_amd import ops
    cols = 512 * J
    g = torch.Generator().manual_seed(1000 + J)
    for rows, rmsnorm, swiglu, res in CASES:
        wrows = 2 * rows if swiglu else rows
        W = (torch.randn(wrows, cols, generator=g) * 0.03).to(torch.bfloat16)
        x = torch.randn(cols, generator=g) * 1.7
        gamma = (1.0 + 0.2 * torch.randn(cols, generator=g)).to(torch.bfloat16)
        resid = torch.randn(rows, generator=g) if res else None
        ref, bound = _definition(W.float().numpy(), x.numpy(), rows, rmsnorm, gamma.float().numpy(), 1e-6,
                                 None if resid is None else resid.numpy(), swiglu)
        Wd, xd = W.cuda(), x.cuda()
        y = torch.full((rows,), float("nan"), device="cuda")
        r = None
        if res == "vec":
            r = resid.cuda()
        elif res == "alias":  # y = W x + y, as the model's residual adds are
            y.copy_(resid)
            r = y
        ops.gemv(Wd, xd, y, prologue=ops.PRO_RMSNORM if rmsnorm else ops.PRO_NONE,
                 gamma=gamma.cuda() if rmsnorm else None, eps=1e-6, residual=r,
                 epilogue=ops.EPI_SWIGLU if swiglu else ops.EPI_STORE)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        what = "J=%d rows=%d rmsnorm=%s swiglu=%s residual=%s" % (J, rows, rmsnorm, swiglu, res)
        assert np.isfinite(got).all(), what
        assert (err <= bound).all(), (what, float(err.max()), float((err / bound).max()))


def test_gemv_gate():
    # a launch whose selector does not match leaves y untouched; a matching one computes
    import torch
    from sparse_kv_recall_amd import ops
    g = torch.Generator().manual_seed(7)
    W = (torch.randn(300, 2048, generator=g) * 0.03).to(torch.bfloat16).cuda()
    x = torch.randn(2048, generator=g).cuda()
    sel = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.full((300,), 5.0, device="cuda")
    ops.gemv(W, x, y, sel=sel, sel_value=1)
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
    sel.fill_(1)
    ops.gemv(W, x, y, sel=sel, sel_value=1)
    ref = W.float() @ x
    torch.cuda.synchronize()
    assert float((y - ref).abs().max()) <= 1e-4 * float(ref.abs().max())
