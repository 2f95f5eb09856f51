"""The GEMV parity gate of the GPU tests, against the fp64 oracle on the same inputs.

rel_l2 (whole [B][M] output) <= 1e-3 is the bar for fp32 accumulation of bf16
activations; worst_row (the largest single output error relative to the RMS of
its output row) <= 1e-3 keeps one wrong row (a wrong scale group, a misrouted
tile) from hiding in the whole-output norm, which divides it by sqrt(M)."""
from oracle import gemv

TOL = 1e-3
ROW_TOL = 1e-3


def check(y, ref, what="", tol=TOL, row_tol=ROW_TOL):
    rel, worst = gemv.rel_l2(y, ref), gemv.worst_row(y, ref)
    assert rel <= tol and worst <= row_tol, "%s rel_l2=%.3e worst_row=%.3e" % (what, rel, worst)
    return rel, worst
