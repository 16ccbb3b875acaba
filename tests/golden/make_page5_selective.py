"""Writes page5_selective_example.json: the selective demo of the page '架构变体：Mamba/SSM'
(section 'Python 演示'), in which the write weight of every step is B_base times the logistic
function of that step's input, evaluated in 50-digit decimal arithmetic from the page's own
decimals. It uses only Python's decimal module (no oracle, no GPU library); the test re-derives
the same values and checks the oracle against them.

    python tests/golden/make_page5_selective.py
"""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 50
X = ["0.5", "-1.2", "0.8", "2.1", "-0.6", "1.3"]
A, B_BASE, C = Decimal("0.9"), Decimal("0.2"), Decimal("1.0")


def derive(xs):
    """B_t = B_base / (1 + e^{-x_t}); h_t = A h_{t-1} + B_t x_t from h = 0; y_t = C h_t."""
    b, y, h = [], [], Decimal(0)
    for s in xs:
        x = Decimal(s)
        bt = B_BASE / (1 + (-x).exp())
        h = A * h + bt * x
        b.append(bt)
        y.append(C * h)
    return b, y


def main():
    b, y = derive(X)
    out = {
        "source": ("Page '架构变体：Mamba/SSM' (aiqz.cc), section 'Python 演示': the selective demo scans "
                   "x = [0.5, -1.2, 0.8, 2.1, -0.6, 1.3] with A = 0.9, B_base = 0.2, C = 1.0 from h = 0, "
                   "the write weight of step t being B_base * sigmoid(x_t). The page prints no output "
                   "values; the B_t and y below are 50-digit decimal evaluations of that definition "
                   "(make_page5_selective.py), rounded to 30 significant digits."),
        "mapping": ("Through the S6 interface: batch = dim = dstate = 1, softplus off, delta = 1, "
                    "delta_bias absent, A = ln(0.9) so that exp(delta*A) = 0.9, the input B_t = "
                    "B_base * sigmoid(x_t) (selectivity computed by the caller, as the projections do), "
                    "C_t = 1.0, no D term, no gate."),
        "x": X, "A_decay": str(A), "B_base": str(B_BASE), "C": str(C),
        "B_t": [f"{v:.30g}" for v in b],
        "y": [f"{v:.30g}" for v in y],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "page5_selective_example.json")
    with open(path, "w") as f:
        json.dump(out, f, ensure_ascii=False, indent=2)
        f.write("\n")


if __name__ == "__main__":
    main()
