"""Write gelu_tanh.json: the tanh approximation of GELU, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
(Hendrycks & Gimpel, "Gaussian Error Linear Units", 2016), evaluated in 40-digit decimal arithmetic
with tanh(u) = (e^{2u} - 1) / (e^{2u} + 1). Uses nothing but the standard library's decimal module.

    python tests/golden/make_gelu_tanh.py
"""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 40
PI = Decimal("3.141592653589793238462643383279502884197")
ZS = ["-3", "-1.5", "-0.5", "0.25", "1", "2", "3.5"]


def gelu_tanh(z: Decimal) -> Decimal:
    c = (Decimal(2) / PI).sqrt()
    u = c * (z + Decimal("0.044715") * z ** 3)
    e = (2 * u).exp()
    return Decimal("0.5") * z * (1 + (e - 1) / (e + 1))


def main():
    vals = [[float(Decimal(z)), float(gelu_tanh(Decimal(z)))] for z in ZS]
    out = {"source": "tanh approximation of GELU, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) (Hendrycks & "
                     "Gimpel 2016), evaluated in 40-digit decimal arithmetic by make_gelu_tanh.py",
           "tolerance": 1e-13, "values": vals}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gelu_tanh.json")
    with open(path, "w") as f:
        json.dump(out, f)
        f.write("\n")


if __name__ == "__main__":
    main()
