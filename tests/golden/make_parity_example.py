"""Writes parity_example.txt: a fixed bit string and the parity sign of each
prefix, (-1)^(x_0 + ... + x_t). This is the parity task the "Mamba-3" summary
page uses to motivate rotations ("Context and Motivation", Gap 2): sum_t x_t
mod 2, solved by h_t = R(pi x_t) h_{t-1} from h = [1, 0]. The expected signs
come from the definition of parity alone (no oracle, no GPU)."""
import os

BITS = "1011001110001011110100101100011101"

with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "parity_example.txt"), "w") as f:
    f.write("# parity worked example: bit x_t, then (-1)^(x_0+...+x_t)\n")
    f.write("# source: 'Mamba-3' summary page, Context and Motivation (Gap 2) and\n")
    f.write("# Complex-Valued SSMs (parity via rotation R(pi x_t)); written by make_parity_example.py\n")
    run = 0
    for ch in BITS:
        run += int(ch)
        f.write(f"{ch} {1 if run % 2 == 0 else -1}\n")
