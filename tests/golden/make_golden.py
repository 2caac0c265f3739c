"""Write the hand-derived attention fixture ``rope_attention_closed_form.json``.

The pages (arXiv 2607.28144 summaries) print no worked numeric example of
the attention or of the rotary embedding, so this fixture is a closed form
derived by hand, evaluated with the ``math`` module only (it imports neither
the oracle nor the HIP path).

Set-up: head_dim 6 with one rotary pair per axis (pairs 1/1/1, so every
ladder has theta = base^0 = 1 and the angle of pair a is simply pos_a);
latent grid (T, H, W) = (2, 2, 2), token n = 4 t + 2 h + w.
Every query row is q = (1,0, 1,0, 1,0) and every key row k = (0,1, 0,1, 0,1).
Rotating (1,0) by a gives (cos a, sin a); rotating (0,1) by b gives
(-sin b, cos b); their dot product is sin(a - b). Hence

    s_mn = [sin(t_m - t_n) + sin(h_m - h_n) + sin(w_m - w_n)] / sqrt(6)

and with v_n = (1, n, n^2, 0, 0, 0) the output is
o_m = sum_n exp(s_mn) v_n / sum_n exp(s_mn).
A reversed rotation sense, another token order, another axis order or an
unscaled product each change these values.
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    grid = (2, 2, 2)
    n_tok = 8
    pos = [(n // 4, (n // 2) % 2, n % 2) for n in range(n_tok)]
    q = [[1.0, 0.0, 1.0, 0.0, 1.0, 0.0] for _ in range(n_tok)]
    k = [[0.0, 1.0, 0.0, 1.0, 0.0, 1.0] for _ in range(n_tok)]
    v = [[1.0, float(n), float(n * n), 0.0, 0.0, 0.0] for n in range(n_tok)]
    out = []
    for m in range(n_tok):
        s = [sum(math.sin(pos[m][a] - pos[n][a]) for a in range(3)) / math.sqrt(6.0)
             for n in range(n_tok)]
        e = [math.exp(x) for x in s]
        den = sum(e)
        out.append([sum(e[n] * v[n][c] for n in range(n_tok)) / den for c in range(6)])
    doc = {
        "what": "3D-RoPE exact attention, hand-derived closed form (see make_golden.py)",
        "citation": "the pages print no worked example; closed form of softmax(QK^T/sqrt(d))V "
                    "with the rotary readings of the oracle",
        "head_dim": 6, "pairs": [1, 1, 1], "base": 10000.0, "grid": list(grid),
        "q": [q], "k": [k], "v": [v], "o": [out],
    }
    with open(os.path.join(HERE, "rope_attention_closed_form.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
