"""Write oracle_regression.txt: a regression lock on the oracle's output.

Calls only ``oracle/`` (and ``workloads`` for the seeded inputs).  The stored
values are not a pin of correctness -- the pages print no worked example --
they only make any later change to the oracle's arithmetic visible.

Run from the repository root:  python tests/golden/make_oracle_regression.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

ADALN_CASES = [("bf16", "fp32"), ("fp16", "bf16")]
GN_CASES = [("bf16", "fp32"), ("fp16", "fp16")]
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.txt")
CASES = [  # (style, x dtype, cos dtype, cos layout, head_dim)
    ("interleaved", "bf16", "fp32", "shared", 64),
    ("rotate_half", "fp16", "fp32", "per_head", 128),
    ("interleaved", "fp16", "bf16", "shared", 128),
]


def cases():
    for style, xdt, cdt, lay, d in CASES:
        T, H = 3, 2
        qkv = wl.fused_qkv(4242, T, H, d, xdt)
        qg, kg = wl.norm_weights(4242, d)
        c, s = wl.rope_tables(np.arange(T) * 37, (d // 2,), d, style, dtype=cdt)
        if lay == "per_head":
            c, s = wl.expand_per_head(c, H), wl.expand_per_head(s, H)
        to_np = (lambda t: t.numpy()) if cdt == "fp32" else wl.u16
        q, k = oracle.fused_qk(wl.u16(qkv), xdt, heads=H, head_dim=d, q_gamma=qg.numpy(),
                               k_gamma=kg.numpy(), eps=wl.EPS, cos=to_np(c), sin=to_np(s),
                               cos_dtype=cdt, cos_layout=lay, style=style)
        yield "%s %s %s %s %d" % (style, xdt, cdt, lay, d), np.concatenate([q.ravel(), k.ravel()])
    for xdt, mdt in ADALN_CASES:
        x, sc, sh = wl.adaln_inputs(4343, 6, 200, 2, xdt, mdt)
        to_np = (lambda t: t.numpy()) if mdt == "fp32" else wl.u16
        y = oracle.adaln(wl.u16(x), xdt, hidden=200, rows_per_batch=3, scale=to_np(sc),
                         shift=to_np(sh), mod_dtype=mdt, eps=wl.EPS)
        yield "adaln %s %s" % (xdt, mdt), y.ravel()
    for xdt, pdt in GN_CASES:
        x, g, b = wl.gn_inputs(4344, 2, 16, 48, xdt, pdt)
        to_np = (lambda t: t.numpy()) if pdt == "fp32" else wl.u16
        y = oracle.group_norm_silu(wl.u16(x), xdt, channels=16, spatial=48, groups=4,
                                   gamma=to_np(g), beta=to_np(b), param_dtype=pdt, eps=wl.EPS)
        yield "group_norm_silu %s %s" % (xdt, pdt), y


def main():
    with open(OUT, "w") as f:
        f.write("# oracle regression lock; written by make_oracle_regression.py\n")
        for name, vals in cases():
            f.write("case %s\n" % name)
            for i in range(0, vals.size, 97):      # every 97th value, as exact hex
                f.write("%d %s\n" % (i, float(vals[i]).hex()))


if __name__ == "__main__":
    main()
