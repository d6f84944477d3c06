"""The README's Python example, run as written (seeded), and checked against the
oracle for its first and last sequence: the documented calls stay valid."""
import os
import re

import numpy as np
import pytest
import torch

import oracle as O

from oracle_inputs import compare

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_bits_to_float(t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def test_readme_example_matches_the_oracle():
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)\n```", text, re.S).group(1)
    torch.manual_seed(0)
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    B, Sq, L = ns["B"], ns["Sq"], ns["L"]
    rows = ns["cache"].view(-1, 576)
    w = f64(ns["w_kv_b"])
    inv = O.yarn_inv_freq()
    for b in (0, B - 1):
        seq = rows[ns["block_table"][b].long().repeat_interleave(64) * 64 + torch.arange(L, device="cuda") % 64]
        c, k = f64(seq[:, :512]), f64(seq[:, 512:])      # rope keys as the library rotated them
        qn = f64(ns["q_nope"][b])
        qp = O.round_to_bf16(O.rope_rotate(f64(ns["q_pe"][b]), (L - Sq + np.arange(Sq))[:, None], inv))
        ref_o, ref_l = O.mla_attention_absorbed(qn, qp, c, k, w, O.softmax_scale())
        s = compare(f64(ns["out"][b]), ns["lse"][b].cpu().numpy(), ref_o, ref_l)
        print(f"README example, sequence {b}: max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}", flush=True)
