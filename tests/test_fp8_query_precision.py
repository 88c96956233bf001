"""Why the FP8-cache decode keeps a bf16 query and the bf16 MFMA chain.

The "练习" exercise 2 of "MLA 推理：两条计算路径与FlashMLA" notes that with an
FP8 latent cache decode becomes compute-bound and that FP8 matrix units could
take QK with care for precision. FP8 MFMA needs both operands in 8 bits, so
the query would be rounded to e4m3. This test measures that rounding alone
(one scale per query row, everything else exact in fp64) against the oracle
of the FP8-cache decode at the workload's length (4096 tokens): on the
workload's own distribution it alone reaches the bf16 gate of 5e-3 relative
L2 (measured 5.25e-3, before the kernel's own bf16 roundings of about 2e-3),
and on sharp scores it is seven times the gate (3.6e-2). So no form of
FP8 QK meets the tolerance; splitting q into an e4m3 high and low part
restores the precision at the cost of two FP8 MFMAs, i.e. the cost of one
bf16 MFMA.
"""
import math

import numpy as np
import torch

from oracle import mla_oracle as orc
from mla_inputs import fp8_case


def _rel_err_of_e4m3_query(q_scale, lens, seed):
    kw = {} if q_scale is None else dict(q_scale=q_scale)
    case = fp8_case(lens, s_q=1, seed=seed, **kw)
    q = case.q_lat.double().numpy()
    codes, scales = case.meta["cache_fp8"], case.meta["row_scales"]
    tab, L = case.block_table.numpy(), case.seqlens.numpy()
    num = den = 0.0
    for b in range(case.B):
        npg = (int(L[b]) + 63) // 64
        sel = torch.from_numpy(tab[b, :npg].astype(np.int64))
        c, sc = codes[sel].numpy(), scales[sel].numpy().astype(np.float64)
        args = (c, sc, np.arange(npg)[None], L[b:b + 1], case.scale, case.causal)
        o_ref, _ = orc.decode_absorbed_fp8(q[b:b + 1], *args, dv=512)
        r = 448.0 / np.maximum(np.max(np.abs(q[b:b + 1]), axis=-1, keepdims=True), 1e-30)
        q8 = orc.e4m3_decode(orc.e4m3_encode((q[b:b + 1] * r).astype(np.float32))).astype(np.float64) / r
        o_8, _ = orc.decode_absorbed_fp8(q8, *args, dv=512)
        num += float(np.sum((o_8 - o_ref) ** 2))
        den += float(np.sum(o_ref ** 2))
    return math.sqrt(num / den)


def test_e4m3_query_misses_the_bf16_gate():
    workload = _rel_err_of_e4m3_query(None, [4096, 4096], seed=120)
    sharp = _rel_err_of_e4m3_query(1.0, [4096, 4096], seed=120)
    print(f"e4m3 query alone: rel-L2 {workload:.2e} (workload q), {sharp:.2e} (unscaled q)")
    assert workload > 4.5e-3  # the whole budget before any kernel rounding
    assert sharp > 2e-2      # several times the budget
