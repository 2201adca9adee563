"""Oracle-side preparation of MoE block cases, shared by the oracle pins and
the GPU parity tests (numpy and the oracle only)."""
import numpy as np
import torch

from mxfp4_w4a4_post_amd import inputs


def stack_rows(wg, wu):
    """[F, H] gate and up weight rows -> [2F, H], alternating blocks of 32 rows."""
    F, H = wg.shape
    return np.stack([wg.reshape(F // 32, 32, H), wu.reshape(F // 32, 32, H)], axis=1).reshape(2 * F, H)


def bf16_round(v):
    return torch.from_numpy(np.asarray(v, np.float64)).float().bfloat16().float().numpy().astype(np.float64)


def oracle_prepare(orc, c, experts=None):
    """Per expert (all, or only those in `experts`): calibrate, multipliers,
    prepared stacked gate/up and down weights (row-major codes and scales).
    Experts left out keep zero weights and unit multipliers."""
    bits = inputs.bf16_bits
    E, F, H, b = c.E, c.F, c.H, c.b
    a_gu = np.ones((E, H), np.float32)
    a_dn = np.ones((E, F), np.float32)
    gc = np.zeros((E, 2 * F, H // 2), np.uint8)
    gs = np.zeros((E, 2 * F, H // 32), np.uint8)
    dc = np.zeros((E, H, F // 2), np.uint8)
    ds = np.zeros((E, H, F // 32), np.uint8)
    for e in (range(E) if experts is None else sorted(set(int(v) for v in experts))):
        if b == 0:
            gc[e], gs[e] = orc.prepare_weights(stack_rows(bits(c.w_gate[e]), bits(c.w_up[e])), None, 0)
            dc[e], ds[e] = orc.prepare_weights(bits(c.w_dn[e]), None, 0)
            continue
        a, r = orc.multipliers(orc.calibrate(bits(c.xcal_gu[e])), b)
        a_gu[e] = a
        gc[e], gs[e] = orc.prepare_weights(stack_rows(bits(c.w_gate[e]), bits(c.w_up[e])), r, b)
        a, r = orc.multipliers(orc.calibrate(bits(c.xcal_dn[e])), b)
        a_dn[e] = a
        dc[e], ds[e] = orc.prepare_weights(bits(c.w_dn[e]), r, b)
    if b == 0:
        return None, gc, gs, None, dc, ds
    return a_gu, gc, gs, a_dn, dc, ds
