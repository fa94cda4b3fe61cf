"""Constructed layers whose output is known exactly, shared by the oracle pins
and the GPU parity tests."""
import torch

import moe_synth as ms


def identity_stored(fmt, rows, cols, dense):
    """Store a matrix whose entries are in {-1, 0, 1} so that it decodes exactly
    (weights in the tiled storage layout, scales row-major)."""
    w, s = identity_rowmajor(fmt, rows, cols, dense)
    return ms.tile_16x64(w), s


def identity_rowmajor(fmt, rows, cols, dense):
    if fmt in ("f32", "bf16"):
        return ms.encode_rowmajor(dense, fmt)
    if fmt == "fp8_b128":
        # 256 * 2^-8 = 1: code 0x78 is +256, 0xF8 is -256
        codes = torch.zeros(rows, cols, dtype=torch.uint8, device=dense.device)
        codes[dense > 0] = 0x78
        codes[dense < 0] = 0xF8
        s = torch.full((-(-rows // 128), -(-cols // 128)), 2.0 ** -8, dtype=torch.float32,
                       device=dense.device)
        return codes, s
    if fmt == "mxfp4":
        # 4 * 2^(125-127) = 1: e2m1 code 6 is +4, 14 is -4
        nib = torch.zeros(rows, cols, dtype=torch.uint8, device=dense.device)
        nib[dense > 0] = 6
        nib[dense < 0] = 14
        packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()
        return packed, torch.full((rows, cols // 32), 125, dtype=torch.uint8, device=dense.device)
    raise ValueError(fmt)


def identity_layer(fmt, h=64, E=4, k=2, scoring="softmax", rsf=1.0, shared=False,
                   zero_routed_down=False, sgate=False, act="bf16", device="cpu"):
    """Experts with I = 2h: gate = [I; -I], up rows = e0, down = [I, -I], so that
    with x[0] = 1 every expert maps x to silu(x) - silu(-x) = x."""
    I = 2 * h
    spec = ms.SPECS["tiny"].with_(hidden=h, num_experts=E, top_k=k, inter=I, scoring=scoring,
                                  routed_scaling=rsf, act_dtype=act, expert_dtype=fmt,
                                  shared_inter=I if shared else 0, shared_gate=sgate,
                                  corr_bias=scoring == "sigmoid")
    eye = torch.eye(h, device=device)
    wg = torch.cat([eye, -eye], 0)
    wu = torch.zeros(I, h, device=device)
    wu[:, 0] = 1
    wd = torch.cat([eye, -eye], 1)
    li = ms.make_layer(spec, seed=11, device=device)
    li.x[:, 0] = 1.0
    mats = {"gate": wg, "up": wu, "down": wd}
    for name in ("gate", "up", "down"):
        m = getattr(li, name)
        for e in range(E):
            d = mats[name] if not (name == "down" and zero_routed_down) else torch.zeros(h, I, device=device)
            w, s = identity_stored(fmt, *d.shape, d)
            m.w[e].copy_(w)
            if m.s is not None:
                m.s[e].copy_(s)
    if shared:
        for name in ("sh_gate", "sh_up", "sh_down"):
            m = getattr(li, name)
            d = mats[name[3:]]
            w, s = identity_stored(fmt, *d.shape, d)
            m.w[0].copy_(w)
            if m.s is not None:
                m.s[0].copy_(s)
    return li
