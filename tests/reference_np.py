"""An independent numpy/torch statement of the fused MoE forward, built from
library routines (torch's float8 decoders, numpy matmul in fp64, torch
sigmoid, torch's fp32->bf16 conversion) and brute-force nearest-value
quantisation.  It shares nothing with the C oracle and pins it in tests.
It is per-token and slow; only small shapes go through it."""
import numpy as np
import torch

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
W4A16, W4A4, MXFP8_MXFP4 = 0, 1, 2


def e2m1_vals(codes):
    codes = np.asarray(codes).astype(np.int64)
    v = E2M1[codes & 7]
    return np.where(codes & 8, -v, v)


def unpack(q):
    q = np.asarray(q, np.uint8)
    return np.stack([q & 15, q >> 4], -1).reshape(q.shape[:-1] + (2 * q.shape[-1],))


def e4m3_vals(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def e8m0_vals(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e8m0fnu).double().numpy()


def bf16_vals(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()


def to_bf16_bits(v):
    """fp64 -> bf16 through torch (via fp32; a double rounding in rare ties)."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def deq_rows(mode, q, sf):
    """decoded weight rows: [..., K] from packed E2M1 codes and block scales"""
    v = e2m1_vals(unpack(q))
    if mode == MXFP8_MXFP4:
        return v * np.repeat(e8m0_vals(sf), 32, axis=-1)
    return v * np.repeat(e4m3_vals(sf), 16, axis=-1)


def nearest_e2m1(r):
    """brute force: the nearest E2M1 magnitude (ties to the even code), saturating, sign kept"""
    a = np.minimum(np.abs(np.asarray(r, np.float64)), 6.0)
    d = np.abs(a[..., None] - E2M1)
    tie_rank = (d > d.min(-1, keepdims=True)) * 2 + (np.arange(8) % 2)
    best = np.argmin(tie_rank, -1)
    return (best | (np.signbit(r).astype(np.int64) << 3)).astype(np.uint8)


def nearest_e4m3(r):
    r = np.clip(np.asarray(r, np.float32), -448.0, 448.0)
    return torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quant_nvfp4(v, gs):
    """NVFP4 of an fp32 row vector [K] with global scale gs, fp32 decisions."""
    v = np.asarray(v, np.float32)
    K = v.size
    gs = np.float32(gs)
    codes = np.zeros(K, np.uint8)
    scales = np.zeros(K // 16, np.uint8)
    deq = np.zeros(K)
    for b in range(K // 16):
        blk = v[b * 16:(b + 1) * 16]
        bamax = np.float32(np.abs(blk).max())
        sc = 0
        if gs > 0 and bamax > 0:
            sc = int(nearest_e4m3(np.array([bamax / (np.float32(6.0) * gs)], np.float32))[0])
        scales[b] = sc
        sd = np.float32(e4m3_vals(np.array([sc]))[0])
        denom = np.float32(sd * gs)
        if denom > 0:
            c = nearest_e2m1((blk / denom).astype(np.float32))
        else:
            c = np.zeros(16, np.uint8)
        codes[b * 16:(b + 1) * 16] = c
        deq[b * 16:(b + 1) * 16] = e2m1_vals(c) * float(sd)
    return codes, scales, deq


def quant_mxfp8(v):
    v = np.asarray(v, np.float32)
    K = v.size
    deq = np.zeros(K)
    for b in range(K // 32):
        blk = v[b * 32:(b + 1) * 32]
        amax = float(np.abs(blk).max())
        code = 0
        if amax > 0:
            m, e = np.frexp(amax)
            code = int(np.clip(e - 1 - 8 + 127, 0, 254))
        X = 2.0 ** (code - 127)
        c = nearest_e4m3((blk / X).astype(np.float32))
        deq[b * 32:(b + 1) * 32] = e4m3_vals(c) * X
    return deq


def swiglu(g, u, alpha, beta, limit):
    g = torch.from_numpy(np.asarray(g, np.float64))
    u = torch.from_numpy(np.asarray(u, np.float64))
    gc = torch.clamp(g, max=float(limit))
    uc = torch.clamp(u, min=-float(limit), max=float(limit))
    return (gc * torch.sigmoid(float(alpha) * gc) * (uc + float(beta))).numpy()


def gated_act(p, g, u):
    """FC1 activation of an oracle.Problem-like p, from torch's own routines
    (gelu with the tanh approximation, tanh, sigmoid) in fp64"""
    if getattr(p, "activation", 0) == 1:
        gt = torch.from_numpy(np.asarray(g, np.float64))
        ut = torch.from_numpy(np.asarray(u, np.float64))
        return (torch.nn.functional.gelu(gt, approximate="tanh") * ut).numpy()
    if getattr(p, "situ_beta", 0.0) > 0.0:
        gt = torch.from_numpy(np.asarray(g, np.float64))
        ut = torch.from_numpy(np.asarray(u, np.float64))
        b = float(np.float32(p.situ_beta))
        up = ut
        if p.situ_linear_beta > 0.0:
            lb = float(np.float32(p.situ_linear_beta))
            up = lb * torch.tanh(ut / lb)
        return (b * torch.tanh(gt / b) * torch.sigmoid(gt) * up).numpy()
    return swiglu(g, u, p.swiglu_alpha, p.swiglu_beta, p.swiglu_limit)


def forward_tokens(p, tokens):
    """out bf16 bits [len(tokens), H] for an oracle.Problem-like object p."""
    H, I, k = p.H, p.I, p.top_k
    out = np.zeros((len(tokens), H), np.uint16)
    w1d_cache = {}
    for i, t in enumerate(tokens):
        if p.mode == W4A16:
            a = bf16_vals(p.x[t])
        elif p.mode == W4A4:
            a = e2m1_vals(unpack(p.x[t])) * np.repeat(e4m3_vals(p.x_sf[t]), 16)
        else:
            a = e4m3_vals(p.x[t]) * np.repeat(e8m0_vals(p.x_sf[t]), 32)
        acc = np.zeros(H, np.float32)
        for j in range(k):
            gid = int(p.topk_ids[t, j])
            le = gid - p.local_expert_offset
            if gid < p.local_expert_offset or le >= p.num_local_experts:
                continue
            if le not in w1d_cache:
                w1d_cache[le] = (deq_rows(p.mode, p.w1[le], p.w1_sf[le]), deq_rows(p.mode, p.w2[le], p.w2_sf[le]))
            W1d, W2d = w1d_cache[le]
            gu = W1d @ a
            al1 = np.float32(p.w1_alpha[le])
            if getattr(p, "activation", 0) == 2:
                # non-gated ReLU^2 (torch's relu) of the single row, scaled like the gate
                h = (gu.astype(np.float32) * al1).astype(np.float32)
                if getattr(p, "per_token_scale", None) is not None:
                    h = (h * np.float32(p.per_token_scale[t])).astype(np.float32)
                if getattr(p, "fc1_bias", None) is not None:
                    h = (h + p.fc1_bias[le]).astype(np.float32)
                r = torch.relu(torch.from_numpy(h.astype(np.float64)))
                y1 = bf16_vals(to_bf16_bits((r * r).numpy()))
            else:
                y1 = None
            al1 = np.float32(p.w1_alpha[le])
            alu = al1 if getattr(p, "w1_alpha_up", None) is None else np.float32(p.w1_alpha_up[le])
            g = (gu[:I].astype(np.float32) * al1).astype(np.float32)
            u = (gu[I:].astype(np.float32) * alu).astype(np.float32)
            if getattr(p, "per_token_scale", None) is not None:
                pts = np.float32(p.per_token_scale[t])
                g = (g * pts).astype(np.float32)
                u = (u * pts).astype(np.float32)
            if getattr(p, "fc1_bias", None) is not None:
                g = (g + p.fc1_bias[le, :I]).astype(np.float32)
                u = (u + p.fc1_bias[le, I:]).astype(np.float32)
            if y1 is None:
                y1 = bf16_vals(to_bf16_bits(gated_act(p, g, u)))
            if p.mode == W4A16:
                a2 = y1
            elif p.mode == W4A4:
                _, _, a2 = quant_nvfp4(y1.astype(np.float32), p.fc2_input_scale)
            else:
                a2 = quant_mxfp8(y1.astype(np.float32))
            Y = W2d @ a2
            Y2 = (Y.astype(np.float32) * np.float32(p.w2_alpha[le])).astype(np.float32)
            if getattr(p, "fc2_bias", None) is not None:
                Y2 = (Y2 + p.fc2_bias[le]).astype(np.float32)
            y2 = bf16_vals(to_bf16_bits(Y2))
            wf = np.float32(np.float32(p.topk_weights[t, j]) * np.float32(p.routed_scaling_factor))
            acc = (acc + (wf * y2.astype(np.float32)).astype(np.float32)).astype(np.float32)
        out[i] = to_bf16_bits(acc.astype(np.float64))
    return out
