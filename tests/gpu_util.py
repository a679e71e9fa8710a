"""Helpers of the GPU parity tests: moving a quantised problem to the
device, running the library's entry points, and the comparison bars."""
import json
import os
import sys

import numpy as np
import torch

import mixture_experts_forward_moe_amd as moe
import oracle
import synth

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    """numpy -> device tensor with the same bytes (uint16 bf16 bits -> int16)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t, dtype=None):
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


class DeviceProblem:
    def __init__(self, p: oracle.Problem):
        self.p = p
        self.x = dev(p.x)
        self.x_sf = dev(p.x_sf)
        self.ids = dev(p.topk_ids)
        self.w = dev(p.topk_weights)
        self.w1, self.w1_sf, self.w1_alpha = dev(p.w1), dev(p.w1_sf), dev(p.w1_alpha)
        self.w2, self.w2_sf, self.w2_alpha = dev(p.w2), dev(p.w2_sf), dev(p.w2_alpha)
        self.fc2 = dev(np.array([p.fc2_input_scale], np.float32)) if p.mode == oracle.W4A4 else None
        self.w1_alpha_up = None if p.w1_alpha_up is None else dev(p.w1_alpha_up)
        self.pts = None if p.per_token_scale is None else dev(p.per_token_scale)
        self.fc1_bias = None if p.fc1_bias is None else dev(p.fc1_bias)
        self.fc2_bias = None if p.fc2_bias is None else dev(p.fc2_bias)

    def forward(self, out=None, tile=0, **kw):
        p = self.p
        if out is None:
            out = torch.zeros((p.M, p.H), dtype=torch.int16, device=DEV)
        moe.moe_forward(self.x, self.x_sf, self.ids, self.w, self.w1, self.w1_sf, self.w1_alpha, self.w2,
                        self.w2_sf, self.w2_alpha, p.num_experts, p.top_k, p.num_local_experts,
                        p.local_expert_offset, p.mode, out, p.H, p.I, tile=tile,
                        swiglu_alpha=p.swiglu_alpha, swiglu_beta=p.swiglu_beta, swiglu_limit=p.swiglu_limit,
                        activation=p.activation, situ_beta=p.situ_beta, situ_linear_beta=p.situ_linear_beta,
                        w1_alpha_up=self.w1_alpha_up, per_token_scale=self.pts, fc1_bias=self.fc1_bias,
                        fc2_bias=self.fc2_bias,
                        fc2_input_scale=self.fc2, routed_scaling_factor=p.routed_scaling_factor, **kw)
        return out


PLAN_ARRAYS = ("expanded_to_permuted", "permuted_to_expanded", "tile_to_expert", "tile_to_mn_limit", "num_tiles",
               "expert_offsets", "expert_counts")


def forward_in_workspace(d: DeviceProblem, tile: int, fill: int = 0xA5, **kw):
    """One moe_forward on a fresh workspace whose bytes all start as `fill`
    (the workspace needs no initial contents); returns the output and a view
    of the routing plan that forward built and used (moe_forward_plan)."""
    p = d.p
    fm = kw.get("finalize_mode", moe.FINALIZE_DETERMINISTIC)
    n = moe.workspace_size(p.M, p.H, p.I, p.top_k, p.num_local_experts, tile, p.mode, fm)
    ws = torch.full((n,), fill, dtype=torch.uint8, device=DEV)
    out = kw.pop("out", None)
    out = d.forward(out=out, tile=tile, workspace=ws, **kw)
    plan = moe.MoePlan(p.M, p.top_k, p.num_local_experts, tile, forward_workspace=ws)
    return out, plan


def assert_plan_equal(plan, ref: oracle.Plan, what=""):
    """All seven plan arrays bit for bit against the oracle's plan."""
    torch.cuda.synchronize()
    for name in PLAN_ARRAYS:
        got = host(getattr(plan, name))
        want = np.atleast_1d(np.asarray(getattr(ref, name)))
        assert got.shape == want.shape, (what, name, got.shape, want.shape)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (what, name, bad[:8], got[bad[:8]], want[bad[:8]])


def bf16(bits):
    return synth.bf16_to_f32(np.asarray(bits).view(np.uint16)).astype(np.float64)


def check_close(got_bits, ref_bits, mode, what=""):
    """The parity bar: rel-L2 <= 5e-3 and every |err| <= 1e-2 max|ref|
    (W4A16 and MXFP8 x MXFP4, the FC1 output requantised to MXFP8 included);
    rel-L2 <= 2e-2 (W4A4 with its NVFP4 requantisation)."""
    g = bf16(got_bits)
    r = bf16(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    maxerr = np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)
    exact = float(np.mean(np.asarray(got_bits).view(np.uint16) == np.asarray(ref_bits).view(np.uint16)))
    say(f"{what}: rel_l2={err:.3e} max_err/max_ref={maxerr:.3e} bit_exact_frac={exact:.4f}")
    log = os.environ.get("MOE_PARITY_LOG")
    if log:  # one JSON line per comparison, for the record of a run
        with open(log, "a") as f:
            f.write(json.dumps({"case": what, "rel_l2": err, "max_err_over_max_ref": maxerr,
                                "bit_exact_frac": exact, "values": int(g.size),
                                "max_bar": mode != oracle.W4A4}) + "\n")
    if mode == oracle.W4A4:
        assert err <= 2e-2, (what, err)
    else:
        assert err <= 5e-3, (what, err)
        assert maxerr <= 1e-2, (what, maxerr)
    return err, maxerr, exact
