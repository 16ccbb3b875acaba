"""GPU parity of the backward's 8-wave tiles and sequence split (ss_bwd with fewer channel
groups than twice the CUs: 32-row tiles; with more groups than CUs as well, or with 4-wave
tiles and more groups than twice the CUs that leave part of the last round of slots empty:
the recomputation and the reverse pass run every sequence in parts — each kernel its own
number, as the checkpoint kernel holds three 4-wave workgroups per CU and the reverse kernel
two (4 groups per CU: only the checkpoint kernel splits; 3.5: 6 parts against 4) — the
reverse pass handing the
adjoint from each part to the one before it — the associative combine of "架构变体：
Mamba/SSM", section "硬件感知算法", in reverse time).

Checks: every gradient against the fp64 oracle's backward element by element (|err| <= tol
* (1 + |ref|), tol 1e-4 fp32 / 2e-3 bf16); the per-channel gradients of a split call equal
those of an unsplit call over a subset of the channels (du, ddelta, dz, dh0 bit for bit: the
parts start on tile boundaries; dA, dD, ddelta_bias to rounding, as they are summed per
part); initial state and final-state gradient; forward and backward split calls alternating
on one stream, the backward's workspace (whose split region both of its kernels use, one
after the other) filled with garbage before every call.
"""
import pytest
import torch

from selective_state_space_86_amd import inputs
from tests import parity_util as pu
from tests.test_bwd_gpu import _announce, _compare, _dy, _gpu, _oracle, KEYS

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _shape(L, dt, groups_per_cu=1.2, seed_name="s"):
    """One batch row with ~1.2 channel groups of 16 per CU (the backward splits there)."""
    groups = int(_cus() * groups_per_cu)
    return inputs.WORKLOADS["mamba130m"].replace(name=f"bs{seed_name}{L}x{groups}{dt}", batch=1, seqlen=L,
                                                 dim=16 * groups, dstate=16, dtype=dt)


@pytest.mark.parametrize("L,dt,gpc", [(600, "f32", 1.2), (1000, "bf16", 1.2), (300, "f32", 1.2),
                                      (700, "f32", 0.5), (2100, "bf16", 1.9), (300, "f32", 3.0),
                                      (520, "bf16", 2.5), (900, "f32", 2.25), (300, "f32", 4.0),
                                      (2000, "bf16", 3.5)])
def test_bwd_split_matches_oracle(L, dt, gpc):
    w = _shape(L, dt, gpc)
    x = inputs.make(w, seed=71, device=DEV)
    dy = _dy((w.batch, w.seqlen, w.dim), 72)
    _announce(f"8-wave / split backward {w.name}")
    g = _gpu(x, dy, True)
    torch.cuda.synchronize()
    _compare(g, _oracle(x, dy, True), pu.tol_of(x), f"split {w.name}")


@pytest.mark.parametrize("gpc", [1.2, 3.0])
def test_bwd_split_per_channel_gradients_equal_unsplit(gpc):
    """Channel groups are independent but for dB and dC: the first groups computed alone
    (no split: 64 groups of 8-wave tiles, or as many 4-wave ones as fill the slots once) give
    the same per-channel gradients as inside the split call with the same tiles."""
    w = _shape(700, "f32", gpc, seed_name="e")
    x = inputs.make(w, seed=73, device=DEV)
    dy = _dy((w.batch, w.seqlen, w.dim), 74)
    sub = (64 if gpc < 2 else 2 * _cus()) * 16
    xs = {k: (v[..., :sub].contiguous() if k in ("u", "delta", "z") else
              v[:sub].contiguous() if k in ("A", "D", "delta_bias") else v) for k, v in x.items()}
    _announce("split vs unsplit per-channel gradients")
    g = _gpu(x, dy, True)
    gs = _gpu(xs, dy[..., :sub].contiguous(), True)
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dz"):
        assert torch.equal(g[k][..., :sub], gs[k]), k
    assert torch.equal(g["dh0"][:, :sub], gs["dh0"])
    for k in ("dA", "dD", "ddelta_bias"):
        d = ((g[k][:sub] - gs[k]).abs() / (1 + gs[k].abs())).max().item()
        assert d <= 2e-5, f"{k}: {d:.3e}"


def test_bwd_split_initial_state_and_final_state_gradient():
    w = _shape(500, "f32", seed_name="h")
    x = inputs.make(w, seed=75, device=DEV)
    dy = _dy((w.batch, w.seqlen, w.dim), 76)
    h0 = _dy((w.batch, w.dim, 16), 77)
    dlast = _dy((w.batch, w.dim, 16), 78)
    _announce("split backward with h0 and dlast")
    g = _gpu(x, dy, True, h0=h0, dlast=dlast)
    torch.cuda.synchronize()
    _compare(g, _oracle(x, dy, True, h0=h0, dlast=dlast), pu.tol_of(x), "split h0/dlast")


def test_forward_and_backward_splits_with_dirty_workspaces():
    """Forward and backward split calls alternate on one stream (1.25 groups per CU: both
    split), each with a persistent workspace filled with 0xff bytes before every call; every
    call repeats the first one's bits and no hand-off wait gives up."""
    import selective_state_space_86_amd as ss

    w = _shape(2000, "bf16", groups_per_cu=1.25, seed_name="m")
    x = inputs.make(w, seed=79, device=DEV)
    dy = _dy((w.batch, w.seqlen, w.dim), 80)
    _announce("forward/backward splits alternating, dirty workspaces")
    fws = torch.empty(ss.fwd_workspace_size(w.batch, w.seqlen, w.dim, 16, torch.bfloat16), dtype=torch.uint8,
                      device=DEV)
    bws = torch.empty(ss.bwd_workspace_size(w.batch, w.seqlen, w.dim, 16), dtype=torch.uint8, device=DEV)
    assert fws.numel() > 0
    y0 = pu.gpu_fwd(x, True, workspace=fws)
    g0 = _gpu(x, dy, True)
    y1 = pu.gpu_fwd(x, True, split_parts=1)
    torch.cuda.synchronize()
    assert torch.equal(y0[0], y1[0]) and torch.equal(y0[1], y1[1])
    for _ in range(3):
        fws.fill_(255)
        bws.fill_(255)
        y = pu.gpu_fwd(x, True, workspace=fws)
        g = ss.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"],
                   delta_bias=x["delta_bias"], workspace=bws)
        torch.cuda.synchronize()
        assert ss.workspace_status(fws) == (0, 0) and ss.workspace_status(bws) == (0, 0)
        assert torch.equal(y[0], y0[0]) and torch.equal(y[1], y0[1])
        for k in KEYS:
            if g[k] is not None:
                assert torch.equal(g[k], g0[k]), k
