"""Every entry point captured together in one HIP graph and replayed, with
new inputs and eager calls of the same entry points between the replays.
Each replay's outputs are compared with the oracle, byte for byte, so a
graph node that misbehaves after the first replay is caught.

The dim0-family calls take one caller workspace (they run one after another
on the capturing stream, and each leaves it zero), so nothing is allocated
during capture."""
import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import assert_same_bytes, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


# dim0 / dim0_t: a 1904-row group is a three-chunk team for both kernels,
# beside a short group on wide strips and an empty one
M0, K0 = 3008, 264
OFF0 = np.array([16, 1920, 1920, 3008], np.int32)
E, D1, D2 = 3, 1000, 136          # experts: two-chunk teams of equal groups
M1, K1 = 64, 1040                 # dim1
OFF1 = np.array([0, 160, 480, 1040], np.int32)
MX_M, MX_K = 256, 1024            # MX cast and dequantisation
T_M, T_K = 256, 136               # MX dim1


def inputs(seed):
    rng = np.random.default_rng(seed)
    return {"x0": wl.randn_bf16(rng, (M0, K0), 0.02, 0.001, 8.0),
            "w": wl.randn_bf16(rng, (E, D1, D2), 0.02, 0.001, 8.0),
            "x1": wl.randn_bf16(rng, (M1, K1), 0.02, 0.001, 8.0),
            "x5": wl.randn_bf16(rng, (MX_M, MX_K), 1.0, 0.001, 100.0),
            "xt": wl.randn_bf16(rng, (T_M, T_K), 1.0, 0.001, 100.0)}


def expected(h):
    """Every output of one replay, from the oracle."""
    out = {}
    out["q0"], out["s0"] = oracle.quant_groups_dim0(h["x0"], OFF0)
    out["qt"], out["st"] = oracle.quant_groups_dim0_t(h["x0"], OFF0, True)
    out["qe"], out["se"] = oracle.quant_experts_dim1(h["w"], False)
    out["q1"], out["s1"] = oracle.quant_groups_dim1(h["x1"], OFF1)
    out["q5f"], out["s5f"] = oracle.mx_quant_dim0(h["x5"], mgs.MGS_MX_FLOOR)
    out["q5r"], out["s5r"] = oracle.mx_quant_dim0(h["x5"], mgs.MGS_MX_RCEIL)
    out["y5"] = oracle.mx_dequant_dim0(out["q5r"], out["s5r"])
    out["qd"], out["sd"] = oracle.mx_quant_dim1(h["xt"], mgs.MGS_MX_RCEIL)
    return out


def test_every_entry_point_in_one_graph():
    h0 = inputs(700)
    dev = {k: to_dev(v) for k, v in h0.items()}
    o0, o1 = to_dev(OFF0), to_dev(OFF1)
    ws = mgs.dim0_workspace(max(M0, E * D1), max(K0, D2))
    u8, f32 = torch.uint8, torch.float32
    out = {"q0": torch.empty((M0, K0), dtype=u8, device="cuda"),
           "s0": torch.empty((4, K0), dtype=f32, device="cuda"),
           "qt": torch.empty((K0, M0), dtype=u8, device="cuda"),
           "st": torch.empty((K0, 4), dtype=f32, device="cuda"),
           "qe": torch.empty((E, D1, D2), dtype=u8, device="cuda"),
           "se": torch.empty((E, D2), dtype=f32, device="cuda"),
           "q1": torch.empty((M1, K1), dtype=u8, device="cuda"),
           "s1": torch.empty((M1, 4), dtype=f32, device="cuda"),
           "q5f": torch.empty((MX_M, MX_K), dtype=u8, device="cuda"),
           "s5f": torch.empty((MX_M, MX_K // 32), dtype=u8, device="cuda"),
           "q5r": torch.empty((MX_M, MX_K), dtype=u8, device="cuda"),
           "s5r": torch.empty((MX_M, MX_K // 32), dtype=u8, device="cuda"),
           "y5": torch.empty((MX_M, MX_K), dtype=torch.bfloat16, device="cuda"),
           "qd": torch.empty((T_K, T_M), dtype=u8, device="cuda"),
           "sd": torch.empty((T_K, T_M // 32), dtype=u8, device="cuda")}

    def run_all():
        mgs.mgs_quant_groups_dim0(dev["x0"], o0, q=out["q0"], scales=out["s0"], workspace=ws)
        mgs.mgs_quant_groups_dim0_t(dev["x0"], o0, True, q_t=out["qt"], scales_t=out["st"], workspace=ws)
        mgs.mgs_quant_experts_dim1(dev["w"], q=out["qe"], scales=out["se"], workspace=ws)
        mgs.mgs_quant_groups_dim1(dev["x1"], o1, q=out["q1"], scales=out["s1"])
        mgs.mgs_mx_quant_dim0(dev["x5"], mgs.MGS_MX_FLOOR, q=out["q5f"], scales=out["s5f"])
        mgs.mgs_mx_quant_dim0(dev["x5"], mgs.MGS_MX_RCEIL, q=out["q5r"], scales=out["s5r"])
        mgs.mgs_mx_dequant_dim0(out["q5r"], out["s5r"], y=out["y5"])
        mgs.mgs_mx_quant_dim1(dev["xt"], mgs.MGS_MX_RCEIL, q_t=out["qd"], scales_t=out["sd"])

    def check(h, what):
        want = expected(h)
        for k, v in want.items():
            got = out[k].view(torch.int16) if out[k].dtype == torch.bfloat16 else out[k]
            got = got.cpu().numpy()
            if out[k].dtype == torch.bfloat16:
                got = got.view(np.uint16)
            assert_same_bytes(got, v, "%s: %s" % (what, k))

    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_all()
    torch.cuda.synchronize()
    def clear_outputs():
        # so that a launch that writes nothing cannot pass on old results
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()

    for i, seed in enumerate((701, 702, 701)):
        h = inputs(seed)
        for k, v in h.items():
            dev[k].copy_(to_dev(v))
        clear_outputs()
        g.replay()
        torch.cuda.synchronize()
        check(h, "replay %d" % i)
        # eager calls of the same entry points on the capturing stream,
        # into the same outputs, between the replays
        clear_outputs()
        with torch.cuda.stream(s):
            run_all()
        torch.cuda.synchronize()
        check(h, "eager after replay %d" % i)
