"""Every entry point captured in a HIP graph: a caller that records its step
once and replays it (HIP graphs replace per-call launches for launch-bound
loops) must get, on every replay, exactly what the same calls give eagerly.

One step on fixed buffers -- EF int4 quantize (fp16 gradient, per-parameter
batched form too), the 8-way reduce with requant and requant EF, the 4-way
reduce, qwZ int8 quantize and dequantize, SR accumulate single and batched
with zeroing -- is run eagerly on buffer set A and replayed from a graph on
buffer set B, three times, with eager work between the replays that changes
the inputs in both sets the same way.  Everything is compared bit for bit
after every replay: the graph must read its buffers' current contents, the
in-place EF buffers must evolve identically, and nothing may be captured
as a memset (the library issues none).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_communication_zero_amd  # noqa: F401  (fails loudly if libzq.so is missing)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


P1, P2, B = 8, 4, 128
M = P1 * P2 * B * 97 + 0  # 397,312 elements: 8 chunks of 49,664 (ragged tiles), 4 sub-chunks
N8 = 3 * 2048 * 40 + 77   # int8 weights, ragged
NS = 4096 * 9 + 13        # SR elements


def make_set(seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    n1, n2 = M // P1, M // (P1 * P2)
    s = {
        "g": (torch.randn(M, device="cuda", generator=g) * 1e-3).half(),
        "ef": torch.zeros(M, device="cuda"),
        "codes": torch.zeros(M // 2, dtype=torch.uint8, device="cuda"),
        "scales": torch.zeros(M // B, device="cuda"),
        "rqc": torch.zeros(n1 // 2, dtype=torch.uint8, device="cuda"),
        "rqs": torch.zeros(-(-n1 // B), device="cuda"),
        "rqe": torch.zeros(n1, device="cuda"),
        "out2": torch.zeros(n2, device="cuda"),
        "w": torch.randn(N8, device="cuda", generator=g).mul(0.02).to(torch.bfloat16),
        "c8": torch.zeros(N8, dtype=torch.int8, device="cuda"),
        "s8": torch.zeros(-(-N8 // 2048), device="cuda"),
        "wd": torch.zeros(N8, dtype=torch.float16, device="cuda"),
        "dst": torch.zeros(NS, dtype=torch.bfloat16, device="cuda"),
        "src": (torch.randn(NS, device="cuda", generator=g) * 1e-2).to(torch.bfloat16),
        "dst_b": [torch.zeros(m, dtype=torch.bfloat16, device="cuda") for m in (1000, 4096, 24)],
        "red_b": [(torch.randn(4 * m, device="cuda", generator=g) * 1e-2).to(torch.bfloat16)
                  for m in (1000, 4096, 24)],
        # per-parameter EF quantize: three tensors carved out of one buffer
        "bg": (torch.randn(9000, device="cuda", generator=g) * 1e-3).half(),
        "bef": torch.zeros(9000, device="cuda"),
        "bc": torch.zeros(4500, dtype=torch.uint8, device="cuda"),
        "bs": torch.zeros(9000 // B + 3, device="cuda"),
    }
    return s


def step(zq, s, tables):
    n1, n2 = M // P1, M // (P1 * P2)
    zq.zq_quantize_ef_int4(s["g"], s["ef"], B, 0.9, 1.0, s["codes"], s["scales"])
    cc = [s["codes"][j * n1 // 2:(j + 1) * n1 // 2] for j in range(P1)]
    ss = [s["scales"][j * n1 // B:(j + 1) * n1 // B] for j in range(P1)]
    zq.zq_dequant_reduce(cc, ss, n1, B, 1.0, rq_codes=s["rqc"], rq_scales=s["rqs"], rq_ef=s["rqe"],
                         rq_beta_e=0.9, rq_beta_r=1.0)
    c2 = [s["rqc"][j * n2 // 2:(j + 1) * n2 // 2] for j in range(P2)]
    s2 = [s["rqs"][j * n2 // B:(j + 1) * n2 // B] for j in range(P2)]
    zq.zq_dequant_reduce(c2, s2, n2, B, 1.0 / (P1 * P2), out=s["out2"])
    zq.zq_quant_int8(s["w"], 2048, s["c8"], s["s8"])
    zq.zq_dequant_int8(s["c8"], s["s8"], 2048, s["wd"])
    zq.zq_sr_accumulate(s["dst"], s["src"], seed=1234, counter_base=77)
    zq.zq_sr_accumulate_batched(tables["sr"], zero_src=True)
    zq.zq_quantize_ef_int4_batched(tables["efq"], B, 0.9, 1.0)


def make_tables(zq, s):
    # reduced buffer of 4 shards; this rank (2) reads shard 2 (offsets are multiples of 8)
    sr = zq.SrSegmentTable([(d, r, d.numel(), 2 * d.numel(), 55 + i, 3 * i)
                            for i, (d, r) in enumerate(zip(s["dst_b"], s["red_b"]))])
    cuts = [(0, 128 * 30), (128 * 30, 128 * 30 + 1001), (128 * 30 + 1024, 9000)]
    segs = []
    for a, b in cuts:
        segs.append((s["bg"][a:b], s["bef"][a:b], s["bc"][a // 2:(b + 1) // 2],
                     s["bs"][a // B:a // B + -(-(b - a) // B)]))
    return {"sr": sr, "efq": zq.EfqSegmentTable(segs, B)}


def perturb(s, k):
    """Eager work between replays: new gradients, weights and sources (the
    reduced buffers were cleared by the batched SR and get new contents)."""
    s["g"].mul_(-1.5 if k % 2 else 0.75)
    s["w"].mul_(1.25)
    s["src"].mul_(0.5)
    s["bg"].mul_(-2.0)
    for r in s["red_b"]:
        r.copy_(torch.arange(r.numel(), device="cuda", dtype=torch.float32).mul_(1e-4).sin_()
                .to(torch.bfloat16))


def bits(t):
    if t.dtype in (torch.float32,):
        return t.view(torch.int32)
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    return t


def assert_sets_equal(a, b, what):
    for k in a:
        xs, ys = (a[k], b[k]) if isinstance(a[k], list) else ([a[k]], [b[k]])
        for i, (x, y) in enumerate(zip(xs, ys)):
            assert torch.equal(bits(x), bits(y)), f"{what}: {k}[{i}] differs"


def test_every_entry_point_replays_from_a_graph_like_eager():
    from weight_communication_zero_amd import zq
    A, Bs = make_set(7), make_set(7)
    assert_sets_equal(A, Bs, "identical inputs")
    tA, tB = make_tables(zq, A), make_tables(zq, Bs)
    # warm-up on a side stream (torch's capture recipe), on throw-away copies
    W = make_set(8)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(zq, W, make_tables(zq, W))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(zq, Bs, tB)
    torch.cuda.synchronize()
    assert_sets_equal(A, Bs, "capture ran nothing")
    for k in range(3):
        step(zq, A, tA)
        graph.replay()
        torch.cuda.synchronize()
        assert_sets_equal(A, Bs, f"replay {k}")
        assert int(torch.count_nonzero(bits(A["ef"]))) > 0
        perturb(A, k)
        perturb(Bs, k)
        torch.cuda.synchronize()
    # the requant EF and the per-parameter EF buffers evolved over 3 steps
    assert int(torch.count_nonzero(bits(Bs["rqe"]))) > 0
    assert int(torch.count_nonzero(bits(Bs["bef"]))) > 0
    assert np.isfinite(Bs["out2"].cpu().numpy()).all()
