"""The library keeps no state between calls: entry points running at the
same time on different streams (default priority) give exactly what they
give one after another.  Four independent jobs -- EF int4 quantize with its
EF buffer, the 8-way reduce with requant EF, qwZ int8 quantize and
dequantize, SR accumulate with zeroing -- are each issued 4 times in a row on
their own stream, all four streams in flight together; a second set of
buffers runs the same calls in sequence on one stream.  Every output and
in-place buffer must agree bit for bit."""
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


B, P = 128, 8
N = 1 << 22          # EF quantize elements
NC = (1 << 21) + 384  # reduce chunk (ragged tile)
N8 = (1 << 22) + 77   # int8 elements
NS = (1 << 22) + 13   # SR elements


def buffers(seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    r = lambda n, s: torch.randn(n, device="cuda", generator=g) * s
    b = {
        "g": r(N, 1e-3), "ef": r(N, 1e-5), "c": torch.zeros(N // 2, dtype=torch.uint8, device="cuda"),
        "s": torch.zeros(N // B, device="cuda"),
        "pc": torch.randint(0, 256, (P * NC // 2,), dtype=torch.uint8, device="cuda", generator=g),
        "ps": r(P * NC // B + P, 1e-4).abs(),
        "rqc": torch.zeros(NC // 2, dtype=torch.uint8, device="cuda"),
        "rqs": torch.zeros(NC // B, device="cuda"), "rqe": r(NC, 1e-6),
        "w": r(N8, 0.02).half(), "c8": torch.zeros(N8, dtype=torch.int8, device="cuda"),
        "s8": torch.zeros(-(-N8 // 2048), device="cuda"),
        "wd": torch.zeros(N8, dtype=torch.bfloat16, device="cuda"),
        "dst": torch.zeros(NS, dtype=torch.bfloat16, device="cuda"),
        "src": r(NS, 1e-2).to(torch.bfloat16),
    }
    return b


def jobs(zq, b):
    cc = [b["pc"][j * NC // 2:(j + 1) * NC // 2] for j in range(P)]
    ss = [b["ps"][j * (NC // B):(j + 1) * (NC // B)] for j in range(P)]

    def efq():
        zq.zq_quantize_ef_int4(b["g"], b["ef"], B, 0.9, 1.0, b["c"], b["s"])

    def dr():
        zq.zq_dequant_reduce(cc, ss, NC, B, 1.0, rq_codes=b["rqc"], rq_scales=b["rqs"],
                             rq_ef=b["rqe"], rq_beta_e=0.9, rq_beta_r=1.0)

    def q8():
        zq.zq_quant_int8(b["w"], 2048, b["c8"], b["s8"])
        zq.zq_dequant_int8(b["c8"], b["s8"], 2048, b["wd"])

    def sr():
        zq.zq_sr_accumulate(b["dst"], b["src"], seed=99, counter_base=5)
        b["src"].mul_(0.5)  # new source for the next round (torch kernel on the same stream)

    return [efq, dr, q8, sr]


def same(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def test_concurrent_streams_match_sequential_calls():
    from weight_communication_zero_amd import zq
    A, S = buffers(11), buffers(11)
    rounds = 4
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    for st, job in zip(streams, jobs(zq, A)):
        with torch.cuda.stream(st):
            for _ in range(rounds):
                job()
    for job in jobs(zq, S):
        for _ in range(rounds):
            job()
    torch.cuda.synchronize()
    for k in A:
        assert same(A[k], S[k]), f"{k} differs between concurrent and sequential calls"
    assert int(torch.count_nonzero(A["dst"].view(torch.int16))) > 0
