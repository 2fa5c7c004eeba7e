"""Checkpoint and resume.  Everything the method carries from one step to
the next lives in caller-owned device buffers: the error-feedback buffer of
every sender, the receiver's requant error-feedback buffer (LoCo's
compensation state, "Merge LoCo with Zero++", review thread) and the bf16
shard accumulator of llm.c's ZeRO-2 loop ("Zero 2 #593", review of
llmc/zero.cuh).  A run of 10 steps split 5 + 5, with that state copied to
the host, serialised, loaded into fresh device buffers and continued, must
end bit for bit where the straight 10-step run ends.

One step, for one receiving rank of 8: every simulated rank quantizes its
gradient with EF, the receiver reduces its chunk from all 8 with requant EF,
dequantizes the requantized chunk (1-peer reduce, alpha = 1/8), rounds it
to bf16 and SR-accumulates it into the shard with a per-step seed."""
import io

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


P, B, RECV = 8, 128, 3
NC = B * 997            # chunk: 127,616 elements
N = P * NC              # per-rank gradient
STEPS, SPLIT = 10, 5


def fresh_state():
    z = lambda n, dt=torch.float32: torch.zeros(n, dtype=dt, device="cuda")
    return {"ef": [z(N) for _ in range(P)], "rq_ef": z(NC), "acc": z(NC, torch.bfloat16)}


def gradient(r, t):
    g = torch.Generator(device="cuda").manual_seed(1000 * t + r)
    return torch.randn(N, device="cuda", generator=g) * (1e-3 * (1 + r % 3))


def step(zq, st, t):
    codes = [torch.empty(N // 2, dtype=torch.uint8, device="cuda") for _ in range(P)]
    scales = [torch.empty(N // B, device="cuda") for _ in range(P)]
    for r in range(P):
        zq.zq_quantize_ef_int4(gradient(r, t), st["ef"][r], B, 0.9, 1.0, codes[r], scales[r])
    cc = [c[RECV * NC // 2:(RECV + 1) * NC // 2] for c in codes]
    ss = [s[RECV * NC // B:(RECV + 1) * NC // B] for s in scales]
    rqc = torch.empty(NC // 2, dtype=torch.uint8, device="cuda")
    rqs = torch.empty(NC // B, device="cuda")
    zq.zq_dequant_reduce(cc, ss, NC, B, 1.0, rq_codes=rqc, rq_scales=rqs, rq_ef=st["rq_ef"],
                         rq_beta_e=0.9, rq_beta_r=1.0)
    out = torch.empty(NC, device="cuda")
    zq.zq_dequant_reduce([rqc], [rqs], NC, B, 1.0 / P, out=out)
    zq.zq_sr_accumulate(st["acc"], out.to(torch.bfloat16), seed=4242 + t, counter_base=RECV * NC)
    return out


def flat(st):
    return st["ef"] + [st["rq_ef"], st["acc"]]


def save(st) -> bytes:
    buf = io.BytesIO()
    torch.save({"ef": [e.cpu() for e in st["ef"]], "rq_ef": st["rq_ef"].cpu(), "acc": st["acc"].cpu()},
               buf)
    return buf.getvalue()


def load(blob: bytes):
    d = torch.load(io.BytesIO(blob), weights_only=True)
    return {"ef": [e.cuda() for e in d["ef"]], "rq_ef": d["rq_ef"].cuda(), "acc": d["acc"].cuda()}


def same_bits(a, b):
    v = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(v), b.view(v))


def test_split_run_with_saved_state_equals_straight_run():
    from weight_communication_zero_amd import zq
    straight = fresh_state()
    for t in range(STEPS):
        last_straight = step(zq, straight, t)

    first = fresh_state()
    for t in range(SPLIT):
        step(zq, first, t)
    torch.cuda.synchronize()
    blob = save(first)
    del first
    torch.cuda.empty_cache()
    resumed = load(blob)
    for t in range(SPLIT, STEPS):
        last_resumed = step(zq, resumed, t)
    torch.cuda.synchronize()

    assert same_bits(last_straight, last_resumed), "last step's reduced chunk differs"
    for i, (a, b) in enumerate(zip(flat(straight), flat(resumed))):
        assert same_bits(a, b), f"state buffer {i} differs after resume"
        assert int(torch.count_nonzero(a)) > 0, f"state buffer {i} never changed"


def test_resume_from_a_different_step_changes_the_result():
    """The state does carry information: resuming the second half from the
    5-step state of a run with other gradients must not land on the
    straight run's end."""
    from weight_communication_zero_amd import zq
    straight = fresh_state()
    for t in range(STEPS):
        step(zq, straight, t)
    other = fresh_state()
    for t in range(SPLIT):
        step(zq, other, t + 100)
    for t in range(SPLIT, STEPS):
        step(zq, other, t)
    torch.cuda.synchronize()
    assert not same_bits(straight["acc"], other["acc"])
    assert not same_bits(straight["rq_ef"], other["rq_ef"])
