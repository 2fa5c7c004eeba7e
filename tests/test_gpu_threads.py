"""The C ABI is reentrant: it keeps no state between calls, so host
threads calling it at the same time, each on its own stream, get exactly
what the same calls give from one thread.  Four threads each run one job
of the concurrent-streams test (EF int4 quantize, the 8-way reduce with
requant EF, qwZ int8 quantize and dequantize, SR accumulate with its
source halved between rounds) 4 times on their own stream; the same jobs on
a second set of buffers run one after another on one stream.  ctypes
releases the interpreter lock during each foreign call, so the library's
host-side validation and launch code runs concurrently."""
import threading

import pytest
import torch

from tests.test_gpu_streams import buffers, jobs, same

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_communication_zero_amd  # noqa: F401  (fails loudly if libzq.so is missing)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def test_threads_on_their_own_streams_match_one_thread():
    from weight_communication_zero_amd import zq
    A, S = buffers(23), buffers(23)
    rounds = 4
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(4)

    def run(stream, job):
        try:
            torch.cuda.set_device(0)
            start.wait(timeout=60)
            with torch.cuda.stream(stream):
                for _ in range(rounds):
                    job()
        except BaseException as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(st, job), daemon=True)
               for st, job in zip(streams, jobs(zq, A))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for job in jobs(zq, S):
        for _ in range(rounds):
            job()
    torch.cuda.synchronize()
    for k in A:
        assert same(A[k], S[k]), f"{k} differs between threaded and single-thread calls"
