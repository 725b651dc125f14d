"""Calls enqueue on the stream they are given and keep no shared state: the same
launches issued on two streams at once (different tokens) give the results of
running them one after another."""
import pytest

from ternary_weight_i2_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_i2_amd as bn
    bn.load()
    return bn


def test_two_streams_match_sequential(bn):
    torch.cuda.set_device(0)
    mats = [(bn.pack(synth.ternary_torch(6912, 2560, 70 + i)), 0.04) for i in range(2)]
    big = bn.pack(synth.ternary_torch(640, 8192, 72))
    xs = [synth.tokens_bf16_torch(1, 2560, 80 + i) for i in range(2)]
    q16 = [bn.quant_act(synth.tokens_bf16_torch(16, 8192, 82 + i)) for i in range(2)]
    q96 = [bn.quant_act(synth.tokens_bf16_torch(96, 2560, 84 + i)) for i in range(2)]

    def work(i):
        a = bn.linear(xs[i], mats)[0]
        b = bn.gemv(big, 0.05, *q16[i])
        c = bn.gemm_group(mats, *q96[i])
        return [t for pair in a + [b] + c for t in pair]

    ref = []
    for i in range(2):
        ref.append(work(i))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [None, None]
    for rep in range(3):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                got[i] = work(i)
        torch.cuda.synchronize()
        for i in range(2):
            for t, e in zip(got[i], ref[i]):
                a = t.view(torch.int32) if t.dtype == torch.float32 else t
                b = e.view(torch.int32) if e.dtype == torch.float32 else e
                assert torch.equal(a, b), f"stream {i}, pass {rep} differs"
