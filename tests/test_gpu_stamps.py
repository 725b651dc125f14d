"""The instrumented build (libbitnet_i2s_stamps.so): the same results as the
product library, and one sane [start, end] stamp pair per decode launch."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture
def bn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_i2_amd as bn
    bn.load()
    yield bn
    bn.use_library("main")


def _case(bn, synth, M, K, seed):
    rng = np.random.default_rng(seed)
    W = torch.from_numpy(synth.ternary(rng, M, K)).cuda()
    x = torch.from_numpy(synth.tokens_bf16(rng, 1, K).view(np.int16)).cuda().view(torch.bfloat16)
    return bn.pack(W), 0.05, x


def test_stamped_launches_match_the_product_build(bn):
    from ternary_weight_i2_amd import synth
    shapes = [(256, 512), (2560, 2560), (640, 6912), (4097, 1024)]
    cases = [_case(bn, synth, M, K, 900 + i) for i, (M, K) in enumerate(shapes)]

    def run():
        outs = []
        for P, a, x in cases:
            M = P.shape[0]
            d = torch.empty((1, M), dtype=torch.int32, device="cuda")
            y = torch.empty((1, M), dtype=torch.float32, device="cuda")
            bn.linear(x, [(P, a)], out=[(d, y)])
            outs.append((d, y))
        torch.cuda.synchronize()
        return [(d.cpu().numpy(), y.cpu().numpy()) for d, y in outs]

    ref = run()
    bn.use_library("stamps")
    bn.stamps_reset(rewind=True)
    got = run()
    pairs = bn.stamps_read(64)
    for (d0, y0), (d1, y1) in zip(ref, got):
        assert np.array_equal(d0, d1)
        assert np.array_equal(y0.view(np.int32), y1.view(np.int32))
    assert len(pairs) == len(cases)            # one fused launch per call at N = 1
    for s, e in pairs:
        assert 0 < e - s < 100_000_000         # under a second of 10 ns ticks
    starts = [s for s, _ in pairs]
    assert starts == sorted(starts)            # one stream: launches in order
