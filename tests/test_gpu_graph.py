"""Launches captured in a HIP graph (as the benchmark times them) replay to the
eager results: every replay, with other eager launches and synchronisations
in between, is compared bit for bit with an eager run of the same calls."""
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


def _mats(bn, projs, seed):
    out = []
    for i, p in enumerate(projs):
        M, K = synth.SHAPES["b2"][p]
        out.append((bn.pack(synth.ternary_torch(M, K, seed + i)), 0.02 + 0.01 * i))
    return out


def _flat(outs):
    return [t for pair in outs for t in pair if t is not None]


def test_graph_replays_match_eager(bn):
    torch.cuda.set_device(0)
    groups = [_mats(bn, p, 10 * i) for i, p in
              enumerate((("q", "k", "v"), ("o",), ("gate", "up"), ("down",)))]
    tokens1 = [synth.tokens_bf16_torch(1, mats[0][0].shape[1] * 4, 50 + i)
               for i, mats in enumerate(groups)]
    q16 = bn.quant_act(synth.tokens_bf16_torch(16, 2560, 61))
    big = bn.pack(synth.ternary_torch(300, 28672, 62))
    q16big = bn.quant_act(synth.tokens_bf16_torch(16, 28672, 63))
    q128 = bn.quant_act(synth.tokens_bf16_torch(128, 2560, 64))

    # eager run: one token through the fused launches of a 2B-class layer,
    # 16 tokens through the grouped batched decode and the 16-token GEMM tiles
    # at K = 28672, 128 tokens through the grouped prefill GEMM
    outs1 = [bn.linear(x, mats)[0] for x, mats in zip(tokens1, groups)]
    outs16 = bn.gemv_group(groups[2], *q16)
    outbig = bn.gemv(big, 0.03, *q16big)
    outs128 = bn.gemm_group(groups[0], *q128)
    torch.cuda.synchronize()
    buffers = [t for o in outs1 for t in _flat(o)] + _flat(outs16) + list(outbig) + _flat(outs128)
    eager = [t.clone() for t in buffers]

    def run():
        for x, mats, o in zip(tokens1, groups, outs1):
            bn.linear(x, mats, out=o)
        bn.gemv_group(groups[2], *q16, out=outs16)
        bn.gemv(big, 0.03, *q16big, out=outbig)
        bn.gemm_group(groups[0], *q128, out=outs128)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()

    other = synth.tokens_bf16_torch(1, 2560, 99)
    for rep in range(3):
        for t in buffers:
            t.zero_()
        # unrelated eager launches between the replays
        bn.linear(other, groups[2])
        bn.gemv_group(groups[0], *q16)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(buffers, eager):
            a = t.view(torch.int32) if t.dtype == torch.float32 else t
            b = e.view(torch.int32) if e.dtype == torch.float32 else e
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
