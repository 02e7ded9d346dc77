"""The run guarantees the headers state: `run` calls are asynchronous,
allocate nothing and never synchronize, so a HIP graph can capture them, and
they honour the stream they are given (gpu).

Each entry point is captured into a graph (torch.cuda.graph, which captures
the calls' own kernels on its capture stream), replayed several times with
eager work and synchronizations between the replays, and every replay is
compared bit for bit with the eager result; the same calls on a non-default
stream give the same bits (Detent, §4.1: a new batch never triggers a
recompile, so the selection can sit inside a captured step)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, assert_bits_equal, to_dev

pytestmark = pytest.mark.gpu


def bits(t):
    return t.detach().contiguous().view(torch.int32).cpu().numpy()


def check_graph_and_stream(fn, outs, what, replays=3):
    """fn() writes into the preallocated tensors `outs`."""
    fn()
    torch.cuda.synchronize()
    eager = [bits(o) for o in outs]
    # a side stream at the default priority
    side = torch.cuda.Stream()
    for o in outs:
        o.fill_(float("nan") if o.is_floating_point() else 0)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        fn()
    side.synchronize()
    for o, e in zip(outs, eager):
        assert_bits_equal(bits(o), e, "%s on a side stream" % what)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for r in range(replays):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 0)
        scratch.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert_bits_equal(bits(o), e, "%s graph replay %d" % (what, r))


@pytest.mark.parametrize("m", [1, 48, 300, 2100])
def test_dense_run_graph_and_stream(gpu, m):
    n, k = 2048, 2048
    g = gpu.Gemm(to_dev(synth.normal_bf16(500, (n, k), 0.02)))
    x = to_dev(synth.normal_bf16(501, (m, k)))
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    check_graph_and_stream(lambda: g(x, out=y), [y], "bi_gemm_run M=%d (%s)" % (m, g.kernel_name(m)))


@pytest.mark.parametrize("kind", ["stream_mb2_n2", "stream_mb4_n4"])
def test_wide_strip_streamer_graph(gpu, kind):
    """The weight streamer over 32- and 64-column strips, forced by the pin's
    tiling, captured and replayed, and on a side stream."""
    n, k = 2048, 2048
    g = gpu.Gemm(to_dev(synth.normal_bf16(504, (n, k), 0.02)),
                 pin={"splits": 1, "stream_max_m": 0, "tiling": [(None, kind)]})
    x = to_dev(synth.normal_bf16(505, (100, k)))
    y = torch.empty((100, n), dtype=torch.float32, device=DEV)
    check_graph_and_stream(lambda: g(x, out=y), [y], "bi_gemm_run %s (%s)" % (kind, g.kernel_name(100)))


def test_split_tree_graph(gpu):
    """An S = 4 tree enqueues four kernels; all are captured in order."""
    n, k = 1024, 4096
    g = gpu.Gemm(to_dev(synth.normal_bf16(502, (n, k), 0.02)), pin={"splits": 4, "stream_max_m": 16})
    x = to_dev(synth.normal_bf16(503, (200, k)))
    y = torch.empty((200, n), dtype=torch.float32, device=DEV)
    check_graph_and_stream(lambda: g(x, out=y), [y], "S=4 M=200")


@pytest.mark.parametrize("t", [1, 256])
def test_grouped_run_graph_and_stream(gpu, t):
    e, n, k = 32, 1024, 2048
    gg = gpu.GroupedGemm(to_dev(synth.normal_bf16(504, (e, n, k), 0.02)))
    tok, off, _ = synth.moe_routing(505 + t, t, e, 4)
    x = to_dev(synth.normal_bf16(506, (len(tok), k)))
    offd = torch.as_tensor(off, device=DEV)
    y = torch.empty((len(tok), n), dtype=torch.float32, device=DEV)
    check_graph_and_stream(lambda: gg(x, offd, out=y), [y], "grouped T=%d" % t)


# T = 3: routing and grouping in one kernel, SwiGLU in the streaming up
# projection; T = 12: the two routing kernels, the same up projection;
# T = 512: the four-wave up projection's SwiGLU epilogue
@pytest.mark.parametrize("t", [3, 12, 512])
def test_moe_layer_graph_and_stream(gpu, t):
    E, H, I, k = 16, 512, 256, 4
    wr = to_dev(synth.normal_bf16(510, (E, H), 0.02))
    wu = to_dev(synth.normal_bf16(511, (E, 2 * I, H), 0.02))
    wd = to_dev(synth.normal_bf16(512, (E, H, I), 0.02))
    layer = gpu.MoeLayer(wr, wu, wd, k=k, max_tokens=512)
    x = to_dev(synth.normal_bf16(513, (t, H)))
    y = torch.empty((t, H), dtype=torch.float32, device=DEV)
    check_graph_and_stream(lambda: layer(x, out=y), [y], "MoE layer T=%d" % t)


def test_decode_attention_graph_and_stream(gpu):
    hq, hkv, d = 32, 8, 128
    lengths = synth.decode_lengths(520, 40, 600.0, 0.8, 1, 3000)
    st = np.zeros(len(lengths) + 1, np.int32)
    st[1:] = np.cumsum(lengths)
    ntok = int(st[-1])
    q = to_dev(synth.normal_bf16(521, (len(lengths), hq, d)))
    kk = to_dev(synth.normal_bf16(522, (ntok, hkv, d)))
    vv = to_dev(synth.normal_bf16(523, (ntok, hkv, d)))
    std = torch.as_tensor(st, device=DEV)
    att = gpu.DecodeAttention(hq, hkv, 256, len(lengths), 3000)
    out = torch.empty((len(lengths), hq, d), dtype=torch.float32, device=DEV)
    check_graph_and_stream(lambda: att(q, kk, vv, std, out=out), [out], "decode attention")


def test_fused_norm_gemm_graph_and_stream(gpu):
    n, k, m = 1024, 2048, 130
    g = gpu.Gemm(to_dev(synth.normal_bf16(530, (n, k), 0.02)))
    x = to_dev(synth.normal_bf16(531, (m, k)))
    gain = to_dev(synth.normal_bf16(532, (k,), 0.5))
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    r = torch.empty(m, dtype=torch.float32, device=DEV)
    check_graph_and_stream(lambda: g.rmsnorm_run(x, gain, 1e-5, out=y, rstd=r), [y, r], "RMSNorm+GEMM M=%d" % m)


def test_concurrent_split_pin_graph(gpu):
    """A pin whose splits run concurrently uses the handle's workspace; the
    captured call replays to the same bits."""
    n, k = 1024, 4096
    g = gpu.Gemm(to_dev(synth.normal_bf16(540, (n, k), 0.02)),
                 pin={"splits": 2, "stream_max_m": 0, "tiling": [(512, "tiled_64x64+cs"), (None, "tiled_64x64")]})
    x = to_dev(synth.normal_bf16(541, (300, k)))
    y = torch.empty((300, n), dtype=torch.float32, device=DEV)
    assert g.kernel_name(300).endswith("concurrent splits")
    check_graph_and_stream(lambda: g(x, out=y), [y], "S=2 concurrent M=300")
