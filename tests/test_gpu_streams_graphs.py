"""The C ABI on a caller's stream, under HIP graph capture, and in place.

Every entry point takes the caller's stream and allocates nothing, so the
whole path can run on a side stream and be captured into a graph.  These
tests check both against the CPU oracle: work launched on a non-default
stream, and a captured quantize -> 4-stream reduce -> unpack pipeline
replayed several times with new inputs written eagerly between the replays
(each replay must compute from the inputs it finds, and no replay may reuse
an earlier result); the two in-place uses the header allows (the reduce
into its first stream, the all-reduce emulation into one of its messages);
and host threads calling the library at once, each on its own stream.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import reduction_codec_amd as rca

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FMTS = ["int4", "int3", "fp8", "mxfp4"]
N = 3 * 2048 + 517                       # several tiles and a ragged tail


def bf16_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)


def message(seed: int) -> np.ndarray:
    return datagen.narrow(datagen.normal_outliers(seed, N, 20.0, 0.001), "bf16")


def oracle_pipeline(fmt: str, x: np.ndarray, peers):
    c = oracle.CODECS[fmt]
    p0 = oracle.quantize_pack(c, x, dtype=oracle.DT_BF16)
    out, _ = oracle.dequant_reduce_requant(c, [p0] + peers, N)
    y = oracle.unpack_dequant(c, out, N, oracle.DT_BF16)
    return p0, out, y


@pytest.mark.parametrize("fmt", FMTS)
def test_side_stream_matches_oracle(fmt):
    print(f"case side stream {fmt}", flush=True)
    x = message(11)
    peers = [oracle.quantize_pack(oracle.CODECS[fmt], message(20 + j), dtype=oracle.DT_BF16) for j in range(3)]
    ref_p0, ref_out, ref_y = oracle_pipeline(fmt, x, peers)
    side = torch.cuda.Stream(device=DEV)
    xd = bf16_dev(x)
    pd = [torch.from_numpy(p).to(DEV) for p in peers]
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        p0 = rca.quantize_pack(xd, rca.CODECS[fmt], stream=side)
        out, _ = rca.dequant_reduce_requant([p0] + pd, rca.CODECS[fmt], N, stream=side)
        y = rca.unpack_dequant(out, rca.CODECS[fmt], N, torch.bfloat16, stream=side)
    side.synchronize()
    assert np.array_equal(p0.cpu().numpy(), ref_p0)
    assert np.array_equal(out.cpu().numpy(), ref_out)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref_y)


@pytest.mark.parametrize("fmt", FMTS)
def test_graph_replays_follow_their_inputs(fmt):
    print(f"case graph replays {fmt}", flush=True)
    codec = rca.CODECS[fmt]
    pb = rca.packed_bytes(codec, N)
    x = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    peers = [torch.empty(pb, dtype=torch.uint8, device=DEV) for _ in range(3)]
    p0 = torch.empty(pb, dtype=torch.uint8, device=DEV)
    out = torch.empty(pb, dtype=torch.uint8, device=DEV)
    y = torch.empty(N, dtype=torch.bfloat16, device=DEV)

    def load(round_: int):
        xs = message(100 + round_)
        ps = [oracle.quantize_pack(oracle.CODECS[fmt], message(200 + 10 * round_ + j), dtype=oracle.DT_BF16)
              for j in range(3)]
        x.copy_(bf16_dev(xs))
        for dst, p in zip(peers, ps):
            dst.copy_(torch.from_numpy(p).to(DEV))
        torch.cuda.synchronize()
        return xs, ps

    load(0)
    # warm up outside capture, then capture the pipeline on a side stream
    rca.quantize_pack(x, codec, out=p0)
    rca.dequant_reduce_requant([p0] + peers, codec, N, out=out)
    rca.unpack_dequant(out, codec, N, torch.bfloat16, out=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rca.quantize_pack(x, codec, out=p0)
        rca.dequant_reduce_requant([p0] + peers, codec, N, out=out)
        rca.unpack_dequant(out, codec, N, torch.bfloat16, out=y)
    torch.cuda.synchronize()

    for round_ in range(1, 4):
        xs, ps = load(round_)
        # unrelated eager work between the replays
        scratch = rca.quantize_pack(bf16_dev(message(999)), codec)
        torch.cuda.synchronize()
        del scratch
        out.fill_(0xA5)
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_p0, ref_out, ref_y = oracle_pipeline(fmt, xs, ps)
        assert np.array_equal(p0.cpu().numpy(), ref_p0), f"replay {round_}: packed message"
        assert np.array_equal(out.cpu().numpy(), ref_out), f"replay {round_}: reduced stream"
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref_y), f"replay {round_}: unpack"


@pytest.mark.parametrize("fmt", FMTS)
def test_reduce_in_place_into_the_first_stream(fmt):
    """rc_dequant_reduce_requant with out == ins[0]: the header allows it
    (every tile is read in full before it is written)."""
    print(f"case in-place reduce {fmt}", flush=True)
    c = oracle.CODECS[fmt]
    streams = [oracle.quantize_pack(c, message(300 + j), dtype=oracle.DT_BF16) for j in range(4)]
    ref, _ = oracle.dequant_reduce_requant(c, streams, N)
    devs = [torch.from_numpy(s).to(DEV) for s in streams]
    rca.dequant_reduce_requant(devs, rca.CODECS[fmt], N, out=devs[0])
    torch.cuda.synchronize()
    assert np.array_equal(devs[0].cpu().numpy(), ref)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("two_shot", [True, False])
def test_allreduce_emulate_in_place(fmt, two_shot):
    """rc_allreduce_emulate with out == msgs[1] (the usual in-place
    all-reduce): same result as into a separate buffer."""
    print(f"case in-place allreduce {fmt} two_shot={two_shot}", flush=True)
    msgs = [message(400 + j) for j in range(3)]
    ref, _ = oracle.allreduce_emulate(oracle.CODECS[fmt], msgs, oracle.DT_BF16, two_shot=two_shot)
    devs = [bf16_dev(m) for m in msgs]
    rca.allreduce_emulate(devs, rca.CODECS[fmt], two_shot=two_shot, out=devs[1])
    torch.cuda.synchronize()
    assert np.array_equal(devs[1].view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_stream_argument_without_switching_streams(fmt):
    """Work enqueued on a side stream through the `stream` argument only (the
    current stream stays the default one): outputs the binding allocates are
    recorded on the side stream and come out equal to the oracle's."""
    print(f"case stream argument {fmt}", flush=True)
    x = message(61)
    peers = [oracle.quantize_pack(oracle.CODECS[fmt], message(70 + j), dtype=oracle.DT_BF16) for j in range(3)]
    ref_p0, ref_out, ref_y = oracle_pipeline(fmt, x, peers)
    side = torch.cuda.Stream(device=DEV)
    xd = bf16_dev(x)
    pd = [torch.from_numpy(p).to(DEV) for p in peers]
    side.wait_stream(torch.cuda.current_stream())
    p0 = rca.quantize_pack(xd, rca.CODECS[fmt], stream=side)
    out, _ = rca.dequant_reduce_requant([p0] + pd, rca.CODECS[fmt], N, stream=side)
    y = rca.unpack_dequant(out, rca.CODECS[fmt], N, torch.bfloat16, stream=side)
    side.synchronize()
    assert np.array_equal(p0.cpu().numpy(), ref_p0)
    assert np.array_equal(out.cpu().numpy(), ref_out)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref_y)


def test_host_threads_on_their_own_streams():
    """The library keeps no state, so host threads may call it at once: four
    threads, each on its own stream with its own codec and data, run the
    quantize -> 4-stream reduce -> unpack pipeline ten times over; every
    result equals the oracle's."""
    import threading

    print("case host threads", flush=True)
    refs, work = {}, {}
    for t, fmt in enumerate(FMTS):
        x = message(40 + t)
        peers = [oracle.quantize_pack(oracle.CODECS[fmt], message(50 + 4 * t + j), dtype=oracle.DT_BF16)
                 for j in range(3)]
        refs[fmt] = oracle_pipeline(fmt, x, peers)
        work[fmt] = (bf16_dev(x), [torch.from_numpy(p).to(DEV) for p in peers])
    rca.lib()                                      # loaded once, before the threads
    torch.cuda.synchronize()
    results, errors = {}, []

    def run(fmt):
        try:
            side = torch.cuda.Stream(device=DEV)
            xd, pd = work[fmt]
            c = rca.CODECS[fmt]
            with torch.cuda.stream(side):
                got = []
                for _ in range(10):
                    p0 = rca.quantize_pack(xd, c, stream=side)
                    out, _ = rca.dequant_reduce_requant([p0] + pd, c, N, stream=side)
                    y = rca.unpack_dequant(out, c, N, torch.bfloat16, stream=side)
                    got.append((p0, out, y))
            side.synchronize()
            results[fmt] = got
        except Exception as e:                     # reported by the main thread
            errors.append((fmt, repr(e)))

    threads = [threading.Thread(target=run, args=(fmt,)) for fmt in FMTS]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not errors, errors
    assert all(not th.is_alive() for th in threads)
    for fmt in FMTS:
        ref_p0, ref_out, ref_y = refs[fmt]
        for p0, out, y in results[fmt]:
            assert np.array_equal(p0.cpu().numpy(), ref_p0), fmt
            assert np.array_equal(out.cpu().numpy(), ref_out), fmt
            assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref_y), fmt
