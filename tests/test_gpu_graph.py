"""libreduce calls captured into a HIP graph and replayed.

A caller whose hot loop is launch-bound can capture library calls in a HIP
graph once the stream has made its first call (that call creates the
stream's workspace, which allocates; later calls only enqueue kernels and
record no memset).  The graph here holds one call of every kind -- the
two-kernel 1-D reductions, the fused call, the atomic variant without
accum (its identity fill is a kernel), the row kernels including the
split-row form with its second pass, the column product and the column sum
with accum -- and is replayed several times with fresh input values copied
in between and eager library calls on another stream in between.  Every
replay must give the eager results: the same bits for the deterministic
calls, the sum tolerance for the atomic sum."""
import pytest

import oracle
import workloads
from gpu_helpers import check_sum, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def red():
    import fp32_reductions_amd as red
    return red


def test_graph_replay_matches_eager(red):
    say("graph capture of library calls and 4 replays")
    dev = "cuda"
    x = torch.empty(1 << 20 | 3, dtype=torch.float32, device=dev)
    rows_a = torch.empty((512, 300), dtype=torch.float32, device=dev)     # lanes per row
    rows_b = torch.empty((16, 200000), dtype=torch.float32, device=dev)   # split rows, 2nd pass
    tile = torch.empty((1024, 4096), dtype=torch.float32, device=dev)
    cols = torch.empty((300, 5000), dtype=torch.float32, device=dev)

    def fill(seed):
        x.copy_(torch.from_numpy(workloads.uniform_f32(seed, x.numel())))
        rows_a.copy_(torch.from_numpy(workloads.uniform_f32(seed + 1, rows_a.shape)))
        rows_b.copy_(torch.from_numpy(workloads.uniform_f32(seed + 2, rows_b.shape)))
        tile.copy_(torch.from_numpy(workloads.uniform_f32(seed + 3, tile.shape, 0.999, 1.001)))
        cols.copy_(torch.from_numpy(workloads.uniform_f32(seed + 4, cols.shape)))

    def make_outs():
        return {"sum": torch.zeros(1, device=dev), "max": torch.zeros(1, device=dev),
                "fused": torch.zeros(3, device=dev), "atomic": torch.zeros(1, device=dev),
                "rows_a": torch.zeros(512, device=dev), "rows_b": torch.zeros(16, device=dev),
                "prod": torch.zeros(4096, device=dev), "cols": torch.zeros(5000, device=dev)}

    def calls(o):
        red.sum_f32(x, o["sum"])
        red.max_f32(x, o["max"])
        red.sum_max_min_f32(x, o["fused"])
        red.sum_f32_atomic(x, o["atomic"])
        red.sum_rows_f32(rows_a, o["rows_a"])
        red.min_rows_f32(rows_b, o["rows_b"])
        red.colprod_f32(tile, o["prod"])
        red.sum_cols_f32(cols, o["cols"], accum=True)

    cap = torch.cuda.Stream()
    eager_stream = torch.cuda.Stream()
    fill(500)
    graph_out = make_outs()
    torch.cuda.synchronize()
    with torch.cuda.stream(cap):      # first call on the stream: workspace created
        calls(graph_out)
    cap.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        calls(graph_out)
    torch.cuda.synchronize()

    for rep in range(4):
        fill(600 + 10 * rep)
        for k, t in graph_out.items():
            t.fill_(0.5 if k == "cols" else 0.0)  # accum base for the column sum
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = make_outs()
        eager["cols"].fill_(0.5)
        torch.cuda.synchronize()
        with torch.cuda.stream(eager_stream):
            calls(eager)
        eager_stream.synchronize()
        for k in graph_out:
            got, want = host(graph_out[k]), host(eager[k])
            if k == "atomic":
                s, a = oracle.get().sum_f32(host(x))
                check_sum(got[0], s, a, "graph replay %d atomic sum" % rep)
            else:
                assert got.tobytes() == want.tobytes(), ("replay", rep, k)
    say("graph replays match eager calls")


def test_graph_replay_tile_layouts(red):
    """The same check for the layouts chosen by tile and row shape: narrow
    rows read as 16-byte vectors and as elements (each with a second pass
    over several row shares), a short, wide tile on the wide-strip kernel,
    a tile whose rows do not start on 128-byte lines (XCD-contiguous order,
    rows shared with a second pass), a tile of 257 column blocks whose rows
    are split 6 ways (second pass), rows of 3 elements (eight per thread)
    and padded rows of 20 staged as one span."""
    say("graph capture of tile-layout calls and 4 replays")
    dev = "cuda"
    narrow_v = torch.empty((100000, 16), dtype=torch.float32, device=dev)
    narrow_e = torch.empty((50000, 15), dtype=torch.bfloat16, device=dev)
    wide = torch.empty((3, 2_100_032), dtype=torch.float32, device=dev)
    unal = torch.empty((20000, 1001), dtype=torch.float32, device=dev)
    short = torch.empty((200000, 3), dtype=torch.float32, device=dev)
    span = torch.empty((50000, 24), dtype=torch.float32, device=dev)
    bal = torch.empty((1000, 16448), dtype=torch.float32, device=dev)

    def fill(seed):
        narrow_v.copy_(torch.from_numpy(workloads.uniform_f32(seed, narrow_v.shape, 0.9999, 1.0001)))
        narrow_e.copy_(torch.from_numpy(workloads.uniform_f32(seed + 1, narrow_e.shape, 0.999, 1.001)))
        wide.copy_(torch.from_numpy(workloads.uniform_f32(seed + 2, wide.shape, 0.5, 1.5)))
        unal.copy_(torch.from_numpy(workloads.uniform_f32(seed + 3, unal.shape)))
        short.copy_(torch.from_numpy(workloads.uniform_f32(seed + 4, short.shape)))
        span.copy_(torch.from_numpy(workloads.uniform_f32(seed + 5, span.shape)))
        bal.copy_(torch.from_numpy(workloads.uniform_f32(seed + 6, bal.shape)))

    def make_outs():
        return {"narrow_v": torch.zeros(16, device=dev),
                "narrow_e": torch.zeros(15, dtype=torch.bfloat16, device=dev),
                "wide": torch.zeros(2_100_032, device=dev),
                "unal": torch.zeros(1000, device=dev),
                "short": torch.zeros(200000, device=dev),
                "span": torch.zeros(50000, device=dev),
                "bal": torch.zeros(16448, device=dev)}

    def calls(o):
        red.colprod_f32(narrow_v, o["narrow_v"])
        red.colprod_bf16(narrow_e, o["narrow_e"])
        red.colprod_f32(wide, o["wide"])
        red.sum_cols_f32(unal, o["unal"], C=1000, accum=True)
        red.sum_rows_f32(short, o["short"], accum=True)
        red.max_rows_f32(span, o["span"], n=20)
        red.sum_cols_f32(bal, o["bal"], accum=True)

    cap = torch.cuda.Stream()
    eager_stream = torch.cuda.Stream()
    fill(700)
    graph_out = make_outs()
    torch.cuda.synchronize()
    with torch.cuda.stream(cap):      # first call on the stream: workspace created
        calls(graph_out)
    cap.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        calls(graph_out)
    torch.cuda.synchronize()

    accum_base = {"unal": 0.25, "short": -1.5, "bal": 2.0}
    for rep in range(4):
        fill(800 + 10 * rep)
        for k, t in graph_out.items():
            t.fill_(accum_base.get(k, 0.0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = make_outs()
        for k, v in accum_base.items():
            eager[k].fill_(v)
        torch.cuda.synchronize()
        with torch.cuda.stream(eager_stream):
            calls(eager)
        eager_stream.synchronize()
        for k in graph_out:
            got, want = graph_out[k], eager[k]
            if got.dtype == torch.bfloat16:
                got, want = got.view(torch.int16), want.view(torch.int16)
            assert host(got).tobytes() == host(want).tobytes(), ("replay", rep, k)
    say("tile-layout graph replays match eager calls")
