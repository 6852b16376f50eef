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
