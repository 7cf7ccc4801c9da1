"""The library's calls inside a captured HIP graph: every call only launches
kernels on the caller's stream (no allocation, no memset, no
synchronization), so a graph of a quantized layer step replays correctly.
The graph is replayed several times on changing inputs, with eager work in
between, and every replay is compared bit for bit with the same calls run
eagerly."""
import numpy as np
import pytest

from nvfp4_bit_block_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch
    assert torch.cuda.is_available()
    import nvfp4_bit_block_amd as m
    m.lib()
    return m


def test_graph_replays_match_eager(nv):
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(61)
    signs = synth.signs_from_rng(rng)
    T, D, O = 512, 256, 384
    X = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    W = torch.empty((O, D), dtype=torch.bfloat16, device=dev)
    dY = torch.empty((T, O), dtype=torch.bfloat16, device=dev)

    def bufs(rows, cols, rnd, axis):
        R, K = (rows, cols) if axis == 0 else (cols, rows)
        q = nv.QTensor(torch.empty((R, K // 2), dtype=torch.uint8, device=dev),
                       torch.empty((R, K // 16), dtype=torch.uint8, device=dev),
                       torch.empty(1, dtype=torch.float32, device=dev))
        return q, torch.empty(nv.workspace_size(rows, cols, rnd, axis), dtype=torch.uint8, device=dev)

    amax = torch.empty(1, dtype=torch.float32, device=dev)

    def step(b):
        """A layer's quantized step: column-wise MS-EDEN of X handing max|X| to
        its row-wise RTN, RTN of W, Y = X W^T, MS-EDEN of dY along rows, dX."""
        nv.quantize_nvfp4(X, rounding="mseden", axis=1, rht_signs=signs, seed=3, out=b["xc"][0],
                          workspace=b["xc"][1], amax_out=amax)
        nv.quantize_nvfp4(X, out=b["x"][0], workspace=b["x"][1], amax_in=amax)
        nv.quantize_nvfp4(W, out=b["w"][0], workspace=b["w"][1])
        nv.gemm_nvfp4(b["x"][0], b["w"][0], out=b["y"])
        nv.quantize_nvfp4(dY, rounding="mseden", rht_signs=signs, seed=4, out=b["dy"][0], workspace=b["dy"][1])
        nv.quantize_nvfp4(W, rounding="mseden", axis=1, rht_signs=signs, seed=5, out=b["wc"][0],
                          workspace=b["wc"][1])
        nv.gemm_nvfp4(b["dy"][0], b["wc"][0], out=b["dx"])
        # Y once more, coded as NVFP4 by the GEMM, with max|Y| (cleared by
        # the call's own kernel: the buffer holds 1e30 before every replay)
        nv.gemm_nvfp4_rtn(b["x"][0], b["w"][0], yts, amax_out=b["ymax"], out=b["yq"])

    yts = torch.full((1,), 6e-4, dtype=torch.float32, device=dev)

    def make():
        return {"xc": bufs(T, D, "mseden", 1), "x": bufs(T, D, "rtn", 0), "w": bufs(O, D, "rtn", 0),
                "dy": bufs(T, O, "mseden", 0), "wc": bufs(O, D, "mseden", 1),
                "y": torch.empty((T, O), dtype=torch.float32, device=dev),
                "dx": torch.empty((T, D), dtype=torch.float32, device=dev),
                "yq": nv.QTensor(torch.empty((T, O // 2), dtype=torch.uint8, device=dev),
                                 torch.empty((T, O // 16), dtype=torch.uint8, device=dev), yts),
                "ymax": torch.empty(1, dtype=torch.float32, device=dev)}

    def fill(seed):
        r = np.random.default_rng(seed)
        X.copy_(torch.from_numpy(r.standard_normal((T, D), dtype=np.float32)).to(torch.bfloat16))
        W.copy_(torch.from_numpy(0.02 * r.standard_normal((O, D), dtype=np.float32)).to(torch.bfloat16))
        dY.copy_(torch.from_numpy(1e-3 * r.standard_normal((T, O), dtype=np.float32)).to(torch.bfloat16))

    gb, eb = make(), make()
    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gb)                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb)

    def tensors(b):
        out = []
        for k in ("xc", "x", "w", "dy", "wc"):
            q = b[k][0]
            out += [q.codes, q.scales, q.tensor_scale]
        return out + [b["y"], b["dx"], b["yq"].codes, b["yq"].scales, b["ymax"]]

    for i in range(4):
        fill(100 + i)
        gb["ymax"].fill_(1e30)
        eb["ymax"].fill_(1e30)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in tensors(gb)]
        assert 0.0 < float(gb["ymax"].cpu()[0]) < 1e29, f"replay {i}: max|Y| was not cleared"
        X.mul_(1.0)                               # eager work between replays
        step(eb)
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(got, tensors(eb))):
            assert torch.equal(a, b), f"replay {i}: output {j} differs from the eager calls"
