"""Child process of test_gpu_parity.py::test_graph_capture_of_the_first_call.

The first gqe_forward calls of a fresh process are made inside HIP graph
capture: no kernel of the library has run before, so every launch attribute
the library sets on first use is set during the capture.  Each graph is then
replayed three times and must equal an eager call made afterwards, bit for
bit.  Arguments: workload names (workloads.WORKLOADS), run in order."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import torch  # noqa: E402

import workloads as W  # noqa: E402
from gpu_util import log, to_dev  # noqa: E402
from sparse_query_moe_amd import gqe  # noqa: E402


def main(names):
    for name in names:
        wl = W.WORKLOADS[name]
        log(f"[graph-first-call] {wl.description}")
        I = W.make_inputs(wl)
        dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
        cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts,
                              wl.top_k, wl.head_dim, dtype=wl.dtype, router_bias=dev["br"])
        ws_g, ws_e = gqe.alloc_workspace(cfg), gqe.alloc_workspace(cfg)
        shape = (wl.batch, wl.seq_len, wl.d_model)
        y_g = torch.zeros(shape, dtype=cfg.torch_dtype, device="cuda")
        y_e = torch.zeros(shape, dtype=cfg.torch_dtype, device="cuda")
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                            y_g, ws_g)
        gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                        y_e, ws_e)
        torch.cuda.synchronize()
        for rep in range(3):
            y_g.zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(y_g.view(torch.int16), y_e.view(torch.int16)):
                raise SystemExit(f"{name}: replay {rep} differs from the eager call")
        del graph
    print("graph first call ok", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
