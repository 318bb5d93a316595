"""Child process of test_zz_no_alloc.py: the device's first allocation-free
call is made under HIP graph capture (the library takes the address of its
static scratch then); the replay must equal an eager call bitwise.
Prints "replay equals eager: True" on success."""
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import tiled_dense_gemm_bias_amd as gba  # noqa: E402


def main():
    gba.lib()   # the library is loaded; nothing has run on the device yet
    M, N, K = 256, 384, 4096   # a split-K shape: the call uses the scratch
    g0 = torch.Generator().manual_seed(0)
    a = torch.randn(M, K, generator=g0).half().cuda()
    b = (torch.randn(K, N, generator=g0) / 64).half().cuda()
    bias = torch.randn(N, generator=g0).half().cuda()
    c = torch.empty(M, N, dtype=torch.half, device="cuda")
    assert gba.workspace_size(M, N, K, "gelu", "f16") > 0
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gba.gemm_bias_act_noalloc(a, b, bias, c, "gelu")
    for _ in range(3):
        c.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
    ref = torch.empty_like(c)
    gba.gemm_bias_act_noalloc(a, b, bias, ref, "gelu")
    torch.cuda.synchronize()
    print("replay equals eager:", torch.equal(c.view(torch.int16), ref.view(torch.int16)), flush=True)


if __name__ == "__main__":
    main()
