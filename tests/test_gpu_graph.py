"""Every library kernel captured into one HIP graph: each replay, with eager
work and synchronisation between replays, must reproduce the eager results
bit for bit (all kernels are deterministic)."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, show, to_dev_bf16, to_dev_i8, to_dev_u8

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import weight_quantized_linear_amd as q
    w_small, s_small = synth.fp8_weight((70,), 4096, 1024)
    w_wide, s_wide = synth.fp8_weight((71,), 65600, 256)
    x1 = to_dev_bf16(synth.bf16_activation((72,), 1, 1024))
    x4 = to_dev_bf16(synth.bf16_activation((73,), 4, 256))
    x16 = to_dev_bf16(synth.bf16_activation((74,), 16, 256))
    x64 = to_dev_bf16(synth.bf16_activation((75,), 64, 1024))
    ws, ww = to_dev_u8(w_small), to_dev_u8(w_wide)
    packed, scales, g = synth.nvfp4_weight((76,), 512, 1024)
    pd, sd = to_dev_u8(packed), to_dev_u8(scales)
    grp = synth.fp8_weight((77,), 4 * 256, 512)[0].reshape(4, 256, 512)
    gx = to_dev_bf16(synth.bf16_activation((78,), 300, 512))
    offs = torch.tensor([0, 100, 100, 250, 300], dtype=torch.int32, device=DEV)
    ids = torch.tensor([2, 0, -1, 3], dtype=torch.int32, device=DEV)
    xi = to_dev_bf16(synth.bf16_activation((79,), 200, 512, outlier_p=0.01))
    bi, bs = synth.int8_weight((80,), 300, 512)
    bid, bsd = to_dev_i8(bi), torch.from_numpy(bs).to(DEV)
    bias = to_dev_bf16(synth.bf16_bias((81,), 300))

    outs = {
        "gemv": torch.empty((1, 4096), dtype=torch.bfloat16, device=DEV),
        "skinny4": torch.empty((4, 65600), dtype=torch.bfloat16, device=DEV),
        "skinny16": torch.empty((16, 65600), dtype=torch.float32, device=DEV),
        "tiled": torch.empty((64, 4096), dtype=torch.bfloat16, device=DEV),
        "nvfp4": torch.empty((64, 512), dtype=torch.bfloat16, device=DEV),
        "nvfp4_gemv": torch.empty((1, 512), dtype=torch.float32, device=DEV),
        "grouped": torch.zeros((300, 256), dtype=torch.bfloat16, device=DEV),
        "q": torch.empty((200, 512), dtype=torch.int8, device=DEV),
        "sa": torch.empty((200,), dtype=torch.float32, device=DEV),
        "int8": torch.empty((200, 300), dtype=torch.bfloat16, device=DEV),
    }

    def work():
        q.fp8_gemm(ws, x1, out=outs["gemv"], alpha=float(s_small))
        q.fp8_gemm(ww, x4, out=outs["skinny4"], alpha=float(s_wide))
        q.fp8_gemm(ww, x16, out=outs["skinny16"], out_dtype=torch.float32)
        q.fp8_gemm(ws, x64, out=outs["tiled"])
        q.nvfp4_gemm(pd, sd, x64, out=outs["nvfp4"], alpha=float(g))
        q.nvfp4_gemm(pd, sd, x1, out=outs["nvfp4_gemv"], out_dtype=torch.float32)
        q.fp8_grouped_gemm(to_grp, gx, offs, ids, out=outs["grouped"], max_tokens_per_group=150)
        q.int8_quantize_act(xi, q=outs["q"], a_scale=outs["sa"])
        q.int8_gemm(outs["q"], bid, outs["sa"], bsd, bias, out=outs["int8"])

    to_grp = to_dev_u8(grp)
    show("graph: eager reference")
    work()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    show("graph: capture")
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.fill_(0)          # eager work between replays
        torch.cuda.synchronize()
        show("graph: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, eager[k]), (rep, k)
