"""The entry points under HIP graph capture (serving and training loops that
replay a captured step): forward, backward and paged decode are each
captured once into a torch CUDA graph, with every output and workspace
allocated beforehand, and the graph is replayed three times with new inputs
copied into the captured tensors in between (eager work and a
synchronisation between replays).  Every replay must equal, bit for bit, an
eager call on the same inputs: the kernels are deterministic, launch no
memory set and allocate nothing, so a replay runs exactly the captured
launches.  The first call of each entry point happens before capture (it
queries the device once)."""
import pytest
import torch

import exact_io_aware_25_amd as attn
from synth import make_paged, make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on the side stream, as torch asks before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_forward_graph_replay():
    B, H, H_kv, L, d = 2, 8, 2, 777, 64
    announce(f"graph forward B={B} H={H}/{H_kv} L={L} d={d}")
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, H_kv, L, d, "f16", 90))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
    attn.forward(q, k, v, causal=True, window=100, out=out, lse=lse)
    g = capture(lambda: attn.forward(q, k, v, causal=True, window=100, out=out, lse=lse))
    for rep in range(3):
        nq, nk, nv = make_qkv(B, H, H_kv, L, d, "f16", 91 + rep)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = attn.forward(q, k, v, causal=True, window=100)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep} differs from the eager call"


def test_backward_graph_replay():
    B, H, H_kv, L, d = 1, 4, 2, 600, 128
    announce(f"graph backward B={B} H={H}/{H_kv} L={L} d={d}")
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, H_kv, L, d, "bf16", 95))
    dout = make_qkv(B, H, H, L, d, "bf16", 96)[0].to(DEV)
    out, lse = attn.forward(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(attn.attn_bwd_workspace_size(B, H, L), 16), dtype=torch.uint8, device=DEV)

    def step():
        attn.backward(q, k, v, out, lse, dout, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    step()
    g = capture(step)
    for rep in range(3):
        nq, nk, nv = make_qkv(B, H, H_kv, L, d, "bf16", 97 + rep)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        o2, l2 = attn.forward(q, k, v, causal=True)  # eager work between replays
        out.copy_(o2)
        lse.copy_(l2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r = attn.backward(q, k, v, out, lse, dout, causal=True)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip((dq, dk, dv), r)), f"replay {rep} differs from the eager call"


def test_decode_graph_replay():
    B, H, H_kv, Lq, d, bs = 3, 16, 4, 2, 128, 16
    lens = [900, 37, 2500]
    announce(f"graph decode B={B} H={H}/{H_kv} Lq={Lq} d={d} lens={lens}")
    q, kc, vc, bt, sl = (t.to(DEV) for t in make_paged(B, H, H_kv, d, "bf16", Lq, lens, bs, seed=98))
    max_len = max(lens)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(attn.attn_decode_workspace_size(B, H, H_kv, Lq, d, max_len), 16), dtype=torch.uint8,
                     device=DEV)

    def step():
        attn.decode(q, kc, vc, bt, sl, max_len, out=out, lse=lse, workspace=ws)
    step()
    g = capture(step)
    for rep in range(3):
        nq, nkc, nvc, _, _ = make_paged(B, H, H_kv, d, "bf16", Lq, lens, bs, seed=99 + rep)
        q.copy_(nq)
        kc.copy_(nkc)
        vc.copy_(nvc)
        sl.copy_(torch.tensor([n - 5 * rep for n in lens], dtype=torch.int32))  # the lengths are data too
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = attn.decode(q, kc, vc, bt, sl, max_len)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep} differs from the eager call"
