"""The allocation-free decode entry point (attn_decode_noalloc) against the
existing one (attn_decode with a caller workspace), through the C ABI.

Both run the same kernels on the same partial-result layout, so their outputs
must be bitwise equal; both are also held to the decode bars against the fp64
paged oracle.  Two calls in a row, the second on a smaller problem, show
that the static scratch shared by every call carries nothing from one call
into the next.  Runs alone in a fresh process (the first call looks up the
device's scratch) and after the other tests.
"""
import pytest
import torch

import exact_io_aware_25_amd as attn
from oracle import paged
from synth import make_paged
from test_gpu_parity import announce, check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def run_both(B, H, H_kv, Lq, d, lens, bs, window, seed):
    q, kc, vc, bt, sl = make_paged(B, H, H_kv, d, "f16", Lq, lens, bs, seed=seed)
    qd, kcd, vcd, btd, sld = (t.to(DEV) for t in (q, kc, vc, bt, sl))
    max_len = max(lens)
    out_a = torch.full_like(qd, float("nan"))
    lse_a = torch.full((B, H, Lq), float("nan"), device=DEV)
    out_b = torch.full_like(qd, float("nan"))
    lse_b = torch.full((B, H, Lq), float("nan"), device=DEV)
    need = attn.attn_decode_workspace_size(B, H, H_kv, Lq, d, max_len)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    num_blocks, max_blocks = kc.shape[0], bt.shape[1]
    st = attn.attn_decode(qd.data_ptr(), kcd.data_ptr(), vcd.data_ptr(), btd.data_ptr(), sld.data_ptr(),
                          out_a.data_ptr(), lse_a.data_ptr(), ws.data_ptr(), B, H, H_kv, Lq, d, bs, max_blocks,
                          num_blocks, max_len, window, 0.0, stream)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    st = attn.attn_decode_noalloc(qd.data_ptr(), kcd.data_ptr(), vcd.data_ptr(), btd.data_ptr(), sld.data_ptr(),
                                  out_b.data_ptr(), lse_b.data_ptr(), B, H, H_kv, Lq, d, bs, max_blocks, num_blocks,
                                  max_len, window, 0.0, stream)
    assert st == attn.ATTN_OK, attn.attn_status_string(st)
    torch.cuda.synchronize(DEV)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
    ref = paged.decode_attention(q, kc, vc, bt, lens, "f16", window, 0.0)
    check(out_b.cpu(), lse_b.cpu(), ref, "f16", f"noalloc B={B} H={H}/{H_kv} Lq={Lq} lens={lens[:3]}")
    return out_b


def test_noalloc_matches_workspace_entry_point_twice():
    announce("attn_decode_noalloc: large call, then a smaller one")
    # first call: 4 sequences up to 20k tokens, 4 new tokens, GQA 32/8, d=128
    run_both(4, 32, 8, 4, 128, [20000, 777, 12345, 4096], 16, -1, seed=501)
    # second call, smaller (fewer sequences, fewer chunks, other shape): the
    # scratch still holds the first call's partials, none of which may leak in
    run_both(2, 8, 2, 1, 64, [300, 1500], 32, 100, seed=502)
