"""The entry points under HIP graph capture: the library allocates nothing, issues no memset and
keeps no host state between calls, so a captured sequence replays to the eager results.  Each
replay is followed by eager work on the same buffers and a synchronisation, and every replay is
compared bitwise with the eager outputs (fills of torch's own kernels clear the buffers)."""
import pytest
import torch

import seeded_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_online_softmax_amd as mod
    return mod


def test_captured_forward_split_combine_fused_replays(sa):
    q, k, v = (t.to(DEV) for t in si.prefill_inputs(B=1, H=4, N=1000))
    dq, dk, dv = (t.to(DEV) for t in si.decode_inputs(B=2, H=4, Nkv=3000))
    P = 8
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    o_p = torch.empty((P, 2, 4, 128), dtype=torch.float32, device=DEV)
    l_p = torch.empty((P, 2, 4), dtype=torch.float32, device=DEV)
    dout = torch.empty((2, 1, 4, 128), dtype=torch.bfloat16, device=DEV)
    dlse = torch.empty((2, 1, 4), dtype=torch.float32, device=DEV)
    tk = torch.zeros(8 * sa.TICKET_STRIDE, dtype=torch.int32, device=DEV)
    fout = torch.empty_like(dout)
    flse = torch.empty_like(dlse)
    fo_p, fl_p = torch.empty_like(o_p), torch.empty_like(l_p)

    def step():
        sa.attn_fwd(q, k, v, out, lse, causal=True)
        sa.attn_fwd_splitk(dq, dk, dv, P, o_p, l_p)
        sa.attn_combine(o_p, l_p, dout, dlse)
        sa.attn_fwd_splitk_fused(dq, dk, dv, P, fo_p, fl_p, tk, fout, flse)

    outs = (out, lse, o_p, l_p, dout, dlse, fout, flse)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                   # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(3):
        for t in outs:
            t.fill_(0)                           # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), f"replay {replay}: output {i} differs from the eager result"
        assert int(tk.abs().sum()) == 0, "tickets not returned to zero"


def test_captured_mask_pack_and_packed_forward_replays(sa):
    """attn_mask_pack then attn_fwd on the bits, captured: every replay repacks the mask (its
    words cleared in between, the groups above the diagonal included) and gives the eager outputs
    bitwise."""
    N, H, D = 700, 2, 128
    rng = si.rng_for(98, 0)
    q, k, v = (si.cast(x, "bf16").to(DEV) for x in si.draw_qkv(rng, (1, N, H, D), (1, N, H, D)))
    mask, _ = si.bernoulli_mask(rng, N, N, 3)
    md = torch.from_numpy(mask).to(DEV)
    bits = torch.zeros(sa.mask_bits_words(N, N), dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)

    def step():
        sa.attn_mask_pack(md, bits, causal=True)
        sa.attn_fwd_packed(q, k, v, out, lse, causal=True, mask_bits=bits)

    step()
    torch.cuda.synchronize()
    ref = [out.clone(), lse.clone()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(3):
        out.fill_(0)
        lse.fill_(0)
        bits.fill_(-1)                               # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {replay} differs"
