"""GPU check of gqa_attn_decode_static, the decode entry point that allocates
nothing (its split-KV partials live in the library's static device array).

Through the C ABI: two calls in a row, the second with a smaller input, each
equal bitwise to gqa_attn_decode on the same inputs (same plan, same kernels)
and within the bf16 bound (1e-2) of the fp64 oracle; a plan whose partials
exceed the array is refused on the host; a call captured in a HIP graph and
replayed, each replay bitwise equal to the eager decode.
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def one_case(w):
    torch = require_gpu()
    inp = synth.make_decode(w)
    bf = torch.bfloat16
    q, k, v = dev(inp["q"], bf), dev(inp["k"], bf), dev(inp["v"], bf)
    qw, kw = dev(inp["q_norm_w"], bf), dev(inp["k_norm_w"], bf)
    sl, pos = ints(inp["seq_lens"]), ints(inp["positions"])
    B, Hq, d = inp["q"].shape
    out_static = torch.full((B, Hq, d), float("nan"), device="cuda")
    out_ws = torch.full((B, Hq, d), float("nan"), device="cuda")
    desc = G.decode_desc(q, k, v, out_static, w.split_tokens, w.eps)
    st, need = G.gqa_attn_decode_workspace_size(desc)
    assert st == G.GQA_OK and 0 < need <= G.GQA_ATTN_STATIC_SCRATCH_BYTES
    p = lambda t: None if t is None else t.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    log(f"case decode_static {w.name} (partials {need} bytes)")
    assert G.gqa_attn_decode_static(desc, p(q), p(k), p(v), p(sl), p(pos), p(qw), p(kw), w.rope_theta,
                                    p(out_static), s) == G.GQA_OK
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert G.gqa_attn_decode(desc, p(q), p(k), p(v), p(sl), p(pos), p(qw), p(kw), w.rope_theta, p(out_ws),
                             p(ws), need, s) == G.GQA_OK
    torch.cuda.synchronize()
    a, b = out_static.cpu().numpy(), out_ws.cpu().numpy()
    assert np.array_equal(a, b), "static-scratch decode differs from the workspace decode"
    want = O.decode_ref(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["positions"], inp["q_norm_w"],
                        inp["k_norm_w"], inp["rope_theta"], inp["eps"])
    compare(a, want, ATOL, f"decode_static {w.name}")


def test_decode_static_two_calls_second_smaller():
    # the ragged B = 32 batch (10.6 MB of partials), then the B = 1 Qwen3-14B
    # step (0.67 MB): the second call reuses the array the first one filled
    one_case(synth.QWEN3_RAGGED)
    one_case(synth.QWEN3_DECODE)


def test_decode_static_refuses_oversized_plans():
    require_gpu()
    d = G.GqaDecodeDesc(batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, max_seq=1 << 17,
                        in_dtype=G.GQA_BF16, out_dtype=G.GQA_F32, kv_split_tokens=512, q_stride_b=64 * 128,
                        q_stride_h=128, k_stride_b=8 * (1 << 17) * 128, k_stride_h=(1 << 17) * 128, k_stride_s=128,
                        v_stride_b=8 * (1 << 17) * 128, v_stride_h=(1 << 17) * 128, v_stride_s=128,
                        out_stride_b=64 * 128, out_stride_h=128, eps=1e-6, scale=0.0)
    fake = 1 << 20
    assert G.gqa_attn_decode_static(d, fake, fake, fake, fake, fake, None, None, 5e5, fake,
                                    None) == G.GQA_ERR_SCRATCH


def test_decode_static_under_graph_capture():
    """The callers this entry point is for may capture it: a HIP graph of one
    call, replayed with new q rows written eagerly between replays (and a
    synchronisation after each), every replay bitwise equal to an eager
    gqa_attn_decode on the same inputs."""
    torch = require_gpu()
    w = synth.QWEN3_DECODE
    inp = synth.make_decode(w)
    bf = torch.bfloat16
    q, k, v = dev(inp["q"], bf), dev(inp["k"], bf), dev(inp["v"], bf)
    qw, kw = dev(inp["q_norm_w"], bf), dev(inp["k_norm_w"], bf)
    sl, pos = ints(inp["seq_lens"]), ints(inp["positions"])
    out_g = torch.full(tuple(q.shape), float("nan"), device="cuda")
    desc = G.decode_desc(q, k, v, out_g, w.split_tokens, w.eps)
    st, need = G.gqa_attn_decode_workspace_size(desc)
    assert st == G.GQA_OK
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    p = lambda t: None if t is None else t.data_ptr()
    call = lambda o, stream: G.gqa_attn_decode_static(desc, p(q), p(k), p(v), p(sl), p(pos), p(qw), p(kw),
                                                      w.rope_theta, p(o), stream)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):   # one eager call first
        assert call(out_g, s.cuda_stream) == G.GQA_OK
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        assert call(out_g, s.cuda_stream) == G.GQA_OK
    rng = np.random.default_rng(91)
    for r in range(4):
        log(f"case decode_static graph replay {r}")
        q.copy_(dev(synth.bf16_round(rng.standard_normal(tuple(q.shape)).astype(np.float32)), bf))
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out_e = torch.full(tuple(q.shape), float("nan"), device="cuda")
        assert G.gqa_attn_decode(desc, p(q), p(k), p(v), p(sl), p(pos), p(qw), p(kw), w.rope_theta, p(out_e),
                                 p(ws), need, torch.cuda.current_stream().cuda_stream) == G.GQA_OK
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"graph replay {r} differs from the eager decode"
