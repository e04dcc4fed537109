"""CPU tests of the C-ABI boundary: the library loads, exports every entry point
include/gqa_attn.h declares, the binding's constants and struct layouts equal
the header's, and every host-side error path returns its status before any
HIP call (no call here reaches a kernel launch)."""

import ctypes
import os
import re
import subprocess

import pytest

import gqa_attention_attn_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(G.LIB_PATH), reason="libgqa_attn.so not built")


def header_text():
    return open(HEADER).read()


def test_every_declared_entry_point_is_exported():
    decl = set(re.findall(r"^\s*(?:const\s+char\*|gqa_status|int32_t)\s+(gqa_attn_\w+)\s*\(", header_text(), re.M))
    assert decl == set(G.EXPORTS)
    L = G.lib()
    for name in decl:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gqa_attn_\w+)", out))
    assert decl <= exported


def test_constants_match_header():
    h = header_text()
    enum = dict((k, int(v)) for k, v in re.findall(r"\b(GQA_(?:OK|ERR_\w+|F32|BF16))\s*=\s*(\d+)", h))
    for k, v in enum.items():
        assert getattr(G, k) == v, k
    for k in ("GQA_ATTN_HEAD_DIM", "GQA_ATTN_MAX_GROUP", "GQA_ATTN_VERSION"):
        v = int(re.search(rf"#define {k} (\d+)", h).group(1))
        assert getattr(G, k) == v
    assert G.gqa_attn_version() == G.GQA_ATTN_VERSION


PROBE = r"""
#include <stdio.h>
#include <stddef.h>
#include "gqa_attn.h"
#define F(T, m) printf(#T " " #m " %zu\n", offsetof(T, m));
int main(void) {
  printf("gqa_decode_desc sizeof %zu\n", sizeof(gqa_decode_desc));
  printf("gqa_prefill_desc sizeof %zu\n", sizeof(gqa_prefill_desc));
  %FIELDS%
  return 0;
}
"""


def test_struct_layouts_match_c(tmp_path):
    lines = []
    for T, cls in (("gqa_decode_desc", G.GqaDecodeDesc), ("gqa_prefill_desc", G.GqaPrefillDesc)):
        for name, _ in cls._fields_:
            lines.append(f"F({T}, {name})")
    src = tmp_path / "probe.c"
    src.write_text(PROBE.replace("%FIELDS%", "\n  ".join(lines)))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        T, m, v = line.split()
        got[(T, m)] = int(v)
    for T, cls in (("gqa_decode_desc", G.GqaDecodeDesc), ("gqa_prefill_desc", G.GqaPrefillDesc)):
        assert got[(T, "sizeof")] == ctypes.sizeof(cls)
        for name, _ in cls._fields_:
            assert got[(T, name)] == getattr(cls, name).offset, (T, name)


def test_status_strings():
    for code in range(0, 7):
        s = G.gqa_attn_status_string(code)
        assert s.startswith("GQA_")
    assert "UNKNOWN" in G.gqa_attn_status_string(99)


# ------------------------------------------------------------------ descriptors

def ddesc(**kw):
    base = dict(batch=2, num_q_heads=40, num_kv_heads=8, head_dim=128, max_seq=4096, in_dtype=G.GQA_BF16,
                out_dtype=G.GQA_F32, kv_split_tokens=0,
                q_stride_b=40 * 128, q_stride_h=128,
                k_stride_b=8 * 4096 * 128, k_stride_h=4096 * 128, k_stride_s=128,
                v_stride_b=8 * 4096 * 128, v_stride_h=4096 * 128, v_stride_s=128,
                out_stride_b=40 * 128, out_stride_h=128, eps=1e-6, scale=0.0)
    base.update(kw)
    return G.GqaDecodeDesc(**base)


def pdesc(**kw):
    S = 256
    base = dict(batch=1, num_q_heads=40, num_kv_heads=8, head_dim=128, max_seq=S, in_dtype=G.GQA_BF16,
                out_dtype=G.GQA_F32, causal=1,
                q_stride_b=40 * S * 128, q_stride_h=S * 128, q_stride_s=128,
                k_stride_b=8 * S * 128, k_stride_h=S * 128, k_stride_s=128,
                v_stride_b=8 * S * 128, v_stride_h=S * 128, v_stride_s=128,
                out_stride_b=40 * S * 128, out_stride_h=S * 128, out_stride_s=128, eps=1e-6, scale=0.0)
    base.update(kw)
    return G.GqaPrefillDesc(**base)


def test_decode_plan_and_workspace_arithmetic():
    # explicit chunk 512 over 131072 keys: 256 chunks per (b, KV head); with 8
    # groups a partition workgroup sweeps 8 chunks (256 * 8 / 256 target
    # workgroups), so 32 workgroups per group write one partial each:
    # workspace = B*Hq*32*(128+2)*4
    d = ddesc(batch=1, num_q_heads=64, max_seq=131072, kv_split_tokens=512,
              k_stride_b=8 * 131072 * 128, k_stride_h=131072 * 128, v_stride_b=8 * 131072 * 128,
              v_stride_h=131072 * 128, q_stride_b=64 * 128, out_stride_b=64 * 128)
    assert G.gqa_attn_decode_plan(d) == (G.GQA_OK, 512, 256)
    assert G.gqa_attn_decode_workspace_size(d) == (G.GQA_OK, 1 * 64 * 32 * 130 * 4)
    # no split: chunk >= max_seq -> one chunk, no workspace
    d2 = ddesc(kv_split_tokens=4096)
    assert G.gqa_attn_decode_plan(d2) == (G.GQA_OK, 4096, 1)
    assert G.gqa_attn_decode_workspace_size(d2) == (G.GQA_OK, 0)
    d3 = ddesc(kv_split_tokens=100000)
    assert G.gqa_attn_decode_plan(d3)[1:] == (4096, 1)
    # ragged chunk that does not divide max_seq
    d4 = ddesc(kv_split_tokens=1000)
    assert G.gqa_attn_decode_plan(d4)[1:] == (1000, 5)


def test_decode_plan_heuristic_properties():
    for B, Hkv, S in ((1, 8, 4096), (1, 8, 131072), (32, 8, 16384), (64, 8, 512), (1, 1, 512)):
        d = ddesc(batch=B, num_q_heads=Hkv * 5, num_kv_heads=Hkv, max_seq=S)
        st, T, n = G.gqa_attn_decode_plan(d)
        assert st == G.GQA_OK
        assert 1 <= T <= S and n == -(-S // T)
        assert T == S or T % 128 == 0
        if T < S:
            assert B * Hkv * n >= 512 or T == 128   # enough workgroups, or the smallest chunk


NULL = None
FAKE = 1 << 20          # a 16-byte aligned, non-null fake address: never dereferenced on these paths


def call_decode(d, q=FAKE, k=FAKE, v=FAKE, sl=FAKE, pos=FAKE, qw=NULL, kw=NULL, out=FAKE, ws=NULL, wsb=0):
    return G.gqa_attn_decode(d, q, k, v, sl, pos, qw, kw, 1e6, out, ws, wsb, None)


def call_prefill(d, q=FAKE, k=FAKE, v=FAKE, sl=FAKE, pos=FAKE, qw=NULL, kw=NULL, out=FAKE, ws=NULL, wsb=0):
    return G.gqa_attn_prefill(d, q, k, v, sl, pos, qw, kw, 1e6, out, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), G.GQA_ERR_SHAPE),
    (dict(num_q_heads=0), G.GQA_ERR_SHAPE),
    (dict(num_kv_heads=0), G.GQA_ERR_SHAPE),
    (dict(max_seq=0), G.GQA_ERR_SHAPE),
    (dict(num_q_heads=41), G.GQA_ERR_SHAPE),
    (dict(kv_split_tokens=-1), G.GQA_ERR_SHAPE),
    (dict(q_stride_h=-128), G.GQA_ERR_SHAPE),
    (dict(batch=70000), G.GQA_ERR_SHAPE),
    (dict(head_dim=64), G.GQA_ERR_UNSUPPORTED),
    (dict(num_q_heads=136, num_kv_heads=8), G.GQA_ERR_UNSUPPORTED),   # G = 17
    (dict(in_dtype=7), G.GQA_ERR_UNSUPPORTED),
    (dict(out_dtype=2), G.GQA_ERR_UNSUPPORTED),
    (dict(k_stride_s=129), G.GQA_ERR_ALIGN),
    (dict(q_stride_h=132), G.GQA_ERR_ALIGN),        # 264 bytes: not a multiple of 16
    (dict(in_dtype=G.GQA_F32, q_stride_h=130), G.GQA_ERR_ALIGN),
])
def test_decode_descriptor_errors(kw, status):
    d = ddesc(**dict(dict(kv_split_tokens=4096), **kw))
    assert call_decode(d) == status
    assert G.gqa_attn_decode_workspace_size(d)[0] == status
    assert G.gqa_attn_decode_plan(d)[0] == status


def test_decode_pointer_errors():
    d = ddesc(kv_split_tokens=4096)
    assert call_decode(None) == G.GQA_ERR_NULL
    for name in ("q", "k", "v", "sl", "pos", "out"):
        assert call_decode(d, **{name: NULL}) == G.GQA_ERR_NULL, name
    for name in ("q", "k", "v", "out", "qw", "kw"):
        assert call_decode(d, **{name: FAKE + 8}) == G.GQA_ERR_ALIGN, name
    assert call_decode(d, sl=FAKE + 2) == G.GQA_ERR_ALIGN
    assert G.gqa_attn_decode_plan(None)[0] == G.GQA_ERR_NULL
    assert G.gqa_attn_decode_workspace_size(None)[0] == G.GQA_ERR_NULL


def test_decode_workspace_errors():
    d = ddesc(kv_split_tokens=512)
    st, need = G.gqa_attn_decode_workspace_size(d)
    # 8 chunks of 512, one per workgroup (16 groups): 8 partials per (b, q head)
    assert st == G.GQA_OK and need == 2 * 40 * 8 * 130 * 4
    assert call_decode(d, ws=NULL, wsb=need) == G.GQA_ERR_WORKSPACE
    assert call_decode(d, ws=FAKE, wsb=need - 1) == G.GQA_ERR_WORKSPACE
    assert call_decode(d, ws=FAKE + 16, wsb=need) == G.GQA_ERR_ALIGN   # workspace must be 256-byte aligned


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), G.GQA_ERR_SHAPE),
    (dict(max_seq=0), G.GQA_ERR_SHAPE),
    (dict(num_q_heads=41), G.GQA_ERR_SHAPE),
    (dict(causal=2), G.GQA_ERR_SHAPE),
    (dict(k_stride_s=-128), G.GQA_ERR_SHAPE),
    (dict(head_dim=256), G.GQA_ERR_UNSUPPORTED),
    (dict(in_dtype=G.GQA_F32), G.GQA_ERR_UNSUPPORTED),
    (dict(out_dtype=5), G.GQA_ERR_UNSUPPORTED),
    (dict(q_stride_s=100), G.GQA_ERR_ALIGN),
    (dict(out_stride_s=130), G.GQA_ERR_ALIGN),
])
def test_prefill_descriptor_errors(kw, status):
    assert call_prefill(pdesc(**kw)) == status


def test_prefill_pointer_errors():
    d = pdesc()
    assert call_prefill(None) == G.GQA_ERR_NULL
    for name in ("q", "k", "v", "sl", "pos", "out"):
        assert call_prefill(d, **{name: NULL}) == G.GQA_ERR_NULL, name
    for name in ("q", "k", "v", "out", "qw", "kw"):
        assert call_prefill(d, **{name: FAKE + 4}) == G.GQA_ERR_ALIGN, name


def test_decode_static_host_checks():
    # the entry point without a workspace: every argument check on the host,
    # and plans whose partials exceed the static array are refused
    st = G.gqa_attn_decode_static
    h = header_text()
    assert G.GQA_ATTN_STATIC_SCRATCH_BYTES == eval(re.search(r"#define GQA_ATTN_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                                                             h).expand(r"\1 << \2"))
    d = ddesc(kv_split_tokens=512)
    assert st(None, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, None) == G.GQA_ERR_NULL
    assert st(d, NULL, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, None) == G.GQA_ERR_NULL
    assert st(d, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, NULL, None) == G.GQA_ERR_NULL
    assert st(d, FAKE + 4, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, None) == G.GQA_ERR_ALIGN
    assert st(ddesc(head_dim=64), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, None) == G.GQA_ERR_UNSUPPORTED
    # 64 sequences x 64 query heads x 256 partials x 520 bytes = 520 MiB > 16 MiB
    big = ddesc(batch=64, num_q_heads=64, max_seq=1 << 17, kv_split_tokens=512, q_stride_b=64 * 128,
                k_stride_b=8 * (1 << 17) * 128, k_stride_h=(1 << 17) * 128, v_stride_b=8 * (1 << 17) * 128,
                v_stride_h=(1 << 17) * 128, out_stride_b=64 * 128)
    stb, need = G.gqa_attn_decode_workspace_size(big)
    assert stb == G.GQA_OK and need > G.GQA_ATTN_STATIC_SCRATCH_BYTES
    assert st(big, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, None) == G.GQA_ERR_SCRATCH
    assert "static decode scratch" in G.gqa_attn_status_string(G.GQA_ERR_SCRATCH)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(G, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(G, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        G.gqa_attn_version()


def test_decode_merge_entry_errors_and_single_chunk_noop():
    d = ddesc(kv_split_tokens=512)
    st, need = G.gqa_attn_decode_workspace_size(d)
    assert G.gqa_attn_decode_merge(None, FAKE, FAKE, FAKE, need, None) == G.GQA_ERR_NULL
    assert G.gqa_attn_decode_merge(d, NULL, FAKE, FAKE, need, None) == G.GQA_ERR_NULL
    assert G.gqa_attn_decode_merge(d, FAKE, NULL, FAKE, need, None) == G.GQA_ERR_NULL
    assert G.gqa_attn_decode_merge(d, FAKE, FAKE, NULL, need, None) == G.GQA_ERR_WORKSPACE
    assert G.gqa_attn_decode_merge(d, FAKE, FAKE, FAKE, need - 4, None) == G.GQA_ERR_WORKSPACE
    assert G.gqa_attn_decode_merge(d, FAKE, FAKE + 4, FAKE, need, None) == G.GQA_ERR_ALIGN
    # one chunk: the merge step has nothing to do and launches nothing
    assert G.gqa_attn_decode_merge(ddesc(kv_split_tokens=4096), FAKE, FAKE, NULL, 0, None) == G.GQA_OK
    assert G.gqa_attn_decode_partition(None, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, NULL, 0,
                                       None) == G.GQA_ERR_NULL


def test_decode_cache_slab_limit():
    # one (b, head) slab of 2^20 rows with a 4096-element row stride spans 8 GiB
    d = ddesc(max_seq=1 << 20, k_stride_s=4096, v_stride_s=128, k_stride_h=(1 << 20) * 4096,
              v_stride_h=(1 << 20) * 128, k_stride_b=8 * (1 << 20) * 4096, v_stride_b=8 * (1 << 20) * 128,
              kv_split_tokens=4096)
    assert call_decode(d) == G.GQA_ERR_UNSUPPORTED


def test_prefill_workspace_size_and_errors():
    d = pdesc()
    st, need = G.gqa_attn_prefill_workspace_size(d)
    # K' and V regions, each 256 / 32 tiles of 9216 bytes per (sequence, KV head)
    assert st == G.GQA_OK and need == 1 * 8 * (256 // 32) * 9216 * 2
    assert G.gqa_attn_prefill_workspace_size(None)[0] == G.GQA_ERR_NULL
    assert G.gqa_attn_prefill_workspace_size(pdesc(head_dim=64))[0] == G.GQA_ERR_UNSUPPORTED
    assert call_prefill(d, ws=FAKE, wsb=need - 1) == G.GQA_ERR_WORKSPACE
    assert call_prefill(d, ws=FAKE + 16, wsb=need) == G.GQA_ERR_ALIGN


def test_prefill_phases_and_cache_write_errors():
    d = pdesc()
    st, need = G.gqa_attn_prefill_workspace_size(d)
    for fn in (G.gqa_attn_prefill_keys, G.gqa_attn_prefill_attend):
        # the phases exist only with a workspace
        assert fn(d, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, NULL, 0, None) == G.GQA_ERR_WORKSPACE
        assert fn(d, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, FAKE, need - 1, None) == G.GQA_ERR_WORKSPACE
        assert fn(None, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, FAKE, need, None) == G.GQA_ERR_NULL
        assert fn(d, NULL, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, FAKE, need, None) == G.GQA_ERR_NULL
        assert fn(pdesc(in_dtype=G.GQA_F32), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, FAKE, need,
                  None) == G.GQA_ERR_UNSUPPORTED
    # the key-cache write-back is done by the key phase: no workspace, no write-back
    assert call_prefill(pdesc(write_k_cache=1)) == G.GQA_ERR_WORKSPACE
    assert call_prefill(pdesc(write_k_cache=2), ws=FAKE, wsb=need) == G.GQA_ERR_SHAPE
    assert call_chunk(pdesc(max_chunk=64, write_k_cache=-1), wsb=need) == G.GQA_ERR_SHAPE


def call_chunk(d, q=FAKE, k=FAKE, v=FAKE, past=FAKE, cl=FAKE, pos=FAKE, qw=NULL, kw=NULL, out=FAKE, ws=FAKE,
               wsb=1 << 40):
    return G.gqa_attn_prefill_chunk(d, q, k, v, past, cl, pos, qw, kw, 1e6, out, ws, wsb, None)


def test_prefill_chunk_errors():
    d = pdesc(max_chunk=64)
    assert G.gqa_attn_prefill_chunk(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 1e6, FAKE, FAKE, 1, None) \
        == G.GQA_ERR_NULL
    assert call_chunk(d, past=NULL) == G.GQA_ERR_NULL
    assert call_chunk(d, cl=NULL) == G.GQA_ERR_NULL
    assert call_chunk(d, ws=NULL) == G.GQA_ERR_WORKSPACE                  # the chunked form needs a workspace
    assert call_chunk(pdesc(max_chunk=-1)) == G.GQA_ERR_SHAPE
    st, need = G.gqa_attn_prefill_workspace_size(d)                        # sized by the cache capacity
    assert st == G.GQA_OK and need == G.gqa_attn_prefill_workspace_size(pdesc())[1]
    assert call_chunk(d, wsb=need - 1) == G.GQA_ERR_WORKSPACE
    assert call_chunk(d, ws=FAKE + 16, wsb=need) == G.GQA_ERR_ALIGN
    assert call_chunk(d, past=FAKE + 2, wsb=need) == G.GQA_ERR_ALIGN
    assert call_chunk(pdesc(max_chunk=64, head_dim=64), wsb=need) == G.GQA_ERR_UNSUPPORTED
    assert call_chunk(pdesc(max_chunk=64, in_dtype=G.GQA_F32), wsb=need) == G.GQA_ERR_UNSUPPORTED


def call_paged(d, bt=FAKE, ws=FAKE, wsb=1 << 40):
    return G.gqa_attn_decode_paged(d, FAKE, FAKE, FAKE, bt, FAKE, FAKE, NULL, NULL, 1e6, FAKE, ws, wsb, None)


def test_decode_paged_errors_and_plan():
    d = ddesc(block_size=64)
    assert call_paged(d, bt=NULL) == G.GQA_ERR_NULL
    assert call_paged(d, bt=FAKE + 2) == G.GQA_ERR_ALIGN
    assert call_paged(ddesc()) == G.GQA_ERR_SHAPE                  # contiguous descriptor
    assert call_decode(d) == G.GQA_ERR_SHAPE                        # paged descriptor, contiguous entry point
    for bad in (16, 48, 96, 3):
        assert call_paged(ddesc(block_size=bad)) == G.GQA_ERR_SHAPE
    assert call_paged(ddesc(block_size=64, max_seq=4096 + 32)) == G.GQA_ERR_SHAPE   # pages do not divide max_seq
    # the chunk length rounds up to a multiple of 32 keys so no step crosses a page
    st, T, n = G.gqa_attn_decode_plan(ddesc(block_size=32, kv_split_tokens=100))
    assert st == G.GQA_OK and T == 128 and n == -(-4096 // 128)
    st, T, n = G.gqa_attn_decode_plan(ddesc(kv_split_tokens=100))
    assert st == G.GQA_OK and T == 100


def test_prefill_chunk_paged_errors():
    d = pdesc(max_chunk=64, block_size=64)
    call = lambda dd, bt=FAKE, past=FAKE, ws=FAKE, wsb=1 << 40: G.gqa_attn_prefill_chunk_paged(
        dd, FAKE, FAKE, FAKE, bt, past, FAKE, FAKE, NULL, NULL, 1e6, FAKE, ws, wsb, None)
    assert call(d, bt=NULL) == G.GQA_ERR_NULL
    assert call(d, past=NULL) == G.GQA_ERR_NULL
    assert call(d, ws=NULL) == G.GQA_ERR_WORKSPACE
    assert call(d, bt=FAKE + 2) == G.GQA_ERR_ALIGN
    assert call(pdesc(max_chunk=64)) == G.GQA_ERR_SHAPE                    # contiguous descriptor
    assert call_chunk(d) == G.GQA_ERR_SHAPE                                 # paged descriptor, contiguous entry
    assert call_prefill(pdesc(block_size=64)) == G.GQA_ERR_SHAPE
    for bad in (8, 24, 96):
        assert call(pdesc(max_chunk=64, block_size=bad)) == G.GQA_ERR_SHAPE


# ---- the measurement probes (include/gqa_probe.h, libgqa_probe.so)

def test_probe_library_exports_and_host_checks():
    from gqa_attention_attn_amd import probe as P
    if not os.path.exists(P.PROBE_LIB_PATH):
        pytest.skip("libgqa_probe.so not built")
    h = open(os.path.join(ROOT, "include", "gqa_probe.h")).read()
    decl = set(re.findall(r"^\s*int32_t\s+(gqa_probe_\w+)\s*\(", h, re.M))
    assert decl == set(P.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", P.PROBE_LIB_PATH], capture_output=True, text=True).stdout
    assert decl <= set(re.findall(r"\bT (gqa_probe_\w+)", out))
    # NULL, misaligned or ragged arguments are rejected on the host (status 1), before any HIP call
    assert P.read(None, 1024, 64, None) == 1
    assert P.read(4096 + 8, 1024, 64, None) == 1
    assert P.read(4096, 1000, 64, None) == 1
    assert P.read(4096, 1024, None, None) == 1
    assert P.copy(4096, None, 1024, None) == 1
    assert P.copy(4096, 8192 + 4, 1024, None) == 1


# ---- the timeline build (include/gqa_timeline.h, libgqa_attn_timeline.so)

def test_timeline_build_exports_and_constants():
    from gqa_attention_attn_amd import build as B, timeline as T
    if not os.path.exists(B.TIMELINE_LIB):
        pytest.skip("libgqa_attn_timeline.so not built")
    h = open(os.path.join(ROOT, "include", "gqa_timeline.h")).read()
    decl = set(re.findall(r"^\s*int32_t\s+(gqa_timeline_\w+)\s*\(", h, re.M))
    assert decl == {"gqa_timeline_clear", "gqa_timeline_read", "gqa_timeline_clock_khz"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.TIMELINE_LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gqa_\w+)", out))
    # the same attention entry points as libgqa_attn.so, plus the timeline's
    assert decl | set(G.EXPORTS) <= exported
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (GQA_TIMELINE_\w+) (\d+)", h))
    assert consts == {"GQA_TIMELINE_SLOTS": T.SLOTS, "GQA_TIMELINE_BLOCKS": T.BLOCKS,
                      "GQA_TIMELINE_DECODE": T.KERNELS["decode"], "GQA_TIMELINE_PREFILL": T.KERNELS["prefill"]}
    assert all(len(names) < T.SLOTS for names in T.NAMES.values()) and T.TILES_SLOT >= len(T.NAMES["prefill"])
    # a NULL host buffer, an unknown kernel or a read beyond the array is
    # rejected before any HIP call
    L = ctypes.CDLL(B.TIMELINE_LIB)
    L.gqa_timeline_read.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t]
    L.gqa_timeline_read.restype = ctypes.c_int32
    buf = (ctypes.c_uint64 * 8)()
    assert L.gqa_timeline_read(0, None, 8) == 1
    assert L.gqa_timeline_read(2, ctypes.addressof(buf), 8) == 1
    assert L.gqa_timeline_read(1, ctypes.addressof(buf), T.SLOTS * T.BLOCKS + 1) == 1
    L.gqa_timeline_clock_khz.argtypes = [ctypes.c_void_p]
    L.gqa_timeline_clock_khz.restype = ctypes.c_int32
    assert L.gqa_timeline_clock_khz(None) == 1
