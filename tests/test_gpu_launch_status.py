"""Launch status is the launch's own, not a sticky error of an earlier HIP call.

Loading the library through a host-only call (a workspace-size query) before
anything has touched the GPU leaves a pending "no device" error in the HIP
runtime of that thread; a launcher that reported hipGetLastError() would
return GQA_ERR_HIP for a launch that succeeded.  The check runs in a fresh
process so that the library really is loaded first.
"""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, ROOT)
sys.path.insert(0, ROOT + "/tests")
import gqa_attention_attn_amd as G
# host-only calls first: the library is loaded before the GPU is used
d = G.GqaPrefillDesc(batch=1, num_q_heads=10, num_kv_heads=2, head_dim=128, max_seq=256, in_dtype=G.GQA_BF16,
                     out_dtype=G.GQA_F32, causal=1, q_stride_b=10 * 256 * 128, q_stride_h=256 * 128, q_stride_s=128,
                     k_stride_b=2 * 256 * 128, k_stride_h=256 * 128, k_stride_s=128, v_stride_b=2 * 256 * 128,
                     v_stride_h=256 * 128, v_stride_s=128, out_stride_b=10 * 256 * 128, out_stride_h=256 * 128,
                     out_stride_s=128, eps=1e-6, scale=0.0)
assert G.gqa_attn_prefill_workspace_size(d)[0] == G.GQA_OK
import numpy as np
import torch
import oracle as O
rng = np.random.default_rng(5)
bf = torch.bfloat16
q = rng.standard_normal((1, 10, 256, 128)).astype(np.float32)
k = rng.standard_normal((1, 2, 256, 128)).astype(np.float32)
v = rng.standard_normal((1, 2, 256, 128)).astype(np.float32)
t = lambda x: torch.from_numpy(x).cuda().to(bf)
lens = torch.tensor([256], dtype=torch.int32, device="cuda")
pos = torch.tensor([0], dtype=torch.int32, device="cuda")
out = G.prefill(t(q), t(k), t(v), lens, pos)          # raises on GQA_ERR_HIP
dec = G.decode(t(q[:, :, 0]), t(k), t(v), lens, pos + 255, kv_split_tokens=64)
torch.cuda.synchronize()
qr, kr, vr = (torch.from_numpy(x).to(bf).float().numpy() for x in (q, k, v))
want = O.prefill_ref(qr, kr, vr, np.array([256]), np.array([0]), None, None, 0.0)
err = float(np.max(np.abs(out.cpu().numpy() - want)))
print("max err", err)
assert err <= 1e-2
"""


def test_launch_after_host_only_load():
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-c", "ROOT = %r\n" % ROOT + SCRIPT], capture_output=True, text=True,
                       timeout=300, env=env, cwd=ROOT)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-2000:]
