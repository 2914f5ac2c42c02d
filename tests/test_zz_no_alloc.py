"""vt_spec_block_noalloc (the block with the library's fixed device scratch instead of a caller
workspace) against vt_spec_block (caller workspace), called through the C ABI with ctypes: two
calls in a row on different shapes, the second smaller, each bit for bit equal to the existing
entry point; and the host-side rejection of a shape whose workspace exceeds the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import draft_sampling_verification_amd as vt
from tests.gpu_harness import dev, dev_bf16, say, target_tensor
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

VT_ERR_WORKSPACE = 3


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _outs(cfg, B):
    M = B * cfg.R
    return dict(logits=torch.full((M, cfg.Vt), -5.0, dtype=torch.float32, device="cuda"),
                dlse=torch.full((M,), -5.0, dtype=torch.float64, device="cuda"),
                dids=torch.full((M,), -5, dtype=torch.int32, device="cuda"),
                tlse=torch.full((B * (cfg.gamma + 1),), -5.0, dtype=torch.float64, device="cuda"),
                tok=torch.full((B, cfg.gamma + 1), -5, dtype=torch.int32, device="cuda"),
                nacc=torch.full((B,), -5, dtype=torch.int32, device="cuda"))


def _run(wl, noalloc, tiled=False):
    """tiled: also hand over the K-tiled W^Trim (as the benchmark does for the large-batch head)."""
    cfg, B = wl.cfg, wl.B
    L = vt.lib()
    ins = dict(hidden=dev_bf16(wl.hidden), weight=dev_bf16(wl.weight),
               keep=dev(wl.keep_ids) if wl.keep_ids is not None else None,
               f2t=dev(wl.full_to_trim) if wl.full_to_trim is not None else None, target=target_tensor(wl),
               ud=dev(wl.u_draft.reshape(-1)), ua=dev(wl.u_acc), uf=dev(wl.u_fin))
    wt = vt.vt_trim_head_tiled(ins["weight"], ins["keep"], k=cfg.Vt) if tiled else None
    o = _outs(cfg, B)
    dt = 0 if cfg.target_dtype == "f32" else 1
    T = float(wl.T)
    args = [_p(ins["hidden"]), _p(ins["weight"]), _p(wt), _p(ins["keep"]), _p(ins["f2t"]), B, cfg.gamma, cfg.R, cfg.H, cfg.Vt,
            cfg.V, _p(ins["target"]), dt, T, T, _p(ins["ud"]), _p(ins["ua"]), _p(ins["uf"]), _p(o["logits"]),
            _p(o["dlse"]), _p(o["dids"]), _p(o["tlse"]), _p(o["tok"]), _p(o["nacc"]), None, None]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = L.vt_spec_block_noalloc(*args, stream)
    else:
        nbytes = L.vt_spec_block_workspace_bytes(B, cfg.gamma, cfg.R, cfg.H, cfg.Vt, cfg.V)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        st = L.vt_spec_block(*args, _p(ws), nbytes, stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def _same(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("order", ["large-then-small", "small-then-large"])
def test_noalloc_matches_block_on_two_calls(order):
    big = make_workload(CONFIGS[5].scaled(B=40, V=20000, Vt=6000, H=512), follow=0.5)   # M = 360: MFMA tiles
    small = make_workload(CONFIGS[3].scaled(V=20000, Vt=5000, H=512), b0=2, follow=0.5)  # batch 1: three launches
    seq = [big, small] if order == "large-then-small" else [small, big]
    for wl in seq:
        say(f"noalloc vs workspace: B={wl.B} R={wl.cfg.R} V={wl.cfg.V} Vt={wl.cfg.Vt}")
        want = _run(wl, noalloc=False)
        got = _run(wl, noalloc=True)
        _same(want, got)
        assert (got["nacc"] >= 0).all()


def test_noalloc_full_size_then_batch_one():
    # the benchmark's large-drafter block (24.5 MiB of scratch, K-tiled W^Trim) and then the
    # batch-1 VocabTrim block
    for c in (5, 3):
        wl = make_workload(CONFIGS[c])
        say(f"noalloc full size config {c}")
        _same(_run(wl, noalloc=False, tiled=c == 5), _run(wl, noalloc=True, tiled=c == 5))


def test_noalloc_rejects_shapes_beyond_the_scratch():
    L = vt.lib()
    B, g, R, H, Vt, V = 4096, 8, 9, 4096, 65536, 128256
    assert L.vt_spec_block_workspace_bytes(B, g, R, H, Vt, V) > 64 << 20
    # rejected on the host before anything is enqueued: the pointers are never dereferenced
    fake = ctypes.c_void_p(256)
    st = L.vt_spec_block_noalloc(fake, fake, None, fake, fake, B, g, R, H, Vt, V, fake, 1, 0.8, 0.8, fake, fake, fake,
                                 fake, fake, fake, fake, fake, fake, None, None, None)
    assert st == VT_ERR_WORKSPACE
