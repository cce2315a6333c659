"""The packing entry point that allocates nothing (bitnet_pack_weights_noalloc):
its float64 row sums live in a scratch array the library holds per GPU.  Checked
against bitnet_pack_weights, the entry point with a caller workspace, bit for bit
on packed bytes and s_w, on consecutive calls that reuse the scratch (the second
smaller than the first), up to the largest row count the scratch holds; beyond it
the call is rejected before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
import ternary_weight_token_amd as tw

DEV = "cuda:0"


def _pack_both(w: torch.Tensor, eps: float):
    N, K = w.shape
    p_ref = torch.full((N, K // 4), 0xEE, dtype=torch.uint8, device=DEV)
    s_ref = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, tw.bitnet_pack_workspace_bytes(N, K) // 8), dtype=torch.float64, device=DEV)
    tw.bitnet_pack_weights(w, eps, p_ref, s_ref, ws)
    p = torch.full((N, K // 4), 0x11, dtype=torch.uint8, device=DEV)
    s = torch.full((1,), -2.0, dtype=torch.float32, device=DEV)
    tw.bitnet_pack_weights_noalloc(w, eps, p, s)
    torch.cuda.synchronize()
    return p, s, p_ref, s_ref


def test_noalloc_rejects_rows_beyond_scratch():
    L = tw.lib()
    assert tw.PACK_NOALLOC_MAX_ROWS == 262144
    # checked on the host before any GPU call: runs without a GPU too
    st = L.bitnet_pack_weights_noalloc(None, tw.PACK_NOALLOC_MAX_ROWS + 1, 64, 1e-5, None, None, None)
    assert st == 2                                   # BITNET_ERR_SHAPE
    assert L.bitnet_pack_weights_noalloc(None, 4, 64, 1e-5, None, None, None) == 1   # NULL w / s_w


@pytest.mark.gpu
def test_noalloc_pack_matches_workspace_pack():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cases = [(6912, 2560, 1e-5), (640, 2560, 1e-5), (tw.PACK_NOALLOC_MAX_ROWS, 4, 1e-5), (33, 68, 0.0)]
    for i, (N, K, eps) in enumerate(cases):
        print(f"noalloc case {i}: N={N} K={K}", flush=True)
        w = synth.latent_weights(synth.stream_key(990, N, K), N, K, 0.02).to(DEV)
        if i == 3:
            w[:, ::5] = 0.0
        p, s, p_ref, s_ref = _pack_both(w, eps)
        assert s.item() == s_ref.item(), (N, K)
        assert torch.equal(p, p_ref), (N, K)
    # the second call of a pair is smaller and reuses the scratch the first one filled
    w_big = synth.latent_weights(synth.stream_key(991), 4096, 640, 0.05).to(DEV)
    w_small = synth.latent_weights(synth.stream_key(992), 100, 640, 0.01).to(DEV)
    p1, s1, p1r, s1r = _pack_both(w_big, 1e-5)
    p2, s2, p2r, s2r = _pack_both(w_small, 1e-5)
    assert s1.item() == s1r.item() and torch.equal(p1, p1r)
    assert s2.item() == s2r.item() and torch.equal(p2, p2r)
    assert s1.item() != s2.item()
    # an empty tensor writes s_w = 0, like the workspace entry point
    z = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    s0 = torch.full((1,), 5.0, dtype=torch.float32, device=DEV)
    tw.bitnet_pack_weights_noalloc(z, 1e-5, torch.empty((0, 16), dtype=torch.uint8, device=DEV), s0)
    torch.cuda.synchronize()
    assert s0.item() == 0.0
    # and on a stream other than the default one, ordered behind the data it reads
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        p3 = torch.empty_like(p1r)
        s3 = torch.empty_like(s1r)
        tw.bitnet_pack_weights_noalloc(w_big, 1e-5, p3, s3)
    st.synchronize()
    assert s3.item() == s1r.item() and torch.equal(p3, p1r)
