"""A decode step (route_score_topk + routed_attention) captured in a HIP graph.

The graph is replayed several times, with fresh tail queries and hidden states
copied into the captured buffers and unrelated eager work between replays;
every replay must equal the eager call on the same inputs bit for bit (the
kernels are deterministic, and they clear nothing with memset, so a replay has
nothing to redo). The first and the last replay are also checked against the
fp64 oracle on the inputs copied back from the device.
"""
import numpy as np
import pytest
import torch

import learned_chunk_routed_amd as lcr
from lcr_inputs import get_config, route_inputs
from oracle import route as O
from gpu_util import to_dev, f64, check_selection, max_err, OUT_TOL

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    cfg = get_config("tiny_fp32", N=64, Hq=8, Hkv=2, d=128, r=32, D=256, K=8, R=128, dtype="bf16")
    print("[case] graph replay: decode step, 32 tail queries, bf16", flush=True)
    inp = route_inputs(cfg)
    dev = {k: to_dev(v) for k, v in inp.items()}
    q, k, v, x, A, Bm = (dev[n] for n in ["q", "k", "v", "x", "A", "Bm"])
    s, H = lcr.chunk_summary(q, k, cfg.scale)
    nq, q0 = 32, cfg.T - 32
    i_tail = np.arange(q0, cfg.T)
    slots = torch.from_numpy((i_tail // 63) * 64 + i_tail % 63).cuda()
    B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    dims = lcr.make_dims(B, Hq, Hkv, N, d, q.dtype)
    idx = torch.empty((B, Hkv, nq, cfg.K), dtype=torch.int32, device="cuda")
    zsel = torch.empty((B, Hq, nq, cfg.K), dtype=torch.float32, device="cuda")
    out = torch.zeros_like(q)
    ws_s = torch.empty(max(1, lcr.workspace_bytes(1, dims, cfg.D, cfg.r, cfg.K, nq)), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, lcr.workspace_bytes(2, dims, 0, 0, cfg.K, nq, cfg.R)), dtype=torch.uint8, device="cuda")

    def step():
        lcr.route_score_topk(q, x, A, Bm, s, H, Hkv=Hkv, K=cfg.K, radius=cfg.R, scale=cfg.scale, q0=q0, nq=nq,
                             idx=idx, zsel=zsel, ws=ws_s)
        lcr.routed_attention(q, k, v, idx, zsel, radius=cfg.R, scale=cfg.scale, q0=q0, nq=nq, out=out, ws=ws_a)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up outside the capture (function attributes, lazy loading)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu").manual_seed(1234)
    for rep in range(4):
        q[:, :, slots] = torch.randn((B, Hq, nq, d), generator=gen).to(q.dtype).cuda()
        x[:, slots] = torch.randn((B, nq, cfg.D), generator=gen).to(x.dtype).cuda()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = (idx.clone(), zsel.clone(), out[:, :, slots].clone())
        # unrelated eager work between the replay and the reference call
        junk = torch.randn((512, 512), device="cuda") @ torch.randn((512, 512), device="cuda")
        float(junk.sum())
        out.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], idx), f"replay {rep}: idx"
        assert torch.equal(got[1], zsel), f"replay {rep}: zsel"
        assert torch.equal(got[2], out[:, :, slots]), f"replay {rep}: output"
        assert bool(torch.isfinite(got[2].float()).all()), f"replay {rep}: non-finite output"
        if rep in (0, 3):
            _replay_against_oracle(cfg, q, k, v, x, A, Bm, i_tail, got, rep)


def _replay_against_oracle(cfg, q, k, v, x, A, Bm, i_tail, got, rep):
    """The replayed step's selection and output against the oracle on the same bits."""
    ref = O.route_layer(f64(q), f64(k), f64(v), f64(x), f64(A), f64(Bm), K=cfg.K, R=cfg.R, beta=cfg.beta,
                        scale=cfg.scale, queries=i_tail)
    idx_gpu = got[0].cpu().numpy().astype(np.int64)
    same = check_selection(idx_gpu, ref, cfg.K, f"graph replay {rep}")
    zref = O.gather_zsel(ref["z"], idx_gpu, cfg.G)
    o_ref = ref["o"].copy()
    diff_t = np.nonzero(~same.all(axis=(0, 1)))[0]
    if len(diff_t):
        qr = f64(q)[:, :, O.slot_of(i_tail[diff_t])]
        o_ref[:, :, diff_t], _ = O.routed_attention(qr, f64(k), f64(v), idx_gpu[:, :, diff_t], zref[:, :, diff_t],
                                                    cfg.R, cfg.scale, i_tail[diff_t])
    o_err = max_err(f64(got[2]), o_ref)
    fin = np.isfinite(zref)
    z_err = max_err(f64(got[1])[fin], zref[fin])
    print(f"    replay {rep}: idx_same={int(same.sum())}/{same.size} o_err={o_err:.2e} z_err={z_err:.2e}", flush=True)
    assert o_err < OUT_TOL["bf16"] and z_err < 5e-5 * max(1.0, np.abs(zref[fin]).max())
