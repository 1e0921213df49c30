"""fd_graph_enable: the decode step recorded once as a HIP graph and
replayed every frame ([FD] §4.6 "Inference Optimization" item (2) names the
optimisation), against plain launches.  A replay runs the same kernels with
the same arguments, so every frame must match plain launches bit for bit:
with latent and pixel buffers that change from frame to frame, a reset, the
program's own device work and synchronisations between replays, and the
graph dropped and recorded again in the middle of a stream.
"""
import numpy as np
import pytest

import transformer_latent_pixel_amd as fd
import workloads as W
from gpu_util import dev, multi_tile_cfg, say, torch_cuda

pytestmark = pytest.mark.gpu

PAPER = dict(n_kv_heads=2, norm="rms", kv_norm=True, rope=True)

CASES = {
    "tiny": lambda: W.CONFIGS["tiny"],
    "multi_tile": lambda: multi_tile_cfg(),
    "paper_block": lambda: multi_tile_cfg(**PAPER),
    "tail": lambda: multi_tile_cfg(**dict(PAPER, n_refine=1, n_layers=1)),
    "two_streams": lambda: multi_tile_cfg(batch=2, n_layers=1),
    "window_3": lambda: multi_tile_cfg(window=3, n_layers=1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_plain_launches(name):
    torch = torch_cuda()
    cfg = CASES[name]()
    frames = 7
    weights = W.make_weights(cfg)
    zs = (W.make_batched_latents(cfg, frames=frames) if cfg.batch > 1
          else W.make_latents(cfg, frames=frames))
    shape = cfg.pixel_shape if cfg.batch == 1 else (cfg.batch,) + cfg.pixel_shape
    s_plain, s_graph = torch.cuda.Stream(), torch.cuda.Stream()
    plain = fd.Decoder(cfg, weights, stream=s_plain)
    graph = fd.Decoder(cfg, weights, stream=s_graph)
    try:
        graph.graph_enable(True)
        # profiling makes per-launch records, which a replay cannot
        with pytest.raises(fd.FdError):
            graph.profile_enable(True)
        lat = [dev(np.asarray(z, np.float32)) for z in zs]     # a buffer per frame
        pix_p = torch.empty(shape, dtype=torch.float32, device="cuda")
        pix_g = [torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
                 for _ in range(2)]                             # alternating outputs
        torch.cuda.synchronize()
        for t in range(frames):
            if t == 3:
                plain.reset()
                graph.reset()
            if t == 5:
                graph.graph_enable(False)
                graph.graph_enable(True)
            out = pix_g[t % 2]
            plain.decode_frame(lat[t], pix_p)
            graph.decode_frame(lat[t], out)
            # the program's own device work between replays
            float(torch.randn(1 << 20, device="cuda").abs().sum())
            torch.cuda.synchronize()
            a, b = pix_p.cpu().numpy(), out.cpu().numpy()
            diff = int((a.view(np.uint32) != b.view(np.uint32)).sum())
            say(f"graph {name} frame {t}: {diff} of {a.size} pixels differ")
            assert np.isfinite(b).all()
            assert diff == 0
        qp, qg = plain.query(), graph.query()
        assert qp["frames_decoded"] == qg["frames_decoded"] == frames - 3
        assert qp["slot_frame"] == qg["slot_frame"]
    finally:
        plain.close()
        graph.close()


def test_graph_needs_a_stream_of_its_own():
    torch_cuda()
    cfg = W.CONFIGS["tiny"]
    dec = fd.Decoder(cfg, W.make_weights(cfg))          # legacy default stream
    try:
        with pytest.raises(fd.FdError) as e:
            dec.graph_enable(True)
        assert e.value.status == fd.FD_ERR_UNSUPPORTED
        dec.graph_enable(False)                          # nothing to drop: fine
    finally:
        dec.close()


@pytest.mark.parametrize("where", ["replay", "recording"])
def test_graph_mode_keeps_the_device_error_contract(where):
    # An injected launch failure (host side: nothing faulty reaches the GPU)
    # while a graph is replayed, or while it is being recorded, breaks the
    # handle like any failed launch; later calls report FD_ERR_STATE.
    torch = torch_cuda()
    cfg = W.CONFIGS["tiny"]
    zs = W.make_latents(cfg, frames=2)
    s = torch.cuda.Stream()
    dec = fd.Decoder(cfg, W.make_weights(cfg), stream=s)
    lib = fd.load_library()
    h = dec.handle
    try:
        lat = dev(np.asarray(zs[0], np.float32))
        pix = torch.empty(cfg.pixel_shape, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        if where == "replay":
            dec.graph_enable(True)
            dec.decode_frame(lat, pix)
            dec.debug_fail_after(1)              # the buffer launch goes, the replay "fails"
            assert lib.fd_decode_frame(h, lat.data_ptr(), pix.data_ptr()) == fd.FD_ERR_DEVICE
        else:
            dec.debug_fail_after(3)              # the fourth recorded launch "fails"
            assert lib.fd_graph_enable(h, 1) == fd.FD_ERR_DEVICE
        s.synchronize()
        assert lib.fd_decode_frame(h, lat.data_ptr(), pix.data_ptr()) == fd.FD_ERR_STATE
        assert lib.fd_graph_enable(h, 1) == fd.FD_ERR_STATE
        assert lib.fd_reset(h) == fd.FD_ERR_STATE
    finally:
        dec.close()                              # fd_destroy on a broken handle
