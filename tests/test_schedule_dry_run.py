"""The pass scheduler and every per-launch check, run on the host in the
library's dry-run mode (no GPU work, no device pointer dereferenced)."""
import pytest

from video_diffusion_vae_amd import synth

FAKE = 1 << 20  # a 256-byte aligned address that is never dereferenced


@pytest.fixture
def dry():
    from video_diffusion_vae_amd import wvd
    wvd.wvd_set_dry_run(True)
    yield wvd
    wvd.wvd_set_dry_run(False)


def plan_for(wvd, c, h, w, deep=False):
    nw = wvd.NUM_WEIGHTS_DEEP if deep else wvd.NUM_WEIGHTS
    n = wvd.wvd_prepared_bytes_n(c, h, w, nw)
    return wvd.wvd_prepare(c, h, w, [FAKE] * nw, wvd.WVD_DTYPE_BF16, FAKE, n, 0)


@pytest.mark.parametrize("cfg", tuple(synth.CONFIGS) + tuple(synth.DEEP_CONFIGS), ids=lambda c: c.name)
def test_every_config_schedules(dry, cfg):
    wvd = dry
    plan = plan_for(wvd, cfg.c, cfg.h, cfg.w, cfg.deep)
    try:
        counts = {}
        for P in sorted(set(cfg.passes) | {1, cfg.T, cfg.T + 3}):
            ws = wvd.wvd_workspace_bytes(plan, cfg.T, P)
            wvd.wvd_decode(plan, FAKE, wvd.WVD_DTYPE_BF16, cfg.T, P, FAKE, FAKE, ws, 0)
            counts[P] = wvd.wvd_last_launch_count(plan)
            assert counts[P] > 0
        # One pass per P latent frames; launches per pass do not depend on P
        # except for pass 0 (no time_conv history) and the frame-0 copies.
        assert counts[cfg.T] == counts[cfg.T + 3]
        assert counts[1] >= counts[cfg.T]
    finally:
        wvd.wvd_destroy(plan)


def test_workspace_depends_on_min_T_P(dry):
    wvd = dry
    plan = plan_for(wvd, 64, 22, 39)
    try:
        assert wvd.wvd_workspace_bytes(plan, 3, 5) == wvd.wvd_workspace_bytes(plan, 3, 3)
        assert wvd.wvd_workspace_bytes(plan, 9, 1) < wvd.wvd_workspace_bytes(plan, 9, 2)
        ws = wvd.wvd_workspace_bytes(plan, 3, 3)
        with pytest.raises(wvd.WvdError) as e:
            wvd.wvd_decode(plan, FAKE, 0, 3, 3, FAKE, FAKE, ws - 1, 0)
        assert e.value.status == wvd.WVD_ENOSPACE
        with pytest.raises(wvd.WvdError) as e:
            wvd.wvd_decode(plan, FAKE, 5, 3, 3, FAKE, FAKE, ws, 0)  # unknown latent dtype
        assert e.value.status == wvd.WVD_EINVAL
        for bad in ((0, 1), (3, 0)):
            with pytest.raises(wvd.WvdError) as e:
                wvd.wvd_decode(plan, FAKE, 0, bad[0], bad[1], FAKE, FAKE, ws, 0)
            assert e.value.status == wvd.WVD_EINVAL
        with pytest.raises(wvd.WvdError) as e:
            wvd.wvd_decode(plan, FAKE, 0, 3, 3, FAKE, FAKE + 8, ws, 0)  # misaligned workspace
        assert e.value.status == wvd.WVD_EINVAL
    finally:
        wvd.wvd_destroy(plan)


def test_workspace_fits_288GB_at_the_largest_sweep_point(dry):
    wvd = dry
    plan = plan_for(wvd, 256, 44, 78)
    try:
        sizes = {P: wvd.wvd_workspace_bytes(plan, 121, P) for P in (2, 4, 8, 16)}
        assert sizes[2] < sizes[4] < sizes[8] < sizes[16] < 200e9
        # X, H and Y are sized by what each holds (H: the fused Winograd
        # blocks keep conv1's output only in the history ring; Y: at most the
        # level-3 activation at width c), not three copies of the widest
        # activation: 51.6 GiB at P=16 and 14.9 GiB at P=4, against 70.8 and
        # 19.8 GiB with three widest buffers
        assert sizes[16] < 56 * 2**30 and sizes[4] < 16 * 2**30
    finally:
        wvd.wvd_destroy(plan)


def test_chunked_decode_schedules_and_validates(dry):
    """wvd_decode_chunk: the chunks of a clip walk the same per-pass schedule
    as the whole clip (same launches when the chunks fall on pass
    boundaries), and bad states, offsets and workspaces are rejected."""
    wvd = dry
    plan = plan_for(wvd, 64, 22, 39)
    try:
        sb = wvd.wvd_state_bytes(plan)
        assert sb > 0
        ws = wvd.wvd_workspace_bytes(plan, 4, 2)
        cws = wvd.wvd_chunk_workspace_bytes(plan, 2, 2)
        assert cws + sb <= ws  # the whole-clip workspace holds the rings itself
        wvd.wvd_decode(plan, FAKE, 0, 4, 2, FAKE, FAKE, ws, 0)
        whole = wvd.wvd_last_launch_count(plan)
        n = 0
        for t0 in (0, 2):
            wvd.wvd_decode_chunk(plan, FAKE, 0, 2, t0, 2, FAKE, sb, FAKE, FAKE, cws, 0)
            n += wvd.wvd_last_launch_count(plan)
        assert n == whole
        bad = [
            (dict(state_bytes=sb - 1), wvd.WVD_ENOSPACE),
            (dict(ws_bytes=cws - 1), wvd.WVD_ENOSPACE),
            (dict(t_begin=-1), wvd.WVD_EINVAL),
            (dict(state_ptr=0), wvd.WVD_EINVAL),
            (dict(state_ptr=FAKE + 8), wvd.WVD_EINVAL),
            (dict(T=0), wvd.WVD_EINVAL),
        ]
        for kw, status in bad:
            a = dict(T=2, t_begin=2, state_ptr=FAKE, state_bytes=sb, ws_bytes=cws)
            a.update(kw)
            with pytest.raises(wvd.WvdError) as e:
                wvd.wvd_decode_chunk(plan, FAKE, 0, a["T"], a["t_begin"], 2, a["state_ptr"], a["state_bytes"], FAKE,
                                     FAKE, a["ws_bytes"], 0)
            assert e.value.status == status, kw
    finally:
        wvd.wvd_destroy(plan)


def test_deep_variant_has_more_launches_and_weights(dry):
    """The deep variant prepares more bytes, keeps more rings in its stream
    state, and launches more kernels per pass than the 84-tensor decoder."""
    wvd = dry
    base, deep = plan_for(wvd, 64, 22, 39), plan_for(wvd, 64, 22, 39, deep=True)
    try:
        assert wvd.wvd_prepared_bytes_n(64, 22, 39, 110) > wvd.wvd_prepared_bytes(64, 22, 39)
        assert wvd.wvd_state_bytes(deep) > wvd.wvd_state_bytes(base)
        counts = []
        for plan in (base, deep):
            ws = wvd.wvd_workspace_bytes(plan, 3, 3)
            wvd.wvd_decode(plan, FAKE, 0, 3, 3, FAKE, FAKE, ws, 0)
            counts.append(wvd.wvd_last_launch_count(plan))
        assert counts[1] > counts[0]
        for bad in (83, 85, 109, 111):
            with pytest.raises(wvd.WvdError):
                wvd.wvd_prepared_bytes_n(64, 22, 39, bad)
    finally:
        wvd.wvd_destroy(base)
        wvd.wvd_destroy(deep)


def test_static_decode_checks_its_workspace_limit(dry):
    """wvd_decode_static takes its workspace from the library's static array:
    decodes that fit run their schedule, larger ones are refused on the host."""
    wvd = dry
    plan = plan_for(wvd, 16, 4, 6)
    try:
        assert wvd.wvd_workspace_bytes(plan, 4, 4) <= wvd.WVD_STATIC_WORKSPACE_BYTES
        wvd.wvd_decode_static(plan, FAKE, wvd.WVD_DTYPE_BF16, 4, 4, FAKE, 0)
        assert wvd.wvd_last_launch_count(plan) > 0
    finally:
        wvd.wvd_destroy(plan)
    plan = plan_for(wvd, 64, 22, 39)
    try:
        assert wvd.wvd_workspace_bytes(plan, 3, 1) > wvd.WVD_STATIC_WORKSPACE_BYTES
        with pytest.raises(wvd.WvdError) as e:
            wvd.wvd_decode_static(plan, FAKE, wvd.WVD_DTYPE_BF16, 3, 1, FAKE, 0)
        assert e.value.status == wvd.WVD_ENOSPACE and "static workspace" in str(e.value)
        for bad in ((0, 1), (3, 0)):
            with pytest.raises(wvd.WvdError) as e:
                wvd.wvd_decode_static(plan, FAKE, wvd.WVD_DTYPE_BF16, bad[0], bad[1], FAKE, 0)
            assert e.value.status == wvd.WVD_EINVAL
    finally:
        wvd.wvd_destroy(plan)


@pytest.mark.parametrize("cfg", __import__("video_diffusion_vae_amd.synth_encoder", fromlist=["x"]).ENCODER_CONFIGS,
                         ids=lambda c: c.name)
def test_every_encoder_config_schedules(dry, cfg):
    """The encoder's pass scheduler and per-launch checks for every workload
    and frames_per_pass; decoder calls refuse an encoder plan."""
    wvd = dry
    n = wvd.wvd_encoder_prepared_bytes(cfg.c, cfg.h, cfg.w)
    plan = wvd.wvd_encoder_prepare(cfg.c, cfg.h, cfg.w, [FAKE] * wvd.NUM_WEIGHTS_ENCODER, wvd.WVD_DTYPE_BF16, FAKE,
                                   n, 0)
    try:
        counts = {}
        for P in sorted(set(cfg.passes) | {1, cfg.T, cfg.T + 3}):
            ws = wvd.wvd_encode_workspace_bytes(plan, cfg.T, P)
            wvd.wvd_encode(plan, FAKE, wvd.WVD_DTYPE_BF16, cfg.T, P, FAKE, FAKE, ws, 0)
            counts[P] = wvd.wvd_last_launch_count(plan)
            assert counts[P] > 0
            with pytest.raises(wvd.WvdError) as e:
                wvd.wvd_encode(plan, FAKE, wvd.WVD_DTYPE_BF16, cfg.T, P, FAKE, FAKE, ws - 1, 0)
            assert e.value.status == wvd.WVD_ENOSPACE
        assert counts[cfg.T] == counts[cfg.T + 3]
        with pytest.raises(wvd.WvdError) as e:
            wvd.wvd_workspace_bytes(plan, cfg.T, 1)
        assert e.value.status == wvd.WVD_EINVAL
    finally:
        wvd.wvd_destroy(plan)
    dplan = plan_for(wvd, cfg.c, cfg.h, cfg.w)
    try:
        with pytest.raises(wvd.WvdError) as e:
            wvd.wvd_encode_workspace_bytes(dplan, cfg.T, 1)
        assert e.value.status == wvd.WVD_EINVAL
    finally:
        wvd.wvd_destroy(dplan)
    with pytest.raises(wvd.WvdError) as e:
        wvd.wvd_encoder_prepare(cfg.c, cfg.h, cfg.w, [FAKE] * wvd.NUM_WEIGHTS_DEEP, wvd.WVD_DTYPE_BF16, FAKE, n, 0)
    assert e.value.status == wvd.WVD_EINVAL
