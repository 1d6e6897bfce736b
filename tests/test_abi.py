"""C ABI checks that need no GPU: symbols, configuration and argument validation."""
import ctypes

import pytest

from diffusion_transformer_joint_amd import flux_attn as fa


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    names = fa.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.flux_attn_abi_version() == 2
    assert lib.flux_attn_status_string(0) == b"ok"
    assert lib.flux_attn_status_string(1) == b"invalid argument"
    assert lib.flux_attn_status_string(99) == b"unknown status"


def test_default_config(lib):
    cfg = fa.default_config(1, 24, 128, 8704)
    assert list(cfg.rope_axes_dim) == [32, 48, 48]
    assert cfg.rope_theta == 10000.0 and cfg.max_segments == 12 and cfg.dtype == fa.BF16
    assert lib.flux_attn_validate_config(ctypes.byref(cfg)) == fa.OK
    cfg64 = fa.default_config(1, 2, 64, 80)
    assert list(cfg64.rope_axes_dim) == [16, 24, 24]


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, fa.INVALID_ARGUMENT),
    ("num_heads", 0, fa.INVALID_ARGUMENT),
    ("head_dim", 96, fa.UNSUPPORTED),
    ("max_tokens", 0, fa.INVALID_ARGUMENT),
    ("max_segments", 0, fa.INVALID_ARGUMENT),
    ("rope_theta", 0.0, fa.INVALID_ARGUMENT),
    ("rope_theta", float("inf"), fa.INVALID_ARGUMENT),
    ("softmax_scale", float("nan"), fa.INVALID_ARGUMENT),
    ("dtype", 7, fa.INVALID_ARGUMENT),
])
def test_invalid_config(lib, field, value, status):
    cfg = fa.default_config(1, 24, 128, 8704)
    setattr(cfg, field, value)
    assert lib.flux_attn_validate_config(ctypes.byref(cfg)) == status
    assert fa.last_error() != ""


@pytest.mark.parametrize("axes", [(32, 48, 40), (30, 50, 48), (-8, 88, 48)])
def test_invalid_axes(lib, axes):
    cfg = fa.default_config(1, 24, 128, 8704, rope_axes_dim=axes)
    assert lib.flux_attn_validate_config(ctypes.byref(cfg)) == fa.INVALID_ARGUMENT


# fake, aligned, non-overlapping device addresses: validation never dereferences them
A = 1 << 40
Q, K, V, O, POS, SC = A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A


def vf(lib, cfg, segs, q=Q, k=K, v=V, sc=None, pos=POS, out=O, nseg=None):
    arr = fa._i32_array(segs) if segs is not None else None
    return lib.flux_attn_validate_forward(ctypes.byref(cfg), q, k, v, sc, arr,
                                          len(segs) if nseg is None else nseg, pos, out)


def test_validate_forward_ok(lib):
    cfg = fa.default_config(1, 24, 128, 8704)
    assert vf(lib, cfg, [512, 4096, 4096]) == fa.OK
    assert vf(lib, cfg, [0, 7, 0]) == fa.OK


@pytest.mark.parametrize("case", [
    "too_many_tokens", "zero_tokens", "negative_segment", "too_many_segments", "null_q", "null_out",
    "null_pos", "unaligned_q", "unaligned_pos", "scale_on_bf16", "overlap", "null_segments",
])
def test_validate_forward_errors(lib, case):
    cfg = fa.default_config(1, 24, 128, 8704)
    kw = {}
    segs = [512, 4096, 4096]
    if case == "too_many_tokens":
        segs = [512, 4096, 4097]
    elif case == "zero_tokens":
        segs = [0, 0]
    elif case == "negative_segment":
        segs = [512, -1, 4096]
    elif case == "too_many_segments":
        segs = [1] * 13
    elif case == "null_q":
        kw["q"] = None
    elif case == "null_out":
        kw["out"] = None
    elif case == "null_pos":
        kw["pos"] = None
    elif case == "unaligned_q":
        kw["q"] = Q + 8
    elif case == "unaligned_pos":
        kw["pos"] = POS + 2
    elif case == "scale_on_bf16":
        kw["sc"] = SC
    elif case == "overlap":
        kw["out"] = Q + 4096
    elif case == "null_segments":
        assert lib.flux_attn_validate_forward(ctypes.byref(cfg), Q, K, V, None, None, 3, POS, O) \
            == fa.INVALID_ARGUMENT
        return
    assert vf(lib, cfg, segs, **kw) == fa.INVALID_ARGUMENT
    assert fa.last_error() != ""


def test_fp8_requires_scales(lib):
    cfg = fa.default_config(1, 24, 128, 66048, dtype="fp8")
    assert vf(lib, cfg, [512, 65536]) == fa.INVALID_ARGUMENT
    assert vf(lib, cfg, [512, 65536], sc=SC) == fa.OK


def test_plan_handles_rejected_without_dereference(lib):
    assert lib.flux_attn_destroy(None) == fa.OK
    assert lib.flux_attn_destroy(0x1234560) == fa.INVALID_ARGUMENT
    segs = fa._i32_array([80])
    for fn in (lib.flux_attn_forward, lib.flux_attn_forward_segment_local):
        assert fn(None, Q, K, V, None, segs, 1, POS, O, None) == fa.INVALID_ARGUMENT
        assert fn(0x1234560, Q, K, V, None, segs, 1, POS, O, None) == fa.INVALID_ARGUMENT
    cfg = fa.Config()
    assert lib.flux_attn_get_config(None, ctypes.byref(cfg)) == fa.INVALID_ARGUMENT
    assert lib.flux_attn_create(None, None) == fa.INVALID_ARGUMENT


def test_batch_entry_over_4gib_is_unsupported(lib):
    # the kernels address one batch entry of q/k/v through 32-bit buffer ranges
    cfg = fa.default_config(1, 24, 128, 699050)           # 699,050 x 3,072 x 2 B < 4 GiB
    assert lib.flux_attn_validate_config(ctypes.byref(cfg)) == fa.OK
    cfg = fa.default_config(1, 24, 128, 699051)           # 699,051 x 3,072 x 2 B >= 4 GiB
    assert lib.flux_attn_validate_config(ctypes.byref(cfg)) == fa.UNSUPPORTED
    assert "4 GiB" in fa.last_error()
    cfg = fa.default_config(1, 24, 128, 699051, dtype="fp8")  # 1 B per e4m3 code: fits
    assert lib.flux_attn_validate_config(ctypes.byref(cfg)) == fa.OK
    cfg = fa.default_config(4, 24, 128, 600000)           # the limit is per batch entry
    assert lib.flux_attn_validate_config(ctypes.byref(cfg)) == fa.OK


def test_wrapper_rejects_host_tensors():
    # the C side cannot tell host from device pointers; the binding refuses
    # anything that is not a device tensor before any call
    import torch
    x = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FluxAttnError, match="must be a tensor on"):
        fa._device_tensor("out", x, torch.device("cuda:0"))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(fa.FluxAttnError):
        fa.load_library(str(tmp_path / "nope.so"))


# ---------------------------------------------------------------------------
# host scheduling policy (split of the last round of query tiles)

@pytest.mark.parametrize("tiles,kv,cus", [(816, 136, 256), (432, 72, 256), (102, 136, 256), (2352, 392, 256),
                                          (2, 2, 256), (256, 136, 256), (512, 64, 256), (6192, 1032, 256),
                                          (1, 1, 256), (300, 5, 80)])
def test_schedule_invariants(tiles, kv, cus):
    cap = 4 * cus
    s = fa.schedule(tiles, kv, cus, cap)
    assert s["whole_tiles"] + s["split_tiles"] == tiles
    assert s["grid"] == s["whole_tiles"] + s["split_tiles"] * s["split"]
    assert 1 <= s["split"] <= max(1, min(16, kv))
    if s["split_tiles"]:
        assert s["split"] >= 2 and s["split_tiles"] * s["split"] <= cap
        assert s["whole_tiles"] % cus == 0          # whole tiles fill complete rounds
    else:
        assert s["split"] == 1 and s["grid"] == tiles


def test_schedule_no_split_when_rounds_are_full():
    for tiles in (256, 512, 768):
        s = fa.schedule(tiles, 136, 256, 1024)
        assert s["split_tiles"] == 0 and s["grid"] == tiles


def test_schedule_fills_last_round():
    # 8,704 tokens x 24 heads: 816 tiles = 3.19 rounds on 256 units; the 48 left
    # over are cut so the final round is short instead of a fourth full round
    s = fa.schedule(816, 136, 256, 1024)
    assert s["whole_tiles"] == 768 and s["split_tiles"] == 48 and s["split"] >= 4
    # one GPU's share of an 8-way head split (3 heads): fewer tiles than units
    s = fa.schedule(102, 136, 256, 1024)
    assert s["whole_tiles"] == 0 and s["split"] >= 2 and s["grid"] >= 200


def test_schedule_keeps_a_large_last_round_whole():
    # 4,608 tokens x 24 heads: 432 tiles, 1.69 rounds.  Cutting the 176 tiles
    # of the second round into pieces saves less loop time than the ~8 us
    # each extra work item and the merge of its partials cost, so the call
    # runs unsplit; the 8,704-token call (0.19 of a round left) still splits.
    s = fa.schedule(432, 72, 256, 1024)
    assert s["split_tiles"] == 0 and s["grid"] == 432
    assert fa.schedule(816, 136, 256, 1024)["split_tiles"] == 48


def test_schedule_respects_piece_cap():
    s = fa.schedule(432, 72, 256, 300)
    assert s["split_tiles"] * s["split"] <= 300 or s["split_tiles"] == 0
