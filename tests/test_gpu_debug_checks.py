"""Debug checks of the decode length precondition, through the C ABI.

With debug checks on, every decode entry point has the device test
s_q <= seqlens_k[b] <= L_cap before anything else runs: a good call gives the
same bits as with the checks off, and a length out of range is refused with
GHA_ERR_PRECONDITION, naming the sequence, before any decode kernel runs (the
output buffer keeps its sentinel).  Inputs are seeded torch normals; these
tests compare the library with itself, the values are checked against the
oracle elsewhere."""
import pytest

import grouped_head_latent_amd as gha

pytestmark = pytest.mark.gpu

PRECONDITION = gha.STATUS.index("GHA_ERR_PRECONDITION")
SENTINEL = 3.0


def _randn(shape, seed, std=1.0):
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16).cuda()


def _lengths(vals):
    import torch
    return torch.tensor(vals, dtype=torch.int32, device="cuda")


def _case_gqa(h_q, h_kv, s_q, d):
    B, L_cap = 3, 256
    q = _randn((B, h_q, s_q, d), 1)
    k, v = _randn((B, h_kv, L_cap, d), 2), _randn((B, h_kv, L_cap, d), 3)
    return B, s_q, L_cap, (B, h_q, s_q, d), lambda sl, out: gha.gqa_decode(q, k, v, sl, out=out)


def _case_noalloc():
    B, h_q, h_kv, s_q, d, L_cap = 3, 8, 2, 2, 128, 256
    q = _randn((B, h_q, s_q, d), 4)
    k, v = _randn((B, h_kv, L_cap, d), 5), _randn((B, h_kv, L_cap, d), 6)
    return B, s_q, L_cap, (B, h_q, s_q, d), lambda sl, out: gha.gqa_decode_noalloc(q, k, v, sl, out=out)


def _case_paged(window):
    import torch
    B, h_q, h_kv, s_q, d, page, per_seq = 3, 8, 2, 1, 128, 64, 4
    q = _randn((B, h_q, s_q, d), 7)
    k, v = _randn((B * per_seq, h_kv, page, d), 8), _randn((B * per_seq, h_kv, page, d), 9)
    g = torch.Generator(device="cpu").manual_seed(10)
    bt = torch.randperm(B * per_seq, generator=g).to(torch.int32).reshape(B, per_seq).cuda()
    return B, s_q, page * per_seq, (B, h_q, s_q, d), lambda sl, out: gha.gqa_decode_paged(
        q, k, v, sl, block_table=bt, page_size=page, window=window, out=out)


def _case_fp8():
    import torch
    B, h_q, h_kv, s_q, d, L_cap = 3, 8, 2, 2, 64, 256
    q = _randn((B, h_q, s_q, d), 11)
    g = torch.Generator(device="cpu").manual_seed(12)
    # finite E4M3 codes only (0x7f and 0xff are NaN)
    kc = torch.randint(0, 0x7f, (B, h_kv, L_cap, d), generator=g, dtype=torch.uint8).cuda()
    vc = torch.randint(0, 0x7f, (B, h_kv, L_cap, d), generator=g, dtype=torch.uint8).cuda()
    return B, s_q, L_cap, (B, h_q, s_q, d), lambda sl, out: gha.gqa_decode_fp8(
        q, kc, vc, sl, k_scale=1 / 64, v_scale=1 / 64, out=out)


def _case_gta():
    B, h, n_grp, s_q, d, L_cap = 3, 8, 2, 2, 64, 256
    q, k = _randn((B, n_grp, s_q, d), 13), _randn((B, n_grp, L_cap, d), 14)
    v = _randn((B, h, L_cap, d), 15)
    return B, s_q, L_cap, (B, h, s_q, d), lambda sl, out: gha.gta_shared_score_decode(q, k, v, sl, out=out)


def _case_gqla():
    B, h_q, g, s_q, L_cap = 3, 16, 2, 2, 256
    qc, qr = _randn((B, h_q, s_q, 128), 16), _randn((B, h_q, s_q, 64), 17)
    kc, kr, v = _randn((B, g, L_cap, 128), 18, 0.45), _randn((B, L_cap, 64), 19), _randn((B, g, L_cap, 128), 20, 0.45)
    return B, s_q, L_cap, (B, h_q, s_q, 128), lambda sl, out: gha.gqla_gqa_decode(
        qc, qr, kc, kr, v, sl, scale=192 ** -0.5, out=out)


def _case_latent():
    B, h_q, s_q, L_cap = 3, 16, 1, 256
    ql, qr = _randn((B, s_q, h_q, 512), 21, 0.25), _randn((B, s_q, h_q, 64), 22)
    cache = _randn((B, L_cap, 576), 23)
    return B, s_q, L_cap, (B, s_q, h_q, 512), lambda sl, out: gha.latent_absorb_decode(
        ql, qr, cache[..., :512], cache[..., 512:], sl, scale=192 ** -0.5, out=out)


def _case_absorb():
    B, h_q, g, s_q, L_cap = 2, 16, 2, 1, 256
    qc, qr = _randn((B, s_q, h_q, 128), 24), _randn((B, s_q, h_q, 64), 25)
    w_uk, w_uv = _randn((g * 128, 512), 26, 0.02), _randn((g * 128, 512), 27, 0.02)
    cache = _randn((B, L_cap, 576), 28)
    return B, s_q, L_cap, (B, s_q, h_q, 128), lambda sl, out: gha.gqla_absorb_decode(
        qc, qr, w_uk, w_uv, cache[..., :512], cache[..., 512:], sl, g=g, scale=192 ** -0.5, out=out)


CASES = {
    "gqa_decode_streaming": lambda: _case_gqa(8, 2, 2, 128),
    "gqa_decode_register": lambda: _case_gqa(64, 1, 1, 128),
    "gqa_decode_noalloc": _case_noalloc,
    "gqa_decode_paged": lambda: _case_paged(0),
    "gqa_decode_paged_window": lambda: _case_paged(100),
    "gqa_decode_fp8": _case_fp8,
    "gta_shared_score_decode": _case_gta,
    "gqla_gqa_decode": _case_gqla,
    "latent_absorb_decode": _case_latent,
    "gqla_absorb_decode": _case_absorb,
}


@pytest.fixture
def debug_on():
    before = gha.debug_checks()
    gha.set_debug_checks(True)
    yield
    gha.set_debug_checks(before)


@pytest.mark.parametrize("name", list(CASES))
def test_debug_checks_pass_good_lengths_and_refuse_bad_ones(name, debug_on):
    import torch
    print(f"[case] {name}", flush=True)
    B, s_q, L_cap, out_shape, call = CASES[name]()
    good = [s_q, L_cap, (s_q + L_cap) // 2][:B]
    out_on = torch.full(out_shape, SENTINEL, dtype=torch.float32, device="cuda")
    call(_lengths(good), out_on)
    gha.set_debug_checks(False)
    out_off = torch.full(out_shape, SENTINEL, dtype=torch.float32, device="cuda")
    call(_lengths(good), out_off)
    gha.set_debug_checks(True)
    torch.cuda.synchronize()
    assert torch.isfinite(out_on).all()
    assert torch.equal(out_on, out_off)

    for b, bad in ((1, s_q - 1), (B - 1, L_cap + 1), (0, -5)):
        lengths = list(good)
        lengths[b] = bad
        out = torch.full(out_shape, SENTINEL, dtype=torch.float32, device="cuda")
        with pytest.raises(gha.GhaError) as e:
            call(_lengths(lengths), out)
        assert e.value.status == PRECONDITION
        assert f"seqlens_k[{b}] = {bad}" in str(e.value)
        torch.cuda.synchronize()
        assert bool((out == SENTINEL).all()), "nothing may run after a refused length"
