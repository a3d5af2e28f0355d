"""GPU parity: every entry point of the C ABI against the fp64 oracle on the
same seeded inputs.  Each case prints its name first so a failure is easy to
place.  Tolerances: fp32 inputs 1e-5 max abs; bf16 inputs with fp32
accumulation 1e-2 max / 1e-3 mean abs (fp32 outputs); for bf16 outputs an
element may instead be off by half a bf16 ulp of the reference,
max(1e-2, ulp/2).  Every call is made twice and the two results must be
bitwise equal (fixed split plans, no atomics).  At the workloads' full sizes
the whole output must be finite and the oracle checks every sequence (decode)
or every (batch, head) slice (prefill) unless a test says otherwise."""
import math
import sys

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_cases import (bf16_to_torch, cache_bits, e4m3_codes, latent_cache_bits, page_pool,
                             tolerance_ok, widen)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gha_lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import grouped_head_latent_amd as gha
    gha.load_library()
    return gha


def gen(shape, seed, stream):
    return synth.normal_bf16(shape, seed, stream)


def check(name, got, ref, bf16_out=False, **kw):
    ok, mx, mean = tolerance_ok(got, ref, bf16_out=bf16_out, **kw)
    say(f"{name}: max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert ok, f"{name}: max_abs={mx:.3e} mean_abs={mean:.3e}"


def twice(name, fn):
    """Call `fn` twice; the results (a tensor or a tuple of tensors) must be
    bitwise equal.  Returns the first."""
    a = fn()
    b = fn()
    torch.cuda.synchronize()
    for x, y in zip(a if isinstance(a, tuple) else (a,), b if isinstance(b, tuple) else (b,)):
        assert torch.equal(x, y), f"{name}: two calls differ"
    return a


def all_finite(name, t):
    bad = int((~torch.isfinite(t)).sum().item())
    say(f"{name}: {t.numel()} outputs, {bad} non-finite")
    assert bad == 0


# ----------------------------------------------------------------- fp32 path

def test_tiny_gqa_fp32_matches_oracle_and_repeated_heads(gha_lib):
    """Worked GQA example shapes: batch 1, 8 query heads, 2 KV heads, 16
    tokens, head dim 64, fp32, causal, seed 0."""
    say("tiny fp32 GQA (1, 8/2, 16, 64)")
    q = synth.normal_f32((1, 8, 16, 64), 0, synth.STREAM["q"])
    k = synth.normal_f32((1, 2, 16, 64), 0, synth.STREAM["k"])
    v = synth.normal_f32((1, 2, 16, 64), 0, synth.STREAM["v"])
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    o, lse = gha_lib.gqa_prefill(dq, dk, dv, causal=True, return_lse=True)
    o_mha = gha_lib.gqa_prefill(dq, dk.repeat_interleave(4, dim=1).contiguous(),
                                dv.repeat_interleave(4, dim=1).contiguous(), causal=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_prefill(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    err = np.abs(o.cpu().numpy() - ref).max()
    say(f"fp32 max_abs={err:.3e}")
    assert err <= 1e-5
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-5
    assert torch.equal(o, o_mha)


@pytest.mark.parametrize("B,h_q,h_kv,S_q,S_k,d,causal", [
    (2, 4, 2, 150, 150, 128, True),   # ragged: 10 q-tiles, the last of 6 rows
    (1, 2, 1, 65, 65, 64, True),
    (1, 8, 2, 20, 173, 64, True),     # chunked prefill: bottom-right causal
    (2, 3, 3, 40, 33, 128, False),    # MHA, no mask, a key tile of one key
    (1, 4, 1, 1, 1, 64, True),        # one token
])
def test_fp32_prefill_ragged(gha_lib, B, h_q, h_kv, S_q, S_k, d, causal):
    say(f"fp32 prefill B={B} h={h_q}/{h_kv} S_q={S_q} S_k={S_k} d={d} causal={causal}")
    q = synth.normal_f32((B, h_q, S_q, d), 7, 1)
    k = synth.normal_f32((B, h_kv, S_k, d), 7, 2)
    v = synth.normal_f32((B, h_kv, S_k, d), 7, 3)
    o, lse = twice("fp32 prefill", lambda: gha_lib.gqa_prefill(*(torch.from_numpy(x).cuda() for x in (q, k, v)),
                                                               causal=causal, return_lse=True))
    ref, ref_lse = oracle.gqa_prefill(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                      causal=causal)
    err = np.abs(o.cpu().numpy() - ref).max()
    say(f"fp32 max_abs={err:.3e}")
    assert err <= 1e-5
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-5


# ------------------------------------------------------------- bf16 prefill

PREFILL_CASES = [
    # B, h_q, h_kv, S_q, S_k, d, causal
    (2, 8, 2, 200, 200, 128, True),   # ragged tail, 4 heads per group
    (1, 4, 1, 130, 130, 128, True),   # MQA
    (1, 4, 4, 97, 97, 128, True),     # MHA
    (2, 4, 2, 77, 77, 64, True),      # 2 heads per group, d=64
    (1, 6, 3, 64, 64, 64, True),      # 2 heads per group, one exact tile
    (1, 8, 2, 1, 1, 128, True),       # one token
    (1, 8, 2, 70, 300, 128, True),    # chunked prefill: bottom-right causal
    (1, 8, 2, 90, 150, 128, False),   # no mask
    # grids larger than the resident work-groups: heavy and light causal
    # q-blocks paired in one work-group, 35 blocks so the middle one is alone
    (2, 32, 8, 1100, 1100, 128, True),
    (2, 32, 8, 1090, 1400, 128, True),  # paired, bottom-right offset
]


@pytest.mark.parametrize("B,h_q,h_kv,S_q,S_k,d,causal", PREFILL_CASES)
def test_gqa_prefill_bf16(gha_lib, B, h_q, h_kv, S_q, S_k, d, causal):
    say(f"bf16 prefill B={B} h={h_q}/{h_kv} S_q={S_q} S_k={S_k} d={d} causal={causal}")
    qb, kb, vb = gen((B, h_q, S_q, d), 8, 1), gen((B, h_kv, S_k, d), 8, 2), gen((B, h_kv, S_k, d), 8, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    o32, lse = twice("prefill", lambda: gha_lib.gqa_prefill(q, k, v, causal=causal, out_dtype=torch.float32,
                                                            return_lse=True))
    o16 = twice("prefill bf16", lambda: gha_lib.gqa_prefill(q, k, v, causal=causal))
    ref, ref_lse = oracle.gqa_prefill(widen(qb), widen(kb), widen(vb), causal=causal)
    check("o fp32", o32.cpu().numpy(), ref)
    check("o bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("lse", lse.cpu().numpy(), ref_lse)


# The d = 128 prefill kernel reads a (batch, KV head) key or value slice
# through a buffer with 32-bit offsets: it takes S_k while S_k + 256 rows span
# less than 2 GiB; longer ones go to the generic bf16 kernel.
LONGEST_PREFILL_KEYS = (1 << 31) // (2 * 128) - 256 - 1  # 8388351 keys


@pytest.mark.parametrize("S_k", [LONGEST_PREFILL_KEYS, LONGEST_PREFILL_KEYS + 1])
def test_gqa_prefill_longest_keys(gha_lib, S_k):
    """16 causal queries (bottom-right) over the longest key slice the d = 128
    kernel's offsets cover, and one key more (generic kernel); output and lse
    against the oracle."""
    B, h_q, h_kv, S_q, d = 1, 4, 1, 16, 128
    say(f"longest prefill S_k={S_k}")
    qb, kb, vb = gen((B, h_q, S_q, d), 45, 1), gen((B, h_kv, S_k, d), 45, 2), gen((B, h_kv, S_k, d), 45, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    o, lse = gha_lib.gqa_prefill(q, k, v, causal=True, out_dtype=torch.float32, return_lse=True)
    all_finite("longest prefill", o)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    del q, k, v
    torch.cuda.empty_cache()
    ref, ref_lse = oracle.gqa_prefill(widen(qb), widen(kb), widen(vb), causal=True)
    check(f"longest prefill S_k={S_k}", o, ref)
    check(f"longest prefill lse S_k={S_k}", lse, ref_lse)


@pytest.mark.parametrize("heads", [None, (1, 6)])
def test_gqa_prefill_growing_scores(gha_lib, heads):
    """Keys whose scores jump far above the first tile's maximum, twice (key
    rows of three magnitudes, the jumps over 96 in log2 units): a prefill
    kernel that fixes each row's reference from its first tile must replace
    it and start the row block again, and the result is still the softmax.
    With `heads`, only those query heads see the jump; the others have a zero
    query and flat scores."""
    say(f"bf16 prefill growing scores, heads={heads}")
    B, h_q, h_kv, S, d = 1, 8, 2, 600, 128
    kb = gen((B, h_kv, S, d), 46, 2)
    vb = gen((B, h_kv, S, d), 46, 3)
    eight = np.float32(8.0).view(np.uint32) >> 16
    sixteen = np.float32(16.0).view(np.uint32) >> 16
    one = np.float32(1.0).view(np.uint32) >> 16
    kb[:, :, 200:400] = eight
    kb[:, :, 400:] = sixteen
    qb = np.full((B, h_q, S, d), one, dtype=np.uint16)
    if heads is not None:
        qb[:] = 0
        qb[:, list(heads)] = one
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    o, lse = gha_lib.gqa_prefill(q, k, v, causal=True, out_dtype=torch.float32, return_lse=True)
    ref, ref_lse = oracle.gqa_prefill(widen(qb), widen(kb), widen(vb), causal=True)
    check("growing scores", o.cpu().numpy(), ref)
    check("growing scores lse", lse.cpu().numpy(), ref_lse)
    # rows past key 400 of the jumping heads average the values of keys 400 ..
    jumped = list(heads) if heads is not None else list(range(h_q))
    v32 = widen(vb)
    for hq in jumped:
        want = v32[0, hq // 4, 400:451].mean(axis=0)
        assert np.allclose(ref[0, hq, 450], want, atol=1e-6)


def test_gqa_prefill_strided_bshd_layout(gha_lib):
    """(B, S, H, D) memory order passed through the strides."""
    say("bf16 prefill BSHD strides")
    B, h_q, h_kv, S, d = 2, 8, 2, 100, 128
    qb, kb, vb = gen((B, S, h_q, d), 9, 1), gen((B, S, h_kv, d), 9, 2), gen((B, S, h_kv, d), 9, 3)
    q, k, v = (bf16_to_torch(x).transpose(1, 2) for x in (qb, kb, vb))
    o = gha_lib.gqa_prefill(q, k, v, out_dtype=torch.float32)
    ref, _ = oracle.gqa_prefill(*(widen(x).transpose(0, 2, 1, 3) for x in (qb, kb, vb)))
    check("bshd", o.cpu().numpy(), ref)


def test_prefill_invariants(gha_lib):
    """Constant V gives exactly-normalised rows; row 0 returns v_0; two runs
    are bitwise equal."""
    say("prefill invariants")
    B, h_q, h_kv, S, d = 1, 8, 2, 129, 128
    q, k = bf16_to_torch(gen((B, h_q, S, d), 10, 1)), bf16_to_torch(gen((B, h_kv, S, d), 10, 2))
    ones = torch.ones((B, h_kv, S, d), dtype=torch.bfloat16, device="cuda")
    o = gha_lib.gqa_prefill(q, k, ones, out_dtype=torch.float32)
    assert (o - 1).abs().max().item() <= 1e-2
    v = bf16_to_torch(gen((B, h_kv, S, d), 10, 3))
    o1 = gha_lib.gqa_prefill(q, k, v, out_dtype=torch.float32)
    o2 = gha_lib.gqa_prefill(q, k, v, out_dtype=torch.float32)
    assert torch.equal(o1, o2)
    for i in range(h_q):
        assert torch.allclose(o1[0, i, 0], v[0, i // 4, 0].float(), atol=0, rtol=0)


def test_gqa_prefill_full_size(gha_lib):
    """Batch 4, 32 query heads over 8 KV heads, 4096 tokens, head dim 128, in
    the launch configuration the benchmark times; the oracle evaluates every
    row of every (batch, head) slice."""
    B, h_q, h_kv, S, d = 4, 32, 8, 4096, 128
    say(f"full-size prefill {B}x{h_q}/{h_kv}x{S}x{d}")
    qb, kb, vb = gen((B, h_q, S, d), 2, 1), gen((B, h_kv, S, d), 2, 2), gen((B, h_kv, S, d), 2, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    o = twice("full prefill", lambda: gha_lib.gqa_prefill(q, k, v, out_dtype=torch.float32))
    o16 = twice("full prefill bf16", lambda: gha_lib.gqa_prefill(q, k, v))
    all_finite("full prefill", o)
    all_finite("full prefill bf16", o16)
    o = o.cpu().numpy()
    o16 = o16.float().cpu().numpy()
    wq, wk, wv = widen(qb), widen(kb), widen(vb)
    for b in range(B):
        ref, _ = oracle.gqa_prefill(wq[b:b + 1], wk[b:b + 1], wv[b:b + 1])
        check(f"full prefill b={b}", o[b:b + 1], ref)
        check(f"full prefill bf16 b={b}", o16[b:b + 1], ref, bf16_out=True)


# ------------------------------------------------------------------- decode

def decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, seed):
    qb = gen((B, h_q, s_q, d), seed, 1)
    kb = cache_bits(B, h_kv, L_cap, d, seqlens, seed, 2)
    vb = cache_bits(B, h_kv, L_cap, d, seqlens, seed, 3)
    return qb, kb, vb


DECODE_CASES = [
    # B, h_q, h_kv, s_q, L_cap, seqlens, d
    (3, 32, 8, 1, 1100, [1, 700, 1100], 128),
    (3, 32, 8, 2, 1100, [2, 333, 1099], 128),
    (2, 8, 1, 2, 600, [64, 599], 128),      # MQA: 16 rows in one block
    (2, 16, 1, 1, 300, [5, 300], 128),      # 16 heads per group
    (2, 32, 1, 1, 300, [257, 299], 128),    # 32 rows: two row blocks
    (2, 4, 4, 1, 260, [256, 260], 128),     # MHA
    (2, 8, 2, 2, 500, [3, 480], 64),        # head dim 64
    (2, 32, 1, 2, 300, [4, 299], 128),      # 64 rows per group: the 16-row-block kernel
    (1, 4, 1, 8, 200, [150], 64),           # 32 rows, head dim 64
]


@pytest.mark.parametrize("B,h_q,h_kv,s_q,L_cap,seqlens,d", DECODE_CASES)
def test_gqa_decode(gha_lib, B, h_q, h_kv, s_q, L_cap, seqlens, d):
    say(f"decode B={B} h={h_q}/{h_kv} s_q={s_q} L_cap={L_cap} L={seqlens} d={d}")
    seqlens = np.array(seqlens, dtype=np.int32)
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 12)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    sl = torch.from_numpy(seqlens).cuda()
    o32, lse = twice("decode", lambda: gha_lib.gqa_decode(q, k, v, sl, out_dtype=torch.float32, return_lse=True))
    o16 = twice("decode bf16", lambda: gha_lib.gqa_decode(q, k, v, sl))
    ref, ref_lse = oracle.gqa_decode(widen(qb), widen(kb), widen(vb), seqlens)
    check("decode fp32", o32.cpu().numpy(), ref)
    check("decode bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("decode lse", lse.cpu().numpy(), ref_lse)


def test_gqa_decode_single_key_returns_value(gha_lib):
    say("decode L=1")
    B, h_q, h_kv, d = 2, 8, 2, 128
    qb, kb, vb = decode_case(B, h_q, h_kv, 1, 64, [1, 1], d, 13)
    o = gha_lib.gqa_decode(*(bf16_to_torch(x) for x in (qb, kb, vb)),
                           torch.ones(B, dtype=torch.int32, device="cuda"), out_dtype=torch.float32)
    ref = np.repeat(widen(vb)[:, :, :1], 4, axis=1)
    assert np.abs(o.cpu().numpy() - ref).max() <= 1e-6


@pytest.mark.parametrize("h_q,h_kv,s_q", [(32, 1, 2), (32, 8, 1)])
def test_gqa_decode_empty_sequence_gives_zeros(gha_lib, h_q, h_kv, s_q):
    """A sequence of length 0 breaks the documented precondition s_q <= L_b;
    both decode kernels (64 rows per KV head: the register-operand kernel;
    4 rows: the streaming kernel) still return zeros and lse = -inf for it
    and leave the other sequences exact."""
    B, L_cap, d = 2, 300, 128
    say(f"decode with an empty sequence h={h_q}/{h_kv} s_q={s_q}")
    seqlens = np.array([0, 299], dtype=np.int32)
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 31)
    o, lse = twice("empty sequence", lambda: gha_lib.gqa_decode(*(bf16_to_torch(x) for x in (qb, kb, vb)),
                                                                torch.from_numpy(seqlens).cuda(),
                                                                out_dtype=torch.float32, return_lse=True))
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf)
    ref, ref_lse = oracle.gqa_decode(widen(qb[1:]), widen(kb[1:]), widen(vb[1:]), seqlens[1:])
    check("non-empty sequence", o[1:], ref)
    check("non-empty sequence lse", lse[1:], ref_lse)


@pytest.mark.parametrize("s_q", [1, 2])
def test_gqa_decode_full_size(gha_lib, s_q):
    """Batch 64, 32/8 heads, head dim 128, lengths uniform in [1024, 32768],
    cache capacity 32768 with NaN beyond each length; every sequence is
    checked against the oracle (output and lse)."""
    B, h_q, h_kv, d, L_cap = 64, 32, 8, 128, 32768
    say(f"full-size decode s_q={s_q}")
    seqlens = synth.uniform_i32(B, 1024, 32768, 3, synth.STREAM["seqlens"])
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    sl = torch.from_numpy(seqlens).cuda()
    ws = torch.empty(gha_lib.gqa_decode_workspace_bytes(B, h_q, h_kv, s_q, L_cap, d), dtype=torch.uint8,
                     device="cuda")
    o, lse = twice("full decode", lambda: gha_lib.gqa_decode(q, k, v, sl, out_dtype=torch.float32, workspace=ws,
                                                             return_lse=True))
    all_finite("full decode", o)
    del q, k, v
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    wq = widen(qb)
    for b in range(B):
        L = int(seqlens[b])
        ref, ref_lse = oracle.gqa_decode(wq[b:b + 1], widen(kb[b:b + 1, :, :L]), widen(vb[b:b + 1, :, :L]),
                                         np.array([L]))
        check(f"full decode b={b} L={L}", o[b:b + 1], ref)
        check(f"full decode lse b={b}", lse[b:b + 1], ref_lse)


# The streaming decode kernel addresses one (sequence, KV head) cache slice
# through a buffer with 32-bit offsets: it takes a slice while L_cap + 64
# token rows span less than 2 GiB; gqa_decode gives longer ones to the
# register-fed kernel (64-bit addresses).
LONGEST_STREAMED = (1 << 31) // (2 * 128) - 64 - 1  # 8388543 tokens at d = 128


@pytest.mark.parametrize("L", [LONGEST_STREAMED, LONGEST_STREAMED + 1])
def test_gqa_decode_longest_sequences(gha_lib, L):
    """One sequence of L = L_cap tokens: the last length the streaming
    kernel's offsets cover, and the first past them.  The new tokens' visible
    keys run to the last row of a 2 GiB cache slice; output and lse against
    the oracle."""
    B, h_q, h_kv, s_q, d = 1, 4, 1, 2, 128
    say(f"longest decode L={L}")
    seqlens = np.array([L], dtype=np.int32)
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L, seqlens, d, 43)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    sl = torch.from_numpy(seqlens).cuda()
    o, lse = gha_lib.gqa_decode(q, k, v, sl, out_dtype=torch.float32, return_lse=True)
    all_finite("longest decode", o)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    del q, k, v
    torch.cuda.empty_cache()
    ref, ref_lse = oracle.gqa_decode(widen(qb), widen(kb), widen(vb), seqlens)
    check(f"longest decode L={L}", o, ref)
    check(f"longest decode lse L={L}", lse, ref_lse)


# ------------------------------------------------ paged and windowed decode

PAGED_CASES = [
    # B, h_q, h_kv, s_q, L_cap, seqlens, d, page_size (0: contiguous), window, tokens-major pool
    (3, 32, 8, 1, 1100, [1, 700, 1100], 128, 64, 0, False),
    (3, 32, 8, 2, 1100, [2, 333, 1099], 128, 32, 0, True),
    (2, 8, 2, 2, 600, [64, 599], 64, 128, 0, False),
    (3, 32, 8, 1, 1100, [1, 700, 1100], 128, 0, 100, False),
    (3, 32, 8, 2, 1100, [2, 333, 1099], 128, 64, 257, False),
    (2, 4, 1, 8, 800, [8, 790], 64, 256, 1, True),       # window 1: each row sees its own key
    (2, 16, 2, 4, 2000, [1500, 2000], 128, 32, 1000, False),  # 32 rows per group
    (2, 32, 8, 1, 500, [100, 500], 128, 0, 5000, False),  # window longer than every sequence
    (2, 8, 8, 3, 700, [3, 650], 64, 96, 130, True),       # MHA, page of 96 tokens
]


@pytest.mark.parametrize("B,h_q,h_kv,s_q,L_cap,seqlens,d,page,window,tmajor", PAGED_CASES)
def test_gqa_decode_paged(gha_lib, B, h_q, h_kv, s_q, L_cap, seqlens, d, page, window, tmajor):
    say(f"paged decode B={B} h={h_q}/{h_kv} s_q={s_q} L_cap={L_cap} L={seqlens} d={d} "
        f"page={page} window={window} tokens_major={tmajor}")
    seqlens = np.array(seqlens, dtype=np.int32)
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 21)
    q = bf16_to_torch(qb)
    sl = torch.from_numpy(seqlens).cuda()
    if page:
        kp, table = page_pool(kb, seqlens, page, 5, window=window, s_q=s_q, tokens_major=tmajor)
        vp, table_v = page_pool(vb, seqlens, page, 5, window=window, s_q=s_q, tokens_major=tmajor)
        assert np.array_equal(table, table_v)
        k, v = bf16_to_torch(kp), bf16_to_torch(vp)
        if tmajor:
            k, v = k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)
        bt = torch.from_numpy(table).cuda()
        kw = dict(block_table=bt, page_size=page, L_cap=L_cap)
    else:
        k, v = bf16_to_torch(kb), bf16_to_torch(vb)
        kw = {}
    o32, lse = twice("paged", lambda: gha_lib.gqa_decode_paged(q, k, v, sl, window=window, out_dtype=torch.float32,
                                                               return_lse=True, **kw))
    o16 = twice("paged bf16", lambda: gha_lib.gqa_decode_paged(q, k, v, sl, window=window, **kw))
    ref, ref_lse = oracle.gqa_decode(widen(qb), widen(kb), widen(vb), seqlens, window=window)
    check("paged decode fp32", o32.cpu().numpy(), ref)
    check("paged decode bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("paged decode lse", lse.cpu().numpy(), ref_lse)


@pytest.mark.parametrize("page,window", [(128, 0), (256, 4096)])
def test_gqa_decode_paged_full_size_sampled(gha_lib, page, window):
    """The decode workload (batch 64, 32/8 heads, head dim 128, lengths uniform
    in [1024, 32768]) with its cache scattered over a shuffled page pool."""
    B, h_q, h_kv, d, L_cap, s_q = 64, 32, 8, 128, 32768, 1
    say(f"full-size paged decode page={page} window={window}")
    seqlens = synth.uniform_i32(B, 1024, 32768, 3, synth.STREAM["seqlens"])
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 3)
    q = bf16_to_torch(qb)
    n_pps = L_cap // page
    perm = torch.from_numpy(np.random.default_rng(9).permutation(B * n_pps)).cuda()
    table = torch.empty(B * n_pps, dtype=torch.int32, device="cuda")
    table[perm] = torch.arange(B * n_pps, dtype=torch.int32, device="cuda")
    pools = []
    for x in (kb, vb):
        # page i of sequence b (pool row b * n_pps + i) goes to pool row table[b, i]
        src = bf16_to_torch(x).view(B, h_kv, n_pps, page, d).permute(0, 2, 1, 3, 4).reshape(B * n_pps, h_kv, page, d)
        pool = torch.empty_like(src)
        pool[table.long()] = src
        pools.append(pool)
        del src
    sl = torch.from_numpy(seqlens).cuda()
    o = twice("full paged", lambda: gha_lib.gqa_decode_paged(q, pools[0], pools[1], sl,
                                                             block_table=table.view(B, n_pps), page_size=page,
                                                             window=window, out_dtype=torch.float32))
    all_finite("full paged decode", o)
    del pools
    o = o.cpu().numpy()
    wq = widen(qb)
    for b in range(B):
        L = int(seqlens[b])
        lo = max(0, L - s_q + 1 - window) if window else 0   # keys no row can see are not widened
        ref, _ = oracle.gqa_decode(wq[b:b + 1], widen(kb[b:b + 1, :, lo:L]), widen(vb[b:b + 1, :, lo:L]),
                                   np.array([L - lo]), window=window)
        check(f"full paged decode b={b} L={L}", o[b:b + 1], ref)


# ------------------------------------------------------- 8-bit caches

FP8_CASES = [
    # B, h_q, h_kv, s_q, L_cap, seqlens, d, page_size (0: contiguous), window
    (3, 32, 8, 1, 1100, [1, 700, 1100], 128, 0, 0),
    (3, 32, 8, 2, 1100, [2, 333, 1099], 128, 64, 0),
    (2, 8, 2, 2, 600, [64, 599], 64, 0, 0),
    (2, 16, 2, 4, 2000, [1500, 2000], 128, 32, 1000),   # 32 rows per group, paged, windowed
    (2, 8, 8, 3, 700, [3, 650], 64, 96, 130),
]


@pytest.mark.parametrize("B,h_q,h_kv,s_q,L_cap,seqlens,d,page,window", FP8_CASES)
def test_gqa_decode_fp8(gha_lib, B, h_q, h_kv, s_q, L_cap, seqlens, d, page, window):
    say(f"fp8 decode B={B} h={h_q}/{h_kv} s_q={s_q} L={seqlens} d={d} page={page} window={window}")
    seqlens = np.array(seqlens, dtype=np.int32)
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 25)
    ks, vs = 1 / 64, 1 / 48
    kc, vc = e4m3_codes(kb, ks), e4m3_codes(vb, vs)
    q = bf16_to_torch(qb)
    sl = torch.from_numpy(seqlens).cuda()
    if page:
        kp, table = page_pool(kc, seqlens, page, 7, window=window, s_q=s_q)
        vp, _ = page_pool(vc, seqlens, page, 7, window=window, s_q=s_q)
        k, v = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
        kw = dict(block_table=torch.from_numpy(table).cuda(), page_size=page, L_cap=L_cap)
    else:
        k, v = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
        kw = {}
    o32, lse = twice("fp8", lambda: gha_lib.gqa_decode_fp8(q, k, v, sl, k_scale=ks, v_scale=vs, window=window,
                                                           out_dtype=torch.float32, return_lse=True, **kw))
    o16 = twice("fp8 bf16", lambda: gha_lib.gqa_decode_fp8(q, k, v, sl, k_scale=ks, v_scale=vs, window=window,
                                                           **kw))
    ref, ref_lse = oracle.gqa_decode_fp8(widen(qb), kc, vc, ks, vs, seqlens, window=window)
    check("fp8 decode fp32", o32.cpu().numpy(), ref)
    check("fp8 decode bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("fp8 decode lse", lse.cpu().numpy(), ref_lse)


@pytest.mark.parametrize("d,page", [(128, 0), (64, 0), (128, 64)])
def test_gqa_decode_fp8_many_chunks_per_work_group(gha_lib, d, page):
    """Batch 8, 32/8 heads, lengths up to 8192: 8 x 8 x 64 = 4096 chunks of
    128 keys over the 8-bit plan's 512 work-groups, so every work-group's
    share spans several chunks and the merge combines partials across team
    boundaries; every sequence and the lse are checked."""
    B, h_q, h_kv, s_q, L_cap = 8, 32, 8, 1, 8192
    say(f"fp8 decode, many chunks per work-group, d={d} page={page}")
    seqlens = np.array([8192, 1, 4097, 8000, 333, 7777, 129, 6000], dtype=np.int32)
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 27)
    ks, vs = 1 / 32, 1 / 40
    kc, vc = e4m3_codes(kb, ks), e4m3_codes(vb, vs)
    sl = torch.from_numpy(seqlens).cuda()
    if page:
        kp, table = page_pool(kc, seqlens, page, 11)
        vp, _ = page_pool(vc, seqlens, page, 11)
        k, v = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
        kw = dict(block_table=torch.from_numpy(table).cuda(), page_size=page, L_cap=L_cap)
    else:
        k, v = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
        kw = {}
    o, lse = twice("fp8 many chunks", lambda: gha_lib.gqa_decode_fp8(
        bf16_to_torch(qb), k, v, sl, k_scale=ks, v_scale=vs, out_dtype=torch.float32, return_lse=True, **kw))
    ref, ref_lse = oracle.gqa_decode_fp8(widen(qb), kc, vc, ks, vs, seqlens)
    check("fp8 many chunks", o.cpu().numpy(), ref)
    check("fp8 many chunks lse", lse.cpu().numpy(), ref_lse)


def test_gqa_decode_fp8_full_size(gha_lib):
    """The decode workload (batch 64, 32/8 heads, head dim 128, lengths uniform
    in [1024, 32768]) with its cache quantized to E4M3; every sequence is
    checked."""
    B, h_q, h_kv, d, L_cap, s_q = 64, 32, 8, 128, 32768, 1
    say("full-size fp8 decode")
    seqlens = synth.uniform_i32(B, 1024, 32768, 3, synth.STREAM["seqlens"])
    qb, kb, vb = decode_case(B, h_q, h_kv, s_q, L_cap, seqlens, d, 3)
    ks, vs = 1 / 64, 1 / 64
    kc = torch.from_numpy(kb).view(torch.bfloat16).cuda()
    vc = torch.from_numpy(vb).view(torch.bfloat16).cuda()
    del kb, vb
    # quantize on the device (input preparation; the same rounding as the host helper)
    k8 = (kc.float() / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (vc.float() / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    del kc, vc
    q, sl = bf16_to_torch(qb), torch.from_numpy(seqlens).cuda()
    o = twice("full fp8", lambda: gha_lib.gqa_decode_fp8(q, k8, v8, sl, k_scale=ks, v_scale=vs,
                                                         out_dtype=torch.float32))
    all_finite("full fp8 decode", o)
    o = o.cpu().numpy()
    for b in range(B):
        L = int(seqlens[b])
        kk, vv = k8[b, :, :L].cpu().numpy(), v8[b, :, :L].cpu().numpy()
        ref, _ = oracle.gqa_decode_fp8(widen(qb[b:b + 1]), kk[None], vv[None], ks, vs, np.array([L]))
        check(f"full fp8 decode b={b} L={L}", o[b:b + 1], ref)


# ----------------------------------------------- GQLA GQA-path prefill

GQLA_PREFILL_CASES = [
    # B, h_q, g, S_q, S_k, causal, kv_std
    (2, 16, 2, 200, 200, True, 0.45),     # ragged last tile
    (1, 8, 8, 77, 77, True, 0.45),        # one head per group
    (1, 16, 4, 100, 300, True, 0.45),     # bottom-right: queries are the last 100 positions
    (1, 8, 2, 130, 130, False, 0.45),
    (1, 32, 8, 1, 40, True, 0.45),        # a single query row
    (1, 64, 4, 1090, 1090, True, 0.45),   # 560 work-groups: paired q-blocks, 35 of them
    (2, 16, 2, 300, 300, True, 1.0),      # N(0, 1) keys and values: larger scores
    (1, 64, 4, 1090, 1200, True, 1.0),    # N(0, 1), paired q-blocks, bottom-right
]


def gqla_prefill_case(B, h_q, g, S_q, S_k, seed, kv_std=0.45):
    return (synth.normal_bf16((B, h_q, S_q, 128), seed, 1), synth.normal_bf16((B, h_q, S_q, 64), seed, 2),
            synth.normal_bf16((B, g, S_k, 128), seed, 3, kv_std), synth.normal_bf16((B, S_k, 64), seed, 4),
            synth.normal_bf16((B, g, S_k, 128), seed, 5, kv_std))


@pytest.mark.parametrize("B,h_q,g,S_q,S_k,causal,kv_std", GQLA_PREFILL_CASES)
def test_gqla_gqa_prefill(gha_lib, B, h_q, g, S_q, S_k, causal, kv_std):
    say(f"gqla prefill B={B} h_q={h_q} g={g} S_q={S_q} S_k={S_k} causal={causal} kv_std={kv_std}")
    bits = gqla_prefill_case(B, h_q, g, S_q, S_k, 23, kv_std)
    qc, qr, kc, kr, v = (bf16_to_torch(x) for x in bits)
    scale = 1.0 / math.sqrt(192)
    o32, lse = twice("gqla prefill", lambda: gha_lib.gqla_gqa_prefill(qc, qr, kc, kr, v, scale=scale, causal=causal,
                                                                      out_dtype=torch.float32, return_lse=True))
    o16 = twice("gqla prefill bf16", lambda: gha_lib.gqla_gqa_prefill(qc, qr, kc, kr, v, scale=scale,
                                                                      causal=causal))
    ref, ref_lse = oracle.gqla_gqa_prefill(*(widen(x) for x in bits), scale=scale, causal=causal)
    check("gqla prefill fp32", o32.cpu().numpy(), ref)
    check("gqla prefill bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("gqla prefill lse", lse.cpu().numpy(), ref_lse)


def test_gqla_gqa_prefill_full_size_sampled(gha_lib):
    """Batch 2, 128 query heads in 8 groups, 4096 tokens, d_h 128 + d^R 64.
    The whole output must be finite; the oracle evaluates every row of 16
    (batch, head) slices, two in each group (the full output would take the
    oracle about a minute)."""
    B, h_q, g, S = 2, 128, 8, 4096
    say(f"full-size gqla prefill {B}x{h_q}/{g}x{S}")
    bits = gqla_prefill_case(B, h_q, g, S, S, 10)
    scale = 1.0 / math.sqrt(192)
    dev = [bf16_to_torch(x) for x in bits]
    o = twice("full gqla prefill", lambda: gha_lib.gqla_gqa_prefill(*dev, scale=scale, out_dtype=torch.float32))
    all_finite("full gqla prefill", o)
    o = o.cpu().numpy()
    pairs = [(j % 2, 16 * j + (5 * j + 3) % 16) for j in range(8)] + [((j + 1) % 2, 16 * j + 15 - j) for j in range(8)]
    ref, _ = oracle.gqla_gqa_prefill(*(widen(x) for x in bits), scale=scale, heads=pairs)
    for b, i in pairs:
        check(f"full gqla prefill (b={b}, head={i})", o[b, i], ref[b, i])


# -------------------------------------------------------------- GTA decode

GTA_DECODE_CASES = [
    # B, h, n_grp, s_q, L_cap, seqlens, d_qk, d_v
    (3, 16, 4, 1, 1100, [1, 700, 1100], 64, 64),
    (3, 16, 4, 2, 1100, [2, 333, 1099], 64, 64),
    (2, 8, 4, 1, 600, [64, 599], 64, 64),        # two heads per group
    (2, 4, 4, 2, 300, [5, 300], 64, 64),         # one head per group
    (2, 8, 2, 1, 500, [3, 480], 128, 64),        # d_qk 128: two waves per work-group
    (1, 16, 4, 16, 400, [390], 64, 64),          # 16 new tokens
    (1, 4, 4, 20, 400, [390], 64, 64),           # 20 rows: two row tiles
    (2, 12, 4, 1, 300, [100, 300], 64, 64),      # three heads per group: one value source a launch
    # wider values: sources of 128 columns, several launches per group
    (2, 8, 4, 1, 600, [64, 599], 64, 128),       # 2 sources, one launch
    (2, 16, 4, 2, 500, [3, 480], 64, 128),       # 4 sources (512 columns), one launch
    (2, 16, 4, 1, 400, [1, 399], 128, 256),      # 8 sources, two launches
    (1, 8, 4, 20, 300, [290], 64, 128),          # 20 rows: at most 256 columns a launch
    (1, 4, 1, 17, 300, [250], 64, 256),          # 8 sources of 17 rows: four launches
]


@pytest.mark.parametrize("B,h,n_grp,s_q,L_cap,seqlens,d_qk,d_v", GTA_DECODE_CASES)
def test_gta_shared_score_decode(gha_lib, B, h, n_grp, s_q, L_cap, seqlens, d_qk, d_v):
    say(f"GTA decode B={B} h={h} groups={n_grp} s_q={s_q} L_cap={L_cap} L={seqlens} d_qk={d_qk} d_v={d_v}")
    seqlens = np.array(seqlens, dtype=np.int32)
    qb = gen((B, n_grp, s_q, d_qk), 22, 1)
    kb = cache_bits(B, n_grp, L_cap, d_qk, seqlens, 22, 2)
    vb = cache_bits(B, h, L_cap, d_v, seqlens, 22, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    sl = torch.from_numpy(seqlens).cuda()
    o32, lse = twice("gta decode", lambda: gha_lib.gta_shared_score_decode(q, k, v, sl, out_dtype=torch.float32,
                                                                           return_lse=True))
    o16 = twice("gta decode bf16", lambda: gha_lib.gta_shared_score_decode(q, k, v, sl))
    ref, ref_lse = oracle.gta_decode(widen(qb), widen(kb), widen(vb), seqlens)
    check("gta decode fp32", o32.cpu().numpy(), ref)
    check("gta decode bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("gta decode lse", lse.cpu().numpy(), ref_lse)


def test_gta_decode_single_key_returns_value(gha_lib):
    say("GTA decode L=1")
    B, h, n_grp = 2, 16, 4
    qb = gen((B, n_grp, 1, 64), 23, 1)
    kb = cache_bits(B, n_grp, 64, 64, np.array([1, 1]), 23, 2)
    vb = cache_bits(B, h, 64, 64, np.array([1, 1]), 23, 3)
    o = gha_lib.gta_shared_score_decode(*(bf16_to_torch(x) for x in (qb, kb, vb)),
                                        torch.ones(B, dtype=torch.int32, device="cuda"), out_dtype=torch.float32)
    assert np.abs(o.cpu().numpy() - widen(vb)[:, :, :1]).max() <= 1e-6


@pytest.mark.parametrize("s_q", [1, 2])
def test_gta_decode_full_size(gha_lib, s_q):
    """Batch 64, 16 heads in 4 groups, dims 64, lengths uniform in
    [1024, 32768], capacity 32768 with NaN beyond each length; every sequence
    is checked."""
    B, h, n_grp, d, L_cap = 64, 16, 4, 64, 32768
    say(f"full-size GTA decode s_q={s_q}")
    seqlens = synth.uniform_i32(B, 1024, 32768, 6, synth.STREAM["seqlens"])
    qb = gen((B, n_grp, s_q, d), 6, 1)
    kb = cache_bits(B, n_grp, L_cap, d, seqlens, 6, 2)
    vb = cache_bits(B, h, L_cap, d, seqlens, 6, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    sl = torch.from_numpy(seqlens).cuda()
    o = twice("full gta decode", lambda: gha_lib.gta_shared_score_decode(q, k, v, sl, out_dtype=torch.float32))
    all_finite("full GTA decode", o)
    del q, k, v
    o = o.cpu().numpy()
    for b in range(B):
        L = int(seqlens[b])
        ref, _ = oracle.gta_decode(widen(qb[b:b + 1]), widen(kb[b:b + 1, :, :L]), widen(vb[b:b + 1, :, :L]),
                                   np.array([L]))
        check(f"full GTA decode b={b} L={L}", o[b:b + 1], ref)


# ------------------------------------------------------ GQLA GQA-path decode

GQLA_CASES = [
    # B, h_q, g, s_q, L_cap, seqlens
    (2, 128, 8, 1, 700, [1, 700]),
    (2, 128, 8, 2, 600, [2, 555]),
    (2, 32, 2, 1, 300, [17, 300]),
    (1, 16, 1, 2, 400, [399]),
]


def gqla_case(B, h_q, g, s_q, L_cap, seqlens, seed, kv_std=1.0):
    qc = gen((B, h_q, s_q, 128), seed, synth.STREAM["q_c"])
    qr = gen((B, h_q, s_q, 64), seed, synth.STREAM["q_rope"])
    kc = synth.cache_bf16(B, g, L_cap, 128, seqlens, seed, synth.STREAM["k"], kv_std)
    kr = synth.cache_bf16(B, 1, L_cap, 64, seqlens, seed, synth.STREAM["k_rope"])[:, 0]
    v = synth.cache_bf16(B, g, L_cap, 128, seqlens, seed, synth.STREAM["v"], kv_std)
    return qc, qr, kc, kr, v


@pytest.mark.parametrize("B,h_q,g,s_q,L_cap,seqlens", GQLA_CASES)
def test_gqla_gqa_decode(gha_lib, B, h_q, g, s_q, L_cap, seqlens):
    say(f"GQLA GQA-path decode B={B} h_q={h_q} g={g} s_q={s_q} L_cap={L_cap} L={seqlens}")
    seqlens = np.array(seqlens, dtype=np.int32)
    qc, qr, kc, kr, v = gqla_case(B, h_q, g, s_q, L_cap, seqlens, 24)
    scale = 1 / math.sqrt(128 + 64)
    args = [bf16_to_torch(x) for x in (qc, qr, kc, kr, v)] + [torch.from_numpy(seqlens).cuda()]
    o32, lse = twice("gqla decode", lambda: gha_lib.gqla_gqa_decode(*args, scale=scale, out_dtype=torch.float32,
                                                                    return_lse=True))
    o16 = twice("gqla decode bf16", lambda: gha_lib.gqla_gqa_decode(*args, scale=scale))
    ref, ref_lse = oracle.gqla_gqa_decode(*(widen(x) for x in (qc, qr, kc, kr, v)), seqlens, scale=scale)
    check("gqla fp32", o32.cpu().numpy(), ref)
    check("gqla bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("gqla lse", lse.cpu().numpy(), ref_lse)


def test_gqla_gqa_path_matches_absorbed_path_on_gpu(gha_lib):
    """GQLA Figure 2 end to end: the GQA path over the per-group expanded
    cache (k^C = W^UK c, v = W^UV c, rounded to bf16) and the absorbed latent
    path (q~ = W^UK^T q^C rounded to bf16, then W^UV o_lat on the host) agree
    within the bf16-input tolerance."""
    B, h_q, g, d_h, s_q, L_cap = 2, 128, 8, 128, 2, 300
    seqlens = np.array([40, 300], dtype=np.int32)
    say("GQLA GQA path vs absorbed path")
    q_c, q_r, cache, w_uk, w_uv, q_lat = latent_inputs(B, s_q, h_q, L_cap, seqlens, 25, g=g)
    c = widen(cache)
    c = np.where(np.isnan(c), 0.0, c)
    K, V = oracle.expand_latent(c[..., :512], c[..., 512:], w_uk, w_uv, g)
    kc = synth.round_bf16(K[..., :d_h].astype(np.float32))
    vb = synth.round_bf16(V.astype(np.float32))
    kr = cache[..., 512:]
    scale = 1 / math.sqrt(d_h + 64)
    sl = torch.from_numpy(seqlens).cuda()
    o_gqa = gha_lib.gqla_gqa_decode(bf16_to_torch(np.ascontiguousarray(q_c.transpose(0, 2, 1, 3))),
                                    bf16_to_torch(np.ascontiguousarray(q_r.transpose(0, 2, 1, 3))),
                                    bf16_to_torch(kc), bf16_to_torch(np.ascontiguousarray(kr)),
                                    bf16_to_torch(vb), sl, scale=scale, out_dtype=torch.float32).cpu().numpy()
    dcache = bf16_to_torch(cache)
    o_lat = gha_lib.latent_absorb_decode(bf16_to_torch(q_lat), bf16_to_torch(q_r), dcache[..., :512],
                                         dcache[..., 512:], sl, scale=scale, out_dtype=torch.float32)
    O_abs = oracle.absorb_output(o_lat.cpu().numpy().astype(np.float64), w_uv, g, d_h)  # (B, s_q, h_q, d_h)
    check("GQA path vs absorbed path", o_gqa.transpose(0, 2, 1, 3), O_abs)


@pytest.mark.parametrize("s_q", [1, 2])
def test_gqla_decode_full_size(gha_lib, s_q):
    """h_q 128 in g = 8 groups, d_h 128, RoPE 64, batch 64, lengths uniform in
    [8192, 65536]: the per-group expanded cache of the latent workload (key
    and value spread 0.45, that of W^UK c with W ~ N(0, 0.02)); every
    sequence is checked."""
    B, h_q, g, L_cap = 64, 128, 8, 65536
    say(f"full-size GQLA decode s_q={s_q}")
    seqlens = synth.uniform_i32(B, 8192, 65536, 7, synth.STREAM["seqlens"])
    qc, qr, kc, kr, v = gqla_case(B, h_q, g, s_q, L_cap, seqlens, 7, kv_std=0.45)
    args = [bf16_to_torch(x) for x in (qc, qr, kc, kr, v)]
    scale = 1 / math.sqrt(128 + 64)
    sl = torch.from_numpy(seqlens).cuda()
    o = twice("full gqla decode", lambda: gha_lib.gqla_gqa_decode(*args, sl, scale=scale, out_dtype=torch.float32))
    all_finite("full GQLA decode", o)
    del args
    o = o.cpu().numpy()
    for b in range(B):
        L = int(seqlens[b])
        ref, _ = oracle.gqla_gqa_decode(widen(qc[b:b + 1]), widen(qr[b:b + 1]), widen(kc[b:b + 1, :, :L]),
                                        widen(kr[b:b + 1, :L]), widen(v[b:b + 1, :, :L]), np.array([L]),
                                        scale=scale)
        check(f"full GQLA decode b={b} L={L}", o[b:b + 1], ref)


# ---------------------------------------------------------------------- GTA

GTA_CASES = [
    # B, h, n_grp, S, d_qk, d_v
    (2, 16, 4, 300, 64, 64),
    (1, 8, 4, 129, 64, 64),
    (1, 4, 4, 70, 64, 64),
    (1, 8, 2, 100, 128, 64),
    (4, 16, 4, 520, 64, 64),  # 16 (batch, group) units of 5 q-blocks: 80 work-groups
    (1, 6, 2, 100, 64, 64),   # three heads per group: one 64-column source a launch
    # wider values: 64-column sources, up to four a launch
    (2, 8, 4, 300, 64, 128),  # 4 sources, one launch
    (1, 16, 4, 200, 64, 128), # 8 sources, two launches
    (1, 4, 4, 150, 64, 256),  # one head of 256: 4 sources
    (1, 8, 2, 130, 128, 256), # 16 sources, four launches, d_qk 128
    (1, 6, 2, 100, 64, 128),  # 6 sources, three launches of 2
    # d_qk 128 with fewer sources (two value waves per source, four per
    # source), ragged against the 64-key tiles
    (1, 4, 2, 150, 128, 64),  # two heads per group: two sources
    (2, 2, 2, 90, 128, 64),   # one head per group: one source
    # shorter than one key tile; one position (its output is v_0)
    (2, 8, 2, 40, 64, 64),
    (1, 8, 2, 1, 64, 64),
]


@pytest.mark.parametrize("B,h,n_grp,S,d_qk,d_v", GTA_CASES)
def test_gta_shared_score(gha_lib, B, h, n_grp, S, d_qk, d_v):
    say(f"GTA B={B} h={h} groups={n_grp} S={S} d_qk={d_qk} d_v={d_v}")
    qb, kb, vb = gen((B, n_grp, S, d_qk), 14, 1), gen((B, n_grp, S, d_qk), 14, 2), gen((B, h, S, d_v), 14, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    o, lse = twice("gta", lambda: gha_lib.gta_shared_score_prefill(q, k, v, out_dtype=torch.float32,
                                                                   return_lse=True))
    o16 = twice("gta bf16", lambda: gha_lib.gta_shared_score_prefill(q, k, v))
    ref, ref_lse = oracle.gta_prefill(widen(qb), widen(kb), widen(vb))
    check("gta fp32", o.cpu().numpy(), ref)
    check("gta bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("gta lse", lse.cpu().numpy(), ref_lse)


# GTA shapes that take the one-stream kernel: grids of more than one round of
# two work-groups per CU (above 512 work-groups on 256 CUs), or no mask
GTA_ONE_STREAM_CASES = [
    # B, h, n_grp, S, d_qk, d_v, causal
    (4, 32, 16, 1100, 64, 64, True),    # 576 work-groups, two heads per group
    (8, 16, 8, 1100, 64, 128, True),    # 576 work-groups, 128-wide values
    (2, 16, 4, 300, 64, 256, False),    # four 256-wide heads: four launches
    (1, 8, 2, 130, 128, 128, False),    # d_qk 128, two launches of four sources
]


@pytest.mark.parametrize("B,h,n_grp,S,d_qk,d_v,causal", GTA_ONE_STREAM_CASES)
def test_gta_one_stream_kernel(gha_lib, B, h, n_grp, S, d_qk, d_v, causal):
    say(f"GTA (one-stream kernel) B={B} h={h} groups={n_grp} S={S} d_qk={d_qk} d_v={d_v} causal={causal}")
    qb, kb, vb = gen((B, n_grp, S, d_qk), 17, 1), gen((B, n_grp, S, d_qk), 17, 2), gen((B, h, S, d_v), 17, 3)
    q, k, v = (bf16_to_torch(x) for x in (qb, kb, vb))
    o, lse = twice("gta one-stream", lambda: gha_lib.gta_shared_score_prefill(q, k, v, causal=causal,
                                                                              out_dtype=torch.float32,
                                                                              return_lse=True))
    o16 = twice("gta one-stream bf16", lambda: gha_lib.gta_shared_score_prefill(q, k, v, causal=causal))
    ref, ref_lse = oracle.gta_prefill(widen(qb), widen(kb), widen(vb), causal=causal)
    check("gta one-stream fp32", o.cpu().numpy(), ref)
    check("gta one-stream bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("gta one-stream lse", lse.cpu().numpy(), ref_lse)


def test_gta_not_causal(gha_lib):
    """Every position sees all S keys; S ragged against the 64-key tiles."""
    B, h, n_grp, S, d = 1, 8, 2, 200, 64
    say(f"GTA non-causal B={B} h={h} groups={n_grp} S={S}")
    qb, kb, vb = gen((B, n_grp, S, d), 15, 1), gen((B, n_grp, S, d), 15, 2), gen((B, h, S, d), 15, 3)
    o = gha_lib.gta_shared_score_prefill(*(bf16_to_torch(x) for x in (qb, kb, vb)), causal=False,
                                         out_dtype=torch.float32)
    ref, _ = oracle.gta_prefill(widen(qb), widen(kb), widen(vb), causal=False)
    check("gta non-causal", o.cpu().numpy(), ref)


def test_gta_growing_scores_restart(gha_lib):
    """Keys whose scores jump far above the first tile's maximum, twice, for a
    few positions held by lanes other than the first of their wave (the other
    positions see flat scores): the kernel's fixed per-row reference must be
    replaced and the work-group recomputed, and the result is still the
    softmax."""
    B, h, n_grp, S, d = 1, 8, 2, 300, 64
    say("GTA growing scores (reference restart)")
    one, k_mid, k_hi = (np.float32(x).view(np.uint32) >> 16 for x in (1.0, 16.0, 32.0))
    qb = np.zeros((B, n_grp, S, d), dtype=np.uint16)
    rows = [150, 170, 250, 299]
    qb[:, 0, rows] = one
    qb[:, 1] = gen((B, 1, S, d), 16, 1)[:, 0]
    kb = gen((B, n_grp, S, d), 16, 2)
    kb[:, 0, 100:200] = k_mid
    kb[:, 0, 200:] = k_hi
    vb = gen((B, h, S, d), 16, 3)
    o = gha_lib.gta_shared_score_prefill(*(bf16_to_torch(x) for x in (qb, kb, vb)), out_dtype=torch.float32)
    ref, _ = oracle.gta_prefill(widen(qb), widen(kb), widen(vb))
    check("gta restart", o.cpu().numpy(), ref)


def test_gta_full_size(gha_lib):
    """Batch 8, 16 heads in 4 groups of 4, 2048 tokens, dims 64; every
    (batch, head) slice and the per-group lse are checked."""
    B, h, n_grp, S, d = 8, 16, 4, 2048, 64
    say("full-size GTA")
    qb, kb, vb = gen((B, n_grp, S, d), 4, 1), gen((B, n_grp, S, d), 4, 2), gen((B, h, S, d), 4, 3)
    dev = [bf16_to_torch(x) for x in (qb, kb, vb)]
    o, lse = twice("full gta", lambda: gha_lib.gta_shared_score_prefill(*dev, out_dtype=torch.float32,
                                                                        return_lse=True))
    o16 = twice("full gta bf16", lambda: gha_lib.gta_shared_score_prefill(*dev))
    all_finite("full GTA", o)
    all_finite("full GTA bf16", o16)
    ref, ref_lse = oracle.gta_prefill(widen(qb), widen(kb), widen(vb))
    check("full GTA", o.cpu().numpy(), ref)
    check("full GTA bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("full GTA lse", lse.cpu().numpy(), ref_lse)


# ------------------------------------------------------------------- latent

def latent_inputs(B, s_q, h_q, L_cap, seqlens, seed, g=8, d_h=128):
    q_c = gen((B, s_q, h_q, d_h), seed, synth.STREAM["q_c"])
    q_r = gen((B, s_q, h_q, 64), seed, synth.STREAM["q_rope"])
    cache = latent_cache_bits(B, L_cap, 576, seqlens, seed, synth.STREAM["latent"])
    w_uk = widen(synth.normal_bf16((g * d_h, 512), seed, synth.STREAM["w_uk"], 0.02))
    w_uv = widen(synth.normal_bf16((g * d_h, 512), seed, synth.STREAM["w_uv"], 0.02))
    # absorbed query, made on the host in fp64 and rounded to bf16 (the input
    # the kernel and the oracle both receive)
    q_lat = synth.round_bf16(oracle.absorb_query(widen(q_c), w_uk, g).astype(np.float32))
    return q_c, q_r, cache, w_uk, w_uv, q_lat


LATENT_CASES = [
    # B, h_q, s_q, L_cap, seqlens
    (2, 128, 1, 700, [1, 700]),
    (2, 128, 2, 600, [2, 555]),
    (1, 16, 1, 300, [299]),
    (2, 96, 2, 400, [37, 400]),
]


@pytest.mark.parametrize("B,h_q,s_q,L_cap,seqlens", LATENT_CASES)
def test_latent_absorb_decode(gha_lib, B, h_q, s_q, L_cap, seqlens):
    say(f"latent B={B} h_q={h_q} s_q={s_q} L_cap={L_cap} L={seqlens}")
    seqlens = np.array(seqlens, dtype=np.int32)
    g = 8 if h_q % 8 == 0 else 1
    q_c, q_r, cache, w_uk, w_uv, q_lat = latent_inputs(B, s_q, h_q, L_cap, seqlens, 15, g=g)
    dcache = bf16_to_torch(cache)
    scale = 1 / math.sqrt(128 + 64)
    dq, dr, sl = bf16_to_torch(q_lat), bf16_to_torch(q_r), torch.from_numpy(seqlens).cuda()
    o32, lse = twice("latent", lambda: gha_lib.latent_absorb_decode(dq, dr, dcache[..., :512], dcache[..., 512:], sl,
                                                                    scale=scale, out_dtype=torch.float32,
                                                                    return_lse=True))
    o16 = twice("latent bf16", lambda: gha_lib.latent_absorb_decode(dq, dr, dcache[..., :512], dcache[..., 512:], sl,
                                                                    scale=scale))
    c = widen(cache)
    ref, ref_lse = oracle.latent_absorb_decode(widen(q_lat), widen(q_r), c[..., :512], c[..., 512:],
                                               seqlens, scale=scale)
    check("latent fp32", o32.cpu().numpy(), ref)
    check("latent bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("latent lse", lse.cpu().numpy(), ref_lse)


# The latent kernel reads a sequence's 1152-byte cache rows through a buffer
# with 32-bit offsets: L_cap + 32 rows must span less than 2 GiB.
LONGEST_LATENT = (1 << 31) // 1152 - 32  # 1864103 tokens


def test_latent_absorb_decode_longest_sequence(gha_lib):
    """One sequence of the longest cache the latent kernel takes, against the
    oracle; one token more is refused before anything is launched."""
    B, h_q, s_q, L = 1, 16, 1, LONGEST_LATENT
    say(f"longest latent L={L}")
    seqlens = np.array([L], dtype=np.int32)
    q_c, q_r, cache, w_uk, w_uv, q_lat = latent_inputs(B, s_q, h_q, L, seqlens, 47, g=1)
    dcache = bf16_to_torch(cache)
    scale = 1 / math.sqrt(128 + 64)
    dq, dr, sl = bf16_to_torch(q_lat), bf16_to_torch(q_r), torch.from_numpy(seqlens).cuda()
    o32, lse = gha_lib.latent_absorb_decode(dq, dr, dcache[..., :512], dcache[..., 512:], sl, scale=scale,
                                            out_dtype=torch.float32, return_lse=True)
    all_finite("longest latent", o32)
    o32, lse = o32.cpu().numpy(), lse.cpu().numpy()
    longer = torch.empty((B, L + 1, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gha_lib.GhaError) as e:
        gha_lib.latent_absorb_decode(dq, dr, longer[..., :512], longer[..., 512:], sl, scale=scale)
    assert e.value.status == gha_lib.STATUS.index("GHA_ERR_SHAPE")
    del dcache, longer
    torch.cuda.empty_cache()
    c = widen(cache)
    ref, ref_lse = oracle.latent_absorb_decode(widen(q_lat), widen(q_r), c[..., :512], c[..., 512:], seqlens,
                                               scale=scale)
    check("longest latent", o32, ref)
    check("longest latent lse", lse, ref_lse)


@pytest.mark.parametrize("heads", [None, (5, 77, 126)])
def test_latent_growing_scores_restart(gha_lib, heads):
    """Scores that jump far above the first tiles' maximum, twice (latent
    rows of three magnitudes): the kernel's fixed per-row reference must be
    replaced and the split recomputed, and the result is still the softmax.
    With `heads`, only those heads (none held by the first lane of a wave)
    see the jump; every other head has a zero query and flat scores."""
    say(f"latent growing scores (reference restart), heads={heads}")
    B, h_q, s_q, L = 1, 128, 1, 300
    rng_bits = gen((B, L, 576), 21, synth.STREAM["latent"])
    cache = rng_bits.copy()
    one = np.float32(1.0).view(np.uint32) >> 16
    two = np.float32(2.0).view(np.uint32) >> 16
    four = np.float32(4.0).view(np.uint32) >> 16
    cache[:, 100:200, :512] = two
    cache[:, 200:, :512] = four
    cache[:, 100:, 512:] = 0
    q_lat = np.full((B, s_q, h_q, 512), one, dtype=np.uint16)
    if heads is not None:
        q_lat[:] = 0
        q_lat[:, :, list(heads)] = one
    q_r = np.zeros((B, s_q, h_q, 64), dtype=np.uint16)
    seqlens = np.array([L], dtype=np.int32)
    scale = 1 / math.sqrt(128 + 64)
    dcache = bf16_to_torch(cache)
    o = gha_lib.latent_absorb_decode(bf16_to_torch(q_lat), bf16_to_torch(q_r), dcache[..., :512],
                                     dcache[..., 512:], torch.from_numpy(seqlens).cuda(), scale=scale,
                                     out_dtype=torch.float32)
    c = widen(cache)
    ref, _ = oracle.latent_absorb_decode(widen(q_lat), widen(q_r), c[..., :512], c[..., 512:],
                                         seqlens, scale=scale)
    check("latent restart", o.cpu().numpy(), ref)
    jumped = list(heads) if heads is not None else slice(None)
    assert np.allclose(ref[:, :, jumped], 4.0)



ABSORB_CASES = [
    # B, h_q, s_q, L_cap, seqlens, g
    (2, 128, 1, 700, [1, 700], 8),
    (2, 128, 2, 600, [2, 555], 8),
    (1, 16, 1, 300, [299], 2),
    (2, 32, 3, 400, [37, 400], 32),   # one head per group (MLA's per-head up-projections)
    (1, 40, 1, 90, [90], 5),          # rows not a multiple of 32
]


@pytest.mark.parametrize("B,h_q,s_q,L_cap,seqlens,g", ABSORB_CASES)
def test_gqla_absorb_decode(gha_lib, B, h_q, s_q, L_cap, seqlens, g):
    say(f"absorbing decode B={B} h_q={h_q} s_q={s_q} L={seqlens} g={g}")
    seqlens = np.array(seqlens, dtype=np.int32)
    q_c, q_r, cache, w_uk, w_uv, _ = latent_inputs(B, s_q, h_q, L_cap, seqlens, 33, g=g)
    w_bits = [synth.normal_bf16((g * 128, 512), 33, synth.STREAM[n], 0.02) for n in ("w_uk", "w_uv")]
    dcache = bf16_to_torch(cache)
    scale = 1 / math.sqrt(128 + 64)
    dev = [bf16_to_torch(x) for x in (q_c, q_r, w_bits[0], w_bits[1])]
    sl = torch.from_numpy(seqlens).cuda()
    o32, lse = twice("absorbing", lambda: gha_lib.gqla_absorb_decode(*dev, dcache[..., :512], dcache[..., 512:], sl,
                                                                     g=g, scale=scale, out_dtype=torch.float32,
                                                                     return_lse=True))
    o16 = twice("absorbing bf16", lambda: gha_lib.gqla_absorb_decode(*dev, dcache[..., :512], dcache[..., 512:], sl,
                                                                     g=g, scale=scale))
    c = widen(cache)
    # oracle: absorb in fp64 (no bf16 rounding of the absorbed query), attend,
    # apply W^UV
    q_abs = oracle.absorb_query(widen(q_c), w_uk, g)
    o_lat, ref_lse = oracle.latent_absorb_decode(q_abs, widen(q_r), c[..., :512], c[..., 512:], seqlens, scale=scale)
    ref = oracle.absorb_output(o_lat, w_uv, g, 128)
    check("absorbing decode fp32", o32.cpu().numpy(), ref)
    check("absorbing decode bf16", o16.float().cpu().numpy(), ref, bf16_out=True)
    check("absorbing decode lse", lse.cpu().numpy(), ref_lse)


@pytest.mark.parametrize("s_q", [1, 2])
def test_latent_full_size_and_expanded_path(gha_lib, s_q):
    """h_q 128, r_kv 512, RoPE 64, batch 64, lengths uniform in [8192, 65536],
    W^UK/W^UV per 8 groups ~ N(0, 0.02).  o_lat and its lse are checked
    against the absorbed oracle on every sequence; on three sequences W^UV
    o_lat (host, fp64) is also checked against the expanded per-group GQA
    oracle (GQLA: the two paths are equal), and so is the output of
    gqla_absorb_decode, which does both absorption products on the device."""
    B, h_q, L_cap, g, d_h = 64, 128, 65536, 8, 128
    say(f"full-size latent s_q={s_q}")
    seqlens = synth.uniform_i32(B, 8192, 65536, 5, synth.STREAM["seqlens"])
    q_c, q_r, cache, w_uk, w_uv, q_lat = latent_inputs(B, s_q, h_q, L_cap, seqlens, 5)
    dcache = bf16_to_torch(cache)
    scale = 1 / math.sqrt(d_h + 64)
    dq, dr, sl = bf16_to_torch(q_lat), bf16_to_torch(q_r), torch.from_numpy(seqlens).cuda()
    o, lse = twice("full latent", lambda: gha_lib.latent_absorb_decode(dq, dr, dcache[..., :512], dcache[..., 512:],
                                                                       sl, scale=scale, out_dtype=torch.float32,
                                                                       return_lse=True))
    all_finite("full latent", o)
    w_bits = [synth.normal_bf16((g * d_h, 512), 5, synth.STREAM[n], 0.02) for n in ("w_uk", "w_uv")]
    dev = [bf16_to_torch(x) for x in (q_c, q_r, w_bits[0], w_bits[1])]
    o_fused = twice("full absorbing", lambda: gha_lib.gqla_absorb_decode(*dev, dcache[..., :512], dcache[..., 512:],
                                                                         sl, g=g, scale=scale,
                                                                         out_dtype=torch.float32))
    all_finite("full absorbing", o_fused)
    del dcache
    o, lse, o_fused = o.cpu().numpy(), lse.cpu().numpy(), o_fused.cpu().numpy()
    wq, wr = widen(q_lat), widen(q_r)
    for b in range(B):
        L = int(seqlens[b])
        c = widen(cache[b:b + 1, :L])
        ref, ref_lse = oracle.latent_absorb_decode(wq[b:b + 1], wr[b:b + 1], c[..., :512], c[..., 512:],
                                                   np.array([L]), scale=scale)
        check(f"full latent b={b} L={L}", o[b:b + 1], ref)
        check(f"full latent lse b={b}", lse[b:b + 1], ref_lse)
    for b in [int(np.argmin(seqlens)), int(np.argmax(seqlens)), 30]:
        L = int(seqlens[b])
        c = widen(cache[b:b + 1, :L])
        # expanded per-group GQA path from the un-absorbed query
        K, V = oracle.expand_latent(c[..., :512], c[..., 512:], w_uk, w_uv, g)
        qf = np.concatenate([widen(q_c[b:b + 1]), widen(q_r[b:b + 1])], -1).transpose(0, 2, 1, 3)
        O_exp, _ = oracle.gqa_decode(qf, K, V, np.array([L]), scale=scale)
        O_gpu = oracle.absorb_output(o[b:b + 1], w_uv, g, d_h)
        check(f"expanded path b={b}", O_gpu, O_exp.transpose(0, 2, 1, 3))
        check(f"device absorption b={b}", o_fused[b:b + 1], O_exp.transpose(0, 2, 1, 3))
