"""The C ABI on the host: the library loads, exports every symbol include/la.h declares, and
rejects invalid arguments with the documented status before any HIP call (CPU only; every
call here fails validation, so nothing is ever enqueued)."""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

import causal_linear_attention_la_amd as la

ROOT = Path(__file__).resolve().parents[1]
A = 1 << 20  # fake, 16-byte aligned "device" addresses; never dereferenced


def declared_symbols():
    text = (ROOT / "include" / "la.h").read_text()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*\**\s*(la_\w+)\s*\(", text, re.M)))


def test_exports_match_header():
    decl = declared_symbols()
    assert set(decl) == set(la.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", str(la.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (la_\w+)$", out, re.M))
    for name in decl:
        assert name in exported, name
        assert hasattr(la.lib, name)


def test_one_hip_runtime():
    """The library binds to the HIP runtime PyTorch already loaded (one copy per process)."""
    rts = la.hip_runtimes()
    assert len(rts) == 1, rts


def test_version_and_strerror():
    assert la.version() >= (0, 1, 0)
    for code in (la.LA_OK, la.LA_EINVAL, la.LA_ENOTSUP, la.LA_EHIP):
        msg = la.strerror(code)
        assert msg and msg != "unknown status"
    assert la.strerror(12345) == "unknown status"


def call(fn, q=A, k=2 * A, v=3 * A, out=4 * A, S=5 * A, z=6 * A, B=1, H=2, N=8, d=16, dv=16,
         chunk=0, dtype=la.LA_BF16, seg=None, S0="same", z0="same", flags=0):
    f = getattr(la.lib, fn)
    if fn in ("la_causal_fwd_state", "la_causal_fwd_ex", "la_causal_fwd_profiled"):
        args = [q, k, v, out, S if S0 == "same" else S0, z if z0 == "same" else z0, S, z, B, H, N,
                d, dv, chunk, 0 if seg is None else seg]
        if fn != "la_causal_fwd_state":
            args.append(flags)
        args += [dtype, None]
        if fn == "la_causal_fwd_profiled":
            args += [1, (ctypes.c_float * 3)()]
        return f(*args)
    if fn == "la_decode_step_ex":
        return f(q, k, v, out, S, z, B, H, N, d, dv, flags, dtype, None)
    args = [q, k, v, out, S, z, B, H, N, d, dv, chunk]
    if fn == "la_causal_fwd_seg":
        args.append(0 if seg is None else seg)
    if fn == "la_global_fwd_ex":
        args.append(flags)
    args += [dtype, None]
    return f(*args)


FORMS = ["la_causal_fwd", "la_causal_fwd_seg", "la_causal_fwd_state", "la_causal_fwd_ex",
         "la_causal_fwd_profiled", "la_global_fwd", "la_global_fwd_ex", "la_decode_step",
         "la_decode_step_ex"]
FLAGGED = ["la_causal_fwd_ex", "la_causal_fwd_profiled", "la_global_fwd_ex", "la_decode_step_ex"]


@pytest.mark.parametrize("fn", FORMS)
def test_null_and_size_checks(fn):
    N = 1 if fn.startswith("la_decode_step") else 8
    assert call(fn, k=None, N=N) == la.LA_EINVAL
    assert call(fn, v=None, N=N) == la.LA_EINVAL
    assert call(fn, B=0, N=N) == la.LA_EINVAL
    assert call(fn, H=-1, N=N) == la.LA_EINVAL
    assert call(fn, N=0) == la.LA_EINVAL
    assert call(fn, d=0, N=N) == la.LA_EINVAL
    assert call(fn, dtype=7, N=N) == la.LA_EINVAL
    assert call(fn, k=2 * A + 8, N=N) == la.LA_EINVAL           # misaligned
    assert call(fn, out=A + 16, N=N) == la.LA_EINVAL            # out overlaps q
    assert call(fn, S=6 * A, z=6 * A, N=N) == la.LA_EINVAL      # S overlaps z
    assert call(fn, S=3 * A, N=N) == la.LA_EINVAL               # S overlaps v
    assert call(fn, d=48, N=N) == la.LA_ENOTSUP
    assert call(fn, dv=256, N=N) == la.LA_ENOTSUP


def test_form_specific_checks():
    assert call("la_decode_step", N=2) == la.LA_EINVAL
    assert call("la_decode_step", S=None) == la.LA_EINVAL
    assert call("la_decode_step", N=1, z=None) == la.LA_EINVAL
    assert call("la_causal_fwd", S=None) == la.LA_EINVAL        # one of S, z
    assert call("la_causal_fwd", q=None) == la.LA_EINVAL
    assert call("la_causal_fwd", out=None) == la.LA_EINVAL
    assert call("la_global_fwd", q=None) == la.LA_EINVAL        # q without out
    assert call("la_global_fwd", S=None) == la.LA_EINVAL
    assert call("la_global_fwd", z=None) == la.LA_EINVAL


@pytest.mark.parametrize("fn", FLAGGED)
def test_flag_checks(fn):
    N = 1 if fn.startswith("la_decode_step") else 8
    for bad in (4, 8, 1 << 30, -1):
        assert call(fn, N=N, flags=bad) == la.LA_EINVAL
    # valid flags still go through the other checks first
    for ok in (0, la.LA_PHI_IDENTITY, la.LA_UNNORMALIZED, la.LA_PHI_IDENTITY | la.LA_UNNORMALIZED):
        assert call(fn, N=N, flags=ok, k=None) == la.LA_EINVAL
        assert call(fn, N=N, flags=ok, d=48) == la.LA_ENOTSUP


def decay(fn, q=A, k=2 * A, v=3 * A, out=4 * A, S=5 * A, z=6 * A, gamma=7 * A, B=1, H=2, N=8,
          d=16, dv=16, flags=0, dtype=la.LA_BF16):
    f = getattr(la.lib, fn)
    if fn == "la_causal_fwd_decay":
        return f(q, k, v, out, S, z, S, z, gamma, B, H, N, d, dv, 0, 0, flags, dtype, None)
    return f(q, k, v, out, S, z, gamma, B, H, 1 if N == 8 else N, d, dv, flags, dtype, None)


@pytest.mark.parametrize("fn", ["la_causal_fwd_decay", "la_decode_step_decay"])
def test_decay_argument_checks(fn):
    assert decay(fn, gamma=None) == la.LA_EINVAL
    assert decay(fn, gamma=7 * A + 2) == la.LA_EINVAL           # not 4-byte aligned
    assert decay(fn, gamma=4 * A + 32) == la.LA_EINVAL          # inside out (64 bytes at N = 1)
    assert decay(fn, gamma=5 * A) == la.LA_EINVAL               # inside S
    assert decay(fn, gamma=6 * A + 4) == la.LA_EINVAL           # inside z
    assert decay(fn, flags=4) == la.LA_EINVAL
    assert decay(fn, k=None) == la.LA_EINVAL
    assert decay(fn, B=0) == la.LA_EINVAL
    assert decay(fn, d=48) == la.LA_ENOTSUP
    assert decay(fn, out=A + 16) == la.LA_EINVAL                # out overlaps q
    if fn == "la_decode_step_decay":
        assert decay(fn, N=2) == la.LA_EINVAL


def rf(x=A, W=2 * A, f=3 * A, rows=64, d=64, m=128, dtype=la.LA_BF16):
    return la.lib.la_rf_features(x, W, f, rows, d, m, dtype, None)


def test_rf_argument_checks():
    assert rf(x=None) == la.LA_EINVAL
    assert rf(W=None) == la.LA_EINVAL
    assert rf(f=None) == la.LA_EINVAL
    assert rf(x=A + 8) == la.LA_EINVAL                          # misaligned
    assert rf(rows=0) == la.LA_EINVAL
    assert rf(d=-1) == la.LA_EINVAL
    assert rf(m=0) == la.LA_EINVAL
    assert rf(dtype=5) == la.LA_EINVAL
    assert rf(f=A + 64) == la.LA_EINVAL                         # f overlaps x
    assert rf(f=2 * A - 16) == la.LA_EINVAL                     # f overlaps W
    assert rf(d=257) == la.LA_ENOTSUP
    assert rf(m=4097) == la.LA_ENOTSUP
    assert rf(rows=1 << 31, f=1 << 46) == la.LA_ENOTSUP


def crf(q=A, k=2 * A, v=3 * A, out=4 * A, W=7 * A, S=5 * A, z=6 * A, B=1, H=2, N=8, d=64, dv=64,
        m=64, chunk=0, seg=0, flags=0, dtype=la.LA_BF16):
    return la.lib.la_causal_fwd_rf(q, k, v, out, W, S, z, S, z, B, H, N, d, dv, m, chunk, seg, flags,
                                   dtype, None)


def test_causal_rf_argument_checks():
    assert crf(W=None) == la.LA_EINVAL
    assert crf(W=7 * A + 8) == la.LA_EINVAL                     # misaligned
    assert crf(W=4 * A + 16) == la.LA_EINVAL                    # W overlaps out
    assert crf(S=7 * A) == la.LA_EINVAL                         # state overlaps W
    assert crf(flags=la.LA_PHI_IDENTITY) == la.LA_EINVAL        # the map is the features
    assert crf(flags=4) == la.LA_EINVAL
    assert crf(q=None) == la.LA_EINVAL
    assert crf(m=0) == la.LA_EINVAL
    assert crf(B=0) == la.LA_EINVAL
    assert crf(S=None) == la.LA_EINVAL                          # one of S, z
    assert crf(out=A + 16) == la.LA_EINVAL                      # out overlaps q
    assert crf(d=257) == la.LA_ENOTSUP
    assert crf(m=48) == la.LA_ENOTSUP                           # the attention runs over m
    assert crf(dv=256) == la.LA_ENOTSUP
    # a chunk whose vector-ALU working set exceeds the LDS of a workgroup
    assert crf(chunk=128, dv=128, dtype=la.LA_F32) == la.LA_ENOTSUP


def test_profiled_argument_checks():
    f = la.lib.la_causal_fwd_profiled
    args = [A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 5 * A, 6 * A, 1, 2, 8, 16, 16, 0, 0, 0,
            la.LA_BF16, None]
    ms = (ctypes.c_float * 3)()
    assert f(*args, 1, None) == la.LA_EINVAL
    assert f(*args, 0, ms) == la.LA_EINVAL
    assert f(*args, 4097, ms) == la.LA_EINVAL


def test_separate_state_checks():
    fn = "la_causal_fwd_state"
    S, z = 5 * A, 6 * A
    assert call(fn, S0=S, z0=None) == la.LA_EINVAL              # half of a pair
    assert call(fn, S0=None, z0=z) == la.LA_EINVAL
    assert call(fn, S0=S + 16, z0=z) == la.LA_EINVAL            # partly overlaps S
    assert call(fn, S0=S, z0=7 * A) == la.LA_EINVAL             # in place for S, not for z
    assert call(fn, S0=A, z0=7 * A) == la.LA_EINVAL             # initial state overlaps q
    assert call(fn, S0=7 * A, z0=7 * A) == la.LA_EINVAL         # S0 overlaps z0
    assert call(fn, S0=7 * A + 8, z0=8 * A) == la.LA_EINVAL     # misaligned


def test_chunk_and_segment_checks():
    assert call("la_causal_fwd", chunk=-1) == la.LA_EINVAL
    assert call("la_causal_fwd", chunk=96) == la.LA_ENOTSUP
    # chunks 64 and 128 outside the matrix-core shapes go to the vector-ALU kernels when their
    # working set fits 160 KiB of LDS: not at d = d_v = 64 or 128 with chunk 128
    assert call("la_causal_fwd", chunk=128, d=128, dv=128) == la.LA_ENOTSUP
    assert call("la_causal_fwd", chunk=128, d=64, dv=64, dtype=la.LA_F32) == la.LA_ENOTSUP
    assert call("la_global_fwd", chunk=128, d=128, dv=64) == la.LA_ENOTSUP
    for d, dv, chunk, dtype in [(16, 16, 128, la.LA_F32), (32, 32, 128, la.LA_BF16),
                                (16, 64, 64, la.LA_F32), (64, 64, 64, la.LA_F32),
                                (64, 128, 64, la.LA_BF16)]:
        assert la.la_segments(0, 1, 2, 1000, d, dv, chunk, 0, dtype) > 0, (d, dv, chunk)
        assert la.la_segments(0, 1, 2, 1000, d, dv, chunk, 2 * chunk, dtype) == -(-1000 // (2 * chunk))
    assert call("la_global_fwd", chunk=48) == la.LA_ENOTSUP
    assert call("la_causal_fwd_seg", chunk=32, seg=48) == la.LA_ENOTSUP
    assert call("la_causal_fwd_seg", chunk=32, seg=-32) == la.LA_EINVAL


def test_workspace_bytes():
    # causal B=2 H=16 N=8192 d=128 bf16: chunk 64; the d = 128 matrix-core kernel takes one
    # workgroup per CU, so 256 / 32 = 8 segments of 1024 tokens per head
    E = 128 * 128 + 128
    assert la.la_segments(0, 2, 16, 8192, 128, 128) == 8
    assert la.la_workspace_bytes(0, 2, 16, 8192, 128, 128) == 32 * 8 * E * 4
    assert la.la_segments(0, 2, 16, 8192, 128, 128, 64, 512) == 16
    assert la.la_workspace_bytes(0, 2, 16, 8192, 128, 128, 64, 512) == 32 * 16 * E * 4
    assert la.la_segments(0, 2, 16, 8192, 128, 128, 64, 192) == 43
    # global B=1 H=8 N=100000 d=128: one segment per CU as well, 256 / 8 = 32 per head
    assert la.la_segments(1, 1, 8, 100000, 128, 128) == 32
    assert la.la_segments(0, 1, 1, 64, 48, 16) == 0
    # d = 64: two workgroups per CU would give 512 / 32 = 16 segments, but a segment keeps at
    # least 4 chunks: 8 segments of 256 tokens (32 chunks per head)
    E64 = 64 * 64 + 64
    assert la.la_segments(0, 4, 8, 2048, 64, 64) == 8
    assert la.la_workspace_bytes(0, 4, 8, 2048, 64, 64) == 32 * 8 * E64 * 4
    assert la.la_segments(0, 4, 8, 8192, 64, 64) == 16
    # N=64 float32 on the vector-ALU kernels: chunk 16 for the causal form, and a sequence of at
    # most 64 tokens runs as one segment (no workspace); an explicit seg_len of 32 tokens gives
    # two segments. N=96 (six chunks): one chunk per segment, as the vector-ALU kernels keep
    # every segment otherwise; with chunk 32 given, N=64 (two chunks) is still one segment and
    # the global form keeps chunk 32 (three chunks at N=96)
    assert la.la_segments(0, 1, 1, 64, 16, 16, 0, 0, la.LA_F32) == 1
    assert la.la_workspace_bytes(0, 1, 1, 64, 16, 16, 0, 0, la.LA_F32) == 0
    assert la.la_segments(0, 1, 1, 96, 16, 16, 0, 0, la.LA_F32) == 6
    assert la.la_segments(0, 1, 1, 64, 16, 16, 32, 0, la.LA_F32) == 1
    assert la.la_segments(1, 1, 1, 96, 16, 16, 0, 0, la.LA_F32) == 3
    assert la.la_workspace_bytes(0, 1, 1, 64, 16, 16, 0, 32, la.LA_F32) == 2 * (16 * 16 + 16) * 4
    assert la.la_workspace_bytes(0, 1, 1, 64, 16, 16, 0, 64, la.LA_F32) == 0
    # float32, d = d_v in {64, 128}: the float32 matrix-core kernels (chunk 32, one causal
    # workgroup per CU, at least 4 chunks per segment): 256 / 32 = 8 segments at both sizes
    assert la.la_segments(0, 2, 16, 8192, 128, 128, 0, 0, la.LA_F32) == 8
    assert la.la_workspace_bytes(0, 2, 16, 8192, 128, 128, 0, 0, la.LA_F32) == 32 * 8 * E * 4
    assert la.la_segments(0, 4, 8, 2048, 64, 64, 0, 0, la.LA_F32) == 8
    assert la.la_segments(0, 2, 16, 8192, 128, 128, 32, 0, la.LA_F32) == 8
    assert la.la_workspace_bytes(1, 1, 8, 100000, 128, 128) > 0
    assert la.la_workspace_bytes(2, 1, 8, 10, 128, 128) == 0
    assert la.la_workspace_bytes(0, 1, 1, 64, 48, 16) == 0


def test_size_limits():
    # 32-bit index arithmetic: N * max(d, d_v) and B * H * segments must stay below 2^31
    n_max = (2**31 - 1) // 128
    assert la.la_segments(0, 1, 1, n_max, 128, 128) > 0
    assert la.la_workspace_bytes(0, 1, 1, n_max, 128, 128) > 0
    assert la.la_segments(0, 1, 1, n_max + 1, 128, 128) == 0
    assert la.la_segments(1, 1, 1, n_max + 1, 128, 128) == 0
    assert la.la_segments(0, 1, 1, 2**31 // 64 - 1, 64, 128) == 0     # d_v decides
    bh_max = (2**31 - 1) // 8
    assert la.la_segments(0, 1, bh_max, 64, 16, 16) > 0               # B * H at the limit
    assert la.la_segments(0, 1, bh_max + 1, 64, 16, 16) == 0
    assert la.la_segments(0, 2**16, 2**12 + 1, 64, 16, 16) == 0       # B * H > (2^31 - 1) / 8
    # the entry points report the same limit as unsupported (fake pointers 1 TiB apart, so no
    # overlap check fires first; nothing is dereferenced)
    T = 1 << 40
    for fn in ("la_causal_fwd", "la_causal_fwd_state", "la_global_fwd"):
        assert call(fn, q=T, k=2 * T, v=3 * T, out=4 * T, S=5 * T, z=6 * T, B=1, H=1,
                    N=n_max + 1, d=128, dv=128) == la.LA_ENOTSUP
        assert call(fn, q=T, k=2 * T, v=3 * T, out=4 * T, S=5 * T, z=6 * T, B=2**16, H=2**12 + 1,
                    N=64, d=16, dv=16) == la.LA_ENOTSUP


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        la.la_causal_fwd(q, q, q, torch.zeros(1, 1, 4, 16))


def test_error_type_carries_status():
    e = la.LAError(la.LA_ENOTSUP, "la_causal_fwd")
    assert e.status == la.LA_ENOTSUP and "unsupported" in str(e)


def _host(*shape, dtype=None):
    torch = pytest.importorskip("torch")
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def test_binding_checks_every_tensor_layout():
    """The C ABI sees pointers and sizes only, so the binding checks each tensor's shape and
    dtype against (B, H, N, d, d_v, dtype) before any call: a wrong one raises ValueError
    naming the tensor (host tensors of the right layout get as far as the device check)."""
    torch = pytest.importorskip("torch")
    f32 = torch.float32
    B, H, N, d, dv = 2, 3, 8, 16, 32
    q, k, v, out = _host(B, H, N, d), _host(B, H, N, d), _host(B, H, N, dv), _host(B, H, N, dv)
    S, z = _host(B, H, d, dv, dtype=f32), _host(B, H, d, dtype=f32)
    with pytest.raises(ValueError, match="device tensors only"):
        la.la_causal_fwd(q, k, v, out, S, z)
    bad = [
        ("q", dict(q=_host(B, H, N + 1, d))),
        ("q", dict(q=_host(B, H, N, d, dtype=f32))),
        ("v", dict(v=_host(B, H, N - 1, dv))),
        ("out", dict(out=_host(B, H, N, dv, dtype=f32))),
        ("out", dict(out=_host(B, H, N, d))),
        ("S", dict(S=_host(B, H, d, dv))),
        ("S", dict(S=_host(B, H, dv, d, dtype=f32))),
        ("z", dict(z=_host(B, H, dv, dtype=f32))),
    ]
    for name, kw in bad:
        a = dict(q=q, k=k, v=v, out=out, S=S, z=z)
        a.update(kw)
        with pytest.raises(ValueError, match=f"^{name} must"):
            la.la_causal_fwd(**a)
        with pytest.raises(ValueError, match=f"^{name} must"):
            la.la_causal_fwd_ex(a["q"], a["k"], a["v"], a["out"], None, None, a["S"], a["z"])
        with pytest.raises(ValueError, match=f"^{name} must"):
            la.la_global_fwd(a["q"], a["k"], a["v"], a["out"], a["S"], a["z"])
    # separate initial state
    with pytest.raises(ValueError, match="^S must"):
        la.la_causal_fwd_state(q, k, v, out, _host(B, H, d, d, dtype=f32), z, S, z)
    with pytest.raises(ValueError, match="^z must"):
        la.la_causal_fwd_state(q, k, v, out, S, _host(B, H, d), S, z)
    # k and v must be 4-D outside decode
    with pytest.raises(ValueError, match="k and v"):
        la.la_causal_fwd(q, _host(B, H, N, d, 1), v, out)
    with pytest.raises(TypeError):
        la.la_causal_fwd(q.half(), k.half(), v.half(), out.half())


def test_binding_checks_decode_layout():
    torch = pytest.importorskip("torch")
    f32 = torch.float32
    B, H, d, dv = 4, 2, 16, 16
    q, k, v, out = _host(B, H, d), _host(B, H, d), _host(B, H, dv), _host(B, H, dv)
    S, z = _host(B, H, d, dv, dtype=f32), _host(B, H, d, dtype=f32)
    gamma = _host(H, dtype=f32)
    with pytest.raises(ValueError, match="device tensors only"):
        la.la_decode_step(q, k, v, out, S, z)
    with pytest.raises(ValueError, match="device tensors only"):
        la.la_decode_step(q[:, :, None], k[:, :, None], v[:, :, None], out[:, :, None], S, z)
    with pytest.raises(ValueError, match="^out must"):
        la.la_decode_step(q, k, v, _host(B, H, dv, dtype=f32), S, z)
    with pytest.raises(ValueError, match="^S must"):
        la.la_decode_step_ex(q, k, v, out, _host(B, H, d, dv), z)
    with pytest.raises(ValueError, match="^q must"):
        la.la_decode_step(_host(B, H, 1, d), k, v, out, S, z)
    with pytest.raises(ValueError, match="gamma"):
        la.la_decode_step_decay(q, k, v, out, S, z, _host(H))
    with pytest.raises(ValueError, match="gamma"):
        la.la_decode_step_decay(q, k, v, out, S, z, _host(H + 1, dtype=f32))
    with pytest.raises(ValueError, match="device tensors only"):
        la.la_decode_step_decay(q, k, v, out, S, z, gamma)


def test_binding_checks_random_feature_layout():
    torch = pytest.importorskip("torch")
    f32 = torch.float32
    B, H, N, d, dv, m = 1, 2, 8, 16, 16, 32
    q, k, v, out = _host(B, H, N, d), _host(B, H, N, d), _host(B, H, N, dv), _host(B, H, N, dv)
    W = _host(m, d)
    S, z = _host(B, H, m, dv, dtype=f32), _host(B, H, m, dtype=f32)
    with pytest.raises(ValueError, match="device tensors only"):
        la.la_causal_fwd_rf(q, k, v, out, W, None, None, S, z)
    with pytest.raises(ValueError, match="^S must"):
        la.la_causal_fwd_rf(q, k, v, out, W, None, None, _host(B, H, d, dv, dtype=f32), z)
    with pytest.raises(ValueError, match="^W must"):
        la.la_causal_fwd_rf(q, k, v, out, _host(m, d, dtype=f32), None, None, S, z)
    with pytest.raises(ValueError, match="^W must"):
        la.la_causal_fwd_rf(q, k, v, out, _host(m, d + 1), None, None, S, z)
    with pytest.raises(ValueError, match="do not match"):
        la.la_rf_features(q, W, _host(B, H, N, m + 1))
    with pytest.raises(ValueError, match="one dtype"):
        la.la_rf_features(q, W, _host(B, H, N, m, dtype=f32))


def test_workspace_argument_checks():
    """The caller-supplied workspace forms reject a missing, misaligned, short or overlapping
    workspace with LA_EINVAL (after the usual argument checks), before any HIP call."""
    B, H, N, d = 1, 2, 4096, 64
    need = la.la_workspace_bytes(0, B, H, N, d, d, 0, 512, la.LA_BF16)
    gneed = la.la_workspace_bytes(1, B, H, N, d, d, 0, 0, la.LA_BF16)
    assert need > 0 and gneed > 0
    W = 64 * A

    def causal(ws, ws_bytes, q=A, gamma=None, seg=512, flags=0, dtype=la.LA_BF16):
        return la.lib.la_causal_fwd_ws(q, 2 * A, 3 * A, 4 * A, None, None, 5 * A, 6 * A, gamma, B,
                                       H, N, d, d, 0, seg, flags, dtype, ws, ws_bytes, None)

    def glob(ws, ws_bytes):
        return la.lib.la_global_fwd_ws(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, B, H, N, d, d, 0, 0,
                                       la.LA_BF16, ws, ws_bytes, None)

    assert causal(None, 0) == la.LA_EINVAL
    assert causal(W, need - 16) == la.LA_EINVAL
    assert causal(W + 8, need) == la.LA_EINVAL
    assert causal(5 * A - 16, need) == la.LA_EINVAL          # overlaps S
    assert causal(W, need, q=None) == la.LA_EINVAL
    assert causal(W, need, flags=4) == la.LA_EINVAL
    assert causal(W, need, seg=100) == la.LA_ENOTSUP
    assert causal(W, need, gamma=A + 2) == la.LA_EINVAL       # misaligned decay vector
    assert causal(W, need, gamma=W + 64) == la.LA_EINVAL      # decay vector inside the workspace
    assert glob(None, 0) == la.LA_EINVAL
    assert glob(W, gneed - 1) == la.LA_EINVAL
    assert glob(3 * A, gneed) == la.LA_EINVAL                 # overlaps v


def test_release_cache_without_blocks():
    assert la.lib.la_release_cache() == la.LA_OK


def test_noalloc_argument_checks():
    """la_causal_fwd_noalloc validates like la_causal_fwd_ex and refuses a split that needs
    more than its 64 MiB static scratch with LA_ENOSPACE, before any HIP call."""
    f = la.lib.la_causal_fwd_noalloc

    def call(q=A, S=5 * A, z=6 * A, B=1, H=2, N=8, d=16, seg=0, flags=0, T=1):
        return f(q * T if q else None, 2 * A * T, 3 * A * T, 4 * A * T, None, None,
                 S * T if S else None, z * T if z else None, B, H, N, d, d, 0, seg, flags,
                 la.LA_BF16, None)

    assert call(q=None) == la.LA_EINVAL
    assert call(S=None) == la.LA_EINVAL
    assert call(flags=8) == la.LA_EINVAL
    assert call(d=48) == la.LA_ENOTSUP
    # 64 heads x 2048 segments of 64 tokens x 66,048 B: far above 64 MiB
    big = dict(B=1, H=64, N=131072, d=128, seg=64, T=1 << 20)
    assert la.la_workspace_bytes(0, 1, 64, 131072, 128, 128, 0, 64) > 64 << 20
    assert call(**big) == la.LA_ENOSPACE
    assert "static scratch" in la.strerror(la.LA_ENOSPACE)
