"""Host-only checks of the C-ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

from selective_state_space_38_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")
MICRO_HEADER = os.path.join(ROOT, "include", "ssm_micro.h")

SSM_OK, SSM_EINVAL, SSM_EDTYPE, SSM_EALIGN, SSM_ENOMEM = 0, -1, -2, -3, -4


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_abi():
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTED), names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_every_header_is_covered():
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["ssm_micro.h", "ssm_scan.h"], headers


def test_probe_library_exports_its_header():
    names = _declared_functions(MICRO_HEADER)
    assert set(names) == set(_lib.EXPORTED_MICRO), names
    lib = _lib.load_micro()
    for name in names:
        assert hasattr(lib, name), name


def test_probe_validation():
    lib = _lib.load_micro()
    ms = ctypes.c_float()
    # bad selectors and sizes are rejected before any HIP call
    assert lib.ssm_micro_valu(3, 8, 256, 1, P[0], P[1], 1, ctypes.byref(ms), None) == -1
    assert lib.ssm_micro_valu(0, 4, 256, 1, P[0], P[1], 1, ctypes.byref(ms), None) == -1
    assert lib.ssm_micro_stream(4, 4, 256, P[0], P[1], 1 << 20, 1, P[2], 1, ctypes.byref(ms),
                                None) == -1
    assert lib.ssm_micro_stream(2, 3, 256, P[0], P[1], 1 << 20, 1, P[2], 1, ctypes.byref(ms),
                                None) == -1
    assert lib.ssm_micro_stream(2, 4, 256, P[0], P[1], 1000, 1, P[2], 1, ctypes.byref(ms),
                                None) == -1
    assert lib.ssm_micro_stream(2, 4, 256, None, P[1], 1 << 20, 1, P[2], 1, ctypes.byref(ms),
                                None) == -1
    assert lib.ssm_micro_stream(3, 4, 256, None, P[1], 1 << 20, 0, P[2], 1, ctypes.byref(ms),
                                None) == -1


def test_status_strings():
    for rc in (0, -1, -2, -3, -4, -5, -6, -7):
        s = _lib.status_string(rc)
        assert s.startswith("SSM_")
    assert "UNKNOWN" in _lib.status_string(12345)


# fake, never dereferenced device addresses (validation fails first)
P = [ctypes.c_void_p(0x100000 + 0x1000 * i) for i in range(16)]


def _dims(b=2, L=8, d=64, n=16, dtype=0):
    return _lib.SsmDims(b, L, d, n, dtype)


def _fwd(dims, *, u=P[0], delta=P[1], A=P[2], B=P[3], C=P[4], D=None, z=None,
         bias=None, h0=None, out=P[5], last=None):
    lib = _lib.load()
    return lib.selective_scan_fwd_h0(u, delta, A, B, C, D, z, bias, 1, h0, out, last,
                                     ctypes.byref(dims), None)


def _upd(dims, *, state=P[0], x=P[1], dt=P[2], A=P[3], B=P[4], C=P[5], out=P[6]):
    lib = _lib.load()
    return lib.selective_state_update(state, x, dt, A, B, C, None, None, None, 1, out,
                                      ctypes.byref(dims), None)


@pytest.mark.parametrize("field,value", [("batch", 0), ("seqlen", 0), ("dim", 0),
                                         ("dstate", 0), ("dstate", 3), ("dstate", 128),
                                         ("batch", -1),
                                         # beyond the 32-bit launch arithmetic
                                         ("dim", (1 << 24) + 1), ("seqlen", 1 << 31),
                                         ("batch", (1 << 30) + 1)])
def test_fwd_rejects_bad_dims(field, value):
    d = _dims()
    setattr(d, field, value)
    assert _fwd(d) == SSM_EINVAL


def test_fwd_rejects_bad_dtype():
    assert _fwd(_dims(dtype=7)) == SSM_EDTYPE


def test_fwd_rejects_null_required_pointers():
    for key in ("u", "delta", "A", "B", "C", "out"):
        assert _fwd(_dims(), **{key: None}) == SSM_EINVAL, key


def test_fwd_rejects_null_dims():
    lib = _lib.load()
    assert lib.selective_scan_fwd(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, P[5],
                                  None, None, None) == SSM_EINVAL


def test_fwd_rejects_misaligned():
    assert _fwd(_dims(), u=ctypes.c_void_p(0x100002)) == SSM_EALIGN


def test_fwd_rejects_aliasing():
    assert _fwd(_dims(), out=P[0]) == SSM_EINVAL
    assert _fwd(_dims(), last=P[5]) == SSM_EINVAL
    assert _fwd(_dims(), last=P[1]) == SSM_EINVAL


def test_fwd_allocation_failure_is_reported(monkeypatch):
    # four 16-step look-back segments: a plan with carry records, so scratch
    # is allocated (a plan of whole chains allocates nothing)
    monkeypatch.setenv("SSM_TEST_FAIL_ALLOC", "1")
    monkeypatch.setenv("SSM_FORCE_LOOKBACK", "1")
    monkeypatch.setenv("SSM_FORCE_SEGMENT", "16")
    assert _fwd(_dims(L=64)) == SSM_ENOMEM


def test_update_rejects_seqlen_not_one():
    assert _upd(_dims(L=2)) == SSM_EINVAL


def test_update_rejects_nulls_alias_alignment():
    assert _upd(_dims(L=1), state=None) == SSM_EINVAL
    assert _upd(_dims(L=1), out=P[1]) == SSM_EINVAL
    assert _upd(_dims(L=1), state=ctypes.c_void_p(0x100004)) == SSM_EALIGN
    assert _upd(_dims(L=1, dtype=3)) == SSM_EDTYPE


def test_plan_query():
    lib = _lib.load()
    plan = _lib.SsmFwdPlan()
    assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(b=4, L=8192, d=5120, n=16, dtype=1)),
                                ctypes.byref(plan)) == SSM_OK
    assert plan.state_groups * plan.states_per_group == 16
    assert plan.segments * plan.segment_len >= 8192
    assert plan.segment_len % plan.chunk == 0
    chains = 4 * 80
    assert 0 <= plan.whole_chains <= chains
    assert plan.workgroups == plan.whole_chains + (chains - plan.whole_chains) * plan.segments
    # 320 chains on 256 CUs: 256 run whole, the other 64 are split
    assert plan.whole_chains == 256 and plan.segments == 4 and plan.lookback == 1
    assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(n=5)), ctypes.byref(plan)) == SSM_EINVAL
    # channel counts past 2^24 do not fit the kernels' 32-bit chunk offsets
    assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(b=1, L=16, d=1 << 24, n=16)),
                                ctypes.byref(plan)) == SSM_OK
    assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(b=1, L=16, d=(1 << 24) + 64, n=16)),
                                ctypes.byref(plan)) == SSM_EINVAL


def test_forced_segments_are_whole_chunks_of_the_instance(monkeypatch):
    lib = _lib.load()
    plan = _lib.SsmFwdPlan()
    monkeypatch.setenv("SSM_FORCE_LOOKBACK", "1")
    for n, seg, want in ((16, 16, 16), (16, 20, 32), (16, 48, 48), (8, 16, 32), (4, 40, 64)):
        monkeypatch.setenv("SSM_FORCE_SEGMENT", str(seg))
        assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(b=1, L=4096, d=64, n=n)),
                                    ctypes.byref(plan)) == SSM_OK
        assert plan.segment_len == want and plan.segment_len % plan.chunk == 0, (n, seg)
        assert plan.segments == -(-4096 // want)


def test_first_segment_override(monkeypatch):
    """The first segment takes the forced length (rounded to the chunk); the
    others share the rest evenly without adding segments."""
    lib = _lib.load()
    plan = _lib.SsmFwdPlan()
    monkeypatch.setenv("SSM_FORCE_LOOKBACK", "1")
    monkeypatch.setenv("SSM_FORCE_SEGMENT", "96")
    L = 1000
    base_segments = -(-L // 96)
    for first, want in ((0, 96), (32, 32), (40, 48), (160, 160), (5000, 96)):
        monkeypatch.setenv("SSM_FORCE_FIRST_SEGMENT", str(first))
        assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(b=2, L=L, d=96)), ctypes.byref(plan)) == 0
        assert plan.first_segment_len == want, (first, plan.first_segment_len)
        f, s = plan.first_segment_len, plan.segment_len
        assert s % plan.chunk == 0 and plan.segments <= base_segments
        assert f + (plan.segments - 2) * s < L <= f + (plan.segments - 1) * s
        assert plan.workgroups == 2 * 2 * plan.segments


def test_plan_covers_every_supported_state_size():
    lib = _lib.load()
    plan = _lib.SsmFwdPlan()
    for n in (1, 2, 4, 8, 16, 32, 64):
        for L in (1, 17, 5000, 1 << 20):
            assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(b=1, L=L, d=100, n=n)),
                                        ctypes.byref(plan)) == SSM_OK
            assert plan.state_groups * plan.states_per_group == n
            assert (plan.segments - 1) * plan.segment_len < L <= plan.segments * plan.segment_len
            # every helper thread owns a whole run of a tile row; a workgroup
            # stays within the hardware's 1024 threads
            assert plan.helper_waves in (4, 8) and plan.chunk % plan.helper_waves == 0
            assert 64 * (plan.state_groups + plan.helper_waves) <= 1024


def test_plan_helper_waves():
    # eight helpers where the chunk is 16 steps and a scan wave holds at most
    # four states, four otherwise
    lib = _lib.load()
    plan = _lib.SsmFwdPlan()
    for n, want in ((4, 4), (8, 4), (16, 8), (32, 8), (64, 4)):
        assert lib.ssm_fwd_plan_for(ctypes.byref(_dims(b=4, L=2048, d=5120, n=n, dtype=1)),
                                    ctypes.byref(plan)) == SSM_OK
        assert plan.helper_waves == want, (n, plan.state_groups, plan.states_per_group)
        assert (plan.chunk == 16) == (plan.state_groups >= 4)


@pytest.mark.parametrize("bbar", [-1, 2, 7])
def test_ex_entry_points_reject_unknown_bbar(bbar):
    lib = _lib.load()
    d = _dims()
    rc = lib.selective_scan_fwd_ex(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None,
                                   bbar, P[5], None, ctypes.byref(d), None)
    assert rc == SSM_EINVAL
    d1 = _dims(L=1)
    rc = lib.selective_state_update_ex(P[0], P[1], P[2], P[3], P[4], P[5], None, None, None,
                                       1, bbar, P[6], ctypes.byref(d1), None)
    assert rc == SSM_EINVAL


def test_ex_entry_points_validate_like_the_plain_ones():
    lib = _lib.load()
    d = _dims(n=3)
    rc = lib.selective_scan_fwd_ex(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None,
                                   1, P[5], None, ctypes.byref(d), None)
    assert rc == SSM_EINVAL
    rc = lib.selective_scan_fwd_ex(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None,
                                   1, P[0], None, ctypes.byref(_dims()), None)
    assert rc == SSM_EINVAL  # out aliases u
    rc = lib.selective_state_update_ex(P[0], P[1], P[2], P[3], P[4], P[5], None, None, None,
                                       1, 1, P[6], ctypes.byref(_dims(L=2)), None)
    assert rc == SSM_EINVAL  # seqlen must be 1


def _conv(dims, *, x=P[0], w=P[1], out=P[2], s_in=None, s_out=None, width=4):
    lib = _lib.load()
    return lib.causal_conv1d_fwd(x, w, None, s_in, width, 1, out, s_out, ctypes.byref(dims), None)


def test_conv_validation():
    assert _conv(_dims(), width=0) == SSM_EINVAL
    assert _conv(_dims(), width=5) == SSM_EINVAL
    assert _conv(_dims(), x=None) == SSM_EINVAL
    assert _conv(_dims(), out=P[0]) == SSM_EINVAL                    # out aliases x
    assert _conv(_dims(), s_in=P[3], s_out=P[3]) == SSM_EINVAL       # state in == out
    assert _conv(_dims(dtype=9)) == SSM_EDTYPE
    assert _conv(_dims(), x=ctypes.c_void_p(0x100002)) == SSM_EALIGN
    lib = _lib.load()
    d1 = _dims(L=2)
    assert lib.causal_conv1d_update(P[0], P[1], P[2], None, 4, 1, P[3], ctypes.byref(d1),
                                    None) == SSM_EINVAL               # seqlen must be 1
    d1 = _dims(L=1)
    assert lib.causal_conv1d_update(None, P[1], P[2], None, 4, 1, P[3], ctypes.byref(d1),
                                    None) == SSM_EINVAL               # state required
    assert lib.causal_conv1d_update(P[0], P[1], P[2], None, 4, 1, P[0], ctypes.byref(d1),
                                    None) == SSM_EINVAL               # out aliases state


def test_training_pair_validation():
    lib = _lib.load()
    d = _dims(b=2, L=20, d=100, n=16)
    # states: 2 rows x 2 channel blocks x ceil(20/8) checkpoints x 16 states x 64 lanes x
    # 4 bytes, padded to 256 bytes; then the readouts: 2 x 20 x 100 float32
    states = 2 * 2 * 3 * 16 * 64 * 4
    assert lib.ssm_ckpt_bytes(ctypes.byref(d)) == -(-states // 256) * 256 + 2 * 20 * 100 * 4
    assert lib.ssm_ckpt_bytes(ctypes.byref(_dims(n=5))) == SSM_EINVAL
    rc = lib.selective_scan_fwd_train(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None,
                                      P[5], None, None, ctypes.byref(d), None)
    assert rc == SSM_EINVAL            # ckpt is required
    rc = lib.selective_scan_fwd_train(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None,
                                      P[5], None, P[0], ctypes.byref(d), None)
    assert rc == SSM_EINVAL            # ckpt aliases u
    rc = lib.selective_scan_bwd_ckpt(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None,
                                     P[5], None, None, P[6], P[7], P[8], P[9], P[10], None,
                                     None, None, None, ctypes.byref(d), None)
    assert rc == SSM_EINVAL            # ckpt is required


def _fwd_noalloc(dims):
    lib = _lib.load()
    return lib.selective_scan_fwd_noalloc(P[0], P[1], P[2], P[3], P[4], None, None, None, 1,
                                          None, P[5], None, ctypes.byref(dims), None)


def test_noalloc_validates_like_the_allocating_forward():
    assert _fwd_noalloc(_dims(L=0)) == SSM_EINVAL
    assert _fwd_noalloc(_dims(dtype=3)) == SSM_EDTYPE
    assert _fwd_noalloc(_dims(n=5)) == SSM_EINVAL


def test_noalloc_rejects_plans_beyond_its_static_scratch(monkeypatch):
    """16-step look-back segments over 65536 steps and 4 channel blocks need
    16384 carry records (~150 MB): refused on the host with SSM_ESCRATCH,
    before any HIP call."""
    monkeypatch.setenv("SSM_FORCE_LOOKBACK", "1")
    monkeypatch.setenv("SSM_FORCE_SEGMENT", "16")
    assert _fwd_noalloc(_dims(b=1, L=65536, d=256, n=16)) == -7
    assert "SSM_ESCRATCH" in _lib.status_string(-7)


def _agg(dims, *, u=P[0], dt=P[1], A=P[2], B=P[3], bias=None, h0=None, bbar=0, sd=P[4],
         st=P[5]):
    lib = _lib.load()
    return lib.selective_scan_fwd_aggregate(u, dt, A, B, bias, 1, h0, bbar, sd, st,
                                            ctypes.byref(dims), None)


def test_aggregate_entry_point_validation():
    d = _dims()
    assert _agg(d, sd=None) == SSM_EINVAL
    assert _agg(d, st=None) == SSM_EINVAL
    assert _agg(d, u=None) == SSM_EINVAL
    assert _agg(d, B=None) == SSM_EINVAL
    assert _agg(d, bbar=2) == SSM_EINVAL
    assert _agg(_dims(n=3)) == SSM_EINVAL
    assert _agg(_dims(dtype=5)) == SSM_EDTYPE
    assert _agg(d, sd=P[0]) == SSM_EINVAL          # aliases u
    assert _agg(d, st=P[4]) == SSM_EINVAL          # state aliases sum_delta
    assert _agg(d, h0=P[5]) == SSM_EINVAL          # h0 aliases state
    assert _agg(d, sd=ctypes.c_void_p(0x100002)) == SSM_EALIGN


def _comb(dims, S=3, *, sd=P[0], agg=P[1], A=P[2], h0=None, h_in=P[3], h_out=None):
    lib = _lib.load()
    return lib.selective_scan_carry_combine(sd, agg, A, h0, h_in, h_out, S, ctypes.byref(dims),
                                            None)


def test_carry_combine_validation():
    d = _dims()
    assert _comb(d, S=0) == SSM_EINVAL
    assert _comb(d, h_in=None) == SSM_EINVAL
    assert _comb(d, sd=None) == SSM_EINVAL
    assert _comb(d, A=None) == SSM_EINVAL
    assert _comb(_dims(n=5)) == SSM_EINVAL
    assert _comb(d, h_in=P[1]) == SSM_EINVAL       # aliases agg
    assert _comb(d, h_out=P[3]) == SSM_EINVAL      # h_out aliases h_in
    assert _comb(d, h0=P[4], h_out=P[4]) == SSM_EINVAL
    assert _comb(d, agg=ctypes.c_void_p(0x100001)) == SSM_EALIGN


def test_record_entry_points_validation():
    lib = _lib.load()
    d = _dims(L=4096, d=256)
    nb = lib.ssm_fwd_record_bytes(ctypes.byref(d))
    assert nb >= 256 and nb % 256 == 0
    assert lib.ssm_fwd_record_bytes(ctypes.byref(_dims(n=3))) == SSM_EINVAL
    rec = ctypes.c_void_p(0x200000)
    agg = lib.selective_scan_fwd_aggregate_rec
    assert agg(P[0], P[1], P[2], P[3], None, 1, 0, P[4], P[5], None, ctypes.byref(d),
               None) == SSM_EINVAL                                   # no buffer
    assert agg(P[0], P[1], P[2], P[3], None, 1, 0, P[4], P[5], ctypes.c_void_p(0x200010),
               ctypes.byref(d), None) == SSM_EINVAL                  # not 256-byte aligned
    assert agg(P[0], P[1], P[2], P[3], None, 1, 0, P[4], P[5], P[0], ctypes.byref(d),
               None) == SSM_EINVAL                                   # aliases u
    assert agg(P[0], P[1], P[2], P[3], None, 1, 5, P[4], P[5], rec, ctypes.byref(d),
               None) == SSM_EINVAL                                   # bad bbar
    frm = lib.selective_scan_fwd_from_rec
    assert frm(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None, 0, None, P[5], None,
               ctypes.byref(d), None) == SSM_EINVAL                  # no buffer
    assert frm(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None, 0, P[5], P[5], None,
               ctypes.byref(d), None) == SSM_EINVAL                  # rec aliases out
    assert frm(P[0], P[1], P[2], P[3], P[4], None, None, None, 1, None, 0, rec, None, None,
               ctypes.byref(d), None) == SSM_EINVAL                  # no out
