"""The C-ABI library loads, exports every symbol include/kvq.h declares, and its
host-side argument checks and workspace planning behave as documented.  No
device work is enqueued: every call here returns before any HIP launch."""
import ctypes
import os
import re

import pytest

torch = pytest.importorskip("torch")

from quantized_kv_cache_gqa_amd import kvq  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.fail("libkvq.so is not built (run __graft_entry__.build())")
    return kvq.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    fns = declared_functions()
    assert fns == sorted(kvq.SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.kvq_abi_version() == kvq.ABI_VERSION == 11
    for s in range(8):
        assert lib.kvq_status_string(s).decode()
    assert lib.kvq_status_string(99) == b"unknown status"


def test_ctypes_structs_match_the_c_layout(tmp_path):
    """Compile the header with gcc and compare sizeof/offsetof of every field."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    structs = {"kvq_region": kvq.Region, "kvq_attn_args": kvq.AttnArgs,
               "kvq_meter_out": kvq.MeterOut, "kvq_quant_args": kvq.QuantArgs,
               "kvq_plan_info": kvq.PlanInfo}
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){"]
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c99", str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(cls, fname).offset, (cname, fname)


FAKE = 1 << 20          # 16-byte aligned dummy "device" addresses: never dereferenced


def _region(length, kf="fp8", vf="fp8", exact=True, witness=True):
    return kvq.Region(k_format=kvq.FMT[kf], v_format=kvq.FMT[vf], k=FAKE, v=FAKE,
                      k_scale=FAKE if kf != "bf16" else None, v_scale=FAKE if vf != "bf16" else None,
                      witness=FAKE if witness else None, k_exact=FAKE if exact else None,
                      k_exact_format=0, length=length)


TEAM_OFF = 256 + (1 << 20)  # team region: after the control words and the counters' MiB


def _args(batch=64, hq=32, hkv=8, prefix=0, suffix=12628, split=0, flags=0, status=FAKE, **kw):
    return kvq.AttnArgs(batch=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                        sm_scale=128 ** -0.5, split_tokens=split, plan_flags=flags, status=status, q=FAKE,
                        prefix=_region(prefix, "bf16", "fp8", False, False) if prefix else kvq.Region(),
                        suffix=_region(suffix, **kw), out=FAKE)


def _plan(lib, a, m, meter_only=0):
    info = kvq.PlanInfo()
    assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(m), meter_only, ctypes.byref(info)) == 0
    return info


def test_workspace_plan_of_the_batch64_step(lib):
    """The per-chunk plan: one chunk per (request, KV head), partials and the
    TV's spill rows, after the control words, the counters' MiB and the team
    region of the same arguments (none without a device)."""
    a = _args(flags=kvq.PLAN_NO_TEAM)
    m = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    n = lib.kvq_workspace_bytes(ctypes.byref(a), ctypes.byref(m))
    groups, chunks, G = 64 * 8, 1, 4        # 512 groups fill the GPU: one chunk each
    team = _plan(lib, _args(), m)           # the team plan of the same arguments, if any
    region = team.workspace_bytes if team.team else TEAM_OFF
    partials = groups * chunks * G * 144 * 4
    spill = groups * 12640 * G * 8                # 12628 tokens padded to 16-token tiles
    assert n == region + partials + spill
    info = _plan(lib, a, m)
    assert (info.team, info.chunk, info.chunks, info.workspace_bytes) == (0, 12672, 1, n)
    # without TV: no spill (and no team plan either)
    m2 = kvq.MeterOut(tv=None, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    assert lib.kvq_workspace_bytes(ctypes.byref(a), ctypes.byref(m2)) == TEAM_OFF + partials


def test_plan_query_matches_workspace_bytes(lib):
    """kvq_decode_plan reports one size for the decode and the meter call;
    kvq_workspace_bytes covers it and the per-chunk plan of the same
    arguments, whose region lies after the team region; without a device
    there is no team plan and the sizes agree."""
    a = _args()
    m = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    n = lib.kvq_workspace_bytes(ctypes.byref(a), ctypes.byref(m))
    d, mo = _plan(lib, a, m, 0), _plan(lib, a, m, 1)
    assert d.workspace_bytes == mo.workspace_bytes <= n
    chunked = _plan(lib, _args(flags=kvq.PLAN_NO_TEAM), m, 0)
    assert chunked.workspace_bytes == n and chunked.team == 0
    if d.team:
        assert TEAM_OFF < d.workspace_bytes < n        # slots after the control words and counters
    else:
        assert d.workspace_bytes == n
    if not torch.cuda.is_available():
        assert d.team == 0
    assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(m), 0, None) == 1


@pytest.mark.parametrize("suffix_k,suffix_v,launches", [
    ("bf16", "bf16", 1),     # K16 cartridge + BF16 suffix: one launch
    ("bf16", "fp8", 1),
    ("fp8", "fp8", 2),       # key formats differ: one launch per region
])
def test_two_region_calls_take_one_launch_where_formats_allow(lib, suffix_k, suffix_v, launches):
    """A shared BF16-key prefix and a suffix: one kernel over both regions
    when the key formats agree, else one per region; KVQ_PLAN_LAUNCH_PER_REGION
    forces one per region; a one-region call is one launch."""
    a = _args(batch=16, prefix=632, suffix=1024, kf=suffix_k, vf=suffix_v, exact=False, witness=False)
    m = kvq.MeterOut()
    for meter_only in (0, 1):
        info = _plan(lib, a, m, meter_only)
        assert (info.team, info.launches, info.reserved) == (0, launches, 0)
        assert info.chunks >= 2
    a.plan_flags = kvq.PLAN_LAUNCH_PER_REGION
    assert _plan(lib, a, m).launches == 2
    one = _args(batch=16, suffix=1024, kf=suffix_k, vf=suffix_v, exact=False, witness=False)
    assert _plan(lib, one, m).launches == 1


def test_tier_b_arguments_are_checked(lib):
    """Tier B needs a failure probability in (0, 1) and keys whose residual is
    the dither's (INT8) or zero (BF16); FP8 keys are rejected, never metered
    with the wrong proxy.  A Tier B call never takes the team plan."""
    good = _args(batch=8, suffix=32768, kf="int8", vf="int8")
    bad = _args(batch=8, suffix=32768, kf="fp8", vf="fp8")
    mk = lambda delta: kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE,
                                    log_a_b=FAKE, bound_b_raw=FAKE, meter_b=FAKE, delta_b=delta)
    assert _plan(lib, good, mk(1e-6)).team == 0
    for delta, status in ((0.0, 2), (1.0, 2), (-1e-3, 2), (float("nan"), 2)):
        info = kvq.PlanInfo()
        assert lib.kvq_decode_plan(ctypes.byref(good), ctypes.byref(mk(delta)), 0, ctypes.byref(info)) == status
    info = kvq.PlanInfo()
    assert lib.kvq_decode_plan(ctypes.byref(bad), ctypes.byref(mk(1e-6)), 0, ctypes.byref(info)) == 5
    assert lib.kvq_decode_attn(ctypes.byref(bad), ctypes.byref(mk(1e-6)), FAKE, 1 << 40, None) == 5
    two = _args(batch=8, prefix=632, suffix=4096, kf="int8", vf="int8")   # BF16 prefix keys: allowed
    assert _plan(lib, two, mk(1e-6)).chunks >= 2
    m_misaligned = mk(1e-6)
    m_misaligned.meter_b = FAKE + 4
    assert lib.kvq_decode_plan(ctypes.byref(good), ctypes.byref(m_misaligned), 0, ctypes.byref(info)) == 4


def test_value_side_and_tier_a_arguments_are_checked(lib):
    """The value side needs every region's value records (KVQ_ERR_NULL
    otherwise); Tier A and the joint bound reject quantized keys without a
    witness instead of metering them as exact keys."""
    a = _args(batch=4, suffix=4096)                       # FP8 keys with a witness
    vals = dict(value_err=FAKE, v_norm_max=FAKE, out_bound=FAKE)
    info = kvq.PlanInfo()
    m = kvq.MeterOut(**vals)
    assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(m), 0, ctypes.byref(info)) == 1
    a.suffix.v_witness = FAKE
    assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(m), 0, ctypes.byref(info)) == 0
    assert info.team == 0
    nowit = _args(batch=4, suffix=4096, witness=False)
    nowit.suffix.v_witness = FAKE
    for fields in ({"meter": FAKE}, {"log_a": FAKE}, {"out_bound": FAKE}):
        assert lib.kvq_decode_plan(ctypes.byref(nowit), ctypes.byref(kvq.MeterOut(**fields)), 0,
                                   ctypes.byref(info)) == 5
    for fields in ({"value_err": FAKE}, {"tv": FAKE}):   # no TV bound needed
        assert lib.kvq_decode_plan(ctypes.byref(nowit), ctypes.byref(kvq.MeterOut(**fields)), 0,
                                   ctypes.byref(info)) == 0
    k16 = _args(batch=4, suffix=4096, kf="bf16", vf="fp8", exact=False, witness=False)
    k16.suffix.v_witness = FAKE
    assert lib.kvq_decode_plan(ctypes.byref(k16), ctypes.byref(kvq.MeterOut(**vals)), 0,
                               ctypes.byref(info)) == 0


def test_block_report_arguments_and_workspace(lib):
    """The report adds the c spill and the per-block radii to the workspace,
    never takes the team plan, needs the Tier B request for Tier B's
    contributions, and ranks at most 512 blocks."""
    a = _args(batch=64, suffix=12628)
    info = kvq.PlanInfo()
    base = kvq.MeterOut(tv=FAKE, meter=FAKE)
    rep = kvq.MeterOut(tv=FAKE, meter=FAKE, block_mass=FAKE, block_excess=FAKE, block_order=FAKE)
    n0 = _plan(lib, _args(batch=64, suffix=12628, flags=kvq.PLAN_NO_TEAM), base).workspace_bytes
    team = _plan(lib, a, base)                            # its team region, if any, is not reserved
    n0 -= (team.workspace_bytes - TEAM_OFF) if team.team else 0   # for the report (no team plan)
    p = _plan(lib, a, rep)
    groups, rows, nb = 64 * 8, 12640, 50
    assert p.team == 0
    assert p.workspace_bytes == n0 + groups * rows * 4 * 4 + groups * nb * 4 * 4
    assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(kvq.MeterOut(block_excess_b=FAKE)), 0,
                               ctypes.byref(info)) == 5
    long = _args(batch=1, suffix=131073)                   # 513 blocks
    assert lib.kvq_decode_plan(ctypes.byref(long), ctypes.byref(kvq.MeterOut(block_order=FAKE)), 0,
                               ctypes.byref(info)) == 5
    assert lib.kvq_decode_plan(ctypes.byref(long), ctypes.byref(kvq.MeterOut(block_mass=FAKE)), 0,
                               ctypes.byref(info)) == 0


@pytest.mark.parametrize("mutate,status", [
    (lambda a: setattr(a, "head_dim", 64), 5),
    (lambda a: setattr(a, "num_q_heads", 24), 5),        # G = 3
    (lambda a: setattr(a, "num_q_heads", 30), 2),        # not a multiple
    (lambda a: setattr(a, "q", None), 1),
    (lambda a: setattr(a, "q", FAKE + 4), 4),
    (lambda a: setattr(a, "out", None), 1),
    (lambda a: setattr(a, "split_tokens", 100), 2),
    (lambda a: setattr(a.suffix, "k_format", 9), 3),
    (lambda a: setattr(a.suffix, "k_scale", None), 1),
    (lambda a: setattr(a.suffix, "length", 0), 2),       # total length 0
    (lambda a: setattr(a.suffix, "page_table", FAKE), 5),  # page_size 0
])
def test_invalid_arguments_are_rejected_before_launch(lib, mutate, status):
    a = _args()
    mutate(a)
    m = kvq.MeterOut()
    rc = lib.kvq_decode_attn(ctypes.byref(a), ctypes.byref(m), FAKE, 1 << 40, None)
    assert rc == status


def test_workspace_too_small_and_paged_int8_rejected(lib):
    a = _args()
    m = kvq.MeterOut(tv=FAKE)
    need = lib.kvq_workspace_bytes(ctypes.byref(a), ctypes.byref(m))
    assert lib.kvq_decode_attn(ctypes.byref(a), ctypes.byref(m), FAKE, need - 1, None) == 6
    assert lib.kvq_decode_attn(ctypes.byref(a), ctypes.byref(m), None, need, None) == 6
    b = _args(kf="int8", vf="int8")
    b.suffix.page_table = FAKE
    b.suffix.page_size = 16
    b.suffix.max_pages = 12628 // 16
    assert lib.kvq_decode_attn(ctypes.byref(b), ctypes.byref(m), FAKE, 1 << 40, None) == 5
    c = _args(prefix=632)
    c.prefix.lengths = FAKE                           # a prefix has no per-request lengths
    assert lib.kvq_decode_attn(ctypes.byref(c), ctypes.byref(m), FAKE, 1 << 40, None) == 5


def test_quantize_argument_checks(lib):
    q = kvq.QuantArgs(k_format=1, v_format=1, in_format=0, k_in=FAKE, v_in=FAKE, n_seq=2,
                      num_kv_heads=8, head_dim=128, capacity=1000, tok_begin=0, tok_end=1000,
                      k_out=FAKE, v_out=FAKE, k_scale_out=FAKE, v_scale_out=FAKE)
    bad = [("head_dim", 64, 5), ("in_format", 1, 3), ("tok_end", 1001, 2), ("tok_begin", 1000, 2),
           ("k_scale_out", None, 1), ("k_out", FAKE + 8, 4)]
    for field, val, st in bad:
        qq = kvq.QuantArgs.from_buffer_copy(q)
        setattr(qq, field, val)
        assert lib.kvq_quantize(ctypes.byref(qq), None) == st, field
    qi = kvq.QuantArgs.from_buffer_copy(q)
    qi.k_format = 2
    qi.tok_begin = 100                                  # INT8 calls start on a block boundary
    assert lib.kvq_quantize(ctypes.byref(qi), None) == 5
    assert lib.kvq_quantize(None, None) == 1


def test_int8_group_scale_format_arguments(lib):
    """INT8 with per-(token, 32-channel group) scales: keys and values of a
    region share the layout (keys alone for the meter); pages are allowed
    since a token's scales sit in its own row; Tier B accepts the keys but
    not Tier B's per-block contributions (the radius is per token); the
    write path needs no block-aligned start."""
    g = _args(batch=8, suffix=32768, kf="int8g32", vf="int8g32")
    tier_b = dict(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE, log_a_b=FAKE, bound_b_raw=FAKE,
                  meter_b=FAKE, delta_b=1e-6)
    info = kvq.PlanInfo()
    assert _plan(lib, g, kvq.MeterOut(**tier_b)).team == 0
    for kf, vf in (("int8g32", "int8"), ("int8", "int8g32"), ("int8g32", "fp8"), ("bf16", "int8g32")):
        mixed = _args(batch=8, suffix=32768, kf=kf, vf=vf)
        assert lib.kvq_decode_plan(ctypes.byref(mixed), ctypes.byref(kvq.MeterOut(tv=FAKE)), 0,
                                   ctypes.byref(info)) == 5, (kf, vf)
    keys = _args(batch=8, suffix=32768, kf="int8g32", vf="int8")
    assert lib.kvq_decode_plan(ctypes.byref(keys), ctypes.byref(kvq.MeterOut(tv=FAKE)), 1,
                               ctypes.byref(info)) == 0          # meter only: values unused
    paged = _args(batch=8, suffix=32768, kf="int8g32", vf="int8g32")
    paged.suffix.page_table = FAKE
    paged.suffix.page_size = 16
    paged.suffix.max_pages = 32768 // 16
    assert lib.kvq_decode_plan(ctypes.byref(paged), ctypes.byref(kvq.MeterOut(tv=FAKE)), 0,
                               ctypes.byref(info)) == 0
    for fields, status in (({"block_excess_b": FAKE}, 5), ({"block_order": FAKE}, 5),
                           ({"block_excess": FAKE}, 0)):
        m = kvq.MeterOut(**tier_b, **fields)
        assert lib.kvq_decode_plan(ctypes.byref(g), ctypes.byref(m), 0, ctypes.byref(info)) == status, fields
    assert lib.kvq_decode_plan(ctypes.byref(g), ctypes.byref(kvq.MeterOut(tv=FAKE, block_order=FAKE)), 0,
                               ctypes.byref(info)) == 0          # Tier A's page-in order
    q = kvq.QuantArgs(k_format=5, v_format=2, in_format=0, k_in=FAKE, v_in=FAKE, n_seq=2,
                      num_kv_heads=8, head_dim=128, capacity=1000, tok_begin=100, tok_end=1000,
                      k_out=FAKE, v_out=FAKE, k_scale_out=FAKE, v_scale_out=FAKE)
    assert lib.kvq_quantize(ctypes.byref(q), None) == 5            # mixed scale layouts
    q.layer = -1
    q.v_format = 5
    assert lib.kvq_quantize(ctypes.byref(q), None) == 2            # dither tag range


def test_outlier_pair_arguments(lib):
    """Fixed outlier pairs need group-scale keys, at most 16 pairs, both
    pointers, and (write path) bf16 input, since the stored values are the
    inputs themselves."""
    info = kvq.PlanInfo()
    m = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    for kf, n, pairs, vals, status in (("int8g32", 4, FAKE, FAKE, 0), ("int8g32", 16, FAKE, FAKE, 0),
                                       ("int8g32", 17, FAKE, FAKE, 2), ("int8g32", -1, FAKE, FAKE, 2),
                                       ("int8g32", 4, None, FAKE, 1), ("int8g32", 4, FAKE, None, 1),
                                       ("int8g32", 4, FAKE + 4, FAKE, 4), ("int8", 4, FAKE, FAKE, 5),
                                       ("fp8", 4, FAKE, FAKE, 5), ("int8g32", 0, None, None, 0)):
        vf = "int8g32" if kf == "int8g32" else kf
        a = _args(batch=8, suffix=4096, kf=kf, vf=vf)
        a.suffix.n_outlier_pairs, a.suffix.outlier_pairs, a.suffix.k_outliers = n, pairs, vals
        assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(m), 0, ctypes.byref(info)) == status, (kf, n)
    q = kvq.QuantArgs(k_format=5, v_format=5, in_format=3, k_in=FAKE, v_in=FAKE, n_seq=2,
                      num_kv_heads=8, head_dim=128, capacity=1000, tok_begin=0, tok_end=1000,
                      k_out=FAKE, v_out=FAKE, k_scale_out=FAKE, v_scale_out=FAKE,
                      outlier_pairs=FAKE, k_outliers_out=FAKE, n_outlier_pairs=4)
    assert lib.kvq_quantize(ctypes.byref(q), None) == 5             # fp32 input
    q.in_format, q.k_format, q.v_format = 0, 2, 2
    assert lib.kvq_quantize(ctypes.byref(q), None) == 5             # block-scale keys
    q.k_format, q.v_format, q.k_outliers_out = 5, 5, None
    assert lib.kvq_quantize(ctypes.byref(q), None) == 1
    q.k_outliers_out, q.n_outlier_pairs = FAKE, 17
    assert lib.kvq_quantize(ctypes.byref(q), None) == 2


def test_outlier_store_bytes_match_the_page(tmp_path):
    """The binding's key store for group-scale INT8 with m outlier pairs
    takes 136 + 4 m bytes per token and KV head (WitCert Sec. 6.2.5, Table 6:
    136, 144, 152, 168, 200 B/tok/head for m = 0, 2, 4, 8, 16)."""
    import torch
    for m, b in ((0, 136), (2, 144), (4, 152), (8, 168), (16, 200)):
        pairs = torch.arange(m, dtype=torch.int32).view(1, m) if m else None
        st = kvq.alloc_stored(1, 1, 10, "int8g32", None, False, "cpu", outlier_pairs=pairs)
        n = st.k.element_size() * st.k.numel() + st.k_scale.element_size() * st.k_scale.numel()
        if st.k_outliers is not None:
            n += st.k_outliers.element_size() * st.k_outliers.numel()
        assert n == 10 * b, (m, n)


def test_automatic_chunks_are_at_least_640_tokens(lib):
    """The per-chunk plan fills about 512 work-groups, but no automatic chunk is
    shorter than 640 tokens (a multiple of 64): fewer, longer chunks won on
    small steps.  A step that would then have fewer work-groups than CUs (256)
    takes chunks of at least 256 tokens instead, unless a region holds
    block-scale INT8.  An explicit split_tokens is taken as given."""
    m = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    nt = kvq.PLAN_NO_TEAM
    for batch, hkv, suffix, chunk in ((64, 8, 12628, 12672), (8, 8, 32768, 4096), (4, 8, 131072, 8192),
                                      (16, 8, 1024, 640), (1, 1, 64, 256), (1, 1, 100000, 256),
                                      (1, 8, 12628, 256), (1, 8, 4096, 256), (2, 8, 12628, 640)):
        info = _plan(lib, _args(batch=batch, hkv=hkv, hq=4 * hkv, suffix=suffix, flags=nt), m)
        assert info.chunk == chunk, (batch, hkv, suffix, info.chunk)
        assert info.chunks == -(-suffix // chunk)
    two = _plan(lib, _args(batch=1, hkv=1, hq=4, prefix=632, suffix=64, kf="bf16", vf="fp8", exact=False,
                           witness=False), kvq.MeterOut())
    assert (two.chunk, two.chunks, two.launches) == (256, 4, 1)
    # block-scale INT8 keeps 640: its wavefronts take whole 256-token blocks
    for meter_only in (0, 1):
        i8 = _plan(lib, _args(batch=1, hkv=8, hq=32, suffix=4096, kf="int8", vf="int8", flags=nt), m, meter_only)
        assert (i8.chunk, i8.chunks) == (640, 7), (meter_only, i8.chunk)
    info = _plan(lib, _args(batch=16, suffix=1024, split=128, flags=nt), m)
    assert (info.chunk, info.chunks) == (128, 8)


def test_several_chunks_per_group_add_a_finish_launch(lib):
    """With several chunks per (request, KV head) and a TV or block report,
    the per-chunk plan runs those passes in one more launch (its normalizers
    and partial sums in the workspace); KVQ_PLAN_FINALIZE_IN_PLACE keeps them
    in the decode launch's last work-group."""
    nt = kvq.PLAN_NO_TEAM
    tv = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    one_chunk = _plan(lib, _args(flags=nt), tv)                  # 512 groups: one chunk each
    assert (one_chunk.chunks, one_chunk.launches) == (1, 1)
    a = _args(batch=4, suffix=131072, flags=nt)
    info = _plan(lib, a, tv)
    assert info.chunks > 1 and info.launches == 2
    assert _plan(lib, a, kvq.MeterOut(meter=FAKE)).launches == 1  # no TV, no report: nothing to finish
    a.plan_flags = nt | kvq.PLAN_FINALIZE_IN_PLACE
    kept = _plan(lib, a, tv)
    assert kept.launches == 1 and kept.workspace_bytes < info.workspace_bytes


def test_group_of_eight_takes_two_launch_sets_on_the_matrix_cores(lib):
    """8 query heads per KV head with formats the matrix-core kernels take:
    two launch sets of 4 heads (the planner reports twice the launches);
    KVQ_PLAN_VECTOR_ALU keeps one vector-ALU launch."""
    nt, va = kvq.PLAN_NO_TEAM, kvq.PLAN_VECTOR_ALU
    m = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    g4 = _plan(lib, _args(batch=2, hq=16, hkv=4, suffix=4096, flags=nt), m)
    g8 = _plan(lib, _args(batch=2, hq=32, hkv=4, suffix=4096, flags=nt), m)
    assert g8.launches == 2 * g4.launches
    assert _plan(lib, _args(batch=2, hq=32, hkv=4, suffix=4096, flags=va), m).launches == g4.launches
    f32 = _args(batch=2, hq=32, hkv=4, suffix=4096, flags=nt)
    f32.suffix.k_exact_format = 3                                 # fp32 exact keys: vector ALUs
    assert _plan(lib, f32, m).launches == g4.launches


def test_groups_of_one_and_two_plan_the_padded_tile(lib):
    """1 or 2 query heads per KV head on matrix-core formats: the per-chunk
    workspace is sized for the 4-head tile (as for a group of 4 with the same
    KV heads); on the vector-ALU kernel it is sized for the group itself."""
    nt, va = kvq.PLAN_NO_TEAM, kvq.PLAN_VECTOR_ALU
    m = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    g4 = _plan(lib, _args(batch=4, hq=32, hkv=8, suffix=4096, flags=nt), m)
    for hq in (8, 16):
        padded = _plan(lib, _args(batch=4, hq=hq, hkv=8, suffix=4096, flags=nt), m)
        assert (padded.workspace_bytes, padded.launches) == (g4.workspace_bytes, g4.launches), hq
        own = _plan(lib, _args(batch=4, hq=hq, hkv=8, suffix=4096, flags=va), m)
        assert own.workspace_bytes < padded.workspace_bytes, hq


# every variable an earlier build of the library read
OLD_ENV = {"KVQ_DECODE_TEAM": "0", "KVQ_DECODE_KERNEL": "generic", "KVQ_TEAM_HALVES": "0",
           "KVQ_DEFER_FINISH": "0", "KVQ_DECODE_TWO": "0", "KVQ_TEAM_SPIN_LIMIT": "1",
           "KVQ_TEAM_SILENT_MEMBER": "0"}


def _plan_tuple(lib, a, m, meter_only=0):
    i = _plan(lib, a, m, meter_only)
    return (i.team, i.n_teams, i.rounds, i.grid, i.chunk, i.chunks, i.launches, i.workspace_bytes,
            lib.kvq_workspace_bytes(ctypes.byref(a), ctypes.byref(m)))


def test_environment_variables_change_nothing(lib, monkeypatch):
    """The product library reads no environment: it imports no getenv, exports
    no test hook, and every plan is the same with each variable that earlier
    builds read set (plan choices are kvq_attn_args.plan_flags only)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    und = subprocess.run([nm, "-D", "--undefined-only", kvq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert not re.search(r"\b(secure_)?getenv\b", und)
    dfn = subprocess.run([nm, "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "kvq_test_set_team_hooks" not in dfn
    tv = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    shapes = [_args(), _args(batch=4, suffix=131072), _args(batch=2, hq=64, hkv=8, suffix=4096),
              _args(batch=2, hq=8, hkv=8, suffix=4096), _args(batch=16, prefix=632, suffix=1024, kf="bf16",
                                                               vf="bf16", exact=False, witness=False)]
    before = [_plan_tuple(lib, a, tv, mo) for a in shapes for mo in (0, 1)]
    for k, v in OLD_ENV.items():
        monkeypatch.setenv(k, v)
    assert [_plan_tuple(lib, a, tv, mo) for a in shapes for mo in (0, 1)] == before


def test_test_build_exports_the_team_hooks():
    """libkvq_test.so is the same library plus kvq_test_set_team_hooks (its
    host layer compiled with KVQ_TEST_HOOKS); only the tests load it."""
    assert os.path.exists(kvq.TEST_LIB_PATH)
    t = kvq.load_test()
    assert t.kvq_abi_version() == kvq.ABI_VERSION
    assert hasattr(t, "kvq_test_set_team_hooks")
    for name in declared_functions():
        assert hasattr(t, name), name


def test_plan_flags_and_status_word_are_checked(lib):
    """Unknown plan flags and a misaligned status word are rejected before
    any launch; each flag narrows the plan as documented."""
    m = kvq.MeterOut(tv=FAKE, bound_raw=FAKE, meter=FAKE, log_a=FAKE)
    info = kvq.PlanInfo()
    for flags in (0x20, 0x80000000, kvq.PLAN_NO_TEAM | 0x40):
        a = _args(flags=flags)
        assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(m), 0, ctypes.byref(info)) == 5, flags
        assert lib.kvq_decode_attn(ctypes.byref(a), ctypes.byref(m), FAKE, 1 << 40, None) == 5, flags
    a = _args(status=FAKE + 4)
    assert lib.kvq_decode_plan(ctypes.byref(a), ctypes.byref(m), 0, ctypes.byref(info)) == 4
    # no team plan without a status word, nor with NO_TEAM or VECTOR_ALU
    for a in (_args(status=None), _args(flags=kvq.PLAN_NO_TEAM), _args(flags=kvq.PLAN_VECTOR_ALU)):
        assert _plan(lib, a, m).team == 0
    # the same workspace size whatever the flags: the per-chunk region always
    # lies after the team region of the arguments
    sizes = {lib.kvq_workspace_bytes(ctypes.byref(_args(flags=f, status=s)), ctypes.byref(m))
             for f in (0, kvq.PLAN_NO_TEAM, kvq.PLAN_GROUP8_SEPARATE) for s in (FAKE, None)}
    assert len(sizes) == 1
    # finalize in place: one launch where the finish launch would be added
    long = _args(batch=4, suffix=131072, flags=kvq.PLAN_NO_TEAM)
    assert _plan(lib, long, m).launches == 2
    long.plan_flags |= kvq.PLAN_FINALIZE_IN_PLACE
    assert _plan(lib, long, m).launches == 1


def test_header_is_c99_and_a_c_client_links_and_plans(tmp_path):
    """include/kvq.h compiles as strict C99 with warnings as errors, and a C
    program linked against libkvq.so plans the batch-64 step (host-only
    calls) with the same answers the Python binding gets."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "c_client"
    src = os.path.join(os.path.dirname(__file__), "helpers", "c_client.c")
    libdir = os.path.dirname(kvq.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                        os.path.dirname(HEADER), src, "-o", str(exe), "-L", libdir, "-lkvq",
                        "-Wl,-rpath," + libdir], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert out["abi"] == str(kvq.ABI_VERSION)
    assert out["status"] == "0 ok"
    assert out["plan"] == "chunk 12672 chunks 1 launches 1 team 0"
    ws = [int(x) for x in out["workspace"].split()]
    assert ws[0] == ws[1] > 0
    assert out["bad"] == "head_dim 5"
