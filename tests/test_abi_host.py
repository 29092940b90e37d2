"""The C-ABI library on the host (no GPU): it loads, exports every function
include/ssm_scan.h, include/ssm_conv_norm.h and include/ssm_gdn.h declare, rejects bad arguments with the documented codes
before touching any device, and reports launch geometry; every compiled
kernel keeps its state in registers (no scratch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import mamba2_selective_scan_amd as m

D = m.Dims


def test_exports_every_declared_symbol():
    names = m.header_symbols()
    assert set(names) == {"ssm_scan_prefill", "ssm_scan_decode", "ssm_scan_strerror",
                          "ssm_scan_version", "ssm_scan_check_metadata",
                          "ssm_scan_check_metadata_host",
                          "ssm_scan_query_geometry", "ssm_scan_last_hip_error",
                          "ssm_scan_last_hip_error_string", "ssm_scan_prefill_ws",
                          "ssm_scan_prefill_workspace_size", "ssm_scan_query_prefill_plan",
                          "ssm_scan_prefill_opt", "ssm_scan_decode_opt", "ssm_scan_prefill_static",
                          "ssm_conv1d_silu_prefill", "ssm_conv1d_silu_decode",
                          "ssm_gated_rmsnorm", "ssm_gdn_prefill", "ssm_gdn_decode",
                          "ssm_gdn_prefill_ws", "ssm_gdn_prefill_workspace_size"}
    for n in names:
        assert hasattr(m.lib(), n), n


def test_calib_library_exports_its_declared_symbol():
    """The benchmark's stream-ceiling aid (include/ssm_calib.h) is a library
    of its own; it loads and exports what its header declares, and rejects
    bad arguments before any launch."""
    path = os.path.join(os.path.dirname(m.LIB_PATH), "libssmcalib.so")
    lib = ctypes.CDLL(path)
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(m.LIB_PATH)), "include",
                            "ssm_calib.h")).read()
    names = set(re.findall(r"^\s*int\s+(ssm_\w+)\s*\(", hdr, re.M))
    assert names == {"ssm_calib_stream_rw"}
    f = lib.ssm_calib_stream_rw
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                  ctypes.c_void_p]
    assert f(None, 1024, 1, 1.0, 0.0, None) == -2
    assert f(FAKE + 4, 1024, 1, 1.0, 0.0, None) == -4
    assert f(FAKE, 0, 1, 1.0, 0.0, None) == -2
    assert f(FAKE, 100, 1, 1.0, 0.0, None) == -2          # not a multiple of 256 * per_lane
    assert f(FAKE, 1024, 3, 1.0, 0.0, None) == -2


def test_version_and_strerror():
    assert m.version() == 2
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert m.strerror(code) and "unknown" not in m.strerror(code)
    assert "unknown" in m.strerror(-99)
    assert m.lib().ssm_scan_last_hip_error() == 0
    assert m.lib().ssm_scan_last_hip_error_string() == b"no error"


FAKE = 0x10000          # never dereferenced: argument checks fail before any launch


def _prefill(dims, n_seqs=1, n_tokens=4, ptrs=None, n_slots=1, fake=FAKE):
    p = dict(cu=fake, slot=fake, fresh=fake, x=fake, dt=fake, A=fake, B=fake, C=fake,
             state=fake, y=fake)
    p.update(ptrs or {})
    return m.lib().ssm_scan_prefill(None if dims is None else ctypes.byref(dims), n_seqs,
                                    n_tokens, p["cu"], p["slot"], p["fresh"], p["x"], p["dt"],
                                    p["A"], p["B"], p["C"], p["state"], n_slots, p["y"], None)


def _decode(dims, n_seqs=1, ptrs=None, n_slots=1, fake=FAKE):
    p = dict(slot=fake, fresh=fake, x=fake, dt=fake, A=fake, B=fake, C=fake, state=fake, y=fake)
    p.update(ptrs or {})
    return m.lib().ssm_scan_decode(None if dims is None else ctypes.byref(dims), n_seqs,
                                   p["slot"], p["fresh"], p["x"], p["dt"], p["A"], p["B"],
                                   p["C"], p["state"], n_slots, p["y"], None)


@pytest.mark.parametrize("call", [_prefill, _decode])
def test_argument_errors(call):
    ok = D(4, 8, 16, 2)
    assert call(None) == m.SSM_ERR_NULL
    for bad in (D(0, 8, 16, 2), D(4, 0, 16, 2), D(4, 8, 0, 2), D(4, 8, 16, 0), D(4, 8, 16, 3),
                D(-4, 8, 16, 2)):
        assert call(bad) == m.SSM_ERR_DIMS
    assert call(D(4, 8, 1025, 2)) == m.SSM_ERR_UNSUPPORTED
    assert call(ok, n_seqs=-1) == m.SSM_ERR_DIMS
    assert call(ok, n_seqs=0) == m.SSM_OK                # no-op, nothing launched
    assert call(ok, n_slots=0) == m.SSM_ERR_DIMS
    assert call(ok, n_slots=-2) == m.SSM_ERR_DIMS
    for name in ("slot", "fresh", "A", "state", "x", "y"):
        assert call(ok, ptrs={name: None}) == m.SSM_ERR_NULL, name
    for name in ("x", "dt", "A", "B", "C", "state", "y", "slot"):
        assert call(ok, ptrs={name: FAKE + 2}) == m.SSM_ERR_ALIGN, name


def test_prefill_specific_errors():
    ok = D(4, 8, 16, 2)
    assert _prefill(ok, n_tokens=-1) == m.SSM_ERR_DIMS
    assert _prefill(ok, ptrs={"cu": None}) == m.SSM_ERR_NULL
    assert _prefill(ok, ptrs={"cu": FAKE + 1}) == m.SSM_ERR_ALIGN


def test_check_metadata():
    cu = np.array([0, 3, 3, 5], np.int32)
    assert m.check_metadata(cu, np.array([2, 0, 1]), 5, 3) == m.SSM_OK
    assert m.check_metadata(cu, np.array([2, 0, 2]), 5, 3) == m.SSM_ERR_METADATA   # repeated
    assert m.check_metadata(cu, np.array([2, 0, 3]), 5, 3) == m.SSM_ERR_METADATA   # range
    assert m.check_metadata(cu, np.array([2, 0, -1]), 5, 3) == m.SSM_ERR_METADATA
    assert m.check_metadata(cu, np.array([2, 0, 1]), 6, 3) == m.SSM_ERR_METADATA   # total
    assert m.check_metadata(np.array([1, 3, 3, 5]), np.array([2, 0, 1]), 5, 3) == m.SSM_ERR_METADATA
    assert m.check_metadata(np.array([0, 3, 2, 5]), np.array([2, 0, 1]), 5, 3) == m.SSM_ERR_METADATA
    assert m.check_metadata(None, np.arange(300)[::-1], 0, 300) == m.SSM_OK       # decode, big
    assert m.check_metadata(None, np.r_[np.arange(200), 7], 0, 300) == m.SSM_ERR_METADATA
    assert m.lib().ssm_scan_check_metadata_host(2, 0, None, None, 4) == m.SSM_ERR_NULL
    # the device form rejects sizes and a missing slot array before any copy
    assert m.lib().ssm_scan_check_metadata(2, 0, None, None, 4, None) == m.SSM_ERR_NULL
    assert m.lib().ssm_scan_check_metadata(-1, 0, None, None, 4, None) == m.SSM_ERR_DIMS
    assert m.lib().ssm_scan_check_metadata(0, 0, None, None, 4, None) == m.SSM_OK


@pytest.mark.parametrize("N", [1, 15, 16, 17, 64, 100, 128, 129, 256, 300, 512, 513, 1024])
@pytest.mark.parametrize("decode", [False, True])
def test_geometry(N, decode):
    for aligned in (True, False):
        g = m.geometry(64, 96, N, 8, 3, decode=decode, aligned=aligned)
        R, E = g["lanes_per_row"], g["elems_per_lane"]
        assert R * E >= N and 64 % R == 0
        assert g["rows_per_block"] == 4 * 64 // R
        assert g["blocks"] == 3 * 64 * -(-96 // g["rows_per_block"])
        assert g["lds_bytes"] <= 160 * 1024
        assert g["chunk_tokens"] == (1 if decode else g["chunk_tokens"])
        assert g["vector_path"] == int(aligned and N % 4 == 0)


def test_vector_path_needs_chunk_in_buffer_range():
    """The vector path stages a chunk of up to 32 tokens' x (and B, C) through
    buffer descriptors with 32-bit byte ranges: H * P (and G * N) times 32
    tokens times 4 bytes must stay below 2^31, else the scalar path runs."""
    assert m.geometry(64, 64, 128, 8, 1)["vector_path"] == 1
    assert m.geometry(4096, 4092, 128, 8, 1)["vector_path"] == 1        # 128 B short of 2^31
    assert m.geometry(4096, 4096, 128, 8, 1)["vector_path"] == 0        # 2^24 rows x 128 B = 2^31
    assert m.geometry(65536, 256, 128, 1, 1)["vector_path"] == 0


def test_no_kernel_uses_scratch():
    """Each lane's state array must stay in VGPRs: every kernel in the build's
    resource report has ScratchSize 0."""
    report = os.path.join(os.path.dirname(m.LIB_PATH), "libssmscan.resources.txt")
    text = open(report).read()
    names = re.findall(r"Function Name: (\S+)", text)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    # 7 state-size classes x (vector, scalar) x (4 option sets x (prefill, decode)
    # + segment scan + correction) + 2 combine kernels + 6 matrix-core corrections
    # (3 contraction lengths, masked or not) + matrix-core segment kernels: the
    # state pass at 32, 64 or 128 columns and the scan pass at 1..8 16-column
    # tiles with one or two row tiles per wave
    # + 7 branch-free decode kernels (one per state-size class, vector path)
    # + 7 x 2 whole-sequence prefills at half the chunk (vector, scalar);
    # conv1d + SiLU: (vector, scalar) x (4 history lengths x (decode, prefill)
    # + 3 with snapshots); gated RMSNorm: (vector, scalar) x 6 row-length classes
    n_scan = 7 * 2 * (4 * 2 + 2) + 2 + 6 + 3 + 8 * 2 + 7 + 7 * 2
    n_conv = 2 * (4 * 2 + 3)
    n_norm = 2 * 6
    # gated delta rule: 5 key-width classes x (vector, scalar) x (prefill, decode)
    # x (snapshots or not)
    # + the chunked prefill: (prep, scan) x key widths 64 and 128
    # + 5 branch-free decode kernels (one per key-width class, vector path)
    n_gdn = 5 * 2 * 2 * 2 + 2 * 2 + 5
    assert len(names) == n_scan + n_conv + n_norm + n_gdn and len(scratch) == len(names)
    assert all(v == 0 for v in scratch), dict(zip(names, scratch))


@pytest.mark.parametrize("n_seqs", [1, 2, 3, 4, 5, 8])
def test_prefill_chunk_by_grid_size(n_seqs):
    """Whole-sequence prefill takes half the table's chunk when its grid would
    not be resident at once with the full chunk (two workgroups of 74 KB of
    LDS per CU, 256 CUs) but would be with half (four per CU)."""
    g = m.geometry(64, 96, 128, 8, n_seqs)          # 6 row blocks per head: 384 per sequence
    assert g["blocks"] == 384 * n_seqs
    half = 512 < g["blocks"] <= 1024
    assert g["chunk_tokens"] == (16 if half else 32)
    assert g["lds_bytes"] * (4 if half else 2) <= 160 * 1024
    mixed = m.geometry(16, 96, 100, 4, 8)            # the mixed edge batch: 768 workgroups
    assert mixed["blocks"] == 768 and mixed["chunk_tokens"] == 16
    assert m.geometry(64, 64, 128, 8, 16, decode=True)["chunk_tokens"] == 1


def test_single_hip_runtime():
    """The library shares torch's HIP runtime (one libamdhip64 mapped)."""
    assert len(m.hip_runtimes_loaded()) == 1, m.hip_runtimes_loaded()


@pytest.mark.parametrize("H,G,P", [(64, 8, 64), (16, 2, 32), (4, 1, 96), (4, 2, 96), (2, 1, 256),
                                   (4, 2, 16), (4, 2, 48), (4, 2, 80), (6, 3, 160), (8, 1, 112),
                                   (3, 3, 32), (12, 4, 208)])
def test_scan_pass_windows(H, G, P):
    """The matrix-core scan pass's geometry, modelled on the host: a workgroup
    owns a window of 64 TW rows of a group's flattened (head, row) space, cut at
    the group's end, and wave w the TW 16-row tiles from row 16 TW w (TW = 2
    when P % 32 == 0).  Every row of every group is covered by exactly one wave;
    a wave's tiles stay in one head; a window touches at most four heads (the
    per-head scalar rows of wave 0); the library plans the same window size and
    grid (16 segments forced, one sequence)."""
    N, n_segs = 128, 16
    tw = 2 if P % 32 == 0 else 1
    rbw = 64 * tw
    hpg = H // G
    group_rows = hpg * P
    wpg = -(-group_rows // rbw)
    covered = np.zeros(H * P, np.int32)
    for g in range(G):
        group_end = (g + 1) * group_rows
        for wb in range(wpg):
            fr_wg = g * group_rows + wb * rbw
            rows_wg = min(rbw, group_end - fr_wg)
            assert rows_wg > 0 and rows_wg % (16 * tw) == 0
            h_wg = fr_wg // P
            n_heads = (fr_wg + rows_wg - 1) // P - h_wg + 1
            assert 1 <= n_heads <= 4 and (fr_wg + rows_wg - 1) // P < (g + 1) * hpg
            for w in range(4):
                fr0 = fr_wg + 16 * tw * w
                if fr0 >= fr_wg + rows_wg:
                    continue
                assert fr0 // P == (fr0 + 16 * tw - 1) // P          # one head
                assert 0 <= fr0 // P - h_wg < n_heads
                covered[fr0:fr0 + 16 * tw] += 1
    assert np.all(covered == 1)
    plan = m.prefill_plan(H, P, N, G, 1, 16 * 256, n_segs)
    assert plan["rows_per_block"] == rbw
    assert plan["blocks"] == plan["segments"] * G * wpg


def test_prefill_plan_and_workspace():
    """The headline prefill (1 x 4096 at H64 P64 N128 G8) gives the wide
    matrix-core scan pass 128 wavefronts per segment, so automatic planning
    cuts it into 16 segments of 256 tokens (2048 waves); the register segment
    scan's shapes aim at 4096 waves; a batch that already fills the GPU is not
    cut; forcing works; the workspace holds one [H][P][N] state per segment
    plus the decay arrays."""
    g = m.prefill_plan(64, 64, 128, 8, 1, 4096)
    assert g["segments"] == 16 and g["segment_tokens"] == 256 and g["blocks"] == 16 * 32
    # the scan pass of this shape takes two tiles per wave: 128 rows (two heads) per
    # workgroup, two workgroups to a CU's 160 KB of LDS
    assert g["chunk_tokens"] == 16 and g["rows_per_block"] == 128 and 2 * g["lds_bytes"] <= 160 * 1024
    ws = m.workspace_size(64, 64, 128, 8, 1, 4096, 4096)
    # + per-segment decay totals [1][16][64] and alignment
    assert 16 * 64 * 64 * 128 * 4 + 4096 * 64 * 4 <= ws <= 16 * 64 * 64 * 128 * 4 + 4096 * 64 * 4 + 16 * 64 * 4 + 512
    g = m.prefill_plan(64, 64, 100, 8, 1, 4096)           # N 100: the matrix-core scan, 7 padded tiles
    assert g["segments"] == 16 and g["segment_tokens"] == 256 and g["blocks"] == 16 * 32
    assert g["elems_per_lane"] == 28 and g["rows_per_block"] == 128
    # the mixed edge batch (longest 150) is too short to split: one pass; forced,
    # the matrix-core split takes it in padded 16-column tiles
    assert m.prefill_plan(16, 96, 100, 4, 8, 150)["segments"] == 1
    g = m.prefill_plan(16, 96, 100, 4, 8, 150, segments=4)
    assert g["segments"] == 4 and g["segment_tokens"] == 48 and g["blocks"] == 4 * 8 * 4 * 3
    g = m.prefill_plan(64, 64, 256, 8, 1, 4096)                       # register segment scan
    assert g["segments"] == 4 and g["segment_tokens"] == 1024 and g["blocks"] == 4 * 256
    assert m.prefill_plan(64, 64, 128, 8, 16, 4096)["segments"] == 1     # 16 seqs fill it
    assert m.workspace_size(64, 64, 128, 8, 16, 65536, 4096) == 0
    g = m.prefill_plan(64, 64, 128, 8, 1, 512)      # at least 128 tokens a segment
    assert g["segments"] == 4 and g["segment_tokens"] == 128
    assert m.prefill_plan(64, 64, 128, 8, 1, 255)["segments"] == 1        # too short
    f = m.prefill_plan(4, 16, 16, 1, 1, 64, segments=3)
    assert f["segments"] == 3 and f["segment_tokens"] == 22     # whole 16-token chunks would give 2
    assert m.prefill_plan(64, 64, 128, 8, 1, 4096, segments=1)["segments"] == 1


@pytest.mark.parametrize("bad", [dict(max_seqlen=-1), dict(n_segments=-2)])
def test_prefill_ws_errors(bad):
    kw = dict(max_seqlen=8, n_segments=0)
    kw.update(bad)
    rc = m.lib().ssm_scan_prefill_ws(ctypes.byref(D(4, 8, 16, 2)), 1, 4, kw["max_seqlen"],
                                     kw["n_segments"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, 1, FAKE, None, 0, None)
    assert rc == m.SSM_ERR_DIMS


# ------------------------------------------------------------ conv1d + SiLU, gated RMSNorm
CD = m.ConvDims


def _conv(dims, n_seqs=1, n_tokens=4, ptrs=None, n_slots=1, fake=FAKE, decode=False):
    p = dict(cu=fake, slot=fake, fresh=fake, x=fake, w=fake, state=fake, out=fake, snaps=None)
    p.update(ptrs or {})
    d = None if dims is None else ctypes.byref(dims)
    if decode:
        return m.lib().ssm_conv1d_silu_decode(d, n_seqs, p["slot"], p["fresh"], p["x"], p["w"],
                                              p["state"], n_slots, p["out"], None)
    return m.lib().ssm_conv1d_silu_prefill(d, n_seqs, n_tokens, p["cu"], p["slot"], p["fresh"],
                                           p["x"], p["w"], p["state"], n_slots, p["out"],
                                           p["snaps"], None)


@pytest.mark.parametrize("decode", [False, True])
def test_conv_argument_errors(decode):
    ok = CD(64, 4)
    call = lambda *a, **k: _conv(*a, decode=decode, **k)
    assert call(None) == m.SSM_ERR_NULL
    assert call(CD(0, 4)) == m.SSM_ERR_DIMS
    assert call(CD(64, 0)) == m.SSM_ERR_DIMS
    assert call(CD(64, 5)) == m.SSM_ERR_UNSUPPORTED
    assert call(ok, n_seqs=-1) == m.SSM_ERR_DIMS
    assert call(ok, n_seqs=0) == m.SSM_OK                 # no-op, nothing touched
    assert call(ok, n_slots=0) == m.SSM_ERR_DIMS
    for name in ("slot", "fresh", "x", "w", "state", "out"):
        assert call(ok, ptrs={name: None}) == m.SSM_ERR_NULL, name
    for name in ("x", "w", "state", "out"):
        assert call(ok, ptrs={name: FAKE + 2}) == m.SSM_ERR_ALIGN, name
    assert call(ok, ptrs={"slot": FAKE + 1}) == m.SSM_ERR_ALIGN
    if not decode:
        assert call(ok, n_tokens=-1) == m.SSM_ERR_DIMS
        assert call(ok, ptrs={"cu": None}) == m.SSM_ERR_NULL
        assert call(ok, ptrs={"cu": FAKE + 2}) == m.SSM_ERR_ALIGN
        assert call(ok, ptrs={"snaps": FAKE + 2}) == m.SSM_ERR_ALIGN


def test_norm_argument_errors():
    f = m.lib().ssm_gated_rmsnorm
    assert f(4, 0, FAKE, FAKE, FAKE, 1e-5, FAKE, None) == m.SSM_ERR_DIMS
    assert f(-1, 8, FAKE, FAKE, FAKE, 1e-5, FAKE, None) == m.SSM_ERR_DIMS
    assert f(4, 8, FAKE, FAKE, FAKE, -1.0, FAKE, None) == m.SSM_ERR_DIMS
    assert f(4, 8, FAKE, FAKE, FAKE, float("nan"), FAKE, None) == m.SSM_ERR_DIMS
    assert f(4, 8, FAKE, FAKE, FAKE, float("inf"), FAKE, None) == m.SSM_ERR_DIMS
    assert f(0, 8, None, None, None, 1e-5, None, None) == m.SSM_OK
    for i in range(4):
        ptrs = [FAKE] * 4
        ptrs[i] = None
        assert f(4, 8, ptrs[0], ptrs[1], ptrs[2], 1e-5, ptrs[3], None) == m.SSM_ERR_NULL
        ptrs[i] = FAKE + 2
        assert f(4, 8, ptrs[0], ptrs[1], ptrs[2], 1e-5, ptrs[3], None) == m.SSM_ERR_ALIGN


# ------------------------------------------------------------ gated delta rule
GD = m.GdnDims


def _gdn(dims, n_seqs=1, n_tokens=4, ptrs=None, n_slots=1, fake=FAKE, decode=False):
    p = dict(cu=fake, slot=fake, fresh=fake, q=fake, k=fake, v=fake, g=fake, beta=fake,
             state=fake, y=fake, snaps=None)
    p.update(ptrs or {})
    d = None if dims is None else ctypes.byref(dims)
    if decode:
        return m.lib().ssm_gdn_decode(d, n_seqs, p["slot"], p["fresh"], p["q"], p["k"], p["v"],
                                      p["g"], p["beta"], 0.125, p["state"], n_slots, p["y"],
                                      p["snaps"], None)
    return m.lib().ssm_gdn_prefill(d, n_seqs, n_tokens, p["cu"], p["slot"], p["fresh"], p["q"],
                                   p["k"], p["v"], p["g"], p["beta"], 0.125, p["state"], n_slots,
                                   p["y"], p["snaps"], None)


@pytest.mark.parametrize("decode", [False, True])
def test_gdn_argument_errors(decode):
    ok = GD(32, 16, 128, 128)
    call = lambda *a, **k: _gdn(*a, decode=decode, **k)
    assert call(None) == m.SSM_ERR_NULL
    for bad in (GD(0, 1, 8, 8), GD(4, 0, 8, 8), GD(4, 2, 0, 8), GD(4, 2, 8, 0), GD(6, 4, 8, 8)):
        assert call(bad) == m.SSM_ERR_DIMS
    assert call(GD(4, 2, 257, 8)) == m.SSM_ERR_UNSUPPORTED
    assert call(ok, n_seqs=-1) == m.SSM_ERR_DIMS
    assert call(ok, n_seqs=0) == m.SSM_OK
    assert call(ok, n_slots=0) == m.SSM_ERR_DIMS
    for name in ("slot", "fresh", "state", "q", "k", "v", "g", "beta", "y"):
        assert call(ok, ptrs={name: None}) == m.SSM_ERR_NULL, name
    for name in ("q", "k", "v", "g", "beta", "state", "y"):
        assert call(ok, ptrs={name: FAKE + 2}) == m.SSM_ERR_ALIGN, name
    assert call(ok, ptrs={"snaps": FAKE + 2}) == m.SSM_ERR_ALIGN
    assert call(ok, ptrs={"slot": FAKE + 1}) == m.SSM_ERR_ALIGN
    if not decode:
        assert call(ok, n_tokens=-1) == m.SSM_ERR_DIMS
        assert call(ok, ptrs={"cu": None}) == m.SSM_ERR_NULL


def test_gdn_workspace_size():
    size = lambda *a: m.gdn_workspace_size(*a)
    # one unit of 1680 floats per (sequence, 32-token chunk, value head)
    assert size(32, 16, 128, 128, 1, 4096) == 128 * 32 * 1680 * 4
    assert size(4, 2, 64, 32, 3, 33) == 3 * 2 * 4 * 1680 * 4
    assert size(4, 2, 128, 64, 3, 31) == 0       # short sequences: per-token kernel
    assert size(4, 2, 100, 64, 3, 500) == 0      # key width without a chunked form
    assert size(4, 2, 128, 24, 3, 500) == 0      # value rows not in 16-row tiles
    # a chunk's rows of v (or of q, k) past 32-bit buffer offsets: per-token kernel
    assert size(1024, 1024, 128, 8192, 1, 64) == 2 * 1024 * 1680 * 4
    assert size(1024, 1024, 128, 16384, 1, 64) == 0
    assert size(2048, 2048, 128, 16384, 1, 64) == 0
    assert size(262144, 262144, 128, 16, 1, 64) == 0
    b = ctypes.c_size_t()
    lib = m.lib()
    assert lib.ssm_gdn_prefill_workspace_size(None, 1, 64, ctypes.byref(b)) == m.SSM_ERR_NULL
    assert lib.ssm_gdn_prefill_workspace_size(ctypes.byref(GD(4, 2, 128, 64)), 1, 64, None) == m.SSM_ERR_NULL
    assert lib.ssm_gdn_prefill_workspace_size(ctypes.byref(GD(4, 2, 128, 64)), -1, 64, ctypes.byref(b)) == m.SSM_ERR_DIMS
    assert lib.ssm_gdn_prefill_workspace_size(ctypes.byref(GD(4, 2, 128, 64)), 1, -1, ctypes.byref(b)) == m.SSM_ERR_DIMS
    assert lib.ssm_gdn_prefill_workspace_size(ctypes.byref(GD(6, 4, 128, 64)), 1, 64, ctypes.byref(b)) == m.SSM_ERR_DIMS


def test_gdn_prefill_ws_argument_errors():
    """Errors the chunked entry point reports before anything is enqueued."""
    lib = m.lib()
    d = GD(4, 2, 128, 64)
    need = m.gdn_workspace_size(4, 2, 128, 64, 1, 64)

    def call(max_seqlen=64, ws=FAKE, ws_bytes=need, dims=d, n_seqs=1):
        return lib.ssm_gdn_prefill_ws(None if dims is None else ctypes.byref(dims), n_seqs, 64,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, FAKE,
                                      1, FAKE, max_seqlen, ws, ws_bytes, None)
    assert call(dims=None) == m.SSM_ERR_NULL
    assert call(max_seqlen=-1) == m.SSM_ERR_DIMS
    assert call(ws=None) == m.SSM_ERR_NULL
    assert call(ws_bytes=need - 1) == m.SSM_ERR_DIMS
    assert call(ws=FAKE + 4) == m.SSM_ERR_ALIGN
    assert call(n_seqs=0) == m.SSM_OK
