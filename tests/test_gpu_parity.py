"""GPU parity of the HIP path against the float64 CPU oracle (through the C ABI).

Tolerances:
* codes: bit-exact;
* h = SiLU(y_gate) * y_up: max |dh| <= 2e-3 * max |h_oracle| per (token, slot);
* z = Phi^T x: max |dz| <= 1e-5 * max |z_oracle| per token (fp16 products are
  exact in float32; only the float32 sum over din rounds);
* y (expert apply alone): max |dy| <= 5e-4 * max |y_oracle| per pair (float32
  accumulation over up to r terms of both signs).
"""
import sys

import numpy as np
import pytest

import synth
from oracle import fmt
from tests.oracle_ref import max_rel_err, pairs_ref, z_ref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

H_TOL = 2e-3
Z_TOL = 1e-5
Y_TOL = 5e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session")
def bm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from spectral_expert_gemv_amd import bitsmoe
    return bitsmoe


_DEV = {}


def device_layer(name):
    from spectral_expert_gemv_amd import DeviceLayer
    if name not in _DEV:
        _say("building layer %s" % name)
        L = synth.make_layer(synth.LAYERS[name])
        _DEV[name] = (L, DeviceLayer.from_synth(L))
    return _DEV[name]


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run_gateup(dev, x, ids):
    h = dev.gateup(_cuda(x), _cuda(ids))
    torch.cuda.synchronize()
    return h.cpu().numpy()


# ------------------------------------------------------------------ codes

def _expected_operands(bm, q, bits, path):
    """What decoder `path` must produce from codes q (r x dout, the oracle
    unpacker's) of columns of widths bits (r): DUMP_I8 takes the int8 operand
    byte (code - 128 for 8-bit columns, i.e. the code with its top bit
    flipped), DUMP_F16 the fp16 bit pattern of the code; 16-bit columns keep
    their stored fp16 bits and 0-bit columns are 0 on every path."""
    out = q.copy()
    if path == bm.DUMP_I8:
        w8 = bits == 8
        out[w8] = q[w8] ^ 0x80
    elif path == bm.DUMP_F16:
        small = (bits > 0) & (bits < 16)
        out[small] = q[small].astype(np.float16).view(np.uint16)
    return out


@pytest.mark.parametrize("name,experts", [("tiny", None), ("wide", None), ("heavy", None),
                                          ("qwen3_30b_a3b", [0, 17, 127]),
                                          ("mixtral_8x7b", [3])])
def test_codes_bit_exact(bm, name, experts):
    """Every decoder the kernels run, read back through the kernels' own
    operand builders, equals the oracle unpacker's codes bit for bit: every
    width group, every row of every segment (ragged dout on wide and heavy),
    all experts of the small layers."""
    L, dev = device_layer(name)
    spec = L.spec
    sel = list(range(spec.E)) if experts is None else experts
    for pj, (proj, blob) in enumerate((("gate", dev.blob_gate), ("up", dev.blob_up))):
        ref = fmt.unpack(dev.host_blobs[pj].tobytes(), experts=sel)
        codes = torch.empty((spec.r, spec.dout), dtype=torch.int16, device="cuda")
        for i, e in enumerate(sel):
            for path in (bm.DUMP_I8, bm.DUMP_F16, bm.DUMP_LANE):
                _say("codes %s %s e=%d path=%d" % (name, proj, e, path))
                bm.dump_codes(blob, spec.E, spec.dout, spec.r, e, codes, path=path)
                torch.cuda.synchronize()
                got = codes.cpu().numpy().view(np.uint16)
                want = _expected_operands(bm, ref["q"][i], ref["bits"][i], path)
                assert np.array_equal(got, want), (proj, e, path,
                                                   int(np.count_nonzero(got != want)))
    if name == "tiny":  # every width group, each one K32 step (a half int8 step)
        assert set(np.unique(L.bits["up"]).tolist()) == {0, 1, 2, 3, 4, 6, 8, 16}


def test_codes_match_oracle_quantizer(bm):
    """The device-decoded codes equal the oracle quantizer's codes."""
    from oracle.quantize import quantize_expert
    L, dev = device_layer("tiny")
    spec = L.spec
    codes = torch.empty((spec.r, spec.dout), dtype=torch.int16, device="cuda")
    for e in range(spec.E):
        bm.dump_codes(dev.blob_up, spec.E, spec.dout, spec.r, e, codes)
        torch.cuda.synchronize()
        q = quantize_expert(L.p["up"][e], L.bits["up"][e])["q"]
        q[L.bits["up"][e] == 0] = 0
        assert np.array_equal(codes.cpu().numpy().view(np.uint16), q)


# ------------------------------------------------------------- projection

@pytest.mark.parametrize("wl_name", ["tiny_t8", "qwen3_30b_a3b_t1", "qwen3_30b_a3b_t32"])
def test_spectral_proj(bm, wl_name):
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    x, _ = synth.make_batch(wl, L)
    T = x.shape[0]
    z = torch.empty((T, 2 * L.spec.r), dtype=torch.float32, device="cuda")
    bm.spectral_proj(dev.phi_t, _cuda(x), z)
    torch.cuda.synchronize()
    got = z.cpu().numpy()
    ref = z_ref(L, x)
    for t in range(T):
        zr = np.concatenate([ref["gate"][t], ref["up"][t]])
        assert max_rel_err(got[t], zr) <= Z_TOL, t


@pytest.mark.parametrize("wl_name,T", [("tiny_t64", 64), ("deepseek_moe_16b_t512", 100),
                                        ("deepseek_moe_16b_t512", 512)])
def test_spectral_proj_batched(bm, wl_name, T):
    """The tiled matrix-core projection (T >= 64): full and ragged token
    counts, against the oracle's z token by token."""
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    x, _ = synth.make_batch(wl, L)
    x = np.ascontiguousarray(x[:T])
    z = torch.empty((T, 2 * L.spec.r), dtype=torch.float32, device="cuda")
    bm.spectral_proj(dev.phi_t, _cuda(x), z)
    torch.cuda.synchronize()
    got = z.cpu().numpy()
    ref = z_ref(L, x)
    for t in range(T):
        zr = np.concatenate([ref["gate"][t], ref["up"][t]])
        assert max_rel_err(got[t], zr) <= Z_TOL, t


# ----------------------------------------------------------- expert apply

def test_expert_apply_tiny(bm):
    wl = synth.workload("tiny_t8")
    L, dev = device_layer("tiny")
    x, ids = synth.make_batch(wl, L)
    _, yg, yu = pairs_ref(L, x, ids, want_y=True)
    zr = z_ref(L, x)
    spec = L.spec
    for proj, blob, yref in (("gate", dev.blob_gate, yg), ("up", dev.blob_up, yu)):
        z = _cuda(zr[proj].astype(np.float32))
        y = torch.empty((x.shape[0], spec.k, spec.dout), dtype=torch.float32, device="cuda")
        bm.expert_apply(blob, spec.E, spec.dout, spec.r, z, _cuda(ids), y)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        for (t, s), ref in yref.items():
            assert max_rel_err(got[t, s], ref) <= Y_TOL, (proj, t, s)


def test_expert_apply_qwen_shape(bm):
    """bitsmoe_expert_apply alone (the lane-per-row kernel) on the Qwen3-shaped
    layer: 2 tokens x 8 experts, every row of each pair against the oracle."""
    wl = synth.workload("qwen3_30b_a3b_t1")
    L, dev = device_layer("qwen3_30b_a3b")
    x, ids = synth.make_batch(wl, L, T=2, step=7)
    _, yg, yu = pairs_ref(L, x, ids, want_y=True)
    zr = z_ref(L, x)
    spec = L.spec
    for proj, blob, yref in (("gate", dev.blob_gate, yg), ("up", dev.blob_up, yu)):
        z = _cuda(zr[proj].astype(np.float32))
        y = torch.empty((x.shape[0], spec.k, spec.dout), dtype=torch.float32, device="cuda")
        _say("expert apply qwen %s" % proj)
        bm.expert_apply(blob, spec.E, spec.dout, spec.r, z, _cuda(ids), y)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        for (t, s), ref in yref.items():
            assert max_rel_err(got[t, s], ref) <= Y_TOL, (proj, t, s)


@pytest.mark.parametrize("wl_name", ["beyond_t1", "beyond_t8"])
def test_gateup_beyond_matrix_core_limits(bm, wl_name):
    """r = din = 4112 (above 4096): neither the one-launch nor the grouped
    kernel takes the call; the projection and the lane-per-row expert kernel
    (k_expert_seg) do, for one token and for eight.  Every pair against the
    oracle, with one id outside [0, E) giving a NaN row."""
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    x, ids = synth.make_batch(wl, L)
    _say("beyond %s" % wl_name)
    got = _run_gateup(dev, x, ids)
    _check_h(got, pairs_ref(L, x, ids))
    bad = ids.copy()
    bad[0, 1] = L.spec.E
    got = _run_gateup(dev, x, bad)
    assert np.all(np.isnan(got[0, 1]))
    assert np.all(np.isfinite(got[0, 0]))


# ------------------------------------------------------------------ gate/up

def _check_h(got, href):
    worst = 0.0
    for (t, s), ref in href.items():
        err = max_rel_err(got[t, s], ref)
        worst = max(worst, err)
        assert err <= H_TOL, (t, s, err)
        assert np.all(np.isfinite(got[t, s]))
    return worst


@pytest.mark.parametrize("wl_name,steps", [("tiny_t1", 3), ("tiny_t4", 3), ("tiny_t8", 3),
                                           ("tiny_t64", 2), ("qwen3_30b_a3b_t1", 3),
                                           ("qwen3_30b_a3b_t4", 1), ("qwen3_30b_a3b_t32", 1),
                                           ("wide_t2", 2), ("wide_t8", 1), ("heavy_t1", 2)])
def test_gateup_full(bm, wl_name, steps):
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    for step in range(steps):
        x, ids = synth.make_batch(wl, L, step=step)
        _say("gateup %s step %d T=%d" % (wl_name, step, x.shape[0]))
        got = _run_gateup(dev, x, ids)
        worst = _check_h(got, pairs_ref(L, x, ids))
        _say("  worst %.3g" % worst)


def _sample_pairs(ids, n, seed):
    """n (token, slot) pairs: the first and last token, every slot of the
    most-routed expert's first token, the rest drawn at random."""
    T, K = ids.shape
    rng = np.random.default_rng(seed)
    vals, cnt = np.unique(ids, return_counts=True)
    top = int(vals[np.argmax(cnt)])
    tt, ss = np.nonzero(ids == top)
    pick = {(0, s) for s in range(K)} | {(T - 1, s) for s in range(K)}
    pick |= {(int(t), int(s_)) for t, s_ in zip(tt[:4], ss[:4])}
    while len(pick) < min(n, T * K):
        pick.add((int(rng.integers(T)), int(rng.integers(K))))
    return sorted(pick)


@pytest.mark.parametrize("wl_name,n_pairs", [("mixtral_8x7b_t1", 0), ("mixtral_8x7b_t8", 4),
                                             ("deepseek_moe_16b_t512", 48)])
def test_gateup_full_size_sampled(bm, wl_name, n_pairs):
    """The remaining full-size workloads in the launch configuration the
    benchmark times (the whole batch in one call); the oracle evaluates a
    sample of (token, slot) pairs (all of them when n_pairs is 0)."""
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    x, ids = synth.make_batch(wl, L, step=0)
    _say("gateup %s T=%d" % (wl_name, x.shape[0]))
    got = _run_gateup(dev, x, ids)
    assert np.all(np.isfinite(got))
    pairs = None if n_pairs == 0 else _sample_pairs(ids, n_pairs, seed=len(wl_name))
    _say("  oracle on %s pairs" % ("all" if pairs is None else len(pairs)))
    worst = _check_h(got, pairs_ref(L, x, ids, pairs=pairs))
    _say("  worst %.3g" % worst)


@pytest.mark.parametrize("wl_name", ["qwen3_30b_a3b_t1", "qwen3_30b_a3b_t32"])
def test_repeat_runs_bit_identical(bm, wl_name):
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    x, ids = synth.make_batch(wl, L)
    a = _run_gateup(dev, x, ids)
    b = _run_gateup(dev, x, ids)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("T", [4, 8])
def test_edges_zero_expert_k1_duplicates(bm, T):
    """All-0-bit expert gives h = 0; k = 1; the same expert on every token.

    T = 4 runs the one-launch kernel, T = 8 the two-launch path."""
    from spectral_expert_gemv_amd import DeviceLayer
    L = synth.make_layer(synth.LAYERS["tiny"])
    bits_g = L.bits["gate"].copy()
    bits_u = L.bits["up"].copy()
    bits_g[2] = 0
    bits_u[2] = 0
    dev = DeviceLayer(L.phi["gate"], L.phi["up"], L.a["gate"], L.a["up"], L.p["gate"],
                      L.p["up"], bits_g, bits_u)
    x, _ = synth.make_batch(synth.workload("tiny_t8"), L)
    x = x[:T]
    ids = np.full((T, 1), 2, np.int32)
    got = _run_gateup(dev, x, ids)
    assert np.all(got == 0)
    ids = np.array([[1], [1], [3], [1], [0], [3], [1], [1]], np.int32)[:T]
    got = _run_gateup(dev, x, ids)
    Lz = synth.generate.Layer(L.spec, L.phi, L.a, L.p, {"gate": bits_g, "up": bits_u},
                              L.outlier_channels)
    _check_h(got, pairs_ref(Lz, x, ids))


@pytest.mark.parametrize("T", [4, 8, 16])
def test_bad_expert_id_and_blob_mismatch_give_nan(bm, T):
    # T = 4: one launch; T = 8 and 16: the route work-group inside the row
    # and the matrix-core projection launch
    L, dev = device_layer("tiny")
    spec = L.spec
    wl = synth.workload("tiny_t8" if T <= 8 else "tiny_t64")
    x, ids = synth.make_batch(wl, L)
    x, ids = x[:T], ids[:T].copy()
    ids[3, 1] = spec.E          # out of range
    ids[T - 3, 0] = -1
    bad = ((3, 1), (T - 3, 0))
    got = _run_gateup(dev, x, ids)
    assert all(np.all(np.isnan(got[t, j])) for t, j in bad)
    ok = [(t, s) for t in range(T) for s in range(2) if (t, s) not in bad]
    _check_h(got, pairs_ref(L, x, ids, pairs=ok))
    # blobs whose header says a different dout than the call: every row NaN
    k = 2
    dout_call = spec.dout - 1
    h = torch.zeros((T, k, dout_call), dtype=torch.float32, device="cuda")
    ws = dev.workspace(T, k)
    good_ids = _cuda(synth.make_batch(wl, L)[1][:T])
    assert good_ids.shape == (T, k)
    bm._check(bm._lib.bitsmoe_moe_gateup(
        dev.blob_gate.data_ptr(), dev.blob_gate.numel(), dev.blob_up.data_ptr(),
        dev.blob_up.numel(), dev.phi_t.data_ptr(), _cuda(x).data_ptr(),
        good_ids.data_ptr(), T, k, spec.E, spec.din, dout_call, spec.r, h.data_ptr(),
        ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert torch.isnan(h).all()


@pytest.mark.parametrize("T", [8, 16])
def test_many_experts_separate_route_launch(bm, T):
    # more than 1024 experts: the pairs are grouped by their own launch (the
    # projection launches host the route work-group up to 1024 experts);
    # T = 8 follows the row projection, T = 16 the matrix-core one
    from spectral_expert_gemv_amd import DeviceLayer
    from synth.configs import LayerSpec, Workload
    spec = LayerSpec("many_experts", E=1040, din=64, dout=32, r=32, k=2, decay=0.5,
                     ln_sigma=0.3, bits="uniform", outlier_frac=0.0, outlier_scale=1.0,
                     phi_fp16=False)
    L = synth.make_layer(spec, cache=False)
    dev = DeviceLayer.from_synth(L)
    x, ids = synth.make_batch(Workload("many_experts_t16", spec, 16, ("uniform",)), L)
    x, ids = x[:T], ids[:T].copy()
    ids[1, 0] = spec.E + 5          # out of range
    got = _run_gateup(dev, x, ids)
    assert np.all(np.isnan(got[1, 0]))
    ok = [(t, s) for t in range(T) for s in range(2) if (t, s) != (1, 0)]
    _check_h(got, pairs_ref(L, x, ids, pairs=ok))


# ------------------------------------------------- workspace and waits

def _gateup_raw(bm, dev, x, ids, E, dout, h, ws):
    T, k = ids.shape
    bm._check(bm._lib.bitsmoe_moe_gateup(
        dev.blob_gate.data_ptr(), dev.blob_gate.numel(), dev.blob_up.data_ptr(),
        dev.blob_up.numel(), dev.phi_t.data_ptr(), x.data_ptr(), ids.data_ptr(), T, k, E,
        dev.din, dout, dev.r, h.data_ptr(), ws.data_ptr(), ws.numel(),
        torch.cuda.current_stream().cuda_stream))


def test_workspace_reused_across_token_counts(bm):
    """One workspace serves calls of different T in turn: T = 1 and T = 4
    (both on the one-launch kernel, with z rings of different sizes) alternate for 12 calls, more than the 8-buffer ring of tagged z, and every
    call matches the oracle on a sample of pairs."""
    L, dev = device_layer("qwen3_30b_a3b")
    spec = L.spec
    ws = dev.workspace(4, spec.k)  # sized for the larger T
    for call in range(12):
        T = 1 if call % 2 == 0 else 4
        wl = synth.workload("qwen3_30b_a3b_t1" if T == 1 else "qwen3_30b_a3b_t4")
        x, ids = synth.make_batch(wl, L, step=100 + call)
        _say("reuse call %d T=%d" % (call, T))
        h = dev.gateup(_cuda(x), _cuda(ids), ws=ws)
        torch.cuda.synchronize()
        got = h.cpu().numpy()
        assert np.all(np.isfinite(got)), call
        pairs = [(0, 0), (T - 1, spec.k - 1)]
        _check_h(got, pairs_ref(L, x, ids, pairs=pairs))


@pytest.mark.parametrize("wl_name", ["tiny_t1", "wide_t2", "tiny_t8"])
def test_blob_expert_count_mismatch_gives_nan(bm, wl_name):
    """A call that passes more experts than the blobs' headers hold: every
    directory record fails its check, every row is NaN and nothing is read
    outside the blobs (T = 1 and T = 2: the one-launch kernel; T = 8: the
    batched path)."""
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    spec = L.spec
    x, ids = synth.make_batch(wl, L)
    E_call = spec.E + 4
    assert dev.blob_gate.numel() >= 128 + 64 * E_call
    T, k = ids.shape
    h = torch.zeros((T, k, spec.dout), dtype=torch.float32, device="cuda")
    n = bm.moe_gateup_workspace_size(T, k, E_call, spec.din, spec.dout, spec.r)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    bm.workspace_init(ws)
    _gateup_raw(bm, dev, _cuda(x), _cuda(ids), E_call, spec.dout, h, ws)
    torch.cuda.synchronize()
    assert torch.isnan(h).all()


@pytest.mark.parametrize("wl_name", ["tiny_t1", "wide_t2"])
def test_wait_limit_zero_gives_nan_rows_then_recovers(bm, wl_name):
    """With the wait bound set to 0 by the host, every wait of the one-launch
    kernels gives up at once: the launch completes, every row is NaN and the
    workspace's time-out count grows.  With the bound restored, the next
    calls on the same workspace are exact again (the launch counter advanced
    normally) and add no time-out."""
    wl = synth.workload(wl_name)
    L, dev = device_layer(wl.layer.name)
    x, ids = synth.make_batch(wl, L)
    T, k = ids.shape
    ws = dev.workspace(T, k)
    t0 = bm.wait_timeouts(ws)
    prev = bm.debug_set_wait_limit(0)
    try:
        h = dev.gateup(_cuda(x), _cuda(ids), ws=ws)
        torch.cuda.synchronize()
        assert torch.isnan(h).all()
    finally:
        assert bm.debug_set_wait_limit(prev) == 0
    t1 = bm.wait_timeouts(ws)
    assert t1 > t0
    for _ in range(2):
        got = dev.gateup(_cuda(x), _cuda(ids), ws=ws)
        torch.cuda.synchronize()
        _check_h(got.cpu().numpy(), pairs_ref(L, x, ids))
    assert bm.wait_timeouts(ws) == t1
