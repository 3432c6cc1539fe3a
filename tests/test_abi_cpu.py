"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any
launch (no call here reaches the GPU)."""
import ctypes
import os
import re

import pytest

import learned_kv_cache_head_amd as kve

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvevict.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kve.library_path()),
                                reason="libkvevict.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kve_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kve_score", "kve_select_evict", "kve_compact",
                     "kve_decode_attn", "kve_step", "kve_append",
                     "kve_workspace_bytes", "kve_status_str"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kve.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_binding_covers_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(kve, name), f"binding lacks {name}"


def test_version_and_status_strings():
    assert kve.kve_version() >= 100
    assert kve.kve_status_str(0) == "ok"
    assert "policy" in kve.kve_status_str(2)
    assert kve.kve_status_str(99) == "unknown status"


def _lib():
    return kve.load_library()


def _shape(**kw):
    d = dict(batch=2, n_kv_heads=8, group=4, head_dim=128, capacity=1152,
             kv_dtype=kve.BF16)
    d.update(kw)
    return kve._Shape(**d)


FAKE = 0x10000  # never dereferenced: every call below fails validation


def _cache():
    return kve._Cache(FAKE, FAKE, FAKE, FAKE)


def test_workspace_bytes_host_math():
    s = _shape()
    n = _lib().kve_workspace_bytes(ctypes.byref(s), 1151)
    # 16 slices: split cap = min(ceil(4096 / 16), ceil(1151 / 64), 256) = 18
    # splits; per query head and split: 128 sums + max + normaliser, float32
    nsplit = 18
    partial = 2 * 32 * nsplit * 130 * 4
    assert n == (partial + 255) // 256 * 256
    # enough slices for one split per slice: one aligned block
    wide = _shape(batch=1024)
    assert _lib().kve_workspace_bytes(ctypes.byref(wide), 64) == 256
    # never decreases with max_len
    sizes = [_lib().kve_workspace_bytes(ctypes.byref(s), m)
             for m in range(1, 3000, 7)]
    assert sizes == sorted(sizes)
    bad = _shape(head_dim=96)
    assert _lib().kve_workspace_bytes(ctypes.byref(bad), 100) == 0
    assert _lib().kve_workspace_bytes(ctypes.byref(s), 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 4), (dict(group=9), 4), (dict(kv_dtype=7), 4),
    (dict(batch=0), 1), (dict(capacity=0), 1)])
def test_decode_attn_rejects_bad_shapes(kw, status):
    s, c = _shape(**kw), _cache()
    st = _lib().kve_decode_attn(ctypes.byref(s), ctypes.byref(c), 10, FAKE,
                                FAKE, None, FAKE, 1 << 20, None)
    assert st == status


def test_decode_attn_rejects_bad_len_and_workspace():
    s, c = _shape(), _cache()
    f = _lib().kve_decode_attn
    assert f(ctypes.byref(s), ctypes.byref(c), 0, FAKE, FAKE, None, FAKE,
             1 << 20, None) == 1
    assert f(ctypes.byref(s), ctypes.byref(c), 2000, FAKE, FAKE, None, FAKE,
             1 << 20, None) == 3
    assert f(ctypes.byref(s), ctypes.byref(c), 1000, FAKE, FAKE, None, FAKE,
             16, None) == 5
    assert f(ctypes.byref(s), ctypes.byref(c), 1000, FAKE, FAKE, None, None,
             1 << 20, None) == 5
    assert f(ctypes.byref(s), ctypes.byref(c), 1000, None, FAKE, None, FAKE,
             1 << 20, None) == 1


@pytest.mark.parametrize("pol,length,n_keep,status", [
    ((100, 60, 50, 8), 500, 100, 2),     # S + W > B
    ((100, 4, 8, 0), 500, 100, 2),       # L < 1
    ((100, 4, 8, 8), 500, 8, 2),         # n_keep < S + W while evicting
    ((100, 4, 8, 8), 500, 600, 2),       # n_keep > len
    ((100, 4, 8, 8), 2000, 100, 3),      # len > capacity
    ((100, -1, 8, 8), 500, 100, 2),
])
def test_select_rejects_bad_policy(pol, length, n_keep, status):
    s, c, p = _shape(), _cache(), kve._Policy(*pol)
    st = _lib().kve_select_evict(ctypes.byref(s), ctypes.byref(p),
                                 ctypes.byref(c), length, n_keep, FAKE, None)
    assert st == status


def test_compact_and_append_reject_bad_args():
    s, c = _shape(), _cache()
    lib = _lib()
    assert lib.kve_compact(ctypes.byref(s), ctypes.byref(c), 100, None, 50,
                           None) == 1
    assert lib.kve_compact(ctypes.byref(s), ctypes.byref(c), 100, FAKE, 200,
                           None) == 1
    assert lib.kve_compact(ctypes.byref(s), ctypes.byref(c), 5000, FAKE, 200,
                           None) == 3
    assert lib.kve_append(ctypes.byref(s), ctypes.byref(c), 1152, 0, FAKE,
                          FAKE, None) == 3
    assert lib.kve_append(ctypes.byref(s), ctypes.byref(c), 5, 0, None,
                          FAKE, None) == 1
    nullc = kve._Cache(FAKE, None, FAKE, FAKE)
    assert lib.kve_append(ctypes.byref(s), ctypes.byref(nullc), 5, 0, FAKE,
                          FAKE, None) == 1


def test_score_rejects_bad_scorers():
    s, c = _shape(), _cache()
    lib = _lib()
    mlp_bad_in = kve._Scorer(0, 0, kve.BF16, 128, 64, FAKE, None, FAKE, None)
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(mlp_bad_in),
                         ctypes.byref(c), 0, 10, None, None) == 4
    mlp_dtype = kve._Scorer(0, 0, kve.F32, 256, 64, FAKE, None, FAKE, None)
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(mlp_dtype),
                         ctypes.byref(c), 0, 10, None, None) == 4
    mlp = kve._Scorer(0, 0, kve.BF16, 256, 64, FAKE, None, FAKE, None)
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(mlp), ctypes.byref(c),
                         0, 10, FAKE, None) == 1   # hidden given to MLP
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(mlp), ctypes.byref(c),
                         5, 2, None, None) == 1
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(mlp), ctypes.byref(c),
                         0, 2000, None, None) == 3
    gate = kve._Scorer(1, 0, kve.BF16, 5120, 0, FAKE, None, None, None)
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(gate), ctypes.byref(c),
                         0, 10, None, None) == 1   # gate needs hidden
    gate_bad = kve._Scorer(1, 0, kve.BF16, 5000, 0, FAKE, None, None, None)
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(gate_bad),
                         ctypes.byref(c), 0, 10, FAKE, None) == 4


def test_step_rejects_bad_state():
    s, c = _shape(), _cache()
    lib = _lib()
    p = kve._Policy(1024, 4, 128, 128)
    mlp = kve._Scorer(0, 0, kve.BF16, 256, 64, FAKE, None, FAKE, None)

    def call(state, shape=s, pol=p, ws_bytes=1 << 24):
        return lib.kve_step(ctypes.byref(shape), ctypes.byref(pol),
                            ctypes.byref(mlp), ctypes.byref(c),
                            ctypes.byref(state), FAKE, FAKE, None, None, FAKE,
                            FAKE, None, FAKE, FAKE, ws_bytes, None)

    assert call(kve._State(1152, 1024, 9000, 0)) == 3       # cache full
    assert call(kve._State(1100, 1200, 9000, 0)) == 1       # scored > len
    assert call(kve._State(1100, 900, 9000, 0)) == 1        # pending >= L
    small = _shape(capacity=1100)
    assert call(kve._State(1000, 1000, 9000, 0), shape=small) == 3  # cap < B+L
    assert call(kve._State(1030, 1024, 9000, 0), ws_bytes=64) == 5


def test_shape_limits():
    """One slice's K rows must stay below 4 GiB (the kernels address a
    slice with 32-bit byte offsets) and batch * n_kv_heads below 2^31."""
    lib = _lib()
    ok = _shape(batch=1, n_kv_heads=1, capacity=(1 << 24) - 1)  # 256 B rows
    assert lib.kve_workspace_bytes(ctypes.byref(ok), 64) > 0
    big = _shape(batch=1, n_kv_heads=1, capacity=1 << 24)
    assert lib.kve_workspace_bytes(ctypes.byref(big), 64) == 0
    big32 = _shape(batch=1, n_kv_heads=1, capacity=1 << 23,
                   kv_dtype=kve.F32)                             # 512 B rows
    assert lib.kve_workspace_bytes(ctypes.byref(big32), 64) == 0
    s = lib.kve_decode_attn(ctypes.byref(big), ctypes.byref(_cache()), 10,
                            FAKE, FAKE, None, FAKE, 1 << 20, None)
    assert s == 4
    many = _shape(batch=65535, n_kv_heads=65535)
    assert lib.kve_workspace_bytes(ctypes.byref(many), 64) == 0


def test_step_checks_every_launch_before_the_first():
    """A step whose compaction grid cannot be launched (2.2M moved rows per
    slice need more than 65535 workgroups of 32 rows) fails with
    KVE_ERR_UNSUPPORTED before anything is enqueued: on this machine, with
    no GPU, an attempted launch would report KVE_ERR_LAUNCH instead. The
    decode state is left as it was."""
    lib = _lib()
    B = L = 2_200_000
    s = _shape(batch=1, n_kv_heads=1, group=1, head_dim=64,
               capacity=B + L)
    p = kve._Policy(B, 0, 0, L)
    mlp = kve._Scorer(0, 0, kve.BF16, 128, 32, FAKE, None, FAKE, None)
    state = kve._State(B + L - 1, B, 9_000_000, 7)
    st = lib.kve_step(ctypes.byref(s), ctypes.byref(p), ctypes.byref(mlp),
                      ctypes.byref(_cache()), ctypes.byref(state), FAKE, FAKE,
                      None, None, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert st == 4
    assert (state.len, state.scored_upto, state.next_position,
            state.evicted) == (B + L - 1, B, 9_000_000, 7)
    # a step one short of the eviction passes every check and reaches the
    # first launch, which fails here for want of a device
    state = kve._State(B + L - 3, B, 9_000_000, 7)
    st = lib.kve_step(ctypes.byref(s), ctypes.byref(p), ctypes.byref(mlp),
                      ctypes.byref(_cache()), ctypes.byref(state), FAKE, FAKE,
                      None, None, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert st == 6
    assert state.len == B + L - 3


def test_step_noalloc_validates_before_its_scratch():
    """kve_step_noalloc checks its arguments, then whether this step's
    split-K plan fits the scratch array (KVE_NOALLOC_SCRATCH_BYTES), before
    it looks up the array or launches anything. 272 slices of 8193 rows at
    G = 8 split 16 ways on 256 CUs: 272 * 8 * 16 * 130 * 4 bytes of
    partials, beyond 2 MiB."""
    lib = _lib()
    assert kve.NOALLOC_SCRATCH_BYTES == 2 << 20
    header = open(HEADER).read()
    assert "#define KVE_NOALLOC_SCRATCH_BYTES (2u << 20)" in header
    mlp = kve._Scorer(0, 0, kve.BF16, 256, 64, FAKE, None, FAKE, None)

    def call(shape, pol, state):
        return lib.kve_step_noalloc(
            ctypes.byref(shape), ctypes.byref(pol), ctypes.byref(mlp),
            ctypes.byref(_cache()), ctypes.byref(state), FAKE, FAKE, None,
            None, FAKE, FAKE, None, FAKE, None)

    big = _shape(batch=34, group=8, capacity=8256)
    pol = kve._Policy(8192, 4, 128, 64)
    state = kve._State(8192, 8192, 9000, 3)
    assert call(big, pol, state) == 5
    assert (state.len, state.scored_upto, state.evicted) == (8192, 8192, 3)
    # argument errors come first, as in kve_step
    assert call(big, pol, kve._State(8192, 9000, 9000, 0)) == 1
    assert call(_shape(capacity=1100), kve._Policy(1024, 4, 128, 128),
                kve._State(1000, 1000, 9000, 0)) == 3


def test_policy_struct_layout_matches_header():
    """kve_policy: four int32 fields, then the log_gamma and gumbel
    pointers."""
    assert ctypes.sizeof(kve._Policy) == 32
    assert kve._Policy.log_gamma.offset == 16
    assert kve._Policy.gumbel.offset == 24
    p = kve.Policy(1024, 4, 128, 128).c()
    assert p.log_gamma is None and p.gumbel is None


def test_cache_and_scorer_struct_layout_matches_header():
    """kve_cache: four pointers then scorer_state; kve_scorer: five int32,
    four pointers, then the int32 delay."""
    assert ctypes.sizeof(kve._Cache) == 40
    assert kve._Cache.scorer_state.offset == 32
    assert kve._Scorer.w1.offset == 24
    assert kve._Scorer.delay.offset == 56
    assert kve._Scorer.n_sink.offset == 60
    assert ctypes.sizeof(kve._Scorer) == 64


def _mlstm(delay=128, hidden=64, in_dim=256, wdtype=kve.BF16, w2=FAKE):
    return kve._Scorer(2, 0, wdtype, in_dim, hidden, FAKE, None, w2, None,
                       delay)


def test_mlstm_state_bytes():
    lib = _lib()
    s = _shape()            # batch 2, 8 KV heads, head_dim 128
    n = lib.kve_scorer_state_bytes(ctypes.byref(s), ctypes.byref(_mlstm()))
    # C [128][64] + z [128] + one 64-float block (log scale, count)
    assert n == 2 * 8 * (128 * 64 + 128 + 64) * 4
    s64 = _shape(head_dim=64)
    n64 = lib.kve_scorer_state_bytes(ctypes.byref(s64), ctypes.byref(
        _mlstm(hidden=32, in_dim=128)))
    assert n64 == 2 * 8 * (64 * 32 + 64 + 64) * 4
    mlp = kve._Scorer(0, 0, kve.BF16, 256, 64, FAKE, None, FAKE, None)
    assert lib.kve_scorer_state_bytes(ctypes.byref(s), ctypes.byref(mlp)) == 0
    assert lib.kve_scorer_state_bytes(ctypes.byref(s), ctypes.byref(
        _mlstm(hidden=32))) == 0   # P must be head_dim / 2


def test_mlstm_rejects_bad_arguments():
    lib = _lib()
    s = _shape()
    with_state = kve._Cache(FAKE, FAKE, FAKE, FAKE, FAKE)
    no_state = _cache()

    def score(sc, cache=with_state, shape=s, hidden=None):
        return lib.kve_score(ctypes.byref(shape), ctypes.byref(sc),
                             ctypes.byref(cache), 0, 10, hidden, None)

    assert score(_mlstm(), cache=no_state) == 1
    assert score(_mlstm(), hidden=FAKE) == 1
    assert score(_mlstm(hidden=32)) == 4
    assert score(_mlstm(in_dim=128)) == 4
    assert score(_mlstm(delay=-1)) == 1
    assert score(_mlstm(w2=None)) == 1
    assert score(_mlstm(), shape=_shape(kv_dtype=kve.F32)) == 4
    p = kve._Policy(1024, 4, 128, 128)

    def step(sc, cache=with_state):
        st = kve._State(1030, 1024, 9000, 0)
        return lib.kve_step(ctypes.byref(s), ctypes.byref(p), ctypes.byref(sc),
                            ctypes.byref(cache), ctypes.byref(st), FAKE, FAKE,
                            None, None, FAKE, FAKE, None, FAKE, FAKE, 1 << 24,
                            None)

    assert step(_mlstm(delay=64)) == 2          # delay != window
    assert step(_mlstm(), cache=no_state) == 1


def test_prefill_workspace_and_validation():
    lib = _lib()
    s = _shape(capacity=10000)
    n = lib.kve_prefill_workspace_bytes(ctypes.byref(s), 9000)
    assert n == 2 * 8 * 12288 * 8            # slices x chunk-rounded len x u64
    assert lib.kve_prefill_workspace_bytes(ctypes.byref(s), 0) == 0
    assert lib.kve_prefill_workspace_bytes(ctypes.byref(s), 262145) == 0
    c = _cache()
    p = kve._Policy(1024, 4, 128, 128)

    def sel(length, rank=FAKE, ws_bytes=1 << 30, shape=s):
        return lib.kve_prefill_select(ctypes.byref(shape), ctypes.byref(p),
                                      ctypes.byref(c), length, rank, FAKE,
                                      FAKE, ws_bytes, None)

    assert sel(0) == 1
    assert sel(10001) == 3
    assert sel(100, rank=None) == 1
    assert sel(9000, ws_bytes=1000) == 5
    big = _shape(capacity=300000)
    assert sel(262145, shape=big) == 4

    def attn(length, shape=s, q=FAKE, ws_bytes=1 << 30):
        return lib.kve_prefill_attn(ctypes.byref(shape), ctypes.byref(p),
                                    ctypes.byref(c), length, FAKE, FAKE, q,
                                    FAKE, None, FAKE, ws_bytes, None)

    assert attn(0) == 1
    assert attn(10001) == 3
    assert attn(100, q=None) == 1
    assert attn(100, shape=_shape(capacity=10000, kv_dtype=kve.F32)) == 4
    assert attn(9000, ws_bytes=100) == 5
    # key lists: k = 892 ints per 64-position query block and slice, then
    # one count and one V maximum per block, then V in float16 (d = 128)
    wsb = lib.kve_prefill_attn_workspace_bytes(ctypes.byref(s), ctypes.byref(p),
                                               9000)
    nqb = (9000 + 63) // 64
    lists = 2 * 8 * nqb * 892 * 4
    blocks = 2 * (2 * 8 * nqb * 4)
    assert wsb == ((lists + 255) // 256 * 256 + (blocks + 255) // 256 * 256 +
                   2 * 8 * 9000 * 128 * 2)
    # stochastic eviction noise: the prefill ranks are deterministic only
    p.gumbel = FAKE
    assert sel(100) == 4
    assert attn(100) == 4


def test_sink_gate_rejects_bad_scorers():
    lib = _lib()
    s, c = _shape(), _cache()

    def score(hidden_dim=5120, hid=16, n_sink=16, w2=FAKE, hidden=FAKE):
        sc = kve._Scorer(3, 0, kve.BF16, hidden_dim, hid, FAKE, None, w2, None,
                         0, n_sink)
        return lib.kve_score(ctypes.byref(s), ctypes.byref(sc),
                             ctypes.byref(c), 0, 10, hidden, None)

    assert score(hidden=None) == 1      # hidden states required
    assert score(hid=8) == 4            # D' must be 16
    assert score(n_sink=17) == 4
    assert score(hidden_dim=5000) == 4
    assert score(w2=None) == 1          # sink keys missing


class _FakeDev:
    """Stands in for a device tensor in the binding's buffer checks."""

    def __init__(self, nbytes, contiguous=True, cuda=True):
        self.nbytes, self.contig, self.is_cuda = nbytes, contiguous, cuda

    def is_contiguous(self):
        return self.contig

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1

    def data_ptr(self):
        return FAKE


def test_binding_refuses_host_small_or_strided_buffers():
    """The C ABI sees bare pointers, so the binding checks every device
    buffer's size, placement and contiguity before a call."""
    import torch
    s = kve.Shape(2, 8, 4, 128, 1152, kve.BF16)
    rows = 2 * 8 * 1152
    good = kve.CacheTensors(_FakeDev(rows * 256), _FakeDev(rows * 256),
                            _FakeDev(rows * 4), _FakeDev(rows * 4))
    kve._check_cache(s, good)
    for bad in (kve.CacheTensors(_FakeDev(rows * 256 - 1), _FakeDev(rows * 256),
                                 _FakeDev(rows * 4), _FakeDev(rows * 4)),
                kve.CacheTensors(_FakeDev(rows * 256), _FakeDev(rows * 256),
                                 _FakeDev(rows * 4, contiguous=False),
                                 _FakeDev(rows * 4)),
                kve.CacheTensors(torch.zeros(rows * 128, dtype=torch.bfloat16),
                                 _FakeDev(rows * 256), _FakeDev(rows * 4),
                                 _FakeDev(rows * 4))):
        with pytest.raises(ValueError):
            kve._check_cache(s, bad)
    pol = kve.Policy(1024, 4, 128, 128, gumbel=_FakeDev(rows * 4 - 4))
    with pytest.raises(ValueError):
        kve._check_policy(s, pol)
    kve._check_policy(s, kve.Policy(1024, 4, 128, 128,
                                    gumbel=_FakeDev(rows * 4)))
    # keep_slots of a select needs batch * H * n_keep int32
    with pytest.raises(ValueError):
        kve.kve_select_evict(s, kve.Policy(1024, 4, 128, 128), good, 1152,
                             1024, _FakeDev(2 * 8 * 1024 * 4 - 1))
    # scorer weights: MLP w1 [H][hidden][2d] bf16
    sc = kve.Scorer(kve.SCORER_MLP_KV, _FakeDev(8 * 64 * 256 * 2 - 2),
                    w2=_FakeDev(8 * 64 * 4), hidden=64, in_dim=256,
                    wdtype=kve.BF16)
    with pytest.raises(ValueError):
        kve._check_scorer(s, sc)


def test_one_library_per_process(tmp_path):
    """Every call goes to the one loaded build; a second build is refused
    (two copies of the device code in one process fail to launch)."""
    lib = _lib()
    assert kve.load_library() is lib
    assert kve.load_library(kve.library_path()) is lib
    with pytest.raises(RuntimeError, match="already loaded"):
        kve.load_library(str(tmp_path / "libkvevict.so"))


def test_library_shares_torchs_hip_runtime():
    """Loaded before anything imports torch, the library still ends up with
    the one HIP runtime torch uses: a fresh process that loads it first and
    then uses torch maps a single libamdhip64."""
    import subprocess
    import sys
    code = (
        "import learned_kv_cache_head_amd as kve\n"
        "kve.load_library()\n"
        "import torch\n"
        "torch.zeros(1)\n"
        "maps = open('/proc/self/maps').read().split('\\n')\n"
        "paths = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
        "print(len(paths), sorted(paths))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    n = int(out.stdout.split()[0])
    assert n == 1, out.stdout


def test_misaligned_pointers_are_rejected():
    """Rows move with 16-byte vector accesses: a misaligned row buffer (or a
    float32 / int32 array off its 4-byte grid) is an argument error, reported
    before any launch."""
    lib, s = _lib(), _shape()
    att = lib.kve_decode_attn
    good = _cache()
    assert att(ctypes.byref(s), ctypes.byref(good), 1000, FAKE + 8, FAKE,
               None, FAKE, 1 << 20, None) == 1                 # q
    assert att(ctypes.byref(s), ctypes.byref(good), 1000, FAKE, FAKE + 4,
               None, FAKE, 1 << 20, None) == 1                 # out
    assert att(ctypes.byref(s), ctypes.byref(good), 1000, FAKE, FAKE,
               FAKE + 2, FAKE, 1 << 20, None) == 1             # lse
    assert att(ctypes.byref(s), ctypes.byref(good), 1000, FAKE, FAKE,
               None, FAKE + 8, 1 << 20, None) == 1             # workspace
    for c in (kve._Cache(FAKE + 8, FAKE, FAKE, FAKE),
              kve._Cache(FAKE, FAKE + 2, FAKE, FAKE),
              kve._Cache(FAKE, FAKE, FAKE + 2, FAKE),
              kve._Cache(FAKE, FAKE, FAKE, FAKE + 1)):
        assert att(ctypes.byref(s), ctypes.byref(c), 1000, FAKE, FAKE, None,
                   FAKE, 1 << 20, None) == 1
    p = kve._Policy(1024, 4, 128, 128)
    assert lib.kve_select_evict(ctypes.byref(s), ctypes.byref(p),
                                ctypes.byref(good), 1152, 1024, FAKE + 2,
                                None) == 1
    assert lib.kve_compact(ctypes.byref(s), ctypes.byref(good), 1152,
                           FAKE + 2, 1024, None) == 1
    assert lib.kve_append(ctypes.byref(s), ctypes.byref(good), 5, 5, FAKE + 8,
                          FAKE, None) == 1
    sc = kve._Scorer(kve.SCORER_MLP_KV, 0, kve.BF16, 256, 64, FAKE + 8, None,
                     FAKE, None, 0, 0)
    assert lib.kve_score(ctypes.byref(s), ctypes.byref(sc), ctypes.byref(good),
                         0, 10, None, None) == 1


def test_bench_library_exports_and_rejects_bad_arguments():
    """libkvebench.so (the benchmark's read ceiling and issue probe) exports
    its three calls, and each rejects bad arguments on the host, before any
    launch."""
    import torch  # noqa: F401  (the library binds torch's HIP runtime)
    path = os.path.join(os.path.dirname(kve.__file__), "_lib", "libkvebench.so")
    lib = ctypes.CDLL(path)
    for name in ("kvebench_read", "kvebench_read_blocks", "kvebench_issue"):
        assert hasattr(lib, name), name
    lib.kvebench_read.restype = ctypes.c_int
    lib.kvebench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.kvebench_read_blocks.restype = ctypes.c_size_t
    lib.kvebench_read_blocks.argtypes = [ctypes.c_size_t]
    lib.kvebench_issue.restype = ctypes.c_int
    lib.kvebench_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    # one workgroup streams 1 MiB
    assert lib.kvebench_read_blocks(1 << 20) == 1
    assert lib.kvebench_read_blocks((1 << 20) + 16) == 2
    assert lib.kvebench_read(None, 1 << 20, FAKE, None) == 1
    assert lib.kvebench_read(FAKE, 24, FAKE, None) == 1        # not 16-byte sized
    assert lib.kvebench_read(FAKE + 8, 64, FAKE, None) == 1    # misaligned
    for mode in (0, 4, 6, 7, 8, 9, 12, 14, 15, 16):            # no such mode
        assert lib.kvebench_issue(mode, 1, 1, FAKE, None) == 1
    assert lib.kvebench_issue(1, 0, 1, FAKE, None) == 1
    assert lib.kvebench_issue(1, 1, 0, FAKE, None) == 1
    assert lib.kvebench_issue(1, 1, 1, None, None) == 1
