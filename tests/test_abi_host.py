"""CPU tests of the C ABI: the library loads, exports every function the header
declares, validates arguments, and plans routing (admission under max_loras,
per-token slots, segments) exactly as the oracle and the pages say."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def m():
    import adapter_deltas_amd
    return adapter_deltas_amd


def header_define(name):
    return int(re.search(rf"#define\s+{name}\s+(\d+)", open(HEADER).read()).group(1))


GATHER_MIN_RANK = header_define("LORA_GATHER_MIN_RANK")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(m):
    from adapter_deltas_amd import _lib
    names = header_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.EXPORTS) == names
    # constants and the info struct mirrored by the binding
    assert _lib.GATHER_MIN_RANK == GATHER_MIN_RANK
    assert _lib.SEG_WORDS == 16 and _lib.DECODE_SEG_ROWS == header_define("LORA_DECODE_SEG_ROWS")
    text = open(HEADER).read()
    body = re.search(r"typedef struct lora_routing_info \{(.*?)\}", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert [n for n, _ in _lib.RoutingInfo._fields_] == fields


def test_validation_errors_without_device(m):
    with pytest.raises(m.LoraError) as e:
        m.lora_pool_bytes(m.make_desc(100, [64], 4, 8))
    assert e.value.status == "LORA_ERR_SHAPE"
    with pytest.raises(m.LoraError) as e:
        m.lora_pool_bytes(m.make_desc(64, [60], 4, 8))
    assert e.value.status == "LORA_ERR_SHAPE"
    with pytest.raises(m.LoraError) as e:
        m.lora_pool_bytes(m.make_desc(64, [64], 4, 300))
    assert e.value.status == "LORA_ERR_RANK"
    d = m.make_desc(64, [64], 4, 8)
    d.x_dtype = 3
    with pytest.raises(m.LoraError) as e:
        m.lora_pool_bytes(d)
    assert e.value.status == "LORA_ERR_DTYPE"
    with pytest.raises(m.LoraError) as e:
        m.lora_routing_bytes(0)
    assert e.value.status == "LORA_ERR_SHAPE"
    # pool creation with too little memory fails before touching the device
    with pytest.raises(m.LoraError) as e:
        m.lora_pool_create(m.make_desc(64, [64], 4, 8), 256, 16, stream=0)
    assert e.value.status == "LORA_ERR_CAPACITY"
    assert "needed" in m.lora_last_error()
    # null handles are refused before any device work
    for call in (lambda: m.lora_build_routing_device(None, 0, 0, None, stream=0),
                 lambda: m.lora_build_routing_moe(None, 0, 0, 0, 0, 0, 1, None, stream=0),
                 lambda: m.lora_routing_device_counts(None),
                 lambda: m.lora_pool_load_folded(None, 1, -1, [0], [64], 0, [0], [8], [4],
                                                 [1.0], 0, 64, stream=0)):
        with pytest.raises(m.LoraError) as e:
            call()
        assert e.value.status == "LORA_ERR_ARG"


def test_moe_slot_layout(m):
    """The pair of (adapter slot a, expert e) sits in slot (a - 1) * E + e + 1:
    an adapter's experts are consecutive slots and the map is one to one."""
    E, A = 6, 4
    slots = [m.moe_slot(a, e, E) for a in range(1, A + 1) for e in range(E)]
    assert slots == list(range(1, A * E + 1))
    assert m.moe_slot(1, 0, E) == 1 and m.moe_slot(A, E - 1, E) == A * E


def test_moe_slot_matches_the_header_macro(m, tmp_path):
    """moe_slot and moe_row_slots of the binding give what LORA_MOE_SLOT in
    include/lora.h gives, for several expert counts (a C program built with
    gcc from the header prints the macro's values)."""
    import subprocess
    cases = [(a, e, n) for n in (1, 3, 8, 128) for a in (1, 2, 5) for e in range(min(n, 4))]
    prog = tmp_path / "moe_slot.c"
    body = "".join(f'    printf("%d\\n", LORA_MOE_SLOT({a}, {e}, {n}));\n' for a, e, n in cases)
    prog.write_text('#include <stdio.h>\n#include "lora.h"\nint main(void)\n{\n' + body +
                    "    return 0;\n}\n")
    exe = tmp_path / "moe_slot"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)],
                   check=True)
    want = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert [m.moe_slot(a, e, n) for a, e, n in cases] == want
    # the per-row form: base tokens and unedited experts give 0
    tok_slot = np.array([0, 2, 5], np.int32)
    row_token = np.array([1, 0, 2, 1, 2], np.int32)
    row_expert = np.array([3, 1, 0, 7, 2], np.int32)
    edited = np.array([True, True, True, False, True])
    got = m.moe_row_slots(tok_slot, row_token, row_expert, 8, edited)
    assert got.tolist() == [m.moe_slot(2, 3, 8), 0, m.moe_slot(5, 0, 8), 0, m.moe_slot(5, 2, 8)]


def test_missing_id_is_the_base_model(m):
    """A sequence whose adapter id is None runs the base model, as id 0 does
    (tokenspeed PR #976, first commit message): the same plan, and it never
    counts against max_loras."""
    resident = {5: 1, 6: 2}
    a = m.lora_plan_routing([5, None, 6, None], [1, 3, 2, 1], 1, 64, resident, 4, 16)
    b = m.lora_plan_routing([5, 0, 6, 0], [1, 3, 2, 1], 1, 64, resident, 4, 16)
    for k in ("seg", "rows", "tok_slot", "admitted"):
        assert np.array_equal(a[k], b[k]), k
    assert a["info"] == b["info"]
    assert list(a["admitted"]) == [True, True, False, True]
    assert a["tok_slot"].tolist() == [1, 0, 0, 0, 0, 0, 0]


def test_pool_bytes_layout(m):
    # A + B^T + B + two metadata tables, each 256-byte aligned
    d = m.make_desc(4096, [4096, 1024, 1024], 8, 16)
    a = 8 * 3 * 16 * 4096 * 2
    b = 8 * 16 * 6144 * 2
    meta = 9 * 4 * 4
    rnd = lambda n: -(-n // 256) * 256
    assert m.lora_pool_bytes(d) == rnd(a) + 2 * rnd(b) + 2 * rnd(meta)


def test_plan_admission_matches_golden_and_oracle(m):
    with open(os.path.join(GOLDEN, "admission_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ids = c["ids"]
        resident = {i: k + 1 for k, i in enumerate(sorted(set(ids) - {0}))}
        p = m.lora_plan_routing(ids, [1] * len(ids), c["max_loras"], 64, resident,
                                max(len(resident), 1), max(len(ids), 1))
        assert list(p["admitted"]) == c["admitted"], c["name"]
        assert p["info"]["n_distinct"] == len(c["distinct"])


def _check_plan(p, ids, lens, resident, cap, pmin, ranks=None):
    adm, _ = oracle.admit(ids, cap)
    assert list(p["admitted"]) == adm
    tok = oracle.token_adapters(ids, lens, adm)
    slots = np.array([resident.get(int(a), 0) for a in tok], dtype=np.int32)
    assert np.array_equal(p["tok_slot"], slots)
    seg, rows = p["seg"], p["rows"]
    info = p["info"]
    assert info["n_tokens"] == int(np.sum(lens))
    assert info["n_active"] == int((slots != 0).sum()) == len(rows)
    # every active row appears exactly once, in a segment of its own slot
    assert sorted(rows.tolist()) == np.nonzero(slots)[0].tolist()
    seq_of = np.repeat(np.arange(len(lens)), lens)
    # an adapter's decode rows take gather segments iff one of its slice ranks
    # reaches the gather threshold (a property of the adapter alone)
    inv = {sl: i for i, sl in resident.items()}
    big = {sl: max((ranks or {}).get(inv[sl], [0])) >= GATHER_MIN_RANK for sl in inv}
    n_dec, n_pre = info["n_decode_segments"], info["n_prefill_segments"]
    assert info["n_segments"] == n_dec + n_pre + info["n_gather_segments"] == len(seg)
    covered = 0
    for k, d in enumerate(seg):
        s, b, n, kind = d[:4]
        assert s >= 1 and n >= 1
        assert b == covered
        covered += n
        r = rows[b:b + n]
        assert np.all(slots[r] == s)
        L = np.asarray(lens)[seq_of[r]]
        if kind == 0:
            assert k < n_dec and n <= 8 and not big[s]
            assert np.all(L < pmin)
            assert np.all(np.diff(r) > 0)
            assert list(d[8:8 + n]) == list(r) and np.all(d[8 + n:] == r[-1])
        elif kind == 1:
            assert n_dec <= k < n_dec + n_pre and n <= 64
            assert np.all(L >= pmin)
            assert np.all(np.diff(r) == 1) and len(set(seq_of[r])) == 1
            assert d[8] == r[0]
            start = r[0] - np.concatenate([[0], np.cumsum(lens)])[seq_of[r[0]]]
            assert start % 64 == 0     # chunking depends only on the sequence
        else:
            assert kind == 2 and k >= n_dec + n_pre and n <= 64 and big[s]
            assert np.all(L < pmin)
            assert np.all(np.diff(r) > 0)
            assert np.all(d[8:] == 0)
    assert covered == len(rows)
    # decode rows of one slot sit in consecutive segments, token order inside
    for part, full in ((seg[:n_dec], 8), (seg[n_dec + n_pre:], 64)):
        for s in set(part[:, 0].tolist()):
            ks = np.nonzero(part[:, 0] == s)[0]
            assert np.all(np.diff(ks) == 1)
            r = np.concatenate([rows[d[1]:d[1] + d[2]] for d in part[ks]])
            assert np.all(np.diff(r) > 0)
            assert np.all(part[ks][:-1, 2] == full)


@pytest.mark.parametrize("seed", range(12))
def test_plan_random_batches(m, seed):
    rng = np.random.default_rng(seed)
    n_ad = int(rng.integers(1, 12))
    ids_pool = (np.arange(n_ad) * 13 + 5).tolist()
    resident = {i: int(s) for i, s in zip(ids_pool, rng.permutation(40)[:n_ad] + 1)}
    n_seq = int(rng.integers(0, 60))
    ids = [0 if rng.random() < 0.3 else int(rng.choice(ids_pool)) for _ in range(n_seq)]
    lens = rng.choice([0, 1, 1, 1, 2, 5, 63, 64, 65, 130], size=n_seq).tolist()
    cap = int(rng.integers(0, n_ad + 1))
    pmin = int(rng.choice([1, 16, 64, 2**31 - 1]))
    T = max(int(np.sum(lens)), 1)
    ranks = {i: [int(x) for x in rng.integers(1, 100, size=4)] for i in ids_pool}
    p = m.lora_plan_routing(ids, lens, cap, pmin, resident, 40, T, resident_rank=ranks)
    _check_plan(p, ids, lens, resident, cap, pmin, ranks)
    _check_mfma_tables(p)
    inv_slot = {s: i for i, s in resident.items()}
    _check_row_meta(p, lambda s: ranks[inv_slot[s]])
    inv = {s: i for i, s in resident.items()}
    for d in p["seg"]:
        assert list(d[4:8]) == ranks[inv[d[0]]]


N_CU = 256          # the device size the host-only plans assume


XCDS = 8
NONE = 0xFFFFFFFF     # an empty place of a task table


def _live(words):
    return words[words != NONE]


def _check_row_meta(p, slot_ranks):
    """Row metadata: active row m holds its slot and the slot's four ranks
    (slot_ranks(slot) -> 4 ranks)."""
    meta = p["row_meta"]
    rows = p["rows"]
    assert meta.shape == (len(rows), 4)
    for m, t in enumerate(rows):
        s = int(p["tok_slot"][t])
        r = slot_ranks(s)
        assert list(meta[m]) == [s, (r[0] & 0xffff) | (r[1] << 16),
                                 (r[2] & 0xffff) | (r[3] << 16), 0], m


def _check_mfma_tables(p):
    """Every table covers each prefill/gather segment's 16-rank tiles of its
    first s slices exactly once, in tasks of 1..4 consecutive tiles, has at
    least 128 tasks, keeps a segment's tasks in one XCD residue class (word
    b runs on XCD b % 8), heaviest (rows + 16 * tiles) first in each class,
    and gives no class more than an equal share of the units (or of the
    tasks) by more than one segment's tasks."""
    seg = p["seg"]
    first = p["info"]["n_decode_segments"]
    rest = seg[first:]
    for s, table in p["mfma_tasks"].items():
        words = _live(table)
        assert 1 <= s <= 4 and len(words) >= 128 and len(table) % XCDS == 0
        si = (words & 0xFFFFFF).astype(np.int64)
        c0 = ((words >> 24) & 63).astype(np.int64)
        cnt = ((words >> 30) + 1).astype(np.int64)
        assert np.all(si < len(rest))
        tiles = ((rest[:, 4:4 + s] + 15) // 16).sum(axis=1)
        cover = [np.zeros(t, np.int64) for t in tiles]
        for a, b, k in zip(si, c0, cnt):
            assert b + k <= tiles[a]
            cover[a][b:b + k] += 1
        assert all(np.all(c == 1) for c in cover)
        home = {}
        room = max(-(-len(words) // XCDS), N_CU // XCDS)
        most = np.bincount(si).max()        # tasks of one segment: the packing grain
        for x in range(XCDS):
            col = table[x::XCDS]
            live = col != NONE
            assert np.all(live[:live.sum()])            # empty places only at the end
            w = col[live]
            cost = np.minimum(rest[w & 0xFFFFFF, 2], 64) + 16 * ((w >> 30) + 1)
            assert np.all(np.diff(cost) <= 0)
            for a in (w & 0xFFFFFF):
                assert home.setdefault(int(a), x) == x
            assert len(w) <= room + most - 1


def test_mfma_task_tables_balance_the_units(m):
    """Prefill chunks of 6 adapters (ranks 8, 8, 16, 16, 64, 64, two slices):
    fewer whole-segment tasks than compute units, so the heavy segments are
    cut until the largest task is as small as 256 tasks allow."""
    resident = {5 + i: i + 1 for i in range(6)}
    ranks = {5 + i: [r, r, 0, 0] for i, r in enumerate((8, 8, 16, 16, 64, 64))}
    lens = [604, 1925, 1047, 409, 1479, 965, 598, 1283]
    ids = [5 + i for i in (5, 0, 2, 4, 1, 3, 0, 5)]
    p = m.lora_plan_routing(ids, lens, 0, 64, resident, 8, sum(lens), resident_rank=ranks)
    _check_mfma_tables(p)
    assert sorted(p["mfma_tasks"]) == [1, 2]
    rest = p["seg"][p["info"]["n_decode_segments"]:]
    for s, table in p["mfma_tasks"].items():
        words = _live(table)
        cnt = (words >> 30) + 1
        cost = np.minimum(rest[words & 0xFFFFFF, 2], 64) + 16 * cnt
        assert len(words) <= N_CU
        # no cut into smaller pieces would still fit the units
        tiles = ((rest[:, 4:4 + s] + 15) // 16)
        tiles = tiles.sum(axis=1)
        rows = np.minimum(rest[:, 2], 64)
        c = int(cost.max()) - 1
        kmax = np.minimum((c - rows) // 16, 4)
        assert np.any(kmax < 1) or np.sum(-(-tiles // np.maximum(kmax, 1))) > N_CU
    def cost(table):
        words = _live(table)
        return np.minimum(rest[words & 0xFFFFFF, 2], 64) + 16 * ((words >> 30) + 1)

    # one slice: 98 light and 38 heavy segments; a full segment and one tile
    # a task fits (at most 250 tasks)
    assert cost(p["mfma_tasks"][1]).max() == 64 + 16
    # two slices: one tile a task would not (500); two do, and a light
    # segment's task takes its tile of both slices, reading its x rows once
    w2 = _live(p["mfma_tasks"][2])
    assert cost(w2).max() == 64 + 32
    for i in np.nonzero(rest[:, 4] <= 16)[0]:
        mine = w2[(w2 & 0xFFFFFF) == i]
        assert len(mine) == 1 and (mine[0] >> 30) + 1 == 2


def test_mfma_task_tables_small_and_many(m):
    """A small batch has no table (its tasks are cut by rows instead); many
    small gather groups get one task per segment covering both slices."""
    resident = {5: 1}
    p = m.lora_plan_routing([5], [300], 0, 64, resident, 4, 300, resident_rank={5: [16, 16, 0, 0]})
    assert p["mfma_tasks"] == {}
    slot_rank = np.zeros((301, 4), np.int32)
    slot_rank[1:, :2] = 16
    row_slot = np.repeat(np.arange(1, 301), 12).astype(np.int32)
    p = m.lora_plan_rows(row_slot, np.ones(len(row_slot), np.uint8), 300, slot_rank, len(row_slot))
    _check_mfma_tables(p)
    assert len(_live(p["mfma_tasks"][2])) == len(_live(p["mfma_tasks"][1])) == 300


def test_plan_errors(m):
    with pytest.raises(m.LoraError) as e:
        m.lora_plan_routing([5, 6], [1, 1], 0, 64, {5: 1}, 4, 4)
    assert e.value.status == "LORA_ERR_UNKNOWN_ADAPTER"
    with pytest.raises(m.LoraError) as e:
        m.lora_plan_routing([5], [9], 0, 64, {5: 1}, 4, 4)
    assert e.value.status == "LORA_ERR_CAPACITY"
    with pytest.raises(m.LoraError) as e:
        m.lora_plan_routing([5], [-1], 0, 64, {5: 1}, 4, 4)
    assert e.value.status == "LORA_ERR_SHAPE"
    with pytest.raises(m.LoraError) as e:
        m.lora_plan_routing([5], [1], 0, 64, {5: 9}, 4, 4)
    assert e.value.status == "LORA_ERR_SLOT"
    # an unknown id that the cap defers is never looked up
    p = m.lora_plan_routing([5, 6], [1, 1], 1, 64, {5: 1}, 4, 4)
    assert list(p["admitted"]) == [True, False]


# ------------------------------------------------ plans from per-row slots

def _check_rows_plan(p, row_slot, row_prefill, slot_rank):
    """Structure of a plan from per-row slots (MoE dispatched rows)."""
    info, seg, rows = p["info"], p["seg"], p["rows"]
    slots = np.asarray(row_slot)
    pre = np.zeros(len(slots), bool) if row_prefill is None else np.asarray(row_prefill, bool)
    assert np.array_equal(p["tok_slot"], slots)
    assert info["n_tokens"] == len(slots) and info["n_prefill_segments"] == 0
    assert info["n_active"] == int((slots != 0).sum()) == len(rows)
    assert sorted(rows.tolist()) == np.nonzero(slots)[0].tolist()
    big = slot_rank.max(axis=1) >= GATHER_MIN_RANK
    gathered = (slots != 0) & (pre | big[slots])
    n_dec = info["n_decode_segments"]
    assert info["n_segments"] == n_dec + info["n_gather_segments"] == len(seg)
    # gather segments: 16 rows when gathered rows average at most 16 per slot
    g_slots = set(slots[gathered].tolist())
    size = 16 if gathered.sum() <= 16 * len(g_slots) else 64
    covered = 0
    for k, d in enumerate(seg):
        s, b, n, kind = d[:4]
        assert b == covered and n >= 1
        covered += n
        r = rows[b:b + n]
        assert np.all(slots[r] == s) and np.all(np.diff(r) > 0)
        assert list(d[4:8]) == list(slot_rank[s])
        if kind == 0:
            assert k < n_dec and n <= 8 and not np.any(gathered[r])
            assert list(d[8:8 + n]) == list(r) and np.all(d[8 + n:] == r[-1])
        else:
            assert kind == 2 and k >= n_dec and n <= size and np.all(gathered[r])
            assert np.all(d[8:] == 0)
    assert covered == len(rows)
    # a slot's rows of one path sit in consecutive segments, full but the last
    for part, full in ((seg[:n_dec], 8), (seg[n_dec:], size)):
        for s in set(part[:, 0].tolist()):
            ks = np.nonzero(part[:, 0] == s)[0]
            assert np.all(np.diff(ks) == 1)
            assert np.all(part[ks][:-1, 2] == full)


@pytest.mark.parametrize("seed", range(10))
def test_plan_rows_random(m, seed):
    rng = np.random.default_rng(100 + seed)
    max_slots = int(rng.integers(1, 40))
    slot_rank = np.zeros((max_slots + 1, 4), np.int32)
    held = rng.random(max_slots + 1) < 0.8
    held[0] = False
    for s in np.nonzero(held)[0]:
        slot_rank[s, :int(rng.integers(1, 5))] = rng.choice([1, 4, 16, 64, 128, 130])
    live = np.nonzero(held)[0]
    n = int(rng.integers(0, 3000)) if seed else 0
    row_slot = np.where(rng.random(n) < 0.2, 0, rng.choice(live, n) if len(live) else 0)
    row_slot = row_slot.astype(np.int32)
    row_prefill = (rng.random(n) < [0.0, 0.5, 1.0][seed % 3]) if seed % 4 else None
    p = m.lora_plan_rows(row_slot, row_prefill, max_slots, slot_rank, max(n, 1))
    _check_rows_plan(p, row_slot, row_prefill, slot_rank)
    _check_mfma_tables(p)
    _check_row_meta(p, lambda s: [int(v) for v in slot_rank[s]])


def test_plan_rows_cuts_small_groups_at_16(m):
    """Many small groups: 16-row gather segments; one big group: 64."""
    slot_rank = np.zeros((9, 4), np.int32)
    slot_rank[1:, 0] = 16
    small = np.repeat(np.arange(1, 9), 12).astype(np.int32)          # 12 rows per slot
    p = m.lora_plan_rows(small, np.ones(len(small), np.uint8), 8, slot_rank, len(small))
    assert p["info"]["n_gather_segments"] == 8 and p["seg"][:, 2].max() == 12
    big = np.full(100, 3, np.int32)
    p = m.lora_plan_rows(big, np.ones(100, np.uint8), 8, slot_rank, 100)
    assert list(p["seg"][:, 2]) == [64, 36]
    mixed = np.concatenate([np.full(40, 2), np.full(8, 5)]).astype(np.int32)   # 24 per slot
    p = m.lora_plan_rows(mixed, np.ones(len(mixed), np.uint8), 8, slot_rank, len(mixed))
    assert list(p["seg"][:, 2]) == [40, 8]


def test_plan_rows_errors(m):
    slot_rank = np.zeros((5, 4), np.int32)
    slot_rank[1:3, 0] = 8
    for bad in (3, 5, -1):                       # empty, out of range, negative
        with pytest.raises(m.LoraError) as e:
            m.lora_plan_rows(np.array([1, bad], np.int32), None, 4, slot_rank, 4)
        assert e.value.status == "LORA_ERR_SLOT"
    with pytest.raises(m.LoraError) as e:
        m.lora_plan_rows(np.array([1, 2], np.int32), None, 0, np.zeros((1, 4), np.int32), 4)
    assert e.value.status == "LORA_ERR_SHAPE"
