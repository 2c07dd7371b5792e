"""Host-side check of the LDS tile layout of the bf16 attention kernels
(video_diffusion_transformer_qk_amd/csrc/attention.hip: SwzLayout, TileDma, rows_begin, rows_tile).

The formulas are restated here from the kernel source and checked for the properties the kernels
rely on, for D = 64 and 128:
  * the direct loads of one K/V tile fill every LDS slot once and bring every logical 16-byte
    chunk of the 64 rows exactly once;
  * every K fragment read (ds_read_b128) and every V transpose read (ds_read_b64_tr_b16) finds the
    logical chunk it asks for, on the row it asks for;
  * no read instruction puts two lanes on the same bank, whether the LDS serves 256 bytes (64
    banks) or 128 bytes (32 banks) per cycle;
  * the per-lane byte offsets of the loads stay non-negative and below 2^31 at the largest head
    count the library accepts, also in the tile that holds the last token.
A wrong rotation is caught: rotating V rows by 4r (D = 128) or leaving K rows unrotated puts lanes
on the same banks. The padded tiles of the fp8 kernels (attention_fp8.hip) are checked the same
way: every staged chunk read back where the MFMA operands expect it, no bank conflicts."""
import pytest

TILE_ROWS = 64
WAVES = 8  # 512 threads per workgroup


def layout(D, vrot_factor=2, rotate_k=True):
    row_bytes, cpr = 2 * D, D // 8
    if D == 128:
        krot = (lambda r: r) if rotate_k else (lambda r: 0)
        vrot = lambda r: vrot_factor * r
    else:
        krot = lambda r: r ^ ((r >> 3) & 1)
        vrot = lambda r: 2 * ((r & 3) ^ ((r >> 2) & 1))
    return dict(
        row=row_bytes, cpr=cpr,
        kcol=lambda r, c: (c + krot(r)) & (cpr - 1),
        vcol=lambda r, c: (c + vrot(r)) & (cpr - 1),
        kchunk=lambda r, col: (col - krot(r)) & (cpr - 1),
        vchunk=lambda r, col: (col - vrot(r)) & (cpr - 1),
    )


def loader_slots(L):
    """(row, column, logical K chunk, logical V chunk) of every slot the direct loads fill."""
    J = L["cpr"] // WAVES
    out = []
    for w in range(WAVES):
        for j in range(J):
            for lane in range(64):
                p = 64 * (J * w + j) + lane
                r, col = divmod(p, L["cpr"])
                out.append((p, r, col, L["kchunk"](r, col), L["vchunk"](r, col)))
    return out


def k_reads(L, D):
    """LDS byte addresses of the K fragment reads, one list of 64 lanes per instruction."""
    for kt in range(4):
        for ks in range(D // 32):
            addrs = []
            for lane in range(64):
                i16, g = lane & 15, lane >> 4
                koff = i16 * L["row"] + L["kcol"](i16, 4 * ks + g) * 16
                addrs.append((16 * kt * L["row"] + koff, 16 * kt + i16, 4 * ks + g))
            yield addrs


def v_reads(L, D):
    """LDS byte addresses of the V transpose reads (8 bytes per lane), one list per instruction."""
    for ks2 in range(2):
        for h in range(2):
            for dt in range(D // 16):
                addrs = []
                for lane in range(64):
                    i16, g = lane & 15, lane >> 4
                    r = 4 * g + (i16 >> 2)
                    byte = 32 * dt + 8 * (i16 & 3)
                    voff = r * L["row"] + L["vcol"](r, byte // 16) * 16 + byte % 16
                    addrs.append((32 * ks2 * L["row"] + voff + (16 * L["row"] if h else 0),
                                  32 * ks2 + 16 * h + r, byte))
                yield addrs


def conflicts(addrs, lanes_per_cycle, cycle_bytes, access_bytes):
    n = 0
    for s in range(0, 64, lanes_per_cycle):
        slots = [(a % cycle_bytes) // access_bytes for a in addrs[s:s + lanes_per_cycle]]
        n += len(slots) - len(set(slots))
    return n


@pytest.mark.parametrize("D", [64, 128])
def test_direct_loads_fill_every_slot_with_every_chunk_once(D):
    L = layout(D)
    slots = loader_slots(L)
    assert sorted(p for p, *_ in slots) == list(range(TILE_ROWS * L["cpr"]))
    assert len({(r, kc) for _, r, _, kc, _ in slots}) == TILE_ROWS * L["cpr"]
    assert len({(r, vc) for _, r, _, _, vc in slots}) == TILE_ROWS * L["cpr"]
    for p, r, col, _, _ in slots:  # a wave instruction writes 1 KB of consecutive LDS bytes
        assert r * L["row"] + col * 16 == 16 * p


@pytest.mark.parametrize("D", [64, 128])
def test_fragment_reads_find_their_chunks(D):
    L = layout(D)
    for addrs in k_reads(L, D):
        for a, row, chunk in addrs:
            r, rem = divmod(a, L["row"])
            assert r == row and rem % 16 == 0 and L["kchunk"](r, rem // 16) == chunk
    for addrs in v_reads(L, D):
        for a, row, byte in addrs:
            r, rem = divmod(a, L["row"])
            assert r == row and L["vchunk"](r, rem // 16) == byte // 16 and rem % 16 == byte % 16


@pytest.mark.parametrize("D", [64, 128])
def test_reads_are_free_of_bank_conflicts(D):
    L = layout(D)
    for addrs in k_reads(L, D):
        a = [x for x, _, _ in addrs]
        assert conflicts(a, 16, 256, 16) == 0 and conflicts(a, 8, 128, 16) == 0
    for addrs in v_reads(L, D):
        a = [x for x, _, _ in addrs]
        assert conflicts(a, 32, 256, 8) == 0 and conflicts(a, 16, 128, 8) == 0


def test_wrong_rotations_conflict():
    L = layout(128, vrot_factor=4)
    assert sum(conflicts([x for x, _, _ in addrs], 16, 128, 8) for addrs in v_reads(L, 128)) > 0
    L = layout(128, rotate_k=False)
    assert sum(conflicts([x for x, _, _ in addrs], 16, 256, 16) for addrs in k_reads(L, 128)) > 0


@pytest.mark.parametrize("D", [64, 128])
def test_load_offsets_fit_32_bits(D):
    L = layout(D)
    heads = 65535  # the largest head count the library accepts
    rs_bytes = 2 * heads * D
    for _, r, col, kc, vc in loader_slots(L):
        koff = r * rs_bytes + 16 * kc
        assert 0 <= koff < 2 ** 31 and 0 <= r * rs_bytes + 16 * vc < 2 ** 31
        for last in range(TILE_ROWS):  # the tile that holds the last token: rows clamped to it
            adj = 0 if r < last else (last - r) * rs_bytes
            assert koff + adj == min(r, last) * rs_bytes + 16 * kc >= 0


# fp8 kernels (attention_fp8.hip: Fp8Tile, Fp8Stage::stash, fp8_qk, fp8_soft_pv): padded rows,
# K rows of D + 16 bytes and V^T rows of 64 + 16 bytes, written by 16-byte stores and read as two
# 16-byte halves of each lane's 32-byte MFMA operand.
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_tiles_round_trip_and_reads_are_conflict_free(D):
    KS, VS = D + 16, 64 + 16
    k_store = {ci: ((ci // (D // 16)) * KS + (ci % (D // 16)) * 16) for ci in range(64 * D // 16)}
    v_store = {ci: ((ci >> 2) * VS + (ci & 3) * 16) for ci in range(D * 64 // 16)}
    assert len(set(k_store.values())) == len(k_store) and len(set(v_store.values())) == len(v_store)
    k_chunk_at = {a: (ci // (D // 16), ci % (D // 16)) for ci, a in k_store.items()}  # (key, chunk)
    v_chunk_at = {a: (ci >> 2, ci & 3) for ci, a in v_store.items()}                  # (channel, chunk)
    for m in range(2):
        for ks in range(D // 64):
            for half in (0, 16):
                addrs = [(32 * m + (l & 31)) * KS + 64 * ks + 32 * (l >> 5) + half for l in range(64)]
                for l, a in enumerate(addrs):
                    assert k_chunk_at[a] == (32 * m + (l & 31), (64 * ks + 32 * (l >> 5) + half) // 16)
                assert conflicts(addrs, 16, 256, 16) == 0 and conflicts(addrs, 8, 128, 16) == 0
    for dt in range(D // 32):
        for half in (0, 16):
            addrs = [(32 * dt + (l & 31)) * VS + 32 * (l >> 5) + half for l in range(64)]
            for l, a in enumerate(addrs):
                assert v_chunk_at[a] == (32 * dt + (l & 31), (32 * (l >> 5) + half) // 16)
            assert conflicts(addrs, 16, 256, 16) == 0 and conflicts(addrs, 8, 128, 16) == 0
