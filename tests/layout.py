"""Test-side reading and writing of the library's K page layout (numpy / torch index maps).

A K page holds the 16 keys of one kv head in 16-byte units: unit (row r, x) holds elements
x*U .. x*U+U-1 of key row r (U = 8 for bf16, 4 for fp32) and sits at unit slot
16*x + (r + 4*(lp % 2) + 4*((x // 8) % 2)) % 16 of the page, lp being the page's logical index in
its sequence.
V pages are [d][row] (the transposed page) and need no map.  Written for the tests only,
independently of the library and of the oracle.
"""
import numpy as np

BS = 16


def unit_elems(dtype: str) -> int:
    return 8 if dtype == "bf16" else 4


def k_page_index(D: int, unit: int, parity: int) -> np.ndarray:
    """[16, D] element offsets inside a K page of logical parity `parity` for (row, d)."""
    r = np.arange(BS)[:, None]
    d = np.arange(D)[None, :]
    x = d // unit
    return x * (BS * unit) + ((r + 4 * parity + 4 * ((x // 8) % 2)) % BS) * unit + d % unit


def page_rows(page_flat: np.ndarray, D: int, unit: int, parity: int) -> np.ndarray:
    """The 16 logical rows [16, D] of one stored K page (flat, 16*D elements)."""
    return page_flat[k_page_index(D, unit, parity)]


def logical_k(kc, block_table, lens, unit: int):
    """Logical K rows of every page the block table uses: a copy of kc ([nb, Hkv, 16, D],
    numpy or torch) where page (blk, g) is re-ordered to [row][d]; unused pages are left as
    stored."""
    nb, Hkv, bs, D = kc.shape
    out = kc.clone() if hasattr(kc, "clone") else kc.copy()
    for par in (0, 1):
        idx = k_page_index(D, unit, par).reshape(-1)
        blks = sorted({int(block_table[b, p]) for b in range(len(lens))
                       for p in range(-(-int(lens[b]) // bs)) if p % 2 == par})
        if not blks:
            continue
        if hasattr(kc, "clone"):
            import torch
            bi = torch.tensor(blks, dtype=torch.long, device=kc.device)
            ii = torch.from_numpy(idx).to(kc.device)
            flat = kc.index_select(0, bi).reshape(len(blks), Hkv, bs * D)
            out[bi] = flat.index_select(2, ii).reshape(len(blks), Hkv, bs, D)
        else:
            flat = kc[blks].reshape(len(blks), Hkv, bs * D)
            out[blks] = flat[:, :, idx].reshape(len(blks), Hkv, bs, D)
    return out


def put_k_rows(kc: np.ndarray, blk: np.ndarray, g: int, pos: np.ndarray, rows: np.ndarray,
               unit: int) -> None:
    """kc[nb, Hkv, 16, D] (numpy): store key rows rows[i] (D elements) of positions pos[i]
    into page blk[i], kv head g."""
    nb, Hkv, bs, D = kc.shape
    flat = kc.reshape(nb, Hkv, bs * D)
    for par in (0, 1):
        sel = (pos // bs) % 2 == par
        if not sel.any():
            continue
        idx = k_page_index(D, unit, par)
        flat[blk[sel][:, None], g, idx[pos[sel] % bs]] = rows[sel]
