"""Index maps of the library's physical chunk layouts (pure numpy)."""
import numpy as np


def chunk_index_maps(kv: str, p: int, D: int) -> dict:
    """Positions, inside one chunk of the library's physical layout
    (include/pkv.h), of each logical element: "k"[t, d] and "v"[d, t] are
    element (16-bit) or byte indices; for INT4 they are the bit offsets of
    the code's nibble in the chunk (byte offset // 8, shift offset % 8);
    "m"[t, group] indexes 32-bit INT4 metadata words."""
    NT, NG = D // 16, D // 32
    tt = np.arange(p)
    hf, g_t, r, jt = tt // 16, (tt % 16) // 4, tt % 4, tt % 16
    d = np.arange(D)
    T, j = d // 16, d % 16
    c, g_d, e = d // 32, (d % 32) // 8, d % 8
    if kv in ("f16", "bf16"):
        return {"k": tt[:, None] * D + d[None, :],
                "v": ((((hf[None, :] * (NT // 2) + T[:, None] // 2) * 16 + j[:, None]) * 4
                       + g_t[None, :]) * 2 + T[:, None] % 2) * 4 + r[None, :]}
    if kv in ("fp8_e4m3", "fp8_e5m2", "fp8_e4m3_block"):
        return {"k": ((((hf[:, None] * (D // 64) + c[None, :] // 2) * 16 + jt[:, None]) * 4
                       + g_d[None, :]) * 16 + 8 * (c[None, :] % 2) + e[None, :]),
                "v": ((((hf[None, :] * (NT // 4) + T[:, None] // 4) * 16 + j[:, None]) * 4
                       + g_t[None, :]) * 16 + (T[:, None] % 4) * 4 + r[None, :])}
    kbyte = (tt[:, None] * (D // 2) + g_d[None, :] * (D // 8) + 4 * c[None, :]
             + e[None, :] // 2)
    # V: one 32-bit word per (unit, j, g, group of two 16-channel tiles); the
    # nibble of token 4 g + r of tile parity T % 2 sits at bit
    # 16 (r % 2) + 8 (r / 2) + 4 (T % 2)
    vword = ((hf[None, :] * 16 + j[:, None]) * 4 + g_t[None, :]) * NG + T[:, None] // 2
    vbit = 16 * (r[None, :] % 2) + 8 * (r[None, :] // 2) + 4 * (T[:, None] % 2)
    return {"k": 8 * kbyte + 4 * (e[None, :] % 2),
            "v": 32 * vword + vbit,
            "m": ((hf[:, None] * 4 + g_t[:, None]) * NG + np.arange(NG)[None, :]) * 4
            + r[:, None]}


def logical_pools(kv: str, p: int, D: int, nb: int, H: int, raw: dict) -> dict:
    """Map the library's physical chunk layouts to the logical layouts the
    oracle keeps: K [block][head][token][channel], V [block][head][channel]
    [token], INT4 two codes per byte (even index in the low nibble), metadata
    [block][head][token](...).  Every map is a bijection inside a chunk, so
    canary bytes map to canary bytes."""
    mp = chunk_index_maps(kv, p, D)
    out = {"k_meta": None, "v_meta": None}
    if kv in ("f16", "bf16"):
        k = raw["k_pool"].view(np.uint16).reshape(nb, H, p * D)
        v = raw["v_pool"].view(np.uint16).reshape(nb, H, p * D)
        out["k_pool"], out["v_pool"] = k[:, :, mp["k"]], v[:, :, mp["v"]]
    elif kv in ("fp8_e4m3", "fp8_e5m2", "fp8_e4m3_block"):
        k = raw["k_pool"].reshape(nb, H, p * D)
        v = raw["v_pool"].reshape(nb, H, p * D)
        out["k_pool"], out["v_pool"] = k[:, :, mp["k"]], v[:, :, mp["v"]]
        out["k_meta"] = raw["k_meta"].view(np.float32).reshape(nb, H, p)
        out["v_meta"] = raw["v_meta"].view(np.float32).reshape(nb, H, p)
    else:
        k = raw["k_pool"].reshape(nb, H, p * D // 2)
        v = raw["v_pool"].reshape(nb, H, p * D // 2)
        kc = (k[:, :, mp["k"] // 8] >> (mp["k"] % 8).astype(np.uint8)) & 0xF  # [.., p, D]
        vc = (v[:, :, mp["v"] // 8] >> (mp["v"] % 8).astype(np.uint8)) & 0xF  # [.., D, p]
        out["k_pool"] = kc[..., 0::2] | (kc[..., 1::2] << 4)
        out["v_pool"] = vc[..., 0::2] | (vc[..., 1::2] << 4)
        for name in ("k_meta", "v_meta"):
            m = raw[name].view(np.uint32).reshape(nb, H, -1)[:, :, mp["m"]]
            out[name] = np.ascontiguousarray(m).view(np.uint16).reshape(nb, H, p, D // 32, 2)
    return {k_: (None if a is None else np.ascontiguousarray(a)) for k_, a in out.items()}
