"""Per-workgroup timeline of the decode kernels, from the diagnostic library liboscar_timeline.so
(the product library with timestamps written by thread 0 of each workgroup; see csrc/timeline.hpp
for the table layout). Call use_timeline_library() before the first library call of the process."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _lib

TIMELINE_LIB = os.path.join(_lib.HERE, "liboscar_timeline.so")
SPLIT_ROWS, MERGE_ROWS, COLS = 16384, 2048, 16
TICK_US = 0.01           # s_memrealtime counts at 100 MHz


def use_timeline_library():
    """Point the binding at liboscar_timeline.so (raises if it is missing or another library is
    already loaded)."""
    if _lib._lib is not None and _lib.LIB_PATH != TIMELINE_LIB:
        raise RuntimeError("the product library is already loaded in this process")
    if not os.path.exists(TIMELINE_LIB):
        raise RuntimeError(f"{TIMELINE_LIB} is missing: build it with `python -m bit_rotated_kv_amd.build`")
    _lib.LIB_PATH = TIMELINE_LIB
    l = _lib.lib()
    l.oscar_timeline_read.restype = ctypes.c_int
    l.oscar_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    l.oscar_timeline_clear.restype = ctypes.c_int
    l.oscar_timeline_clear.argtypes = []


def clear():
    if _lib.lib().oscar_timeline_clear() != 0:
        raise RuntimeError("oscar_timeline_clear failed")


def read() -> np.ndarray:
    tab = np.zeros((SPLIT_ROWS + MERGE_ROWS, COLS), np.uint64)
    if _lib.lib().oscar_timeline_read(tab.ctypes.data, tab.nbytes) != 0:
        raise RuntimeError("oscar_timeline_read failed")
    return tab


def _pct(x):
    x = np.asarray(x, np.float64)
    if x.size == 0:
        return None
    return [round(float(v), 2) for v in np.percentile(x, [10, 50, 90])] + [round(float(x.max()), 2)]


def summarize(tabs) -> dict:
    """p10/p50/p90 and the maximum (microseconds) of each phase over the workgroups of several recorded launches;
    times are relative to the first workgroup entry of the launch's split kernel. Workgroups are
    grouped by the segments they ran: "first_unit" (the step and/or window pages, then history) and
    "history" (history pages only)."""
    acc = {}
    spans, merge_spans, ends = [], [], []
    n_split = n_merge = 0
    for tab in tabs:
        sp = tab[:SPLIT_ROWS]
        used = np.nonzero(sp[:, 0])[0]
        if used.size == 0:
            continue
        n_split = max(n_split, int(used.max()) + 1)
        t0 = np.int64(sp[used, 0].min())
        col = lambda c: sp[used, c].astype(np.int64)
        rel = lambda c: (col(c) - t0) * TICK_US
        dur = lambda c1, c0: (col(c1) - col(c0)) * TICK_US
        segs = (col(6) & 0xFF).astype(int)
        pages = (col(6) >> 8).astype(int)
        xcc = (col(7) >> 32).astype(int) & 0xF
        hist = (segs & 12) != 0
        exit_ = rel(5)
        spans.append(float(exit_.max()))
        groups = {"first_unit": (segs & 3) != 0, "history": (segs & 3) == 0}
        for name, m in groups.items():
            if not m.any():
                continue
            d = acc.setdefault(name, {})
            d.setdefault("entry", []).extend(rel(0)[m])
            d.setdefault("exit", []).extend(exit_[m])
            d.setdefault("run", []).extend(dur(5, 0)[m])
            d.setdefault("plan", []).extend(dur(1, 0)[m])
            d.setdefault("step_window", []).extend(dur(2, 1)[m])
            st = m & ((segs & 1) != 0)
            d.setdefault("step_loads", []).extend(dur(9, 1)[st])
            d.setdefault("step_rotate", []).extend(dur(10, 9)[st])
            d.setdefault("step_quantize_store", []).extend(dur(11, 10)[st])
            d.setdefault("step_partials", []).extend(dur(2, 11)[st])
            h = m & hist
            d.setdefault("prologue", []).extend(dur(3, 2)[h])
            d.setdefault("page_loop", []).extend(dur(4, 3)[h])
            d.setdefault("wave_wait", []).extend(dur(8, 4)[h])
            d.setdefault("wg_merge", []).extend(dur(5, 8)[h])
            d.setdefault("wg_state_to_lds", []).extend(dur(12, 8)[h])
            d.setdefault("wg_barrier", []).extend(dur(13, 12)[h])
            d.setdefault("wg_reduce_store", []).extend(dur(14, 13)[h])
            d.setdefault("wg_to_exit", []).extend(dur(5, 14)[h])
            d.setdefault("history_pages", []).extend(pages[h])
            # history units of the interleaved one-request launch (column 9 set): the prologue in parts
            il = h & (col(9) != 0) & ((segs & 3) == 0)
            if il.any():
                # the first page loads go out after the wavefront's query products (11, then 9)
                d.setdefault("il_query_products", []).extend(dur(11, 0)[il])
                d.setdefault("il_first_loads", []).extend(dur(9, 11)[il])
                d.setdefault("il_query_barrier", []).extend(dur(15, 9)[il])
                d.setdefault("il_query_head_pass", []).extend(dur(3, 15)[il])
                d.setdefault("il_first_pair", []).extend(dur(10, 3)[il])
                d.setdefault("il_loop_rest", []).extend(dur(4, 10)[il])
            d["count"] = d.get("count", 0) + int(m.sum())
        ends.append({int(x): round(float(exit_[xcc == x].max()), 2) for x in np.unique(xcc)})
        mg = tab[SPLIT_ROWS:]
        mu = np.nonzero(mg[:, 0])[0]
        if mu.size:
            n_merge = max(n_merge, int(mu.max()) + 1)
            me = (mg[mu, 0].astype(np.int64) - t0) * TICK_US
            mf = (mg[mu, 1].astype(np.int64) - t0) * TICK_US
            mc = (mg[mu, 3].astype(np.int64) - t0) * TICK_US
            mx = (mg[mu, 5].astype(np.int64) - t0) * TICK_US
            merge_spans.append((float(me.min()), float(mx.max())))
            d = acc.setdefault("merge", {})
            d.setdefault("entry", []).extend(me)
            d.setdefault("exit", []).extend(mx)
            d.setdefault("run", []).extend(mx - me)
            d.setdefault("fold", []).extend(mf - me)
            d.setdefault("combine", []).extend(mc - mf)
            d.setdefault("unrotate_store", []).extend(mx - mc)
            d["count"] = d.get("count", 0) + int(mu.size)
    out = {"launches": len(spans), "split_workgroups": n_split, "merge_workgroups": n_merge,
           "split_span_us": _pct(spans),
           "merge_entry_exit_us": [round(float(np.median([m[0] for m in merge_spans])), 2),
                                   round(float(np.median([m[1] for m in merge_spans])), 2)] if merge_spans else None,
           "last_exit_per_xcd_us": ends[-1] if ends else None, "groups": {}}
    for name, d in acc.items():
        cnt = d.pop("count")
        out["groups"][name] = {k: _pct(v) for k, v in d.items()}
        out["groups"][name]["workgroups_per_launch"] = cnt // max(1, len(spans))
    return out
