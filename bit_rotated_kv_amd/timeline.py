"""Per-workgroup timeline of the decode kernels, from the diagnostic library liboscar_timeline.so
(the product library with timestamps written by thread 0 of each workgroup; see csrc/timeline.hpp
for the table layout). Call use_timeline_library() before the first library call of the process."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _lib

TIMELINE_LIB = os.path.join(_lib.HERE, "liboscar_timeline.so")
SPLIT_ROWS, MERGE_ROWS, COLS = 16384, 2048, 8
TICK_US = 0.01           # s_memrealtime counts at 100 MHz
ROLES = {0: "int2_history", 1: "int4_history", 2: "window", 3: "step"}


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
    return [round(float(v), 2) for v in np.percentile(x, [10, 50, 90])]


def summarize(tabs) -> dict:
    """p10/p50/p90 (microseconds) of each phase over the workgroups of several recorded launches;
    times are relative to the first workgroup entry of the launch's split kernel."""
    acc = {}
    spans, merge_spans, ends = [], [], []
    n_split = n_merge = 0
    for tab in tabs:
        sp = tab[:SPLIT_ROWS]
        used = np.nonzero(sp[:, 0])[0]
        if used.size == 0:
            continue
        n_split = max(n_split, int(used.max()) + 1)
        t0 = sp[used, 0].min()
        rel = lambda c: (sp[used, c].astype(np.int64) - np.int64(t0)) * TICK_US
        entry, ready, loop, exit_ = rel(0), rel(1), rel(2), rel(3)
        role = (sp[used, 4] & 0xFF).astype(int)
        pages = (sp[used, 4] >> 8).astype(int)
        xcc = (sp[used, 5] >> 32).astype(int) & 0xF
        spans.append(float(exit_.max()))
        for r, name in ROLES.items():
            m = role == r
            if not m.any():
                continue
            d = acc.setdefault(name, {"entry": [], "exit": [], "run": []})
            d["entry"] += list(entry[m])
            d["exit"] += list(exit_[m])
            d["run"] += list(exit_[m] - entry[m])
            if r in (0, 1):
                d.setdefault("prologue", []).extend(list(ready[m] - entry[m]))
                d.setdefault("page_loop", []).extend(list(loop[m] - ready[m]))
                d.setdefault("wg_merge", []).extend(list(exit_[m] - loop[m]))
                d.setdefault("pages_wave0", []).extend(list(pages[m]))
        hist = role <= 1
        if hist.any():
            ends.append({int(x): round(float(exit_[hist & (xcc == x)].max()), 2) for x in np.unique(xcc[hist])})
        mg = tab[SPLIT_ROWS:]
        mu = np.nonzero(mg[:, 0])[0]
        if mu.size:
            n_merge = max(n_merge, int(mu.max()) + 1)
            me = (mg[mu, 0].astype(np.int64) - np.int64(t0)) * TICK_US
            mx = (mg[mu, 3].astype(np.int64) - np.int64(t0)) * TICK_US
            merge_spans.append((float(me.min()), float(mx.max())))
            acc.setdefault("merge", {"entry": [], "exit": [], "run": []})
            acc["merge"]["entry"] += list(me)
            acc["merge"]["exit"] += list(mx)
            acc["merge"]["run"] += list(mx - me)
    out = {"launches": len(spans), "split_workgroups": n_split, "merge_workgroups": n_merge,
           "split_span_us": _pct(spans),
           "merge_entry_exit_us": [round(float(np.median([m[0] for m in merge_spans])), 2),
                                   round(float(np.median([m[1] for m in merge_spans])), 2)] if merge_spans else None,
           "last_history_exit_per_xcd_us": ends[-1] if ends else None, "roles": {}}
    for name, d in acc.items():
        out["roles"][name] = {k: _pct(v) for k, v in d.items()}
        out["roles"][name]["workgroups_per_launch"] = len(d["entry"]) // max(1, len(spans))
    return out
