"""Errors of every GPU-vs-oracle comparison in a test session, summarised at
the end of the run (pytest's terminal summary, see conftest.py)."""
RECORDS = []


def record(test, name, kind, rows, max_abs_o, rel_rms_o, max_abs_lse):
    RECORDS.append(dict(test=test, name=name, kind=kind, rows=rows, max_abs_o=float(max_abs_o),
                        rel_rms_o=float(rel_rms_o), max_abs_lse=float(max_abs_lse)))


def summary_lines():
    if not RECORDS:
        return []
    out = ["parity against the oracle, worst case per input type "
           "(max |dO|, relative RMS of O, max |dLSE|; comparisons / rows compared):"]
    for kind in sorted({r["kind"] for r in RECORDS}):
        rs = [r for r in RECORDS if r["kind"] == kind]
        wo = max(rs, key=lambda r: r["max_abs_o"])
        wr = max(rs, key=lambda r: r["rel_rms_o"])
        wl = max(rs, key=lambda r: r["max_abs_lse"])
        out.append(f"  {kind:5s} {len(rs):4d} comparisons, {sum(r['rows'] for r in rs)} rows: "
                   f"max|dO| {wo['max_abs_o']:.3e} ({wo['name']}), relRMS(O) {wr['rel_rms_o']:.3e} "
                   f"({wr['name']}), max|dLSE| {wl['max_abs_lse']:.3e} ({wl['name']})")
    return out
