"""Markdown tables from the parity report that the GPU tests append to
$LAYA_REPORT_DIR/parity_report.jsonl (per-layer and end-to-end nRMS of the
whole-pass tests against the CPU oracle).

    python tests/report_table.py <dir>/parity_report.jsonl > table.md
"""
import json
import sys

CONFIGS = ["short_1", "short_3", "long_3", "mixed_16", "marker_subset"]


def main(path):
    recs = [json.loads(line) for line in open(path)]
    work = {}
    for r in recs:
        if r.get("test") == "workload":
            work[r["workload"]] = r
    names = CONFIGS + sorted(k for k in work if k not in CONFIGS)
    names = [n for n in names if n in work]
    print("## Per layer: each oracle layer fed the GPU's input to it (nRMS, limit 0.005)\n")
    layers = list(work[names[0]]["per_layer_nrms"])
    print("| Layer | " + " | ".join(names) + " |")
    print("|---|" + "---|" * len(names))
    for lay in layers:
        cells = []
        for n in names:
            v = work[n]["per_layer_nrms"].get(lay)
            cells.append("–" if v is None else f"{v:.2e}")
        print(f"| {lay} | " + " | ".join(cells) + " |")
    worst = [max(work[n]["per_layer_nrms"].values()) for n in names]
    print("| **worst** | " + " | ".join(f"**{w:.2e}**" for w in worst) + " |")
    print("\n## End to end: the GPU's final hidden states\n")
    print("| Workload | T | final nRMS vs oracle | oracle float32 vs float64 | floor | ratio to floor "
          "| GPU vs float64 oracle | max abs | within 0.005 |")
    print("|---|---|---|---|---|---|---|---|---|")
    for n in names:
        r = work[n]
        sp = r["oracle_f32_vs_f64_final_nrms"]
        fl = r.get("floor", sp)
        f64 = r.get("final_nrms_vs_f64_oracle")
        ok = r.get("end_to_end_within_0.005", r["final_nrms"] <= 5e-3)
        print(f"| {n} | {r['T']} | {r['final_nrms']:.4f} | {sp:.4f} | {fl:.4f} | {r['final_nrms'] / fl:.3f} "
              f"| {'–' if f64 is None else f'{f64:.4f}'} | {r['max_abs']:.3g} | {'yes' if ok else 'no'} |")


if __name__ == "__main__":
    main(sys.argv[1])
