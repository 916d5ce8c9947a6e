"""Per-kernel summary of a rocprofv3 kernel-trace database (SQLite, rocpd
format): calls, average / min / max duration in microseconds."""
import sqlite3
import sys


def summarize(db, top=20):
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(end-start), min(end-start), max(end-start), sum(end-start) "
                       "from kernels group by name order by sum(end-start) desc").fetchall()
    total = sum(r[5] for r in rows) or 1
    out = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for name, n, avg, mn, mx, sm in rows[:top]:
        out.append(f"| `{name[:80]}` | {n} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {100 * sm / total:.1f}% |")
    return "\n".join(out)


if __name__ == "__main__":
    print(summarize(sys.argv[1]))
