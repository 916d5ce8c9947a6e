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


def gaps(db, kernel):
    """For back-to-back dispatches of a kernel whose name contains `kernel`:
    the time from one dispatch's end to the next one's start (median, 10th
    and 90th percentile, microseconds), and the dispatch period (start to
    next start)."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, end from kernels order by start").fetchall()
    g, p = [], []
    for (n0, s0, e0), (n1, s1, _) in zip(rows, rows[1:]):
        if kernel in n0 and kernel in n1:
            g.append((s1 - e0) / 1e3)
            p.append((s1 - s0) / 1e3)
    if not g:
        return f"no back-to-back dispatches of {kernel}"
    g.sort()
    p.sort()

    def q(v, f):
        return v[min(len(v) - 1, int(f * len(v)))]
    return (f"{kernel}: {len(g)} back-to-back pairs; end-to-next-start gap median {q(g, 0.5):.2f} us "
            f"(p10 {q(g, 0.1):.2f}, p90 {q(g, 0.9):.2f}); start-to-next-start median {q(p, 0.5):.2f} us")


if __name__ == "__main__":
    if len(sys.argv) > 3 and sys.argv[2] == "--gaps":
        print(gaps(sys.argv[1], sys.argv[3]))
    else:
        print(summarize(sys.argv[1]))
