"""The XCD placement of consumer positions, compiled from the same header
the kernels use (schedule.hpp is plain integer C++): for every grid the
planner accepts, the workgroups of one round take each position exactly
once, the workgroups of one XCD take a block of whole row panels x n-tile
groups, and a grid it cannot split keeps list order; where rounds do not
hold whole panels, the grouped placement is a permutation of positions and
of tiles, and each XCD's stretch of a round is a compact block."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "communication_gemm_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "schedule.hpp"
using namespace agg;
int main() {
    int checked = 0, split = 0;
    for (int nt = 1; nt <= 64; ++nt)
    for (int G = 1; G <= 1024; ++G) {
        Schedule s{};
        s.nt = nt; s.tm = 256; s.tn = (nt % 3) ? 128 : 256;
        s.xf = pick_xcd_split(s, G);
        std::vector<int> seen(G, 0);
        for (int b = 0; b < G; ++b) {
            long p = wg_position(s, b, G);
            if (p < 0 || p >= G) { printf("out of range G=%d nt=%d b=%d p=%ld\n", G, nt, b, p); return 1; }
            seen[p]++;
            if (s.xf == 0 && p != b) { printf("not identity G=%d nt=%d\n", G, nt); return 1; }
        }
        for (int p = 0; p < G; ++p)
            if (seen[p] != 1) { printf("not a permutation G=%d nt=%d p=%d\n", G, nt, p); return 1; }
        if (s.xf) {
            ++split;
            // one XCD: its positions form a block of panels x n-tiles
            int f = s.xf, gp = kXcds / f;
            for (int x = 0; x < kXcds; ++x) {
                long pmin = 1L << 40, pmax = -1, nmin = 1L << 40, nmax = -1, cnt = 0;
                for (int b = x; b < G; b += kXcds) {
                    long p = wg_position(s, b, G);
                    long panel = p / nt, n = p % nt;
                    pmin = panel < pmin ? panel : pmin; pmax = panel > pmax ? panel : pmax;
                    nmin = n < nmin ? n : nmin; nmax = n > nmax ? n : nmax; ++cnt;
                }
                long P = G / nt;
                if (pmax - pmin + 1 != P / gp || nmax - nmin + 1 != nt / f || cnt != (P / gp) * (nt / f)) {
                    printf("bad block G=%d nt=%d x=%d\n", G, nt, x); return 1;
                }
            }
        }
        ++checked;
    }
    // the shapes the workloads run: 256 workgroups, 16 n-tiles
    Schedule s{}; s.nt = 16; s.tm = 256; s.tn = 256;
    int f = pick_xcd_split(s, 256);
    printf("%d %d %d\n", checked, split, f);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ needed")
def test_xcd_placement_is_a_blocked_permutation(tmp_path):
    src = tmp_path / "sched.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "sched"
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    checked, split, f = map(int, out.stdout.split())
    assert checked == 64 * 1024 and split > 1000
    assert f in (2, 4)          # 16 panels x 16 n-tiles: 4 x 8 or 8 x 4 blocks


CHUNK_ORDER = r"""
#include <cstdio>
#include "schedule.hpp"
using namespace agg;
// The send order by its definition.  Parallel links: K-block after K-block;
// inside one, m-tile group after m-tile group, the row chunks each group
// needs first, source after source.  One serial link: source after source,
// each source's chunks in its own order (K-block major).  Chunk index
// within a source: K-block * row chunks + row chunk.
static bool by_definition(const Schedule& s, long c, int* src, int* j) {
    int remotes = s.n_shards - 1;
    if (s.link_model != 0) { *src = (int)(c / s.cps); *j = (int)(c % s.cps); return c < (long)remotes * s.cps; }
    long per_kb = (long)remotes * s.rcs;
    if (c >= per_kb * s.nkb) return false;
    int kb = (int)(c / per_kb);
    c %= per_kb;
    int prev = 0;
    for (int g = 0; g < s.mt; ++g) {
        int cur = need_chunks(s, g);
        long span = (long)(cur - prev) * remotes;
        if (c < span) { *src = (int)(c / (cur - prev)); *j = kb * s.rcs + prev + (int)(c % (cur - prev)); return true; }
        c -= span; prev = cur;
    }
    return false;
}
int main() {
    long checked = 0;
    const int Ss[] = {1, 7, 63, 64, 100, 128, 1000, 1024, 4096, 8192, 65536};
    const int tms[] = {32, 64, 128, 256};
    const int nkbs[] = {1, 3, 8};
    for (int S : Ss) for (int tm : tms) for (int n = 2; n <= 9; n += 3) for (int lm = 0; lm < 2; ++lm)
    for (int nkb : nkbs)
    for (int cr = 1; cr <= S; cr = cr < 8 ? cr + 1 : cr * 2 + (cr % 3)) {
        Schedule s{};
        s.n_shards = n; s.link_model = lm; s.cr = cr; s.S = S; s.tm = tm;
        s.rcs = (int)cdiv(S, cr); s.nkb = nkb; s.cps = s.rcs * nkb; s.mt = (int)cdiv(S, tm);
        if (s.cps > kFlagCap) continue;
        for (int i = 0; i < n; ++i) s.order[i] = (i * 5 + 1) % n;
        long total = (long)(n - 1) * s.cps;
        for (long c = -1; c <= total; ++c) {
            int src = -1, j = -1;
            bool in = c >= 0 && by_definition(s, c, &src, &j);
            ChunkRef r = chunk_at(s, c);
            if (!in) { if (r.src != -1) { printf("range S=%d cr=%d tm=%d c=%ld\n", S, cr, tm, c); return 1; } continue; }
            if (r.src != src || r.j != j || r.shard != s.order[1 + src] ||
                r.j != r.kb * s.rcs + r.jr || r.jr < 0 || r.jr >= s.rcs || r.kb < 0 || r.kb >= nkb) {
                printf("S=%d cr=%d tm=%d n=%d lm=%d nkb=%d c=%ld: %d/%d vs %d/%d\n", S, cr, tm, n, lm, nkb, c, r.src, r.j, src, j);
                return 1;
            }
            ++checked;
        }
    }
    printf("%ld\n", checked);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ needed")
def test_chunk_order_closed_form_matches_definition(tmp_path):
    """chunk_at's constant-time form (used for every producer piece) gives
    the send order defined K-block by K-block and group by group: for many
    shard, chunk and tile heights, 1, 3 and 8 K-blocks, both link models,
    every position and one past each end."""
    src = tmp_path / "chunks.cpp"
    src.write_text(CHUNK_ORDER)
    exe = tmp_path / "chunks"
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    assert int(out.stdout) > 100000


PACED = r"""
#include <cstdio>
#include <initializer_list>
#include "schedule.hpp"
using namespace agg;
// paced_bytes(chunk) is the bytes of the source's chunks up to and
// including it in the source's own order (parallel links), plus every
// earlier source whole (serial link): summed chunk by chunk here.
int main() {
    long checked = 0;
    const int Ss[] = {1, 33, 100, 1024};
    const long Ks[] = {1024, 2560, 4096};
    for (int S : Ss) for (long K : Ks) for (int lm = 0; lm < 2; ++lm)
    for (long kbk : {256L, 512L, 1024L, 4096L}) for (int cr : {1, 7, 16, 100}) {
        if (cr > S) continue;
        Schedule s{};
        s.n_shards = 4; s.link_model = lm; s.cr = cr; s.S = S; s.K = K; s.tm = 64;
        s.rcs = (int)cdiv(S, cr); s.kbk = kbk < K ? kbk : K; s.nkb = (int)(K / s.kbk);
        s.cps = s.rcs * s.nkb; s.mt = (int)cdiv(S, s.tm);
        if (s.cps > kFlagCap) continue;
        for (int i = 0; i < 4; ++i) s.order[i] = i;
        for (int src = 0; src < 3; ++src) {
            long sum = lm ? (long)src * S * K * 2 : 0;
            for (int j = 0; j < s.cps; ++j) {
                ChunkRef r; r.src = src; r.shard = src + 1; r.j = j; r.kb = j / s.rcs; r.jr = j % s.rcs;
                const long rows = chunk_row_end(s, r.jr) - (long)r.jr * cr;
                sum += rows * (kblock_end(s, r.kb) - kblock_begin(s, r.kb)) * 2;
                if (paced_bytes(s, r, 2) != sum) {
                    printf("S=%d K=%ld kbk=%ld cr=%d lm=%d src=%d j=%d: %ld vs %ld\n", S, K, kbk, cr,
                           lm, src, j, (long)paced_bytes(s, r, 2), sum);
                    return 1;
                }
                ++checked;
            }
            if (sum != (lm ? (long)(src + 1) : 1L) * S * K * 2) { printf("total\n"); return 1; }
        }
    }
    printf("%ld\n", checked);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ needed")
def test_paced_bytes_follow_each_sources_order(tmp_path):
    """The emulated link's byte count for a chunk is what the source has
    sent up to and including it: K-blocks before it whole, then its
    K-block's rows up to its last; the serial link adds earlier sources."""
    src = tmp_path / "paced.cpp"
    src.write_text(PACED)
    exe = tmp_path / "paced"
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    assert int(out.stdout) > 10000


CU_MASK = r"""
#include <cstdio>
#include "plan.hpp"
using namespace agg;
// The producer's CU mask has `cus` bits, cus/8 on every XCD: the driver
// deals a queue's mask bits round-robin over the XCDs (bit b on XCD b % 8).
int main() {
    for (int cus = 32; cus <= 64; cus += 32) {
        uint32_t m[8];
        producer_cu_mask(cus, m);
        int n = 0, rr[8] = {0};
        for (int b = 0; b < 256; ++b)
            if (m[b / 32] >> (b % 32) & 1) { ++n; ++rr[b % 8]; }
        if (n != cus) { printf("count %d %d\n", cus, n); return 1; }
        for (int x = 0; x < 8; ++x)
            if (rr[x] != cus / 8) { printf("xcd %d %d\n", cus, x); return 1; }
    }
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ needed")
def test_producer_cu_mask_spreads_over_xcds(tmp_path):
    src = tmp_path / "mask.cpp"
    src.write_text(CU_MASK)
    exe = tmp_path / "mask"
    inc = os.path.join(ROOT, "include")
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", f"-I{inc}", str(src),
                    os.path.join(CSRC, "plan.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout


GROUPED = r"""
#include <cstdio>
#include <vector>
#include "schedule.hpp"
using namespace agg;
int main() {
    long checked = 0, grouped = 0;
    for (int nt = 1; nt <= 120; nt += (nt < 20 ? 1 : 7))
    for (int mt = 1; mt <= 40; mt += (mt < 8 ? 1 : 5))
    for (int n_shards = 1; n_shards <= 4; ++n_shards)
    for (int link = 0; link <= 1; ++link)
    for (int G : {8, 16, 64, 200, 224, 256, 512}) {
        Schedule s{};
        s.nt = nt; s.mt = mt; s.tm = 256; s.tn = (nt % 3) ? 128 : 256;
        s.n_shards = n_shards; s.local = 0; s.link_model = link; s.ks = 1;
        s.S = (int64_t)mt * 256; s.cr = 64;
        for (int q = 0; q < n_shards; ++q) s.order[q] = q;
        s.xf = pick_xcd_split(s, G);
        s.gm = pick_group(s, G);
        if (s.xf && s.gm) { printf("both placements G=%d nt=%d\n", G, nt); return 1; }
        if (!s.gm) continue;
        ++grouped;
        // positions of one round: a permutation of [0, G)
        std::vector<int> seen(G, 0);
        for (int b = 0; b < G; ++b) {
            const long p = wg_position(s, b, G);
            if (p < 0 || p >= G || seen[p]++) { printf("not a permutation G=%d\n", G); return 1; }
        }
        // tile list: each (shard, m, n) exactly once
        const long T = total_tiles(s);
        std::vector<char> hit((size_t)n_shards * mt * nt, 0);
        for (long p = 0; p < T; ++p) {
            const TileRef t = tile_at(s, p);
            if (t.shard < 0 || t.shard >= n_shards || t.m < 0 || t.m >= mt || t.n < 0 || t.n >= nt) {
                printf("tile out of range p=%ld\n", p); return 1;
            }
            char& h = hit[((size_t)t.shard * mt + t.m) * nt + t.n];
            if (h++) { printf("tile twice p=%ld\n", p); return 1; }
        }
        // an XCD's stretch of a round that stays inside one group of the
        // local segment spans the group's panels and about G / (8 gm) n-tiles
        const long per = G / kXcds, local = (long)mt * nt;
        for (long r0 = 0; r0 + G <= local; r0 += G)
            for (int x = 0; x < kXcds; ++x) {
                long p0 = r0 + x * per, p1 = p0 + per;
                if (p0 / ((long)s.gm * nt) != (p1 - 1) / ((long)s.gm * nt)) continue;
                int mlo = 1 << 30, mhi = -1, nlo = 1 << 30, nhi = -1;
                for (long p = p0; p < p1; ++p) {
                    const TileRef t = tile_at(s, p);
                    mlo = t.m < mlo ? t.m : mlo; mhi = t.m > mhi ? t.m : mhi;
                    nlo = t.n < nlo ? t.n : nlo; nhi = t.n > nhi ? t.n : nhi;
                }
                const long g = p0 / ((long)s.gm * nt), left = mt - g * s.gm;
                const long gsz = left < s.gm ? left : s.gm;   // a short last group
                if (mhi - mlo + 1 > gsz || nhi - nlo + 1 > (per + gsz - 1) / gsz + 1) {
                    printf("loose block G=%d nt=%d mt=%d gm=%d\n", G, nt, mt, s.gm); return 1;
                }
            }
        ++checked;
    }
    // the int8 workload's shape: 256 workgroups, 107 n-tiles of 256
    Schedule s{}; s.nt = 107; s.mt = 32; s.tm = 256; s.tn = 256; s.ks = 1;
    s.xf = pick_xcd_split(s, 256);
    printf("%ld %ld %d %d\n", checked, grouped, s.xf, pick_group(s, 256));
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ needed")
def test_grouped_placement_is_a_compact_permutation(tmp_path):
    src = tmp_path / "grouped.cpp"
    src.write_text(GROUPED)
    exe = tmp_path / "grouped"
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    checked, grouped, xf, gm = map(int, out.stdout.split())
    assert grouped > 100 and checked == grouped
    assert xf == 0 and gm == 4     # 32 workgroups per XCD: 4 panels x 8 n-tiles
