"""Liveness of the chunk protocol, checked by simulation on the CPU.

A g++ program builds real plans with the library's own plan.cpp and
schedule.hpp, then runs every agent of both kernels as the kernels do:
producer wave w takes items w, w + P, ... in order, and before a piece of a
ring panel it waits for the stage's finished tiles, having counted every
piece it copied before (a wave that waited on a stage while holding an
uncounted piece could stall the tiles it waits for); consumer workgroup
b takes positions wg_position(b) + r G in order, and before a tile it waits
for its source's counter (every source's, in the barrier scheme), then
counts the tile on its ring stage.  Counters advance over contiguous
released chunks.  Each case must finish with every item and every tile
done; a planted cyclic configuration (a barrier iteration larger than the
ring) must be caught as a stall, which shows the check can fail."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "communication_gemm_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ needed")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "plan.hpp"
using namespace agg;

// 0: every item and tile done; 1: stall
static int simulate(Schedule s, int ppc, int G, int P)
{
    s.xf = pick_xcd_split(s, G);
    s.gm = pick_group(s, G);
    const long tiles = total_tiles(s), chunks = total_chunks(s), items = chunks * ppc;
    std::vector<long> pnext(P), cnext(G, 0);
    for (int w = 0; w < P; ++w) pnext[w] = w;
    std::vector<int> pieces(chunks, 0);
    std::vector<std::vector<char>> released(s.n_shards, std::vector<char>(s.cps, 0));
    std::vector<int> counter(s.n_shards, 0);
    std::vector<std::vector<long>> stage(s.n_shards, std::vector<long>(kMaxStages, 0));
    long items_done = 0, tiles_done = 0;
    for (;;) {
        bool progress = false;
        for (int w = 0; w < P; ++w) {
            for (;;) {
                const long it = pnext[w];
                if (it >= items) break;
                const long c = it / ppc;
                const ChunkRef r = chunk_at(s, c);
                const long row0 = (long)r.j * s.cr;
                if (s.ring > 0) {
                    const int m = (int)(row0 / s.tm);
                    if (stage[r.shard][m % s.ring] < stage_tiles_before(s, m)) break;
                }
                if (++pieces[c] == ppc) {
                    released[r.shard][r.j] = 1;
                    while (counter[r.shard] < s.cps && released[r.shard][counter[r.shard]])
                        ++counter[r.shard];
                }
                pnext[w] += P; ++items_done; progress = true;
            }
        }
        for (int b = 0; b < G; ++b) {
            for (;;) {
                const long pos = wg_position(s, b, G) + cnext[b] * (long)G;
                if (pos >= tiles) break;
                const TileRef t = tile_at(s, pos);
                bool ok = true;
                if (t.need > 0) {
                    if (s.pv > 0) {
                        for (int q = 1; q < s.n_shards; ++q)
                            ok = ok && counter[s.order[q]] >= t.need;
                    } else {
                        ok = counter[t.shard] >= t.need;
                    }
                }
                if (!ok) break;
                if (s.ring > 0 && t.shard != s.local) ++stage[t.shard][t.m % s.ring];
                ++cnext[b]; ++tiles_done; progress = true;
            }
        }
        if (items_done == items && tiles_done == tiles) return 0;
        if (!progress) return 1;
    }
}

int main()
{
    long cases = 0, rings = 0, barriers = 0;
    const int tiles_ids[] = {3, 2, 8};
    for (int n : {2, 3, 4, 8})
    for (long S : {100L, 256L, 1000L, 1024L})
    for (long N : {64L, 384L, 4096L})
    for (int tile : tiles_ids)
    for (int scheme = 0; scheme < 2; ++scheme)
    for (int pv : {1, 2, 3})
    for (int ring : {0, 1, 2, 3, 4})
    for (int link : {0, 1})
    for (int cr : {0, 8, 64}) {
        if (scheme == 0 && pv > 1) continue;
        agg_options o;
        ag_gemm_options_init(&o);
        o.tile = tile; o.link_model = link; o.workspace_stages = ring;
        o.scheme = scheme; o.pvalue = pv; o.local_shard = n - 1;
        Plan p;
        if (make_plan(kF16, n, n * S, 64, N, cr, &o, 256, &p) != AGG_OK) continue;
        for (int G : {1, 2, 7, 64, 256})
        for (int P : {1, 3, 256}) {
            if (simulate(p.sched, p.ppc, G, P)) {
                printf("stall n=%d S=%ld N=%ld tile=%d scheme=%d pv=%d ring=%d link=%d cr=%d G=%d P=%d\n",
                       n, S, N, tile, scheme, pv, p.sched.ring, link, cr, G, P);
                return 1;
            }
            ++cases;
            rings += p.sched.ring > 0;
            barriers += p.sched.pv > 0;
        }
    }
    // planted cycle: a barrier iteration of 2 panels over a 1-stage ring
    // (the planner refuses it); the simulation must stall
    agg_options o;
    ag_gemm_options_init(&o);
    o.tile = 3; o.workspace_stages = 2; o.scheme = 1; o.pvalue = 2;
    Plan p;
    if (make_plan(kF16, 4, 4 * 1024, 64, 384, 8, &o, 256, &p) != AGG_OK) { printf("plan\n"); return 1; }
    Schedule bad = p.sched;
    bad.ring = 1;
    const int planted = simulate(bad, p.ppc, 64, 16);
    printf("%ld %ld %ld %d\n", cases, rings, barriers, planted);
    return 0;
}
"""


def test_no_schedule_stalls(tmp_path):
    src = tmp_path / "sim.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "sim"
    subprocess.run(["g++", "-std=c++17", "-O2", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
                    str(src), os.path.join(CSRC, "plan.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    cases, rings, barriers, planted = (int(x) for x in out.stdout.split())
    assert cases > 10000 and rings > 1000 and barriers > 1000
    assert planted == 1          # the checker does find a cycle
