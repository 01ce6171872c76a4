"""Host-side work decomposition (csrc/sv_plan.hpp, plain integer C++): compiled
with the host compiler and checked against the rules it documents, re-derived
here independently: chunk sizes, finish parts, the early-exit grouping, the
one-pass draft choice, the workspace layout, and sizes at the largest shapes
the C ABI accepts (built with the address and undefined-behaviour sanitizers)."""
import json
import math
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PLAN = os.path.join(ROOT, "lossless_draft_verification_05_amd", "csrc", "sv_plan.hpp")

PROGRAM = r'''
#include <cstdio>
#include "sv_plan.hpp"
using namespace sv;
int main() {
  std::printf("{");
  std::printf("\"chunk\": [");
  const long long totals[] = {1LL << 20, 36866560LL, 1116358656LL, 4194328576LL, 1LL << 40};
  for (int i = 0; i < 5; ++i) std::printf("%s%lld", i ? "," : "", (long long)chunk_bytes_for(totals[i]));
  std::printf("], \"parts\": [");
  const long long pb[][2] = {{512, 125}, {256, 63}, {64, 16}, {1, 125}, {1, 63}, {3, 147}, {40, 63}, {1, 2051}, {1, 1},
                             {255, 2048}, {100, 7}};
  for (int i = 0; i < 11; ++i) std::printf("%s%d", i ? "," : "", finish_parts(pb[i][0], pb[i][1]));
  std::printf("], \"shape\": [");
  for (int i = 0; i < 11; ++i) {
    int k, nw;
    finish_shape(pb[i][0], pb[i][1], &k, &nw);
    std::printf("%s[%d,%d]", i ? "," : "", k, nw);
  }
  std::printf("], \"tail\": [");
  const long long tb[][5] = {{512, 5, 256000, 2, 4}, {256, 8, 128256, 2, 2}, {64, 4, 32000, 2, 2},
                             {1, 8, 128256, 2, 2}, {4096, 64, 256000, 4, 4}, {1024, 1, 256000, 2, 2}};
  for (int i = 0; i < 6; ++i)
    std::printf("%s%d", i ? "," : "", early_tail_start(tb[i][0], tb[i][1], tb[i][2], (int)tb[i][3], (int)tb[i][4]));
  std::printf("], \"one_pass\": [%d,%d,%d,%d,%d]", (int)draft_one_pass(512, 256000, 4), (int)draft_one_pass(127, 256000, 4),
              (int)draft_one_pass(8, 16384, 4), (int)draft_one_pass(8, 16385, 4), (int)draft_one_pass(200, 5000000, 4));
  const SampleLayout L1 = sample_layout(64, 4, 32000), L2 = sample_layout(64, 4, 64000), L3 = sample_layout(128, 4, 32000);
  std::printf(", \"layout\": [[%lld,%lld,%lld,%lld,%lld],[%lld],[%lld]]", (long long)L1.off_part, (long long)L1.off_step,
              (long long)L1.off_reach, (long long)L1.off_done, (long long)L1.total, (long long)L2.total,
              (long long)L3.total);
  int nch, cu, nch2, cu2;
  split_row(128256, 2, 136 << 10, &nch, &cu);
  split_row(128256, 2, chunk_bytes_for(1116358656LL), &nch2, &cu2, kBatchUnits);
  std::printf(", \"split\": [%d,%d,%d,%d]", nch, cu, nch2, cu2);
  const SampleLayout L4 = sample_layout(3, 2, 5000000);
  std::printf(", \"steps3\": [%lld,%lld,%lld]", (long long)L4.off_step, (long long)L4.off_reach,
              (long long)(L1.off_reach - L1.off_step));
  // the largest shapes the C ABI accepts (B 2^24, gamma 64, V 2^30, N 1024):
  // every size is computed in 64-bit arithmetic without overflow
  const long long Bm = 1LL << 24, Vm = 1LL << 30;
  const SampleLayout Lm = sample_layout(Bm, 64, Vm);
  const TreeLayout Tm = tree_layout(Bm, 1024, Vm);
  int nchm, cum;
  split_row(Vm, 4, chunk_bytes_for((Bm / 2) * (129LL * Vm * 4)), &nchm, &cum, kBatchUnits);
  std::printf(", \"max\": [%lld,%lld,%lld,%d,%d,%d,%d,%lld]", (long long)Lm.total, (long long)Tm.total,
              (long long)chunk_bytes_for((Bm / 2) * (129LL * Vm * 4)), nchm, cum, finish_parts(Bm, draw_steps(Vm)),
              early_tail_start(Bm, 64, Vm, 4, 4), (long long)draw_steps(Vm));
  std::printf("}\n");
  return 0;
}
'''


@pytest.fixture(scope="module")
def plan():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    import tempfile
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "plan.cpp"), os.path.join(d, "plan")
    with open(src, "w") as f:
        f.write(PROGRAM)
    # host build with the address and undefined-behaviour sanitizers: any
    # signed overflow or out-of-bounds access in the plan arithmetic aborts
    subprocess.run([gxx, "-std=c++17", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.dirname(PLAN), src, "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    shutil.rmtree(d)
    return json.loads(out)


def test_chunk_bytes(plan):
    # total / 8192 work units, clamped to [16 KB, 256 KB], rounded up to 16 KB
    # (one batch: 256 threads x 4 units x 16 B), so chunks start on batch boundaries
    for total, got in zip([1 << 20, 36866560, 1116358656, 4194328576, 1 << 40], plan["chunk"]):
        c = min(max(total // 8192, 16 << 10), 256 << 10)
        assert got == -(-c // 16384) * 16384, (total, got)


def test_finish_parts(plan):
    # up to ceil(256 / B) parts per sequence, at most one per 8 steps, one when the steps do not fit in LDS
    def parts(B, ns2):
        if ns2 > 2048:
            return 1
        return max(1, min(-(-256 // B), ns2 // 8))
    cases = [(512, 125), (256, 63), (64, 16), (1, 125), (1, 63), (3, 147), (40, 63), (1, 2051), (1, 1), (255, 2048),
             (100, 7)]
    assert plan["parts"] == [parts(B, n) for B, n in cases]
    assert plan["parts"][:4] == [1, 1, 2, 15]


def test_finish_shape(plan):
    # a split whose 8-wave parts stream at most two steps per wave runs as
    # ceil(K / 2) parts of 16 waves; otherwise K parts of 8 waves
    def parts(B, ns2):
        if ns2 > 2048:
            return 1
        return max(1, min(-(-256 // B), ns2 // 8))

    def shape(B, ns2):
        k = parts(B, ns2)
        if k >= 2 and ns2 <= 2 * k * 8:
            return [(k + 1) // 2, 16]
        return [k, 8]
    cases = [(512, 125), (256, 63), (64, 16), (1, 125), (1, 63), (3, 147), (40, 63), (1, 2051), (1, 1), (255, 2048),
             (100, 7)]
    assert plan["shape"] == [shape(B, n) for B, n in cases]
    # config 5 and 3 batches: one 8-wave part; config 2: one 16-wave part (no hand-off);
    # one sequence of 256k tokens: 8 parts of 16 waves; 64 sequences of 256k: 4 of 8
    assert plan["shape"][:4] == [[1, 8], [1, 8], [1, 16], [8, 16]]
    k, nw = shape(64, 125)
    assert (k, nw) == (4, 8)


def test_early_exit_grouping(plan):
    # position p gets its own launch while alpha^p (1 - alpha) (bytes of the later rows) >= 64 MB
    def tail(B, G, V, et, ed, a=0.7, L=64e6):
        pair, bonus, act = B * V * (et + ed), B * V * et, 1.0
        for p in range(G):
            if act * (1 - a) * ((G - p - 1) * pair + bonus) < L:
                return p
            act *= a
        return G
    cases = [(512, 5, 256000, 2, 4), (256, 8, 128256, 2, 2), (64, 4, 32000, 2, 2), (1, 8, 128256, 2, 2),
             (4096, 64, 256000, 4, 4), (1024, 1, 256000, 2, 2)]
    assert plan["tail"] == [tail(*c) for c in cases]
    assert plan["tail"][:4] == [4, 3, 0, 0]


def test_draft_one_pass_choice(plan):
    # one pass: steps fit in LDS (V <= 2048 * 2048) and (>= 128 rows or rows of at most 64 KB)
    assert plan["one_pass"] == [1, 0, 1, 0, 0]


def test_workspace_layout(plan):
    (part, step, reach, done, total), (total_v2,), (total_b2,) = plan["layout"]
    assert part == 0 and part < step < reach < done < total
    assert all(x % 256 == 0 for x in (step, reach, done, total))
    # partials: B (2 gamma + 1) rows x ceil(4 V / 16 KB) chunks x 4 waves x 16 B
    assert step >= 64 * 9 * math.ceil(4 * 32000 / (16 << 10)) * 4 * 16
    assert reach - step >= 64 * 4 * math.ceil(32000 / 2048) * 8     # step sums
    assert total_v2 > total and total_b2 > total


def test_row_split(plan):
    # a 256 KB row in chunks of at most 136 KB: two chunks of 4 KB-multiple units covering the row
    nch, cu, nch2, cu2 = plan["split"]
    assert nch == 2 and cu % 256 == 0 and nch * cu * 16 >= 128256 * 2 and (nch - 1) * cu * 16 < 128256 * 2
    # the statistics pass's split (configuration 3's call): 16 KB-multiple chunks covering the row
    assert cu2 % 1024 == 0 and nch2 * cu2 * 16 >= 128256 * 2 and (nch2 - 1) * cu2 * 16 < 128256 * 2
    assert cu2 * 16 <= 144 << 10


def test_step_sums(plan):
    # four fp64 values per draw step and sequence (mass, q-mass of the positive
    # residual, signed sum, form flag): LDS overflow and the finish parts' hand-off
    step, reach, small = plan["steps3"]
    assert reach - step == -(-3 * 4 * -(-5000000 // 2048) * 8 // 256) * 256
    assert small == -(-64 * 4 * 16 * 8 // 256) * 256


def test_largest_shapes(plan):
    """B = 2^24, gamma = 64, V = 2^30 (fp32), N = 1024: the sizes the C ABI's
    limits allow are computed without overflow (the sanitized build aborts on
    signed overflow) and are consistent."""
    lay_total, tree_total, chunk, nch, cu, parts, tail, steps = plan["max"]
    B, G, V = 1 << 24, 64, 1 << 30
    assert steps == V // 2048
    # partials of (2 gamma + 1) rows of up to V * 4 / 16 KB chunks, plus the step masses
    assert lay_total >= B * (2 * G + 1) * (V * 4 // (16 << 10)) * 4 * 16 + B * 4 * steps * 8
    assert lay_total < 1 << 62 and tree_total >= B * 1024 * (V * 4 // (16 << 10)) * 16
    assert (16 << 10) <= chunk <= (256 << 10) and cu % 1024 == 0 and nch * cu * 16 >= V * 4
    assert parts == 1 and 0 <= tail <= G
