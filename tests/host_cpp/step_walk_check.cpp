// Host check of the backward producers' step cursor (mx_layout.h step_walk / step_next): for
// many batched and packed geometries, every step of the head-major walk must sit exactly where
// the closed formulas (elem_offset_k, token_index_k, seq_group_row_k) put (hq, q0). Prints the
// number of cases and mismatches; exits non-zero on any mismatch.
#include <cstdio>

#include "../../block_scaled_mxfp8_amd/csrc/mx_layout.h"

using namespace mx;

static long long g_cases = 0;

template <bool kPacked>
static int walk(const Geom& g, int H, int D, int s, int doc_start, int n, int hq0, int group, int qfirst, int step) {
  const StepWalk sw = step_walk<kPacked>(g, H, D, s, doc_start, n, hq0, qfirst, step);
  StepPos c = sw.first;
  int hq = hq0, q0 = qfirst, bad = 0;
  const int nsteps = ((n - qfirst + step - 1) / step) * group;
  for (int j = 0; j < nsteps; j++) {
    const long long e = elem_offset_k<kPacked>(g, H, D, kPacked ? (long long)doc_start : (long long)s, hq, q0, 0);
    const long long t = token_index_k<kPacked>(g, H, s, doc_start, hq, q0);
    const long long r = seq_group_row_k<kPacked>(g, H, s, hq, doc_start, q0 >> 5);
    if (c.hq != hq || c.q0 != q0 || c.elem != e || c.tok != t || c.srow != r) {
      if (bad < 3)
        std::printf("mismatch: packed %d s %d hq %d q0 %d | got hq %d q0 %d elem %lld/%lld tok %lld/%lld srow %lld/%lld\n",
                    (int)kPacked, s, hq, q0, c.hq, c.q0, c.elem, e, c.tok, t, c.srow, r);
      bad++;
    }
    g_cases++;
    step_next(c, sw, step);
    q0 += step;
    if (q0 >= n) {
      q0 = qfirst;
      hq++;
    }
  }
  return bad;
}

int main() {
  int bad = 0;
  const int Ls[] = {1, 31, 63, 64, 65, 200, 4096};
  const int Ds[] = {64, 128};
  for (int L : Ls)
    for (int D : Ds)
      for (int H : {1, 4, 32})
        for (int group : {1, 2, 4}) {
          if (H % group) continue;
          Geom g{};
          g.batch = 3;
          g.seqlen = L;
          g.cu = nullptr;
          g.n_docs = 3;
          g.max_seqlen = L;
          g.total = 3LL * L;
          g.gseq = (L + 31) / 32;
          for (int s = 0; s < 3; s++)
            for (int hkv = 0; hkv < H / group; hkv++)
              for (int qfirst = 0; qfirst < L; qfirst += 64) bad += walk<false>(g, H, D, s, 0, L, hkv * group, group, qfirst, 64);
        }
  // packed: documents of assorted lengths back to back
  static const int lens[] = {1, 31, 32, 33, 100, 7, 300, 129, 64, 4096};
  int cu[11] = {0};
  for (int i = 0; i < 10; i++) cu[i + 1] = cu[i] + lens[i];
  for (int D : Ds)
    for (int H : {1, 4, 16})
      for (int group : {1, 4}) {
        if (H % group) continue;
        Geom g{};
        g.batch = 1;
        g.seqlen = 0;
        g.cu = cu;
        g.n_docs = 10;
        g.max_seqlen = 4096;
        g.total = cu[10];
        g.gseq = cu[10] / 32 + 10;
        for (int j = 0; j < 10; j++)
          for (int hkv = 0; hkv < H / group; hkv++)
            for (int qfirst = 0; qfirst < lens[j]; qfirst += 64)
              bad += walk<true>(g, H, D, j, cu[j], lens[j], hkv * group, group, qfirst, 64);
      }
  std::printf("step walk: %lld steps checked, %d mismatches\n", g_cases, bad);
  return bad != 0;
}
