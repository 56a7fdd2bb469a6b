// The plain SelectRep tournaments of one lane group (InfiniteHiP page,
// 2502.08910, section 3.4, "The Representative Token Selection Algorithm
// (SelectRep)"), generic over where the key rows come from.
#pragma once

#include "prune_common.h"

namespace dsa {

// One lane group's SelectRep tournaments: the G query heads of one kv head
// over the chunk of l = chunk[stage] keys starting at st, side by side; rows
// come from `rows` (rows.at(position) returns this lane's slice of a key row:
// as stored, or transformed). The first split's two representatives are shared
// by all heads; with SPEC, the SPEC keys that can represent the first
// log2(SPEC) splits are loaded in one round; with TAIL4 (latency-bound
// launches), the last two splits of a 4-key range too. Returns the best
// representative score over the heads.
template <typename T, int D, int G, int SPEC, class Rows, bool TAIL4 = false>
__device__ __forceinline__ float selectrep_group(const PruneArgs& a, int stage, int li, int st, const Rows& rows,
                                                 const RowSlice<T, D / 16> (&q)[G]) {
  using Row = RowSlice<T, D / 16>;
  const int l = a.chunk[stage];
  float best = -INFINITY;
  auto dot = [&](const Row& kr, int hh) { return group16_sum(kr.dot(q[hh])); };

  float sa[G];
  int lo[G], hi[G];
  unsigned long long nvis = 0;
  int width;                                   // size of every head's remaining range
  if (l == 1) {
    const Row k0 = rows.at(st);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) { sa[hh] = dot(k0, hh); lo[hh] = hi[hh] = 0; }
    nvis = 1;
    width = 1;
  } else if (SPEC == 4 && l >= 4) {
    // the 4 keys that can represent the first two splits (positions i*l/4)
    // in one round
    const int u = l >> 2;
    float sc4[G][4];
    {
      Row kr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = rows.at(st + i * u);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) sc4[hh][i] = dot(kr[i], hh);
    }
    int a1[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      int A = 0;
      float s0 = sc4[hh][0];
      if (sc4[hh][2] > s0) { A = 2; s0 = sc4[hh][2]; }
      a1[hh] = A;
      const float s2 = A ? sc4[hh][3] : sc4[hh][1];
      if (s2 > s0) { A += 1; s0 = s2; }
      lo[hh] = A * u;
      hi[hh] = A * u + u - 1;
      sa[hh] = s0;
    }
    if (a.visited) {
      nvis = 2;                                 // split 1: keys 0 and l/2
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {          // split 2: distinct midpoints
        bool f2 = true;
#pragma unroll
        for (int h2 = 0; h2 < hh; ++h2) f2 = f2 && (a1[h2] != a1[hh]);
        nvis += f2 ? 1 : 0;
      }
    }
    width = u;
  } else if (SPEC == 8 && l >= 8) {
    const int u = l >> 3;
    float sc8[G][8];
    {
      Row kr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = rows.at(st + i * u);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) sc8[hh][i] = dot(kr[i], hh);
    }
    int a1[G], a2[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      int A = 0;
      float s0 = sc8[hh][0];
      if (sc8[hh][4] > s0) { A = 4; s0 = sc8[hh][4]; }
      a1[hh] = A;
      const float s2 = A ? sc8[hh][6] : sc8[hh][2];
      if (s2 > s0) { A += 2; s0 = s2; }
      a2[hh] = A;
      const float s3 = A == 0 ? sc8[hh][1] : A == 2 ? sc8[hh][3] : A == 4 ? sc8[hh][5] : sc8[hh][7];
      if (s3 > s0) { A += 1; s0 = s3; }
      lo[hh] = A * u;
      hi[hh] = A * u + u - 1;
      sa[hh] = s0;
    }
    if (a.visited) {
      nvis = 2;                                 // split 1: keys 0 and l/2
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {          // splits 2 and 3: distinct midpoints
        bool f2 = true, f3 = true;
#pragma unroll
        for (int h2 = 0; h2 < hh; ++h2) {
          f2 = f2 && (a1[h2] != a1[hh]);
          f3 = f3 && (a2[h2] != a2[hh]);
        }
        nvis += (f2 ? 1 : 0) + (f3 ? 1 : 0);
      }
    }
    width = u;
  } else {
    const int mid0 = l >> 1;
    const Row k0 = rows.at(st), k1 = rows.at(st + mid0);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float a0 = dot(k0, hh), a1 = dot(k1, hh);
      if (a1 > a0) { lo[hh] = mid0; hi[hh] = l - 1; sa[hh] = a1; }
      else         { lo[hh] = 0;    hi[hh] = mid0 - 1; sa[hh] = a0; }
    }
    nvis = 2;
    width = mid0;
  }
  for (int wdt = width >> 1; wdt >= 1; wdt >>= 1) {   // remaining splits
    if (TAIL4 && wdt == 2) {
      // The last two splits of a 4-key range [lo, lo + 3]: its other three
      // keys are loaded in one round (one dependent round fewer, one row per
      // head more); the first split compares lo with lo + 2, the second the
      // winner with its neighbour; the visits counted are the method's.
      Row k1[G], k2[G], k3[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        k1[hh] = rows.at(st + lo[hh] + 1);
        k2[hh] = rows.at(st + lo[hh] + 2);
        k3[hh] = rows.at(st + lo[hh] + 3);
      }
      int m1[G], m2[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float s1 = dot(k1[hh], hh), s2 = dot(k2[hh], hh), s3 = dot(k3[hh], hh);
        m1[hh] = lo[hh] + 2;
        float sn = s1;
        if (s2 > sa[hh]) { lo[hh] += 2; sa[hh] = s2; sn = s3; }
        m2[hh] = lo[hh] + 1;
        if (sn > sa[hh]) { lo[hh] += 1; sa[hh] = sn; }
      }
      if (a.visited) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          bool f1 = true, f2 = true;
#pragma unroll
          for (int h2 = 0; h2 < hh; ++h2) {
            f1 = f1 && (m1[h2] != m1[hh]);
            f2 = f2 && (m2[h2] != m2[hh]);
          }
          nvis += (f1 ? 1 : 0) + (f2 ? 1 : 0);
        }
      }
      break;
    }
    Row kk[G];
    int mid[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      mid[hh] = (lo[hh] + hi[hh] + 1) >> 1;
      kk[hh] = rows.at(st + mid[hh]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float acc = dot(kk[hh], hh);
      if (acc > sa[hh]) { lo[hh] = mid[hh]; sa[hh] = acc; }
      else              { hi[hh] = mid[hh] - 1; }
    }
    if (a.visited) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        bool fresh = true;
#pragma unroll
        for (int h2 = 0; h2 < hh; ++h2) fresh = fresh && (mid[h2] != mid[hh]);
        nvis += fresh ? 1 : 0;
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) best = fmaxf(best, sa[hh]);
  if (a.visited && li == 0) atomicAdd(a.visited + stage, nvis);
  return best;
}

}  // namespace dsa
