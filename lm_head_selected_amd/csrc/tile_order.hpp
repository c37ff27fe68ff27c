// Tile order of the matrix-core launches.  Plain integer arithmetic with no
// device dependency, so the host test suite compiles this header on its own and
// checks that every mapping is a bijection.
#pragma once

#ifndef GH_HOST_DEVICE
#define GH_HOST_DEVICE __host__ __device__
#endif

namespace gh {

// Workgroups are dispatched round-robin over the 8 XCDs (bid % 8).  The logical
// tile id renumbers them so each XCD receives a contiguous run of ids.
GH_HOST_DEVICE inline int xcd_logical(int bid, int nwg) {
  const int q = nwg >> 3, r = nwg & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// The run of logical ids [start, start + len) that xcd_logical gives XCD `xcd` in a
// launch of `total` workgroups.
GH_HOST_DEVICE inline void xcd_run(int xcd, int total, int& start, int& len) {
  const int q = total >> 3, r = total & 7;
  start = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  len = q + (xcd < r ? 1 : 0);
}

// Logical tile id -> (M tile, N tile): ids walk `group_m` M-tiles down one N-tile
// before moving to the next N-tile, so workgroups resident together on one XCD
// share operand slices in that XCD's L2.
GH_HOST_DEVICE inline void logical_coords(int logical, int tiles_m, int tiles_n, int group_m,
                                          int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * group_m;
  int gsize = tiles_m - first_m;
  gsize = gsize < group_m ? gsize : group_m;
  const int in_g = logical - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

// The (M tile, N tile) workgroup `bid` of a launch of `nwg` workgroups computes;
// with nwg smaller than tiles_m * tiles_n it covers the logical ids [0, nwg).
GH_HOST_DEVICE inline void tile_coords(int bid, int nwg, int tiles_m, int tiles_n, int group_m,
                                       int& tm, int& tn) {
  logical_coords(xcd_logical(bid, nwg), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace gh
