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

// The next tile of a persistent launch for a workgroup on XCD `xcd`: a logical id
// from that XCD's own run while it lasts, then from the other XCDs' runs in turn
// ((xcd + 1) & 7, ...), or -1 once every run is handed out.  take(x) returns the
// number of ids handed out of XCD x's run so far and counts one more (on the device
// an atomic add on a per-XCD counter that starts each launch at zero).
template <typename Take>
GH_HOST_DEVICE inline int queue_next(Take take, int xcd, int total) {
  for (int k = 0; k < 8; ++k) {
    const int x = (xcd + k) & 7;
    int start, len;
    xcd_run(x, total, start, len);
    const int t = take(x);
    if (t < len) return start + t;
  }
  return -1;
}

}  // namespace gh
