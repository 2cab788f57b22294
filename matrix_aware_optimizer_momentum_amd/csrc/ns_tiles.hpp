// Walk order of the 256 x 256 output tiles of one problem of the persistent
// NS GEMMs (plain C++, shared by the kernel and a host-side check).
//
// The tiles go in bands of kTileBand tile rows; within a band, column by
// column, and within a column the band's rows from the top.  A workgroup
// round hands consecutive tiles to the 32 CUs of one XCD, so those tiles
// come from about kTileBand row panels and 32 / kTileBand column panels of
// the operands, which that XCD's L2 then shares (a row-major walk would
// touch one or two row panels but up to 32 column panels).  A symmetric
// product has only its tiles with tm >= tn, the same walk restricted to
// them.
#pragma once

#ifndef SM_HD
#define SM_HD
#endif

namespace sm {

constexpr int kTileBand = 4;

// Tiles of band b (rows b*kTileBand .. of tm_count): all columns for a
// rectangle, columns up to the band's last row for the lower triangle.
SM_HD inline int ns_band_tiles(int b, int tm_count, int tn_count, int sym) {
  const int r0 = b * kTileBand;
  const int h = tm_count - r0 < kTileBand ? tm_count - r0 : kTileBand;
  if (!sym) return h * tn_count;
  return r0 * h + h * (h + 1) / 2;   // full columns 0 .. r0-1, then the triangle
}

// (tm, tn) of the u-th tile in the walk (0 <= u < tiles of the problem).
SM_HD inline void ns_tile_coords(int u, int tm_count, int tn_count, int sym, int* tm, int* tn) {
  int b = 0;
  for (;;) {
    const int nb = ns_band_tiles(b, tm_count, tn_count, sym);
    if (u < nb) break;
    u -= nb;
    ++b;
  }
  const int r0 = b * kTileBand;
  const int h = tm_count - r0 < kTileBand ? tm_count - r0 : kTileBand;
  const int full = sym ? r0 : tn_count;   // columns with all h rows of the band
  if (u < full * h) {
    *tn = u / h;
    *tm = r0 + (u - *tn * h);
    return;
  }
  // the band's diagonal triangle: column r0 + j holds rows r0 + j .. r0 + h - 1
  u -= full * h;
  int j = 0;
  while (u >= h - j) {
    u -= h - j;
    ++j;
  }
  *tn = r0 + j;
  *tm = r0 + j + u;
}

}  // namespace sm
