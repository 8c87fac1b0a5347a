// Output-tile order of the large GEMM kernels on the 8 XCDs of gfx950.
#pragma once

namespace ck4 {

// Workgroup ids are dealt round-robin to the 8 XCDs (id & 7), and each XCD
// has its own L2. With xcd_m > 0 the tile grid is cut into xcd_m x (8 / xcd_m)
// blocks, one per XCD, walked row-major inside, so an XCD's L2 holds only
// its block's A rows and B rows; otherwise each XCD walks a contiguous run of
// tiles.
__device__ __forceinline__ void tile_coords(int id, int tiles_n, int tiles_total, int xcd_m, int &tm, int &tn) {
    if (xcd_m > 0) {
        const int xcd_n = 8 / xcd_m;
        const int x = id & 7, li = id >> 3;
        const int bm = (tiles_total / tiles_n) / xcd_m, bn = tiles_n / xcd_n;
        tm = (x / xcd_n) * bm + li / bn;
        tn = (x % xcd_n) * bn + li % bn;
    } else {
        if ((tiles_total & 7) == 0) id = (id & 7) * (tiles_total >> 3) + (id >> 3);
        tm = id / tiles_n;
        tn = id - tm * tiles_n;
    }
}

// Shape of the per-XCD tile blocks: xcd_m rows of blocks by 8 / xcd_m
// columns, chosen to minimise the A and B rows one XCD fetches (0: the grid
// does not split evenly; fall back to contiguous runs).
inline int pick_xcd_m(int tiles_m, int tiles_n, int bm, int bn) {
    int best = 0;
    long best_rows = 0;
    for (int xm = 1; xm <= 8; xm *= 2) {
        const int xn = 8 / xm;
        if (tiles_m % xm != 0 || tiles_n % xn != 0) continue;
        const long rows = (long)(tiles_m / xm) * bm + (long)(tiles_n / xn) * bn;
        if (best == 0 || rows < best_rows) {
            best = xm;
            best_rows = rows;
        }
    }
    return best;
}

}  // namespace ck4
