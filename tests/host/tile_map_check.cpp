// Host-side check of the work-group -> output-tile mapping used by the GEMM
// kernels: for every grid shape tried, each tile is produced exactly once and
// every (tm, tn) lies inside the grid.  Prints "ok" or the first failure.
#include <cstdio>
#include <vector>

#include "gemm_internal.hpp"

int main() {
    const int group_sizes[] = {1, 2, 4, 8, 16};
    for (int tiles_m = 1; tiles_m <= 40; ++tiles_m)
        for (int tiles_n = 1; tiles_n <= 40; ++tiles_n)
            for (int gm : group_sizes) {
                std::vector<int> seen(tiles_m * tiles_n, 0);
                for (int b = 0; b < tiles_m * tiles_n; ++b) {
                    int tm, tn;
                    sgemm::tile_of_block(b, tiles_m, tiles_n, gm, tm, tn);
                    if (tm < 0 || tm >= tiles_m || tn < 0 || tn >= tiles_n) {
                        std::printf("out of range: grid %dx%d group %d block %d -> (%d,%d)\n",
                                    tiles_m, tiles_n, gm, b, tm, tn);
                        return 1;
                    }
                    ++seen[tm * tiles_n + tn];
                }
                for (int v : seen)
                    if (v != 1) {
                        std::printf("not a bijection: grid %dx%d group %d\n", tiles_m, tiles_n, gm);
                        return 1;
                    }
            }
    // The headline grid: 32 x 32 tiles, and a large one.
    for (int shape : {32, 64, 86, 1000}) {
        std::vector<int> seen(shape * shape, 0);
        for (int b = 0; b < shape * shape; ++b) {
            int tm, tn;
            sgemm::tile_of_block(b, shape, shape, 8, tm, tn);
            if (tm < 0 || tm >= shape || tn < 0 || tn >= shape || seen[tm * shape + tn]++) {
                std::printf("failure on %dx%d\n", shape, shape);
                return 1;
            }
        }
    }
    std::printf("ok\n");
    return 0;
}
