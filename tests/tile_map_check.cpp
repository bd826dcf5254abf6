// Host-side check of gemm::tile_coords (built and run by test_tile_map.py):
// for every grid shape and band height tried, the mapping from workgroup id
// to (tile row, tile column) must hit every tile exactly once.
#include <cstdio>
#include <vector>

#include "gemm_device.hpp"

int main() {
    int failures = 0, cases = 0;
    const int groups[] = {1, 2, 4, 8, 16};
    for (int tm = 1; tm <= 40; ++tm) {
        for (int tn = 1; tn <= 40; ++tn) {
            for (int g : groups) {
                std::vector<int> seen(tm * tn, 0);
                bool ok = true;
                for (int w = 0; w < tm * tn; ++w) {
                    int r, c;
                    gemm::tile_coords(w, tm, tn, g, r, c);
                    if (r < 0 || r >= tm || c < 0 || c >= tn) { ok = false; break; }
                    seen[r * tn + c]++;
                }
                for (int v : seen) ok = ok && v == 1;
                ++cases;
                if (!ok) {
                    if (failures < 10) std::printf("FAIL tiles %dx%d group %d\n", tm, tn, g);
                    ++failures;
                }
            }
        }
    }
    // Large grids used by the benchmark shapes.
    const int big[][3] = {{16, 16, 4}, {32, 32, 4}, {64, 64, 8}, {63, 47, 8}, {128, 2, 8}};
    for (const auto &b : big) {
        std::vector<int> seen(b[0] * b[1], 0);
        for (int w = 0; w < b[0] * b[1]; ++w) {
            int r, c;
            gemm::tile_coords(w, b[0], b[1], b[2], r, c);
            if (r >= 0 && r < b[0] && c >= 0 && c < b[1]) seen[r * b[1] + c]++;
        }
        bool ok = true;
        for (int v : seen) ok = ok && v == 1;
        ++cases;
        if (!ok) { std::printf("FAIL big %dx%d\n", b[0], b[1]); ++failures; }
    }
    // Square-round mapping (falls back to tile_coords off multiples of 16).
    for (int tm = 1; tm <= 72; tm += (tm < 40 ? 1 : 8)) {
        for (int tn = 1; tn <= 72; tn += (tn < 40 ? 1 : 8)) {
            std::vector<int> seen(tm * tn, 0);
            bool ok = true;
            for (int w = 0; w < tm * tn; ++w) {
                int r, c;
                gemm::tile_coords_square(w, tm, tn, 4, r, c);
                if (r < 0 || r >= tm || c < 0 || c >= tn) { ok = false; break; }
                seen[r * tn + c]++;
            }
            for (int v : seen) ok = ok && v == 1;
            ++cases;
            if (!ok) { std::printf("FAIL square %dx%d\n", tm, tn); ++failures; }
        }
    }
    std::printf("%s %d cases\n", failures ? "FAILED" : "OK", cases);
    return failures ? 1 : 0;
}
