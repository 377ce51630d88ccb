// Host-side check of the LDS tile layouts of the 16-bit kernels (Tile<128>, Tile<64> in
// fa_device.h), compiled from the same header the kernels use.
//
// For a [64][D] tile it places every byte the way the DMA copies do (instruction i, lane l:
// global offset Tile<D>::dma_offset, LDS byte kRunBytes * i + 16 * l), then checks that
//   - every byte of the tile lands once, inside kElems values of LDS;
//   - each row read and each transposing read of every lane, at every row base, column block
//     and half the kernels use, addresses exactly the bytes of the row and columns it stands for;
//   - the lanes of one LDS transfer hit distinct banks: 16 lanes of a row read cover 16
//     distinct 16-byte bank groups, 32 lanes of a transposing read all 64 banks (D = 128) or,
//     for D = 64, 16 lanes 32 banks.
// Prints "ok" and exits 0, or prints the first failures and exits 1.
#include <cstdio>
#include <set>
#include <vector>

#include "fa_device.h"

static int g_fail = 0;
#define CHECK(c, ...)                      \
    do {                                   \
        if (!(c)) {                        \
            if (g_fail < 20) {             \
                std::printf(__VA_ARGS__);  \
                std::printf("\n");         \
            }                              \
            ++g_fail;                      \
        }                                  \
    } while (0)

template <int D>
void check_layout() {
    using Tl = fa::Tile<D>;
    constexpr int kRowBytes = 2 * D;
    constexpr int kTileBytes = 64 * kRowBytes;
    constexpr int kRuns = kTileBytes / 1024;
    // global byte (row stride D values) -> LDS byte
    std::vector<int> phys(kTileBytes, -1);
    std::set<int> used;
    for (int i = 0; i < kRuns; ++i) {
        for (int lane = 0; lane < 64; ++lane) {
            const int g = Tl::dma_offset(i, lane, D);
            const int l = Tl::kRunBytes * i + 16 * lane;
            for (int b = 0; b < 16; ++b) {
                CHECK(g + b >= 0 && g + b < kTileBytes, "D=%d run %d lane %d: global byte %d outside", D, i, lane, g + b);
                if (g + b < 0 || g + b >= kTileBytes) continue;
                CHECK(phys[g + b] < 0, "D=%d global byte %d copied twice", D, g + b);
                phys[g + b] = l + b;
                CHECK(l + b < 2 * Tl::kElems, "D=%d LDS byte %d outside the tile's %d values", D, l + b, Tl::kElems);
                CHECK(used.insert(l + b).second, "D=%d LDS byte %d written twice", D, l + b);
            }
        }
    }
    for (int g = 0; g < kTileBytes; ++g) CHECK(phys[g] >= 0, "D=%d global byte %d never copied", D, g);

    Tl lanes[64];
    for (int lane = 0; lane < 64; ++lane) lanes[lane].init(lane);
    // row reads: lane (col, h) reads values 16 s + 8 h .. + 7 of row R + col
    for (int R = 0; R < 64; R += 32) {
        for (int s = 0; s < D / 16; ++s) {
            int addr[64];
            for (int lane = 0; lane < 64; ++lane) {
                const int col = lane & 31, h = lane >> 5;
                addr[lane] = 2 * (Tl::row_imm(R, s) + lanes[lane].row_off(s));
                for (int b = 0; b < 16; ++b)
                    CHECK(addr[lane] + b == phys[(R + col) * kRowBytes + 2 * (16 * s + 8 * h) + b],
                          "D=%d row read R=%d s=%d lane %d byte %d", D, R, s, lane, b);
            }
            for (int g0 = 0; g0 < 64; g0 += 16) {
                std::set<int> groups;
                for (int lane = g0; lane < g0 + 16; ++lane) groups.insert((addr[lane] / 16) % 16);
                CHECK(groups.size() == 16, "D=%d row read R=%d s=%d lanes %d..: %zu bank groups", D, R, s, g0,
                      groups.size());
            }
        }
    }
    // transposing reads: lane reads 4 values at row R + 4h + (lane % 16) / 4 + 8x, columns
    // 32 t + 16 ((lane / 16) % 2) + 4 (lane % 4)
    for (int R = 0; R < 64; R += 16) {
        for (int t = 0; t < D / 32; ++t) {
            for (int x = 0; x < 2; ++x) {
                int addr[64];
                for (int lane = 0; lane < 64; ++lane) {
                    const int h = lane >> 5, gi = lane & 15;
                    const int row = R + 4 * h + (gi >> 2) + 8 * x;
                    const int c = 32 * t + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
                    addr[lane] = 2 * (Tl::tr_imm(R, t, x) + lanes[lane].tr_off(t, x));
                    for (int b = 0; b < 8; ++b)
                        CHECK(addr[lane] + b == phys[row * kRowBytes + 2 * c + b],
                              "D=%d tr read R=%d t=%d x=%d lane %d byte %d", D, R, t, x, lane, b);
                }
                const int width = D == 128 ? 32 : 16;  // lanes per transfer checked
                for (int g0 = 0; g0 < 64; g0 += width) {
                    std::set<int> banks;
                    for (int lane = g0; lane < g0 + width; ++lane) {
                        banks.insert((addr[lane] / 4) % 64);
                        banks.insert((addr[lane] / 4 + 1) % 64);
                    }
                    CHECK(static_cast<int>(banks.size()) == 2 * width, "D=%d tr read R=%d t=%d x=%d lanes %d..: %zu banks",
                          D, R, t, x, g0, banks.size());
                }
            }
        }
    }
}

int main() {
    check_layout<128>();
    check_layout<64>();
    if (g_fail) {
        std::printf("%d failures\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
