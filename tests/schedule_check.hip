// Host-only check of the kernels' workgroup -> tile schedules (fa_schedule.hpp).
//
// For each grid shape it walks every workgroup index the way the kernels do
// and counts how often each tile is issued.  A tile issued twice would be
// computed twice (and raced on); a tile never issued leaves its output
// unwritten.  Prints "ok <shapes>" and exits 0, or the first failure and 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fa_schedule.hpp"

using namespace fa;

static int g_fail = 0;
static long g_shapes = 0;

#define CHECK(cond, ...)                                         \
    do {                                                         \
        if (!(cond)) {                                           \
            if (!g_fail) {                                       \
                std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
                std::printf(__VA_ARGS__);                        \
                std::printf("\n");                               \
            }                                                    \
            g_fail = 1;                                          \
            return;                                              \
        }                                                        \
    } while (0)

// Dense forward (one query-tile count for every head), as the forward kernel
// decodes its workgroup index: split tail when the host grid has one, else
// the plain unit schedule; pairs under causal masking.
static void dense_fwd(int heads, int n_qt, bool causal) {
    ++g_shapes;
    int per_head = n_qt, tail = 0;
    int64_t units = (int64_t)heads * n_qt;
    if (causal) {
        const FwdGrid g = fwd_causal_grid(heads, n_qt);
        per_head = (n_qt + 1) / 2;
        tail = g.tail;
        units = g.units;
        CHECK(tail == 0 || (heads % 8 == 0 && tail <= heads / 8),
              "heads %d n_qt %d: tail %d", heads, n_qt, tail);
    }
    std::vector<int> count((size_t)heads * n_qt, 0);
    std::vector<int> last_single(8, 1 << 30);  // per XCD, heaviest first
    for (int64_t i = 0; i < units; ++i) {
        int head, uidx, rank = -1;
        if (tail > 0)
            tail_unit((int)i, heads, per_head, tail, head, uidx, rank);
        else
            unit_of((int)i, (int)units, per_head, head, uidx);
        CHECK(head >= 0 && head < heads, "heads %d n_qt %d causal %d: wg %lld -> head %d",
              heads, n_qt, causal, (long long)i, head);
        if (heads % 8 == 0)
            CHECK(head % 8 == (int)(i % 8), "heads %d: wg %lld on XCD %d got head %d", heads,
                  (long long)i, (int)(i % 8), head);
        int t0, t1;
        // every unit of a dense grid has work: no workgroup slot is wasted
        CHECK(fwd_tiles(causal, rank, uidx, n_qt, t0, t1),
              "heads %d n_qt %d causal %d: wg %lld empty", heads, n_qt, causal, (long long)i);
        CHECK(t0 >= 0 && t0 < n_qt && t1 >= -1 && t1 < n_qt, "tile out of range");
        ++count[(size_t)head * n_qt + t0];
        if (t1 >= 0) {
            CHECK(t0 + t1 == n_qt - 1 && t0 > t1, "pair (%d, %d) of %d", t0, t1, n_qt);
            ++count[(size_t)head * n_qt + t1];
        }
        if (rank >= 0) {
            CHECK(t0 <= last_single[i % 8], "tail not heaviest first on XCD %d",
                  (int)(i % 8));
            last_single[i % 8] = t0;
        }
    }
    for (int h = 0; h < heads; ++h)
        for (int t = 0; t < n_qt; ++t)
            CHECK(count[(size_t)h * n_qt + t] == 1,
                  "heads %d n_qt %d causal %d: head %d tile %d issued %d times", heads, n_qt,
                  causal, h, t, count[(size_t)h * n_qt + t]);
}

// Packed sequences: per_head from the longest sequence, each head's own
// tile count decides which units have work.
static void varlen_fwd(const std::vector<int>& tiles, int H, bool causal) {
    ++g_shapes;
    const int nseq = (int)tiles.size(), heads = nseq * H;
    int n_max = 0;
    for (int t : tiles) n_max = t > n_max ? t : n_max;
    if (n_max == 0) return;  // the host launches nothing
    const int per_head = causal ? (n_max + 1) / 2 : n_max;
    const int units = heads * per_head;
    std::vector<std::vector<int>> count(heads);
    for (int hd = 0; hd < heads; ++hd) count[hd].assign(tiles[hd / H], 0);
    for (int i = 0; i < units; ++i) {
        int head, uidx;
        unit_of(i, units, per_head, head, uidx);
        CHECK(head >= 0 && head < heads && uidx >= 0, "varlen head %d", head);
        const int n = tiles[head / H];
        int t0, t1;
        if (!fwd_tiles(causal, -1, uidx, n, t0, t1)) continue;
        CHECK(t0 >= 0 && t0 < n && t1 >= -1 && t1 < n, "varlen tile out of range");
        ++count[head][t0];
        if (t1 >= 0) ++count[head][t1];
    }
    for (int hd = 0; hd < heads; ++hd)
        for (int t = 0; t < tiles[hd / H]; ++t)
            CHECK(count[hd][t] == 1, "varlen head %d tile %d issued %d times", hd, t,
                  count[hd][t]);
}

// Split keys: unit = (query tile, key range); no pairing, no tail.
static void split_fwd(int heads, int n_qt, int splits) {
    ++g_shapes;
    const int per_head = n_qt * splits, units = heads * per_head;
    std::vector<int> count((size_t)heads * n_qt * splits, 0);
    for (int i = 0; i < units; ++i) {
        int head, uidx;
        unit_of(i, units, per_head, head, uidx);
        CHECK(head >= 0 && head < heads && uidx >= 0 && uidx < per_head, "split unit range");
        const int split = uidx % splits;
        uidx /= splits;
        int t0, t1;
        CHECK(fwd_tiles(false, -1, uidx, n_qt, t0, t1) && t1 == -1, "split unit empty");
        CHECK(t0 >= 0 && t0 < n_qt, "split tile out of range");
        ++count[((size_t)head * n_qt + t0) * splits + split];
    }
    for (size_t c = 0; c < count.size(); ++c)
        CHECK(count[c] == 1, "split heads %d n_qt %d splits %d: slot %zu issued %d times",
              heads, n_qt, splits, c, count[c]);
}

// Backward passes: dK/dV over key tiles (light tile first), dQ over query
// tiles (heavy first); pairs under causal masking.
static void bwd_pass(int heads, int n_tiles, bool causal, bool heavy_first) {
    ++g_shapes;
    const int per_head = causal ? (n_tiles + 1) / 2 : n_tiles;
    const int units = heads * per_head;
    std::vector<int> count((size_t)heads * n_tiles, 0);
    for (int i = 0; i < units; ++i) {
        int head, uidx;
        unit_of(i, units, per_head, head, uidx);
        CHECK(head >= 0 && head < heads, "bwd head %d of %d", head, heads);
        int t0, t1;
        CHECK(unit_tiles(causal, heavy_first, uidx, n_tiles, t0, t1), "bwd unit empty");
        CHECK(t0 >= 0 && t0 < n_tiles && t1 >= -1 && t1 < n_tiles, "bwd tile out of range");
        if (t1 >= 0) CHECK((t0 > t1) == heavy_first, "bwd pair order (%d, %d)", t0, t1);
        ++count[(size_t)head * n_tiles + t0];
        if (t1 >= 0) ++count[(size_t)head * n_tiles + t1];
    }
    for (size_t c = 0; c < count.size(); ++c)
        CHECK(count[c] == 1, "bwd heads %d tiles %d causal %d: tile %zu issued %d times", heads,
              n_tiles, causal, c, count[c]);
}

// Decoding: one workgroup per (head, key range).
static void decode(int heads, int splits) {
    ++g_shapes;
    const int units = heads * splits;
    std::vector<int> count((size_t)units, 0);
    for (int i = 0; i < units; ++i) {
        int head, split;
        unit_of(i, units, splits, head, split);
        CHECK(head >= 0 && head < heads && split >= 0 && split < splits, "decode range");
        ++count[(size_t)head * splits + split];
    }
    for (int c : count) CHECK(c == 1, "decode heads %d splits %d", heads, splits);
}

int main() {
    for (int heads = 1; heads <= 96; ++heads)
        for (int n_qt = 1; n_qt <= 80; ++n_qt)
            for (int causal = 0; causal < 2; ++causal) dense_fwd(heads, n_qt, causal != 0);
    // the measured shapes: B4 H32 N4096, B1 H32 N65536, B16 H32 N8192 (tiles of 128)
    dense_fwd(128, 32, true);
    dense_fwd(32, 512, true);
    dense_fwd(512, 64, true);
    dense_fwd(1024, 8, true);

    std::srand(7);
    for (int trial = 0; trial < 400; ++trial) {
        const int nseq = 1 + std::rand() % 20, H = 1 + std::rand() % 9;
        std::vector<int> tiles(nseq);
        for (int& t : tiles) t = std::rand() % 70;  // zero-length sequences included
        varlen_fwd(tiles, H, trial & 1);
    }
    for (int heads = 1; heads <= 40; ++heads)
        for (int n_qt = 1; n_qt <= 12; ++n_qt)
            for (int splits = 1; splits <= 9; ++splits) split_fwd(heads, n_qt, splits);
    for (int heads = 1; heads <= 72; ++heads)
        for (int n_tiles = 1; n_tiles <= 70; ++n_tiles)
            for (int causal = 0; causal < 2; ++causal) {
                bwd_pass(heads, n_tiles, causal != 0, false);
                bwd_pass(heads, n_tiles, causal != 0, true);
            }
    for (int heads = 1; heads <= 300; ++heads)
        for (int splits = 1; splits <= 130; splits += 3) decode(heads, splits);

    if (g_fail) return 1;
    std::printf("ok %ld\n", g_shapes);
    return 0;
}
