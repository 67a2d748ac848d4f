// Host-side checker of libzsp's offset tables: builds the piece and tile
// tables with the library's own host code (zsp_layout.cpp) and verifies
// every property the kernels' indexing relies on, so that no kernel can
// address memory outside its buffers. Input on stdin: nd rank T numel...
// (rank -1 = all ranks). Prints "ok" or the first violated property.
#include <algorithm>
#include <cstdio>
#include <vector>

#include "zsp_internal.hpp"

using namespace zsp;

static int bad(const char* what, long long a, long long b) {
    std::printf("FAIL %s (%lld, %lld)\n", what, a, b);
    return 1;
}

static int check_tiles(const std::vector<int64_t>& starts, const std::vector<int32_t>& tile,
                       int64_t total) {
    const int64_t n = int64_t(starts.size()) - 1;
    if (total == 0) return tile.empty() ? 0 : bad("tile table for empty space", 0, 0);
    const int64_t ntile = (total + kTile - 1) / kTile;
    if (int64_t(tile.size()) != ntile + 1) return bad("tile size", tile.size(), ntile + 1);
    for (int64_t g = 0; g <= ntile; ++g) {
        const int64_t x = std::min(g * kTile, total - 1);
        const int64_t p = tile[g];
        if (p < 0 || p >= n) return bad("tile entry out of range", g, p);
        if (!(starts[p] <= x && x < starts[p + 1])) return bad("tile entry misses", g, p);
    }
    return 0;
}

int main() {
    long long nd, rank, T;
    if (std::scanf("%lld %lld %lld", &nd, &rank, &T) != 3) return 2;
    std::vector<int64_t> numel(T), pad(T), sl(T), fo(T + 1, 0), so(T + 1, 0), flo(T + 1, 0);
    for (long long t = 0; t < T; ++t) {
        long long x;
        if (std::scanf("%lld", &x) != 1) return 2;
        numel[t] = x;
        pad[t] = pad_for(x, int32_t(nd));
        sl[t] = (x + pad[t]) / nd;
        fo[t + 1] = fo[t] + x + pad[t];
        so[t + 1] = so[t] + sl[t];
        flo[t + 1] = flo[t] + x;
    }
    const int64_t S = so[T];
    HostShardTable hs;
    build_shard_table(numel, sl, fo, so, flo, S, int32_t(nd), int32_t(rank), hs);
    const int64_t np = int64_t(hs.info.size());
    const int64_t total = rank < 0 ? nd * S : S;
    if (hs.total != total) return bad("shard total", hs.total, total);
    if (int64_t(hs.e0.size()) != np + 1 || hs.e0[np] != total) return bad("sentinel", np, total);
    if (np > 0 && hs.e0[0] != 0) return bad("first piece start", hs.e0[0], 0);
    for (int64_t p = 0; p < np; ++p) {
        const PieceInfo& I = hs.info[p];
        if (hs.e0[p + 1] <= hs.e0[p]) return bad("empty or unordered piece", p, hs.e0[p]);
        if (I.end != hs.e0[p + 1]) return bad("piece end", p, I.end);
        if (I.vend < hs.e0[p] || I.vend > I.end) return bad("valid end", p, I.vend);
        if (I.vend > hs.e0[p]) {
            if (hs.e0[p] + I.gdelta < 0 || I.vend + I.gdelta > fo[T])
                return bad("gradient range", p, I.gdelta);
            if (hs.e0[p] + I.idelta < 0 || I.vend + I.idelta > flo[T])
                return bad("parameter range", p, I.idelta);
        }
    }
    if (check_tiles(hs.e0, hs.tile, total)) return 1;
    if (rank < 0) {
        HostGatherTable hg;
        build_gather_table(numel, sl, so, flo, S, int32_t(nd), hg);
        const int64_t nq = int64_t(hg.delta.size());
        if (hg.total != flo[T] || hg.k0[nq] != flo[T]) return bad("gather total", hg.total, flo[T]);
        for (int64_t q = 0; q < nq; ++q) {
            const int64_t a = hg.k0[q], b = hg.k0[q + 1];
            if (b <= a) return bad("empty gather piece", q, a);
            const int64_t r = (a + hg.delta[q]) / (S ? S : 1);
            if (a + hg.delta[q] < r * S || b + hg.delta[q] > (r + 1) * S)
                return bad("gather source leaves its rank", q, r);
        }
        if (nq > 0 && hg.k0[0] != 0) return bad("first gather piece", hg.k0[0], 0);
        if (check_tiles(hg.k0, hg.tile, hg.total)) return 1;
        // tile_delta[g]: the piece delta exactly when the full tile g lies
        // in one piece, else the marker
        const int64_t gt = hg.total == 0 ? 0 : (hg.total + kTile - 1) / kTile;
        if (int64_t(hg.tile_delta.size()) != gt) return bad("tile_delta size", hg.tile_delta.size(), gt);
        if (int64_t(hg.tile_pair.size()) != 3 * gt) return bad("tile_pair size", hg.tile_pair.size(), 3 * gt);
        for (int64_t g = 0; g < gt; ++g) {
            const int64_t a = g * kTile, b = a + kTile;
            const int64_t p = int64_t(std::upper_bound(hg.k0.begin(), hg.k0.end() - 1, a) -
                                      hg.k0.begin()) - 1;
            const bool one = b <= hg.total && b <= hg.k0[p + 1];
            const int64_t want = one ? hg.delta[p] : kNoTileDelta;
            if (hg.tile_delta[g] != want) return bad("tile_delta", g, hg.tile_delta[g]);
            // tile_pair: pieces holding the tile's first and last element
            const int64_t e = std::min(b, hg.total) - 1;
            const int64_t q = int64_t(std::upper_bound(hg.k0.begin(), hg.k0.end() - 1, e) -
                                      hg.k0.begin()) - 1;
            const int64_t* r = &hg.tile_pair[size_t(3 * g)];
            if (q - p >= 2) {
                if (r[0] != kNoTileDelta) return bad("tile_pair marker", g, r[0]);
            } else {
                const int64_t split = q > p ? hg.k0[q] : INT64_MAX;
                if (r[0] != split || r[1] != hg.delta[p] || r[2] != hg.delta[q])
                    return bad("tile_pair", g, r[0]);
            }
        }
    }
    std::printf("ok %lld pieces\n", (long long)np);
    return 0;
}
