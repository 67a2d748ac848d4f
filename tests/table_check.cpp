// Host-side checker of libzsp's offset tables: builds the piece and tile
// tables with the library's own host code (zsp_layout.cpp) and verifies
// every property the kernels' indexing relies on, so that no kernel can
// address memory outside its buffers. Input on stdin: nd rank T numel...
// [force] (rank -1 = all ranks; force = 1 builds span tables for any
// layout). Prints "ok <pieces> pieces <spans> spans" or the first violated
// property.
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

// Span tables: spans cover every tile in order within the limits, each
// rank run stays inside the source array, and the span gather's addressing
// -- run chunks into LDS, then per element its piece's offset, found as the
// kernel finds it -- reads, for every flat index K, source element
// K + delta(piece of K).
static int check_spans(const HostGatherTable& g, int64_t S, int64_t nd) {
    if (g.spans.empty()) {
        if (!g.span_runs.empty() || !g.span_segs.empty() || !g.tile_segs.empty())
            return bad("span parts without spans", 0, 0);
        return 0;
    }
    const int64_t total = g.total, ntile = (total + kTile - 1) / kTile;
    const int64_t C = kSpanChunkElems, src_elems = nd * S;
    const int64_t src_chunks = (src_elems + C - 1) / C;
    if (int64_t(g.tile_segs.size()) != ntile) return bad("tile_segs size", g.tile_segs.size(), ntile);
    int64_t next_tile = 0, runs = 0, segs = 0;
    std::vector<int64_t> lds_src;  // source element of each LDS element
    for (size_t i = 0; i < g.spans.size(); ++i) {
        const SpanRec& R = g.spans[i];
        if (R.k_a != next_tile * kTile) return bad("span start", int64_t(i), R.k_a);
        if (R.tiles < 1 || R.tiles > kSpanTiles) return bad("span tiles", int64_t(i), R.tiles);
        if (R.chunks < 1 || R.chunks > kSpanChunks) return bad("span chunks", int64_t(i), R.chunks);
        if (R.nseg < 1 || R.nseg > kSpanSegs) return bad("span pieces", int64_t(i), R.nseg);
        if (R.nrun < 1 || R.nrun > kSpanRuns) return bad("span runs", int64_t(i), R.nrun);
        if (R.run_first != runs || R.seg_first != segs) return bad("span table order", int64_t(i), R.run_first);
        runs += R.nrun;
        segs += R.nseg;
        if (runs > int64_t(g.span_runs.size()) || segs > int64_t(g.span_segs.size()))
            return bad("span tables short", runs, segs);
        next_tile += R.tiles;
        if (next_tile > ntile) return bad("spans past the last tile", int64_t(i), next_tile);
        // every span of a small table; of a large one the first and last
        // 512 and every seventh
        const size_t ns = g.spans.size();
        const bool full_check = ns <= 4096 || i < 512 || i + 512 >= ns || i % 7 == 0;
        lds_src.assign(size_t(R.chunks * C), -1);
        int32_t at = 0;
        for (int32_t q = 0; q < R.nrun; ++q) {
            const SpanRun& U = g.span_runs[size_t(R.run_first + q)];
            if (U.lds0 != at || U.nchunk < 1) return bad("run placement", q, U.lds0);
            if (U.chunk0 < 0 || U.chunk0 + U.nchunk > src_chunks) return bad("run outside source", q, U.chunk0);
            for (int64_t c = 0; c < U.nchunk; ++c)
                for (int64_t e = 0; e < C; ++e)
                    lds_src[size_t((at + c) * C + e)] = (U.chunk0 + c) * C + e;
            at += U.nchunk;
        }
        if (at != R.chunks) return bad("run chunks", int64_t(i), at);
        const SpanSeg* sg = &g.span_segs[size_t(R.seg_first)];
        for (int32_t j = 0; j < R.nseg; ++j) {
            if (sg[j].k < 0 || sg[j].k >= R.tiles * kTile) return bad("piece start", j, sg[j].k);
            if (j > 0 && sg[j].k <= sg[j - 1].k) return bad("pieces unordered", j, sg[j].k);
        }
        if (sg[0].k != 0) return bad("first piece of span", int64_t(i), sg[0].k);
        for (int32_t tau = 0; tau < R.tiles && full_check; ++tau) {
            const int64_t gt = R.k_a / kTile + tau;
            const int lo = int(g.tile_segs[size_t(gt)] & 0xffffu), hi = int(g.tile_segs[size_t(gt)] >> 16);
            if (lo > hi || hi >= R.nseg) return bad("tile pieces", gt, lo);
            const int64_t kl_last = std::min<int64_t>(total - R.k_a, R.tiles * kTile) - 1;
            for (int lane = 0; lane < kWaveLanes; ++lane) {
                const int64_t kl = int64_t(tau) * kTile + lane * C;
                // the kernel's search: binary over [lo, hi], then forward
                // (lanes past the end search from the last element)
                const int64_t kls = std::min(kl, kl_last);
                int s = lo;
                for (int h = hi; s < h;) {
                    const int mid = (s + h + 1) >> 1;
                    if (sg[mid].k <= kls) s = mid;
                    else h = mid - 1;
                }
                for (int64_t e = 0; e < C; ++e) {
                    const int64_t K = std::min(kl + e, kl_last);
                    while (s < hi && sg[s + 1].k <= K) ++s;
                    const int64_t pos = K + sg[s].off;
                    if (pos < 0 || pos >= int64_t(lds_src.size())) return bad("LDS index", R.k_a + K, pos);
                    const int64_t Kg = R.k_a + K;
                    const int64_t p = int64_t(std::upper_bound(g.k0.begin(), g.k0.end() - 1, Kg) -
                                              g.k0.begin()) - 1;
                    if (lds_src[size_t(pos)] != Kg + g.delta[size_t(p)])
                        return bad("span element source", Kg, lds_src[size_t(pos)]);
                }
            }
        }
    }
    if (next_tile != ntile) return bad("spans cover the tiles", next_tile, ntile);
    // device records: the same spans, packed as the kernel reads them; its
    // chunk-to-run choice (last run whose LDS start is at or below the chunk)
    // names the run holding every chunk
    if (g.wspans.size() != g.spans.size()) return bad("span records", g.wspans.size(), g.spans.size());
    for (size_t i = 0; i < g.spans.size(); ++i) {
        const SpanRec& R = g.spans[i];
        const WaveSpan& w = g.wspans[i];
        if (int64_t(w.tile0) * kTile != R.k_a || w.seg_first != R.seg_first ||
            w.chunks != R.chunks || w.nrun != R.nrun || w.nseg != R.nseg || w.ntile != R.tiles)
            return bad("span record header", int64_t(i), R.k_a);
        for (int32_t t = 0; t < R.tiles; ++t) {
            const uint32_t ts = g.tile_segs[size_t(R.k_a / kTile + t)];
            const uint32_t pair = w.tseg[t];
            if ((pair & 0xff) != (ts & 0xffffu) || (pair >> 8) != (ts >> 16))
                return bad("span record pieces", int64_t(i), t);
        }
        if (w.lds0[0] != 0) return bad("first run's LDS start", int64_t(i), w.lds0[0]);
        for (int32_t c = 0; c < R.chunks; ++c) {
            int64_t gd = w.chunk0;
            for (int q = 1; q < kSpanRuns && q < w.nrun; ++q)
                if (c >= w.lds0[q]) gd = w.chunk0 + w.dchunk[q - 1] - w.lds0[q];
            // the generic run holding chunk c
            int64_t want = -1;
            for (int32_t q = 0; q < R.nrun; ++q) {
                const SpanRun& U = g.span_runs[size_t(R.run_first + q)];
                if (c >= U.lds0 && c < U.lds0 + U.nchunk) want = U.chunk0 + (c - U.lds0);
            }
            if (c + gd != want) return bad("span record chunk", int64_t(i), c);
        }
    }
    if (runs != int64_t(g.span_runs.size()) || segs != int64_t(g.span_segs.size()))
        return bad("span tables long", runs, segs);
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
    long long nspan = 0;
    if (rank < 0) {
        HostGatherTable hg;
        build_gather_table(numel, sl, so, flo, S, int32_t(nd), hg);
        // span tables where the library builds them (short-piece layouts),
        // or of any layout when a nonzero value follows the sizes
        long long force = 0;
        if (std::scanf("%lld", &force) != 1) force = 0;
        if (force || wants_span_table(hg)) build_span_table(S, int32_t(nd), hg);
        if (check_spans(hg, S, nd)) return 1;
        nspan = (long long)hg.spans.size();
    }
    std::printf("ok %lld pieces %lld spans\n", (long long)np, nspan);
    return 0;
}
