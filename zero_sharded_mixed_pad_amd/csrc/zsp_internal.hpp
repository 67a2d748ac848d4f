// zsp_internal.hpp -- device-table formats and kernel launch interfaces
// shared by the host side (zsp_layout.cpp, zsp_capi.cpp) and the HIP kernels
// (zsp_kernels.hip) of libzsp.
#pragma once

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstdint>
#include <vector>

#include "zsp.h"

namespace zsp {

// Elements one wavefront handles per tile (64 lanes x 8 elements); the
// kernels launch one wavefront per workgroup. Offset tables are indexed at
// this granularity.
constexpr int64_t kTile = 512;
constexpr int kWaveLanes = 64;

// One piece of the shard index space ("E-space"): the run of elements of
// one rank's slice of one parameter. E-space is the index space of the bound
// state arrays (n_d*S for an all-rank binding, S for a one-rank binding).
// The piece covers [e0, end); [e0, vend) are real elements, [vend, end) pad.
// For an element e of the piece, its gradient in the full padded layout is
// at e + gdelta and its value in the unpadded flat parameter buffer at
// e + idelta.
struct PieceInfo {
    int64_t vend;
    int64_t end;
    int64_t gdelta;
    int64_t idelta;
};

// Device copy of a piece table: e0[np+1] (e0[np] = total), info[np], and
// tile[ntile+1] where tile[g] is the piece holding element
// min(g*kTile, total-1). Pieces are never empty.
struct ShardTable {
    const int64_t* e0 = nullptr;
    const PieceInfo* info = nullptr;
    const int32_t* tile = nullptr;
    int64_t np = 0;
    int64_t ntile = 0;
    int64_t total = 0;
};

// Device copy of the gather table over the unpadded flat index space
// ("K-space", parameter t at flat_off[t]): piece q is the run of parameter t
// held by one rank, starting at k0[q] (k0[nq] = total); element K of it
// reads source element K + delta[q] of the n_d*S shard arrays. tile[] as
// above.
struct GatherTable {
    const int64_t* k0 = nullptr;
    const int64_t* delta = nullptr;
    const int32_t* tile = nullptr;
    // per tile g: the delta of its piece when all kTile elements of the tile
    // lie in one piece, else kNoTileDelta (one lookup for the common tile)
    const int64_t* tile_delta = nullptr;
    // per tile g, three values at 3g: when the tile's elements lie in at most
    // two pieces, the start of the second (INT64_MAX if one) and the deltas
    // of the first and second; else kNoTileDelta first (short-piece gathers)
    const int64_t* tile_pair = nullptr;
    int64_t nq = 0;
    int64_t ntile = 0;
    int64_t total = 0;
    // Span tables of the bf16 work copy (NULL when the layout does not fit
    // them; see WaveSpan).
    const struct WaveSpan* spans = nullptr;
    const struct SpanSeg* span_segs = nullptr;
    int64_t nspan = 0;
};
constexpr int64_t kNoTileDelta = INT64_MIN;

// ---- Span gather of the bf16 work copy over short pieces -----------------
// A span is a run of consecutive whole tiles of K-space. For any run of
// consecutive flat indices, the elements that one rank holds lie in one
// contiguous range of its shard (a rank keeps its slices of consecutive
// parameters one after another), pad slots between them included. So one
// wave gathers a span: it reads each rank's range -- aligned 16-byte
// chunks, one run per rank -- into LDS, then writes the span's output with
// aligned 16-byte stores, taking each element from LDS at its piece's
// offset. The host cuts spans so that their tiles, runs, pieces and chunks
// fit the limits below; a layout in which one tile alone does not fit gets
// no span tables and gathers by tiles.
constexpr int kSpanTiles = 2;                        // tiles per span at most
constexpr int kSpanChunkElems = 8;                   // bf16 elements per chunk
constexpr int kSpanChunks = kSpanTiles * 64 + 32;    // 16-byte LDS chunks per span at most
constexpr int kSpanSegs = 128;                       // pieces meeting a span at most
constexpr int kSpanRuns = 8;                         // ranks with elements in a span at most

// Generic span tables (host side; also what the table checks read). One
// span: tiles [k_a / kTile, k_a / kTile + tiles); runs [run_first, run_first
// + nrun) and pieces [seg_first, seg_first + nseg); chunks = LDS chunks of
// all runs.
struct SpanRec {
    int64_t k_a;
    int32_t tiles;
    int32_t nrun;
    int32_t run_first;
    int32_t seg_first;
    int32_t nseg;
    int32_t chunks;
};

// One rank's range: source chunks [chunk0, chunk0 + nchunk) of the n_d*S
// work array (chunk c = elements 8c .. 8c+7) go to LDS chunks
// [lds0, lds0 + nchunk).
struct SpanRun {
    int64_t chunk0;
    int32_t lds0;
    int32_t nchunk;
};

// One piece meeting a span, in K order: it starts at span-local index k (0
// for a piece begun in an earlier span), and its element at span-local index
// x sits at LDS element x + off.
struct SpanSeg {
    int32_t k;
    int32_t off;
};

// The device record of one span (64 bytes, one scalar load): its first
// tile, its pieces' place in the SpanSeg table, run 0's first source chunk
// and every other run's as an offset from it, each run's first LDS chunk,
// per tile the first and last piece meeting it (span-local, first | last
// << 8), and the span's chunk, run, piece and tile counts.
struct WaveSpan {
    int64_t chunk0;
    int32_t tile0;
    int32_t seg_first;
    int32_t dchunk[kSpanRuns - 1];  // chunk0 of run q + 1 minus chunk0
    uint8_t lds0[kSpanRuns];        // lds0[0] = 0
    uint16_t tseg[kSpanTiles];
    uint8_t chunks;
    uint8_t nrun;
    uint8_t nseg;
    uint8_t ntile;
    uint32_t reserved;
};
static_assert(sizeof(WaveSpan) == 64, "span record is 64 bytes");
static_assert(kSpanSegs <= 255 && kSpanChunks <= 255, "span record field widths");


// Host-side tables before upload.
struct HostShardTable {
    std::vector<int64_t> e0;
    std::vector<PieceInfo> info;
    std::vector<int32_t> tile;
    int64_t total = 0;
};

struct HostGatherTable {
    std::vector<int64_t> k0;
    std::vector<int64_t> delta;
    std::vector<int32_t> tile;
    std::vector<int64_t> tile_delta;
    std::vector<int64_t> tile_pair;
    int64_t total = 0;
    // span tables (empty when the layout does not fit them)
    std::vector<SpanRec> spans;
    std::vector<SpanRun> span_runs;
    std::vector<SpanSeg> span_segs;
    std::vector<uint32_t> tile_segs;  // per tile: first | last piece << 16, span-local
    std::vector<WaveSpan> wspans;     // device records of the spans
};

// Kernel operations over E-space.
enum ShardOp : int {
    OP_COPYIN = 0,      // flat params -> master, work, m = v = 0
    OP_REDUCE_SET = 1,  // acc = sum_r grads
    OP_REDUCE_ACC = 2,  // acc = acc + sum_r grads
    OP_FUSED = 3,       // g = sum_r grads; Adam; cast
    OP_FUSED_ACC = 4,   // g = acc + sum_r grads; Adam; cast
    OP_ADAM = 5         // g = acc; Adam; cast
};

struct AdamScalars {
    float lr, b1, b2, eps;
    float omb1, omb2, bc1, bc2;
};

struct ShardLaunch {
    ShardTable tab;
    int64_t e_begin = 0;  // processed range of E-space
    int64_t e_end = 0;
    float* master = nullptr;
    float* m = nullptr;
    float* v = nullptr;
    uint16_t* work = nullptr;
    float* acc = nullptr;
    const void* src = nullptr;  // flat params (OP_COPYIN)
    AdamScalars hp{};
    int32_t nd = 0;
    int32_t shard_layout = 0;  // 1: grads indexed like E-space
    const void* const* grads = nullptr;  // host array of nd device pointers
    int64_t grad_len = 0;  // elements of each gradient buffer
    bool short_pieces = false;  // pieces in range average under kShortPiece elements
};

struct GatherLaunch {
    GatherTable tab;
    int64_t k_first = 0;  // first global flat index
    int64_t count = 0;    // elements to write
    const void* src = nullptr;
    void* out = nullptr;
    bool short_pieces = false;  // pieces average under kShortPiece elements
    // tab.tile_delta offset to the launch's first tile when k_first is a
    // multiple of kTile (local tile t is then global tile k_first/kTile + t),
    // else NULL
    const int64_t* tile_delta = nullptr;
    const int64_t* tile_pair = nullptr;  // tab.tile_pair likewise, or NULL
    // Span form (bf16, short pieces, tile-aligned k_first): spans
    // [span_first, span_first + nspan) of tab.spans cover the launch.
    int64_t span_first = -1;
    int64_t nspan = 0;
    int64_t src_elems = 0;  // elements of src (n_d*S)
};
// Range gathers of at least this many elements take the span form when
// they can (fewer leave too few spans to fill the chip).
constexpr int64_t kSpanMinElems = 64 * kTile;

// Below this average piece length (elements) a gather takes its short-piece
// form: shared boundary lines make up a few percent of the bytes or more.
constexpr int64_t kShortPiece = 4096;

// ---- Gather of a list of parameters into separate outputs ----------------
// The list's outputs are cut into tiles of kTile elements, each tile inside
// one output; the tiles of the list are numbered 0, 1, ... in list order.

// Device table, one record per parameter (all-rank bindings): where its
// slots start in a rank's shard, its shard length and its element count.
struct ParamInfo {
    int64_t shard_off;
    int64_t shard_len;
    int64_t numel;
    int64_t reserved;
};

// One output of a staged list, in device memory: the parameter, the output
// and the list tile its first element falls in. Parameters without
// elements are left out of the staged list, so tile0 strictly increases.
struct ListEntry {
    void* out;
    int32_t id;
    int32_t tile0;
};

// One output of a list short enough to travel in the kernel arguments.
struct ArgEntry {
    void* out;
    int64_t shard_off;
    int64_t shard_len;
    int64_t numel;
};
constexpr int kListArgMax = 64;

// Where one tile of a list gather reads and writes. Local element k of the
// tile (k < count) goes to out[k]. Two-piece tiles (split >= 0, shard length
// at least kTile, so the tile meets at most two ranks' slices): it comes
// from source element base + k, plus step when k >= split. Many-piece tiles
// (split = -shard length): from base + k + step * ((rem + k) / shard
// length), where rem is the tile's offset into the slice it starts in;
// count holds the element count in its low 16 bits and rem above them.
struct TileRec {
    void* out;
    int64_t base;
    int64_t step;
    int32_t split;
    int32_t count;
};

struct ListLaunch {
    const ParamInfo* params = nullptr;  // plan's device table
    int64_t S = 0;
    const void* src = nullptr;
    bool short_pieces = false;
    int64_t tiles = 0;  // tiles of the whole list
    // Argument form (tiles of every output from the arguments): n entries
    // and their first tiles (tile0[n] = tiles).
    int32_t n_args = 0;
    ArgEntry args[kListArgMax];
    int32_t arg_tile0[kListArgMax + 1];
    // Staged form: entries and the coarse index (entry of tile 64c, for
    // every c) in device memory, and a record area for up to rec_cap tiles;
    // the list is processed in chunks of rec_cap tiles (a multiple of 64).
    const ListEntry* ents = nullptr;
    int32_t n_ents = 0;
    const int32_t* coarse = nullptr;
    TileRec* recs = nullptr;
    int64_t rec_cap = 0;
    // Staged form only: 0, expand then gather, chunk by chunk; 1, expand
    // only (records of every tile, rec_cap >= tiles); 2, gather only, from
    // records built before (rec_cap >= tiles).
    int32_t mode = 0;
};

// Launch a list gather (argument form if n_args > 0, else staged); esz is
// the element size of src and the outputs (2: bf16, 4: fp32).
hipError_t launch_gather_list(const ListLaunch& L, int esz, hipStream_t stream);
// Copies `bytes` (a multiple of 16) from pinned host memory `src` to device
// memory `dst` with a kernel on `stream`; both 16-byte aligned.
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t stream);

// Launch one E-space operation; dtype is the gradient / parameter dtype.
hipError_t launch_shard_op(const ShardLaunch& L, ShardOp op, zsp_dtype dtype,
                           hipStream_t stream);
// Launch a gather; dtype is the element type of src/out.
hipError_t launch_gather(const GatherLaunch& L, zsp_dtype dtype, hipStream_t stream);

// Host layout helpers (zsp_layout.cpp).
int64_t pad_for(int64_t numel, int32_t nd);
void build_shard_table(const std::vector<int64_t>& numel, const std::vector<int64_t>& shard_len,
                       const std::vector<int64_t>& full_off,
                       const std::vector<int64_t>& shard_off,
                       const std::vector<int64_t>& flat_off, int64_t S, int32_t nd,
                       int32_t rank_or_all, HostShardTable& out);
void build_gather_table(const std::vector<int64_t>& numel,
                        const std::vector<int64_t>& shard_len,
                        const std::vector<int64_t>& shard_off,
                        const std::vector<int64_t>& flat_off, int64_t S, int32_t nd,
                        HostGatherTable& out);
void build_tile_index(const std::vector<int64_t>& starts, int64_t total,
                      std::vector<int32_t>& tile);
// A tile handed to build_spans: flat indices [K0, K0 + n).
struct SpanTileIn {
    int64_t K0;
    int64_t n;
};
// What build_spans makes: spans (k_a = the flat index of their first tile's
// first element, span-local indices counted from it), their runs and pieces,
// and per input tile the first and last piece meeting it (span-local, first
// | last << 16). Span i holds the tiles after those of spans 0 .. i-1.
struct SpanBuild {
    std::vector<SpanRec> spans;
    std::vector<SpanRun> runs;
    std::vector<SpanSeg> segs;
    std::vector<uint32_t> tile_segs;
};
// Spans over tiles in[0 .. n_in) of an n_d*S source (gather table k0,
// delta filled), at most max_tiles tiles each; a tile joins the span before
// it only when it starts where the previous tile ended. False when some tile
// alone exceeds the span limits (or a tile lies outside the flat indices).
bool build_spans(const HostGatherTable& g, int64_t S, int32_t nd, const SpanTileIn* in,
                 int64_t n_in, int32_t max_tiles, SpanBuild& out);
// Runs of a span in record form: run 0's first source chunk, the others' as
// offsets from it, and each run's first LDS chunk (0xff for none). False
// when an offset does not fit 32 bits.
bool pack_runs(const SpanRun* U, int32_t nrun, int64_t& chunk0,
               int32_t (&dchunk)[kSpanRuns - 1], uint8_t (&lds0)[kSpanRuns]);
// Span tables of the range gather from a gather table (k0, delta, tile
// filled) of an n_d*S source. Leaves them empty when some tile alone
// exceeds the span limits.
void build_span_table(int64_t S, int32_t nd, HostGatherTable& g);
// Whether a layout gets span tables: only layouts of short pieces, whose
// gathers take the span form.
bool wants_span_table(const HostGatherTable& g);

}  // namespace zsp
