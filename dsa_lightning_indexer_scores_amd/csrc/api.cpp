// C ABI of the IndexCache hot path: argument validation, workspace sizing,
// the F/S layer-stack driver (prefill and decode) and the index cache.
//
// Stack semantics ("Indexcache Sparse Attention Acceleration", Step 3, and
// "When the Optimizer Becomes the Bottleneck", "The Redundancy That Was
// Sitting There"): an F layer computes fresh top-k indices and overwrites the
// one cached index tensor; an S layer reuses whatever the nearest preceding F
// layer left there; an S layer with nothing cached is an error; the cache is
// per call (cleared between sequences, as the skill page's Common Pitfalls
// ask).  The per-layer branch is the only difference between F and S layers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/indexcache.h"
#include "common.h"

namespace {

thread_local std::string g_err;
thread_local ic_stats g_stats = {0, 0, 0, 0};

constexpr int kDefaultChunk = 4096;
constexpr int kMaxK = 4096;

ic_status fail(ic_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ic_status fail(ic_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

ic_status hip_fail(hipError_t e, const char* what) {
    return fail(IC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int chunk_of(const ic_shape& s) { return s.chunk == 0 ? kDefaultChunk : s.chunk; }

// A second stream per device, at the default priority, for work that overlaps the
// caller's stream inside one call: an F layer's attention over a finished score tile runs
// there while the next tile is scored.  Created on first use, kept until the process ends.
// Concurrent calls on one device share it, which can only add waiting, never reorder a
// call's own work (each call forks and joins through its own events).  nullptr if it
// cannot be created; the caller then keeps everything on its own stream.
hipStream_t side_stream() {
    static std::mutex mu;
    static hipStream_t streams[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!streams[dev]) {
        hipStream_t h = nullptr;
        if (hipStreamCreateWithFlags(&h, hipStreamNonBlocking) != hipSuccess) return nullptr;
        streams[dev] = h;
    }
    return streams[dev];
}

// The F layer's own attention, run tile by tile on the side stream as the tiles' top-k
// rows land (tile t's attention overlaps tile t + 1's scoring).  With a second score
// tile, tile t's top-k runs there too: the caller's stream scores tile t + 1 into the
// other buffer meanwhile, and waits only for the top-k of tile t - 1 (which read that
// buffer) before doing so.
struct TileAttn {
    const void* q;          // the layer's q [B, Lq, H, d]
    const void* kv;         // kv [B, Lk, 2, d]
    void* out;              // out [B, Lq, H, d]
    hipStream_t side;
    hipEvent_t fork;
    float* tile2;           // second score tile, or nullptr (top-k on the caller's stream)
    hipEvent_t freed[2];    // recorded on the side stream after the top-k reading buffer i
    int64_t* ntiles;        // tiles scored so far in the call (buffer parity)
    bool* forked;           // set once any work of the call went to the side stream
};

// One stack call's use of the side stream: an F layer's tile attentions (and, with room for
// two score tiles in the workspace, its tile top-k) run there, forked from the caller's
// stream by events of the call's own; join() makes the caller's stream wait for them.  The
// caller joins after every F layer and on every return once work went there (an error
// part-way through a layer included), so no work of the call is left running unordered
// with its stream.
class SideWork {
public:
    // ws / ws_bytes: the call's workspace; tile_bytes: one score tile (a second one after it
    // moves the tile top-k to the side stream as well; tile_bytes 0: never a second tile)
    SideWork(void* ws, size_t ws_bytes, size_t tile_bytes) {
        side_ = side_stream();
        for (int i = 0; side_ && i < 4; ++i)
            if (hipEventCreateWithFlags(&ev_[i], hipEventDisableTiming) != hipSuccess) side_ = nullptr;
        tile2_ = side_ && tile_bytes > 0 && ws_bytes >= 2 * tile_bytes
                     ? reinterpret_cast<float*>(static_cast<char*>(ws) + tile_bytes) : nullptr;
    }
    ~SideWork() {
        for (int i = 0; i < 4; ++i)
            if (ev_[i]) (void)hipEventDestroy(ev_[i]);
    }
    SideWork(const SideWork&) = delete;
    SideWork& operator=(const SideWork&) = delete;
    bool active() const { return side_ != nullptr; }
    // the F layer's tile-attention hand-off, or nullptr to keep everything on the caller's stream
    const TileAttn* tile_attn(const ic_layer& L) {
        if (!side_) return nullptr;
        ta_ = {L.q, L.kv, L.out, side_, ev_[0], tile2_, {ev_[2], ev_[3]}, &ntiles_, &forked_};
        return &ta_;
    }
    hipError_t join(hipStream_t st) {
        if (!forked_) return hipSuccess;
        forked_ = false;
        hipError_t e = hipEventRecord(ev_[1], side_);
        return e == hipSuccess ? hipStreamWaitEvent(st, ev_[1], 0) : e;
    }

private:
    hipStream_t side_ = nullptr;
    hipEvent_t ev_[4] = {nullptr, nullptr, nullptr, nullptr};   // fork, join, two tile-freed events
    float* tile2_ = nullptr;
    int64_t ntiles_ = 0;
    bool forked_ = false;
    TileAttn ta_{};
};

// Sizes the kernels support; `decode` relaxes the prefill position checks, and `varlen`
// leaves them to the per-sequence check (Lq is then the packed query count).
ic_status check_shape(const ic_shape* sp, bool need_indexer, bool decode, bool varlen = false) {
    if (!sp) return fail(IC_ERR_ARG, "shape is NULL");
    const ic_shape& s = *sp;
    if (s.B < 1 || s.Lq < 1 || s.Lk < 1) return fail(IC_ERR_SHAPE, "B, Lq, Lk must be >= 1 (got %d, %d, %d)", s.B, s.Lq, s.Lk);
    // query rows are grid and row indices of 32 bits in the kernels
    if ((int64_t)s.B * s.Lq > INT32_MAX)
        return fail(IC_ERR_SHAPE, "B x Lq (%lld query rows) exceeds 2^31 - 1", (long long)s.B * s.Lq);
    if (decode) {
        if (s.Lq != 1) return fail(IC_ERR_SHAPE, "decode needs Lq == 1 (got %d)", s.Lq);
    } else if (varlen) {
        if (s.pos0 != 0) return fail(IC_ERR_SHAPE, "ragged prefill takes per-sequence pos0; shape.pos0 must be 0");
    } else {
        if (s.pos0 < 0) return fail(IC_ERR_SHAPE, "pos0 must be >= 0 (got %d)", s.pos0);
        if ((int64_t)s.pos0 + s.Lq > s.Lk)
            return fail(IC_ERR_SHAPE, "pos0 + Lq (%lld) exceeds Lk (%d)", (long long)s.pos0 + s.Lq, s.Lk);
    }
    if (s.k < 1 || s.k > kMaxK) return fail(IC_ERR_SHAPE, "k must be in 1..%d (got %d)", kMaxK, s.k);
    if (s.H < 1 || s.H > 4096) return fail(IC_ERR_SHAPE, "H must be in 1..4096 (got %d)", s.H);
    if (s.d != 64 && s.d != 128) return fail(IC_ERR_SHAPE, "d must be 64 or 128 (got %d)", s.d);
    // the gather kernels address a sequence's KV rows with 32-bit byte offsets
    if ((int64_t)s.Lk * 4 * s.d > (int64_t)UINT32_MAX)
        return fail(IC_ERR_SHAPE, "Lk (%d) x %d-byte KV rows exceeds 4 GiB per sequence", s.Lk, 4 * s.d);
    if (need_indexer) {
        if (s.idx_dtype != IC_BF16 && s.idx_dtype != IC_FP8_E4M3)
            return fail(IC_ERR_DTYPE, "idx_dtype must be IC_BF16 or IC_FP8_E4M3 (got %d)", s.idx_dtype);
        if (s.H_I < 1 || s.H_I > 64) return fail(IC_ERR_SHAPE, "H_I must be in 1..64 (got %d)", s.H_I);
        if (s.d_I != 32 && s.d_I != 64 && s.d_I != 128)
            return fail(IC_ERR_SHAPE, "d_I must be 32, 64 or 128 (got %d)", s.d_I);
        if (s.chunk != 0 && (s.chunk < 16 || s.chunk > 65536 || s.chunk % 16 != 0))
            return fail(IC_ERR_SHAPE, "chunk must be 0 or a multiple of 16 in 16..65536 (got %d)", s.chunk);
    }
    return IC_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Score tile of the prefill indexer: chunk rows x (pos0 + Lq) columns, fp32.
size_t indexer_ws(const ic_shape& s) {
    const int64_t rows = std::min<int64_t>(chunk_of(s), s.Lq);
    return (size_t)round_up(rows * round_up((int64_t)s.pos0 + s.Lq, 4) * 4, 256);
}

// Ragged prefill: a tile for any one sequence (<= chunk rows x <= Lk columns).
size_t indexer_ws_varlen(const ic_shape& s) {
    const int64_t rows = std::min<int64_t>(chunk_of(s), s.Lq);
    return (size_t)round_up(rows * round_up((int64_t)s.Lk, 4) * 4, 256);
}

// Key splits per decode query: about 1024 waves in all (one per SIMD; more splits
// only add partials for the combine to merge, fewer leave CUs idle), at most one
// 32-row tile per split, and a multiple of 4 (a workgroup merges 4 splits).
int decode_splits(const ic_shape& s) {
    const int64_t groups = (int64_t)s.B * ((s.H + 15) / 16);   // (query, head group) pairs
    const int want = (int)((1024 + groups - 1) / groups);
    const int tiles = (s.k + 31) / 32;
    const int ns = std::min(want, tiles);
    return ns < 4 ? 1 : ns / 4 * 4;
}

// Decode workspace: scores [B, round_up(Lk, 4)] fp32 | attention partials | top-k
// candidates (segmented top-k of long rows; cand_off == 0 when not used).
struct DecodeWs {
    int64_t score_stride;
    size_t scores_off, part_off, cand_off, total;
};
DecodeWs decode_layout(const ic_shape& s) {
    DecodeWs w;
    w.score_stride = round_up(s.Lk, 4);                   // 16-byte rows for the top-k's vector loads
    w.scores_off = 0;
    w.part_off = (size_t)round_up((int64_t)s.B * w.score_stride * 4, 256);
    const size_t cand_at = w.part_off + (size_t)round_up(sparse_attn_ws_bytes(s.B, s.H, s.d, decode_splits(s)), 256);
    ic_topk_args t{};
    t.rows = s.B;
    t.k = s.k;
    t.max_len = s.Lk;
    const size_t cand_bytes = topk_ws_bytes(t);
    w.cand_off = cand_bytes ? cand_at : 0;
    w.total = cand_at + (size_t)round_up((int64_t)cand_bytes, 256);
    return w;
}
size_t decode_ws(const ic_shape& s) { return decode_layout(s).total; }

// Dynamic refresh: the indexer tile, then the probe's region: scores [P, round_up(pos0 + Lq, 4)]
// fp32 | own top-k [P, k] int32 | intersections [P] int32 | refresh flag.
struct DynWs {
    int P;
    int t0;                       // first probe query
    int64_t score_stride;
    size_t probe_scores_off, probe_idx_off, inter_off, flag_off, total;
};
DynWs dyn_layout(const ic_shape& s, int stride) {
    DynWs d;
    d.t0 = (s.Lq - 1) % stride;
    d.P = (s.Lq - 1 - d.t0) / stride + 1;
    d.score_stride = round_up((int64_t)s.pos0 + s.Lq, 4);
    d.probe_scores_off = (size_t)round_up((int64_t)indexer_ws(s), 256);
    d.probe_idx_off = d.probe_scores_off + (size_t)round_up((int64_t)d.P * d.score_stride * 4, 256);
    d.inter_off = d.probe_idx_off + (size_t)round_up((int64_t)d.P * s.k * 4, 256);
    d.flag_off = d.inter_off + (size_t)round_up((int64_t)d.P * 4, 256);
    d.total = d.flag_off + 256;
    return d;
}

ic_status check_ws(const void* ws, size_t have, size_t need) {
    if (need == 0) return IC_OK;
    if (!ws) return fail(IC_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(IC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (have < need) return fail(IC_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    return IC_OK;
}

size_t elem_bytes(int dtype) { return dtype == IC_FP8_E4M3 ? 1 : 2; }

// Tensor pointers must be aligned to what the kernels load at once: 16 bytes for q_I, k_I,
// q, kv and out (vector and LDS-DMA loads of row pieces), 4 bytes for the fp32 and int32
// arrays.  Every torch allocation is; a view starting at an odd element may not be.  NULL
// entries are left to the callers' own checks.
struct AlignReq {
    const void* p;
    const char* name;
    unsigned align;
};
ic_status check_aligned(std::initializer_list<AlignReq> reqs) {
    for (const AlignReq& a : reqs)
        if (a.p && reinterpret_cast<uintptr_t>(a.p) % a.align != 0)
            return fail(IC_ERR_ARG, "%s must be %u-byte aligned", a.name, a.align);
    return IC_OK;
}

// a1 + a2 for one sequence: its Lq queries at positions pos0.. against its keys, in score
// tiles of <= chunk queries, then top-k into idx [Lq, k].
ic_status run_indexer_topk_one(const ic_shape& s, int Lq, int pos0, const uint8_t* qb, const float* wb,
                               const uint8_t* kb, int32_t* idx, void* ws, hipStream_t st, int64_t* tiles,
                               const int32_t* run_if = nullptr, const TileAttn* ta = nullptr, int b = 0) {
    const int chunk = chunk_of(s);
    const bool two = ta && ta->tile2;                       // top-k and attention both on the side stream
    // Tiles are independent, so they run last first: the work left after the final tile is
    // scored (that tile's top-k and attention) is then the shortest rows' (stack32k,
    // alternating runs, identical indices: 37.3-37.6 against 37.6-38.1 ms per step).
    const int nchunks = (int)(((int64_t)Lq + chunk - 1) / chunk);
    for (int ci = nchunks - 1; ci >= 0; --ci) {
        const int c0 = ci * chunk;
        const int nq = std::min(chunk, Lq - c0);
        const int64_t stride = round_up((int64_t)pos0 + c0 + nq, 4);
        float* tile = static_cast<float*>(ws);
        hipError_t e;
        const int64_t n = two ? (*ta->ntiles)++ : 0;        // this tile's number in the call
        if (two) {
            if (n & 1) tile = ta->tile2;
            if (n >= 2 && (e = hipStreamWaitEvent(st, ta->freed[n & 1], 0)) != hipSuccess)
                return hip_fail(e, "stream wait");           // tile n - 2's top-k read this buffer
        }
        ic_indexer_args a;
        a.q_I = qb;
        a.w = wb;
        a.k_I = kb;
        a.scores = tile;
        a.row_stride = stride;
        a.q_begin = c0;
        a.nq = nq;
        a.pos_begin = pos0 + c0;
        a.H_I = s.H_I;
        a.d_I = s.d_I;
        a.fp8 = s.idx_dtype == IC_FP8_E4M3;
        a.run_if = run_if;
        e = launch_indexer_prefill(a, st);
        if (e != hipSuccess) return hip_fail(e, "indexer launch");
        ic_topk_args t;
        t.run_if = run_if;
        t.scores = tile;
        t.row_stride = stride;
        t.rows = nq;
        t.first_len = pos0 + c0 + 1;
        t.seq_len = nullptr;
        t.k = s.k;
        t.idx = idx + (size_t)c0 * s.k;
        t.max_len = pos0 + c0 + nq;
        t.cand = nullptr;
        // fork to the side stream once the work it depends on is enqueued: the scores
        // (two tiles: the top-k goes there too) or the top-k rows (one tile)
        auto fork = [&]() -> hipError_t {
            hipError_t r = hipEventRecord(ta->fork, st);
            if (r == hipSuccess) r = hipStreamWaitEvent(ta->side, ta->fork, 0);
            if (r == hipSuccess) *ta->forked = true;
            return r;
        };
        if (two && (e = fork()) != hipSuccess) return hip_fail(e, "stream fork");
        e = launch_topk(t, two ? ta->side : st);
        if (e != hipSuccess) return hip_fail(e, "top-k launch");
        if (two && (e = hipEventRecord(ta->freed[n & 1], ta->side)) != hipSuccess)
            return hip_fail(e, "event record");
        if (tiles) ++*tiles;
        if (ta) {                                           // this tile's attention, on the side stream
            if (!two && (e = fork()) != hipSuccess) return hip_fail(e, "stream fork");
            const size_t row = (size_t)s.H * s.d;          // bf16 elements per query row
            ic_attn_args at;
            at.q = static_cast<const uint16_t*>(ta->q) + ((size_t)b * s.Lq + c0) * row;
            at.kv = static_cast<const uint16_t*>(ta->kv) + (size_t)b * s.Lk * 2 * s.d;
            at.idx = t.idx;
            at.out = static_cast<uint16_t*>(ta->out) + ((size_t)b * s.Lq + c0) * row;
            at.kv_seq_stride = (int64_t)s.Lk * 2 * s.d;
            at.Lk = s.Lk;
            at.nq = nq;
            at.q_per_seq = nq;
            at.H = s.H;
            at.d = s.d;
            at.k = s.k;
            at.nsplit = 1;
            at.ws = nullptr;
            if ((e = launch_sparse_attn(at, ta->side)) != hipSuccess) return hip_fail(e, "sparse attention launch");
        }
    }
    return IC_OK;
}

// a1 + a2 for every sequence of the call (all with Lq queries at pos0).
ic_status run_indexer_topk(const ic_shape& s, const void* q_I, const float* w, const void* k_I, int32_t* idx,
                           void* ws, hipStream_t st, int64_t* tiles, const TileAttn* ta = nullptr) {
    const size_t eb = elem_bytes(s.idx_dtype);
    for (int b = 0; b < s.B; ++b) {
        const uint8_t* qb = static_cast<const uint8_t*>(q_I) + (size_t)b * s.Lq * s.H_I * s.d_I * eb;
        const float* wb = w + (size_t)b * s.Lq * s.H_I;
        const uint8_t* kb = static_cast<const uint8_t*>(k_I) + (size_t)b * s.Lk * s.d_I * eb;
        ic_status r = run_indexer_topk_one(s, s.Lq, s.pos0, qb, wb, kb, idx + (size_t)b * s.Lq * s.k, ws, st, tiles,
                                           nullptr, ta, b);
        if (r != IC_OK) return r;
    }
    return IC_OK;
}

ic_status run_attn(const ic_shape& s, int nq_per_seq, const void* q, const void* kv, const int32_t* idx, void* out,
                   int nsplit, float* part, hipStream_t st) {
    ic_attn_args a;
    a.q = q;
    a.kv = kv;
    a.idx = idx;
    a.out = out;
    a.kv_seq_stride = (int64_t)s.Lk * 2 * s.d;
    a.Lk = s.Lk;
    a.nq = s.B * nq_per_seq;
    a.q_per_seq = nq_per_seq;
    a.H = s.H;
    a.d = s.d;
    a.k = s.k;
    a.nsplit = nsplit;
    a.ws = part;
    hipError_t e = launch_sparse_attn(a, st);
    if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
    return IC_OK;
}

// Pattern check shared by prefill and decode: charset, length, S before any F.
ic_status check_stack(const char* pattern, int32_t n_layers, const ic_layer* layers) {
    if (!pattern) return fail(IC_ERR_ARG, "pattern is NULL");
    if (n_layers < 1) return fail(IC_ERR_ARG, "n_layers must be >= 1 (got %d)", n_layers);
    if (!layers) return fail(IC_ERR_ARG, "layers is NULL");
    const size_t len = strnlen(pattern, (size_t)n_layers + 1);
    if (len != (size_t)n_layers)
        return fail(IC_ERR_PATTERN, "pattern length %zu != n_layers %d", len, n_layers);
    bool cached = false;
    for (int l = 0; l < n_layers; ++l) {
        const char c = pattern[l];
        const bool full = (c == 'F' || c == '1');
        if (!full && c != 'S' && c != '0')
            return fail(IC_ERR_PATTERN, "pattern[%d] = '%c' is not one of F, S, 1, 0", l, c);
        if (!full && !cached)
            return fail(IC_ERR_NO_CACHED_INDICES, "no cached indices: layer %d is S and no F layer precedes it", l);
        if (full) {
            cached = true;
            if (!layers[l].q_I || !layers[l].w || !layers[l].k_I)
                return fail(IC_ERR_ARG, "F layer %d needs q_I, w and k_I", l);
        }
        if (!layers[l].q || !layers[l].kv || !layers[l].out)
            return fail(IC_ERR_ARG, "layer %d needs q, kv and out", l);
        const ic_layer& L = layers[l];
        if (ic_status r = check_aligned({{L.q_I, "q_I", 16}, {L.k_I, "k_I", 16}, {L.w, "w", 4}, {L.q, "q", 16},
                                         {L.kv, "kv", 16}, {L.out, "out", 16}}))
            return r;
    }
    return IC_OK;
}

// The decode step once its arguments are validated; ws holds decode_ws(shape) bytes.
ic_status decode_step_run(const char* pattern, int32_t n_layers, const ic_layer* layers, const ic_shape& s,
                          const int32_t* seq_len, int32_t* idx_cache, void* ws, ic_stats* stats, hipStream_t st) {
    ic_status r = IC_OK;
    const DecodeWs lay = decode_layout(s);
    float* scores = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.scores_off);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.part_off);
    const int nsplit = decode_splits(s);
    ic_stats cnt = {0, 0, 0, 0};
    bool cached = false;
    for (int l = 0; l < n_layers; ++l) {
        const ic_layer& L = layers[l];
        if (pattern[l] == 'F' || pattern[l] == '1') {
            ic_indexer_decode_args a;
            a.q_I = L.q_I;
            a.w = L.w;
            a.k_I = L.k_I;
            a.seq_len = seq_len;
            a.scores = scores;
            a.score_stride = lay.score_stride;
            a.B = s.B;
            a.Lk = s.Lk;
            a.H_I = s.H_I;
            a.d_I = s.d_I;
            a.fp8 = s.idx_dtype == IC_FP8_E4M3;
            hipError_t e = launch_indexer_decode(a, st);
            if (e != hipSuccess) return hip_fail(e, "decode indexer launch");
            ic_topk_args t;
            t.scores = scores;
            t.row_stride = lay.score_stride;
            t.rows = s.B;
            t.first_len = 0;
            t.seq_len = seq_len;
            t.k = s.k;
            t.idx = idx_cache;
            t.max_len = s.Lk;
            t.cand = lay.cand_off ? reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + lay.cand_off) : nullptr;
            e = launch_topk(t, st);
            if (e != hipSuccess) return hip_fail(e, "decode top-k launch");
            cached = true;
            ++cnt.indexer_calls;
            ++cnt.score_tiles;
        } else if (!cached) {
            return fail(IC_ERR_NO_CACHED_INDICES, "no cached indices: S layer before any F layer");
        }
        r = run_attn(s, 1, L.q, L.kv, idx_cache, L.out, nsplit, part, st);
        if (r != IC_OK) return r;
        ++cnt.attn_calls;
        ++cnt.layers;
    }
    g_stats = cnt;
    if (stats) *stats = cnt;
    return IC_OK;
}

// Scratch of ic_decode_step_static, for callers that cannot allocate a workspace: one
// array per GPU (each device that loads the library holds its own copy until the process
// ends).  Host code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
__device__ __align__(256) uint8_t scratch[IC_DECODE_STATIC_SCRATCH_BYTES];

ic_status static_scratch(void** out) {
    static std::mutex mu;
    static void* ptrs[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(IC_ERR_HIP, "device %d out of range for the static scratch", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(IC_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return IC_OK;
}

}  // namespace

extern "C" {

size_t ic_workspace_size(const ic_shape* shape, int op) {
    switch (op) {
        case IC_OP_INDEXER_TOPK:
            if (check_shape(shape, true, false) != IC_OK) return 0;
            return indexer_ws(*shape);
        case IC_OP_RUN_STACK:                       // two score tiles (one is enough to run)
            if (check_shape(shape, true, false) != IC_OK) return 0;
            return 2 * (size_t)round_up((int64_t)indexer_ws(*shape), 256);
        case IC_OP_SPARSE_ATTN:
        case IC_OP_INDEXER_SCORES:
            if (check_shape(shape, op == IC_OP_INDEXER_SCORES, false) != IC_OK) return 0;
            return 0;
        case IC_OP_RUN_STACK_VARLEN:
            if (check_shape(shape, true, false, true) != IC_OK) return 0;
            return indexer_ws_varlen(*shape);
        case IC_OP_DECODE_STEP:
            if (check_shape(shape, true, true) != IC_OK) return 0;
            return decode_ws(*shape);
        case IC_OP_DISTILL_KL:
            if (check_shape(shape, true, false) != IC_OK) return 0;
            return indexer_ws(*shape);
        case IC_OP_DECODE_ATTN:
            if (check_shape(shape, false, true) != IC_OK) return 0;
            return sparse_attn_ws_bytes(shape->B, shape->H, shape->d, decode_splits(*shape));
        default:
            fail(IC_ERR_ARG, "unknown op %d", op);
            return 0;
    }
}

ic_status ic_indexer_topk(const ic_shape* shape, const void* q_I, const float* w, const void* k_I, int32_t* idx,
                          void* ws, size_t ws_bytes, void* stream) {
    ic_status r = check_shape(shape, true, false);
    if (r != IC_OK) return r;
    if (!q_I || !w || !k_I || !idx) return fail(IC_ERR_ARG, "q_I, w, k_I and idx must be non-NULL");
    if ((r = check_aligned({{q_I, "q_I", 16}, {k_I, "k_I", 16}, {w, "w", 4}, {idx, "idx", 4}})) != IC_OK) return r;
    if ((r = check_ws(ws, ws_bytes, indexer_ws(*shape))) != IC_OK) return r;
    return run_indexer_topk(*shape, q_I, w, k_I, idx, ws, (hipStream_t)stream, nullptr);
}

ic_status ic_indexer_scores(const ic_shape* shape, const void* q_I, const float* w, const void* k_I, float* scores,
                            int64_t row_stride, void* stream) {
    ic_status r = check_shape(shape, true, false);
    if (r != IC_OK) return r;
    if (!q_I || !w || !k_I || !scores) return fail(IC_ERR_ARG, "q_I, w, k_I and scores must be non-NULL");
    if ((r = check_aligned({{q_I, "q_I", 16}, {k_I, "k_I", 16}, {w, "w", 4}, {scores, "scores", 4}})) != IC_OK)
        return r;
    const ic_shape& s = *shape;
    if (row_stride < (int64_t)s.pos0 + s.Lq) return fail(IC_ERR_SHAPE, "row_stride %lld < pos0 + Lq", (long long)row_stride);
    const size_t eb = elem_bytes(s.idx_dtype);
    for (int b = 0; b < s.B; ++b) {
        ic_indexer_args a;
        a.q_I = static_cast<const uint8_t*>(q_I) + (size_t)b * s.Lq * s.H_I * s.d_I * eb;
        a.w = w + (size_t)b * s.Lq * s.H_I;
        a.k_I = static_cast<const uint8_t*>(k_I) + (size_t)b * s.Lk * s.d_I * eb;
        a.scores = scores + (size_t)b * s.Lq * row_stride;
        a.row_stride = row_stride;
        a.q_begin = 0;
        a.nq = s.Lq;
        a.pos_begin = s.pos0;
        a.H_I = s.H_I;
        a.d_I = s.d_I;
        a.fp8 = s.idx_dtype == IC_FP8_E4M3;
        hipError_t e = launch_indexer_prefill(a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "indexer launch");
    }
    return IC_OK;
}

ic_status ic_topk_rows(const float* scores, int64_t row_stride, int32_t rows, int32_t first_len, int32_t k,
                       int32_t* idx, void* stream) {
    if (!scores || !idx) return fail(IC_ERR_ARG, "scores and idx must be non-NULL");
    if (ic_status r = check_aligned({{scores, "scores", 4}, {idx, "idx", 4}})) return r;
    if (rows < 1 || first_len < 1 || k < 1 || k > kMaxK)
        return fail(IC_ERR_SHAPE, "need rows >= 1, first_len >= 1, 1 <= k <= %d", kMaxK);
    if ((int64_t)first_len + rows - 1 > row_stride)
        return fail(IC_ERR_SHAPE, "last row length %lld exceeds row_stride %lld",
                    (long long)first_len + rows - 1, (long long)row_stride);
    if ((int64_t)first_len + rows - 1 > INT32_MAX)
        return fail(IC_ERR_SHAPE, "last row length %lld exceeds 2^31 - 1", (long long)first_len + rows - 1);
    ic_topk_args t;
    t.scores = scores;
    t.row_stride = row_stride;
    t.rows = rows;
    t.first_len = first_len;
    t.seq_len = nullptr;
    t.k = k;
    t.idx = idx;
    t.max_len = first_len + rows - 1;
    t.cand = nullptr;
    hipError_t e = launch_topk(t, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return IC_OK;
}

size_t ic_topk_rows_seq_ws(int32_t rows, int32_t max_len, int32_t k) {
    if (rows < 1 || max_len < 1 || k < 1 || k > kMaxK) return 0;
    ic_topk_args t{};
    t.rows = rows;
    t.max_len = max_len;
    t.k = k;
    return topk_ws_bytes(t);
}

ic_status ic_topk_rows_seq(const float* scores, int64_t row_stride, int32_t rows, const int32_t* seq_len,
                           int32_t max_len, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    if (!scores || !seq_len || !idx) return fail(IC_ERR_ARG, "scores, seq_len and idx must be non-NULL");
    if (ic_status r = check_aligned({{scores, "scores", 4}, {seq_len, "seq_len", 4}, {idx, "idx", 4}})) return r;
    if (rows < 1 || max_len < 1 || k < 1 || k > kMaxK)
        return fail(IC_ERR_SHAPE, "need rows >= 1, max_len >= 1, 1 <= k <= %d", kMaxK);
    if (max_len > row_stride)
        return fail(IC_ERR_SHAPE, "max_len %d exceeds row_stride %lld", max_len, (long long)row_stride);
    ic_topk_args t;
    t.scores = scores;
    t.row_stride = row_stride;
    t.rows = rows;
    t.first_len = 0;
    t.seq_len = seq_len;
    t.k = k;
    t.idx = idx;
    t.max_len = max_len;
    t.cand = nullptr;
    if (ws != nullptr) {
        const size_t need = topk_ws_bytes(t);
        if (ic_status r = check_ws(ws, ws_bytes, need)) return r;
        if (need) t.cand = static_cast<int32_t*>(ws);
    }
    hipError_t e = launch_topk(t, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return IC_OK;
}

ic_status ic_sparse_attn(const ic_shape* shape, const void* q, const void* kv, const int32_t* idx, void* out, void* ws,
                         size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    ic_status r = check_shape(shape, false, false);
    if (r != IC_OK) return r;
    if (!q || !kv || !idx || !out) return fail(IC_ERR_ARG, "q, kv, idx and out must be non-NULL");
    if ((r = check_aligned({{q, "q", 16}, {kv, "kv", 16}, {out, "out", 16}, {idx, "idx", 4}})) != IC_OK) return r;
    return run_attn(*shape, shape->Lq, q, kv, idx, out, 1, nullptr, (hipStream_t)stream);
}

ic_status ic_run_stack(const char* pattern, int32_t n_layers, const ic_layer* layers, const ic_shape* shape,
                       int32_t* idx_cache, void* ws, size_t ws_bytes, ic_stats* stats, void* stream) {
    ic_status r = check_shape(shape, true, false);
    if (r != IC_OK) return r;
    if ((r = check_stack(pattern, n_layers, layers)) != IC_OK) return r;
    if (!idx_cache) return fail(IC_ERR_ARG, "idx_cache is NULL");
    if ((r = check_aligned({{idx_cache, "idx_cache", 4}})) != IC_OK) return r;
    if ((r = check_ws(ws, ws_bytes, indexer_ws(*shape))) != IC_OK) return r;
    hipStream_t st = (hipStream_t)stream;
    // With room for two score tiles, a tile's top-k also leaves the caller's stream.
    SideWork side(ws, ws_bytes, (size_t)round_up((int64_t)indexer_ws(*shape), 256));
    ic_stats cnt = {0, 0, 0, 0};
    bool cached = false;                       // the index cache starts empty on every call
    for (int l = 0; l < n_layers; ++l) {
        const ic_layer& L = layers[l];
        const bool full = pattern[l] == 'F' || pattern[l] == '1';
        if (full) {
            r = run_indexer_topk(*shape, L.q_I, L.w, L.k_I, idx_cache, ws, st, &cnt.score_tiles, side.tile_attn(L));
            if (r != IC_OK) {
                (void)side.join(st);           // keeps the failure's own status and message
                return r;
            }
            cached = true;
            ++cnt.indexer_calls;
        } else if (!cached) {
            return fail(IC_ERR_NO_CACHED_INDICES, "no cached indices: S layer before any F layer");
        }
        if (full && side.active()) {           // join: the layer's tile attentions are done
            hipError_t e = side.join(st);
            if (e != hipSuccess) return hip_fail(e, "stream join");
        } else {
            r = run_attn(*shape, shape->Lq, L.q, L.kv, idx_cache, L.out, 1, nullptr, st);
            if (r != IC_OK) return r;
        }
        ++cnt.attn_calls;
        ++cnt.layers;
    }
    g_stats = cnt;
    if (stats) *stats = cnt;
    return IC_OK;
}

size_t ic_run_stack_dynamic_ws(const ic_shape* shape, int32_t probe_stride) {
    if (check_shape(shape, true, false) != IC_OK) return 0;
    if (probe_stride < 1) {
        fail(IC_ERR_ARG, "probe_stride must be >= 1 (got %d)", probe_stride);
        return 0;
    }
    return dyn_layout(*shape, probe_stride).total;
}

ic_status ic_run_stack_dynamic(const char* pattern, int32_t n_layers, const ic_layer* layers, const ic_shape* shape,
                               int32_t probe_stride, double tau, int32_t* idx_cache, int32_t* refreshed,
                               float* recall, void* ws, size_t ws_bytes, ic_stats* stats, void* stream) {
    ic_status r = check_shape(shape, true, false);
    if (r != IC_OK) return r;
    if ((r = check_stack(pattern, n_layers, layers)) != IC_OK) return r;
    if (!idx_cache) return fail(IC_ERR_ARG, "idx_cache is NULL");
    if ((r = check_aligned({{idx_cache, "idx_cache", 4}})) != IC_OK) return r;
    if (probe_stride < 1) return fail(IC_ERR_ARG, "probe_stride must be >= 1 (got %d)", probe_stride);
    if (!(tau >= 0.0 && tau <= 2.0)) return fail(IC_ERR_ARG, "tau must be in [0, 2] (got %g)", tau);
    if ((r = check_aligned({{refreshed, "refreshed", 4}, {recall, "recall", 4}})) != IC_OK) return r;
    for (int l = 0; l < n_layers; ++l) {
        const ic_layer& L = layers[l];
        const int have = (L.q_I != nullptr) + (L.w != nullptr) + (L.k_I != nullptr);
        if (have != 0 && have != 3)
            return fail(IC_ERR_ARG, "layer %d: q_I, w and k_I must be all set or all NULL", l);
    }
    const ic_shape& s = *shape;
    const DynWs d = dyn_layout(s, probe_stride);
    if ((r = check_ws(ws, ws_bytes, d.total)) != IC_OK) return r;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    float* pscores = reinterpret_cast<float*>(wsb + d.probe_scores_off);
    int32_t* pidx = reinterpret_cast<int32_t*>(wsb + d.probe_idx_off);
    int32_t* inter = reinterpret_cast<int32_t*>(wsb + d.inter_off);
    int32_t* flag = reinterpret_cast<int32_t*>(wsb + d.flag_off);
    const size_t eb = elem_bytes(s.idx_dtype);
    // own entries of the probe rows: every probe row is full once it sees k keys
    int64_t own = 0;
    for (int j = 0; j < d.P; ++j) own += std::min<int64_t>(s.k, (int64_t)s.pos0 + d.t0 + (int64_t)j * probe_stride + 1);
    // As in ic_run_stack, an F layer's tile attentions run beside its next tiles' scoring (one
    // score tile here: the rest of the workspace is the probe's, so the top-k stays put).
    SideWork side(ws, 0, 0);
    ic_stats cnt = {0, 0, 0, 0};
    bool cached = false;
    for (int l = 0; l < n_layers; ++l) {
        const ic_layer& L = layers[l];
        const bool full = pattern[l] == 'F' || pattern[l] == '1';
        if (full) {
            r = run_indexer_topk(s, L.q_I, L.w, L.k_I, idx_cache, ws, st, &cnt.score_tiles, side.tile_attn(L));
            if (r != IC_OK) {
                (void)side.join(st);
                return r;
            }
            cached = true;
            ++cnt.indexer_calls;
            if (side.active()) {               // the layer's tile attentions are done
                hipError_t e = side.join(st);
                if (e != hipSuccess) return hip_fail(e, "stream join");
                ++cnt.attn_calls;
                ++cnt.layers;
                continue;
            }
        } else if (!cached) {
            return fail(IC_ERR_NO_CACHED_INDICES, "no cached indices: S layer before any F layer");
        } else if (L.q_I) {
            for (int b = 0; b < s.B; ++b) {
                const uint8_t* qb = static_cast<const uint8_t*>(L.q_I) + (size_t)b * s.Lq * s.H_I * s.d_I * eb;
                const float* wb = L.w + (size_t)b * s.Lq * s.H_I;
                const uint8_t* kb = static_cast<const uint8_t*>(L.k_I) + (size_t)b * s.Lk * s.d_I * eb;
                int32_t* idxb = idx_cache + (size_t)b * s.Lq * s.k;
                // probe: this layer's own scores and top-k for every probe_stride-th query (the
                // prefill indexer over strided query rows: the probe queries share each k_I block)
                ic_indexer_args a;
                a.q_I = qb;
                a.w = wb;
                a.k_I = kb;
                a.scores = pscores;
                a.row_stride = d.score_stride;
                a.q_begin = d.t0;
                a.nq = d.P;
                a.pos_begin = s.pos0 + d.t0;
                a.q_step = probe_stride;
                a.H_I = s.H_I;
                a.d_I = s.d_I;
                a.fp8 = s.idx_dtype == IC_FP8_E4M3;
                hipError_t e = launch_indexer_prefill(a, st);
                if (e != hipSuccess) return hip_fail(e, "probe indexer launch");
                ic_topk_args t{};
                t.scores = pscores;
                t.row_stride = d.score_stride;
                t.rows = d.P;
                t.first_len = s.pos0 + d.t0 + 1;
                t.seq_len = nullptr;
                t.k = s.k;
                t.idx = pidx;
                t.max_len = s.pos0 + s.Lq;
                t.cand = nullptr;
                t.len_step = probe_stride;
                e = launch_topk(t, st);
                if (e != hipSuccess) return hip_fail(e, "probe top-k launch");
                // |cached row & own row| for the probe rows, then the decision on the device
                e = launch_overlap(idxb + (size_t)d.t0 * s.k, pidx, d.P, s.k, inter, nullptr, nullptr, nullptr, st,
                                   probe_stride);
                if (e != hipSuccess) return hip_fail(e, "probe overlap launch");
                e = launch_drift_decision(inter, d.P, own, tau, flag, refreshed ? refreshed + (size_t)l * s.B + b : nullptr,
                                          recall ? recall + (size_t)l * s.B + b : nullptr, st);
                if (e != hipSuccess) return hip_fail(e, "drift decision launch");
                // the refresh: every launch of it returns at once unless the flag is set
                r = run_indexer_topk_one(s, s.Lq, s.pos0, qb, wb, kb, idxb, ws, st, &cnt.score_tiles, flag);
                if (r != IC_OK) return r;
            }
        }
        r = run_attn(s, s.Lq, L.q, L.kv, idx_cache, L.out, 1, nullptr, st);
        if (r != IC_OK) return r;
        ++cnt.attn_calls;
        ++cnt.layers;
    }
    g_stats = cnt;
    if (stats) *stats = cnt;
    return IC_OK;
}

ic_status ic_run_stack_varlen(const char* pattern, int32_t n_layers, const ic_layer* layers, const ic_shape* shape,
                              const int32_t* q_len, const int32_t* pos0, int32_t* idx_cache, void* ws, size_t ws_bytes,
                              ic_stats* stats, void* stream) {
    ic_status r = check_shape(shape, true, false, true);
    if (r != IC_OK) return r;
    if ((r = check_stack(pattern, n_layers, layers)) != IC_OK) return r;
    if (!idx_cache) return fail(IC_ERR_ARG, "idx_cache is NULL");
    if ((r = check_aligned({{idx_cache, "idx_cache", 4}})) != IC_OK) return r;
    if (!q_len || !pos0) return fail(IC_ERR_ARG, "q_len and pos0 must be non-NULL host arrays");
    const ic_shape& s = *shape;
    int64_t total = 0;
    for (int b = 0; b < s.B; ++b) {
        if (q_len[b] < 0 || pos0[b] < 0)
            return fail(IC_ERR_SHAPE, "sequence %d: q_len %d and pos0 %d must be >= 0", b, q_len[b], pos0[b]);
        if ((int64_t)pos0[b] + q_len[b] > s.Lk)
            return fail(IC_ERR_SHAPE, "sequence %d: pos0 + q_len (%lld) exceeds Lk (%d)", b,
                        (long long)pos0[b] + q_len[b], s.Lk);
        total += q_len[b];
    }
    if (total != s.Lq) return fail(IC_ERR_SHAPE, "q_len sums to %lld, shape.Lq is %d", (long long)total, s.Lq);
    if ((r = check_ws(ws, ws_bytes, indexer_ws_varlen(s))) != IC_OK) return r;
    hipStream_t st = (hipStream_t)stream;
    const size_t eb = elem_bytes(s.idx_dtype);
    const int chunk = chunk_of(s);
    // Plan: consecutive sequences of at most `chunk` queries in all (and at most IC_GROUP_MAX
    // of them) share one launch per kernel, their score rows packed into one tile; a sequence
    // longer than a chunk runs alone in chunks.  Empty sequences are skipped.
    struct Piece {
        bool grouped;
        ic_seq_group g;       // grouped: the sequences, rows relative to q0
        int64_t q0;           // first packed query row
        int rows;             // packed rows of the piece
        int b;                // single: the sequence
        int max_keys;         // keys visible to the piece's longest row
    };
    std::vector<Piece> plan;
    try {
        plan.reserve((size_t)s.B);
    } catch (...) {
        return fail(IC_ERR_ARG, "cannot plan %d sequences", s.B);
    }
    {
        Piece cur{};
        cur.grouped = true;
        auto flush = [&]() {
            if (cur.g.n > 0) plan.push_back(cur);
            cur = Piece{};
            cur.grouped = true;
        };
        int64_t q0 = 0;
        for (int b = 0; b < s.B; ++b) {
            const int n = q_len[b];
            if (n > chunk) {
                flush();
                Piece one{};
                one.grouped = false;
                one.q0 = q0;
                one.rows = n;
                one.b = b;
                one.max_keys = pos0[b] + n;
                plan.push_back(one);
            } else if (n > 0) {
                if (cur.g.n == IC_GROUP_MAX || cur.rows + n > chunk) flush();
                if (cur.g.n == 0) cur.q0 = q0;
                const int i = cur.g.n++;
                cur.g.row0[i] = cur.rows;
                cur.g.pos0[i] = pos0[b];
                cur.g.seq[i] = b;
                cur.rows += n;
                cur.g.row0[i + 1] = cur.rows;
                cur.max_keys = std::max(cur.max_keys, pos0[b] + n);
            }
            q0 += n;
        }
        flush();
    }
    ic_stats cnt = {0, 0, 0, 0};
    bool cached = false;                       // the index cache starts empty on every call
    for (int l = 0; l < n_layers; ++l) {
        const ic_layer& L = layers[l];
        const bool full = pattern[l] == 'F' || pattern[l] == '1';
        if (!full && !cached) return fail(IC_ERR_NO_CACHED_INDICES, "no cached indices: S layer before any F layer");
        for (const Piece& pc : plan) {
            int32_t* idxp = idx_cache + pc.q0 * s.k;
            hipError_t e;
            if (full && pc.grouped) {
                const int64_t stride = round_up(pc.max_keys, 4);
                ic_indexer_args a;
                a.q_I = L.q_I;
                a.w = L.w;
                a.k_I = L.k_I;
                a.scores = static_cast<float*>(ws);
                a.row_stride = stride;
                a.q_begin = (int32_t)pc.q0;
                a.nq = pc.rows;
                a.pos_begin = 0;
                a.H_I = s.H_I;
                a.d_I = s.d_I;
                a.fp8 = s.idx_dtype == IC_FP8_E4M3;
                a.grp = &pc.g;
                a.k_seq_bytes = (int64_t)s.Lk * s.d_I * eb;
                if ((e = launch_indexer_prefill(a, st)) != hipSuccess) return hip_fail(e, "indexer launch");
                ic_topk_args t{};
                t.scores = static_cast<float*>(ws);
                t.row_stride = stride;
                t.rows = pc.rows;
                t.first_len = 1;
                t.seq_len = nullptr;
                t.k = s.k;
                t.idx = idxp;
                t.max_len = pc.max_keys;
                t.cand = nullptr;
                t.grp = &pc.g;
                if ((e = launch_topk(t, st)) != hipSuccess) return hip_fail(e, "top-k launch");
                ++cnt.score_tiles;
            } else if (full) {
                r = run_indexer_topk_one(s, pc.rows, pos0[pc.b],
                                         static_cast<const uint8_t*>(L.q_I) + pc.q0 * s.H_I * s.d_I * eb,
                                         L.w + pc.q0 * s.H_I,
                                         static_cast<const uint8_t*>(L.k_I) + (size_t)pc.b * s.Lk * s.d_I * eb, idxp,
                                         ws, st, &cnt.score_tiles);
                if (r != IC_OK) return r;
            }
            ic_attn_args a;
            a.q = static_cast<const uint16_t*>(L.q) + pc.q0 * s.H * s.d;
            a.kv = static_cast<const uint16_t*>(L.kv) + (pc.grouped ? 0 : (size_t)pc.b * s.Lk * 2 * s.d);
            a.idx = idxp;
            a.out = static_cast<uint16_t*>(L.out) + pc.q0 * s.H * s.d;
            a.kv_seq_stride = (int64_t)s.Lk * 2 * s.d;
            a.Lk = s.Lk;
            a.nq = pc.rows;
            a.q_per_seq = pc.rows;
            a.H = s.H;
            a.d = s.d;
            a.k = s.k;
            a.nsplit = 1;
            a.ws = nullptr;
            a.grp = pc.grouped ? &pc.g : nullptr;
            if ((e = launch_sparse_attn(a, st)) != hipSuccess) return hip_fail(e, "sparse attention launch");
        }
        if (full) {
            cached = true;
            ++cnt.indexer_calls;
        }
        ++cnt.attn_calls;
        ++cnt.layers;
    }
    g_stats = cnt;
    if (stats) *stats = cnt;
    return IC_OK;
}

ic_status ic_decode_step(const char* pattern, int32_t n_layers, const ic_layer* layers, const ic_shape* shape,
                         const int32_t* seq_len, int32_t* idx_cache, void* ws, size_t ws_bytes, ic_stats* stats,
                         void* stream) {
    ic_status r = check_shape(shape, true, true);
    if (r != IC_OK) return r;
    if ((r = check_stack(pattern, n_layers, layers)) != IC_OK) return r;
    if (!seq_len || !idx_cache) return fail(IC_ERR_ARG, "seq_len and idx_cache must be non-NULL");
    if ((r = check_aligned({{seq_len, "seq_len", 4}, {idx_cache, "idx_cache", 4}})) != IC_OK) return r;
    if ((r = check_ws(ws, ws_bytes, decode_ws(*shape))) != IC_OK) return r;
    return decode_step_run(pattern, n_layers, layers, *shape, seq_len, idx_cache, ws, stats, (hipStream_t)stream);
}

ic_status ic_decode_step_static(const char* pattern, int32_t n_layers, const ic_layer* layers, const ic_shape* shape,
                                const int32_t* seq_len, int32_t* idx_cache, ic_stats* stats, void* stream) {
    ic_status r = check_shape(shape, true, true);
    if (r != IC_OK) return r;
    if ((r = check_stack(pattern, n_layers, layers)) != IC_OK) return r;
    if (!seq_len || !idx_cache) return fail(IC_ERR_ARG, "seq_len and idx_cache must be non-NULL");
    if ((r = check_aligned({{seq_len, "seq_len", 4}, {idx_cache, "idx_cache", 4}})) != IC_OK) return r;
    const size_t need = decode_ws(*shape);
    if (need > (size_t)IC_DECODE_STATIC_SCRATCH_BYTES)
        return fail(IC_ERR_WORKSPACE, "this decode shape needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use ic_decode_step with a workspace)", need, (size_t)IC_DECODE_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((r = static_scratch(&ws)) != IC_OK) return r;
    return decode_step_run(pattern, n_layers, layers, *shape, seq_len, idx_cache, ws, stats, (hipStream_t)stream);
}

ic_status ic_decode_indexer_scores(const ic_shape* shape, const void* q_I, const float* w, const void* k_I,
                                   const int32_t* seq_len, float* scores, int64_t row_stride, void* stream) {
    ic_status r = check_shape(shape, true, true);
    if (r != IC_OK) return r;
    if (!q_I || !w || !k_I || !seq_len || !scores)
        return fail(IC_ERR_ARG, "q_I, w, k_I, seq_len and scores must be non-NULL");
    if ((r = check_aligned({{q_I, "q_I", 16}, {k_I, "k_I", 16}, {w, "w", 4}, {seq_len, "seq_len", 4},
                            {scores, "scores", 4}})) != IC_OK)
        return r;
    const ic_shape& s = *shape;
    if (row_stride < s.Lk) return fail(IC_ERR_SHAPE, "row_stride %lld < Lk %d", (long long)row_stride, s.Lk);
    ic_indexer_decode_args a;
    a.q_I = q_I;
    a.w = w;
    a.k_I = k_I;
    a.seq_len = seq_len;
    a.scores = scores;
    a.score_stride = row_stride;
    a.B = s.B;
    a.Lk = s.Lk;
    a.H_I = s.H_I;
    a.d_I = s.d_I;
    a.fp8 = s.idx_dtype == IC_FP8_E4M3;
    hipError_t e = launch_indexer_decode(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode indexer launch");
    return IC_OK;
}

ic_status ic_decode_attn(const ic_shape* shape, const void* q, const void* kv, const int32_t* idx, void* out, void* ws,
                         size_t ws_bytes, void* stream) {
    ic_status r = check_shape(shape, false, true);
    if (r != IC_OK) return r;
    if (!q || !kv || !idx || !out) return fail(IC_ERR_ARG, "q, kv, idx and out must be non-NULL");
    if ((r = check_aligned({{q, "q", 16}, {kv, "kv", 16}, {out, "out", 16}, {idx, "idx", 4}})) != IC_OK) return r;
    const ic_shape& s = *shape;
    const int nsplit = decode_splits(s);
    if ((r = check_ws(ws, ws_bytes, sparse_attn_ws_bytes(s.B, s.H, s.d, nsplit))) != IC_OK) return r;
    return run_attn(s, 1, q, kv, idx, out, nsplit, static_cast<float*>(ws), (hipStream_t)stream);
}

ic_status ic_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t rows, int32_t k, int32_t* inter,
                           float* jaccard, float* recall, float* means, void* stream) {
    if (!idx_a || !idx_b) return fail(IC_ERR_ARG, "idx_a and idx_b must be non-NULL");
    if (rows < 0 || rows > INT32_MAX || k < 1 || k > kMaxK)
        return fail(IC_ERR_SHAPE, "need 0 <= rows <= 2^31-1 and 1 <= k <= %d", kMaxK);
    if (means && (!jaccard || !recall)) return fail(IC_ERR_ARG, "means needs jaccard and recall");
    if (ic_status r = check_aligned({{idx_a, "idx_a", 4}, {idx_b, "idx_b", 4}, {inter, "inter", 4},
                                     {jaccard, "jaccard", 4}, {recall, "recall", 4}, {means, "means", 4}}))
        return r;
    hipError_t e = launch_overlap(idx_a, idx_b, rows, k, inter, jaccard, recall, means, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "overlap launch");
    return IC_OK;
}

ic_status ic_distill_kl(const ic_shape* shape, const void* q_I, const float* w, const void* k_I, const int32_t* idx,
                        int32_t n_served, const void* const* q, const void* const* kv, float* kl, float* kl_mean,
                        void* ws, size_t ws_bytes, void* stream) {
    ic_status st = check_shape(shape, true, false);
    if (st != IC_OK) return st;
    const ic_shape& s = *shape;
    if (!q_I || !w || !k_I || !idx || !kl) return fail(IC_ERR_ARG, "q_I, w, k_I, idx and kl must be non-NULL");
    if (n_served < 1 || n_served > IC_DISTILL_MAX_SERVED)
        return fail(IC_ERR_ARG, "n_served must be in 1..%d (got %d)", IC_DISTILL_MAX_SERVED, n_served);
    if (!q || !kv) return fail(IC_ERR_ARG, "q and kv must be host arrays of n_served device pointers");
    for (int j = 0; j < n_served; ++j) {
        if (!q[j] || !kv[j]) return fail(IC_ERR_ARG, "served layer %d has a NULL q or kv", j);
        if ((st = check_aligned({{q[j], "served q", 16}, {kv[j], "served kv", 16}})) != IC_OK) return st;
    }
    if ((st = check_aligned({{q_I, "q_I", 16}, {k_I, "k_I", 16}, {w, "w", 4}, {idx, "idx", 4}, {kl, "kl", 4},
                             {kl_mean, "kl_mean", 4}})) != IC_OK)
        return st;
    if ((st = check_ws(ws, ws_bytes, indexer_ws(s))) != IC_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    const size_t eb = elem_bytes(s.idx_dtype);
    const int chunk = chunk_of(s);
    float* tile = static_cast<float*>(ws);
    for (int b = 0; b < s.B; ++b) {
        const uint8_t* qb = static_cast<const uint8_t*>(q_I) + (size_t)b * s.Lq * s.H_I * s.d_I * eb;
        const float* wb = w + (size_t)b * s.Lq * s.H_I;
        const uint8_t* kb = static_cast<const uint8_t*>(k_I) + (size_t)b * s.Lk * s.d_I * eb;
        ic_distill_args d{};
        d.idx = idx + (size_t)b * s.Lq * s.k;
        for (int j = 0; j < n_served; ++j) {
            d.q[j] = static_cast<const uint16_t*>(q[j]) + (size_t)b * s.Lq * s.H * s.d;
            d.kv[j] = static_cast<const uint16_t*>(kv[j]) + (size_t)b * s.Lk * 2 * s.d;
        }
        d.kl = kl + (size_t)b * s.Lq;
        d.pos0 = s.pos0;
        d.Lk = s.Lk;
        d.nserved = n_served;
        d.H = s.H;
        d.d = s.d;
        d.k = s.k;
        for (int c0 = 0; c0 < s.Lq; c0 += chunk) {
            const int nq = std::min(chunk, s.Lq - c0);
            const int64_t stride = round_up((int64_t)s.pos0 + c0 + nq, 4);
            ic_indexer_args a;
            a.q_I = qb;
            a.w = wb;
            a.k_I = kb;
            a.scores = tile;
            a.row_stride = stride;
            a.q_begin = c0;
            a.nq = nq;
            a.pos_begin = s.pos0 + c0;
            a.H_I = s.H_I;
            a.d_I = s.d_I;
            a.fp8 = s.idx_dtype == IC_FP8_E4M3;
            hipError_t e = launch_indexer_prefill(a, hs);
            if (e != hipSuccess) return hip_fail(e, "indexer launch");
            d.scores = tile;
            d.score_stride = stride;
            d.q_begin = c0;
            d.nrows = nq;
            e = launch_distill(d, hs);
            if (e != hipSuccess) return hip_fail(e, "distillation loss launch");
        }
    }
    if (kl_mean) {
        hipError_t e = launch_mean(kl, (int64_t)s.B * s.Lq, kl_mean, hs);
        if (e != hipSuccess) return hip_fail(e, "mean launch");
    }
    return IC_OK;
}

ic_status ic_get_stats(ic_stats* out) {
    if (!out) return fail(IC_ERR_ARG, "out is NULL");
    *out = g_stats;
    return IC_OK;
}

const char* ic_last_error(void) { return g_err.c_str(); }

int32_t ic_version(void) { return 100; }

}  // extern "C"
