/*
 * indexcache.h -- C ABI of the IndexCache / DSA hot path on AMD MI355X (gfx950).
 *
 * What the library computes (page titles and sections, as cited throughout):
 *
 *  - "IndexCache: Accelerating Sparse Attention via Cross-Layer Index Reuse",
 *    arXiv abstract: DeepSeek Sparse Attention's lightweight lightning
 *    indexer picks the top-k tokens per query, so core attention costs O(Lk);
 *    the indexer itself stays O(L^2) and runs at every layer.  IndexCache
 *    splits layers into Full layers, which run their own indexer, and Shared
 *    layers, which reuse the nearest Full layer's top-k indices.
 *  - "Indexcache Sparse Attention Acceleration" (agent skill page), Step 3:
 *    an IndexCacheManager driven by a binary pattern ('1' = F, '0' = S);
 *    F computes and caches, S returns the cached indices, and an S layer
 *    with nothing cached is an error.  Practical Guidance, Common Pitfalls:
 *    the cache must be cleared between sequences.
 *  - "When the Optimizer Becomes the Bottleneck: A Close Look at IndexCache"
 *    (blog), "The Redundancy That Was Sitting There": the inference change is
 *    one conditional branch, and the cache is a single index tensor that is
 *    overwritten at every F layer (no memory beyond what DSA allocates).
 *
 * The indexer score is the DSA lightning indexer's head-weighted ReLU dot
 * product (named but not written out on the pages):
 *     I[t,s] = sum_j w[t,j] * max(0, q_I[t,j,:] . k_I[s,:]),   s <= p(t)
 * with H_I indexer heads sharing one key vector per token, and p(t) the
 * absolute position of query t (a query sees itself).  Top-k keeps the k
 * highest scores per query; ties go to the lower key index; each idx row
 * lists the chosen positions in ascending order, padded with -1 when fewer
 * than k keys are visible.  Sparse attention is, per head,
 *     out = softmax_s(q . K[s] / sqrt(d)) V[s]  over s in idx (-1 skipped),
 * with one KV head shared by all H query heads.
 *
 * Conventions for every call:
 *  - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *    library never frees, keeps or reallocates it, and never allocates on
 *    the hot path: scratch space is the caller's workspace `ws`, at least
 *    ic_workspace_size() bytes, 256-byte aligned.
 *  - Tensors are dense and row-major in the layouts given below.
 *      bf16 = IEEE binary32 upper half; fp8 = OCP E4M3FN byte codes.
 *    q_I, k_I, q, kv and out (and distillation's served q / kv) must be 16-byte
 *    aligned, the fp32 and int32 arrays 4-byte aligned: every torch allocation
 *    is, while a view that starts at an odd element may not be.  A misaligned
 *    pointer fails with IC_ERR_ARG.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work and return; nothing synchronises the host.  All of a call's work is
 *    ordered on `stream`: work after the call on `stream` sees its results.
 *    ic_run_stack and ic_run_stack_dynamic also run part of their work on a
 *    second stream of the library's (one per device, default priority,
 *    created on first use), forked from and joined back to `stream` with
 *    events inside the call, so the call stays capturable in a HIP graph.  Concurrent calls on one device
 *    share that stream: they may wait on each other there, never reorder.
 *  - Arguments are validated before any launch; a call that fails validation
 *    returns a non-zero ic_status, launches nothing and leaves outputs
 *    untouched.  A HIP error part-way through a call (IC_ERR_HIP) can leave
 *    outputs partly written; work the call already sent to the library's
 *    second stream is joined back into `stream` before it returns.
 *    ic_last_error() describes any failure (thread-local string).  A fault
 *    inside a kernel surfaces later, at the caller's next sync.
 *  - No C++ exception crosses this interface.
 */
#ifndef INDEXCACHE_H
#define INDEXCACHE_H

#include <stddef.h>
#include <stdint.h>

/* Only the calls below are exported from the library (it is built with hidden
 * default visibility). */
#if defined(__GNUC__) || defined(__clang__)
#define IC_API __attribute__((visibility("default")))
#else
#define IC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ic_status {
    IC_OK = 0,
    IC_ERR_ARG = 1,               /* NULL pointer or out-of-range scalar */
    IC_ERR_SHAPE = 2,             /* sizes outside what the kernels support, or inconsistent */
    IC_ERR_DTYPE = 3,             /* unknown indexer dtype */
    IC_ERR_PATTERN = 4,           /* pattern char not in {F,S,1,0}, or length != n_layers */
    IC_ERR_NO_CACHED_INDICES = 5, /* an S layer precedes every F layer (skill page, Step 3) */
    IC_ERR_WORKSPACE = 6,         /* workspace NULL, misaligned or smaller than required */
    IC_ERR_HIP = 7                /* a HIP runtime call failed */
} ic_status;

typedef enum ic_dtype {
    IC_BF16 = 0,                  /* q_I / k_I stored as bf16 */
    IC_FP8_E4M3 = 1               /* q_I / k_I stored as OCP e4m3fn codes */
} ic_dtype;

/* Sizes of one call.  Limits: B >= 1; 1 <= Lq; B * Lq <= 2^31 - 1 (query rows);
 * pos0 >= 0; pos0 + Lq <= Lk (prefill); H_I in 1..64; d_I in {32, 64, 128}; k in 1..4096; H in 1..4096;
 * d in {64, 128}; Lk * 4 * d < 4 GiB (one sequence's KV rows, addressed with
 * 32-bit offsets); chunk 0 (= 4096) or 16..65536 in steps of 16. */
typedef struct ic_shape {
    int32_t B;          /* sequences in the batch */
    int32_t Lq;         /* queries per sequence in this call (decode: 1) */
    int32_t Lk;         /* row capacity of k_I and kv per sequence (token stride) */
    int32_t pos0;       /* absolute position of query 0 (prefill; 0 for a fresh prompt) */
    int32_t H_I;        /* indexer heads */
    int32_t d_I;        /* indexer head dim */
    int32_t k;          /* top-k per query */
    int32_t H;          /* attention query heads (all share one KV head) */
    int32_t d;          /* attention head dim */
    int32_t idx_dtype;  /* ic_dtype of q_I and k_I */
    int32_t chunk;      /* queries per indexer score tile (0 = 4096) */
} ic_shape;

/* One layer of a stack.  Layouts (per call; B sequences):
 *   q_I [B, Lq, H_I, d_I] idx_dtype   (F layers; may be NULL on S layers)
 *   w   [B, Lq, H_I]      fp32        (F layers; may be NULL on S layers)
 *   k_I [B, Lk, d_I]      idx_dtype   (F layers; may be NULL on S layers)
 *   q   [B, Lq, H, d]     bf16
 *   kv  [B, Lk, 2, d]     bf16        (token row = K[d] then V[d])
 *   out [B, Lq, H, d]     bf16        (written) */
typedef struct ic_layer {
    const void*  q_I;
    const float* w;
    const void*  k_I;
    const void*  q;
    const void*  kv;
    void*        out;
} ic_layer;

/* Counters of the last ic_run_stack / ic_decode_step on this thread. */
typedef struct ic_stats {
    int64_t layers;          /* layers run */
    int64_t indexer_calls;   /* F layers whose indexer + top-k ran (== pattern count of F) */
    int64_t attn_calls;      /* sparse-attention launches (one per layer) */
    int64_t score_tiles;     /* indexer score tiles (query chunks x sequences) launched */
} ic_stats;

/* Operation codes for ic_workspace_size. */
enum {
    IC_OP_INDEXER_TOPK = 0,
    IC_OP_SPARSE_ATTN = 1,
    IC_OP_RUN_STACK = 2,
    IC_OP_DECODE_STEP = 3,
    IC_OP_INDEXER_SCORES = 4,
    IC_OP_RUN_STACK_VARLEN = 5,
    IC_OP_DISTILL_KL = 6,
    IC_OP_DECODE_ATTN = 7
};

/* Bytes of workspace the operation needs for this shape (0 if none).
 * Returns 0 and sets ic_last_error() for an invalid shape or op. */
IC_API size_t ic_workspace_size(const ic_shape* shape, int op);

/* Lightning indexer + top-k of one F layer (arXiv abstract; agent skill page,
 * Step 1 gives the (batch, seq_len, k) shape of the result).
 * Queries t = 0..Lq-1 of every sequence sit at positions pos0 + t and see
 * keys 0..pos0+t of k_I.  Writes idx [B, Lq, k] int32: the chosen key
 * positions of each query in ascending order, -1 padded.  The scores are
 * produced in query chunks of shape.chunk rows inside `ws`; no L x L buffer
 * is ever formed. */
IC_API ic_status ic_indexer_topk(const ic_shape* shape, const void* q_I, const float* w, const void* k_I,
                          int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* The raw fp32 indexer scores of one F layer, for verification and
 * measurement: scores [B, Lq, row_stride], row t holding keys 0..pos0+t
 * (entries beyond are not written).  row_stride >= pos0 + Lq.  No workspace. */
IC_API ic_status ic_indexer_scores(const ic_shape* shape, const void* q_I, const float* w, const void* k_I,
                            float* scores, int64_t row_stride, void* stream);

/* Top-k of caller-supplied score rows with the same rule as ic_indexer_topk:
 * scores [rows, row_stride] fp32, row r has n_r = first_len + r visible
 * entries (first_len >= 1, n_r <= row_stride and <= 2^31 - 1); writes idx [rows, k] int32.
 * Used to test the selection on chosen inputs (ties, -0.0, k >= n). */
IC_API ic_status ic_topk_rows(const float* scores, int64_t row_stride, int32_t rows, int32_t first_len,
                       int32_t k, int32_t* idx, void* stream);

/* Top-k of score rows with per-row lengths (the decode shape: one row per
 * sequence), same rule as ic_indexer_topk: scores [rows, row_stride] fp32,
 * row r has n_r = seq_len[r] visible entries, seq_len a DEVICE int32 [rows]
 * whose values are clamped to 1..max_len (max_len <= row_stride, host-known
 * bound); writes idx [rows, k] int32.  When rows are long (max_len > 32768)
 * and few (rows <= 1024), each 16384-key segment is ranked first and then the
 * segments' candidates, which needs ic_topk_rows_seq_ws() bytes of `ws`;
 * with ws NULL such rows take the one-workgroup streaming path instead (same
 * result). */
IC_API ic_status ic_topk_rows_seq(const float* scores, int64_t row_stride, int32_t rows, const int32_t* seq_len,
                           int32_t max_len, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes ic_topk_rows_seq can use for these sizes (0 if none). */
IC_API size_t ic_topk_rows_seq_ws(int32_t rows, int32_t max_len, int32_t k);

/* Sparse attention of one layer (arXiv abstract: core attention over the k
 * selected tokens): out [B, Lq, H, d] bf16 from q, kv and idx [B, Lq, k].
 * Entries outside [0, Lk) (the top-k's -1 padding) are skipped; a row with no
 * entry inside [0, Lk) has nothing to attend to and its output vectors are
 * zero.  The rows named may repeat and need not be sorted.  Softmax scale
 * 1/sqrt(d), fp32 accumulation.  ws is unused (NULL, 0). */
IC_API ic_status ic_sparse_attn(const ic_shape* shape, const void* q, const void* kv, const int32_t* idx,
                         void* out, void* ws, size_t ws_bytes, void* stream);

/* Prefill through an F/S layer stack (agent skill page, Step 3; blog, "The
 * Redundancy That Was Sitting There").  pattern[l] in {'F','1'} runs the
 * indexer + top-k of layer l into idx_cache; {'S','0'} reuses idx_cache as
 * the nearest preceding F layer left it.  Every layer then runs sparse
 * attention with idx_cache into layers[l].out.  The cache is reset at entry
 * (each call is a fresh sequence batch), so a pattern whose first layer is
 * S fails with IC_ERR_NO_CACHED_INDICES before any launch.
 * idx_cache: [B, Lq, k] int32, caller-owned, holds the last F layer's
 * indices on return.  stats (may be NULL) receives the counters.
 * An F layer's own attention runs score tile by score tile on the library's
 * second stream, overlapping the scoring of the layer's next tile.  With a
 * workspace of ic_workspace_size(IC_OP_RUN_STACK) bytes (two score tiles) a
 * tile's top-k runs there too, and the caller's stream scores the next tile
 * into the other buffer meanwhile; one tile's worth is the minimum (then the
 * top-k stays on `stream`). */
IC_API ic_status ic_run_stack(const char* pattern, int32_t n_layers, const ic_layer* layers,
                       const ic_shape* shape, int32_t* idx_cache, void* ws, size_t ws_bytes,
                       ic_stats* stats, void* stream);

/* Ragged batched prefill through the stack: B sequences of different lengths,
 * each continuing its own cached prefix (so a chunked prefill can resume and then
 * hand over to ic_decode_step).  Sequence b brings q_len[b] >= 0 new queries at
 * positions pos0[b] .. pos0[b]+q_len[b]-1 and sees its own keys 0..position;
 * q_len and pos0 are HOST int32 arrays [B] with pos0[b] + q_len[b] <= Lk.  The
 * queries are packed in sequence order, so shape.Lq = sum of q_len is the
 * packed row count and shape.pos0 must be 0:
 *   q_I [Lq, H_I, d_I], w [Lq, H_I], q [Lq, H, d], out [Lq, H, d] (packed rows)
 *   k_I [B, Lk, d_I], kv [B, Lk, 2, d]                        (per-sequence caches)
 *   idx_cache [Lq, k] int32.
 * Pattern and cache rules as ic_run_stack; the workspace is
 * ic_workspace_size(shape, IC_OP_RUN_STACK_VARLEN).  Consecutive sequences of at most
 * shape.chunk queries in all (up to 64 of them) share one launch of each kernel per layer;
 * a longer sequence runs alone, in chunks. */
IC_API ic_status ic_run_stack_varlen(const char* pattern, int32_t n_layers, const ic_layer* layers,
                                     const ic_shape* shape, const int32_t* q_len, const int32_t* pos0,
                                     int32_t* idx_cache, void* ws, size_t ws_bytes, ic_stats* stats, void* stream);

/* Prefill through the stack with drift-triggered refresh (blog, Conclusion:
 * decide at runtime whether a layer's neighbour is still a good proxy, and
 * refresh only when the drift exceeds a threshold; agent skill page, Step 1:
 * top-k set overlap as the measure).  Pattern, shapes and cache rules as
 * ic_run_stack, except that an S layer may also bring its own q_I, w and k_I
 * (all three, or none).  Such an S layer first probes the cache of each
 * sequence: for the queries t = (Lq-1) mod probe_stride, ... , Lq-1 it takes
 * its own top-k and counts hit = sum |cached row & own row| against own =
 * sum |own row|; when hit < tau * own (tau in [0, 2]; 0 never refreshes,
 * above 1 always does) it re-runs its indexer and top-k for every query of
 * that sequence, overwriting the cache, as an F layer would.  The decision
 * stays on the device (the refresh launches return at once when it is not
 * taken), so the call never waits for the GPU.  refreshed [n_layers, B] int32
 * and recall [n_layers, B] fp32 (device, each may be NULL) receive the
 * decision and hit / own of every probed (layer, sequence); entries of layers
 * without a probe are left untouched.  The workspace is
 * ic_run_stack_dynamic_ws(shape, probe_stride) bytes.  As in ic_run_stack, an F
 * layer's own attention runs score tile by score tile on the library's second
 * stream (its top-k stays on `stream`: the workspace holds one score tile). */
IC_API ic_status ic_run_stack_dynamic(const char* pattern, int32_t n_layers, const ic_layer* layers,
                                      const ic_shape* shape, int32_t probe_stride, double tau, int32_t* idx_cache,
                                      int32_t* refreshed, float* recall, void* ws, size_t ws_bytes,
                                      ic_stats* stats, void* stream);

/* Workspace bytes of ic_run_stack_dynamic for this shape and probe stride (0 if invalid). */
IC_API size_t ic_run_stack_dynamic_ws(const ic_shape* shape, int32_t probe_stride);

/* One decode step through the stack.  shape.Lq must be 1 and shape.Lk is
 * the cache capacity.  seq_len [B] int32 (device) counts each sequence's
 * tokens including the new one, whose k_I (F layers) and kv rows the caller
 * has already written at row seq_len[b]-1; the new query sits at that
 * position and sees keys 0..seq_len[b]-1 (1 <= seq_len[b] <= Lk).
 * idx_cache [B, 1, k].  Same pattern and cache rules as ic_run_stack. */
IC_API ic_status ic_decode_step(const char* pattern, int32_t n_layers, const ic_layer* layers,
                         const ic_shape* shape, const int32_t* seq_len, int32_t* idx_cache,
                         void* ws, size_t ws_bytes, ic_stats* stats, void* stream);

/* The decode step's kernels one at a time (the same launches ic_decode_step makes), so a
 * caller can time or compose them.  Shapes as ic_decode_step (Lq = 1, Lk = cache capacity).
 *
 * Lightning-indexer scores of one F layer's new queries (arXiv abstract: the indexer
 * scores every preceding token): sequence b's query q_I [B, 1, H_I, d_I], w [B, 1, H_I]
 * against keys 0..seq_len[b]-1 of k_I [B, Lk, d_I]; scores [B, row_stride] fp32 (row_stride
 * >= Lk), row b written for its first seq_len[b] entries (seq_len device int32 [B], values
 * clamped to 1..Lk).  The top-k of these rows is ic_topk_rows_seq.  No workspace. */
IC_API ic_status ic_decode_indexer_scores(const ic_shape* shape, const void* q_I, const float* w, const void* k_I,
                                          const int32_t* seq_len, float* scores, int64_t row_stride, void* stream);

/* Sparse attention of one decode layer (arXiv abstract: core attention over the k selected
 * tokens): q [B, 1, H, d], kv [B, Lk, 2, d], idx [B, 1, k] -> out [B, 1, H, d] bf16, with
 * the same entry rules as ic_sparse_attn.  Each query's rows are split over several waves
 * and merged in a fixed order (deterministic); the partials need
 * ic_workspace_size(shape, IC_OP_DECODE_ATTN) bytes of ws. */
IC_API ic_status ic_decode_attn(const ic_shape* shape, const void* q, const void* kv, const int32_t* idx, void* out,
                                void* ws, size_t ws_bytes, void* stream);

/* Scratch bytes ic_decode_step_static can use on each GPU (32 MiB). */
#define IC_DECODE_STATIC_SCRATCH_BYTES (32u << 20)

/* ic_decode_step for callers that cannot allocate or pass a workspace: code under HIP
 * graph capture that may not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation.  Same arguments minus the workspace, same kernels, same results.  The
 * scratch is a fixed array of IC_DECODE_STATIC_SCRATCH_BYTES inside the library, one per
 * GPU, which that GPU holds from the library's first use on it until the process ends.
 * A shape whose ic_workspace_size(shape, IC_OP_DECODE_STEP) exceeds it fails with
 * IC_ERR_WORKSPACE before any launch (decode64k, B = 32 x 65600 keys, needs about 13 MB).
 * Nothing is allocated.  Every call on a GPU shares that GPU's array and leaves its last
 * contents there: calls that overlap on one GPU (on different streams, or from several
 * threads) race on it, so the caller must order them. */
IC_API ic_status ic_decode_step_static(const char* pattern, int32_t n_layers, const ic_layer* layers,
                                       const ic_shape* shape, const int32_t* seq_len, int32_t* idx_cache,
                                       ic_stats* stats, void* stream);

/* Cross-layer overlap of two index caches, the diagnostic the agent skill page
 * (Step 1) uses to choose which layers may share indices: per row r of idx_a,
 * idx_b [rows, k] int32 (each row ascending and then -1 padded, as the top-k
 * writes it; k <= 4096), inter[r] = |A & B|, jaccard[r] = inter / (|A | B| +
 * 1e-8) and recall[r] = inter / |B| (0 when B is empty).  Any of inter,
 * jaccard, recall may be NULL; means (NULL, or 2 floats) receives the means of
 * jaccard and recall over the rows, summed in a fixed order, and then needs
 * jaccard and recall.  All pointers are device pointers. */
IC_API ic_status ic_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t rows, int32_t k,
                                  int32_t* inter, float* jaccard, float* recall, float* means, void* stream);

/* Multi-layer distillation loss, forward only (arXiv abstract: training-aware
 * IndexCache trains each retained indexer against the averaged attention
 * distributions of all the layers it serves; gist.science summary,
 * "Methodologie": a KL divergence to that average).  For one F layer and the
 * n_served layers it serves (itself first, then its S layers; 1..16), per
 * query t of sequence b, over its entries S_t = { idx[b,t,j] : 0 <= idx <=
 * pos0 + t } (the F layer's top-k; listing every visible key gives the dense
 * loss; other entries are ignored, and every row needs at least one):
 *   p[s] = mean over the served layers and their H heads of
 *          softmax over S_t of q[t,h] . K[s] / sqrt(d)
 *   r[s] = softmax over S_t of the F layer's indexer scores I[t,s]
 *   kl[b,t] = sum over S_t of p[s] (ln p[s] - ln r[s])      (nats, fp32)
 * q_I [B,Lq,H_I,d_I], w [B,Lq,H_I], k_I [B,Lk,d_I]: the F layer's indexer
 * inputs (shape.idx_dtype); idx [B,Lq,k] int32 (k <= 4096); q and kv: HOST
 * arrays of n_served device pointers, q[j] [B,Lq,H,d] bf16 and kv[j]
 * [B,Lk,2,d] bf16; kl [B,Lq] fp32 (device); kl_mean (device, 1 float, or
 * NULL) receives the mean of kl over all B*Lq queries, summed in a fixed
 * order.  The indexer scores are recomputed in tiles of shape.chunk queries
 * into ws (ic_workspace_size(shape, IC_OP_DISTILL_KL) bytes). */
IC_API ic_status ic_distill_kl(const ic_shape* shape, const void* q_I, const float* w, const void* k_I,
                               const int32_t* idx, int32_t n_served, const void* const* q, const void* const* kv,
                               float* kl, float* kl_mean, void* ws, size_t ws_bytes, void* stream);

/* Counters of the last stack call on this thread. */
IC_API ic_status ic_get_stats(ic_stats* out);

/* Description of the last failure on this thread ("" if none). */
IC_API const char* ic_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
IC_API int32_t ic_version(void);

#ifdef __cplusplus
}
#endif

#endif /* INDEXCACHE_H */
