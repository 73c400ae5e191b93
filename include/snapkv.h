/*
 * snapkv.h -- C ABI of libsnapkv: SnapKV prefill-time KV-cache compression on
 * one AMD MI355X (gfx950).
 *
 * The method is the one described on the page
 * "論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮"
 * (0h-n0.github.io/posts/paper-2404-14469/):
 *   - プロンプトの分割: each request of L tokens is split into a prefix of
 *     P = L - L_obs positions and an observation window of the last L_obs.
 *   - 投票メカニズム: for every query head, the L_obs window queries attend
 *     (softmax of q k^T / sqrt(d)) to the keys; the weights are summed over the
 *     window rows into a vote C per prefix position.  Under grouped-query
 *     attention the G = H_q / H_kv query heads that share a KV head add their
 *     votes (query head h reads KV head h / G).
 *   - クラスタリングによる文脈保持: C is max-pooled with width K_pool, stride 1,
 *     padding K_pool/2 (windows are clipped at the prefix ends).
 *   - top-k: k = floor(p * P) (ratio mode) or min(budget, P) (budget mode)
 *     positions per (request, KV head), ties broken toward the lower position,
 *     emitted in ascending order (アルゴリズム listing: top-k, then sort).
 *   - the chosen K/V rows are gathered and the full window K/V is appended.
 * Softmax denominator: by default every key a window row can see, i.e. the
 * prefix plus the window up to and including the row's own position (causal
 * inside the window).  SNAPKV_PREFIX_ONLY selects the listing's variant whose
 * softmax runs over the prefix keys only.
 *
 * Conventions shared by every call:
 *   - Device pointers unless a name ends in _host.  The caller owns every
 *     buffer; the library never allocates and keeps no per-call state.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without synchronising.  Outputs are valid once the
 *     stream reaches that point.  Calls on different streams must use
 *     different workspaces.
 *   - All argument checks run on the host before any launch: on an error the
 *     call returns a negative snapkv_status, launches nothing and writes
 *     nothing.  After launching, a HIP launch error returns SNAPKV_EHIP and
 *     leaves the outputs undefined.
 *   - Pointers must be 16-byte aligned and K/V strides must keep every row
 *     16-byte aligned.  Inputs and outputs must not alias.  Inputs must be
 *     finite (not checked: a check would cost a pass over K).
 *
 * Layouts (elements of the problem's dtype unless stated):
 *   q_obs   [B][H_q][L_obs][d], contiguous: the last L_obs queries of every
 *           request and query head.
 *   K, V    token-packed: element (g, t, c) at g*kv_head_stride +
 *           t*kv_token_stride + c, t in [0, T), T = cu_seqlens[B]; request r
 *           owns tokens [cu_seqlens[r], cu_seqlens[r+1]).  Head-major
 *           [H_kv][T][d] and token-major [T][H_kv][d] are both expressible.
 *   votes,
 *   pooled  float32 [H_kv][sum_r P_r]: (g, r, j) at g*sum_P + cu_pfx[r] + j.
 *   idx     int32 [H_kv][sum_r k_r]: (g, r, t) at g*sum_k + cu_k[r] + t, the
 *           request-local prefix positions in [0, P_r), strictly ascending.
 *   K_out,
 *   V_out   [H_kv][sum_r (k_r + L_obs)][d], contiguous: rows cu_out[r] ..
 *           cu_out[r+1]-1 of head g hold request r's chosen rows (ascending
 *           position) followed by its L_obs window rows in order.
 */
#ifndef SNAPKV_H
#define SNAPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SNAPKV_OK = 0,
    SNAPKV_EINVAL = -1,       /* an argument is invalid (message: snapkv_last_error) */
    SNAPKV_EWORKSPACE = -2,   /* workspace missing, misaligned or smaller than snapkv_plan asks */
    SNAPKV_EUNSUPPORTED = -3, /* valid but not supported: head_dim, G*L_obs > 1024, device */
    SNAPKV_EHIP = -4          /* the HIP runtime reported an error */
} snapkv_status;

typedef enum { SNAPKV_F32 = 0, SNAPKV_BF16 = 1 } snapkv_dtype;
typedef enum { SNAPKV_RATIO = 0, SNAPKV_BUDGET = 1 } snapkv_mode;
typedef enum { SNAPKV_CAUSAL_WINDOW = 0, SNAPKV_PREFIX_ONLY = 1 } snapkv_variant;

/* flags */
#define SNAPKV_FLAG_TWO_PASS 0x1u /* score with two passes over K (stats, then votes) */
#define SNAPKV_FLAG_STREAM 0x2u   /* score with the streaming two-phase kernel (rows of 256 bytes,
                                     G * L_obs <= 256; chosen by itself for grouped-query heads
                                     and the lse calls) */
#define SNAPKV_FLAG_FUSED 0x4u    /* score with the fused barrier kernel (logits resident, one grid
                                     iteration per set of whole segments).  Without a flag, rows of
                                     256 bytes with G * L_obs <= 32 use a one-read kernel: the
                                     single-slot one when the group's 2048-key items fit one pass of
                                     the resident grid (256 workgroups on an MI355X), else the
                                     two-slot one when no segment has more than twice the grid's
                                     1024-key items (524288 tokens), else the two-phase kernel; other
                                     problems use the two-phase kernel when it takes them, then the
                                     fused kernel, then two passes.  The three flags exclude each
                                     other. */
#define SNAPKV_FLAG_SELECT_ONE_WG 0x8u /* top-k of segments of up to 32768 positions with one
                                     workgroup per segment.  Without it, when a launch group has a
                                     segment of more than 16384 positions, such segments are split
                                     over workgroups of 8192 positions that wait for each other
                                     (needs the launch's whole grid resident at once, which the
                                     library checks with the occupancy API: a caller running other
                                     kernels on the device at the same time should set it) */

typedef struct {
    int32_t batch;            /* B >= 1 requests */
    int32_t num_q_heads;      /* H_q >= 1 */
    int32_t num_kv_heads;     /* H_kv >= 1, H_q % H_kv == 0 */
    int32_t head_dim;         /* d: 64 or 128 */
    int32_t obs_window;       /* L_obs >= 1 */
    int32_t pool_kernel;      /* K_pool, odd, >= 1 */
    int32_t mode;             /* snapkv_mode */
    int32_t dtype;            /* snapkv_dtype of q_obs, K, V, K_out, V_out */
    int32_t variant;          /* snapkv_variant */
    uint32_t flags;           /* SNAPKV_FLAG_* */
    double ratio;             /* p in (0, 1], ratio mode */
    int64_t budget;           /* >= 0, budget mode */
    int64_t kv_head_stride;   /* elements between KV heads of K and V */
    int64_t kv_token_stride;  /* elements between tokens of K and V */
    const int32_t *cu_seqlens_host; /* host [B+1]: 0 = cu[0] <= ..., L_r = cu[r+1]-cu[r] >= L_obs */
} snapkv_problem;

/*
 * snapkv_plan -- validate a problem and size its outputs and workspace.
 * Host only; touches no device.  Every output pointer may be NULL.
 *   k_host      [B]   : k_r = floor(p * P_r) or min(budget, P_r)
 *                       (投票メカニズム: k = floor(p * L_prefix); listing: min(max_cap, pfx)).
 *   cu_pfx_host [B+1] : exclusive prefix sums of P_r (votes/pooled offsets).
 *   cu_k_host   [B+1] : exclusive prefix sums of k_r (idx offsets).
 *   cu_out_host [B+1] : exclusive prefix sums of k_r + L_obs (K_out/V_out rows).
 *   ws_bytes          : workspace bytes that snapkv_scores, snapkv_select and
 *                       snapkv_compress need for this problem (device
 *                       independent; 0 is never returned).
 * Workspace contract: zero-fill it once before its first use.  Every call
 * leaves its counters and tagged slots at zero again, so later calls (also
 * under graph replay) need no clearing.  Where they lie depends on the
 * problem: a call whose counters lie elsewhere than those of the previous call
 * on the same workspace (same address and device; another shape reusing it)
 * first zeroes its own with one small kernel on its stream.  The first 4 bytes hold a sticky error
 * word that only the caller clears:
 *   bit 0 = a scoring workgroup gave up waiting for others of its launch.  The
 *           fused and the one-read kernels need all workgroups of a (request,
 *           KV head) segment resident at once (their grid never exceeds what the
 *           device keeps resident); other work holding part of the GPU for
 *           about a second can break that.  The two-phase streaming kernel only
 *           waits for workgroups already running.
 *   bit 1 = a counter was not zero when a call started (the workspace was not
 *           zero-filled, or was shared by calls running at the same time).
 *   bit 2 = a row's sum of exponentials still overflowed after 8 raises of its
 *           shift (needs logits spanning more than about 2^100 in one slab).
 * With any bit set the outputs of the calls since it was last clear may be
 * invalid; SNAPKV_FLAG_TWO_PASS, which has no wait and no shift, computes them.
 * Returns SNAPKV_OK or SNAPKV_EINVAL / SNAPKV_EUNSUPPORTED.
 */
int snapkv_plan(const snapkv_problem *pb, int64_t *k_host, int64_t *cu_pfx_host, int64_t *cu_k_host,
                int64_t *cu_out_host, size_t *ws_bytes);

/*
 * snapkv_scores -- votes and pooled votes (投票メカニズム; クラスタリングによる文脈保持).
 *   q_obs, K : inputs as laid out above (dtype of the problem).
 *   votes    : out, float32 [H_kv][sum_P], or NULL to skip writing C.
 *   pooled   : out, float32 [H_kv][sum_P], max pooled votes.
 *   ws       : device workspace of at least snapkv_plan's ws_bytes, 256-byte
 *              aligned, zero-filled before its first use (see snapkv_plan).
 */
int snapkv_scores(const snapkv_problem *pb, const void *q_obs, const void *K, float *votes, float *pooled,
                  void *ws, size_t ws_bytes, void *stream);

/*
 * snapkv_select -- top-k of the pooled votes per (request, KV head): the k_r
 * largest values, ties to the lower position, written ascending
 * (投票メカニズム I = Top_k; アルゴリズム listing: topk then sort).
 *   pooled : float32 [H_kv][sum_P], values >= 0 (as snapkv_scores writes them).
 *   idx    : out, int32 [H_kv][sum_k].
 */
int snapkv_select(const snapkv_problem *pb, const float *pooled, int32_t *idx, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * snapkv_gather -- compressed cache rows (アルゴリズム listing: gather per head,
 * then concat with the window).  Copies bytes; no arithmetic.
 *   K, V         : inputs (strided as above).
 *   idx          : int32 [H_kv][sum_k], ascending request-local positions < P_r.
 *   K_out, V_out : out, [H_kv][sum_out][d] contiguous.
 */
int snapkv_gather(const snapkv_problem *pb, const void *K, const void *V, const int32_t *idx, void *K_out,
                  void *V_out, void *stream);

/*
 * snapkv_compress -- the whole path: scores, select, gather.
 *   idx    : out, int32 [H_kv][sum_k], or NULL (then kept in the workspace).
 *   pooled : out, float32 [H_kv][sum_P], or NULL (then kept in the workspace).
 */
int snapkv_compress(const snapkv_problem *pb, const void *q_obs, const void *K, const void *V, void *K_out,
                    void *V_out, int32_t *idx, float *pooled, void *ws, size_t ws_bytes, void *stream);

/*
 * snapkv_scores_lse, snapkv_compress_lse -- the same outputs as snapkv_scores and
 * snapkv_compress from a single read of K, for callers that already hold every window
 * row's softmax normaliser (prefill attention computes it for these rows):
 *   lse : float32 [B][H_q][L_obs], contiguous, 16-byte aligned: lse[r][h][i] =
 *         ln sum_j exp(q . k_j / sqrt(d)) over exactly the keys row i sees under the
 *         problem's variant (prefix plus window up to the row for SNAPKV_CAUSAL_WINDOW,
 *         the prefix only for SNAPKV_PREFIX_ONLY); -infinity for a row that sees no key.
 * The weights are exp(q . k_j / sqrt(d) - lse), so a wrong lse scales that row's
 * weights instead of being detected.  Same conventions and errors as the calls above;
 * SNAPKV_FLAG_TWO_PASS has no effect (there is no stats pass).
 */
int snapkv_scores_lse(const snapkv_problem *pb, const void *q_obs, const void *K, const float *lse, float *votes,
                      float *pooled, void *ws, size_t ws_bytes, void *stream);
int snapkv_compress_lse(const snapkv_problem *pb, const void *q_obs, const void *K, const void *V, const float *lse,
                        void *K_out, void *V_out, int32_t *idx, float *pooled, void *ws, size_t ws_bytes,
                        void *stream);

/*
 * snapkv_compress_noalloc -- snapkv_compress for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * takes no workspace: its workspace is a device array of SNAPKV_NOALLOC_SCRATCH_BYTES inside
 * the library, one per device, which the library holds until the process ends.  The call
 * itself allocates nothing; the caller still provides every input and output.
 *   q_obs, K, V, K_out, V_out, idx, pooled : as for snapkv_compress.
 *   error_word : out, device uint32 (4-byte aligned) or NULL: receives the call's error bits
 *                (the same bits as the workspace error word described under snapkv_plan),
 *                which the call then clears in its array.
 * A problem whose snapkv_plan ws_bytes exceeds SNAPKV_NOALLOC_SCRATCH_BYTES returns
 * SNAPKV_EWORKSPACE before any launch.  The first call on a device zero-fills the array on
 * `stream`.  Every call on a device shares that device's array: calls that overlap in time on
 * one device (other streams, other threads) race and give wrong results; order them.
 */
#define SNAPKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int snapkv_compress_noalloc(const snapkv_problem *pb, const void *q_obs, const void *K, const void *V, void *K_out,
                            void *V_out, int32_t *idx, float *pooled, uint32_t *error_word, void *stream);

/*
 * snapkv_hit_rate -- the Hit Rate of a selection (section Hit Rate（適中率）の定式化):
 * for each (request, KV head), `above` = the prefix positions whose attention in the
 * current generation step exceeds theta (strictly), and `hits` = those among them that
 * the selection kept.  The rate is hits / above (undefined, NaN, when above = 0); sums of
 * the counts give the rate over several heads or requests.
 *   a_cur  : float32 [H_kv][sum_P] (the votes layout), attention to each prefix position.
 *   idx    : int32 [H_kv][sum_k], strictly ascending per (request, KV head), as
 *            snapkv_select writes it.
 *   theta  : threshold (the page uses 0.05); compared in double against each value.
 *   counts : out, uint32 [B][H_kv][2] = (hits, above); every entry is written, so it
 *            needs no initial value.
 * No workspace.  Errors as for the other calls (theta NaN -> SNAPKV_EINVAL).
 */
int snapkv_hit_rate(const snapkv_problem *pb, const float *a_cur, const int32_t *idx, double theta, uint32_t *counts,
                    void *stream);

/*
 * Decode attention over the compressed cache -- the step after the compression (page
 * section デコード速度とメモリ効率; the KV-cache chapter's decode step): one new query row
 * per (request, query head) attends to every cached row of its KV head,
 *   out[r][h] = sum_j softmax_j(q[r][h] . K[g][j] / sqrt(d)) V[g][j],  g = h / G,
 * over the rows j of request r: cu_rows_host[r] .. cu_rows_host[r+1]-1 (snapkv_plan's
 * cu_out for a cache that snapkv_compress wrote; rows appended since are just a longer
 * range).  A request with no rows gets zeros.
 *   q      : [B][H_q][d] of the problem's dtype, contiguous.
 *   K, V   : element (g, t, c) at g*kv_head_stride + t*kv_token_stride + c (K_out/V_out
 *            of snapkv_compress: kv_head_stride = sum_out*d, kv_token_stride = d).
 *   out    : float32 [B][H_q][d].
 *   ws     : snapkv_decode_plan's ws_bytes (no zero-fill needed), 256-byte aligned.
 * Supported: rows of 256 bytes (bf16 d = 128, fp32 d = 64); otherwise SNAPKV_EUNSUPPORTED.
 */
typedef struct {
    int32_t batch;            /* B >= 1 */
    int32_t num_q_heads;      /* H_q */
    int32_t num_kv_heads;     /* H_kv, H_q % H_kv == 0 */
    int32_t head_dim;         /* d */
    int32_t dtype;            /* snapkv_dtype */
    int64_t kv_head_stride;   /* elements */
    int64_t kv_token_stride;  /* elements, >= d */
    const int64_t *cu_rows_host; /* host [B+1], non-decreasing, cu_rows_host[0] >= 0 */
} snapkv_decode_problem;

int snapkv_decode_plan(const snapkv_decode_problem *dp, size_t *ws_bytes);
int snapkv_decode(const snapkv_decode_problem *dp, const void *q, const void *K, const void *V, float *out, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * Kernel trace (profiling hook).  While a trace is open on the calling thread,
 * the i-th kernel a snapkv_* call launches (i < n_pairs) carries events[2i] and
 * events[2i+1] as the start and stop events of its dispatch
 * (hipExtLaunchKernel), so their elapsed time is that kernel's own duration on
 * the launch stream; later launches are not recorded.  The events are the
 * caller's hipEvent_t handles, created with timing enabled.
 *   snapkv_trace_begin: opens a trace (events non-NULL, n_pairs >= 1).
 *   snapkv_trace_end  : closes it, writes the snapkv_kernel_id of each recorded
 *                       launch into kernel_ids[0 .. min(count, capacity)) and
 *                       returns count (>= 0).
 */
typedef enum {
    SNAPKV_K_RESERVED0 = 0,   /* not launched (ids stay stable) */
    SNAPKV_K_OBS_FUSED = 1,   /* obs_score, logits resident, one read of K */
    SNAPKV_K_OBS_STATS = 2,   /* obs_score two-pass: row stats */
    SNAPKV_K_STATS_MERGE = 3, /* obs_score two-pass: merge of row stats */
    SNAPKV_K_OBS_VOTES = 4,   /* obs_score two-pass: votes */
    SNAPKV_K_POOL = 5,        /* vote_pool */
    SNAPKV_K_SELECT = 6,      /* topk_select */
    SNAPKV_K_GATHER = 7,      /* kv_gather */
    SNAPKV_K_SUM_CHUNKS = 8,  /* sum of the votes of the row chunks (G * L_obs > 32) */
    SNAPKV_K_SELECT_TILES = 9, /* topk_select of segments longer than 32768 positions (3 launches) */
    SNAPKV_K_HIT_RATE = 10,    /* snapkv_hit_rate */
    SNAPKV_K_DECODE = 11,      /* snapkv_decode: split-K partials */
    SNAPKV_K_DECODE_COMBINE = 12, /* snapkv_decode: merge of the splits */
    SNAPKV_K_HIT_CLEAR = 13,      /* snapkv_hit_rate: zeroes the counts its tiles add to */
    SNAPKV_K_SCRATCH_CLEAR = 14,  /* snapkv_compress_noalloc: zero-fills the device's array (first call) */
    SNAPKV_K_OBS_STREAM = 15,     /* obs_score, streaming two-phase kernel (work tickets, no barrier) */
    SNAPKV_K_OBS_ONEPASS = 16,    /* obs_score, streaming one-read kernel (<= 32 rows, weights resident) */
    SNAPKV_K_OBS_ONEPASS2 = 17,   /* obs_score, one-read kernel with two items in flight per workgroup
                                     (<= 32 rows, long segments) */
    SNAPKV_K_WS_CLEAR = 18,       /* zeroes a workspace's counters when its layout changed */
    SNAPKV_K_SELECT_SPLIT = 19    /* topk_select with segments of up to 32768 positions split over
                                     workgroups of 8192 positions (all resident, two meetings) */
} snapkv_kernel_id;

int snapkv_trace_begin(void *const *events, int n_pairs);
int snapkv_trace_end(int32_t *kernel_ids, int capacity);

/* Name of a snapkv_kernel_id ("obs_score_fused", ...); never NULL. */
const char *snapkv_kernel_name(int id);

/* Text of a status code; never NULL. */
const char *snapkv_strerror(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *snapkv_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int snapkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SNAPKV_H */
