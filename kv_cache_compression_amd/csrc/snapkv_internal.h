// snapkv_internal.h -- shared between the host API and the gfx950 kernels of libsnapkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace snapkv {

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so register arrays
// are only ever indexed by constants (no reliance on the unroller).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Requests handled by one group of launches.  Larger batches are cut into
// groups; the per-request table travels as a kernel argument (no copies).
constexpr int kMaxReq = 32;
// Barrier counters sit one 256-byte line apart, so the polls of different segments do not
// pile onto one memory channel while other workgroups still stream keys.
constexpr int kCounterStride = 64;  // uint32 words

struct ReqTable {
    int32_t n;                    // requests in this group
    int32_t L[kMaxReq];           // request length
    int32_t k[kMaxReq];           // kept prefix positions
    int32_t qi[kMaxReq];          // request index into q_obs
    int32_t slab0[kMaxReq + 1];   // first slab of the request (all KV heads), cumulative
    int64_t tok0[kMaxReq];        // first token in K/V
    int64_t pfx0[kMaxReq];        // first column in votes/pooled
    int64_t k0[kMaxReq];          // first column in idx
    int64_t out0[kMaxReq];        // first row in K_out/V_out
};

// Scoring kernel modes.
enum ObsMode : int {
    kFused = 0,   // logits stay in registers: local stats, per-segment barrier, votes
    kStats = 1,   // first pass of the two-pass path: per-slab (max, sum-exp)
    kVotes = 2    // second pass: logits again, normalised by merged stats
};

struct ObsParams {
    const void *q;              // q_obs
    const void *K;
    float *votes;               // [H_kv][sum_P]
    float2 *partial;            // [slabs][M_pad]: (max of raw logits, sum of exp2((s-max)*c))
    const float2 *merged;       // [segments][M_pad]: merged (max, sum) for kVotes
    uint32_t *counters;         // [segments * kCounterStride]: arrival count (kFused)
    uint32_t *err;              // error word (bit 0: a barrier wait gave up; bit 1: counters not zero)
    int64_t head_stride;        // elements
    int64_t token_stride;       // elements
    int64_t sum_P;
    int32_t Hq, Hkv, G, w, M, M_pad, variant;
    float c;                    // log2(e) / sqrt(d)
    int32_t n_slabs;            // slabs in this group
    int32_t slab_keys;          // keys per slab
    uint32_t spin_limit;        // polls before a barrier wait gives up
    int32_t n_chunks;           // row chunks of kChunkRows query rows per KV head
    int64_t vplane;             // floats between the votes planes of consecutive chunks
    const float *lse;           // kVotes: caller's row log-sum-exp [B][H_q][L_obs] instead of merged
    float lse_scale;            // sqrt(d): lse * lse_scale * c = lse * log2(e)
    // Packed item order (kFused over several grid iterations): request i's items start at
    // slot vb[i] of a sequence of pack_grid-slot iterations, and no (request, KV head)
    // segment crosses an iteration boundary (see packed_item).  pack_grid = 0: items in
    // their natural order, slot = item.
    int32_t pack_grid;
    int32_t vb[kMaxReq + 1];
    ReqTable rt;
};

// Query rows scored by one kernel pass (a row chunk); heads with more rows (G * L_obs)
// are scored chunk by chunk into separate votes planes that are then summed.
constexpr int kChunkRows = 32;
constexpr int kMaxRows = 1024;  // longest G * L_obs

struct ObsConfig {
    int wr, wk, rtw, ctw;       // waves over rows, waves over keys, 16-row tiles / wave, 16-key tiles / wave
    int threads() const { return 64 * wr * wk; }
    int slab_keys() const { return wk * ctw * 16; }
    int rows() const { return wr * rtw * 16; }
};

// Chooses the tile shape for (dtype, d); false if unsupported.
bool obs_config(int dtype, int d, ObsConfig *cfg);
// The shorter-slab shape for (dtype, d), where one exists (rows of 256 bytes).
bool obs_config_short(int dtype, int d, ObsConfig *cfg);
// Kernel entry of the chosen instantiation; keep = cached key loads.
const void *obs_kernel(int dtype, int d, const ObsConfig &cfg, int mode, bool keep);

// Streaming two-phase scoring (persistent grid, work tickets).  Items are (request, KV head,
// slab of slab_keys keys) in request-major order; every item is visited twice: a stats pass
// (row max and sum of exponentials over the slab's keys) and a votes pass (weights
// normalised by the segment's merged row stats).  Ticket t maps to a pass and an item so that
// every stats item of a segment precedes every votes item of it (lag >= items per segment).
struct StreamParams {
    const void *q;              // q_obs
    const void *K;
    float *votes;               // [H_kv][sum_P]
    float2 *partial;            // [items][M_pad]: (shift, sum of exp2(s*c - shift)) per stats item and row
    float *final_shift;         // [segments][M_pad]: shift + log2(sum) of the whole segment
    uint32_t *ticket;           // one counter (own 256-byte line); returns to zero after every launch
    uint32_t *seg_ctl;          // [segments][3 lines of 64 words]: stats done, stats ready, votes started
    uint32_t *err;              // error word (bit 0: a wait gave up)
    const float *lse;           // caller's row log-sum-exp [B][H_q][L_obs]: votes pass only
    int64_t head_stride, token_stride, sum_P;
    int32_t Hq, Hkv, G, w, M, M_pad, variant;
    float c;                    // log2(e) / sqrt(d)
    int32_t n_items;            // items of this group (each visited by both passes)
    int32_t slab_keys;          // keys per item (multiple of 64)
    int32_t lag;                // stats items issued before the first votes item (two-phase kernel)
    uint32_t spin_limit;
    ReqTable rt;                // slab0 counts items of slab_keys
};
constexpr int kStreamSegLine = 64;  // uint32 words per control line
// rows = 32, 64, 128 or 256 (>= G * L_obs), keys of 256 bytes; *threads = its workgroup size
const void *stream_kernel(int dtype, int rows, int *threads);
// one-read streaming kernel for up to 32 rows per KV head, keys of 256 bytes; *threads = its
// workgroup size, *slab = the keys of one item
const void *onepass_kernel(int dtype, int *threads, int *slab);
// the same with several items in flight per workgroup; *slots = items held at once (a segment
// may have up to slots x grid items)
const void *onepass2_kernel(int dtype, int *threads, int *slab, int *slots);

struct MergeParams {
    const float2 *partial;
    float2 *merged;
    int32_t M, M_pad, slab_keys, Hkv, n_chunks;
    float c;
    ReqTable rt;
};
const void *merge_kernel();

struct SumParams {
    const float *planes;        // [n_chunks][H_kv][sum_P]
    float *votes;               // [H_kv][sum_P]
    int64_t sum_P, vplane, col0, col1;  // columns [col0, col1) of every KV head
    int32_t n_chunks;
};
const void *sum_kernel();

struct PoolParams {
    const float *votes;
    float *pooled;
    int64_t sum_P;
    int32_t w, half;            // half = K_pool / 2
    ReqTable rt;
};
const void *pool_kernel();

struct SelectParams {
    const float *votes;         // votes to pool first (segments held in LDS), or null
    const float *pooled;        // pooled votes to select from when votes is null
    float *pooled_out;          // pooled votes written here when pooling here, or null
    int32_t *idx;               // chosen positions, or null (pooling only)
    int64_t sum_P, sum_k;
    int32_t w, Hkv, half;       // half = K_pool / 2
    ReqTable rt;
};
const void *select_kernel();
int select_threads();
int select_lds_positions();     // longest segment selected from LDS / registers
int select_max_half(int max_P); // widest pool half-width (K_pool / 2) the select kernel pools itself

// Per-segment state of the long-segment select (64 bytes; zero in a fresh workspace, and
// the counters return to zero after every call).
struct LongState {
    uint32_t arrived;           // tiles arrived in the current phase
    uint32_t ncand;             // candidates appended in phase 1
    uint32_t prefix, mask, need, done;
    uint32_t pad[10];
};

struct LongParams {
    const float *votes;         // raw votes to pool in phase 0, or null (pooled given)
    float *pooled;              // pooled votes: written in phase 0 when votes is set, read after
    int32_t *idx;
    LongState *state;           // [segments]
    uint32_t *ghist;            // [segments][4096]
    uint32_t *cand;             // [H_kv][sum_P] candidate values
    uint32_t *tilecnt;          // [segments][max_tiles][4]: above first bin, candidate start, count, packed counts
    int64_t sum_P, sum_k;
    int32_t w, Hkv, half, phase, max_tiles;
    ReqTable rt;
};
const void *long_kernel();
int select_tile_positions();
int long_threads();             // workgroup size of long_kernel

// Top-k with a segment of up to 32768 positions split over workgroups of split_chunk()
// positions that wait for each other (every workgroup of the launch must be resident at once).
constexpr int kSplitLine = 64;       // uint32 words per counter line
constexpr int kSplitMaxChunks = 4;   // chunks of the longest segment it takes
struct SplitParams {
    const float *votes;         // raw votes to pool, or null (pooled given)
    const float *pooled;        // pooled votes to select from when votes is null
    float *pooled_out;          // pooled votes written here when pooling here, or null
    int32_t *idx;
    uint32_t *ctl;              // [segments][2 lines]: the two meetings' counters (zero between calls)
    uint32_t *ghist;            // [segments][4096 + 64]: histogram of bits 30..19, its block sums (zero between calls)
    uint32_t *cand;             // [H_kv][sum_P]: each chunk's candidates in its own columns
    uint32_t *rec;              // [segments][kSplitMaxChunks]: (count above the bin) | (count in it) << 16
    uint32_t *err;              // error word (bit 0: a wait gave up)
    int64_t sum_P, sum_k;
    int32_t w, Hkv, half;       // half = K_pool / 2 (<= split_max_half())
    uint32_t spin_limit;
    int32_t wg0[kMaxReq + 1];   // first workgroup of each request's segments (no workgroups when
                                // P <= 0 or P > 32768)
    ReqTable rt;
};
const void *split_kernel(int threads);  // 1024 (8 positions per thread) or 512 (16)
int split_chunk();
int split_max_half();

struct HitParams {
    const float *a_cur;         // [H_kv][sum_P]
    const int32_t *idx;         // [H_kv][sum_k], ascending per segment
    uint32_t *counts;           // [B][H_kv][2]: (kept and above theta, above theta)
    double theta;
    int64_t sum_P, sum_k;
    int32_t w, Hkv;
    ReqTable rt;
};
const void *hit_kernel();
struct ClearParams {
    uint32_t *data;
    int32_t n;
};
const void *hit_clear();       // zeroes data[0, n); grid ceil(n / 256) x 256 threads (also used to clear scratch)
constexpr int kMaxClearRanges = 4;
struct WsClearParams {
    unsigned char *base;
    int64_t off[kMaxClearRanges];  // byte offsets (16-byte aligned)
    int64_t n16[kMaxClearRanges];  // lengths in 16-byte units
    int32_t n_ranges;
};
const void *ws_clear();        // zeroes the ranges; any grid of 256-thread workgroups
int hit_tile_positions();      // positions per hit_rate workgroup (grid x = tiles of the longest)

struct DecodeParams {
    const void *q;              // [B][H_q][d]
    const void *K, *V;          // cache rows (token-packed, as for compression)
    float *part;                // [items][max_splits][head_tile][d + 2] partials
    float *out;                 // [B][H_q][d] fp32
    int64_t head_stride, token_stride;  // elements
    int32_t Hq, Hkv, G, d, n_hchunks, head_tile, max_splits, split_rows;
    float c;                    // log2(e) / sqrt(d)
    ReqTable rt;                // L = cached rows, tok0 = first row, qi = request
};
const void *decode_partial_kernel_for(int dtype, int head_tile);
const void *decode_combine_kernel_ptr();
int decode_threads();
int decode_rows_per_iter();
int decode_max_splits();      // splits one combine workgroup merges

struct GatherParams {
    const void *K, *V;
    const int32_t *idx;
    void *K_out, *V_out;
    int64_t head_stride, token_stride;  // elements of the input
    int64_t sum_k, sum_out;
    int32_t row_bytes, esz, w, Hkv;
    uint32_t *err_word;         // when set: copied to err_out (if set) and cleared by thread 0 of block (0, 0)
    uint32_t *err_out;
    ReqTable rt;
};
const void *gather_kernel();
int gather_rows_per_thread();


}  // namespace snapkv
