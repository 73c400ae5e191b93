// api.hip -- host side of libsnapkv: validation, planning, workspace layout, launches.
//
// Every argument check runs here before the first launch, so an invalid call writes
// nothing.  The per-request table travels as a kernel argument; batches larger than
// kMaxReq requests run as several groups of launches on the same stream.
#include <math.h>
#include <string.h>

#include <mutex>
#include <unordered_map>
#include <string>
#include <vector>

#include <hip/hip_ext.h>

#include "snapkv.h"
#include "snapkv_internal.h"

using namespace snapkv;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

constexpr size_t kWsAlign = 256;
constexpr uint32_t kSpinLimit = 1u << 20;  // polls of a barrier counter before giving up (~1 s)

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct Group {
    ReqTable rt;
    int n_slabs;       // slabs of all KV heads of the group's requests
    int max_ns;        // largest slab count of one (request, KV head)
    int max_P;         // largest prefix in the group
    int64_t out_rows;  // output rows of the group per KV head
};

struct Plan {
    int B, Hq, Hkv, d, w, K_pool, mode, dtype, variant;
    uint32_t flags;
    int G, M, M_pad, n_chunks, esz, row_bytes;
    double ratio;
    int64_t budget, head_stride, token_stride;
    std::vector<int64_t> L, P, k, cu_pfx, cu_k, cu_out;
    int64_t sum_P, sum_k, sum_out;
    ObsConfig cfg;
    std::vector<Group> groups;
    int max_group_slabs, max_group_segs;
    int64_t max_P;
    int max_tiles;     // tiles of the longest segment (long-segment select)
    // streaming two-phase scoring (rows of 256 bytes, G * L_obs <= 256)
    bool st_ok;        // the streaming kernel supports this problem
    int st_rows;       // rows per KV head the kernel covers: 32, 64, 128 or 256 (>= M)
    int st_slab;       // keys per item
    int64_t st_max_items;  // items of the largest group
    // workspace layout (bytes)
    size_t off_err, off_cnt, off_partial, off_merged, off_planes, off_votes, off_pooled, off_idx;
    size_t off_long_state, off_ghist, off_cand, off_tilecnt;
    size_t off_split_ctl, off_split_hist, off_split_rec;  // split select: counters, histograms, records
    bool has_split;    // some segment is short enough for the split select
    size_t off_st_ticket, off_st_ctl, off_st_partial, off_st_final;
    size_t off_op_partial, off_op_final, ws_bytes;  // one-read kernel: tagged row stats, row shifts
};

// Streaming scoring: grid of two workgroups per CU (the plan assumes the MI355X's 256 CUs;
// the launch uses whatever the device keeps resident).
constexpr int kStreamNominalGrid = 512;

// Items of slab keys for the requests of one group.
static int64_t stream_items(const Plan &p, const Group &gr, int slab, int *max_ns) {
    int64_t n = 0;
    int mx = 0;
    for (int i = 0; i < gr.rt.n; ++i) {
        const int ns = (gr.rt.L[i] + slab - 1) / slab;
        n += (int64_t)ns * p.Hkv;
        mx = ns > mx ? ns : mx;
    }
    if (max_ns) *max_ns = mx;
    return n;
}

// Groups of at most kMaxReq requests, for the slab size of p.cfg.
static int build_groups(Plan &p, const int32_t *cu) {
    const int slab = p.cfg.slab_keys();
    p.groups.clear();
    p.max_group_slabs = 0;
    p.max_group_segs = 0;
    for (int r0 = 0; r0 < p.B; r0 += kMaxReq) {
        Group gr;
        memset(&gr, 0, sizeof gr);
        const int n = p.B - r0 < kMaxReq ? p.B - r0 : kMaxReq;
        gr.rt.n = n;
        int64_t slabs = 0;
        for (int i = 0; i < n; ++i) {
            const int r = r0 + i;
            gr.rt.L[i] = (int32_t)p.L[r];
            gr.rt.k[i] = (int32_t)p.k[r];
            gr.rt.qi[i] = r;
            gr.rt.slab0[i] = (int32_t)slabs;
            gr.rt.tok0[i] = cu[r];
            gr.rt.pfx0[i] = p.cu_pfx[r];
            gr.rt.k0[i] = p.cu_k[r];
            gr.rt.out0[i] = p.cu_out[r];
            const int64_t ns = (p.L[r] + slab - 1) / slab;
            slabs += ns * p.Hkv;
            if (ns > gr.max_ns) gr.max_ns = (int)ns;
            if (p.P[r] > gr.max_P) gr.max_P = (int)p.P[r];
        }
        if (slabs * p.n_chunks > (1 << 30)) return fail(SNAPKV_EUNSUPPORTED, "problem too large");
        gr.rt.slab0[n] = (int32_t)slabs;
        gr.n_slabs = (int)slabs;
        gr.out_rows = p.cu_out[r0 + n] - p.cu_out[r0];
        p.groups.push_back(gr);
        if (gr.n_slabs > p.max_group_slabs) p.max_group_slabs = gr.n_slabs;
        if (n * p.Hkv > p.max_group_segs) p.max_group_segs = n * p.Hkv;
    }
    return SNAPKV_OK;
}

static int64_t pack_segments(const Plan &p, const Group &gr, int grid, int32_t *vb);

// Estimated time of the fused scoring launches, in units of one key tile per wave: every grid
// iteration streams its slabs (CTW tiles per wave) and then pays a fixed tail (row stats,
// segment barrier, votes) of about ten tiles.  The grid is the 256 workgroups an MI355X keeps
// resident (one per CU).
static double fused_cost(const Plan &p) {
    constexpr int kGrid = 256;
    double cost = 0;
    for (const Group &gr : p.groups) {
        int32_t vb[kMaxReq + 1];
        const int64_t slots = (int64_t)gr.max_ns * p.n_chunks > kGrid ? -1 : pack_segments(p, gr, kGrid, vb);
        if (slots < 0) return 1e300;
        cost += (double)((slots + kGrid - 1) / kGrid) * (p.cfg.ctw + 10);
    }
    return cost;
}

int make_plan(const snapkv_problem *pb, Plan *pl) {
    g_last_error.clear();
    if (!pb) return fail(SNAPKV_EINVAL, "problem is NULL");
    Plan &p = *pl;
    p.B = pb->batch;
    p.Hq = pb->num_q_heads;
    p.Hkv = pb->num_kv_heads;
    p.d = pb->head_dim;
    p.w = pb->obs_window;
    p.K_pool = pb->pool_kernel;
    p.mode = pb->mode;
    p.dtype = pb->dtype;
    p.variant = pb->variant;
    p.flags = pb->flags;
    p.ratio = pb->ratio;
    p.budget = pb->budget;
    p.head_stride = pb->kv_head_stride;
    p.token_stride = pb->kv_token_stride;
    if (p.B < 1) return fail(SNAPKV_EINVAL, "batch must be >= 1");
    if (p.Hq < 1 || p.Hkv < 1) return fail(SNAPKV_EINVAL, "head counts must be >= 1");
    if (p.Hq % p.Hkv != 0) return fail(SNAPKV_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
    if (p.w < 1) return fail(SNAPKV_EINVAL, "obs_window must be >= 1");
    if (p.K_pool < 1 || p.K_pool % 2 == 0) return fail(SNAPKV_EINVAL, "pool_kernel must be odd and >= 1");
    if (p.mode != SNAPKV_RATIO && p.mode != SNAPKV_BUDGET) return fail(SNAPKV_EINVAL, "mode must be RATIO or BUDGET");
    if (p.dtype != SNAPKV_F32 && p.dtype != SNAPKV_BF16) return fail(SNAPKV_EINVAL, "dtype must be F32 or BF16");
    if (p.variant != SNAPKV_CAUSAL_WINDOW && p.variant != SNAPKV_PREFIX_ONLY)
        return fail(SNAPKV_EINVAL, "variant must be CAUSAL_WINDOW or PREFIX_ONLY");
    if (p.flags & ~(SNAPKV_FLAG_TWO_PASS | SNAPKV_FLAG_STREAM | SNAPKV_FLAG_FUSED | SNAPKV_FLAG_SELECT_ONE_WG))
        return fail(SNAPKV_EINVAL, "unknown flag bits");
    {
        const uint32_t path = p.flags & (SNAPKV_FLAG_TWO_PASS | SNAPKV_FLAG_STREAM | SNAPKV_FLAG_FUSED);
        if (path & (path - 1))
            return fail(SNAPKV_EINVAL, "SNAPKV_FLAG_TWO_PASS, SNAPKV_FLAG_STREAM and SNAPKV_FLAG_FUSED exclude each other");
    }
    if (p.mode == SNAPKV_RATIO && !(p.ratio > 0.0 && p.ratio <= 1.0))
        return fail(SNAPKV_EINVAL, "ratio must lie in (0, 1]");
    if (p.mode == SNAPKV_BUDGET && p.budget < 0) return fail(SNAPKV_EINVAL, "budget must be >= 0");
    if (!pb->cu_seqlens_host) return fail(SNAPKV_EINVAL, "cu_seqlens_host is NULL");
    if (p.d != 64 && p.d != 128) return fail(SNAPKV_EUNSUPPORTED, "head_dim must be 64 or 128");
    p.G = p.Hq / p.Hkv;
    const int64_t M = (int64_t)p.G * p.w;
    if (M > kMaxRows) return fail(SNAPKV_EUNSUPPORTED, "G * obs_window must be <= " + std::to_string(kMaxRows));
    p.M = (int)M;
    p.M_pad = kChunkRows;
    p.n_chunks = (p.M + kChunkRows - 1) / kChunkRows;
    if (!obs_config(p.dtype, p.d, &p.cfg)) return fail(SNAPKV_EUNSUPPORTED, "no kernel for this shape");
    p.esz = p.dtype == SNAPKV_F32 ? 4 : 2;
    p.row_bytes = p.d * p.esz;
    if (p.token_stride < p.d) return fail(SNAPKV_EINVAL, "kv_token_stride must be >= head_dim");
    if (p.head_stride < 0) return fail(SNAPKV_EINVAL, "kv_head_stride must be >= 0");
    if ((p.token_stride * p.esz) % 16 || (p.head_stride * p.esz) % 16)
        return fail(SNAPKV_EINVAL, "K/V strides must keep rows 16-byte aligned");
    // a slab's keys are addressed with 32-bit offsets from the slab's first key
    if ((double)p.token_stride * p.esz * p.cfg.slab_keys() >= 2147483648.0)
        return fail(SNAPKV_EUNSUPPORTED, "kv_token_stride too large (one slab of keys must span < 2 GiB)");

    const int32_t *cu = pb->cu_seqlens_host;
    if (cu[0] != 0) return fail(SNAPKV_EINVAL, "cu_seqlens[0] must be 0");
    p.L.resize(p.B);
    p.P.resize(p.B);
    p.k.resize(p.B);
    p.cu_pfx.assign(p.B + 1, 0);
    p.cu_k.assign(p.B + 1, 0);
    p.cu_out.assign(p.B + 1, 0);
    for (int r = 0; r < p.B; ++r) {
        const int64_t L = (int64_t)cu[r + 1] - cu[r];
        if (L < p.w) return fail(SNAPKV_EINVAL, "request " + std::to_string(r) + " is shorter than obs_window");
        const int64_t P = L - p.w;
        int64_t k;
        if (p.mode == SNAPKV_RATIO) {
            k = (int64_t)floor(p.ratio * (double)P);
            if (k > P) k = P;
            if (k < 0) k = 0;
        } else {
            k = p.budget < P ? p.budget : P;
        }
        p.L[r] = L;
        p.P[r] = P;
        p.k[r] = k;
        p.cu_pfx[r + 1] = p.cu_pfx[r] + P;
        p.cu_k[r + 1] = p.cu_k[r] + k;
        p.cu_out[r + 1] = p.cu_out[r] + k + p.w;
    }
    p.sum_P = p.cu_pfx[p.B];
    p.max_P = 0;
    for (int r = 0; r < p.B; ++r) p.max_P = p.P[r] > p.max_P ? p.P[r] : p.max_P;
    p.sum_k = p.cu_k[p.B];
    p.sum_out = p.cu_out[p.B];

    // groups of at most kMaxReq requests; rows of 256 bytes take the shorter slab when its
    // slab counts pack into fewer grid iterations' worth of time (see fused_cost)
    int st = build_groups(p, cu);
    if (st) return st;
    ObsConfig alt;
    if (!(p.flags & SNAPKV_FLAG_TWO_PASS) && obs_config_short(p.dtype, p.d, &alt)) {
        const double c0 = fused_cost(p);
        const ObsConfig keep_cfg = p.cfg;
        p.cfg = alt;
        st = build_groups(p, cu);
        if (st) return st;
        if (!(fused_cost(p) < c0)) {
            p.cfg = keep_cfg;
            st = build_groups(p, cu);
            if (st) return st;
        }
    }
    for (int r = 0; r < p.B; ++r)
        if (cu[r + 1] > 0x7fffffff - 1) return fail(SNAPKV_EUNSUPPORTED, "token count exceeds int32");

    // streaming kernel: 1024-key items, halved (down to 256) while a group has fewer items than
    // the grid has workgroups
    p.st_ok = p.row_bytes == 256 && p.M <= 256 && !(p.flags & SNAPKV_FLAG_TWO_PASS);
    if ((p.flags & SNAPKV_FLAG_STREAM) && !p.st_ok)
        return fail(SNAPKV_EUNSUPPORTED, "SNAPKV_FLAG_STREAM needs rows of 256 bytes and G * obs_window <= 256");
    p.st_rows = p.M <= 32 ? 32 : p.M <= 64 ? 64 : p.M <= 128 ? 128 : 256;
    p.st_slab = 1024;
    p.st_max_items = 0;
    if (p.st_ok) {
        int64_t mx = 0;
        for (const Group &gr : p.groups) {
            const int64_t n = stream_items(p, gr, 1024, nullptr);
            mx = n > mx ? n : mx;
        }
        const int grid = p.st_rows <= 128 ? kStreamNominalGrid : kStreamNominalGrid / 2;
        while (p.st_slab > 256 && mx * 1024 / p.st_slab < grid) p.st_slab /= 2;
        for (const Group &gr : p.groups) {
            const int64_t n = stream_items(p, gr, p.st_slab, nullptr);
            if (n > (1 << 29)) return fail(SNAPKV_EUNSUPPORTED, "problem too large");
            p.st_max_items = n > p.st_max_items ? n : p.st_max_items;
        }
    }

    // workspace: [err (one 256-byte line)] [counters, one line per (segment, chunk)] [partial]
    // [merged] [votes planes, when rows come in several chunks] [votes] [pooled] [idx]
    const size_t C = (size_t)p.n_chunks;
    size_t off = 0;
    p.off_err = off;
    p.off_cnt = kWsAlign;
    off = align_up(p.off_cnt + sizeof(uint32_t) * kCounterStride * (size_t)p.max_group_segs * C);
    p.off_partial = off;
    off = align_up(off + sizeof(float) * 2 * (size_t)p.max_group_slabs * C * p.M_pad);
    p.off_merged = off;
    off = align_up(off + sizeof(float) * 2 * (size_t)p.max_group_segs * C * p.M_pad);
    p.off_planes = off;
    if (C > 1) off = align_up(off + sizeof(float) * C * (size_t)p.Hkv * (size_t)p.sum_P);
    p.off_votes = off;
    off = align_up(off + sizeof(float) * (size_t)p.Hkv * (size_t)p.sum_P);
    p.off_pooled = off;
    off = align_up(off + sizeof(float) * (size_t)p.Hkv * (size_t)p.sum_P);
    p.off_idx = off;
    off = align_up(off + sizeof(int32_t) * (size_t)p.Hkv * (size_t)p.sum_k);
    // long-segment select: per-segment state, histograms, candidates, tile counts
    const bool has_long = p.max_P > select_lds_positions();
    p.max_tiles = has_long ? (int)((p.max_P + select_tile_positions() - 1) / select_tile_positions()) : 0;
    p.off_long_state = off;
    if (has_long) off = align_up(off + sizeof(LongState) * (size_t)p.max_group_segs);
    p.off_ghist = off;
    if (has_long) off = align_up(off + sizeof(uint32_t) * 4096 * (size_t)p.max_group_segs);
    // split select (segments of up to select_lds_positions()): two counter lines and a histogram
    // of 4096 + 64 words per segment (zero between calls, like the tile select's state), then
    // per-chunk records after the candidates
    p.has_split = false;
    for (int r = 0; r < p.B; ++r) p.has_split = p.has_split || (p.P[r] > 0 && p.P[r] <= select_lds_positions());
    p.off_split_ctl = off;
    if (p.has_split) off = align_up(off + sizeof(uint32_t) * 2 * kSplitLine * (size_t)p.max_group_segs);
    p.off_split_hist = off;
    if (p.has_split) off = align_up(off + sizeof(uint32_t) * (4096 + 64) * (size_t)p.max_group_segs);
    p.off_cand = off;
    if (has_long || p.has_split) off = align_up(off + sizeof(uint32_t) * (size_t)p.Hkv * (size_t)p.sum_P);
    p.off_tilecnt = off;
    if (has_long) off = align_up(off + sizeof(uint32_t) * 4 * (size_t)p.max_tiles * (size_t)p.max_group_segs);
    p.off_split_rec = off;
    if (p.has_split) off = align_up(off + sizeof(uint32_t) * kSplitMaxChunks * (size_t)p.max_group_segs);
    // streaming scoring: ticket line, three control lines per segment, per-item row stats,
    // per-segment row shifts
    const size_t st_rows = (size_t)p.st_rows;
    p.off_st_ticket = off;
    if (p.st_ok) off = align_up(off + kWsAlign);
    p.off_st_ctl = off;
    if (p.st_ok) off = align_up(off + sizeof(uint32_t) * 3 * kStreamSegLine * (size_t)p.max_group_segs);
    p.off_st_partial = off;
    if (p.st_ok) off = align_up(off + sizeof(float) * 2 * st_rows * (size_t)p.st_max_items);
    p.off_st_final = off;
    if (p.st_ok) off = align_up(off + sizeof(float) * st_rows * (size_t)p.max_group_segs);
    // one-read scoring (32 rows): per-item row stats and per-segment row shifts, both tagged so
    // that zero means "not yet written"; every call leaves them at zero
    const bool op_ok = p.st_ok && p.st_rows == 32;
    int64_t op_max_items = 0;  // items of the largest group at the one-read kernels' smallest slab
    if (op_ok) {
        int thr = 0, slab1 = 0, slab2 = 0, slots = 0;
        (void)onepass_kernel(p.dtype, &thr, &slab1);
        (void)onepass2_kernel(p.dtype, &thr, &slab2, &slots);
        const int slab = slab1 < slab2 ? slab1 : slab2;
        for (const Group &gr : p.groups) {
            const int64_t n = stream_items(p, gr, slab, nullptr);
            op_max_items = n > op_max_items ? n : op_max_items;
        }
    }
    p.off_op_partial = off;
    if (op_ok) off = align_up(off + sizeof(uint64_t) * 32 * (size_t)op_max_items);
    p.off_op_final = off;
    if (op_ok) off = align_up(off + sizeof(float) * 32 * (size_t)p.max_group_segs);
    p.ws_bytes = off;
    return SNAPKV_OK;
}

// ---- device facts (cached per device) ----

struct DevInfo {
    bool init = false;
    int status = SNAPKV_OK;
    int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

int device_info(DevInfo *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SNAPKV_EHIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(SNAPKV_EUNSUPPORTED, "device ordinal out of range");
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DevInfo &di = g_dev[dev];
    if (!di.init) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(SNAPKV_EHIP, "hipGetDeviceProperties failed");
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            di.status = SNAPKV_EUNSUPPORTED;
        } else {
            di.cus = prop.multiProcessorCount;
        }
        di.init = true;
    }
    *out = di;
    if (di.status != SNAPKV_OK) return fail(di.status, "libsnapkv runs on gfx950 (MI355X) only");
    return SNAPKV_OK;
}

int occupancy(const void *kernel, int threads) {
    static std::mutex mu;
    static std::vector<std::pair<const void *, int>> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lk(mu);
    const void *key = (const char *)kernel + dev;  // kernels are distinct; device folded in
    for (auto &e : cache)
        if (e.first == key) return e.second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) n = 0;
    cache.emplace_back(key, n);
    return n;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int check_ws(const Plan &p, void *ws, size_t ws_bytes) {
    if (!ws) return fail(SNAPKV_EWORKSPACE, "workspace is NULL");
    if ((uintptr_t)ws % kWsAlign) return fail(SNAPKV_EWORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < p.ws_bytes)
        return fail(SNAPKV_EWORKSPACE, "workspace too small: need " + std::to_string(p.ws_bytes) + " bytes");
    return SNAPKV_OK;
}

// ---- kernel trace: caller's events recorded around each launch (per thread) ----

struct Trace {
    void *const *events = nullptr;
    int n_pairs = 0;
    int count = 0;
    int32_t ids[4096];
};
thread_local Trace g_trace;

// Every kernel goes through hipExtLaunchKernel: when a trace is open its start/stop
// events are stamped by the dispatch itself, so traced durations are the kernels' own.
int launch_traced(int id, const void *kernel, dim3 grid, dim3 block, void *arg, hipStream_t stream) {
    void *args[] = {arg};
    Trace &tr = g_trace;
    const bool rec = tr.events && tr.count < tr.n_pairs;
    hipEvent_t e0 = rec ? (hipEvent_t)tr.events[2 * tr.count] : nullptr;
    hipEvent_t e1 = rec ? (hipEvent_t)tr.events[2 * tr.count + 1] : nullptr;
    if (hipExtLaunchKernel(kernel, grid, block, args, 0, stream, e0, e1, 0) != hipSuccess)
        return fail(SNAPKV_EHIP, std::string("kernel launch failed: ") + hipGetErrorString(hipGetLastError()));
    if (tr.events) {
        if (rec && tr.count < 4096) tr.ids[tr.count] = id;
        ++tr.count;
    }
    return SNAPKV_OK;
}

int launch(int id, const void *kernel, dim3 grid, dim3 block, void *arg, hipStream_t stream) {
    return launch_traced(id, kernel, grid, block, arg, stream);
}

int run_pool(const Plan &p, const Group &gr, const float *votes, float *pooled, hipStream_t stream);

// Slot layout of a fused launch that needs several grid iterations: each (request, KV head)
// segment of z items starts at the next iteration boundary when it would cross one, so all
// of its items run in the same iteration (its barrier never waits for a later iteration).
// The device side (packed_item) inverts this layout.  Returns the number of slots.
static int64_t pack_segments(const Plan &p, const Group &gr, int grid, int32_t *vb) {
    const int slab = p.cfg.slab_keys();
    int64_t pos = 0;
    for (int i = 0; i < gr.rt.n; ++i) {
        vb[i] = (int32_t)pos;
        const int64_t z = (int64_t)((gr.rt.L[i] + slab - 1) / slab) * p.n_chunks;
        if (z == 0) continue;
        for (int g = 0; g < p.Hkv; ++g) {
            if (pos % grid + z > grid) pos += grid - pos % grid;
            pos += z;
        }
    }
    vb[gr.rt.n] = (int32_t)pos;
    return pos;
}

// Votes of every group (into `votes`); with `pool`, also the pooled votes (into `pooled`).
int run_scores(const Plan &p, const void *q, const void *K, const float *lse, float *votes, float *pooled,
               bool pool, char *ws, hipStream_t stream) {
    DevInfo di;
    int st = device_info(&di);
    if (st) return st;
    const ObsConfig &cfg = p.cfg;
    const int slab = cfg.slab_keys();
    const int C = p.n_chunks;
    const bool keep = C > 1;  // row chunks of a slab re-read it: keep it cached
    uint32_t *err = (uint32_t *)(ws + p.off_err);
    uint32_t *counters = (uint32_t *)(ws + p.off_cnt);
    float2 *partial = (float2 *)(ws + p.off_partial);
    float2 *merged = (float2 *)(ws + p.off_merged);
    float *planes = C > 1 ? (float *)(ws + p.off_planes) : votes;
    const void *kf = obs_kernel(p.dtype, p.d, cfg, kFused, keep);
    const int occ = occupancy(kf, cfg.threads());
    const int resident = occ * di.cus;
    int st_threads = 0;
    const void *ks = p.st_ok ? stream_kernel(p.dtype, p.st_rows, &st_threads) : nullptr;
    const int st_grid = p.st_ok ? occupancy(ks, st_threads) * di.cus : 0;
    int op_threads = 0, op_slab = 0;
    const void *ko = p.st_ok && p.st_rows == 32 ? onepass_kernel(p.dtype, &op_threads, &op_slab) : nullptr;
    const int op_grid = ko ? occupancy(ko, op_threads) * di.cus : 0;
    int o2_threads = 0, o2_slab = 0, o2_slots = 0;
    const void *ko2 = ko ? onepass2_kernel(p.dtype, &o2_threads, &o2_slab, &o2_slots) : nullptr;
    const int o2_grid = ko2 ? occupancy(ko2, o2_threads) * di.cus : 0;
    const bool forced = (p.flags & (SNAPKV_FLAG_TWO_PASS | SNAPKV_FLAG_STREAM | SNAPKV_FLAG_FUSED)) != 0;
    for (const Group &gr : p.groups) {
        int max_ns = 0;
        if (p.st_ok) (void)stream_items(p, gr, p.st_slab, &max_ns);
        int op_max_ns = 0;
        const int64_t op_items = ko ? stream_items(p, gr, op_slab, &op_max_ns) : 0;
        // Up to 32 rows per KV head: the one-read streaming kernel when all of the group's items
        // fit one pass of the resident grid (its segment waits then cost one tail, and they
        // need the segment's items resident at once); past that its waits grow with the
        // segment's share of the grid, and the two-phase streaming kernel, which reads K twice
        // (the second time partly from the Infinity Cache) but never waits on a slower item,
        // is faster (825 against 965 us at the 380K-token layer).  Grouped-query heads and the
        // caller's row stats: the two-phase kernel too (it reads each key once per pass for all
        // of a group's rows).  Otherwise the fused kernel, else two passes.
        int o2_max_ns = 0;
        const int64_t o2_items = ko2 ? stream_items(p, gr, o2_slab, &o2_max_ns) : 0;
        const bool use_onepass = ko && !lse && !forced && op_grid > 0 && op_items <= op_grid && op_max_ns <= op_grid;
        const int o2_launch = o2_items < o2_grid ? (int)o2_items : o2_grid;
        const bool use_onepass2 = !use_onepass && ko2 && !lse && !forced && o2_launch > 0 &&
                                  o2_max_ns <= o2_slots * o2_launch;
        const bool use_stream = !use_onepass && !use_onepass2 && p.st_ok && st_grid > 0 && !(p.flags & SNAPKV_FLAG_FUSED) &&
                                !(p.flags & SNAPKV_FLAG_TWO_PASS);
        const bool one_read = use_onepass || use_onepass2;
        if (one_read || use_stream) {
            StreamParams sp;
            memset(&sp, 0, sizeof sp);
            sp.q = q;
            sp.K = K;
            sp.votes = votes;
            sp.partial = (float2 *)(ws + (one_read ? p.off_op_partial : p.off_st_partial));
            sp.final_shift = (float *)(ws + (one_read ? p.off_op_final : p.off_st_final));
            sp.ticket = (uint32_t *)(ws + p.off_st_ticket);
            sp.seg_ctl = (uint32_t *)(ws + p.off_st_ctl);
            sp.err = err;
            sp.lse = lse;
            sp.head_stride = p.head_stride;
            sp.token_stride = p.token_stride;
            sp.sum_P = p.sum_P;
            sp.Hq = p.Hq;
            sp.Hkv = p.Hkv;
            sp.G = p.G;
            sp.w = p.w;
            sp.M = p.M;
            sp.M_pad = p.st_rows;
            sp.variant = p.variant;
            sp.c = (float)(1.4426950408889634 / sqrt((double)p.d));
            // the one-read kernel always takes its largest slab: it runs every step of an item
            // whatever the slab's length
            const int slab_keys = use_onepass ? op_slab : use_onepass2 ? o2_slab : p.st_slab;
            sp.slab_keys = slab_keys;
            sp.spin_limit = kSpinLimit;
            sp.rt = gr.rt;
            int64_t n = 0;
            for (int i = 0; i < gr.rt.n; ++i) {
                sp.rt.slab0[i] = (int32_t)n;
                n += (int64_t)((gr.rt.L[i] + slab_keys - 1) / slab_keys) * p.Hkv;
            }
            sp.rt.slab0[gr.rt.n] = (int32_t)n;
            sp.n_items = (int32_t)n;
            if (one_read && (size_t)n * 32 * sizeof(uint64_t) > p.off_op_final - p.off_op_partial)
                return fail(SNAPKV_EUNSUPPORTED, "one-read stats region smaller than the launch's items");
            if (use_onepass) {
                const int grid = n < op_grid ? (int)n : op_grid;
                st = launch(SNAPKV_K_OBS_ONEPASS, ko, dim3(grid), dim3(op_threads), &sp, stream);
            } else if (use_onepass2) {
                st = launch(SNAPKV_K_OBS_ONEPASS2, ko2, dim3(o2_launch), dim3(o2_threads), &sp, stream);
            } else {
                // Votes items trail the stats items of their segment by about one pass of the grid:
                // close enough that part of the second read still comes from the Infinity Cache,
                // far enough that a votes item rarely waits.
                const int64_t lag = (int64_t)max_ns + st_grid;
                sp.lag = (int32_t)(lag < n ? lag : n);
                const int64_t tickets = lse ? n : 2 * n;
                const int grid = tickets < st_grid ? (int)tickets : st_grid;
                st = launch(SNAPKV_K_OBS_STREAM, ks, dim3(grid), dim3(st_threads), &sp, stream);
            }
            if (st) return st;
            if (gr.max_P > 0 && pool) {
                st = run_pool(p, gr, votes, pooled, stream);
                if (st) return st;
            }
            continue;
        }
        ObsParams op;
        memset(&op, 0, sizeof op);
        op.q = q;
        op.K = K;
        op.votes = planes;
        op.partial = partial;
        op.merged = merged;
        op.counters = counters;
        op.err = err;
        op.head_stride = p.head_stride;
        op.token_stride = p.token_stride;
        op.sum_P = p.sum_P;
        op.Hq = p.Hq;
        op.Hkv = p.Hkv;
        op.G = p.G;
        op.w = p.w;
        op.M = p.M;
        op.M_pad = p.M_pad;
        op.variant = p.variant;
        op.c = (float)(1.4426950408889634 / sqrt((double)p.d));
        op.n_slabs = gr.n_slabs;
        op.slab_keys = slab;
        op.spin_limit = kSpinLimit;
        op.n_chunks = C;
        op.vplane = (int64_t)p.Hkv * p.sum_P;
        op.lse = lse;
        op.lse_scale = (float)sqrt((double)p.d);
        op.rt = gr.rt;
        const int64_t items = (int64_t)gr.n_slabs * C;
        // The fused kernel's grid never exceeds what the device keeps resident, and no
        // segment has more work items than that grid; with more items than the grid, the
        // packed layout keeps each segment inside one iteration, so every segment barrier
        // completes within its iteration.
        // A packing that leaves more than a fifth of the slots idle loses to the two-pass path
        // (which reads K twice but keeps every workgroup busy).
        bool fused = !(p.flags & SNAPKV_FLAG_TWO_PASS) && resident > 0 && (int64_t)gr.max_ns * C <= resident;
        const int grid = items < resident ? (int)items : resident;
        if (!lse && fused && items > resident) {
            op.pack_grid = resident;
            const int64_t slots = pack_segments(p, gr, resident, op.vb);
            if (slots > 0x7fffffff) return fail(SNAPKV_EUNSUPPORTED, "problem too large");
            const int64_t iters = (slots + resident - 1) / resident;
            if (iters * resident * 4 > items * 5) {
                fused = false;
                op.pack_grid = 0;
            }
        }
        const int n_seg = gr.rt.n * p.Hkv;
        if (lse) {
            // the caller's row stats: one read of K, no barrier
            st = launch(SNAPKV_K_OBS_VOTES, obs_kernel(p.dtype, p.d, cfg, kVotes, keep), dim3((unsigned)items),
                        dim3(cfg.threads()), &op, stream);
            if (st) return st;
        } else if (fused) {
            st = launch(SNAPKV_K_OBS_FUSED, kf, dim3(grid), dim3(cfg.threads()), &op, stream);
            if (st) return st;
        } else {
            st = launch(SNAPKV_K_OBS_STATS, obs_kernel(p.dtype, p.d, cfg, kStats, keep), dim3((unsigned)items),
                        dim3(cfg.threads()), &op, stream);
            if (st) return st;
            MergeParams mp;
            memset(&mp, 0, sizeof mp);
            mp.partial = partial;
            mp.merged = merged;
            mp.M = p.M;
            mp.M_pad = p.M_pad;
            mp.slab_keys = slab;
            mp.Hkv = p.Hkv;
            mp.n_chunks = C;
            mp.c = op.c;
            mp.rt = gr.rt;
            st = launch(SNAPKV_K_STATS_MERGE, merge_kernel(), dim3(n_seg * C, (p.M_pad + 3) / 4), dim3(256), &mp,
                        stream);
            if (st) return st;
            st = launch(SNAPKV_K_OBS_VOTES, obs_kernel(p.dtype, p.d, cfg, kVotes, keep), dim3((unsigned)items),
                        dim3(cfg.threads()), &op, stream);
            if (st) return st;
        }
        if (C > 1 && gr.max_P > 0) {
            SumParams sp;
            memset(&sp, 0, sizeof sp);
            sp.planes = planes;
            sp.votes = votes;
            sp.sum_P = p.sum_P;
            sp.vplane = op.vplane;
            sp.col0 = gr.rt.pfx0[0];
            sp.col1 = gr.rt.pfx0[gr.rt.n - 1] + (gr.rt.L[gr.rt.n - 1] - p.w);
            sp.n_chunks = C;
            st = launch(SNAPKV_K_SUM_CHUNKS, sum_kernel(), dim3((unsigned)((sp.col1 - sp.col0 + 255) / 256), p.Hkv),
                        dim3(256), &sp, stream);
            if (st) return st;
        }
        if (gr.max_P > 0 && pool) {
            st = run_pool(p, gr, votes, pooled, stream);
            if (st) return st;
        }
    }
    return SNAPKV_OK;
}

// Whether the select kernel pools the votes itself: every segment of the group fits its
// resident path and the pool window is narrow enough.
bool select_pools(const Plan &p, int max_P) {
    return max_P <= select_lds_positions() && p.K_pool / 2 <= select_max_half(max_P);
}

// Pooled votes of one group: in the select kernel when it can pool (see select_pools),
// else with the pooling kernel.
int run_pool(const Plan &p, const Group &gr, const float *votes, float *pooled, hipStream_t stream) {
    {
        if (select_pools(p, gr.max_P)) {
            SelectParams sp;
            memset(&sp, 0, sizeof sp);
            sp.votes = votes;
            sp.pooled_out = pooled;
            sp.sum_P = p.sum_P;
            sp.sum_k = p.sum_k;
            sp.w = p.w;
            sp.Hkv = p.Hkv;
            sp.half = p.K_pool / 2;
            sp.rt = gr.rt;
            return launch(SNAPKV_K_POOL, select_kernel(), dim3(gr.rt.n * p.Hkv), dim3(select_threads()), &sp, stream);
        }
        {
            PoolParams pp;
            memset(&pp, 0, sizeof pp);
            pp.votes = votes;
            pp.pooled = pooled;
            pp.sum_P = p.sum_P;
            pp.w = p.w;
            pp.half = p.K_pool / 2;
            pp.rt = gr.rt;
            return launch(SNAPKV_K_POOL, pool_kernel(), dim3((gr.max_P + 255) / 256, gr.rt.n, p.Hkv), dim3(256), &pp,
                          stream);
        }
    }
}

// Whether the select kernels pool the votes themselves: the pool window fits every kernel
// the group uses (the resident kernel for segments of up to select_lds_positions(), the
// tile kernel beyond).
bool select_fuses_pool(const Plan &p, int max_P) {
    const int m = max_P < select_lds_positions() ? max_P : select_lds_positions();
    return p.K_pool / 2 <= select_max_half(m);
}

// Top-k of every group.  With `votes` the select kernels pool first when the window allows
// (pooled votes also written to `pooled` if it is not null), else the pooling kernel writes
// `pooled`.  Segments longer than select_lds_positions() need `pooled` (the tile kernel
// passes the pooled votes between its phases) and the workspace.
int run_select(const Plan &p, const float *votes, float *pooled, int32_t *idx, char *ws, hipStream_t stream) {
    for (const Group &gr : p.groups) {
        const bool fuse = votes && select_fuses_pool(p, gr.max_P);
        if (votes && !fuse) {
            int st = run_pool(p, gr, votes, pooled, stream);
            if (st) return st;
        }
        const bool any_k = p.cu_k[gr.rt.qi[gr.rt.n - 1] + 1] != p.cu_k[gr.rt.qi[0]];
        bool any_resident = false;  // a segment the resident kernel takes (the others return at once)
        for (int i = 0; i < gr.rt.n; ++i) any_resident = any_resident || gr.rt.L[i] - p.w <= select_lds_positions();
        // Segments of up to select_lds_positions() go to the split kernel (workgroups of
        // split_chunk() positions that wait for each other) when the group has one longer than
        // 16 positions per thread of the single-workgroup kernel (its slowest runs: 20 against
        // 10 us for 32K against 16K positions, where the split's two round trips pay) and the
        // device holds the whole grid; else to one workgroup per segment.
        SplitParams xp;
        memset(&xp, 0, sizeof xp);
        int64_t split_grid = 0;
        for (int i = 0; i < gr.rt.n; ++i) {
            xp.wg0[i] = (int32_t)split_grid;
            const int64_t P = gr.rt.L[i] - p.w;
            if (P > 0 && P <= select_lds_positions()) split_grid += (int64_t)p.Hkv * ((P + split_chunk() - 1) / split_chunk());
        }
        xp.wg0[gr.rt.n] = (int32_t)split_grid;
        bool use_split = false;
        int split_thr = 0;
        if (any_resident && (any_k || (fuse && pooled)) && p.has_split && split_grid > 0 &&
            gr.max_P > 16 * select_threads() && !(p.flags & SNAPKV_FLAG_SELECT_ONE_WG) &&
            (!fuse || p.K_pool / 2 <= split_max_half())) {
            DevInfo di;
            int st = device_info(&di);
            if (st) return st;
            // 1024 threads per workgroup where the grid is resident at one per CU, else 512
            // threads (more of them stay resident)
            for (int t : {1024, 512}) {
                if (split_grid <= (int64_t)occupancy(split_kernel(t), t) * di.cus) {
                    split_thr = t;
                    break;
                }
            }
            use_split = split_thr > 0;
        }
        if (use_split) {
            xp.votes = fuse ? votes : nullptr;
            xp.pooled = pooled;
            xp.pooled_out = fuse ? pooled : nullptr;
            xp.idx = idx;
            xp.ctl = (uint32_t *)(ws + p.off_split_ctl);
            xp.ghist = (uint32_t *)(ws + p.off_split_hist);
            xp.cand = (uint32_t *)(ws + p.off_cand);
            xp.rec = (uint32_t *)(ws + p.off_split_rec);
            xp.err = (uint32_t *)(ws + p.off_err);
            xp.sum_P = p.sum_P;
            xp.sum_k = p.sum_k;
            xp.w = p.w;
            xp.Hkv = p.Hkv;
            xp.half = p.K_pool / 2;
            xp.spin_limit = kSpinLimit;
            xp.rt = gr.rt;
            int st = launch(SNAPKV_K_SELECT_SPLIT, split_kernel(split_thr), dim3((unsigned)split_grid), dim3(split_thr), &xp,
                            stream);
            if (st) return st;
        } else if (any_resident && (any_k || (fuse && pooled))) {
            SelectParams sp;
            memset(&sp, 0, sizeof sp);
            sp.votes = fuse ? votes : nullptr;
            sp.pooled = pooled;
            sp.pooled_out = fuse ? pooled : nullptr;
            sp.idx = idx;
            sp.sum_P = p.sum_P;
            sp.sum_k = p.sum_k;
            sp.w = p.w;
            sp.Hkv = p.Hkv;
            sp.half = p.K_pool / 2;
            sp.rt = gr.rt;
            int st = launch(SNAPKV_K_SELECT, select_kernel(), dim3(gr.rt.n * p.Hkv), dim3(select_threads()), &sp,
                            stream);
            if (st) return st;
        }
        if (gr.max_P > select_lds_positions()) {
            LongParams lp;
            memset(&lp, 0, sizeof lp);
            lp.votes = fuse ? votes : nullptr;
            lp.pooled = pooled;
            lp.idx = idx;
            lp.state = (LongState *)(ws + p.off_long_state);
            lp.ghist = (uint32_t *)(ws + p.off_ghist);
            lp.cand = (uint32_t *)(ws + p.off_cand);
            lp.tilecnt = (uint32_t *)(ws + p.off_tilecnt);
            lp.sum_P = p.sum_P;
            lp.sum_k = p.sum_k;
            lp.w = p.w;
            lp.Hkv = p.Hkv;
            lp.half = p.K_pool / 2;
            lp.max_tiles = p.max_tiles;
            lp.rt = gr.rt;
            const int tiles = (gr.max_P + select_tile_positions() - 1) / select_tile_positions();
            for (int phase : {0, 1, 3}) {  // phase 1's last tile records what a phase 2 would
                lp.phase = phase;
                int st = launch(SNAPKV_K_SELECT_TILES, long_kernel(), dim3(tiles, gr.rt.n * p.Hkv),
                                dim3(long_threads()), &lp, stream);
                if (st) return st;
            }
        }
    }
    return SNAPKV_OK;
}

// err_word (optional): the call's workspace error word, which the last gather launch copies
// to err_out (optional) and clears.
int run_gather(const Plan &p, const void *K, const void *V, const int32_t *idx, void *K_out, void *V_out,
               hipStream_t stream, uint32_t *err_word = nullptr, uint32_t *err_out = nullptr) {
    for (size_t gi = 0; gi < p.groups.size(); ++gi) {
        const Group &gr = p.groups[gi];
        GatherParams gp;
        memset(&gp, 0, sizeof gp);
        gp.K = K;
        gp.V = V;
        gp.idx = idx;
        gp.K_out = K_out;
        gp.V_out = V_out;
        gp.head_stride = p.head_stride;
        gp.token_stride = p.token_stride;
        gp.sum_k = p.sum_k;
        gp.sum_out = p.sum_out;
        gp.row_bytes = p.row_bytes;
        gp.esz = p.esz;
        gp.w = p.w;
        gp.Hkv = p.Hkv;
        if (gi + 1 == p.groups.size()) {
            gp.err_word = err_word;
            gp.err_out = err_out;
        }
        gp.rt = gr.rt;
        const int tile = 256 / (p.row_bytes / 16) * gather_rows_per_thread();
        int64_t blocks = (gr.out_rows + tile - 1) / tile;
        if (blocks > 65535) blocks = 65535;
        if (blocks < 1) blocks = 1;
        int st = launch(SNAPKV_K_GATHER, gather_kernel(), dim3((unsigned)blocks, p.Hkv), dim3(256), &gp, stream);
        if (st) return st;
    }
    return SNAPKV_OK;
}

// ---- the allocation-free call's workspace: one array per device --------------------------
// A file-scope device array stands in for the caller's workspace.  Its name is a host-side
// stand-in in host code, so every host use goes through the address hipGetSymbolAddress
// returns for the current device (each device holds its own copy).
static __device__ __align__(256) unsigned char scratch[SNAPKV_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
char *g_scratch_ptr[64];

// The current device's scratch address.  The first call on a device looks it up and zero-fills
// the array on `stream` (every later call finds its barrier counters back at zero, as a
// zero-filled workspace requires).
int scratch_for_device(hipStream_t stream, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SNAPKV_EHIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(SNAPKV_EUNSUPPORTED, "device ordinal out of range");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(SNAPKV_EHIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
        ClearParams cp;
        cp.data = (uint32_t *)ptr;
        cp.n = (int32_t)(SNAPKV_NOALLOC_SCRATCH_BYTES / sizeof(uint32_t));
        const int st = launch(SNAPKV_K_SCRATCH_CLEAR, hit_clear(), dim3((unsigned)((cp.n + 255) / 256)), dim3(256), &cp,
                              stream);
        if (st) return st;
        g_scratch_ptr[dev] = (char *)ptr;
    }
    *out = g_scratch_ptr[dev];
    return SNAPKV_OK;
}

// ---- control regions of a workspace --------------------------------------------------------
// The ranges a call expects to find at zero: the fused kernel's arrival lines, the tile select's
// per-segment state and histograms, the streaming kernels' ticket and control lines, and the
// one-read kernels' tagged row stats and shifts.  Every call leaves them at zero again.  Their
// offsets depend on the problem, so a call whose ranges differ from those of the previous call
// on the same workspace (another shape reusing it) may find there the data the previous call
// wrote (votes, indices, ...): such a call clears its ranges first, with one small kernel.
struct CtlRange {
    size_t off, bytes;
};
static int control_ranges(const Plan &p, CtlRange *r) {
    int n = 0;
    auto add = [&](size_t a, size_t b) {
        if (b > a) r[n++] = CtlRange{a, b - a};
    };
    add(p.off_cnt, p.off_partial);         // arrival lines
    add(p.off_long_state, p.off_cand);     // tile and split selects: state, counters, histograms
    add(p.off_st_ticket, p.off_st_partial);  // ticket line, control lines
    add(p.off_op_partial, p.ws_bytes);     // tagged stats and shifts
    return n;
}

std::mutex g_ws_mu;
std::unordered_map<uint64_t, uint64_t> g_ws_layout;  // (device, workspace address) -> ranges' hash

int prepare_ws(const Plan &p, char *ws, hipStream_t stream) {
    CtlRange r[kMaxClearRanges];
    const int n = control_ranges(p, r);
    uint64_t h = 1469598103934665603ull;  // FNV-1a over the ranges
    auto mix = [&](uint64_t v) {
        for (int b = 0; b < 8; ++b) h = (h ^ ((v >> (8 * b)) & 0xFF)) * 1099511628211ull;
    };
    for (int i = 0; i < n; ++i) {
        mix(r[i].off);
        mix(r[i].bytes);
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SNAPKV_EHIP, "hipGetDevice failed");
    const uint64_t key = (uint64_t)(uintptr_t)ws ^ ((uint64_t)dev << 56);
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws_layout.find(key);
    if (it != g_ws_layout.end() && it->second == h) return SNAPKV_OK;
    if (n > 0) {
        WsClearParams cp;
        memset(&cp, 0, sizeof cp);
        cp.base = (unsigned char *)ws;
        int64_t most = 0;
        for (int i = 0; i < n; ++i) {
            cp.off[i] = (int64_t)r[i].off;
            cp.n16[i] = (int64_t)(r[i].bytes / 16);
            most = cp.n16[i] > most ? cp.n16[i] : most;
        }
        cp.n_ranges = n;
        int64_t blocks = (most + 255) / 256;
        blocks = blocks > 1024 ? 1024 : (blocks < 1 ? 1 : blocks);
        const int st = launch(SNAPKV_K_WS_CLEAR, ws_clear(), dim3((unsigned)blocks), dim3(256), &cp, stream);
        if (st) return st;
    }
    g_ws_layout[key] = h;
    return SNAPKV_OK;
}

int check_ptr(const void *ptr, const char *name) {
    if (!ptr) return fail(SNAPKV_EINVAL, std::string(name) + " is NULL");
    if (!aligned16(ptr)) return fail(SNAPKV_EINVAL, std::string(name) + " must be 16-byte aligned");
    return SNAPKV_OK;
}

int check_opt_ptr(const void *ptr, const char *name) { return ptr ? check_ptr(ptr, name) : SNAPKV_OK; }

int finish(int st) {
    if (st) return st;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SNAPKV_EHIP, std::string("HIP error: ") + hipGetErrorString(e));
    return SNAPKV_OK;
}

}  // namespace

extern "C" {

int snapkv_plan(const snapkv_problem *pb, int64_t *k_host, int64_t *cu_pfx_host, int64_t *cu_k_host,
                int64_t *cu_out_host, size_t *ws_bytes) {
    Plan p;
    int st = make_plan(pb, &p);
    if (st) return st;
    for (int r = 0; r < p.B; ++r)
        if (k_host) k_host[r] = p.k[r];
    for (int r = 0; r <= p.B; ++r) {
        if (cu_pfx_host) cu_pfx_host[r] = p.cu_pfx[r];
        if (cu_k_host) cu_k_host[r] = p.cu_k[r];
        if (cu_out_host) cu_out_host[r] = p.cu_out[r];
    }
    if (ws_bytes) *ws_bytes = p.ws_bytes;
    return SNAPKV_OK;
}

static int scores_impl(const snapkv_problem *pb, const void *q_obs, const void *K, const float *lse, bool need_lse,
                       float *votes, float *pooled, void *ws, size_t ws_bytes, void *stream) {
    Plan p;
    int st = make_plan(pb, &p);
    if (!st) st = check_ptr(q_obs, "q_obs");
    if (!st) st = check_ptr(K, "K");
    if (!st && need_lse) st = check_ptr(lse, "lse");
    if (!st) st = check_opt_ptr(votes, "votes");
    if (!st) st = check_ptr(pooled, "pooled");
    if (!st) st = check_ws(p, ws, ws_bytes);
    if (!st) st = prepare_ws(p, (char *)ws, (hipStream_t)stream);
    if (st) return st;
    char *w = (char *)ws;
    float *v = votes ? votes : (float *)(w + p.off_votes);
    return finish(run_scores(p, q_obs, K, lse, v, pooled, true, w, (hipStream_t)stream));
}

int snapkv_scores(const snapkv_problem *pb, const void *q_obs, const void *K, float *votes, float *pooled,
                  void *ws, size_t ws_bytes, void *stream) {
    return scores_impl(pb, q_obs, K, nullptr, false, votes, pooled, ws, ws_bytes, stream);
}

int snapkv_scores_lse(const snapkv_problem *pb, const void *q_obs, const void *K, const float *lse, float *votes,
                      float *pooled, void *ws, size_t ws_bytes, void *stream) {
    return scores_impl(pb, q_obs, K, lse, true, votes, pooled, ws, ws_bytes, stream);
}

int snapkv_select(const snapkv_problem *pb, const float *pooled, int32_t *idx, void *ws, size_t ws_bytes,
                  void *stream) {
    Plan p;
    int st = make_plan(pb, &p);
    if (!st) st = check_ptr(pooled, "pooled");
    if (!st) st = check_ptr(idx, "idx");
    if (!st) st = check_ws(p, ws, ws_bytes);
    if (!st) st = prepare_ws(p, (char *)ws, (hipStream_t)stream);
    if (st) return st;
    DevInfo di;
    st = device_info(&di);
    if (st) return st;
    return finish(run_select(p, nullptr, (float *)pooled, idx, (char *)ws, (hipStream_t)stream));
}

int snapkv_gather(const snapkv_problem *pb, const void *K, const void *V, const int32_t *idx, void *K_out,
                  void *V_out, void *stream) {
    Plan p;
    int st = make_plan(pb, &p);
    if (!st) st = check_ptr(K, "K");
    if (!st) st = check_ptr(V, "V");
    if (!st) st = check_ptr(idx, "idx");
    if (!st) st = check_ptr(K_out, "K_out");
    if (!st) st = check_ptr(V_out, "V_out");
    if (st) return st;
    DevInfo di;
    st = device_info(&di);
    if (st) return st;
    return finish(run_gather(p, K, V, idx, K_out, V_out, (hipStream_t)stream));
}

// ws == nullptr: the allocation-free call, whose workspace is the device's scratch array.
static int compress_impl(const snapkv_problem *pb, const void *q_obs, const void *K, const void *V, const float *lse,
                         bool need_lse, void *K_out, void *V_out, int32_t *idx, float *pooled, void *ws,
                         size_t ws_bytes, void *stream, bool noalloc = false, uint32_t *err_out = nullptr) {
    Plan p;
    int st = make_plan(pb, &p);
    if (!st) st = check_ptr(q_obs, "q_obs");
    if (!st) st = check_ptr(K, "K");
    if (!st) st = check_ptr(V, "V");
    if (!st && need_lse) st = check_ptr(lse, "lse");
    if (!st) st = check_ptr(K_out, "K_out");
    if (!st) st = check_ptr(V_out, "V_out");
    if (!st) st = check_opt_ptr(idx, "idx");
    if (!st) st = check_opt_ptr(pooled, "pooled");
    if (!st && noalloc && err_out && ((uintptr_t)err_out & 3u)) st = fail(SNAPKV_EINVAL, "error_word must be 4-byte aligned");
    if (!st && noalloc && p.ws_bytes > SNAPKV_NOALLOC_SCRATCH_BYTES)
        st = fail(SNAPKV_EWORKSPACE, "problem needs " + std::to_string(p.ws_bytes) + " bytes of scratch; the "
                  "allocation-free call holds " + std::to_string((size_t)SNAPKV_NOALLOC_SCRATCH_BYTES));
    if (!st && !noalloc) st = check_ws(p, ws, ws_bytes);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (noalloc) {
        st = scratch_for_device(s, &ws);
        if (st) return st;
    }
    st = prepare_ws(p, (char *)ws, s);
    if (st) return st;
    char *w = (char *)ws;
    float *votes = (float *)(w + p.off_votes);
    // pooled votes: the caller's buffer, or workspace when long segments need them in memory
    const bool need_pooled = p.max_P > select_lds_positions() || !select_fuses_pool(p, p.max_P);
    float *pl = pooled ? pooled : (need_pooled ? (float *)(w + p.off_pooled) : nullptr);
    int32_t *ix = idx ? idx : (int32_t *)(w + p.off_idx);
    st = run_scores(p, q_obs, K, lse, votes, nullptr, false, w, s);
    if (!st) st = run_select(p, votes, pl, ix, w, s);
    if (!st) st = run_gather(p, K, V, ix, K_out, V_out, s, noalloc ? (uint32_t *)(w + p.off_err) : nullptr, err_out);
    return finish(st);
}

int snapkv_compress(const snapkv_problem *pb, const void *q_obs, const void *K, const void *V, void *K_out,
                    void *V_out, int32_t *idx, float *pooled, void *ws, size_t ws_bytes, void *stream) {
    return compress_impl(pb, q_obs, K, V, nullptr, false, K_out, V_out, idx, pooled, ws, ws_bytes, stream);
}

int snapkv_compress_lse(const snapkv_problem *pb, const void *q_obs, const void *K, const void *V, const float *lse,
                        void *K_out, void *V_out, int32_t *idx, float *pooled, void *ws, size_t ws_bytes,
                        void *stream) {
    return compress_impl(pb, q_obs, K, V, lse, true, K_out, V_out, idx, pooled, ws, ws_bytes, stream);
}

int snapkv_compress_noalloc(const snapkv_problem *pb, const void *q_obs, const void *K, const void *V, void *K_out,
                            void *V_out, int32_t *idx, float *pooled, uint32_t *error_word, void *stream) {
    return compress_impl(pb, q_obs, K, V, nullptr, false, K_out, V_out, idx, pooled, nullptr, 0, stream, true,
                         error_word);
}

int snapkv_hit_rate(const snapkv_problem *pb, const float *a_cur, const int32_t *idx, double theta, uint32_t *counts,
                    void *stream) {
    Plan p;
    int st = make_plan(pb, &p);
    if (!st) st = check_ptr(a_cur, "a_cur");
    if (!st) st = check_ptr(idx, "idx");
    if (!st) st = check_ptr(counts, "counts");
    if (!st && !(theta == theta)) st = fail(SNAPKV_EINVAL, "theta is NaN");
    if (st) return st;
    DevInfo di;
    st = device_info(&di);
    if (st) return st;
    // the tiles of a segment longer than one tile add their counts, so they start from zero
    // (a segment of one tile stores them)
    if (p.max_P > hit_tile_positions()) {
        ClearParams cp;
        cp.data = counts;
        cp.n = p.B * p.Hkv * 2;
        st = launch(SNAPKV_K_HIT_CLEAR, hit_clear(), dim3((unsigned)((cp.n + 255) / 256)), dim3(256), &cp,
                    (hipStream_t)stream);
        if (st) return finish(st);
    }
    for (const Group &gr : p.groups) {
        HitParams hp;
        memset(&hp, 0, sizeof hp);
        hp.a_cur = a_cur;
        hp.idx = idx;
        hp.counts = counts;
        hp.theta = theta;
        hp.sum_P = p.sum_P;
        hp.sum_k = p.sum_k;
        hp.w = p.w;
        hp.Hkv = p.Hkv;
        hp.rt = gr.rt;
        // at least one tile: the first tile of an empty prefix writes its zero counts
        const unsigned tiles =
            gr.max_P > 0 ? (unsigned)((gr.max_P + hit_tile_positions() - 1) / hit_tile_positions()) : 1u;
        st = launch(SNAPKV_K_HIT_RATE, hit_kernel(), dim3(tiles, gr.rt.n * p.Hkv), dim3(select_threads()), &hp,
                    (hipStream_t)stream);
        if (st) return finish(st);
    }
    return finish(SNAPKV_OK);
}

// ---- decode attention ----

// Cached rows per decode workgroup (split-K): at least 256, more when the longest request
// would otherwise give over ~1024 workgroups, in multiples of the rows one pass covers.
constexpr int kDecSplitMin = 256;

struct DecodePlan {
    int B, Hq, Hkv, G, d, dtype, head_tile, n_hchunks, max_splits, split_rows;
    int64_t head_stride, token_stride;
    std::vector<ReqTable> groups;
    size_t ws_bytes;
};

static int make_decode_plan(const snapkv_decode_problem *dp, DecodePlan *pl) {
    g_last_error.clear();
    if (!dp) return fail(SNAPKV_EINVAL, "problem is NULL");
    DecodePlan &p = *pl;
    p.B = dp->batch;
    p.Hq = dp->num_q_heads;
    p.Hkv = dp->num_kv_heads;
    p.d = dp->head_dim;
    p.dtype = dp->dtype;
    p.head_stride = dp->kv_head_stride;
    p.token_stride = dp->kv_token_stride;
    if (p.B < 1) return fail(SNAPKV_EINVAL, "batch must be >= 1");
    if (p.Hq < 1 || p.Hkv < 1 || p.Hq % p.Hkv) return fail(SNAPKV_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
    if (p.dtype != SNAPKV_F32 && p.dtype != SNAPKV_BF16) return fail(SNAPKV_EINVAL, "dtype must be F32 or BF16");
    if (p.d < 1) return fail(SNAPKV_EINVAL, "head_dim must be >= 1");
    const int esz = p.dtype == SNAPKV_F32 ? 4 : 2;
    if (p.d * esz != 256) return fail(SNAPKV_EUNSUPPORTED, "decode supports rows of 256 bytes (bf16 d=128, fp32 d=64)");
    if (p.token_stride < p.d || p.head_stride < 0) return fail(SNAPKV_EINVAL, "kv strides must be >= head_dim and >= 0");
    if ((p.token_stride * esz) % 16 || (p.head_stride * esz) % 16)
        return fail(SNAPKV_EINVAL, "kv strides must keep rows 16-byte aligned");
    if (!dp->cu_rows_host) return fail(SNAPKV_EINVAL, "cu_rows_host is NULL");
    const int64_t *cu = dp->cu_rows_host;
    if (cu[0] < 0) return fail(SNAPKV_EINVAL, "cu_rows_host[0] must be >= 0");
    int64_t max_rows = 0;
    for (int r = 0; r < p.B; ++r) {
        const int64_t n = cu[r + 1] - cu[r];
        if (n < 0) return fail(SNAPKV_EINVAL, "cu_rows_host must be non-decreasing");
        if (n > 0x3fffffff) return fail(SNAPKV_EUNSUPPORTED, "too many rows in one request");
        if (n > max_rows) max_rows = n;
    }
    p.G = p.Hq / p.Hkv;
    p.head_tile = p.G >= 8 ? 8 : (p.G >= 4 ? (p.G == 4 ? 4 : 8) : (p.G == 1 ? 1 : (p.G == 2 ? 2 : 4)));
    p.n_hchunks = (p.G + p.head_tile - 1) / p.head_tile;
    const int items = (p.B < kMaxReq ? p.B : kMaxReq) * p.Hkv * p.n_hchunks;
    const int rpi = decode_rows_per_iter();
    int64_t split = (max_rows * items + 1023) / 1024;
    split = (split + rpi - 1) / rpi * rpi;
    if (split < kDecSplitMin) split = kDecSplitMin;
    if ((max_rows + split - 1) / split > decode_max_splits())
        split = (max_rows + decode_max_splits() - 1) / decode_max_splits();
    p.split_rows = (int)((split + rpi - 1) / rpi * rpi);
    p.max_splits = (int)((max_rows + p.split_rows - 1) / p.split_rows);
    if (p.max_splits < 1) p.max_splits = 1;
    p.groups.clear();
    for (int r0 = 0; r0 < p.B; r0 += kMaxReq) {
        ReqTable rt;
        memset(&rt, 0, sizeof rt);
        rt.n = p.B - r0 < kMaxReq ? p.B - r0 : kMaxReq;
        for (int i = 0; i < rt.n; ++i) {
            rt.L[i] = (int32_t)(cu[r0 + i + 1] - cu[r0 + i]);
            rt.tok0[i] = cu[r0 + i];
            rt.qi[i] = r0 + i;
        }
        p.groups.push_back(rt);
    }
    p.ws_bytes = align_up(sizeof(float) * (size_t)items * p.max_splits * p.head_tile * (p.d + 2));
    return SNAPKV_OK;
}

int snapkv_decode_plan(const snapkv_decode_problem *dp, size_t *ws_bytes) {
    DecodePlan p;
    const int st = make_decode_plan(dp, &p);
    if (!st && ws_bytes) *ws_bytes = p.ws_bytes;
    return st;
}

int snapkv_decode(const snapkv_decode_problem *dp, const void *q, const void *K, const void *V, float *out, void *ws,
                  size_t ws_bytes, void *stream) {
    DecodePlan p;
    int st = make_decode_plan(dp, &p);
    if (!st) st = check_ptr(q, "q");
    if (!st) st = check_ptr(K, "K");
    if (!st) st = check_ptr(V, "V");
    if (!st) st = check_ptr(out, "out");
    if (!st && (!ws || (uintptr_t)ws % kWsAlign)) st = fail(SNAPKV_EWORKSPACE, "workspace missing or not 256-byte aligned");
    if (!st && ws_bytes < p.ws_bytes) st = fail(SNAPKV_EWORKSPACE, "workspace too small: need " + std::to_string(p.ws_bytes) + " bytes");
    if (st) return st;
    DevInfo di;
    st = device_info(&di);
    if (st) return st;
    for (const ReqTable &rt : p.groups) {
        DecodeParams dpar;
        memset(&dpar, 0, sizeof dpar);
        dpar.q = q;
        dpar.K = K;
        dpar.V = V;
        dpar.part = (float *)ws;
        dpar.out = out;
        dpar.head_stride = p.head_stride;
        dpar.token_stride = p.token_stride;
        dpar.Hq = p.Hq;
        dpar.Hkv = p.Hkv;
        dpar.G = p.G;
        dpar.d = p.d;
        dpar.n_hchunks = p.n_hchunks;
        dpar.head_tile = p.head_tile;
        dpar.max_splits = p.max_splits;
        dpar.split_rows = p.split_rows;
        dpar.c = (float)(1.4426950408889634 / sqrt((double)p.d));
        dpar.rt = rt;
        st = launch(SNAPKV_K_DECODE, decode_partial_kernel_for(p.dtype, p.head_tile),
                    dim3(p.max_splits, rt.n * p.Hkv * p.n_hchunks), dim3(decode_threads()), &dpar, (hipStream_t)stream);
        if (!st)
            st = launch(SNAPKV_K_DECODE_COMBINE, decode_combine_kernel_ptr(), dim3(rt.n * p.Hq), dim3(128), &dpar,
                        (hipStream_t)stream);
        if (st) return finish(st);
    }
    return finish(SNAPKV_OK);
}

int snapkv_trace_begin(void *const *events, int n_pairs) {
    g_last_error.clear();
    if (!events || n_pairs < 1) return fail(SNAPKV_EINVAL, "trace needs events and n_pairs >= 1");
    g_trace.events = events;
    g_trace.n_pairs = n_pairs;
    g_trace.count = 0;
    return SNAPKV_OK;
}

int snapkv_trace_end(int32_t *kernel_ids, int capacity) {
    const int n = g_trace.count < g_trace.n_pairs ? g_trace.count : g_trace.n_pairs;
    for (int i = 0; kernel_ids && i < n && i < capacity && i < 4096; ++i) kernel_ids[i] = g_trace.ids[i];
    const int count = g_trace.count;
    g_trace.events = nullptr;
    g_trace.n_pairs = 0;
    g_trace.count = 0;
    return count;
}

const char *snapkv_kernel_name(int id) {
    switch (id) {
        case SNAPKV_K_RESERVED0: return "reserved";
        case SNAPKV_K_OBS_FUSED: return "obs_score_fused";
        case SNAPKV_K_OBS_STATS: return "obs_score_stats";
        case SNAPKV_K_STATS_MERGE: return "obs_stats_merge";
        case SNAPKV_K_OBS_VOTES: return "obs_score_votes";
        case SNAPKV_K_POOL: return "vote_pool";
        case SNAPKV_K_SELECT: return "topk_select";
        case SNAPKV_K_GATHER: return "kv_gather";
        case SNAPKV_K_SUM_CHUNKS: return "sum_chunks";
        case SNAPKV_K_SELECT_TILES: return "topk_select_tiles";
        case SNAPKV_K_HIT_RATE: return "hit_rate";
        case SNAPKV_K_DECODE: return "decode_attention";
        case SNAPKV_K_DECODE_COMBINE: return "decode_combine";
        case SNAPKV_K_HIT_CLEAR: return "hit_rate_clear";
        case SNAPKV_K_SCRATCH_CLEAR: return "scratch_clear";
        case SNAPKV_K_WS_CLEAR: return "ws_clear";
        case SNAPKV_K_SELECT_SPLIT: return "topk_select_split";
        case SNAPKV_K_OBS_STREAM: return "obs_score_stream";
        case SNAPKV_K_OBS_ONEPASS: return "obs_score_onepass";
        case SNAPKV_K_OBS_ONEPASS2: return "obs_score_onepass2";
        default: return "unknown";
    }
}

const char *snapkv_strerror(int status) {
    switch (status) {
        case SNAPKV_OK: return "success";
        case SNAPKV_EINVAL: return "invalid argument";
        case SNAPKV_EWORKSPACE: return "workspace missing, misaligned or too small";
        case SNAPKV_EUNSUPPORTED: return "unsupported problem or device";
        case SNAPKV_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *snapkv_last_error(void) { return g_last_error.c_str(); }

int snapkv_version(void) { return 100; }

}  // extern "C"
