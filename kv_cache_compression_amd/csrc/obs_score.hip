// obs_score.hip -- the stats merge and chunk-sum kernels of the scoring step, and the
// choice of the scoring kernel's instantiation (the kernel itself: obs_score_kernel.h).
#include "obs_score_kernel.h"

namespace snapkv {

// Two-pass path: combine the per-slab stats of every (request, KV head, row chunk, row).
// grid: (segments * chunks, ceil(chunk rows / 4)); each wave merges one row, its lanes
// striding over the segment's slabs.
__global__ void __launch_bounds__(256) merge_stats_kernel(const MergeParams p) {
    const int C = p.n_chunks;
    const int vs = blockIdx.x, seg = vs / C, chunk = vs - (vs / C) * C;
    const int r = seg / p.Hkv, g = seg - (seg / p.Hkv) * p.Hkv;
    const int ns = (p.rt.L[r] + p.slab_keys - 1) / p.slab_keys;
    const int base = p.rt.slab0[r] + g * ns;
    const int row = blockIdx.y * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int Mc = p.M - chunk * p.M_pad < p.M_pad ? p.M - chunk * p.M_pad : p.M_pad;
    if (row >= Mc) return;  // whole wave
    float m = neg_inf(), l = 0.f;
    for (int s = lane; s < ns; s += 64) {
        const float2 pr = p.partial[((int64_t)(base + s) * C + chunk) * p.M_pad + row];
        merge_stats(m, l, pr.x, pr.y, p.c);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o), l2 = __shfl_xor(l, o);
        merge_stats(m, l, m2, l2, p.c);
    }
    if (lane == 0) p.merged[(int64_t)vs * p.M_pad + row] = make_float2(m, l);
}

// Row-chunked scoring: votes[g][j] = sum over the chunk planes.  grid: (column blocks, H_kv).
__global__ void __launch_bounds__(256) sum_chunks_kernel(const SumParams p) {
    const int64_t j = p.col0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= p.col1) return;
    const int64_t o = (int64_t)blockIdx.y * p.sum_P + j;
    float a = p.planes[o];
    for (int c = 1; c < p.n_chunks; ++c) a += p.planes[c * p.vplane + o];
    p.votes[o] = a;
}
const void *sum_kernel() { return (const void *)&sum_chunks_kernel; }

const void *merge_kernel() { return (const void *)&merge_stats_kernel; }

// ---- instantiation table ---------------------------------------------------------------

// Every kernel scores 32 query rows (a row chunk): rows of 256 bytes take the
// register-staged key stream (eight waves, 16 key tiles per wave), other rows direct
// MFMA-layout loads.
bool obs_config(int dtype, int d, ObsConfig *cfg) {
    if (d != 64 && d != 128) return false;
    const int rowb = d * (dtype == 0 ? 4 : 2);
    *cfg = rowb <= 256 ? ObsConfig{1, 8, 2, 16} : ObsConfig{1, 8, 2, 8};
    return true;
}

// Rows of 256 bytes also come with 12 key tiles per wave (1536-key slabs), for segments
// whose 2048-key slab count packs badly into the grid's iterations.
bool obs_config_short(int dtype, int d, ObsConfig *cfg) {
    if (!obs_config(dtype, d, cfg) || d * (dtype == 0 ? 4 : 2) != 256) return false;
    cfg->ctw = 12;
    return true;
}

const void *obs_kernel(int dtype, int d, const ObsConfig &cfg, int mode, bool keep) {
    if (dtype == 1) return d == 64 ? obs_kernel_bf16_d64(mode, keep, cfg.ctw) : obs_kernel_bf16_d128(mode, keep, cfg.ctw);
    return d == 64 ? obs_kernel_f32_d64(mode, keep, cfg.ctw) : obs_kernel_f32_d128(mode, keep, cfg.ctw);
}

}  // namespace snapkv
