// topk_select.hip -- exact per-row top-k over [0, L_r) on gfx950.
//
// Order (glm5next_dsa/layer.rs source page, doc of the prefill row-group
// selector before `batch_select_enabled`): score descending, then index
// ascending -- a total order, so the top-k set is unique. Read per token
// (pools of one token); -0.0 equals +0.0. Output: the selected ids in
// ascending order, -1 past min(top_k, L_r).
//
// Radix selection on the order-preserving 32-bit key of each score:
//  1. A 2048-bin histogram of the key's top 11 bits per row (fused into the
//     scoring pass by dsa_decode_k; a separate pass for dsa_topk_select).
//  2. k_select_candidates, one workgroup per 4096-token chunk of a row: every
//     workgroup finds the bin b* that holds the k-th largest key, counts the
//     keys above b* in its chunk and compacts the keys inside b* into the
//     chunk's own candidate region. The last workgroup of the row (an
//     atomic ticket; no workgroup ever waits) resolves the exact threshold
//     key T and the index cut among keys equal to T with four more radix
//     passes over the candidates, then turns per-chunk selected counts into
//     output offsets.
//  3. k_select_compact, again one workgroup per chunk: writes the selected
//     ids of its chunk in ascending order at the chunk's offset.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kSelThreads = 256;
constexpr int kSelPerThread = kSelChunk / kSelThreads; // 16

__global__ void k_clear(u32x4 *p, size_t n16)
{
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

int launch_clear(void *ws, size_t bytes, hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0)
        return 0;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 1024)
        blocks = 1024;
    hipLaunchKernelGGL(k_clear, dim3((unsigned)blocks), dim3(256), 0, stream, (u32x4 *)ws, n16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Histogram of the top 11 key bits of scores[r, 0..L) (rows with L > top_k).
__global__ __launch_bounds__(kSelThreads) void k_score_hist(const float *__restrict__ scores,
                                                            const int32_t *__restrict__ seq_lens,
                                                            uint32_t *__restrict__ hist,
                                                            int max_len, int top_k)
{
    __shared__ uint32_t h[kHistBins];
    const int r = blockIdx.y;
    const int L = min(max(seq_lens[r], 0), max_len);
    const int base = blockIdx.x * kSelChunk;
    if (L <= top_k || base >= L)
        return;
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads)
        h[i] = 0u;
    __syncthreads();
    const float *row = scores + (int64_t)r * max_len;
    for (int i = 0; i < kSelPerThread; i++) {
        const int t = base + i * kSelThreads + threadIdx.x;
        if (t < L)
            atomicAdd(&h[score_key(row[t]) >> kHistShift], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads)
        if (h[i])
            atomicAdd(&hist[(int64_t)r * kHistBins + i], h[i]);
}

int launch_score_hist(const LaunchShape &ls, const float *scores, const int32_t *seq_lens,
                      uint32_t *hist, hipStream_t stream)
{
    dim3 grid(sel_chunks(ls), ls.num_rows);
    hipLaunchKernelGGL(k_score_hist, grid, dim3(kSelThreads), 0, stream, scores, seq_lens, hist,
                       ls.max_len, ls.top_k);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Shared state of one block-wide bin search.
struct BinSearch {
    uint32_t scan[kSelThreads / kWave + 1];
    uint32_t bin;
    uint32_t before;
};

// Over the LDS histogram h[0..nbins), walked from the highest bin down
// (descending) or from bin 0 up (ascending), find the bin where the running
// count first reaches `need` (1 <= need <= total). Returns the bin; *before is
// the count of everything walked before it. All threads must call.
template <bool Descending>
__device__ uint32_t find_bin(const uint32_t *h, int nbins, uint32_t need, BinSearch *bs,
                             uint32_t *before)
{
    const int bpt = nbins / kSelThreads;
    const int tid = threadIdx.x;
    if (tid == 0) {
        bs->bin = 0u; // defined result even for an inconsistent histogram
        bs->before = 0u;
    }
    uint32_t local = 0;
    for (int i = 0; i < bpt; i++) {
        const int p = tid * bpt + i;
        local += h[Descending ? nbins - 1 - p : p];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<kSelThreads>(local, bs->scan, &total);
    for (int i = 0; i < bpt; i++) {
        const int p = tid * bpt + i;
        const int b = Descending ? nbins - 1 - p : p;
        const uint32_t c = h[b];
        if (run < need && run + c >= need) {
            bs->bin = (uint32_t)b;
            bs->before = run;
        }
        run += c;
    }
    __syncthreads();
    const uint32_t b = bs->bin;
    *before = bs->before;
    __syncthreads();
    return b;
}

__global__ __launch_bounds__(kSelThreads) void k_select_candidates(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    const uint32_t *__restrict__ hist, SelRow *__restrict__ rows, uint32_t *__restrict__ n_gt,
    uint32_t *__restrict__ n_cand, uint32_t *__restrict__ offsets, u32x2 *__restrict__ cand,
    int max_len, int top_k, int nc_max)
{
    __shared__ uint32_t h[kHistBins];
    __shared__ uint32_t chunk_cnt[1024];
    __shared__ uint32_t chunk_cand[1024];
    __shared__ BinSearch bs;
    __shared__ uint32_t scan[kSelThreads / kWave + 1];
    __shared__ int is_last;

    const int r = blockIdx.y;
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = min(max(seq_lens[r], 0), max_len);
    if (L <= top_k)
        return;
    const int nc = (L + kSelChunk - 1) / kSelChunk;
    if (c >= nc)
        return;
    SelRow *st = rows + r;

    // ---- the bin b* of the top_k-th largest key ----
    for (int i = tid; i < kHistBins; i += kSelThreads)
        h[i] = hist[(int64_t)r * kHistBins + i];
    __syncthreads();
    uint32_t above;
    const uint32_t bstar = find_bin<true>(h, kHistBins, (uint32_t)top_k, &bs, &above);
    const uint32_t need = (uint32_t)top_k - above; // keys to take from bin b*

    // ---- this chunk: count keys above b*, gather keys inside b* into the
    //      chunk's own candidate region (no cross-workgroup atomics) ----
    const float *row = scores + (int64_t)r * max_len;
    u32x2 *rc = cand + (int64_t)r * max_len;
    uint32_t keys[kSelPerThread];
    uint32_t inmask = 0, gt = 0, nin = 0;
#pragma unroll
    for (int i = 0; i < kSelPerThread; i++) {
        const int t = c * kSelChunk + i * kSelThreads + tid;
        keys[i] = 0;
        if (t < L) {
            keys[i] = score_key(row[t]);
            const uint32_t b = keys[i] >> kHistShift;
            gt += b > bstar;
            if (b == bstar) {
                inmask |= 1u << i;
                nin++;
            }
        }
    }
    uint32_t n_in_chunk;
    uint32_t at = block_exclusive_scan<kSelThreads>(nin, scan, &n_in_chunk);
#pragma unroll
    for (int i = 0; i < kSelPerThread; i++)
        if (inmask & (1u << i))
            rc[c * kSelChunk + at++] = u32x2{keys[i], (uint32_t)(c * kSelChunk + i * kSelThreads + tid)};
    uint32_t n_gt_chunk;
    block_exclusive_scan<kSelThreads>(gt, scan, &n_gt_chunk);
    if (tid == 0) {
        n_gt[(int64_t)r * nc_max + c] = n_gt_chunk;
        n_cand[(int64_t)r * nc_max + c] = n_in_chunk;
    }

    // ---- the last workgroup of the row resolves the threshold ----
    __threadfence();
    __syncthreads();
    if (tid == 0)
        is_last = atomicAdd(&st->ticket, 1u) == (uint32_t)(nc - 1);
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();
    for (int i = tid; i < nc; i += kSelThreads) {
        chunk_cand[i] = min(__hip_atomic_load(&n_cand[(int64_t)r * nc_max + i], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT),
                            (uint32_t)kSelChunk);
        chunk_cnt[i] = __hip_atomic_load(&n_gt[(int64_t)r * nc_max + i], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // visit every candidate of the row (chunk regions, in any order)
    auto for_each = [&](auto &&f) {
        for (int cc = 0; cc < nc; cc++) {
            const uint32_t n = chunk_cand[cc];
            for (uint32_t i = tid; i < n; i += kSelThreads)
                f(rc[cc * kSelChunk + i]);
        }
    };

    // pass A: key bits [20:10] of the candidates, descending
    for (int i = tid; i < kHistBins; i += kSelThreads)
        h[i] = 0u;
    __syncthreads();
    for_each([&](u32x2 e) { atomicAdd(&h[(e.x >> 10) & 0x7FFu], 1u); });
    __syncthreads();
    uint32_t bef;
    const uint32_t a_bin = find_bin<true>(h, 2048, need, &bs, &bef);
    const uint32_t need_a = need - bef;
    const uint32_t hi21 = (bstar << 11) | a_bin; // key >> 10

    // pass B: key bits [9:0] among key >> 10 == hi21, descending
    for (int i = tid; i < kHistBins; i += kSelThreads)
        h[i] = 0u;
    __syncthreads();
    for_each([&](u32x2 e) {
        if ((e.x >> 10) == hi21)
            atomicAdd(&h[e.x & 0x3FFu], 1u);
    });
    __syncthreads();
    const uint32_t b_bin = find_bin<true>(h, 1024, need_a, &bs, &bef);
    const uint32_t need_t = need_a - bef; // keys equal to T to take
    const uint32_t eq_count = h[b_bin];
    const uint32_t T = (hi21 << 10) | b_bin;
    __syncthreads();

    int32_t cut = 0x7FFFFFFF;
    if (need_t < eq_count) {
        // pass C: index bits [21:11] among keys == T, ascending
        for (int i = tid; i < kHistBins; i += kSelThreads)
            h[i] = 0u;
        __syncthreads();
        for_each([&](u32x2 e) {
            if (e.x == T)
                atomicAdd(&h[(e.y >> 11) & 0x7FFu], 1u);
        });
        __syncthreads();
        const uint32_t c_bin = find_bin<false>(h, 2048, need_t, &bs, &bef);
        const uint32_t need_c = need_t - bef;
        // pass D: index bits [10:0] among keys == T in index block c_bin
        for (int i = tid; i < kHistBins; i += kSelThreads)
            h[i] = 0u;
        __syncthreads();
        for_each([&](u32x2 e) {
            if (e.x == T && (e.y >> 11) == c_bin)
                atomicAdd(&h[e.y & 0x7FFu], 1u);
        });
        __syncthreads();
        const uint32_t d_bin = find_bin<false>(h, 2048, need_c, &bs, &bef);
        cut = (int32_t)((c_bin << 11) | d_bin);
    }

    // per-chunk selected counts -> exclusive offsets
    for_each([&](u32x2 e) {
        if (e.x > T || (e.x == T && (int32_t)e.y <= cut))
            atomicAdd(&chunk_cnt[e.y / kSelChunk], 1u);
    });
    __syncthreads();
    if (tid == 0) {
        uint32_t run = 0;
        for (int i = 0; i < nc; i++) {
            offsets[(int64_t)r * nc_max + i] = run;
            run += chunk_cnt[i];
        }
        st->thr_key = T;
        st->idx_cut = cut;
    }
}

__global__ __launch_bounds__(kSelThreads) void k_select_compact(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    const SelRow *__restrict__ rows, const uint32_t *__restrict__ offsets,
    int32_t *__restrict__ sel, int max_len, int top_k, int nc_max)
{
    __shared__ uint32_t scan[kSelThreads / kWave + 1];
    const int r = blockIdx.y;
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = min(max(seq_lens[r], 0), max_len);
    int32_t *out = sel + (int64_t)r * top_k;

    if (L <= top_k) {
        // every token is selected; slots past L are padding
        for (int i = 0; i < kSelPerThread; i++) {
            const int slot = c * kSelChunk + i * kSelThreads + tid;
            if (slot < top_k)
                out[slot] = slot < L ? slot : -1;
        }
        return;
    }
    const int nc = (L + kSelChunk - 1) / kSelChunk;
    if (c >= nc)
        return;
    const uint32_t T = rows[r].thr_key;
    const int32_t cut = rows[r].idx_cut;
    const float *row = scores + (int64_t)r * max_len;
    const int t0 = c * kSelChunk + tid * kSelPerThread;
    uint32_t flags = 0;
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < kSelPerThread; i++) {
        const int t = t0 + i;
        if (t < L) {
            const uint32_t k = score_key(row[t]);
            if (k > T || (k == T && t <= cut)) {
                flags |= 1u << i;
                cnt++;
            }
        }
    }
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kSelThreads>(cnt, scan, &total) +
                   offsets[(int64_t)r * nc_max + c];
#pragma unroll
    for (int i = 0; i < kSelPerThread; i++)
        if ((flags & (1u << i)) && pos < (uint32_t)top_k)
            out[pos++] = t0 + i;
}

int launch_select(const LaunchShape &ls, const float *scores, const int32_t *seq_lens,
                  int32_t *sel, char *ws, const Workspace &wl, hipStream_t stream)
{
    const int nc = sel_chunks(ls);
    const uint32_t *hist = (const uint32_t *)(ws + wl.hist);
    SelRow *rows = (SelRow *)(ws + wl.selrow);
    uint32_t *n_gt = (uint32_t *)(ws + wl.n_gt);
    uint32_t *n_cand = (uint32_t *)(ws + wl.n_cand);
    uint32_t *offs = (uint32_t *)(ws + wl.offsets);
    u32x2 *cand = (u32x2 *)(ws + wl.cand);
    hipLaunchKernelGGL(k_select_candidates, dim3(nc, ls.num_rows), dim3(kSelThreads), 0, stream,
                       scores, seq_lens, hist, rows, n_gt, n_cand, offs, cand, ls.max_len,
                       ls.top_k, nc);
    if (hipGetLastError() != hipSuccess)
        return -1;
    const int ncc = (ls.max_len > ls.top_k ? ls.max_len : ls.top_k);
    const int gx = (ncc + kSelChunk - 1) / kSelChunk;
    hipLaunchKernelGGL(k_select_compact, dim3(gx, ls.num_rows), dim3(kSelThreads), 0, stream,
                       scores, seq_lens, rows, offs, sel, ls.max_len, ls.top_k, nc);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
