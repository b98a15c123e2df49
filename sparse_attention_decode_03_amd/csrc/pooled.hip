// pooled.hip -- pooled selection (pools of kp consecutive tokens) and its
// expansion back to token ids.
//
// Doc of the prefill row-group selector on the glm5next_dsa layer.rs source
// page: a pool is a candidate of a row only when it is complete and its last
// token is visible to the row's query, so row r sees pools [0, L_r / kp); the
// row takes row_select_k = min(select_k, L_r / kp) pools under the total
// order (score descending, pool index ascending); the selected pools expand
// to their kp tokens, and the row's visible tail (the incomplete pool's
// tokens, L_r / kp * kp .. L_r - 1) goes from slot row_select_k * kp on. The
// per-row tail base is the pages' correction that keeps a row's slot
// geometry independent of the rows it is batched with.
//
// The same doc's candidacy test has a second term, pool_valid[p]: a pool
// that is not complete is no candidate. With the caller's pool_valid the
// incomplete pools score -inf (a copy of the row's pool scores), so they rank
// below every candidate, and the expansion drops any that was still taken
// (a row with fewer candidates than row_select_k): the candidates' tokens
// fill the first slots, the places of dropped pools are -1, and the tail
// still starts at row_select_k * kp (the row's slot geometry is a function of
// its position alone).
//
// The selection over pool scores is the per-token selector of topk_select.hip
// run on per-row pool counts; the pool scores are the caller's.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kPoolThreads = 256;

// Pools each row sees.
__global__ __launch_bounds__(kPoolThreads) void k_pool_lens(const int32_t *__restrict__ seq_lens,
                                                            int32_t *__restrict__ pool_lens, int R,
                                                            int max_len, int kp)
{
    const int r = blockIdx.x * kPoolThreads + threadIdx.x;
    if (r < R)
        pool_lens[r] = min(max(seq_lens[r], 0), max_len) / kp;
}

// Incomplete pools of each row at -inf, the others' scores copied.
__global__ __launch_bounds__(kPoolThreads) void k_pool_mask(const float *__restrict__ pool_scores,
                                                            const uint8_t *__restrict__ pool_valid,
                                                            const int32_t *__restrict__ pool_lens,
                                                            float *__restrict__ masked, int K,
                                                            int stride)
{
    const int r = blockIdx.y;
    const int p = blockIdx.x * kPoolThreads + threadIdx.x;
    if (p < pool_lens[r]) {
        const int64_t i = (int64_t)r * stride + p;
        masked[i] = pool_valid[(int64_t)(r / K) * stride + p] ? pool_scores[i] : -__builtin_huge_valf();
    }
}

// One workgroup per row: the selected pools (ascending ids) to their kp
// tokens each -- with pool_valid, the complete ones only, packed to the
// front, the dropped ones' places -1 -- then the visible tail from slot
// row_select_k * kp, then -1.
__global__ __launch_bounds__(kPoolThreads) void k_expand_pools(
    const int32_t *__restrict__ sel_pools, const uint8_t *__restrict__ pool_valid,
    const int32_t *__restrict__ seq_lens, int32_t *__restrict__ sel, int max_len, int kp,
    int select_k, int width, int K, int pstride)
{
    __shared__ uint32_t scan[kPoolThreads / kWave + 1];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = min(max(seq_lens[r], 0), max_len);
    const int pvis = L / kp;
    const int rsk = min(select_k, pvis);
    const int head = rsk * kp;
    const int tail = L - pvis * kp;
    const int32_t *sp = sel_pools + (int64_t)r * select_k;
    const uint8_t *pv = pool_valid != nullptr ? pool_valid + (int64_t)(r / K) * pstride : nullptr;
    // thread t owns selected places [j0, j1): its kept pools, counted and
    // then placed after the kept pools of lower places
    const int per = (rsk + kPoolThreads - 1) / kPoolThreads;
    const int j0 = min(tid * per, rsk), j1 = min(j0 + per, rsk);
    auto kept = [&](int j) {
        const int p = sp[j];
        return p >= 0 && (pv == nullptr || pv[p] != 0);
    };
    uint32_t mine = 0;
    for (int j = j0; j < j1; j++)
        mine += kept(j) ? 1u : 0u;
    uint32_t nkept;
    uint32_t c = block_exclusive_scan<kPoolThreads>(mine, scan, &nkept);
    int32_t *out = sel + (int64_t)r * width;
    for (int j = j0; j < j1; j++) {
        if (kept(j)) {
            const int p = sp[j];
            for (int i = 0; i < kp; i++)
                out[c * kp + i] = p * kp + i;
            c++;
        }
    }
    for (int slot = (int)nkept * kp + tid; slot < width; slot += kPoolThreads)
        out[slot] = (slot >= head && slot < head + tail) ? pvis * kp + (slot - head) : -1;
}

int launch_select_pooled(const LaunchShape &ls_pool, int max_len, int kp, const float *pool_scores,
                         const uint8_t *pool_valid, const int32_t *seq_lens, int32_t *sel, char *ws,
                         const Workspace &wl, size_t pool_lens_off, size_t sel_pools_off,
                         size_t masked_off, bool any_pool, hipStream_t stream)
{
    const int R = ls_pool.num_rows;
    const int pstride = score_stride(ls_pool);
    int32_t *pool_lens = (int32_t *)(ws + pool_lens_off);
    int32_t *sel_pools = (int32_t *)(ws + sel_pools_off);
    if (any_pool) {
        hipLaunchKernelGGL(k_pool_lens, dim3((R + kPoolThreads - 1) / kPoolThreads),
                           dim3(kPoolThreads), 0, stream, seq_lens, pool_lens, R, max_len, kp);
        if (hipGetLastError() != hipSuccess)
            return -1;
        const float *scores = pool_scores;
        if (pool_valid != nullptr) {
            float *masked = (float *)(ws + masked_off);
            hipLaunchKernelGGL(k_pool_mask, dim3((ls_pool.max_len + kPoolThreads - 1) / kPoolThreads, R),
                               dim3(kPoolThreads), 0, stream, pool_scores, pool_valid, pool_lens,
                               masked, ls_pool.rows_per_seq, pstride);
            if (hipGetLastError() != hipSuccess)
                return -1;
            scores = masked;
        }
        if (launch_select(ls_pool, scores, pool_lens, sel_pools, ws, wl, false, stream) != 0)
            return -1;
    }
    const int width = ls_pool.top_k * kp + kp - 1;
    hipLaunchKernelGGL(k_expand_pools, dim3(R), dim3(kPoolThreads), 0, stream, sel_pools,
                       any_pool ? pool_valid : nullptr, seq_lens, sel, max_len, kp, ls_pool.top_k,
                       width, ls_pool.rows_per_seq, pstride);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
