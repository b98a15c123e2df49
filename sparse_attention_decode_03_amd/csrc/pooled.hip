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

// One workgroup per row: the selected pools (ascending ids, -1 padded) to
// their kp tokens each, then the visible tail, then -1.
__global__ __launch_bounds__(kPoolThreads) void k_expand_pools(
    const int32_t *__restrict__ sel_pools, const int32_t *__restrict__ seq_lens,
    int32_t *__restrict__ sel, int max_len, int kp, int select_k, int width)
{
    const int r = blockIdx.x;
    const int L = min(max(seq_lens[r], 0), max_len);
    const int pvis = L / kp;
    const int head = min(select_k, pvis) * kp;
    const int tail = L - pvis * kp;
    for (int slot = threadIdx.x; slot < width; slot += kPoolThreads) {
        int t = -1;
        if (slot < head) {
            const int p = sel_pools[(int64_t)r * select_k + slot / kp];
            t = p >= 0 ? p * kp + slot % kp : -1;
        } else if (slot < head + tail) {
            t = pvis * kp + (slot - head);
        }
        sel[(int64_t)r * width + slot] = t;
    }
}

int launch_select_pooled(const LaunchShape &ls_pool, int max_len, int kp, const float *pool_scores,
                         const int32_t *seq_lens, int32_t *sel, char *ws, const Workspace &wl,
                         size_t pool_lens_off, size_t sel_pools_off, bool any_pool,
                         hipStream_t stream)
{
    const int R = ls_pool.num_rows;
    int32_t *pool_lens = (int32_t *)(ws + pool_lens_off);
    int32_t *sel_pools = (int32_t *)(ws + sel_pools_off);
    if (any_pool) {
        hipLaunchKernelGGL(k_pool_lens, dim3((R + kPoolThreads - 1) / kPoolThreads),
                           dim3(kPoolThreads), 0, stream, seq_lens, pool_lens, R, max_len, kp);
        if (hipGetLastError() != hipSuccess)
            return -1;
        if (launch_select(ls_pool, pool_scores, pool_lens, sel_pools, ws, wl, false, stream) != 0)
            return -1;
    }
    const int width = ls_pool.top_k * kp + kp - 1;
    hipLaunchKernelGGL(k_expand_pools, dim3(R), dim3(kPoolThreads), 0, stream, sel_pools, seq_lens,
                       sel, max_len, kp, ls_pool.top_k, width);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
