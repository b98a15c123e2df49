// index_scores.hip -- lightning-indexer scores on the gfx950 matrix cores.
//
// score[r, t] = sum_h w[r, h] * max(0, q_idx[r, h, :] . k_normed[s, t, :])
// (glm5next_dsa/layer.rs source page: module header trap list and the
// `weights_proj` field doc -- the head weights already carry
// index_heads^-0.5, the scorer adds no scale; `indexer_forward` -- the key
// cache is read token-major as k[raw * D + d]).
//
// Design (HBM-bound: 256 B of keys per token at D = 128 against 8 kflop):
//  - One workgroup owns a tile of 256 tokens of one sequence and scores it
//    for every row of that sequence (the K rows of a verify share one key
//    read). Keys stream HBM -> VGPR with fully coalesced 16-byte loads and are
//    parked in LDS with an XOR swizzle, then re-read in matrix-core operand
//    order without bank conflicts.
//  - The contraction is a 32x32x16 bf16 MFMA with the (up to 32) index heads
//    as M and 32 tokens as N; D is the reduction. A lane ends with 16 head
//    partials of one token; ReLU, weight and head sum run in fp32 in a fixed
//    order and one cross-lane add finishes the token (deterministic).
//  - Optionally the pass also builds, per row, the 2048-bin histogram of the
//    top 11 bits of each score's order key (LDS, flushed with integer global
//    atomics), which the exact top-k selection consumes.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kIdxTile = 256;    // tokens per workgroup
constexpr int kIdxThreads = 256; // 4 waves x 64 tokens

template <int D>
__global__ __launch_bounds__(kIdxThreads, 2) void k_index_scores(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
    const uint16_t *__restrict__ k_normed, const int32_t *__restrict__ seq_lens,
    float *__restrict__ scores, uint32_t *__restrict__ hist, int K, int Hi, int64_t cap,
    int max_len, int top_k)
{
    constexpr int CH = D / 8;  // 16-byte chunks per key row
    constexpr int KS = D / 16; // MFMA k-steps
    constexpr int LOADS = kIdxTile * CH / kIdxThreads;
    // 64 KiB: the key tile, later reused for the per-row histograms.
    __shared__ u32x4 lds[kIdxTile * 16];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int hl = lane / 32;
    const int s = blockIdx.y;
    const int t0 = blockIdx.x * kIdxTile;

    int lmax = 0;
    for (int j = 0; j < K; j++)
        lmax = max(lmax, min(max(seq_lens[s * K + j], 0), max_len));
    if (t0 >= lmax)
        return;

    // ---- stream the key tile into LDS (coalesced, swizzled) ----
    const uint16_t *kbase = k_normed + ((int64_t)s * cap + t0) * D;
    u32x4 regs[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
        const int g = i * kIdxThreads + tid;
        const int row = g / CH;
        const int c = g % CH;
        if (t0 + row < lmax)
            regs[i] = *(const u32x4 *)(kbase + (int64_t)row * D + c * 8);
        else
            regs[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
        const int g = i * kIdxThreads + tid;
        const int row = g / CH;
        const int c = g % CH;
        lds[row * CH + (c ^ (row & (CH - 1)))] = regs[i];
    }
    __syncthreads();

    // ---- key operands: column (token) lane%32, k-chunks hl*KS + ks ----
    bf16x8 kb[2][KS];
#pragma unroll
    for (int b = 0; b < 2; b++) {
        const int row = wave * 64 + b * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const int c = hl * KS + ks;
            kb[b][ks] = as_bf16x8(lds[row * CH + (c ^ (row & (CH - 1)))]);
        }
    }
    __syncthreads();

    // ---- per-row LDS histograms live where the tile was ----
    uint32_t *hl_lds = (uint32_t *)lds;
    const bool any_hist = hist != nullptr;
    if (any_hist) {
        for (int i = tid; i < K * kHistBins; i += kIdxThreads)
            hl_lds[i] = 0u;
        __syncthreads();
    }

    const int h_row = lane & 31;
    for (int j = 0; j < K; j++) {
        const int r = s * K + j;
        const int L = min(max(seq_lens[r], 0), max_len);
        if (t0 >= L)
            continue;
        // query operands: row (head) lane%32, same k-chunk order as the keys
        bf16x8 qa[KS];
        const uint16_t *qrow = q_idx + ((int64_t)r * Hi + h_row) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (h_row < Hi)
                v = *(const u32x4 *)(qrow + (hl * KS + ks) * 8);
            qa[ks] = as_bf16x8(v);
        }
        float wv[16];
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int h = 8 * (v / 4) + 4 * hl + (v % 4);
            wv[v] = (h < Hi) ? w[(int64_t)r * Hi + h] : 0.0f;
        }
        const bool do_hist = any_hist && L > top_k;
#pragma unroll
        for (int b = 0; b < 2; b++) {
            floatx16 acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                acc = mfma32x32x16(qa[ks], kb[b][ks], acc);
            float part = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; v++)
                part = __builtin_fmaf(wv[v], __builtin_fmaxf(acc[v], 0.0f), part);
            const float tot = part + __shfl_xor(part, 32, kWave);
            const int t = t0 + wave * 64 + b * 32 + (lane & 31);
            if (hl == 0 && t < L) {
                scores[(int64_t)r * max_len + t] = tot;
                if (do_hist)
                    atomicAdd(&hl_lds[j * kHistBins + (score_key(tot) >> kHistShift)], 1u);
            }
        }
    }

    if (any_hist) {
        __syncthreads();
        for (int j = 0; j < K; j++) {
            const int r = s * K + j;
            const int L = min(max(seq_lens[r], 0), max_len);
            if (t0 >= L || L <= top_k)
                continue;
            for (int bin = tid; bin < kHistBins; bin += kIdxThreads) {
                const uint32_t n = hl_lds[j * kHistBins + bin];
                if (n)
                    atomicAdd(&hist[(int64_t)r * kHistBins + bin], n);
            }
        }
    }
}

int launch_index_scores(const LaunchShape &ls, const uint16_t *q_idx, const float *w,
                        const uint16_t *k_normed, const int32_t *seq_lens, float *scores,
                        uint32_t *hist, hipStream_t stream)
{
    dim3 grid((ls.max_len + kIdxTile - 1) / kIdxTile, ls.num_seqs);
    dim3 block(kIdxThreads);
    if (ls.index_dim == 128)
        hipLaunchKernelGGL(k_index_scores<128>, grid, block, 0, stream, q_idx, w, k_normed,
                           seq_lens, scores, hist, ls.rows_per_seq, ls.index_heads,
                           (int64_t)ls.k_capacity, ls.max_len, ls.top_k);
    else if (ls.index_dim == 64)
        hipLaunchKernelGGL(k_index_scores<64>, grid, block, 0, stream, q_idx, w, k_normed,
                           seq_lens, scores, hist, ls.rows_per_seq, ls.index_heads,
                           (int64_t)ls.k_capacity, ls.max_len, ls.top_k);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
