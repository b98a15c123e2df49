// index_scores.hip -- lightning-indexer scores on the gfx950 matrix cores.
//
// score[r, t] = sum_h w[r, h] * max(0, q_idx[r, h, :] . k_normed[s, t, :])
// (glm5next_dsa/layer.rs source page: module header trap list and the
// `weights_proj` field doc -- the head weights already carry
// index_heads^-0.5, the scorer adds no scale; `indexer_forward` -- the key
// cache is read token-major as k[raw * D + d]).
//
// Design (HBM-bound: 256 B of keys per token at D = 128 against 8 kflop):
//  - One workgroup walks a run of 256-token tiles of one sequence and scores
//    each tile for every row of that sequence (the K rows of a verify share
//    one key read). Keys stream HBM -> VGPR with fully coalesced 16-byte
//    loads (the next tile's loads are in flight while the current tile
//    computes) and are parked in LDS with an XOR swizzle, then re-read in
//    matrix-core operand order without bank conflicts.
//  - The contraction is a 32x32x16 bf16 MFMA with the (up to 32) index heads
//    as M and 32 tokens as N; D is the reduction. A lane ends with 16 head
//    partials of one token; ReLU, weight and head sum run in fp32 in a fixed
//    order and one cross-lane add finishes the token (deterministic).
//  - Optionally the pass also builds, per row, the 2048-bin histogram of the
//    top 11 bits of each score's order key (16-bit LDS counters, flushed once
//    per workgroup with integer global atomics), which the exact top-k
//    selection consumes.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kIdxTile = 256;    // tokens per tile
constexpr int kIdxThreads = 256; // 4 waves x 64 tokens of a tile
constexpr int kIdxTargetWgs = 512; // two resident workgroups per CU

// Dynamic LDS: the key tile (64 KiB), then K packed per-row histograms
// (2048 16-bit counters = 4 KiB per row).
constexpr size_t kIdxTileBytes = kIdxTile * 16 * sizeof(u32x4);

template <int D, bool ONE_ROW>
__global__ __launch_bounds__(kIdxThreads, 2) void k_index_scores(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
    const uint16_t *__restrict__ k_normed, const int32_t *__restrict__ seq_lens,
    float *__restrict__ scores, uint32_t *__restrict__ hist, int K, int Hi, int64_t cap,
    int max_len, int top_k, int tiles_per_wg)
{
    constexpr int CH = D / 8;  // 16-byte chunks per key row
    constexpr int KS = D / 16; // MFMA k-steps
    constexpr int LOADS = kIdxTile * CH / kIdxThreads;
    extern __shared__ u32x4 lds[];
    uint32_t *hpack = (uint32_t *)(lds + kIdxTile * 16);

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int hl = lane / 32;
    const int s = blockIdx.y;

    int lmax = 0;
    for (int j = 0; j < K; j++)
        lmax = max(lmax, min(max(seq_lens[s * K + j], 0), max_len));
    const int tile_first = blockIdx.x * tiles_per_wg;
    const int tile_end = min(tile_first + tiles_per_wg, (lmax + kIdxTile - 1) / kIdxTile);
    if (tile_first >= tile_end)
        return;
    const bool any_hist = hist != nullptr;
    if (any_hist) {
        for (int i = tid; i < K * (kHistBins / 2); i += kIdxThreads)
            hpack[i] = 0u;
    }

    const uint16_t *kseq = k_normed + (int64_t)s * cap * D;
    u32x4 regs[LOADS];
    auto load_tile = [&](int tile) {
        const int t0 = tile * kIdxTile;
#pragma unroll
        for (int i = 0; i < LOADS; i++) {
            const int g = i * kIdxThreads + tid;
            const int row = g / CH;
            const int c = g % CH;
            if (t0 + row < lmax)
                regs[i] = *(const u32x4 *)(kseq + (int64_t)(t0 + row) * D + c * 8);
            else
                regs[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // query operands: row (head) lane%32, k-chunks hl*KS + ks (the same k
    // order as the key operands); weights of the 16 heads this lane reduces
    const int h_row = lane & 31;
    bf16x8 qa[KS];
    float wv[16];
    auto load_row = [&](int r) {
        const uint16_t *qrow = q_idx + ((int64_t)r * Hi + (h_row < Hi ? h_row : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (h_row < Hi)
                v = *(const u32x4 *)(qrow + (hl * KS + ks) * 8);
            qa[ks] = as_bf16x8(v);
        }
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int h = 8 * (v / 4) + 4 * hl + (v % 4);
            wv[v] = (h < Hi) ? w[(int64_t)r * Hi + h] : 0.0f;
        }
    };
    if (ONE_ROW)
        load_row(s);

    load_tile(tile_first);
    for (int tile = tile_first; tile < tile_end; tile++) {
        const int t0 = tile * kIdxTile;
        __syncthreads(); // every wave is done reading the previous tile
#pragma unroll
        for (int i = 0; i < LOADS; i++) {
            const int g = i * kIdxThreads + tid;
            const int row = g / CH;
            const int c = g % CH;
            lds[row * CH + (c ^ (row & (CH - 1)))] = regs[i];
        }
        __syncthreads();
        if (tile + 1 < tile_end)
            load_tile(tile + 1); // in flight while this tile computes

        // key operands: column (token) lane%32, k-chunks hl*KS + ks
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

        for (int j = 0; j < K; j++) {
            const int r = s * K + j;
            const int L = min(max(seq_lens[r], 0), max_len);
            if (t0 >= L)
                continue;
            if (!ONE_ROW)
                load_row(r);
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
                    if (do_hist) {
                        const uint32_t bin = score_key(tot) >> kHistShift;
                        atomicAdd(&hpack[j * (kHistBins / 2) + (bin >> 1)], 1u << (16 * (bin & 1)));
                    }
                }
            }
        }
    }

    if (any_hist) {
        __syncthreads();
        for (int j = 0; j < K; j++) {
            const int r = s * K + j;
            const int L = min(max(seq_lens[r], 0), max_len);
            if (tile_first * kIdxTile >= L || L <= top_k)
                continue;
            for (int word = tid; word < kHistBins / 2; word += kIdxThreads) {
                const uint32_t pk = hpack[j * (kHistBins / 2) + word];
                if (pk & 0xFFFFu)
                    atomicAdd(&hist[(int64_t)r * kHistBins + 2 * word], pk & 0xFFFFu);
                if (pk >> 16)
                    atomicAdd(&hist[(int64_t)r * kHistBins + 2 * word + 1], pk >> 16);
            }
        }
    }
}

template <int D, bool ONE_ROW>
static void launch_one(const LaunchShape &ls, dim3 grid, size_t lds, const uint16_t *q_idx,
                       const float *w, const uint16_t *k_normed, const int32_t *seq_lens,
                       float *scores, uint32_t *hist, int tpw, hipStream_t stream)
{
    hipLaunchKernelGGL((k_index_scores<D, ONE_ROW>), grid, dim3(kIdxThreads), lds, stream, q_idx,
                       w, k_normed, seq_lens, scores, hist, ls.rows_per_seq, ls.index_heads,
                       (int64_t)ls.k_capacity, ls.max_len, ls.top_k, tpw);
}

int launch_index_scores(const LaunchShape &ls, const uint16_t *q_idx, const float *w,
                        const uint16_t *k_normed, const int32_t *seq_lens, float *scores,
                        uint32_t *hist, hipStream_t stream)
{
    static bool attr_done = false;
    const size_t lds = kIdxTileBytes + (size_t)ls.rows_per_seq * (kHistBins / 2) * 4;
    if (!attr_done) {
        const int mx = (int)(kIdxTileBytes + 8 * (kHistBins / 2) * 4);
        hipFuncSetAttribute((const void *)k_index_scores<128, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, mx);
        hipFuncSetAttribute((const void *)k_index_scores<128, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, mx);
        hipFuncSetAttribute((const void *)k_index_scores<64, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, mx);
        hipFuncSetAttribute((const void *)k_index_scores<64, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, mx);
        attr_done = true;
    }
    // Spread the sequence's tiles over ~kIdxTargetWgs workgroups; each walks
    // its run of tiles with the next tile's loads in flight (the histogram
    // counters of one workgroup stay 16-bit: at most 255 tiles of 256).
    const int tiles_per_seq = (ls.max_len + kIdxTile - 1) / kIdxTile;
    const long total = (long)tiles_per_seq * ls.num_seqs;
    int tpw = (int)((total + kIdxTargetWgs - 1) / kIdxTargetWgs);
    tpw = tpw < 1 ? 1 : (tpw > 64 ? 64 : tpw);
    dim3 grid((tiles_per_seq + tpw - 1) / tpw, ls.num_seqs);
    const bool one = ls.rows_per_seq == 1;
    if (ls.index_dim == 128) {
        if (one)
            launch_one<128, true>(ls, grid, lds, q_idx, w, k_normed, seq_lens, scores, hist, tpw, stream);
        else
            launch_one<128, false>(ls, grid, lds, q_idx, w, k_normed, seq_lens, scores, hist, tpw, stream);
    } else if (ls.index_dim == 64) {
        if (one)
            launch_one<64, true>(ls, grid, lds, q_idx, w, k_normed, seq_lens, scores, hist, tpw, stream);
        else
            launch_one<64, false>(ls, grid, lds, q_idx, w, k_normed, seq_lens, scores, hist, tpw, stream);
    } else {
        return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
