// topk_select.hip -- exact per-row top-k over [0, L_r) on gfx950.
//
// Order (glm5next_dsa/layer.rs source page, doc of the prefill row-group
// selector before `batch_select_enabled`): score descending, then index
// ascending -- a total order, so the top-k set is unique. Read per token
// (pools of one token); -0.0 equals +0.0. Output: the selected ids in
// ascending order, -1 past min(top_k, L_r).
//
// One workgroup of 1024 threads owns one row, so no step ever waits on
// another workgroup. Radix selection on the order-preserving 32-bit key of
// each score:
//  1. sweep 1: a 2048-bin histogram of the key's top 11 bits (four LDS copies
//     to spread atomic contention); the bin b* holding the k-th largest key
//     follows from a suffix scan;
//  2. sweep 2: keys above b* go straight into a bitmap of the row (one wave
//     ballot builds eight bitmap words, no atomics); keys inside b* are the
//     candidates, appended to LDS (or to a workspace spill past capacity);
//  3. four radix passes over the candidates resolve the exact threshold key T
//     and, among keys equal to T, the largest selected index;
//  4. the selected candidates join the bitmap, and a block-wide scan of the
//     bitmap's popcounts writes the ids in ascending order.
// Sweeps read the row with 16-byte loads, two batches in flight.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kVecBatch = 8;           // float4 loads per thread per batch
constexpr int kCandCap = 6144;         // candidates kept in LDS (48 KiB)
constexpr int kBitmapLdsWords = 12288; // rows up to 393216 tokens keep the bitmap in LDS

// Shared state of one block-wide bin search.
struct BinSearch {
    uint32_t scan[kRowWaves + 1];
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
    const int bpt = (nbins + kRowThreads - 1) / kRowThreads;
    const int tid = threadIdx.x;
    if (tid == 0) {
        bs->bin = 0u; // defined result even for an inconsistent histogram
        bs->before = 0u;
    }
    uint32_t local = 0;
    for (int i = 0; i < bpt; i++) {
        const int p = tid * bpt + i;
        if (p < nbins)
            local += h[Descending ? nbins - 1 - p : p];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<kRowThreads>(local, bs->scan, &total);
    for (int i = 0; i < bpt; i++) {
        const int p = tid * bpt + i;
        if (p >= nbins)
            break;
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

// Spread the 8 bits of x to bit positions 0, 4, 8, ..., 28.
__device__ __forceinline__ uint32_t spread8(uint32_t x)
{
    x = (x | (x << 12)) & 0x000F000Fu;
    x = (x | (x << 6)) & 0x03030303u;
    x = (x | (x << 3)) & 0x11111111u;
    return x;
}

__global__ __launch_bounds__(kRowThreads) void k_select_row(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    int32_t *__restrict__ sel, u32x2 *__restrict__ spill, uint32_t *__restrict__ gbitmap,
    int max_len, int stride, int top_k)
{
    __shared__ uint32_t hsub[4][kHistBins];
    __shared__ u32x2 cbuf[kCandCap];
    __shared__ uint32_t lbitmap[kBitmapLdsWords];
    __shared__ BinSearch bs;
    __shared__ uint32_t ccount;

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int L = min(max(seq_lens[r], 0), max_len);
    int32_t *out = sel + (int64_t)r * top_k;

    if (L <= top_k) { // every token is selected; slots past L are padding
        for (int slot = tid; slot < top_k; slot += kRowThreads)
            out[slot] = slot < L ? slot : -1;
        return;
    }

    const float4 *row4 = (const float4 *)(scores + (int64_t)r * stride);
    const int nvec = (L + 3) / 4; // float4s covering [0, L) (all inside the row stride)
    constexpr int kBatchTok = kRowThreads * kVecBatch * 4;
    // Two batches of kVecBatch float4 per thread in flight; f(t, v) runs for
    // the float4 v holding tokens t .. t+3 (t a multiple of 4; entries at or
    // past L are masked by f).
    auto sweep = [&](auto &&f) {
        float4 a[kVecBatch], b[kVecBatch];
        auto load = [&](float4(&x)[kVecBatch], int base) {
#pragma unroll
            for (int k = 0; k < kVecBatch; k++)
                x[k] = row4[min(base / 4 + k * kRowThreads + tid, nvec - 1)];
        };
        auto use = [&](const float4(&x)[kVecBatch], int base) {
#pragma unroll
            for (int k = 0; k < kVecBatch; k++)
                f(base + 4 * (k * kRowThreads + tid), x[k]);
        };
        load(a, 0);
        for (int base = 0; base < L; base += 2 * kBatchTok) {
            if (base + kBatchTok < L)
                load(b, base + kBatchTok);
            use(a, base);
            if (base + kBatchTok >= L)
                break;
            if (base + 2 * kBatchTok < L)
                load(a, base + 2 * kBatchTok);
            use(b, base + kBatchTok);
        }
    };

    // ---- sweep 1: histogram of the top 11 key bits ----
    for (int i = tid; i < 4 * kHistBins; i += kRowThreads)
        (&hsub[0][0])[i] = 0u;
    __syncthreads();
    uint32_t *myh = hsub[wave & 3];
    sweep([&](int t, float4 v) {
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; j++)
            if (t + j < L)
                atomicAdd(&myh[score_key(e[j]) >> kHistShift], 1u);
    });
    __syncthreads();
    for (int i = tid; i < kHistBins; i += kRowThreads)
        hsub[0][i] += hsub[1][i] + hsub[2][i] + hsub[3][i];
    if (tid == 0)
        ccount = 0u;
    __syncthreads();
    uint32_t above;
    const uint32_t bstar = find_bin<true>(hsub[0], kHistBins, (uint32_t)top_k, &bs, &above);
    const uint32_t need = (uint32_t)top_k - above; // keys to take from bin b*

    // ---- sweep 2: keys above b* -> bitmap; keys inside b* -> candidates ----
    const int nwords = (L + 31) / 32;
    uint32_t *bm = nwords <= kBitmapLdsWords ? lbitmap : gbitmap + (int64_t)r * (stride / 32);
    u32x2 *rspill = spill + (int64_t)r * stride;
    sweep([&](int t, float4 v) {
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint64_t ab[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const bool valid = t + j < L;
            const uint32_t key = score_key(e[j]);
            const uint32_t bin = key >> kHistShift;
            ab[j] = __ballot(valid && bin > bstar);
            const bool in = valid && bin == bstar;
            const uint64_t cm = __ballot(in);
            if (cm) {
                const int leader = __ffsll((unsigned long long)cm) - 1;
                uint32_t pos = 0;
                if (lane == leader)
                    pos = atomicAdd(&ccount, (uint32_t)__popcll(cm));
                pos = __shfl(pos, leader, kWave);
                if (in) {
                    const uint32_t at = pos + (uint32_t)__popcll(cm & ((1ull << lane) - 1ull));
                    const u32x2 ent = u32x2{key, (uint32_t)(t + j)};
                    if (at < (uint32_t)kCandCap)
                        cbuf[at] = ent;
                    else if (at < (uint32_t)L)
                        rspill[at] = ent;
                }
            }
        }
        // The wave's 256 tokens start at a multiple of 256: lane q < 8 writes
        // bitmap word q (tokens 32q..32q+31 = lanes 8q..8q+7, 4 elements
        // each). Every word of [0, nwords) is written exactly once.
        const int s0 = t - 4 * lane;
        if (lane < 8 && s0 + 32 * lane < L) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; j++)
                word |= spread8((uint32_t)(ab[j] >> (8 * lane)) & 0xFFu) << j;
            bm[(s0 >> 5) + lane] = word;
        }
    });
    __syncthreads();
    const uint32_t m = min(ccount, (uint32_t)L);
    auto cand_at = [&](uint32_t i) -> u32x2 { return i < (uint32_t)kCandCap ? cbuf[i] : rspill[i]; };

    // ---- radix passes over the candidates ----
    uint32_t *h = hsub[0];
    auto clear_h = [&]() {
        for (int i = tid; i < kHistBins; i += kRowThreads)
            h[i] = 0u;
        __syncthreads();
    };
    // pass A: key bits [20:10], descending
    clear_h();
    for (uint32_t i = tid; i < m; i += kRowThreads)
        atomicAdd(&h[(cand_at(i).x >> 10) & 0x7FFu], 1u);
    __syncthreads();
    uint32_t bef;
    const uint32_t a_bin = find_bin<true>(h, 2048, need, &bs, &bef);
    const uint32_t need_a = need - bef;
    const uint32_t hi21 = (bstar << 11) | a_bin; // key >> 10
    // pass B: key bits [9:0] among key >> 10 == hi21, descending
    clear_h();
    for (uint32_t i = tid; i < m; i += kRowThreads) {
        const uint32_t k = cand_at(i).x;
        if ((k >> 10) == hi21)
            atomicAdd(&h[k & 0x3FFu], 1u);
    }
    __syncthreads();
    const uint32_t b_bin = find_bin<true>(h, 1024, need_a, &bs, &bef);
    const uint32_t need_t = need_a - bef; // keys equal to T to take
    const uint32_t eq_count = h[b_bin];
    const uint32_t T = (hi21 << 10) | b_bin;
    __syncthreads();
    int32_t cut = 0x7FFFFFFF;
    if (need_t < eq_count) {
        // pass C: index bits [21:11] among keys == T, ascending
        clear_h();
        for (uint32_t i = tid; i < m; i += kRowThreads) {
            const u32x2 e = cand_at(i);
            if (e.x == T)
                atomicAdd(&h[(e.y >> 11) & 0x7FFu], 1u);
        }
        __syncthreads();
        const uint32_t c_bin = find_bin<false>(h, 2048, need_t, &bs, &bef);
        const uint32_t need_c = need_t - bef;
        // pass D: index bits [10:0] among keys == T in index block c_bin
        clear_h();
        for (uint32_t i = tid; i < m; i += kRowThreads) {
            const u32x2 e = cand_at(i);
            if (e.x == T && (e.y >> 11) == c_bin)
                atomicAdd(&h[e.y & 0x7FFu], 1u);
        }
        __syncthreads();
        const uint32_t d_bin = find_bin<false>(h, 2048, need_c, &bs, &bef);
        cut = (int32_t)((c_bin << 11) | d_bin);
    }

    // ---- selected candidates join the bitmap ----
    for (uint32_t i = tid; i < m; i += kRowThreads) {
        const u32x2 e = cand_at(i);
        if (e.x > T || (e.x == T && (int32_t)e.y <= cut))
            atomicOr(&bm[e.y >> 5], 1u << (e.y & 31));
    }
    __syncthreads();

    // ---- ascending ids: block scan of the bitmap's popcounts ----
    const int wpt = (nwords + kRowThreads - 1) / kRowThreads;
    const int w0 = tid * wpt;
    uint32_t cnt = 0;
    for (int i = 0; i < wpt; i++)
        if (w0 + i < nwords)
            cnt += __popc(bm[w0 + i]);
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kRowThreads>(cnt, bs.scan, &total);
    for (int i = 0; i < wpt; i++) {
        if (w0 + i >= nwords)
            break;
        uint32_t word = bm[w0 + i];
        while (word && pos < (uint32_t)top_k) {
            const int bit = __ffs(word) - 1;
            out[pos++] = 32 * (w0 + i) + bit;
            word &= word - 1;
        }
    }
}

int launch_select(const LaunchShape &ls, const float *scores, const int32_t *seq_lens,
                  int32_t *sel, char *ws, const Workspace &wl, hipStream_t stream)
{
    hipLaunchKernelGGL(k_select_row, dim3(ls.num_rows), dim3(kRowThreads), 0, stream, scores,
                       seq_lens, sel, (u32x2 *)(ws + wl.spill), (uint32_t *)(ws + wl.bitmap),
                       ls.max_len, score_stride(ls), ls.top_k);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
