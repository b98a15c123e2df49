// topk_select.hip -- exact per-row top-k over [0, L_r) on gfx950.
//
// Order (glm5next_dsa/layer.rs source page, doc of the prefill row-group
// selector before `batch_select_enabled`): score descending, then index
// ascending -- a total order, so the top-k set is unique. Read per token
// (pools of one token); -0.0 equals +0.0. Output: the selected ids in
// ascending order, -1 past min(top_k, L_r).
//
// Every comparison runs on the order-preserving 32-bit key of a score.
//
// Threshold. The index pass (or, for a standalone selection, a group-max
// pass) leaves the largest key of each aligned 4-token and 32-token group.
// Let tau be the k-th largest of a row's group keys: at least k distinct
// tokens (the groups' maxima) have key >= tau, so the top-k of the row lies
// inside {key >= tau}. For keys spread over the row, that set holds little
// more than k tokens (about 1.4 k for 32-token groups at k = L / 64). This
// holds for any input: the group keys only have to be keys of distinct
// tokens of the row.
//
// Three steps, each a kernel boundary apart (no inter-workgroup waiting):
//  1. filter (many workgroups per row, one 4096-token slice each): every
//     workgroup finds tau by radix selection over the row's group keys
//     (redundantly, so no workgroup waits on another), then writes the
//     slice's keys >= tau, in ascending token order, to the slice's own
//     candidate region;
//  2. finish (one workgroup per row): gathers the candidates (already in
//     ascending token order), radix-selects the exact k-th key T among them,
//     and writes the tokens with key > T plus the lowest-index tokens with
//     key == T, in ascending order;
//  3. rows whose candidates do not fit the finishing workgroup (massive ties,
//     adversarial orders, top_k beyond 2048 on mid-length rows) take a
//     full-row radix selection in the same workgroup instead: slower, and
//     exact in the same order.
// Radix digits are taken relative to the block's key range (minimum key to
// maximum key), so even a narrow score distribution spreads over the bins
// and the LDS counters see little contention.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kSliceThreads = 256;          // filter workgroup
constexpr int kSliceTokPerThread = kSelSlice / kSliceThreads; // 16
constexpr int kGmRegs = 32;                 // group keys a filter thread keeps in registers
constexpr int kFinThreads = 1024;           // finishing workgroup
constexpr int kFinCap = 8192;               // candidates the finishing workgroup holds
constexpr int kRowThreads = kFinThreads;    // full-row fallback runs in the same workgroup
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kVecBatch = 8;                // float4 loads per thread per batch (full row)
constexpr int kCandCap = 6144;              // full-row candidates kept in LDS (48 KiB)
constexpr int kBitmapLdsWords = 12288;      // full-row bitmap in LDS up to 393216 tokens
constexpr int kSelDigit = 12;               // bits of a threshold / cut digit
constexpr int kSelBins = 1 << kSelDigit;    // its histogram bins
// Those histograms sit in LDS with 16 bytes of padding after every 64 bins:
// the wave that walks one walks 64 bins per lane, and with the padding the
// lanes' blocks start on different banks (unpadded, every lane's 16-byte
// read would hit the same four banks).
constexpr int kHistPad = 4;
constexpr int kSelHistWords = kSelBins + kSelBins / 64 * kHistPad;
__device__ __forceinline__ uint32_t hslot(uint32_t bin) { return bin + (bin >> 6) * kHistPad; }
constexpr int kRankList = 256;              // boundary-bin members ranked directly

// Shared state of block-wide searches and reductions.
struct BinSearch {
    uint32_t scan[kRowWaves + 1];
    uint32_t red[2][kRowWaves];
    float fsum[kRowWaves]; // block_minmax_sum's partial sums
    uint32_t bin;
    uint32_t before;
    uint32_t total; // count of the last histogram walked by find_bin_desc_wave0
};

// Over the LDS histogram h[0..nbins), walked from the highest bin down
// (descending) or from bin 0 up (ascending), find the bin where the running
// count first reaches `need` (1 <= need <= total). Returns the bin; *before is
// the count of everything walked before it. All NT threads must call.
template <bool Descending, int NT>
__device__ uint32_t find_bin(const uint32_t *h, int nbins, uint32_t need, BinSearch *bs,
                             uint32_t *before)
{
    const int bpt = (nbins + NT - 1) / NT;
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
    uint32_t run = block_exclusive_scan<NT>(local, bs->scan, &total);
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

// Block-wide minimum and maximum of one pair per thread (one barrier; call
// at most once per kernel, as the exchange words are not guarded for reuse).
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t &lo, uint32_t &hi, BinSearch *bs)
{
    constexpr int NW = NT / kWave;
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    const int wid = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        bs->red[0][wid] = lo;
        bs->red[1][wid] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; w++) {
        lo = min(lo, bs->red[0][w]);
        hi = max(hi, bs->red[1][w]);
    }
}

// block_minmax that also sums a float over the block, under the same
// barrier (waves' partials added in wave order: deterministic).
template <int NT>
__device__ __forceinline__ void block_minmax_sum(uint32_t &lo, uint32_t &hi, float &x, BinSearch *bs)
{
    constexpr int NW = NT / kWave;
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    x = wave_total_f32(x);
    const int wid = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        bs->red[0][wid] = lo;
        bs->red[1][wid] = hi;
        bs->fsum[wid] = x;
    }
    __syncthreads();
    x = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        lo = min(lo, bs->red[0][w]);
        hi = max(hi, bs->red[1][w]);
        x += bs->fsum[w];
    }
}

// Descending walk over the kSelBins-bin padded LDS histogram h (16-byte
// aligned; bin b at h[hslot(b)]): the bin where the running count first
// reaches `need`, the count of everything above it and the histogram's
// total, into bs. Run by wave 0 alone: every lane sums its 64 bins, a lane
// scan finds the lane whose bins cross `need`, and a second lane scan over
// those 64 bins finds the bin. A barrier of the caller publishes the result.
// An inconsistent histogram (total < need) yields bin 0.
__device__ __forceinline__ void find_bin_desc_wave0(const uint32_t *h, uint32_t need,
                                                    BinSearch *bs)
{
    constexpr int BPL = kSelBins / kWave; // 64
    const int lane = threadIdx.x;
    const int lo_b = kSelBins - BPL * (lane + 1); // lane 0 holds the top bins
    const u32x4 *h4 = (const u32x4 *)(h + hslot(lo_b));
    uint32_t local = 0;
#pragma unroll
    for (int q = 0; q < BPL / 4; q++) {
        const u32x4 v = h4[q];
        local += (v.x + v.y) + (v.z + v.w);
    }
    const uint32_t x = wave_incl_scan_add(local);
    const uint32_t run = x - local; // count in the bins of lower lanes (higher bins)
    if (lane == kWave - 1)
        bs->total = x;
    const uint64_t hit = __ballot(run < need && x >= need);
    if (hit == 0) { // inconsistent histogram
        if (lane == 0) {
            bs->bin = 0u;
            bs->before = 0u;
        }
        return;
    }
    const int lx = __ffsll((unsigned long long)hit) - 1; // the crossing lane (uniform)
    const uint32_t run_x = (uint32_t)__builtin_amdgcn_readlane((int)run, lx);
    // lane i: bin top - i of that lane's block, walked downwards
    const int top = kSelBins - BPL * lx - 1;
    const uint32_t c = h[hslot((uint32_t)(top - lane))];
    const uint32_t y = run_x + wave_incl_scan_add(c); // count down to and with this bin
    const uint64_t hit2 = __ballot(y >= need && y - c < need);
    if (lane == __ffsll((unsigned long long)hit2) - 1) {
        bs->bin = (uint32_t)(top - lane);
        bs->before = y - c;
    }
}

// Bit length of x (0 for 0).
__device__ __forceinline__ int bit_len(uint32_t x) { return x ? 32 - __clz(x) : 0; }

// The score value of an order key (the inverse of score_key; -0 came back
// as +0).
__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int row_len(const int32_t *seq_lens, int r, int max_len)
{
    return min(max(seq_lens[r], 0), max_len);
}

// ---------------------------------------------------------------------------
// Group maxima from a scores buffer (standalone selection only; the index
// pass of a whole step writes the same arrays itself). Grid (slices, R).
__global__ __launch_bounds__(kSliceThreads) void k_group_max(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    uint32_t *__restrict__ gm4, uint32_t *__restrict__ gm32, int max_len, int stride)
{
    const int r = blockIdx.y;
    const int L = row_len(seq_lens, r, max_len);
    const int s0 = blockIdx.x * kSelSlice;
    if (s0 >= L)
        return;
    const int t0 = s0 + kSliceTokPerThread * threadIdx.x;
    const float4 *row4 = (const float4 *)(scores + (int64_t)r * stride);
    const int nvec = (L + 3) / 4;
    uint32_t m4[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float4 v = row4[min(t0 / 4 + j, nvec - 1)];
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < 4; i++)
            m = max(m, t0 + 4 * j + i < L ? score_key(e[i]) : 0u);
        m4[j] = m;
    }
    uint32_t m16 = max(max(m4[0], m4[1]), max(m4[2], m4[3]));
    const uint32_t m32 = max(m16, (uint32_t)__shfl_xor((int)m16, 1, kWave));
    uint32_t *g4 = gm4 + (int64_t)r * (stride / 4);
#pragma unroll
    for (int j = 0; j < 4; j++)
        if (t0 + 4 * j < L)
            g4[t0 / 4 + j] = m4[j];
    if ((threadIdx.x & 1) == 0 && t0 < L)
        gm32[(int64_t)r * (stride / 32) + t0 / 32] = m32;
}

// ---------------------------------------------------------------------------
// Filter: grid (slices, R). Slice p of row r covers tokens
// [4096 p, 4096 p + 4096) of [0, L); its candidates (key >= tau) go, in
// ascending token order, to cand[r][4096 p ...], their number to cnt[r][p].
__global__ __launch_bounds__(kSliceThreads) void k_select_filter(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    const uint32_t *__restrict__ gm4, const uint32_t *__restrict__ gm32,
    u32x2 *__restrict__ cand, uint32_t *__restrict__ cnt, int max_len, int stride, int top_k,
    int pmax)
{
    __shared__ __align__(16) uint32_t hist[kSelHistWords];
    __shared__ BinSearch bs;
    const int r = blockIdx.y;
    const int p = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = row_len(seq_lens, r, max_len);
    const int s0 = p * kSelSlice;
    if (L <= top_k || s0 >= L)
        return;

    // this slice's scores: issued first, they land while tau is found
    const int t0 = s0 + kSliceTokPerThread * tid;
    const float4 *row4 = (const float4 *)(scores + (int64_t)r * stride);
    const int nvec = (L + 3) / 4;
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
        v[j] = row4[min(t0 / 4 + j, nvec - 1)];

    // group keys: the finest level that still has at least top_k groups and
    // whose keys fit the registers; failing both, every token is a
    // candidate (then L < 4 top_k)
    const int ng32 = (L + 31) / 32;
    const int ng4 = (L + 3) / 4;
    const uint32_t *gm = nullptr;
    int ng = 0;
    if (ng4 >= top_k && ng4 <= kGmRegs * kSliceThreads) {
        gm = gm4 + (int64_t)r * (stride / 4);
        ng = ng4;
    } else if (ng32 >= top_k) {
        gm = gm32 + (int64_t)r * (stride / 32);
        ng = ng32;
    } else if (ng4 >= top_k) {
        gm = gm4 + (int64_t)r * (stride / 4);
        ng = ng4;
    }
    // tau: the lower edge of the 12-bit digit bin (relative to the group
    // keys' range) that holds the top_k-th largest group key. Every group
    // key of that bin and above is >= tau, so at least top_k tokens are.
    uint32_t tau = 0u;
    if (gm != nullptr) {
        const bool in_regs = ng <= kGmRegs * kSliceThreads;
        const int nj = (ng + kSliceThreads - 1) / kSliceThreads;
        uint32_t kk[kGmRegs];
        if (in_regs) {
#pragma unroll
            for (int j = 0; j < kGmRegs; j++)
                kk[j] = gm[min(tid + kSliceThreads * j, ng - 1)];
        }
        auto for_keys = [&](auto &&f) {
            if (in_regs) {
#pragma unroll
                for (int j = 0; j < kGmRegs; j++)
                    if (j < nj && tid + kSliceThreads * j < ng)
                        f(kk[j]);
            } else {
                for (int i = tid; i < ng; i += kSliceThreads)
                    f(gm[i]);
            }
        };
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
        for_keys([&](uint32_t k) {
            lo = min(lo, k);
            hi = max(hi, k);
        });
        for (int i = tid; i < kSelHistWords; i += kSliceThreads)
            hist[i] = 0u;
        block_minmax<kSliceThreads>(lo, hi, &bs); // its barrier also publishes the cleared bins
        const int shift = max(bit_len(hi - lo) - kSelDigit, 0);
        for_keys([&](uint32_t k) { atomicAdd(&hist[hslot((k - lo) >> shift)], 1u); });
        __syncthreads();
        if (tid < kWave)
            find_bin_desc_wave0(hist, (uint32_t)top_k, &bs);
        __syncthreads();
        tau = lo + (bs.bin << shift);
    }

    uint32_t key[kSliceTokPerThread];
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = t0 + 4 * j + i;
            key[4 * j + i] = score_key(e[i]);
            c += (t < L && key[4 * j + i] >= tau) ? 1u : 0u;
        }
    }
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kSliceThreads>(c, bs.scan, &total);
    u32x2 *dst = cand + (int64_t)r * stride + s0;
#pragma unroll
    for (int i = 0; i < kSliceTokPerThread; i++) {
        const int t = t0 + i;
        if (t < L && key[i] >= tau)
            dst[pos++] = u32x2{key[i], (uint32_t)t};
    }
    if (tid == 0)
        cnt[(int64_t)r * pmax + p] = total;
}

// ---------------------------------------------------------------------------
// Full-row radix selection (fallback of the finishing workgroup). LDS comes
// from the caller: hsub [4][kHistBins], cbuf [kCandCap], lbitmap
// [kBitmapLdsWords].
//  1. sweep 1: histogram of the key's top 11 bits (four LDS copies to spread
//     contention); the bin b* holding the k-th largest key follows;
//  2. sweep 2: keys above b* go straight into a bitmap of the row (one wave
//     ballot builds eight bitmap words); keys inside b* are appended to LDS
//     (or to the workspace past capacity);
//  3. four radix passes over those resolve the exact threshold key T and,
//     among keys equal to T, the largest selected index;
//  4. the selected ones join the bitmap; a block-wide scan of its popcounts
//     writes the ids in ascending order.
__device__ __forceinline__ uint32_t spread8(uint32_t x)
{
    // the 8 bits of x to bit positions 0, 4, 8, ..., 28
    x = (x | (x << 12)) & 0x000F000Fu;
    x = (x | (x << 6)) & 0x03030303u;
    x = (x | (x << 3)) & 0x11111111u;
    return x;
}

__device__ __forceinline__ void select_row_full(const float *__restrict__ scores, int r, int L, int32_t *out,
                                u32x2 *rspill, uint32_t *gbitmap_row, int stride, int top_k,
                                uint32_t (*hsub)[kHistBins], u32x2 *cbuf, uint32_t *lbitmap,
                                BinSearch *bs, uint32_t *ccount)
{
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const float4 *row4 = (const float4 *)(scores + (int64_t)r * stride);
    const int nvec = (L + 3) / 4; // float4s covering [0, L) (all inside the row stride)
    constexpr int kBatchTok = kRowThreads * kVecBatch * 4;
    // Two batches of kVecBatch float4 per thread in flight; f(t, v) runs for
    // the float4 v holding tokens t .. t+3 (entries at or past L are masked
    // by f).
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
                atomicAdd(&myh[score_key(e[j]) >> 21], 1u);
    });
    __syncthreads();
    for (int i = tid; i < kHistBins; i += kRowThreads)
        hsub[0][i] += hsub[1][i] + hsub[2][i] + hsub[3][i];
    if (tid == 0)
        *ccount = 0u;
    __syncthreads();
    uint32_t above;
    const uint32_t bstar =
        find_bin<true, kRowThreads>(hsub[0], kHistBins, (uint32_t)top_k, bs, &above);
    const uint32_t need = (uint32_t)top_k - above; // keys to take from bin b*

    // ---- sweep 2: keys above b* -> bitmap; keys inside b* -> candidates ----
    const int nwords = (L + 31) / 32;
    uint32_t *bm = nwords <= kBitmapLdsWords ? lbitmap : gbitmap_row;
    sweep([&](int t, float4 v) {
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint64_t ab[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const bool valid = t + j < L;
            const uint32_t key = score_key(e[j]);
            const uint32_t bin = key >> 21;
            ab[j] = __ballot(valid && bin > bstar);
            const bool in = valid && bin == bstar;
            const uint64_t cm = __ballot(in);
            if (cm) {
                const int leader = __ffsll((unsigned long long)cm) - 1;
                uint32_t pos = 0;
                if (lane == leader)
                    pos = atomicAdd(ccount, (uint32_t)__popcll(cm));
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
    const uint32_t m = min(*ccount, (uint32_t)L);
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
    const uint32_t a_bin = find_bin<true, kRowThreads>(h, 2048, need, bs, &bef);
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
    const uint32_t b_bin = find_bin<true, kRowThreads>(h, 1024, need_a, bs, &bef);
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
        const uint32_t c_bin = find_bin<false, kRowThreads>(h, 2048, need_t, bs, &bef);
        const uint32_t need_c = need_t - bef;
        // pass D: index bits [10:0] among keys == T in index block c_bin
        clear_h();
        for (uint32_t i = tid; i < m; i += kRowThreads) {
            const u32x2 e = cand_at(i);
            if (e.x == T && (e.y >> 11) == c_bin)
                atomicAdd(&h[e.y & 0x7FFu], 1u);
        }
        __syncthreads();
        const uint32_t d_bin = find_bin<false, kRowThreads>(h, 2048, need_c, bs, &bef);
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
    uint32_t pos = block_exclusive_scan<kRowThreads>(cnt, bs->scan, &total);
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

// ---------------------------------------------------------------------------
// Exact cut and output of the finishing workgroup. The kFinThreads threads
// hold the row's candidates, N each, thread-major in ascending token order
// (bit j of `valid` marks a held candidate), with every candidate key in
// [lo, hi]. Relative 12-bit digits narrow a key window to the bin holding
// the top_k-th candidate; the bin's members are then ranked directly under
// (key desc, index asc), and the selected ids leave in ascending order.
// Needs the first histogram (the area's first kSelHistWords words) cleared
// and ccount zero, both published by a barrier. Returns false, having
// written nothing, when fewer than top_k candidates are held (the same
// answer in every thread).
template <int N, bool VALUE_ANY = false>
__device__ __forceinline__ bool exact_cut_write(const uint32_t (&kk)[N], const uint32_t (&id)[N],
                                                uint32_t valid, uint32_t lo, uint32_t hi,
                                                int top_k, int32_t *out, uint8_t *area,
                                                BinSearch &bs, uint32_t &ccount,
                                                float vmean = 0.0f)
{
    static_assert(N <= 32, "one mask bit per held candidate");
    const int tid = threadIdx.x;
    uint32_t *hist0 = (uint32_t *)area;                        // two histograms,
    uint32_t *hist1 = (uint32_t *)(area + kSelHistWords * 4);  // then the member list
    u32x2 *list = (u32x2 *)(area + 2 * kSelHistWords * 4);
    uint32_t need = (uint32_t)top_k;
    uint32_t *h = hist0, *hn = hist1;
    bool first = true;
    uint32_t pre_take = 0; // bit j: held candidate j is selected by the value pass
    bool ranked_direct = false;

    // Keys on both sides of zero: the order-preserving key image is close to
    // logarithmic in the value, so a relative key digit over such a range
    // piles most keys of a bell-shaped row into a few bins (a 1024-thread
    // histogram then serialises on their atomics; measured 8.5 -> 28 us for
    // one 8192-key row of N(0, 1) scores). The first pass then bins by value
    // instead, linearly over [value(lo), value(hi)]: bin(v) = min(4095,
    // floor((v - value(lo)) * 4096 / (value(hi) - value(lo)))) never
    // decreases with the key, so the bins above the boundary bin are taken,
    // those below are not, and the boundary bin's members form one key
    // interval that the key passes below narrow.
    // With VALUE_ANY (a whole row held), keys on one side of zero take the
    // value pass too when it pays: for a row whose values spread over their
    // span (a bell, a plateau) the key image piles them into a few bins as
    // well (measured, a 16k-token row of non-negative scores: 18.0 -> 13.6
    // us), but a heavy tail's outliers set the span and leave nearly every
    // value in the lowest value bins. The mean's place in the span tells the
    // two apart (a heavy tail's mean sits near its bottom); vmean is the
    // held values' mean, from the caller's range reduction.
    const bool straddle = lo < 0x80000000u && hi >= 0x80000000u;
    if (straddle || VALUE_ANY) {
        const float vlo = key_value(lo);
        const float span = key_value(hi) - vlo;
        const float scale = (float)kSelBins / span;
        bool use = span > 0.0f && __builtin_isfinite(span) && __builtin_isfinite(scale);
        if (VALUE_ANY && !straddle && use)
            use = 16.0f * (vmean - vlo) >= span;
        if (use) {
            auto vbin = [&](uint32_t k) {
                return (uint32_t)fminf((key_value(k) - vlo) * scale, (float)(kSelBins - 1));
            };
#pragma unroll
            for (int j = 0; j < N; j++)
                if (valid & (1u << j))
                    atomicAdd(&h[hslot(vbin(kk[j]))], 1u);
            __syncthreads();
            for (int i = tid; i < kSelHistWords; i += kFinThreads)
                hn[i] = 0u;
            if (tid < kWave)
                find_bin_desc_wave0(h, need, &bs);
            __syncthreads();
            if (bs.total < (uint32_t)top_k)
                return false; // every held candidate was counted
            first = false;
            const uint32_t b = bs.bin;
            need -= bs.before;
            const uint32_t count_v = h[hslot(b)];
            uint32_t members = 0;
            uint32_t mlo = 0xFFFFFFFFu, mhi = 0u;
#pragma unroll
            for (int j = 0; j < N; j++) {
                if (valid & (1u << j)) {
                    const uint32_t vb = vbin(kk[j]);
                    if (vb > b)
                        pre_take |= 1u << j;
                    if (vb == b) {
                        members |= 1u << j;
                        mlo = min(mlo, kk[j]);
                        mhi = max(mhi, kk[j]);
                    }
                }
            }
            valid = members;
            uint32_t *t = h;
            h = hn;
            hn = t;
            if (count_v <= (uint32_t)kRankList) {
                ranked_direct = true; // few members: straight to the ranking
                __syncthreads();       // every thread has read h[b] before the area is reused
            } else {
                block_minmax<kFinThreads>(mlo, mhi, &bs); // its barrier also retires the reads of h[b]
                lo = mlo;
                hi = mhi;
            }
        }
    }

    uint32_t base = lo;
    int bits = bit_len(hi - lo); // window [base, base + 2^bits) holds every key
    uint32_t bin_lo = base;      // the boundary bin [bin_lo, bin_lo + 2^shift)
    int shift = 0;
    uint32_t count_b = 0u;
    while (!ranked_direct) {
        shift = max(bits - kSelDigit, 0);
        // Only keys inside the window [base, base + 2^bits) are counted: it
        // has 2^(bits - shift) <= kSelBins bins. After a narrowing pass, keys
        // of the bins above the old boundary bin can still fall within
        // kSelBins units of the new base; `need` has already discounted
        // them, so counting them again would move the cut.
        const uint32_t nbins = 1u << (bits - shift);
#pragma unroll
        for (int j = 0; j < N; j++) {
            if ((valid & (1u << j)) && kk[j] >= base) {
                const uint32_t d = (kk[j] - base) >> shift;
                if (d < nbins)
                    atomicAdd(&h[hslot(d)], 1u);
            }
        }
        __syncthreads();
        for (int i = tid; i < kSelHistWords; i += kFinThreads)
            hn[i] = 0u;
        if (tid < kWave)
            find_bin_desc_wave0(h, need, &bs);
        __syncthreads();
        if (first && bs.total < (uint32_t)top_k)
            return false; // the first window holds every candidate
        first = false;
        const uint32_t b = bs.bin;
        need -= bs.before;           // members of bin b to take
        count_b = h[hslot(b)];
        bin_lo = base + (b << shift);
        if (count_b <= (uint32_t)kRankList || shift == 0)
            break;
        base = bin_lo;
        bits = shift;
        uint32_t *t = h;
        h = hn;
        hn = t;
        __syncthreads(); // everyone has read h[b] before it is cleared again
    }
    // keys >= bin_lo + 2^shift are taken, keys < bin_lo are not; the bin's
    // members take `need` places (after a value pass whose boundary bin was
    // small, the members are that bin's)
    uint32_t take = pre_take; // bit j: held candidate j is selected
    uint32_t inbin = 0;
    if (ranked_direct) {
        inbin = valid;
        count_b = (uint32_t)kRankList;
    } else {
#pragma unroll
        for (int j = 0; j < N; j++) {
            if ((valid & (1u << j)) && kk[j] >= bin_lo) {
                if (((kk[j] - bin_lo) >> shift) >= 1u)
                    take |= 1u << j;
                else
                    inbin |= 1u << j;
            }
        }
    }
    if (count_b <= (uint32_t)kRankList) {
        // few members: each ranks itself against the member list (one
        // atomic per thread places its members)
        const uint32_t mine = (uint32_t)__popc(inbin);
        uint32_t at = 0;
        if (mine != 0u)
            at = atomicAdd(&ccount, mine);
#pragma unroll
        for (int j = 0; j < N; j++) {
            if (inbin & (1u << j)) {
                if (at < (uint32_t)kRankList)
                    list[at] = u32x2{kk[j], id[j]};
                at++;
            }
        }
        __syncthreads();
        const uint32_t nl = min(ccount, (uint32_t)kRankList);
#pragma unroll
        for (int j = 0; j < N; j++) {
            if (inbin & (1u << j)) {
                uint32_t rank = 0;
#pragma unroll 8
                for (uint32_t i = 0; i < nl; i++) {
                    const u32x2 y = list[i];
                    rank += (y.x > kk[j] || (y.x == kk[j] && y.y < id[j])) ? 1u : 0u;
                }
                if (rank < need)
                    take |= 1u << j;
            }
        }
    } else {
        // one key shared by many members (shift == 0): lowest indices first;
        // the held candidates are in ascending index order, thread-major, so
        // a scan of member counts ranks them
        uint32_t tot;
        uint32_t rank = block_exclusive_scan<kFinThreads>((uint32_t)__popc(inbin), bs.scan, &tot);
#pragma unroll
        for (int j = 0; j < N; j++) {
            if (inbin & (1u << j)) {
                if (rank < need)
                    take |= 1u << j;
                rank++;
            }
        }
    }

    // ascending ids: one scan of the per-thread counts places every id
    uint32_t tot;
    uint32_t pos = block_exclusive_scan<kFinThreads>((uint32_t)__popc(take), bs.scan, &tot);
#pragma unroll
    for (int j = 0; j < N; j++) {
        if ((take & (1u << j)) && pos < (uint32_t)top_k)
            out[pos++] = (int32_t)id[j];
    }
    return true;
}

// ---------------------------------------------------------------------------
// Finish: one workgroup per row. Thread t owns the contiguous run of
// candidates [t * run, t * run + run) in registers (run <= kFinRun), so the
// selected ids leave in ascending order straight from registers.
constexpr int kFinRun = kFinCap / kFinThreads; // 8
constexpr int kFullLdsBytes = 4 * kHistBins * 4 + kCandCap * 8 + kBitmapLdsWords * 4;
static_assert(2 * kSelHistWords * 4 + kRankList * 8 <= kFullLdsBytes, "cut LDS must fit the area");

__global__ __launch_bounds__(kFinThreads) void k_select_finish(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens,
    u32x2 *__restrict__ cand, const uint32_t *__restrict__ cnt, int32_t *__restrict__ sel,
    uint32_t *__restrict__ gbitmap, int max_len, int stride, int top_k, int pmax)
{
    __shared__ __align__(16) uint8_t area[kFullLdsBytes]; // full-row fallback, or the cut's
                                                          // histograms and member list
    __shared__ uint32_t pre[kFinThreads];  // candidate offset of each slice
    __shared__ uint32_t cntl[kFinThreads]; // candidate count of each slice
    __shared__ uint32_t cmaxl[kFinThreads / kWave]; // per-wave largest count
    __shared__ BinSearch bs;
    __shared__ uint32_t ccount;

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = row_len(seq_lens, r, max_len);
    int32_t *out = sel + (int64_t)r * top_k;

    if (L <= top_k) { // every token is selected; slots past L are padding
        for (int slot = tid; slot < top_k; slot += kFinThreads)
            out[slot] = slot < L ? slot : -1;
        return;
    }

    // candidate counts of the row's slices -> offsets
    const int P = (L + kSelSlice - 1) / kSelSlice; // <= pmax <= kFinThreads
    const uint32_t c = tid < P ? cnt[(int64_t)r * pmax + tid] : 0u;
    uint32_t mu;
    const uint32_t off = block_exclusive_scan<kFinThreads>(c, bs.scan, &mu);
    // Usually every slice's candidates fit a fixed block of tps threads,
    // srun each (srun from the largest count), and thread t takes its share
    // of slice t / tps directly. Otherwise they are spread evenly over the
    // threads, each finding its slices by a search of the offsets.
    const int tps = kFinThreads / P;
    if (tid < P) {
        pre[tid] = off;
        cntl[tid] = c;
    }
    const uint32_t cmax_w = wave_max_u32(c);
    if (tid % kWave == 0)
        cmaxl[tid / kWave] = cmax_w; // words of their own: read after the barrier, never rewritten
    __syncthreads();
    uint32_t cmax = 0;
#pragma unroll
    for (int w = 0; w < kFinThreads / kWave; w++)
        cmax = max(cmax, cmaxl[w]);
    const int srun = ((int)cmax + tps - 1) / tps;
    const bool by_slice = srun <= kFinRun;
    const int m = (int)mu;

    if (m < top_k || m > kFinCap) {
        uint32_t(*hsub)[kHistBins] = (uint32_t(*)[kHistBins])area;
        u32x2 *cbuf = (u32x2 *)(area + 4 * kHistBins * 4);
        uint32_t *lbitmap = (uint32_t *)(area + 4 * kHistBins * 4 + kCandCap * 8);
        select_row_full(scores, r, L, out, cand + (int64_t)r * stride,
                        gbitmap + (int64_t)r * (stride / 32), stride, top_k, hsub, cbuf, lbitmap,
                        &bs, &ccount);
        return;
    }

    const u32x2 *src = cand + (int64_t)r * stride;
    uint32_t kk[kFinRun], id[kFinRun];
    int n_own;
    if (by_slice) {
        const int p = tid / tps; // threads past P * tps hold nothing
        const int u = tid % tps;
        const int cp = p < P ? (int)cntl[p] : 0;
        n_own = min(srun, max(cp - u * srun, 0));
        const u32x2 *sp = src + (int64_t)min(p, P - 1) * kSelSlice + u * srun;
#pragma unroll
        for (int j = 0; j < kFinRun; j++) {
            u32x2 e = u32x2{0u, 0u};
            if (j < n_own)
                e = sp[j];
            kk[j] = e.x;
            id[j] = e.y;
        }
    } else {
        // this thread's run, gathered from the slices' regions (all loads in
        // flight at once; indices past the run repeat the last candidate)
        const int run = (m + kFinThreads - 1) / kFinThreads;
        const int i0 = min(tid * run, m);
        n_own = min(run, m - i0);
        int sl = 0; // slice of candidate min(i0, m - 1): last offset <= it
        {
            const int i = min(i0, m - 1);
            int lo = 0, hi = P - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pre[mid] <= (uint32_t)i)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            sl = lo;
        }
        // the run usually stays inside one slice: keep that slice's bounds in
        // registers and touch LDS again only when the run crosses into the next
        int src_off[kFinRun];
        int sl_lo = (int)pre[sl];
        int sl_hi = sl + 1 < P ? (int)pre[sl + 1] : m; // first candidate of the next slice
#pragma unroll
        for (int j = 0; j < kFinRun; j++) {
            const int i = min(i0 + min(j, max(n_own - 1, 0)), m - 1);
            while (i >= sl_hi) {
                sl++;
                sl_lo = sl_hi;
                sl_hi = sl + 1 < P ? (int)pre[sl + 1] : m;
            }
            src_off[j] = sl * kSelSlice + (i - sl_lo);
        }
#pragma unroll
        for (int j = 0; j < kFinRun; j++) {
            const u32x2 e = src[src_off[j]];
            kk[j] = e.x;
            id[j] = e.y;
        }
    }

    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int j = 0; j < kFinRun; j++) {
        if (j < n_own) {
            lo = min(lo, kk[j]);
            hi = max(hi, kk[j]);
        }
    }
    for (int i = tid; i < kSelHistWords; i += kFinThreads)
        ((uint32_t *)area)[i] = 0u;
    if (tid == 0)
        ccount = 0u;
    block_minmax<kFinThreads>(lo, hi, &bs); // its barrier publishes the cleared bins
    const uint32_t valid = (1u << n_own) - 1u;
    if (!exact_cut_write<kFinRun>(kk, id, valid, lo, hi, top_k, out, area, bs, ccount)) {
        // the regions held fewer candidates than the counts promised
        __syncthreads();
        select_row_full(scores, r, L, out, cand + (int64_t)r * stride,
                        gbitmap + (int64_t)r * (stride / 32), stride, top_k,
                        (uint32_t(*)[kHistBins])area, (u32x2 *)(area + 4 * kHistBins * 4),
                        (uint32_t *)(area + 4 * kHistBins * 4 + kCandCap * 8), &bs, &ccount);
    }
}

// ---------------------------------------------------------------------------
// Direct: rows of at most kSelDirectMax tokens in one kernel. One workgroup
// per row holds the whole row, thread t the tokens [t * RUN, t * RUN + RUN)
// (ascending, thread-major, as the finish holds its candidates), and runs
// the finish's exact cut on all of them: no threshold, no candidate lists,
// no second kernel. The result is the same unique top-k.
template <int RUN>
__global__ __launch_bounds__(kFinThreads) void k_select_direct(const float *__restrict__ scores,
                                                               const int32_t *__restrict__ seq_lens,
                                                               int32_t *__restrict__ sel, int max_len,
                                                               int stride, int top_k)
{
    static_assert(RUN % 4 == 0 && RUN <= 32, "float4 loads, one mask bit per token");
    __shared__ __align__(16) uint8_t area[2 * kSelHistWords * 4 + kRankList * 8];
    __shared__ BinSearch bs;
    __shared__ uint32_t ccount;

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = row_len(seq_lens, r, max_len);
    int32_t *out = sel + (int64_t)r * top_k;
    if (L <= top_k) { // every token is selected; slots past L are padding
        for (int slot = tid; slot < top_k; slot += kFinThreads)
            out[slot] = slot < L ? slot : -1;
        return;
    }
    const float *srow = scores + (int64_t)r * stride;
    const int t0 = tid * RUN;
    uint32_t kk[RUN], id[RUN];
    floatx4 v[RUN / 4];
#pragma unroll
    for (int q = 0; q < RUN / 4; q++) // a load only where its first token is in the row
        v[q] = (t0 + 4 * q < L) ? *(const floatx4 *)(srow + t0 + 4 * q)
                                : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t valid = 0u, lo = 0xFFFFFFFFu, hi = 0u;
    float vsum = 0.0f; // the row's values summed for their mean (see exact_cut_write)
#pragma unroll
    for (int j = 0; j < RUN; j++) {
        kk[j] = score_key(v[j / 4][j % 4]);
        id[j] = (uint32_t)(t0 + j);
        if (t0 + j < L) {
            valid |= 1u << j;
            lo = min(lo, kk[j]);
            hi = max(hi, kk[j]);
            vsum += v[j / 4][j % 4];
        }
    }
    for (int i = tid; i < 2 * kSelHistWords; i += kFinThreads)
        ((uint32_t *)area)[i] = 0u;
    if (tid == 0)
        ccount = 0u;
    block_minmax_sum<kFinThreads>(lo, hi, vsum, &bs); // its barrier publishes the cleared bins
    // every token of the row is a candidate, so the first window holds
    // L > top_k of them and the cut never reports a shortfall
    (void)exact_cut_write<RUN, true>(kk, id, valid, lo, hi, top_k, out, area, bs, ccount,
                                     vsum / (float)L);
}

int launch_select(const LaunchShape &ls, const float *scores, const int32_t *seq_lens,
                  int32_t *sel, char *ws, const Workspace &wl, bool have_group_max,
                  hipStream_t stream, KTimer t_filter, KTimer t_finish)
{
    const int pmax = sel_slices(ls);
    const int stride = score_stride(ls);
    uint32_t *gm4 = (uint32_t *)(ws + wl.gm4);
    uint32_t *gm32 = (uint32_t *)(ws + wl.gm32);
    u32x2 *cand = (u32x2 *)(ws + wl.cand);
    uint32_t *cnt = (uint32_t *)(ws + wl.cnt);
    if (select_direct(ls)) {
        // one kernel; the filter's events, if any, span nothing
        for (hipEvent_t e : {t_filter.start, t_filter.stop})
            if (e != nullptr && hipEventRecord(e, stream) != hipSuccess)
                return -1;
        // tokens a thread: the row length over the threads, rounded up to a
        // multiple of 4 (float4 loads), at least 8
        static_assert(kSelDirectMax <= 24 * kFinThreads, "at most 24 tokens a thread");
        const int run = ls.max_len <= 8 * kFinThreads ? 8 : 4 * ((ls.max_len + 4 * kFinThreads - 1) / (4 * kFinThreads));
        auto kern = run == 8 ? k_select_direct<8> : run == 12 ? k_select_direct<12>
                  : run == 16 ? k_select_direct<16> : run == 20 ? k_select_direct<20> : k_select_direct<24>;
        hipExtLaunchKernelGGL(kern, dim3(ls.num_rows), dim3(kFinThreads), 0, stream, t_finish.start,
                              t_finish.stop, 0u, scores, seq_lens, sel, ls.max_len, stride, ls.top_k);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const dim3 slices(pmax, ls.num_rows);
    if (!have_group_max)
        hipLaunchKernelGGL(k_group_max, slices, dim3(kSliceThreads), 0, stream, scores, seq_lens,
                           gm4, gm32, ls.max_len, stride);
    hipExtLaunchKernelGGL(k_select_filter, slices, dim3(kSliceThreads), 0, stream, t_filter.start,
                          t_filter.stop, 0u, scores, seq_lens, gm4, gm32, cand, cnt, ls.max_len,
                          stride, ls.top_k, pmax);
    hipExtLaunchKernelGGL(k_select_finish, dim3(ls.num_rows), dim3(kFinThreads), 0, stream,
                          t_finish.start, t_finish.stop, 0u, scores, seq_lens, cand, cnt, sel,
                          (uint32_t *)(ws + wl.bitmap), ls.max_len, stride, ls.top_k, pmax);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

} // namespace dsa
